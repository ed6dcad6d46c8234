"""spec_verify_probs_noalloc (the entry point for callers that cannot
allocate: the library's fixed per-device scratch in place of a workspace)
called through the C ABI, against spec_verify_probs with a workspace of its
own: identical tokens and accept counts on two calls in a row, the second
with a smaller batch and vocabulary, then a batch larger than the scratch is
refused before anything is launched."""

import ctypes

import numpy as np
import pytest
import torch

from rejection_sampling_verifier_spec_amd import api
from rejection_sampling_verifier_spec_amd.workloads import make_workload

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    api.load()


def _inputs(w):
    if w["dtype"] == "bf16":
        l = torch.from_numpy(np.ascontiguousarray(w["logits_bits"]).view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        l = torch.from_numpy(np.ascontiguousarray(w["logits"])).to(DEV)
    q = None if w["draft_probs"] is None else torch.from_numpy(w["draft_probs"]).to(DEV)
    return l, q, torch.from_numpy(w["draft_tokens"]).to(DEV), torch.from_numpy(w["uniforms"]).to(DEV)


def _noalloc(l, q, x, u, T, out, nacc):
    """spec_verify_probs_noalloc through ctypes, outputs preallocated by the test."""
    lib = api.load()
    B, g1, V = l.shape
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    dt = api.SV_DTYPE_BF16 if l.dtype == torch.bfloat16 else api.SV_DTYPE_F32
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    return lib.spec_verify_probs_noalloc(p(l), dt, p(q), p(x), p(u), B, g1 - 1, V, float(T), 0, p(out), p(nacc),
                                         None, stream)


@pytest.mark.parametrize("first,second", [
    (("peaked_bf16", 64, 128256), ("peaked_bf16", 8, 20000)),
    (("dense_f32", 64, 32000), ("onehot_bf16", 12, 9000)),
])
def test_noalloc_equals_the_workspace_entry_point(first, second):
    for name, B, V in (first, second):
        w = make_workload(name, 13, B=B, V=V)
        l, q, x, u = _inputs(w)
        T = w["temperature"] if w["temperature"] > 0 else 1.0
        ref_out, ref_n, _, _ = api.verify_probs(l, q, x, u, T)
        out = torch.full(ref_out.shape, -7, dtype=torch.int64, device=DEV)
        nacc = torch.full(ref_n.shape, -7, dtype=torch.int32, device=DEV)
        assert _noalloc(l, q, x, u, T, out, nacc) == 0
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), (name, B, V)
        assert torch.equal(nacc, ref_n), (name, B, V)
        o2, n2, _ = api.verify_probs_noalloc(l, q, x, u, T)
        torch.cuda.synchronize()
        assert torch.equal(o2, ref_out) and torch.equal(n2, ref_n)


def test_noalloc_refuses_a_batch_beyond_its_scratch():
    B, g, V = 1200, 7, 128256  # needs about 17 MiB of workspace
    assert api.workspace_size(B * (g + 1), V) > api.SV_NOALLOC_SCRATCH_BYTES
    l = torch.zeros((B, g + 1, V), dtype=torch.bfloat16, device=DEV)
    q = torch.full((B, g, V), 1.0 / V, dtype=torch.float32, device=DEV)
    x = torch.zeros((B, g), dtype=torch.int64, device=DEV)
    u = torch.ones((B, g + 1), dtype=torch.float32, device=DEV)
    out = torch.full((B, g + 1), -7, dtype=torch.int64, device=DEV)
    nacc = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    assert _noalloc(l, q, x, u, 1.0, out, nacc) == -4  # SV_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == -7) and torch.all(nacc == -7)  # nothing launched
