"""ctypes binding of ``libspecverify.so`` (C ABI in include/specverify.h).

Argument marshalling only: tensors are checked for device, dtype and
contiguity, their data pointers and the current HIP stream are handed to the
library, and a nonzero status raises. Every step of the verification runs in
the library's kernels; there is no other path. PyTorch supplies device memory
(outputs, workspace) and the stream.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# SPECVERIFY_LIB: another build of the same library (e.g. the host-sanitized one)
LIB_PATH = os.environ.get("SPECVERIFY_LIB") or os.path.join(_PKG, "libspecverify.so")

SV_DTYPE_F32 = 0
SV_DTYPE_BF16 = 1
SV_FLAG_EXACT = 0x1
SV_FLAG_ALL_RESIDUALS = 0x2
SV_FLAG_EAGER = 0x4
SV_ROW_ACCEPTED = 0x1
SV_ROW_EXACT = 0x2
SV_ROW_RESIDUAL = 0x4
SV_ROW_FALLBACK = 0x8
SV_ROW_DEFERRED = 0x400
SV_ROW_UNDECIDED = 0x800
SV_ROW_UNREAD = 0x1000
SV_ROW_HEAD2 = 0x2000
SV_ROW_ROW_SELECT = 0x4000
SV_ROW_TILE_SUMS = 0x8000
SV_ROW_WHY = {0x10: "accept", 0x20: "fallback", 0x40: "search", 0x80: "margin", 0x100: "forced"}
SV_PROFILE_ROWS = 0
SV_PROFILE_REQUEST = 1
SV_PROFILE_ROWS_FIRST = 2

EXPORTS = ("spec_verify_workspace_size", "spec_verify_status_string", "spec_verify_version",
           "spec_verify_probs", "spec_verify_greedy", "spec_verify_ragged", "spec_verify_selftest_exp2",
           "spec_verify_exp2_error_bound", "spec_verify_profile_start", "spec_verify_profile_stop",
           "spec_verify_probs_filtered", "spec_verify_ragged_filtered", "spec_verify_stream_read",
           "spec_verify_probs_noalloc", "spec_verify_profile_every")
SV_NOALLOC_SCRATCH_BYTES = 16 << 20

_lib = None


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what} failed with status {status}: {status_string(status)}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load the library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, u32, i64, f64, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_int64,
                                  ctypes.c_double, ctypes.c_size_t)
    lib.spec_verify_workspace_size.argtypes = [i64, i32]
    lib.spec_verify_workspace_size.restype = sz
    lib.spec_verify_status_string.argtypes = [ctypes.c_int]
    lib.spec_verify_status_string.restype = ctypes.c_char_p
    lib.spec_verify_version.argtypes = []
    lib.spec_verify_version.restype = ctypes.c_int
    lib.spec_verify_selftest_exp2.argtypes = [vp, vp]
    lib.spec_verify_selftest_exp2.restype = ctypes.c_int
    lib.spec_verify_stream_read.argtypes = [vp, sz, vp, vp]
    lib.spec_verify_stream_read.restype = ctypes.c_int
    lib.spec_verify_exp2_error_bound.argtypes = []
    lib.spec_verify_exp2_error_bound.restype = ctypes.c_double
    lib.spec_verify_profile_start.argtypes = [u32, i32]
    lib.spec_verify_profile_start.restype = ctypes.c_int
    lib.spec_verify_profile_every.argtypes = [i32]
    lib.spec_verify_profile_every.restype = ctypes.c_int
    lib.spec_verify_profile_stop.argtypes = [vp, vp]
    lib.spec_verify_profile_stop.restype = ctypes.c_int
    lib.spec_verify_probs.argtypes = [vp, ctypes.c_int, vp, vp, vp, i32, i32, i32, f64, u32, vp, vp, vp, vp, sz, vp]
    lib.spec_verify_probs.restype = ctypes.c_int
    lib.spec_verify_probs_noalloc.argtypes = [vp, ctypes.c_int, vp, vp, vp, i32, i32, i32, f64, u32, vp, vp, vp, vp]
    lib.spec_verify_probs_noalloc.restype = ctypes.c_int
    lib.spec_verify_greedy.argtypes = [vp, ctypes.c_int, vp, i32, i32, i32, vp, vp, vp, sz, vp]
    lib.spec_verify_greedy.restype = ctypes.c_int
    lib.spec_verify_ragged.argtypes = [vp, ctypes.c_int, vp, vp, vp, vp, i32, i32, i32, f64, u32, vp, vp, vp, vp,
                                       sz, vp]
    lib.spec_verify_ragged.restype = ctypes.c_int
    lib.spec_verify_probs_filtered.argtypes = [vp, ctypes.c_int, vp, vp, vp, i32, i32, i32, f64, i32, f64, vp, vp,
                                               vp, sz, vp]
    lib.spec_verify_probs_filtered.restype = ctypes.c_int
    lib.spec_verify_ragged_filtered.argtypes = [vp, ctypes.c_int, vp, vp, vp, vp, i32, i32, i32, f64, i32, f64, vp,
                                                vp, vp, sz, vp]
    lib.spec_verify_ragged_filtered.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().spec_verify_status_string(int(status)).decode()


def workspace_size(num_target_rows: int, vocab_size: int) -> int:
    return int(load().spec_verify_workspace_size(int(num_target_rows), int(vocab_size)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SV_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return SV_DTYPE_BF16
    raise TypeError(f"target logits must be float32 or bfloat16, got {t.dtype}")


def _check(t, name, dtype=None, device=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _launch_stream(device, stream):
    """The stream the library's kernels are enqueued on: `stream`, else torch's
    current stream of `device`."""
    return stream if stream is not None else torch.cuda.current_stream(device)


def _handle(s):
    return ctypes.c_void_p(s.cuda_stream)


def _workspace(rows, vocab, device, workspace):
    """The library needs a zero-filled workspace on first use (it leaves it
    ready for the next call, of any kind and shape); a fresh one is allocated
    zeroed. Called with the launch stream current (see the verify functions),
    so that the zero-fill is ordered before the library's kernels and the
    allocator ties the memory to the stream that uses it."""
    need = workspace_size(rows, vocab)
    if workspace is None:
        workspace = torch.zeros(max(need, 512), dtype=torch.uint8, device=device)
    elif workspace.numel() < need:
        raise ValueError(f"workspace of {workspace.numel()} bytes, {need} needed")
    return workspace, need


def verify_probs(logits, draft_probs, draft_tokens, uniforms, temperature, flags=0, row_stats=False,
                 workspace=None, stream=None):
    """logits [B, g+1, V] f32/bf16; draft_probs [B, g, V] f32 or None (one-hot);
    draft_tokens [B, g] int64; uniforms [B, g+1] f32. Returns
    (out_tokens [B, g+1] int64, num_accepted [B] int32, row_stats or None, workspace)."""
    lib = load()
    dev = logits.device
    if logits.dim() != 3:
        raise ValueError("logits must be [B, gamma+1, V]")
    B, g1, V = logits.shape
    g = g1 - 1
    _check(logits, "logits", device=dev)
    _check(draft_probs, "draft_probs", torch.float32, dev)
    _check(draft_tokens, "draft_tokens", torch.int64, dev)
    _check(uniforms, "uniforms", torch.float32, dev)
    if draft_probs is not None and tuple(draft_probs.shape) != (B, g, V):
        raise ValueError("draft_probs must be [B, gamma, V]")
    if tuple(draft_tokens.shape) != (B, g) or tuple(uniforms.shape) != (B, g1):
        raise ValueError("draft_tokens must be [B, gamma] and uniforms [B, gamma+1]")
    s = _launch_stream(dev, stream)
    with torch.cuda.stream(s):  # outputs and a fresh workspace belong to the launch stream
        out = torch.empty((B, g1), dtype=torch.int64, device=dev)
        nacc = torch.empty((B,), dtype=torch.int32, device=dev)
        stats = torch.empty((B, g1, 4), dtype=torch.float32, device=dev) if row_stats else None
        workspace, need = _workspace(B * g1, V, dev, workspace)
        rc = lib.spec_verify_probs(_ptr(logits), _dtype_code(logits), _ptr(draft_probs), _ptr(draft_tokens),
                                   _ptr(uniforms), B, g, V, float(temperature), int(flags), _ptr(out), _ptr(nacc),
                                   _ptr(stats), _ptr(workspace), workspace.numel(), _handle(s))
    if rc != 0:
        raise SpecVerifyError(rc, "spec_verify_probs")
    return out, nacc, stats, workspace


def verify_probs_noalloc(logits, draft_probs, draft_tokens, uniforms, temperature, flags=0, row_stats=False,
                         out=None, stream=None):
    """verify_probs through spec_verify_probs_noalloc: no workspace (the
    library's fixed per-device scratch instead), and with `out` = (out_tokens,
    num_accepted[, row_stats]) given, no allocation here either. Returns
    (out_tokens, num_accepted, row_stats or None)."""
    lib = load()
    dev = logits.device
    if logits.dim() != 3:
        raise ValueError("logits must be [B, gamma+1, V]")
    B, g1, V = logits.shape
    g = g1 - 1
    _check(logits, "logits", device=dev)
    _check(draft_probs, "draft_probs", torch.float32, dev)
    _check(draft_tokens, "draft_tokens", torch.int64, dev)
    _check(uniforms, "uniforms", torch.float32, dev)
    if draft_probs is not None and tuple(draft_probs.shape) != (B, g, V):
        raise ValueError("draft_probs must be [B, gamma, V]")
    if tuple(draft_tokens.shape) != (B, g) or tuple(uniforms.shape) != (B, g1):
        raise ValueError("draft_tokens must be [B, gamma] and uniforms [B, gamma+1]")
    s = _launch_stream(dev, stream)
    with torch.cuda.stream(s):
        if out is None:
            o = torch.empty((B, g1), dtype=torch.int64, device=dev)
            nacc = torch.empty((B,), dtype=torch.int32, device=dev)
            stats = torch.empty((B, g1, 4), dtype=torch.float32, device=dev) if row_stats else None
        else:
            o, nacc = out[0], out[1]
            stats = out[2] if row_stats else None
            _check(o, "out_tokens", torch.int64, dev)
            _check(nacc, "num_accepted", torch.int32, dev)
            _check(stats, "row_stats", torch.float32, dev)
        rc = lib.spec_verify_probs_noalloc(_ptr(logits), _dtype_code(logits), _ptr(draft_probs), _ptr(draft_tokens),
                                           _ptr(uniforms), B, g, V, float(temperature), int(flags), _ptr(o),
                                           _ptr(nacc), _ptr(stats), _handle(s))
    if rc != 0:
        raise SpecVerifyError(rc, "spec_verify_probs_noalloc")
    return o, nacc, stats


def verify_greedy(logits, draft_tokens, workspace=None, stream=None):
    """Argmax verification. Returns (out_tokens, num_accepted, workspace)."""
    lib = load()
    dev = logits.device
    B, g1, V = logits.shape
    g = g1 - 1
    _check(logits, "logits", device=dev)
    _check(draft_tokens, "draft_tokens", torch.int64, dev)
    if tuple(draft_tokens.shape) != (B, g):
        raise ValueError("draft_tokens must be [B, gamma]")
    s = _launch_stream(dev, stream)
    with torch.cuda.stream(s):
        out = torch.empty((B, g1), dtype=torch.int64, device=dev)
        nacc = torch.empty((B,), dtype=torch.int32, device=dev)
        workspace, need = _workspace(B * g1, V, dev, workspace)
        rc = lib.spec_verify_greedy(_ptr(logits), _dtype_code(logits), _ptr(draft_tokens), B, g, V, _ptr(out),
                                    _ptr(nacc), _ptr(workspace), workspace.numel(), _handle(s))
    if rc != 0:
        raise SpecVerifyError(rc, "spec_verify_greedy")
    return out, nacc, workspace


def verify_ragged(logits, draft_probs, draft_tokens, cu_num_draft_tokens, uniforms, temperature, flags=0,
                  row_stats=False, workspace=None, stream=None):
    """logits [T+B, V]; draft_probs [T, V] or None; draft_tokens [T] int64;
    cu_num_draft_tokens [B+1] int32; uniforms [T+B] f32. Returns
    (out_tokens [T+B], num_accepted [B], row_stats or None, workspace)."""
    lib = load()
    dev = logits.device
    nb = cu_num_draft_tokens.numel() - 1
    T = draft_tokens.numel()
    V = logits.shape[-1]
    _check(logits, "logits", device=dev)
    _check(draft_probs, "draft_probs", torch.float32, dev)
    _check(draft_tokens, "draft_tokens", torch.int64, dev)
    _check(cu_num_draft_tokens, "cu_num_draft_tokens", torch.int32, dev)
    _check(uniforms, "uniforms", torch.float32, dev)
    if tuple(logits.shape) != (T + nb, V) or uniforms.numel() != T + nb:
        raise ValueError("logits must be [T+B, V] and uniforms [T+B]")
    if draft_probs is not None and tuple(draft_probs.shape) != (T, V):
        raise ValueError("draft_probs must be [T, V]")
    s = _launch_stream(dev, stream)
    with torch.cuda.stream(s):
        out = torch.empty((T + nb,), dtype=torch.int64, device=dev)
        nacc = torch.empty((nb,), dtype=torch.int32, device=dev)
        stats = torch.empty((T + nb, 4), dtype=torch.float32, device=dev) if row_stats else None
        workspace, need = _workspace(T + nb, V, dev, workspace)
        rc = lib.spec_verify_ragged(_ptr(logits), _dtype_code(logits), _ptr(draft_probs), _ptr(draft_tokens),
                                    _ptr(cu_num_draft_tokens), _ptr(uniforms), nb, T, V, float(temperature),
                                    int(flags), _ptr(out), _ptr(nacc), _ptr(stats), _ptr(workspace),
                                    workspace.numel(), _handle(s))
    if rc != 0:
        raise SpecVerifyError(rc, "spec_verify_ragged")
    return out, nacc, stats, workspace


def verify_probs_filtered(logits, draft_probs, draft_tokens, uniforms, temperature, top_k=0, top_p=1.0,
                          workspace=None, stream=None):
    """verify_probs on the target adjusted by top-k (top_k <= 0 or >= V: off)
    and top-p (in (0, 1], 1: off); draft_probs required. Returns
    (out_tokens [B, g+1] int64, num_accepted [B] int32, workspace)."""
    lib = load()
    dev = logits.device
    if logits.dim() != 3:
        raise ValueError("logits must be [B, gamma+1, V]")
    B, g1, V = logits.shape
    g = g1 - 1
    _check(logits, "logits", device=dev)
    _check(draft_probs, "draft_probs", torch.float32, dev)
    _check(draft_tokens, "draft_tokens", torch.int64, dev)
    _check(uniforms, "uniforms", torch.float32, dev)
    if draft_probs is None or tuple(draft_probs.shape) != (B, g, V):
        raise ValueError("draft_probs must be [B, gamma, V]")
    if tuple(draft_tokens.shape) != (B, g) or tuple(uniforms.shape) != (B, g1):
        raise ValueError("draft_tokens must be [B, gamma] and uniforms [B, gamma+1]")
    s = _launch_stream(dev, stream)
    with torch.cuda.stream(s):
        out = torch.empty((B, g1), dtype=torch.int64, device=dev)
        nacc = torch.empty((B,), dtype=torch.int32, device=dev)
        workspace, need = _workspace(B * g1, V, dev, workspace)
        rc = lib.spec_verify_probs_filtered(_ptr(logits), _dtype_code(logits), _ptr(draft_probs),
                                            _ptr(draft_tokens), _ptr(uniforms), B, g, V, float(temperature),
                                            int(top_k), float(top_p), _ptr(out), _ptr(nacc), _ptr(workspace),
                                            workspace.numel(), _handle(s))
    if rc != 0:
        raise SpecVerifyError(rc, "spec_verify_probs_filtered")
    return out, nacc, workspace


def verify_ragged_filtered(logits, draft_probs, draft_tokens, cu_num_draft_tokens, uniforms, temperature, top_k=0,
                           top_p=1.0, workspace=None, stream=None):
    """verify_ragged on the target adjusted by top-k and top-p (see
    verify_probs_filtered). Returns (out_tokens [T+B], num_accepted [B], workspace)."""
    lib = load()
    dev = logits.device
    nb = cu_num_draft_tokens.numel() - 1
    T = draft_tokens.numel()
    V = logits.shape[-1]
    _check(logits, "logits", device=dev)
    _check(draft_probs, "draft_probs", torch.float32, dev)
    _check(draft_tokens, "draft_tokens", torch.int64, dev)
    _check(cu_num_draft_tokens, "cu_num_draft_tokens", torch.int32, dev)
    _check(uniforms, "uniforms", torch.float32, dev)
    if tuple(logits.shape) != (T + nb, V) or uniforms.numel() != T + nb:
        raise ValueError("logits must be [T+B, V] and uniforms [T+B]")
    if draft_probs is None or tuple(draft_probs.shape) != (T, V):
        raise ValueError("draft_probs must be [T, V]")
    s = _launch_stream(dev, stream)
    with torch.cuda.stream(s):
        out = torch.empty((T + nb,), dtype=torch.int64, device=dev)
        nacc = torch.empty((nb,), dtype=torch.int32, device=dev)
        workspace, need = _workspace(T + nb, V, dev, workspace)
        rc = lib.spec_verify_ragged_filtered(_ptr(logits), _dtype_code(logits), _ptr(draft_probs),
                                             _ptr(draft_tokens), _ptr(cu_num_draft_tokens), _ptr(uniforms), nb, T, V,
                                             float(temperature), int(top_k), float(top_p), _ptr(out), _ptr(nacc),
                                             _ptr(workspace), workspace.numel(), _handle(s))
    if rc != 0:
        raise SpecVerifyError(rc, "spec_verify_ragged_filtered")
    return out, nacc, workspace


def selftest_exp2(device=None, stream=None):
    """Measured max relative error of the device's fp32 exp2 on [-126, 0] and
    the bound the certified fast path assumes: (measured, assumed)."""
    lib = load()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    s = _launch_stream(dev, stream)
    with torch.cuda.stream(s):
        out = torch.empty(1, dtype=torch.float64, device=dev)
        rc = lib.spec_verify_selftest_exp2(_ptr(out), _handle(s))
    if rc != 0:
        raise SpecVerifyError(rc, "spec_verify_selftest_exp2")
    return float(out.item()), float(lib.spec_verify_exp2_error_bound())


def stream_read(buf, out=None, stream=None):
    """Read the device buffer `buf` (contiguous, 16-byte aligned, a multiple of
    16 bytes) once; returns a one-element int64 tensor holding the sum of its
    32-bit words as unsigned integers modulo 2^64 (bit pattern)."""
    lib = load()
    dev = buf.device
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    nbytes = buf.numel() * buf.element_size()
    s = _launch_stream(dev, stream)
    with torch.cuda.stream(s):
        out = torch.empty(1, dtype=torch.int64, device=dev) if out is None else out
        rc = lib.spec_verify_stream_read(_ptr(buf), nbytes, _ptr(out), _handle(s))
    if rc != 0:
        raise SpecVerifyError(rc, "spec_verify_stream_read")
    return out


def profile_start(kernels=(SV_PROFILE_ROWS, SV_PROFILE_REQUEST), capacity=1024, every=1):
    """Start recording HIP events around the given kernels (see the header),
    on one call in `every`."""
    mask = 0
    for k in kernels:
        mask |= 1 << int(k)
    rc = load().spec_verify_profile_start(mask, int(capacity))
    if rc != 0:
        raise SpecVerifyError(rc, "spec_verify_profile_start")
    rc = load().spec_verify_profile_every(int(every))
    if rc != 0:
        raise SpecVerifyError(rc, "spec_verify_profile_every")


def profile_stop():
    """Stop recording; returns {kernel id: (summed ms, launches)}."""
    total = (ctypes.c_double * 3)()
    count = (ctypes.c_int32 * 3)()
    rc = load().spec_verify_profile_stop(ctypes.cast(total, ctypes.c_void_p), ctypes.cast(count, ctypes.c_void_p))
    if rc != 0:
        raise SpecVerifyError(rc, "spec_verify_profile_stop")
    return {k: (float(total[k]), int(count[k])) for k in (SV_PROFILE_ROWS, SV_PROFILE_REQUEST, SV_PROFILE_ROWS_FIRST)}


RECORDS_OFFSET = 256  # the records follow a 256-byte block of counters


def row_records(workspace, num_target_rows):
    """Diagnostics: the per-row {token, row_flags} records the last call left
    in `workspace` (int32 [rows, 2])."""
    rec = workspace[RECORDS_OFFSET: RECORDS_OFFSET + num_target_rows * 8]
    return rec.view(torch.int32).view(num_target_rows, 2)
