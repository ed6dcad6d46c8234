// specverify.hip - HIP kernels (gfx950) and C ABI of the batched
// speculative-sampling verifier. The operation is declared and cited in
// include/specverify.h; this file holds the kernels and the host layer.
//
// Method (bloss0m.com, "Speculative Decoding：用小模型打草稿、大模型一次驗…",
// section "技術機制 / Technical mechanism", Algorithm 1 and speculative
// sampling; blog.vllbc.top, "Speculative Decoding：draft 先猜，target 一次验证",
// Algorithm 1): p = softmax(logits / T) per target row; draft x_i is kept iff
// p_i(x_i) > 0 and u_i q_i(x_i) <= p_i(x_i); the first rejection n decides the
// emitted token, drawn from norm(max(0, p_n - q_n)) (from p_n when that mass
// is <= 1e-8, timinsight.com "Step 2") or from p_{g+1} when all drafts pass.
//
// Kernel design (MI355X: 256 CUs in 8 XCDs, wave64, 160 KB LDS per CU,
// ~8 TB/s HBM3E; the path is bandwidth-bound, there is no dense contraction):
//  * one 512-thread block (8 waves) per target row; draft rows are dispatched
//    first and bonus rows last, so the round-robin dispatch over the XCDs
//    spreads the heavy rows (logits + q) evenly and light rows fill the tail;
//  * a row is cut into 2048-element tiles; wave w streams tiles w, w+8, ...
//    with 16-byte loads (32 elements per lane per tile), double-buffered so the
//    next tile's loads are in flight while one is reduced; loads are issued
//    unconditionally (addresses clamped into the row) so the compiler waits
//    only for the tile it consumes. Each tile leaves its sum (and, in the
//    logits pass, its running max) in LDS, so the inverse-CDF search re-reads
//    one tile only;
//  * pass 1 reads the logits: running row max per wave and the tile sums of
//    exp2((l - M_j) s), one sweep per tile (a ballot re-sums a tile that
//    raised the maximum); pass 2 (draft rows with q whose replacement is
//    needed) re-reads the logits and reads q once: tile sums of max(0, p - q);
//  * every row computes its replacement or bonus sample in parallel
//    (speculatively); a select kernel then picks, per request, the first
//    rejection. A draft row whose own test passes skips its residual (its
//    sample can never be emitted) unless SV_FLAG_ALL_RESIDUALS is set;
//  * exactness: the fp32 fast path carries a rigorous error bound for Z, for
//    every prefix of the sampling CDF and for p(x). When the accept decision,
//    the 1e-8 fallback decision or the sampled token is not separated from its
//    threshold by twice the bound, the row is appended to a list and
//    recomputed in fp64 by three small kernels that spread the work over the
//    whole GPU. Results therefore equal exact arithmetic except within ~1e-15
//    relative of a decision boundary.
//
// All kernels read inputs only in bounds, whatever the device-side inputs
// hold (out-of-range tokens, bad offsets), and every loop has a fixed bound.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "specverify.h"

// The error bound of the fast path follows the rounding steps as written:
// no multiply-add is fused unless the source says fmaf.
#pragma clang fp contract(off)

namespace {

constexpr int kNT = 256;                // threads per block of the fixed-size kernels
constexpr int kWaves = kNT / 64;        // waves per row block
constexpr int kTile = 2048;             // elements per tile (one wave, 32 per lane)
constexpr int kLaneElems = kTile / 64;  // 32
constexpr int kSelectNT = 256;

// ----------------------------------------------------------------------------
// numerics constants of the fast path error bound
constexpr double kU = 5.9604644775390625e-08;   // 2^-24, fp32 unit roundoff
constexpr double kLn2 = 0.6931471805599453;
constexpr double kEpsExp = 2.384185791015625e-07;  // 2^-22 >= relative error of v_exp_f32
// per-term relative error of e_k ~ exp2(a_k): C1 |a_k| + C0 (see bound_terms)
constexpr double kC1 = 4.0 * kU * kLn2;
constexpr double kC0 = 2.0 * kEpsExp + 3.0 * kU;
// fp32 summation: a lane sums its 32 terms of a tile in 4 interleaved
// accumulators (<= 7 additions each) joined by a 2-level tree, then a 6-level
// wave tree and one product (tile rescale): every term passes <= 16 roundings.
// The in-tile search sums 8 terms per thread (<= 7). Bound: gamma_20.
constexpr double kSumErr = 20.0 * kU;
constexpr double kSafety = 1.25;
constexpr double kFallbackMass = 1e-8;  // timinsight.com "Step 2" constant

constexpr uint32_t kRowAccepted = SV_ROW_ACCEPTED;
constexpr uint32_t kRowExact = SV_ROW_EXACT;
constexpr uint32_t kRowResidual = SV_ROW_RESIDUAL;
constexpr uint32_t kRowFallback = SV_ROW_FALLBACK;

// ----------------------------------------------------------------------------
// element access

template <typename LT>
struct LogitTraits;
template <>
struct LogitTraits<float> {
  static constexpr int kVecElems = 4;  // 16 bytes
};
template <>
struct LogitTraits<uint16_t> {  // bf16 bit patterns
  static constexpr int kVecElems = 8;
};

__device__ __forceinline__ float to_float(float v) { return v; }
__device__ __forceinline__ float to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Elements per contiguous run a lane owns in a tile (VEC) or 1 (scalar path).
template <typename LT, bool VEC>
struct Lay {
  static constexpr int kE = VEC ? LogitTraits<LT>::kVecElems : 1;
  static constexpr int kRuns = kLaneElems / kE;
  // element k (0..31) of `lane` in the tile starting at `base`
  __device__ static __forceinline__ int index(int base, int lane, int k) {
    return base + ((k / kE) * 64 + lane) * kE + (k % kE);
  }
  // inverse of index(): the k at which `lane` holds tile offset d (0..kTile-1),
  // or -1 if another lane holds it
  __device__ static __forceinline__ int local(int d, int lane) {
    const int run = d / (64 * kE), w = d % (64 * kE);
    return (w / kE == lane) ? run * kE + (w % kE) : -1;
  }
};

// Load the lane's 16 logits of a tile as fp32; out-of-range elements are -inf.
template <typename LT, bool VEC>
__device__ __forceinline__ void load_logits(const LT* __restrict__ row, int V, int base, int lane,
                                            float (&v)[kLaneElems]) {
  using L = Lay<LT, VEC>;
#pragma unroll
  for (int r = 0; r < L::kRuns; ++r) {
    const int i0 = base + (r * 64 + lane) * L::kE;
    if constexpr (VEC && sizeof(LT) == 2) {
      if (i0 < V) {
        const uint4 d = *reinterpret_cast<const uint4*>(row + i0);
        const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          v[r * 8 + 2 * h] = __uint_as_float(w[h] << 16);
          v[r * 8 + 2 * h + 1] = __uint_as_float(w[h] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[r * 8 + e] = -INFINITY;
      }
    } else if constexpr (VEC) {
      if (i0 < V) {
        const float4 d = *reinterpret_cast<const float4*>(row + i0);
        v[r * 4 + 0] = d.x;
        v[r * 4 + 1] = d.y;
        v[r * 4 + 2] = d.z;
        v[r * 4 + 3] = d.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[r * 4 + e] = -INFINITY;
      }
    } else {
      v[r] = i0 < V ? to_float(row[i0]) : -INFINITY;
    }
  }
}

// Load q for the same 16 elements; out-of-range elements are 0.
template <typename LT, bool VEC>
__device__ __forceinline__ void load_q(const float* __restrict__ row, int V, int base, int lane,
                                       float (&q)[kLaneElems]) {
  using L = Lay<LT, VEC>;
#pragma unroll
  for (int r = 0; r < L::kRuns; ++r) {
    const int i0 = base + (r * 64 + lane) * L::kE;
    const bool in = i0 < V;
    if constexpr (VEC) {
      const int ic = in ? i0 : V - L::kE;
#pragma unroll
      for (int h = 0; h < L::kE / 4; ++h) {
        const float4 d = *reinterpret_cast<const float4*>(row + ic + 4 * h);
        q[r * L::kE + 4 * h + 0] = in ? d.x : 0.f;
        q[r * L::kE + 4 * h + 1] = in ? d.y : 0.f;
        q[r * L::kE + 4 * h + 2] = in ? d.z : 0.f;
        q[r * L::kE + 4 * h + 3] = in ? d.w : 0.f;
      }
    } else {
      const float d = row[in ? i0 : V - 1];
      q[r] = in ? d : 0.f;
    }
  }
}

// A lane's 32 logits of one tile kept packed as loaded (bf16 pairs or fp32),
// so a prefetched tile costs 16 (bf16) or 32 (fp32) VGPRs.
//   load():        unconditional loads with the address clamped into the row,
//                  so the compiler counts outstanding loads and waits only for
//                  the tile it consumes. Elements past the end of the row hold
//                  copies of the row's last elements: real values (harmless
//                  to a maximum), which every sum must leave out.
//   load_padded(): the same, with elements past the end set to -inf.
template <typename LT, bool VEC>
struct RawTile;

template <>
struct RawTile<uint16_t, true> {
  uint4 d[4];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ row, int V, int base, int lane) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i0 = base + (r * 64 + lane) * 8;
      d[r] = *reinterpret_cast<const uint4*>(row + min(i0, V - 8));
    }
  }
  __device__ __forceinline__ void load_padded(const uint16_t* __restrict__ row, int V, int base, int lane) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i0 = base + (r * 64 + lane) * 8;
      const uint4 v = *reinterpret_cast<const uint4*>(row + min(i0, V - 8));
      // per-component selects (a select on the whole vector becomes a branch
      // around the load); 0xff80 is bf16 -inf
      const bool in = i0 < V;
      d[r].x = in ? v.x : 0xff80ff80u;
      d[r].y = in ? v.y : 0xff80ff80u;
      d[r].z = in ? v.z : 0xff80ff80u;
      d[r].w = in ? v.w : 0xff80ff80u;
    }
  }
  __device__ __forceinline__ float get(int k) const {
    const uint4& q = d[k >> 3];
    const int h = (k & 7) >> 1;
    const uint32_t w = h == 0 ? q.x : h == 1 ? q.y : h == 2 ? q.z : q.w;
    return (k & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
  // same value as get(k), written differently so that the compiler re-derives
  // it from the packed word instead of keeping 32 unpacked values live
  __device__ __forceinline__ float get2(int k) const {
    const uint4& q = d[k >> 3];
    const int h = (k & 7) >> 1;
    const uint32_t w = h == 0 ? q.x : h == 1 ? q.y : h == 2 ? q.z : q.w;
    return (k & 1) ? __uint_as_float((w >> 16) << 16) : __uint_as_float((w & 0xffffu) << 16);
  }
};

template <>
struct RawTile<float, true> {
  float4 d[8];
  __device__ __forceinline__ void load(const float* __restrict__ row, int V, int base, int lane) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int i0 = base + (r * 64 + lane) * 4;
      d[r] = *reinterpret_cast<const float4*>(row + min(i0, V - 4));
    }
  }
  __device__ __forceinline__ void load_padded(const float* __restrict__ row, int V, int base, int lane) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int i0 = base + (r * 64 + lane) * 4;
      const float4 v = *reinterpret_cast<const float4*>(row + min(i0, V - 4));
      const bool in = i0 < V;
      d[r].x = in ? v.x : -INFINITY;
      d[r].y = in ? v.y : -INFINITY;
      d[r].z = in ? v.z : -INFINITY;
      d[r].w = in ? v.w : -INFINITY;
    }
  }
  __device__ __forceinline__ float get(int k) const {
    const float4& q = d[k >> 2];
    const int h = k & 3;
    return h == 0 ? q.x : h == 1 ? q.y : h == 2 ? q.z : q.w;
  }
  __device__ __forceinline__ float get2(int k) const { return get(k); }
};

template <typename LT>
struct RawTile<LT, false> {
  float d[kLaneElems];
  __device__ __forceinline__ void load(const LT* __restrict__ row, int V, int base, int lane) {
#pragma unroll
    for (int r = 0; r < kLaneElems; ++r) d[r] = to_float(row[min(base + r * 64 + lane, V - 1)]);
  }
  __device__ __forceinline__ void load_padded(const LT* __restrict__ row, int V, int base, int lane) {
#pragma unroll
    for (int r = 0; r < kLaneElems; ++r) {
      const int i = base + r * 64 + lane;
      const float v = to_float(row[min(i, V - 1)]);
      d[r] = i < V ? v : -INFINITY;
    }
  }
  __device__ __forceinline__ float get(int k) const { return d[k]; }
  __device__ __forceinline__ float get2(int k) const { return d[k]; }
};

__device__ __forceinline__ float fexp2(float a) { return __builtin_amdgcn_exp2f(a); }

// ----------------------------------------------------------------------------
// reductions

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// Row (16-lane) reduction by DPP: xor 1, xor 2 (quad permutes), then rotate
// by 4 and 8 within the row; every lane ends with its row's total. The four
// row totals are then combined in a fixed order, so every lane of the wave
// holds the same, deterministic result.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x124>(v);
  v += dpp<0x128>(v);
  return ((lane_f(v, 0) + lane_f(v, 16)) + lane_f(v, 32)) + lane_f(v, 48);
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x124>(v));
  v = fmaxf(v, dpp<0x128>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

template <int NT>
struct BlockScratchT {
  double d[NT];
};
using BlockScratch = BlockScratchT<kNT>;

// Sum over the block in a fixed order; every thread gets the same value.
template <int NT>
__device__ double block_sum(double v, BlockScratchT<NT>& s) {
  constexpr int kWaves = NT / 64;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) s.d[wave] = v;
  __syncthreads();
  double r = 0.0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) r += s.d[w];
  __syncthreads();
  return r;
}

// Two fixed-order block sums with one pair of barriers.
template <int NT>
__device__ void block_sum2(double v, double w, BlockScratchT<NT>& s, double& rv, double& rw) {
  constexpr int kWaves = NT / 64;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    v += __shfl_xor(v, o);
    w += __shfl_xor(w, o);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    s.d[wave] = v;
    s.d[kWaves + wave] = w;
  }
  __syncthreads();
  rv = 0.0;
  rw = 0.0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    rv += s.d[k];
    rw += s.d[kWaves + k];
  }
  __syncthreads();
}

template <int NT>
__device__ float block_max(float v, BlockScratchT<NT>& s) {
  constexpr int kWaves = NT / 64;
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) s.d[wave] = v;
  __syncthreads();
  float r = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) r = fmaxf(r, static_cast<float>(s.d[w]));
  __syncthreads();
  return r;
}

// Exclusive scan over the block's threads in thread order. Thread t gets
// excl_t and incl_t with incl_t == excl_{t+1} bit for bit; `total` is the
// inclusive value of the last thread.
template <int NT>
__device__ void block_scan(double v, BlockScratchT<NT>& s, double& excl, double& incl, double& total) {
  constexpr int kWaves = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  double xe = __shfl_up(x, 1);
  if (lane == 0) xe = 0.0;
  if (lane == 63) s.d[wave] = x;
  __syncthreads();
  double off = 0.0;
  for (int w = 0; w < wave; ++w) off += s.d[w];
  double tot = 0.0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) tot += s.d[w];
  __syncthreads();
  // thread 64w's excl equals the running offset, which is the previous wave's
  // last incl computed with the same association
  excl = lane == 0 ? off : off + xe;
  incl = off + x;
  total = tot;
  // make `total` identical to the last thread's incl
  if (threadIdx.x == NT - 1) s.d[0] = incl;
  __syncthreads();
  total = s.d[0];
  __syncthreads();
}

// ----------------------------------------------------------------------------
// row task decoding (dense: cu == nullptr)

struct Task {
  int b;          // request
  int g;          // drafts of the request
  int i;          // position 0..g (g = bonus row)
  int64_t trow;   // target row
  int64_t drow;   // draft row or -1
  int64_t srow;   // target row holding the sample uniform (bonus row)
  bool valid;
};

__device__ __forceinline__ Task decode_task(int blk, const int32_t* __restrict__ cu, int B, int gamma,
                                            int ndraft) {
  Task t;
  t.valid = true;
  int d0, d1;
  if (blk < ndraft) {
    t.drow = blk;
    if (cu) {
      int lo = 0, hi = B;  // largest b with cu[b] <= drow
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu[mid] <= blk) lo = mid; else hi = mid;
      }
      t.b = lo;
    } else {
      t.b = blk / gamma;
    }
  } else {
    t.drow = -1;
    t.b = blk - ndraft;
  }
  if (cu) {
    d0 = cu[t.b];
    d1 = cu[t.b + 1];
    if (d0 < 0 || d1 < d0 || d1 > ndraft) {
      t.valid = false;
      d0 = d1 = 0;
    }
  } else {
    d0 = t.b * gamma;
    d1 = d0 + gamma;
  }
  t.g = d1 - d0;
  if (t.drow >= 0) {
    t.i = static_cast<int>(t.drow - d0);
    if (t.i < 0 || t.i >= t.g) t.valid = false;
  } else {
    t.i = t.g;
  }
  t.trow = static_cast<int64_t>(d0) + t.i + t.b;
  t.srow = static_cast<int64_t>(d1) + t.b;
  return t;
}

// ----------------------------------------------------------------------------
// probabilistic verification

struct ProbsArgs {
  const void* logits;
  const float* q;        // nullptr: one-hot drafts
  const int64_t* x;
  const float* u;
  const int32_t* cu;     // nullptr: dense
  int2* ws;
  float* stats;          // nullptr: no statistics
  double s64;            // log2(e) / T
  float s32;             // fp32(s64)
  double temperature;
  int B, gamma, ndraft, V;
  uint32_t flags;
  int* xcount;    // list of rows for the fp64 path (see ExactArgs)
  int2* xlist;
  double4* rstat; // lazy mode: {m, Z, sum e|a|} of deferred rows
};

struct RowShared {
  float wmax[16];  // per-wave maxima (blocks of up to 1024 threads)
  float m;
  double z;        // Z (e-units)
  double px;
  int accepted;
  int uncertain;
  int found;
  int token;
  double c_lo, c_hi;
  int tile;
  double p_before;
  int cross;
  int lastpos;
};

// Bound on sum_k |e~_k - e_k| in e-units (e_k relative to the row max):
// each term has relative error <= C1 |a_k| + C0, so the sum is bounded by
// C1 sum_k e_k |a_k| + C0 Z (the sums, computed in floating point, are
// inflated by 1%). Terms that underflow add at most 2^-126 each (1e-30 total).
__device__ __forceinline__ double bound_terms(double z, double sum_e_abs_a) {
  return kSafety * (kC1 * 1.01 * sum_e_abs_a + kC0 * 1.01 * z + 1e-30);
}

template <typename LT>
__device__ __forceinline__ float logit_at(const LT* row, int64_t k) {
  return to_float(row[k]);
}

// ----------------------------------------------------------------------------
// fp64 path for the rows the fast kernel could not certify.
//
// The fast kernel appends such a row to a list in the workspace; three small
// fixed-grid kernels then spread the fp64 work over the whole GPU:
//   exact_tiles_kernel:    one (row, tile) item per block iteration; fp64 sum of
//                          e_k = 2^((l_k - m) log2(e) / T) over the tile.
//   exact_residual_kernel: same items, rows with q only; fp64 sum of
//                          max(0, e_k / Z - q_k) over the tile.
//   exact_finish_kernel:   one row per block iteration; accept test, residual
//                          mass, fallback, tile search and in-tile search, all
//                          in fp64; writes the row's record and statistics.
// With an empty list each kernel reads the count and exits.

constexpr uint32_t kRowNeedExact = 0x200u;  // set by the fast kernel, cleared by exact_finish_kernel
constexpr uint32_t kRowDeferred = SV_ROW_DEFERRED;
constexpr uint32_t kFlagLazy = 0x80000000u;  // internal: set by the host for the lazy mode
constexpr int kExactGrid = 512;             // blocks of the item kernels
constexpr int kExactPer = kTile / kNT;      // elements per thread of one tile (8)

struct ExactArgs {
  int* count;     // number of listed rows (reset to 0 by the select kernel)
  int2* list;     // {row block index, bits of the row max m}
  double* etile;  // [rows][nt] fp64 tile sums of e
  double* wtile;  // [rows][nt] fp64 tile sums of max(0, p - q)
  int nt;
  int rows;
};

// Thread t of a block covers elements [base + 8t, base + 8t + 8) of a tile,
// so the tile is covered in ascending token order by ascending threads.
template <typename LT>
__device__ __forceinline__ void load8(const LT* __restrict__ row, int V, int k0, double (&l)[kExactPer]) {
#pragma unroll
  for (int e = 0; e < kExactPer; ++e) {
    const int k = k0 + e;
    l[e] = k < V ? static_cast<double>(to_float(row[k])) : -INFINITY;
  }
}

struct ExactRow {
  Task t;
  const void* lrow;
  const float* qrow;
  int64_t x;
  bool x_ok, is_draft, onehot;
  double m;
};

__device__ __forceinline__ ExactRow exact_row_info(const ProbsArgs& a, const ExactArgs& e, int pos) {
  ExactRow r;
  const int2 li = e.list[pos];
  // a list entry is a row block index of this call; anything else (a
  // workspace that was not zero-filled) is skipped rather than decoded
  const bool in_range = li.x >= 0 && li.x < e.rows;
  r.t = decode_task(in_range ? li.x : 0, a.cu, a.B, a.gamma, a.ndraft);
  r.t.valid = r.t.valid && in_range;
  r.m = static_cast<double>(__int_as_float(li.y));
  r.is_draft = r.t.drow >= 0;
  r.qrow = (r.is_draft && a.q) ? a.q + r.t.drow * static_cast<int64_t>(a.V) : nullptr;
  r.x = r.is_draft ? a.x[r.t.drow] : -1;
  r.x_ok = r.is_draft && r.x >= 0 && r.x < a.V;
  r.onehot = r.is_draft && r.qrow == nullptr;
  r.lrow = nullptr;
  return r;
}

__device__ __forceinline__ int exact_count(const ExactArgs& e) {
  const int n = *e.count;
  return n < 0 ? 0 : (n > e.rows ? e.rows : n);
}

template <typename LT>
__global__ __launch_bounds__(kNT) void exact_tiles_kernel(ProbsArgs a, ExactArgs e) {
  __shared__ BlockScratch sc;
  const int n = exact_count(e);
  const int64_t items = static_cast<int64_t>(n) * e.nt;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int pos = static_cast<int>(it / e.nt), j = static_cast<int>(it % e.nt);
    const ExactRow r = exact_row_info(a, e, pos);
    if (!r.t.valid) continue;
    const LT* lrow = static_cast<const LT*>(a.logits) + r.t.trow * static_cast<int64_t>(a.V);
    double l[kExactPer];
    load8<LT>(lrow, a.V, j * kTile + kExactPer * threadIdx.x, l);
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < kExactPer; ++k) acc += exp2((l[k] - r.m) * a.s64);
    acc = block_sum(acc, sc);
    if (threadIdx.x == 0) e.etile[static_cast<int64_t>(pos) * e.nt + j] = acc;
  }
}

// Z of listed row `pos` from its fp64 tile sums: thread t adds tiles t,
// t + 256, ..., then a fixed-order block sum (identical in every kernel).
__device__ __forceinline__ double exact_z(const double* __restrict__ et, int nt, BlockScratch& sc) {
  double z = 0.0;
  for (int j = threadIdx.x; j < nt; j += kNT) z += et[j];
  return block_sum(z, sc);
}

template <typename LT>
__global__ __launch_bounds__(kNT) void exact_residual_kernel(ProbsArgs a, ExactArgs e) {
  __shared__ BlockScratch sc;
  const int n = exact_count(e);
  const int64_t items = static_cast<int64_t>(n) * e.nt;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int pos = static_cast<int>(it / e.nt), j = static_cast<int>(it % e.nt);
    const ExactRow r = exact_row_info(a, e, pos);
    if (!r.t.valid || r.qrow == nullptr) continue;  // uniform over the block
    const double iz = 1.0 / exact_z(e.etile + static_cast<int64_t>(pos) * e.nt, e.nt, sc);
    const LT* lrow = static_cast<const LT*>(a.logits) + r.t.trow * static_cast<int64_t>(a.V);
    const int k0 = j * kTile + kExactPer * threadIdx.x;
    double l[kExactPer];
    load8<LT>(lrow, a.V, k0, l);
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < kExactPer; ++k) {
      const double q = k0 + k < a.V ? static_cast<double>(r.qrow[k0 + k]) : 0.0;
      acc += fmax(0.0, exp2((l[k] - r.m) * a.s64) * iz - q);
    }
    acc = block_sum(acc, sc);
    if (threadIdx.x == 0) e.wtile[static_cast<int64_t>(pos) * e.nt + j] = acc;
  }
}

template <typename LT>
__global__ __launch_bounds__(kNT) void exact_finish_kernel(ProbsArgs a, ExactArgs e) {
  extern __shared__ double xtile[];  // [nt] e tile sums, [nt] residual tile sums
  __shared__ BlockScratch sc;
  __shared__ RowShared sh;
  const int n = exact_count(e);
  const int tid = threadIdx.x;
  const int nt = e.nt;
  double* ets = xtile;
  double* wts = xtile + nt;
  const int tper = (nt + kNT - 1) / kNT;
  const int tlo = min(nt, tid * tper), thi = min(nt, tlo + tper);
  for (int pos = blockIdx.x; pos < n; pos += gridDim.x) {
    const ExactRow r = exact_row_info(a, e, pos);
    if (!r.t.valid) continue;
    const Task& t = r.t;
    const LT* lrow = static_cast<const LT*>(a.logits) + t.trow * static_cast<int64_t>(a.V);
    const double* et = e.etile + static_cast<int64_t>(pos) * nt;
    const double* wt = e.wtile + static_cast<int64_t>(pos) * nt;
    for (int j = tid; j < nt; j += kNT) {
      ets[j] = et[j];
      wts[j] = r.qrow ? wt[j] : 0.0;
    }
    const double Z = exact_z(et, nt, sc);  // barriers inside also publish ets / wts
    const double iz = 1.0 / Z;
    const double s = a.s64;
    const uint32_t why = static_cast<uint32_t>(a.ws[t.trow].y) & 0x1f0u;

    double ex = 0.0, px = 0.0;
    bool accepted = false;
    if (r.is_draft) {
      if (r.x_ok) {
        ex = exp2((static_cast<double>(logit_at(lrow, r.x)) - r.m) * s);
        px = ex * iz;
      }
      const double qx = r.onehot ? 1.0 : (r.x_ok ? static_cast<double>(r.qrow[r.x]) : 0.0);
      accepted = r.x_ok && px > 0.0 && static_cast<double>(a.u[t.trow]) * qx <= px;
    }
    const bool all_res = (a.flags & SV_FLAG_ALL_RESIDUALS) || a.stats != nullptr;
    uint32_t flags = kRowExact | why | (accepted ? kRowAccepted : 0u);
    int token = -1;
    double rmass = 1.0;
    if (!r.is_draft || !accepted || all_res) {
      // tile values in tile order: mode 1 residual, 2 p without x, 0 p
      int mode = r.is_draft ? (r.onehot ? 2 : 1) : 0;
      const int jx = r.x_ok ? static_cast<int>(r.x / kTile) : -1;
      auto tile_val = [&](int j) -> double {
        if (mode == 1) return wts[j];
        double v = ets[j];
        if (mode == 2 && j == jx) v = fmax(0.0, v - ex);
        return v * iz;
      };
      double tv = 0.0;
      for (int j = tlo; j < thi; ++j) tv += tile_val(j);
      double excl, incl, total;
      block_scan(tv, sc, excl, incl, total);
      if (mode != 0) {
        rmass = total;
        if (total <= kFallbackMass) {
          mode = 0;
          flags |= kRowFallback;
          tv = 0.0;
          for (int j = tlo; j < thi; ++j) tv += tile_val(j);
          block_scan(tv, sc, excl, incl, total);
        }
        flags |= kRowResidual;
      }
      const double tau = static_cast<double>(a.u[t.srow]) * total;
      // crossing tile: smallest positive tile reaching tau, else the last positive tile
      if (tid == 0) {
        sh.cross = 0x7fffffff;
        sh.lastpos = -1;
      }
      __syncthreads();
      if (excl < tau) {
        double c = 0.0;
        int tok = -1, lastpos = -1;
        for (int j = tlo; j < thi && tok < 0; ++j) {
          const double v = tile_val(j);
          c += v;
          if (v > 0.0) {
            lastpos = j;
            if (excl + c >= tau) tok = j;
          }
        }
        if (tok >= 0) atomicMin(&sh.cross, tok);
        if (lastpos >= 0) atomicMax(&sh.lastpos, lastpos);
      }
      __syncthreads();
      const int jt = sh.cross != 0x7fffffff ? sh.cross : (sh.lastpos >= 0 ? sh.lastpos : 0);
      double pbl = 0.0;
      for (int j = tlo; j < thi; ++j)
        if (j < jt) pbl += tile_val(j);
      const double pb = block_sum(pbl, sc);
      // in-tile search, fp64, 8 consecutive elements per thread
      const int k0 = jt * kTile + kExactPer * tid;
      double l[kExactPer], w[kExactPer];
      load8<LT>(lrow, a.V, k0, l);
      double tsum = 0.0;
#pragma unroll
      for (int k = 0; k < kExactPer; ++k) {
        const int kk = k0 + k;
        double v = 0.0;
        if (kk < a.V) {
          const double p = exp2((l[k] - r.m) * s) * iz;
          if (mode == 1) v = fmax(0.0, p - static_cast<double>(r.qrow[kk]));
          else if (mode == 2 && kk == r.x) v = 0.0;
          else v = p;
        }
        w[k] = v;
        tsum += v;
      }
      double e2, i2, t2;
      block_scan(tsum, sc, e2, i2, t2);
      const double tl = tau - pb;
      if (tid == 0) {
        sh.cross = 0x7fffffff;
        sh.lastpos = -1;
      }
      __syncthreads();
      if (e2 < tl) {
        int tok = -1, lastpos = -1;
        double cl = 0.0;
#pragma unroll
        for (int k = 0; k < kExactPer; ++k) {
          cl += w[k];
          if (w[k] > 0.0 && tok < 0) {
            lastpos = k0 + k;
            if (e2 + cl >= tl) tok = k0 + k;
          }
        }
        if (tok >= 0) atomicMin(&sh.cross, tok);
        if (lastpos >= 0) atomicMax(&sh.lastpos, lastpos);
      }
      __syncthreads();
      token = sh.cross != 0x7fffffff ? sh.cross : (sh.lastpos >= 0 ? sh.lastpos : jt * kTile);
      __syncthreads();
    }
    if (tid == 0) {
      a.ws[t.trow] = make_int2(token, static_cast<int>(flags));
      if (a.stats) {
        float* st = a.stats + t.trow * 4;
        st[0] = static_cast<float>(r.m / a.temperature);
        st[1] = static_cast<float>(log(Z));
        st[2] = r.is_draft ? static_cast<float>(px) : NAN;
        st[3] = static_cast<float>(rmass);
      }
    }
    __syncthreads();
  }
}

// Hand a row to the fp64 path: mark its record and append it to the list.
__device__ __forceinline__ void flag_exact(const ProbsArgs& a, const Task& t, uint32_t why, float m,
                                           bool accepted = false) {
  // the accept bit is meaningful unless the accept test itself is the reason
  a.ws[t.trow] = make_int2(-1, static_cast<int>(kRowNeedExact | why | (accepted ? kRowAccepted : 0u)));
  const int pos = atomicAdd(a.xcount, 1);
  const int blk = t.drow >= 0 ? static_cast<int>(t.drow) : a.ndraft + t.b;  // the row's index in the rows grid
  if (pos < a.B + a.ndraft) a.xlist[pos] = make_int2(blk, __float_as_int(m));
}

// Reasons a row was recomputed on the fp64 path (row_flags bits 4..8).
constexpr uint32_t kWhyAccept = SV_ROW_WHY_ACCEPT;
constexpr uint32_t kWhyFallback = SV_ROW_WHY_FALLBACK;
constexpr uint32_t kWhySearch = SV_ROW_WHY_SEARCH;
constexpr uint32_t kWhyMargin = SV_ROW_WHY_MARGIN;
constexpr uint32_t kWhyForced = SV_ROW_WHY_FORCED;

// Draws the token of one row and certifies it: the replacement of a draft row
// with q (pass 2 over logits and q, then the tile and in-tile search), or the
// p-based sample of a bonus or one-hot row from the pass-1 tile sums S, M.
// Writes the row's record (and statistics), or hands the row to the fp64 path.
// Called by every thread of the block.
template <typename LT, bool VEC, int NT, bool WITH_Q>
__device__ void sample_row(const ProbsArgs& a, const Task& t, const LT* __restrict__ lrow,
                           const float* __restrict__ qrow, int xmask, bool accepted, float m, double Z, double bt,
                           double relZ, double px, const float* S, const float* M, float* W,
                           BlockScratchT<NT>& sc, RowShared& sh) {
  constexpr int kWaves = NT / 64;
  constexpr int kSearchPer = kTile / NT;  // elements per thread in the in-tile search
  const int V = a.V;
  const int nt = (V + kTile - 1) / kTile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float s = a.s32;
  const bool is_draft = t.drow >= 0;
  const bool onehot = is_draft && qrow == nullptr;
  const bool want_stats = a.stats != nullptr;
  using Raw = RawTile<LT, VEC>;

  // ---------------- pass 2: residual tile sums (draft rows with q)
  const bool mode_w = WITH_Q && qrow != nullptr;
  const float izr = static_cast<float>(1.0 / Z);
  const float cm = -(m * s);  // c_m, as in pass 1
  if constexpr (WITH_Q) if (mode_w) {
    for (int j = wave; j < nt; j += kWaves) {
      const int base = j * kTile;
      Raw r;
      float q[kLaneElems];
      r.load_padded(lrow, V, base, lane);
      load_q<LT, VEC>(qrow, V, base, lane, q);
      float w4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g8 = 0; g8 < kLaneElems; g8 += 8) {
#pragma unroll
        for (int k = g8; k < g8 + 8; ++k) {
          const float p = fexp2(fmaf(r.get(k), s, cm)) * izr;
          w4[k & 3] += fmaxf(p - q[k], 0.f);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      float ws = (w4[0] + w4[1]) + (w4[2] + w4[3]);
      ws = wave_sum(ws);
      if (lane == 0) W[j] = ws;
    }
    __syncthreads();
  }

  // ---------------- tile-level CDF: prefix over tiles in token order
  // value of tile j in global units: W[j] (p-units) or S[j] * f_j (e-units)
  auto tile_val = [&](int j) -> double {
    if (mode_w) return static_cast<double>(W[j]);
    if (M[j] == -INFINITY) return 0.0;
    const float cj = -(M[j] * s);
    const float f = fexp2(cm - cj);  // bit for bit the factor Z was summed with
    return static_cast<double>(S[j] * f);
  };
  const int tper = (nt + NT - 1) / NT;
  const int tlo = min(nt, tid * tper), thi = min(nt, tlo + tper);
  double tv = 0.0;
  for (int j = tlo; j < thi; ++j) tv += tile_val(j);
  double excl, incl, total;
  block_scan(tv, sc, excl, incl, total);

  // error bound of every CDF prefix (same units as total)
  double dC;
  uint32_t why = 0;
  if (mode_w) {
    const double dp = (bt / Z + relZ + 2.0 * kU) * 1.01;  // sum_k |p~_k - p_k|
    dC = kSafety * (dp + kU + kSumErr * total);
    if (total <= kFallbackMass + 2.0 * dC) why |= kWhyFallback;
  } else {
    dC = kSafety * (bt + kSumErr * Z);
    if (onehot && total / Z <= kFallbackMass + 2.0 * kSafety * (dC / Z + relZ)) why |= kWhyFallback;
  }
  const double tau = static_cast<double>(a.u[t.srow]) * total;
  if (tid == 0) {
    sh.found = 0;
    sh.uncertain = static_cast<int>(why);
  }
  __syncthreads();
  if (!why && tau > 0.0 && excl < tau && incl >= tau) {
    // same sequential association as tv, so the last partial equals tv
    double cl = 0.0;
    for (int j = tlo; j < thi; ++j) {
      const double prev = cl;
      cl += tile_val(j);
      if (excl + cl >= tau) {
        sh.tile = j;
        sh.p_before = excl + prev;
        sh.found = 1;
        break;
      }
    }
  }
  __syncthreads();
  if (!sh.found || sh.uncertain) {
    const uint32_t w2 = sh.uncertain ? static_cast<uint32_t>(sh.uncertain) : kWhySearch;
    if (tid == 0) flag_exact(a, t, w2, m, accepted);
    return;
  }

  // ---------------- in-tile search: kSearchPer consecutive elements per thread
  const int jt = sh.tile;
  const double pb = sh.p_before;
  const int base = jt * kTile + kSearchPer * tid;
  float unit = 1.f;  // global units per local unit
  float cref = cm;   // exponent offset of the local weights (c_j of the tile)
  if (!mode_w) {
    cref = -(M[jt] * s);
    unit = fexp2(cm - cref);
  }
  float wl[kSearchPer];
#pragma unroll
  for (int e = 0; e < kSearchPer; ++e) {
    const int k = base + e;
    float w = 0.f;
    if (k < V) {
      const float l = to_float(lrow[k]);
      const float ek = fexp2(fmaf(l, s, cref));
      if (WITH_Q && mode_w) w = fmaxf(ek * izr - qrow[k], 0.f);
      else w = (k == xmask) ? 0.f : ek;
    }
    wl[e] = w;
  }
  float tsum = 0.f;
#pragma unroll
  for (int e = 0; e < kSearchPer; ++e) tsum += wl[e];
  const double tau_loc = (tau - pb) / static_cast<double>(unit);
  double e2, i2, tot2;
  block_scan(static_cast<double>(tsum), sc, e2, i2, tot2);
  if (tid == 0) sh.found = 0;
  __syncthreads();
  if (e2 < tau_loc && i2 >= tau_loc) {
    float cl = 0.f;
#pragma unroll
    for (int e = 0; e < kSearchPer; ++e) {
      const float prev = cl;
      cl += wl[e];
      if (e2 + static_cast<double>(cl) >= tau_loc) {
        sh.token = base + e;
        sh.c_lo = pb + (e2 + static_cast<double>(prev)) * static_cast<double>(unit);
        sh.c_hi = pb + (e2 + static_cast<double>(cl)) * static_cast<double>(unit);
        sh.found = 1;
        break;
      }
    }
  }
  __syncthreads();
  uint32_t why2 = sh.found ? 0u : kWhySearch;
  if (!why2) {
    // unit conversion adds a relative rounding of ~3u to the local prefix
    const double d2 = 2.0 * (dC + 4.0 * kU * total);
    if (!((tau - sh.c_lo) > d2 && (sh.c_hi - tau) > d2)) why2 = kWhyMargin;
  }
  if (why2) {
    if (tid == 0) flag_exact(a, t, why2, m, accepted);
    return;
  }
  if (tid == 0) {
    uint32_t fl = (accepted ? kRowAccepted : 0u) | (is_draft ? kRowResidual : 0u);
    a.ws[t.trow] = make_int2(sh.token, static_cast<int>(fl));
    if (want_stats) {
      float* st = a.stats + t.trow * 4;
      st[0] = static_cast<float>(static_cast<double>(m) / a.temperature);
      // Z carries the factor 2^D, D = c_m + m s (see pass 1)
      const double shift = static_cast<double>(cm) + static_cast<double>(m) * static_cast<double>(s);
      st[1] = static_cast<float>(log(Z) - shift * kLn2);
      st[2] = is_draft ? static_cast<float>(px) : NAN;
      st[3] = is_draft ? static_cast<float>(mode_w ? total : total / Z) : 1.f;
    }
  }
}

// EAGER: rejected draft rows with q draw their replacement here (eager and
// all-residual modes); otherwise (lazy mode) they are deferred, and the kernel
// has no q pass at all.
template <typename LT, bool VEC, int NT, bool EAGER>
__global__ __launch_bounds__(NT) void probs_rows_kernel(ProbsArgs a) {
  constexpr int kWaves = NT / 64;
  extern __shared__ float dyn[];
  __shared__ BlockScratchT<NT> sc;
  __shared__ RowShared sh;
  using L = Lay<LT, VEC>;
  using Raw = RawTile<LT, VEC>;

  const int V = a.V;
  const int nt = (V + kTile - 1) / kTile;
  float* S = dyn;           // tile sums of exp2((l - M_j) s), local units
  float* M = dyn + nt;      // running max when the tile was summed (>= every element of the tile)
  float* W = dyn + 2 * nt;  // tile sums of max(0, p - q)
  float* EA = dyn + 3 * nt; // tile sums of e |a| (a = the exp argument), for the error bound
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  const Task t = decode_task(blockIdx.x, a.cu, a.B, a.gamma, a.ndraft);
  if (!t.valid) return;  // request with invalid offsets: the select kernel skips it
  const LT* __restrict__ lrow = static_cast<const LT*>(a.logits) + t.trow * static_cast<int64_t>(V);
  const bool is_draft = t.drow >= 0;
  const float* __restrict__ qrow = (is_draft && a.q) ? a.q + t.drow * static_cast<int64_t>(V) : nullptr;
  const int64_t x = is_draft ? a.x[t.drow] : -1;
  const bool x_ok = is_draft && x >= 0 && x < V;
  const bool onehot = is_draft && qrow == nullptr;
  const int xmask = (onehot && x_ok) ? static_cast<int>(x) : -1;
  const float s = a.s32;
  const bool want_stats = a.stats != nullptr;
  const bool all_res = (a.flags & SV_FLAG_ALL_RESIDUALS) || want_stats;
  // the accept test's inputs, loaded now so that they arrive during pass 1
  const float lx = x_ok ? to_float(lrow[x]) : -INFINITY;
  const float qx_in = (x_ok && qrow) ? qrow[x] : 0.f;
  const float u_acc = is_draft ? a.u[t.trow] : 0.f;

  // ---------------- pass 1: per tile j, with reference M_j (the wave's running
  // maximum, >= every element of the tile) and c_j = fl(-M_j s):
  //   S_j = sum_k exp2(a_k),  a_k = fma(l_k, s, c_j)  (<= 0 up to u |c_j|),
  //   EA_j = -sum_k e_k a_k  (for the error bound).
  // The running maximum starts at the block-wide maximum of every wave's first
  // tile, so a tile is rarely summed twice; when a tile does raise it (a
  // wave-wide ballot), the tile is summed again against the new maximum. The
  // next tile's loads are in flight meanwhile. The row's last tile (when it
  // is partial), a tile holding the one-hot draft token, and a tile with a
  // -inf or a NaN (e a = NaN) take the careful sum, which leaves out the
  // elements past the end and the token, and clamps the argument.
  auto tile_sum_careful = [&](const Raw& r, int base, float ref, float& es, float& ea) {
    const float c = -(ref * s);
    const int lpos = (xmask >= base && xmask < base + kTile) ? L::local(xmask - base, lane) : -1;
    const int lim = V - L::index(base, lane, 0);  // element k is in the row iff its offset < lim
    float e4[4] = {0.f, 0.f, 0.f, 0.f};
    float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g8 = 0; g8 < kLaneElems; g8 += 8) {
#pragma unroll
      for (int k = g8; k < g8 + 8; ++k) {
        constexpr int kE = L::kE;
        const int off = (k / kE) * 64 * kE + (k % kE);
        const float arg = fmaxf(fmaf(r.get(k), s, c), -4096.f);
        const float e = (k == lpos || off >= lim) ? 0.f : fexp2(arg);
        e4[k & 3] += e;
        a4[k & 3] = fmaf(e, arg, a4[k & 3]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    es = (e4[0] + e4[1]) + (e4[2] + e4[3]);
    ea = (a4[0] + a4[1]) + (a4[2] + a4[3]);
  };
  float ref = -INFINITY;
  auto tile1 = [&](const Raw& r, int j) {
    const int base = j * kTile;
    const float c = -(ref * s);
    float lm = -INFINITY;
    float e4[4] = {0.f, 0.f, 0.f, 0.f};
    float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kLaneElems; ++k) {
      const float v = r.get(k);
      lm = fmaxf(lm, v);
      const float arg = fmaf(v, s, c);
      const float e = fexp2(arg);
      e4[k & 3] += e;
      a4[k & 3] = fmaf(e, arg, a4[k & 3]);
    }
    float es = (e4[0] + e4[1]) + (e4[2] + e4[3]);
    float ea = (a4[0] + a4[1]) + (a4[2] + a4[3]);
    const bool redo = lm > ref || !(ea == ea) || base + kTile > V || (xmask >= base && xmask < base + kTile);
    if (__any(redo)) {
      ref = fmaxf(ref, wave_max(lm));
      es = 0.f;
      ea = 0.f;
      if (ref != -INFINITY) tile_sum_careful(r, base, ref, es, ea);
    }
    es = wave_sum(es);
    ea = wave_sum(ea);
    if (lane == 0) {
      S[j] = es;
      M[j] = ref;
      EA[j] = -ea;
    }
  };
  {
    // the prefetch of a tile past the end re-reads the last tile (in bounds,
    // results unused) so that every iteration issues the same loads
    Raw ra, rb;
    int j = wave;
    if (j < nt) {
      ra.load(lrow, V, j * kTile, lane);
      float lm0 = -INFINITY;
#pragma unroll
      for (int k = 0; k < kLaneElems; ++k) lm0 = fmaxf(lm0, ra.get(k));
      lm0 = wave_max(lm0);
      if (lane == 0) sh.wmax[wave] = lm0;
    } else if (lane == 0) {
      sh.wmax[wave] = -INFINITY;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) ref = fmaxf(ref, sh.wmax[w]);
    if (j < nt) {
      while (true) {
        rb.load(lrow, V, min(j + kWaves, nt - 1) * kTile, lane);
        tile1(ra, j);
        j += kWaves;
        if (j >= nt) break;
        ra.load(lrow, V, min(j + kWaves, nt - 1) * kTile, lane);
        tile1(rb, j);
        j += kWaves;
        if (j >= nt) break;
      }
    }
  }
  __syncthreads();

  // Row max m, c_m = fl(-m s) and Z = sum_j S_j exp2(c_m - c_j) in e-units.
  // The c_j cancel exactly, so Z approximates 2^D sum_k 2^((l_k - m) s) with
  // D = c_m + m s (|D| <= u |m s|); D is carried into p(x) exactly.
  float mloc = -INFINITY;
  for (int j = tid; j < nt; j += NT) mloc = fmaxf(mloc, M[j]);
  const float m = block_max(mloc, sc);
  const float cm = -(m * s);
  double zl = 0.0, eal = 0.0;
  for (int j = tid; j < nt; j += NT) {
    if (M[j] == -INFINITY) continue;
    const float cj = -(M[j] * s);
    const float d = cm - cj;  // <= 0
    const float f = fexp2(d);
    zl += static_cast<double>(S[j] * f);
    // sum_k e_k |a_k| in global units: |a_k| <= -a_k,local + |d| + the
    // rounding of c_j (elements at M_j may give a_k,local up to u |c_j| > 0)
    if (f > 0.f)
      eal += static_cast<double>(f) * (static_cast<double>(EA[j]) +
                                       (-static_cast<double>(d) + 2.0 * kU * fabs(static_cast<double>(cj))) *
                                           static_cast<double>(S[j]));
  }
  if (tid == 0 && xmask >= 0) {  // one-hot rows left x out of S
    const float ax = fmaxf(fmaf(lx, s, cm), -4096.f);
    const float ex = fexp2(ax);
    zl += static_cast<double>(ex);
    eal += static_cast<double>(ex) * (-static_cast<double>(ax) + 2.0 * kU * fabs(static_cast<double>(cm)));
  }
  double Z, sea;
  block_sum2(zl, eal, sc, Z, sea);
  const double bt = bound_terms(Z, sea);
  const double dZ = bt + kSumErr * Z;  // |Z~ - 2^D Z|
  const double relZ = dZ / Z;
  const double shift = static_cast<double>(cm) + static_cast<double>(m) * static_cast<double>(s);  // D, exact

  // ---------------- accept test of a draft row (fp64 p(x), certified)
  if (tid == 0) {
    sh.m = m;
    sh.z = Z;
    int accepted = 0;
    uint32_t why = 0;
    double px = 0.0;
    if (is_draft) {
      if (x_ok) px = exp2((static_cast<double>(lx) - static_cast<double>(m)) * a.s64 + shift) / Z;
      const double qx = onehot ? 1.0 : static_cast<double>(qx_in);
      const double lhs = static_cast<double>(u_acc) * qx;
      accepted = (x_ok && px > 0.0 && lhs <= px) ? 1 : 0;
      if (x_ok) {
        const double dpx = kSafety * (px * relZ * 1.01) + 1e-300;
        if (fabs(lhs - px) <= 2.0 * dpx || px < 1e-30) why |= kWhyAccept;
      }
    }
    if (!(Z > 0.0) || m == -INFINITY || (a.flags & SV_FLAG_EXACT)) why |= kWhyForced;
    sh.px = px;
    sh.accepted = accepted;
    sh.uncertain = static_cast<int>(why);
  }
  __syncthreads();
  const bool accepted = sh.accepted != 0;
  if (sh.uncertain) {
    if (tid == 0) flag_exact(a, t, static_cast<uint32_t>(sh.uncertain), m);
    return;
  }
  const bool sample = !is_draft || !accepted || all_res;
  if (!sample) {
    if (tid == 0) a.ws[t.trow] = make_int2(-1, static_cast<int>(kRowAccepted));
    return;
  }

  // a rejected draft row with q: in the lazy mode its residual is drawn later,
  // and only if it is the request's first rejection
  if (!EAGER && qrow != nullptr && !accepted && !all_res) {
    if (tid == 0) {
      a.rstat[t.trow] = make_double4(static_cast<double>(m), Z, sea, shift);
      a.ws[t.trow] = make_int2(-1, static_cast<int>(kRowDeferred));
    }
    return;
  }
  sample_row<LT, VEC, NT, EAGER>(a, t, lrow, qrow, xmask, accepted, m, Z, bt, relZ, sh.px, S, M, W, sc, sh);
}

// ----------------------------------------------------------------------------
// lazy mode, phase 2: one block per request. The first draft row that is
// certainly rejected decides the emitted token; if its residual was deferred,
// it is drawn here. Rows whose accept test was left to the fp64 path are
// passed over (that path decides them, and draws their token if they are
// rejected), so the row drawn here may turn out unused; the select kernel
// settles the request from the final records.
template <typename LT, bool VEC, int NT>
__global__ __launch_bounds__(NT) void residual_request_kernel(ProbsArgs a) {
  extern __shared__ float dynw[];  // residual tile sums of the row drawn here
  __shared__ BlockScratchT<NT> sc;
  __shared__ RowShared sh;
  const int b = blockIdx.x;
  int d0, d1;
  if (a.cu) {
    d0 = a.cu[b];
    d1 = a.cu[b + 1];
    if (d0 < 0 || d1 < d0 || d1 > a.ndraft) return;
  } else {
    d0 = b * a.gamma;
    d1 = d0 + a.gamma;
  }
  const int g = d1 - d0;
  const int64_t t0 = static_cast<int64_t>(d0) + b;
  int n = g;
  for (int i = 0; i < g; ++i) {
    const uint32_t f = static_cast<uint32_t>(a.ws[t0 + i].y);
    if ((f & kRowNeedExact) && (f & (kWhyAccept | kWhyForced))) continue;
    if (f & kRowAccepted) continue;
    n = i;
    break;
  }
  if (n == g) return;
  if (!(static_cast<uint32_t>(a.ws[t0 + n].y) & kRowDeferred)) return;
  Task t;
  t.b = b;
  t.g = g;
  t.i = n;
  t.trow = t0 + n;
  t.drow = d0 + n;
  t.srow = static_cast<int64_t>(d1) + b;
  t.valid = true;
  const double4 st = a.rstat[t.trow];
  const float m = static_cast<float>(st.x);
  const double Z = st.y;
  const double bt = bound_terms(Z, st.z);
  const double relZ = (bt + kSumErr * Z) / Z;
  const LT* __restrict__ lrow = static_cast<const LT*>(a.logits) + t.trow * static_cast<int64_t>(a.V);
  const float* __restrict__ qrow = a.q + t.drow * static_cast<int64_t>(a.V);
  sample_row<LT, VEC, NT, true>(a, t, lrow, qrow, -1, false, m, Z, bt, relZ, 0.0, nullptr, nullptr, dynw, sc, sh);
}

// ----------------------------------------------------------------------------
// greedy verification (argmax, lowest index on ties)

struct GreedyArgs {
  const void* logits;
  const int64_t* x;
  const int32_t* cu;
  int2* ws;
  int B, gamma, ndraft, V;
};

__device__ __forceinline__ void argmax_combine(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

template <typename LT, bool VEC>
__global__ __launch_bounds__(kNT) void greedy_rows_kernel(GreedyArgs a) {
  __shared__ float bv[kWaves];
  __shared__ int bi[kWaves];
  using L = Lay<LT, VEC>;
  const int V = a.V;
  const int nt = (V + kTile - 1) / kTile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Task t = decode_task(blockIdx.x, a.cu, a.B, a.gamma, a.ndraft);
  if (!t.valid) return;
  const LT* __restrict__ lrow = static_cast<const LT*>(a.logits) + t.trow * static_cast<int64_t>(V);

  float best = -INFINITY;
  int bidx = 0x7fffffff;
  for (int j = wave; j < nt; j += kWaves) {
    const int base = j * kTile;
    float v[kLaneElems];
    load_logits<LT, VEC>(lrow, V, base, lane, v);
#pragma unroll
    for (int k = 0; k < kLaneElems; ++k) {
      if (v[k] > best) {
        best = v[k];
        bidx = L::index(base, lane, k);
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(best, o);
    const int i2 = __shfl_xor(bidx, o);
    argmax_combine(best, bidx, v2, i2);
  }
  if (lane == 0) {
    bv[wave] = best;
    bi[wave] = bidx;
  }
  __syncthreads();
  if (tid == 0) {
    float v = bv[0];
    int i = bi[0];
    for (int w = 1; w < kWaves; ++w) argmax_combine(v, i, bv[w], bi[w]);
    if (i == 0x7fffffff) i = 0;  // every entry -inf: the first index
    int acc = 0;
    if (t.drow >= 0) acc = (a.x[t.drow] == static_cast<int64_t>(i)) ? 1 : 0;
    a.ws[t.trow] = make_int2(i, acc ? static_cast<int>(kRowAccepted) : 0);
  }
}

// ----------------------------------------------------------------------------
// per-request select: first rejection, then accepted drafts + one token

struct SelectArgs {
  const int64_t* x;
  const int32_t* cu;
  const int2* ws;
  int64_t* out;
  int32_t* nacc;
  int* xcount;  // fp64-path list count, reset here for the next call (may be null)
  int B, gamma, ndraft;
};

__global__ __launch_bounds__(kSelectNT) void select_kernel(SelectArgs a) {
  const int b = blockIdx.x * kSelectNT + threadIdx.x;
  if (b == 0 && a.xcount) *a.xcount = 0;
  if (b >= a.B) return;
  int d0, d1;
  if (a.cu) {
    d0 = a.cu[b];
    d1 = a.cu[b + 1];
    if (d0 < 0 || d1 < d0 || d1 > a.ndraft) {
      // invalid offsets: emit nothing for this request
      a.nacc[b] = 0;
      return;
    }
  } else {
    d0 = b * a.gamma;
    d1 = d0 + a.gamma;
  }
  const int g = d1 - d0;
  const int64_t t0 = static_cast<int64_t>(d0) + b;
  int n = 0;
  while (n < g && (static_cast<uint32_t>(a.ws[t0 + n].y) & kRowAccepted)) ++n;
  for (int i = 0; i < n; ++i) a.out[t0 + i] = a.x[d0 + i];
  a.out[t0 + n] = static_cast<int64_t>(a.ws[t0 + n].x);
  for (int i = n + 1; i <= g; ++i) a.out[t0 + i] = -1;
  a.nacc[b] = n;
}

// ----------------------------------------------------------------------------
// self-check of the exp2 accuracy the fast path's error bound assumes

__global__ void zero_double_kernel(double* p) { *p = 0.0; }

// Relative error of the hardware exp2 for every fp32 input in [-126, 0]
// (bit patterns 0x80000000 .. 0xC2FC0000), against fp64 exp2; the maximum is
// combined with an integer atomicMax on the bit pattern (non-negative doubles
// order like their bit patterns).
__global__ __launch_bounds__(kNT) void exp2_error_kernel(double* out) {
  constexpr uint32_t kFirst = 0x80000000u, kLast = 0xC2FC0000u;
  double mx = 0.0;
  const uint32_t stride = gridDim.x * kNT;
  for (uint32_t i = blockIdx.x * kNT + threadIdx.x; i <= kLast - kFirst; i += stride) {
    const float x = __uint_as_float(kFirst + i);
    const double ref = exp2(static_cast<double>(x));
    const double got = static_cast<double>(fexp2(x));
    mx = fmax(mx, fabs(got - ref) / ref);
  }
  __shared__ BlockScratch sc;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
  if ((threadIdx.x & 63) == 0) sc.d[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    double m = sc.d[0];
    for (int w = 1; w < kWaves; ++w) m = fmax(m, sc.d[w]);
    atomicMax(reinterpret_cast<unsigned long long*>(out), static_cast<unsigned long long>(__double_as_longlong(m)));
  }
}

// ----------------------------------------------------------------------------
// host side

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

// Workspace layout: [records rows x int2][count, 256 B][list rows x int2]
// [etile rows x nt doubles][wtile rows x nt doubles][rstat rows x 4 doubles].
struct WsLayout {
  size_t rec, count, list, etile, wtile, rstat, total;
};
WsLayout ws_layout(int64_t rows, int V) {
  WsLayout l;
  const size_t nt = static_cast<size_t>((V + kTile - 1) / kTile);
  l.rec = 0;
  l.count = align256(static_cast<size_t>(rows) * sizeof(int2));
  l.list = l.count + 256;
  l.etile = l.list + align256(static_cast<size_t>(rows) * sizeof(int2));
  l.wtile = l.etile + align256(static_cast<size_t>(rows) * nt * sizeof(double));
  l.rstat = l.wtile + align256(static_cast<size_t>(rows) * nt * sizeof(double));
  l.total = l.rstat + align256(static_cast<size_t>(rows) * 4 * sizeof(double));
  return l;
}
size_t ws_bytes(int64_t rows) { return align256(static_cast<size_t>(rows) * sizeof(int2)); }

// Block sizes: the lazy first pass reads logits only and keeps more rows in
// flight with small blocks; the eager modes and the per-request second pass
// stream logits and q per row and prefer larger blocks (shorter per-row time).
constexpr int kRowsNTLazy = 256;
constexpr int kRowsNTEager = 512;
constexpr int kRequestNT = 512;

template <typename LT, bool VEC, int NT, bool EAGER>
void launch_rows(const ProbsArgs& a, int64_t rows, size_t lds, hipStream_t st) {
  hipLaunchKernelGGL((probs_rows_kernel<LT, VEC, NT, EAGER>), dim3(static_cast<unsigned>(rows)), dim3(NT), lds, st,
                     a);
}

template <typename LT>
int launch_probs(const ProbsArgs& a, const ExactArgs& e, int64_t rows, hipStream_t st) {
  const int nt = (a.V + kTile - 1) / kTile;
  const size_t lds = static_cast<size_t>(nt) * 4 * sizeof(float);
  const bool vec = aligned16(a.logits) && (static_cast<int64_t>(a.V) * sizeof(LT)) % 16 == 0 &&
                   (a.q == nullptr || (aligned16(a.q) && (a.V % 4) == 0));
  const bool lazy = (a.flags & kFlagLazy) != 0;
  if (vec) {
    if (lazy) launch_rows<LT, true, kRowsNTLazy, false>(a, rows, lds, st);
    else launch_rows<LT, true, kRowsNTEager, true>(a, rows, lds, st);
  } else {
    if (lazy) launch_rows<LT, false, kRowsNTLazy, false>(a, rows, lds, st);
    else launch_rows<LT, false, kRowsNTEager, true>(a, rows, lds, st);
  }
  if (lazy) {
    const size_t lds2 = static_cast<size_t>(nt) * sizeof(float);
    if (vec)
      hipLaunchKernelGGL((residual_request_kernel<LT, true, kRequestNT>), dim3(static_cast<unsigned>(a.B)),
                         dim3(kRequestNT), lds2, st, a);
    else
      hipLaunchKernelGGL((residual_request_kernel<LT, false, kRequestNT>), dim3(static_cast<unsigned>(a.B)),
                         dim3(kRequestNT), lds2, st, a);
  }
  hipLaunchKernelGGL((exact_tiles_kernel<LT>), dim3(kExactGrid), dim3(kNT), 0, st, a, e);
  hipLaunchKernelGGL((exact_residual_kernel<LT>), dim3(kExactGrid), dim3(kNT), 0, st, a, e);
  hipLaunchKernelGGL((exact_finish_kernel<LT>), dim3(kNT), dim3(kNT), static_cast<size_t>(e.nt) * 2 * sizeof(double),
                     st, a, e);
  return 0;
}

template <typename LT>
int launch_greedy(const GreedyArgs& a, int64_t rows, hipStream_t st) {
  const bool vec = aligned16(a.logits) && (static_cast<int64_t>(a.V) * sizeof(LT)) % 16 == 0;
  if (vec)
    hipLaunchKernelGGL((greedy_rows_kernel<LT, true>), dim3(static_cast<unsigned>(rows)), dim3(kNT), 0, st, a);
  else
    hipLaunchKernelGGL((greedy_rows_kernel<LT, false>), dim3(static_cast<unsigned>(rows)), dim3(kNT), 0, st, a);
  return 0;
}

int finish_launch() { return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH; }

// Shared implementation of the three entry points.
int verify_common(const void* logits, int dtype, const float* q, const int64_t* x, const int32_t* cu,
                  const float* u, int32_t B, int32_t gamma, int32_t ndraft, int32_t V, double T, uint32_t flags,
                  int64_t* out, int32_t* nacc, float* stats, void* ws, size_t ws_size, void* stream,
                  bool greedy_only) {
  if (dtype != SV_DTYPE_F32 && dtype != SV_DTYPE_BF16) return SV_ERR_UNSUPPORTED;
  if (B < 0 || gamma < 0 || ndraft < 0 || V < 1) return SV_ERR_INVALID_ARGUMENT;
  if (V > SV_MAX_VOCAB) return SV_ERR_UNSUPPORTED;
  if (!(T >= 0.0) || !isfinite(T)) return SV_ERR_INVALID_ARGUMENT;
  if (flags & ~static_cast<uint32_t>(SV_FLAG_EXACT | SV_FLAG_ALL_RESIDUALS | SV_FLAG_EAGER))
    return SV_ERR_INVALID_ARGUMENT;
  if (stats && !(T > 0.0)) return SV_ERR_INVALID_ARGUMENT;
  const int64_t rows = static_cast<int64_t>(ndraft) + B;
  if (rows > 0x7fffffffLL) return SV_ERR_UNSUPPORTED;
  if (B == 0) return SV_OK;
  if (!logits || !out || !nacc) return SV_ERR_INVALID_ARGUMENT;
  if (ndraft > 0 && !x) return SV_ERR_INVALID_ARGUMENT;
  if (!greedy_only && T > 0.0 && !u) return SV_ERR_INVALID_ARGUMENT;
  const bool greedy = greedy_only || T == 0.0;
  const WsLayout wl = ws_layout(rows, V);
  if (!ws || ws_size < (greedy ? ws_bytes(rows) : wl.total) || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return SV_ERR_WORKSPACE;
  (void)hipGetLastError();
  hipStream_t st = static_cast<hipStream_t>(stream);
  int2* wsp = static_cast<int2*>(ws);

  char* wsb = static_cast<char*>(ws);
  int* xcount = greedy ? nullptr : reinterpret_cast<int*>(wsb + wl.count);
  if (greedy) {
    GreedyArgs g{logits, x, cu, wsp, B, gamma, ndraft, V};
    if (dtype == SV_DTYPE_BF16) launch_greedy<uint16_t>(g, rows, st);
    else launch_greedy<float>(g, rows, st);
  } else {
    ProbsArgs p;
    p.logits = logits;
    p.q = q;
    p.x = x;
    p.u = u;
    p.cu = cu;
    p.ws = wsp;
    p.stats = stats;
    p.s64 = 1.4426950408889634 / T;
    p.s32 = static_cast<float>(p.s64);
    p.temperature = T;
    p.B = B;
    p.gamma = gamma;
    p.ndraft = ndraft;
    p.V = V;
    const bool lazy = !(flags & (SV_FLAG_EAGER | SV_FLAG_ALL_RESIDUALS)) && stats == nullptr && q != nullptr;
    p.flags = flags | (lazy ? kFlagLazy : 0u);
    p.rstat = reinterpret_cast<double4*>(wsb + wl.rstat);
    p.xcount = xcount;
    p.xlist = reinterpret_cast<int2*>(wsb + wl.list);
    ExactArgs e;
    e.count = xcount;
    e.list = p.xlist;
    e.etile = reinterpret_cast<double*>(wsb + wl.etile);
    e.wtile = reinterpret_cast<double*>(wsb + wl.wtile);
    e.nt = (V + kTile - 1) / kTile;
    e.rows = static_cast<int>(rows);
    if (dtype == SV_DTYPE_BF16) launch_probs<uint16_t>(p, e, rows, st);
    else launch_probs<float>(p, e, rows, st);
  }
  int rc = finish_launch();
  if (rc != SV_OK) return rc;
  SelectArgs sa{x, cu, wsp, out, nacc, xcount, B, gamma, ndraft};
  hipLaunchKernelGGL(select_kernel, dim3(static_cast<unsigned>((B + kSelectNT - 1) / kSelectNT)), dim3(kSelectNT),
                     0, st, sa);
  return finish_launch();
}

}  // namespace

extern "C" {

size_t spec_verify_workspace_size(int64_t num_target_rows, int32_t vocab_size) {
  if (num_target_rows < 0 || vocab_size < 1 || vocab_size > SV_MAX_VOCAB) return 0;
  return ws_layout(num_target_rows, vocab_size).total;
}

const char* spec_verify_status_string(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SV_ERR_UNSUPPORTED: return "unsupported dtype or size";
    case SV_ERR_LAUNCH: return "kernel launch failed";
    case SV_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    default: return "unknown status";
  }
}

int spec_verify_version(void) { return 1; }

double spec_verify_exp2_error_bound(void) { return kEpsExp; }

int spec_verify_selftest_exp2(double* max_rel_err, void* stream) {
  if (!max_rel_err) return SV_ERR_INVALID_ARGUMENT;
  (void)hipGetLastError();
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(zero_double_kernel, dim3(1), dim3(1), 0, st, max_rel_err);
  hipLaunchKernelGGL(exp2_error_kernel, dim3(2048), dim3(kNT), 0, st, max_rel_err);
  return finish_launch();
}

int spec_verify_probs(const void* target_logits, int logits_dtype, const float* draft_probs,
                      const int64_t* draft_tokens, const float* uniforms, int32_t num_requests,
                      int32_t gamma, int32_t vocab_size, double temperature, uint32_t flags,
                      int64_t* out_tokens, int32_t* num_accepted, float* row_stats, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (num_requests < 0 || gamma < 0) return SV_ERR_INVALID_ARGUMENT;
  const int64_t nd = static_cast<int64_t>(num_requests) * gamma;
  if (nd > 0x7fffffffLL) return SV_ERR_UNSUPPORTED;
  return verify_common(target_logits, logits_dtype, draft_probs, draft_tokens, nullptr, uniforms, num_requests,
                       gamma, static_cast<int32_t>(nd), vocab_size, temperature, flags, out_tokens, num_accepted,
                       row_stats, workspace, workspace_bytes, stream, false);
}

int spec_verify_greedy(const void* target_logits, int logits_dtype, const int64_t* draft_tokens,
                       int32_t num_requests, int32_t gamma, int32_t vocab_size, int64_t* out_tokens,
                       int32_t* num_accepted, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_requests < 0 || gamma < 0) return SV_ERR_INVALID_ARGUMENT;
  const int64_t nd = static_cast<int64_t>(num_requests) * gamma;
  if (nd > 0x7fffffffLL) return SV_ERR_UNSUPPORTED;
  return verify_common(target_logits, logits_dtype, nullptr, draft_tokens, nullptr, nullptr, num_requests, gamma,
                       static_cast<int32_t>(nd), vocab_size, 0.0, 0u, out_tokens, num_accepted, nullptr, workspace,
                       workspace_bytes, stream, true);
}

int spec_verify_ragged(const void* target_logits, int logits_dtype, const float* draft_probs,
                       const int64_t* draft_tokens, const int32_t* cu_num_draft_tokens, const float* uniforms,
                       int32_t num_requests, int32_t num_draft_tokens, int32_t vocab_size, double temperature,
                       uint32_t flags, int64_t* out_tokens, int32_t* num_accepted, float* row_stats,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (num_requests > 0 && !cu_num_draft_tokens) return SV_ERR_INVALID_ARGUMENT;
  return verify_common(target_logits, logits_dtype, draft_probs, draft_tokens, cu_num_draft_tokens, uniforms,
                       num_requests, 0, num_draft_tokens, vocab_size, temperature, flags, out_tokens, num_accepted,
                       row_stats, workspace, workspace_bytes, stream, false);
}

}  // extern "C"
