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

#include <float.h>
#include <math.h>
#include <atomic>
#include <mutex>
#include <type_traits>
#include <stdint.h>

#include "specverify.h"

// The error bound of the fast path follows the rounding steps as written:
// no multiply-add is fused unless the source says fmaf.
#pragma clang fp contract(off)

// Scratch of spec_verify_probs_noalloc (see scratch_for_device).
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

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
  // a tile wholly inside the row: no clamping
  __device__ __forceinline__ void load_full(const uint16_t* __restrict__ row, int base, int lane) {
#pragma unroll
    for (int r = 0; r < 4; ++r) d[r] = *reinterpret_cast<const uint4*>(row + base + (r * 64 + lane) * 8);
  }
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
  __device__ __forceinline__ void load_full(const float* __restrict__ row, int base, int lane) {
#pragma unroll
    for (int r = 0; r < 8; ++r) d[r] = *reinterpret_cast<const float4*>(row + base + (r * 64 + lane) * 4);
  }
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
  __device__ __forceinline__ void load_full(const LT* __restrict__ row, int base, int lane) {
#pragma unroll
    for (int r = 0; r < kLaneElems; ++r) d[r] = to_float(row[base + r * 64 + lane]);
  }
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
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int wave_sum_i(int v) {
  v += dpp_i<0xB1>(v);
  v += dpp_i<0x4E>(v);
  v += dpp_i<0x124>(v);
  v += dpp_i<0x128>(v);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}
__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, dpp_i<0xB1>(v));
  v = min(v, dpp_i<0x4E>(v));
  v = min(v, dpp_i<0x124>(v));
  v = min(v, dpp_i<0x128>(v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ int wave_max_i(int v) {
  v = max(v, dpp_i<0xB1>(v));
  v = max(v, dpp_i<0x4E>(v));
  v = max(v, dpp_i<0x124>(v));
  v = max(v, dpp_i<0x128>(v));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
// 64-bit integer sums and inclusive scans (lane order) by DPP moves of the
// two halves; integer sums are exact in any order.
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v) {
  const uint32_t lo = static_cast<uint32_t>(dpp_i<CTRL>(static_cast<int>(static_cast<uint32_t>(v))));
  const uint32_t hi = static_cast<uint32_t>(dpp_i<CTRL>(static_cast<int>(static_cast<uint32_t>(v >> 32))));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}
__device__ __forceinline__ unsigned long long lane_u64(unsigned long long v, int l) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), l));
  const uint32_t hi =
      static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), l));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
  v += dpp_u64<0xB1>(v);
  v += dpp_u64<0x4E>(v);
  v += dpp_u64<0x124>(v);
  v += dpp_u64<0x128>(v);
  return (lane_u64(v, 0) + lane_u64(v, 16)) + (lane_u64(v, 32) + lane_u64(v, 48));
}
__device__ __forceinline__ unsigned long long wave_scan_incl_u64(unsigned long long v) {
  // within each 16-lane row: shifts right by 1, 2, 4, 8 (lanes before the
  // row's start read 0), then the earlier rows' totals
  v += dpp_u64<0x111>(v);
  v += dpp_u64<0x112>(v);
  v += dpp_u64<0x114>(v);
  v += dpp_u64<0x118>(v);
  const unsigned long long t0 = lane_u64(v, 15), t1 = lane_u64(v, 31), t2 = lane_u64(v, 47);
  const int lane = threadIdx.x & 63;
  return v + (lane < 16 ? 0ull : lane < 32 ? t0 : lane < 48 ? t0 + t1 : t0 + t1 + t2);
}
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

__device__ __forceinline__ double wave_sum_d_dpp(double v);

// Two fixed-order block sums with one pair of barriers (DPP wave sums, then
// the waves' sums in order).
template <int NT>
__device__ void block_sum2(double v, double w, BlockScratchT<NT>& s, double& rv, double& rw) {
  constexpr int kWaves = NT / 64;
  v = wave_sum_d_dpp(v);
  w = wave_sum_d_dpp(w);
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

// Sum over a wave by an xor butterfly: every lane ends with the same value
// (a + b == b + a), in a fixed association.
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// The same sum by DPP row moves on the two 32-bit halves (no lane-index
// registers, no LDS), the four row totals then added in a fixed order: every
// lane ends with the same value.
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double lane_d(double v, int l) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                          __builtin_amdgcn_readlane(__double2loint(v), l));
}
__device__ __forceinline__ double wave_sum_d_dpp(double v) {
  v += dpp_d<0xB1>(v);
  v += dpp_d<0x4E>(v);
  v += dpp_d<0x124>(v);
  v += dpp_d<0x128>(v);
  return ((lane_d(v, 0) + lane_d(v, 16)) + lane_d(v, 32)) + lane_d(v, 48);
}

// Inclusive scan over the 64 lanes in lane order by DPP: a shift-and-add scan
// within each 16-lane row (shifts 1, 2, 4, 8; lanes past the row's start
// read 0), then the earlier rows' totals added in a fixed order. Every lane's
// result is deterministic; no LDS traffic.
template <int N>
__device__ __forceinline__ double dpp_shr_d(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), 0x110 + N, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), 0x110 + N, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double wave_scan_incl_d_dpp(double v) {
  v += dpp_shr_d<1>(v);
  v += dpp_shr_d<2>(v);
  v += dpp_shr_d<4>(v);
  v += dpp_shr_d<8>(v);
  const double t0 = lane_d(v, 15), t1 = lane_d(v, 31), t2 = lane_d(v, 47);
  const int lane = threadIdx.x & 63;
  if (lane < 16) return v;
  const double t01 = t0 + t1;
  return v + (lane < 32 ? t0 : lane < 48 ? t01 : t01 + t2);
}
// Sum over the block by DPP wave sums, then the waves' sums in a fixed order.
template <int NT>
__device__ double block_sum_dpp(double v, BlockScratchT<NT>& s) {
  constexpr int kWaves = NT / 64;
  v = wave_sum_d_dpp(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) s.d[wave] = v;
  __syncthreads();
  double r = 0.0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) r += s.d[w];
  __syncthreads();
  return r;
}

// Inclusive integer scan over the 64 lanes by DPP (as wave_scan_incl_d_dpp).
__device__ __forceinline__ int wave_scan_incl_i_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);
  const int t0 = __builtin_amdgcn_readlane(v, 15), t1 = __builtin_amdgcn_readlane(v, 31),
            t2 = __builtin_amdgcn_readlane(v, 47);
  const int lane = threadIdx.x & 63;
  return v + (lane < 16 ? 0 : lane < 32 ? t0 : lane < 48 ? t0 + t1 : t0 + t1 + t2);
}

// Inclusive scan over the 64 lanes (lane order), fixed association.
__device__ __forceinline__ double wave_scan_incl_d(double v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  return v;
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
                                            int ndraft);

// Lazy mode: the row of position i of request b (invalid when the request's
// offsets are, or when i is past its bonus row).
__device__ __forceinline__ Task lazy_task(int b, int i, const int32_t* __restrict__ cu, int B, int gamma,
                                          int ndraft) {
  Task t;
  t.valid = true;
  t.b = b;
  t.i = i;
  int d0, d1;
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
  if (t.i > t.g) t.valid = false;
  t.drow = t.i < t.g ? static_cast<int64_t>(d0) + t.i : -1;
  t.trow = static_cast<int64_t>(d0) + t.i + t.b;
  t.srow = static_cast<int64_t>(d1) + t.b;
  return t;
}

// Lazy mode. First launch (tasks == nullptr): block blk takes position
// blk / B of request b = blk % B (all first drafts, then all second drafts,
// ...). Second launch: block blk takes task blk of the list the first launch
// wrote ({request, position}, request by request), if there is one.
__device__ __forceinline__ Task decode_task_lazy(int blk, const int32_t* __restrict__ cu, int B, int gamma,
                                                 int ndraft, const int2* __restrict__ tasks, int ntasks) {
  if (tasks) {
    Task t;
    t.valid = false;
    if (blk >= ntasks) return t;
    const int2 tk = tasks[blk];
    // entries come from the first launch; any other value (a workspace that
    // was not zero-filled, a list left by an interrupted call) is no task
    if (static_cast<unsigned>(tk.x) >= static_cast<unsigned>(B) || tk.y < 0) return t;
    return lazy_task(tk.x, tk.y, cu, B, gamma, ndraft);
  }
  return lazy_task(blk % B, blk / B, cu, B, gamma, ndraft);
}

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

// One listed row, self-contained so that the fp64 kernel decodes nothing.
struct ExactEntry {
  double z, dz;  // the fast path's Z and the bound on its error (fp64 units), or {0, inf}
  int trow, drow, srow, b;  // target row, draft row (-1: bonus row), row of the sample uniform, request
  int x;                    // draft token if in [0, V), else -1
  float m;                  // row max
  int pad0, pad1;
};

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
  ExactEntry* xlist;
  int* xdone;     // the list's per-row finished-tile counters (zeroed when a row is listed)
  double4* rstat; // lazy mode: {m, Z, sum e|a|} of deferred rows
  int* mark;      // lazy mode, per request: kMarkBase - (first position known to be a certain rejection), or 0
  double* rsum;   // lazy mode, one-hot drafts with bf16 logits: [rows][nt] fp64 tile sums of the rows not accepted
  int pm;         // lazy mode: most positions of the first launch (all of a dense batch)
  int2* tasks;    // lazy mode: {request, position} of the rows the second launch takes (count at surv_n)
  int* surv_n;    // lazy mode: [0] the task count, [16] the first launch's finished-block counter
  int top_k;      // filtered lazy mode: keep the top_k largest logits (with ties); off unless 0 < top_k < V
  double top_p;   // filtered lazy mode: keep the smallest top set of mass >= top_p; off when >= 1
  int cus;        // the device's compute units
};

struct RowShared {
  int skip;        // lazy mode: an earlier position of the request is a certain rejection
  int stop;        // lazy mode, second launch: that became known while the row was read
  int last;        // lazy mode: this block is the last of the first launch to finish
  int mark_old;    // lazy mode: the values this block's mark atomics returned (stored to wait for them)
  int2 qtask;      // lazy mode, self-listed second launch: this block's {request, position}, or {-1, 0}
  int wcount[16];  // lazy mode: per-wave counts of the survivor list
  float wmax[16];  // per-wave maxima (blocks of up to 1024 threads)
  float wref[16];  // per-wave final references of pass 1 (the row max is their maximum)
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
  double lx, qx, ua, us;  // fp64 finish: l_x, q(x), accept and sample uniforms
  uint32_t why;
  int nund;               // fp64 finish: tiles with undecided elements
  int und[16];
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
// per-request select: first rejection, then the accepted drafts and one token

constexpr uint32_t kRowNeedExactBit = 0x200u;  // a row waiting for the fp64 path

struct SelectArgs {
  const int64_t* x;
  const int32_t* cu;
  const int2* ws;
  int64_t* out;
  int32_t* nacc;
  int B, gamma, ndraft;
};

// With final_only, a request is left alone while a row up to its first
// rejection still waits for the fp64 path (it is selected again afterwards).
__device__ void select_request(const SelectArgs& a, int b, bool final_only) {
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
  // every record is read (independent loads); n = first row whose own test failed
  int n = g;
  bool pending = false;
#pragma unroll 4
  for (int i = 0; i <= g; ++i) {
    const uint32_t f = static_cast<uint32_t>(a.ws[t0 + i].y);
    if (i <= n) {
      pending = pending || (f & kRowNeedExactBit) != 0;
      if (i < n && !(f & kRowAccepted)) n = i;
    }
  }
  if (final_only && pending) return;
  for (int i = 0; i < n; ++i) a.out[t0 + i] = a.x[d0 + i];
  a.out[t0 + n] = static_cast<int64_t>(a.ws[t0 + n].x);
  for (int i = n + 1; i <= g; ++i) a.out[t0 + i] = -1;
  a.nacc[b] = n;
}

__global__ __launch_bounds__(kSelectNT) void select_kernel(SelectArgs a) {
  const int b = blockIdx.x * kSelectNT + threadIdx.x;
  if (b < a.B) select_request(a, b, false);
}

// ----------------------------------------------------------------------------
// fp64 path for the rows the fast kernels could not certify.
//
// The fast kernels append such a row to a list in the workspace, with the fast
// path's Z and its certified error bound when they have them. One fixed-grid
// kernel then spreads the fp64 work over the whole GPU, one (row, tile) item
// per block iteration:
//   - the item: the fp64 sum E_j of e_k = 2^((l_k - m) log2(e) / T) over the
//     tile and, for rows with q, the part of the residual sum that the Z
//     interval already decides: P_j and Q_j, the sums of e_k and of q_k over
//     the elements with e_k / Z > q_k for every Z in the interval, and whether
//     any element is left undecided (e_k / Z - q_k changes sign within it);
//   - the block that completes a row's last tile (a device-scope counter per
//     row, fence before and after) finishes the row: Z = sum_j E_j, the accept
//     test, the residual tile sums W_j = P_j / Z - Q_j (a tile with undecided
//     elements is summed again with the final Z), fallback, tile search and
//     in-tile search, all in fp64; it writes the row's record and statistics;
//   - the block that finishes the last listed row (a second counter) runs the
//     per-request select and resets the counters for the next call.
// With an empty list, block 0 runs the select and the other blocks exit. No
// block ever waits for another.

constexpr uint32_t kRowNeedExact = kRowNeedExactBit;  // set by the fast kernels, cleared by the fp64 finish
constexpr uint32_t kRowDeferred = SV_ROW_DEFERRED;
constexpr uint32_t kRowUnread = SV_ROW_UNREAD;
constexpr uint32_t kRowHead2 = SV_ROW_HEAD2;
constexpr uint32_t kRowRowSelect = SV_ROW_ROW_SELECT;
constexpr uint32_t kRowUndecided = SV_ROW_UNDECIDED;
constexpr uint32_t kRowTileSums = SV_ROW_TILE_SUMS;
constexpr uint32_t kFlagLazy = 0x80000000u;    // internal: set by the host for the lazy mode
constexpr uint32_t kFlagFilter = 0x40000000u;  // internal: lazy mode with top-k / top-p
constexpr int kMarkBase = 1 << 30;              // lazy mode: per-request mark = kMarkBase - position
constexpr int kExactPer = kTile / kNT;      // elements per thread of one tile (8)
constexpr double kZSlack = 1e-12;           // widening of the Z interval for fp64 rounding
constexpr int kItemTiles = 4;               // tiles per item of the fp64 kernel
constexpr int kMaxUndecided = 16;           // undecided tiles the finish lists in LDS
constexpr int kExactItemGrid = 256;         // blocks of the fp64 kernel


struct ExactArgs {
  int* count;         // listed rows (reset by the block that finishes the last one)
  int* finished;      // listed rows finished (reset likewise)
  int* done;          // [rows] tiles finished per listed row (reset by the row's finisher)
  ExactEntry* list;   // [rows]
  double* etile;   // [rows][nt] sum of e_k
  double* ptile;   // [rows][nt] sum of e_k over the elements certainly in the residual's support
  double* qtile;   // [rows][nt] sum of q_k over the same elements
  int* amb;        // [rows][nt] 1 if the Z interval leaves an element of the tile undecided
  int nt;
  int rows;
};

// Thread t of a block covers elements [base + 8t, base + 8t + 8) of a tile,
// so the tile is covered in ascending token order by ascending threads.
// The loads are unconditional (index clamped into the row) so that all of
// them are in flight at once; elements past the end read as -inf (logits) or
// 0 (q).
template <typename LT>
__device__ __forceinline__ void load8(const LT* __restrict__ row, int V, int k0, double (&l)[kExactPer]) {
  LT raw[kExactPer];
#pragma unroll
  for (int e = 0; e < kExactPer; ++e) raw[e] = row[min(k0 + e, V - 1)];
#pragma unroll
  for (int e = 0; e < kExactPer; ++e) l[e] = k0 + e < V ? static_cast<double>(to_float(raw[e])) : -INFINITY;
}
// q of the same elements; zeros when q == nullptr (uniform over the block: a
// row without a q row), which reads nothing.
__device__ __forceinline__ void load8q(const float* __restrict__ q, int V, int k0, double (&v)[kExactPer]) {
  if (q == nullptr) {
#pragma unroll
    for (int e = 0; e < kExactPer; ++e) v[e] = 0.0;
    return;
  }
  float raw[kExactPer];
#pragma unroll
  for (int e = 0; e < kExactPer; ++e) raw[e] = q[min(k0 + e, V - 1)];
#pragma unroll
  for (int e = 0; e < kExactPer; ++e) v[e] = k0 + e < V ? static_cast<double>(raw[e]) : 0.0;
}

struct ExactRow {
  Task t;
  const float* qrow;
  int64_t x;
  bool x_ok, is_draft, onehot;
  double m, z, dz;
};

__device__ __forceinline__ ExactRow exact_row_info(const ProbsArgs& a, const ExactArgs& e, int pos) {
  ExactRow r;
  const ExactEntry en = e.list[pos];
  // an entry out of range (a workspace that was not zero-filled) is skipped
  r.t.valid = en.trow >= 0 && en.trow < e.rows && en.drow >= -1 && en.drow < a.ndraft && en.srow >= 0 &&
              en.srow < e.rows && en.b >= 0 && en.b < a.B && en.x >= -1 && en.x < a.V;
  r.t.trow = r.t.valid ? en.trow : 0;
  r.t.drow = r.t.valid ? en.drow : -1;
  r.t.srow = r.t.valid ? en.srow : 0;
  r.t.b = r.t.valid ? en.b : 0;
  r.t.i = 0;
  r.t.g = 0;
  r.m = static_cast<double>(en.m);
  r.z = en.z;
  r.dz = en.dz;
  r.is_draft = r.t.drow >= 0;
  r.qrow = (r.is_draft && a.q) ? a.q + r.t.drow * static_cast<int64_t>(a.V) : nullptr;
  r.x = r.is_draft ? en.x : -1;
  r.x_ok = r.is_draft && r.x >= 0;
  r.onehot = r.is_draft && r.qrow == nullptr;
  return r;
}

__device__ __forceinline__ int exact_count(const ExactArgs& e) {
  const int n = *e.count;
  return n < 0 ? 0 : (n > e.rows ? e.rows : n);
}

// N fixed-order block sums with one pair of barriers (s.d holds N * waves).
template <int N>
__device__ void block_sum_n(double (&v)[N], BlockScratch& s) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += __shfl_xor(v[i], o);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) s.d[i * kWaves + wave] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    double r = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) r += s.d[i * kWaves + w];
    v[i] = r;
  }
  __syncthreads();
}

// One item: kItemTiles consecutive tiles of a listed row. Per tile, the fp64
// sum of e_k and, for rows with q, the sums over the elements the Z interval
// decides: e_k / Z > q_k for every Z in [zlo, zhi] iff e_k > q_k zhi, and
// e_k / Z <= q_k for every Z iff e_k <= q_k zlo.
template <typename LT>
__device__ void exact_item(const ProbsArgs& a, const ExactArgs& e, const ExactRow& r, int pos, int j0,
                           BlockScratch& sc) {
  const LT* lrow = static_cast<const LT*>(a.logits) + r.t.trow * static_cast<int64_t>(a.V);
  const double zhi = (r.z + r.dz) * (1.0 + kZSlack), zlo = (r.z - r.dz) * (1.0 - kZSlack);
  // tiles past the end of the row (the last item) read clamped, unused data
  double l[kItemTiles][kExactPer], qv[kItemTiles][kExactPer];
  const bool has_q = r.qrow != nullptr;
#pragma unroll
  for (int u = 0; u < kItemTiles; ++u) {
    const int k0 = (j0 + u) * kTile + kExactPer * threadIdx.x;
    load8<LT>(lrow, a.V, k0, l[u]);
    load8q(r.qrow, a.V, k0, qv[u]);
  }
  double v[3 * kItemTiles];
  int undecided = 0;
#pragma unroll
  for (int u = 0; u < kItemTiles; ++u) {
    double es = 0.0, ps = 0.0, qs = 0.0;
#pragma unroll
    for (int k = 0; k < kExactPer; ++k) {
      const double ek = exp2((l[u][k] - r.m) * a.s64);
      es += ek;
      if (has_q) {
        const double q = qv[u][k];  // 0 past the end, where e_k = 0 too: decided, not in the support
        if (ek > q * zhi) {
          ps += ek;
          qs += q;
        } else if (!(ek <= q * zlo)) {
          undecided |= 1 << u;
        }
      }
    }
    v[3 * u] = es;
    v[3 * u + 1] = ps;
    v[3 * u + 2] = qs;
  }
  block_sum_n<3 * kItemTiles>(v, sc);
  // the per-tile undecided bits, OR-ed over the block
  __shared__ int und;
  if (threadIdx.x == 0) und = 0;
  __syncthreads();
  if (undecided) atomicOr(&und, undecided);
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int u = 0; u < kItemTiles; ++u) {
      if (j0 + u >= e.nt) break;
      const int64_t idx = static_cast<int64_t>(pos) * e.nt + j0 + u;
      e.etile[idx] = v[3 * u];
      e.ptile[idx] = v[3 * u + 1];
      e.qtile[idx] = v[3 * u + 2];
      e.amb[idx] = (und >> u) & 1;
    }
  }
}

template <typename LT>
__device__ void exact_finish_row(const ProbsArgs& a, const ExactArgs& e, const ExactRow& r, int pos,
                                 double* xtile, BlockScratch& sc, RowShared& sh) {
  const int tid = threadIdx.x;
  const int nt = e.nt;
  double* ets = xtile;
  double* wts = xtile + nt;
  double* pts = xtile + 2 * nt;
  double* qts = xtile + 3 * nt;
  const int tper = (nt + kNT - 1) / kNT;
  const int tlo = min(nt, tid * tper), thi = min(nt, tlo + tper);
  const Task& t = r.t;
  const LT* lrow = static_cast<const LT*>(a.logits) + t.trow * static_cast<int64_t>(a.V);
  const int64_t row0 = static_cast<int64_t>(pos) * nt;
  // every load that does not depend on Z, issued together
  double zl = 0.0;
  for (int j = tid; j < nt; j += kNT) {
    const double ev = e.etile[row0 + j];
    ets[j] = ev;
    zl += ev;
    if (r.qrow) {
      pts[j] = e.amb[row0 + j] ? -1.0 : e.ptile[row0 + j];  // -1: the tile has undecided elements
      qts[j] = e.qtile[row0 + j];
    }
  }
  if (tid == 0) {
    sh.why = static_cast<uint32_t>(a.ws[t.trow].y) & 0x1f0u;
    sh.lx = r.x_ok ? static_cast<double>(logit_at(lrow, r.x)) : 0.0;
    sh.qx = r.onehot ? 1.0 : (r.x_ok ? static_cast<double>(r.qrow[r.x]) : 0.0);
    sh.ua = r.is_draft ? static_cast<double>(a.u[t.trow]) : 0.0;
    sh.us = static_cast<double>(a.u[t.srow]);
  }
  // Z: thread t adds tiles t, t + 256, ..., then a fixed-order block sum
  // (whose barriers also publish the loads above)
  const double Z = block_sum(zl, sc);
  const double iz = 1.0 / Z;
  const double s = a.s64;
  if (r.qrow) {
    // residual tile sums: decided tiles from P_j and Q_j, then the tiles with
    // undecided elements (listed in LDS, any order) summed again with the final Z
    if (tid == 0) sh.nund = 0;
    __syncthreads();
    for (int j = tid; j < nt; j += kNT) {
      if (pts[j] < 0.0) {
        const int k = atomicAdd(&sh.nund, 1);
        if (k < kMaxUndecided) sh.und[k] = j;
        wts[j] = -1.0;
      } else {
        wts[j] = fmax(0.0, pts[j] * iz - qts[j]);
      }
    }
    __syncthreads();
    const int nund = sh.nund;
    for (int kk = 0; kk < nund; ++kk) {
      int j = -1;
      if (nund <= kMaxUndecided) {
        j = sh.und[kk];
      } else {  // many undecided tiles: the first one not yet summed (its W_j is still -1)
        for (int jj = 0; jj < nt && j < 0; ++jj)
          if (wts[jj] < 0.0) j = jj;
      }
      const int k0 = j * kTile + kExactPer * tid;
      double l[kExactPer], qv[kExactPer];
      load8<LT>(lrow, a.V, k0, l);
      load8q(r.qrow, a.V, k0, qv);
      double acc = 0.0;
#pragma unroll
      for (int k = 0; k < kExactPer; ++k) acc += fmax(0.0, exp2((l[k] - r.m) * s) * iz - qv[k]);
      acc = block_sum(acc, sc);
      if (tid == 0) wts[j] = acc;
      __syncthreads();
    }
  } else {
    for (int j = tid; j < nt; j += kNT) wts[j] = 0.0;
    __syncthreads();
  }
  const uint32_t why = sh.why;

  double ex = 0.0, px = 0.0;
  bool accepted = false;
  if (r.is_draft) {
    if (r.x_ok) {
      ex = exp2((sh.lx - r.m) * s);
      px = ex * iz;
    }
    accepted = r.x_ok && px > 0.0 && sh.ua * sh.qx <= px;
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
    const double tau = sh.us * total;
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
    double l[kExactPer], w[kExactPer], qv[kExactPer];
    load8<LT>(lrow, a.V, k0, l);
    load8q(mode == 1 ? r.qrow : nullptr, a.V, k0, qv);
    double tsum = 0.0;
#pragma unroll
    for (int k = 0; k < kExactPer; ++k) {
      const int kk = k0 + k;
      double v = 0.0;
      if (kk < a.V) {
        const double p = exp2((l[k] - r.m) * s) * iz;
        if (mode == 1) v = fmax(0.0, p - qv[k]);
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

template <typename LT>
__global__ __launch_bounds__(kNT) void exact_kernel(ProbsArgs a, ExactArgs e, SelectArgs sel) {
  extern __shared__ double xtile[];  // [nt] each: e tile sums, residual tile sums, P_j, Q_j
  __shared__ BlockScratch sc;
  __shared__ RowShared sh;
  __shared__ int last;
  const int n = exact_count(e);
  const int nt = e.nt;
  const int per_row = (nt + kItemTiles - 1) / kItemTiles;  // items per row
  const int64_t items = static_cast<int64_t>(n) * per_row;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int pos = static_cast<int>(it / per_row), j0 = static_cast<int>(it % per_row) * kItemTiles;
    const ExactRow r = exact_row_info(a, e, pos);
    __syncthreads();  // every thread is done with `last` of the previous item
    if (r.t.valid) exact_item<LT>(a, e, r, pos, j0, sc);
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // release this item's tile sums
      last = atomicAdd(&e.done[pos], 1) == per_row - 1;
    }
    __syncthreads();
    if (!last) continue;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // acquire every tile sum of the row
    if (r.t.valid) exact_finish_row<LT>(a, e, r, pos, xtile, sc, sh);
    if (threadIdx.x == 0) {
      e.done[pos] = 0;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // release the row's record
      last = atomicAdd(e.finished, 1) == n - 1;
    }
    __syncthreads();
    if (!last) continue;
    // the last listed row is done: select every request that holds a listed row
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // acquire every record
    for (int p = threadIdx.x; p < n; p += kNT) {
      const ExactRow rr = exact_row_info(a, e, p);
      if (rr.t.valid) select_request(sel, rr.t.b, false);
    }
    if (threadIdx.x == 0) {
      *e.finished = 0;
      *e.count = 0;
    }
  }
  // every other request is final already (no row up to its first rejection
  // waits for the fp64 path): select it here, spread over the blocks
  for (int b = blockIdx.x * kNT + threadIdx.x; b < sel.B; b += gridDim.x * kNT) select_request(sel, b, true);
  if (n == 0 && blockIdx.x == 0 && threadIdx.x == 0) *e.count = 0;
}

// Hand a row to the fp64 path: mark its record and append it to the list.
// Z and dZ are the fast path's Z (carrying the factor 2^D of pass 1) and the
// bound on its error; they are handed on in fp64 units (without 2^D), or as
// {0, inf} when the fast path has no usable Z.
__device__ __forceinline__ void flag_exact(const ProbsArgs& a, const Task& t, uint32_t why, float m, bool accepted,
                                           double Z, double dZ) {
  // the accept bit is meaningful unless the accept test itself is the reason
  a.ws[t.trow] = make_int2(-1, static_cast<int>(kRowNeedExact | why | (accepted ? kRowAccepted : 0u)));
  const int pos = atomicAdd(a.xcount, 1);
  if (pos < a.B + a.ndraft) {
    ExactEntry en;
    en.z = 0.0;
    en.dz = INFINITY;
    if (Z > 0.0 && Z < INFINITY && dZ >= 0.0 && dZ < Z && m != -INFINITY) {
      const float s = a.s32;
      const float cm = -(m * s);
      const double unshift =
          exp2(-(static_cast<double>(cm) + static_cast<double>(m) * static_cast<double>(s)));  // 2^-D
      en.z = Z * unshift;
      en.dz = dZ * unshift;
    }
    en.trow = static_cast<int>(t.trow);
    en.drow = static_cast<int>(t.drow);
    en.srow = static_cast<int>(t.srow);
    en.b = t.b;
    const int64_t x = t.drow >= 0 ? a.x[t.drow] : -1;
    en.x = (x >= 0 && x < a.V) ? static_cast<int>(x) : -1;
    en.m = m;
    en.pad0 = en.pad1 = 0;
    a.xlist[pos] = en;
    a.xdone[pos] = 0;  // (the fp64 kernel, a later launch, counts from zero)
  }
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
    if (tid == 0) flag_exact(a, t, w2, m, accepted, Z, relZ * Z);
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
  // unconditional loads (index clamped into the row), all in flight at once
  // (without q, the q loads read u[0], a valid address, and are unused)
  LT lraw[kSearchPer];
  float qraw[kSearchPer];
  const bool use_q = WITH_Q && mode_w;
  const float* qsrc = use_q ? qrow : a.u;
#pragma unroll
  for (int e = 0; e < kSearchPer; ++e) {
    lraw[e] = lrow[min(base + e, V - 1)];
    qraw[e] = qsrc[use_q ? min(base + e, V - 1) : 0];
  }
  float wl[kSearchPer];
#pragma unroll
  for (int e = 0; e < kSearchPer; ++e) {
    const int k = base + e;
    float w = 0.f;
    if (k < V) {
      const float ek = fexp2(fmaf(to_float(lraw[e]), s, cref));
      if (WITH_Q && mode_w) w = fmaxf(ek * izr - qraw[e], 0.f);
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
    if (tid == 0) flag_exact(a, t, why2, m, accepted, Z, relZ * Z);
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
// ----------------------------------------------------------------------------
// top-k / top-p: the threshold on the logit value (lazy mode)
//
// blog.vllbc.top, note on paper §2.2: top-k and top-p, like the temperature,
// fold into an adjusted target p on which the same rejection sampling runs
// (q arrives already adjusted by the drafter). The pages give no further
// detail; the reading taken: both filters act on the temperature-scaled
// target, top-k first, then top-p on the renormalised top-k distribution,
// and both are thresholds on the logit value with ties kept. tau_k is the
// k-th largest logit, counted with multiplicity; tau_p is the largest logit
// value v >= tau_k such that the tokens with l >= v carry at least top_p of
// the top-k mass Z_K. The kept set is {l >= tau}, tau = max(tau_k, tau_p),
// and p is renormalised over it: p(x) = e_x / Z_tau if l_x >= tau, else 0.
//
// Both thresholds come out of a radix select over a monotone 32-bit key of
// the logit, 8-bit digits from the top (two levels for bf16 logits, whose key
// is fixed by its top 16 bits; four for fp32), one sweep over the row per
// level, with per-digit histograms in LDS:
//  * top-k counts the elements per digit (integer atomics: exact, whatever
//    the order in which they land);
//  * top-p sums per digit the masses e = 2^((l - m) s) of the elements with
//    key >= key(tau_k), computed in fp32 exactly as in pass 1 (same error
//    model), as 64-bit fixed-point integers (order-independent sums), with
//    e |a| beside them for the error bound. A digit is taken when the
//    cumulative mass clears the target top_p Z_K by more than the bound;
//    otherwise fp64 sweeps in a fixed order compute the cumulative mass at up
//    to eight undecided digit boundaries and Z_K, and decide.
// Z_tau and its bound are the sums of the masses taken on the way down.

constexpr int kSelDigits = 256;
constexpr int kSelCand = 8;  // digit boundaries per fp64 sweep
constexpr int kHeadCap = 4096;  // elements of the gathered head (see head_threshold)
// Cutoffs of the gathered head: pass 1 gathers {l >= c1}, c1 = ref - kHeadH1 / s
// (ref the block maximum of the first tiles, so e >= 2^-12 relative to it;
// measured with top-k 50 / top-p 0.9 on the peaked bf16 batch, 2^-12 beat
// 2^-6 ... 2^-28: a deeper head costs more appends in pass 1 than the
// second tier it saves);
// a head gathered by its own sweeps takes the lowest of kRungs cutoffs whose
// elements fit the buffer: c1 - kRungBelow[i] / s when pass 1's head was too
// small, c1 + (m - c1) kRungAbove[i] when it overflowed.
constexpr float kHeadH1 = 12.f;
constexpr int kHeadFix = 50;  // fraction bits of the head masses: kHeadCap terms <= 1 stay below 2^63
constexpr int kRungs = 4;
__constant__ float kRungBelow[kRungs] = {48.f, 32.f, 16.f, 8.f};
// with top-k on and pass 1's head too small, a second head at
// c2 = c1 - kCount2 / s is gathered in one sweep (it holds the top-k set
// when it holds k elements; an overflow of its slices falls to the rungs)
constexpr float kCount2 = 8.f;
__constant__ float kRungAbove[kRungs] = {0.25f, 0.5f, 0.75f, 1.f};

struct FilterShared {
  union {
    struct {
      unsigned long long mass[kSelDigits];  // radix select, per digit: fixed-point sum of e
      unsigned long long mea[kSelDigits];   // per digit: fixed-point sum of e |a|
      uint32_t cnt[kSelDigits];             // per digit: elements
    };
    uint32_t head2[kHeadCap];  // head gather: compaction buffer
  };
  uint32_t head[kHeadCap];              // keys of the head elements
  unsigned long long hfix[kHeadCap];    // their masses 2^((l - m) s64) as fixed point (kHeadFix bits)
  int wcnt[16];                         // per-wave counts
  float cut1;                           // pass 1's head cutoff
  float cut2;                           // the second head's cutoff (cut1 - kCount2 / s)
  int ik, ip;                           // head indices: end of tau_k's tie group, top-p crossing
  int amb;                              // top-p: first tie-group end within the bound of the target
  double zk;                            // exact Z_K (head sum) when top-k is on
  double zt;                            // exact mass at the crossing
  int pos;                              // chosen position of the level (digit 255 - pos), -1: undecided
  int amb_lo, amb_hi;                   // undecided positions (pos == -1)
  uint32_t above;                       // top-k: elements above the chosen digit
  unsigned long long m_above, e_above;  // sums over the digits above the chosen one
  unsigned long long m_at, e_at;        // sums of the chosen digit
};
struct NoFilterShared {};

// Monotone key of a logit: a < b iff key(a) < key(b); -0 and +0 share a key.
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// floor(v 2^F) for a finite v >= 0 (denormals count as 0): v = mt 2^(ex - 150).
__device__ __forceinline__ unsigned long long to_fixed(float v, int F) {
  const uint32_t b = __float_as_uint(v);
  const int ex = static_cast<int>(b >> 23);
  const unsigned long long mt = static_cast<unsigned long long>((b & 0x7fffffu) | 0x800000u);
  const int sh = ex - 150 + F;
  const unsigned long long up = mt << min(max(sh, 0), 63);
  const unsigned long long dn = mt >> min(max(-sh, 0), 63);
  return ex == 0 ? 0ull : (sh >= 0 ? up : dn);
}

// Bound on |fixed-point mass - exact mass| of a set of elements whose
// fixed-point sums are M (of e) and EA (of e |a|), in e-units: the relative
// error C1 |a| + C0 of each fp32 term (pass 1's model), the flooring of each
// term to 2^-F (quant = V 2^-F covers any set), and the rounding of the
// conversions to fp64.
__device__ __forceinline__ double fixed_bound(double M, double EA, double quant) {
  return kSafety * 1.01 * (kC1 * (EA + quant) + kC0 * (M + quant)) + quant + 1e-14 * M;
}

// Calls f(v) for every element of the row: wave w visits tiles w, w + waves,
// ... Used by the rare paths of the threshold (radix select, fp64 sweeps):
// one tile in flight and a partly unrolled visit keep their registers below
// those of pass 1, so that they do not set the kernel's occupancy.
template <typename LT, bool VEC, int NT, typename Fn>
__device__ __forceinline__ void sweep_row(const LT* __restrict__ lrow, int V, Fn&& f) {
  constexpr int kW = NT / 64;
  using L = Lay<LT, VEC>;
  using Raw = RawTile<LT, VEC>;
  const int lane = threadIdx.x & 63;
  const int nt = (V + kTile - 1) / kTile;
  for (int j = threadIdx.x >> 6; j < nt; j += kW) {
    Raw r;
    r.load(lrow, V, j * kTile, lane);
    const int base = j * kTile;
    const bool full = base + kTile <= V;
#pragma unroll 4
    for (int k = 0; k < kLaneElems; ++k)
      if (full || L::index(base, lane, k) < V) f(r.get(k));
  }
}

// Positions t = 0..255 stand for the digits 255 - t, in descending key order;
// lane l of wave 0 holds positions 4l .. 4l + 3.

// Wave 0: the position at which the count from the top first reaches kk
// (1 <= kk <= the level's total), and the count above it.
__device__ void pick_count(FilterShared& fs, uint32_t kk) {
  const int lane = threadIdx.x & 63;
  uint32_t c[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) c[r] = fs.cnt[255 - 4 * lane - r];
  const uint32_t ls = (c[0] + c[1]) + (c[2] + c[3]);
  const uint32_t incl = static_cast<uint32_t>(wave_scan_incl_i_dpp(static_cast<int>(ls)));
  const uint32_t excl = incl - ls;
  if (excl < kk && incl >= kk) {  // exactly one lane
    uint32_t cum = excl;
    int t = 4 * lane + 3;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (cum + c[r] >= kk) {
        t = 4 * lane + r;
        break;
      }
      cum += c[r];
    }
    fs.pos = t;
    fs.above = cum;
  }
}

// Wave 0: fixed-point sums over the positions before t, and of position t
// (t = 256: the level's totals in m_above, e_above).
__device__ void level_take(FilterShared& fs, int t) {
  const int lane = threadIdx.x & 63;
  unsigned long long ma = 0, ea = 0, mt = 0, et = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int p = 4 * lane + r;
    const unsigned long long mv = fs.mass[255 - p], ev = fs.mea[255 - p];
    if (p < t) {
      ma += mv;
      ea += ev;
    } else if (p == t) {
      mt = mv;
      et = ev;
    }
  }
  ma = wave_sum_u64(ma);
  ea = wave_sum_u64(ea);
  mt = wave_sum_u64(mt);
  et = wave_sum_u64(et);
  if (lane == 0) {
    fs.m_above = ma;
    fs.e_above = ea;
    fs.m_at = mt;
    fs.e_at = et;
  }
}

// Wave 0: top-p at one level. With C (mass above the level's prefix, bound
// Cerr) and the target tgt (bound tgterr), position t is certainly below the
// target when C + cum(t) + err(t) < tgt and certainly at or above it when
// C + cum(t) - err(t) >= tgt (cum(t) = mass of positions 0..t). The crossing
// is the first position at or above; when some positions are neither, their
// range is left to the fp64 sweeps (pos = -1).
__device__ void pick_mass(FilterShared& fs, double C, double Cerr, double tgt, double tgterr, double inv,
                          double quant) {
  const int lane = threadIdx.x & 63;
  unsigned long long mv[4], ev[4], ls = 0, le = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    mv[r] = fs.mass[255 - 4 * lane - r];
    ev[r] = fs.mea[255 - 4 * lane - r];
    ls += mv[r];
    le += ev[r];
  }
  unsigned long long im = ls, ie = le;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long ym = __shfl_up(im, o), ye = __shfl_up(ie, o);
    if (lane >= o) {
      im += ym;
      ie += ye;
    }
  }
  unsigned long long cm = im - ls, ce = ie - le;
  int hat = 256, alo = 256, ahi = -1;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    cm += mv[r];
    ce += ev[r];
    const double mc = static_cast<double>(cm) * inv;
    const double v = C + mc;
    const double err = Cerr + fixed_bound(mc, static_cast<double>(ce) * inv, quant) + tgterr;
    const int t = 4 * lane + r;
    if (v >= tgt) hat = min(hat, t);
    if (!(v + err < tgt) && !(v - err >= tgt)) {
      alo = min(alo, t);
      ahi = max(ahi, t);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    hat = min(hat, __shfl_xor(hat, o));
    alo = min(alo, __shfl_xor(alo, o));
    ahi = max(ahi, __shfl_xor(ahi, o));
  }
  if (lane == 0) {
    if (ahi < 0 && hat < 256) {
      fs.pos = hat;
    } else {  // undecided positions (or, defensively, no crossing found: all of them)
      fs.pos = -1;
      fs.amb_lo = ahi < 0 ? 0 : alo;
      fs.amb_hi = ahi < 0 ? 255 : ahi;
    }
  }
}

// N fixed-order block sums with one pair of barriers (s.d holds N * waves).
template <int NT, int N>
__device__ void block_sum_nt(double (&v)[N], BlockScratchT<NT>& s) {
  constexpr int kW = NT / 64;
  static_assert(N * kW <= NT, "scratch too small");
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += __shfl_xor(v[i], o);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) s.d[i * kW + wave] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    double r = 0.0;
#pragma unroll
    for (int w = 0; w < kW; ++w) r += s.d[i * kW + w];
    v[i] = r;
  }
  __syncthreads();
}

// fp64 sweep in a fixed order (per thread in element order, then a fixed
// block reduction): acc[c] = mass of the elements with key >= max(B[c], klo)
// for c < kSelCand, acc[kSelCand] = Z_K (key >= klo); masses 2^((l - m) s64).
template <typename LT, bool VEC, int NT>
__device__ void exact_masses(const LT* __restrict__ lrow, int V, float m, double s64, uint32_t klo,
                             const uint32_t (&B)[kSelCand], double (&acc)[kSelCand + 1], BlockScratchT<NT>& sc) {
#pragma unroll
  for (int c = 0; c <= kSelCand; ++c) acc[c] = 0.0;
  const double md = static_cast<double>(m);
  sweep_row<LT, VEC, NT>(lrow, V, [&](float v) {
    const uint32_t key = order_key(v);
    if (key >= klo) {
      const double e = exp2((static_cast<double>(v) - md) * s64);
#pragma unroll
      for (int c = 0; c < kSelCand; ++c) acc[c] += key >= B[c] ? e : 0.0;
      acc[kSelCand] += e;
    }
  });
  block_sum_nt<NT, kSelCand + 1>(acc, sc);
}

// The key of tau for a prefix of `levels` digits (bf16: the key whose top 16
// bits are the prefix and whose low bits are those of a bf16 value).
__device__ __forceinline__ uint32_t prefix_key(uint32_t prefix, int levels) {
  if (levels == 4) return prefix;
  return (prefix << 16) | ((prefix & 0x8000u) ? 0u : 0xffffu);
}

// Append inside pass 1: each wave fills its own slice of the head buffer
// (`slice` entries from `dst`), counting in `cnt` (wave-uniform), one element
// slot at a time with a ballot: no atomics. cnt counts every element offered;
// cnt > slice after the sweep means the slice overflowed.
template <typename LT, bool VEC>
__device__ __forceinline__ void head_append_wave(const RawTile<LT, VEC>& r, int base, int V, int lane, float c,
                                                 uint32_t* dst, int slice, int& cnt) {
  using L = Lay<LT, VEC>;
  const bool full = base + kTile <= V;
#pragma unroll
  for (int g = 0; g < kLaneElems; g += 8) {  // groups of 8 slots, skipped when no lane has a candidate
    float gm = r.get(g);
#pragma unroll
    for (int k = g + 1; k < g + 8; ++k) gm = fmaxf(gm, r.get(k));
    if (!__any(gm >= c)) continue;
#pragma unroll
    for (int k = g; k < g + 8; ++k) {
      const float v = r.get(k);
      const bool in = (full || L::index(base, lane, k) < V) && v >= c;
      const uint64_t mk = __ballot(in);
      if (mk) {
        const int at = cnt + static_cast<int>(__popcll(mk & ((1ull << lane) - 1)));
        if (in && at < slice) dst[at] = order_key(v);
        cnt += static_cast<int>(__popcll(mk));
      }
    }
  }
}

// head_append_wave for pass 1: groups of 8 slots (their per-lane maxima gm)
// without an element at or above c are skipped.
template <typename LT, bool VEC>
__device__ __forceinline__ void head_append_groups_wave(const RawTile<LT, VEC>& r, const float (&gm)[kLaneElems / 8],
                                                        int base, int V, int lane, float c, uint32_t* dst, int slice,
                                                        int& cnt) {
  using L = Lay<LT, VEC>;
  const bool full = base + kTile <= V;  // uniform
#pragma unroll
  for (int g = 0; g < kLaneElems; g += 8) {
    if (!__any(gm[g / 8] >= c)) continue;
#pragma unroll
    for (int k = g; k < g + 8; ++k) {
      const float v = r.get(k);
      const bool in = (full || L::index(base, lane, k) < V) && v >= c;
      const uint64_t mk = __ballot(in);
      if (mk) {
        const int at = cnt + static_cast<int>(__popcll(mk & ((1ull << lane) - 1)));
        if (in && at < slice) dst[at] = order_key(v);
        cnt += static_cast<int>(__popcll(mk));
      }
    }
  }
}

// The per-wave slices of the head buffer (counts in fs.wcnt) made
// contiguous through head2; returns the head size, or kHeadCap + 1 when some
// slice overflowed (its count above the slice). Called by every thread.
template <int NT>
__device__ int compact_slices(FilterShared& fs) {
  constexpr int kW = NT / 64;
  constexpr int kSlice = kHeadCap / kW;
  int n = 0, off = 0;
  bool over = false;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    const int c = fs.wcnt[w];
    over = over || c > kSlice;
    if (w < wave) off += c;
    n += c;
  }
  if (over) {
    __syncthreads();
    return kHeadCap + 1;
  }
  const int mine = fs.wcnt[wave];
  for (int i = threadIdx.x & 63; i < mine; i += 64) fs.head2[off + i] = fs.head[wave * kSlice + i];
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += NT) fs.head[i] = fs.head2[i];
  __syncthreads();
  return n;
}

template <typename LT, bool VEC, int NT>
__device__ int gather_at(const LT* __restrict__ lrow, int V, float cut, FilterShared& fs);

// A head gathered by its own two sweeps, after pass 1 (m known): the first
// counts, per wave, the elements at or above each of kRungs increasing
// cutoffs (registers only); the lowest cutoff whose per-wave counts all fit a
// wave's slice of the buffer is taken, and the second sweep appends the
// elements at or above it to the per-wave slices, which are then made
// contiguous. Returns the head size, or -1 if no cutoff fits.
template <typename LT, bool VEC, int NT>
__device__ int gather_head(const LT* __restrict__ lrow, int V, const float (&cuts)[kRungs], FilterShared& fs) {
  constexpr int kW = NT / 64;
  constexpr int kSlice = kHeadCap / kW;
  using L = Lay<LT, VEC>;
  using Raw = RawTile<LT, VEC>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nt = (V + kTile - 1) / kTile;
  // ---- counts per cutoff
  int cnt[kRungs];
#pragma unroll
  for (int i = 0; i < kRungs; ++i) cnt[i] = 0;
  {
    Raw ra, rb;
    int j = wave;
    auto tally = [&](const Raw& r, int jj) {
      const int base = jj * kTile;
      const bool full = base + kTile <= V;
#pragma unroll
      for (int k = 0; k < kLaneElems; ++k) {
        const float v = r.get(k);
        const bool in = full || L::index(base, lane, k) < V;
#pragma unroll
        for (int i = 0; i < kRungs; ++i) cnt[i] += (in && v >= cuts[i]) ? 1 : 0;
      }
    };
    if (j < nt) {
      ra.load(lrow, V, j * kTile, lane);
      while (true) {
        rb.load(lrow, V, min(j + kW, nt - 1) * kTile, lane);
        tally(ra, j);
        j += kW;
        if (j >= nt) break;
        ra.load(lrow, V, min(j + kW, nt - 1) * kTile, lane);
        tally(rb, j);
        j += kW;
        if (j >= nt) break;
      }
    }
  }
  // the lowest cutoff whose count fits in every wave's slice
  int ok_from = kRungs;  // first rung that fits this wave
#pragma unroll
  for (int i = kRungs - 1; i >= 0; --i) {
    const int c = wave_sum_i(cnt[i]);
    if (c <= kSlice && ok_from == i + 1) ok_from = i;
  }
  if (lane == 0) fs.wcnt[wave] = ok_from;
  __syncthreads();
  int li = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) li = max(li, fs.wcnt[w]);
  __syncthreads();
  if (li >= kRungs) return -1;
  return gather_at<LT, VEC, NT>(lrow, V, cuts[li], fs);
}

// The gathering sweep: every element at or above `cut` into the per-wave
// slices, then made contiguous; returns the head size (kHeadCap + 1 if a
// slice overflowed).
template <typename LT, bool VEC, int NT>
__device__ int gather_at(const LT* __restrict__ lrow, int V, float cut, FilterShared& fs) {
  constexpr int kW = NT / 64;
  constexpr int kSlice = kHeadCap / kW;
  using Raw = RawTile<LT, VEC>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nt = (V + kTile - 1) / kTile;
  int hc = 0;
  {
    Raw ra, rb;
    int j = wave;
    uint32_t* dst = fs.head + wave * kSlice;
    if (j < nt) {
      ra.load(lrow, V, j * kTile, lane);
      while (true) {
        rb.load(lrow, V, min(j + kW, nt - 1) * kTile, lane);
        head_append_wave<LT, VEC>(ra, j * kTile, V, lane, cut, dst, kSlice, hc);
        j += kW;
        if (j >= nt) break;
        ra.load(lrow, V, min(j + kW, nt - 1) * kTile, lane);
        head_append_wave<LT, VEC>(rb, j * kTile, V, lane, cut, dst, kSlice, hc);
        j += kW;
        if (j >= nt) break;
      }
    }
  }
  if (lane == 0) fs.wcnt[wave] = hc;
  __syncthreads();
  return compact_slices<NT>(fs);
}

// floor(x 2^F) for 0 <= x < 2^(63 - F), x in fp64.
__device__ __forceinline__ unsigned long long to_fixed64(double x, int F) {
  const double y = ldexp(x, F);
  const uint32_t hi = static_cast<uint32_t>(y * 0x1p-32);
  const uint32_t lo = static_cast<uint32_t>(fma(static_cast<double>(hi), -4294967296.0, y));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// Histograms over the head's keys (LDS) at one level of the select: counts,
// and with `masses` the fixed-point masses, of the elements with key >= klo
// whose key starts with `prefix` (lv digits).
template <int NT>
__device__ void head_hist(FilterShared& fs, int n, int lv, uint32_t prefix, uint32_t klo, bool masses) {
  const int tid = threadIdx.x;
  const int shift_d = 24 - 8 * lv, hs = shift_d + 8;
  for (int d = tid; d < kSelDigits; d += NT) {
    fs.cnt[d] = 0u;
    fs.mass[d] = 0ull;
  }
  __syncthreads();
  for (int i = tid; i < n; i += NT) {
    const uint32_t key = fs.head[i];
    if (key >= klo && (hs >= 32 || (key >> hs) == prefix)) {
      const uint32_t d = (key >> shift_d) & 255u;
      atomicAdd(&fs.cnt[d], 1u);
      if (masses) atomicAdd(&fs.mass[d], fs.hfix[i]);
    }
  }
  __syncthreads();
}

// Wave 0: top-p at one level over exact (fixed-point) masses. Position t is
// at or above the target when C + cum(t) >= thi and below it when
// C + cum(t) < tlo (thi == tlo when Z_K is exact); the crossing is the first
// position at or above, unless a position in between is undecided
// (pos = -1). Values in units of 2^-kHeadFix.
__device__ void pick_head_mass(FilterShared& fs, double C, double tlo, double thi) {
  const int lane = threadIdx.x & 63;
  unsigned long long mv[4], ls = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    mv[r] = fs.mass[255 - 4 * lane - r];
    ls += mv[r];
  }
  const unsigned long long im = wave_scan_incl_u64(ls);
  unsigned long long cm = im - ls;
  int hat = 256, und = 256;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    cm += mv[r];
    const double v = C + static_cast<double>(cm);
    const int t = 4 * lane + r;
    if (v >= thi) hat = min(hat, t);
    else if (v >= tlo) und = min(und, t);
  }
  hat = wave_min_i(hat);
  und = wave_min_i(und);
  if (lane == 0) fs.pos = (und < hat || hat >= 256) ? -1 : hat;
}

// Decides the thresholds from a gathered head of n elements, {l >= c} for
// some cutoff c. Every element >= c is in the head, so the mass at or above
// any head value is a sum over the head: each element's mass 2^((l - m) s64)
// is computed once in fp64 and kept as a 64-bit fixed-point integer, so that
// sums in any order are equal (to n 2^-kHeadFix, below 4e-12 of the row max's
// mass). tau_k and tau_p come out of a radix select over the head's keys (as
// the row select, but in LDS). top-k needs k <= n; top-p needs its crossing
// in the head (with top-k off, Z_K is the whole row's Z: pass 1's certified
// value, or an fp64 sweep when the bound cannot decide). Returns false when
// the head cannot decide. Called by every thread; the result is uniform.
template <typename LT, bool VEC, int NT>
__device__ bool decide_head(const ProbsArgs& a, const LT* __restrict__ lrow, float m, double shift, double Zp,
                            double dZp, int n, FilterShared& fs, BlockScratchT<NT>& sc, float& tau, double& Zt,
                            double& dZt) {
  constexpr int kLevels = sizeof(LT) == 2 ? 2 : 4;
  const int V = a.V, tid = threadIdx.x;
  const bool use_k = a.top_k > 0 && a.top_k < V;
  const bool use_p = a.top_p < 1.0;
  if (n < 1 || n > kHeadCap || (use_k && a.top_k > n)) return false;
  const double md = static_cast<double>(m);
  for (int i = tid; i < n; i += NT)
    fs.hfix[i] = to_fixed64(exp2((static_cast<double>(key_value(fs.head[i])) - md) * a.s64), kHeadFix);
  __syncthreads();
  // ---- top-k: counts
  uint32_t klo = 0;
  if (use_k) {
    uint32_t prefix = 0, kk = static_cast<uint32_t>(a.top_k);
    for (int lv = 0; lv < kLevels; ++lv) {
      if (tid == 0) {
        fs.pos = kSelDigits - 1;
        fs.above = 0u;
      }
      head_hist<NT>(fs, n, lv, prefix, 0u, false);
      if (tid < 64) pick_count(fs, kk);
      __syncthreads();
      kk -= fs.above;
      prefix = (prefix << 8) | static_cast<uint32_t>(255 - fs.pos);
      __syncthreads();
    }
    klo = prefix_key(prefix, kLevels);
  }
  // ---- Z_K over the head (exact when top-k is on or the head is the whole row)
  unsigned long long zpart = 0;
  for (int i = tid; i < n; i += NT)
    if (fs.head[i] >= klo) zpart += fs.hfix[i];
  zpart = wave_sum_u64(zpart);
  if ((tid & 63) == 0) fs.m_at = 0;
  __syncthreads();
  if ((tid & 63) == 0) atomicAdd(&fs.m_at, zpart);
  __syncthreads();
  const double zhead = static_cast<double>(fs.m_at);  // units of 2^-kHeadFix
  __syncthreads();
  const double scale = ldexp(1.0, kHeadFix);
  const double unshift = exp2(-shift);  // 2^-D: pass 1's units to fp64 units
  bool zexact = use_k || n == V;
  double zk = zexact ? zhead : Zp * unshift * scale;
  double dzk = zexact ? 0.0 : dZp * unshift * scale * 1.01;
  double z_tau = zhead;  // Z_tau (top-k alone: Z_K)
  uint32_t kt = klo;
  if (use_p) {
    for (int attempt = 0; attempt < 2; ++attempt) {
      const double qerr = static_cast<double>(n) + 1.0;  // flooring of the terms, in units of 2^-kHeadFix
      const double thi = a.top_p * (zk + dzk) + qerr, tlo = a.top_p * (zk - dzk) - qerr;
      const double texact = a.top_p * zk;
      uint32_t prefix = 0;
      double C = 0.0;
      bool undecided = false;
      for (int lv = 0; lv < kLevels; ++lv) {
        head_hist<NT>(fs, n, lv, prefix, klo, true);
        if (tid < 64) pick_head_mass(fs, C, zexact ? texact : tlo, zexact ? texact : thi);
        __syncthreads();
        const int t = fs.pos;
        if (t < 0) {
          undecided = true;
          break;
        }
        if (tid < 64) level_take(fs, t);
        __syncthreads();
        C += static_cast<double>(fs.m_above);
        prefix = (prefix << 8) | static_cast<uint32_t>(255 - t);
        if (lv == kLevels - 1) z_tau = C + static_cast<double>(fs.m_at);
        __syncthreads();
      }
      if (!undecided) {
        kt = prefix_key(prefix, kLevels);
        break;
      }
      // undecided: either the crossing lies below the head, or Z_K is not
      // known well enough
      if (zexact || attempt == 1) return false;
      if (!(zhead >= tlo)) return false;  // (cannot reach even the lowest target)
      uint32_t B[kSelCand];
#pragma unroll
      for (int cc = 0; cc < kSelCand; ++cc) B[cc] = 0xffffffffu;
      double acc[kSelCand + 1];
      exact_masses<LT, VEC, NT>(lrow, V, m, a.s64, 0u, B, acc, sc);
      zk = acc[kSelCand] * scale;
      dzk = 0.0;
      zexact = true;
    }
  }
  tau = key_value(kt);
  Zt = z_tau / scale / unshift;  // back to pass 1's units
  dZt = Zt * 4e-12 + static_cast<double>(n + 1) / scale / unshift;
  return true;
}

// Fast path of the threshold, in two tiers: the head pass 1 gathered (cutoff
// ref - kHeadH1 / s, ref the block maximum of the first tiles), then, if that
// head overflowed or cannot decide, a head gathered by its own sweeps.
// Returns the tier that decided (1, 2), or 0 (the radix select then runs).
template <typename LT, bool VEC, int NT>
__device__ int head_threshold(const ProbsArgs& a, const LT* __restrict__ lrow, float m, double shift, double Zp,
                               double dZp, FilterShared& fs, BlockScratchT<NT>& sc, float& tau, double& Zt,
                               double& dZt) {
  const int n1 = compact_slices<NT>(fs);  // pass 1's slices (> kHeadCap: one overflowed)
  if (n1 <= kHeadCap && decide_head<LT, VEC, NT>(a, lrow, m, shift, Zp, dZp, n1, fs, sc, tau, Zt, dZt)) return 1;
  // top-k on and pass 1's head too small: the head at the second cutoff (when
  // it fits every wave's slice and holds k elements, the top-k set, and so
  // the top-p crossing within it, lie at or above that cutoff)
  if (n1 <= kHeadCap && a.top_k > 0 && a.top_k < a.V) {
    const int n2 = gather_at<LT, VEC, NT>(lrow, a.V, fs.cut2, fs);
    if (n2 <= kHeadCap && decide_head<LT, VEC, NT>(a, lrow, m, shift, Zp, dZp, n2, fs, sc, tau, Zt, dZt)) return 2;
  }
  // a head of its own: below pass 1's cutoff when that head was too small
  // (the crossing or the k-th element lay below it), above it when it overflowed
  const float cut1 = fs.cut1;
  float cuts[kRungs];
#pragma unroll
  for (int i = 0; i < kRungs; ++i)
    cuts[i] = n1 <= kHeadCap ? cut1 - kRungBelow[i] / a.s32 : cut1 + (m - cut1) * kRungAbove[i];
  const int n2 = gather_head<LT, VEC, NT>(lrow, a.V, cuts, fs);
  return (n2 >= 0 && decide_head<LT, VEC, NT>(a, lrow, m, shift, Zp, dZp, n2, fs, sc, tau, Zt, dZt)) ? 2 : 0;
}

// Threshold tau of one row and Z_tau with the bound on its error (e-units of
// pass 1, carrying 2^D). m is the row max; called by every thread of the block.
template <typename LT, bool VEC, int NT>
__device__ void row_threshold(const ProbsArgs& a, const LT* __restrict__ lrow, float m, double shift,
                              FilterShared& fs, BlockScratchT<NT>& sc, float& tau, double& Zt, double& dZt) {
  constexpr int kLevels = sizeof(LT) == 2 ? 2 : 4;
  const int V = a.V, tid = threadIdx.x;
  const float s = a.s32, cm = -(m * s);
  const int F = 62 - (V > 1 ? 32 - __clz(V - 1) : 0);  // V terms <= 1 (+ rounding) stay below 2^63
  const double inv = ldexp(1.0, -F);
  const double quant = static_cast<double>(V) * inv;
  const bool use_k = a.top_k > 0 && a.top_k < V;
  const bool use_p = a.top_p < 1.0;
  auto add_mass = [&](float v, uint32_t d) {
    const float arg = fmaxf(fmaf(v, s, cm), -4096.f);
    const float e = fexp2(arg);
    atomicAdd(&fs.mass[d], to_fixed(e, F));
    atomicAdd(&fs.mea[d], to_fixed(e * fabsf(arg), F));
  };
  uint32_t klo = 0;
  double Z = 0.0, dZ = 0.0;
  if (use_k) {
    const bool wm = !use_p;  // top-k alone: Z_tau comes out of these sweeps
    uint32_t prefix = 0, kk = static_cast<uint32_t>(a.top_k);
    for (int lv = 0; lv < kLevels; ++lv) {
      const int shift_d = 24 - 8 * lv, hs = shift_d + 8;
      for (int d = tid; d < kSelDigits; d += NT) {
        fs.cnt[d] = 0u;
        fs.mass[d] = 0ull;
        fs.mea[d] = 0ull;
      }
      if (tid == 0) {
        fs.pos = kSelDigits - 1;
        fs.above = 0u;
      }
      __syncthreads();
      sweep_row<LT, VEC, NT>(lrow, V, [&](float v) {
        const uint32_t key = order_key(v);
        if (hs >= 32 || (key >> hs) == prefix) {
          const uint32_t d = (key >> shift_d) & 255u;
          atomicAdd(&fs.cnt[d], 1u);
          if (wm) add_mass(v, d);
        }
      });
      __syncthreads();
      if (tid < 64) pick_count(fs, kk);
      __syncthreads();
      const int t = fs.pos;
      kk -= fs.above;
      prefix = (prefix << 8) | static_cast<uint32_t>(255 - t);
      if (wm) {
        if (tid < 64) level_take(fs, t);
        __syncthreads();
        const double ma = static_cast<double>(fs.m_above) * inv, ea = static_cast<double>(fs.e_above) * inv;
        Z += ma;
        dZ += fixed_bound(ma, ea, quant);
        if (lv == kLevels - 1) {
          const double mt = static_cast<double>(fs.m_at) * inv, et = static_cast<double>(fs.e_at) * inv;
          Z += mt;
          dZ += fixed_bound(mt, et, quant);
        }
      }
      __syncthreads();  // fs is cleared by the next level
    }
    klo = prefix_key(prefix, kLevels);
  }
  uint32_t kt = klo;
  if (use_p) {
    uint32_t prefix = 0;
    double C = 0.0, Cerr = 0.0, tgt = 0.0, tgterr = 0.0;
    for (int lv = 0; lv < kLevels; ++lv) {
      const int shift_d = 24 - 8 * lv, hs = shift_d + 8;
      for (int d = tid; d < kSelDigits; d += NT) {
        fs.mass[d] = 0ull;
        fs.mea[d] = 0ull;
      }
      __syncthreads();
      sweep_row<LT, VEC, NT>(lrow, V, [&](float v) {
        const uint32_t key = order_key(v);
        if (key >= klo && (hs >= 32 || (key >> hs) == prefix)) add_mass(v, (key >> shift_d) & 255u);
      });
      __syncthreads();
      if (lv == 0) {  // Z_K: the mass of every element with key >= key(tau_k)
        if (tid < 64) level_take(fs, kSelDigits);
        __syncthreads();
        const double zk = static_cast<double>(fs.m_above) * inv;
        tgt = a.top_p * zk;
        tgterr = a.top_p * fixed_bound(zk, static_cast<double>(fs.e_above) * inv, quant);
        __syncthreads();
      }
      if (tid < 64) pick_mass(fs, C, Cerr, tgt, tgterr, inv, quant);
      __syncthreads();
      int t = fs.pos;
      if (t < 0) {
        // fp64 sweeps: t lies in [lo, hi + 1], position hi + 1 (if any) at or
        // above the target; candidates split the range evenly, the last is hi
        int lo = fs.amb_lo, hi = fs.amb_hi;
        double te = 0.0;
        for (int guard = 0; guard < 8; ++guard) {  // the range shrinks 8-fold per sweep
          const int n = min(kSelCand, hi - lo + 1);
          int cand[kSelCand];
          uint32_t B[kSelCand];
#pragma unroll
          for (int c = 0; c < kSelCand; ++c) {
            cand[c] = c < n ? lo + ((hi - lo + 1) * (c + 1)) / n - 1 : hi;
            B[c] = (((prefix << 8) | static_cast<uint32_t>(255 - cand[c])) << shift_d);
          }
          double acc[kSelCand + 1];
          exact_masses<LT, VEC, NT>(lrow, V, m, a.s64, klo, B, acc, sc);
          te = a.top_p * acc[kSelCand];
          int c1 = n;
          for (int c = n - 1; c >= 0; --c)
            if (acc[c] >= te) c1 = c;
          if (c1 == n) {
            t = min(hi + 1, kSelDigits - 1);
            break;
          }
          const int prev = c1 == 0 ? lo - 1 : cand[c1 - 1];
          if (cand[c1] - prev == 1) {
            t = cand[c1];
            break;
          }
          lo = prev + 1;
          hi = cand[c1] - 1;
          t = cand[c1];  // at or above the target (taken if the guard runs out)
        }
        // the exact Z_K replaces the fixed-point target below this level
        tgt = te * exp2(shift);
        tgterr = 1e-11 * tgt;
      }
      if (tid < 64) level_take(fs, t);
      __syncthreads();
      const double ma = static_cast<double>(fs.m_above) * inv, ea = static_cast<double>(fs.e_above) * inv;
      C += ma;
      Cerr += fixed_bound(ma, ea, quant);
      prefix = (prefix << 8) | static_cast<uint32_t>(255 - t);
      if (lv == kLevels - 1) {
        const double mt = static_cast<double>(fs.m_at) * inv, et = static_cast<double>(fs.e_at) * inv;
        Z = C + mt;
        dZ = Cerr + fixed_bound(mt, et, quant);
      }
      __syncthreads();  // fs is cleared by the next level
    }
    kt = prefix_key(prefix, kLevels);
  }
  tau = key_value(kt);
  Zt = Z;
  dZt = dZ;
}

// Returns (thread 0 of a lazy-mode block) the value its mark raise returned
// (RET_MARK), or 0: the caller consumes it later, so that the atomic's round
// trip overlaps the rest of the row's work. Without RET_MARK the raise returns
// nothing and the block never waits for it.
//
// STOP (the second launch of the lazy mode) with stop_on, for a row after
// its request's first position: the row stops as soon as an earlier
// position of its request is known to be a certain rejection (its mark
// raised during this launch; the first launch cleared the marks before),
// and is recorded as not read.
template <typename LT, bool VEC, int NT, bool EAGER, bool FILTER = false, bool RET_MARK = false, bool STOP = false>
__device__ __forceinline__ int probs_row(const ProbsArgs& a, const Task& t, float* dyn, BlockScratchT<NT>& sc,
                                         RowShared& sh,
                                         std::conditional_t<FILTER, FilterShared, NoFilterShared>* fsp = nullptr,
                                         bool stop_on = false) {
  const bool can_stop = STOP && stop_on && t.i > 0;
  static_assert(!(EAGER && FILTER), "top-k / top-p run in the lazy mode only");
  constexpr int kWaves = NT / 64;
  using L = Lay<LT, VEC>;
  using Raw = RawTile<LT, VEC>;

  const int V = a.V;
  const int nt = (V + kTile - 1) / kTile;
  float* S = dyn;           // tile sums of exp2((l - M_j) s), local units
  float* M = dyn + nt;      // running max when the tile was summed (>= every element of the tile)
  float* W = dyn + 2 * nt;  // tile sums of max(0, p - q)
  float* EA = dyn + 3 * nt; // tile sums of e |a| (a = the exp argument), for the error bound
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);

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
  float cut1 = -INFINITY;  // top-k / top-p: pass 1 gathers the head {l >= cut1}
  int hcnt = 0;            // (into per-wave slices, hcnt elements offered by this wave)
  auto tile1 = [&](const Raw& r, int j) {
    const int base = j * kTile;
    // the tile's maximum first: a tile that raises the wave's reference is
    // summed once, against the raised one
    float lm = -INFINITY;
    float gm[kLaneElems / 8];  // (top-k / top-p: the maxima of the lane's groups of 8 slots)
    if constexpr (FILTER) {
#pragma unroll
      for (int g = 0; g < kLaneElems; g += 8) {
        gm[g / 8] = r.get(g);
#pragma unroll
        for (int k = g + 1; k < g + 8; ++k) gm[g / 8] = fmaxf(gm[g / 8], r.get(k));
        lm = fmaxf(lm, gm[g / 8]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < kLaneElems; ++k) lm = fmaxf(lm, r.get(k));
    }
    if (__any(lm > ref)) ref = fmaxf(ref, wave_max(lm));
    if constexpr (FILTER) {
      if (__any(lm >= cut1))
        head_append_groups_wave<LT, VEC>(r, gm, base, V, lane, cut1, fsp->head + wave * (kHeadCap / kWaves),
                                         kHeadCap / kWaves, hcnt);
    }
    float es = 0.f, ea = 0.f;
    const bool special = base + kTile > V || (xmask >= base && xmask < base + kTile);  // uniform
    if (!special && ref != -INFINITY) {
      const float c = -(ref * s);
      float e4[4] = {0.f, 0.f, 0.f, 0.f};
      float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < kLaneElems; ++k) {
        const float arg = fmaf(r.get(k), s, c);
        const float e = fexp2(arg);
        e4[k & 3] += e;
        a4[k & 3] = fmaf(e, arg, a4[k & 3]);
      }
      es = (e4[0] + e4[1]) + (e4[2] + e4[3]);
      ea = (a4[0] + a4[1]) + (a4[2] + a4[3]);
    }
    // the careful sum: the partial last tile, the one-hot token's tile, and a
    // tile with a -inf or a NaN (e a = NaN)
    if (__any(special || !(ea == ea))) {
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
    if (STOP && tid == 0) sh.stop = 0;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) ref = fmaxf(ref, sh.wmax[w]);
    if constexpr (FILTER) {
      cut1 = ref - kHeadH1 / s;
    }
    // (can_stop) each wave loads the request's mark at every step (one
    // request for the wave) and tests the value it loaded the step before,
    // whose round trip the step's tile overlapped
    int mk = 0;
    bool halted = false;
    auto stopped = [&]() {
      halted = __builtin_amdgcn_readfirstlane(mk) > kMarkBase - t.i;
      mk = __hip_atomic_load(a.mark + t.b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return halted;
    };
    if (j < nt) {
      while (true) {
        rb.load(lrow, V, min(j + kWaves, nt - 1) * kTile, lane);
        tile1(ra, j);
        j += kWaves;
        if (j >= nt) break;
        if (can_stop && stopped()) break;
        ra.load(lrow, V, min(j + kWaves, nt - 1) * kTile, lane);
        tile1(rb, j);
        j += kWaves;
        if (j >= nt) break;
        if (can_stop && stopped()) break;
      }
    }
    if (can_stop && halted && lane == 0) sh.stop = 1;
    // the wave's final reference is the largest M_j of its tiles (every raise
    // sets it to the raising tile's M_j); a wave without tiles holds the block
    // maximum of the first tiles
    if (lane == 0) sh.wref[wave] = ref;
    if constexpr (FILTER) {
      if (lane == 0) {
        fsp->wcnt[wave] = hcnt;
      }
      if (tid == 0) {
        fsp->cut1 = cut1;
        fsp->cut2 = cut1 - kCount2 / s;
      }
    }
  }
  __syncthreads();
  if (can_stop && sh.stop) {  // (uniform: no wave writes it after the barrier)
    if (tid == 0) a.ws[t.trow] = make_int2(-1, static_cast<int>(kRowUnread));
    return 0;
  }

  // Row max m, c_m = fl(-m s) and Z = sum_j S_j exp2(c_m - c_j) in e-units.
  // The c_j cancel exactly, so Z approximates 2^D sum_k 2^((l_k - m) s) with
  // D = c_m + m s (|D| <= u |m s|); D is carried into p(x) exactly.
  float m = -INFINITY;  // = max_j M_j
#pragma unroll
  for (int w = 0; w < kWaves; ++w) m = fmaxf(m, sh.wref[w]);
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
  double dZ = bt + kSumErr * Z;  // |Z~ - 2^D Z|
  const double shift = static_cast<double>(cm) + static_cast<double>(m) * static_cast<double>(s);  // D, exact
  // top-k / top-p: the threshold tau, and Z over the kept set {l >= tau}
  float tau = -INFINITY;
  uint32_t tier = 0;  // record bits: how tau was found (beyond pass 1's head)
  if constexpr (FILTER) {
    if (m != -INFINITY && Z > 0.0 && Z < INFINITY) {
      const int h = head_threshold<LT, VEC, NT>(a, lrow, m, shift, Z, dZ, *fsp, sc, tau, Z, dZ);
      if (h == 0) {
        row_threshold<LT, VEC, NT>(a, lrow, m, shift, *fsp, sc, tau, Z, dZ);
        tier = kRowHead2 | kRowRowSelect;
      } else if (h == 2) {
        tier = kRowHead2;
      }
    }
  }
  const double relZ = dZ / Z;

  // ---------------- accept test of a draft row (fp64 p(x), certified)
  if (tid == 0) {
    sh.m = m;
    sh.z = Z;
    int accepted = 0;
    uint32_t why = 0;
    double px = 0.0;
    if (is_draft) {
      const bool kept = x_ok && lx >= tau;  // p(x) = 0 exactly for a token outside the kept set
      if (kept) px = exp2((static_cast<double>(lx) - static_cast<double>(m)) * a.s64 + shift) / Z;
      const double qx = onehot ? 1.0 : static_cast<double>(qx_in);
      const double lhs = static_cast<double>(u_acc) * qx;
      accepted = (x_ok && px > 0.0 && lhs <= px) ? 1 : 0;
      if (kept) {
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
  int mark_ret = 0;
  if constexpr (!EAGER) {
    // lazy mode: an accept test the bound cannot settle, every rejection and
    // every bonus row are left to the per-request pass, with the row max and
    // the certified Z interval in fp64 units (or {0, inf} when there is none)
    if (tid == 0) {
      const uint32_t f = sh.uncertain ? kRowUndecided : ((is_draft && accepted) ? kRowAccepted : kRowDeferred);
      // a certain rejection raises the request's mark; with RET_MARK the
      // returned value goes back to the caller, which stores it (waiting for
      // the atomic) before the first launch's count; otherwise the atomic
      // returns nothing (the block's slot is not held for its round trip)
      if (is_draft && f == kRowDeferred) {
        if constexpr (RET_MARK)
          mark_ret = __hip_atomic_fetch_max(a.mark + t.b, kMarkBase - t.i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          (void)__hip_atomic_fetch_max(a.mark + t.b, kMarkBase - t.i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (f != kRowAccepted) {
        double z = 0.0, dz = INFINITY;
        if (Z > 0.0 && Z < INFINITY && dZ < Z && m != -INFINITY) {
          const double unshift = exp2(-shift);  // 2^-D
          z = Z * unshift;
          dz = dZ * unshift;
        }
        a.rstat[t.trow] = make_double4(static_cast<double>(m), z, dz, static_cast<double>(tau));
      }
      a.ws[t.trow] = make_int2(-1, static_cast<int>(f | tier));
    }
    return mark_ret;
  }
  if (sh.uncertain) {
    if (tid == 0) flag_exact(a, t, static_cast<uint32_t>(sh.uncertain), m, false, Z, dZ);
    return 0;
  }
  const bool sample = !is_draft || !accepted || all_res;
  if (!sample) {
    if (tid == 0) a.ws[t.trow] = make_int2(-1, static_cast<int>(kRowAccepted));
    return 0;
  }

  sample_row<LT, VEC, NT, EAGER>(a, t, lrow, qrow, xmask, accepted, m, Z, bt, relZ, sh.px, S, M, W, sc, sh);
  return 0;
}

// Eager modes: one block per row (draft rows first, then bonus rows).
template <typename LT, bool VEC, int NT>
__global__ __launch_bounds__(NT) void probs_rows_kernel(ProbsArgs a) {
  extern __shared__ float dyn[];
  __shared__ BlockScratchT<NT> sc;
  __shared__ RowShared sh;
  const Task t = decode_task(blockIdx.x, a.cu, a.B, a.gamma, a.ndraft);
  if (!t.valid) return;  // request with invalid offsets: the select kernel skips it
  probs_row<LT, VEC, NT, true>(a, t, dyn, sc, sh);
}

// Lazy mode: one block per row of positions [p0, p1) (see decode_task_lazy).
// Algorithm 1 stops at the first rejection ([READING] and [VISUAL],
// Algorithm 1): a row after a position already known to be a certain
// rejection is not needed and is not read (it is recorded as unread). The
// host launches the first positions (as many as fill the chip once: two at
// 256 requests) first; the second launch then sees every mark those rows
// set and reads only the rows of requests that survived them (rows whose
// earlier positions are still undecided are read speculatively).
// The second launch's tasks, written by the last block of the first launch
// to finish: every row at a position >= p1 of each request still undecided
// after positions [0, p1) (no certain rejection there), request by request
// in request order, so that the rows that can matter are dispatched first
// and no block is launched for a request already decided. The rows at
// positions >= p1 of every other request are recorded as unread.
template <int NT>
__device__ void list_survivors(const ProbsArgs& a, int p1, RowShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kW = NT / 64;
  int base = 0;
  for (int b0 = 0; b0 < a.B; b0 += NT) {
    const int b = b0 + static_cast<int>(threadIdx.x);
    int cnt = 0;  // this request's tasks
    if (b < a.B) {
      int d0, d1;
      if (a.cu) {
        d0 = a.cu[b];
        d1 = a.cu[b + 1];
      } else {
        d0 = b * a.gamma;
        d1 = d0 + a.gamma;
      }
      const bool ok = !a.cu || (d0 >= 0 && d1 >= d0 && d1 <= a.ndraft);
      const int g = d1 - d0;
      const bool keep = ok && g >= p1 &&
                        __hip_atomic_load(a.mark + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <= kMarkBase - p1;
      if (keep) {
        cnt = g + 1 - p1;
      } else if (ok) {
        for (int i = p1; i <= g; ++i)
          a.ws[static_cast<int64_t>(d0) + b + i] = make_int2(-1, static_cast<int>(kRowUnread));
      }
    }
    // offsets: exclusive scan of the counts over the block (lanes, then waves)
    const int incl = wave_scan_incl_i_dpp(cnt);
    if (lane == 63) sh.wcount[wave] = incl;
    __syncthreads();
    int off = base + incl - cnt;
    for (int w = 0; w < wave; ++w) off += sh.wcount[w];
    for (int k = 0; k < cnt; ++k) a.tasks[off + k] = make_int2(b, p1 + k);
    for (int w = 0; w < kW; ++w) base += sh.wcount[w];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.surv_n[0] = base;
}

// The second launch without a list (see kSelfListMaxReads): every block derives the same list from the marks the first
// launch left (its survivors, request by request, in request order) and takes
// entry blockIdx.x, so the first launch ends with its last row instead of
// counting its blocks and listing serially. The later rows of every request
// that did not survive are recorded unread by the block that owns the
// request (b mod the grid). Raises made in this launch (positions >= p1)
// never change a request's survival, so any value a block reads agrees.
template <int NT>
__device__ Task self_listed_task(const ProbsArgs& a, int p1, RowShared& sh, int& ntask) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kW = NT / 64;
  const int k = blockIdx.x;
  if (threadIdx.x == 0) sh.qtask = make_int2(-1, 0);
  int base = 0;
  for (int b0 = 0; b0 < a.B; b0 += NT) {
    const int b = b0 + static_cast<int>(threadIdx.x);
    int cnt = 0;
    int d0 = 0;
    if (b < a.B) {
      int d1;
      if (a.cu) {
        d0 = a.cu[b];
        d1 = a.cu[b + 1];
      } else {
        d0 = b * a.gamma;
        d1 = d0 + a.gamma;
      }
      const bool ok = !a.cu || (d0 >= 0 && d1 >= d0 && d1 <= a.ndraft);
      const int g = d1 - d0;
      const bool keep = ok && g >= p1 &&
                        __hip_atomic_load(a.mark + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <= kMarkBase - p1;
      if (keep) {
        cnt = g + 1 - p1;
      } else if (ok && b % static_cast<int>(gridDim.x) == k) {
        for (int i = p1; i <= g; ++i)
          a.ws[static_cast<int64_t>(d0) + b + i] = make_int2(-1, static_cast<int>(kRowUnread));
      }
    }
    // offsets: exclusive scan of the counts over the block (lanes, then waves)
    const int incl = wave_scan_incl_i_dpp(cnt);
    if (lane == 63) sh.wcount[wave] = incl;
    __syncthreads();
    int off = base + incl - cnt;
    for (int w = 0; w < wave; ++w) off += sh.wcount[w];
    if (cnt > 0 && k >= off && k < off + cnt) sh.qtask = make_int2(b, p1 + (k - off));
    for (int w = 0; w < kW; ++w) base += sh.wcount[w];
    __syncthreads();
  }
  ntask = base;
  const int2 e = sh.qtask;
  if (e.x < 0) {
    Task t;
    t.valid = false;
    return t;
  }
  return lazy_task(e.x, e.y, a.cu, a.B, a.gamma, a.ndraft);
}

constexpr int kExpW = 4;  // exps in flight per lane in the fp64 pass
constexpr int kExp2Bits = 8;                  // table index bits
constexpr int kExp2Tab = 1 << kExp2Bits;      // 2^(j/256), j = 0..255 (2 KB of LDS)
constexpr double kExp2Scale = kExp2Tab;       // 256
constexpr double kExp2InvScale = -1.0 / kExp2Tab;

// 2^a in fp64 for a <= 0 (or -inf), to about 1 ulp (measured on the host
// against long double: at most 3.5e-16 relative). J = round(256 a) comes out
// of one fma with 1.5 * 2^52 (the integer is left in the low word), so
// a = J / 256 + r with |r| <= 1/512 exactly; J = 256 n + j with 0 <= j < 256;
// 2^r from its Taylor series to degree 4 (truncation < 4e-17 relative:
// (ln 2 / 512)^5 / 5!), 2^(j/256) from `tab` (an LDS copy), 2^n by ldexp.
// Arguments below -1100 (and -inf) give 0. (A 64-entry table with degree 5
// is as accurate and one fma slower per element.)
__device__ __forceinline__ double exp2_neg(double a, const double* __restrict__ tab) {
  constexpr double kRnd = 6755399441055744.0;  // 1.5 * 2^52
  constexpr double c1 = 0.6931471805599453, c2 = 0.2402265069591007, c3 = 0.05550410866482158,
                   c4 = 0.009618129107628477;
  a = fmax(a, -1100.0);
  const double t = fma(a, kExp2Scale, kRnd);
  const double r = fma(t - kRnd, kExp2InvScale, a);  // a - J / 256, exact
  const int J = __double2loint(t);
  double p = fma(c4, r, c3);
  p = fma(p, r, c2);
  p = fma(p, r, c1);
  p = fma(p, r, 1.0);
  return ldexp(p * tab[J & (kExp2Tab - 1)], J >> kExp2Bits);
}

// Fill the table of exp2_neg (every thread of the block takes part).
__device__ __forceinline__ void exp2_table_init(double* tab) {
  for (int i = threadIdx.x; i < kExp2Tab; i += blockDim.x) tab[i] = exp2(static_cast<double>(i) / kExp2Scale);
}

// The constants of exp2_neg as fp64 instruction operands: an fp64 instruction
// can take only one scalar operand, so two uniform constants in one fma would
// otherwise be copied into VGPRs at every use; as compile-time constants the
// compiler keeps or rematerialises them without holding VGPRs.
// The two fmas whose other constant operand is already scalar take theirs
// from a vector register held for the whole pass (scale_v, c4_v: the asm
// keeps the compiler from folding them back into constants), so no constant
// is copied at each use.
struct Exp2Consts {
  double rnd, scale, inv_scale, lo, c1, c2, c3, c4;
  double scale_v, c4_v;
};
__device__ __forceinline__ Exp2Consts exp2_consts_load() {
  Exp2Consts c{6755399441055744.0, kExp2Scale, kExp2InvScale, -1100.0, 0.6931471805599453, 0.2402265069591007,
               0.05550410866482158, 0.009618129107628477, kExp2Scale, 0.009618129107628477};
  asm volatile("" : "+v"(c.scale_v));
  asm volatile("" : "+v"(c.c4_v));
  return c;
}

// exp2_neg of N arguments at once, in phases (all table reads, then all
// polynomials, then the scaling), so that the LDS latency is paid once.
template <int N>
__device__ __forceinline__ void exp2_negN(const double (&a)[N], const double* __restrict__ tab, const Exp2Consts& C,
                                          double (&e)[N]) {
  const double kRnd = C.rnd;
  const double c1 = C.c1, c2 = C.c2, c3 = C.c3, c4 = C.c4;
  double r[N], tv[N];
  int J[N];
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const double ak = fmax(a[k], C.lo);
    const double t = fma(ak, C.scale_v, kRnd);
    r[k] = fma(t - kRnd, C.inv_scale, ak);
    J[k] = __double2loint(t);
    tv[k] = tab[J[k] & (kExp2Tab - 1)];
  }
#pragma unroll
  for (int k = 0; k < N; ++k) {
    double p = fma(C.c4_v, r[k], c3);
    p = fma(p, r[k], c2);
    p = fma(p, r[k], c1);
    p = fma(p, r[k], 1.0);
    e[k] = ldexp(p * tv[k], J[k] >> kExp2Bits);
  }
}

// Memo of the fp64 sums for bf16 logits: e(l) = 2^((l - m) s) of one row for
// every bf16 value l with 2^-10 <= |l| < 2^6 (16 binades of 128 codes, both
// signs: 4096 entries, 32 KB of LDS), each computed by the same fma and
// exp2_neg as the direct path, so a looked-up e equals the computed one bit
// for bit. Entry of code c: (c & 0x7fff) - kMemoLo, plus kMemoHalf when the
// sign bit is set. A bf16 row holds at most 65536 distinct values and the
// bulk of a logit row lies in these binades, so a block builds the table once
// per row (4096 exp2) and then reads one entry per element instead of
// evaluating the exp2; groups holding a value outside the range (tiny or large
// magnitudes, inf, NaN) take the direct path.
constexpr int kMemoHalf = 16 * 128;
constexpr int kMemoN = 2 * kMemoHalf;
constexpr uint32_t kMemoLo = (127u - 10u) << 7;  // bf16 magnitude code of 2^-10
template <typename LT, bool VEC>
constexpr bool kMemo = VEC && std::is_same_v<LT, uint16_t>;

// Memo entries of the two bf16 values packed in w (low half first), as two
// 16-bit fields; the 16-bit offsets from kMemoLo are or-ed into `miss`, where
// any bit of 0xf800 in a half marks a value outside the memo (its entry is
// then some other in-range one, replaced by the direct path).
__device__ __forceinline__ uint32_t memo_index2(uint32_t w, uint32_t& miss) {
  using u16x2 = unsigned short __attribute__((ext_vector_type(2)));
  const u16x2 mag = __builtin_bit_cast(u16x2, w & 0x7fff7fffu);
  const u16x2 lo = {static_cast<unsigned short>(kMemoLo), static_cast<unsigned short>(kMemoLo)};
  const uint32_t off = __builtin_bit_cast(uint32_t, mag - lo);
  miss |= off;
  return (off & 0x07ff07ffu) | ((w >> 4) & 0x08000800u);  // sign bit 15 -> entry bit 11
}

// Build the memo of one row (every thread of the block takes part; the caller
// waits at a barrier before reading it). With MASK, values below tau are 0.
template <int NT, bool MASK>
__device__ __forceinline__ void memo_build(double* memo, double s, double nms, float tau,
                                           const double* __restrict__ tab, const Exp2Consts& C) {
  static_assert(kMemoN % (kExpW * NT) == 0, "whole rounds of the block");
  for (int i0 = threadIdx.x; i0 < kMemoN; i0 += kExpW * NT) {
    double ar[kExpW], e[kExpW];
#pragma unroll
    for (int k = 0; k < kExpW; ++k) {
      const uint32_t i = static_cast<uint32_t>(i0 + k * NT);
      const uint32_t code = ((i / kMemoHalf) << 15) | (kMemoLo + i % kMemoHalf);
      float l = __uint_as_float(code << 16);
      if constexpr (MASK) l = l < tau ? -INFINITY : l;
      ar[k] = fma(static_cast<double>(l), s, nms);
    }
    exp2_negN<kExpW>(ar, tab, C, e);
#pragma unroll
    for (int k = 0; k < kExpW; ++k) memo[i0 + k * NT] = e[k];
  }
}


// One-hot drafts with bf16 logits (no q rows; the lazy mode without top-k /
// top-p): the per-row pass sums the row in fp64 itself, e_k = 2^((l_k - A) s)
// with A the block maximum of the first tiles (the anchor, carried as the
// row's m), through the per-row memo (values outside its binades by the
// direct fp64 exp2), so that the per-request stage never reads the row
// again: with q = onehot(x) the residual is p without x's element, which the
// tile sums E_j give. Z = sum_j E_j and the accept test p(x) = e_x / Z are
// taken in fp64 (nothing left to certify); a row that is not accepted keeps
// its E_j in the workspace (SV_ROW_TILE_SUMS). A row whose anchor or Z is
// not finite and positive (all -inf first tiles, a value far above the
// anchor) takes the general body.
template <int NT, bool RET_MARK>
__device__ int onehot_memo_row(const ProbsArgs& a, const Task& t, float* dyn, BlockScratchT<NT>& sc, RowShared& sh,
                               double* memo, double* tab) {
  constexpr int kWaves = NT / 64;
  using Raw = RawTile<uint16_t, true>;
  const int V = a.V;
  const int nt = (V + kTile - 1) / kTile;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // (uniform: tile indices and their tests too)
  // the task is the block's (a second launch takes it from LDS): uniform, so
  // that the row's address stays in scalar registers
  auto uni64 = [](int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
  };
  const int64_t trow = uni64(t.trow), drow = uni64(t.drow);
  const uint16_t* __restrict__ lrow = static_cast<const uint16_t*>(a.logits) + trow * static_cast<int64_t>(V);
  const bool is_draft = drow >= 0;
  const int64_t x = is_draft ? a.x[drow] : -1;
  const bool x_ok = is_draft && x >= 0 && x < V;
  const float lx = x_ok ? to_float(lrow[x]) : -INFINITY;
  const float u_acc = is_draft ? a.u[trow] : 0.f;
  double* E = reinterpret_cast<double*>(dyn);  // [nt] (the dynamic LDS holds 4 nt floats)
  auto load = [&](Raw& r, int j) {
    if (j * kTile + kTile > V) r.load_padded(lrow, V, j * kTile, lane);  // -inf past the end
    else r.load_full(lrow, j * kTile, lane);
  };
  exp2_table_init(tab);
  Raw ra, rb;
  int j = wave;
  float lm = -INFINITY;
  if (j < nt) {
    load(ra, j);
#pragma unroll
    for (int k = 0; k < kLaneElems; ++k) lm = fmaxf(lm, ra.get(k));
    lm = wave_max(lm);
    if (j + kWaves < nt) load(rb, j + kWaves);  // in flight while the memo is built
  }
  if (lane == 0) sh.wmax[wave] = lm;
  __syncthreads();  // (also publishes tab)
  float A = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) A = fmaxf(A, sh.wmax[w]);
  if (A > -INFINITY && A < INFINITY) {
  const double s = a.s64;
  const double nms = -(static_cast<double>(A) * s);
  const Exp2Consts C = exp2_consts_load();
  memo_build<NT, false>(memo, s, nms, 0.f, tab, C);
  __syncthreads();
  auto tile_sum = [&](const Raw& r) {
    double es = 0.0;
#pragma unroll
    for (int w4 = 0; w4 < 16; w4 += 2) {  // the lane's 16 words, two at a time (four values)
      const uint4& q0 = r.d[w4 >> 2];
      const uint32_t w0 = (w4 & 3) == 0 ? q0.x : q0.z;
      const uint32_t w1 = (w4 & 3) == 0 ? q0.y : q0.w;
      uint32_t miss = 0;
      const uint32_t i01 = memo_index2(w0, miss), i23 = memo_index2(w1, miss);
      double e[4] = {memo[i01 & 0xffffu], memo[i01 >> 16], memo[i23 & 0xffffu], memo[i23 >> 16]};
      if (__builtin_amdgcn_ballot_w64((miss & 0xf800f800u) != 0u)) {  // rare; same values elsewhere
        const double ar[4] = {fma(static_cast<double>(__uint_as_float(w0 << 16)), s, nms),
                              fma(static_cast<double>(__uint_as_float(w0 & 0xffff0000u)), s, nms),
                              fma(static_cast<double>(__uint_as_float(w1 << 16)), s, nms),
                              fma(static_cast<double>(__uint_as_float(w1 & 0xffff0000u)), s, nms)};
        exp2_negN<4>(ar, tab, C, e);
      }
      es += (e[0] + e[1]) + (e[2] + e[3]);
    }
    return wave_sum_d_dpp(es);
  };
  // tiles wave, wave + kWaves, ...: ra holds the current one, rb the next
  // (its loads in flight), the one after goes into ra once ra is summed
  if (j < nt) {
    while (true) {
      const double ta = tile_sum(ra);
      if (lane == 0) E[j] = ta;
      if (j + 2 * kWaves < nt) load(ra, j + 2 * kWaves);
      j += kWaves;
      if (j >= nt) break;
      const double tb = tile_sum(rb);
      if (lane == 0) E[j] = tb;
      if (j + 2 * kWaves < nt) load(rb, j + 2 * kWaves);
      j += kWaves;
      if (j >= nt) break;
    }
  }
  __syncthreads();
  double zl = 0.0;
  for (int q = tid; q < nt; q += NT) zl += E[q];
  const double Z = block_sum_dpp<NT>(zl, sc);
  if (Z > 0.0 && Z < INFINITY) {
  if (tid == 0) {
    int accepted = 0;
    if (x_ok) {
      const double px = exp2_neg(fma(static_cast<double>(lx), s, nms), tab) / Z;
      accepted = (px > 0.0 && static_cast<double>(u_acc) <= px) ? 1 : 0;  // q(x) = 1
    }
    sh.accepted = accepted;
  }
  __syncthreads();
  const bool accepted = sh.accepted != 0;
  int mark_ret = 0;
  if (!accepted) {
    double* rs = a.rsum + trow * static_cast<int64_t>(nt);
    for (int q = tid; q < nt; q += NT) rs[q] = E[q];
  }
  if (tid == 0) {
    const uint32_t f = accepted ? kRowAccepted : (kRowDeferred | kRowTileSums);
    if (is_draft && !accepted) {  // a certain rejection raises the request's mark
      if constexpr (RET_MARK)
        mark_ret = __hip_atomic_fetch_max(a.mark + t.b, kMarkBase - t.i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        (void)__hip_atomic_fetch_max(a.mark + t.b, kMarkBase - t.i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!accepted) a.rstat[trow] = make_double4(static_cast<double>(A), Z, 0.0, -static_cast<double>(INFINITY));
    a.ws[trow] = make_int2(-1, static_cast<int>(f));
  }
  return mark_ret;
  }  // Z finite and positive
  }  // anchor finite
  __syncthreads();  // the general body reuses the shared state
  return probs_row<uint16_t, true, NT, false, false, RET_MARK>(a, t, dyn, sc, sh);
}

// (FILTER: at least four waves per SIMD, two blocks per CU as without it;
// the rare radix-select path of the threshold may then spill)
template <typename LT, bool VEC, int NT, bool FILTER, bool LIST, bool ONEHOT = false, bool STOP = false>
__global__ __launch_bounds__(NT, (FILTER || ONEHOT) ? 4 : 1) void lazy_rows_kernel(ProbsArgs a, int p1, int phase) {
  // phase 0: first launch, alone; 1: first launch, a second follows (its last
  // block lists the tasks); 2: second launch, from that list; 3: first
  // launch, a second follows that lists for itself; 4: that second launch.
  // LIST: built for phase 1 (the mark atomics return their values, which the
  // count waits for); otherwise they return nothing and no block waits for
  // their round trips. ONEHOT: bf16 rows of a batch with one-hot drafts, summed
  // in fp64 through the memo (onehot_memo_row).
  static_assert(!ONEHOT || (std::is_same_v<LT, uint16_t> && VEC && !FILTER), "one-hot memo rows: bf16, no filter");
  extern __shared__ float dyn[];
  __shared__ double memo_s[ONEHOT ? kMemoN : 1];
  __shared__ double tab_s[ONEHOT ? kExp2Tab : 1];
  __shared__ BlockScratchT<NT> sc;
  __shared__ RowShared sh;
  __shared__ std::conditional_t<FILTER, FilterShared, NoFilterShared> fsh;
  const bool second = phase == 2 || phase == 4;
  Task t;
  int ntask = 0;  // (second launch) rows it holds
  if constexpr (!FILTER) {
    if (phase == 4) t = self_listed_task<NT>(a, p1, sh, ntask);
  }
  if (FILTER || phase != 4)
    t = decode_task_lazy(blockIdx.x, a.cu, a.B, a.gamma, a.ndraft, phase == 2 ? a.tasks : nullptr,
                         phase == 2 ? a.surv_n[0] : 0);
  // the task is the block's (uniform): keep it in scalar registers
  {
    auto uni64 = [](int64_t v) {
      const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
      const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
      return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
    };
    t.b = __builtin_amdgcn_readfirstlane(t.b);
    t.g = __builtin_amdgcn_readfirstlane(t.g);
    t.i = __builtin_amdgcn_readfirstlane(t.i);
    t.trow = uni64(t.trow);
    t.drow = uni64(t.drow);
    t.srow = uni64(t.srow);
    t.valid = __builtin_amdgcn_readfirstlane(t.valid ? 1 : 0) != 0;
  }
  bool read = t.valid;
  // The request's mark starts at zero in every call: its position-0 block (in
  // the first launch) clears it before anything else. Blocks of the first
  // launch therefore never read marks (its rows start in one round anyway);
  // a mark raised there before the clear is lost, which only leaves a row to
  // be read that could have been skipped. The second launch and the task
  // list read marks after the first launch has completed.
  // (a returning exchange whose result is stored before this block's count
  // below: the clear has been performed before the count is issued; the
  // result is consumed only then, so the round trip overlaps the row)
  int mark_ret = 0;
  if (!second && t.valid && t.i == 0 && threadIdx.x == 0) {
    if constexpr (LIST)
      mark_ret = __hip_atomic_exchange(a.mark + t.b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      __hip_atomic_store(a.mark + t.b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (second && t.valid && t.i > 0) {
    if (threadIdx.x == 0)
      sh.skip = __hip_atomic_load(a.mark + t.b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) > kMarkBase - t.i;
    __syncthreads();
    if (sh.skip) {
      if (threadIdx.x == 0) a.ws[t.trow] = make_int2(-1, static_cast<int>(kRowUnread));
      read = false;
    }
  }
  if (read) {
    if constexpr (ONEHOT) mark_ret ^= onehot_memo_row<NT, LIST>(a, t, dyn, sc, sh, memo_s, tab_s);
    else {
      // (rows stop early only when the launch holds more rows than the chip
      // has compute units: then some units run two, and a row found
      // unneeded would otherwise set the launch's end)
      if (STOP && phase == 2) ntask = a.surv_n[0];
      mark_ret ^= probs_row<LT, VEC, NT, false, FILTER, LIST, STOP>(a, t, dyn, sc, sh, &fsh, ntask > a.cus);
    }
  }
  if (!LIST || phase != 1) return;
  if (threadIdx.x == 0) sh.mark_old = mark_ret;  // waits for this thread's mark atomics
  // first launch: the last block to finish lists the tasks of the second launch
  // reads. Marks and the count are device-scope atomics; every mark update
  // (the clear above, a raise in probs_row) is a returning atomic whose result
  // thread 0 stores above (so it has been performed) before that block's count
  // is issued, and the last block reads the marks with device-scope atomic
  // loads after its own count has returned, behind an acquire fence. No
  // block needs a release fence (a cache write-back) of its own.
  __syncthreads();
  if (threadIdx.x == 0)
    sh.last = __hip_atomic_fetch_add(a.surv_n + 16, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              static_cast<int>(gridDim.x) - 1;
  __syncthreads();
  if (!sh.last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  list_survivors<NT>(a, p1, sh);
  if (threadIdx.x == 0) a.surv_n[16] = 0;  // ready for the next call
}

// ----------------------------------------------------------------------------
// lazy mode, phase 2: one block per request decides the request in fp64.
//
// The rows are taken in order; an accepted row passes. The first row that is
// not (certainly rejected, or with an accept test the bound could not settle)
// gets one fp64 pass over its logits and q: per tile, the sum E_j of
// e_k = 2^((l_k - m) log2(e) / T) and the part of the residual sum that the
// certified Z interval [zlo, zhi] of the fast pass already decides: P_j and
// Q_j, the sums of e_k and of q_k over the elements with e_k / Z > q_k for
// every Z in the interval, and whether any element is left undecided. Then
// Z = sum_j E_j; an undecided accept test is settled exactly (an accepted row
// passes, and the next row is taken); W_j = P_j / Z - Q_j, the tiles with
// undecided elements summed again with Z; residual mass <= 1e-8 falls back to
// p; the tile search and the in-tile search draw the token in fp64. If every
// draft is accepted, the bonus row is sampled from p the same way. The block
// then writes the request's outputs.

// Chunk c (0..3) of a lane's part of the tile at `base`: the lane's elements
// k = 8c .. 8c + 7 in the tile layout (see Lay), as fp32 logits (-inf past the
// end of the row) and q (0 past the end; q == nullptr: zeros). Loads are
// unconditional, with addresses clamped into the row.
template <typename LT, bool VEC, bool PAD>
__device__ __forceinline__ void load_chunk(const LT* __restrict__ lrow, const float* __restrict__ qrow, int V,
                                           int base, int lane, int c, float (&lv)[8], float (&qv)[8]) {
  using L = Lay<LT, VEC>;
  if constexpr (VEC && sizeof(LT) == 2) {
    const int i0 = L::index(base, lane, 8 * c);
    const uint4 w = *reinterpret_cast<const uint4*>(lrow + min(i0, V - 8));
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    const bool in = !PAD || i0 < V;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      lv[2 * h] = in ? __uint_as_float(ww[h] << 16) : -INFINITY;
      lv[2 * h + 1] = in ? __uint_as_float(ww[h] & 0xffff0000u) : -INFINITY;
    }
    if (qrow) {
      const float4 q0 = *reinterpret_cast<const float4*>(qrow + min(i0, V - 8));
      const float4 q1 = *reinterpret_cast<const float4*>(qrow + min(i0, V - 8) + 4);
      qv[0] = in ? q0.x : 0.f; qv[1] = in ? q0.y : 0.f; qv[2] = in ? q0.z : 0.f; qv[3] = in ? q0.w : 0.f;
      qv[4] = in ? q1.x : 0.f; qv[5] = in ? q1.y : 0.f; qv[6] = in ? q1.z : 0.f; qv[7] = in ? q1.w : 0.f;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[e] = 0.f;
    }
  } else if constexpr (VEC) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i0 = L::index(base, lane, 8 * c + 4 * h);
      const bool in = !PAD || i0 < V;
      const float4 v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(lrow) + min(i0, V - 4));
      lv[4 * h + 0] = in ? v.x : -INFINITY; lv[4 * h + 1] = in ? v.y : -INFINITY;
      lv[4 * h + 2] = in ? v.z : -INFINITY; lv[4 * h + 3] = in ? v.w : -INFINITY;
      if (qrow) {
        const float4 q = *reinterpret_cast<const float4*>(qrow + min(i0, V - 4));
        qv[4 * h + 0] = in ? q.x : 0.f; qv[4 * h + 1] = in ? q.y : 0.f;
        qv[4 * h + 2] = in ? q.z : 0.f; qv[4 * h + 3] = in ? q.w : 0.f;
      } else {
        qv[4 * h + 0] = qv[4 * h + 1] = qv[4 * h + 2] = qv[4 * h + 3] = 0.f;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = L::index(base, lane, 8 * c + e);
      const bool in = !PAD || i < V;
      lv[e] = in ? to_float(lrow[min(i, V - 1)]) : -INFINITY;
      qv[e] = (qrow && in) ? qrow[min(i, V - 1)] : 0.f;
    }
  }
}

// A lane's chunk (elements k = 8c .. 8c + 7 of a tile, see Lay) kept raw as
// loaded, so that several chunks can be in flight: bf16 logits take 4 VGPRs,
// fp32 logits 8, q 8. Addresses are clamped into the row; elements past the
// end are masked when the chunk is used (get_l / get_q with PAD).
template <typename LT, bool VEC>
struct RawChunk;
template <>
struct RawChunk<uint16_t, true> {
  uint4 l;
  float4 q0, q1;
  int i0;
  __device__ __forceinline__ uint32_t word(int i) const { return i == 0 ? l.x : i == 1 ? l.y : i == 2 ? l.z : l.w; }
  __device__ __forceinline__ void load(const uint16_t* __restrict__ lrow, const float* __restrict__ qrow, int V,
                                       int base, int lane, int c, bool has_q) {
    i0 = Lay<uint16_t, true>::index(base, lane, 8 * c);
    const int ic = min(i0, V - 8);
    l = *reinterpret_cast<const uint4*>(lrow + ic);
    if (has_q) {
      q0 = *reinterpret_cast<const float4*>(qrow + ic);
      q1 = *reinterpret_cast<const float4*>(qrow + ic + 4);
    }
  }
  template <bool PAD>
  __device__ __forceinline__ float get_l(int e, int V) const {
    const uint32_t w = (e >> 1) == 0 ? l.x : (e >> 1) == 1 ? l.y : (e >> 1) == 2 ? l.z : l.w;
    const float v = (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
    return (!PAD || i0 + e < V) ? v : -INFINITY;
  }
  template <bool PAD>
  __device__ __forceinline__ float get_q(int e, int V) const {
    const float4& h = e < 4 ? q0 : q1;
    const int k = e & 3;
    const float v = k == 0 ? h.x : k == 1 ? h.y : k == 2 ? h.z : h.w;
    return (!PAD || i0 + e < V) ? v : 0.f;
  }
};
template <>
struct RawChunk<float, true> {
  float4 l0, l1, q0, q1;
  int i0;
  __device__ __forceinline__ void load(const float* __restrict__ lrow, const float* __restrict__ qrow, int V,
                                       int base, int lane, int c, bool has_q) {
    // two runs of 4 consecutive elements (Lay<float, true>: kE = 4)
    i0 = Lay<float, true>::index(base, lane, 8 * c);
    const int i1 = Lay<float, true>::index(base, lane, 8 * c + 4);
    l0 = *reinterpret_cast<const float4*>(lrow + min(i0, V - 4));
    l1 = *reinterpret_cast<const float4*>(lrow + min(i1, V - 4));
    if (has_q) {
      q0 = *reinterpret_cast<const float4*>(qrow + min(i0, V - 4));
      q1 = *reinterpret_cast<const float4*>(qrow + min(i1, V - 4));
    }
  }
  __device__ __forceinline__ int idx(int e) const { return e < 4 ? i0 + e : i0 + 64 * 4 + (e - 4); }
  template <bool PAD>
  __device__ __forceinline__ float get_l(int e, int V) const {
    const float4& h = e < 4 ? l0 : l1;
    const int k = e & 3;
    const float v = k == 0 ? h.x : k == 1 ? h.y : k == 2 ? h.z : h.w;
    return (!PAD || idx(e) < V) ? v : -INFINITY;
  }
  template <bool PAD>
  __device__ __forceinline__ float get_q(int e, int V) const {
    const float4& h = e < 4 ? q0 : q1;
    const int k = e & 3;
    const float v = k == 0 ? h.x : k == 1 ? h.y : k == 2 ? h.z : h.w;
    return (!PAD || idx(e) < V) ? v : 0.f;
  }
};
template <typename LT>
struct RawChunk<LT, false> {
  float l[8], q[8];
  int base, lane, c;
  __device__ __forceinline__ void load(const LT* __restrict__ lrow, const float* __restrict__ qrow, int V, int b_,
                                       int lane_, int c_, bool has_q) {
    base = b_;
    lane = lane_;
    c = c_;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = min(Lay<LT, false>::index(base, lane, 8 * c + e), V - 1);
      l[e] = to_float(lrow[i]);
      q[e] = has_q ? qrow[i] : 0.f;
    }
  }
  template <bool PAD>
  __device__ __forceinline__ float get_l(int e, int V) const {
    return (!PAD || Lay<LT, false>::index(base, lane, 8 * c + e) < V) ? l[e] : -INFINITY;
  }
  template <bool PAD>
  __device__ __forceinline__ float get_q(int e, int V) const {
    return (!PAD || Lay<LT, false>::index(base, lane, 8 * c + e) < V) ? q[e] : 0.f;
  }
};

// 8 consecutive elements from k0 (a multiple of 8), as fp32 logits (-inf past
// the end of the row) or q (0 past the end; q == nullptr: zeros, nothing
// read). Loads are unconditional, with addresses clamped into the row.
template <typename LT, bool VEC>
__device__ __forceinline__ void load8f(const LT* __restrict__ row, int V, int k0, float (&v)[8]) {
  if constexpr (VEC && sizeof(LT) == 2) {
    const uint4 w = *reinterpret_cast<const uint4*>(row + min(k0, V - 8));
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(ww[i] << 16);
      v[2 * i + 1] = __uint_as_float(ww[i] & 0xffff0000u);
    }
  } else if constexpr (VEC) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float4 w = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(row) + min(k0 + 4 * h, V - 4));
      v[4 * h] = w.x;
      v[4 * h + 1] = w.y;
      v[4 * h + 2] = w.z;
      v[4 * h + 3] = w.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = to_float(row[min(k0 + k, V - 1)]);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (k0 + k >= V) v[k] = -INFINITY;
}
template <bool VEC>
__device__ __forceinline__ void load8qf(const float* __restrict__ q, int V, int k0,
                                        float (&v)[8]) {
  if (q == nullptr) {  // uniform over the block: no q row, no load
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = 0.f;
    return;
  }
  if constexpr (VEC) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float4 w = *reinterpret_cast<const float4*>(q + min(k0 + 4 * h, V - 4));
      v[4 * h] = w.x;
      v[4 * h + 1] = w.y;
      v[4 * h + 2] = w.z;
      v[4 * h + 3] = w.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = q[min(k0 + k, V - 1)];
  }
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (k0 + k >= V) v[k] = 0.f;
}

// whether tile j of a row of V elements reaches past its end
__device__ __forceinline__ bool base_partial(int j, int nt, int V) { return j == nt - 1 && j * kTile + kTile > V; }

constexpr int kPassNT = 256;       // threads per block of the per-request kernel
constexpr int kPassWaves = kPassNT / 64;

// Shared state of the per-request kernel; the memo only with bf16 logits.
template <bool MEMO>
struct ReqSharedT {
  double part[4];  // per-wave partial sums (an undecided tile; the in-tile scan's wave totals)
  double memo[MEMO ? kMemoN : 1];
  int nund;     // tiles with undecided elements
  int cross, lastpos;
  int tile;
  double p_before;
  int token;
  int pad;
};

// The fp64 pass of one row over tiles j = j0, j0 + step, ... < j1, one tile
// per wave at a time, in four chunks of 8 elements per lane; a ring of four
// raw chunks keeps the loads of the next three chunks in flight while one is
// computed. Per tile it writes E_j (sum of e_k) and, for a draft row, Q_j and
// P_j, with P_j = -1 (impossible otherwise) marking a tile in which the Z
// interval leaves an element undecided (LDS or global, indexed by tile). With
// MASK, logits below tau (outside the top-k / top-p kept set) count as -inf.
template <typename LT, bool VEC, bool MASK, bool SPLIT = false, bool TAIL = false>
__device__ void fp64_row_pass(const LT* __restrict__ lrow, const float* __restrict__ qrow, int V, int nt, double m,
                              double s, double zhi, double zlo, bool draft, int j0, int j1, int step,
                              const double* __restrict__ tab, const Exp2Consts& C, double* E, double* P, double* Q,
                              float tau, double* memo, double (*cpart)[4][3] = nullptr, int (*cund)[4] = nullptr) {
  constexpr bool MEMO = kMemo<LT, VEC>;
  const int lane = threadIdx.x & 63;
  const double nms = -(m * s);  // e_k = 2^(l_k s - m s): the common rounding of m s cancels in p
  using Chunk = RawChunk<LT, VEC>;
  Chunk ring[4];
  auto load = [&](int slot, int jj, int c) {
    // chunks past the wave's last tile re-read the row's last tile (in bounds, unused)
    ring[slot].load(lrow, qrow, V, min(jj, nt - 1) * kTile, lane, c, draft);
  };
  double es = 0.0, ps = 0.0, qs = 0.0;
  uint64_t und = 0;  // lanes with an undecided element (wave masks: scalar operations)
  auto compute = [&](int slot, auto pad) {
    constexpr bool PD = decltype(pad)::value;
#pragma unroll
    for (int h = 0; h < 8; h += kExpW) {
      double ar[kExpW], e[kExpW];
      auto direct = [&]() {
#pragma unroll
        for (int k = 0; k < kExpW; ++k) {
          float l = ring[slot].template get_l<PD>(h + k, V);
          if constexpr (MASK) l = l < tau ? -INFINITY : l;
          ar[k] = fma(static_cast<double>(l), s, nms);
        }
        exp2_negN<kExpW>(ar, tab, C, e);
      };
      if constexpr (MEMO) {
        static_assert(kExpW == 4, "the memo lookup takes two words of two bf16 values");
        uint32_t miss = 0;
        const uint32_t i01 = memo_index2(ring[slot].word(h >> 1), miss);
        const uint32_t i23 = memo_index2(ring[slot].word((h >> 1) + 1), miss);
        // (the row's last tile: bf16 rows hold a multiple of 8 values, so a
        // lane's chunk lies wholly inside the row or wholly past its end;
        // one past the end adds nothing and misses nothing)
        const bool in = !PD || ring[slot].i0 < V;
        if (!in) miss = 0;
        e[0] = in ? memo[i01 & 0xffffu] : 0.0;
        e[1] = in ? memo[i01 >> 16] : 0.0;
        e[2] = in ? memo[i23 & 0xffffu] : 0.0;
        e[3] = in ? memo[i23 >> 16] : 0.0;
        if (__builtin_amdgcn_ballot_w64((miss & 0xf800f800u) != 0u)) direct();  // rare; same values elsewhere
      } else {
        direct();
      }
#pragma unroll
      for (int k = 0; k < kExpW; ++k) es += e[k];
      if (draft) {  // uniform; the element's side by a 0/1 factor
#pragma unroll
        for (int k = 0; k < kExpW; ++k) {
          const double q = static_cast<double>(ring[slot].template get_q<PD>(h + k, V));
          const bool pos = e[k] > q * zhi;
          const double w = pos ? 1.0 : 0.0;
          ps = fma(e[k], w, ps);
          qs = fma(q, w, qs);
          und |= __ballot(e[k] > q * zlo) & ~__ballot(pos);
        }
      }
    }
  };
  auto flush = [&](int jj) {
    const double te = wave_sum_d_dpp(es);
    double tp = 0.0, tq = 0.0;
    if (draft) {
      tp = wave_sum_d_dpp(ps);
      tq = wave_sum_d_dpp(qs);
    }
    const bool tu = und != 0;
    if (lane == 0) {
      E[jj] = te;
      P[jj] = tu ? -1.0 : tp;
      Q[jj] = tq;
    }
    es = ps = qs = 0.0;
    und = 0;
  };
  // chunk w (the wave) of each tile in [a0, a1), at most 3 tiles, all loads
  // at once; the tiles' sums are the four waves' partial sums added in wave
  // order (LDS partials, one barrier; every wave of the block takes part)
  auto split_tiles = [&](int a0, int a1, auto build) {
    const int w = threadIdx.x >> 6, nl = a1 - a0;
#pragma unroll
    for (int t = 0; t < 3; ++t)
      if (t < nl) load(t, a0 + t, w);
    if constexpr (MEMO && decltype(build)::value) {
      memo_build<kPassNT, MASK>(memo, s, nms, tau, tab, C);
      __syncthreads();
    }
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      if (t < nl) {
        if (base_partial(a0 + t, nt, V)) compute(t, std::true_type{});
        else compute(t, std::false_type{});
        const double te = wave_sum_d_dpp(es);
        double tp = 0.0, tq = 0.0;
        if (draft) {
          tp = wave_sum_d_dpp(ps);
          tq = wave_sum_d_dpp(qs);
        }
        if (lane == 0) {
          cpart[t][w][0] = te;
          cpart[t][w][1] = tp;
          cpart[t][w][2] = tq;
          cund[t][w] = und != 0 ? 1 : 0;
        }
        es = ps = qs = 0.0;
        und = 0;
      }
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < nl) {
      double te = 0.0, tp = 0.0, tq = 0.0;
      int tu = 0;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        te += cpart[t][v][0];
        tp += cpart[t][v][1];
        tq += cpart[t][v][2];
        tu |= cund[t][v];
      }
      E[a0 + t] = te;
      P[a0 + t] = tu ? -1.0 : tp;
      Q[a0 + t] = tq;
    }
  };
  // whole tiles j, j + stp, ... < jend of one wave (the first tile's first
  // three chunks already loaded)
  auto run = [&](int j, int jend, int stp) {
    for (; j < jend; j += stp) {
      const int jn = j + stp < jend ? j + stp : j;
      if (base_partial(j, nt, V)) {
        load(3, j, 3); compute(0, std::true_type{});
        load(0, jn, 0); compute(1, std::true_type{});
        load(1, jn, 1); compute(2, std::true_type{});
        load(2, jn, 2); compute(3, std::true_type{});
      } else {
        load(3, j, 3); compute(0, std::false_type{});
        load(0, jn, 0); compute(1, std::false_type{});
        load(1, jn, 1); compute(2, std::false_type{});
        load(2, jn, 2); compute(3, std::false_type{});
      }
      flush(j);
    }
  };
  if constexpr (SPLIT) {  // a slice of fewer tiles than waves
    split_tiles(j0, j1, std::true_type{});
    return;
  }
  if constexpr (TAIL) {
    // a slice [j0, j1): its whole rounds of four tiles one tile per wave,
    // then the last (j1 - j0) mod 4 tiles by chunks over the four waves, so
    // that no wave takes a tile more than the others
    const int w = threadIdx.x >> 6;
    const int jm = j0 + kPassWaves * ((j1 - j0) / kPassWaves);
    const int jw = j0 + w;
    if (jw < jm) {
      load(0, jw, 0);
      load(1, jw, 1);
      load(2, jw, 2);
    }
    if constexpr (MEMO) {
      memo_build<kPassNT, MASK>(memo, s, nms, tau, tab, C);
      __syncthreads();
    }
    run(jw, jm, kPassWaves);
    if (jm < j1) split_tiles(jm, j1, std::false_type{});  // (uniform)
    return;
  }
  int j = j0;
  if constexpr (MEMO) {
    // the first loads go out before the memo is built (every thread of the
    // block builds it and waits at the barrier, with or without tiles)
    if (j < j1) {
      load(0, j, 0);
      load(1, j, 1);
      load(2, j, 2);
    }
    memo_build<kPassNT, MASK>(memo, s, nms, tau, tab, C);
    __syncthreads();
    if (j >= j1) return;
  } else {
    if (j >= j1) return;
    load(0, j, 0);
    load(1, j, 1);
    load(2, j, 2);
  }
  run(j, j1, step);
}

// The request's first row >= start whose own accept test did not pass (g if
// none), found by every wave alike (a ballot over 64 rows at a time: no LDS,
// no barrier); uniform on return.
template <int NT>
__device__ __forceinline__ int first_open_row(const int2* __restrict__ ws, int64_t t0, int start, int g) {
  const int lane = threadIdx.x & 63;
  for (int i0 = start; i0 < g; i0 += 64) {
    const int i = i0 + lane;
    const uint64_t open = __ballot(i < g && !(static_cast<uint32_t>(ws[t0 + i].y) & kRowAccepted));
    if (open) return i0 + __ffsll(static_cast<unsigned long long>(open)) - 1;
  }
  return g;
}

__device__ __forceinline__ bool request_range(const ProbsArgs& a, int b, int& d0, int& d1) {
  if (a.cu) {
    d0 = a.cu[b];
    d1 = a.cu[b + 1];
    return d0 >= 0 && d1 >= d0 && d1 <= a.ndraft;
  }
  d0 = b * a.gamma;
  d1 = d0 + a.gamma;
  return true;
}

constexpr int kMaxSlices = 16;     // most blocks per request
static_assert(kPassWaves == 4, "the finish's in-tile search maps 16 scan lanes to each of four waves");

// One-hot drafts (no q rows): the draft token of draft row d when it lies in
// the vocabulary, else -1; -1 for a bonus row or when q rows are given.
__device__ __forceinline__ int onehot_index(const ProbsArgs& a, bool draft, int64_t d) {
  if (!draft || a.q) return -1;
  const int64_t x = a.x[d];
  return (x >= 0 && x < a.V) ? static_cast<int>(x) : -1;
}

struct PassArrays {  // per request: [B][nt] tile sums of its deciding row (the fp64 path's tile arrays)
  double* E;
  double* P;
  double* Q;
};

// The finish of one request at its open row n (the first row whose own
// accept test did not pass), by one block of kPassNT threads, with the row's
// tile sums E_j, P_j, Q_j already in LDS: Z = sum_j E_j; an undecided accept
// test settled exactly - if the row is accepted after all, its record says so
// and the function returns true (the caller takes the next open row);
// otherwise residual tile sums W_j = P_j / Z - Q_j, tiles with undecided
// elements summed again with Z, residual mass <= 1e-8 falls back to p, wave 0
// draws the token (tile search, then in-tile search, in fp64) and writes the
// request's outputs, and the function returns false.
template <typename LT, bool VEC, bool FILTER>
__device__ bool finish_row(const ProbsArgs& a, const SelectArgs& sel, int b, int d0, int d1, int n, double* rbuf,
                           BlockScratchT<kPassNT>& sc, ReqSharedT<kMemo<LT, VEC>>& rs,
                           const double* __restrict__ tab,
                           const Exp2Consts& C) {
  const int V = a.V;
  const int nt = (V + kTile - 1) / kTile;
  double* E = rbuf;
  double* P = rbuf + nt;
  double* Q = rbuf + 2 * nt;
  double* W = rbuf + 3 * nt;
  int* ulist = reinterpret_cast<int*>(rbuf + 4 * nt);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = d1 - d0;
  const int64_t t0 = static_cast<int64_t>(d0) + b;
  const double s = a.s64;
  const double u_smp = static_cast<double>(a.u[t0 + g]);  // the request's sample uniform

  {
    const int64_t trow = t0 + n;
    const bool draft = n < g;
    const uint32_t f0 = static_cast<uint32_t>(a.ws[trow].y);
    const bool undecided = draft && (f0 & kRowUndecided);
    const double4 st = a.rstat[trow];
    const double m = st.x;
    const double nms = -(m * s);
    const float keep_min = static_cast<float>(st.w);  // top-k / top-p threshold tau (-inf: no filter)
    auto masked = [&](float l) { return (FILTER && l < keep_min) ? -INFINITY : l; };
    const LT* __restrict__ lrow = static_cast<const LT*>(a.logits) + trow * static_cast<int64_t>(V);
    const float* __restrict__ qrow = (draft && a.q) ? a.q + static_cast<int64_t>(d0 + n) * V : nullptr;
    const int hot = onehot_index(a, draft, d0 + n);
    const bool onehot = draft && !a.q;
    for (int j = tid; j < nt; j += kPassNT) W[j] = P[j] < 0.0 ? -1.0 : 0.0;  // -1: undecided elements
    double zl = 0.0;
    for (int j = tid; j < nt; j += kPassNT) zl += E[j];
    const double Z = block_sum_dpp<kPassNT>(zl, sc);
    const double iz = 1.0 / Z;

    uint32_t rflags = undecided ? (kRowExact | kWhyAccept) : 0u;
    if (undecided) {
      const int64_t x = a.x[d0 + n];
      const bool x_ok = x >= 0 && x < V;
      const double px =
          x_ok ? exp2_neg(fma(static_cast<double>(masked(to_float(lrow[x]))), s, nms), tab) * iz : 0.0;
      const double qx = x_ok ? (onehot ? 1.0 : static_cast<double>(qrow[x])) : 0.0;
      if (x_ok && px > 0.0 && static_cast<double>(a.u[trow]) * qx <= px) {
        if (tid == 0)
          a.ws[trow] = make_int2(
              -1, static_cast<int>(kRowAccepted | rflags | (f0 & (kRowHead2 | kRowRowSelect | kRowTileSums))));
        __syncthreads();
        return true;
      }
    }

    // ---- tile values: residual (draft row) or p (bonus row, or fallback)
    int mode = draft ? 1 : 0;
    if (onehot) {
      // q = onehot(x): the residual max(0, p - q) is p without x's element
      // (p(x) <= 1), so W_j = E_j / Z except in x's tile, which loses e_x
      // (computed as in the pass); a token outside the vocabulary removes
      // nothing
      const int jx = hot >= 0 ? hot / kTile : -1;
      const double ex = hot >= 0 ? exp2_neg(fma(static_cast<double>(to_float(lrow[hot])), s, nms), tab) : 0.0;
      for (int j = tid; j < nt; j += kPassNT) W[j] = (j == jx ? fmax(0.0, E[j] - ex) : E[j]) * iz;
      __syncthreads();
    } else if (draft) {
      if (tid == 0) rs.nund = 0;
      __syncthreads();
      for (int j = tid; j < nt; j += kPassNT) {
        if (W[j] < 0.0) ulist[atomicAdd(&rs.nund, 1)] = j;
        else W[j] = fmax(0.0, P[j] * iz - Q[j]);
      }
      __syncthreads();
      // tiles with undecided elements (usually none or one), summed again
      // with Z by the whole block: wave w takes chunk w of each lane's part
      for (int k = 0; k < rs.nund; ++k) {
        const int j = ulist[k];
        float lv[8], qv[8];
        load_chunk<LT, VEC, true>(lrow, qrow, V, j * kTile, lane, wave, lv, qv);
        double ws = 0.0;
#pragma unroll
        for (int g4 = 0; g4 < 8; g4 += kExpW) {
          double ar[kExpW], e[kExpW];
#pragma unroll
          for (int kk = 0; kk < kExpW; ++kk) ar[kk] = fma(static_cast<double>(masked(lv[g4 + kk])), s, nms);
          exp2_negN<kExpW>(ar, tab, C, e);
#pragma unroll
          for (int kk = 0; kk < kExpW; ++kk) ws += fmax(0.0, e[kk] * iz - static_cast<double>(qv[g4 + kk]));
        }
        ws = wave_sum_d(ws);
        if (lane == 0) rs.part[wave] = ws;
        __syncthreads();
        if (tid == 0) W[j] = (rs.part[0] + rs.part[1]) + (rs.part[2] + rs.part[3]);
        __syncthreads();
      }
    }
    auto tile_val = [&](int j) -> double { return mode == 1 ? W[j] : E[j] * iz; };
    // ---- tile-level search: every wave computes it (the same LDS values in
    // the same order give identical results in each), with wave-level scans
    // (lanes in token order) and no block barriers
    // tile-level CDF: lane l owns tiles [l tp, (l + 1) tp)
    const int tp = (nt + 63) / 64;
    const int jlo = min(nt, lane * tp), jhi = min(nt, jlo + tp);
    double tv = 0.0;
    for (int j = jlo; j < jhi; ++j) tv += tile_val(j);
    double incl = wave_scan_incl_d_dpp(tv);
    double total = lane_d(incl, 63);
    if (mode == 1) {
      rflags |= kRowResidual;
      if (total <= kFallbackMass) {  // residual mass too small: sample from p
        mode = 0;
        rflags |= kRowFallback;
        tv = 0.0;
        for (int j = jlo; j < jhi; ++j) tv += tile_val(j);
        incl = wave_scan_incl_d_dpp(tv);
        total = lane_d(incl, 63);
      }
    }
    const double tau = u_smp * total;
    // crossing tile: the smallest positive tile whose prefix reaches tau, else
    // the last positive tile; pb = the prefix before it, in the scan's order
    int jt = -1, jlast = -1;
    double pb = 0.0;
    {
      double c = incl - tv;  // exclusive prefix of the lane
      for (int j = jlo; j < jhi; ++j) {
        const double v = tile_val(j);
        if (v > 0.0) {
          jlast = j;
          if (jt < 0 && c + v >= tau) {
            jt = j;
            pb = c;
          }
        }
        c += v;
      }
    }
    const uint64_t hit = __ballot(jt >= 0);
    if (hit) {
      const int src = __ffsll(static_cast<unsigned long long>(hit)) - 1;
      jt = __shfl(jt, src);
      pb = __shfl(pb, src);
    } else {
      const int jl = wave_max_i(jlast);
      jt = jl >= 0 ? jl : 0;
      // prefix before the last positive tile
      double pl = 0.0;
      for (int j = jlo; j < jhi; ++j)
        if (j < jt) pl += tile_val(j);
      pb = wave_sum_d_dpp(pl);
    }
    // in-tile search: lane l of wave w computes the weights of elements
    // jt*kTile + 8 (64 w + l) + (0..7), so the block holds the tile in token
    // order (wave-major, then lane); each wave scans its quarter (DPP), the
    // waves' totals are added in order, and every lane finds the crossing
    // among its own eight (the block minimum of the lanes' finds).
    double w8[8];
    const int k0 = jt * kTile + 8 * (64 * wave + lane);
    {
      float lv[8], qv[8];
      load8f<LT, VEC>(lrow, V, k0, lv);
      load8qf<VEC>(mode == 1 ? qrow : nullptr, V, k0, qv);
      if (mode == 1 && onehot) {
#pragma unroll
        for (int k = 0; k < 8; ++k) qv[k] = k0 + k == hot ? 1.f : 0.f;
      }
#pragma unroll
      for (int g4 = 0; g4 < 8; g4 += kExpW) {
        double ar[kExpW], e[kExpW];
#pragma unroll
        for (int k = 0; k < kExpW; ++k) ar[k] = fma(static_cast<double>(masked(lv[g4 + k])), s, nms);
        exp2_negN<kExpW>(ar, tab, C, e);
#pragma unroll
        for (int k = 0; k < kExpW; ++k) {
          const double p = e[k] * iz;
          w8[g4 + k] = mode == 1 ? fmax(0.0, p - static_cast<double>(qv[g4 + k])) : p;
        }
      }
    }
    double s8 = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) s8 += w8[k];
    const double lincl = wave_scan_incl_d_dpp(s8);
    if (lane == 63) rs.part[wave] = lincl;
    if (tid == 0) {
      rs.cross = 0x7fffffff;
      rs.lastpos = -1;
    }
    __syncthreads();
    double c = 0.0;
    for (int w = 0; w < wave; ++w) c += rs.part[w];
    c += lincl - s8;
    const double tl = tau - pb;
    {
      int tok = -1, lastpos = -1;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        c += w8[k];
        if (w8[k] > 0.0) {
          lastpos = k0 + k;
          if (tok < 0 && c >= tl) tok = k0 + k;
        }
      }
      const uint64_t hit = __ballot(tok >= 0);
      if (hit && lane == __ffsll(static_cast<unsigned long long>(hit)) - 1) atomicMin(&rs.cross, tok);
      const int lp = wave_max_i(lastpos);
      if (lane == 0 && lp >= 0) atomicMax(&rs.lastpos, lp);
    }
    __syncthreads();
    if (wave != 0) return false;
    const int token = rs.cross != 0x7fffffff ? rs.cross : (rs.lastpos >= 0 ? rs.lastpos : jt * kTile);
    // ---- outputs of the request
    for (int i = lane; i <= g; i += 64) {
      int64_t o = -1;
      if (i < n) o = a.x[d0 + i];
      else if (i == n) o = token;
      sel.out[t0 + i] = o;
    }
    if (lane == 0) {
      sel.nacc[b] = n;
      a.ws[trow] = make_int2(token, static_cast<int>(rflags | (f0 & (kRowHead2 | kRowRowSelect | kRowTileSums))));
    }
    return false;
  }
}

// Lazy mode, per-request stage: for each request, the fp64 pass over its
// deciding row (its first open row) - per tile, the sum E_j of
// e_k = 2^((l_k - m) log2(e) / T) and the part of the residual sum that the
// certified Z interval [zlo, zhi] of the per-row pass already decides: P_j
// and Q_j, the sums of e_k and of q_k over the elements with e_k / Z > q_k for
// every Z in the interval (P_j = -1: an element left undecided) - then
// finish_row. One kernel template, five ways to launch it:
//   kReqFused:  one block per request does the whole row into LDS and the
//               finish (when the requests alone fill the chip's block slots);
//   kReqPass:   `slices` blocks per request, each a slice of the row's tiles,
//               the sums to device memory (plain stores: the finish is a
//               launch of its own);
//   kReqFinish: one block per request reads the sums into LDS and finishes;
//   kReqPassSplit: as kReqPass for slices of fewer tiles than the block's
//               waves (small batches): each tile's chunks spread over the
//               waves, their sums added in wave order;
//   kReqPassTail: as kReqPass when the slices take more than one round of
//               the chip's block slots: the slice's last (tiles mod 4) tiles
//               spread by chunks over the waves in the same way.
// A later open row (an undecided accept test that turned out accepted, rare)
// gets its whole pass from the finishing block alone, in LDS.
// HASQ = false (one-hot drafts, no q rows): every deciding row needs only its
// tile sums of e, and the kernel is built without the residual's per-element
// work (fewer registers, more waves per SIMD).
enum RequestMode { kReqFused = 0, kReqPass = 1, kReqFinish = 2, kReqPassSplit = 3, kReqPassTail = 4 };
// dynamic LDS of kReqPassSplit: per tile (at most 3) and wave, E, P, Q, then
// whether the wave's chunk left an element undecided
constexpr int kSplitParts = 3 * kPassWaves * 3;
constexpr size_t kSplitLds = kSplitParts * sizeof(double) + 3 * kPassWaves * sizeof(int);

// Blocks of the per-request kernel resident per compute unit, the register
// budget its pass builds are held to: three with bf16 logits and q rows (at
// most 168 VGPRs), two with fp32 logits (their raw chunks take twice the
// registers) or scalar loads, four without q rows (128 VGPRs).
template <typename LT, bool VEC, bool HASQ>
constexpr int request_blocks_per_cu() {
  return !HASQ ? 4 : ((VEC && sizeof(LT) == 2) ? 3 : 2);
}

template <typename LT, bool VEC, bool FILTER, bool HASQ, int MODE>
__global__ __launch_bounds__(kPassNT, (MODE == kReqFinish ? 1 : request_blocks_per_cu<LT, VEC, HASQ>())) void
request_kernel(ProbsArgs a, SelectArgs sel, PassArrays pa, int slices) {
  constexpr bool kSlicePass = MODE == kReqPass || MODE == kReqPassSplit || MODE == kReqPassTail;
  extern __shared__ double rbuf[];  // [nt] each: E_j, P_j, Q_j, W_j; then [nt] int: undecided tile list
  __shared__ BlockScratchT<kPassNT> sc;
  __shared__ ReqSharedT<kMemo<LT, VEC>> rs;
  __shared__ double tab[kExp2Tab];
  const int b = kSlicePass ? blockIdx.x / slices : blockIdx.x;
  const int sl = kSlicePass ? blockIdx.x % slices : 0;
  const int V = a.V, nt = (V + kTile - 1) / kTile;
  const int tid = threadIdx.x, wave = tid >> 6;
  int d0, d1;
  if (!request_range(a, b, d0, d1)) {
    if (!kSlicePass && tid == 0) sel.nacc[b] = 0;  // invalid offsets: nothing emitted
    return;
  }
  const int g = d1 - d0;
  const int64_t t0 = static_cast<int64_t>(d0) + b;
  const int64_t o = static_cast<int64_t>(b) * nt;
  // the finish's first tile sums (they do not depend on the open row): their
  // loads go out before the row search and the table
  double pf[3] = {0.0, 0.0, 0.0};
  if (MODE == kReqFinish && tid < nt) {
    pf[0] = pa.E[o + tid];
    pf[1] = pa.P[o + tid];
    pf[2] = pa.Q[o + tid];
  }
  exp2_table_init(tab);
  __syncthreads();  // (publishes tab)
  int n = first_open_row<kPassNT>(a.ws, t0, 0, g);
  const Exp2Consts C = exp2_consts_load();
  for (int guard = 0; guard <= g; ++guard) {  // at most g + 1 rows are taken
    const int64_t trow = t0 + n;
    if (static_cast<uint32_t>(a.ws[trow].y) & kRowTileSums) {
      // one-hot drafts with bf16 logits: the per-row pass kept the row's fp64
      // tile sums (relative to the m it recorded); no q, so P and Q are 0
      if constexpr (kSlicePass) return;
      const double* src = a.rsum + trow * static_cast<int64_t>(nt);
      for (int j = tid; j < nt; j += kPassNT) {
        rbuf[j] = src[j];
        rbuf[nt + j] = 0.0;
        rbuf[2 * nt + j] = 0.0;
      }
    } else if (MODE == kReqFinish && guard == 0) {
      for (int j = tid; j < nt; j += kPassNT) {
        const bool mine = j == tid;
        rbuf[j] = mine ? pf[0] : pa.E[o + j];
        rbuf[nt + j] = mine ? pf[1] : pa.P[o + j];
        rbuf[2 * nt + j] = mine ? pf[2] : pa.Q[o + j];
      }
    } else {
      const bool draft = n < g;
      const double4 st = a.rstat[trow];
      const double zhi = (st.y + st.z) * (1.0 + kZSlack), zlo = (st.y - st.z) * (1.0 - kZSlack);
      const LT* __restrict__ lrow = static_cast<const LT*>(a.logits) + trow * static_cast<int64_t>(V);
      const float* __restrict__ qrow =
          (HASQ && draft && a.q) ? a.q + static_cast<int64_t>(d0 + n) * V : nullptr;
      if constexpr (kSlicePass) {
        const int per = (nt + slices - 1) / slices;
        const int j0 = min(nt, sl * per), j1 = min(nt, j0 + per);
        if constexpr (MODE == kReqPassTail)
          fp64_row_pass<LT, VEC, FILTER, false, true>(lrow, qrow, V, nt, st.x, a.s64, zhi, zlo, qrow != nullptr, j0,
                                                      j1, kPassWaves, tab, C, pa.E + o, pa.P + o, pa.Q + o,
                                                      static_cast<float>(st.w), rs.memo,
                                                      reinterpret_cast<double(*)[4][3]>(rbuf),
                                                      reinterpret_cast<int(*)[4]>(rbuf + kSplitParts));
        else if constexpr (MODE == kReqPassSplit)  // (the host launches it when per < kPassWaves)
          fp64_row_pass<LT, VEC, FILTER, true>(lrow, qrow, V, nt, st.x, a.s64, zhi, zlo, qrow != nullptr, j0,
                                               min(j1, j0 + kPassWaves - 1), kPassWaves, tab, C, pa.E + o,
                                               pa.P + o, pa.Q + o, static_cast<float>(st.w), rs.memo,
                                               reinterpret_cast<double(*)[4][3]>(rbuf),
                                               reinterpret_cast<int(*)[4]>(rbuf + kSplitParts));
        else
          fp64_row_pass<LT, VEC, FILTER>(lrow, qrow, V, nt, st.x, a.s64, zhi, zlo, qrow != nullptr, j0 + wave, j1,
                                         kPassWaves, tab, C, pa.E + o, pa.P + o, pa.Q + o,
                                         static_cast<float>(st.w), rs.memo);
        return;
      } else {
        fp64_row_pass<LT, VEC, FILTER>(lrow, qrow, V, nt, st.x, a.s64, zhi, zlo, qrow != nullptr, wave, nt,
                                       kPassWaves, tab, C, rbuf, rbuf + nt, rbuf + 2 * nt, static_cast<float>(st.w),
                                       rs.memo);
      }
    }
    if constexpr (!kSlicePass) {
      __syncthreads();
      if (!finish_row<LT, VEC, FILTER>(a, sel, b, d0, d1, n, rbuf, sc, rs, tab, C)) return;
      n = first_open_row<kPassNT>(a.ws, t0, n + 1, g);
    }
  }
}

// ----------------------------------------------------------------------------
// greedy verification (argmax, lowest index on ties)

// Threads per row block of the greedy kernel: 16 waves per row, two rows per
// CU at a time (measured: 2-3% faster than 4 or 8 waves per row at
// B = 1024, gamma = 4, V = 128256; loading two tiles per step was slower).
constexpr int kGreedyNT = 1024;

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
__global__ __launch_bounds__(kGreedyNT) void greedy_rows_kernel(GreedyArgs a) {
  constexpr int kW = kGreedyNT / 64;
  __shared__ float bv[kW];
  __shared__ int bi[kW];
  using L = Lay<LT, VEC>;
  const int V = a.V;
  const int nt = (V + kTile - 1) / kTile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Task t = decode_task(blockIdx.x, a.cu, a.B, a.gamma, a.ndraft);
  if (!t.valid) return;
  const LT* __restrict__ lrow = static_cast<const LT*>(a.logits) + t.trow * static_cast<int64_t>(V);

  // each lane visits its elements in increasing index order, so a strict >
  // keeps the lowest index among equal values
  float best = -INFINITY;
  int bidx = 0x7fffffff;
  auto scan = [&](const float (&v)[kLaneElems], int base) {
#pragma unroll
    for (int k = 0; k < kLaneElems; ++k) {
      if (v[k] > best) {
        best = v[k];
        bidx = L::index(base, lane, k);
      }
    }
  };
  for (int j = wave; j < nt; j += kW) {
    float v[kLaneElems];
    load_logits<LT, VEC>(lrow, V, j * kTile, lane, v);
    scan(v, j * kTile);
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
    for (int w = 1; w < kW; ++w) argmax_combine(v, i, bv[w], bi[w]);
    if (i == 0x7fffffff) i = 0;  // every entry -inf: the first index
    int acc = 0;
    if (t.drow >= 0) acc = (a.x[t.drow] == static_cast<int64_t>(i)) ? 1 : 0;
    a.ws[t.trow] = make_int2(i, acc ? static_cast<int>(kRowAccepted) : 0);
  }
}

// ----------------------------------------------------------------------------
// self-check of the exp2 accuracy the fast path's error bound assumes

__global__ void zero_double_kernel(double* p) { *p = 0.0; }
__global__ void zero_u64_kernel(unsigned long long* p) { *p = 0ull; }

// Read-only stream (benchmark context): each step a block reads four
// consecutive 4 KB pieces (16-byte loads, four in flight per thread), then
// moves on by the grid's span; the 32-bit words are summed per thread, per
// wave, per block, then one atomic add per block. Two blocks per CU with
// block-contiguous steps measured 6.4 TB/s on 2 GiB; grid-stride single
// loads at 4-32 blocks per CU, 5.1-5.3 TB/s.
constexpr int kStreamNT = 256;
constexpr int kStreamBlocksPerCU = 2;
__global__ __launch_bounds__(kStreamNT) void stream_read_kernel(const uint4* __restrict__ src, size_t n,
                                                                unsigned long long* word_sum) {
  __shared__ unsigned long long part[kStreamNT / 64];
  unsigned long long acc = 0;
  auto add = [&](const uint4& v) {
    acc += static_cast<unsigned long long>(v.x) + v.y + static_cast<unsigned long long>(v.z) + v.w;
  };
  const size_t step = static_cast<size_t>(gridDim.x) * kStreamNT * 4;
  size_t j = static_cast<size_t>(blockIdx.x) * kStreamNT * 4 + threadIdx.x;
  for (; j + 3 * kStreamNT < n; j += step) {
    const uint4 a = src[j], b = src[j + kStreamNT], c = src[j + 2 * kStreamNT], d = src[j + 3 * kStreamNT];
    add(a);
    add(b);
    add(c);
    add(d);
  }
  for (int k = 0; k < 4; ++k)
    if (j + k * kStreamNT < n) add(src[j + k * kStreamNT]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long t = 0;
#pragma unroll
    for (int w = 0; w < kStreamNT / 64; ++w) t += part[w];
    atomicAdd(word_sum, t);
  }
}

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
// Workspace: row records, then the fp64 path's counters, list and per-tile
// arrays, then the lazy mode's per-row statistics. Every part starts on a
// 256-byte boundary.
struct WsLayout {
  size_t rec, count, list, done, etile, ptile, qtile, amb, rstat, mark, surv, total;
};
WsLayout ws_layout(int64_t rows, int V) {
  WsLayout l;
  const size_t nt = static_cast<size_t>((V + kTile - 1) / kTile);
  const size_t r = static_cast<size_t>(rows);
  // the counters first, at the same offset for every row count and
  // vocabulary size, so that whatever a call of another shape left elsewhere
  // never lands on them; then the records
  l.count = 0;  // list count at +0, finished rows at +64, task count at +128, first-launch count at +192
  l.rec = 256;
  l.list = l.rec + align256(r * sizeof(int2));
  l.done = l.list + align256(r * sizeof(ExactEntry));
  l.etile = l.done + align256(r * sizeof(int));
  l.ptile = l.etile + align256(r * nt * sizeof(double));
  l.qtile = l.ptile + align256(r * nt * sizeof(double));
  l.amb = l.qtile + align256(r * nt * sizeof(double));
  l.rstat = l.amb + align256(r * nt * sizeof(int));
  l.mark = l.rstat + align256(r * 4 * sizeof(double));
  l.surv = l.mark + align256(r * sizeof(int));
  l.total = l.surv + align256(r * sizeof(int2));
  return l;
}
size_t ws_bytes(int64_t rows) { return 256 + align256(static_cast<size_t>(rows) * sizeof(int2)); }

// Block sizes: the lazy first pass reads logits only and keeps more rows in
// flight with small blocks; the eager modes and the per-request second pass
// stream logits and q per row and prefer larger blocks (shorter per-row time).
constexpr int kRowsNTLazy = 512;
constexpr int kRaggedFirstMax = 4;  // ragged batches: most positions in the first lazy launch
constexpr int kLazyBlocksPerCU = 2;      // lazy per-row kernel: 512-thread blocks resident per CU
// Most mark reads (requests x blocks of the second launch) for which every
// block of the second lazy launch derives the task list itself: each block,
// the empty ones too, reads every request's mark, so beyond this the first
// launch's last block lists the tasks instead (measured: the headline batch,
// 256 x 1280, and the ragged one, 512 x 2307, gain about 1%; one-hot drafts
// at B = 1024, 1024 x 4096, lose 6%)
constexpr int64_t kSelfListMaxReads = int64_t{1} << 21;

// Compute units of the current device (cached per device; 256 if the query
// fails). Callers on several host threads may fill an entry at the same time:
// they store the same value, through atomics.
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Positions of the lazy mode's first launch: as many as fill the blocks the
// chip holds at once (at least one, at most every position launched
// position-major). A launch of one round gains nothing from stopping early;
// beyond one round, rows of later positions mostly start before the row that
// would make them unneeded has finished, and are read for nothing.
int lazy_first_positions(int B, int pm) {
  const int resident = kLazyBlocksPerCU * device_cus();
  const int p = B > 0 ? resident / B : pm;
  return max(1, min(p, pm));
}
constexpr int kRowsNTEager = 512;

// Benchmark diagnostics (spec_verify_profile_start / _stop): HIP event pairs
// recorded on the launch stream around the selected kernels. Host state.
constexpr int kProfileIds = 3;  // SV_PROFILE_ROWS, SV_PROFILE_REQUEST, SV_PROFILE_ROWS_FIRST
struct Profiler {
  uint32_t mask = 0;
  int capacity = 0;
  int every = 1;                           // record one call in `every`
  hipEvent_t* ev[kProfileIds] = {};       // per kernel id: [capacity][2] start, stop
  int used[kProfileIds] = {};
  int calls[kProfileIds] = {};            // calls seen since the start
  bool on[kProfileIds] = {};              // the current call is recorded
};
Profiler g_prof;

void prof_record(int id, int which, hipStream_t st) {
  if (!(g_prof.mask & (1u << id))) return;
  if (which == 0) g_prof.on[id] = (g_prof.calls[id]++ % g_prof.every) == 0 && g_prof.used[id] < g_prof.capacity;
  if (!g_prof.on[id]) return;
  (void)hipEventRecord(g_prof.ev[id][2 * g_prof.used[id] + which], st);
  if (which == 1) ++g_prof.used[id];
}

template <typename LT, bool VEC, int NT, bool EAGER, bool FILTER = false>
void launch_rows(const ProbsArgs& a, int64_t rows, size_t lds, hipStream_t st) {
  if constexpr (EAGER) {
    hipLaunchKernelGGL((probs_rows_kernel<LT, VEC, NT>), dim3(static_cast<unsigned>(rows)), dim3(NT), lds, st, a);
  } else {
    // positions [0, split) position-major, then the listed tasks: at most
    // every later row (every draft row of a ragged batch but one per request)
    const int split = lazy_first_positions(a.B, a.pm);
    const int64_t rest = a.cu ? static_cast<int64_t>(a.ndraft) : static_cast<int64_t>(a.B) * (a.pm - split);
    // the second launch lists for itself when every block's pass over the
    // marks stays cheap (without top-k / top-p)
    const bool self = !FILTER && static_cast<int64_t>(a.B) * rest <= kSelfListMaxReads;
    const int phase1 = rest > 0 ? (self ? 3 : 1) : 0;
    prof_record(SV_PROFILE_ROWS_FIRST, 0, st);
    if constexpr (kMemo<LT, VEC> && !FILTER) {
      if (a.q == nullptr) {  // one-hot drafts: rows summed in fp64 through the memo
        if (phase1 == 1)
          hipLaunchKernelGGL((lazy_rows_kernel<LT, VEC, NT, false, true, true>),
                             dim3(static_cast<unsigned>(a.B) * split), dim3(NT), lds, st, a, split, phase1);
        else
          hipLaunchKernelGGL((lazy_rows_kernel<LT, VEC, NT, false, false, true>),
                             dim3(static_cast<unsigned>(a.B) * split), dim3(NT), lds, st, a, split, phase1);
        prof_record(SV_PROFILE_ROWS_FIRST, 1, st);
        if (rest > 0)
          hipLaunchKernelGGL((lazy_rows_kernel<LT, VEC, NT, false, false, true>), dim3(static_cast<unsigned>(rest)),
                             dim3(NT), lds, st, a, split, self ? 4 : 2);
        return;
      }
    }
    if (phase1 == 1)
      hipLaunchKernelGGL((lazy_rows_kernel<LT, VEC, NT, FILTER, true>), dim3(static_cast<unsigned>(a.B) * split),
                         dim3(NT), lds, st, a, split, phase1);
    else
      hipLaunchKernelGGL((lazy_rows_kernel<LT, VEC, NT, FILTER, false>), dim3(static_cast<unsigned>(a.B) * split),
                         dim3(NT), lds, st, a, split, phase1);
    prof_record(SV_PROFILE_ROWS_FIRST, 1, st);
    if (rest > 0)  // (without top-k / top-p, rows that stop once an earlier position is a certain rejection)
      hipLaunchKernelGGL((lazy_rows_kernel<LT, VEC, NT, FILTER, false, false, !FILTER>),
                         dim3(static_cast<unsigned>(rest)), dim3(NT), lds, st, a, split, self ? 4 : 2);
  }
}

// The per-request stage of the lazy mode. Slices per request: the fewest
// reaching the shortest estimated span (rounds of the chip's resident block
// slots, request_blocks_per_cu per compute unit, times the tiles of one
// block), at most one per two tiles. One slice: the fused kernel (pass and
// finish in one block); more: the slice pass, then the finish.
int request_slices(int B, int nt, int per_cu) {
  const int64_t resident = static_cast<int64_t>(per_cu) * device_cus();
  const int most = max(1, min(min(kMaxSlices, nt / 2), 0x7fffffff / max(B, 1)));
  int best = 1;
  double best_span = 0.0;
  for (int sl = 1; sl <= most; ++sl) {
    const int64_t rounds = (static_cast<int64_t>(B) * sl + resident - 1) / resident;
    const double span = static_cast<double>(rounds) * static_cast<double>((nt + sl - 1) / sl);
    if (sl == 1 || span < best_span * 0.999) {
      best = sl;
      best_span = span;
    }
  }
  return best;
}

template <typename LT, bool VEC, bool FILTER, bool HASQ>
void launch_request_modes(const ProbsArgs& a, const SelectArgs& sel, const PassArrays& pa, size_t lds2,
                          hipStream_t st) {
  const int nt = (a.V + kTile - 1) / kTile;
  // (one-hot drafts with bf16 logits: the per-row pass kept the deciding
  // rows' tile sums, and one block per request only finishes)
  const int sl = (!HASQ && kMemo<LT, VEC>) ? 1 : request_slices(a.B, nt, request_blocks_per_cu<LT, VEC, HASQ>());
  if (sl == 1) {
    hipLaunchKernelGGL((request_kernel<LT, VEC, FILTER, HASQ, kReqFused>), dim3(static_cast<unsigned>(a.B)),
                       dim3(kPassNT), lds2, st, a, sel, pa, 1);
    return;
  }
  if ((nt + sl - 1) / sl < kPassWaves)  // slices of fewer tiles than waves
    hipLaunchKernelGGL((request_kernel<LT, VEC, FILTER, HASQ, kReqPassSplit>),
                       dim3(static_cast<unsigned>(a.B) * static_cast<unsigned>(sl)), dim3(kPassNT), kSplitLds, st, a,
                       sel, pa, sl);
  else if (static_cast<int64_t>(a.B) * sl > static_cast<int64_t>(request_blocks_per_cu<LT, VEC, HASQ>()) * device_cus())
    // more than one round of the chip's block slots: a block that ends late
    // delays the next round's start, so no wave of it takes a tile more
    hipLaunchKernelGGL((request_kernel<LT, VEC, FILTER, HASQ, kReqPassTail>),
                       dim3(static_cast<unsigned>(a.B) * static_cast<unsigned>(sl)), dim3(kPassNT), kSplitLds, st, a,
                       sel, pa, sl);
  else
    hipLaunchKernelGGL((request_kernel<LT, VEC, FILTER, HASQ, kReqPass>),
                       dim3(static_cast<unsigned>(a.B) * static_cast<unsigned>(sl)), dim3(kPassNT), 0, st, a, sel,
                       pa, sl);
  hipLaunchKernelGGL((request_kernel<LT, VEC, FILTER, HASQ, kReqFinish>), dim3(static_cast<unsigned>(a.B)),
                     dim3(kPassNT), lds2, st, a, sel, pa, 1);
}

template <typename LT, bool VEC, bool FILTER>
void launch_request(const ProbsArgs& a, const SelectArgs& sel, const PassArrays& pa, size_t lds2, hipStream_t st) {
  if (!FILTER && a.q == nullptr) launch_request_modes<LT, VEC, false, false>(a, sel, pa, lds2, st);
  else launch_request_modes<LT, VEC, FILTER, true>(a, sel, pa, lds2, st);
}

template <typename LT>
int launch_probs(const ProbsArgs& a, const ExactArgs& e, const SelectArgs& sel, int64_t rows, hipStream_t st) {
  const int nt = (a.V + kTile - 1) / kTile;
  const size_t lds = static_cast<size_t>(nt) * 4 * sizeof(float);
  const bool vec = aligned16(a.logits) && (static_cast<int64_t>(a.V) * sizeof(LT)) % 16 == 0 &&
                   (a.q == nullptr || (aligned16(a.q) && (a.V % 4) == 0));
  const bool lazy = (a.flags & kFlagLazy) != 0;
  const bool filter = (a.flags & kFlagFilter) != 0;
  prof_record(SV_PROFILE_ROWS, 0, st);
  if (vec) {
    if (filter) launch_rows<LT, true, kRowsNTLazy, false, true>(a, rows, lds, st);
    else if (lazy) launch_rows<LT, true, kRowsNTLazy, false>(a, rows, lds, st);
    else launch_rows<LT, true, kRowsNTEager, true>(a, rows, lds, st);
  } else {
    if (filter) launch_rows<LT, false, kRowsNTLazy, false, true>(a, rows, lds, st);
    else if (lazy) launch_rows<LT, false, kRowsNTLazy, false>(a, rows, lds, st);
    else launch_rows<LT, false, kRowsNTEager, true>(a, rows, lds, st);
  }
  prof_record(SV_PROFILE_ROWS, 1, st);
  if (lazy) {
    const size_t lds2 = static_cast<size_t>(nt) * (4 * sizeof(double) + sizeof(int));
    const PassArrays pa{e.etile, e.ptile, e.qtile};
    prof_record(SV_PROFILE_REQUEST, 0, st);
    if (vec) {
      if (filter) launch_request<LT, true, true>(a, sel, pa, lds2, st);
      else launch_request<LT, true, false>(a, sel, pa, lds2, st);
    } else {
      if (filter) launch_request<LT, false, true>(a, sel, pa, lds2, st);
      else launch_request<LT, false, false>(a, sel, pa, lds2, st);
    }
    prof_record(SV_PROFILE_REQUEST, 1, st);
    return 0;
  }
  hipLaunchKernelGGL((exact_kernel<LT>), dim3(kExactItemGrid), dim3(kNT), static_cast<size_t>(e.nt) * 4 * sizeof(double),
                     st, a, e, sel);
  return 0;
}

template <typename LT>
int launch_greedy(const GreedyArgs& a, int64_t rows, hipStream_t st) {
  const bool vec = aligned16(a.logits) && (static_cast<int64_t>(a.V) * sizeof(LT)) % 16 == 0;
  if (vec)
    hipLaunchKernelGGL((greedy_rows_kernel<LT, true>), dim3(static_cast<unsigned>(rows)), dim3(kGreedyNT), 0, st, a);
  else
    hipLaunchKernelGGL((greedy_rows_kernel<LT, false>), dim3(static_cast<unsigned>(rows)), dim3(kGreedyNT), 0, st, a);
  return 0;
}

int finish_launch() { return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH; }

// Shared implementation of the three entry points.
// Filter settings of the *_filtered entry points (filtered = false: none).
struct FilterArgs {
  bool filtered = false;
  int32_t top_k = 0;
  double top_p = 1.0;
};

int verify_common(const void* logits, int dtype, const float* q, const int64_t* x, const int32_t* cu,
                  const float* u, int32_t B, int32_t gamma, int32_t ndraft, int32_t V, double T, uint32_t flags,
                  int64_t* out, int32_t* nacc, float* stats, void* ws, size_t ws_size, void* stream,
                  bool greedy_only, FilterArgs fa = FilterArgs{}) {
  if (dtype != SV_DTYPE_F32 && dtype != SV_DTYPE_BF16) return SV_ERR_UNSUPPORTED;
  if (B < 0 || gamma < 0 || ndraft < 0 || V < 1) return SV_ERR_INVALID_ARGUMENT;
  if (V > SV_MAX_VOCAB) return SV_ERR_UNSUPPORTED;
  if (!(T >= 0.0) || !isfinite(T)) return SV_ERR_INVALID_ARGUMENT;
  // the fp32 scale log2(e) / T must be finite: T > 0 below about 4.2e-39 is
  // rejected (T = 0 is argmax decoding)
  if (T > 0.0 && !(1.4426950408889634 / T < static_cast<double>(FLT_MAX))) return SV_ERR_INVALID_ARGUMENT;
  if (fa.filtered && (!(T > 0.0) || !(fa.top_p > 0.0 && fa.top_p <= 1.0))) return SV_ERR_INVALID_ARGUMENT;
  if (flags & ~static_cast<uint32_t>(SV_FLAG_EXACT | SV_FLAG_ALL_RESIDUALS | SV_FLAG_EAGER))
    return SV_ERR_INVALID_ARGUMENT;
  if (stats && !(T > 0.0)) return SV_ERR_INVALID_ARGUMENT;
  const int64_t rows = static_cast<int64_t>(ndraft) + B;
  // (the first lazy launch of a ragged batch has up to kRaggedFirstMax blocks per request)
  if (rows + static_cast<int64_t>(kRaggedFirstMax) * B > 0x7fffffffLL) return SV_ERR_UNSUPPORTED;
  if (B == 0) return SV_OK;
  if (!logits || !out || !nacc) return SV_ERR_INVALID_ARGUMENT;
  if (ndraft > 0 && !x) return SV_ERR_INVALID_ARGUMENT;
  if (!greedy_only && T > 0.0 && !u) return SV_ERR_INVALID_ARGUMENT;
  if (fa.filtered && !q) return SV_ERR_INVALID_ARGUMENT;
  const bool greedy = greedy_only || T == 0.0;
  const WsLayout wl = ws_layout(rows, V);
  if (!ws || ws_size < (greedy ? ws_bytes(rows) : wl.total) || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return SV_ERR_WORKSPACE;
  (void)hipGetLastError();
  hipStream_t st = static_cast<hipStream_t>(stream);
  int2* wsp = reinterpret_cast<int2*>(static_cast<char*>(ws) + wl.rec);

  char* wsb = static_cast<char*>(ws);
  int* xcount = greedy ? nullptr : reinterpret_cast<int*>(wsb + wl.count);
  const SelectArgs sa{x, cu, wsp, out, nacc, B, gamma, ndraft};
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
    // lazy (default): no statistics, and not every row forced through the fp64 path
    const bool lazy = !(flags & (SV_FLAG_EAGER | SV_FLAG_ALL_RESIDUALS | SV_FLAG_EXACT)) && stats == nullptr;
    const bool filter = fa.filtered && ((fa.top_k > 0 && fa.top_k < V) || fa.top_p < 1.0);
    p.flags = flags | (lazy ? kFlagLazy : 0u) | (filter ? kFlagFilter : 0u);
    p.top_k = filter ? fa.top_k : 0;
    p.top_p = filter ? fa.top_p : 1.0;
    p.rstat = reinterpret_cast<double4*>(wsb + wl.rstat);
    p.mark = reinterpret_cast<int*>(wsb + wl.mark);
    p.rsum = reinterpret_cast<double*>(wsb + wl.etile);
    p.tasks = reinterpret_cast<int2*>(wsb + wl.surv);
    p.surv_n = reinterpret_cast<int*>(wsb + wl.count + 128);

    p.pm = cu ? kRaggedFirstMax : gamma + 1;
    p.cus = device_cus();
    p.xcount = xcount;
    p.xlist = reinterpret_cast<ExactEntry*>(wsb + wl.list);
    p.xdone = reinterpret_cast<int*>(wsb + wl.done);
    ExactArgs e;
    e.count = xcount;
    e.finished = reinterpret_cast<int*>(wsb + wl.count + 64);
    e.done = reinterpret_cast<int*>(wsb + wl.done);
    e.list = p.xlist;
    e.etile = reinterpret_cast<double*>(wsb + wl.etile);
    e.ptile = reinterpret_cast<double*>(wsb + wl.ptile);
    e.qtile = reinterpret_cast<double*>(wsb + wl.qtile);
    e.amb = reinterpret_cast<int*>(wsb + wl.amb);
    e.nt = (V + kTile - 1) / kTile;
    e.rows = static_cast<int>(rows);
    // the fp64 kernel ends with the per-request select
    if (dtype == SV_DTYPE_BF16) launch_probs<uint16_t>(p, e, sa, rows, st);
    else launch_probs<float>(p, e, sa, rows, st);
    return finish_launch();
  }
  int rc = finish_launch();
  if (rc != SV_OK) return rc;
  hipLaunchKernelGGL(select_kernel, dim3(static_cast<unsigned>((B + kSelectNT - 1) / kSelectNT)), dim3(kSelectNT),
                     0, st, sa);
  return finish_launch();
}

// ----------------------------------------------------------------------------
// fixed scratch of spec_verify_probs_noalloc (callers that cannot allocate)

// One copy per device, held until the process ends; its address on a device
// comes from hipGetSymbolAddress with that device current (the array's name
// is a host-side stand-in in host code and is never passed to a kernel).
constexpr size_t kScratchBytes = SV_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte blocks");

__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* __restrict__ p, size_t n) {
  const size_t step = static_cast<size_t>(gridDim.x) * 256;
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += step) p[i] = make_uint4(0, 0, 0, 0);
}

std::mutex g_scratch_mu;
void* g_scratch_dev[64];  // per device: the scratch's device address, once set up

// The scratch's device address on the current device. The first call on a
// device looks it up and enqueues a zero-fill of the whole scratch on `st`
// (the workspace contract: zero-filled before its first use; every completed
// call leaves it ready for the next).
int scratch_for_device(void** out, hipStream_t st);

}  // namespace

namespace {
int scratch_for_device(void** out, hipStream_t st) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SV_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return SV_ERR_LAUNCH;
    (void)hipGetLastError();
    hipLaunchKernelGGL(zero_fill_kernel, dim3(256), dim3(256), 0, st, static_cast<uint4*>(ptr), kScratchBytes / 16);
    if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return SV_OK;
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

int spec_verify_version(void) { return 3; }

double spec_verify_exp2_error_bound(void) { return kEpsExp; }

int spec_verify_profile_start(uint32_t kernel_mask, int32_t capacity) {
  if (capacity < 1 || capacity > (1 << 20) || (kernel_mask & ~7u) || !kernel_mask) return SV_ERR_INVALID_ARGUMENT;
  spec_verify_profile_stop(nullptr, nullptr);  // drops any earlier recording
  for (int id = 0; id < kProfileIds; ++id) {
    if (!(kernel_mask & (1u << id))) continue;
    g_prof.ev[id] = new hipEvent_t[2 * static_cast<size_t>(capacity)];
    for (int i = 0; i < 2 * capacity; ++i) {
      // timing only: no system-scope fence (cache writeback and invalidate) at
      // each record, which would otherwise slow the work around the events
      if (hipEventCreateWithFlags(&g_prof.ev[id][i], hipEventDisableSystemFence) != hipSuccess) {
        for (int k = 0; k < i; ++k) (void)hipEventDestroy(g_prof.ev[id][k]);
        delete[] g_prof.ev[id];
        g_prof.ev[id] = nullptr;
        spec_verify_profile_stop(nullptr, nullptr);
        return SV_ERR_LAUNCH;
      }
    }
  }
  g_prof.mask = kernel_mask;
  g_prof.capacity = capacity;
  g_prof.every = 1;
  for (int id = 0; id < kProfileIds; ++id) g_prof.used[id] = g_prof.calls[id] = 0;
  return SV_OK;
}

int spec_verify_profile_every(int32_t every) {
  if (every < 1) return SV_ERR_INVALID_ARGUMENT;
  g_prof.every = every;
  for (int id = 0; id < kProfileIds; ++id) g_prof.calls[id] = 0;
  return SV_OK;
}

int spec_verify_profile_stop(double* total_ms, int32_t* launches) {
  int rc = SV_OK;
  for (int id = 0; id < kProfileIds; ++id) {
    double sum = 0.0;
    int used = 0;
    if (g_prof.ev[id]) {
      used = g_prof.used[id];
      for (int i = 0; i < used; ++i) {
        float ms = 0.f;
        if (hipEventSynchronize(g_prof.ev[id][2 * i + 1]) != hipSuccess ||
            hipEventElapsedTime(&ms, g_prof.ev[id][2 * i], g_prof.ev[id][2 * i + 1]) != hipSuccess)
          rc = SV_ERR_LAUNCH;
        sum += ms;
      }
      for (int i = 0; i < 2 * g_prof.capacity; ++i) (void)hipEventDestroy(g_prof.ev[id][i]);
      delete[] g_prof.ev[id];
      g_prof.ev[id] = nullptr;
    }
    if (total_ms) total_ms[id] = sum;
    if (launches) launches[id] = used;
  }
  g_prof.mask = 0;
  g_prof.capacity = 0;
  g_prof.every = 1;
  for (int id = 0; id < kProfileIds; ++id) {
    g_prof.used[id] = g_prof.calls[id] = 0;
    g_prof.on[id] = false;
  }
  return rc;
}

int spec_verify_selftest_exp2(double* max_rel_err, void* stream) {
  if (!max_rel_err) return SV_ERR_INVALID_ARGUMENT;
  (void)hipGetLastError();
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(zero_double_kernel, dim3(1), dim3(1), 0, st, max_rel_err);
  hipLaunchKernelGGL(exp2_error_kernel, dim3(2048), dim3(kNT), 0, st, max_rel_err);
  return finish_launch();
}

int spec_verify_stream_read(const void* src, size_t bytes, unsigned long long* word_sum, void* stream) {
  if (!word_sum || (bytes % 16) != 0 || (bytes > 0 && (!src || !aligned16(src)))) return SV_ERR_INVALID_ARGUMENT;
  (void)hipGetLastError();
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(1), 0, st, word_sum);
  const size_t n = bytes / 16;
  if (n > 0) {
    const size_t want = (n + 4 * kStreamNT - 1) / (4 * kStreamNT);
    const size_t grid = want < static_cast<size_t>(kStreamBlocksPerCU) * device_cus()
                            ? want
                            : static_cast<size_t>(kStreamBlocksPerCU) * device_cus();
    hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<unsigned>(grid)), dim3(kStreamNT), 0, st,
                       static_cast<const uint4*>(src), n, word_sum);
  }
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

int spec_verify_probs_noalloc(const void* target_logits, int logits_dtype, const float* draft_probs,
                              const int64_t* draft_tokens, const float* uniforms, int32_t num_requests,
                              int32_t gamma, int32_t vocab_size, double temperature, uint32_t flags,
                              int64_t* out_tokens, int32_t* num_accepted, float* row_stats, void* stream) {
  if (num_requests < 0 || gamma < 0) return SV_ERR_INVALID_ARGUMENT;
  const int64_t nd = static_cast<int64_t>(num_requests) * gamma;
  if (nd > 0x7fffffffLL) return SV_ERR_UNSUPPORTED;
  if (vocab_size < 1 || vocab_size > SV_MAX_VOCAB) return SV_ERR_UNSUPPORTED;
  if (num_requests == 0) return SV_OK;
  if (ws_layout(nd + num_requests, vocab_size).total > kScratchBytes) return SV_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  const int rc = scratch_for_device(&ws, st);
  if (rc != SV_OK) return rc;
  return verify_common(target_logits, logits_dtype, draft_probs, draft_tokens, nullptr, uniforms, num_requests,
                       gamma, static_cast<int32_t>(nd), vocab_size, temperature, flags, out_tokens, num_accepted,
                       row_stats, ws, kScratchBytes, stream, false);
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

int spec_verify_probs_filtered(const void* target_logits, int logits_dtype, const float* draft_probs,
                               const int64_t* draft_tokens, const float* uniforms, int32_t num_requests,
                               int32_t gamma, int32_t vocab_size, double temperature, int32_t top_k, double top_p,
                               int64_t* out_tokens, int32_t* num_accepted, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (num_requests < 0 || gamma < 0) return SV_ERR_INVALID_ARGUMENT;
  const int64_t nd = static_cast<int64_t>(num_requests) * gamma;
  if (nd > 0x7fffffffLL) return SV_ERR_UNSUPPORTED;
  FilterArgs fa;
  fa.filtered = true;
  fa.top_k = top_k;
  fa.top_p = top_p;
  return verify_common(target_logits, logits_dtype, draft_probs, draft_tokens, nullptr, uniforms, num_requests,
                       gamma, static_cast<int32_t>(nd), vocab_size, temperature, 0u, out_tokens, num_accepted,
                       nullptr, workspace, workspace_bytes, stream, false, fa);
}

int spec_verify_ragged_filtered(const void* target_logits, int logits_dtype, const float* draft_probs,
                                const int64_t* draft_tokens, const int32_t* cu_num_draft_tokens,
                                const float* uniforms, int32_t num_requests, int32_t num_draft_tokens,
                                int32_t vocab_size, double temperature, int32_t top_k, double top_p,
                                int64_t* out_tokens, int32_t* num_accepted, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (num_requests > 0 && !cu_num_draft_tokens) return SV_ERR_INVALID_ARGUMENT;
  FilterArgs fa;
  fa.filtered = true;
  fa.top_k = top_k;
  fa.top_p = top_p;
  return verify_common(target_logits, logits_dtype, draft_probs, draft_tokens, cu_num_draft_tokens, uniforms,
                       num_requests, 0, num_draft_tokens, vocab_size, temperature, 0u, out_tokens, num_accepted,
                       nullptr, workspace, workspace_bytes, stream, false, fa);
}

}  // extern "C"
