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
// Kernel design (MI355X: 256 CUs, wave64, 160 KB LDS per CU, ~8 TB/s HBM):
//  * one 256-thread block per target row; draft rows are dispatched first and
//    bonus rows last, so the round-robin dispatch over the 8 XCDs spreads the
//    heavy rows (logits + q) evenly and the light rows fill the tail;
//  * a row is cut into 1024-element tiles; wave w streams tiles w, w+4, ...
//    with 16-byte loads, 16 elements per lane per tile; each tile leaves one
//    float (its sum) and, in the logits pass, its own max in LDS, so the
//    inverse-CDF search later re-reads a single tile;
//  * pass 1 reads the logits: tile max and sum of exp2((l - max_tile) s);
//    pass 2 (draft rows with q whose replacement is needed) re-reads the
//    logits (L2 / MALL resident by then) and reads q once: tile sums of
//    max(0, p - q);
//  * every row computes its replacement or bonus sample in parallel
//    (speculatively); a tiny select kernel then picks, per request, the
//    first rejection. A draft row whose own test passes skips its residual
//    (its sample can never be emitted) unless SV_FLAG_ALL_RESIDUALS is set.
//  * exactness: the fp32 fast path carries a rigorous error bound for Z, for
//    every prefix of the sampling CDF and for p(x). When the accept decision,
//    the 1e-8 fallback decision or the sampled token is not separated from its
//    threshold by twice the bound, the block recomputes the whole row in fp64
//    (exact_row). Results therefore equal exact arithmetic except within ~1e-15
//    relative of a decision boundary.
//
// All kernels read inputs only in bounds, whatever the device-side inputs
// hold (out-of-range tokens, bad offsets), and every loop has a fixed bound.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "specverify.h"

namespace {

constexpr int kNT = 256;                // threads per row block
constexpr int kWaves = kNT / 64;        // waves per row block
constexpr int kTile = 1024;             // elements per tile (one wave, 16 per lane)
constexpr int kLaneElems = kTile / 64;  // 16
constexpr int kSelectNT = 256;

// ----------------------------------------------------------------------------
// numerics constants of the fast path error bound
constexpr double kU = 5.9604644775390625e-08;   // 2^-24, fp32 unit roundoff
constexpr double kLn2 = 0.6931471805599453;
constexpr double kEpsExp = 2.384185791015625e-07;  // 2^-22 >= relative error of v_exp_f32
// per-term relative error of e_k ~ exp2(a_k): C1 |a_k| + C0 (see bound_terms)
constexpr double kC1 = 4.0 * kU * kLn2;
constexpr double kC0 = 2.0 * kEpsExp + 3.0 * kU;
constexpr double kSumErr = 26.0 * kU;   // fp32 summation chains (<= 24 levels) + slack
constexpr double kBoundA = 21.0;        // split point of the |a| bound (V <= 2^21)
constexpr double kSafety = 1.5;
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
  // element k (0..15) of `lane` in the tile starting at `base`
  __device__ static __forceinline__ int index(int base, int lane, int k) {
    return base + ((k / kE) * 64 + lane) * kE + (k % kE);
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
    if constexpr (VEC) {
#pragma unroll
      for (int h = 0; h < L::kE / 4; ++h) {
        if (i0 < V) {
          const float4 d = *reinterpret_cast<const float4*>(row + i0 + 4 * h);
          q[r * L::kE + 4 * h + 0] = d.x;
          q[r * L::kE + 4 * h + 1] = d.y;
          q[r * L::kE + 4 * h + 2] = d.z;
          q[r * L::kE + 4 * h + 3] = d.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) q[r * L::kE + 4 * h + e] = 0.f;
        }
      }
    } else {
      q[r] = i0 < V ? row[i0] : 0.f;
    }
  }
}

__device__ __forceinline__ float fexp2(float a) { return __builtin_amdgcn_exp2f(a); }

// ----------------------------------------------------------------------------
// reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

struct BlockScratch {
  double d[kNT];
  int i[kNT];
};

// Sum over the block in a fixed order; every thread gets the same value.
__device__ double block_sum(double v, BlockScratch& s) {
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

__device__ float block_max(float v, BlockScratch& s) {
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
__device__ void block_scan(double v, BlockScratch& s, double& excl, double& incl, double& total) {
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
  if (threadIdx.x == kNT - 1) s.d[0] = incl;
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
};

struct RowShared {
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

// Bound on sum_k |e~_k - e_k| in e-units (e_k relative to the row max), and
// with it the bound on |Z~ - Z|.
__device__ __forceinline__ double bound_terms(double z, int V) {
  // sum_k e_k |a_k| <= A Z + V A 2^-A ; per-term error C1 |a_k| + C0
  return kSafety * (kC1 * kBoundA * (1.01 * z + static_cast<double>(V) * 4.76837158203125e-07 /* 2^-21 */)
                    + kC0 * 1.01 * z + 1e-30);
}

template <typename LT>
__device__ __forceinline__ float logit_at(const LT* row, int64_t k) {
  return to_float(row[k]);
}

// Exact (fp64) recomputation of one row; all threads of the block call it.
template <typename LT>
__device__ void exact_row(const ProbsArgs& a, const Task& t, const LT* __restrict__ lrow,
                          const float* __restrict__ qrow, int64_t x, bool need_sample,
                          BlockScratch& sc, RowShared& sh) {
  const int V = a.V;
  const int tid = threadIdx.x;
  const int per = (V + kNT - 1) / kNT;
  const int lo = min(V, tid * per), hi = min(V, lo + per);
  const double m = static_cast<double>(sh.m);
  const double s = a.s64;
  const bool is_draft = t.drow >= 0;
  const bool x_ok = is_draft && x >= 0 && x < V;
  const bool onehot = is_draft && qrow == nullptr;

  double zl = 0.0;
  for (int k = lo; k < hi; ++k) zl += exp2((static_cast<double>(logit_at(lrow, k)) - m) * s);
  const double Z = block_sum(zl, sc);

  double px = 0.0;
  bool accepted = false;
  if (is_draft) {
    if (x_ok) px = exp2((static_cast<double>(logit_at(lrow, x)) - m) * s) / Z;
    const double qx = onehot ? 1.0 : (x_ok ? static_cast<double>(qrow[x]) : 0.0);
    accepted = x_ok && px > 0.0 && static_cast<double>(a.u[t.trow]) * qx <= px;
  }

  uint32_t flags = kRowExact | (accepted ? kRowAccepted : 0u);
  int token = -1;
  double rmass = 1.0;
  const bool sample = !is_draft || !accepted || need_sample;
  if (sample) {
    // weight mode: 0 = p (bonus / fallback), 1 = max(0, p - q), 2 = p without x (one-hot)
    int mode = is_draft ? (onehot ? 2 : 1) : 0;
    auto weight = [&](int k) -> double {
      const double p = exp2((static_cast<double>(logit_at(lrow, k)) - m) * s) / Z;
      if (mode == 1) return fmax(0.0, p - static_cast<double>(qrow[k]));
      if (mode == 2) return (x_ok && k == x) ? fmax(0.0, p - 1.0) : p;
      return p;
    };
    double wl = 0.0;
    for (int k = lo; k < hi; ++k) wl += weight(k);
    double excl, incl, total;
    block_scan(wl, sc, excl, incl, total);
    if (mode != 0) {
      rmass = total;
      if (total <= kFallbackMass) {
        mode = 0;
        flags |= kRowFallback;
        wl = 0.0;
        for (int k = lo; k < hi; ++k) wl += weight(k);
        block_scan(wl, sc, excl, incl, total);
      }
    }
    flags |= is_draft ? kRowResidual : 0u;
    const double tau = static_cast<double>(a.u[t.srow]) * total;
    // Smallest k with C_k >= tau. The tree scan does not make incl_t equal
    // excl_t + v_t bit for bit, so every thread whose range starts below tau
    // walks it; only positive weights can be chosen; the smallest crossing
    // index wins, else the last positive weight below tau (tau at the very
    // top of the CDF, within rounding).
    if (tid == 0) {
      sh.cross = 0x7fffffff;
      sh.lastpos = -1;
    }
    __syncthreads();
    if (tau > 0.0 && excl < tau) {
      int tok = -1, lastpos = -1;
      double c = 0.0;
      for (int k = lo; k < hi; ++k) {
        const double w = weight(k);
        c += w;
        if (w > 0.0) {
          lastpos = k;
          if (excl + c >= tau) {
            tok = k;
            break;
          }
        }
      }
      if (tok >= 0) atomicMin(&sh.cross, tok);
      if (lastpos >= 0) atomicMax(&sh.lastpos, lastpos);
    }
    __syncthreads();
    token = sh.cross != 0x7fffffff ? sh.cross : (sh.lastpos >= 0 ? sh.lastpos : 0);
  }
  if (tid == 0) {
    a.ws[t.trow] = make_int2(token, static_cast<int>(flags));
    if (a.stats) {
      float* st = a.stats + t.trow * 4;
      st[0] = static_cast<float>(m / a.temperature);
      st[1] = static_cast<float>(log(Z));
      st[2] = is_draft ? static_cast<float>(px) : NAN;
      st[3] = static_cast<float>(rmass);
    }
  }
  __syncthreads();
}

template <typename LT, bool VEC>
__global__ __launch_bounds__(kNT) void probs_rows_kernel(ProbsArgs a) {
  extern __shared__ float dyn[];
  __shared__ BlockScratch sc;
  __shared__ RowShared sh;
  using L = Lay<LT, VEC>;

  const int V = a.V;
  const int nt = (V + kTile - 1) / kTile;
  float* S = dyn;        // tile sums of exp2((l - M_j) s), local units
  float* M = dyn + nt;   // tile max
  float* W = dyn + 2 * nt;  // tile sums of max(0, p - q)
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

  // ---------------- pass 1: tile max and tile sum of exp2((l - M_j) s)
  for (int j = wave; j < nt; j += kWaves) {
    const int base = j * kTile;
    float v[kLaneElems];
    load_logits<LT, VEC>(lrow, V, base, lane, v);
    float mx = v[0];
#pragma unroll
    for (int k = 1; k < kLaneElems; ++k) mx = fmaxf(mx, v[k]);
    mx = wave_max(mx);
    float es = 0.f;
    if (mx != -INFINITY) {
      if (xmask >= base && xmask < base + kTile) {
#pragma unroll
        for (int k = 0; k < kLaneElems; ++k) {
          const float e = fexp2((v[k] - mx) * s);
          es += (L::index(base, lane, k) == xmask) ? 0.f : e;
        }
      } else {
#pragma unroll
        for (int k = 0; k < kLaneElems; ++k) es += fexp2((v[k] - mx) * s);
      }
    }
    es = wave_sum(es);
    if (lane == 0) {
      S[j] = es;
      M[j] = mx;
    }
  }
  __syncthreads();

  // row max and Z (e-units relative to the row max)
  float mloc = -INFINITY;
  for (int j = tid; j < nt; j += kNT) mloc = fmaxf(mloc, M[j]);
  const float m = block_max(mloc, sc);
  double zl = 0.0;
  for (int j = tid; j < nt; j += kNT) {
    const float f = M[j] == -INFINITY ? 0.f : fexp2((M[j] - m) * s);
    zl += static_cast<double>(S[j] * f);
  }
  float ex = 0.f, lx = -INFINITY;
  if (x_ok) {
    lx = to_float(lrow[x]);
    ex = fexp2((lx - m) * s);
  }
  if (tid == 0 && xmask >= 0) zl += static_cast<double>(ex);  // one-hot rows left x out of S
  const double Z = block_sum(zl, sc);
  const double bt = bound_terms(Z, V);
  const double dZ = bt + kSumErr * Z;   // |Z~ - Z|
  const double relZ = dZ / Z;

  // ---------------- accept test of a draft row (fp64 p(x), certified)
  if (tid == 0) {
    sh.m = m;
    sh.z = Z;
    int accepted = 0, uncertain = 0;
    double px = 0.0;
    if (is_draft) {
      if (x_ok) px = exp2((static_cast<double>(lx) - static_cast<double>(m)) * a.s64) / Z;
      const double qx = onehot ? 1.0 : (x_ok ? static_cast<double>(qrow[x]) : 0.0);
      const double lhs = static_cast<double>(a.u[t.trow]) * qx;
      accepted = (x_ok && px > 0.0 && lhs <= px) ? 1 : 0;
      if (x_ok) {
        const double dpx = kSafety * (px * relZ * 1.01) + 1e-300;
        if (fabs(lhs - px) <= 2.0 * dpx || px < 1e-30 || !(Z > 0.0)) uncertain = 1;
      }
    }
    if (!(Z > 0.0) || m == -INFINITY || (a.flags & SV_FLAG_EXACT)) uncertain = 1;
    sh.px = px;
    sh.accepted = accepted;
    sh.uncertain = uncertain;
  }
  __syncthreads();
  const bool accepted = sh.accepted != 0;
  if (sh.uncertain) {
    exact_row<LT>(a, t, lrow, qrow, x, all_res, sc, sh);
    return;
  }
  const bool sample = !is_draft || !accepted || all_res;
  if (!sample) {
    if (tid == 0) a.ws[t.trow] = make_int2(-1, static_cast<int>(kRowAccepted));
    return;
  }

  // ---------------- pass 2: residual tile sums (draft rows with q)
  const bool mode_w = qrow != nullptr;
  const float izr = static_cast<float>(1.0 / Z);
  if (mode_w) {
    for (int j = wave; j < nt; j += kWaves) {
      const int base = j * kTile;
      float v[kLaneElems], q[kLaneElems];
      load_logits<LT, VEC>(lrow, V, base, lane, v);
      load_q<LT, VEC>(qrow, V, base, lane, q);
      float ws = 0.f;
#pragma unroll
      for (int k = 0; k < kLaneElems; ++k) {
        const float p = fexp2((v[k] - m) * s) * izr;
        ws += fmaxf(p - q[k], 0.f);
      }
      ws = wave_sum(ws);
      if (lane == 0) W[j] = ws;
    }
    __syncthreads();
  }

  // ---------------- tile-level CDF: prefix over tiles in token order
  // value of tile j in global units: W[j] (p-units) or S[j] * f_j (e-units)
  auto tile_val = [&](int j) -> double {
    if (mode_w) return static_cast<double>(W[j]);
    const float f = M[j] == -INFINITY ? 0.f : fexp2((M[j] - m) * s);
    return static_cast<double>(S[j] * f);
  };
  const int tper = (nt + kNT - 1) / kNT;
  const int tlo = min(nt, tid * tper), thi = min(nt, tlo + tper);
  double tv = 0.0;
  for (int j = tlo; j < thi; ++j) tv += tile_val(j);
  double excl, incl, total;
  block_scan(tv, sc, excl, incl, total);

  // error bound of every CDF prefix (same units as total)
  double dC, dcheck = 0.0;
  bool uncertain = false;
  if (mode_w) {
    const double dp = (bt / Z + relZ + 2.0 * kU) * 1.01;   // sum_k |p~_k - p_k|
    dC = kSafety * (dp + kU + kSumErr * total);
    if (total <= kFallbackMass + 2.0 * dC) uncertain = true;
  } else {
    dC = kSafety * (bt + kSumErr * Z);
    if (onehot) {
      dcheck = dC / Z + relZ;
      if (total / Z <= kFallbackMass + 2.0 * kSafety * dcheck) uncertain = true;
    }
  }
  const double tau = static_cast<double>(a.u[t.srow]) * total;
  if (tid == 0) {
    sh.found = 0;
    sh.uncertain = uncertain ? 1 : 0;
  }
  __syncthreads();
  if (!uncertain && tau > 0.0 && excl < tau && incl >= tau) {
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
    exact_row<LT>(a, t, lrow, qrow, x, all_res, sc, sh);
    return;
  }

  // ---------------- in-tile search: 4 consecutive elements per thread
  const int jt = sh.tile;
  const double pb = sh.p_before;
  const int base = jt * kTile + 4 * tid;
  float unit = 1.f;   // global units per local unit
  float mref = m;     // exponent reference of the local weights
  if (!mode_w) {
    mref = M[jt];
    unit = fexp2((M[jt] - m) * s);
  }
  float w4[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int k = base + e;
    float w = 0.f;
    if (k < V) {
      const float l = to_float(lrow[k]);
      const float ek = fexp2((l - mref) * s);
      if (mode_w) w = fmaxf(ek * izr - qrow[k], 0.f);
      else w = (k == xmask) ? 0.f : ek;
    }
    w4[e] = w;
  }
  const float tsum = ((w4[0] + w4[1]) + w4[2]) + w4[3];
  const double tau_loc = (tau - pb) / static_cast<double>(unit);
  double e2, i2, tot2;
  block_scan(static_cast<double>(tsum), sc, e2, i2, tot2);
  if (tid == 0) sh.found = 0;
  __syncthreads();
  if (e2 < tau_loc && i2 >= tau_loc) {
    float cl = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float prev = cl;
      cl += w4[e];
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
  bool ok = sh.found != 0;
  if (ok) {
    // unit conversion adds a relative rounding of ~3u to the local prefix
    const double d2 = 2.0 * (dC + 4.0 * kU * total);
    ok = (tau - sh.c_lo) > d2 && (sh.c_hi - tau) > d2;
  }
  if (!ok) {
    exact_row<LT>(a, t, lrow, qrow, x, all_res, sc, sh);
    return;
  }
  if (tid == 0) {
    uint32_t fl = (accepted ? kRowAccepted : 0u) | (is_draft ? kRowResidual : 0u);
    a.ws[t.trow] = make_int2(sh.token, static_cast<int>(fl));
    if (want_stats) {
      float* st = a.stats + t.trow * 4;
      st[0] = static_cast<float>(static_cast<double>(m) / a.temperature);
      st[1] = static_cast<float>(log(Z));
      st[2] = is_draft ? static_cast<float>(sh.px) : NAN;
      st[3] = is_draft ? static_cast<float>(mode_w ? total : total / Z) : 1.f;
    }
  }
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
  int B, gamma, ndraft;
};

__global__ __launch_bounds__(kSelectNT) void select_kernel(SelectArgs a) {
  const int b = blockIdx.x * kSelectNT + threadIdx.x;
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
// host side

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t ws_bytes(int64_t rows) {
  const size_t b = static_cast<size_t>(rows) * sizeof(int2);
  return (b + 255) & ~static_cast<size_t>(255);
}

template <typename LT>
int launch_probs(const ProbsArgs& a, int64_t rows, hipStream_t st) {
  const int nt = (a.V + kTile - 1) / kTile;
  const size_t lds = static_cast<size_t>(nt) * 3 * sizeof(float);
  const bool vec = aligned16(a.logits) && (static_cast<int64_t>(a.V) * sizeof(LT)) % 16 == 0 &&
                   (a.q == nullptr || (aligned16(a.q) && (a.V % 4) == 0));
  if (vec)
    hipLaunchKernelGGL((probs_rows_kernel<LT, true>), dim3(static_cast<unsigned>(rows)), dim3(kNT), lds, st, a);
  else
    hipLaunchKernelGGL((probs_rows_kernel<LT, false>), dim3(static_cast<unsigned>(rows)), dim3(kNT), lds, st, a);
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
  if (flags & ~static_cast<uint32_t>(SV_FLAG_EXACT | SV_FLAG_ALL_RESIDUALS)) return SV_ERR_INVALID_ARGUMENT;
  if (stats && !(T > 0.0)) return SV_ERR_INVALID_ARGUMENT;
  const int64_t rows = static_cast<int64_t>(ndraft) + B;
  if (rows > 0x7fffffffLL) return SV_ERR_UNSUPPORTED;
  if (B == 0) return SV_OK;
  if (!logits || !out || !nacc) return SV_ERR_INVALID_ARGUMENT;
  if (ndraft > 0 && !x) return SV_ERR_INVALID_ARGUMENT;
  if (!greedy_only && T > 0.0 && !u) return SV_ERR_INVALID_ARGUMENT;
  if (!ws || ws_size < ws_bytes(rows) || (reinterpret_cast<uintptr_t>(ws) & 7u)) return SV_ERR_WORKSPACE;
  (void)hipGetLastError();
  hipStream_t st = static_cast<hipStream_t>(stream);
  int2* wsp = static_cast<int2*>(ws);

  if (greedy_only || T == 0.0) {
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
    p.flags = flags;
    if (dtype == SV_DTYPE_BF16) launch_probs<uint16_t>(p, rows, st);
    else launch_probs<float>(p, rows, st);
  }
  int rc = finish_launch();
  if (rc != SV_OK) return rc;
  SelectArgs sa{x, cu, wsp, out, nacc, B, gamma, ndraft};
  hipLaunchKernelGGL(select_kernel, dim3(static_cast<unsigned>((B + kSelectNT - 1) / kSelectNT)), dim3(kSelectNT),
                     0, st, sa);
  return finish_launch();
}

}  // namespace

extern "C" {

size_t spec_verify_workspace_size(int64_t num_target_rows) {
  if (num_target_rows < 0) return 0;
  return ws_bytes(num_target_rows);
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
