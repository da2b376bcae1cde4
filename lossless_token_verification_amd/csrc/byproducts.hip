// By-products of a verification call.
//
// Row entropy: the chunk partials (c_i, S_i) and T_i of a row merge to a common
// reference c = max c_i as S = sum 2^(c_i - c) S_i and
// T = sum 2^(c_i - c) (T_i + (c_i - c) S_i); the entropy in nats is then
// ln S - ln 2 * T / S, since ln P_v = (y_v ln 2) - ln S for y_v = l_v s - c.
// The entropy of the draft's distribution is the uncertainty signal of
// entropy-driven adaptive draft lengths ("Optimierung der
// Inferenzgeschwindigkeit von Sprachmodellen durch spekulative Dekodierung",
// mind-verse.de, paragraphs on SVIP).
//
// Outcome export: for a tested position with draft distribution q and target
// p, beta = sum_v min(p_v, q_v) is the probability that the standard rule
// accepts there, and r = max(0, p - q) is the residual the correction is drawn
// from ("Speculative Speculative Decoding", gist.science 2603.03251, section
// 3.B); r_v is the probability of rejecting there and emitting v.  The
// largest r_v are the likely outcomes a speculation cache prepares for (same
// summary, section 2 items 1-2 and section 3.A).
#include "sv_args.h"

namespace sv {

namespace {

__device__ __forceinline__ bool greedy_tau(float tau) { return !(tau > 0.0f) || !(tau < INFINITY); }

__device__ __forceinline__ int row_exit(const ByArgs& a, int row) {
  int e = 0;
  if (row >= a.exit_row0[1]) e = 1;
  if (a.hier && row >= a.exit_row0[2]) e = 2;
  return e;
}

// Merged (c, S) of a sampled row; S = 0 when the row has no finite logit.
__device__ inline void merge_row(const Partial* p, int nc, float& c, double& S) {
  c = -INFINITY;
  for (int i = 0; i < nc; ++i)
    if (p[i].S > 0.0) c = fmaxf(c, p[i].key);
  S = 0.0;
  for (int i = 0; i < nc; ++i)
    if (p[i].S > 0.0) S += p[i].S * exp2(static_cast<double>(p[i].key) - static_cast<double>(c));
}

// Merged greedy argmax of a row: largest key, lowest index among equals
// (chunks are in index order and each holds its lowest maximising index).
__device__ inline int merge_argmax(const Partial* p, int nc) {
  float m = -INFINITY;
  int idx = 0x7fffffff;
  for (int i = 0; i < nc; ++i)
    if (p[i].amax != 0x7fffffff && (idx == 0x7fffffff || p[i].key > m)) {
      m = p[i].key;
      idx = p[i].amax;
    }
  return idx;
}

__global__ __launch_bounds__(kThreads) void entropy_kernel(ByArgs a) {
  const int row = blockIdx.x * kThreads + threadIdx.x;
  if (row >= a.rows) return;
  const int e = row_exit(a, row);
  const int b = (row - a.exit_row0[e]) / a.exit_pos[e];
  const float tau = a.temperature ? a.temperature[b] : 1.0f;
  if (greedy_tau(tau)) {
    a.entropy[row] = 0.0f;   // a one-hot
    return;
  }
  const Partial* p = a.partials + static_cast<int64_t>(row) * a.nc;
  const double* t = a.tpart + static_cast<int64_t>(row) * a.nc;
  float c;
  double S;
  merge_row(p, a.nc, c, S);
  double T = 0.0;
  for (int i = 0; i < a.nc; ++i)
    if (p[i].S > 0.0) {
      const double d = static_cast<double>(p[i].key) - static_cast<double>(c);
      T += (t[i] + d * p[i].S) * exp2(d);
    }
  const double H = S > 0.0 ? log(S) - 0.69314718055994530942 * T / S : NAN;
  a.entropy[row] = static_cast<float>(H);
}

// Per-thread lists of the largest residuals (r, v), largest first; elements
// arrive in increasing v, so strict comparisons keep equal r in index order.
//
// TopList keeps kTopM entries: exact, but its insertion is a chain of
// compare-swaps that a wavefront runs whenever any lane inserts.  Top2 keeps
// two entries branch-free, plus `drop`, the largest value it ever left out;
// it takes elements four at a time and lists only each group's largest.  The
// workgroup's top m taken from the Top2 lists is the chunk's exact top m
// whenever every value left out lies strictly below the m-th selected one
// (otherwise the chunk is scanned again with TopList): a rare event, since it
// needs two of the chunk's m largest residuals in one group of four, or three
// in one thread.
struct TopList {
  float val[kTopM];
  int32_t idx[kTopM];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int i = 0; i < kTopM; ++i) {
      val[i] = 0.0f;
      idx[i] = -1;
    }
  }
  __device__ __forceinline__ void push(float r, int v) {
    if (!(r > val[kTopM - 1])) return;
    val[kTopM - 1] = r;
    idx[kTopM - 1] = v;
#pragma unroll
    for (int i = kTopM - 1; i > 0; --i) {
      if (val[i] > val[i - 1]) {
        const float tv = val[i];
        val[i] = val[i - 1];
        val[i - 1] = tv;
        const int ti = idx[i];
        idx[i] = idx[i - 1];
        idx[i - 1] = ti;
      }
    }
  }
  // four consecutive elements (increasing v), each pushed exactly
  __device__ __forceinline__ void push4(const float (&r)[4], int v0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) push(r[q], v0 + q);
  }
  __device__ __forceinline__ float head_val() const { return val[0]; }
  __device__ __forceinline__ int head_idx() const { return idx[0]; }
  __device__ __forceinline__ void pop() {
#pragma unroll
    for (int i = 0; i < kTopM - 1; ++i) {
      val[i] = val[i + 1];
      idx[i] = idx[i + 1];
    }
    val[kTopM - 1] = 0.0f;
    idx[kTopM - 1] = -1;
  }
  __device__ __forceinline__ float dropped() const { return 0.0f; }
};

// Residuals and probabilities here are non-negative floats (or +0), whose
// bit patterns order like unsigned integers: min runs as an integer
// operation, exact and free of the float min NaN handling.
__device__ __forceinline__ float uminf(float a, float b) {
  return __uint_as_float(min(__float_as_uint(a), __float_as_uint(b)));
}

struct Top2 {
  uint32_t v1, v2, drop;   // float bits of non-negative values
  int32_t i1, i2;
  __device__ __forceinline__ void init() {
    v1 = v2 = drop = 0u;
    i1 = i2 = -1;
  }
  __device__ __forceinline__ void push(float rf, int v) {
    const uint32_t r = __float_as_uint(rf);
    const bool g1 = r > v1, g2 = r > v2;
    drop = max(drop, min(r, v2));   // the value that leaves (or never enters)
    i2 = g1 ? i1 : (g2 ? v : i2);
    v2 = max(v2, min(r, v1));
    i1 = g1 ? v : i1;
    v1 = max(v1, r);
  }
  // Four consecutive elements (increasing v): only the group's largest (the
  // lowest index among equals) enters the list; the second largest of the
  // group, the largest of the three left out, joins `drop`.
  __device__ __forceinline__ void push4(const float (&rf)[4], int v0) {
    const uint32_t a = __float_as_uint(rf[0]), b = __float_as_uint(rf[1]);
    const uint32_t c = __float_as_uint(rf[2]), d = __float_as_uint(rf[3]);
    const bool gb = b > a, gd = d > c;
    const uint32_t m_ab = max(a, b), m_cd = max(c, d);
    const int i_ab = gb ? 1 : 0, i_cd = gd ? 3 : 2;
    const bool g2 = m_cd > m_ab;
    const uint32_t second = max(max(min(a, b), min(c, d)), min(m_ab, m_cd));
    drop = max(drop, second);
    push(__uint_as_float(max(m_ab, m_cd)), v0 + (g2 ? i_cd : i_ab));
  }
  __device__ __forceinline__ float head_val() const { return __uint_as_float(v1); }
  __device__ __forceinline__ int head_idx() const { return i1; }
  __device__ __forceinline__ void pop() {
    v1 = v2;
    i1 = i2;
    v2 = 0u;
    i2 = -1;
  }
  __device__ __forceinline__ float dropped() const { return __uint_as_float(drop); }
};

// (va, ia) ranks before (vb, ib): larger value, then lower index; empty
// entries (index -1, value 0) rank last.
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
  if (ia < 0) return false;
  if (ib < 0) return true;
  return va > vb || (va == vb && ia < ib);
}

struct PairShared {
  float key[kWaves];
  int32_t idx[kWaves];
  double sum[kWaves];
  float c[3];     // per row: the reference c of the merged statistics
  float inv[3];   // and 1 / S
};

__device__ inline float block_max(float v, PairShared& sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  v = wave_max(v);
  if (lane == 0) sh.key[wave] = v;
  __syncthreads();
  float m = sh.key[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) m = fmaxf(m, sh.key[w]);
  __syncthreads();
  return m;
}

// Workgroup top-m of the threads' lists: m rounds of a (value, index) arg-max;
// the winning thread drops its head.  Thread 0 writes the chunk's list (padded
// to kTopM).  Returns true when the list is the chunk's exact top m: no
// thread discarded a value that could belong to it.
template <class List>
__device__ inline bool block_top(List& L, int m, PairPart* out, PairShared& sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  float last = 0.0f;
  int count = 0;
  for (int r = 0; r < m; ++r) {
    float bv = L.head_val();
    int bi = L.head_idx();
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (ranks_before(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == 0) {
      sh.key[wave] = bv;
      sh.idx[wave] = bi;
    }
    __syncthreads();
    bv = sh.key[0];
    bi = sh.idx[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
      if (ranks_before(sh.key[w], sh.idx[w], bv, bi)) {
        bv = sh.key[w];
        bi = sh.idx[w];
      }
    __syncthreads();
    if (bi >= 0 && L.head_idx() == bi) L.pop();
    if (threadIdx.x == 0) {
      out->mass[r] = bi >= 0 ? bv : 0.0f;
      out->tok[r] = bi;
    }
    if (bi >= 0) {
      last = bv;
      ++count;
    }
  }
  if (threadIdx.x == 0)
    for (int q = m; q < kTopM; ++q) {
      out->mass[q] = 0.0f;
      out->tok[q] = -1;
    }
  const float dropped = block_max(L.dropped(), sh);
  return count == m ? dropped < last : !(dropped > 0.0f);
}

__device__ inline double block_sum(double v, PairShared& sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  v = wave_sum(v);
  if (lane == 0) sh.sum[wave] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) s += sh.sum[w];
  __syncthreads();
  return s;
}

// One pass over elements [e0, e1) of the rows q = base[0], p = base[1],
// f = base[2] (absent rows alias p): p_v = 2^(l_v s - c) / S per row; stage 0
// (HAS0) adds min(p, q) to B0 and offers p - min(p, q) to L0, stage 1 (HAS1)
// likewise for (f, p).  Each thread visits its elements in increasing v, four
// consecutive ones at a time where the rows allow 16-byte loads.
template <int DT, bool HAS0, bool HAS1, class List>
__device__ inline void pair_scan(const char* const* base, int e0, int e1, float s,
                                 const PairShared& sh, List& L0, List& L1, double& B0,
                                 double& B1) {
  constexpr int VPE = DT == 1 ? 8 : 4;
  const int tid = threadIdx.x;
  const float cq = sh.c[0], cp = sh.c[1], cf = sh.c[2];
  const float iq = sh.inv[0], ip = sh.inv[1], i_f = sh.inv[2];
  float b0 = 0.0f, b1 = 0.0f;
  // residuals of one element for both stages
  auto elem = [&](float xq, float xp, float xf, float& r0, float& r1) {
    // no contraction: p - min(p, q) must see the same rounded p as the min,
    // so that it is exactly 0 (never negative) where q >= p
#pragma clang fp contract(off)
    const float pp = __builtin_amdgcn_exp2f(fmaf(xp, s, -cp)) * ip;
    r0 = r1 = 0.0f;
    if constexpr (HAS0) {
      const float pq = __builtin_amdgcn_exp2f(fmaf(xq, s, -cq)) * iq;
      const float mn = uminf(pp, pq);
      b0 += mn;
      r0 = pp - mn;
    }
    if constexpr (HAS1) {
      const float pf = __builtin_amdgcn_exp2f(fmaf(xf, s, -cf)) * i_f;
      const float mn = uminf(pp, pf);
      b1 += mn;
      r1 = pf - mn;
    }
  };
  auto visit = [&](float xq, float xp, float xf, int v) {
    float r0, r1;
    elem(xq, xp, xf, r0, r1);
    if constexpr (HAS0) L0.push(r0, v);
    if constexpr (HAS1) L1.push(r1, v);
  };
  auto visit4 = [&](const float* xq, const float* xp, const float* xf, int v0) {
    float r0[4], r1[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) elem(xq[q], xp[q], xf[q], r0[q], r1[q]);
    if constexpr (HAS0) L0.push4(r0, v0);
    if constexpr (HAS1) L1.push4(r1, v0);
  };
  auto flush = [&]() {
    B0 += static_cast<double>(b0);
    B1 += static_cast<double>(b1);
    b0 = b1 = 0.0f;
  };
  const bool vec = ((reinterpret_cast<uintptr_t>(base[0]) | reinterpret_cast<uintptr_t>(base[1]) |
                     reinterpret_cast<uintptr_t>(base[2])) & 15) == 0;
  if (vec) {
    // Vectors vi = i * 256 + tid in increasing i, two per row at a time from
    // two register stages: the loads of the next pair are issued before the
    // current pair is used (clamped in-row indices past the end).
    constexpr int kBatch = 2;
    const int nfull = (e1 - e0) / VPE;
    const u32x4* vr[3];
#pragma unroll
    for (int e = 0; e < 3; ++e) vr[e] = reinterpret_cast<const u32x4*>(base[e]) + e0 / VPE;
    auto fetch = [&](int i0, u32x4 (&w)[3][kBatch]) {
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int vc = min((i0 + q) * kThreads + tid, nfull - 1);
#pragma unroll
        for (int e = 0; e < 3; ++e) w[e][q] = __builtin_nontemporal_load(vr[e] + vc);
      }
    };
    auto use = [&](int i0, const u32x4 (&w)[3][kBatch]) {
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int vi = (i0 + q) * kThreads + tid;
        if (vi >= nfull) continue;
        float x[3][VPE];
#pragma unroll
        for (int e = 0; e < 3; ++e) {
          const uint32_t ww[4] = {w[e][q].x, w[e][q].y, w[e][q].z, w[e][q].w};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            if constexpr (DT == 1) {
              x[e][2 * h] = bf16_lo(ww[h]);
              x[e][2 * h + 1] = bf16_hi(ww[h]);
            } else {
              x[e][h] = __uint_as_float(ww[h]);
            }
          }
        }
        const int v0 = e0 + vi * VPE;
#pragma unroll
        for (int g = 0; g < VPE; g += 4) visit4(&x[0][g], &x[1][g], &x[2][g], v0 + g);
        flush();
      }
    };
    if (nfull > 0) {
      u32x4 wa[3][kBatch], wb[3][kBatch];
      fetch(0, wa);
      for (int i0 = 0; i0 < kVecPerThread && i0 * kThreads < nfull; i0 += 2 * kBatch) {
        fetch(i0 + kBatch, wb);
        use(i0, wa);
        if ((i0 + kBatch) >= kVecPerThread || (i0 + kBatch) * kThreads >= nfull) break;
        fetch(i0 + 2 * kBatch, wa);
        use(i0 + kBatch, wb);
      }
    }
    const int v = e0 + nfull * VPE + tid;
    if (v < e1) visit(load_elem(base[0], v, DT), load_elem(base[1], v, DT), load_elem(base[2], v, DT), v);
  } else {
    int n = 0;
    for (int v = e0 + tid; v < e1; v += kThreads) {
      visit(load_elem(base[0], v, DT), load_elem(base[1], v, DT), load_elem(base[2], v, DT), v);
      if (++n == 8) {
        flush();
        n = 0;
      }
    }
  }
  flush();
}

// pair_scan with the stages present at this position (stage 0 needs a draft
// row, j < k; stage 1 the hierarchy); at least one of them is.
template <int DT, class List>
__device__ inline void pair_scan_any(const char* const* base, int e0, int e1, bool has0,
                                     bool has1, float s, const PairShared& sh, List& L0, List& L1,
                                     double& B0, double& B1) {
  if (has0 && has1)
    pair_scan<DT, true, true>(base, e0, e1, s, sh, L0, L1, B0, B1);
  else if (has1)
    pair_scan<DT, false, true>(base, e0, e1, s, sh, L0, L1, B0, B1);
  else
    pair_scan<DT, true, false>(base, e0, e1, s, sh, L0, L1, B0, B1);
}

// One workgroup per (sequence b, position j, chunk).  Rows: q = exit 0 row j
// (present for j < k), p = exit 1 row j, f = exit 2 row j (hierarchy).
// Stage 0 pairs (q, p), stage 1 pairs (p, f).  Greedy sequences are left to
// the merge kernel (their distributions are one-hots).
template <int DT>
__global__ __launch_bounds__(kThreads) void pair_kernel(ByArgs a) {
  constexpr int ES = DT == 1 ? 2 : 4;
  constexpr int CE = kChunkBytes / ES;
  __shared__ PairShared sh;
  const int npos = a.hier ? a.k + 1 : a.k;
  const int chunk = blockIdx.x % a.nc;
  const int rest = blockIdx.x / a.nc;
  const int j = rest % npos, b = rest / npos;
  const float tau = a.temperature ? a.temperature[b] : 1.0f;
  if (greedy_tau(tau)) return;
  const bool has0 = j < a.k;
  const bool has1 = a.hier != 0;
  const int rq = has0 ? a.exit_row0[0] + b * a.exit_pos[0] + j : -1;
  const int rp = a.exit_row0[1] + b * a.exit_pos[1] + j;
  const int rf = has1 ? a.exit_row0[2] + b * a.exit_pos[2] + j : -1;
  const int tid = threadIdx.x;
  if (tid < 3) {
    const int r = tid == 0 ? rq : (tid == 1 ? rp : rf);
    float c = 0.0f;
    double S = 1.0;
    if (r >= 0) merge_row(a.partials + static_cast<int64_t>(r) * a.nc, a.nc, c, S);
    // p_v = 2^(l_v s - c) / S, the exponent relative to the row's own
    // reference c (folding log2 S into c would cost c's float rounding);
    // a row without a finite logit has no distribution: every p_v = 0
    sh.c[tid] = c;
    sh.inv[tid] = S > 0.0 ? static_cast<float>(1.0 / S) : 0.0f;
  }
  __syncthreads();
  const float s = kLog2e / tau;
  // Absent rows alias the p row; their values are never used.
  auto row_ptr = [&](int e, int r) {
    return static_cast<const char*>(a.exit_ptr[e]) + static_cast<int64_t>(r - a.exit_row0[e]) * a.ld * ES;
  };
  const char* pp_row = row_ptr(1, rp);
  const char* base[3] = {has0 ? row_ptr(0, rq) : pp_row, pp_row, has1 ? row_ptr(2, rf) : pp_row};
  const int e0 = chunk * CE, e1 = min(a.V, e0 + CE);

  Top2 L0, L1;
  L0.init();
  L1.init();
  double B0 = 0.0, B1 = 0.0;
  pair_scan_any<DT>(base, e0, e1, has0, has1, s, sh, L0, L1, B0, B1);

  const int64_t stride_s = static_cast<int64_t>(a.k + 1) * a.nc;
  PairPart* out0 = a.pair + (static_cast<int64_t>(b) * 2 * (a.k + 1) + j) * a.nc + chunk;
  PairPart* out1 = out0 + stride_s;
  bool exact = true;
  if (has0) {
    const double beta = block_sum(B0, sh);
    if (tid == 0) out0->beta = beta;
    exact = block_top(L0, a.top_m, out0, sh) && exact;
  }
  if (has1) {
    const double beta = block_sum(B1, sh);
    if (tid == 0) out1->beta = beta;
    exact = block_top(L1, a.top_m, out1, sh) && exact;
  }
  if (exact) return;
  // Some thread held three or more of the chunk's largest residuals: rescan
  // with the exact lists (rare: ties or residuals clustered in one thread).
  TopList X0, X1;
  X0.init();
  X1.init();
  double D0 = 0.0, D1 = 0.0;
  pair_scan_any<DT>(base, e0, e1, has0, has1, s, sh, X0, X1, D0, D1);
  if (has0) block_top(X0, a.top_m, out0, sh);
  if (has1) block_top(X1, a.top_m, out1, sh);
}

// One wavefront per (sequence b, stage s, position j): sums the chunks' beta
// and merges their lists into the top_m largest residuals.
__global__ __launch_bounds__(kWave) void outcome_merge_kernel(ByArgs a) {
  const int lane = threadIdx.x;
  const int P = a.k + 1;
  const int j = blockIdx.x % P;
  const int s = (blockIdx.x / P) % 2;
  const int b = blockIdx.x / (2 * P);
  const int64_t o = static_cast<int64_t>(blockIdx.x);
  const bool valid = s == 0 ? j < a.k : (a.hier != 0 && j <= a.k);
  float* tmass = a.top_mass ? a.top_mass + o * a.top_m : nullptr;
  int32_t* ttok = a.top_tok ? a.top_tok + o * a.top_m : nullptr;
  if (!valid) {
    if (lane == 0 && a.beta) a.beta[o] = NAN;
    if (lane < a.top_m) {
      if (tmass) tmass[lane] = 0.0f;
      if (ttok) ttok[lane] = -1;
    }
    return;
  }
  const float tau = a.temperature ? a.temperature[b] : 1.0f;
  if (greedy_tau(tau)) {
    // one-hots at the rows' argmax: beta = [equal], residual = one-hot of p's
    const int eq = s == 0 ? 0 : 1, ep = eq + 1;
    const int rq = a.exit_row0[eq] + b * a.exit_pos[eq] + j;
    const int rp = a.exit_row0[ep] + b * a.exit_pos[ep] + j;
    const int xq = merge_argmax(a.partials + static_cast<int64_t>(rq) * a.nc, a.nc);
    const int xp = merge_argmax(a.partials + static_cast<int64_t>(rp) * a.nc, a.nc);
    const bool same = xq == xp;
    if (lane == 0 && a.beta) a.beta[o] = same ? 1.0f : 0.0f;
    if (lane < a.top_m) {
      const bool first = lane == 0 && !same;
      if (tmass) tmass[lane] = first ? 1.0f : 0.0f;
      if (ttok) ttok[lane] = first ? xp : -1;
    }
    return;
  }
  const PairPart* parts = a.pair + o * a.nc;
  double beta = 0.0;
  for (int c = lane; c < a.nc; c += kWave) beta += parts[c].beta;
  beta = wave_sum(beta);
  if (lane == 0 && a.beta) a.beta[o] = static_cast<float>(beta);
  if (!tmass && !ttok) return;
  // candidates: chunk c entry q is candidate c * kTopM + q; lane l holds
  // l, l + 64, ... (at most kMaxVocab / chunk / 8 per lane)
  constexpr int kPerLane = (kMaxVocab / (kChunkBytes / 4)) * kTopM / kWave;
  float cv[kPerLane];
  int ci[kPerLane];
  const int n = a.nc * kTopM;
#pragma unroll
  for (int t = 0; t < kPerLane; ++t) {
    const int id = lane + t * kWave;
    cv[t] = 0.0f;
    ci[t] = -1;
    if (id < n) {
      const PairPart& pp = parts[id / kTopM];
      cv[t] = pp.mass[id % kTopM];
      ci[t] = pp.tok[id % kTopM];
    }
  }
  for (int r = 0; r < a.top_m; ++r) {
    float bv = 0.0f;
    int bi = -1;
#pragma unroll
    for (int t = 0; t < kPerLane; ++t)
      if (ranks_before(cv[t], ci[t], bv, bi)) {
        bv = cv[t];
        bi = ci[t];
      }
#pragma unroll
    for (int sh = 32; sh > 0; sh >>= 1) {
      const float ov = __shfl_xor(bv, sh, kWave);
      const int oi = __shfl_xor(bi, sh, kWave);
      if (ranks_before(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
#pragma unroll
    for (int t = 0; t < kPerLane; ++t)
      if (bi >= 0 && ci[t] == bi) {
        cv[t] = 0.0f;
        ci[t] = -1;
      }
    if (lane == 0) {
      if (tmass) tmass[r] = bi >= 0 ? bv : 0.0f;
      if (ttok) ttok[r] = bi;
    }
  }
}

}  // namespace

hipError_t launch_entropy(const ByArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((a.rows + kThreads - 1) / kThreads));
  hipLaunchKernelGGL(entropy_kernel, grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_outcome(const ByArgs& a, hipStream_t st) {
  const int npos = a.hier ? a.k + 1 : a.k;
  const int64_t wg = static_cast<int64_t>(a.B) * npos * a.nc;
  if (wg > 0) {
    if (a.dtype == 1)
      hipLaunchKernelGGL(pair_kernel<1>, dim3(static_cast<unsigned>(wg)), dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL(pair_kernel<0>, dim3(static_cast<unsigned>(wg)), dim3(kThreads), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const unsigned entries = static_cast<unsigned>(static_cast<int64_t>(a.B) * 2 * (a.k + 1));
  hipLaunchKernelGGL(outcome_merge_kernel, dim3(entries), dim3(kWave), 0, st, a);
  return hipGetLastError();
}

}  // namespace sv
