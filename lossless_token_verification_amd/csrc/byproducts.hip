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

// Per-thread lists of the largest residuals, largest first; elements arrive
// in increasing token order, so strict comparisons keep equal values in token
// order.
//
// TopList keeps kTopM (value, token) entries: exact, but its insertion is a
// chain of compare-swaps that a wavefront runs whenever any lane inserts.
//
// Top3 keeps, branch-free, the three largest *group maxima* a thread has
// seen, plus `drop`, the largest group maximum it pushed out.  A group is the
// pair of vectors a thread takes at a time (its maximum costs one three-way
// max per two elements), listed under the key 2 * v0 + 1 (v0 the first token
// of its first vector), or a single element v under the key 2 * v.  Every
// element of the chunk's top m lies in a group whose maximum is at least the
// m-th largest group maximum (the floor); so, when no dropped group maximum
// reaches the floor, reading again the listed groups at or above it (ties
// included) finds the chunk's top m exactly (pair_lists).  Otherwise the
// chunk is scanned again with TopList: rare, since it needs four of the
// chunk's largest groups in one thread, or more than kMaxExpand groups tied
// at the floor.
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
  __device__ __forceinline__ void push_one(float r, int v) {
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
  // a group's elements, each pushed exactly: vectors of VPE consecutive
  // tokens, the vectors `stride` tokens apart
  template <int VPE, int NV>
  __device__ __forceinline__ void push_group(const float (&r)[NV][VPE], int v0, int stride) {
#pragma unroll
    for (int q = 0; q < NV; ++q)
#pragma unroll
      for (int g = 0; g < VPE; ++g) push_one(r[q][g], v0 + q * stride + g);
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

struct Top3 {
  uint32_t v1, v2, v3, drop;   // float bits of non-negative values
  int32_t i1, i2, i3;          // keys (-1: empty)
  __device__ __forceinline__ void init() {
    v1 = v2 = v3 = drop = 0u;
    i1 = i2 = i3 = -1;
  }
  // group maximum r under key k
  __device__ __forceinline__ void push(uint32_t r, int k) {
    const bool g1 = r > v1, g2 = r > v2, g3 = r > v3;
    drop = max(drop, min(r, v3));   // what leaves (or never enters)
    i3 = g2 ? i2 : (g3 ? k : i3);
    v3 = max(v3, min(r, v2));
    i2 = g1 ? i1 : (g2 ? k : i2);
    v2 = max(v2, min(r, v1));
    i1 = g1 ? k : i1;
    v1 = max(v1, r);
  }
  __device__ __forceinline__ void push_one(float r, int v) { push(__float_as_uint(r), 2 * v); }
  // a group's values (see TopList::push_group), under the key of its first
  // token v0
  template <int VPE, int NV>
  __device__ __forceinline__ void push_group(const float (&r)[NV][VPE], int v0, int) {
    uint32_t M = 0u;
#pragma unroll
    for (int q = 0; q < NV; ++q)
#pragma unroll
      for (int g = 0; g < VPE; ++g) M = max(M, __float_as_uint(r[q][g]));
    push(M, 2 * v0 + 1);
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

// The workgroup's Top3 lists are merged by rank.  The threads form kGroups
// sets of consecutive lanes; the largest list head of a lane set is a real
// entry, distinct from the other sets' ones, so the smallest of the kGroups
// set maxima is a lower bound of the m-th largest entry for every
// m <= kGroups.  Only entries at or above the bound are gathered in LDS (a
// wavefront holds at most 3 * kWave of them), and each gathered entry's rank
// is the number of gathered entries that rank before it.
constexpr int kGroups = 8;                       // lane sets
constexpr int kGroupLanes = kThreads / kGroups;  // lanes per set
constexpr int kCandCap = 3 * kWave;   // a Top3 list per lane
constexpr int kGroupElems = 2 * 8;    // elements of a group: two vectors of at most 8
constexpr int kMaxExpand = 2 * kTopM; // chosen groups (ties at the floor included) read again
static_assert(kTopM <= kGroups, "the group bound covers at most kGroups list entries");
static_assert(kWave % kGroupLanes == 0, "a lane group lies within one wavefront");

struct PairShared {
  float key[kWaves];
  int32_t idx[kWaves];
  float c[3];     // per row: the merged reference c
  double S[3];    // per row: the merged S
  double S1[3];   // per row: the merged S relative to c' (pair_kernel)
  double M[3];    // per row: this chunk's sum of 2^(l s - c), then of 2^(l s - c')
  float kc[6];    // PairK (pair_kernel)
  double zinv[2]; // per stage: 1 / Z
  double mass[2]; // per stage: the target row's mass in this chunk, in units of 1 / Z
  // pair_lists, per stage:
  double rsum[2][kWaves];            // wavefront sums of the residuals
  uint32_t gmax[2][kGroups];         // the lane groups' largest list heads
  uint32_t dmax[2][kGroups];         // and largest dropped group maxima
  int32_t ncand[2][kWaves];          // gathered entries per wavefront
  uint32_t last[2];                  // the m-th largest group maximum (the floor)
  int32_t lost[2];                   // a chosen group whose maximum was not met again
  int32_t nexp[2];                   // groups at or above the floor
  int32_t nsel[2];                   // gathered elements of those groups
  uint2 cand[2][kWaves][kCandCap];   // (residual bits, key)
  uint2 sel[2][kMaxExpand * kGroupElems];   // their elements >= floor: (residual bits, token)
};

// Workgroup top-m of the threads' TopLists: m rounds of a (value, token)
// arg-max; the winning thread drops its head.  Thread 0 writes the chunk's
// list (padded to kTopM).
__device__ inline void block_top(TopList& L, int m, float scale, PairPart* out, PairShared& sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
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
      out->mass[r] = bi >= 0 ? bv * scale : 0.0f;
      out->tok[r] = bi;
    }
  }
  if (threadIdx.x == 0)
    for (int q = m; q < kTopM; ++q) {
      out->mass[q] = 0.0f;
      out->tok[q] = -1;
    }
}

__device__ __forceinline__ uint32_t group_max(uint32_t x) {
#pragma unroll
  for (int o = 1; o < kGroupLanes; o <<= 1)
    x = max(x, static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), o, kWave)));
  return x;
}

// Rank of entry c among n entries of `list` (value bits descending, then
// key or token ascending): the number of entries that rank before it.
__device__ __forceinline__ int rank_of(const uint2 c, const uint2* list, int n) {
  int rank = 0;
  for (int e = 0; e < n; ++e) {
    const uint2 o = list[e];
    rank += (o.x > c.x || (o.x == c.x && o.y < c.y)) ? 1 : 0;
  }
  return rank;
}

// The acceptance masses and the residual lists of both stages of one chunk,
// from the threads' residual sums B0, B1 and Top3 lists, in four barriers:
// (1) the sums and, per lane group, the largest list head and dropped group
// maximum are published; (2) per stage, the list entries at or above the
// bound are gathered; (3) half of the threads per stage rank the gathered
// entries: the m-th one's maximum is the floor; (4) every gathered group at or
// above the floor (ties included) is read again by `elems(st, max, key,
// floor, append)`, which hands its elements at or above the floor to
// append(value bits, token) and returns whether it met the maximum again;
// (5) those elements are ranked: the first m are the chunk's list, padded to
// kTopM.  mass0, mass1: the target rows' masses of the chunk; z0, z1: the
// stages' 1 / Z.  Returns false (and leaves the lists unwritten) when a
// stage's top m may lie outside the groups read: a dropped group maximum
// reaches the floor, or more than kMaxExpand groups do.
template <class Elems>
__device__ inline bool pair_lists(bool has0, bool has1, const Top3& L0, const Top3& L1, double B0,
                                  double B1, int m, double mass0, double mass1, double z0,
                                  double z1, PairPart* out0, PairPart* out1, PairShared& sh,
                                  Elems elems) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  // (1)
  const double s0 = wave_sum(B0), s1 = wave_sum(B1);
  if (lane == 0) {
    sh.rsum[0][wave] = s0;
    sh.rsum[1][wave] = s1;
  }
  const uint32_t g0 = group_max(L0.v1), g1 = group_max(L1.v1);
  const uint32_t d0 = group_max(L0.drop), d1 = group_max(L1.drop);
  if ((tid & (kGroupLanes - 1)) == 0) {
    sh.gmax[0][tid / kGroupLanes] = g0;
    sh.gmax[1][tid / kGroupLanes] = g1;
    sh.dmax[0][tid / kGroupLanes] = d0;
    sh.dmax[1][tid / kGroupLanes] = d1;
  }
  if (tid < 2) {
    sh.lost[tid] = 0;
    sh.nexp[tid] = 0;
    sh.nsel[tid] = 0;
  }
  __syncthreads();
  if (tid == 0) {
    double r0 = 0.0, r1 = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      r0 += sh.rsum[0][w];
      r1 += sh.rsum[1][w];
    }
    if (has0) out0->beta = (mass0 - r0) * z0;
    if (has1) out1->beta = (mass1 - r1) * z1;
  }
  if (m == 0) {   // nothing to list (uniform)
    if (tid < kTopM) {
      if (has0) {
        out0->mass[tid] = 0.0f;
        out0->tok[tid] = -1;
      }
      if (has1) {
        out1->mass[tid] = 0.0f;
        out1->tok[tid] = -1;
      }
    }
    return true;
  }
  uint32_t th[2], dropped[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    uint32_t t = sh.gmax[st][0], d = sh.dmax[st][0];
#pragma unroll
    for (int i = 1; i < kGroups; ++i) {
      t = min(t, sh.gmax[st][i]);
      d = max(d, sh.dmax[st][i]);
    }
    th[st] = max(t, 1u);   // the lists hold positive values only
    dropped[st] = d;
  }
  // (2) gather each stage's entries >= its bound (at most three per lane)
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    if (st == 0 ? !has0 : !has1) continue;
    const Top3& L = st == 0 ? L0 : L1;
    int n = 0;
#pragma unroll
    for (int e = 0; e < 3; ++e) {
      const uint32_t v = e == 0 ? L.v1 : (e == 1 ? L.v2 : L.v3);
      const int32_t k = e == 0 ? L.i1 : (e == 1 ? L.i2 : L.i3);
      const bool c = v >= th[st] && k >= 0;
      const uint64_t mask = __ballot(c);
      if (c) {
        const int pos = static_cast<int>(__builtin_amdgcn_mbcnt_hi(
            static_cast<uint32_t>(mask >> 32),
            __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), static_cast<uint32_t>(n))));
        sh.cand[st][wave][pos] = make_uint2(v, static_cast<uint32_t>(k));
      }
      n += __popcll(mask);
    }
    if (lane == 0) sh.ncand[st][wave] = n;
  }
  __syncthreads();
  // (3) half of the threads per stage (all of them with one stage)
  const int nst = (has0 ? 1 : 0) + (has1 ? 1 : 0);
  const int span = kThreads / nst;
  const int st = nst == 2 ? tid / span : (has0 ? 0 : 1);
  const int t0 = nst == 2 ? tid % span : tid;
  int N = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) N += sh.ncand[st][w];
  auto cand_at = [&](int t) {
    int w = 0, e = t;
    while (e >= sh.ncand[st][w]) {
      e -= sh.ncand[st][w];
      ++w;
    }
    return sh.cand[st][w][e];
  };
  if (N >= m)
    for (int t = t0; t < N; t += span) {
      const uint2 c = cand_at(t);
      int rank = 0;
      for (int w2 = 0; w2 < kWaves; ++w2) rank += rank_of(c, sh.cand[st][w2], sh.ncand[st][w2]);
      if (rank == m - 1) sh.last[st] = c.x;
    }
  __syncthreads();
  // (4) every group at or above the floor is read again (the floor is the
  // bound when fewer than m groups are listed: then all of them are)
  const uint32_t floor = N >= m ? sh.last[st] : (st == 0 ? th[0] : th[1]);
  for (int t = t0; t < N; t += span) {
    const uint2 c = cand_at(t);
    if (c.x < floor) continue;
    if (atomicAdd(&sh.nexp[st], 1) >= kMaxExpand) continue;
    const bool met = elems(st, c.x, static_cast<int32_t>(c.y), floor, [&](uint32_t v, int32_t tok) {
      const int pos = atomicAdd(&sh.nsel[st], 1);
      sh.sel[st][pos] = make_uint2(v, static_cast<uint32_t>(tok));
    });
    if (!met) sh.lost[st] = 1;
  }
  __syncthreads();
  // (5) exactness of both stages (uniform), then the lists
  bool exact = true;
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    if (s2 == 0 ? !has0 : !has1) continue;
    int N2 = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) N2 += sh.ncand[s2][w];
    // no dropped group maximum reaches the floor (with fewer than m groups
    // listed, none was dropped at all)
    const bool kept = N2 >= m ? dropped[s2] < sh.last[s2] : dropped[s2] == 0u;
    exact = exact && kept && sh.lost[s2] == 0 && sh.nexp[s2] <= kMaxExpand;
  }
  if (!exact) return false;
  const int n2 = sh.nsel[st];
  PairPart* out = st == 0 ? out0 : out1;
  const float scale = static_cast<float>(st == 0 ? z0 : z1);
  for (int t = t0; t < n2; t += span) {
    const uint2 c = sh.sel[st][t];
    const int rank = rank_of(c, sh.sel[st], n2);
    if (rank < m) {
      out->mass[rank] = __uint_as_float(c.x) * scale;
      out->tok[rank] = static_cast<int32_t>(c.y);
    }
  }
  if (t0 == 0)
    for (int q = min(n2, m); q < kTopM; ++q) {
      out->mass[q] = 0.0f;
      out->tok[q] = -1;
    }
  return true;
}

// Constants of one workgroup's rows (see pair_kernel): s = log2(e) / tau, the
// exponent offsets of q, p, f, the factor of q in stage 0's units and of p
// in stage 1's.
struct PairK {
  float s, cq, cp, cf, iq, ip1;
};

// The residuals of one element: stage 0 pairs (q, p), r0 = max(0, p - q);
// stage 1 pairs (p, f), r1 = max(0, f - p).  Each stage works in units in
// which its target row's values are 2^(l s - c') <= 1 (c' at or above
// l_max s, see pair_kernel); the difference target - draft is then at most 1
// and max(0, .) is a clamp to [0, 1], which folds into the subtraction.
template <bool HAS0, bool HAS1>
__device__ __forceinline__ void pair_elem(const PairK& k, float xq, float xp, float xf, float& r0,
                                          float& r1) {
#pragma clang fp contract(off)
  const float pp = __builtin_amdgcn_exp2f(fmaf(xp, k.s, -k.cp));
  r0 = r1 = 0.0f;
  if constexpr (HAS0) {
    const float pq = __builtin_amdgcn_exp2f(fmaf(xq, k.s, -k.cq)) * k.iq;
    r0 = __builtin_amdgcn_fmed3f(pp - pq, 0.0f, 1.0f);
  }
  if constexpr (HAS1) {
    const float pf = __builtin_amdgcn_exp2f(fmaf(xf, k.s, -k.cf));
    r1 = __builtin_amdgcn_fmed3f(pf - pp * k.ip1, 0.0f, 1.0f);
  }
}

template <int DT, int VPE>
__device__ __forceinline__ void unpack_vec(const u32x4& w, float (&x)[VPE]) {
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    if constexpr (DT == 1) {
      x[2 * h] = bf16_lo(ww[h]);
      x[2 * h + 1] = bf16_hi(ww[h]);
    } else {
      x[h] = __uint_as_float(ww[h]);
    }
  }
}

// One pass over elements [e0, e1) of the rows q = base[0], p = base[1],
// f = base[2] (absent rows alias p): stage 0 (HAS0) adds r0 = max(0, p - q)
// to B0 and offers it to L0, stage 1 (HAS1) likewise r1 = max(0, f - p).
// Each thread visits its elements in increasing token order, a 16-byte vector
// at a time where the rows allow 16-byte loads.  `pro()` (called by the whole
// workgroup: it may hold barriers) yields the constants, after the first
// loads are on their way.
template <int DT, bool HAS0, bool HAS1, class List, class Pro>
__device__ inline void pair_scan(const char* const* base, int e0, int e1, Pro&& pro, List& L0,
                                 List& L1, double& B0, double& B1) {
  constexpr int VPE = DT == 1 ? 8 : 4;
  const int tid = threadIdx.x;
  float b0 = 0.0f, b1 = 0.0f;
  PairK k;
  auto visit = [&](float xq, float xp, float xf, int v) {
    float r0, r1;
    pair_elem<HAS0, HAS1>(k, xq, xp, xf, r0, r1);
    b0 += r0;
    b1 += r1;
    if constexpr (HAS0) L0.push_one(r0, v);
    if constexpr (HAS1) L1.push_one(r1, v);
  };
  auto flush = [&]() {
    B0 += static_cast<double>(b0);
    B1 += static_cast<double>(b1);
    b0 = b1 = 0.0f;
  };
  // only the rows of the stages present are read (an absent row's values
  // are never used)
  auto has_row = [](int e) { return e == 1 || (e == 0 ? HAS0 : HAS1); };
  auto elem_at = [&](int e, int v) { return has_row(e) ? load_elem(base[e], v, DT) : 0.0f; };
  const bool vec = ((reinterpret_cast<uintptr_t>(base[0]) | reinterpret_cast<uintptr_t>(base[1]) |
                     reinterpret_cast<uintptr_t>(base[2])) & 15) == 0;
  if (vec) {
    // Vectors vi = i * kThreads + tid in increasing i, two per row at a time
    // from two register stages: the loads of the next pair are issued before
    // the current pair is used (clamped in-row indices past the end).
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
        for (int e = 0; e < 3; ++e)
          if (has_row(e)) w[e][q] = __builtin_nontemporal_load(vr[e] + vc);
      }
    };
    // a pair of vectors (tokens v0.. and v0 + kThreads * VPE..) is one group
    auto use = [&](int i0, const u32x4 (&w)[3][kBatch]) {
      float r0[kBatch][VPE], r1[kBatch][VPE];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int vi = (i0 + q) * kThreads + tid;
#pragma unroll
        for (int g = 0; g < VPE; ++g) r0[q][g] = r1[q][g] = 0.0f;
        if (vi >= nfull) continue;
        float x[3][VPE];
#pragma unroll
        for (int e = 0; e < 3; ++e)
          if (has_row(e)) unpack_vec<DT, VPE>(w[e][q], x[e]);
#pragma unroll
        for (int g = 0; g < VPE; ++g) {
          pair_elem<HAS0, HAS1>(k, x[0][g], x[1][g], x[2][g], r0[q][g], r1[q][g]);
          b0 += r0[q][g];
          b1 += r1[q][g];
        }
        flush();
      }
      const int v0 = e0 + (i0 * kThreads + tid) * VPE;
      if constexpr (HAS0) L0.push_group(r0, v0, kThreads * VPE);
      if constexpr (HAS1) L1.push_group(r1, v0, kThreads * VPE);
    };
    u32x4 wa[3][kBatch], wb[3][kBatch];
    if (nfull > 0) fetch(0, wa);
    k = pro();
    if (nfull > 0) {
      // unrolled: straight-line code lets each load wait only for its own batch
#pragma unroll
      for (int i0 = 0; i0 < kVecPerThread; i0 += 2 * kBatch) {
        if (i0 * kThreads >= nfull) break;
        fetch(i0 + kBatch, wb);
        use(i0, wa);
        if ((i0 + kBatch) >= kVecPerThread || (i0 + kBatch) * kThreads >= nfull) break;
        fetch(i0 + 2 * kBatch, wa);
        use(i0 + kBatch, wb);
      }
    }
    const int v = e0 + nfull * VPE + tid;
    if (v < e1) visit(elem_at(0, v), elem_at(1, v), elem_at(2, v), v);
  } else {
    k = pro();
    int n = 0;
    for (int v = e0 + tid; v < e1; v += kThreads) {
      visit(elem_at(0, v), elem_at(1, v), elem_at(2, v), v);
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
template <int DT, class List, class Pro>
__device__ inline void pair_scan_any(const char* const* base, int e0, int e1, bool has0,
                                     bool has1, Pro&& pro, List& L0, List& L1, double& B0,
                                     double& B1) {
  if (has0 && has1)
    pair_scan<DT, true, true>(base, e0, e1, pro, L0, L1, B0, B1);
  else if (has1)
    pair_scan<DT, false, true>(base, e0, e1, pro, L0, L1, B0, B1);
  else
    pair_scan<DT, true, false>(base, e0, e1, pro, L0, L1, B0, B1);
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
  const float s = kLog2e / tau;
  // Absent rows alias the p row; their values are never used.
  auto row_ptr = [&](int e, int r) {
    return static_cast<const char*>(a.exit_ptr[e]) + static_cast<int64_t>(r - a.exit_row0[e]) * a.ld * ES;
  };
  const char* pp_row = row_ptr(1, rp);
  const char* base[3] = {has0 ? row_ptr(0, rq) : pp_row, pp_row, has1 ? row_ptr(2, rf) : pp_row};
  const int e0 = chunk * CE, e1 = min(a.V, e0 + CE);

  // The constants, from the rows' chunk partials (while the first loads are
  // in flight).  Every row gets the offset c', the float just above its
  // merged reference c (c is l_max s rounded to nearest, so c' >= l_max s
  // and every value 2^(l s - c') is at most 1), and S' = S * 2^(c - c').  A
  // stage counts in units of 1 / Z, Z = S' of its target row (1 for a row
  // without a finite logit): the target's value at v is 2^(l_v s - c'), the
  // draft's 2^(l_v s - c'_d) * (Z / S'_d).
  // A row without a finite logit (S = 0) gets an offset of +inf: every value
  // is 0.  The acceptance mass sum_v min(p_v, q_v) of the chunk is its target
  // mass minus its residual sum, the target mass being the row statistics'
  // own chunk partial, rescaled to c'.
  const Partial* const partials = a.partials;
  const int nc = a.nc;
  const int my_row = tid == 0 ? rq : (tid == 1 ? rp : rf);   // threads 0, 1, 2
  auto prologue = [partials, nc, chunk, tid, my_row, s]() -> PairK {
    if (tid < 3) {
      const int r = my_row;
      float c = 0.0f;
      double S = 1.0, M = 0.0;
      if (r >= 0) {
        const Partial* pr = partials + static_cast<int64_t>(r) * nc;
        merge_row(pr, nc, c, S);
        const Partial own = pr[chunk];
        if (own.S > 0.0) M = own.S * exp2(static_cast<double>(own.key) - static_cast<double>(c));
      }
      sh.c[tid] = c;
      sh.S[tid] = S;
      sh.M[tid] = M;
    }
    __syncthreads();
    if (tid < 3) {
      // every row alike (so that identical rows give identical values):
      // c' just above c, and S, M rescaled to it
      const double S = sh.S[tid];
      const float c1 = S > 0.0 ? nextafterf(sh.c[tid], INFINITY) : INFINITY;
      const double u = S > 0.0 ? exp2(static_cast<double>(sh.c[tid]) - static_cast<double>(c1)) : 0.0;
      sh.kc[1 + tid] = c1;
      sh.S1[tid] = S * u;
      sh.M[tid] *= u;
    }
    __syncthreads();
    if (tid == 0) {
      const double Sq = sh.S1[0], Sp = sh.S1[1], Sf = sh.S1[2];
      const double Z0 = Sp > 0.0 ? Sp : 1.0, Z1 = Sf > 0.0 ? Sf : 1.0;
      sh.kc[0] = s;
      sh.kc[4] = Sq > 0.0 ? static_cast<float>(Z0 / Sq) : 0.0f;
      sh.kc[5] = Sp > 0.0 ? static_cast<float>(Z1 / Z0) : 0.0f;
      sh.zinv[0] = 1.0 / Z0;
      sh.zinv[1] = 1.0 / Z1;
      sh.mass[0] = sh.M[1];
      sh.mass[1] = sh.M[2];
    }
    __syncthreads();
    return PairK{sh.kc[0], sh.kc[1], sh.kc[2], sh.kc[3], sh.kc[4], sh.kc[5]};
  };

  Top3 L0, L1;
  L0.init();
  L1.init();
  double B0 = 0.0, B1 = 0.0;
  pair_scan_any<DT>(base, e0, e1, has0, has1, prologue, L0, L1, B0, B1);
  const PairK kk{sh.kc[0], sh.kc[1], sh.kc[2], sh.kc[3], sh.kc[4], sh.kc[5]};
  auto consts = [&]() { return kk; };

  // Reading a chosen group again: a single element (even key) is its own
  // maximum; a pair of vectors (key 2 * v0 + 1, tokens v0.. and
  // v0 + kThreads * VPE..) is read again and its residuals redone (the same
  // operations as the scan, so the same values).
  constexpr int VPE = DT == 1 ? 8 : 4;
  constexpr int kStride = kThreads * VPE;
  const int vend = e0 + (e1 - e0) / VPE * VPE;   // end of the whole vectors
  auto elems = [&](int st, uint32_t val, int32_t key, uint32_t bound, auto&& append) -> bool {
    if ((key & 1) == 0) {
      append(val, key >> 1);
      return true;
    }
    const int v0 = key >> 1;
    bool met = false;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int vb = v0 + q * kStride;
      if (vb >= vend) break;
      // the stage's two rows (the other one's values are left unused)
      float x[3][VPE];
#pragma unroll
      for (int e = 0; e < 3; ++e) {
        const bool need = e == 1 || e == (st == 0 ? 0 : 2);
        const u32x4 raw = need ? *reinterpret_cast<const u32x4*>(base[e] + static_cast<int64_t>(vb) * ES)
                               : u32x4{0u, 0u, 0u, 0u};
        unpack_vec<DT, VPE>(raw, x[e]);
      }
#pragma unroll
      for (int g = 0; g < VPE; ++g) {
        float r0, r1;
        pair_elem<true, true>(kk, x[0][g], x[1][g], x[2][g], r0, r1);
        const uint32_t r = __float_as_uint(st == 0 ? r0 : r1);
        if (r >= bound) append(r, vb + g);
        met = met || r == val;
      }
    }
    return met;
  };

  const int64_t stride_s = static_cast<int64_t>(a.k + 1) * a.nc;
  PairPart* out0 = a.pair + (static_cast<int64_t>(b) * 2 * (a.k + 1) + j) * a.nc + chunk;
  PairPart* out1 = out0 + stride_s;
  const double z0 = sh.zinv[0], z1 = sh.zinv[1];
  const bool exact = pair_lists(has0, has1, L0, L1, B0, B1, a.top_m, sh.mass[0], sh.mass[1], z0,
                                z1, out0, out1, sh, elems);
  if (exact) return;
  // A group maximum left out of the lists could reach the chosen groups (rare:
  // three of the chunk's largest groups in one thread, or a tie): rescan with
  // the exact lists, one stage at a time (two lists of kTopM entries at once
  // would raise the kernel's register count, and with it lower every
  // launch's occupancy).
  TopList X0, X1;
  X0.init();
  X1.init();
  double D0 = 0.0, D1 = 0.0;
  if (has0) {
    pair_scan_any<DT>(base, e0, e1, true, false, consts, X0, X1, D0, D1);
    block_top(X0, a.top_m, static_cast<float>(z0), out0, sh);
  }
  if (has1) {
    pair_scan_any<DT>(base, e0, e1, false, true, consts, X0, X1, D0, D1);
    block_top(X1, a.top_m, static_cast<float>(z1), out1, sh);
  }
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
  // each chunk's mass is its target mass minus its residual sum: clamp the
  // rounding of that difference to [0, 1]
  if (lane == 0 && a.beta) a.beta[o] = static_cast<float>(fmin(fmax(beta, 0.0), 1.0));
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
