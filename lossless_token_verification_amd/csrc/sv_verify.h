// Per-sequence verification, run by one 256-thread workgroup once the
// statistics of the sequence's rows are complete:
//
//   1. merge the chunk partials of the rows into (reference c, sum S) or
//      (max, argmax) per (exit, position);
//   2. wavefront 0, lane j = position j: gather the logits of the drafted token
//      in the draft and target rows, p(x) and q(x), one Philox4x32-10 block for
//      (j, b, stage, offset), accept iff u * q(x) < p(x); a ballot gives the
//      first rejection (windows of the given size are examined in order);
//   3. the whole workgroup draws the correction from max(0, p - q), or the bonus
//      from p, at the stop position by an inverse CDF: tile sums of the weights
//      (one 16-byte load per lane and tile) into LDS, a workgroup scan of the
//      tile sums in fp64, then one wavefront rescans the selected tile.
//
// Stage 1 (or the single stage) compares the draft exit with the target exit;
// stage 2 of the hierarchy compares L_i with L_f on the tentative tokens (HiSpec
// summary, section 2 "Kernmechanismus" and bullet "Verlustfreie Garantie").  The
// rule is the standard speculative-sampling rule; the residual follows the SSD
// summary (section 3.B) and the bonus token its section 2 item 1.
#pragma once

#include "sv_common.h"

namespace sv {

struct RowStat {
  float key;    // c (sampled) or max (greedy)
  int amax;     // greedy argmax
  double S;     // sampled: sum 2^(l s - c)
  float inv_S;  // (float)(1 / S)
};

struct DrawResult {
  int y;
  double R, t, c_lo, c_hi;
};

struct VerifyShared {
  RowStat st[3][kMaxPositions];
  float tiles[kMaxTiles];
  double dscan[kThreads];
  int iscr[8];
  double dscr[8];
  int toks[kMaxPositions];   // tokens of the current stage
  float vs[kMaxPositions];   // draw uniforms of the current stage
  int sh[8];
};

template <int DT>
struct RowT {
  static constexpr int VPE = DT == 1 ? 8 : 4;
  static constexpr int ES = DT == 1 ? 2 : 4;
};

// Draw weight of one element: p(v) or max(0, p(v) - q(v)), in fp32.
// Contraction is off so every evaluation of the same element gives the same
// bits (the tile pass and the rescan must agree).
__device__ __forceinline__ float weight(float lp, float lq, float s, float cp, float isp, float cq,
                                        float isq, bool has_q) {
#pragma clang fp contract(off)
  const float p = __builtin_amdgcn_exp2f(fmaf(lp, s, -cp)) * isp;
  if (!has_q) return p;
  const float q = __builtin_amdgcn_exp2f(fmaf(lq, s, -cq)) * isq;
  return fmaxf(p - q, 0.0f);
}

template <int DT>
__device__ __forceinline__ void unpack_vec(const u32x4& v, float (&x)[RowT<DT>::VPE]) {
  if constexpr (DT == 1) {
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
    x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
    x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
  } else {
    x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
  }
}

// Load elements [e, e + VPE) of a row (out-of-range elements read as -inf).
template <int DT>
__device__ __forceinline__ void load_group(const char* row, int e, int V, bool vec_ok,
                                           float (&x)[RowT<DT>::VPE]) {
  constexpr int VPE = RowT<DT>::VPE;
  if (vec_ok && e + VPE <= V) {
    unpack_vec<DT>(*reinterpret_cast<const u32x4*>(row + static_cast<int64_t>(e) * RowT<DT>::ES), x);
  } else {
#pragma unroll
    for (int q = 0; q < VPE; ++q) x[q] = (e + q < V) ? load_elem(row, e + q, DT) : -INFINITY;
  }
}

// Sum of the weights of one lane's VPE elements (pairwise, fp32).
template <int DT>
__device__ __forceinline__ float lane_weight_sum(const float (&xp)[RowT<DT>::VPE],
                                                 const float (&xq)[RowT<DT>::VPE], float s,
                                                 float cp, float isp, float cq, float isq,
                                                 bool has_q) {
  constexpr int VPE = RowT<DT>::VPE;
  float w[VPE];
#pragma unroll
  for (int q = 0; q < VPE; ++q) w[q] = weight(xp[q], xq[q], s, cp, isp, cq, isq, has_q);
#pragma unroll
  for (int h = VPE / 2; h > 0; h >>= 1)
#pragma unroll
    for (int q = 0; q < h; ++q) w[q] += w[q + h];
  return w[0];
}

// Inverse-CDF draw over the weights of one row (pair), executed by the whole
// workgroup.  Returns y = the smallest index with C(y) > v * R, or, when
// rounding leaves none, the largest index with a positive weight; y = -1 when
// R == 0.  All threads must call it (it contains barriers).
template <int DT>
__device__ DrawResult draw_tokens(const char* prow, const RowStat& ps, const char* qrow,
                                  const RowStat& qs, bool has_q, float s, int V, float v,
                                  VerifyShared& sm) {
  constexpr int VPE = RowT<DT>::VPE;
  constexpr int ES = RowT<DT>::ES;
  constexpr int TE = kWave * VPE;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int NT = (V + TE - 1) / TE;
  const bool vec_ok = ((reinterpret_cast<uintptr_t>(prow) |
                        (has_q ? reinterpret_cast<uintptr_t>(qrow) : 0)) & 15) == 0;
  const float cp = ps.key, isp = ps.inv_S;
  const float cq = has_q ? qs.key : 0.0f, isq = has_q ? qs.inv_S : 0.0f;
  float* tiles = sm.tiles;

  // Pass 1: tile sums.  Wavefront w takes groups of G consecutive tiles, the
  // groups of the four wavefronts interleaved; all G loads are issued first.
  constexpr int G = 4;
  for (int t0 = wave * G; t0 < NT; t0 += kWaves * G) {
    float sums[G];
    if (vec_ok && (t0 + G) * TE <= V) {
      u32x4 vp[G], vq[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int64_t off = static_cast<int64_t>((t0 + g) * TE + lane * VPE) * ES;
        vp[g] = *reinterpret_cast<const u32x4*>(prow + off);
        if (has_q) vq[g] = *reinterpret_cast<const u32x4*>(qrow + off);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float xp[VPE], xq[VPE];
        unpack_vec<DT>(vp[g], xp);
        if (has_q) unpack_vec<DT>(vq[g], xq);
        else
#pragma unroll
          for (int q = 0; q < VPE; ++q) xq[q] = 0.0f;
        sums[g] = wave_sum(lane_weight_sum<DT>(xp, xq, s, cp, isp, cq, isq, has_q));
      }
    } else {
#pragma unroll 1
      for (int g = 0; g < G; ++g) {
        float xp[VPE], xq[VPE];
        const int e = (t0 + g) * TE + lane * VPE;
        load_group<DT>(prow, e, V, vec_ok, xp);
        if (has_q) load_group<DT>(qrow, e, V, vec_ok, xq);
        else
#pragma unroll
          for (int q = 0; q < VPE; ++q) xq[q] = 0.0f;
        sums[g] = wave_sum(lane_weight_sum<DT>(xp, xq, s, cp, isp, cq, isq, has_q));
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
        if (t0 + g < NT) tiles[t0 + g] = sums[g];
    }
  }
  __syncthreads();

  // Pass 2: fp64 scan of the tile sums.  Thread t owns tiles [t*per, t*per+per).
  double* dscan = sm.dscan;
  int* iscr = sm.iscr;
  double* dscr = sm.dscr;
  const int per = (NT + kThreads - 1) / kThreads;
  const int lo = min(NT, tid * per), hi = min(NT, lo + per);
  double mine = 0.0;
  for (int i = lo; i < hi; ++i) mine += static_cast<double>(tiles[i]);
  dscan[tid] = mine;
  if (tid == 0) {
    iscr[0] = 0x7fffffff;   // first crossing tile
    iscr[1] = -1;           // last tile with positive sum
  }
  __syncthreads();
  for (int o = 1; o < kThreads; o <<= 1) {   // Hillis-Steele inclusive scan
    const double add = tid >= o ? dscan[tid - o] : 0.0;
    __syncthreads();
    dscan[tid] += add;
    __syncthreads();
  }
  const double R = dscan[kThreads - 1];
  const double excl = tid > 0 ? dscan[tid - 1] : 0.0;
  DrawResult res;
  res.R = R;
  res.t = static_cast<double>(v) * R;
  res.y = -1;
  res.c_lo = res.c_hi = 0.0;
  __syncthreads();   // every thread has read the scan before any early return
  if (!(R > 0.0)) return res;   // uniform across the workgroup
  const double tv = res.t;
  {
    // The chosen token has a positive weight, so only tiles with a positive
    // sum can hold it (this also absorbs rounding between the owners' runs).
    double run = excl;
    for (int i = lo; i < hi; ++i) {
      const double nxt = run + static_cast<double>(tiles[i]);
      if (nxt > tv && tiles[i] > 0.0f) {
        atomicMin(&iscr[0], i);
        break;
      }
      run = nxt;
    }
    for (int i = hi - 1; i >= lo; --i) {
      if (tiles[i] > 0.0f) {
        atomicMax(&iscr[1], i);
        break;
      }
    }
  }
  __syncthreads();
  const int T = iscr[0];
  const bool overrun = (T == 0x7fffffff);
  const int TT = overrun ? iscr[1] : T;   // tile to rescan
  if (TT >= lo && TT < hi) {
    double run = excl;
    for (int i = lo; i < TT; ++i) run += static_cast<double>(tiles[i]);
    dscr[0] = run;
  }
  __syncthreads();

  // Pass 3: wavefront 0 rescans tile TT element by element in fp64.
  if (wave == 0) {
    const int e = TT * TE + lane * VPE;
    float xp[VPE], xq[VPE], w[VPE];
    load_group<DT>(prow, e, V, vec_ok, xp);
    if (has_q) load_group<DT>(qrow, e, V, vec_ok, xq);
    double lsum = 0.0;
#pragma unroll
    for (int q = 0; q < VPE; ++q) {
      w[q] = weight(xp[q], has_q ? xq[q] : 0.0f, s, cp, isp, cq, isq, has_q);
      lsum += static_cast<double>(w[q]);
    }
    double incl = lsum;   // inclusive prefix of lane sums
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const double up = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += up;
    }
    const double lane_excl = __shfl_up(incl, 1, kWave);
    double run = dscr[0] + (lane > 0 ? lane_excl : 0.0);
    int cross = -1;
    double c_lo = 0.0, c_hi = 0.0;
    int lastpos = -1;
    double last_lo = 0.0, last_hi = 0.0;
#pragma unroll
    for (int q = 0; q < VPE; ++q) {
      const double nxt = run + static_cast<double>(w[q]);
      if (!overrun && cross < 0 && nxt > tv && w[q] > 0.0f) {
        cross = q;
        c_lo = run;
        c_hi = nxt;
      }
      if (w[q] > 0.0f) {
        lastpos = q;
        last_lo = run;
        last_hi = nxt;
      }
      run = nxt;
    }
    const unsigned long long cm = __ballot(cross >= 0);
    if (cm) {
      const int src = __ffsll(cm) - 1;
      const int yq = __shfl(cross, src, kWave);
      const double lo_ = __shfl(c_lo, src, kWave), hi_ = __shfl(c_hi, src, kWave);
      if (lane == 0) {
        iscr[2] = TT * TE + src * VPE + yq;
        dscr[1] = lo_;
        dscr[2] = hi_;
      }
    } else {
      // no crossing: the last element of the tile with a positive weight
      const unsigned long long pm = __ballot(lastpos >= 0);
      const int src = pm ? 63 - __clzll(pm) : 0;
      const int yq = __shfl(lastpos, src, kWave);
      const double lo_ = __shfl(last_lo, src, kWave), hi_ = __shfl(last_hi, src, kWave);
      if (lane == 0) {
        iscr[2] = pm ? TT * TE + src * VPE + yq : -1;
        dscr[1] = lo_;
        dscr[2] = hi_;
      }
    }
  }
  __syncthreads();
  res.y = iscr[2];
  res.c_lo = dscr[1];
  res.c_hi = dscr[2];
  __syncthreads();   // scratch may be reused by the caller
  return res;
}

__device__ __forceinline__ RowStat merge_row(const Partial* pp, int nc, bool greedy) {
  RowStat r;
  if (greedy) {
    r.key = -INFINITY;
    r.amax = 0x7fffffff;
    for (int c = 0; c < nc; ++c) {
      const Partial q = fetch_partial(pp + c);
      if (q.key > r.key || (q.key == r.key && q.amax < r.amax)) {
        r.key = q.key;
        r.amax = q.amax;
      }
    }
    r.S = 0.0;
    r.inv_S = 0.0f;
  } else {
    // the reference of the whole row first, then the rescaled sums
    float cm = -INFINITY;
    for (int c = 0; c < nc; ++c) cm = fmaxf(cm, fetch_partial(pp + c).key);
    double S = 0.0;
    for (int c = 0; c < nc; ++c) {
      const Partial q = fetch_partial(pp + c);
      if (q.S > 0.0) S += q.S * exp2(static_cast<double>(q.key) - static_cast<double>(cm));
    }
    r.key = cm;
    r.amax = -1;
    r.S = S;
    r.inv_S = static_cast<float>(1.0 / S);
  }
  return r;
}

// Per-sequence context shared by the two stages.
template <int DT>
struct SeqCtx {
  const FusedArgs& a;
  VerifyShared& sm;
  int b, k, V;
  bool greedy;
  float s;

  __device__ SeqCtx(const FusedArgs& a_, VerifyShared& sm_, int b_) : a(a_), sm(sm_), b(b_) {
    k = a.k;
    V = a.V;
    const float tau = a.temperature ? a.temperature[b] : 1.0f;
    const bool bad_tau = !(tau >= 0.0f) || !(tau < INFINITY);
    greedy = !(tau > 0.0f) || bad_tau;
    s = greedy ? 0.0f : kLog2e / tau;
    if (bad_tau && threadIdx.x == 0) atomicOr(a.flags, kFlagTemperature);
  }

  __device__ int positions(int e) const { return e == 0 ? k : k + 1; }

  __device__ const char* row_ptr(int e, int j) const {
    return static_cast<const char*>(a.exit_ptr[e]) +
           (static_cast<int64_t>(b) * positions(e) + j) * a.ld * RowT<DT>::ES;
  }

  // Merged statistics of positions [0, n) of exit e into sm.st[e] (all threads).
  __device__ void merge(int e, int n) {
    const int tid = threadIdx.x;
    if (tid < n) {
      const int64_t row = a.exit_row0[e] + static_cast<int64_t>(b) * positions(e) + tid;
      sm.st[e][tid] = merge_row(a.partials + row * a.nc, a.nc, greedy);
    }
  }

  // One verification chain over tokens sm.toks[0..n): q rows of exit qe, p rows
  // of exit pe, Philox stage `stage`.  Returns the accept count; leaves the
  // draw uniforms in sm.vs[0..n] (position n only with a bonus).
  __device__ int decide(int qe, int pe, int n, int stage, bool bonus, int window) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int diag_pos = k + 1;
    if (tid < kWave) {
      const int j = lane;
      bool reject = false;
      float u = NAN, v = NAN;
      double pj = NAN, qj = NAN;
      if (j < n + (bonus ? 1 : 0)) {
        const uint4 w = philox4x32_10(
            make_uint4(static_cast<uint32_t>(j), static_cast<uint32_t>(b),
                       static_cast<uint32_t>(stage), a.offset), a.key0, a.key1);
        u = uniform24(w.x);
        v = uniform24(w.y);
        sm.vs[j] = v;
      }
      if (j < n) {
        const int x = sm.toks[j];
        const bool valid = x >= 0 && x < V;
        if (!valid) atomicOr(a.flags, kFlagTokenRange);
        if (greedy) {
          reject = !(valid && x == sm.st[pe][j].amax);
          pj = valid && x == sm.st[pe][j].amax ? 1.0 : 0.0;
          qj = valid && x == sm.st[qe][j].amax ? 1.0 : 0.0;
        } else if (valid) {
          const float lp = load_elem(row_ptr(pe, j), x, DT);
          const float lq = load_elem(row_ptr(qe, j), x, DT);
          const float ep = __builtin_amdgcn_exp2f(fmaf(lp, s, -sm.st[pe][j].key));
          const float eq = __builtin_amdgcn_exp2f(fmaf(lq, s, -sm.st[qe][j].key));
          pj = static_cast<double>(ep) / sm.st[pe][j].S;
          qj = static_cast<double>(eq) / sm.st[qe][j].S;
          reject = !(static_cast<double>(u) * qj < pj);
        } else {
          reject = true;
          pj = 0.0;
          qj = 0.0;
        }
      }
      if (a.diag_probs && j < diag_pos) {
        double* d = a.diag_probs + ((static_cast<int64_t>(b) * 2 + stage) * diag_pos + j) * 2;
        d[0] = j < n ? pj : NAN;
        d[1] = j < n ? qj : NAN;
      }
      if (a.diag_uniforms && j < diag_pos) {
        float* d = a.diag_uniforms + ((static_cast<int64_t>(b) * 2 + stage) * diag_pos + j) * 2;
        d[0] = u;
        d[1] = v;
      }
      const unsigned long long rm = __ballot(reject);
      // windows of `window` positions, examined in order
      int acc = n;
      for (int w0 = 0; w0 < n; w0 += window) {
        const int w1 = min(n, w0 + window);
        const unsigned long long wm =
            (w1 - w0 >= 64 ? ~0ull : ((1ull << (w1 - w0)) - 1ull)) << w0;
        if (rm & wm) {
          acc = __ffsll(rm & wm) - 1;
          break;
        }
      }
      if (lane == 0) sm.sh[0] = acc;
    }
    __syncthreads();
    const int r = sm.sh[0];
    __syncthreads();
    return r;
  }

  // Correction (has_q) or bonus token at position apos, drawn with sm.vs[apos].
  // Uniform across the workgroup.
  __device__ int correct(int qe, int pe, int apos, bool has_q, int stage) {
    DrawResult r;
    int y;
    if (greedy) {
      y = sm.st[pe][apos].amax;
      r.R = r.t = r.c_lo = r.c_hi = NAN;
    } else {
      const float v = sm.vs[apos];
      const char* pr = row_ptr(pe, apos);
      const char* qr = has_q ? row_ptr(qe, apos) : nullptr;
      r = draw_tokens<DT>(pr, sm.st[pe][apos], qr, has_q ? sm.st[qe][apos] : sm.st[pe][apos],
                          has_q, s, V, v, sm);
      if (r.y < 0)   // no residual mass: draw from p
        r = draw_tokens<DT>(pr, sm.st[pe][apos], nullptr, sm.st[pe][apos], false, s, V, v, sm);
      y = r.y;
    }
    if (a.diag_draws && threadIdx.x == 0) {
      double* d = a.diag_draws + (static_cast<int64_t>(b) * 2 + stage) * 4;
      d[0] = r.R;
      d[1] = r.t;
      d[2] = r.c_lo;
      d[3] = r.c_hi;
    }
    return y;
  }

  __device__ void write_outputs(int emitted_n, int last_tok, int a1, int a2) {
    const int tid = threadIdx.x;
    if (tid <= k) {
      int t = -1;
      if (tid < emitted_n - 1) t = sm.toks[tid];
      else if (tid == emitted_n - 1) t = last_tok;
      a.out_tokens[static_cast<int64_t>(b) * (k + 1) + tid] = t;
    }
    if (tid == 0) {
      a.accept_len[b] = a1;
      if (a.accept_len_final) a.accept_len_final[b] = a2;
      a.num_emitted[b] = emitted_n;
      if (a.num_drop) a.num_drop[b] = k - (emitted_n - 1);
    }
  }
};

// Stage 1 (or the single stage): q = exit 0, p = exit 1.  For the hierarchy
// the result (a1, y) goes to the workspace; returns true when this workgroup
// must also run stage 2 (its L_f rows are already complete).
template <int DT>
__device__ bool verify_stage1(const FusedArgs& a, int b, VerifyShared& sm) {
  SeqCtx<DT> cx(a, sm, b);
  const int tid = threadIdx.x, k = a.k;
  const int diag_pos = k + 1;
  if (tid >= kWave && tid < kWave + k) sm.toks[tid - kWave] = a.tokens[static_cast<int64_t>(b) * k + tid - kWave];
  if (tid >= 2 * kWave && tid < 2 * kWave + 8 && a.diag_draws)
    a.diag_draws[static_cast<int64_t>(b) * 8 + tid - 2 * kWave] = NAN;
  if (!a.hier && tid >= 3 * kWave && tid < 3 * kWave + diag_pos) {
    const int j = tid - 3 * kWave;
    if (a.diag_probs) {
      double* d = a.diag_probs + ((static_cast<int64_t>(b) * 2 + 1) * diag_pos + j) * 2;
      d[0] = d[1] = NAN;
    }
    if (a.diag_uniforms) {
      float* d = a.diag_uniforms + ((static_cast<int64_t>(b) * 2 + 1) * diag_pos + j) * 2;
      d[0] = d[1] = NAN;
    }
  }
  cx.merge(0, k);
  __syncthreads();
  cx.merge(1, k + 1);
  __syncthreads();
  const int a1 = cx.decide(0, 1, k, 0, true, k > 0 ? k : 1);
  const int y = cx.correct(0, 1, a1, a1 < k, 0);
  if (!a.hier) {
    cx.write_outputs(a1 + 1, y, a1, -1);
    return false;
  }
  __shared__ int last;
  if (tid == 0) {
    a.accept_len[b] = a1;
    publish_u64(a.st1 + b, static_cast<uint64_t>(static_cast<uint32_t>(a1)) |
                               (static_cast<uint64_t>(static_cast<uint32_t>(y)) << 32));
    const int old = atomicAdd(&a.cnt2[b], 1);
    last = (old == a.n2);
  }
  __syncthreads();
  return last != 0;
}

// Stage 2 of the hierarchy: tentative t = (x_0..x_{a1-1}, y), q = L_i, p = L_f.
template <int DT>
__device__ void verify_stage2(const FusedArgs& a, int b, VerifyShared& sm) {
  SeqCtx<DT> cx(a, sm, b);
  const int tid = threadIdx.x, k = a.k;
  const uint64_t r1 = fetch_u64(a.st1 + b);
  const int a1 = static_cast<int>(static_cast<uint32_t>(r1));
  const int y = static_cast<int>(static_cast<uint32_t>(r1 >> 32));
  const int n2 = a1 + 1;
  if (tid < a1) sm.toks[tid] = a.tokens[static_cast<int64_t>(b) * k + tid];
  if (tid == a1) sm.toks[tid] = y;
  cx.merge(1, n2);
  __syncthreads();
  cx.merge(2, n2);
  __syncthreads();
  const int a2 = cx.decide(1, 2, n2, 1, false, a.window);
  int emitted_n, last_tok;
  if (a2 < n2) {
    last_tok = cx.correct(1, 2, a2, true, 1);
    emitted_n = a2 + 1;
  } else {
    last_tok = y;
    emitted_n = n2;
  }
  cx.write_outputs(emitted_n, last_tok, a1, a2);
}

}  // namespace sv
