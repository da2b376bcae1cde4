// Per-sequence verification (one verification stage, all sequences).
//
// A launch runs as B * ns workgroups, ns slices of the vocabulary per sequence.
// Every workgroup of a sequence first takes the stage's decision itself (the
// same bits in every slice):
//   1. merge the chunk partials of the sequence's rows into (reference c,
//      sum S) or (max, argmax) per (exit, position);
//   2. wavefront 0, lane j = position j: gather the logits of the drafted
//      token in the draft and target rows, p(x) and q(x), one Philox4x32-10
//      block for (j, b, stage, offset), accept iff u * q(x) < p(x); a ballot
//      gives the first rejection (windows of the given size examined in order).
// Then each workgroup sums the draw weights -- max(0, p - q) for a correction,
// p for the bonus -- over its slice of tiles (one 16-byte load per lane and
// row per tile; 128 tiles per slice, 64 for the hierarchy's joint draw of y
// and z), and the last workgroup of the sequence locates the token: an fp64
// scan of the tile sums, then one wavefront rescans the chosen tile.
//
// Stage 1 (or the single stage) compares the draft exit with the target exit;
// stage 2 of the hierarchy compares L_i with L_f on the tentative tokens (HiSpec
// summary, section 2 "Kernmechanismus" and bullet "Verlustfreie Garantie").  The
// rule is the standard speculative-sampling rule; the residual follows the SSD
// summary (section 3.B) and the bonus token its section 2 item 1.
#pragma once

#include "sv_args.h"

namespace sv {

// Tiles each wavefront of a draw loads before summing them.
constexpr int kDrawGroup = 4;

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
  // draw tile sums of the one-workgroup fallback draw; also the staging area
  // of the chunk partials when they are merged
  alignas(16) float tiles[kMaxTiles];
  RowStat st[3][kMaxPositions];
  int iscr[8];
  double dscr[8];
  int toks[kMaxPositions];   // tokens of the current stage
  float vs[kMaxPositions];   // draw uniforms of the last chain decided
  float vs1[kMaxPositions];  // stage-1 draw uniforms (hierarchy)
  float vs2[kMaxPositions];  // stage-2 draw uniforms (hierarchy)
  float us2[kMaxPositions];  // stage-2 accept uniforms (hierarchy)
  DrawResult pr[2];          // draws located side by side by two wavefronts
  int sh[8];
};
static_assert(sizeof(float) * kMaxTiles >= 1024 * sizeof(Partial), "partial staging");

template <int DT>
struct RowT {
  static constexpr int VPE = DT == 1 ? 8 : 4;
  static constexpr int ES = DT == 1 ? 2 : 4;
};

// Sum over the wavefront of one float per lane, returned to every lane.  DPP
// moves (VALU only, no LDS round trip): an inclusive scan within each row of 16
// lanes (row_shr 1, 2, 4, 8), then row 1 and 3 add the last lane of the row
// before (row_bcast 15) and rows 2 and 3 that of row 1 (row_bcast 31); lane
// 63 then holds the total.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf,
                                                         false));
}
__device__ __forceinline__ float wave_total(float v) {
  v = dpp_add<0x111, 0xf>(v);   // row_shr:1
  v = dpp_add<0x112, 0xf>(v);   // row_shr:2
  v = dpp_add<0x114, 0xf>(v);   // row_shr:4
  v = dpp_add<0x118, 0xf>(v);   // row_shr:8
  v = dpp_add<0x142, 0xa>(v);   // row_bcast:15
  v = dpp_add<0x143, 0xc>(v);   // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));   // the bits, not a cast
}

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

  // Sums of the draw weights over tiles [t_begin, t_end) of one row (pair),
  // written to out[t] (device-scope stores, staged in LDS at `stage`, when
  // `coherent`; plain LDS stores otherwise).  Tiles
  // that lie wholly inside the row are read as 16-byte vectors: each wavefront
  // takes groups of G consecutive tiles, and the loads of its next group are in
  // flight while the current group is summed.  Every load of that loop is
  // unconditional (an index past the last whole tile reloads that tile, an
  // absent q row reads the p row), so the compiler waits only for the group it
  // sums; they are nontemporal, as in the statistics stream (the rows are read
  // once more at most, by the one-tile rescan).  The ragged last tile, and
  // misaligned rows, go element by element.
  template <int DT>
  __device__ __forceinline__ void tile_pass(const char* prow, const RowStat& ps, const char* qrow,
                            const RowStat& qs, bool has_q, float s, int V, int t_begin, int t_end,
                            float* out, bool coherent, float* stage) {
    constexpr int VPE = RowT<DT>::VPE;
    constexpr int ES = RowT<DT>::ES;
    constexpr int TE = kWave * VPE;
    constexpr int G = kDrawGroup;
    constexpr int stride = kWaves * G;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    // uniform across the wavefront (scalar), so the tile loop is not divergent
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const char* qsrc = has_q ? qrow : prow;
    const bool vec_ok = ((reinterpret_cast<uintptr_t>(prow) | reinterpret_cast<uintptr_t>(qsrc)) &
                         15) == 0;
    const float cp = ps.key, isp = ps.inv_S;
    const float cq = has_q ? qs.key : 0.0f, isq = has_q ? qs.inv_S : 0.0f;
    // sums go to LDS inside the loops (LDS stores do not hold up the wait on
    // the next group's loads); global sums are copied out afterwards
    auto put = [&](int t, float v) {
      if (coherent) stage[t - t_begin] = v;
      else out[t] = v;
    };
    // loop bounds are uniform: keep them scalar so the loops are not divergent
    t_begin = __builtin_amdgcn_readfirstlane(t_begin);
    t_end = __builtin_amdgcn_readfirstlane(t_end);
    const int t_full =
        __builtin_amdgcn_readfirstlane(vec_ok ? max(t_begin, min(t_end, V / TE)) : t_begin);

    auto fetch = [&](int t0, u32x4 (&vp)[G], u32x4 (&vq)[G]) {
  #pragma unroll
      for (int g = 0; g < G; ++g) {
        const int t = min(t0 + g, t_full - 1);
        const int64_t off = static_cast<int64_t>(t * TE + lane * VPE) * ES;
        vp[g] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(prow + off));
        vq[g] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qsrc + off));
      }
    };
    auto reduce = [&](int t0, const u32x4 (&vp)[G], const u32x4 (&vq)[G]) {
      float sums[G];
  #pragma unroll
      for (int g = 0; g < G; ++g) {
        float xp[VPE], xq[VPE];
        unpack_vec<DT>(vp[g], xp);
        unpack_vec<DT>(vq[g], xq);
        sums[g] = wave_total(lane_weight_sum<DT>(xp, xq, s, cp, isp, cq, isq, has_q));
      }
      if (lane == 0) {
  #pragma unroll
        for (int g = 0; g < G; ++g)
          if (t0 + g < t_full) put(t0 + g, sums[g]);
      }
    };
    if (t_full > t_begin) {
      int t = t_begin + wave * G;
      u32x4 ap[G], aq[G], bp[G], bq[G];
      fetch(t, ap, aq);
      while (t < t_full) {
        fetch(t + stride, bp, bq);
        __builtin_amdgcn_sched_barrier(0);   // the next group's loads go out first
        reduce(t, ap, aq);
        t += stride;
        if (t >= t_full) break;
        fetch(t + stride, ap, aq);
        __builtin_amdgcn_sched_barrier(0);
        reduce(t, bp, bq);
        t += stride;
      }
    }
    // tiles past the whole-vector range: element loads
    for (int t = t_full + wave; t < t_end; t += kWaves) {
      float xp[VPE], xq[VPE];
      const int e = t * TE + lane * VPE;
      load_group<DT>(prow, e, V, vec_ok, xp);
      if (has_q) load_group<DT>(qrow, e, V, vec_ok, xq);
      else
  #pragma unroll
        for (int q = 0; q < VPE; ++q) xq[q] = 0.0f;
      const float sum = wave_total(lane_weight_sum<DT>(xp, xq, s, cp, isp, cq, isq, has_q));
      if (lane == 0) put(t, sum);
    }
    if (coherent) {
      __syncthreads();
      for (int i = tid; i < t_end - t_begin; i += kThreads) store_coherent(out + t_begin + i, stage[i]);
    }
  }

  // The hierarchy's two draws at one position in one pass: over tiles
  // [t_begin, t_end), the weights of y (p = L_i, q = L_d, or L_i alone for the
  // bonus) and of z (p = L_f, q = L_i) are summed per tile from one read of each
  // of the three rows and stored (device-scope, staged in LDS at `stage`) to
  // out_y[t] and out_z[t].  Same pipelining as tile_pass.
  template <int DT>
  __device__ __forceinline__ void tile_pass_joint(const char* irow, const RowStat& ist,
                                                  const char* drow, const RowStat& dst, bool has_d,
                                                  const char* frow, const RowStat& fst, float s,
                                                  int V, int t_begin, int t_end, float* out_y,
                                                  float* out_z, float* stage) {
    constexpr int VPE = RowT<DT>::VPE;
    constexpr int ES = RowT<DT>::ES;
    constexpr int TE = kWave * VPE;
    constexpr int G = 2;
    constexpr int stride = kWaves * G;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    // uniform across the wavefront (scalar), so the tile loop is not divergent
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const char* dsrc = has_d ? drow : irow;
    const bool vec_ok = ((reinterpret_cast<uintptr_t>(irow) | reinterpret_cast<uintptr_t>(frow) |
                          reinterpret_cast<uintptr_t>(dsrc)) & 15) == 0;
    const float ci = ist.key, isi = ist.inv_S, cf = fst.key, isf = fst.inv_S;
    const float cd = has_d ? dst.key : 0.0f, isd = has_d ? dst.inv_S : 0.0f;
    // loop bounds are uniform: keep them scalar so the loops are not divergent
    t_begin = __builtin_amdgcn_readfirstlane(t_begin);
    t_end = __builtin_amdgcn_readfirstlane(t_end);
    const int t_full =
        __builtin_amdgcn_readfirstlane(vec_ok ? max(t_begin, min(t_end, V / TE)) : t_begin);

    auto sums = [&](const float (&xi)[VPE], const float (&xd)[VPE], const float (&xf)[VPE],
                    float& sy, float& sz) {
      sy = wave_total(lane_weight_sum<DT>(xi, xd, s, ci, isi, cd, isd, has_d));
      sz = wave_total(lane_weight_sum<DT>(xf, xi, s, cf, isf, ci, isi, true));
    };
    auto fetch = [&](int t0, u32x4 (&vi)[G], u32x4 (&vd)[G], u32x4 (&vf)[G]) {
  #pragma unroll
      for (int g = 0; g < G; ++g) {
        const int t = min(t0 + g, t_full - 1);
        const int64_t off = static_cast<int64_t>(t * TE + lane * VPE) * ES;
        vi[g] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(irow + off));
        vf[g] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(frow + off));
        vd[g] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(dsrc + off));
      }
    };
    auto reduce = [&](int t0, const u32x4 (&vi)[G], const u32x4 (&vd)[G], const u32x4 (&vf)[G]) {
      float sy[G], sz[G];
  #pragma unroll
      for (int g = 0; g < G; ++g) {
        float xi[VPE], xd[VPE], xf[VPE];
        unpack_vec<DT>(vi[g], xi);
        unpack_vec<DT>(vf[g], xf);
        unpack_vec<DT>(vd[g], xd);
        sums(xi, xd, xf, sy[g], sz[g]);
      }
      if (lane == 0) {
  #pragma unroll
        for (int g = 0; g < G; ++g) {
          if (t0 + g < t_full) {
            stage[2 * (t0 + g - t_begin)] = sy[g];
            stage[2 * (t0 + g - t_begin) + 1] = sz[g];
          }
        }
      }
    };
    if (t_full > t_begin) {
      int t = t_begin + wave * G;
      u32x4 ai[G], ad[G], af[G], bi[G], bd[G], bf[G];
      fetch(t, ai, ad, af);
      while (t < t_full) {
        fetch(t + stride, bi, bd, bf);
        __builtin_amdgcn_sched_barrier(0);   // the next group's loads go out first
        reduce(t, ai, ad, af);
        t += stride;
        if (t >= t_full) break;
        fetch(t + stride, ai, ad, af);
        __builtin_amdgcn_sched_barrier(0);
        reduce(t, bi, bd, bf);
        t += stride;
      }
    }
    for (int t = t_full + wave; t < t_end; t += kWaves) {
      float xi[VPE], xd[VPE], xf[VPE];
      const int e = t * TE + lane * VPE;
      load_group<DT>(irow, e, V, vec_ok, xi);
      load_group<DT>(frow, e, V, vec_ok, xf);
      if (has_d) load_group<DT>(drow, e, V, vec_ok, xd);
      else
  #pragma unroll
        for (int q = 0; q < VPE; ++q) xd[q] = 0.0f;
      float sy, sz;
      sums(xi, xd, xf, sy, sz);
      if (lane == 0) {
        stage[2 * (t - t_begin)] = sy;
        stage[2 * (t - t_begin) + 1] = sz;
      }
    }
    __syncthreads();
    for (int i = tid; i < 2 * (t_end - t_begin); i += kThreads)
      store_coherent((i & 1 ? out_z : out_y) + t_begin + (i >> 1), stage[i]);
  }

  // Inverse CDF over NT tile sums (from LDS, or coherent loads from global when
  // `coherent`): y = the smallest index with C(y) > v * R, or, when rounding
  // leaves none, the largest index with a positive weight; y = -1 when R == 0.
  // One wavefront does the work (lane l owns a contiguous run of tiles: fp64
  // lane sums, a wavefront scan, then a rescan of the chosen tile); the result
  // is the same in every lane of that wavefront.
  template <int DT>
  __device__ __forceinline__ DrawResult locate_wave(const char* prow, const RowStat& ps,
                                                    const char* qrow, const RowStat& qs, bool has_q,
                                                    float s, int V, float v, int NT,
                                                    const float* tiles, bool coherent) {
    constexpr int VPE = RowT<DT>::VPE;
    constexpr int TE = kWave * VPE;
    const int lane = threadIdx.x & (kWave - 1);
    const bool vec_ok = ((reinterpret_cast<uintptr_t>(prow) |
                          (has_q ? reinterpret_cast<uintptr_t>(qrow) : 0)) & 15) == 0;
    const float cp = ps.key, isp = ps.inv_S;
    const float cq = has_q ? qs.key : 0.0f, isq = has_q ? qs.inv_S : 0.0f;
    auto tile_at = [&](int i) -> float { return coherent ? load_coherent(tiles + i) : tiles[i]; };
    const int per = (NT + kWave - 1) / kWave;
    const int lo = min(NT, lane * per), hi = min(NT, lo + per);
    double mine = 0.0;
    for (int i = lo; i < hi; ++i) mine += static_cast<double>(tile_at(i));
    double incl = mine;
  #pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const double up = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += up;
    }
    const double R = __shfl(incl, kWave - 1, kWave);
    const double up1 = __shfl_up(incl, 1, kWave);
    const double excl = lane > 0 ? up1 : 0.0;
    const double tv = static_cast<double>(v) * R;
    int y = -1;
    double c_lo = 0.0, c_hi = 0.0;
    if (R > 0.0) {
      // The chosen token has a positive weight, so only tiles with a positive
      // sum can hold it (this also absorbs rounding between the lanes' runs).
      int cross_t = -1, last_t = -1;
      double cross_base = 0.0, last_base = 0.0, run = excl;
      for (int i = lo; i < hi; ++i) {
        const float ti = tile_at(i);
        const double nxt = run + static_cast<double>(ti);
        if (ti > 0.0f) {
          if (cross_t < 0 && nxt > tv) {
            cross_t = i;
            cross_base = run;
          }
          last_t = i;
          last_base = run;
        }
        run = nxt;
      }
      const unsigned long long cmask = __ballot(cross_t >= 0);
      const bool overrun = cmask == 0;
      int TT;
      double base;
      if (!overrun) {
        const int src = __ffsll(cmask) - 1;
        TT = __shfl(cross_t, src, kWave);
        base = __shfl(cross_base, src, kWave);
      } else {
        const unsigned long long lmask = __ballot(last_t >= 0);
        const int src = 63 - __clzll(lmask);
        TT = __shfl(last_t, src, kWave);
        base = __shfl(last_base, src, kWave);
      }
      // rescan tile TT element by element in fp64
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
      double li = lsum;   // inclusive prefix of lane sums
  #pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const double up = __shfl_up(li, o, kWave);
        if (lane >= o) li += up;
      }
      const double lup = __shfl_up(li, 1, kWave);
      double r2 = base + (lane > 0 ? lup : 0.0);
      int cross = -1, lastpos = -1;
      double x_lo = 0.0, x_hi = 0.0, l_lo = 0.0, l_hi = 0.0;
  #pragma unroll
      for (int q = 0; q < VPE; ++q) {
        const double nxt = r2 + static_cast<double>(w[q]);
        if (w[q] > 0.0f) {
          if (!overrun && cross < 0 && nxt > tv) {
            cross = q;
            x_lo = r2;
            x_hi = nxt;
          }
          lastpos = q;
          l_lo = r2;
          l_hi = nxt;
        }
        r2 = nxt;
      }
      const unsigned long long xm = __ballot(cross >= 0);
      if (xm) {
        const int src = __ffsll(xm) - 1;
        y = TT * TE + src * VPE + __shfl(cross, src, kWave);
        c_lo = __shfl(x_lo, src, kWave);
        c_hi = __shfl(x_hi, src, kWave);
      } else {
        // no crossing: the last element of the tile with a positive weight
        const unsigned long long pm = __ballot(lastpos >= 0);
        const int src = pm ? 63 - __clzll(pm) : 0;
        const int yq = __shfl(lastpos, src, kWave);
        c_lo = __shfl(l_lo, src, kWave);
        c_hi = __shfl(l_hi, src, kWave);
        y = pm ? TT * TE + src * VPE + yq : -1;
      }
    }
    DrawResult res;
    res.y = y;
    res.R = R;
    res.t = tv;
    res.c_lo = c_lo;
    res.c_hi = c_hi;
    return res;
  }

  // locate_wave on wavefront 0, result returned to every thread (all threads
  // call it; it contains barriers).
  template <int DT>
  __device__ __forceinline__ DrawResult locate(const char* prow, const RowStat& ps, const char* qrow,
                               const RowStat& qs, bool has_q, float s, int V, float v, int NT,
                               const float* tiles, bool coherent, VerifyShared& sm) {
    if (threadIdx.x < kWave) {
      const DrawResult r = locate_wave<DT>(prow, ps, qrow, qs, has_q, s, V, v, NT, tiles, coherent);
      if (threadIdx.x == 0) sm.pr[0] = r;
    }
    __syncthreads();
    const DrawResult res = sm.pr[0];
    __syncthreads();   // scratch may be reused by the caller
    return res;
  }

  // A whole draw by one workgroup (the rare R == 0 fallback to p).
  template <int DT>
  __device__ __attribute__((noinline)) DrawResult draw_tokens(const char* prow, const RowStat& ps, const char* qrow,
                                    const RowStat& qs, bool has_q, float s, int V, float v,
                                    VerifyShared& sm) {
    constexpr int TE = kWave * RowT<DT>::VPE;
    const int NT = (V + TE - 1) / TE;
    tile_pass<DT>(prow, ps, qrow, qs, has_q, s, V, 0, NT, sm.tiles, false, nullptr);
    __syncthreads();
    return locate<DT>(prow, ps, qrow, qs, has_q, s, V, v, NT, sm.tiles, false, sm);
  }

  __device__ __forceinline__ RowStat merge_row(const Partial* pp, int nc, bool greedy) {
    RowStat r;
    if (greedy) {
      r.key = -INFINITY;
      r.amax = 0x7fffffff;
      for (int c = 0; c < nc; ++c) {
        const Partial q = pp[c];
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
      for (int c = 0; c < nc; ++c) cm = fmaxf(cm, pp[c].key);
      double S = 0.0;
      for (int c = 0; c < nc; ++c) {
        const Partial q = pp[c];
        if (q.S > 0.0) S += q.S * exp2(static_cast<double>(q.key) - static_cast<double>(cm));
      }
      r.key = cm;
      r.amax = -1;
      r.S = S;
      r.inv_S = static_cast<float>(1.0 / S);
    }
    return r;
  }

  // Per-sequence context of one verification stage.
  template <int DT>
  struct SeqCtx {
    const VerifyArgs& a;
    VerifyShared& sm;
    int b, k, V;
    bool greedy;
    bool rep;   // this workgroup reports the sequence's diagnostics
    float s;

    __device__ SeqCtx(const VerifyArgs& a_, VerifyShared& sm_, int b_, bool report)
        : a(a_), sm(sm_), b(b_), rep(report) {
      k = a.k;
      V = a.V;
      const float tau = a.temperature ? a.temperature[b] : 1.0f;
      const bool bad_tau = !(tau >= 0.0f) || !(tau < INFINITY);
      greedy = !(tau > 0.0f) || bad_tau;
      s = greedy ? 0.0f : kLog2e / tau;
      if (report && bad_tau && threadIdx.x == 0) atomicOr(a.flags, kFlagTemperature);
    }

    // Logits of each drafted token in the rows at its position (wavefront 0,
    // lane j < k), loaded before the statistics merge so that the two memory
    // latencies overlap; the LM-head path reads them from `gath`.
    float g[3] = {0.0f, 0.0f, 0.0f};

    __device__ void pregather(int nexits) {
      const int j = threadIdx.x;
      if (j >= k || greedy) return;
      const int x = a.tokens[static_cast<int64_t>(b) * k + j];
      if (x < 0 || x >= V) return;
      auto at = [&](int e) {
        return a.gath ? a.gath[row_index(e, j)] : load_elem(row_ptr(e, j), x, DT);
      };
      g[0] = at(0);
      g[1] = at(1);
      if (nexits > 2) g[2] = at(2);
    }
    __device__ float gathered(int e) const { return e == 0 ? g[0] : (e == 1 ? g[1] : g[2]); }

    __device__ int positions(int e) const { return e == 0 ? k : k + 1; }

    __device__ int64_t row_index(int e, int j) const {
      return a.exit_row0[e] + static_cast<int64_t>(b) * positions(e) + j;
    }

    __device__ const char* row_ptr(int e, int j) const {
      return static_cast<const char*>(a.exit_ptr[e]) +
             (static_cast<int64_t>(b) * positions(e) + j) * a.ld * RowT<DT>::ES;
    }

    // Export of a merged row's statistics (the reporting workgroup only).
    __device__ void export_row(int64_t row, const RowStat& r) const {
      if (!rep) return;
      if (a.row_log2z)
        a.row_log2z[row] = greedy || !(r.S > 0.0) ? NAN : static_cast<double>(r.key) + log2(r.S);
      if (a.row_argmax) a.row_argmax[row] = greedy ? r.amax : -1;
    }

    // Merged statistics of positions [0, n) of exit e into sm.st[e]; threads
    // [t0, t0 + n) do the work.
    __device__ void merge(int e, int n, int t0) {
      const int t = static_cast<int>(threadIdx.x) - t0;
      if (t >= 0 && t < n) {
        const int64_t row = a.exit_row0[e] + static_cast<int64_t>(b) * positions(e) + t;
        sm.st[e][t] = merge_row(a.partials + row * a.nc, a.nc, greedy);
        export_row(row, sm.st[e][t]);
      }
    }

    // Merged statistics of positions [0, n_e) of exits 0..2 (n_e = 0 to skip an
    // exit): every chunk partial is loaded once, one thread per partial, into
    // LDS, then one thread per row merges its chunks.  All threads.
    __device__ void merge_all(int n0, int n1, int n2) {
      const int tid = threadIdx.x;
      const int nc = a.nc;
      const int rows = n0 + n1 + n2;
      if (rows * nc > 1024) {   // too many chunks to stage: merge straight from memory
        merge(0, n0, 0);
        merge(1, n1, kWave);
        __syncthreads();
        merge(2, n2, 0);
        __syncthreads();
        return;
      }
      Partial* stage = reinterpret_cast<Partial*>(sm.tiles);
      for (int i = tid; i < rows * nc; i += kThreads) {
        const int r = i / nc, c = i - r * nc;
        const int e = r < n0 ? 0 : (r < n0 + n1 ? 1 : 2);
        const int j = r - (e == 0 ? 0 : (e == 1 ? n0 : n0 + n1));
        const int64_t row = a.exit_row0[e] + static_cast<int64_t>(b) * positions(e) + j;
        stage[i] = a.partials[row * nc + c];
      }
      __syncthreads();
      if (tid < rows) {
        const int e = tid < n0 ? 0 : (tid < n0 + n1 ? 1 : 2);
        const int j = tid - (e == 0 ? 0 : (e == 1 ? n0 : n0 + n1));
        sm.st[e][j] = merge_row(stage + tid * nc, nc, greedy);
        export_row(row_index(e, j), sm.st[e][j]);
      }
      __syncthreads();
    }

    // Both stages' decisions over the drafted tokens at once (hierarchy): stage 1
    // tests x_j with q = L_d, p = L_i (a1 = first rejection, else k); stage 2
    // tests x_j, j < a1, with q = L_i, p = L_f in windows of `window`
    // (returned a2p = first rejection before a1, else a1).  Stage 2's test of x_j
    // is the one it would make on the tentative tokens, since t_j = x_j for
    // j < a1.  One gather of L_d, L_i, L_f at x_j per lane.  Fills vs1, vs2, us2.
    __device__ int2 decide_pre(int window, bool diag) {
      const int tid = threadIdx.x, lane = tid & (kWave - 1);
      const int diag_pos = k + 1;
      if (tid < kWave) {
        const int j = lane;
        bool rej1 = false, rej2 = false;
        float u1 = NAN, v1 = NAN, u2 = NAN, v2 = NAN;
        double p1 = NAN, q1 = NAN, p2 = NAN, q2 = NAN;
        if (j <= k) {
          const uint4 w1 = philox4x32_10(make_uint4(j, b, 0u, a.offset), a.key0, a.key1);
          const uint4 w2 = philox4x32_10(make_uint4(j, b, 1u, a.offset), a.key0, a.key1);
          u1 = uniform24(w1.x);
          v1 = uniform24(w1.y);
          u2 = uniform24(w2.x);
          v2 = uniform24(w2.y);
          sm.vs1[j] = v1;
          sm.vs2[j] = v2;
          sm.us2[j] = u2;
        }
        if (j < k) {
          const int x = sm.toks[j];
          const bool valid = x >= 0 && x < V;
          if (!valid && diag) atomicOr(a.flags, kFlagTokenRange);
          if (greedy) {
            const bool mi = valid && x == sm.st[1][j].amax;
            const bool mf = valid && x == sm.st[2][j].amax;
            rej1 = !mi;
            rej2 = !mf;
            p1 = q2 = mi ? 1.0 : 0.0;
            q1 = valid && x == sm.st[0][j].amax ? 1.0 : 0.0;
            p2 = mf ? 1.0 : 0.0;
          } else if (valid) {
            const float ld = g[0];
            const float li = g[1];
            const float lf = g[2];
            q1 = static_cast<double>(__builtin_amdgcn_exp2f(fmaf(ld, s, -sm.st[0][j].key))) /
                 sm.st[0][j].S;
            p1 = static_cast<double>(__builtin_amdgcn_exp2f(fmaf(li, s, -sm.st[1][j].key))) /
                 sm.st[1][j].S;
            p2 = static_cast<double>(__builtin_amdgcn_exp2f(fmaf(lf, s, -sm.st[2][j].key))) /
                 sm.st[2][j].S;
            q2 = p1;
            rej1 = !(static_cast<double>(u1) * q1 < p1);
            rej2 = !(static_cast<double>(u2) * q2 < p2);
          } else {
            rej1 = rej2 = true;
            p1 = q1 = p2 = q2 = 0.0;
          }
        }
        const unsigned long long m1 = __ballot(rej1);
        const int a1 = m1 ? min(k, __ffsll(m1) - 1) : k;
        const unsigned long long m2 = __ballot(rej2);
        int a2p = a1;
        for (int w0 = 0; w0 < a1; w0 += window) {   // windows examined in order
          const int w1 = min(a1, w0 + window);
          const unsigned long long wm =
              (w1 - w0 >= 64 ? ~0ull : ((1ull << (w1 - w0)) - 1ull)) << w0;
          if (m2 & wm) {
            a2p = __ffsll(m2 & wm) - 1;
            break;
          }
        }
        if (diag && j < diag_pos) {
          const int64_t base0 = (static_cast<int64_t>(b) * 2 + 0) * diag_pos + j;
          const int64_t base1 = (static_cast<int64_t>(b) * 2 + 1) * diag_pos + j;
          if (a.diag_probs) {
            // tested positions only: stage 1 stops at a1, stage 2 at a2
            const bool t1 = j < k && j <= a1, t2 = j < a1 && j <= a2p;
            a.diag_probs[base0 * 2] = t1 ? p1 : NAN;
            a.diag_probs[base0 * 2 + 1] = t1 ? q1 : NAN;
            // position a1 of stage 2 belongs to the test of y when it happens
            // (one writer per entry: stores from different XCDs are not ordered)
            if (j != a1 || a2p < a1) {
              a.diag_probs[base1 * 2] = t2 ? p2 : NAN;
              a.diag_probs[base1 * 2 + 1] = t2 ? q2 : NAN;
            }
          }
          if (a.diag_uniforms) {
            a.diag_uniforms[base0 * 2] = u1;
            a.diag_uniforms[base0 * 2 + 1] = v1;
            a.diag_uniforms[base1 * 2] = j <= a1 ? u2 : NAN;
            a.diag_uniforms[base1 * 2 + 1] = j <= a1 ? v2 : NAN;
          }
        }
        if (lane == 0) {
          sm.sh[2] = a1;
          sm.sh[3] = a2p;
        }
      }
      __syncthreads();
      const int2 r = make_int2(sm.sh[2], sm.sh[3]);
      __syncthreads();
      return r;
    }

    // Stage 2's test of the L_i token y at position a1 (every earlier position
    // accepted): returns true when L_f accepts it.  Writes position a1's
    // stage-2 diagnostics.  All threads.
    __device__ bool accept_y(int a1, int y, bool diag) {
      const int tid = threadIdx.x;
      if (tid == 0) {
        const bool valid = y >= 0 && y < V;
        const float u2 = sm.us2[a1];
        bool acc;
        double p2 = 0.0, q2 = 0.0;
        if (greedy) {
          acc = valid && y == sm.st[2][a1].amax;
          p2 = acc ? 1.0 : 0.0;
          q2 = valid && y == sm.st[1][a1].amax ? 1.0 : 0.0;
        } else if (valid) {
          const float li = load_elem(row_ptr(1, a1), y, DT);
          const float lf = load_elem(row_ptr(2, a1), y, DT);
          q2 = static_cast<double>(__builtin_amdgcn_exp2f(fmaf(li, s, -sm.st[1][a1].key))) /
               sm.st[1][a1].S;
          p2 = static_cast<double>(__builtin_amdgcn_exp2f(fmaf(lf, s, -sm.st[2][a1].key))) /
               sm.st[2][a1].S;
          acc = static_cast<double>(u2) * q2 < p2;
        } else {
          acc = false;
        }
        if (diag && a.diag_probs) {
          double* d = a.diag_probs + ((static_cast<int64_t>(b) * 2 + 1) * (k + 1) + a1) * 2;
          d[0] = p2;
          d[1] = q2;
        }
        sm.sh[4] = acc ? 1 : 0;
      }
      __syncthreads();
      const bool r = sm.sh[4] != 0;
      __syncthreads();
      return r;
    }

    // One verification chain over tokens sm.toks[0..n): q rows of exit qe, p rows
    // of exit pe, Philox stage `stage`.  Returns the accept count; leaves the
    // draw uniforms in sm.vs[0..n] (position n only with a bonus).
    __device__ int decide(int qe, int pe, int n, int stage, bool bonus, int window, bool diag) {
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
          if (!valid && diag) atomicOr(a.flags, kFlagTokenRange);
          if (greedy) {
            reject = !(valid && x == sm.st[pe][j].amax);
            pj = valid && x == sm.st[pe][j].amax ? 1.0 : 0.0;
            qj = valid && x == sm.st[qe][j].amax ? 1.0 : 0.0;
          } else if (valid) {
            const float lp = gathered(pe);
            const float lq = gathered(qe);
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
        if (diag && a.diag_uniforms && j < diag_pos) {
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
        if (diag && a.diag_probs && j < diag_pos) {   // tested positions: 0..acc
          double* d = a.diag_probs + ((static_cast<int64_t>(b) * 2 + stage) * diag_pos + j) * 2;
          d[0] = j < n && j <= acc ? pj : NAN;
          d[1] = j < n && j <= acc ? qj : NAN;
        }
        if (lane == 0) sm.sh[0] = acc;
      }
      __syncthreads();
      const int r = sm.sh[0];
      __syncthreads();
      return r;
    }

    __device__ void write_draw_diag(int stage, const DrawResult& r) {
      if (a.diag_draws && threadIdx.x == 0) {
        double* d = a.diag_draws + (static_cast<int64_t>(b) * 2 + stage) * 4;
        d[0] = r.R;
        d[1] = r.t;
        d[2] = r.c_lo;
        d[3] = r.c_hi;
      }
    }

    // Outputs of a flush of c pending tokens: t_0..t_{emitted_n-2} and last_tok,
    // a2, and the pending tokens discarded (c - a2 on a rejection, else 0).
    __device__ void write_flush(int c, int emitted_n, int last_tok, int a2) {
      const int tid = threadIdx.x;
      if (tid <= k) {
        int t = -1;
        if (tid < emitted_n - 1) t = sm.toks[tid];
        else if (tid == emitted_n - 1) t = last_tok;
        a.out_tokens[static_cast<int64_t>(b) * (k + 1) + tid] = t;
      }
      if (tid == 0) {
        a.accept_len[b] = a2;
        a.num_emitted[b] = emitted_n;
        if (a.num_drop) a.num_drop[b] = a2 >= 0 && a2 < c ? c - a2 : 0;
      }
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
        const int drop = k - (emitted_n - 1);
        a.accept_len[b] = a1;
        if (a.accept_len_final) a.accept_len_final[b] = a2;
        a.num_emitted[b] = emitted_n;
        if (a.num_drop) a.num_drop[b] = drop;
        if (a.kv_lens)
          kv_rollback_one(a.kv_table + static_cast<int64_t>(b) * a.kv_max_blocks, a.kv_lens + b,
                          drop, a.kv_freed + static_cast<int64_t>(b) * a.kv_max_freed,
                          a.kv_num_freed + b, a.kv_max_blocks, a.kv_block_size,
                          a.kv_max_freed);
      }
    }
  };

  __device__ __forceinline__ void nan_draw(DrawResult& r) { r.R = r.t = r.c_lo = r.c_hi = NAN; }

  // Loads the drafted tokens of sequence b into sm.toks[0, n) (the last
  // wavefront; n <= 63).
  template <int DT>
  __device__ __forceinline__ void load_drafts(SeqCtx<DT>& cx, int n) {
    const int t = static_cast<int>(threadIdx.x) - (kWaves - 1) * kWave;
    if (t >= 0 && t < n) cx.sm.toks[t] = cx.a.tokens[static_cast<int64_t>(cx.b) * cx.k + t];
  }

  // Counts slice g of a sequence done after its tile sums were published; true
  // in the workgroup that completes the draw.  Uniform across the workgroup.
  __device__ __forceinline__ bool slice_done(int32_t* cnt, int ns, VerifyShared& sm) {
    wait_memory();
    __syncthreads();
    if (threadIdx.x == 0) sm.sh[1] = (atomicAdd(cnt, 1) == ns - 1);
    __syncthreads();
    const bool last = sm.sh[1] != 0;
    __syncthreads();
    return last;
  }

  // Sums slice g of a draw's tiles (p rows at pr, q rows at qr when has_q) and
  // counts it done; true in the workgroup that completes the draw.
  template <int DT>
  __device__ bool draw_slice(SeqCtx<DT>& cx, int g, int stage, const char* pr, const char* qr,
                             bool has_q, const RowStat& ps, const RowStat& qs) {
    const VerifyArgs& a = cx.a;
    float* tsum = a.tsum[stage] + static_cast<int64_t>(cx.b) * a.nt;
    const int t0 = g * a.tps;
    tile_pass<DT>(pr, ps, qr, qs, has_q, cx.s, cx.V, t0, min(a.nt, t0 + a.tps), tsum, true,
                  cx.sm.tiles);
    return slice_done(a.cnt[stage] + cx.b, a.ns, cx.sm);
  }

  // In the workgroup that completed a draw: locate the token from the tile sums
  // (or, with no residual mass, draw from p) and write the stage's diagnostics.
  template <int DT>
  __device__ int draw_finish(SeqCtx<DT>& cx, int stage, const char* pr, const char* qr,
                             bool has_q, const RowStat& ps, const RowStat& qs, float v) {
    const float* tsum = cx.a.tsum[stage] + static_cast<int64_t>(cx.b) * cx.a.nt;
    DrawResult r = locate<DT>(pr, ps, qr, qs, has_q, cx.s, cx.V, v, cx.a.nt, tsum, true, cx.sm);
    if (r.y < 0)   // no residual mass: draw from p
      r = draw_tokens<DT>(pr, ps, nullptr, ps, false, cx.s, cx.V, v, cx.sm);
    cx.write_draw_diag(stage, r);
    return r.y;
  }

  // The draw of one stage for sequence b at position apos (p rows of exit pe,
  // q rows of exit qe when has_q), slice `slice` of it in this workgroup.
  // Returns the token in the workgroup that completes the draw and -2 in the
  // others.  Uniform across the workgroup.
  template <int DT>
  __device__ int sliced_draw(SeqCtx<DT>& cx, int slice, int qe, int pe, int apos, bool has_q,
                             int stage, float v, const RowStat& ps, const RowStat& qs) {
    const char* pr;
    const char* qr;
    if (cx.a.draw_rows) {   // LM-head path: the recomputed rows of this sequence
      const float* base = cx.a.draw_rows + static_cast<int64_t>(cx.b) * 2 * cx.a.draw_ld;
      pr = reinterpret_cast<const char*>(base);
      qr = has_q ? reinterpret_cast<const char*>(base + cx.a.draw_ld) : nullptr;
    } else {
      pr = cx.row_ptr(pe, apos);
      qr = has_q ? cx.row_ptr(qe, apos) : nullptr;
    }
    if (!draw_slice<DT>(cx, slice, stage, pr, qr, has_q, ps, qs)) return -2;
    return draw_finish<DT>(cx, stage, pr, qr, has_q, ps, qs, v);
  }

  // One launch, grid B * ns: workgroup w of sequence b works on vocabulary slice
  // w.  Every workgroup takes stage 1's decision itself (and, for the hierarchy,
  // stage 2's decision on the drafted tokens before a1, which does not depend on
  // the L_i token y).  Then:
  //  - single stage: the correction or bonus draw;
  //  - hierarchy, stage 2 rejects drafted token a2p < a1: y is never emitted;
  //    stage 2's correction at a2p is drawn;
  //  - hierarchy otherwise: y (stage 1's correction, or its bonus) and stage 2's
  //    correction z at a1 are summed in one pass over L_d[a1], L_i[a1], L_f[a1];
  //    the workgroup completing the last slice locates y, tests it against L_f,
  //    and locates z only if L_f rejects y.
  template <int DT>
  __device__ void verify_slice(const VerifyArgs& a, int b, int slice, VerifyShared& sm) {
    const bool first = slice == 0;
    SeqCtx<DT> cx(a, sm, b, first);
    const int tid = threadIdx.x, k = a.k;
    const int diag_pos = k + 1;
    load_drafts(cx, k);
    if (first && !a.hier && tid >= (kWaves - 2) * kWave && tid < (kWaves - 2) * kWave + diag_pos) {
      // the single stage has no second stage: its diagnostics are empty
      const int j = tid - (kWaves - 2) * kWave;
      if (a.diag_probs) {
        double* d = a.diag_probs + ((static_cast<int64_t>(b) * 2 + 1) * diag_pos + j) * 2;
        d[0] = d[1] = NAN;
      }
      if (a.diag_uniforms) {
        float* d = a.diag_uniforms + ((static_cast<int64_t>(b) * 2 + 1) * diag_pos + j) * 2;
        d[0] = d[1] = NAN;
      }
    }
    int a1 = 0, a2p = 0, flush_n = 0;
    float v1 = 0.0f;
    if (a.flush_lim) {
      // flush of pending tentative tokens (stage 2 of the hierarchy, across
      // calls); a correction is drawn by the common single-stage draw below
      const int n = a.flush_lim[b] + 1;
      if (n <= 0) {   // not flushed: nothing was streamed for this sequence
        if (first) cx.write_flush(0, 0, -1, -1);
        return;
      }
      cx.pregather(2);
      cx.merge_all(n, n, 0);
      const int a2 = cx.decide(0, 1, n, 1, false, n, first);
      if (a2 == n) {   // every pending token accepted: no draw, no bonus
        if (first) cx.write_flush(n, n, sm.toks[n - 1], a2);
        return;
      }
      if (cx.greedy) {
        if (first) cx.write_flush(n, a2 + 1, sm.st[1][a2].amax, a2);
        return;
      }
      flush_n = n;
      a1 = a2p = a2;
      v1 = sm.vs[a2];
    } else {
    if (a.stage1_only) {
      // lazy call, stage 1 alone from the L_d and L_i rows of the first
      // positions: where a draft is rejected there (or the window covers every
      // draft) a1 is fixed and the L_f rows 0..a1 are listed; otherwise the
      // remaining L_d / L_i rows and every L_f row of the sequence are listed,
      // and the final pass decides stage 1 over all positions
      if (!first) return;
      const int n0 = min(a.stage1_window, k);
      cx.pregather(2);
      cx.merge_all(n0, n0 + (n0 == k ? 1 : 0), 0);
      const int s1 = cx.decide(0, 1, n0, 0, false, n0 > 0 ? n0 : 1, false);
      if (tid == 0) {
        const bool fixed = s1 < n0 || n0 == k;
        const int n_rest = fixed ? 0 : 2 * (k - n0) + 1;
        const int n_f = fixed ? s1 + 1 : k + 1;
        a.lazy_a1[b] = fixed ? s1 : -1;
        const int base = atomicAdd(a.row_count_out, n_rest + n_f);
        for (int j = n0; j < n0 + n_rest; ++j) {   // L_d rows n0..k-1, L_i rows n0..k
          const int e = j < k ? 0 : 1, pos = j < k ? j : j - (k - n0);
          a.row_list_out[base + j - n0] = static_cast<int32_t>(cx.row_index(e, pos));
        }
        for (int j = 0; j < n_f; ++j)
          a.row_list_out[base + n_rest + j] = static_cast<int32_t>(cx.row_index(2, j));
      }
      return;
    }
    cx.pregather(a.hier ? 3 : 2);
    // stage 2 reads L_f rows 0..a1 only (all of them unless the final exit is lazy)
    // (lazy: a1 where the window pass fixed it, else every L_f row was listed)
    cx.merge_all(k, k + 1, a.hier ? (a.lazy_a1 && a.lazy_a1[b] >= 0 ? a.lazy_a1[b] + 1 : k + 1) : 0);
    if (a.hier) {
      const int2 r = cx.decide_pre(a.window, first);
      a1 = r.x;
      a2p = r.y;
      v1 = sm.vs1[a1];
    } else {
      a1 = cx.decide(0, 1, k, 0, true, k > 0 ? k : 1, first);
      a2p = a1;
      v1 = sm.vs[a1];
    }
    if (a.decide_only) {
      // LM-head first pass: name the rows to recompute (target row a1, and the
      // draft row a1 for a correction); greedy sequences end here
      if (!first) return;
      if (tid == 0) {
        const bool draws = !cx.greedy;
        a.stop_rows[2 * b] = draws ? static_cast<int32_t>(cx.row_index(1, a1)) : -1;
        a.stop_rows[2 * b + 1] = draws && a1 < k ? static_cast<int32_t>(cx.row_index(0, a1)) : -1;
      }
      if (cx.greedy) cx.write_outputs(a1 + 1, sm.st[1][a1].amax, a1, -1);
      return;
    }
  }
  const bool early = a.hier && a2p < a1;   // stage 2 rejects drafted token a2p
  if (!flush_n) {
    if (first && a.diag_draws && tid < 8) {
      // draws that do not happen (the workgroup completing each draw writes the
      // others; the hierarchy's stage-2 entry is always written there)
      const int stage = tid / 4;
      const bool drawn = !cx.greedy && (stage == 0 ? !early : a.hier);
      if (!drawn) a.diag_draws[static_cast<int64_t>(b) * 8 + tid] = NAN;
    }

    if (cx.greedy) {   // argmax tokens: no draw, the first workgroup finishes
      if (!first) return;
      if (early) {
        cx.write_outputs(a2p + 1, sm.st[2][a2p].amax, a1, a2p);
        return;
      }
      const int y = sm.st[1][a1].amax;
      if (!a.hier) {
        cx.write_outputs(a1 + 1, y, a1, -1);
        return;
      }
      if (tid == 0) sm.toks[a1] = y;
      if (cx.accept_y(a1, y, true)) cx.write_outputs(a1 + 1, y, a1, a1 + 1);
      else cx.write_outputs(a1 + 1, sm.st[2][a1].amax, a1, a1);
      return;
    }

    if (a.hier && !early) {
      const bool has_q = a1 < k;
      const char* li = cx.row_ptr(1, a1);
      const char* ld = has_q ? cx.row_ptr(0, a1) : nullptr;
      const char* lf = cx.row_ptr(2, a1);
      float* ty = a.tsum[0] + static_cast<int64_t>(b) * a.nt;
      float* tz = a.tsum[1] + static_cast<int64_t>(b) * a.nt;
      const int t0 = slice * a.tps;
      const RowStat& si = sm.st[1][a1];
      const RowStat& sd = sm.st[0][has_q ? a1 : 0];
      const RowStat& sf = sm.st[2][a1];
      tile_pass_joint<DT>(li, si, ld, sd, has_q, lf, sf, cx.s, cx.V, t0, min(a.nt, t0 + a.tps),
                          ty, tz, sm.tiles);
      if (!slice_done(a.cnt[0] + b, a.ns, sm)) return;
      // y on wavefront 0 and z on wavefront 1, side by side
      const float v2 = sm.vs2[a1];
      const int wave = tid / kWave;
      if (wave < 2) {
        const DrawResult r =
            wave == 0 ? locate_wave<DT>(li, si, ld, sd, has_q, cx.s, cx.V, v1, a.nt, ty, true)
                      : locate_wave<DT>(lf, sf, li, si, true, cx.s, cx.V, v2, a.nt, tz, true);
        if ((tid & (kWave - 1)) == 0) sm.pr[wave] = r;
      }
      __syncthreads();
      DrawResult ry = sm.pr[0], rz = sm.pr[1];
      __syncthreads();
      if (ry.y < 0) ry = draw_tokens<DT>(li, si, nullptr, si, false, cx.s, cx.V, v1, sm);
      cx.write_draw_diag(0, ry);
      const int y = ry.y;
      if (tid == 0) sm.toks[a1] = y;
      if (cx.accept_y(a1, y, true)) {
        DrawResult none;
        nan_draw(none);
        cx.write_draw_diag(1, none);
        cx.write_outputs(a1 + 1, y, a1, a1 + 1);
        return;
      }
      if (rz.y < 0) rz = draw_tokens<DT>(lf, sf, nullptr, sf, false, cx.s, cx.V, v2, sm);
      cx.write_draw_diag(1, rz);
      cx.write_outputs(a1 + 1, rz.y, a1, a1);
      return;
    }

  }

  // single stage (and a flush), or the hierarchy's stage-2 correction at a2p < a1
  const int stage = early ? 1 : 0;
  const int apos = early ? a2p : a1;
  const bool has_q = early || a1 < k;
  const float v = early ? sm.vs2[a2p] : v1;
  const int tok = sliced_draw<DT>(cx, slice, stage, stage + 1, apos, has_q, stage, v,
                                  sm.st[stage + 1][apos], sm.st[stage][has_q ? apos : 0]);
  if (tok == -2) return;
  if (flush_n) cx.write_flush(flush_n, a1 + 1, tok, a1);
  else if (early) cx.write_outputs(a2p + 1, tok, a1, a2p);
  else cx.write_outputs(a1 + 1, tok, a1, -1);
}

}  // namespace sv
