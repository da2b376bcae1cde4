// Chunk statistics: the HBM stream of the verification path.
//
// Every logit row of every exit (draft / target, or L_d / L_i / L_f) is read
// once, in 64 KiB chunks.  Each of the 256 threads of a workgroup issues its 16
// nontemporal 128-bit loads up front, keeps the chunk in registers and reduces
// it to partial softmax statistics:
//   temperature > 0: c = max * s (fp32 product) and S = sum 2^(l * s - c), with
//                    s = log2(e) / temperature (fp32 exponent; fp32 pairwise sums,
//                    fp64 across vectors or, for plain bf16 rows, across threads);
//   temperature = 0: the maximum and its lowest index (greedy decoding).
// With ENT the sampled rows also give T = sum 2^(l * s - c) * (l * s - c),
// which turns the row's merged (c, S, T) into its entropy ln S - ln 2 * T / S
// at the cost of one multiply-add per element.
// The softmax of a row is the token distribution of that exit at that position
// (HiSpec summary, section 2 "Kernmechanismus": L_d, L_i and L_f each yield a
// token distribution).
#pragma once

#include "sv_common.h"

namespace sv {

struct Red {
  float key;
  int idx;
  double S;
  double T;
};

// Workgroup reduction of greedy (max, lowest index) pairs.
__device__ inline void block_argmax(float& m, int& idx, Red* lds) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(m, o, kWave);
    const int oi = __shfl_xor(idx, o, kWave);
    if (om > m || (om == m && oi < idx)) {
      m = om;
      idx = oi;
    }
  }
  if (lane == 0) {
    lds[wave].key = m;
    lds[wave].idx = idx;
  }
  __syncthreads();
  m = lds[0].key;
  idx = lds[0].idx;
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    if (lds[w].key > m || (lds[w].key == m && lds[w].idx < idx)) {
      m = lds[w].key;
      idx = lds[w].idx;
    }
  }
}

// Workgroup reduction of (c, S) partial sums: common reference max(c), then
// each S rescaled by 2^(c_t - c) in double and summed.
__device__ inline void block_logsum(float& c, double& S, Red* lds) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  float cm = wave_max(c);
  if (lane == 0) lds[wave].key = cm;
  __syncthreads();
  cm = lds[0].key;
#pragma unroll
  for (int w = 1; w < kWaves; ++w) cm = fmaxf(cm, lds[w].key);
  double Sr = 0.0;
  if (S > 0.0) Sr = S * exp2(static_cast<double>(c) - static_cast<double>(cm));
  Sr = wave_sum(Sr);
  __syncthreads();
  if (lane == 0) lds[wave].S = Sr;
  __syncthreads();
  S = lds[0].S;
#pragma unroll
  for (int w = 1; w < kWaves; ++w) S += lds[w].S;
  c = cm;
}

// The same reduction carrying T: moving a partial from reference c_t to cm
// shifts every exponent by c_t - cm, so T becomes 2^(c_t - cm) * (T + (c_t - cm) * S).
__device__ inline void block_logsum_t(float& c, double& S, double& T, Red* lds) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  float cm = wave_max(c);
  if (lane == 0) lds[wave].key = cm;
  __syncthreads();
  cm = lds[0].key;
#pragma unroll
  for (int w = 1; w < kWaves; ++w) cm = fmaxf(cm, lds[w].key);
  double Sr = 0.0, Tr = 0.0;
  if (S > 0.0) {
    const double d = static_cast<double>(c) - static_cast<double>(cm);
    const double f = exp2(d);
    Sr = S * f;
    Tr = (T + d * S) * f;
  }
  Sr = wave_sum(Sr);
  Tr = wave_sum(Tr);
  __syncthreads();
  if (lane == 0) {
    lds[wave].S = Sr;
    lds[wave].T = Tr;
  }
  __syncthreads();
  S = lds[0].S;
  T = lds[0].T;
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    S += lds[w].S;
    T += lds[w].T;
  }
  c = cm;
}

// Exponent times weight for T; a weight of 0 (l = -inf included) adds 0.
__device__ __forceinline__ float xlogw(float t, float y) { return t * fmaxf(y, -1e30f); }

template <int DT>
__device__ __forceinline__ void unpack(const u32x4& v, float (&x)[DT == 1 ? 8 : 4]) {
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

// Partial statistics of elements [e0, e1) of one row (e1 - e0 <= one chunk).
// Called by the whole workgroup (it contains barriers).  With ENT, T_out
// receives the chunk's T (0 for a greedy row).  CLAMP (with ENT): the vector
// loop clamps the exponent of each T term, so that an element of weight 0
// (l = -inf) adds 0; without it such an element makes T NaN, which the caller
// detects and answers with a clamped rescan (identical otherwise: the clamp
// only moves exponents below -1e30).
template <int DT, bool ENT, bool CLAMP = true, bool REUNPACK = ENT, bool CACHED = false>
__device__ Partial chunk_stats(const char* rowp, int e0, int e1, bool greedy, float s, Red* lds,
                               double& T_out) {
  constexpr int VPE = DT == 1 ? 8 : 4;
  const int tid = threadIdx.x;
  float m = -INFINITY;
  int idx = 0x7fffffff;
  double S = 0.0, T = 0.0;
  float c = -INFINITY;

  if ((reinterpret_cast<uintptr_t>(rowp) & 15) == 0) {
    // 16-byte aligned row: vectors [e0/VPE, e0/VPE + nfull) then < VPE scalars.
    const u32x4* vp = reinterpret_cast<const u32x4*>(rowp) + e0 / VPE;
    const int nfull = (e1 - e0) / VPE;
    const uint32_t pad = DT == 1 ? 0xff80ff80u : 0xff800000u;  // -inf
    u32x4 buf[kVecPerThread];
#pragma unroll
    for (int i = 0; i < kVecPerThread; ++i) {
      const int vi = i * kThreads + tid;
      buf[i] = vi < nfull ? (CACHED ? vp[vi] : __builtin_nontemporal_load(vp + vi))
                          : u32x4{pad, pad, pad, pad};
    }
    const int tail0 = e0 + nfull * VPE;
    const bool has_tail = tid < e1 - tail0;
    const float xt = has_tail ? load_elem(rowp, tail0 + tid, DT) : -INFINITY;

    float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
    for (int i = 0; i < kVecPerThread; ++i) {
      float x[VPE];
      unpack<DT>(buf[i], x);
#pragma unroll
      for (int q = 0; q < VPE; q += 2) {
        m0 = fmaxf(m0, x[q]);
        m1 = fmaxf(m1, x[q + 1]);
      }
    }
    m = fmaxf(fmaxf(m0, m1), xt);
    const bool empty = !(m > -INFINITY);   // no finite element in this thread's share
    // REUNPACK: unpack the vectors again for the second pass instead of
    // keeping the first pass's floats live.  The entropy stream takes it (93
    // registers instead of 159: five wavefronts per SIMD instead of three,
    // and a faster stream), and so does the looping row-list kernel; the
    // plain stream is faster keeping them (156 registers).
#pragma unroll
    for (int i = 0; i < kVecPerThread; ++i)
      if constexpr (REUNPACK) asm volatile("" : "+v"(buf[i]));

    if (greedy) {
      // lowest index attaining the thread's maximum
#pragma unroll
      for (int i = kVecPerThread - 1; i >= 0; --i) {
        float x[VPE];
        unpack<DT>(buf[i], x);
#pragma unroll
        for (int q = VPE - 1; q >= 0; --q)
          if (x[q] == m) idx = e0 + (i * kThreads + tid) * VPE + q;
      }
      if (idx == 0x7fffffff && has_tail && xt == m) idx = tail0 + tid;
      if (empty) idx = 0x7fffffff;
    } else if (!empty) {
      c = m * s;
      const float nc_ = -c;
      // bf16 without entropy sums: the vector sums are added pairwise in fp32
      // and converted once (fewer instructions at the same occupancy); the
      // other variants, whose registers are tighter, add each vector's sum
      // in fp64
      constexpr bool kTree = DT == 1 && !ENT;
      float vsum[kVecPerThread];
#pragma unroll
      for (int i = 0; i < kVecPerThread; ++i) {
        float x[VPE];
        unpack<DT>(buf[i], x);
        float t[VPE];
        float ty = 0.0f;
#pragma unroll
        for (int q = 0; q < VPE; ++q) {
          const float y = fmaf(x[q], s, nc_);
          t[q] = __builtin_amdgcn_exp2f(y);
          if constexpr (ENT) ty = fmaf(t[q], CLAMP ? fmaxf(y, -1e30f) : y, ty);
        }
        // pairwise within the vector
#pragma unroll
        for (int w = VPE / 2; w > 0; w >>= 1)
#pragma unroll
          for (int q = 0; q < w; ++q) t[q] += t[q + w];
        if constexpr (kTree) vsum[i] = t[0];
        else S += static_cast<double>(t[0]);
        // (a padding vector past the chunk adds nothing: its -inf pads would
        // make an unclamped T NaN)
        if constexpr (ENT) T += i * kThreads + tid < nfull ? static_cast<double>(ty) : 0.0;
      }
      if constexpr (kTree) {
        // pairwise across the vectors too, one conversion to fp64
#pragma unroll
        for (int w = kVecPerThread / 2; w > 0; w >>= 1)
#pragma unroll
          for (int q = 0; q < w; ++q) vsum[q] += vsum[q + w];
        S += static_cast<double>(vsum[0]);
      }
      if (has_tail) {
        const float y = fmaf(xt, s, nc_);
        const float t = __builtin_amdgcn_exp2f(y);
        S += static_cast<double>(t);
        if constexpr (ENT) T += static_cast<double>(xlogw(t, y));
      }
    }
  } else {
    // Misaligned row: scalar loads, two passes over the chunk.
    for (int i = e0 + tid; i < e1; i += kThreads) {
      const float x = load_elem(rowp, i, DT);
      if (x > m) {
        m = x;
        idx = i;
      }
    }
    if (!greedy && m > -INFINITY) {
      c = m * s;
      float acc = 0.0f, acct = 0.0f;
      int n = 0;
      for (int i = e0 + tid; i < e1; i += kThreads) {
        const float y = fmaf(load_elem(rowp, i, DT), s, -c);
        const float t = __builtin_amdgcn_exp2f(y);
        acc += t;
        if constexpr (ENT) acct += xlogw(t, y);
        if (++n == 8) {
          S += static_cast<double>(acc);
          if constexpr (ENT) T += static_cast<double>(acct);
          acc = 0.0f;
          acct = 0.0f;
          n = 0;
        }
      }
      S += static_cast<double>(acc);
      if constexpr (ENT) T += static_cast<double>(acct);
    }
  }

  Partial out;
  T_out = 0.0;
  if (greedy) {
    block_argmax(m, idx, lds);
    out.key = m;
    out.amax = idx;
    out.S = 0.0;
  } else {
    if (!(S > 0.0)) c = -INFINITY;   // thread saw no element
    if constexpr (ENT) {
      block_logsum_t(c, S, T, lds);
      T_out = T;
    } else {
      block_logsum(c, S, lds);
    }
    out.key = c;
    out.amax = -1;
    out.S = S;
  }
  return out;
}

}  // namespace sv
