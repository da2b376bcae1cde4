// LM-head path: the logit matrix of the draft and final exits is never written
// to memory.  A bf16 GEMM on the matrix cores (v_mfma_f32_32x32x16_bf16) multiplies
// the exits' hidden states by the shared head W [V, d] and reduces each
// 192 x 384 output tile in its epilogue to the per-(row, vocabulary tile)
// softmax partials; a merge launch combines them per row and forms the logit
// at each row's drafted token (one dot product per row).  After the
// decisions, the same GEMM recomputes into the workspace only the two rows
// each sequence draws from (the target row at the stop position and, for a
// correction, the draft row there).
//
// In an early-exit model each exit turns its hidden state into a token
// distribution (HiSpec summary, section 2 "Kernmechanismus"); with a linear
// head the distribution is the softmax of hidden . W^T.
//
// Tiling (512 threads, 2 x 4 wavefronts of 96 x 96 outputs each; the
// recompute GEMM 256 x 256 tiles, 128 x 64 per wavefront): both
// operands are K-contiguous (hidden states [rows, d], head [V, d]), so each
// 64-element K step of the A and W tiles is loaded from global memory straight
// into LDS (16-byte direct loads, no register stage, rows of 128 bytes with an
// XOR-permuted vector order), and every MFMA operand is one 16-byte LDS read
// per lane.  The direct loads of a step are issued one step ahead into the
// other of two LDS buffers (one barrier per step).  Workgroup i runs on XCD
// i % 8; the M tiles of one vocabulary tile are consecutive on one XCD, so
// the W tile is fetched from HBM once and served to the other M tiles from
// that XCD's L2.  The epilogue keeps each wavefront's row reductions apart
// (row maximum by an all-lane butterfly, sum relative to it) and merges the
// wavefronts' pairs once, so its reductions run side by side.
#include <algorithm>
#include <type_traits>

#include "sv_args.h"

namespace sv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Tile configuration: MT x NT outputs per workgroup on a WM x WN grid of
// wavefronts, each holding (MT / WM / 32) x (NT / WN / 32) MFMA tiles.
template <int MT_, int NT_, int WM_, int WN_, int KT_>
struct GemmCfg {
  static constexpr int WM = WM_, WN = WN_;
  static constexpr int MT = MT_, NT = NT_;
  static constexpr int FM = MT / (WM * 32), FN = NT / (WN * 32);
  static constexpr int WAVES = WM * WN;
  static constexpr int GT = WAVES * kWave;            // threads per workgroup
  static constexpr int KT = KT_;
  static constexpr int VPR = KT / 8;                  // 16-byte vectors per tile row
  // A direct load of one wavefront fills 1 KiB of LDS (64 lanes x 16 bytes),
  // KROWS whole tile rows.  Load slot j < A_LOADS fills A rows j * KROWS ..,
  // the other slots W rows; wavefront w takes slots w, w + WAVES, ...
  static constexpr int KROWS = kWave / VPR;
  static constexpr int A_LOADS = MT / KROWS, LOADS = A_LOADS + NT / KROWS;
  static constexpr int LPW = (LOADS + WAVES - 1) / WAVES;
  static_assert(FM * WM * 32 == MT && FN * WN * 32 == NT, "tile shape");
  static_assert(VPR == 4 || VPR == 8, "64- or 128-byte LDS rows");
  static_assert(A_LOADS * KROWS == MT && (LOADS - A_LOADS) * KROWS == NT, "copy slots");

  struct alignas(16) Epi {
    float m[WN][MT];  // per wavefront column block: row maximum
    int i[WN][MT];    // its lowest column (greedy rows)
    float s[WN][MT];  // sum of 2^(l * s - c) over the block
    float rs[MT];     // log2(e) / temperature of the row (0: greedy)
    int tok[MT];      // rows mode: source row (-1: skipped)
    float rmax[MT];
    int ridx[MT];
  };
};

// LDS position (16-byte vector) of vector kv of tile row r: rows are VPR
// vectors, unpadded, and the vectors of a row are permuted by
// (r / (16 / VPR)) mod VPR, so that the 16 consecutive rows one MFMA operand
// read takes at the same kv fall on 16 different 16-byte bank groups.
template <int VPR>
__device__ __forceinline__ int swz(int r, int kv) {
  return r * VPR + (kv ^ ((r / (16 / VPR)) & (VPR - 1)));
}

// statistics over all B(2k+1) rows; recompute of the 2B stopped rows
using StatsCfg = GemmCfg<kGemmMT, kGemmNT, kGemmWM, kGemmWN, kGemmKT>;
using RowsCfg = GemmCfg<kGemmRowsMT, kGemmRowsNT, kGemmWM, kGemmWN, kGemmKT>;

// Sums over each 32-lane half of a wavefront (the lanes holding one output
// row of a 32 x 32 MFMA tile) with DPP moves on the VALU: a scan within each
// row of 16 lanes (row_shr 1, 2, 4, 8), then rows 1 and 3 fold in the last
// lane of rows 0 and 2 (row_bcast 15).  Lane 31 ends with the sum of lanes
// 0..31, lane 63 with that of lanes 32..63.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add_step(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf,
                                                         false));
}
__device__ __forceinline__ float half_sum(float x) {
  x = dpp_add_step<0x111, 0xf>(x);
  x = dpp_add_step<0x112, 0xf>(x);
  x = dpp_add_step<0x114, 0xf>(x);
  x = dpp_add_step<0x118, 0xf>(x);
  return dpp_add_step<0x142, 0xa>(x);
}
// One DPP move of an integer within each row of 16 lanes (every lane has a
// source for the patterns used here: quad permutations and mirrors).
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, false);
}
// Ordered-integer key of a float: keys compare as signed integers in the
// order of the floats (-0 below +0); the map is its own inverse.
__device__ __forceinline__ int ord_key(float x) {
  const int i = __float_as_int(x);
  return i ^ ((i >> 31) & 0x7fffffff);
}
__device__ __forceinline__ int ord_key_inv(int k) { return k ^ ((k >> 31) & 0x7fffffff); }

__device__ __forceinline__ const uint16_t* a_row(const GemmArgs& a, int g) {
  return g < a.m_draft ? a.a_draft + static_cast<int64_t>(g) * a.d
                       : a.a_target + static_cast<int64_t>(g - a.m_draft) * a.d;
}

// Sequence and drafted token of GEMM row g (stats numbering).
__device__ __forceinline__ void row_meta(const GemmArgs& a, int g, int& b, int& tok) {
  if (g < a.m_draft) {
    b = g / a.k;
    tok = a.tokens[g];
  } else {
    const int r = g - a.m_draft;
    b = r / (a.k + 1);
    const int j = r - b * (a.k + 1);
    tok = j < a.k ? a.tokens[static_cast<int64_t>(b) * a.k + j] : -1;
  }
}

// Two wavefronts per SIMD (up to 256 registers each).
template <class C, bool ROWS>
__global__ __launch_bounds__(C::GT) __attribute__((amdgpu_waves_per_eu(2))) void lmhead_gemm(
    GemmArgs a) {
  constexpr int WN = C::WN, FM = C::FM, FN = C::FN;
  constexpr int MT = C::MT, NT = C::NT, KT = C::KT, VPR = C::VPR, KROWS = C::KROWS;
  constexpr int A_LOADS = C::A_LOADS, LOADS = C::LOADS, LPW = C::LPW;
  // two buffers of each operand, each its own LDS object: the compiler then
  // knows a direct load into one buffer cannot change the other, and does not
  // wait for it before reading the other
  __shared__ __attribute__((aligned(1024))) uint16_t sa0[MT * KT], sa1[MT * KT];
  __shared__ __attribute__((aligned(1024))) uint16_t sb0[NT * KT], sb1[NT * KT];
  __shared__ typename C::Epi ep;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int wm = wave / WN, wn = wave - wm * WN;
  const int nM = (a.M + MT - 1) / MT;
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int ntile = (local / nM) * 8 + xcd;
  const int mtile = local - (local / nM) * nM;
  if (ntile >= a.n_tiles) return;   // padding of the grid to a multiple of 8 tiles
  const int m0 = mtile * MT, n0 = ntile * NT;

  // Direct loads (global memory to LDS, no register stage): lane l of a load
  // fills LDS vector l of that 1 KiB, which holds vector kv of tile row r with
  // swz(r, kv) = that position.  Rows past the matrix read a valid row instead
  // (clamped, or row 0 for a skipped recompute row): each output depends only
  // on its own A and W rows, and the epilogue never reports those rows or
  // columns.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint16_t* gp[LPW];
  {
    const int rl = lane / VPR, slot = lane - rl * VPR;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int j = min(wave_u + i * C::WAVES, LOADS - 1);
      if (j < A_LOADS) {
        const int r = j * KROWS + rl;
        const int kv = slot ^ ((r / (16 / VPR)) & (VPR - 1));
        int g = min(m0 + r, a.M - 1);
        if (ROWS) g = max(a.a_rows[g], 0);
        gp[i] = a_row(a, g) + kv * 8;
      } else {
        const int r = (j - A_LOADS) * KROWS + rl;
        const int kv = slot ^ ((r / (16 / VPR)) & (VPR - 1));
        const int n = min(n0 + r, a.V - 1);
        gp[i] = a.w + static_cast<int64_t>(n) * a.ldw + kv * 8;
      }
    }
  }
  typedef const void __attribute__((address_space(1)))* gptr_t;
  typedef void __attribute__((address_space(3)))* lptr_t;
  auto dload = [&](int k0, uint16_t* la, uint16_t* lb) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int j = wave_u + i * C::WAVES;
      if (LOADS % C::WAVES == 0 || j < LOADS) {
        uint16_t* dst = j < A_LOADS ? la + j * 512 : lb + (j - A_LOADS) * 512;
        __builtin_amdgcn_global_load_lds((gptr_t)(gp[i] + k0), (lptr_t)dst, 16, 0, 0);
      }
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[fm][fn][q] = 0.0f;

  // a wavefront whose rows all lie past the matrix skips its MFMAs
  const bool active = m0 + wm * FM * 32 < a.M;
  const int nK = a.d / KT;
  const int frow = lane & 31, fh = lane >> 5;
  auto compute = [&](const uint16_t* la, const uint16_t* lb) {
    if (!active) return;
#pragma unroll
    for (int ks = 0; ks < KT / 16; ++ks) {
      const int kv = ks * 2 + fh;
      bf16x8 af[FM], bf[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int r = wm * FM * 32 + fm * 32 + frow;
        af[fm] = __builtin_bit_cast(bf16x8,
                                    *reinterpret_cast<const u32x4*>(la + swz<VPR>(r, kv) * 8));
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int r = wn * FN * 32 + fn * 32 + frow;
        bf[fn] = __builtin_bit_cast(bf16x8,
                                    *reinterpret_cast<const u32x4*>(lb + swz<VPR>(r, kv) * 8));
      }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fm], bf[fn], acc[fm][fn], 0, 0, 0);
    }
  };
  // Step t computes on buffer t % 2 while the direct loads of step t + 1 fill
  // the other; the barrier closing each step also waits for those loads
  // (__syncthreads waits for every outstanding memory operation of the
  // wavefront, direct loads to LDS included).
  dload(0, sa0, sb0);
  __syncthreads();
  int kt = 0;
  for (; kt + 2 <= nK; kt += 2) {
    dload((kt + 1) * KT, sa1, sb1);
    compute(sa0, sb0);
    __syncthreads();
    if (kt + 2 < nK) dload((kt + 2) * KT, sa0, sb0);
    compute(sa1, sb1);
    __syncthreads();
  }
  if (kt < nK) compute(sa0, sb0);   // odd number of steps: the last one is in buffer 0

  // Output element (fm, fn, q) of this lane: row wm*FM*32 + fm*32 + (q/4)*8 +
  // h*4 + q%4, column wn*FN*32 + fn*32 + c32 (h = lane / 32, c32 = lane % 32).
  const int h = lane >> 5, c32 = lane & 31;
  auto row_of = [&](int fm, int q) { return wm * FM * 32 + fm * 32 + (q >> 2) * 8 + h * 4 + (q & 3); };
  auto col_of = [&](int fn) { return n0 + wn * FN * 32 + fn * 32 + c32; };

  if (ROWS) {
    if (tid < MT) ep.tok[tid] = m0 + tid < a.M ? a.a_rows[m0 + tid] : -1;
    __syncthreads();
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int rl = row_of(fm, q);
        if (ep.tok[rl] < 0) continue;
        float* orow = a.out + static_cast<int64_t>(m0 + rl) * a.ldo;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int col = col_of(fn);
          if (col < a.V) orow[col] = acc[fm][fn][q];
        }
      }
    return;
  }

  if (tid < MT) {
    const int g = m0 + tid;
    float s = 0.0f;
    if (g < a.M) {
      int b, tok;
      row_meta(a, g, b, tok);
      const float tau = a.temperature ? a.temperature[b] : 1.0f;
      const bool greedy = !(tau > 0.0f) || !(tau < INFINITY);
      s = greedy ? 0.0f : kLog2e / tau;
    }
    ep.rs[tid] = s;
  }
  // greedy rows need the lowest column of the maximum as well
  const bool any_greedy = __syncthreads_or(tid < MT && m0 + tid < a.M && ep.rs[tid] == 0.0f);

  if (!any_greedy) {
    // Every row sampled: each wavefront reduces its column block of a row to
    // its maximum m_w and S_w = sum 2^(l * s - m_w * s) with no exchange
    // between wavefronts; the workgroup then merges the WN pairs.  A column
    // past the vocabulary (last tile only) counts nowhere.
    auto block_stats = [&](auto full_tile) {
      constexpr bool kFull = decltype(full_tile)::value;
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int rb = wm * FM * 32 + fm * 32 + h * 4;   // row of q = 0; row of q: rb + (q/4)*8 + q%4
        // the 16 rows' scales, four consecutive rows per 16-byte read
        float sc[16];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const float4 v = *reinterpret_cast<const float4*>(&ep.rs[rb + qq * 8]);
          sc[qq * 4 + 0] = v.x;
          sc[qq * 4 + 1] = v.y;
          sc[qq * 4 + 2] = v.z;
          sc[qq * 4 + 3] = v.w;
        }
        // row maxima over the wavefront's columns, every lane of the half
        // ending with its rows' maxima (ordered-integer keys: the integer
        // maximum of the keys is the float maximum)
        int key[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          float m = -INFINITY;
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            if (kFull || col_of(fn) < a.V) m = fmaxf(m, acc[fm][fn][q]);
          key[q] = ord_key(m);
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) key[q] = max(key[q], dpp_i32<0xb1>(key[q]));   // lane ^ 1
#pragma unroll
        for (int q = 0; q < 16; ++q) key[q] = max(key[q], dpp_i32<0x4e>(key[q]));   // lane ^ 2
#pragma unroll
        for (int q = 0; q < 16; ++q) key[q] = max(key[q], dpp_i32<0x141>(key[q]));  // half-row mirror
#pragma unroll
        for (int q = 0; q < 16; ++q) key[q] = max(key[q], dpp_i32<0x140>(key[q]));  // row mirror
#pragma unroll
        for (int q = 0; q < 16; ++q)
          key[q] = max(key[q], __builtin_amdgcn_ds_swizzle(key[q], 0x401f));      // lane ^ 16
        float mrow[16], sum[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          mrow[q] = __int_as_float(ord_key_inv(key[q]));
          const float nc = -(mrow[q] * sc[q]);
          float t = 0.0f;
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            if (kFull || col_of(fn) < a.V) t += __builtin_amdgcn_exp2f(fmaf(acc[fm][fn][q], sc[q], nc));
          sum[q] = t;
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) sum[q] = dpp_add_step<0x111, 0xf>(sum[q]);
#pragma unroll
        for (int q = 0; q < 16; ++q) sum[q] = dpp_add_step<0x112, 0xf>(sum[q]);
#pragma unroll
        for (int q = 0; q < 16; ++q) sum[q] = dpp_add_step<0x114, 0xf>(sum[q]);
#pragma unroll
        for (int q = 0; q < 16; ++q) sum[q] = dpp_add_step<0x118, 0xf>(sum[q]);
#pragma unroll
        for (int q = 0; q < 16; ++q) sum[q] = dpp_add_step<0x142, 0xa>(sum[q]);
        if (c32 == 31) {
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int rl = rb + (q >> 2) * 8 + (q & 3);
            ep.m[wn][rl] = mrow[q];
            ep.s[wn][rl] = sum[q];
          }
        }
      }
    };
    if (n0 + NT <= a.V) block_stats(std::true_type{});
    else block_stats(std::false_type{});
    __syncthreads();
    if (tid < MT && m0 + tid < a.M) {
      const float s = ep.rs[tid];
      float m = ep.m[0][tid];
#pragma unroll
      for (int w = 1; w < WN; ++w) m = fmaxf(m, ep.m[w][tid]);
      const float c = m * s;
      double S = 0.0;
#pragma unroll
      for (int w = 0; w < WN; ++w) {
        const float sw = ep.s[w][tid];
        if (sw > 0.0f)
          S += static_cast<double>(sw) *
               exp2(static_cast<double>(ep.m[w][tid] * s) - static_cast<double>(c));
      }
      Partial p;
      p.key = c;
      p.amax = -1;
      p.S = S;
      a.partials[static_cast<int64_t>(m0 + tid) * a.n_tiles + ntile] = p;
    }
    return;
  }

  // Greedy rows present.  Pass 1: the maximum of each row over the tile and
  // its lowest column.
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      float m = -INFINITY;
      int idx = 0x7fffffff;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int col = col_of(fn);
        const float v = acc[fm][fn][q];
        if (col < a.V && v > m) {
          m = v;
          idx = col;
        }
      }
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) {
        const float om = __shfl_xor(m, o, kWave);
        const int oi = __shfl_xor(idx, o, kWave);
        if (om > m || (om == m && oi < idx)) {
          m = om;
          idx = oi;
        }
      }
      if (c32 == 0) {
        const int rl = row_of(fm, q);
        ep.m[wn][rl] = m;
        ep.i[wn][rl] = idx;
      }
    }
  __syncthreads();
  if (tid < MT) {
    float m = ep.m[0][tid];
    int idx = ep.i[0][tid];
#pragma unroll
    for (int w = 1; w < WN; ++w) {
      if (ep.m[w][tid] > m || (ep.m[w][tid] == m && ep.i[w][tid] < idx)) {
        m = ep.m[w][tid];
        idx = ep.i[w][tid];
      }
    }
    ep.rmax[tid] = m;
    ep.ridx[tid] = idx;
  }
  __syncthreads();

  // pass 2 (sampled rows of the tile): sum of 2^(l * s - c), c = max * s
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int rl = row_of(fm, q);
      const float s = ep.rs[rl];
      const float nc = -(ep.rmax[rl] * s);
      float sum = 0.0f;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        if (col_of(fn) < a.V && s > 0.0f) sum += __builtin_amdgcn_exp2f(fmaf(acc[fm][fn][q], s, nc));
      sum = half_sum(sum);
      if (c32 == 31) ep.s[wn][rl] = sum;
    }
  __syncthreads();
  if (tid < MT && m0 + tid < a.M) {
    Partial p;
    if (ep.rs[tid] > 0.0f) {
      double S = 0.0;
#pragma unroll
      for (int w = 0; w < WN; ++w) S += static_cast<double>(ep.s[w][tid]);
      p.key = ep.rmax[tid] * ep.rs[tid];
      p.amax = -1;
      p.S = S;
    } else {
      p.key = ep.rmax[tid];
      p.amax = ep.ridx[tid];
      p.S = 0.0;
    }
    a.partials[static_cast<int64_t>(m0 + tid) * a.n_tiles + ntile] = p;
  }
}

// One wavefront per row: merge the row's n partials (a greedy row's partials
// carry an argmax >= 0, a sampled row's -1), and form the logit at the row's
// drafted token as the dot product of its hidden state with that head row
// (fp32 products and sums).  The first workgroups also clear the counters of
// the verification launches.
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeArgs a, GemmArgs g) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + tid;
    if (i < a.n_clear) a.clear_words[i] = 0;
    if (i == 0) a.flags[0] = 0u;
  }
  const int row = blockIdx.x * kWaves + tid / kWave;
  if (row >= a.rows) return;
  // The drafted token's logit: the loads go out before the partials' (a row
  // without a token reads head row 0 and discards the result; d is a
  // multiple of 64, so every vector is whole).
  int b, tok;
  row_meta(g, row, b, tok);
  const bool has_tok = tok >= 0 && tok < g.V;
  const uint16_t* hr = a_row(g, row);
  const uint16_t* wr = g.w + static_cast<int64_t>(has_tok ? tok : 0) * g.ldw;
  float dot = 0.0f;
  for (int e0 = lane * 8; e0 < g.d; e0 += 8 * kWave * 8) {
    u32x4 hv[8], wv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = min(e0 + j * kWave * 8, g.d - 8);
      hv[j] = *reinterpret_cast<const u32x4*>(hr + e);
      wv[j] = *reinterpret_cast<const u32x4*>(wr + e);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (e0 + j * kWave * 8 >= g.d) break;
      dot = fmaf(bf16_lo(hv[j].x), bf16_lo(wv[j].x), dot);
      dot = fmaf(bf16_hi(hv[j].x), bf16_hi(wv[j].x), dot);
      dot = fmaf(bf16_lo(hv[j].y), bf16_lo(wv[j].y), dot);
      dot = fmaf(bf16_hi(hv[j].y), bf16_hi(wv[j].y), dot);
      dot = fmaf(bf16_lo(hv[j].z), bf16_lo(wv[j].z), dot);
      dot = fmaf(bf16_hi(hv[j].z), bf16_hi(wv[j].z), dot);
      dot = fmaf(bf16_lo(hv[j].w), bf16_lo(wv[j].w), dot);
      dot = fmaf(bf16_hi(hv[j].w), bf16_hi(wv[j].w), dot);
    }
  }
  // The partials, eight per lane in flight at a time: greedy rows keep the
  // largest key and its lowest index, sampled rows an online (c, S) pair per
  // lane, merged across the wavefront at the end.
  const Partial* pp = a.in + static_cast<int64_t>(row) * a.n;
  bool greedy = false;
  float m = -INFINITY;
  int idx = 0x7fffffff;
  double S = 0.0;
  for (int c0 = lane; c0 < a.n; c0 += 8 * kWave) {
    Partial q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = pp[min(c0 + j * kWave, a.n - 1)];
    greedy = q[0].amax >= 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (c0 + j * kWave >= a.n) break;
      if (greedy) {
        if (q[j].key > m || (q[j].key == m && q[j].amax < idx)) {
          m = q[j].key;
          idx = q[j].amax;
        }
      } else if (q[j].S > 0.0) {
        if (q[j].key > m) {
          S = S * exp2(static_cast<double>(m) - static_cast<double>(q[j].key)) + q[j].S;
          m = q[j].key;
        } else {
          S += q[j].S * exp2(static_cast<double>(q[j].key) - static_cast<double>(m));
        }
      }
    }
  }
  // every row has a.n >= 1 partials, so lane 0 saw the row's kind
  greedy = __shfl(greedy, 0, kWave);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) dot += __shfl_xor(dot, o, kWave);
  if (lane == 0 && has_tok) g.gath[row] = dot;
  Partial out;
  if (greedy) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float om = __shfl_xor(m, o, kWave);
      const int oi = __shfl_xor(idx, o, kWave);
      if (om > m || (om == m && oi < idx)) {
        m = om;
        idx = oi;
      }
    }
    out.key = m;
    out.amax = idx;
    out.S = 0.0;
  } else {
    const float cm = wave_max(m);
    if (S > 0.0) S *= exp2(static_cast<double>(m) - static_cast<double>(cm));
    S = wave_sum(S);
    out.key = cm;
    out.amax = -1;
    out.S = S;
  }
  if (lane == 0) a.out[row] = out;
}

template <class C>
unsigned gemm_grid(const GemmArgs& a) {
  const unsigned nM = static_cast<unsigned>((a.M + C::MT - 1) / C::MT);
  const unsigned nN8 = static_cast<unsigned>((a.n_tiles + 7) / 8) * 8u;
  return nM * nN8;
}

}  // namespace

hipError_t launch_lmhead_stats(const GemmArgs& a, hipStream_t st, hipEvent_t ev_start,
                               hipEvent_t ev_stop) {
  launch_timed(lmhead_gemm<StatsCfg, false>, dim3(gemm_grid<StatsCfg>(a)), dim3(StatsCfg::GT), st,
               ev_start, ev_stop, a);
  return hipGetLastError();
}

hipError_t launch_lmhead_rows(const GemmArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((lmhead_gemm<RowsCfg, true>), dim3(gemm_grid<RowsCfg>(a)),
                     dim3(RowsCfg::GT), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, const GemmArgs& g, hipStream_t st) {
  const int64_t by_rows = (static_cast<int64_t>(a.rows) + kWaves - 1) / kWaves;
  const int64_t by_clear = (static_cast<int64_t>(a.n_clear) + kThreads - 1) / kThreads;
  const unsigned grid = static_cast<unsigned>(std::max<int64_t>(1, std::max(by_rows, by_clear)));
  hipLaunchKernelGGL(merge_kernel, dim3(grid), dim3(kThreads), 0, st, a, g);
  return hipGetLastError();
}

}  // namespace sv
