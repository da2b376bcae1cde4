// Internal definitions shared by every HIP source of libspecverify.so, the
// row-statistics stream included: sizes, the chunk partial, the stream's
// argument block, bf16 decode and wavefront reductions.  The other kernels'
// argument blocks and helpers are in sv_args.h.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

// Threads per workgroup of every kernel but the LM-head GEMM: 256, or 128 in
// the variant build that checks the kernels for races that depend on the
// workgroup size (libspecverify_t128.so; results must not change).
#ifndef SV_THREADS
#define SV_THREADS 256
#endif
constexpr int kThreads = SV_THREADS;
static_assert(kThreads == 256 || kThreads == 128, "workgroup size");
constexpr int kWave = 64;              // CDNA wavefront width
constexpr int kWaves = kThreads / kWave;
constexpr int kVecPerThread = 16;      // 16-byte vectors each row-stats thread holds
constexpr int kChunkBytes = kThreads * kVecPerThread * 16;   // 64 KiB of one row
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxVocab = 1 << 20;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Elements per 16-byte vector.
__host__ __device__ constexpr int vec_elems(int dtype) { return dtype == 1 ? 8 : 4; }
__host__ __device__ constexpr int elem_bytes(int dtype) { return dtype == 1 ? 2 : 4; }
// Elements of one row covered by one row-stats workgroup.
__host__ __device__ constexpr int chunk_elems(int dtype) { return kChunkBytes / elem_bytes(dtype); }
// Elements of one draw tile (one 16-byte vector per lane of a wavefront).
__host__ __device__ constexpr int tile_elems(int dtype) { return kWave * vec_elems(dtype); }

// Partial statistics of one (row, chunk).  For a sampled row (temperature > 0)
// key = c, a float reference in log2 units, and S = sum over the chunk of
// 2^(l * s - c) with s = log2(e) / temperature.  For a greedy row key = the
// maximum logit and amax = its lowest index.
struct Partial {
  float key;
  int32_t amax;
  double S;
};
static_assert(sizeof(Partial) == 16, "Partial layout");

// Row statistics of every logit row (the HBM stream).
struct StatsArgs {
  const void* exit_ptr[3];
  int32_t exit_pos[3];     // rows per sequence in each exit (k or k + 1)
  int32_t exit_row0[3];    // first global row id of each exit
  int32_t num_exits, V, nc, dtype;
  int64_t ld;              // row stride in elements
  const float* temperature;
  Partial* partials;       // [rows_total * nc]
  int32_t* clear_words;    // zeroed by the first workgroups (slice counters)
  int32_t n_clear;
  uint32_t* flags;
  int32_t row_begin;       // first row of this launch (rows are launched in order)
  // Position window (win_b > 0 sequences): the launch covers rows j < win_r0
  // of exit 0, then rows j < win_r1 of exit 1, win_b * (win_r0 + win_r1) rows
  // (the lazy call's first stage-1 window).
  int32_t win_b, win_r0, win_r1;
  // Row entropies requested: per (row, chunk) T = sum 2^(l*s - c) * (l*s - c)
  // beside the partial (same reference c); NULL: not computed.
  double* tpart;
  // Row-list launch (launch_stats_list): the *row_count global row ids of
  // row_list, written by an earlier launch.
  const int32_t* row_list;
  const int32_t* row_count;
  // Row-list launch: cache-allocating instead of nontemporal loads (the
  // tentative flush, whose verification reads the pending rows again).
  int32_t cached_loads;
};

// A kernel launch that, given events, has them take the kernel's own start and
// end times (hipExtLaunchKernelGGL) instead of recording them around it.
template <typename K, typename A>
inline void launch_timed(K kernel, dim3 grid, dim3 block, hipStream_t st, hipEvent_t ev_start,
                         hipEvent_t ev_stop, const A& args) {
  if (ev_start || ev_stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, ev_start, ev_stop, 0, args);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args);
}

// ev_start / ev_stop (either may be NULL): events that take the kernel's own
// start and end times (an extended launch: no marker packets on the stream).
hipError_t launch_stats(const StatsArgs& a, int64_t rows_total, hipStream_t st,
                        hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
// The rows of a.row_list only: a grid of at most max_wg workgroups loops over
// (listed row, chunk) items, so a launch costs the rows it reads rather than
// one dispatched workgroup per possible row.
hipError_t launch_stats_list(const StatsArgs& a, int64_t max_items, hipStream_t st,
                             hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

// ---------------------------------------------------------------------------
// device helpers

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float load_elem(const void* row, int64_t i, int dtype) {
  if (dtype == 1) {
    const uint16_t h = static_cast<const uint16_t*>(row)[i];
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
  }
  return static_cast<const float*>(row)[i];
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

}  // namespace sv
