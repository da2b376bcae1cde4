// The HBM stream: partial softmax statistics of every 64 KiB chunk of every
// logit row of every exit (see sv_stats.h).  One workgroup per (row, chunk) of
// the launch's rows; the first workgroups also clear the slice counters of the
// verification that follows on the same stream.  The ENT variant (row
// entropies requested) also writes each chunk's T.  A row-list launch covers
// only the rows an earlier launch listed (the lazy final exit's L_f rows up to
// each stage-1 stop, a flush's pending rows and final-exit rows).
#include <algorithm>

#include "sv_stats.h"

namespace sv {

namespace {

template <int DT, bool ENT>
__global__ __launch_bounds__(kThreads) void rowstats_kernel(StatsArgs a) {
  constexpr int ES = DT == 1 ? 2 : 4;
  constexpr int CE = kChunkBytes / ES;
  __shared__ Red lds[kWaves];
  const int tid = threadIdx.x;
  {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + tid;
    if (i < a.n_clear) a.clear_words[i] = 0;
    if (i == 0) a.flags[0] = 0u;
  }
  const int rel = blockIdx.x / a.nc;
  const int chunk = blockIdx.x - rel * a.nc;
  int row = a.row_begin + rel;
  if (a.win_b > 0) {   // rows j < win_r0 of exit 0, then rows j < win_r1 of exit 1
    const int rows0 = a.win_b * a.win_r0;
    if (rel < rows0) {
      const int b0 = rel / a.win_r0;
      row = a.exit_row0[0] + b0 * a.exit_pos[0] + (rel - b0 * a.win_r0);
    } else {
      const int r = rel - rows0, b1 = r / a.win_r1;
      row = a.exit_row0[1] + b1 * a.exit_pos[1] + (r - b1 * a.win_r1);
    }
  }
  int e = 0;
  if (a.num_exits > 1 && row >= a.exit_row0[1]) e = 1;
  if (a.num_exits > 2 && row >= a.exit_row0[2]) e = 2;
  const int local = row - a.exit_row0[e];
  const int b = local / a.exit_pos[e];
  const float tau = a.temperature ? a.temperature[b] : 1.0f;
  const bool greedy = !(tau > 0.0f) || !(tau < INFINITY);
  const float s = greedy ? 0.0f : kLog2e / tau;
  const char* rowp = static_cast<const char*>(a.exit_ptr[e]) + static_cast<int64_t>(local) * a.ld * ES;
  const int e0 = chunk * CE;
  double T;
  // the entropy sums first without the clamp; a chunk holding a -inf logit
  // (T comes out NaN in every thread) is scanned again with it
  Partial p = chunk_stats<DT, ENT, !ENT>(rowp, e0, min(a.V, e0 + CE), greedy, s, lds, T);
  if constexpr (ENT) {
    if (T != T) {
      __syncthreads();   // lds is read by the reduction just finished
      p = chunk_stats<DT, true, true>(rowp, e0, min(a.V, e0 + CE), greedy, s, lds, T);
    }
  }
  if (tid == 0) {
    a.partials[static_cast<int64_t>(row) * a.nc + chunk] = p;
    if constexpr (ENT) a.tpart[static_cast<int64_t>(row) * a.nc + chunk] = T;
  }
}

// Row-list mode: the workgroups loop over (listed row, chunk) items.  The
// first workgroups clear the verification counters as above.  CACHED: the
// rows are loaded with cache-allocating loads (the tentative flush, whose
// verification reads its pending rows again: 2-3 us less per round and
// flush; the lazy call is faster with nontemporal loads).
template <int DT, bool CACHED>
__global__ __launch_bounds__(kThreads) void rowstats_list_kernel(StatsArgs a) {
  constexpr int ES = DT == 1 ? 2 : 4;
  constexpr int CE = kChunkBytes / ES;
  __shared__ Red lds[kWaves];
  const int tid = threadIdx.x;
  {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + tid;
    if (i < a.n_clear) a.clear_words[i] = 0;
    if (i == 0) a.flags[0] = 0u;
  }
  // the count and the row ids are uniform: keep them (and all that follows
  // from them) in scalar registers
  const int n_items = __builtin_amdgcn_readfirstlane(*a.row_count) * a.nc;
  for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int rel = it / a.nc;
    const int chunk = it - rel * a.nc;
    const int row = __builtin_amdgcn_readfirstlane(a.row_list[rel]);
    int e = 0;
    if (a.num_exits > 1 && row >= a.exit_row0[1]) e = 1;
    if (a.num_exits > 2 && row >= a.exit_row0[2]) e = 2;
    const int local = row - a.exit_row0[e];
    const int b = local / a.exit_pos[e];
    const float tau = a.temperature ? a.temperature[b] : 1.0f;
    const bool greedy = !(tau > 0.0f) || !(tau < INFINITY);
    const float s = greedy ? 0.0f : kLog2e / tau;
    const char* rowp = static_cast<const char*>(a.exit_ptr[e]) + static_cast<int64_t>(local) * a.ld * ES;
    const int e0 = chunk * CE;
    double T;
    const Partial p = chunk_stats<DT, false, true, true, CACHED>(rowp, e0, min(a.V, e0 + CE), greedy, s, lds, T);
    if (tid == 0) a.partials[static_cast<int64_t>(row) * a.nc + chunk] = p;
    __syncthreads();   // the next item reuses lds
  }
}

}  // namespace

hipError_t launch_stats_list(const StatsArgs& a, int64_t max_items, hipStream_t st,
                             hipEvent_t ev_start, hipEvent_t ev_stop) {
  // three resident workgroups per CU (133 registers for bf16 rows)
  constexpr int64_t kListWorkgroups = 768;
  const int64_t clear_wg = (a.n_clear + kThreads - 1) / kThreads;
  const dim3 grid(static_cast<unsigned>(std::max<int64_t>(
      1, std::max(clear_wg, std::min(max_items, kListWorkgroups)))));
  if (a.dtype == 1) {
    if (a.cached_loads)
      launch_timed(rowstats_list_kernel<1, true>, grid, dim3(kThreads), st, ev_start, ev_stop, a);
    else
      launch_timed(rowstats_list_kernel<1, false>, grid, dim3(kThreads), st, ev_start, ev_stop, a);
  } else if (a.cached_loads) {
    launch_timed(rowstats_list_kernel<0, true>, grid, dim3(kThreads), st, ev_start, ev_stop, a);
  } else {
    launch_timed(rowstats_list_kernel<0, false>, grid, dim3(kThreads), st, ev_start, ev_stop, a);
  }
  return hipGetLastError();
}

hipError_t launch_stats(const StatsArgs& a, int64_t rows_total, hipStream_t st,
                        hipEvent_t ev_start, hipEvent_t ev_stop) {
  const dim3 grid(static_cast<unsigned>(rows_total * a.nc));
  const dim3 block(kThreads);
  if (a.tpart) {
    if (a.dtype == 1)
      launch_timed(rowstats_kernel<1, true>, grid, block, st, ev_start, ev_stop, a);
    else
      launch_timed(rowstats_kernel<0, true>, grid, block, st, ev_start, ev_stop, a);
  } else if (a.dtype == 1) {
    launch_timed(rowstats_kernel<1, false>, grid, block, st, ev_start, ev_stop, a);
  } else {
    launch_timed(rowstats_kernel<0, false>, grid, block, st, ev_start, ev_stop, a);
  }
  return hipGetLastError();
}

}  // namespace sv
