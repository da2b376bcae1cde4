// The verification path in one launch.
//
// Every workgroup computes the partial statistics of one 64 KiB chunk of one
// logit row (the HBM stream, sv_stats.h) and counts itself done for its
// sequence.  The workgroup that completes a sequence's stage-1 rows (draft and
// target, or L_d and L_i) runs stage 1 for that sequence (sv_verify.h) while
// the rest of the grid keeps streaming; for the hierarchy, the workgroup that
// completes both the sequence's L_f rows and its stage 1 runs stage 2.  No
// workgroup ever waits for another: whoever arrives last does the work.
//
// Chunks are ordered by sequence: stage-1 rows of sequence b, then the L_f rows
// of sequence b - lag, so a sequence's rows are read close together in time and
// the rows its draws re-read are recent.
#include "sv_stats.h"
#include "sv_verify.h"

namespace sv {

namespace {

struct Item {
  int b;   // sequence
  int f;   // 0: a stage-1 row chunk, 1: an L_f row chunk
  int r;   // chunk index within that part of the sequence
};

__device__ __forceinline__ Item map_item(int64_t idx, int B, int n1, int n2, int D) {
  if (n2 == 0) return {static_cast<int>(idx / n1), 0, static_cast<int>(idx % n1)};
  const int64_t head = static_cast<int64_t>(D) * n1;
  if (idx < head) return {static_cast<int>(idx / n1), 0, static_cast<int>(idx % n1)};
  const int64_t gs = n1 + n2;
  const int64_t mid = static_cast<int64_t>(B - D) * gs;
  int64_t x = idx - head;
  if (x < mid) {
    const int g = static_cast<int>(x / gs), r = static_cast<int>(x % gs);
    if (r < n1) return {D + g, 0, r};
    return {g, 1, r - n1};
  }
  x -= mid;
  return {B - D + static_cast<int>(x / n2), 1, static_cast<int>(x % n2)};
}

union FusedShared {
  Red red[kWaves];
  VerifyShared v;
};

template <int DT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8)))
void fused_kernel(FusedArgs a) {
  constexpr int ES = DT == 1 ? 2 : 4;
  constexpr int CE = kChunkBytes / ES;
  __shared__ FusedShared sm;
  __shared__ int is_last;
  const int tid = threadIdx.x;
  const Item it = map_item(blockIdx.x, a.B, a.n1, a.n2, a.lag);
  const int b = it.b;
  const int row_in = it.r / a.nc;   // row within the part
  const int c = it.r - row_in * a.nc;
  int e, j;
  if (it.f) {
    e = 2;
    j = row_in;
  } else if (row_in < a.k) {
    e = 0;
    j = row_in;
  } else {
    e = 1;
    j = row_in - a.k;
  }
  const int P = e == 0 ? a.k : a.k + 1;
  const float tau = a.temperature ? a.temperature[b] : 1.0f;
  const bool greedy = !(tau > 0.0f) || !(tau < INFINITY);
  const float s = greedy ? 0.0f : kLog2e / tau;
  const int64_t row_local = static_cast<int64_t>(b) * P + j;
  const char* rowp = static_cast<const char*>(a.exit_ptr[e]) + row_local * a.ld * ES;
  const int e0 = c * CE;
  const Partial p = chunk_stats<DT>(rowp, e0, min(a.V, e0 + CE), greedy, s, sm.red);

  if (tid == 0) {
    publish_partial(a.partials + (a.exit_row0[e] + row_local) * a.nc + c, p);
    const int old = atomicAdd(it.f ? &a.cnt2[b] : &a.cnt1[b], 1);
    is_last = it.f ? (old == a.n2) : (old == a.n1 - 1);
  }
  __syncthreads();
  if (!is_last) return;
  // every partial of this sequence's rows has been published
  bool stage2 = it.f != 0;
  if (!stage2) stage2 = verify_stage1<DT>(a, b, sm.v);
  if (stage2) verify_stage2<DT>(a, b, sm.v);
}

__global__ __launch_bounds__(kThreads) void clear_kernel(ClearArgs a) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < a.n) a.words[i] = 0;
  if (i == 0) a.flags[0] = 0u;
}

// Packed (unpadded) tokens: cu_offsets by a single-workgroup scan of the
// emitted counts, then each sequence's tokens copied back to back.
__global__ __launch_bounds__(kThreads) void pack_kernel(PackArgs a) {
  __shared__ int scan[kThreads];
  __shared__ int carry;
  const int tid = threadIdx.x;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < a.B; base += kThreads) {
    const int b = base + tid;
    const int n = b < a.B ? a.num_emitted[b] : 0;
    scan[tid] = n;
    __syncthreads();
    for (int o = 1; o < kThreads; o <<= 1) {
      const int add = tid >= o ? scan[tid - o] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    const int off = carry + scan[tid] - n;
    if (b < a.B) {
      a.cu_offsets[b] = off;
      for (int i = 0; i < n; ++i)
        a.packed[off + i] = a.out_tokens[static_cast<int64_t>(b) * (a.k + 1) + i];
    }
    __syncthreads();
    if (tid == kThreads - 1) carry = off + n;
    __syncthreads();
  }
  if (tid == 0) a.cu_offsets[a.B] = carry;
}

}  // namespace

hipError_t launch_clear(const ClearArgs& a, hipStream_t st) {
  const unsigned grid = static_cast<unsigned>((a.n + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(clear_kernel, dim3(grid > 0 ? grid : 1), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_fused(const FusedArgs& a, int64_t items, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(items));
  if (a.dtype == 1)
    hipLaunchKernelGGL(fused_kernel<1>, grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(fused_kernel<0>, grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_pack(const PackArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(pack_kernel, dim3(1), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace sv
