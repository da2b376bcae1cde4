// Verification launches (see sv_verify.h): B * ns workgroups for stage 1 and
// its draw, then (hierarchy) B * ns for the stage-2 draws left over; plus the
// packed-output scan.
#include "sv_verify.h"

namespace sv {

namespace {

template <int DT, int STAGE>
__global__ __launch_bounds__(kThreads) void slice_kernel(VerifyArgs a) {
  __shared__ VerifyShared sm;
  const int b = blockIdx.x / a.ns;
  const int slice = blockIdx.x - b * a.ns;
  if (STAGE == 0)
    stage1_slice<DT>(a, b, slice, sm);
  else
    stage2_slice<DT>(a, b, slice, sm);
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

hipError_t launch_slices(const VerifyArgs& a, int stage, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.B) * static_cast<unsigned>(a.ns));
  if (a.dtype == 1) {
    if (stage == 0) hipLaunchKernelGGL((slice_kernel<1, 0>), grid, dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((slice_kernel<1, 1>), grid, dim3(kThreads), 0, st, a);
  } else {
    if (stage == 0) hipLaunchKernelGGL((slice_kernel<0, 0>), grid, dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((slice_kernel<0, 1>), grid, dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_pack(const PackArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(pack_kernel, dim3(1), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace sv
