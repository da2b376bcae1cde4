// The verification launch (see sv_verify.h): B * ns workgroups take both
// stages' decisions and draw the correction / bonus tokens; plus the
// packed-output scan.
#include "sv_verify.h"

namespace sv {

namespace {

template <int DT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8)))
void verify_kernel(VerifyArgs a) {
  __shared__ VerifyShared sm;
  const int b = blockIdx.x / a.ns;
  verify_slice<DT>(a, b, blockIdx.x - b * a.ns, sm);
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

hipError_t launch_verify(const VerifyArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.B) * static_cast<unsigned>(a.ns));
  if (a.dtype == 1)
    hipLaunchKernelGGL(verify_kernel<1>, grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(verify_kernel<0>, grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_pack(const PackArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(pack_kernel, dim3(1), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace sv
