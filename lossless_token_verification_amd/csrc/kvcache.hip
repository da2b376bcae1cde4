// Paged-KV rollback: one thread per sequence drops the KV slots of rejected
// drafted tokens from its block table (HiSpec summary, section 2, bullets on
// KV-cache reuse -- entries of discarded tokens are removed before the next
// phase, without recomputation -- and on batch inference with paged attention
// and block tables, which lets each sequence keep its own length unpadded).
#include "sv_args.h"

namespace sv {

namespace {

__global__ __launch_bounds__(kThreads) void kv_truncate_kernel(KvArgs a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.B) return;
  kv_rollback_one(a.table + static_cast<int64_t>(b) * a.max_blocks, a.lens + b, a.drop[b],
                  a.freed ? a.freed + static_cast<int64_t>(b) * a.max_freed : nullptr,
                  a.num_freed + b, a.max_blocks, a.block_size, a.max_freed);
}

}  // namespace

hipError_t launch_kv_truncate(const KvArgs& a, hipStream_t st) {
  const unsigned grid = static_cast<unsigned>((a.B + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(kv_truncate_kernel, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace sv
