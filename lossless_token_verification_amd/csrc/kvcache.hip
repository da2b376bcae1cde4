// Paged-KV rollback: one thread per sequence drops the KV slots of rejected
// drafted tokens from its block table (HiSpec summary, section 2, bullets on
// KV-cache reuse -- entries of discarded tokens are removed before the next
// phase, without recomputation -- and on batch inference with paged attention
// and block tables, which lets each sequence keep its own length unpadded).
#include "sv_common.h"

namespace sv {

namespace {

__global__ __launch_bounds__(kThreads) void kv_truncate_kernel(KvArgs a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.B) return;
  const int64_t L = a.lens[b];
  const int64_t d = a.drop[b];
  const int64_t bs = a.block_size;
  const int64_t used = (L + bs - 1) / bs;
  const int64_t keep = (L - d + bs - 1) / bs;
  const bool ok = d >= 0 && d <= L && used <= a.max_blocks && used - keep <= a.max_freed;
  int32_t* row = a.table + static_cast<int64_t>(b) * a.max_blocks;
  int32_t* fr = a.freed ? a.freed + static_cast<int64_t>(b) * a.max_freed : nullptr;
  if (!ok) {
    for (int i = 0; i < a.max_freed; ++i) fr[i] = -1;
    a.num_freed[b] = -1;
    return;
  }
  const int n = static_cast<int>(used - keep);
  for (int i = 0; i < n; ++i) {
    fr[i] = row[keep + i];
    row[keep + i] = -1;
  }
  for (int i = n; i < a.max_freed; ++i) fr[i] = -1;
  a.num_freed[b] = n;
  a.lens[b] = static_cast<int32_t>(L - d);
}

}  // namespace

hipError_t launch_kv_truncate(const KvArgs& a, hipStream_t st) {
  const unsigned grid = static_cast<unsigned>((a.B + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(kv_truncate_kernel, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace sv
