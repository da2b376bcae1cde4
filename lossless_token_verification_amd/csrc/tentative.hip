// Pending tentative tokens across calls (HiSpec summary, section 2, bullet
// "Dynamische Verifizierungsrichtlinie": tentatively accepted tokens are
// accumulated, N_i = 4 by default, before the full model verifies them; bullet
// "Wiederverwendung von KV-Cache ...": entries of discarded tokens are dropped
// before the next phase).
//
// A round appends each active sequence's stage-1 output -- the a1 accepted
// drafts and the L_i correction or bonus y -- to its pending tokens, and the
// L_i rows 0..a1 (the rows those tokens were accepted or drawn under, stage
// 2's q) to its pending rows.  A flush verifies the pending tokens against the
// final exit (the verification kernel's flush mode) and empties the state.
#include "sv_args.h"

namespace sv {

namespace {

// One workgroup per (sequence, position j <= k, 64 KiB chunk): copies that
// chunk of L_i row j to pending row count + j (rows that would not fit are
// skipped; the count update flags them); workgroups past a1 exit at once.
// The (a1 + 1) x chunks others read the old count before they arrive on the
// sequence's counter; the last to arrive appends the a1 + 1 output tokens
// and advances the count.
template <int DT>
__global__ __launch_bounds__(kThreads) void append_rows_kernel(PendArgs a) {
  constexpr int ES = DT == 1 ? 2 : 4;
  constexpr int VPE = 16 / ES;
  constexpr int CE = kChunkBytes / ES;
  __shared__ int c0_sh;
  const int ch = blockIdx.x % a.nch;
  const int rest = blockIdx.x / a.nch;
  const int j = rest % (a.k + 1), b = rest / (a.k + 1);
  if (a.active && !a.active[b]) return;
  const int a1 = a.a1[b];
  if (j > a1) return;
  const int tid = threadIdx.x;
  if (tid == 0) c0_sh = min(max(a.count[b], 0), a.cap);
  __syncthreads();
  const int c0 = c0_sh;   // the old count, read before this workgroup arrives
  const int dst = c0 + j;
  if (dst < a.cap) {
    const char* src =
        static_cast<const char*>(a.li) + (static_cast<int64_t>(b) * (a.k + 1) + j) * a.ld * ES;
    char* out = static_cast<char*>(a.rows) + (static_cast<int64_t>(b) * a.cap + dst) * a.ld * ES;
    const int e0 = ch * CE, e1 = min(a.V, e0 + CE);
    if (((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(out)) & 15) == 0) {
      const int nfull = (e1 - e0) / VPE;
      const u32x4* s4 = reinterpret_cast<const u32x4*>(src) + e0 / VPE;
      u32x4* d4 = reinterpret_cast<u32x4*>(out) + e0 / VPE;
      for (int v = tid; v < nfull; v += kThreads) d4[v] = __builtin_nontemporal_load(s4 + v);
      for (int e = e0 + nfull * VPE + tid; e < e1; e += kThreads) {
        if constexpr (DT == 1)
          reinterpret_cast<uint16_t*>(out)[e] = reinterpret_cast<const uint16_t*>(src)[e];
        else
          reinterpret_cast<uint32_t*>(out)[e] = reinterpret_cast<const uint32_t*>(src)[e];
      }
    } else {
      for (int e = e0 + tid; e < e1; e += kThreads) {
        if constexpr (DT == 1)
          reinterpret_cast<uint16_t*>(out)[e] = reinterpret_cast<const uint16_t*>(src)[e];
        else
          reinterpret_cast<uint32_t*>(out)[e] = reinterpret_cast<const uint32_t*>(src)[e];
      }
    }
  }
  if (tid != 0) return;
  const int total = (a1 + 1) * a.nch;
  if (atomicAdd(a.arrive + b, 1) != total - 1) return;
  // every copying workgroup of the sequence has read the old count
  int n = a1 + 1;
  const int room = a.cap - c0;
  if (n > room) {
    atomicOr(a.flags, kFlagPendingFull);
    n = room > 0 ? room : 0;
  }
  for (int i = 0; i < n; ++i)
    a.tokens[static_cast<int64_t>(b) * a.cap + c0 + i] = a.t_out[static_cast<int64_t>(b) * (a.k + 1) + i];
  a.count[b] = c0 + n;
}

// Flush bookkeeping (one workgroup): lim = last pending position of a
// sequence with at least max(1, min_pending) pending tokens, else -1, and the
// list of rows the flush streams -- each flushed sequence's pending rows 0..c-1
// then its L_f rows 0..c-1, sequences in order (a workgroup-wide exclusive scan
// of 2c per batch of 256 sequences).  The flushed sequences' counts drop to 0
// here: the rest of the flush reads the limits, the list and the pending
// tokens and rows, never the count.
__global__ __launch_bounds__(kThreads) void flush_prep_kernel(PendArgs a) {
  __shared__ int scan[kThreads];
  const int tid = threadIdx.x;
  int base = 0;
  for (int b0 = 0; b0 < a.B; b0 += kThreads) {
    const int b = b0 + tid;
    int n = 0;
    if (b < a.B) {
      const int c = min(max(a.count[b], 0), a.cap);
      n = c >= max(1, a.min_pending) ? c : 0;
      a.lim[b] = n - 1;
      if (n > 0) a.count[b] = 0;
    }
    scan[tid] = 2 * n;
    __syncthreads();
    for (int o = 1; o < kThreads; o <<= 1) {   // inclusive scan (Hillis-Steele)
      const int v = tid >= o ? scan[tid - o] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int off = base + scan[tid] - 2 * n;
    for (int j = 0; j < n; ++j) {
      a.row_list[off + j] = a.row0_q + b * a.cap + j;
      a.row_list[off + n + j] = a.row0_p + b * (a.cap + 1) + j;
    }
    base += scan[kThreads - 1];
    __syncthreads();   // scan[] is rewritten by the next batch
  }
  if (tid == 0) *a.row_count = base;
}


}  // namespace

hipError_t launch_pending_append(const PendArgs& a, hipStream_t st) {
  const int64_t wg = static_cast<int64_t>(a.B) * (a.k + 1) * a.nch;
  if (wg == 0) return hipSuccess;
  if (a.dtype == 1)
    hipLaunchKernelGGL(append_rows_kernel<1>, dim3(static_cast<unsigned>(wg)), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(append_rows_kernel<0>, dim3(static_cast<unsigned>(wg)), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_flush_prep(const PendArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(flush_prep_kernel, dim3(1), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace sv
