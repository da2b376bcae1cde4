// Internal definitions shared by the HIP sources of libspecverify.so:
// kernel argument blocks, the workspace layout, and small device helpers
// (bf16 decode, Philox4x32-10, wavefront reductions).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kThreads = 256;          // threads per workgroup of every kernel
constexpr int kWave = 64;              // CDNA wavefront width
constexpr int kWaves = kThreads / kWave;
constexpr int kVecPerThread = 16;      // 16-byte vectors each row-stats thread holds
constexpr int kChunkBytes = kThreads * kVecPerThread * 16;   // 64 KiB of one row
constexpr int kMaxPositions = 64;      // k + 1 <= 64
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxVocab = 1 << 20;
// Draw tiles of the largest vocabulary (fp32 has the most tiles).
constexpr int kMaxTiles = kMaxVocab / (kWave * 4);

constexpr uint32_t kFlagTokenRange = 1u;
constexpr uint32_t kFlagTemperature = 2u;

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

// Workspace: [flags (256 B)] [cnt1, cnt2, st1: 4 int32 per sequence, padded
// to 256 B] [partials: rows_total * nc]
constexpr size_t kFlagsBytes = 256;
constexpr int kLagSeqs = 32;

// One launch of the fused kernel: the HBM stream of row statistics plus, for
// each sequence, the verification run by the workgroup that completes its
// statistics.
struct FusedArgs {
  int32_t hier;            // 0: single stage (q = exit 0, p = exit 1); 1: L_d, L_i, L_f
  int32_t B, k, V, dtype, nc, window;
  int64_t ld;              // row stride in elements
  const void* exit_ptr[3];
  int32_t exit_row0[3];    // first global row id of each exit (partials layout)
  int32_t n1, n2;          // workgroups per sequence: stage-1 rows, L_f rows
  int32_t lag;             // L_f rows of sequence b follow stage-1 rows of b + lag
  Partial* partials;       // [rows_total * nc]
  int32_t* cnt1;           // [B] stage-1 chunks done
  int32_t* cnt2;           // [B] L_f chunks done + 1 when stage 1 is done
  uint64_t* st1;           // [B] stage-1 result: a1 | (correction or bonus token) << 32
  const int32_t* tokens;
  const float* temperature;
  uint32_t key0, key1, offset;
  int32_t* accept_len;        // a (single) or a1 (hier)
  int32_t* accept_len_final;  // a2 (hier) or NULL
  int32_t* out_tokens;
  int32_t* num_emitted;
  int32_t* num_drop;
  float* diag_uniforms;
  double* diag_probs;
  double* diag_draws;
  uint32_t* flags;
};

struct ClearArgs {
  int32_t n;
  int32_t* words;          // n int32 set to 0
  uint32_t* flags;
};

struct PackArgs {
  int32_t B, k;
  const int32_t* out_tokens;
  const int32_t* num_emitted;
  int32_t* packed;
  int32_t* cu_offsets;
};

struct KvArgs {
  int32_t B, max_blocks, block_size, max_freed;
  int32_t* table;
  int32_t* lens;
  const int32_t* drop;
  int32_t* freed;
  int32_t* num_freed;
};

hipError_t launch_clear(const ClearArgs& a, hipStream_t st);
hipError_t launch_fused(const FusedArgs& a, int64_t items, hipStream_t st);
hipError_t launch_pack(const PackArgs& a, hipStream_t st);
hipError_t launch_kv_truncate(const KvArgs& a, hipStream_t st);

// ---------------------------------------------------------------------------
// device helpers

// Publication of per-sequence data between workgroups without cache-wide
// fences: writers swap the words in with device-scope atomics and wait for the
// swaps to return before counting themselves done; readers load them with
// device-scope atomic loads, which read the coherent copy.
__device__ __forceinline__ void publish_u64(uint64_t* p, uint64_t v) {
  const unsigned long long old = atomicExch(reinterpret_cast<unsigned long long*>(p),
                                            static_cast<unsigned long long>(v));
  asm volatile("" ::"v"(old));   // the swap has completed before anything later is issued
}
__device__ __forceinline__ uint64_t fetch_u64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish_partial(Partial* dst, const Partial& v) {
  uint64_t* w = reinterpret_cast<uint64_t*>(dst);
  publish_u64(w, static_cast<uint64_t>(__float_as_uint(v.key)) |
                     (static_cast<uint64_t>(static_cast<uint32_t>(v.amax)) << 32));
  publish_u64(w + 1, static_cast<uint64_t>(__double_as_longlong(v.S)));
}
__device__ __forceinline__ Partial fetch_partial(const Partial* src) {
  const uint64_t* w = reinterpret_cast<const uint64_t*>(src);
  const uint64_t a = fetch_u64(w), b = fetch_u64(w + 1);
  Partial r;
  r.key = __uint_as_float(static_cast<uint32_t>(a));
  r.amax = static_cast<int32_t>(static_cast<uint32_t>(a >> 32));
  r.S = __longlong_as_double(static_cast<long long>(b));
  return r;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float load_elem(const void* row, int64_t i, int dtype) {
  if (dtype == 1) {
    const uint16_t h = static_cast<const uint16_t*>(row)[i];
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
  }
  return static_cast<const float*>(row)[i];
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of the
// two-multiply S-box; the key is bumped by the Weyl constants before every
// round after the first.
__device__ __forceinline__ uint4 philox4x32_10(uint4 x, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t m0 = static_cast<uint64_t>(0xD2511F53u) * x.x;
    const uint64_t m1 = static_cast<uint64_t>(0xCD9E8D57u) * x.z;
    const uint32_t hi0 = static_cast<uint32_t>(m0 >> 32), lo0 = static_cast<uint32_t>(m0);
    const uint32_t hi1 = static_cast<uint32_t>(m1 >> 32), lo1 = static_cast<uint32_t>(m1);
    x = make_uint4(hi1 ^ x.y ^ k0, lo1, hi0 ^ x.w ^ k1, lo0);
  }
  return x;
}

// 24-bit uniform in [0, 1 - 2^-24] from a 32-bit word (exact in float).
__device__ __forceinline__ float uniform24(uint32_t w) {
  return static_cast<float>(w >> 8) * 5.9604644775390625e-08f;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

}  // namespace sv
