// Slot mapping, KV append and the copy-on-write block copy for gfx950.
//
// Slot of logical position p: T[p / B] * B + p % B ("PagedAttention Paper
// Breakdown", section 2, Address Translation Formula).  A sequence holding L
// tokens writes its next token at position L, into the block the engine added
// to its table when L reached a block boundary ("PagedAttention and vLLM
// Architecture", Why Internal Fragmentation is Bounded).  K and V of a token
// share the slot (same page, section 1).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_internal.h"
#include "pkv_ops.h"

namespace pkv {
namespace {

// A position outside the table or a block id outside [0, NB) gives slot -1,
// so a stray entry can never name another block's slot (the product of an id
// and B is taken only for ids inside the pool, where it fits in int32).
__global__ __launch_bounds__(256) void slot_mapping_kernel(int32_t* __restrict__ slots,
                                                           const int32_t* __restrict__ tables,
                                                           const int32_t* __restrict__ positions, int S, int MB,
                                                           int B, int NB) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= S) return;
  const int p = positions[s];
  int slot = -1;
  if (p >= 0 && (long long)p < (long long)MB * B) {
    const int b = p / B;
    const int blk = tables[(size_t)s * MB + b];
    if (blk >= 0 && blk < NB) slot = blk * B + (p - b * B);
  }
  slots[s] = slot;
}

// One thread per 16-byte column of a row; consecutive threads cover
// consecutive columns of one token's row, so both the read of k_new / v_new
// and the write into the slot are fully coalesced.
__global__ __launch_bounds__(256) void append_kernel(char* __restrict__ kc, char* __restrict__ vc,
                                                     const char* __restrict__ kn, const char* __restrict__ vn,
                                                     const int32_t* __restrict__ slots, int N, long long num_slots,
                                                     int cols16) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long t = gid / cols16;
  const int c = (int)(gid - t * cols16);
  if (t >= N) return;
  const int slot = slots[t];
  if (slot < 0 || (long long)slot >= num_slots) return;
  const size_t row = (size_t)cols16 * 16;
  const uint4 kv = reinterpret_cast<const uint4*>(kn + (size_t)t * row)[c];
  const uint4 vv = reinterpret_cast<const uint4*>(vn + (size_t)t * row)[c];
  reinterpret_cast<uint4*>(kc + (size_t)slot * row)[c] = kv;
  reinterpret_cast<uint4*>(vc + (size_t)slot * row)[c] = vv;
}

// Slot mapping and append in one pass: thread (t, c) computes the slot of
// sequence t's position itself (every thread of the row gets the same value
// from the same two loads), copies column c, and column 0 records the slot.
// A position outside [0, pos_end) (pos_end at most the table's extent) or a
// block id outside the pool gives slot -1 and no write.
__global__ __launch_bounds__(256) void append_at_kernel(char* __restrict__ kc, char* __restrict__ vc,
                                                        const char* __restrict__ kn, const char* __restrict__ vn,
                                                        const int32_t* __restrict__ tables,
                                                        const int32_t* __restrict__ positions,
                                                        int32_t* __restrict__ slots, int N, int MB, int B, int NB,
                                                        int cols16, long long pos_end) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long t = gid / cols16;
  const int c = (int)(gid - t * cols16);
  if (t >= N) return;
  const int p = positions[t];
  int slot = -1;
  if (p >= 0 && (long long)p < pos_end) {
    const int b = p / B;
    const int blk = tables[(size_t)t * MB + b];
    if (blk >= 0 && blk < NB) slot = blk * B + (p - b * B);
  }
  if (slots != nullptr && c == 0) slots[t] = slot;
  if (slot < 0) return;
  const size_t row = (size_t)cols16 * 16;
  const uint4 kv = reinterpret_cast<const uint4*>(kn + (size_t)t * row)[c];
  const uint4 vv = reinterpret_cast<const uint4*>(vn + (size_t)t * row)[c];
  reinterpret_cast<uint4*>(kc + (size_t)slot * row)[c] = kv;
  reinterpret_cast<uint4*>(vc + (size_t)slot * row)[c] = vv;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Copy-on-write block copy ("PagedAttention and vLLM Architecture", section
// 3): block src[pair] -> block dst[pair] of both caches.  blockIdx.y picks the
// pair, blockIdx.x a 16 KiB slice of the block; each thread moves four
// 16-byte vectors of K and four of V with all eight loads in flight.  The data
// is touched once, so loads and stores are nontemporal.
constexpr int kCopyPerThread = 4;
constexpr int kCopyVecPerWG = 256 * kCopyPerThread;

__global__ __launch_bounds__(256) void copy_blocks_kernel(char* __restrict__ kc, char* __restrict__ vc,
                                                          const int32_t* __restrict__ src,
                                                          const int32_t* __restrict__ dst, int NB, int vpb,
                                                          long long block_bytes, int pair0) {
  const int pair = pair0 + (int)blockIdx.y;
  const int s = src[pair];
  const int d = dst[pair];
  if (s < 0 || s >= NB || d < 0 || d >= NB) return;
  const u32x4* ks = reinterpret_cast<const u32x4*>(kc + (size_t)s * (size_t)block_bytes);
  const u32x4* vs = reinterpret_cast<const u32x4*>(vc + (size_t)s * (size_t)block_bytes);
  u32x4* kd = reinterpret_cast<u32x4*>(kc + (size_t)d * (size_t)block_bytes);
  u32x4* vd = reinterpret_cast<u32x4*>(vc + (size_t)d * (size_t)block_bytes);
  const int base = (int)blockIdx.x * kCopyVecPerWG + (int)threadIdx.x;
  u32x4 a[kCopyPerThread], b[kCopyPerThread];
#pragma unroll
  for (int i = 0; i < kCopyPerThread; ++i) {
    const int j = base + i * 256;
    if (j < vpb) {
      a[i] = __builtin_nontemporal_load(ks + j);
      b[i] = __builtin_nontemporal_load(vs + j);
    }
  }
#pragma unroll
  for (int i = 0; i < kCopyPerThread; ++i) {
    const int j = base + i * 256;
    if (j < vpb) {
      __builtin_nontemporal_store(a[i], kd + j);
      __builtin_nontemporal_store(b[i], vd + j);
    }
  }
}

// Swap staging: move whole blocks between the pool and a contiguous staging
// area.  gather: staging slot i <- pool block ids[i]; otherwise pool block
// ids[i] <- staging slot i.  Same tiling as the block copy.
__global__ __launch_bounds__(256) void stage_blocks_kernel(char* __restrict__ pk, char* __restrict__ pv,
                                                           char* __restrict__ sk, char* __restrict__ sv,
                                                           const int32_t* __restrict__ ids, int NB, int vpb,
                                                           long long block_bytes, int gather, int pair0) {
  const int i = pair0 + (int)blockIdx.y;
  const int b = ids[i];
  if (b < 0 || b >= NB) return;
  const size_t pool_off = (size_t)b * (size_t)block_bytes, stage_off = (size_t)i * (size_t)block_bytes;
  const u32x4* fk = reinterpret_cast<const u32x4*>(gather ? pk + pool_off : sk + stage_off);
  const u32x4* fv = reinterpret_cast<const u32x4*>(gather ? pv + pool_off : sv + stage_off);
  u32x4* tk = reinterpret_cast<u32x4*>(gather ? sk + stage_off : pk + pool_off);
  u32x4* tv = reinterpret_cast<u32x4*>(gather ? sv + stage_off : pv + pool_off);
  const int base = (int)blockIdx.x * kCopyVecPerWG + (int)threadIdx.x;
  u32x4 a[kCopyPerThread], c[kCopyPerThread];
#pragma unroll
  for (int k = 0; k < kCopyPerThread; ++k) {
    const int j = base + k * 256;
    if (j < vpb) {
      a[k] = __builtin_nontemporal_load(fk + j);
      c[k] = __builtin_nontemporal_load(fv + j);
    }
  }
#pragma unroll
  for (int k = 0; k < kCopyPerThread; ++k) {
    const int j = base + k * 256;
    if (j < vpb) {
      __builtin_nontemporal_store(a[k], tk + j);
      __builtin_nontemporal_store(c[k], tv + j);
    }
  }
}

}  // namespace

hipError_t launch_stage_blocks(void* pool_k, void* pool_v, void* stage_k, void* stage_v, const int32_t* ids, int n,
                               int num_blocks, long long block_bytes, bool gather, hipStream_t stream) {
  const int vpb = (int)(block_bytes / 16);
  const unsigned gx = (unsigned)((vpb + kCopyVecPerWG - 1) / kCopyVecPerWG);
  for (int p0 = 0; p0 < n; p0 += 65535) {
    const unsigned gy = (unsigned)((n - p0) < 65535 ? (n - p0) : 65535);
    hipLaunchKernelGGL(stage_blocks_kernel, dim3(gx, gy), dim3(256), 0, stream, static_cast<char*>(pool_k),
                       static_cast<char*>(pool_v), static_cast<char*>(stage_k), static_cast<char*>(stage_v), ids,
                       num_blocks, vpb, block_bytes, gather ? 1 : 0, p0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst, int n_pairs,
                              int num_blocks, long long block_bytes, hipStream_t stream) {
  const int vpb = (int)(block_bytes / 16);
  const unsigned gx = (unsigned)((vpb + kCopyVecPerWG - 1) / kCopyVecPerWG);
  for (int p0 = 0; p0 < n_pairs; p0 += 65535) {  // grid y is at most 65535
    const unsigned gy = (unsigned)((n_pairs - p0) < 65535 ? (n_pairs - p0) : 65535);
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(gx, gy), dim3(256), 0, stream, static_cast<char*>(k_cache),
                       static_cast<char*>(v_cache), src, dst, num_blocks, vpb, block_bytes, p0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_append_at(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                            const int32_t* tables, const int32_t* positions, int32_t* slots, int N, int MB, int B,
                            int NB, int row_bytes, long long pos_end, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const int cols16 = row_bytes / 16;
  const long long total = (long long)N * cols16;
  const int threads = 256;
  const long long blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(append_at_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, static_cast<char*>(k_cache),
                     static_cast<char*>(v_cache), static_cast<const char*>(k_new), static_cast<const char*>(v_new),
                     tables, positions, slots, N, MB, B, NB, cols16, pos_end);
  return hipGetLastError();
}

hipError_t launch_slot_mapping(int32_t* slots, const int32_t* tables, const int32_t* positions, int S, int MB,
                               int B, int NB, hipStream_t stream) {
  if (S == 0) return hipSuccess;
  const int threads = 256;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3((S + threads - 1) / threads), dim3(threads), 0, stream, slots,
                     tables, positions, S, MB, B, NB);
  return hipGetLastError();
}

hipError_t launch_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new, const int32_t* slots,
                         int N, long long num_slots, int row_bytes, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const int cols16 = row_bytes / 16;
  const long long total = (long long)N * cols16;
  const int threads = 256;
  const long long blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, static_cast<char*>(k_cache),
                     static_cast<char*>(v_cache), static_cast<const char*>(k_new), static_cast<const char*>(v_new),
                     slots, N, num_slots, cols16);
  return hipGetLastError();
}

}  // namespace pkv
