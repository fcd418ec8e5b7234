// Internal declarations shared by the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Tokens a wavefront consumes per step.  Block sizes are multiples of it, and
// partitions start at multiples of it, so a chunk never straddles two
// physical blocks.
constexpr int kChunk = 16;
// Largest partition (tokens) one decode unit of the partitioned schedule covers.
constexpr int kMaxPartition = 8192;
// Waves per decode workgroup.  Each wave is an independent worker.
constexpr int kWavesPerWG = 4;
// SIMDs of a CDNA compute unit.
constexpr int kSimdsPerCU = 4;
// Compute units of one accelerator complex die (XCD) of gfx950, each XCD
// with its own L2; consecutive workgroup ids of a launch are dealt round robin
// over the XCDs.  The device's CU count is queried at run time; a whole
// MI355X has 256 CUs in 8 XCDs, a partition of it fewer.
constexpr int kCUsPerXcd = 32;
constexpr int kMaxXcds = 8;
// Sequences whose tiles the partitioned schedule keeps together on one XCD.
constexpr int kSeqGroup = 4;
// Longest batch the balanced schedule takes (its per-sequence tables live in
// LDS: 8 bytes per sequence).
constexpr int kBalancedMaxSeqs = 2048;
// Fewest chunks the balanced schedule gives one wave.
constexpr int kBalancedMinChunks = 8;
// Logical workgroups the balanced schedule keeps together on one XCD.
constexpr int kBalancedXcdGroup = 8;

// bf16 caches with at least this many query heads per kv head use the
// matrix-core kernels; everything else uses the vector-ALU kernels.
constexpr int kMfmaMinGroup = 4;

// Resident waves per SIMD each balanced-schedule kernel is compiled for (its
// register budget is capped accordingly); the balanced grid holds exactly
// that many waves on every SIMD of the chip, so all of them run at once.
// Fewer, deeper streams read the paged pool faster than many shallow ones.
#ifndef PKV_BALANCED_WAVES
#define PKV_BALANCED_WAVES 1
#endif
#ifndef PKV_PIPELINE
#define PKV_PIPELINE 3
#endif
constexpr __host__ __device__ int balanced_waves_per_simd(int dtype, int head_dim, int group) {
  return (dtype == 0 && (group >= 4 || (head_dim == 128 && group >= 2))) ? 1 : PKV_BALANCED_WAVES;
}
// Chunks in flight per wave in the balanced schedule (registers of the
// fp32 kernels with wide groups allow only two).
constexpr __host__ __device__ int balanced_pipeline_depth(int dtype, int head_dim, int group) {
  return (dtype == 0 && (group >= 4 || (head_dim == 128 && group >= 2))) ? 2 : PKV_PIPELINE;
}

// LDS one balanced-schedule workgroup may use (prefix tables, K staging
// tiles, finished-piece queues, fused-append rows): a gfx950 workgroup may
// allocate 160 KiB, and the balanced grid holds one workgroup per CU.  The
// most any wave's piece queue takes, and the most rows a wave keeps (larger
// queues measured slightly slower: the plain llama-shaped step lost about
// 0.7% with 32 KiB queues against 16 KiB).
constexpr int kLdsBudget = 160 * 1024;
constexpr int kQueueMaxBytes = 16 * 1024;
constexpr int kAppendRowsMax = 24;
// Bytes of one fused-append row kept in LDS: its pool offset (8 bytes, -1 for
// none, then 8 spare) and the new K and V rows of one kv head.
constexpr __host__ __device__ int append_row_entry_bytes(int dtype, int head_dim) {
  return 16 + 2 * head_dim * (dtype == 1 ? 2 : 4);
}
// Bytes of one queued finished piece: a 16-byte header (global destinations
// of the rows and of the (max, sum) pairs), group * head_dim floats, group
// (max, sum) pairs; a multiple of 16.
constexpr __host__ __device__ int piece_record_bytes(int group, int head_dim) {
  return (16 + 4 * group * head_dim + 8 * group + 15) & ~15;
}
// Per-wave LDS tile of the balanced stage-1 core (the matrix-core core stages
// a chunk's K rows, the vector core none).
constexpr __host__ __device__ int balanced_stage_bytes(int dtype, int head_dim, int group) {
  return (dtype == 1 && group >= kMfmaMinGroup) ? kChunk * head_dim * 2 : 16;
}

enum Schedule : int32_t {
  kPartitioned = 0,  // one wave per (partition, sequence, kv head)
  kBalanced = 1      // equal shares of all chunks, one share per resident wave
};

struct DecodeParams {
  float* out;             // [S, Hq, D]
  float* ws_acc;          // partial accumulators (rows of D)
  float2* ws_ml;          // partial (max, sum) pairs, one per accumulator row
  int32_t* ws_pref;       // balanced: [S + 1] chunk prefix sums, then [S + 1] cost prefix sums
  const void* q;          // [S, Hq, D]
  const void* k;          // [NB, B, Hkv, D]
  const void* v;          // [NB, B, Hkv, D]
  const int32_t* tables;  // [S, MB]
  const int32_t* lens;    // [S]
  const void* k_new;      // fused append: [S, Hkv, D] rows written at position lens[s]; else null
  const void* v_new;
  int32_t append;         // 1: lens hold the lengths before the fused append, L + 1 tokens are attended
  int32_t S, Hq, Hkv, NB, MB, max_len;
  int32_t schedule;       // Schedule
  int32_t P, NP;          // partitioned: partition size and count
  int32_t n_units;        // partitioned: decode units; balanced: worker waves
  int32_t n_wg;           // workgroups holding them: ceil(n_units / kWavesPerWG)
  int32_t xcd_group;      // consecutive logical workgroups kept on one XCD (0: no remap)
  int32_t xcds;           // XCDs of the device (launched workgroup b runs on XCD b % xcds)
  int32_t head_group;     // balanced: adjacent kv heads the waves of a workgroup take in lockstep (1 or 4)
  int32_t grid;           // launched workgroups (>= n_wg; the surplus exits at once)
  int32_t queue_bytes;    // balanced: LDS bytes of each wave's finished-piece queue (>= one record)
  int32_t row_bytes;      // balanced, fused append: LDS bytes of each wave's new rows (0: stored directly)
  int32_t fuse_rows;      // fused append: the balanced stage-1 kernel writes the new rows itself
  int32_t row_b;          // fused append: bytes of one token's K (or V) row over all kv heads
  int32_t block_size;
  float scale_log2;       // scale * log2(e): scores live in the base-2 domain
  // Shared-prefix decode (decode_shared.hip) only:
  int32_t* ws_share;      // [S] tokens sequence s shares with sequence s - 1 (0 for s = 0), prepare stage
  int32_t* ws_split;      // [workers][4]: the segment (group * head groups + head group) a worker began
                          // and left to later workers (or -1), its first member, columns, last worker
  int32_t max_members;    // sequences one group may hold: 16 / G (one matrix-product column per query row)
};

// Shared-prefix decode: query columns of one group (its members' query rows of
// one kv head) in a matrix-core tile, and the LDS ints its stage-1 prologue
// keeps per sequence (attended lengths, shares with the previous sequence,
// group ids, group starts, prefix lengths, chunk and cost prefix sums).
constexpr int kSharedCols = 16;
constexpr __host__ __device__ int shared_lds_ints(int num_seqs) { return 7 * num_seqs + 4; }
// Bytes of one queued finished piece of the shared-prefix kernel with `cols`
// query columns: a 32-byte header, cols * head_dim floats, cols (max, sum)
// pairs; a multiple of 16.
constexpr __host__ __device__ int shared_record_bytes(int cols, int head_dim) {
  return (32 + cols * (4 * head_dim + 8) + 15) & ~15;
}

// Stage 1 / stage 2 launchers (decode.hip).  Return hipSuccess or the launch error.
hipError_t launch_decode_partitions(const DecodeParams& p, int dtype, int head_dim, int block_size,
                                    int group, hipStream_t stream);
hipError_t launch_decode_reduce(const DecodeParams& p, int head_dim, int group, hipStream_t stream);

// Shared-prefix decode launchers (decode_shared.hip): the prepare stage
// (fused-append rows, prefix shared with the previous sequence), stage 1 and
// the merge.  bf16 caches only.
hipError_t launch_shared_prepare(const DecodeParams& p, int head_dim, hipStream_t stream);
hipError_t launch_shared_stage1(const DecodeParams& p, int head_dim, int block_size, int group, hipStream_t stream);
hipError_t launch_shared_merge(const DecodeParams& p, int head_dim, int group, hipStream_t stream);

}  // namespace pkv
