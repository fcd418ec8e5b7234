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
// Largest partition (tokens) one decode unit covers.
constexpr int kMaxPartition = 8192;
// Waves per decode workgroup.  Each wave is an independent work unit.
constexpr int kWavesPerWG = 4;
// Accelerator complex dies of the MI355X; consecutive workgroup ids of a
// launch are dealt round robin over them.
constexpr int kXcds = 8;
// Sequences whose tiles are kept together on one XCD (so that sequences
// forked from one prompt, which are usually neighbours, read the shared
// blocks through the same L2).
#ifndef PKV_SEQ_GROUP
#define PKV_SEQ_GROUP 4
#endif
constexpr int kSeqGroup = PKV_SEQ_GROUP;

struct DecodeParams {
  float* out;             // [S, Hq, D]
  float* ws_acc;          // [S, Hq, NP, D]     (NP > 1 only)
  float2* ws_ml;          // [S, Hq, NP] (m, l) (NP > 1 only)
  const void* q;          // [S, Hq, D]
  const void* k;          // [NB, B, Hkv, D]
  const void* v;          // [NB, B, Hkv, D]
  const int32_t* tables;  // [S, MB]
  const int32_t* lens;    // [S]
  int32_t S, Hq, Hkv, NB, MB, max_len, P, NP;
  int32_t n_units;        // NP * S * Hkv decode units (one wave each)
  int32_t n_wg;           // workgroups holding them: ceil(n_units / kWavesPerWG)
  int32_t xcd_group;      // consecutive logical workgroups kept on one XCD (0: no remap)
  int32_t grid;           // launched workgroups (>= n_wg; the surplus exits at once)
  float scale_log2;       // scale * log2(e): scores live in the base-2 domain
};

// Stage 1 / stage 2 launchers (decode.hip).  Return hipSuccess or the launch error.
hipError_t launch_decode_partitions(const DecodeParams& p, int dtype, int head_dim, int block_size,
                                    int group, hipStream_t stream);
hipError_t launch_decode_reduce(const DecodeParams& p, int head_dim, hipStream_t stream);

// Slot mapping and append launchers (append.hip).
hipError_t launch_slot_mapping(int32_t* slots, const int32_t* tables, const int32_t* positions, int S, int MB,
                               int B, hipStream_t stream);
hipError_t launch_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                         const int32_t* slots, int N, long long num_slots, int row_bytes, hipStream_t stream);

}  // namespace pkv
