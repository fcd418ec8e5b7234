// Internal declarations of the non-decode kernels: slot mapping, append,
// block copy (append.hip) and the prompt pass (prefill.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Prompt pass: query columns per wave ((token, head) pairs of 32 / G tokens).
constexpr int kPrefillColumns = 32;

// Arguments of the prompt (prefill) attention kernel.
struct PrefillParams {
  float* out;               // [total_q, Hq, D]
  const void* q;            // [total_q, Hq, D]
  const void* k;            // [NB, B, Hkv, D]
  const void* v;            // [NB, B, Hkv, D]
  const int32_t* tables;    // [S, MB]
  const int32_t* lens;      // [S] tokens held, the new chunk included
  const int32_t* q_start;   // [S + 1] rows of sequence s: q_start[s] .. q_start[s+1]-1
  int32_t S, Hq, Hkv, NB, MB, max_len;
  int32_t n_qt;             // workgroup tiles per (sequence, kv head): ceil(max_q_len / tile tokens)
  int32_t n_units;          // S * Hkv * n_qt workgroups
  float scale_log2;
};

hipError_t launch_prefill(const PrefillParams& p, int head_dim, int block_size, int group, hipStream_t stream);

// Slot mapping and append launchers (append.hip).
// Positions outside the table and block ids outside [0, NB) give slot -1.
hipError_t launch_slot_mapping(int32_t* slots, const int32_t* tables, const int32_t* positions, int S, int MB,
                               int B, int NB, hipStream_t stream);
hipError_t launch_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                         const int32_t* slots, int N, long long num_slots, int row_bytes, hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst, int n_pairs,
                              int num_blocks, long long block_bytes, hipStream_t stream);
hipError_t launch_stage_blocks(void* pool_k, void* pool_v, void* stage_k, void* stage_v, const int32_t* ids, int n,
                               int num_blocks, long long block_bytes, bool gather, hipStream_t stream);
// Positions outside [0, pos_end) are skipped (pos_end <= MB * B).
hipError_t launch_append_at(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                            const int32_t* tables, const int32_t* positions, int32_t* slots, int N, int MB, int B,
                            int NB, int row_bytes, long long pos_end, hipStream_t stream);

}  // namespace pkv
