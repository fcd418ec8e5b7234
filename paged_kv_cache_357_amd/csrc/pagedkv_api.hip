// C ABI of the paged KV-cache library: argument checks, launch planning and
// dispatch.  Nothing here allocates device memory or synchronises; every
// check happens on the host before the first launch.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "pagedkv.h"
#include "pkv_internal.h"

namespace {

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool valid_dtype(int dtype) { return dtype == PKV_DTYPE_F32 || dtype == PKV_DTYPE_BF16; }
int elt_bytes(int dtype) { return dtype == PKV_DTYPE_BF16 ? 2 : 4; }

struct Plan {
  int P = 0;
  int NP = 0;
  int n_units = 0;
  int n_wg = 0;
  int xcd_group = 0;
  int grid = 0;
  size_t acc_bytes = 0;  // workspace region of partial accumulators
  size_t ml_bytes = 0;   // workspace region of partial (max, sum) pairs
  size_t total() const { return acc_bytes + ml_bytes; }
};

#ifndef PKV_AUTO_PARTITION
#define PKV_AUTO_PARTITION 512
#endif

// Automatic partition size.  Sequences no longer than one partition are
// finished in a single pass; longer ones are cut into partitions of a fixed
// size, which bounds the work of one wave (so lengths that differ by 16x still
// spread evenly over the chip) at a merge cost of (D + 2) * 4 bytes per
// partition and query head.
int auto_partition(int max_len) {
  constexpr int kDefault = PKV_AUTO_PARTITION;
  if (max_len <= kDefault) return max_len <= pkv::kChunk ? pkv::kChunk : (max_len + 15) / 16 * 16;
  return kDefault;
}

int plan_sizes(int32_t num_seqs, int32_t q_heads, int32_t kv_heads, int32_t head_dim, int32_t block_size,
               int32_t max_context_len, int32_t dtype, int32_t partition_size, Plan* plan) {
  if (num_seqs < 0 || q_heads <= 0 || kv_heads <= 0 || max_context_len < 0) return PKV_ERR_SHAPE;
  if (!valid_dtype(dtype)) return PKV_ERR_DTYPE;
  if (q_heads % kv_heads) return PKV_ERR_SHAPE;
  const int group = q_heads / kv_heads;
  if (!(group == 1 || group == 2 || group == 4 || group == 8 || group == 16)) return PKV_ERR_UNSUPPORTED;
  if (!(head_dim == 64 || head_dim == 128)) return PKV_ERR_UNSUPPORTED;
  if (!(block_size == 16 || block_size == 32)) return PKV_ERR_UNSUPPORTED;
  int P = partition_size;
  if (P == 0) {
    P = auto_partition(max_context_len);
  } else if (P < pkv::kChunk || P > pkv::kMaxPartition || P % pkv::kChunk) {
    return PKV_ERR_UNSUPPORTED;
  }
  const long long np = max_context_len == 0 ? 1 : ((long long)max_context_len + P - 1) / P;
  // one wave per (partition, sequence, kv head); ids and the launch grid are int
  const long long units = np * num_seqs * kv_heads;
  const long long n_wg = (units + pkv::kWavesPerWG - 1) / pkv::kWavesPerWG;
  const long long seqs_grouped = num_seqs < pkv::kSeqGroup ? (num_seqs > 0 ? num_seqs : 1) : pkv::kSeqGroup;
  long long xg = (seqs_grouped * kv_heads) / pkv::kWavesPerWG;
  if (xg < 1) xg = 1;
  const long long span = (long long)pkv::kXcds * xg;
  const long long grid = (n_wg + span - 1) / span * span;
  if (grid > 0x7fffffffLL || (long long)num_seqs * q_heads > 0x7fffffffLL) return PKV_ERR_UNSUPPORTED;
  plan->P = P;
  plan->NP = (int)np;
  plan->n_units = (int)units;
  plan->n_wg = (int)n_wg;
  plan->xcd_group = (int)xg;
  plan->grid = (int)grid;
  if (plan->NP > 1) {
    const size_t rows = (size_t)num_seqs * q_heads * plan->NP;
    plan->acc_bytes = round_up(rows * head_dim * sizeof(float), 256);
    plan->ml_bytes = round_up(rows * 2 * sizeof(float), 256);
  } else {
    plan->acc_bytes = plan->ml_bytes = 0;
  }
  return PKV_OK;
}

int prepare_decode(float* out, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs, int32_t q_heads,
                   int32_t kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                   int32_t max_blocks_per_seq, int32_t max_context_len, float scale, int32_t dtype,
                   int32_t partition_size, void* workspace, size_t workspace_bytes, pkv::DecodeParams* p) {
  Plan plan;
  int st = plan_sizes(num_seqs, q_heads, kv_heads, head_dim, block_size, max_context_len, dtype, partition_size,
                      &plan);
  if (st != PKV_OK) return st;
  if (num_blocks <= 0 || max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
  if ((long long)max_context_len > (long long)max_blocks_per_seq * block_size) return PKV_ERR_SHAPE;
  if (num_seqs > 0 && (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)) return PKV_ERR_NULL;
  if (plan.total() > 0 && (!workspace || workspace_bytes < plan.total())) return PKV_ERR_WORKSPACE;
  (void)elt_bytes;
  p->out = out;
  p->ws_acc = plan.total() ? static_cast<float*>(workspace) : nullptr;
  p->ws_ml = plan.total() ? reinterpret_cast<float2*>(static_cast<char*>(workspace) + plan.acc_bytes) : nullptr;
  p->q = q;
  p->k = k_cache;
  p->v = v_cache;
  p->tables = block_tables;
  p->lens = context_lens;
  p->S = num_seqs;
  p->Hq = q_heads;
  p->Hkv = kv_heads;
  p->NB = num_blocks;
  p->MB = max_blocks_per_seq;
  p->max_len = max_context_len;
  p->P = plan.P;
  p->NP = plan.NP;
  p->n_units = plan.n_units;
  p->n_wg = plan.n_wg;
  p->xcd_group = plan.xcd_group;
  p->grid = plan.grid;
  p->scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)
  return PKV_OK;
}

}  // namespace

extern "C" {

int paged_kv_slot_mapping(int32_t* slot_mapping, const int32_t* block_tables, const int32_t* positions,
                          int32_t num_seqs, int32_t max_blocks_per_seq, int32_t block_size, int32_t num_blocks,
                          void* stream) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || block_size <= 0 || num_blocks <= 0) return PKV_ERR_SHAPE;
  if ((long long)num_blocks * block_size > 0x7fffffffLL) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!slot_mapping || !block_tables || !positions) return PKV_ERR_NULL;
  const hipError_t e = pkv::launch_slot_mapping(slot_mapping, block_tables, positions, num_seqs,
                                                max_blocks_per_seq, block_size, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int paged_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new, const int32_t* slot_mapping,
                    int32_t num_tokens, int32_t num_blocks, int32_t block_size, int32_t kv_heads, int32_t head_dim,
                    int32_t dtype, void* stream) {
  if (!valid_dtype(dtype)) return PKV_ERR_DTYPE;
  if (num_tokens < 0 || num_blocks <= 0 || block_size <= 0 || kv_heads <= 0 || head_dim <= 0) return PKV_ERR_SHAPE;
  const long long row = (long long)kv_heads * head_dim * elt_bytes(dtype);
  if (row % 16 || row > 0x7fffffffLL) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping) return PKV_ERR_NULL;
  const hipError_t e = pkv::launch_append(k_cache, v_cache, k_new, v_new, slot_mapping, num_tokens,
                                          (long long)num_blocks * block_size, (int)row,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int paged_attn_decode_plan(int32_t num_seqs, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t max_context_len, int32_t dtype, int32_t partition_size,
                           int32_t* resolved_partition_size, int32_t* num_partitions) {
  Plan plan;
  const int st = plan_sizes(num_seqs, q_heads, kv_heads, head_dim, block_size, max_context_len, dtype,
                            partition_size, &plan);
  if (st != PKV_OK) return st;
  if (resolved_partition_size) *resolved_partition_size = plan.P;
  if (num_partitions) *num_partitions = plan.NP;
  return PKV_OK;
}

size_t paged_attn_decode_workspace_size(int32_t num_seqs, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                                        int32_t block_size, int32_t max_context_len, int32_t dtype,
                                        int32_t partition_size) {
  Plan plan;
  if (plan_sizes(num_seqs, q_heads, kv_heads, head_dim, block_size, max_context_len, dtype, partition_size,
                 &plan) != PKV_OK)
    return 0;
  return plan.total();
}

int paged_attn_decode_partitions(float* out, const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                 int32_t q_heads, int32_t kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                                 float scale, int32_t dtype, int32_t partition_size, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  pkv::DecodeParams p;
  const int st = prepare_decode(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, q_heads, kv_heads,
                                head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, dtype,
                                partition_size, workspace, workspace_bytes, &p);
  if (st != PKV_OK) return st;
  const hipError_t e = pkv::launch_decode_partitions(p, dtype, head_dim, block_size, q_heads / kv_heads,
                                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int paged_attn_decode_reduce(float* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                             int32_t q_heads, int32_t kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                             int32_t dtype, int32_t partition_size, void* workspace, size_t workspace_bytes,
                             void* stream) {
  pkv::DecodeParams p;
  const int st = prepare_decode(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, q_heads, kv_heads,
                                head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, dtype,
                                partition_size, workspace, workspace_bytes, &p);
  if (st != PKV_OK) return st;
  const hipError_t e = pkv::launch_decode_reduce(p, head_dim, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int paged_attn_decode(float* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs, int32_t q_heads,
                      int32_t kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                      int32_t max_blocks_per_seq, int32_t max_context_len, float scale, int32_t dtype,
                      int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
  pkv::DecodeParams p;
  const int st = prepare_decode(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, q_heads, kv_heads,
                                head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, dtype,
                                partition_size, workspace, workspace_bytes, &p);
  if (st != PKV_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = pkv::launch_decode_partitions(p, dtype, head_dim, block_size, q_heads / kv_heads, s);
  if (e == hipSuccess) e = pkv::launch_decode_reduce(p, head_dim, s);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

const char* paged_status_str(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "null pointer";
    case PKV_ERR_SHAPE: return "invalid shape";
    case PKV_ERR_DTYPE: return "invalid dtype";
    case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

}  // extern "C"
