// C ABI of the paged KV-cache library: argument checks, launch planning and
// dispatch.  Nothing here allocates device memory or synchronises; every
// check happens on the host before the first launch.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "pagedkv.h"
#include "pkv_internal.h"
#include "pkv_ops.h"

namespace {

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Compute units and XCDs of the calling thread's current device, queried once
// per device.  Without a device (the planning calls used on a host with no
// GPU) a whole MI355X is assumed: 256 CUs in 8 XCDs.
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_cus[kMaxDevices];

struct ChipShape {
  int cus;
  int xcds;
};

ChipShape chip_shape() {
  ChipShape c{pkv::kCUsPerXcd * pkv::kMaxXcds, pkv::kMaxXcds};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();  // leave no sticky error behind for the caller
    return c;
  }
  int cus = g_device_cus[dev].load(std::memory_order_relaxed);
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
      (void)hipGetLastError();
      return c;
    }
    g_device_cus[dev].store(cus, std::memory_order_relaxed);
  }
  c.cus = cus;
  c.xcds = cus / pkv::kCUsPerXcd;
  if (c.xcds < 1) c.xcds = 1;
  if (c.xcds > pkv::kMaxXcds) c.xcds = pkv::kMaxXcds;
  return c;
}

bool valid_dtype(int dtype) { return dtype == PKV_DTYPE_F32 || dtype == PKV_DTYPE_BF16; }
int elt_bytes(int dtype) { return dtype == PKV_DTYPE_BF16 ? 2 : 4; }

struct Plan {
  int schedule = pkv::kPartitioned;
  int P = 0;             // partitioned: tokens per partition
  int NP = 0;            // partitioned: partitions per sequence
  int n_units = 0;       // partitioned: decode units; balanced: worker waves
  int n_wg = 0;
  int xcd_group = 0;
  int xcds = pkv::kMaxXcds;
  int head_group = 1;
  int grid = 0;
  int queue_bytes = 0;   // balanced: LDS queue of finished pieces per wave
  size_t acc_bytes = 0;  // workspace region of partial accumulators
  size_t ml_bytes = 0;   // workspace region of partial (max, sum) pairs
  size_t pref_bytes = 0; // workspace region of per-sequence chunk and cost prefix sums (balanced)
  size_t share_bytes = 0;  // shared-prefix decode: per-sequence shares with the previous sequence
  size_t split_bytes = 0;  // shared-prefix decode: per-worker split segments for the merge
  bool shared = false;     // the shared-prefix kernels run this plan
  size_t total() const { return acc_bytes + ml_bytes + pref_bytes + share_bytes + split_bytes; }
};

// Automatic partition size of the partitioned schedule.  A batch whose
// longest sequence fits in one partition is finished in a single pass with
// no merge; longer ones use the balanced schedule when it applies, else
// partitions of this size.
constexpr int kAutoPartition = 512;

int auto_partition(int max_len) {
  if (max_len <= kAutoPartition) return max_len <= pkv::kChunk ? pkv::kChunk : (max_len + 15) / 16 * 16;
  return kAutoPartition;
}

// Consecutive logical workgroups put on one XCD, and the launched grid.
void set_grid(long long n_wg, long long group, Plan* plan) {
  const long long span = (long long)plan->xcds * group;
  plan->n_wg = (int)n_wg;
  plan->xcd_group = (int)group;
  plan->grid = (int)((n_wg + span - 1) / span * span);
}

// LDS left to each wave of a balanced workgroup for its queues, a multiple of 16.
long long balanced_wave_lds(int32_t num_seqs, int32_t head_dim, int group, int32_t dtype) {
  const long long fixed = (long long)round_up((3 * (size_t)num_seqs + 2) * 4, 16) +
                          (long long)pkv::kWavesPerWG * pkv::balanced_stage_bytes(dtype, head_dim, group) + 256;
  return ((pkv::kLdsBudget - fixed) / pkv::kWavesPerWG) & ~15LL;
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
  if (partition_size != 0 &&
      (partition_size < pkv::kChunk || partition_size > pkv::kMaxPartition || partition_size % pkv::kChunk))
    return PKV_ERR_UNSUPPORTED;
  if ((long long)num_seqs * q_heads > 0x7fffffffLL) return PKV_ERR_UNSUPPORTED;
  const ChipShape chip = chip_shape();
  plan->xcds = chip.xcds;

  // Balanced schedule: automatic partitioning, some sequence longer than one
  // partition, a batch whose tables fit in LDS, and chunk counts whose
  // products with the worker count stay within 62 bits.
  const long long chunk_bound = (long long)num_seqs * kv_heads * ((max_context_len + pkv::kChunk - 1) / pkv::kChunk);
  // the kernels keep chunk and cost prefix sums over sequences in int
  const bool sums_fit = (long long)num_seqs * ((max_context_len + pkv::kChunk - 1) / pkv::kChunk + 2) < (1LL << 31);
  const bool spills = dtype == PKV_DTYPE_F32 && head_dim == 128 && group == 16;  // one wave per SIMD is not enough
  // Each wave keeps its finished pieces in an LDS queue and writes them out
  // at its end; the queue takes what the prefix tables and staging tiles
  // leave of the LDS budget, and must hold at least one piece.
  const long long wave_lds = balanced_wave_lds(num_seqs, head_dim, group, dtype);
  long long queue = wave_lds > pkv::kQueueMaxBytes ? pkv::kQueueMaxBytes : wave_lds;
  const bool queue_fits = queue >= pkv::piece_record_bytes(group, head_dim);
  if (partition_size == 0 && max_context_len > kAutoPartition && num_seqs <= pkv::kBalancedMaxSeqs &&
      chunk_bound < (1LL << 48) && sums_fit && !spills && queue_fits) {
    const long long waves =
        (long long)chip.cus * pkv::kSimdsPerCU * pkv::balanced_waves_per_simd(dtype, head_dim, group);
    plan->schedule = pkv::kBalanced;
    plan->P = 0;
    plan->NP = 0;
    plan->queue_bytes = (int)queue;
    // matrix-core kernels: four waves of a workgroup on four adjacent heads
    plan->head_group = (dtype == PKV_DTYPE_BF16 && group >= pkv::kMfmaMinGroup && kv_heads % 4 == 0) ? 4 : 1;
    plan->n_units = (int)waves;
    set_grid(waves / pkv::kWavesPerWG, pkv::kBalancedXcdGroup, plan);
    const size_t rows = (size_t)waves * 2 * group;  // two partial slots per wave, a row per query head
    plan->acc_bytes = round_up(rows * head_dim * sizeof(float), 256);
    plan->ml_bytes = round_up(rows * 2 * sizeof(float), 256);
    plan->pref_bytes = round_up(2 * ((size_t)num_seqs + 1) * sizeof(int32_t), 256);
    return PKV_OK;
  }

  const int P = partition_size == 0 ? auto_partition(max_context_len) : partition_size;
  const long long np = max_context_len == 0 ? 1 : ((long long)max_context_len + P - 1) / P;
  // one wave per (partition, sequence, kv head); ids and the launch grid are int
  const long long units = np * num_seqs * kv_heads;
  const long long n_wg = (units + pkv::kWavesPerWG - 1) / pkv::kWavesPerWG;
  const long long seqs_grouped = num_seqs < pkv::kSeqGroup ? (num_seqs > 0 ? num_seqs : 1) : pkv::kSeqGroup;
  long long xg = (seqs_grouped * kv_heads) / pkv::kWavesPerWG;
  if (xg < 1) xg = 1;
  const long long span = (long long)plan->xcds * xg;
  if ((n_wg + span - 1) / span * span > 0x7fffffffLL) return PKV_ERR_UNSUPPORTED;
  plan->schedule = pkv::kPartitioned;
  plan->P = P;
  plan->NP = (int)np;
  plan->n_units = (int)units;
  set_grid(n_wg, xg, plan);
  if (plan->NP > 1) {
    const size_t rows = (size_t)num_seqs * q_heads * plan->NP;
    plan->acc_bytes = round_up(rows * head_dim * sizeof(float), 256);
    plan->ml_bytes = round_up(rows * 2 * sizeof(float), 256);
  }
  return PKV_OK;
}

// Shared-prefix plan ("PagedAttention and vLLM Architecture", section 3:
// forked sequences share their prompt's blocks): the balanced layout of
// (group, kv head group) segments on matrix-core workers.  Applies to bf16
// caches and batches whose tables fit the LDS; *applies is false (and the
// plain plan is returned) otherwise.
int plan_shared(int32_t num_seqs, int32_t q_heads, int32_t kv_heads, int32_t head_dim, int32_t block_size,
                int32_t max_context_len, int32_t dtype, Plan* plan) {
  int st = plan_sizes(num_seqs, q_heads, kv_heads, head_dim, block_size, max_context_len, dtype, 0, plan);
  if (st != PKV_OK) return st;
  if (dtype != PKV_DTYPE_BF16 || num_seqs < 1 || num_seqs > pkv::kBalancedMaxSeqs) return PKV_OK;
  if ((long long)num_seqs * ((max_context_len + pkv::kChunk - 1) / pkv::kChunk + 2) >= (1LL << 31)) return PKV_OK;
  const long long fixed = (long long)round_up((size_t)pkv::shared_lds_ints(num_seqs) * 4, 16) +
                          (long long)pkv::kWavesPerWG * pkv::balanced_stage_bytes(dtype, head_dim, pkv::kSharedCols) +
                          256;
  long long queue = ((pkv::kLdsBudget - fixed) / pkv::kWavesPerWG) & ~15LL;
  if (queue > pkv::kQueueMaxBytes) queue = pkv::kQueueMaxBytes;
  if (queue < pkv::shared_record_bytes(pkv::kSharedCols, head_dim)) return PKV_OK;
  const ChipShape chip = chip_shape();
  Plan sp;
  sp.shared = true;
  sp.xcds = chip.xcds;
  sp.schedule = pkv::kBalanced;
  sp.queue_bytes = (int)queue;
  sp.head_group = kv_heads % 4 == 0 ? 4 : 1;
  const long long waves = (long long)chip.cus * pkv::kSimdsPerCU;  // one matrix-core worker wave per SIMD
  sp.n_units = (int)waves;
  set_grid(waves / pkv::kWavesPerWG, pkv::kBalancedXcdGroup, &sp);
  const size_t rows = (size_t)waves * 2 * pkv::kSharedCols;  // two partial slots per wave, a row per column
  sp.acc_bytes = round_up(rows * head_dim * sizeof(float), 256);
  sp.ml_bytes = round_up(rows * 2 * sizeof(float), 256);
  sp.share_bytes = round_up((size_t)num_seqs * sizeof(int32_t), 256);
  sp.split_bytes = round_up((size_t)waves * 4 * sizeof(int32_t), 256);
  *plan = sp;
  return PKV_OK;
}

// Checks every pointer and size of a decode call against `plan` and fills
// the kernel parameters.
int fill_decode(const Plan& plan, float* out, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs, int32_t q_heads,
                int32_t kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                int32_t max_blocks_per_seq, int32_t max_context_len, float scale, void* workspace,
                size_t workspace_bytes, pkv::DecodeParams* p) {
  (void)head_dim;
  if (num_blocks <= 0 || max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
  if ((long long)max_context_len > (long long)max_blocks_per_seq * block_size) return PKV_ERR_SHAPE;
  if (num_seqs > 0 && (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)) return PKV_ERR_NULL;
  if (plan.total() > 0 && (!workspace || workspace_bytes < plan.total())) return PKV_ERR_WORKSPACE;
  (void)elt_bytes;
  p->out = out;
  char* ws = plan.total() ? static_cast<char*>(workspace) : nullptr;
  p->ws_acc = ws ? reinterpret_cast<float*>(ws) : nullptr;
  p->ws_ml = ws ? reinterpret_cast<float2*>(ws + plan.acc_bytes) : nullptr;
  p->ws_pref = ws ? reinterpret_cast<int32_t*>(ws + plan.acc_bytes + plan.ml_bytes) : nullptr;
  p->ws_share = plan.shared ? reinterpret_cast<int32_t*>(ws + plan.acc_bytes + plan.ml_bytes + plan.pref_bytes) : nullptr;
  p->ws_split = plan.shared ? p->ws_share + plan.share_bytes / sizeof(int32_t) : nullptr;
  p->max_members = plan.shared ? pkv::kSharedCols / (q_heads / kv_heads) : 0;
  p->schedule = plan.schedule;
  p->q = q;
  p->k = k_cache;
  p->v = v_cache;
  p->tables = block_tables;
  p->lens = context_lens;
  p->k_new = nullptr;
  p->v_new = nullptr;
  p->append = 0;
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
  p->xcds = plan.xcds;
  p->head_group = plan.head_group;
  p->grid = plan.grid;
  p->queue_bytes = plan.queue_bytes;
  p->row_bytes = 0;
  p->fuse_rows = 0;
  p->row_b = 0;
  p->block_size = block_size;
  p->scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)
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
  return fill_decode(plan, out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, q_heads, kv_heads,
                     head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, workspace,
                     workspace_bytes, p);
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
                                                max_blocks_per_seq, block_size, num_blocks,
                                                static_cast<hipStream_t>(stream));
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

int paged_kv_append_at(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                       const int32_t* block_tables, const int32_t* positions, int32_t* slot_mapping,
                       int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks, int32_t block_size,
                       int32_t kv_heads, int32_t head_dim, int32_t dtype, void* stream) {
  if (!valid_dtype(dtype)) return PKV_ERR_DTYPE;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || block_size <= 0 || kv_heads <= 0 ||
      head_dim <= 0)
    return PKV_ERR_SHAPE;
  if ((long long)num_blocks * block_size > 0x7fffffffLL) return PKV_ERR_SHAPE;
  const long long row = (long long)kv_heads * head_dim * elt_bytes(dtype);
  if (row % 16 || row > 0x7fffffffLL) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !block_tables || !positions) return PKV_ERR_NULL;
  const hipError_t e = pkv::launch_append_at(k_cache, v_cache, k_new, v_new, block_tables, positions, slot_mapping,
                                             num_seqs, max_blocks_per_seq, block_size, num_blocks, (int)row,
                                             (long long)max_blocks_per_seq * block_size, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int paged_kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst, int32_t n_pairs,
                         int32_t num_blocks, int32_t block_size, int32_t kv_heads, int32_t head_dim, int32_t dtype,
                         void* stream) {
  if (!valid_dtype(dtype)) return PKV_ERR_DTYPE;
  if (n_pairs < 0 || num_blocks <= 0 || block_size <= 0 || kv_heads <= 0 || head_dim <= 0) return PKV_ERR_SHAPE;
  const long long row = (long long)kv_heads * head_dim * elt_bytes(dtype);
  if (row % 16) return PKV_ERR_SHAPE;
  const long long block_bytes = row * block_size;
  if (block_bytes > 0x7fffffffLL) return PKV_ERR_SHAPE;
  if (n_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !src || !dst) return PKV_ERR_NULL;
  const hipError_t e = pkv::launch_copy_blocks(k_cache, v_cache, src, dst, n_pairs, num_blocks, block_bytes,
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int paged_attn_prefill(float* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens, const int32_t* q_start,
                       int32_t num_seqs, int32_t max_q_len, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                       float scale, int32_t dtype, void* stream) {
  if (!valid_dtype(dtype)) return PKV_ERR_DTYPE;
  if (num_seqs < 0 || max_q_len < 0 || q_heads <= 0 || kv_heads <= 0 || max_context_len < 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || block_size <= 0 || head_dim <= 0)
    return PKV_ERR_SHAPE;
  if (q_heads % kv_heads) return PKV_ERR_SHAPE;
  if ((long long)max_context_len > (long long)max_blocks_per_seq * block_size) return PKV_ERR_SHAPE;
  if (max_q_len > max_context_len) return PKV_ERR_SHAPE;
  const int group = q_heads / kv_heads;
  if (dtype != PKV_DTYPE_BF16) return PKV_ERR_UNSUPPORTED;  // the matrix-core path takes bf16
  if (!(group == 1 || group == 2 || group == 4 || group == 8 || group == 16)) return PKV_ERR_UNSUPPORTED;
  if (!(head_dim == 64 || head_dim == 128)) return PKV_ERR_UNSUPPORTED;
  if (!(block_size == 16 || block_size == 32)) return PKV_ERR_UNSUPPORTED;
  const int tile = pkv::kWavesPerWG * pkv::kPrefillColumns / group;  // tokens per workgroup
  const long long n_qt = ((long long)max_q_len + tile - 1) / tile;
  const long long units = (long long)num_seqs * kv_heads * n_qt;
  if (units > 0x7fffffffLL - 4) return PKV_ERR_UNSUPPORTED;
  if (units == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !q_start) return PKV_ERR_NULL;
  pkv::PrefillParams p;
  p.out = out;
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.tables = block_tables;
  p.lens = context_lens;
  p.q_start = q_start;
  p.S = num_seqs;
  p.Hq = q_heads;
  p.Hkv = kv_heads;
  p.NB = num_blocks;
  p.MB = max_blocks_per_seq;
  p.max_len = max_context_len;
  p.n_qt = (int)n_qt;
  p.n_units = (int)units;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)
  const hipError_t e = pkv::launch_prefill(p, head_dim, block_size, group, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int paged_kv_swap_out(const void* k_cache, const void* v_cache, const int32_t* blocks, int32_t n_blocks, void* host_k,
                      void* host_v, void* staging, size_t staging_bytes, int32_t num_blocks, int32_t block_size,
                      int32_t kv_heads, int32_t head_dim, int32_t dtype, void* stream);
int paged_kv_swap_in(void* k_cache, void* v_cache, const int32_t* blocks, int32_t n_blocks, const void* host_k,
                     const void* host_v, void* staging, size_t staging_bytes, int32_t num_blocks, int32_t block_size,
                     int32_t kv_heads, int32_t head_dim, int32_t dtype, void* stream);

size_t paged_kv_swap_staging_bytes(int32_t n_blocks, int32_t block_size, int32_t kv_heads, int32_t head_dim,
                                   int32_t dtype);

static size_t staging_need(int32_t n_blocks, size_t bb) { return round_up((size_t)n_blocks * 4, 256) + 2 * (size_t)n_blocks * bb; }

static int swap_blocks(bool out, char* dev_k, char* dev_v, const int32_t* blocks, int32_t n_blocks, char* host_k,
                char* host_v, void* staging, size_t staging_bytes, int32_t num_blocks, int32_t block_size,
                int32_t kv_heads, int32_t head_dim, int32_t dtype, void* stream) {
  if (!valid_dtype(dtype)) return PKV_ERR_DTYPE;
  if (n_blocks < 0 || num_blocks <= 0 || block_size <= 0 || kv_heads <= 0 || head_dim <= 0) return PKV_ERR_SHAPE;
  if (n_blocks == 0) return PKV_OK;
  if (!dev_k || !dev_v || !blocks || !host_k || !host_v) return PKV_ERR_NULL;
  for (int32_t i = 0; i < n_blocks; ++i)
    if (blocks[i] < 0 || blocks[i] >= num_blocks) return PKV_ERR_SHAPE;
  const size_t bb = (size_t)block_size * kv_heads * head_dim * elt_bytes(dtype);
  if (bb % 16 || bb > 0x7fffffffULL) return PKV_ERR_SHAPE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (staging && staging_bytes >= staging_need(n_blocks, bb)) {
    // ids into the staging area, blocks gathered into (or scattered from)
    // contiguous K and V runs, one DMA per cache across PCIe
    char* st = static_cast<char*>(staging);
    int32_t* ids = reinterpret_cast<int32_t*>(st);
    char* st_k = st + round_up((size_t)n_blocks * 4, 256);
    char* st_v = st_k + (size_t)n_blocks * bb;
    const size_t bytes = (size_t)n_blocks * bb;
    hipError_t e = hipMemcpyAsync(ids, blocks, (size_t)n_blocks * 4, hipMemcpyHostToDevice, s);
    if (out) {
      if (e == hipSuccess) e = pkv::launch_stage_blocks(dev_k, dev_v, st_k, st_v, ids, n_blocks, num_blocks, (long long)bb, true, s);
      if (e == hipSuccess) e = hipMemcpyAsync(host_k, st_k, bytes, hipMemcpyDeviceToHost, s);
      if (e == hipSuccess) e = hipMemcpyAsync(host_v, st_v, bytes, hipMemcpyDeviceToHost, s);
    } else {
      if (e == hipSuccess) e = hipMemcpyAsync(st_k, host_k, bytes, hipMemcpyHostToDevice, s);
      if (e == hipSuccess) e = hipMemcpyAsync(st_v, host_v, bytes, hipMemcpyHostToDevice, s);
      if (e == hipSuccess) e = pkv::launch_stage_blocks(dev_k, dev_v, st_k, st_v, ids, n_blocks, num_blocks, (long long)bb, false, s);
    }
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
  }
  for (int32_t i = 0; i < n_blocks;) {
    int32_t j = i + 1;  // the run blocks[i] .. blocks[j-1] is consecutive
    while (j < n_blocks && blocks[j] == blocks[j - 1] + 1) ++j;
    const size_t bytes = (size_t)(j - i) * bb;
    char* d_k = dev_k + (size_t)blocks[i] * bb;
    char* d_v = dev_v + (size_t)blocks[i] * bb;
    char* h_k = host_k + (size_t)i * bb;
    char* h_v = host_v + (size_t)i * bb;
    hipError_t e;
    if (out) {
      e = hipMemcpyAsync(h_k, d_k, bytes, hipMemcpyDeviceToHost, s);
      if (e == hipSuccess) e = hipMemcpyAsync(h_v, d_v, bytes, hipMemcpyDeviceToHost, s);
    } else {
      e = hipMemcpyAsync(d_k, h_k, bytes, hipMemcpyHostToDevice, s);
      if (e == hipSuccess) e = hipMemcpyAsync(d_v, h_v, bytes, hipMemcpyHostToDevice, s);
    }
    if (e != hipSuccess) return PKV_ERR_HIP;
    i = j;
  }
  return PKV_OK;
}

int paged_kv_swap_out(const void* k_cache, const void* v_cache, const int32_t* blocks, int32_t n_blocks, void* host_k,
                      void* host_v, void* staging, size_t staging_bytes, int32_t num_blocks, int32_t block_size,
                      int32_t kv_heads, int32_t head_dim, int32_t dtype, void* stream) {
  return swap_blocks(true, static_cast<char*>(const_cast<void*>(k_cache)),
                     static_cast<char*>(const_cast<void*>(v_cache)), blocks, n_blocks, static_cast<char*>(host_k),
                     static_cast<char*>(host_v), staging, staging_bytes, num_blocks, block_size, kv_heads, head_dim,
                     dtype, stream);
}

int paged_kv_swap_in(void* k_cache, void* v_cache, const int32_t* blocks, int32_t n_blocks, const void* host_k,
                     const void* host_v, void* staging, size_t staging_bytes, int32_t num_blocks, int32_t block_size,
                     int32_t kv_heads, int32_t head_dim, int32_t dtype, void* stream) {
  return swap_blocks(false, static_cast<char*>(k_cache), static_cast<char*>(v_cache), blocks, n_blocks,
                     static_cast<char*>(const_cast<void*>(host_k)), static_cast<char*>(const_cast<void*>(host_v)),
                     staging, staging_bytes, num_blocks, block_size, kv_heads, head_dim, dtype, stream);
}

size_t paged_kv_swap_staging_bytes(int32_t n_blocks, int32_t block_size, int32_t kv_heads, int32_t head_dim,
                                   int32_t dtype) {
  if (!valid_dtype(dtype) || n_blocks < 0 || block_size <= 0 || kv_heads <= 0 || head_dim <= 0) return 0;
  return staging_need(n_blocks, (size_t)block_size * kv_heads * head_dim * elt_bytes(dtype));
}

int paged_attn_decode_plan(int32_t num_seqs, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t max_context_len, int32_t dtype, int32_t partition_size,
                           int32_t* resolved_partition_size, int32_t* num_partitions) {
  Plan plan;
  const int st = plan_sizes(num_seqs, q_heads, kv_heads, head_dim, block_size, max_context_len, dtype,
                            partition_size, &plan);
  if (st != PKV_OK) return st;
  if (resolved_partition_size) *resolved_partition_size = plan.P;
  if (num_partitions) *num_partitions = plan.schedule == pkv::kBalanced ? plan.n_units : plan.NP;
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
  const hipError_t e = pkv::launch_decode_reduce(p, head_dim, q_heads / kv_heads, static_cast<hipStream_t>(stream));
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
  if (e == hipSuccess) e = pkv::launch_decode_reduce(p, head_dim, q_heads / kv_heads, s);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

// The rows of a fused append whose stage-1 kernel does not write them:
// position L of every sequence whose L + 1 fits the bound, as the kernels
// would (the partitioned kernel writes its rows itself).
static hipError_t append_rows_apart(const pkv::DecodeParams& p, hipStream_t s) {
  if (!p.append || p.schedule != pkv::kBalanced || p.fuse_rows) return hipSuccess;
  // L is written when 0 <= L < max_len (L + 1 attended); max_len <= MB * B
  return pkv::launch_append_at(const_cast<void*>(p.k), const_cast<void*>(p.v), p.k_new, p.v_new, p.tables, p.lens,
                               nullptr, p.S, p.MB, p.block_size, p.NB, p.row_b, (long long)p.max_len, s);
}

// The fused append: the same plan and checks as the decode of L + 1 tokens,
// plus the new rows.
static int prepare_decode_append(float* out, const void* q, void* k_cache, void* v_cache, const void* k_new,
                                 const void* v_new, const int32_t* block_tables, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                                 int32_t max_context_len, float scale, int32_t dtype, int32_t partition_size,
                                 void* workspace, size_t workspace_bytes, pkv::DecodeParams* p) {
  const int st = prepare_decode(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, q_heads, kv_heads,
                                head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, dtype,
                                partition_size, workspace, workspace_bytes, p);
  if (st != PKV_OK) return st;
  if (num_seqs > 0 && (!k_new || !v_new)) return PKV_ERR_NULL;
  if ((long long)num_blocks * block_size > 0x7fffffffLL) return PKV_ERR_SHAPE;  // slots are int32, as for append_at
  p->k_new = k_new;
  p->v_new = v_new;
  p->append = 1;
  p->row_b = head_dim * (dtype == PKV_DTYPE_BF16 ? 2 : 4) * kv_heads;
  const int group = q_heads / kv_heads;
  // The balanced kernels write the rows themselves: one launch fewer, which
  // measured 2.4 us (GQA) and 2.4 us (long context) faster per flushed step
  // on the matrix-core kernels than a launch of their own before stage 1.
  p->fuse_rows = p->schedule == pkv::kBalanced;
  if (p->fuse_rows) {
    // The balanced kernel keeps each segment's new row in LDS until the
    // segment's last chunk substitutes it, and writes the rows out with the
    // finished pieces: up to a third of the wave's LDS, the rest for pieces.
    const long long wave_lds = balanced_wave_lds(num_seqs, head_dim, group, dtype);
    const int entry = pkv::append_row_entry_bytes(dtype, head_dim);
    long long rows = wave_lds / 3 / entry;
    if (rows > pkv::kAppendRowsMax) rows = pkv::kAppendRowsMax;
    long long queue = wave_lds - rows * entry;
    if (queue > pkv::kQueueMaxBytes) queue = pkv::kQueueMaxBytes;
    queue &= ~15LL;
    if (queue < pkv::piece_record_bytes(group, head_dim)) {  // no room: rows go straight to the pool
      rows = 0;
      queue = p->queue_bytes;
    }
    p->row_bytes = (int)(rows * entry);
    p->queue_bytes = (int)queue;
  }
  return PKV_OK;
}

int paged_attn_decode_append(float* out, const void* q, void* k_cache, void* v_cache, const void* k_new,
                             const void* v_new, const int32_t* block_tables, const int32_t* context_lens,
                             int32_t num_seqs, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                             int32_t max_context_len, float scale, int32_t dtype, int32_t partition_size,
                             void* workspace, size_t workspace_bytes, void* stream) {
  pkv::DecodeParams p;
  const int st = prepare_decode_append(out, q, k_cache, v_cache, k_new, v_new, block_tables, context_lens, num_seqs,
                                       q_heads, kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                       max_context_len, scale, dtype, partition_size, workspace, workspace_bytes, &p);
  if (st != PKV_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = append_rows_apart(p, s);
  if (e == hipSuccess) e = pkv::launch_decode_partitions(p, dtype, head_dim, block_size, q_heads / kv_heads, s);
  if (e == hipSuccess) e = pkv::launch_decode_reduce(p, head_dim, q_heads / kv_heads, s);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

// ------------------------------------------------------- decode, no allocation
//
// paged_attn_decode_noalloc keeps its partial records and prefix sums in this
// file-scope device array instead of a caller's workspace.  Each GPU holds its
// own copy for the life of the process.  In host code `scratch` names a host
// stand-in, not device memory: the kernels get the device address that
// hipGetSymbolAddress returns, looked up once per device and kept here.
static __device__ __align__(256) char scratch[PKV_NOALLOC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of this device's scratch array: the current device, which
// must be the stream's device.
static int scratch_for(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return PKV_ERR_HIP;
  }
  if (dev >= kMaxDevices) return PKV_ERR_UNSUPPORTED;
  if (stream != nullptr) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) {
      (void)hipGetLastError();
      return PKV_ERR_HIP;
    }
    if (sdev != dev) return PKV_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return PKV_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

int paged_attn_decode_noalloc(float* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                              int32_t q_heads, int32_t kv_heads, int32_t head_dim, int32_t block_size,
                              int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                              int32_t dtype, int32_t partition_size, void* stream) {
  // Every host check of paged_attn_decode first, with the whole array as the
  // workspace (too small a plan fails with PKV_ERR_WORKSPACE before anything
  // touches the device); then the array's device address.
  pkv::DecodeParams p;
  const char* fake = reinterpret_cast<const char*>(256);  // stands in for the address until it is known
  int st = prepare_decode(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, q_heads, kv_heads,
                          head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, dtype,
                          partition_size, const_cast<char*>(fake), PKV_NOALLOC_SCRATCH_BYTES, &p);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return PKV_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  st = scratch_for(s, &ws);
  if (st != PKV_OK) return st;
  st = prepare_decode(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, q_heads, kv_heads, head_dim,
                      block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, dtype, partition_size, ws,
                      PKV_NOALLOC_SCRATCH_BYTES, &p);
  if (st != PKV_OK) return st;
  hipError_t e = pkv::launch_decode_partitions(p, dtype, head_dim, block_size, q_heads / kv_heads, s);
  if (e == hipSuccess) e = pkv::launch_decode_reduce(p, head_dim, q_heads / kv_heads, s);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int paged_attn_decode_append_partitions(float* out, const void* q, void* k_cache, void* v_cache, const void* k_new,
                                        const void* v_new, const int32_t* block_tables, const int32_t* context_lens,
                                        int32_t num_seqs, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                                        int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                                        int32_t max_context_len, float scale, int32_t dtype,
                                        int32_t partition_size, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  pkv::DecodeParams p;
  const int st = prepare_decode_append(out, q, k_cache, v_cache, k_new, v_new, block_tables, context_lens, num_seqs,
                                       q_heads, kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                       max_context_len, scale, dtype, partition_size, workspace, workspace_bytes, &p);
  if (st != PKV_OK) return st;
  hipError_t e = append_rows_apart(p, static_cast<hipStream_t>(stream));
  if (e == hipSuccess)
    e = pkv::launch_decode_partitions(p, dtype, head_dim, block_size, q_heads / kv_heads,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int paged_attn_decode_append_reduce(float* out, const void* q, void* k_cache, void* v_cache, const void* k_new,
                                    const void* v_new, const int32_t* block_tables, const int32_t* context_lens,
                                    int32_t num_seqs, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                                    int32_t max_context_len, float scale, int32_t dtype, int32_t partition_size,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  pkv::DecodeParams p;
  const int st = prepare_decode_append(out, q, k_cache, v_cache, k_new, v_new, block_tables, context_lens, num_seqs,
                                       q_heads, kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                       max_context_len, scale, dtype, partition_size, workspace, workspace_bytes, &p);
  if (st != PKV_OK) return st;
  const hipError_t e = pkv::launch_decode_reduce(p, head_dim, q_heads / kv_heads, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int paged_attn_decode_shared(float* out, const void* q, void* k_cache, void* v_cache, const void* k_new,
                             const void* v_new, const int32_t* block_tables, const int32_t* context_lens,
                             int32_t num_seqs, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                             int32_t max_context_len, float scale, int32_t dtype, int32_t stages, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (stages & ~PKV_STAGES_ALL) return PKV_ERR_UNSUPPORTED;
  const bool fused = k_new != nullptr || v_new != nullptr;
  if (fused && (k_new == nullptr || v_new == nullptr)) return PKV_ERR_NULL;
  Plan plan;
  int st = plan_shared(num_seqs, q_heads, kv_heads, head_dim, block_size, max_context_len, dtype, &plan);
  if (st != PKV_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int group = q_heads / kv_heads;
  if (!plan.shared) {
    // fp32 caches or a batch too long for the LDS tables: the plain decode
    // (no reads shared); the attend stage holds stage 1, the merge stage 2
    pkv::DecodeParams p;
    st = fused ? prepare_decode_append(out, q, k_cache, v_cache, k_new, v_new, block_tables, context_lens, num_seqs,
                                       q_heads, kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                       max_context_len, scale, dtype, 0, workspace, workspace_bytes, &p)
               : prepare_decode(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, q_heads, kv_heads,
                                head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, dtype, 0,
                                workspace, workspace_bytes, &p);
    if (st != PKV_OK) return st;
    hipError_t e = hipSuccess;
    if (stages & PKV_STAGE_ATTEND) {
      e = append_rows_apart(p, s);
      if (e == hipSuccess) e = pkv::launch_decode_partitions(p, dtype, head_dim, block_size, group, s);
    }
    if (e == hipSuccess && (stages & PKV_STAGE_MERGE)) e = pkv::launch_decode_reduce(p, head_dim, group, s);
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
  }
  pkv::DecodeParams p;
  st = fill_decode(plan, out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, q_heads, kv_heads, head_dim,
                   block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, workspace, workspace_bytes,
                   &p);
  if (st != PKV_OK) return st;
  if (fused) {
    if ((long long)num_blocks * block_size > 0x7fffffffLL) return PKV_ERR_SHAPE;  // as for paged_kv_append_at
    p.k_new = k_new;
    p.v_new = v_new;
    p.append = 1;
    p.row_b = head_dim * 2 * kv_heads;
  }
  hipError_t e = hipSuccess;
  if (stages & PKV_STAGE_PREPARE) e = pkv::launch_shared_prepare(p, head_dim, s);
  if (e == hipSuccess && (stages & PKV_STAGE_ATTEND)) e = pkv::launch_shared_stage1(p, head_dim, block_size, group, s);
  if (e == hipSuccess && (stages & PKV_STAGE_MERGE)) e = pkv::launch_shared_merge(p, head_dim, group, s);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

size_t paged_attn_decode_shared_workspace_size(int32_t num_seqs, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                                               int32_t block_size, int32_t max_context_len, int32_t dtype) {
  Plan plan;
  if (plan_shared(num_seqs, q_heads, kv_heads, head_dim, block_size, max_context_len, dtype, &plan) != PKV_OK)
    return 0;
  return plan.total();
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
    case PKV_ERR_OUT_OF_BLOCKS: return "out of blocks";
    case PKV_ERR_BAD_SEQUENCE: return "not a live sequence";
    default: return "unknown status";
  }
}

}  // extern "C"
