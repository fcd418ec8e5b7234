/*
 * pagedkv.h — paged KV-cache decode attention and KV append for AMD Instinct
 * MI355X (gfx950).  C ABI: plain pointers and sizes, no framework types.
 *
 * The operations follow two web pages:
 *   [A] "PagedAttention Paper Breakdown: Virtual Memory Allocation for LLM KV
 *       Cache Serving", section 2, "Address Translation Formula": token i of a
 *       sequence lives in logical block b = floor(i / B) at offset o = i mod B,
 *       and its physical location is T[b] * B + o, T being the sequence's
 *       block table.
 *   [B] "PagedAttention and vLLM Architecture: Virtual Memory for LLM Serving":
 *       section 1 (a physical page holds the Key and Value of B tokens; the
 *       block table is kept by the serving engine), "Why Internal Fragmentation
 *       is Bounded" (a block is added only when a new token overflows the last
 *       one) and section 2, "PagedAttention Attention CUDA Kernel Mechanics"
 *       (the decode kernel takes the query and the block table, walks the
 *       physical blocks, dots the query with every key, and finishes with an
 *       online softmax fused with the product by the Value blocks).
 *
 * Common conventions
 *   - Every pointer argument is a DEVICE pointer owned by the caller, except
 *     where stated.  Buffers are dense, row-major, 16-byte aligned.
 *   - Cache layout: k_cache and v_cache are [num_blocks, B, kv_heads, head_dim]
 *     of `dtype`.  Slot s = T[b] * B + o names row s of the pool viewed as
 *     [num_blocks * B, kv_heads, head_dim]; K and V share tables and slots.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  The library never allocates, frees or synchronises, and keeps
 *     no state between calls: it is safe to call from several host threads.
 *   - Arguments are checked on the host before anything is launched; a
 *     negative status means nothing was enqueued.  PKV_ERR_HIP means a launch
 *     failed (hipGetLastError after the launch).
 *   - Device-side contract (not checked, for cost, except where stated):
 *     table entries read by a call lie in [0, num_blocks); append slots are
 *     distinct; no slot is written while its block is shared by several
 *     sequences (copy-on-write must already have given the writer a private
 *     block).
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define PKV_API __attribute__((visibility("default")))
#else
#define PKV_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_NULL = -1,        /* a required pointer is NULL                        */
  PKV_ERR_SHAPE = -2,       /* a size is negative, zero where it must not be, or
                               inconsistent with another                          */
  PKV_ERR_DTYPE = -3,       /* dtype is not PKV_DTYPE_F32 or PKV_DTYPE_BF16       */
  PKV_ERR_UNSUPPORTED = -4, /* valid but outside the compiled set (head_dim,
                               block size, group size, partition size)            */
  PKV_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required         */
  PKV_ERR_HIP = -6,         /* a kernel launch failed                             */
  PKV_ERR_OUT_OF_BLOCKS = -7, /* block manager: the free pool (or a table's
                               max_blocks_per_seq) cannot hold the request      */
  PKV_ERR_BAD_SEQUENCE = -8 /* block manager: not a live sequence id              */
};

enum pkv_dtype {
  PKV_DTYPE_F32 = 0,  /* IEEE binary32                                          */
  PKV_DTYPE_BF16 = 1  /* bfloat16: the upper 16 bits of a binary32             */
};

/*
 * paged_kv_slot_mapping — [A] applied to the position each sequence writes
 * next ([B], "Why Internal Fragmentation is Bounded": a sequence holding L
 * tokens writes its next token at logical position L, in the block the engine
 * appended to its table when L crossed a block boundary).
 *
 *   slot_mapping [num_seqs]  int32, written: T[s][p / B] * B + p % B for
 *                            p = positions[s]; -1 when p < 0,
 *                            p >= max_blocks_per_seq * B, or the entry
 *                            T[s][p / B] lies outside [0, num_blocks).
 *   block_tables [num_seqs, max_blocks_per_seq] int32, read at column p / B only.
 *   positions    [num_seqs]  int32.
 * Requires num_blocks * block_size <= INT32_MAX (slots are int32).
 * Errors: PKV_ERR_NULL, PKV_ERR_SHAPE; num_seqs == 0 enqueues nothing.
 */
PKV_API int paged_kv_slot_mapping(int32_t* slot_mapping, const int32_t* block_tables, const int32_t* positions,
                          int32_t num_seqs, int32_t max_blocks_per_seq, int32_t block_size,
                          int32_t num_blocks, void* stream);

/*
 * paged_kv_append — the slot write of [B] ("Why Internal Fragmentation is
 * Bounded"; section 1: K and V of a token share its slot).  For every token t
 * with 0 <= slot_mapping[t] < num_blocks * block_size, copies the row
 * k_new[t] ([kv_heads, head_dim]) to k_cache slot slot_mapping[t] and v_new[t]
 * to v_cache at the same slot, bit for bit.  Tokens with any other slot are
 * skipped (so a stray slot can never write outside the pool).
 *
 *   k_cache, v_cache [num_blocks, block_size, kv_heads, head_dim] dtype, in/out.
 *   k_new, v_new     [num_tokens, kv_heads, head_dim] dtype, read.
 *   slot_mapping     [num_tokens] int32, read.
 * kv_heads * head_dim * element size must be a multiple of 16 bytes.
 * Errors: PKV_ERR_NULL, PKV_ERR_SHAPE, PKV_ERR_DTYPE; num_tokens == 0 enqueues
 * nothing.
 */
PKV_API int paged_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                    const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                    int32_t block_size, int32_t kv_heads, int32_t head_dim, int32_t dtype,
                    void* stream);

/*
 * paged_kv_append_at — paged_kv_slot_mapping and paged_kv_append in one launch
 * (the same two passages).  For every sequence s, with p = positions[s]: when
 * 0 <= p < max_blocks_per_seq * block_size and the table entry
 * T[s][p / block_size] lies in [0, num_blocks), copies k_new[s] and v_new[s]
 * bit for bit to slot T[s][p / block_size] * block_size + p % block_size of
 * k_cache and v_cache; otherwise writes nothing.  When slot_mapping is not
 * NULL it receives that slot, or -1.
 *
 *   k_cache, v_cache [num_blocks, block_size, kv_heads, head_dim] dtype, in/out.
 *   k_new, v_new     [num_seqs, kv_heads, head_dim] dtype, read.
 *   block_tables     [num_seqs, max_blocks_per_seq] int32, read at column p / B only.
 *   positions        [num_seqs] int32.
 *   slot_mapping     [num_seqs] int32, written, or NULL.
 * Requires num_blocks * block_size <= INT32_MAX and kv_heads * head_dim *
 * element size a multiple of 16 bytes.  Errors: PKV_ERR_NULL, PKV_ERR_SHAPE,
 * PKV_ERR_DTYPE; num_seqs == 0 enqueues nothing.
 */
PKV_API int paged_kv_append_at(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                               const int32_t* block_tables, const int32_t* positions, int32_t* slot_mapping,
                               int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
                               int32_t block_size, int32_t kv_heads, int32_t head_dim, int32_t dtype, void* stream);

/*
 * paged_attn_decode — one decode step of paged attention, [B] section 2 with
 * the table walk of [A].  For every sequence s (L = context_lens[s]) and query
 * head h (kv head g = h / (q_heads / kv_heads)):
 *
 *   x_i = scale * <q[s,h,:], K_i[g,:]>   for logical positions i = 0 .. L-1,
 *   out[s,h,:] = sum_i softmax(x)_i * V_i[g,:]
 *
 * where K_i / V_i are read from slot T[s][i / B] * B + i % B.  Scores, the
 * online softmax and the V accumulation are fused in one pass over each
 * sequence's physical blocks, all in fp32.  Two schedules split the work:
 *   - balanced (partition_size 0, some L above 512 tokens, num_seqs <= 2048):
 *     the 16-token chunks of all (sequence, kv head) pairs, laid end to end,
 *     are cut into one share of equal cost per resident worker (a pair costs
 *     its chunks plus a small charge for starting it);
 *   - partitioned (otherwise): partitions of `partition_size` tokens, one
 *     wave each.
 * Pieces of a (sequence, kv head) pair computed apart are merged by a second
 * kernel (log-sum-exp rescaling).  Which tokens each piece holds depends on
 * the lengths and the plan only, so repeated calls are bitwise deterministic;
 * the result does not depend on which physical blocks hold the tokens
 * (reductions follow logical positions only), so permuting the pool, or
 * sharing blocks between sequences, gives bitwise identical outputs.
 *
 *   out          [num_seqs, q_heads, head_dim] fp32, written (every element).
 *   q            [num_seqs, q_heads, head_dim] dtype.
 *   k_cache, v_cache [num_blocks, block_size, kv_heads, head_dim] dtype.
 *   block_tables [num_seqs, max_blocks_per_seq] int32; only entries
 *                b < ceil(L / B) are read.
 *   context_lens [num_seqs] int32.  L = 0 gives zeros.  A sequence with
 *                L < 0 or L > max_context_len gets NaN rows (it cannot be
 *                covered by the launch); a table entry outside
 *                [0, num_blocks) is not dereferenced and also gives NaN rows.
 *   max_context_len  host-side upper bound of context_lens; sizes the grid.
 *                    Must be <= max_blocks_per_seq * block_size.
 *   scale        multiplies the dot products (e.g. 1/sqrt(head_dim)).
 *   partition_size   tokens per partition: 0 = choose automatically, else a
 *                    multiple of 16 in [16, 8192].
 *   workspace    device scratch of at least
 *                paged_attn_decode_workspace_size(...) bytes, same arguments;
 *                may be NULL when that size is 0.  Overwritten.
 *
 * Supported: dtype F32 or BF16 (q, K, V share it); head_dim 64 or 128;
 * block_size 16 or 32; q_heads % kv_heads == 0 with group size 1, 2, 4, 8 or 16.
 * Errors: PKV_ERR_NULL, PKV_ERR_SHAPE, PKV_ERR_DTYPE, PKV_ERR_UNSUPPORTED,
 * PKV_ERR_WORKSPACE, PKV_ERR_HIP.  num_seqs == 0 enqueues nothing.
 */
PKV_API int paged_attn_decode(float* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                      int32_t q_heads, int32_t kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                      float scale, int32_t dtype, int32_t partition_size, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * The two stages of paged_attn_decode, for callers that time or schedule them
 * apart.  Same arguments and checks.  Stage 1 runs the fused score / online
 * softmax / V pass; when the resolved plan is partitioned with a single
 * partition it writes `out` directly and stage 2 enqueues nothing.
 * Otherwise stage 1 writes the rows it finishes alone to `out` and partial
 * (max, sum, accumulator) records of split pairs to the workspace, and
 * stage 2 merges those into `out` (and writes the rows of invalid and empty
 * sequences).  Stage 2 must follow stage 1 on the same stream with the same
 * arguments and lengths.
 */
PKV_API int paged_attn_decode_partitions(float* out, const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                                 int32_t max_context_len, float scale, int32_t dtype,
                                 int32_t partition_size, void* workspace, size_t workspace_bytes,
                                 void* stream);
PKV_API int paged_attn_decode_reduce(float* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                             int32_t q_heads, int32_t kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                             float scale, int32_t dtype, int32_t partition_size, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * paged_attn_decode_append — a decode step that appends and attends in one
 * pass: the slot write of each sequence's new token ("PagedAttention and vLLM
 * Architecture", Why Internal Fragmentation is Bounded: a sequence holding L
 * tokens puts its next one at position L, into the block the engine added to
 * its table when L reached a block boundary; the slot is T[L / B] * B + L % B,
 * "PagedAttention Paper Breakdown", section 2) fused with paged_attn_decode
 * over the L + 1 tokens that then make up the context.  For every sequence s
 * with L = context_lens[s] (the length before the append):
 *
 *   K_L, V_L := k_new[s], v_new[s]   (bit copy into slot T[s][L / B] * B + L % B)
 *   out[s,h,:] = paged_attn_decode over positions 0 .. L
 *
 * The result equals paged_kv_append_at(positions = context_lens) followed by
 * paged_attn_decode with context_lens + 1, bitwise.  Stage 1 writes the new
 * rows itself (no launch of their own).
 *
 *   k_cache, v_cache [num_blocks, block_size, kv_heads, head_dim] dtype, in/out:
 *                the new rows are written, nothing else.
 *   k_new, v_new [num_seqs, kv_heads, head_dim] dtype, read.
 *   context_lens [num_seqs] int32, lengths before the append.  A sequence with
 *                L < 0 or L + 1 > max_context_len gets NaN rows and no write.
 *                A table entry outside [0, num_blocks) among its first
 *                ceil((L + 1) / B) gives NaN rows; if it is the entry of
 *                block L / B, nothing is written either.
 *   max_context_len  host-side bound of the attended length L + 1; sizes the
 *                grid and the workspace (paged_attn_decode_workspace_size with
 *                the same value).  Must be <= max_blocks_per_seq * block_size.
 *   Everything else as paged_attn_decode.  The new slots must be distinct
 *   and must not lie in a block another sequence shares (copy-on-write first).
 *
 * Errors: those of paged_attn_decode; PKV_ERR_NULL also for a missing k_new
 * or v_new; PKV_ERR_SHAPE also when num_blocks * block_size exceeds
 * INT32_MAX (as for paged_kv_append_at).  The _partitions / _reduce pair splits the call into its two
 * stages like paged_attn_decode_partitions / _reduce (the append happens in
 * the first).
 */
PKV_API int paged_attn_decode_append(float* out, const void* q, void* k_cache, void* v_cache,
                                     const void* k_new, const void* v_new, const int32_t* block_tables,
                                     const int32_t* context_lens, int32_t num_seqs, int32_t q_heads,
                                     int32_t kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                     int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                                     int32_t dtype, int32_t partition_size, void* workspace,
                                     size_t workspace_bytes, void* stream);
PKV_API int paged_attn_decode_append_partitions(float* out, const void* q, void* k_cache, void* v_cache,
                                                const void* k_new, const void* v_new,
                                                const int32_t* block_tables, const int32_t* context_lens,
                                                int32_t num_seqs, int32_t q_heads, int32_t kv_heads,
                                                int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                                int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                                                int32_t dtype, int32_t partition_size, void* workspace,
                                                size_t workspace_bytes, void* stream);
PKV_API int paged_attn_decode_append_reduce(float* out, const void* q, void* k_cache, void* v_cache,
                                            const void* k_new, const void* v_new, const int32_t* block_tables,
                                            const int32_t* context_lens, int32_t num_seqs, int32_t q_heads,
                                            int32_t kv_heads, int32_t head_dim, int32_t block_size,
                                            int32_t num_blocks, int32_t max_blocks_per_seq,
                                            int32_t max_context_len, float scale, int32_t dtype,
                                            int32_t partition_size, void* workspace, size_t workspace_bytes,
                                            void* stream);

/*
 * paged_attn_decode_shared — paged_attn_decode (k_new = v_new = NULL) or
 * paged_attn_decode_append (both given) that reads the blocks neighbouring
 * sequences share once for all of them.  Forked sequences (parallel
 * sampling, beam search) alias the physical blocks of their common prompt
 * until a write gives one of them a private copy ("PagedAttention and vLLM
 * Architecture: Virtual Memory for LLM Serving", section 3, Copy-on-Write for
 * Parallel Sampling & Beam Search; "PagedAttention Paper Breakdown", section
 * 3, Dynamic Copy-on-Write).  The outputs are those of the decode defined
 * above for every sequence, row by row; only the reads are shared.
 *
 * Sharing is found on the device, every call, from the tables: sequence s
 * shares with sequence s - 1 the leading tokens whose table entries are
 * equal, in whole 16-token chunks, at most the shorter of their two lengths
 * (before the append).  Runs of neighbours that each share something form
 * groups of at most 16 / G sequences (G = q_heads / kv_heads), which share
 * the shortest of their neighbour-to-neighbour prefixes; a group's prefix is
 * read once and scored against all its members' query rows on the matrix
 * cores, and each member's own tail against its rows only.  Siblings that are
 * not neighbours in the batch are not found (their results are the same,
 * only their shared blocks are read once per sibling).
 *
 *   stages     PKV_STAGES_ALL, or the bits of the stages to enqueue, in order:
 *              PKV_STAGE_PREPARE (the new rows of the fused append; the
 *              shares), PKV_STAGE_ATTEND (stage 1: the score / online softmax
 *              / V pass), PKV_STAGE_MERGE (stage 2: the log-sum-exp merge of
 *              segments split between workers, and the rows of empty and
 *              invalid sequences).  A call that enqueues a later stage alone
 *              must follow one that enqueued the earlier ones, on the same
 *              stream, with the same arguments.
 *   workspace  at least paged_attn_decode_shared_workspace_size(...) bytes.
 *   Everything else as paged_attn_decode (k_new = NULL) or
 *   paged_attn_decode_append (k_new given); max_context_len bounds the
 *   attended length.
 *
 * Supported: as paged_attn_decode.  With bf16 caches and num_seqs <= 2048 the
 * shared-prefix kernels run; otherwise (fp32 caches, longer batches) the call
 * is the plain decode with the automatic partition size, its stage 1 under
 * PKV_STAGE_ATTEND and its stage 2 under PKV_STAGE_MERGE.  Outputs are
 * bitwise reproducible and do not depend on which physical blocks hold the
 * tokens; siblings given equal query rows and equal tokens get bitwise equal
 * rows.  They may differ from paged_attn_decode's in rounding (another
 * order of the same sums), within the stated tolerances.  Errors: those of
 * paged_attn_decode / paged_attn_decode_append; PKV_ERR_UNSUPPORTED for
 * unknown stage bits; PKV_ERR_NULL when only one of k_new, v_new is given.
 */
#define PKV_STAGE_PREPARE 1
#define PKV_STAGE_ATTEND 2
#define PKV_STAGE_MERGE 4
#define PKV_STAGES_ALL 7
PKV_API int paged_attn_decode_shared(float* out, const void* q, void* k_cache, void* v_cache, const void* k_new,
                                     const void* v_new, const int32_t* block_tables, const int32_t* context_lens,
                                     int32_t num_seqs, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                                     int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                                     int32_t max_context_len, float scale, int32_t dtype, int32_t stages,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attn_decode_shared_workspace_size — bytes of workspace
 * paged_attn_decode_shared needs for these arguments (same current device as
 * the call).  Shared-prefix kernels: partial records for W worker waves (two
 * records of 16 rows of head_dim + 2 floats each), num_seqs ints of shares
 * and 4 W ints of split segments, each rounded up to 256 bytes;
 * otherwise paged_attn_decode_workspace_size with partition_size 0.  Host
 * only; 0 for arguments the call would reject.
 */
PKV_API size_t paged_attn_decode_shared_workspace_size(int32_t num_seqs, int32_t q_heads, int32_t kv_heads,
                                                       int32_t head_dim, int32_t block_size,
                                                       int32_t max_context_len, int32_t dtype);

/*
 * paged_attn_decode_noalloc — paged_attn_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results (bitwise: the
 * same plan and kernels) and errors as paged_attn_decode, without the
 * workspace: the partial records and prefix sums live in a fixed device array
 * of PKV_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends.  The call allocates nothing and calls no allocating routine.
 *
 *   - A plan whose workspace (paged_attn_decode_workspace_size with the same
 *     arguments) exceeds PKV_NOALLOC_SCRATCH_BYTES is rejected with
 *     PKV_ERR_WORKSPACE before anything is enqueued.
 *   - The calling thread's current device must be the device of `stream`
 *     (PKV_ERR_UNSUPPORTED otherwise).  The first call on a device looks up
 *     the array's device address (hipGetSymbolAddress) and keeps it.
 *   - Every call on one GPU uses that GPU's one array, and it keeps the last
 *     call's contents (nothing in it needs to start at zero).  Calls that can
 *     overlap on one GPU (several streams, several host threads) race on it
 *     and must be serialised by the caller.
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
PKV_API int paged_attn_decode_noalloc(float* out, const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                      int32_t q_heads, int32_t kv_heads, int32_t head_dim, int32_t block_size,
                                      int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                                      float scale, int32_t dtype, int32_t partition_size, void* stream);

/*
 * paged_attn_decode_plan — the schedule a call with these arguments uses
 * (partition_size 0 = the automatic choice).  The balanced schedule's worker
 * count follows the compute units of the calling thread's current device (a
 * whole MI355X when no device is present), so plan, workspace size and call
 * must be made with the same current device.  Host only; writes
 * *resolved_partition_size and *num_partitions (either may be NULL):
 * (P, partitions per sequence) for the partitioned schedule, (0, worker
 * waves) for the balanced one.  Returns PKV_OK or the error the decode call
 * would return for these sizes.
 */
PKV_API int paged_attn_decode_plan(int32_t num_seqs, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t max_context_len, int32_t dtype,
                           int32_t partition_size, int32_t* resolved_partition_size,
                           int32_t* num_partitions);

/*
 * paged_attn_decode_workspace_size — bytes of workspace paged_attn_decode needs
 * for these arguments.  Partitioned: 0 for a single partition, else
 * num_seqs * q_heads * num_partitions * (head_dim + 2) * 4 bytes (each part
 * rounded up to 256).  Balanced: partial records for W worker waves (two
 * records of group-size rows each, head_dim + 2 floats per row) and
 * 2 * (num_seqs + 1) * 4 bytes of chunk and cost prefix sums.  Host only.  Returns 0 for
 * arguments the decode call would reject.
 */
PKV_API size_t paged_attn_decode_workspace_size(int32_t num_seqs, int32_t q_heads, int32_t kv_heads,
                                        int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                        int32_t dtype, int32_t partition_size);

/*
 * paged_attn_prefill — attention of a chunk of new prompt tokens over the
 * paged cache ("PagedAttention and vLLM Architecture: Virtual Memory for LLM
 * Serving", section 3, item 1: a prompt is processed and its logical blocks
 * are assigned physical blocks; section 2: attention reads K and V through
 * the block table and applies softmax to the scaled dot products; the
 * translation formula of "PagedAttention Paper Breakdown", section 2).
 * Sequence s owns query rows q_start[s] .. q_start[s+1]-1 (n_s of them,
 * n_s <= max_q_len); they are its newest tokens, at positions L-n_s .. L-1
 * (L = context_lens[s], the chunk included: write the chunk's K and V with
 * paged_kv_append first).  The row at position p attends causally to
 * positions 0 .. p:
 *
 *   out[r, h, :] = sum_{i <= p} softmax_i(scale * <q[r, h, :], K_i[g, :]>) V_i[g, :]
 *
 * with g = h / (q_heads / kv_heads), scores, softmax and the V sum in fp32
 * on the matrix cores.  n_s = L gives a whole prompt; n_s < L continues an
 * earlier context (chunked prefill).
 *
 *   out          [total_q, q_heads, head_dim] fp32, rows of every sequence
 *                written (NaN rows when L < n_s or L > max_context_len, or a
 *                table entry outside the pool).
 *   q            [total_q, q_heads, head_dim] bf16.
 *   q_start      [num_seqs + 1] int32, device: nondecreasing, q_start[0] = 0.
 *   block_tables, context_lens, caches: as paged_attn_decode.
 *   max_q_len    host-side upper bound of n_s; sizes the grid.
 * Supported: dtype BF16 (PKV_ERR_UNSUPPORTED for F32); head_dim 64 or 128;
 * block_size 16 or 32; group size 1, 2, 4, 8 or 16.  Errors: PKV_ERR_NULL,
 * PKV_ERR_SHAPE, PKV_ERR_DTYPE, PKV_ERR_UNSUPPORTED, PKV_ERR_HIP.
 */
PKV_API int paged_attn_prefill(float* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens, const int32_t* q_start,
                               int32_t num_seqs, int32_t max_q_len, int32_t q_heads, int32_t kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t num_blocks,
                               int32_t max_blocks_per_seq, int32_t max_context_len, float scale, int32_t dtype,
                               void* stream);

/*
 * paged_kv_copy_blocks — the block copy of copy-on-write ("PagedAttention and
 * vLLM Architecture: Virtual Memory for LLM Serving", section 3: a stream that
 * must write into a shared block first gets a fresh block holding a copy of
 * it).  For every pair i with both ids in [0, num_blocks), copies block
 * src[i] of k_cache to block dst[i] of k_cache, and the same in v_cache, bit
 * for bit (all block_size token rows); pairs with an id outside the pool are
 * skipped.
 *
 *   k_cache, v_cache [num_blocks, block_size, kv_heads, head_dim] dtype, in/out.
 *   src, dst         [n_pairs] int32, device.  The dst blocks must be distinct
 *                    and none may be a src of the same call (the pairs run in
 *                    parallel); the block manager's copies always satisfy this.
 * kv_heads * head_dim * element size must be a multiple of 16 bytes.
 * Errors: PKV_ERR_NULL, PKV_ERR_SHAPE, PKV_ERR_DTYPE; n_pairs == 0 enqueues
 * nothing.
 */
PKV_API int paged_kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst,
                                 int32_t n_pairs, int32_t num_blocks, int32_t block_size, int32_t kv_heads,
                                 int32_t head_dim, int32_t dtype, void* stream);

/*
 * paged_kv_swap_out / paged_kv_swap_in — move whole blocks between the device
 * pool and host memory ("PagedAttention Paper Breakdown", Engineering
 * Limitations: under memory pressure blocks are swapped between CPU and GPU
 * over PCIe).  Entry i of `blocks` (a HOST array of n_blocks ids in
 * [0, num_blocks)) pairs device block blocks[i] with host slot i:
 *   swap_out: host_k[i] <- k_cache[blocks[i]], host_v[i] <- v_cache[blocks[i]];
 *   swap_in:  k_cache[blocks[i]] <- host_k[i], v_cache[blocks[i]] <- host_v[i].
 * host_k, host_v: [n_blocks, block_size, kv_heads, head_dim] of dtype in host
 * memory allocated pinned (hipHostMalloc or an equivalent pinned allocation),
 * owned by the caller.  With a device `staging` area of at least
 * paged_kv_swap_staging_bytes(n_blocks, ...) bytes, the ids are copied into
 * it, a kernel gathers the blocks into contiguous K and V runs there (or
 * scatters them back) and one copy per cache crosses PCIe; with staging NULL
 * (or too small) runs of consecutive ids become one copy each.  Everything
 * is enqueued on `stream` (hipMemcpyAsync), so the caller synchronises before
 * reading host data (swap_out) or reusing host data or staging (swap_in).
 * Errors: PKV_ERR_NULL, PKV_ERR_SHAPE (an id outside the pool), PKV_ERR_DTYPE,
 * PKV_ERR_HIP; n_blocks == 0 enqueues nothing.
 */
PKV_API int paged_kv_swap_out(const void* k_cache, const void* v_cache, const int32_t* blocks, int32_t n_blocks,
                              void* host_k, void* host_v, void* staging, size_t staging_bytes, int32_t num_blocks,
                              int32_t block_size, int32_t kv_heads, int32_t head_dim, int32_t dtype, void* stream);
PKV_API int paged_kv_swap_in(void* k_cache, void* v_cache, const int32_t* blocks, int32_t n_blocks,
                             const void* host_k, const void* host_v, void* staging, size_t staging_bytes,
                             int32_t num_blocks, int32_t block_size, int32_t kv_heads, int32_t head_dim,
                             int32_t dtype, void* stream);
/* Device staging bytes a swap of n_blocks blocks can use (0 for bad sizes). */
PKV_API size_t paged_kv_swap_staging_bytes(int32_t n_blocks, int32_t block_size, int32_t kv_heads,
                                           int32_t head_dim, int32_t dtype);

/*
 * Block manager — host-side bookkeeping of the physical block pool
 * ("PagedAttention and vLLM Architecture: Virtual Memory for LLM Serving",
 * section 1: a pool of fixed-size blocks set up at start and a per-request
 * block table kept by the engine; "Why Internal Fragmentation is Bounded": a
 * block is added only when a token overflows the last one; section 3: forked
 * streams share blocks under a reference count, and a write into a shared
 * block first moves the writer to a private copy and lowers the count).
 *
 * All pointers here are HOST pointers; nothing touches the device.  The free
 * pool hands out the lowest-numbered free block first.  A fork makes one
 * child that shares every block of its parent.  Sequence ids count up from 0
 * and are never reused.  A call that fails returns a negative status and
 * changes nothing (pkv_bm_append_batch: nothing beyond the first *n_done
 * sequences).  One manager must not be used from two threads at once.
 *
 * pkv_bm_create         a pool of num_blocks blocks of block_size tokens, tables of
 *                       at most max_blocks_per_seq blocks; NULL on bad sizes
 *                       (num_blocks * block_size must fit int32) or no memory.
 * pkv_bm_add_sequence   a new empty sequence; its id in *seq.
 * pkv_bm_fork           a new sequence sharing all blocks (and the length) of parent.
 * pkv_bm_free           drops a sequence (also a swapped one); blocks no sequence holds
 *                       return to the pool.
 * pkv_bm_append         reserves the slots of n_tokens new tokens of seq (positions
 *                       L .. L+n_tokens-1) in slots[n_tokens].  When the first of
 *                       them falls into a block shared with another sequence, a
 *                       fresh block replaces it in seq's table and the copy
 *                       (copy_src[0] -> copy_dst[0]) is reported in *n_copies (0 or
 *                       1); run it with paged_kv_copy_blocks before writing the
 *                       tokens.  PKV_ERR_OUT_OF_BLOCKS when the pool or the table
 *                       limit cannot hold them.
 * pkv_bm_append_batch   one new token for each of seqs[0..n_seqs-1], in order
 *                       (the decode step): slots[n_seqs]; copies (at most one per
 *                       sequence) in copy_src/copy_dst[*n_copies]; *n_done sequences
 *                       were served before any failure.
 * pkv_bm_table          seq's block ids into blocks[capacity] (*n_blocks of them) and
 *                       its length into *length (may be NULL).
 * pkv_bm_tables         the rows of seqs as an [n_seqs, max_blocks_per_seq] int32
 *                       table padded with `fill`, and their lengths in lens[n_seqs],
 *                       ready to upload for paged_attn_decode.
 * pkv_bm_swap_out       moves seq to the host side: writes its block ids (table order,
 *                       *n_blocks of them, capacity >= that) for the caller to save
 *                       with paged_kv_swap_out, then drops seq's hold on them (blocks
 *                       no other sequence holds return to the pool).  A swapped
 *                       sequence cannot append, fork or swap out until swapped in.
 * pkv_bm_swap_in        gives a swapped seq fresh private blocks (lowest first) for
 *                       all its tokens and writes their ids for paged_kv_swap_in;
 *                       PKV_ERR_OUT_OF_BLOCKS when the pool cannot hold them.
 * pkv_bm_ref_count      sequences holding a block.
 * pkv_bm_free_blocks    blocks in the free pool (-1 for a NULL manager).
 * pkv_bm_usage          blocks in use, slots of those blocks holding a token (a block
 *                       shared by several sequences counted once), live sequences and
 *                       tokens they hold (shared tokens counted per sequence): the
 *                       internal fragmentation of the pool is 1 - filled / (used * B).
 */
typedef struct pkv_block_manager pkv_block_manager;
PKV_API pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq);
PKV_API void pkv_bm_destroy(pkv_block_manager* m);
PKV_API int pkv_bm_add_sequence(pkv_block_manager* m, int32_t* seq);
PKV_API int pkv_bm_fork(pkv_block_manager* m, int32_t parent, int32_t* child);
PKV_API int pkv_bm_free(pkv_block_manager* m, int32_t seq);
PKV_API int pkv_bm_append(pkv_block_manager* m, int32_t seq, int32_t n_tokens, int32_t* slots, int32_t* copy_src,
                          int32_t* copy_dst, int32_t* n_copies);
PKV_API int pkv_bm_append_batch(pkv_block_manager* m, const int32_t* seqs, int32_t n_seqs, int32_t* slots,
                                int32_t* copy_src, int32_t* copy_dst, int32_t* n_copies, int32_t* n_done);
PKV_API int pkv_bm_table(const pkv_block_manager* m, int32_t seq, int32_t* blocks, int32_t capacity,
                         int32_t* n_blocks, int64_t* length);
PKV_API int pkv_bm_tables(const pkv_block_manager* m, const int32_t* seqs, int32_t n_seqs, int32_t* tables,
                          int32_t max_blocks_per_seq, int32_t fill, int32_t* lens);
PKV_API int pkv_bm_swap_out(pkv_block_manager* m, int32_t seq, int32_t* blocks, int32_t capacity,
                            int32_t* n_blocks);
PKV_API int pkv_bm_swap_in(pkv_block_manager* m, int32_t seq, int32_t* blocks, int32_t capacity,
                           int32_t* n_blocks);
PKV_API int pkv_bm_ref_count(const pkv_block_manager* m, int32_t block, int32_t* ref);
PKV_API int32_t pkv_bm_free_blocks(const pkv_block_manager* m);
PKV_API int pkv_bm_usage(const pkv_block_manager* m, int64_t* used_blocks, int64_t* filled_slots,
                         int64_t* live_seqs, int64_t* held_tokens);

/* paged_status_str — a static, human-readable name for a status code. */
PKV_API const char* paged_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
