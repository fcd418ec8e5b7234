// Host-side block manager of the paged KV cache: the pool of physical
// blocks, per-sequence block tables, reference counts for blocks shared after
// a fork, and the copy-on-write decision.
//
// It follows "PagedAttention and vLLM Architecture: Virtual Memory for LLM
// Serving": section 1 (a pool of fixed-size blocks set up at start, one table
// per request mapping logical to physical blocks, kept by the engine), "Why
// Internal Fragmentation is Bounded" (a block is added only when a token
// overflows the last one) and section 3, "Copy-on-Write (CoW) for Parallel
// Sampling & Beam Search" (forked streams share blocks with a reference
// count; a write into a shared block first moves the writer to a private copy
// and lowers the shared block's count).
//
// Choices the pages leave open: the lowest-numbered free block is handed out
// first; a fork makes one child sharing all of the parent's blocks; a write
// lands in an existing block only when the length is not a multiple of B, so
// full shared blocks are never copied; a failing call changes nothing.
//
// Pure host code: no device memory is touched here.  The copies a call asks
// for are returned to the caller, who runs them on the device
// (paged_kv_copy_blocks) before writing the new tokens.

#include <stdint.h>

#include <new>
#include <vector>

#include "pagedkv.h"

namespace {

// Free-block set with lowest-first lookup: one bit per block (1 = free) and a
// summary bit per 64-block word (1 = the word has a free block).
class FreePool {
 public:
  explicit FreePool(int32_t n) : words_(((size_t)n + 63) / 64, 0), summary_((words_.size() + 63) / 64, 0) {
    for (int32_t b = 0; b < n; ++b) put(b);
  }
  int32_t count() const { return count_; }
  void put(int32_t b) {
    const size_t w = (size_t)b >> 6;
    words_[w] |= 1ull << (b & 63);
    summary_[w >> 6] |= 1ull << (w & 63);
    ++count_;
  }
  // Lowest free block, removed from the set; -1 when empty.
  int32_t take() {
    for (size_t s = 0; s < summary_.size(); ++s) {
      if (!summary_[s]) continue;
      const size_t w = (s << 6) + (size_t)__builtin_ctzll(summary_[s]);
      const int32_t b = (int32_t)((w << 6) + (size_t)__builtin_ctzll(words_[w]));
      words_[w] &= words_[w] - 1;
      if (!words_[w]) summary_[s] &= ~(1ull << (w & 63));
      --count_;
      return b;
    }
    return -1;
  }

 private:
  int32_t count_ = 0;
  std::vector<uint64_t> words_;
  std::vector<uint64_t> summary_;
};

struct Sequence {
  std::vector<int32_t> blocks;  // logical block b -> physical block
  int64_t len = 0;              // tokens held
  bool live = false;            // on the device
  bool swapped = false;         // saved to the host, holding no blocks
};

}  // namespace

struct pkv_block_manager {
  int32_t num_blocks, block_size, max_blocks;
  FreePool pool;
  std::vector<int32_t> ref;     // sequences holding each block
  std::vector<Sequence> seqs;   // by id; ids are never reused

  pkv_block_manager(int32_t nb, int32_t bs, int32_t mb)
      : num_blocks(nb), block_size(bs), max_blocks(mb), pool(nb), ref((size_t)nb, 0) {}

  bool valid(int32_t s) const { return s >= 0 && (size_t)s < seqs.size() && seqs[(size_t)s].live; }

  int32_t take() {
    const int32_t b = pool.take();
    ref[(size_t)b] = 1;
    return b;
  }

  void release(int32_t b) {
    if (--ref[(size_t)b] == 0) pool.put(b);
  }

  // Fresh blocks and copies an append of n tokens to s needs.
  void needs(const Sequence& q, int64_t n, int64_t* fresh, int* cow) const {
    const int64_t B = block_size;
    *cow = (n > 0 && q.len % B != 0 && ref[(size_t)q.blocks.back()] > 1) ? 1 : 0;
    const int64_t want = (q.len + n + B - 1) / B;
    *fresh = want > (int64_t)q.blocks.size() ? want - (int64_t)q.blocks.size() : 0;
  }

  int append(int32_t s, int32_t n, int32_t* slots, int32_t* copy_src, int32_t* copy_dst, int32_t* n_copies) {
    Sequence& q = seqs[(size_t)s];
    int64_t fresh;
    int cow;
    needs(q, n, &fresh, &cow);
    if ((q.len + n + block_size - 1) / block_size > max_blocks) return PKV_ERR_OUT_OF_BLOCKS;
    if (fresh + cow > pool.count()) return PKV_ERR_OUT_OF_BLOCKS;
    *n_copies = 0;
    if (cow) {  // the write would land in a shared block: move to a private copy
      const int32_t old = q.blocks.back();
      const int32_t mine = take();
      copy_src[0] = old;
      copy_dst[0] = mine;
      *n_copies = 1;
      --ref[(size_t)old];  // still held by the other sequences, so never freed here
      q.blocks.back() = mine;
    }
    for (int32_t i = 0; i < n; ++i) {
      const int64_t p = q.len;
      if (p % block_size == 0) q.blocks.push_back(take());  // overflow opens a block
      slots[i] = (int32_t)((int64_t)q.blocks[(size_t)(p / block_size)] * block_size + p % block_size);
      q.len = p + 1;
    }
    return PKV_OK;
  }
};

extern "C" {

pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq) {
  if (num_blocks <= 0 || block_size <= 0 || max_blocks_per_seq <= 0) return nullptr;
  if ((int64_t)num_blocks * block_size > 0x7fffffffLL) return nullptr;  // slots are int32
  return new (std::nothrow) pkv_block_manager(num_blocks, block_size, max_blocks_per_seq);
}

void pkv_bm_destroy(pkv_block_manager* m) { delete m; }

int pkv_bm_add_sequence(pkv_block_manager* m, int32_t* seq) {
  if (!m || !seq) return PKV_ERR_NULL;
  if (m->seqs.size() >= 0x7fffffffu) return PKV_ERR_SHAPE;
  m->seqs.emplace_back();
  m->seqs.back().live = true;
  *seq = (int32_t)(m->seqs.size() - 1);
  return PKV_OK;
}

int pkv_bm_fork(pkv_block_manager* m, int32_t parent, int32_t* child) {
  if (!m || !child) return PKV_ERR_NULL;
  if (!m->valid(parent)) return PKV_ERR_BAD_SEQUENCE;
  if (m->seqs.size() >= 0x7fffffffu) return PKV_ERR_SHAPE;
  Sequence c;
  c.blocks = m->seqs[(size_t)parent].blocks;
  c.len = m->seqs[(size_t)parent].len;
  c.live = true;
  for (int32_t b : c.blocks) ++m->ref[(size_t)b];
  m->seqs.push_back(std::move(c));
  *child = (int32_t)(m->seqs.size() - 1);
  return PKV_OK;
}

int pkv_bm_free(pkv_block_manager* m, int32_t seq) {
  if (!m) return PKV_ERR_NULL;
  if (seq >= 0 && (size_t)seq < m->seqs.size() && m->seqs[(size_t)seq].swapped) {
    m->seqs[(size_t)seq].swapped = false;  // holds no blocks
    m->seqs[(size_t)seq].len = 0;
    return PKV_OK;
  }
  if (!m->valid(seq)) return PKV_ERR_BAD_SEQUENCE;
  Sequence& q = m->seqs[(size_t)seq];
  for (int32_t b : q.blocks) m->release(b);
  q.blocks.clear();
  q.blocks.shrink_to_fit();
  q.len = 0;
  q.live = false;
  return PKV_OK;
}

int pkv_bm_append(pkv_block_manager* m, int32_t seq, int32_t n_tokens, int32_t* slots, int32_t* copy_src,
                  int32_t* copy_dst, int32_t* n_copies) {
  if (!m || !n_copies) return PKV_ERR_NULL;
  if (n_tokens < 0) return PKV_ERR_SHAPE;
  if (n_tokens > 0 && (!slots || !copy_src || !copy_dst)) return PKV_ERR_NULL;
  if (!m->valid(seq)) return PKV_ERR_BAD_SEQUENCE;
  *n_copies = 0;
  if (n_tokens == 0) return PKV_OK;
  return m->append(seq, n_tokens, slots, copy_src, copy_dst, n_copies);
}

int pkv_bm_append_batch(pkv_block_manager* m, const int32_t* seqs, int32_t n_seqs, int32_t* slots,
                        int32_t* copy_src, int32_t* copy_dst, int32_t* n_copies, int32_t* n_done) {
  if (!m || !n_copies || !n_done) return PKV_ERR_NULL;
  if (n_seqs < 0) return PKV_ERR_SHAPE;
  *n_copies = 0;
  *n_done = 0;
  if (n_seqs == 0) return PKV_OK;
  if (!seqs || !slots || !copy_src || !copy_dst) return PKV_ERR_NULL;
  for (int32_t i = 0; i < n_seqs; ++i) {
    if (!m->valid(seqs[i])) return PKV_ERR_BAD_SEQUENCE;
    int32_t c = 0;
    const int st = m->append(seqs[i], 1, slots + i, copy_src + *n_copies, copy_dst + *n_copies, &c);
    if (st != PKV_OK) return st;
    *n_copies += c;
    *n_done = i + 1;
  }
  return PKV_OK;
}

int pkv_bm_table(const pkv_block_manager* m, int32_t seq, int32_t* blocks, int32_t capacity, int32_t* n_blocks,
                 int64_t* length) {
  if (!m || !n_blocks) return PKV_ERR_NULL;
  if (!m->valid(seq)) return PKV_ERR_BAD_SEQUENCE;
  const Sequence& q = m->seqs[(size_t)seq];
  *n_blocks = (int32_t)q.blocks.size();
  if (length) *length = q.len;
  if ((int32_t)q.blocks.size() > capacity) return PKV_ERR_SHAPE;
  if (!q.blocks.empty() && !blocks) return PKV_ERR_NULL;
  for (size_t i = 0; i < q.blocks.size(); ++i) blocks[i] = q.blocks[i];
  return PKV_OK;
}

int pkv_bm_tables(const pkv_block_manager* m, const int32_t* seqs, int32_t n_seqs, int32_t* tables,
                  int32_t max_blocks_per_seq, int32_t fill, int32_t* lens) {
  if (!m) return PKV_ERR_NULL;
  if (n_seqs < 0 || max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
  if (n_seqs == 0) return PKV_OK;
  if (!seqs || !tables || !lens) return PKV_ERR_NULL;
  for (int32_t i = 0; i < n_seqs; ++i) {
    if (!m->valid(seqs[i])) return PKV_ERR_BAD_SEQUENCE;
    if ((int32_t)m->seqs[(size_t)seqs[i]].blocks.size() > max_blocks_per_seq) return PKV_ERR_SHAPE;
    if (m->seqs[(size_t)seqs[i]].len > 0x7fffffffLL) return PKV_ERR_SHAPE;
  }
  for (int32_t i = 0; i < n_seqs; ++i) {
    const Sequence& q = m->seqs[(size_t)seqs[i]];
    int32_t* row = tables + (size_t)i * max_blocks_per_seq;
    size_t j = 0;
    for (; j < q.blocks.size(); ++j) row[j] = q.blocks[j];
    for (; j < (size_t)max_blocks_per_seq; ++j) row[j] = fill;
    lens[i] = (int32_t)q.len;
  }
  return PKV_OK;
}

int pkv_bm_swap_out(pkv_block_manager* m, int32_t seq, int32_t* blocks, int32_t capacity, int32_t* n_blocks) {
  if (!m || !n_blocks) return PKV_ERR_NULL;
  if (!m->valid(seq)) return PKV_ERR_BAD_SEQUENCE;
  Sequence& q = m->seqs[(size_t)seq];
  *n_blocks = (int32_t)q.blocks.size();
  if ((int32_t)q.blocks.size() > capacity) return PKV_ERR_SHAPE;
  if (!q.blocks.empty() && !blocks) return PKV_ERR_NULL;
  for (size_t i = 0; i < q.blocks.size(); ++i) blocks[i] = q.blocks[i];
  for (int32_t b : q.blocks) m->release(b);
  q.blocks.clear();
  q.live = false;
  q.swapped = true;
  return PKV_OK;
}

int pkv_bm_swap_in(pkv_block_manager* m, int32_t seq, int32_t* blocks, int32_t capacity, int32_t* n_blocks) {
  if (!m || !n_blocks) return PKV_ERR_NULL;
  if (seq < 0 || (size_t)seq >= m->seqs.size() || !m->seqs[(size_t)seq].swapped) return PKV_ERR_BAD_SEQUENCE;
  Sequence& q = m->seqs[(size_t)seq];
  const int64_t need = (q.len + m->block_size - 1) / m->block_size;
  *n_blocks = (int32_t)need;
  if (need > capacity) return PKV_ERR_SHAPE;
  if (need > 0 && !blocks) return PKV_ERR_NULL;
  if (need > m->pool.count()) return PKV_ERR_OUT_OF_BLOCKS;
  for (int64_t i = 0; i < need; ++i) {
    const int32_t b = m->take();
    q.blocks.push_back(b);
    blocks[i] = b;
  }
  q.live = true;
  q.swapped = false;
  return PKV_OK;
}

int pkv_bm_ref_count(const pkv_block_manager* m, int32_t block, int32_t* ref) {
  if (!m || !ref) return PKV_ERR_NULL;
  if (block < 0 || block >= m->num_blocks) return PKV_ERR_SHAPE;
  *ref = m->ref[(size_t)block];
  return PKV_OK;
}

int32_t pkv_bm_free_blocks(const pkv_block_manager* m) { return m ? m->pool.count() : -1; }

int pkv_bm_usage(const pkv_block_manager* m, int64_t* used_blocks, int64_t* filled_slots, int64_t* live_seqs,
                 int64_t* held_tokens) {
  if (!m || !used_blocks || !filled_slots || !live_seqs || !held_tokens) return PKV_ERR_NULL;
  // A block's filled slots are those of any sequence holding it: sharers hold
  // identical prefixes (a write into a shared block first makes a copy).
  std::vector<int32_t> fill((size_t)m->num_blocks, 0);
  int64_t live = 0, held = 0;
  for (const Sequence& q : m->seqs) {
    if (!q.live) continue;
    ++live;
    held += q.len;
    for (size_t b = 0; b < q.blocks.size(); ++b) {
      const int64_t f = q.len - (int64_t)b * m->block_size;
      const int32_t fb = (int32_t)(f < m->block_size ? f : m->block_size);
      int32_t& slot = fill[(size_t)q.blocks[b]];
      if (fb > slot) slot = fb;
    }
  }
  int64_t filled = 0;
  for (int32_t f : fill) filled += f;
  *used_blocks = m->num_blocks - m->pool.count();
  *filled_slots = filled;
  *live_seqs = live;
  *held_tokens = held;
  return PKV_OK;
}

}  // extern "C"
