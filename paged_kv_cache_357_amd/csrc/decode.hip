// Paged decode attention for gfx950 (MI355X, CDNA4).
//
// What is computed follows "PagedAttention and vLLM Architecture: Virtual
// Memory for LLM Serving", section 2 (PagedAttention Attention CUDA Kernel
// Mechanics): the query of the decoded token is dotted with the keys of every
// cached token, fetched physical block by physical block through the
// sequence's block table, and an online softmax is fused with the product by
// the Value rows.  Token i is read from slot T[i / B] * B + i % B
// ("PagedAttention Paper Breakdown", section 2, Address Translation Formula).
//
// Work is cut into 16-token chunks of one (sequence s, kv head g) segment; a
// chunk lies inside one physical block, so its rows start at a wave-uniform
// address.  One wavefront (64 lanes) is one worker: it streams its chunks
// with the loads of the next chunk in flight while the current one is
// consumed, keeps the online-softmax state of the kv head's GQA group of
// query heads in registers, and at the end of each segment piece produces
// either the finished rows or a partial (max, sum, accumulator) record that a
// second kernel merges with the log-sum-exp rule.  Pieces wait in the wave's
// LDS queue and are written after its last chunk: stores share the in-order
// memory counter with the loads, so one amid the stream would hold up the
// waits for the chunks issued after it.  The waves of a workgroup share
// nothing after the prologue (each has its own LDS tile and queue; no barrier
// in the loop).
//
// Two schedules hand out the chunks:
//   * balanced: all segments laid end to end, (s, g) in order, are cut into
//     one share of equal cost per worker wave (a segment costs its chunks
//     plus a small charge for its start), and the grid holds exactly as many
//     waves as the chip keeps resident, so every wave starts at once and all
//     finish together (no tail of long units started late).  A share may
//     begin or end inside a segment; such pieces leave partial records (at
//     most two per wave).  Each workgroup first builds the per-sequence chunk
//     prefix sums in LDS to locate its shares.
//   * partitioned: a unit is (s, g, partition p) of P consecutive tokens, one
//     wave per unit, units numbered ((p * S + s) * Hkv + g); used when the
//     caller fixes the partition size, when every sequence fits one
//     partition, or for batches too long for the LDS tables.
// In both, the hardware deals consecutive workgroup ids round robin over the
// 8 XCDs; the launch permutes ids so that groups of consecutive logical
// workgroups (neighbouring heads of the same tokens) share an XCD and its L2.
//
// Two compute cores consume a chunk:
//   * ValuCore (fp32 caches, and bf16 with fewer than 4 query heads per kv
//     head): a token row of one kv head is D * elt bytes; LPT lanes cover it
//     with one 16-byte load each (one wave load instruction reads TPI =
//     64 / LPT whole rows); partial dot products are finished with DPP adds
//     across the LPT lanes; each lane group keeps its own softmax state, and
//     the groups are merged at the end of a piece.
//   * MfmaCore (bf16 with 4 or more query heads per kv head): scores and the
//     V product are 16x16 matrix products on the matrix cores (see below).
//
// Every reduction order depends only on logical token positions and on the
// lengths of the batch, never on which physical block holds a token, so
// outputs are bitwise independent of the block layout and bitwise
// reproducible.
//
// Fused append (paged_attn_decode_append): the lengths are those before the
// append, L + 1 tokens are attended, and each sequence's new K/V row goes to
// position L.  The balanced kernel (either core) loads the row ahead through
// its pipeline, keeps it in LDS, substitutes it for the slot's old contents in
// the segment's last chunk and writes it to the pool after its last chunk; the
// partitioned kernel writes it before its first load.
//
// Masking: rows at or beyond a piece's end inside its last chunk read as zero
// through a bounds-checked buffer resource; their scores are -inf, hence
// weight exactly 0.  Running maxima start at -1e30 rather than -inf so that a
// lane that has seen no token yet rescales by exp2(0) = 1 instead of
// exp2(-inf + inf) = NaN.

#include "decode_core.h"

namespace pkv {
namespace {

// ---------------------------------------------------- partitioned schedule

template <class Core>
__global__ __launch_bounds__(kThreads) void decode_partitioned_kernel(DecodeParams a) {
  constexpr int B = Core::kBlock, D = Core::kHeadDim, G = Core::kGroup, ROW = Core::ROW;
  __shared__ __attribute__((aligned(16))) char s_stage[kWavesPerWG][Core::kStageBytes];
  const int ell = logical_workgroup(blockIdx.x, a.xcd_group, a.n_wg, a.xcds);
  if (ell < 0) return;
  const int wave = uniform(threadIdx.x >> 6);
  const int u = ell * kWavesPerWG + wave;
  if (u >= a.n_units) return;
  const int lane = threadIdx.x & 63;
  const int g = u % a.Hkv;
  const int sp = u / a.Hkv;
  const int s = sp % a.S;
  const int part = sp / a.S;

  const int L = attended_len(a, s);
  const int tok0 = part * a.P;
  const bool bad_len = L < 0;
  const bool direct = (L <= a.P);  // this sequence fits one partition: write out directly
  float* orow = a.out + ((size_t)s * a.Hq + (size_t)g * G) * D;

  if (bad_len || tok0 >= L) {
    // Nothing to attend to.  The partition-0 unit owns the output rows of
    // sequences handled directly (L = 0 gives zeros, a bad length NaN);
    // otherwise the merge kernel writes them.
    if (part == 0 && (bad_len || direct)) {
      const float fill = bad_len ? __builtin_nanf("") : 0.0f;
      for (int i = lane; i < G * D; i += 64) orow[i] = fill;
    }
    return;
  }

  const int tok_end = min(tok0 + a.P, L);
  const int n_chunks = (tok_end - tok0 + kChunk - 1) / kChunk;
  const int blk0 = tok0 / B;
  const int n_blk = (tok_end - 1) / B - blk0 + 1;
  const int32_t* trow = a.tables + (size_t)s * a.MB + blk0;
  const uint32_t rs = (uint32_t)a.Hkv * ROW;  // bytes between slots of one head
  const char* kbase = static_cast<const char*>(a.k) + (size_t)g * ROW;
  const char* vbase = static_cast<const char*>(a.v) + (size_t)g * ROW;

  Core core;
  core.init(lane, rs, s_stage[wave]);
  // Fused append: the unit holding the last position writes the new token
  // before it loads any row.
  const bool appends = a.append && L - 1 < tok_end;
  NewRow<ROW> nr;
  if (appends) nr = load_new_row<ROW>(a, B, s, g, L - 1, lane);
  bool bad = false;
  int wbase = 0;
  int tbl = load_table_window(trow, 0, n_blk, lane, a.NB, &bad);
  core.load_q(a, s, g);
  core.reset();
  if (appends) store_new_row<ROW>(a, B, nr, g, L - 1, lane);

  auto issue = [&](int c, typename Core::Buf& b) {
    const int cs = tok0 + c * kChunk;
    const int bi = cs / B - blk0;
    if (bi - wbase >= 64) {
      wbase += 64;
      tbl = load_table_window(trow, wbase, n_blk, lane, a.NB, &bad);
    }
    const int phys = __builtin_amdgcn_readlane(tbl, bi - wbase);
    const size_t cbase = ((size_t)phys * B + (size_t)(cs % B)) * rs;
    const int lim = min(kChunk - 1, tok_end - 1 - cs);  // last valid row of the chunk
    core.issue(kbase + cbase, vbase + cbase, rs, (uint32_t)lim * rs + ROW, b);
  };

  // The loads of chunk c+1 are issued before chunk c is consumed.  The steady
  // state issues unconditionally (the last one or two chunks are peeled), so
  // the wait before each consume covers only the older chunk's loads.
  auto consume = [&](int c, const typename Core::Buf& b) {
    core.consume(tok_end - 1 - (tok0 + c * kChunk), a.scale_log2, b);
  };
  typename Core::Buf ba, bb;
  issue(0, ba);
  int c = 0;
  for (; c + 2 < n_chunks; c += 2) {
    issue(c + 1, bb);
    consume(c, ba);
    issue(c + 2, ba);
    consume(c + 1, bb);
  }
  if (c + 1 < n_chunks) {
    issue(c + 1, bb);
    consume(c, ba);
    consume(c + 1, bb);
  } else {
    consume(c, ba);
  }

  PieceSink o;
  o.direct = direct;
  o.bad = bad;
  o.out = orow;
  const size_t r0 = ((size_t)s * a.Hq + (size_t)g * G) * a.NP + part;  // head 0 of the group
  o.acc = a.ws_acc + r0 * D;
  o.acc_stride = (size_t)a.NP;
  o.ml = a.ws_ml + r0;
  o.ml_stride = (size_t)a.NP;
  core.finish(o);
}

// Stage 2 of the partitioned schedule: merge the partitions of sequences
// longer than one partition.  One workgroup of 4 waves per (sequence, query
// head).  Partition p contributes exp2(m_p - M) * (acc_p, l_p), M the largest
// m_p.  Wave w sums a contiguous quarter of the partitions in increasing
// order, then wave 0 adds the four partial sums in wave order.  Lane j owns
// columns j*CPL .. j*CPL + CPL - 1.
template <int D>
__global__ __launch_bounds__(kThreads) void decode_reduce_partitioned_kernel(DecodeParams a) {
  constexpr int CPL = D / 64;  // columns per lane (1 or 2)
  __shared__ float s_num[kWavesPerWG][D];
  __shared__ float s_den[kWavesPerWG];
  const int row = blockIdx.x;  // s * Hq + h
  const int s = row / a.Hq;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int L = attended_len(a, s);
  const bool bad_len = L < 0;
  if (!bad_len && L <= a.P) return;  // written by stage 1 (or L = 0 zeros); uniform over the workgroup
  float* o = a.out + (size_t)row * D + lane * CPL;
  if (bad_len) {
    if (wave == 0) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) o[j] = __builtin_nanf("");
    }
    return;
  }
  const int np = (L + a.P - 1) / a.P;
  const float2* ml = a.ws_ml + (size_t)row * a.NP;
  const float* acc = a.ws_acc + (size_t)row * a.NP * D + lane * CPL;

  float M = kNegBig;
  for (int p = lane; p < np; p += 64) M = fmaxf(M, ml[p].x);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));

  const int p_begin = (int)((long long)np * wave / kWavesPerWG);
  const int p_end = (int)((long long)np * (wave + 1) / kWavesPerWG);
  float den = 0.0f;
  float num[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) num[j] = 0.0f;
  for (int p0 = p_begin; p0 < p_end; p0 += 64) {
    float f = 0.0f;
    if (p0 + lane < p_end) {
      const float2 t = ml[p0 + lane];
      f = fast_exp2(t.x - M);
      den = fmaf(t.y, f, den);
    }
    const int cnt = min(64, p_end - p0);
    const float* ap = acc + (size_t)p0 * D;
    // eight partitions per step, so eight loads are in flight at once
    for (int j0 = 0; j0 < cnt; j0 += 8) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int j = j0 + jj;
        if (j < cnt) {
          const float fj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), j));
          if constexpr (CPL == 2) {
            const float2 t = *reinterpret_cast<const float2*>(ap + (size_t)j * D);
            num[0] = fmaf(t.x, fj, num[0]);
            num[1] = fmaf(t.y, fj, num[1]);
          } else {
            num[0] = fmaf(ap[(size_t)j * D], fj, num[0]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
#pragma unroll
  for (int j = 0; j < CPL; ++j) s_num[wave][lane * CPL + j] = num[j];
  if (lane == 0) s_den[wave] = den;
  __syncthreads();
  if (wave != 0) return;
  float tn[CPL], td = 0.0f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) tn[j] = 0.0f;
#pragma unroll
  for (int w = 0; w < kWavesPerWG; ++w) {
    td += s_den[w];
#pragma unroll
    for (int j = 0; j < CPL; ++j) tn[j] += s_num[w][lane * CPL + j];
  }
  if constexpr (CPL == 2) {
    *reinterpret_cast<float2*>(o) = make_float2(tn[0] / td, tn[1] / td);
  } else {
    o[0] = tn[0] / td;
  }
}

// ------------------------------------------------------- balanced schedule
//
// Segment (s, g) holds n_s = ceil(L_s / 16) chunks (0 for L_s <= 0 or an
// invalid length); segments are laid out in (s, g) order, so segment (s, g)
// starts at chunk Hkv * C_s + g * n_s, C_s = n_0 + .. + n_{s-1}, and the
// whole batch is T = Hkv * C_S chunks.  Shares are cut in cost units: a
// segment costs kSegCost for its start plus its n_s chunks, the batch TC
// units, and with W worker waves (W_eff = min(W, max(1, T /
// kBalancedMinChunks)) of them get work) wave w takes the chunks whose cost
// positions lie in [w TC / W_eff, (w+1) TC / W_eff).  A piece of a segment
// that this wave both starts and ends is written directly; otherwise the
// wave leaves a partial record in slot 0 (the piece continues a segment
// begun by an earlier wave) or slot 1 (the piece begins a segment that a
// later wave continues).


template <class Core, bool APPEND>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Core::kWavesPerSimd)))
void decode_balanced_kernel(DecodeParams a) {
  constexpr int B = Core::kBlock, D = Core::kHeadDim, G = Core::kGroup, ROW = Core::ROW;
  constexpr int REC = piece_record_bytes(G, D);
  extern __shared__ __attribute__((aligned(16))) int smem[];
  __shared__ __attribute__((aligned(16))) char s_stage[kWavesPerWG][Core::kStageBytes];
  int* pref = smem;               // [S + 1] chunk prefix sums C_s
  int* slen = smem + a.S + 1;     // [S] lengths (0 for invalid ones)
  int* pcost = smem + 2 * a.S + 1;  // [S + 1] cost prefix sums: chunks + kSegCost per non-empty sequence
  __shared__ int s_wave_sum[kWavesPerWG];
  __shared__ int s_wave_cost[kWavesPerWG];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);

  // Per-sequence chunk counts and their exclusive prefix sums.
  {
    const int per = (a.S + kThreads - 1) / kThreads;
    const int s_lo = min(a.S, tid * per);
    const int s_hi = min(a.S, s_lo + per);
    int local = 0, local_c = 0;
    for (int s = s_lo; s < s_hi; ++s) {
      const int Lv = max(attended_len(a, s), 0);
      slen[s] = Lv;
      const int n = (Lv + kChunk - 1) / kChunk;
      local += n;
      local_c += n > 0 ? n + kSegCost : 0;
    }
    int incl = local, incl_c = local_c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off);
      const int tc = __shfl_up(incl_c, off);
      if (lane >= off) {
        incl += t;
        incl_c += tc;
      }
    }
    if (lane == 63) {
      s_wave_sum[wave] = incl;
      s_wave_cost[wave] = incl_c;
    }
    __syncthreads();
    int run = incl - local, run_c = incl_c - local_c;
    for (int w = 0; w < wave; ++w) {
      run += s_wave_sum[w];
      run_c += s_wave_cost[w];
    }
    for (int s = s_lo; s < s_hi; ++s) {
      pref[s] = run;
      pcost[s] = run_c;
      const int n = (slen[s] + kChunk - 1) / kChunk;
      run += n;
      run_c += n > 0 ? n + kSegCost : 0;
    }
    if (tid == kThreads - 1) {
      pref[a.S] = run;
      pcost[a.S] = run_c;
    }
    __syncthreads();
  }
  if (blockIdx.x == 0)
    for (int s = tid; s <= a.S; s += kThreads) {
      a.ws_pref[s] = pref[s];
      a.ws_pref[a.S + 1 + s] = pcost[s];
    }

  // Work is laid out over (sequence, head group, chunk); a head group is HG
  // adjacent kv heads.  With HG = 1 each wave is a worker; with HG = 4 the
  // four waves of a workgroup share one share and take one head of the group
  // each, so they read adjacent 256-byte rows of the same tokens together.
  const int Hkv = a.Hkv;
  const int HG = a.head_group;
  const int NGR = Hkv / HG;
  const long long T = (long long)NGR * uniform(pref[a.S]);
  const int ell = logical_workgroup(blockIdx.x, a.xcd_group, a.n_wg, a.xcds);
  if (ell < 0 || T == 0) return;
  const int w = ell * kWavesPerWG + wave;               // this wave's partial-record slots
  const int worker = HG == 1 ? w : ell;
  const long long W_eff = balanced_workers(T, HG == 1 ? a.n_units : a.n_wg);
  if (worker >= W_eff) return;
  const int hsub = HG == 1 ? 0 : wave;                  // head of the group this wave takes
  // Shares are equal in cost: a segment costs its chunks plus kSegCost for
  // its start (query fetch, table entries, piece write).  chunk_at maps a
  // cost position to the first chunk at or after it.
  const long long TC = (long long)NGR * uniform(pcost[a.S]);
  auto chunk_at = [&](long long x) -> long long {
    if (x >= TC) return T;
    const int sa2 = last_at_most(pcost, a.S, NGR, x, lane);
    const int n = uniform(pref[sa2 + 1]) - uniform(pref[sa2]);
    const long long rel = x - (long long)NGR * uniform(pcost[sa2]);
    const long long seg = n + kSegCost;
    const long long g2 = rel / seg;
    const long long r = rel - g2 * seg;
    const long long j = r < kSegCost ? 0 : r - kSegCost;
    return (long long)NGR * uniform(pref[sa2]) + g2 * n + j;
  };
  const long long lo = chunk_at((long long)worker * TC / W_eff);
  const long long hi = chunk_at((long long)(worker + 1) * TC / W_eff);

  // Locate the segment holding chunk lo: the last s with NGR * C_s <= lo.
  const int sa = last_at_most(pref, a.S, NGR, lo, lane);
  struct Cursor {
    int s, g, j, n, L;  // g: head group
  };
  auto chunks_of = [&](int s) { return uniform(pref[s + 1]) - uniform(pref[s]); };
  Cursor ic;
  ic.s = sa;
  ic.n = chunks_of(sa);
  ic.L = uniform(slen[sa]);
  {
    const long long rel = lo - (long long)NGR * uniform(pref[sa]);
    ic.g = (int)(rel / ic.n);
    ic.j = (int)(rel - (long long)ic.g * ic.n);
  }
  auto advance = [&](Cursor& c) {
    if (++c.j < c.n) return;
    c.j = 0;
    if (++c.g < NGR) return;
    c.g = 0;
    do {
      ++c.s;
    } while (c.s < a.S && chunks_of(c.s) == 0);
    if (c.s < a.S) {
      c.n = chunks_of(c.s);
      c.L = uniform(slen[c.s]);
    }
  };
  Cursor cc = ic;

  const uint32_t rs = (uint32_t)Hkv * ROW;  // bytes between slots of one head
  const char* kpool = static_cast<const char*>(a.k);
  const char* vpool = static_cast<const char*>(a.v);
  char* kpool_w = static_cast<char*>(const_cast<void*>(a.k));  // fused append writes
  char* vpool_w = static_cast<char*>(const_cast<void*>(a.v));
  Core core;
  core.init(lane, rs, s_stage[wave]);

  // Software pipeline of depth NB: the loads of the next NB-1 chunks are in
  // flight while a chunk is consumed.  Every step issues the same load
  // sequence: the next chunk of the share, or past its end a load-free dummy
  // (zero-size resources), so the wait before each consume covers only the
  // consumed chunk's loads.  A chunk that opens a segment (or the wave's
  // first chunk) also brings the segment's query rows, loaded before the
  // chunk's rows.
  //
  // Block-table entries are read NB issues ahead: each pipeline slot also
  // loads the entry of the chunk that will be issued into it next (a
  // lookahead cursor runs NB chunks ahead of the issue cursor), and that
  // entry is used only after the slot's own chunk has been consumed, that is
  // after the wait that covers it.  A table read at the point of use would
  // have to wait for every load in flight (the memory counter is in order),
  // emptying the pipeline at each new sequence.
  //
  // With the fused append (APPEND), the same lookahead brings the new rows:
  // when the lookahead chunk begins a segment whose last chunk lies in this
  // share, the slot also loads that segment's new K and V row and the table
  // entry of the row's block.  After the slot's chunk is consumed the row
  // goes into the wave's LDS row store; the segment's last chunk, which was
  // loaded from the pool before the row is written there, takes the row from
  // LDS in place of the slot's old contents, and the rows are written to the
  // pool with the finished pieces after the wave's last chunk (a store amid
  // the stream would hold up the loads issued after it).  Rows beyond the
  // store's capacity are written to the pool at once instead, before any
  // chunk of their segment is issued: a wave's memory operations on one
  // address take effect in program order, so the segment's loads see them.
  // Only this wave reads a segment's last chunk.
  constexpr int NB = Core::kPipeline;
  long long to_issue = hi - lo, to_consume = hi - lo;
  typename Core::Buf buf[NB];
  bool bad[NB];
  bool first_issue = true;
  Cursor la = ic;        // lookahead cursor
  long long la_pos = lo; // chunk index of la
  auto next_entry = [&](AppendSlot<ROW>& sl) {
    sl.off = -1;
    if (la_pos >= hi) return;
    sl.nid = a.tables[(size_t)la.s * a.MB + (la.j * kChunk) / B];
    if constexpr (APPEND) {
      if ((la.j == 0 || la_pos == lo) && la_pos + (la.n - 1 - la.j) < hi) {
        const int p = la.L - 1;  // the appended position
        const int head = la.g * HG + hsub;
        sl.row = load_new_row<ROW>(a, B, la.s, head, p, lane);
        sl.off = ((long long)(p % B) * Hkv + head) * ROW;
      }
    }
    if (++la_pos < hi) advance(la);
  };
  // LDS of this wave: the finished-piece queue, then the row store (entries
  // of RENTRY bytes: the row's pool offset or -1, 8 spare, the K row, the V
  // row).
  char* queue = reinterpret_cast<char*>(smem + ((3 * a.S + 2 + 3) & ~3)) +
                (size_t)wave * (a.queue_bytes + a.row_bytes);
  char* rowst = queue + a.queue_bytes;
  constexpr int RENTRY = 16 + 2 * ROW;
  const int r_cap = a.row_bytes / RENTRY;
  int r_commit = 0, r_use = 0;  // rows stored, rows substituted (the same segments, in order)
  typedef __attribute__((address_space(1))) u32x4 g_u32x4;  // global memory
  auto commit = [&](AppendSlot<ROW>& sl) {
    if constexpr (APPEND) {
      if (sl.off >= 0) {
        const int blk = uniform(sl.row.blk);
        const bool valid = blk >= 0 && blk < a.NB;  // an id outside the pool writes nothing
        const long long d = valid ? (long long)blk * B * rs + sl.off : -1;
        if (r_commit < r_cap) {
          char* e = rowst + r_commit * RENTRY;
          if (lane == 0) *reinterpret_cast<long long*>(e) = d;
          uint32_t* ek = reinterpret_cast<uint32_t*>(e + 16);
          uint32_t* ev = reinterpret_cast<uint32_t*>(e + 16 + ROW);
#pragma unroll
          for (int j = 0; j < NewRow<ROW>::NW; ++j) {
            const int wd = lane + 64 * j;
            if (wd < NewRow<ROW>::NWORD) {
              ek[wd] = sl.row.k[j];
              ev[wd] = sl.row.v[j];
            }
          }
        } else if (valid) {
          put_new_row<ROW>(a, sl.row, (size_t)d, lane);
        }
        ++r_commit;
        sl.off = -1;
      }
    }
  };
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    buf[k].app.nid = 0;
    next_entry(buf[k].app);  // entries (and rows) of the first NB chunks
  }
#pragma unroll
  for (int k = 0; k < NB; ++k) commit(buf[k].app);

  auto issue_next = [&](typename Core::Buf& b, bool& bbad) {
    const char* kc = kpool;
    const char* vc = vpool;
    uint32_t nbytes = 0;
    bbad = false;
    if (to_issue > 0) {
      if (first_issue || ic.j == 0) core.fetch_q(a, ic.s, ic.g * HG + hsub, b);
      first_issue = false;
      const int cs = ic.j * kChunk;
      const int id = uniform(b.app.nid);      // this chunk's table entry, loaded NB issues ago
      const bool ok = id >= 0 && id < a.NB;   // an id outside the pool is never dereferenced
      bbad = !ok;
      const size_t cbase =
          ((size_t)(ok ? id : 0) * B + (size_t)(cs % B)) * rs + (size_t)(ic.g * HG + hsub) * ROW;
      kc = kpool + cbase;
      vc = vpool + cbase;
      nbytes = ok ? (uint32_t)min(kChunk - 1, ic.L - 1 - cs) * rs + ROW : 0u;  // rows 0 .. lim of this head
      next_entry(b.app);  // for the chunk issued into this slot next
      --to_issue;
      if (to_issue > 0) advance(ic);
    }
    core.issue(kc, vc, rs, nbytes, b);
  };

  // Finished pieces wait in this wave's LDS queue and are written out after
  // its last chunk (or when the queue is full).  The memory counter is in
  // order and counts stores too, so a store issued amid the stream would
  // hold up the wait for every chunk issued after it until the store is
  // acknowledged, which under a full read stream takes longer than a load.
  // A record: global destinations of the rows and of the (max, sum) pairs
  // (0: none), then G * D floats, then G pairs.
  const int q_cap = a.queue_bytes / REC;  // at least one (the plan sees to it)
  int q_n = 0;
  auto flush = [&]() {
    for (int r = 0; r < q_n; ++r) {
      const char* rec = queue + r * REC;
      const uint64_t gd = *reinterpret_cast<const uint64_t*>(rec);
      const uint64_t gm = *reinterpret_cast<const uint64_t*>(rec + 8);
      typedef __attribute__((address_space(1))) f32x4 g_f32x4;  // global memory
      typedef __attribute__((address_space(1))) u32x2 g_u32x2;
      g_f32x4* dst = (g_f32x4*)(
          ((uint64_t)(uint32_t)uniform((int)(uint32_t)(gd >> 32)) << 32) | (uint32_t)uniform((int)(uint32_t)gd));
      const f32x4* src = reinterpret_cast<const f32x4*>(rec + 16);
      for (int i = lane; i < G * D / 4; i += 64) dst[i] = src[i];
      if (gm != 0 && lane < G) ((g_u32x2*)gm)[lane] = reinterpret_cast<const u32x2*>(rec + 16 + 4 * G * D)[lane];
    }
    q_n = 0;
  };

  bool started = false;
  bool seg_bad = false;
  bool first_consume = true;
  // One step: issue into the slot consumed one step earlier, consume the
  // current chunk, write the new row the slot brought, close the segment
  // piece if it ends here (into the queue), step the cursor.
  auto step = [&](typename Core::Buf& cur, bool curbad, typename Core::Buf& nxt, bool& nxtbad) {
    issue_next(nxt, nxtbad);
    if (to_consume <= 0) return;
    if (first_consume || cc.j == 0) {
      core.take_q(cur);
      core.reset();
      started = (cc.j == 0);
      seg_bad = false;
      first_consume = false;
    }
    const int lim = min(kChunk - 1, cc.L - 1 - cc.j * kChunk);
    const bool seg_end = (cc.j == cc.n - 1);
    if constexpr (APPEND) {
      if (seg_end) {  // row lim is the new token
        if (r_use < r_cap) {
          const char* e = rowst + r_use * RENTRY;
          core.substitute(lim, cur, e + 16, e + 16 + ROW);
        }
        ++r_use;
      }
    }
    core.consume(lim, a.scale_log2, cur);
    commit(cur.app);
    seg_bad |= curbad;
    --to_consume;
    if (seg_end || to_consume == 0) {
      if (q_n == q_cap) flush();
      char* rec = queue + q_n * REC;
      PieceSink o;
      o.direct = started && seg_end;
      o.bad = seg_bad;
      o.out = reinterpret_cast<float*>(rec + 16);  // G rows of D, then G pairs
      o.acc = o.out;
      o.acc_stride = 1;
      o.ml = reinterpret_cast<float2*>(rec + 16 + 4 * G * D);
      o.ml_stride = 1;
      if (lane == 0) {
        const size_t r0 = ((size_t)w * 2 + (started ? 1 : 0)) * G;
        float* rows = o.direct ? a.out + ((size_t)cc.s * a.Hq + (size_t)(cc.g * HG + hsub) * G) * D
                               : a.ws_acc + r0 * D;
        reinterpret_cast<uint64_t*>(rec)[0] = reinterpret_cast<uint64_t>(rows);
        reinterpret_cast<uint64_t*>(rec)[1] = o.direct ? 0 : reinterpret_cast<uint64_t>(a.ws_ml + r0);
      }
      core.finish(o);
      ++q_n;
    }
    if (to_consume > 0) advance(cc);
  };

#pragma unroll
  for (int k = 0; k < NB - 1; ++k) issue_next(buf[k], bad[k]);
  while (to_consume > 0) {
#pragma unroll
    for (int k = 0; k < NB; ++k) step(buf[k], bad[k], buf[(k + NB - 1) % NB], bad[(k + NB - 1) % NB]);
  }
  flush();
  if constexpr (APPEND) {
    const int nr = min(r_commit, r_cap);
    for (int r = 0; r < nr; ++r) {
      const char* e = rowst + r * RENTRY;
      const long long d = *reinterpret_cast<const long long*>(e);
      if (d >= 0 && lane < ROW / 16) {  // 16 bytes a lane from LDS
        *(g_u32x4*)(kpool_w + d + lane * 16) = *reinterpret_cast<const u32x4*>(e + 16 + lane * 16);
        *(g_u32x4*)(vpool_w + d + lane * 16) = *reinterpret_cast<const u32x4*>(e + 16 + ROW + lane * 16);
      }
    }
  }
}

// Stage 2 of the balanced schedule: one wave per segment (s, g), merging the
// G query-head rows h of kv head g together, four segments per workgroup.  An
// invalid length gives NaN rows and L = 0 zeros; a segment that one wave
// finished was written by stage 1; otherwise the pieces of waves w0 .. w1
// (slot 1 of w0, slot 0 of the later ones) are merged in wave order:
// exp2(m_w - M) * (acc_w, l_w) summed, M the largest m_w.  Lane j owns
// columns j*CPL .. j*CPL + CPL - 1.
template <int D, int G>
__global__ __launch_bounds__(kThreads) void decode_reduce_balanced_kernel(DecodeParams a) {
  constexpr int CPL = D / 64;  // columns per lane (1 or 2)
  // Pieces whose records are loaded together (registers: KB * G * (CPL + 2)).
  constexpr int KB = G <= 2 ? 8 : (G <= 4 ? 4 : 2);
  const int lane = threadIdx.x & 63;
  const int seg = blockIdx.x * kWavesPerWG + uniform(threadIdx.x >> 6);  // s * Hkv + kv head
  if (seg >= a.S * a.Hkv) return;
  const int s = seg / a.Hkv;
  const int g = seg - s * a.Hkv;
  // Everything that depends on s alone is loaded before anything is decided,
  // so the loads are in flight together.
  const int L = attended_len(a, s);
  const int pref_S = a.ws_pref[a.S];
  const int cost_S = a.ws_pref[a.S + 1 + a.S];
  const int cost_s = a.ws_pref[a.S + 1 + s];
  float* o0 = a.out + ((size_t)s * a.Hq + (size_t)g * G) * D + lane * CPL;  // row h at o0 + h * D
  if (L <= 0) {
    const float fill = L == 0 ? 0.0f : __builtin_nanf("");
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int j = 0; j < CPL; ++j) o0[(size_t)h * D + j] = fill;
    return;
  }
  const int HG = a.head_group;
  const int NGR = a.Hkv / HG;
  const long long T = (long long)NGR * pref_S;
  const long long W_eff = balanced_workers(T, HG == 1 ? a.n_units : a.n_wg);
  const int n = (L + kChunk - 1) / kChunk;
  const long long TC = (long long)NGR * cost_S;
  const long long cbase = (long long)NGR * cost_s + (long long)(g / HG) * (n + kSegCost) + kSegCost;
  const long long w0 = balanced_wave_of(cbase, TC, W_eff);  // first and last worker of the segment
  const long long w1 = balanced_wave_of(cbase + n - 1, TC, W_eff);
  const int hsub = g % HG;
  if (w0 == w1) return;
  const int k = (int)(w1 - w0 + 1);
  auto piece_row = [&](int p) -> size_t {  // row of head 0 of the group; head h is + h
    const size_t wave_id = HG == 1 ? (size_t)(w0 + p) : (size_t)(w0 + p) * kWavesPerWG + hsub;
    return (wave_id * 2 + (p == 0 ? 1 : 0)) * G;
  };

  // Pieces in wave order, KB at a time: M is the largest max so far, and a
  // later batch with a larger one rescales the sums.  With k <= KB this is
  // one batch: M over all pieces, then the sums in piece order.
  float M[G], num[G][CPL], den[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    M[h] = kNegBig;
    den[h] = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) num[h][j] = 0.0f;
  }
  for (int p0 = 0; p0 < k; p0 += KB) {
    float2 t[KB][G];
    float x[KB][G][CPL];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const bool in = p0 + i < k;
      const size_t r = piece_row(in ? p0 + i : p0);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        t[i][h] = in ? a.ws_ml[r + h] : make_float2(kNegBig, 0.0f);
        if constexpr (CPL == 2) {
          const float2 v = in ? *reinterpret_cast<const float2*>(a.ws_acc + (r + h) * D + lane * CPL)
                              : make_float2(0.0f, 0.0f);
          x[i][h][0] = v.x;
          x[i][h][1] = v.y;
        } else {
          x[i][h][0] = in ? a.ws_acc[(r + h) * D + lane] : 0.0f;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float Mn = M[h];
#pragma unroll
      for (int i = 0; i < KB; ++i) Mn = fmaxf(Mn, t[i][h].x);
      if (p0 > 0) {
        const float sc = fast_exp2(M[h] - Mn);
        den[h] *= sc;
#pragma unroll
        for (int j = 0; j < CPL; ++j) num[h][j] *= sc;
      }
      M[h] = Mn;
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        if (p0 + i < k) {
          const float f = fast_exp2(t[i][h].x - M[h]);
          den[h] = fmaf(t[i][h].y, f, den[h]);
#pragma unroll
          for (int j = 0; j < CPL; ++j) num[h][j] = fmaf(x[i][h][j], f, num[h][j]);
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float* o = o0 + (size_t)h * D;
    if constexpr (CPL == 2) {
      *reinterpret_cast<float2*>(o) = make_float2(num[h][0] / den[h], num[h][1] / den[h]);
    } else {
      o[0] = num[h][0] / den[h];
    }
  }
}

// The same merge for long segments cut into many pieces: a workgroup of four
// waves per query-head row.  Thread t owns column t % D and the pieces
// w0 + t / D, w0 + t / D + SUBS, .. (SUBS = 256 / D subsets, each summed in
// increasing order); the subsets are then added in subset order.
template <int D>
__global__ __launch_bounds__(kThreads) void decode_reduce_balanced_wide_kernel(DecodeParams a) {
  constexpr int SUBS = kThreads / D;
  __shared__ float s_max[kWavesPerWG];
  __shared__ float s_num[SUBS][D];
  __shared__ float s_den[SUBS];
  const int row = blockIdx.x;  // s * Hq + query head
  const int s = row / a.Hq;
  const int hq = row - s * a.Hq;
  const int G = a.Hq / a.Hkv;
  const int g = hq / G;
  const int h = hq - g * G;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int L = attended_len(a, s);
  float* orow = a.out + (size_t)row * D;
  if (L <= 0) {
    const float fill = L == 0 ? 0.0f : __builtin_nanf("");
    for (int i = tid; i < D; i += kThreads) orow[i] = fill;
    return;
  }
  const int HG = a.head_group;
  const int NGR = a.Hkv / HG;
  const long long T = (long long)NGR * a.ws_pref[a.S];
  const long long W_eff = balanced_workers(T, HG == 1 ? a.n_units : a.n_wg);
  const int n = (L + kChunk - 1) / kChunk;
  const long long TC = (long long)NGR * a.ws_pref[a.S + 1 + a.S];
  const long long cbase = (long long)NGR * a.ws_pref[a.S + 1 + s] + (long long)(g / HG) * (n + kSegCost) + kSegCost;
  const long long w0 = balanced_wave_of(cbase, TC, W_eff);  // first and last worker of the segment
  const long long w1 = balanced_wave_of(cbase + n - 1, TC, W_eff);
  const int hsub = g % HG;
  if (w0 == w1) return;  // uniform over the workgroup
  const int k = (int)(w1 - w0 + 1);
  auto piece_row = [&](int p) -> size_t {
    const size_t wave_id = HG == 1 ? (size_t)(w0 + p) : (size_t)(w0 + p) * kWavesPerWG + hsub;
    return (wave_id * 2 + (p == 0 ? 1 : 0)) * G + h;
  };

  float M = kNegBig;
  for (int p = tid; p < k; p += kThreads) M = fmaxf(M, a.ws_ml[piece_row(p)].x);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if (lane == 0) s_max[wave] = M;
  __syncthreads();
  M = s_max[0];
#pragma unroll
  for (int w = 1; w < kWavesPerWG; ++w) M = fmaxf(M, s_max[w]);

  const int d = tid % D;
  const int sub = tid / D;
  float num = 0.0f, den = 0.0f;
  int p = sub;
  for (; p + 3 * SUBS < k; p += 4 * SUBS) {  // four pieces in flight
    float2 t[4];
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t r = piece_row(p + i * SUBS);
      t[i] = a.ws_ml[r];
      x[i] = a.ws_acc[r * D + d];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float f = fast_exp2(t[i].x - M);
      den = fmaf(t[i].y, f, den);
      num = fmaf(x[i], f, num);
    }
  }
  for (; p < k; p += SUBS) {
    const size_t r = piece_row(p);
    const float2 t = a.ws_ml[r];
    const float f = fast_exp2(t.x - M);
    den = fmaf(t.y, f, den);
    num = fmaf(a.ws_acc[r * D + d], f, num);
  }
  s_num[sub][d] = num;
  if (d == 0) s_den[sub] = den;
  __syncthreads();
  if (sub != 0) return;
  float tn = 0.0f, td = 0.0f;
#pragma unroll
  for (int i = 0; i < SUBS; ++i) {
    tn += s_num[i][d];
    td += s_den[i];
  }
  orow[d] = tn / td;
}

// ------------------------------------------------------------------ launch

template <int DT, int D, int B, int G>
using CoreFor = typename std::conditional<(DT == 1 && G >= kMfmaMinGroup), MfmaCore<D, B, G>,
                                          ValuCore<DT, D, B, G>>::type;

template <int DT, int D, int B, int G>
hipError_t launch_stage1(const DecodeParams& p, hipStream_t stream) {
  using Core = CoreFor<DT, D, B, G>;
  static_assert(Core::kStageBytes == balanced_stage_bytes(DT, D, G), "the plan's LDS estimate must match the core");
  const dim3 grid(p.grid);
  const dim3 block(kThreads);
  if (p.schedule == kBalanced) {
    const size_t lds = (((size_t)(3 * p.S + 2) + 3) & ~(size_t)3) * sizeof(int) +
                       (size_t)kWavesPerWG * ((size_t)p.queue_bytes + (size_t)p.row_bytes);
    if (p.append && p.fuse_rows)
      hipLaunchKernelGGL((decode_balanced_kernel<Core, true>), grid, block, lds, stream, p);
    else
      hipLaunchKernelGGL((decode_balanced_kernel<Core, false>), grid, block, lds, stream, p);
  } else {
    hipLaunchKernelGGL((decode_partitioned_kernel<Core>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

template <int DT, int D, int B>
hipError_t launch_g(const DecodeParams& p, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_stage1<DT, D, B, 1>(p, stream);
    case 2: return launch_stage1<DT, D, B, 2>(p, stream);
    case 4: return launch_stage1<DT, D, B, 4>(p, stream);
    case 8: return launch_stage1<DT, D, B, 8>(p, stream);
    case 16: return launch_stage1<DT, D, B, 16>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT, int D>
hipError_t launch_b(const DecodeParams& p, int block_size, int group, hipStream_t stream) {
  switch (block_size) {
    case 16: return launch_g<DT, D, 16>(p, group, stream);
    case 32: return launch_g<DT, D, 32>(p, group, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t launch_d(const DecodeParams& p, int head_dim, int block_size, int group, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_b<DT, 64>(p, block_size, group, stream);
    case 128: return launch_b<DT, 128>(p, block_size, group, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_partitions(const DecodeParams& p, int dtype, int head_dim, int block_size, int group,
                                    hipStream_t stream) {
  if (p.S == 0 || p.n_units == 0) return hipSuccess;
  return dtype == 1 ? launch_d<1>(p, head_dim, block_size, group, stream)
                    : launch_d<0>(p, head_dim, block_size, group, stream);
}

template <int D>
hipError_t launch_narrow_merge(const DecodeParams& p, int group, dim3 grid, hipStream_t stream) {
  switch (group) {
    case 1: hipLaunchKernelGGL((decode_reduce_balanced_kernel<D, 1>), grid, dim3(kThreads), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_reduce_balanced_kernel<D, 2>), grid, dim3(kThreads), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((decode_reduce_balanced_kernel<D, 4>), grid, dim3(kThreads), 0, stream, p); break;
    case 8: hipLaunchKernelGGL((decode_reduce_balanced_kernel<D, 8>), grid, dim3(kThreads), 0, stream, p); break;
    case 16: hipLaunchKernelGGL((decode_reduce_balanced_kernel<D, 16>), grid, dim3(kThreads), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_reduce(const DecodeParams& p, int head_dim, int group, hipStream_t stream) {
  if (p.S == 0) return hipSuccess;
  if (p.schedule == kBalanced) {
    // Segments are cut into about W / (S * Hkv) pieces when the lengths are
    // alike; many pieces per segment get four waves per row.
    const bool wide = (long long)p.n_units >= 8LL * p.S * p.Hkv;
    if (wide) {
      const dim3 grid((unsigned)p.S * (unsigned)p.Hq);
      switch (head_dim) {
        case 64: hipLaunchKernelGGL((decode_reduce_balanced_wide_kernel<64>), grid, dim3(kThreads), 0, stream, p); break;
        case 128: hipLaunchKernelGGL((decode_reduce_balanced_wide_kernel<128>), grid, dim3(kThreads), 0, stream, p); break;
        default: return hipErrorInvalidValue;
      }
    } else {
      const dim3 grid((unsigned)(((long long)p.S * p.Hkv + kWavesPerWG - 1) / kWavesPerWG));
      if (head_dim == 64) return launch_narrow_merge<64>(p, group, grid, stream);
      if (head_dim == 128) return launch_narrow_merge<128>(p, group, grid, stream);
      return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (p.NP <= 1) return hipSuccess;
  const dim3 grid((unsigned)p.S * (unsigned)p.Hq);
  switch (head_dim) {
    case 64: hipLaunchKernelGGL((decode_reduce_partitioned_kernel<64>), grid, dim3(kThreads), 0, stream, p); break;
    case 128: hipLaunchKernelGGL((decode_reduce_partitioned_kernel<128>), grid, dim3(kThreads), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
