// Paged decode attention that reads the blocks neighbouring sequences share
// once for all of them, on the matrix cores (bf16 caches), for gfx950.
//
// Forked sequences (parallel sampling, beam search) alias the physical blocks
// of their common prompt until a write gives one of them a private copy
// ("PagedAttention and vLLM Architecture", section 3, Copy-on-Write for
// Parallel Sampling & Beam Search; "PagedAttention Paper Breakdown", section
// 3, Dynamic Copy-on-Write).  A decode that walks the sequences one by one
// reads every shared block once per sibling.  Here a group of neighbouring
// sequences whose tables agree on a leading run of P tokens (P a multiple of
// 16, at most every member's length) is one unit of work: each chunk of the
// P shared tokens is read once and scored against the query rows of every
// member together, as columns of the score and V products (member k, query
// head h of the kv head: column k * G + h, at most 16 columns), and each
// member's private tail (positions P .. L-1, read through its own table) is
// scored against that member's columns only, the other columns being masked
// for those chunks.  Every column therefore runs one online softmax over
// exactly its own sequence's tokens, in logical order (the prefix, then its
// tail), which is the decode of "PagedAttention and vLLM Architecture",
// section 2, unchanged: only the reads are shared.  Token i of a run is read
// from slot T[i / B] * B + i % B of the run's table ("PagedAttention Paper
// Breakdown", section 2, Address Translation Formula).
//
// Three kernels:
//   prepare: one wave per sequence writes the fused-append row (the new
//     token's K and V at position L) and counts the leading tokens its table
//     has in common with the previous sequence's (whole 16-token chunks, at
//     most the shorter of the two lengths before the append).
//   stage 1: every workgroup forms the groups from those counts (a group
//     starts where a sequence shares nothing with the previous one, and after
//     16 / G members), lays the (group, kv head group) segments end to end
//     and cuts them into shares of equal cost per worker, as the balanced
//     schedule of decode.hip does; a worker streams its chunks through
//     MfmaCore and queues its finished pieces in LDS until its last chunk.
//   merge: one wave per (sequence, kv head) merges the pieces of segments cut
//     between workers with the log-sum-exp rule.
// A table entry outside the pool makes the rows that would read it NaN (all
// members' rows for a shared chunk, one member's for its tail); a length
// outside [0, max_context_len] makes that sequence's rows NaN.  Every
// reduction order depends only on logical positions and the batch's lengths
// and sharing, never on physical block ids, so outputs are bitwise
// reproducible and invariant under relabelling the pool.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "decode_core.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

// Tokens sequence s attends to, or -1 for a length the launch cannot cover
// (with the fused append the stored length is the one before it).
__device__ __forceinline__ int shared_attended_len(const DecodeParams& a, int s) {
  const int L = a.lens[s];
  if (a.append) return (L >= 0 && L < a.max_len) ? L + 1 : -1;
  return (L >= 0 && L <= a.max_len) ? L : -1;
}

// ---------------------------------------------------------------- prepare

// One workgroup per sequence s: the fused-append row, the rows of a sequence
// with nothing to attend to (zeros for L = 0, NaN for a length the launch
// cannot cover; no later stage writes them), and the share with s - 1.  The
// loads come in two dependent rounds: the new rows and both lengths, then
// the slot's table entry and the first 64 entries of both tables.
__global__ __launch_bounds__(kThreads) void shared_prepare_kernel(DecodeParams a, int head_dim) {
  const int s = (int)blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int B = a.block_size;
  constexpr int kRowRegs = 4;  // 16-byte pieces a thread holds: rows up to 16 KiB
  const int n16 = a.row_b / 16;
  const bool held = a.append && n16 <= kRowRegs * kThreads;
  const uint4* __restrict__ kn =
      reinterpret_cast<const uint4*>(static_cast<const char*>(a.k_new) + (size_t)s * a.row_b);
  const uint4* __restrict__ vn =
      reinterpret_cast<const uint4*>(static_cast<const char*>(a.v_new) + (size_t)s * a.row_b);
  // round 1
  uint4 k0 = make_uint4(0, 0, 0, 0), k1 = k0, k2 = k0, k3 = k0, v0 = k0, v1 = k0, v2 = k0, v3 = k0;
  if (held) {
    if (tid < n16) { k0 = kn[tid]; v0 = vn[tid]; }
    if (tid + kThreads < n16) { k1 = kn[tid + kThreads]; v1 = vn[tid + kThreads]; }
    if (tid + 2 * kThreads < n16) { k2 = kn[tid + 2 * kThreads]; v2 = vn[tid + 2 * kThreads]; }
    if (tid + 3 * kThreads < n16) { k3 = kn[tid + 3 * kThreads]; v3 = vn[tid + 3 * kThreads]; }
  }
  const int L = a.lens[s];
  const int La = shared_attended_len(a, s);
  const bool pair = s > 0 && La >= 0 && shared_attended_len(a, s - 1) >= 0;
  // round 2: the slot's block; the tables of s - 1 and s (shared tokens are
  // counted within the tokens both held before this step's append)
  const int m = pair ? min(L, a.lens[s - 1]) : 0;
  const int nb = (m + B - 1) / B;
  const int32_t* t0 = a.tables + (size_t)(s > 0 ? s - 1 : 0) * a.MB;
  const int32_t* t1 = a.tables + (size_t)s * a.MB;
  int e0 = 0, e1 = 0;
  if (tid < 64 && lane < nb) {
    e0 = t0[lane];
    e1 = t1[lane];
  }
  const int blk = (a.append && La > 0) ? a.tables[(size_t)s * a.MB + L / B] : -1;
  if (blk >= 0 && blk < a.NB) {
    // the new token's K and V rows (all kv heads) into slot T[L / B] * B + L % B
    const size_t dst = ((size_t)blk * B + (size_t)(L % B)) * (size_t)a.row_b;
    uint4* __restrict__ kd = reinterpret_cast<uint4*>(static_cast<char*>(const_cast<void*>(a.k)) + dst);
    uint4* __restrict__ vd = reinterpret_cast<uint4*>(static_cast<char*>(const_cast<void*>(a.v)) + dst);
    if (held) {
      if (tid < n16) { kd[tid] = k0; vd[tid] = v0; }
      if (tid + kThreads < n16) { kd[tid + kThreads] = k1; vd[tid + kThreads] = v1; }
      if (tid + 2 * kThreads < n16) { kd[tid + 2 * kThreads] = k2; vd[tid + 2 * kThreads] = v2; }
      if (tid + 3 * kThreads < n16) { kd[tid + 3 * kThreads] = k3; vd[tid + 3 * kThreads] = v3; }
    } else {
      for (int i = tid; i < n16; i += kThreads) {
        const uint4 kv = kn[i];
        const uint4 vv = vn[i];
        kd[i] = kv;
        vd[i] = vv;
      }
    }
  }
  if (La <= 0) {
    const float fill = La == 0 ? 0.0f : __builtin_nanf("");
    float* o = a.out + (size_t)s * a.Hq * head_dim;
    for (int i = tid; i < a.Hq * head_dim; i += kThreads) o[i] = fill;
  }
  if (tid >= 64) return;
  // Leading equal entries: the first difference by a ballot, 64 entries a round.
  int e = nb;
  unsigned long long diff = __ballot(lane < nb && e0 != e1);
  if (diff != 0ull) {
    e = __builtin_ctzll(diff);
  } else {
    for (int b0 = 64; b0 < nb; b0 += 64) {
      const int b = b0 + lane;
      diff = __ballot(b < nb && t0[b] != t1[b]);
      if (diff != 0ull) {
        e = b0 + __builtin_ctzll(diff);
        break;
      }
    }
  }
  if (lane == 0) a.ws_share[s] = pair ? min(e * B, m) & ~(kChunk - 1) : 0;
}

// ------------------------------------------------------------ block scans

// Exclusive prefix sum of v over the workgroup's threads, in thread order;
// *total gets the sum.  Every thread must call it.
__device__ int block_excl_sum(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int run = incl - v, tot = 0;
#pragma unroll
  for (int w = 0; w < kWavesPerWG; ++w) {
    if (w < wave) run += tmp[w];
    tot += tmp[w];
  }
  __syncthreads();
  *total = tot;
  return run;
}

// Two exclusive prefix sums at once (one pair of barriers); tmp holds
// 2 * kWavesPerWG ints.
__device__ int2 block_excl_sum2(int v, int u, int* tmp, int* total_v, int* total_u) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int iv = v, iu = u;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int tv = __shfl_up(iv, off);
    const int tu = __shfl_up(iu, off);
    if (lane >= off) {
      iv += tv;
      iu += tu;
    }
  }
  if (lane == 63) {
    tmp[wave] = iv;
    tmp[kWavesPerWG + wave] = iu;
  }
  __syncthreads();
  int rv = iv - v, ru = iu - u, sv = 0, su = 0;
#pragma unroll
  for (int w = 0; w < kWavesPerWG; ++w) {
    if (w < wave) {
      rv += tmp[w];
      ru += tmp[kWavesPerWG + w];
    }
    sv += tmp[w];
    su += tmp[kWavesPerWG + w];
  }
  __syncthreads();
  *total_v = sv;
  *total_u = su;
  return make_int2(rv, ru);
}

// Largest v among the threads before this one (-1 if none).
__device__ int block_excl_max(int v, int* tmp) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off);
    if (lane >= off) incl = max(incl, t);
  }
  int excl = __shfl_up(incl, 1);
  if (lane == 0) excl = -1;
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kWavesPerWG; ++w)
    if (w < wave) excl = max(excl, tmp[w]);
  __syncthreads();
  return excl;
}

// ---------------------------------------------------------------- stage 1

#ifdef PKV_WAVE_TIMING
// Timing build only (libpagedkv_timing.so): per stage-1 wave, the real-time
// counter (100 MHz) at entry, when its stream starts and when its last piece
// is queued, and (share chunks << 32) | workgroup id.  Waves that get no
// share leave zeros; pkv_wave_timing_read copies the table out and clears it.
constexpr int kTimingWaves = 8192;
__device__ unsigned long long g_wave_times[kTimingWaves][4];
#endif

template <int D, int B, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1)))
void decode_shared_kernel(DecodeParams a) {
  using Core = MfmaCore<D, B, kSharedCols>;
  constexpr int ROW = Core::ROW;
  constexpr int CW = Core::CW;
  constexpr int NM = kSharedCols / G;  // members a group may hold
  extern __shared__ __attribute__((aligned(16))) int smem[];
  __shared__ __attribute__((aligned(16))) char s_stage[kWavesPerWG][Core::kStageBytes];
  __shared__ int s_tmp[2 * kWavesPerWG];

#ifdef PKV_WAVE_TIMING
  const unsigned long long t_entry = __builtin_amdgcn_s_memrealtime();
#endif
  const int S = a.S;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);

  // LDS tables: attended lengths, shares with the previous sequence, group
  // of each sequence, then per group: first member, prefix tokens, chunk and
  // cost prefix sums.
  int* slen = smem;
  int* shv = slen + S;
  int* gidv = shv + S;
  int* gstart = gidv + S;
  int* gP = gstart + S + 1;
  int* gpref = gP + S;
  int* gcost = gpref + S + 1;

  // ---- groups, in parallel over contiguous ranges of sequences
  const int per = (S + kThreads - 1) / kThreads;
  const int s_lo = min(S, tid * per);
  const int s_hi = min(S, s_lo + per);
  // Lengths and shares in one round of loads (global address space: the
  // loads need not wait for the LDS stores in between).
  {
    typedef __attribute__((address_space(1))) const int32_t g_i32;
    g_i32* glens = (g_i32*)a.lens;
    g_i32* gshare = (g_i32*)a.ws_share;
    static_assert(kBalancedMaxSeqs % kThreads == 0, "a thread's range of sequences is at most this long");
#pragma unroll
    for (int i = 0; i < kBalancedMaxSeqs / kThreads; ++i) {
      const int s = s_lo + i;
      if (s < s_hi) {
        const int L = glens[s];
        const int La = a.append ? ((L >= 0 && L < a.max_len) ? L + 1 : -1) : ((L >= 0 && L <= a.max_len) ? L : -1);
        slen[s] = max(La, 0);
        shv[s] = s > 0 ? gshare[s] : 0;
      }
    }
  }
  __syncthreads();
  int last_break = -1;
  for (int s = s_lo; s < s_hi; ++s) {
    // A share never exceeds what both sequences held before the append, so
    // a prefix is only ever read within each member's own tokens.
    const int held = s > 0 ? min(slen[s], slen[s - 1]) - a.append : 0;
    const int sh = max(0, min(shv[s], held)) & ~(kChunk - 1);
    shv[s] = sh;
    if (sh <= 0) last_break = s;
  }
  const int run_in = block_excl_max(last_break, s_tmp);  // start of the run entering this range
  int cnt = 0;
  {
    int rs = run_in;
    for (int s = s_lo; s < s_hi; ++s) {
      if (shv[s] <= 0) rs = s;
      cnt += ((s - rs) % NM) == 0 ? 1 : 0;
    }
  }
  int R = 0;
  const int gbase = block_excl_sum(cnt, s_tmp, &R);
  {
    int rs = run_in, id = gbase - 1;
    for (int s = s_lo; s < s_hi; ++s) {
      if (shv[s] <= 0) rs = s;
      if (((s - rs) % NM) == 0) {
        ++id;
        gstart[id] = s;
      }
      gidv[s] = id;
    }
  }
  const int perR = (R + kThreads - 1) / kThreads;
  const int r_lo = min(R, tid * perR);
  const int r_hi = min(R, r_lo + perR);
  for (int r = r_lo; r < r_hi; ++r) gP[r] = 0x7fffffff;
  if (tid == 0) gstart[R] = S;
  __syncthreads();
  for (int s = s_lo; s < s_hi; ++s) {
    const int r = gidv[s];
    if (gstart[r] != s) atomicMin(&gP[r], shv[s]);  // the prefix all members share
  }
  __syncthreads();
  int n_loc = 0, c_loc = 0;
  for (int r = r_lo; r < r_hi; ++r) {
    const int a0 = gstart[r], a1 = gstart[r + 1];
    const int P = a1 - a0 > 1 ? gP[r] : 0;
    gP[r] = P;
    int n = P / kChunk;
    for (int m = a0; m < a1; ++m) n += (max(slen[m] - P, 0) + kChunk - 1) / kChunk;
    gpref[r] = n;
    n_loc += n;
    c_loc += n > 0 ? n + kSegCost : 0;
  }
  int T_chunks = 0, T_cost = 0;
  const int2 ncb = block_excl_sum2(n_loc, c_loc, s_tmp, &T_chunks, &T_cost);
  int nb = ncb.x, cb = ncb.y;
  for (int r = r_lo; r < r_hi; ++r) {
    const int n = gpref[r];
    gpref[r] = nb;
    gcost[r] = cb;
    nb += n;
    cb += n > 0 ? n + kSegCost : 0;
  }
  if (tid == 0) {
    gpref[R] = T_chunks;
    gcost[R] = T_cost;
  }
  __syncthreads();
  // ---- this worker's share (see the balanced schedule of decode.hip)
  const int Hkv = a.Hkv;
  const int HG = a.head_group;
  const int NGR = Hkv / HG;
  const int Ru = uniform(R);
  const long long T = (long long)NGR * uniform(T_chunks);
  const int ell = logical_workgroup(blockIdx.x, a.xcd_group, a.n_wg, a.xcds);
  if (ell < 0) return;
  const int w = ell * kWavesPerWG + wave;  // this wave's partial-record slots
  const int worker = HG == 1 ? w : ell;
  const int hsub = HG == 1 ? 0 : wave;
  // What the merge reads of this worker: the segment it began and left to
  // later workers (or -1), that segment's first member, columns and last worker.
  auto put_split = [&](int4 v) {
    if (hsub == 0 && lane == 0) reinterpret_cast<int4*>(a.ws_split)[worker] = v;
  };
  if (T == 0) {
    put_split(make_int4(-1, 0, 0, 0));
    return;
  }
  const long long W_eff = balanced_workers(T, HG == 1 ? a.n_units : a.n_wg);
  if (worker >= W_eff) {
    put_split(make_int4(-1, 0, 0, 0));
    return;
  }
  const long long TC = (long long)NGR * uniform(T_cost);
  // Last group r with NGR * pre[r] <= x (pre nondecreasing, pre[0] = 0).
  auto last_group_at = [&](const int* pre, long long x) { return last_at_most(pre, Ru, NGR, x, lane); };
  auto chunk_at = [&](long long x) -> long long {
    if (x >= TC) return T;
    const int r = last_group_at(gcost, x);
    const int n = uniform(gpref[r + 1]) - uniform(gpref[r]);
    const long long rel = x - (long long)NGR * uniform(gcost[r]);
    const long long seg = n + kSegCost;
    const long long g2 = rel / seg;
    const long long rr = rel - g2 * seg;
    const long long j = rr < kSegCost ? 0 : rr - kSegCost;
    return (long long)NGR * uniform(gpref[r]) + g2 * n + j;
  };
  const long long lo = chunk_at((long long)worker * TC / W_eff);
  const long long hi = chunk_at((long long)(worker + 1) * TC / W_eff);

#ifdef PKV_WAVE_TIMING
  const unsigned long long t_start = __builtin_amdgcn_s_memrealtime();
#endif
  // Cursor over the chunks of the (group, head group) segments: chunk j of a
  // segment is the prefix's chunk j for j < P / 16, then the tails of the
  // members in order.  part = -1 in the prefix, else the member index.
  struct Cursor {
    int r, g, j, n, a0, nm, P, part, pos, end;  // end: of the current run (P, or the member's length)
  };
  // member whose table the chunk is read through
  auto row_of = [&](const Cursor& c) { return c.a0 + (c.part < 0 ? 0 : c.part); };
  auto tail_chunks = [&](int m, int P) { return (max(uniform(slen[m]) - P, 0) + kChunk - 1) / kChunk; };
  auto enter = [&](Cursor& c, int r) {
    c.r = r;
    c.a0 = uniform(gstart[r]);
    c.nm = uniform(gstart[r + 1]) - c.a0;
    c.P = uniform(gP[r]);
    c.n = uniform(gpref[r + 1]) - uniform(gpref[r]);
  };
  auto seek = [&](Cursor& c, int j) {
    c.j = j;
    const int np = c.P / kChunk;
    if (j < np) {
      c.part = -1;
      c.pos = j * kChunk;
      c.end = c.P;
      return;
    }
    j -= np;
    int k = 0;
    for (; k < c.nm - 1; ++k) {
      const int t = tail_chunks(c.a0 + k, c.P);
      if (j < t) break;
      j -= t;
    }
    c.part = k;
    c.pos = c.P + j * kChunk;
    c.end = uniform(slen[c.a0 + k]);
  };
  auto advance = [&](Cursor& c) {
    if (++c.j < c.n) {
      c.pos += kChunk;
      if (c.pos >= c.end) {  // the next member whose tail holds tokens
        int k = c.part + 1;
        int e = uniform(slen[c.a0 + k]);
        while (k < c.nm - 1 && e <= c.P) e = uniform(slen[c.a0 + ++k]);
        c.part = k;
        c.pos = c.P;
        c.end = e;
      }
      return;
    }
    if (++c.g < NGR) {
      seek(c, 0);
      return;
    }
    c.g = 0;
    int r = c.r;
    do {
      ++r;
    } while (r < Ru - 1 && uniform(gpref[r + 1]) == uniform(gpref[r]));
    enter(c, r);
    seek(c, 0);
  };
  Cursor ic;
  {
    const int r = last_group_at(gpref, lo);
    enter(ic, r);
    const long long rel = lo - (long long)NGR * uniform(gpref[r]);
    ic.g = (int)(rel / ic.n);
    seek(ic, (int)(rel - (long long)ic.g * ic.n));
  }
  Cursor cc = ic;

  const uint32_t rs = (uint32_t)Hkv * ROW;  // bytes between slots of one head
  const char* kpool = static_cast<const char*>(a.k);
  const char* vpool = static_cast<const char*>(a.v);
  const char* qbase = static_cast<const char*>(a.q);
  Core core;
  core.init(lane, rs, s_stage[wave]);
  const int cl = core.cl;
  const int gl = core.gl;

  // Query operand of a segment: column cl is query head (kv head) * G + cl % G
  // of member cl / G (zero for columns beyond the group's members).
  auto fetch_q = [&](const Cursor& c, typename Core::Buf& b) {
    const int kvh = c.g * HG + hsub;
    const bool on = cl < c.nm * G;
    const int sm = c.a0 + (on ? cl / G : 0);
    const char* qsrc = qbase + ((size_t)sm * a.Hq + (size_t)kvh * G + (size_t)(cl % G)) * ROW;
#pragma unroll
    for (int j = 0; j < Core::KSTEPS; ++j) {
      uint4 t = make_uint4(0, 0, 0, 0);
      if (on) t = *reinterpret_cast<const uint4*>(qsrc + 16 * (gl + 4 * j));
      b.q[j] = __builtin_bit_cast(bf16x8, make_u32x4(t));
    }
  };

  // Software pipeline of depth NB with the table entries read NB issues
  // ahead, exactly as in the balanced kernel of decode.hip.
  constexpr int NB = Core::kPipeline;
  long long to_issue = hi - lo, to_consume = hi - lo;
  typename Core::Buf buf[NB];
  bool bad[NB];
  bool first_issue = true;
  Cursor la = ic;
  long long la_pos = lo;
  auto next_entry = [&](AppendSlot<ROW>& sl) {
    if (la_pos >= hi) return;
    sl.nid = a.tables[(size_t)row_of(la) * a.MB + la.pos / B];
    if (++la_pos < hi) advance(la);
  };
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    buf[k].app.nid = 0;
    next_entry(buf[k].app);
  }

  auto issue_next = [&](typename Core::Buf& b, bool& bbad) {
    const char* kc = kpool;
    const char* vc = vpool;
    uint32_t nbytes = 0;
    bbad = false;
    if (to_issue > 0) {
      if (first_issue || ic.j == 0) fetch_q(ic, b);
      first_issue = false;
      const int id = uniform(b.app.nid);
      const bool ok = id >= 0 && id < a.NB;
      bbad = !ok;
      const size_t cbase =
          ((size_t)(ok ? id : 0) * B + (size_t)(ic.pos % B)) * rs + (size_t)(ic.g * HG + hsub) * ROW;
      kc = kpool + cbase;
      vc = vpool + cbase;
      nbytes = ok ? (uint32_t)min(kChunk - 1, ic.end - 1 - ic.pos) * rs + ROW : 0u;
      next_entry(b.app);
      --to_issue;
      if (to_issue > 0) advance(ic);
    }
    core.issue(kc, vc, rs, nbytes, b);
  };

  // Finished pieces wait in this wave's LDS queue (records of
  // shared_record_bytes(columns, D): the global destination of column 0's
  // row, that of its (max, sum) pair or 0 for a finished row, the column
  // count; the columns' rows; their pairs) and are written out after the
  // wave's last chunk, or when the queue is full.
  char* queue = reinterpret_cast<char*>(smem + ((shared_lds_ints(S) + 3) & ~3)) + (size_t)wave * a.queue_bytes;
  int q_used = 0;
  typedef __attribute__((address_space(1))) float g_f32;
  typedef __attribute__((address_space(1))) f32x4 g_f32x4;
  typedef __attribute__((address_space(1))) u32x2 g_u32x2;
  auto flush = [&]() {
    int off = 0;
    while (off < q_used) {
      const char* rec = queue + off;
      const uint64_t gd = *reinterpret_cast<const uint64_t*>(rec);
      const uint64_t gm = *reinterpret_cast<const uint64_t*>(rec + 8);
      const int ncols = uniform(*reinterpret_cast<const int*>(rec + 16));
      g_f32* dst = (g_f32*)(((uint64_t)(uint32_t)uniform((int)(uint32_t)(gd >> 32)) << 32) |
                            (uint32_t)uniform((int)(uint32_t)gd));
      const bool direct = gm == 0;
      const f32x4* src = reinterpret_cast<const f32x4*>(rec + 32);
      constexpr int V4 = D / 4;  // float4 per row
      for (int i = lane; i < ncols * V4; i += 64) {
        const int c = i / V4;
        const int e = i - c * V4;
        const size_t row = direct ? ((size_t)(c / G) * a.Hq + (size_t)(c % G)) * D : (size_t)c * D;
        *(g_f32x4*)(dst + row + 4 * e) = src[i];
      }
      if (!direct && lane < ncols)
        ((g_u32x2*)gm)[lane] = reinterpret_cast<const u32x2*>(rec + 32 + 4 * ncols * D)[lane];
      off += shared_record_bytes(ncols, D);
    }
    q_used = 0;
  };

  bool started = false;
  bool col_bad = false;
  bool first_consume = true;
  int split = -1;  // the segment this worker began and left to later workers
  const float nan = __builtin_nanf("");
  auto step = [&](typename Core::Buf& cur, bool curbad, typename Core::Buf& nxt, bool& nxtbad) {
    issue_next(nxt, nxtbad);
    if (to_consume <= 0) return;
    if (first_consume || cc.j == 0) {
      core.take_q(cur);
      core.reset();
      started = (cc.j == 0);
      col_bad = false;
      first_consume = false;
    }
    const int lim = min(kChunk - 1, cc.end - 1 - cc.pos);
    const bool seg_end = (cc.j == cc.n - 1);
    const bool col_on = cc.part < 0 ? (cl < cc.nm * G) : (cl / G == cc.part);
    core.consume(lim, a.scale_log2, cur, col_on);
    col_bad = col_bad || (curbad && col_on);
    --to_consume;
    if (seg_end || to_consume == 0) {
      const int ncols = cc.nm * G;
      const int rb = shared_record_bytes(ncols, D);
      if (q_used + rb > a.queue_bytes) flush();
      char* rec = queue + q_used;
      const bool direct = started && seg_end;
      const int kvh = cc.g * HG + hsub;
      if (lane == 0) {
        const size_t r0 = ((size_t)w * 2 + (started ? 1 : 0)) * kSharedCols;
        float* rows = direct ? a.out + ((size_t)cc.a0 * a.Hq + (size_t)kvh * G) * D : a.ws_acc + r0 * D;
        reinterpret_cast<uint64_t*>(rec)[0] = reinterpret_cast<uint64_t>(rows);
        reinterpret_cast<uint64_t*>(rec)[1] = direct ? 0 : reinterpret_cast<uint64_t>(a.ws_ml + r0);
        reinterpret_cast<int*>(rec)[4] = ncols;
      }
      // Lane (gl, cl) holds column cl, elements CW * (4 gl + r) + dt; the
      // four lane groups share the running max and their sums add.
      float lt = core.l_run + __shfl_xor(core.l_run, 16);
      lt += __shfl_xor(lt, 32);
      if (cl < ncols) {
        float v[4 * CW];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int dt = 0; dt < CW; ++dt) v[r * CW + dt] = core.acc[dt][r];
        float4* col = reinterpret_cast<float4*>(rec + 32 + (size_t)cl * D * 4) + CW * gl;
        if (direct) {
#pragma unroll
          for (int e = 0; e < 4 * CW; e += 4)
            col[e / 4] = col_bad ? make_float4(nan, nan, nan, nan)
                                 : make_float4(v[e] / lt, v[e + 1] / lt, v[e + 2] / lt, v[e + 3] / lt);
        } else {
#pragma unroll
          for (int e = 0; e < 4 * CW; e += 4) col[e / 4] = make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
          if (gl == 0)
            reinterpret_cast<float2*>(rec + 32 + 4 * ncols * D)[cl] =
                col_bad ? make_float2(INFINITY, nan) : make_float2(core.m_run, lt);
        }
      }
      q_used += rb;
      if (to_consume == 0 && started && !seg_end) split = cc.r * NGR + cc.g;
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
#ifdef PKV_WAVE_TIMING
  {
    const unsigned long long t_end = __builtin_amdgcn_s_memrealtime();
    if (lane == 0 && w < kTimingWaves) {
      g_wave_times[w][0] = t_entry;
      g_wave_times[w][1] = t_start;
      g_wave_times[w][2] = t_end;
      g_wave_times[w][3] = ((unsigned long long)(hi - lo) << 32) | blockIdx.x;
    }
  }
#endif
  int4 rec = make_int4(-1, 0, 0, 0);
  if (split >= 0) {  // the last piece began cc's segment, which later workers continue
    const long long cbase =
        (long long)NGR * uniform(gcost[cc.r]) + (long long)cc.g * (cc.n + kSegCost) + kSegCost;
    rec = make_int4(split, cc.a0, cc.nm * G, (int)balanced_wave_of(cbase + cc.n - 1, TC, W_eff));
  }
  put_split(rec);
}

// ------------------------------------------------------------------ merge

// Workgroup (w0, y), one wave per row: if worker w0 began a segment (group,
// head group gg) that later workers continued, wave i merges row y * 4 + i of
// the segment's HG * columns rows (kv head gg * HG + row / columns, column
// row % columns) from the pieces of workers w0 .. w1, in worker order, eight
// pieces' loads in flight at a time: with M the largest piece max so far,
// sum(exp2(m_p - M) acc_p) / sum(exp2(m_p - M) l_p).  Stage 1 leaves, per
// worker, the segment id, its first member, its columns and its last worker.
// A segment one worker finished was written by stage 1; the rows of empty
// and invalid sequences by the prepare stage.  A record that does not fit
// the call (no stage 1 before the merge) makes the kernel write nothing
// rather than read out of place.
template <int D, int G>
__global__ __launch_bounds__(kThreads) void decode_reduce_shared_kernel(DecodeParams a) {
  constexpr int CPL = D / 64;  // columns per lane (1 or 2)
  constexpr int KB = 8;        // pieces loaded together
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int w0 = (int)blockIdx.x;
  const int HG = a.head_group;
  const int NGR = a.Hkv / HG;
  const int workers = HG == 1 ? a.n_units : a.n_wg;
  const int4 rec = reinterpret_cast<const int4*>(a.ws_split)[w0];
  const int split = uniform(rec.x);
  if (split < 0) return;
  const int a0 = uniform(rec.y);
  const int ncols = uniform(rec.z);
  const int w1 = uniform(rec.w);
  const int gg = split % NGR;
  if (ncols < 1 || ncols > kSharedCols || a0 < 0 || a0 + (ncols - 1) / G >= a.S || w1 <= w0 || w1 >= workers)
    return;
  const int row = (int)blockIdx.y * kWavesPerWG + wave;
  if (row >= HG * ncols) return;
  const int hsub = row / ncols;
  const int c = row - hsub * ncols;
  const int s = a0 + c / G;
  const int kvh = gg * HG + hsub;
  const int pieces = w1 - w0 + 1;
  auto piece_row = [&](int p) -> size_t {
    const size_t wave_id = HG == 1 ? (size_t)(w0 + p) : (size_t)(w0 + p) * kWavesPerWG + hsub;
    return (wave_id * 2 + (p == 0 ? 1 : 0)) * kSharedCols + (size_t)c;
  };
  float M = kNegBig, den = 0.0f, num[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) num[j] = 0.0f;
  for (int p0 = 0; p0 < pieces; p0 += KB) {
    float2 t[KB];
    float x[KB][CPL];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const bool in = p0 + i < pieces;
      const size_t rr = piece_row(in ? p0 + i : p0);
      t[i] = in ? a.ws_ml[rr] : make_float2(kNegBig, 0.0f);
      if constexpr (CPL == 2) {
        const float2 v = in ? *reinterpret_cast<const float2*>(a.ws_acc + rr * D + lane * CPL) : make_float2(0.0f, 0.0f);
        x[i][0] = v.x;
        x[i][1] = v.y;
      } else {
        x[i][0] = in ? a.ws_acc[rr * D + lane] : 0.0f;
      }
    }
    float Mn = M;
#pragma unroll
    for (int i = 0; i < KB; ++i) Mn = fmaxf(Mn, t[i].x);
    if (p0 > 0) {  // a later batch with a larger max rescales the sums so far
      const float sc = fast_exp2(M - Mn);
      den *= sc;
#pragma unroll
      for (int j = 0; j < CPL; ++j) num[j] *= sc;
    }
    M = Mn;
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      if (p0 + i < pieces) {
        const float f = fast_exp2(t[i].x - M);
        den = fmaf(t[i].y, f, den);
#pragma unroll
        for (int j = 0; j < CPL; ++j) num[j] = fmaf(x[i][j], f, num[j]);
      }
    }
  }
  float* o = a.out + ((size_t)s * a.Hq + (size_t)kvh * G + (size_t)(c % G)) * D + lane * CPL;
  if constexpr (CPL == 2) {
    *reinterpret_cast<float2*>(o) = make_float2(num[0] / den, num[1] / den);
  } else {
    o[0] = num[0] / den;
  }
}

// ------------------------------------------------------------------ launch

template <int D, int B, int G>
hipError_t launch_s1(const DecodeParams& p, hipStream_t stream) {
  static_assert(MfmaCore<D, B, kSharedCols>::kStageBytes == balanced_stage_bytes(1, D, kSharedCols),
                "the plan's LDS estimate must match the core");
  const size_t lds = (size_t)((shared_lds_ints(p.S) + 3) & ~3) * sizeof(int) +
                     (size_t)kWavesPerWG * (size_t)p.queue_bytes;
  hipLaunchKernelGGL((decode_shared_kernel<D, B, G>), dim3(p.grid), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

template <int D, int B>
hipError_t launch_s1_g(const DecodeParams& p, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_s1<D, B, 1>(p, stream);
    case 2: return launch_s1<D, B, 2>(p, stream);
    case 4: return launch_s1<D, B, 4>(p, stream);
    case 8: return launch_s1<D, B, 8>(p, stream);
    case 16: return launch_s1<D, B, 16>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_s1_b(const DecodeParams& p, int block_size, int group, hipStream_t stream) {
  switch (block_size) {
    case 16: return launch_s1_g<D, 16>(p, group, stream);
    case 32: return launch_s1_g<D, 32>(p, group, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_merge_g(const DecodeParams& p, int group, hipStream_t stream) {
  // (worker, slice of four rows of the worker's split segment: HG * 16 rows at most)
  const dim3 grid((unsigned)(p.head_group == 1 ? p.n_units : p.n_wg), (unsigned)(p.head_group * kSharedCols / kWavesPerWG));
  switch (group) {
    case 1: hipLaunchKernelGGL((decode_reduce_shared_kernel<D, 1>), grid, dim3(kThreads), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_reduce_shared_kernel<D, 2>), grid, dim3(kThreads), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((decode_reduce_shared_kernel<D, 4>), grid, dim3(kThreads), 0, stream, p); break;
    case 8: hipLaunchKernelGGL((decode_reduce_shared_kernel<D, 8>), grid, dim3(kThreads), 0, stream, p); break;
    case 16: hipLaunchKernelGGL((decode_reduce_shared_kernel<D, 16>), grid, dim3(kThreads), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_shared_prepare(const DecodeParams& p, int head_dim, hipStream_t stream) {
  if (p.S == 0) return hipSuccess;
  hipLaunchKernelGGL(shared_prepare_kernel, dim3((unsigned)p.S), dim3(kThreads), 0, stream, p, head_dim);
  return hipGetLastError();
}

hipError_t launch_shared_stage1(const DecodeParams& p, int head_dim, int block_size, int group, hipStream_t stream) {
  if (p.S == 0) return hipSuccess;
  switch (head_dim) {
    case 64: return launch_s1_b<64>(p, block_size, group, stream);
    case 128: return launch_s1_b<128>(p, block_size, group, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_shared_merge(const DecodeParams& p, int head_dim, int group, hipStream_t stream) {
  if (p.S == 0) return hipSuccess;
  switch (head_dim) {
    case 64: return launch_merge_g<64>(p, group, stream);
    case 128: return launch_merge_g<128>(p, group, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv

#ifdef PKV_WAVE_TIMING
// Declared in include/pagedkv_timing.h; exported by the timing build only.
extern "C" __attribute__((visibility("default"))) int pkv_wave_timing_read(unsigned long long* host, int n_waves) {
  if (!host || n_waves < 0 || n_waves > pkv::kTimingWaves) return -2;
  const size_t bytes = (size_t)n_waves * 4 * sizeof(unsigned long long);
  if (hipMemcpyFromSymbol(host, HIP_SYMBOL(pkv::g_wave_times), bytes, 0, hipMemcpyDeviceToHost) != hipSuccess) return -6;
  static const unsigned long long zeros[pkv::kTimingWaves][4] = {};
  if (hipMemcpyToSymbol(HIP_SYMBOL(pkv::g_wave_times), zeros, sizeof(zeros), 0, hipMemcpyHostToDevice) != hipSuccess)
    return -6;
  return 0;
}
#endif
