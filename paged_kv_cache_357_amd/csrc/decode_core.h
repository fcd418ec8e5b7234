// Building blocks of the decode kernels for gfx950, shared by the kernels of
// decode.hip and decode_shared.hip: buffer-resource loads, DPP and lane
// helpers, the two compute cores that consume a 16-token chunk (ValuCore on
// the vector ALUs, MfmaCore on the matrix cores) and the share arithmetic of
// the balanced schedule.  Everything here lives in an anonymous namespace:
// each translation unit that includes it gets its own copy.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "pkv_internal.h"

#ifndef PKV_NT_LOADS
#define PKV_NT_LOADS 1
#endif

namespace pkv {
namespace {

constexpr float kNegBig = -1.0e30f;
// Balanced schedule: the cost, in chunks, charged for starting a segment
// (query rows, table entries, piece epilogue) when the shares are cut.
// Measured: 2 evens out shares that start many short segments (lognormal
// GQA batch +3%), and changes nothing measurable elsewhere.
constexpr int kSegCost = 2;
constexpr int kThreads = kWavesPerWG * 64;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Cache-policy operand of the K / V buffer loads: bit 1 is the nontemporal
// hint (the rows are streamed once per call).
constexpr int kStreamPolicy = PKV_NT_LOADS ? 2 : 0;
// Fourth word of a raw buffer resource on gfx9-family parts (gfx950).
constexpr int kBufferConfig = 0x00020000;

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Tokens sequence s attends to, or -1 for a length the launch cannot cover
// (its rows become NaN).  With the fused append the stored length is the one
// before the append: position L receives the new token and L + 1 tokens are
// attended, so L + 1 must not exceed max_len.
__device__ __forceinline__ int attended_len(const DecodeParams& a, int s) {
  const int L = a.lens[s];
  if (a.append) return (L >= 0 && L < a.max_len) ? L + 1 : -1;
  return (L >= 0 && L <= a.max_len) ? L : -1;
}

// Fused append of one (sequence s, kv head g) row, as the partitioned
// schedule does it: the new K and V rows go to position p, slot
// T[p / B] * B + p % B of the pool ("PagedAttention Paper Breakdown", section
// 2, Address Translation Formula; K and V share the slot).  The row is spread
// over the wave as dwords (dword w in lane w % 64, register w / 64), so it
// takes one or two registers a lane.  A block id outside [0, NB) writes nothing
// (the table window check already turns the segment's rows into NaN).  The
// unit that writes the row is the one that later streams that row's chunk,
// and a wave's own memory operations on one address take effect in program
// order, so its loads see the new row.  (The balanced schedule loads the
// row ahead through its pipeline instead; see there.)
template <int ROW>
struct NewRow {
  static constexpr int NWORD = ROW / 4;             // dwords of a row
  static constexpr int NW = (NWORD + 63) / 64;      // dwords a lane holds
  uint32_t k[NW], v[NW];
  int blk;
};

template <int ROW>
__device__ __forceinline__ NewRow<ROW> load_new_row(const DecodeParams& a, int B, int s, int g, int p, int lane) {
  NewRow<ROW> r;
  r.blk = a.tables[(size_t)s * a.MB + p / B];
  const uint32_t* kn = reinterpret_cast<const uint32_t*>(static_cast<const char*>(a.k_new) + ((size_t)s * a.Hkv + g) * ROW);
  const uint32_t* vn = reinterpret_cast<const uint32_t*>(static_cast<const char*>(a.v_new) + ((size_t)s * a.Hkv + g) * ROW);
#pragma unroll
  for (int j = 0; j < NewRow<ROW>::NW; ++j) {
    const int w = lane + 64 * j;
    r.k[j] = w < NewRow<ROW>::NWORD ? kn[w] : 0u;
    r.v[j] = w < NewRow<ROW>::NWORD ? vn[w] : 0u;
  }
  return r;
}

// Stores the row's dwords at byte offset `row_off` of both pools.
template <int ROW>
__device__ __forceinline__ void put_new_row(const DecodeParams& a, const NewRow<ROW>& r, size_t row_off, int lane) {
  typedef __attribute__((address_space(1))) uint32_t g_u32;  // global memory
  g_u32* kd = (g_u32*)(static_cast<char*>(const_cast<void*>(a.k)) + row_off);
  g_u32* vd = (g_u32*)(static_cast<char*>(const_cast<void*>(a.v)) + row_off);
#pragma unroll
  for (int j = 0; j < NewRow<ROW>::NW; ++j) {
    const int w = lane + 64 * j;
    if (w < NewRow<ROW>::NWORD) {
      kd[w] = r.k[j];
      vd[w] = r.v[j];
    }
  }
}

template <int ROW>
__device__ __forceinline__ void store_new_row(const DecodeParams& a, int B, const NewRow<ROW>& r, int g, int p,
                                              int lane) {
  if (r.blk < 0 || r.blk >= a.NB) return;
  put_new_row<ROW>(a, r, (((size_t)r.blk * B + (size_t)(p % B)) * a.Hkv + g) * ROW, lane);
}

// What a balanced-schedule pipeline slot loads beside its chunk: the table
// entry of the chunk issued into the slot next, and, with the fused append,
// the new row of a segment that begins there (see the balanced kernel).
template <int ROW>
struct AppendSlot {
  int nid;            // table entry of the next chunk issued into this slot
  NewRow<ROW> row;    // fused append: the new K / V row and the table entry of its block
  long long off;      // fused append: byte offset of the row inside its block, or -1: none
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reinterpret one 32-bit word as two bf16.  The word is taken by value: a
// bit cast applied directly to an element of an ext_vector_type value (k.y)
// has been seen to read element 0 instead, so vector elements always go
// through this copy.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

__device__ __forceinline__ u32x4 make_u32x4(const uint4& t) { return u32x4{t.x, t.y, t.z, t.w}; }
__device__ __forceinline__ u32x2 make_u32x2(uint32_t x, uint32_t y) { return u32x2{x, y}; }

// Two floats rounded to bf16 (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the LPT consecutive lanes that hold one token row; every lane of
// the group ends with the same (bitwise) total.
template <int LPT>
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  x += dpp<0x141>(x);  // row_half_mirror: the other quad of the 8-lane half
  if constexpr (LPT >= 16) x += dpp<0x140>(x);  // row_mirror: the other half of the 16-lane row
  if constexpr (LPT >= 32) x += __shfl_xor(x, 16);
  return x;
}

// Logical workgroup index of launched workgroup b, or -1 for the surplus.
// Launched workgroup b runs on XCD b % xcds.  Logical workgroups are taken in
// groups of `group` consecutive ids; group k runs on XCD k % xcds, its
// members one after the other.
__device__ __forceinline__ int logical_workgroup(int b, int group, int n_wg, int xcds) {
  if (group <= 0) return b < n_wg ? b : -1;
  const int x = b % xcds;
  const int j = b / xcds;
  const int l = (j / group) * (xcds * group) + x * group + (j % group);
  return l < n_wg ? l : -1;
}

// Physical block ids of logical blocks base .. base+63 of a sequence, one
// per lane (0 past its last block), for the partitioned schedule.  An id
// outside [0, NB) is replaced by 0 so it is never dereferenced, and reported
// through *bad.
__device__ __forceinline__ int load_table_window(const int32_t* trow, int base, int n_blk, int lane, int NB,
                                                 bool* bad) {
  int b = 0;
  if (base + lane < n_blk) b = trow[base + lane];
  const bool ok = (b >= 0) && (b < NB);
  if (__any(!ok)) *bad = true;
  return ok ? b : 0;
}

// Where the output of a finished piece goes.  Direct: the G rows of out
// starting at `out` (D floats apart).  Partial: G accumulator rows starting at
// `acc` (acc_stride rows apart) and their (max, sum) pairs at `ml`
// (ml_stride apart).
struct PieceSink {
  bool direct;
  bool bad;
  float* out;
  float* acc;
  size_t acc_stride;
  float2* ml;
  size_t ml_stride;
};

// --------------------------------------------------------------- ValuCore

template <int DT, int D, int B, int G>
struct ValuCore {
  static constexpr int ELT = DT == 1 ? 2 : 4;
  static constexpr int EPL = 16 / ELT;      // elements per lane per row
  static constexpr int LPT = D / EPL;       // lanes per token row
  static constexpr int TPI = 64 / LPT;      // token rows per wave load instruction
  static constexpr int NI = kChunk / TPI;   // load instructions per tensor per chunk
  static constexpr int ROW = D * ELT;       // bytes of one token row of one kv head
  static constexpr int kBlock = B;
  static constexpr int kHeadDim = D;
  static constexpr int kGroup = G;
  static constexpr int kWavesPerSimd = balanced_waves_per_simd(DT, D, G);
  static constexpr int kPipeline = balanced_pipeline_depth(DT, D, G);
  static_assert(LPT == 8 || LPT == 16 || LPT == 32, "row must span 8, 16 or 32 lanes");
  static_assert(B % kChunk == 0, "block size must be a multiple of the chunk");

  // One chunk in flight: its K and V columns and, when the chunk opens a
  // segment, that segment's query columns.
  struct Buf {
    u32x4 k[NI], v[NI];
    uint32_t q[G][4];
    AppendSlot<ROW> app;  // balanced schedule: table entry ahead, fused append
  };

  int grp, seg;
  uint32_t q[G][4];
  float m[G], l[G], acc[G][EPL];

  static constexpr int kStageBytes = 16;  // no LDS tile

  __device__ void init(int lane, uint32_t /*rs*/, char* /*stage_tile*/) {
    grp = lane / LPT;
    seg = lane % LPT;
  }

  __device__ void reset() {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = kNegBig;
      l[h] = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;
    }
  }

  // Query rows of heads g*G .. g*G+G-1 of sequence s: this lane's column.
  __device__ void fetch_q(const DecodeParams& a, int s, int g, uint32_t (&dst)[G][4]) const {
    const char* qsrc = static_cast<const char*>(a.q) + ((size_t)s * a.Hq + (size_t)g * G) * ROW + seg * 16;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint4 t = *reinterpret_cast<const uint4*>(qsrc + h * ROW);
      dst[h][0] = t.x; dst[h][1] = t.y; dst[h][2] = t.z; dst[h][3] = t.w;
    }
  }
  __device__ void load_q(const DecodeParams& a, int s, int g) { fetch_q(a, s, g, q); }
  __device__ void fetch_q(const DecodeParams& a, int s, int g, Buf& b) const { fetch_q(a, s, g, b.q); }

  __device__ void take_q(const Buf& b) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) q[h][i] = b.q[h][i];
  }

  // Fused append: replace row lim of a loaded chunk (the slot of the new
  // token, loaded before the new row is written) by the new K and V rows
  // kept in LDS.  Row lim is row lim % TPI of load lim / TPI.
  __device__ void substitute(int lim, Buf& b, const char* krow, const char* vrow) const {
    const u32x4 nk = *reinterpret_cast<const u32x4*>(krow + seg * 16);
    const u32x4 nv = *reinterpret_cast<const u32x4*>(vrow + seg * 16);
    const bool mine = grp == lim % TPI;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (mine && i == lim / TPI) {
        b.k[i] = nk;
        b.v[i] = nv;
      }
    }
  }

  // Loads of one chunk: kc / vc point at the chunk's first row of this kv
  // head; the buffer resources cover `nbytes` from there (rows 0 .. lim, or
  // nothing for a load-free dummy), so rows past the end read as zero.
  __device__ void issue(const char* kc, const char* vc, uint32_t rs, uint32_t nbytes, Buf& b) const {
    const __amdgpu_buffer_rsrc_t kres =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kc), 0, (int)nbytes, kBufferConfig);
    const __amdgpu_buffer_rsrc_t vres =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vc), 0, (int)nbytes, kBufferConfig);
    const uint32_t off = (uint32_t)grp * rs + (uint32_t)seg * 16;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      b.k[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kres, (int)(off + (uint32_t)(i * TPI) * rs),
                                                                               0, kStreamPolicy));
#pragma unroll
    for (int i = 0; i < NI; ++i)
      b.v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vres, (int)(off + (uint32_t)(i * TPI) * rs),
                                                                               0, kStreamPolicy));
  }

  // Partial dot product of this lane's 16-byte column of q and of a K row.
  __device__ float dot16(const uint32_t (&qh)[4], const u32x4& k) const {
    if constexpr (DT == 1) {
      const uint32_t k0 = k.x, k1 = k.y, k2 = k.z, k3 = k.w;
      float d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qh[0]), as_bf16x2(k0), 0.0f, false);
      d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qh[1]), as_bf16x2(k1), d, false);
      d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qh[2]), as_bf16x2(k2), d, false);
      d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qh[3]), as_bf16x2(k3), d, false);
      return d;
    } else {
      float d = __uint_as_float(qh[0]) * __uint_as_float(k.x);
      d = fmaf(__uint_as_float(qh[1]), __uint_as_float(k.y), d);
      d = fmaf(__uint_as_float(qh[2]), __uint_as_float(k.z), d);
      d = fmaf(__uint_as_float(qh[3]), __uint_as_float(k.w), d);
      return d;
    }
  }

  // The EPL values of this lane's 16-byte column of a V row, widened to fp32.
  __device__ void widen16(const u32x4& v, float* f) const {
    if constexpr (DT == 1) {
      f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
      f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
      f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
      f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
    } else {
      f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
      f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    }
  }

  // Scores, online softmax and V accumulation of one chunk (rows 0 .. lim valid).
  __device__ void consume(int lim, float sl2, const Buf& b) {
    float p[G][NI];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < NI; ++i) p[h][i] = row_sum<LPT>(dot16(q[h], b.k[i]));

#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = m[h];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const float x = (i * TPI + grp <= lim) ? p[h][i] * sl2 : -INFINITY;
        p[h][i] = x;
        mx = fmaxf(mx, x);
      }
      const float alpha = fast_exp2(m[h] - mx);
      m[h] = mx;
      float ps = 0.0f;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        p[h][i] = fast_exp2(p[h][i] - mx);
        ps += p[h][i];
      }
      l[h] = fmaf(l[h], alpha, ps);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
    }

#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float vf[EPL];
      widen16(b.v[i], vf);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p[h][i], vf[e], acc[h][e]);
    }
  }

  // Merge the TPI lane groups, then write the piece.  Lane group 0 holds the
  // merged columns seg * EPL .. seg * EPL + EPL - 1.
  __device__ void finish(const PieceSink& o) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float M = m[h];
#pragma unroll
      for (int off = LPT; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
      const float w = fast_exp2(m[h] - M);
      float lw = l[h] * w;
#pragma unroll
      for (int off = LPT; off < 64; off <<= 1) lw += __shfl_xor(lw, off);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float aw = acc[h][e] * w;
#pragma unroll
        for (int off = LPT; off < 64; off <<= 1) aw += __shfl_xor(aw, off);
        acc[h][e] = aw;
      }
      m[h] = M;
      l[h] = lw;
    }
    if (grp != 0) return;
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (o.direct) {
        float4* dst = reinterpret_cast<float4*>(o.out + h * D + seg * EPL);
#pragma unroll
        for (int e = 0; e < EPL; e += 4)
          dst[e / 4] = o.bad ? make_float4(nan, nan, nan, nan)
                             : make_float4(acc[h][e] / l[h], acc[h][e + 1] / l[h], acc[h][e + 2] / l[h],
                                           acc[h][e + 3] / l[h]);
      } else {
        float4* dst = reinterpret_cast<float4*>(o.acc + h * o.acc_stride * D + seg * EPL);
#pragma unroll
        for (int e = 0; e < EPL; e += 4)
          dst[e / 4] = make_float4(acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]);
        if (seg == 0) o.ml[h * o.ml_stride] = o.bad ? make_float2(INFINITY, nan) : make_float2(m[h], l[h]);
      }
    }
  }
};

// --------------------------------------------------------------- MfmaCore
//
// The 16 token slots of a chunk are the rows of two small matrix products,
// computed with MFMA instructions (64 lanes, 16x16 tiles; lane l has lane
// group gl = l / 16 and column cl = l % 16):
//   scores  S[t][h] = sum_d K[t][d] q[h][d]          v_mfma_f32_16x16x32_bf16
//           A = K (row t = cl; its k values are the 16-byte column
//           gl + 4j of token t's row in step j), B = q^T (column h = cl,
//           query head h of the group, zero for h >= G).  The result puts
//           slots 4 gl + r (r = 0..3) of head cl in lane l.
//   output  O^T[d][h] += sum_t V[t][d] P[h][t]       v_mfma_f32_16x16x16_bf16
//           A = V^T (row cl is column CW cl + dt of the row, tile dt; its four
//           k values are token slots 4 gl + r), B = P^T, which is exactly
//           the layout the score product left in the registers.
// Both operands of a product assign the contraction index through the same
// lane-to-k rule, so every d (and every token slot) is paired with itself.
// The softmax weights P are fp32; they enter the bf16 product split into a
// high part (the top 16 bits) and a low part (the rest, rounded to bf16), so
// the weight carried into the fp32 accumulation is within 2^-16 of P.  V and
// K are bf16 inputs and enter exactly.
//
// Each lane keeps the online-softmax state of its head cl over its own four
// token slots; the running maximum is shared by the four lane groups (one
// cross-group max per chunk), so the matrix product adds their terms
// directly.  The accumulator is rescaled only when some running maximum grew
// (a factor of exactly 1 is skipped, which changes nothing).
//
// K and V rows are fetched with buffer loads whose resource covers only the
// chunk's valid rows: rows past the piece's end read as zero and take no
// memory traffic; their scores are masked to -inf.

template <int D, int B, int G>
struct MfmaCore {
  static constexpr int ROW = D * 2;        // bytes of one token row of one kv head
  static constexpr int KSTEPS = D / 32;    // score products per chunk
  static constexpr int CW = D / 16;        // bf16 of a V row per lane (8 or 4) = output tiles
  static constexpr int kBlock = B;
  static constexpr int kHeadDim = D;
  static constexpr int kGroup = G;
  static constexpr int kWavesPerSimd = balanced_waves_per_simd(1, D, G);
  static constexpr int kPipeline = balanced_pipeline_depth(1, D, G);
  static_assert(G <= 16, "a group must fit the 16 columns of a tile");
  static_assert(B % kChunk == 0, "block size must be a multiple of the chunk");
  using VRow = typename std::conditional<CW == 8, u32x4, u32x2>::type;
  // K rows are loaded whole (LPR lanes of 16 bytes per row, RPI rows per
  // instruction), staged in a per-wave LDS tile and read back in operand
  // layout.  Tile position of 16-byte column c of row r: c ^ (r mod LPR),
  // so that both the row-wise writes and the operand reads (16 rows at one
  // column) spread over distinct banks.
  static constexpr int LPR = ROW / 16;
  static constexpr int RPI = 64 / LPR;
  static constexpr int NK = kChunk / RPI;
  static constexpr int kStageBytes = kChunk * ROW;

  // One chunk in flight: its K rows, V operands and, when the chunk opens a
  // segment, that segment's q^T operand.
  struct Buf {
    u32x4 k[NK];
    VRow v[4];
    bf16x8 q[KSTEPS];
    AppendSlot<ROW> app;  // balanced schedule: table entry ahead, fused append
  };

  int gl, cl;
  uint32_t kld, voff;
  char* stage;  // this wave's LDS tile
  bf16x8 q[KSTEPS];
  f32x4 acc[CW];
  float m_run, l_run;

  __device__ void init(int lane, uint32_t rs, char* stage_tile) {
    gl = lane >> 4;
    cl = lane & 15;
    kld = (uint32_t)(lane / LPR) * rs + (uint32_t)(lane % LPR) * 16;   // + RPI i rs
    voff = (uint32_t)(4 * gl) * rs + (uint32_t)cl * (2 * CW);        // + r rs
    stage = stage_tile;
  }

  __device__ void reset() {
#pragma unroll
    for (int dt = 0; dt < CW; ++dt) acc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    m_run = kNegBig;
    l_run = 0.0f;
  }

  // q^T operand: column cl is query head g*G + cl of the group.
  __device__ void fetch_q(const DecodeParams& a, int s, int g, bf16x8 (&dst)[KSTEPS]) const {
    const char* qsrc = static_cast<const char*>(a.q) + ((size_t)s * a.Hq + (size_t)g * G + cl) * ROW;
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) {
      uint4 t = make_uint4(0, 0, 0, 0);
      if (cl < G) t = *reinterpret_cast<const uint4*>(qsrc + 16 * (gl + 4 * j));
      dst[j] = __builtin_bit_cast(bf16x8, make_u32x4(t));
    }
  }
  __device__ void load_q(const DecodeParams& a, int s, int g) { fetch_q(a, s, g, q); }
  __device__ void fetch_q(const DecodeParams& a, int s, int g, Buf& b) const { fetch_q(a, s, g, b.q); }

  __device__ void take_q(const Buf& b) {
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) q[j] = b.q[j];
  }

  // Fused append: replace row lim of a loaded chunk by the new K and V rows
  // kept in LDS, in the layouts of the K row loads (row lim is row lim % RPI
  // of K load lim / RPI) and of the V operand (token slot lim is register
  // lim % 4 of lane group lim / 4).
  __device__ void substitute(int lim, Buf& b, const char* krow, const char* vrow) const {
    const int lane = gl * 16 + cl;
    const u32x4 nk = *reinterpret_cast<const u32x4*>(krow + (lane % LPR) * 16);
    const VRow nv = *reinterpret_cast<const VRow*>(vrow + cl * (2 * CW));
    const bool mine_k = lane / LPR == lim % RPI;
#pragma unroll
    for (int i = 0; i < NK; ++i)
      if (mine_k && i == lim / RPI) b.k[i] = nk;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * gl + r == lim) b.v[r] = nv;
  }

  __device__ void issue(const char* kc, const char* vc, uint32_t rs, uint32_t nbytes, Buf& b) const {
    const __amdgpu_buffer_rsrc_t kres =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kc), 0, (int)nbytes, kBufferConfig);
    const __amdgpu_buffer_rsrc_t vres =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vc), 0, (int)nbytes, kBufferConfig);
#pragma unroll
    for (int i = 0; i < NK; ++i)
      b.k[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kres, (int)(kld + (uint32_t)(RPI * i) * rs),
                                                                               0, kStreamPolicy));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (CW == 8)
        b.v[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vres, (int)(voff + r * rs), 0,
                                                                                 kStreamPolicy));
      else
        b.v[r] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(vres, (int)(voff + r * rs), 0,
                                                                                kStreamPolicy));
    }
  }

  // Scores, online softmax and V product of one chunk (rows 0 .. lim valid).
  // col_on false masks this lane's column for the chunk: all its scores are
  // -inf, so its running max, sum and accumulator stay exactly as they were
  // (the chunk belongs to another column's rows).
  __device__ void consume(int lim, float sl2, const Buf& b, bool col_on = true) {
    const int lane = gl * 16 + cl;
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int r = RPI * i + lane / LPR;
      const int c = (lane % LPR) ^ (r % LPR);
      *reinterpret_cast<u32x4*>(stage + r * ROW + c * 16) = b.k[i];
    }
    f32x4 sc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) {
      const int c = (gl + 4 * j) ^ (cl % LPR);
      const u32x4 k = *reinterpret_cast<const u32x4*>(stage + cl * ROW + c * 16);
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k), q[j], sc, 0, 0, 0);
    }

    float x[4];
    float mx = m_run;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = (col_on && 4 * gl + r <= lim) ? sc[r] * sl2 : -INFINITY;
      mx = fmaxf(mx, x[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float alpha = fast_exp2(m_run - mx);
    m_run = mx;
    float p[4];
    float ps = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = fast_exp2(x[r] - mx);
      ps += p[r];
    }
    l_run = fmaf(l_run, alpha, ps);
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < CW; ++dt) acc[dt] *= alpha;
    }

    // P^T operand, high and low bf16 parts.
    uint32_t hb[4];
    float res[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      hb[r] = __float_as_uint(p[r]) & 0xffff0000u;
      res[r] = p[r] - __uint_as_float(hb[r]);
    }
    const s16x4 phi = __builtin_bit_cast(s16x4, make_u32x2((hb[0] >> 16) | hb[1], (hb[2] >> 16) | hb[3]));
    const s16x4 plo =
        __builtin_bit_cast(s16x4, make_u32x2(pack_bf16_rne(res[0], res[1]), pack_bf16_rne(res[2], res[3])));

#pragma unroll
    for (int dt = 0; dt < CW; ++dt) {
      // element dt of token slots 4 gl + 0..3
      const uint32_t w0 = b.v[0][dt / 2], w1 = b.v[1][dt / 2], w2 = b.v[2][dt / 2], w3 = b.v[3][dt / 2];
      uint32_t lo, hi;
      if (dt % 2 == 0) {
        lo = (w0 & 0xffffu) | (w1 << 16);
        hi = (w2 & 0xffffu) | (w3 << 16);
      } else {
        lo = (w0 >> 16) | (w1 & 0xffff0000u);
        hi = (w2 >> 16) | (w3 & 0xffff0000u);
      }
      const s16x4 vt = __builtin_bit_cast(s16x4, make_u32x2(lo, hi));
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, phi, acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, plo, acc[dt], 0, 0, 0);
    }
  }

  // Lane (gl, cl) holds head cl, columns CW * (4 gl + r) + dt: 4 * CW
  // consecutive columns starting at 4 * CW * gl, in the order r * CW + dt.
  // The four lane groups share m_run; their sums add.
  __device__ void finish(const PieceSink& o) {
    float lt = l_run + __shfl_xor(l_run, 16);
    lt += __shfl_xor(lt, 32);
    if (cl >= G) return;
    float v[4 * CW];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int dt = 0; dt < CW; ++dt) v[r * CW + dt] = acc[dt][r];
    const int col0 = 4 * CW * gl;
    const float nan = __builtin_nanf("");
    if (o.direct) {
      float4* dst = reinterpret_cast<float4*>(o.out + cl * D + col0);
#pragma unroll
      for (int e = 0; e < 4 * CW; e += 4)
        dst[e / 4] = o.bad ? make_float4(nan, nan, nan, nan)
                           : make_float4(v[e] / lt, v[e + 1] / lt, v[e + 2] / lt, v[e + 3] / lt);
    } else {
      float4* dst = reinterpret_cast<float4*>(o.acc + cl * o.acc_stride * D + col0);
#pragma unroll
      for (int e = 0; e < 4 * CW; e += 4) dst[e / 4] = make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
      if (gl == 0) o.ml[cl * o.ml_stride] = o.bad ? make_float2(INFINITY, nan) : make_float2(m_run, lt);
    }
  }
};

// ------------------------------------------------- balanced share arithmetic

// Last r in [0, n) with scale * pre[r] <= x, for pre nondecreasing in LDS
// with scale * pre[0] <= x.  Each round the 64 lanes probe evenly spaced
// positions of the interval and a ballot keeps the piece between the last
// probe that holds and the next one, so two rounds cover 4096 entries
// (a one-lane binary search needs one dependent LDS read per halving).
__device__ __forceinline__ int last_at_most(const int* pre, int n, long long scale, long long x, int lane) {
  int ra = 0, rb = n;
  while (rb - ra > 1) {
    const long long span = rb - ra;
    const int pos = ra + (int)((span * lane) >> 6);
    const unsigned long long m = __ballot(scale * pre[pos] <= x);
    const int last = 63 - __builtin_clzll(m | 1ull);
    const int nb = last == 63 ? rb : ra + (int)((span * (last + 1)) >> 6);
    ra = ra + (int)((span * last) >> 6);
    rb = nb;
  }
  return uniform(ra);
}

// Wave whose share contains cost position c.
__device__ __forceinline__ long long balanced_wave_of(long long c, long long T, long long W_eff) {
  return ((c + 1) * W_eff - 1) / T;
}

__device__ __forceinline__ long long balanced_workers(long long T, int W) {
  long long w = T / kBalancedMinChunks;
  if (w > W) w = W;
  return w < 1 ? 1 : w;
}

}  // namespace
}  // namespace pkv
