// Prompt (prefill) attention over the paged KV cache for gfx950.
//
// "PagedAttention and vLLM Architecture: Virtual Memory for LLM Serving",
// section 3, item 1: a prompt is processed and its logical blocks are
// assigned physical blocks; section 2: attention reads K and V through the
// block table and applies softmax to the scaled dot products.  Positions
// follow the translation formula of "PagedAttention Paper Breakdown",
// section 2.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "pkv_internal.h"
#include "pkv_ops.h"

namespace pkv {
namespace {

constexpr float kNegBig = -1.0e30f;
constexpr int kThreads = kWavesPerWG * 64;
// Fourth word of a raw buffer resource on gfx9-family parts (gfx950).
constexpr int kBufferConfig = 0x00020000;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ u32x4 make_u32x4(const uint4& t) { return u32x4{t.x, t.y, t.z, t.w}; }

// Two floats rounded to bf16 (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// ------------------------------------------------------------ prompt pass
//
// Causal attention of a chunk of new query tokens over their sequence's
// cache (the chunk's own K and V already written): the token at position p
// attends to positions 0 .. p.  A wave takes 32 query columns, the (token,
// head) pairs of 32 / G consecutive tokens and the G query heads of kv head
// g; a workgroup takes four such waves of one (sequence, kv head).  The
// workgroup streams the sequence's keys from position 0 to its last token's
// position in tiles of 64: all 256 threads load a tile's K and V rows once
// into a double-buffered LDS tile (one barrier per tile), and each wave runs
// 32-key steps of matrix-core math on its columns: scores K q^T
// (v_mfma_f32_32x32x16_bf16), an online softmax per column with the mask
// limit at the column's own position, and O^T += V^T P^T with the weights
// carried as two bf16 parts.  A wave past its own last position only helps
// load.  Workgroup tiles are numbered tile-major, last (longest) tiles first.
//
// Lane layout of v_mfma_f32_32x32x16_bf16 (measured on gfx950 with a
// one-wave probe): lane l holds row l % 32 of the A operand at k = 8 (l / 32)
// + t and column l % 32 of the B operand at the same k, t < 8; result element
// r of lane l is row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.

// Headroom (base 2) a weight may reach before the prompt pass moves its
// softmax reference.
constexpr float kLazy = 8.0f;

// Compute steps of 32 keys staged per LDS tile: the workgroup's four waves
// meet at one barrier per tile.
constexpr int kSubSteps = 2;

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Two waves per SIMD: with that register budget the accumulators stay in
// VGPRs.
template <int D, int B, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kernel(PrefillParams a) {
  static_assert(kPrefillColumns == 32, "a wave takes the 32 columns of one 32x32 product");
  constexpr int ROW = D * 2;            // bytes of one token row of one kv head
  constexpr int LPR = ROW / 16;         // 16-byte pieces per row
  constexpr int KS = D / 16;            // score products per step (16 of d each)
  constexpr int DB = D / 32;            // output blocks of 32 columns of d
  constexpr int WT = 32 / G;            // tokens per wave
  constexpr int STEP = 32;              // keys per compute step
  constexpr int SUB = kSubSteps;        // compute steps per LDS tile (one barrier each tile)
  constexpr int KROW = ROW + 16;        // LDS row strides of K and V (padding against bank conflicts)
  constexpr int VROW = ROW + 64;
  __shared__ __attribute__((aligned(16))) char s_k[2][SUB * STEP * KROW];
  __shared__ __attribute__((aligned(16))) char s_v[2][SUB * STEP * VROW];

  // Tile-major numbering, last (longest) tiles first: workgroups are dealt to
  // the XCDs round robin, so each XCD gets every eighth (sequence, kv head)
  // pair with all its tiles and runs them longest first.  (Numbering the
  // tiles of a pair consecutively would give each XCD one tile index only
  // whenever the tile count is a multiple of eight.)
  const int u = (int)blockIdx.x;
  const int n_sg = a.S * a.Hkv;
  const int wgt = a.n_qt - 1 - u / n_sg;
  const int sg = u - (u / n_sg) * n_sg;
  const int s = sg / a.Hkv;
  const int g = sg - s * a.Hkv;
  const int r0 = a.q_start[s];
  const int n = a.q_start[s + 1] - r0;
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int wg_t0 = wgt * kWavesPerWG * WT;
  if (wg_t0 >= n) return;  // uniform over the workgroup
  const int L = a.lens[s];
  const int col = lane & 31, hl = lane >> 5;  // this lane's query column; which half of the k range it holds
  const int t0 = wg_t0 + wave * WT;
  const int tok = t0 + col / G;               // the column's token and query head g * G + col % G
  const bool ok = tok < n;
  float* orow = a.out + ((size_t)(r0 + tok) * a.Hq + (size_t)g * G + col % G) * D;
  if (L < n || L > a.max_len) {  // lengths that cannot hold the chunk: NaN rows
    if (ok)
      for (int d = hl; d < D; d += 2) orow[d] = __builtin_nanf("");
    return;
  }
  const int p_col = ok ? L - n + tok : -1;                            // last key this column sees
  const int p_wave = t0 < n ? L - n + min(t0 + WT, n) - 1 : -1;       // last key of this wave
  const int p_first = L - n + t0;                                     // last key of the wave's first column
  const int p_wg = L - n + min(wg_t0 + kWavesPerWG * WT, n) - 1;      // last key of the workgroup
  const int n_tiles = p_wg / (SUB * STEP) + 1;
  const int32_t* trow = a.tables + (size_t)s * a.MB;
  const uint32_t rs = (uint32_t)a.Hkv * ROW;
  const char* kbase = static_cast<const char*>(a.k) + (size_t)g * ROW;
  const char* vbase = static_cast<const char*>(a.v) + (size_t)g * ROW;

  // q^T operands: for score product j the lane holds d = 16 j + 8 hl .. + 7
  // of its column.
  // The scores are scaled by sl2 = |scale| log2(e) >= the smallest normal
  // float: a negative scale is moved into q as a sign flip (exact), so the
  // column maximum can be taken over the raw scores and scaled once (rounding
  // is monotone: the same value as the maximum of the scaled scores), each
  // weight is exp2 of one fused multiply-add, and a masked -inf stays -inf.
  const float sl2 = fmaxf(fabsf(a.scale_log2), 1.17549435e-38f);
  bf16x8 q[KS];
  {
    const char* qsrc = static_cast<const char*>(a.q) + ((size_t)(r0 + tok) * a.Hq + (size_t)g * G + col % G) * ROW;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      uint4 v4 = make_uint4(0, 0, 0, 0);
      if (ok) v4 = *reinterpret_cast<const uint4*>(qsrc + 32 * j + 16 * hl);
      if (a.scale_log2 < 0.0f) v4 = make_uint4(v4.x ^ 0x80008000u, v4.y ^ 0x80008000u, v4.z ^ 0x80008000u, v4.w ^ 0x80008000u);
      q[j] = __builtin_bit_cast(bf16x8, make_u32x4(v4));
    }
  }
  f32x16 acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.0f;
  float m_run = kNegBig, l_run = 0.0f;  // l_run: this lane's half of the column's keys

  // Tile loads: wave w moves rows w RPW .. w RPW + RPW - 1 of the tile (K
  // and V), so each wave builds the addresses of one piece of one block.
  // Each load instruction reads RPI whole rows (lane l: row l / LPR + RPI j,
  // 16-byte piece l % LPR): whole 256-byte rows per instruction read faster
  // than 64-byte pieces of 16 rows.  Rows past the last needed key go
  // through zero-size resources (no data moves), so every tile issues the
  // same loads and each wait is exact.
  constexpr int RPW = SUB * STEP / kWavesPerWG;  // rows per wave: 16 / RPW of them share a 16-key chunk
  constexpr int RPI = 64 / LPR;                  // whole rows per load instruction
  static_assert(kChunk % RPW == 0 && RPW % RPI == 0, "a wave's rows lie in one block; whole rows per load");
  constexpr int PPL = RPW / RPI;                 // load instructions per wave and tile (16 bytes a lane each)
  const int lr = lane / LPR, lp = lane % LPR;    // row of the first instruction, 16-byte piece of the row
  int bad = 0;
  // Table entry of this wave's rows, read one tile before their loads are
  // issued: the scalar read then completes under a whole tile of work (the
  // barrier's wait covers it) instead of stalling the issue.
  auto entry = [&](int c) {
    const int cs = c * SUB * STEP + wave * RPW;
    return trow[(cs <= p_wg ? cs : 0) / B];
  };
  int nid = entry(0);
  auto load = [&](int c, u32x4 (&kr)[PPL], u32x4 (&vr)[PPL]) {
    int blk = nid;
    nid = entry(c + 1);
    const int cs = c * SUB * STEP + wave * RPW;
    const bool live = cs <= p_wg;
    const bool inpool = (unsigned)blk < (unsigned)a.NB;  // an id outside the pool is never dereferenced
    bad |= (live && !inpool) ? 1 : 0;                     // its rows become NaN
    blk = inpool ? blk : 0;
    const size_t cbase = ((size_t)blk * B + (size_t)(cs % B)) * rs;
    const int lim = min(RPW - 1, p_wg - cs);  // rows past the last needed key read as zero
    const uint32_t nbytes = live ? (uint32_t)lim * rs + ROW : 0u;
    const __amdgpu_buffer_rsrc_t kres =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbase + cbase), 0, (int)nbytes, kBufferConfig);
    const __amdgpu_buffer_rsrc_t vres =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbase + cbase), 0, (int)nbytes, kBufferConfig);
    const int off = (int)((uint32_t)lr * rs) + lp * 16;  // + RPI rs per instruction
#pragma unroll
    for (int jj = 0; jj < PPL; ++jj) {
      kr[jj] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kres, off + (int)(RPI * jj * rs), 0, 0));
      vr[jj] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vres, off + (int)(RPI * jj * rs), 0, 0));
    }
  };
  // K and V go into LDS as they are laid out in the pool, one row per key,
  // padded so that every operand address is a lane base plus a constant and
  // the operand reads spread over the banks: K rows KROW = ROW + 16 bytes
  // apart put the K operand reads (16 rows at one 16-byte piece) in 16
  // different 16-byte bank slots; V rows VROW = ROW + 32 bytes apart put each
  // lane group's transposing read (four rows at 32 bytes each) in four
  // different 32-byte slots.
  const int krow = wave * RPW + lr;  // row of the tile this lane stores
  auto store = [&](int buf, const u32x4 (&kr)[PPL], const u32x4 (&vr)[PPL]) {
#pragma unroll
    for (int jj = 0; jj < PPL; ++jj) {
      *reinterpret_cast<u32x4*>(s_k[buf] + (krow + RPI * jj) * KROW + lp * 16) = kr[jj];
      *reinterpret_cast<u32x4*>(s_v[buf] + (krow + RPI * jj) * VROW + lp * 16) = vr[jj];
    }
  };
  // V operand of output block db for keys 16 m .. 16 m + 15 of a step by two
  // transposing reads (ds_read_b64_tr_b16): within a group of 16 lanes, lane
  // i receives as element e the 16-bit element i % 4 of the 8 bytes that
  // lane 4 e + i / 4 addresses (measured lane layout on gfx950).  Lane l
  // addresses row 16 m + 8 t + 4 hl + (l % 16) / 4 (read t = 0, 1), columns
  // 32 db + 16 ((l / 16) % 2) + 4 (l % 4) .. + 3, so it receives column
  // 32 db + l % 32 of keys 16 m + 8 t + 4 hl + 0..3: k slot 8 hl + 4 t + e of
  // the product is key 16 m + 8 t + 4 hl + e, the key the lane's weight
  // 8 m + 4 t + e holds.
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const int tr_off = (4 * hl + ((lane & 15) >> 2)) * VROW + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
  auto v_operand = [&](const char* vtile, int db, int m) -> bf16x8 {
    u32x2 h2[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const char* src = vtile + tr_off + (16 * m + 8 * t) * VROW + 64 * db;
      h2[t] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)src));
    }
    return __builtin_bit_cast(bf16x8, u32x4{h2[0][0], h2[0][1], h2[1][0], h2[1][1]});
  };

  // One 32-key step for this wave's 32 columns.  Lane l ends the score
  // products holding keys 8 (r / 4) + 4 hl + r % 4, r < 16, of its column;
  // lanes l and l ^ 32 hold the column's 32 keys between them.
  auto compute = [&](int c, int buf, int sub) {
    const int cs = c * STEP;
    const char* ktile = s_k[buf] + sub * (STEP * KROW);
    const char* vtile = s_v[buf] + sub * (STEP * VROW);
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.0f;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const bf16x8 kop =
          __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ktile + col * KROW + 32 * j + 16 * hl));
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, q[j], sc, 0, 0, 0);
    }

    // Online softmax with a lazily moved reference: the running reference
    // m_run follows the column's maximum only when the maximum exceeds it by
    // more than kLazy (base 2), so weights stay below 2^kLazy and the
    // accumulator is rescaled rarely.  Any reference gives the same softmax;
    // only rounding depends on it, and it depends on the data alone, so
    // results stay deterministic.  The causal mask is applied only on steps
    // that reach past the wave's first column's last key (columns past the
    // chunk's end are never written, so they need no mask).
    float x[16], mx;
    auto scores_to_exponents = [&](auto masked) {
      const int lim = p_col - cs;
      mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * hl + (r & 3);
        const float v = sc[r];
        x[r] = (!decltype(masked)::value || key <= lim) ? v : -INFINITY;
        mx = fmaxf(mx, x[r]);
      }
    };
    if (cs + STEP - 1 > p_first) scores_to_exponents(std::true_type{});
    else scores_to_exponents(std::false_type{});
    {
      // the column's other 16 keys sit in lane l ^ 32 (v_permlane32_swap with
      // both operands x leaves a lane its own x in one result and its xor-32
      // partner's in the other; the maximum is exact)
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * sl2;
    }
    const bool move = mx > m_run + kLazy;
    if (__any(move)) {  // rare
      const float mn = move ? mx : m_run;
      const float alpha = fast_exp2(m_run - mn);
      m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b) acc[b] *= alpha;
    }
    float pw[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) pw[r] = fast_exp2(fmaf(x[r], sl2, -m_run));
    l_run += (((pw[0] + pw[1]) + (pw[2] + pw[3])) + ((pw[4] + pw[5]) + (pw[6] + pw[7]))) +
             (((pw[8] + pw[9]) + (pw[10] + pw[11])) + ((pw[12] + pw[13]) + (pw[14] + pw[15])));
    // P^T operands of the two 16-key products, high (truncated) and low
    // (rounded rest) bf16 parts: product m takes the lane's weights 8 m .. 8 m + 7.
    bf16x8 phi[2], plo[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      uint32_t hb[8];
      float res[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        hb[i] = __float_as_uint(pw[8 * m + i]) & 0xffff0000u;
        res[i] = pw[8 * m + i] - __uint_as_float(hb[i]);
      }
      phi[m] = __builtin_bit_cast(
          bf16x8, u32x4{(hb[0] >> 16) | hb[1], (hb[2] >> 16) | hb[3], (hb[4] >> 16) | hb[5], (hb[6] >> 16) | hb[7]});
      plo[m] = __builtin_bit_cast(
          bf16x8, u32x4{pack_bf16_rne(res[0], res[1]), pack_bf16_rne(res[2], res[3]), pack_bf16_rne(res[4], res[5]),
                        pack_bf16_rne(res[6], res[7])});
    }
#pragma unroll
    for (int b = 0; b < DB; ++b) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const bf16x8 vt = v_operand(vtile, b, m);
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt, phi[m], acc[b], 0, 0, 0);
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt, plo[m], acc[b], 0, 0, 0);
      }
    }
  };

  // Tile loop: the next tile (SUB compute steps of K and V) is loaded into
  // registers while tile c is computed from one LDS buffer, then stored into
  // the other; one barrier per tile.  (Deeper prefetch measured no faster:
  // the pass is bound by the wave's own instruction chain, not by load
  // latency.)
  u32x4 kr[PPL], vr[PPL];
  load(0, kr, vr);
  store(0, kr, vr);
  __syncthreads();
  for (int c = 0; c < n_tiles; ++c) {
    if (c + 1 < n_tiles) load(c + 1, kr, vr);
#pragma unroll
    for (int sub = 0; sub < SUB; ++sub) {
      const int cstep = c * SUB + sub;
      if (cstep * STEP <= p_wave) compute(cstep, c & 1, sub);
    }
    if (c + 1 < n_tiles) store((c + 1) & 1, kr, vr);
    __syncthreads();
  }
  bad = __syncthreads_or(bad);

  // Lane l holds output columns 32 db + 8 (r / 4) + 4 hl + r % 4 of its row;
  // lanes l and l ^ 32 share the running reference, their sums add.
  const float lt = l_run + __shfl_xor(l_run, 32);
  if (!ok) return;
  const float nan = __builtin_nanf("");
#pragma unroll
  for (int b = 0; b < DB; ++b) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 v = make_float4(acc[b][4 * q4] / lt, acc[b][4 * q4 + 1] / lt, acc[b][4 * q4 + 2] / lt,
                                   acc[b][4 * q4 + 3] / lt);
      *reinterpret_cast<float4*>(orow + 32 * b + 8 * q4 + 4 * hl) = bad ? make_float4(nan, nan, nan, nan) : v;
    }
  }
}

}  // namespace

template <int D, int B>
hipError_t launch_prefill_g(const PrefillParams& p, int group, hipStream_t stream) {
  const dim3 grid((unsigned)p.n_units);  // one workgroup per (sequence, kv head, tile of four wave tiles)
  switch (group) {
    case 1: hipLaunchKernelGGL((prefill_kernel<D, B, 1>), grid, dim3(kThreads), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<D, B, 2>), grid, dim3(kThreads), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<D, B, 4>), grid, dim3(kThreads), 0, stream, p); break;
    case 8: hipLaunchKernelGGL((prefill_kernel<D, B, 8>), grid, dim3(kThreads), 0, stream, p); break;
    case 16: hipLaunchKernelGGL((prefill_kernel<D, B, 16>), grid, dim3(kThreads), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams& p, int head_dim, int block_size, int group, hipStream_t stream) {
  if (p.n_units == 0) return hipSuccess;
  if (head_dim == 128) {
    return block_size == 16 ? launch_prefill_g<128, 16>(p, group, stream) : launch_prefill_g<128, 32>(p, group, stream);
  }
  return block_size == 16 ? launch_prefill_g<64, 16>(p, group, stream) : launch_prefill_g<64, 32>(p, group, stream);
}

}  // namespace pkv
