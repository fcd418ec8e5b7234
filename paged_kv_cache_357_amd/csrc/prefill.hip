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

// Largest x over lanes l, l ^ 16, l ^ 32 and l ^ 48, without an LDS round
// trip: with both operands x, v_permlane16_swap leaves each lane its own x
// in one result and lane l ^ 16's in the other (rows of 16 lanes swap in
// pairs), and v_permlane32_swap does the same for lane l ^ 32 (measured lane
// layout on gfx950).  The maximum is exact, so the result equals the shuffle
// form bit for bit.
__device__ __forceinline__ float max_over_lane_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Two floats rounded to bf16 (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// ------------------------------------------------------------ prompt pass
//
// Causal attention of a chunk of new query tokens over their sequence's
// cache (the chunk's own K and V already written): the token at position p
// attends to positions 0 .. p.  A wave takes a tile of 16 query columns,
// the (token, head) pairs of QT = 16 / G consecutive tokens and the G query
// heads of kv head g; a workgroup takes four consecutive tiles of one
// (sequence, kv head).  The workgroup streams the sequence's 16-token chunks
// from position 0 to its last token's position: all 256 threads load a
// chunk's K and V rows once into a double-buffered LDS tile (one barrier
// per chunk), and each wave runs the decode step's matrix-core math on its
// columns: scores K q^T, an online softmax per column with the mask limit
// at the column's own position, and O^T += V^T P^T with the weights carried
// as two bf16 parts.  A wave past its own last position only helps load.
// Workgroup tiles are numbered tile-major, last (longest) tiles first.

// Headroom (base 2) a weight may reach before the prompt pass moves its
// softmax reference.
constexpr float kLazy = 8.0f;

// Query tiles per wave: each K operand read and each assembled V operand
// feeds NT products, and the NT softmax chains interleave.
constexpr int kTilesPerWave = kPrefillTilesPerWave;

// Compute steps of 32 keys staged per LDS tile: the workgroup's four waves
// meet at one barrier per tile.
constexpr int kSubSteps = 2;

// Two waves per SIMD: with that register budget the accumulators stay in
// VGPRs (left to itself the compiler parks them in AGPRs and pays a copy
// each way around every rescale).
template <int D, int B, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kernel(PrefillParams a) {
  constexpr int ROW = D * 2;            // bytes of one token row of one kv head
  constexpr int LPR = ROW / 16;         // 16-byte pieces per row
  constexpr int KSTEPS = D / 32;
  constexpr int CW = D / 16;            // bf16 per lane of a V row = output tiles
  constexpr int QT = 16 / G;            // tokens per 16-column tile
  constexpr int NT = kTilesPerWave;
  constexpr int WT = NT * QT;           // tokens per wave
  constexpr int STEP = 2 * kChunk;      // keys per compute step: two 16-key halves
  constexpr int SUB = kSubSteps;        // compute steps per LDS tile (one barrier each tile)
  constexpr int KROW = ROW + 16;        // LDS row strides of K and V (padding against bank conflicts)
  constexpr int VROW = ROW + 32;
  static_assert(kThreads >= kChunk * LPR, "one load per thread covers a quarter");
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
  const int cl = lane & 15, gl = lane >> 4;
  const int t0 = wg_t0 + wave * WT;
  const int h = cl % G;                    // this lane's column in tile k: token t0 + k QT + cl / G, head h
  int tk[NT];
  bool ok[NT];
  float* orow[NT];
#pragma unroll
  for (int k = 0; k < NT; ++k) {
    tk[k] = t0 + k * QT + cl / G;
    ok[k] = tk[k] < n;
    orow[k] = a.out + ((size_t)(r0 + tk[k]) * a.Hq + (size_t)g * G + h) * D;
  }
  if (L < n || L > a.max_len) {            // lengths that cannot hold the chunk: NaN rows
#pragma unroll
    for (int k = 0; k < NT; ++k)
      if (ok[k])
        for (int d = gl; d < D; d += 4) orow[k][d] = __builtin_nanf("");
    return;
  }
  int p_col[NT];                                                      // last key each column sees
#pragma unroll
  for (int k = 0; k < NT; ++k) p_col[k] = ok[k] ? L - n + tk[k] : -1;
  const int p_wave = t0 < n ? L - n + min(t0 + WT, n) - 1 : -1;       // last key of this wave
  const int p_first = L - n + t0;                                     // last key of the wave's first column
  const int p_wg = L - n + min(wg_t0 + kWavesPerWG * WT, n) - 1;      // last key of the workgroup
  const int n_tiles = p_wg / (SUB * STEP) + 1;
  const int32_t* trow = a.tables + (size_t)s * a.MB;
  const uint32_t rs = (uint32_t)a.Hkv * ROW;
  const char* kbase = static_cast<const char*>(a.k) + (size_t)g * ROW;
  const char* vbase = static_cast<const char*>(a.v) + (size_t)g * ROW;

  // q^T operands: column cl of tile k is query row r0 + tk[k], head g * G + h.
  bf16x8 q[NT][KSTEPS];
#pragma unroll
  for (int k = 0; k < NT; ++k) {
    const char* qsrc = static_cast<const char*>(a.q) + ((size_t)(r0 + tk[k]) * a.Hq + (size_t)g * G + h) * ROW;
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) {
      uint4 v4 = make_uint4(0, 0, 0, 0);
      if (ok[k]) v4 = *reinterpret_cast<const uint4*>(qsrc + 16 * (gl + 4 * j));
      q[k][j] = __builtin_bit_cast(bf16x8, make_u32x4(v4));
    }
  }
  f32x4 acc[NT][CW];
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int k = 0; k < NT; ++k) {
#pragma unroll
    for (int dt = 0; dt < CW; ++dt) acc[k][dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    m_run[k] = kNegBig;
    l_run[k] = 0.0f;
  }

  // Tile loads: wave w moves rows w RPW .. w RPW + RPW - 1 of the tile (K
  // and V), so each wave builds the addresses of one piece of one block;
  // lane l takes row l / LPW of them and its 16-byte pieces l % LPW + LPW j,
  // j < PPL.  Rows past the last needed key go through zero-size resources
  // (no data moves), so every tile issues the same loads and each wait is
  // exact.
  constexpr int RPW = SUB * STEP / kWavesPerWG;  // rows per wave: 16 / RPW of them share a 16-key chunk
  constexpr int LPW = 64 / RPW;                  // lanes per row
  static_assert(kChunk % RPW == 0 && LPR % LPW == 0, "a wave's rows lie in one block; whole pieces per lane");
  constexpr int PPL = LPR / LPW;
  const int lr = lane / LPW, lp = lane % LPW;
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
    const int off = (int)((uint32_t)lr * rs) + lp * 16;
#pragma unroll
    for (int jj = 0; jj < PPL; ++jj) {
      kr[jj] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kres, off + 16 * LPW * jj, 0, 0));
      vr[jj] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vres, off + 16 * LPW * jj, 0, 0));
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
      *reinterpret_cast<u32x4*>(s_k[buf] + krow * KROW + (lp + LPW * jj) * 16) = kr[jj];
      *reinterpret_cast<u32x4*>(s_v[buf] + krow * VROW + (lp + LPW * jj) * 16) = vr[jj];
    }
  };
  // V operand of output tile dt (columns d = 16 dt + i, i < 16) by two
  // transposing reads (ds_read_b64_tr_b16): within a group of 16 lanes, lane
  // i receives as element j the 16-bit element i % 4 of the 8 bytes that
  // lane 4 j + i / 4 addresses (measured lane layout on gfx950).  Lane
  // 4 j + q of group gl addresses row 4 gl + j (16 + 4 gl + j for the second
  // read), columns 16 dt + 4 q .. + 3, so lane (gl, cl) gets column
  // 16 dt + cl of keys 4 gl + 0..3 and 16 + 4 gl + 0..3: the k slots of its
  // weights.
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const int tr_row = 4 * gl + (cl >> 2);
  const int tr_q = cl & 3;
  auto v_operand = [&](const char* vtile, int dt) -> bf16x8 {
    u32x2 h[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const char* src = vtile + (half * kChunk + tr_row) * VROW + 32 * dt + 8 * tr_q;
      h[half] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)src));
    }
    return __builtin_bit_cast(bf16x8, u32x4{h[0][0], h[0][1], h[1][0], h[1][1]});
  };

  // One 32-key step for this wave's NT tiles of 16 columns.  Lane (gl, cl)
  // ends the score products holding keys 4 gl + r (first half) and
  // 16 + 4 gl + r (second half), r = 0..3, of its column in each tile.  The
  // V product contracts over 32 keys with one 16x16x32 product per output
  // tile; its k index order is the same for both operands (k slot 8 gl + i
  // is key 4 gl + i for i < 4, 16 + 4 gl + i - 4 after), so the lane's eight
  // weights are its B operand as they stand.
  auto compute = [&](int c, int buf, int sub) {
    const int cs = c * STEP;
    const char* ktile = s_k[buf] + sub * (STEP * KROW);
    const char* vtile = s_v[buf] + sub * (STEP * VROW);
    f32x4 sc[NT][2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int k = 0; k < NT; ++k) sc[k][half] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      const int r = half * kChunk + cl;
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j) {
        const bf16x8 kop =
            __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ktile + r * KROW + (gl + 4 * j) * 16));
#pragma unroll
        for (int k = 0; k < NT; ++k) sc[k][half] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, q[k][j], sc[k][half], 0, 0, 0);
      }
    }

    // Online softmax with a lazily moved reference: the running reference
    // m_run follows a column's maximum only when the maximum exceeds it by
    // more than kLazy (base 2), so weights stay below 2^kLazy and the
    // accumulator is rescaled rarely.  Any reference gives the same
    // softmax; only rounding depends on it, and it depends on the data
    // alone, so results stay deterministic.  The causal mask is applied only
    // on steps that reach past the wave's first column's last key (columns
    // past the chunk's end are never written, so they need no mask); one
    // branch covers the rescale of every tile.
    float x[NT][8], mx[NT];
    auto scores_to_exponents = [&](auto masked) {
#pragma unroll
      for (int k = 0; k < NT; ++k) {
        const int lim = p_col[k] - cs;
        mx[k] = kNegBig;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int key = (i < 4 ? 0 : kChunk) + 4 * gl + (i & 3);
          const float v = sc[k][i >> 2][i & 3] * a.scale_log2;
          x[k][i] = (!decltype(masked)::value || key <= lim) ? v : -INFINITY;
          mx[k] = fmaxf(mx[k], x[k][i]);
        }
      }
    };
    if (cs + STEP - 1 > p_first) scores_to_exponents(std::true_type{});
    else scores_to_exponents(std::false_type{});
    bool move[NT];
    bool any_move = false;
#pragma unroll
    for (int k = 0; k < NT; ++k) {
      mx[k] = max_over_lane_groups(mx[k]);
      move[k] = mx[k] > m_run[k] + kLazy;
      any_move = any_move || move[k];
    }
    if (__any(any_move)) {  // rare: a tile whose columns keep their reference is scaled by exactly 1
#pragma unroll
      for (int k = 0; k < NT; ++k) {
        const float mn = move[k] ? mx[k] : m_run[k];
        const float alpha = fast_exp2(m_run[k] - mn);
        m_run[k] = mn;
        l_run[k] *= alpha;
#pragma unroll
        for (int dt = 0; dt < CW; ++dt) acc[k][dt] *= alpha;
      }
    }
    bf16x8 phi[NT], plo[NT];
#pragma unroll
    for (int k = 0; k < NT; ++k) {
      float pw[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pw[i] = fast_exp2(x[k][i] - m_run[k]);
      l_run[k] += ((pw[0] + pw[1]) + (pw[2] + pw[3])) + ((pw[4] + pw[5]) + (pw[6] + pw[7]));
      // P^T operand, high (truncated) and low (rounded rest) bf16 parts.
      uint32_t hb[8];
      float res[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        hb[i] = __float_as_uint(pw[i]) & 0xffff0000u;
        res[i] = pw[i] - __uint_as_float(hb[i]);
      }
      phi[k] = __builtin_bit_cast(
          bf16x8, u32x4{(hb[0] >> 16) | hb[1], (hb[2] >> 16) | hb[3], (hb[4] >> 16) | hb[5], (hb[6] >> 16) | hb[7]});
      plo[k] = __builtin_bit_cast(
          bf16x8, u32x4{pack_bf16_rne(res[0], res[1]), pack_bf16_rne(res[2], res[3]), pack_bf16_rne(res[4], res[5]),
                        pack_bf16_rne(res[6], res[7])});
    }
#pragma unroll
    for (int dt = 0; dt < CW; ++dt) {
      const bf16x8 vt = v_operand(vtile, dt);
#pragma unroll
      for (int k = 0; k < NT; ++k) {
        acc[k][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, phi[k], acc[k][dt], 0, 0, 0);
        acc[k][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, plo[k], acc[k][dt], 0, 0, 0);
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

  // Lane (gl, cl) holds output columns 16 dt + 4 gl + r of its row; the four
  // lane groups share the running reference, their sums add.
  const int col0 = 4 * gl;
  const float nan = __builtin_nanf("");
#pragma unroll
  for (int k = 0; k < NT; ++k) {
    float lt = l_run[k] + __shfl_xor(l_run[k], 16);
    lt += __shfl_xor(lt, 32);
    if (!ok[k]) continue;
#pragma unroll
    for (int dt = 0; dt < CW; ++dt) {
      const f32x4 v4 = acc[k][dt];
      *reinterpret_cast<float4*>(orow[k] + 16 * dt + col0) =
          bad ? make_float4(nan, nan, nan, nan) : make_float4(v4[0] / lt, v4[1] / lt, v4[2] / lt, v4[3] / lt);
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
