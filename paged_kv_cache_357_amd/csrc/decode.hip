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
// Work decomposition (one wavefront = 64 lanes):
//   * one workgroup of kWaves waves per (partition, kv head, sequence); a
//     partition is P consecutive logical tokens;
//   * the workgroup stages its slice of the block table and its GQA group of
//     query rows in LDS;
//   * each wave takes 16-token chunks of the partition round robin; a chunk
//     lies inside one physical block, so its base address is a scalar;
//   * a token's K (or V) row of one kv head is D * elt = 256 bytes for both
//     bf16 D=128 and fp32 D=64; LPT lanes cover it with one 16-byte load
//     each, so a wave load instruction reads 64/LPT whole rows, and every
//     lane keeps the same 16-byte column of the row for the whole kernel;
//   * the dot product is finished with DPP adds across the LPT lanes;
//   * each group of LPT lanes keeps its own online-softmax state (running
//     max m, running sum l, accumulator for its columns); groups, then waves,
//     then partitions are merged with the log-sum-exp rule.
// Every reduction order depends only on logical token positions, never on
// which physical block holds a token, so outputs are bitwise independent of
// the block layout and bitwise reproducible.
//
// Masking: tokens at or beyond L inside the last chunk load the row of token
// L-1 (always in bounds and written) and get score -inf, hence weight exactly 0.
// Running maxima start at -1e30 rather than -inf so that a group that has
// seen no token yet rescales by exp2(0) = 1 instead of exp2(-inf + inf) = NaN.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr float kNegBig = -1.0e30f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

// Partial dot product of one lane's 16-byte column of q and of a K row.
template <int DT>
__device__ __forceinline__ float dot16(const uint32_t (&q)[4], const uint4& k) {
  if constexpr (DT == 1) {
    float d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[0]), __builtin_bit_cast(bf16x2, k.x),
                                              0.0f, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[1]), __builtin_bit_cast(bf16x2, k.y), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[2]), __builtin_bit_cast(bf16x2, k.z), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[3]), __builtin_bit_cast(bf16x2, k.w), d, false);
    return d;
  } else {
    float d = __uint_as_float(q[0]) * __uint_as_float(k.x);
    d = fmaf(__uint_as_float(q[1]), __uint_as_float(k.y), d);
    d = fmaf(__uint_as_float(q[2]), __uint_as_float(k.z), d);
    d = fmaf(__uint_as_float(q[3]), __uint_as_float(k.w), d);
    return d;
  }
}

// The EPL values of one lane's 16-byte column of a V row, widened to fp32.
template <int DT>
__device__ __forceinline__ void widen16(const uint4& v, float* f) {
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

template <int DT, int D, int B, int G>
__global__ __launch_bounds__(kWaves * 64) void decode_partition_kernel(DecodeParams a) {
  constexpr int ELT = DT == 1 ? 2 : 4;
  constexpr int EPL = 16 / ELT;         // elements per lane per row
  constexpr int LPT = D / EPL;          // lanes per token row
  constexpr int TPI = 64 / LPT;         // token rows per wave load instruction
  constexpr int NI = kChunk / TPI;      // load instructions per tensor per chunk
  constexpr int ROW = D * ELT;          // bytes of one token row of one kv head
  constexpr int NT = kWaves * 64;
  static_assert(LPT == 8 || LPT == 16 || LPT == 32, "row must span 8, 16 or 32 lanes");
  static_assert(B % kChunk == 0, "block size must be a multiple of the chunk");

  __shared__ int s_tbl[kMaxPartition / kChunk + 1];
  __shared__ uint4 s_q[G * ROW / 16];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ float s_acc[kWaves][G][D];

  const int part = blockIdx.x;
  const int g = blockIdx.y;
  const int s = blockIdx.z;
  const int tid = threadIdx.x;
  const int L = a.lens[s];
  const int tok0 = part * a.P;
  const bool bad_len = (L < 0) || (L > a.max_len);
  const bool direct = (L <= a.P);  // this sequence fits one partition: write out directly

  if (bad_len || tok0 >= L) {
    // Nothing to attend to here.  The partition-0 workgroup owns the output
    // rows of sequences handled directly (L = 0 gives zeros, a bad length NaN);
    // otherwise the merge kernel writes them.
    if (part == 0 && (bad_len || direct)) {
      const float fill = bad_len ? __builtin_nanf("") : 0.0f;
      float* o = a.out + ((size_t)s * a.Hq + (size_t)g * G) * D;
      for (int i = tid; i < G * D; i += NT) o[i] = fill;
    }
    return;
  }

  const int tok_end = min(tok0 + a.P, L);
  const int n_chunks = (tok_end - tok0 + kChunk - 1) / kChunk;
  const int blk0 = tok0 / B;
  const int n_blk = (tok_end - 1) / B - blk0 + 1;

  // Stage the block-table slice and the query group.
  const int32_t* trow = a.tables + (size_t)s * a.MB + blk0;
  int bad_blk = 0;
  for (int i = tid; i < n_blk; i += NT) {
    int b = trow[i];
    const bool ok = (b >= 0) && (b < a.NB);
    bad_blk |= !ok;
    s_tbl[i] = ok ? b : 0;  // never dereference an out-of-range block id
  }
  const uint4* qsrc = reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) +
                                                     ((size_t)s * a.Hq + (size_t)g * G) * ROW);
  for (int i = tid; i < G * ROW / 16; i += NT) s_q[i] = qsrc[i];
  bad_blk = __syncthreads_or(bad_blk);

  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = lane / LPT;
  const int seg = lane % LPT;

  uint32_t qw[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 t = s_q[(h * ROW) / 16 + seg];
    qw[h][0] = t.x; qw[h][1] = t.y; qw[h][2] = t.z; qw[h][3] = t.w;
  }

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;
  }

  const uint32_t row_stride = (uint32_t)a.Hkv * ROW;  // bytes between slots of one head
  const size_t block_stride = (size_t)B * row_stride;
  const char* kbase = static_cast<const char*>(a.k) + (size_t)g * ROW;
  const char* vbase = static_cast<const char*>(a.v) + (size_t)g * ROW;
  const float sl2 = a.scale_log2;

  for (int c = wave; c < n_chunks; c += kWaves) {
    const int cs = tok0 + c * kChunk;                  // first token of the chunk
    const int phys = __builtin_amdgcn_readfirstlane(s_tbl[cs / B - blk0]);
    const size_t cbase = (size_t)phys * block_stride + (size_t)(cs % B) * row_stride;
    const char* kb = kbase + cbase;
    const char* vb = vbase + cbase;
    const int lim = tok_end - 1 - cs;                  // last valid token of the chunk

    uint4 kr[NI], vr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t = min(i * TPI + grp, lim);
      kr[i] = *reinterpret_cast<const uint4*>(kb + (t * row_stride + seg * 16));
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t = min(i * TPI + grp, lim);
      vr[i] = *reinterpret_cast<const uint4*>(vb + (t * row_stride + seg * 16));
    }

    float p[G][NI];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < NI; ++i) p[h][i] = row_sum<LPT>(dot16<DT>(qw[h], kr[i]));

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
      widen16<DT>(vr[i], vf);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p[h][i], vf[e], acc[h][e]);
    }
  }

  // Merge the TPI lane groups of the wave.
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
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wave][h][seg * EPL + e] = acc[h][e];
      if (seg == 0) {
        s_m[wave][h] = m[h];
        s_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();

  // Merge the waves; finish (one partition) or write the partition's partials.
  const size_t row0 = (size_t)s * a.Hq + (size_t)g * G;  // first q-head row of the group
  for (int idx = tid; idx < G * D; idx += NT) {
    const int h = idx / D;
    const int d = idx % D;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(s_m[w][h] - M);
      num = fmaf(s_acc[w][h][d], f, num);
      den = fmaf(s_l[w][h], f, den);
    }
    if (direct) {
      a.out[(row0 + h) * D + d] = bad_blk ? __builtin_nanf("") : num / den;
    } else {
      const size_t r = (row0 + h) * a.NP + part;
      a.ws_acc[r * D + d] = bad_blk ? __builtin_nanf("") : num;
      if (d == 0) a.ws_ml[r] = bad_blk ? make_float2(INFINITY, __builtin_nanf("")) : make_float2(M, den);
    }
  }
}

// Stage 2: merge the partitions of sequences longer than one partition.
// One wave per (q head, sequence); lane j owns columns j, j+64, ...
template <int D>
__global__ __launch_bounds__(64) void decode_reduce_kernel(DecodeParams a) {
  constexpr int PER = D / 64;
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int lane = threadIdx.x;
  const int L = a.lens[s];
  const bool bad_len = (L < 0) || (L > a.max_len);
  if (!bad_len && L <= a.P) return;  // written by stage 1 (or L = 0 zeros)
  float* o = a.out + ((size_t)s * a.Hq + h) * D;
  if (bad_len) {
#pragma unroll
    for (int j = 0; j < PER; ++j) o[lane + 64 * j] = __builtin_nanf("");
    return;
  }
  const int np = (L + a.P - 1) / a.P;
  const size_t r0 = ((size_t)s * a.Hq + h) * a.NP;
  const float2* ml = a.ws_ml + r0;
  const float* acc = a.ws_acc + r0 * D;
  float M = kNegBig;
  for (int p = 0; p < np; ++p) M = fmaxf(M, ml[p].x);
  float den = 0.0f;
  float num[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) num[j] = 0.0f;
  for (int p = 0; p < np; ++p) {
    const float2 t = ml[p];
    const float f = fast_exp2(t.x - M);
    den = fmaf(t.y, f, den);
#pragma unroll
    for (int j = 0; j < PER; ++j) num[j] = fmaf(acc[(size_t)p * D + lane + 64 * j], f, num[j]);
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) o[lane + 64 * j] = num[j] / den;
}

template <int DT, int D, int B>
hipError_t launch_g(const DecodeParams& p, int group, hipStream_t stream) {
  const dim3 grid(p.NP, p.Hkv, p.S);
  const dim3 block(kWaves * 64);
  switch (group) {
    case 1: hipLaunchKernelGGL((decode_partition_kernel<DT, D, B, 1>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_partition_kernel<DT, D, B, 2>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((decode_partition_kernel<DT, D, B, 4>), grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL((decode_partition_kernel<DT, D, B, 8>), grid, block, 0, stream, p); break;
    case 16: hipLaunchKernelGGL((decode_partition_kernel<DT, D, B, 16>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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
  if (p.S == 0) return hipSuccess;
  return dtype == 1 ? launch_d<1>(p, head_dim, block_size, group, stream)
                    : launch_d<0>(p, head_dim, block_size, group, stream);
}

hipError_t launch_decode_reduce(const DecodeParams& p, int head_dim, hipStream_t stream) {
  if (p.S == 0 || p.NP <= 1) return hipSuccess;
  const dim3 grid(p.Hq, p.S);
  switch (head_dim) {
    case 64: hipLaunchKernelGGL((decode_reduce_kernel<64>), grid, dim3(64), 0, stream, p); break;
    case 128: hipLaunchKernelGGL((decode_reduce_kernel<128>), grid, dim3(64), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
