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
// Work decomposition
//   * A decode unit is (sequence s, kv head g, partition p): P consecutive
//     logical tokens of one sequence for one kv head and its GQA group of
//     query heads.  One wavefront (64 lanes) runs one unit from start to end;
//     nothing is shared between the waves of a workgroup, so there is no LDS
//     and no barrier.
//   * Units are numbered ((p * S + s) * Hkv + g); workgroup l holds units
//     4l .. 4l+3.  The hardware deals consecutive workgroup ids round robin
//     over the 8 XCDs; the launch permutes ids so that the workgroups of a
//     few neighbouring sequences (all their heads, one partition) run on the
//     same XCD, one after the other, while successive such groups still
//     alternate over the XCDs.  A token's K rows of all heads are then read
//     through one L2, and sequences forked from one prompt share their
//     prompt blocks in it.
//   * A token's K (or V) row of one kv head is D * elt bytes (256 B for bf16
//     D=128 and fp32 D=64).  LPT lanes cover it with one 16-byte load each, so
//     one wave load instruction reads TPI = 64 / LPT whole rows and every lane
//     keeps the same 16-byte column of the row for the whole unit.
//   * The unit's slice of the block table sits in one VGPR (lane i holds the
//     physical block of the unit's i-th logical block, 64 blocks per window);
//     each 16-token chunk reads its block id with a lane read, so address
//     computation never waits on memory.
//   * K and V rows are fetched with nontemporal loads (they are read once),
//     two chunks deep: the loads of chunk c+1 are in flight while chunk c is
//     being consumed.
//   * Scores: partial dot products of the 16-byte columns, finished with DPP
//     adds across the LPT lanes of a row.  Each group of LPT lanes keeps its
//     own online-softmax state (running max m, running sum l, accumulator of
//     its columns); the groups are merged at the end of the unit with the
//     log-sum-exp rule, and partitions are merged the same way by the second
//     kernel.
// Every reduction order depends only on logical token positions, never on
// which physical block holds a token, so outputs are bitwise independent of
// the block layout and bitwise reproducible.
//
// Masking: tokens at or beyond the unit's end inside its last chunk load the
// row of its last token (always in bounds and written) and get score -inf,
// hence weight exactly 0.  Running maxima start at -1e30 rather than -inf so
// that a group that has seen no token yet rescales by exp2(0) = 1 instead of
// exp2(-inf + inf) = NaN.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pkv_internal.h"

#ifndef PKV_PREFETCH
#define PKV_PREFETCH 1
#endif
#ifndef PKV_NT_LOADS
#define PKV_NT_LOADS 1
#endif

namespace pkv {
namespace {

constexpr float kNegBig = -1.0e30f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// One 16-byte column of a K or V row.  The rows are streamed once per call,
// so they are fetched with the nontemporal hint.
__device__ __forceinline__ u32x4 load_row16(const char* p) {
#if PKV_NT_LOADS
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
  return *reinterpret_cast<const u32x4*>(p);
#endif
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

// Reinterpret one 32-bit word as two bf16.  The word is taken by value: a
// bit cast applied directly to an element of an ext_vector_type value (k.y)
// has been seen to read element 0 instead, so vector elements always go
// through this copy.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

// Partial dot product of one lane's 16-byte column of q and of a K row.
template <int DT>
__device__ __forceinline__ float dot16(const uint32_t (&q)[4], const u32x4& k) {
  if constexpr (DT == 1) {
    const uint32_t k0 = k.x, k1 = k.y, k2 = k.z, k3 = k.w;
    float d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q[0]), as_bf16x2(k0), 0.0f, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q[1]), as_bf16x2(k1), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q[2]), as_bf16x2(k2), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q[3]), as_bf16x2(k3), d, false);
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
__device__ __forceinline__ void widen16(const u32x4& v, float* f) {
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

// Logical workgroup index of launched workgroup b, or -1 for the surplus.
// Launched workgroup b runs on XCD b % 8.  Logical workgroups are taken in
// groups of `group` consecutive ids; group k runs on XCD k % 8, its members
// one after the other.
__device__ __forceinline__ int logical_workgroup(int b, int group, int n_wg) {
  if (group <= 0) return b < n_wg ? b : -1;
  const int x = b % kXcds;
  const int j = b / kXcds;
  const int l = (j / group) * (kXcds * group) + x * group + (j % group);
  return l < n_wg ? l : -1;
}

// Physical block ids of logical blocks base .. base+63 of the unit, one per
// lane (0 past the unit's last block).  An id outside [0, NB) is replaced by 0
// so it is never dereferenced, and reported through *bad.
__device__ __forceinline__ int load_table_window(const int32_t* trow, int base, int n_blk, int lane, int NB,
                                                 bool* bad) {
  int b = 0;
  if (base + lane < n_blk) b = trow[base + lane];
  const bool ok = (b >= 0) && (b < NB);
  if (__any(!ok)) *bad = true;
  return ok ? b : 0;
}

template <int DT, int D, int B, int G>
__global__ __launch_bounds__(kWavesPerWG * 64) void decode_units_kernel(DecodeParams a) {
  constexpr int ELT = DT == 1 ? 2 : 4;
  constexpr int EPL = 16 / ELT;         // elements per lane per row
  constexpr int LPT = D / EPL;          // lanes per token row
  constexpr int TPI = 64 / LPT;         // token rows per wave load instruction
  constexpr int NI = kChunk / TPI;      // load instructions per tensor per chunk
  constexpr int ROW = D * ELT;          // bytes of one token row of one kv head
  static_assert(LPT == 8 || LPT == 16 || LPT == 32, "row must span 8, 16 or 32 lanes");
  static_assert(B % kChunk == 0, "block size must be a multiple of the chunk");

  const int ell = logical_workgroup(blockIdx.x, a.xcd_group, a.n_wg);
  if (ell < 0) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int u = ell * kWavesPerWG + wave;
  if (u >= a.n_units) return;
  const int lane = threadIdx.x & 63;
  const int g = u % a.Hkv;
  const int sp = u / a.Hkv;
  const int s = sp % a.S;
  const int part = sp / a.S;

  const int L = a.lens[s];
  const int tok0 = part * a.P;
  const bool bad_len = (L < 0) || (L > a.max_len);
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

  const int grp = lane / LPT;
  const int seg = lane % LPT;
  const int tok_end = min(tok0 + a.P, L);
  const int n_chunks = (tok_end - tok0 + kChunk - 1) / kChunk;
  const int blk0 = tok0 / B;
  const int n_blk = (tok_end - 1) / B - blk0 + 1;
  const int32_t* trow = a.tables + (size_t)s * a.MB + blk0;

  bool bad_blk = false;
  int wbase = 0;
  int tbl = load_table_window(trow, 0, n_blk, lane, a.NB, &bad_blk);

  uint32_t qw[G][4];
  {
    const char* qsrc = static_cast<const char*>(a.q) + ((size_t)s * a.Hq + (size_t)g * G) * ROW + seg * 16;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint4 t = *reinterpret_cast<const uint4*>(qsrc + h * ROW);
      qw[h][0] = t.x; qw[h][1] = t.y; qw[h][2] = t.z; qw[h][3] = t.w;
    }
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
  const char* kbase = static_cast<const char*>(a.k) + (size_t)g * ROW + seg * 16;
  const char* vbase = static_cast<const char*>(a.v) + (size_t)g * ROW + seg * 16;
  const float sl2 = a.scale_log2;

  // Issue the K and V loads of chunk c.
  auto issue = [&](int c, u32x4 (&kr)[NI], u32x4 (&vr)[NI]) {
    const int cs = tok0 + c * kChunk;
    const int bi = cs / B - blk0;
    if (bi - wbase >= 64) {
      wbase += 64;
      tbl = load_table_window(trow, wbase, n_blk, lane, a.NB, &bad_blk);
    }
    const int phys = __builtin_amdgcn_readlane(tbl, bi - wbase);
    const size_t cbase = ((size_t)phys * B + (size_t)(cs % B)) * row_stride;
    const int lim = tok_end - 1 - cs;  // last valid row of the chunk
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t t = (uint32_t)min(i * TPI + grp, lim);
      kr[i] = load_row16(kbase + cbase + t * row_stride);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t t = (uint32_t)min(i * TPI + grp, lim);
      vr[i] = load_row16(vbase + cbase + t * row_stride);
    }
  };

  // Scores, online softmax and V accumulation of chunk c.
  auto consume = [&](int c, const u32x4 (&kr)[NI], const u32x4 (&vr)[NI]) {
    const int lim = tok_end - 1 - (tok0 + c * kChunk);
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
  };

  u32x4 ka[NI], va[NI];
  issue(0, ka, va);
#if PKV_PREFETCH
  u32x4 kb[NI], vb[NI];
  for (int c = 0; c < n_chunks; c += 2) {
    if (c + 1 < n_chunks) issue(c + 1, kb, vb);
    consume(c, ka, va);
    if (c + 1 < n_chunks) {
      if (c + 2 < n_chunks) issue(c + 2, ka, va);
      consume(c + 1, kb, vb);
    }
  }
#else
  for (int c = 0; c < n_chunks; ++c) {
    if (c > 0) issue(c, ka, va);
    consume(c, ka, va);
  }
#endif

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

  // Finish (one partition) or write the partition's partials.  Lane group 0
  // holds the merged columns seg * EPL .. seg * EPL + EPL - 1.
  if (grp != 0) return;
  if (direct) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float o[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = bad_blk ? __builtin_nanf("") : acc[h][e] / l[h];
      float4* dst = reinterpret_cast<float4*>(orow + h * D + seg * EPL);
#pragma unroll
      for (int e = 0; e < EPL; e += 4) dst[e / 4] = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
    }
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const size_t r = ((size_t)s * a.Hq + (size_t)g * G + h) * a.NP + part;
      float4* dst = reinterpret_cast<float4*>(a.ws_acc + r * D + seg * EPL);
#pragma unroll
      for (int e = 0; e < EPL; e += 4) {
        dst[e / 4] = bad_blk ? make_float4(__builtin_nanf(""), 0.0f, 0.0f, 0.0f)
                             : make_float4(acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]);
      }
      if (seg == 0) a.ws_ml[r] = bad_blk ? make_float2(INFINITY, __builtin_nanf("")) : make_float2(m[h], l[h]);
    }
  }
}

// Stage 2: merge the partitions of sequences longer than one partition.
// One wave per (sequence, query head).  Partition p contributes
// exp2(m_p - M) * (acc_p, l_p), M the largest m_p; partitions are visited in
// increasing order.  Lane j owns columns j*CPL .. j*CPL + CPL - 1.
template <int D>
__global__ __launch_bounds__(64) void decode_reduce_kernel(DecodeParams a) {
  constexpr int CPL = D / 64;  // columns per lane (1 or 2)
  const int row = blockIdx.x;  // s * Hq + h
  const int s = row / a.Hq;
  const int lane = threadIdx.x;
  const int L = a.lens[s];
  const bool bad_len = (L < 0) || (L > a.max_len);
  if (!bad_len && L <= a.P) return;  // written by stage 1 (or L = 0 zeros)
  float* o = a.out + (size_t)row * D + lane * CPL;
  if (bad_len) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) o[j] = __builtin_nanf("");
    return;
  }
  const int np = (L + a.P - 1) / a.P;
  const float2* ml = a.ws_ml + (size_t)row * a.NP;
  const float* acc = a.ws_acc + (size_t)row * a.NP * D + lane * CPL;

  float M = kNegBig;
  for (int p = lane; p < np; p += 64) M = fmaxf(M, ml[p].x);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));

  float den = 0.0f;
  float num[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) num[j] = 0.0f;
  for (int p0 = 0; p0 < np; p0 += 64) {
    float f = 0.0f;
    if (p0 + lane < np) {
      const float2 t = ml[p0 + lane];
      f = fast_exp2(t.x - M);
      den = fmaf(t.y, f, den);
    }
    const int cnt = min(64, np - p0);
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
  if constexpr (CPL == 2) {
    *reinterpret_cast<float2*>(o) = make_float2(num[0] / den, num[1] / den);
  } else {
    o[0] = num[0] / den;
  }
}

template <int DT, int D, int B>
hipError_t launch_g(const DecodeParams& p, int group, hipStream_t stream) {
  const dim3 grid(p.grid);
  const dim3 block(kWavesPerWG * 64);
  switch (group) {
    case 1: hipLaunchKernelGGL((decode_units_kernel<DT, D, B, 1>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_units_kernel<DT, D, B, 2>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((decode_units_kernel<DT, D, B, 4>), grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL((decode_units_kernel<DT, D, B, 8>), grid, block, 0, stream, p); break;
    case 16: hipLaunchKernelGGL((decode_units_kernel<DT, D, B, 16>), grid, block, 0, stream, p); break;
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
  if (p.S == 0 || p.n_units == 0) return hipSuccess;
  return dtype == 1 ? launch_d<1>(p, head_dim, block_size, group, stream)
                    : launch_d<0>(p, head_dim, block_size, group, stream);
}

hipError_t launch_decode_reduce(const DecodeParams& p, int head_dim, hipStream_t stream) {
  if (p.S == 0 || p.NP <= 1) return hipSuccess;
  const dim3 grid((unsigned)p.S * (unsigned)p.Hq);
  switch (head_dim) {
    case 64: hipLaunchKernelGGL((decode_reduce_kernel<64>), grid, dim3(64), 0, stream, p); break;
    case 128: hipLaunchKernelGGL((decode_reduce_kernel<128>), grid, dim3(64), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
