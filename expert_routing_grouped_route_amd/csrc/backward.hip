// Backward pass of the MoE layer: gradients of the layer output with respect
// to the tokens, the router weights and bias, and every expert's weights.
//
// The pages time training runs (the DeepSeek-V3 MoE layers of the
// FarSkip-Collective review, "What carries the argument"; the Luffy review's
// training speed-ups, Fig. 8 caption), so the layer's backward pass is part of
// the work they measure; they do not write its formulas out.  It follows from
// the forward pass by the chain rule, with these readings: no gradient through
// the choice of the top-k experts; the kept weights are the softmax over the
// kept logits, so a token's logit gradient is w_i (dw_i - sum_j w_j dw_j) on
// its kept experts; the bf16 rounding of the SwiGLU product passes the
// gradient through unchanged; the bias gradient sums the logit gradient over
// tokens.
//
// bf16 layers run every large product on the forward pass's bf16 GEMM
// machinery: the recomputed G, U and expert outputs on the forward kernels,
// the input gradients on the down kernel against transposed weight copies,
// and the weight gradients, which reduce over an expert's ragged rows, on a
// segment kernel over per-expert zero-padded transposed operands.  Each fp32
// operand enters as a bf16 high part and a bf16 low part.  fp32 layers use a
// grouped GEMM with free element strides, on the matrix cores with split
// operands (or, in the vector-ALU variant, on the VALU in fp32).  The router-weight
// gradient is a two-pass fixed-order reduction on the VALU.  Every output
// element is summed in a fixed order and no atomics are used, so results are
// reproducible bit for bit.
#include <algorithm>
#include <climits>

#include "common.h"
#include "kernels.h"
#include "backward.h"

namespace moe {
namespace {

constexpr int GT = 64;   // output tile edge
constexpr int GK = 16;   // K per LDS stage

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* p, int64_t i) {
  if (BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
  return static_cast<const float*>(p)[i];
}

// C(m, n) = [C(m, n) +] sum_k A(m, k) B(k, n), with A(m, k) at
// A[g*a_g + m*a_sm + k*a_sk] and so on.  RAGGED_K false: group g owns the
// rows off[g] .. off[g+1] of A and C (global row numbers) and tiles come from
// `prefix`; off null: one group of `ext` rows.  RAGGED_K true: group g reduces
// over k = off[g] .. off[g+1] (or 0 .. ext), blockIdx.y = g.
template <bool A_BF16, bool B_BF16, bool RAGGED_K>
__global__ __launch_bounds__(256) void gemm_f32_grouped_kernel(
    const void* __restrict__ A, int64_t a_sm, int64_t a_sk, int64_t a_g,
    const void* __restrict__ B, int64_t b_sk, int64_t b_sn, int64_t b_g,
    float* __restrict__ C, int64_t c_sm, int64_t c_sn, int64_t c_g,
    const int32_t* __restrict__ off, const int32_t* __restrict__ prefix, int G, int ext,
    int M, int N, int K, int accumulate) {
  __shared__ float As[GK][GT + 4];
  __shared__ float Bs[GK][GT + 4];
  const int nt = (N + GT - 1) / GT;
  const int tile = blockIdx.x;
  const int n0 = (tile % nt) * GT;
  int g = 0, m0, m1, k0, k1;
  if (!RAGGED_K) {
    const int mt = tile / nt;
    if (off) {
      if (mt >= prefix[G]) return;
      int lo = 0, hi = G - 1;  // last g with prefix[g] <= mt
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (prefix[mid] <= mt) lo = mid;
        else hi = mid - 1;
      }
      g = lo;
      m0 = off[g] + (mt - prefix[g]) * GT;
      m1 = off[g + 1];
    } else {
      m0 = mt * GT;
      m1 = ext;
      if (m0 >= m1) return;
    }
    k0 = 0;
    k1 = K;
  } else {
    g = blockIdx.y;
    m0 = (tile / nt) * GT;
    m1 = M;
    k0 = off ? off[g] : 0;
    k1 = off ? off[g + 1] : ext;
  }
  const void* Ab = A_BF16 ? (const void*)(static_cast<const uint16_t*>(A) + g * a_g)
                          : (const void*)(static_cast<const float*>(A) + g * a_g);
  const void* Bb = B_BF16 ? (const void*)(static_cast<const uint16_t*>(B) + g * b_g)
                          : (const void*)(static_cast<const float*>(B) + g * b_g);
  float* Cb = C + g * c_g;
  const int t = threadIdx.x, tm = t >> 4, tn = t & 15;
  const bool a_kc = a_sk == 1, b_nc = b_sn == 1;  // which index is contiguous in memory
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int kb = k0; kb < k1; kb += GK) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = t + 256 * u;
      int m, k;
      if (a_kc) { m = q / GK; k = q % GK; }
      else { k = q / GT; m = q % GT; }
      const int gm = m0 + m, gk = kb + k;
      As[k][m] = (gm < m1 && gk < k1) ? load_elem<A_BF16>(Ab, gm * a_sm + gk * a_sk) : 0.f;
      int n, k2;
      if (b_nc) { k2 = q / GT; n = q % GT; }
      else { n = q / GK; k2 = q % GK; }
      const int gn = n0 + n, gk2 = kb + k2;
      Bs[k2][n] = (gn < N && gk2 < k1) ? load_elem<B_BF16>(Bb, gk2 * b_sk + gn * b_sn) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < GK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][tm + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[k][tn + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gm = m0 + tm + 16 * i;
    if (gm >= m1) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + tn + 16 * j;
      if (gn >= N) continue;
      float* c = Cb + gm * c_sm + (int64_t)gn * c_sn;
      *c = accumulate ? *c + acc[i][j] : acc[i][j];
    }
  }
}

// The same products on the bf16 matrix cores.  Operands are staged in LDS as
// fp32 exactly as above (any strides); each fragment is rounded to bf16 when
// read, and an fp32 operand is taken as hi + lo, hi = bf16(v), lo =
// bf16(v - hi) (|v - hi - lo| <= 2^-16 |v|): D += hi_a hi_b + lo_a hi_b +
// hi_a lo_b, the lo_a lo_b term dropped, accumulation in fp32.  128x128 tile,
// K-stages of 32, four waves of 64x64 (2x2 MFMA 32x32x16 tiles).
constexpr int MT = 128;
constexpr int MK = 32;
constexpr int MLD = MT + 1;  // LDS row stride (floats): a row's 8-wide column writes spread over banks

// 8 consecutive elements as fp32 (16-byte aligned source).
template <bool BF16>
__device__ __forceinline__ void load8(const void* p, float (&v)[8]) {
  if (BF16) {
    const u32x4 w = *static_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const f32x4 a = static_cast<const f32x4*>(p)[0], b = static_cast<const f32x4*>(p)[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
}

// One operand's tile into LDS: dst[k][r] = X(rb + r, kb + k) for r < MT,
// k < MK, zero outside rows [.., r1) and k-values [.., k1); X(r, k) at
// base[r * s_r + k * s_k].  Along whichever index is contiguous in memory each
// lane reads 8 elements at once (16-byte aligned, wholly inside the bounds),
// else element by element.
template <bool BF16>
__device__ __forceinline__ void load_tile(const void* base, int64_t s_r, int64_t s_k, int rb,
                                          int r1, int kb, int k1, float (*dst)[MLD]) {
  const int t = threadIdx.x;
  const size_t es = BF16 ? 2 : 4;
  if (s_k == 1 || s_r == 1) {
    const bool along_k = s_k == 1;
#pragma unroll
    for (int u = 0; u < (MT * MK) / (8 * 256); ++u) {
      const int q = t + 256 * u;
      int r, k;
      if (along_k) { r = q / (MK / 8); k = (q % (MK / 8)) * 8; }
      else { k = q / (MT / 8); r = (q % (MT / 8)) * 8; }
      const int gr = rb + r, gk = kb + k;
      const int64_t idx = (int64_t)gr * s_r + (int64_t)gk * s_k;
      const uint8_t* ptr = static_cast<const uint8_t*>(base) + idx * (int64_t)es;
      const bool whole = along_k ? (gr < r1 && gk + 8 <= k1) : (gk < k1 && gr + 8 <= r1);
      float v[8];
      if (whole && ((reinterpret_cast<uintptr_t>(ptr) & 15) == 0)) {
        load8<BF16>(ptr, v);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int er = along_k ? gr : gr + e, ek = along_k ? gk + e : gk;
          v[e] = (er < r1 && ek < k1) ? load_elem<BF16>(base, (int64_t)er * s_r + (int64_t)ek * s_k)
                                      : 0.f;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (along_k) dst[k + e][r] = v[e];
        else dst[k][r + e] = v[e];
      }
    }
  } else {
#pragma unroll 4
    for (int u = 0; u < (MT * MK) / 256; ++u) {
      const int q = t + 256 * u;
      const int k = q / MT, r = q % MT;
      const int gr = rb + r, gk = kb + k;
      dst[k][r] = (gr < r1 && gk < k1) ? load_elem<BF16>(base, (int64_t)gr * s_r + (int64_t)gk * s_k)
                                       : 0.f;
    }
  }
}

// bf16 hi and lo parts of 8 fp32 values.
__device__ __forceinline__ void split8(const float (&v)[8], bool want_lo, bf16x8& hi, bf16x8& lo) {
  u32x4 h, l;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    h[p] = pack_bf16x2_rne(v[2 * p], v[2 * p + 1]);
    if (want_lo) {
      const float r0 = v[2 * p] - __uint_as_float(h[p] << 16);
      const float r1 = v[2 * p + 1] - __uint_as_float(h[p] & 0xFFFF0000u);
      l[p] = pack_bf16x2_rne(r0, r1);
    }
  }
  hi = as_bf16x8(h);
  if (want_lo) lo = as_bf16x8(l);
}

template <bool A_BF16, bool B_BF16, bool RAGGED_K>
__global__ __launch_bounds__(256) void gemm_mfma_grouped_kernel(
    const void* __restrict__ A, int64_t a_sm, int64_t a_sk, int64_t a_g,
    const void* __restrict__ B, int64_t b_sk, int64_t b_sn, int64_t b_g,
    float* __restrict__ C, int64_t c_sm, int64_t c_sn, int64_t c_g,
    const int32_t* __restrict__ off, const int32_t* __restrict__ prefix, int G, int ext,
    int M, int N, int K, int accumulate) {
  __shared__ float As[MK][MLD];
  __shared__ float Bs[MK][MLD];
  const int nt = (N + MT - 1) / MT;
  const int tile = blockIdx.x;
  const int n0 = (tile % nt) * MT;
  int g = 0, m0, m1, k0, k1;
  if (!RAGGED_K) {
    const int mt = tile / nt;
    if (off) {
      if (mt >= prefix[G]) return;
      int lo = 0, hi = G - 1;  // last g with prefix[g] <= mt
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (prefix[mid] <= mt) lo = mid;
        else hi = mid - 1;
      }
      g = lo;
      m0 = off[g] + (mt - prefix[g]) * MT;
      m1 = off[g + 1];
    } else {
      m0 = mt * MT;
      m1 = ext;
      if (m0 >= m1) return;
    }
    k0 = 0;
    k1 = K;
  } else {
    g = blockIdx.y;
    m0 = (tile / nt) * MT;
    m1 = M;
    k0 = off ? off[g] : 0;
    k1 = off ? off[g + 1] : ext;
  }
  const void* Ab = A_BF16 ? (const void*)(static_cast<const uint16_t*>(A) + g * a_g)
                          : (const void*)(static_cast<const float*>(A) + g * a_g);
  const void* Bb = B_BF16 ? (const void*)(static_cast<const uint16_t*>(B) + g * b_g)
                          : (const void*)(static_cast<const float*>(B) + g * b_g);
  float* Cb = C + g * c_g;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r32 = lane & 31, kg = lane >> 5;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  for (int kb = k0; kb < k1; kb += MK) {
    load_tile<A_BF16>(Ab, a_sm, a_sk, m0, m1, kb, k1, As);
    load_tile<B_BF16>(Bb, b_sn, b_sk, n0, N, kb, k1, Bs);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < MK / 16; ++ks) {
      bf16x8 ah[2], al[2], bh[2], bl[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = As[ks * 16 + kg * 8 + e][wm * 64 + i * 32 + r32];
        split8(v, !A_BF16, ah[i], al[i]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = Bs[ks * 16 + kg * 8 + e][wn * 64 + j * 32 + r32];
        split8(v, !B_BF16, bh[j], bl[j]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = mfma_32x32x16_bf16(ah[i], bh[j], acc[i][j]);
          if (!A_BF16) acc[i][j] = mfma_32x32x16_bf16(al[i], bh[j], acc[i][j]);
          if (!B_BF16) acc[i][j] = mfma_32x32x16_bf16(ah[i], bl[j], acc[i][j]);
        }
    }
    __syncthreads();
  }
  // lane l holds column l % 32 and rows 8 (v / 4) + 4 (l / 32) + v % 4 of each 32x32 tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int gn = n0 + wn * 64 + j * 32 + r32;
      if (gn >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int gm = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * kg + (v & 3);
        if (gm >= m1) continue;
        float* c = Cb + gm * c_sm + (int64_t)gn * c_sn;
        *c = accumulate ? *c + acc[i][j][v] : acc[i][j][v];
      }
    }
}

struct GemmOp {
  const void* A; bool a_bf16; int64_t a_sm, a_sk, a_g;
  const void* B; bool b_bf16; int64_t b_sk, b_sn, b_g;
  float* C; int64_t c_sm, c_sn, c_g;
  const int32_t* off;     // ragged offsets [G+1] or null
  const int32_t* prefix;  // ragged M: M-tile prefix [G+1] (launch_segment_tables)
  int G, ext;             // groups; extent when off is null
  int64_t m_bound;        // ragged M: bound of the M-tiles over all groups
  int M, N, K;
  bool ragged_k;
  bool accumulate;
  bool mfma;              // the matrix-core kernel (tiles of MT) or the VALU one (GT)
};

template <bool AB, bool BB, bool RK>
void launch_gemm_t(const GemmOp& o, hipStream_t s) {
  const int tt = o.mfma ? MT : GT;
  const int nt = (o.N + tt - 1) / tt;
  dim3 grid;
  if (RK) grid = dim3((unsigned)(((int64_t)o.M + tt - 1) / tt * nt), (unsigned)o.G);
  else grid = dim3((unsigned)(o.m_bound * nt));
  if (grid.x == 0 || grid.y == 0) return;
  if (o.mfma)
    hipLaunchKernelGGL((gemm_mfma_grouped_kernel<AB, BB, RK>), grid, dim3(256), 0, s, o.A, o.a_sm,
                       o.a_sk, o.a_g, o.B, o.b_sk, o.b_sn, o.b_g, o.C, o.c_sm, o.c_sn, o.c_g,
                       o.off, o.prefix, o.G, o.ext, o.M, o.N, o.K, (int)o.accumulate);
  else
    hipLaunchKernelGGL((gemm_f32_grouped_kernel<AB, BB, RK>), grid, dim3(256), 0, s, o.A, o.a_sm,
                       o.a_sk, o.a_g, o.B, o.b_sk, o.b_sn, o.b_g, o.C, o.c_sm, o.c_sn, o.c_g,
                       o.off, o.prefix, o.G, o.ext, o.M, o.N, o.K, (int)o.accumulate);
}

void launch_gemm(const GemmOp& o, hipStream_t s) {
#define MOE_G(AB, BB)                                   \
  if (o.a_bf16 == AB && o.b_bf16 == BB) {               \
    if (o.ragged_k) launch_gemm_t<AB, BB, true>(o, s);  \
    else launch_gemm_t<AB, BB, false>(o, s);            \
    return;                                             \
  }
  MOE_G(false, false)
  MOE_G(false, true)
  MOE_G(true, false)
  MOE_G(true, true)
#undef MOE_G
}

// dY[i] = w[a] * dout[t] and dw[a] = dout[t] . y[i] for sorted row i holding
// assignment a = perm[i] of token t = a / k; one wave per row.
__global__ __launch_bounds__(256) void bwd_rows_kernel(const float* __restrict__ dout,
                                                       const float* __restrict__ y,
                                                       const int32_t* __restrict__ perm,
                                                       const float* __restrict__ w, int R, int k,
                                                       int d, float* __restrict__ dY,
                                                       float* __restrict__ dw) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + wave;
  if (i >= R) return;
  const int a = perm[i], t = a / k;
  const float wa = w[a];
  const float* dr = dout + (size_t)t * d;
  const float* yr = y + (size_t)i * d;
  float* o = dY + (size_t)i * d;
  float s = 0.f;
  for (int c = lane; c < d; c += 64) {
    const float g = dr[c];
    o[c] = wa * g;
    s = fmaf(g, yr[c], s);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
  if (lane == 0) dw[a] = s;
}

// bf16 layers, per sorted row i (a = perm[i]), with dA'[i] = dout[t] W_d[e]
// (unweighted) in dA and the forward's bf16 SwiGLU row A[i] in Abf:
//   dw[a] = sum_c A[i][c] dA'[i][c]   (= dout[t] . y[i], y = A W_d^T),
//   dG = w[a] dA' * U * silu'(G),  dU = w[a] dA' * silu(G),
// written as row i of dGU [R, 4I]: [dG hi | dG lo | dU hi | dU lo] (bf16
// parts, hi = bf16(v), lo = bf16(v - hi), round to nearest even).
// One block per row; each lane sums its four-column chunks in order, then a
// fixed xor tree in the wave and the four waves in order.
__global__ __launch_bounds__(256) void swiglu_bwd_rows_kernel(const float* __restrict__ G,
                                                              const float* __restrict__ U,
                                                              const float* __restrict__ dA,
                                                              const uint16_t* __restrict__ Abf,
                                                              const int32_t* __restrict__ perm,
                                                              const float* __restrict__ w, int I,
                                                              float* __restrict__ dw,
                                                              uint16_t* __restrict__ dGU) {
  __shared__ float part[4];
  const int i = blockIdx.x, tid = threadIdx.x;
  const int a = perm[i];
  const float wa = w[a];
  const f32x4* g4 = reinterpret_cast<const f32x4*>(G + (size_t)i * I);
  const f32x4* u4 = reinterpret_cast<const f32x4*>(U + (size_t)i * I);
  uint16_t* o = dGU + (size_t)i * 4 * I;
  const f32x4* d4 = reinterpret_cast<const f32x4*>(dA + (size_t)i * I);
  const uint2* a4 = reinterpret_cast<const uint2*>(Abf + (size_t)i * I);
  float sum = 0.f;
  for (int c = tid; c < I / 4; c += 256) {
    const f32x4 g = g4[c], u = u4[c], da = d4[c];
    const uint2 q = a4[c];
    const float av[4] = {__uint_as_float(q.x << 16), __uint_as_float(q.x & 0xffff0000u),
                         __uint_as_float(q.y << 16), __uint_as_float(q.y & 0xffff0000u)};
    f32x4 og, ou;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sum = fmaf(av[j], da[j], sum);
      const float sg = 1.0f / (1.0f + __expf(-g[j]));
      const float dd = wa * da[j];
      og[j] = dd * u[j] * (sg * (1.0f + g[j] * (1.0f - sg)));
      ou[j] = dd * (g[j] * sg);
    }
    uint32_t h[4], l[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      h[j] = pack_bf16x2_rne(og[2 * j], og[2 * j + 1]);
      l[j] = pack_bf16x2_rne(og[2 * j] - __uint_as_float(h[j] << 16),
                             og[2 * j + 1] - __uint_as_float(h[j] & 0xffff0000u));
      h[2 + j] = pack_bf16x2_rne(ou[2 * j], ou[2 * j + 1]);
      l[2 + j] = pack_bf16x2_rne(ou[2 * j] - __uint_as_float(h[2 + j] << 16),
                                 ou[2 * j + 1] - __uint_as_float(h[2 + j] & 0xffff0000u));
    }
    *reinterpret_cast<uint2*>(o + 4 * c) = make_uint2(h[0], h[1]);
    *reinterpret_cast<uint2*>(o + I + 4 * c) = make_uint2(l[0], l[1]);
    *reinterpret_cast<uint2*>(o + 2 * I + 4 * c) = make_uint2(h[2], h[3]);
    *reinterpret_cast<uint2*>(o + 3 * I + 4 * c) = make_uint2(l[2], l[3]);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m);
  if ((tid & 63) == 0) part[tid >> 6] = sum;
  __syncthreads();
  if (tid == 0) dw[a] = ((part[0] + part[1]) + part[2]) + part[3];
}

// Logit gradient of each token's kept weights: dL_j = w_j (dw_j - sum w dw),
// in assignment order (dl) and in sorted-row order (dls[inv[a]] = dl[a]).
__global__ __launch_bounds__(256) void bwd_gate_kernel(const float* __restrict__ w,
                                                       const float* __restrict__ dw,
                                                       const int32_t* __restrict__ inv, int T,
                                                       int k, float* __restrict__ dl,
                                                       float* __restrict__ dls) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  const float* wt = w + (size_t)t * k;
  const float* dt = dw + (size_t)t * k;
  float s = 0.f;
  for (int j = 0; j < k; ++j) s = fmaf(wt[j], dt[j], s);
  for (int j = 0; j < k; ++j) {
    const size_t a = (size_t)t * k + j;
    const float v = wt[j] * (dt[j] - s);
    dl[a] = v;
    dls[inv[a]] = v;
  }
}

// The forward's SwiGLU product from fp32 G and U: A = silu(g) * u, stored as
// fp32 values.  For bf16 layers it is formed as the forward's gate/up
// epilogue forms it (hardware reciprocal, round to nearest even to bf16), so
// from the same G and U it is the same A bit for bit, and Abf (if given)
// receives the bf16 bits.  A may be null (only the bf16 bits are kept).
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const float* __restrict__ G,
                                                         const float* __restrict__ U, int64_t n,
                                                         int round_bf16, float* __restrict__ A,
                                                         uint16_t* __restrict__ Abf) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    float a;
    if (round_bf16) {
      const uint32_t b = pack_bf16x2_rne(silu_times_rcp(G[i], U[i]), 0.f);
      a = __uint_as_float(b << 16);
      if (Abf) Abf[i] = (uint16_t)b;
    } else {
      a = silu_times(G[i], U[i]);
    }
    if (A) A[i] = a;
  }
}

// In place: G <- dA * U * silu'(G), U <- dA * silu(G).
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(float* __restrict__ G,
                                                         float* __restrict__ U,
                                                         const float* __restrict__ dA, int64_t n) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float g = G[i], u = U[i], da = dA[i];
    const float s = 1.0f / (1.0f + __expf(-g));
    G[i] = da * u * (s * (1.0f + g * (1.0f - s)));
    U[i] = da * (g * s);
  }
}

// dx[t] = sum_j dXs[inv[t*k+j]] + sum_j dl[t*k+j] W_r[ids[t*k+j]] (+ the
// shared experts' term: dxs[t], then dxs[T + t] with two slabs), slot order,
// then the router term, then the shared term.  One wave
// per token, four consecutive columns per lane and step.
template <bool WR_BF16>
__global__ __launch_bounds__(256) void bwd_dx_kernel(const float* __restrict__ dXs,
                                                     const int32_t* __restrict__ inv,
                                                     const int32_t* __restrict__ ids,
                                                     const float* __restrict__ dl,
                                                     const void* __restrict__ wr,
                                                     const float* __restrict__ dxs, int slabs,
                                                     int T, int k, int d,
                                                     float* __restrict__ dx) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  int row[kMaxK], ex[kMaxK];
  float g[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    row[j] = 0;
    ex[j] = 0;
    g[j] = 0.f;
    if (j < k) {
      row[j] = inv[(size_t)t * k + j];
      ex[j] = ids[(size_t)t * k + j];
      g[j] = dl[(size_t)t * k + j];
    }
  }
  const int d4 = d >> 2;
  for (int c = lane; c < d4; c += 64) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k) {
        const f32x4 v = reinterpret_cast<const f32x4*>(dXs + (size_t)row[j] * d)[c];
        acc[0] += v[0];
        acc[1] += v[1];
        acc[2] += v[2];
        acc[3] += v[3];
      }
    }
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k) {
        float w[4];
        if (WR_BF16) {
          const uint2 q = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(wr) +
                                                         (size_t)ex[j] * d)[c];
          w[0] = __uint_as_float(q.x << 16);
          w[1] = __uint_as_float(q.x & 0xFFFF0000u);
          w[2] = __uint_as_float(q.y << 16);
          w[3] = __uint_as_float(q.y & 0xFFFF0000u);
        } else {
          const f32x4 q = reinterpret_cast<const f32x4*>(static_cast<const float*>(wr) +
                                                         (size_t)ex[j] * d)[c];
          w[0] = q[0];
          w[1] = q[1];
          w[2] = q[2];
          w[3] = q[3];
        }
        acc[0] = fmaf(g[j], w[0], acc[0]);
        acc[1] = fmaf(g[j], w[1], acc[1]);
        acc[2] = fmaf(g[j], w[2], acc[2]);
        acc[3] = fmaf(g[j], w[3], acc[3]);
      }
    }
    for (int sl = 0; dxs && sl < slabs; ++sl) {
      const f32x4 v = reinterpret_cast<const f32x4*>(dxs + ((size_t)sl * T + t) * d)[c];
      acc[0] += v[0];
      acc[1] += v[1];
      acc[2] += v[2];
      acc[3] += v[3];
    }
    reinterpret_cast<f32x4*>(dx + (size_t)t * d)[c] = acc;
  }
}

// Router-weight gradient dW_r[e] = sum over expert e's sorted rows i of
// dls[i] * xs[i], in two fixed-order passes.  Pass 1: block (m, c) takes M-tile
// m of `tile` rows (tiles from `prefix`, as the grouped GEMMs number them) and
// the 512 columns c*512 .. ; lane l of wave w owns 8 columns and sums the rows
// w, w+4, ... of the tile in increasing order; the four waves' sums are added
// in wave order into part[m][:].  Pass 2 adds each expert's tile partials in
// tile order.  xs is bf16 or fp32; d is a multiple of 64.
template <bool XBF>
__device__ __forceinline__ void load8(const void* xs, int64_t at, float (&v)[8]) {
  if (XBF) {
    const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xs) + at);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(xs) + at);
    const f32x4 b = *reinterpret_cast<const f32x4*>(static_cast<const float*>(xs) + at + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = a[j];
      v[4 + j] = b[j];
    }
  }
}

template <bool XBF>
__global__ __launch_bounds__(256) void router_grad_part_kernel(
    const float* __restrict__ dls, const void* __restrict__ xs, const int32_t* __restrict__ off,
    const int32_t* __restrict__ prefix, int E, int d, int tile, float* __restrict__ part) {
  __shared__ float red[3][512];
  const int m = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (m >= prefix[E]) return;  // tiles past the last expert's
  int lo = 0, hi = E - 1;      // the expert e with prefix[e] <= m < prefix[e + 1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= m) lo = mid;
    else hi = mid - 1;
  }
  const int e = lo;
  const int r0 = off[e] + (m - prefix[e]) * tile;
  const int r1 = min(r0 + tile, off[e + 1]);
  const int c = blockIdx.y * 512 + lane * 8;
  const bool on = c < d;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (on) {
    int i = r0 + w;
    for (; i + 12 < r1; i += 16) {  // four rows in flight
      float v[4][8];
#pragma unroll
      for (int q = 0; q < 4; ++q) load8<XBF>(xs, (int64_t)(i + 4 * q) * d + c, v[q]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float g = dls[i + 4 * q];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = fmaf(g, v[q][j], acc[j]);
      }
    }
    for (; i < r1; i += 4) {
      float v[8];
      load8<XBF>(xs, (int64_t)i * d + c, v);
      const float g = dls[i];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = fmaf(g, v[j], acc[j]);
    }
  }
  if (w > 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) red[w - 1][lane * 8 + j] = acc[j];
  }
  __syncthreads();
  if (w == 0 && on) {
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += red[q][lane * 8 + j];
    f32x4* o = reinterpret_cast<f32x4*>(part + (int64_t)m * d + c);
    o[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    o[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
}

// Pass 2: block (e, c) sums part[prefix[e] .. prefix[e+1]) over 1024 columns
// (4 per thread), in tile order; an expert without rows gets zeros.
__global__ __launch_bounds__(256) void router_grad_reduce_kernel(const float* __restrict__ part,
                                                                 const int32_t* __restrict__ prefix,
                                                                 int d, float* __restrict__ dwr) {
  const int e = blockIdx.x;
  const int c = blockIdx.y * 1024 + threadIdx.x * 4;
  if (c >= d) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int m = prefix[e]; m < prefix[e + 1]; ++m) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(part + (int64_t)m * d + c);
    acc[0] += v[0];
    acc[1] += v[1];
    acc[2] += v[2];
    acc[3] += v[3];
  }
  *reinterpret_cast<f32x4*>(dwr + (int64_t)e * d + c) = acc;
}

// dbias[e] = sum of dls over expert e's sorted rows: 256 strided partial sums,
// then a fixed-order tree in LDS.  One block per expert.
__global__ __launch_bounds__(256) void bwd_bias_kernel(const float* __restrict__ dls,
                                                       const int32_t* __restrict__ off,
                                                       float* __restrict__ db) {
  __shared__ float part[256];
  const int e = blockIdx.x, tid = threadIdx.x;
  float s = 0.f;
  for (int i = off[e] + tid; i < off[e + 1]; i += 256) s += dls[i];
  part[tid] = s;
  __syncthreads();
  for (int h = 128; h >= 1; h >>= 1) {
    if (tid < h) part[tid] += part[tid + h];
    __syncthreads();
  }
  if (tid == 0) db[e] = part[0];
}

unsigned ew_grid(int64_t n) { return (unsigned)std::min<int64_t>((n + 255) / 256, 65536); }

// out[e][q][p] = in[e][p][q] for bf16 [E][P][Q]; 64x64 tiles through LDS.
// Each lane reads 8 consecutive elements of a row (16 bytes) and writes 8
// consecutive elements of a transposed row; edges and unaligned rows go
// element by element.  Block (q-tile, p-tile, e).
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ in,
                                                             int P, int Q,
                                                             uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];  // 144-byte rows
  const int q0 = blockIdx.x * 64, p0 = blockIdx.y * 64, e = blockIdx.z;
  const uint16_t* src = in + (size_t)e * P * Q;
  uint16_t* dst = out + (size_t)e * P * Q;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int v = threadIdx.x + 256 * u, r = v >> 3, c = (v & 7) * 8;
    const int p = p0 + r, q = q0 + c;
    const uint16_t* sp = src + (size_t)p * Q + q;
    if (p < P && q + 8 <= Q && ((reinterpret_cast<uintptr_t>(sp) & 15) == 0)) {
      *reinterpret_cast<u32x4*>(&tile[r][c]) = *reinterpret_cast<const u32x4*>(sp);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) tile[r][c + i] = (p < P && q + i < Q) ? sp[i] : 0;
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int v = threadIdx.x + 256 * u, r = v >> 3, c = (v & 7) * 8;
    const int q = q0 + r, p = p0 + c;
    if (q >= Q) continue;
    uint16_t* dp = dst + (size_t)q * P + p;
    uint16_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = tile[c + i][r];
    if (p + 8 <= P && ((reinterpret_cast<uintptr_t>(dp) & 15) == 0)) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = (uint32_t)w[2 * i] | ((uint32_t)w[2 * i + 1] << 16);
      *reinterpret_cast<u32x4*>(dp) = o;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (p + i < P) dp[i] = w[i];
    }
  }
}

// Row r of v [rows, cols] (fp32) as bf16 parts hi = bf16(v), lo = bf16(v - hi),
// round to nearest even (|v - hi - lo| <= 2^-16 |v|), inside row r of out
// (out_ld elements per row): hi at columns hi_col .., lo at lo_col ..; a
// product on the bf16 matrix cores then takes both parts in one K loop.
// cols % 4 == 0.  One row per block iteration, 4 elements per lane.
__global__ __launch_bounds__(256) void split_rows_bf16_kernel(const float* __restrict__ v,
                                                              int64_t rows, int cols,
                                                              uint16_t* __restrict__ out,
                                                              int64_t out_ld, int hi_col,
                                                              int lo_col) {
  const int c4 = cols / 4;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const f32x4* src = reinterpret_cast<const f32x4*>(v + r * cols);
    uint16_t* o = out + r * out_ld;
    for (int c = threadIdx.x; c < c4; c += 256) {
      const f32x4 x = src[c];
      uint32_t h[2], l[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        h[j] = pack_bf16x2_rne(x[2 * j], x[2 * j + 1]);
        l[j] = pack_bf16x2_rne(x[2 * j] - __uint_as_float(h[j] << 16),
                               x[2 * j + 1] - __uint_as_float(h[j] & 0xffff0000u));
      }
      *reinterpret_cast<uint2*>(o + hi_col + 4 * c) = make_uint2(h[0], h[1]);
      *reinterpret_cast<uint2*>(o + lo_col + 4 * c) = make_uint2(l[0], l[1]);
    }
  }
}

void launch_split_rows(const float* v, int64_t rows, int cols, uint16_t* out, int64_t out_ld,
                       int hi_col, int lo_col, hipStream_t s) {
  if (rows <= 0) return;
  hipLaunchKernelGGL(split_rows_bf16_kernel, dim3((unsigned)std::min<int64_t>(rows, 16384)),
                     dim3(256), 0, s, v, rows, cols, out, out_ld, hi_col, lo_col);
}

// Experts to XCDs, longest first: expert e costs 2 ceil(n_e / 64) K-steps
// per tile plus about five for a tile's start and epilogue (every expert has
// the same number of tiles), experts are taken by falling cost (ties by
// index) and each goes to the XCD with the least cost so far among those
// with fewer than cap experts (ties to the lowest XCD).  The choices are made
// by one wave, lane x < 8 holding XCD x's cost and count: the minimum over
// the eight lanes through DPP moves, then the lowest lane holding it from a
// ballot; the sorted costs and experts sit in registers, lane l holding
// places l, l + 64, ...  The records are written by all threads.
template <int CTRL>
__device__ __forceinline__ int sched_dpp(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}

// The whole block (256 threads) makes the schedule.
__device__ void seg_sched_block(const int32_t* __restrict__ off, int E, int cap,
                                int32_t* __restrict__ rec) {
  __shared__ int cost[256], ocost[256], order[256], place[kSegXcds * kSegCapMax];
  if (E <= 0 || E > 256) return;  // (the layer's dimension checks keep E <= 256)
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) cost[e] = 2 * ((off[e + 1] - off[e] + 63) / 64) + 5;
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    const int c = cost[e];
    int rank = 0;
#pragma unroll 8
    for (int j = 0; j < E; ++j) rank += (cost[j] > c) | ((cost[j] == c) & (j < e));
    order[rank] = e;
    ocost[rank] = c;
  }
  for (int i = tid; i < kSegXcds * cap; i += 256) place[i] = -1;
  __syncthreads();
  if (tid < 64) {
    int oc[4], oe[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = tid + 64 * i;
      oc[i] = r < E ? ocost[r] : 0;
      oe[i] = r < E ? order[r] : 0;
    }
    const bool xl = tid < kSegXcds;  // this lane stands for XCD tid
    int load = 0, n = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int jn = min(64, E - 64 * i);
      for (int j = 0; j < jn; ++j) {
        const int key = xl && n < cap ? load : INT_MAX;
        int m = min(key, sched_dpp<0xB1>(key));  // lanes xor 1
        m = min(m, sched_dpp<0x4E>(m));          // lanes xor 2
        m = min(m, sched_dpp<0x141>(m));         // lane i with 7 - i of its eight
        const unsigned long long b = __ballot(xl && key == m);
        if (tid == __builtin_ctzll(b)) {
          place[tid * cap + n] = __builtin_amdgcn_readlane(oe[i], j);
          ++n;
          load += __builtin_amdgcn_readlane(oc[i], j);
        }
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < kSegXcds * cap; i += 256) {
    const int e = place[i];
    *reinterpret_cast<int4*>(rec + 4 * i) =
        e >= 0 ? make_int4(e, off[e], off[e + 1] - off[e], 1) : make_int4(0, 0, 0, 0);
  }
}

__global__ __launch_bounds__(256) void seg_sched_kernel(const int32_t* __restrict__ off, int E,
                                                        int cap, int32_t* __restrict__ rec) {
  seg_sched_block(off, E, cap, rec);
}


// Sorted row r of the gate-weighted dout, w[perm[r]] * v[perm[r] / k], as its
// bf16 hi parts (columns 0..cols-1 of out row r) and lo parts (cols..2 cols-1),
// rounded as split_rows_bf16_kernel rounds.  With sched_rec, block 0 makes
// the weight-gradient schedule instead (seg_sched_block, from the expert
// offsets sched_off) while the other blocks take the rows: dispatched first,
// it finishes under their work.
__global__ __launch_bounds__(256) void gather_split_rows_kernel(const float* __restrict__ v,
                                                                const int32_t* __restrict__ perm,
                                                                const float* __restrict__ w, int k,
                                                                int64_t rows, int cols,
                                                                uint16_t* __restrict__ out,
                                                                const int32_t* __restrict__ sched_off,
                                                                int sched_E,
                                                                int32_t* __restrict__ sched_rec) {
#pragma clang fp contract(off)  // the lo parts come from the rounded products
  const int b0 = sched_rec ? 1 : 0;
  if ((int)blockIdx.x < b0) {
    seg_sched_block(sched_off, sched_E, seg_sched_cap(sched_E), sched_rec);
    return;
  }
  const int c4 = cols / 4;
  for (int64_t r = blockIdx.x - b0; r < rows; r += gridDim.x - b0) {
    const int a = perm[r];
    const float sc = w[a];
    const f32x4* src = reinterpret_cast<const f32x4*>(v + (int64_t)(a / k) * cols);
    uint16_t* o = out + r * 2 * cols;
    for (int c = threadIdx.x; c < c4; c += 256) {
      const f32x4 x0 = src[c];
      const float x[4] = {sc * x0[0], sc * x0[1], sc * x0[2], sc * x0[3]};
      uint32_t h[2], l[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        h[j] = pack_bf16x2_rne(x[2 * j], x[2 * j + 1]);
        l[j] = pack_bf16x2_rne(x[2 * j] - __uint_as_float(h[j] << 16),
                               x[2 * j + 1] - __uint_as_float(h[j] & 0xffff0000u));
      }
      *reinterpret_cast<uint2*>(o + 4 * c) = make_uint2(h[0], h[1]);
      *reinterpret_cast<uint2*>(o + cols + 4 * c) = make_uint2(l[0], l[1]);
    }
  }
}

// Padded part of each expert along the reduction index of a weight-gradient
// product: 2 * roundup(n_e, 64) columns (the hi half, then the lo half, or
// twice the same bf16 rows), starting at poff[e].
__global__ __launch_bounds__(64) void seg_offsets_kernel(const int32_t* __restrict__ off, int E,
                                                         int32_t* __restrict__ poff) {
  if (threadIdx.x != 0) return;
  int acc = 0;
  for (int e = 0; e < E; ++e) {
    poff[e] = acc;
    acc += 2 * ((off[e + 1] - off[e] + 63) / 64 * 64);
  }
  poff[E] = acc;
}

// S slices of one segment's reduction index, 2 * roundup(T, 64) columns:
// slice e covers the 64-column steps [e*n/S, (e+1)*n/S) of its n steps.
__global__ __launch_bounds__(64) void split_seg_offsets_kernel(int T, int S,
                                                               int32_t* __restrict__ poff) {
  const int n = 2 * ((T + 63) / 64);
  for (int e = threadIdx.x; e <= S; e += 64) poff[e] = (int)((int64_t)e * n / S) * 64;
}

// out[i] = sum over e < S of part[e*n + i], in slice order; n % 4 == 0.
__global__ __launch_bounds__(256) void sum_slices_kernel(const float* __restrict__ part, int S,
                                                         int64_t n, float* __restrict__ out) {
  const int64_t n4 = n / 4;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    f32x4 acc = reinterpret_cast<const f32x4*>(part)[i];
    for (int e = 1; e < S; ++e) {
      const f32x4 v = reinterpret_cast<const f32x4*>(part + (int64_t)e * n)[i];
      acc[0] += v[0];
      acc[1] += v[1];
      acc[2] += v[2];
      acc[3] += v[3];
    }
    reinterpret_cast<f32x4*>(out)[i] = acc;
  }
}

// dst[c][poff[e] + h*seg + j] = part h of src[off[e] + j][c] for the sorted
// rows j < n_e of expert e (seg = roundup(n_e, 64)), zero for j >= n_e: the
// rows transposed so that the reduction over an expert's rows is contiguous.
// F32: part 0 = bf16(v), part 1 = bf16(v - part 0); bf16 source: both parts
// are v.  64x64 tiles through LDS, 8 elements per lane on each side.  Block
// (64 destination columns, 64 destination rows); tiles past poff[E] return.
// GATHER (fp32 sources): sorted row r is g_w[g_perm[r]] times source row
// g_perm[r] / g_k (the gate-weighted dout rows, formed here instead of stored).
template <bool F32, bool GATHER = false>
__global__ __launch_bounds__(256) void seg_transpose_kernel(const void* __restrict__ src, int C,
                                                            int64_t sld, int part_col,
                                                            const int32_t* __restrict__ g_perm,
                                                            const float* __restrict__ g_w, int g_k,
                                                            const int32_t* __restrict__ off,
                                                            const int32_t* __restrict__ poff, int E,
                                                            int64_t ld, uint16_t* __restrict__ dst) {
#pragma clang fp contract(off)  // the lo parts come from the rounded products
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];  // [j][c]
  const int j0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  if (j0 >= poff[E]) return;
  int lo = 0, hi = E - 1;  // last e with poff[e] <= j0 (the expert whose part holds j0)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (poff[mid] <= j0) lo = mid;
    else hi = mid - 1;
  }
  const int e = lo;
  const int seg = (poff[e + 1] - poff[e]) / 2, local = j0 - poff[e];
  const int half = local >= seg ? 1 : 0, col = local - half * seg;
  const int n_e = off[e + 1] - off[e], r0 = off[e] + col;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int v = threadIdx.x + 256 * u, jj = v >> 3, cc = (v & 7) * 8;
    const bool ok = col + jj < n_e && c0 + cc + 8 <= C;
    uint16_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = 0;
    if (ok) {
      int srow = r0 + jj;
      float scale = 1.f;
      if (GATHER) {
        const int a = g_perm[srow];
        srow = a / g_k;
        scale = g_w[a];
      }
      const size_t at = (size_t)srow * sld + c0 + cc + (F32 ? 0 : half * part_col);
      if (F32) {
        const f32x4 x0 = reinterpret_cast<const f32x4*>(static_cast<const float*>(src) + at)[0];
        const f32x4 x1 = reinterpret_cast<const f32x4*>(static_cast<const float*>(src) + at)[1];
        float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        if (GATHER) {
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] = scale * x[i];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t h = pack_bf16x2_rne(x[i], 0.f);
          w[i] = half ? (uint16_t)pack_bf16x2_rne(x[i] - __uint_as_float(h << 16), 0.f)
                      : (uint16_t)h;
        }
      } else {
        const u32x4 q = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + at);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          w[2 * i] = (uint16_t)q[i];
          w[2 * i + 1] = (uint16_t)(q[i] >> 16);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) tile[jj][cc + i] = w[i];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int v = threadIdx.x + 256 * u, r = v >> 3, jc = (v & 7) * 8;
    if (c0 + r >= C) continue;
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = (uint32_t)tile[jc + 2 * i][r] | ((uint32_t)tile[jc + 2 * i + 1][r] << 16);
    *reinterpret_cast<u32x4*>(dst + (size_t)(c0 + r) * ld + j0 + jc) = o;
  }
}

// sld: elements between source rows (0: C).  part_col (bf16 sources): part h
// reads the columns h * part_col further on (0: both parts the same values).
void launch_seg_transpose(const void* src, bool f32, int C, const int32_t* off,
                          const int32_t* poff, int E, int64_t ld, uint16_t* dst, hipStream_t s,
                          int64_t sld = 0, int part_col = 0) {
  const dim3 grid((unsigned)(ld / 64), (unsigned)((C + 63) / 64));
  if (sld == 0) sld = C;
  if (f32)
    hipLaunchKernelGGL(seg_transpose_kernel<true>, grid, dim3(256), 0, s, src, C, sld, 0, nullptr,
                       nullptr, 1, off, poff, E, ld, dst);
  else
    hipLaunchKernelGGL(seg_transpose_kernel<false>, grid, dim3(256), 0, s, src, C, sld, part_col,
                       nullptr, nullptr, 1, off, poff, E, ld, dst);
}

// The same for the gate-weighted rows w[perm[r]] * src[perm[r] / k] of an fp32
// source [T, C] (split into hi and lo parts).
void launch_seg_transpose_gather(const float* src, int C, const int32_t* perm, const float* w,
                                 int k, const int32_t* off, const int32_t* poff, int E, int64_t ld,
                                 uint16_t* dst, hipStream_t s) {
  const dim3 grid((unsigned)(ld / 64), (unsigned)((C + 63) / 64));
  hipLaunchKernelGGL((seg_transpose_kernel<true, true>), grid, dim3(256), 0, s, src, C,
                     (int64_t)C, 0, perm, w, k, off, poff, E, ld, dst);
}

void launch_transpose_bf16(const void* in, int E, int P, int Q, void* out, hipStream_t s) {
  const dim3 grid((unsigned)((Q + 63) / 64), (unsigned)((P + 63) / 64), (unsigned)E);
  hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, s,
                     static_cast<const uint16_t*>(in), P, Q, static_cast<uint16_t*>(out));
}

}  // namespace

void launch_seg_sched(const int32_t* offsets, int E, int32_t* rec, hipStream_t stream) {
  if (E <= 0 || E > 256) return;
  hipLaunchKernelGGL(seg_sched_kernel, dim3(1), dim3(256), 0, stream, offsets, E,
                     seg_sched_cap(E), rec);
}

void launch_layer_bwd(const BwdArgs& a, hipStream_t s) {
  const int64_t T = a.T, R = a.T * a.k;
  const int d = a.d, I = a.I, E = a.E;
  const bool bf = a.bf16;
  // products on the matrix cores (bf16 hi/lo parts), or on the VALU in fp32
  // (the caller's choice, for comparisons of the two)
  const bool mf = !a.valu;
  const int tt = mf ? MT : GT;
  // M-tile prefix of the experts' row segments, and (bf16 layers with shared
  // experts) the one- and two-segment tables of the shared experts' products
  const bool shtab = bf && a.ns > 0;
  launch_segment_tables(a.offsets, E, tt, a.prefix, T, shtab ? a.off1 : nullptr, a.poff1,
                        a.tiles1, a.off2, a.tiles2, a.ctr, s);
  const int64_t mt_bound = (R + (int64_t)E * (tt - 1)) / tt;

  auto ragged_m = [&](const void* A, bool ab, int64_t a_sm, const void* B, bool bb, int64_t b_sk,
                      int64_t b_sn, int64_t b_g, float* C, int64_t c_sm, int N, int K, bool acc) {
    GemmOp o = {A, ab, a_sm, 1, 0, B, bb, b_sk, b_sn, b_g, C, c_sm, 1, 0, a.offsets, a.prefix,
                E, 0, mt_bound, 0, N, K, false, acc, mf};
    launch_gemm(o, s);
  };
  auto ragged_k = [&](const void* A, bool ab, int64_t a_sk, const void* B, bool bb, int64_t b_sk,
                      float* C, int64_t c_sm, int64_t c_g, int M, int N) {
    GemmOp o = {A, ab, 1, a_sk, 0, B, bb, b_sk, 1, 0, C, c_sm, 1, c_g, a.offsets, nullptr,
                E, 0, 0, M, N, 0, true, false, mf};
    launch_gemm(o, s);
  };

  // forward recompute: G, U, the rounded SwiGLU product and the expert outputs.
  // bf16 layers run them on the forward pass's own grouped GEMMs (G and U
  // stored raw, then the down product of the bf16 SwiGLU rows).
  const int64_t nRI = R * I;
  if (bf) {
    FfnArgs f = {};
    f.xs = a.xs;
    f.perm = a.perm;
    f.k = a.k;
    f.x = a.x;
    f.wg = a.wg;
    f.wu = a.wu;
    f.wd = a.wd;
    f.offsets = a.offsets;
    f.tile_off = a.tile_off;
    f.ctr = a.ctr;
    f.a = a.G;
    f.u_raw = a.U;
    f.a_bf16 = a.Abf;
    f.T = T;
    f.R = R;
    f.d = d;
    f.E = E;
    f.I = I;
    f.bf16 = true;
    f.part = kRoutedTiles;
    f.force_global = a.force_global;
    launch_gate_up_raw_bf16(f, s);  // G, U and the bf16 A
  } else {
    ragged_m(a.xs, bf, d, a.wg, bf, 1, d, (int64_t)I * d, a.G, I, I, d, false);
    ragged_m(a.xs, bf, d, a.wu, bf, 1, d, (int64_t)I * d, a.U, I, I, d, false);
    hipLaunchKernelGGL(swiglu_fwd_kernel, dim3(ew_grid(nRI)), dim3(256), 0, s, a.G, a.U, nRI, 0,
                       a.Ar, nullptr);
    ragged_m(a.Ar, false, I, a.wd, bf, 1, I, (int64_t)d * I, a.y, d, d, I, false);
  }
  // dY, dw, the gate's logit gradient.  bf16 layers take dw later, as the
  // row dot product of A with the unweighted dA' = dout W_d (no expert
  // outputs y needed); they form no dY but the hi/lo parts of dout's token
  // rows, which the products gather through perm.
  if (bf) {
    launch_split_rows(a.dout, T, d, a.dOp, 2 * (int64_t)d, 0, d, s);
  } else {
    hipLaunchKernelGGL(bwd_rows_kernel, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, s, a.dout,
                       a.y, a.perm, a.w, (int)R, a.k, d, a.dY, a.dw);
    hipLaunchKernelGGL(bwd_gate_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, s, a.w,
                       a.dw, a.inv, (int)T, a.k, a.dl, a.dls);
  }
  // bf16 layers run the input-gradient products dA = dY W_d[e] and
  // dX = dG W_g[e] + dU W_u[e] on the forward down kernel with the fp32
  // operand split into bf16 hi and lo rows; the kernel reads the weights in
  // their stored layout (W_d [d,I], W_g and W_u [I,d]: the reduction index
  // outer) and forms their MFMA fragments with transposing LDS reads.
  FfnArgs fd = {};
  if (bf) {
    fd.offsets = a.offsets;
    fd.tile_off = a.tile_off;
    fd.ctr = a.ctr;
    fd.T = T;
    fd.R = R;
    fd.E = E;
    fd.bf16 = true;
    fd.part = kRoutedTiles;
    fd.force_global = a.force_global;
  }
  // out = sum over the `parts` K blocks of A's rows (K columns each) of block
  // b times weight block b / 2 (w for block 0, w2 for block 1), the weights
  // [E, K, N]: one launch of the down kernel, which reduces over its K and
  // writes N columns (rows_perm: A holds token rows, sorted row r reading
  // token row rows_perm[r] / k)
  auto down_parts = [&](const uint16_t* A, int parts, const void* w, const void* w2, int K, int N,
                        float* out, const int32_t* rows_perm) {
    fd.perm = rows_perm;
    fd.k = a.k;
    fd.wd = w;
    fd.wd2 = w2;
    fd.wt = true;
    fd.I = K;
    fd.d = N;
    fd.y = out;
    fd.a = const_cast<uint16_t*>(A);
    fd.a_parts = parts;
    fd.w_part = 0;
    launch_down_routed_bf16(fd, s);
  };

  // dA = dY W_d[e] (bf16 layers: dA' = dout W_d[e], the gate weight applied
  // in the SwiGLU backward); dW_d[e] = dY_e^T A_e
  if (bf) {
    down_parts(a.dOp, 2, a.wd, nullptr, d, I, a.dA, a.perm);
  } else {
    ragged_m(a.dY, false, d, a.wd, bf, I, 1, (int64_t)d * I, a.dA, I, I, d, false);
  }
  // weight gradients.  bf16 layers: the operands transposed into per-expert
  // zero-padded parts (an fp32 operand as its hi half then its lo half, the
  // bf16 one twice), then one product per weight on the forward tile loop.
  // With the buffer loads, the routed weight gradients read their operands in
  // row layout (the gate-weighted dout rows formed once as hi and lo parts,
  // in tA); otherwise through the transposed, zero-padded parts.
  const bool km = bf && !a.force_global &&
                  seg_gemm_km_fits(SegKmArgs{nullptr, std::max<int64_t>(4 * (int64_t)I, 2 * (int64_t)d),
                                             0, nullptr, std::max<int64_t>(I, d), nullptr, nullptr,
                                             E, 0, 0},
                                   R);
  if (km) {
    // the gathered dout rows, and (block 0 of the same launch) the schedule
    // of the weight-gradient tiles: all tiles of an expert on one XCD, the
    // experts spread over the XCDs by cost (a tile's K loop runs over its
    // expert's rows)
    if (R > 0)
      hipLaunchKernelGGL(gather_split_rows_kernel, dim3((unsigned)std::min<int64_t>(R, 16384) + 1),
                         dim3(256), 0, s, a.dout, a.perm, a.w, a.k, R, d, a.tA, a.offsets, E,
                         a.srec);
    else
      launch_seg_sched(a.offsets, E, a.srec, s);
    launch_seg_gemm_km_bf16(SegKmArgs{a.tA, 2 * (int64_t)d, d, a.Abf, I, a.offsets, a.dw_down, E,
                                      d, I, 0, a.srec, seg_sched_cap(E)},
                            s);
  } else if (bf) {
    hipLaunchKernelGGL(seg_offsets_kernel, dim3(1), dim3(64), 0, s, a.offsets, E, a.poff);
    launch_seg_transpose_gather(a.dout, d, a.perm, a.w, a.k, a.offsets, a.poff, E, a.seg_ld,
                                a.tA, s);
    launch_seg_transpose(a.Abf, false, I, a.offsets, a.poff, E, a.seg_ld, a.tB, s);
    SegGemmArgs sg = {a.tA, a.tB, a.seg_ld, a.poff, a.dw_down, E, d, I};
    launch_seg_gemm_bf16(sg, s);
  } else {
    ragged_k(a.dY, false, d, a.Ar, false, I, a.dw_down, I, (int64_t)d * I, d, I);
  }
  // dG, dU (bf16 layers: as the hi/lo rows of dGU; fp32: in place of G, U);
  // dW_g, dW_u; dXs = dG W_g[e] + dU W_u[e]
  if (bf) {
    if (R > 0)
      hipLaunchKernelGGL(swiglu_bwd_rows_kernel, dim3((unsigned)R), dim3(256), 0, s, a.G, a.U,
                         a.dA, a.Abf, a.perm, a.w, I, a.dw, a.dGU);
    hipLaunchKernelGGL(bwd_gate_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, s, a.w,
                       a.dw, a.inv, (int)T, a.k, a.dl, a.dls);
  } else {
    hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(ew_grid(nRI)), dim3(256), 0, s, a.G, a.U, a.dA,
                       nRI);
  }
  if (km) {  // dGU rows: dG hi, dG lo, dU hi, dU lo
    const int64_t ld4 = 4 * (int64_t)I;
    launch_seg_gemm_km_bf16(SegKmArgs{a.dGU, ld4, I, static_cast<const uint16_t*>(a.xs), d,
                                      a.offsets, a.dw_gate, E, I, d, 0, a.srec, seg_sched_cap(E)},
                            s);
    launch_seg_gemm_km_bf16(SegKmArgs{a.dGU + 2 * (size_t)I, ld4, I,
                                      static_cast<const uint16_t*>(a.xs), d, a.offsets, a.dw_up, E,
                                      I, d, 0, a.srec, seg_sched_cap(E)},
                            s);
  } else if (bf) {
    launch_seg_transpose(a.xs, false, d, a.offsets, a.poff, E, a.seg_ld, a.tB, s);
    const int64_t ld4 = 4 * (int64_t)I;  // dGU rows: dG hi, dG lo, dU hi, dU lo
    launch_seg_transpose(a.dGU, false, I, a.offsets, a.poff, E, a.seg_ld, a.tA, s, ld4, I);
    SegGemmArgs sg = {a.tA, a.tB, a.seg_ld, a.poff, a.dw_gate, E, I, d};
    launch_seg_gemm_bf16(sg, s);
    launch_seg_transpose(a.dGU + 2 * (size_t)I, false, I, a.offsets, a.poff, E, a.seg_ld, a.tA, s,
                         ld4, I);
    sg.out = a.dw_up;
    launch_seg_gemm_bf16(sg, s);
  } else {
    ragged_k(a.G, false, I, a.xs, bf, d, a.dw_gate, d, (int64_t)I * d, I, d);
    ragged_k(a.U, false, I, a.xs, bf, d, a.dw_up, d, (int64_t)I * d, I, d);
  }
  if (bf) {
    down_parts(a.dGU, 4, a.wg, a.wu, I, d, a.dXs, nullptr);
  } else {
    ragged_m(a.G, false, I, a.wg, bf, d, 1, (int64_t)I * d, a.dXs, d, d, I, false);
    ragged_m(a.U, false, I, a.wu, bf, d, 1, (int64_t)I * d, a.dXs, d, d, I, true);
  }

  // shared experts on all T rows with weight 1; their G, U and products sit
  // side by side in [T, ns*Is] arrays (expert s in columns s*Is ..)
  const int Is = a.Is, ns = a.ns;
  const int64_t ld = (int64_t)ns * Is;
  auto uni_m = [&](const void* A, bool ab, int64_t a_sm, const void* B, bool bb, int64_t b_sk,
                   int64_t b_sn, float* C, int64_t c_sm, int N, int K, bool acc) {
    GemmOp o = {A, ab, a_sm, 1, 0, B, bb, b_sk, b_sn, 0, C, c_sm, 1, 0, nullptr, nullptr,
                1, (int)T, (T + tt - 1) / tt, 0, N, K, false, acc, mf};
    launch_gemm(o, s);
  };
  auto uni_k = [&](const void* A, bool ab, int64_t a_sk, const void* B, bool bb, int64_t b_sk,
                   float* C, int64_t c_sm, int M, int N) {
    GemmOp o = {A, ab, 1, a_sk, 0, B, bb, b_sk, 1, 0, C, c_sm, 1, 0, nullptr, nullptr,
                1, (int)T, 0, M, N, 0, true, false, mf};
    launch_gemm(o, s);
  };
  auto wslice = [&](const void* w, int sh) -> const void* {
    const size_t wo = (size_t)sh * Is * d;
    return bf ? (const void*)(static_cast<const uint16_t*>(w) + wo)
              : (const void*)(static_cast<const float*>(w) + wo);
  };
  if (ns > 0) {
    const int64_t nT = T * ld;
    if (bf) {
      FfnArgs f = {};
      f.x = a.x;
      f.wsg = a.wsg;
      f.wsu = a.wsu;
      f.tile_off = a.tile_off;
      f.ctr = a.ctr;
      f.a = a.Gs;
      f.u_raw = a.Us;
      f.a_bf16 = a.Asbf;
      f.T = T;
      f.R = R;
      f.d = d;
      f.E = E;
      f.I = I;
      f.ns = ns;
      f.Is = Is;
      f.bf16 = true;
      f.part = kSharedTiles;
      f.force_global = a.force_global;
      launch_gate_up_raw_bf16(f, s);
    } else {
      for (int sh = 0; sh < ns; ++sh) {
        uni_m(a.x, bf, d, wslice(a.wsg, sh), bf, 1, d, a.Gs + (size_t)sh * Is, ld, Is, d, false);
        uni_m(a.x, bf, d, wslice(a.wsu, sh), bf, 1, d, a.Us + (size_t)sh * Is, ld, Is, d, false);
      }
    }
    if (!bf)  // bf16 layers have A_s from the gate/up epilogue
      hipLaunchKernelGGL(swiglu_fwd_kernel, dim3(ew_grid(nT)), dim3(256), 0, s, a.Gs, a.Us, nT, 0,
                         a.As, nullptr);
    // dA_s = dout W_sd[s]; dW_sd[s] = dout^T A_s.  bf16 layers take the
    // weight gradients on the forward tile loop with the T rows as one
    // segment (dout and the shared experts' tensors transposed once each),
    // and the input-gradient products of all shared experts at once on the
    // forward down kernel: dA_all = dout [W_sd[0] | W_sd[1] | ..] and
    // dx_shared = [dG_0 | dG_1 | ..] [W_sg[0]; W_sg[1]; ..] + the same for U,
    // with the weights transposed and dout, dG, dU as bf16 hi and lo rows.
    FfnArgs f1 = {};
    auto down1 = [&](const uint16_t* A, int parts, const uint16_t* wT, int64_t w_part, int K,
                     int N, float* out) {
      f1.wd = wT;
      f1.I = K;
      f1.d = N;
      f1.y = out;
      f1.a = const_cast<uint16_t*>(A);
      f1.a_parts = parts;
      f1.w_part = w_part;
      launch_down_routed_bf16(f1, s);
    };
    if (bf) {
      f1.offsets = a.off1;
      f1.tile_off = a.tiles1;
      f1.ctr = a.ctr;
      f1.T = T;
      f1.R = T;
      f1.E = 1;
      f1.bf16 = true;
      f1.part = kRoutedTiles;
      f1.force_global = a.force_global;
      launch_transpose_bf16(a.wsd, ns, d, Is, a.wsdT, s);        // [ns*Is, d]
      launch_transpose_bf16(a.wsg, 1, (int)ld, d, a.wsgT, s);    // [d, ns*Is]
      launch_transpose_bf16(a.wsu, 1, (int)ld, d, a.wsuT, s);
      down1(a.dOp, 2, a.wsdT, 0, d, (int)ld, a.dAs);  // dOp: formed for the routed part
    } else {
      for (int sh = 0; sh < ns; ++sh)
        uni_m(a.dout, false, d, wslice(a.wsd, sh), bf, Is, 1, a.dAs + (size_t)sh * Is, ld, Is, d,
              false);
    }
    // A shared expert's weight gradient has few 256x256 tiles and a long
    // reduction (all T rows): with ksplit > 1 the reduction is cut into
    // ksplit slices, each slice's product goes to its own slab of kpart, and
    // the slabs are added in slice order.
    auto seg1 = [&](const uint16_t* A_, const uint16_t* B_, float* out, int M, int N) {
      if (a.ksplit > 1) {
        SegGemmArgs g1 = {A_, B_, a.seg_ld, a.poffS, a.kpart, a.ksplit, M, N};
        launch_seg_gemm_bf16(g1, s);
        const int64_t n = (int64_t)M * N;
        hipLaunchKernelGGL(sum_slices_kernel, dim3(ew_grid(n / 4)), dim3(256), 0, s, a.kpart,
                           a.ksplit, n, out);
      } else {
        SegGemmArgs g1 = {A_, B_, a.seg_ld, a.poff1, out, 1, M, N};
        launch_seg_gemm_bf16(g1, s);
      }
    };
    // the same product from row-layout operands (one segment of T rows,
    // the same K-step slices, so the same sums)
    const bool kms = km && seg_gemm_km_fits(SegKmArgs{nullptr, 2 * std::max<int64_t>(ld, d), 0,
                                                      nullptr, std::max<int64_t>(ld, d), nullptr,
                                                      nullptr, 1, 0, 0, 0},
                                            T);
    auto seg1_km = [&](const uint16_t* X_, int64_t x_ld, int64_t x_part, const uint16_t* W_,
                       int64_t w_ld, float* out, int M, int N) {
      const int S = a.ksplit > 1 ? a.ksplit : 1;
      launch_seg_gemm_km_bf16(
          SegKmArgs{X_, x_ld, x_part, W_, w_ld, a.off1, S > 1 ? a.kpart : out, S, M, N, S}, s);
      if (S > 1) {
        const int64_t n = (int64_t)M * N;
        hipLaunchKernelGGL(sum_slices_kernel, dim3(ew_grid(n / 4)), dim3(256), 0, s, a.kpart, S,
                           n, out);
      }
    };
    if (kms) {  // dOp: dout's hi and lo parts, formed for the routed part
      for (int sh = 0; sh < ns; ++sh)
        seg1_km(a.dOp, 2 * (int64_t)d, d, a.Asbf + (size_t)sh * Is, ld,
                a.dwsh_down + (size_t)sh * d * Is, d, Is);
    } else if (bf) {
      if (a.ksplit > 1)
        hipLaunchKernelGGL(split_seg_offsets_kernel, dim3(1), dim3(64), 0, s, (int)T, a.ksplit,
                           a.poffS);
      launch_seg_transpose(a.dout, true, d, a.off1, a.poff1, 1, a.seg_ld, a.tA, s);
      launch_seg_transpose(a.Asbf, false, (int)ld, a.off1, a.poff1, 1, a.seg_ld, a.tB, s);
      for (int sh = 0; sh < ns; ++sh)
        seg1(a.tA, a.tB + (size_t)sh * Is * a.seg_ld, a.dwsh_down + (size_t)sh * d * Is, d, Is);
    } else {
      for (int sh = 0; sh < ns; ++sh) {
        const size_t cs = (size_t)sh * Is;
        uni_k(a.dout, false, d, a.As + cs, false, ld, a.dwsh_down + cs * d, Is, d, Is);
      }
    }
    hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(ew_grid(nT)), dim3(256), 0, s, a.Gs, a.Us, a.dAs, nT);
    // sGU: rows 0..T-1 [dG_s hi | lo], rows T..2T-1 [dU_s hi | lo]
    if (bf) {
      launch_split_rows(a.Gs, T, (int)ld, a.sGU, 2 * ld, 0, (int)ld, s);
      launch_split_rows(a.Us, T, (int)ld, a.sGU + (size_t)T * 2 * ld, 2 * ld, 0, (int)ld, s);
    }
    if (kms) {
      const uint16_t* xb = static_cast<const uint16_t*>(a.x);
      for (int sh = 0; sh < ns; ++sh) {
        seg1_km(a.sGU + (size_t)sh * Is, 2 * ld, ld, xb, d, a.dwsh_gate + (size_t)sh * Is * d, Is, d);
        seg1_km(a.sGU + (size_t)T * 2 * ld + (size_t)sh * Is, 2 * ld, ld, xb, d,
                a.dwsh_up + (size_t)sh * Is * d, Is, d);
      }
    } else if (bf) {
      launch_seg_transpose(a.x, false, d, a.off1, a.poff1, 1, a.seg_ld, a.tB, s);
      launch_seg_transpose(a.Gs, true, (int)ld, a.off1, a.poff1, 1, a.seg_ld, a.tA, s);
      for (int sh = 0; sh < ns; ++sh)
        seg1(a.tA + (size_t)sh * Is * a.seg_ld, a.tB, a.dwsh_gate + (size_t)sh * Is * d, Is, d);
      launch_seg_transpose(a.Us, true, (int)ld, a.off1, a.poff1, 1, a.seg_ld, a.tA, s);
      for (int sh = 0; sh < ns; ++sh)
        seg1(a.tA + (size_t)sh * Is * a.seg_ld, a.tB, a.dwsh_up + (size_t)sh * Is * d, Is, d);
    } else {
      for (int sh = 0; sh < ns; ++sh) {
        const size_t cs = (size_t)sh * Is;
        uni_k(a.Gs + cs, false, ld, a.x, bf, d, a.dwsh_gate + cs * d, d, Is, d);
        uni_k(a.Us + cs, false, ld, a.x, bf, d, a.dwsh_up + cs * d, d, Is, d);
      }
    }
    if (bf) {
      // dxs = dG_s W_sg + dU_s W_su as two row groups of one launch (256
      // tiles rather than 128 for T = 4096): rows 0..T-1 of sGU hold
      // [dG_s hi | lo] against W_sg^T, rows T..2T-1 [dU_s hi | lo] against
      // W_su^T (the group-1 weight, d*ld elements after W_sg^T); their
      // products go to the two slabs of dxs, added in bwd_dx_kernel
      f1.offsets = a.off2;
      f1.tile_off = a.tiles2;
      f1.R = 2 * T;
      f1.E = 2;
      down1(a.sGU, 2, a.wsgT, 0, (int)ld, d, a.dxs);
    } else {
      for (int sh = 0; sh < ns; ++sh) {
        const size_t cs = (size_t)sh * Is;
        uni_m(a.Gs + cs, false, ld, wslice(a.wsg, sh), bf, d, 1, a.dxs, d, d, Is, sh > 0);
        uni_m(a.Us + cs, false, ld, wslice(a.wsu, sh), bf, d, 1, a.dxs, d, d, Is, true);
      }
    }
  }

  // router weights (dW_r[e] = dls_e^T X_e, one output row per expert) and
  // bias, then the token gradients
  if (mt_bound > 0) {
    const dim3 g1((unsigned)mt_bound, (unsigned)((d + 511) / 512));
    hipLaunchKernelGGL((bf ? router_grad_part_kernel<true> : router_grad_part_kernel<false>), g1,
                       dim3(256), 0, s, a.dls, a.xs, a.offsets, a.prefix, E, d, tt, a.rpart);
  }
  hipLaunchKernelGGL(router_grad_reduce_kernel, dim3((unsigned)E, (unsigned)((d + 1023) / 1024)),
                     dim3(256), 0, s, a.rpart, a.prefix, d, a.dw_router);
  if (a.dbias)
    hipLaunchKernelGGL(bwd_bias_kernel, dim3((unsigned)E), dim3(256), 0, s, a.dls, a.offsets,
                       a.dbias);
  hipLaunchKernelGGL((bf ? bwd_dx_kernel<true> : bwd_dx_kernel<false>),
                     dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, a.dXs, a.inv, a.ids, a.dl,
                     a.wr, a.ns ? a.dxs : nullptr, bf ? 2 : 1, (int)T, a.k, d, a.dx);
}

}  // namespace moe
