// Token condensation in the MoE layer: a routed assignment whose token is a
// near-duplicate of an earlier token routed to the same expert gets no row of
// its own and reuses that token's expert output.
//
// The method is Luffy's token condensation (Luffy review, "Core claim" and
// "What carries the argument": similar tokens bound for one expert send one
// representative, and its expert output is reused).  How similar tokens are
// found in one forward pass, and the similarity's normalisation, are
// readings (the pages' fast measurement relies on training history):
//   key:    16 bits per token, bit b set when the token's projection onto the
//           caller's hyperplane b is >= 0 (sign random projections); the
//           projections are the router kernel run with the hyperplanes as
//           its 16 "experts", so they cost one more pass over x on the
//           matrix cores;
//   bucket: tokens with equal keys, in ascending token order, from a stable
//           two-pass radix sort (low byte, then high byte) built from the
//           dispatch's stable counting sort with 256 buckets;
//   rep:    c(t) = the first of the bucket's first 32 members before t whose
//           cosine with t is >= h (else t); rep(t) = c(t) if c(c(t)) == c(t),
//           else t.  One wave per token, fp32 dot products;
//   use:    assignment (t, j) is condensed when rep(t) != t and rep(t) is
//           routed to the same expert; the dispatch gives it no row, and
//           afterwards its inv_perm entry is pointed at the row of rep(t)'s
//           assignment to that expert, so the GEMMs run on fewer rows and the
//           combine needs no change.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void condense_key_kernel(const float* __restrict__ proj, int T,
                                                           int32_t* __restrict__ key,
                                                           int32_t* __restrict__ key_lo) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  int k = 0;
#pragma unroll
  for (int b = 0; b < kCondenseBits; ++b)
    if (proj[(size_t)t * kCondenseBits + b] >= 0.0f) k |= 1 << b;  // -0.0 counts as >= 0
  key[t] = k;
  key_lo[t] = k & 255;
}

// Second radix pass: the high byte of the key of the token in position i
// after the first pass.
__global__ __launch_bounds__(256) void condense_key_hi_kernel(const int32_t* __restrict__ key,
                                                              const int32_t* __restrict__ perm1,
                                                              int T, int32_t* __restrict__ key_hi) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < T) key_hi[i] = key[perm1[i]] >> 8;
}

// Tokens in key order (ascending token within a key) and their keys.
__global__ __launch_bounds__(256) void condense_order_kernel(const int32_t* __restrict__ key,
                                                             const int32_t* __restrict__ perm1,
                                                             const int32_t* __restrict__ perm2,
                                                             int T, int32_t* __restrict__ tok,
                                                             int32_t* __restrict__ skey) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= T) return;
  const int t = perm1[perm2[i]];
  tok[i] = t;
  skey[i] = key[t];
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return __shfl(v, 0);  // lane 0's sum on every lane, so that decisions are wave-uniform
}

// 8 consecutive elements of a row as floats (bf16 or fp32 storage).
template <bool BF16>
__device__ __forceinline__ void load8(const void* row, int e, float (&v)[8]) {
  if (BF16) {
    const u32x4 u = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(row) + e);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(row) + e);
    const f32x4 b = *reinterpret_cast<const f32x4*>(static_cast<const float*>(row) + e + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
}

// c(t) for the token in sorted position i: one wave per position.
template <bool BF16>
__global__ __launch_bounds__(256) void condense_cand_kernel(const void* __restrict__ x, int d,
                                                            const int32_t* __restrict__ tok,
                                                            const int32_t* __restrict__ skey, int T,
                                                            float h, int32_t* __restrict__ cand) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + wave;
  if (i >= T) return;
  const int p = tok[i], K = skey[i];
  // first position of key K (skey is ascending and skey[i] == K): most buckets
  // hold a few tokens, so step back up to 32 positions, then binary search
  int lo = i;
  for (int s = 0; s < 32 && lo > 0 && skey[lo - 1] == K; ++s) --lo;
  if (lo > 0 && skey[lo - 1] == K) {
    int a = 0, b = lo - 1;  // skey[b] == K
    while (a < b) {
      const int mid = (a + b) >> 1;
      if (skey[mid] < K) a = mid + 1;
      else b = mid;
    }
    lo = a;
  }
  const size_t es = BF16 ? 2 : 4;
  const uint8_t* xp = static_cast<const uint8_t*>(x) + (size_t)p * d * es;
  int c = p;
  const int end = min(i, lo + kCondenseCandidates);
  for (int j = lo; j < end; ++j) {
    const int q = tok[j];
    const uint8_t* xq = static_cast<const uint8_t*>(x) + (size_t)q * d * es;
    float dot = 0.f, np = 0.f, nq = 0.f;
    for (int e = lane * 8; e < d; e += 512) {
      float a[8], b[8];
      load8<BF16>(xp, e, a);
      load8<BF16>(xq, e, b);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        dot = fmaf(a[u], b[u], dot);
        np = fmaf(a[u], a[u], np);
        nq = fmaf(b[u], b[u], nq);
      }
    }
    dot = wave_sum(dot);
    np = wave_sum(np);
    nq = wave_sum(nq);
    if (np > 0.f && nq > 0.f && dot >= h * (sqrtf(np) * sqrtf(nq))) {  // wave-uniform
      c = q;
      break;
    }
  }
  if (lane == 0) cand[p] = c;
}

// The chain cut: a token whose candidate is itself condensed stays.
__global__ __launch_bounds__(256) void condense_rep_kernel(const int32_t* __restrict__ cand, int T,
                                                           int32_t* __restrict__ rep) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  const int c = cand[t];
  rep[t] = cand[c] == c ? c : t;
}

// A condensed assignment reads the row of its source: the assignment of
// rep(t) to the same expert (rep(t) itself is never condensed).
__global__ __launch_bounds__(256) void condense_inv_kernel(const int32_t* __restrict__ ids,
                                                           const int32_t* __restrict__ rep, int R,
                                                           int k, int32_t* __restrict__ inv) {
  const int a = blockIdx.x * 256 + threadIdx.x;
  if (a >= R) return;
  const int t = a / k, r = rep[t];
  if (r == t) return;
  const int e = ids[a];
  for (int j = 0; j < k; ++j)
    if (ids[(size_t)r * k + j] == e) {
      inv[a] = inv[(size_t)r * k + j];
      return;
    }
}

}  // namespace

void launch_condense(const CondenseArgs& a, hipStream_t stream) {
  const int T = (int)a.T;
  if (T == 0) return;
  const dim3 block(256);
  const unsigned g1 = (unsigned)((T + 255) / 256);
  // projections onto the hyperplanes: the router with 16 "experts", top-1
  RouteArgs ra = {a.x, a.hyperplanes, nullptr, nullptr, a.proj, a.pids, a.pwts, a.T, a.d,
                  kCondenseBits, 1, a.bf16};
  launch_route(ra, stream);
  hipLaunchKernelGGL(condense_key_kernel, dim3(g1), block, 0, stream, a.proj, T, a.key, a.key_lo);
  // stable LSD radix sort of the 16-bit keys: low byte, then high byte
  DispatchArgs d1 = {nullptr, a.key_lo, nullptr, a.off1, nullptr, nullptr, a.perm1, a.inv1,
                     nullptr, a.blk, a.T, 0, 256, 1, 0, nullptr};
  launch_dispatch(d1, stream);
  hipLaunchKernelGGL(condense_key_hi_kernel, dim3(g1), block, 0, stream, a.key, a.perm1, T,
                     a.key_hi);
  DispatchArgs d2 = {nullptr, a.key_hi, nullptr, a.off2, nullptr, nullptr, a.perm2, a.inv2,
                     nullptr, a.blk, a.T, 0, 256, 1, 0, nullptr};
  launch_dispatch(d2, stream);
  hipLaunchKernelGGL(condense_order_kernel, dim3(g1), block, 0, stream, a.key, a.perm1, a.perm2, T,
                     a.tok, a.skey);
  const unsigned gw = (unsigned)((T + 3) / 4);
  if (a.bf16)
    hipLaunchKernelGGL(condense_cand_kernel<true>, dim3(gw), block, 0, stream, a.x, a.d, a.tok,
                       a.skey, T, a.cos_threshold, a.cand);
  else
    hipLaunchKernelGGL(condense_cand_kernel<false>, dim3(gw), block, 0, stream, a.x, a.d, a.tok,
                       a.skey, T, a.cos_threshold, a.cand);
  hipLaunchKernelGGL(condense_rep_kernel, dim3(g1), block, 0, stream, a.cand, T, a.rep);
}

void launch_condense_inv(const int32_t* ids, const int32_t* rep, int64_t R, int k, int32_t* inv,
                         hipStream_t stream) {
  if (R == 0) return;
  hipLaunchKernelGGL(condense_inv_kernel, dim3((unsigned)((R + 255) / 256)), dim3(256), 0, stream,
                     ids, rep, (int)R, k, inv);
}

}  // namespace moe
