// Gate of the MoE layer: router logits, top-k with lowest-index tie-break,
// renormalised softmax weights.
//
// Top-k routing over the router's scores is the gate the expert-prototyping
// abstract of the "Daily Papers" search page speaks of (k experts activated
// per token); it is the T_gate term of the overlap window in the
// FarSkip-Collective review (axiom ledger, Eq. 9).  Softmax, renormalisation
// over the kept k and the tie rule are readings: the pages name none of them.
//
// bf16 logits run on the matrix cores, eight waves splitting the hidden
// dimension, each wave holding its tokens x E experts of fp32 partial sums;
// the partials meet in LDS in a fixed order.  Two kernels:
//   * one block per 16, 32 or 64 tokens, the waves taking pairs of K-steps of
//     32 round-robin (in an order rotated per block) and reading both x and
//     W_r as they go;
//   * for inputs with more 16-token groups than the GPU has CUs (and up to 64
//     experts, d a power of two from 256 to 2048), one block per CU that keeps
//     its share of W_r in registers and walks 16-token groups, loading the
//     next group's x rows while the current one is reduced and routed.
// fp32 logits run on the vector ALUs in a fixed lane order.  The top-k then
// takes one token per 16-lane row, each slot a row-wide arg-max through the
// VALU's cross-lane data-parallel moves.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

// Row-wide exchange within each group of 16 lanes on the VALU's data-parallel
// primitives: CTRL 0xB1 swaps neighbours (quad_perm 1,0,3,2), 0x4E swaps lane
// pairs (quad_perm 2,3,0,1), 0x141 mirrors each half row of 8, 0x140 mirrors
// the row of 16.  Applied in that order, a symmetric pairwise rule leaves
// every lane of the row with the row's result.
template <int CTRL>
__device__ __forceinline__ int row16_swap(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}

// Keep the larger of (bv, bi) and (ov, oi): larger value first, then the lower
// index; bi == kNone marks no candidate.  Bitwise logic and selects only, so
// the comparison compiles without branches.
constexpr int kNone = 0x7fffffff;
__device__ __forceinline__ void keep_better(float& bv, int& bi, float ov, int oi) {
  const bool take = (oi != kNone) & ((bi == kNone) | (ov > bv) | ((ov == bv) & (oi < bi)));
  bv = take ? ov : bv;
  bi = take ? oi : bi;
}

template <int CTRL>
__device__ __forceinline__ void row16_step(float& bv, int& bi) {
  const float ov = __int_as_float(row16_swap<CTRL>(__float_as_int(bv)));
  const int oi = row16_swap<CTRL>(bi);
  keep_better(bv, bi, ov, oi);
}

// Top-k of one token per 16-lane row.  The token's E logits sit in LDS at `L`;
// lane c of the row considers experts c, c+16, ... (ascending, so a strict '>'
// keeps the lowest index among equal values), and each slot is one row-wide
// arg-max; lane c keeps slot c.  All 16 lanes of a row call this together;
// `valid` false (a row past T) writes nothing.  Lane c < k writes slot c.
template <int NV>  // E <= 16 * NV
__device__ __forceinline__ void topk_row16(const float* L, int E, int k, bool valid,
                                           int32_t* __restrict__ ids_out,
                                           float* __restrict__ w_out) {
  const int c = threadIdx.x & 15;
  float v[NV];
  bool live[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = c + 16 * i;
    live[i] = e < E;
    v[i] = live[i] ? L[e] : 0.0f;
  }
  // w_j = exp(L_j - L_0) / sum_j' exp(L_j' - L_0): the softmax over all E
  // restricted to the kept k and renormalised (the full denominator cancels);
  // the sum runs over j in order in every lane.
  float v0 = 0.0f, s = 0.0f;
  float my_v = 0.0f;
  int my_i = 0;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {  // uniform across the row
      float bv = 0.0f;
      int bi = kNone;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const bool take = live[i] & ((bi == kNone) | (v[i] > bv));
        bv = take ? v[i] : bv;
        bi = take ? c + 16 * i : bi;
      }
      row16_step<0xB1>(bv, bi);
      row16_step<0x4E>(bv, bi);
      row16_step<0x141>(bv, bi);
      row16_step<0x140>(bv, bi);
      if (j == 0) v0 = bv;
      s += expf(bv - v0);
      my_v = c == j ? bv : my_v;
      my_i = c == j ? bi : my_i;
#pragma unroll
      for (int i = 0; i < NV; ++i) live[i] = live[i] & (bi != c + 16 * i);
    }
  }
  if (valid && c < k) {
    ids_out[c] = my_i;
    w_out[c] = expf(my_v - v0) / s;
  }
}

// Logits of 16 * NTT tokens x E experts, bf16 in, fp32 accumulate on the
// matrix cores.  Eight waves split the hidden dimension (pairs of K-steps of
// 32, one 128-byte line per row, dealt round-robin); each wave issues the
// loads of its next few K-steps before their MFMAs.  A block reads all of W_r once, so larger token blocks (NTT)
// cut the router-weight traffic on long inputs.
constexpr int kRouteWaves = 8;

// NET 16-expert column tiles (E <= 16 * NET); NTT 16-token row tiles; BP pairs
// of K-steps whose loads each wave has in flight at once (it only changes when
// loads are issued, not the order of the sums)
template <int NET, int NTT, int BP = (NTT >= 4 ? 1 : 2)>
__global__ __launch_bounds__(64 * kRouteWaves) void route_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int T, int d, int E, int k,
    float* __restrict__ logits_out, int32_t* __restrict__ ids, float* __restrict__ wts) {
  constexpr int TB = 16 * NTT;                  // tokens per block
  constexpr int EP = NET * 16 + 1;
  __shared__ float part[kRouteWaves][TB][EP];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * TB;
  const int r = lane & 15, kq = (lane >> 4) * 8;
  // rows past T and experts past E read a valid row; their results are dropped
  const uint16_t* xp[NTT];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) xp[tt] = x + (size_t)min(t0 + tt * 16 + r, T - 1) * d + kq;
  const uint16_t* wp[NET];
#pragma unroll
  for (int et = 0; et < NET; ++et) wp[et] = wr + (size_t)min(et * 16 + r, E - 1) * d + kq;

  f32x4 acc[NTT][NET];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
    for (int et = 0; et < NET; ++et) acc[tt][et] = f32x4{0.f, 0.f, 0.f, 0.f};
  // K-steps of 32 taken in pairs: a wave loads both 64-byte halves of each
  // row's 128-byte line back to back, so each line is fetched for one wave
  // rather than for two.  The pairs are rotated per block (blocks b, b+8, ...
  // share an XCD) so that the blocks of an XCD do not all read the same lines
  // of W_r at once.  The order of the products within each sum is fixed per
  // block, so results are reproducible.
  const int npair = d >> 6;
  const int rot = (int)((blockIdx.x >> 3) % (unsigned)npair);
  for (int p0 = wave; p0 < npair; p0 += kRouteWaves * BP) {
    u32x4 av[BP][NTT][2], bv[BP][NET][2];
#pragma unroll
    for (int u = 0; u < BP; ++u) {
      int pp = min(p0 + u * kRouteWaves, npair - 1) + rot;  // clamped pairs are not used
      if (pp >= npair) pp -= npair;
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
        av[u][tt][0] = ld_u32x4(xp[tt] + pp * 64);
        av[u][tt][1] = ld_u32x4(xp[tt] + pp * 64 + 32);
      }
#pragma unroll
      for (int et = 0; et < NET; ++et) {
        bv[u][et][0] = ld_u32x4(wp[et] + pp * 64);
        bv[u][et][1] = ld_u32x4(wp[et] + pp * 64 + 32);
      }
    }
#pragma unroll
    for (int u = 0; u < BP; ++u) {
      if (p0 + u * kRouteWaves < npair) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
            for (int et = 0; et < NET; ++et)
              acc[tt][et] = mfma_16x16x32_bf16(as_bf16x8(av[u][tt][h]), as_bf16x8(bv[u][et][h]), acc[tt][et]);
      }
    }
  }
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int q = 0; q < 4; ++q) part[wave][tt * 16 + (lane >> 4) * 4 + q][et * 16 + r] = acc[tt][et][q];
  __syncthreads();

  for (int idx = threadIdx.x; idx < TB * E; idx += 64 * kRouteWaves) {
    const int t = idx / E, e = idx - t * E;
    float v = part[0][t][e];
#pragma unroll
    for (int w = 1; w < kRouteWaves; ++w) v += part[w][t][e];
    if (bias) v += bias[e];
    part[0][t][e] = v;
    if (logits_out && t0 + t < T) logits_out[(size_t)(t0 + t) * E + e] = v;
  }
  __syncthreads();
  // one token per 16-lane row: 32 tokens per pass of the 8 waves
#pragma unroll
  for (int p0 = 0; p0 < TB; p0 += 4 * kRouteWaves) {
    const int t = p0 + wave * 4 + (lane >> 4);
    if (t < TB) {  // wave-uniform
      const size_t tg = (size_t)min(t0 + t, T - 1);
      topk_row16<NET>(&part[0][t][0], E, k, t0 + t < T, ids + tg * k, wts + tg * k);
    }
  }
}

// Barrier for LDS traffic only: waits for this wave's LDS accesses, not for
// its global loads, which stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Logits and top-k of 16-token groups by a grid of at most one block per CU
// that holds the router weights in registers: wave w keeps W_r's columns
// [w d/8, (w+1) d/8) of every expert as MFMA fragments, loaded once, and the
// block walks the groups g = blockIdx.x, blockIdx.x + gridDim.x, ...  A
// group's x rows are loaded while the group before it is reduced and routed
// (the barriers wait for LDS traffic only).  Each wave's partial sums over its
// columns meet in LDS in wave order, then the bias; two LDS buffers let a
// group's partials be written while the previous group's top-k still reads.
template <int NET, int KS>  // E <= 16 * NET; d == 256 * KS
__global__ __launch_bounds__(64 * kRouteWaves) void route_resident_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int T, int d, int E, int k,
    float* __restrict__ logits_out, int32_t* __restrict__ ids, float* __restrict__ wts) {
  constexpr int EP = NET * 16 + 1;
  constexpr int NR = (16 * 16 * NET + 64 * kRouteWaves - 1) / (64 * kRouteWaves);
  __shared__ float part[2][kRouteWaves][16][EP];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, kq = (lane >> 4) * 8;
  const int k0 = wave * (KS * 32) + kq;     // this wave's columns, plus the lane's 8
  const int ngroups = (T + 15) >> 4;
  if ((int)blockIdx.x >= ngroups) return;  // block-uniform
  // experts past E read a valid row; their results are dropped
  bf16x8 w[KS][NET];
#pragma unroll
  for (int et = 0; et < NET; ++et) {
    const uint16_t* wp = wr + (size_t)min(et * 16 + r, E - 1) * d + k0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) w[ks][et] = as_bf16x8(ld_u32x4(wp + ks * 32));
  }
  // the (token, expert) entries this thread sums: idx = tid + 512 j
  int rt[NR], re[NR];
  float rb[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int idx = (int)threadIdx.x + j * 64 * kRouteWaves;
    rt[j] = idx < 16 * E ? idx / E : -1;
    re[j] = idx < 16 * E ? idx - rt[j] * E : 0;
    rb[j] = (bias && rt[j] >= 0) ? bias[re[j]] : 0.0f;
  }
  auto load_x = [&](int g, bf16x8 (&xv)[KS]) {
    // rows past T read a valid row; their results are dropped
    const uint16_t* xp = x + (size_t)min(g * 16 + r, T - 1) * d + k0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) xv[ks] = as_bf16x8(ld_u32x4(xp + ks * 32));
    __builtin_amdgcn_sched_barrier(0);  // issue them here, before this group's products
  };
  auto group = [&](int g, int b, const bf16x8 (&xv)[KS]) {
    f32x4 acc[NET];
#pragma unroll
    for (int et = 0; et < NET; ++et) acc[et] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int et = 0; et < NET; ++et) acc[et] = mfma_16x16x32_bf16(xv[ks], w[ks][et], acc[et]);
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int q = 0; q < 4; ++q) part[b][wave][(lane >> 4) * 4 + q][et * 16 + r] = acc[et][q];
    lds_barrier();
    const int t0 = g * 16;
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      if (rt[j] >= 0) {
        const int t = rt[j], e = re[j];
        float pv[kRouteWaves];
#pragma unroll
        for (int w2 = 0; w2 < kRouteWaves; ++w2) pv[w2] = part[b][w2][t][e];
        float v = pv[0];
#pragma unroll
        for (int w2 = 1; w2 < kRouteWaves; ++w2) v += pv[w2];
        if (bias) v += rb[j];
        part[b][0][t][e] = v;
        if (logits_out && t0 + t < T) logits_out[(size_t)(t0 + t) * E + e] = v;
      }
    }
    lds_barrier();
    if (wave < 4) {  // one token per 16-lane row: waves 0..3 hold the group's 16 rows
      const int t = wave * 4 + (lane >> 4);
      const size_t tg = (size_t)min(t0 + t, T - 1);
      topk_row16<NET>(&part[b][0][t][0], E, k, t0 + t < T, ids + tg * k, wts + tg * k);
    }
    // the next group writes the other buffer; the one after passes that
    // group's first barrier, which every wave reaches only after this top-k
  };
  // Two groups per trip, so that the register buffers swap without copies.
  // The next group's loads are issued on every path (the last group of a
  // block reads its own rows again, from cache), so the wait before a
  // group's products leaves exactly the next group's loads in flight.
  bf16x8 xa[KS], xb[KS];
  int g = blockIdx.x;
  load_x(g, xa);
  for (;;) {
    int gn = g + (int)gridDim.x;
    load_x(gn < ngroups ? gn : g, xb);
    group(g, 0, xa);
    if (gn >= ngroups) break;
    g = gn;
    gn = g + (int)gridDim.x;
    load_x(gn < ngroups ? gn : g, xa);
    group(g, 1, xb);
    if (gn >= ngroups) break;
    g = gn;
  }
}

// fp32 logits on the vector ALUs in a fixed order: lane l sums the rounded
// products of i = l, l+64, ... in ascending i (no fused multiply-add), a xor
// butterfly over 32..1 combines the 64 partials, then the bias is added.
__global__ __launch_bounds__(256) void route_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    int T, int d, int E, int k, float* __restrict__ logits_out, int32_t* __restrict__ ids,
    float* __restrict__ wts) {
  __shared__ float Ls[kRouteTokens][257];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * kRouteTokens;
#pragma unroll 1
  for (int q = 0; q < 4; ++q) {
    const int t = t0 + wave * 4 + q;
    if (t >= T) break;
    const float* xr = x + (size_t)t * d;
#pragma unroll 1
    for (int e = 0; e < E; ++e) {
      const float* w = wr + (size_t)e * d;
      float s = 0.0f;
      {
        // separate multiply and add: no fused multiply-add in this order
#pragma clang fp contract(off)
        for (int i = lane; i < d; i += 64) {
          const float p = xr[i] * w[i];
          s = s + p;
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) s = s + __shfl_xor(s, m);
        if (bias) s = s + bias[e];
      }
      if (lane == 0) Ls[wave * 4 + q][e] = s;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < kRouteTokens * E; idx += 256) {
    const int t = idx / E, e = idx - t * E;
    if (logits_out && t0 + t < T) logits_out[(size_t)(t0 + t) * E + e] = Ls[t][e];
  }
  {  // one token per 16-lane row: 4 waves x 4 rows = the block's 16 tokens
    const int t = wave * 4 + (lane >> 4);
    const size_t tg = (size_t)min(t0 + t, T - 1);
    topk_row16<16>(&Ls[t][0], E, k, t0 + t < T, ids + tg * k, wts + tg * k);
  }
}

// Top-k on logits given from outside.
__global__ __launch_bounds__(256) void route_from_logits_kernel(
    const float* __restrict__ logits_in, int T, int E, int k, float* __restrict__ logits_out,
    int32_t* __restrict__ ids, float* __restrict__ wts) {
  __shared__ float Ls[kRouteTokens][257];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * kRouteTokens;
  for (int idx = threadIdx.x; idx < kRouteTokens * E; idx += 256) {
    const int t = idx / E, e = idx - t * E;
    if (t0 + t < T) {
      const float v = logits_in[(size_t)(t0 + t) * E + e];
      Ls[t][e] = v;
      if (logits_out) logits_out[(size_t)(t0 + t) * E + e] = v;
    }
  }
  __syncthreads();
  {  // one token per 16-lane row: 4 waves x 4 rows = the block's 16 tokens
    const int t = wave * 4 + (lane >> 4);
    const size_t tg = (size_t)min(t0 + t, T - 1);
    topk_row16<16>(&Ls[t][0], E, k, t0 + t < T, ids + tg * k, wts + tg * k);
  }
}

void launch_route(const RouteArgs& a, hipStream_t stream) {
  const int grid = (int)((a.T + kRouteTokens - 1) / kRouteTokens);
  if (grid == 0) return;
  const dim3 block(256);
  if (a.logits_in) {
    hipLaunchKernelGGL(route_from_logits_kernel, dim3(grid), block, 0, stream, a.logits_in,
                       (int)a.T, a.E, a.k, a.logits_out, a.ids, a.wts);
    return;
  }
  if (!a.bf16) {
    hipLaunchKernelGGL(route_f32_kernel, dim3(grid), block, 0, stream,
                       static_cast<const float*>(a.x), static_cast<const float*>(a.wr), a.bias,
                       (int)a.T, a.d, a.E, a.k, a.logits_out, a.ids, a.wts);
    return;
  }
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* wr = static_cast<const uint16_t*>(a.wr);
  const int ngroups = (int)((a.T + 15) / 16);
  // router weights held in registers: up to 64 experts, d / 256 K-steps of 32
  // per wave within the register budget of two waves per SIMD
  const int n_cu = device_cu_count();
  if (ngroups > n_cu && a.E <= 64 && (a.d == 256 || a.d == 512 || a.d == 1024 || a.d == 2048)) {
    const int grid_r = n_cu;
#define MOE_ROUTE_RES(N, K)                                                                      \
  hipLaunchKernelGGL((route_resident_bf16_kernel<N, K>), dim3(grid_r), dim3(64 * kRouteWaves), 0, \
                     stream, x, wr, a.bias, (int)a.T, a.d, a.E, a.k, a.logits_out, a.ids, a.wts)
#define MOE_ROUTE_RES_D(N)            \
  if (a.d == 256) MOE_ROUTE_RES(N, 1); \
  else if (a.d == 512) MOE_ROUTE_RES(N, 2); \
  else if (a.d == 1024) MOE_ROUTE_RES(N, 4); \
  else MOE_ROUTE_RES(N, 8)
    if (a.E <= 16) { MOE_ROUTE_RES_D(1); }
    else if (a.E <= 32) { MOE_ROUTE_RES_D(2); }
    else { MOE_ROUTE_RES_D(4); }
    return;
#undef MOE_ROUTE_RES_D
#undef MOE_ROUTE_RES
  }
  // tokens per block: 16 while that still gives a block per CU, more on long
  // inputs (each block reads all of W_r), within the LDS of the partial sums
  // (for up to 64 experts a block of 16 tokens keeps all of a wave's K-step
  // pairs in flight at once for d = 2048, which measured fastest; the larger
  // token blocks keep fewer)
  const int net = a.E <= 16 ? 1 : a.E <= 32 ? 2 : a.E <= 64 ? 4 : a.E <= 128 ? 8 : 16;
  int ntt = a.T <= 4096 ? 1 : a.T <= 16384 ? 2 : 4;
  if (net == 8) ntt = ntt < 2 ? ntt : 2;
  if (net == 16) ntt = 1;
  const int grid_tb = (int)((a.T + 16 * ntt - 1) / (16 * ntt));
#define MOE_ROUTE_CASE(N, M, B)                                                                     \
  hipLaunchKernelGGL((route_bf16_kernel<N, M, B>), dim3(grid_tb), dim3(64 * kRouteWaves), 0, stream, \
                     x, wr, a.bias, (int)a.T, a.d, a.E, a.k, a.logits_out, a.ids, a.wts)
#define MOE_ROUTE_NTT(N)                      \
  if (ntt == 1) MOE_ROUTE_CASE(N, 1, N == 4 ? 4 : 2); \
  else if (ntt == 2) MOE_ROUTE_CASE(N, 2, 2); \
  else MOE_ROUTE_CASE(N, 4, 1)
  if (net == 1) { MOE_ROUTE_NTT(1); }
  else if (net == 2) { MOE_ROUTE_NTT(2); }
  else if (net == 4) { MOE_ROUTE_NTT(4); }
  else if (net == 8) {
    if (ntt == 1) MOE_ROUTE_CASE(8, 1, 2);
    else MOE_ROUTE_CASE(8, 2, 2);
  } else MOE_ROUTE_CASE(16, 1, 2);
#undef MOE_ROUTE_NTT
#undef MOE_ROUTE_CASE
}

}  // namespace moe
