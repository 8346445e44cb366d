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
//   * for up to 64 experts and d a power of two from 256 to 2048: one block
//     per 16-token group, up to one per CU, that keeps its share of W_r in
//     registers (loaded once, through LDS in whole cache lines) and walks
//     the groups, loading the next group's x rows while the current one is
//     reduced and routed;
//   * otherwise one block per 16, 32 or 64 tokens, the waves taking pairs of
//     K-steps of 32 round-robin (in an order rotated per block) and reading
//     both x and W_r as they go.
// fp32 logits run on the vector ALUs in a fixed lane order.  The top-k then
// takes one token per 16-lane row, each slot a row-wide max of the logits'
// integer images, then a row-wide min of the indices holding it, through the
// VALU's cross-lane data-parallel moves.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

// Row-wide reductions within each group of 16 lanes on the VALU's
// data-parallel moves: CTRL 0xB1 swaps neighbours (quad_perm 1,0,3,2), 0x4E
// swaps lane pairs (quad_perm 2,3,0,1), 0x141 mirrors each half row of 8,
// 0x140 mirrors the row of 16.  Combining each lane with its partner in that
// order leaves every lane of the row with the row's max (or min).
template <int CTRL>
__device__ __forceinline__ int row16_partner(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ int row16_max(int v) {
  v = max(v, row16_partner<0xB1>(v));
  v = max(v, row16_partner<0x4E>(v));
  v = max(v, row16_partner<0x141>(v));
  return max(v, row16_partner<0x140>(v));
}
__device__ __forceinline__ int row16_min(int v) {
  v = min(v, row16_partner<0xB1>(v));
  v = min(v, row16_partner<0x4E>(v));
  v = min(v, row16_partner<0x141>(v));
  return min(v, row16_partner<0x140>(v));
}
// Lane j's value, in every lane of its row of 16.
template <int J>
__device__ __forceinline__ float row16_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + J, 0xF, 0xF, false));
}

// An integer image of an fp32 value whose signed order is the values' order,
// with -0 taken to +0 so that the two compare equal (then the lower index
// wins, as for any tie).  kDead lies below the image of every value.
constexpr int kNone = 0x7fffffff;
constexpr int kDead = (int)0x80000000;
__device__ __forceinline__ int order_key(float v) {
  int b = __float_as_int(v);
  b = b == kDead ? 0 : b;
  return b ^ ((b >> 31) & 0x7fffffff);
}
__device__ __forceinline__ float key_value(int key) {
  return __int_as_float(key ^ ((key >> 31) & 0x7fffffff));
}

// Top-k of one token per 16-lane row.  The token's E logits sit in LDS at `L`
// (16 * NV floats readable there); lane c of the row holds experts c, c+16,
// ...  Each slot takes the row's largest remaining value (a row-wide max of
// the integer images), then the lowest index holding it (a row-wide min),
// which leaves the race.  Lane c = threadIdx.x % 16 < k receives slot c's
// expert and weight (other lanes: unspecified).  All 16 lanes of a row call
// this together.
template <int NV>  // E <= 16 * NV
__device__ __forceinline__ void topk_row16_slot(const float* L, int E, int k, int& id_c,
                                                float& w_c) {
  const int c = threadIdx.x & 15;
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = L[c + 16 * i];  // all issued before the first use
  int key[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) key[i] = c + 16 * i < E ? order_key(v[i]) : kDead;
  int key0 = 0, my_key = 0, my_i = 0;
#pragma unroll 1
  for (int j = 0; j < k; ++j) {
    int lk = key[0];
#pragma unroll
    for (int i = 1; i < NV; ++i) lk = max(lk, key[i]);
    const int m = row16_max(lk);
    int cand = kNone;
#pragma unroll
    for (int i = NV - 1; i >= 0; --i) cand = key[i] == m ? c + 16 * i : cand;
    const int win = row16_min(cand);
    key0 = j == 0 ? m : key0;
    my_key = c == j ? m : my_key;
    my_i = c == j ? win : my_i;
#pragma unroll
    for (int i = 0; i < NV; ++i) key[i] = win == c + 16 * i ? kDead : key[i];
  }
  // w_j = exp(L_j - L_0) / sum_j' exp(L_j' - L_0): the softmax over all E
  // restricted to the kept k and renormalised (the full denominator cancels);
  // lane j holds term j, and the sum runs over j in order in every lane
  // (adding +0 for the slots past k leaves it unchanged).
  const float v0 = key_value(key0);
  const float term = expf(key_value(my_key) - v0);
  float s = 0.0f;
#define MOE_TOPK_SUM(J) s += J < k ? row16_bcast<J>(term) : 0.0f;
  MOE_TOPK_SUM(0) MOE_TOPK_SUM(1) MOE_TOPK_SUM(2) MOE_TOPK_SUM(3)
  MOE_TOPK_SUM(4) MOE_TOPK_SUM(5) MOE_TOPK_SUM(6) MOE_TOPK_SUM(7)
  MOE_TOPK_SUM(8) MOE_TOPK_SUM(9) MOE_TOPK_SUM(10) MOE_TOPK_SUM(11)
  MOE_TOPK_SUM(12) MOE_TOPK_SUM(13) MOE_TOPK_SUM(14) MOE_TOPK_SUM(15)
#undef MOE_TOPK_SUM
  static_assert(kMaxK == 16, "one broadcast per slot");
  id_c = my_i;
  w_c = term / s;
}

template <int NV>  // E <= 16 * NV
__device__ __forceinline__ void topk_row16(const float* L, int E, int k, bool valid,
                                           int32_t* __restrict__ ids_out,
                                           float* __restrict__ w_out) {
  const int c = threadIdx.x & 15;
  int id_c;
  float w_c;
  topk_row16_slot<NV>(L, E, k, id_c, w_c);
  if (valid && c < k) {
    ids_out[c] = id_c;
    w_out[c] = w_c;
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
// s_waitcnt immediate for vmcnt(n), the other counters left alone
constexpr int vmcnt_imm(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | 0x70 | 0xF00; }
typedef __attribute__((address_space(3))) void* lds_ptr_t;

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
  // LDS holds first the staged W_r (two buffers of KS KB per wave), then the
  // groups' partial sums
  constexpr bool STAGE = KS >= 2;
  constexpr int PART_BYTES = 2 * kRouteWaves * 16 * EP * 4;
  constexpr int STAGE_BYTES = STAGE ? 2 * kRouteWaves * KS * 1024 : 0;
  __shared__ __align__(16) uint8_t lds[PART_BYTES > STAGE_BYTES ? PART_BYTES : STAGE_BYTES];
  float(&part)[2][kRouteWaves][16][EP] =
      *reinterpret_cast<float(*)[2][kRouteWaves][16][EP]>(lds);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, kq = (lane >> 4) * 8;
  const int k0 = wave * (KS * 32) + kq;     // this wave's columns, plus the lane's 8
  const int ngroups = (T + 15) >> 4;
  if ((int)blockIdx.x >= ngroups) return;  // block-uniform
  // experts past E read a valid row; their results are dropped
  bf16x8 w[KS][NET];
  if constexpr (STAGE) {
    // W_r through LDS, one 16-expert tile per round, two rounds in flight:
    // each load takes 8 rows x 128 B (whole cache lines; loading the
    // fragments directly would take 16 rows x 64 B per instruction, half a
    // line per row, which moves half as many bytes per cache request), and
    // the fragments are then read from LDS in the product's layout.  A
    // wave's slice of a row is KS * 64 B, bytes [wave KS 64, +KS 64) of it.
    uint8_t* const sw = lds + wave * (2 * KS * 1024);
    const uint8_t* const wb = reinterpret_cast<const uint8_t*>(wr);
    auto issue = [&](int et) {
      uint8_t* const dst = sw + (et & 1) * (KS * 1024);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = min(et * 16 + h * 8 + (lane >> 3), E - 1);
        const uint8_t* src = wb + (size_t)row * d * 2 + wave * KS * 64 + (lane & 7) * 16;
#pragma unroll
        for (int cc = 0; cc < KS / 2; ++cc)
          __builtin_amdgcn_global_load_lds(src + cc * 128,
                                           (lds_ptr_t)(dst + (h * (KS / 2) + cc) * 1024), 16, 0, 0);
      }
    };
    issue(0);
    if (NET > 1) issue(1);
#pragma unroll
    for (int et = 0; et < NET; ++et) {
      if (et + 1 < NET) __builtin_amdgcn_s_waitcnt(vmcnt_imm(KS));  // tile et landed
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      const uint8_t* const src = sw + (et & 1) * (KS * 1024);
      // row r = 8 h + r8 of the tile, K-chunk 4 ks + lane / 16 of the slice
      const int h = (lane >> 3) & 1, r8 = lane & 7;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int off = (h * (KS / 2) + (ks >> 1)) * 1024 + (r8 * 8 + (ks & 1) * 4 + (lane >> 4)) * 16;
        w[ks][et] = as_bf16x8(*reinterpret_cast<const u32x4*>(src + off));
      }
      if (et + 2 < NET) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this buffer read out
        issue(et + 2);
      }
    }
    lds_barrier();  // every wave's staging read out before the partial sums land there
  } else {
#pragma unroll
    for (int et = 0; et < NET; ++et) {
      const uint16_t* wp = wr + (size_t)min(et * 16 + r, E - 1) * d + k0;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) w[ks][et] = as_bf16x8(ld_u32x4(wp + ks * 32));
    }
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
  // A group's ids and weights are stored at the start of the next group,
  // before its x loads are issued, by every lane of every wave (buffer
  // stores; lanes with nothing to store point past the arrays, and such
  // stores are dropped); the logits likewise, right after their sums (none
  // without logits_out).  So the number of stores between a group's loads
  // and their use is the same on every path.
  constexpr uint32_t kDrop = 0x80000000u;
  const __amdgpu_buffer_rsrc_t ids_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(ids, 0, (int)((uint32_t)T * k * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t wts_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(wts, 0, (int)((uint32_t)T * k * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t lg_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      logits_out, 0, logits_out ? (int)((uint32_t)T * E * 4) : 0, 0x00020000);
  uint32_t p_off = kDrop;  // byte offset of this lane's pending slot
  int p_id = 0;
  float p_w = 0.0f;
  auto flush = [&]() {
    __builtin_amdgcn_raw_buffer_store_b32((uint32_t)p_id, ids_rsrc, (int)p_off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(p_w), wts_rsrc, (int)p_off, 0, 0);
    p_off = kDrop;
  };
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
      float v = 0.0f;
      const int t = rt[j], e = re[j];
      if (t >= 0) {
        float pv[kRouteWaves];
#pragma unroll
        for (int w2 = 0; w2 < kRouteWaves; ++w2) pv[w2] = part[b][w2][t][e];
        v = pv[0];
#pragma unroll
        for (int w2 = 1; w2 < kRouteWaves; ++w2) v += pv[w2];
        if (bias) v += rb[j];
        part[b][0][t][e] = v;
      }
      const uint32_t lo = (t >= 0 && t0 + t < T) ? (uint32_t)((t0 + t) * E + e) * 4 : kDrop;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), lg_rsrc, (int)lo, 0, 0);
    }
    lds_barrier();
    if (wave < 4) {  // one token per 16-lane row: waves 0..3 hold the group's 16 rows
      const int t = wave * 4 + (lane >> 4), c = lane & 15;
      topk_row16_slot<NET>(&part[b][0][t][0], E, k, p_id, p_w);
      if (t0 + t < T && c < k) p_off = (uint32_t)((t0 + t) * k + c) * 4;
    }
    // the next group writes the other buffer; the one after passes that
    // group's first barrier, which every wave reaches only after this top-k
  };
  // Two groups per trip, so that the register buffers swap without copies;
  // the loop has its only exit at the bottom (an exit in the middle turns,
  // once the control flow is structured, into a path back to the top on
  // which the other buffer's loads still count as in flight, and the top
  // then waits for them).  In the loop every group's products start with the
  // next group's loads in flight (after the last pair: the pair's second
  // group again, from cache); an odd last group runs after the loop.
  bf16x8 xa[KS], xb[KS];
  const int gs = (int)gridDim.x;
  int g = blockIdx.x;
  load_x(g, xa);
  // The first group's rows arrive before the second group's are asked for:
  // issued together, the two would share the memory system and the first
  // group would wait for both.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  while (g + gs < ngroups) {
    const int g2 = g + gs, g3 = g2 + gs;
    flush();
    load_x(g2, xb);
    group(g, 0, xa);
    flush();
    load_x(g3 < ngroups ? g3 : g2, xa);
    group(g2, 1, xb);
    g = g3;
  }
  if (g < ngroups) {
    flush();
    group(g, 0, xa);
  }
  flush();
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
  // per wave within the register budget of two waves per SIMD.  It is the
  // faster kernel at any token count: each block reads W_r once, in whole
  // cache lines, where the other reads it in half lines.
  const int n_cu = device_cu_count();
  // (its stores are ranged buffer stores: byte offsets of ids, weights and
  // logits within 2^31)
  if (a.E <= 64 && (a.d == 256 || a.d == 512 || a.d == 1024 || a.d == 2048) &&
      (int64_t)a.T * a.E * 4 < ((int64_t)1 << 31) && a.k <= a.E) {
    const int grid_r = ngroups < n_cu ? ngroups : n_cu;
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
