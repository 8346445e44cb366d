// Combine of the MoE layer on one GPU: each token gathers its k expert output
// rows, weights them by its gate weights and adds the shared-expert output.
//
// On the pages Combine is the all-to-all that returns expert outputs to each
// token's device (FarSkip-Collective review, "Core claim"; Fig. 11 caption,
// where it is overlapped with the shared expert; the Luffy review, "Core
// claim").  On one GPU's share it is an HBM-bound gather with an fp32
// weighted sum.  Accumulation order (ascending slot, shared term last) is a
// reading, fixed so that results are reproducible bit for bit.
//
// One wave per token; 16-byte vectors along the hidden dimension.  The rows
// of y and of the shared-expert output are read once, with non-temporal loads
// (on MI355X streaming reads marked so run about 10% faster than plain ones).
// For the common k (1, 2, 4, 6, 8) the kernel is specialised on k so that
// every row's loads are issued before the sums (the generic loop serialises
// them behind its per-slot branches); the sum order is the same in both.
#include "common.h"
#include "kernels.h"

namespace moe {

__device__ __forceinline__ f32x4 ld_once(const f32x4* p) { return __builtin_nontemporal_load(p); }

__global__ __launch_bounds__(256) void combine_kernel(const f32x4* __restrict__ y,
                                                      const int32_t* __restrict__ inv_perm,
                                                      const float* __restrict__ w,
                                                      const f32x4* __restrict__ ysh, int T, int k,
                                                      int R, int d4, f32x4* __restrict__ out) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  int rows[kMaxK];
  float wt[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    rows[j] = -1;
    wt[j] = 0.0f;
    if (j < k) {
      const int r = inv_perm[(size_t)t * k + j];
      rows[j] = (unsigned)r < (unsigned)R ? r : -1;
      wt[j] = w[(size_t)t * k + j];
    }
  }
  for (int c = lane; c < d4; c += 64) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k && rows[j] >= 0) {
        const f32x4 v = ld_once(y + (size_t)rows[j] * d4 + c);
        acc[0] = fmaf(wt[j], v[0], acc[0]);
        acc[1] = fmaf(wt[j], v[1], acc[1]);
        acc[2] = fmaf(wt[j], v[2], acc[2]);
        acc[3] = fmaf(wt[j], v[3], acc[3]);
      }
    }
    if (ysh) {
      const f32x4 s = ld_once(ysh + (size_t)t * d4 + c);
      acc[0] += s[0];
      acc[1] += s[1];
      acc[2] += s[2];
      acc[3] += s[3];
    }
    out[(size_t)t * d4 + c] = acc;
  }
}

// k known at compile time: every row's loads are issued before the sums.
template <int K, int U, bool SH>
__global__ __launch_bounds__(256) void combine_k_kernel(const f32x4* __restrict__ y,
                                                        const int32_t* __restrict__ inv_perm,
                                                        const float* __restrict__ w,
                                                        const f32x4* __restrict__ ysh, int T, int R,
                                                        int d4, f32x4* __restrict__ out) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const f32x4* src[K];
  float wt[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int r = inv_perm[(size_t)t * K + j];
    const bool ok = (unsigned)r < (unsigned)R;
    src[j] = y + (size_t)(ok ? r : 0) * d4;
    wt[j] = ok ? w[(size_t)t * K + j] : 0.0f;
  }
  const f32x4* s_row = SH ? ysh + (size_t)t * d4 : nullptr;
  f32x4* o_row = out + (size_t)t * d4;
  int c = lane;
  for (; c + 64 * (U - 1) < d4; c += 64 * U) {
    f32x4 v[K][U], s[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < K; ++j) v[j][u] = ld_once(src[j] + c + 64 * u);
    if (SH) {
#pragma unroll
      for (int u = 0; u < U; ++u) s[u] = ld_once(s_row + c + 64 * u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < K; ++j) {
        acc[0] = fmaf(wt[j], v[j][u][0], acc[0]);
        acc[1] = fmaf(wt[j], v[j][u][1], acc[1]);
        acc[2] = fmaf(wt[j], v[j][u][2], acc[2]);
        acc[3] = fmaf(wt[j], v[j][u][3], acc[3]);
      }
      if (SH) {
        acc[0] += s[u][0];
        acc[1] += s[u][1];
        acc[2] += s[u][2];
        acc[3] += s[u][3];
      }
      o_row[c + 64 * u] = acc;
    }
  }
  for (; c < d4; c += 64) {
    f32x4 v[K];
#pragma unroll
    for (int j = 0; j < K; ++j) v[j] = ld_once(src[j] + c);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < K; ++j) {
      acc[0] = fmaf(wt[j], v[j][0], acc[0]);
      acc[1] = fmaf(wt[j], v[j][1], acc[1]);
      acc[2] = fmaf(wt[j], v[j][2], acc[2]);
      acc[3] = fmaf(wt[j], v[j][3], acc[3]);
    }
    if (SH) {
      const f32x4 sv = ld_once(s_row + c);
      acc[0] += sv[0];
      acc[1] += sv[1];
      acc[2] += sv[2];
      acc[3] += sv[3];
    }
    o_row[c] = acc;
  }
}

constexpr int kCombineChunks = 4;  // 16-byte chunks per lane and row in flight
template <int K>
static void launch_k(const CombineArgs& a, int64_t grid, hipStream_t stream) {
  auto kern = a.ysh ? combine_k_kernel<K, kCombineChunks, true> : combine_k_kernel<K, kCombineChunks, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, stream,
                     reinterpret_cast<const f32x4*>(a.y), a.inv, a.w,
                     reinterpret_cast<const f32x4*>(a.ysh), (int)a.T, (int)(a.T * a.k), a.d / 4,
                     reinterpret_cast<f32x4*>(a.out));
}

void launch_combine(const CombineArgs& a, hipStream_t stream) {
  const int64_t grid = (a.T + 3) / 4;
  if (grid == 0) return;
  switch (a.k) {
    case 1: launch_k<1>(a, grid, stream); return;
    case 2: launch_k<2>(a, grid, stream); return;
    case 4: launch_k<4>(a, grid, stream); return;
    case 6: launch_k<6>(a, grid, stream); return;
    case 8: launch_k<8>(a, grid, stream); return;
    default: break;
  }
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     reinterpret_cast<const f32x4*>(a.y), a.inv, a.w,
                     reinterpret_cast<const f32x4*>(a.ysh), (int)a.T, a.k, (int)(a.T * a.k),
                     a.d / 4, reinterpret_cast<f32x4*>(a.out));
}

}  // namespace moe
