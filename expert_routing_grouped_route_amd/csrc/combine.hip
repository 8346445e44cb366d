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
// One wave per token; 16-byte vectors along the hidden dimension.
#include "common.h"
#include "kernels.h"

namespace moe {

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
        const f32x4 v = y[(size_t)rows[j] * d4 + c];
        acc[0] = fmaf(wt[j], v[0], acc[0]);
        acc[1] = fmaf(wt[j], v[1], acc[1]);
        acc[2] = fmaf(wt[j], v[2], acc[2]);
        acc[3] = fmaf(wt[j], v[3], acc[3]);
      }
    }
    if (ysh) {
      const f32x4 s = ysh[(size_t)t * d4 + c];
      acc[0] += s[0];
      acc[1] += s[1];
      acc[2] += s[2];
      acc[3] += s[3];
    }
    out[(size_t)t * d4 + c] = acc;
  }
}

void launch_combine(const CombineArgs& a, hipStream_t stream) {
  const int64_t grid = (a.T + 3) / 4;
  if (grid == 0) return;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     reinterpret_cast<const f32x4*>(a.y), a.inv, a.w,
                     reinterpret_cast<const f32x4*>(a.ysh), (int)a.T, a.k, (int)(a.T * a.k),
                     a.d / 4, reinterpret_cast<f32x4*>(a.out));
}

}  // namespace moe
