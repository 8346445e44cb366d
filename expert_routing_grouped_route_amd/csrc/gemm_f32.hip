// Grouped SwiGLU experts for float32 workloads, on the vector ALUs.
//
// Same layer and tile table as the bf16 matrix-core kernels (see
// gemm_bf16.hip for the pages these steps follow); A stays in fp32.  Tiles are
// 128 rows x 64 columns (each M-tile of the table is taken in two halves),
// K-steps of 16 staged through LDS, each thread accumulating 8 rows x 4
// columns with fused multiply-adds.  These kernels serve small float32
// layers; large layers are bf16.
#include "grouped_gemm.h"

namespace moe {
namespace {

constexpr int FBM = 128;  // rows per tile (half an M-tile of the table)
constexpr int FBN = 64;   // output columns per tile
constexpr int HALVES = kBM / FBM;
constexpr int FBK = 16;   // K per LDS step

struct F32Tile {
  const float* X;       // first A row (or the token rows when rmap is set)
  size_t x_ld;          // floats between A rows
  int rows;             // valid rows
  const int32_t* rmap;  // or null: A row r is token row rmap[r] / rdiv of X
  int rdiv;
  const float* W0;      // first weight row (gate, or down)
  const float* W1;      // first up-weight row (gate/up only)
  size_t w_ld;          // floats between weight rows
  int cols;             // valid output columns
  int k;                // reduction length
  int k_seg;            // shared down tiles: K per shared expert (0 = one segment)
  size_t w_seg_stride;  // floats between shared experts' weight blocks
  float* Out;
  size_t out_ld;
};

// n-tiles of 64 columns
__device__ __forceinline__ bool f32_gate_up_tile(const FfnArgs& p, const GemmGrid& g, int L,
                                                 F32Tile& t) {
  if (L < g.routed) {
    int e, m, n;
    if (!routed_tile(L / HALVES, p.tile_off, p.E, g.nt_r, e, m, n)) return false;
    const int r0 = p.offsets[e] + m * kBM + (L % HALVES) * FBM;
    t.rows = min(FBM, p.offsets[e + 1] - r0);
    if (t.rows <= 0) return false;
    if (p.xs) {
      t.X = static_cast<const float*>(p.xs) + (size_t)r0 * p.d;
      t.rmap = nullptr;
    } else {  // gather the token rows of x through the dispatch permutation
      t.X = static_cast<const float*>(p.x);
      t.rmap = p.perm + r0;
      t.rdiv = p.k;
    }
    const size_t w_off = ((size_t)e * p.I + (size_t)n * FBN) * p.d;
    t.W0 = static_cast<const float*>(p.wg) + w_off;
    t.W1 = static_cast<const float*>(p.wu) + w_off;
    t.cols = min(FBN, p.I - n * FBN);
    t.Out = static_cast<float*>(p.a) + (size_t)r0 * p.I + (size_t)n * FBN;
    t.out_ld = p.I;
  } else {
    const int sb = L - (int)g.routed;
    const int per_s = g.mt_s * g.nt_s;
    const int s = sb / per_s, rem = sb - s * per_s;
    const int n = rem / g.mt_s, m = rem - n * g.mt_s;
    const int r0 = m * FBM;
    t.rows = (int)min((int64_t)FBM, p.T - r0);
    t.X = static_cast<const float*>(p.x) + (size_t)r0 * p.d;
    t.rmap = nullptr;
    const size_t w_off = ((size_t)s * p.Is + (size_t)n * FBN) * p.d;
    t.W0 = static_cast<const float*>(p.wsg) + w_off;
    t.W1 = static_cast<const float*>(p.wsu) + w_off;
    t.cols = min(FBN, p.Is - n * FBN);
    const size_t ld = (size_t)p.ns * p.Is;
    t.Out = static_cast<float*>(p.ash) + (size_t)r0 * ld + (size_t)s * p.Is + (size_t)n * FBN;
    t.out_ld = ld;
  }
  t.x_ld = p.d;
  t.w_ld = p.d;
  t.k = p.d;
  t.k_seg = 0;
  t.w_seg_stride = 0;
  return true;
}

__device__ __forceinline__ bool f32_down_tile(const FfnArgs& p, const GemmGrid& g, int L,
                                              F32Tile& t) {
  if (L < g.routed) {
    int e, m, n;
    if (!routed_tile(L / HALVES, p.tile_off, p.E, g.nt_r, e, m, n)) return false;
    const int r0 = p.offsets[e] + m * kBM + (L % HALVES) * FBM;
    t.rows = min(FBM, p.offsets[e + 1] - r0);
    if (t.rows <= 0) return false;
    t.X = static_cast<const float*>(p.a) + (size_t)r0 * p.I;
    t.x_ld = p.I;
    t.W0 = static_cast<const float*>(p.wd) + ((size_t)e * p.d + (size_t)n * FBN) * p.I;
    t.w_ld = p.I;
    t.cols = min(FBN, p.d - n * FBN);
    t.k = p.I;
    t.k_seg = 0;
    t.w_seg_stride = 0;
    t.Out = p.y + (size_t)r0 * p.d + (size_t)n * FBN;
  } else {
    const int sb = L - (int)g.routed;
    const int n = sb / g.mt_s, m = sb - n * g.mt_s;
    const int r0 = m * FBM;
    t.rows = (int)min((int64_t)FBM, p.T - r0);
    const size_t ld = (size_t)p.ns * p.Is;
    t.X = static_cast<const float*>(p.ash) + (size_t)r0 * ld;
    t.x_ld = ld;
    t.W0 = static_cast<const float*>(p.wsd) + (size_t)n * FBN * p.Is;
    t.w_ld = p.Is;
    t.cols = min(FBN, p.d - n * FBN);
    t.k = (int)ld;
    t.k_seg = p.Is;
    t.w_seg_stride = (size_t)p.d * p.Is;
    t.Out = p.ysh + (size_t)r0 * p.d + (size_t)n * FBN;
  }
  t.W1 = nullptr;
  t.rmap = nullptr;
  t.out_ld = p.d;
  return true;
}

template <int NW>
__device__ __forceinline__ void f32_tile_loop(const F32Tile& t, float (&acc)[NW][8][4]) {
  __shared__ float sX[FBK][FBM + 4];
  __shared__ float sW[NW][FBK][FBN + 4];
  const int tid = threadIdx.x;
  const int tn = tid & 15, tm = tid >> 4;
  for (int k0 = 0; k0 < t.k; k0 += FBK) {
    // weights of the shared down tiles sit in one block per shared expert
    const size_t wk = t.k_seg ? (size_t)(k0 / t.k_seg) * t.w_seg_stride + (k0 % t.k_seg) : (size_t)k0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {  // X: 128 rows x 16 = 512 float4
      const int c = tid + 256 * q, row = c >> 2, k4 = (c & 3) * 4;
      const int rr = min(row, t.rows - 1);
      const size_t xrow = t.rmap ? (size_t)(t.rmap[rr] / t.rdiv) : (size_t)rr;
      const float4 v = *reinterpret_cast<const float4*>(t.X + xrow * t.x_ld + k0 + k4);
      sX[k4 + 0][row] = v.x;
      sX[k4 + 1][row] = v.y;
      sX[k4 + 2][row] = v.z;
      sX[k4 + 3][row] = v.w;
    }
#pragma unroll
    for (int w = 0; w < NW; ++w) {  // W: 64 rows x 16 = 256 float4
      const int row = tid >> 2, k4 = (tid & 3) * 4;
      const float* base = w == 0 ? t.W0 : t.W1;
      const float4 v = *reinterpret_cast<const float4*>(
          base + (size_t)min(row, t.cols - 1) * t.w_ld + wk + k4);
      sW[w][k4 + 0][row] = v.x;
      sW[w][k4 + 1][row] = v.y;
      sW[w][k4 + 2][row] = v.z;
      sW[w][k4 + 3][row] = v.w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FBK; ++kk) {
      float a[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] = sX[kk][tm * 8 + i];
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        float b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = sW[w][kk][tn * 4 + j];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[w][i][j] = fmaf(a[i], b[j], acc[w][i][j]);
      }
    }
    __syncthreads();
  }
}

// A launch of the shared experts' tiles alone starts after the routed slots.
__device__ __forceinline__ int f32_slot(const FfnArgs& p, const GemmGrid& g) {
  return (int)blockIdx.x + (p.part == kSharedTiles ? (int)g.routed : 0);
}

__global__ __launch_bounds__(256) void gate_up_f32_kernel(FfnArgs p, GemmGrid g) {
  F32Tile t;
  if (!f32_gate_up_tile(p, g, f32_slot(p, g), t)) return;
  float acc[2][8][4] = {};
  f32_tile_loop<2>(t, acc);
  const int tn = threadIdx.x & 15, tm = threadIdx.x >> 4;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = tm * 8 + i, col = tn * 4 + j;
      if (row < t.rows && col < t.cols)
        t.Out[(size_t)row * t.out_ld + col] = silu_times(acc[0][i][j], acc[1][i][j]);
    }
}

__global__ __launch_bounds__(256) void down_f32_kernel(FfnArgs p, GemmGrid g) {
  F32Tile t;
  if (!f32_down_tile(p, g, f32_slot(p, g), t)) return;
  float acc[1][8][4] = {};
  f32_tile_loop<1>(t, acc);
  const int tn = threadIdx.x & 15, tm = threadIdx.x >> 4;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = tm * 8 + i, col = tn * 4 + j;
      if (row < t.rows && col < t.cols) t.Out[(size_t)row * t.out_ld + col] = acc[0][i][j];
    }
}

GemmGrid f32_gate_up_grid(const FfnArgs& a) {
  GemmGrid g;
  g.nt_r = (a.I + FBN - 1) / FBN;
  g.nt_s = a.ns ? (a.Is + FBN - 1) / FBN : 0;
  g.mt_s = (int)((a.T + FBM - 1) / FBM);
  g.routed = routed_mtile_bound(a.R, a.E) * HALVES * g.nt_r;
  g.total = g.routed + (int64_t)a.ns * g.nt_s * g.mt_s;
  return g;
}

GemmGrid f32_down_grid(const FfnArgs& a) {
  GemmGrid g;
  g.nt_r = (a.d + FBN - 1) / FBN;
  g.nt_s = g.nt_r;
  g.mt_s = (int)((a.T + FBM - 1) / FBM);
  g.routed = routed_mtile_bound(a.R, a.E) * HALVES * g.nt_r;
  g.total = g.routed + (a.ns ? (int64_t)g.nt_r * g.mt_s : 0);
  return g;
}

}  // namespace

int64_t gate_up_grid_f32(const FfnArgs& a) { return f32_gate_up_grid(a).total; }
int64_t down_grid_f32(const FfnArgs& a) { return f32_down_grid(a).total; }

// Blocks of one launch: all tiles, the routed slots or the shared tiles.
int64_t f32_blocks(const FfnArgs& a, const GemmGrid& g) {
  return a.part == kRoutedTiles ? g.routed : a.part == kSharedTiles ? g.total - g.routed : g.total;
}

void launch_gate_up_f32(const FfnArgs& a, hipStream_t stream) {
  const GemmGrid g = f32_gate_up_grid(a);
  const int64_t n = f32_blocks(a, g);
  if (n == 0) return;
  hipLaunchKernelGGL(gate_up_f32_kernel, dim3((unsigned)n), dim3(256), 0, stream, a, g);
}

void launch_down_f32(const FfnArgs& a, hipStream_t stream) {
  const GemmGrid g = f32_down_grid(a);
  const int64_t n = f32_blocks(a, g);
  if (n == 0) return;
  hipLaunchKernelGGL(down_f32_kernel, dim3((unsigned)n), dim3(256), 0, stream, a, g);
}

}  // namespace moe
