// Routed and shared experts of the MoE layer as grouped GEMMs.
//
// The routed experts are the T_routed term of the FarSkip-Collective review's
// overlap window (axiom ledger, Eq. 9); the always-on shared expert is the
// branch its Fig. 11 caption overlaps with Combine.  Grouping every expert's
// tokens into one dense product is the "Expert-Centric Scheduling" of the
// OmniMoE abstract on the "Daily Papers" search page.  The expert FFN itself
// (SwiGLU, no biases) is a reading; the pages do not spell it out.
//
// Tile space.  M-tiles of kBM = 128 rows per expert come from the tile table
// that the dispatch scan wrote (tile_off[e] = M-tiles of experts < e); within
// an expert the tiles run n-tile outer, m-tile inner, so tiles that share a
// weight slice are adjacent in launch order.  The grid is sized by an upper
// bound of the routed tiles (no host read-back); blocks past the device-side
// count return at once.  Shared experts follow as extra tiles over all T rows.
//
// bf16 kernels: 256 threads = 4 waves in a 2x2 arrangement over a 128-row
// tile.  Operands stream global -> registers -> LDS in K-steps of 64,
// double-buffered so the next step's loads are in flight during the current
// step's MFMAs.  LDS rows are padded to 72 elements (144 bytes) so that the
// 16-byte fragment reads of 8 consecutive rows hit distinct banks.
//   gate/up: each wave owns 64 rows x 64 gate columns and the same 64 up
//            columns (two accumulators), so the epilogue forms
//            bf16(silu(g) * u) in registers and only A reaches memory.
//   down:    each wave owns 64 rows x 64 output columns, fp32 out.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int BN = 128;   // output columns per tile
constexpr int BK = 64;    // K per pipeline step
constexpr int LDK = BK + 8;

// Routed tile L -> expert e, m-tile m, n-tile n (false when L is past the end).
__device__ __forceinline__ bool routed_tile(int L, const int32_t* __restrict__ tile_off, int E,
                                            int nt, int& e, int& m, int& n) {
  const int total = tile_off[E] * nt;
  if (L >= total) return false;
  int lo = 0, hi = E - 1;  // largest e with tile_off[e] * nt <= L
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_off[mid] * nt <= L) lo = mid;
    else hi = mid - 1;
  }
  e = lo;
  const int mt = tile_off[e + 1] - tile_off[e];
  const int local = L - tile_off[e] * nt;
  n = local / mt;
  m = local - n * mt;
  return true;
}

// Everything a block needs to know about its tile.
struct Tile {
  const uint8_t* X;     // first row of the A operand
  size_t x_ld;          // elements between A rows
  int rows;             // valid rows (<= kBM)
  const uint8_t* W0;    // first weight row (gate, or down)
  const uint8_t* W1;    // first up-weight row (gate/up only)
  size_t w_ld;          // elements between weight rows
  int cols;             // valid output columns (<= BN)
  int nk;               // K-steps
  // shared down tiles: K runs over the shared experts one after another
  int k_per_expert_steps;   // K-steps per shared expert (0 = single segment)
  size_t w_expert_stride;   // elements between shared experts' weight blocks
  uint8_t* Out;
  size_t out_ld;
};

template <int ESZ>
__device__ __forceinline__ bool gate_up_tile(const FfnArgs& p, int nt_r, int nt_s, int mt_s,
                                             int routed_blocks, int bid, Tile& t) {
  if (bid < routed_blocks) {
    int e, m, n;
    if (!routed_tile(bid, p.tile_off, p.E, nt_r, e, m, n)) return false;
    const int r0 = p.offsets[e] + m * kBM;
    t.rows = min(kBM, p.offsets[e + 1] - r0);
    t.X = static_cast<const uint8_t*>(p.xs) + (size_t)r0 * p.d * ESZ;
    const size_t w_off = ((size_t)e * p.I + (size_t)n * BN) * p.d * ESZ;
    t.W0 = static_cast<const uint8_t*>(p.wg) + w_off;
    t.W1 = static_cast<const uint8_t*>(p.wu) + w_off;
    t.cols = min(BN, p.I - n * BN);
    t.Out = static_cast<uint8_t*>(p.a) + ((size_t)r0 * p.I + (size_t)n * BN) * ESZ;
    t.out_ld = p.I;
  } else {
    const int sb = bid - routed_blocks;
    const int per_s = mt_s * nt_s;
    const int s = sb / per_s, rem = sb - s * per_s;
    const int n = rem / mt_s, m = rem - n * mt_s;
    const int r0 = m * kBM;
    t.rows = min((int64_t)kBM, p.T - r0);
    t.X = static_cast<const uint8_t*>(p.x) + (size_t)r0 * p.d * ESZ;
    const size_t w_off = ((size_t)s * p.Is + (size_t)n * BN) * p.d * ESZ;
    t.W0 = static_cast<const uint8_t*>(p.wsg) + w_off;
    t.W1 = static_cast<const uint8_t*>(p.wsu) + w_off;
    t.cols = min(BN, p.Is - n * BN);
    const size_t ld = (size_t)p.ns * p.Is;
    t.Out = static_cast<uint8_t*>(p.ash) + ((size_t)r0 * ld + (size_t)s * p.Is + (size_t)n * BN) * ESZ;
    t.out_ld = ld;
  }
  t.x_ld = p.d;
  t.w_ld = p.d;
  t.nk = p.d / BK;
  t.k_per_expert_steps = 0;
  t.w_expert_stride = 0;
  return true;
}

template <int ESZ>
__device__ __forceinline__ bool down_tile(const FfnArgs& p, int nt, int mt_s, int routed_blocks,
                                          int bid, Tile& t) {
  if (bid < routed_blocks) {
    int e, m, n;
    if (!routed_tile(bid, p.tile_off, p.E, nt, e, m, n)) return false;
    const int r0 = p.offsets[e] + m * kBM;
    t.rows = min(kBM, p.offsets[e + 1] - r0);
    t.X = static_cast<const uint8_t*>(p.a) + (size_t)r0 * p.I * ESZ;
    t.x_ld = p.I;
    t.W0 = static_cast<const uint8_t*>(p.wd) + ((size_t)e * p.d + (size_t)n * BN) * p.I * ESZ;
    t.w_ld = p.I;
    t.cols = min(BN, p.d - n * BN);
    t.nk = p.I / BK;
    t.k_per_expert_steps = 0;
    t.w_expert_stride = 0;
    t.Out = reinterpret_cast<uint8_t*>(p.y + (size_t)r0 * p.d + (size_t)n * BN);
  } else {
    const int sb = bid - routed_blocks;
    const int n = sb / mt_s, m = sb - n * mt_s;
    const int r0 = m * kBM;
    t.rows = min((int64_t)kBM, p.T - r0);
    const size_t ld = (size_t)p.ns * p.Is;
    t.X = static_cast<const uint8_t*>(p.ash) + (size_t)r0 * ld * ESZ;
    t.x_ld = ld;
    t.W0 = static_cast<const uint8_t*>(p.wsd) + (size_t)n * BN * p.Is * ESZ;
    t.w_ld = p.Is;
    t.cols = min(BN, p.d - n * BN);
    t.nk = (int)(ld / BK);
    t.k_per_expert_steps = p.Is / BK;
    t.w_expert_stride = (size_t)p.d * p.Is;
    t.Out = reinterpret_cast<uint8_t*>(p.ysh + (size_t)r0 * p.d + (size_t)n * BN);
  }
  t.W1 = nullptr;
  t.out_ld = p.d;
  return true;
}

// Byte offset of K-step kt inside a weight row block (shared down tiles walk
// across the shared experts' separate weight blocks).
template <int ESZ>
__device__ __forceinline__ size_t w_step_offset(const Tile& t, int kt) {
  if (t.k_per_expert_steps == 0) return (size_t)kt * BK * ESZ;
  const int s = kt / t.k_per_expert_steps;
  const int kin = kt - s * t.k_per_expert_steps;
  return ((size_t)s * t.w_expert_stride + (size_t)kin * BK) * ESZ;
}

// ---------------------------------------------------------------------------
// bf16 matrix-core kernels
// ---------------------------------------------------------------------------

// NW = weight tiles per block (2: gate and up, 1: down).
template <int NW>
struct Bf16Pipe {
  static constexpr int XCH = kBM * BK / 8 / 256;      // 16-byte chunks of X per thread (4)
  static constexpr int WCH = NW * BN * BK / 8 / 256;  // of W per thread (8 or 4)
  const uint8_t* xp[XCH];
  const uint8_t* wp[WCH];
  u32x4 xr[XCH];
  u32x4 wr[WCH];
  int col8;  // element column of this thread's chunks

  __device__ __forceinline__ void init(const Tile& t) {
    const int tid = threadIdx.x;
    col8 = (tid & 7) * 8;
#pragma unroll
    for (int q = 0; q < XCH; ++q) {
      const int row = (tid >> 3) + 32 * q;
      xp[q] = t.X + ((size_t)min(row, t.rows - 1) * t.x_ld + col8) * 2;
    }
#pragma unroll
    for (int q = 0; q < WCH; ++q) {
      const int row = (tid >> 3) + 32 * q;  // 0..NW*BN-1
      const int wsel = row / BN, wrow = min(row - wsel * BN, t.cols - 1);
      const uint8_t* base = wsel == 0 ? t.W0 : t.W1;
      wp[q] = base + ((size_t)wrow * t.w_ld + col8) * 2;
    }
  }
  __device__ __forceinline__ void load(const Tile& t, int kt) {
    const size_t xo = (size_t)kt * BK * 2;
    const size_t wo = w_step_offset<2>(t, kt);
#pragma unroll
    for (int q = 0; q < XCH; ++q) xr[q] = ld_u32x4(xp[q] + xo);
#pragma unroll
    for (int q = 0; q < WCH; ++q) wr[q] = ld_u32x4(wp[q] + wo);
  }
  __device__ __forceinline__ void store(uint16_t* sX, uint16_t* sW) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int q = 0; q < XCH; ++q)
      *reinterpret_cast<u32x4*>(&sX[((tid >> 3) + 32 * q) * LDK + col8]) = xr[q];
#pragma unroll
    for (int q = 0; q < WCH; ++q)
      *reinterpret_cast<u32x4*>(&sW[((tid >> 3) + 32 * q) * LDK + col8]) = wr[q];
  }
};

__global__ __launch_bounds__(256) void gate_up_bf16_kernel(FfnArgs p, int nt_r, int nt_s,
                                                           int mt_s, int routed_blocks) {
  __shared__ __attribute__((aligned(16))) uint16_t sX[2][kBM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sW[2][2 * BN * LDK];
  Tile t;
  if (!gate_up_tile<2>(p, nt_r, nt_s, mt_s, routed_blocks, blockIdx.x, t)) return;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, kg = lane >> 4;

  Bf16Pipe<2> pipe;
  pipe.init(t);
  f32x4 accg[4][4], accu[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      accg[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      accu[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  pipe.load(t, 0);
  pipe.store(sX[0], sW[0]);
  __syncthreads();
  for (int kt = 0; kt < t.nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < t.nk) pipe.load(t, kt + 1);
    const uint16_t* X = sX[cur];
    const uint16_t* W = sW[cur];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kc = ks * 32 + kg * 8;
      bf16x8 a[4], bg[4], bu[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = as_bf16x8(ld_u32x4(&X[(wm * 64 + i * 16 + r16) * LDK + kc]));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bg[j] = as_bf16x8(ld_u32x4(&W[(wn * 64 + j * 16 + r16) * LDK + kc]));
        bu[j] = as_bf16x8(ld_u32x4(&W[(BN + wn * 64 + j * 16 + r16) * LDK + kc]));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          accg[i][j] = mfma_16x16x32_bf16(a[i], bg[j], accg[i][j]);
          accu[i][j] = mfma_16x16x32_bf16(a[i], bu[j], accu[i][j]);
        }
    }
    if (kt + 1 < t.nk) pipe.store(sX[cur ^ 1], sW[cur ^ 1]);
    __syncthreads();
  }

  uint16_t* out = reinterpret_cast<uint16_t*>(t.Out);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = wm * 64 + i * 16 + kg * 4 + q;
        const int col = wn * 64 + j * 16 + r16;
        if (row < t.rows && col < t.cols)
          out[(size_t)row * t.out_ld + col] = f32_to_bf16_bits(silu_times(accg[i][j][q], accu[i][j][q]));
      }
}

__global__ __launch_bounds__(256) void down_bf16_kernel(FfnArgs p, int nt, int mt_s,
                                                        int routed_blocks) {
  __shared__ __attribute__((aligned(16))) uint16_t sX[2][kBM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sW[2][BN * LDK];
  Tile t;
  if (!down_tile<2>(p, nt, mt_s, routed_blocks, blockIdx.x, t)) return;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, kg = lane >> 4;

  Bf16Pipe<1> pipe;
  pipe.init(t);
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  pipe.load(t, 0);
  pipe.store(sX[0], sW[0]);
  __syncthreads();
  for (int kt = 0; kt < t.nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < t.nk) pipe.load(t, kt + 1);
    const uint16_t* X = sX[cur];
    const uint16_t* W = sW[cur];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kc = ks * 32 + kg * 8;
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = as_bf16x8(ld_u32x4(&X[(wm * 64 + i * 16 + r16) * LDK + kc]));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = as_bf16x8(ld_u32x4(&W[(wn * 64 + j * 16 + r16) * LDK + kc]));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_16x16x32_bf16(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < t.nk) pipe.store(sX[cur ^ 1], sW[cur ^ 1]);
    __syncthreads();
  }

  float* out = reinterpret_cast<float*>(t.Out);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = wm * 64 + i * 16 + kg * 4 + q;
        const int col = wn * 64 + j * 16 + r16;
        if (row < t.rows && col < t.cols) out[(size_t)row * t.out_ld + col] = acc[i][j][q];
      }
}

// ---------------------------------------------------------------------------
// fp32 kernels (vector ALUs): 128-row x 64-column tiles, K-steps of 16,
// each thread 8 rows x 4 columns.
// ---------------------------------------------------------------------------

constexpr int FBN = 64, FBK = 16;

template <int NW>
__device__ __forceinline__ void f32_tile_loop(const Tile& t, float (&acc)[NW][8][4]) {
  __shared__ float sX[FBK][kBM + 4];
  __shared__ float sW[NW][FBK][FBN + 4];
  const int tid = threadIdx.x;
  const int tn = tid & 15, tm = tid >> 4;
  const int nsteps = t.nk * (BK / FBK);
  for (int ks = 0; ks < nsteps; ++ks) {
    const int kt = ks / (BK / FBK), kin = (ks % (BK / FBK)) * FBK;
#pragma unroll
    for (int q = 0; q < 2; ++q) {  // X: 128 rows x 16 = 512 float4
      const int c = tid + 256 * q, row = c >> 2, k4 = (c & 3) * 4;
      const float* src = reinterpret_cast<const float*>(t.X) +
                         (size_t)min(row, t.rows - 1) * t.x_ld + (size_t)kt * BK + kin + k4;
      const float4 v = *reinterpret_cast<const float4*>(src);
      sX[k4 + 0][row] = v.x;
      sX[k4 + 1][row] = v.y;
      sX[k4 + 2][row] = v.z;
      sX[k4 + 3][row] = v.w;
    }
#pragma unroll
    for (int w = 0; w < NW; ++w) {  // W: 64 rows x 16 = 256 float4
      const int row = tid >> 2, k4 = (tid & 3) * 4;
      const uint8_t* base = w == 0 ? t.W0 : t.W1;
      const float* src = reinterpret_cast<const float*>(base + w_step_offset<4>(t, kt)) +
                         (size_t)min(row, t.cols - 1) * t.w_ld + kin + k4;
      const float4 v = *reinterpret_cast<const float4*>(src);
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

// fp32 tiles reuse the bf16 tile description with 64-column n-tiles: the
// n-tile index of the 128-column scheme is split in two halves.
__global__ __launch_bounds__(256) void gate_up_f32_kernel(FfnArgs p, int nt_r, int nt_s, int mt_s,
                                                          int routed_blocks) {
  Tile t;
  if (!gate_up_tile<4>(p, nt_r, nt_s, mt_s, routed_blocks, blockIdx.x >> 1, t)) return;
  const int half = blockIdx.x & 1;
  if (half * FBN >= t.cols) return;
  t.cols -= half * FBN;
  t.cols = min(t.cols, FBN);
  t.W0 += (size_t)half * FBN * t.w_ld * 4;
  t.W1 += (size_t)half * FBN * t.w_ld * 4;
  t.Out += (size_t)half * FBN * 4;
  float acc[2][8][4] = {};
  f32_tile_loop<2>(t, acc);
  const int tn = threadIdx.x & 15, tm = threadIdx.x >> 4;
  float* out = reinterpret_cast<float*>(t.Out);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = tm * 8 + i, col = tn * 4 + j;
      if (row < t.rows && col < t.cols)
        out[(size_t)row * t.out_ld + col] = silu_times(acc[0][i][j], acc[1][i][j]);
    }
}

__global__ __launch_bounds__(256) void down_f32_kernel(FfnArgs p, int nt, int mt_s,
                                                       int routed_blocks) {
  Tile t;
  if (!down_tile<4>(p, nt, mt_s, routed_blocks, blockIdx.x >> 1, t)) return;
  const int half = blockIdx.x & 1;
  if (half * FBN >= t.cols) return;
  t.cols -= half * FBN;
  t.cols = min(t.cols, FBN);
  t.W0 += (size_t)half * FBN * t.w_ld * 4;
  t.Out += (size_t)half * FBN * 4;
  float acc[1][8][4] = {};
  f32_tile_loop<1>(t, acc);
  const int tn = threadIdx.x & 15, tm = threadIdx.x >> 4;
  float* out = reinterpret_cast<float*>(t.Out);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = tm * 8 + i, col = tn * 4 + j;
      if (row < t.rows && col < t.cols) out[(size_t)row * t.out_ld + col] = acc[0][i][j];
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

static int64_t routed_mtile_bound(const FfnArgs& a) {
  // sum_e ceil(n_e / kBM) <= floor((R + E*(kBM-1)) / kBM)
  return (a.R + (int64_t)a.E * (kBM - 1)) / kBM;
}

struct GateUpGrid { int nt_r, nt_s, mt_s; int64_t routed, total; };
static GateUpGrid gate_up_shape(const FfnArgs& a) {
  GateUpGrid g;
  g.nt_r = (a.I + BN - 1) / BN;
  g.nt_s = a.ns ? (a.Is + BN - 1) / BN : 0;
  g.mt_s = (int)((a.T + kBM - 1) / kBM);
  g.routed = a.R > 0 ? routed_mtile_bound(a) * g.nt_r : 0;
  g.total = g.routed + (int64_t)a.ns * g.nt_s * g.mt_s;
  return g;
}

int64_t gate_up_grid(const FfnArgs& a) { return gate_up_shape(a).total * (a.bf16 ? 1 : 2); }

void launch_gate_up(const FfnArgs& a, hipStream_t stream) {
  const GateUpGrid g = gate_up_shape(a);
  if (g.total == 0) return;
  if (a.bf16)
    hipLaunchKernelGGL(gate_up_bf16_kernel, dim3((unsigned)g.total), dim3(256), 0, stream, a,
                       g.nt_r, g.nt_s, g.mt_s, (int)g.routed);
  else
    hipLaunchKernelGGL(gate_up_f32_kernel, dim3((unsigned)(g.total * 2)), dim3(256), 0, stream, a,
                       g.nt_r, g.nt_s, g.mt_s, (int)g.routed);
}

struct DownGrid { int nt, mt_s; int64_t routed, total; };
static DownGrid down_shape(const FfnArgs& a) {
  DownGrid g;
  g.nt = (a.d + BN - 1) / BN;
  g.mt_s = (int)((a.T + kBM - 1) / kBM);
  g.routed = a.R > 0 ? routed_mtile_bound(a) * g.nt : 0;
  g.total = g.routed + (a.ns ? (int64_t)g.nt * g.mt_s : 0);
  return g;
}

int64_t down_grid(const FfnArgs& a) { return down_shape(a).total * (a.bf16 ? 1 : 2); }

void launch_down(const FfnArgs& a, hipStream_t stream) {
  const DownGrid g = down_shape(a);
  if (g.total == 0) return;
  if (a.bf16)
    hipLaunchKernelGGL(down_bf16_kernel, dim3((unsigned)g.total), dim3(256), 0, stream, a, g.nt,
                       g.mt_s, (int)g.routed);
  else
    hipLaunchKernelGGL(down_f32_kernel, dim3((unsigned)(g.total * 2)), dim3(256), 0, stream, a,
                       g.nt, g.mt_s, (int)g.routed);
}

}  // namespace moe
