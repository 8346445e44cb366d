// Routed and shared experts of the MoE layer as grouped GEMMs on the bf16
// matrix cores of gfx950.
//
// The routed experts are the T_routed term of the FarSkip-Collective review's
// overlap window (axiom ledger, Eq. 9); the always-on shared expert is the
// branch its Fig. 11 caption overlaps with Combine.  Grouping every expert's
// tokens into one dense product is the "Expert-Centric Scheduling" of the
// OmniMoE abstract on the "Daily Papers" search page.  The expert FFN itself
// (SwiGLU without biases, A rounded to bf16) is a reading; the pages do not
// spell it out.
//
// One kernel template serves both products.  A block computes a 128-row x
// 256-column tile with 8 waves (two per SIMD, so one wave's MFMAs issue while
// the other waits on LDS) in a 2 x 4 arrangement: 64 x 64 per wave, 4 x 4
// MFMA 16x16x32 fragments, fp32 accumulators:
//   gate/up: the 256 columns are 128 gate and the same 128 up columns of W_g
//            and W_u; a wave holds 32 gate and the matching 32 up columns,
//            so the epilogue forms bf16(silu(g) * u) in registers;
//   down:    256 output columns of y, fp32.
// Operands stream global -> LDS with the gfx950 direct 16-byte LDS loads
// (no register staging) through a ring of 3 K-steps of 64, two steps ahead
// of the MFMAs, one barrier per step.  Each 128-byte LDS row holds its eight 16-byte
// K-chunks in an order permuted by (row mod 8), which keeps the fragment
// reads at the full LDS rate.  The compiler places the LDS waits and
// interleaves fragment reads with MFMAs.  The epilogue stages the tile
// through LDS and writes whole rows with 16-byte stores.
//
// Work order: the routed tiles of expert 0, 1, ... (within an expert n-tile
// outer, m-tile inner, so consecutive tiles share a weight slice), then the
// shared experts' tiles; the expert of a routed tile is one lookup in the tile
// table the dispatch scan wrote.
#include <algorithm>

#include "grouped_gemm.h"

namespace moe {
namespace {

constexpr int BK = 64;                     // K per stage
constexpr int WROWS = 256;                 // weight rows per tile
constexpr int HALF = 128;                  // rows of each weight half
constexpr int STAGES = 3;
constexpr int ROW_BYTES = BK * 2;          // one LDS row: 64 bf16
constexpr int X_BYTES = kBM * ROW_BYTES;   // 16 KB
constexpr int W_BYTES = WROWS * ROW_BYTES; // 32 KB
constexpr int STAGE_BYTES = X_BYTES + W_BYTES;
constexpr int LDS_BYTES = STAGES * STAGE_BYTES;  // 144 KB

typedef __attribute__((address_space(3))) void* lds_void_t;

constexpr int NWAVES = 8;
constexpr int XCD_RUN = 8;  // consecutive work indices per XCD
constexpr int NTHREADS = 64 * NWAVES;

// Position permutation of the 16-byte chunks of LDS row `row`.
__device__ __forceinline__ int chunk_xor(int row) { return row & 7; }

// Hardware barrier with compiler-only fences: the waits that make LDS data
// visible are issued explicitly before it.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding; expcnt untouched).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (((N >> 4) & 0x3) << 14) | (0x7 << 4) | (0x0 << 8));
}

// Routed tile t (experts in order; within an expert n-tile outer, m-tile
// inner) -> expert e, m-tile m, n-tile n.  The expert comes from the tile
// table: t / nt lies in the expert's M-tile range.
__device__ __forceinline__ void routed_decode(const FfnArgs& p, const GemmGrid& g, int t, int& e,
                                              int& m, int& n) {
  e = p.tile_off[p.E + 1 + t / g.nt_r];
  const int m0 = p.tile_off[e];
  const int mt = p.tile_off[e + 1] - m0;
  const int local = t - m0 * g.nt_r;
  n = local / mt;
  m = local - n * mt;
}

struct BTile {
  const uint8_t* X;       // first A row (or the token rows when rmap is set)
  size_t x_ld;            // bytes between A rows
  int rows;               // valid rows
  const int32_t* rmap;    // or null: A row r is token row rmap[r] / rdiv of X
  int rdiv;
  const uint8_t* W[2];    // first row of each 128-row weight half
  int wcols[2];           // valid rows of each half
  size_t w_ld;            // bytes between weight rows
  int nk;                 // K-steps
  int kps;                // shared down tiles: K-steps per shared expert (0: one segment)
  size_t w_seg;           // bytes between shared experts' weight blocks
  uint8_t* Out;
  size_t out_ld;          // elements between output rows
  int out_cols;           // valid output columns
};

__device__ __forceinline__ void gate_up_tile(const FfnArgs& p, const GemmGrid& g, int L, int n_routed,
                                             BTile& t) {
  if (L < n_routed) {
    int e, m, n;
    routed_decode(p, g, L, e, m, n);
    const int r0 = p.offsets[e] + m * kBM;
    t.rows = min(kBM, p.offsets[e + 1] - r0);
    if (p.xs) {
      t.X = static_cast<const uint8_t*>(p.xs) + (size_t)r0 * p.d * 2;
      t.rmap = nullptr;
    } else {  // gather the token rows of x through the dispatch permutation
      t.X = static_cast<const uint8_t*>(p.x);
      t.rmap = p.perm + r0;
      t.rdiv = p.k;
    }
    const size_t w_off = ((size_t)e * p.I + (size_t)n * HALF) * p.d * 2;
    t.W[0] = static_cast<const uint8_t*>(p.wg) + w_off;
    t.W[1] = static_cast<const uint8_t*>(p.wu) + w_off;
    t.wcols[0] = t.wcols[1] = min(HALF, p.I - n * HALF);
    t.Out = static_cast<uint8_t*>(p.a) + ((size_t)r0 * p.I + (size_t)n * HALF) * 2;
    t.out_ld = p.I;
  } else {
    const int sb = L - n_routed;
    const int per_s = g.mt_s * g.nt_s;
    const int s = sb / per_s, rem = sb - s * per_s;
    const int n = rem / g.mt_s, m = rem - n * g.mt_s;
    const int r0 = m * kBM;
    t.rows = (int)min((int64_t)kBM, p.T - r0);
    t.X = static_cast<const uint8_t*>(p.x) + (size_t)r0 * p.d * 2;
    t.rmap = nullptr;
    const size_t w_off = ((size_t)s * p.Is + (size_t)n * HALF) * p.d * 2;
    t.W[0] = static_cast<const uint8_t*>(p.wsg) + w_off;
    t.W[1] = static_cast<const uint8_t*>(p.wsu) + w_off;
    t.wcols[0] = t.wcols[1] = min(HALF, p.Is - n * HALF);
    const size_t ld = (size_t)p.ns * p.Is;
    t.Out = static_cast<uint8_t*>(p.ash) + ((size_t)r0 * ld + (size_t)s * p.Is + (size_t)n * HALF) * 2;
    t.out_ld = ld;
  }
  t.x_ld = (size_t)p.d * 2;
  t.w_ld = (size_t)p.d * 2;
  t.nk = p.d / BK;
  t.kps = 0;
  t.w_seg = 0;
  t.out_cols = t.wcols[0];
}

__device__ __forceinline__ void down_tile(const FfnArgs& p, const GemmGrid& g, int L, int n_routed,
                                          BTile& t) {
  int n, r0;
  const uint8_t* w0;
  if (L < n_routed) {
    int e, m;
    routed_decode(p, g, L, e, m, n);
    r0 = p.offsets[e] + m * kBM;
    t.rows = min(kBM, p.offsets[e + 1] - r0);
    t.X = static_cast<const uint8_t*>(p.a) + (size_t)r0 * p.I * 2;
    t.x_ld = (size_t)p.I * 2;
    w0 = static_cast<const uint8_t*>(p.wd) + ((size_t)e * p.d + (size_t)n * WROWS) * p.I * 2;
    t.w_ld = (size_t)p.I * 2;
    t.nk = p.I / BK;
    t.kps = 0;
    t.w_seg = 0;
    t.Out = reinterpret_cast<uint8_t*>(p.y + (size_t)r0 * p.d + (size_t)n * WROWS);
  } else {
    const int sb = L - n_routed;
    n = sb / g.mt_s;
    const int m = sb - n * g.mt_s;
    r0 = m * kBM;
    t.rows = (int)min((int64_t)kBM, p.T - r0);
    const size_t ld = (size_t)p.ns * p.Is;
    t.X = static_cast<const uint8_t*>(p.ash) + (size_t)r0 * ld * 2;
    t.x_ld = ld * 2;
    w0 = static_cast<const uint8_t*>(p.wsd) + (size_t)n * WROWS * p.Is * 2;
    t.w_ld = (size_t)p.Is * 2;
    t.nk = (int)(ld / BK);
    t.kps = p.Is / BK;
    t.w_seg = (size_t)p.d * p.Is * 2;
    t.Out = reinterpret_cast<uint8_t*>(p.ysh + (size_t)r0 * p.d + (size_t)n * WROWS);
  }
  t.rmap = nullptr;
  const int left = p.d - n * WROWS;  // output columns from this tile on
  t.W[0] = w0;
  t.wcols[0] = min(HALF, left);
  if (left > HALF) {
    t.W[1] = w0 + (size_t)HALF * t.w_ld;
    t.wcols[1] = min(HALF, left - HALF);
  } else {  // no second half: load valid rows of the first, results are dropped
    t.W[1] = w0;
    t.wcols[1] = t.wcols[0];
  }
  t.out_ld = p.d;
  t.out_cols = min(WROWS, left);
}

// One tile: pipeline fill, K loop and epilogue.  Ends with the LDS free.
template <bool GATE_UP>
__device__ __forceinline__ void run_tile(const BTile& t, uint8_t* smem) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;


  // ---- loader: 2 X and 4 W direct-to-LDS loads of 1 KB (8 rows) per wave per step
  const uint8_t* src[6];
  {
    const int sub = lane >> 3, pos = lane & 7;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = wave * 16 + q * 8 + sub;
      const int c = pos ^ chunk_xor(row);
      const int rr = min(row, t.rows - 1);
      const size_t xrow = t.rmap ? (size_t)(t.rmap[rr] / t.rdiv) : (size_t)rr;
      src[q] = t.X + xrow * t.x_ld + c * 16;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = wave * 32 + q * 8 + sub;  // 0..255
      const bool hi = row >= HALF;
      const int r = row & (HALF - 1);
      const int c = pos ^ chunk_xor(row);
      const uint8_t* base = hi ? t.W[1] : t.W[0];
      const int valid = hi ? t.wcols[1] : t.wcols[0];
      src[2 + q] = base + (size_t)min(r, valid - 1) * t.w_ld + c * 16;
    }
  }
  auto issue = [&](int kt) {
    uint8_t* st = smem + (kt % STAGES) * STAGE_BYTES;
    const size_t xo = (size_t)kt * ROW_BYTES;
    const size_t wo = t.kps ? (size_t)(kt / t.kps) * t.w_seg + (size_t)(kt % t.kps) * ROW_BYTES
                            : (size_t)kt * ROW_BYTES;
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_global_load_lds(src[q] + xo, (lds_void_t)(st + (wave * 16 + q * 8) * ROW_BYTES),
                                       16, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_global_load_lds(src[2 + q] + wo,
                                       (lds_void_t)(st + X_BYTES + (wave * 32 + q * 8) * ROW_BYTES),
                                       16, 0, 0);
  };

  // ---- fragment addresses (bytes within a stage)
  const int r16 = lane & 15, kg = lane >> 4;
  const int lane_off = r16 * ROW_BYTES + ((kg ^ chunk_xor(r16)) << 4);  // K-chunk kg; +32 K: ^64
  int a_off[4], b_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a_off[i] = (wm * 64 + i * 16) * ROW_BYTES + lane_off;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int wrow = GATE_UP ? (j < 2 ? wn * 32 + j * 16 : HALF + wn * 32 + (j - 2) * 16)
                             : wn * 64 + j * 16;
    b_off[j] = X_BYTES + wrow * ROW_BYTES + lane_off;
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = t.nk;
  issue(0);
  if (nk > 1) issue(1);
  for (int kt = 0; kt < nk; ++kt) {
    // this step's loads have landed (the next step's 6 may still be in flight)
    if (kt + 1 < nk) wait_vm_lgkm0<6>();
    else wait_vm_lgkm0<0>();
    block_barrier();
    if (kt + 2 < nk) issue(kt + 2);  // into the stage of step kt-1, read by everyone now
    const uint8_t* st = smem + (kt % STAGES) * STAGE_BYTES;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kx = ks * 64;  // second half of the step: K-chunks 4..7
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = as_bf16x8(ld_u32x4(st + (a_off[i] ^ kx)));
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = as_bf16x8(ld_u32x4(st + (b_off[j] ^ kx)));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_16x16x32_bf16(a[i], b[j], acc[i][j]);
    }
  }

  // ---- epilogue through LDS
  wait_vm_lgkm0<0>();
  block_barrier();
  if (GATE_UP) {
    constexpr int LD = HALF + 8;  // bf16 per staged row
    uint16_t* stg = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = wm * 64 + i * 16 + kg * 4 + q;
          const int col = wn * 32 + j * 16 + r16;
          stg[row * LD + col] = f32_to_bf16_bits(silu_times(acc[i][j][q], acc[i][j + 2][q]));
        }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    block_barrier();
    uint16_t* out = reinterpret_cast<uint16_t*>(t.Out);
    for (int c = tid; c < kBM * (HALF / 8); c += NTHREADS) {
      const int row = c >> 4, ch = c & 15;
      if (row < t.rows && ch * 8 < t.out_cols)
        *reinterpret_cast<u32x4*>(out + (size_t)row * t.out_ld + ch * 8) =
            *reinterpret_cast<const u32x4*>(stg + row * LD + ch * 8);
    }
  } else {
    constexpr int LD = WROWS + 4;  // floats per staged row
    float* stg = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = wm * 64 + i * 16 + kg * 4 + q;
          const int col = wn * 64 + j * 16 + r16;
          stg[row * LD + col] = acc[i][j][q];
        }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    block_barrier();
    float* out = reinterpret_cast<float*>(t.Out);
    for (int c = tid; c < kBM * (WROWS / 4); c += NTHREADS) {
      const int row = c >> 6, ch = c & 63;
      if (row < t.rows && ch * 4 < t.out_cols)
        *reinterpret_cast<u32x4*>(out + (size_t)row * t.out_ld + ch * 4) =
            *reinterpret_cast<const u32x4*>(stg + row * LD + ch * 4);
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): staged reads done before the LDS is reused
  block_barrier();
}

// Launch slot -> work index: blocks are dealt to the 8 XCDs round-robin, so
// slot b runs on XCD b % 8; each XCD receives runs of XCD_RUN consecutive work
// indices, tiles that share weight slices, in its own L2.
__device__ __forceinline__ int xcd_remap(int bid) {
  const int run = 8 * XCD_RUN;
  const int base = bid / run * run, w = bid - base;
  return base + (w & 7) * XCD_RUN + (w >> 3);
}

// One block per work slot; slots past the device-side tile count return.
template <bool GATE_UP>
__global__ __launch_bounds__(NTHREADS) void grouped_gemm_bf16_kernel(FfnArgs p, GemmGrid g) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];
  const int n_routed = p.tile_off[p.E] * g.nt_r;
  const int L = xcd_remap(blockIdx.x);
  if (L >= n_routed + g.n_shared) return;
  BTile t;
  if (GATE_UP) gate_up_tile(p, g, L, n_routed, t);
  else down_tile(p, g, L, n_routed, t);
  run_tile<GATE_UP>(t, smem);
}

GemmGrid bf16_gate_up_grid(const FfnArgs& a) {
  GemmGrid g;
  g.mtb = (int)routed_mtile_bound(a.R, a.E);
  g.nt_r = (a.I + HALF - 1) / HALF;
  g.nt_s = a.ns ? (a.Is + HALF - 1) / HALF : 0;
  g.mt_s = (int)((a.T + kBM - 1) / kBM);
  g.n_shared = a.ns * g.nt_s * g.mt_s;
  g.routed = (int64_t)g.mtb * g.nt_r;
  g.total = g.routed + g.n_shared;
  return g;
}

int64_t pad_slots(int64_t n) { return (n + 8 * XCD_RUN - 1) / (8 * XCD_RUN) * (8 * XCD_RUN); }

GemmGrid bf16_down_grid(const FfnArgs& a) {
  GemmGrid g;
  g.mtb = (int)routed_mtile_bound(a.R, a.E);
  g.nt_r = (a.d + WROWS - 1) / WROWS;
  g.nt_s = g.nt_r;
  g.mt_s = (int)((a.T + kBM - 1) / kBM);
  g.n_shared = a.ns ? g.nt_r * g.mt_s : 0;
  g.routed = (int64_t)g.mtb * g.nt_r;
  g.total = g.routed + g.n_shared;
  return g;
}

}  // namespace

int64_t gate_up_grid_bf16(const FfnArgs& a) { return pad_slots(bf16_gate_up_grid(a).total); }
int64_t down_grid_bf16(const FfnArgs& a) { return pad_slots(bf16_down_grid(a).total); }

void launch_gate_up_bf16(const FfnArgs& a, hipStream_t stream) {
  const GemmGrid g = bf16_gate_up_grid(a);
  if (g.total == 0) return;
  hipLaunchKernelGGL(grouped_gemm_bf16_kernel<true>, dim3((unsigned)pad_slots(g.total)),
                     dim3(NTHREADS), 0, stream, a, g);
}

void launch_down_bf16(const FfnArgs& a, hipStream_t stream) {
  const GemmGrid g = bf16_down_grid(a);
  if (g.total == 0) return;
  hipLaunchKernelGGL(grouped_gemm_bf16_kernel<false>, dim3((unsigned)pad_slots(g.total)),
                     dim3(NTHREADS), 0, stream, a, g);
}

}  // namespace moe
