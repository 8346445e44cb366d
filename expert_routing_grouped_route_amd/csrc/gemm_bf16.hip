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
// One kernel template serves both products.  What bounds it is the number of
// 128-byte cache lines a CU can have in flight between its L1 and L2, so the
// block tile is the largest square the accumulators allow: 256 rows x 256
// weight rows, 8 waves (two per SIMD) in a 2 x 4 arrangement, each wave 128
// rows x 64 weight rows as 4 x 2 MFMA 32x32x16 tiles with fp32 accumulators.
// The weight fragment is the MFMA's first operand, so a lane ends with four
// consecutive output columns of one row:
//   gate/up: the 256 weight rows are 128 gate and the same 128 up rows of
//            W_g and W_u; a wave holds 32 gate and the matching 32 up
//            columns, so the epilogue forms bf16(silu(g) * u) in registers;
//   down:    256 output columns of y, fp32.
// Operands stream global -> LDS with the gfx950 direct 16-byte LDS loads (no
// register staging) in K-steps of 64, one barrier per step: the A rows through
// three 32 KB buffers, loaded two steps ahead, the weight rows through two,
// loaded one step ahead (160 KB of LDS in all).  The loads are spread between
// the MFMAs of the current step, so no wave stalls on a full memory queue
// while its matrix core idles; fragment reads run one K-sub-step ahead of the
// MFMAs that use them.
// Each 128-byte LDS row holds its eight 16-byte K-chunks in an order permuted
// by (row / 2 mod 8), which keeps the 32-row fragment reads free of bank
// conflicts.  The forward epilogues stage their tiles through LDS and store
// whole rows: the gate/up's bf16 A in one pass, the down's fp32 y in two
// halves; the raw gate/up epilogue of the backward pass stores fp32 G and U
// from registers.
//
// Work order: the routed tiles of expert 0, 1, ... (within an expert groups of
// 4 m-tiles, n-tile outer and m-tile inner within a group), then the shared
// experts' tiles in the same raster (for the down product the shared tiles
// come first, being the longest); the expert of a routed tile is one lookup in
// the tile table the dispatch scan wrote.  Each XCD takes runs of 8
// consecutive works, which share A-row tiles and weight slices in its L2.
#include <algorithm>
#include <type_traits>

#include "grouped_gemm.h"

namespace moe {
namespace {

static_assert(kBM == 256, "the bf16 tile is 256 rows");
constexpr int BK = 64;                          // K per stage
constexpr int BN = 256;                         // weight rows per tile
constexpr int GU_COLS = BN / 2;                 // gate/up: output columns per tile
constexpr int ROW_BYTES = BK * 2;               // one LDS row: 64 bf16
constexpr int X_BYTES = kBM * ROW_BYTES;        // 32 KB
// The A rows (X) are the deep operand: three buffers, loaded two K-steps
// ahead; the weight rows have two buffers and are loaded one step ahead.
constexpr bool DEEP_X = true;
constexpr int W_BYTES = BN * ROW_BYTES;         // 32 KB
constexpr int NXB = DEEP_X ? 3 : 2;             // buffers of the A rows (X) ...
constexpr int NWB = DEEP_X ? 2 : 3;             // ... and of the weight rows
constexpr int W_BASE = NXB * X_BYTES;
constexpr int LDS_BYTES = NXB * X_BYTES + NWB * W_BYTES;  // 160 KB

constexpr int NWAVES = 8;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int XLOADS = kBM / 8 / NWAVES;        // 1 KB direct loads per wave per stage: 4 of X
constexpr int WLOADS = BN / 8 / NWAVES;         // and 4 of weights
constexpr int LOADS = XLOADS + WLOADS;          // 8
// Work placement (measured on the prefill-scale and DeepSeek-V2-Lite layers):
// the gate/up product takes runs of 16 consecutive works per XCD over a
// raster of 8 m-tiles, the down product runs of 8 over a raster of 4.
constexpr int GU_RUN = 16, GU_GROUP_M = 8;
constexpr int DN_RUN = 8, DN_GROUP_M = 4;
constexpr int SEG_RUN = 8;                      // the backward's segment products

typedef __attribute__((address_space(3))) void* lds_void_t;

// Raw buffer descriptor for an operand: base address, no stride, the full
// 32-bit range (offsets are checked on the host), default data format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint8_t* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, -1, 0x00020000);
}
// The same with a byte range: loads at offsets past `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_n(const uint8_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, __builtin_bit_cast(int, bytes),
                                           0x00020000);
}

// Position permutation of the 16-byte chunks of LDS row `row`.
__device__ __forceinline__ int chunk_xor(int row) { return (row >> 1) & 7; }

// gfx950 transposing LDS read of 16-bit elements (ds_read_b64_tr_b16).
// Within each group of 16 lanes, lane j = 4m + q passes the address of 4
// consecutive elements; lane i of the group receives element i % 4 of the
// reads of lanes 4m + i / 4, m = 0..3.  So if lane 4m + q points at row
// k0 + m, columns c0 + 4q .. +3 of a row-major tile, lane i receives rows
// k0 .. k0 + 3 of column c0 + i.
// Two such reads per operand fragment, at a0 and a0 + 2048 (rows k0 + 4 ..),
// for two fragments, then a wait for them in the same block (the outputs are
// complete when it ends).  Written out because the compiler puts a wait for
// every outstanding global load before its builtin form (it cannot tell the
// read from the direct-to-LDS loads still in flight into other buffers); the
// LDS stage read here is made visible by the K loop's own waits and barrier.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void lds_read_tr16_frags(uint32_t a0, uint32_t a1, bf16x8& f0,
                                                    bf16x8& f1) {
  u32x2 l0, h0, l1, h1;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %4 offset:2048\n\t"
      "ds_read_b64_tr_b16 %2, %5\n\t"
      "ds_read_b64_tr_b16 %3, %5 offset:2048\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(l0), "=&v"(h0), "=&v"(l1), "=&v"(h1)
      : "v"(a0), "v"(a1)
      : "memory");
  f0 = __builtin_bit_cast(bf16x8, u32x4{l0.x, l0.y, h0.x, h0.y});
  f1 = __builtin_bit_cast(bf16x8, u32x4{l1.x, l1.y, h1.x, h1.y});
}

// The same for six fragments (both operands of a K-major sub-step) in one
// block: twelve reads, then one wait, so a wave waits for the LDS once per
// sub-step instead of once per pair of fragments.
__device__ __forceinline__ void lds_read_tr16_frags6(uint32_t a0, uint32_t a1, uint32_t a2,
                                                     uint32_t a3, uint32_t a4, uint32_t a5,
                                                     bf16x8 (&f)[6]) {
  u32x2 l0, h0, l1, h1, l2, h2, l3, h3, l4, h4, l5, h5;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %12\n\t"
      "ds_read_b64_tr_b16 %1, %12 offset:2048\n\t"
      "ds_read_b64_tr_b16 %2, %13\n\t"
      "ds_read_b64_tr_b16 %3, %13 offset:2048\n\t"
      "ds_read_b64_tr_b16 %4, %14\n\t"
      "ds_read_b64_tr_b16 %5, %14 offset:2048\n\t"
      "ds_read_b64_tr_b16 %6, %15\n\t"
      "ds_read_b64_tr_b16 %7, %15 offset:2048\n\t"
      "ds_read_b64_tr_b16 %8, %16\n\t"
      "ds_read_b64_tr_b16 %9, %16 offset:2048\n\t"
      "ds_read_b64_tr_b16 %10, %17\n\t"
      "ds_read_b64_tr_b16 %11, %17 offset:2048\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(l0), "=&v"(h0), "=&v"(l1), "=&v"(h1), "=&v"(l2), "=&v"(h2), "=&v"(l3), "=&v"(h3),
        "=&v"(l4), "=&v"(h4), "=&v"(l5), "=&v"(h5)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(a4), "v"(a5)
      : "memory");
  f[0] = __builtin_bit_cast(bf16x8, u32x4{l0.x, l0.y, h0.x, h0.y});
  f[1] = __builtin_bit_cast(bf16x8, u32x4{l1.x, l1.y, h1.x, h1.y});
  f[2] = __builtin_bit_cast(bf16x8, u32x4{l2.x, l2.y, h2.x, h2.y});
  f[3] = __builtin_bit_cast(bf16x8, u32x4{l3.x, l3.y, h3.x, h3.y});
  f[4] = __builtin_bit_cast(bf16x8, u32x4{l4.x, l4.y, h4.x, h4.y});
  f[5] = __builtin_bit_cast(bf16x8, u32x4{l5.x, l5.y, h5.x, h5.y});
}

// Hardware barrier with compiler-only fences: the waits that make LDS data
// visible are issued explicitly before it.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(0) lgkmcnt(0) (gfx9 encoding; expcnt untouched).
__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0x70); }

// Tile l of an mt x nt grid in raster order: groups of GM m-tiles, and
// within a group n-tile outer, m-tile inner.  So with GM = 4 a run of 8
// consecutive tiles of a large expert spans 4 m-tiles (A rows) and 2 n-tiles
// (weight slices): 6 operand tiles for 8 output tiles, where a run along one
// n-tile would need 9.
__device__ __forceinline__ void raster(int l, int mt, int nt, int GM, int& m, int& n) {
  const int gsize = GM * nt;
  const int q = l / gsize, r = l - q * gsize;
  const int gm = min(GM, mt - q * GM);
  n = r / gm;
  m = q * GM + (r - n * gm);
}

// Routed tile t (experts in order; within an expert the raster above) ->
// expert e, m-tile m, n-tile n.  An expert's tiles are [m0 * nt, (m0 + mt) *
// nt) for its M-tile range [m0, m0 + mt), so the tile table's entry t / nt
// names the expert.
__device__ __forceinline__ void routed_decode(const FfnArgs& p, const GemmGrid& g, int t, int& e,
                                              int& m, int& n) {
  e = p.tile_off[p.E + 1 + t / g.nt_r];
  const int m0 = p.tile_off[e];
  const int mt = p.tile_off[e + 1] - m0;
  raster(t - m0 * g.nt_r, mt, g.nt_r, g.gm, m, n);
}

struct BTile {
  const uint8_t* X;       // first A row (or the token rows when rmap is set)
  size_t x_ld;            // bytes between A rows
  int rows;               // valid rows
  const int32_t* rmap;    // or null: A row r is token row rmap[r] / rdiv of X
  int rdiv;
  const uint8_t* W[2];    // gate/up: first gate and first up row; down: first row (both)
  int wrows;              // valid weight rows of each half (gate/up) or of the tile (down)
  size_t w_ld;            // bytes between weight rows
  int nk;                 // K-steps
  int kps;                // K-steps per K block (0: one block; shared down tiles: per expert)
  int wsh;                // PARTS tiles: 2^wsh K blocks share one weight block
  size_t w_seg;           // bytes between weight blocks
  uint8_t* Out;           // element (0, 0) of the tile
  size_t out_ld;          // elements between output rows
  int out_cols;           // valid output columns (a multiple of 64)
  int64_t raw_off;        // gate/up RAW: element offset of the tile's (0, 0) in G and U
  // K-major A (KX tiles): bytes between its K blocks, and the byte ranges of
  // the A and weight buffer descriptors (loads past them read zeros)
  size_t x_seg;
  uint32_t x_bytes, w_bytes;
  int kt0;                // KX tiles: K-step of the operands' layout where this tile starts
};

template <bool RAW = false>  // RAW: also the tile's offset in the raw G and U arrays
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
    const size_t w_off = ((size_t)e * p.I + (size_t)n * GU_COLS) * p.d * 2;
    t.W[0] = static_cast<const uint8_t*>(p.wg) + w_off;
    t.W[1] = static_cast<const uint8_t*>(p.wu) + w_off;
    t.wrows = min(GU_COLS, p.I - n * GU_COLS);
    t.Out = static_cast<uint8_t*>(p.a) + ((size_t)r0 * p.I + (size_t)n * GU_COLS) * 2;
    t.out_ld = p.I;
    if (RAW) t.raw_off = (int64_t)r0 * p.I + (int64_t)n * GU_COLS;
  } else {
    const int sb = L - n_routed;
    const int per_s = g.mt_s * g.nt_s;
    const int s = sb / per_s;
    int m, n;
    raster(sb - s * per_s, g.mt_s, g.nt_s, g.gm, m, n);
    const int r0 = m * kBM;
    t.rows = (int)min((int64_t)kBM, p.T - r0);
    t.X = static_cast<const uint8_t*>(p.x) + (size_t)r0 * p.d * 2;
    t.rmap = nullptr;
    const size_t w_off = ((size_t)s * p.Is + (size_t)n * GU_COLS) * p.d * 2;
    t.W[0] = static_cast<const uint8_t*>(p.wsg) + w_off;
    t.W[1] = static_cast<const uint8_t*>(p.wsu) + w_off;
    t.wrows = min(GU_COLS, p.Is - n * GU_COLS);
    const size_t ld = (size_t)p.ns * p.Is;
    t.Out = static_cast<uint8_t*>(p.ash) + ((size_t)r0 * ld + (size_t)s * p.Is + (size_t)n * GU_COLS) * 2;
    t.out_ld = ld;
    if (RAW) t.raw_off = (int64_t)r0 * ld + (int64_t)s * p.Is + (int64_t)n * GU_COLS;
  }
  t.x_ld = (size_t)p.d * 2;
  t.w_ld = (size_t)p.d * 2;
  t.nk = p.d / BK;
  t.kps = 0;
  t.w_seg = 0;
  t.out_cols = t.wrows;
}

// PARTS: the routed rows of `a` may hold a_parts K blocks (FfnArgs::a_parts).
// WT (routed tiles): weights in their stored layout (FfnArgs::wt).
template <bool PARTS = false, bool WT = false>
__device__ __forceinline__ void down_tile(const FfnArgs& p, const GemmGrid& g, int L, int n_routed,
                                          BTile& t) {
  int n, r0;
  const uint8_t* w0;
  if (L < n_routed) {
    int e, m;
    routed_decode(p, g, L, e, m, n);
    r0 = p.offsets[e] + m * kBM;
    t.rows = min(kBM, p.offsets[e + 1] - r0);
    const int parts = PARTS && p.a_parts > 1 ? p.a_parts : 1;  // blocks of I columns per A row
    t.X = static_cast<const uint8_t*>(p.a) + (size_t)r0 * parts * p.I * 2;
    t.x_ld = (size_t)parts * p.I * 2;
    w0 = static_cast<const uint8_t*>(p.wd) + ((size_t)e * p.d + (size_t)n * BN) * p.I * 2;
    t.w_ld = (size_t)p.I * 2;
    t.nk = parts * (p.I / BK);
    t.kps = parts > 1 ? p.I / BK : 0;
    if (PARTS) t.wsh = 1;  // the hi and lo blocks of one operand share a weight
    t.w_seg = parts > 1 ? (size_t)p.w_part * 2 : 0;
    if (WT) {  // expert e's [I][d] block (K-rows of d elements), from column n * BN
      const size_t eo = ((size_t)e * p.I * p.d + (size_t)n * BN) * 2;
      w0 = static_cast<const uint8_t*>(p.wd) + eo;
      t.w_ld = (size_t)p.d * 2;
      t.w_seg = 0;
    }
    t.Out = reinterpret_cast<uint8_t*>(p.y + (size_t)r0 * p.d + (size_t)n * BN);
  } else {
    int m;
    raster(L - n_routed, g.mt_s, g.nt_r, g.gm, m, n);
    r0 = m * kBM;
    t.rows = (int)min((int64_t)kBM, p.T - r0);
    const size_t ld = (size_t)p.ns * p.Is;
    t.X = static_cast<const uint8_t*>(p.ash) + (size_t)r0 * ld * 2;
    t.x_ld = ld * 2;
    w0 = static_cast<const uint8_t*>(p.wsd) + (size_t)n * BN * p.Is * 2;
    t.w_ld = (size_t)p.Is * 2;
    t.nk = (int)(ld / BK);
    t.kps = p.Is / BK;
    if (PARTS) t.wsh = 0;
    t.w_seg = (size_t)p.d * p.Is * 2;
    t.Out = reinterpret_cast<uint8_t*>(p.ysh + (size_t)r0 * p.d + (size_t)n * BN);
  }
  t.rmap = nullptr;
  if (PARTS && L < n_routed && p.perm) {  // A row r is token row perm[r] / k of `a`
    t.X = static_cast<const uint8_t*>(p.a);
    t.rmap = p.perm + r0;
    t.rdiv = p.k;
  }
  t.W[0] = t.W[1] = w0;
  if (WT && L < n_routed && p.wd2)
    t.W[1] = static_cast<const uint8_t*>(p.wd2) + (w0 - static_cast<const uint8_t*>(p.wd));
  t.wrows = min(BN, p.d - n * BN);
  t.out_ld = p.d;
  t.out_cols = t.wrows;
}

// One tile: pipeline fill, K loop and epilogue.
// BUF: the operands stream in through buffer loads (a descriptor per operand
// and 32-bit lane offsets), which cost the address path less than 64-bit
// global addresses; the launcher uses them when every operand offset fits in
// 32 bits.
// RAW (gate/up): store G and U as fp32 (and, with a_raw, the SwiGLU product
// in bf16 at the same element offsets).
// NT (down): store the fp32 output with non-temporal stores, for outputs larger
// than the MALL (they stream to memory instead of filling the L2 with dirty
// lines; smaller outputs stay cached for the combine that reads them next).
// WT (down product only): the weight tile arrives as 64 K-rows of 256 output
// columns (the weights' stored layout, reduction index outer) and its MFMA
// fragments come out of LDS through transposing reads.
// KX (with WT and BUF): the A tile too arrives as 64 K-rows of 256 rows of
// the output (an operand stored with the reduction index outer), K blocks
// t.x_seg bytes apart, and loads past t.x_bytes / t.w_bytes read zeros.
template <bool GATE_UP, bool BUF, bool RAW = false, bool PARTS = false, bool NT = false,
          bool WT = false, bool KX = false>
__device__ __forceinline__ void run_tile(const BTile& t, uint8_t* smem, float* g_raw = nullptr,
                                         float* u_raw = nullptr, uint16_t* a_raw = nullptr) {
  static_assert(!WT || !GATE_UP, "k-major weights: down product only");
  static_assert(!KX || (WT && BUF && !PARTS), "k-major A: with k-major weights, buffer loads");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wm = wave >> 2, wn = wave & 3;

  // ---- loader.  Direct load q of a wave fills 8 LDS rows (1 KB): lane L
  // writes row (L / 8), position L % 8, which holds K-chunk (L % 8) ^ chunk_xor(row).
  // X: LDS rows wave*32 + q*8 + L/8 (q < 4).  Weights: LDS rows 256 + wave*32 +
  // q*8 + L/8 (q < 4): gate/up waves 0..3 load gate rows, waves 4..7 up rows.
  const int sub = lane >> 3, pos = lane & 7;
  size_t xoff[XLOADS];  // byte offsets from t.X (below 2^32 with BUF)
#pragma unroll
  for (int q = 0; q < XLOADS; ++q) {
    if (KX) {  // as the K-major weight tile below, over the tile's 256 A rows
      const int kr = 2 * (wave * XLOADS + q) + (lane >> 5);
      const int cl = min((lane & 31) ^ ((kr & 3) << 2), (t.rows >> 3) - 1);
      xoff[q] = (size_t)kr * t.x_ld + (cl << 4);
    } else {
      const int row = wave * (8 * XLOADS) + q * 8 + sub;
      const int rr = min(row, t.rows - 1);
      const size_t xrow = t.rmap ? (size_t)(t.rmap[rr] / t.rdiv) : (size_t)rr;
      xoff[q] = xrow * t.x_ld + ((pos ^ chunk_xor(row)) << 4);
    }
  }
  const uint8_t* wbase;  // wave-uniform
  int wfirst;            // first weight row of this wave within its half (gate/up) or tile (down)
  if (GATE_UP) {
    wbase = wave < 4 ? t.W[0] : t.W[1];
    wfirst = (wave & 3) * (8 * WLOADS);
  } else {
    wbase = t.W[0];
    wfirst = wave * (8 * WLOADS);
  }
  uint32_t woff[WLOADS];  // byte offsets from wbase, rows clamped to the valid ones
#pragma unroll
  for (int q = 0; q < WLOADS; ++q) {
    if (WT) {
      // load q fills K-rows 2 (wave*WLOADS + q) + L/32 of the stage (512 bytes
      // each): lane L writes chunk position L % 32, which holds the chunk of
      // 8 columns (L % 32) ^ (4 (row % 4)); columns past the valid ones read
      // the last valid chunk (their outputs are not stored)
      const int kr = 2 * (wave * WLOADS + q) + (lane >> 5);
      const int cl = min((lane & 31) ^ ((kr & 3) << 2), (t.wrows >> 3) - 1);
      woff[q] = (uint32_t)((size_t)kr * t.w_ld) + (cl << 4);
    } else {
      const int r = wfirst + q * 8 + sub;  // its LDS row kBM + wave*32 + q*8 + sub has the same row mod 16
      woff[q] = (uint32_t)((size_t)min(r, t.wrows - 1) * t.w_ld) + ((pos ^ chunk_xor(r)) << 4);
    }
  }
  // weight byte offset of K-step kt (the shared down tiles' K runs over the
  // shared experts' blocks one after the other)
  auto w_step = [&](int kt) -> size_t {
    if (KX) return (size_t)((kt + t.kt0) % t.kps) * BK * t.w_ld;
    if (WT) return (size_t)(t.kps ? kt % t.kps : kt) * BK * t.w_ld;  // K-rows within the weight block
    return t.kps ? (size_t)(PARTS ? (kt / t.kps) >> t.wsh : kt / t.kps) * t.w_seg +
                       (size_t)(kt % t.kps) * ROW_BYTES
                 : (size_t)kt * ROW_BYTES;
  };
  // direct loads of K-step kt: X load q (0..XLOADS-1), weight load q (0..WLOADS-1)
  const __amdgpu_buffer_rsrc_t x_rsrc = KX ? make_rsrc_n(t.X, t.x_bytes) : make_rsrc(t.X);
  const __amdgpu_buffer_rsrc_t w_rsrc = KX ? make_rsrc_n(wbase, t.w_bytes) : make_rsrc(wbase);
  // WT: K-steps from kb1 on read weight block 1 (t.W[1]): with up to four K
  // blocks of A, blocks 2 and 3 share weight block 1
  const uint8_t* const wbase1 = WT ? t.W[1] : wbase;
  const int kb1 = t.kps ? (t.kps << (PARTS ? t.wsh : 0)) : (1 << 30);
  auto issue_x = [&](int kt, int q) {
    const lds_void_t dst =
        (lds_void_t)(smem + (kt % NXB) * X_BYTES + (wave * (8 * XLOADS) + q * 8) * ROW_BYTES);
    if (KX) {
      // K block kt / kps, its K-rows (kt % kps) * 64 ..: the whole offset in
      // the lane offset, which the descriptor's range check covers
      const int g = kt + t.kt0;
      const uint32_t ks_off =
          (uint32_t)((size_t)(g / t.kps) * t.x_seg + (size_t)(g % t.kps) * BK * t.x_ld);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(x_rsrc, dst, 16, (uint32_t)xoff[q] + ks_off, 0, 0,
                                               0);
    } else if (BUF) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(x_rsrc, dst, 16, (uint32_t)xoff[q],
                                               (uint32_t)(kt * ROW_BYTES), 0, 0);
    }
    else
      __builtin_amdgcn_global_load_lds(t.X + xoff[q] + (size_t)kt * ROW_BYTES, dst, 16, 0, 0);
  };
  auto issue_w = [&](int kt, size_t wstep, int q) {
    const lds_void_t dst = (lds_void_t)(smem + W_BASE + (kt % NWB) * W_BYTES +
                                        (wave * (8 * WLOADS) + q * 8) * ROW_BYTES);
    if (WT) {
      const uint8_t* wb = kt >= kb1 ? wbase1 : wbase;  // wave-uniform
      if (KX)  // one weight block, through the ranged descriptor, offset in the lane
        __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc, dst, 16, woff[q] + (uint32_t)wstep, 0, 0,
                                                 0);
      else if (BUF)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(wb), dst, 16, woff[q], (uint32_t)wstep,
                                                 0, 0);
      else
        __builtin_amdgcn_global_load_lds(wb + wstep + woff[q], dst, 16, 0, 0);
    } else if (BUF) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc, dst, 16, woff[q], (uint32_t)wstep, 0, 0);
    } else {
      __builtin_amdgcn_global_load_lds(wbase + wstep + woff[q], dst, 16, 0, 0);
    }
  };

  // ---- fragments (bytes within a stage).  MFMA 32x32x16: lane l reads row
  // (l % 32) with K-chunk 2s + l/32 of sub-step s.  First operand: 32 weight
  // rows (output columns); second: 32 A rows.
  const int r32 = lane & 31, kg = lane >> 5;
  const int cx = chunk_xor(r32);
  int a_off[4], b_off[2];
  // transposing-read lane roles (KX and WT tiles): source row (l % 16) / 4,
  // column group l % 4, half-group (l / 16) % 2
  const int mq = (lane & 15) >> 2, qq = lane & 3, g2 = (lane >> 4) & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (KX) {  // as b_off below, for the 32 A rows wm*128 + i*32 ..
      const int chunk = ((wm * 128 + i * 32) >> 3) + 2 * g2 + (qq >> 1);
      a_off[i] = (8 * kg + mq) * (kBM * 2) + ((chunk ^ (mq << 2)) << 4) + (qq & 1) * 8;
    } else {
      a_off[i] = (wm * 128 + i * 32 + r32) * ROW_BYTES;
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int wrow = GATE_UP ? j * GU_COLS + wn * 32 : wn * 64 + j * 32;
    if (WT) {
      // transposing reads of the K-major stage (512-byte rows): lane l needs
      // columns wrow + l % 32 at K-rows 16 s + 8 (l / 32) + 0..7 of sub-step s,
      // two reads of 4 rows each; as a source lane it points at K-row
      // 8 (l / 32) + (l % 16) / 4 (+ 16 s, + 4 for the second read), columns
      // wrow + 16 ((l / 16) % 2) + 4 (l % 4) .. +3, in the row's swizzled chunk
      const int chunk = (wrow >> 3) + 2 * g2 + (qq >> 1);
      b_off[j] = (8 * kg + mq) * (BN * 2) + ((chunk ^ (mq << 2)) << 4) + (qq & 1) * 8;
    } else {
      b_off[j] = (wrow + r32) * ROW_BYTES;
    }
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // K loop.  The A rows are loaded into three buffers, the weight rows into
  // two.  The block barrier that makes step kt+1's operands visible to every
  // wave sits inside step kt, before its last 8 MFMAs: each wave first waits
  // for its own loads of step kt+1 and for its fragment reads of step kt, then
  // passes the barrier, issues the fragment reads of step kt+1's first
  // sub-step, and only then runs step kt's last MFMAs, which cover the
  // barrier's skew and the LDS read latency.  Past that barrier every read of
  // step kt is done, so step kt's buffers take the next loads at once.  Loads
  // issued in step kt, two per sub-step between the MFMAs:
  //   sub-step 0: weight rows of step kt+1, second half;
  //   sub-steps 1, 2: A rows of step kt+2;
  //   sub-step 3 (after the barrier): weight rows of step kt+2, first half.
  // So a weight load has three to four sub-steps to land and an A-row load
  // five to six.
  // MS: there is a step kt+1 (its loads, the barrier, its first reads);
  // MD: there is a step kt+2 (its loads).
  // XL: this wave's 32 A rows hold valid rows, so it loads them; MM: its 128
  // output rows hold valid rows, so it computes.  Rows past the tile's valid
  // ones cost neither loads nor, in 128-row halves, matrix-core time.
  static_assert(DEEP_X && XLOADS == 4 && WLOADS == 4, "the K loop's load slots");
  bf16x8 F[2][6];
  auto rd = [&](int kt, int ks, bf16x8 (&f)[6]) {
    const uint8_t* xs_ = smem + (kt % NXB) * X_BYTES;
    const uint8_t* ws_ = smem + W_BASE + (kt % NWB) * W_BYTES;
    const int c = (((ks * 2 + kg) ^ cx) << 4);
    if (KX) {  // (KX implies WT) both operands in one block
      const uint32_t xb = (uint32_t)(uintptr_t)xs_ + ks * 16 * (kBM * 2);  // LDS byte addresses
      const uint32_t wb = (uint32_t)(uintptr_t)ws_ + ks * 16 * (BN * 2);
      lds_read_tr16_frags6(xb + a_off[0], xb + a_off[1], xb + a_off[2], xb + a_off[3],
                           wb + b_off[0], wb + b_off[1], f);
      return;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] = as_bf16x8(ld_u32x4(xs_ + a_off[i] + c));
    }
    if (WT) {
      const uint32_t base = (uint32_t)(uintptr_t)ws_ + ks * 16 * (BN * 2);  // LDS byte address
      lds_read_tr16_frags(base + b_off[0], base + b_off[1], f[4], f[5]);
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) f[4 + j] = as_bf16x8(ld_u32x4(ws_ + b_off[j] + c));
    }
  };
  // PART: only the first ni of this wave's four 32-row blocks hold valid rows
  // (the last M-tile of an expert), so the products of the others are skipped
  const int ni = min(4, max(0, (t.rows - wm * 128 + 31) / 32));  // wave-uniform
  auto step = [&](int kt, auto ms_c, auto md_c, auto xl_c, auto mm_c, auto part_c) {
    constexpr bool MS = decltype(ms_c)::value;
    constexpr bool MD = decltype(md_c)::value;
    constexpr bool XL = decltype(xl_c)::value;
    constexpr bool MM = decltype(mm_c)::value;
    constexpr bool PART = decltype(part_c)::value;
    // loads this wave may still have in flight at step kt+1's barrier: the A
    // rows of step kt+2
    constexpr int PENDING = MD && XL ? XLOADS : 0;
    const size_t w1 = MS ? w_step(kt + 1) : 0;
    const size_t w2 = MD ? w_step(kt + 2) : 0;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks == 3 && MS) {
        __builtin_amdgcn_s_waitcnt(PENDING | (0x7 << 4));  // vmcnt(PENDING) lgkmcnt(0)
        block_barrier();  // step kt+1's operands are in LDS; every read of step kt is done
        if (MM) rd(kt + 1, 0, F[0]);
      }
      if (MM) {
        if (ks < 3) rd(kt, ks + 1, F[(ks + 1) & 1]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (PART && i >= ni) continue;
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = mfma_32x32x16_bf16(F[ks & 1][4 + j], F[ks & 1][i], acc[i][j]);
        }
      }
      bool has[2] = {false, false};
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (ks == 0) {
          if (MS) { issue_w(kt + 1, w1, 2 + u); has[u] = true; }
        } else if (ks < 3) {
          if (MD && XL) { issue_x(kt + 2, (ks - 1) * 2 + u); has[u] = true; }
        } else if (MD) {
          issue_w(kt + 2, w2, u);
          has[u] = true;
        }
      }
      if (MM && !PART) {
        // the fragment reads of the next sub-step (the transposing ones are
        // asm blocks, outside the scheduler's DS-read class)
        constexpr int NDS = (KX ? 0 : 4) + (WT ? 0 : 2);
        if (NDS && (ks < 3 || MS)) __builtin_amdgcn_sched_group_barrier(0x100, NDS, 0);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (m % 4 == 0 && has[m / 4]) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
      }
    }
  };

  const int nk = t.nk;
  auto k_loop = [&](auto xl_c, auto mm_c, auto part_c) {
    constexpr bool XL = decltype(xl_c)::value;
    constexpr bool MM = decltype(mm_c)::value;
    using T_ = std::true_type;
    using F_ = std::false_type;
    // prologue: the weight and A rows of step 0, then the A rows of step 1 and
    // the first half of its weight rows
#pragma unroll
    for (int q = 0; q < WLOADS; ++q) issue_w(0, w_step(0), q);
#pragma unroll
    for (int q = 0; q < XLOADS; ++q)
      if (XL) issue_x(0, q);
    if (nk >= 2) {
#pragma unroll
      for (int q = 0; q < XLOADS; ++q)
        if (XL) issue_x(1, q);
      const size_t w1 = w_step(1);
      issue_w(1, w1, 0);
      issue_w(1, w1, 1);
    }
    // step 0's operands: only the loads of step 1 may still be in flight
    if (nk >= 2) {
      if (XL) __builtin_amdgcn_s_waitcnt((XLOADS + 2) | (0x7 << 4));  // vmcnt(6) lgkmcnt(0)
      else __builtin_amdgcn_s_waitcnt(2 | (0x7 << 4));                // vmcnt(2) lgkmcnt(0)
    } else {
      wait_all_loads();
    }
    block_barrier();
    if (MM) rd(0, 0, F[0]);
    int kt = 0;
    for (; kt + 2 < nk; ++kt) step(kt, T_{}, T_{}, xl_c, mm_c, part_c);
    if (kt + 1 < nk) { step(kt, T_{}, F_{}, xl_c, mm_c, part_c); ++kt; }
    step(kt, F_{}, F_{}, xl_c, mm_c, part_c);
  };
  const bool mm = wm * 128 < t.rows;  // wave-uniform
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (KX) {  // every wave loads K-rows of A; only waves with valid A rows compute
    if (!mm) k_loop(T_{}, F_{}, F_{});
    else if (ni == 4) k_loop(T_{}, T_{}, F_{});
    else k_loop(T_{}, T_{}, T_{});
  } else if (wave * (8 * XLOADS) < t.rows) {
    if (ni == 4) k_loop(T_{}, T_{}, F_{});
    else k_loop(T_{}, T_{}, T_{});
  } else if (mm) {  // its A rows are past the tile's rows, so ni < 4
    k_loop(F_{}, T_{}, T_{});
  } else {
    k_loop(F_{}, F_{}, F_{});
  }

  // ---- epilogue.  Lane l holds, for A-block i and weight block j, row
  // wm*128 + i*32 + l%32 and the four columns 8q + 4(l/32) + 0..3 of the block
  // in acc[i][j][4q..4q+3].  The outputs of the forward products go through
  // LDS (free once every wave's fragment reads are done), so that each store
  // instruction writes whole rows; staged rows keep their 16-byte pieces at
  // position (piece ^ row), which spreads both the column writes and the row
  // reads over the banks.  Waves without valid rows write nothing but take
  // part in every barrier.
  if (GATE_UP && RAW) {
    // G and U themselves, fp32: each lane stores its four columns of each
    if (!mm || wn * 32 >= t.out_cols) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 128 + i * 32 + r32;
      if (row >= t.rows) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = wn * 32 + 8 * q + 4 * kg;
        const int64_t o = t.raw_off + (int64_t)row * t.out_ld + col;
        *reinterpret_cast<f32x4*>(g_raw + o) =
            f32x4{acc[i][0][4 * q], acc[i][0][4 * q + 1], acc[i][0][4 * q + 2], acc[i][0][4 * q + 3]};
        *reinterpret_cast<f32x4*>(u_raw + o) =
            f32x4{acc[i][1][4 * q], acc[i][1][4 * q + 1], acc[i][1][4 * q + 2], acc[i][1][4 * q + 3]};
        if (a_raw) {  // and the SwiGLU product as the forward epilogue forms it
          float h[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = silu_times_rcp(acc[i][0][4 * q + r], acc[i][1][4 * q + r]);
          *reinterpret_cast<uint2*>(a_raw + o) =
              make_uint2(pack_bf16x2_rne(h[0], h[1]), pack_bf16x2_rne(h[2], h[3]));
        }
      }
    }
  } else if (GATE_UP) {
    // bf16 A [256 rows][128 columns] goes through LDS as 16 pieces of 16 bytes
    // per row, piece p of row r at position p ^ (r & 15), so that each store
    // instruction writes 4 whole rows (8 full cache lines) instead of 16-byte
    // parts of 32 rows
    block_barrier();  // every wave's fragment reads are done: the LDS is free
    if (mm) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + r32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float h[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = silu_times_rcp(acc[i][0][4 * q + r], acc[i][1][4 * q + r]);
          uint2 v;
          v.x = pack_bf16x2_rne(h[0], h[1]);
          v.y = pack_bf16x2_rne(h[2], h[3]);
          const int piece = wn * 4 + q;  // columns 8 * piece .. + 7; this lane's half: kg
          *reinterpret_cast<uint2*>(smem + row * 256 + ((piece ^ (row & 15)) << 4) + kg * 8) = v;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    block_barrier();
    uint16_t* out = reinterpret_cast<uint16_t*>(t.Out);
    const int piece = lane & 15;
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // rows wave*32 .. +31, four per instruction
      const int row = wave * 32 + u * 4 + (lane >> 4);
      if (row < t.rows && piece * 8 < t.out_cols) {
        const u32x4 v = ld_u32x4(smem + row * 256 + ((piece ^ (row & 15)) << 4));
        *reinterpret_cast<u32x4*>(out + (size_t)row * t.out_ld + piece * 8) = v;
      }
    }
  } else {
    // fp32 [128 rows][256 columns] per half: 64 pieces of 4 columns per row
    block_barrier();  // every wave's fragment reads are done: the LDS is free
    float* sm = reinterpret_cast<float*>(smem);
    float* out = reinterpret_cast<float*>(t.Out);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (wm == h && mm) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = i * 32 + r32;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int piece = wn * 16 + j * 8 + 2 * q + kg;
              f32x4 v = {acc[i][j][4 * q + 0], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                         acc[i][j][4 * q + 3]};
              *reinterpret_cast<f32x4*>(sm + row * 256 + ((piece ^ (row & 63)) << 2)) = v;
            }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      block_barrier();
#pragma unroll
      for (int u = 0; u < 16; ++u) {  // one row per instruction, 16 rows per wave
        const int row = wave * 16 + u, grow = h * 128 + row;
        if (grow < t.rows && lane * 4 < t.out_cols)
        {
          f32x4* o = reinterpret_cast<f32x4*>(out + (size_t)grow * t.out_ld + lane * 4);
          const f32x4 v = *reinterpret_cast<const f32x4*>(sm + row * 256 + ((lane ^ (row & 63)) << 2));
          if (NT) __builtin_nontemporal_store(v, o);
          else *o = v;
        }
      }
      if (h == 0) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // staged reads done before the second half
        block_barrier();
      }
    }
  }
}

// Launch slot -> work index.  Blocks are dealt to the 8 XCDs round-robin, so
// slot b runs on XCD b % 8; within each group of 8 * run slots XCD x receives
// the run of consecutive works run * x .. run * x + run - 1, neighbours in the
// raster that share A rows and weight slices in its L2.  Longer runs (32
// works, one per CU of an XCD) halve the L2 misses again but leave the XCDs
// unevenly loaded where tile costs differ (shared-expert tiles, ragged last
// M-tiles), which measured slower.
__device__ __forceinline__ int slot_work(int b, int run) {
  const int group = 8 * run;
  const int base = b / group * group, w = b - base;
  return base + (w & 7) * run + (w >> 3);
}

// One block per work slot; slots past the device-side tile count return.  A
// launch of the shared experts' tiles alone reads nothing the dispatch writes
// (it may run before the dispatch); a launch of the routed tiles alone has no
// shared ones.
template <bool GATE_UP, bool BUF, bool NT = false>
__global__ __launch_bounds__(NTHREADS) void grouped_gemm_bf16_kernel(FfnArgs p, GemmGrid g) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];
  const int n_routed = p.part == kSharedTiles ? 0 : p.tile_off[p.E] * g.nt_r;
  const int ns_t = p.part == kRoutedTiles ? 0 : g.n_shared;
  const int end = n_routed + ns_t;
  const int L0 = slot_work(blockIdx.x, g.run);
  if (L0 >= end) return;
  // The down product takes the shared experts' tiles first: their K runs over
  // all shared experts (n_s * I_s, twice a routed tile's I for two shared
  // experts), so as the last tiles of the launch they would form its tail.
  const int first = GATE_UP ? 0 : ns_t;
  const int L = L0 < first ? n_routed + L0 : L0 - first;
  BTile t;
  if (GATE_UP) gate_up_tile(p, g, L, n_routed, t);
  else down_tile(p, g, L, n_routed, t);
  run_tile<GATE_UP, BUF, false, false, NT>(t, smem);
}

// Gate/up tiles with G and U stored as fp32 (RAW epilogue): the routed
// tiles into [R,I], or (part: shared) the shared experts' into [T, n_s*I_s].
template <bool BUF>
__global__ __launch_bounds__(NTHREADS) void gate_up_raw_bf16_kernel(FfnArgs p, GemmGrid g) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];
  const int n_routed = p.part == kSharedTiles ? 0 : p.tile_off[p.E] * g.nt_r;
  const int ns_t = p.part == kRoutedTiles ? 0 : g.n_shared;
  const int L = slot_work(blockIdx.x, g.run);
  if (L >= n_routed + ns_t) return;
  BTile t;
  gate_up_tile<true>(p, g, L, n_routed, t);
  run_tile<true, BUF, true>(t, smem, static_cast<float*>(p.a), p.u_raw, p.a_bf16);
}

// The routed down tiles alone (PARTS: A rows of several K blocks; WT:
// weights in their stored layout).
template <bool BUF, bool WT, bool NT = false>
__global__ __launch_bounds__(NTHREADS) void down_routed_bf16_kernel(FfnArgs p, GemmGrid g) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];
  const int n_routed = p.tile_off[p.E] * g.nt_r;
  const int L = slot_work(blockIdx.x, g.run);
  if (L >= n_routed) return;
  BTile t;
  down_tile<true, WT>(p, g, L, n_routed, t);
  run_tile<false, BUF, false, true, NT, WT>(t, smem);
}

// Weight-gradient tiles: expert e, 256-row m-tile, 256-column n-tile; K runs
// over the expert's zero-padded part of the shared reduction index.
template <bool BUF>
__global__ __launch_bounds__(NTHREADS) void seg_gemm_bf16_kernel(SegGemmArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];
  const int mt = (p.M + kBM - 1) / kBM, ntl = (p.N + BN - 1) / BN;
  const int per_e = mt * ntl;
  const int L = slot_work(blockIdx.x, SEG_RUN);
  if (L >= p.E * per_e) return;
  const int e = L / per_e, rem = L - e * per_e;
  const int m0 = (rem / ntl) * kBM, n0 = (rem % ntl) * BN;
  const int k0 = p.poff[e], nk = (p.poff[e + 1] - k0) / BK;
  BTile t;
  t.rows = min(kBM, p.M - m0);
  t.wrows = min(BN, p.N - n0);
  float* out = p.out + (size_t)e * p.M * p.N + (size_t)m0 * p.N + n0;
  if (nk == 0) {  // no rows: the gradient is zero
    for (int i = threadIdx.x; i < t.rows * (t.wrows / 4); i += NTHREADS) {
      const int r = i / (t.wrows / 4), c = (i % (t.wrows / 4)) * 4;
      *reinterpret_cast<f32x4*>(out + (size_t)r * p.N + c) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }
  t.X = reinterpret_cast<const uint8_t*>(p.A + (size_t)m0 * p.ld + k0);
  t.x_ld = (size_t)p.ld * 2;
  t.rmap = nullptr;
  t.rdiv = 1;
  t.W[0] = t.W[1] = reinterpret_cast<const uint8_t*>(p.B + (size_t)n0 * p.ld + k0);
  t.w_ld = (size_t)p.ld * 2;
  t.nk = nk;
  t.kps = 0;
  t.w_seg = 0;
  t.Out = reinterpret_cast<uint8_t*>(out);
  t.out_ld = p.N;
  t.out_cols = t.wrows;
  t.raw_off = 0;
  run_tile<false, BUF>(t, smem);
}

// Weight-gradient tiles with both operands in their row layout: out[e] =
// sum over expert e's sorted rows r of the outer products X[r] (x) W[r], the
// reduction running over the rows twice, X's first K block (columns 0..M-1,
// the hi parts of an fp32 operand) and then its second (x_part columns on, the
// lo parts), against the same W rows.  Both tiles arrive as 64 rows of 256
// columns and their fragments come out of LDS through transposing reads;
// rows past the expert's last read zeros through the descriptors' ranges.
template <bool NT>  // non-temporal output stores
__global__ __launch_bounds__(NTHREADS) void seg_gemm_km_bf16_kernel(SegKmArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];
  const int mt = (p.M + kBM - 1) / kBM, ntl = (p.N + BN - 1) / BN;
  const int per_e = mt * ntl;
  // With the schedule (p.rec): block b runs on XCD b % 8 (blocks are dealt
  // to the XCDs round-robin) and takes tile j % per_e of the (j / per_e)-th
  // expert in that XCD's list, j = b / 8: all tiles of an expert on one XCD,
  // so the tiles running there together share each K-step's operand rows in
  // its L2 instead of every XCD fetching them.  Without it: expert L / per_e,
  // runs of SEG_RUN works per XCD; with slices, all "experts" share segment
  // 0 and take slices of its K-steps.
  int e, s0, ne, rem;
  if (p.rec) {
    const int j = blockIdx.x >> 3, i = j / per_e;
    if (i >= p.cap) return;
    const int4 rc = *reinterpret_cast<const int4*>(p.rec + 4 * ((blockIdx.x & 7) * p.cap + i));
    if (!rc.w) return;  // no expert in this place of the list
    e = rc.x;
    s0 = rc.y;
    ne = rc.z;
    rem = j - i * per_e;
  } else {
    const int L = slot_work(blockIdx.x, SEG_RUN);
    if (L >= p.E * per_e) return;
    e = L / per_e;
    rem = L - e * per_e;
    const int sg = p.slices > 1 ? 0 : e;
    s0 = p.offsets[sg];
    ne = p.offsets[sg + 1] - s0;
  }
  const int m0 = (rem / ntl) * kBM, n0 = (rem % ntl) * BN;
  const int kpe = (ne + BK - 1) / BK;  // K-steps per K block
  const int nks = 2 * kpe;
  const int g0 = p.slices > 1 ? (int)((int64_t)e * nks / p.slices) : 0;
  const int g1 = p.slices > 1 ? (int)((int64_t)(e + 1) * nks / p.slices) : nks;
  BTile t;
  t.rows = min(kBM, p.M - m0);
  t.wrows = min(BN, p.N - n0);
  float* out = p.out + (size_t)e * p.M * p.N + (size_t)m0 * p.N + n0;
  if (g1 <= g0) {  // no rows (or an empty slice): the product is zero
    for (int i = threadIdx.x; i < t.rows * (t.wrows / 4); i += NTHREADS) {
      const int r = i / (t.wrows / 4), c = (i % (t.wrows / 4)) * 4;
      *reinterpret_cast<f32x4*>(out + (size_t)r * p.N + c) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }
  t.X = reinterpret_cast<const uint8_t*>(p.X + (size_t)s0 * p.x_ld + m0);
  t.x_ld = (size_t)p.x_ld * 2;
  t.x_seg = (size_t)p.x_part * 2;
  t.x_bytes = (uint32_t)((size_t)ne * p.x_ld * 2);
  t.rmap = nullptr;
  t.rdiv = 1;
  t.W[0] = t.W[1] = reinterpret_cast<const uint8_t*>(p.W + (size_t)s0 * p.w_ld + n0);
  t.w_ld = (size_t)p.w_ld * 2;
  t.w_bytes = (uint32_t)((size_t)ne * p.w_ld * 2);
  t.nk = g1 - g0;
  t.kt0 = g0;
  t.kps = kpe;
  t.wsh = 0;
  t.w_seg = 0;
  t.Out = reinterpret_cast<uint8_t*>(out);
  t.out_ld = p.N;
  t.out_cols = t.wrows;
  t.raw_off = 0;
  run_tile<false, true, false, false, NT, true, true>(t, smem);
}

GemmGrid bf16_gate_up_grid(const FfnArgs& a) {
  GemmGrid g;
  g.mtb = (int)routed_mtile_bound(a.R, a.E);
  g.nt_r = (a.I + GU_COLS - 1) / GU_COLS;
  g.nt_s = a.ns ? (a.Is + GU_COLS - 1) / GU_COLS : 0;
  g.mt_s = (int)((a.T + kBM - 1) / kBM);
  g.n_shared = a.ns * g.nt_s * g.mt_s;
  g.routed = (int64_t)g.mtb * g.nt_r;
  g.total = g.routed + g.n_shared;
  g.run = GU_RUN;
  g.gm = GU_GROUP_M;
  return g;
}

int64_t pad_slots(int64_t n, int run) { return (n + 8 * run - 1) / (8 * run) * (8 * run); }

GemmGrid bf16_down_grid(const FfnArgs& a) {
  GemmGrid g;
  g.mtb = (int)routed_mtile_bound(a.R, a.E);
  g.nt_r = (a.d + BN - 1) / BN;
  g.nt_s = g.nt_r;
  g.mt_s = (int)((a.T + kBM - 1) / kBM);
  g.n_shared = a.ns ? g.nt_r * g.mt_s : 0;
  g.routed = (int64_t)g.mtb * g.nt_r;
  g.total = g.routed + g.n_shared;
  g.run = DN_RUN;
  g.gm = DN_GROUP_M;
  return g;
}

}  // namespace

int64_t gate_up_grid_bf16(const FfnArgs& a) { return pad_slots(bf16_gate_up_grid(a).total, GU_RUN); }
int64_t down_grid_bf16(const FfnArgs& a) { return pad_slots(bf16_down_grid(a).total, DN_RUN); }

// Slots of one launch: all tiles, the routed tiles (an upper bound) or the
// shared experts' tiles.
int64_t launch_slots(const FfnArgs& a, const GemmGrid& g) {
  const int64_t n = a.part == kRoutedTiles ? g.routed
                  : a.part == kSharedTiles ? (int64_t)g.n_shared : g.total;
  return n ? pad_slots(n, g.run) : 0;
}

// Whether every byte offset a tile adds to its operand bases fits in 32 bits:
// the gathered token rows span all of x (T*d*2 bytes); other A and weight
// tiles span at most 256 rows of d, I or n_s*I_s elements plus one row; the
// shared experts' down tiles walk across all their down weights.
// force_global asks for the global-load variant regardless.
bool buffer_offsets_fit(const FfnArgs& a) {
  if (a.force_global) return false;
  const uint64_t lim = 1ull << 32;
  const uint64_t w = (uint64_t)std::max(std::max(a.d, a.I), a.ns * a.Is);
  const uint64_t tile = 514 * w;  // a tile's rows plus the K offset, with margin
  // A rows of a_parts blocks (their K offsets; all T token rows when gathered
  // through perm), and the weight blocks they step through
  const uint64_t parts = a.a_parts > 1 ? (uint64_t)a.a_parts : 1;
  const uint64_t xrows = (a.perm ? (uint64_t)a.T + 2 : 258) * parts * (uint64_t)a.I * 2;
  const uint64_t wpart = parts > 1 ? (uint64_t)a.w_part * 2 * (parts / 2) : 0;
  // k-major weights: an expert's block of I K-rows of d elements
  const bool wt_fits = !a.wt || (uint64_t)a.I * a.d * 2 + 1024 < lim;
  return (uint64_t)a.T * a.d * 2 + tile < lim && (uint64_t)a.ns * a.d * a.Is * 2 + tile < lim &&
         xrows < lim && wpart + tile < lim && wt_fits;
}

void launch_gate_up_bf16(const FfnArgs& a, hipStream_t stream) {
  const int64_t slots = launch_slots(a, bf16_gate_up_grid(a));
  if (slots == 0) return;
  auto kern = buffer_offsets_fit(a) ? grouped_gemm_bf16_kernel<true, true>
                                    : grouped_gemm_bf16_kernel<true, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)slots), dim3(NTHREADS), 0, stream, a,
                     bf16_gate_up_grid(a));
}

void launch_gate_up_raw_bf16(const FfnArgs& a, hipStream_t stream) {
  const GemmGrid g = bf16_gate_up_grid(a);
  const int64_t slots = launch_slots(a, g);
  if (slots == 0) return;
  auto kern = buffer_offsets_fit(a) ? gate_up_raw_bf16_kernel<true> : gate_up_raw_bf16_kernel<false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)slots), dim3(NTHREADS), 0, stream, a, g);
}

void launch_down_routed_bf16(const FfnArgs& a, hipStream_t stream) {
  const GemmGrid g = bf16_down_grid(a);
  const int64_t slots = g.routed ? pad_slots(g.routed, g.run) : 0;
  if (slots == 0) return;
  const bool buf = buffer_offsets_fit(a);
  // outputs larger than the 256 MB MALL take non-temporal stores
  const bool nt = a.wt && buf && (uint64_t)a.R * a.d * 4 > (256ull << 20);
  auto kern = a.wt ? (buf ? (nt ? down_routed_bf16_kernel<true, true, true>
                                : down_routed_bf16_kernel<true, true>)
                          : down_routed_bf16_kernel<false, true>)
                   : (buf ? down_routed_bf16_kernel<true, false> : down_routed_bf16_kernel<false, false>);
  hipLaunchKernelGGL(kern, dim3((unsigned)slots), dim3(NTHREADS), 0, stream, a, g);
}

void launch_seg_gemm_bf16(const SegGemmArgs& a, hipStream_t stream) {
  const int64_t tiles = (int64_t)a.E * ((a.M + kBM - 1) / kBM) * ((a.N + BN - 1) / BN);
  if (tiles == 0) return;
  // buffer loads when a tile's offsets (256 rows of ld elements) fit in 32 bits
  const bool buf = (uint64_t)(kBM + 2) * (uint64_t)a.ld * 2 < (1ull << 32);
  auto kern = buf ? seg_gemm_bf16_kernel<true> : seg_gemm_bf16_kernel<false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)pad_slots(tiles, SEG_RUN)), dim3(NTHREADS), 0, stream, a);
}

bool seg_gemm_km_fits(const SegKmArgs& a, int64_t max_rows) {
  // descriptor ranges and offsets of one expert's rows (at most max_rows)
  const uint64_t lim = 1ull << 32;
  return (uint64_t)max_rows * a.x_ld * 2 + 1024 < lim && (uint64_t)max_rows * a.w_ld * 2 + 1024 < lim;
}

void launch_seg_gemm_km_bf16(const SegKmArgs& a, hipStream_t stream) {
  const int64_t tiles = (int64_t)a.E * ((a.M + kBM - 1) / kBM) * ((a.N + BN - 1) / BN);
  if (tiles == 0) return;
  // outputs larger than the 256 MB MALL take non-temporal stores
  const bool nt = (uint64_t)a.E * a.M * a.N * 4 > (256ull << 20);
  const int64_t per_e = tiles / a.E;
  const int64_t grid = a.rec ? (int64_t)kSegXcds * a.cap * per_e : pad_slots(tiles, SEG_RUN);
  hipLaunchKernelGGL(nt ? seg_gemm_km_bf16_kernel<true> : seg_gemm_km_bf16_kernel<false>,
                     dim3((unsigned)grid), dim3(NTHREADS), 0, stream, a);
}

void launch_down_bf16(const FfnArgs& a, hipStream_t stream) {
  const int64_t slots = launch_slots(a, bf16_down_grid(a));
  if (slots == 0) return;
  // outputs (y and the shared experts' sum) larger than the 256 MB MALL take
  // non-temporal stores
  const bool nt = ((uint64_t)a.R + (a.ns ? (uint64_t)a.T : 0)) * a.d * 4 > (256ull << 20);
  const bool buf = buffer_offsets_fit(a);
  auto kern = buf ? (nt ? grouped_gemm_bf16_kernel<false, true, true> : grouped_gemm_bf16_kernel<false, true>)
                  : (nt ? grouped_gemm_bf16_kernel<false, false, true> : grouped_gemm_bf16_kernel<false, false>);
  hipLaunchKernelGGL(kern, dim3((unsigned)slots), dim3(NTHREADS), 0, stream, a,
                     bf16_down_grid(a));
}

}  // namespace moe
