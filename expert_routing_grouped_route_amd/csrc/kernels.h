// Host-side launchers of the MoE-layer kernels (internal to the library).
// Each enqueues on `stream` and returns without synchronising; sizes have
// been validated by the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace moe {

struct RouteArgs {
  const void* x;          // [T,d] bf16 or fp32
  const void* wr;         // [E,d]
  const float* bias;      // [E] or null
  const float* logits_in; // [T,E] or null
  float* logits_out;      // [T,E] or null
  int32_t* ids;           // [T,k]
  float* wts;             // [T,k]
  int64_t T;
  int d, E, k;
  bool bf16;
};
void launch_route(const RouteArgs& a, hipStream_t stream);

// Dispatch.  `blk` is an [nblk, E] int32 scratch matrix; nblk from
// dispatch_blocks().
int dispatch_chunk(int64_t R);
int dispatch_blocks(int64_t R);
struct DispatchArgs {
  const void* x;        // [T,d]
  const int32_t* ids;   // [T,k]
  int32_t* counts;      // [E] or null
  int32_t* offsets;     // [E+1]
  int32_t* tiles;       // or null: tile table, [E+1] M-tile prefix (units of kBM
                        // rows) then the expert of each M-tile (tile_table_ints)
  int32_t* ctr;         // or null: kGemmCounters work counters of the GEMMs, zeroed
  int32_t* perm;        // [R]
  int32_t* inv_perm;    // [R]
  void* x_sorted;       // [R,d] or null (skip the row gather)
  int32_t* blk;         // [nblk,E] scratch
  int64_t T;
  int d, E, k;
  int elem_bytes;
  const int32_t* rep;   // or null: token condensation, [T] representative of each token;
                        // an assignment (t, j) with rep[t] != t whose expert is among
                        // rep[t]'s gets no row (its inv_perm entry is left for
                        // launch_condense_inv)
};
void launch_dispatch(const DispatchArgs& a, hipStream_t stream);

// Tile table from expert offsets (for a grouped FFN call on its own); also
// zeroes the GEMM work counters.
// The backward's small tables, one launch: the M-tile prefix of G <= 256 row
// segments (tiles of `tile` rows), and with off1 non-null the row offsets and
// tile tables of one segment of T rows (off1, poff1, tiles1) and of two
// segments of T rows (off2, tiles2).
void launch_segment_tables(const int32_t* offsets, int G, int tile, int32_t* prefix, int64_t T,
                           int32_t* off1, int32_t* poff1, int32_t* tiles1, int32_t* off2,
                           int32_t* tiles2, int32_t* ctr, hipStream_t stream);
void launch_tile_table(const int32_t* offsets, int E, int32_t* tiles, int32_t* ctr,
                       hipStream_t stream);
constexpr int kGemmCounters = 16;  // 8 per grouped GEMM launch (one per XCD)
// Compute units of the current device (cached per device).
int device_cu_count();
// Upper bound of the M-tiles of R rows over E experts, and the table's size.
inline int64_t routed_mtile_bound(int64_t R, int E) {
  // sum_e ceil(n_e / kBM) <= floor((R + E * (kBM - 1)) / kBM)
  return R > 0 ? (R + (int64_t)E * (kBM - 1)) / kBM : 0;
}
inline int64_t tile_table_ints(int64_t R, int E) { return E + 1 + routed_mtile_bound(R, E); }

// Grouped SwiGLU FFN: gate/up GEMM with the SiLU product fused, then down GEMM.
struct FfnArgs {
  const void* xs;         // [R,d] rows grouped by expert, or null: then row i of the
                          // routed operand is x[perm[i] / k] (gathered by the GEMM)
  const int32_t* perm;    // [R] (with xs == null)
  int k;                  // top-k (with xs == null)
  const void* x;          // [T,d] (shared experts) or null
  const void *wg, *wu, *wd;        // routed weights
  const void *wsg, *wsu, *wsd;     // shared weights or null
  const int32_t* offsets; // [E+1]
  const int32_t* tile_off;// tile table: [E+1] M-tile prefix, then expert per M-tile
  int32_t* ctr;           // kGemmCounters zeroed work counters
  void* a;                // [R,I]
  void* ash;              // [T, ns*Is]
  float* y;               // [R,d]
  float* ysh;             // [T,d] or null
  int64_t T, R;
  int d, E, I, ns, Is;
  bool bf16;
  int part;               // tiles launched: 0 all, 1 routed experts only, 2 shared experts only
  float* u_raw;           // launch_gate_up_raw_bf16: [R,I] fp32 U (G goes to `a`, fp32)
  // launch_down_routed_bf16 only: with a_parts > 1 each row of `a` holds
  // a_parts blocks of I columns, and block b is multiplied by weight block
  // b / 2, which starts w_part elements after block 0 per block index (the
  // bf16 hi and lo parts of an fp32 operand against one weight, and so on).
  // With perm set as well, `a` holds token rows and routed row r reads token
  // row perm[r] / k.
  int a_parts;
  int64_t w_part;
  // launch_down_routed_bf16 only: with wt set, the weights are read in their
  // stored layout, reduction index outer: expert e's element (k, n) at
  // wd[(e * I + k) * d + n] (I = K and d = N here) rather than [E, d, I], and
  // weight block 1 of the a_parts blocks (block b / 2 == 1) comes from wd2
  // (same layout; w_part is then unused).
  bool wt;
  const void* wd2;
  // launch_gate_up_raw_bf16 only: also the bf16 SwiGLU product, in the layout
  // of G and U (or null)
  uint16_t* a_bf16;
  // take the operands through 64-bit global loads even where the buffer-load
  // offsets fit in 32 bits (the variant the launchers otherwise use only for
  // very large operands; same data in LDS, same results)
  bool force_global;
};
constexpr int kAllTiles = 0, kRoutedTiles = 1, kSharedTiles = 2;
void launch_gate_up_bf16(const FfnArgs& a, hipStream_t stream);
// The gate/up products G = X W_g^T and U = X W_u^T as fp32 (G in `a`, U in
// `u_raw`) instead of the SwiGLU product: the same tiles and K loop.  part
// kRoutedTiles: the routed experts' [R,I]; kSharedTiles: the shared experts'
// [T, n_s*I_s].
void launch_gate_up_raw_bf16(const FfnArgs& a, hipStream_t stream);
// The routed experts' down product Y[rows] = A[rows] W_d[e]^T alone (no
// shared tiles), stored to `y` (a_parts and w_part apply).
void launch_down_routed_bf16(const FfnArgs& a, hipStream_t stream);

// Per-expert products reduced over each expert's rows (weight gradients):
// out[e] [M,N] = sum over k of A(m, k) B(n, k), where A [M, ld] and B [N, ld]
// are bf16 with the reduction index contiguous, and expert e's part spans
// columns poff[e] .. poff[e+1] (multiples of 64, zero-padded).  Experts with
// an empty part get zeros.  On the gate/up and down kernels' tile loop.
struct SegGemmArgs {
  const uint16_t* A;      // [M, ld]
  const uint16_t* B;      // [N, ld]
  int64_t ld;             // elements between rows of A and of B
  const int32_t* poff;    // [E+1]
  float* out;             // [E, M, N] fp32
  int E, M, N;
};
void launch_seg_gemm_bf16(const SegGemmArgs& a, hipStream_t stream);
// Weight gradients from operands in their row layout: out[e][m][n] =
// sum over expert e's rows r in [offsets[e], offsets[e+1]) and h in {0, 1} of
// X[r][h * x_part + m] * W[r][n] (X: the bf16 hi and lo parts of an fp32
// operand side by side; W: a bf16 operand).  Needs the buffer loads:
// seg_gemm_km_fits() with the largest expert's row count.
struct SegKmArgs {
  const uint16_t* X;      // [rows, x_ld]
  int64_t x_ld, x_part;   // elements between rows; between the hi and lo parts
  const uint16_t* W;      // [rows, w_ld]
  int64_t w_ld;
  const int32_t* offsets; // [E+1] rows of each expert
  float* out;             // [E, M, N] fp32
  int E, M, N;
  // slices > 1: one segment (offsets[0..1]) whose 2 * ceil(rows / 64) K-steps
  // are cut into E = slices contiguous ranges, range e summed into out[e]
  int slices;
  // or null: the schedule of launch_seg_sched, [8][cap][4] records
  // {expert, first row, rows, 1} (or zeros) listing the experts each XCD
  // takes, all of an expert's tiles on one XCD
  const int32_t* rec;
  int cap;                // places per XCD in rec: seg_sched_cap(E)
};
bool seg_gemm_km_fits(const SegKmArgs& a, int64_t max_rows);
// The schedule of SegKmArgs::rec from offsets [E+1] (E <= 256): experts to
// the 8 XCDs by falling cost, each to the least loaded XCD with room.
constexpr int kSegXcds = 8;
constexpr int kSegCapMax = 256 / kSegXcds + 2;
constexpr int seg_sched_cap(int E) { return (E + kSegXcds - 1) / kSegXcds + 2; }
void launch_seg_sched(const int32_t* offsets, int E, int32_t* rec, hipStream_t stream);
void launch_seg_gemm_km_bf16(const SegKmArgs& a, hipStream_t stream);
void launch_down_bf16(const FfnArgs& a, hipStream_t stream);
void launch_gate_up_f32(const FfnArgs& a, hipStream_t stream);
void launch_down_f32(const FfnArgs& a, hipStream_t stream);
// Grid sizes in blocks (for validation against the 2^31 grid limit).
int64_t gate_up_grid_bf16(const FfnArgs& a);
int64_t down_grid_bf16(const FfnArgs& a);
int64_t gate_up_grid_f32(const FfnArgs& a);
int64_t down_grid_f32(const FfnArgs& a);

inline void launch_gate_up(const FfnArgs& a, hipStream_t stream) {
  if (a.bf16) launch_gate_up_bf16(a, stream);
  else launch_gate_up_f32(a, stream);
}
inline void launch_down(const FfnArgs& a, hipStream_t stream) {
  if (a.bf16) launch_down_bf16(a, stream);
  else launch_down_f32(a, stream);
}
inline int64_t gate_up_grid(const FfnArgs& a) {
  return a.bf16 ? gate_up_grid_bf16(a) : gate_up_grid_f32(a);
}
inline int64_t down_grid(const FfnArgs& a) { return a.bf16 ? down_grid_bf16(a) : down_grid_f32(a); }

// Token condensation (see condense.hip): keys from 16 hyperplanes, a stable
// radix sort of the keys, and the representative of every token.
constexpr int kCondenseBits = 16;        // hyperplanes, key bits
constexpr int kCondenseCandidates = 32;  // bucket members a token is compared with
struct CondenseArgs {
  const void* x;            // [T,d]
  const void* hyperplanes;  // [16,d], the dtype of x
  int64_t T;
  int d;
  bool bf16;
  float cos_threshold;
  // scratch
  float* proj;                         // [T,16]
  int32_t* pids;                       // [T]
  float* pwts;                         // [T]
  int32_t *key, *key_lo, *key_hi;      // [T] each
  int32_t *off1, *off2;                // [257] each
  int32_t *perm1, *inv1, *perm2, *inv2;// [T] each
  int32_t* blk;                        // [dispatch_blocks(T), 256]
  int32_t *tok, *skey, *cand;          // [T] each
  int32_t* rep;                        // [T] output
};
void launch_condense(const CondenseArgs& a, hipStream_t stream);
// inv_perm of every condensed assignment := the row of its source.
void launch_condense_inv(const int32_t* ids, const int32_t* rep, int64_t R, int k, int32_t* inv,
                         hipStream_t stream);

struct CombineArgs {
  const float* y;        // [R,d]
  const int32_t* inv;    // [R]
  const float* w;        // [T,k]
  const float* ysh;      // [T,d] or null
  float* out;            // [T,d]
  int64_t T;
  int d, k;
};
void launch_combine(const CombineArgs& a, hipStream_t stream);

}  // namespace moe
