// Host-side launchers of the MoE-layer kernels (internal to the library).
// Each enqueues on `stream` and returns without synchronising; sizes have
// been validated by the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

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
  int32_t* tile_off;    // [E+1] or null: M-tile prefix (units of kBM rows)
  int32_t* perm;        // [R]
  int32_t* inv_perm;    // [R]
  void* x_sorted;       // [R,d] or null (skip the row gather)
  int32_t* blk;         // [nblk,E] scratch
  int64_t T;
  int d, E, k;
  int elem_bytes;
};
void launch_dispatch(const DispatchArgs& a, hipStream_t stream);

// M-tile prefix table from expert offsets (for a grouped FFN call on its own).
void launch_tile_table(const int32_t* offsets, int E, int32_t* tile_off, hipStream_t stream);

// Grouped SwiGLU FFN: gate/up GEMM with the SiLU product fused, then down GEMM.
struct FfnArgs {
  const void* xs;         // [R,d] rows grouped by expert
  const void* x;          // [T,d] (shared experts) or null
  const void *wg, *wu, *wd;        // routed weights
  const void *wsg, *wsu, *wsd;     // shared weights or null
  const int32_t* offsets; // [E+1]
  const int32_t* tile_off;// [E+1]
  void* a;                // [R,I]
  void* ash;              // [T, ns*Is]
  float* y;               // [R,d]
  float* ysh;             // [T,d] or null
  int64_t T, R;
  int d, E, I, ns, Is;
  bool bf16;
};
void launch_gate_up(const FfnArgs& a, hipStream_t stream);
void launch_down(const FfnArgs& a, hipStream_t stream);
// Upper bounds of the grid sizes (for validation of the 2^31 grid limit).
int64_t gate_up_grid(const FfnArgs& a);
int64_t down_grid(const FfnArgs& a);

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
