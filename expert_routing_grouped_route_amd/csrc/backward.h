// Host-side launcher of the layer's backward pass (internal to the library).
#pragma once

#include <algorithm>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Backward pass of the layer (backward.hip), after the route and the
// dispatch (with its row gather) have run on the same inputs.
struct BwdArgs {
  const void *x, *wr, *wg, *wu, *wd;       // forward inputs (dtype of the layer)
  const void *wsg, *wsu, *wsd;             // shared experts' weights or null
  const float* dout;                       // [T,d]
  const int32_t* ids;                      // [T,k] routing
  const float* w;                          // [T,k] kept weights
  const int32_t *offsets, *perm, *inv;     // dispatch
  const void* xs;                          // [R,d] sorted token rows
  float *dx, *dw_router, *dbias;           // [T,d], [E,d], [E] or null
  float *dw_gate, *dw_up, *dw_down;        // [E,I,d], [E,I,d], [E,d,I]
  float *dwsh_gate, *dwsh_up, *dwsh_down;  // [ns,Is,d], [ns,Is,d], [ns,d,Is]
  // scratch
  int32_t* tile_off;                       // bf16: the dispatch's M-tile table
  int32_t* ctr;                            // bf16: the GEMM counters (zeroed by the dispatch)
  uint16_t* Abf;                           // bf16: [R,I] the SwiGLU product in bf16
  uint16_t* dGU;                           // bf16: [R, 4I] rows [dG hi | dG lo | dU hi | dU lo]
  int32_t* poff;                           // bf16: [E+1] padded per-expert parts (seg_offsets_kernel)
  int32_t* srec;                           // bf16: [8][cap][4] experts per XCD (launch_seg_sched)
  int64_t seg_ld;                          // bf16: row length of tA and tB (>= poff[E])
  uint16_t *tA, *tB;                       // bf16: [max(d, I, ns*Is), seg_ld] transposed operands
  int32_t *off1, *poff1;                   // bf16: [2] each, the T rows as one segment
  int32_t* tiles1;                         // bf16: M-tile table of that one segment
  int32_t *off2, *tiles2;                  // bf16, shared: {0, T, 2T} and its M-tile table
  uint16_t *wsdT, *wsgT, *wsuT;            // bf16: [ns*Is, d], [d, ns*Is], [d, ns*Is]
                                           // (wsuT = wsgT + d*ns*Is, read as one [2, d, ns*Is])
  uint16_t* dOp;                           // bf16: [T, 2d] rows of dout as [hi | lo] parts
  uint16_t* sGU;                           // bf16: [T, 4*ns*Is] rows [dG_s hi | lo | dU_s hi | lo]
  int32_t* prefix;                         // [E+1]
  float *G, *U, *Ar, *dA;                  // [R,I] each (Ar: fp32 layers only; bf16: dA = dout W_d)
  float *y, *dY, *dXs;                     // [R,d] each (y, dY: fp32 layers only)
  float *dw, *dl, *dls;                    // [R] each (dls: dl in sorted-row order)
  float* rpart;                            // [router_part_rows(R, E), d] router-gradient partials
  int32_t* poffS;                          // bf16, shared: [ksplit+1] slices of the shared K range
  float* kpart;                            // bf16, shared: [ksplit, d*Is] split-K partial products
  int ksplit;                              // bf16, shared: shared_k_split(T, d, Is)
  float *Gs, *Us, *As, *dAs;               // [T, ns*Is] each (all shared experts)
  uint16_t* Asbf;                          // bf16: [T, ns*Is] the shared SwiGLU products in bf16
  float* dxs;                              // [T,d]; bf16: [2T,d], the dG and the dU terms
  int64_t T;
  int d, E, k, I, ns, Is;
  bool bf16;
  bool valu;          // fp32 layers: products on the vector ALUs in fp32
  bool force_global;  // bf16 layers: GEMM operands through 64-bit global loads
};
void launch_layer_bwd(const BwdArgs& a, hipStream_t stream);

// Slices of the reduction index (2 * roundup(T, 64) columns, as 64-column
// steps) for a shared expert's weight gradient [M, N] on 256x256 tiles: as
// many as keep all tiles within one round on 256 compute units, each at least
// four steps long.
inline int shared_k_split(int64_t T, int M, int N) {
  const int64_t tiles = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
  const int64_t steps = 2 * ((T + 63) / 64);
  const int64_t s = std::min<int64_t>(256 / std::max<int64_t>(tiles, 1), steps / 4);
  return (int)std::max<int64_t>(s, 1);
}

// Rows of BwdArgs::rpart: one per M-tile of the experts' row segments, for
// tiles of 64 or of 128 rows (the VALU and matrix-core variants).
inline int64_t router_part_rows(int64_t R, int E) {
  return std::max((R + (int64_t)E * 63) / 64, (R + (int64_t)E * 127) / 128);
}

}  // namespace moe
