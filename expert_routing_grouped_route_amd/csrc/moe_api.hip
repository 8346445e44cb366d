// C ABI of the MoE-layer forward pass: argument validation, workspace
// carving and launch sequencing on the caller's stream.  Declarations and
// the contract of every entry point are in include/moe.h.
#include <algorithm>
#include <atomic>
#include <initializer_list>
#include <mutex>

#include "moe.h"
#include "common.h"
#include "kernels.h"
#include "backward.h"

// The workspace of moe_layer_fwd_static, for callers that cannot allocate:
// one copy per GPU, alive until the process ends.  Host code never passes
// this name to a kernel (on the host it is only a stand-in for the symbol);
// it uses the device address static_scratch() looked up for the device.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

using namespace moe;

// Device address of `scratch` on the current device, looked up once per
// device with that device current; null if the lookup fails.
void* static_scratch() {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  static std::mutex lock;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> guard(lock);
  p = addr[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    addr[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

constexpr int64_t kI32Limit = int64_t(1) << 31;

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

size_t elem_bytes(const moe_dims_t& D) { return D.dtype == MOE_BF16 ? 2 : 4; }

// Workspace layout.  The grouped FFN's SwiGLU products come first (the
// documented contents of the workspace after moe_grouped_ffn).
struct Layout {
  size_t a, ash, tile_off, ctr, blk, ids, wts, counts, offsets, perm, inv, y, ysh, total;
};

Layout layout_of(const moe_dims_t& D) {
  const size_t es = elem_bytes(D);
  const size_t T = (size_t)D.T, R = T * (size_t)D.k, E = (size_t)D.E;
  Layout L;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  L.a = take(R * D.I * es);
  L.ash = take(T * (size_t)D.n_shared * D.I_shared * es);
  L.tile_off = take((size_t)tile_table_ints((int64_t)R, D.E) * 4);
  L.ctr = take(kGemmCounters * 4);
  L.blk = take((size_t)dispatch_blocks((int64_t)R) * E * 4);
  L.ids = take(R * 4);
  L.wts = take(R * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.perm = take(R * 4);
  L.inv = take(R * 4);
  L.y = take(R * D.d * 4);
  L.ysh = take(D.n_shared ? T * D.d * 4 : 0);
  L.total = o;
  return L;
}

// Scratch of token condensation, after the layer's own workspace.
struct CLayout {
  size_t proj, pids, pwts, key, key_lo, key_hi, off1, off2, perm1, inv1, perm2, inv2, blk, tok,
      skey, cand, rep, total;
};

CLayout condense_layout_of(const moe_dims_t& D) {
  const size_t T = (size_t)D.T;
  CLayout C;
  size_t o = layout_of(D).total;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  C.proj = take(T * kCondenseBits * 4);
  C.pids = take(T * 4);
  C.pwts = take(T * 4);
  C.key = take(T * 4);
  C.key_lo = take(T * 4);
  C.key_hi = take(T * 4);
  C.off1 = take(257 * 4);
  C.off2 = take(257 * 4);
  C.perm1 = take(T * 4);
  C.inv1 = take(T * 4);
  C.perm2 = take(T * 4);
  C.inv2 = take(T * 4);
  C.blk = take((size_t)dispatch_blocks((int64_t)T) * 256 * 4);
  C.tok = take(T * 4);
  C.skey = take(T * 4);
  C.cand = take(T * 4);
  C.rep = take(T * 4);
  C.total = o;
  return C;
}

// Token condensation inputs of a layer call.
struct CondenseIn {
  const void* hyperplanes;
  float cos_threshold;
  int32_t* rep_out;
};

FfnArgs ffn_shape(const moe_dims_t& D) {
  FfnArgs f = {};
  f.T = D.T;
  f.R = D.T * D.k;
  f.d = D.d;
  f.E = D.E;
  f.I = D.I;
  f.ns = D.n_shared;
  f.Is = D.I_shared;
  f.bf16 = D.dtype == MOE_BF16;
  return f;
}

moe_status_t check_dims(const moe_dims_t* D) {
  if (!D) return MOE_ERR_INVALID_ARG;
  if (D->T < 0 || D->d <= 0 || D->E <= 0 || D->k <= 0 || D->I <= 0 || D->n_shared < 0 ||
      D->I_shared < 0)
    return MOE_ERR_INVALID_ARG;
  if ((D->n_shared == 0) != (D->I_shared == 0)) return MOE_ERR_INVALID_ARG;
  if (D->dtype != MOE_F32 && D->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (D->E > 256 || D->k > D->E || D->k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (D->d % 64 || D->I % 64 || D->I_shared % 64) return MOE_ERR_UNSUPPORTED;
  if (D->T * (int64_t)D->k >= kI32Limit) return MOE_ERR_UNSUPPORTED;
  const FfnArgs f = ffn_shape(*D);
  if (gate_up_grid(f) >= kI32Limit || down_grid(f) >= kI32Limit) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)D->n_shared * D->I_shared >= kI32Limit) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

struct Buf {
  const void* p;
  size_t bytes;
  bool required;
  bool output;
};

// Presence, 16-byte alignment, and no overlap of an output with any other buffer.
moe_status_t check_bufs(std::initializer_list<Buf> bufs) {
  for (const Buf& b : bufs) {
    if (b.bytes == 0) continue;
    if (!b.p) {
      if (b.required) return MOE_ERR_INVALID_ARG;
      continue;
    }
    if (reinterpret_cast<uintptr_t>(b.p) & 15u) return MOE_ERR_INVALID_ARG;
  }
  for (const Buf* i = bufs.begin(); i != bufs.end(); ++i) {
    if (!i->p || !i->bytes) continue;
    for (const Buf* j = i + 1; j != bufs.end(); ++j) {
      if (!j->p || !j->bytes || !(i->output || j->output)) continue;
      const uintptr_t a0 = reinterpret_cast<uintptr_t>(i->p), a1 = a0 + i->bytes;
      const uintptr_t b0 = reinterpret_cast<uintptr_t>(j->p), b1 = b0 + j->bytes;
      if (a0 < b1 && b0 < a1) return MOE_ERR_INVALID_ARG;
    }
  }
  return MOE_OK;
}

moe_status_t launched() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<uint8_t*>(ws) + off);
}

moe_status_t layer_fwd(const moe_dims_t* dims, const void* x, const void* w_router,
                       const float* bias, const void* w_gate, const void* w_up,
                       const void* w_down, const void* wsh_gate, const void* wsh_up,
                       const void* wsh_down, float* out, int32_t* topk_ids_out,
                       float* topk_w_out, int32_t* counts_out, int32_t* offsets_out,
                       int32_t* perm_out, void* ws, size_t ws_bytes, hipEvent_t* events,
                       int n_events, hipStream_t stream, hipStream_t side = nullptr,
                       hipEvent_t fork = nullptr, hipEvent_t join = nullptr,
                       const CondenseIn* cond = nullptr, int variant = 0) {
  moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  const moe_dims_t& D = *dims;
  if (variant & ~MOE_VARIANT_GLOBAL_LOADS) return MOE_ERR_INVALID_ARG;
  if (n_events < 0 || n_events > 6 || (n_events > 0 && !events)) return MOE_ERR_INVALID_ARG;
  const bool two_streams = side || fork || join;
  if (two_streams && (!side || !fork || !join || n_events)) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < n_events; ++i)
    if (!events[i]) return MOE_ERR_INVALID_ARG;
  const Layout L = layout_of(D);
  const size_t es = elem_bytes(D);
  const size_t T = (size_t)D.T, R = T * D.k, E = D.E, d = D.d;
  const bool sh = D.n_shared > 0;
  const size_t wsh_in = (size_t)D.n_shared * D.I_shared * d * es;
  if (cond && cond->cos_threshold != cond->cos_threshold) return MOE_ERR_INVALID_ARG;  // NaN
  const CLayout C = cond ? condense_layout_of(D) : CLayout{};
  const size_t ws_need = cond ? C.total : L.total;
  st = check_bufs({{x, T * d * es, true, false},
                   {w_router, E * d * es, true, false},
                   {bias, E * 4, false, false},
                   {w_gate, E * D.I * d * es, true, false},
                   {w_up, E * D.I * d * es, true, false},
                   {w_down, E * D.I * d * es, true, false},
                   {wsh_gate, wsh_in, sh, false},
                   {wsh_up, wsh_in, sh, false},
                   {wsh_down, wsh_in, sh, false},
                   {out, T * d * 4, true, true},
                   {topk_ids_out, R * 4, false, true},
                   {topk_w_out, R * 4, false, true},
                   {counts_out, E * 4, false, true},
                   {offsets_out, (E + 1) * 4, false, true},
                   {perm_out, R * 4, false, true},
                   {cond ? cond->hyperplanes : nullptr, (size_t)kCondenseBits * d * es, cond != nullptr,
                    false},
                   {cond ? cond->rep_out : nullptr, T * 4, false, true},
                   {ws, ws_need, true, true}});
  if (st != MOE_OK) return st;
  if (ws_bytes < ws_need) return MOE_ERR_WORKSPACE;

  (void)hipGetLastError();
  auto mark = [&](int i) -> bool {
    return i >= n_events || hipEventRecord(events[i], stream) == hipSuccess;
  };
  if (!mark(0)) return MOE_ERR_HIP;

  FfnArgs fa = ffn_shape(D);
  fa.xs = nullptr;
  fa.k = D.k;
  fa.x = x;
  fa.wg = w_gate;
  fa.wu = w_up;
  fa.wd = w_down;
  fa.wsg = wsh_gate;
  fa.wsu = wsh_up;
  fa.wsd = wsh_down;
  fa.tile_off = at<int32_t>(ws, L.tile_off);
  fa.ctr = at<int32_t>(ws, L.ctr);
  fa.a = at<void>(ws, L.a);
  fa.ash = at<void>(ws, L.ash);
  fa.y = at<float>(ws, L.y);
  fa.ysh = sh ? at<float>(ws, L.ysh) : nullptr;
  fa.force_global = (variant & MOE_VARIANT_GLOBAL_LOADS) != 0;
  if (two_streams) {
    // the shared experts depend on x alone: they run on the side stream from
    // the start, beside the gate, the dispatch and the routed experts
    if (hipEventRecord(fork, stream) != hipSuccess || hipStreamWaitEvent(side, fork, 0) != hipSuccess)
      return MOE_ERR_HIP;
    if (sh) {
      FfnArgs fs = fa;
      fs.part = kSharedTiles;
      launch_gate_up(fs, side);
      launch_down(fs, side);
    }
    if (hipEventRecord(join, side) != hipSuccess) return MOE_ERR_HIP;
    fa.part = kRoutedTiles;
  }

  int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(ws, L.ids);
  float* wts = topk_w_out ? topk_w_out : at<float>(ws, L.wts);
  int32_t* counts = counts_out ? counts_out : at<int32_t>(ws, L.counts);
  int32_t* offsets = offsets_out ? offsets_out : at<int32_t>(ws, L.offsets);
  int32_t* perm = perm_out ? perm_out : at<int32_t>(ws, L.perm);
  int32_t* inv = at<int32_t>(ws, L.inv);

  RouteArgs ra = {x, w_router, bias, nullptr, nullptr, ids, wts, D.T, D.d, D.E, D.k,
                  D.dtype == MOE_BF16};
  launch_route(ra, stream);
  if (!mark(1)) return MOE_ERR_HIP;

  int32_t* rep = nullptr;
  if (cond) {
    rep = cond->rep_out ? cond->rep_out : at<int32_t>(ws, C.rep);
    CondenseArgs cn = {x, cond->hyperplanes, D.T, D.d, D.dtype == MOE_BF16, cond->cos_threshold,
                       at<float>(ws, C.proj), at<int32_t>(ws, C.pids), at<float>(ws, C.pwts),
                       at<int32_t>(ws, C.key), at<int32_t>(ws, C.key_lo), at<int32_t>(ws, C.key_hi),
                       at<int32_t>(ws, C.off1), at<int32_t>(ws, C.off2), at<int32_t>(ws, C.perm1),
                       at<int32_t>(ws, C.inv1), at<int32_t>(ws, C.perm2), at<int32_t>(ws, C.inv2),
                       at<int32_t>(ws, C.blk), at<int32_t>(ws, C.tok), at<int32_t>(ws, C.skey),
                       at<int32_t>(ws, C.cand), rep};
    launch_condense(cn, stream);
  }

  // no row gather here: the gate/up GEMM reads the token rows through perm
  DispatchArgs da = {x, ids, counts, offsets, at<int32_t>(ws, L.tile_off), at<int32_t>(ws, L.ctr),
                     perm, inv, nullptr, at<int32_t>(ws, L.blk), D.T, D.d, D.E, D.k, (int)es, rep};
  launch_dispatch(da, stream);
  if (rep) launch_condense_inv(ids, rep, (int64_t)R, D.k, inv, stream);
  if (!mark(2)) return MOE_ERR_HIP;

  fa.perm = perm;
  fa.offsets = offsets;
  launch_gate_up(fa, stream);
  if (!mark(3)) return MOE_ERR_HIP;
  launch_down(fa, stream);
  if (!mark(4)) return MOE_ERR_HIP;
  if (two_streams && hipStreamWaitEvent(stream, join, 0) != hipSuccess) return MOE_ERR_HIP;

  CombineArgs ca = {fa.y, inv, wts, fa.ysh, out, D.T, D.d, D.k};
  launch_combine(ca, stream);
  if (!mark(5)) return MOE_ERR_HIP;
  return launched();
}

// Workspace of the backward pass: the routing and dispatch parts of the
// forward layout, then the backward scratch.
struct BLayout {
  size_t xs, prefix, G, U, Ar, Abf, dA, y, dY, dXs, dw, dl, dls, rpart, Gs, Us, As, Asbf, dAs, dxs,
      dGU, poff, srec, tA, tB, off1, poff1, tiles1, off2, tiles2, wsdT,
      wsgT, wsuT, dOp, sGU, poffS, kpart, total;
  int64_t seg_ld;
  int ksplit;
};

BLayout backward_layout_of(const moe_dims_t& D) {
  const size_t T = (size_t)D.T, R = T * D.k, d = D.d, I = D.I, Is = D.I_shared;
  BLayout B;
  size_t o = layout_of(D).total;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  B.xs = take(R * d * elem_bytes(D));
  B.prefix = take(((size_t)D.E + 1) * 4);
  B.G = take(R * I * 4);
  B.U = take(R * I * 4);
  B.Ar = take(D.dtype == MOE_BF16 ? 0 : R * I * 4);  // fp32 layers only
  B.Abf = take(D.dtype == MOE_BF16 ? R * I * 2 : 0);
  B.dA = take(R * I * 4);
  B.y = take(D.dtype == MOE_BF16 ? 0 : R * d * 4);   // fp32 layers only
  B.dY = take(D.dtype == MOE_BF16 ? 0 : R * d * 4);   // fp32 layers only
  B.dXs = take(R * d * 4);
  B.dw = take(R * 4);
  B.dl = take(R * 4);
  B.dls = take(R * 4);
  B.rpart = take((size_t)router_part_rows((int64_t)R, D.E) * d * 4);
  const size_t ts = T * (size_t)D.n_shared * Is;  // all shared experts side by side
  B.Gs = take(ts * 4);
  B.Us = take(ts * 4);
  B.As = take(ts * 4);
  B.Asbf = take(D.dtype == MOE_BF16 ? ts * 2 : 0);
  B.dAs = take(ts * 4);
  B.dxs = take(D.n_shared ? (D.dtype == MOE_BF16 ? 2 : 1) * T * d * 4 : 0);
  const bool bf = D.dtype == MOE_BF16;
  B.dOp = take(bf ? T * d * 4 : 0);
  B.dGU = take(bf ? R * I * 8 : 0);
  // weight-gradient operands: per expert 2 * roundup(n_e, 64) columns
  B.seg_ld = ((int64_t)(2 * (R + 63 * (size_t)D.E)) + 63) / 64 * 64;
  const size_t rows = std::max(std::max(d, I), (size_t)D.n_shared * Is);
  B.poff = take(bf ? ((size_t)D.E + 1) * 4 : 0);
  B.srec = take(bf ? (size_t)kSegXcds * seg_sched_cap((int)D.E) * 16 : 0);
  B.off1 = take(bf ? 8 : 0);
  B.poff1 = take(bf ? 8 : 0);
  const bool bsh = bf && D.n_shared > 0;
  const size_t nsI = (size_t)D.n_shared * Is;
  B.tiles1 = take(bsh ? (size_t)tile_table_ints((int64_t)T, 1) * 4 : 0);
  B.off2 = take(bsh ? 12 : 0);
  B.tiles2 = take(bsh ? (size_t)tile_table_ints(2 * (int64_t)T, 2) * 4 : 0);
  B.wsdT = take(bsh ? nsI * d * 2 : 0);
  B.wsgT = take(bsh ? 2 * nsI * d * 2 : 0);  // W_sg^T then W_su^T, one after the other
  B.wsuT = B.wsgT + nsI * d * 2;
  B.sGU = take(bsh ? T * nsI * 8 : 0);
  B.ksplit = bsh ? shared_k_split((int64_t)T, (int)d, (int)Is) : 1;
  B.poffS = take(bsh ? ((size_t)B.ksplit + 1) * 4 : 0);
  B.kpart = take(bsh && B.ksplit > 1 ? (size_t)B.ksplit * d * Is * 4 : 0);
  B.tA = take(bf ? rows * (size_t)B.seg_ld * 2 : 0);
  B.tB = take(bf ? rows * (size_t)B.seg_ld * 2 : 0);
  B.total = o;
  return B;
}

moe_status_t layer_bwd(const moe_dims_t* dims, const void* x, const void* w_router,
                       const float* bias, const void* w_gate, const void* w_up,
                       const void* w_down, const void* wsh_gate, const void* wsh_up,
                       const void* wsh_down, const float* dout, float* dx, float* dw_router,
                       float* dbias, float* dw_gate, float* dw_up, float* dw_down,
                       float* dwsh_gate, float* dwsh_up, float* dwsh_down, void* ws,
                       size_t ws_bytes, int variant, hipStream_t stream) {
  moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  const moe_dims_t& D = *dims;
  if (variant & ~(MOE_VARIANT_GLOBAL_LOADS | MOE_VARIANT_BWD_VALU)) return MOE_ERR_INVALID_ARG;
  const Layout L = layout_of(D);
  const BLayout B = backward_layout_of(D);
  const size_t es = elem_bytes(D), T = (size_t)D.T, R = T * D.k, E = D.E, d = D.d;
  const bool sh = D.n_shared > 0;
  const size_t w_in = E * D.I * d * es, wsh_in = (size_t)D.n_shared * D.I_shared * d * es;
  const size_t gw = E * D.I * d * 4, gsh = (size_t)D.n_shared * D.I_shared * d * 4;
  st = check_bufs({{x, T * d * es, true, false},
                   {w_router, E * d * es, true, false},
                   {bias, E * 4, false, false},
                   {w_gate, w_in, true, false},
                   {w_up, w_in, true, false},
                   {w_down, w_in, true, false},
                   {wsh_gate, wsh_in, sh, false},
                   {wsh_up, wsh_in, sh, false},
                   {wsh_down, wsh_in, sh, false},
                   {dout, T * d * 4, true, false},
                   {dx, T * d * 4, true, true},
                   {dw_router, E * d * 4, true, true},
                   {dbias, E * 4, false, true},
                   {dw_gate, gw, true, true},
                   {dw_up, gw, true, true},
                   {dw_down, gw, true, true},
                   {dwsh_gate, gsh, sh, true},
                   {dwsh_up, gsh, sh, true},
                   {dwsh_down, gsh, sh, true},
                   {ws, B.total, true, true}});
  if (st != MOE_OK) return st;
  if (ws_bytes < B.total) return MOE_ERR_WORKSPACE;
  if (D.T == 0) return MOE_OK;
  (void)hipGetLastError();
  int32_t* ids = at<int32_t>(ws, L.ids);
  float* wts = at<float>(ws, L.wts);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* perm = at<int32_t>(ws, L.perm);
  int32_t* inv = at<int32_t>(ws, L.inv);
  // the forward routing on the same inputs, and the dispatch with its row gather
  RouteArgs ra = {x, w_router, bias, nullptr, nullptr, ids, wts, D.T, D.d, D.E, D.k,
                  D.dtype == MOE_BF16};
  launch_route(ra, stream);
  DispatchArgs da = {x, ids, at<int32_t>(ws, L.counts), offsets, at<int32_t>(ws, L.tile_off),
                     at<int32_t>(ws, L.ctr), perm, inv, at<void>(ws, B.xs), at<int32_t>(ws, L.blk),
                     D.T, D.d, D.E, D.k, (int)es, nullptr};
  launch_dispatch(da, stream);
  BwdArgs ba = {};
  ba.x = x;
  ba.wr = w_router;
  ba.wg = w_gate;
  ba.wu = w_up;
  ba.wd = w_down;
  ba.wsg = wsh_gate;
  ba.wsu = wsh_up;
  ba.wsd = wsh_down;
  ba.dout = dout;
  ba.ids = ids;
  ba.w = wts;
  ba.offsets = offsets;
  ba.perm = perm;
  ba.inv = inv;
  ba.xs = at<void>(ws, B.xs);
  ba.dx = dx;
  ba.dw_router = dw_router;
  ba.dbias = dbias;
  ba.dw_gate = dw_gate;
  ba.dw_up = dw_up;
  ba.dw_down = dw_down;
  ba.dwsh_gate = dwsh_gate;
  ba.dwsh_up = dwsh_up;
  ba.dwsh_down = dwsh_down;
  ba.tile_off = at<int32_t>(ws, L.tile_off);
  ba.ctr = at<int32_t>(ws, L.ctr);
  ba.Abf = D.dtype == MOE_BF16 ? at<uint16_t>(ws, B.Abf) : nullptr;
  if (D.dtype == MOE_BF16) {
    ba.dOp = at<uint16_t>(ws, B.dOp);
    ba.dGU = at<uint16_t>(ws, B.dGU);
    ba.poff = at<int32_t>(ws, B.poff);
    ba.srec = at<int32_t>(ws, B.srec);
    ba.seg_ld = B.seg_ld;
    ba.tA = at<uint16_t>(ws, B.tA);
    ba.tB = at<uint16_t>(ws, B.tB);
    ba.off1 = at<int32_t>(ws, B.off1);
    ba.poff1 = at<int32_t>(ws, B.poff1);
    if (sh) {
      ba.tiles1 = at<int32_t>(ws, B.tiles1);
    ba.off2 = at<int32_t>(ws, B.off2);
    ba.tiles2 = at<int32_t>(ws, B.tiles2);
      ba.wsdT = at<uint16_t>(ws, B.wsdT);
      ba.wsgT = at<uint16_t>(ws, B.wsgT);
      ba.wsuT = at<uint16_t>(ws, B.wsuT);
      ba.sGU = at<uint16_t>(ws, B.sGU);
    }
  }
  ba.prefix = at<int32_t>(ws, B.prefix);
  ba.G = at<float>(ws, B.G);
  ba.U = at<float>(ws, B.U);
  ba.Ar = at<float>(ws, B.Ar);
  ba.dA = at<float>(ws, B.dA);
  ba.y = at<float>(ws, B.y);
  ba.dY = at<float>(ws, B.dY);
  ba.dXs = at<float>(ws, B.dXs);
  ba.dw = at<float>(ws, B.dw);
  ba.dl = at<float>(ws, B.dl);
  ba.dls = at<float>(ws, B.dls);
  ba.rpart = at<float>(ws, B.rpart);
  ba.ksplit = B.ksplit;
  ba.poffS = B.ksplit > 0 && D.n_shared && D.dtype == MOE_BF16 ? at<int32_t>(ws, B.poffS) : nullptr;
  ba.kpart = B.ksplit > 1 ? at<float>(ws, B.kpart) : nullptr;
  ba.Gs = sh ? at<float>(ws, B.Gs) : nullptr;
  ba.Us = sh ? at<float>(ws, B.Us) : nullptr;
  ba.As = sh ? at<float>(ws, B.As) : nullptr;
  ba.dAs = sh ? at<float>(ws, B.dAs) : nullptr;
  ba.Asbf = sh && D.dtype == MOE_BF16 ? at<uint16_t>(ws, B.Asbf) : nullptr;
  ba.dxs = sh ? at<float>(ws, B.dxs) : nullptr;
  ba.T = D.T;
  ba.d = D.d;
  ba.E = D.E;
  ba.k = D.k;
  ba.I = D.I;
  ba.ns = D.n_shared;
  ba.Is = D.I_shared;
  ba.bf16 = D.dtype == MOE_BF16;
  ba.valu = !ba.bf16 && (variant & MOE_VARIANT_BWD_VALU) != 0;
  ba.force_global = (variant & MOE_VARIANT_GLOBAL_LOADS) != 0;
  launch_layer_bwd(ba, stream);
  return launched();
}

}  // namespace

extern "C" {

size_t moe_backward_workspace_bytes(const moe_dims_t* dims) {
  if (check_dims(dims) != MOE_OK) return 0;
  return backward_layout_of(*dims).total;
}

moe_status_t moe_layer_bwd(const moe_dims_t* dims, const void* x, const void* w_router,
                           const float* bias, const void* w_gate, const void* w_up,
                           const void* w_down, const void* wsh_gate, const void* wsh_up,
                           const void* wsh_down, const float* dout, float* dx, float* dw_router,
                           float* dbias, float* dw_gate, float* dw_up, float* dw_down,
                           float* dwsh_gate, float* dwsh_up, float* dwsh_down, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  return layer_bwd(dims, x, w_router, bias, w_gate, w_up, w_down, wsh_gate, wsh_up, wsh_down,
                   dout, dx, dw_router, dbias, dw_gate, dw_up, dw_down, dwsh_gate, dwsh_up,
                   dwsh_down, ws, ws_bytes, 0, stream);
}

moe_status_t moe_layer_bwd_variant(const moe_dims_t* dims, const void* x, const void* w_router,
                                   const float* bias, const void* w_gate, const void* w_up,
                                   const void* w_down, const void* wsh_gate, const void* wsh_up,
                                   const void* wsh_down, const float* dout, float* dx,
                                   float* dw_router, float* dbias, float* dw_gate, float* dw_up,
                                   float* dw_down, float* dwsh_gate, float* dwsh_up,
                                   float* dwsh_down, void* ws, size_t ws_bytes, int variant,
                                   hipStream_t stream) {
  return layer_bwd(dims, x, w_router, bias, w_gate, w_up, w_down, wsh_gate, wsh_up, wsh_down,
                   dout, dx, dw_router, dbias, dw_gate, dw_up, dw_down, dwsh_gate, dwsh_up,
                   dwsh_down, ws, ws_bytes, variant, stream);
}

size_t moe_workspace_bytes(const moe_dims_t* dims) {
  if (check_dims(dims) != MOE_OK) return 0;
  return layout_of(*dims).total;
}

const char* moe_status_str(moe_status_t status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: null, misaligned or overlapping buffer, or invalid size";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: sizes outside the supported limits";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace smaller than moe_workspace_bytes()";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch failed";
    case MOE_ERR_SCRATCH:
      return "MOE_ERR_SCRATCH: these sizes need more workspace than moe_layer_fwd_static's "
             "static scratch (MOE_STATIC_SCRATCH_BYTES) holds; use moe_layer_fwd with a workspace";
  }
  return "unknown moe_status_t";
}

moe_status_t moe_route(const moe_dims_t* dims, const void* x, const void* w_router,
                       const float* bias, const float* logits_in, float* logits_out,
                       int32_t* topk_ids, float* topk_w, hipStream_t stream) {
  moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  const moe_dims_t& D = *dims;
  const size_t es = elem_bytes(D), T = (size_t)D.T, E = D.E, d = D.d;
  const bool computed = logits_in == nullptr;
  st = check_bufs({{x, T * d * es, computed, false},
                   {w_router, E * d * es, computed, false},
                   {bias, E * 4, false, false},
                   {logits_in, T * E * 4, false, false},
                   {logits_out, T * E * 4, false, true},
                   {topk_ids, T * D.k * 4, true, true},
                   {topk_w, T * D.k * 4, true, true}});
  if (st != MOE_OK) return st;
  if (D.T == 0) return MOE_OK;
  (void)hipGetLastError();
  RouteArgs ra = {x, w_router, bias, logits_in, logits_out, topk_ids, topk_w, D.T, D.d, D.E, D.k,
                  D.dtype == MOE_BF16};
  launch_route(ra, stream);
  return launched();
}

moe_status_t moe_dispatch(const moe_dims_t* dims, const void* x, const int32_t* topk_ids,
                          int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                          void* x_sorted, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  const moe_dims_t& D = *dims;
  const Layout L = layout_of(D);
  const size_t es = elem_bytes(D), T = (size_t)D.T, R = T * D.k, E = D.E, d = D.d;
  st = check_bufs({{x, T * d * es, true, false},
                   {topk_ids, R * 4, true, false},
                   {counts, E * 4, true, true},
                   {offsets, (E + 1) * 4, true, true},
                   {perm, R * 4, true, true},
                   {inv_perm, R * 4, true, true},
                   {x_sorted, R * d * es, true, true},
                   {ws, L.total, true, true}});
  if (st != MOE_OK) return st;
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  (void)hipGetLastError();
  DispatchArgs da = {x, topk_ids, counts, offsets, nullptr, nullptr, perm, inv_perm, x_sorted,
                     at<int32_t>(ws, L.blk), D.T, D.d, D.E, D.k, (int)es};
  launch_dispatch(da, stream);
  return launched();
}

moe_status_t moe_grouped_ffn(const moe_dims_t* dims, const void* x_sorted, const int32_t* offsets,
                             const void* w_gate, const void* w_up, const void* w_down,
                             const void* x, const void* wsh_gate, const void* wsh_up,
                             const void* wsh_down, float* y_sorted, float* y_shared, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  const moe_dims_t& D = *dims;
  const Layout L = layout_of(D);
  const size_t es = elem_bytes(D), T = (size_t)D.T, R = T * D.k, E = D.E, d = D.d;
  const bool sh = D.n_shared > 0;
  const size_t wsh_in = (size_t)D.n_shared * D.I_shared * d * es;
  st = check_bufs({{x_sorted, R * d * es, true, false},
                   {offsets, (E + 1) * 4, true, false},
                   {w_gate, E * D.I * d * es, true, false},
                   {w_up, E * D.I * d * es, true, false},
                   {w_down, E * D.I * d * es, true, false},
                   {x, sh ? T * d * es : 0, sh, false},
                   {wsh_gate, wsh_in, sh, false},
                   {wsh_up, wsh_in, sh, false},
                   {wsh_down, wsh_in, sh, false},
                   {y_sorted, R * d * 4, true, true},
                   {y_shared, sh ? T * d * 4 : 0, sh, true},
                   {ws, L.total, true, true}});
  if (st != MOE_OK) return st;
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (D.T == 0) return MOE_OK;
  (void)hipGetLastError();
  FfnArgs fa = ffn_shape(D);
  fa.xs = x_sorted;
  fa.perm = nullptr;
  fa.k = D.k;
  fa.x = x;
  fa.wg = w_gate;
  fa.wu = w_up;
  fa.wd = w_down;
  fa.wsg = wsh_gate;
  fa.wsu = wsh_up;
  fa.wsd = wsh_down;
  fa.offsets = offsets;
  fa.tile_off = at<int32_t>(ws, L.tile_off);
  fa.ctr = at<int32_t>(ws, L.ctr);
  fa.a = at<void>(ws, L.a);
  fa.ash = at<void>(ws, L.ash);
  fa.y = y_sorted;
  fa.ysh = sh ? y_shared : nullptr;
  launch_tile_table(offsets, D.E, at<int32_t>(ws, L.tile_off), at<int32_t>(ws, L.ctr), stream);
  launch_gate_up(fa, stream);
  launch_down(fa, stream);
  return launched();
}

moe_status_t moe_combine(const moe_dims_t* dims, const float* y_sorted, const int32_t* inv_perm,
                         const float* topk_w, const float* y_shared, float* out,
                         hipStream_t stream) {
  moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  const moe_dims_t& D = *dims;
  const size_t T = (size_t)D.T, R = T * D.k, d = D.d;
  st = check_bufs({{y_sorted, R * d * 4, true, false},
                   {inv_perm, R * 4, true, false},
                   {topk_w, R * 4, true, false},
                   {y_shared, T * d * 4, false, false},
                   {out, T * d * 4, true, true}});
  if (st != MOE_OK) return st;
  if (D.T == 0) return MOE_OK;
  (void)hipGetLastError();
  CombineArgs ca = {y_sorted, inv_perm, topk_w, y_shared, out, D.T, D.d, D.k};
  launch_combine(ca, stream);
  return launched();
}

moe_status_t moe_layer_fwd(const moe_dims_t* dims, const void* x, const void* w_router,
                           const float* bias, const void* w_gate, const void* w_up,
                           const void* w_down, const void* wsh_gate, const void* wsh_up,
                           const void* wsh_down, float* out, int32_t* topk_ids_out,
                           float* topk_w_out, int32_t* counts_out, int32_t* offsets_out,
                           int32_t* perm_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return layer_fwd(dims, x, w_router, bias, w_gate, w_up, w_down, wsh_gate, wsh_up, wsh_down, out,
                   topk_ids_out, topk_w_out, counts_out, offsets_out, perm_out, ws, ws_bytes,
                   nullptr, 0, stream);
}

moe_status_t moe_layer_fwd_static(const moe_dims_t* dims, const void* x, const void* w_router,
                                  const float* bias, const void* w_gate, const void* w_up,
                                  const void* w_down, const void* wsh_gate, const void* wsh_up,
                                  const void* wsh_down, float* out, int32_t* topk_ids_out,
                                  float* topk_w_out, int32_t* counts_out, int32_t* offsets_out,
                                  int32_t* perm_out, hipStream_t stream) {
  const moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  const size_t need = layout_of(*dims).total;
  if (need > MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  void* ws = static_scratch();
  if (!ws) return MOE_ERR_HIP;
  return layer_fwd(dims, x, w_router, bias, w_gate, w_up, w_down, wsh_gate, wsh_up, wsh_down, out,
                   topk_ids_out, topk_w_out, counts_out, offsets_out, perm_out, ws, need,
                   nullptr, 0, stream);
}

moe_status_t moe_layer_fwd_variant(const moe_dims_t* dims, const void* x, const void* w_router,
                                   const float* bias, const void* w_gate, const void* w_up,
                                   const void* w_down, const void* wsh_gate, const void* wsh_up,
                                   const void* wsh_down, float* out, int32_t* topk_ids_out,
                                   float* topk_w_out, int32_t* counts_out, int32_t* offsets_out,
                                   int32_t* perm_out, void* ws, size_t ws_bytes, int variant,
                                   hipStream_t stream) {
  return layer_fwd(dims, x, w_router, bias, w_gate, w_up, w_down, wsh_gate, wsh_up, wsh_down, out,
                   topk_ids_out, topk_w_out, counts_out, offsets_out, perm_out, ws, ws_bytes,
                   nullptr, 0, stream, nullptr, nullptr, nullptr, nullptr, variant);
}

moe_status_t moe_layer_fwd_timed(const moe_dims_t* dims, const void* x, const void* w_router,
                                 const float* bias, const void* w_gate, const void* w_up,
                                 const void* w_down, const void* wsh_gate, const void* wsh_up,
                                 const void* wsh_down, float* out, int32_t* topk_ids_out,
                                 float* topk_w_out, int32_t* counts_out, int32_t* offsets_out,
                                 int32_t* perm_out, void* ws, size_t ws_bytes,
                                 hipEvent_t* events, int n_events, hipStream_t stream) {
  return layer_fwd(dims, x, w_router, bias, w_gate, w_up, w_down, wsh_gate, wsh_up, wsh_down, out,
                   topk_ids_out, topk_w_out, counts_out, offsets_out, perm_out, ws, ws_bytes,
                   events, n_events, stream);
}

moe_status_t moe_layer_fwd_overlap(const moe_dims_t* dims, const void* x, const void* w_router,
                                   const float* bias, const void* w_gate, const void* w_up,
                                   const void* w_down, const void* wsh_gate, const void* wsh_up,
                                   const void* wsh_down, float* out, int32_t* topk_ids_out,
                                   float* topk_w_out, int32_t* counts_out, int32_t* offsets_out,
                                   int32_t* perm_out, void* ws, size_t ws_bytes,
                                   hipStream_t stream, hipStream_t side, hipEvent_t fork,
                                   hipEvent_t join) {
  if (!side || !fork || !join) return MOE_ERR_INVALID_ARG;
  return layer_fwd(dims, x, w_router, bias, w_gate, w_up, w_down, wsh_gate, wsh_up, wsh_down, out,
                   topk_ids_out, topk_w_out, counts_out, offsets_out, perm_out, ws, ws_bytes,
                   nullptr, 0, stream, side, fork, join);
}

size_t moe_condensed_workspace_bytes(const moe_dims_t* dims) {
  if (check_dims(dims) != MOE_OK) return 0;
  return condense_layout_of(*dims).total;
}

moe_status_t moe_layer_fwd_condensed(const moe_dims_t* dims, const void* x, const void* w_router,
                                     const float* bias, const void* w_gate, const void* w_up,
                                     const void* w_down, const void* wsh_gate, const void* wsh_up,
                                     const void* wsh_down, const void* hyperplanes,
                                     float cos_threshold, float* out, int32_t* topk_ids_out,
                                     float* topk_w_out, int32_t* counts_out, int32_t* offsets_out,
                                     int32_t* perm_out, int32_t* rep_out, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  const CondenseIn cond = {hyperplanes, cos_threshold, rep_out};
  return layer_fwd(dims, x, w_router, bias, w_gate, w_up, w_down, wsh_gate, wsh_up, wsh_down, out,
                   topk_ids_out, topk_w_out, counts_out, offsets_out, perm_out, ws, ws_bytes,
                   nullptr, 0, stream, nullptr, nullptr, nullptr, &cond);
}

}  // extern "C"
