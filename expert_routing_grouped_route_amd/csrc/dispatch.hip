// Dispatch of the MoE layer on one GPU: every (token, slot) assignment gets a
// row in a per-expert contiguous segment, and the token rows are copied there.
//
// On the pages Dispatch is the all-to-all that sends each token to the device
// holding its expert (FarSkip-Collective review, "Core claim" and Fig. 11
// caption; the Luffy review, "Core claim", on dispatch and combine traffic).
// On one GPU's share it is a stable counting sort by expert plus a row gather.
// The order inside a segment (ascending assignment index t*k + j) is a
// reading; the pages do not fix it.
//
// Three kernels, no atomics on results and no host round trip:
//   count:  per block of `chunk` assignments, an LDS histogram of expert ids
//   rank:   per block of the same chunk: from the histograms of all blocks
//           (at most 256 x E ints), each expert's total and this block's base
//           (the sum over earlier blocks), the offsets as an exclusive scan
//           of the totals; then its chunk in order, 256 assignments at a
//           time: the stable rank within a wave from ballots on the id bits,
//           across waves from LDS counts; writes perm and inv_perm.  Block 0
//           also writes counts, offsets and the M-tile table of the grouped
//           GEMMs (M-tile prefix per expert and the expert of every M-tile).
//   scatter: one wave per token reads its row once (16-byte vectors) and
//           writes it to the sorted rows of its k assignments
#include "common.h"
#include "kernels.h"

namespace moe {

int dispatch_chunk(int64_t R) {
  // at most 256 blocks, so the per-expert scan over blocks stays short
  int64_t c = (R + 255) / 256;
  c = (c + 255) / 256 * 256;
  return (int)(c < kDispatchChunk ? kDispatchChunk : c);
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cached[dev]) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cached[dev] = n;
  return n;
}

int dispatch_blocks(int64_t R) {
  const int64_t c = dispatch_chunk(R);
  return (int)((R + c - 1) / c);
}

// Token condensation: assignment a = t*k + j (expert e) is condensed when the
// token's representative is another token that is also routed to e.
__device__ __forceinline__ bool is_condensed(const int32_t* __restrict__ ids,
                                             const int32_t* __restrict__ rep, int k, int a, int e) {
  if (!rep) return false;
  const int t = a / k, r = rep[t];
  if (r == t) return false;
  for (int j = 0; j < k; ++j)
    if (ids[(size_t)r * k + j] == e) return true;
  return false;
}

__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ ids,
                                                             int R, int E, int chunk,
                                                             const int32_t* __restrict__ rep, int k,
                                                             int32_t* __restrict__ blk) {
  __shared__ int h[256];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int a0 = blockIdx.x * chunk, a1 = min(R, a0 + chunk);
  // one LDS atomic per distinct expert of a wave's 64 assignments: the lanes
  // of an expert found by ballots over the bits of e, the lowest adding them
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const uint64_t below = (1ull << (threadIdx.x & 63)) - 1ull;
  for (int p = a0; p < a1; p += 256) {
    const int a = p + (int)threadIdx.x;
    const int e = a < a1 ? ids[a] : -1;
    const bool ok = (unsigned)e < (unsigned)E && !is_condensed(ids, rep, k, a, e);
    uint64_t peers = __ballot(ok);
    for (int bit = 0; bit < nbits; ++bit) {
      const uint64_t m = __ballot(ok && ((e >> bit) & 1));
      peers &= ((e >> bit) & 1) ? m : ~m;
    }
    if (ok && (peers & below) == 0) atomicAdd(&h[e], __popcll(peers));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) blk[(size_t)blockIdx.x * E + e] = h[e];
}

// Inclusive scan of one value per thread over a 256-thread block.
__device__ __forceinline__ int block_inclusive_scan(int v, int* buf) {
  buf[threadIdx.x] = v;
  __syncthreads();
#pragma unroll
  for (int off = 1; off < 256; off <<= 1) {
    const int add = threadIdx.x >= off ? buf[threadIdx.x - off] : 0;
    __syncthreads();
    buf[threadIdx.x] += add;
    __syncthreads();
  }
  return buf[threadIdx.x];
}

// The GEMM tile table: tiles[0..E] = M-tile prefix per expert (units of kBM
// rows), followed by tiles[E+1+j] = expert of M-tile j.
__device__ __forceinline__ void write_tile_table(int cnt, int E, int32_t* __restrict__ tiles,
                                                 int* buf) {
  const int e = threadIdx.x;
  const int nt = (cnt + kBM - 1) / kBM;
  const int tincl = block_inclusive_scan(nt, buf);
  if (e < E) {
    tiles[e] = tincl - nt;
    for (int j = tincl - nt; j < tincl; ++j) tiles[E + 1 + j] = e;
  }
  if (e == E - 1) tiles[E] = tincl;
}

__global__ __launch_bounds__(256) void tile_table_kernel(const int32_t* __restrict__ offsets,
                                                         int E, int32_t* __restrict__ tiles,
                                                         int32_t* __restrict__ ctr) {
  __shared__ int buf[256];
  const int e = threadIdx.x;
  if (e < kGemmCounters) ctr[e] = 0;
  const int cnt = e < E ? offsets[e + 1] - offsets[e] : 0;
  write_tile_table(cnt, E, tiles, buf);
}

__global__ __launch_bounds__(256) void dispatch_rank_kernel(
    const int32_t* __restrict__ ids, int R, int E, int chunk, const int32_t* __restrict__ rep,
    int k, const int32_t* __restrict__ blk,
    int nblk, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ tiles, int32_t* __restrict__ ctr, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv_perm) {
  __shared__ int run[256];     // next free row per expert for this block
  __shared__ int wc[4][256];   // per-wave counts of the current 256 assignments
  __shared__ int buf[256];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int a0 = blockIdx.x * chunk, a1 = min(R, a0 + chunk);
  // expert e's total over all blocks and its count in the blocks before this
  // one: ng = 256 / E threads per expert, thread g of expert e summing the
  // blocks g, g + ng, ..., sixteen loads in flight at a time; then the ng
  // partial sums per expert (integers: the order does not matter)
  int total = 0, before = 0;
  {
    const int ng = 256 / E, e = tid % E, g = tid / E;
    int tp = 0, bp = 0;
    if (g < ng) {
      constexpr int U = 16;
      for (int b0 = g; b0 < nblk; b0 += U * ng) {
        int c[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int b = b0 + u * ng;
          c[u] = b < nblk ? blk[(size_t)b * E + e] : 0;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          tp += c[u];
          bp += b0 + u * ng < (int)blockIdx.x ? c[u] : 0;
        }
      }
    }
    wc[0][tid] = tp;  // wc is free until the loop below
    wc[1][tid] = bp;
    __syncthreads();
    if (tid < E)
      for (int j = 0; j < ng; ++j) {
        total += wc[0][j * E + tid];
        before += wc[1][j * E + tid];
      }
    __syncthreads();
  }
  const int incl = block_inclusive_scan(tid < E ? total : 0, buf);
  if (tid < E) run[tid] = incl - total + before;
  if (blockIdx.x == 0) {
    if (ctr && tid < kGemmCounters) ctr[tid] = 0;
    if (counts && tid < E) counts[tid] = total;
    if (tid < E) offsets[tid] = incl - total;
    if (tid == E - 1) offsets[E] = incl;
    __syncthreads();
    if (tiles) write_tile_table(tid < E ? total : 0, E, tiles, buf);
  }
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int p = a0; p < a1; p += 256) {
    for (int i = tid; i < 4 * 256; i += 256) (&wc[0][0])[i] = 0;
    __syncthreads();
    const int a = p + tid;
    const int e = a < a1 ? ids[a] : -1;
    const bool ok = (unsigned)e < (unsigned)E && !is_condensed(ids, rep, k, a, e);
    uint64_t peers = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = ok && ((e >> b) & 1);
      const uint64_t m = __ballot(bit);
      peers &= ((e >> b) & 1) ? m : ~m;
    }
    const int rank = __popcll(peers & below);
    if (ok && rank == 0) wc[wave][e] = __popcll(peers);
    __syncthreads();
    if (ok) {
      int dest = run[e] + rank;
      for (int w = 0; w < wave; ++w) dest += wc[w][e];
      perm[dest] = a;
      inv_perm[a] = dest;
    }
    __syncthreads();
    for (int e2 = tid; e2 < E; e2 += 256)
      run[e2] += wc[0][e2] + wc[1][e2] + wc[2][e2] + wc[3][e2];
    __syncthreads();
  }
}

// x_sorted[inv_perm[t*k + j]] = x[t] for every assignment with a valid expert:
// one wave per token reads the row once, 16-byte vectors, up to four per lane
// in flight, and writes it to its k sorted rows (so x is read once rather than
// k times).  Assignments whose id is outside [0,E) have no row and are
// skipped; a row index past the total is never written.
__global__ __launch_bounds__(256) void scatter_rows_kernel(const u32x4* __restrict__ x,
                                                           const int32_t* __restrict__ ids,
                                                           const int32_t* __restrict__ inv_perm,
                                                           const int32_t* __restrict__ total_ptr,
                                                           int T, int k, int E, int vec_per_row,
                                                           u32x4* __restrict__ xs) {
  const int total = *total_ptr;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int t = blockIdx.x * 4 + wave; t < T; t += gridDim.x * 4) {
    int dst[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      dst[j] = -1;
      if (j < k) {
        const size_t a = (size_t)t * k + j;
        const int e = ids[a];
        const int r = (unsigned)e < (unsigned)E ? inv_perm[a] : -1;
        dst[j] = (unsigned)r < (unsigned)total ? r : -1;
      }
    }
    const u32x4* src = x + (size_t)t * vec_per_row;
    for (int c0 = 0; c0 < vec_per_row; c0 += 256) {
      u32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + u * 64 + lane;
        if (c < vec_per_row) v[u] = src[c];
      }
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        if (dst[j] < 0) continue;
        u32x4* out = xs + (size_t)dst[j] * vec_per_row;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = c0 + u * 64 + lane;
          if (c < vec_per_row) out[c] = v[u];
        }
      }
    }
  }
}

void launch_dispatch(const DispatchArgs& a, hipStream_t stream) {
  const int64_t R = a.T * a.k;
  const int chunk = dispatch_chunk(R);
  const int nblk = dispatch_blocks(R);
  const dim3 block(256);
  if (nblk > 0)
    hipLaunchKernelGGL(dispatch_count_kernel, dim3(nblk), block, 0, stream, a.ids, (int)R, a.E,
                       chunk, a.rep, a.k, a.blk);
  // at least one block, so that R == 0 still writes zero counts and offsets
  hipLaunchKernelGGL(dispatch_rank_kernel, dim3(nblk > 0 ? nblk : 1), block, 0, stream, a.ids,
                     (int)R, a.E, chunk, a.rep, a.k, a.blk, nblk, a.counts, a.offsets, a.tiles, a.ctr, a.perm,
                     a.inv_perm);
  if (nblk == 0) return;
  if (a.x_sorted) {  // (never asked for together with token condensation)
    const int vec = (int)((size_t)a.d * a.elem_bytes / 16);
    const int64_t grid = (a.T + 3) / 4;
    hipLaunchKernelGGL(scatter_rows_kernel, dim3((unsigned)grid), block, 0, stream,
                       static_cast<const u32x4*>(a.x), a.ids, a.inv_perm, a.offsets + a.E,
                       (int)a.T, a.k, a.E, vec, static_cast<u32x4*>(a.x_sorted));
  }
}

void launch_tile_table(const int32_t* offsets, int E, int32_t* tiles, int32_t* ctr,
                       hipStream_t stream) {
  hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(256), 0, stream, offsets, E, tiles, ctr);
}

// The backward's small tables in one launch: the M-tile prefix of G row
// segments (offsets [G+1], tiles of `tile` rows: prefix[g] = tiles before
// segment g, prefix[G] = all; G <= 256), and, with off1 non-null, the tables
// of one segment of T rows (off1 = {0, T}, poff1 = {0, 2 roundup(T, 64)}, its
// tile table tiles1) and of two segments of T rows each (off2 = {0, T, 2T},
// tiles2), with the GEMM counters zeroed as the tile table's launch zeroes
// them.
__global__ __launch_bounds__(256) void segment_tables_kernel(
    const int32_t* __restrict__ offsets, int G, int tile, int32_t* __restrict__ prefix, int T,
    int32_t* __restrict__ off1, int32_t* __restrict__ poff1, int32_t* __restrict__ tiles1,
    int32_t* __restrict__ off2, int32_t* __restrict__ tiles2, int32_t* __restrict__ ctr) {
  __shared__ int buf[256];
  const int tid = threadIdx.x;
  const int nt = tid < G ? (offsets[tid + 1] - offsets[tid] + tile - 1) / tile : 0;
  const int incl = block_inclusive_scan(nt, buf);
  if (tid < G) prefix[tid] = incl - nt;
  if (tid == G - 1) prefix[G] = incl;
  if (G == 0 && tid == 0) prefix[0] = 0;
  if (!off1) return;  // block-uniform
  if (tid == 0) {
    off1[0] = 0;
    off1[1] = T;
    poff1[0] = 0;
    poff1[1] = 2 * ((T + 63) / 64 * 64);
    off2[0] = 0;
    off2[1] = T;
    off2[2] = 2 * T;
  }
  if (tid < kGemmCounters) ctr[tid] = 0;
  __syncthreads();  // buf is reused
  write_tile_table(tid < 1 ? T : 0, 1, tiles1, buf);
  __syncthreads();
  write_tile_table(tid < 2 ? T : 0, 2, tiles2, buf);
}

void launch_segment_tables(const int32_t* offsets, int G, int tile, int32_t* prefix, int64_t T,
                           int32_t* off1, int32_t* poff1, int32_t* tiles1, int32_t* off2,
                           int32_t* tiles2, int32_t* ctr, hipStream_t stream) {
  hipLaunchKernelGGL(segment_tables_kernel, dim3(1), dim3(256), 0, stream, offsets, G, tile,
                     prefix, (int)T, off1, poff1, tiles1, off2, tiles2, ctr);
}

}  // namespace moe
