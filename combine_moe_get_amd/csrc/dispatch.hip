// dispatch.hip -- quantize (optionally) and scatter the routed copies of each
// token into its expert-major receive rows.
//
// What is computed follows the CANN "low_latency_dispatch" page, Function /
// Formula, dynamic quantization scenario: quant_out = x (mode 0) or
// CastToInt8(fp32(x) * scales) (static) or, in the dynamic mode,
// x_fp32 = fp32(x) * scales, dyn = 127 / max|x_fp32|,
// q = CastToInt8(x_fp32 * dyn), with 1/dyn sent along with every row.  The
// alltoallv of quant_out becomes a copy of the row to every receive row the
// layout gave the token's routed slots.
//
// Work split (measured on gfx950: more, smaller waves keep more HBM traffic
// in flight than one wave per token holding the whole row):
//  - bf16 copy: one wave per (token, 2 KB slice of the row); lane l loads two
//    16-byte chunks and stores them to each of the token's K rows.
//  - int8: one workgroup per token, one lane per 16 channels (32 bytes of
//    bf16 in, 16 bytes of codes out, so every store instruction of a wave
//    writes 1 KB contiguous); the dynamic scale needs the row's amax: a wave
//    max, then a max over the <= 8 waves through LDS.
//  - int8 with per-expert scales: one workgroup per token (dynamic) or per
//    (token, expert-id parity) (static), the copies quantized one at a time (see
//    dispatch_quant_expert_kernel).
// Static codes from moe_dispatch on large batches are preceded by a sequential read-ahead
// of the token rows (dispatch_read_ahead_kernel, see launch_dispatch).
// Every kernel also has a looping form for moe_dispatch_capped: a grid of at most
// max_workgroups workgroups walks the same work items with a grid stride (the per-item
// code is shared, so the results are identical).
// Loads are ordinary (the row is read once, K stores reuse it from VGPRs; the bf16
// copy reads through a buffer resource, row_load).
// Receive rows are written once and read by a later kernel: the int8 codes are
// stored non-temporally, the bf16 copies of dispatch_copy_kernel with the sc1
// policy (row_store_sc1), whichever measured faster for each; after the
// read-ahead of moe_layout_dispatch the bf16 copies are stored non-temporally
// too (the NT form), and the single-launch layout + dispatch kernel, for
// batches of at most 8192 slots, keeps non-temporal stores for both.
#include "dispatch_dev.hpp"

namespace moe {

// ---- bf16 passthrough --------------------------------------------------------
// one wave per workgroup; wave gw = (token, slice), slice sl covers the 16-byte chunks
// [128 sl, 128 sl + 128) of the row: lane l copies chunks 128 sl + l and 128 sl + 64 + l.
// Measured on gfx950 at T=4096, H=7168, top-8 with every input read from HBM (non-temporal
// stores then): 104.2-104.6 us against 105.6-106.5 us for 1 KB slices in four-wave workgroups.
// With buffer-resource loads and sc1 stores (98-100 us), 1, 3 and 4 KB slices measured
// 102.6-103.5, 104.7-105.3 and 106.2-106.7 us against 100.1-100.8 us for 2 KB in one run.
template <bool NT>
__device__ __forceinline__ void dispatch_copy_item(const DispatchArgs &a, int nslice, int gw) {
  const int lane = threadIdx.x;
  const int t = gw / nslice, sl = gw - t * nslice;
  if (t >= a.T) return;
  const int K = a.K, H = a.H, nch = H >> 3;

  // the slice is requested together with the slot rows (not after them): one load latency
  // less per wave, at the price of reading the slice of a token with no routed copy
  int myrow = -1;
  if (lane < K) myrow = a.dst_row[(size_t)t * K + lane];
  const int c0 = lane + 128 * sl, c1 = c0 + 64;
  const uint16_t *xr = a.x + (size_t)t * H;
  u32x4 v0 = u32x4{0u, 0u, 0u, 0u}, v1 = v0;
  if (c0 < nch) v0 = row_load(xr, 2 * H, c0 * 16);
  if (c1 < nch) v1 = row_load(xr, 2 * H, c1 * 16);
  uint64_t valid = ballot(myrow >= 0);
  if (valid == 0ull) return;  // masked token, or only special / dropped slots
  const bool write_w = sl == 0 && myrow >= 0 && a.expand_w;

  while (valid) {
    const int j = __builtin_ctzll(valid);
    valid &= valid - 1;
    void *dst = (uint16_t *)a.expand_x + (size_t)readlane(myrow, j) * H;
    if (NT) {
      if (c0 < nch) __builtin_nontemporal_store(v0, (u32x4 *)dst + c0);
      if (c1 < nch) __builtin_nontemporal_store(v1, (u32x4 *)dst + c1);
    } else {
      if (c0 < nch) row_store_sc1(v0, dst, 2 * H, c0 * 16);
      if (c1 < nch) row_store_sc1(v1, dst, 2 * H, c1 * 16);
    }
  }
  if (write_w) a.expand_w[myrow] = a.w ? a.w[(size_t)t * K + lane] : 1.0f;
}

// items: T * nslice (token, slice) pairs.  LOOP: a grid smaller than that (a capped launch) walks
// them with a grid stride; otherwise one workgroup per item (the loop costs registers: 12 -> 18).
// NT: non-temporal stores, used when the token rows were just read ahead into the Infinity Cache
// (moe_layout_dispatch).  With the read-ahead, sc1 stores made the layer slower (T=4096, H=7168,
// top-8, Zipf: 202.8 against 196.4 us per layer without read-ahead), non-temporal ones did not
// (194.4-195.4); without the read-ahead sc1 stores are the faster (101.5 against 104 us for the
// copy alone).
template <bool LOOP, bool NT>
__global__ void __launch_bounds__(64) dispatch_copy_kernel(DispatchArgs a, int nslice, int items) {
  if constexpr (LOOP) {
    for (int gw = blockIdx.x; gw < items; gw += gridDim.x) dispatch_copy_item<NT>(a, nslice, gw);
  } else {
    dispatch_copy_item<NT>(a, nslice, blockIdx.x);
  }
}

// ---- int8 (static or dynamic) -----------------------------------------------
// one workgroup per token, blockDim = 64 * ceil(pairs / 64) <= 512; lane p of the
// block owns channels [16p, 16p + 16) (chunks 2p and 2p + 1).  One code row per
// token (no smoothing, or one smooth vector for all experts), stored to every
// routed copy.
template <int MODE>
__device__ __forceinline__ void dispatch_quant_item(const DispatchArgs &a, int t, float (*red)[8], int &par) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int K = a.K, H = a.H;

  // every load of the lane is issued before the first use: slot rows, row chunks, scales.
  // The row is requested before the slot rows are known (one load latency less per
  // token; a token with no routed copy has its row read for nothing).
  int myrow = -1;
  if (lane < K) myrow = a.dst_row[(size_t)t * K + lane];
  const QuantLane q(H);
  const u32x4 *xr = (const u32x4 *)(a.x + (size_t)t * H);
  const u32x4 v0 = xr[q.l0], v1 = xr[q.l1];
  f32x4 s4[4] = {f32x4{1.f, 1.f, 1.f, 1.f}, f32x4{1.f, 1.f, 1.f, 1.f}, f32x4{1.f, 1.f, 1.f, 1.f},
                 f32x4{1.f, 1.f, 1.f, 1.f}};
  if (a.smooth) q.load_scales(a.smooth, s4);
  uint64_t valid = ballot(myrow >= 0);
  if (valid == 0ull) return;  // same for every wave of the block: no barrier is skipped

  float f[16], g[16];
  unpack8(v0, f);
  unpack8(v1, f + 8);
  q.scale16(f, s4, g);
  float dyn = 1.0f;
  if constexpr (MODE == 2) {
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(g[e]));
    m = wave_max(m);
    if (lane == 0) red[par][wv] = m;
    __syncthreads();
    const float amax = block_max_of(red[par], nw);
    par ^= 1;
    dyn = amax > 0.0f ? 127.0f / amax : 0.0f;
    if (wv == 0 && myrow >= 0 && a.dyn_scales) a.dyn_scales[myrow] = amax > 0.0f ? 1.0f / dyn : 0.0f;
  }
  const bool write_w = wv == 0 && myrow >= 0 && a.expand_w;
  while (valid) {
    const int j = __builtin_ctzll(valid);
    valid &= valid - 1;
    q.store_codes<MODE>(g, dyn, (int8_t *)a.expand_x + (size_t)readlane(myrow, j) * H);
  }
  if (write_w) a.expand_w[myrow] = a.w ? a.w[(size_t)t * K + lane] : 1.0f;
}

// items: the T tokens.  With a capped grid a workgroup quantizes several tokens in turn; the two
// halves of red[][] alternate from one amax to the next (across tokens too), so one barrier per
// token keeps a wave's next write away from the half the slower waves still read.
template <int MODE, bool LOOP>
__global__ void __launch_bounds__(512) dispatch_quant_kernel(DispatchArgs a) {
  __shared__ float red[2][8];
  int par = 0;
  if constexpr (LOOP) {
    for (int t = blockIdx.x; t < a.T; t += gridDim.x) dispatch_quant_item<MODE>(a, t, red, par);
  } else {
    dispatch_quant_item<MODE>(a, blockIdx.x, red, par);
  }
}

// ---- int8 with per-expert smooth scales [E, H] --------------------------------
// Every copy is quantized with its own expert's scale row, so a token yields up to
// K different code rows.  The scale matrix (E * H * 4 bytes, 7.3 MB at E = 256,
// H = 7168) is larger than one XCD's L2; scale rows are re-read for every copy,
// so where they are served from decides the speed.  Block b handles token b / G
// and only the copies whose expert id e has e % G == b % G; workgroups are placed
// on the 8 XCDs round-robin by block id, so with G = 2 each XCD's L2 sees half of
// the scale rows.  Measured on gfx950 with every input read from HBM: G = 2 is
// best for static codes (109 us against 117 for G = 1, 112 for G = 4 at T=4096,
// H=7168, top-8); with the dynamic scale's block-wide amax per copy, G = 1 is
// (121 against 127 for G = 2) -- splitting a token's copies adds barriers to fewer
// copies per block.  G = 4 and G = 8 lose in both, also when a block requests the token
// row only after it knows it has a copy (G = 8: 175-185 against 134-147 us dynamic): each
// block then has one or two copies and its chain of dependent loads is not hidden.
// Copies are quantized one at a time with the codes kept in registers across the
// block-wide amax, so each scale row is read once per copy.
template <int MODE>
constexpr int expert_groups() { return MODE == 1 ? 2 : 1; }

template <int MODE>
__device__ __forceinline__ void dispatch_quant_expert_item(const DispatchArgs &a, int item, float (*red)[8],
                                                           int &par) {
  constexpr int G = expert_groups<MODE>();
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int t = item / G, grp = item % G;
  const int K = a.K, H = a.H;

  int myrow = -1, myid = 0;
  if (lane < K) {
    myrow = a.dst_row[(size_t)t * K + lane];
    myid = a.topk_idx[(size_t)t * K + lane];
  }
  const QuantLane q(H);  // the row is requested with the slots, before they are known
  const u32x4 *xr = (const u32x4 *)(a.x + (size_t)t * H);
  const u32x4 v0 = xr[q.l0], v1 = xr[q.l1];
  const bool mine = myrow >= 0 && myid % G == grp;  // routed rows have 0 <= id < E
  uint64_t sel = ballot(mine);
  if (sel == 0ull) return;  // same for every wave of the block

  if (wv == 0 && mine && a.expand_w) a.expand_w[myrow] = a.w ? a.w[(size_t)t * K + lane] : 1.0f;
  float f[16];
  unpack8(v0, f);
  unpack8(v1, f + 8);
  while (sel) {
    const int j = __builtin_ctzll(sel);
    sel &= sel - 1;
    const int row = readlane(myrow, j);
    f32x4 s4[4];
    q.load_scales(a.smooth + (size_t)readlane(myid, j) * H, s4);
    float g[16];
    q.scale16(f, s4, g);
    float dyn = 1.0f;
    if constexpr (MODE == 2) {
      float m = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(g[e]));
      m = wave_max(m);
      if (lane == 0) red[par][wv] = m;
      __syncthreads();
      const float amax = block_max_of(red[par], nw);
      par ^= 1;
      dyn = amax > 0.0f ? 127.0f / amax : 0.0f;
      if (threadIdx.x == 0 && a.dyn_scales) a.dyn_scales[row] = amax > 0.0f ? 1.0f / dyn : 0.0f;
    }
    q.store_codes<MODE>(g, dyn, (int8_t *)a.expand_x + (size_t)row * H);
  }
}

// items: T * G (token, expert-id group) pairs; the halves of red[][] alternate per copy, across
// items too (see dispatch_quant_kernel)
template <int MODE, bool LOOP>
__global__ void __launch_bounds__(512) dispatch_quant_expert_kernel(DispatchArgs a, int items) {
  __shared__ float red[2][8];
  int par = 0;
  if constexpr (LOOP) {
    for (int it = blockIdx.x; it < items; it += gridDim.x) dispatch_quant_expert_item<MODE>(a, it, red, par);
  } else {
    dispatch_quant_expert_item<MODE>(a, blockIdx.x, red, par);
  }
}

template <bool LOOP>
static void launch_dispatch_grid(const DispatchArgs &a, int quant_mode, bool per_expert, hipStream_t stream,
                                 int max_wg, bool rows_cached) {
  // grid over `items` work items: one workgroup per item, or at most max_wg (LOOP)
  auto grid = [max_wg](int64_t items) { return dim3((unsigned)(LOOP && items > max_wg ? max_wg : items)); };
  const int nch = a.H / 8;
  if (quant_mode == 0) {
    const int nslice = (nch + 127) / 128;
    const int64_t items = (int64_t)a.T * nslice;
    if (rows_cached)
      hipLaunchKernelGGL((dispatch_copy_kernel<LOOP, true>), grid(items), dim3(64), 0, stream, a, nslice, (int)items);
    else
      hipLaunchKernelGGL((dispatch_copy_kernel<LOOP, false>), grid(items), dim3(64), 0, stream, a, nslice, (int)items);
    return;
  }
  const int pairs = (nch + 1) / 2;  // <= 512 for H <= 8192
  const dim3 blk(64 * ((pairs + 63) / 64));
  const int64_t ie1 = (int64_t)a.T * expert_groups<1>(), ie2 = (int64_t)a.T * expert_groups<2>();
  if (quant_mode == 1 && !per_expert)
    hipLaunchKernelGGL((dispatch_quant_kernel<1, LOOP>), grid(a.T), blk, 0, stream, a);
  else if (quant_mode == 1)
    hipLaunchKernelGGL((dispatch_quant_expert_kernel<1, LOOP>), grid(ie1), blk, 0, stream, a, (int)ie1);
  else if (!per_expert)
    hipLaunchKernelGGL((dispatch_quant_kernel<2, LOOP>), grid(a.T), blk, 0, stream, a);
  else
    hipLaunchKernelGGL((dispatch_quant_expert_kernel<2, LOOP>), grid(ie2), blk, 0, stream, a, (int)ie2);
}

// Static codes (quant_mode 1) from moe_dispatch: a short kernel first reads the token rows in
// address order (into the Infinity Cache), then the dispatch kernel runs with its rows cached.
// The static kernels have no amax barrier, and their row reads from HBM interleave with their
// stores and scale reads; read in one sequential pass first, moe_dispatch measured (T=4096,
// H=7168, top-8, ten rotating sets, same process) 108.3 -> 98.1 us with [E, H] scales and
// 61.1 -> 57.9 us with one [H] vector, at T=2048 58.0 -> 53.6 and 32.3 -> 30.1 us; at T <= 1024
// (x <= 14.7 MB) the extra launch cost more than it saved (12.4 -> 16.0 us at T=1024, [H]), so
// the pass runs only for x of at least 24 MiB.  The dynamic kernels lost with it (120.5 -> 125.4
// and 58.7 -> 59.5 us at T=4096), so they read their rows themselves.  256 workgroups measured
// as 1024.
static constexpr int kPrepassWorkgroups = 256;
static constexpr int64_t kPrepassMinBytes = (int64_t)24 << 20;

__global__ void __launch_bounds__(1024) dispatch_read_ahead_kernel(const void *x, int64_t bytes) {
  read_ahead(x, 0, bytes, blockIdx.x, gridDim.x);
}

static bool use_prepass(int quant_mode, int max_wg, bool rows_cached, int64_t x_bytes) {
  return quant_mode == 1 && !rows_cached && max_wg == 0 && x_bytes >= kPrepassMinBytes;
}

int dispatch_launch_count(int quant_mode, int max_wg, bool rows_cached, int64_t x_bytes) {
  return use_prepass(quant_mode, max_wg, rows_cached, x_bytes) ? 2 : 1;
}

hipError_t launch_dispatch(const DispatchArgs &a, int quant_mode, bool per_expert, hipStream_t stream,
                           int max_wg, bool rows_cached) {
  if (a.T == 0) return hipSuccess;
  const int64_t x_bytes = (int64_t)a.T * a.H * 2;
  if (use_prepass(quant_mode, max_wg, rows_cached, x_bytes))
    hipLaunchKernelGGL(dispatch_read_ahead_kernel, dim3(kPrepassWorkgroups), dim3(1024), 0, stream,
                       (const void *)a.x, x_bytes);
  if (max_wg > 0)
    launch_dispatch_grid<true>(a, quant_mode, per_expert, stream, max_wg, rows_cached);
  else
    launch_dispatch_grid<false>(a, quant_mode, per_expert, stream, 0, rows_cached);
  return hipGetLastError();
}

}  // namespace moe
