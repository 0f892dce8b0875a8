// combine.hip -- top-k weighted gather-reduce back to token order, with the
// zero, copy and constant special experts.
//
// out[t] = bf16( sum_j w[t,j] * Moe_j(t) ), fp32 accumulation in slot order;
// Moe_j is the expert-output row dst_row[t,j] for a routed slot, 0 for a zero
// expert, ori_x[t] for a copy expert and alpha1[c] * ori_x[t] + alpha2[c] * v[c]
// for a constant expert (CANN "low_latency_dispatch", Function / Formula,
// special expert scenario; the partner low_latency_combine takes topk_weights,
// ori_x and the alpha / v tensors, Example section).
//
// One wave per (token, 2 KB slice of the row): measured on gfx950, many small
// waves keep more reads in flight than one wave walking a whole token.  The
// slot descriptors (kind, row, weight) are read by lanes 0..K-1 and broadcast
// to scalar registers, so the slot loop is uniform; a lane issues the 16-byte
// loads of both its chunks for every routed slot before the first FMA.  One
// exception: rows of 7 slices (6144 < H <= 7168) with many tokens, no mask and
// no special experts run one wave per whole token that writes its row last
// (combine_row_kernel), which measured faster there and only there.  moe_combine_capped
// runs the slice kernel on at most max_workgroups workgroups that walk the same items
// with a grid stride (same per-item code, identical results).
#include "moe_internal.hpp"

namespace moe {

enum : int { SK_NONE = 0, SK_ROUTED = 1, SK_COPY = 2, SK_CONST = 3 };

__device__ __forceinline__ void fma8(float w, const u32x4 &y, float *acc) {
  acc[0] = __builtin_fmaf(w, bf16_lo(y.x), acc[0]);
  acc[1] = __builtin_fmaf(w, bf16_hi(y.x), acc[1]);
  acc[2] = __builtin_fmaf(w, bf16_lo(y.y), acc[2]);
  acc[3] = __builtin_fmaf(w, bf16_hi(y.y), acc[3]);
  acc[4] = __builtin_fmaf(w, bf16_lo(y.z), acc[4]);
  acc[5] = __builtin_fmaf(w, bf16_hi(y.z), acc[5]);
  acc[6] = __builtin_fmaf(w, bf16_lo(y.w), acc[6]);
  acc[7] = __builtin_fmaf(w, bf16_hi(y.w), acc[7]);
}

__device__ __forceinline__ float bf16_at(const u32x4 &v, int e) {
  const uint32_t u = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return (e & 1) ? bf16_hi(u) : bf16_lo(u);
}

// wave gw = (token, slice); slice sl covers the 16-byte chunks [128 sl, 128 sl + 128) of
// the row: lane l handles chunks 128 sl + l and 128 sl + 64 + l.  All K * 2 routed
// loads of a lane are issued before its first FMA.
//
// One wave per workgroup: measured on gfx950 at T=4096, H=7168, top-8 with every input read from
// HBM, 89.5 us against 91 us for four waves per workgroup (and 91 / 91 us for two / eight).
template <int KMAX, bool SPECIAL>
__device__ __forceinline__ void combine_item(const CombineArgs &a, int nslice, int gw) {
  constexpr int U = 2;
  const int lane = threadIdx.x;
  const int t = gw / nslice, sl = gw - t * nslice;
  if (t >= a.T) return;  // whole wave
  const int H = a.H, K = a.K;
  const int nch = H >> 3;
  const int cb = sl * 64 * U + lane;
  u32x4 *o = (u32x4 *)(a.out + (size_t)t * H);

  // the token's mask byte and its slots' ids, weights and rows are requested together, so
  // the wave waits out one load latency before its row loads, not three
  const bool active = !a.mask || a.mask[t];
  int id = -1, row = -1;
  float wt = 0.0f;
  if (lane < K) {
    id = a.topk_idx[(size_t)t * K + lane];
    wt = a.w[(size_t)t * K + lane];
    row = a.dst_row[(size_t)t * K + lane];
  }
  if (!active) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (cb + 64 * u < nch) __builtin_nontemporal_store((u32x4{0u, 0u, 0u, 0u}), o + cb + 64 * u);
    return;
  }

  int kind = SK_NONE, ci = 0;
  if (lane < K) {
    const int zc = a.E + a.Z;
    if (id >= 0 && id < a.E) {
      kind = row >= 0 ? SK_ROUTED : SK_NONE;
    } else if (SPECIAL && id >= zc && id < zc + a.C) {
      kind = SK_COPY;
    } else if (SPECIAL && id >= zc + a.C && id < zc + a.C + a.Kc) {
      kind = SK_CONST;
      ci = id - zc - a.C;
    }
  }
  const bool need_ori = SPECIAL && ballot(kind == SK_COPY || kind == SK_CONST) != 0ull;

  int skind[KMAX], srow[KMAX], sci[KMAX];
  float sw[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    skind[j] = readlane(kind, j);
    srow[j] = readlane(row, j);
    sci[j] = readlane(ci, j);
    sw[j] = readlane_f(wt, j);
  }

  const u32x4 *ybase = (const u32x4 *)a.y;
  const size_t rstride = (size_t)nch;  // row stride in 16-byte chunks
  const u32x4 *orow = (const u32x4 *)(a.ori_x + (size_t)t * H);

  u32x4 yv[U][KMAX];
  u32x4 ov[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = cb + 64 * u;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      yv[u][j] = u32x4{0u, 0u, 0u, 0u};
      if (skind[j] == SK_ROUTED && c < nch)
        yv[u][j] = __builtin_nontemporal_load(ybase + (size_t)srow[j] * rstride + c);
    }
    ov[u] = u32x4{0u, 0u, 0u, 0u};
    if (need_ori && c < nch) ov[u] = orow[c];
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = cb + 64 * u;
    if (c >= nch) continue;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (skind[j] == SK_ROUTED) {
        fma8(sw[j], yv[u][j], acc);
      } else if (SPECIAL && skind[j] == SK_COPY) {
        fma8(sw[j], ov[u], acc);
      } else if (SPECIAL && skind[j] == SK_CONST) {
        const size_t off = (size_t)sci[j] * H + (size_t)c * 8;
        const u32x4 a1 = *(const u32x4 *)(a.a1 + off);
        const u32x4 a2 = *(const u32x4 *)(a.a2 + off);
        const u32x4 cv = *(const u32x4 *)(a.cv + off);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float y = __builtin_fmaf(bf16_at(a1, e), bf16_at(ov[u], e), bf16_at(a2, e) * bf16_at(cv, e));
          acc[e] = __builtin_fmaf(sw[j], y, acc[e]);
        }
      }
    }
    const u32x4 r = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                          pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
    __builtin_nontemporal_store(r, o + c);
  }
}

// items: T * nslice (token, slice) pairs.  LOOP: a capped grid walks them with a grid stride;
// otherwise one workgroup per item (the loop costs registers: 76 -> 82 at top-8, one wave per
// SIMD less)
template <int KMAX, bool SPECIAL, bool LOOP>
__global__ void __launch_bounds__(64) combine_kernel(CombineArgs a, int nslice, int items) {
  if constexpr (LOOP) {
    for (int gw = blockIdx.x; gw < items; gw += gridDim.x) combine_item<KMAX, SPECIAL>(a, nslice, gw);
  } else {
    combine_item<KMAX, SPECIAL>(a, nslice, blockIdx.x);
  }
}

// Routed slots only, rows of NS 2 KB slices: one wave per whole token, its output row kept in
// registers and written after all of the token's reads.  The waves resident together then read
// first and write together, instead of every wave writing 2 KB between other waves' reads.
// Measured on gfx950 at T=4096, H=7168 (NS = 7), top-8 with every input read from HBM: 87.0-87.6
// against 89.9 us for the slice kernel; at other row sizes or with a run-time slice count it was
// slower (e.g. 126 against 103 us at H=4096), below T ~ 2048 one wave per token leaves the chip
// idle, and with an active-token mask (10% of tokens masked) it lost (88.3 against 84.5 us at
// T=4096; 351 against 338 us at T=16384) -- so it is used for NS = 7, large T and no mask only.
// Arithmetic per element is the slice kernel's (same slot order, same fma chain), so the
// results are bit-identical.
template <int KMAX, int NS>
__device__ __forceinline__ void combine_row_item(const CombineArgs &a, int t) {
  const int lane = threadIdx.x;
  if (t >= a.T) return;  // whole wave
  const int H = a.H, K = a.K;
  const int nch = H >> 3;
  u32x4 *o = (u32x4 *)(a.out + (size_t)t * H);

  const bool active = !a.mask || a.mask[t];
  int id = -1, row = -1;
  float wt = 0.0f;
  if (lane < K) {
    id = a.topk_idx[(size_t)t * K + lane];
    wt = a.w[(size_t)t * K + lane];
    row = a.dst_row[(size_t)t * K + lane];
  }
  const bool routed = active && id >= 0 && id < a.E && row >= 0;  // a masked token adds nothing: +0
  int srow[KMAX];
  float sw[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    srow[j] = readlane(routed ? row : -1, j);
    sw[j] = readlane_f(wt, j);
  }

  const u32x4 *ybase = (const u32x4 *)a.y;
  u32x4 outv[2 * NS];
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) {
    u32x4 yv[2][KMAX];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = sl * 128 + 64 * u + lane;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        yv[u][j] = u32x4{0u, 0u, 0u, 0u};
        if (srow[j] >= 0 && c < nch) yv[u][j] = __builtin_nontemporal_load(ybase + (size_t)srow[j] * nch + c);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (srow[j] >= 0) fma8(sw[j], yv[u][j], acc);
      outv[2 * sl + u] = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                               pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
    }
  }
#pragma unroll
  for (int i = 0; i < 2 * NS; ++i) {
    const int c = i * 64 + lane;
    if (c < nch) __builtin_nontemporal_store(outv[i], o + c);
  }
}

// one wave per token (uncapped launches only)
template <int KMAX, int NS>
__global__ void __launch_bounds__(64) combine_row_kernel(CombineArgs a) {
  combine_row_item<KMAX, NS>(a, blockIdx.x);
}

template <int KMAX>
static void launch_k(const CombineArgs &a, hipStream_t st, int max_wg) {
  const int nch = a.H / 8;
  const int nslice = (nch + 127) / 128;
  const int64_t items = (int64_t)a.T * nslice;
  if (max_wg > 0) {  // capped grid: the slice kernel walking its items
    const dim3 g((unsigned)(items > max_wg ? max_wg : items));
    if (a.C + a.Kc > 0)
      hipLaunchKernelGGL((combine_kernel<KMAX, true, true>), g, dim3(64), 0, st, a, nslice, (int)items);
    else
      hipLaunchKernelGGL((combine_kernel<KMAX, false, true>), g, dim3(64), 0, st, a, nslice, (int)items);
    return;
  }
  const dim3 g((unsigned)items);
  if (a.C + a.Kc > 0)
    hipLaunchKernelGGL((combine_kernel<KMAX, true, false>), g, dim3(64), 0, st, a, nslice, (int)items);
  else if (KMAX == 8 && nslice == 7 && a.T >= 2048 && !a.mask)  // see combine_row_kernel
    hipLaunchKernelGGL((combine_row_kernel<8, 7>), dim3((unsigned)a.T), dim3(64), 0, st, a);
  else  // no copy / constant ids can occur: the routed-only kernel needs fewer registers
    hipLaunchKernelGGL((combine_kernel<KMAX, false, false>), g, dim3(64), 0, st, a, nslice, (int)items);
}

// max_wg > 0 caps the grid (the kernels then walk their items with a grid stride); a capped
// launch keeps the slice kernel, whose small waves spread a bounded grid over more of the row
hipError_t launch_combine(const CombineArgs &a, hipStream_t stream, int max_wg) {
  if (a.T == 0) return hipSuccess;
  if (a.K <= 1) launch_k<1>(a, stream, max_wg);
  else if (a.K <= 2) launch_k<2>(a, stream, max_wg);
  else if (a.K <= 4) launch_k<4>(a, stream, max_wg);
  else if (a.K <= 8) launch_k<8>(a, stream, max_wg);
  else launch_k<16>(a, stream, max_wg);
  return hipGetLastError();
}

}  // namespace moe
