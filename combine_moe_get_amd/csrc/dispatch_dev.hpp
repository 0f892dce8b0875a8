// dispatch_dev.hpp -- device code of the int8 / bf16 dispatch shared by the
// dispatch kernels (dispatch.hip) and the single-launch layout + dispatch
// kernel (layout.hip).  What is computed: CANN "low_latency_dispatch",
// Function / Formula, dynamic quantization scenario (see dispatch.hip).
#pragma once

#include "moe_internal.hpp"

namespace moe {

__device__ __forceinline__ int sat_code(float p) {
  float r = __builtin_rintf(p);  // round half to even
  if (r != r) return 0;          // NaN (0 * inf): code 0
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

__device__ __forceinline__ uint32_t pack_i8x4(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
         ((uint32_t)(d & 0xff) << 24);
}

__device__ __forceinline__ void unpack8(const u32x4 &v, float *f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// Lane p = threadIdx.x of a workgroup quantizing one row owns channels
// [16p, 16p + 16) (chunks 2p and 2p + 1); needs blockDim.x >= ceil(H / 16).
struct QuantLane {
  int p, l0, l1;
  bool has0, has1, wide;
  __device__ QuantLane(int H) {
    const int nch = H >> 3;
    p = threadIdx.x;
    has0 = 2 * p < nch;
    has1 = 2 * p + 1 < nch;
    l0 = has0 ? 2 * p : 0;  // in-bounds chunks for lanes past the row end
    l1 = has1 ? 2 * p + 1 : 0;
    wide = (H & 15) == 0;  // 16-byte code stores stay aligned
  }
  __device__ void load_scales(const float *s, f32x4 *s4) const {
    const f32x4 *sp = (const f32x4 *)s;
    s4[0] = sp[2 * l0];
    s4[1] = sp[2 * l0 + 1];
    s4[2] = sp[2 * l1];
    s4[3] = sp[2 * l1 + 1];
  }
  // g = fp32(x) * scales, zero on channels past the row end
  __device__ void scale16(const float *f, const f32x4 *s4, float *g) const {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const f32x4 &sv = s4[e >> 2];
      const float sc = (e & 3) == 0 ? sv.x : (e & 3) == 1 ? sv.y : (e & 3) == 2 ? sv.z : sv.w;
      g[e] = ((e < 8) ? has0 : has1) ? f[e] * sc : 0.0f;
    }
  }
  template <int MODE>
  __device__ void store_codes(const float *g, float dyn, int8_t *row_base) const {
    int cd[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) cd[e] = sat_code(MODE == 2 ? g[e] * dyn : g[e]);
    const u32x2 lo = u32x2{pack_i8x4(cd[0], cd[1], cd[2], cd[3]), pack_i8x4(cd[4], cd[5], cd[6], cd[7])};
    const u32x2 hi = u32x2{pack_i8x4(cd[8], cd[9], cd[10], cd[11]), pack_i8x4(cd[12], cd[13], cd[14], cd[15])};
    int8_t *dst = row_base + (size_t)p * 16;
    if (wide && has1) {
      __builtin_nontemporal_store((u32x4{lo.x, lo.y, hi.x, hi.y}), (u32x4 *)dst);
    } else {
      if (has0) __builtin_nontemporal_store(lo, (u32x2 *)dst);
      if (has1) __builtin_nontemporal_store(hi, (u32x2 *)(dst + 8));
    }
  }
};

// max over the block of the per-wave maxima in red[0..nw)
__device__ __forceinline__ float block_max_of(const float *red, int nw) {
  float m = red[0];
  for (int w = 1; w < nw; ++w) m = fmaxf(m, red[w]);
  return m;
}

__device__ __forceinline__ float max_abs16(const float *g) {
  float m = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(g[e]));
  return m;
}

// max over the workgroup of m; red[2][16] in LDS alternates between calls (par), so
// one barrier per call suffices.  Every thread of the block must call it.
__device__ __forceinline__ float block_amax(float m, float (*red)[16], int &par) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  m = wave_max(m);
  if (lane == 0) red[par][wv] = m;
  __syncthreads();
  m = block_max_of(red[par], (int)(blockDim.x >> 6));
  par ^= 1;
  return m;
}

// The first loads of a token's dispatch, issued early (before the layout phase of the
// single-launch kernel) so their latency overlaps other work: the row chunks a thread
// needs and, for one smooth vector, its scales.
struct TokenPrefetch {
  u32x4 v0, v1;
  f32x4 s4[4];
};

template <int MODE, bool PE>
__device__ __forceinline__ void dispatch_prefetch(const DispatchArgs &a, int t, TokenPrefetch &pf) {
  const u32x4 *xr = (const u32x4 *)(a.x + (size_t)t * a.H);
  if constexpr (MODE == 0) {  // chunks tid and tid + blockDim.x (nch <= 1024 <= 2 blockDim.x)
    const int nch = a.H >> 3, c0 = threadIdx.x, c1 = threadIdx.x + blockDim.x;
    pf.v0 = c0 < nch ? xr[c0] : u32x4{0u, 0u, 0u, 0u};
    pf.v1 = c1 < nch ? xr[c1] : u32x4{0u, 0u, 0u, 0u};
  } else {
    const QuantLane q(a.H);
    pf.v0 = xr[q.l0];
    pf.v1 = xr[q.l1];
#pragma unroll
    for (int i = 0; i < 4; ++i) pf.s4[i] = f32x4{1.f, 1.f, 1.f, 1.f};
    if (!PE && a.smooth) q.load_scales(a.smooth, pf.s4);
  }
}

// Dispatch of token t by a whole workgroup (blockDim.x >= ceil(H / 16), every thread
// calls it with the same arguments, so barriers match).  rows[j] / ids[j], j < K: the
// receive row (or -1) and expert id of each slot, in memory every thread can read.
// MODE 0: bf16 copy; 1: static int8; 2: dynamic int8.  PE: per-expert scales [E, H].
// With use_pf the row chunks (and shared scales) come from dispatch_prefetch of token t.
template <int MODE, bool PE>
__device__ __forceinline__ void dispatch_token_block(const DispatchArgs &a, int t, const int *rows,
                                                     const int *ids, float (*red)[16], int &par,
                                                     const TokenPrefetch &pf, bool use_pf) {
  const int tid = threadIdx.x;
  const int K = a.K, H = a.H;
  bool any = false;  // the same in every thread: rows[] is shared
  for (int j = 0; j < K; ++j) any = any || rows[j] >= 0;
  if (!any) return;  // masked token, or only special / dropped slots
  if (tid < K && rows[tid] >= 0 && a.expand_w) a.expand_w[rows[tid]] = a.w ? a.w[(size_t)t * K + tid] : 1.0f;
  if constexpr (MODE == 0) {
    const int nch = H >> 3;
    const u32x4 *xr = (const u32x4 *)(a.x + (size_t)t * H);
    for (int it = 0, c = tid; c < nch; ++it, c += blockDim.x) {
      const u32x4 v = (use_pf && it == 0) ? pf.v0 : (use_pf && it == 1) ? pf.v1 : xr[c];
      for (int j = 0; j < K; ++j) {
        const int r = rows[j];
        if (r >= 0) __builtin_nontemporal_store(v, (u32x4 *)((uint16_t *)a.expand_x + (size_t)r * H) + c);
      }
    }
  } else {
    const QuantLane q(H);
    TokenPrefetch p;
    if (use_pf)
      p = pf;
    else
      dispatch_prefetch<MODE, PE>(a, t, p);
    float f[16];
    unpack8(p.v0, f);
    unpack8(p.v1, f + 8);
    if constexpr (!PE) {
      float g[16];
      q.scale16(f, p.s4, g);
      float dyn = 1.0f;
      if constexpr (MODE == 2) {
        const float amax = block_amax(max_abs16(g), red, par);
        dyn = amax > 0.0f ? 127.0f / amax : 0.0f;
        if (tid < K && rows[tid] >= 0 && a.dyn_scales) a.dyn_scales[rows[tid]] = amax > 0.0f ? 1.0f / dyn : 0.0f;
      }
      for (int j = 0; j < K; ++j) {
        const int r = rows[j];
        if (r >= 0) q.store_codes<MODE>(g, dyn, (int8_t *)a.expand_x + (size_t)r * H);
      }
    } else {
      for (int j = 0; j < K; ++j) {
        const int r = rows[j];
        if (r < 0) continue;
        f32x4 s4[4];
        q.load_scales(a.smooth + (size_t)ids[j] * H, s4);
        float g[16];
        q.scale16(f, s4, g);
        float dyn = 1.0f;
        if constexpr (MODE == 2) {
          const float amax = block_amax(max_abs16(g), red, par);
          dyn = amax > 0.0f ? 127.0f / amax : 0.0f;
          if (tid == 0 && a.dyn_scales) a.dyn_scales[r] = amax > 0.0f ? 1.0f / dyn : 0.0f;
        }
        q.store_codes<MODE>(g, dyn, (int8_t *)a.expand_x + (size_t)r * H);
      }
    }
  }
}

}  // namespace moe
