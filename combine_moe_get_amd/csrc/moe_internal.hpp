// moe_internal.hpp -- device helpers, kernel argument blocks and launcher
// declarations shared by the HIP translation units of libmoe_get.
// gfx950 (CDNA4) only: wave64, 16-byte global accesses, LDS for counters.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_get.h"

namespace moe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---- wave64 helpers -------------------------------------------------------

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

__device__ __forceinline__ int lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// number of set bits of m in lanes below the calling lane
__device__ __forceinline__ int popc_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ int readlane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// wave-wide max over the 64 lanes, returned to every lane.  A running max with DPP moves:
// shifts by 1, 2, 4, 8 lanes inside each row of 16 leave the row's max in its lane 15; lane 15
// of rows 0 / 2 is folded into rows 1 / 3 and lane 31 into rows 2 / 3, so lane 63 holds the max
// of all lanes, which readlane broadcasts.  A lane whose DPP source lies outside its row, or whose
// row is masked off, keeps its own value (the `old` operand).  max is exact, so the order of the
// folds does not matter; inputs are finite.  Every lane of the wave must call it.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_fold_max(float v) {
  const int b = __float_as_int(v);
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(b, b, CTRL, ROW_MASK, 0xf, false)));
}
__device__ __forceinline__ float wave_max(float v) {
  v = dpp_fold_max<0x111, 0xf>(v);  // row_shr:1
  v = dpp_fold_max<0x112, 0xf>(v);  // row_shr:2
  v = dpp_fold_max<0x114, 0xf>(v);  // row_shr:4
  v = dpp_fold_max<0x118, 0xf>(v);  // row_shr:8
  v = dpp_fold_max<0x142, 0xa>(v);  // row_bcast:15 -> rows 1, 3
  v = dpp_fold_max<0x143, 0xc>(v);  // row_bcast:31 -> rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// inclusive prefix sum over the 64 lanes with DPP moves (no LDS round trips): shifts by
// 1, 2, 4, 8 lanes inside each row of 16, then lane 15 of rows 0 / 2 into rows 1 / 3 and
// lane 31 into rows 2 and 3.  A lane whose DPP source is outside its row, or whose row is
// masked off, reads the `old` operand, 0.  Every lane of the wave must call it.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

// ---- bf16 <-> fp32 --------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// round to nearest, ties to even (finite values)
__device__ __forceinline__ uint32_t bf16_rne_hi(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (bf16_rne_hi(lo) >> 16) | bf16_rne_hi(hi);
}

// ---- row loads and stores through buffer resources ------------------------------

// 16-byte load at byte offset `off` of a row of `row_bytes` bytes that starts at the wave-uniform
// address `row`, through a buffer resource (32-bit offsets, the base in scalar registers).  The bf16
// dispatch reads its token rows this way: 98.4-99.1 against 99.4-99.5 us for 64-bit global loads in
// the same run (T=4096, H=7168, top-8, ten rotating input sets).  An offset at or past row_bytes
// reads 0.
__device__ __forceinline__ u32x4 row_load(const void *row, int row_bytes, int off) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)row, (short)0, row_bytes, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
}

// 16-byte store at byte offset `off` of a row of `row_bytes` bytes that starts at `row`, a
// wave-uniform address (the buffer resource lives in scalar registers), with the "sc1" cache
// policy and no "nt" hint.  Used for the bf16 receive rows: measured on gfx950 at T=4096,
// H=7168, top-8 with ten rotating input and output sets (no reuse through the 256 MB
// Infinity Cache), 104 -> 101.5 us against non-temporal stores.  The int8 dispatch (57.9 ->
// 60.5 us) and the combine's output rows (90.2 -> 91.5 us) measured slower with it and keep
// non-temporal stores; with only four output sets (235 MB, which the Infinity Cache holds)
// the combine had looked faster with it (89.6 -> 88.1 us).  An offset at or past row_bytes
// is dropped by the buffer range check.
__device__ __forceinline__ void row_store_sc1(u32x4 v, void *row, int row_bytes, int off) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(row, (short)0, row_bytes, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, 16 /* sc1 */);
}

// ---- kernel argument blocks -----------------------------------------------

struct LayoutArgs {
  const int32_t *topk_idx;
  const uint8_t *mask;
  int32_t T, K, E, P, BS, L, NS, nbits, Epad, Spad;
  int32_t m, BSv, Svpad;  // two-launch layout: sub-chunks per chunk, tokens per sub-chunk, padded slots
  int64_t Etot;
  int64_t rank_stride;  // 0: compact rows; A > 0: rank r owns rows [r A, r A + A)
  int32_t *cnt, *expert_offsets, *recv_counts, *special_counts, *num_tokens_per_rank,
      *rank_offsets, *dst_row, *src_info;
  uint8_t *itr;
  uint32_t *status;
  int32_t *ws_cnt_t;     // [P m][E]  routed copies of expert e sent by sub-chunk v
  int32_t *ws_rank_tok;  // [P m][P]  per sub-chunk: tokens with a copy on rank r
  int32_t *ws_special;   // [P m][NS] per sub-chunk: special slots per id
  int32_t mt;            // 64-bit words per wave of the count kernel's LDS match tables; set by the launcher
  uint32_t divL, divK, divBSv, divE;  // div_magic of L, K, BSv and E: see fast_div
  // read-ahead of the dispatch's token rows (layout + dispatch in one call): pf_wgs extra
  // workgroups of the count kernel read bytes [0, pf_half) of pf, as many of the scan kernel
  // [pf_half, pf_bytes), so the rows sit in the Infinity Cache when the dispatch reads them.
  // pf_wgs = 0: no extra workgroups.
  const void *pf;
  int64_t pf_half, pf_bytes;
  int32_t pf_wgs;
};

// Read bytes [lo, hi) of buf (16-byte aligned, hi - lo a multiple of 16) with ordinary loads,
// workgroup wg of nwg, eight 16-byte loads per thread in flight: the lines are left in the caches
// for a later kernel.  Nothing is stored; an empty asm statement consumes the loaded values so
// the loads are kept.
__device__ __forceinline__ void read_ahead(const void *buf, int64_t lo, int64_t hi, int wg, int nwg) {
  const u32x4 *p = (const u32x4 *)((const unsigned char *)buf + lo);
  const int64_t n = (hi - lo) >> 4;
  const int64_t step = (int64_t)nwg * blockDim.x;
  u32x4 acc = u32x4{0u, 0u, 0u, 0u};
  for (int64_t i = (int64_t)wg * blockDim.x + threadIdx.x; i < n; i += 8 * step) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t j = i + u * step;
      v[u] = j < n ? p[j] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  asm volatile("" ::"v"(acc.x), "v"(acc.y), "v"(acc.z), "v"(acc.w));
}

// Division by a divisor d fixed for the whole call, as a multiply-high: m = div_magic(d) =
// ceil(2^32 / d) (0 for d = 1) and n / d = umulhi(n, m) for 0 <= n with n d < 2^32 (then
// n m / 2^32 lies in [n / d, n / d + n / 2^32) and n / 2^32 < 1 / d, so the floor is exact).
// Every use here divides a lane, an expert id, a slot of a (sub-)chunk or a token of a chunk
// (all below 2^13) by L, K, E or a sub-chunk size (all at most 2^11).
inline uint32_t div_magic(int d) { return d > 1 ? (uint32_t)(((1ull << 32) + (uint64_t)d - 1) / (uint64_t)d) : 0u; }
__device__ __forceinline__ int fast_div(int n, uint32_t m) { return m ? (int)__umulhi((uint32_t)n, m) : n; }

struct DispatchArgs {
  const uint16_t *x;
  const float *smooth;
  const float *w;
  const int32_t *topk_idx;
  const int32_t *dst_row;
  void *expand_x;
  float *dyn_scales;
  float *expand_w;
  int32_t T, H, K;
};

struct CombineArgs {
  const uint16_t *y;
  const int32_t *topk_idx;
  const float *w;
  const uint8_t *mask;
  const int32_t *dst_row;
  const uint16_t *ori_x, *a1, *a2, *cv;
  uint16_t *out;
  int32_t T, H, K, E, Z, C, Kc;
};

// Sub-chunks per source rank in the two-launch layout: a chunk of more than 128 tokens is
// counted by up to 4 workgroups, as long as the count matrix keeps at most 64 rows (every
// workgroup of the scan kernel sums all of them) and m E <= 4096 (the scan kernel's LDS).
inline int layout_subchunks(int BS, int E, int P) {
  int m = (BS + 127) / 128;
  if (m > 4) m = 4;
  while (m > 1 && (m * E > 4096 || m * P > 64)) --m;
  return m < 1 ? 1 : m;
}

// ---- launchers (return hipSuccess or the launch error) ---------------------

hipError_t launch_layout(const LayoutArgs &a, hipStream_t stream);
int layout_launch_count(const LayoutArgs &a);  // kernels launch_layout runs for these sizes
// layout and dispatch of the same call (one kernel for small worlds, else the two paths in turn)
hipError_t launch_layout_dispatch(const LayoutArgs &a, const DispatchArgs &d, int quant_mode, bool per_expert,
                                  hipStream_t stream);
int layout_dispatch_launch_count(const LayoutArgs &a, int quant_mode, int64_t x_bytes);
// kernels launch_dispatch runs (uncapped when max_wg == 0) for T > 0
int dispatch_launch_count(int quant_mode, int max_wg, bool rows_cached, int64_t x_bytes);
// max_wg > 0: launch at most that many workgroups, each walking several work items (a capped
// grid, which leaves the rest of the GPU to kernels running beside it); 0: one per item.
// rows_cached: the token rows were just read ahead into the caches (the bf16 copy then stores
// non-temporally)
hipError_t launch_dispatch(const DispatchArgs &a, int quant_mode, bool per_expert, hipStream_t stream,
                           int max_wg = 0, bool rows_cached = false);
hipError_t launch_combine(const CombineArgs &a, hipStream_t stream, int max_wg = 0);

// LDS bytes of the layout count kernel and its waves per block
int layout_waves(int E);
size_t layout_lds_bytes(int waves, int Epad, int Spad, int P, int NS, int BS, int mt);

}  // namespace moe
