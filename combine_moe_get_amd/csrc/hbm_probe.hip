// hbm_probe.hip -- access-pattern probes for the rooflines of the dispatch and the combine
// (libmoe_hbm_probe.so, loaded by the benchmark only; the dispatch / combine library does not use it).
//
// The dispatch writes every routed copy of a token into a receive row somewhere in an
// expert-major buffer: rows land at scattered places.  These kernels store the same bytes with
// no reads and no arithmetic, (a) at the rows a layout's dst_row map names, in the launch shape
// of the int8 dispatch (one workgroup per token, one lane per 16 bytes of the row, every copy
// stored by all lanes), and (b) in address order (one workgroup per row, in row order),
// so the benchmark can report what HBM accepts for each pattern next to the dispatch itself.
// Stores are non-temporal, as the int8 dispatch's.  The gather probe is the combine's read side
// alone: the same rows read in the combine's launch shape, with no output rows written; the
// reduce probe is the combine's reads and writes with XOR in place of its arithmetic, on the
// combine's row map or on rows in address order.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// one workgroup per token; thread p stores 16 bytes at offset 16 p of each of the token's rows
__global__ void __launch_bounds__(1024) probe_scatter_kernel(const int32_t *dst_row, int K, int row_bytes,
                                                            unsigned char *buf) {
  const int t = blockIdx.x;
  const int p = threadIdx.x;
  const bool on = 16 * p < row_bytes;
  const u32x4 v = u32x4{(unsigned)t, (unsigned)p, 0x5a5a5a5au, 0xa5a5a5a5u};
  for (int j = 0; j < K; ++j) {
    const int r = dst_row[(size_t)t * K + j];  // uniform across the workgroup
    if (r >= 0 && on) __builtin_nontemporal_store(v, (u32x4 *)(buf + (size_t)r * row_bytes + 16 * p));
  }
}

// one workgroup per row, workgroups in address order (measured on gfx950: one row per workgroup
// writes in address order faster than eight consecutive rows per workgroup, 6.3 against 5.1 TB/s
// for 8 KB rows)
__global__ void __launch_bounds__(1024) probe_ordered_kernel(int64_t nrows, int row_bytes, unsigned char *buf) {
  const int64_t r = blockIdx.x;
  const int p = threadIdx.x;
  const u32x4 v = u32x4{(unsigned)blockIdx.x, (unsigned)p, 0x5a5a5a5au, 0xa5a5a5a5u};
  if (r < nrows && 16 * p < row_bytes) __builtin_nontemporal_store(v, (u32x4 *)(buf + (size_t)r * row_bytes + 16 * p));
}

// reads only: one wave per (token, 2 KB slice of the row), as the combine's slice kernel -- lane l
// loads the 16-byte chunks l and l + 64 of the slice from each of the token's K rows named by
// dst_row (non-temporal loads, all issued before any use) and folds them with XOR; a lane stores
// its 16-byte fold to `sink` only if it equals one fixed 128-bit pattern (never, in practice), so
// the loads cannot be dropped while the stores add no traffic
template <int KMAX>
__global__ void __launch_bounds__(64) probe_gather_kernel(const int32_t *dst_row, int K, int row_bytes,
                                                          const unsigned char *buf, int nslice, u32x4 *sink) {
  const int lane = threadIdx.x;
  const int gw = blockIdx.x;
  const int t = gw / nslice, sl = gw - t * nslice;
  const int nch = row_bytes / 16;
  const int c0 = 128 * sl + lane, c1 = c0 + 64;
  int myrow = -1;
  if (lane < K) myrow = dst_row[(size_t)t * K + lane];
  u32x4 acc = u32x4{0u, 0u, 0u, 0u};
  u32x4 v[2 * KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int r = __builtin_amdgcn_readlane(myrow, j);
    v[2 * j] = v[2 * j + 1] = u32x4{0u, 0u, 0u, 0u};
    if (j < K && r >= 0) {
      const u32x4 *row = (const u32x4 *)(buf + (size_t)r * row_bytes);
      if (c0 < nch) v[2 * j] = __builtin_nontemporal_load(row + c0);
      if (c1 < nch) v[2 * j + 1] = __builtin_nontemporal_load(row + c1);
    }
  }
#pragma unroll
  for (int i = 0; i < 2 * KMAX; ++i) acc ^= v[i];
  if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u && acc.z == 0xf39cc060u && acc.w == 0x5ced2c1du)
    sink[(size_t)gw * 64 + lane] = acc;
}

// the combine's bytes without its arithmetic: one wave per (token, 2 KB slice) as above, the
// token's K rows folded with XOR and the fold stored (non-temporal) to out row t.  GATHER: rows
// dst_row[t, j] (skipped when negative), the combine's pattern; otherwise rows t K + j, every
// row read once in address order and the outputs written in address order.
template <int KMAX, bool GATHER>
__global__ void __launch_bounds__(64) probe_reduce_kernel(const int32_t *dst_row, int K, int row_bytes,
                                                          const unsigned char *buf, int nslice, unsigned char *out) {
  const int lane = threadIdx.x;
  const int gw = blockIdx.x;
  const int t = gw / nslice, sl = gw - t * nslice;
  const int nch = row_bytes / 16;
  const int c0 = 128 * sl + lane, c1 = c0 + 64;
  int myrow = -1;
  if (lane < K) myrow = GATHER ? dst_row[(size_t)t * K + lane] : t * K + lane;
  u32x4 v[2 * KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int r = __builtin_amdgcn_readlane(myrow, j);
    v[2 * j] = v[2 * j + 1] = u32x4{0u, 0u, 0u, 0u};
    if (j < K && r >= 0) {
      const u32x4 *row = (const u32x4 *)(buf + (size_t)r * row_bytes);
      if (c0 < nch) v[2 * j] = __builtin_nontemporal_load(row + c0);
      if (c1 < nch) v[2 * j + 1] = __builtin_nontemporal_load(row + c1);
    }
  }
  u32x4 a0 = u32x4{0u, 0u, 0u, 0u}, a1 = a0;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    a0 ^= v[2 * j];
    a1 ^= v[2 * j + 1];
  }
  u32x4 *o = (u32x4 *)(out + (size_t)t * row_bytes);
  if (c0 < nch) __builtin_nontemporal_store(a0, o + c0);
  if (c1 < nch) __builtin_nontemporal_store(a1, o + c1);
}

int block_for(int row_bytes) { return 64 * ((row_bytes / 16 + 63) / 64); }

}  // namespace

extern "C" {

// Store row_bytes (a multiple of 16, at most 16384) into every row buf[dst_row[t, j]] with
// dst_row[t, j] >= 0, t < T, j < K.  buf must hold max(dst_row) + 1 rows; 16-byte aligned.
// Returns 0, or -1 for bad arguments, -5 when the launch fails.
int moe_probe_scatter_write(const int32_t *dst_row, int T, int K, int row_bytes, void *buf, void *stream) {
  if (T < 0 || K <= 0 || K > 16 || row_bytes <= 0 || row_bytes % 16 || row_bytes > 16384 || !buf ||
      (T > 0 && !dst_row))
    return -1;
  if (((uintptr_t)buf & 15u) != 0) return -1;
  if (T == 0) return 0;
  hipLaunchKernelGGL(probe_scatter_kernel, dim3((unsigned)T), dim3(block_for(row_bytes)), 0, (hipStream_t)stream,
                     dst_row, K, row_bytes, (unsigned char *)buf);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Store row_bytes into rows [0, nrows) of buf in address order.  Same rules as above.
int moe_probe_ordered_write(int64_t nrows, int row_bytes, void *buf, void *stream) {
  if (nrows < 0 || row_bytes <= 0 || row_bytes % 16 || row_bytes > 16384 || !buf) return -1;
  if (((uintptr_t)buf & 15u) != 0) return -1;
  if (nrows == 0) return 0;
  const int64_t blocks = nrows;
  if (blocks > 0x7fffffff) return -1;
  hipLaunchKernelGGL(probe_ordered_kernel, dim3((unsigned)blocks), dim3(block_for(row_bytes)), 0,
                     (hipStream_t)stream, nrows, row_bytes, (unsigned char *)buf);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Read every row buf[dst_row[t, j]] (dst_row[t, j] >= 0) in the combine's launch shape: one wave
// per (token, 2 KB slice), row_bytes a multiple of 16, at most 16384, K at most 16.  sink receives
// T * ceil(row_bytes / 2048) * 64 16-byte words.  Returns 0, or -1 for bad arguments, -5 when the
// launch fails.
int moe_probe_gather_read(const int32_t *dst_row, int T, int K, int row_bytes, const void *buf, void *sink,
                          void *stream) {
  if (T < 0 || K <= 0 || K > 16 || row_bytes <= 0 || row_bytes % 16 || row_bytes > 16384 || !buf || !sink ||
      (T > 0 && !dst_row))
    return -1;
  if ((((uintptr_t)buf | (uintptr_t)sink) & 15u) != 0) return -1;
  if (T == 0) return 0;
  const int nslice = (row_bytes / 16 + 127) / 128;
  const dim3 grid((unsigned)((int64_t)T * nslice));
  if (K <= 8)
    hipLaunchKernelGGL(probe_gather_kernel<8>, grid, dim3(64), 0, (hipStream_t)stream, dst_row, K, row_bytes,
                       (const unsigned char *)buf, nslice, (u32x4 *)sink);
  else
    hipLaunchKernelGGL(probe_gather_kernel<16>, grid, dim3(64), 0, (hipStream_t)stream, dst_row, K, row_bytes,
                       (const unsigned char *)buf, nslice, (u32x4 *)sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// The combine's reads and writes without its arithmetic (probe_reduce_kernel): out row t (T rows
// of row_bytes) = XOR of the token's K rows of buf.  gather != 0: rows dst_row[t, j] (negative
// entries skipped; buf holds max(dst_row) + 1 rows); gather == 0: rows t K + j (buf holds T K
// rows, dst_row unused).  row_bytes a multiple of 16, at most 16384; K at most 16; buf and out
// 16-byte aligned.  Returns 0, or -1 for bad arguments, -5 when the launch fails.
int moe_probe_reduce(const int32_t *dst_row, int T, int K, int row_bytes, const void *buf, void *out, int gather,
                     void *stream) {
  if (T < 0 || K <= 0 || K > 16 || row_bytes <= 0 || row_bytes % 16 || row_bytes > 16384 || !buf || !out ||
      (T > 0 && gather && !dst_row) || (int64_t)T * K > 0x7fffffff)
    return -1;
  if ((((uintptr_t)buf | (uintptr_t)out) & 15u) != 0) return -1;
  if (T == 0) return 0;
  const int nslice = (row_bytes / 16 + 127) / 128;
  const dim3 grid((unsigned)((int64_t)T * nslice));
  const hipStream_t st = (hipStream_t)stream;
  const unsigned char *b = (const unsigned char *)buf;
  unsigned char *o = (unsigned char *)out;
  if (K <= 8) {
    if (gather)
      hipLaunchKernelGGL((probe_reduce_kernel<8, true>), grid, dim3(64), 0, st, dst_row, K, row_bytes, b, nslice, o);
    else
      hipLaunchKernelGGL((probe_reduce_kernel<8, false>), grid, dim3(64), 0, st, dst_row, K, row_bytes, b, nslice, o);
  } else {
    if (gather)
      hipLaunchKernelGGL((probe_reduce_kernel<16, true>), grid, dim3(64), 0, st, dst_row, K, row_bytes, b, nslice, o);
    else
      hipLaunchKernelGGL((probe_reduce_kernel<16, false>), grid, dim3(64), 0, st, dst_row, K, row_bytes, b, nslice, o);
  }
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
