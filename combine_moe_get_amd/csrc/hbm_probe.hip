// hbm_probe.hip -- write-pattern probes for the roofline of the dispatch (libmoe_hbm_probe.so,
// loaded by the benchmark only; the dispatch / combine library does not use it).
//
// The dispatch writes every routed copy of a token into a receive row somewhere in an
// expert-major buffer: rows land at scattered places.  These kernels store the same bytes with
// no reads and no arithmetic, (a) at the rows a layout's dst_row map names, in the launch shape
// of the int8 dispatch (one workgroup per token, one lane per 16 bytes of the row, every copy
// stored by all lanes), and (b) in address order (one workgroup per run of 8 consecutive rows),
// so the benchmark can report what HBM accepts for each pattern next to the dispatch itself.
// Stores are non-temporal, as the int8 dispatch's.
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

// one workgroup per run of 8 consecutive rows, stored in address order
__global__ void __launch_bounds__(1024) probe_ordered_kernel(int64_t nrows, int row_bytes, unsigned char *buf) {
  const int64_t r0 = (int64_t)blockIdx.x * 8;
  const int p = threadIdx.x;
  const bool on = 16 * p < row_bytes;
  const u32x4 v = u32x4{(unsigned)blockIdx.x, (unsigned)p, 0x5a5a5a5au, 0xa5a5a5a5u};
  for (int j = 0; j < 8; ++j) {
    const int64_t r = r0 + j;
    if (r < nrows && on) __builtin_nontemporal_store(v, (u32x4 *)(buf + (size_t)r * row_bytes + 16 * p));
  }
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
  const int64_t blocks = (nrows + 7) / 8;
  if (blocks > 0x7fffffff) return -1;
  hipLaunchKernelGGL(probe_ordered_kernel, dim3((unsigned)blocks), dim3(block_for(row_bytes)), 0,
                     (hipStream_t)stream, nrows, row_bytes, (unsigned char *)buf);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
