/*
 * moe_client.c -- a plain C caller of libmoe_get: no Python, no PyTorch.
 *
 * usage: moe_client DIR
 *
 * DIR/shape.txt holds twelve to fourteen integers: T H K E P Z C Kc num_max
 * quant_mode has_mask smooth_rows [path [max_workgroups]].  The inputs are raw little-endian files in DIR:
 * topk_idx.bin (int32 [T,K]), x.bin (bf16 [T,H]), w.bin (fp32 [T,K]),
 * y.bin (bf16 [rows,H], the expert outputs the combine reads), mask.bin (u8 [T],
 * when has_mask), smooth.bin (fp32 [smooth_rows,H], when smooth_rows > 0) and,
 * when Kc > 0, a1.bin, a2.bin, cv.bin (bf16 [Kc,H]).  The client allocates
 * device memory with the HIP runtime, runs moe_get_layout, moe_dispatch and
 * moe_combine through the C ABI of moe_get.h on the null stream (path 1:
 * moe_layout_dispatch in place of the first two; path 2: moe_get_layout_noalloc,
 * moe_dispatch_capped and moe_combine_capped on max_workgroups workgroups, with no
 * workspace allocated), and writes every output next to the inputs (out_*.bin).
 * Exit status 0 on success.
 */
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_get.h"

#define CHECK_HIP(x)                                                       \
  do {                                                                     \
    hipError_t e_ = (x);                                                   \
    if (e_ != hipSuccess) {                                                \
      fprintf(stderr, "HIP error %d at line %d\n", (int)e_, __LINE__);     \
      exit(2);                                                             \
    }                                                                      \
  } while (0)

static const char *g_dir;

static void *read_file(const char *name, size_t n) {
  char path[1024];
  void *p = calloc(1, n ? n : 1);
  FILE *f;
  snprintf(path, sizeof path, "%s/%s.bin", g_dir, name);
  f = fopen(path, "rb");
  if (!f || !p || (n && fread(p, 1, n, f) != n)) {
    fprintf(stderr, "cannot read %zu bytes of %s\n", n, path);
    exit(1);
  }
  fclose(f);
  return p;
}

static void write_file(const char *name, const void *p, size_t n) {
  char path[1024];
  FILE *f;
  snprintf(path, sizeof path, "%s/out_%s.bin", g_dir, name);
  f = fopen(path, "wb");
  if (!f || (n && fwrite(p, 1, n, f) != n)) {
    fprintf(stderr, "cannot write %s\n", path);
    exit(1);
  }
  fclose(f);
}

/* device buffer of n bytes (at least one), optionally filled from host */
static void *dev_buf(const void *host, size_t n) {
  void *d = NULL;
  CHECK_HIP(hipMalloc(&d, n ? n : 1));
  if (host && n) CHECK_HIP(hipMemcpy(d, host, n, hipMemcpyHostToDevice));
  return d;
}

/* copy a device buffer to DIR/out_<name>.bin */
static void save(const char *name, const void *d, size_t n) {
  void *h = malloc(n ? n : 1);
  if (!h) exit(1);
  if (n) CHECK_HIP(hipMemcpy(h, d, n, hipMemcpyDeviceToHost));
  write_file(name, h, n);
  free(h);
}

static void check_moe(int s, const char *what) {
  if (s != MOE_OK) {
    fprintf(stderr, "%s failed: %d (%s)\n", what, s, moe_get_status_string(s));
    exit(3);
  }
}

int main(int argc, char **argv) {
  long v[14];
  int i, has_mask, quant_mode, fused, max_wg;
  int64_t smooth_rows, rows;
  moe_get_shape_t sh;
  FILE *f;
  char path[1024];
  if (argc < 2) {
    fprintf(stderr, "usage: moe_client DIR\n");
    return 1;
  }
  g_dir = argv[1];
  snprintf(path, sizeof path, "%s/shape.txt", g_dir);
  f = fopen(path, "r");
  if (!f) return 1;
  for (i = 0; i < 12; ++i)
    if (fscanf(f, "%ld", &v[i]) != 1) return 1;
  if (fscanf(f, "%ld", &v[12]) != 1) v[12] = 0;
  if (fscanf(f, "%ld", &v[13]) != 1) v[13] = 0;
  fclose(f);
  sh.num_tokens = (int32_t)v[0];
  sh.hidden = (int32_t)v[1];
  sh.topk = (int32_t)v[2];
  sh.num_experts = (int32_t)v[3];
  sh.num_ranks = (int32_t)v[4];
  sh.zero_expert_num = (int32_t)v[5];
  sh.copy_expert_num = (int32_t)v[6];
  sh.const_expert_num = (int32_t)v[7];
  sh.num_max_dispatch_tokens_per_rank = (int32_t)v[8];
  quant_mode = (int)v[9];
  has_mask = (int)v[10];
  smooth_rows = v[11];
  fused = (int)v[12];
  max_wg = (int)v[13];

  if (moe_get_abi_version() != MOE_GET_ABI_VERSION) return 4;
  check_moe(moe_get_check_shape(&sh), "moe_get_check_shape");
  {
    const size_t T = (size_t)sh.num_tokens, H = (size_t)sh.hidden, K = (size_t)sh.topk;
    const size_t E = (size_t)sh.num_experts, P = (size_t)sh.num_ranks;
    const size_t NS = (size_t)(sh.zero_expert_num + sh.copy_expert_num + sh.const_expert_num);
    const size_t Kc = (size_t)sh.const_expert_num;
    const size_t cap = (size_t)moe_get_recv_capacity(&sh);
    const size_t wsb = fused == 2 ? 0 : moe_get_workspace_size(&sh);
    const size_t qbytes = quant_mode == MOE_QUANT_NONE ? 2 : 1;
    void *topk = read_file("topk_idx", T * K * 4), *x = read_file("x", T * H * 2);
    void *w = read_file("w", T * K * 4);
    void *d_topk = dev_buf(topk, T * K * 4), *d_x = dev_buf(x, T * H * 2), *d_w = dev_buf(w, T * K * 4);
    void *d_mask = NULL, *d_smooth = NULL, *d_a1 = NULL, *d_a2 = NULL, *d_cv = NULL, *d_y, *y;
    void *d_cnt = dev_buf(NULL, E * 4), *d_eoff = dev_buf(NULL, (E + 1) * 4);
    void *d_recv = dev_buf(NULL, E * P * 4), *d_spec = dev_buf(NULL, NS * 4);
    void *d_ntpr = dev_buf(NULL, P * 4), *d_roff = dev_buf(NULL, (P + 1) * 4);
    void *d_itr = dev_buf(NULL, T * P), *d_dst = dev_buf(NULL, T * K * 4);
    void *d_src = dev_buf(NULL, cap * 4), *d_status = dev_buf(NULL, 4), *d_ws = wsb ? dev_buf(NULL, wsb) : NULL;
    void *d_ex = dev_buf(NULL, cap * H * qbytes), *d_ds = dev_buf(NULL, cap * 4);
    void *d_ew = dev_buf(NULL, cap * 4), *d_out = dev_buf(NULL, T * H * 2);
    int32_t n_rows = 0;
    free(topk);
    free(x);
    free(w);
    if (has_mask) {
      void *m = read_file("mask", T);
      d_mask = dev_buf(m, T);
      free(m);
    }
    if (smooth_rows > 0) {
      void *s = read_file("smooth", (size_t)smooth_rows * H * 4);
      d_smooth = dev_buf(s, (size_t)smooth_rows * H * 4);
      free(s);
    }
    if (Kc > 0) {
      void *a1 = read_file("a1", Kc * H * 2), *a2 = read_file("a2", Kc * H * 2), *cv = read_file("cv", Kc * H * 2);
      d_a1 = dev_buf(a1, Kc * H * 2);
      d_a2 = dev_buf(a2, Kc * H * 2);
      d_cv = dev_buf(cv, Kc * H * 2);
      free(a1);
      free(a2);
      free(cv);
    }
    CHECK_HIP(hipMemset(d_status, 0, 4));

    if (fused == 2) {
      if (wsb != 0 || moe_get_workspace_size(&sh) > moe_get_noalloc_scratch_bytes()) return 5;
      check_moe(moe_get_layout_noalloc(&sh, 0, (const int32_t *)d_topk, (const uint8_t *)d_mask, (int32_t *)d_cnt,
                                       (int32_t *)d_eoff, (int32_t *)d_recv, (int32_t *)d_spec, (int32_t *)d_ntpr,
                                       (int32_t *)d_roff, (uint8_t *)d_itr, (int32_t *)d_dst, (int32_t *)d_src,
                                       (uint32_t *)d_status, NULL),
                "moe_get_layout_noalloc");
      check_moe(moe_dispatch_capped(&sh, max_wg, quant_mode, (const uint16_t *)d_x, (const float *)d_smooth,
                                    (int32_t)smooth_rows, (const float *)d_w, (const int32_t *)d_topk,
                                    (const int32_t *)d_dst, d_ex,
                                    quant_mode == MOE_QUANT_DYNAMIC_INT8 ? (float *)d_ds : NULL, (float *)d_ew, NULL),
                "moe_dispatch_capped");
    } else if (fused) {
      check_moe(moe_layout_dispatch(&sh, 0, quant_mode, (const int32_t *)d_topk, (const uint8_t *)d_mask,
                                    (const uint16_t *)d_x, (const float *)d_smooth, (int32_t)smooth_rows,
                                    (const float *)d_w, (int32_t *)d_cnt, (int32_t *)d_eoff, (int32_t *)d_recv,
                                    (int32_t *)d_spec, (int32_t *)d_ntpr, (int32_t *)d_roff, (uint8_t *)d_itr,
                                    (int32_t *)d_dst, (int32_t *)d_src, d_ex,
                                    quant_mode == MOE_QUANT_DYNAMIC_INT8 ? (float *)d_ds : NULL, (float *)d_ew,
                                    (uint32_t *)d_status, d_ws, wsb, NULL),
                "moe_layout_dispatch");
    } else {
      check_moe(moe_get_layout(&sh, (const int32_t *)d_topk, (const uint8_t *)d_mask, (int32_t *)d_cnt,
                               (int32_t *)d_eoff, (int32_t *)d_recv, (int32_t *)d_spec, (int32_t *)d_ntpr,
                               (int32_t *)d_roff, (uint8_t *)d_itr, (int32_t *)d_dst, (int32_t *)d_src,
                               (uint32_t *)d_status, d_ws, wsb, NULL),
                "moe_get_layout");
      check_moe(moe_dispatch(&sh, quant_mode, (const uint16_t *)d_x, (const float *)d_smooth,
                             (int32_t)smooth_rows, (const float *)d_w, (const int32_t *)d_topk,
                             (const int32_t *)d_dst, d_ex, quant_mode == MOE_QUANT_DYNAMIC_INT8 ? (float *)d_ds : NULL,
                             (float *)d_ew, NULL),
                "moe_dispatch");
    }
    CHECK_HIP(hipMemcpy(&n_rows, (int32_t *)d_eoff + E, 4, hipMemcpyDeviceToHost));
    rows = n_rows > 0 ? n_rows : 0;
    y = read_file("y", (size_t)rows * H * 2);
    d_y = dev_buf(y, (size_t)rows * H * 2);
    free(y);
    check_moe(moe_combine_capped(&sh, fused == 2 ? max_wg : 0, (const uint16_t *)d_y, (const int32_t *)d_topk,
                                 (const float *)d_w, (const uint8_t *)d_mask, (const int32_t *)d_dst,
                                 (const uint16_t *)d_x, (const uint16_t *)d_a1, (const uint16_t *)d_a2,
                                 (const uint16_t *)d_cv, (uint16_t *)d_out, NULL),
              "moe_combine_capped");
    CHECK_HIP(hipDeviceSynchronize());

    save("num_tokens_per_expert", d_cnt, E * 4);
    save("expert_offsets", d_eoff, (E + 1) * 4);
    save("recv_counts", d_recv, E * P * 4);
    save("special_counts", d_spec, NS * 4);
    save("num_tokens_per_rank", d_ntpr, P * 4);
    save("rank_offsets", d_roff, (P + 1) * 4);
    save("is_token_in_rank", d_itr, T * P);
    save("dst_row", d_dst, T * K * 4);
    save("src_info", d_src, (size_t)rows * 4);
    save("status", d_status, 4);
    save("expand_x", d_ex, (size_t)rows * H * qbytes);
    save("dynamic_scales", d_ds, (size_t)rows * 4);
    save("expand_weights", d_ew, (size_t)rows * 4);
    save("out", d_out, T * H * 2);
    printf("moe_client ok: T=%zu H=%zu K=%zu E=%zu P=%zu rows=%d quant=%d path=%d max_workgroups=%d\n", T, H, K, E,
           P, n_rows, quant_mode, fused, max_wg);
  }
  return 0;
}
