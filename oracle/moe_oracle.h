/*
 * moe_oracle.h -- declarations of the CPU oracle for MoE dispatch/combine.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the package smoke check
 * and the CPU-baseline leg of the benchmark, never by the product library.
 * All buffers are host memory, row-major and owned by the caller.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_OK = 0, ORC_ERR_ARG = -1, ORC_ERR_SHAPE = -2, ORC_ERR_CAPACITY = -3 };

typedef struct {
  int32_t num_tokens; /* T = P * BS */
  int32_t hidden;     /* H */
  int32_t topk;       /* K */
  int32_t num_experts;
  int32_t num_ranks;  /* P */
  int32_t zero_expert_num;
  int32_t copy_expert_num;
  int32_t const_expert_num;
  int32_t num_max_dispatch_tokens_per_rank;
} orc_shape_t;

int orc_check_shape(const orc_shape_t *s);

int orc_layout(const orc_shape_t *s, const int32_t *topk_idx, const uint8_t *mask,
               int32_t *cnt, int32_t *expert_offsets, int32_t *recv_counts,
               int32_t *special_counts, int32_t *num_tokens_per_rank, int32_t *rank_offsets,
               uint8_t *is_token_in_rank, int32_t *dst_row, int32_t *src_info);

int64_t orc_rank_capacity(const orc_shape_t *s);

int orc_layout_ex(const orc_shape_t *s, int64_t rank_stride, const int32_t *topk_idx,
                  const uint8_t *mask, int32_t *cnt, int32_t *expert_offsets, int32_t *recv_counts,
                  int32_t *special_counts, int32_t *num_tokens_per_rank, int32_t *rank_offsets,
                  uint8_t *is_token_in_rank, int32_t *dst_row, int32_t *src_info);

void orc_quant_token(int H, const uint16_t *x, const float *scales, int8_t *q, float *scale);
void orc_quant_static(int H, const uint16_t *x, const float *scales, int8_t *q);

int orc_dispatch(const orc_shape_t *s, int quant_mode, const uint16_t *x, const float *smooth,
                 int smooth_rows, const float *topk_weights, const int32_t *topk_idx,
                 const int32_t *dst_row, void *expand_x, float *dynamic_scales,
                 float *expand_weights);

int orc_combine(const orc_shape_t *s, const uint16_t *expert_out, const int32_t *topk_idx,
                const float *topk_weights, const uint8_t *mask, const int32_t *dst_row,
                const uint16_t *ori_x, const uint16_t *alpha1, const uint16_t *alpha2,
                const uint16_t *const_v, double *out);

uint16_t orc_double_to_bf16(double v);

#ifdef __cplusplus
}
#endif

#endif
