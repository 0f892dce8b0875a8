/*
 * moe_oracle.c -- plain, sequential CPU oracle for MoE expert-parallel
 * token dispatch and combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the CPU-baseline leg of the benchmark may load this library.  The product
 * library (combine_moe_get_amd) never calls it, and the two share no source,
 * header, table or helper.
 *
 * Sources, by page title and section:
 *  [CANN] "low_latency_dispatch" (Huawei CANN operator page)
 *         - Function / Formula, dynamic quantization scenario: quant_out,
 *           x_fp32, dynamic_scales_value, CastToInt8, alltoallv, 1/dyn scale.
 *         - Function / Formula, special expert scenario: zero, copy and
 *           constant experts.
 *         - Prototype: argument names (x, topk_idx, num_experts, quant_mode,
 *           x_active_mask, topk_weights, zero/copy/const_expert_num,
 *           num_max_dispatch_tokens_per_rank).
 *         - Constraints: BS, K, H, A and local_expert_num limits.
 *         - Deterministic Computation.
 *         - Example, single-operator mode call: every rank owns its own batch
 *           of bs tokens; num_experts % moe_rank_num == 0 is checked first.
 *  [DEEPEP-84] "[GH-ISSUE #84] Questions on Profiling dispatch_t for
 *         Low-Latency Kernel Dispatch Bandwidth Calculation": an expert is
 *         owned by rank topk_idx // (num_experts // num_ranks); a slot whose
 *         id is -1 is not sent anywhere.
 *
 * Readings taken where the pages are silent (each one is repeated at the
 * function it affects):
 *  R1  token t belongs to source rank t / BS (contiguous batches).
 *  R2  special expert ids follow the routed ones: zero ids [E, E+Z), copy ids
 *      [E+Z, E+Z+C), constant ids [E+Z+C, E+Z+C+Kc).
 *  R3  x_active_mask false: the token sends nothing, is counted nowhere, and
 *      its combine output is +0.  Its ids are not inspected.
 *  R4  id -1 drops the slot; any other id outside [-1, Etot) is an error that
 *      is reported and drops the slot.
 *  R5  rows of expert e are ordered by (source rank, token, slot); since the
 *      source rank is monotone in t this is (t, j) order.  Receive rows are
 *      compact and expert-major over the whole simulated world.
 *  R6  CastToInt8 rounds half to even and saturates to [-127, 127]; a NaN
 *      product (0 * inf when 127/amax overflows) becomes 0.  amax == 0 gives
 *      q = 0 and scale = 0.
 *  R7  combine: out[t] = sum_j w[t,j] * expert_j(x_t), special experts as in
 *      the special expert formulas, evaluated here in double precision.
 *  R8  the fixed-capacity layout gives rank r the receive window
 *      [r*A, r*A + A) with A >= num_max * ep_world_size * min(L, K) (the
 *      Constraints section's A); its rows keep the compact order.
 *
 * Every function is pinned by the tests to something other than itself (hand
 * cases, the page's routing tables, brute force, exact rational arithmetic,
 * closed forms).  Parity unpinned against the pages themselves: readings R2
 * and R3 (no output is printed that would fix the special-id order or the
 * mask semantics), and the export choices for num_tokens_per_rank (distinct
 * tokens) and the carried top-k weight; these rest on the readings only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "moe_oracle.h"

/* bf16 -> binary32 is exact: the 16 bits are the top half of the float. */
static float bf16_to_float(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Constraints section of [CANN]: 0 < K <= 16, K <= E+Z+C+Kc,
 * 0 < BS <= 512, num_experts a multiple of the number of MoE ranks,
 * local_expert_num * ep_world_size <= 2048, and when
 * num_max_dispatch_tokens_per_rank != 0 the receive capacity is sized from it,
 * so BS may not exceed it.  T == 0 is accepted as an empty world. */
int orc_check_shape(const orc_shape_t *s) {
  if (!s) return ORC_ERR_ARG;
  if (s->num_tokens < 0 || s->hidden <= 0 || s->num_ranks <= 0) return ORC_ERR_SHAPE;
  if (s->topk <= 0 || s->topk > 16) return ORC_ERR_SHAPE;
  if (s->num_experts <= 0 || s->num_experts % s->num_ranks != 0) return ORC_ERR_SHAPE;
  if (s->num_experts > 2048) return ORC_ERR_SHAPE;
  if (s->zero_expert_num < 0 || s->copy_expert_num < 0 || s->const_expert_num < 0)
    return ORC_ERR_SHAPE;
  {
    int64_t etot = (int64_t)s->num_experts + s->zero_expert_num + s->copy_expert_num +
                   s->const_expert_num;
    if (etot >= INT32_MAX) return ORC_ERR_SHAPE;
    if (s->topk > etot) return ORC_ERR_SHAPE;
  }
  if (s->num_tokens % s->num_ranks != 0) return ORC_ERR_SHAPE;
  {
    int bs = s->num_tokens / s->num_ranks;
    if (bs > 512) return ORC_ERR_SHAPE;
    if (s->num_max_dispatch_tokens_per_rank < 0) return ORC_ERR_SHAPE;
    if (s->num_max_dispatch_tokens_per_rank > 0 && bs > s->num_max_dispatch_tokens_per_rank)
      return ORC_ERR_CAPACITY;
  }
  return ORC_OK;
}

/* Slot classes (R2, R3, R4). */
enum { SLOT_NONE = 0, SLOT_ROUTED = 1, SLOT_ZERO = 2, SLOT_COPY = 3, SLOT_CONST = 4, SLOT_BAD = 5 };

static int slot_class(const orc_shape_t *s, const uint8_t *mask, int t, int32_t id) {
  int E = s->num_experts, Z = s->zero_expert_num, C = s->copy_expert_num;
  int64_t etot = (int64_t)E + Z + C + s->const_expert_num;
  if (mask && !mask[t]) return SLOT_NONE;
  if (id == -1) return SLOT_NONE;
  if (id < 0 || (int64_t)id >= etot) return SLOT_BAD;
  if (id < E) return SLOT_ROUTED;
  if (id < E + Z) return SLOT_ZERO;
  if (id < E + Z + C) return SLOT_COPY;
  return SLOT_CONST;
}

/* Routing layout.  Definitions (R1, R5 and the owner rule of [DEEPEP-84]):
 *   cnt[e]            = number of routed slots with id e
 *   recv_counts[e][s] = the same, restricted to tokens of source rank s
 *   expert_offsets    = exclusive prefix sum of cnt; N = expert_offsets[E]
 *   rank_offsets[r]   = expert_offsets[r * L]  (rank r owns experts [rL, rL+L))
 *   dst_row[t][j]     = receive row of slot (t, j), or -1 if it is not routed
 *   src_info[row]     = t * K + j for the slot that occupies row
 *   is_token_in_rank[t][r] = 1 if some routed slot of t goes to an expert of r
 *   num_tokens_per_rank[r] = number of distinct tokens with a slot on rank r
 *   special_counts[i] = number of slots with id E + i
 * Rows are handed out expert by expert, and inside an expert in (t, j) order,
 * which is the stable order asked for by the Deterministic Computation
 * section.  Returns 0, or 1 when a bad id was seen (its slot dropped). */
int orc_layout(const orc_shape_t *s, const int32_t *topk_idx, const uint8_t *mask,
               int32_t *cnt, int32_t *expert_offsets, int32_t *recv_counts,
               int32_t *special_counts, int32_t *num_tokens_per_rank, int32_t *rank_offsets,
               uint8_t *is_token_in_rank, int32_t *dst_row, int32_t *src_info) {
  return orc_layout_ex(s, 0, topk_idx, mask, cnt, expert_offsets, recv_counts, special_counts,
                       num_tokens_per_rank, rank_offsets, is_token_in_rank, dst_row, src_info);
}

/* Smallest per-rank receive window the Constraints section of [CANN] allows:
 * A >= num_max * ep_world_size * min(local_expert_num, K), num_max = BS when 0. */
int64_t orc_rank_capacity(const orc_shape_t *s) {
  int64_t bs = s->num_ranks > 0 ? s->num_tokens / s->num_ranks : 0;
  int64_t nm = s->num_max_dispatch_tokens_per_rank > 0 ? s->num_max_dispatch_tokens_per_rank : bs;
  int64_t L = s->num_ranks > 0 ? s->num_experts / s->num_ranks : 0;
  int64_t m = L < s->topk ? L : s->topk;
  return nm * s->num_ranks * m;
}

/* Layout with fixed per-rank receive windows (rank_stride A > 0): the rows rank r
 * receives, in the compact order, are placed at r*A, r*A + 1, ...; a row that would
 * pass r*A + A - 1 (possible only with a repeated expert id in one token) is dropped
 * (dst_row -1) and the return value gets bit 2.  rank_stride 0 is the compact layout.
 * Counts and offsets describe the routing in both cases. */
int orc_layout_ex(const orc_shape_t *s, int64_t rank_stride, const int32_t *topk_idx,
                  const uint8_t *mask, int32_t *cnt, int32_t *expert_offsets, int32_t *recv_counts,
                  int32_t *special_counts, int32_t *num_tokens_per_rank, int32_t *rank_offsets,
                  uint8_t *is_token_in_rank, int32_t *dst_row, int32_t *src_info) {
  const int T = s->num_tokens, K = s->topk, E = s->num_experts, P = s->num_ranks;
  const int L = E / P;
  const int BS = T / P;
  const int NS = s->zero_expert_num + s->copy_expert_num + s->const_expert_num;
  int bad = 0;
  int t, j, e, r;

  for (e = 0; e < E; ++e) {
    cnt[e] = 0;
    for (r = 0; r < P; ++r) recv_counts[(size_t)e * P + r] = 0;
  }
  for (e = 0; e < NS; ++e) special_counts[e] = 0;
  for (r = 0; r < P; ++r) num_tokens_per_rank[r] = 0;
  for (t = 0; t < T; ++t) {
    for (r = 0; r < P; ++r) is_token_in_rank[(size_t)t * P + r] = 0;
    for (j = 0; j < K; ++j) dst_row[(size_t)t * K + j] = -1;
  }

  /* counts and token-in-rank flags */
  for (t = 0; t < T; ++t) {
    for (j = 0; j < K; ++j) {
      int32_t id = topk_idx[(size_t)t * K + j];
      int c = slot_class(s, mask, t, id);
      if (c == SLOT_BAD) bad = 1;
      if (c == SLOT_ZERO || c == SLOT_COPY || c == SLOT_CONST) special_counts[id - E] += 1;
      if (c != SLOT_ROUTED) continue;
      cnt[id] += 1;
      recv_counts[(size_t)id * P + t / BS] += 1;
      is_token_in_rank[(size_t)t * P + id / L] = 1;
    }
  }
  for (t = 0; t < T; ++t)
    for (r = 0; r < P; ++r) num_tokens_per_rank[r] += is_token_in_rank[(size_t)t * P + r];

  expert_offsets[0] = 0;
  for (e = 0; e < E; ++e) expert_offsets[e + 1] = expert_offsets[e] + cnt[e];
  for (r = 0; r <= P; ++r) rank_offsets[r] = expert_offsets[r * L];

  /* rows: expert by expert, then token, then slot */
  {
    int32_t row = 0;
    for (e = 0; e < E; ++e)
      for (t = 0; t < T; ++t)
        for (j = 0; j < K; ++j) {
          int32_t id = topk_idx[(size_t)t * K + j];
          int64_t placed = row;
          if (id != e || slot_class(s, mask, t, id) != SLOT_ROUTED) continue;
          if (rank_stride > 0) {
            int owner = e / L;
            int64_t local = row - rank_offsets[owner];
            placed = -1;
            if (local < rank_stride) placed = (int64_t)owner * rank_stride + local;
            else bad |= 2;
          }
          ++row;
          if (placed < 0) continue;
          dst_row[(size_t)t * K + j] = (int32_t)placed;
          src_info[placed] = t * K + j;
        }
  }
  return bad;
}

/* Dynamic quantization of one token, Formula / dynamic quantization scenario
 * of [CANN], in binary32 as the formula's CastToFp32 fixes:
 *   x_fp32 = fp32(x) * scales          (scales == NULL reads as all ones)
 *   dyn    = 127.0 / max|x_fp32|
 *   q      = CastToInt8(x_fp32 * dyn)  (R6: round half to even, saturate)
 *   scale  = 1.0 / dyn                 (the value sent with the row)
 * amax == 0 gives q = 0 and scale = 0 (R6). */
void orc_quant_token(int H, const uint16_t *x, const float *scales, int8_t *q, float *scale) {
  float amax = 0.0f;
  int h;
  for (h = 0; h < H; ++h) {
    float xf = bf16_to_float(x[h]) * (scales ? scales[h] : 1.0f);
    float a = fabsf(xf);
    if (a > amax) amax = a;
  }
  if (!(amax > 0.0f)) {
    for (h = 0; h < H; ++h) q[h] = 0;
    *scale = 0.0f;
    return;
  }
  {
    float dyn = 127.0f / amax;
    for (h = 0; h < H; ++h) {
      float xf = bf16_to_float(x[h]) * (scales ? scales[h] : 1.0f);
      float p = xf * dyn;
      float rr = rintf(p);
      int v;
      if (isnan(rr)) v = 0;
      else if (rr > 127.0f) v = 127;
      else if (rr < -127.0f) v = -127;
      else v = (int)rr;
      q[h] = (int8_t)v;
    }
    *scale = 1.0f / dyn;
  }
}

/* Static quantization, Formula of [CANN] for quant_mode not 0 and not 2:
 * q = CastToInt8(fp32(x) * scales), with the rounding and saturation of R6. */
void orc_quant_static(int H, const uint16_t *x, const float *scales, int8_t *q) {
  int h;
  for (h = 0; h < H; ++h) {
    float p = bf16_to_float(x[h]) * (scales ? scales[h] : 1.0f);
    float rr = rintf(p);
    int v;
    if (isnan(rr)) v = 0;
    else if (rr > 127.0f) v = 127;
    else if (rr < -127.0f) v = -127;
    else v = (int)rr;
    q[h] = (int8_t)v;
  }
}

/* Dispatch: every routed slot (t, j) writes the token's (quantized) row to
 * receive row dst_row[t][j] (the alltoallv of quant_out, here a copy into the
 * expert-major receive buffer), with the token's scale (quant_mode 2) and the
 * slot's weight when those outputs are given.
 * quant_mode 0: rows are the bf16 tokens, bit for bit.
 * quant_mode 1: static int8, no scale output.
 * quant_mode 2: dynamic int8 + one fp32 scale per row.
 * smooth_rows: 0 no scales, 1 one [H] vector for all rows, E one [H] vector
 * per routed expert (the [num_experts, H] scales of the Example section),
 * picked by the slot's expert. */
int orc_dispatch(const orc_shape_t *s, int quant_mode, const uint16_t *x, const float *smooth,
                 int smooth_rows, const float *topk_weights, const int32_t *topk_idx,
                 const int32_t *dst_row, void *expand_x, float *dynamic_scales,
                 float *expand_weights) {
  const int T = s->num_tokens, H = s->hidden, K = s->topk;
  int8_t *q = NULL;
  int t, j;
  if (quant_mode != 0 && quant_mode != 1 && quant_mode != 2) return ORC_ERR_ARG;
  if (smooth_rows != 0 && smooth_rows != 1 && smooth_rows != s->num_experts) return ORC_ERR_ARG;
  if (quant_mode != 0) {
    q = (int8_t *)malloc((size_t)H > 0 ? (size_t)H : 1);
    if (!q) return ORC_ERR_ARG;
  }
  for (t = 0; t < T; ++t) {
    const uint16_t *xt = x + (size_t)t * H;
    float scale = 0.0f;
    int have_shared = 0;
    for (j = 0; j < K; ++j) {
      int32_t row = dst_row[(size_t)t * K + j];
      const float *sv = NULL;
      if (row < 0) continue;
      if (smooth && smooth_rows == 1) sv = smooth;
      if (smooth && smooth_rows > 1) sv = smooth + (size_t)topk_idx[(size_t)t * K + j] * H;
      if (quant_mode == 0) {
        memcpy((uint16_t *)expand_x + (size_t)row * H, xt, (size_t)H * 2);
      } else if (quant_mode == 1) {
        orc_quant_static(H, xt, sv, q);
        memcpy((int8_t *)expand_x + (size_t)row * H, q, (size_t)H);
      } else {
        /* the token is quantized once when its scale vector is shared */
        if (!(smooth_rows <= 1 && have_shared)) orc_quant_token(H, xt, sv, q, &scale);
        have_shared = 1;
        memcpy((int8_t *)expand_x + (size_t)row * H, q, (size_t)H);
        if (dynamic_scales) dynamic_scales[row] = scale;
      }
      if (expand_weights) expand_weights[row] = topk_weights ? topk_weights[(size_t)t * K + j] : 1.0f;
    }
  }
  free(q);
  return ORC_OK;
}

/* Combine (R7), with the special experts of the special expert scenario:
 *   zero:  Moe(ori_x) = 0
 *   copy:  Moe(ori_x) = ori_x
 *   const: Moe(ori_x) = alpha1[c] * ori_x + alpha2[c] * v[c]   (element-wise, [Kc, H])
 * out[t] = sum over the token's slots of w[t,j] * Moe_j, in double precision;
 * routed experts read the expert-output row dst_row[t][j]; dropped slots (and a
 * routed copy whose dst_row is -1 because its rank window was full, R8) add
 * nothing; a masked token (R3) gets +0.  Products of a binary32 weight and a
 * bf16 value are exact in double, so the only rounding is in the sums. */
int orc_combine(const orc_shape_t *s, const uint16_t *expert_out, const int32_t *topk_idx,
                const float *topk_weights, const uint8_t *mask, const int32_t *dst_row,
                const uint16_t *ori_x, const uint16_t *alpha1, const uint16_t *alpha2,
                const uint16_t *const_v, double *out) {
  const int T = s->num_tokens, H = s->hidden, K = s->topk, E = s->num_experts;
  const int ZC = s->zero_expert_num + s->copy_expert_num;
  int t, j, h;
  int bad = 0;
  for (t = 0; t < T; ++t) {
    double *o = out + (size_t)t * H;
    for (h = 0; h < H; ++h) o[h] = 0.0;
    if (mask && !mask[t]) continue;
    for (j = 0; j < K; ++j) {
      int32_t id = topk_idx[(size_t)t * K + j];
      int c = slot_class(s, mask, t, id);
      double w = (double)topk_weights[(size_t)t * K + j];
      if (c == SLOT_BAD) bad = 1;
      /* R8: a copy that did not fit its rank window was never sent (dst_row -1), so its
       * expert returns nothing for it */
      if (c == SLOT_ROUTED && dst_row[(size_t)t * K + j] < 0) c = SLOT_NONE;
      if (c == SLOT_ROUTED) {
        const uint16_t *y = expert_out + (size_t)dst_row[(size_t)t * K + j] * H;
        for (h = 0; h < H; ++h) o[h] += w * (double)bf16_to_float(y[h]);
      } else if (c == SLOT_COPY) {
        const uint16_t *xo = ori_x + (size_t)t * H;
        for (h = 0; h < H; ++h) o[h] += w * (double)bf16_to_float(xo[h]);
      } else if (c == SLOT_CONST) {
        int ci = id - E - ZC;
        const uint16_t *xo = ori_x + (size_t)t * H;
        const uint16_t *a1 = alpha1 + (size_t)ci * H;
        const uint16_t *a2 = alpha2 + (size_t)ci * H;
        const uint16_t *cv = const_v + (size_t)ci * H;
        for (h = 0; h < H; ++h) {
          double y = (double)bf16_to_float(a1[h]) * (double)bf16_to_float(xo[h]) +
                     (double)bf16_to_float(a2[h]) * (double)bf16_to_float(cv[h]);
          o[h] += w * y;
        }
      }
      /* SLOT_ZERO, SLOT_NONE, SLOT_BAD contribute nothing */
    }
  }
  return bad;
}

/* Round a double to the nearest bf16, ties to even (finite values only). */
uint16_t orc_double_to_bf16(double v) {
  /* Work on the exact binary value: split off the sign, scale into
   * [2^7, 2^8) so the bf16 significand is the integer part. */
  double a = fabs(v);
  int sign = v < 0 || (v == 0 && signbit(v));
  uint16_t out;
  if (a == 0.0) {
    out = 0;
  } else {
    int ex;
    double m = frexp(a, &ex); /* a = m * 2^ex, m in [0.5, 1) */
    /* normal bf16 has 8 significant bits: value = n * 2^(ex - 8), n in [128, 256) */
    int e2 = ex - 8;
    if (ex - 1 < -126) e2 = -126 - 7; /* subnormal: fixed quantum 2^-133 */
    {
      double n = ldexp(a, -e2);
      double fl = floor(n);
      double fr = n - fl;
      if (fr > 0.5 || (fr == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
      {
        float f = (float)ldexp(fl, e2); /* exact: fl has <= 9 bits */
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        out = (uint16_t)(u >> 16);
      }
    }
    (void)m;
  }
  if (sign) out |= 0x8000u;
  return out;
}
