/*
 * moe_get.h -- C ABI of the MI355X (gfx950) library for MoE expert-parallel
 * token dispatch and combine.
 *
 * One GPU lays out and moves the tokens of a whole simulated expert-parallel
 * world of P ranks: the all-to-all of the multi-GPU operation becomes a
 * scatter into (dispatch) and a gather from (combine) expert-major receive
 * rows in HBM.  There is no transport and no collective.
 *
 * The operation is the one of the CANN operator page "low_latency_dispatch"
 * (and its partner low_latency_combine): Function / Formula (dynamic
 * quantization scenario, special expert scenario), Prototype, Constraints,
 * Deterministic Computation.  Expert ownership and -1 slots follow the DeepEP
 * issue "[GH-ISSUE #84] Questions on Profiling dispatch_t for Low-Latency
 * Kernel Dispatch Bandwidth Calculation".  The routing layout is split out of
 * dispatch as its own call.
 *
 * Conventions for every entry point
 *  - All array arguments are device pointers (HIP global memory), row-major,
 *    contiguous, allocated and owned by the caller.  The library allocates
 *    nothing and keeps no state between calls (moe_get_layout_noalloc's static
 *    scratch holds nothing a later call reads).
 *  - bf16 tensors are passed as uint16_t bit patterns.
 *  - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *    enqueued on it in order; no call synchronizes the host.  Calls on
 *    different streams that share output buffers race.
 *  - Return value: MOE_OK or a negative moe_get_status_t.  Argument errors are
 *    found on the host before anything is enqueued; nothing is launched then.
 *  - Shared symbols: T = num_tokens (all ranks), P = num_ranks, BS = T / P
 *    tokens per rank (token t belongs to rank t / BS), H = hidden, K = topk,
 *    E = num_experts (routed), L = E / P experts per rank (rank r owns experts
 *    [rL, rL + L)), Z / C / Kc = zero / copy / constant expert counts,
 *    Etot = E + Z + C + Kc, N = number of routed copies (rows actually used).
 *    Special ids: zero [E, E+Z), copy [E+Z, E+Z+C), constant [E+Z+C, Etot).
 */
#ifndef MOE_GET_H
#define MOE_GET_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_GET_ABI_VERSION 2

/* Sizes of one call.  Constraints section of "low_latency_dispatch":
 * 0 < K <= 16 and K <= Etot; BS <= 512; E a multiple of P; L * P <= 2048;
 * num_max_dispatch_tokens_per_rank = 0 means BS, otherwise BS may not exceed
 * it.  The kernels add: hidden a multiple of 8 and at most 8192 (the top of
 * the page's H range; smaller H is accepted), Z + C + Kc <= 1024.
 * T = 0 is accepted and does nothing but zero the counts. */
typedef struct moe_get_shape {
  int32_t num_tokens;
  int32_t hidden;
  int32_t topk;
  int32_t num_experts;
  int32_t num_ranks;
  int32_t zero_expert_num;
  int32_t copy_expert_num;
  int32_t const_expert_num;
  int32_t num_max_dispatch_tokens_per_rank;
} moe_get_shape_t;

typedef enum moe_get_status {
  MOE_OK = 0,
  MOE_ERR_ARG = -1,         /* NULL where a buffer is required, bad mode, small workspace */
  MOE_ERR_SHAPE = -2,       /* sizes outside the Constraints section */
  MOE_ERR_CAPACITY = -3,    /* BS > num_max_dispatch_tokens_per_rank, or a rank window below capacity */
  MOE_ERR_UNSUPPORTED = -4, /* allowed by the page but not by these kernels (H % 8, H > 8192, Z+C+Kc > 1024) */
  MOE_ERR_HIP = -5,         /* the HIP runtime refused a launch (or a device lookup) */
  MOE_ERR_SCRATCH = -6      /* moe_get_layout_noalloc: the shape needs more than its static scratch */
} moe_get_status_t;

/* Bits of the device status word written by moe_get_layout (sticky: the
 * library only ORs bits in; the caller clears the word). */
#define MOE_DEV_STATUS_BAD_EXPERT_ID 1u /* an id outside [-1, Etot) was seen; its slot was dropped */
#define MOE_DEV_STATUS_RANK_OVERFLOW 2u /* a copy did not fit its rank's receive window; it was dropped */

/* Quantization modes of dispatch (Formula, dynamic quantization scenario). */
#define MOE_QUANT_NONE 0          /* expand_x rows are the bf16 tokens, bit for bit */
#define MOE_QUANT_STATIC_INT8 1   /* q = CastToInt8(fp32(x) * scales) */
#define MOE_QUANT_DYNAMIC_INT8 2  /* q = CastToInt8(x_fp32 * 127 / max|x_fp32|), 1/dyn per row */

int moe_get_abi_version(void);

/* Static English text of a status code. */
const char *moe_get_status_string(int status);

/* Validate a shape against the Constraints section and the kernel limits. */
int moe_get_check_shape(const moe_get_shape_t *shape);

/* Receive rows the caller must allocate for expand_x / expert outputs /
 * src_info: T * K (every slot routed).  Returns -1 for an invalid shape.
 * The rows actually used, N, are expert_offsets[E] after moe_get_layout;
 * rows >= N are never written or read. */
int64_t moe_get_recv_capacity(const moe_get_shape_t *shape);

/* Smallest per-rank receive window A of the fixed-capacity layout: the
 * Constraints section's A >= num_max * P * min(L, K), with num_max = BS when
 * num_max_dispatch_tokens_per_rank is 0.  Returns -1 for an invalid shape. */
int64_t moe_get_rank_capacity(const moe_get_shape_t *shape);

/* Kernel launches one moe_get_layout / moe_get_layout_ex call makes for this
 * shape: 1 (T * K <= 8192 slots: every workgroup histograms all ids itself)
 * or 2 (a count kernel, then a scan-and-finalize kernel).  For profiling and
 * launch accounting only; a negative MOE_ERR_* for an invalid shape. */
int moe_get_layout_launches(const moe_get_shape_t *shape);

/* Bytes of device workspace moe_get_layout needs (0 for an invalid shape). */
size_t moe_get_workspace_size(const moe_get_shape_t *shape);

/* Routing layout (the per-expert / per-rank bookkeeping the page's dispatch
 * returns as expert_token_nums, ep_recv_counts and assist_info_for_combine).
 *  in  topk_idx [T, K] int32            expert id per slot; -1 drops the slot
 *  in  x_active_mask [T] uint8 or NULL  0: the token sends nothing, counts
 *                                       nowhere and combines to +0
 *  out num_tokens_per_expert [E]        routed copies per expert
 *  out expert_offsets [E + 1]           exclusive prefix sum; [E] = N
 *  out recv_counts [E, P]               copies of expert e sent by rank s
 *  out special_counts [Z + C + Kc]      slots per special id (NULL if none)
 *  out num_tokens_per_rank [P]          distinct tokens with a copy on rank r
 *  out rank_offsets [P + 1]             first row of rank r = expert_offsets[rL]
 *  out is_token_in_rank [T, P] uint8    1 if token t has a copy on rank r
 *  out dst_row [T, K]                   receive row of each slot, -1 if not routed
 *  out src_info [T * K]                 t * K + j of the slot in each row < N
 *  out status_dev (1 uint32 or NULL)    MOE_DEV_STATUS_* bits ORed in
 *  workspace / workspace_bytes          >= moe_get_workspace_size(shape) bytes
 * Rows of expert e are ordered by (source rank, token, slot): the stable
 * order that makes the result deterministic (Deterministic Computation). */
int moe_get_layout(const moe_get_shape_t *shape, const int32_t *topk_idx,
                   const uint8_t *x_active_mask, int32_t *num_tokens_per_expert,
                   int32_t *expert_offsets, int32_t *recv_counts, int32_t *special_counts,
                   int32_t *num_tokens_per_rank, int32_t *rank_offsets,
                   uint8_t *is_token_in_rank, int32_t *dst_row, int32_t *src_info,
                   uint32_t *status_dev, void *workspace, size_t workspace_bytes, void *stream);

/* moe_get_layout with fixed per-rank receive windows: rank_stride A > 0 puts
 * the rows rank r receives (in the same stable order) at r*A, r*A + 1, ..., so
 * every rank owns the window [r*A, (r+1)*A) of a [P * A, H] receive buffer --
 * the per-rank buffer of capacity A that the Constraints section sizes, and the
 * layout a transport between ranks needs (one fixed window per destination;
 * alternate two such buffers between consecutive calls to keep one in flight,
 * the "two sets of buffers" of the DeepEP issue #84 thread).
 *  rank_stride   0 (compact rows, exactly moe_get_layout) or
 *                >= moe_get_rank_capacity(shape), with P * rank_stride < 2^31
 *                (else MOE_ERR_CAPACITY)
 *  src_info      [P * rank_stride]; rows of a window past the rank's count are
 *                left as they were
 * Counts and offsets (num_tokens_per_expert, expert_offsets, rank_offsets, ...)
 * describe the routing as in the compact layout; the rows of expert e start at
 * r*A + expert_offsets[e] - rank_offsets[r] for its owner r.  A copy that would
 * pass the end of its window (possible only when a token repeats an expert id)
 * is dropped and MOE_DEV_STATUS_RANK_OVERFLOW is set. */
int moe_get_layout_ex(const moe_get_shape_t *shape, int64_t rank_stride, const int32_t *topk_idx,
                      const uint8_t *x_active_mask, int32_t *num_tokens_per_expert,
                      int32_t *expert_offsets, int32_t *recv_counts, int32_t *special_counts,
                      int32_t *num_tokens_per_rank, int32_t *rank_offsets,
                      uint8_t *is_token_in_rank, int32_t *dst_row, int32_t *src_info,
                      uint32_t *status_dev, void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of the static device scratch of moe_get_layout_noalloc (per device). */
#define MOE_GET_NOALLOC_SCRATCH_BYTES (4u << 20)

/* moe_get_layout_ex without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Results are those of moe_get_layout_ex(shape, rank_stride, ...) bit for bit.  Its workspace
 * is a static device array of MOE_GET_NOALLOC_SCRATCH_BYTES that every device holds for the
 * life of the process (moe_get_workspace_size(shape) must fit in it, else MOE_ERR_SCRATCH and
 * nothing is launched); it allocates nothing and keeps nothing that a later call depends on.
 * Calls that overlap on one device (concurrent streams, or several host threads) share that
 * device's scratch and race: order them on one stream.  The first call on a device looks up the
 * array's device address once (with that device made current); the device is the one of
 * `stream` (the current device for a NULL stream). */
int moe_get_layout_noalloc(const moe_get_shape_t *shape, int64_t rank_stride, const int32_t *topk_idx,
                           const uint8_t *x_active_mask, int32_t *num_tokens_per_expert,
                           int32_t *expert_offsets, int32_t *recv_counts, int32_t *special_counts,
                           int32_t *num_tokens_per_rank, int32_t *rank_offsets,
                           uint8_t *is_token_in_rank, int32_t *dst_row, int32_t *src_info,
                           uint32_t *status_dev, void *stream);

/* MOE_GET_NOALLOC_SCRATCH_BYTES, for bindings that cannot read the macro. */
size_t moe_get_noalloc_scratch_bytes(void);

/* Dispatch: quantize (optionally) and scatter every routed copy of every
 * token into its receive row (the alltoallv of quant_out of the Formula, and
 * the alltoall of 1/dynamic_scales in quant mode 2).
 *  quant_mode        MOE_QUANT_NONE / _STATIC_INT8 / _DYNAMIC_INT8
 *  in  x [T, H] bf16
 *  in  x_smooth_scale float32 or NULL   the formula's `scales`
 *  smooth_rows       0: none (all ones); 1: one [H] vector; E: [E, H], the row
 *                    of the copy's expert (then every copy is quantized alone)
 *  in  topk_weights [T, K] or NULL      copied to expand_weights
 *  in  topk_idx [T, K]                  needed only when smooth_rows == E
 *  in  dst_row [T, K]                   from moe_get_layout with the same shape/mask
 *  out expand_x [cap, H]                bf16 (mode 0) or int8 (modes 1, 2)
 *  out dynamic_scales [cap] or NULL     mode 2: 1 / dyn of the row's token
 *  out expand_weights [cap] or NULL     weight of the row's slot (1 if no weights)
 * int8 codes: x_fp32 = fp32(x) * scales rounded to binary32; dyn = 127 / amax
 * correctly rounded; q = round-half-even(x_fp32 * dyn) saturated to
 * [-127, 127] (a NaN product, 0 * inf, gives 0); amax == 0 gives q = 0 and
 * scale 0.  Launches one kernel; with quant_mode MOE_QUANT_STATIC_INT8 and x of
 * at least 24 MiB (T * H * 2 bytes), two (a sequential read of x ahead of the
 * dispatch kernel). */
int moe_dispatch(const moe_get_shape_t *shape, int32_t quant_mode, const uint16_t *x,
                 const float *x_smooth_scale, int32_t smooth_rows, const float *topk_weights,
                 const int32_t *topk_idx, const int32_t *dst_row, void *expand_x,
                 float *dynamic_scales, float *expand_weights, void *stream);

/* moe_dispatch on a capped grid: at most max_workgroups workgroups, each quantizing and
 * scattering several work items in turn (max_workgroups 0: one per item, exactly moe_dispatch;
 * negative: MOE_ERR_ARG).  Results are those of moe_dispatch bit for bit.  It bounds the part of
 * the GPU the data movement holds, so that it can run beside other kernels on other streams --
 * the compute-unit reservation of dual-batch overlap ("Wide-EP / DBO / DeepEP hardware cliff",
 * section 1) DBO: hiding the wire, VLLM_DBO_COMM_SMS) -- without masking compute units. */
int moe_dispatch_capped(const moe_get_shape_t *shape, int32_t max_workgroups, int32_t quant_mode, const uint16_t *x,
                        const float *x_smooth_scale, int32_t smooth_rows, const float *topk_weights,
                        const int32_t *topk_idx, const int32_t *dst_row, void *expand_x, float *dynamic_scales,
                        float *expand_weights, void *stream);

/* Layout and dispatch in one call, the way the CANN dispatch operator returns
 * the routing layout (expert_token_nums, ep_recv_counts, assist_info_for_combine)
 * together with the dispatched rows (its Prototype and Formula).  Results are
 * identical, bit for bit, to moe_get_layout_ex(shape, rank_stride, ...)
 * followed by moe_dispatch(shape, quant_mode, ...) with the same arguments;
 * argument rules and errors are the union of theirs.  Small worlds (T * K <=
 * 8192 slots with bf16 rows, <= 2048 with int8 codes) run as a single kernel --
 * every workgroup derives its chunk's rows itself and dispatches a share of the
 * chunk's tokens -- which saves the launches between layout and dispatch on the
 * decode-sized batches the low-latency kernels target; larger worlds run the
 * layout (one kernel up to 8192 slots, else two, which also read x, T * H * 2
 * bytes, loads only, so that the dispatch finds its rows in the GPU's caches),
 * then the dispatch (see moe_dispatch).  x is read,
 * never written; it must not be written by other work while the call runs, as
 * for moe_dispatch.  Workspace as for moe_get_layout. */
int moe_layout_dispatch(const moe_get_shape_t *shape, int64_t rank_stride, int32_t quant_mode,
                        const int32_t *topk_idx, const uint8_t *x_active_mask, const uint16_t *x,
                        const float *x_smooth_scale, int32_t smooth_rows, const float *topk_weights,
                        int32_t *num_tokens_per_expert, int32_t *expert_offsets, int32_t *recv_counts,
                        int32_t *special_counts, int32_t *num_tokens_per_rank, int32_t *rank_offsets,
                        uint8_t *is_token_in_rank, int32_t *dst_row, int32_t *src_info, void *expand_x,
                        float *dynamic_scales, float *expand_weights, uint32_t *status_dev, void *workspace,
                        size_t workspace_bytes, void *stream);

/* Kernel launches one moe_layout_dispatch call makes for this shape and
 * quant_mode (1 when layout and dispatch run as a single kernel, else the
 * layout's launches plus the dispatch's); a negative MOE_ERR_* for an invalid
 * shape, MOE_ERR_ARG for a quant_mode outside 0..2. */
int moe_layout_dispatch_launches(const moe_get_shape_t *shape, int32_t quant_mode);

/* Combine: out[t] = bf16( sum_j w[t,j] * Moe_j(t) ), fp32 accumulation in
 * slot order j = 0..K-1, where Moe_j is
 *   routed expert:   expert_out[dst_row[t, j]]
 *   zero expert:     0
 *   copy expert:     ori_x[t]
 *   constant expert: alpha1[c] * ori_x[t] + alpha2[c] * v[c]   (element-wise)
 * (special expert scenario of the Formula).  Slots with id -1 or a bad id add
 * nothing; tokens with x_active_mask 0 get +0.
 *  in  expert_out [cap, H] bf16         rows produced by the experts from expand_x
 *  in  topk_idx, topk_weights [T, K]    as given to moe_get_layout / dispatch
 *  in  x_active_mask [T] or NULL        as given to moe_get_layout
 *  in  dst_row [T, K]                   from moe_get_layout
 *  in  ori_x [T, H] bf16                required when C + Kc > 0
 *  in  const_alpha1, const_alpha2, const_v [Kc, H] bf16   required when Kc > 0
 *  out out [T, H] bf16 */
int moe_combine(const moe_get_shape_t *shape, const uint16_t *expert_out,
                const int32_t *topk_idx, const float *topk_weights,
                const uint8_t *x_active_mask, const int32_t *dst_row, const uint16_t *ori_x,
                const uint16_t *const_alpha1, const uint16_t *const_alpha2,
                const uint16_t *const_v, uint16_t *out, void *stream);

/* moe_combine on a capped grid (see moe_dispatch_capped): at most max_workgroups workgroups,
 * results identical to moe_combine bit for bit; 0 means uncapped. */
int moe_combine_capped(const moe_get_shape_t *shape, int32_t max_workgroups, const uint16_t *expert_out,
                       const int32_t *topk_idx, const float *topk_weights, const uint8_t *x_active_mask,
                       const int32_t *dst_row, const uint16_t *ori_x, const uint16_t *const_alpha1,
                       const uint16_t *const_alpha2, const uint16_t *const_v, uint16_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_GET_H */
