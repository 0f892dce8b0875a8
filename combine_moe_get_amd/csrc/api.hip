// api.hip -- the extern "C" entry points of libmoe_get: argument checks on
// the host, then kernel launches on the caller's stream.  Nothing here
// allocates or synchronizes; the only state is the per-device address of the
// static scratch of moe_get_layout_noalloc, looked up once per device.
//
// Shape limits come from the Constraints section of the CANN
// "low_latency_dispatch" page (K, BS, H, local_expert_num * ep_world_size)
// and its single-operator Example (num_experts a multiple of the rank count,
// checked before the call); the kernels add H % 8 == 0, H <= 8192 and at most
// 1024 special ids.
#include <string.h>

#include <mutex>

#include "moe_internal.hpp"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int n_special(const moe_get_shape_t *s) {
  return s->zero_expert_num + s->copy_expert_num + s->const_expert_num;
}

int check_shape(const moe_get_shape_t *s) {
  if (!s) return MOE_ERR_ARG;
  const int T = s->num_tokens, H = s->hidden, K = s->topk, E = s->num_experts, P = s->num_ranks;
  if (T < 0 || H <= 0 || P <= 0) return MOE_ERR_SHAPE;
  if (K <= 0 || K > 16) return MOE_ERR_SHAPE;
  if (E <= 0 || E % P != 0 || E > 2048) return MOE_ERR_SHAPE;
  if (s->zero_expert_num < 0 || s->copy_expert_num < 0 || s->const_expert_num < 0)
    return MOE_ERR_SHAPE;
  const int64_t etot = (int64_t)E + s->zero_expert_num + s->copy_expert_num + s->const_expert_num;
  if (etot >= INT32_MAX || K > etot) return MOE_ERR_SHAPE;
  if (T % P != 0) return MOE_ERR_SHAPE;
  const int BS = T / P;
  if (BS > 512) return MOE_ERR_SHAPE;
  if (s->num_max_dispatch_tokens_per_rank < 0) return MOE_ERR_SHAPE;
  if (s->num_max_dispatch_tokens_per_rank > 0 && BS > s->num_max_dispatch_tokens_per_rank)
    return MOE_ERR_CAPACITY;
  if (H % 8 != 0 || H > 8192) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)s->zero_expert_num + s->copy_expert_num + s->const_expert_num > 1024)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// workspace: [P m][E] per-sub-chunk expert counts | [P m][P] per-sub-chunk rank tokens |
// [P m][NS] per-sub-chunk specials | status word (m: sub-chunks per source rank)
struct WsLayout {
  size_t base, rank_tok, special, status, total;
};

WsLayout ws_layout(const moe_get_shape_t *s) {
  const size_t P = s->num_ranks, E = s->num_experts, NS = n_special(s);
  const size_t Pv = P * (size_t)layout_subchunks(s->num_tokens / s->num_ranks, s->num_experts, s->num_ranks);
  WsLayout w;
  w.base = 0;
  w.rank_tok = w.base + align_up(Pv * E * 4);
  w.special = w.rank_tok + align_up(Pv * P * 4);
  w.status = w.special + align_up(Pv * (NS > 0 ? NS : 1) * 4);
  w.total = w.status + kAlign;
  return w;
}

// ---- static scratch of the allocation-free layout entry point ------------------------------
// The workspace of moe_get_layout_noalloc: the per-sub-chunk count matrices that the two-launch
// layout's count kernel writes and its scan kernel reads, and the status word used when the caller
// passes none.  Every element the scan kernel reads is written first by the count kernel of the
// same call, so nothing has to be cleared between calls.  Each device holds its own copy for the life of
// the process; calls that overlap on one device share it and race.  In host code `scratch` names a
// host-side stand-in: kernels get the device address from hipGetSymbolAddress (scratch_on), never
// the name.
constexpr size_t kScratchBytes = (size_t)MOE_GET_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_addr[kMaxDevices];  // device address of `scratch` per device, looked up once

// device address of the scratch array on the device that runs `stream` (its first use on a device
// makes that device current for the lookup, then restores the caller's device)
int scratch_on(hipStream_t stream, void **out) {
  int cur = -1, dev = -1;
  if (hipGetDevice(&cur) != hipSuccess) return MOE_ERR_HIP;
  dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_addr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return MOE_ERR_HIP;
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return MOE_ERR_HIP;
    if (e != hipSuccess || !p || ((uintptr_t)p & (kAlign - 1)) != 0) return MOE_ERR_HIP;
    scratch_addr[dev] = p;
  }
  *out = scratch_addr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_get_abi_version(void) { return MOE_GET_ABI_VERSION; }

const char *moe_get_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument (NULL buffer, misaligned pointer, bad mode or small workspace)";
    case MOE_ERR_SHAPE: return "shape outside the operator constraints";
    case MOE_ERR_CAPACITY: return "tokens per rank exceed num_max_dispatch_tokens_per_rank";
    case MOE_ERR_UNSUPPORTED: return "shape not supported by the kernels (hidden % 8, hidden > 8192 or > 1024 special ids)";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_SCRATCH:
      return "the layout's workspace for this shape exceeds the static scratch of moe_get_layout_noalloc "
             "(MOE_GET_NOALLOC_SCRATCH_BYTES); use moe_get_layout_ex with a workspace";
    default: return "unknown status";
  }
}

int moe_get_check_shape(const moe_get_shape_t *shape) { return check_shape(shape); }

int64_t moe_get_recv_capacity(const moe_get_shape_t *shape) {
  if (check_shape(shape) != MOE_OK) return -1;
  return (int64_t)shape->num_tokens * shape->topk;
}

int64_t moe_get_rank_capacity(const moe_get_shape_t *shape) {
  if (check_shape(shape) != MOE_OK) return -1;
  const int64_t P = shape->num_ranks, BS = shape->num_tokens / shape->num_ranks;
  const int64_t nm = shape->num_max_dispatch_tokens_per_rank > 0 ? shape->num_max_dispatch_tokens_per_rank : BS;
  const int64_t L = shape->num_experts / P;
  return nm * P * (L < shape->topk ? L : shape->topk);
}

// the size fields of the layout kernels' arguments (pointers null)
static LayoutArgs layout_sizes(const moe_get_shape_t *shape) {
  LayoutArgs a;
  memset(&a, 0, sizeof a);
  const int T = shape->num_tokens, K = shape->topk, E = shape->num_experts, P = shape->num_ranks;
  const int NS = n_special(shape);
  a.T = T;
  a.K = K;
  a.E = E;
  a.P = P;
  a.BS = T / P;
  a.L = E / P;
  a.NS = NS;
  a.nbits = 32 - __builtin_clz((unsigned)E);  // bits of the sentinel key E
  a.Epad = E + (E & 1);
  const int S = a.BS * K;
  a.Spad = S + (S & 1);
  a.m = layout_subchunks(a.BS, E, P);
  a.BSv = a.BS > 0 ? (a.BS + a.m - 1) / a.m : 1;
  const int Sv = a.BSv * K;
  a.Svpad = Sv + (Sv & 1);
  a.Etot = (int64_t)E + NS;
  a.divL = div_magic(a.L);
  a.divK = div_magic(K);
  a.divBSv = div_magic(a.BSv);
  a.divE = div_magic(E);
  return a;
}

int moe_get_layout_launches(const moe_get_shape_t *shape) {
  const int st = check_shape(shape);
  if (st != MOE_OK) return st;
  return layout_launch_count(layout_sizes(shape));
}

size_t moe_get_workspace_size(const moe_get_shape_t *shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return ws_layout(shape).total;
}

int moe_get_layout(const moe_get_shape_t *shape, const int32_t *topk_idx,
                   const uint8_t *x_active_mask, int32_t *num_tokens_per_expert,
                   int32_t *expert_offsets, int32_t *recv_counts, int32_t *special_counts,
                   int32_t *num_tokens_per_rank, int32_t *rank_offsets,
                   uint8_t *is_token_in_rank, int32_t *dst_row, int32_t *src_info,
                   uint32_t *status_dev, void *workspace, size_t workspace_bytes, void *stream) {
  return moe_get_layout_ex(shape, 0, topk_idx, x_active_mask, num_tokens_per_expert, expert_offsets,
                           recv_counts, special_counts, num_tokens_per_rank, rank_offsets,
                           is_token_in_rank, dst_row, src_info, status_dev, workspace, workspace_bytes,
                           stream);
}

}  // extern "C"

namespace {

// checks of moe_get_layout_ex's arguments; fills the kernel argument block
int layout_args(const moe_get_shape_t *shape, int64_t rank_stride, const int32_t *topk_idx,
                const uint8_t *x_active_mask, int32_t *num_tokens_per_expert, int32_t *expert_offsets,
                int32_t *recv_counts, int32_t *special_counts, int32_t *num_tokens_per_rank,
                int32_t *rank_offsets, uint8_t *is_token_in_rank, int32_t *dst_row, int32_t *src_info,
                uint32_t *status_dev, void *workspace, size_t workspace_bytes, LayoutArgs &a) {
  const int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (rank_stride < 0) return MOE_ERR_ARG;
  if (rank_stride > 0 && (rank_stride < moe_get_rank_capacity(shape) ||
                          rank_stride * shape->num_ranks >= (int64_t)INT32_MAX))
    return MOE_ERR_CAPACITY;
  const int T = shape->num_tokens;
  const int NS = n_special(shape);
  if (!num_tokens_per_expert || !expert_offsets || !recv_counts || !num_tokens_per_rank ||
      !rank_offsets)
    return MOE_ERR_ARG;
  if (T > 0 && (!topk_idx || !is_token_in_rank || !dst_row || !src_info)) return MOE_ERR_ARG;
  if (NS > 0 && !special_counts) return MOE_ERR_ARG;
  const WsLayout w = ws_layout(shape);
  if (!workspace || workspace_bytes < w.total || ((uintptr_t)workspace & (kAlign - 1)) != 0)
    return MOE_ERR_ARG;

  a = layout_sizes(shape);
  a.topk_idx = topk_idx;
  a.mask = x_active_mask;
  a.rank_stride = rank_stride;
  a.cnt = num_tokens_per_expert;
  a.expert_offsets = expert_offsets;
  a.recv_counts = recv_counts;
  a.special_counts = special_counts;
  a.num_tokens_per_rank = num_tokens_per_rank;
  a.rank_offsets = rank_offsets;
  a.dst_row = dst_row;
  a.src_info = src_info;
  a.itr = is_token_in_rank;
  char *ws = (char *)workspace;
  a.ws_cnt_t = (int32_t *)(ws + w.base);
  a.ws_rank_tok = (int32_t *)(ws + w.rank_tok);
  a.ws_special = (int32_t *)(ws + w.special);
  a.status = status_dev ? status_dev : (uint32_t *)(ws + w.status);
  return MOE_OK;
}

// checks of moe_dispatch's arguments; fills the kernel argument block and says whether the
// scales are per expert
int dispatch_args(const moe_get_shape_t *shape, int32_t quant_mode, const uint16_t *x,
                  const float *x_smooth_scale, int32_t smooth_rows, const float *topk_weights,
                  const int32_t *topk_idx, const int32_t *dst_row, void *expand_x, float *dynamic_scales,
                  float *expand_weights, DispatchArgs &a, bool &per_expert) {
  const int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (quant_mode < 0 || quant_mode > 2) return MOE_ERR_ARG;
  const int T = shape->num_tokens, E = shape->num_experts;
  per_expert = false;
  const float *smooth = nullptr;
  if (quant_mode != 0) {
    if (smooth_rows != 0 && smooth_rows != 1 && smooth_rows != E) return MOE_ERR_ARG;
    if (smooth_rows > 0) {
      if (!x_smooth_scale || !aligned16(x_smooth_scale)) return MOE_ERR_ARG;
      smooth = x_smooth_scale;
      per_expert = smooth_rows > 1;
      if (per_expert && !topk_idx) return MOE_ERR_ARG;
    }
  }
  memset(&a, 0, sizeof a);
  if (T > 0) {
    if (!x || !dst_row || !expand_x) return MOE_ERR_ARG;
    if (!aligned16(x) || !aligned16(expand_x)) return MOE_ERR_ARG;
  }
  a.x = x;
  a.smooth = smooth;
  a.w = topk_weights;
  a.topk_idx = topk_idx;
  a.dst_row = dst_row;
  a.expand_x = expand_x;
  a.dyn_scales = quant_mode == 2 ? dynamic_scales : nullptr;
  a.expand_w = expand_weights;
  a.T = T;
  a.H = shape->hidden;
  a.K = shape->topk;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_get_layout_ex(const moe_get_shape_t *shape, int64_t rank_stride, const int32_t *topk_idx,
                      const uint8_t *x_active_mask, int32_t *num_tokens_per_expert,
                      int32_t *expert_offsets, int32_t *recv_counts, int32_t *special_counts,
                      int32_t *num_tokens_per_rank, int32_t *rank_offsets,
                      uint8_t *is_token_in_rank, int32_t *dst_row, int32_t *src_info,
                      uint32_t *status_dev, void *workspace, size_t workspace_bytes, void *stream) {
  LayoutArgs a;
  const int st = layout_args(shape, rank_stride, topk_idx, x_active_mask, num_tokens_per_expert, expert_offsets,
                             recv_counts, special_counts, num_tokens_per_rank, rank_offsets, is_token_in_rank,
                             dst_row, src_info, status_dev, workspace, workspace_bytes, a);
  if (st != MOE_OK) return st;
  return launch_layout(a, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_get_layout_noalloc(const moe_get_shape_t *shape, int64_t rank_stride, const int32_t *topk_idx,
                           const uint8_t *x_active_mask, int32_t *num_tokens_per_expert,
                           int32_t *expert_offsets, int32_t *recv_counts, int32_t *special_counts,
                           int32_t *num_tokens_per_rank, int32_t *rank_offsets,
                           uint8_t *is_token_in_rank, int32_t *dst_row, int32_t *src_info,
                           uint32_t *status_dev, void *stream) {
  const int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (ws_layout(shape).total > kScratchBytes) return MOE_ERR_SCRATCH;
  // every argument is checked before the runtime is asked for anything (an aligned stand-in for
  // the scratch address first, then the real one)
  LayoutArgs a;
  int ast = layout_args(shape, rank_stride, topk_idx, x_active_mask, num_tokens_per_expert, expert_offsets,
                        recv_counts, special_counts, num_tokens_per_rank, rank_offsets, is_token_in_rank, dst_row,
                        src_info, status_dev, (void *)kAlign, kScratchBytes, a);
  if (ast != MOE_OK) return ast;
  void *ws = nullptr;
  const int sst = scratch_on((hipStream_t)stream, &ws);
  if (sst != MOE_OK) return sst;
  ast = layout_args(shape, rank_stride, topk_idx, x_active_mask, num_tokens_per_expert, expert_offsets, recv_counts,
                    special_counts, num_tokens_per_rank, rank_offsets, is_token_in_rank, dst_row, src_info,
                    status_dev, ws, kScratchBytes, a);
  if (ast != MOE_OK) return ast;
  return launch_layout(a, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

size_t moe_get_noalloc_scratch_bytes(void) { return kScratchBytes; }

int moe_dispatch(const moe_get_shape_t *shape, int32_t quant_mode, const uint16_t *x,
                 const float *x_smooth_scale, int32_t smooth_rows, const float *topk_weights,
                 const int32_t *topk_idx, const int32_t *dst_row, void *expand_x,
                 float *dynamic_scales, float *expand_weights, void *stream) {
  return moe_dispatch_capped(shape, 0, quant_mode, x, x_smooth_scale, smooth_rows, topk_weights, topk_idx, dst_row,
                             expand_x, dynamic_scales, expand_weights, stream);
}

int moe_dispatch_capped(const moe_get_shape_t *shape, int32_t max_workgroups, int32_t quant_mode, const uint16_t *x,
                        const float *x_smooth_scale, int32_t smooth_rows, const float *topk_weights,
                        const int32_t *topk_idx, const int32_t *dst_row, void *expand_x, float *dynamic_scales,
                        float *expand_weights, void *stream) {
  if (max_workgroups < 0) return MOE_ERR_ARG;
  DispatchArgs a;
  bool per_expert = false;
  const int st = dispatch_args(shape, quant_mode, x, x_smooth_scale, smooth_rows, topk_weights, topk_idx, dst_row,
                               expand_x, dynamic_scales, expand_weights, a, per_expert);
  if (st != MOE_OK) return st;
  if (a.T == 0) return MOE_OK;
  return launch_dispatch(a, quant_mode, per_expert, (hipStream_t)stream, max_workgroups) == hipSuccess ? MOE_OK
                                                                                                      : MOE_ERR_HIP;
}

int moe_layout_dispatch(const moe_get_shape_t *shape, int64_t rank_stride, int32_t quant_mode,
                        const int32_t *topk_idx, const uint8_t *x_active_mask, const uint16_t *x,
                        const float *x_smooth_scale, int32_t smooth_rows, const float *topk_weights,
                        int32_t *num_tokens_per_expert, int32_t *expert_offsets, int32_t *recv_counts,
                        int32_t *special_counts, int32_t *num_tokens_per_rank, int32_t *rank_offsets,
                        uint8_t *is_token_in_rank, int32_t *dst_row, int32_t *src_info, void *expand_x,
                        float *dynamic_scales, float *expand_weights, uint32_t *status_dev, void *workspace,
                        size_t workspace_bytes, void *stream) {
  LayoutArgs la;
  int st = layout_args(shape, rank_stride, topk_idx, x_active_mask, num_tokens_per_expert, expert_offsets,
                       recv_counts, special_counts, num_tokens_per_rank, rank_offsets, is_token_in_rank, dst_row,
                       src_info, status_dev, workspace, workspace_bytes, la);
  if (st != MOE_OK) return st;
  DispatchArgs da;
  bool per_expert = false;
  st = dispatch_args(shape, quant_mode, x, x_smooth_scale, smooth_rows, topk_weights, topk_idx, dst_row, expand_x,
                     dynamic_scales, expand_weights, da, per_expert);
  if (st != MOE_OK) return st;
  return launch_layout_dispatch(la, da, quant_mode, per_expert, (hipStream_t)stream) == hipSuccess ? MOE_OK
                                                                                                  : MOE_ERR_HIP;
}

int moe_layout_dispatch_launches(const moe_get_shape_t *shape, int32_t quant_mode) {
  const int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (quant_mode < 0 || quant_mode > 2) return MOE_ERR_ARG;
  return layout_dispatch_launch_count(layout_sizes(shape), quant_mode,
                                      (int64_t)shape->num_tokens * shape->hidden * 2);
}

int moe_combine(const moe_get_shape_t *shape, const uint16_t *expert_out,
                const int32_t *topk_idx, const float *topk_weights,
                const uint8_t *x_active_mask, const int32_t *dst_row, const uint16_t *ori_x,
                const uint16_t *const_alpha1, const uint16_t *const_alpha2,
                const uint16_t *const_v, uint16_t *out, void *stream) {
  return moe_combine_capped(shape, 0, expert_out, topk_idx, topk_weights, x_active_mask, dst_row, ori_x,
                            const_alpha1, const_alpha2, const_v, out, stream);
}

int moe_combine_capped(const moe_get_shape_t *shape, int32_t max_workgroups, const uint16_t *expert_out,
                       const int32_t *topk_idx, const float *topk_weights, const uint8_t *x_active_mask,
                       const int32_t *dst_row, const uint16_t *ori_x, const uint16_t *const_alpha1,
                       const uint16_t *const_alpha2, const uint16_t *const_v, uint16_t *out, void *stream) {
  if (max_workgroups < 0) return MOE_ERR_ARG;
  const int st = check_shape(shape);
  if (st != MOE_OK) return st;
  const int T = shape->num_tokens;
  const int C = shape->copy_expert_num, Kc = shape->const_expert_num;
  if (T == 0) return MOE_OK;
  if (!expert_out || !topk_idx || !topk_weights || !dst_row || !out) return MOE_ERR_ARG;
  if (!aligned16(expert_out) || !aligned16(out)) return MOE_ERR_ARG;
  if (C + Kc > 0 && (!ori_x || !aligned16(ori_x))) return MOE_ERR_ARG;
  if (Kc > 0 && (!const_alpha1 || !const_alpha2 || !const_v || !aligned16(const_alpha1) ||
                 !aligned16(const_alpha2) || !aligned16(const_v)))
    return MOE_ERR_ARG;

  CombineArgs a;
  a.y = expert_out;
  a.topk_idx = topk_idx;
  a.w = topk_weights;
  a.mask = x_active_mask;
  a.dst_row = dst_row;
  a.ori_x = ori_x;
  a.a1 = const_alpha1;
  a.a2 = const_alpha2;
  a.cv = const_v;
  a.out = out;
  a.T = T;
  a.H = shape->hidden;
  a.K = shape->topk;
  a.E = shape->num_experts;
  a.Z = shape->zero_expert_num;
  a.C = C;
  a.Kc = Kc;
  return launch_combine(a, (hipStream_t)stream, max_workgroups) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
