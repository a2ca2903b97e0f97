// C-ABI entry points of libfa: argument validation, status text, dispatch to the kernels.
// The operation and the argument contract are documented in include/fa.h.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "fa.h"
#include "fa_launch.h"

namespace {

thread_local const char* g_last_hip_error = "no HIP error recorded";

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Strides are element counts for (batch, head, token). All must be non-negative multiples of
// 8 (16-byte rows); token rows may not overlap, and a token stride is at most 2^23 elements so
// that the byte extent of one 64-row K/V tile fits a 32-bit buffer range.
// a * b * c > limit, for non-negative factors, without overflowing int64.
bool product_exceeds(int64_t a, int64_t b, int64_t c, int64_t limit) {
  if (a == 0 || b == 0 || c == 0) return false;
  if (a > limit / b) return true;
  return a * b > limit / c;
}

bool stride_ok(const int64_t s[3], int32_t head_dim, int32_t seqlen, int64_t multiple = 8) {
  for (int i = 0; i < 3; ++i)
    if (s[i] < 0 || s[i] % multiple != 0) return false;
  if (seqlen > 1 && (s[2] < head_dim || s[2] > (int64_t(1) << 23))) return false;
  return true;
}

}  // namespace

extern "C" {

int32_t fa_abi_version(void) { return FA_ABI_VERSION; }

uint32_t fa_params_size(void) { return static_cast<uint32_t>(sizeof(fa_fwd_params)); }

fa_status fa_check_args(const fa_fwd_params* p) {
  if (p == nullptr) return FA_ERR_NULL;
  if (p->struct_size != sizeof(fa_fwd_params)) return FA_ERR_ABI;
  if (p->dtype != FA_F16 && p->dtype != FA_BF16 && p->dtype != FA_E4M3) return FA_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(p->scale)) return FA_ERR_UNSUPPORTED;
  if (p->dtype == FA_E4M3 && p->rope_cos != nullptr) return FA_ERR_UNSUPPORTED;
  if (p->batch < 1 || p->heads_q < 1 || p->heads_kv < 1 || p->seqlen < 0 || p->seqlen_k < 0 ||
      p->reserved0 != 0)
    return FA_ERR_SHAPE;
  if (p->heads_q % p->heads_kv != 0) return FA_ERR_GQA;
  if (p->cu_seqlens != nullptr) {
    if (p->batch != 1 || p->num_seqs < 1) return FA_ERR_VARLEN;
    if (p->max_seqlen < 0 || p->max_seqlen > p->seqlen) return FA_ERR_VARLEN;
    if (p->seqlen > 0 && p->max_seqlen < 1) return FA_ERR_VARLEN;
    if (p->cu_seqlens_k == nullptr && p->seqlen_k != p->seqlen) return FA_ERR_VARLEN;
  } else if (p->cu_seqlens_k != nullptr) {
    return FA_ERR_VARLEN;
  }
  if (p->seqlen == 0) return FA_OK;
  // k and v may be NULL only when there are no keys at all
  if (!p->q || !p->o || !p->lse || (p->seqlen_k > 0 && (!p->k || !p->v))) return FA_ERR_NULL;
  if (!aligned16(p->q) || !aligned16(p->k) || !aligned16(p->v) || !aligned16(p->o))
    return FA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(p->lse) & 3u) != 0) return FA_ERR_ALIGN;
  const int64_t in_multiple = p->dtype == FA_E4M3 ? 16 : 8;  // 16-byte rows
  if (!stride_ok(p->q_stride, p->head_dim, p->seqlen, in_multiple) ||
      !stride_ok(p->k_stride, p->head_dim, p->seqlen_k, in_multiple) ||
      !stride_ok(p->v_stride, p->head_dim, p->seqlen_k, in_multiple) ||
      !stride_ok(p->o_stride, p->head_dim, p->seqlen))
    return FA_ERR_ALIGN;
  const float* descales[] = {p->q_descale, p->k_descale, p->v_descale};
  for (const float* d : descales)
    if (d != nullptr && (reinterpret_cast<uintptr_t>(d) & 3u) != 0) return FA_ERR_ALIGN;
  if ((p->rope_cos == nullptr) != (p->rope_sin == nullptr)) return FA_ERR_NULL;
  if (p->rope_cos == nullptr) {
    if (p->k_rot != nullptr) return FA_ERR_NULL;
  } else {
    if (!aligned16(p->rope_cos) || !aligned16(p->rope_sin)) return FA_ERR_ALIGN;
    if (p->rope_rows < 1) return FA_ERR_SHAPE;
    if (p->cu_seqlens == nullptr && p->rope_rows < p->seqlen_k) return FA_ERR_SHAPE;
    if (p->k_rot != nullptr &&
        (!aligned16(p->k_rot) || !stride_ok(p->k_rot_stride, p->head_dim, p->seqlen_k)))
      return FA_ERR_ALIGN;
    // the key rotation runs one thread per 16 head-dims of every key row
    if (p->k_rot != nullptr &&
        product_exceeds(p->batch, p->heads_kv, p->seqlen_k, int64_t(UINT32_MAX) * 16))
      return FA_ERR_SHAPE;
  }
  // The kernel runs one workgroup per (256 query rows, query head, batch entry or sequence);
  // the bound below counts 128-row blocks, so it is conservative.
  const int64_t rows = p->cu_seqlens ? p->max_seqlen : p->seqlen;
  const int64_t groups = p->cu_seqlens ? p->num_seqs : p->batch;
  if (product_exceeds((rows + 127) / 128, p->heads_q, groups, INT32_MAX)) return FA_ERR_SHAPE;
  // element counts of Q/O/LSE and of K/V stay far inside int64
  if (product_exceeds(p->batch, p->heads_q, p->seqlen, INT64_MAX / 4)) return FA_ERR_SHAPE;
  if (product_exceeds(p->batch, p->heads_kv, p->seqlen_k, INT64_MAX / 4)) return FA_ERR_SHAPE;
  return FA_OK;
}

fa_status fa_fwd(const fa_fwd_params* p, void* stream) {
  const fa_status st = fa_check_args(p);
  if (st != FA_OK) return st;
  if (p->seqlen == 0) return FA_OK;
  if (p->cu_seqlens != nullptr && p->max_seqlen == 0) return FA_OK;
  const char* err = nullptr;
  const fa_status ls = p->dtype == FA_E4M3 ? fa::launch_forward_fp8(*p, stream, &err)
                                           : fa::launch_forward(*p, stream, &err);
  if (ls != FA_OK && err != nullptr) g_last_hip_error = err;
  return ls;
}

namespace {

// The split-KV plan for validated arguments, or FA_ERR_SHAPE when a grid would not fit.
fa_status checked_plan(const fa_fwd_params* p, int32_t num_splits, fa::SplitPlan* plan) {
  const fa_status st = fa_check_args(p);
  if (st != FA_OK) return st;
  if (p->dtype == FA_E4M3) return FA_ERR_UNSUPPORTED;
  if (num_splits < 0 || num_splits > FA_MAX_SPLITS) return FA_ERR_SHAPE;
  *plan = fa::plan_splitkv(*p, num_splits);
  if (plan->grid > INT32_MAX || (plan->rows_total + 3) / 4 > INT32_MAX) return FA_ERR_SHAPE;
  return FA_OK;
}

}  // namespace

fa_status fa_splitkv_plan(const fa_fwd_params* p, int32_t num_splits, int32_t* splits,
                          uint64_t* workspace_bytes) {
  fa::SplitPlan plan;
  const fa_status st = checked_plan(p, num_splits, &plan);
  if (st != FA_OK) return st;
  if (splits != nullptr) *splits = plan.splits;
  if (workspace_bytes != nullptr) *workspace_bytes = plan.workspace_bytes;
  return FA_OK;
}

fa_status fa_fwd_splitkv(const fa_fwd_params* p, int32_t num_splits, void* workspace,
                         uint64_t workspace_bytes, void* stream) {
  fa::SplitPlan plan;
  const fa_status st = checked_plan(p, num_splits, &plan);
  if (st != FA_OK) return st;
  if (plan.workspace_bytes > 0) {
    if (workspace == nullptr) return FA_ERR_NULL;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
    if (workspace_bytes < plan.workspace_bytes) return FA_ERR_SHAPE;
  }
  if (p->seqlen == 0) return FA_OK;
  if (p->cu_seqlens != nullptr && p->max_seqlen == 0) return FA_OK;
  const char* err = nullptr;
  const fa_status ls = fa::launch_forward_splitkv(*p, plan, workspace, stream, &err);
  if (ls != FA_OK && err != nullptr) g_last_hip_error = err;
  return ls;
}

fa_status fa_fwd_splitkv_noalloc(const fa_fwd_params* p, int32_t num_splits, void* stream) {
  fa::SplitPlan plan;
  const fa_status st = checked_plan(p, num_splits, &plan);
  if (st != FA_OK) return st;
  if (plan.workspace_bytes > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  if (p->seqlen == 0) return FA_OK;
  if (p->cu_seqlens != nullptr && p->max_seqlen == 0) return FA_OK;
  const char* err = nullptr;
  void* ws = nullptr;
  if (plan.workspace_bytes > 0) {
    ws = fa::noalloc_scratch(&err);
    if (ws == nullptr) {
      g_last_hip_error = err;
      return FA_ERR_LAUNCH;
    }
  }
  const fa_status ls = fa::launch_forward_splitkv(*p, plan, ws, stream, &err);
  if (ls != FA_OK && err != nullptr) g_last_hip_error = err;
  return ls;
}

uint32_t fa_bwd_params_size(void) { return static_cast<uint32_t>(sizeof(fa_bwd_params)); }

fa_status fa_bwd_check_args(const fa_bwd_params* p) {
  if (p == nullptr) return FA_ERR_NULL;
  if (p->struct_size != sizeof(fa_bwd_params)) return FA_ERR_ABI;
  if (p->dtype != FA_F16 && p->dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(p->scale)) return FA_ERR_UNSUPPORTED;
  if (p->batch < 1 || p->heads_q < 1 || p->heads_kv < 1 || p->seqlen < 0 || p->reserved0 != 0)
    return FA_ERR_SHAPE;
  if (p->heads_q % p->heads_kv != 0) return FA_ERR_GQA;
  if (p->cu_seqlens != nullptr) {
    if (p->batch != 1 || p->num_seqs < 1) return FA_ERR_VARLEN;
    if (p->max_seqlen < 0 || p->max_seqlen > p->seqlen) return FA_ERR_VARLEN;
    if (p->seqlen > 0 && p->max_seqlen < 1) return FA_ERR_VARLEN;
  }
  if (p->seqlen == 0) return FA_OK;
  const void* ptrs[] = {p->q, p->k, p->v, p->o, p->dout, p->dq, p->dk, p->dv};
  for (const void* t : ptrs) {
    if (t == nullptr) return FA_ERR_NULL;
    if (!aligned16(t)) return FA_ERR_ALIGN;
  }
  if (!p->lse || !p->delta) return FA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(p->lse) & 3u) || (reinterpret_cast<uintptr_t>(p->delta) & 3u))
    return FA_ERR_ALIGN;
  const int64_t* strides[] = {p->q_stride, p->k_stride, p->v_stride, p->o_stride,
                              p->do_stride, p->dq_stride, p->dk_stride, p->dv_stride};
  for (const int64_t* st : strides)
    if (!stride_ok(st, p->head_dim, p->seqlen)) return FA_ERR_ALIGN;
  const int64_t rows = p->cu_seqlens ? p->max_seqlen : p->seqlen;
  const int64_t groups = p->cu_seqlens ? p->num_seqs : p->batch;
  if (product_exceeds((rows + 127) / 128, p->heads_q, groups, INT32_MAX)) return FA_ERR_SHAPE;
  if (product_exceeds(p->batch, p->heads_q, p->seqlen, INT32_MAX - 16)) return FA_ERR_SHAPE;
  return FA_OK;
}

fa_status fa_bwd(const fa_bwd_params* p, void* stream) {
  const fa_status st = fa_bwd_check_args(p);
  if (st != FA_OK) return st;
  if (p->seqlen == 0) return FA_OK;
  if (p->cu_seqlens != nullptr && p->max_seqlen == 0) return FA_OK;
  const char* err = nullptr;
  const fa_status ls = fa::launch_backward(*p, stream, &err);
  if (ls != FA_OK && err != nullptr) g_last_hip_error = err;
  return ls;
}

const char* fa_status_string(int32_t status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: a size is out of range";
    case FA_ERR_UNSUPPORTED:
      return "FA_ERR_UNSUPPORTED: head_dim must be 64 or 128, dtype FA_F16, FA_BF16 or FA_E4M3, "
             "scale finite; FA_E4M3 takes no RoPE tables and no split-KV";
    case FA_ERR_ALIGN:
      return "FA_ERR_ALIGN: base pointers must be 16-byte aligned, strides non-negative "
             "multiples of 8 elements, token strides in [head_dim, 2^23]";
    case FA_ERR_GQA: return "FA_ERR_GQA: heads_q must be a multiple of heads_kv";
    case FA_ERR_VARLEN:
      return "FA_ERR_VARLEN: cu_seqlens needs batch == 1, num_seqs >= 1 and "
             "1 <= max_seqlen <= seqlen; cu_seqlens_k needs cu_seqlens, and packed keys of "
             "another total length need cu_seqlens_k";
    case FA_ERR_ABI: return "FA_ERR_ABI: struct_size does not match sizeof(fa_fwd_params)";
    case FA_ERR_LAUNCH: return g_last_hip_error;
    case FA_ERR_SCRATCH:
      return "FA_ERR_SCRATCH: the split partials need more than the library's static scratch "
             "(FA_NOALLOC_SCRATCH_BYTES = 16 MiB); use fa_fwd_splitkv with a workspace, or "
             "fewer splits";
    default: return "unknown fa_status";
  }
}

}  // extern "C"
