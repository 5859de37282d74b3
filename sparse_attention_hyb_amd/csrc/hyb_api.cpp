// C-ABI front end: argument validation (host only, before any HIP call), workspace sizing and
// dispatch to the kernel launchers. Declarations, argument meaning and error behaviour are in
// include/hyb.h.
#include "hyb.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "hyb_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int launch_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return HYB_OK;
  return fail(HYB_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
}

bool is_plain(int32_t dt) { return dt == HYB_F32 || dt == HYB_BF16; }

int64_t entry_bytes(int32_t dtype, int32_t dim) {
  switch (dtype) {
    case HYB_F32: return 4LL * dim;
    case HYB_BF16: return 2LL * dim;
    case HYB_FP8_E4M3: return dim;
    case HYB_FP4_E2M1: return dim / 2;
    default: return 0;
  }
}

// Pool descriptor checks. ratio_mask bit 0: ratio 1, bit 1: ratio 4, bit 2: ratio 128.
int check_pool(const hyb_paged* p, const char* op, const char* name, bool fp8_ok, bool fp4_ok,
               int ratio_mask, hyb::PoolDev* out) {
  if (!p) return fail(HYB_EINVAL, "%s: %s descriptor is NULL", op, name);
  if (!p->data) return fail(HYB_EINVAL, "%s: %s.data is NULL", op, name);
  if (!p->block_table) return fail(HYB_EINVAL, "%s: %s.block_table is NULL", op, name);
  if (p->reserved != 0) return fail(HYB_EINVAL, "%s: %s.reserved must be 0", op, name);
  const int r = p->ratio;
  const int bit = r == 1 ? 1 : (r == 4 ? 2 : (r == 128 ? 4 : 0));
  if (!(bit & ratio_mask)) return fail(HYB_EINVAL, "%s: %s.ratio %d not allowed here", op, name, r);
  if (p->dim <= 0 || p->dim % 2) return fail(HYB_EINVAL, "%s: %s.dim %d must be positive and even", op, name, p->dim);
  if (p->num_blocks <= 0 || p->max_blocks <= 0)
    return fail(HYB_EINVAL, "%s: %s needs num_blocks > 0 and max_blocks > 0", op, name);
  if ((int64_t)p->num_blocks * (HYB_BLOCK_POSITIONS / (r > 0 ? r : 1)) >= (1LL << 31))
    return fail(HYB_EINVAL, "%s: %s holds 2^31 entries or more", op, name);
  switch (p->dtype) {
    case HYB_F32:
    case HYB_BF16:
      break;
    case HYB_FP8_E4M3:
      if (!fp8_ok) return fail(HYB_ENOTSUP, "%s: %s dtype FP8_E4M3 not supported here", op, name);
      if (!p->scale) return fail(HYB_EINVAL, "%s: %s.scale is NULL for FP8_E4M3", op, name);
      break;
    case HYB_FP4_E2M1:
      if (!fp4_ok) return fail(HYB_ENOTSUP, "%s: %s dtype FP4_E2M1 not supported here", op, name);
      if (!p->scale) return fail(HYB_EINVAL, "%s: %s.scale is NULL for FP4_E2M1", op, name);
      if (p->dim % 32) return fail(HYB_EINVAL, "%s: %s.dim %d must be a multiple of 32 for FP4_E2M1", op, name, p->dim);
      break;
    default:
      return fail(HYB_EINVAL, "%s: %s.dtype %d unknown", op, name, p->dtype);
  }
  out->data = static_cast<uint8_t*>(p->data);
  out->scale = p->scale;
  out->block_table = p->block_table;
  out->dtype = p->dtype;
  out->dim = p->dim;
  out->ratio = r;
  out->num_blocks = p->num_blocks;
  out->max_blocks = p->max_blocks;
  out->per_block = HYB_BLOCK_POSITIONS / r;
  out->entry_bytes = entry_bytes(p->dtype, p->dim);
  return HYB_OK;
}

int check_rope(const char* op, int32_t rope_dim, double base, int32_t dim) {
  if (rope_dim < 0 || rope_dim % 2 || rope_dim > dim)
    return fail(HYB_EINVAL, "%s: rope_dim %d must be even and within [0, dim=%d]", op, rope_dim, dim);
  if (rope_dim > 128) return fail(HYB_ENOTSUP, "%s: rope_dim %d > 128", op, rope_dim);
  if (!(base > 0.0) || !std::isfinite(base)) return fail(HYB_EINVAL, "%s: rope_base must be positive", op);
  return HYB_OK;
}

// RoPE frequencies base^(-2i / rope_dim) for the compressor kernels (rope_dim <= 128).
void fill_theta(hyb::CompressArgs* a, int32_t rope_dim, double base) {
  for (int i = 0; i < rope_dim / 2; ++i)
    a->theta[i] = std::exp(-2.0 * (double)i / (double)rope_dim * std::log(base));
}

int64_t visible(int64_t p, int64_t ratio, int64_t window) {
  int64_t ws = p - window + 1;
  if (ws < 0) ws = 0;
  return (ws + ratio - 1) / ratio;
}

size_t score_ld(int32_t max_pos, int32_t window, int32_t ratio) {
  int64_t nv = visible(max_pos, ratio, window);
  if (nv < 1) nv = 1;
  return (size_t)((nv + 63) / 64 * 64);
}

#define HYB_TRY(expr)          \
  do {                         \
    int _st = (expr);          \
    if (_st != HYB_OK) return _st; \
  } while (0)

int check_compress_common(const char* op, const void* x, int32_t x_dtype,
                          const int32_t* cu_seqlens, const int32_t* start_pos, int32_t batch,
                          int32_t max_new_tokens) {
  if (batch < 0) return fail(HYB_EINVAL, "%s: batch %d < 0", op, batch);
  if (max_new_tokens < 0) return fail(HYB_EINVAL, "%s: max_new_tokens %d < 0", op, max_new_tokens);
  if (!x || !cu_seqlens || !start_pos) return fail(HYB_EINVAL, "%s: x, cu_seqlens and start_pos must be non-NULL", op);
  if (!is_plain(x_dtype)) return fail(HYB_ENOTSUP, "%s: x_dtype must be F32 or BF16", op);
  return HYB_OK;
}

int check_compress(const char* op, const hyb_compress_call& c, hyb::CompressArgs* a) {
  HYB_TRY(check_compress_common(op, c.x, c.x_dtype, c.cu_seqlens, c.start_pos, c.batch,
                                c.max_new_tokens));
  if (!c.state) return fail(HYB_EINVAL, "%s: state is NULL", op);
  if (c.mode != HYB_POOL_MEAN && c.mode != HYB_POOL_SOFTMAX_GATE)
    return fail(HYB_EINVAL, "%s: mode %d unknown", op, c.mode);
  if (c.mode == HYB_POOL_SOFTMAX_GATE && (!c.gate_logits || !c.state_logits))
    return fail(HYB_EINVAL, "%s: softmax-gate pooling needs gate_logits and state_logits", op);
  if (!(c.eps >= 0.f) || !std::isfinite(c.eps)) return fail(HYB_EINVAL, "%s: eps must be >= 0", op);
  hyb::PoolDev po{};
  HYB_TRY(check_pool(c.out, op, "out", true, true, 2 | 4, &po));
  if (po.dim > 2048) return fail(HYB_ENOTSUP, "%s: dim %d > 2048", op, po.dim);
  HYB_TRY(check_rope(op, c.rope_dim, c.rope_base, po.dim));
  *a = hyb::CompressArgs{c.x, c.x_dtype, c.gate_logits, c.cu_seqlens, c.start_pos, c.batch,
                         c.max_new_tokens, c.state, c.state_logits, c.mode, po, c.rope_dim,
                         c.rope_base, c.eps, {}};
  fill_theta(a, c.rope_dim, c.rope_base);
  return HYB_OK;
}

struct AttnCommon {
  hyb::AttnArgs args;
  hyb::AttnPlan plan;
};

int check_attention(const char* op, const void* q, int32_t q_dtype, int32_t n_q, int32_t n_heads,
                    const hyb_paged* swa, const hyb_paged* comp, const int32_t* topk_idx,
                    int32_t k, int32_t window, float softmax_scale, int32_t rope_dim,
                    double rope_base, void* out, int32_t out_dtype, float* out_scale,
                    int64_t max_pos, AttnCommon* c) {
  if (!q || !out) return fail(HYB_EINVAL, "%s: q and out must be non-NULL", op);
  if (n_q < 0) return fail(HYB_EINVAL, "%s: query count %d < 0", op, n_q);
  if (n_heads <= 0 || n_heads > 128) return fail(HYB_EINVAL, "%s: n_heads %d outside [1, 128]", op, n_heads);
  const bool fp8_out = out_dtype == HYB_FP8_E4M3;
  if (!is_plain(q_dtype) || !(is_plain(out_dtype) || fp8_out))
    return fail(HYB_ENOTSUP, "%s: q_dtype must be F32 or BF16, out_dtype F32, BF16 or FP8_E4M3", op);
  if (fp8_out != (out_scale != nullptr))
    return fail(HYB_EINVAL, "%s: out_scale is required with an FP8_E4M3 output and must be NULL "
                "otherwise", op);
  if (window <= 0) return fail(HYB_EINVAL, "%s: window %d must be positive", op, window);
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(HYB_EINVAL, "%s: softmax_scale must be positive and finite", op);
  hyb::PoolDev ps{}, pc{};
  HYB_TRY(check_pool(swa, op, "swa", true, false, 1, &ps));
  HYB_TRY(check_pool(comp, op, "comp", true, false, 2 | 4, &pc));
  if (ps.dim != pc.dim) return fail(HYB_EINVAL, "%s: swa.dim %d != comp.dim %d", op, ps.dim, pc.dim);
  if (ps.dtype != pc.dtype) return fail(HYB_EINVAL, "%s: swa and comp must share one dtype", op);
  if (ps.dtype == HYB_FP8_E4M3 && q_dtype != HYB_BF16)
    return fail(HYB_ENOTSUP, "%s: FP8_E4M3 pools need a BF16 query", op);
  if (topk_idx && (k < 1 || k > HYB_KMAX)) return fail(HYB_EINVAL, "%s: k %d outside [1, %d]", op, k, HYB_KMAX);
  HYB_TRY(check_rope(op, rope_dim, rope_base, ps.dim));
  const int dim = ps.dim;
  if (fp8_out && (dim % 8 || dim > 2048))
    return fail(HYB_ENOTSUP, "%s: an FP8_E4M3 output needs dim %% 8 == 0 and dim <= 2048", op);
  const int64_t n_win = max_pos + 1 < window ? max_pos + 1 : window;
  const int64_t n_comp = topk_idx ? k : visible(max_pos, pc.ratio, window);
  const int64_t max_keys = n_win + n_comp;
  if (max_keys > (1LL << 30)) return fail(HYB_EINVAL, "%s: too many keys per query", op);
  c->plan = hyb::plan_attention(n_q, n_heads, dim, (int32_t)max_keys, q_dtype, ps.dtype);
  if (!c->plan.use_mfma && ((int64_t)n_heads * dim > 4096 || n_heads > 64))
    return fail(HYB_ENOTSUP, "%s: heads x dim = %d x %d needs the 64 x 512 bf16 kernel (bf16 query, bf16/fp8 pools)",
                op, n_heads, dim);
  hyb::AttnArgs& a = c->args;
  a = hyb::AttnArgs{};
  a.q = q;
  a.q_dtype = q_dtype;
  a.n_q = n_q;
  a.n_heads = n_heads;
  a.dim = dim;
  a.swa = ps;
  a.comp = pc;
  a.topk = topk_idx;
  a.k = topk_idx ? k : 0;
  a.window = window;
  a.scale = softmax_scale;
  a.rope_dim = rope_dim;
  a.rope_base = rope_base;
  a.out = out;
  a.out_dtype = out_dtype;
  a.out_scale = out_scale;
  a.max_keys = (int32_t)max_keys;
  a.n_split = c->plan.n_split;
  a.chunk = c->plan.chunk;
  a.use_mfma = c->plan.use_mfma;
  return HYB_OK;
}

int attach_workspace(const char* op, AttnCommon* c, void* ws, size_t ws_bytes) {
  if (c->plan.ws_bytes > 0 && (!ws || ws_bytes < c->plan.ws_bytes))
    return fail(HYB_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", op, c->plan.ws_bytes,
                ws ? ws_bytes : (size_t)0);
  c->args.part_o = ws;
  c->args.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + c->plan.o_bytes);
  return HYB_OK;
}

size_t attn_ws(int32_t n_q, int32_t n_heads, int32_t dim, int64_t max_pos, int32_t ratio,
               int32_t k, int32_t window, int32_t dtype_hint) {
  if (n_q <= 0 || n_heads <= 0 || dim <= 0 || window <= 0 || max_pos < 0 ||
      (ratio != 4 && ratio != 128))
    return 0;
  const int64_t n_win = max_pos + 1 < window ? max_pos + 1 : window;
  const int64_t n_comp = k > 0 ? k : visible(max_pos, ratio, window);
  // the plan depends on whether the MFMA kernel runs; size for the larger of the two plans
  hyb::AttnPlan a = hyb::plan_attention(n_q, n_heads, dim, (int32_t)(n_win + n_comp), HYB_BF16, HYB_BF16);
  hyb::AttnPlan b = hyb::plan_attention(n_q, n_heads, dim, (int32_t)(n_win + n_comp), HYB_F32, HYB_F32);
  (void)dtype_hint;
  return a.ws_bytes > b.ws_bytes ? a.ws_bytes : b.ws_bytes;
}

}  // namespace

extern "C" {

int32_t hyb_abi_version(void) { return HYB_ABI_VERSION; }

const char* hyb_status_str(int32_t status) {
  switch (status) {
    case HYB_OK: return "HYB_OK";
    case HYB_EINVAL: return "HYB_EINVAL";
    case HYB_ENOTSUP: return "HYB_ENOTSUP";
    case HYB_EWORKSPACE: return "HYB_EWORKSPACE";
    case HYB_ELAUNCH: return "HYB_ELAUNCH";
    default: return "HYB_UNKNOWN";
  }
}

const char* hyb_last_error(void) { return g_last_error.c_str(); }

int32_t hyb_compress(const void* x, int32_t x_dtype, const float* gate_logits,
                     const int32_t* cu_seqlens, const int32_t* start_pos, int32_t batch,
                     int32_t max_new_tokens, void* state, float* state_logits, int32_t mode,
                     const hyb_paged* out, int32_t rope_dim, double rope_base, float eps,
                     void* stream) {
  const char* op = "hyb_compress";
  const hyb_compress_call call{x, x_dtype, gate_logits, cu_seqlens, start_pos, batch,
                               max_new_tokens, state, state_logits, mode, out, rope_dim,
                               rope_base, eps};
  hyb::CompressArgs a;
  HYB_TRY(check_compress(op, call, &a));
  if (batch == 0 || max_new_tokens == 0) return HYB_OK;
  return launch_status(hyb::launch_compress(a, static_cast<hipStream_t>(stream)), op);
}

int32_t hyb_swa_insert(const void* x, int32_t x_dtype, const int32_t* cu_seqlens,
                       const int32_t* start_pos, int32_t batch, int32_t max_new_tokens,
                       const hyb_paged* swa, int32_t rope_dim, double rope_base, void* stream) {
  const char* op = "hyb_swa_insert";
  HYB_TRY(check_compress_common(op, x, x_dtype, cu_seqlens, start_pos, batch, max_new_tokens));
  hyb::PoolDev ps{};
  HYB_TRY(check_pool(swa, op, "swa", true, false, 1, &ps));
  if (ps.dtype == HYB_FP8_E4M3 && ps.dim > 2048)
    return fail(HYB_ENOTSUP, "%s: FP8_E4M3 window pool dim %d > 2048", op, ps.dim);
  HYB_TRY(check_rope(op, rope_dim, rope_base, ps.dim));
  if (batch == 0 || max_new_tokens == 0) return HYB_OK;
  hyb::CompressArgs a{x, x_dtype, nullptr, cu_seqlens, start_pos, batch, max_new_tokens,
                      nullptr, nullptr, 0, ps, rope_dim, rope_base, 0.f, {}};
  fill_theta(&a, rope_dim, rope_base);
  return launch_status(hyb::launch_swa_insert(a, static_cast<hipStream_t>(stream)), op);
}

int32_t hyb_q_norm_kv_insert(const void* q, int32_t q_dtype, int32_t n_heads, const void* kv,
                             int32_t kv_dtype, const int32_t* cu_seqlens, const int32_t* start_pos,
                             int32_t batch, int32_t max_new_tokens, void* q_out,
                             const hyb_paged* swa, int32_t rope_dim, double rope_base, float eps,
                             void* stream) {
  const char* op = "hyb_q_norm_kv_insert";
  HYB_TRY(check_compress_common(op, kv, kv_dtype, cu_seqlens, start_pos, batch, max_new_tokens));
  if (!q || !q_out) return fail(HYB_EINVAL, "%s: q and q_out must be non-NULL", op);
  if (!is_plain(q_dtype)) return fail(HYB_ENOTSUP, "%s: q_dtype must be F32 or BF16", op);
  if (n_heads <= 0 || n_heads > 128) return fail(HYB_EINVAL, "%s: n_heads %d outside [1, 128]", op, n_heads);
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(HYB_EINVAL, "%s: eps must be >= 0", op);
  hyb::PoolDev ps{};
  HYB_TRY(check_pool(swa, op, "swa", true, false, 1, &ps));
  if (ps.dim > 2048) return fail(HYB_ENOTSUP, "%s: dim %d > 2048", op, ps.dim);
  HYB_TRY(check_rope(op, rope_dim, rope_base, ps.dim));
  if (batch == 0 || max_new_tokens == 0) return HYB_OK;
  hyb::QNormArgs a{};
  a.kv = hyb::CompressArgs{kv, kv_dtype, nullptr, cu_seqlens, start_pos, batch, max_new_tokens,
                           nullptr, nullptr, 0, ps, rope_dim, rope_base, 0.f, {}};
  fill_theta(&a.kv, rope_dim, rope_base);
  a.q = q;
  a.q_dtype = q_dtype;
  a.q_out = q_out;
  a.n_heads = n_heads;
  a.eps = eps;
  return launch_status(hyb::launch_q_norm_kv_insert(a, static_cast<hipStream_t>(stream)), op);
}

int32_t hyb_gather_pages(const void* src_host, void* dst, const int32_t* src_page,
                         const int32_t* dst_page, int32_t n, int64_t page_bytes, void* stream) {
  const char* op = "hyb_gather_pages";
  if (!src_host || !dst || !src_page || !dst_page)
    return fail(HYB_EINVAL, "%s: src_host, dst, src_page and dst_page must be non-NULL", op);
  if (n < 0) return fail(HYB_EINVAL, "%s: n %d < 0", op, n);
  if (page_bytes <= 0 || page_bytes % 16)
    return fail(HYB_EINVAL, "%s: page_bytes %lld must be a positive multiple of 16", op,
                (long long)page_bytes);
  if ((reinterpret_cast<uintptr_t>(src_host) | reinterpret_cast<uintptr_t>(dst)) & 15u)
    return fail(HYB_EINVAL, "%s: src_host and dst must be 16-byte aligned", op);
  if (n == 0) return HYB_OK;
  void* src_dev = nullptr;
  if (hipHostGetDevicePointer(&src_dev, const_cast<void*>(src_host), 0) != hipSuccess || !src_dev) {
    (void)hipGetLastError();
    return fail(HYB_EINVAL, "%s: src_host is not pinned host memory with a device alias", op);
  }
  return launch_status(hyb::launch_gather_pages(src_dev, dst, src_page, dst_page, n, page_bytes,
                                                static_cast<hipStream_t>(stream)), op);
}

static int check_score(const char* op, const void* q_idx, int32_t q_dtype, const float* w,
                       const int32_t* q_pos, int32_t n_q, int32_t n_heads, int32_t max_pos,
                       int32_t window, const hyb_paged* idx_pool, hyb::ScoreArgs* a) {
  if (!q_idx || !w || !q_pos) return fail(HYB_EINVAL, "%s: q_idx, w and q_pos must be non-NULL", op);
  if (n_q < 0) return fail(HYB_EINVAL, "%s: n_q %d < 0", op, n_q);
  if (n_heads <= 0) return fail(HYB_EINVAL, "%s: n_heads %d must be positive", op, n_heads);
  if (max_pos < 0) return fail(HYB_EINVAL, "%s: max_pos %d < 0", op, max_pos);
  if (window <= 0) return fail(HYB_EINVAL, "%s: window %d must be positive", op, window);
  if (!is_plain(q_dtype)) return fail(HYB_ENOTSUP, "%s: q_dtype must be F32 or BF16", op);
  hyb::PoolDev pp{};
  HYB_TRY(check_pool(idx_pool, op, "idx_pool", false, true, 2 | 4, &pp));
  const bool mfma = n_heads == 64 && pp.dim == 128 && q_dtype == HYB_BF16 &&
                    (pp.dtype == HYB_BF16 || pp.dtype == HYB_FP4_E2M1);
  if (!mfma && (int64_t)n_heads * pp.dim > 8192)
    return fail(HYB_ENOTSUP, "%s: heads x dim = %d x %d exceeds the generic kernel (8192); the "
                "MFMA kernel takes 64 x 128 with a bf16 query", op, n_heads, pp.dim);
  *a = hyb::ScoreArgs{};
  a->q = q_idx;
  a->q_dtype = q_dtype;
  a->w = w;
  a->n_q = n_q;
  a->n_heads = n_heads;
  a->max_pos = max_pos;
  a->window = window;
  a->pool = pp;
  return HYB_OK;
}

int32_t hyb_index_score(const void* q_idx, int32_t q_dtype, const float* w, const int32_t* q_seq,
                        const int32_t* q_pos, int32_t n_q, int32_t n_heads, int32_t max_pos,
                        int32_t window, const hyb_paged* idx_pool, float* scores,
                        int64_t scores_ld, void* stream) {
  const char* op = "hyb_index_score";
  hyb::ScoreArgs a;
  HYB_TRY(check_score(op, q_idx, q_dtype, w, q_pos, n_q, n_heads, max_pos, window, idx_pool, &a));
  if (!scores) return fail(HYB_EINVAL, "%s: scores is NULL", op);
  if (scores_ld < visible(max_pos, a.pool.ratio, window))
    return fail(HYB_EINVAL, "%s: scores_ld %lld < visible entries %lld", op, (long long)scores_ld,
                (long long)visible(max_pos, a.pool.ratio, window));
  a.qd = hyb::QueryDev{nullptr, q_seq, q_pos};
  a.scores = scores;
  a.ld = scores_ld;
  return launch_status(hyb::launch_index_score(a, static_cast<hipStream_t>(stream)), op);
}

int32_t hyb_topk(const float* scores, int64_t scores_ld, const int32_t* lengths, int32_t n_q,
                 int32_t max_len, int32_t k, int32_t* out_idx, void* stream) {
  const char* op = "hyb_topk";
  if (!scores || !lengths || !out_idx) return fail(HYB_EINVAL, "%s: scores, lengths and out_idx must be non-NULL", op);
  if (n_q < 0 || max_len < 0) return fail(HYB_EINVAL, "%s: n_q and max_len must be >= 0", op);
  if (k < 1 || k > HYB_KMAX) return fail(HYB_EINVAL, "%s: k %d outside [1, %d]", op, k, HYB_KMAX);
  if (scores_ld < max_len) return fail(HYB_EINVAL, "%s: scores_ld %lld < max_len %d", op, (long long)scores_ld, max_len);
  hyb::TopkArgs a{};
  a.scores = scores;
  a.ld = scores_ld;
  a.lengths = lengths;
  a.n_q = n_q;
  a.max_len = max_len;
  a.k = k;
  a.out = out_idx;
  return launch_status(hyb::launch_topk(a, static_cast<hipStream_t>(stream)), op);
}

static int64_t part_blocks(int64_t nv) { return (nv + hyb::kScorePartKeys - 1) / hyb::kScorePartKeys; }
// uint32 words of one row of the selector hand-off: a (key, index) pair per entry, per part
static int64_t pair_words(int64_t parts) { return 2 * hyb::kScorePartKeys * parts; }

int32_t hyb_index_score_keys(const void* q_idx, int32_t q_dtype, const float* w, const int32_t* q_seq,
                             const int32_t* q_pos, int32_t n_q, int32_t n_heads, int32_t max_pos,
                             int32_t window, const hyb_paged* idx_pool, uint32_t* keys,
                             int64_t keys_ld, uint16_t* part_hist, int64_t part_ld, void* stream) {
  const char* op = "hyb_index_score_keys";
  hyb::ScoreArgs a;
  HYB_TRY(check_score(op, q_idx, q_dtype, w, q_pos, n_q, n_heads, max_pos, window, idx_pool, &a));
  if (!keys || !part_hist) return fail(HYB_EINVAL, "%s: keys and part_hist must be non-NULL", op);
  const int64_t nv = visible(max_pos, a.pool.ratio, window);
  if (part_ld < part_blocks(nv) || part_ld > hyb::kTopkMaxParts)
    return fail(HYB_EINVAL, "%s: part_ld %lld outside [%lld, %d]", op, (long long)part_ld,
                (long long)part_blocks(nv), hyb::kTopkMaxParts);
  if (keys_ld < pair_words(part_ld) || (keys_ld & 1) || (reinterpret_cast<uintptr_t>(keys) & 7))
    return fail(HYB_EINVAL, "%s: keys needs 8-byte alignment and an even keys_ld >= 2048 * part_ld = %lld (got %lld)",
                op, (long long)pair_words(part_ld), (long long)keys_ld);
  a.qd = hyb::QueryDev{nullptr, q_seq, q_pos};
  a.scores = reinterpret_cast<float*>(keys);
  a.ld = keys_ld;
  a.part_hist = part_hist;
  a.part_ld = (int32_t)part_ld;
  return launch_status(hyb::launch_index_score(a, static_cast<hipStream_t>(stream)), op);
}

int32_t hyb_topk_keys(const uint32_t* keys, int64_t keys_ld, const uint16_t* part_hist,
                      int64_t part_ld, const int32_t* q_pos, int32_t n_q, int32_t max_pos,
                      int32_t window, int32_t ratio, int32_t k, int32_t* out_idx, void* stream) {
  const char* op = "hyb_topk_keys";
  if (!keys || !part_hist || !q_pos || !out_idx)
    return fail(HYB_EINVAL, "%s: keys, part_hist, q_pos and out_idx must be non-NULL", op);
  if (n_q < 0 || max_pos < 0) return fail(HYB_EINVAL, "%s: n_q and max_pos must be >= 0", op);
  if (window <= 0) return fail(HYB_EINVAL, "%s: window %d must be positive", op, window);
  if (ratio != 4 && ratio != 128) return fail(HYB_EINVAL, "%s: ratio %d must be 4 or 128", op, ratio);
  if (k < 1 || k > HYB_KMAX) return fail(HYB_EINVAL, "%s: k %d outside [1, %d]", op, k, HYB_KMAX);
  const int64_t nv = visible(max_pos, ratio, window);
  if (part_ld < part_blocks(nv) || part_ld > hyb::kTopkMaxParts)
    return fail(HYB_EINVAL, "%s: part_ld %lld outside [%lld, %d]", op, (long long)part_ld,
                (long long)part_blocks(nv), hyb::kTopkMaxParts);
  if (keys_ld < pair_words(part_ld) || (keys_ld & 1) || (reinterpret_cast<uintptr_t>(keys) & 7))
    return fail(HYB_EINVAL, "%s: keys needs 8-byte alignment and an even keys_ld >= 2048 * part_ld = %lld (got %lld)",
                op, (long long)pair_words(part_ld), (long long)keys_ld);
  if (n_q == 0) return HYB_OK;
  hyb::TopkArgs t{};
  t.scores = reinterpret_cast<const float*>(keys);
  t.ld = keys_ld;
  t.lengths = nullptr;
  t.qd = hyb::QueryDev{nullptr, nullptr, q_pos};
  t.ratio = ratio;
  t.window = window;
  t.n_q = n_q;
  t.max_len = (int32_t)nv;
  t.k = k;
  t.out = out_idx;
  t.part_hist = part_hist;
  t.part_ld = (int32_t)part_ld;
  return launch_status(hyb::launch_topk(t, static_cast<hipStream_t>(stream)), op);
}

// Workspace of hyb_index_topk: the selector hand-off, (key, index) pairs [n_q][part_ld *
// kScorePartKeys] (uint2), then the cumulative histograms [n_q][part_ld][kTopBins] (uint16),
// part_ld = ld / kScorePartKeys rounded up.
static size_t topk_part_ld(int64_t ld) {
  return (size_t)((ld + hyb::kScorePartKeys - 1) / hyb::kScorePartKeys);
}
static size_t topk_ws_bytes(int32_t n_q, int64_t ld) {
  return (size_t)n_q * pair_words((int64_t)topk_part_ld(ld)) * sizeof(uint32_t) +
         (size_t)n_q * topk_part_ld(ld) * hyb::kTopBins * sizeof(uint16_t);
}

size_t hyb_index_topk_workspace_bytes(int32_t n_q, int32_t max_pos, int32_t window, int32_t ratio) {
  if (n_q <= 0 || max_pos < 0 || window <= 0 || (ratio != 4 && ratio != 128)) return 0;
  return topk_ws_bytes(n_q, (int64_t)score_ld(max_pos, window, ratio));
}

int32_t hyb_index_topk(const void* q_idx, int32_t q_dtype, const float* w, const int32_t* q_seq,
                       const int32_t* q_pos, int32_t n_q, int32_t n_heads, int32_t max_pos,
                       int32_t window, const hyb_paged* idx_pool, int32_t k, int32_t* out_idx,
                       void* workspace, size_t workspace_bytes, void* stream) {
  const char* op = "hyb_index_topk";
  hyb::ScoreArgs a;
  HYB_TRY(check_score(op, q_idx, q_dtype, w, q_pos, n_q, n_heads, max_pos, window, idx_pool, &a));
  if (!out_idx) return fail(HYB_EINVAL, "%s: out_idx is NULL", op);
  if (k < 1 || k > HYB_KMAX) return fail(HYB_EINVAL, "%s: k %d outside [1, %d]", op, k, HYB_KMAX);
  const size_t need = hyb_index_topk_workspace_bytes(n_q, max_pos, window, a.pool.ratio);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(HYB_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", op, need,
                workspace ? workspace_bytes : (size_t)0);
  if (n_q == 0) return HYB_OK;
  const int64_t ld = (int64_t)score_ld(max_pos, window, a.pool.ratio);
  if ((int64_t)topk_part_ld(ld) > hyb::kTopkMaxParts)
    return fail(HYB_ENOTSUP, "%s: %lld visible entries exceed the selector (%d x 1024)", op,
                (long long)ld, hyb::kTopkMaxParts);
  const int64_t pld = pair_words((int64_t)topk_part_ld(ld));
  a.qd = hyb::QueryDev{nullptr, q_seq, q_pos};
  a.scores = static_cast<float*>(workspace);
  a.ld = pld;
  a.part_hist = reinterpret_cast<uint16_t*>(static_cast<uint32_t*>(workspace) + (size_t)n_q * pld);
  a.part_ld = (int32_t)topk_part_ld(ld);
  hipStream_t s = static_cast<hipStream_t>(stream);
  HYB_TRY(launch_status(hyb::launch_index_score(a, s), op));
  hyb::TopkArgs t{};
  t.scores = a.scores;
  t.ld = pld;
  t.lengths = nullptr;
  t.qd = a.qd;
  t.ratio = a.pool.ratio;
  t.window = window;
  t.n_q = n_q;
  t.max_len = (int32_t)visible(max_pos, a.pool.ratio, window);
  t.k = k;
  t.out = out_idx;
  t.part_hist = a.part_hist;
  t.part_ld = a.part_ld;
  return launch_status(hyb::launch_topk(t, s), op);
}

size_t hyb_attn_decode_workspace_bytes(int32_t batch, int32_t n_heads, int32_t dim,
                                       int32_t max_seq_len, int32_t comp_ratio, int32_t k,
                                       int32_t window) {
  return attn_ws(batch, n_heads, dim, (int64_t)max_seq_len - 1, comp_ratio, k, window, 0);
}

int32_t hyb_attn_decode(const void* q, int32_t q_dtype, const int32_t* seq_lens, int32_t batch,
                        int32_t n_heads, int32_t max_seq_len, const hyb_paged* swa,
                        const hyb_paged* comp, const int32_t* topk_idx, int32_t k, int32_t window,
                        float softmax_scale, int32_t rope_dim, double rope_base, void* out,
                        int32_t out_dtype, float* out_scale, void* workspace,
                        size_t workspace_bytes, void* stream) {
  const char* op = "hyb_attn_decode";
  if (!seq_lens) return fail(HYB_EINVAL, "%s: seq_lens is NULL", op);
  if (max_seq_len < 1) return fail(HYB_EINVAL, "%s: max_seq_len %d < 1", op, max_seq_len);
  AttnCommon c;
  HYB_TRY(check_attention(op, q, q_dtype, batch, n_heads, swa, comp, topk_idx, k, window,
                          softmax_scale, rope_dim, rope_base, out, out_dtype, out_scale,
                          (int64_t)max_seq_len - 1, &c));
  HYB_TRY(attach_workspace(op, &c, workspace, workspace_bytes));
  if (batch == 0) return HYB_OK;
  c.args.qd = hyb::QueryDev{seq_lens, nullptr, nullptr};
  return launch_status(hyb::launch_attention(c.args, static_cast<hipStream_t>(stream)), op);
}

int32_t hyb_attn_decode_compress(const void* q, int32_t q_dtype, const int32_t* seq_lens,
                                 int32_t batch, int32_t n_heads, int32_t max_seq_len,
                                 const hyb_paged* swa, const hyb_paged* comp,
                                 const int32_t* topk_idx, int32_t k, int32_t window,
                                 float softmax_scale, int32_t rope_dim, double rope_base,
                                 void* out, int32_t out_dtype, float* out_scale, void* workspace,
                                 size_t workspace_bytes, const hyb_compress_call* compress,
                                 void* stream) {
  const char* op = "hyb_attn_decode_compress";
  if (!seq_lens) return fail(HYB_EINVAL, "%s: seq_lens is NULL", op);
  if (max_seq_len < 1) return fail(HYB_EINVAL, "%s: max_seq_len %d < 1", op, max_seq_len);
  if (!compress) return fail(HYB_EINVAL, "%s: compress is NULL", op);
  AttnCommon c;
  HYB_TRY(check_attention(op, q, q_dtype, batch, n_heads, swa, comp, topk_idx, k, window,
                          softmax_scale, rope_dim, rope_base, out, out_dtype, out_scale,
                          (int64_t)max_seq_len - 1, &c));
  HYB_TRY(attach_workspace(op, &c, workspace, workspace_bytes));
  hyb::CompressArgs ca;
  HYB_TRY(check_compress(op, *compress, &ca));
  c.args.qd = hyb::QueryDev{seq_lens, nullptr, nullptr};
  return launch_status(hyb::launch_attention_compress(c.args, ca, static_cast<hipStream_t>(stream)), op);
}

size_t hyb_attn_prefill_workspace_bytes(int32_t n_q, int32_t n_heads, int32_t dim,
                                        int32_t max_pos, int32_t comp_ratio, int32_t k,
                                        int32_t window) {
  return attn_ws(n_q, n_heads, dim, max_pos, comp_ratio, k, window, 0);
}

int32_t hyb_attn_prefill(const void* q, int32_t q_dtype, const int32_t* q_seq,
                         const int32_t* q_pos, int32_t n_q, int32_t n_heads, int32_t max_pos,
                         const hyb_paged* swa, const hyb_paged* comp, const int32_t* topk_idx,
                         int32_t k, int32_t window, float softmax_scale, int32_t rope_dim,
                         double rope_base, void* out, int32_t out_dtype, float* out_scale,
                         void* workspace, size_t workspace_bytes, void* stream) {
  const char* op = "hyb_attn_prefill";
  if (!q_pos) return fail(HYB_EINVAL, "%s: q_pos is NULL", op);
  if (max_pos < 0) return fail(HYB_EINVAL, "%s: max_pos %d < 0", op, max_pos);
  AttnCommon c;
  HYB_TRY(check_attention(op, q, q_dtype, n_q, n_heads, swa, comp, topk_idx, k, window,
                          softmax_scale, rope_dim, rope_base, out, out_dtype, out_scale, max_pos,
                          &c));
  HYB_TRY(attach_workspace(op, &c, workspace, workspace_bytes));
  if (n_q == 0) return HYB_OK;
  c.args.qd = hyb::QueryDev{nullptr, q_seq, q_pos};
  return launch_status(hyb::launch_attention(c.args, static_cast<hipStream_t>(stream)), op);
}

}  // extern "C"
