// C ABI of the MLA library: host-side argument checks, launch planning and
// dispatch to the kernel families. Every check runs before anything is
// enqueued, so a rejected call touches neither the stream nor any output.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "launch.h"
#include "mla.h"

using mla::CacheView;

namespace {

bool trace_on() {
  static int on = -1;
  if (on < 0) {
    const char* e = getenv("MLA_TRACE");
    on = (e && e[0] && e[0] != '0') ? 1 : 0;
  }
  return on == 1;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

mla_status check_dims(const mla_dims* d) {
  if (!d) return MLA_ERR_NULL_ARG;
  if (d->dtype != MLA_F32 && d->dtype != MLA_BF16) return MLA_ERR_BAD_DTYPE;
  if (d->n_heads < 1 || d->n_heads > 256) return MLA_ERR_BAD_SHAPE;
  if (d->d_c < 8 || d->d_c > 1024 || d->d_c % 8) return MLA_ERR_BAD_SHAPE;
  if (d->d_rope < 2 || d->d_rope > 128 || d->d_rope % 2 || (d->d_c + d->d_rope) % 8) return MLA_ERR_BAD_SHAPE;
  if (d->d_nope < 1 || d->d_nope > 256 || d->d_v < 1 || d->d_v > 256) return MLA_ERR_BAD_SHAPE;
  if (!(d->rope_base > 1.f) || !isfinite(d->rope_base) || !isfinite(d->softmax_scale)) return MLA_ERR_BAD_SHAPE;
  return MLA_OK;
}

float scale_of(const mla_dims* d) {
  return d->softmax_scale > 0.f ? d->softmax_scale : 1.f / sqrtf((float)(d->d_nope + d->d_rope));
}

mla_status check_cache(const mla_cache* c, CacheView* v) {
  if (!c) return MLA_ERR_NULL_ARG;
  if (!c->rows || !c->context_lens) return MLA_ERR_NULL_ARG;
  if (c->max_context < 1) return MLA_ERR_BAD_SHAPE;
  if (c->block_table) {
    if (c->block_size < 1 || c->num_blocks < 1 || c->max_blocks_per_seq < 1) return MLA_ERR_BAD_SHAPE;
    if ((int64_t)c->max_blocks_per_seq * c->block_size < c->max_context) return MLA_ERR_BAD_SHAPE;
    if (!aligned(c->block_table, 4)) return MLA_ERR_ALIGNMENT;
  }
  if (!aligned(c->rows, 16) || !aligned(c->context_lens, 4)) return MLA_ERR_ALIGNMENT;
  v->rows = c->rows;
  v->block_table = c->block_table;
  v->context_lens = c->context_lens;
  v->paged = c->block_table != nullptr;
  v->block_size = v->paged ? c->block_size : c->max_context;
  v->max_blocks = v->paged ? c->max_blocks_per_seq : 1;
  v->seq_stride = c->max_context;
  return MLA_OK;
}

mla_status check_ws(void* ws, size_t have, size_t need) {
  if (have < need) return MLA_ERR_WORKSPACE;
  if (need > 0 && !ws) return MLA_ERR_NULL_ARG;
  if (need > 0 && !aligned(ws, 256)) return MLA_ERR_ALIGNMENT;
  return MLA_OK;
}

// query rows of one decode call (a grid dimension of the split kernel)
constexpr int64_t MAX_QUERY_ROWS = 65535;
constexpr int32_t MAX_Q_LEN = 64;

mla_status hip_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

bool fast_dims(const mla_dims* d) {
  mla::CacheView v{};
  v.paged = 1;
  v.block_size = 64;
  return mla::decode_fast_supported(*d, v);
}

bool prefill_fast_dims(const mla_dims* d) {
  mla::CacheView v{};
  v.paged = 1;
  v.block_size = 64;
  return mla::prefill_fast_supported(*d, v);
}

}  // namespace

extern "C" {

static mla_status mla_rope_latent_project_rows(const mla_dims* d, int32_t n_tokens, int32_t d_model, const void* h,
                                               const void* w_dkv, const void* w_kr, const int32_t* positions,
                                               const int32_t* slots, const mla_cache* cache, const mla_qproj* qp,
                                               void* ws, size_t ws_bytes, void* stream);

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL_ARG: return "a required pointer is NULL";
    case MLA_ERR_BAD_SHAPE: return "a size or dimension is out of range or inconsistent";
    case MLA_ERR_BAD_DTYPE: return "dtype must be MLA_F32 or MLA_BF16";
    case MLA_ERR_UNSUPPORTED: return "valid but not implemented by this library";
    case MLA_ERR_WORKSPACE: return "workspace smaller than required";
    case MLA_ERR_HIP: return "a HIP launch or query failed";
    case MLA_ERR_ALIGNMENT: return "a pointer is not suitably aligned (16 bytes for data, 4 for int32)";
  }
  return "unknown status";
}

int32_t mla_version(void) { return 100; }

mla_status mla_project_workspace_size(const mla_dims* d, int32_t n_tokens, int32_t d_q, size_t* bytes) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!bytes) return MLA_ERR_NULL_ARG;
  if (n_tokens < 0 || d_q < 0) return MLA_ERR_BAD_SHAPE;
  *bytes = (size_t)n_tokens * d_q * sizeof(float);
  return MLA_OK;
}

mla_status mla_decode_multi_workspace_size(const mla_dims* d, int32_t batch, int32_t q_len, int32_t max_context,
                                           size_t* bytes) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!bytes) return MLA_ERR_NULL_ARG;
  if (batch < 0 || max_context < 0 || q_len < 1 || q_len > MAX_Q_LEN) return MLA_ERR_BAD_SHAPE;
  if ((int64_t)batch * q_len > MAX_QUERY_ROWS) return MLA_ERR_BAD_SHAPE;
  *bytes = (fast_dims(d) && batch > 0 && max_context > 0 && mla::decode_fast_context_ok(max_context))
               ? mla::decode_fast_workspace(*d, batch, q_len, max_context)
               : 0;
  return MLA_OK;
}

mla_status mla_decode_workspace_size(const mla_dims* d, int32_t batch, int32_t max_context, size_t* bytes) {
  return mla_decode_multi_workspace_size(d, batch, 1, max_context, bytes);
}

mla_status mla_prefill_workspace_size(const mla_dims* d, int32_t batch, int32_t seq_len, int32_t max_context,
                                      size_t* bytes) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!bytes) return MLA_ERR_NULL_ARG;
  if (batch < 0 || seq_len < 0 || max_context < 0) return MLA_ERR_BAD_SHAPE;
  *bytes = (prefill_fast_dims(d) && batch > 0 && seq_len > 0)
               ? mla::prefill_fast_workspace(*d, batch, max_context > seq_len ? max_context : seq_len)
               : 0;
  return MLA_OK;
}

mla_status mla_workspace_size(int32_t op, const mla_dims* d, int32_t size_a, int32_t size_b, size_t* bytes) {
  switch (op) {
    case MLA_OP_PROJECT: return mla_project_workspace_size(d, size_a, size_b, bytes);
    case MLA_OP_DECODE: return mla_decode_workspace_size(d, size_a, size_b, bytes);
    case MLA_OP_PREFILL: return mla_prefill_workspace_size(d, size_a, size_b, size_b, bytes);
    default: return MLA_ERR_UNSUPPORTED;
  }
}

int32_t mla_decode_path(const mla_dims* d, int32_t block_size, int32_t paged) {
  if (check_dims(d) != MLA_OK) return -1;
  mla::CacheView v{};
  v.paged = paged;
  v.block_size = block_size;
  return mla::decode_fast_supported(*d, v) ? 1 : 0;
}

int32_t mla_prefill_path(const mla_dims* d, int32_t block_size, int32_t paged) {
  if (check_dims(d) != MLA_OK) return -1;
  mla::CacheView v{};
  v.paged = paged;
  v.block_size = block_size;
  return mla::prefill_fast_supported(*d, v) ? 1 : 0;
}

mla_status mla_rope_latent_project(const mla_dims* d, int32_t n_tokens, int32_t d_model, const void* h,
                                   const void* w_dkv, const void* w_kr, const int32_t* positions,
                                   const int32_t* slots, const mla_cache* cache, const mla_qproj* qp,
                                   void* ws, size_t ws_bytes, void* stream) {
  if (n_tokens > 0 && !slots) return MLA_ERR_NULL_ARG;
  return mla_rope_latent_project_rows(d, n_tokens, d_model, h, w_dkv, w_kr, positions, slots, cache, qp, ws,
                                      ws_bytes, stream);
}

// As mla_rope_latent_project; slots == NULL writes token i to row i.
static mla_status mla_rope_latent_project_rows(const mla_dims* d, int32_t n_tokens, int32_t d_model, const void* h,
                                               const void* w_dkv, const void* w_kr, const int32_t* positions,
                                               const int32_t* slots, const mla_cache* cache, const mla_qproj* qp,
                                               void* ws, size_t ws_bytes, void* stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (n_tokens < 0 || d_model < 1 || d_model > 16384) return MLA_ERR_BAD_SHAPE;
  if (n_tokens == 0) return MLA_OK;
  if (!h || !w_dkv || !w_kr || !positions || !cache || !cache->rows) return MLA_ERR_NULL_ARG;
  if (!aligned(h, 16) || !aligned(w_dkv, 16) || !aligned(w_kr, 16) || !aligned(cache->rows, 16) ||
      !aligned(positions, 4) || (slots && !aligned(slots, 4)))
    return MLA_ERR_ALIGNMENT;
  size_t need = 0;
  if (qp) {
    if (qp->d_q < 8 || qp->d_q > 4096 || qp->d_q % 8) return MLA_ERR_BAD_SHAPE;
    if (!qp->w_dq || !qp->w_uq || !qp->w_qr || !qp->q_nope || !qp->q_pe) return MLA_ERR_NULL_ARG;
    if (!aligned(qp->w_dq, 16) || !aligned(qp->w_uq, 16) || !aligned(qp->w_qr, 16) ||
        !aligned(qp->q_nope, 16) || !aligned(qp->q_pe, 16))
      return MLA_ERR_ALIGNMENT;
    need = (size_t)n_tokens * qp->d_q * sizeof(float);
  }
  if ((st = check_ws(ws, ws_bytes, need)) != MLA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const bool fast = mla::project_fast_supported(*d, d_model, qp ? qp->d_q : 0);
  if (trace_on())
    fprintf(stderr, "[mla] project n_tokens=%d d_model=%d d_q=%d path=%s\n", n_tokens, d_model, qp ? qp->d_q : 0,
            fast ? "mfma" : "generic");
  if (fast)
    return hip_status(mla::project_fast(*d, n_tokens, d_model, h, w_dkv, w_kr, positions, slots, cache->rows, qp, ws, s));
  hipError_t e = mla::project_latent_generic(*d, n_tokens, d_model, h, w_dkv, w_kr, positions, slots,
                                             cache->rows, s);
  if (e != hipSuccess || !qp) return hip_status(e);
  // query path: c_Q (kept in fp32 in the workspace) then both up-projections
  const int dt = d->dtype;
  e = mla::gemm_nt_generic(dt, dt, MLA_F32, n_tokens, qp->d_q, d_model, h, d_model, qp->w_dq, qp->w_dq,
                           qp->d_q, d_model, ws, qp->d_q, s);
  if (e != hipSuccess) return MLA_ERR_HIP;
  const int hn = d->n_heads * d->d_nope, hr = d->n_heads * d->d_rope;
  e = mla::gemm_nt_generic(MLA_F32, dt, dt, n_tokens, hn, qp->d_q, ws, qp->d_q, qp->w_uq, qp->w_uq, hn,
                           qp->d_q, qp->q_nope, hn, s);
  if (e != hipSuccess) return MLA_ERR_HIP;
  return hip_status(mla::gemm_nt_generic(MLA_F32, dt, dt, n_tokens, hr, qp->d_q, ws, qp->d_q, qp->w_qr,
                                         qp->w_qr, hr, qp->d_q, qp->q_pe, hr, s));
}

// FP8 projection: the latent rows go to a bf16 staging area at the front of
// the workspace (row i for token i), then the quantiser writes them into the
// FP8 pages at their slots; the query path's c_Q follows the staging area.
static size_t fp8_stage_bytes(const mla_dims* d, int32_t n_tokens) {
  return ((size_t)n_tokens * (d->d_c + d->d_rope) * 2 + 255) & ~(size_t)255;
}

mla_status mla_project_fp8_workspace_size(const mla_dims* d, int32_t n_tokens, int32_t d_q, size_t* bytes) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!bytes) return MLA_ERR_NULL_ARG;
  if (n_tokens < 0 || d_q < 0) return MLA_ERR_BAD_SHAPE;
  *bytes = fp8_stage_bytes(d, n_tokens) + (size_t)n_tokens * d_q * sizeof(float);
  return MLA_OK;
}

mla_status mla_rope_latent_project_fp8(const mla_dims* d, int32_t n_tokens, int32_t d_model, const void* h,
                                       const void* w_dkv, const void* w_kr, const int32_t* positions,
                                       const int32_t* slots, void* pool, int32_t block_size, const mla_qproj* qp,
                                       void* ws, size_t ws_bytes, void* stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (d->dtype != MLA_BF16) return MLA_ERR_BAD_DTYPE;
  if (n_tokens < 0 || d_model < 1 || d_model > 16384 || block_size < 1 || block_size > 4096) return MLA_ERR_BAD_SHAPE;
  if (n_tokens == 0) return MLA_OK;
  if (!pool || !slots) return MLA_ERR_NULL_ARG;
  if (!aligned(pool, 16)) return MLA_ERR_ALIGNMENT;
  size_t need = 0;
  if ((st = mla_project_fp8_workspace_size(d, n_tokens, qp ? qp->d_q : 0, &need)) != MLA_OK) return st;
  if ((st = check_ws(ws, ws_bytes, need)) != MLA_OK) return st;
  // the bf16 rows into the staging area (a contiguous "cache" of n_tokens rows)
  const size_t stage = fp8_stage_bytes(d, n_tokens);
  mla_cache staging{};
  staging.rows = ws;
  staging.num_blocks = 1;
  staging.block_size = n_tokens;
  staging.context_lens = slots;  // not read by the projection
  staging.max_context = n_tokens;
  if ((st = mla_rope_latent_project_rows(d, n_tokens, d_model, h, w_dkv, w_kr, positions, nullptr, &staging, qp,
                                         (char*)ws + stage, ws_bytes - stage, stream)) != MLA_OK)
    return st;
  hipStream_t s = (hipStream_t)stream;
  if (trace_on()) fprintf(stderr, "[mla] project_fp8 n_tokens=%d block_size=%d\n", n_tokens, block_size);
  return hip_status(mla::quant_fp8(*d, n_tokens, ws, slots, block_size, pool, s));
}

mla_status mla_decode_multi(const mla_dims* d, int32_t batch, int32_t q_len, const void* q_nope, const void* q_pe,
                            const void* w_uk, const void* w_uv, const mla_cache* cache, void* out, void* ws,
                            size_t ws_bytes, void* stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (batch < 0 || q_len < 1 || q_len > MAX_Q_LEN) return MLA_ERR_BAD_SHAPE;
  if ((int64_t)batch * q_len > MAX_QUERY_ROWS) return MLA_ERR_BAD_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!q_nope || !q_pe || !w_uk || !w_uv || !out) return MLA_ERR_NULL_ARG;
  if (!aligned(q_nope, 16) || !aligned(q_pe, 16) || !aligned(w_uk, 16) || !aligned(w_uv, 16) ||
      !aligned(out, 16))
    return MLA_ERR_ALIGNMENT;
  CacheView v{};
  if ((st = check_cache(cache, &v)) != MLA_OK) return st;
  if (q_len > cache->max_context) return MLA_ERR_BAD_SHAPE;
  const bool fast = mla::decode_fast_supported(*d, v) && mla::decode_fast_context_ok(cache->max_context);
  const size_t need = fast ? mla::decode_fast_workspace(*d, batch, q_len, cache->max_context) : 0;
  if ((st = check_ws(ws, ws_bytes, need)) != MLA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (trace_on())
    fprintf(stderr, "[mla] decode batch=%d q_len=%d heads=%d max_context=%d path=%s ws=%zu\n", batch, q_len,
            d->n_heads, cache->max_context, fast ? "mfma" : "generic", need);
  if (fast)
    return hip_status(mla::decode_fast(*d, scale_of(d), batch, q_len, cache->max_context, q_nope, q_pe, w_uk,
                                       w_uv, v, out, ws, ws_bytes, s));
  return hip_status(mla::attn_generic(*d, scale_of(d), batch, q_len, q_nope, q_pe, w_uk, w_uv, v, out, s));
}

mla_status mla_decode(const mla_dims* d, int32_t batch, const void* q_nope, const void* q_pe,
                      const void* w_uk, const void* w_uv, const mla_cache* cache, void* out, void* ws,
                      size_t ws_bytes, void* stream) {
  return mla_decode_multi(d, batch, 1, q_nope, q_pe, w_uk, w_uv, cache, out, ws, ws_bytes, stream);
}

mla_status mla_fp8_page_bytes(const mla_dims* d, int32_t block_size, size_t* bytes) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!bytes) return MLA_ERR_NULL_ARG;
  if (block_size < 1 || block_size > 4096) return MLA_ERR_BAD_SHAPE;
  *bytes = mla::fp8_page_bytes(block_size, d->d_c, d->d_rope);
  return MLA_OK;
}

mla_status mla_quantize_fp8(const mla_dims* d, int32_t n_rows, const void* rows, const int32_t* slots,
                            int32_t block_size, void* pool, void* stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (d->dtype != MLA_BF16) return MLA_ERR_BAD_DTYPE;
  if (n_rows < 0 || block_size < 1 || block_size > 4096) return MLA_ERR_BAD_SHAPE;
  if (n_rows == 0) return MLA_OK;
  if (!rows || !pool) return MLA_ERR_NULL_ARG;
  if (!aligned(rows, 16) || !aligned(pool, 16) || (slots && !aligned(slots, 4))) return MLA_ERR_ALIGNMENT;
  hipStream_t s = (hipStream_t)stream;
  if (trace_on()) fprintf(stderr, "[mla] quantize_fp8 n_rows=%d block_size=%d\n", n_rows, block_size);
  return hip_status(mla::quant_fp8(*d, n_rows, rows, slots, block_size, pool, s));
}

mla_status mla_decode_fp8_workspace_size(const mla_dims* d, int32_t batch, int32_t q_len, int32_t max_context,
                                         size_t* bytes) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!bytes) return MLA_ERR_NULL_ARG;
  if (batch < 0 || max_context < 0 || q_len < 1 || q_len > MAX_Q_LEN) return MLA_ERR_BAD_SHAPE;
  if ((int64_t)batch * q_len > MAX_QUERY_ROWS) return MLA_ERR_BAD_SHAPE;
  mla::CacheView v{};
  v.paged = 1;
  v.block_size = 64;
  *bytes = (mla::decode_fp8_supported(*d, v) && batch > 0 && max_context > 0 &&
            mla::decode_fast_context_ok(max_context))
               ? mla::decode_fp8_workspace(*d, batch, q_len, max_context)
               : 0;
  return MLA_OK;
}

mla_status mla_decode_fp8(const mla_dims* d, int32_t batch, int32_t q_len, const void* q_nope, const void* q_pe,
                          const void* w_uk, const void* w_uv, const mla_cache* cache, void* out, void* ws,
                          size_t ws_bytes, void* stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (batch < 0 || q_len < 1 || q_len > MAX_Q_LEN) return MLA_ERR_BAD_SHAPE;
  if ((int64_t)batch * q_len > MAX_QUERY_ROWS) return MLA_ERR_BAD_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!q_nope || !q_pe || !w_uk || !w_uv || !out) return MLA_ERR_NULL_ARG;
  if (!aligned(q_nope, 16) || !aligned(q_pe, 16) || !aligned(w_uk, 16) || !aligned(w_uv, 16) ||
      !aligned(out, 16))
    return MLA_ERR_ALIGNMENT;
  CacheView v{};
  if ((st = check_cache(cache, &v)) != MLA_OK) return st;
  if (q_len > cache->max_context) return MLA_ERR_BAD_SHAPE;
  if (!mla::decode_fp8_supported(*d, v) || !mla::decode_fast_context_ok(cache->max_context))
    return MLA_ERR_UNSUPPORTED;
  const size_t need = mla::decode_fp8_workspace(*d, batch, q_len, cache->max_context);
  if ((st = check_ws(ws, ws_bytes, need)) != MLA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (trace_on())
    fprintf(stderr, "[mla] decode_fp8 batch=%d q_len=%d heads=%d max_context=%d ws=%zu\n", batch, q_len, d->n_heads,
            cache->max_context, need);
  return hip_status(mla::decode_fp8(*d, scale_of(d), batch, q_len, cache->max_context, q_nope, q_pe, w_uk, w_uv, v,
                                    out, ws, ws_bytes, s));
}

// ---- output side: W_O, and W_UV folded into W_O ---------------------------

static bool d_model_ok(int32_t d_model) { return d_model >= 1 && d_model <= 65536; }

mla_status mla_output_workspace_size(const mla_dims* d, int32_t n_rows, int32_t d_model, int32_t folded,
                                     size_t* bytes) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!bytes) return MLA_ERR_NULL_ARG;
  if (n_rows < 0 || !d_model_ok(d_model)) return MLA_ERR_BAD_SHAPE;
  const int K = d->n_heads * (folded ? d->d_c : d->d_v);
  *bytes = n_rows > 0 ? mla::rows_times_weight_workspace(*d, n_rows, d_model, K) : 0;
  return MLA_OK;
}

mla_status mla_output_project(const mla_dims* d, int32_t n_rows, int32_t d_model, const void* attn_out,
                              const void* w_o, void* out, void* ws, size_t ws_bytes, void* stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (n_rows < 0 || !d_model_ok(d_model)) return MLA_ERR_BAD_SHAPE;
  if (n_rows == 0) return MLA_OK;
  if (!attn_out || !w_o || !out) return MLA_ERR_NULL_ARG;
  if (!aligned(attn_out, 16) || !aligned(w_o, 16) || !aligned(out, 16)) return MLA_ERR_ALIGNMENT;
  const int K = d->n_heads * d->d_v;
  const size_t need = mla::rows_times_weight_workspace(*d, n_rows, d_model, K);
  if ((st = check_ws(ws, ws_bytes, need)) != MLA_OK) return st;
  if (trace_on()) fprintf(stderr, "[mla] output_project rows=%d d_model=%d K=%d ws=%zu\n", n_rows, d_model, K, need);
  return hip_status(mla::rows_times_weight(*d, n_rows, d_model, K, attn_out, w_o, out, ws, ws_bytes,
                                           "mla_output_project", (hipStream_t)stream));
}

mla_status mla_fold_output_weights(const mla_dims* d, int32_t d_model, const void* w_uv, const void* w_o,
                                   void* w_ouv, void* stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!d_model_ok(d_model)) return MLA_ERR_BAD_SHAPE;
  if (!w_uv || !w_o || !w_ouv) return MLA_ERR_NULL_ARG;
  if (!aligned(w_uv, 16) || !aligned(w_o, 16) || !aligned(w_ouv, 16)) return MLA_ERR_ALIGNMENT;
  if (trace_on()) fprintf(stderr, "[mla] fold_output_weights d_model=%d heads=%d\n", d_model, d->n_heads);
  return hip_status(mla::fold_output_weights(*d, d_model, w_uv, w_o, w_ouv, (hipStream_t)stream));
}

// workspace of the folded decode: the decode's own, then o_c [rows, H, d_c]
// bf16, then the output GEMM's partial sums
static size_t folded_ws(const mla_dims* d, int32_t batch, int32_t q_len, int32_t max_context, int32_t d_model,
                        size_t* oc_off, size_t* gemm_off) {
  const size_t a = (mla::decode_fast_workspace(*d, batch, q_len, max_context) + 255) & ~(size_t)255;
  const int64_t rows = (int64_t)batch * q_len;
  const size_t b = ((size_t)rows * d->n_heads * d->d_c * 2 + 255) & ~(size_t)255;
  *oc_off = a;
  *gemm_off = a + b;
  return a + b + mla::rows_times_weight_workspace(*d, (int)rows, d_model, d->n_heads * d->d_c);
}

mla_status mla_decode_folded_workspace_size(const mla_dims* d, int32_t batch, int32_t q_len, int32_t max_context,
                                            int32_t d_model, size_t* bytes) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!bytes) return MLA_ERR_NULL_ARG;
  if (batch < 0 || max_context < 0 || q_len < 1 || q_len > MAX_Q_LEN || !d_model_ok(d_model))
    return MLA_ERR_BAD_SHAPE;
  if ((int64_t)batch * q_len > MAX_QUERY_ROWS) return MLA_ERR_BAD_SHAPE;
  size_t o1, o2;
  *bytes = (fast_dims(d) && batch > 0 && max_context > 0 && mla::decode_fast_context_ok(max_context))
               ? folded_ws(d, batch, q_len, max_context, d_model, &o1, &o2)
               : 0;
  return MLA_OK;
}

mla_status mla_decode_folded(const mla_dims* d, int32_t batch, int32_t q_len, const void* q_nope, const void* q_pe,
                             const void* w_uk, const void* w_ouv, int32_t d_model, const mla_cache* cache, void* out,
                             void* ws, size_t ws_bytes, void* stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (batch < 0 || q_len < 1 || q_len > MAX_Q_LEN || !d_model_ok(d_model)) return MLA_ERR_BAD_SHAPE;
  if ((int64_t)batch * q_len > MAX_QUERY_ROWS) return MLA_ERR_BAD_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!q_nope || !q_pe || !w_uk || !w_ouv || !out) return MLA_ERR_NULL_ARG;
  if (!aligned(q_nope, 16) || !aligned(q_pe, 16) || !aligned(w_uk, 16) || !aligned(w_ouv, 16) ||
      !aligned(out, 16))
    return MLA_ERR_ALIGNMENT;
  CacheView v{};
  if ((st = check_cache(cache, &v)) != MLA_OK) return st;
  if (q_len > cache->max_context) return MLA_ERR_BAD_SHAPE;
  if (!(mla::decode_fast_supported(*d, v) && mla::decode_fast_context_ok(cache->max_context)))
    return MLA_ERR_UNSUPPORTED;
  size_t oc_off, gemm_off;
  const size_t need = folded_ws(d, batch, q_len, cache->max_context, d_model, &oc_off, &gemm_off);
  if ((st = check_ws(ws, ws_bytes, need)) != MLA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (trace_on())
    fprintf(stderr, "[mla] decode_folded batch=%d q_len=%d heads=%d d_model=%d ws=%zu\n", batch, q_len, d->n_heads,
            d_model, need);
  char* w = (char*)ws;
  hipError_t e = mla::decode_fast(*d, scale_of(d), batch, q_len, cache->max_context, q_nope, q_pe, w_uk, nullptr, v,
                                  w + oc_off, ws, oc_off, s);
  if (e != hipSuccess) return MLA_ERR_HIP;
  const int rows = batch * q_len;
  return hip_status(mla::rows_times_weight(*d, rows, d_model, d->n_heads * d->d_c, w + oc_off, w_ouv, out,
                                           w + gemm_off, need - gemm_off, "mla_output_project_folded", s));
}

mla_status mla_prefill(const mla_dims* d, int32_t batch, int32_t seq_len, const void* q_nope, const void* q_pe,
                       const void* w_uk, const void* w_uv, const mla_cache* cache, void* out, void* ws,
                       size_t ws_bytes, void* stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (batch < 0 || seq_len < 0) return MLA_ERR_BAD_SHAPE;
  if (batch == 0 || seq_len == 0) return MLA_OK;
  if (!q_nope || !q_pe || !w_uk || !w_uv || !out) return MLA_ERR_NULL_ARG;
  if (!aligned(q_nope, 16) || !aligned(q_pe, 16) || !aligned(w_uk, 16) || !aligned(w_uv, 16) ||
      !aligned(out, 16))
    return MLA_ERR_ALIGNMENT;
  CacheView v{};
  if ((st = check_cache(cache, &v)) != MLA_OK) return st;
  if (seq_len > cache->max_context) return MLA_ERR_BAD_SHAPE;
  const bool fast = mla::prefill_fast_supported(*d, v);
  const size_t need = fast ? mla::prefill_fast_workspace(*d, batch, cache->max_context) : 0;
  if ((st = check_ws(ws, ws_bytes, need)) != MLA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (trace_on())
    fprintf(stderr, "[mla] prefill batch=%d seq_len=%d heads=%d path=%s ws=%zu\n", batch, seq_len, d->n_heads,
            fast ? "mfma" : "generic", need);
  if (fast)
    return hip_status(mla::prefill_fast(*d, scale_of(d), batch, seq_len, cache->max_context, q_nope, q_pe, w_uk,
                                        w_uv, v, out, ws, ws_bytes, s));
  return hip_status(mla::attn_generic(*d, scale_of(d), batch, seq_len, q_nope, q_pe, w_uk, w_uv, v, out, s));
}

}  // extern "C"
