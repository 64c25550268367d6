/*
 * mla.h -- C ABI of an MI355X (gfx950) library for Multi-head Latent
 * Attention (MLA) over a compressed, paged latent KV cache.
 *
 * The method (DeepSeek-V2 / V3 attention):
 *   - "DeepSeek-V2 paper digest" (www.hncyxsy.com/news/273095) §2.1: keys and
 *     values of all heads are compressed jointly into one latent vector per
 *     token, c_KV = W_DKV h_t (W_DKV is [d_c, d_model]); the per-head keys and
 *     values are W_UK c_KV and W_UV c_KV (W_UK, W_UV are [n_heads*d, d_c]).
 *     Only c_KV is cached.
 *   - same page §2.2: W_UK can be folded into the query (q^T W_UK is formed
 *     first and dotted with the cached c_KV directly) and W_UV is applied to
 *     the attention output afterwards, so keys and values are never formed.
 *   - same page §2.3: RoPE is decoupled. A small rotary key k_pe, shared by all
 *     heads, is cached beside c_KV and only that slice carries position.
 *   - "8.1 DeepSeek architecture" (www.hdu-wiki.cn/courses/deepseek-architecture)
 *     §2: the same three equations, and the query path compressed likewise.
 *   - "DeepSeek 2025 technical report walkthrough" (m.nlpx.cn/news/79410) §3.3:
 *     with d_c = 512 and a 64-wide RoPE part a token costs 576 cached values.
 *
 * One cache row per token is [c_KV (d_c) || k_pe (d_rope)], row-major, in the
 * library's dtype. Rows live in pages of `block_size` tokens; a block table maps
 * each sequence's logical pages to physical pages of the pool.
 *
 * Conventions for every entry point
 *   - Pointers marked "device" are device memory owned by the caller; the
 *     library never frees or retains them and allocates no device memory
 *     (mla_decode_noalloc's fixed scratch array is part of the library's
 *     code object, one per GPU). All arrays are dense, row-major and 16-byte
 *     aligned.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and the call returns without waiting. Results are ready once the stream
 *     is synchronised. Calls on different streams need separate workspaces.
 *   - Arguments are checked on the host before anything is enqueued. On any
 *     status other than MLA_OK nothing has been enqueued and no output has been
 *     written, except MLA_ERR_HIP (a launch failed; outputs are undefined).
 *   - Device-side contents (block-table entries, context lengths, positions,
 *     slots) are not checked: values outside the documented ranges give
 *     undefined results.
 *   - RoPE rotates element pairs (2i, 2i+1) by pos * base^(-2i/d_rope). Keys are
 *     rotated once, when written; queries are passed unrotated and rotated
 *     inside decode/prefill at their own position.
 *   - Accumulation is fp32 for both dtypes. bf16 results round to nearest even.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL_ARG = 1,     /* a required pointer is NULL */
  MLA_ERR_BAD_SHAPE = 2,    /* a size or dimension is out of range or inconsistent */
  MLA_ERR_BAD_DTYPE = 3,    /* dtype is neither MLA_F32 nor MLA_BF16 */
  MLA_ERR_UNSUPPORTED = 4,  /* valid, but outside what this library implements */
  MLA_ERR_WORKSPACE = 5,    /* workspace smaller than the matching *_workspace_size */
  MLA_ERR_HIP = 6,          /* a HIP launch or query failed */
  MLA_ERR_ALIGNMENT = 7     /* a pointer is not 16-byte aligned */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

/* Model dimensions, shared by all entry points.
 * n_heads in [1, 256]; d_c in [8, 1024] and a multiple of 8; d_rope in [2, 128]
 * and even, with d_c + d_rope a multiple of 8; d_nope, d_v in [1, 256].
 * The DeepSeek-V3 shape is n_heads 128, d_c 512, d_rope 64, d_nope 128, d_v 128. */
typedef struct {
  int32_t n_heads;
  int32_t d_c;        /* latent width (c_KV) */
  int32_t d_rope;     /* decoupled rotary key width (k_pe, q_pe) */
  int32_t d_nope;     /* per-head non-rotary query/key width */
  int32_t d_v;        /* per-head value width */
  float softmax_scale;/* <= 0 selects 1/sqrt(d_nope + d_rope) */
  float rope_base;    /* RoPE base, e.g. 10000; must be > 1 */
  int32_t dtype;      /* mla_dtype of every array: cache, q, weights, h, outputs */
} mla_dims;

/* The latent cache.
 * Paged (block_table != NULL): rows is device [num_blocks, block_size, d_c + d_rope];
 *   token t of sequence b lives in page block_table[b * max_blocks_per_seq + t / block_size]
 *   at offset t % block_size. Entries must lie in [0, num_blocks).
 * Contiguous (block_table == NULL): rows is device [batch, max_context, d_c + d_rope]
 *   and token t of sequence b is row b * max_context + t; block_size,
 *   num_blocks and max_blocks_per_seq are ignored.
 * context_lens is device int32 [batch]; each entry is the number of cached
 * tokens of that sequence, in [1, max_context]. max_context is the host-side
 * upper bound used to size the launch without reading device memory. */
typedef struct {
  void* rows;
  int32_t num_blocks;
  int32_t block_size;
  const int32_t* block_table;
  int32_t max_blocks_per_seq;
  const int32_t* context_lens;
  int32_t max_context;
} mla_cache;

/* Optional low-rank query path of mla_rope_latent_project
 * ("DeepSeek-V2 paper digest" §4.3; "8.1 DeepSeek architecture" §2):
 * c_Q = W_DQ h, q_nope = W_UQ c_Q, q_pe = W_QR c_Q (q_pe left unrotated). */
typedef struct {
  int32_t d_q;          /* query latent width, in [8, 4096], multiple of 8 */
  const void* w_dq;     /* device [d_q, d_model] */
  const void* w_uq;     /* device [n_heads * d_nope, d_q] */
  const void* w_qr;     /* device [n_heads * d_rope, d_q] */
  void* q_nope;         /* device out [n_tokens, n_heads, d_nope] */
  void* q_pe;           /* device out [n_tokens, n_heads, d_rope] */
} mla_qproj;

/* Latent projection, RoPE and cache write ("DeepSeek-V2 paper digest" §2.1, §2.3).
 * For each token i: [c || k] = [W_DKV; W_KR] h_i (fp32 accumulate), k_pe =
 * RoPE(k, positions[i]), and the row [c || k_pe], rounded to the dtype, is
 * written to cache slot slots[i] (paged: page slots[i] / block_size, offset
 * slots[i] % block_size; contiguous: row slots[i]). Only the written rows of
 * the cache change; context_lens is not read or updated.
 *   h          device [n_tokens, d_model]
 *   w_dkv      device [d_c, d_model]
 *   w_kr       device [d_rope, d_model]
 *   positions  device int32 [n_tokens], >= 0
 *   slots      device int32 [n_tokens], distinct, inside the pool
 *   qproj      NULL, or the query path to run on the same tokens
 *   workspace  device scratch of at least mla_project_workspace_size bytes
 * n_tokens == 0 is a no-op returning MLA_OK. d_model in [1, 16384]. */
mla_status mla_rope_latent_project(const mla_dims* dims, int32_t n_tokens, int32_t d_model,
                                   const void* h, const void* w_dkv, const void* w_kr,
                                   const int32_t* positions, const int32_t* slots,
                                   const mla_cache* cache, const mla_qproj* qproj,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* Decode: one new query per sequence, attending to all of its cached tokens
 * ("DeepSeek-V2 paper digest" §2.2 absorbed form, §2.3 decoupled RoPE).
 * Sequence b's query sits at position context_lens[b] - 1 and sees cached
 * tokens 0 .. context_lens[b] - 1 (the new token's own row must already be in
 * the cache). Per head h:
 *   q_abs = W_UK,h^T q_nope[b,h]   (W_UK,h = rows h*d_nope .. of W_UK)
 *   s_t   = scale * (q_abs . c_t + RoPE(q_pe[b,h]) . k_pe_t)
 *   o_c   = sum_t softmax(s)_t c_t
 *   out[b,h] = W_UV,h o_c          (W_UV,h = rows h*d_v .. of W_UV)
 *   q_nope device [batch, n_heads, d_nope]
 *   q_pe   device [batch, n_heads, d_rope], unrotated
 *   w_uk   device [n_heads * d_nope, d_c]
 *   w_uv   device [n_heads * d_v, d_c]
 *   out    device [batch, n_heads, d_v]
 * batch == 0 is a no-op returning MLA_OK. */
mla_status mla_decode(const mla_dims* dims, int32_t batch,
                      const void* q_nope, const void* q_pe, const void* w_uk, const void* w_uv,
                      const mla_cache* cache, void* out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Multi-token decode: q_len new queries per sequence, the last q_len tokens
 * of its context, as a draft step of speculative decoding with multi-token
 * prediction produces them ("DeepSeek 2025 technical report walkthrough" §2.3;
 * "8.1 DeepSeek architecture" §6). Query j of sequence b sits at position
 * context_lens[b] - q_len + j and sees cached tokens 0 .. that position (causal
 * among the new tokens; their rows must already be in the cache). The result
 * is that of mla_prefill with seq_len = q_len, computed in the absorbed form of
 * mla_decode, which reads each cached row once per query instead of
 * up-projecting the context; mla_decode is the case q_len == 1.
 *   q_nope device [batch, q_len, n_heads, d_nope]
 *   q_pe   device [batch, q_len, n_heads, d_rope], unrotated
 *   out    device [batch, q_len, n_heads, d_v]
 * q_len in [1, 64] and <= max_context, batch * q_len <= 65535, else
 * MLA_ERR_BAD_SHAPE. context_lens[b] must be >= q_len: a query that sees no
 * cached token gets a zero output. batch == 0 is a no-op returning MLA_OK. */
mla_status mla_decode_multi(const mla_dims* dims, int32_t batch, int32_t q_len,
                            const void* q_nope, const void* q_pe, const void* w_uk, const void* w_uv,
                            const mla_cache* cache, void* out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* FP8 latent cache ("DeepSeek core techniques: MoE and MLA attention" §6.3:
 * the KV cache is quantised to FP8 dynamically for deployment; "8.1 DeepSeek
 * architecture" §5: one scale per block, not one global scale).
 * Format: E4M3 codes (OCP "fn": largest value 448, round to nearest even)
 * with one power-of-two scale per token. A page of block_size tokens is
 * block_size rows of [d_c code bytes || d_rope bf16 values of k_pe (kept
 * unquantised)], then block_size scale bytes E (scale 2^(E - 127)), then
 * padding to a multiple of 16 bytes (mla_fp8_page_bytes; 41,024 bytes for the
 * DeepSeek-V3 shape with 64-token pages, against 73,728 in bf16). A token's
 * scale is the smallest 2^e, e >= -127, with max|c_KV| <= 448 * 2^e; its
 * codes are RNE(c_KV / 2^e), so no code saturates. */
mla_status mla_fp8_page_bytes(const mla_dims* dims, int32_t block_size, size_t* bytes);

/* Quantises n_rows bf16 cache rows [n_rows, d_c + d_rope] (the layout
 * mla_rope_latent_project writes) into FP8 pages: row r goes to slot slots[r]
 * (slot r when slots is NULL), i.e. page slot / block_size, offset
 * slot % block_size. Only that row's bytes and scale byte are written (not the
 * padding). dims->dtype must be MLA_BF16. block_size in [1, 4096]. pool is
 * device memory of whole pages, 16-byte aligned. n_rows == 0 is a no-op. */
mla_status mla_quantize_fp8(const mla_dims* dims, int32_t n_rows, const void* rows, const int32_t* slots,
                            int32_t block_size, void* pool, void* stream);

/* Latent projection straight into an FP8 cache: the rows of
 * mla_rope_latent_project ("DeepSeek-V2 paper digest" §2.1, §2.3), quantised
 * as mla_quantize_fp8 does ("DeepSeek core techniques" §6.3: the cache is
 * quantised to FP8 as it is written), so the caller needs no bf16 cache. The
 * rows are formed in bf16 (fp32 accumulate, RoPE, rounding) in the workspace,
 * then quantised into pool (FP8 pages of block_size tokens) at slots; the pool
 * holds the same bytes as mla_rope_latent_project into a bf16 cache followed by
 * mla_quantize_fp8 of those rows. dims->dtype must be MLA_BF16; qproj as for
 * mla_rope_latent_project. workspace: mla_project_fp8_workspace_size bytes.
 * n_tokens == 0 is a no-op. */
mla_status mla_rope_latent_project_fp8(const mla_dims* dims, int32_t n_tokens, int32_t d_model, const void* h,
                                       const void* w_dkv, const void* w_kr, const int32_t* positions,
                                       const int32_t* slots, void* pool, int32_t block_size,
                                       const mla_qproj* qproj, void* workspace, size_t workspace_bytes,
                                       void* stream);

/* mla_decode_multi over an FP8 cache: cache->rows is the FP8 page pool, the
 * block table and lengths as for mla_decode. The scores use the FP8 matrix
 * core with the query q~ quantised like a cache row (one scale per head, its
 * RoPE slice in bf16), and P is rounded to FP8 for the value product, so the
 * result differs from the bf16 path's by FP8 rounding (a few percent of the
 * output, relative). Requires the DeepSeek-V3 latent shape (d_c 512, d_rope
 * 64, d_nope = d_v = 128, n_heads <= 128), bf16 queries and weights, 64-token
 * pages and a paged cache; other shapes return MLA_ERR_UNSUPPORTED. q_len and
 * batch bounds as for mla_decode_multi. */
mla_status mla_decode_fp8(const mla_dims* dims, int32_t batch, int32_t q_len,
                          const void* q_nope, const void* q_pe, const void* w_uk, const void* w_uv,
                          const mla_cache* cache, void* out,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Causal prefill: seq_len new queries per sequence, the last seq_len tokens of
 * its context. Query s of sequence b sits at position context_lens[b] - seq_len + s
 * and sees cached tokens 0 .. context_lens[b] - seq_len + s. With
 * context_lens[b] == seq_len this is plain causal self-attention over the
 * sequence; with a longer context it attends to the cached prefix as well
 * (chunked prefill). The math per query and head is that of mla_decode.
 *   q_nope device [batch, seq_len, n_heads, d_nope]
 *   q_pe   device [batch, seq_len, n_heads, d_rope], unrotated
 *   out    device [batch, seq_len, n_heads, d_v]
 * context_lens[b] must be >= seq_len. batch == 0 or seq_len == 0 is a no-op. */
mla_status mla_prefill(const mla_dims* dims, int32_t batch, int32_t seq_len,
                       const void* q_nope, const void* q_pe, const void* w_uk, const void* w_uv,
                       const mla_cache* cache, void* out,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Output side of the attention layer. W_O is device [d_model, n_heads * d_v]
 * ([out, in], like every weight here); head h's output feeds columns
 * h*d_v .. h*d_v + d_v - 1, the order in which the heads' outputs are
 * concatenated. d_model in [1, 65536].
 *
 * mla_output_project: out = W_O applied to each row's concatenated per-head
 * outputs, out[r] = W_O attn_out[r] (fp32 accumulate).
 *   attn_out device [n_rows, n_heads, d_v] (e.g. mla_decode's output)
 *   out      device [n_rows, d_model]
 *   workspace at least mla_output_workspace_size(dims, n_rows, d_model, 0)
 * n_rows == 0 is a no-op. */
mla_status mla_output_project(const mla_dims* dims, int32_t n_rows, int32_t d_model, const void* attn_out,
                              const void* w_o, void* out, void* workspace, size_t workspace_bytes, void* stream);

/* W_UV absorbed into W_O ("DeepSeek-V2 paper digest" §2.2: on the output side
 * W_UV can be absorbed into the output projection W_O, the weights being fused
 * before inference). Writes W_OUV, device [d_model, n_heads * d_c], whose
 * column block h (columns h*d_c .. h*d_c + d_c - 1) is W_O,h W_UV,h, with W_O,h
 * the d_v columns of W_O that take head h's output (fp32 accumulate, rounded
 * to the dtype). A one-time weight preparation for mla_decode_folded. */
mla_status mla_fold_output_weights(const mla_dims* dims, int32_t d_model, const void* w_uv, const void* w_o,
                                   void* w_ouv, void* stream);

/* Decode with the folded output weights: the scores and the latent output
 * o_c of each head as in mla_decode_multi (absorbed form), then
 * out[r] = sum_h W_OUV,h o_c[r, h], the attention layer's output, without
 * forming the per-head outputs. Equal to mla_decode_multi followed by
 * mla_output_project up to rounding (the fused weights are rounded to the
 * dtype once).
 *   w_ouv device [d_model, n_heads * d_c] (mla_fold_output_weights)
 *   out   device [batch, q_len, d_model]
 *   workspace at least mla_decode_folded_workspace_size bytes
 * Needs the MFMA decode path (bf16, the DeepSeek-V3 latent shape, 64-token
 * pages, paged cache); other shapes return MLA_ERR_UNSUPPORTED. Other bounds
 * as for mla_decode_multi. batch == 0 is a no-op. */
mla_status mla_decode_folded(const mla_dims* dims, int32_t batch, int32_t q_len, const void* q_nope,
                             const void* q_pe, const void* w_uk, const void* w_ouv, int32_t d_model,
                             const mla_cache* cache, void* out, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Decode without allocation and without a caller workspace, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation. Arguments, checks and result are
 * those of mla_decode_multi (q_len == 1 is mla_decode). The scratch memory it
 * needs comes from a device array inside the library of
 * MLA_NOALLOC_SCRATCH_BYTES (64 MiB), one per GPU the library runs on, held
 * until the process ends; its device address is looked up on the first call
 * on each device. A call whose mla_decode_multi_workspace_size exceeds the
 * array returns MLA_ERR_WORKSPACE before anything is enqueued (the DeepSeek-V3
 * shape with B = 64 sequences of 8192 tokens needs 43.3 MB). The array keeps
 * whatever the last call left; nothing in it needs to start cleared. Calls
 * that overlap on one GPU (other streams or threads) share the array and
 * race: serialise them. */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20)
mla_status mla_decode_noalloc(const mla_dims* dims, int32_t batch, int32_t q_len,
                              const void* q_nope, const void* q_pe, const void* w_uk, const void* w_uv,
                              const mla_cache* cache, void* out, void* stream);
size_t mla_noalloc_scratch_bytes(void);

/* Workspace each entry point needs for the given sizes (bytes, 0 possible). */
mla_status mla_project_workspace_size(const mla_dims* dims, int32_t n_tokens, int32_t d_q, size_t* bytes);
mla_status mla_decode_workspace_size(const mla_dims* dims, int32_t batch, int32_t max_context, size_t* bytes);
mla_status mla_decode_multi_workspace_size(const mla_dims* dims, int32_t batch, int32_t q_len,
                                           int32_t max_context, size_t* bytes);
mla_status mla_project_fp8_workspace_size(const mla_dims* dims, int32_t n_tokens, int32_t d_q, size_t* bytes);
mla_status mla_decode_fp8_workspace_size(const mla_dims* dims, int32_t batch, int32_t q_len,
                                         int32_t max_context, size_t* bytes);
mla_status mla_prefill_workspace_size(const mla_dims* dims, int32_t batch, int32_t seq_len,
                                      int32_t max_context, size_t* bytes);
/* folded = 0: mla_output_project; folded != 0: a product with W_OUV */
mla_status mla_output_workspace_size(const mla_dims* dims, int32_t n_rows, int32_t d_model, int32_t folded,
                                     size_t* bytes);
mla_status mla_decode_folded_workspace_size(const mla_dims* dims, int32_t batch, int32_t q_len,
                                            int32_t max_context, int32_t d_model, size_t* bytes);

/* One call for the three core entry points, with two sizes whose meaning
 * depends on op (the same values as the specific functions above):
 *   MLA_OP_PROJECT  size_a = n_tokens, size_b = d_q (0: no query path)
 *   MLA_OP_DECODE   size_a = batch,    size_b = max_context
 *   MLA_OP_PREFILL  size_a = batch,    size_b = seq_len (no cached prefix:
 *                   max_context = seq_len; for a prefix use
 *                   mla_prefill_workspace_size)
 * Another op gives MLA_ERR_UNSUPPORTED and leaves *bytes untouched. */
typedef enum { MLA_OP_PROJECT = 0, MLA_OP_DECODE = 1, MLA_OP_PREFILL = 2 } mla_op;
mla_status mla_workspace_size(int32_t op, const mla_dims* dims, int32_t size_a, int32_t size_b, size_t* bytes);

/* Static description of a status code (never NULL). */
const char* mla_status_string(mla_status status);

/* Which kernel family decode/prefill would use for these dims (for logs and
 * tests): 0 = generic fp32-FMA kernels, 1 = MFMA kernels. -1 on invalid dims. */
int32_t mla_decode_path(const mla_dims* dims, int32_t block_size, int32_t paged);
int32_t mla_prefill_path(const mla_dims* dims, int32_t block_size, int32_t paged);

/* Per-kernel timing for measurement tools. After mla_profile_begin, every
 * kernel the library launches is bracketed by HIP events on its stream (this
 * adds no synchronisation). mla_profile_end stops recording, waits for the
 * recorded events, and reports, per kernel name, the summed duration in ms
 * and the launch count: names is a caller buffer of max_kernels entries of
 * name_len chars each; *n_kernels receives the number of distinct kernels
 * (entries beyond max_kernels are dropped). Host-side state is shared by all
 * threads of the process. */
mla_status mla_profile_begin(void);
/* Restricts the timing to launches named kernel_name (as reported by
 * mla_profile_end), so a measured loop carries two events per step instead of
 * two per kernel; NULL or "" times every launch again. */
mla_status mla_profile_only(const char* kernel_name);
mla_status mla_profile_end(int32_t max_kernels, char* names, int32_t name_len, double* total_ms,
                           int32_t* launches, int32_t* n_kernels);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t mla_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_H */
