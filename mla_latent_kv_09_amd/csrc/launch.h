// Internal launchers (host side) of the MLA kernel families.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

// Records HIP events around the launches in its scope when profiling is on
// (mla_profile_begin); a no-op otherwise.
class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t s);
  ~ProfScope();

 private:
  const char* name_;
  hipStream_t s_;
  void* start_;
};

// Where cache row (b, t) lives. Paged: rows + (table[b][t / bs] * bs + t % bs) * R.
// Contiguous: rows + (b * seq_stride + t) * R.
struct CacheView {
  void* rows;
  const int32_t* block_table;
  const int32_t* context_lens;
  int32_t block_size;
  int32_t max_blocks;
  int32_t paged;
  int32_t seq_stride;
};

// ---- generic kernels (fp32 FMA, any supported dims, both dtypes) ----------
// C[m, n] = sum_k A[m, k] * B[n, k]; B rows n < n_split come from b0, the rest
// from b1 (row n - n_split). Each operand has its own dtype (MLA_F32/MLA_BF16).
hipError_t gemm_nt_generic(int a_dtype, int b_dtype, int c_dtype, int M, int N, int K,
                           const void* a, int lda, const void* b0, const void* b1, int n_split,
                           int ldb, void* c, int ldc, hipStream_t s);
// Latent rows: [c || RoPE(k)] = [W_DKV; W_KR] h, written to row slots[i] of rows
// (row i when slots is null; likewise for project_fast).
hipError_t project_latent_generic(const mla_dims& d, int n_tokens, int d_model, const void* h,
                                  const void* w_dkv, const void* w_kr, const int32_t* positions,
                                  const int32_t* slots, void* rows, hipStream_t s);
// Attention for n_seq * q_per_seq queries, query s of sequence b at position
// context_lens[b] - q_per_seq + s, seeing tokens 0 .. that position.
hipError_t attn_generic(const mla_dims& d, float scale, int n_seq, int q_per_seq,
                        const void* q_nope, const void* q_pe, const void* w_uk, const void* w_uv,
                        const CacheView& c, void* out, hipStream_t s);

// ---- MFMA kernels (bf16, DeepSeek-V3 latent shape) ------------------------
bool decode_fast_supported(const mla_dims& d, const CacheView& c);
// contexts up to 256 runs of 64 pages (1,048,576 tokens) per sequence
bool decode_fast_context_ok(int max_context);
// n_seq sequences with q_len new queries each (query j of sequence b at
// position context_lens[b] - q_len + j); q_len == 1 is plain decode
size_t decode_fast_workspace(const mla_dims& d, int n_seq, int q_len, int max_context);
hipError_t decode_fast(const mla_dims& d, float scale, int n_seq, int q_len, int max_context,
                       const void* q_nope, const void* q_pe, const void* w_uk, const void* w_uv,
                       const CacheView& c, void* out, void* ws, size_t ws_bytes, hipStream_t s);

// Pieces of the decode path that the FP8-cache decode shares (rows = query
// rows, n_seq * q_len). decode_absorb writes q~ [rows, H, 576] bf16;
// decode_combine merges per-split partials [H][rows][splits][512] bf16 and
// (m, l) [H][rows][splits][2] and applies W_UV (w_uv == nullptr: writes the
// merged latent output o_c [rows, H, 512] bf16 instead; so does decode_fast).
// run_pages (device) holds the pages per run the split kernel used, at least
// decode_plan's pages_per_split, so a row has at most `splits` runs.
// device_cus is the current device's compute-unit count.
void decode_plan(int rows, int max_context, int q_len, int* pages_per_split, int* splits);
int device_cus();
hipError_t decode_absorb(const mla_dims& d, float scale, int rows, int q_len, const void* q_nope, const void* q_pe,
                         const void* w_uk, const int32_t* ctx_lens, void* qt, const char* prof_name, hipStream_t s);
hipError_t decode_combine(const mla_dims& d, int rows, int q_len, int splits, const int32_t* run_pages,
                          const int32_t* ctx_lens, const void* part_o, const float* part_ml, const void* w_uv,
                          void* out, const char* prof_name, hipStream_t s);

// ---- FP8 latent cache (E4M3 codes, one power-of-two scale per token) ------
// Page of P tokens: P rows of [d_c codes || d_rope bf16 k_pe], then P scale
// bytes (value 2^(E - 127)), padded to 16 bytes.
size_t fp8_page_bytes(int page, int d_c, int d_rope);
hipError_t quant_fp8(const mla_dims& d, int n_rows, const void* src, const int32_t* slots, int page, void* dst,
                     hipStream_t s);
bool decode_fp8_supported(const mla_dims& d, const CacheView& c);
size_t decode_fp8_workspace(const mla_dims& d, int n_seq, int q_len, int max_context);
hipError_t decode_fp8(const mla_dims& d, float scale, int n_seq, int q_len, int max_context, const void* q_nope,
                      const void* q_pe, const void* w_uk, const void* w_uv, const CacheView& c, void* out, void* ws,
                      size_t ws_bytes, hipStream_t s);

// ---- MFMA GEMM (bf16, K multiple of 64, N multiple of 4) -----------------
// C[m, n] = sum_k A[m, k] B[n, k]; A and B rows are K-contiguous.
struct GemmArgs {
  int M, N, K;
  // A operand rows: plain (a + m * lda) or gathered from a paged latent cache
  // (row m = (b, t) with b = m / a_seq, t = m % a_seq; rows t >= context are
  // read from row 0 of the sequence and never used).
  const uint16_t* a;
  int lda;
  const int32_t* a_table;
  const int32_t* a_lens;
  int a_seq, a_max_blocks, a_block;
  // B operand rows n < n_split from b0, the rest from b1 (row n - n_split)
  const uint16_t* b0;
  const uint16_t* b1;
  int n_split, ldb;
  // plain epilogue: columns n < c_split to c0[m, n], the rest to c1[m, n - c_split]
  uint16_t* c0;
  uint16_t* c1;
  int ldc0, ldc1, c_split;
  // latent epilogue
  const int32_t* slots;
  const int32_t* positions;
  int d_c, d_rope;
  float rope_base;
};

bool gemm_fast_supported(int M, int N, int K);
// epi 0: store C[m, n]; 1: latent rows (RoPE + slot scatter). With m = (b, t)
// as for the gathered A rows and n = (h, d), heads of 128 columns (N % 128 == 0,
// a_seq a multiple of 64):
// 2: c0[b][h][t / 64][d][t % 64] (values transposed in 64-token blocks);
// 3: c0[b][h][t][d] (head-major)
hipError_t gemm_fast(const GemmArgs& g, int epi, hipStream_t s);

// ---- output side: W_O, and W_UV folded into W_O ---------------------------
// out[m, n] = sum_k X[m, k] W[n, k] for X [M, K] and W [N, K] (K-contiguous,
// the dims' dtype): the MFMA row GEMM (bf16, K % 32 == 0, N % 4 == 0) for few
// rows, the tiled MFMA GEMM for many, the generic kernel otherwise.
size_t rows_times_weight_workspace(const mla_dims& d, int M, int N, int K);
hipError_t rows_times_weight(const mla_dims& d, int M, int N, int K, const void* x, const void* w, void* out,
                             void* ws, size_t ws_bytes, const char* prof_name, hipStream_t s);
// W_OUV[:, h*d_c .. h*d_c + d_c) = W_O[:, h*d_v .. h*d_v + d_v) W_UV,h
hipError_t fold_output_weights(const mla_dims& d, int d_model, const void* w_uv, const void* w_o, void* w_ouv,
                               hipStream_t s);

// ---- MFMA prefill attention (bf16, DeepSeek-V3 latent shape) --------------
bool prefill_fast_supported(const mla_dims& d, const CacheView& c);
size_t prefill_fast_workspace(const mla_dims& d, int batch, int max_context);
hipError_t prefill_fast(const mla_dims& d, float scale, int batch, int seq_len, int max_context,
                        const void* q_nope, const void* q_pe, const void* w_uk, const void* w_uv,
                        const CacheView& c, void* out, void* ws, size_t ws_bytes, hipStream_t s);

// ---- projection with the MFMA GEMM ----------------------------------------
bool project_fast_supported(const mla_dims& d, int d_model, int d_q);
hipError_t project_fast(const mla_dims& d, int n_tokens, int d_model, const void* h, const void* w_dkv,
                        const void* w_kr, const int32_t* positions, const int32_t* slots, void* rows,
                        const mla_qproj* qp, void* ws, hipStream_t s);

}  // namespace mla
