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
// Latent rows: [c || RoPE(k)] = [W_DKV; W_KR] h, written to row slots[i] of rows.
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
size_t decode_fast_workspace(const mla_dims& d, int batch, int max_context);
hipError_t decode_fast(const mla_dims& d, float scale, int batch, int max_context,
                       const void* q_nope, const void* q_pe, const void* w_uk, const void* w_uv,
                       const CacheView& c, void* out, void* ws, size_t ws_bytes, hipStream_t s);

}  // namespace mla
