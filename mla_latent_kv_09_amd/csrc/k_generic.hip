// Generic MLA kernels: fp32 FMA arithmetic, any supported dims, fp32 or bf16
// storage. They cover every shape the C ABI accepts (the MFMA kernels cover the
// DeepSeek-V3 latent shape in bf16) and are the correctness-first path.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace mla {

// ------------------------------------------------------------------ GEMM ---
// 64x64 output tile per block, K in steps of 16 through LDS, 4x4 per thread.
// Epilogue 0 stores C; epilogue 1 writes latent cache rows: columns < d_c as
// they are, columns >= d_c rotated in pairs at the token's position
// ("DeepSeek-V2 paper digest" §2.3: only the decoupled key slice is rotated).
struct Epi {
  int mode;
  void* c;
  int ldc;
  const int32_t* positions;
  const int32_t* slots;
  int d_c, d_rope;
  float base;
};

template <typename TA, typename TB, typename TC>
__global__ __launch_bounds__(256) void k_gemm_nt(int M, int N, int K, const TA* __restrict__ a, int lda,
                                                 const TB* __restrict__ b0, const TB* __restrict__ b1,
                                                 int n_split, int ldb, Epi ep) {
  __shared__ float As[16][65];
  __shared__ float Bs[16][65];
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int i = threadIdx.x; i < 64 * 16; i += 256) {
      const int r = i / 16, kk = i % 16, k = k0 + kk;
      const int m = m0 + r, n = n0 + r;
      As[kk][r] = (m < M && k < K) ? ld<TA>(a + (size_t)m * lda + k) : 0.f;
      float bv = 0.f;
      if (n < N && k < K)
        bv = n < n_split ? ld<TB>(b0 + (size_t)n * ldb + k) : ld<TB>(b1 + (size_t)(n - n_split) * ldb + k);
      Bs[kk][r] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { av[i] = As[kk][ty * 4 + i]; bv[i] = Bs[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
    if (ep.mode == 0) {
      TC* c = (TC*)ep.c + (size_t)m * ep.ldc;
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + tx * 4 + j;
        if (n < N) st<TC>(c + n, acc[i][j]);
      }
    } else {
      TC* row = (TC*)ep.c + (size_t)(ep.slots ? ep.slots[m] : m) * (ep.d_c + ep.d_rope);
      const int pos = ep.positions[m];
      for (int j = 0; j < 4; j += 2) {
        const int n = n0 + tx * 4 + j;   // even; d_c is a multiple of 8
        if (n >= N) continue;
        float x0 = acc[i][j], x1 = acc[i][j + 1];
        if (n >= ep.d_c) {
          double sn, cs;
          sincos(rope_angle(pos, (n - ep.d_c) / 2, ep.d_rope, ep.base), &sn, &cs);
          const float c = (float)cs, s = (float)sn;
          const float y0 = x0 * c - x1 * s, y1 = x0 * s + x1 * c;
          x0 = y0; x1 = y1;
        }
        st<TC>(row + n, x0);
        st<TC>(row + n + 1, x1);
      }
    }
  }
}

template <typename TA, typename TB, typename TC>
static hipError_t launch_gemm(int M, int N, int K, const void* a, int lda, const void* b0, const void* b1,
                              int n_split, int ldb, const Epi& ep, hipStream_t s) {
  dim3 grid((N + 63) / 64, (M + 63) / 64);
  hipLaunchKernelGGL((k_gemm_nt<TA, TB, TC>), grid, dim3(256), 0, s, M, N, K, (const TA*)a, lda,
                     (const TB*)b0, (const TB*)b1, n_split, ldb, ep);
  return hipGetLastError();
}

hipError_t gemm_nt_generic(int a_dtype, int b_dtype, int c_dtype, int M, int N, int K, const void* a, int lda,
                           const void* b0, const void* b1, int n_split, int ldb, void* c, int ldc,
                           hipStream_t s) {
  Epi ep{};
  ep.mode = 0;
  ep.c = c;
  ep.ldc = ldc;
  const int key = a_dtype * 4 + b_dtype * 2 + c_dtype;
  switch (key) {
    case 0: return launch_gemm<float, float, float>(M, N, K, a, lda, b0, b1, n_split, ldb, ep, s);
    case 1: return launch_gemm<float, float, bf16>(M, N, K, a, lda, b0, b1, n_split, ldb, ep, s);
    case 2: return launch_gemm<float, bf16, float>(M, N, K, a, lda, b0, b1, n_split, ldb, ep, s);
    case 3: return launch_gemm<float, bf16, bf16>(M, N, K, a, lda, b0, b1, n_split, ldb, ep, s);
    case 6: return launch_gemm<bf16, bf16, float>(M, N, K, a, lda, b0, b1, n_split, ldb, ep, s);
    case 7: return launch_gemm<bf16, bf16, bf16>(M, N, K, a, lda, b0, b1, n_split, ldb, ep, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t project_latent_generic(const mla_dims& d, int n_tokens, int d_model, const void* h,
                                  const void* w_dkv, const void* w_kr, const int32_t* positions,
                                  const int32_t* slots, void* rows, hipStream_t s) {
  Epi ep{};
  ep.mode = 1;
  ep.c = rows;
  ep.positions = positions;
  ep.slots = slots;
  ep.d_c = d.d_c;
  ep.d_rope = d.d_rope;
  ep.base = d.rope_base;
  const int N = d.d_c + d.d_rope;
  return d.dtype == MLA_F32
             ? launch_gemm<float, float, float>(n_tokens, N, d_model, h, d_model, w_dkv, w_kr, d.d_c, d_model, ep, s)
             : launch_gemm<bf16, bf16, bf16>(n_tokens, N, d_model, h, d_model, w_dkv, w_kr, d.d_c, d_model, ep, s);
}

// ------------------------------------------------------------- attention ---
// One block per (query, head), four waves. The block forms the absorbed query
// q_abs = W_UK,h^T q_nope and the rotated q_pe ("DeepSeek-V2 paper digest"
// §2.2, §2.3), then each wave walks every fourth cached token with an online
// softmax, keeping its share of the latent output o_c; the waves merge their
// (max, sum, o_c) through LDS and the block applies W_UV,h.
constexpr int GA_THREADS = 256;
constexpr int GA_MAX_DC = 1024;
constexpr int GA_MAX_DR = 128;

template <typename T>
__global__ __launch_bounds__(GA_THREADS) void k_attn_generic(
    int n_heads, int d_c, int d_rope, int d_nope, int d_v, float scale, float base, int q_per_seq,
    const T* __restrict__ q_nope, const T* __restrict__ q_pe, const T* __restrict__ w_uk,
    const T* __restrict__ w_uv, CacheView cv, T* __restrict__ out) {
  __shared__ float qabs[GA_MAX_DC + GA_MAX_DR];
  __shared__ float qn[256];
  __shared__ float opart[4][GA_MAX_DC];
  __shared__ float mw[4], lw[4];
  const int qi = blockIdx.x, h = blockIdx.y;
  const int b = qi / q_per_seq, s = qi % q_per_seq;
  const int R = d_c + d_rope;
  const int ctx = cv.context_lens[b] - q_per_seq + s + 1;  // tokens this query sees
  const int pos = ctx - 1;
  const int tid = threadIdx.x, lane = tid % 64, w = tid / 64;
  const size_t qrow = (size_t)qi * n_heads + h;
  T* o = out + qrow * d_v;
  if (ctx < 1) {  // no visible token (context shorter than the query count)
    for (int j = tid; j < d_v; j += GA_THREADS) st<T>(o + j, 0.f);
    return;
  }
  for (int j = tid; j < d_nope; j += GA_THREADS) qn[j] = ld<T>(q_nope + qrow * d_nope + j);
  for (int i = tid; i < d_rope / 2; i += GA_THREADS) {
    double sn, cs;
    sincos(rope_angle(pos, i, d_rope, base), &sn, &cs);
    const float x0 = ld<T>(q_pe + qrow * d_rope + 2 * i), x1 = ld<T>(q_pe + qrow * d_rope + 2 * i + 1);
    qabs[d_c + 2 * i] = x0 * (float)cs - x1 * (float)sn;
    qabs[d_c + 2 * i + 1] = x0 * (float)sn + x1 * (float)cs;
  }
  __syncthreads();
  const T* wk = w_uk + (size_t)h * d_nope * d_c;
  for (int c = tid; c < d_c; c += GA_THREADS) {
    float acc = 0.f;
    for (int j = 0; j < d_nope; ++j) acc = fmaf(ld<T>(wk + (size_t)j * d_c + c), qn[j], acc);
    qabs[c] = acc;
  }
  __syncthreads();

  float m = -INFINITY, l = 0.f;
  float acc[GA_MAX_DC / 64];
  const int n_own = (d_c + 63 - lane) / 64;  // latent columns lane, lane+64, ...
#pragma unroll
  for (int k = 0; k < GA_MAX_DC / 64; ++k) acc[k] = 0.f;
  for (int t = w; t < ctx; t += 4) {
    const T* row;
    if (cv.paged)
      row = (const T*)cv.rows +
            ((size_t)cv.block_table[(size_t)b * cv.max_blocks + t / cv.block_size] * cv.block_size +
             t % cv.block_size) * R;
    else
      row = (const T*)cv.rows + ((size_t)b * cv.seq_stride + t) * R;
    float part = 0.f;
    for (int e = lane; e < R; e += 64) part = fmaf(qabs[e], ld<T>(row + e), part);
    const float sc = wave_sum(part) * scale;
    const float mn = fmaxf(m, sc);
    const float alpha = expf(m - mn), p = expf(sc - mn);
    l = l * alpha + p;
#pragma unroll
    for (int k = 0; k < GA_MAX_DC / 64; ++k)
      if (k < n_own) acc[k] = acc[k] * alpha + p * ld<T>(row + lane + 64 * k);
    m = mn;
  }
#pragma unroll
  for (int k = 0; k < GA_MAX_DC / 64; ++k)
    if (k < n_own) opart[w][lane + 64 * k] = acc[k];
  if (lane == 0) { mw[w] = m; lw[w] = l; }
  __syncthreads();
  float M = -INFINITY;
  for (int i = 0; i < 4; ++i) M = fmaxf(M, mw[i]);
  float f[4], L = 0.f;
  for (int i = 0; i < 4; ++i) {
    f[i] = mw[i] == -INFINITY ? 0.f : expf(mw[i] - M);
    L += f[i] * lw[i];
  }
  const float invL = 1.f / L;
  __syncthreads();
  for (int c = tid; c < d_c; c += GA_THREADS)
    qabs[c] = (f[0] * opart[0][c] + f[1] * opart[1][c] + f[2] * opart[2][c] + f[3] * opart[3][c]) * invL;
  __syncthreads();
  const T* wv = w_uv + (size_t)h * d_v * d_c;
  for (int j = w; j < d_v; j += 4) {
    float part = 0.f;
    for (int c = lane; c < d_c; c += 64) part = fmaf(ld<T>(wv + (size_t)j * d_c + c), qabs[c], part);
    part = wave_sum(part);
    if (lane == 0) st<T>(o + j, part);
  }
}

hipError_t attn_generic(const mla_dims& d, float scale, int n_seq, int q_per_seq, const void* q_nope,
                        const void* q_pe, const void* w_uk, const void* w_uv, const CacheView& c,
                        void* out, hipStream_t s) {
  dim3 grid(n_seq * q_per_seq, d.n_heads);
  if (d.dtype == MLA_F32)
    hipLaunchKernelGGL(k_attn_generic<float>, grid, dim3(GA_THREADS), 0, s, d.n_heads, d.d_c, d.d_rope,
                       d.d_nope, d.d_v, scale, d.rope_base, q_per_seq, (const float*)q_nope,
                       (const float*)q_pe, (const float*)w_uk, (const float*)w_uv, c, (float*)out);
  else
    hipLaunchKernelGGL(k_attn_generic<bf16>, grid, dim3(GA_THREADS), 0, s, d.n_heads, d.d_c, d.d_rope,
                       d.d_nope, d.d_v, scale, d.rope_base, q_per_seq, (const bf16*)q_nope,
                       (const bf16*)q_pe, (const bf16*)w_uk, (const bf16*)w_uv, c, (bf16*)out);
  return hipGetLastError();
}

}  // namespace mla
