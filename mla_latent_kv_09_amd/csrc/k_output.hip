// Output side of the attention layer: the output projection W_O
// ([d_model, n_heads * d_v]; head h's output feeds columns h*d_v .. +d_v) and
// its fold with W_UV ("DeepSeek-V2 paper digest" §2.2: the value up-projection
// W_UV can be absorbed into W_O, fused once before inference, so the latent
// output o_c of each head goes straight into the layer output).
//
//   k_fold_wo      W_OUV[:, h*d_c + c] = sum_v W_O[:, h*d_v + v] W_UV[h*d_v + v, c]
//                  (one-time weight preparation; fp32 FMA, any dims)
//   k_rowgemm      partial[s][m][n] = sum over the s-th slice of k of
//                  X[m][k] W[n][k] for few rows m (decode: one row per query):
//                  16x16x32 bf16 MFMA with both operands loaded straight from
//                  memory into registers; the weight streams from HBM once,
//                  split over k so that enough workgroups stream it at once
//   k_rowgemm_sum  out[m][n] = sum_s partial[s][m][n], rounded to bf16
#include <math.h>

#include "common.h"
#include "launch.h"

namespace mla {
namespace {

// block: 64 output rows j x 64 latent columns c of head h = blockIdx.z; v in
// steps of 32 through LDS, 4 x 4 outputs per thread
template <typename T>
__global__ __launch_bounds__(256) void k_fold_wo(int d_model, int H, int dv, int dc, const T* __restrict__ w_uv,
                                                 const T* __restrict__ w_o, T* __restrict__ w_ouv) {
  __shared__ float As[32][65];  // W_O[j0 + r, h*dv + v0 + kk] at [kk][r]
  __shared__ float Bs[32][65];  // W_UV[h*dv + v0 + kk, c0 + r] at [kk][r]
  const int h = blockIdx.z, j0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const size_t ld_o = (size_t)H * dv;
  float acc[4][4] = {};
  for (int v0 = 0; v0 < dv; v0 += 32) {
    for (int i = threadIdx.x; i < 64 * 32; i += 256) {
      const int r = i / 32, kk = i % 32, j = j0 + r, v = v0 + kk;
      As[kk][r] = (j < d_model && v < dv) ? ld<T>(w_o + (size_t)j * ld_o + (size_t)h * dv + v) : 0.f;
    }
    for (int i = threadIdx.x; i < 64 * 32; i += 256) {
      const int kk = i / 64, r = i % 64, v = v0 + kk, c = c0 + r;
      Bs[kk][r] = (v < dv && c < dc) ? ld<T>(w_uv + ((size_t)h * dv + v) * dc + c) : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = As[kk][ty * 4 + i];
        bv[i] = Bs[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  const size_t ld_ouv = (size_t)H * dc;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = j0 + ty * 4 + i;
    if (j >= d_model) continue;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int c = c0 + tx * 4 + jj;
      if (c < dc) st<T>(w_ouv + (size_t)j * ld_ouv + (size_t)h * dc + c, acc[i][jj]);
    }
  }
}

constexpr int RG_N = 64;     // weight rows per work item
constexpr int RG_M = 64;     // activation rows per work item
constexpr int RG_SK = 128;   // k per LDS stage: 4 MFMA steps, one per wave
constexpr int RG_STAGES = 5;
constexpr int RG_TILE_BYTES = 64 * RG_SK * 2;            // 16 KB: 64 rows x 256 bytes
constexpr int RG_STAGE_BYTES = 2 * RG_TILE_BYTES;        // weight tile, then activation tile
constexpr int RG_DMA = RG_TILE_BYTES / 16 / 256;         // 4 copies per lane per tile
static_assert(RG_STAGES * RG_STAGE_BYTES <= 160 * 1024, "LDS budget of one workgroup");
static_assert(RG_M * RG_N * 4 <= RG_STAGE_BYTES, "an item's sums fit in one stage");

template <int N>
__device__ __forceinline__ void rg_wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ void rg_lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// one 16-byte HBM -> LDS copy per lane, to lds_addr + 16 * lane (lds_addr
// wave-uniform, through M0); base uniform, voff the lane's byte offset. Issued
// from asm so that the compiler does not drain all loads before each LDS read;
// the kernel orders the copies with explicit vmcnt waits before the barrier
// that publishes a stage. Nothing else in the kernel uses M0.
__device__ __forceinline__ void rg_dma16(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds_addr)
               : "memory", "m0");
}

// Persistent: one workgroup of 4 waves per CU walks the work items
// blockIdx.x, blockIdx.x + gridDim.x, ... An item (weight tile nt, k slice sp,
// activation tile mt) computes C^T[n, m] for 64 weight rows n and 64
// activation rows m over k in [sp kc, (sp + 1) kc): the partial sum
// part[sp][m][n]. The stages of all of a workgroup's items form one stream:
// weight and activation tiles of 64 rows x 128 k go HBM -> LDS (each copy
// instruction moves four whole 256-byte row segments) through a ring of five
// stages, four in flight across item boundaries, so 64 KB of the weight per
// CU stays outstanding from the first stage to the last, with no register
// loads in the loop (whose waits the compiler would place behind the copies).
// Tile position p (16-byte units) holds chunk (p % 16) ^ (row % 16) of row
// p / 16, so the 16 rows one fragment read touches sit in 16 distinct bank
// groups. Wave w takes MFMA step w of every stage with all 64 x 64 outputs
// (4 x 4 tiles of 16 x 16: A = weight rows, lane row 16i + l%16, k +
// 8(l/16) .. +7; B = activation rows 16t + l%16, the same k), so each
// fragment feeds four MFMAs. At an item's last stage the four waves' sums
// are added in LDS, in the slot of that stage (whose next copies are issued
// only after the following barrier), and stored. Rows past M or N are
// clamped to the last row
// (read, never stored). K % 128 == 0 and kc % 128 == 0, kc divides K.
__global__ __launch_bounds__(256, 1) void k_rowgemm(int M, int N, int K, int kc, int n_items,
                                                    const bf16* __restrict__ x, const bf16* __restrict__ wt,
                                                    float* __restrict__ part) {
  __shared__ __attribute__((aligned(1024))) char lds[RG_STAGES * RG_STAGE_BYTES];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i16 = lane & 15, G = lane >> 4;
  const int n_tiles = (N + RG_N - 1) / RG_N, m_tiles = (M + RG_M - 1) / RG_M;
  const int spi = kc / RG_SK;  // stages per item
  const int my_items = n_items > (int)blockIdx.x ? (n_items - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  const int total = my_items * spi;
  // item j of this workgroup: id = blockIdx.x + j gridDim.x = (sp n_tiles + nt) m_tiles + mt, so the
  // items that run at the same time share k slices (and the activation rows in L2)
  auto item_coords = [&](int j, int& nt, int& sp, int& mt) {
    const int id = (int)blockIdx.x + j * (int)gridDim.x;
    mt = id % m_tiles;
    nt = (id / m_tiles) % n_tiles;
    sp = id / (m_tiles * n_tiles);
  };
  // copy j of wave w fills tile positions (4w + j) * 64 + lane: row r, chunk c
  uint32_t rel[RG_DMA];  // r * K * 2 + 16 c (the row is clamped per item)
  int rows_r[RG_DMA];
#pragma unroll
  for (int j = 0; j < RG_DMA; ++j) {
    const int pos = (4 * w + j) * 64 + lane, r = pos >> 4, c = (pos & 15) ^ (r & 15);
    rows_r[j] = r;
    rel[j] = 16u * c;
  }
  const uint32_t lds_base = (uint32_t)(size_t)(LDS_AS char*)lds;
  auto issue_stage = [&](int g) {
    int nt, sp, mt;
    item_coords(g / spi, nt, sp, mt);
    const int st = g % spi, n0 = nt * RG_N, m0 = mt * RG_M;
    const size_t k0 = (size_t)sp * kc + (size_t)st * RG_SK;
    const char* ws = (const char*)(wt + (size_t)n0 * K + k0);
    const char* xs = (const char*)(x + (size_t)m0 * K + k0);
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_base + (g % RG_STAGES) * RG_STAGE_BYTES +
                                                        w * RG_DMA * 1024);
#pragma unroll
    for (int j = 0; j < RG_DMA; ++j)
      rg_dma16(ws, (uint32_t)(min(n0 + rows_r[j], N - 1) - n0) * (uint32_t)K * 2u + rel[j], dst + j * 1024);
#pragma unroll
    for (int j = 0; j < RG_DMA; ++j)
      rg_dma16(xs, (uint32_t)(min(m0 + rows_r[j], M - 1) - m0) * (uint32_t)K * 2u + rel[j],
               dst + RG_TILE_BYTES + j * 1024);
  };
  // fragment reads: row 16i + i16 of a tile, chunk (4w + G) ^ i16
  const uint32_t f_off = (uint32_t)(i16 * 256 + (((4 * w + G) ^ i16) << 4));

  f32x4 acc[4][4] = {};  // [weight tile i][activation tile t]
  for (int g = 0; g < RG_STAGES - 1 && g < total; ++g) issue_stage(g);
  for (int g = 0; g < total; ++g) {
    // stage g's copies (8 per lane) are done once at most those of the
    // stages after it that were issued are still out
    const int after = min(RG_STAGES - 2, total - 1 - g);
    if (after >= 3) rg_wait_vmcnt<3 * 2 * RG_DMA>();
    else if (after == 2) rg_wait_vmcnt<2 * 2 * RG_DMA>();
    else if (after == 1) rg_wait_vmcnt<2 * RG_DMA>();
    else rg_wait_vmcnt<0>();
    rg_lds_barrier();  // stage g visible to all; stage g - 1 (the slot of g + 4) read by all
    if (g + RG_STAGES - 1 < total) issue_stage(g + RG_STAGES - 1);
    const LDS_AS char* sb = (const LDS_AS char*)lds + (g % RG_STAGES) * RG_STAGE_BYTES + f_off;
    u32x4 a[4], bx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *(const LDS_AS u32x4*)(sb + i * 16 * 256);
#pragma unroll
    for (int t = 0; t < 4; ++t) bx[t] = *(const LDS_AS u32x4*)(sb + RG_TILE_BYTES + t * 16 * 256);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[i]),
                                                            __builtin_bit_cast(bf16x8_t, bx[t]), acc[i][t], 0, 0, 0);
    if (g % spi != spi - 1) continue;
    // last stage of an item: lane holds C^T[n0 + 16i + 4G + r][m0 + 16t + l%16]
    // (4 consecutive n of one m); the waves add theirs in turn into [m][n]
    // sums in this stage's slot, once every wave has read its fragments
    float* red = (float*)(lds + (g % RG_STAGES) * RG_STAGE_BYTES);
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      rg_lds_barrier();
      if (w == ww) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            float* r = red + (16 * t + i16) * RG_N + 16 * i + 4 * G;
            if (ww == 0) {
              *(f32x4*)r = acc[i][t];
            } else {
              const f32x4 o = *(const f32x4*)r;
              *(f32x4*)r = (f32x4){o[0] + acc[i][t][0], o[1] + acc[i][t][1], o[2] + acc[i][t][2],
                                   o[3] + acc[i][t][3]};
            }
            acc[i][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
          }
      }
    }
    rg_lds_barrier();
    int nt, sp, mt;
    item_coords(g / spi, nt, sp, mt);
    const int n0 = nt * RG_N, m0 = mt * RG_M;
    // 64 rows m of 64 n: 16 threads per row, 4 n each
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int mm = 16 * u + (threadIdx.x >> 4), nn = 4 * (threadIdx.x & 15);
      const int m = m0 + mm, n = n0 + nn;
      if (m < M && n < N) *(f32x4*)(part + ((size_t)sp * M + m) * N + n) = *(const f32x4*)(red + mm * RG_N + nn);
    }
    // the copies into this slot are issued only after the next stage's
    // barrier, which every wave reaches after these reads
  }
}

// out[m, n .. n+3] = sum_s part[s][m][n .. n+3] (N % 4 == 0)
__global__ __launch_bounds__(256) void k_rowgemm_sum(int M, int N, int splits, const float* __restrict__ part,
                                                     bf16* __restrict__ out) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4, total = (size_t)M * N;
  if (i >= total) return;
  f32x4 s = *(const f32x4*)(part + i);
  for (int sp = 1; sp < splits; ++sp) {
    const f32x4 v = *(const f32x4*)(part + (size_t)sp * total + i);
    s[0] += v[0];
    s[1] += v[1];
    s[2] += v[2];
    s[3] += v[3];
  }
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
  *(bf16x4_t*)(out + i) = (bf16x4_t){(__bf16)s[0], (__bf16)s[1], (__bf16)s[2], (__bf16)s[3]};
}

struct RowPlan {
  int splits, kc, items, grid;
};

// k slices: kc a multiple of 128 that divides K. A CU streams its items one
// after another at a rate set by the bytes it keeps in flight, so the time
// goes as (rounds of items per CU) x (weight bytes per item), plus the fp32
// partial sums of every slice (written, then read by the sum), spread over
// all CUs; the plan takes the slice count with the least of that.
RowPlan row_plan(int M, int N, int K, int cus) {
  const int tiles = ((N + RG_N - 1) / RG_N) * ((M + RG_M - 1) / RG_M);
  const int S = K / RG_SK;
  const double w_bytes = 2.0 * N * K, p_bytes = 8.0 * M * N;
  RowPlan best{1, K, tiles, tiles < cus ? tiles : cus};
  double best_cost = -1.0;
  for (int s = 1; s <= S && s <= 64; ++s) {
    if (S % s) continue;
    const int items = tiles * s;
    const int rounds = (items + cus - 1) / cus;
    const double cost = rounds * w_bytes / items + (s > 1 ? p_bytes * s / cus : 0.0);
    if (best_cost < 0.0 || cost < best_cost) {
      best_cost = cost;
      best = RowPlan{s, K / s, items, items < cus ? items : cus};
    }
  }
  return best;
}

bool row_path(const mla_dims& d, int M, int N, int K) {
  return d.dtype == MLA_BF16 && M <= 256 && K % RG_SK == 0 && N % 4 == 0;
}

}  // namespace

size_t rows_times_weight_workspace(const mla_dims& d, int M, int N, int K) {
  if (!row_path(d, M, N, K)) return 0;
  const RowPlan p = row_plan(M, N, K, device_cus());
  return (size_t)p.splits * M * N * sizeof(float);
}

hipError_t rows_times_weight(const mla_dims& d, int M, int N, int K, const void* x, const void* w, void* out,
                             void* ws, size_t ws_bytes, const char* prof_name, hipStream_t s) {
  ProfScope ps(prof_name, s);
  if (row_path(d, M, N, K)) {
    const RowPlan p = row_plan(M, N, K, device_cus());
    if (ws_bytes < (size_t)p.splits * M * N * sizeof(float)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_rowgemm, dim3(p.grid), dim3(256), 0, s, M, N, K, p.kc, p.items, (const bf16*)x,
                       (const bf16*)w, (float*)ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t quads = (size_t)M * N / 4;
    hipLaunchKernelGGL(k_rowgemm_sum, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, s, M, N, p.splits,
                       (const float*)ws, (bf16*)out);
    return hipGetLastError();
  }
  if (d.dtype == MLA_BF16 && gemm_fast_supported(M, N, K)) {
    GemmArgs g{};
    g.M = M;
    g.N = N;
    g.K = K;
    g.a = (const bf16*)x;
    g.lda = K;
    g.b0 = g.b1 = (const bf16*)w;
    g.n_split = N;
    g.ldb = K;
    g.c0 = g.c1 = (bf16*)out;
    g.ldc0 = g.ldc1 = N;
    g.c_split = N;
    return gemm_fast(g, 0, s);
  }
  return gemm_nt_generic(d.dtype, d.dtype, d.dtype, M, N, K, x, K, w, w, N, K, out, N, s);
}

hipError_t fold_output_weights(const mla_dims& d, int d_model, const void* w_uv, const void* w_o, void* w_ouv,
                               hipStream_t s) {
  ProfScope ps("mla_fold_output_weights", s);
  const dim3 grid((d.d_c + 63) / 64, (d_model + 63) / 64, d.n_heads);
  if (d.dtype == MLA_BF16)
    hipLaunchKernelGGL(k_fold_wo<bf16>, grid, dim3(256), 0, s, d_model, d.n_heads, d.d_v, d.d_c, (const bf16*)w_uv,
                       (const bf16*)w_o, (bf16*)w_ouv);
  else
    hipLaunchKernelGGL(k_fold_wo<float>, grid, dim3(256), 0, s, d_model, d.n_heads, d.d_v, d.d_c,
                       (const float*)w_uv, (const float*)w_o, (float*)w_ouv);
  return hipGetLastError();
}

}  // namespace mla
