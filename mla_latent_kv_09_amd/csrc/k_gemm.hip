// bf16 MFMA GEMM for the projections of the prefill path (gfx950):
//   C[m, n] = sum_k A[m, k] * B[n, k]       (fp32 accumulate)
// Both operands are K-contiguous ([rows, K] row-major), the orientation of the
// pages' [out, in] weights applied to [tokens, in] activations.
//
// Block tile: 256 rows of A x 128 (or 256) rows of B, K in steps of 64
// through a ring of LDS stages filled by direct 16-byte HBM -> LDS copies.
// Four (or eight) waves, each owning 128 A-rows x 64 B-rows as 4 x 2 tiles of
// 32 x 32 (or 4 x 4 with 256-wide tiles and four waves). Each wave computes
// the transposed tile C^T[n, m] (B rows as the MFMA M side), so a lane ends with
// 4 consecutive output columns n of one row m: RoPE pairs (2i, 2i+1) sit in one
// lane and stores are 8 bytes wide.
//
// Epilogues: plain store (optionally split into two outputs by column), the
// latent-cache epilogue of "DeepSeek-V2 paper digest" §2.1/§2.3 (columns >=
// d_c are rotated in pairs at the token's position, then the row
// [c_KV || k_pe] is written to its cache slot), and two per-head stores for
// the prefill keys and values: C[m, n] with m = (sequence b, token t) and n =
// (head h, dim d) goes head-major to [b][h][t][d], or transposed in blocks of
// 64 tokens to [b][h][t / 64][d][t % 64] (for the latter the MFMA operands
// swap sides, so a lane holds 4 consecutive rows m of one column n and stores
// them as 8 bytes).
#include <math.h>

#include "common.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int BM = 256, BK = 64;
constexpr int A_STAGE = BM * BK * 2;  // 32 KB
constexpr int HEAD_W = 128;  // head width of the per-head epilogues

// Block tile 256 x BN with BN = 64 NI, WAVES waves: two along the A rows (128
// each) and WAVES / 2 along the B rows, so each wave owns 128 A-rows x
// 64 NI / (WAVES / 2) B-rows (4 x NW MFMA tiles of 32 x 32). NI = 2: 256 x
// 128, three 48 KB stages; NI = 3: 256 x 192, two 56 KB stages (the latent
// projection, whose 576 columns are three such tiles); NI = 4: 256 x 256, two
// 64 KB stages (half the copies per MFMA). With 8 waves (NI = 4 only) two waves share each SIMD, so
// one wave's copies, LDS reads and epilogue stores issue while the other's
// MFMAs run; each then holds 128 accumulators instead of 256.
template <int NI, int WAVES>
struct Tile {
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int WN = WAVES / 2;
  static constexpr int NW = 2 * NI / WN;  // 32-wide B tiles per wave
  static constexpr int BN = 64 * NI;
  static constexpr int B_STAGE = BN * BK * 2;
  static constexpr int STAGE = A_STAGE + B_STAGE;
  static constexpr int N_STAGES = NI == 2 ? 3 : 2;
  static constexpr int A_LOADS = A_STAGE / 16 / THREADS;  // 8 or 4 per lane
  static constexpr int B_LOADS = B_STAGE / 16 / THREADS;  // 4 or 8 (or 4) per lane
  static constexpr int LOADS = A_LOADS + B_LOADS;
  static_assert(NW >= 1 && 2 * WN == WAVES, "wave layout");
};

template <int N>
__device__ __forceinline__ void g_wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ void g_lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void g_dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_addr)
               : "memory", "m0");
}
__device__ __forceinline__ bf16x8_t g_as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// 16-byte chunk c (of 8) of tile row r sits at chunk c ^ ((r >> 1) & 7): 16
// consecutive rows reading the same chunk hit 16 distinct bank groups.
__device__ __forceinline__ int g_swz(int r) { return (r >> 1) & 7; }

}  // namespace


namespace {

__device__ __forceinline__ const bf16* a_row_ptr(const GemmArgs& g, int m) {
  m = min(m, g.M - 1);
  if (!g.a_table) return g.a + (size_t)m * g.lda;
  const int b = m / g.a_seq, t = m % g.a_seq;
  const int tt = t < g.a_lens[b] ? t : 0;
  const int slot = g.a_table[(size_t)b * g.a_max_blocks + tt / g.a_block] * g.a_block + tt % g.a_block;
  return g.a + (size_t)slot * g.lda;
}

__device__ __forceinline__ const bf16* b_row_ptr(const GemmArgs& g, int n) {
  n = min(n, g.N - 1);
  return n < g.n_split ? g.b0 + (size_t)n * g.ldb : g.b1 + (size_t)(n - g.n_split) * g.ldb;
}

template <int EPI, int NI, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 1) void k_gemm(GemmArgs g) {
  using TL = Tile<NI, WAVES>;
  constexpr int BN = TL::BN, STAGE = TL::STAGE, N_STAGES = TL::N_STAGES, B_LOADS = TL::B_LOADS;
  constexpr int LOADS = TL::LOADS, A_LOADS = TL::A_LOADS, NW = TL::NW, G_THREADS = TL::THREADS;
  // the K-step stages, reused at the end to stage the output tile (rows of
  // 256 columns plus 16 bytes of padding)
  constexpr int CT_PITCH = 256 + 8;  // bf16 elements per staged row
  constexpr int LDS_BYTES = N_STAGES * STAGE > 256 * CT_PITCH * 2 ? N_STAGES * STAGE : 256 * CT_PITCH * 2;
  __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];
  const int n_tiles = (g.N + BN - 1) / BN;
  const int bid = blockIdx.x;
  // Tile order. Block i runs on XCD i % 8. With few N-tiles per M-tile (the
  // long-K projections from the hidden state), the N-tiles of one M-tile are
  // given to one XCD back to back, so its L2 fetches each A slice once for all
  // of them; otherwise plain row order (A shared across the XCDs).
  const int m_tiles = (g.M + BM - 1) / BM;
  int mt = bid / n_tiles, nt = bid % n_tiles;
  if ((NI == 2 || NI == 3) && n_tiles <= 16 && m_tiles % 8 == 0) {
    const int xcd = bid & 7, local = bid >> 3;
    mt = (local / n_tiles) * 8 + xcd;
    nt = local % n_tiles;
  }
  const int m0 = mt * BM, n0 = nt * BN;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wm = w & 1, wn = w >> 1;  // wave covers A rows m0 + 128wm .., B rows n0 + 32 NW wn ..
  const int k_steps = g.K / BK;

  // per-lane source rows and LDS positions of the copies (fixed over K)
  // instruction k of wave w fills tile chunks [(w*L + k)*64, +64): 8 rows x 8 chunks
  const bf16* a_src[A_LOADS];
  const bf16* b_src[B_LOADS];
#pragma unroll
  for (int k = 0; k < A_LOADS; ++k) {
    const int pos = (w * A_LOADS + k) * 64 + lane, r = pos >> 3, cp = pos & 7;
    a_src[k] = a_row_ptr(g, m0 + r) + 8 * (cp ^ g_swz(r));
  }
#pragma unroll
  for (int k = 0; k < B_LOADS; ++k) {
    const int pos = (w * B_LOADS + k) * 64 + lane, r = pos >> 3, cp = pos & 7;
    b_src[k] = b_row_ptr(g, n0 + r) + 8 * (cp ^ g_swz(r));
  }
  const uint32_t lds_base = (uint32_t)(size_t)(LDS_AS char*)lds;
  // copy q (of LOADS) of this wave for K step ks (A copies first)
  auto load_one = [&](int ks, int q) __attribute__((always_inline)) {
    const uint32_t st = lds_base + (ks % N_STAGES) * STAGE;
    const int kofs = ks * BK;
    if (q < A_LOADS)
      g_dma16(a_src[q] + kofs, __builtin_amdgcn_readfirstlane(st + (w * A_LOADS + q) * 1024));
    else
      g_dma16(b_src[q - A_LOADS] + kofs,
              __builtin_amdgcn_readfirstlane(st + A_STAGE + (w * B_LOADS + q - A_LOADS) * 1024));
  };
  for (int v = 0; v < N_STAGES - 1 && v < k_steps; ++v)
#pragma unroll
    for (int q = 0; q < LOADS; ++q) load_one(v, q);

  // operand read offsets inside a stage: MFMA A side = B rows (n), B side = A rows (m)
  //   step s (16 of K) reads chunk 2s + g of its row
  const int hl = lane & 31, gq = lane >> 5;
  int an_off[NW][4], bm_off[4][4];  // [tile][k-step within BK]
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int r = 32 * NW * wn + 32 * i + hl;
#pragma unroll
    for (int s = 0; s < 4; ++s) an_off[i][s] = A_STAGE + r * 128 + (((2 * s + gq) ^ g_swz(r)) << 4);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 128 * wm + 32 * j + hl;
#pragma unroll
    for (int s = 0; s < 4; ++s) bm_off[j][s] = r * 128 + (((2 * s + gq) ^ g_swz(r)) << 4);
  }

  f32x16 acc[NW][4];  // [n tile][m tile]
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){};

  // Per K step: wait for its stage and publish it with a barrier (which also
  // frees the stage read in the previous step), then issue the copies of step
  // ks + N_STAGES - 1 a quarter at a time before each 16-wide sub-step, so the
  // texture unit drains them behind the MFMAs. Operand fragments are read one
  // sub-step ahead into a second register set.
  bf16x8_t fa[2][NW], fb[2][4];
  for (int ks = 0; ks < k_steps; ++ks) {
    if (N_STAGES == 3 && ks + 1 < k_steps) g_wait_vmcnt<(N_STAGES == 3 ? LOADS : 0)>();
    else g_wait_vmcnt<0>();
    g_lds_barrier();
    const int next = ks + N_STAGES - 1;
    const LDS_AS char* st = (const LDS_AS char*)(lds + (ks % N_STAGES) * STAGE);
    auto read_frags = [&](int sub, int set) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NW; ++i) fa[set][i] = g_as_bf16x8(*(const LDS_AS u32x4*)(st + an_off[i][sub]));
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[set][j] = g_as_bf16x8(*(const LDS_AS u32x4*)(st + bm_off[j][sub]));
    };
    read_frags(0, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) read_frags(s + 1, (s + 1) & 1);
      if (next < k_steps)
#pragma unroll
        for (int q = s * LOADS / 4; q < (s + 1) * LOADS / 4; ++q) load_one(next, q);
#pragma unroll
      for (int i = 0; i < NW; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = EPI == 2 ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[s & 1][j], fa[s & 1][i], acc[i][j], 0, 0, 0)
                               : __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s & 1][i], fb[s & 1][j], acc[i][j], 0, 0, 0);
    }
  }

  // Plain, head-major and blocked-transposed stores go through LDS: the tile
  // is staged (as C for EPI 0/3, as C^T for EPI 2) and then written as whole
  // 16-byte pieces of consecutive output bytes, instead of each store
  // instruction touching 32 rows. The stores are non-temporal: the outputs
  // (up to 805 MB for the query up-projection) would otherwise stream through
  // the 256 MB last-level cache and push out the operands that every round
  // of blocks reads again.
  if constexpr (EPI != 1) {
    const bool aligned16 = g.N % 8 == 0 && g.c_split % 8 == 0 && g.ldc0 % 8 == 0 && g.ldc1 % 8 == 0 &&
                           ((size_t)g.c0 & 15) == 0 && ((size_t)g.c1 & 15) == 0;
    if (EPI >= 2 || aligned16) {
      g_lds_barrier();  // every wave is done with the stages
      LDS_AS bf16* ct = (LDS_AS bf16*)lds;
      typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
      typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
#pragma unroll
      for (int i = 0; i < NW; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const bf16x4_t o = {(__bf16)acc[i][j][4 * q], (__bf16)acc[i][j][4 * q + 1], (__bf16)acc[i][j][4 * q + 2],
                                (__bf16)acc[i][j][4 * q + 3]};
            // EPI 2 holds C^T[n][m .. m+3]: staged as rows n; others C[m][n .. n+3]: rows m
            const int row = EPI == 2 ? 32 * NW * wn + 32 * i + hl : 128 * wm + 32 * j + hl;
            const int col = EPI == 2 ? 128 * wm + 32 * j + 8 * q + 4 * gq : 32 * NW * wn + 32 * i + 8 * q + 4 * gq;
            *(LDS_AS u32x2_t*)(ct + row * CT_PITCH + col) = __builtin_bit_cast(u32x2_t, o);
          }
      g_lds_barrier();
      const int n_heads = g.N / HEAD_W;
      if constexpr (EPI == 2) {
        // rows n (BN of them) x 256 columns m, in 16-byte pieces of 8 m
        for (int idx = threadIdx.x; idx < BN * (BM / 8); idx += G_THREADS) {
          const int r = idx / (BM / 8), ch = idx % (BM / 8);
          const int n = n0 + r, m = m0 + 8 * ch;
          if (n >= g.N || m >= g.M) continue;
          const int b = m / g.a_seq, t = m - b * g.a_seq;
          bf16* dst = g.c0 + ((((size_t)b * n_heads + n / HEAD_W) * (g.a_seq / 64) + t / 64) * HEAD_W + n % HEAD_W) * 64 +
                      t % 64;
          __builtin_nontemporal_store(*(const LDS_AS u32x4*)(ct + r * CT_PITCH + 8 * ch), (u32x4*)dst);
        }
      } else {
        // rows m (256 of them) x BN columns n, in 16-byte pieces of 8 n
        for (int idx = threadIdx.x; idx < BM * (BN / 8); idx += G_THREADS) {
          const int r = idx / (BN / 8), ch = idx % (BN / 8);
          const int m = m0 + r, n = n0 + 8 * ch;
          if (m >= g.M || n >= g.N) continue;
          const u32x4 v = *(const LDS_AS u32x4*)(ct + r * CT_PITCH + 8 * ch);
          if constexpr (EPI == 3) {
            const int b = m / g.a_seq, t = m - b * g.a_seq;
            __builtin_nontemporal_store(v, (u32x4*)(g.c0 + (((size_t)b * n_heads + n / HEAD_W) * g.a_seq + t) * HEAD_W + n % HEAD_W));
          } else {
            if (n < g.c_split) __builtin_nontemporal_store(v, (u32x4*)(g.c0 + (size_t)m * g.ldc0 + n));
            else __builtin_nontemporal_store(v, (u32x4*)(g.c1 + (size_t)m * g.ldc1 + (n - g.c_split)));
          }
        }
      }
      return;
    }
  }
  // rows m = (sequence, token): a_seq is a multiple of 64 for the per-head
  // epilogues, so each aligned group of 64 rows belongs to one sequence
  int seq_of[2] = {0, 0};
  if constexpr (EPI >= 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) seq_of[u] = (m0 + 128 * wm + 64 * u) / g.a_seq;
  }
  const int n_heads = g.N / HEAD_W;
  if constexpr (EPI == 2) {
    // lane holds C[m .. m+3][n] for n = n0 + 32 NW wn + 32i + hl,
    // m = m0 + 128wm + 32j + 8q + 4gq (q = r / 4)
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int n = n0 + 32 * NW * wn + 32 * i + hl;
      if (n >= g.N) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int b = seq_of[j >> 1];
        const int t_base = m0 + 128 * wm + 32 * j - b * g.a_seq;
        bf16* dst = g.c0 + ((((size_t)b * n_heads + n / HEAD_W) * (g.a_seq / 64) + t_base / 64) * HEAD_W +
                            n % HEAD_W) * 64 + t_base % 64;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = m0 + 128 * wm + 32 * j + 8 * q + 4 * gq;
          if (m >= g.M) continue;
          typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
          const bf16x4_t o = {(__bf16)acc[i][j][4 * q], (__bf16)acc[i][j][4 * q + 1], (__bf16)acc[i][j][4 * q + 2],
                              (__bf16)acc[i][j][4 * q + 3]};
          *(bf16x4_t*)(dst + 8 * q + 4 * gq) = o;
        }
      }
    }
    return;
  }
  // epilogue: lane holds C[m][n .. n+3] for m = m0 + 128wm + 32j + hl,
  // n = n0 + 32 NW wn + 32i + 8q + 4gq (q = r / 4)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + 128 * wm + 32 * j + hl;
    if (m >= g.M) continue;
    bf16* crow;
    int pos = 0;
    if (EPI == 1) {
      crow = g.c0 + (size_t)(g.slots ? g.slots[m] : m) * g.ldc0;
      pos = g.positions[m];
    }
    const int seq_b = seq_of[j >> 1], seq_t = m - seq_b * g.a_seq;
#pragma unroll
    for (int i = 0; i < NW; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + 32 * NW * wn + 32 * i + 8 * q + 4 * gq;
        if (n >= g.N) continue;
        float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
        if (EPI == 1) {
          if (n >= g.d_c) {  // d_c is a multiple of 8: all four columns are RoPE columns
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
              const int pr = (n + e - g.d_c) >> 1;
              const double ang = (double)pos * pow((double)g.rope_base, -2.0 * pr / (double)g.d_rope);
              const float r = (float)(ang - 6.283185307179586 * rint(ang * 0.15915494309189535));
              float sn, cs;
              sincosf(r, &sn, &cs);
              const float x0 = v[e], x1 = v[e + 1];
              v[e] = x0 * cs - x1 * sn;
              v[e + 1] = x0 * sn + x1 * cs;
            }
          }
          const bf16x4_t o = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
          *(bf16x4_t*)(crow + n) = o;
        } else if (EPI == 3) {
          const bf16x4_t o = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
          *(bf16x4_t*)(g.c0 + (((size_t)seq_b * n_heads + n / HEAD_W) * g.a_seq + seq_t) * HEAD_W + n % HEAD_W) = o;
        } else {
          const bf16x4_t o = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
          if (n < g.c_split) *(bf16x4_t*)(g.c0 + (size_t)m * g.ldc0 + n) = o;
          else *(bf16x4_t*)(g.c1 + (size_t)m * g.ldc1 + (n - g.c_split)) = o;
        }
      }
  }
}

}  // namespace

bool gemm_fast_supported(int M, int N, int K) { return M > 0 && N > 0 && N % 4 == 0 && K > 0 && K % BK == 0; }

hipError_t gemm_fast(const GemmArgs& g, int epi, hipStream_t s) {
  if (epi >= 2 && (g.N % HEAD_W != 0 || g.a_seq % 64 != 0 || g.a_seq < 64)) return hipErrorInvalidValue;
  const int m_tiles = (g.M + BM - 1) / BM;
  // 256-wide tiles where there are enough of them to fill the chip several
  // times over (and no partial tile); 128-wide otherwise
  const bool wide = epi != 1 && g.N % 256 == 0 && m_tiles * (g.N / 256) >= 1024;
  // The latent projection (N = d_c + d_rope, 576 for the DeepSeek-V3 shape)
  // has few column tiles, so the last round of blocks can be mostly empty:
  // 64 row tiles x 5 tiles of 128 columns are 320 blocks, two rounds on 256
  // CUs with the second a quarter full. Where N is a whole number of
  // 192-column tiles and those take less time by rounds x tile width (64 x 3
  // = 192 blocks: one round of 1.5x the work), the 256 x 192 tile is used.
  bool w192 = false;
  if (epi == 1 && g.N % 192 == 0) {
    const int cus = device_cus();
    const long r128 = ((long)m_tiles * ((g.N + 127) / 128) + cus - 1) / cus;
    const long r192 = ((long)m_tiles * (g.N / 192) + cus - 1) / cus;
    w192 = r192 * 192 < r128 * 128;
  }
  const int grid = m_tiles * (wide ? g.N / 256 : w192 ? g.N / 192 : (g.N + 127) / 128);
  auto go = [&](auto kern, int waves) { hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * waves), 0, s, g); };
  // The K/V up-projections (K = 512: eight K steps, then a 128 KB output
  // tile) run 8 waves, two per SIMD, which measured 7 % faster there; the
  // long-K query up-projection stays at 4 waves, where 8 measured 3 % slower.
  if (wide) {
    if (epi == 2) go(k_gemm<2, 4, 8>, 8);
    else if (epi == 3) go(k_gemm<3, 4, 8>, 8);
    else go(k_gemm<0, 4, 4>, 4);
  } else {
    if (epi == 1 && w192) go(k_gemm<1, 3, 4>, 4);
    else if (epi == 1) go(k_gemm<1, 2, 4>, 4);
    else if (epi == 2) go(k_gemm<2, 2, 4>, 4);
    else if (epi == 3) go(k_gemm<3, 2, 4>, 4);
    else go(k_gemm<0, 2, 4>, 4);
  }
  return hipGetLastError();
}

bool project_fast_supported(const mla_dims& d, int d_model, int d_q) {
  // The epilogues store 4 (register path) or 8 (staged path) consecutive
  // columns at once. The latent GEMM's column groups stay inside c_KV or k_pe
  // when d_c % 8 == 0 (checked with the dims) and d_rope % 4 == 0; the query
  // GEMM's groups must not straddle the q_nope / q_pe split or a row end, so
  // both widths are multiples of 8.
  const int n_latent = d.d_c + d.d_rope;
  const bool latent_ok = d.d_rope % 4 == 0 && gemm_fast_supported(1, n_latent, d_model);
  const bool query_ok = d_q == 0 || (gemm_fast_supported(1, d_q, d_model) && d_q % BK == 0 &&
                                     (d.n_heads * d.d_nope) % 8 == 0 && (d.n_heads * d.d_rope) % 8 == 0);
  return d.dtype == MLA_BF16 && latent_ok && query_ok;
}

// Latent rows (RoPE + scatter epilogue), then the optional query path: c_Q in
// bf16 in the workspace, then [q_nope | q_pe] = c_Q [W_UQ; W_QR]^T split by column.
hipError_t project_fast(const mla_dims& d, int n_tokens, int d_model, const void* h, const void* w_dkv,
                        const void* w_kr, const int32_t* positions, const int32_t* slots, void* rows,
                        const mla_qproj* qp, void* ws, hipStream_t s) {
  GemmArgs g{};
  g.M = n_tokens;
  g.N = d.d_c + d.d_rope;
  g.K = d_model;
  g.a = (const bf16*)h;
  g.lda = d_model;
  g.b0 = (const bf16*)w_dkv;
  g.b1 = (const bf16*)w_kr;
  g.n_split = d.d_c;
  g.ldb = d_model;
  g.c0 = g.c1 = (bf16*)rows;
  g.ldc0 = g.ldc1 = d.d_c + d.d_rope;
  g.c_split = g.N;
  g.slots = slots;
  g.positions = positions;
  g.d_c = d.d_c;
  g.d_rope = d.d_rope;
  g.rope_base = d.rope_base;
  hipError_t e;
  {
    ProfScope ps("mla_project_latent", s);
    e = gemm_fast(g, 1, s);
  }
  if (e != hipSuccess || !qp) return e;
  bf16* cq = (bf16*)ws;
  GemmArgs q{};
  q.M = n_tokens;
  q.N = qp->d_q;
  q.K = d_model;
  q.a = (const bf16*)h;
  q.lda = d_model;
  q.b0 = q.b1 = (const bf16*)qp->w_dq;
  q.n_split = q.N;
  q.ldb = d_model;
  q.c0 = q.c1 = cq;
  q.ldc0 = q.ldc1 = qp->d_q;
  q.c_split = q.N;
  {
    ProfScope ps("mla_project_q_down", s);
    e = gemm_fast(q, 0, s);
  }
  if (e != hipSuccess) return e;
  const int hn = d.n_heads * d.d_nope, hr = d.n_heads * d.d_rope;
  GemmArgs u{};
  u.M = n_tokens;
  u.N = hn + hr;
  u.K = qp->d_q;
  u.a = cq;
  u.lda = qp->d_q;
  u.b0 = (const bf16*)qp->w_uq;
  u.b1 = (const bf16*)qp->w_qr;
  u.n_split = hn;
  u.ldb = qp->d_q;
  u.c0 = (bf16*)qp->q_nope;
  u.c1 = (bf16*)qp->q_pe;
  u.ldc0 = hn;
  u.ldc1 = hr;
  u.c_split = hn;
  {
    ProfScope ps("mla_project_q_up", s);
    e = gemm_fast(u, 0, s);
  }
  return e;
}

}  // namespace mla
