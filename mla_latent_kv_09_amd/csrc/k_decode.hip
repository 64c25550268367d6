// MFMA decode path for the DeepSeek-V3 latent shape (bf16, d_c 512,
// d_rope 64, d_nope = d_v = 128, 64-token pages, up to 128 heads).
//
// Three kernels, one stream:
//   k_absorb       Qt[b,h] = s*log2(e) * [W_UK,h^T q_nope[b,h] || RoPE(q_pe[b,h], L_b - 1)]
//                  ("DeepSeek-V2 paper digest" §2.2: W_UK folded into the query;
//                  §2.3: only the decoupled slice is rotated).
//   k_split        one workgroup per (sequence, run of pages): every page of
//                  64 cache rows (64 x 576 bf16 = 72 KB, contiguous in HBM) is
//                  streamed into LDS once and shared by all heads. Scores
//                  S^T[t,h] = row_t . Qt[h] are one 64 x H x 576 MFMA product per
//                  page (every head reads the same row), the online softmax
//                  keeps (max, sum) per head, and the latent output
//                  O^T[c,h] += sum_t row_t[c] P[t,h] is a 512 x H x 64 MFMA product
//                  reading the first 512 columns of the same LDS tile.
//   k_combine_uv   merges the page runs of a sequence (log-sum-exp weights)
//                  and applies W_UV,h to the latent output, batched over the
//                  sequences so each head's W_UV is read once.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int DC = 512, DR = 64, ROW = DC + DR, DN = 128, DV = 128;
constexpr int PAGE = 64;
constexpr int ROW_BYTES = ROW * 2;               // 1152
constexpr int ROW_CHUNKS = ROW_BYTES / 16;       // 72 chunks of 16 B
constexpr int PAGE_BYTES = PAGE * ROW_BYTES;     // 73728
constexpr int PAGE_CHUNKS = PAGE * ROW_CHUNKS;   // 4608
constexpr int SPLIT_THREADS = 256;               // 4 waves
constexpr int LOADS_PER_THREAD = PAGE_CHUNKS / SPLIT_THREADS;  // 18
constexpr float LOG2E = 1.4426950408889634f;
constexpr int MAX_SPLITS = 256;
constexpr int MAX_HEADS = 128;

// Chunk position swizzle inside a cache row held in LDS. Row t's 16-byte chunk
// j sits at chunk j ^ swz(t) (the XOR only moves chunks inside aligned groups of
// 8). With 64 banks of 4 bytes, 16 consecutive rows reading the same chunk
// (score operand) and 4 aligned rows reading 4 neighbouring chunks (transposed
// value operand) then hit distinct banks.
__device__ __forceinline__ int swz(int t) {
  const int k = (t >> 1) & 7;
  return ((k & 1) << 2) | (k >> 1);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ bf16x8_t cat_tr(short4_t a, short4_t b) {
  typedef __attribute__((ext_vector_type(8))) short short8_t;
  short8_t s = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8_t, s);
}

__device__ __forceinline__ short4_t tr_read(const LDS_AS char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS short4_t*)p);
}

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0); }

// x *= a for an MFMA accumulator that lives in an AGPR. Written out so the
// compiler keeps the 256 output accumulators in AGPRs across the page loop
// (a plain multiply makes it shuttle them through VGPRs and spill). The
// leading s_nops (21 wait states) cover an MFMA that may still be writing the
// register, the trailing one a following MFMA that reads it as its C operand.
__device__ __forceinline__ void scale_acc(float& x, float a) {
  float t;
  asm volatile(
      "s_nop 7\n\ts_nop 7\n\ts_nop 4\n\t"
      "v_accvgpr_read_b32 %1, %0\n\t"
      "v_mul_f32 %1, %1, %2\n\t"
      "v_accvgpr_write_b32 %0, %1\n\t"
      "s_nop 4"
      : "+a"(x), "=&v"(t)
      : "v"(a));
}

struct Plan {
  int pages_per_split;
  int splits;
};

Plan plan_splits(int batch, int max_context) {
  const int max_pages = (max_context + PAGE - 1) / PAGE;
  // aim for one workgroup per compute unit across the batch, 4..32 pages each
  int pps = (int)(((int64_t)batch * max_pages + 255) / 256);
  pps = pps < 4 ? 4 : (pps > 32 ? 32 : pps);
  const int min_pps = (max_pages + MAX_SPLITS - 1) / MAX_SPLITS;
  if (pps < min_pps) pps = min_pps;
  Plan p;
  p.pages_per_split = pps;
  p.splits = (max_pages + pps - 1) / pps;
  return p;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t qt, part_o, part_ml, total;
};

WsLayout ws_layout(int H, int batch, int splits) {
  WsLayout l;
  l.qt = 0;
  l.part_o = align256((size_t)batch * H * ROW * 2);
  l.part_ml = l.part_o + align256((size_t)H * batch * splits * DC * 4);
  l.total = l.part_ml + align256((size_t)H * batch * splits * 2 * 4);
  return l;
}

// ------------------------------------------------------------ k_absorb ----
// grid (H, DC / 64); 4 waves. Block (h, c0): Qt[:, h, c0 .. c0+63] for every
// sequence, as a [B x 128] x [128 x 64] MFMA product with W_UK,h staged in LDS
// and read transposed; block (h, 0) also writes the rotated q_pe slice.
__global__ __launch_bounds__(256) void k_absorb(int B, int H, const bf16* __restrict__ q_nope,
                                                const bf16* __restrict__ q_pe, const bf16* __restrict__ w_uk,
                                                const int32_t* __restrict__ ctx_lens, float qscale, float base,
                                                bf16* __restrict__ qt) {
  constexpr int LD = 72;  // padded row (144 B) keeps the transposed reads conflict-free
  __shared__ __attribute__((aligned(16))) bf16 wt[DN * LD];
  const int h = blockIdx.x, c0 = blockIdx.y * 64;
  for (int i = threadIdx.x; i < DN * 8; i += 256) {
    const int j = i >> 3, ch = i & 7;
    *(u32x4*)&wt[j * LD + ch * 8] = *(const u32x4*)(w_uk + (size_t)(h * DN + j) * DC + c0 + ch * 8);
  }
  __syncthreads();
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, i16 = lane & 15, G = lane >> 4;
  const LDS_AS char* wbase = (const LDS_AS char*)wt;
  for (int mt = w; mt * 16 < B; mt += 4) {
    f32x4 acc[4] = {};
    const int brow = mt * 16 + i16;
#pragma unroll
    for (int ks = 0; ks < DN / 32; ++ks) {
      u32x4 av = {0, 0, 0, 0};
      if (brow < B) av = *(const u32x4*)(q_nope + ((size_t)brow * H + h) * DN + 32 * ks + 8 * G);
      const bf16x8_t a = as_bf16x8(av);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int k0 = 32 * ks + 8 * G, col = 16 * nt + 4 * (i16 & 3);
        const short4_t r1 = tr_read(wbase + ((k0 + (i16 >> 2)) * LD + col) * 2);
        const short4_t r2 = tr_read(wbase + ((k0 + 4 + (i16 >> 2)) * LD + col) * 2);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, cat_tr(r1, r2), acc[nt], 0, 0, 0);
      }
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int b = mt * 16 + 4 * G + r;
        if (b < B) qt[((size_t)b * H + h) * ROW + c0 + 16 * nt + i16] = f2bf(acc[nt][r] * qscale);
      }
  }
  if (blockIdx.y == 0) {
    for (int idx = threadIdx.x; idx < B * (DR / 2); idx += 256) {
      const int b = idx / (DR / 2), i = idx % (DR / 2);
      const int pos = ctx_lens[b] - 1;
      double sn, cs;
      sincos(rope_angle(pos, i, DR, base), &sn, &cs);
      const bf16* src = q_pe + ((size_t)b * H + h) * DR + 2 * i;
      const float x0 = bf2f(src[0]), x1 = bf2f(src[1]);
      bf16* dst = qt + ((size_t)b * H + h) * ROW + DC + 2 * i;
      dst[0] = f2bf((x0 * (float)cs - x1 * (float)sn) * qscale);
      dst[1] = f2bf((x0 * (float)sn + x1 * (float)cs) * qscale);
    }
  }
}

// ------------------------------------------------------------- k_split ----
// grid (splits, B); 256 threads. Wave w owns heads 32w .. 32w+31 (lanes of
// heads >= H compute on a copy of head H-1 and store nothing); every wave
// streams a quarter of each page. Partials per (head, sequence, split):
// O (512 fp32, unnormalised, relative to max m) and (m, l), log2 domain.
//
// Registers per lane: the latent part of the query (32 steps x 4 = 128) and
// the output accumulators (16 tiles x 16 = 256) stay resident; the query's
// 64-wide RoPE slice lives in LDS (16 KB next to the two 72 KB page buffers)
// and the softmax runs per 32-token half page, so scores and probabilities
// take 16 + 8 registers.
constexpr int QR_BYTES = MAX_HEADS * DR * 2;  // 16 KB
constexpr int LAT_STEPS = DC / 16;            // 32 MFMA steps over the latent columns
constexpr int ROPE_STEPS = DR / 16;           // 4 steps over the RoPE columns

__global__ __launch_bounds__(SPLIT_THREADS, 1) void k_split(int H, int B, int splits, int pps,
                                                            const bf16* __restrict__ qt,
                                                            const bf16* __restrict__ rows,
                                                            const int32_t* __restrict__ block_table,
                                                            int max_blocks, const int32_t* __restrict__ ctx_lens,
                                                            float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ __attribute__((aligned(1024))) char lds[2 * PAGE_BYTES + QR_BYTES];
  const int split = blockIdx.x, b = blockIdx.y;
  const int L = ctx_lens[b];
  const int n_pages = (L + PAGE - 1) / PAGE;
  const int p0 = split * pps;
  const int p1 = min(p0 + pps, n_pages);
  if (p0 >= n_pages) return;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hl = lane & 31, g = lane >> 5;
  const int h = w * 32 + hl;
  const int32_t* table = block_table + (size_t)b * max_blocks;
  char* const qr = lds + 2 * PAGE_BYTES;

  // Streams page p into buffer buf: 18 direct-to-LDS 16-byte loads per lane.
  // Instruction k of wave w fills LDS chunks [(w*18+k)*64, +64) in order; the
  // lane picks the global chunk that belongs at its (swizzled) position.
  auto load_page = [&](int p, int buf) {
    const char* src = (const char*)(rows + (size_t)table[p] * PAGE * ROW);
#pragma unroll
    for (int k = 0; k < LOADS_PER_THREAD; ++k) {
      const int base = (w * LOADS_PER_THREAD + k) * 64;
      const int pos = base + lane;
      const int t = pos / ROW_CHUNKS, jp = pos - t * ROW_CHUNKS;
      const uint32_t off = (uint32_t)(t * ROW_BYTES + ((jp ^ swz(t)) << 4));
      __builtin_amdgcn_global_load_lds((const void*)(src + off), (LDS_AS void*)(lds + buf * PAGE_BYTES + base * 16),
                                       16, 0, 0);
    }
  };

  load_page(p0, 0);

  // RoPE slice of the query for every head of the block, in LDS: head h's
  // 16-byte chunk c (of 8) at h*128 + ((c ^ ((h >> 1) & 7)) * 16).
  for (int i = threadIdx.x; i < MAX_HEADS * (DR / 8); i += SPLIT_THREADS) {
    const int hh = i >> 3, c = i & 7;
    u32x4 v = {0, 0, 0, 0};
    if (hh < H) v = *(const u32x4*)(qt + ((size_t)b * H + hh) * ROW + DC + 8 * c);
    *(u32x4*)(qr + hh * 128 + ((c ^ ((hh >> 1) & 7)) << 4)) = v;
  }
  // latent part of this lane's query: Qt[b, h, 16s + 8g .. +7], s < 32
  // (lanes of heads >= H read head H-1; their columns are never stored)
  bf16x8_t qf[LAT_STEPS];
  {
    const bf16* q = qt + ((size_t)b * H + min(h, H - 1)) * ROW + 8 * g;
#pragma unroll
    for (int s = 0; s < LAT_STEPS; ++s) qf[s] = as_bf16x8(*(const u32x4*)(q + 16 * s));
  }
  f32x16 o[DC / 32];
#pragma unroll
  for (int i = 0; i < DC / 32; ++i) o[i] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;

  // LDS byte offsets of this lane's operand reads, split into a lane part
  // (below) and a compile-time part, so each read is one ds_read with an
  // immediate offset. The swizzle only permutes the low three chunk bits and
  // depends on row bits 1..3, so it folds into the lane part.
  //  score operand (step s, tile mt): row 32mt + hl, chunk (2s + g) ^ swz(hl)
  //    = qk_off[s % 4] + 32*mt*ROW_BYTES + (s / 4) * 128
  //  value operand (column tile ct, step j, half a/b): rows 16j + 4g + i16/4
  //    (+8 for b), columns 32ct + 16(G%2) + 4(i16%4) .. +3
  //    = pv_off[ct % 2][a/b] + 16*j*ROW_BYTES + (ct / 2) * 128
  //  RoPE query operand (step r): head h, chunk 2r + g
  const int i16 = lane & 15, G = lane >> 4;
  int qk_off[4], pv_off[2][2], qr_off[ROPE_STEPS];
  {
    const int x = swz(hl);
#pragma unroll
    for (int u = 0; u < 4; ++u) qk_off[u] = hl * ROW_BYTES + (((2 * u + g) ^ x) << 4);
    const int ra = 4 * g + (i16 >> 2), rb = ra + 8;
    const int y0 = 2 * (G & 1) + ((i16 & 3) >> 1), sub = 8 * (i16 & 1);
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      pv_off[par][0] = ra * ROW_BYTES + (((4 * par + y0) ^ swz(ra)) << 4) + sub;
      pv_off[par][1] = rb * ROW_BYTES + (((4 * par + y0) ^ swz(rb)) << 4) + sub;
    }
    const int hq = min(h, MAX_HEADS - 1);
#pragma unroll
    for (int r = 0; r < ROPE_STEPS; ++r) qr_off[r] = hq * 128 + (((2 * r + g) ^ ((hq >> 1) & 7)) << 4);
  }

  for (int p = p0; p < p1; ++p) {
    const int buf = (p - p0) & 1;
    wait_vmem_all();
    __syncthreads();
    if (p + 1 < p1) load_page(p + 1, buf ^ 1);
    const LDS_AS char* page = (const LDS_AS char*)(lds + buf * PAGE_BYTES);
    const LDS_AS char* qrl = (const LDS_AS char*)qr;
    const int valid = L - p * PAGE;

#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      // scores S^T[t, h] of the 32 rows 32mt .. 32mt+31
      f32x16 sc = {};
#pragma unroll
      for (int s = 0; s < ROW / 16; ++s) {
        const u32x4 a =
            *(const LDS_AS u32x4*)(page + qk_off[s & 3] + (32 * mt * ROW_BYTES + (s >> 2) * 128));
        const bf16x8_t bq = s < LAT_STEPS ? qf[s < LAT_STEPS ? s : 0]
                                          : as_bf16x8(*(const LDS_AS u32x4*)(qrl + qr_off[(s - LAT_STEPS) & 3]));
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), bq, sc, 0, 0, 0);
        if ((s & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
      // mask rows past the context (last page only)
      if (valid < PAGE) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = 32 * mt + 8 * (r >> 2) + 4 * g + (r & 3);
          if (t >= valid) sc[r] = -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // Lazy rescaling: the reference max only moves when the tile max exceeds
      // it by more than 8 (so p <= 2^8), so most tiles skip the rescale. A
      // fully masked tile has mx = -inf and never moves it.
      // A lane's first tile only sets the reference (its O and l are still 0).
      float alpha = 1.f;
      if (mx > m_run + 8.f) {
        if (m_run != -INFINITY) alpha = exp2f(m_run - mx);
        m_run = mx;
      }
      if (__ballot(alpha != 1.f)) {
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < DC / 32; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x = o[i][r];
            scale_acc(x, alpha);
            o[i][r] = x;
          }
      }
      // probabilities as the PV operand: step jj covers rows 32mt + 16jj .. +15
      bf16x8_t pf[2];
      float lsum = 0.f;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = exp2f(sc[8 * jj + 2 * e] - m_run);
          const float x1 = exp2f(sc[8 * jj + 2 * e + 1] - m_run);
          lsum += x0 + x1;
          pk[e] = pack_bf16x2(x0, x1);
        }
        const u32x4 v = {pk[0], pk[1], pk[2], pk[3]};
        pf[jj] = as_bf16x8(v);
      }
      l_run += lsum;
      // O^T[c, h] += V^T[c, t] P[t, h]; V^T fragments by transposed LDS reads
      // (lane i of a 16-lane group receives 4 consecutive rows of column n0 + i).
#pragma unroll
      for (int ct = 0; ct < DC / 32; ++ct) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int k = 16 * (2 * mt + jj) * ROW_BYTES + (ct >> 1) * 128;
          const short4_t r1 = tr_read(page + pv_off[ct & 1][0] + k);
          const short4_t r2 = tr_read(page + pv_off[ct & 1][1] + k);
          o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cat_tr(r1, r2), pf[jj], o[ct], 0, 0, 0);
        }
        if (ct & 1) __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if (h >= H) return;
  l_run += __shfl_xor(l_run, 32, 64);
  const size_t prow = ((size_t)h * B + b) * splits + split;
  if (g == 0) {
    part_ml[prow * 2] = m_run;
    part_ml[prow * 2 + 1] = l_run;
  }
  float* po = part_o + prow * DC;
#pragma unroll
  for (int ct = 0; ct < DC / 32; ++ct)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 v = {o[ct][4 * q], o[ct][4 * q + 1], o[ct][4 * q + 2], o[ct][4 * q + 3]};
      *(f32x4*)(po + 32 * ct + 8 * q + 4 * g) = v;
    }
}

// -------------------------------------------------------- k_combine_uv ----
// One block per (head, tile of 16 sequences). Blocks of the same head share
// blockIdx % 8, i.e. the same XCD and L2, so W_UV,h is fetched from HBM once.
__global__ __launch_bounds__(256) void k_combine_uv(int H, int B, int splits, int pps,
                                                    const int32_t* __restrict__ ctx_lens,
                                                    const float* __restrict__ part_o,
                                                    const float* __restrict__ part_ml,
                                                    const bf16* __restrict__ w_uv, bf16* __restrict__ out) {
  constexpr int LDO = DC + 8;
  __shared__ __attribute__((aligned(16))) bf16 oc[16 * LDO];
  __shared__ float wgt[16][MAX_SPLITS];
  __shared__ float inv_l[16];
  const int nbt = (B + 15) / 16;
  const int bid = blockIdx.x, xcd = bid & 7, k = bid >> 3;
  const int bt = k % nbt, h = (k / nbt) * 8 + xcd;
  if (h >= H) return;
  const int b0 = bt * 16;
  const int tid = threadIdx.x;
  if (tid < 16) {
    const int b = b0 + tid;
    if (b < B) {
      const int n_pages = (ctx_lens[b] + PAGE - 1) / PAGE;
      const int ns = (n_pages + pps - 1) / pps;
      const float* ml = part_ml + ((size_t)h * B + b) * splits * 2;
      float M = -INFINITY;
      for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[2 * s]);
      float l = 0.f;
      for (int s = 0; s < splits; ++s) {
        const float e = s < ns ? exp2f(ml[2 * s] - M) : 0.f;
        wgt[tid][s] = e;
        if (s < ns) l += e * ml[2 * s + 1];
      }
      inv_l[tid] = 1.f / l;
    } else {
      for (int s = 0; s < splits; ++s) wgt[tid][s] = 0.f;
      inv_l[tid] = 0.f;
    }
  }
  __syncthreads();
  // latent output o_c of the 16 sequences, normalised, as bf16 in LDS
  for (int idx = tid; idx < 16 * (DC / 4); idx += 256) {
    const int r = idx / (DC / 4), c4 = idx % (DC / 4);
    const int b = b0 + r;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (b < B) {
      const float* po = part_o + ((size_t)h * B + b) * splits * DC + 4 * c4;
      for (int s = 0; s < splits; ++s) {
        const float e = wgt[r][s];
        if (e != 0.f) {
          const f32x4 v = *(const f32x4*)(po + (size_t)s * DC);
          acc += e * v;
        }
      }
      acc *= inv_l[r];
    }
    uint32_t* d = (uint32_t*)&oc[r * LDO + 4 * c4];
    d[0] = pack_bf16x2(acc[0], acc[1]);
    d[1] = pack_bf16x2(acc[2], acc[3]);
  }
  __syncthreads();
  // out[b, h, v] = sum_c o_c[b, c] W_UV[h*128 + v, c]; wave w: v in 32w .. 32w+31
  const int w = tid >> 6, lane = tid & 63, i16 = lane & 15, G = lane >> 4;
  f32x4 acc[2] = {};
  const bf16* wv = w_uv + (size_t)h * DV * DC;
#pragma unroll 4
  for (int ks = 0; ks < DC / 32; ++ks) {
    const bf16x8_t a = as_bf16x8(*(const u32x4*)&oc[i16 * LDO + 32 * ks + 8 * G]);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int v = 32 * w + 16 * nt + i16;
      const bf16x8_t bv = as_bf16x8(*(const u32x4*)(wv + (size_t)v * DC + 32 * ks + 8 * G));
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv, acc[nt], 0, 0, 0);
    }
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int b = b0 + 4 * G + r;
      if (b < B) out[((size_t)b * H + h) * DV + 32 * w + 16 * nt + i16] = f2bf(acc[nt][r]);
    }
}

}  // namespace

bool decode_fast_supported(const mla_dims& d, const CacheView& c) {
  return d.dtype == MLA_BF16 && d.d_c == DC && d.d_rope == DR && d.d_nope == DN && d.d_v == DV &&
         d.n_heads <= MAX_HEADS && c.paged &&
         c.block_size == PAGE;
}

size_t decode_fast_workspace(const mla_dims& d, int batch, int max_context) {
  const Plan p = plan_splits(batch, max_context);
  return ws_layout(d.n_heads, batch, p.splits).total;
}

hipError_t decode_fast(const mla_dims& d, float scale, int batch, int max_context, const void* q_nope,
                       const void* q_pe, const void* w_uk, const void* w_uv, const CacheView& c, void* out,
                       void* ws, size_t ws_bytes, hipStream_t s) {
  const int H = d.n_heads;
  const Plan p = plan_splits(batch, max_context);
  const WsLayout l = ws_layout(H, batch, p.splits);
  if (ws_bytes < l.total) return hipErrorInvalidValue;
  char* base = (char*)ws;
  bf16* qt = (bf16*)(base + l.qt);
  float* part_o = (float*)(base + l.part_o);
  float* part_ml = (float*)(base + l.part_ml);

  {
    ProfScope ps("mla_decode_absorb", s);
    hipLaunchKernelGGL(k_absorb, dim3(H, DC / 64), dim3(256), 0, s, batch, H, (const bf16*)q_nope,
                       (const bf16*)q_pe, (const bf16*)w_uk, c.context_lens, scale * LOG2E, d.rope_base, qt);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(p.splits, batch);
  {
    ProfScope ps("mla_decode_split", s);
    hipLaunchKernelGGL(k_split, grid, dim3(SPLIT_THREADS), 0, s, H, batch, p.splits, p.pages_per_split, qt,
                       (const bf16*)c.rows, c.block_table, c.max_blocks, c.context_lens, part_o, part_ml);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int nbt = (batch + 15) / 16;
  const int hpad = (H + 7) / 8 * 8;
  {
    ProfScope ps("mla_decode_combine_uv", s);
    hipLaunchKernelGGL(k_combine_uv, dim3(hpad * nbt), dim3(256), 0, s, H, batch, p.splits,
                       p.pages_per_split, c.context_lens, part_o, part_ml, (const bf16*)w_uv, (bf16*)out);
  }
  return hipGetLastError();
}

}  // namespace mla
