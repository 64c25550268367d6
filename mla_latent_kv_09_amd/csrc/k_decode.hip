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
// grid (H, DC / 64); 4 waves. Block (h, c0) forms Qt[:, h, c0 .. c0+63] for
// every sequence as the transposed product Qt^T[c, b] = sum_j W_UK[h*128+j, c]
// q_nope[b, h, j]: the 128 x 64 slice of W_UK,h is staged in LDS and read
// transposed (as the A operand); each lane then holds 4 consecutive columns of
// one sequence and stores them with one 8-byte write. Block (h, 0) also writes
// the rotated, scaled q_pe slice.
__global__ __launch_bounds__(256) void k_absorb(int B, int H, const bf16* __restrict__ q_nope,
                                                const bf16* __restrict__ q_pe, const bf16* __restrict__ w_uk,
                                                const int32_t* __restrict__ ctx_lens, float qscale, float base,
                                                bf16* __restrict__ qt) {
  constexpr int LD = 72;  // padded row (144 B) keeps the transposed reads conflict-free
  constexpr int BT_CHUNK = 4;  // sequence tiles whose query loads are in flight together
  __shared__ __attribute__((aligned(16))) bf16 wt[DN * LD];
  const int h = blockIdx.x, c0 = blockIdx.y * 64;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, i16 = lane & 15, G = lane >> 4;
  // every independent load first: the W_UK slice and the first chunk of queries
  u32x4 wr[DN * 8 / 256];
#pragma unroll
  for (int u = 0; u < DN * 8 / 256; ++u) {
    const int i = threadIdx.x + 256 * u, j = i >> 3, ch = i & 7;
    wr[u] = *(const u32x4*)(w_uk + (size_t)(h * DN + j) * DC + c0 + ch * 8);
  }
  auto load_q = [&](int bt0, u32x4 (&qv)[BT_CHUNK][DN / 32]) {
#pragma unroll
    for (int t = 0; t < BT_CHUNK; ++t)
#pragma unroll
      for (int ks = 0; ks < DN / 32; ++ks) {
        const int b = (bt0 + t) * 16 + i16;
        qv[t][ks] = b < B ? *(const u32x4*)(q_nope + ((size_t)b * H + h) * DN + 32 * ks + 8 * G) : (u32x4){0, 0, 0, 0};
      }
  };
  u32x4 qv[BT_CHUNK][DN / 32];
  load_q(0, qv);
#pragma unroll
  for (int u = 0; u < DN * 8 / 256; ++u) {
    const int i = threadIdx.x + 256 * u, j = i >> 3, ch = i & 7;
    *(u32x4*)&wt[j * LD + ch * 8] = wr[u];
  }
  __syncthreads();
  const LDS_AS char* wbase = (const LDS_AS char*)wt;
  // A fragments of column tile w (columns c0 + 16w .. +15), all 4 K-steps
  bf16x8_t af[DN / 32];
#pragma unroll
  for (int ks = 0; ks < DN / 32; ++ks) {
    const int k0 = 32 * ks + 8 * G, col = 16 * w + 4 * (i16 & 3);
    af[ks] = cat_tr(tr_read(wbase + ((k0 + (i16 >> 2)) * LD + col) * 2),
                    tr_read(wbase + ((k0 + 4 + (i16 >> 2)) * LD + col) * 2));
  }
  for (int bt0 = 0; bt0 * 16 < B; bt0 += BT_CHUNK) {
    u32x4 cur[BT_CHUNK][DN / 32];
#pragma unroll
    for (int t = 0; t < BT_CHUNK; ++t)
#pragma unroll
      for (int ks = 0; ks < DN / 32; ++ks) cur[t][ks] = qv[t][ks];
    if ((bt0 + BT_CHUNK) * 16 < B) load_q(bt0 + BT_CHUNK, qv);
#pragma unroll
    for (int t = 0; t < BT_CHUNK; ++t) {
      const int b = (bt0 + t) * 16 + i16;
      f32x4 acc = {};
#pragma unroll
      for (int ks = 0; ks < DN / 32; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks], as_bf16x8(cur[t][ks]), acc, 0, 0, 0);
      if (b < B) {
        typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
        const bf16x4_t v = {(__bf16)(acc[0] * qscale), (__bf16)(acc[1] * qscale), (__bf16)(acc[2] * qscale),
                            (__bf16)(acc[3] * qscale)};
        *(bf16x4_t*)(qt + ((size_t)b * H + h) * ROW + c0 + 16 * w + 4 * G) = v;
      }
    }
  }
  if (blockIdx.y == 0) {
    // thread -> pair i = tid % 32 (fixed), sequences tid / 32, +8, ...
    const int i = threadIdx.x & (DR / 2 - 1);
    const double theta = pow((double)base, -2.0 * (double)i / (double)DR);
    for (int b = threadIdx.x / (DR / 2); b < B; b += 256 / (DR / 2)) {
      const double ang = (double)(ctx_lens[b] - 1) * theta;
      // reduce to [-pi, pi] in double, then single-precision sin/cos
      const float r = (float)(ang - 6.283185307179586 * rint(ang * 0.15915494309189535));
      float sn, cs;
      sincosf(r, &sn, &cs);
      const bf16* src = q_pe + ((size_t)b * H + h) * DR + 2 * i;
      const float x0 = bf2f(src[0]), x1 = bf2f(src[1]);
      typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
      const bf16x2_t v = {(__bf16)((x0 * cs - x1 * sn) * qscale), (__bf16)((x0 * sn + x1 * cs) * qscale)};
      *(bf16x2_t*)(qt + ((size_t)b * H + h) * ROW + DC + 2 * i) = v;
    }
  }
}

// ------------------------------------------------------------- k_split ----
// grid (splits, B); 256 threads (4 waves); one block per (sequence, run of
// pages). The run is walked in tiles of 32 cache rows (half a page, 36 KB).
//
// Work split inside the block, per tile:
//   scores    wave w owns heads 32w .. 32w+31: S^T[t, h] = row_t . Qt[h]
//             (36 MFMA steps of K = 16 over the 576 columns), then the online
//             softmax of those heads (running max m and sum l stay with the
//             owner). The probabilities P (bf16) and each head's rescale
//             factor go to LDS.
//   values    wave w owns latent columns 128w .. 128w+127 of every head:
//             O^T[c, h] += V^T[c, t] P[t, h] (4 column tiles x 4 head tiles x
//             2 steps). Each value fragment, read once from LDS, feeds four
//             MFMAs; so does each P fragment.
// Rows stream HBM -> LDS with direct 16-byte loads into a ring of three tile
// slots: while tile i is computed, tiles i+1 and i+2 are in flight.
//
// Partials per (head, sequence, split): O (512 fp32, unnormalised, relative to
// the head's reference max m) and (m, l), both in the log2 domain.
constexpr int TILE = 32;                                  // rows per tile
constexpr int TILE_BYTES = TILE * ROW_BYTES;              // 36864
constexpr int TILE_LOADS = TILE * ROW_CHUNKS / SPLIT_THREADS;  // 9 per lane
constexpr int N_SLOTS = 3;
constexpr int QR_BYTES = MAX_HEADS * DR * 2;              // 16 KB: RoPE slice of Qt
constexpr int PB_BYTES = MAX_HEADS * TILE * 2;            // 8 KB: P of one tile
constexpr int LAT_STEPS = DC / 16;                        // 32 score steps over c_KV
constexpr int ROPE_STEPS = DR / 16;                       // 4 score steps over k_pe
constexpr int SPLIT_LDS = N_SLOTS * TILE_BYTES + QR_BYTES + PB_BYTES + MAX_HEADS * 4;

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// One 16-byte HBM -> LDS load per lane: lane l's bytes land at LDS byte address
// lds_addr + 16 l (lds_addr is wave-uniform and goes through M0). Issued from
// asm so that the compiler does not treat every later LDS read as a possible
// alias of the copy and drain all loads first; the kernel orders these copies
// with explicit vmcnt waits before the barrier that publishes a tile. Nothing
// else in the kernel uses M0.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_addr)
               : "memory", "m0");
}

// Workgroup barrier for LDS traffic only. __syncthreads() also waits for all
// outstanding global loads (vmcnt 0), which would drain the tile prefetch.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__global__ __launch_bounds__(SPLIT_THREADS, 1) void k_split(int H, int B, int splits, int pps,
                                                            const bf16* __restrict__ qt,
                                                            const bf16* __restrict__ rows,
                                                            const int32_t* __restrict__ block_table,
                                                            int max_blocks, const int32_t* __restrict__ ctx_lens,
                                                            float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ __attribute__((aligned(1024))) char lds[SPLIT_LDS];
  char* const qr = lds + N_SLOTS * TILE_BYTES;
  char* const pb = qr + QR_BYTES;
  float* const ab = (float*)(pb + PB_BYTES);
  const int split = blockIdx.x, b = blockIdx.y;
  const int L = ctx_lens[b];
  const int t_begin = split * pps * PAGE;
  const int t_end = min(t_begin + pps * PAGE, L);
  if (t_begin >= t_end) return;
  const int n_tiles = (t_end - t_begin + TILE - 1) / TILE;
  // the wave index is uniform: keep it (and the LDS bases derived from it) in SGPRs
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hl = lane & 31, g = lane >> 5, i16 = lane & 15, G = lane >> 4;
  const int h_own = w * 32 + hl;  // head of this lane in the score phase
  const int32_t* table = block_table + (size_t)b * max_blocks;

  // Streams tile i into ring slot i % 3: 9 direct-to-LDS 16-byte loads per
  // lane. Instruction k of wave w fills slot chunks [(w*9+k)*64, +64) in
  // order; each lane picks the global chunk that belongs at its (swizzled)
  // position.
  // The 9 loads of wave w cover exactly rows 8w .. 8w+7 of the tile, so the
  // per-lane global offsets are the same for every tile: computed once here.
  uint32_t ld_off[TILE_LOADS];
#pragma unroll
  for (int k = 0; k < TILE_LOADS; ++k) {
    const int pos = (w * TILE_LOADS + k) * 64 + lane;
    const int t = pos / ROW_CHUNKS, jp = pos - t * ROW_CHUNKS;
    ld_off[k] = (uint32_t)(t * ROW_BYTES + ((jp ^ swz(t)) << 4));
  }
  const uint32_t lds_base = (uint32_t)(size_t)(LDS_AS char*)lds;
  auto load_tile = [&](int i) {
    const int t0 = t_begin + i * TILE;
    const char* src = (const char*)(rows + ((size_t)table[t0 / PAGE] * PAGE + (t0 % PAGE)) * ROW);
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_base + (i % N_SLOTS) * TILE_BYTES +
                                                        w * TILE_LOADS * 64 * 16);
#pragma unroll
    for (int k = 0; k < TILE_LOADS; ++k) dma16(src + ld_off[k], dst + k * 64 * 16);
  };

  // RoPE slice of the query of every head, in LDS: head h's 16-byte chunk c
  // (of 8) at h*128 + ((c ^ ((h >> 1) & 7)) * 16).
  for (int i = threadIdx.x; i < MAX_HEADS * (DR / 8); i += SPLIT_THREADS) {
    const int hh = i >> 3, c = i & 7;
    u32x4 v = {0, 0, 0, 0};
    if (hh < H) v = *(const u32x4*)(qt + ((size_t)b * H + hh) * ROW + DC + 8 * c);
    *(u32x4*)(qr + hh * 128 + ((c ^ ((hh >> 1) & 7)) << 4)) = v;
  }
  // latent part of this lane's query: Qt[b, h_own, 16s + 8g .. +7], s < 32
  // (lanes of heads >= H read head H-1; nothing of theirs is stored)
  bf16x8_t qf[LAT_STEPS];
  {
    const bf16* q = qt + ((size_t)b * H + min(h_own, H - 1)) * ROW + 8 * g;
#pragma unroll
    for (int s = 0; s < LAT_STEPS; ++s) qf[s] = as_bf16x8(*(const u32x4*)(q + 16 * s));
  }
  wait_vmcnt<0>();  // query loads done: from here on only tile loads use vmcnt
  load_tile(0);
  if (n_tiles > 1) load_tile(1);

  f32x16 o[4][4];  // [column tile][head tile]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) o[i][j] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;

  // LDS byte offsets of this lane's operand reads (lane part; the rest is a
  // compile-time immediate):
  //  score operand, step s: row hl, chunk (2s + g) ^ swz(hl)
  //    = qk_off[s % 4] + (s / 4) * 128
  //  RoPE query operand, step r: head h_own, chunk 2r + g
  //  value operand (column tile ct, step j, half a/b): rows 16j + 4g + i16/4
  //    (+8 for b), columns 128w + 32ct + 16(G%2) + 4(i16%4) .. +3
  //    = pv_off[ct % 2][a/b] + 16*j*ROW_BYTES + (ct / 2) * 128
  int qk_off[4], pv_off[2][2], qr_off[ROPE_STEPS];
  {
    const int x = swz(hl);
#pragma unroll
    for (int u = 0; u < 4; ++u) qk_off[u] = hl * ROW_BYTES + (((2 * u + g) ^ x) << 4);
    const int ra = 4 * g + (i16 >> 2), rb = ra + 8;
    const int y0 = 2 * (G & 1) + ((i16 & 3) >> 1), sub = 8 * (i16 & 1);
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      pv_off[par][0] = ra * ROW_BYTES + (((4 * par + y0) ^ swz(ra)) << 4) + sub + w * 256;
      pv_off[par][1] = rb * ROW_BYTES + (((4 * par + y0) ^ swz(rb)) << 4) + sub + w * 256;
    }
#pragma unroll
    for (int r = 0; r < ROPE_STEPS; ++r) qr_off[r] = h_own * 128 + (((2 * r + g) ^ ((h_own >> 1) & 7)) << 4);
  }
  const LDS_AS char* qrl = (const LDS_AS char*)qr;
  const LDS_AS char* pbl = (const LDS_AS char*)pb;

  for (int i = 0; i < n_tiles; ++i) {
    if (i + 1 < n_tiles) wait_vmcnt<TILE_LOADS>();  // tile i landed, tile i+1 may fly
    else wait_vmcnt<0>();
    lds_barrier();  // tile i visible to all; slot (i+2)%3 and P/alpha buffers free
    if (i + 2 < n_tiles) load_tile(i + 2);
    const LDS_AS char* tile = (const LDS_AS char*)(lds + (i % N_SLOTS) * TILE_BYTES);

    // ---- scores of this wave's 32 heads over the tile's 32 rows ----
    // Issue order is pinned to "MFMA s, read s+QK_AHEAD" so the LDS reads run
    // while the MFMAs execute (in-order issue would otherwise hold them back).
    f32x16 sc = {};
    {
      constexpr int QK_AHEAD = 4;
      u32x4 fa[QK_AHEAD], fb[QK_AHEAD];
      auto qk_read = [&](int s) {
        fa[s % QK_AHEAD] = *(const LDS_AS u32x4*)(tile + qk_off[s & 3] + (s >> 2) * 128);
        if (s >= LAT_STEPS) fb[s % QK_AHEAD] = *(const LDS_AS u32x4*)(qrl + qr_off[(s - LAT_STEPS) & 3]);
      };
#pragma unroll
      for (int s = 0; s < QK_AHEAD; ++s) qk_read(s);
#pragma unroll
      for (int s = 0; s < ROW / 16; ++s) {
        const bf16x8_t bq = s < LAT_STEPS ? qf[s < LAT_STEPS ? s : 0] : as_bf16x8(fb[s % QK_AHEAD]);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fa[s % QK_AHEAD]), bq, sc, 0, 0, 0);
        if (s + QK_AHEAD < ROW / 16) qk_read(s + QK_AHEAD);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // mask rows past the context (last tile only); lane rows: 8(r/4) + 4g + r%4
    const int valid = t_end - (t_begin + i * TILE);
    if (valid < TILE) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + 4 * g + (r & 3) >= valid) sc[r] = -INFINITY;
    }
    // ---- online softmax of the owned heads ----
    float mx = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // Lazy rescaling: the reference max only moves when the tile max exceeds
    // it by more than 8 (so p <= 2^8); a lane's first tile just sets it.
    float alpha = 1.f;
    if (mx > m_run + 8.f) {
      if (m_run != -INFINITY) alpha = __builtin_amdgcn_exp2f(m_run - mx);
      m_run = mx;
    }
    l_run *= alpha;
    {
      float lsum = 0.f;
      // P fragment (head tile w, step j, lane group g, head hl): the 8 rows
      // 16j + 8(k/4) + 4g + k%4 = this lane's registers 8j .. 8j+7
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf16x8_t pk;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float e = __builtin_amdgcn_exp2f(sc[8 * j + k] - m_run);
          lsum += e;
          pk[k] = (__bf16)e;
        }
        *(LDS_AS bf16x8_t*)((LDS_AS char*)pb + (w * 2 + j) * 1024 + lane * 16) = pk;
      }
      l_run += lsum;
    }
    if (g == 0) ab[h_own] = alpha;
    lds_barrier();  // P and alpha of all heads visible

    // ---- rescale (rare), then O^T[c, h] += V^T[c, t] P[t, h] ----
    float al[4];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) al[ht] = ab[32 * ht + hl];
    if (__ballot(al[0] != 1.f || al[1] != 1.f || al[2] != 1.f || al[3] != 1.f)) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x = o[ct][ht][r];
            scale_acc(x, al[ht]);
            o[ct][ht][r] = x;
          }
    }
    // value fragments (4 column tiles) and P fragments (4 head tiles) of step
    // j; step 1's reads are issued between step 0's MFMAs
    bf16x8_t va[2][4], pf[2][4];
    auto pv_read = [&](int j, int ct) {
      const int k = 16 * j * ROW_BYTES + (ct >> 1) * 128;
      va[j][ct] = cat_tr(tr_read(tile + pv_off[ct & 1][0] + k), tr_read(tile + pv_off[ct & 1][1] + k));
      pf[j][ct] = *(const LDS_AS bf16x8_t*)(pbl + (ct * 2 + j) * 1024 + lane * 16);
    };
#pragma unroll
    for (int q = 0; q < 4; ++q) pv_read(0, q);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
          o[ct][ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[j][ct], pf[j][ht], o[ct][ht], 0, 0, 0);
        if (j == 0) pv_read(1, ct);
        __builtin_amdgcn_sched_barrier(0);
      }
  }

  // ---- partials: (m, l) by the head owner, O slices by the column owner ----
  l_run += __shfl_xor(l_run, 32, 64);
  if (g == 0 && h_own < H) {
    const size_t prow = ((size_t)h_own * B + b) * splits + split;
    part_ml[prow * 2] = m_run;
    part_ml[prow * 2 + 1] = l_run;
  }
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    const int hh = 32 * ht + hl;
    if (hh >= H) continue;
    float* po = part_o + (((size_t)hh * B + b) * splits + split) * DC + 128 * w;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = {o[ct][ht][4 * q], o[ct][ht][4 * q + 1], o[ct][ht][4 * q + 2], o[ct][ht][4 * q + 3]};
        *(f32x4*)(po + 32 * ct + 8 * q + 4 * g) = v;
      }
  }
}

// -------------------------------------------------------- k_combine_uv ----
// One block per (head, tile of 16 sequences). Blocks of the same head share
// blockIdx % 8, i.e. the same XCD and L2, so W_UV,h is fetched from HBM once.
//   1. per sequence: M = max_s m_s, weights e_s = 2^(m_s - M), 1 / sum_s e_s l_s
//      (one wave per 4 sequences, lanes over splits)
//   2. o_c = sum_s e_s O_s / sum_s e_s l_s, 16 threads per sequence, all the
//      split loads of a thread issued together; bf16 into LDS
//   3. out^T[v, b] = sum_c W_UV[h*128 + v, c] o_c[b, c] on MFMA; each lane ends
//      with 4 consecutive outputs of one sequence (one 8-byte store)
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
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int i16 = lane & 15, G = lane >> 4;
  // W_UV,h fragments of this wave (rows 32w .. 32w+31, all 512 columns) are
  // independent of everything else: request them first
  const bf16* wv = w_uv + (size_t)h * DV * DC;
  u32x4 wf[DC / 32][2];
#pragma unroll
  for (int ks = 0; ks < DC / 32; ++ks)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) wf[ks][mt] = *(const u32x4*)(wv + (size_t)(32 * w + 16 * mt + i16) * DC + 32 * ks + 8 * G);
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int r = 4 * w + rr, b = b0 + r;
    const int ns = b < B ? ((ctx_lens[b] + PAGE - 1) / PAGE + pps - 1) / pps : 0;
    const float* ml = part_ml + ((size_t)h * B + (b < B ? b : 0)) * splits * 2;
    float M = -INFINITY;
    for (int s = lane; s < ns; s += 64) M = fmaxf(M, ml[2 * s]);
    M = wave_max(M);
    float l = 0.f;
    for (int s = lane; s < splits; s += 64) {
      const float e = s < ns ? __builtin_amdgcn_exp2f(ml[2 * s] - M) : 0.f;
      wgt[r][s] = e;
      if (s < ns) l += e * ml[2 * s + 1];
    }
    l = wave_sum(l);
    if (lane == 0) inv_l[r] = ns > 0 ? 1.f / l : 0.f;
  }
  __syncthreads();
  {
    const int r = tid >> 4, q = tid & 15, b = b0 + r;  // 16 threads per sequence, 8 float4 each
    f32x4 acc[8] = {};
    if (b < B) {
      const float* po = part_o + ((size_t)h * B + b) * splits * DC + 4 * q;
      // two splits' loads in flight per step; splits past the context were
      // never written, so their (arbitrary) values are selected away, not scaled
      for (int s = 0; s < splits; s += 2) {
        f32x4 v[2][8];
#pragma unroll
        for (int d = 0; d < 2; ++d)
#pragma unroll
          for (int u = 0; u < 8; ++u)
            v[d][u] = s + d < splits ? *(const f32x4*)(po + (size_t)(s + d) * DC + 64 * u) : (f32x4){0, 0, 0, 0};
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const float e = s + d < splits ? wgt[r][s + d] : 0.f;
#pragma unroll
          for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int x = 0; x < 4; ++x) acc[u][x] += e != 0.f ? e * v[d][u][x] : 0.f;
        }
      }
    }
    const float il = inv_l[r];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
      const bf16x4_t v = {(__bf16)(acc[u][0] * il), (__bf16)(acc[u][1] * il), (__bf16)(acc[u][2] * il),
                          (__bf16)(acc[u][3] * il)};
      *(bf16x4_t*)&oc[r * LDO + 4 * q + 64 * u] = v;
    }
  }
  __syncthreads();
  // wave w: outputs v = 32w .. 32w+31 (two 16-row tiles), all 16 sequences
  f32x4 acc[2] = {};
#pragma unroll
  for (int ks = 0; ks < DC / 32; ++ks) {
    const bf16x8_t bo = as_bf16x8(*(const u32x4*)&oc[i16 * LDO + 32 * ks + 8 * G]);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wf[ks][mt]), bo, acc[mt], 0, 0, 0);
  }
  const int b = b0 + i16;
  if (b < B) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
      const bf16x4_t v = {(__bf16)acc[mt][0], (__bf16)acc[mt][1], (__bf16)acc[mt][2], (__bf16)acc[mt][3]};
      *(bf16x4_t*)(out + ((size_t)b * H + h) * DV + 32 * w + 16 * mt + 4 * G) = v;
    }
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
