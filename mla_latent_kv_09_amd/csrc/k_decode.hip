// MFMA decode path for the DeepSeek-V3 latent shape (bf16, d_c 512,
// d_rope 64, d_nope = d_v = 128, 64-token pages, up to 256 heads: groups of
// 128 heads run side by side).
//
// Three kernels, one stream:
//   k_absorb       Qt[b,h] = s*log2(e) * [W_UK,h^T q_nope[b,h] || RoPE(q_pe[b,h], L_b - 1)]
//                  ("DeepSeek-V2 paper digest" §2.2: W_UK folded into the query;
//                  §2.3: only the decoupled slice is rotated).
//   k_split        one workgroup per (query row, run of pages, head group),
//                  runs dispatched longest first (common.h): every page of
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

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int DC = 512, DR = 64, ROW = DC + DR, DN = 128, DV = 128;
constexpr int PAGE = 64;
constexpr int ROW_BYTES = ROW * 2;               // 1152
constexpr int ROW_CHUNKS = ROW_BYTES / 16;       // 72 chunks of 16 B
constexpr int SPLIT_THREADS = 256;               // 4 waves
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

// x[0..7] *= a for MFMA accumulators that live in AGPRs, written out so the
// compiler keeps the 256 output accumulators in AGPRs across the page loop
// (a plain multiply makes it shuttle them through VGPRs and spill). Eight
// reads, eight multiplies, eight writes: each VGPR is written two or more
// instructions before it is read. The caller pads the wait states an
// accumulator read needs after an MFMA wrote it (rescale_fence), once per
// rescale rather than per register.
__device__ __forceinline__ void scale_acc8(float& x0, float& x1, float& x2, float& x3, float& x4, float& x5,
                                           float& x6, float& x7, float a) {
  float t0, t1, t2, t3, t4, t5, t6, t7;
  asm volatile(
      "v_accvgpr_read_b32 %8, %0\n\tv_accvgpr_read_b32 %9, %1\n\t"
      "v_accvgpr_read_b32 %10, %2\n\tv_accvgpr_read_b32 %11, %3\n\t"
      "v_accvgpr_read_b32 %12, %4\n\tv_accvgpr_read_b32 %13, %5\n\t"
      "v_accvgpr_read_b32 %14, %6\n\tv_accvgpr_read_b32 %15, %7\n\t"
      "v_mul_f32 %8, %8, %16\n\tv_mul_f32 %9, %9, %16\n\tv_mul_f32 %10, %10, %16\n\tv_mul_f32 %11, %11, %16\n\t"
      "v_mul_f32 %12, %12, %16\n\tv_mul_f32 %13, %13, %16\n\tv_mul_f32 %14, %14, %16\n\tv_mul_f32 %15, %15, %16\n\t"
      "v_accvgpr_write_b32 %0, %8\n\tv_accvgpr_write_b32 %1, %9\n\t"
      "v_accvgpr_write_b32 %2, %10\n\tv_accvgpr_write_b32 %3, %11\n\t"
      "v_accvgpr_write_b32 %4, %12\n\tv_accvgpr_write_b32 %5, %13\n\t"
      "v_accvgpr_write_b32 %6, %14\n\tv_accvgpr_write_b32 %7, %15"
      : "+a"(x0), "+a"(x1), "+a"(x2), "+a"(x3), "+a"(x4), "+a"(x5), "+a"(x6), "+a"(x7), "=&v"(t0), "=&v"(t1),
        "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&v"(t5), "=&v"(t6), "=&v"(t7)
      : "v"(a));
}
// 21 wait states: an MFMA that may still be writing an accumulator before it
// is read, or an accumulator write before an MFMA reads it.
__device__ __forceinline__ void rescale_fence() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" ::: "memory"); }

// Scales the 16 accumulators of one MFMA tile.
__device__ __forceinline__ void scale_tile(f32x16& v, float a) {
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = v[r];
  scale_acc8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7], a);
  scale_acc8(x[8], x[9], x[10], x[11], x[12], x[13], x[14], x[15], a);
#pragma unroll
  for (int r = 0; r < 16; ++r) v[r] = x[r];
}

struct Plan {
  int pages_per_split;
  int splits;
};

// batch counts query rows; q_len > 1 rows per sequence share their pages
Plan plan_splits(int batch, int max_context, int q_len) {
  const int max_pages = (max_context + PAGE - 1) / PAGE;
  // aim for one workgroup per compute unit across the batch, 4..32 pages each;
  // with several rows per sequence up to 64, which halves the partials
  // (one per row and run) where the rows alone fill the chip. This sees only
  // the longest context; with one new token per row the split kernel may
  // lengthen the runs once it has the actual lengths (never shorten them, so
  // `splits` bounds every row's runs).
  const int cap = q_len > 1 ? 64 : 32;
  int pps = (int)(((int64_t)batch * max_pages + 255) / 256);
  pps = pps < 4 ? 4 : (pps > cap ? cap : pps);
  const int min_pps = (max_pages + MAX_SPLITS - 1) / MAX_SPLITS;
  if (pps < min_pps) pps = min_pps;
  Plan p;
  p.pages_per_split = pps;
  p.splits = (max_pages + pps - 1) / pps;
  return p;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t qt, part_o, part_ml, run, total;
};

WsLayout ws_layout(int H, int batch, int splits) {
  WsLayout l;
  l.qt = 0;
  l.part_o = align256((size_t)batch * H * ROW * 2);
  l.part_ml = l.part_o + align256((size_t)H * batch * splits * DC * 2);
  l.run = l.part_ml + align256((size_t)H * batch * splits * 2 * 4);
  l.total = l.run + 256;  // the run length the split kernel used, for the combine
  return l;
}

// Query row v of a step with q_len new tokens per sequence belongs to sequence
// v / q_len, whose last q_len cached tokens are the new ones; token j = v %
// q_len sits at position ctx - q_len + j and sees ctx - (q_len - 1 - j) rows.
// With q_len == 1 this is the sequence's whole context.
__device__ __forceinline__ int visible_rows(const int32_t* ctx_lens, int v, int q_len) {
  if (q_len == 1) return ctx_lens[v];
  const int seq = v / q_len;
  return ctx_lens[seq] - (q_len - 1 - (v - seq * q_len));
}

// ------------------------------------------------------------ k_absorb ----
// RoPE inverse frequencies base^(-2i/d_rope), formed on the host in double
struct RopeFreq {
  double theta[DR / 2];
};

// grid (H, DC / CW); 4 waves; one block round on the chip for H = 128. Block
// (h, c0) forms Qt[:, h, c0 .. c0+CW-1] for every query row as the transposed
// product Qt^T[c, b] = sum_j W_UK[h*128+j, c] q_nope[b, h, j]. CW is 128
// columns, or 64 or 32 with fewer than 64 heads, so that the grid still has
// about one block per compute unit. The 128 x CW slice of W_UK,h and the first
// 64 query rows are requested before anything else, so each block has all of
// its HBM reads in flight at once.
// The slice is staged in LDS and read transposed (the A operand); wave w takes
// query rows 16w .. 16w+15 of each 64-row chunk (the B operand, straight from
// memory: 8 consecutive j of one row per lane) against all CW / 16 column
// tiles, so every query element is loaded once per block. Results go through
// LDS so that each row segment (CW columns) is written whole. The blocks
// of head h also write its rotated, scaled q_pe slice, each for every 4th row.
template <int CW>
__global__ __launch_bounds__(256) void k_absorb(int B, int H, int q_len, const bf16* __restrict__ q_nope,
                                                const bf16* __restrict__ q_pe, const bf16* __restrict__ w_uk,
                                                const int32_t* __restrict__ ctx_lens, float qscale, RopeFreq rope,
                                                bf16* __restrict__ qt) {
  constexpr int LD = CW + 8;    // padded row (272 B at CW = 128): two-way LDS conflicts at most on the transposed reads
  constexpr int NCB = DC / CW;  // column blocks per head
  constexpr int CPR = CW / 8;   // 16-byte chunks per slice row
  __shared__ __attribute__((aligned(16))) bf16 wt[DN * LD];
  __shared__ __attribute__((aligned(16))) bf16 ot[64 * LD];
  const int h = blockIdx.x, c0 = blockIdx.y * CW;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, i16 = lane & 15, G = lane >> 4;
  // W_UK slice: 128 rows of 2 CW bytes, CPR lanes per row
  u32x4 wr[DN * CW / 8 / 256];
#pragma unroll
  for (int u = 0; u < DN * CW / 8 / 256; ++u) {
    const int i = threadIdx.x + 256 * u, j = i / CPR, ch = i % CPR;
    wr[u] = *(const u32x4*)(w_uk + (size_t)(h * DN + j) * DC + c0 + ch * 8);
  }
  auto load_q = [&](int b0, u32x4 (&qv)[DN / 32]) {
    const int b = b0 + 16 * w + i16;
#pragma unroll
    for (int ks = 0; ks < DN / 32; ++ks)
      qv[ks] = b < B ? *(const u32x4*)(q_nope + ((size_t)b * H + h) * DN + 32 * ks + 8 * G) : (u32x4){0, 0, 0, 0};
  };
  u32x4 qv[DN / 32];
  load_q(0, qv);
  // RoPE part of this thread: pair i = tid % 32 of rows b = NCB k + blockIdx.y
  // with k = tid / 32, tid / 32 + 8, ... (first one's inputs requested now)
  const int rp_i = threadIdx.x & (DR / 2 - 1);
  const int rp_b0 = (threadIdx.x / (DR / 2)) * NCB + blockIdx.y;
  constexpr int RP_STEP = (256 / (DR / 2)) * NCB;
  int rp_len = 0;
  uint32_t rp_x = 0;
  if (rp_b0 < B) {
    rp_len = visible_rows(ctx_lens, rp_b0, q_len);
    rp_x = *(const uint32_t*)(q_pe + ((size_t)rp_b0 * H + h) * DR + 2 * rp_i);
  }
#pragma unroll
  for (int u = 0; u < DN * CW / 8 / 256; ++u) {
    const int i = threadIdx.x + 256 * u, j = i / CPR, ch = i % CPR;
    *(u32x4*)&wt[j * LD + ch * 8] = wr[u];
  }
  __syncthreads();
  const LDS_AS char* wbase = (const LDS_AS char*)wt;
  for (int b0 = 0; b0 < B; b0 += 64) {
    u32x4 cur[DN / 32];
#pragma unroll
    for (int ks = 0; ks < DN / 32; ++ks) cur[ks] = qv[ks];
    if (b0 + 64 < B) load_q(b0 + 64, qv);
    // one K step at a time over the CW / 16 column tiles (independent
    // accumulators); the next step's transposing reads go out before this
    // step's MFMAs
    f32x4 acc[CW / 16];
#pragma unroll
    for (int ct = 0; ct < CW / 16; ++ct) acc[ct] = (f32x4){0.f, 0.f, 0.f, 0.f};
    bf16x8_t af[2][CW / 16];
    auto read_step = [&](int ks, bf16x8_t (&a)[CW / 16]) __attribute__((always_inline)) {
#pragma unroll
      for (int ct = 0; ct < CW / 16; ++ct) {
        const int k0 = 32 * ks + 8 * G, col = 16 * ct + 4 * (i16 & 3);
        a[ct] = cat_tr(tr_read(wbase + ((k0 + (i16 >> 2)) * LD + col) * 2),
                       tr_read(wbase + ((k0 + 4 + (i16 >> 2)) * LD + col) * 2));
      }
    };
    read_step(0, af[0]);
    __builtin_amdgcn_sched_group_barrier(0x100, CW / 8, 0);
#pragma unroll
    for (int ks = 0; ks < DN / 32; ++ks) {
      if (ks + 1 < DN / 32) {
        read_step(ks + 1, af[(ks + 1) & 1]);
        __builtin_amdgcn_sched_group_barrier(0x100, CW / 8, 0);
      }
#pragma unroll
      for (int ct = 0; ct < CW / 16; ++ct)
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks & 1][ct], as_bf16x8(cur[ks]), acc[ct], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, CW / 16, 0);
    }
    // lane: columns 16 ct + 4 G .. +3 of row 16 w + i16; each wave stages and
    // stores only its own 16 rows
    typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
#pragma unroll
    for (int ct = 0; ct < CW / 16; ++ct)
      *(bf16x4_t*)&ot[(16 * w + i16) * LD + 16 * ct + 4 * G] =
          (bf16x4_t){(__bf16)(acc[ct][0] * qscale), (__bf16)(acc[ct][1] * qscale), (__bf16)(acc[ct][2] * qscale),
                     (__bf16)(acc[ct][3] * qscale)};
    __syncthreads();
#pragma unroll
    for (int k = 0; k < CPR / 4; ++k) {
      const int r = 16 * w + (64 / CPR) * k + lane / CPR, ch = lane % CPR, b = b0 + r;
      if (b < B) *(u32x4*)(qt + ((size_t)b * H + h) * ROW + c0 + 8 * ch) = *(const u32x4*)&ot[r * LD + 8 * ch];
    }
    __syncthreads();  // this chunk's rows are out of ot before the next one lands
  }
  // the rotated, scaled q_pe slice: reduce the angle to [-pi, pi] in double,
  // then single-precision sin/cos
  const double theta = rope.theta[rp_i];
  for (int b = rp_b0; b < B; b += RP_STEP) {
    if (b != rp_b0) {
      rp_len = visible_rows(ctx_lens, b, q_len);
      rp_x = *(const uint32_t*)(q_pe + ((size_t)b * H + h) * DR + 2 * rp_i);
    }
    const double ang = (double)(rp_len - 1) * theta;
    const float r = (float)(ang - 6.283185307179586 * rint(ang * 0.15915494309189535));
    float sn, cs;
    sincosf(r, &sn, &cs);
    const float x0 = __uint_as_float(rp_x << 16), x1 = __uint_as_float(rp_x & 0xFFFF0000u);
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    const bf16x2_t v = {(__bf16)((x0 * cs - x1 * sn) * qscale), (__bf16)((x0 * sn + x1 * cs) * qscale)};
    *(bf16x2_t*)(qt + ((size_t)b * H + h) * ROW + DC + 2 * rp_i) = v;
  }
}

// ------------------------------------------------------------- k_split ----
// grid (splits, B, head groups); 256 threads (4 waves); one block per
// (sequence, run of pages, group of up to 128 heads: one group unless there
// are more than 128 heads). The run is walked in tiles of 32 cache rows (half
// a page, 36 KB).
//
// Work split inside the block, per tile:
//   scores    wave w owns heads 32w .. 32w+31: S^T[t, h] = row_t . Qt[h]
//             (36 MFMA steps of K = 16 over the 576 columns; the query of the
//             lane's head stays in registers), then the online softmax of those
//             heads (running max m and sum l stay with the owner). The
//             probabilities P (bf16) go to LDS.
//   values    wave w owns latent columns 128w .. 128w+127 of every head:
//             O^T[c, h] += V^T[c, t] P[t, h] (4 column tiles x 4 head tiles x
//             2 steps). Each value fragment, read once from LDS, feeds four
//             MFMAs; so does each P fragment.
// Software pipeline, one barrier per tile: iteration i computes the scores of
// tile i, then the value product of tile i - 1 with the softmax of tile i
// spread between its MFMAs (they are independent), then publishes P of tile
// i. P is double-buffered; tiles stream HBM -> LDS with direct 16-byte loads
// into a ring of four slots (tile i - 1 in the value step, tile i in the score
// step, tiles i + 1 and i + 2 in flight): 4 x 36 KB + 2 x 8 KB = 160 KB.
//
// The reference max is set by the first tile and then moves lazily (only when
// a tile's max exceeds it by more than 8) and only by whole steps k, so the
// rescale factor of the other waves' accumulators is an exact power of two
// 2^-k; a jump of 255 or more resets the reference to the tile's max and
// sends k = 255 (factor 0 in fp32). The owner sends k (8 bits) in
// the sign bits of the head's first P fragment (P >= 0, so those bits are
// otherwise clear); the readers test them, and in the rare case decode k,
// clear the bits and rescale.
//
// Partials per (head, sequence, split): O (512 values, unnormalised, relative
// to the head's reference max m; accumulated in fp32, stored as bf16, which
// halves the partials' HBM traffic for one bf16 rounding of each partial) and
// (m, l) in fp32, both in the log2 domain.
constexpr int TILE = 32;                                  // rows per tile
constexpr int TILE_BYTES = TILE * ROW_BYTES;              // 36864
constexpr int TILE_LOADS = TILE * ROW_CHUNKS / SPLIT_THREADS;  // 9 per lane
constexpr int N_SLOTS = 4;
constexpr int PB_BYTES = MAX_HEADS * TILE * 2;            // 8 KB: P of one tile
constexpr int QK_STEPS = ROW / 16;                        // 36 score steps
constexpr int SPLIT_LDS = N_SLOTS * TILE_BYTES + 2 * PB_BYTES;
static_assert(SPLIT_LDS <= 160 * 1024, "LDS budget of one workgroup");

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

// Same copy with the address split into a uniform 64-bit base (SGPRs) and a
// per-lane 32-bit byte offset, so no 64-bit per-lane pointer is kept live.
__device__ __forceinline__ void dma16s(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds_addr)
               : "memory", "m0");
}

// Score MFMA (32x32x16 bf16) with its accumulator in VGPRs, written out so the
// compiler does not place it in AGPRs (all of which hold the value
// accumulators) and shuttle registers around it. Chained MFMAs on the same
// accumulator need no wait states; mfma_qk_done() pads the wait states a
// vector instruction needs before it reads (or writes) the result.
__device__ __forceinline__ void mfma_qk_first(f32x16& acc, bf16x8_t a, bf16x8_t b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_qk(f32x16& acc, bf16x8_t a, bf16x8_t b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_qk_done(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
}

// Workgroup barrier for LDS traffic only. __syncthreads() also waits for all
// outstanding global loads (vmcnt 0), which would drain the tile prefetch.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int NHT>
__global__ __launch_bounds__(SPLIT_THREADS, 1) void k_split(int H, int B, int q_len, int order, int splits,
                                                            int pps, int budget, int32_t* __restrict__ run_out,
                                                            const bf16* __restrict__ qt,
                                                            const bf16* __restrict__ rows,
                                                            const int32_t* __restrict__ block_table,
                                                            int max_blocks, const int32_t* __restrict__ ctx_lens,
                                                            bf16* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ __attribute__((aligned(1024))) char lds[SPLIT_LDS];
  // b is the query row (sequence b / q_len, new token b % q_len)
  // block order: 0 plain (split fastest), 1 rows of one sequence paired on
  // an XCD (below), 2 longest runs first (one new token per row)
  // With the longest-first order the run length may grow from pps so that
  // the step's runs fit in one round of `budget` workgroups; the first block
  // records the length used for the combine.
  int split = blockIdx.x, b = blockIdx.y, len_b = 0;
  int lens[4] = {0, 0, 0, 0};
  if (order == 2) load_row_lens(B, ctx_lens, lens);
  // (only when the launch's slots, splits x B, exceed one round: otherwise
  // the runs of pps fit whatever the lengths)
  const int pps_run = order == 2 && splits * B > budget ? one_round_run_pages(pps, 64, budget, PAGE, lens) : pps;
  if ((blockIdx.x | blockIdx.y | blockIdx.z) == 0 && threadIdx.x == 0) *run_out = pps_run;
  if (order == 2) {
    if (!longest_run_first(B, pps_run * PAGE, lens, blockIdx.y * gridDim.x + blockIdx.x, b, split, len_b))
      return;
  } else if (order == 1) {
    // the q_len rows of one (sequence, split) read the same pages: give them
    // consecutive dispatch slots of one XCD (block i runs on XCD i % 8) so
    // that all but the first find the pages in that XCD's L2. Needs the
    // number of (sequence, split) units to be a multiple of 8.
    const int lin = blockIdx.y * gridDim.x + blockIdx.x, local = lin >> 3;
    const int unit_local = local / q_len, j = local - unit_local * q_len;
    const int unit = unit_local * 8 + (lin & 7), seq = unit / splits;
    split = unit - seq * splits;
    b = seq * q_len + j;
  }
  const int seq = b / q_len;
  const int L = order == 2 ? len_b : visible_rows(ctx_lens, b, q_len);
  const int t_begin = split * pps_run * PAGE;
  const int t_end = min(t_begin + pps_run * PAGE, L);
  if (t_begin >= t_end) return;
  const int n_tiles = (t_end - t_begin + TILE - 1) / TILE;
  // the wave index is uniform: keep it (and the LDS bases derived from it) in SGPRs
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hl = lane & 31, g = lane >> 5, i16 = lane & 15, G = lane >> 4;
  // head group: blocks with blockIdx.z = z take heads 128z .. 128z+127
  // (several groups only for more than 128 heads; each streams the run)
  const int h0 = MAX_HEADS * blockIdx.z;
  const int h_own = h0 + w * 32 + hl;  // head of this lane in the score phase
  const int32_t* table = block_table + (size_t)seq * max_blocks;

  // Streams tile i into ring slot i % 4: 9 direct-to-LDS 16-byte loads per
  // lane. Instruction k of wave w fills slot chunks [(w*9+k)*64, +64) in
  // order; each lane picks the global chunk that belongs at its (swizzled)
  // position. The 9 loads of wave w cover exactly rows 8w .. 8w+7 of the
  // tile, so the per-lane global offsets are the same for every tile.
  // (offsets < 36864: two per register, unpacked at each use)
  uint32_t ld_off[(TILE_LOADS + 1) / 2];
#pragma unroll
  for (int k = 0; k < TILE_LOADS; ++k) {
    const int pos = (w * TILE_LOADS + k) * 64 + lane;
    const int t = pos / ROW_CHUNKS, jp = pos - t * ROW_CHUNKS;
    const uint32_t off = (uint32_t)(t * ROW_BYTES + ((jp ^ swz(t)) << 4));
    if (k & 1) ld_off[k / 2] |= off << 16;
    else ld_off[k / 2] = off;
  }
  // The run's page numbers (at most 32), one per lane, read once: each tile
  // then takes its page from a register, so no scalar load (and its latency)
  // sits in front of the copies.
  const int run_pages = (t_end - t_begin + PAGE - 1) / PAGE;
  const int page_of_lane = lane < run_pages ? table[t_begin / PAGE + lane] : 0;
  const uint32_t lds_base = (uint32_t)(size_t)(LDS_AS char*)lds;
  auto load_tile = [&](int i) {
    const int page = __builtin_amdgcn_readlane(page_of_lane, i >> 1);  // TILE is half a page
    const char* src = (const char*)(rows + ((size_t)page * PAGE + (i & 1) * TILE) * ROW);
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_base + (i % N_SLOTS) * TILE_BYTES +
                                                        w * TILE_LOADS * 64 * 16);
#pragma unroll
    for (int k = 0; k < TILE_LOADS; ++k) {
      const uint32_t off = (k & 1) ? (ld_off[k / 2] >> 16) : (ld_off[k / 2] & 0xFFFFu);
      dma16s(src, off, dst + k * 64 * 16);
    }
  };

  // Rows past the context in the last tile hold whatever the page holds
  // beyond the sequence, possibly non-finite bit patterns. The score step
  // masks them (a select), but in the value product 0 * NaN is NaN, so before
  // that tile's value step each lane zeroes the chunks its own copies brought
  // in for those rows. A wave still in the tile's score step may read either
  // value there; it discards both.
  auto clear_tail = [&](int i) {
    const int valid = t_end - (t_begin + i * TILE);
    if (valid >= TILE) return;
    // copy k of this lane filled chunk pos = (9w + k) * 64 + lane, of row pos / 72
    // (the lane index is recomputed here so that nothing stays live across the loop)
    const int first = w * TILE_LOADS * 64 + (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int lim = valid * ROW_CHUNKS - first;  // chunk pos is past the context iff 64 k >= lim
    LDS_AS char* base = (LDS_AS char*)lds + (i % N_SLOTS) * TILE_BYTES + first * 16;
#pragma unroll
    for (int k = 0; k < TILE_LOADS; ++k)
      if (64 * k >= lim) *(LDS_AS u32x4*)(base + k * 1024) = (u32x4){0, 0, 0, 0};
  };

  // query of this lane's head: Qt[b, h_own, 16s + 8g .. +7], s < 36 (lanes of
  // heads >= H read head H-1; nothing of theirs is stored)
  bf16x8_t qf[QK_STEPS];
  __builtin_amdgcn_sched_barrier(0);  // the page numbers are requested before the query
  {
    const bf16* q = qt + ((size_t)b * H + min(h_own, H - 1)) * ROW + 8 * g;
#pragma unroll
    for (int s = 0; s < QK_STEPS; ++s) qf[s] = as_bf16x8(*(const u32x4*)(q + 16 * s));
  }
  // page numbers in (loads complete in order), the query may still fly: the
  // first tiles' copies go out now and travel together with the query
  wait_vmcnt<QK_STEPS>();
  load_tile(0);
  if (n_tiles > 1) load_tile(1);

  f32x16 o[4][NHT];  // [column tile][head tile]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NHT; ++j) o[i][j] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;

  // LDS byte offsets of this lane's operand reads (lane part; the rest is a
  // compile-time immediate):
  //  score operand, step s: row hl, chunk (2s + g) ^ swz(hl)
  //    = qk_off[s % 4] + (s / 4) * 128
  //  value operand (column tile ct, step j, half a/b): rows 16j + 4g + i16/4
  //    (+8 for b), columns 128w + 32ct + 16(G%2) + 4(i16%4) .. +3
  //    = pv_off[ct % 2][a/b] + 16*j*ROW_BYTES + (ct / 2) * 128
  //  P fragment (head tile ht, step j): buffer + (2ht + j) * 1024 + 16 lane
  int qk_off[4], pv_off[2][2];
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
  }
  auto slot = [&](int i) { return (const LDS_AS char*)(lds + ((i + N_SLOTS) % N_SLOTS) * TILE_BYTES); };
  auto pbuf = [&](int i) { return (LDS_AS char*)(lds + N_SLOTS * TILE_BYTES + (i & 1) * PB_BYTES) + lane * 16; };

  // ---- online softmax of the owned heads, in 8 slices (slice k of 8) ----
  // slices 0-1: tile max, new reference and its shift k; slices
  // 2-7: exponentials, row sum, bf16 P fragments
  float sm_mx, sm_sub, sm_alpha, sm_ls[3];
  int sm_k;
  bf16x8_t pk[2];
  auto softmax_slice = [&](const f32x16& sc, int k) {
    if (k == 0) {
      sm_mx = sc[0];
#pragma unroll
      for (int r = 1; r < 8; ++r) sm_mx = fmaxf(sm_mx, sc[r]);
    } else if (k == 1) {
#pragma unroll
      for (int r = 8; r < 16; ++r) sm_mx = fmaxf(sm_mx, sc[r]);
      {
        // the other half of the head's rows sits 32 lanes away
        const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(sm_mx), __float_as_uint(sm_mx), false, false);
        sm_mx = fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
      }
      // first tile: the reference is the exact max (its p is exactly 1);
      // later moves are by whole steps k >= 9. A jump of 255 or more resets
      // the reference to the max and sends k = 255: every earlier term then
      // weighs less than 2^-246 against the new max (its score was at most
      // 8 above the old reference), below the smallest fp32 number, so the
      // factor 2^-255 (0 in fp32) that the sum and the accumulators are
      // scaled by is their weight rounded to fp32.
      const bool first = m_run == -INFINITY;
      const bool up = !first && sm_mx > m_run + 8.f;
      const float kc = up ? ceilf(sm_mx - m_run) : 0.f;
      const bool reset = !(kc < 255.f);
      sm_k = reset ? 255 : (int)kc;
      sm_alpha = __builtin_amdgcn_ldexpf(1.f, -sm_k);
      m_run = (first || reset) ? sm_mx : m_run + kc;
      sm_sub = m_run;
    } else {
      // slices 2..7 take elements 0-2, 3-5, 6-8, 9-11, 12-14, 15; the row
      // sum is kept as three running sums of the slices' own short sums, so
      // no long chain of dependent adds is left for the end of the step
      const int e0 = 3 * (k - 2), e1 = min(e0 + 3, 16);
      float ps = 0.f;
#pragma unroll
      for (int e = e0; e < e1; ++e) {
        const float pe = __builtin_amdgcn_exp2f(sc[e] - sm_sub);
        ps = e == e0 ? pe : ps + pe;
        pk[e >> 3][e & 7] = (__bf16)pe;
      }
      const int a = (k - 2) % 3;
      sm_ls[a] = k < 5 ? ps : sm_ls[a] + ps;
      if (k == 7) {
        l_run = l_run * sm_alpha + ((sm_ls[0] + sm_ls[1]) + sm_ls[2]);
      }
    }
  };

  // publish P of tile i (after its softmax); a moved reference travels in the
  // sign bits of the first fragment, re-stored in that (rare) case. Storing
  // first keeps the exponentials in the MFMA groups: nothing lets them sink
  // past a branch to their store.
  auto publish = [&](int i) {
    LDS_AS char* pb = pbuf(i);
    *(LDS_AS bf16x8_t*)(pb + (w * 2) * 1024) = pk[0];
    *(LDS_AS bf16x8_t*)(pb + (w * 2 + 1) * 1024) = pk[1];
    if (__ballot(sm_k != 0)) {
      u32x4 v = __builtin_bit_cast(u32x4, pk[0]);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v[q] |= (((uint32_t)sm_k >> (2 * q)) & 1u) << 15 | (((uint32_t)sm_k >> (2 * q + 1)) & 1u) << 31;
      *(LDS_AS u32x4*)(pb + (w * 2) * 1024) = v;
    }
  };

  // ---- one pipeline step -------------------------------------------------
  // QK: scores of this wave's 32 heads over the 32 rows of tile i (36 MFMAs).
  // PV: O^T[c, h] += V^T[c, t] P[t, h] for tile i - 1 (8 groups of 4 MFMAs,
  // group k = step k / 4, column tile k % 4).
  // The score MFMAs are interleaved with PV groups 0-3 (9 score steps per
  // group), so the score operands' LDS reads are spread over 52 MFMAs; the
  // softmax of tile i then runs between PV groups 4-7. Issue order is pinned
  // with scheduling barriers, LDS reads a few MFMAs ahead of their use. The
  // nine copies of tile dma_i (= i + 2) go out one every fourth score step, so
  // the texture unit takes them as it frees up instead of in a burst.
  auto step = [&](auto do_qk, auto do_pv, int i, int dma_i) {
    // source and destination of this wave's copies of tile dma_i (uniform)
    const char* dma_src = nullptr;
    uint32_t dma_dst = 0;
    if (dma_i >= 0) {
      const int page = __builtin_amdgcn_readlane(page_of_lane, dma_i >> 1);
      dma_src = (const char*)(rows + ((size_t)page * PAGE + (dma_i & 1) * TILE) * ROW);
      dma_dst = __builtin_amdgcn_readfirstlane(lds_base + (dma_i % N_SLOTS) * TILE_BYTES + w * TILE_LOADS * 64 * 16);
    }
    constexpr bool QK = decltype(do_qk)::value, PV = decltype(do_pv)::value;
    const LDS_AS char* tq = slot(i);
    const LDS_AS char* tv = slot(i - 1);
    const LDS_AS char* pb = pbuf(i - 1);
    bf16x8_t pf[NHT];  // P fragments of the current PV step j (j = 0 first)
    bf16x8_t va[2];
    auto va_read = [&](int k) {
      const int j = k >> 2, ct = k & 3;
      const int off = 16 * j * ROW_BYTES + (ct >> 1) * 128;
      return cat_tr(tr_read(tv + pv_off[ct & 1][0] + off), tr_read(tv + pv_off[ct & 1][1] + off));
    };
    auto pv_group = [&](int k) {
      const int ct = k & 3;
      if (k + 1 < 8) va[(k + 1) & 1] = va_read(k + 1);
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        o[ct][ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[k & 1], pf[ht], o[ct][ht], 0, 0, 0);
        if (k == 3) pf[ht] = *(const LDS_AS bf16x8_t*)(pb + (2 * ht + 1) * 1024);
      }
    };
    // every operand read that does not depend on the rescale test is issued
    // before it, so its LDS latency overlaps the test's
    constexpr int QK_AHEAD = 4;
    u32x4 fa[QK_AHEAD];
    if constexpr (PV) {
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) pf[ht] = *(const LDS_AS bf16x8_t*)(pb + (2 * ht) * 1024);
    }
    if constexpr (QK) {
#pragma unroll
      for (int s = 0; s < QK_AHEAD; ++s) fa[s] = *(const LDS_AS u32x4*)(tq + qk_off[s & 3] + (s >> 2) * 128);
    }
    if constexpr (PV) va[0] = va_read(0);
    __builtin_amdgcn_sched_barrier(0);
    // sign bits set: the owner moved its reference; decode k from the raw
    // fragment, then clear the bits (always: a branch that rewrites the
    // fragments costs more registers than the 16 ANDs). With scores in the
    // step it runs after the first score MFMAs, while their results are
    // pending, instead of holding them back until the fragments arrive.
    auto p_flags = [&]() __attribute__((always_inline)) {
      u32x4 raw[NHT];
      uint32_t flag = 0;
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        raw[ht] = __builtin_bit_cast(u32x4, pf[ht]);
        flag |= (raw[ht][0] | raw[ht][1] | raw[ht][2] | raw[ht][3]) & 0x80008000u;
        u32x4 v = raw[ht];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] &= 0x7FFF7FFFu;
        pf[ht] = __builtin_bit_cast(bf16x8_t, v);
      }
      if (__ballot(flag != 0)) {
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
          int kk = 0;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            kk |= (int)((raw[ht][q] >> 15) & 1u) << (2 * q) | (int)((raw[ht][q] >> 31) & 1u) << (2 * q + 1);
          const float al = __builtin_amdgcn_ldexpf(1.f, -kk);
          if (ht == 0) rescale_fence();
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) scale_tile(o[ct][ht], al);
        }
        rescale_fence();
      }
    };
    if constexpr (PV && !QK) p_flags();
    f32x16 sc;
    if constexpr (QK) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < QK_STEPS; ++s) {
        if (s == 0) mfma_qk_first(sc, as_bf16x8(fa[0]), qf[0]);
        else mfma_qk(sc, as_bf16x8(fa[s % QK_AHEAD]), qf[s]);
        if (s == QK_STEPS - 1) mfma_qk_done(sc);
        if (s + QK_AHEAD < QK_STEPS)
          fa[s % QK_AHEAD] = *(const LDS_AS u32x4*)(tq + qk_off[(s + QK_AHEAD) & 3] + ((s + QK_AHEAD) >> 2) * 128);
        __builtin_amdgcn_sched_barrier(0);
        if (s % 4 == 1 && dma_i >= 0) {
          const int k = s / 4;
          const uint32_t off = (k & 1) ? (ld_off[k / 2] >> 16) : (ld_off[k / 2] & 0xFFFFu);
          dma16s(dma_src, off, dma_dst + k * 64 * 16);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (PV) {
          if (s == 3) {
            p_flags();
            __builtin_amdgcn_sched_barrier(0);
          }
          if (s % 9 == 8) {
            pv_group(s / 9);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      // mask rows past the context (last tile only); lane rows: 8(r/4) + 4g + r%4
      const int valid = t_end - (t_begin + i * TILE);
      if (valid < TILE) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + 4 * g + (r & 3) >= valid) sc[r] = -INFINITY;
      }
    } else if constexpr (PV) {
      // a wave without heads of its own (fewer than 128 heads) still brings
      // in its share of tile dma_i: two copies per value group, one more after
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        pv_group(k);
        if (dma_i >= 0) {
#pragma unroll
          for (int c = 2 * k; c < 2 * k + 2; ++c) {
            const uint32_t off = (c & 1) ? (ld_off[c / 2] >> 16) : (ld_off[c / 2] & 0xFFFFu);
            dma16s(dma_src, off, dma_dst + c * 64 * 16);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (dma_i >= 0) {
        constexpr int c = TILE_LOADS - 1;
        dma16s(dma_src, (c & 1) ? (ld_off[c / 2] >> 16) : (ld_off[c / 2] & 0xFFFFu), dma_dst + c * 64 * 16);
      }
    } else if (dma_i >= 0) {
      // neither product (the first step of a wave without heads): the copies only
#pragma unroll
      for (int c = 0; c < TILE_LOADS; ++c) {
        const uint32_t off = (c & 1) ? (ld_off[c / 2] >> 16) : (ld_off[c / 2] & 0xFFFFu);
        dma16s(dma_src, off, dma_dst + c * 64 * 16);
      }
    }
#pragma unroll
    for (int k = 4; k < 8; ++k) {
      if constexpr (PV) pv_group(k);
      if constexpr (QK) {
        softmax_slice(sc, 2 * (k - 4));
        softmax_slice(sc, 2 * (k - 4) + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (QK) publish(i);
  };

  using T = std::true_type;
  using F = std::false_type;
  // iteration 0: scores and softmax of tile 0. Tile 0 landed means the query
  // (requested before it) has too; the empty asm tells the compiler so, so
  // that it places no wait for the query inside the step, where the step's
  // own copies would make that wait drain them (it may wait here for tile 1)
  wait_vmcnt<TILE_LOADS>();
  if (n_tiles == 1) wait_vmcnt<0>();
#pragma unroll
  for (int s = 0; s < QK_STEPS; ++s) asm volatile("" : "+v"(qf[s]));
  lds_barrier();
  // With fewer than 128 heads (NHT < 4 head tiles of 32), waves w >= NHT own
  // no heads: they skip the scores and the softmax, and take only their value
  // columns (of the NHT real head tiles) and their copies.
  const bool qk_wave = NHT == 4 || w < NHT;
  // the copies of tile i + 2 go out during step i (spread over its score MFMAs)
  if (qk_wave) step(T{}, F{}, 0, n_tiles > 2 ? 2 : -1);
  else step(F{}, F{}, 0, n_tiles > 2 ? 2 : -1);
  for (int i = 1; i < n_tiles; ++i) {
    if (i + 1 < n_tiles) wait_vmcnt<TILE_LOADS>();  // tile i landed, tile i+1 may fly
    else wait_vmcnt<0>();
    lds_barrier();  // tile i and P of tile i-1 visible; slot (i+2)%4 and P buffer i%2 free
    if (qk_wave) step(T{}, T{}, i, i + 2 < n_tiles ? i + 2 : -1);
    else step(F{}, T{}, i, i + 2 < n_tiles ? i + 2 : -1);
  }
  clear_tail(n_tiles - 1);
  lds_barrier();
  step(F{}, T{}, n_tiles, -1);

  // ---- partials: (m, l) by the head owner, O slices by the column owner ----
  l_run += __shfl_xor(l_run, 32, 64);
  if (g == 0 && h_own < H) {
    const size_t prow = ((size_t)h_own * B + b) * splits + split;
    part_ml[prow * 2] = m_run;
    part_ml[prow * 2 + 1] = l_run;
  }
  // O rows go out through LDS, 32 heads at a time: each store instruction
  // then writes 1 KB of one head's row rather than 32-byte pieces of 32 rows.
  constexpr int OP = DC + 4;  // staged row pitch in floats (2064 bytes)
  LDS_AS float* ost = (LDS_AS float*)lds;
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    lds_barrier();  // the previous rows (or the last step's operands) are read
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = {o[ct][ht][4 * q], o[ct][ht][4 * q + 1], o[ct][ht][4 * q + 2], o[ct][ht][4 * q + 3]};
        *(LDS_AS f32x4*)(ost + hl * OP + 128 * w + 32 * ct + 8 * q + 4 * g) = v;
      }
    lds_barrier();
    // rows of 512 values as bf16: 64 lanes per row, 8 values (16 bytes) each
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int row = 4 * k + (threadIdx.x >> 6), c8 = threadIdx.x & 63, hh = h0 + 32 * ht + row;
      if (hh < H) {
        const f32x4 x = *(const LDS_AS f32x4*)(ost + row * OP + 8 * c8);
        const f32x4 y = *(const LDS_AS f32x4*)(ost + row * OP + 8 * c8 + 4);
        *(bf16x8_t*)(part_o + (((size_t)hh * B + b) * splits + split) * DC + 8 * c8) =
            (bf16x8_t){(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3],
                       (__bf16)y[0], (__bf16)y[1], (__bf16)y[2], (__bf16)y[3]};
      }
    }
  }
}

// -------------------------------------------------------- k_combine_uv ----
// One block per (head, tile of TR query rows), TR = 16, or 4 where 16 would
// leave most of the chip idle. Blocks of the same head share blockIdx % 8,
// i.e. the same XCD and L2, so W_UV,h is fetched from HBM once. Thread
// (r, q) = (tid / TPR, tid % TPR), TPR = 256 / TR, owns row b0 + r and the
// latent columns 8q + 8 TPR u .. +7. It reads (m, l) and its columns of the
// row's partials itself, SG splits at a time (4 with TR = 16, 8 with TR = 4),
// and merges them online:
//   M = max_s m_s, o_c = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s
// When no row has more than SG splits (MULTI false, the common case) that is
// one group, loaded before anything else and merged with no rescale. With
// more, each following group is requested while the one before it is merged.
// This wave's W_UV,h fragments (128 registers) are loaded only once the merge
// is done, which keeps the kernel at two waves per SIMD (holding both would
// take one block round more). Then out^T[v, b] = sum_c W_UV[h*128 + v, c]
// o_c[b, c] on MFMA from o_c staged in LDS as bf16; each lane ends with 4
// consecutive outputs of one row (one 8-byte store).
// With UV false, the W_UV product is left out and o_c itself is written, as
// out [B, H, 512] bf16, for an output projection with W_UV folded into W_O.
template <bool UV, int TR, bool MULTI>
__global__ __launch_bounds__(256) void k_combine_uv(int H, int B, int q_len, int splits,
                                                    const int32_t* __restrict__ run_pages,
                                                    const int32_t* __restrict__ ctx_lens,
                                                    const bf16* __restrict__ part_o,
                                                    const float* __restrict__ part_ml,
                                                    const bf16* __restrict__ w_uv, bf16* __restrict__ out) {
  // TR query rows per block (16, or 4 when the grid would be small), TPR
  // threads per row, each with CPT latent columns in NU loads of 8 per split
  constexpr int TPR = 256 / TR, CPT = DC / TPR, NU = CPT / 8;
  constexpr int LDO = DC + 8;
  constexpr int SG = TR == 16 ? 4 : 8;  // splits per load group
  __shared__ __attribute__((aligned(16))) bf16 oc[16 * LDO];
  const int nbt = (B + TR - 1) / TR;
  const int bid = blockIdx.x, xcd = bid & 7, k = bid >> 3;
  const int bt = k % nbt, h = (k / nbt) * 8 + xcd;
  if (h >= H) return;
  const int b0 = bt * TR;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int i16 = lane & 15, G = lane >> 4;
  const int r = tid / TPR, q = tid % TPR, b = b0 + r;
  // the row's sequence length is requested first and used only after the
  // partials' loads are out (visible_rows with its arithmetic deferred)
  const int seq = b / q_len;
  const int seq_len = b < B ? ctx_lens[seq] : 0;
  const int pps = *run_pages;  // pages per run, as the split kernel used them
  // splits that hold rows of this query row; the others were never written
  auto row_splits = [&]() __attribute__((always_inline)) {
    const int len = b < B ? seq_len - (q_len - 1 - (b - seq * q_len)) : 0;
    return len > 0 ? ((len + PAGE - 1) / PAGE + pps - 1) / pps : 0;
  };
  int ns = MULTI ? row_splits() : 0;
  const bf16* po = part_o + ((size_t)h * B + (b < B ? b : 0)) * splits * DC + 8 * q;
  const float* ml = part_ml + ((size_t)h * B + (b < B ? b : 0)) * splits * 2;
  typedef __attribute__((ext_vector_type(2))) float f32x2_t;
  // two groups of partials in registers: the next group's loads are in
  // flight while the current one is merged (with up to 16 splits, four
  // groups in turn would otherwise each wait a whole memory round trip)
  u32x4 pv0[SG][NU], pv1[SG][NU];
  f32x2_t ml0[SG], ml1[SG];
  // With one group every slot is loaded, without waiting for the context
  // length: slots past the launch's splits repeat its last split, and a split
  // past the row's context holds stale or unwritten values; both are loaded
  // but never merged.
  auto issue = [&](int s0, u32x4 (&pv)[SG][NU], f32x2_t (&mlv)[SG]) __attribute__((always_inline)) {
#pragma unroll
    for (int d = 0; d < SG; ++d) {
      int sp = s0 + d;
      if (!MULTI) sp = sp < splits ? sp : splits - 1;
      if (!MULTI || sp < ns) {
        mlv[d] = *(const f32x2_t*)(ml + 2 * sp);
#pragma unroll
        for (int u = 0; u < NU; ++u) pv[d][u] = *(const u32x4*)(po + (size_t)sp * DC + 8 * TPR * u);
      }
    }
  };
  float acc[NU][8] = {};
  float M = -INFINITY, l = 0.f;
  auto merge = [&](int s0, const u32x4 (&pv)[SG][NU], const f32x2_t (&mlv)[SG]) __attribute__((always_inline)) {
    float Mg = M;
#pragma unroll
    for (int d = 0; d < SG; ++d)
      if (s0 + d < ns) Mg = fmaxf(Mg, mlv[d][0]);
    if (Mg > M) {  // a later group raised the max: rescale what is summed so far
      const float a = __builtin_amdgcn_exp2f(M - Mg);
      l *= a;
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[u][x] *= a;
      M = Mg;
    }
#pragma unroll
    for (int d = 0; d < SG; ++d) {
      if (s0 + d < ns) {
        const float e = __builtin_amdgcn_exp2f(mlv[d][0] - M);
        l += e * mlv[d][1];
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            acc[u][2 * x] += e * __uint_as_float(pv[d][u][x] << 16);
            acc[u][2 * x + 1] += e * __uint_as_float(pv[d][u][x] & 0xFFFF0000u);
          }
      }
    }
  };
  issue(0, pv0, ml0);
  // W_UV,h fragments of this wave (rows 32w .. 32w+31, all 512 columns)
  u32x4 wf[DC / 32][2];
  auto load_wuv = [&]() __attribute__((always_inline)) {
    const bf16* wv = w_uv + (size_t)h * DV * DC;
#pragma unroll
    for (int ks = 0; ks < DC / 32; ++ks)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        wf[ks][mt] = *(const u32x4*)(wv + (size_t)(32 * w + 16 * mt + i16) * DC + 32 * ks + 8 * G);
  };
  // with one group they go out right behind the partials, and the context
  // length is needed only for the merge; so they do with 4-row tiles (used
  // only where the grid is small, so registers do not limit the waves that
  // run at once)
  constexpr bool EARLY_WUV = UV && (!MULTI || TR == 4);
  if constexpr (EARLY_WUV) load_wuv();
  if constexpr (!MULTI) {
    __builtin_amdgcn_sched_barrier(0);
    ns = row_splits();
  }
  if constexpr (!MULTI) {
    merge(0, pv0, ml0);  // every row has at most SG splits
  } else {
    for (int s0 = 0; s0 < ns; s0 += 2 * SG) {
      if (s0 + SG < ns) issue(s0 + SG, pv1, ml1);
      merge(s0, pv0, ml0);
      if (s0 + SG >= ns) break;
      if (s0 + 2 * SG < ns) issue(s0 + 2 * SG, pv0, ml0);
      merge(s0 + SG, pv1, ml1);
    }
  }
  // with several groups, once they are merged (their loads fly while o_c is
  // staged)
  if constexpr (UV && !EARLY_WUV) load_wuv();
  const float il = ns > 0 ? 1.f / l : 0.f;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    bf16x8_t v;
#pragma unroll
    for (int x = 0; x < 8; ++x) v[x] = (__bf16)(acc[u][x] * il);
    *(bf16x8_t*)&oc[r * LDO + 8 * q + 8 * TPR * u] = v;
  }
  __syncthreads();
  if constexpr (!UV) {
    // o_c rows of the block's query rows: TPR threads per row, CPT columns each
    if (b < B) {
      bf16* dst = out + ((size_t)b * H + h) * DC + CPT * q;
#pragma unroll
      for (int u = 0; u < NU; ++u) *(u32x4*)(dst + 8 * u) = *(const u32x4*)&oc[r * LDO + CPT * q + 8 * u];
    }
    return;
  }
  // wave w: outputs v = 32w .. 32w+31 (two 16-row tiles), the block's query
  // rows as the 16 MFMA columns (with TR = 4, columns 4-15 are left over and
  // not stored)
  f32x4 oacc[2] = {};
#pragma unroll
  for (int ks = 0; ks < DC / 32; ++ks) {
    const bf16x8_t bo = as_bf16x8(*(const u32x4*)&oc[i16 * LDO + 32 * ks + 8 * G]);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      oacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wf[ks][mt]), bo, oacc[mt], 0, 0, 0);
  }
  const int bo_seq = b0 + i16;
  if (i16 < TR && bo_seq < B) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
      const bf16x4_t v = {(__bf16)oacc[mt][0], (__bf16)oacc[mt][1], (__bf16)oacc[mt][2], (__bf16)oacc[mt][3]};
      *(bf16x4_t*)(out + ((size_t)bo_seq * H + h) * DV + 32 * w + 16 * mt + 4 * G) = v;
    }
  }
}

}  // namespace

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

bool decode_fast_supported(const mla_dims& d, const CacheView& c) {
  return d.dtype == MLA_BF16 && d.d_c == DC && d.d_rope == DR && d.d_nope == DN && d.d_v == DV &&
         d.n_heads <= 2 * MAX_HEADS && c.paged &&
         c.block_size == PAGE;
}

void decode_plan(int rows, int max_context, int q_len, int* pages_per_split, int* splits) {
  const Plan p = plan_splits(rows, max_context, q_len);
  *pages_per_split = p.pages_per_split;
  *splits = p.splits;
}

hipError_t decode_absorb(const mla_dims& d, float scale, int rows, int q_len, const void* q_nope, const void* q_pe,
                         const void* w_uk, const int32_t* ctx_lens, void* qt, const char* prof_name, hipStream_t s) {
  ProfScope ps(prof_name, s);
  RopeFreq rope;
  for (int i = 0; i < DR / 2; ++i) rope.theta[i] = pow((double)d.rope_base, -2.0 * i / (double)DR);
  // narrower column blocks with fewer heads, so the grid stays near one block
  // per compute unit
  const int H = d.n_heads;
  auto go = [&](auto kern, int cw) {
    hipLaunchKernelGGL(kern, dim3(H, DC / cw), dim3(256), 0, s, rows, H, q_len, (const bf16*)q_nope,
                       (const bf16*)q_pe, (const bf16*)w_uk, ctx_lens, scale * LOG2E, rope, (bf16*)qt);
  };
  if (H >= 64) go(k_absorb<128>, 128);
  else if (H >= 32) go(k_absorb<64>, 64);
  else go(k_absorb<32>, 32);
  return hipGetLastError();
}

hipError_t decode_combine(const mla_dims& d, int rows, int q_len, int splits, const int32_t* run_pages,
                          const int32_t* ctx_lens,
                          const void* part_o, const float* part_ml, const void* w_uv, void* out,
                          const char* prof_name, hipStream_t s) {
  const int H = d.n_heads;
  const int hpad = (H + 7) / 8 * 8;
  // 16 query rows per block, or 4 where that would leave most of the chip idle
  // (few heads and rows: the blocks then each stream fewer partials)
  const bool small = hpad * ((rows + 15) / 16) < 128;
  const int nbt = small ? (rows + 3) / 4 : (rows + 15) / 16;
  ProfScope ps(prof_name, s);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(hpad * nbt), dim3(256), 0, s, H, rows, q_len, splits, run_pages, ctx_lens,
                       (const bf16*)part_o, part_ml, (const bf16*)w_uv, (bf16*)out);
  };
  // one group of splits per row (the common case) or several
  const bool multi = splits > (small ? 8 : 4);
  if (w_uv) {
    if (small) multi ? go(k_combine_uv<true, 4, true>) : go(k_combine_uv<true, 4, false>);
    else multi ? go(k_combine_uv<true, 16, true>) : go(k_combine_uv<true, 16, false>);
  } else {
    if (small) multi ? go(k_combine_uv<false, 4, true>) : go(k_combine_uv<false, 4, false>);
    else multi ? go(k_combine_uv<false, 16, true>) : go(k_combine_uv<false, 16, false>);
  }
  return hipGetLastError();
}

bool decode_fast_context_ok(int max_context) {
  // a run's page numbers are held one per lane of a wave
  return plan_splits(1, max_context, 1).pages_per_split <= 64;
}

size_t decode_fast_workspace(const mla_dims& d, int batch, int q_len, int max_context) {
  const Plan p = plan_splits(batch * q_len, max_context, q_len);
  return ws_layout(d.n_heads, batch * q_len, p.splits).total;
}

// w_uv == nullptr: out receives the latent output o_c [rows, H, 512] instead
hipError_t decode_fast(const mla_dims& d, float scale, int n_seq, int q_len, int max_context, const void* q_nope,
                       const void* q_pe, const void* w_uk, const void* w_uv, const CacheView& c, void* out,
                       void* ws, size_t ws_bytes, hipStream_t s) {
  const int H = d.n_heads;
  const int batch = n_seq * q_len;  // query rows
  const Plan p = plan_splits(batch, max_context, q_len);
  const WsLayout l = ws_layout(H, batch, p.splits);
  if (ws_bytes < l.total) return hipErrorInvalidValue;
  char* base = (char*)ws;
  bf16* qt = (bf16*)(base + l.qt);
  bf16* part_o = (bf16*)(base + l.part_o);
  float* part_ml = (float*)(base + l.part_ml);
  int32_t* run = (int32_t*)(base + l.run);

  hipError_t e = decode_absorb(d, scale, batch, q_len, q_nope, q_pe, w_uk, c.context_lens, qt, "mla_decode_absorb", s);
  if (e != hipSuccess) return e;
  const dim3 grid(p.splits, batch, (H + MAX_HEADS - 1) / MAX_HEADS);
  {
    ProfScope ps("mla_decode_split", s);
    const bool pair_xcd = q_len > 1 && ((int64_t)n_seq * p.splits) % 8 == 0;
    const int order = pair_xcd ? 1 : (q_len == 1 && batch <= 256 ? 2 : 0);
    // head tiles of 32 with real heads: 1 or 2 for small head counts, else 4
    const int nht = H <= 32 ? 1 : (H <= 64 ? 2 : 4);
    // workgroups of one round per head group (one split workgroup per CU)
    const int budget = max(1, device_cus() / (int)grid.z);
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, dim3(SPLIT_THREADS), 0, s, H, batch, q_len, order, p.splits,
                         p.pages_per_split, budget, run, qt, (const bf16*)c.rows, c.block_table, c.max_blocks,
                         c.context_lens, part_o, part_ml);
    };
    if (nht == 1) go(k_split<1>);
    else if (nht == 2) go(k_split<2>);
    else go(k_split<4>);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return decode_combine(d, batch, q_len, p.splits, run, c.context_lens, part_o, part_ml, w_uv, out,
                        "mla_decode_combine_uv", s);
}

}  // namespace mla
