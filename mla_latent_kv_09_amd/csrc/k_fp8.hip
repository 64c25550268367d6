// FP8 latent cache: the cache quantised to FP8 with one power-of-two scale
// per token ("DeepSeek core techniques: MoE and MLA attention" §6.3: the KV
// cache is quantised to FP8 dynamically for deployment; "8.1 DeepSeek
// architecture" §5: a scale per block rather than one global scale).
//
// Format. E4M3 (OCP "fn", largest value 448). A page of P tokens holds P rows
// of [d_c codes of c_KV || d_rope bf16 values of k_pe], then P scale bytes E
// (scale 2^(E - 127)), then zero padding to 16 bytes. A token's scale is the
// smallest 2^e, e >= -127, with max|c_KV| <= 448 * 2^e; its codes are
// RNE(c_KV / 2^e). For the DeepSeek-V3 shape a row is 640 bytes and a 64-token
// page 41,024 bytes (0.56 of the bf16 page).
//
//   k_quant_fp8   bf16 rows -> FP8 rows at cache slots, one wave per row.
//   k_split8      decode over FP8 pages (one workgroup per query row and run
//                 of pages, as in the bf16 decode). Scores run on the
//                 MX-scaled FP8 MFMA (32x32x64): the token's scale and the
//                 query head's scale are applied by the matrix core. P goes to
//                 FP8 with the token's scale folded in, relative to the largest
//                 token scale of the page, and the latent output uses the same
//                 MFMA with that page scale.
// The query q~ is quantised the same way (one scale per query row and head),
// by the split kernel itself as it loads q~, with k_pe's slice of it left in
// bf16.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(2))) int i32x2;

constexpr int DC = 512, DR = 64, PAGE = 64;
constexpr int ROW8 = DC + 2 * DR;           // 640 bytes: codes || k_pe
constexpr int ROW8_CHUNKS = ROW8 / 16;      // 40
constexpr int SCALE_OFF = PAGE * ROW8;      // 40960: the page's scale bytes
constexpr int PAGE8 = SCALE_OFF + PAGE;     // 41024
constexpr int PAGE8_CHUNKS = PAGE8 / 16;    // 2564
constexpr int THREADS = 256;
constexpr int COPIES = (PAGE8_CHUNKS + THREADS - 1) / THREADS;  // 11; the last covers 4 chunks
constexpr int N_SLOTS = 3;
constexpr int MAX_HEADS = 128;
constexpr int PB_BYTES = MAX_HEADS * PAGE;  // P of one page, fp8: [head][64 tokens]
constexpr int KB_BYTES = MAX_HEADS;        // reference shift per head, [head % 32][head / 32]
constexpr int SPLIT8_LDS = N_SLOTS * PAGE8 + 2 * PB_BYTES + 2 * KB_BYTES;
static_assert(SPLIT8_LDS <= 160 * 1024, "LDS budget of one workgroup");
constexpr int MAX_SPLITS = 256;

size_t page_bytes_of(int page, int d_c, int d_rope) {
  const size_t raw = (size_t)page * (d_c + 2 * d_rope) + page;
  return (raw + 15) / 16 * 16;
}

// --------------------------------------------------------- k_quant_fp8 ----
// Block of 4 waves; wave w quantises row 4 * blockIdx.x + w of src
// [n, d_c + d_rope] (bf16) into cache slot slots[r] (r when slots is NULL).
__global__ __launch_bounds__(256) void k_quant_fp8(int n, int d_c, int d_rope, const bf16* __restrict__ src,
                                                   const int32_t* __restrict__ slots, int page, int page_bytes,
                                                   uint8_t* __restrict__ dst) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= n) return;
  const int slot = slots ? slots[r] : r;
  const bf16* x = src + (size_t)r * (d_c + d_rope);
  uint8_t* pg = dst + (size_t)(slot / page) * page_bytes;
  const int off = slot % page;
  const int row_bytes = d_c + 2 * d_rope;
  uint8_t* row = pg + (size_t)off * row_bytes;
  // largest magnitude, as bf16 bits (their order is that of the magnitudes)
  uint32_t mb = 0;
  for (int j = lane; j < d_c / 8; j += 64) {
    const u32x4 v = *(const u32x4*)(x + 8 * j);
#pragma unroll
    for (int q = 0; q < 4; ++q) mb = max(mb, max(v[q] & 0x7FFFu, (v[q] >> 16) & 0x7FFFu));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mb = max(mb, (uint32_t)__shfl_xor((int)mb, o, 64));
  // smallest e >= -127 with amax <= 448 * 2^e: amax * 2^-(k - 8) lies in
  // [256, 512) for amax in [2^k, 2^(k+1)); above 448 the next exponent
  const uint32_t fb = mb << 16;
  const int field = (int)(fb >> 23);
  int e = -127;
  if (field != 0) {
    e = field - 127 - 8;
    if (__builtin_amdgcn_ldexpf(__uint_as_float(fb), -e) > 448.f) ++e;
    e = max(e, -127);
  }
  for (int j = lane; j < d_c / 8; j += 64) {
    const u32x4 v = *(const u32x4*)(x + 8 * j);
    float f[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f[2 * q] = __builtin_amdgcn_ldexpf(__uint_as_float(v[q] << 16), -e);
      f[2 * q + 1] = __builtin_amdgcn_ldexpf(__uint_as_float(v[q] & 0xFFFF0000u), -e);
    }
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
    *(i32x2*)(row + 8 * j) = (i32x2){lo, hi};
  }
  for (int j = lane; j < d_rope / 4; j += 64) *(i32x2*)(row + d_c + 8 * j) = *(const i32x2*)(x + d_c + 4 * j);
  if (lane == 0) pg[(size_t)page * row_bytes + off] = (uint8_t)(e + 127);
}

// ------------------------------------------------------------ k_split8 ----
// As the bf16 split kernel: grid (splits, rows), 4 waves, one workgroup per
// (query row, run of pages); query row b is token b % q_len of sequence
// b / q_len. The run is walked a page (tile) at a time.
//
//   scores   wave w owns heads 32w .. 32w+31. For each half page (32 rows):
//            S^T[t, h] = sum over 8 MX-scaled FP8 MFMAs (K = 64) of the codes,
//            with scale_a = the token's scale byte and scale_b = the head's,
//            plus 4 bf16 MFMAs over k_pe. The query's codes (64 VGPRs), its
//            bf16 k_pe slice (16) and scale byte stay in registers.
//   softmax  log2 domain, reference max per head moved lazily by whole steps
//            k (as in the bf16 kernel); the owner publishes k beside P, and
//            the other waves rescale that head's columns by 2^-k (rare).
//            P' = P * 2^(E_t - E_page) with E_page the largest scale of the
//            page's valid tokens, rounded to FP8.
//   values   wave w owns latent columns 128w .. 128w+127 of every head:
//            O^T[c, h] += sum_t code[t, c] P'[t, h] * 2^(E_page - 127), one
//            MX-scaled MFMA (K = 64 tokens) per (column tile, head tile). The
//            value operand is read transposed from the row-major page with
//            ds_read_b64_tr_b8.
// Pipeline: a ring of three page slots (page i - 1 in the value step, page i
// in the score step, page i + 1 in flight) and two P (and shift) buffers; one
// barrier per page. Partials are those of the bf16 kernel, merged by the same
// combine.
//
// LDS layout of a page: row t at t * 640, its 16-byte chunk j at position
// j ^ sw(t) inside its aligned group of 8 (rows 0..15 reading one chunk then
// hit 16 distinct bank groups); the 64 scale bytes at 40960, as in HBM.
__device__ __forceinline__ int sw(int t) { return (t >> 1) & 7; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One 16-byte HBM -> LDS copy per active lane, to lds_addr + 16 * lane (see
// the bf16 decode kernel: issued from asm so the compiler does not order
// every later LDS read behind it; ordered with explicit vmcnt waits).
__device__ __forceinline__ void dma16s(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds_addr)
               : "memory", "m0");
}

// x[0..7] *= a for accumulators held in AGPRs, written out so that the
// compiler keeps the 256 value accumulators in AGPRs (a plain multiply makes
// it move them through VGPRs). The caller pads the wait states around it
// (rescale_fence), once per rescale.
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
__device__ __forceinline__ void rescale_fence() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" ::: "memory"); }
__device__ __forceinline__ void scale_tile(f32x16& v, float a) {
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = v[r];
  scale_acc8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7], a);
  scale_acc8(x[8], x[9], x[10], x[11], x[12], x[13], x[14], x[15], a);
#pragma unroll
  for (int r = 0; r < 16; ++r) v[r] = x[r];
}

__device__ __forceinline__ i32x8 cat8(u32x4 a, u32x4 b) {
  return (i32x8){(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}
__device__ __forceinline__ i32x2 tr8(const LDS_AS char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2*)p);
}
__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}
// Score MFMAs with their accumulators in VGPRs, written out so the compiler
// does not place them in AGPRs (which all hold the value accumulators).
// Chained MFMAs on one accumulator need no wait states; score_done() pads the
// wait states a vector instruction needs before it reads the result.
__device__ __forceinline__ void qk8(f32x16& acc, i32x8 a, i32x8 b, int sa, int sb) {
  asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
               : "+v"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
}
__device__ __forceinline__ void qk16_first(f32x16& acc, bf16x8_t a, bf16x8_t b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk16(f32x16& acc, bf16x8_t a, bf16x8_t b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void score_done(f32x16& x) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x));
}
// between the bf16 chain and the FP8 chain on one accumulator (different
// MFMA kinds chain only after the first one's result is written)
__device__ __forceinline__ void mfma_switch(f32x16& x) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x)); }

// The lane index, computed in asm that the compiler cannot merge with an
// earlier computation of it: code after the page loop that takes it from here
// keeps nothing of the prologue live across the loop (the loop needs every
// register, and a value held over it is spilled to scratch).
__device__ __forceinline__ int opaque_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

__global__ __launch_bounds__(THREADS, 1) void k_split8(int H, int B, int q_len, int order, int splits, int pps,
                                                       int budget, int32_t* __restrict__ run_out,
                                                       const bf16* __restrict__ qt,
                                                       const uint8_t* __restrict__ pages,
                                                       const int32_t* __restrict__ block_table, int max_blocks,
                                                       const int32_t* __restrict__ ctx_lens,
                                                       bf16* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ __attribute__((aligned(1024))) char lds[SPLIT8_LDS];
  // block order: 0 plain, 1 rows of one sequence paired on an XCD, 2 longest
  // runs first (one new token per row) with the run length that fits one
  // round, as in the bf16 kernel (the first block records it for the combine)
  int split = blockIdx.x, b = blockIdx.y, len_b = 0;
  int lens[4] = {0, 0, 0, 0};
  if (order == 2) load_row_lens(B, ctx_lens, lens);
  // (only when the launch's slots, splits x B, exceed one round: otherwise
  // the runs of pps fit whatever the lengths)
  const int pps_run = order == 2 && splits * B > budget ? one_round_run_pages(pps, 64, budget, PAGE, lens) : pps;
  if ((blockIdx.x | blockIdx.y) == 0 && threadIdx.x == 0) *run_out = pps_run;
  if (order == 2) {
    if (!longest_run_first(B, pps_run * PAGE, lens, blockIdx.y * gridDim.x + blockIdx.x, b, split, len_b))
      return;
  } else if (order == 1) {
    // the q_len rows of one (sequence, split) on consecutive slots of one XCD
    const int lin = blockIdx.y * gridDim.x + blockIdx.x, local = lin >> 3;
    const int unit_local = local / q_len, j = local - unit_local * q_len;
    const int unit = unit_local * 8 + (lin & 7), seq = unit / splits;
    split = unit - seq * splits;
    b = seq * q_len + j;
  }
  // the block's row and split are the same in every lane: keep them (and
  // what derives from them) in scalar registers
  b = __builtin_amdgcn_readfirstlane(b);
  split = __builtin_amdgcn_readfirstlane(split);
  len_b = __builtin_amdgcn_readfirstlane(len_b);
  const int seq = b / q_len;
  const int L = order == 2 ? len_b : ctx_lens[seq] - (q_len - 1 - (b - seq * q_len));
  const int t_begin = split * pps_run * PAGE;
  const int t_end = min(t_begin + pps_run * PAGE, L);
  if (t_begin >= t_end) return;
  const int n_tiles = (t_end - t_begin + PAGE - 1) / PAGE;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hl = lane & 31, g = lane >> 5;
  const int h_own = w * 32 + hl;
  const int32_t* table = block_table + (size_t)seq * max_blocks;

  // copy k of this lane: LDS chunk pos = 256k + 64w + lane; its global chunk
  // (rows swizzled, scale bytes as they are); two 16-bit offsets per register
  uint32_t ld_off[(COPIES + 1) / 2];
#pragma unroll
  for (int k = 0; k < COPIES; ++k) {
    const int pos = k * THREADS + w * 64 + lane;
    uint32_t off;
    if (pos < PAGE * ROW8_CHUNKS) {
      const int t = pos / ROW8_CHUNKS, p = pos - t * ROW8_CHUNKS;
      off = (uint32_t)(t * ROW8 + ((p ^ sw(t)) << 4));
    } else {
      off = (uint32_t)(min(pos, PAGE8_CHUNKS - 1) << 4);  // scale bytes; lanes past them copy nothing
    }
    if (k & 1) ld_off[k / 2] |= off << 16;
    else ld_off[k / 2] = off;
  }
  const int run_pages = (t_end - t_begin + PAGE - 1) / PAGE;
  const int page_of_lane = lane < run_pages ? table[t_begin / PAGE + lane] : 0;
  const uint32_t lds_base = (uint32_t)(size_t)(LDS_AS char*)lds;
  // source page and destination slot of the copies of page i (uniform)
  auto copy_src = [&](int i) {
    return (const char*)(pages + (size_t)__builtin_amdgcn_readlane(page_of_lane, i) * PAGE8);
  };
  auto copy_dst = [&](int i) {
    return (uint32_t)__builtin_amdgcn_readfirstlane(lds_base + (i % N_SLOTS) * PAGE8 + w * 64 * 16);
  };
  auto copy_one = [&](const char* src, uint32_t dst, int k) {
    // unpacked at each use (the empty asm keeps the compiler from hoisting
    // eleven unpacked offsets out of the page loop)
    uint32_t word = ld_off[k / 2];
    asm volatile("" : "+v"(word));
    const uint32_t off = (k & 1) ? (word >> 16) : (word & 0xFFFFu);
    if (k < COPIES - 1) {
      dma16s(src, off, dst + k * THREADS * 16);
    } else if (w == 0) {
      if (lane < PAGE8_CHUNKS - (COPIES - 1) * THREADS) dma16s(src, off, dst + k * THREADS * 16);
    }
  };

  // query of this lane's head (rows of heads >= H read head H - 1; nothing
  // of theirs is stored), read in bf16 and quantised here by the cache's
  // rule (k_quant_fp8, the same operations): one power-of-two scale per
  // (query row, head), the smallest 2^e with max|q~| <= 448 * 2^e, and codes
  // RNE(q~ / 2^e). The lane holds latent columns 64 ks + 32 g .. +31 (its K
  // step ks, as codes) and k_pe values 16 s + 8 g .. +7 (bf16).
  const int hq = min(h_own, H - 1);
  const bf16* qrow = qt + ((size_t)b * H + hq) * (DC + DR);
  u32x4 qb[8][4];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
#pragma unroll
    for (int u = 0; u < 4; ++u) qb[ks][u] = *(const u32x4*)(qrow + 64 * ks + 32 * g + 8 * u);
  bf16x8_t qp[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) qp[s] = __builtin_bit_cast(bf16x8_t, *(const u32x4*)(qrow + DC + 16 * s + 8 * g));
  int e_q;
  i32x8 qf[8];
  {
    // largest magnitude as bf16 bits (ordered as the magnitudes), over both
    // halves of the head's columns (the other half is 32 lanes away)
    uint32_t mb = 0;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) mb = max(mb, max(qb[ks][u][q] & 0x7FFFu, (qb[ks][u][q] >> 16) & 0x7FFFu));
    mb = max(mb, (uint32_t)__shfl_xor((int)mb, 32, 64));
    const uint32_t fb = mb << 16;
    const int field = (int)(fb >> 23);
    int e = -127;
    if (field != 0) {
      e = field - 127 - 8;
      if (__builtin_amdgcn_ldexpf(__uint_as_float(fb), -e) > 448.f) ++e;
      e = max(e, -127);
    }
    e_q = e + 127;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const u32x4 v = qb[ks][u];
        float f[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f[2 * q] = __builtin_amdgcn_ldexpf(__uint_as_float(v[q] << 16), -e);
          f[2 * q + 1] = __builtin_amdgcn_ldexpf(__uint_as_float(v[q] & 0xFFFF0000u), -e);
        }
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
        int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
        qf[ks][2 * u] = lo;
        qf[ks][2 * u + 1] = hi;
      }
  }
  wait_vmcnt<0>();
  {
    const char* src0 = copy_src(0);
    const uint32_t dst0 = copy_dst(0);
#pragma unroll
    for (int k = 0; k < COPIES; ++k) copy_one(src0, dst0, k);
  }

  f32x16 o[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) o[i][j] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;
  int e_prev = 127;  // page scale of the page in the value step

  // LDS byte offsets of this lane's accesses (lane part; the rest is an
  // immediate or a uniform base):
  //  score codes, half page rb, K step ks, 16-byte half hh: row 32rb + hl,
  //    chunk 4ks + 2g + hh = o_qa[2(ks & 1) + hh] + 128 (ks >> 1) + 20480 rb
  //  score k_pe, step s: chunk 32 + 2s + g = o_pe[s] + 20480 rb
  //  values, column tile ct, read q: rows 32(G>>1) + 8q + (i>>1), chunk
  //    8w + 2ct + (G&1), byte 8(i&1) (G = lane / 16, i = lane % 16; the
  //    transposing read hands lane i of a group column i of 8 rows)
  //    = o_tv + o_tx[ct] ^ 64 (q & 1) + 5120 q
  //  P read (value step), head 32ht + hl, tokens 32g .. +31: o_pr[hh] + 2048 ht
  //  P write (score step), head h_own, tokens 32rb + 8a + 4g .. +3:
  //    o_pw[2rb + (a >> 1)] + 8 (a & 1)
  //  scale bytes: hl + 32 rb (score operand), 4g + 32rb + 8a (this lane's tokens)
  // They are made opaque at each step, so the compiler forms the addresses
  // there instead of keeping one register per address across the page loop.
  uint32_t o_qa[4], o_pe[4], o_tv, o_tx[4], o_pr[2], o_pw[4];
  {
    const int x = sw(hl);
#pragma unroll
    for (int u = 0; u < 4; ++u) o_qa[u] = hl * ROW8 + (((4 * (u >> 1) + 2 * g + (u & 1)) ^ x) << 4);
#pragma unroll
    for (int s = 0; s < 4; ++s) o_pe[s] = hl * ROW8 + DC + (((2 * s + g) ^ x) << 4);
    const int G = lane >> 4, i = lane & 15;
    o_tv = (32 * (G >> 1) + (i >> 1)) * ROW8 + 128 * w + 8 * (i & 1);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) o_tx[ct] = ((2 * ct + (G & 1)) ^ (i >> 2)) << 4;
    const int xp = (hl >> 2) & 3;  // P row swizzle of heads 32ht + hl (and of h_own)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) o_pr[hh] = hl * PAGE + (((2 * g + hh) ^ xp) << 4);
#pragma unroll
    for (int c = 0; c < 4; ++c) o_pw[c] = h_own * PAGE + ((c ^ xp) << 4) + 4 * g;
  }
  auto opq = [](uint32_t& v) { asm volatile("" : "+v"(v)); };
  auto slot_addr = [&](int i) { return (uint32_t)(lds_base + ((i + N_SLOTS) % N_SLOTS) * PAGE8); };
  auto pb_addr = [&](int i) { return (uint32_t)(lds_base + N_SLOTS * PAGE8 + (i & 1) * PB_BYTES); };
  auto kb_addr = [&](int i) { return (uint32_t)(lds_base + N_SLOTS * PAGE8 + 2 * PB_BYTES + (i & 1) * KB_BYTES); };
  auto r128 = [](uint32_t a) { return *(const LDS_AS u32x4*)(size_t)a; };

  // rows past the context in the last page: zero their codes before the
  // value step (0 * NaN would be NaN); each lane clears the chunks its own
  // copies brought in
  auto clear_tail = [&](int i) {
    const int valid = t_end - (t_begin + i * PAGE);
    if (valid >= PAGE) return;
    LDS_AS char* base = (LDS_AS char*)(size_t)slot_addr(i);
    const int first = w * 64 + opaque_lane();
#pragma unroll
    for (int k = 0; k < COPIES - 1; ++k) {
      const int pos = k * THREADS + first;
      const int t = pos / ROW8_CHUNKS;
      if (t >= valid && t < PAGE) *(LDS_AS u32x4*)(base + pos * 16) = (u32x4){0, 0, 0, 0};
    }
  };

  int e_page = 127;  // of the page in the score step

  // ---- one pipeline step. Scores of page i (24 MFMAs, their operands read
  // two ahead, the copies of page dma_i after every second), then the
  // softmax of page i. The value product of page i - 1 (16 MFMAs) is spread
  // over both: one after every third score MFMA and one per softmax group, so
  // that the score operands' LDS reads (40 KB per wave and page) overlap
  // MFMAs that read little. ----
  auto step = [&](auto do_qk, auto do_pv, int i, int dma_i) {
    constexpr bool QK = decltype(do_qk)::value, PV = decltype(do_pv)::value;
    const uint32_t tq = slot_addr(i), tv = slot_addr(i - 1);
    // the reference shifts of heads 32ht + hl (ht = byte), published with P
    // of page i - 1 by the heads' owners (read first: it alone gates the
    // rescale test), then the P fragments: head 32ht + hl, tokens 32g .. +31
    uint32_t kword = 0;
    if constexpr (PV) kword = *(const LDS_AS uint32_t*)(size_t)(kb_addr(i - 1) + 4 * hl);
    i32x8 pf[4];
    if constexpr (PV) {
      const uint32_t pb = pb_addr(i - 1);
      uint32_t a_pr0 = pb + o_pr[0], a_pr1 = pb + o_pr[1];
      opq(a_pr0);
      opq(a_pr1);
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) pf[ht] = cat8(r128(a_pr0 + 2048 * ht), r128(a_pr1 + 2048 * ht));
    }
    f32x16 sc[2];
    int e_t[2] = {0, 0}, ep = 0;
    uint32_t ew[8];  // scale bytes of this lane's tokens 32rb + 8a + 4g .. +3, as [4rb + a]
    constexpr int AHEAD = 2;
    u32x4 fa[AHEAD][2];
    // score operand op: half page rb = op / 12; k = op % 12 < 4: k_pe step k
    // (bf16, 16 bytes), else code step k - 4 (FP8, 32 bytes)
    // lane bases of this step's accesses, formed once (opaque to the
    // compiler, so it neither re-forms them per access nor keeps one register
    // per access across the page loop); the rest of each address is an
    // instruction immediate
    uint32_t b_qa[4], b_pe[4];
    if constexpr (QK) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        b_qa[u] = tq + o_qa[u];
        opq(b_qa[u]);
        b_pe[u] = tq + o_pe[u];
        opq(b_pe[u]);
      }
    }
    auto a_read = [&](int op, u32x4 (&f)[2]) {
      const int rb = op / 12, k = op % 12;
      if (k < 4) {
        f[0] = r128(b_pe[k] + rb * 32 * ROW8);
      } else {
        const int ks = k - 4;
        const uint32_t imm = rb * 32 * ROW8 + (ks >> 1) * 128;
        f[0] = r128(b_qa[2 * (ks & 1)] + imm);
        f[1] = r128(b_qa[2 * (ks & 1) + 1] + imm);
      }
    };
    if constexpr (QK) {
      // scale bytes, read ahead of their use: the score rows', this lane's
      // tokens', and one per lane for the page scale
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) e_t[rb] = (int)*(const LDS_AS uint8_t*)(size_t)(tq + SCALE_OFF + 32 * rb + hl);
      ep = (int)*(const LDS_AS uint8_t*)(size_t)(tq + SCALE_OFF + lane);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        ew[k] = *(const LDS_AS uint32_t*)(size_t)(tq + SCALE_OFF + 4 * g + 32 * (k >> 2) + 8 * (k & 3));
#pragma unroll
      for (int op = 0; op < AHEAD; ++op) a_read(op, fa[op]);
    }
    // value operand of column tile ct: four transposing reads of 8 rows each
    uint32_t b_tv[4][2];  // [column tile][read parity]
    if constexpr (PV) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        b_tv[ct][0] = tv + o_tv + o_tx[ct];
        b_tv[ct][1] = tv + o_tv + (o_tx[ct] ^ 64);
        opq(b_tv[ct][0]);
        opq(b_tv[ct][1]);
      }
    }
    auto va_read = [&](int ct) {
      i32x2 r[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) r[q] = tr8((const LDS_AS char*)(size_t)(b_tv[ct][q & 1] + q * 8 * ROW8));
      return (i32x8){r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
    };
    i32x8 va[2];
    if constexpr (PV) va[0] = va_read(0);
    // a head's owner moved its reference by k: rescale that head's columns
    // by 2^-k (rare)
    auto p_flags = [&]() {
      if (__ballot(kword != 0)) {
        rescale_fence();
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) {
          const float al = __builtin_amdgcn_ldexpf(1.f, -(int)((kword >> (8 * ht)) & 0xFFu));
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) scale_tile(o[ct][ht], al);
        }
        rescale_fence();
      }
    };
    // value MFMA m of 16: column tile m / 4, head tile m % 4; the next column
    // tile's operand is read when a tile starts
    auto pv_mfma = [&](int m) {
      const int ct = m >> 2, ht = m & 3;
      if (ht == 0 && ct + 1 < 4) va[(ct + 1) & 1] = va_read(ct + 1);
      o[ct][ht] = mfma8(va[ct & 1], pf[ht], o[ct][ht], 127, e_prev);
    };
    if constexpr (PV && QK) p_flags();
    if constexpr (QK) {
      const bool dma = dma_i >= 0;
      const char* dsrc = dma ? copy_src(dma_i) : nullptr;
      const uint32_t ddst = dma ? copy_dst(dma_i) : 0u;
#pragma unroll
      for (int op = 0; op < 24; ++op) {
        const int rb = op / 12, k = op % 12;
        const u32x4 f0 = fa[op % AHEAD][0], f1 = fa[op % AHEAD][1];
        if (op + AHEAD < 24) a_read(op + AHEAD, fa[op % AHEAD]);
        if (k < 4) {
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, f0);
          if (k == 0) qk16_first(sc[rb], a, qp[k]);
          else qk16(sc[rb], a, qp[k]);
          if (k == 3) mfma_switch(sc[rb]);
        } else {
          qk8(sc[rb], cat8(f0, f1), qf[k - 4], e_t[rb], e_q);
        }
        // copies: after ops 1, 3, 5, ... (11 of them)
        if ((op & 1) && dma && (op >> 1) < COPIES) copy_one(dsrc, ddst, op >> 1);
        if constexpr (PV) {
          if (op % 3 == 2) pv_mfma(op / 3);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // ---- softmax of page i, head h_own: tile max, reference, shift ----
    float alpha = 1.f, lsum2[2] = {0.f, 0.f};
    uint32_t pw = 0;
    if constexpr (QK) {
      score_done(sc[1]);
      // mask rows past the context; lane rows of half page rb: 32rb + 8(r/4) + 4g + r%4
      const int valid = t_end - (t_begin + i * PAGE);
      if (valid < PAGE) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * rb + 8 * (r >> 2) + 4 * g + (r & 3) >= valid) sc[rb][r] = -INFINITY;
      }
      // page scale: the largest scale byte of the valid tokens
      // (bit by bit from the top, one ballot per bit: no lane shuffles)
      {
        if (lane >= valid) ep = 0;
        int m = 0;
#pragma unroll
        for (int bit = 7; bit >= 0; --bit)
          if (__ballot(ep >= (m | (1 << bit)))) m |= 1 << bit;
        e_page = __builtin_amdgcn_readfirstlane(m);
      }
      float mx = sc[0][0];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[rb][r]);
      {
        const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
      }
      // a jump of 255 or more resets the reference to the max and sends
      // k = 255: the earlier terms weigh less than 2^-246 against it (each
      // was at most 8 above the old reference), below the smallest fp32
      // number, so the factor 2^-255 (0 in fp32) is their weight rounded
      const bool first = m_run == -INFINITY;
      const bool up = !first && mx > m_run + 8.f;
      const float kc = up ? ceilf(mx - m_run) : 0.f;
      const bool reset = !(kc < 255.f);
      const int k_shift = reset ? 255 : (int)kc;
      alpha = __builtin_amdgcn_ldexpf(1.f, -k_shift);
      m_run = (first || reset) ? mx : m_run + kc;
      // the shift goes to the other waves beside P
      if (g == 0) *(LDS_AS uint8_t*)(size_t)(kb_addr(i) + 4 * hl + w) = (uint8_t)k_shift;
      pw = pb_addr(i);
    }
    uint32_t b_pw[4];
    if constexpr (QK) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        b_pw[c] = pw + o_pw[c];
        opq(b_pw[c]);
      }
    }
    // P' of page i for tokens 32rb + 8a + 4g .. +3 (group 4rb + a), published
    // as produced into head h_own's row of the P buffer
    auto p_group = [&](int grp) {
      const int rb = grp >> 2, a = grp & 3;
      float p[4], pv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        p[q] = __builtin_amdgcn_exp2f(sc[rb][4 * a + q] - m_run);
        pv[q] = __builtin_amdgcn_ldexpf(p[q], (int)((ew[grp] >> (8 * q)) & 0xFFu) - e_page);
      }
      // row sum: a short tree per group, two running sums (no long serial chain)
      lsum2[grp & 1] += (p[0] + p[1]) + (p[2] + p[3]);
      // (the first conversion's upper half is overwritten by the second)
      int wv = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], (int)ew[grp], false);
      wv = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], wv, true);
      *(LDS_AS int*)(size_t)(b_pw[2 * rb + (a >> 1)] + 8 * (a & 1)) = wv;
    };
    if constexpr (PV && QK) {
#pragma unroll
      for (int grp = 0; grp < 8; ++grp) {
        pv_mfma(8 + grp);
        p_group(grp);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (PV) {
      p_flags();
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        pv_mfma(m);
        if ((m & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (QK) {
#pragma unroll
      for (int grp = 0; grp < 8; ++grp) p_group(grp);
    }
    if constexpr (QK) l_run = l_run * alpha + (lsum2[0] + lsum2[1]);
  };

  using T = std::true_type;
  using F = std::false_type;
  wait_vmcnt<0>();
  lds_barrier();
  step(T{}, F{}, 0, n_tiles > 1 ? 1 : -1);
  int e_hold = e_page;
  for (int i = 1; i < n_tiles; ++i) {
    wait_vmcnt<0>();  // page i landed
    lds_barrier();    // page i and P of page i - 1 visible; slot (i + 1) % 3 and P buffer i % 2 free
    e_prev = e_hold;
    step(T{}, T{}, i, i + 1 < n_tiles ? i + 1 : -1);
    e_hold = e_page;
  }
  clear_tail(n_tiles - 1);
  lds_barrier();
  e_prev = e_hold;
  step(F{}, T{}, n_tiles, -1);

  // ---- partials (the bf16 kernel's layout): (m, l) by the head owner, O
  // rows through LDS, 32 heads at a time ----
  // The lane index is derived again (see opaque_lane), so nothing
  // lane-dependent of the prologue stays live across the page loop.
  const int lane_e = opaque_lane();
  const int hl_e = lane_e & 31, g_e = lane_e >> 5, h_own_e = w * 32 + hl_e;
  {
    // row sum of the head over both halves of its rows (lanes l and l ^ 32)
    const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    l_run = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
  }
  if (g_e == 0 && h_own_e < H) {
    const size_t prow = ((size_t)h_own_e * B + b) * splits + split;
    part_ml[prow * 2] = m_run;
    part_ml[prow * 2 + 1] = l_run;
  }
  constexpr int OP = DC + 4;
  LDS_AS float* ost = (LDS_AS float*)lds;
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    lds_barrier();
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = {o[ct][ht][4 * q], o[ct][ht][4 * q + 1], o[ct][ht][4 * q + 2], o[ct][ht][4 * q + 3]};
        *(LDS_AS f32x4*)(ost + hl_e * OP + 128 * w + 32 * ct + 8 * q + 4 * g_e) = v;
      }
    lds_barrier();
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int hh = rr * 4 + w, h = 32 * ht + hh;
      if (h < H) {
        // 512 values as bf16: 8 per lane
        const f32x4 x = *(const LDS_AS f32x4*)(ost + hh * OP + 8 * lane_e);
        const f32x4 y = *(const LDS_AS f32x4*)(ost + hh * OP + 8 * lane_e + 4);
        *(bf16x8_t*)(part_o + (((size_t)h * B + b) * splits + split) * DC + 8 * lane_e) =
            (bf16x8_t){(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3],
                       (__bf16)y[0], (__bf16)y[1], (__bf16)y[2], (__bf16)y[3]};
      }
    }
  }
}

}  // namespace

size_t fp8_page_bytes(int page, int d_c, int d_rope) { return page_bytes_of(page, d_c, d_rope); }

hipError_t quant_fp8(const mla_dims& d, int n_rows, const void* src, const int32_t* slots, int page, void* dst,
                     hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  ProfScope ps("mla_quant_fp8", s);
  hipLaunchKernelGGL(k_quant_fp8, dim3((n_rows + 3) / 4), dim3(256), 0, s, n_rows, d.d_c, d.d_rope, (const bf16*)src,
                     slots, page, (int)page_bytes_of(page, d.d_c, d.d_rope), (uint8_t*)dst);
  return hipGetLastError();
}

bool decode_fp8_supported(const mla_dims& d, const CacheView& c) {
  return d.dtype == MLA_BF16 && d.d_c == DC && d.d_rope == DR && d.d_nope == 128 && d.d_v == 128 &&
         d.n_heads <= MAX_HEADS && c.paged && c.block_size == PAGE;
}

namespace {
struct Ws8 {
  size_t qt, part_o, part_ml, run, total;
  int splits, pps;
};
size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }
Ws8 ws8_layout(int H, int rows, int q_len, int max_context) {
  Ws8 l;
  decode_plan(rows, max_context, q_len, &l.pps, &l.splits);
  l.qt = 0;
  l.part_o = al256((size_t)rows * H * (DC + DR) * 2);
  l.part_ml = l.part_o + al256((size_t)H * rows * l.splits * DC * 2);
  l.run = l.part_ml + al256((size_t)H * rows * l.splits * 2 * 4);
  l.total = l.run + 256;  // the run length the split kernel used, for the combine
  return l;
}
}  // namespace

size_t decode_fp8_workspace(const mla_dims& d, int n_seq, int q_len, int max_context) {
  return ws8_layout(d.n_heads, n_seq * q_len, q_len, max_context).total;
}

hipError_t decode_fp8(const mla_dims& d, float scale, int n_seq, int q_len, int max_context, const void* q_nope,
                      const void* q_pe, const void* w_uk, const void* w_uv, const CacheView& c, void* out, void* ws,
                      size_t ws_bytes, hipStream_t s) {
  const int H = d.n_heads, rows = n_seq * q_len;
  const Ws8 l = ws8_layout(H, rows, q_len, max_context);
  if (ws_bytes < l.total || l.splits > MAX_SPLITS) return hipErrorInvalidValue;
  char* base = (char*)ws;
  void* qt = base + l.qt;
  bf16* part_o = (bf16*)(base + l.part_o);
  float* part_ml = (float*)(base + l.part_ml);
  int32_t* run = (int32_t*)(base + l.run);
  hipError_t e = decode_absorb(d, scale, rows, q_len, q_nope, q_pe, w_uk, c.context_lens, qt, "mla_decode8_absorb", s);
  if (e != hipSuccess) return e;
  {
    ProfScope ps("mla_decode8_split", s);
    const bool pair_xcd = q_len > 1 && ((int64_t)n_seq * l.splits) % 8 == 0;
    const int order = pair_xcd ? 1 : (q_len == 1 && rows <= 256 ? 2 : 0);
    hipLaunchKernelGGL(k_split8, dim3(l.splits, rows), dim3(THREADS), 0, s, H, rows, q_len, order, l.splits, l.pps,
                       device_cus(), run, (const bf16*)qt, (const uint8_t*)c.rows, c.block_table, c.max_blocks,
                       c.context_lens, part_o, part_ml);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return decode_combine(d, rows, q_len, l.splits, run, c.context_lens, part_o, part_ml, w_uv, out,
                        "mla_decode8_combine_uv", s);
}

}  // namespace mla
