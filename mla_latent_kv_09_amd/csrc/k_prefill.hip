// MFMA prefill attention for the DeepSeek-V3 latent shape (bf16, d_nope 128,
// d_rope 64, d_v 128), in the unabsorbed form: per head, keys are
// [W_UK,h c_t || k_pe_t] (192 wide, k_pe shared by all heads) and values
// W_UV,h c_t (128 wide), both up-projected beforehand by the GEMM
// ("DeepSeek-V2 paper digest" §2.1). For prefill this costs 192 + 128 MACs per
// (query, key, head) instead of 576 + 512 in the absorbed form of decode.
//
// Block = (sequence b, head h, 128 queries); wave w owns queries 32w .. 32w+31.
// Keys stream in tiles of 64 through a ring of three LDS stages (K tile 64 x
// 192, V tile 64 x 128, direct 16-byte HBM -> LDS copies). Per tile and wave:
//   S^T[t, s] = K[t] . Q[s]      2 key tiles x 12 steps of K = 16 (MFMA 32x32x16)
//   online softmax per query (lane column), causal and context masks
//   O^T[d, s] += V^T[d, t] P[t, s]  4 value tiles x 4 steps; V^T by transposed
//                                   LDS reads, P straight from the score registers
// Query s of sequence b sits at position L_b - S + s and sees keys 0 .. that.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int DN = 128, DR = 64, DK = DN + DR, DV = 128, DC = 512, ROW = DC + DR;
constexpr int P_THREADS = 256, QT = 128, KT = 64;
constexpr int K_ROW_BYTES = DK * 2;           // 384
constexpr int V_ROW_BYTES = DV * 2;           // 256
constexpr int K_TILE = KT * K_ROW_BYTES;      // 24 KB
constexpr int V_TILE = KT * V_ROW_BYTES;      // 16 KB
constexpr int P_STAGE = K_TILE + V_TILE;      // 40 KB
constexpr int P_STAGES = 3;
constexpr int P_LOADS = (K_TILE + V_TILE) / 16 / P_THREADS;  // 10 per lane
constexpr float LOG2E_P = 1.4426950408889634f;

template <int N>
__device__ __forceinline__ void p_wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ void p_lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void p_dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_addr)
               : "memory", "m0");
}
__device__ __forceinline__ bf16x8_t p_as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ bf16x8_t p_cat(short4_t a, short4_t b) {
  typedef __attribute__((ext_vector_type(8))) short short8_t;
  short8_t s = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8_t, s);
}
__device__ __forceinline__ void p_scale_acc(float& x, float a) {
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
// K tile: 24 chunks per row; chunk c of row t sits at (c & ~7) | ((c & 7) ^
// ((t >> 1) & 7)): the 16 consecutive rows of a score-operand read hit 16
// distinct bank groups. V tile: 16 chunks per row (a 256-byte stride, so every
// row starts on bank 0); chunk c of row t sits at c ^ (4 (t & 3)): the 4 rows x
// 4 chunks that 32 lanes of a transposed read touch land on 16 distinct chunk
// positions.
__device__ __forceinline__ int k_swz(int t) { return (t >> 1) & 7; }
__device__ __forceinline__ int v_pos(int t, int c) { return c ^ (4 * (t & 3)); }

__global__ __launch_bounds__(P_THREADS, 1) void k_prefill_attn(
    int H, int S, float qscale, float base, const bf16* __restrict__ q_nope, const bf16* __restrict__ q_pe,
    const bf16* __restrict__ kn, const bf16* __restrict__ vv, int seq_stride, const bf16* __restrict__ rows,
    const int32_t* __restrict__ table, int max_blocks, int block_size, const int32_t* __restrict__ ctx_lens,
    bf16* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) char lds[P_STAGES * P_STAGE];
  const int qtile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int L = ctx_lens[b];
  const int s0 = qtile * QT;
  if (s0 >= S) return;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hl = lane & 31, g = lane >> 5, i16 = lane & 15, G = lane >> 4;
  const int s_lane = min(s0 + 32 * w + hl, S - 1);         // this lane's query (clamped)
  const int pos = L - S + s_lane;                           // its position = last visible key
  const int last_key = min(L - S + min(s0 + QT, S) - 1, L - 1);  // of the whole block
  const int n_kv = last_key < 0 ? 0 : last_key / KT + 1;
  const int32_t* tb = table + (size_t)b * max_blocks;

  // ---- query fragments (B operand): 12 steps of 16 over [q_nope || RoPE(q_pe)]
  bf16x8_t qf[DK / 16];
  {
    const bf16* qn = q_nope + (((size_t)b * S + s_lane) * H + h) * DN + 8 * g;
#pragma unroll
    for (int st = 0; st < DN / 16; ++st) {
      const bf16x8_t v = p_as_bf16x8(*(const u32x4*)(qn + 16 * st));
      bf16x8_t o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (__bf16)((float)v[e] * qscale);
      qf[st] = o;
    }
    const bf16* qp = q_pe + (((size_t)b * S + s_lane) * H + h) * DR + 8 * g;
#pragma unroll
    for (int st = 0; st < DR / 16; ++st) {
      const bf16x8_t v = p_as_bf16x8(*(const u32x4*)(qp + 16 * st));
      bf16x8_t o;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int pr = 8 * st + 4 * g + e / 2;  // pair index in 0 .. 31
        const double ang = (double)pos * pow((double)base, -2.0 * pr / (double)DR);
        const float r = (float)(ang - 6.283185307179586 * rint(ang * 0.15915494309189535));
        float sn, cs;
        sincosf(r, &sn, &cs);
        const float x0 = (float)v[e], x1 = (float)v[e + 1];
        o[e] = (__bf16)((x0 * cs - x1 * sn) * qscale);
        o[e + 1] = (__bf16)((x0 * sn + x1 * cs) * qscale);
      }
      qf[DN / 16 + st] = o;
    }
  }

  // ---- copies of key tile j: per lane 10 chunks (K_nope 4, k_pe 2, V 4) ----
  // LDS chunk position p of a stage: K rows (24 chunks each) then V rows (16).
  // A 64-key tile lies in one cache page (block_size is a multiple of 64), so
  // its page comes from one scalar load; no per-lane global load precedes the
  // copies (those would make the compiler drain the copies in flight).
  const uint32_t lds_base = (uint32_t)(size_t)(LDS_AS char*)lds;
  auto load_tile = [&](int j) {
    const uint32_t st = lds_base + (j % P_STAGES) * P_STAGE;
    const int page = tb[(j * KT) / block_size];
    const size_t pslot = (size_t)page * block_size + (j * KT) % block_size;
#pragma unroll
    for (int k = 0; k < P_LOADS; ++k) {
      const int p = (w * P_LOADS + k) * 64 + lane;  // chunk position within the stage
      const bf16* src;
      if (p < KT * 24) {
        const int t = p / 24, cp = p % 24, c = (cp & ~7) | ((cp & 7) ^ k_swz(t));
        const int dt = min(j * KT + t, L - 1) - j * KT;  // clamp into the context
        const bf16* ksrc = kn + ((size_t)b * seq_stride + j * KT + dt) * H * DN + h * DN + 8 * c;
        const bf16* psrc = rows + (pslot + dt) * ROW + DC + 8 * (c - 16);
        src = c < 16 ? ksrc : psrc;
      } else {
        const int q = p - KT * 24, t = q >> 4, c = v_pos(t, q & 15);
        const int dt = min(j * KT + t, L - 1) - j * KT;
        src = vv + ((size_t)b * seq_stride + j * KT + dt) * H * DV + h * DV + 8 * c;
      }
      p_dma16(src, __builtin_amdgcn_readfirstlane(st + (w * P_LOADS + k) * 1024));
    }
  };
  if (n_kv > 0) load_tile(0);
  if (n_kv > 1) load_tile(1);

  // operand read offsets (lane part)
  //  score operand, key tile half kh, step st: row 32kh + hl, chunk 2st + g
  //  value operand, value tile dt, step ks (16 keys), half a/b:
  //    rows 16ks + 4g + i16/4 (+8), columns 32dt + 16(G%2) + 4(i16%4)
  int k_off[2][DK / 16];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    const int t = 32 * kh + hl;
#pragma unroll
    for (int st = 0; st < DK / 16; ++st) {
      const int c = 2 * st + g;
      k_off[kh][st] = t * K_ROW_BYTES + (((c & ~7) | ((c & 7) ^ k_swz(t))) << 4);
    }
  }
  int v_off[4][2];  // [dt][a/b] for ks = 0; rows advance by 16 per ks (the swizzle has period 4)
  {
    const int ra = 4 * g + (i16 >> 2), rb = ra + 8;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int col = 32 * dt + 16 * (G & 1) + 4 * (i16 & 3);
      const int c = col >> 3, sub = (col & 7) * 2;
      v_off[dt][0] = K_TILE + ra * V_ROW_BYTES + (v_pos(ra, c) << 4) + sub;
      v_off[dt][1] = K_TILE + rb * V_ROW_BYTES + (v_pos(rb, c) << 4) + sub;
    }
  }

  f32x16 o[DV / 32];
#pragma unroll
  for (int i = 0; i < DV / 32; ++i) o[i] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;

  for (int j = 0; j < n_kv; ++j) {
    if (j + 1 < n_kv) p_wait_vmcnt<P_LOADS>();
    else p_wait_vmcnt<0>();
    p_lds_barrier();
    if (j + 2 < n_kv) load_tile(j + 2);
    const LDS_AS char* st = (const LDS_AS char*)(lds + (j % P_STAGES) * P_STAGE);

    f32x16 sc[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      sc[kh] = (f32x16){};
#pragma unroll
      for (int s = 0; s < DK / 16; ++s) {
        const bf16x8_t a = p_as_bf16x8(*(const LDS_AS u32x4*)(st + k_off[kh][s]));
        sc[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sc[kh], 0, 0, 0);
      }
    }
    // masks: key t visible iff t <= pos (causal; pos < L always)
    const int t0 = j * KT;
    if (t0 + KT - 1 > pos) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (t0 + 32 * kh + 8 * (r >> 2) + 4 * g + (r & 3) > pos) sc[kh][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kh][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    float alpha = 1.f;
    if (mx > m_run + 8.f) {
      if (m_run != -INFINITY) alpha = __builtin_amdgcn_exp2f(m_run - mx);
      m_run = mx;
    }
    if (__ballot(alpha != 1.f)) {
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DV / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = o[i][r];
          p_scale_acc(x, alpha);
          o[i][r] = x;
        }
    }
    // P as the PV operand: step ks covers keys 16ks .. 16ks+15 = registers
    // 8(ks%2) .. +7 of key tile ks/2 (fully masked tiles give p = 0)
    bf16x8_t pf[4];
    float lsum = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = sc[ks >> 1][8 * (ks & 1) + e];
        const float pe = x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x - m_run);
        lsum += pe;
        pf[ks][e] = (__bf16)pe;
      }
    }
    l_run += lsum;
#pragma unroll
    for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kofs = 16 * ks * V_ROW_BYTES;
        const bf16x8_t a = p_cat(__builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS short4_t*)(st + v_off[dt][0] + kofs)),
                                 __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS short4_t*)(st + v_off[dt][1] + kofs)));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], o[dt], 0, 0, 0);
      }
  }

  // ---- normalise and store: lane holds d = 32dt + 8q + 4g .. +3 of query s
  l_run += __shfl_xor(l_run, 32, 64);
  const int s_out = s0 + 32 * w + hl;
  if (s_out >= S) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  bf16* op = out + (((size_t)b * S + s_out) * H + h) * DV + 4 * g;
#pragma unroll
  for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
      const bf16x4_t v = {(__bf16)(o[dt][4 * q] * inv), (__bf16)(o[dt][4 * q + 1] * inv),
                          (__bf16)(o[dt][4 * q + 2] * inv), (__bf16)(o[dt][4 * q + 3] * inv)};
      *(bf16x4_t*)(op + 32 * dt + 8 * q) = v;
    }
}

}  // namespace

bool prefill_fast_supported(const mla_dims& d, const CacheView& c) {
  return d.dtype == MLA_BF16 && d.d_c == DC && d.d_rope == DR && d.d_nope == DN && d.d_v == DV && c.paged &&
         c.block_size % KT == 0 && d.n_heads <= 256;
}

size_t prefill_fast_workspace(const mla_dims& d, int batch, int max_context) {
  // K_nope and V of every cached token: [batch * max_context, H * 128] each
  return 2 * (size_t)batch * max_context * d.n_heads * DN * 2;
}

hipError_t prefill_fast(const mla_dims& d, float scale, int batch, int seq_len, int max_context,
                        const void* q_nope, const void* q_pe, const void* w_uk, const void* w_uv,
                        const CacheView& c, void* out, void* ws, size_t ws_bytes, hipStream_t s) {
  const int H = d.n_heads;
  if (ws_bytes < prefill_fast_workspace(d, batch, max_context)) return hipErrorInvalidValue;
  bf16* kn = (bf16*)ws;
  bf16* vv = kn + (size_t)batch * max_context * H * DN;
  // K_nope = c W_UK^T and V = c W_UV^T for every cached token (rows gathered
  // through the block table; rows past a sequence's context are never read)
  GemmArgs g{};
  g.M = batch * max_context;
  g.K = DC;
  g.a = (const bf16*)c.rows;
  g.lda = ROW;
  g.a_table = c.block_table;
  g.a_lens = c.context_lens;
  g.a_seq = max_context;
  g.a_max_blocks = c.max_blocks;
  g.a_block = c.block_size;
  g.N = H * DN;
  g.b0 = g.b1 = (const bf16*)w_uk;
  g.n_split = g.N;
  g.ldb = DC;
  g.c0 = g.c1 = kn;
  g.ldc0 = g.ldc1 = H * DN;
  g.c_split = g.N;
  hipError_t e;
  {
    ProfScope ps("mla_prefill_kv_up", s);
    e = gemm_fast(g, 0, s);
    if (e != hipSuccess) return e;
    g.b0 = g.b1 = (const bf16*)w_uv;
    g.c0 = g.c1 = vv;
    e = gemm_fast(g, 0, s);
  }
  if (e != hipSuccess) return e;
  {
    ProfScope ps("mla_prefill_attn", s);
    const dim3 grid((seq_len + QT - 1) / QT, H, batch);
    hipLaunchKernelGGL(k_prefill_attn, grid, dim3(P_THREADS), 0, s, H, seq_len, scale * LOG2E_P, d.rope_base,
                       (const bf16*)q_nope, (const bf16*)q_pe, kn, vv, max_context, (const bf16*)c.rows,
                       c.block_table, c.max_blocks, c.block_size, c.context_lens, (bf16*)out);
  }
  return hipGetLastError();
}

}  // namespace mla
