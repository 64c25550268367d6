// MFMA prefill attention for the DeepSeek-V3 latent shape (bf16, d_nope 128,
// d_rope 64, d_v 128), in the unabsorbed form: per head, keys are
// [W_UK,h c_t || k_pe_t] (192 wide, k_pe shared by all heads) and values
// W_UV,h c_t (128 wide), both up-projected beforehand by the GEMM
// ("DeepSeek-V2 paper digest" §2.1). For prefill this costs 192 + 128 MACs per
// (query, key, head) instead of 576 + 512 in the absorbed form of decode.
//
// Block = (sequence b, head h, 256 queries); wave w owns queries 64w .. 64w+63
// as two halves of 32 (one MFMA column block each), so every key operand read
// from LDS feeds two MFMAs. Keys stream in sub-tiles of 32 through a ring of
// eight 20 KB LDS stages (K 32 x 192, V 32 x 128; direct 16-byte HBM -> LDS
// copies issued six sub-tiles ahead). Iteration u of a wave:
//   S^T[t, s] = K[t] . Q[s] for sub-tile u   12 steps of K = 16, 2 halves
//   interleaved with the online softmax of sub-tile u - 1 (exp2, row sums, bf16
//   probabilities), so matrix cores and vector ALUs overlap
//   O^T[d, s] += V^T[d, t] P[t, s] for u - 1  4 value tiles x 2 steps, 2 halves;
//                                             V^T by transposed LDS reads
// Query s of sequence b sits at position L_b - S + s and sees keys 0 .. that.
#include <math.h>

#include <type_traits>

#ifndef PREFILL_SGB
#define PREFILL_SGB 0
#endif

#include "common.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int DN = 128, DR = 64, DK = DN + DR, DV = 128, DC = 512, ROW = DC + DR;
constexpr int P_THREADS = 256, QW = 64, QT = 4 * QW, KS = 32;
// A stage holds sub-tile u in the order the MFMA operand reads consume it:
// 12 score-operand blocks of 1 KB (step st: lane l's 16 bytes = key l % 32,
// dims 16st + 8(l / 32) .. +7 of [K_nope || k_pe]) and 16 value-operand blocks
// of 512 B (lane l's 8 bytes for one transposed read). Every read is then 64
// consecutive lanes over consecutive bytes (no bank conflicts), and its lane
// offset is the same for all blocks. Each 16-byte piece is a contiguous slice
// of one key row, so the HBM -> LDS copies can scatter rows into this order.
constexpr int K_BLOCK = 1024, V_BLOCK = 512;
constexpr int V_OFF = (DK / 16) * K_BLOCK;     // 12 KB
constexpr int P_STAGE = V_OFF + 16 * V_BLOCK;  // 20 KB
constexpr int P_STAGES = 8;                    // 160 KB of LDS
constexpr int P_AHEAD = P_STAGES - 2;          // sub-tiles in flight
constexpr int P_LOADS = P_STAGE / 16 / P_THREADS;  // 5 copies per lane and sub-tile
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
// The two values a lane and its partner 32 lanes away hold, in either order.
__device__ __forceinline__ void p_halves(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
constexpr int WL_KP = 8, WL_V = 12;  // wave-copies 0-7 K_nope, 8-11 k_pe, 12-19 V

// Value-operand read block I = 4dt + 2ks + ab (value tile dt, step ks of 16
// keys, half ab of the key octet): PV lane p gets the 4 keys
// 16ks + 8ab + 4(p / 32) + 0..3 of value column 32dt + (p % 32) from a
// transposed read, so it supplies key row vr_row and columns vr_col .. +3.
__device__ __forceinline__ int vr_row(int I, int p) { return 16 * ((I >> 1) & 1) + 8 * (I & 1) + 4 * (p >> 5) + ((p & 15) >> 2); }
__device__ __forceinline__ int vr_col(int I, int p) { return 32 * (I >> 2) + 16 * ((p >> 4) & 1) + 4 * (p & 3); }

// Source row (within the sub-tile) and byte offset within that row of the
// 16-byte piece that lane `lane` of wave-copy wl brings in.
__device__ __forceinline__ int piece_row(int wl, int lane) {
  if (wl < WL_V) return lane & 31;
  const int x = (wl - WL_V) * 64 + lane;  // piece: lanes 2(x % 32), +1 of block x / 32
  return vr_row(x >> 5, 2 * (x & 31));
}
__device__ __forceinline__ uint32_t piece_col_bytes(int wl, int lane) {
  if (wl < WL_KP) return 2 * (16 * wl + 8 * (lane >> 5));
  if (wl < WL_V) return 2 * (16 * (wl - WL_KP) + 8 * (lane >> 5));
  const int x = (wl - WL_V) * 64 + lane;
  return 2 * vr_col(x >> 5, 2 * (x & 31));
}
__device__ __forceinline__ uint32_t row_bytes(int wl, int H) {
  return wl < WL_KP ? H * DN * 2 : (wl < WL_V ? ROW * 2 : H * DV * 2);
}

__global__ __launch_bounds__(P_THREADS, 1) void k_prefill_attn(
    int H, int B, int S, int nq, float qscale, float base, const bf16* __restrict__ q_nope,
    const bf16* __restrict__ q_pe, const bf16* __restrict__ kn, const bf16* __restrict__ vv, int seq_stride,
    const bf16* __restrict__ rows, const int32_t* __restrict__ table, int max_blocks, int block_size,
    const int32_t* __restrict__ ctx_lens, bf16* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) char lds[P_STAGES * P_STAGE];
  // Blocks of one (b, h) share its keys: with the group count a multiple of 8
  // they go to one XCD (block i runs on XCD i % 8) and so share its L2; the
  // longest query tiles go first.
  int group, qtile;
  {
    const int i = blockIdx.x, G = H * B;
    if ((G & 7) == 0) {
      const int slot = i >> 3;
      group = (slot / nq) * 8 + (i & 7);
      qtile = nq - 1 - slot % nq;
    } else {
      group = i / nq;
      qtile = nq - 1 - i % nq;
    }
  }
  const int h = group % H, b = group / H;
  const int L = ctx_lens[b];
  const int s0 = qtile * QT;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hl = lane & 31, g = lane >> 5, i16 = lane & 15, G4 = lane >> 4;
  const int last_key = min(L - S + min(s0 + QT, S) - 1, L - 1);  // of the whole block
  const int n_sub = last_key < 0 ? 0 : last_key / KS + 1;
  const int32_t* tb = table + (size_t)b * max_blocks;

  int pos[2], pos_lo[2];  // this lane's query position; the half's smallest
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    pos[q] = L - S + min(s0 + QW * w + 32 * q + hl, S - 1);
    pos_lo[q] = L - S + min(s0 + QW * w + 32 * q, S - 1);
  }

  // ---- copies of sub-tile u into stage u % 8 ----
  // Wave-copy wl (0 .. 19, 1 KB of the stage each) is all K_nope, all k_pe or
  // all V, so its source base is uniform; per lane only a fixed byte offset
  // is added. A sub-tile lies in one cache page (block_size is a multiple of
  // 32), whose number comes from one scalar load; no per-lane global load sits
  // between the copies in flight. Rows past the context (last sub-tile only)
  // are clamped to the last row: they are masked, but must stay finite.
  uint32_t soff[P_LOADS];
#pragma unroll
  for (int k = 0; k < P_LOADS; ++k) {
    const int wl = w * P_LOADS + k;
    soff[k] = piece_row(wl, lane) * row_bytes(wl, H) + piece_col_bytes(wl, lane);
  }
  const uint32_t lds_base = (uint32_t)(size_t)(LDS_AS char*)lds;
  const char* kn_b = (const char*)kn + ((size_t)b * seq_stride * H + h) * DN * 2;
  const char* vv_b = (const char*)vv + ((size_t)b * seq_stride * H + h) * DV * 2;
  auto load_sub = [&](int u) {
    const uint32_t st = lds_base + (u % P_STAGES) * P_STAGE;
    const int t0 = u * KS;
    const int page = tb[t0 / block_size];
    const char* bn = kn_b + (size_t)t0 * H * DN * 2;
    const char* bp = (const char*)rows + (((size_t)page * block_size + t0 % block_size) * ROW + DC) * 2;
    const char* bv = vv_b + (size_t)t0 * H * DV * 2;
    if (t0 + KS <= L) {
#pragma unroll
      for (int k = 0; k < P_LOADS; ++k) {
        const int wl = w * P_LOADS + k;
        const char* base = wl < WL_KP ? bn : (wl < WL_V ? bp : bv);
        p_dma16(base + soff[k], __builtin_amdgcn_readfirstlane(st + wl * 1024));
      }
    } else {
#pragma unroll
      for (int k = 0; k < P_LOADS; ++k) {
        const int wl = w * P_LOADS + k;
        const char* base = wl < WL_KP ? bn : (wl < WL_V ? bp : bv);
        const uint32_t off = min(piece_row(wl, lane), L - 1 - t0) * row_bytes(wl, H) + piece_col_bytes(wl, lane);
        p_dma16(base + off, __builtin_amdgcn_readfirstlane(st + wl * 1024));
      }
    }
  };
  for (int v = 0; v < min(P_AHEAD, n_sub); ++v) load_sub(v);

  // ---- query fragments (B operand): 12 steps of 16 over [q_nope || RoPE(q_pe)]
  bf16x8_t qf[2][DK / 16];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int s_lane = min(s0 + QW * w + 32 * q + hl, S - 1);
    const bf16* qn = q_nope + (((size_t)b * S + s_lane) * H + h) * DN + 8 * g;
#pragma unroll
    for (int st = 0; st < DN / 16; ++st) {
      const bf16x8_t v = p_as_bf16x8(*(const u32x4*)(qn + 16 * st));
      bf16x8_t o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (__bf16)((float)v[e] * qscale);
      qf[q][st] = o;
    }
    const bf16* qp = q_pe + (((size_t)b * S + s_lane) * H + h) * DR + 8 * g;
#pragma unroll
    for (int st = 0; st < DR / 16; ++st) {
      const bf16x8_t v = p_as_bf16x8(*(const u32x4*)(qp + 16 * st));
      bf16x8_t o;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int pr = 8 * st + 4 * g + e / 2;  // pair index in 0 .. 31
        const double ang = (double)pos[q] * pow((double)base, -2.0 * pr / (double)DR);
        const float r = (float)(ang - 6.283185307179586 * rint(ang * 0.15915494309189535));
        float sn, cs;
        sincosf(r, &sn, &cs);
        const float x0 = (float)v[e], x1 = (float)v[e + 1];
        o[e] = (__bf16)((x0 * cs - x1 * sn) * qscale);
        o[e + 1] = (__bf16)((x0 * sn + x1 * cs) * qscale);
      }
      qf[q][DN / 16 + st] = o;
    }
  }

  // operand reads: score step st at K_BLOCK st + 16 lane, value block I at
  // V_OFF + V_BLOCK I + 8 lane of the stage
  const int k_lane = 16 * lane, v_lane = V_OFF + 8 * lane;

  f32x16 o[2][DV / 32];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int i = 0; i < DV / 32; ++i) o[q][i] = (f32x16){};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  auto stage_of = [&](int u) { return (const LDS_AS char*)(lds + (u % P_STAGES) * P_STAGE); };

  // wait for sub-tile u, make it visible, refill the stage freed by u - 2
  auto begin = [&](int u) {
    const int ahead = min(P_AHEAD - 1, n_sub - 1 - u);
    switch (ahead) {
      case 5: p_wait_vmcnt<5 * P_LOADS>(); break;
      case 4: p_wait_vmcnt<4 * P_LOADS>(); break;
      case 3: p_wait_vmcnt<3 * P_LOADS>(); break;
      case 2: p_wait_vmcnt<2 * P_LOADS>(); break;
      case 1: p_wait_vmcnt<1 * P_LOADS>(); break;
      default: p_wait_vmcnt<0>(); break;
    }
    p_lds_barrier();
    if (u + P_AHEAD < n_sub) load_sub(u + P_AHEAD);
  };

  // causal mask of sub-tile u (only where it reaches past a half's first query)
  auto mask = [&](f32x16 (&sc)[2], int u) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
      if (KS * u + KS - 1 > pos_lo[q]) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (KS * u + 8 * (r >> 2) + 4 * g + (r & 3) > pos[q]) sc[q][r] = -INFINITY;
      }
  };

  // One step of the pipeline: scores of sub-tile u into sc (QK) and, for the
  // previous sub-tile (SM; sp already masked), the online softmax and its
  // value product. The running maximum and the (rare) rescale of the
  // accumulators come first, so that the score MFMAs, the exponentials and the
  // value MFMAs form one straight run the scheduler can interleave.
  auto step = [&](auto do_qk, auto do_sm, int u, f32x16 (&sc)[2], f32x16 (&sp)[2]) {
    constexpr bool QK = decltype(do_qk)::value, SM = decltype(do_sm)::value;
    float msub[2], alpha[2];
    if constexpr (SM) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float mx = sp[q][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sp[q][r]);
        float x0, x1;
        p_halves(mx, x0, x1);
        mx = fmaxf(x0, x1);
        const bool up = mx > m_run[q] + 8.f;
        alpha[q] = (up && m_run[q] != -INFINITY) ? __builtin_amdgcn_exp2f(m_run[q] - mx) : 1.f;
        m_run[q] = up ? mx : m_run[q];
        msub[q] = m_run[q] == -INFINITY ? 0.f : m_run[q];
        if (__ballot(alpha[q] != 1.f)) {
#pragma unroll
          for (int i = 0; i < DV / 32; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              float x = o[q][i][r];
              p_scale_acc(x, alpha[q]);
              o[q][i][r] = x;
            }
        }
      }
    }
    if constexpr (QK) {
      const LDS_AS char* st = stage_of(u);
      bf16x8_t ka[3];
      const LDS_AS char* kp = st + k_lane;
      ka[0] = p_as_bf16x8(*(const LDS_AS u32x4*)(kp));
      ka[1] = p_as_bf16x8(*(const LDS_AS u32x4*)(kp + K_BLOCK));
#pragma unroll
      for (int s = 0; s < DK / 16; ++s) {
        if (s + 2 < DK / 16) ka[(s + 2) % 3] = p_as_bf16x8(*(const LDS_AS u32x4*)(kp + K_BLOCK * (s + 2)));
        if (s == 0) {
          sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], qf[0][0], (f32x16){}, 0, 0, 0);
          sc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], qf[1][0], (f32x16){}, 0, 0, 0);
        } else {
          sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s % 3], qf[0][s], sc[0], 0, 0, 0);
          sc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s % 3], qf[1][s], sc[1], 0, 0, 0);
        }
      }
    }
    if constexpr (SM) {
      // P as the value-product operand: step ks covers keys 16ks .. 16ks+15 =
      // registers 8ks .. 8ks+7 (masked keys give p = 0)
      bf16x8_t pf[2][2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float lsum = 0.f;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float pe = __builtin_amdgcn_exp2f(sp[q][8 * ks + e] - msub[q]);
            lsum += pe;
            pf[q][ks][e] = (__bf16)pe;
          }
        l_run[q] = l_run[q] * alpha[q] + lsum;
      }
      const LDS_AS char* vp = stage_of(u - 1) + v_lane;
#pragma unroll
      for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int I = 4 * dt + 2 * ks;
          const bf16x8_t a =
              p_cat(__builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS short4_t*)(vp + V_BLOCK * I)),
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS short4_t*)(vp + V_BLOCK * (I + 1))));
          o[0][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[0][ks], o[0][dt], 0, 0, 0);
          o[1][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[1][ks], o[1][dt], 0, 0, 0);
        }
    }
#if PREFILL_SGB
    if constexpr (QK && SM) {
#pragma unroll
      for (int s = 0; s < 12; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);  // VALU / transcendental
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);  // VALU / transcendental
      }
    }
#endif
  };

  using T = std::true_type;
  using F = std::false_type;
  f32x16 sa[2], sb[2];
  if (n_sub > 0) {
    begin(0);
    step(T{}, F{}, 0, sa, sb);
    int u = 1;
    for (; u + 1 < n_sub; u += 2) {
      mask(sa, u - 1);
      begin(u);
      step(T{}, T{}, u, sb, sa);
      mask(sb, u);
      begin(u + 1);
      step(T{}, T{}, u + 1, sa, sb);
    }
    if (u < n_sub) {
      mask(sa, u - 1);
      begin(u);
      step(T{}, T{}, u, sb, sa);
      mask(sb, u);
      step(F{}, T{}, u + 1, sa, sb);
    } else {
      mask(sa, u - 1);
      step(F{}, T{}, u, sb, sa);
    }
  }

  // ---- normalise and store: lane holds d = 32dt + 8r' + 4g .. +3 of its query
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    float l0, l1;
    p_halves(l_run[q], l0, l1);
    const float lt = l0 + l1;
    const int s_out = s0 + QW * w + 32 * q + hl;
    if (s_out >= S) continue;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    bf16* op = out + (((size_t)b * S + s_out) * H + h) * DV + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
        const bf16x4_t v = {(__bf16)(o[q][dt][4 * r4] * inv), (__bf16)(o[q][dt][4 * r4 + 1] * inv),
                            (__bf16)(o[q][dt][4 * r4 + 2] * inv), (__bf16)(o[q][dt][4 * r4 + 3] * inv)};
        *(bf16x4_t*)(op + 32 * dt + 8 * r4) = v;
      }
  }
}

}  // namespace

bool prefill_fast_supported(const mla_dims& d, const CacheView& c) {
  return d.dtype == MLA_BF16 && d.d_c == DC && d.d_rope == DR && d.d_nope == DN && d.d_v == DV && c.paged &&
         c.block_size % KS == 0 && d.n_heads <= 256;
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
    const int nq = (seq_len + QT - 1) / QT;
    hipLaunchKernelGGL(k_prefill_attn, dim3(nq * H * batch), dim3(P_THREADS), 0, s, H, batch, seq_len, nq,
                       scale * LOG2E_P, d.rope_base, (const bf16*)q_nope, (const bf16*)q_pe, kn, vv, max_context,
                       (const bf16*)c.rows, c.block_table, c.max_blocks, c.block_size, c.context_lens, (bf16*)out);
  }
  return hipGetLastError();
}

}  // namespace mla
