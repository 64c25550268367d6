// MFMA prefill attention for the DeepSeek-V3 latent shape (bf16, d_nope 128,
// d_rope 64, d_v 128), in the unabsorbed form: per head, keys are
// [W_UK,h c_t || k_pe_t] (192 wide, k_pe shared by all heads) and values
// W_UV,h c_t (128 wide), both up-projected beforehand by the GEMM
// ("DeepSeek-V2 paper digest" §2.1). For prefill this costs 192 + 128 MACs per
// (query, key, head) instead of 576 + 512 in the absorbed form of decode.
//
// Block = (sequence b, head h, 256 queries): eight waves, two per SIMD, each
// owning 32 queries. Keys stream in sub-tiles of 64 through a ring of four
// 40 KB LDS stages (direct 16-byte HBM -> LDS copies). Per sub-tile and wave:
//   S^T[t, s] = K[t] . Q[s]           2 key halves x 12 steps of K = 16
//   online softmax per query (lane column), causal mask on the diagonal
//   O^T[d, s] += V^T[d, t] P[t, s]    4 value tiles x 4 steps of 16 keys
// The waves form two groups (one wave of each per SIMD) that alternate, with
// a barrier per phase: while one group runs the MFMAs of a sub-tile (values of
// sub-tile u, then scores of u + 1), the other runs a softmax, so each SIMD's
// matrix core and vector ALU work at the same time.
// The score operand of half kh, step st is key 32kh + swap23(l % 32), dims
// 16st + 8(l / 32) .. +7 for lane l; swap23 exchanges bits 2 and 3 of the key
// index, so that the score MFMA's output rows (8(r/4) + 4(l/32) + r%4) come out
// as keys 16(r/8) + 8(l/32) + r%8: each lane's probabilities are then exactly
// the 8 consecutive keys its value-step B operand needs, with no exchange
// between lanes. Values come from the transposed copy the GEMM wrote.
// Query s of sequence b sits at position L_b - S + s and sees keys 0 .. that.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int DN = 128, DR = 64, DK = DN + DR, DV = 128, DC = 512, ROW = DC + DR;
constexpr int P_THREADS = 512, QW = 32, QT = 8 * QW, KS = 64;
constexpr int QK_STEPS = DK / 16;                // 12
constexpr int PE_OFF = KS * DN * 2;              // stage: K_nope rows (16 KB),
constexpr int V_OFF = PE_OFF + KS * DR * 2;      // k_pe rows (8 KB),
constexpr int P_STAGE = V_OFF + DV * KS * 2;     // V^T rows (16 KB)
constexpr int P_STAGES = 4;                      // 160 KB of LDS
constexpr int P_LOADS = P_STAGE / 16 / P_THREADS;  // 5 copies per lane and sub-tile
constexpr int WL_PE = PE_OFF / 1024, WL_V = V_OFF / 1024;  // first wave-copy of k_pe and V^T
constexpr float LOG2E_P = 1.4426950408889634f;
constexpr int PAIRS = DR / 2;

// RoPE inverse frequencies base^(-2i/d_rope), formed on the host in double
struct RopeTab {
  double theta[PAIRS];
};

template <int N>
__device__ __forceinline__ void p_wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ void p_lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void p_dma16s(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds_addr)
               : "memory", "m0");
}
// MFMAs with their accumulators in VGPRs (no AGPR is used, so the two waves of
// a SIMD each get up to 256 VGPRs); chained MFMAs on one accumulator need no
// wait states, and p_mfma_done() pads those a vector instruction needs before
// touching a result.
__device__ __forceinline__ void p_mfma_first(f32x16& acc, bf16x8_t a, bf16x8_t b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void p_mfma(f32x16& acc, bf16x8_t a, bf16x8_t b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void p_mfma_done(f32x16& a0, f32x16& a1) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a0), "+v"(a1));
}
__device__ __forceinline__ bf16x8_t p_as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }
// 21 wait states between an MFMA writing an accumulator and a vector
// instruction touching it (or the reverse), for the rare rescale and the final
// normalisation: the MFMAs here are inline asm, so the compiler does not pad.
__device__ __forceinline__ void p_fence() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" ::: "memory"); }
// The two values a lane and its partner 32 lanes away hold, in either order.
__device__ __forceinline__ void p_halves(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ int swap23(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

// k_pe of every cached token, gathered through the block table into a
// contiguous [B * seq_stride, d_rope] array (zeros past a sequence's context)
// so the attention kernel streams keys without a page lookup.
__global__ __launch_bounds__(256) void k_gather_kpe(int B, int seq_stride, const bf16* __restrict__ rows,
                                                    const int32_t* __restrict__ table, int max_blocks,
                                                    int block_size, const int32_t* __restrict__ ctx_lens,
                                                    bf16* __restrict__ kpe) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;  // 16-byte chunk index
  const int c = (int)(i % (DR / 8));
  const size_t tok = i / (DR / 8);
  const int b = (int)(tok / seq_stride), t = (int)(tok % seq_stride);
  if (b >= B) return;
  u32x4 v = {0, 0, 0, 0};
  if (t < ctx_lens[b]) {
    const int page = table[(size_t)b * max_blocks + t / block_size];
    v = *(const u32x4*)(rows + ((size_t)page * block_size + t % block_size) * ROW + DC + 8 * c);
  }
  *(u32x4*)(kpe + tok * DR + 8 * c) = v;
}

// cos and sin of the RoPE angle pos * theta_i for every position below
// n_pos and pair i (DeepSeek-V2 paper digest, decoupled RoPE): entry
// [pos][i] = (cos, sin) as fp32, the angle reduced to [-pi, pi] and both
// evaluated in double. Every query of every head at that position reads it.
__global__ __launch_bounds__(256) void k_rope_table(int n_pos, RopeTab rope, float2* __restrict__ cs) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n_pos * PAIRS) return;
  const double ang = (double)(i / PAIRS) * rope.theta[i % PAIRS];
  const double r = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
  double sn, cn;
  sincos(r, &sn, &cn);
  cs[i] = make_float2((float)cn, (float)sn);
}

// Stage layout: row t of K_nope (256 B), of k_pe (128 B) and row d of V^T
// (128 B = 64 keys) as in the workspace, with the 16-byte chunks of each row
// permuted: chunk c of K_nope row t sits at c ^ (t % 16), chunk c of a 128-byte
// row r at c ^ ((r / 2) % 8). Sixteen lanes reading the same chunk of sixteen
// consecutive rows (the operand reads) then hit sixteen distinct groups of
// banks, while each 1 KB copy still reads 1 KB of consecutive workspace bytes.
// Wave-copy wl fills stage bytes [1024 wl, +1024): K_nope for wl < 16, k_pe
// for wl < 24, V^T after.
__device__ __forceinline__ uint32_t piece_off(int wl, int lane) {
  if (wl < WL_PE) {  // rows 4wl .. 4wl+3, lane -> row 4wl + lane / 16, position lane % 16
    const int t = 4 * wl + (lane >> 4);
    return (uint32_t)(t * 256 + (((lane & 15) ^ (t & 15)) << 4));
  }
  // 128-byte rows 8j .. 8j+7, lane -> row 8j + lane / 8, position lane % 8
  const int j = wl < WL_V ? wl - WL_PE : wl - WL_V;
  const int r = 8 * j + (lane >> 3);
  return (uint32_t)(r * 128 + (((lane & 7) ^ ((r >> 1) & 7)) << 4));
}

__global__ __launch_bounds__(P_THREADS, 1) void k_prefill_attn(
    int H, int B, int S, int nq, float qscale, const float2* __restrict__ rope_cs, const bf16* __restrict__ q_nope,
    const bf16* __restrict__ q_pe, const bf16* __restrict__ kn, const bf16* __restrict__ vt, int seq_stride,
    const bf16* __restrict__ kpe, const int32_t* __restrict__ ctx_lens, bf16* __restrict__ out) {
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
  // contexts are at most seq_stride (the workspace rows of a sequence); the
  // clamp only keeps a bad length from reading past them
  const int L = min(ctx_lens[b], seq_stride);
  const int s0 = qtile * QT;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hl = lane & 31, g = lane >> 5;
  const int last_key = min(L - S + min(s0 + QT, S) - 1, L - 1);  // of the whole block
  const int n_sub = last_key < 0 ? 0 : last_key / KS + 1;
  // query block of the wave: the two groups (waves 0-3, 4-7) take alternate
  // blocks of 32, so their causal work is alike
  const int qb = 2 * (w & 3) + (w >> 2);
  const int pos = L - S + min(s0 + QW * qb + hl, S - 1);  // this lane's query position
  const int pos_lo = L - S + min(s0 + QW * qb, S - 1);    // the wave's first query
  const int pos_hi = L - S + min(s0 + QW * qb + QW - 1, S - 1);

  // ---- copies of sub-tile u into stage u % 4: wave-copy wl = 5w + k (1 KB
  // of the stage) is all K_nope, all k_pe or all V^T, so its source base is
  // uniform (SGPRs) and each lane adds a fixed offset. The workspace rows run
  // to a multiple of 64 tokens and hold finite values past the context.
  uint32_t soff[P_LOADS];
#pragma unroll
  for (int k = 0; k < P_LOADS; ++k) soff[k] = piece_off(w * P_LOADS + k, lane);
  const uint32_t lds_base = (uint32_t)(size_t)(LDS_AS char*)lds;
  const char* kn_b = (const char*)kn + ((size_t)b * H + h) * seq_stride * DN * 2;
  const char* kp_b = (const char*)kpe + (size_t)b * seq_stride * DR * 2;
  const char* vt_b = (const char*)vt + ((size_t)b * H + h) * DV * seq_stride * 2;
  // source of copy k of this wave (uniform): base and bytes per sub-tile
  const char* src_base[P_LOADS];
  uint32_t src_step[P_LOADS];
#pragma unroll
  for (int k = 0; k < P_LOADS; ++k) {
    const int wl = w * P_LOADS + k;
    const bool is_v = wl >= WL_V, is_n = wl < WL_PE;
    src_base[k] = is_v ? vt_b : (is_n ? kn_b : kp_b);
    src_step[k] = is_v ? KS * DV * 2 : (is_n ? KS * DN * 2 : KS * DR * 2);
  }
  // copy k (of P_LOADS) of this wave for sub-tile u
  auto load_piece = [&](int u, int k) __attribute__((always_inline)) {
    const uint32_t st = lds_base + (u % P_STAGES) * P_STAGE;
    p_dma16s(src_base[k] + (size_t)u * src_step[k], soff[k],
             __builtin_amdgcn_readfirstlane(st + (w * P_LOADS + k) * 1024));
  };
  auto load_sub = [&](int u) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < P_LOADS; ++k) load_piece(u, k);
  };
  for (int v = 0; v < min(2, n_sub); ++v) load_sub(v);

  // ---- query fragments (B operand): 12 steps of 16 over [q_nope || RoPE(q_pe)]
  bf16x8_t qf[QK_STEPS];
  {
    const int s_lane = min(s0 + QW * qb + hl, S - 1);
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
      // (cos, sin) of pairs 8st + 4g .. +3 at this lane's position
      const float2* cs_p = rope_cs + (size_t)max(pos, 0) * PAIRS + 8 * st + 4 * g;
      const float4 cs01 = *(const float4*)cs_p;
      const float4 cs23 = *(const float4*)(cs_p + 2);
      const float cs[8] = {cs01.x, cs01.y, cs01.z, cs01.w, cs23.x, cs23.y, cs23.z, cs23.w};
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float c = cs[e], sn = cs[e + 1];
        const float x0 = (float)v[e], x1 = (float)v[e + 1];
        o[e] = (__bf16)((x0 * c - x1 * sn) * qscale);
        o[e + 1] = (__bf16)((x0 * sn + x1 * c) * qscale);
      }
      qf[DN / 16 + st] = o;
    }
  }

  f32x16 o[DV / 32];
#pragma unroll
  for (int i = 0; i < DV / 32; ++i) o[i] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;
  // operand read offsets in a stage (see piece_off): score step st < 8 reads
  // K_nope row t = swap23(hl) (+32 for the second key half), chunk 2st + g;
  // step st >= 8 reads k_pe row t, chunk 2(st - 8) + g; value step ks of
  // value tile dt reads V^T row 32dt + hl, chunk 2ks + g
  uint32_t kq_off[DN / 16], pq_off[DR / 16], vq_off[4];
  {
    const int t = swap23(hl);
#pragma unroll
    for (int st = 0; st < DN / 16; ++st) kq_off[st] = t * 256 + (((2 * st + g) ^ (t & 15)) << 4);
#pragma unroll
    for (int j = 0; j < DR / 16; ++j) pq_off[j] = PE_OFF + t * 128 + (((2 * j + g) ^ ((t >> 1) & 7)) << 4);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) vq_off[ks] = V_OFF + hl * 128 + (((2 * ks + g) ^ ((hl >> 1) & 7)) << 4);
  }
  // sub-tiles holding a key that one of this wave's queries sees
  const int n_own = pos_hi < 0 ? 0 : min(n_sub, pos_hi / KS + 1);
  auto stage = [&](int u) __attribute__((always_inline)) { return (const LDS_AS char*)(lds + (u % P_STAGES) * P_STAGE); };

  f32x16 sc[2];   // scores of the sub-tile between its score and softmax steps
  bf16x8_t pf[4]; // its probabilities between the softmax and value steps

  // ---- MFMA step: values of sub-tile u (PV), then scores of sub-tile u + 1
  // (QK); the first score operands are read during the value MFMAs.
  // dma_v >= 0: this step also issues this wave's copies of sub-tile dma_v,
  // spread over its work so the copies reach the texture unit a few at a time
  auto mfma_step = [&](auto do_pv, auto do_qk, int u, int dma_v) __attribute__((always_inline)) {
    constexpr bool PV = decltype(do_pv)::value, QK = decltype(do_qk)::value;
    __builtin_amdgcn_s_setprio(1);
    const LDS_AS char* kp = stage(u + 1);
    const LDS_AS char* vp = stage(PV ? u : 0);
    // score operand of step st, key half kh; value operand of step k = 4dt + ks
    auto k_read = [&](int st, int kh) __attribute__((always_inline)) {
      return st < DN / 16 ? *(const LDS_AS u32x4*)(kp + kq_off[st] + kh * 32 * 256)
                          : *(const LDS_AS u32x4*)(kp + pq_off[st - DN / 16] + kh * 32 * 128);
    };
    auto v_read = [&](int k) __attribute__((always_inline)) {
      return *(const LDS_AS u32x4*)(vp + vq_off[k & 3] + (k >> 2) * 32 * 128);
    };
    // operands are read 3 MFMA steps ahead (rings of 4)
    u32x4 ka[4][2];
    u32x4 va[4];
    if constexpr (PV) {
#pragma unroll
      for (int k = 0; k < 3; ++k) va[k] = v_read(k);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int dt = k >> 2, ks = k & 3;
        if (k + 3 < 16) va[(k + 3) & 3] = v_read(k + 3);
        if constexpr (QK) {
          // the first three score steps' operands, over the last value MFMAs
          if (k >= 10) ka[(k - 10) >> 1][(k - 10) & 1] = k_read((k - 10) >> 1, (k - 10) & 1);
        }
        p_mfma(o[dt], p_as_bf16x8(va[k & 3]), pf[ks]);
        if (k % 3 == 0 && k / 3 < P_LOADS && dma_v >= 0) load_piece(dma_v, k / 3);
      }
    } else if constexpr (QK) {
#pragma unroll
      for (int st = 0; st < 3; ++st)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) ka[st][kh] = k_read(st, kh);
    }
    if constexpr (QK) {
#pragma unroll
      for (int st = 0; st < QK_STEPS; ++st) {
        if (st + 3 < QK_STEPS)
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) ka[(st + 3) & 3][kh] = k_read(st + 3, kh);
        if (st == 0) {
          p_mfma_first(sc[0], p_as_bf16x8(ka[0][0]), qf[0]);
          p_mfma_first(sc[1], p_as_bf16x8(ka[0][1]), qf[0]);
        } else {
          p_mfma(sc[0], p_as_bf16x8(ka[st & 3][0]), qf[st]);
          p_mfma(sc[1], p_as_bf16x8(ka[st & 3][1]), qf[st]);
        }
      }
      p_mfma_done(sc[0], sc[1]);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- softmax step of sub-tile u (log2 domain): the reference max moves
  // only when the sub-tile's max exceeds it by more than 8; a lane's first
  // sub-tile sets it
  auto softmax_step = [&](int u) __attribute__((always_inline)) {
    const int t0 = u * KS;
    // causal mask (only where the sub-tile reaches past the wave's first
    // query): register r of half kh is key t0 + 32kh + 16(r/8) + 8g + r%8
    if (t0 + KS - 1 > pos_lo) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (t0 + 32 * kh + 16 * (r >> 3) + 8 * g + (r & 7) > pos) sc[kh][r] = -INFINITY;
    }
    float mx = sc[0][0];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kh][r]);
    {
      float x0, x1;
      p_halves(mx, x0, x1);
      mx = fmaxf(x0, x1);
    }
    const bool up = mx > m_run + 8.f;
    const float alpha = (up && m_run != -INFINITY) ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
    m_run = up ? mx : m_run;
    const float msub = m_run == -INFINITY ? 0.f : m_run;
    if (__ballot(alpha != 1.f)) {
      p_fence();
#pragma unroll
      for (int i = 0; i < DV / 32; ++i) o[i] *= alpha;
      p_fence();
    }
    // probabilities: step ks (16 keys) = registers 8(ks % 2) .. +7 of half ks / 2
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[ks][e] = (__bf16)__builtin_amdgcn_exp2f(sc[ks >> 1][8 * (ks & 1) + e] - msub);
    // row sum of the probabilities as rounded for the value MFMAs
    float lsum0 = 0.f, lsum1 = 0.f;
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    const bf16x2_t one2 = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2_t pr = {pf[ks][e], pf[ks][e + 1]};
        if (ks & 1) lsum1 = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, lsum1, false);
        else lsum0 = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, lsum0, false);
      }
    const float lsum = lsum0 + lsum1;
    l_run = l_run * alpha + lsum;
    // wait states between the vector writes of P and the MFMAs reading it
    asm volatile("s_nop 4" : "+v"(pf[0]), "+v"(pf[1]), "+v"(pf[2]), "+v"(pf[3]));
  };

  // ---- two groups in alternation: waves 0-3 (group 0, one per SIMD) run
  // the step sequence QK(0), SM(0), M(0), SM(1), M(1), ... (SM = softmax,
  // M(u) = PV(u) + QK(u+1)); waves 4-7 run the same sequence one phase
  // later. A barrier closes every phase, so on each SIMD one wave's MFMAs
  // overlap the other wave's softmax.
  // Copies: sub-tile k + 2 goes into the stage that sub-tile k - 2 left (its
  // last reader, group 1's M(k - 2), ran in phase 2k - 1); each group issues
  // its share piecewise inside its next MFMA step (group 0 in phase 2k, group
  // 1 in phase 2k + 1). At the end of phase 2k + 1 the copies of sub-tile
  // k + 1 (read from phase 2k + 2 on) are complete.
  // closes phase ph: after an odd phase the copies of the sub-tile read from
  // the next phase on are complete; then the barrier
  auto phase_end = [&](int ph) __attribute__((always_inline)) {
    if (ph & 1) {
      const int v = (ph >> 1) + 1;
      if (v + 1 < n_sub) p_wait_vmcnt<P_LOADS>();
      else p_wait_vmcnt<0>();
    }
    p_lds_barrier();
  };
  using T = std::true_type;
  using F = std::false_type;
  if (n_sub > 1) p_wait_vmcnt<P_LOADS>();  // sub-tile 0 landed
  else p_wait_vmcnt<0>();
  p_lds_barrier();
  if (w < 4) {
    if (2 < n_sub) load_sub(2);
    if (n_own > 0) mfma_step(F{}, T{}, -1, -1);  // QK(0)
    phase_end(0);
    for (int u = 0; u < n_sub; ++u) {
      if (u < n_own) softmax_step(u);
      phase_end(2 * u + 1);
      const int dv = u + 3 < n_sub ? u + 3 : -1;  // copies of phase 2u + 2
      if (u < n_own) mfma_step(T{}, T{}, u, dv);
      else if (dv >= 0) load_sub(dv);
      phase_end(2 * u + 2);
    }
    phase_end(2 * n_sub + 1);
  } else {
    phase_end(0);
    if (2 < n_sub) load_sub(2);
    if (n_own > 0) mfma_step(F{}, T{}, -1, -1);  // QK(0)
    phase_end(1);
    for (int u = 0; u < n_sub; ++u) {
      if (u < n_own) softmax_step(u);
      phase_end(2 * u + 2);
      const int dv = u + 3 < n_sub ? u + 3 : -1;  // copies of phase 2u + 3
      if (u < n_own) mfma_step(T{}, T{}, u, dv);
      else if (dv >= 0) load_sub(dv);
      phase_end(2 * u + 3);
    }
  }

  // ---- normalise and store: lane holds d = 32dt + 8r' + 4g .. +3 of its
  // query. The block's 256 output rows (256 bytes each) go through LDS so that
  // each store instruction writes four whole rows.
  p_fence();
  float l0, l1;
  p_halves(l_run, l0, l1);
  const float lt = l0 + l1;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  constexpr int OP = DV + 8;  // staged row pitch in bf16 (272 bytes)
  LDS_AS bf16* ost = (LDS_AS bf16*)lds;
  typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
#pragma unroll
  for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
      const bf16x4_t v = {(__bf16)(o[dt][4 * r4] * inv), (__bf16)(o[dt][4 * r4 + 1] * inv),
                          (__bf16)(o[dt][4 * r4 + 2] * inv), (__bf16)(o[dt][4 * r4 + 3] * inv)};
      *(LDS_AS u32x2_t*)(ost + (QW * qb + hl) * OP + 32 * dt + 8 * r4 + 4 * g) = __builtin_bit_cast(u32x2_t, v);
    }
  p_lds_barrier();
#pragma unroll
  for (int k = 0; k < QT * (DV / 8) / P_THREADS; ++k) {
    const int idx = threadIdx.x + P_THREADS * k, row = idx / (DV / 8), ch = idx % (DV / 8);
    const int s_out = s0 + row;
    if (s_out < S)
      __builtin_nontemporal_store(*(const LDS_AS u32x4*)(ost + row * OP + 8 * ch),
                                  (u32x4*)(out + (((size_t)b * S + s_out) * H + h) * DV + 8 * ch));
  }
}

}  // namespace

bool prefill_fast_supported(const mla_dims& d, const CacheView& c) {
  return d.dtype == MLA_BF16 && d.d_c == DC && d.d_rope == DR && d.d_nope == DN && d.d_v == DV && c.paged &&
         d.n_heads <= 256;
}

namespace {
// rows per sequence in the workspace: whole sub-tiles of 64 keys
int ws_stride(int max_context) { return (max_context + KS - 1) / KS * KS; }
}  // namespace

size_t prefill_fast_workspace(const mla_dims& d, int batch, int max_context) {
  // K_nope [batch][H][stride][128], V^T [batch][H][stride / 64][128][64] and
  // k_pe [batch * stride, 64] of every cached token, then the RoPE table
  // [stride, 32] of (cos, sin)
  const size_t rows = (size_t)batch * ws_stride(max_context);
  return 2 * rows * d.n_heads * DN * 2 + rows * DR * 2 + (size_t)ws_stride(max_context) * PAIRS * 8;
}

hipError_t prefill_fast(const mla_dims& d, float scale, int batch, int seq_len, int max_context,
                        const void* q_nope, const void* q_pe, const void* w_uk, const void* w_uv,
                        const CacheView& c, void* out, void* ws, size_t ws_bytes, hipStream_t s) {
  const int H = d.n_heads;
  if (ws_bytes < prefill_fast_workspace(d, batch, max_context)) return hipErrorInvalidValue;
  const int stride = ws_stride(max_context);
  const size_t rows = (size_t)batch * stride;
  bf16* kn = (bf16*)ws;
  bf16* vt = kn + rows * H * DN;
  bf16* kpe = vt + rows * H * DV;
  float2* rope_cs = (float2*)(kpe + rows * DR);
  // K_nope = c W_UK^T and V = c W_UV^T for every cached token (rows gathered
  // through the block table; rows past a sequence's context repeat its row 0
  // and are masked), head-major so that a sub-tile of one head is contiguous;
  // V is stored transposed in blocks of 64 tokens
  GemmArgs g{};
  g.M = (int)rows;
  g.K = DC;
  g.a = (const bf16*)c.rows;
  g.lda = ROW;
  g.a_table = c.block_table;
  g.a_lens = c.context_lens;
  g.a_seq = stride;
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
    e = gemm_fast(g, 3, s);
    if (e != hipSuccess) return e;
    g.b0 = g.b1 = (const bf16*)w_uv;
    g.c0 = g.c1 = vt;
    e = gemm_fast(g, 2, s);
  }
  if (e != hipSuccess) return e;
  {
    ProfScope ps("mla_prefill_kpe", s);
    const size_t chunks = rows * (DR / 8);
    hipLaunchKernelGGL(k_gather_kpe, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s, batch, stride,
                       (const bf16*)c.rows, c.block_table, c.max_blocks, c.block_size, c.context_lens, kpe);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    ProfScope ps("mla_prefill_rope", s);
    RopeTab rope;
    for (int i = 0; i < PAIRS; ++i) rope.theta[i] = pow((double)d.rope_base, -2.0 * i / (double)DR);
    hipLaunchKernelGGL(k_rope_table, dim3((unsigned)((stride * PAIRS + 255) / 256)), dim3(256), 0, s, stride, rope,
                       rope_cs);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    ProfScope ps("mla_prefill_attn", s);
    const int nq = (seq_len + QT - 1) / QT;
    hipLaunchKernelGGL(k_prefill_attn, dim3(nq * H * batch), dim3(P_THREADS), 0, s, H, batch, seq_len, nq,
                       scale * LOG2E_P, rope_cs, (const bf16*)q_nope, (const bf16*)q_pe, kn, vt, stride, kpe,
                       c.context_lens, (bf16*)out);
  }
  return hipGetLastError();
}

}  // namespace mla
