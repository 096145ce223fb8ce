// Fused, tiled attention forward kernel for gfx950 (MI355X).
//
// Pages cited (title, then the section on that page):
//   [DF] "FlashAttention数据流优化：MI50显存与带宽瓶颈实战"  (kwkr.cn/news/544806)
//   [AI] "AIInfra笔记01"                                   (kwkr.cn/news/547341)
//   [OP] "FlashAttention优化原理与工程实践"                (lbrq.cn/news/50349)
//
// One workgroup = 4 waves = 128 query rows of one (batch, head); each wave owns
// 32 rows.  The method ([DF §2.2], first and second layers; [OP §2.1], blocked
// loop over query and key blocks):
//   * the Q tile is loaded once and stays in VGPRs as MFMA operands;
//   * K/V tiles of BC keys stream through a double-buffered LDS ring; the loads
//     of tile j+2 are in flight (in VGPRs) while tile j is computed, and tile
//     j+1 is written to the other LDS buffer after tile j's compute ([DF §2.3]
//     prefetch of the next block, done here as register-staged double buffering);
//   * Sᵀ = K·Qᵀ runs on v_mfma_f32_32x32x16_{bf16,f16} with fp32 accumulation,
//     so each lane holds 32 keys of ONE query row: the row max and row sums are
//     in-lane, plus one exchange with the other half-wave;
//   * online softmax in base 2: t = S·(|scale|·log2 e), running max m, running
//     sums, rescale α = 2^(m_old − m_new) of the partial output ([DF §2.2],
//     second layer), exp on v_exp_f32;
//   * P is rounded to the input type and fed straight from the Sᵀ accumulator
//     layout into Oᵀ = Vᵀ·Pᵀ (same MFMA), V being transposed into LDS on the
//     way in (a key permutation inside each 16-key block makes every MFMA
//     A-operand one 128-bit LDS read);
//   * epilogue: O / l_r, rounded to the input type, and lse = (m + log2 l_f)·ln 2.
// Causal ([DF §4.1] flag): key tiles above a workgroup's last row are never
// loaded or computed, a wave skips tiles above its own rows, and only tiles that
// cross the diagonal pay for the mask.
//
// The MFMA 32x32 accumulator layout used throughout: lane l, register r hold
// C[row = 8*(r/4) + 4*(l/32) + r%4][col = l%32].  A-operand lane l holds row
// l%32, B-operand lane l holds column l%32; both hold 8 contraction elements,
// and because the A and B of one instruction assign contraction indices to
// (lane-half, element) identically, any consistent assignment of keys / head
// dims to those slots gives the same product.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa355 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

enum { DT_F16 = 0, DT_BF16 = 1 };

// Buffer resource word 3 for gfx9-family raw buffers: 32-bit data format, so
// untyped loads/stores work and out-of-range accesses read 0 / are dropped.
constexpr int kBufferFlags = 0x00020000;

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int Lq, Lk;
  int n_qt;         // query tiles per head: ceil(Lq / 128)
  int num_wg;       // B * H * n_qt
  int xcd_remap;    // 1: group consecutive work items on one XCD
  float c;          // |scale| * log2(e), or log2(e) when scale == 0 (always > 0)
  uint32_t q_and;   // 0xffffffff, or 0 when scale == 0 (Q forced to zero)
  uint32_t q_xor;   // 0x80008000 when scale < 0 (Q negated exactly), else 0
};

template <int DT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == DT_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
}

// Two fp32 -> one dword of two 16-bit values, round to nearest even.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  f32x2 f = {lo, hi};
  if constexpr (DT == DT_BF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
}

// acc + lo + hi of a packed pair of 16-bit values (exact products with 1.0, fp32 sum).
template <int DT>
__device__ __forceinline__ float sum2(uint32_t pk, float acc) {
  if constexpr (DT == DT_BF16)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(i16x2, pk), __builtin_bit_cast(i16x2, 0x3f803f80u),
                                           acc, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk), __builtin_bit_cast(f16x2, 0x3c003c00u), acc,
                                  false);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFlags);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}

__device__ __forceinline__ float xhalf_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float xhalf_sum(float x) { return x + __shfl_xor(x, 32); }

// Tile geometry shared by the kernel and the host launcher.
template <int D>
struct Geo {
  static constexpr int NW = 4;                 // waves per workgroup
  static constexpr int NT = 64 * NW;           // threads per workgroup
  static constexpr int BR = 32 * NW;           // query rows per workgroup
  static constexpr int BC = D == 128 ? 64 : 128;  // keys per K/V tile
  static constexpr int KB = BC / 32;           // 32-key blocks of a tile (Sᵀ MFMA row blocks)
  static constexpr int NB = D / 32;            // 32-dim blocks of the output (Oᵀ MFMA row blocks)
  static constexpr int KS = D / 16;            // contraction steps of QKᵀ
  static constexpr int NCH = D / 8;            // 16-byte chunks per K/V row
  static constexpr int KP = D * 2 + 16;        // LDS pitch of a K row (bytes), padded
  static constexpr int VP = BC * 2 + 16;       // LDS pitch of a Vᵀ row (bytes), padded
  static constexpr int KBYTES = BC * KP;
  static constexpr int VBYTES = D * VP;
  static constexpr int BUF = KBYTES + VBYTES;  // one stage of the ring
  static constexpr int LDS = 2 * BUF;
  static_assert((BC / 4) * NCH == NT, "one (4-key group, 16-byte chunk) pair per thread");
  static_assert(LDS <= 163840, "LDS budget of one gfx950 workgroup");
};

// Position of key offset u (0..BC-1) inside a Vᵀ row: within each 16-key block the
// 4-key groups are stored in the order 0, 2, 1, 3, so that the 8 keys one lane
// contributes to a 32x32x16 MFMA (4 from rows 8(r/4)+4g.. of the Sᵀ accumulator,
// twice) are contiguous.
__device__ __forceinline__ int vt_pos(int u) {
  const int a = (u & 15) >> 2;
  return (u & ~15) + 8 * (a & 1) + 4 * (a >> 1) + (u & 3);
}

template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(256) void fa_fwd_kernel(FwdParams p) {
  using G = Geo<D>;
  constexpr int BC = G::BC, KB = G::KB, NB = G::NB, KS = G::KS, NCH = G::NCH;
  constexpr int KP = G::KP, VP = G::VP, KBYTES = G::KBYTES, BUF = G::BUF;
  constexpr float NEG_INF = -__builtin_inff();
  __shared__ __attribute__((aligned(16))) unsigned char smem[G::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

  // ---- work item: (batch*head, query tile); heaviest causal tiles first, and
  // consecutive items (all query tiles of one head) on the same XCD, whose L2
  // then serves the K/V re-reads of that head.
  const int bid = blockIdx.x;
  const int item = p.xcd_remap ? (bid & 7) * (p.num_wg >> 3) + (bid >> 3) : bid;
  const int bh = item / p.n_qt;
  const int qt_r = item - bh * p.n_qt;
  const int qt = CAUSAL ? p.n_qt - 1 - qt_r : qt_r;
  const int i0 = qt * G::BR;
  const int i0w = i0 + 32 * wave;
  const int Lq = p.Lq, Lk = p.Lk;

  const size_t qbase = (size_t)bh * (size_t)Lq * D * 2;
  const size_t kbase = (size_t)bh * (size_t)Lk * D * 2;
  const auto qrs = make_rsrc((const char*)p.q + qbase, (uint32_t)Lq * D * 2);
  const auto krs = make_rsrc((const char*)p.k + kbase, (uint32_t)Lk * D * 2);
  const auto vrs = make_rsrc((const char*)p.v + kbase, (uint32_t)Lk * D * 2);
  const auto ors = make_rsrc((char*)p.o + qbase, (uint32_t)Lq * D * 2);

  // ---- Q tile -> VGPRs, as the B operand of Sᵀ = K·Qᵀ (column = query row l%32,
  // contraction slots of half g = head dims 16s+8g .. 16s+8g+7).  Rows past Lq read 0.
  const int qrow = i0w + l32;
  u32x4 qr[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u32x4 x = buf_load16(qrs, (uint32_t)(qrow * D + 16 * s + 8 * g) * 2);
    qr[s] = (x & p.q_and) ^ p.q_xor;
  }

  // ---- key range of this workgroup
  int n_kv = (Lk + BC - 1) / BC;
  if constexpr (CAUSAL) {
    const int last_row = min(i0 + G::BR, Lq) - 1;
    n_kv = min(n_kv, last_row / BC + 1);
  }

  // ---- K/V tile loader: thread = (4-key group lG, 16-byte chunk lc)
  const int lc = tid % NCH, lG = tid / NCH;
  u32x4 kreg[4], vreg[4];
  auto gload = [&](int j0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t off = (uint32_t)((j0 + 4 * lG + r) * D + 8 * lc) * 2;  // keys >= Lk read 0
      kreg[r] = buf_load16(krs, off);
      vreg[r] = buf_load16(vrs, off);
    }
  };
  const int vpos = vt_pos(4 * lG);
  auto swrite = [&](int buf) {
    unsigned char* Ks = smem + buf * BUF;
    unsigned char* Vs = Ks + KBYTES;
#pragma unroll
    for (int r = 0; r < 4; ++r) *(u32x4*)(Ks + (4 * lG + r) * KP + 16 * lc) = kreg[r];
    // transpose 4 keys x 8 dims into 8 rows of Vᵀ, 4 keys (8 bytes) each
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const int w = d >> 1;
      uint32_t lo, hi;
      if (d & 1) {
        lo = (vreg[0][w] >> 16) | (vreg[1][w] & 0xffff0000u);
        hi = (vreg[2][w] >> 16) | (vreg[3][w] & 0xffff0000u);
      } else {
        lo = (vreg[0][w] & 0xffffu) | (vreg[1][w] << 16);
        hi = (vreg[2][w] & 0xffffu) | (vreg[3][w] << 16);
      }
      *(u32x2*)(Vs + (8 * lc + d) * VP + 2 * vpos) = u32x2{lo, hi};
    }
  };

  const float c = p.c;
  float m_run = NEG_INF, l_f = 0.f, l_r = 0.f;
  f32x16 oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x16{};

  gload(0);
  swrite(0);
  if (n_kv > 1) gload(BC);
  __syncthreads();

  for (int j = 0; j < n_kv; ++j) {
    const int j0 = j * BC;
    const unsigned char* Ks = smem + (j & 1) * BUF;
    const unsigned char* Vs = Ks + KBYTES;
    const bool active = !CAUSAL || j0 <= i0w + 31;  // wave-uniform
    if (active) {
      // ---- Sᵀ = K·Qᵀ for this tile: KB blocks of 32 keys x 32 query rows
      f32x16 sacc[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        sacc[kb] = f32x16{};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const u32x4 a = *(const u32x4*)(Ks + (32 * kb + l32) * KP + 16 * (2 * s + g));
          sacc[kb] = mfma32<DT>(a, qr[s], sacc[kb]);
        }
      }
      // ---- mask: only tiles that cross the diagonal or the end of the keys
      const bool need_mask = (CAUSAL && j0 + BC - 1 > i0w) || (j0 + BC > Lk);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
            const bool masked = (CAUSAL && key > qrow) || key >= Lk;
            sacc[kb][r] = masked ? NEG_INF : sacc[kb][r];
          }
      }
      // ---- online softmax (base 2)
      float mx = NEG_INF;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = xhalf_max(mx);
      const float m_new = fmaxf(m_run, mx * c);
      const float mb = m_new == NEG_INF ? 0.f : m_new;  // no visible key yet: keep weights 0
      const float alpha = __builtin_amdgcn_exp2f(m_run - mb);
      m_run = m_new;
      u32x4 pb[KB][2];
      float sf = 0.f, sr = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][8 * h + 2 * e], c, -mb));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][8 * h + 2 * e + 1], c, -mb));
            sf += p0 + p1;
            const uint32_t pk = pack2<DT>(p0, p1);
            sr = sum2<DT>(pk, sr);
            pb[kb][h][e] = pk;
          }
      l_f = l_f * alpha + sf;
      l_r = l_r * alpha + sr;
      // ---- Oᵀ = α·Oᵀ + Vᵀ·Pᵀ
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        oacc[nb] *= alpha;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const u32x4 a = *(const u32x4*)(Vs + (32 * nb + l32) * VP + 16 * (4 * kb + 2 * h + g));
            oacc[nb] = mfma32<DT>(a, pb[kb][h], oacc[nb]);
          }
      }
    }
    if (j + 1 < n_kv) {
      swrite((j + 1) & 1);
      if (j + 2 < n_kv) gload((j + 2) * BC);
    }
    __syncthreads();
  }

  // ---- epilogue: normalise by the sum of the rounded weights, store O and LSE
  const float lf_t = xhalf_sum(l_f);
  const float lr_t = xhalf_sum(l_r);
  const float inv = 1.0f / lr_t;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * nb + 8 * q4 + 4 * g;
      const u32x2 w = {pack2<DT>(oacc[nb][4 * q4] * inv, oacc[nb][4 * q4 + 1] * inv),
                       pack2<DT>(oacc[nb][4 * q4 + 2] * inv, oacc[nb][4 * q4 + 3] * inv)};
      buf_store8(ors, (uint32_t)(qrow * D + d0) * 2, w);  // rows >= Lq are dropped
    }
  if (g == 0 && qrow < Lq) p.lse[(size_t)bh * Lq + qrow] = (m_run + log2f(lf_t)) * 0.69314718055994530942f;
}

}  // namespace fa355
