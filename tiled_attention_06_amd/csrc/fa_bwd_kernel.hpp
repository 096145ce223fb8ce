// Attention backward kernels for gfx950 (MI355X): dQ, dK, dV by recomputing the
// probabilities from the forward pass's per-row log-sum-exp.
//
// Pages cited (title, then the section on that page):
//   [DF] "FlashAttention数据流优化：MI50显存与带宽瓶颈实战"  (kwkr.cn/news/544806)
//
// [DF §2.2] (third layer, recomputation): the backward pass stores no score
// matrix; it recomputes the score blocks from Q and K in the forward pass's
// block order with the softmax statistics the forward pass kept (here the LSE).
// The gradients are those of the forward definition: with s = scale·q·k,
// P = exp(s − LSE) on visible pairs, for an upstream gradient dO of O:
//   dV_j = Σ_i P_ij dO_i,  dP_ij = dO_i·v_j,  Δ_i = Σ_j P_ij dP_ij = dO_i·O_i,
//   dS_ij = P_ij (dP_ij − Δ_i),  dQ_i = scale Σ_j dS_ij k_j,  dK_j = scale Σ_i dS_ij q_i.
//
// Two kernels on one stream:
//   * fa_bwd_dq_kernel: one workgroup = 8 waves = 256 query rows (as the forward
//     pass); each lane first forms its row's Δ = dO·O (fp32 from the stored
//     values) and LSE·log2(e) and writes both to the workspace for the second
//     kernel; per 64-key tile Sᵀ = K·Qᵀ and dPᵀ = V·dOᵀ on MFMA (Q and dO rows
//     resident in VGPRs as B operands), P and dS in registers (one row per lane),
//     dQᵀ += Kᵀ·dSᵀ with Kᵀ read through transposing LDS reads;
//   * fa_bwd_dkdv_kernel: one workgroup = 4 waves = 128 keys, each wave owns 32
//     keys (K and V rows resident in VGPRs); per 64-row query tile S = Q·Kᵀ and
//     dP = dO·Vᵀ on MFMA, P and dS in registers (one key per lane), then
//     dVᵀ += dOᵀ·P and dKᵀ += Qᵀ·dS with dOᵀ and Qᵀ read transposed from LDS;
//     at D = 128 without dropout fa_bwd_dkdv2_kernel instead: 8 waves, two per
//     32 keys, one making S, P and dV, the other dP, dS and dK.
// Each tile reaches LDS through the buffer unit (buffer_load ... lds, no VGPR
// staging) in the forward pass's two LDS images: a row image for operands read
// row by row and a transposing image for operands read across rows.  Two
// stages: the copies of the next tile are issued before the current one is
// computed.  Every wave owns disjoint outputs, so there are no atomics and the
// results are deterministic.
//
// Numerics: fp32 accumulation; P and dS are rounded to the input type as MFMA
// operands (fa_bwd_dkdv2_kernel forms dK's dS from P as rounded); dQ and dK are
// scaled in fp32 before the final rounding.

#pragma once

#include "fa_fwd_kernel.hpp"

namespace fa355 {

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;   // forward LSE, natural log, fp32 [B*H][Lq]
  void* dq;
  void* dk;
  void* dv;
  float* ws_lse2;     // LSE·log2(e), fp32 [B*H][Lq4] (rows Lq..Lq4-1 hold 0)
  float* ws_delta;    // Δ = dO·O, fp32 [B*H][Lq4] (rows Lq..Lq4-1 hold 0)
  int Lq, Lk;
  int Lq4;            // Lq rounded up to a multiple of 4: 16-byte groups of rows never straddle the end
  int bh;             // B*H
  int H;              // heads (b = bh / H, h = bh % H)
  // element strides of batch, head and row of q, k, v, o, dout, dq, dk, dv (in
  // that order, indices T_Q .. T_DV); the head dim is contiguous
  int64_t sb[8], sh[8];
  int sl[8];
  int kv_off;         // causal: key position of query row 0 (Lk - Lq >= 0)
  int n_qt;           // query tiles of 256 rows per head (dq kernel)
  int n_kt;           // key tiles of 128 keys per head (dkdv kernel)
  int num_wg;         // workgroups of the kernel being launched
  int xcd_remap;      // 1: group consecutive work items on one XCD
  float c;            // scale·log2(e) (any sign)
  float scale;
  // dropout (kernels instantiated with DROP): the forward pass's keep bits
  // (byte < drop_t), kept weights scaled by drop_scale = 256 / drop_t
  uint32_t drop_t, seed_lo, seed_hi;
  float drop_scale;
};

enum { T_Q = 0, T_K, T_V, T_O, T_DO, T_DQ, T_DK, T_DV };

// Start of tensor T's (batch, head) slab; its rows are sl[T] elements apart.
template <typename Ptr>
__device__ __forceinline__ Ptr bwd_slab(Ptr base, const BwdParams& p, int T, int bh) {
  const int b = bh / p.H, h = bh - b * p.H;
  return (Ptr)((const char*)base + ((int64_t)b * p.sb[T] + (int64_t)h * p.sh[T]) * 2);
}
// Bytes from a slab's start to the end of its last row of `rows` (the buffer range)
template <int D>
__device__ __forceinline__ uint32_t bwd_end(const BwdParams& p, int T, int rows) {
  return (uint32_t)(((int64_t)(rows - 1) * p.sl[T] + D) * 2);
}

// The two 16-bit values of a dword as fp32 (exact), low half first.
template <int DT>
__device__ __forceinline__ float2 unpack2(uint32_t u) {
  if constexpr (DT == DT_BF16)
    return make_float2(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
  else
    return make_float2((float)__builtin_bit_cast(_Float16, (unsigned short)(u & 0xffffu)),
                       (float)__builtin_bit_cast(_Float16, (unsigned short)(u >> 16)));
}

// Tile copies HBM -> LDS for the backward kernels: a tile of 64 rows of one
// (batch, head) slab into the forward pass's row image (block pitch KBS) or
// transposing image (block pitch VBS).  Copy j of wave w fills block w + NW·j.
// Store a wave's 32 rows (row r0 + l%32, dims 32nb + 8(r/4) + 4g + r%4 in lane l,
// register r of acc[nb]) times sc, rounded to the input type: the rows are laid out
// row-major in the LDS buffer stg (rows 2·D + 16 bytes apart: 16-byte aligned row
// reads, the 8-byte writes of 16 lanes on distinct banks), then stored as whole
// rows, 16 bytes per lane, instead of 8-byte pieces scattered over 32 rows per
// instruction.  The wave reads back only what its own lanes wrote (LDS keeps a
// wave's accesses in order).  Rows past the buffer range's end are dropped.
template <int D, int DT>
__device__ __forceinline__ void stage_rows_out(const f32x16 (&acc)[D / 32], float sc, unsigned char* stg, int lane,
                                               __amdgpu_buffer_rsrc_t rs, int r0, int row_stride) {
  constexpr int PITCH = 2 * D + 16, CPR = D / 8;
  const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * nb + 8 * q4 + 4 * g;
      *(u32x2*)(stg + l32 * PITCH + d0 * 2) =
          u32x2{pack2<DT>(acc[nb][4 * q4] * sc, acc[nb][4 * q4 + 1] * sc),
                pack2<DT>(acc[nb][4 * q4 + 2] * sc, acc[nb][4 * q4 + 3] * sc)};
    }
#pragma unroll
  for (int j = 0; j < 32 * CPR / 64; ++j) {
    const int r = j * (64 / CPR) + lane / CPR, ch = lane % CPR;
    buf_store16(rs, (uint32_t)((r0 + r) * row_stride + ch * 8) * 2, *(const u32x4*)(stg + r * PITCH + ch * 16));
  }
}

template <int D, int NW, int NWC = NW>
struct BwdCopy {
  using G = Geo<D>;
  // waves 0..NWC-1 issue the copies, CPW each per tile
  static constexpr int NCH = G::NCH, NBLK = G::NBLK, CPW = NBLK / NWC;
  static_assert(NBLK % NWC == 0 && NWC <= NW, "copy layout");
  uint32_t lane_src, step, row_bytes;  // per-lane source offset in a tile, offset between a wave's copies
  int wave;
  __device__ __forceinline__ BwdCopy(int wave_, int lane, int row_stride) : wave(wave_) {
    row_bytes = (uint32_t)row_stride * 2u;
    const int lrow = wave_ + NBLK * (lane / NCH), lchunk = 16 * (lane % NCH);
    lane_src = (uint32_t)lrow * row_bytes + (uint32_t)lchunk;
    step = (uint32_t)NWC * row_bytes;
  }
  // rows [64·tile, 64·tile + 64) of a slab whose last row ends `end` bytes after
  // its start; rows past the end read 0
  template <int BS>
  __device__ __forceinline__ void copy(const char* slab, uint32_t end, int tile, unsigned char* dst) const {
    const uint32_t off = (uint32_t)tile * 64u * row_bytes;
    const uint64_t base = (uint64_t)(uintptr_t)(slab + off);
    const u32x4 rs = {(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base),
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(base >> 32) & 0xffffu)),
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(end - off)), (uint32_t)kBufferFlags};
    if constexpr (NWC < NW)
      if (wave >= NWC) return;  // wave-uniform
    const uint32_t l0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(lds_addr(dst) + BS * wave));
#pragma unroll
    for (int j = 0; j < CPW; ++j) dma16(rs, l0 + BS * NWC * j, lane_src + step * j);
  }
};

// end of a step: own copies landed (vmcnt), then a bare barrier
__device__ __forceinline__ void bwd_wait_join() {
  __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));  // vmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// dQ: 8 waves x 32 query rows; loop over 64-key tiles
// ---------------------------------------------------------------------------
template <int D, int DT, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_bwd_dq_kernel(BwdParams p) {
  using G = Geo<D>;
  constexpr int NW = 8, BR = 256, BC = 64, KB = 2, NB = D / 32, KS = D / 16;
  constexpr int NBLK = G::NBLK, KBS = G::KBS, VBS = G::VBS, KT = G::KT, VT = G::VT;
  // per stage: K row image, K transposing image, V row image
  __shared__ __attribute__((aligned(16))) unsigned char kr0[KT], kr1[KT], kt0[VT], kt1[VT], vr0[KT], vr1[KT];
  // dropout: per wave and 32-key half, the buffer of the Philox words' quad transpose
  __shared__ __attribute__((aligned(16))) uint32_t dxp[DROP ? 8 * 2 * 320 : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  const int bid = blockIdx.x;
  const int item = p.xcd_remap ? (bid & 7) * (p.num_wg >> 3) + (bid >> 3) : bid;
  const int bh = __builtin_amdgcn_readfirstlane(item / p.n_qt);
  const int qt_r = __builtin_amdgcn_readfirstlane(item - bh * p.n_qt);
  const int qt = CAUSAL ? p.n_qt - 1 - qt_r : qt_r;  // causal: heaviest query tiles first
  const int Lq = p.Lq, Lk = p.Lk;
  const int i0 = qt * BR, i0w = i0 + 32 * wave;
  const int off = CAUSAL ? p.kv_off : 0;

  const char* const qslab = bwd_slab((const char*)p.q, p, T_Q, bh);
  const char* const doslab = bwd_slab((const char*)p.dout, p, T_DO, bh);
  const char* const kslab = bwd_slab((const char*)p.k, p, T_K, bh);
  const char* const vslab = bwd_slab((const char*)p.v, p, T_V, bh);
  const auto qrs = make_rsrc(qslab, bwd_end<D>(p, T_Q, Lq));
  const auto dors = make_rsrc(doslab, bwd_end<D>(p, T_DO, Lq));
  const uint32_t end_k = bwd_end<D>(p, T_K, Lk), end_v = bwd_end<D>(p, T_V, Lk);

  int n_kv = (Lk + BC - 1) / BC;
  if constexpr (CAUSAL) n_kv = min(n_kv, (min(i0 + BR, Lq) - 1 + off) / BC + 1);

  // the tile copies are issued by waves 0-3, one per SIMD (waves w and w+4 share
  // a SIMD): the other wave of each SIMD is not held up by the copy burst after
  // each barrier, as in the forward kernel
  const BwdCopy<D, NW, 4> cpk(wave, lane, p.sl[T_K]), cpv(wave, lane, p.sl[T_V]);
  auto copies = [&](int t, int st) {
    cpk.template copy<KBS>(kslab, end_k, t, st ? kr1 : kr0);
    cpk.template copy<VBS>(kslab, end_k, t, st ? kt1 : kt0);
    cpv.template copy<KBS>(vslab, end_v, t, st ? vr1 : vr0);
  };
  if (n_kv > 0) copies(0, 0);

  // Q and dO rows of this lane as B operands (column = row l%32; slots of half g
  // = head dims 16s+8g .. +7); the lane's LSE·log2(e) and Δ
  const int qrow = i0w + l32;
  u32x4 qr[KS], dr[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    qr[s] = buf_load16(qrs, (uint32_t)(qrow * p.sl[T_Q] + 16 * s + 8 * g) * 2);
    dr[s] = buf_load16(dors, (uint32_t)(qrow * p.sl[T_DO] + 16 * s + 8 * g) * 2);
  }
  // Δ = dO·O of the lane's row from the stored O (fp32, this lane's half of the
  // head dims, then the other half-wave's), and LSE·log2(e); both are also written
  // to the workspace for the dK/dV kernel, with zeros for the padding rows
  // Lq..Lq4-1 (rows past Lq read O = dO = 0 through the buffer range)
  const bool row_ok = qrow < Lq;
  float delta = 0.f;
  {
    const char* const oslab = bwd_slab((const char*)p.o, p, T_O, bh);
    const auto ors = make_rsrc(oslab, bwd_end<D>(p, T_O, Lq));
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4 ov = buf_load16(ors, (uint32_t)(qrow * p.sl[T_O] + 16 * s + 8 * g) * 2);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float2 x = unpack2<DT>(ov[e]), y = unpack2<DT>(dr[s][e]);
        delta = __builtin_fmaf(x.x, y.x, delta);
        delta = __builtin_fmaf(x.y, y.y, delta);
      }
    }
    delta = xhalf_sum(delta);
  }
  const float lse2 = row_ok ? p.lse[(int64_t)bh * Lq + qrow] * 1.44269504088896340736f : 0.f;
  if (g == 0 && qrow < p.Lq4) {
    p.ws_lse2[(int64_t)bh * p.Lq4 + qrow] = lse2;
    p.ws_delta[(int64_t)bh * p.Lq4 + qrow] = delta;
  }
  const float c = p.c;

  auto row_off = [](int rows, int BS) { return (rows % NBLK) * BS + (rows / NBLK) * 2 * D; };
  const int k_off = (l32 % NBLK) * KBS + (l32 / NBLK) * 2 * D + 16 * g;
  const int gi = lane >> 4, li = lane & 15;
  const int t_off = (4 * (gi >> 1) + (li >> 2)) * VBS + 2 * (16 * (gi & 1) + 4 * (li & 3));

  f32x16 dq[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) dq[nb] = f32x16{};

  bwd_wait_join();
  for (int t = 0; t < n_kv; ++t) {
    const int st = t & 1;
    if (t + 1 < n_kv) copies(t + 1, st ^ 1);
    const int j0 = t * BC;
    const bool active = !CAUSAL || j0 <= i0w + 31 + off;  // wave-uniform
    if (active) {
      // LLVM's single-wave MFMA interleave strategy for this body: 3.9% faster on the
      // 7B 4K shape than the default schedule, same results
      __builtin_amdgcn_iglp_opt(1);
      const unsigned char* krb = st ? kr1 : kr0;
      const unsigned char* ktb = st ? kt1 : kt0;
      const unsigned char* vrb = st ? vr1 : vr0;
      f32x16 S[KB], dP[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        S[kb] = f32x16{};
        dP[kb] = f32x16{};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          S[kb] = mfma32<DT>(lds_read16(krb + k_off + row_off(32 * kb, KBS) + 32 * s), qr[s], S[kb]);
          dP[kb] = mfma32<DT>(lds_read16(vrb + k_off + row_off(32 * kb, KBS) + 32 * s), dr[s], dP[kb]);
        }
      }
      // key of S[kb][r] within the tile: 32kb + 8(r/4) + 4g + r%4; row = qrow
      const bool need_mask = (CAUSAL && j0 + BC - 1 > i0w + off) || (j0 + BC > Lk);
      const int lim_tail = Lk - j0 - 4 * g;
      const int lim = CAUSAL ? min(qrow + off - j0 - 4 * g + 1, lim_tail) : lim_tail;
      // dropout words of the tile: lane j of a quad computes blocks 4kb + j for both halves kb,
      // the quad transposes each half's words
      uint32_t words[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
      if constexpr (DROP) {
        const int j = lane & 3;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const u32x4 mine =
              drop_block((j0 + 32 * kb + 16 * (j >> 1) + 8 * (j & 1) + 4 * g) >> 2, qrow >> 2, bh, p.seed_lo,
                         p.seed_hi);
          // quad transpose through LDS, as in the forward kernel: word i of lane (quad q, j)
          // at dword 20q + 4i + j of this wave's buffer for half kb, then 16 bytes at 20q + 4j
          uint32_t* const xb = dxp + (wave * 2 + kb) * 320 + 20 * (lane >> 2);
#pragma unroll
          for (int i = 0; i < 4; ++i) xb[4 * i + j] = mine[i];
          const u32x4 got = *(const u32x4*)(xb + 4 * j);
#pragma unroll
          for (int i = 0; i < 4; ++i) words[4 * kb + i] = got[i];
        }
      }
      u32x4 db[KB][2];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        uint32_t* wd = words + 4 * kb;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          // dropout words of registers 8h..8h+7
          uint32_t dwd[2] = {0u, 0u};
          if constexpr (DROP) {
            dwd[0] = wd[2 * h];
            dwd[1] = wd[2 * h + 1];
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float ds[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int r = 8 * h + 2 * e + u;
              float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][r], c, -lse2));
              if (need_mask) {
                const int ko = 32 * kb + 8 * (r >> 2) + (r & 3);
                pr = ko >= lim ? 0.f : pr;
              }
              float dp = dP[kb][r];
              if constexpr (DROP) {
                // dP of the weight before dropout: the dropped-out weight's gradient times its factor
                const uint32_t byte = (dwd[e >> 1] >> (8 * (2 * (e & 1) + u))) & 0xffu;
                dp = byte < p.drop_t ? dp * p.drop_scale : 0.f;
              }
              ds[u] = pr * (dp - delta);
            }
            db[kb][h][e] = pack2<DT>(ds[0], ds[1]);
          }
        }
      }
      // dQᵀ += Kᵀ·dSᵀ: A = 8 keys of one head dim (two transposing reads)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const unsigned char* a0 = ktb + t_off + 64 * nb;
            const u32x2 lo = lds_read_tr(a0 + row_off(32 * kb + 16 * h, VBS));
            const u32x2 hi = lds_read_tr(a0 + row_off(32 * kb + 16 * h + 8, VBS));
            dq[nb] = mfma32<DT>(u32x4{lo[0], lo[1], hi[0], hi[1]}, db[kb][h], dq[nb]);
          }
    }
    bwd_wait_join();
  }

  // epilogue: dQ = scale·dQᵀ; lane holds dims 32nb + 8(r/4) + 4g + r%4 of row qrow.
  // The wave's 32 rows go row-major through LDS (free since the last barrier)
  // and out as whole rows, 16 bytes per lane (see stage_rows_out)
  const auto ors = make_rsrc(bwd_slab((char*)p.dq, p, T_DQ, bh), bwd_end<D>(p, T_DQ, Lq));
  if constexpr (D == 128) {
    // waves 0-3 two to a transposing K stage, waves 4-7 one to each row stage
    static_assert(2 * 32 * (2 * D + 16) <= VT && 32 * (2 * D + 16) <= KT, "staging fits");
    unsigned char* const stg = wave < 4 ? (wave < 2 ? kt0 : kt1) + (wave & 1) * 32 * (2 * D + 16)
                                        : (wave == 4 ? kr0 : wave == 5 ? kr1 : wave == 6 ? vr0 : vr1);
    stage_rows_out<D, DT>(dq, p.scale, stg, lane, ors, i0w, p.sl[T_DQ]);
  } else {
    // (at D = 64 the six stages cannot take eight waves' rows: direct 8-byte stores)
    const float sc = p.scale;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * nb + 8 * q4 + 4 * g;
        const u32x2 w = {pack2<DT>(dq[nb][4 * q4] * sc, dq[nb][4 * q4 + 1] * sc),
                         pack2<DT>(dq[nb][4 * q4 + 2] * sc, dq[nb][4 * q4 + 3] * sc)};
        buf_store8(ors, (uint32_t)(qrow * p.sl[T_DQ] + d0) * 2, w);  // rows >= Lq are dropped
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV: 4 waves x 32 keys; loop over 64-row query tiles
// ---------------------------------------------------------------------------
template <int D, int DT, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void fa_bwd_dkdv_kernel(BwdParams p) {
  using G = Geo<D>;
  constexpr int NW = 4, BKV = 128, BQ = 64, QB = 2, NB = D / 32, KS = D / 16;
  constexpr int NBLK = G::NBLK, KBS = G::KBS, VBS = G::VBS, KT = G::KT, VT = G::VT;
  // per stage: Q row image, Q transposing image, dO row image, dO transposing image
  __shared__ __attribute__((aligned(16))) unsigned char qr0[KT], qr1[KT], qt0[VT], qt1[VT];
  __shared__ __attribute__((aligned(16))) unsigned char or0[KT], or1[KT], ot0[VT], ot1[VT];
  // per stage: LSE·log2(e) and Δ of the tile's 64 rows (a 1 KB copy each; the
  // first 256 bytes are used)
  __shared__ __attribute__((aligned(16))) float ls0[256], ls1[256], de0[256], de1[256];
  // dropout: per wave and 32-row half, the exchange buffer of the Philox blocks (64 lanes x 16 bytes)
  __shared__ __attribute__((aligned(16))) uint32_t dxk[DROP ? 4 * 2 * 256 : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  const int bid = blockIdx.x;
  const int item = p.xcd_remap ? (bid & 7) * (p.num_wg >> 3) + (bid >> 3) : bid;
  const int bh = __builtin_amdgcn_readfirstlane(item / p.n_kt);
  const int kt = __builtin_amdgcn_readfirstlane(item - bh * p.n_kt);  // causal: low tiles see most rows
  const int Lq = p.Lq, Lk = p.Lk;
  const int j0 = kt * BKV, j0w = j0 + 32 * wave;
  const int off = CAUSAL ? p.kv_off : 0;

  const char* const qslab = bwd_slab((const char*)p.q, p, T_Q, bh);
  const char* const doslab = bwd_slab((const char*)p.dout, p, T_DO, bh);
  const char* const kslab = bwd_slab((const char*)p.k, p, T_K, bh);
  const char* const vslab = bwd_slab((const char*)p.v, p, T_V, bh);
  const auto krs = make_rsrc(kslab, bwd_end<D>(p, T_K, Lk));
  const auto vrs = make_rsrc(vslab, bwd_end<D>(p, T_V, Lk));
  const uint32_t end_q = bwd_end<D>(p, T_Q, Lq), end_do = bwd_end<D>(p, T_DO, Lq);

  // query tiles that see any key of this workgroup: rows i >= j0 - off (causal)
  const int n_q = (Lq + BQ - 1) / BQ;
  const int t_b = CAUSAL ? max(0, j0 - off) / BQ : 0;

  const BwdCopy<D, NW> cpq(wave, lane, p.sl[T_Q]), cpo(wave, lane, p.sl[T_DO]);
  // row statistics of tile t: rows past the padded end read 0
  auto copy_stats = [&](const float* base, int t, float* dst) {
    const uint64_t a = (uint64_t)(uintptr_t)(base + (int64_t)bh * p.Lq4 + (int64_t)t * BQ);
    const u32x4 rs = {(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu)),
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(p.Lq4 - t * BQ) * 4u)),
                      (uint32_t)kBufferFlags};
    dma16(rs, (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(dst)), (uint32_t)(16 * lane));
  };
  auto copies = [&](int t, int st) {
    cpq.template copy<KBS>(qslab, end_q, t, st ? qr1 : qr0);
    cpq.template copy<VBS>(qslab, end_q, t, st ? qt1 : qt0);
    cpo.template copy<KBS>(doslab, end_do, t, st ? or1 : or0);
    cpo.template copy<VBS>(doslab, end_do, t, st ? ot1 : ot0);
    if (wave == 0) copy_stats(p.ws_lse2, t, st ? ls1 : ls0);
    if (wave == 1) copy_stats(p.ws_delta, t, st ? de1 : de0);
  };
  if (t_b < n_q) copies(t_b, 0);

  // K and V rows of this lane's key as B operands (column = key l%32; slots of
  // half g = head dims 16s+8g .. +7); keys past Lk read 0
  const int key = j0w + l32;
  u32x4 kr[KS], vr[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    kr[s] = buf_load16(krs, (uint32_t)(key * p.sl[T_K] + 16 * s + 8 * g) * 2);
    vr[s] = buf_load16(vrs, (uint32_t)(key * p.sl[T_V] + 16 * s + 8 * g) * 2);
  }
  const float c = p.c;

  auto row_off = [](int rows, int BS) { return (rows % NBLK) * BS + (rows / NBLK) * 2 * D; };
  const int k_off = (l32 % NBLK) * KBS + (l32 / NBLK) * 2 * D + 16 * g;
  const int gi = lane >> 4, li = lane & 15;
  const int t_off = (4 * (gi >> 1) + (li >> 2)) * VBS + 2 * (16 * (gi & 1) + 4 * (li & 3));

  f32x16 dv[NB], dk[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    dv[nb] = f32x16{};
    dk[nb] = f32x16{};
  }

  // One 64-row query tile.  In S and dP the lane holds key l%32 and rows
  // 32qb + 8(r/4) + 4g + r%4 of the tile.  Half qb: S = Q·Kᵀ and dP = dO·Vᵀ, the
  // weights and dS in registers, then dVᵀ += dOᵀ·P and dKᵀ += Qᵀ·dS.
  auto products = [&](int qb, const unsigned char* qrb, const unsigned char* orb, f32x16& S, f32x16& dP) {
    S = f32x16{};
    dP = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      S = mfma32<DT>(lds_read16(qrb + k_off + row_off(32 * qb, KBS) + 32 * s), kr[s], S);
      dP = mfma32<DT>(lds_read16(orb + k_off + row_off(32 * qb, KBS) + 32 * s), vr[s], dP);
    }
  };
  // The weights and dS of one register pair (h, e) of half qb: registers
  // r = 8h + 2e + u, rows 32qb + 8(r/4) + 4g + r%4 of the tile, this lane's key.
  // dw: the dropout words of rows group a = 2h + e/2 (DROP only).
  auto valu_pair = [&](auto MASK, int qb, int h, int e, int i0, const f32x16& S, const f32x16& dP,
                       const f32x4 (&ls)[4], const f32x4 (&de)[4], const u32x4& dw, u32x4 (&pb)[2],
                       u32x4 (&db)[2]) {
    float pp[2], ds[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r = 8 * h + 2 * e + u;
      float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r], c, -ls[r >> 2][r & 3]));
      if constexpr (decltype(MASK)::value) {
        // key j0w + l32 visible to row i iff j <= i + off
        const int row = i0 + 32 * qb + 8 * (r >> 2) + 4 * g + (r & 3);
        pr = key > row + off ? 0.f : pr;
      }
      float dp = dP[r];
      if constexpr (DROP) {
        const uint32_t byte = (dw[2 * (e & 1) + u] >> (8 * (key & 3))) & 0xffu;
        const float f = byte < p.drop_t ? p.drop_scale : 0.f;
        pp[u] = pr * f;   // the dropped-out weight multiplies dO in dV
        dp *= f;          // dP of the weight before dropout
      } else {
        pp[u] = pr;
      }
      ds[u] = pr * (dp - de[r >> 2][r & 3]);
    }
    pb[h][e] = pack2<DT>(pp[0], pp[1]);
    db[h][e] = pack2<DT>(ds[0], ds[1]);
  };
  auto load_stats = [&](int qb, const float* lsb, const float* deb, f32x4 (&ls)[4], f32x4 (&de)[4]) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      ls[a] = *(const f32x4*)(lsb + 32 * qb + 8 * a + 4 * g);
      de[a] = *(const f32x4*)(deb + 32 * qb + 8 * a + 4 * g);
    }
  };
  // Dropout blocks of half qb: blocks x = 2h + a cover rows i0 + 32qb + 16h + 8a + 4g +
  // 0..3 of this lane's key.  The four lanes of a quad share the key block, so lane
  // j computes block j and the quad exchanges all four words of each block.
  auto drop_half = [&](int qb, int i0, u32x4 (&blk)[4]) {
    const int j = lane & 3, h = j >> 1, a = j & 1;
    const u32x4 mine = drop_block(key >> 2, (i0 + 32 * qb + 16 * h + 8 * a + 4 * g) >> 2, bh, p.seed_lo, p.seed_hi);
    // the exchange goes through LDS: each lane stores its block (16 bytes, the wave's
    // 64 lanes contiguous), then reads its quad's four blocks (the quad's lanes read
    // the same addresses: broadcasts)
    u32x4* const xb = (u32x4*)(dxk + (wave * 2 + qb) * 256) + 4 * (lane >> 2);
    xb[j] = mine;
#pragma unroll
    for (int x = 0; x < 4; ++x) blk[x] = xb[x];
  };
  // dVᵀ += dOᵀ·P and dKᵀ += Qᵀ·dS for register half h, dims block nb of half qb
  auto grad_mfma = [&](int qb, int h, int nb, const u32x4 (&pb)[2], const u32x4 (&db)[2],
                       const unsigned char* qtb, const unsigned char* otb) {
    const unsigned char* ao = otb + t_off + 64 * nb;
    const u32x2 olo = lds_read_tr(ao + row_off(32 * qb + 16 * h, VBS));
    const u32x2 ohi = lds_read_tr(ao + row_off(32 * qb + 16 * h + 8, VBS));
    dv[nb] = mfma32<DT>(u32x4{olo[0], olo[1], ohi[0], ohi[1]}, pb[h], dv[nb]);
    const unsigned char* aq = qtb + t_off + 64 * nb;
    const u32x2 qlo = lds_read_tr(aq + row_off(32 * qb + 16 * h, VBS));
    const u32x2 qhi = lds_read_tr(aq + row_off(32 * qb + 16 * h + 8, VBS));
    dk[nb] = mfma32<DT>(u32x4{qlo[0], qlo[1], qhi[0], qhi[1]}, db[h], dk[nb]);
  };
  // One 64-row query tile, software-pipelined over its two 32-row halves so that
  // with one wave per SIMD the MFMAs of one stage overlap the VALU work of
  // another (the program order fixes the interleave; at D = 128 scheduling
  // barriers keep it, measured 8% faster there and 2.5% slower at D = 64):
  //   S0, dP0  |  S1, dP1 (MFMA) with weights/dS of half 0 (VALU)
  //            |  dV, dK of half 0 (MFMA) with weights/dS of half 1 (VALU)
  //            |  dV, dK of half 1 (MFMA)
  // In S and dP the lane holds key l%32 and rows 32qb + 8(r/4) + 4g + r%4.
  constexpr int PAIRS = 8;                    // (h, e) register pairs per half
  constexpr int PPS = PAIRS / KS;             // pairs per S/dP step
  constexpr int GSTEPS = 2 * NB;              // (h, nb) dV/dK steps per half
  constexpr int PPG = PAIRS / GSTEPS;         // pairs per dV/dK step
  static_assert(PAIRS % KS == 0 && PAIRS % GSTEPS == 0, "interleave");
  auto tile_body = [&](auto MASK, int i0, const unsigned char* qrb, const unsigned char* qtb,
                       const unsigned char* orb, const unsigned char* otb, const float* lsb, const float* deb) {
    f32x16 S0, dP0, S1 = f32x16{}, dP1 = f32x16{};
    products(0, qrb, orb, S0, dP0);
    u32x4 pb0[2], db0[2], pb1[2], db1[2];
    {
      f32x4 ls[4], de[4];
      load_stats(0, lsb, deb, ls, de);
      u32x4 blk[4];
      if constexpr (DROP) drop_half(0, i0, blk);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        S1 = mfma32<DT>(lds_read16(qrb + k_off + row_off(32, KBS) + 32 * s), kr[s], S1);
        dP1 = mfma32<DT>(lds_read16(orb + k_off + row_off(32, KBS) + 32 * s), vr[s], dP1);
#pragma unroll
        for (int j = 0; j < PPS; ++j) {
          const int pr = s * PPS + j, h = pr >> 2, e = pr & 3;
          valu_pair(MASK, 0, h, e, i0, S0, dP0, ls, de, blk[2 * h + (e >> 1)], pb0, db0);
        }
        if constexpr (D == 128) __builtin_amdgcn_sched_barrier(0);
      }
    }
    {
      f32x4 ls[4], de[4];
      load_stats(1, lsb, deb, ls, de);
      u32x4 blk[4];
      if constexpr (DROP) drop_half(1, i0, blk);
#pragma unroll
      for (int st = 0; st < GSTEPS; ++st) {
        grad_mfma(0, st / NB, st % NB, pb0, db0, qtb, otb);
#pragma unroll
        for (int j = 0; j < PPG; ++j) {
          const int pr = st * PPG + j, h = pr >> 2, e = pr & 3;
          valu_pair(MASK, 1, h, e, i0, S1, dP1, ls, de, blk[2 * h + (e >> 1)], pb1, db1);
        }
        if constexpr (D == 128) __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int st = 0; st < GSTEPS; ++st) grad_mfma(1, st / NB, st % NB, pb1, db1, qtb, otb);
  };

  bwd_wait_join();
  for (int t = t_b; t < n_q; ++t) {
    const int st = (t - t_b) & 1;
    if (t + 1 < n_q) copies(t + 1, st ^ 1);
    const int i0 = t * BQ;
    // a wave whose keys no row of this tile sees skips it (wave-uniform)
    const bool active = !CAUSAL || j0w <= i0 + BQ - 1 + off;
    if (active) {
      const unsigned char* qrb = st ? qr1 : qr0;
      const unsigned char* qtb = st ? qt1 : qt0;
      const unsigned char* orb = st ? or1 : or0;
      const unsigned char* otb = st ? ot1 : ot0;
      const float* lsb = st ? ls1 : ls0;
      const float* deb = st ? de1 : de0;
      // causal: every tile takes the masked body (one compare and select per
      // element; a second, unmasked copy of the body for tiles below the diagonal
      // made the compiler spill)
      if constexpr (CAUSAL)
        tile_body(std::true_type{}, i0, qrb, qtb, orb, otb, lsb, deb);
      else
        tile_body(std::false_type{}, i0, qrb, qtb, orb, otb, lsb, deb);
    }
    bwd_wait_join();
  }

  // epilogue: lane holds dims 32nb + 8(r/4) + 4g + r%4 of key `key`; each wave's
  // 32 rows of dK and of dV go row-major through two LDS stages (free since the
  // last barrier) and out as whole rows (see stage_rows_out)
  const auto dkrs = make_rsrc(bwd_slab((char*)p.dk, p, T_DK, bh), bwd_end<D>(p, T_DK, Lk));
  const auto dvrs = make_rsrc(bwd_slab((char*)p.dv, p, T_DV, bh), bwd_end<D>(p, T_DV, Lk));
  static_assert(32 * (2 * D + 16) <= KT, "staging fits");
  unsigned char* const stk = wave == 0 ? qr0 : wave == 1 ? qr1 : wave == 2 ? or0 : or1;
  unsigned char* const stv = wave == 0 ? qt0 : wave == 1 ? qt1 : wave == 2 ? ot0 : ot1;
  stage_rows_out<D, DT>(dk, p.scale, stk, lane, dkrs, j0w, p.sl[T_DK]);
  stage_rows_out<D, DT>(dv, 1.0f, stv, lane, dvrs, j0w, p.sl[T_DV]);
}

// ---------------------------------------------------------------------------
// dK/dV with two waves per key block: 8 waves = 128 keys.  Waves w and w + 4
// (one SIMD) share keys 32w .. 32w + 31 of the workgroup and split the four
// products of each 64-row query tile: wave w makes S = Q·Kᵀ, the weights P and
// dVᵀ += dOᵀ·P; wave w + 4 makes dP = dO·Vᵀ, dS = P(dP − Δ) and dKᵀ += Qᵀ·dS.
// The weights pass from one to the other through LDS as the rounded matrix-core
// operand of dV (16 bytes per lane and 16-row group), between the two joins of a
// step.  Each wave keeps one key operand and one accumulator (K and dV, or V and
// dK): half the registers of one wave doing all four products, so two waves fit
// on a SIMD and one's VALU work runs beside the other's MFMAs.
// ---------------------------------------------------------------------------
// the middle of a step: this wave's LDS writes are done, then a bare barrier
__device__ __forceinline__ void bwd_lds_join() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D, int DT, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_bwd_dkdv2_kernel(BwdParams p) {
  using G = Geo<D>;
  constexpr int NW = 8, BKV = 128, BQ = 64, NB = D / 32, KS = D / 16;
  constexpr int NBLK = G::NBLK, KBS = G::KBS, VBS = G::VBS, KT = G::KT, VT = G::VT;
  // per stage: Q row image, Q transposing image, dO row image, dO transposing image
  __shared__ __attribute__((aligned(16))) unsigned char qr0[KT], qr1[KT], qt0[VT], qt1[VT];
  __shared__ __attribute__((aligned(16))) unsigned char or0[KT], or1[KT], ot0[VT], ot1[VT];
  // per stage: LSE·log2(e) and Δ of the tile's 64 rows (a 1 KB copy each; the
  // first 256 bytes are used)
  __shared__ __attribute__((aligned(16))) float ls0[256], ls1[256], de0[256], de1[256];
  // the tile's weights, per key block, 32-row half qb and 16-row group h: [block][2qb + h][lane]
  __shared__ __attribute__((aligned(16))) u32x4 xw[4][4][64];
  static_assert(2 * (2 * KT + 2 * VT) + 4 * 1024 + 4 * 4 * 64 * 16 <= 163840, "one workgroup per CU");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave & 3;          // key block
  const bool mk = wave < NW / 2;    // makes S, P, dV (else dP, dS, dK); wave-uniform
  const int l32 = lane & 31, g = lane >> 5;

  const int bid = blockIdx.x;
  const int item = p.xcd_remap ? (bid & 7) * (p.num_wg >> 3) + (bid >> 3) : bid;
  const int bh = __builtin_amdgcn_readfirstlane(item / p.n_kt);
  const int kt = __builtin_amdgcn_readfirstlane(item - bh * p.n_kt);  // causal: low tiles see most rows
  const int Lq = p.Lq, Lk = p.Lk;
  const int j0 = kt * BKV, j0w = j0 + 32 * kw;
  const int off = CAUSAL ? p.kv_off : 0;

  const char* const qslab = bwd_slab((const char*)p.q, p, T_Q, bh);
  const char* const doslab = bwd_slab((const char*)p.dout, p, T_DO, bh);
  const uint32_t end_q = bwd_end<D>(p, T_Q, Lq), end_do = bwd_end<D>(p, T_DO, Lq);

  // query tiles that see any key of this workgroup: rows i >= j0 - off (causal)
  const int n_q = (Lq + BQ - 1) / BQ;
  const int t_b = CAUSAL ? max(0, j0 - off) / BQ : 0;

  const BwdCopy<D, NW> cpq(wave, lane, p.sl[T_Q]), cpo(wave, lane, p.sl[T_DO]);
  // row statistics of tile t: rows past the padded end read 0
  auto copy_stats = [&](const float* base, int t, float* dst) {
    const uint64_t a = (uint64_t)(uintptr_t)(base + (int64_t)bh * p.Lq4 + (int64_t)t * BQ);
    const u32x4 rs = {(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu)),
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(p.Lq4 - t * BQ) * 4u)),
                      (uint32_t)kBufferFlags};
    dma16(rs, (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(dst)), (uint32_t)(16 * lane));
  };
  auto copies = [&](int t, int st) {
    cpq.template copy<KBS>(qslab, end_q, t, st ? qr1 : qr0);
    cpq.template copy<VBS>(qslab, end_q, t, st ? qt1 : qt0);
    cpo.template copy<KBS>(doslab, end_do, t, st ? or1 : or0);
    cpo.template copy<VBS>(doslab, end_do, t, st ? ot1 : ot0);
    if (wave == 0) copy_stats(p.ws_lse2, t, st ? ls1 : ls0);
    if (wave == 1) copy_stats(p.ws_delta, t, st ? de1 : de0);
  };
  if (t_b < n_q) copies(t_b, 0);

  // this wave's key rows as B operands (column = key l%32; slots of half g = head
  // dims 16s+8g .. +7): K for S, or V for dP; keys past Lk read 0
  const int key = j0w + l32;
  const int T_B = mk ? T_K : T_V;
  const auto brs = make_rsrc(bwd_slab((const char*)(mk ? p.k : p.v), p, T_B, bh), bwd_end<D>(p, T_B, Lk));
  u32x4 br[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) br[s] = buf_load16(brs, (uint32_t)(key * p.sl[T_B] + 16 * s + 8 * g) * 2);
  const float c = p.c;

  auto row_off = [](int rows, int BS) { return (rows % NBLK) * BS + (rows / NBLK) * 2 * D; };
  const int k_off = (l32 % NBLK) * KBS + (l32 / NBLK) * 2 * D + 16 * g;
  const int gi = lane >> 4, li = lane & 15;
  const int t_off = (4 * (gi >> 1) + (li >> 2)) * VBS + 2 * (16 * (gi & 1) + 4 * (li & 3));

  // dV (waves that make the weights) or dK (the others)
  f32x16 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16{};

  // S (or dP) of both 32-row halves of a tile: the lane holds key l%32 and rows
  // 32qb + 8(r/4) + 4g + r%4 of the tile (rows from the row image `rb`)
  auto products = [&](const unsigned char* rb, f32x16 (&X)[2]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      X[qb] = f32x16{};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        X[qb] = mfma32<DT>(lds_read16(rb + k_off + row_off(32 * qb, KBS) + 32 * s), br[s], X[qb]);
    }
  };
  // acc[nb] += Aᵀ·B over the tile's 64 rows: A from the transposing image `tb`
  // (dims block nb, rows 32qb + 16h .. +15), B = x[qb][h] (this lane's key, those rows)
  auto grads = [&](const unsigned char* tb, const u32x4 (&x)[2][2]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const unsigned char* a = tb + t_off + 64 * nb;
          const u32x2 lo = lds_read_tr(a + row_off(32 * qb + 16 * h, VBS));
          const u32x2 hi = lds_read_tr(a + row_off(32 * qb + 16 * h + 8, VBS));
          acc[nb] = mfma32<DT>(u32x4{lo[0], lo[1], hi[0], hi[1]}, x[qb][h], acc[nb]);
        }
  };
  // Dropout words of half qb for this lane's key: block x = 2h + a covers rows
  // i0 + 32qb + 16h + 8a + 4g + 0..3.  The four lanes of a quad share the key block,
  // so lane j computes block j and the quad exchanges them through LDS (in this key
  // block's weight buffer, slot 2qb, which the weights of the half overwrite after).
  auto drop_half = [&](int qb, int i0, u32x4 (&blk)[4]) {
    const int j = lane & 3, h = j >> 1, a = j & 1;
    const u32x4 mine = drop_block(key >> 2, (i0 + 32 * qb + 16 * h + 8 * a + 4 * g) >> 2, bh, p.seed_lo, p.seed_hi);
    u32x4* const xb = &xw[kw][2 * qb][0] + 4 * (lane >> 2);
    xb[j] = mine;
#pragma unroll
    for (int x = 0; x < 4; ++x) blk[x] = xb[x];
  };
  // the weights P = 2^(S·c − LSE₂) of the tile, packed as the B operand of dV
  // (registers r = 8h + 2e + u of half qb: x[qb][h][e]); MASK: causal, keys right of
  // a row's diagonal get 0.  The other wave of the key block gets them in the same
  // form; with dropout x holds the kept weights times 1/(1 − p), and the other wave
  // gets the weights before dropout with the sign bit of each dropped one set.
  auto weights = [&](auto MASK, int i0, const f32x16 (&S)[2], const float* lsb, u32x4 (&x)[2][2]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x4 ls[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) ls[a] = *(const f32x4*)(lsb + 32 * qb + 8 * a + 4 * g);
      u32x4 blk[4];
      if constexpr (DROP) drop_half(qb, i0, blk);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 xo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float pr[2];
          bool kept[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int r = 8 * h + 2 * e + u;
            pr[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[qb][r], c, -ls[r >> 2][r & 3]));
            if constexpr (decltype(MASK)::value) {
              const int row = i0 + 32 * qb + 8 * (r >> 2) + 4 * g + (r & 3);
              pr[u] = key > row + off ? 0.f : pr[u];
            }
            if constexpr (DROP)
              kept[u] = ((blk[2 * h + (e >> 1)][2 * (e & 1) + u] >> (8 * (key & 3))) & 0xffu) < p.drop_t;
          }
          if constexpr (DROP) {
            x[qb][h][e] = pack2<DT>(kept[0] ? pr[0] * p.drop_scale : 0.f, kept[1] ? pr[1] * p.drop_scale : 0.f);
            xo[e] = pack2<DT>(pr[0], pr[1]) | (kept[0] ? 0u : 0x8000u) | (kept[1] ? 0u : 0x80000000u);
          } else {
            x[qb][h][e] = pack2<DT>(pr[0], pr[1]);
          }
        }
        xw[kw][2 * qb + h][lane] = DROP ? xo : x[qb][h];
      }
    }
  };
  // dS = P(dP − Δ) of the tile from the weights as rounded, packed like the weights
  // (with dropout dS = P(dP·m − Δ), m the kept weight's scale or 0)
  auto dscores = [&](const f32x16 (&dP)[2], const float* deb, u32x4 (&x)[2][2]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x4 de[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) de[a] = *(const f32x4*)(deb + 32 * qb + 8 * a + 4 * g);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 pw = xw[kw][2 * qb + h][lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * h + 2 * e;
          float dp0 = dP[qb][r], dp1 = dP[qb][r + 1];
          uint32_t w = pw[e];
          if constexpr (DROP) {
            dp0 *= (w & 0x8000u) ? 0.f : p.drop_scale;
            dp1 *= (w & 0x80000000u) ? 0.f : p.drop_scale;
            w &= 0x7fff7fffu;
          }
          const float2 pr = unpack2<DT>(w);
          x[qb][h][e] = pack2<DT>(pr.x * (dp0 - de[r >> 2][r & 3]), pr.y * (dp1 - de[(r + 1) >> 2][(r + 1) & 3]));
        }
      }
    }
  };

  bwd_wait_join();
  for (int t = t_b; t < n_q; ++t) {
    const int st = (t - t_b) & 1;
    if (t + 1 < n_q) copies(t + 1, st ^ 1);
    const int i0 = t * BQ;
    // Every key block takes every tile from the first one that any of the
    // workgroup's keys sees: a block that no row of the tile sees gets all-zero
    // weights from the mask, which adds nothing (skipping it made the compiler
    // copy the accumulators between registers on every step).  One code path for
    // both roles, which differ in the operands and the VALU step, for the same
    // reason.
    f32x16 X[2];
    products(mk ? (st ? qr1 : qr0) : (st ? or1 : or0), X);  // S, or dP
    u32x4 x[2][2];
    if (mk) {
      // causal: only tiles that reach right of some row's diagonal are masked
      if (CAUSAL && j0w + 31 > i0 + off)
        weights(std::true_type{}, i0, X, st ? ls1 : ls0, x);
      else
        weights(std::false_type{}, i0, X, st ? ls1 : ls0, x);
    }
    bwd_lds_join();
    if (!mk) dscores(X, st ? de1 : de0, x);
    grads(mk ? (st ? ot1 : ot0) : (st ? qt1 : qt0), x);  // dVᵀ += dOᵀ·P, or dKᵀ += Qᵀ·dS
    bwd_wait_join();
  }

  // epilogue: lane holds dims 32nb + 8(r/4) + 4g + r%4 of key `key`; each wave's
  // 32 rows of dV or dK go row-major through its own LDS buffer (free since the
  // last barrier) and out as whole rows (see stage_rows_out)
  static_assert(32 * (2 * D + 16) <= KT, "staging fits");
  unsigned char* const stg = wave == 0 ? qt0 : wave == 1 ? qt1 : wave == 2 ? ot0 : wave == 3 ? ot1
                           : wave == 4 ? qr0 : wave == 5 ? qr1 : wave == 6 ? or0 : or1;
  const int T_G = mk ? T_DV : T_DK;
  const auto grs = make_rsrc(bwd_slab((char*)(mk ? p.dv : p.dk), p, T_G, bh), bwd_end<D>(p, T_G, Lk));
  stage_rows_out<D, DT>(acc, mk ? 1.0f : p.scale, stg, lane, grs, j0w, p.sl[T_G]);
}

}  // namespace fa355
