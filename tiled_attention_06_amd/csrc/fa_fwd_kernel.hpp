// Fused, tiled attention forward kernel for gfx950 (MI355X).
//
// Pages cited (title, then the section on that page):
//   [DF] "FlashAttention数据流优化：MI50显存与带宽瓶颈实战"  (kwkr.cn/news/544806)
//   [AI] "AIInfra笔记01"                                   (kwkr.cn/news/547341)
//   [OP] "FlashAttention优化原理与工程实践"                (lbrq.cn/news/50349)
//
// One workgroup = 4 waves = 128 query rows of one (batch, head); each wave owns
// 32 rows.  The method ([DF §2.2], first and second layers; [OP §2.1], a loop
// over key blocks inside a loop over query blocks):
//   * the Q tile is loaded once and stays in VGPRs as MFMA operands;
//   * K and V tiles of BC keys are copied HBM -> LDS by the buffer unit itself
//     (buffer_load ... lds, no VGPR staging), into two K and two V buffers: the
//     copy of K tile j+2 and V tile j+1 runs while tile j is computed ([DF §2.3]
//     prefetch of the next block);
//   * Sᵀ = K·Qᵀ runs on v_mfma_f32_32x32x16_{bf16,f16} with fp32 accumulation, so
//     each lane holds 32 keys of ONE query row and the row max / row sums are
//     in-lane plus one v_permlane32_swap with the other half-wave;
//   * software pipelining inside each wave: the MFMAs of Sᵀ for tile j+1 are
//     issued before the softmax of tile j, so the VALU work of one tile runs
//     under the matrix work of the next;
//   * online softmax in base 2 ([DF §2.2], second layer): t = S·(|scale|·log2 e),
//     running max m and sums, exp on v_exp_f32.  The running max only moves when a
//     tile's max exceeds it by more than TAU (then the partial output and sums
//     are rescaled by 2^(m_old − m_new)); otherwise weights up to 2^TAU are
//     accumulated against the older max, which leaves O and LSE exact because
//     numerator and denominators share that max;
//   * P is rounded to the input type and fed straight from the Sᵀ accumulator
//     layout into Oᵀ = Vᵀ·Pᵀ; V stays row-major in LDS and its MFMA operand is
//     read with ds_read_b64_tr_b16 (a 4-key x 16-dim block per 16 lanes,
//     delivered transposed);
//   * epilogue: O / l_r (l_r: sum of the rounded weights that multiplied V),
//     rounded to the input type; lse = (m + log2 l_f)·ln 2 (l_f: fp32 sum).
// Causal ([DF §4.1] flag): key tiles above a workgroup's last row are never
// loaded or computed, a wave skips tiles above its own rows, and only tiles that
// cross the diagonal or the end of the keys pay for the mask.
//
// MFMA 32x32 accumulator layout used throughout: lane l, register r hold
// C[row = 8*(r/4) + 4*(l/32) + r%4][col = l%32].  A-operand lane l holds row l%32
// and B-operand lane l column l%32, each with 8 contraction elements; since A and
// B assign contraction indices to (lane half, element) identically, any
// assignment of head dims / keys to those slots that is the same for every lane
// gives the same product.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

enum { DT_F16 = 0, DT_BF16 = 1 };

// Buffer resource word 3 for gfx9-family raw buffers: 32-bit data format, so
// untyped loads/stores work and out-of-range accesses read 0 / are dropped.
constexpr int kBufferFlags = 0x00020000;

// Running-max slack in log2 units: weights can reach 2^TAU before a rescale.
constexpr float TAU = 8.0f;

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

// max / sum of a value over lanes l and l^32 (every lane gets the result)
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ u32x4 lds_read16(const unsigned char* p) { return *(const u32x4*)p; }

// 4 keys x 1 head dim per lane from a row-major V tile (see the kernel comment).
__device__ __forceinline__ u32x2 lds_read_tr(const unsigned char* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Tile geometry shared by the kernel and the host launcher.
template <int D>
struct Geo {
  static constexpr int NW = 4;                 // waves per workgroup
  static constexpr int NT = 64 * NW;           // threads per workgroup
  static constexpr int BR = 32 * NW;           // query rows per workgroup
  static constexpr int BC = 64;                // keys per K/V tile
  static constexpr int KB = BC / 32;           // 32-key blocks of a tile (Sᵀ MFMA row blocks)
  static constexpr int NB = D / 32;            // 32-dim blocks of the output (Oᵀ MFMA row blocks)
  static constexpr int KS = D / 16;            // contraction steps of QKᵀ
  static constexpr int NCH = D / 8;            // 16-byte chunks per K/V row
  // LDS row pitches in 16-byte chunks: the padding chunks spread the rows of one
  // MFMA operand read over distinct banks.
  static constexpr int KPC = NCH + 1;
  static constexpr int VPC = NCH + 2;
  static constexpr int KP = 16 * KPC, VP = 16 * VPC;  // bytes
  static constexpr int KT = BC * KP, VT = BC * VP;    // bytes per K / V tile
  static constexpr int KI = BC * KPC / 64, VI = BC * VPC / 64;  // 1 KB copy instructions per tile
  static constexpr int LDS = 2 * KT + 2 * VT;
  static_assert(BC * KPC % 64 == 0 && BC * VPC % 64 == 0, "tiles are whole 1 KB copy blocks");
  static_assert(LDS <= 81920, "two workgroups per CU");
};

template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_fwd_kernel(FwdParams p) {
  using G = Geo<D>;
  constexpr int BC = G::BC, KB = G::KB, NB = G::NB, KS = G::KS, NCH = G::NCH;
  constexpr int KP = G::KP, VP = G::VP, KT = G::KT, VT = G::VT;
  constexpr float NEG_INF = -__builtin_inff();
  __shared__ __attribute__((aligned(1024))) unsigned char smem[G::LDS];
  unsigned char* const kbuf0 = smem;
  unsigned char* const vbuf0 = smem + 2 * KT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  // ---- work item: (batch*head, query tile); heaviest causal tiles first, and
  // consecutive items (all query tiles of one head) on one XCD, whose L2 then
  // serves the K/V re-reads of that head.
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

  // ---- HBM -> LDS copy of one tile.  LDS slot s (16 bytes) of the tile holds
  // chunk s % PC of row s / PC; padding slots (chunk >= NCH) get a duplicate of
  // chunk 0.  Keys >= Lk read 0 (outside the buffer range).
  auto copy_tile = [&](__amdgpu_buffer_rsrc_t rs, unsigned char* dst, int key0, auto PCc, auto NIc) {
    constexpr int PC = decltype(PCc)::value, NI = decltype(NIc)::value;
#pragma unroll
    for (int bi0 = 0; bi0 < NI; bi0 += G::NW) {
      const int bi = bi0 + wave;
      if (bi < NI) {
        const int s = 64 * bi + lane;
        const int r = s / PC;
        int ch = s - r * PC;
        ch = ch < NCH ? ch : 0;
        const uint32_t off = (uint32_t)((key0 + r) * D + 8 * ch) * 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + 1024 * bi), 16, off, 0, 0, 0);
      }
    }
  };
  auto copy_k = [&](int tile, int buf) {
    copy_tile(krs, kbuf0 + buf * KT, tile * BC, std::integral_constant<int, G::KPC>{},
              std::integral_constant<int, G::KI>{});
  };
  auto copy_v = [&](int tile, int buf) {
    copy_tile(vrs, vbuf0 + buf * VT, tile * BC, std::integral_constant<int, G::VPC>{},
              std::integral_constant<int, G::VI>{});
  };

  // ---- key range of this workgroup
  int n_kv = (Lk + BC - 1) / BC;
  if constexpr (CAUSAL) {
    const int last_row = min(i0 + G::BR, Lq) - 1;
    n_kv = min(n_kv, last_row / BC + 1);
  }
  auto active = [&](int t) { return !CAUSAL || t * BC <= i0w + 31; };  // wave-uniform

  copy_k(0, 0);
  copy_v(0, 0);
  if (n_kv > 1) copy_k(1, 1);

  // ---- Q tile -> VGPRs, as the B operand of Sᵀ = K·Qᵀ (column = query row l%32,
  // contraction slots of half g = head dims 16s+8g .. 16s+8g+7).  Rows past Lq read 0.
  const int qrow = i0w + l32;
  u32x4 qr[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const u32x4 x = buf_load16(qrs, (uint32_t)(qrow * D + 16 * s + 8 * g) * 2);
    qr[s] = (x & p.q_and) ^ p.q_xor;
  }

  // per-lane LDS offsets of the MFMA operand reads
  const int k_off = l32 * KP + 16 * g;  // K row l%32, chunk 2s+g at +32s
  const int gi = lane >> 4, li = lane & 15;
  const int v_off = (4 * (gi >> 1) + (li >> 2)) * VP + 2 * (16 * (gi & 1) + 4 * (li & 3));

  auto compute_s = [&](const unsigned char* kb_, f32x16 (&S)[KB]) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      S[kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < KS; ++s) S[kb] = mfma32<DT>(lds_read16(kb_ + k_off + kb * 32 * KP + 32 * s), qr[s], S[kb]);
    }
  };

  const float c = p.c;
  float m_run = NEG_INF, l_f = 0.f, l_r = 0.f;
  f32x16 oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x16{};

  // softmax of tile t (in S) and Oᵀ += Vᵀ·Pᵀ with V from vb_
  auto softmax_pv = [&](f32x16 (&S)[KB], int t, const unsigned char* vb_) {
    const int j0 = t * BC;
    const bool need_mask = (CAUSAL && j0 + BC - 1 > i0w) || (j0 + BC > Lk);
    if (need_mask) {
      // key offset within the tile of S[kb][r] is 32kb + 8(r/4) + 4g + r%4
      const int lim_tail = Lk - j0 - 4 * g;
      const int lim = CAUSAL ? min(qrow - j0 - 4 * g + 1, lim_tail) : lim_tail;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ko = 32 * kb + 8 * (r >> 2) + (r & 3);
          S[kb][r] = ko >= lim ? NEG_INF : S[kb][r];
        }
    }
    float mx = NEG_INF;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kb][r]);
    const float m_tile = xhalf_max(mx) * c;
    const bool grow = m_tile > m_run + TAU;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? m_tile : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_f *= alpha;
      l_r *= alpha;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) oacc[nb] *= alpha;
    }
    const float mb = m_run == NEG_INF ? 0.f : m_run;  // no visible key yet: weights stay 0
    u32x4 pb[KB][2];
    float sf = 0.f, sr = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][8 * h + 2 * e], c, -mb));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][8 * h + 2 * e + 1], c, -mb));
          sf += p0 + p1;
          const uint32_t pk = pack2<DT>(p0, p1);
          sr = sum2<DT>(pk, sr);
          pb[kb][h][e] = pk;
        }
    l_f += sf;
    l_r += sr;
    // Oᵀ += Vᵀ·Pᵀ: A operand = 8 keys of one head dim, two transposing reads
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const unsigned char* a0 = vb_ + v_off + (32 * kb + 16 * h) * VP + 64 * nb;
          const u32x2 lo = lds_read_tr(a0);
          const u32x2 hi = lds_read_tr(a0 + 8 * VP);
          oacc[nb] = mfma32<DT>(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb[kb][h], oacc[nb]);
        }
  };

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 sA[KB], sB[KB];
  compute_s(kbuf0, sA);  // tile 0 is active for every wave
  __syncthreads();       // every wave is done with K buffer 0 before it is refilled

  // iteration t: copies K t+2 -> kbuf[t&1], V t+1 -> vbuf[(t+1)&1]; Sᵀ of tile t+1 from
  // kbuf[(t+1)&1]; softmax + PV of tile t with V from vbuf[t&1].
  auto iteration = [&](int t, f32x16 (&Sc)[KB], f32x16 (&Sn)[KB], auto PARc) {
    constexpr int P = decltype(PARc)::value;
    if (t + 2 < n_kv) copy_k(t + 2, P);
    if (t + 1 < n_kv) copy_v(t + 1, P ^ 1);
    if (t + 1 < n_kv && active(t + 1)) compute_s(kbuf0 + (P ^ 1) * KT, Sn);
    if (active(t)) softmax_pv(Sc, t, vbuf0 + P * VT);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  for (int t = 0; t < n_kv; t += 2) {
    iteration(t, sA, sB, std::integral_constant<int, 0>{});
    if (t + 1 < n_kv) iteration(t + 1, sB, sA, std::integral_constant<int, 1>{});
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
