// Fused, tiled attention forward kernel for gfx950 (MI355X).
//
// Pages cited (title, then the section on that page):
//   [DF] "FlashAttention数据流优化：MI50显存与带宽瓶颈实战"  (kwkr.cn/news/544806)
//   [AI] "AIInfra笔记01"                                   (kwkr.cn/news/547341)
//   [OP] "FlashAttention优化原理与工程实践"                (lbrq.cn/news/50349)
//
// One workgroup = 8 waves (two per SIMD) = 256 query rows of one (batch, head);
// each wave owns 32 rows.  One workgroup per CU.  (Grids with no more such
// workgroups than CUs use 128 rows per workgroup instead: twice the workgroups,
// and waves w and w+4 own the same rows and take alternate key tiles, merging
// their partial results through LDS at the end.)  The method ([DF §2.2], first
// and second layers; [OP §2.1], a loop over key blocks inside a loop over query
// blocks):
//   * the Q tile is loaded once and stays in VGPRs as MFMA operands;
//   * K and V tiles of BC keys are copied HBM -> LDS by the buffer unit itself
//     (buffer_load ... lds, no VGPR staging) into a ring of four stages: the
//     copies of tile t+3 are issued while tile t is computed ([DF §2.3] prefetch
//     of the next block, three tiles ahead here).  At the end of an iteration
//     each wave waits for its own copies (vmcnt) and the workgroup joins with a
//     bare s_barrier, without the memory fence a __syncthreads would add;
//   * in LDS, 1 KB copy block b of a tile holds rows b, b+NBLK, b+2·NBLK, ... and
//     blocks are padded apart: every copy uses one per-lane offset, and the rows
//     read together by an MFMA operand fall on distinct banks;
//   * Sᵀ = K·Qᵀ runs on v_mfma_f32_32x32x16_{bf16,f16} with fp32 accumulation, so
//     each lane holds 32 keys of ONE query row and the row max / row sums are
//     in-lane plus one v_permlane32_swap with the other half-wave;
//   * full tiles are software-pipelined inside each wave: the MFMAs of Sᵀ for
//     tile t+1 are issued in the same basic block as the softmax and PV of tile
//     t, with the rescale decision for tile t taken from the max found one
//     iteration earlier; tiles that cross the diagonal or the end of the keys
//     run afterwards, unpipelined and masked;
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
// cross the diagonal or the end of the keys pay for the mask.  Causal work items
// are ordered heads in pairs, heaviest query tiles first within a pair.
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
typedef float f32x4 __attribute__((ext_vector_type(4)));
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
  int H;            // heads (b = bh / H, h = bh % H)
  // element strides of batch, head and row; the head dim is contiguous
  int64_t q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh;
  int q_sl, k_sl, v_sl, o_sl;
  int kv_off;       // causal: key position of query row 0 (Lk - Lq >= 0)
  int n_qt;         // query tiles per head: ceil(Lq / BR)
  int n_split;      // key splits per (batch*head, query tile); 1: one pass, output written directly
  int num_wg;       // B * H * n_qt * n_split
  int bh;           // B * H
  float* ws_o;      // n_split > 1: unnormalised partial outputs, fp32 [n_split][B*H][Lq][D]
  float* ws_ml;     // n_split > 1: per row (m, l_f, l_r, 0), fp32 [n_split][B*H][Lq][4]
  int wg_order;     // bit 0: group consecutive work items on one XCD; bit 1: two
                    // work items per workgroup (paired form, two key groups only)
  float c;          // |scale| * log2(e), or log2(e) when scale == 0 (always > 0)
  uint32_t q_and;   // 0xffffffff, or 0 when scale == 0 (Q forced to zero)
  uint32_t q_xor;   // 0x80008000 when scale < 0 (Q negated exactly), else 0
  // dropout (kernels instantiated with DROP): keep iff mask byte < drop_t; kept
  // weights scaled by drop_scale = 256 / drop_t; Philox key (seed_lo, seed_hi)
  uint32_t drop_t, seed_lo, seed_hi;
  float drop_scale;
};

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC 2011): ten rounds of two 32x32 -> 64-bit products, the high
// halves xored into the other two words with the key, and the key advanced by
// the Weyl constants between rounds.  Each product is written as one 64-bit
// multiply, which gfx950 does in a single v_mad_u64_u32 (both halves) instead of
// a v_mul_lo_u32 and a v_mul_hi_u32 (all of them quarter-rate instructions).
// With B3, from the second round on each three-way xor is one v_bitop3_b32
// (truth table 0x96: odd parity).  The first round keeps plain xors: there the
// counter words and the key can all be uniform, and a VOP3 instruction reads at
// most one scalar register, so a bitop3 would need a register copy; plain xors
// let the scalar unit take the uniform part.  (Callers whose registers are
// tightest — the dropout forward's masked tiles and its last full tile — take
// B3 = false: the bitop3 schedule ran those paths out of registers.)  Same bits
// either way.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}
template <bool B3 = true>
__device__ __forceinline__ u32x4 philox10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                          uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)c0 * 0xD2511F53u;
    const uint64_t p1 = (uint64_t)c2 * 0xCD9E8D57u;
    c0 = (r == 0 || !B3) ? (uint32_t)(p1 >> 32) ^ c1 ^ k0 : xor3((uint32_t)(p1 >> 32), c1, k0);
    c1 = (uint32_t)p1;
    c2 = (r == 0 || !B3) ? (uint32_t)(p0 >> 32) ^ c3 ^ k1 : xor3((uint32_t)(p0 >> 32), c3, k1);
    c3 = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return u32x4{c0, c1, c2, c3};
}

// Dropout bits of a 4 x 4 block of (query row, key) of one (batch, head): the
// counter is (key / 4, row / 4, batch*head, 0); output word w, byte b covers row
// 4*(row/4) + w and key 4*(key/4) + b.  A weight is kept iff its byte < T.
template <bool B3 = true>
__device__ __forceinline__ u32x4 drop_block(int key4, int row4, int bh, uint32_t k0, uint32_t k1) {
  return philox10<B3>((uint32_t)key4, (uint32_t)row4, (uint32_t)bh, 0u, k0, k1);
}
// 16-bit lane masks of the kept weights of word w's bytes b0 and b0+1
__device__ __forceinline__ uint32_t keep_pair(uint32_t w, int b0, uint32_t T) {
  const uint32_t lo = (w >> (8 * b0)) & 0xffu, hi = (w >> (8 * b0 + 8)) & 0xffu;
  return (lo < T ? 0x0000ffffu : 0u) | (hi < T ? 0xffff0000u : 0u);
}

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

__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

// One 16-byte-per-lane HBM -> LDS copy (buffer_load_dwordx4 ... lds): lane l's
// 16 bytes land at LDS byte lds + 16·l (M0 holds the LDS base; the asm declares
// M0 as an output, so the compiler knows it changes).  Written as inline
// assembly so that the compiler neither tracks nor waits for these LDS writes:
// the kernel orders them itself with explicit vmcnt waits and barriers.  rsrc and
// lds must be uniform.
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t lds, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  uint32_t m0v;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds"
               : "={m0}"(m0v)
               : "s"(lds), "v"(voff), "s"(rsrc)
               : "memory");
#endif
}
// Two such copies in one statement.
__device__ __forceinline__ void dma16x2(u32x4 rsrc, uint32_t lds0, uint32_t voff0, uint32_t lds1, uint32_t voff1) {
#if defined(__HIP_DEVICE_COMPILE__)
  uint32_t m0v;
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %5, 0 offen lds\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %4, %5, 0 offen lds"
      : "={m0}"(m0v)
      : "s"(lds0), "v"(voff0), "s"(lds1), "v"(voff1), "s"(rsrc)
      : "memory");
#endif
}

// 32-bit LDS address of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// A copy of x that the compiler cannot relate to x: values derived from it are
// recomputed where they are needed instead of being kept live (and spilled)
// across the whole kernel.
__device__ __forceinline__ int opaque(int x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(x));
#endif
  return x;
}

// The kernel's argument block read afresh from the kernel-argument segment (the
// explicit arguments start at its offset 0).  The empty asm hides the segment
// address, so that a loop over work items reads the arguments again in each
// iteration instead of keeping all of them in scalar registers across it.
template <class T>
__device__ __forceinline__ T reread_args() {
#if defined(__HIP_DEVICE_COMPILE__)
  uint64_t a = (uint64_t)(uintptr_t)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(a));
  return *(const __attribute__((address_space(4))) T*)a;
#else
  return T{};
#endif
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

// Tile geometry shared by the kernel and the host launcher: NW_ = 8 waves, two
// per SIMD.  KG_ = 1: 256 query rows per workgroup, every wave takes every key
// tile (the default).  KG_ = 2: 128 rows, and the waves form two key groups of
// four that share those rows and take alternate key tiles, for grids too small
// to give every CU a workgroup of 256 rows.
template <int D, int NW_ = 8, int KG_ = 1>
struct Geo {
  static constexpr int NW = NW_;               // waves per workgroup
  static constexpr int KG = KG_;               // key groups
  static constexpr int NT = 64 * NW;           // threads per workgroup
  static constexpr int BR = 32 * NW / KG;      // query rows per workgroup
  static constexpr int BC = 64;                // keys per K/V tile
  static constexpr int KB = BC / 32;           // 32-key blocks of a tile (Sᵀ MFMA row blocks)
  static constexpr int NB = D / 32;            // 32-dim blocks of the output (Oᵀ MFMA row blocks)
  static constexpr int KS = D / 16;            // contraction steps of QKᵀ
  static constexpr int NCH = D / 8;            // 16-byte chunks per K/V row
  // LDS image of a K/V tile: NBLK blocks of 1 KB, one per copy instruction; block
  // b holds the RPB rows b, b+NBLK, b+2·NBLK, ... back to back, and blocks are
  // separated by a pad.  The pads put the rows read together by one MFMA operand
  // read on distinct banks, and every copy needs the same per-lane source offset.
  static constexpr int RPB = 512 / D;          // rows per block (4 at D=128, 8 at D=64)
  static constexpr int NBLK = BC / RPB;        // blocks per tile
  static constexpr int KBS = 1024 + 16;        // bytes per K block (rows 16 bytes apart in bank space)
  static constexpr int VBS = 1024 + 64;        // bytes per V block (rows 64 bytes apart in bank space)
  static constexpr int KT = NBLK * KBS, VT = NBLK * VBS;  // bytes per K / V tile

  static constexpr int NS = 4;                 // K and V tiles resident in LDS (ring of stages)
  static constexpr int LDS = NS * (KT + VT);
  static_assert(NBLK % NW == 0 && 32 % NBLK == 0 && NBLK >= 8, "copy and read layout");
  static_assert(LDS <= 163840, "one workgroup per CU");
  static_assert(KG == 1 || (KG == 2 && NW == 8), "key groups of four waves");
};

template <int D, int DT, bool CAUSAL, bool DROP, int NW = 8, int KG = 1>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_fwd_kernel(FwdParams args) {
  using G = Geo<D, NW, KG>;
  constexpr int BC = G::BC, KB = G::KB, NB = G::NB, KS = G::KS, NCH = G::NCH;
  constexpr int NBLK = G::NBLK, KBS = G::KBS, VBS = G::VBS, KT = G::KT, VT = G::VT;
  // Tile copies are issued by waves 0..NWC-1: without dropout one wave per SIMD
  // (waves w and w+4 share a SIMD).  The copy instructions of a step are slow to
  // issue when all waves issue them at once after the barrier; this way the
  // other wave of each SIMD goes straight on with its products (1-2% faster).
  // The dropout kernels keep every wave copying: they are register-bound, and
  // the longer copy sequence made them spill.
  constexpr int NWC = DROP ? NW : 4;
  constexpr int CPW = NBLK / NWC;  // copy instructions per copying wave and tile
  static_assert(NBLK % NWC == 0 && NW >= NWC && 3 * CPW <= 15, "copy layout, vmcnt immediates");
  constexpr float NEG_INF = -__builtin_inff();
  // One array per stage: the compiler can then tell that a tile copy in flight
  // into one stage does not alias reads of another, and waits for it only where
  // the code says so.
  __shared__ __attribute__((aligned(16))) unsigned char ks0[KT], ks1[KT], ks2[KT], ks3[KT];
  __shared__ __attribute__((aligned(16))) unsigned char vs0[VT], vs1[VT], vs2[VT], vs3[VT];
  static_assert(G::NS == 4, "four stages");
  auto kst = [&](auto Sc) -> unsigned char* {
    constexpr int S = decltype(Sc)::value;
    if constexpr (S == 0) return ks0; else if constexpr (S == 1) return ks1; else if constexpr (S == 2) return ks2;
    else return ks3;
  };
  auto vst = [&](auto Sc) -> unsigned char* {
    constexpr int S = decltype(Sc)::value;
    if constexpr (S == 0) return vs0; else if constexpr (S == 1) return vs1; else if constexpr (S == 2) return vs2;
    else return vs3;
  };
  using I0 = std::integral_constant<int, 0>;
  // dropout: per wave and 32-key half, the buffer of the Philox words' quad
  // transpose (16 quads of 4 lanes x 4 words, quads 20 dwords apart)
  __shared__ __attribute__((aligned(16))) uint32_t dxp[DROP ? NW * 2 * 320 : 4];

  const int tid = threadIdx.x;

  // ---- work item: (batch*head, query tile); heaviest causal tiles first, and
  // consecutive items (all query tiles of one head) on one XCD, whose L2 then
  // serves the K/V re-reads of that head.
  const int bid = blockIdx.x;
  // Two items per workgroup (the paired form) only in the two-key-group kernels
  // without dropout; the dropout kernels have no scalar registers to spare for
  // the loop.
  constexpr bool PAIRABLE = KG == 2 && !DROP;
  const int n_rep = PAIRABLE ? 1 + ((args.wg_order >> 1) & 1) : 1;
  // Q rows of the current item as loaded (the sign / zero transform of the scale
  // is applied once they are in)
  u32x4 qr[G::KS];
  // One work item (the rep-th of this workgroup); false: there is none.  A lambda
  // called once outside the paired form, so that those kernels compile as a plain
  // body (with a loop around it their register allocation and schedule shifted:
  // the dropout kernel lost 9%).
  auto item_body = [&](int rep) -> bool {
    const FwdParams p = PAIRABLE ? reread_args<FwdParams>() : args;
    // Item r of this workgroup: batch*head, query tile counted from the heaviest,
    // key split; false if there is none.  Paired form (n_rep == 2): the items of an
    // XCD's block (all of the block when the grid is not spread over the XCDs) are
    // taken from both ends, the first from the start and the second from the end,
    // so that a workgroup runs a heavy causal tile and then a light one.
    auto locate = [&](const FwdParams& pa, int r, int& bh_, int& qtr_, int& split_) -> bool {
      int item_s;
      if (PAIRABLE && n_rep == 2) {
        const int nb = (pa.wg_order & 1) ? 8 : 1;
        const int x = bid % nb, i = bid / nb, mi = pa.bh * pa.n_qt / nb;
        if (r && mi - 1 - i == i) return false;  // the middle item of an odd block runs once
        item_s = x * mi + (r ? mi - 1 - i : i);
      } else {
        item_s = (pa.wg_order & 1) ? (bid & 7) * (pa.num_wg >> 3) + (bid >> 3) : bid;
      }
      // the key splits of one (batch*head, query tile) are consecutive items
      const int item = item_s / pa.n_split;
      split_ = item_s - item * pa.n_split;
      if (CAUSAL) {
        // Heads in pairs, and within a pair the query tiles of both heads heaviest
        // first: work is then dispatched nearly longest-first while only two heads'
        // K/V are streamed at a time on each XCD (an odd last head runs alone).
        const int hp = item / (2 * pa.n_qt), j = item - hp * 2 * pa.n_qt;
        if (2 * hp + 1 < pa.bh) {
          bh_ = 2 * hp + (j & 1);
          qtr_ = j >> 1;
        } else {
          bh_ = 2 * hp;
          qtr_ = j;
        }
      } else {
        bh_ = item / pa.n_qt;
        qtr_ = item - bh_ * pa.n_qt;
      }
      bh_ = __builtin_amdgcn_readfirstlane(bh_);  // uniform: keep it in scalar registers
      qtr_ = __builtin_amdgcn_readfirstlane(qtr_);
      return true;
    };
    int bh, qt_r, split;
    if (!locate(p, rep, bh, qt_r, split)) return false;
    // in the paired form thread-derived values are taken afresh for each item (see
    // opaque()): derived once before the loop, they and what the compiler computes
    // from them would stay live across all of it
    const int tid_i = PAIRABLE ? opaque(tid) : tid;
    const int lane = tid_i & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid_i >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    const int qt = CAUSAL ? p.n_qt - 1 - qt_r : qt_r;
    const int i0 = qt * G::BR;
    // rows of this wave; with two key groups, waves w and w + NW/2 share rows
    const int wr = KG == 2 ? wave & (NW / 2 - 1) : wave;
    const int kg = KG == 2 ? wave / (NW / 2) : 0;  // key group (wave-uniform)
    const int i0w = i0 + 32 * wr;
    const int Lq = p.Lq, Lk = p.Lk;

    // (batch, head) slabs; a slab's rows are q_sl (k_sl, ...) elements apart and its
    // buffer range ends with the last row, so rows past the end read 0 / drop stores
    auto slab = [&](const void* base, int64_t sb, int64_t sh, int H, int bh_) -> const char* {
      const int b_ = __builtin_amdgcn_readfirstlane(bh_ / H), h_ = bh_ - b_ * H;
      return (const char*)base + ((int64_t)b_ * sb + (int64_t)h_ * sh) * 2;
    };
    const int q_sl = p.q_sl, k_sl = p.k_sl, v_sl = p.v_sl, o_sl = p.o_sl;
    const char* const kslab = slab(p.k, p.k_sb, p.k_sh, p.H, bh);
    const char* const vslab = slab(p.v, p.v_sb, p.v_sh, p.H, bh);
    char* const oslab = (char*)slab(p.o, p.o_sb, p.o_sh, p.H, bh);
    const uint32_t end_q = (uint32_t)((Lq - 1) * q_sl + D) * 2;
    const auto ors = make_rsrc(oslab, (uint32_t)((Lq - 1) * o_sl + D) * 2);

    // ---- HBM -> LDS copy of one tile.  Copy j of wave w < NWC fills block b = w + NWC·j:
    // lane l brings the 16-byte chunk l % NCH of tile row b + NBLK·(l / NCH).  The
    // buffer resource starts at the tile's first key and ends with the last key's
    // row, so keys >= Lk read 0; the per-lane offset is the same for every tile.
    const int lrow = wave + NBLK * (lane / NCH), lchunk = 16 * (lane % NCH);
    const uint32_t src_k = (uint32_t)(lrow * k_sl * 2 + lchunk), src_v = (uint32_t)(lrow * v_sl * 2 + lchunk);
    // per tensor: bytes per tile of BC rows, bytes from the slab start to the end of
    // its last row, and the offset between a wave's copies
    const int64_t tb_k = (int64_t)BC * k_sl * 2, tb_v = (int64_t)BC * v_sl * 2;
    const uint32_t end_k = (uint32_t)((Lk - 1) * k_sl + D) * 2, end_v = (uint32_t)((Lk - 1) * v_sl + D) * 2;
    const uint32_t step_k = (uint32_t)(NWC * k_sl * 2), step_v = (uint32_t)(NWC * v_sl * 2);
    auto copy_tile = [&](const char* slab, int64_t tb, uint32_t end, uint32_t step, uint32_t lane_src,
                         unsigned char* dst, int tile, auto BSc) {
      constexpr int BS = decltype(BSc)::value;
      if constexpr (NWC < NW)
        if (wave >= NWC) return;  // wave-uniform
      const int64_t off = (int64_t)tile * tb;
      const uint64_t base = (uint64_t)(uintptr_t)(slab + off);
      const u32x4 rs = {(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base),
                        (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(base >> 32) & 0xffffu)),
                        (uint32_t)__builtin_amdgcn_readfirstlane((int)(end - (uint32_t)off)),
                        (uint32_t)kBufferFlags};
      const uint32_t l0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(lds_addr(dst) + BS * wave));
  #pragma unroll
      for (int j = 0; j < CPW; j += 2) {
        if (j + 1 < CPW)
          dma16x2(rs, l0 + BS * NWC * j, lane_src + step * j, l0 + BS * NWC * (j + 1), lane_src + step * (j + 1));
        else
          dma16(rs, l0 + BS * NWC * j, lane_src + step * j);
      }

    };
    auto copy_k = [&](int tile, auto Sc) {
      copy_tile(kslab, tb_k, end_k, step_k, src_k, kst(Sc), tile, std::integral_constant<int, KBS>{});
    };
    auto copy_v = [&](int tile, auto Sc) {
      copy_tile(vslab, tb_v, end_v, step_v, src_v, vst(Sc), tile, std::integral_constant<int, VBS>{});
    };

    // ---- key range of this workgroup
    // Causal (bottom-right): query row i sits at key position i + off, key j is
    // visible to it iff j <= i + off.
    const int off = CAUSAL ? p.kv_off : 0;
    auto kv_tiles = [&](int i0_) {  // key tiles seen by the rows from i0_ on
      int n = (Lk + BC - 1) / BC;
      if constexpr (CAUSAL) n = min(n, (min(i0_ + G::BR, Lq) - 1 + off) / BC + 1);
      return n;
    };
    const int n_kv = kv_tiles(i0);
    // this item's tiles: [t_b, t_e), an equal share of the n_kv tiles per split
    const int t_b = __builtin_amdgcn_readfirstlane((int)((int64_t)split * n_kv / p.n_split));
    const int t_e = __builtin_amdgcn_readfirstlane((int)((int64_t)(split + 1) * n_kv / p.n_split));
    auto active = [&](int t) { return !CAUSAL || t * BC <= i0w + 31 + off; };  // wave-uniform
    // a wave whose 32 rows all lie past the last query row only copies and joins
    const bool live = i0w < p.Lq;  // wave-uniform

    // ---- Q tile -> VGPRs, as the B operand of Sᵀ = K·Qᵀ (column = query row l%32,
    // contraction slots of half g = head dims 16s+8g .. 16s+8g+7).  Rows past Lq read 0.
    auto load_q = [&](const char* qslab_, int i0w_) {
      const auto rs = make_rsrc(qslab_, end_q);
  #pragma unroll
      for (int s = 0; s < KS; ++s) qr[s] = buf_load16(rs, (uint32_t)((i0w_ + l32) * q_sl + 16 * s + 8 * g) * 2);
    };
    auto fix_q = [&]() {
  #pragma unroll
      for (int s = 0; s < KS; ++s) qr[s] = (qr[s] & p.q_and) ^ p.q_xor;
    };
    // stage of tile t: (t - t_b) % NS.  Only what the first Sᵀ needs is copied
    // before the first wait (K of tile t_b, and with two key groups of t_b+1 too);
    // the other first tiles follow once it is in, while that Sᵀ is computed.  The
    // second item of a pair had its Q rows and those K tiles requested while the
    // first one finished.
    if (rep == 0) {
      load_q(slab(p.q, p.q_sb, p.q_sh, p.H, bh), i0w);
      if (t_b < t_e) copy_k(t_b, I0{});
      if constexpr (KG == 2)
        if (t_b + 1 < t_e) copy_k(t_b + 1, std::integral_constant<int, 1>{});
    }

    // per-lane LDS offsets of the MFMA operand reads.  Tile row r sits in block
    // r % NBLK at position r / NBLK; rows r and r + 8m (m >= 0, r < 8) differ by a
    // lane-independent offset, which goes into the instruction's immediate.
    auto row_off = [](int rows, int BS) { return (rows % NBLK) * BS + (rows / NBLK) * 2 * D; };
    const int k_off = (l32 % NBLK) * KBS + (l32 / NBLK) * 2 * D + 16 * g;  // K row l%32, chunk 2s+g at +32s
    const int gi = lane >> 4, li = lane & 15;
    const int v_off = (4 * (gi >> 1) + (li >> 2)) * VBS + 2 * (16 * (gi & 1) + 4 * (li & 3));

    auto compute_s = [&](const unsigned char* kb_, f32x16 (&S)[KB]) {
  #pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        S[kb] = f32x16{};
  #pragma unroll
        for (int s = 0; s < KS; ++s)
          S[kb] = mfma32<DT>(lds_read16(kb_ + k_off + row_off(32 * kb, KBS) + 32 * s), qr[s], S[kb]);
      }
    };

    const float c = p.c;
    // The running max starts at a finite -1e30 (not -inf): a row that sees no key of
    // this item (possible only within a key split) keeps weights 2^(-inf) = 0 and
    // sums 0, and the first visible tile always moves the max (scale 2^(-1e30) = 0).
    float m_run = -1e30f, l_f = 0.f, l_r = 0.f;
    f32x16 oacc[NB];
  #pragma unroll
    for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x16{};

    // Tiles [t_b, n_full) are visible in full to every row of the workgroup: no
    // mask, every wave active.  Causal: tile t is full for row i0 iff 64t+63 <= i0 + off.
    int n_full = Lk / BC;
    if constexpr (CAUSAL) n_full = min(n_full, (i0 + off + 1) / BC);
    n_full = min(n_full, t_e);

    // mask of a tile crossing the diagonal or the end of the keys (wave-uniform test)
    auto need_mask = [&](int t) { return (CAUSAL && t * BC + BC - 1 > i0w + off) || (t * BC + BC > Lk); };
    auto mask_tile = [&](f32x16(&S)[KB], int t) {
      const int j0 = t * BC;
      if (need_mask(t)) {
        // key offset within the tile of S[kb][r] is 32kb + 8(r/4) + 4g + r%4
        // (lane-derived values taken afresh, see opaque())
        const int lane_m = opaque(tid) & 63;
        const int g_m = lane_m >> 5, row_m = i0w + (lane_m & 31);
        const int lim_tail = Lk - j0 - 4 * g_m;
        const int lim = CAUSAL ? min(row_m + off - j0 - 4 * g_m + 1, lim_tail) : lim_tail;
  #pragma unroll
        for (int kb = 0; kb < KB; ++kb)
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ko = 32 * kb + 8 * (r >> 2) + (r & 3);
            S[kb][r] = ko >= lim ? NEG_INF : S[kb][r];
          }
      }
    };
    // row max of a tile, in log2 units (c > 0)
    auto row_max = [&](const f32x16(&S)[KB]) {
      float mx = NEG_INF;
  #pragma unroll
      for (int kb = 0; kb < KB; ++kb)
  #pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kb][r]);
      return xhalf_max(mx) * c;
    };
    // Lazy rescale: the running max moves only when a tile's max exceeds it by
    // more than TAU; then both sums and the partial output are scaled by
    // 2^(m_old - m_new).  In two steps, so that a caller can scale the output after
    // the tile's weights are made (S is dead by then, which keeps register
    // pressure down).
    float alpha = 1.f;
    auto move_max = [&](float m_tile) -> bool {
      const bool grow = m_tile > m_run + TAU;
      const bool any = __builtin_amdgcn_ballot_w64(grow) != 0;
      if (any) {
        const float m_new = grow ? m_tile : m_run;
        alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_f *= alpha;
        l_r *= alpha;
      }
      return any;
    };
    auto scale_o = [&](bool any) {
      if (any) {
  #pragma unroll
        for (int nb = 0; nb < NB; ++nb) oacc[nb] *= alpha;
      }
    };
    auto rescale = [&](float m_tile) { scale_o(move_max(m_tile)); };
    // weights of a tile against the running max, and their two row sums.  Every
    // row sees key 0 in tile 0, so m_run is finite from the first tile on.
    // With DROP, the weights that multiply V are masked by the dropout bits of
    // their (row, key); the sums stay those of all weights (dropout acts on the
    // normalised weights, and LSE is that of the scores).
    // Dropout words of one 32-key half kb of a tile: the lane needs, for blocks
    // x = 4kb + 2h + a (keys 32kb + 16h + 8a + 4g + 0..3 of its row), word row % 4.
    // The four lanes of a quad share the row block, so lane j computes block
    // 4kb + j and the quad transposes the words (one Philox call per four elements
    // becomes one per 16); wd[2h + a] is then this lane's word of block 4kb + 2h + a.
    // The transpose goes through LDS (four 4-byte writes and one 16-byte read per
    // lane): LDS has room beside the operand reads, the VALU does not, and the DPP
    // butterfly took 16 VALU instructions per transpose (2.4% faster at the 7B 4K
    // shape with dropout 0.1).
    auto drop_words = [&](int t, int kb, uint32_t (&wd)[4], auto B3c) {
      const int lane_d = opaque(tid) & 63;
      const int row_d = i0w + (lane_d & 31), g_d = lane_d >> 5, j = lane_d & 3;
      const u32x4 mine = drop_block<decltype(B3c)::value>(
          (t * BC + 32 * kb + 16 * (j >> 1) + 8 * (j & 1) + 4 * g_d) >> 2, row_d >> 2, bh, p.seed_lo, p.seed_hi);
      // quad transpose through LDS: word i of lane (quad q, j) at dword 20q + 4i + j of
      // this wave's buffer for half kb (writes on distinct banks), then lane j reads
      // the 16 bytes at 20q + 4j: word j of blocks 0..3
      uint32_t* const xb = dxp + (wave * 2 + kb) * 320 + 20 * (lane_d >> 2);
  #pragma unroll
      for (int i = 0; i < 4; ++i) xb[4 * i + j] = mine[i];
      const u32x4 got = *(const u32x4*)(xb + 4 * j);
  #pragma unroll
      for (int i = 0; i < 4; ++i) wd[i] = got[i];
    };
    // (B3c: std::true_type or std::false_type, the generator form for drop_words)
    auto make_p = [&](const f32x16(&S)[KB], u32x4(&pb)[KB][2], int t, auto B3c) {
      const float mb = m_run;
      float sf = 0.f, sr = 0.f;
  #pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        uint32_t wd[4];
        if constexpr (DROP) drop_words(t, kb, wd, B3c);
  #pragma unroll
        for (int h = 0; h < 2; ++h) {
          // keys of registers 8h..8h+7: 32kb + 16h + 4g + {0..3} and + 8 + 4g + {0..3}
          u32x4 dw[2];
          if constexpr (DROP) {
  #pragma unroll
            for (int a = 0; a < 2; ++a) {
              const uint32_t w = wd[2 * h + a];
              dw[a] = u32x4{keep_pair(w, 0, p.drop_t), keep_pair(w, 2, p.drop_t), 0u, 0u};
            }
          }
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][8 * h + 2 * e], c, -mb));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][8 * h + 2 * e + 1], c, -mb));
            sf += p0 + p1;
            const uint32_t pk = pack2<DT>(p0, p1);
            sr = sum2<DT>(pk, sr);
            if constexpr (DROP)
              pb[kb][h][e] = pk & dw[e >> 1][e & 1];
            else
              pb[kb][h][e] = pk;
          }
        }
      }
      l_f += sf;
      l_r += sr;
    };
    // Oᵀ += Vᵀ·Pᵀ: A operand = 8 keys of one head dim, two transposing reads
    auto pv = [&](const u32x4(&pb)[KB][2], const unsigned char* vb_) {
  #pragma unroll
      for (int kb = 0; kb < KB; ++kb)
  #pragma unroll
        for (int h = 0; h < 2; ++h)
  #pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const unsigned char* a0 = vb_ + v_off + 64 * nb;
            const u32x2 lo = lds_read_tr(a0 + row_off(32 * kb + 16 * h, VBS));
            const u32x2 hi = lds_read_tr(a0 + row_off(32 * kb + 16 * h + 8, VBS));
            oacc[nb] = mfma32<DT>(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb[kb][h], oacc[nb]);
          }
    };

    // End of a step: every wave waits for its own tile copies, then the workgroup
    // joins with a bare s_barrier (no memory fence: the copies are ordered by the
    // explicit vmcnt wait, and the compiler is kept from moving LDS accesses
    // across).  The copies of a step are issued three tiles ahead of their use and
    // land well within the step, so waiting for all of them costs nothing.
    auto wait_join = [&]() {
      __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));  // vmcnt(0)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    auto kst_rt = [&](int st) -> unsigned char* { return st == 0 ? ks0 : st == 1 ? ks1 : st == 2 ? ks2 : ks3; };
    auto vst_rt = [&](int st) -> unsigned char* { return st == 0 ? vs0 : st == 1 ? vs1 : st == 2 ? vs2 : vs3; };
    // K and V of tile t+NS-1, copied in iteration t into the stage of tile t-1,
    // which every wave finished with before the last barrier
    auto copies_rt = [&](int t) {
      using S1 = std::integral_constant<int, 1>;
      using S2 = std::integral_constant<int, 2>;
      using S3 = std::integral_constant<int, 3>;
      const int tn = t + G::NS - 1;
      switch ((t - t_b + G::NS - 1) % G::NS) {
        case 0: copy_k(tn, I0{}); copy_v(tn, I0{}); break;
        case 1: copy_k(tn, S1{}); copy_v(tn, S1{}); break;
        case 2: copy_k(tn, S2{}); copy_v(tn, S2{}); break;
        default: copy_k(tn, S3{}); copy_v(tn, S3{}); break;
      }
    };
    auto end_iter = [&](int) { wait_join(); };

    auto copy_k_rt = [&](int t) {
      switch ((t - t_b) & 3) {
        case 0: copy_k(t, I0{}); break;
        case 1: copy_k(t, std::integral_constant<int, 1>{}); break;
        case 2: copy_k(t, std::integral_constant<int, 2>{}); break;
        default: copy_k(t, std::integral_constant<int, 3>{}); break;
      }
    };
    auto copy_v_rt = [&](int t) {
      switch ((t - t_b) & 3) {
        case 0: copy_v(t, I0{}); break;
        case 1: copy_v(t, std::integral_constant<int, 1>{}); break;
        case 2: copy_v(t, std::integral_constant<int, 2>{}); break;
        default: copy_v(t, std::integral_constant<int, 3>{}); break;
      }
    };
    if constexpr (KG == 1) {
      wait_join();  // Q and K of tile t_b are in
      fix_q();
      // V of tile t_b, then K and V of tiles t_b+1 and t_b+2, in the order the loop
      // needs them (the steps copy tile t+3 in step t)
      if (t_b < t_e) copy_v(t_b, I0{});
      if (t_b + 1 < t_e) {
        copy_k(t_b + 1, std::integral_constant<int, 1>{});
        copy_v(t_b + 1, std::integral_constant<int, 1>{});
      }
      if (t_b + 2 < t_e) {
        copy_k(t_b + 2, std::integral_constant<int, 2>{});
        copy_v(t_b + 2, std::integral_constant<int, 2>{});
      }
      f32x16 sA[KB], sB[KB];
      float mxA = NEG_INF, mxB = NEG_INF;
      // Sᵀ of the first full tile while those copies land
      if (n_full > t_b && live) {
        compute_s(kst(I0{}), sA);
        mxA = row_max(sA);
      }
      // then wait only for V of tile t_b and K of tile t_b+1 (the copies return in
      // the order they were issued: those of V(t_b+1), K(t_b+2), V(t_b+2) may still
      // be in flight) and join
      if (t_b + 2 < t_e)
        __builtin_amdgcn_s_waitcnt(((3 * CPW) & 15) | (7 << 4) | (15 << 8));
      else if (t_b + 1 < t_e)
        __builtin_amdgcn_s_waitcnt((CPW & 15) | (7 << 4) | (15 << 8));
      else
        __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      int t_tail = t_b;
      if (n_full > t_b) {
        // ---- full tiles, software-pipelined: iteration t computes Sᵀ of tile t+1
        // and its row max while the weights and PV of tile t run; the rescale for
        // tile t uses the max found one iteration earlier.  No mask and no branch
        // inside the body (a wave with no live rows skips it whole).
        auto it_main = [&](int t, f32x16(&Sc)[KB], f32x16(&Sn)[KB], float& mxc, float& mxn, auto Pc) {
          constexpr int P = decltype(Pc)::value;
          using PN = std::integral_constant<int, (P + 1) % G::NS>;
          using PC = std::integral_constant<int, (P + G::NS - 1) % G::NS>;
          using PP = std::integral_constant<int, (P + 2) % G::NS>;
          if (live) rescale(mxc);
          // Without dropout the waves join only after the even steps (counted from
          // t_b), and step t copies K of tile t+3 and V of tile t+2 (V of tile t_b+2
          // comes from the prologue).  Between two joins run an odd step t and step
          // t+1: they read K of tiles t+1, t+2 and V of tiles t, t+1, all copied and
          // waited for before the join that precedes them, and write K of tiles t+3,
          // t+4 and V of tiles t+2, t+3, whose stages ((tile - t_b) mod 4) are none of
          // those read.  With dropout every step joins and copies tile t+3.
          if (t + G::NS - 1 < t_e) copy_k(t + G::NS - 1, PC{});
          if constexpr (DROP) {
            if (t + G::NS - 1 < t_e) copy_v(t + G::NS - 1, PC{});
          } else {
            if (t > t_b && t + 2 < t_e) copy_v(t + 2, PP{});
          }
          if (live) {
            // LLVM's interleave strategy for small-GEMM bodies (MFMAs spaced between the
            // LDS operand reads and the VALU work): 1.8% faster on the 7B 4K shape than
            // the default schedule, same results
            __builtin_amdgcn_iglp_opt(0);
            compute_s(kst(PN{}), Sn);
            u32x4 pb[KB][2];
            make_p(Sc, pb, t, std::true_type{});
            pv(pb, vst(Pc));
            mxn = row_max(Sn);
          }
          if constexpr (DROP || !(P & 1)) end_iter(t);
        };
        static_assert(G::NS == 4, "the loop below is unrolled over the stages");
        for (int t = t_b; t + 1 < n_full; t += 4) {
          it_main(t, sA, sB, mxA, mxB, I0{});
          if (t + 2 < n_full) it_main(t + 1, sB, sA, mxB, mxA, std::integral_constant<int, 1>{});
          if (t + 3 < n_full) it_main(t + 2, sA, sB, mxA, mxB, std::integral_constant<int, 2>{});
          if (t + 4 < n_full) it_main(t + 3, sB, sA, mxB, mxA, std::integral_constant<int, 3>{});
        }
        // back to the state of one join and one tile copied per step (K and V
        // requested through tile n_full + 1): after an odd last step the waves join,
        // then V of tile n_full + 1 is requested
        const int r_last = n_full - 2 - t_b;
        if (!DROP && r_last >= 0) {
          if (r_last & 1) wait_join();
          if (n_full + 1 < t_e) copy_v_rt(n_full + 1);
        }
        // weights and PV of the last full tile, whose Sᵀ is already computed
        const int tf = n_full - 1;
        auto finish = [&](f32x16(&Sc)[KB], float mxc) {
          if (live) rescale(mxc);
          if (tf + G::NS - 1 < t_e) copies_rt(tf);
          if (live) {
            u32x4 pb[KB][2];
            make_p(Sc, pb, tf, std::false_type{});
            // (with dropout, the V reads are not hoisted over the weights: that
            // schedule spilled a register here)
            if constexpr (DROP) __builtin_amdgcn_sched_barrier(0);
            pv(pb, vst_rt((tf - t_b) % G::NS));
          }
          end_iter(tf);
        };
        if ((tf - t_b) & 1)
          finish(sB, mxB);
        else
          finish(sA, mxA);
        t_tail = n_full;
      }
      // ---- tiles that cross the diagonal or the end of the keys: not pipelined,
      // masked; a wave skips tiles above its own rows but still copies and joins.
      for (int t = t_tail; t < t_e; ++t) {
        if (t + G::NS - 1 < t_e) copies_rt(t);
        if (live && active(t)) {
          compute_s(kst_rt((t - t_b) % G::NS), sA);
          // (scheduling barriers: the operand reads of one product are not hoisted
          // over the softmax, which would run this path out of registers)
          __builtin_amdgcn_sched_barrier(0);
          mask_tile(sA, t);
          const bool any = move_max(row_max(sA));
          u32x4 pb[KB][2];
          make_p(sA, pb, t, std::false_type{});
          scale_o(any);
          __builtin_amdgcn_sched_barrier(0);
          pv(pb, vst_rt((t - t_b) % G::NS));
        }
        end_iter(t);
      }

    } else {
      // ---- two key groups: group kg takes tiles t_b+kg, t_b+kg+2, ...; step s covers
      // tiles t_b+2s and t_b+2s+1.  Each group runs the software pipeline of the
      // one-group loop over its own tiles: Sᵀ of its next tile while the weights and
      // PV of the current one run.  A tile that crosses the diagonal or the end of the
      // keys is masked at the start of its step and its max taken again.  Step s
      // copies K of tiles t_b+2s+4 and +5 into the stages of the step's own tiles
      // (whose Sᵀ was made one step earlier) and V of tiles t_b+2s+2 and +3 into the
      // stages of the previous step's tiles (whose PV ran one step earlier).
      wait_join();  // Q and K of tiles t_b, t_b+1 are in
      fix_q();
      // V of tiles t_b, t_b+1 and K of tiles t_b+2, t_b+3 while the first Sᵀ is made
      if (t_b < t_e) copy_v(t_b, I0{});
      if (t_b + 1 < t_e) copy_v(t_b + 1, std::integral_constant<int, 1>{});
      if (t_b + 2 < t_e) copy_k(t_b + 2, std::integral_constant<int, 2>{});
      if (t_b + 3 < t_e) copy_k(t_b + 3, std::integral_constant<int, 3>{});
      f32x16 sA[KB], sB[KB];
      float mxA = NEG_INF, mxB = NEG_INF;
      const int t0 = t_b + kg;
      if (live && t0 < t_e && active(t0)) {
        compute_s(kst_rt((t0 - t_b) & 3), sA);
        mxA = row_max(sA);
      }
      wait_join();  // those copies are in, and every wave is done with the K stages that step 0 refills
      const int n_steps = (t_e - t_b + 1) >> 1;
      auto kstep = [&](int s, f32x16(&Sc)[KB], f32x16(&Sn)[KB], float& mxc, float& mxn) {
        const int tc = t_b + 2 * s;
        if (tc + 4 < t_e) copy_k_rt(tc + 4);
        if (tc + 5 < t_e) copy_k_rt(tc + 5);
        if (tc + 2 < t_e) copy_v_rt(tc + 2);
        if (tc + 3 < t_e) copy_v_rt(tc + 3);
        const int t = tc + kg;
        if (live && t < t_e && active(t)) {
          if (need_mask(t)) {
            mask_tile(Sc, t);
            mxc = row_max(Sc);
          }
          rescale(mxc);
          // LLVM's interleave strategy for small-GEMM bodies, as in the one-group loop.
          // Sᵀ of the group's next tile is made even when that tile lies past the end
          // or above the wave's rows (then from a stage no copy is writing in this
          // step, and never used): one straight block per step.  (Peeling the last
          // step to skip it costs more in spills than the products it saves.)
          __builtin_amdgcn_iglp_opt(0);
          compute_s(kst_rt((t + 2 - t_b) & 3), Sn);
          u32x4 pb[KB][2];
          make_p(Sc, pb, t, std::true_type{});
          pv(pb, vst_rt((t - t_b) & 3));
          mxn = row_max(Sn);
        }
        end_iter(t);
      };
      for (int s = 0; s < n_steps; s += 2) {
        kstep(s, sA, sB, mxA, mxB);
        if (s + 1 < n_steps) kstep(s + 1, sB, sA, mxB, mxA);
      }
      // The two groups' partial results for the same rows meet in LDS (every copy has
      // landed and every read of the ring finished before the last barrier): group 1
      // leaves its output accumulators in V stage wr and its running max and sums in
      // xst; group 0 combines them with its own (the running maxima and exp-sums of
      // disjoint key sets combine exactly, as across key splits) and goes on to the
      // epilogue.
      __shared__ float xst[NW / 2][3][64];
      float* const xo = (float*)vst_rt(wr);
      static_assert(NB * 16 * 64 * 4 <= VT, "one wave's accumulators fit a V stage");
      if (kg == 1 && live) {
  #pragma unroll
        for (int nb = 0; nb < NB; ++nb)
  #pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            *(f32x4*)(xo + ((nb * 4 + q4) * 64 + lane) * 4) =
                f32x4{oacc[nb][4 * q4], oacc[nb][4 * q4 + 1], oacc[nb][4 * q4 + 2], oacc[nb][4 * q4 + 3]};
        xst[wr][0][lane] = m_run;
        xst[wr][1][lane] = l_f;
        xst[wr][2][lane] = l_r;
      }
      __syncthreads();
      // Paired form: Q rows and the first two K tiles of the next item are requested
      // now (its first tile is tile 0, stage 0; the K stages are free once every wave
      // passed the barrier above), and land while this item's results are merged
      // and stored; the output rows are staged in the V stages for that.
      if (PAIRABLE && n_rep == 2 && rep == 0) {
        // (the arguments read once more: kept from the top of the item, they would
        // stay in scalar registers across all of it)
        const FwdParams pn = reread_args<FwdParams>();
        int bh2, qtr2, split2;
        if (locate(pn, 1, bh2, qtr2, split2)) {
          const int i02 = (CAUSAL ? pn.n_qt - 1 - qtr2 : qtr2) * G::BR;
          load_q(slab(pn.q, pn.q_sb, pn.q_sh, pn.H, bh2), i02 + 32 * wr);
          const char* const kslab2 = slab(pn.k, pn.k_sb, pn.k_sh, pn.H, bh2);
          const int te2 = kv_tiles(i02);
          constexpr auto KBSc = std::integral_constant<int, KBS>{};
          if (te2 > 0) copy_tile(kslab2, tb_k, end_k, step_k, src_k, ks0, 0, KBSc);
          if (te2 > 1) copy_tile(kslab2, tb_k, end_k, step_k, src_k, ks1, 1, KBSc);
        }
      }
      if (kg == 1) return true;
      if (live) {
        const float m1 = xst[wr][0][lane];
        const float mm = fmaxf(m_run, m1);
        const float a0 = __builtin_amdgcn_exp2f(m_run - mm), a1 = __builtin_amdgcn_exp2f(m1 - mm);
  #pragma unroll
        for (int nb = 0; nb < NB; ++nb)
  #pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 x = *(const f32x4*)(xo + ((nb * 4 + q4) * 64 + lane) * 4);
  #pragma unroll
            for (int i = 0; i < 4; ++i) oacc[nb][4 * q4 + i] = oacc[nb][4 * q4 + i] * a0 + x[i] * a1;
          }
        l_f = l_f * a0 + xst[wr][1][lane] * a1;
        l_r = l_r * a0 + xst[wr][2][lane] * a1;
        m_run = mm;
      }
    }

    // ---- epilogue.  The lane's row and half are derived afresh (see opaque()).
    const int lane_e = opaque(tid) & 63;
    const int g_e = lane_e >> 5, row_e = i0w + (lane_e & 31);
    const float lf_t = xhalf_sum(l_f);
    const float lr_t = xhalf_sum(l_r);
    if (p.n_split > 1) {
      // A key split stores its partial result: the unnormalised output and the
      // row's running max and two sums, all relative to that max (fa_merge_kernel
      // combines the splits).  Rows >= Lq are dropped by the buffer range.
      const size_t part = (size_t)split * p.bh + bh;
      const auto wrs = make_rsrc(p.ws_o + part * Lq * D, (uint32_t)Lq * D * 4);
  #pragma unroll
      for (int nb = 0; nb < NB; ++nb)
  #pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d0 = 32 * nb + 8 * q4 + 4 * g_e;
          const u32x4 w = {__float_as_uint(oacc[nb][4 * q4]), __float_as_uint(oacc[nb][4 * q4 + 1]),
                           __float_as_uint(oacc[nb][4 * q4 + 2]), __float_as_uint(oacc[nb][4 * q4 + 3])};
          buf_store16(wrs, (uint32_t)(row_e * D + d0) * 4, w);
        }
      if (g_e == 0 && row_e < Lq) {
        const u32x4 st = {__float_as_uint(m_run), __float_as_uint(lf_t), __float_as_uint(lr_t), 0u};
        *(u32x4*)(p.ws_ml + (part * Lq + row_e) * 4) = st;
      }
      return true;
    }
    // one pass: normalise by the sum of the rounded weights, store O and LSE.  The
    // accumulator layout gives a lane 4 dims of one row per 8 bytes, scattered over
    // 32 rows per instruction; the wave first lays its 32 rows out row-major in an
    // LDS stage of the ring (free since the last barrier: every copy has landed and
    // every read is done; one stage per wave.  With two key groups only group 0,
    // waves 0..3, gets here, and wave w uses V stage w, whose hand-over from its
    // partner it has just read: the K stages may be filling for the next item),
    // then stores whole rows, 16 bytes per lane.  Rows are OPITCH bytes apart in LDS
    // (16 bytes of pad: 16-byte aligned row reads, and the 8-byte writes of lanes
    // 0..15 on distinct banks).
    const float inv = DROP ? p.drop_scale / lr_t : 1.0f / lr_t;
    constexpr int OPITCH = 2 * D + 16;
    static_assert(32 * OPITCH <= KT && 32 * OPITCH <= VT, "one wave's output rows fit a stage");
    unsigned char* const stg = KG == 2 ? vst_rt(wr) : wave < 4 ? kst_rt(wave) : vst_rt(wave - 4);
    const int l32_e = lane_e & 31;
  #pragma unroll
    for (int nb = 0; nb < NB; ++nb)
  #pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * nb + 8 * q4 + 4 * g_e;
        const u32x2 w = {pack2<DT>(oacc[nb][4 * q4] * inv, oacc[nb][4 * q4 + 1] * inv),
                         pack2<DT>(oacc[nb][4 * q4 + 2] * inv, oacc[nb][4 * q4 + 3] * inv)};
        *(u32x2*)(stg + l32_e * OPITCH + d0 * 2) = w;
      }
    // (the wave reads back only what its own lanes wrote, and LDS keeps one wave's
    // accesses in order: no barrier)
    constexpr int CPR = D / 8;  // 16-byte chunks per row
  #pragma unroll
    for (int j = 0; j < 32 * CPR / 64; ++j) {
      const int r = j * (64 / CPR) + lane_e / CPR, ch = lane_e % CPR;
      const u32x4 x = *(const u32x4*)(stg + r * OPITCH + ch * 16);
      buf_store16(ors, (uint32_t)((i0w + r) * o_sl + ch * 8) * 2, x);  // rows >= Lq are dropped
    }
    if (g_e == 0 && row_e < Lq) p.lse[(size_t)bh * Lq + row_e] = (m_run + log2f(lf_t)) * 0.69314718055994530942f;
    return true;
  };
  if constexpr (PAIRABLE) {
    for (int rep = 0; rep < n_rep; ++rep)
      if (!item_body(rep)) break;
  } else {
    item_body(0);
  }
}

// ---- merge of key splits ([DF §2.2], second layer, applied across splits: the
// running max and exp-sums of independent key ranges combine exactly).  For row
// i with split partials (Ô_s, m_s, lf_s, lr_s), all relative to m_s in log2 units:
//   M = max_s m_s,  w_s = 2^(m_s - M),
//   O = Σ w_s Ô_s / Σ w_s lr_s,   LSE = (M + log2 Σ w_s lf_s) · ln 2,
// which is what one pass over all keys computes.  One pass over the splits in
// batches of MB (2..16, the launcher's pick for the split count): the loads of a
// batch are issued together (a serial loop would
// pay one memory round trip per split, which dominated decode steps with many
// splits), the running max moves to the batch's max and the sums are rescaled
// by 2^(M_old - M_new) — the streaming update once more.  HBM-bound; one row per
// D/4 lanes, 4 dims per lane.
struct MergeParams {
  const float* ws_o;
  const float* ws_ml;
  void* o;
  float* lse;
  int Lq, H, n_split, bh;
  int64_t o_sb, o_sh;
  int o_sl;
};

template <int D, int DT, int MB>
__global__ __launch_bounds__(256) void fa_merge_kernel(MergeParams p) {
  constexpr int LPR = D / 4, RPB = 256 / LPR;
  const int tid = threadIdx.x;
  const int64_t r = (int64_t)blockIdx.x * RPB + tid / LPR;  // row over B*H*Lq
  const int d0 = (tid % LPR) * 4;
  if (r >= (int64_t)p.bh * p.Lq) return;
  const int bh = (int)(r / p.Lq), i = (int)(r - (int64_t)bh * p.Lq);
  const size_t stride = (size_t)p.bh * p.Lq;  // rows per split
  // M starts below every split's max (an empty split keeps -1e30): the first
  // batch's scale 2^(M - M_new) is then 0 and the zero sums stay zero
  float M = -3.0e38f, lf = 0.f, lr = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < p.n_split; s0 += MB) {
    f32x4 st[MB], x[MB];
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      if (s0 + u < p.n_split) {
        const size_t row = (size_t)(s0 + u) * stride + r;
        st[u] = *(const f32x4*)(p.ws_ml + row * 4);
        x[u] = *(const f32x4*)(p.ws_o + row * D + d0);
      }
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < MB; ++u)
      if (s0 + u < p.n_split) Mn = fmaxf(Mn, st[u][0]);
    const float sc = __builtin_amdgcn_exp2f(M - Mn);
    M = Mn;
    lf *= sc;
    lr *= sc;
    acc *= sc;
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      if (s0 + u < p.n_split) {
        const float w = __builtin_amdgcn_exp2f(st[u][0] - M);
        lf += w * st[u][1];
        lr += w * st[u][2];
        acc += w * x[u];
      }
    }
  }
  const float inv = 1.0f / lr;
  const int b = bh / p.H, h = bh - b * p.H;
  char* const orow = (char*)p.o + ((int64_t)b * p.o_sb + (int64_t)h * p.o_sh + (int64_t)i * p.o_sl + d0) * 2;
  *(u32x2*)orow = u32x2{pack2<DT>(acc[0] * inv, acc[1] * inv), pack2<DT>(acc[2] * inv, acc[3] * inv)};
  if (d0 == 0) p.lse[r] = (M + log2f(lf)) * 0.69314718055994530942f;
}

// Merge for grids of few rows and many splits (a decode step: a handful of rows,
// tens of splits): one workgroup per row.  Its NG = 256 / (D/4) lane groups each
// combine the splits g, g+NG, g+2·NG, ... (at most MB of them, their loads issued
// together) into a partial (max, sums and output relative to it), and group 0
// combines the NG partials through LDS with the same streaming update.  One round
// trip to memory instead of one per batch of splits; exact like the batched merge,
// only the order of the fp32 additions differs.
template <int D, int DT, int MB>
__global__ __launch_bounds__(256) void fa_merge_wide_kernel(MergeParams p) {
  constexpr int LPR = D / 4, NG = 256 / LPR;
  __shared__ float sml[NG][4];
  __shared__ f32x4 sacc[NG][LPR];
  const int tid = threadIdx.x, grp = tid / LPR, lg = tid % LPR, d0 = lg * 4;
  const int64_t r = blockIdx.x;  // row over B*H*Lq
  const int bh = (int)(r / p.Lq), i = (int)(r - (int64_t)bh * p.Lq);
  const size_t stride = (size_t)p.bh * p.Lq;  // rows per split
  f32x4 st[MB], x[MB];
#pragma unroll
  for (int u = 0; u < MB; ++u) {
    const int s = grp + NG * u;
    if (s < p.n_split) {
      const size_t row = (size_t)s * stride + r;
      st[u] = *(const f32x4*)(p.ws_ml + row * 4);
      x[u] = *(const f32x4*)(p.ws_o + row * D + d0);
    }
  }
  // a group without splits keeps M below every split's max and zero sums
  float M = -3.0e38f;
#pragma unroll
  for (int u = 0; u < MB; ++u)
    if (grp + NG * u < p.n_split) M = fmaxf(M, st[u][0]);
  float lf = 0.f, lr = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < MB; ++u) {
    if (grp + NG * u < p.n_split) {
      const float w = __builtin_amdgcn_exp2f(st[u][0] - M);
      lf += w * st[u][1];
      lr += w * st[u][2];
      acc += w * x[u];
    }
  }
  if (lg == 0) {
    sml[grp][0] = M;
    sml[grp][1] = lf;
    sml[grp][2] = lr;
  }
  sacc[grp][lg] = acc;
  __syncthreads();
  if (grp != 0) return;
  float Mt = sml[0][0];
#pragma unroll
  for (int gi = 1; gi < NG; ++gi) Mt = fmaxf(Mt, sml[gi][0]);
  lf = 0.f;
  lr = 0.f;
  acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const float w = __builtin_amdgcn_exp2f(sml[gi][0] - Mt);
    lf += w * sml[gi][1];
    lr += w * sml[gi][2];
    acc += w * sacc[gi][lg];
  }
  const float inv = 1.0f / lr;
  const int b = bh / p.H, h = bh - b * p.H;
  char* const orow = (char*)p.o + ((int64_t)b * p.o_sb + (int64_t)h * p.o_sh + (int64_t)i * p.o_sl + d0) * 2;
  *(u32x2*)orow = u32x2{pack2<DT>(acc[0] * inv, acc[1] * inv), pack2<DT>(acc[2] * inv, acc[3] * inv)};
  if (d0 == 0) p.lse[r] = (Mt + log2f(lf)) * 0.69314718055994530942f;
}

}  // namespace fa355
