// libfa355: C ABI around the gfx950 attention forward and backward kernels.
//
// Argument validation happens here, on the host, before any HIP call, so every
// FA_ERR_* of a bad argument can be produced without a GPU.  A valid call
// selects the kernel instance for (head dim, dtype, causal, workgroup size) and
// enqueues one launch on the caller's stream (two with key splits: partials, then
// the merge; two for the backward pass: dQ with the row statistics, then dK and dV).
// No allocation, no synchronisation, no global mutable state apart from the
// per-thread last HIP error, a per-thread cache of each device's CU count, and
// the device address of each GPU's copy of the allocation-free entry point's
// scratch array (looked up once per device).

#include <math.h>
#include <stdint.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "fa355.h"
#include "fa_bwd_kernel.hpp"
#include "fa_fwd_kernel.hpp"

// Partials of fa_fwd_splitkv_noalloc: a device global instead of a caller's
// workspace, one copy per GPU, held until the process ends.  Host code never
// passes this name to a kernel (on the host it only stands for the symbol); it
// passes the device address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kVersion = 1 * 10000 + 4 * 100 + 0;
constexpr int kMaxSplits = 256;

int launch_status() {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return FA_OK;
  g_last_hip_error = (int)e;
  if (e == hipErrorInvalidDeviceFunction || e == hipErrorNoBinaryForGpu || e == hipErrorInvalidImage ||
      e == hipErrorInvalidDevice)
    return FA_ERR_DEVICE;
  return FA_ERR_LAUNCH;
}

template <int D, int DT, bool CAUSAL, bool DROP, int KG>
int launch(const fa355::FwdParams& p, const fa355::MergeParams& m, hipStream_t stream) {
  using G = fa355::Geo<D, 8, KG>;
  hipLaunchKernelGGL((fa355::fa_fwd_kernel<D, DT, CAUSAL, DROP, 8, KG>), dim3(p.num_wg), dim3(G::NT), 0, stream, p);
  int st = launch_status();
  if (st != FA_OK || p.n_split == 1) return st;
  constexpr int rows_per_block = 256 / (D / 4);
  const int64_t rows = (int64_t)m.bh * m.Lq;
  // Few rows (under one workgroup per CU with the batched merge) and enough
  // splits to share among a row's lane groups: one workgroup per row, each lane
  // group taking up to 8 splits in one batch of loads.
  constexpr int NG = 256 / (D / 4);
  if (rows * 8 <= 2048 && m.n_split >= 8 && m.n_split <= 8 * NG) {
    const dim3 wgrid((unsigned)rows);
    if (m.n_split <= 2 * NG)
      hipLaunchKernelGGL((fa355::fa_merge_wide_kernel<D, DT, 2>), wgrid, dim3(256), 0, stream, m);
    else if (m.n_split <= 4 * NG)
      hipLaunchKernelGGL((fa355::fa_merge_wide_kernel<D, DT, 4>), wgrid, dim3(256), 0, stream, m);
    else
      hipLaunchKernelGGL((fa355::fa_merge_wide_kernel<D, DT, 8>), wgrid, dim3(256), 0, stream, m);
    return launch_status();
  }
  const dim3 grid((unsigned)((rows + rows_per_block - 1) / rows_per_block));
  // splits merged per batch of loads: as many as there are, up to 16 (a batch
  // larger than the split count only adds predicated-off slots and registers)
  if (m.n_split <= 2)
    hipLaunchKernelGGL((fa355::fa_merge_kernel<D, DT, 2>), grid, dim3(256), 0, stream, m);
  else if (m.n_split <= 4)
    hipLaunchKernelGGL((fa355::fa_merge_kernel<D, DT, 4>), grid, dim3(256), 0, stream, m);
  else if (m.n_split <= 8)
    hipLaunchKernelGGL((fa355::fa_merge_kernel<D, DT, 8>), grid, dim3(256), 0, stream, m);
  else
    hipLaunchKernelGGL((fa355::fa_merge_kernel<D, DT, 16>), grid, dim3(256), 0, stream, m);
  return launch_status();
}

template <int D, bool DROP, int KG = 1>
int dispatch_dtype(const fa355::FwdParams& p, const fa355::MergeParams& m, int dtype, bool causal, hipStream_t s) {
  if (dtype == FA_DTYPE_BF16)
    return causal ? launch<D, fa355::DT_BF16, true, DROP, KG>(p, m, s)
                  : launch<D, fa355::DT_BF16, false, DROP, KG>(p, m, s);
  return causal ? launch<D, fa355::DT_F16, true, DROP, KG>(p, m, s)
                : launch<D, fa355::DT_F16, false, DROP, KG>(p, m, s);
}

// Compute units of the current device (0 if it cannot be read), cached per thread and device.
int cu_count() {
  constexpr int kMaxDev = 64;
  thread_local int cache[kMaxDev] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();  // the failed query's error is not a launch error
    return 0;
  }
  if (dev < kMaxDev && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    n = 0;
  }
  if (dev < kMaxDev) cache[dev] = n;
  return n;
}

// Device address of the current device's copy of `scratch`, looked up once per
// device (nullptr, with the HIP error kept, if the lookup fails).
void* scratch_ptr() {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDev] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDev) {
    g_last_hip_error = (int)(e != hipSuccess ? e : hipErrorInvalidDevice);
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      g_last_hip_error = (int)(e != hipSuccess ? e : hipErrorInvalidSymbol);
      (void)hipGetLastError();
      return nullptr;
    }
    ptrs[dev] = ptr;
  }
  return ptrs[dev];
}

// Dropout keep threshold T = round((1 - p)·256): 256 keeps everything (no
// dropout), 0 (p too close to 1) and p outside [0, 1) are errors (-1 returned).
int drop_threshold(float p) {
  if (!(p >= 0.0f && p < 1.0f)) return -1;
  const int t = (int)floor((1.0 - (double)p) * 256.0 + 0.5);
  return t < 1 ? -1 : (t > 256 ? 256 : t);
}

bool aligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

// bytes of the partials workspace: outputs, then row statistics
size_t ws_o_bytes(int B, int H, int Lq, int D, int splits) { return (size_t)splits * B * H * Lq * D * 4; }
size_t ws_bytes(int B, int H, int Lq, int D, int splits) {
  return splits <= 1 ? 0 : ws_o_bytes(B, H, Lq, D, splits) + (size_t)splits * B * H * Lq * 4 * 4;
}

// The forward kernel's grid for valid sizes.  Workgroups of 8 waves and 256
// rows; a single pass (no key splits) whose grid would not exceed the CU count
// takes 128 rows per workgroup instead, with the 8 waves in two key groups that
// take alternate key tiles: twice the workgroups, the heaviest causal ones half
// as long, and still two waves per SIMD.  When those items outnumber the CUs (and
// without dropout), each workgroup runs two of them, from both ends of its XCD's
// block of items (the whole grid when the item count is no multiple of 16): a
// heavy causal tile and then a light one, whose sum is the same for every
// workgroup when a block holds whole pairs of heads (causal grids are paired only
// then).  The second item's first loads overlap the first one's merge and stores,
// and no workgroup is launched twice on a CU.
struct FwdPlan {
  int64_t n_qt;     // query tiles per head
  bool narrow;      // 128-row two-key-group form
  int n_rep;        // items per workgroup
  int64_t num_wg;   // workgroups
  int wg_order;     // the kernel's order flags (FwdParams::wg_order)
};
FwdPlan plan_fwd(int B, int H, int Lq, int causal, int splits, int drop_t) {
  static_assert(fa355::Geo<64>::BR == fa355::Geo<128>::BR && fa355::Geo<64, 8, 2>::BR == fa355::Geo<128, 8, 2>::BR,
                "row tile independent of D");
  FwdPlan pl;
  pl.n_qt = ((int64_t)Lq + fa355::Geo<128>::BR - 1) / fa355::Geo<128>::BR;
  pl.narrow = false;
  pl.n_rep = 1;
  if (splits == 1 && (int64_t)B * H * pl.n_qt <= 2048) {
    const int cus = cu_count();
    pl.narrow = cus > 0 && (int64_t)B * H * pl.n_qt <= cus;
    if (pl.narrow) {
      pl.n_qt = ((int64_t)Lq + fa355::Geo<128, 8, 2>::BR - 1) / fa355::Geo<128, 8, 2>::BR;
      const int64_t n_items = (int64_t)B * H * pl.n_qt;
      const int64_t per_block = n_items % 16 == 0 ? n_items / 8 : n_items;
      if (drop_t >= 256 && n_items > cus && (!causal || per_block % (2 * pl.n_qt) == 0)) pl.n_rep = 2;
    }
  }
  const int64_t n_items = (int64_t)B * H * pl.n_qt;
  pl.num_wg = pl.n_rep == 2 ? (n_items + 1) / 2 : n_items * splits;
  pl.wg_order = ((pl.n_rep == 2 ? n_items % 16 == 0 : pl.num_wg % 8 == 0) ? 1 : 0) | (pl.n_rep == 2 ? 2 : 0);
  return pl;
}

int fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lq, int Lk, int D,
        const int64_t* q_stride, const int64_t* k_stride, const int64_t* v_stride, const int64_t* o_stride,
        float scale, int causal, int dtype, int splits, void* ws, size_t ws_size, fa_stream_t stream,
        float dropout_p = 0.0f, uint64_t seed = 0, bool use_scratch = false) {
  if (!q || !k || !v || !o || !lse || !q_stride || !k_stride || !v_stride || !o_stride) return FA_ERR_NULL;
  if (B < 1 || H < 1 || Lq < 1 || Lk < 1) return FA_ERR_SHAPE;
  if (D != 64 && D != 128) return FA_ERR_HEAD_DIM;
  if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  const int64_t* st[4] = {q_stride, k_stride, v_stride, o_stride};
  for (int i = 0; i < 4; ++i)
    if (st[i][0] < 0 || st[i][1] < 0 || st[i][2] < D) return FA_ERR_STRIDE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_ALIGN;
  for (int i = 0; i < 4; ++i)  // every row starts on a 16-byte boundary
    if (st[i][0] % 8 || st[i][1] % 8 || st[i][2] % 8) return FA_ERR_ALIGN;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if (causal && Lq > Lk) return FA_ERR_CAUSAL_SHAPE;
  const int drop_t = drop_threshold(dropout_p);
  if (drop_t < 0) return FA_ERR_DROPOUT;
  if (splits < 1 || splits > kMaxSplits) return FA_ERR_SPLITS;
  if (splits > 1 && use_scratch) {
    if (ws_bytes(B, H, Lq, D, splits) > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_WORKSPACE;
  } else if (splits > 1) {
    if (!ws) return FA_ERR_NULL;
    if (!aligned(ws, 256)) return FA_ERR_ALIGN;
    if (ws_size < ws_bytes(B, H, Lq, D, splits)) return FA_ERR_WORKSPACE;
  }

  // One head's slab is addressed with 32-bit byte offsets, including up to 256
  // rows of tile padding past its end: (len + 256)·row_stride + D elements must
  // stay below 2^31 (checked by division, so that no product can overflow);
  // batch and head offsets are 64-bit.
  const int64_t lens[4] = {Lq, Lk, Lk, Lq};
  for (int i = 0; i < 4; ++i)
    if (st[i][2] > ((1ll << 31) - 1 - D) / (lens[i] + 256)) return FA_ERR_SHAPE;
  if (splits > 1 && ((int64_t)Lq + 256) * D * 4 >= (1ll << 32)) return FA_ERR_SHAPE;  // one partial slab
  const FwdPlan pl = plan_fwd(B, H, Lq, causal, splits, drop_t);
  const int64_t n_qt = pl.n_qt, num_wg = pl.num_wg;
  const bool narrow = pl.narrow;
  if ((int64_t)B * H >= (1ll << 31) || num_wg >= (1ll << 22)) return FA_ERR_SHAPE;

  if (splits > 1 && use_scratch) {  // every argument is valid: now the one HIP query
    ws = scratch_ptr();
    if (!ws) return FA_ERR_DEVICE;
    ws_size = FA_NOALLOC_SCRATCH_BYTES;
  }

  fa355::FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.Lq = Lq;
  p.Lk = Lk;
  p.H = H;
  p.q_sb = q_stride[0], p.q_sh = q_stride[1], p.q_sl = (int)q_stride[2];
  p.k_sb = k_stride[0], p.k_sh = k_stride[1], p.k_sl = (int)k_stride[2];
  p.v_sb = v_stride[0], p.v_sh = v_stride[1], p.v_sl = (int)v_stride[2];
  p.o_sb = o_stride[0], p.o_sh = o_stride[1], p.o_sl = (int)o_stride[2];
  p.kv_off = Lk - Lq;  // used only when causal (then >= 0)
  p.n_qt = (int)n_qt;
  p.n_split = splits;
  p.num_wg = (int)num_wg;
  p.bh = (int)((int64_t)B * H);
  p.ws_o = splits > 1 ? (float*)ws : nullptr;
  p.ws_ml = splits > 1 ? (float*)((char*)ws + ws_o_bytes(B, H, Lq, D, splits)) : nullptr;
  p.wg_order = pl.wg_order;
  // The softmax runs in base 2 with the scale folded into one positive factor;
  // a negative scale negates Q (exact in fp16/bf16) and a zero scale zeroes it.
  const double log2e = 1.4426950408889634074;
  p.c = (float)((scale != 0.0f ? fabs((double)scale) : 1.0) * log2e);
  p.q_and = scale == 0.0f ? 0u : 0xffffffffu;
  p.q_xor = scale < 0.0f ? 0x80008000u : 0u;
  p.drop_t = (uint32_t)drop_t;
  p.seed_lo = (uint32_t)seed;
  p.seed_hi = (uint32_t)(seed >> 32);
  p.drop_scale = (float)(256.0 / drop_t);

  fa355::MergeParams m;
  m.ws_o = p.ws_o;
  m.ws_ml = p.ws_ml;
  m.o = o;
  m.lse = lse;
  m.Lq = Lq;
  m.H = H;
  m.n_split = splits;
  m.bh = p.bh;
  m.o_sb = p.o_sb, m.o_sh = p.o_sh, m.o_sl = p.o_sl;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (drop_t < 256) {  // (only the single-pass entry point takes a dropout probability)
    if (narrow)
      return D == 128 ? dispatch_dtype<128, true, 2>(p, m, dtype, causal != 0, s)
                      : dispatch_dtype<64, true, 2>(p, m, dtype, causal != 0, s);
    return D == 128 ? dispatch_dtype<128, true>(p, m, dtype, causal != 0, s)
                    : dispatch_dtype<64, true>(p, m, dtype, causal != 0, s);
  }
  if (narrow)
    return D == 128 ? dispatch_dtype<128, false, 2>(p, m, dtype, causal != 0, s)
                    : dispatch_dtype<64, false, 2>(p, m, dtype, causal != 0, s);
  return D == 128 ? dispatch_dtype<128, false>(p, m, dtype, causal != 0, s)
                  : dispatch_dtype<64, false>(p, m, dtype, causal != 0, s);
}

// ---- backward

constexpr int kBwdDqRows = 256;   // query rows per dQ workgroup
constexpr int kBwdKvKeys = 128;   // keys per dK/dV workgroup

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
// workspace: LSE·log2(e), then Δ, fp32 [B*H][Lq4] each with Lq4 = Lq rounded up to
// a multiple of 4 (the second array 256-byte aligned)
size_t lq4(int Lq) { return ((size_t)Lq + 3) & ~(size_t)3; }
size_t bwd_ws_bytes(int B, int H, int Lq) {
  return align256((size_t)B * H * lq4(Lq) * 4) + (size_t)B * H * lq4(Lq) * 4;
}

template <int D, int DT, bool CAUSAL, bool DROP>
int launch_bwd(fa355::BwdParams p, hipStream_t stream) {
  // the dQ kernel also writes each row's Δ and LSE·log2(e) to the workspace, which
  // the dK/dV kernel (next on the stream) reads
  p.num_wg = p.bh * p.n_qt;
  p.xcd_remap = (p.num_wg % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((fa355::fa_bwd_dq_kernel<D, DT, CAUSAL, DROP>), dim3(p.num_wg), dim3(512), 0, stream, p);
  int st = launch_status();
  if (st != FA_OK) return st;
  p.num_wg = p.bh * p.n_kt;
  p.xcd_remap = (p.num_wg % 8 == 0) ? 1 : 0;
  // D = 128: two waves per key block (measured 10% faster per backward call at
  // the 7B 4K shape); D = 64: one wave doing all four products (half the matrix
  // work per step does not pay for the split's second join: 10% slower there)
  if constexpr (D == 64)
    hipLaunchKernelGGL((fa355::fa_bwd_dkdv_kernel<D, DT, CAUSAL, DROP>), dim3(p.num_wg), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((fa355::fa_bwd_dkdv2_kernel<D, DT, CAUSAL, DROP>), dim3(p.num_wg), dim3(512), 0, stream, p);
  return launch_status();
}

template <int D, bool DROP>
int dispatch_bwd(const fa355::BwdParams& p, int dtype, bool causal, hipStream_t s) {
  if (dtype == FA_DTYPE_BF16)
    return causal ? launch_bwd<D, fa355::DT_BF16, true, DROP>(p, s) : launch_bwd<D, fa355::DT_BF16, false, DROP>(p, s);
  return causal ? launch_bwd<D, fa355::DT_F16, true, DROP>(p, s) : launch_bwd<D, fa355::DT_F16, false, DROP>(p, s);
}

// strides: 24 values, (batch, head, row) element strides of q, k, v, o, dout, dq,
// dk, dv in that order; NULL means dense [B, H, L, D] for all eight.
int bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse, void* dq,
        void* dk, void* dv, int B, int H, int Lq, int Lk, int D, const int64_t* strides, float scale, int causal,
        int dtype, void* ws, size_t ws_size, fa_stream_t stream, float dropout_p = 0.0f, uint64_t seed = 0) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !ws) return FA_ERR_NULL;
  if (B < 1 || H < 1 || Lq < 1 || Lk < 1) return FA_ERR_SHAPE;
  if (D != 64 && D != 128) return FA_ERR_HEAD_DIM;
  if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  // rows of q, o, dout, dq have Lq entries; rows of k, v, dk, dv have Lk
  const int64_t len[8] = {Lq, Lk, Lk, Lq, Lq, Lq, Lk, Lk};
  int64_t st[8][3];
  for (int i = 0; i < 8; ++i) {
    st[i][0] = strides ? strides[3 * i] : (int64_t)H * len[i] * D;
    st[i][1] = strides ? strides[3 * i + 1] : len[i] * D;
    st[i][2] = strides ? strides[3 * i + 2] : D;
    if (st[i][0] < 0 || st[i][1] < 0 || st[i][2] < D) return FA_ERR_STRIDE;
  }
  const void* p16[8] = {q, k, v, o, dout, dq, dk, dv};
  for (int i = 0; i < 8; ++i)
    if (!aligned(p16[i], 16)) return FA_ERR_ALIGN;
  for (int i = 0; i < 8; ++i)  // every row starts on a 16-byte boundary
    if (st[i][0] % 8 || st[i][1] % 8 || st[i][2] % 8) return FA_ERR_ALIGN;
  if (!aligned(lse, 4) || !aligned(ws, 256)) return FA_ERR_ALIGN;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if (causal && Lq > Lk) return FA_ERR_CAUSAL_SHAPE;
  const int drop_t = drop_threshold(dropout_p);
  if (drop_t < 0) return FA_ERR_DROPOUT;
  if (ws_size < bwd_ws_bytes(B, H, Lq)) return FA_ERR_WORKSPACE;
  // one head's slab plus a tile of padding in 32-bit byte offsets
  for (int i = 0; i < 8; ++i)  // (len + 256)·row_stride + D < 2^31, by division (no overflow)
    if (st[i][2] > ((1ll << 31) - 1 - D) / (len[i] + 256)) return FA_ERR_SHAPE;
  const int64_t n_qt = ((int64_t)Lq + kBwdDqRows - 1) / kBwdDqRows;
  const int64_t n_kt = ((int64_t)Lk + kBwdKvKeys - 1) / kBwdKvKeys;
  if ((int64_t)B * H >= (1ll << 31) || (int64_t)B * H * n_qt >= (1ll << 22) || (int64_t)B * H * n_kt >= (1ll << 22))
    return FA_ERR_SHAPE;

  fa355::BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.ws_lse2 = (float*)ws;
  p.ws_delta = (float*)((char*)ws + align256((size_t)B * H * lq4(Lq) * 4));
  p.Lq = Lq;
  p.Lq4 = (int)lq4(Lq);
  p.Lk = Lk;
  p.bh = (int)((int64_t)B * H);
  p.H = H;
  for (int i = 0; i < 8; ++i) {
    p.sb[i] = st[i][0];
    p.sh[i] = st[i][1];
    p.sl[i] = (int)st[i][2];
  }
  p.kv_off = Lk - Lq;
  p.n_qt = (int)n_qt;
  p.n_kt = (int)n_kt;
  p.num_wg = 0;
  p.xcd_remap = 0;
  p.c = (float)((double)scale * 1.4426950408889634074);
  p.scale = scale;
  p.drop_t = (uint32_t)drop_t;
  p.seed_lo = (uint32_t)seed;
  p.seed_hi = (uint32_t)(seed >> 32);
  p.drop_scale = (float)(256.0 / drop_t);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (drop_t < 256)
    return D == 128 ? dispatch_bwd<128, true>(p, dtype, causal != 0, s)
                    : dispatch_bwd<64, true>(p, dtype, causal != 0, s);
  return D == 128 ? dispatch_bwd<128, false>(p, dtype, causal != 0, s)
                  : dispatch_bwd<64, false>(p, dtype, causal != 0, s);
}

}  // namespace

extern "C" {

int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lq, int Lk,
                   int D, const int64_t* q_stride, const int64_t* k_stride, const int64_t* v_stride,
                   const int64_t* o_stride, float scale, int causal, int dtype, fa_stream_t stream) {
  return fwd(q, k, v, o, lse, B, H, Lq, Lk, D, q_stride, k_stride, v_stride, o_stride, scale, causal, dtype, 1,
             nullptr, 0, stream);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lq, int Lk, int D,
           float scale, int causal, int dtype, fa_stream_t stream) {
  // dense [B, H, L, D]: the strided form with the natural strides
  const int64_t sq[3] = {(int64_t)H * Lq * D, (int64_t)Lq * D, D};
  const int64_t sk[3] = {(int64_t)H * Lk * D, (int64_t)Lk * D, D};
  return fwd(q, k, v, o, lse, B, H, Lq, Lk, D, sq, sk, sk, sq, scale, causal, dtype, 1, nullptr, 0, stream);
}

size_t fa_fwd_splitkv_workspace_size(int B, int H, int Lq, int D, int num_splits) {
  if (B < 1 || H < 1 || Lq < 1 || (D != 64 && D != 128) || num_splits < 1 || num_splits > kMaxSplits) return 0;
  return ws_bytes(B, H, Lq, D, num_splits);
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lq, int Lk,
                   int D, const int64_t* q_stride, const int64_t* k_stride, const int64_t* v_stride,
                   const int64_t* o_stride, float scale, int causal, int dtype, int num_splits, void* workspace,
                   size_t workspace_bytes, fa_stream_t stream) {
  return fwd(q, k, v, o, lse, B, H, Lq, Lk, D, q_stride, k_stride, v_stride, o_stride, scale, causal, dtype,
             num_splits, workspace, workspace_bytes, stream);
}

int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lq,
                           int Lk, int D, const int64_t* q_stride, const int64_t* k_stride, const int64_t* v_stride,
                           const int64_t* o_stride, float scale, int causal, int dtype, int num_splits,
                           fa_stream_t stream) {
  return fwd(q, k, v, o, lse, B, H, Lq, Lk, D, q_stride, k_stride, v_stride, o_stride, scale, causal, dtype,
             num_splits, nullptr, 0, stream, 0.0f, 0, true);
}

size_t fa_bwd_workspace_size(int B, int H, int Lq) {
  if (B < 1 || H < 1 || Lq < 1) return 0;
  return bwd_ws_bytes(B, H, Lq);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse, void* dq,
           void* dk, void* dv, int B, int H, int Lq, int Lk, int D, float scale, int causal, int dtype,
           void* workspace, size_t workspace_bytes, fa_stream_t stream) {
  return bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Lq, Lk, D, nullptr, scale, causal, dtype, workspace,
             workspace_bytes, stream);
}

int fa_bwd_strided(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int Lq, int Lk, int D, const int64_t* strides,
                   float scale, int causal, int dtype, float dropout_p, uint64_t seed, void* workspace,
                   size_t workspace_bytes, fa_stream_t stream) {
  if (!strides) return FA_ERR_NULL;
  return bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Lq, Lk, D, strides, scale, causal, dtype, workspace,
             workspace_bytes, stream, dropout_p, seed);
}

int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lq, int Lk,
                   int D, float scale, int causal, int dtype, float dropout_p, uint64_t seed, fa_stream_t stream) {
  const int64_t sq[3] = {(int64_t)H * Lq * D, (int64_t)Lq * D, D};
  const int64_t sk[3] = {(int64_t)H * Lk * D, (int64_t)Lk * D, D};
  return fwd(q, k, v, o, lse, B, H, Lq, Lk, D, sq, sk, sk, sq, scale, causal, dtype, 1, nullptr, 0, stream, dropout_p,
             seed);
}

int fa_fwd_dropout_strided(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lq,
                           int Lk, int D, const int64_t* q_stride, const int64_t* k_stride, const int64_t* v_stride,
                           const int64_t* o_stride, float scale, int causal, int dtype, float dropout_p,
                           uint64_t seed, fa_stream_t stream) {
  return fwd(q, k, v, o, lse, B, H, Lq, Lk, D, q_stride, k_stride, v_stride, o_stride, scale, causal, dtype, 1,
             nullptr, 0, stream, dropout_p, seed);
}

int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int Lq, int Lk, int D, float scale, int causal,
                   int dtype, float dropout_p, uint64_t seed, void* workspace, size_t workspace_bytes,
                   fa_stream_t stream) {
  return bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Lq, Lk, D, nullptr, scale, causal, dtype, workspace,
             workspace_bytes, stream, dropout_p, seed);
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL (q, k, v, o, lse; dout, dq, dk, dv or workspace for fa_bwd)";
    case FA_ERR_SHAPE: return "fa_fwd: B, H, Lq and Lk must be >= 1 and within the size limits";
    case FA_ERR_HEAD_DIM: return "fa_fwd: head dimension D must be 64 or 128";
    case FA_ERR_DTYPE: return "fa_fwd: dtype must be FA_DTYPE_F16 (0) or FA_DTYPE_BF16 (1)";
    case FA_ERR_ALIGN: return "fa_fwd: q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
    case FA_ERR_SCALE: return "fa_fwd: scale must be finite";
    case FA_ERR_CAUSAL_SHAPE: return "fa_fwd: causal attention requires Lq <= Lk";
    case FA_ERR_DEVICE: return "fa_fwd: no gfx950 kernel for the current device";
    case FA_ERR_LAUNCH: return "fa_fwd: kernel launch failed (see fa_last_hip_error)";
    case FA_ERR_STRIDE: return "fa_fwd: strides must be >= 0, with a row stride of at least D";
    case FA_ERR_SPLITS: return "fa_fwd_splitkv: num_splits must be between 1 and 256";
    case FA_ERR_DROPOUT: return "dropout probability must be in [0, 1) with round((1 - p) * 256) >= 1";
    case FA_ERR_WORKSPACE:
      return "workspace smaller than the size query returns (fa_fwd_splitkv / fa_bwd), or partials larger than "
             "the scratch array of fa_fwd_splitkv_noalloc";
    default: return "fa_fwd: unknown status code";
  }
}

int fa_last_hip_error(void) { return g_last_hip_error; }

int fa_version(void) { return kVersion; }

int fa_fwd_launch_shape(int B, int H, int Lq, int Lk, int D, int causal, float dropout_p, int num_splits,
                        int* workgroups, int* rows_per_workgroup, int* items_per_workgroup) {
  if (!workgroups || !rows_per_workgroup || !items_per_workgroup) return FA_ERR_NULL;
  if (B < 1 || H < 1 || Lq < 1 || Lk < 1) return FA_ERR_SHAPE;
  if (D != 64 && D != 128) return FA_ERR_HEAD_DIM;
  if (causal && Lq > Lk) return FA_ERR_CAUSAL_SHAPE;
  const int drop_t = drop_threshold(dropout_p);
  if (drop_t < 0) return FA_ERR_DROPOUT;
  if (num_splits < 1 || num_splits > kMaxSplits || (drop_t < 256 && num_splits > 1)) return FA_ERR_SPLITS;
  const FwdPlan pl = plan_fwd(B, H, Lq, causal, num_splits, drop_t);
  if ((int64_t)B * H >= (1ll << 31) || pl.num_wg >= (1ll << 22)) return FA_ERR_SHAPE;
  *workgroups = (int)pl.num_wg;
  *rows_per_workgroup = pl.narrow ? fa355::Geo<128, 8, 2>::BR : fa355::Geo<128>::BR;
  *items_per_workgroup = pl.n_rep;
  return FA_OK;
}

}  // extern "C"
