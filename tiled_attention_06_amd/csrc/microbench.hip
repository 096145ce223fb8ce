// Microbenchmarks of the MI355X units the attention kernels are bound by: the
// rates that say what a fraction of the datasheet peak can mean on the box.
// Built into libfa355_mb.so, separate from libfa355 (nothing on the attention
// path uses it); bench.py --microbench runs them.
//
//   mb_mfma   v_mfma_f32_32x32x16_bf16 throughput: every wave runs eight
//             independent accumulation chains on operands loaded from memory
//             (random data: all-zero operands draw less power and let the clock
//             rise, which would overstate the rate the attention kernel sees)
//   mb_exp    v_exp_f32 throughput: eight independent chains x <- 2^-x per lane (the
//             negation is a free input modifier)
//   mb_lds    ds_read_b128 bandwidth out of LDS: eight waves per CU read 16-byte
//             rows of a resident 128 KB block at a conflict-free lane pattern
//   mb_copy   HBM copy with 16-byte loads and stores (grid-stride)
//
//
// Each kernel writes one value per lane derived from its results so that no
// work can be removed, and each takes an iteration count so that a launch can be
// made long enough (tens of milliseconds) for the clock to settle under the load.
// The clock of a run is measured in the kernel itself: cycle counter against the
// 100 MHz real-time counter over workgroup 0's lifetime.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Shader clock over a wave's lifetime: the 64-bit cycle counter (s_memtime) and
// the 100 MHz real-time counter (s_memrealtime) read at the start and the end by
// thread 0 of workgroup 0 (every workgroup of these kernels runs for the whole
// launch), written with an ordinary vector store.
struct Stamp {
  uint64_t cyc, rt;
};
__device__ __forceinline__ Stamp stamp() {
  Stamp s;
  s.rt = __builtin_amdgcn_s_memrealtime();
  s.cyc = __builtin_amdgcn_s_memtime();
  return s;
}
__device__ __forceinline__ void put_clock(uint64_t* clk, const Stamp& a) {
  if (clk && blockIdx.x == 0 && threadIdx.x == 0) {
    const Stamp b = stamp();
    clk[0] = b.cyc - a.cyc;
    clk[1] = b.rt - a.rt;
  }
}

__global__ __launch_bounds__(256) void mb_mfma_kernel(const u32x4* __restrict__ src, float* __restrict__ out,
                                                      int iters, uint64_t* clk) {
  const Stamp t0 = stamp();
  const int lane = threadIdx.x & 63;
  const u32x4 a0 = src[lane], a1 = src[64 + lane], b0 = src[128 + lane], b1 = src[192 + lane];
  const bf16x8 A0 = __builtin_bit_cast(bf16x8, a0), A1 = __builtin_bit_cast(bf16x8, a1);
  const bf16x8 B0 = __builtin_bit_cast(bf16x8, b0), B1 = __builtin_bit_cast(bf16x8, b1);
  f32x16 c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16((j & 1) ? A1 : A0, (j & 2) ? B1 : B0, c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[j][r];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
  put_clock(clk, t0);
}

__global__ __launch_bounds__(256) void mb_exp_kernel(const float* __restrict__ src, float* __restrict__ out,
                                                     int iters, uint64_t* clk) {
  const Stamp t0 = stamp();
  const int t = threadIdx.x;
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = 0.5f + 0.25f * src[(t + 37 * j) & 255];
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);  // stays in (0.5, 1]: no overflow
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += x[j];
  out[(size_t)blockIdx.x * blockDim.x + t] = s;
  put_clock(clk, t0);
}

// 128 KB of LDS as 8192 rows of 16 bytes, 8 waves per workgroup (one workgroup
// per CU).  In iteration it, lane l of wave w reads rows r + 64j (j < 8) with
// r = (1024w + l + 512·it) mod 4096: the 64 lanes of one read cover 1 KB of
// consecutive bytes (every bank once per 256 bytes, no conflict), the eight reads
// share one address register with immediate offsets, and every byte read is
// xored into the result (four 32-bit xors per 16-byte read).
__global__ __launch_bounds__(512) void mb_lds_kernel(const u32x4* __restrict__ src, uint32_t* __restrict__ out,
                                                     int iters, uint64_t* clk) {
  const Stamp t0 = stamp();
  __shared__ u32x4 buf[8192];
  for (int i = threadIdx.x; i < 8192; i += blockDim.x) buf[i] = src[i];
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int it = 0; it < iters; ++it) {
    const u32x4* p = buf + ((1024 * wave + lane + 512 * it) & 4095);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= p[64 * j];
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  put_clock(clk, t0);
}

__global__ __launch_bounds__(256) void mb_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                      size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

int status() { return (int)hipGetLastError(); }

}  // namespace

extern "C" {

// src: >= 256 16-byte values (random bits of bf16 operands); out: grid*256 floats.
// clk (optional): 2 uint64, shader cycles and 100 MHz ticks over workgroup 0's lifetime.
int mb_mfma(const void* src, float* out, int grid, int iters, uint64_t* clk, hipStream_t stream) {
  if (!src || !out || grid < 1 || iters < 1) return -1;
  hipLaunchKernelGGL(mb_mfma_kernel, dim3(grid), dim3(256), 0, stream, (const u32x4*)src, out, iters, clk);
  return status();
}

// src: >= 256 floats; out: grid*256 floats.
int mb_exp(const float* src, float* out, int grid, int iters, uint64_t* clk, hipStream_t stream) {
  if (!src || !out || grid < 1 || iters < 1) return -1;
  hipLaunchKernelGGL(mb_exp_kernel, dim3(grid), dim3(256), 0, stream, src, out, iters, clk);
  return status();
}

// src: >= 8192 16-byte values; out: grid*512 uint32.
int mb_lds(const void* src, uint32_t* out, int grid, int iters, uint64_t* clk, hipStream_t stream) {
  if (!src || !out || grid < 1 || iters < 1) return -1;
  hipLaunchKernelGGL(mb_lds_kernel, dim3(grid), dim3(512), 0, stream, (const u32x4*)src, out, iters, clk);
  return status();
}

// bytes: a multiple of 16; src and dst 16-byte aligned, not overlapping.
int mb_copy(const void* src, void* dst, size_t bytes, int grid, hipStream_t stream) {
  if (!src || !dst || bytes % 16 || grid < 1) return -1;
  hipLaunchKernelGGL(mb_copy_kernel, dim3(grid), dim3(256), 0, stream, (const u32x4*)src, (u32x4*)dst, bytes / 16);
  return status();
}

}  // extern "C"
