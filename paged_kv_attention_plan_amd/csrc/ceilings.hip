// Measurement probes for the benchmark, built as their own library
// (libpkv_ceilings.so) next to libpkv.so and used by nothing on the attention
// path: what this GPU sustains on a pure bf16 MFMA loop and on a pure
// streaming read, the two rates the attention kernels are bound by, and the
// shader clock while the MFMA loops run.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

// Shader-clock cycles (s_memtime) and constant-rate ticks (s_memrealtime,
// hipDeviceAttributeWallClockRate); each waits for its own result.
__device__ __forceinline__ uint64_t shader_cycles() {
  uint64_t t;
  asm volatile("s_memtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t));
  return t;
}
__device__ __forceinline__ uint64_t wall_ticks() {
  uint64_t t;
  asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t));
  return t;
}
// clk (optional, device): clk[0] += the wave's shader cycles over its loop,
// clk[1] += its wall ticks; the ratio times the wall-clock rate is the clock.
__device__ __forceinline__ void add_clock(unsigned long long* clk, uint64_t c0, uint64_t r0) {
  const uint64_t c1 = shader_cycles(), r1 = wall_ticks();
  if (clk != nullptr && (threadIdx.x & 63) == 0) {
    atomicAdd(&clk[0], (unsigned long long)(c1 - c0));
    atomicAdd(&clk[1], (unsigned long long)(r1 - r0));
  }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Every wave runs `iters` rounds of four independent v_mfma_f32_32x32x16_bf16
// chains on register operands (32768 FLOP each), then stores one value per
// lane so that the work is kept.
__global__ __launch_bounds__(256, 2) void mfma_loop_kernel(float* out, int iters) {
  const uint32_t t = threadIdx.x;
  u32x4_t ai = {t * 2654435761u, t ^ 0x3f800000u, t + 7u, t * 97u};
  u32x4_t bi = {t + 1u, t * 3u, t ^ 0x40000000u, t * 13u};
  // keep the operands finite: clear the top exponent bit of every bf16
  ai &= 0x3fff3fffu;
  bi &= 0x3fff3fffu;
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, ai);
  const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bi);
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) s += c0[k] + c1[k] + c2[k] + c3[k];
  out[(size_t)blockIdx.x * blockDim.x + t] = s;
}

// The same with v_mfma_f32_16x16x32_bf16 (16384 FLOP each), the shape of the
// prefill kernel: eight independent chains per wave.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256, 2) void mfma16_loop_kernel(float* out,
                                                             unsigned long long* clk, int iters) {
  const uint32_t t = threadIdx.x;
  u32x4_t ai = {t * 2654435761u, t ^ 0x3f800000u, t + 7u, t * 97u};
  u32x4_t bi = {t + 1u, t * 3u, t ^ 0x40000000u, t * 13u};
  ai &= 0x3fff3fffu;
  bi &= 0x3fff3fffu;
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, ai);
  const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bi);
  f32x4_t c[8] = {};
  const uint64_t c0 = shader_cycles(), r0 = wall_ticks();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      c[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16((k & 1) ? a : b, (k & 2) ? a : b, c[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += c[k][0] + c[k][1] + c[k][2] + c[k][3];
  add_clock(clk, c0, r0);
  out[(size_t)blockIdx.x * blockDim.x + t] = s;
}

// The same product with operands that change from one MFMA to the next, as
// in any real contraction: sixteen pseudo-random operand pairs per lane, taken
// in turn (16 products per round, iters / 2 rounds).  The multipliers' power
// grows with the input bits that toggle between products: with the fixed
// operands above the clock holds its maximum, with changing ones it settles
// lower, so this loop gives the rate the matrix cores sustain on real data.
// Every bf16 operand has bit 14 clear and bit 13 set (magnitude in
// [2^-63, 2)), so products and sums stay finite and normal.
__global__ __launch_bounds__(256, 2) void mfma16_rot_kernel(float* out, unsigned long long* clk,
                                                            int iters) {
  uint32_t h = (threadIdx.x + 1u) * 0x9e3779b9u ^ (blockIdx.x + 1u) * 0x85ebca6bu;
  auto next = [&h]() {  // xorshift32
    h ^= h << 13;
    h ^= h >> 17;
    h ^= h << 5;
    return (h & 0xbfffbfffu) | 0x20002000u;
  };
  u32x4_t av[16], bv[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    av[k] = u32x4_t{next(), next(), next(), next()};
    bv[k] = u32x4_t{next(), next(), next(), next()};
  }
  f32x4_t c[8] = {};
  const uint64_t c0 = shader_cycles(), r0 = wall_ticks();
  for (int i = 0; i < iters; i += 2) {
#pragma unroll
    for (int k = 0; k < 16; ++k)
      c[k & 7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8_t, av[k]), __builtin_bit_cast(bf16x8_t, bv[(5 * k + 3) & 15]),
          c[k & 7], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += c[k][0] + c[k][1] + c[k][2] + c[k][3];
  add_clock(clk, c0, r0);
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Grid-stride read of n_vec 16-byte vectors (non-temporal: each byte once),
// four loads in flight per thread, folded into one word per thread.
__global__ __launch_bounds__(256) void read_kernel(const u32x4_t* src, int64_t n_vec,
                                                   uint32_t* out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  u32x4_t x = {0u, 0u, 0u, 0u};
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n_vec; i += 4 * stride) {
    const u32x4_t a = __builtin_nontemporal_load(src + i);
    const u32x4_t b = __builtin_nontemporal_load(src + i + stride);
    const u32x4_t c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4_t d = __builtin_nontemporal_load(src + i + 3 * stride);
    x ^= a ^ b ^ c ^ d;
  }
  for (; i < n_vec; i += stride) x ^= __builtin_nontemporal_load(src + i);
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

}  // namespace

extern "C" {

// out: device float[blocks * 256].  FLOPs = blocks * 4 waves * iters * 4 * 32768.
int pkv_ceiling_mfma(float* out, int blocks, int iters, void* stream) {
  if (out == nullptr || blocks < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

// out: device float[blocks * 256]; clk: device uint64[2] or null (see
// add_clock).  FLOPs = blocks * 4 waves * iters * 8 * 16384.
int pkv_ceiling_mfma16(float* out, unsigned long long* clk, int blocks, int iters, void* stream) {
  if (out == nullptr || blocks < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(mfma16_loop_kernel, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), out, clk, iters);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

// As pkv_ceiling_mfma16, with changing operands; iters must be even.
int pkv_ceiling_mfma16_rot(float* out, unsigned long long* clk, int blocks, int iters,
                           void* stream) {
  if (out == nullptr || blocks < 1 || iters < 2 || (iters & 1) != 0) return 1;
  hipLaunchKernelGGL(mfma16_rot_kernel, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), out, clk, iters);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

// Rate of the constant wall clock that s_memrealtime counts, in kHz (0 on error).
int pkv_ceiling_wallclock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz;
}

// src: device buffer of `bytes` (a multiple of 16); out: device uint32[blocks * 256].
int pkv_ceiling_read(const void* src, int64_t bytes, uint32_t* out, int blocks, void* stream) {
  if (src == nullptr || out == nullptr || blocks < 1 || bytes < 16 || (bytes & 15) != 0) return 1;
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4_t*>(src), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // extern "C"
