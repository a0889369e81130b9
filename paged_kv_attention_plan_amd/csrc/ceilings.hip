// Measurement probes for the benchmark, built as their own library
// (libpkv_ceilings.so) next to libpkv.so and used by nothing on the attention
// path: what this GPU sustains on a pure bf16 MFMA loop and on a pure
// streaming read, the two rates the attention kernels are bound by.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

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
__global__ __launch_bounds__(256, 2) void mfma16_loop_kernel(float* out, int iters) {
  const uint32_t t = threadIdx.x;
  u32x4_t ai = {t * 2654435761u, t ^ 0x3f800000u, t + 7u, t * 97u};
  u32x4_t bi = {t + 1u, t * 3u, t ^ 0x40000000u, t * 13u};
  ai &= 0x3fff3fffu;
  bi &= 0x3fff3fffu;
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, ai);
  const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bi);
  f32x4_t c[8] = {};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      c[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16((k & 1) ? a : b, (k & 2) ? a : b, c[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += c[k][0] + c[k][1] + c[k][2] + c[k][3];
  out[(size_t)blockIdx.x * blockDim.x + t] = s;
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

// out: device float[blocks * 256].  FLOPs = blocks * 4 waves * iters * 8 * 16384.
int pkv_ceiling_mfma16(float* out, int blocks, int iters, void* stream) {
  if (out == nullptr || blocks < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(mfma16_loop_kernel, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

// src: device buffer of `bytes` (a multiple of 16); out: device uint32[blocks * 256].
int pkv_ceiling_read(const void* src, int64_t bytes, uint32_t* out, int blocks, void* stream) {
  if (src == nullptr || out == nullptr || blocks < 1 || bytes < 16 || (bytes & 15) != 0) return 1;
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4_t*>(src), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // extern "C"
