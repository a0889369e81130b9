// Split-KV merge, KV append and the plan metadata upload.
//
// Merge (the workspace page, mstar attn.workspace, keeps split-KV partials):
// a row whose keys were cut into chunks c has, per query head, a partial output
// o_c normalised over chunk c alone and its log-sum-exp lse_c.  Over all keys,
// lse = ln sum_c exp(lse_c) and out = sum_c exp(lse_c - lse) * o_c.
//
// Append (FlashInferDecodeWrapper.plan computes the write location; the KV
// resource stores K/V before attention runs, attn.dense requires_kv_write):
// token t's K row goes to cache[page, 0, off] and its V row to
// cache[page, 1, off] with page * page_size + off = slot[t].
//
// Upload (kv.plan PinnedIndexRing stages the plan in page-locked memory): the
// GPU reads the staged bytes over the host link and stores them into the
// workspace.  For the tens to hundreds of KB of a plan this costs a few
// microseconds, where a DMA copy pays its engine's start-up latency.
#include "common.cuh"
#include "kernels.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;

// One workgroup per (merge entry, query head).  The log-sum-exp of all chunks
// is found first (every lane reads a strided subset of the chunk LSEs); then
// each wave accumulates a quarter of the chunks with all of its loads
// independent, and the four partial sums are added through LDS.
template <int D>
__global__ __launch_bounds__(64 * kWaves) void merge_kernel(MergeArgs a) {
  constexpr int E = D / 64;  // output elements per lane
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.group;
  const int mi = blockIdx.x / G, h = blockIdx.x - mi * G;
  const pkv_merge_entry e = a.merges[mi];
  const int n = e.n_chunks;
  const float* pl = a.part_lse + (int64_t)e.slot_base * G + h;
  __shared__ float red[kWaves][D + 1];
  __shared__ float s_max[kWaves];

  float M = -INFINITY;
  for (int c = threadIdx.x; c < n; c += 64 * kWaves) M = fmaxf(M, pl[(int64_t)c * G]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if (lane == 0) s_max[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));

  float wsum = 0.f, acc[E];
#pragma unroll
  for (int k = 0; k < E; ++k) acc[k] = 0.f;
  const float* po = a.part_o + ((int64_t)e.slot_base * G + h) * D + lane * E;
  const int64_t cstride = (int64_t)G * D;
#pragma unroll 4
  for (int c = wave; c < n; c += kWaves) {
    const float wc = __expf(pl[(int64_t)c * G] - M);
    wsum += wc;
#pragma unroll
    for (int k = 0; k < E; ++k) acc[k] = fmaf(wc, po[c * cstride + k], acc[k]);
  }
#pragma unroll
  for (int k = 0; k < E; ++k) red[wave][lane * E + k] = acc[k];
  if (lane == 0) red[wave][D] = wsum;
  __syncthreads();
  if (wave != 0) return;
  float tot = red[0][D] + red[1][D] + red[2][D] + red[3][D];
#pragma unroll
  for (int k = 0; k < E; ++k)
    acc[k] = red[0][lane * E + k] + red[1][lane * E + k] + red[2][lane * E + k] + red[3][lane * E + k];
  const float inv = 1.f / tot;
  const int qh = e.kv_head * G + h;
  uint16_t* dst = a.out + ((int64_t)e.q_index * a.num_qo_heads + qh) * D + lane * E;
  if constexpr (E == 2) {
    *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  } else {
    dst[0] = (uint16_t)bf16_rne(acc[0] * inv);
  }
  if (a.lse != nullptr && lane == 0)
    a.lse[(int64_t)e.q_index * a.num_qo_heads + qh] = M + logf(tot);
}

__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int t = blockIdx.x;
  const int64_t slot = a.slots[t];
  const int ps = a.page_size;
  const int64_t page = slot / ps;
  const int off = (int)(slot - page * ps);
  const int row = a.num_kv_heads * a.head_dim;  // elements per token slot
  const int nvec = row / 8;                     // 16-byte vectors per row
  uint16_t* dk = a.cache + ((page * 2 + 0) * ps + off) * (int64_t)row;
  uint16_t* dv = dk + (int64_t)ps * row;
  const uint4* sk = reinterpret_cast<const uint4*>(a.k_new + (int64_t)t * row);
  const uint4* sv = reinterpret_cast<const uint4*>(a.v_new + (int64_t)t * row);
  for (int i = threadIdx.x; i < 2 * nvec; i += blockDim.x) {
    if (i < nvec) reinterpret_cast<uint4*>(dk)[i] = sk[i];
    else reinterpret_cast<uint4*>(dv)[i - nvec] = sv[i - nvec];
  }
}

__global__ __launch_bounds__(256) void upload_kernel(UploadArgs a) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.n_vec; i += stride)
    a.dst[i] = a.src[i];
}

}  // namespace

hipError_t launch_upload(const UploadArgs& a, hipStream_t stream) {
  if (a.n_vec <= 0) return hipSuccess;
  // Every vector in flight at once up to 256 workgroups (1 MiB); larger
  // plans loop.
  int64_t blocks = (a.n_vec + 255) / 256;
  blocks = blocks > 256 ? 256 : blocks;
  hipLaunchKernelGGL(upload_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  if (a.n_merges <= 0) return hipSuccess;
  const dim3 grid(a.n_merges * a.group), block(64 * kWaves);
  if (a.head_dim == 128) hipLaunchKernelGGL(merge_kernel<128>, grid, block, 0, stream, a);
  else if (a.head_dim == 64) hipLaunchKernelGGL(merge_kernel<64>, grid, block, 0, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  if (a.n_tokens <= 0) return hipSuccess;
  const int nvec2 = 2 * a.num_kv_heads * a.head_dim / 8;
  int threads = ((nvec2 + 63) / 64) * 64;
  threads = threads > 256 ? 256 : threads;
  hipLaunchKernelGGL(append_kernel, dim3(a.n_tokens), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
