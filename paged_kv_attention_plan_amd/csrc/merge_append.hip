// Split-KV merge, KV append, the plan metadata upload and the dense gather.
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

// Each (merge entry, query head) pair is merged by W waves (W = kWaves for
// entries with many chunks, one wave otherwise, four pairs per workgroup).
// A wave takes chunks c = w, w + W, ... in batches of U: lane i loads the LSE
// of the batch's i-th chunk while every lane loads its slice of all U partial
// outputs, so a batch costs one round trip to memory.  The wave keeps a
// running maximum, so no pass over the LSEs precedes the sums.  With W > 1
// the waves' (max, sum, acc) meet in LDS and are rescaled to the common
// maximum there.
template <int D, int W>
__global__ __launch_bounds__(64 * kWaves) void merge_kernel(MergeArgs a) {
  constexpr int E = D / 64;          // output elements per lane
  constexpr int U = W == 1 ? 8 : 16;  // chunks per batch
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.group;
  // pair index and this wave's rank among the pair's W waves
  const int pair = W == 1 ? blockIdx.x * kWaves + wave : blockIdx.x;
  const int rank = W == 1 ? 0 : wave;
  const int n_merges = a.counts != nullptr ? (int)as_const4(a.counts)[1] : a.n_merges;
  if (pair >= n_merges * G) return;
  const int mi = pair / G, h = pair - mi * G;
  const pkv_merge_entry e = a.merges[mi];
  const int n = e.n_chunks;
  const float* pl = a.part_lse + (int64_t)e.slot_base * G + h;
  const float* po = a.part_o + ((int64_t)e.slot_base * G + h) * D + lane * E;
  const int64_t cstride = (int64_t)G * D;

  float m_w = -INFINITY, wsum = 0.f, acc[E];
#pragma unroll
  for (int k = 0; k < E; ++k) acc[k] = 0.f;
  for (int c0 = rank; c0 < n; c0 += W * U) {
    // lane i: LSE of chunk c0 + (i mod U) W (clamped; every lane loads, so the
    // load is issued with the partials and not behind a branch)
    const int cl = c0 + (lane & (U - 1)) * W;
    const float lv = pl[(int64_t)(cl < n ? cl : n - 1) * G];
    float o[U][E];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * W;
      const int cc = c < n ? c : n - 1;  // in-range address; its weight is zero
#pragma unroll
      for (int k = 0; k < E; ++k) o[u][k] = po[cc * cstride + k];
    }
    float l[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      l[u] = c0 + u * W < n
                 ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lv), u))
                 : -INFINITY;
    // chunk c0 exists, so mb and mn are finite
    float mb = l[0];
#pragma unroll
    for (int u = 1; u < U; ++u) mb = fmaxf(mb, l[u]);
    const float mn = fmaxf(m_w, mb);
    const float sc = __expf(m_w - mn);
    wsum *= sc;
#pragma unroll
    for (int k = 0; k < E; ++k) acc[k] *= sc;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float wc = __expf(l[u] - mn);
      wsum += wc;
#pragma unroll
      for (int k = 0; k < E; ++k) acc[k] = fmaf(wc, o[u][k], acc[k]);
    }
    m_w = mn;
  }
  float M = m_w, tot = wsum;
  if constexpr (W > 1) {
    __shared__ float red[W][D];
    __shared__ float s_m[W], s_s[W];
#pragma unroll
    for (int k = 0; k < E; ++k) red[wave][lane * E + k] = acc[k];
    if (lane == 0) {
      s_m[wave] = m_w;
      s_s[wave] = wsum;
    }
    __syncthreads();
    if (wave != 0) return;
    M = s_m[0];
#pragma unroll
    for (int w = 1; w < W; ++w) M = fmaxf(M, s_m[w]);
    tot = 0.f;
#pragma unroll
    for (int k = 0; k < E; ++k) acc[k] = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      // a wave without chunks holds max -inf and contributes nothing
      const float f = s_m[w] == -INFINITY ? 0.f : __expf(s_m[w] - M);
      tot = fmaf(f, s_s[w], tot);
#pragma unroll
      for (int k = 0; k < E; ++k) acc[k] = fmaf(f, red[w][lane * E + k], acc[k]);
    }
  }
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

// One workgroup per token.  The token's K and V vectors are requested before
// the slot is needed, so the slot load and the data loads share one round
// trip; page_size is a power of two, so the slot splits by shift and mask.
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int t = blockIdx.x;
  if (a.counts != nullptr && t >= (int)as_const4(a.counts)[4]) return;
  const int64_t slot = a.slots[t];
  const int ps = a.page_size;
  const int ps_log2 = __builtin_ctz(ps);
  const int row = a.num_kv_heads * a.head_dim;  // elements per token slot
  const int nvec = row / 8;                     // 16-byte vectors per row
  const uint4* sk = reinterpret_cast<const uint4*>(a.k_new + (int64_t)t * row);
  const uint4* sv = reinterpret_cast<const uint4*>(a.v_new + (int64_t)t * row);
  auto store = [&](int i, const uint4& v) {
    const int64_t page = slot >> ps_log2;
    const int off = (int)(slot & (ps - 1));
    uint16_t* dk = a.cache + ((page * 2 + 0) * ps + off) * (int64_t)row;
    uint16_t* dst = i < nvec ? dk : dk + (int64_t)ps * row;
    reinterpret_cast<uint4*>(dst)[i < nvec ? i : i - nvec] = v;
  };
  // The first vector of each thread (all of them when 2 nvec <= blockDim) is
  // loaded before any use of the slot.
  const int i0 = threadIdx.x;
  if (i0 < 2 * nvec) {
    const uint4 v = i0 < nvec ? sk[i0] : sv[i0 - nvec];
    // keep the slot arithmetic (and its wait) behind the load's issue
    __builtin_amdgcn_sched_barrier(0);
    store(i0, v);
  }
  for (int i = i0 + blockDim.x; i < 2 * nvec; i += blockDim.x) store(i, i < nvec ? sk[i] : sv[i - nvec]);
}

// Dense gather (attn.dense DenseAttentionManager: the frozen prefix gathered
// from the pages and the step's fresh K/V concatenated after it): one wave per
// copied token.  With the prefix, wave t copies dense row t, and its (request)
// row is the last with cu_k <= t; without it, wave t copies fresh token t, and
// its row is the last with cu_q <= t.  Rows are found by binary search over
// the row table.
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= (a.with_prefix ? a.total_k : (int64_t)a.total_q)) return;
  int lo = 0, hi = a.n_rows - 1;  // rows[0] starts at 0, so rows[lo] starts at or before t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((a.with_prefix ? a.rows[mid].cu_k : a.rows[mid].cu_q) <= t) lo = mid;
    else hi = mid - 1;
  }
  const DenseRowMeta rm = a.rows[lo];
  // key index within the row and the dense row it goes to
  const int j = a.with_prefix ? (int)(t - rm.cu_k) : rm.prefix + (int)(t - rm.cu_q);
  const int64_t dst_row = (int64_t)rm.cu_k + j;
  const int row = a.num_kv_heads * a.head_dim;
  const int nvec = row / 8;
  const uint16_t* src_k;
  const uint16_t* src_v;
  if (j < rm.prefix) {
    const int ps = a.page_size;
    const int64_t page = a.indices[rm.page_base + (j >> __builtin_ctz(ps))];
    src_k = a.cache + ((page * 2 + 0) * ps + (j & (ps - 1))) * (int64_t)row;
    src_v = src_k + (int64_t)ps * row;
  } else {
    const int64_t f = (int64_t)rm.cu_q + (j - rm.prefix);
    src_k = a.k_fresh + f * row;
    src_v = a.v_fresh + f * row;
  }
  uint4* dk = reinterpret_cast<uint4*>(a.k_out + dst_row * row);
  uint4* dv = reinterpret_cast<uint4*>(a.v_out + dst_row * row);
  for (int i = lane; i < 2 * nvec; i += 64) {
    if (i < nvec) dk[i] = reinterpret_cast<const uint4*>(src_k)[i];
    else dv[i - nvec] = reinterpret_cast<const uint4*>(src_v)[i - nvec];
  }
}

__global__ __launch_bounds__(256) void upload_kernel(UploadArgs a) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.n_vec; i += stride)
    a.dst[i] = a.src[i];
  // Every thread's loads have returned (their data is stored): the host may
  // rewrite this workgroup's share of the staging buffer.
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_store(a.flags + blockIdx.x, a.seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

}  // namespace

hipError_t launch_upload(const UploadArgs& a, hipStream_t stream, int* blocks) {
  *blocks = 0;
  if (a.n_vec <= 0) return hipSuccess;
  // Every vector in flight at once up to max_blocks workgroups; larger plans
  // loop.
  int64_t nb = (a.n_vec + 255) / 256;
  nb = nb > a.max_blocks ? a.max_blocks : nb;
  hipLaunchKernelGGL(upload_kernel, dim3((unsigned)nb), dim3(256), 0, stream, a);
  *blocks = (int)nb;
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t stream) {
  const int64_t n = a.with_prefix ? a.total_k : (int64_t)a.total_q;  // waves
  if (n <= 0 || a.n_rows <= 0) return hipSuccess;
  const int64_t blocks = (n + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  if (a.n_merges <= 0) return hipSuccess;
  const int64_t pairs = (int64_t)a.n_merges * a.group;
  const dim3 block(64 * kWaves);
  // Entries of up to 8 chunks: one wave per pair, four pairs per workgroup.
  // Longer ones: the four waves of a workgroup share a pair's chunks.
  const bool wide = a.max_chunks > 8;
  const dim3 grid(wide ? (unsigned)pairs : (unsigned)((pairs + kWaves - 1) / kWaves));
  if (a.head_dim == 128) {
    if (wide) hipLaunchKernelGGL((merge_kernel<128, kWaves>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((merge_kernel<128, 1>), grid, block, 0, stream, a);
  } else if (a.head_dim == 64) {
    if (wide) hipLaunchKernelGGL((merge_kernel<64, kWaves>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((merge_kernel<64, 1>), grid, block, 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
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
