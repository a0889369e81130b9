// Batched GQA decode launch (FlashInferDecodeWrapper.run on the mstar
// attn.wrappers page): one wave per (decode worker, KV head); the device code
// and its design notes are in decode_body.cuh.
#include "decode_body.cuh"

namespace pkv {
namespace {

using dec::kWaves;
using dec::decode_loads;

template <int D, int G, bool ONE_PAGE_PER_ITER>
__global__ __launch_bounds__(64 * kWaves) void decode_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  dec::decode_wave<D, G, ONE_PAGE_PER_ITER>(a, blockIdx.x * kWaves + wave, lane);
}

template <int D, int G>
hipError_t launch_dg(const DecodeArgs& a, hipStream_t stream) {
  constexpr int KB = (64 / (D / 8)) * decode_loads(G);
  const int64_t waves = (int64_t)a.n_workers * a.num_kv_heads;
  const dim3 grid((uint32_t)((waves + kWaves - 1) / kWaves)), block(64 * kWaves);
  if (a.page_size >= KB)
    hipLaunchKernelGGL((decode_kernel<D, G, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<D, G, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  switch (a.group) {
    case 1: return launch_dg<D, 1>(a, stream);
    case 2: return launch_dg<D, 2>(a, stream);
    case 4: return launch_dg<D, 4>(a, stream);
    case 8: return launch_dg<D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.n_workers <= 0) return hipSuccess;
  if (a.head_dim == 128) return launch_d<128>(a, stream);
  if (a.head_dim == 64) return launch_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
