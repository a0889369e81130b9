// The mixed step in one launch (FlashInferMixedWrapper on the mstar
// attn.wrappers page: one-token rows on the decode plan, prompt rows on the
// prefill plan, both in one step).  The first workgroups run the decode waves,
// the rest the prefill tiles, so a CU holds a decode workgroup streaming K/V
// from HBM next to a prefill workgroup keeping its matrix cores busy: the
// prefill time hides under the decode's memory stream instead of following it.
// The device code is that of the two separate launches (decode_body.cuh,
// prefill_body.cuh); the merge of split decode rows still follows as its own
// launch.
#include "decode_body.cuh"
#include "prefill_body.cuh"

namespace pkv {
namespace {

template <int D, int G, bool ONE_PAGE_PER_ITER>
__global__ __launch_bounds__(256, 2) void mixed_kernel(DecodeArgs da, PrefillArgs pa,
                                                        int dec_blocks) {
  if ((int)blockIdx.x < dec_blocks) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    dec::decode_wave<D, G, ONE_PAGE_PER_ITER>(da, blockIdx.x * dec::kWaves + wave, lane);
    return;
  }
  pre::prefill_tile<D, true, false, false>(pa, (int)blockIdx.x - dec_blocks);
}

template <int D, int G>
hipError_t launch_mg(const DecodeArgs& da, const PrefillArgs& pa, hipStream_t stream) {
  constexpr int KB = (64 / (D / 8)) * dec::decode_loads(G);
  const int64_t waves = (int64_t)da.n_workers * da.num_kv_heads;
  const int dec_blocks = (int)((waves + dec::kWaves - 1) / dec::kWaves);
  const dim3 grid((uint32_t)(dec_blocks + pa.n_tiles)), block(256);
  if (da.page_size >= KB)
    hipLaunchKernelGGL((mixed_kernel<D, G, true>), grid, block, 0, stream, da, pa, dec_blocks);
  else
    hipLaunchKernelGGL((mixed_kernel<D, G, false>), grid, block, 0, stream, da, pa, dec_blocks);
  return hipGetLastError();
}

template <int D>
hipError_t launch_md(const DecodeArgs& da, const PrefillArgs& pa, hipStream_t stream) {
  switch (da.group) {
    case 1: return launch_mg<D, 1>(da, pa, stream);
    case 2: return launch_mg<D, 2>(da, pa, stream);
    case 4: return launch_mg<D, 4>(da, pa, stream);
    case 8: return launch_mg<D, 8>(da, pa, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool mixed_launch_fits(const DecodeArgs& da, const PrefillArgs& pa) {
  return pa.page_size >= 16 && pa.k_dense == nullptr && da.head_dim == pa.head_dim &&
         (da.head_dim == 64 || da.head_dim == 128) &&
         (da.group == 1 || da.group == 2 || da.group == 4 || da.group == 8);
}

hipError_t launch_mixed(const DecodeArgs& da, const PrefillArgs& pa, hipStream_t stream) {
  if (!mixed_launch_fits(da, pa)) return hipErrorInvalidValue;
  if (da.n_workers <= 0 && pa.n_tiles <= 0) return hipSuccess;
  if (da.head_dim == 128) return launch_md<128>(da, pa, stream);
  return launch_md<64>(da, pa, stream);
}

}  // namespace pkv
