// Causal ragged prefill launch (FlashInferPrefillWrapper.run on the mstar
// attn.wrappers page): one workgroup per tile; the device code and its design
// notes are in prefill_body.cuh.
#include "prefill_body.cuh"

namespace pkv {
namespace {

template <int D, bool WAVE_PAGE, bool DENSE>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillArgs a) {
  pre::prefill_tile<D, WAVE_PAGE, DENSE>(a, blockIdx.x);
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t stream) {
  const dim3 grid(a.n_tiles), block(256);
  if (a.k_dense != nullptr)
    hipLaunchKernelGGL((prefill_kernel<D, true, true>), grid, block, 0, stream, a);
  else if (a.page_size >= 16)
    hipLaunchKernelGGL((prefill_kernel<D, true, false>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<D, false, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.n_tiles <= 0) return hipSuccess;
  if (a.head_dim == 128) return launch_d<128>(a, stream);
  if (a.head_dim == 64) return launch_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
