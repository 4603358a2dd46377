// Kernels compiled with the compiler's default instruction scheduling, in a
// translation unit of their own; the rest of the library uses the
// ILP-oriented strategy.  Measured on MI355X, the default schedule is the
// better one for these two:
//   - the gate/up GEMM (about 1% faster);
//   - the split-K MLP dX variant: under the ILP strategy it kept values live
//     through its K-loops and reloaded them from scratch every K tile, each
//     reload's vmcnt wait serialising the tile's loads.
#include "kernels_bwd.h"
#include "kernels_fwd.h"

namespace lora {

hipError_t launch_mlp_dx_split_bf16(const MlpDxArgs& a, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((k_mlp_dx_bwd<bf16, true, true>), grid, dim3(kGemmThreads), 0, st, a);
  return hipGetLastError();
}

template <class T, int ACT>
hipError_t launch_gateup(bool fast, const GateUpArgs& a, dim3 grid, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    if (fast) {
      hipLaunchKernelGGL((k_gateup_run<ACT>), grid, dim3(kGemmThreads), 0, st, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((k_gateup_fwd<T, ACT, false>), grid, dim3(kGemmThreads), 0, st, a);
  return hipGetLastError();
}

template hipError_t launch_gateup<bf16, 0>(bool, const GateUpArgs&, dim3, hipStream_t);
template hipError_t launch_gateup<bf16, 1>(bool, const GateUpArgs&, dim3, hipStream_t);
template hipError_t launch_gateup<bf16, 2>(bool, const GateUpArgs&, dim3, hipStream_t);
template hipError_t launch_gateup<float, 0>(bool, const GateUpArgs&, dim3, hipStream_t);
template hipError_t launch_gateup<float, 1>(bool, const GateUpArgs&, dim3, hipStream_t);
template hipError_t launch_gateup<float, 2>(bool, const GateUpArgs&, dim3, hipStream_t);

}  // namespace lora
