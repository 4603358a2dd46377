// Kernels compiled with the compiler's default instruction scheduling, in a
// translation unit of their own; the rest of the library uses the
// ILP-oriented strategy.  Measured on MI355X (alternating builds on one
// device), the default schedule is the better one for these:
//   - the single / down-projection LoRA linear forward (about 10 us of 820 at
//     8192 x 14336 -> 4096) and the QKV forward (about 7 us of 400);
//   - the split-K MLP dX variant: under the ILP strategy it kept values live
//     through its K-loops and reloaded them from scratch every K tile, each
//     reload's vmcnt wait serialising the tile's loads.
// The ILP strategy is the better one for the MLP dX GEMM (1780 vs 1844 us),
// the down-projection backward and the gate/up runs, which stay in the main
// unit.
#include "kernels_bwd.h"
#include "kernels_fwd.h"

namespace lora {

// Split-K MLP dX: the partial pass (tiles x S workgroups), then the merge
// pass (one workgroup per tile).
hipError_t launch_mlp_dx_split_bf16(const MlpDxArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((k_mlp_dx_bwd<bf16, true, true>), dim3(a.R * a.NC * a.sk.S), dim3(kGemmThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MlpDxArgs m = a;
  m.sk.pass = 1;
  hipLaunchKernelGGL((k_mlp_dx_bwd<bf16, true, true>), dim3(a.R * a.NC), dim3(kGemmThreads), 0, st, m);
  return hipGetLastError();
}

// The linear forward as runs of column tiles (a.L, a.RPB, a.nruns set).
hipError_t launch_linear_run_bf16(const LinearArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((k_linear_run<bf16>), dim3(a.nruns), dim3(kGemmThreads), 0, st, a);
  return hipGetLastError();
}

// The head_dim-128 QKV forward as runs of column tiles (a.L, a.RPB, a.nruns set).
hipError_t launch_qkv_run_bf16(const QKVFwdArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((k_qkv_run<bf16>), dim3(a.nruns), dim3(kGemmThreads), 0, st, a);
  return hipGetLastError();
}

template <class T>
hipError_t launch_linear_fwd(bool fast, const LinearArgs& a, dim3 grid, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    if (fast) {
      hipLaunchKernelGGL((k_linear_fwd<T, true>), grid, dim3(kGemmThreads), 0, st, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((k_linear_fwd<T, false>), grid, dim3(kGemmThreads), 0, st, a);
  return hipGetLastError();
}

template <class T, int LG, int NS>
static hipError_t launch_qkv_one(bool fast, const QKVFwdArgs& a, dim3 grid, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    if (fast) {
      hipLaunchKernelGGL((k_qkv_fwd<T, LG, true, NS>), grid, dim3(kGemmThreads), 0, st, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((k_qkv_fwd<T, LG, false, NS>), grid, dim3(kGemmThreads), 0, st, a);
  return hipGetLastError();
}

// head_dim 128 -> LG 1, 64 -> LG 2; ns = most projections one column tile overlaps.
template <class T>
hipError_t launch_qkv_fwd(bool fast, int head_dim, int ns, const QKVFwdArgs& a, dim3 grid, hipStream_t st) {
  if (head_dim == 128) {
    if (ns == 1) return launch_qkv_one<T, 1, 1>(fast, a, grid, st);
    if (ns == 2) return launch_qkv_one<T, 1, 2>(fast, a, grid, st);
    return launch_qkv_one<T, 1, 3>(fast, a, grid, st);
  }
  if (ns == 1) return launch_qkv_one<T, 2, 1>(fast, a, grid, st);
  if (ns == 2) return launch_qkv_one<T, 2, 2>(fast, a, grid, st);
  return launch_qkv_one<T, 2, 3>(fast, a, grid, st);
}

template hipError_t launch_linear_fwd<bf16>(bool, const LinearArgs&, dim3, hipStream_t);
template hipError_t launch_linear_fwd<float>(bool, const LinearArgs&, dim3, hipStream_t);
template hipError_t launch_qkv_fwd<bf16>(bool, int, int, const QKVFwdArgs&, dim3, hipStream_t);
template hipError_t launch_qkv_fwd<float>(bool, int, int, const QKVFwdArgs&, dim3, hipStream_t);

}  // namespace lora
