// Cross-entropy finalize: the separate final reduction after the XENT epilogue ([Epilogue]
// §模式C: every tile leaves (m, s) running statistics per row; an auxiliary pass merges them
// along the vocabulary with m = max(m1, m2), s = s1 e^(m1 - m) + s2 e^(m2 - m), and the loss is
// m + log s minus the logit at the label). No atomics: the merge order is fixed, so the result
// is reproducible.
//
// One wave per row: lane l folds chunks l, l + 64, ... in order, then a butterfly merges the
// 64 lane states; lane 0 writes the loss.
#include "common.h"
#include "kernels.h"

namespace fusedops {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 64;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ void merge(float& m, float& s, float mo, float so) {
  const float mn = fmaxf(m, mo);
  s = mn == -INFINITY ? 0.f : s * exp2f((m - mn) * kLog2e) + so * exp2f((mo - mn) * kLog2e);
  m = mn;
}

__global__ __launch_bounds__(kThreads) void xent_finalize_kernel(XentFinalizeArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + wave;
  if (row >= a.M) return;
  const float* st = a.stats + row * a.ld;
  float m = -INFINITY, s = 0.f;
  for (int t = lane; t < a.T; t += 64) merge(m, s, st[2 * t], st[2 * t + 1]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float mo = __shfl_xor(m, o, kWave), so = __shfl_xor(s, o, kWave);
    merge(m, s, mo, so);
  }
  if (lane == 0) {
    const int lab = a.labels[row];
    a.loss[row] = lab >= 0 && (int64_t)lab < a.n_cols ? m + logf(s) - a.target[row] : 0.f;
  }
}

}  // namespace

hipError_t launch_xent_finalize(const XentFinalizeArgs& a, hipStream_t stream) {
  const int64_t grid = (a.M + kRowsPerBlock - 1) / kRowsPerBlock;
  XentFinalizeArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(&xent_finalize_kernel), dim3((unsigned)grid),
                         dim3(kThreads), args, 0, stream);
}

}  // namespace fusedops
