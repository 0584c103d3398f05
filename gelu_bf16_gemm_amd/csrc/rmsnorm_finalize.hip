// RMSNorm finalize: the small aux reduction after an epilogue that wrote per-tile
// row sum-of-squares partials ([Epilogue] §模式A: sum the partials by row, take the
// root and the reciprocal). It reads M x T floats instead of the M x N activation.
//
// One wave per row: lanes stride over the row's T partials, a wavefront reduction
// sums them, and lane 0 writes r = 1 / sqrt(sum / N + eps). With `h` / `y` given, the
// same wave then streams the row once more in 16-byte chunks and writes
// y = r * h (* gamma).
#include "common.h"
#include "kernels.h"

namespace fusedops {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 64;

__global__ __launch_bounds__(kThreads) void rmsnorm_finalize_kernel(FinalizeArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + wave;
  if (row >= a.M) return;
  const float* p = a.partials + row * a.ldp;
  float s = 0.f;
  for (int t = lane; t < a.T; t += 64) s += p[t];
  s = wave_sum(s);
  const float r = 1.0f / sqrtf(s / (float)a.N + a.eps);
  if (lane == 0) a.r[row] = r;
  if (!a.h) return;

  const int es = a.dtype == FUSEDOPS_F32 ? 4 : 2;
  const int epc = 16 / es;  // elements per 16-byte chunk
  const int nchunks = (int)(a.N / epc);
  const char* hrow = static_cast<const char*>(a.h) + row * a.ldh * es;
  char* yrow = static_cast<char*>(a.y) + row * a.ldy * es;
  for (int c = lane; c < nchunks; c += 64) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (es == 4 && half == 1) break;
      // 4 elements per step (8 bytes of a 2-byte type, 16 bytes of fp32)
      const int64_t idx = (int64_t)c * epc + half * 4;
      f32x4 v = load4(hrow, a.dtype, idx);
      if (a.gamma) {
        const f32x4 g = load4(a.gamma, a.dtype, idx);
        v = v * g;
      }
      v = v * r;
      store4(yrow, a.dtype, idx, v);
    }
  }
}

}  // namespace

hipError_t launch_rmsnorm_finalize(const FinalizeArgs& a, hipStream_t stream) {
  const int64_t grid = (a.M + kRowsPerBlock - 1) / kRowsPerBlock;
  FinalizeArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(&rmsnorm_finalize_kernel), dim3((unsigned)grid),
                         dim3(kThreads), args, 0, stream);
}

}  // namespace fusedops
