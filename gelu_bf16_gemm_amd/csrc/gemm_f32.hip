// fp32 fused linear layer for gfx950: IEEE fp32 products and fp32 accumulation with
// v_mfma_f32_32x32x2_f32 ([Fusion] §Linear算子剖析 and its Python demo computed in fp32).
//
// A workgroup of 4 waves owns 128 features x 64 tokens; wave w takes features
// [32 w, 32 w + 32) and both 32-token blocks. K advances 32 at a time through one
// LDS buffer (rows padded to 33 floats so a column read is bank-conflict-free).
// The epilogue is the shared LDS-staged one (the whole 64 x 128 tile in one pass).
#include "epilogue.h"
#include "kernels.h"

namespace fusedops {

namespace {

constexpr int BF = 128;
constexpr int BT = 64;
constexpr int BK = 32;
constexpr int PAD = BK + 1;
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmArgs a) {
  // mainloop operands, then (after the loop) the staged 64 x 128 fp32 output tile
  __shared__ __attribute__((aligned(16))) float lds[BT * BF > (BF + BT) * PAD ? BT * BF : (BF + BT) * PAD];
  __shared__ float s_amax[BT];
  __shared__ int slot[2];
  float* wl = lds;
  float* xl = lds + BF * PAD;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;

  int tt, ft;
  if (a.ep.quant && a.ep.tickets) {
    const int ticket = draw_ticket(a.ep.ws, a.tiles_t * a.tiles_f, slot);
    tt = ticket / a.tiles_f;
    ft = ticket - tt * a.tiles_f;
    if (tt >= a.tiles_t) return;  // a workspace that was not zero-filled: touch nothing
  } else {
    tt = blockIdx.x / a.tiles_f;
    ft = blockIdx.x - tt * a.tiles_f;
  }
  const int f0 = ft * BF, t0 = tt * BT;
  const int K = a.K;
  const int w_rows = min(BF, a.N - f0), x_rows = min(BT, a.M - t0);
  const float* Wt = static_cast<const float*>(a.W) + (int64_t)f0 * a.ldw;
  const float* Xt = static_cast<const float*>(a.X) + (int64_t)t0 * a.ldx;
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(Wt, (uint32_t)(((int64_t)(w_rows - 1) * a.ldw + K) * 4));
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(Xt, (uint32_t)(((int64_t)(x_rows - 1) * a.ldx + K) * 4));

  f32x16 acc[1][2] = {{f32x16{}, f32x16{}}};
  const int steps = (K + BK - 1) / BK;
  for (int s = 0; s < steps; ++s) {
    const int k0 = s * BK;
    // W: 128 rows x 8 float4 chunks = 1024 chunks, 4 per thread; X: 512 chunks, 2 per thread
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int id = j * kThreads + tid, row = id >> 3, c = id & 7;
      const bool ok = k0 + c * 4 < K;
      u32x4 v = buffer_load_16B(rW, ok ? (uint32_t)((row * a.ldw + k0 + c * 4) * 4) : kOobOffset);
#pragma unroll
      for (int i = 0; i < 4; ++i) wl[row * PAD + c * 4 + i] = __uint_as_float(v[i]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int id = j * kThreads + tid, row = id >> 3, c = id & 7;
      const bool ok = k0 + c * 4 < K;
      u32x4 v = buffer_load_16B(rX, ok ? (uint32_t)((row * a.ldx + k0 + c * 4) * 4) : kOobOffset);
#pragma unroll
      for (int i = 0; i < 4; ++i) xl[row * PAD + c * 4 + i] = __uint_as_float(v[i]);
    }
    __syncthreads();
    const int ar = (wave * 32 + (lane & 31)) * PAD + (lane >> 5);
    const int br = (lane & 31) * PAD + (lane >> 5);
#pragma unroll
    for (int kk = 0; kk < BK / 2; ++kk) {
      const float av = wl[ar + kk * 2];
      const float b0 = xl[br + kk * 2];
      const float b1 = xl[br + 32 * PAD + kk * 2];
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, b1, acc[0][1], 0, 0, 0);
    }
    __syncthreads();
  }

  run_staged_epilogue<BF, 1, BT, 1>(a, lds, t0, f0, min(BT, a.M - t0), tt, ft, slot, s_amax,
                                    [&](int, float* tile) {
                                      stage_block<BF>(tile, acc[0][0], wave * 32, 0);
                                      stage_block<BF>(tile, acc[0][1], wave * 32, 32);
                                    });
}

}  // namespace

hipError_t launch_gemm_f32(GemmArgs a, hipStream_t stream) {
  a.tiles_t = (a.M + BT - 1) / BT;
  a.tiles_f = (a.N + BF - 1) / BF;
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_f32_kernel), dim3(a.tiles_t * a.tiles_f),
                         dim3(kThreads), args, 0, stream);
}

int gemm_f32_tile_t() { return BT; }
int gemm_f32_tile_f() { return BF; }
const void* gemm_f32_symbol() { return reinterpret_cast<const void*>(&gemm_f32_kernel); }

}  // namespace fusedops
