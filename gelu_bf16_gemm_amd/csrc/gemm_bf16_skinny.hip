// bf16 fused linear layer for few tokens (decode): the contraction degenerates into a
// weight stream ([Epilogue] §边界五 and §端到端账本: with few tokens the weight read
// dominates), so the kernel is built to keep HBM busy rather than the matrix cores.
//
// A workgroup owns 64 features x 32 tokens. Its 4 waves split the work as
// (feature block fb = w & 1) x (K half kh = w >> 1): each wave streams 32 W rows over
// every other 64-wide K block straight from HBM into MFMA operand registers (no LDS),
// so each lane reads 64 contiguous bytes of one row per block and a pair of lanes
// covers a full 128-byte line. Within a block, lane half h supplies K elements
// [32 h, 32 h + 32) of the block, 8 per MFMA step, for both operands alike, which is
// a fixed permutation of K and leaves the dot products unchanged.
// The two K halves are staged as two fp32 tiles in LDS and summed, in a fixed order, by
// the shared epilogue.
#include "epilogue.h"
#include "kernels.h"

namespace fusedops {

namespace {

constexpr int BF = 64;
constexpr int BT = 32;
constexpr int KB = 64;        // K block
constexpr int UNROLL = 4;     // K blocks in flight per wave
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void gemm_bf16_skinny_kernel(GemmArgs a) {
  // two staged 32 x 64 fp32 tiles, one per K half, summed by the epilogue
  __shared__ __attribute__((aligned(16))) float lds[2 * BT * BF];
  __shared__ float s_amax[BT];
  __shared__ int slot[2];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int fb = wave & 1, kh = wave >> 1;
  const int h = lane >> 5;

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
  const uint16_t* Wt = static_cast<const uint16_t*>(a.W) + (int64_t)f0 * a.ldw;
  const uint16_t* Xt = static_cast<const uint16_t*>(a.X) + (int64_t)t0 * a.ldx;
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(Wt, (uint32_t)(((int64_t)(w_rows - 1) * a.ldw + K) * 2));
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(Xt, (uint32_t)(((int64_t)(x_rows - 1) * a.ldx + K) * 2));

  const uint32_t w_row_off = (uint32_t)((fb * 32 + (lane & 31)) * a.ldw * 2);
  const uint32_t x_row_off = (uint32_t)((lane & 31) * a.ldx * 2);

  f32x16 acc = {};
  const int nkb = (K + KB - 1) / KB;
  for (int kb0 = kh; kb0 < nkb; kb0 += 2 * UNROLL) {
    u32x4 wv[UNROLL][4], xv[UNROLL][4];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int kb = kb0 + 2 * u;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int k = kb * KB + h * 32 + s * 8;
        const bool ok = kb < nkb && k < K;
        wv[u][s] = buffer_load_16B(rW, ok ? w_row_off + (uint32_t)k * 2 : kOobOffset);
        xv[u][s] = buffer_load_16B(rX, ok ? x_row_off + (uint32_t)k * 2 : kOobOffset);
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wv[u][s]),
                                                      __builtin_bit_cast(bf16x8, xv[u][s]), acc, 0, 0, 0);
  }

  run_staged_epilogue<BF, 2, BT, 1>(a, lds, t0, f0, min(BT, a.M - t0), tt, ft, slot, s_amax,
                                    [&](int, float* tile) {
                                      stage_block<BF>(tile + kh * BT * BF, acc, fb * 32, 0);
                                    });
}

}  // namespace

hipError_t launch_gemm_bf16_skinny(GemmArgs a, hipStream_t stream) {
  a.tiles_t = (a.M + BT - 1) / BT;
  a.tiles_f = (a.N + BF - 1) / BF;
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_bf16_skinny_kernel), dim3(a.tiles_t * a.tiles_f),
                         dim3(kThreads), args, 0, stream);
}

int gemm_bf16_skinny_tile_t() { return BT; }
int gemm_bf16_skinny_tile_f() { return BF; }
const void* gemm_bf16_skinny_symbol() { return reinterpret_cast<const void*>(&gemm_bf16_skinny_kernel); }

}  // namespace fusedops
