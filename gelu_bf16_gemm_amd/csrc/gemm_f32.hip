// fp32 fused linear layer for gfx950: IEEE fp32 products and fp32 accumulation with
// v_mfma_f32_32x32x2_f32 ([Fusion] §Linear算子剖析 and its Python demo computed in fp32).
//
// Built for latency (the fp32 workload is a few MFLOP): a workgroup of 8 waves owns BF
// features x 32 tokens, so even a small problem spreads over several CUs, and K goes in
// chunks of KC: a chunk's W (BF rows) and X (32 rows) are loaded whole, all loads in flight,
// into LDS (the next chunk's loads are issued into registers while the current one is
// multiplied), and wave w multiplies its KC/8-wide K slice of the chunk for every 32-feature
// block. The eight K-slice partial tiles are summed, in a fixed order, by the shared
// LDS-staged epilogue. BF = 64 with KC = 256; op lists with RMSNorm row partials take BF = 128
// (KC = 128), so that a tile covers whole 128-column partial chunks. Rows are padded to
// KC + 33 floats (= 33 mod 64 banks) so the MFMA operand reads (32 rows at one k, the other
// lane half at k + 1) are free of bank conflicts.
#include "epilogue.h"
#include "kernels.h"

namespace fusedops {

namespace {

constexpr int BT = 32;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;

template <int BF>
__global__ __launch_bounds__(kThreads, 1) void gemm_f32_kernel(GemmArgs a) {
  constexpr int KC = BF == 64 ? 256 : 128;        // K per chunk
  constexpr int PAD = KC + 33;                     // row stride in floats
  constexpr int FB = BF / 32;                      // 32-feature blocks per wave
  constexpr int CPR = KC / 4;                      // 16-byte pieces per row of a chunk
  constexpr int kWChunks = BF * CPR / kThreads;    // pieces of W per thread and chunk
  constexpr int kXChunks = BT * CPR / kThreads;    // and of X
  constexpr int KS = KC / kWaves;                  // K slice of a wave per chunk
  // mainloop operands, then (after the loop) the eight staged 32 x 64 fp32 partial tiles
  __shared__ __attribute__((aligned(16))) float lds[(BF + BT) * PAD > kWaves * BT * BF ? (BF + BT) * PAD
                                                                                      : kWaves * BT * BF];
  __shared__ float s_amax[BT];
  __shared__ int slot[2];
  float* wl = lds;
  float* xl = lds + BF * PAD;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;

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
  // rows past N / M and K past K read as zero (buffer range / out-of-range offset)
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(Wt, (uint32_t)(((int64_t)(w_rows - 1) * a.ldw + K) * 4));
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(Xt, (uint32_t)(((int64_t)(x_rows - 1) * a.ldx + K) * 4));

  // piece id = j * kThreads + tid: row id / CPR, 16-byte column id % CPR of the chunk
  u32x4 wr[kWChunks], xr[kXChunks];
  auto load = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kWChunks; ++j) {
      const int id = j * kThreads + tid, row = id / CPR, c = id % CPR;
      wr[j] = buffer_load_16B(rW, k0 + c * 4 < K ? (uint32_t)((row * a.ldw + k0 + c * 4) * 4) : kOobOffset);
    }
#pragma unroll
    for (int j = 0; j < kXChunks; ++j) {
      const int id = j * kThreads + tid, row = id / CPR, c = id % CPR;
      xr[j] = buffer_load_16B(rX, k0 + c * 4 < K ? (uint32_t)((row * a.ldx + k0 + c * 4) * 4) : kOobOffset);
    }
  };
  auto store = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kWChunks; ++j) {
      const int id = j * kThreads + tid, row = id / CPR, c = id % CPR;
#pragma unroll
      for (int i = 0; i < 4; ++i) wl[row * PAD + c * 4 + i] = __uint_as_float(wr[j][i]);
    }
#pragma unroll
    for (int j = 0; j < kXChunks; ++j) {
      const int id = j * kThreads + tid, row = id / CPR, c = id % CPR;
#pragma unroll
      for (int i = 0; i < 4; ++i) xl[row * PAD + c * 4 + i] = __uint_as_float(xr[j][i]);
    }
  };

  f32x16 acc[FB];  // feature block b: features 32 b .. 32 b + 31 of the tile, all 32 tokens
#pragma unroll
  for (int b = 0; b < FB; ++b) acc[b] = f32x16{};
  const int chunks = (K + KC - 1) / KC;
  // operand rows of this lane: row lane % 32, k offset lane / 32 within each pair
  const int a0 = (lane & 31) * PAD + wave * KS + (lane >> 5);
  load(0);
#pragma clang loop unroll(disable)
  for (int ck = 0; ck < chunks; ++ck) {
    if (ck > 0) __syncthreads();  // every wave is done with the previous chunk
    store();
    __syncthreads();
    if (ck + 1 < chunks) load((ck + 1) * KC);
#pragma unroll
    for (int kk = 0; kk < KS / 2; ++kk) {
      const float x = xl[a0 + 2 * kk];
#pragma unroll
      for (int b = 0; b < FB; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(wl[a0 + 32 * b * PAD + 2 * kk], x, acc[b], 0, 0, 0);
    }
  }
  __syncthreads();  // LDS is reused for the partial tiles

  run_staged_epilogue<BF, kWaves, BT, 1>(a, lds, t0, f0, x_rows, ft, slot, s_amax, [&](int, float* tile) {
    float* part = tile + wave * BT * BF;
#pragma unroll
    for (int b = 0; b < FB; ++b) stage_block<BF>(part, acc[b], 32 * b, 0);
  });
}

// RMSNorm row partials cover 128-column chunks: those op lists take the 128-feature tile.
int f32_tile_f(const GemmArgs& a) { return a.ep.partials ? 128 : 64; }
const void* f32_kernel_for(const GemmArgs& a) {
  return a.ep.partials ? reinterpret_cast<const void*>(&gemm_f32_kernel<128>)
                       : reinterpret_cast<const void*>(&gemm_f32_kernel<64>);
}

}  // namespace

hipError_t launch_gemm_f32(GemmArgs a, hipStream_t stream) {
  a.tiles_t = (a.M + BT - 1) / BT;
  a.tiles_f = (a.N + f32_tile_f(a) - 1) / f32_tile_f(a);
  void* args[] = {&a};
  return hipLaunchKernel(f32_kernel_for(a), dim3(a.tiles_t * a.tiles_f), dim3(kThreads), args, 0, stream);
}

int gemm_f32_tile_t() { return BT; }
int gemm_f32_tile_f(const GemmArgs& a) { return f32_tile_f(a); }
int gemm_f32_threads() { return kThreads; }
const void* gemm_f32_symbol(const GemmArgs& a) { return f32_kernel_for(a); }

}  // namespace fusedops
