// bf16 fused linear layer for gfx950: Y = epilogue(X W^T + b).
//
// Mainloop ([Fusion] §Linear算子剖析; [Epilogue] §主循环与尾声): one workgroup of
// 4 waves owns a 256-feature x 256-token output tile and walks K in steps of 64.
// Each step's W and X tiles (256 rows x 64 bf16, both K-contiguous in HBM) are
// staged in LDS, double buffered: the next step's 16-byte global loads are in
// flight in registers while the MFMAs of the current step run, and are written
// to the other LDS buffer afterwards, so each step needs one barrier.
//
// LDS layout: a 64-wide K tile row is 128 bytes = 8 chunks of 16 bytes; chunk c
// of row r is stored at chunk position c ^ (r & 7). Eight consecutive rows read
// at the same logical chunk then hit 8 different 16-byte bank groups, so the
// ds_read_b128 operand fetches and the ds_write_b128 fills are conflict-free.
//
// Each wave computes 128 features x 128 tokens as 4 x 4 v_mfma_f32_32x32x16_bf16
// blocks (A = W rows, B = X rows, D[f][t]); the epilogue then stages the tile in LDS.
#include "epilogue.h"
#include "kernels.h"

namespace fusedops {

namespace {

constexpr int BF = 256;   // features per tile
constexpr int BT = 256;   // tokens per tile
constexpr int BK = 64;    // K per step
constexpr int kThreads = 256;
constexpr int kTileBytes = 256 * BK * 2;  // one operand tile in LDS (32 KB)

__device__ __forceinline__ uint32_t lds_off(int row, int chunk) {
  return (uint32_t)(row * 128 + ((chunk ^ (row & 7)) << 4));
}

// Map a linear tile id to (token tile, feature tile). Consecutive workgroups are
// dealt round-robin to the 8 XCDs; regroup so that each XCD walks a contiguous
// range of tile ids, and within that range cover GROUP_T token tiles x all
// feature tiles so concurrently running tiles share operand rows in the XCD's L2.
__device__ __forceinline__ void tile_coords(int pid, int tiles_t, int tiles_f, int& tt, int& ft) {
  const int G = tiles_t * tiles_f;
  const int xcd = pid & 7, local = pid >> 3;
  const int base = G >> 3, rem = G & 7;
  const int p2 = xcd * base + min(xcd, rem) + local;
  constexpr int GROUP_T = 4;
  const int group_size = GROUP_T * tiles_f;
  const int g = p2 / group_size;
  const int first_t = g * GROUP_T;
  const int gt = min(tiles_t - first_t, GROUP_T);
  const int in = p2 - g * group_size;
  tt = first_t + in % gt;
  ft = in / gt;
}

__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_t256_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * 2 * kTileBytes];  // [stage][W, X]
  __shared__ int slot[2];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wf = wave >> 1, wt = wave & 1;

  int tt, ft;
  if (a.ep.quant) {
    // FP8 row scales need every feature tile of a token block: hand out tiles in
    // row-block-major ticket order so no block waits on a tile that is not running.
    const int ticket = draw_ticket(a.ep.ws, a.tiles_t * a.tiles_f, slot);
    tt = ticket / a.tiles_f;
    ft = ticket - tt * a.tiles_f;
    if (tt >= a.tiles_t) return;  // a workspace that was not zero-filled: touch nothing
  } else {
    tile_coords(blockIdx.x, a.tiles_t, a.tiles_f, tt, ft);
  }
  const int f0 = ft * BF, t0 = tt * BT;
  const int K = a.K;

  // Buffer resources over this tile's rows: rows past M / N read as zero.
  const int w_rows = min(BF, a.N - f0), x_rows = min(BT, a.M - t0);
  const uint16_t* Wt = static_cast<const uint16_t*>(a.W) + (int64_t)f0 * a.ldw;
  const uint16_t* Xt = static_cast<const uint16_t*>(a.X) + (int64_t)t0 * a.ldx;
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(Wt, (uint32_t)(((int64_t)(w_rows - 1) * a.ldw + K) * 2));
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(Xt, (uint32_t)(((int64_t)(x_rows - 1) * a.ldx + K) * 2));

  // Global->LDS assignment: 8 chunks per thread per operand; chunk id j*256 + tid is
  // row j*32 + tid/8, 16-byte chunk tid%8 (8 threads read one 128-byte row segment).
  const int ld_row = tid >> 3, ld_c = tid & 7;
  uint32_t w_voff[8], x_voff[8], st_off[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = j * 32 + ld_row;
    w_voff[j] = (uint32_t)(row * a.ldw * 2 + ld_c * 16);
    x_voff[j] = (uint32_t)(row * a.ldx * 2 + ld_c * 16);
    st_off[j] = lds_off(row, ld_c);
  }

  u32x4 wreg[8], xreg[8];
  auto load_step = [&](int k0) {
    const bool k_ok = k0 + ld_c * 8 < K;  // K is a multiple of 8: a chunk is all-in or all-out
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      wreg[j] = buffer_load_16B(rW, k_ok ? w_voff[j] + k0 * 2 : kOobOffset);
      xreg[j] = buffer_load_16B(rX, k_ok ? x_voff[j] + k0 * 2 : kOobOffset);
    }
  };
  auto store_step = [&](int stage) {
    uint8_t* wb = smem + stage * 2 * kTileBytes;
    uint8_t* xb = wb + kTileBytes;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      *reinterpret_cast<u32x4*>(wb + st_off[j]) = wreg[j];
      *reinterpret_cast<u32x4*>(xb + st_off[j]) = xreg[j];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // Per-lane operand read offsets: row (lane % 32) of each 32-row block, logical chunk
  // 2*kk + lane/32. Block bases are multiples of 8 rows, so the swizzle uses lane % 8.
  const int a_row0 = wf * 128 + (lane & 31);
  const int b_row0 = wt * 128 + (lane & 31);
  uint32_t koff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) koff[kk] = (uint32_t)((((kk * 2 + (lane >> 5)) ^ (lane & 7))) << 4);

  const int steps = (K + BK - 1) / BK;
  load_step(0);
  store_step(0);
  __syncthreads();

  for (int s = 0; s < steps; ++s) {
    if (s + 1 < steps) load_step((s + 1) * BK);
    const uint8_t* wb = smem + (s & 1) * 2 * kTileBytes;
    const uint8_t* xb = wb + kTileBytes;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int fb = 0; fb < 4; ++fb)
        af[fb] = *reinterpret_cast<const bf16x8*>(wb + (a_row0 + fb * 32) * 128 + koff[kk]);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        bfr[tb] = *reinterpret_cast<const bf16x8*>(xb + (b_row0 + tb * 32) * 128 + koff[kk]);
#pragma unroll
      for (int fb = 0; fb < 4; ++fb)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
          acc[fb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fb], bfr[tb], acc[fb][tb], 0, 0, 0);
    }
    if (s + 1 < steps) store_step((s + 1) & 1);
    __syncthreads();
  }

  // Epilogue: the 256 x 256 fp32 tile is staged through LDS in two 128-token passes
  // (128 KB each); pass p takes the accumulators of the waves with wt == p.
  run_staged_epilogue<BF, 1, 128, 2>(
      a, reinterpret_cast<float*>(smem), t0, f0, min(BT, a.M - t0), tt, slot,
      [&](int p, float* tile) {
        if (wt != p) return;
#pragma unroll
        for (int fb = 0; fb < 4; ++fb)
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) stage_block<BF>(tile, acc[fb][tb], wf * 128 + fb * 32, tb * 32);
      });
}

}  // namespace

hipError_t launch_gemm_bf16_t256(GemmArgs a, hipStream_t stream) {
  a.tiles_t = (a.M + BT - 1) / BT;
  a.tiles_f = (a.N + BF - 1) / BF;
  const int grid = a.tiles_t * a.tiles_f;
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_bf16_t256_kernel), dim3(grid), dim3(kThreads),
                         args, 0, stream);
}

int gemm_bf16_t256_tile_t() { return BT; }
int gemm_bf16_t256_tile_f() { return BF; }

const void* gemm_bf16_t256_symbol() { return reinterpret_cast<const void*>(&gemm_bf16_t256_kernel); }

}  // namespace fusedops
