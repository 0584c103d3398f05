// bf16 fused linear layer for gfx950: Y = epilogue(X W^T + b).
//
// Mainloop ([Fusion] §Linear算子剖析; [Epilogue] §主循环与尾声): one workgroup of
// 4 waves owns a 256-feature x 256-token output tile and walks K in steps of 64.
// Each step's W and X tiles (256 rows x 64 bf16, both K-contiguous in HBM) are
// staged in LDS, double buffered, with two register stage sets in front: during
// step s the MFMAs read LDS buffer s&1 while the data of step s+1 (already in
// registers) is written to the other buffer and the 16-byte global loads of step
// s+2 are issued; MFMAs, operand reads, fills and loads are interleaved so that
// the single wave per SIMD always has matrix work queued. One barrier per step.
//
// LDS layout: a 64-wide K tile row is 128 bytes = 8 chunks of 16 bytes, XOR-swizzled
// per row (see swz) so the ds_read_b128 operand fetches and the ds_write_b128
// fills are free of bank conflicts.
//
// Each wave computes 128 features x 128 tokens as 4 x 4 v_mfma_f32_32x32x16_bf16
// blocks (A = W rows, B = X rows, D[f][t]); the epilogue then stages the tile in LDS.
#include <type_traits>

#include "acc_epilogue.h"
#include "kernels.h"
#include "tile256.h"

namespace fusedops {

namespace {

using t256::lds_off;
using t256::swz;
using t256::tile_coords;

constexpr int BF = 256;   // features per tile
constexpr int BT = 256;   // tokens per tile
constexpr int BK = 64;    // K per step
constexpr int kThreads = 256;
constexpr int kTileBytes = 256 * BK * 2;  // one operand tile in LDS (32 KB)

template <uint32_t F>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_t256_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * 2 * kTileBytes];  // [stage][W, X]
  __shared__ __attribute__((aligned(16))) float svec[4 * 256];               // epilogue vectors
  __shared__ int slot[2];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wf = wave >> 1, wt = wave & 1;

  int tt, ft;
  if (a.ep.quant && a.ep.tickets) {
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

  // the epilogue's per-feature / per-token vectors, fetched now and kept in LDS
  accepi::VecPrefetch vp;
  if constexpr ((F & epi::kStatic) != 0) vp.load<F>(a.ep, t0, f0, a.M, a.N);

  // Buffer resources over this tile's rows: rows past M / N read as zero.
  const int w_rows = min(BF, a.N - f0), x_rows = min(BT, a.M - t0);
  const uint16_t* Wt = static_cast<const uint16_t*>(a.W) + (int64_t)f0 * a.ldw;
  const uint16_t* Xt = static_cast<const uint16_t*>(a.X) + (int64_t)t0 * a.ldx;
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(Wt, (uint32_t)(((int64_t)(w_rows - 1) * a.ldw + K) * 2));
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(Xt, (uint32_t)(((int64_t)(x_rows - 1) * a.ldx + K) * 2));

  // Global->LDS assignment: 8 chunks per thread per operand; chunk id j*256 + tid is
  // row j*32 + tid/8, 16-byte chunk tid%8 (8 threads read one 128-byte row segment).
  // The per-lane part of the address is a VGPR; the j*32-row part is a scalar offset.
  const int ld_row = tid >> 3, ld_c = tid & 7;
  const uint32_t w_voff = (uint32_t)(ld_row * a.ldw * 2 + ld_c * 16);
  const uint32_t x_voff = (uint32_t)(ld_row * a.ldx * 2 + ld_c * 16);
  const uint32_t w_rowstep = (uint32_t)(32 * a.ldw * 2), x_rowstep = (uint32_t)(32 * a.ldx * 2);
  // rows j*32 + ld_row share row & 15, so the fill offset of chunk j is st_off + j * 4096
  const uint32_t st_off = lds_off(ld_row, ld_c);

  // One register stage set: chunks 0..7 of W then 0..7 of X. During step s, quarter q of
  // the set (holding step s+1) is written to LDS buffer (s+1)&1, then the same registers
  // receive quarter q of step s+2 — a full step of latency for every load.
  u32x4 stage[16];

  // Chunks at or past K read as zero: the high offset bit makes the access out of range
  // (arithmetic rather than a select, so the loads stay branch-free).
  auto load_q = [&](int k0, int q) __attribute__((always_inline)) {
    const uint32_t oob = (uint32_t)(k0 + ld_c * 8 >= K) << 31;  // K is a multiple of 8
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = q * 4 + i;
      const int j = c & 7;
      const uint32_t voff = ((c < 8 ? w_voff : x_voff) + (uint32_t)k0 * 2) | oob;
      stage[c] = __builtin_amdgcn_raw_buffer_load_b128(c < 8 ? rW : rX, voff,
                                                       j * (c < 8 ? w_rowstep : x_rowstep), 0);
    }
  };
  auto store_q = [&](int buf, int q) __attribute__((always_inline)) {
    uint8_t* wb = smem + buf * (2 * kTileBytes) + st_off;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = q * 4 + i;
      *reinterpret_cast<u32x4*>(wb + (c < 8 ? 0 : kTileBytes) + (c & 7) * 4096) = stage[c];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // Per-lane operand read offsets: row (lane % 32) of each 32-row block, logical chunk
  // 2*kk + lane/32. Block bases are multiples of 32 rows, so the swizzle uses lane % 32.
  const int a_row0 = wf * 128 + (lane & 31);
  const int b_row0 = wt * 128 + (lane & 31);
  uint32_t koff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) koff[kk] = (uint32_t)((((kk * 2 + (lane >> 5)) ^ swz(lane & 31))) << 4);

  bf16x8 fa[2][4], fb_[2][4];
  auto read_frags = [&](int buf, int kk, bf16x8 (&af)[4], bf16x8 (&bf)[4]) __attribute__((always_inline)) {
    const uint8_t* wb = smem + buf * (2 * kTileBytes);
    const uint8_t* xb = wb + kTileBytes;
#pragma unroll
    for (int f = 0; f < 4; ++f) af[f] = *reinterpret_cast<const bf16x8*>(wb + (a_row0 + f * 32) * 128 + koff[kk]);
#pragma unroll
    for (int t = 0; t < 4; ++t) bf[t] = *reinterpret_cast<const bf16x8*>(xb + (b_row0 + t * 32) * 128 + koff[kk]);
  };

  // One K step s from LDS buffer s&1: the MFMAs of the step, the fill of buffer (s+1)&1
  // from the stage set (data of step s+1), and the loads of step s+2 into the stage set.
  // The fills and loads are done in sub-steps 0..2 and the step's one barrier comes after
  // sub-step 2: by then every wave has read its last fragments of buffer s&1 and written its
  // part of buffer (s+1)&1. Sub-step 3's MFMAs then run while the first fragments of step
  // s+1 are read, so no fragment read waits behind the barrier. The fragments of sub-step 0
  // arrive from the previous step (or the prologue). The last two steps fill and load past
  // the end of K: those loads read zeros into a buffer that is not read again.
  auto kstep = [&](int s) __attribute__((always_inline)) {
    const int CUR = s & 1;
    // sub-step kk is a compile-time constant so every register array index is static
    auto sub = [&](auto kk_c) __attribute__((always_inline)) {
      constexpr int kk = decltype(kk_c)::value;
      // keep each sub-step's work together: at most one sub-step of fragments in flight
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kk < 3) read_frags(CUR, kk + 1, fa[(kk + 1) & 1], fb_[(kk + 1) & 1]);
      else read_frags(CUR ^ 1, 0, fa[0], fb_[0]);
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[f][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk & 1][f], fb_[kk & 1][t], acc[f][t], 0, 0, 0);
      // fills and loads: quarters 0 and 1 in sub-step 0, 2 in sub-step 1, 3 in sub-step 2
      if constexpr (kk == 0) {
        store_q(CUR ^ 1, 0);
        store_q(CUR ^ 1, 1);
        load_q((s + 2) * BK, 0);
        load_q((s + 2) * BK, 1);
      } else if constexpr (kk < 3) {
        store_q(CUR ^ 1, kk + 1);
        load_q((s + 2) * BK, kk + 1);
      }
      // issue pattern per sub-step: MFMA / DS-read pairs, then MFMAs interleaved with the
      // fills and the global loads
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if constexpr (kk == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
      } else if constexpr (kk < 3) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      }
    };
    sub(std::integral_constant<int, 0>{});
    sub(std::integral_constant<int, 1>{});
    sub(std::integral_constant<int, 2>{});
    __syncthreads();
    sub(std::integral_constant<int, 3>{});
  };

  const int steps = (K + BK - 1) / BK;
  // prologue: step 0 into LDS buffer 0, step 1 into the stage set, step 0's first fragments
#pragma unroll
  for (int q = 0; q < 4; ++q) load_q(0, q);
#pragma unroll
  for (int q = 0; q < 4; ++q) store_q(0, q);
#pragma unroll
  for (int q = 0; q < 4; ++q) load_q(BK, q);
  if constexpr ((F & epi::kStatic) != 0) vp.store(svec);
  __syncthreads();
  read_frags(0, 0, fa[0], fb_[0]);

#pragma clang loop unroll(disable)
  for (int s = 0; s < steps; ++s) kstep(s);
  __syncthreads();  // every wave's last fragment reads are done before LDS is reused

  if constexpr ((F & epi::kStatic) != 0) {
    // Epilogue on the accumulators in place; the mainloop's LDS buffers (128 KB) stage
    // the finished values for coalesced stores.
    acc_epilogue<F>(a, acc, smem, svec, t0, f0, tt, ft, slot);
  } else {
    // Any other op list: the fp32 tile is staged through LDS in two 128-token passes
    // (128 KB each; pass p takes the accumulators of the waves with wt == p) and the
    // row-layout chain reads every choice at run time.
    __shared__ float s_amax[BT];
    run_staged_epilogue<BF, 1, 128, 2>(
        a, reinterpret_cast<float*>(smem), t0, f0, min(BT, a.M - t0), tt, ft, slot, s_amax,
        [&](int p, float* tile) __attribute__((always_inline)) {
          if (wt != p) return;
#pragma unroll
          for (int fb = 0; fb < 4; ++fb)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) stage_block<BF>(tile, acc[fb][tb], wf * 128 + fb * 32, tb * 32);
        });
  }
}

// Epilogue configurations with an instance of their own (the op sets of the fused QKV
// projection, MLP-up, out-projection, gate/up, FP8 gate/up, gate/up after a deferred RMSNorm,
// and the LM head with cross-entropy statistics); any other op list runs the generic instance,
// which reads its choices at run time.
constexpr uint32_t kCfgBiasGeluErf = epi::config(epi::kBias, ACT_GELU_ERF, FUSEDOPS_BF16);
constexpr uint32_t kCfgBiasSplit = epi::config(epi::kBias | epi::kSplit, ACT_NONE, FUSEDOPS_BF16);
constexpr uint32_t kCfgResidualRms = epi::config(epi::kZ | epi::kAux | epi::kPart | epi::kGamma, ACT_NONE,
                                                 FUSEDOPS_BF16);
constexpr uint32_t kCfgSwiglu = epi::config(0, ACT_SWIGLU, FUSEDOPS_BF16);
constexpr uint32_t kCfgSwigluFp8 = epi::config(epi::kQuant, ACT_SWIGLU, FUSEDOPS_F8E4M3);
constexpr uint32_t kCfgRscaleSwiglu = epi::config(epi::kRscale, ACT_SWIGLU, FUSEDOPS_BF16);
constexpr uint32_t kCfgXent = epi::config(epi::kXent, ACT_NONE, FUSEDOPS_BF16);

const void* t256_kernel_for(const EpiParams& e) {
  switch (epi::config_of(e)) {
    case kCfgBiasGeluErf: return reinterpret_cast<const void*>(&gemm_bf16_t256_kernel<kCfgBiasGeluErf>);
    case kCfgBiasSplit: return reinterpret_cast<const void*>(&gemm_bf16_t256_kernel<kCfgBiasSplit>);
    case kCfgResidualRms: return reinterpret_cast<const void*>(&gemm_bf16_t256_kernel<kCfgResidualRms>);
    case kCfgSwiglu: return reinterpret_cast<const void*>(&gemm_bf16_t256_kernel<kCfgSwiglu>);
    case kCfgSwigluFp8: return reinterpret_cast<const void*>(&gemm_bf16_t256_kernel<kCfgSwigluFp8>);
    case kCfgRscaleSwiglu: return reinterpret_cast<const void*>(&gemm_bf16_t256_kernel<kCfgRscaleSwiglu>);
    case kCfgXent: return reinterpret_cast<const void*>(&gemm_bf16_t256_kernel<kCfgXent>);
    default: return reinterpret_cast<const void*>(&gemm_bf16_t256_kernel<0>);
  }
}

}  // namespace

hipError_t launch_gemm_bf16_t256(GemmArgs a, hipStream_t stream) {
  a.tiles_t = (a.M + BT - 1) / BT;
  a.tiles_f = (a.N + BF - 1) / BF;
  const int grid = a.tiles_t * a.tiles_f;
  void* args[] = {&a};
  return hipLaunchKernel(t256_kernel_for(a.ep), dim3(grid), dim3(kThreads), args, 0, stream);
}

int gemm_bf16_t256_tile_t() { return BT; }
int gemm_bf16_t256_tile_f() { return BF; }

const void* gemm_bf16_t256_symbol(const EpiParams& e) { return t256_kernel_for(e); }

}  // namespace fusedops
