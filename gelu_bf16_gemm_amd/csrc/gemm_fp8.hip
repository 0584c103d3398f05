// Fused linear layer with E4M3 inputs for gfx950: Y = epilogue(sa[m] sw[n] (Xq Wq^T) + b).
//
// The scale-after-accumulate form of a low-precision GEMM ([Epilogue] §量化尾声的完整形态,
// per-group scales with one group over K): the MFMAs multiply the stored E4M3 codes with
// fp32 accumulation, and the activation scale of the row and the weight scale of the
// output channel multiply the finished accumulator before the bias and the rest of the
// epilogue chain.
//
// Same workgroup shape as the bf16 kernel: 4 waves own a 256-feature x 256-token tile, each
// wave 128 x 128 as 4 x 4 blocks of v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, unit
// block scales). A K step is 128 codes, i.e. the same 128 bytes per row as a bf16 step of
// 64, so the LDS layout, its swizzle, the fills and the register stage set are those of the
// bf16 kernel. One MFMA consumes 64 K per row: lane half h supplies the 32 codes of chunks
// 4 kk + 2 h and 4 kk + 2 h + 1 of its row (two 16-byte operand reads); W and X fragments
// are read alike, so both operands list the same K positions in the same order.
//
// A step has four sub-steps of 8 MFMAs (K half kk = sub / 2, feature-block pair sub % 2).
// Fragment reads run one sub-step ahead: 4, 12, 4 and 12 reads; the fills and loads of the
// next steps are spread over sub-steps 0..2 and the step's barrier follows sub-step 2, after
// which sub-step 3 reads the next step's first fragments from the other buffer.
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
constexpr int BK = 128;   // K codes (bytes) per step
constexpr int kThreads = 256;
constexpr int kTileBytes = 256 * BK;  // one operand tile in LDS (32 KB)

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma_e4m3(const i32x8& a, const i32x8& b, const f32x16& c) {
  // formats 0 / 0: both operands E4M3; block scales 127 = 2^0 (E8M0), i.e. unscaled
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <uint32_t F>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_t256_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * 2 * kTileBytes];  // [stage][W, X]
  __shared__ __attribute__((aligned(16))) float svec[4 * 256];               // epilogue vectors
  __shared__ __attribute__((aligned(16))) float dqv[2 * 256];                // sw[f], sa[t]
  __shared__ int slot[2];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wf = wave >> 1, wt = wave & 1;

  int tt, ft;
  if (a.ep.quant && a.ep.tickets) {
    const int ticket = draw_ticket(a.ep.ws, a.tiles_t * a.tiles_f, slot);
    tt = ticket / a.tiles_f;
    ft = ticket - tt * a.tiles_f;
    if (tt >= a.tiles_t) return;  // a workspace that was not zero-filled: touch nothing
  } else {
    tile_coords(blockIdx.x, a.tiles_t, a.tiles_f, tt, ft);
  }
  const int f0 = ft * BF, t0 = tt * BT;
  const int K = a.K;

  accepi::VecPrefetch vp;
  if constexpr ((F & epi::kStatic) != 0) vp.load<F>(a.ep, t0, f0, a.M, a.N);
  // dequantisation scales of this tile's features and tokens (1 where absent or past N / M)
  const float sw = a.ep.dq_col && f0 + tid < a.N ? a.ep.dq_col[f0 + tid] : 1.f;
  const float sa = a.ep.dq_row && t0 + tid < a.M ? a.ep.dq_row[t0 + tid] : 1.f;

  // Buffer resources over this tile's rows: rows past M / N read as zero.
  const int w_rows = min(BF, a.N - f0), x_rows = min(BT, a.M - t0);
  const uint8_t* Wt = static_cast<const uint8_t*>(a.W) + (int64_t)f0 * a.ldw;
  const uint8_t* Xt = static_cast<const uint8_t*>(a.X) + (int64_t)t0 * a.ldx;
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(Wt, (uint32_t)((int64_t)(w_rows - 1) * a.ldw + K));
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(Xt, (uint32_t)((int64_t)(x_rows - 1) * a.ldx + K));

  // Global->LDS assignment as in the bf16 kernel: chunk id j*256 + tid is row j*32 + tid/8,
  // 16-byte chunk tid%8 of the step's 128 bytes.
  const int ld_row = tid >> 3, ld_c = tid & 7;
  const uint32_t w_voff = (uint32_t)(ld_row * a.ldw + ld_c * 16);
  const uint32_t x_voff = (uint32_t)(ld_row * a.ldx + ld_c * 16);
  const uint32_t w_rowstep = (uint32_t)(32 * a.ldw), x_rowstep = (uint32_t)(32 * a.ldx);
  const uint32_t st_off = lds_off(ld_row, ld_c);

  u32x4 stage[16];
  auto load_q = [&](int k0, int q) __attribute__((always_inline)) {
    const uint32_t oob = (uint32_t)(k0 + ld_c * 16 >= K) << 31;  // K is a multiple of 16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = q * 4 + i;
      const int j = c & 7;
      const uint32_t voff = ((c < 8 ? w_voff : x_voff) + (uint32_t)k0) | oob;
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

  // Operand read offsets: row (lane % 32) of each 32-row block; K half kk, piece p (0, 1) is
  // logical chunk 4 kk + 2 (lane / 32) + p.
  const int a_row0 = wf * 128 + (lane & 31);
  const int b_row0 = wt * 128 + (lane & 31);
  uint32_t koff[2][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int p = 0; p < 2; ++p) koff[kk][p] = (uint32_t)(((kk * 4 + (lane >> 5) * 2 + p) ^ swz(lane & 31)) << 4);

  auto frag = [&](const uint8_t* base, int row, int kk) __attribute__((always_inline)) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + row * 128 + koff[kk][0]);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + row * 128 + koff[kk][1]);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  // A fragments of one feature-block pair, B fragments of all four token blocks
  i32x8 fa[2][2], fb_[2][4];
  auto read_a = [&](int buf, int kk, int pair, i32x8 (&dst)[2]) __attribute__((always_inline)) {
    const uint8_t* wb = smem + buf * (2 * kTileBytes);
#pragma unroll
    for (int i = 0; i < 2; ++i) dst[i] = frag(wb, a_row0 + (pair * 2 + i) * 32, kk);
  };
  auto read_b = [&](int buf, int kk, i32x8 (&dst)[4]) __attribute__((always_inline)) {
    const uint8_t* xb = smem + buf * (2 * kTileBytes) + kTileBytes;
#pragma unroll
    for (int t = 0; t < 4; ++t) dst[t] = frag(xb, b_row0 + t * 32, kk);
  };

  auto kstep = [&](int s) __attribute__((always_inline)) {
    const int CUR = s & 1;
    auto sub = [&](auto j_c) __attribute__((always_inline)) {
      constexpr int j = decltype(j_c)::value;
      constexpr int kk = j >> 1, pair = j & 1;
      __builtin_amdgcn_sched_barrier(0);
      // operand reads for the next sub-step
      if constexpr (j == 0) {
        read_a(CUR, 0, 1, fa[1]);
      } else if constexpr (j == 1) {
        read_a(CUR, 1, 0, fa[0]);
        read_b(CUR, 1, fb_[1]);
      } else if constexpr (j == 2) {
        read_a(CUR, 1, 1, fa[1]);
      } else {
        read_a(CUR ^ 1, 0, 0, fa[0]);
        read_b(CUR ^ 1, 0, fb_[0]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[pair * 2 + i][t] = mfma_e4m3(fa[pair][i], fb_[kk][t], acc[pair * 2 + i][t]);
      // fills and loads: quarters 0 and 1 in sub-step 0, 2 in sub-step 1, 3 in sub-step 2
      if constexpr (j == 0) {
        store_q(CUR ^ 1, 0);
        store_q(CUR ^ 1, 1);
        load_q((s + 2) * BK, 0);
        load_q((s + 2) * BK, 1);
      } else if constexpr (j < 3) {
        store_q(CUR ^ 1, j + 1);
        load_q((s + 2) * BK, j + 1);
      }
      // issue pattern: each MFMA followed by its share of the operand reads (4 or 12), the
      // fills and the global loads (8, 4, 4, 0 of each)
      if constexpr (j == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
      } else if constexpr (j == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      } else if constexpr (j == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
    };
    sub(std::integral_constant<int, 0>{});
    sub(std::integral_constant<int, 1>{});
    sub(std::integral_constant<int, 2>{});
    __syncthreads();
    sub(std::integral_constant<int, 3>{});
  };

  const int steps = (K + BK - 1) / BK;
#pragma unroll
  for (int q = 0; q < 4; ++q) load_q(0, q);
#pragma unroll
  for (int q = 0; q < 4; ++q) store_q(0, q);
#pragma unroll
  for (int q = 0; q < 4; ++q) load_q(BK, q);
  if constexpr ((F & epi::kStatic) != 0) vp.store(svec, threadIdx.x);
  dqv[tid] = sw;
  dqv[256 + tid] = sa;
  __syncthreads();
  read_a(0, 0, 0, fa[0]);
  read_b(0, 0, fb_[0]);

#pragma clang loop unroll(disable)
  for (int s = 0; s < steps; ++s) kstep(s);
  __syncthreads();  // every wave's last fragment reads are done before LDS is reused

  // dequantise the accumulators: register r of block (fb, tb) is feature
  // wf*128 + fb*32 + 8 (r / 4) + 4 (lane / 32) + r % 4 and token wt*128 + tb*32 + lane % 32
  {
    const int hb = lane >> 5, tl = lane & 31;
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
      f32x16 w;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(dqv + wf * 128 + fb * 32 + q * 8 + hb * 4);
        w[4 * q] = x[0]; w[4 * q + 1] = x[1]; w[4 * q + 2] = x[2]; w[4 * q + 3] = x[3];
      }
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) acc[fb][tb] = acc[fb][tb] * dqv[256 + wt * 128 + tb * 32 + tl] * w;
    }
  }

  if constexpr ((F & epi::kStatic) != 0) {
    acc_epilogue<F>(a, acc, smem, svec, t0, f0, ft, slot, threadIdx.x);
  } else {
    __shared__ float s_amax[BT];
    run_staged_epilogue<BF, 1, 128, 2>(
        a, reinterpret_cast<float*>(smem), t0, f0, min(BT, a.M - t0), ft, slot, s_amax,
        [&](int p, float* tile) __attribute__((always_inline)) {
          if (wt != p) return;
#pragma unroll
          for (int fb = 0; fb < 4; ++fb)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) stage_block<BF>(tile, acc[fb][tb], wf * 128 + fb * 32, tb * 32);
        });
  }
}

// Epilogue configurations with an instance of their own (the MLP-up layer and the
// down-projection with its residual); any other op list runs the generic instance.
constexpr uint32_t kCfgBiasGeluErf = epi::config(epi::kBias, ACT_GELU_ERF, FUSEDOPS_BF16);
constexpr uint32_t kCfgResidual = epi::config(epi::kZ, ACT_NONE, FUSEDOPS_BF16);

const void* fp8_kernel_for(const EpiParams& e) {
  switch (epi::config_of(e)) {
    case kCfgBiasGeluErf: return reinterpret_cast<const void*>(&gemm_fp8_t256_kernel<kCfgBiasGeluErf>);
    case kCfgResidual: return reinterpret_cast<const void*>(&gemm_fp8_t256_kernel<kCfgResidual>);
    default: return reinterpret_cast<const void*>(&gemm_fp8_t256_kernel<0>);
  }
}

}  // namespace

hipError_t launch_gemm_fp8_t256(GemmArgs a, hipStream_t stream) {
  a.tiles_t = (a.M + BT - 1) / BT;
  a.tiles_f = (a.N + BF - 1) / BF;
  void* args[] = {&a};
  return hipLaunchKernel(fp8_kernel_for(a.ep), dim3(a.tiles_t * a.tiles_f), dim3(kThreads), args, 0, stream);
}

int gemm_fp8_t256_tile_f() { return BF; }
const void* gemm_fp8_t256_symbol(const EpiParams& e) { return fp8_kernel_for(e); }

}  // namespace fusedops
