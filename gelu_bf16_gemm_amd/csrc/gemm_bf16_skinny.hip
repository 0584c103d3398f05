// bf16 fused linear layer for few tokens (decode): the contraction degenerates into a
// weight stream ([Epilogue] §边界五 and §端到端账本: with few tokens the weight read
// dominates), so the kernel is built to keep HBM busy rather than the matrix cores.
//
// A workgroup owns 64 features x 32 tokens and has 8 waves. W streams in stages of
// 64 rows x 256 K (32 KB): each load instruction reads 1 KB of memory as two 512-byte row
// segments, so HBM is read in linear runs rather than in the row-strided 16-byte pieces
// MFMA operands would need straight from memory. The stage's X slab (32 token rows x 256 K,
// 16 KB, read by every workgroup and served by L2) travels the same way, once per
// workgroup. Loads run DR stages ahead in a register ring, and each workgroup walks the
// stages in its own rotated order, so at any moment the workgroups read different offsets
// of their rows rather than all the same one (measured: deeper rings and longer stages were
// slower). One stage before it is needed a stage is written into one of two LDS buffers,
// where a row's 16-byte chunk c sits at position c ^ (row % 32) so that both the 64-lane
// writes and the 32-row MFMA operand reads are free of bank conflicts. Wave w multiplies
// feature half w % 2 over the 64-wide K quarter w / 2 of every stage, both operands read
// from LDS. The four K-quarter partial tiles of each feature half are staged in LDS and
// summed, in a fixed order, by the shared epilogue.
#include "epilogue.h"
#include "kernels.h"

namespace fusedops {

namespace {

constexpr int BF = 64;
constexpr int BT = 32;
constexpr int KS = 256;                      // K per stage
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowBytes = KS * 2;            // 512 bytes of a W row per stage
constexpr int kWBytes = BF * kRowBytes;      // 32 KB of W per stage
constexpr int kBufBytes = (BF + BT) * kRowBytes;  // 48 KB per stage buffer: W rows, then X rows
constexpr int DR = 2;                        // stages in flight in registers

// F: the epilogue configuration (epi::config) the instance is compiled for, or 0 for the generic
// instance, which reads every choice at run time.
template <uint32_t F>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_skinny_kernel(GemmArgs a) {
  // two stage buffers; afterwards they hold the 4 partial 32 x 64 fp32 tiles (32 KB) the
  // epilogue sums
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kBufBytes];
  __shared__ float s_amax[BT];
  __shared__ int slot[2];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int fb = wave & 1, kq = wave >> 1;
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
  // rows past N / M and chunks past K read as zero
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(Wt, (uint32_t)(((int64_t)(w_rows - 1) * a.ldw + K) * 2));
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(Xt, (uint32_t)(((int64_t)(x_rows - 1) * a.ldx + K) * 2));

  // W load i (0..3) of a stage: rows 8 wave + 2 i + h, chunk lane % 32 (8 K elements)
  const int lc = lane & 31;
  uint32_t w_voff[4], w_lds[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave * 8 + 2 * i + h;
    w_voff[i] = (uint32_t)(r * a.ldw * 2 + lc * 16);
    w_lds[i] = (uint32_t)(r * kRowBytes + ((lc ^ (r & 31)) << 4));
  }
  // X load i (0..1) of a stage: token rows 16 i + 2 wave + h, chunk lane % 32
  uint32_t x_voff[2], x_lds[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 16 * i + 2 * wave + h;
    x_voff[i] = (uint32_t)(r * a.ldx * 2 + lc * 16);
    x_lds[i] = (uint32_t)(kWBytes + r * kRowBytes + ((lc ^ (r & 31)) << 4));
  }
  // operands of MFMA step j (0..3) of the wave's K quarter: lane half h supplies K elements
  // [8h, 8h + 8) of the step, i.e. chunk kq * 8 + 2 j + h of W row wr and of token row xr
  const int wr = fb * 32 + (lane & 31), xr = lane & 31;
  uint32_t f_lds[4], g_lds[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f_lds[j] = (uint32_t)(wr * kRowBytes + (((kq * 8 + 2 * j + h) ^ (wr & 31)) << 4));
    g_lds[j] = (uint32_t)(kWBytes + xr * kRowBytes + (((kq * 8 + 2 * j + h) ^ xr) << 4));
  }

  const int stages = (K + KS - 1) / KS;
  u32x4 wreg[DR][4], xreg[DR][2];
  auto load = [&](int s, int d) __attribute__((always_inline)) {
    const uint32_t k0 = (uint32_t)(s < stages ? (s + ft) % stages : s) * KS;
    const uint32_t oob = (uint32_t)(k0 + lc * 8 >= (uint32_t)K) << 31;
#pragma unroll
    for (int i = 0; i < 4; ++i)  // each W byte is read once: nontemporal
      wreg[d][i] = __builtin_amdgcn_raw_buffer_load_b128(rW, (w_voff[i] + k0 * 2) | oob, 0, kNonTemporal);
#pragma unroll
    for (int i = 0; i < 2; ++i) xreg[d][i] = buffer_load_16B(rX, (x_voff[i] + k0 * 2) | oob);
  };
  auto put = [&](int buf, int d) __attribute__((always_inline)) {
    uint8_t* b = lds + buf * kBufBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(b + w_lds[i]) = wreg[d][i];
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4*>(b + x_lds[i]) = xreg[d][i];
  };
  f32x16 acc = {};
  auto compute = [&](int buf) __attribute__((always_inline)) {
    const uint8_t* b = lds + buf * kBufBytes;
    bf16x8 wf[4], xf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wf[j] = *reinterpret_cast<const bf16x8*>(b + f_lds[j]);
      xf[j] = *reinterpret_cast<const bf16x8*>(b + g_lds[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], xf[j], acc, 0, 0, 0);
  };

  // Step s handles the s-th stage of the rotated order. Stage s sits in register slot s % DR
  // and, once written, in LDS buffer s % 2. Step s: multiply stage s; write stage s + 1 to the
  // other buffer (free: everyone passed the barrier after multiplying stage s - 1); load stage
  // s + DR into slot s % DR (stage s left it when it was written to LDS a step earlier). A
  // stage past the last reads only zeros and adds nothing.
#pragma unroll
  for (int d = 0; d < DR; ++d) load(d, d);
  put(0, 0);
  __syncthreads();
  for (int s0 = 0; s0 < stages; s0 += DR) {
#pragma unroll
    for (int d = 0; d < DR; ++d) {
      const int s = s0 + d;
      compute(d & 1);
      put((d + 1) & 1, (d + 1) % DR);
      load(s + DR, d);
      __syncthreads();
    }
  }
  __syncthreads();

  run_staged_epilogue<BF, 4, BT, 1, F>(a, reinterpret_cast<float*>(lds), t0, f0, min(BT, a.M - t0), ft, slot,
                                    s_amax, [&](int, float* tile) {
                                      stage_block<BF>(tile + kq * BT * BF, acc, fb * 32, 0);
                                    });
}

// The decode layer's epilogue (SwiGLU, then FP8 rows) has an instance of its own; any other op
// list runs the generic one.
constexpr uint32_t kCfgSwigluFp8 = epi::config(epi::kQuant, ACT_SWIGLU, FUSEDOPS_F8E4M3);

const void* skinny_kernel_for(const EpiParams& e) {
  if (epi::config_of(e) == kCfgSwigluFp8)
    return reinterpret_cast<const void*>(&gemm_bf16_skinny_kernel<kCfgSwigluFp8>);
  return reinterpret_cast<const void*>(&gemm_bf16_skinny_kernel<0>);
}

}  // namespace

hipError_t launch_gemm_bf16_skinny(GemmArgs a, hipStream_t stream) {
  a.tiles_t = (a.M + BT - 1) / BT;
  a.tiles_f = (a.N + BF - 1) / BF;
  void* args[] = {&a};
  return hipLaunchKernel(skinny_kernel_for(a.ep), dim3(a.tiles_t * a.tiles_f), dim3(kThreads), args, 0, stream);
}

int gemm_bf16_skinny_tile_t() { return BT; }
int gemm_bf16_skinny_tile_f() { return BF; }
int gemm_bf16_skinny_threads() { return kThreads; }
const void* gemm_bf16_skinny_symbol(const EpiParams& e) { return skinny_kernel_for(e); }

}  // namespace fusedops
