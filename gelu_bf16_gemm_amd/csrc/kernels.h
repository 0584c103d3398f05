// Host-side launchers of the fusedops kernels (internal; the public surface is fusedops.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fusedops {

struct GemmArgs;
struct EpiParams;

// bf16 GEMM + epilogue, 256 x 256 tiles (tokens x features), 4 waves. The kernel instance
// depends on the epilogue configuration and on the shape (whole W tiles and an even number
// of K steps take the LDS-DMA mainloop); the symbol is the one a call with `a` launches.
hipError_t launch_gemm_bf16_t256(GemmArgs a, hipStream_t stream);
int gemm_bf16_t256_tile_t();
int gemm_bf16_t256_tile_f();
const void* gemm_bf16_t256_symbol(const GemmArgs& a);

// E4M3 inputs, 256 x 256 tiles (any M): v_mfma_scale_f32_32x32x64_f8f6f4 mainloop, the
// dequantisation scales applied to the accumulators, then the same epilogues as above
hipError_t launch_gemm_fp8_t256(GemmArgs a, hipStream_t stream);
int gemm_fp8_t256_tile_f();
const void* gemm_fp8_t256_symbol(const EpiParams& e);

// bf16 GEMM + epilogue for few tokens (decode): 32-token x 64-feature tiles, K split
// over the 8 waves of a workgroup.
hipError_t launch_gemm_bf16_skinny(GemmArgs a, hipStream_t stream);
int gemm_bf16_skinny_tile_t();
int gemm_bf16_skinny_tile_f();
int gemm_bf16_skinny_threads();
const void* gemm_bf16_skinny_symbol(const EpiParams& e);

// fp32 GEMM + epilogue (v_mfma_f32_32x32x2_f32), 32-token x 64-feature tiles (128 features
// when the op list writes RMSNorm row partials), K split over the 8 waves of a workgroup.
hipError_t launch_gemm_f32(GemmArgs a, hipStream_t stream);
int gemm_f32_tile_t();
int gemm_f32_tile_f(const GemmArgs& a);
int gemm_f32_threads();
const void* gemm_f32_symbol(const GemmArgs& a);

// The device array behind fusedops_linear_epilogue_noalloc (FUSEDOPS_NOALLOC_SCRATCH_BYTES on
// each GPU): its address on the current device, looked up once per device.
hipError_t noalloc_scratch(void** ptr);
// Zero the ticket counter and the control lines of `records` rendezvous records (ctl_words
// words at the start of each record_words-word record) of a workspace, on `stream`.
hipError_t launch_clear_rendezvous(void* ws, int64_t records, int ctl_words, int64_t record_words,
                                   hipStream_t stream);

struct LnArgs {
  const void* x; int64_t ldx;
  void* y; int64_t ldy;
  int64_t rows; int cols;
  int io_dtype, out_dtype;
  const void* gamma; const void* beta; int param_dtype;
  float eps;
  int gelu_form;
};
hipError_t launch_layernorm_gelu(const LnArgs& a, hipStream_t stream);

struct FinalizeArgs {
  const float* partials; int64_t ldp;
  int64_t M; int T; int64_t N;
  float eps;
  float* r;
  const void* h; int64_t ldh;
  const void* gamma;
  void* y; int64_t ldy;
  int dtype;
};
hipError_t launch_rmsnorm_finalize(const FinalizeArgs& a, hipStream_t stream);

struct XentFinalizeArgs {
  const float* stats;     // M x 2T (max, sum-exp) pairs, row stride ld
  int64_t ld, M, T, n_cols;
  const float* target;    // y at the label, per row
  const int* labels;
  float* loss;
};
hipError_t launch_xent_finalize(const XentFinalizeArgs& a, hipStream_t stream);

}  // namespace fusedops
