// LayerNorm + GELU row kernel ([LN+GELU] §用Triton手写融合内核): one pass over each
// row, fp32 statistics, GELU applied in registers, one store.
//
// A row is read with 16-byte loads: chunk j of lane l is the 16 bytes at chunk index
// j * (64 * WPR) + l, so every load instruction of a wave covers 1 KB of contiguous
// memory. All of a lane's chunks are loaded before any arithmetic, the row sits in
// registers as fp32, and the statistics take two wavefront reductions (mean, then
// the sum of squared deviations from it, matching the two-pass definition). Rows of
// up to 64 * CH * EPC elements use one wave (WPR = 1); longer rows use a whole
// workgroup (WPR = 4) with an LDS merge of the four waves' sums. Chunks past the row
// end are masked out of both sums.
#include "common.h"
#include "kernels.h"

namespace fusedops {

namespace {

constexpr int kThreads = 256;

// Load EPC consecutive elements (16 bytes of x, or params of any dtype) as fp32.
template <int EPC>
__device__ __forceinline__ void load_chunk(const void* base, int dtype, int64_t idx, float (&o)[EPC]) {
  if (dtype == FUSEDOPS_F32) {
#pragma unroll
    for (int i = 0; i < EPC; i += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx + i);
      o[i] = v[0]; o[i + 1] = v[1]; o[i + 2] = v[2]; o[i + 3] = v[3];
    }
    return;
  }
  // 2-byte types: EPC / 2 packed words (8 or 16 bytes)
  uint32_t w[EPC / 2];
  if constexpr (EPC >= 8) {
#pragma unroll
    for (int i = 0; i < EPC; i += 8) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + idx + i);
      w[i / 2] = v[0]; w[i / 2 + 1] = v[1]; w[i / 2 + 2] = v[2]; w[i / 2 + 3] = v[3];
    }
  } else {
    const u32x2 v = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(base) + idx);
    w[0] = v[0]; w[1] = v[1];
  }
#pragma unroll
  for (int j = 0; j < EPC / 2; ++j) {
    if (dtype == FUSEDOPS_BF16) {
      o[2 * j] = __uint_as_float(w[j] << 16);
      o[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    } else {
      o[2 * j] = f16_bits_to_f32(w[j] & 0xFFFF);
      o[2 * j + 1] = f16_bits_to_f32(w[j] >> 16);
    }
  }
}

template <int EPC>
__device__ __forceinline__ void store_chunk(void* base, int dtype, int64_t idx, const float (&v)[EPC]) {
  if (dtype == FUSEDOPS_F32) {
#pragma unroll
    for (int i = 0; i < EPC; i += 4)
      *reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx + i) = f32x4{v[i], v[i + 1], v[i + 2], v[i + 3]};
    return;
  }
  uint32_t w[EPC / 2];
#pragma unroll
  for (int j = 0; j < EPC / 2; ++j)
    w[j] = dtype == FUSEDOPS_BF16 ? pack_bf16x2(v[2 * j], v[2 * j + 1]) : pack_f16x2(v[2 * j], v[2 * j + 1]);
  if constexpr (EPC >= 8) {
#pragma unroll
    for (int i = 0; i < EPC; i += 8)
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + idx + i) =
          u32x4{w[i / 2], w[i / 2 + 1], w[i / 2 + 2], w[i / 2 + 3]};
  } else {
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(base) + idx) = u32x2{w[0], w[1]};
  }
}

template <int WPR>
__device__ __forceinline__ float row_sum(float v, float* lds, int wave_in_row) {
  v = wave_sum(v);
  if constexpr (WPR > 1) {
    const int lane = threadIdx.x & 63;
    __syncthreads();
    if (lane == 0) lds[wave_in_row] = v;
    __syncthreads();
    v = 0.f;
#pragma unroll
    for (int w = 0; w < WPR; ++w) v += lds[w];
  }
  return v;
}

// CH chunks of EPC elements per lane, WPR waves per row.
template <int CH, int EPC, int WPR>
__global__ __launch_bounds__(kThreads) void ln_gelu_kernel(LnArgs a) {
  __shared__ float lds[4];
  constexpr int kRowsPerBlock = 4 / WPR;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row_in_block = wave / WPR, wave_in_row = wave % WPR;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + row_in_block;
  // WPR > 1 has one row per block, so `row < rows` is uniform across the block's barriers.
  if (row >= a.rows) return;
  const int cols = a.cols;
  const int nchunks = cols / EPC;
  const int xb = a.io_dtype == FUSEDOPS_F32 ? 4 : 2;
  const char* xrow = static_cast<const char*>(a.x) + row * a.ldx * xb;

  float v[CH][EPC];
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int c = j * 64 * WPR + wave_in_row * 64 + lane;
    if (c < nchunks) {
      load_chunk<EPC>(xrow, a.io_dtype, (int64_t)c * EPC, v[j]);
    } else {
#pragma unroll
      for (int i = 0; i < EPC; ++i) v[j][i] = 0.f;
    }
  }

  float s = 0.f;
#pragma unroll
  for (int j = 0; j < CH; ++j)
#pragma unroll
    for (int i = 0; i < EPC; ++i) s += v[j][i];
  const float mean = row_sum<WPR>(s, lds, wave_in_row) / (float)cols;

  float q = 0.f;
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int c = j * 64 * WPR + wave_in_row * 64 + lane;
    if (c < nchunks) {
#pragma unroll
      for (int i = 0; i < EPC; ++i) {
        const float d = v[j][i] - mean;
        q += d * d;
      }
    }
  }
  const float var = row_sum<WPR>(q, lds, wave_in_row) / (float)cols;
  const float rstd = 1.0f / sqrtf(var + a.eps);

  const int yb = a.out_dtype == FUSEDOPS_F32 ? 4 : 2;
  char* yrow = static_cast<char*>(a.y) + row * a.ldy * yb;
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int c = j * 64 * WPR + wave_in_row * 64 + lane;
    if (c >= nchunks) continue;
    float g[EPC], b[EPC];
    if (a.gamma) {
      load_chunk<EPC>(a.gamma, a.param_dtype, (int64_t)c * EPC, g);
    } else {
#pragma unroll
      for (int i = 0; i < EPC; ++i) g[i] = 1.f;
    }
    if (a.beta) {
      load_chunk<EPC>(a.beta, a.param_dtype, (int64_t)c * EPC, b);
    } else {
#pragma unroll
      for (int i = 0; i < EPC; ++i) b[i] = 0.f;
    }
    float o[EPC];
#pragma unroll
    for (int i = 0; i < EPC; ++i) {
      const float yv = (v[j][i] - mean) * rstd * g[i] + b[i];
      o[i] = a.gelu_form == FUSEDOPS_GELU_TANH ? gelu_tanh_f32(yv)
             : a.gelu_form == FUSEDOPS_GELU_ERF ? gelu_erf_f32(yv) : yv;
    }
    store_chunk<EPC>(yrow, a.out_dtype, (int64_t)c * EPC, o);
  }
}

template <int CH, int EPC, int WPR>
hipError_t launch(const LnArgs& a, hipStream_t stream) {
  const int rows_per_block = 4 / WPR;
  const int64_t grid = (a.rows + rows_per_block - 1) / rows_per_block;
  LnArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(&ln_gelu_kernel<CH, EPC, WPR>), dim3((unsigned)grid),
                         dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_layernorm_gelu(const LnArgs& a, hipStream_t stream) {
  if (a.io_dtype == FUSEDOPS_F32) {
    const int chunks = a.cols / 4;
    if (chunks <= 64) return launch<1, 4, 1>(a, stream);
    if (chunks <= 128) return launch<2, 4, 1>(a, stream);
    if (chunks <= 256) return launch<4, 4, 1>(a, stream);
    if (chunks <= 512) return launch<8, 4, 1>(a, stream);
    if (chunks <= 1024) return launch<16, 4, 1>(a, stream);
    return launch<16, 4, 4>(a, stream);
  }
  const int chunks = a.cols / 8;
  if (chunks <= 64) return launch<1, 8, 1>(a, stream);
  if (chunks <= 128) return launch<2, 8, 1>(a, stream);
  if (chunks <= 256) return launch<4, 8, 1>(a, stream);
  if (chunks <= 512) return launch<8, 8, 1>(a, stream);
  return launch<8, 8, 4>(a, stream);
}

}  // namespace fusedops
