// Epilogue of the 256 x 256 bf16 tile kernel, run on the MFMA accumulators in place.
//
// The tile is computed transposed, D[f][t] = sum_k W[f][k] X[t][k]. Wave (wf, wt) of the
// workgroup holds features wf*128 .. +127 and tokens wt*128 .. +127 of the tile as
// acc[fb][tb] (4 x 4 blocks of v_mfma_f32_32x32x16_bf16 output). Register r of block
// (fb, tb) in lane l holds
//     local feature  wf*128 + fb*32 + 8*(r / 4) + 4*(l / 32) + (r % 4)
//     local token    wt*128 + tb*32 + (l % 32)
// so each lane owns runs ("groups") of four consecutive features of four tokens: 16 groups
// (fb, q = r / 4) per token. This is the layout the chain runs in ([Epilogue] §模式A,
// §模式B, §仿射量化与尾声的五步; op order as in the row-layout epilogue):
//   * per-feature vectors (bias, column scale) and the row scales are read from a small
//     LDS copy the kernel makes before its mainloop, so their load latency is hidden;
//   * SwiGLU pairs (2j, 2j+1) lie in one group, so gate and up meet in the same lane;
//   * a token's sum of squares over the wave's 128 features (one RMSNorm partial chunk)
//     is an in-lane sum over 64 registers plus one exchange with lane l ^ 32; the FP8
//     row absmax is reduced the same way;
//   * only finished values cross LDS: they are written in the output storage type into a
//     token-major, XOR-swizzled LDS tile, and the workgroup then stores whole rows with
//     16-byte coalesced writes (plain, or split across up to three destinations).
// Residual rows come in the other direction: a coalesced copy into the same LDS tile
// layout, then per-group reads. On the LDS-DMA path the static configurations with a bias or
// a 16-bit residual do that before the mainloop instead and start the accumulators from those
// values (seed_residual, or the bias in the mainloop's prologue), so the epilogue adds neither.
#pragma once

#include "epilogue.h"

namespace fusedops {


namespace accepi {

constexpr int kTileRows = 256;           // tokens per tile
constexpr int kTileCols = 256;           // features per tile
constexpr int kStageBytes = 128 * 1024;  // LDS available for one staged tile

__device__ __forceinline__ int dt_bytes(int dt) {
  return dt == FUSEDOPS_F32 ? 4 : (dt == FUSEDOPS_F8E4M3 ? 1 : 2);
}

// Byte offset of byte b of row r in a staged tile of C 16-byte chunks per row (C a power of
// two): chunk c sits at position c ^ (r mod min(C, 32)). Rows of one group write are 32
// consecutive tokens at one column, so those land on distinct chunk positions; row-wise
// copies touch all positions of a row.
__device__ __forceinline__ uint32_t st_off(int r, int b, int C) {
  const int m = (C < 32 ? C : 32) - 1;
  return (uint32_t)(r * C * 16 + ((((b >> 4) ^ (r & m))) << 4) + (b & 15));
}

// Write n = 4 (or 2) values of storage type dt at LDS byte offset off.
__device__ __forceinline__ void lds_put(uint8_t* lds, uint32_t off, int dt, f32x4 v, int n) {
  if (dt == FUSEDOPS_F32) {
    if (n == 4) *reinterpret_cast<f32x4*>(lds + off) = v;
    else *reinterpret_cast<float2*>(lds + off) = make_float2(v[0], v[1]);
  } else if (dt == FUSEDOPS_F8E4M3) {
    if (n == 4) *reinterpret_cast<uint32_t*>(lds + off) = pack_e4m3x2(v[0], v[1]) | (pack_e4m3x2(v[2], v[3]) << 16);
    else *reinterpret_cast<uint16_t*>(lds + off) = (uint16_t)pack_e4m3x2(v[0], v[1]);
  } else {
    const bool bf = dt == FUSEDOPS_BF16;
    const uint32_t lo = bf ? pack_bf16x2(v[0], v[1]) : pack_f16x2(v[0], v[1]);
    if (n == 4) {
      const uint32_t hi = bf ? pack_bf16x2(v[2], v[3]) : pack_f16x2(v[2], v[3]);
      *reinterpret_cast<u32x2*>(lds + off) = u32x2{lo, hi};
    } else {
      *reinterpret_cast<uint32_t*>(lds + off) = lo;
    }
  }
}

// Read 4 values of storage type dt (bf16 / fp16 / fp32) at LDS byte offset off.
__device__ __forceinline__ f32x4 lds_get4(const uint8_t* lds, uint32_t off, int dt) {
  if (dt == FUSEDOPS_F32) return *reinterpret_cast<const f32x4*>(lds + off);
  const u32x2 w = *reinterpret_cast<const u32x2*>(lds + off);
  if (dt == FUSEDOPS_BF16)
    return f32x4{bf16_bits_to_f32(w[0] & 0xFFFF), bf16_bits_to_f32(w[0] >> 16), bf16_bits_to_f32(w[1] & 0xFFFF),
                 bf16_bits_to_f32(w[1] >> 16)};
  return f32x4{f16_bits_to_f32(w[0] & 0xFFFF), f16_bits_to_f32(w[0] >> 16), f16_bits_to_f32(w[1] & 0xFFFF),
               f16_bits_to_f32(w[1] >> 16)};
}

// Four consecutive elements of a feature vector (bias, column scale) as fp32, or `fill`
// past the N features.
__device__ __forceinline__ f32x4 vec4(const void* p, int dt, int f, int N, float fill) {
  if (f >= N) return f32x4{fill, fill, fill, fill};
  return load4(p, dt, f);
}

// The tile's per-feature and per-token vectors, copied to LDS (as fp32) before the
// mainloop: [0] bias (0 past N), [1] column scale (1 past N), [2] row scale (0 past M).
// Thread tid loads element tid of each vector the configuration uses; the caller stores the
// values with `store` after issuing its own first loads, so the latency overlaps.
struct VecPrefetch {
  float v[3];
  int lab;
  template <uint32_t F>
  __device__ __forceinline__ void load(const EpiParams& e, int t0, int f0, int M, int N) {
    const epi::Cfg<F> cfg{e};
    const int tid = threadIdx.x;
    const int f = f0 + tid, t = t0 + tid;
    v[0] = cfg.bias() && f < N ? load1(e.bias, cfg.bias_dt(), f) : 0.f;
    v[1] = cfg.gamma() && f < N ? load1(e.gamma, cfg.gamma_dt(), f) : 1.f;
    v[2] = cfg.rscale() && t < M ? row_scale_of(e, t) : 0.f;
    lab = cfg.xent() && t < M ? e.xent_labels[t] : -1;
  }
  // svec: [0, 256) bias, [256, 512) column scale, [512, 768) row scale, [768, 1024) label bits.
  // tid: the thread index (a caller may pass an opaque copy, as for acc_epilogue)
  __device__ __forceinline__ void store(float* svec, int tid) const {
    svec[tid] = v[0];
    svec[256 + tid] = v[1];
    svec[512 + tid] = v[2];
    svec[768 + tid] = __int_as_float(lab);
  }
};

// Where a staged tile's rows go in global memory.
struct Dest {
  uint8_t* base[3];  // destination(s); more than one for a split store
  __device__ uint8_t* at(int seg) const { return seg == 0 ? base[0] : (seg == 1 ? base[1] : base[2]); }
  int64_t ld;        // elements per row
  int64_t split_w;   // columns per destination (0: a single destination)
  int es;            // bytes per element
  int cols;          // valid columns of the whole output (N, or N/2 after SwiGLU)
  int col0;          // first output column of the tile
};

// Copy a staged tile (R rows of C chunks) to global memory: thread tid takes chunks
// tid, tid + 256, ...; a chunk is one 16-byte store when it lies wholly inside the output
// and one destination, otherwise 4-byte stores of its valid words. The 16-byte stores are
// nontemporal: an output tile is written once, and kept in L2 its dirty lines would be
// written back later while the next tiles' operand loads need the space (measured on the
// out-projection, whose h1 and h2 are 2 M N bf16 per launch: 167.8 -> 143.1 us).
__device__ __forceinline__ void copy_out(const uint8_t* lds, int R, int C, int row0, int M, const Dest& d, int tid) {
  const int cshift = __builtin_ctz(C);
  const int per = 16 / d.es;  // elements per chunk
  const int sw = (int)d.split_w;
  // Interior tile (the usual case): every row valid and the whole column range inside the
  // output and inside one destination. Thread tid then copies chunk tid % C of rows
  // tid / C, tid / C + 256 / C, ... with no per-chunk tests (C <= 64, so every thread has
  // a chunk); a wave stores 1 KB of consecutive row pieces per instruction.
  const int col_end = d.col0 + C * per;
  const int seg0 = sw ? d.col0 / sw : 0;
  if (row0 + R <= M && col_end <= d.cols && (!sw || (col_end - 1) / sw == seg0)) {
    const int c = tid & (C - 1);
    const int rstep = kEpiThreads >> cshift;
    const int m = (C < 32 ? C : 32) - 1;
    int r = tid >> cshift;
    uint8_t* g = d.at(seg0) + ((int64_t)(row0 + r) * d.ld + (d.col0 - seg0 * sw) + c * per) * d.es;
    const int64_t gstep = (int64_t)rstep * d.ld * d.es;
#pragma unroll 8
    for (; r < R; r += rstep, g += gstep)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(lds + r * C * 16 + ((c ^ (r & m)) << 4)),
                                  reinterpret_cast<u32x4*>(g));
    return;
  }
#pragma unroll 8
  for (int id = tid; id < R * C; id += kEpiThreads) {
    const int r = id >> cshift, c = id & (C - 1);
    const int t = row0 + r;
    const int col = d.col0 + c * per;
    if (t >= M || col >= d.cols) continue;
    const u32x4 v = *reinterpret_cast<const u32x4*>(lds + st_off(r, c * 16, C));
    const int seg = sw ? col / sw : 0;
    const int cseg = col - seg * sw;
    const bool whole = col + per <= d.cols && (!sw || cseg + per <= sw);
    if (whole) {
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(d.at(seg) + ((int64_t)t * d.ld + cseg) * d.es));
    } else {
      // the row's last chunk (or one crossing a split boundary): whole 4-byte words, then
      // single elements of a word the output ends in (rows need not end on a word)
      const int nel = 4 / d.es;  // elements per word
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int cw = col + w * nel;  // first column of word w
        if (cw >= d.cols) break;
        const int sg = sw ? cw / sw : 0;
        uint8_t* p = d.at(sg) + ((int64_t)t * d.ld + (cw - sg * sw)) * d.es;
        if (cw + nel <= d.cols) {
          *reinterpret_cast<uint32_t*>(p) = v[w];
        } else if (d.es == 2) {
          *reinterpret_cast<uint16_t*>(p) = (uint16_t)v[w];   // one 2-byte element left
        } else {
          for (int i = 0; i < d.cols - cw; ++i) p[i] = (uint8_t)(v[w] >> (8 * i));  // 1-3 codes left
        }
      }
    }
  }
}

// Keep an updated accumulator block in AGPRs (the residual seed and the epilogue). The chain visits all 16 blocks per step and keeps
// every block between steps; left to itself the compiler holds the updated values in VGPRs,
// runs out of them and spills to scratch, each reload then waiting with vmcnt(0) for every
// load and store in flight. AGPRs are where the MFMAs left the blocks, and there is room.
// (Not for the FP8 row quantisation, where the pinned blocks measured more spills and a slower
// prefill: there the compiler's own placement is kept.)
template <uint32_t F>
__device__ __forceinline__ void to_agpr(f32x16& v) {
  if constexpr ((F & epi::kStatic) != 0 && (F & epi::kQuant) == 0) asm volatile("" : "+a"(v));
}

// Copy pass p (rows p * R .. p * R + R - 1 of the tile, R = 256 / passes) of the residual
// z into LDS in the staged-tile layout by DMA (each wave instruction fills 1 KB: lane i lands
// at position 16 i, so it fetches the chunk whose swizzled position that is), all
// instructions in flight at once, then wait until every wave's copies have landed. Rows past
// M and columns past N read as zero; a pass with no valid rows is zero-filled. The caller
// has made `lds` free (a barrier after its last reads).
template <class Cfg>
__device__ __forceinline__ void z_pass_to_lds(const EpiParams& e, const Cfg& cfg, uint8_t* lds, int t0, int f0,
                                              int M, int N, int p, int R, int C) {
  const int es = dt_bytes(cfg.z_dt());
  const int cshift = __builtin_ctz(C);
  const int m = (C < 32 ? C : 32) - 1;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane_u = threadIdx.x & 63;
  const int rows = min(R, M - t0 - p * R);  // valid rows of this pass (>= 1 for p = 0)
  if (rows > 0) {
    // The range ends at the 16-byte chunk boundary after the last valid column: a load that
    // crosses the end of the range reads as zero as a whole, which would drop the valid
    // columns of a chunk that N cuts through. The chunk lies inside its row's storage (the
    // leading dimension keeps rows 16-byte aligned); its columns past N are the caller's.
    const uint8_t* zb = static_cast<const uint8_t*>(e.z) + ((int64_t)(t0 + p * R) * e.ldz + f0) * es;
    const int zcols = (min(kTileCols, N - f0) + 16 / es - 1) / (16 / es) * (16 / es);
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(zb, (uint32_t)(((int64_t)(rows - 1) * e.ldz + zcols) * es));
#pragma unroll 8
    for (int j = 0; j < R * C / kEpiThreads; ++j) {
      const int id = j * kEpiThreads + wave * 64 + lane_u;
      const int r = id >> cshift, pos = id & (C - 1);
      const int c = pos ^ (r & m);
      const uint32_t oob = (uint32_t)(f0 + c * 16 / es >= N) << 31;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rz, (lds_void*)(lds + (j * kEpiThreads + wave * 64) * 16), 16,
                                               ((uint32_t)(r * e.ldz * es + c * 16)) | oob, 0, 0, kNonTemporal);
    }
  } else {
    for (int id = threadIdx.x; id < R * C; id += kEpiThreads)
      *reinterpret_cast<u32x4*>(lds + id * 16) = u32x4{0, 0, 0, 0};
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMA has landed
  lds_barrier();
}

// Whether a configuration's accumulators start from the residual (see seed_residual; a 16-bit
// residual, whose 256 x 256 tile fits the 128 KB of LDS at once), or, with no residual, from the
// bias (written by the LDS-DMA mainloop before its first MFMA).
template <uint32_t F>
constexpr bool seeds_residual() {
  return (F & epi::kStatic) != 0 && (F & epi::kZ) != 0 && ((F >> epi::kZShift) & 3) != FUSEDOPS_F32;
}
// (Not with RoPE: that instance measured 660 B of spills per lane seeded against 56 unseeded.)
template <uint32_t F>
constexpr bool seeds_bias() {
  return (F & epi::kStatic) != 0 && (F & epi::kBias) != 0 && (F & epi::kZ) == 0 && (F & epi::kRope) == 0;
}

// Start a tile's accumulators from its residual rows plus the bias, acc = z + b, before the
// mainloop: the MFMAs then accumulate the product on top, and the epilogue has neither the
// residual copy nor the add ([Epilogue] §模式A: h1 = residual + the GEMM output, computed here in
// the other association, fp32 throughout). At the start of a tile no accumulator is live, so
// the per-group reads need no registers the epilogue would have to give up. For tiles whose
// columns are all inside N (the LDS-DMA mainloop's condition, N % 256 == 0). `lds` is 128 KB
// of LDS no wave is using; `svec` holds the bias when the configuration has one; on return
// `lds` is free again.
template <uint32_t F>
__device__ __forceinline__ void seed_residual(const GemmArgs& a, f32x16 (&acc)[4][4], uint8_t* lds, const float* svec,
                                              int t0, int f0) {
  const EpiParams& e = a.ep;
  const epi::Cfg<F> cfg{e};
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wf = wave >> 1, wt = wave & 1;
  const int hb = lane >> 5, tl = lane & 31;
  static_assert(seeds_residual<F>(), "a 16-bit residual: the whole tile in one pass");
  const int zdt = cfg.z_dt();
  constexpr int es = 2;
  constexpr int C = kTileCols * es / 16;
  z_pass_to_lds(e, cfg, lds, t0, f0, a.M, a.N, 0, kTileRows, C);
#pragma unroll
  for (int fb = 0; fb < 4; ++fb) {
    f32x4 b[4] = {};
    if (cfg.bias()) {
#pragma unroll
      for (int q = 0; q < 4; ++q) b[q] = *reinterpret_cast<const f32x4*>(svec + wf * 128 + fb * 32 + q * 8 + hb * 4);
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int r = wt * 128 + tb * 32 + tl;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 z = lds_get4(lds, st_off(r, (wf * 128 + fb * 32 + q * 8 + hb * 4) * es, C), zdt);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[fb][tb][4 * q + j] = z[j] + b[q][j];
      }
      to_agpr<F>(acc[fb][tb]);
    }
  }
  lds_barrier();  // every wave has read its groups: `lds` is free
}

}  // namespace accepi

// Run the whole epilogue of one 256 x 256 tile whose accumulators are in `acc` (the
// layout above). `lds` is at least 128 KB of LDS that the mainloop no longer uses and
// `svec` the tile's vectors (VecPrefetch); every thread of the workgroup must call this.
// kSeeded: the accumulators started from the residual and the bias (seed_residual, or the bias
// alone when there is no residual), so neither is added here.
// tid: the thread index. A caller may pass an opaque copy, so that the per-lane constants are
// recomputed in every tile of a walk instead of computed once and, short of registers, spilled:
// a reload waits for every load in flight, including DMAs issued for the next tile.
// kStage: bytes of `lds` a staged tile may use (a larger one goes in two passes of 128 tokens).
template <uint32_t F, bool kSeeded = false, int kStage = accepi::kStageBytes>
__device__ __forceinline__ void acc_epilogue(const GemmArgs& a, f32x16 (&acc)[4][4], uint8_t* lds, const float* svec,
                                             int t0, int f0, int ft, int* slot, int tid) {
  using namespace accepi;
  const EpiParams& e = a.ep;
  const epi::Cfg<F> cfg{e};
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf = wave >> 1, wt = wave & 1;
  const int hb = lane >> 5, tl = lane & 31;
  const int M = a.M, N = a.N;
  // local feature of group (fb, q) and local token of block row tb
  auto fl = [&](int fb, int q) { return wf * 128 + fb * 32 + q * 8 + hb * 4; };
  auto tk = [&](int tb) { return wt * 128 + tb * 32 + tl; };

  const int act = cfg.act();
  const bool pairs = act == ACT_SWIGLU;
  const bool fused = !cfg.z() && !cfg.aux() && !cfg.part() && !cfg.quant() && !cfg.xent();

  // Stage the lane's values (4 per group, or the 2 SwiGLU outputs per group) in storage
  // type dt and store the tile to `d`. `val(fb, tb)` yields block (fb, tb); tiles larger
  // than 128 KB go in two passes of 128 tokens, each staged by the waves that own them.
  auto emit = [&](int dt, bool pr, const accepi::Dest& d, auto&& val) __attribute__((always_inline)) {
    const int es = dt_bytes(dt);
    const int cols = pr ? kTileCols / 2 : kTileCols;
    const int C = cols * es / 16;
    const int passes = kTileRows * cols * es > kStage ? 2 : 1;
    const int R = kTileRows / passes;
#pragma clang loop unroll(disable)
    for (int p = 0; p < passes; ++p) {
      lds_barrier();  // earlier stores may still drain
      if (passes == 1 || wt == p) {
#pragma unroll
        for (int fb = 0; fb < 4; ++fb)
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) {
            const f32x16 v = val(fb, tb);
            const int r = tk(tb) - p * R;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x4 g{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
              if (pr) lds_put(lds, st_off(r, fl(fb, q) / 2 * es, C), dt, g, 2);
              else lds_put(lds, st_off(r, fl(fb, q) * es, C), dt, g, 4);
            }
          }
      }
      lds_barrier();
      copy_out(lds, R, C, t0 + p * R, M, d, tid);
    }
  };

  // per-feature vector k (0 bias, 1 column scale) of feature block fb (16 values per lane)
  auto feat = [&](int k, int fb) __attribute__((always_inline)) {
    f32x16 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(svec + k * 256 + fl(fb, q));
      o[4 * q] = x[0]; o[4 * q + 1] = x[1]; o[4 * q + 2] = x[2]; o[4 * q + 3] = x[3];
    }
    return o;
  };
  auto rs_of = [&](int tb) __attribute__((always_inline)) { return svec[512 + tk(tb)]; };
  // column scale, row scale, activation on one block (SwiGLU leaves the two outputs of
  // group q in registers 4q and 4q + 1, zeros in 4q + 2 and 4q + 3)
  auto post = [&](f32x16 v, const f32x16& g, int tb) __attribute__((always_inline)) {
    if (cfg.gamma()) v *= g;
    if (cfg.rscale()) v *= rs_of(tb);
    if (act == ACT_GELU_ERF) {
      // a seeded tile with no scale feeds the accumulators straight in; a static bf16 output
      // takes the degree-6 h
      constexpr bool raw = kSeeded && (F & (epi::kGamma | epi::kRscale)) == 0;
      constexpr bool bf16 = (F & epi::kStatic) != 0 && ((F >> epi::kYShift) & 3) == FUSEDOPS_BF16 &&
                            (F & epi::kQuant) == 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = raw ? gelu_erf_acc_f32<bf16>(v[r]) : gelu_erf_f32<bf16>(v[r]);
    } else if (act == ACT_GELU_TANH) {
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = gelu_tanh_f32(v[r]);
    } else if (pairs) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float o0 = silu_f32(v[4 * q]) * v[4 * q + 1];
        const float o1 = silu_f32(v[4 * q + 2]) * v[4 * q + 3];
        v[4 * q] = o0; v[4 * q + 1] = o1; v[4 * q + 2] = 0.f; v[4 * q + 3] = 0.f;
      }
    }
    return v;
  };

  const int ydt = cfg.y_dt();
  accepi::Dest dy;
  dy.es = dt_bytes(ydt);
  dy.cols = pairs ? N / 2 : N;
  dy.col0 = pairs ? f0 / 2 : f0;
  if (cfg.split()) {
    dy.base[0] = static_cast<uint8_t*>(e.yv0);
    dy.base[1] = static_cast<uint8_t*>(e.yv1);
    dy.base[2] = static_cast<uint8_t*>(e.yv2);
    dy.ld = e.ldv;
    dy.split_w = e.split_w;
  } else {
    dy.base[0] = static_cast<uint8_t*>(e.y);
    dy.base[1] = dy.base[2] = nullptr;
    dy.ld = e.ldy;
    dy.split_w = 0;
  }

  if (fused && cfg.rope()) {
    // RoPE on adjacent feature pairs after bias and activation ([Epilogue] §模式B: a pairwise
    // map on the accumulators): a lane's group of four features f .. f+3 holds the pairs
    // (f, f+1) and (f+2, f+3), whose cos / sin are the four floats at column f mod d of the
    // token's table row (d divides the 256-feature tile, so f mod d = local feature mod d).
    // Groups at or past rope_cols (V under a Q/K/V split) stay as computed; that test depends
    // only on the feature, so it is uniform in a wave. Table rows past M read as zero.
    if (cfg.bias() && !kSeeded) {
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) {
        const f32x16 b = feat(0, fb);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) acc[fb][tb] += b;
      }
    }
    if (f0 < e.rope_cols) {
      // The tile's table rows (tokens t0 .., rope_d floats each) are copied into LDS by DMA in
      // the staged-tile layout (16-byte chunk c of row r at position c ^ (r mod min(C, 32))),
      // with every wave instruction filling 1 KB of consecutive positions; each lane then reads
      // its 16-byte (cos, sin, cos, sin) runs from LDS, free of bank conflicts for rope_d >= 64.
      // Table rows past M are not read (their outputs are never stored).
      const int rows = min(kTileRows, M - t0);
      const int C = e.rope_d >> 2;  // 16-byte chunks per table row (rope_d a power of two >= 8)
      const int cshift = __builtin_ctz(C);
      const int m = (C < 32 ? C : 32) - 1;
      const __amdgpu_buffer_rsrc_t rc = make_rsrc(e.rope_cs + (int64_t)t0 * e.rope_ld,
                                                  (uint32_t)(((int64_t)(rows - 1) * e.rope_ld + e.rope_d) * 4));
      const int lane_u = threadIdx.x & 63;
#pragma unroll 8
      for (int j = 0; j < C; ++j) {  // kTileRows * C chunks, kEpiThreads per instruction round
        const int id = j * kEpiThreads + wave * 64 + lane_u;
        const int r = id >> cshift, pos = id & (C - 1);
        const int c = pos ^ (r & m);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (lds_void*)(lds + (j * kEpiThreads + wave * 64) * 16), 16,
                                                 (uint32_t)((r * e.rope_ld + c * 4) * 4), 0, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMA has landed
      lds_barrier();
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) {
        f32x4 cs4[4][4];  // [q][tb]: cos_i, sin_i, cos_i+1, sin_i+1
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int tb = 0; tb < 4; ++tb)
            cs4[q][tb] = *reinterpret_cast<const f32x4*>(lds + st_off(tk(tb), (fl(fb, q) & (e.rope_d - 1)) * 4, C));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (f0 + fl(fb, q) >= e.rope_cols) continue;
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) {
            f32x16& v = acc[fb][tb];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const float x0 = v[4 * q + 2 * j], x1 = v[4 * q + 2 * j + 1];
              const float cs = cs4[q][tb][2 * j], sn = cs4[q][tb][2 * j + 1];
              v[4 * q + 2 * j] = x0 * cs - x1 * sn;
              v[4 * q + 2 * j + 1] = x0 * sn + x1 * cs;
            }
          }
        }
      }
    }
    emit(ydt, pairs, dy, [&](int fb, int tb) __attribute__((always_inline)) { return acc[fb][tb]; });
    return;
  }

  if (fused) {
    // bias, scales and activation straight into the staged output tile
    f32x16 b = {}, g = {};
    int fb_loaded = -1;
    emit(ydt, pairs, dy, [&](int fb, int tb) __attribute__((always_inline)) {
      if (fb != fb_loaded) {
        if (cfg.bias() && !kSeeded) b = feat(0, fb);
        if (cfg.gamma()) g = feat(1, fb);
        fb_loaded = fb;
      }
      f32x16 v = acc[fb][tb];
      if (cfg.bias() && !kSeeded) v += b;
      return post(v, g, tb);
    });
    return;
  }

  // ---- pre-activation h1 = acc + bias + residual, in place
  if (cfg.bias() && !kSeeded) {
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
      const f32x16 b = feat(0, fb);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        acc[fb][tb] += b;
        to_agpr<F>(acc[fb][tb]);
      }
    }
  }
  if (cfg.z() && !kSeeded) {
    // The residual rows are copied into the staged-tile layout (z_pass_to_lds), then read
    // back per group.
    const int zdt = cfg.z_dt();
    const int es = dt_bytes(zdt);
    const int C = kTileCols * es / 16;
    const int passes = kTileRows * kTileCols * es > kStage ? 2 : 1;
    const int R = kTileRows / passes;
#pragma clang loop unroll(disable)
    for (int p = 0; p < passes; ++p) {
      lds_barrier();
      z_pass_to_lds(e, cfg, lds, t0, f0, M, N, p, R, C);
      if (passes == 1 || wt == p) {
        // a 16-byte chunk that N cuts through was loaded whole: in the wave whose features reach
        // past N (uniform), its columns past N are zeroed so they add nothing to h1 and to the
        // row partials
        const bool tail = f0 + wf * 128 + 128 > N;
#pragma unroll
        for (int fb = 0; fb < 4; ++fb)
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) {
            f32x16 v = acc[fb][tb];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              f32x4 z = lds_get4(lds, st_off(tk(tb) - p * R, fl(fb, q) * es, C), zdt);
              if (tail) {
#pragma unroll
                for (int j = 0; j < 4; ++j) z[j] = f0 + fl(fb, q) + j < N ? z[j] : 0.f;
              }
#pragma unroll
              for (int j = 0; j < 4; ++j) v[4 * q + j] += z[j];
            }
            acc[fb][tb] = v;
            to_agpr<F>(acc[fb][tb]);
          }
      }
    }
  }
  if (cfg.aux()) {
    accepi::Dest d{{static_cast<uint8_t*>(e.aux), nullptr, nullptr}, e.ld_aux, 0, dt_bytes(cfg.aux_dt()), N, f0};
    emit(cfg.aux_dt(), false, d, [&](int fb, int tb) __attribute__((always_inline)) { return acc[fb][tb]; });
  }
  if (cfg.part()) {
    // sum of squares of the token's 128 features of this wave: one RMSNorm partial chunk
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      float s = 0.f;
#pragma unroll
      for (int fb = 0; fb < 4; ++fb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s = __builtin_fmaf(acc[fb][tb][r], acc[fb][tb][r], s);
      s += __shfl_xor(s, 32, kWave);
      const int t = t0 + tk(tb);
      if (hb == 0 && t < M && f0 + wf * 128 < N) e.partials[(int64_t)t * e.ldp + f0 / 128 + wf] = s;
    }
  }

  // ---- column scale, row scale, activation, in place
  if (cfg.gamma() || cfg.rscale() || act != ACT_NONE) {
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
      f32x16 g = {};
      if (cfg.gamma()) g = feat(1, fb);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        acc[fb][tb] = post(acc[fb][tb], g, tb);
        to_agpr<F>(acc[fb][tb]);
      }
    }
  }

  if (cfg.xent()) {
    // Cross-entropy statistics on the accumulators ([Epilogue] §模式C): a wave's 128 features
    // are two 64-column chunks (block pairs fb 0-1 and 2-3); a lane holds 32 of a chunk's values
    // for each of its tokens and lane l ^ 32 the other 32, so each (max, sum-exp) is an in-lane
    // reduction plus one exchange. Columns at or past N are left out. The lane holding a token's
    // label column writes the target.
    constexpr float kLog2e = 1.4426950408889634f;
    const int wbase = f0 + wf * 128;  // first column of the wave's 128
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int t = t0 + tk(tb);
      const bool t_ok = t < M;
      // the label's register in this lane, if the lane holds it: column wbase + 32 fb + 8 q +
      // 4 hb + j sits in register 4 q + j of block fb
      const int o = __float_as_int(svec[768 + tk(tb)]) - wbase;  // label, fetched before the mainloop
      const bool mine = o >= 0 && o < 128 && wbase + o < N && ((o >> 2) & 1) == hb;
      // a token's label lies in one column tile of its row, so most waves hold none: the
      // register select runs only when some lane of the wave holds its label (uniform test)
      if (__ballot(mine) != 0) {
        const int want = (o >> 5) * 16 + ((o >> 3) & 3) * 4 + (o & 3);  // fb * 16 + r
        float tv = 0.f;
#pragma unroll
        for (int fb = 0; fb < 4; ++fb)
#pragma unroll
          for (int r = 0; r < 16; ++r) tv = want == fb * 16 + r ? acc[fb][tb][r] : tv;
        if (mine) e.xent_tgt[t] = tv;
      }
      // columns at or past N (last tile only, a wave-uniform test) become -inf: they drop out
      // of the maximum, and e^-inf = 0 out of the sum; they are never stored
      if (wbase + 128 > N) {
#pragma unroll
        for (int fb = 0; fb < 4; ++fb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            acc[fb][tb][r] = f0 + fl(fb, r >> 2) + (r & 3) < N ? acc[fb][tb][r] : -INFINITY;
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int cf = wbase + c * 64;  // first column of the chunk
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) m = fmaxf(m, acc[2 * c + i][tb][r]);
        float sx = 0.f;
        const float mb = m == -INFINITY ? 0.f : m * kLog2e;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) sx += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[2 * c + i][tb][r], kLog2e, -mb));
        const float mo = __shfl_xor(m, 32, kWave), so = __shfl_xor(sx, 32, kWave);
        const float mn = fmaxf(m, mo);
        // (terms below 2^-126 of the chunk maximum flush to zero: the sums are at least 1)
        sx = mn == -INFINITY ? 0.f
                             : sx * __builtin_amdgcn_exp2f((m - mn) * kLog2e) + so * __builtin_amdgcn_exp2f((mo - mn) * kLog2e);
        if (hb == 0 && t_ok && cf < N) {
          float* st = e.xent_stats + (int64_t)t * e.xent_ld + 2 * (cf / 64);
          st[0] = mn;
          st[1] = sx;
        }
      }
    }
    if (!e.y) return;  // logits not stored
  }

  if (!cfg.quant()) {
    emit(ydt, pairs, dy, [&](int fb, int tb) __attribute__((always_inline)) { return acc[fb][tb]; });
    return;
  }

  // ---- FP8 per-row quantisation: publish this tile's row absmax in its own workspace slots,
  // meet every other column tile of the row block, reduce the slots of the tile's rows, then
  // scale by 1 / s with s = fl32(absmax / 448)
  float* s_half = reinterpret_cast<float*>(lds);  // [2][256]: per feature half (wf)
  float* s_amax = s_half + 2 * kTileRows;         // [256]: row absmax over all column tiles
  __syncthreads();
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    float m = 0.f;
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(acc[fb][tb][r]));
    m = fmaxf(m, __shfl_xor(m, 32, kWave));
    if (hb == 0) s_half[wf * kTileRows + tk(tb)] = m;
  }
  __syncthreads();
  {
    const int i = threadIdx.x, t = t0 + i;
    if (t < M) publish_row_amax(e, ft, t, fmaxf(s_half[i], s_half[kTileRows + i]));
  }
  rendezvous_row_amax<kTileRows>(e, ft, a.tiles_f, t0, min(kTileRows, M - t0), s_amax, slot);
  __syncthreads();
  {
    const int i = threadIdx.x, t = t0 + i;
    if (f0 == 0 && t < M) e.scales[t] = __fdiv_rn(s_amax[i], 448.0f);
  }
  Fp8RowFactor fac[4];
  bool tiny = false;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    fac[tb] = fp8_row_factor(__fdiv_rn(s_amax[tk(tb)], 448.0f));  // IEEE division: s = fl32(a / 448)
    tiny |= fac[tb].pre != 1.f;
  }
  // rows with a scale below 2^-100 (the pre-scaled path) are rare: a wave-uniform test keeps
  // the extra multiply out of every other wave
  const bool any_tiny = __ballot(tiny) != 0;
  emit(ydt, pairs, dy, [&](int fb, int tb) __attribute__((always_inline)) {
    f32x16 v = acc[fb][tb];
    if (any_tiny) v *= fac[tb].pre;
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = fminf(fmaxf(v[r] * fac[tb].inv, -448.f), 448.f);
    return v;
  });
}

}  // namespace fusedops
