// bf16 fused linear layer for gfx950: Y = epilogue(X W^T + b).
//
// Mainloop ([Fusion] §Linear算子剖析; [Epilogue] §主循环与尾声): one workgroup of
// 4 waves owns a 256-feature x 256-token output tile and walks K in steps of 64.
// Each step's W and X tiles (256 rows x 64 bf16, both K-contiguous in HBM) are
// staged in LDS, double buffered. Two ways of filling LDS:
//  * LDS DMA (tiles with whole W rows and an even number of K steps, every workload
//    shape): buffer loads write LDS directly, two steps ahead, into space the MFMAs of
//    the current step have just finished reading (mainloop_dma);
//  * register staging (any shape): during step s the MFMAs read LDS buffer s&1 while
//    the data of step s+1 (already in registers) is written to the other buffer and the
//    16-byte global loads of step s+2 are issued. One barrier per step.
// In both, MFMAs, operand reads and fills or loads are interleaved so that the single
// wave per SIMD always has matrix work queued.
//
// LDS layout: a 64-wide K tile row is 128 bytes = 8 chunks of 16 bytes, XOR-swizzled
// per row (see swz) so the ds_read_b128 operand fetches and the fills are free of
// bank conflicts.
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
constexpr int kBuf = 2 * kTileBytes;      // one stage: W tile then X tile

// One 16-byte-per-lane LDS DMA: lane l's 16 bytes at rsrc + soff + voff land at LDS byte
// lds + 16 l. Issued as inline assembly so that the compiler, which cannot tell the DMA's LDS
// destination from the buffers being read, does not wait for it before every LDS read; M0
// (the LDS base of the DMA) is set inside the same statement. Every wait on these DMAs is
// placed by hand (dma_wait_barrier).
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "s"(lds)
               : "memory");
}

// Wait until at most N of this wave's LDS DMAs are still in flight and all of its LDS reads
// have returned, then meet the other waves. The DMAs write LDS without the compiler tracking
// them, so every wait on them is placed by hand; the "memory" clobber keeps the compiler from
// moving LDS accesses across the barrier.
template <int N>
__device__ __forceinline__ void dma_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// The per-lane addressing of one tile's operand DMAs on the LDS-DMA path. One DMA instruction
// fills 8 consecutive LDS rows (1 KB): lane l writes position l % 8 of row l / 8, which holds
// logical chunk (l % 8) ^ swz(row). For a group of rows starting at a multiple of 8, swz(row) =
// l / 8 ^ (bit 3 of the group's first row). Step t goes to stage t & 1; DMAs of steps past the
// last read nothing (the offset's top bit puts them out of range) and leave LDS as it is.
struct DmaPlan {
  const GemmArgs& a;
  __amdgpu_buffer_rsrc_t rW, rX;
  uint32_t lds0;          // LDS byte address of the stages
  int wave;
  uint32_t w_lane[2];     // W row group g of a block
  uint32_t x_lane[2][4];  // X token half h, row group g (rows past M read row M - 1)

  // tid: the thread index (the caller may pass an opaque copy, see mainloop_dma)
  __device__ __forceinline__ DmaPlan(const GemmArgs& args, uint8_t* smem, int t0, int f0, int tid) : a(args) {
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int x_rows = min(BT, a.M - t0);
    const uint16_t* Wt = static_cast<const uint16_t*>(a.W) + (int64_t)f0 * a.ldw;
    const uint16_t* Xt = static_cast<const uint16_t*>(a.X) + (int64_t)t0 * a.ldx;
    rW = make_rsrc(Wt, (uint32_t)(((int64_t)(BF - 1) * a.ldw + a.K) * 2));
    rX = make_rsrc(Xt, (uint32_t)(((int64_t)(x_rows - 1) * a.ldx + a.K) * 2));
    lds0 = (uint32_t)(uintptr_t)(lds_void*)smem;
    const int l8 = lane >> 3, p8 = lane & 7;
#pragma unroll
    for (int g = 0; g < 2; ++g) w_lane[g] = (uint32_t)(l8 * a.ldw * 2 + ((p8 ^ l8 ^ g) << 4));
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r = min(x_row0(h) + g * 8 + l8, x_rows - 1);
        x_lane[h][g] = (uint32_t)(r * a.ldx * 2 + ((p8 ^ l8 ^ (g & 1)) << 4));
      }
  }
  // W: wave w fills rows (w >> 1) * 128 + j * 32 + (w & 1) * 16 + g * 8 .. of block j, g = 0, 1
  __device__ __forceinline__ int w_row0() const { return (wave >> 1) * 128 + (wave & 1) * 16; }
  // X: token half h of the tile is token blocks 2h and 2h + 1 of both 128-token halves (what
  // every wave reads for those blocks); wave w fills its rows x_row0(h) + g * 8 .., g = 0..3
  __device__ __forceinline__ int x_row0(int h) const { return (wave >> 1) * 128 + (2 * h + (wave & 1)) * 32; }
  __device__ __forceinline__ int steps() const { return a.K / BK; }
  __device__ __forceinline__ void w1(int t, int j, int g) const {
    const uint32_t oob = t < steps() ? 0u : kOobOffset;
    const int r0 = w_row0() + j * 32 + g * 8;
    lds_dma16(rW, w_lane[g] | oob, (uint32_t)(r0 * a.ldw * 2 + t * BK * 2), lds0 + (t & 1) * kBuf + r0 * 128);
  }
  __device__ __forceinline__ void x1(int t, int h, int g) const {
    const uint32_t oob = t < steps() ? 0u : kOobOffset;
    lds_dma16(rX, x_lane[h][g] | oob, (uint32_t)(t * BK * 2), lds0 + (t & 1) * kBuf + kTileBytes + (x_row0(h) + g * 8) * 128);
  }
  __device__ __forceinline__ void w(int t, int j) const { w1(t, j, 0); w1(t, j, 1); }
  __device__ __forceinline__ void x(int t, int h) const {
#pragma unroll
    for (int g = 0; g < 4; ++g) x1(t, h, g);
  }
  // A tile's first 16 DMAs per wave, in the prologue's order: all of step 0 (stage 0 only).
  __device__ __forceinline__ void head() const { x(0, 0); x(0, 1); w(0, 0); w(0, 1); w(0, 2); w(0, 3); }
};

// Static configurations whose epilogue leaves LDS stage 0 alone: SwiGLU halves in 16 bits
// (a 64 KB staged tile, placed in stage 1) and the cross-entropy statistics (nothing staged
// unless the logits are stored, which is checked at run time). In the tile walk they issue the
// next tile's first DMAs (DmaPlan::head) as soon as the mainloop is done, so that data lands
// while the epilogue runs instead of at the start of the next tile. (A whole 16-bit tile would
// need two 64 KB passes in stage 1; for MLP-up that cost more than the early DMAs saved.)
template <uint32_t F>
constexpr bool prefetches_head() {
  constexpr uint32_t kStages = epi::kZ | epi::kAux | epi::kPart | epi::kQuant | epi::kSplit | epi::kRope;
  if ((F & epi::kStatic) == 0 || (F & kStages) != 0) return false;
  if ((F & epi::kXent) != 0) return true;
  constexpr int y = (F >> epi::kYShift) & 3;
  return ((F >> epi::kActShift) & 3) == ACT_SWIGLU && (y == FUSEDOPS_BF16 || y == FUSEDOPS_F16);
}

// Static configurations whose epilogue reads per-feature or per-token vectors (bias, column
// or row scale, labels); the others fetch and store none.
template <uint32_t F>
constexpr bool has_vectors() {
  return (F & epi::kStatic) != 0 && (F & (epi::kBias | epi::kGamma | epi::kRscale | epi::kXent)) != 0;
}

// Of the prefetching ones, those with vectors but no bias (which would start the accumulators
// in the mainloop): only their epilogue reads the vectors, which are then stored to LDS after
// the mainloop. Stored in the prologue, they would need the wait for their loads there, which
// the compiler places after the prologue's DMAs, draining them.
template <uint32_t F>
constexpr bool late_vectors() {
  return prefetches_head<F>() && has_vectors<F>() && (F & epi::kBias) == 0;
}

// Compile-time loop: f(integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, class Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Mainloop fed by LDS DMA (buffer loads that write LDS directly: no staging registers and no
// ds_write), for tiles whose W rows and K steps are all whole (N % 256 == 0, K % 128 == 0;
// checked on the host). An LDS DMA instruction whose lanes are all out of range leaves LDS
// untouched instead of writing zeros, so ragged token tiles do not rely on out-of-range reads:
// X rows past M are read from the tile's last valid row instead (their outputs are never stored
// and no reduction mixes rows).
//
// Buffers: W and X tiles of a step (256 rows x 128 bytes each, the swizzled layout of
// tile256.h), two of each. A step is walked in two regions: A multiplies feature blocks 0-1
// (W rows wf*128 + 0..63 of each wave's half), B blocks 2-3, each wave against its 128 tokens,
// whose fragments for the whole step sit in registers (read during the previous step: token
// blocks 0-1 in region A, 2-3 in region B). A region reads the W fragments the next region
// multiplies, so after A W blocks 2-3 of a buffer and X token half 0 (token blocks 0-1 of
// both 128-token halves) are free, after B W blocks 0-1 and X token half 1. Each region ends
// with a barrier after which the space just freed is refilled by DMA with data two steps
// ahead. Per wave and step the DMAs are (2 instructions per W block, 4 per X half)
//   region A: W blocks 0-1, X half 1 of s+2        region B: W blocks 2-3 of s+2, X half 0 of s+3
// so every DMA has 1.5 steps to land, and each is paired with an MFMA: the four waves leave a
// barrier together, and DMAs issued back to back would queue at the CU's address unit while
// the matrix core idles. Each barrier waits for exactly the DMAs the next region reads; the
// counts follow from this fixed issue order, which the prologue reproduces.
//
// kBiasStart: the accumulators start from the tile's bias (written here, once the prologue's
// first barrier has made the LDS copy of the vectors visible) instead of from zero.
template <uint32_t F, bool kBiasStart>
__device__ __forceinline__ void mainloop_dma(const GemmArgs& a, uint8_t* smem, float* svec,
                                             const accepi::VecPrefetch& vp, f32x16 (&acc)[4][4], int t0, int f0,
                                             bool head_loaded) {
  // The per-lane DMA and fragment offsets below are the same for every tile, so the compiler
  // would compute them once, keep them live across the whole tile walk and, short of registers,
  // spill them; each reload in the prologue then needs vmcnt(0), which also waits for every DMA
  // and store in flight. An opaque copy of the thread index makes them per-tile values that are
  // recomputed (a few dozen VALU ops per tile) instead.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const DmaPlan d(a, smem, t0, f0, tid);
  const int wave = d.wave, lane = tid & 63;
  const int wf = wave >> 1, wt = wave & 1;
  // With the next tile's head prefetched, and with the residual seed, the step count is opaque
  // too: the loop's entry test would otherwise be hoisted out of the walk and held across every
  // tile, and spilled, its reload waiting for the DMAs in flight. (The other instances measured
  // more spills with it.)
  int steps = a.K / BK;
  if constexpr (prefetches_head<F>() || accepi::seeds_residual<F>()) asm volatile("" : "+s"(steps));
  // DMAs of steps past the last are still issued so that the wait counts stay exact.
  auto dma_w1 = [&](int t, int j, int g) __attribute__((always_inline)) { d.w1(t, j, g); };
  auto dma_x1 = [&](int t, int h, int g) __attribute__((always_inline)) { d.x1(t, h, g); };
  auto dma_w = [&](int t, int j) __attribute__((always_inline)) { d.w(t, j); };
  auto dma_x = [&](int t, int h) __attribute__((always_inline)) { d.x(t, h); };

  // Operand fragments: row (lane % 32) of a 32-row block, logical chunk 2 kk + lane / 32.
  const int a_row0 = wf * 128 + (lane & 31);
  const int b_row0 = wt * 128 + (lane & 31);
  uint32_t koff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) koff[kk] = (uint32_t)((((kk * 2 + (lane >> 5)) ^ swz(lane & 31))) << 4);
  bf16x8 wfr[2][2][4];  // W fragments of two feature blocks [set][block][kk], double buffered
  bf16x8 xf[2][4][4];   // X fragments of a whole step [set][token block][kk], double buffered
  auto frag = [&](int t, bool x, int row, int kk) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(smem + (t & 1) * kBuf + (x ? kTileBytes : 0) + row * 128 + koff[kk]);
  };

  // One half-step region: MFMA i of the 32 (feature block J0 + i / 16, kk = i / 4 % 4, token
  // block i % 4), with the region's 16 fragment reads after the even MFMAs and its 8 DMAs
  // after MFMAs 1, 5, .., 29 (a wave's LDS reads are latency-bound, so bursts stall the
  // MFMAs); sched barriers keep that order. rd(q) and dm(d) are the region's reads and DMAs.
  auto region = [&](auto j0_c, const bf16x8 (&w)[2][4], const bf16x8 (&x)[4][4], auto&& rd, auto&& dm)
                    __attribute__((always_inline)) {
    constexpr int J0 = decltype(j0_c)::value;
    static_for<0, 32>([&](auto i_c) __attribute__((always_inline)) {
      constexpr int i = decltype(i_c)::value;
      constexpr int jb = i / 16, kk = (i / 4) % 4, tb = i % 4;
      __builtin_amdgcn_sched_barrier(0);
      acc[J0 + jb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[jb][kk], x[tb][kk], acc[J0 + jb][tb], 0, 0, 0);
      if constexpr (i % 2 == 0) rd(std::integral_constant<int, i / 2>{});
      if constexpr (i % 4 == 1) dm(std::integral_constant<int, i / 4>{});
    });
    __builtin_amdgcn_sched_barrier(0);
  };

  // Step s with X fragments in set P (the next step's go to set P ^ 1). Region A multiplies
  // feature blocks 0-1 (W fragments in wfr[0]) and reads W blocks 2-3 of s and X token blocks
  // 0-1 of s+1; region B multiplies blocks 2-3 and reads W blocks 0-1 and X token blocks 2-3
  // of s+1. Each region reads 16 KB per wave and issues 8 DMAs; every DMA lands 1.5 steps
  // before its data is read.
  auto step = [&](auto p_c, int s) __attribute__((always_inline)) {
    constexpr int P = decltype(p_c)::value;
    // A: DMA W blocks 0-1 of s+2 (read in B of s-1) and X token half 1 of s+2 (read in B of s-1)
    region(std::integral_constant<int, 0>{}, wfr[0], xf[P],
           [&](auto r) __attribute__((always_inline)) {
             constexpr int q = decltype(r)::value;
             if constexpr (q < 8) wfr[1][q / 4][q % 4] = frag(s, false, a_row0 + (2 + q / 4) * 32, q % 4);
             else xf[P ^ 1][(q - 8) / 4][(q - 8) % 4] = frag(s + 1, true, b_row0 + ((q - 8) / 4) * 32, (q - 8) % 4);
           },
           [&](auto d) __attribute__((always_inline)) {
             constexpr int q = decltype(d)::value;
             if constexpr (q < 4) dma_w1(s + 2, q / 2, q % 2);
             else dma_x1(s + 2, 1, q - 4);
           });
    dma_wait_barrier<16>();  // next: W blocks 0-1 and X token half 1 of s+1 (region A of s-1)
    // B: DMA W blocks 2-3 of s+2 and X token half 0 of s+3 (both read in A of s)
    region(std::integral_constant<int, 2>{}, wfr[1], xf[P],
           [&](auto r) __attribute__((always_inline)) {
             constexpr int q = decltype(r)::value;
             if constexpr (q < 8) wfr[0][q / 4][q % 4] = frag(s + 1, false, a_row0 + (q / 4) * 32, q % 4);
             else
               xf[P ^ 1][2 + (q - 8) / 4][(q - 8) % 4] =
                   frag(s + 1, true, b_row0 + (2 + (q - 8) / 4) * 32, (q - 8) % 4);
           },
           [&](auto d) __attribute__((always_inline)) {
             constexpr int q = decltype(d)::value;
             if constexpr (q < 4) dma_w1(s + 2, 2 + q / 2, q % 2);
             else dma_x1(s + 3, 0, q - 4);
           });
    dma_wait_barrier<16>();  // next: W blocks 2-3 of s+1 and X token half 0 of s+2 (region B of s-1)
  };

  // Prologue: X and W blocks 0-1 of step 0, then the loop's own DMA order from region B of
  // step -2 (W blocks 2-3 of step 0, X half 0 of step 1) and region A of step -1 (W blocks
  // 0-1 and X half 1 of step 1); the fragments of step 0; region B of step -1 (W blocks 2-3 of
  // step 1, X half 0 of step 2, into space the step-0 fragments were read from). With
  // head_loaded the previous tile's epilogue issued all of step 0 (DmaPlan::head) and the first
  // wait takes it whole, with the stores issued after it; from the next wait on, the DMAs in
  // flight are the same either way.
  // the epilogue vectors go to LDS before the DMAs: their values are in registers by now, and
  // a spilled one's reload after the DMAs would wait for all of them
  if constexpr (has_vectors<F>() && !late_vectors<F>() && !accepi::seeds_residual<F>()) vp.store(svec, tid);
  head_loaded = prefetches_head<F>() && head_loaded;
  if (!head_loaded) {  // the same DMAs as DmaPlan::head
    dma_x(0, 0); dma_x(0, 1);
    dma_w(0, 0); dma_w(0, 1);
    dma_w(0, 2); dma_w(0, 3);
  }
  dma_x(1, 0);
  dma_w(1, 0); dma_w(1, 1); dma_x(1, 1);
  if (head_loaded) dma_wait_barrier<12>();  // step 0, and every store before this tile
  else dma_wait_barrier<16>();              // X and W blocks 0-1 of step 0
  if constexpr (kBiasStart) {
    // register 4q + j of block (fb, tb) holds feature wf*128 + fb*32 + 8q + 4*(lane/32) + j
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 b = *reinterpret_cast<const f32x4*>(svec + wf * 128 + fb * 32 + q * 8 + (lane >> 5) * 4);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[fb][tb][4 * q + j] = b[j];
      }
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) accepi::to_agpr<F>(acc[fb][tb]);
  }
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) xf[0][tb][kk] = frag(0, true, b_row0 + tb * 32, kk);
#pragma unroll
  for (int jb = 0; jb < 2; ++jb)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) wfr[0][jb][kk] = frag(0, false, a_row0 + jb * 32, kk);
  dma_wait_barrier<40>();  // every wave holds its step-0 fragments: X buffer 0 and W blocks 0-1 are free
  dma_w(1, 2); dma_w(1, 3); dma_x(2, 0);
  dma_wait_barrier<16>();  // W blocks 2-3 of step 0 and X half 0 of step 1

#pragma clang loop unroll(disable)
  for (int s = 0; s < steps; s += 2) {
    step(std::integral_constant<int, 0>{}, s);
    step(std::integral_constant<int, 1>{}, s + 1);
  }
  dma_wait_barrier<0>();  // every DMA has landed and every fragment read is done before LDS is reused
}

// One output tile (token tile tt, feature tile ft): mainloop and epilogue. head_loaded: the
// previous tile issued this tile's head DMAs. next_tt >= 0 names the workgroup's next tile;
// returns whether this tile issued that tile's head DMAs.
template <uint32_t F, bool kDma>
__device__ __forceinline__ bool gemm_tile(const GemmArgs& a, int tt, int ft, uint8_t* smem, float* svec, int* slot,
                                          bool head_loaded = false, int next_tt = -1, int next_ft = 0) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wf = wave >> 1, wt = wave & 1;
  const int f0 = ft * BF, t0 = tt * BT;
  const int K = a.K;

  // the epilogue's per-feature / per-token vectors, fetched now and kept in LDS (a row scale
  // that late_vectors stores after the mainloop is also fetched there: it is computed from
  // its loads at once, and the waits for them would delay the prologue's DMAs)
  constexpr bool kLateLoad = kDma && late_vectors<F>() && (F & epi::kRscale) != 0;
  accepi::VecPrefetch vp;
  if constexpr (has_vectors<F>() && !kLateLoad) vp.load<F>(a.ep, t0, f0, a.M, a.N);

  // On the LDS-DMA path a static configuration's accumulators start from its residual and
  // bias (seed_residual) or, without a residual, from its bias (in mainloop_dma): the MFMAs
  // accumulate the product on top and the epilogue adds neither. Every other tile starts from
  // zero.
  constexpr bool kSeed = kDma && (accepi::seeds_residual<F>() || accepi::seeds_bias<F>());
  f32x16 acc[4][4];
  if constexpr (kDma && accepi::seeds_residual<F>()) {
    // seed_residual reads the bias; the other vectors are stored here too, while nothing is
    // in flight (after the prologue's DMAs a spilled vector value's reload would drain them)
    if constexpr (has_vectors<F>()) vp.store(svec, tid);
    accepi::seed_residual<F>(a, acc, smem, svec, t0, f0);
  } else if constexpr (kSeed) {
    // written in mainloop_dma
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  }

  bool next_head = false;
  int tid_e = tid;  // the epilogue's thread index
  if constexpr (kDma) {
    mainloop_dma<F, kSeed && !accepi::seeds_residual<F>()>(a, smem, svec, vp, acc, t0, f0, head_loaded);
    // An opaque copy of the thread index, taken before the next tile's DMAs: the epilogue's
    // lane constants then come from it, and the thread index itself (held in scratch across the
    // walk) is reloaded here, where nothing is in flight, not after the DMAs.
    if constexpr (prefetches_head<F>()) asm volatile("" : "+v"(tid_e));
    if constexpr (late_vectors<F>()) {
      if constexpr (kLateLoad) vp.load<F>(a.ep, t0, f0, a.M, a.N);
      vp.store(svec, tid_e);  // nothing is in flight here
      lds_barrier();
    }
    if constexpr (prefetches_head<F>()) {
      // the mainloop's last barrier has retired every read of both stages
      if (next_tt >= 0 && ((F & epi::kXent) == 0 || a.ep.y == nullptr)) {
        DmaPlan(a, smem, next_tt * BT, next_ft * BF, tid_e).head();
        next_head = true;
      }
    }
  } else {
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
    if constexpr (has_vectors<F>()) vp.store(svec, tid);
    __syncthreads();
    read_frags(0, 0, fa[0], fb_[0]);

  #pragma clang loop unroll(disable)
    for (int s = 0; s < steps; ++s) kstep(s);
    __syncthreads();  // every wave's last fragment reads are done before LDS is reused
  }

  if constexpr ((F & epi::kStatic) != 0) {
    // Epilogue on the accumulators in place; the mainloop's LDS buffers (128 KB) stage
    // the finished values for coalesced stores, or stage 1 alone (64 KB) when the next tile's
    // head may be landing in stage 0. (The stage-1 offset is passed opaque: as a constant it
    // would be folded into every LDS access and overflow their 16-bit offset fields, costing an
    // address add per access.)
    constexpr bool kStage1 = kDma && prefetches_head<F>() && (F & epi::kXent) == 0;
    uint8_t* lds = smem;
    if constexpr (kStage1) {
      int off = kBuf;
      asm volatile("" : "+s"(off));
      lds += off;
    }
    acc_epilogue<F, kSeed, kStage1 ? kBuf : 2 * kBuf>(a, acc, lds, svec, t0, f0, ft, slot, tid_e);
  } else {
    // Any other op list: the fp32 tile is staged through LDS in two 128-token passes
    // (128 KB each; pass p takes the accumulators of the waves with wt == p) and the
    // row-layout chain reads every choice at run time.
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
  return next_head;
}

template <uint32_t F, bool kDma>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_t256_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * 2 * kTileBytes];  // [stage][W, X]
  __shared__ __attribute__((aligned(16))) float svec[4 * 256];               // epilogue vectors
  __shared__ int slot[2];

  // A static configuration fixes quant() at compile time: the instances without FP8 rows carry
  // no code for them (which also leaves the compiler fewer values to keep across the walk).
  const epi::Cfg<F> cfg{a.ep};
  if (cfg.quant()) {
    int tt, ft;
    if (a.ep.tickets) {
      // FP8 row scales need every feature tile of a token block: hand out tiles in
      // row-block-major ticket order so no block waits on a tile that is not running.
      const int ticket = draw_ticket(a.ep.ws, a.tiles_t * a.tiles_f, slot);
      tt = ticket / a.tiles_f;
      ft = ticket - tt * a.tiles_f;
      if (tt >= a.tiles_t) return;  // a workspace that was not zero-filled: touch nothing
    } else {
      tile_coords(blockIdx.x, a.tiles_t, a.tiles_f, tt, ft);
    }
    gemm_tile<F, kDma>(a, tt, ft, smem, svec, slot);
    return;
  }
  // Resident workgroups walk the tiles: workgroup b takes tile ids b, b + grid, ... (the same
  // XCD each time, in the XCD-aware order), so a tile's first loads are issued while the
  // previous tile's stores are still in flight, and no workgroup launch sits between tiles.
  const int tiles = a.tiles_t * a.tiles_f;
  bool head = false;  // this tile's head DMAs were issued by the previous one
#pragma clang loop unroll(disable)
  for (int id = blockIdx.x; id < tiles; id += gridDim.x) {
    // the previous tile's epilogue is done with LDS (its global stores may still be in flight)
    if (id != (int)blockIdx.x) lds_barrier();
    int tt, ft, ntt = -1, nft = 0;
    tile_coords(id, a.tiles_t, a.tiles_f, tt, ft);
    if constexpr (kDma && prefetches_head<F>())
      if (id + (int)gridDim.x < tiles) tile_coords(id + gridDim.x, a.tiles_t, a.tiles_f, ntt, nft);
    const bool issued = gemm_tile<F, kDma>(a, tt, ft, smem, svec, slot, head, ntt, nft);
    if constexpr (kDma && prefetches_head<F>()) head = issued;
  }
}

// Epilogue configurations with an instance of their own (the op sets of the fused QKV
// projection, with and without RoPE, MLP-up, out-projection, gate/up, FP8 gate/up, gate/up
// after a deferred RMSNorm, and the LM head with cross-entropy statistics); any other op list
// runs the generic instance, which reads its choices at run time.
constexpr uint32_t kCfgBiasGeluErf = epi::config(epi::kBias, ACT_GELU_ERF, FUSEDOPS_BF16);
constexpr uint32_t kCfgBiasSplit = epi::config(epi::kBias | epi::kSplit, ACT_NONE, FUSEDOPS_BF16);
constexpr uint32_t kCfgResidualRms = epi::config(epi::kZ | epi::kAux | epi::kPart | epi::kGamma, ACT_NONE,
                                                 FUSEDOPS_BF16);
constexpr uint32_t kCfgSwiglu = epi::config(0, ACT_SWIGLU, FUSEDOPS_BF16);
constexpr uint32_t kCfgSwigluFp8 = epi::config(epi::kQuant, ACT_SWIGLU, FUSEDOPS_F8E4M3);
constexpr uint32_t kCfgRscaleSwiglu = epi::config(epi::kRscale, ACT_SWIGLU, FUSEDOPS_BF16);
constexpr uint32_t kCfgXent = epi::config(epi::kXent, ACT_NONE, FUSEDOPS_BF16);
constexpr uint32_t kCfgBiasSplitRope = epi::config(epi::kBias | epi::kSplit | epi::kRope, ACT_NONE, FUSEDOPS_BF16);

// The RoPE instance reads the table at column (local feature mod d): d must divide the tile.
bool rope_fits(const EpiParams& e) {
  return e.rope_d <= 128 && BF % e.rope_d == 0 && e.rope_ld * 4 * BT < (int64_t(1) << 31);
}

template <bool kDma>
const void* t256_kernel_for(const EpiParams& e) {
  switch (epi::config_of(e)) {
    case kCfgBiasGeluErf: return reinterpret_cast<const void*>(&gemm_bf16_t256_kernel<kCfgBiasGeluErf, kDma>);
    case kCfgBiasSplit: return reinterpret_cast<const void*>(&gemm_bf16_t256_kernel<kCfgBiasSplit, kDma>);
    case kCfgResidualRms: return reinterpret_cast<const void*>(&gemm_bf16_t256_kernel<kCfgResidualRms, kDma>);
    case kCfgSwiglu: return reinterpret_cast<const void*>(&gemm_bf16_t256_kernel<kCfgSwiglu, kDma>);
    case kCfgSwigluFp8: return reinterpret_cast<const void*>(&gemm_bf16_t256_kernel<kCfgSwigluFp8, kDma>);
    case kCfgRscaleSwiglu: return reinterpret_cast<const void*>(&gemm_bf16_t256_kernel<kCfgRscaleSwiglu, kDma>);
    case kCfgXent: return reinterpret_cast<const void*>(&gemm_bf16_t256_kernel<kCfgXent, kDma>);
    case kCfgBiasSplitRope:
      if (rope_fits(e)) return reinterpret_cast<const void*>(&gemm_bf16_t256_kernel<kCfgBiasSplitRope, kDma>);
      return reinterpret_cast<const void*>(&gemm_bf16_t256_kernel<0, kDma>);
    default: return reinterpret_cast<const void*>(&gemm_bf16_t256_kernel<0, kDma>);
  }
}

// The LDS-DMA mainloop needs whole W tiles and an even number of K steps.
bool use_dma(const GemmArgs& a) { return a.N % BF == 0 && a.K % (2 * BK) == 0; }

const void* kernel_for(const GemmArgs& a) {
  return use_dma(a) ? t256_kernel_for<true>(a.ep) : t256_kernel_for<false>(a.ep);
}

}  // namespace

hipError_t launch_gemm_bf16_t256(GemmArgs a, hipStream_t stream) {
  a.tiles_t = (a.M + BT - 1) / BT;
  a.tiles_f = (a.N + BF - 1) / BF;
  const int tiles = a.tiles_t * a.tiles_f;
  // without FP8 row scales, one resident workgroup per CU walks the tiles (a multiple of the 8
  // XCDs, so each workgroup stays on one XCD's tile range)
  int grid = tiles;
  if (!a.ep.quant) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus >= 8 &&
        tiles > cus)
      grid = cus / 8 * 8;
  }
  void* args[] = {&a};
  return hipLaunchKernel(kernel_for(a), dim3(grid), dim3(kThreads), args, 0, stream);
}

int gemm_bf16_t256_tile_t() { return BT; }
int gemm_bf16_t256_tile_f() { return BF; }

const void* gemm_bf16_t256_symbol(const GemmArgs& a) { return kernel_for(a); }

}  // namespace fusedops
