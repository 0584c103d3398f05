// The epilogue of the fused linear layer, shared by every GEMM kernel.
//
// The contraction is computed transposed, D[f][t] = sum_k W[f][k] X[t][k], with
// v_mfma_f32_32x32x{16 bf16, 2 f32}. In that instruction's D layout lane l holds
// column t = l % 32 and rows f = 8 (r / 4) + 4 (l / 32) + (r % 4) of register r: one
// lane owns one token and runs of four consecutive features, so a wave can drop a
// block into a token-major LDS tile with 16-byte writes.
//
// The finished fp32 accumulator tile is staged in LDS (token-major; 16-byte chunk c of
// row r sits at chunk position c ^ (r & 15), which keeps both the 16-byte writes from
// the MFMA layout and the row reads below free of bank conflicts). All 256 threads then
// run the epilogue chain in a row layout: a thread owns 8 consecutive features of one
// token, so SwiGLU pairs (2j, 2j+1) sit in the same thread's registers, residual loads
// and all stores are 16-byte accesses that are contiguous along a row, and a 128-column
// row partial is a reduction over 16 adjacent lanes.
//
// Op order ([Epilogue] §模式A Epilogue 1 / 2, §模式B, §仿射量化与尾声的五步):
// bias, residual add, store-aux, sum-of-squares partials, column scale, row scale,
// activation, then FP8 per-row quantisation or a plain / split store.
#pragma once

#include "common.h"

namespace fusedops {

enum Act { ACT_NONE = 0, ACT_GELU_ERF = 1, ACT_GELU_TANH = 2, ACT_SWIGLU = 3 };

struct EpiParams {
  const void* bias;       int bias_dtype;
  const void* z;          int64_t ldz;     int z_dtype;
  void* aux;              int64_t ld_aux;  int aux_dtype;
  float* partials;        int64_t ldp;
  const void* gamma;      int gamma_dtype;
  const float* rscale;
  const float* dq_row;    // FP8 inputs: activation scale per row of X (null: 1)
  const float* dq_col;    // FP8 inputs: weight scale per output channel (null: 1)
  const float* rms_p;     // ROW_RMS: row partials of the previous layer (null: none)
  int64_t rms_ldp;        //   their row stride
  int rms_T;              //   partials per row
  int rms_n;              //   width the partials cover
  float rms_eps;
  const int* xent_labels; // XENT: label per row (null: no cross-entropy statistics)
  float* xent_stats;      //   (max, sum-exp) per row and 64-column chunk
  int64_t xent_ld;        //   row stride of the statistics
  float* xent_tgt;        //   y at the label, per row
  const float* rope_cs;   // RoPE: per-row cos / sin table (null: no rotation)
  int64_t rope_ld;        //   its row stride in floats
  int rope_d;             //   head width (pair index i = (column mod d) / 2)
  int rope_cols;          //   columns [0, rope_cols) rotated
  int act;
  int quant;              // FP8 per-row quantised writeback
  float* scales;
  uint32_t* ws;           // rendezvous workspace (quant only)
  uint32_t ws_bytes;      //   its size
  int ws_bs;              //   words per 32-token block record
  int ws_s;               //   absmax slots per token (one per 64-feature column tile)
  int ws_g;               //   column-tile groups per control record
  int ws_gs;              //   group absmax slots per token
  int tickets;            // hand out tiles by ticket (the grid exceeds what is resident at once)
  void* y;                int64_t ldy;     int y_dtype;
  int n_split;            int64_t split_w; int64_t ldv;
  void* yv0;              void* yv1;       void* yv2;
};

// The row scale of token t: ROW_SCALE's r[t], or ROW_RMS's r computed from the token's row
// partials with the formula of the finalize kernel, 1 / sqrt(sum / width + eps).
// The partials are loaded 16 at a time with all loads in flight before the first is added (a
// plain loop loaded, waited and added one at a time: 16 round trips per tile at width 2048, each
// wait also covering every other load and store in flight); they are added in index order.
__device__ inline float row_scale_of(const EpiParams& e, int t) {
  if (e.rscale) return e.rscale[t];
  const float* p = e.rms_p + (int64_t)t * e.rms_ldp;
  const int T = e.rms_T;
  float s = 0.f;
  int i = 0;
  for (; i + 16 <= T; i += 16) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = p[i + j];
#pragma unroll
    for (int j = 0; j < 16; ++j) s += v[j];
  }
  for (; i < T; ++i) s += p[i];
  return 1.0f / sqrtf(s / (float)e.rms_n + e.rms_eps);
}

struct GemmArgs {
  const void* X; int64_t ldx;
  const void* W; int64_t ldw;
  int M, N, K;
  int tiles_t, tiles_f;   // token tiles x feature tiles
  EpiParams ep;
};

namespace epi {

// Compile-time description of a kernel instance's epilogue. With kStatic set, the op set,
// activation and storage types are fixed at compile time; otherwise every choice is read
// from EpiParams at run time (the generic instance).
constexpr uint32_t kStatic = 1u << 31;
constexpr uint32_t kBias = 1u << 0, kZ = 1u << 1, kAux = 1u << 2, kPart = 1u << 3, kGamma = 1u << 4,
                   kRscale = 1u << 5, kQuant = 1u << 6, kSplit = 1u << 7;
// RoPE rotations (kRope) have an instance for the fused QKV projection (bias + split) when
// the head width divides the 256-feature tile; other RoPE op lists run the generic one
constexpr uint32_t kRope = 1u << 20;
constexpr uint32_t kXent = 1u << 21;
constexpr int kActShift = 8, kYShift = 10, kZShift = 12, kAuxShift = 14, kBiasShift = 16, kGammaShift = 18;

constexpr uint32_t config(uint32_t ops, int act, int y_dtype, int z_dtype = FUSEDOPS_BF16,
                          int aux_dtype = FUSEDOPS_BF16, int bias_dtype = FUSEDOPS_BF16,
                          int gamma_dtype = FUSEDOPS_BF16) {
  return kStatic | ops | ((uint32_t)act << kActShift) | ((uint32_t)y_dtype << kYShift) |
         ((uint32_t)z_dtype << kZShift) | ((uint32_t)aux_dtype << kAuxShift) |
         ((uint32_t)bias_dtype << kBiasShift) | ((uint32_t)gamma_dtype << kGammaShift);
}

// The configuration a call's parameters describe (always with kStatic set).
__host__ __device__ inline uint32_t config_of(const EpiParams& e) {
  uint32_t ops = 0;
  if (e.bias) ops |= kBias;
  if (e.z) ops |= kZ;
  if (e.aux) ops |= kAux;
  if (e.partials) ops |= kPart;
  if (e.gamma) ops |= kGamma;
  if (e.rscale || e.rms_p) ops |= kRscale;
  if (e.quant) ops |= kQuant;
  if (e.n_split) ops |= kSplit;
  if (e.rope_cs) ops |= kRope;
  if (e.xent_labels) ops |= kXent;
  return config(ops, e.act, e.y_dtype, e.z ? e.z_dtype : FUSEDOPS_BF16, e.aux ? e.aux_dtype : FUSEDOPS_BF16,
                e.bias ? e.bias_dtype : FUSEDOPS_BF16, e.gamma ? e.gamma_dtype : FUSEDOPS_BF16);
}

template <uint32_t F>
struct Cfg {
  static constexpr bool S = (F & kStatic) != 0;
  const EpiParams& e;
  __device__ bool bias() const { if constexpr (S) return F & kBias; else return e.bias != nullptr; }
  __device__ bool z() const { if constexpr (S) return F & kZ; else return e.z != nullptr; }
  __device__ bool aux() const { if constexpr (S) return F & kAux; else return e.aux != nullptr; }
  __device__ bool part() const { if constexpr (S) return F & kPart; else return e.partials != nullptr; }
  __device__ bool gamma() const { if constexpr (S) return F & kGamma; else return e.gamma != nullptr; }
  __device__ bool rscale() const { if constexpr (S) return F & kRscale; else return e.rscale || e.rms_p; }
  __device__ bool quant() const { if constexpr (S) return F & kQuant; else return e.quant != 0; }
  __device__ bool split() const { if constexpr (S) return F & kSplit; else return e.n_split != 0; }
  __device__ bool xent() const { if constexpr (S) return F & kXent; else return e.xent_labels != nullptr; }
  __device__ bool rope() const { if constexpr (S) return F & kRope; else return e.rope_cs != nullptr; }
  __device__ int act() const { if constexpr (S) return (F >> kActShift) & 3; else return e.act; }
  __device__ int y_dt() const { if constexpr (S) return (F >> kYShift) & 3; else return e.y_dtype; }
  __device__ int z_dt() const { if constexpr (S) return (F >> kZShift) & 3; else return e.z_dtype; }
  __device__ int aux_dt() const { if constexpr (S) return (F >> kAuxShift) & 3; else return e.aux_dtype; }
  __device__ int bias_dt() const { if constexpr (S) return (F >> kBiasShift) & 3; else return e.bias_dtype; }
  __device__ int gamma_dt() const { if constexpr (S) return (F >> kGammaShift) & 3; else return e.gamma_dtype; }
};

}  // namespace epi

constexpr int kEpiThreads = 256;

// ---------------------------------------------------------------------------
// FP8 row rendezvous
// ---------------------------------------------------------------------------
// Workspace layout (uint32 words):
//   [0]                error word: set to 1 if a wait ever hit its spin bound (never cleared here)
//   [1]                tile ticket counter (back at zero after every call)
//   [32 + BS b, ...)   record of the 32-token block b (tokens 32 b .. 32 b + 31), BS = ws_bs words:
//     control lines    32 (2 + G) words, one counter per 128-byte line, used by the row block
//                      of a tile whose first token is 32 b: line 0 counts arriving groups,
//                      line 1 is the release flag (a generation count: it goes up by one per
//                      call), line 2 + g counts the arrivals of column-tile group g
//                      (kGroupTiles tiles each; G = ws_g)
//     tile slots       S words per token (S = ws_s, a multiple of 4): word ft of token t holds
//                      the absmax of token t over the features of column tile ft
//     group slots      GS words per token (GS = ws_gs, a multiple of 4): word g of token t
//                      holds its absmax over column-tile group g
// The records depend on N only, so calls with the same N (and any M up to the size the
// workspace was made for) may share one. Each tile writes its own slots and the last tile
// to arrive in a group writes the group's slots; no two tiles touch the same word. Readers
// take only the words of the current call (a run's words past the valid count may hold
// another call's values). The arrival counters are reset by the tile that completes them,
// and the flag is only ever compared with the value a tile saw before arriving, so nothing
// needs clearing after a call: the workspace must be zero-filled once after allocation and
// then handed to every call unchanged.
//
// Memory ordering. Each XCD has its own L2; agent-scope release / acquire fences are
// L2-wide write-back / invalidate operations that would disturb every other tile on the XCD.
// The rendezvous avoids them: every word other tiles read is written and read with the
// agent-scope coherence policy (sc1, the policy of agent-scope atomic loads and stores),
// which makes the access at the device's coherence point. A tile's slot stores complete
// (s_waitcnt) before its thread 0 arrives; the flag is raised only after every arrival
// has been counted, and slots are read only after the raised flag was seen, so the reads
// return the published values.
// In C++ terms the atomics are relaxed, so the language model alone would not order the slot
// accesses; the ordering is the ISA's, the same properties the compiler's own agent-scope
// release and acquire sequences rest on. Release there is a write-back of dirty L2 lines,
// then a wait for every earlier memory operation, then the store: the write-back only serves
// data written with the default policy, and the slots are written with sc1, so what remains
// is the wait (s_waitcnt vmcnt(0) here). Acquire there is the load, a wait for it, then an
// invalidation of non-coherent cached lines: the slots are read with sc1 and never cached
// non-coherently, so what remains is that the slot loads are issued only after the flag's
// value has returned (the spin loop's exit depends on it). The flag itself is read before the
// tile arrives and that load is waited for, so the value it waits to see change cannot
// already include its own arrival.
constexpr uint32_t kSpinLimit = 1u << 22;
constexpr int kGroupTiles = 16;
constexpr int kPolicyCoherent = 16;  // sc1: agent-scope coherence policy of a buffer access

// Word offsets in the workspace: the record of token t's block, the control record of the row
// block starting at token t0 (a multiple of 32), token t's tile slots and its group slots.
__device__ __forceinline__ int64_t ws_block(const EpiParams& e, int t) { return 32 + (int64_t)(t >> 5) * e.ws_bs; }
__device__ __forceinline__ uint32_t* ws_ctl(const EpiParams& e, int t0) { return e.ws + ws_block(e, t0); }
__device__ __forceinline__ int64_t ws_slot_word(const EpiParams& e, int t) {
  return ws_block(e, t) + 32 * (2 + e.ws_g) + (t & 31) * e.ws_s;
}
__device__ __forceinline__ int64_t ws_gslot_word(const EpiParams& e, int t) {
  return ws_block(e, t) + 32 * (2 + e.ws_g) + 32 * e.ws_s + (t & 31) * e.ws_gs;
}

// Publish the absmax m of token t over column tile ft.
__device__ __forceinline__ void publish_row_amax(const EpiParams& e, int ft, int t, float m) {
  __hip_atomic_store(e.ws + ws_slot_word(e, t) + ft, __float_as_uint(m), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Maximum of the workspace words [w, w + count) of each of `nrows` rows (w = run(i) for row i,
// 16-byte aligned), read at the coherence point. ROWS rows (a power of two dividing the 256
// threads) share the workgroup, 256 / ROWS threads per row, each taking 16-byte runs with all
// of its loads in flight; words of a run past `count` are ignored. Every thread of row `row`
// gets the row's maximum (absmax values: non-negative floats order like their bit patterns).
template <int ROWS, typename Run>
__device__ __forceinline__ uint32_t coherent_row_max(const EpiParams& e, Run&& run, int count, int nrows, int& row) {
  constexpr int TPR = 256 / ROWS;
  static_assert(TPR >= 1 && TPR <= 64 && 256 % ROWS == 0, "threads per row");
  row = threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(e.ws, e.ws_bytes);
  uint32_t m = 0;
  if (row < nrows) {
    const uint32_t w = (uint32_t)run(row);
    // batches of 8 runs: all loads in flight before the first is used
    constexpr int kBatch = 8;
    for (int j0 = part * 4; j0 < count; j0 += kBatch * TPR * 4) {
      u32x4 v[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int j = j0 + b * TPR * 4;
        v[b] = j < count ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (w + j) * 4u, 0,
                                                                                           kPolicyCoherent))
                         : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = j0 + b * TPR * 4 + i < count ? max(m, v[b][i]) : m;
    }
  }
#pragma unroll
  for (int o = 1; o < TPR; o <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, kWave));
  return m;
}

// Take the next tile ticket (thread 0 draws, the block shares it through LDS). The block
// that draws the last ticket resets the counter: every other ticket was already drawn.
__device__ __forceinline__ int draw_ticket(uint32_t* ws, int total, int* lds_slot) {
  if (threadIdx.x == 0) {
    uint32_t t = __hip_atomic_fetch_add(ws + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((int)t == total - 1)
      __hip_atomic_store(ws + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *lds_slot = (int)t;
  }
  __syncthreads();
  int t = *lds_slot;
  __syncthreads();
  return t;
}

// Arrive at the row block starting at token t0 as column tile ft of `need` (this tile's slots
// for its rows are published), wait until every column tile of the block has arrived, and return in out[i]
// the absmax of token t0 + i over all of them (i < nrows; ROWS as for coherent_row_max).
// Arrivals are counted in groups of kGroupTiles tiles on separate lines, so no counter sees
// more than a few dozen atomics; the tile that completes the last group raises the block's
// flag. With 128 or more rows per tile the last tile to arrive in a group first folds the
// group's slots into the group slot of each token, and every tile then reads only the group
// slots (a few words per token instead of one per column tile): for 256-row tiles that is
// 4 KB of reads per tile instead of 64 KB, at the price of two more round trips to the
// coherence point on the last arrival's path, which is why few-row tiles (decode, where the
// one rendezvous is the kernel's tail) read the tile slots directly. The wait is bounded; on
// timeout the error word is set.
template <int ROWS>
__device__ __forceinline__ void rendezvous_row_amax(const EpiParams& e, int ft, int need, int t0, int nrows,
                                                    float* out, int* lds_slot) {
  constexpr int TPR = 256 / ROWS;
  constexpr bool kTwoLevel = ROWS >= 128;
  __builtin_amdgcn_s_waitcnt(0);  // this thread's slot stores have completed
  __syncthreads();
  uint32_t* rec = ws_ctl(e, t0);
  uint32_t* flag = rec + 32;
  const int g = ft / kGroupTiles, groups = (need + kGroupTiles - 1) / kGroupTiles;
  const int in_group = min(kGroupTiles, need - g * kGroupTiles);
  auto arrive_block = [&](uint32_t gen) {
    if (__hip_atomic_fetch_add(rec, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)groups - 1) {
      __hip_atomic_store(rec, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(flag, gen + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  uint32_t gen = 0;
  if (threadIdx.x == 0) {
    gen = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // The flag must be read before this tile arrives: relaxed accesses to different words may
    // be performed in either order, and a read performed after the last arrival could return
    // the raised value (the tile would then wait for a generation that never comes). Waiting
    // for the load's data before issuing the arrival orders them.
    __builtin_amdgcn_s_waitcnt(0);
    uint32_t* gc = rec + 64 + 32 * g;
    const bool last = __hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                      (uint32_t)in_group - 1;
    if (last) __hip_atomic_store(gc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if constexpr (kTwoLevel) *lds_slot = last ? 1 : 0;
    else if (last) arrive_block(gen);  // the group's arrival, straight away
  }
  if constexpr (kTwoLevel) {
    __syncthreads();
    if (*lds_slot) {
      // every tile of the group has published: its maxima per token go to the group slot,
      // then the group arrives at the block
      int row;
      const uint32_t m = coherent_row_max<ROWS>(
          e, [&](int i) { return ws_slot_word(e, t0 + i) + g * kGroupTiles; }, in_group, nrows, row);
      if (row < nrows && threadIdx.x % TPR == 0)
        __hip_atomic_store(e.ws + ws_gslot_word(e, t0 + row) + g, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);  // the group slot stores have completed
      __syncthreads();
      if (threadIdx.x == 0) arrive_block(gen);
    }
  }
  if (threadIdx.x == 0) {
    uint32_t it = 0;
    while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gen) {
      __builtin_amdgcn_s_sleep(1);
      if (++it > kSpinLimit) {
        __hip_atomic_store(e.ws, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
  int row;
  uint32_t m;
  if constexpr (kTwoLevel)
    m = coherent_row_max<ROWS>(e, [&](int i) { return ws_gslot_word(e, t0 + i); }, groups, nrows, row);
  else
    m = coherent_row_max<ROWS>(e, [&](int i) { return ws_slot_word(e, t0 + i); }, need, nrows, row);
  if (row < nrows && threadIdx.x % TPR == 0) out[row] = __uint_as_float(m);
}

// ---------------------------------------------------------------------------
// staged tile
// ---------------------------------------------------------------------------

// Float offset of element (r, c) of a token-major fp32 tile with COLS columns
// (c a multiple of 4 for 16-byte accesses).
template <int COLS>
__device__ __forceinline__ int tile_off(int r, int c) {
  static_assert(COLS % 64 == 0, "rows must span at least 16 chunks");
  return r * COLS + ((((c >> 2) ^ (r & 15))) << 2) + (c & 3);
}

// Write one 32 x 32 MFMA D block (features f_loc.., tokens r_loc..) into the tile.
template <int COLS>
__device__ __forceinline__ void stage_block(float* tile, const f32x16& d, int f_loc, int r_loc) {
  const int lane = threadIdx.x & 63;
  const int r = r_loc + (lane & 31);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = f_loc + q * 8 + (lane >> 5) * 4;
    *reinterpret_cast<f32x4*>(tile + tile_off<COLS>(r, c)) = f32x4{d[q * 4], d[q * 4 + 1], d[q * 4 + 2], d[q * 4 + 3]};
  }
}

// ---------------------------------------------------------------------------
// 8-wide loads / stores with a runtime dtype
// ---------------------------------------------------------------------------

__device__ __forceinline__ void load8(const void* base, int dtype, int64_t idx, float (&o)[8]) {
  if (dtype == FUSEDOPS_F32) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx);
    const f32x4 b = *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx + 4);
    o[0] = a[0]; o[1] = a[1]; o[2] = a[2]; o[3] = a[3];
    o[4] = b[0]; o[5] = b[1]; o[6] = b[2]; o[7] = b[3];
  } else {
    const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + idx);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (dtype == FUSEDOPS_BF16) {
        o[2 * j] = __uint_as_float(v[j] << 16);
        o[2 * j + 1] = __uint_as_float(v[j] & 0xFFFF0000u);
      } else {
        o[2 * j] = f16_bits_to_f32(v[j] & 0xFFFF);
        o[2 * j + 1] = f16_bits_to_f32(v[j] >> 16);
      }
    }
  }
}

// Outputs are written once and not read again by this kernel: nontemporal stores, so they do
// not stay in L2 as dirty lines that later operand loads would have to evict.
__device__ __forceinline__ void store8(void* base, int dtype, int64_t idx, const float (&v)[8]) {
  if (dtype == FUSEDOPS_F32) {
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx));
    __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]},
                                reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx + 4));
  } else {
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = dtype == FUSEDOPS_BF16 ? pack_bf16x2(v[2 * j], v[2 * j + 1]) : pack_f16x2(v[2 * j], v[2 * j + 1]);
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + idx));
  }
}

// The last group of a row when N is not a multiple of 8: the first n (< 8) elements only; the
// others read as 0 and are not written.
__device__ __forceinline__ void load8_n(const void* base, int dtype, int64_t idx, int n, float (&o)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = i < n ? load1(base, dtype, idx + i) : 0.f;
}

__device__ __forceinline__ void store1(void* base, int dtype, int64_t idx, float v) {
  if (dtype == FUSEDOPS_F32) static_cast<float*>(base)[idx] = v;
  else if (dtype == FUSEDOPS_BF16) static_cast<uint16_t*>(base)[idx] = (uint16_t)f32_to_bf16_bits(v);
  else static_cast<uint16_t*>(base)[idx] = (uint16_t)f32_to_f16_bits(v);
}

template <int W>
__device__ __forceinline__ void store_n(void* base, int dtype, int64_t idx, int n, const float (&v)[W]) {
#pragma unroll
  for (int i = 0; i < W; ++i)
    if (i < n) store1(base, dtype, idx + i, v[i]);
}

// ---------------------------------------------------------------------------
// the chain over a staged tile
// ---------------------------------------------------------------------------

enum EpiMode {
  EPI_STORE = 0,  // chain + side outputs + main store
  EPI_AMAX = 1,   // chain + side outputs + per-row absmax published to the workspace
  EPI_QUANT = 2,  // chain (no side outputs) + FP8 quantisation with the final row scales
};

// Run the epilogue over rows [0, nrows) of a staged tile whose element (r, c) is the
// accumulator of token t0 + r and feature f0 + c. NSRC tiles (each ROWS_ALLOC x COLS) are
// summed element-wise first, in order (used to merge split-K partial sums). Every thread
// of the block must call this (it contains wave-wide shuffles but no barriers).
template <int COLS, int NSRC, int ROWS_ALLOC, uint32_t F = 0>
__device__ __forceinline__ void epilogue_pass(const GemmArgs& a, const float* tile, int t0,
                                              int nrows, int f0, int ft, const float* amax_rows, int mode) {
  constexpr int TPR = COLS / 8;            // threads per row
  constexpr int RPI = kEpiThreads / TPR;   // rows per iteration
  static_assert(TPR <= 64 && 64 % TPR == 0, "a row's threads must sit in one wave");
  const EpiParams& e = a.ep;
  const epi::Cfg<F> cfg{e};  // F = 0: every choice read at run time
  const int M = a.M, N = a.N;
  const int tid = threadIdx.x;
  const int g = tid % TPR;
  const int c = g * 8;
  const int f = f0 + c;
  const bool f_ok = f < N;
  // columns of this thread's group inside the output: 8, or fewer in the last group of a row
  // whose width is not a multiple of 8 (the rest read as 0 and are neither stored nor reduced)
  const int nv = f_ok ? min(8, N - f) : 0;
  const bool full = nv == 8;
  const int act = cfg.act();
  const bool swiglu = act == ACT_SWIGLU;
  const bool side = mode != EPI_QUANT;
  const int zdt = cfg.z_dt(), adt = cfg.aux_dt(), ydt = cfg.y_dt();
  const int zb = zdt == FUSEDOPS_F32 ? 4 : 2;
  const int ab = adt == FUSEDOPS_F32 ? 4 : 2;
  const int yb = ydt == FUSEDOPS_F32 ? 4 : (ydt == FUSEDOPS_F8E4M3 ? 1 : 2);

  // per-feature vectors, loaded once per pass
  float bias[8], gam[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { bias[i] = 0.f; gam[i] = 1.f; }
  if (cfg.bias() && f_ok) {
    if (full) load8(e.bias, cfg.bias_dt(), f, bias);
    else load8_n(e.bias, cfg.bias_dt(), f, nv, bias);
  }
  if (cfg.gamma() && f_ok) {
    if (full) load8(e.gamma, cfg.gamma_dt(), f, gam);
    else load8_n(e.gamma, cfg.gamma_dt(), f, nv, gam);
  }

  // When one iteration covers the whole tile (the few-token and fp32 kernels), the bound says so:
  // with a trip count the compiler cannot bound it strength-reduced the output addresses of every
  // optional output over several iterations, ~400 instructions ahead of the first barrier.
  const int r0 = tid / TPR;
  const int r_end = ROWS_ALLOC <= RPI ? min(nrows, r0 + 1) : nrows;
  for (int r = r0; r < r_end; r += RPI) {
    const int t = t0 + r;
    const bool t_ok = t < M;
    const bool ok = t_ok && f_ok;
    float v[8];
    {
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(tile + tile_off<COLS>(r, c));
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(tile + tile_off<COLS>(r, c + 4));
      v[0] = a0[0]; v[1] = a0[1]; v[2] = a0[2]; v[3] = a0[3];
      v[4] = a1[0]; v[5] = a1[1]; v[6] = a1[2]; v[7] = a1[3];
#pragma unroll
      for (int s = 1; s < NSRC; ++s) {
        const float* ts = tile + s * ROWS_ALLOC * COLS;
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(ts + tile_off<COLS>(r, c));
        const f32x4 b1 = *reinterpret_cast<const f32x4*>(ts + tile_off<COLS>(r, c + 4));
        v[0] += b0[0]; v[1] += b0[1]; v[2] += b0[2]; v[3] += b0[3];
        v[4] += b1[0]; v[5] += b1[1]; v[6] += b1[2]; v[7] += b1[3];
      }
    }
    // bias, residual
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] += bias[i];
    if (cfg.z() && ok) {
      float z[8];
      if (full) load8(static_cast<const char*>(e.z) + (int64_t)t * e.ldz * zb, zdt, f, z);
      else load8_n(static_cast<const char*>(e.z) + (int64_t)t * e.ldz * zb, zdt, f, nv, z);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] += z[i];
    }
    // store-aux (h1) and its row sum-of-squares partials over 128-column chunks
    if (side && cfg.aux() && ok) {
      char* arow = static_cast<char*>(e.aux) + (int64_t)t * e.ld_aux * ab;
      if (full) store8(arow, adt, f, v);
      else store_n<8>(arow, adt, f, nv, v);
    }
    if (COLS >= 128 && cfg.part()) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) s += v[i] * v[i];
      // 16 adjacent lanes = 128 columns; columns >= N hold exact zeros
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o, kWave);
      if (side && t_ok && (g & 15) == 0 && f_ok) e.partials[(int64_t)t * e.ldp + f / 128] = s;
    }
    // column scale, row scale
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= gam[i];
    if (cfg.rscale()) {
      const float rs = t_ok ? row_scale_of(e, t) : 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] *= rs;
    }
    // activation; SwiGLU leaves its 4 outputs in v[0..3]
    if (act == ACT_GELU_ERF) {
      // fp32 outputs keep fp32 relative accuracy in the negative tail; 16-bit and E4M3
      // outputs take the one-exp2 form, whose error is far below their rounding
      if (ydt == FUSEDOPS_F32) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = gelu_erf_precise_f32(v[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = gelu_erf_f32(v[i]);
      }
    } else if (act == ACT_GELU_TANH) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = gelu_tanh_f32(v[i]);
    } else if (swiglu) {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = silu_f32(v[2 * j]) * v[2 * j + 1];
#pragma unroll
      for (int j = 4; j < 8; ++j) v[j] = 0.f;
    }
    // RoPE on adjacent pairs: the thread's 8 columns lie in one head (d is a multiple of 8)
    if (cfg.rope() && ok && f < e.rope_cols) {
      const float* cs = e.rope_cs + (int64_t)t * e.rope_ld + (f % e.rope_d);
      const f32x4 c0 = *reinterpret_cast<const f32x4*>(cs);
      const f32x4 c1 = *reinterpret_cast<const f32x4*>(cs + 4);
      const float cv[4] = {c0[0], c0[2], c1[0], c1[2]}, sv[4] = {c0[1], c0[3], c1[1], c1[3]};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x0 = v[2 * j], x1 = v[2 * j + 1];
        v[2 * j] = x0 * cv[j] - x1 * sv[j];
        v[2 * j + 1] = x0 * sv[j] + x1 * cv[j];
      }
    }
    // cross-entropy statistics: (max, sum of e^(y - max)) of each 64-column chunk, merged over
    // the chunk's 8 threads, and y at the row's label (tile-local index selection)
    if (cfg.xent()) {
      constexpr float kLog2e = 1.4426950408889634f;
      float m = -INFINITY, sx = 0.f;
      if (ok) {
        m = v[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) m = i < nv ? fmaxf(m, v[i]) : m;   // columns past N left out
#pragma unroll
        for (int i = 0; i < 8; ++i) sx += i < nv ? __builtin_amdgcn_exp2f((v[i] - m) * kLog2e) : 0.f;
      }
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) {
        const float mo = __shfl_xor(m, o, kWave), so = __shfl_xor(sx, o, kWave);
        const float mn = fmaxf(m, mo);
        sx = mn == -INFINITY ? 0.f
                             : sx * __builtin_amdgcn_exp2f((m - mn) * kLog2e) + so * __builtin_amdgcn_exp2f((mo - mn) * kLog2e);
        m = mn;
      }
      if (ok && (g & 7) == 0) {
        float* st = e.xent_stats + (int64_t)t * e.xent_ld + 2 * (f / 64);
        st[0] = m;
        st[1] = sx;
      }
      if (ok) {
        const int o = e.xent_labels[t] - f;
        if (o >= 0 && o < nv) {   // labels at or past N mark ignored rows
          float val = v[0];
#pragma unroll
          for (int i = 1; i < 8; ++i) val = o == i ? v[i] : val;
          e.xent_tgt[t] = val;
        }
      }
    }
    const int fo = swiglu ? f / 2 : f;  // output column of v[0]

    if (mode == EPI_STORE) {
      if (!ok || (!e.y && !cfg.split())) continue;  // no Y: the logits are not stored (XENT)
      if (swiglu) {
        char* yrow = static_cast<char*>(e.y) + (int64_t)t * e.ldy * yb;
        if (full) {
          store4(yrow, ydt, fo, f32x4{v[0], v[1], v[2], v[3]});
        } else {
          const float o4[4] = {v[0], v[1], v[2], v[3]};
          store_n<4>(yrow, ydt, fo, nv / 2, o4);   // N is even with SwiGLU
        }
      } else if (cfg.split()) {
        const int seg = (int)(f / e.split_w);
        void* base = seg == 0 ? e.yv0 : (seg == 1 ? e.yv1 : e.yv2);
        store8(static_cast<char*>(base) + (int64_t)t * e.ldv * yb, ydt, f - (int64_t)seg * e.split_w, v);
      } else {
        char* yrow = static_cast<char*>(e.y) + (int64_t)t * e.ldy * yb;
        if (full) store8(yrow, ydt, f, v);
        else store_n<8>(yrow, ydt, f, nv, v);
      }
    } else if (mode == EPI_AMAX) {
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
      if (!f_ok) m = 0.f;
#pragma unroll
      for (int o = 1; o < TPR; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
      if (g == 0 && t_ok) publish_row_amax(e, ft, t, m);
    } else {
      if (!t_ok) continue;
      const float amax = amax_rows[r];
      const float s = __fdiv_rn(amax, 448.0f);  // IEEE division: s = fl32(a / 448)
      const Fp8RowFactor fac = fp8_row_factor(s);
      if (f0 == 0 && g == 0) e.scales[t] = s;
      if (!f_ok) continue;
      float q[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = fminf(fmaxf((v[i] * fac.pre) * fac.inv, -448.f), 448.f);
      uint8_t* yrow = static_cast<uint8_t*>(e.y) + (int64_t)t * e.ldy;
      const u32x2 w = {pack_e4m3x2(q[0], q[1]) | (pack_e4m3x2(q[2], q[3]) << 16),
                       pack_e4m3x2(q[4], q[5]) | (pack_e4m3x2(q[6], q[7]) << 16)};
      if (full) {
        if (swiglu) *reinterpret_cast<uint32_t*>(yrow + fo) = w[0];
        else *reinterpret_cast<u32x2*>(yrow + fo) = w;
      } else {
        // the row's last group: one byte per valid code
        const int nq = swiglu ? nv / 2 : nv;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (i < nq) yrow[fo + i] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
      }
    }
  }
}

// Drive the epilogue for one tile held in registers, staging PASSES token slices through
// LDS. `stage(pass, tile)` must write this pass's accumulator blocks into the tile (it is
// called by every wave; waves that own nothing in a pass write nothing). The tile origin
// is (t0, f0) and each pass covers ROWS tokens (`nrows_total` valid tokens in the tile).
// For FP8 row quantisation the chain runs twice: first to publish the row absmax, then,
// after every column tile of the token block has done so, to quantise.
template <int COLS, int NSRC, int ROWS, int PASSES, uint32_t F = 0, typename StageFn>
__device__ __forceinline__ void run_staged_epilogue(const GemmArgs& a, float* tile, int t0, int f0,
                                                    int nrows_total, int ft, int* lds_slot,
                                                    float* lds_amax, StageFn&& stage) {
  const EpiParams& e = a.ep;
  const epi::Cfg<F> cfg{e};
  const int rounds = cfg.quant() ? 2 : 1;
  // rolled loops: one inlined copy of the chain serves every round and pass
#pragma clang loop unroll(disable)
  for (int round = 0; round < rounds; ++round) {
    if (round == 1) {
      // every column tile of the row block publishes: this tile's rows' maxima, once
      rendezvous_row_amax<ROWS * PASSES>(e, ft, a.tiles_f, t0, nrows_total, lds_amax, lds_slot);
    }
    const int mode = cfg.quant() ? (round == 0 ? EPI_AMAX : EPI_QUANT) : EPI_STORE;
#pragma clang loop unroll(disable)
    for (int p = 0; p < PASSES; ++p) {
      const int rows = min(ROWS, nrows_total - p * ROWS);
      if (rows <= 0) break;
      __syncthreads();
      stage(p, tile);
      __syncthreads();
      epilogue_pass<COLS, NSRC, ROWS, F>(a, tile, t0 + p * ROWS, rows, f0, ft, lds_amax + p * ROWS, mode);
    }
  }
}

}  // namespace fusedops
