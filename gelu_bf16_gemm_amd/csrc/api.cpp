// C ABI of libfusedops.so (see include/fusedops.h): argument validation, op-list
// canonicalisation, kernel selection and launch on the caller's stream.
//
// Every check runs on the host before anything is enqueued, so a validation error
// leaves the stream untouched. No exception crosses the ABI.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/fusedops.h"
#include "epilogue.h"
#include "kernels.h"

using namespace fusedops;

namespace {

int dtype_size(int32_t dt) {
  switch (dt) {
    case FUSEDOPS_F32: return 4;
    case FUSEDOPS_BF16: return 2;
    case FUSEDOPS_F16: return 2;
    case FUSEDOPS_F8E4M3: return 1;
    default: return 0;
  }
}

bool valid_dtype(int32_t dt) { return dt >= FUSEDOPS_F32 && dt <= FUSEDOPS_F8E4M3; }
bool float_dtype(int32_t dt) { return dt == FUSEDOPS_F32 || dt == FUSEDOPS_BF16 || dt == FUSEDOPS_F16; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte extent of a row-major rows x cols tensor with leading dimension ld.
struct Span {
  uintptr_t lo = 0, hi = 0;  // [lo, hi)
  bool valid = false;
};
Span span2d(const void* p, int64_t rows, int64_t cols, int64_t ld, int es) {
  Span s;
  if (!p || rows <= 0 || cols <= 0) return s;
  s.lo = reinterpret_cast<uintptr_t>(p);
  s.hi = s.lo + (uintptr_t)(((rows - 1) * ld + cols) * es);
  s.valid = true;
  return s;
}
bool overlap(const Span& a, const Span& b) { return a.valid && b.valid && a.lo < b.hi && b.lo < a.hi; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Parsed epilogue op list.
struct OpList {
  const fusedops_op* by_kind[16] = {};
  int act = ACT_NONE;
  bool quant = false;
};

int32_t parse_ops(const fusedops_op* ops, int32_t n_ops, OpList& out) {
  if (n_ops < 0 || (n_ops > 0 && !ops)) return FUSEDOPS_ERR_INVALID_ARG;
  int last = 0;
  int n_act = 0;
  for (int i = 0; i < n_ops; ++i) {
    const fusedops_op& op = ops[i];
    if (op.kind < FUSEDOPS_OP_RESIDUAL_ADD || op.kind > FUSEDOPS_OP_XENT) return FUSEDOPS_ERR_INVALID_ARG;
    if (op.kind <= last) return FUSEDOPS_ERR_INVALID_ARG;  // increasing kind order, each kind once
    if (op.reserved != 0 && op.kind != FUSEDOPS_OP_ROW_RMS) return FUSEDOPS_ERR_INVALID_ARG;
    last = op.kind;
    out.by_kind[op.kind] = &op;
    if (op.kind == FUSEDOPS_OP_GELU_ERF || op.kind == FUSEDOPS_OP_GELU_TANH || op.kind == FUSEDOPS_OP_SWIGLU)
      ++n_act;
  }
  if (n_act > 1) return FUSEDOPS_ERR_INVALID_ARG;
  if (out.by_kind[FUSEDOPS_OP_GELU_ERF]) out.act = ACT_GELU_ERF;
  if (out.by_kind[FUSEDOPS_OP_GELU_TANH]) out.act = ACT_GELU_TANH;
  if (out.by_kind[FUSEDOPS_OP_SWIGLU]) out.act = ACT_SWIGLU;
  out.quant = out.by_kind[FUSEDOPS_OP_QUANT_FP8_ROW] != nullptr;
  return FUSEDOPS_OK;
}

// FP8 workspace: a 32-word header, then one record per block of 32 tokens (the finest token
// tile): a control record with one 128-byte line per counter (groups of 16 column tiles of
// the finest feature tile, 64 features), then per token one absmax slot per column tile and
// one per group, each run rounded up to a multiple of 4 slots so it starts 16-byte aligned.
// A record's size depends on N only, so calls with the same N may share a workspace.
int64_t ws_slots_per_token(int64_t N) { return cdiv(cdiv(N, 64), 4) * 4; }
int64_t ws_groups(int64_t N) { return cdiv(cdiv(N, 64), 16); }
int64_t ws_group_slots_per_token(int64_t N) { return cdiv(ws_groups(N), 4) * 4; }
int64_t ws_block_words(int64_t N) {
  return 32 * (2 + ws_groups(N)) + 32 * ws_slots_per_token(N) + 32 * ws_group_slots_per_token(N);
}
size_t ws_bytes_for(int64_t M, int64_t N) {
  const int64_t words = 32 + cdiv(M, 32) * ws_block_words(N);
  return (size_t)(cdiv(words * 4, 256) * 256);
}

enum class Kernel { T256, SKINNY, F32, FP8 };

// Map a launch result to a status; with FUSEDOPS_VERBOSE set, name the refused launch on stderr.
int32_t launch_status(hipError_t err, const char* what) {
  if (err == hipSuccess) return FUSEDOPS_OK;
  const char* v = std::getenv("FUSEDOPS_VERBOSE");
  if (v && *v && *v != '0') std::fprintf(stderr, "fusedops: launch of %s failed: %s (%d)\n", what, hipGetErrorName(err), (int)err);
  return FUSEDOPS_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int32_t fusedops_abi_version(void) { return FUSEDOPS_ABI_VERSION; }
int32_t fusedops_partial_cols(void) { return FUSEDOPS_PARTIAL_COLS; }

const char* fusedops_status_string(int32_t status) {
  switch (status) {
    case FUSEDOPS_OK: return "ok";
    case FUSEDOPS_ERR_INVALID_ARG: return "invalid argument";
    case FUSEDOPS_ERR_UNSUPPORTED: return "unsupported configuration";
    case FUSEDOPS_ERR_MISALIGNED: return "misaligned pointer, leading dimension or width";
    case FUSEDOPS_ERR_WORKSPACE: return "workspace missing or too small";
    case FUSEDOPS_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

size_t fusedops_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, const fusedops_op* ops,
                                       int32_t n_ops) {
  (void)N;
  (void)K;
  OpList ol;
  if (M < 1 || parse_ops(ops, n_ops, ol) != FUSEDOPS_OK) return 0;
  return ol.quant ? ws_bytes_for(M, N) : 0;
}

// The fused linear call. With clear_ws (the allocation-free entry point, whose workspace is the
// library's shared device scratch) a quantised call first zeroes the scratch's counters on the
// stream, since the previous call may have used another N's layout.
static int32_t linear_call(const void* X, int64_t ldx, const void* W, int64_t ldw, const void* bias, int64_t M,
                           int64_t N, int64_t K, int32_t in_dtype, const fusedops_op* ops, int32_t n_ops, void* Y,
                           int64_t ldy, int32_t out_dtype, void* workspace, size_t workspace_bytes, void* stream,
                           bool clear_ws) {
  // ---- scalars and enums
  if (!X || !W) return FUSEDOPS_ERR_INVALID_ARG;
  if (M < 1 || N < 1 || K < 1) return FUSEDOPS_ERR_INVALID_ARG;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return FUSEDOPS_ERR_INVALID_ARG;
  if (in_dtype == FUSEDOPS_F16) return FUSEDOPS_ERR_UNSUPPORTED;
  if (M > (1 << 30) || N > (1 << 30) || K > (1 << 30)) return FUSEDOPS_ERR_UNSUPPORTED;
  OpList ol;
  if (int32_t st = parse_ops(ops, n_ops, ol)) return st;
  const fusedops_op* op_res = ol.by_kind[FUSEDOPS_OP_RESIDUAL_ADD];
  const fusedops_op* op_aux = ol.by_kind[FUSEDOPS_OP_STORE_AUX];
  const fusedops_op* op_par = ol.by_kind[FUSEDOPS_OP_ROWSUMSQ_PARTIAL];
  const fusedops_op* op_gam = ol.by_kind[FUSEDOPS_OP_COL_SCALE];
  const fusedops_op* op_row = ol.by_kind[FUSEDOPS_OP_ROW_SCALE];
  const fusedops_op* op_q = ol.by_kind[FUSEDOPS_OP_QUANT_FP8_ROW];
  const fusedops_op* op_split = ol.by_kind[FUSEDOPS_OP_SPLIT_COLS];
  const fusedops_op* op_dqr = ol.by_kind[FUSEDOPS_OP_DEQUANT_ROW];
  const fusedops_op* op_dqc = ol.by_kind[FUSEDOPS_OP_DEQUANT_COL];
  const fusedops_op* op_rope = ol.by_kind[FUSEDOPS_OP_ROPE];
  const fusedops_op* op_rms = ol.by_kind[FUSEDOPS_OP_ROW_RMS];
  const fusedops_op* op_xe = ol.by_kind[FUSEDOPS_OP_XENT];
  const int64_t xent_T = cdiv(N, FUSEDOPS_XENT_COLS);
  float rms_eps = 0.f;
  if (op_rms) std::memcpy(&rms_eps, &op_rms->reserved, sizeof(float));
  const int64_t rms_T = op_rms ? cdiv(op_rms->n_split, FUSEDOPS_PARTIAL_COLS) : 0;
  const bool fp8_in = in_dtype == FUSEDOPS_F8E4M3;
  const bool swiglu = ol.act == ACT_SWIGLU;
  const int64_t n_out = swiglu ? N / 2 : N;
  const int64_t T = cdiv(N, FUSEDOPS_PARTIAL_COLS);
  const int es_in = dtype_size(in_dtype);
  const int bias_dtype = fp8_in ? FUSEDOPS_BF16 : in_dtype;  // FP8 inputs take a bf16 bias

  // ---- output dtype rules
  if (ol.quant) {
    if (out_dtype != FUSEDOPS_F8E4M3) return FUSEDOPS_ERR_INVALID_ARG;
  } else if (!float_dtype(out_dtype)) {
    return FUSEDOPS_ERR_INVALID_ARG;
  }
  if (op_split) {
    if (Y) return FUSEDOPS_ERR_INVALID_ARG;
    if (swiglu || ol.quant) return FUSEDOPS_ERR_UNSUPPORTED;
    if (op_split->n_split != 2 && op_split->n_split != 3) return FUSEDOPS_ERR_INVALID_ARG;
    for (int i = 0; i < op_split->n_split; ++i)
      if (!op_split->out_v[i]) return FUSEDOPS_ERR_INVALID_ARG;
    if (N % op_split->n_split) return FUSEDOPS_ERR_INVALID_ARG;
  } else if (!Y && !op_xe) {
    return FUSEDOPS_ERR_INVALID_ARG;
  }
  const int es_out = dtype_size(out_dtype);

  // ---- per-op fields
  if (op_res && (!op_res->in || !float_dtype(op_res->dtype) || op_res->ld < N)) return FUSEDOPS_ERR_INVALID_ARG;
  if (op_aux && (!op_aux->out || !float_dtype(op_aux->dtype) || op_aux->ld < N)) return FUSEDOPS_ERR_INVALID_ARG;
  if (op_par && (!op_par->out || op_par->ld < T)) return FUSEDOPS_ERR_INVALID_ARG;
  if (op_gam && (!op_gam->in || !float_dtype(op_gam->dtype))) return FUSEDOPS_ERR_INVALID_ARG;
  if (op_row && !op_row->in) return FUSEDOPS_ERR_INVALID_ARG;
  if (op_q && !op_q->out) return FUSEDOPS_ERR_INVALID_ARG;
  if ((op_dqr || op_dqc) && !fp8_in) return FUSEDOPS_ERR_INVALID_ARG;  // scales of FP8 inputs only
  if ((op_dqr && !op_dqr->in) || (op_dqc && !op_dqc->in)) return FUSEDOPS_ERR_INVALID_ARG;
  if (op_xe) {
    if (!op_xe->in || !op_xe->out || !op_xe->out_v[0] || op_xe->ld < 2 * xent_T) return FUSEDOPS_ERR_INVALID_ARG;
    if (swiglu || ol.quant || op_split) return FUSEDOPS_ERR_INVALID_ARG;
  }
  if (op_rms) {
    if (op_row || !op_rms->in || op_rms->n_split < 1 || op_rms->ld < rms_T) return FUSEDOPS_ERR_INVALID_ARG;
    if (!(rms_eps > 0.f) || !std::isfinite(rms_eps)) return FUSEDOPS_ERR_INVALID_ARG;
  }
  // RoPE: table of M rows, head width d a multiple of 8, rotated width a multiple of d
  const int64_t rope_cols = op_rope ? (op_split ? N - N / op_split->n_split : N) : 0;
  if (op_rope) {
    if (!op_rope->in || op_rope->dtype != FUSEDOPS_F32 || swiglu) return FUSEDOPS_ERR_INVALID_ARG;
    const int64_t d = op_rope->n_split;
    if (d < 8 || d % 8 || op_rope->ld < d || rope_cols % d) return FUSEDOPS_ERR_INVALID_ARG;
  }
  if (swiglu && (N % 2)) return FUSEDOPS_ERR_INVALID_ARG;
  if (ldx < K || ldw < K) return FUSEDOPS_ERR_INVALID_ARG;
  if (Y && ldy < n_out) return FUSEDOPS_ERR_INVALID_ARG;
  if (op_split && op_split->ld < N / op_split->n_split) return FUSEDOPS_ERR_INVALID_ARG;

  // ---- alignment: 16-byte bases and rows; K and N granularity
  const int k_gran = 16 / es_in;
  if (K % k_gran) return FUSEDOPS_ERR_MISALIGNED;
  if (!aligned(X, 16) || !aligned(W, 16) || (ldx * es_in) % 16 || (ldw * es_in) % 16) return FUSEDOPS_ERR_MISALIGNED;
  if (bias && !aligned(bias, 16)) return FUSEDOPS_ERR_MISALIGNED;
  if (Y && (!aligned(Y, 16) || (ldy * es_out) % 16)) return FUSEDOPS_ERR_MISALIGNED;
  if (op_res && (!aligned(op_res->in, 16) || (op_res->ld * dtype_size(op_res->dtype)) % 16)) return FUSEDOPS_ERR_MISALIGNED;
  if (op_aux && (!aligned(op_aux->out, 16) || (op_aux->ld * dtype_size(op_aux->dtype)) % 16)) return FUSEDOPS_ERR_MISALIGNED;
  if (op_par && !aligned(op_par->out, 4)) return FUSEDOPS_ERR_MISALIGNED;
  if (op_gam && !aligned(op_gam->in, 16)) return FUSEDOPS_ERR_MISALIGNED;
  if (op_row && !aligned(op_row->in, 4)) return FUSEDOPS_ERR_MISALIGNED;
  if (op_q && !aligned(op_q->out, 4)) return FUSEDOPS_ERR_MISALIGNED;
  if ((op_dqr && !aligned(op_dqr->in, 4)) || (op_dqc && !aligned(op_dqc->in, 4))) return FUSEDOPS_ERR_MISALIGNED;
  if (op_rope && (!aligned(op_rope->in, 16) || op_rope->ld % 4)) return FUSEDOPS_ERR_MISALIGNED;
  if (op_rms && !aligned(op_rms->in, 4)) return FUSEDOPS_ERR_MISALIGNED;
  if (op_xe && (!aligned(op_xe->in, 4) || !aligned(op_xe->out, 4) || !aligned(op_xe->out_v[0], 4)))
    return FUSEDOPS_ERR_MISALIGNED;
  if (op_split) {
    if ((N / op_split->n_split) % 8) return FUSEDOPS_ERR_MISALIGNED;
    if ((op_split->ld * es_out) % 16) return FUSEDOPS_ERR_MISALIGNED;
    for (int i = 0; i < op_split->n_split; ++i)
      if (!aligned(op_split->out_v[i], 16)) return FUSEDOPS_ERR_MISALIGNED;
  }

  // ---- aliasing: outputs may not overlap inputs or each other, except Y == z exactly
  constexpr int kInSpans = 11;
  Span in_spans[kInSpans] = {
      span2d(X, M, K, ldx, es_in), span2d(W, N, K, ldw, es_in), span2d(bias, 1, N, N, dtype_size(bias_dtype)),
      op_res ? span2d(op_res->in, M, N, op_res->ld, dtype_size(op_res->dtype)) : Span{},
      op_gam ? span2d(op_gam->in, 1, N, N, dtype_size(op_gam->dtype)) : Span{},
      op_row ? span2d(op_row->in, 1, M, M, 4) : Span{},
      op_dqr ? span2d(op_dqr->in, 1, M, M, 4) : Span{},
      op_dqc ? span2d(op_dqc->in, 1, N, N, 4) : Span{},
      op_rope ? span2d(op_rope->in, M, op_rope->n_split, op_rope->ld, 4) : Span{},
      op_rms ? span2d(op_rms->in, M, rms_T, op_rms->ld, 4) : Span{},
      op_xe ? span2d(op_xe->in, 1, M, M, 4) : Span{}};
  Span out_spans[10];
  int n_out_spans = 0;
  if (Y) out_spans[n_out_spans++] = span2d(Y, M, n_out, ldy, es_out);
  if (op_split)
    for (int i = 0; i < op_split->n_split; ++i)
      out_spans[n_out_spans++] = span2d(op_split->out_v[i], M, N / op_split->n_split, op_split->ld, es_out);
  if (op_aux) out_spans[n_out_spans++] = span2d(op_aux->out, M, N, op_aux->ld, dtype_size(op_aux->dtype));
  if (op_par) out_spans[n_out_spans++] = span2d(op_par->out, M, T, op_par->ld, 4);
  if (op_q) out_spans[n_out_spans++] = span2d(op_q->out, 1, M, M, 4);
  if (op_xe) {
    out_spans[n_out_spans++] = span2d(op_xe->out, M, 2 * xent_T, op_xe->ld, 4);
    out_spans[n_out_spans++] = span2d(op_xe->out_v[0], 1, M, M, 4);
  }
  const bool y_is_z = Y && op_res && Y == op_res->in && ldy == op_res->ld && out_dtype == op_res->dtype &&
                      !swiglu;
  for (int o = 0; o < n_out_spans; ++o) {
    for (int i = 0; i < kInSpans; ++i) {
      if (!overlap(out_spans[o], in_spans[i])) continue;
      if (y_is_z && o == 0 && i == 3) continue;
      return FUSEDOPS_ERR_INVALID_ARG;
    }
    for (int p = o + 1; p < n_out_spans; ++p)
      if (overlap(out_spans[o], out_spans[p])) return FUSEDOPS_ERR_INVALID_ARG;
  }

  // ---- workspace
  if (ol.quant) {
    if (ws_bytes_for(M, N) > 0xFFFFFFFFu) return FUSEDOPS_ERR_UNSUPPORTED;  // the kernels address it in 32 bits
    if (!workspace || workspace_bytes < ws_bytes_for(M, N) || !aligned(workspace, 16)) return FUSEDOPS_ERR_WORKSPACE;
    const Span sw{reinterpret_cast<uintptr_t>(workspace),
                  reinterpret_cast<uintptr_t>(workspace) + workspace_bytes, true};
    for (int o = 0; o < n_out_spans; ++o)
      if (overlap(sw, out_spans[o])) return FUSEDOPS_ERR_INVALID_ARG;
    for (int i = 0; i < kInSpans; ++i)
      if (overlap(sw, in_spans[i])) return FUSEDOPS_ERR_INVALID_ARG;
  }

  // ---- kernel selection
  Kernel kern;
  if (in_dtype == FUSEDOPS_F32) {
    kern = Kernel::F32;
  } else if (fp8_in) {
    kern = Kernel::FP8;
  } else {
    const int64_t big_tiles = cdiv(M, 256) * cdiv(N, 256);
    kern = (M <= 128 && !op_par && big_tiles < 256) ? Kernel::SKINNY : Kernel::T256;
  }
  const bool big = kern == Kernel::T256 || kern == Kernel::FP8;  // the 256 x 256 tile kernels
  const int tile_rows = big ? 256 : (kern == Kernel::SKINNY ? 64 : 128);  // at most, for the fp32 kernel
  const int tile_tok = big ? 256 : 32;                                     // few-token and fp32 kernels
  // 32-bit buffer offsets cover one tile's rows (operands, and the residual rows the
  // 256 x 256 kernel copies into LDS)
  if (((int64_t)(tile_rows - 1) * ldw + K) * es_in >= (int64_t(1) << 31) ||
      ((int64_t)(tile_tok - 1) * ldx + K) * es_in >= (int64_t(1) << 31))
    return FUSEDOPS_ERR_UNSUPPORTED;
  if (op_res && big &&
      ((int64_t)(tile_tok - 1) * op_res->ld + 256) * dtype_size(op_res->dtype) >= (int64_t(1) << 31))
    return FUSEDOPS_ERR_UNSUPPORTED;

  GemmArgs a;
  std::memset(&a, 0, sizeof(a));
  a.X = X; a.ldx = ldx; a.W = W; a.ldw = ldw;
  a.M = (int)M; a.N = (int)N; a.K = (int)K;
  EpiParams& e = a.ep;
  e.bias = bias; e.bias_dtype = bias_dtype;
  if (op_dqr) e.dq_row = static_cast<const float*>(op_dqr->in);
  if (op_dqc) e.dq_col = static_cast<const float*>(op_dqc->in);
  if (op_xe) {
    e.xent_labels = static_cast<const int*>(op_xe->in);
    e.xent_stats = static_cast<float*>(op_xe->out);
    e.xent_ld = op_xe->ld;
    e.xent_tgt = static_cast<float*>(op_xe->out_v[0]);
  }
  if (op_rms) {
    e.rms_p = static_cast<const float*>(op_rms->in);
    e.rms_ldp = op_rms->ld;
    e.rms_T = (int)rms_T;
    e.rms_n = (int)op_rms->n_split;
    e.rms_eps = rms_eps;
  }
  if (op_rope) {
    e.rope_cs = static_cast<const float*>(op_rope->in);
    e.rope_ld = op_rope->ld;
    e.rope_d = (int)op_rope->n_split;
    e.rope_cols = (int)rope_cols;
  }
  if (op_res) { e.z = op_res->in; e.ldz = op_res->ld; e.z_dtype = op_res->dtype; }
  if (op_aux) { e.aux = op_aux->out; e.ld_aux = op_aux->ld; e.aux_dtype = op_aux->dtype; }
  if (op_par) { e.partials = static_cast<float*>(op_par->out); e.ldp = op_par->ld; }
  if (op_gam) { e.gamma = op_gam->in; e.gamma_dtype = op_gam->dtype; }
  if (op_row) e.rscale = static_cast<const float*>(op_row->in);
  e.act = ol.act;
  e.quant = ol.quant ? 1 : 0;
  if (op_q) {
    e.scales = static_cast<float*>(op_q->out);
    e.ws = static_cast<uint32_t*>(workspace);
    e.ws_bytes = (uint32_t)ws_bytes_for(M, N);
    e.ws_bs = (int)ws_block_words(N);
    e.ws_s = (int)ws_slots_per_token(N);
    e.ws_g = (int)ws_groups(N);
    e.ws_gs = (int)ws_group_slots_per_token(N);
  }
  e.y = Y; e.ldy = ldy; e.y_dtype = out_dtype;
  if (op_split) {
    e.n_split = op_split->n_split;
    e.split_w = N / op_split->n_split;
    e.ldv = op_split->ld;
    e.yv0 = op_split->out_v[0];
    e.yv1 = op_split->out_v[1];
    e.yv2 = op_split->n_split > 2 ? op_split->out_v[2] : nullptr;
  }

  // The FP8 row rendezvous needs every column tile of a token block to be able to run
  // at the same time: check the device can hold that many workgroups at once.
  if (ol.quant) {
    const int tile_f = kern == Kernel::T256 ? gemm_bf16_t256_tile_f()
                       : kern == Kernel::FP8 ? gemm_fp8_t256_tile_f()
                       : kern == Kernel::SKINNY ? gemm_bf16_skinny_tile_f() : gemm_f32_tile_f(a);
    const void* sym = kern == Kernel::T256 ? gemm_bf16_t256_symbol(a)
                      : kern == Kernel::FP8 ? gemm_fp8_t256_symbol(a.ep)
                      : kern == Kernel::SKINNY ? gemm_bf16_skinny_symbol(a.ep) : gemm_f32_symbol(a);
    const int threads = kern == Kernel::SKINNY ? gemm_bf16_skinny_threads()
                        : kern == Kernel::F32 ? gemm_f32_threads() : 256;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, sym, threads, 0) != hipSuccess)
      return launch_status(hipErrorInvalidValue, "occupancy query");
    if (cdiv(N, tile_f) > (int64_t)cus * per_cu) return FUSEDOPS_ERR_UNSUPPORTED;
    // Tiles are handed out in row-block-major ticket order only when the grid does not fit
    // on the device at once; otherwise every tile is resident and any order is safe.
    a.ep.tickets = cdiv(M, tile_tok) * cdiv(N, tile_f) > (int64_t)cus * per_cu ? 1 : 0;
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (clear_ws && ol.quant) {
    if (int32_t st = launch_status(launch_clear_rendezvous(workspace, cdiv(M, 32), (int)(32 * (2 + ws_groups(N))),
                                                           ws_block_words(N), s),
                                   "clear_rendezvous"))
      return st;
  }
  switch (kern) {
    case Kernel::T256: return launch_status(launch_gemm_bf16_t256(a, s), "gemm_bf16_t256");
    case Kernel::SKINNY: return launch_status(launch_gemm_bf16_skinny(a, s), "gemm_bf16_skinny");
    case Kernel::FP8: return launch_status(launch_gemm_fp8_t256(a, s), "gemm_fp8_t256");
    default: return launch_status(launch_gemm_f32(a, s), "gemm_f32");
  }
}

int32_t fusedops_rendezvous_error(void* workspace, int32_t clear, int32_t* error, void* stream) {
  if (!error) return FUSEDOPS_ERR_INVALID_ARG;
  if (!workspace) {
    // the no-allocation entry point's scratch on the current device
    if (hipError_t e = noalloc_scratch(&workspace)) return launch_status(e, "no-allocation scratch lookup");
  }
  if (!aligned(workspace, 16)) return FUSEDOPS_ERR_MISALIGNED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t word = 0;
  if (hipMemcpyAsync(&word, workspace, sizeof(word), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return launch_status(hipErrorInvalidValue, "rendezvous error read");
  if (clear && word != 0) {
    const uint32_t zero = 0;
    if (hipMemcpyAsync(workspace, &zero, sizeof(zero), hipMemcpyHostToDevice, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return launch_status(hipErrorInvalidValue, "rendezvous error clear");
  }
  *error = word != 0 ? 1 : 0;
  return FUSEDOPS_OK;
}

int32_t fusedops_linear_epilogue(const void* X, int64_t ldx, const void* W, int64_t ldw,
                                 const void* bias, int64_t M, int64_t N, int64_t K,
                                 int32_t in_dtype, const fusedops_op* ops, int32_t n_ops, void* Y,
                                 int64_t ldy, int32_t out_dtype, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return linear_call(X, ldx, W, ldw, bias, M, N, K, in_dtype, ops, n_ops, Y, ldy, out_dtype, workspace,
                     workspace_bytes, stream, false);
}

int32_t fusedops_linear_epilogue_noalloc(const void* X, int64_t ldx, const void* W, int64_t ldw,
                                         const void* bias, int64_t M, int64_t N, int64_t K, int32_t in_dtype,
                                         const fusedops_op* ops, int32_t n_ops, void* Y, int64_t ldy,
                                         int32_t out_dtype, void* stream) {
  // The scratch is only needed (and only looked up) for quantised op lists; a size beyond it is
  // reported as a workspace error before anything is enqueued.
  OpList ol;
  if (parse_ops(ops, n_ops, ol) != FUSEDOPS_OK || !ol.quant)
    return linear_call(X, ldx, W, ldw, bias, M, N, K, in_dtype, ops, n_ops, Y, ldy, out_dtype, nullptr, 0,
                       stream, false);
  if (M >= 1 && N >= 1 && ws_bytes_for(M, N) > FUSEDOPS_NOALLOC_SCRATCH_BYTES) return FUSEDOPS_ERR_WORKSPACE;
  void* scratch = nullptr;
  if (hipError_t e = noalloc_scratch(&scratch)) return launch_status(e, "no-allocation scratch lookup");
  return linear_call(X, ldx, W, ldw, bias, M, N, K, in_dtype, ops, n_ops, Y, ldy, out_dtype, scratch,
                     FUSEDOPS_NOALLOC_SCRATCH_BYTES, stream, true);
}

int32_t fusedops_layernorm_gelu(const void* x, int64_t ldx, void* y, int64_t ldy, int64_t rows,
                                int64_t cols, int32_t io_dtype, int32_t out_dtype, const void* gamma,
                                const void* beta, int32_t param_dtype, float eps, int32_t gelu_form,
                                void* stream) {
  if (!x || !y) return FUSEDOPS_ERR_INVALID_ARG;
  if (rows < 1 || cols < 1) return FUSEDOPS_ERR_INVALID_ARG;
  if (!valid_dtype(io_dtype) || !valid_dtype(out_dtype)) return FUSEDOPS_ERR_INVALID_ARG;
  if (!float_dtype(io_dtype) || !float_dtype(out_dtype)) return FUSEDOPS_ERR_UNSUPPORTED;
  if ((gamma || beta) && !valid_dtype(param_dtype)) return FUSEDOPS_ERR_INVALID_ARG;
  if ((gamma || beta) && !float_dtype(param_dtype)) return FUSEDOPS_ERR_UNSUPPORTED;
  if (!(eps > 0.f) || !std::isfinite(eps)) return FUSEDOPS_ERR_INVALID_ARG;
  if (gelu_form < FUSEDOPS_GELU_NONE || gelu_form > FUSEDOPS_GELU_ERF) return FUSEDOPS_ERR_INVALID_ARG;
  if (ldx < cols || ldy < cols) return FUSEDOPS_ERR_INVALID_ARG;
  if (cols > FUSEDOPS_LN_MAX_COLS) return FUSEDOPS_ERR_UNSUPPORTED;
  if (rows > ((int64_t)1 << 24) - 1) return FUSEDOPS_ERR_UNSUPPORTED;  // grid size bound
  const int es_in = dtype_size(io_dtype), es_out = dtype_size(out_dtype);
  const int gran = 16 / es_in;
  if (cols % gran) return FUSEDOPS_ERR_MISALIGNED;
  if (!aligned(x, 16) || !aligned(y, 16) || (ldx * es_in) % 16 || (ldy * es_out) % 16) return FUSEDOPS_ERR_MISALIGNED;
  if ((gamma && !aligned(gamma, 16)) || (beta && !aligned(beta, 16))) return FUSEDOPS_ERR_MISALIGNED;
  const Span sx = span2d(x, rows, cols, ldx, es_in), sy = span2d(y, rows, cols, ldy, es_out);
  const int es_p = (gamma || beta) ? dtype_size(param_dtype) : 1;
  const Span sg = span2d(gamma, 1, cols, cols, es_p), sb = span2d(beta, 1, cols, cols, es_p);
  const bool inplace = x == y && ldx == ldy && io_dtype == out_dtype;
  if ((overlap(sy, sx) && !inplace) || overlap(sy, sg) || overlap(sy, sb)) return FUSEDOPS_ERR_INVALID_ARG;

  LnArgs a;
  a.x = x; a.ldx = ldx; a.y = y; a.ldy = ldy; a.rows = rows; a.cols = (int)cols;
  a.io_dtype = io_dtype; a.out_dtype = out_dtype; a.gamma = gamma; a.beta = beta;
  a.param_dtype = param_dtype; a.eps = eps; a.gelu_form = gelu_form;
  return launch_status(launch_layernorm_gelu(a, static_cast<hipStream_t>(stream)), "layernorm_gelu");
}

int32_t fusedops_rmsnorm_finalize(const float* partials, int64_t ldp, int64_t M, int64_t T, int64_t N,
                                  float eps, float* r, const void* h, int64_t ldh, const void* gamma,
                                  void* y, int64_t ldy, int32_t dtype, void* stream) {
  if (!partials || !r) return FUSEDOPS_ERR_INVALID_ARG;
  if (M < 1 || T < 1 || N < 1 || ldp < T) return FUSEDOPS_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || !std::isfinite(eps)) return FUSEDOPS_ERR_INVALID_ARG;
  if ((h == nullptr) != (y == nullptr)) return FUSEDOPS_ERR_INVALID_ARG;
  if (M > ((int64_t)1 << 26) || T > (1 << 30)) return FUSEDOPS_ERR_UNSUPPORTED;  // grid size bound
  if (!aligned(partials, 4) || !aligned(r, 4)) return FUSEDOPS_ERR_MISALIGNED;
  const Span sp = span2d(partials, M, T, ldp, 4), sr = span2d(r, 1, M, M, 4);
  Span sh, sy, sg;
  if (h) {
    if (!valid_dtype(dtype)) return FUSEDOPS_ERR_INVALID_ARG;
    if (!float_dtype(dtype)) return FUSEDOPS_ERR_UNSUPPORTED;
    if (ldh < N || ldy < N) return FUSEDOPS_ERR_INVALID_ARG;
    const int es = dtype_size(dtype);
    if (N % (16 / es)) return FUSEDOPS_ERR_MISALIGNED;
    if (!aligned(h, 16) || !aligned(y, 16) || (ldh * es) % 16 || (ldy * es) % 16) return FUSEDOPS_ERR_MISALIGNED;
    if (gamma && !aligned(gamma, 16)) return FUSEDOPS_ERR_MISALIGNED;
    sh = span2d(h, M, N, ldh, es);
    sy = span2d(y, M, N, ldy, es);
    sg = span2d(gamma, 1, N, N, es);
    const bool inplace = h == y && ldh == ldy;
    if ((overlap(sy, sh) && !inplace) || overlap(sy, sg) || overlap(sy, sp)) return FUSEDOPS_ERR_INVALID_ARG;
  }
  if (overlap(sr, sp) || overlap(sr, sh) || overlap(sr, sy) || overlap(sr, sg)) return FUSEDOPS_ERR_INVALID_ARG;

  FinalizeArgs a;
  a.partials = partials; a.ldp = ldp; a.M = M; a.T = (int)T; a.N = N; a.eps = eps; a.r = r;
  a.h = h; a.ldh = ldh; a.gamma = gamma; a.y = y; a.ldy = ldy; a.dtype = dtype;
  return launch_status(launch_rmsnorm_finalize(a, static_cast<hipStream_t>(stream)), "rmsnorm_finalize");
}

int32_t fusedops_cross_entropy_finalize(const float* stats, int64_t ld, int64_t M, int64_t n_cols,
                                        const float* target, const int32_t* labels, float* loss,
                                        void* stream) {
  if (!stats || !target || !labels || !loss || M < 1 || n_cols < 1) return FUSEDOPS_ERR_INVALID_ARG;
  const int64_t T = cdiv(n_cols, FUSEDOPS_XENT_COLS);
  if (ld < 2 * T || M > (int64_t(1) << 31) || n_cols > (int64_t(1) << 31)) return FUSEDOPS_ERR_INVALID_ARG;
  if (!aligned(stats, 4) || !aligned(target, 4) || !aligned(labels, 4) || !aligned(loss, 4))
    return FUSEDOPS_ERR_MISALIGNED;
  const Span out = span2d(loss, 1, M, M, 4);
  if (overlap(out, span2d(stats, M, 2 * T, ld, 4)) || overlap(out, span2d(target, 1, M, M, 4)) ||
      overlap(out, span2d(labels, 1, M, M, 4)))
    return FUSEDOPS_ERR_INVALID_ARG;
  XentFinalizeArgs a{stats, ld, M, T, n_cols, target, labels, loss};
  return launch_status(launch_xent_finalize(a, static_cast<hipStream_t>(stream)), "xent_finalize");
}

}  // extern "C"
