/*
 * fusedops.h — C ABI of libfusedops.so, a fused linear layer with an
 * in-register epilogue and a LayerNorm+GELU row kernel for AMD MI355X (gfx950).
 *
 * Pages cited (by title; section / equation / table on that page):
 *   [Fusion]   Triton operator fusion: Linear+GELU, QKV projection, attention
 *              (aiqz.cc, triton-operator-fusion-linear-attention)
 *   [LN+GELU]  什么是算子融合？LayerNorm与GeLU融合如何为深度学习推理提速 (ipipp.com)
 *   [Epilogue] GEMM Epilogue 完全拆解:推理内核的最后一公里——累加器布局、融合归约与量化写回
 *              (pinghaoyang.com.cn, gemm-epilogue-fusion)
 *
 * General conventions (every entry point):
 *   - All tensor pointers are DEVICE pointers the caller allocated and owns.
 *     The library allocates and frees no device memory and keeps no global
 *     mutable state.
 *   - Matrices are row-major with an explicit leading dimension (elements
 *     between consecutive rows, >= the row width). Columns are contiguous.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *     on it and the call returns without synchronising.
 *   - Every function returns an int32 status (enum fusedops_status). Argument
 *     checks run on the host before anything is enqueued: a non-zero status
 *     other than FUSEDOPS_ERR_LAUNCH means nothing was enqueued. Faults during
 *     execution surface at the caller's next synchronisation on the stream.
 *     No C++ exception crosses this ABI.
 *   - Base pointers must be 16-byte aligned and row strides must keep rows
 *     16-byte aligned (leading dimension a multiple of 8 elements for 2-byte
 *     types, 4 for fp32, 16 for fp8), else FUSEDOPS_ERR_MISALIGNED.
 */
#ifndef FUSEDOPS_H
#define FUSEDOPS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FUSEDOPS_ABI_VERSION 5
/* Width of one RMSNorm row partial: p[m,t] covers columns [128 t, 128 t + 128). */
#define FUSEDOPS_PARTIAL_COLS 128
/* Column width of the cross-entropy chunk statistics (XENT). */
#define FUSEDOPS_XENT_COLS 64
/* Bytes of the per-GPU device array fusedops_linear_epilogue_noalloc keeps its FP8 rendezvous
 * state in (32 MiB: quantised calls up to about M N = 2^29, e.g. 16384 x 16384 on 16384 tokens). */
#define FUSEDOPS_NOALLOC_SCRATCH_BYTES (32u << 20)
/* Largest LayerNorm row supported by fusedops_layernorm_gelu (elements). */
#define FUSEDOPS_LN_MAX_COLS 16384

enum fusedops_status {
  FUSEDOPS_OK = 0,
  FUSEDOPS_ERR_INVALID_ARG = -1,  /* null required pointer, bad size, bad enum, bad op list, aliasing */
  FUSEDOPS_ERR_UNSUPPORTED = -2,  /* valid request that the library has no kernel for */
  FUSEDOPS_ERR_MISALIGNED = -3,   /* pointer / leading dimension / width alignment rule broken */
  FUSEDOPS_ERR_WORKSPACE = -4,    /* workspace missing or smaller than required */
  FUSEDOPS_ERR_LAUNCH = -5        /* the HIP runtime refused this call's kernel launch */
};

enum fusedops_dtype {
  FUSEDOPS_F32 = 0,
  FUSEDOPS_BF16 = 1,
  FUSEDOPS_F16 = 2,
  FUSEDOPS_F8E4M3 = 3   /* OCP E4M3FN: bias 7, max 448, S.1111.111 = NaN, no infinity */
};

/*
 * Epilogue op kinds. An op list is given in increasing kind value, each kind at
 * most once, and with at most one of GELU_ERF / GELU_TANH / SWIGLU. With
 * acc = X W^T the chain is, per output element (m, n) (the two DEQUANT kinds,
 * numbered after the others, act first):
 *
 *   acc = acc * sa[m] * sw[n]           DEQUANT_ROW (sa), DEQUANT_COL (sw); FP8 inputs only
 *                                       [Epilogue] §量化尾声的完整形态 (per-group scales, one group)
 *   h  = acc + b[n]                     bias, when `bias` != NULL   [Fusion] §Linear算子剖析 Y_{m,n}
 *   h1 = h + z[m,n]                     RESIDUAL_ADD                [Epilogue] §模式A, Epilogue 1
 *        STORE_AUX writes h1            (rank-2 tile store)         [Epilogue] §六类尾声原语 item 4
 *        ROWSUMSQ_PARTIAL writes p[m,t] = sum_{n in chunk t} h1^2   [Epilogue] §模式A partialRMS
 *   h2 = h1 * gamma[n]                  COL_SCALE                   [Epilogue] §模式A, Epilogue 1
 *   h3 = r[m] * h2                      ROW_SCALE, or ROW_RMS (r from row partials)  [Epilogue] §模式A, Epilogue 2
 *   y  = act(h3)                        GELU_ERF | GELU_TANH | SWIGLU
 *   y  = rotate(y)                      ROPE: adjacent column pairs   [Epilogue] §背景, §模式B
 *   XENT: per-row (max, sum-exp) of y over 64-column chunks + y at the label   [Epilogue] §模式C
 *   QUANT_FP8_ROW: Y is E4M3 codes with one fp32 scale per row    [Epilogue] §仿射量化与尾声的五步
 *   SPLIT_COLS: Y is written as n_split column blocks              [Fusion] §QKV投影融合
 *
 * Fields used per kind (others ignored):
 *   RESIDUAL_ADD      in = z (M x N, dtype = op.dtype in {BF16, F16, F32}), ld = row stride of z.
 *                     A row is read in 16-byte chunks: when N ends inside a chunk, the chunk's
 *                     elements past N (inside the row's 16-byte-aligned storage) are read and
 *                     ignored.
 *                     z may alias Y exactly (same pointer, same ld, same dtype) for an in-place
 *                     residual update; any other overlap with an output is not allowed.
 *   STORE_AUX         out = h1 (M x N, dtype = op.dtype in {BF16, F16, F32}), ld = row stride.
 *   ROWSUMSQ_PARTIAL  out = p (fp32, M x T with T = ceil(N / 128)), ld >= T. Sums use the fp32
 *                     value of h1 before any rounding.
 *   COL_SCALE         in = gamma (length N, dtype = op.dtype in {BF16, F16, F32}).
 *   ROW_SCALE         in = r (length M, fp32).
 *   GELU_ERF          y = 0.5 v (1 + erf(v / sqrt 2))               [Fusion] §GELU激活融合
 *   GELU_TANH         y = 0.5 v (1 + tanh(sqrt(2/pi)(v + 0.044715 v^3)))  [LN+GELU] §用Triton手写融合内核
 *   SWIGLU            y[m,j] = silu(v[m,2j]) * v[m,2j+1], silu(g) = g / (1 + e^-g); the output is
 *                     N/2 columns wide (compacted)                 [Epilogue] §模式B, §末尾布局调整
 *   QUANT_FP8_ROW     out = scales (fp32, length M). Requires out_dtype = F8E4M3. With a[m] the max
 *                     |y| over the whole output row (all column tiles), s[m] = fl32(a[m] / 448)
 *                     (IEEE division) and q = E4M3_RNE(clamp(y / s[m], +-448)); a row with a = 0
 *                     has s = 0 and all-zero codes. Dequantise as q * s[m]. Needs a workspace.
 *   SPLIT_COLS        out_v[0..n_split-1] = destination blocks, n_split in {2, 3}, ld = row stride
 *                     of each block. Block i receives output columns [i d, (i+1) d), d = N / n_split
 *                     (Q, K, V order for n_split = 3). Y must be NULL. Not combinable with SWIGLU.
 *   DEQUANT_ROW       in = sa (fp32, length M): the activation scale of each row of X, i.e. X holds
 *                     E4M3 codes of x / sa[m] (as QUANT_FP8_ROW writes them). Requires in_dtype =
 *                     F8E4M3. Absent: sa = 1.
 *   DEQUANT_COL       in = sw (fp32, length N): the weight scale of each output channel (row of W).
 *                     Requires in_dtype = F8E4M3. Absent: sw = 1.
 *   ROW_RMS           The row scale of the deferred RMSNorm, computed by the kernel itself: in =
 *                     partials (fp32, M x T, row stride ld >= T) as a previous call's ROWSUMSQ_PARTIAL
 *                     wrote them for rows of width d, n_split = d (T = ceil(d / 128)), reserved = the
 *                     bit pattern of eps (fp32, > 0). r[m] = 1 / sqrt(sum_t p[m,t] / d + eps), the
 *                     formula of fusedops_rmsnorm_finalize, then used as ROW_SCALE's r: the light
 *                     reduction runs inside this GEMM, overlapping its mainloop ([Epilogue] §模式A,
 *                     Fig. 4). Not combinable with ROW_SCALE.
 *   XENT              The stateful cross-entropy epilogue. in = labels (int32, length M; a label
 *                     outside [0, N) marks an ignored row), out = stats (fp32, M x 2T with T =
 *                     ceil(N / 64), row stride ld >= 2T): for chunk t of columns [64t, 64t + 64) the
 *                     pair m = max y, s = sum e^(y - m) over the chunk's columns < N; out_v[0] =
 *                     target (fp32, length M): y[m, label[m]] for rows with a valid label (others
 *                     untouched). y is the fp32 value before any rounding. Y may be NULL (logits not
 *                     stored). fusedops_cross_entropy_finalize merges the chunks. Not combinable with
 *                     SWIGLU, QUANT_FP8_ROW or SPLIT_COLS.
 *   ROPE              in = table (fp32, M rows, row stride ld >= d floats), n_split = d (head width,
 *                     a multiple of 8). Column pair (2j, 2j+1) of output row m, with i = (2j mod d)/2,
 *                     becomes (a c - b s, a s + b c) where c = table[m][2i], s = table[m][2i+1]: row
 *                     m holds the cos / sin of its token's rotation angles, so the caller gathers
 *                     the table by position. Rotated: every column, or with SPLIT_COLS every block
 *                     but the last (Q and K rotated, V not: [Epilogue] §用形状与步长把约定钉死); the
 *                     rotated width must be a multiple of d. Not combinable with SWIGLU.
 */
enum fusedops_op_kind {
  FUSEDOPS_OP_RESIDUAL_ADD = 1,
  FUSEDOPS_OP_STORE_AUX = 2,
  FUSEDOPS_OP_ROWSUMSQ_PARTIAL = 3,
  FUSEDOPS_OP_COL_SCALE = 4,
  FUSEDOPS_OP_ROW_SCALE = 5,
  FUSEDOPS_OP_GELU_ERF = 6,
  FUSEDOPS_OP_GELU_TANH = 7,
  FUSEDOPS_OP_SWIGLU = 8,
  FUSEDOPS_OP_QUANT_FP8_ROW = 9,
  FUSEDOPS_OP_SPLIT_COLS = 10,
  FUSEDOPS_OP_DEQUANT_ROW = 11,
  FUSEDOPS_OP_DEQUANT_COL = 12,
  FUSEDOPS_OP_ROPE = 13,
  FUSEDOPS_OP_ROW_RMS = 14,
  FUSEDOPS_OP_XENT = 15
};

enum fusedops_gelu_form {
  FUSEDOPS_GELU_NONE = 0,  /* plain LayerNorm (affine only) */
  FUSEDOPS_GELU_TANH = 1,
  FUSEDOPS_GELU_ERF = 2
};

/* One epilogue op (64 bytes). */
typedef struct fusedops_op {
  int32_t kind;       /* enum fusedops_op_kind */
  int32_t dtype;      /* enum fusedops_dtype of `in` / `out` where the kind takes one */
  const void* in;     /* device input (z, gamma, r) */
  void* out;          /* device output (h1, partials, fp8 scales) */
  int64_t ld;         /* row stride of a 2-D `in` / `out` / out_v block, in elements */
  void* out_v[3];     /* SPLIT_COLS destinations */
  int32_t n_split;    /* SPLIT_COLS block count */
  int32_t reserved;   /* 0, except ROW_RMS: the fp32 bit pattern of eps */
} fusedops_op;

/*
 * fusedops_linear_epilogue — Y = epilogue(X W^T + b) in one kernel.
 *
 * Defines: [Fusion] §Linear算子剖析 (Y_{m,n} = sum_k X_{m,k} W_{n,k} + b_n, W stored N x K with
 * row n = output neuron) and [Epilogue] §主循环与尾声 (the epilogue transforms each finished output
 * tile in registers before it is written back; see the op kinds above).
 *
 *   X      M x K, row stride ldx, dtype in_dtype: BF16, F32 (the fp32 path) or F8E4M3 (codes;
 *          the MFMA contraction runs on E4M3 operands with fp32 accumulation).
 *   W      N x K, row stride ldw, dtype in_dtype.
 *   bias   length N, dtype in_dtype (BF16 when in_dtype is F8E4M3), or NULL for no bias.
 *   M,N,K  >= 1. K must be a multiple of 8 (BF16), 4 (F32) or 16 (F8E4M3); N is any width (an
 *          output row may end inside a 16-byte chunk: its last elements are written singly, and
 *          nothing past the row's N_out columns is written). Leading dimensions still keep rows
 *          16-byte aligned.
 *   ops    n_ops ops in canonical order (n_ops = 0 allowed; ops may be NULL then).
 *   Y      M x N_out (N_out = N/2 with SWIGLU, else N), row stride ldy, dtype out_dtype
 *          in {BF16, F16, F32}, or F8E4M3 exactly when QUANT_FP8_ROW is present.
 *          Must be NULL when SPLIT_COLS is present; may be NULL when XENT is present.
 *   workspace / workspace_bytes
 *          Device scratch of at least fusedops_linear_workspace_bytes(...) bytes, 16-byte
 *          aligned (0 bytes when no op needs one; then workspace may be NULL). Only
 *          QUANT_FP8_ROW uses it: per 32-token block, arrival counters and a release flag
 *          for the row rendezvous, and per token one absmax slot per 64-feature column tile
 *          and one per group of 16 such tiles (about 4 * M * N / 64 bytes in all; a call
 *          needing more than 4 GiB returns UNSUPPORTED). Zero-fill it once after allocation,
 *          then pass it unchanged to every call: the library keeps state in it between calls
 *          (release flags count calls; slots hold the last call's maxima). Its layout depends
 *          on N only: calls with the same N and any M up to the one it was sized for may share
 *          it (say decode and prefill of one layer); calls with different N need workspaces of
 *          their own. Its first 32-bit word is an error word the kernels set to 1 if a row
 *          rendezvous ever gave up waiting (the quantised output of that call is then
 *          unreliable); fusedops_rendezvous_error reads and clears it, the kernels never clear
 *          it. Calls that may run concurrently (different streams) must not share a workspace.
 *   stream hipStream_t.
 * Outputs are written in fp32 -> out dtype with round-to-nearest-even.
 * Errors: INVALID_ARG, UNSUPPORTED, MISALIGNED, WORKSPACE, LAUNCH (see enum).
 */
int32_t fusedops_linear_epilogue(const void* X, int64_t ldx, const void* W, int64_t ldw,
                                 const void* bias, int64_t M, int64_t N, int64_t K,
                                 int32_t in_dtype, const fusedops_op* ops, int32_t n_ops,
                                 void* Y, int64_t ldy, int32_t out_dtype,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * fusedops_linear_epilogue_noalloc — fusedops_linear_epilogue for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, rules and results, without the workspace pair.
 *
 *   QUANT_FP8_ROW's rendezvous state (what the workspace holds in fusedops_linear_epilogue) lives
 *   in a library-owned device array of FUSEDOPS_NOALLOC_SCRATCH_BYTES that each GPU the library
 *   runs on holds from the first such call until the process ends. A quantised call first
 *   enqueues a small kernel that zeroes the array's counters, then the GEMM: two launches, no
 *   hipMalloc, hipFree or other allocating call. Op lists without QUANT_FP8_ROW use no array
 *   and launch exactly what fusedops_linear_epilogue launches.
 *   Every call on one GPU shares its array, so calls that may overlap in time on one GPU (on
 *   different streams) race and must not be issued; calls on one stream are ordered.
 *   A quantised call needing more than the array (fusedops_linear_workspace_bytes of the same
 *   call above FUSEDOPS_NOALLOC_SCRATCH_BYTES) returns FUSEDOPS_ERR_WORKSPACE, enqueuing
 *   nothing. The array's error word is sticky across calls: read it with
 *   fusedops_rendezvous_error(NULL, ...).
 * Errors: as fusedops_linear_epilogue; LAUNCH also when the array's address lookup fails.
 */
int32_t fusedops_linear_epilogue_noalloc(const void* X, int64_t ldx, const void* W, int64_t ldw,
                                         const void* bias, int64_t M, int64_t N, int64_t K,
                                         int32_t in_dtype, const fusedops_op* ops, int32_t n_ops,
                                         void* Y, int64_t ldy, int32_t out_dtype, void* stream);

/* Bytes of workspace the same call needs (0 if none). Returns 0 for an invalid op list too;
 * the call itself then reports the error. */
size_t fusedops_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, const fusedops_op* ops,
                                       int32_t n_ops);

/*
 * fusedops_rendezvous_error — whether an FP8 row rendezvous gave up waiting.
 *
 * A QUANT_FP8_ROW call merges each row's absmax across the column tiles of the row inside the
 * kernel ([Epilogue] §仿射量化与尾声的五步, step 1: per-tile maxima merged over the whole row);
 * a tile waits for the other tiles of its rows with a bounded wait, and on a timeout the kernel
 * still finishes but sets the workspace's error word. Kernel faults cannot be returned by the
 * asynchronous call itself, so this query reports them.
 *
 *   workspace  a workspace passed to fusedops_linear_epilogue (device pointer, 16-byte aligned),
 *              or NULL for the device array of fusedops_linear_epilogue_noalloc on the current GPU.
 *   clear      non-zero: reset the error word to 0 after reading it.
 *   error      host output: 0 if every rendezvous since the word was last cleared completed,
 *              1 if one gave up (the quantised output of that call is unreliable).
 *   stream     synchronised before the word is read (the query waits for the calls on it).
 * Allocates nothing. Errors: INVALID_ARG (null error), MISALIGNED, LAUNCH (a HIP copy,
 * synchronisation or the array's lookup failed; *error is then untouched).
 */
int32_t fusedops_rendezvous_error(void* workspace, int32_t clear, int32_t* error, void* stream);

/*
 * fusedops_layernorm_gelu — y = GELU(LayerNorm(x) * gamma + beta) per row.
 *
 * Defines: [LN+GELU] §用Triton手写融合内核: per row, mean mu = sum x / cols and biased variance
 * var = sum (x - mu)^2 / cols in fp32, rstd = 1 / sqrt(var + eps), y = (x - mu) rstd gamma + beta,
 * then GELU applied in registers and one store.
 *
 *   x      rows x cols, row stride ldx, dtype io_dtype in {F16, BF16, F32}.
 *   y      rows x cols, row stride ldy, dtype out_dtype in {F16, BF16, F32}. y may alias x exactly
 *          (same pointer and stride, same dtype); other overlap is not allowed.
 *   gamma, beta  length cols, dtype param_dtype in {F16, BF16, F32}; either may be NULL
 *          (gamma = 1, beta = 0).
 *   rows >= 1; 1 <= cols <= FUSEDOPS_LN_MAX_COLS (else UNSUPPORTED); cols a multiple of 8
 *          (2-byte types) or 4 (F32) — padding lanes are masked out of the statistics.
 *   eps    > 0 and finite.  gelu_form in enum fusedops_gelu_form.
 */
int32_t fusedops_layernorm_gelu(const void* x, int64_t ldx, void* y, int64_t ldy, int64_t rows,
                                int64_t cols, int32_t io_dtype, int32_t out_dtype,
                                const void* gamma, const void* beta, int32_t param_dtype, float eps,
                                int32_t gelu_form, void* stream);

/*
 * fusedops_rmsnorm_finalize — the small aux reduction that turns per-tile row partials into the
 * per-row RMSNorm scale, optionally applying it.
 *
 * Defines: [Epilogue] §模式A (the auxiliary kernel sums each row's partials, then takes the root
 * and the reciprocal: r = 1 / sqrt(reduce(r̂) + eps), with reduce read as the mean over N).
 *
 *   partials  fp32, M x T, row stride ldp >= T (as written by ROWSUMSQ_PARTIAL, T = ceil(N/128)).
 *   r         fp32 output, length M: r[m] = 1 / sqrt((sum_{t<T} p[m,t]) / N + eps).
 *   h, y      optional (both NULL or both set): y[m,n] = r[m] * h[m,n] * (gamma ? gamma[n] : 1)
 *             for n < N; h and y are M x N with row strides ldh, ldy and element type `dtype`
 *             in {BF16, F16, F32}; gamma has the same dtype. y may alias h exactly.
 *   M, T, N >= 1; eps >= 0 and finite.
 */
int32_t fusedops_rmsnorm_finalize(const float* partials, int64_t ldp, int64_t M, int64_t T,
                                  int64_t N, float eps, float* r, const void* h, int64_t ldh,
                                  const void* gamma, void* y, int64_t ldy, int32_t dtype,
                                  void* stream);

/*
 * fusedops_cross_entropy_finalize — the final merge of the XENT chunk statistics.
 *
 * Defines: [Epilogue] §模式C: per row, fold the chunks' (m, s) pairs along the vocabulary with
 * m = max(m1, m2), s = s1 e^(m1 - m) + s2 e^(m2 - m) (a separate reduction, no atomics), then
 * loss[i] = m + log s - target[i], the cross-entropy -y[i, label] + log sum_k e^y[i, k].
 *
 *   stats   fp32 M x 2T as XENT wrote it (T = ceil(n_cols / 64)), row stride ld >= 2T.
 *   target  fp32 length M (XENT's out_v[0]); labels int32 length M; n_cols = N of that call.
 *   loss    fp32 length M: the loss, or 0 for a row whose label is outside [0, n_cols).
 * Errors: INVALID_ARG (null pointer, M < 1, n_cols < 1, ld < 2T), MISALIGNED (unaligned fp32 /
 * int32 pointers), LAUNCH.
 */
int32_t fusedops_cross_entropy_finalize(const float* stats, int64_t ld, int64_t M, int64_t n_cols,
                                        const float* target, const int32_t* labels, float* loss,
                                        void* stream);

/* The fixed partial width, FUSEDOPS_PARTIAL_COLS. */
int32_t fusedops_partial_cols(void);
/* FUSEDOPS_ABI_VERSION of the built library. */
int32_t fusedops_abi_version(void);
/* Static, NUL-terminated description of a status code (never NULL). */
const char* fusedops_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* FUSEDOPS_H */
