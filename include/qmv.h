/*
 * qmv.h -- C ABI of libqmv.so: dequantize-fused matrix-vector products over
 * GGUF block-quantised weights on AMD Instinct MI355X (gfx950).
 *
 * What the library computes (the pages are prior art written for CPUs and
 * WebGPU; the operations below are what they describe):
 *  - Weights stay in their GGUF block formats and are dequantised on the fly;
 *    activations and results are f32.  BebeLM page ("BebeLM：纯Rust实现的端侧
 *    大模型推理引擎"), section "量化格式支持": Q4_K super-blocks of 256 weights
 *    in 144 bytes, Q6_K for sensitive tensors, run-time dequantisation with f32
 *    activations.  Wick page, section "量化支持": Q4_K_M and Q8_0.
 *  - Fused QKV and gate/up row stacks, greedy fused argmax, small-batch verify
 *    for n-gram speculative decoding and preallocated buffers with no
 *    allocation during inference: FlareLLM page, section "推理层面的深度优化".
 *  - Sigmoid-routed top-k MoE FFN: BebeLM page, section "核心算子".
 *  - Decode is memory-bandwidth bound: BebeLM page, section "性能表现".
 *
 * Block layouts (bytes, little-endian; rows are consecutive blocks, matrices
 * consecutive rows; B = weights per block):
 *   Q8_0 (B = 32, 34 bytes):  fp16 d | int8 q[32];           w = d*q
 *   Q4_K (B = 256, 144 bytes): fp16 d | fp16 dmin | 12 bytes of packed 6-bit
 *        sub-block scales/mins | 128 bytes of nibbles;    w = d*sc*q - dmin*m
 *   Q6_K (B = 256, 210 bytes): 128 bytes low nibbles | 64 bytes high 2-bit
 *        pairs | int8 sc[16] | fp16 d;                    w = d*sc*(q - 32)
 *   (the bit order inside the fields is the standard GGUF one.)
 *
 * Conventions shared by every entry point:
 *  - Ownership: the caller allocates and owns every buffer (device memory,
 *    unless a parameter says "host").  The library never allocates, frees,
 *    copies between host and device or synchronises, and keeps no pointer
 *    after it returns.
 *  - Asynchrony: all work is enqueued on `stream` (0 = the null stream) of the
 *    current device and the call returns at once; results are valid after the
 *    stream is synchronised.
 *  - Outputs are overwritten, never accumulated into.  Outputs must not alias
 *    inputs or the workspace.
 *  - Alignment: activations (`x`, `X`, `h`, the MoE router) and outputs must
 *    be 4-byte aligned (any f32 element of a tensor may start one), `blocks`
 *    2-byte (so row slices of any matrix are valid; 16-byte-aligned block
 *    buffers stream fastest), workspaces as stated per call.
 *  - Errors: every argument check runs on the host before anything is
 *    enqueued, so a call that returns QMV_EINVAL, QMV_ESHAPE, QMV_EALIGN or
 *    QMV_EWORKSPACE has enqueued nothing.  QMV_EHIP means that HIP refused a
 *    launch (each launch's own status is checked); in a call of several
 *    launches (MoE, argmax, short convolution, split-K products) the
 *    launches before the failing one may already be enqueued.
 *    qmv_last_hip_error() returns the raw HIP code.  No exception crosses
 *    the ABI.
 *  - Re-entrancy: calls may come from several host threads at once.  The
 *    library's state is a per-device cache of the compute-unit count, two
 *    mutex-guarded caches (per-kernel occupancy, and the dynamic-LDS limit
 *    already raised per kernel and device, so hipFuncSetAttribute runs once
 *    per kernel and device), and per-thread values (the last HIP error and
 *    the timing hook below).  Calls on one stream run in order; calls on
 *    different streams must not share an output or a workspace.
 *  - Shapes: M >= 1, K >= 1, K a multiple of B, K <= QMV_MAX_K.
 */
#ifndef QMV_H
#define QMV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Block formats, numbered with their GGUF tensor type ids.  Q8_0, Q4_K and
 * Q6_K are the formats of the pages' models; Q4_0, Q4_1, Q5_0, Q5_1, Q8_1
 * (FlareLLM page, section "量化技术的全面支持": the standard 4- to 8-bit
 * quantisations), Q2_K and Q3_K (same section: K-quants from Q2K up) and
 * Q5_K (BebeLM page, section "局限与未来": Q5_K_M) are
 * served by the single-token, fused-row, gated gate/up, argmax, MoE and
 * dequantisation calls; the matrix-core products qmv_gemm_n and qmv_gemm
 * take the first three and Q5_K, qmv_quantize the first three only.  Blocks
 * (standard GGUF layouts, little-endian):
 *   Q4_0 18 B: fp16 d, 16 code bytes;                w = d * (q - 8)
 *   Q4_1 20 B: fp16 d, fp16 m, 16 code bytes;        w = d * q + m
 *   Q5_0 22 B: fp16 d, u32 fifth bits, 16 code bytes; w = d * (q - 16)
 *   Q5_1 24 B: fp16 d, fp16 m, u32 fifth bits, 16 code bytes; w = d * q + m
 *   Q8_1 36 B: fp16 d, fp16 s (unused for weights), 32 int8; w = d * q
 *   Q5_K 176 B: Q4_K's d, dmin and 12 scale bytes, 32 bytes of fifth bits,
 *     128 nibble bytes; w = d * sc_j * q - dmin * m_j, q in 0..31
 *   Q2_K 84 B: 16 bytes (scale low / min high nibble of each 16-weight
 *     sub-block j), 64 bytes of 2-bit codes, fp16 d, fp16 dmin;
 *     w = d * sc_j * q - dmin * m_j, q in 0..3
 *   Q3_K 110 B: 32 bytes of high bits, 64 bytes of 2-bit low codes, 12 bytes
 *     of 6-bit scales (stored + 32), fp16 d; w = d * sc_j * q, q in -4..3
 *     (a clear high bit lowers the code by 4)
 *   (K-quant 2-bit codes: byte 32n + l holds weight 128n + 32p + l in bits
 *   2p..2p+1; Q3_K's high bit of that weight is bit 4n + p of byte l.)
 * (32-weight formats: code byte l holds weight l in its low nibble and l + 16
 * in its high nibble; bit i of the u32 is the fifth bit of weight i.) */
typedef enum {
    QMV_Q4_0 = 2,
    QMV_Q4_1 = 3,
    QMV_Q5_0 = 6,
    QMV_Q5_1 = 7,
    QMV_Q8_0 = 8,
    QMV_Q8_1 = 9,
    QMV_Q2_K = 10,
    QMV_Q3_K = 11,
    QMV_Q4_K = 12,
    QMV_Q5_K = 13,
    QMV_Q6_K = 14
} qmv_type;

typedef enum {
    QMV_OK = 0,
    QMV_EINVAL = 1,      /* null pointer, unknown type, bad count */
    QMV_ESHAPE = 2,      /* M, K, n, E, k or a segment size out of range */
    QMV_EALIGN = 3,      /* pointer not aligned as required */
    QMV_EWORKSPACE = 4,  /* workspace missing or smaller than required */
    QMV_EHIP = 5         /* a HIP call failed; see qmv_last_hip_error() */
} qmv_status;

/* Operations that need a workspace, for qmv_workspace_bytes(). */
typedef enum {
    QMV_OP_ARGMAX = 1,
    QMV_OP_MOE = 2,
    QMV_OP_GEMM_N = 3,
    QMV_OP_SHORT_CONV = 4,
    QMV_OP_GEMM = 5
} qmv_op;

/* Largest K (columns) any entry point accepts: x is staged whole in LDS. */
#define QMV_MAX_K 32768
/* Most segments in one qmv_fused_rows call. */
#define QMV_MAX_SEGMENTS 8
/* Most columns in one qmv_gemm_n call. */
#define QMV_MAX_N 16
/* Most tokens in one qmv_gemm call. */
#define QMV_MAX_PREFILL_N 16384

/* ---- single token: y[M] = dequant(W)[M x K] . x[K] ----------------------
 * blocks: M*K/B blocks, row-major (row i is K/B consecutive blocks).
 * x: f32[K].  y: f32[M].  Wick page, section "量化支持" (Q8_0, Q4_K_M);
 * BebeLM page, section "量化格式支持" (Q4_K, Q6_K, f32 activations). */
qmv_status qmv_q8_0(const void *blocks, int64_t M, int64_t K, const float *x, float *y,
                    hipStream_t stream);
qmv_status qmv_q4_k(const void *blocks, int64_t M, int64_t K, const float *x, float *y,
                    hipStream_t stream);
qmv_status qmv_q6_k(const void *blocks, int64_t M, int64_t K, const float *x, float *y,
                    hipStream_t stream);
/* The same for the further formats above (FlareLLM page, section
 * "量化技术的全面支持"; BebeLM page, section "局限与未来"). */
qmv_status qmv_q4_0(const void *blocks, int64_t M, int64_t K, const float *x, float *y,
                    hipStream_t stream);
qmv_status qmv_q4_1(const void *blocks, int64_t M, int64_t K, const float *x, float *y,
                    hipStream_t stream);
qmv_status qmv_q5_0(const void *blocks, int64_t M, int64_t K, const float *x, float *y,
                    hipStream_t stream);
qmv_status qmv_q5_1(const void *blocks, int64_t M, int64_t K, const float *x, float *y,
                    hipStream_t stream);
qmv_status qmv_q8_1(const void *blocks, int64_t M, int64_t K, const float *x, float *y,
                    hipStream_t stream);
qmv_status qmv_q5_k(const void *blocks, int64_t M, int64_t K, const float *x, float *y,
                    hipStream_t stream);
qmv_status qmv_q2_k(const void *blocks, int64_t M, int64_t K, const float *x, float *y,
                    hipStream_t stream);
qmv_status qmv_q3_k(const void *blocks, int64_t M, int64_t K, const float *x, float *y,
                    hipStream_t stream);

/* ---- fused row stack: one launch over nseg row segments sharing x --------
 * FlareLLM page, section "推理层面的深度优化" (fused QKV and gate/up
 * projections cut the matvec calls per layer).  The stack holds
 * sum(seg_rows) rows of K columns in format t; segment s is rows
 * [sum_{r<s} seg_rows[r], sum_{r<=s} seg_rows[r]) and its result goes to the
 * device buffer y_seg[s] (f32[seg_rows[s]]).  seg_rows and y_seg are HOST
 * arrays of nseg entries, 1 <= nseg <= QMV_MAX_SEGMENTS, each seg_rows >= 1.
 * Each output equals, bit for bit, what the single-token call returns for
 * the same rows. */
qmv_status qmv_fused_rows(qmv_type t, const void *blocks, int64_t K, const float *x,
                          int32_t nseg, const int64_t *seg_rows, float *const *y_seg,
                          hipStream_t stream);

/* ---- two row stacks of different formats in one launch ------------------
 * FlareLLM page, section "推理层面的深度优化" (fused QKV) with the BebeLM
 * page, section "量化格式支持" (Q4_K_M keeps the attention V projection in
 * Q6_K while Q and K are Q4_K).  Each group (t_i, blocks_i, nseg_i,
 * seg_rows_i, y_seg_i) is what qmv_fused_rows takes, both with K columns and
 * the same x; every output equals, bit for bit, what qmv_fused_rows (and so
 * the single-token call) returns for its group.  t1 != t2, both among Q4_K,
 * Q5_K and Q6_K (the formats with 64-weight lane steps); others QMV_EINVAL. */
qmv_status qmv_fused_rows2(qmv_type t1, const void *blocks1, int32_t nseg1,
                           const int64_t *seg_rows1, float *const *y_seg1, qmv_type t2,
                           const void *blocks2, int32_t nseg2, const int64_t *seg_rows2,
                           float *const *y_seg2, int64_t K, const float *x, hipStream_t stream);

/* ---- fused gate/up with the gated product: h[j] = silu(g_j) * u_j --------
 * BebeLM page, section "核心算子" (the gated FFN: h = silu(g) * u feeds the
 * down projection) and FlareLLM page, section "推理层面的深度优化" (gate and
 * up as one fused row stack).  blocks: a stacked matrix of 2I rows x K
 * columns in format t, rows 0..I-1 gate and I..2I-1 up (the fused gate+up
 * layout).  x: f32[K]; h: f32[I] (device).  g_j and u_j equal, bit for bit,
 * rows j and I + j of the single-token call on the stack; silu(v) =
 * v / (1 + e^-v) in f32.  One launch; g and u are never written.  Needs
 * I * row bytes < 2^31 (32-bit offsets between a gate row and its up row). */
qmv_status qmv_gate_up_silu(qmv_type t, const void *blocks, int64_t I, int64_t K, const float *x,
                            float *h, hipStream_t stream);

/* ---- gated short convolution, one token -----------------------------------
 * BebeLM page, section "门控短卷积" (B, C, x = split(in_proj(h), 3); Bx = B * x;
 * causal depthwise convolution over the Bx sequence; y = C * conv;
 * out = out_proj(y); only the last 2 positions are cached) and section
 * "核心算子" (kernel size 3, a convolution state instead of a KV cache).
 * in_proj: 3D rows x H columns in format in_t (rows 0..D-1 B, D..2D-1 C,
 *   2D..3D-1 x).  out_proj: H rows x D columns in format out_t.
 * h: f32[H].  w_conv: f32[D][3]; tap k multiplies the input k - 2 positions
 *   back (tap 2 the current Bx).  state: f32[D][2], (older, newer) cached Bx
 *   per channel, read and then replaced by (newer, current Bx) -- zero it
 *   before the first token.  out: f32[H].
 * workspace: device, >= qmv_workspace_bytes(QMV_OP_SHORT_CONV, D, 0, 0, 0)
 *   bytes, 16-byte aligned; it receives y (f32[D]).
 * Two launches: in_proj with the gates, the convolution and the state shift
 * (the 3D row results are never written), then out_proj on y.  state, out
 * and workspace must not overlap each other or the inputs.  Needs 2D * row
 * bytes < 2^31 (32-bit offsets from a channel's B row to its x row). */
qmv_status qmv_short_conv(qmv_type in_t, const void *in_proj, int64_t D, int64_t H, const float *h,
                          const float *w_conv, float *state, qmv_type out_t, const void *out_proj,
                          float *out, void *workspace, size_t ws_bytes, hipStream_t stream);

/* ---- fused greedy argmax: the index and value of max_i (dequant(W) x)_i ---
 * FlareLLM page, section "推理层面的深度优化": at temperature 0 the next
 * token is found during the output projection, without a logits buffer.
 * Ties go to the lowest index.  idx_out: int32[1], max_out: f32[1] (device).
 * workspace: device, >= qmv_workspace_bytes(QMV_OP_ARGMAX, M, K, 0, 0) bytes,
 * 8-byte aligned, no initial contents needed.  The per-row values are the
 * ones qmv_q*_* returns for the same (t, M, K). */
qmv_status qmv_argmax(qmv_type t, const void *blocks, int64_t M, int64_t K, const float *x,
                      int32_t *idx_out, float *max_out, void *workspace, size_t ws_bytes,
                      hipStream_t stream);

/* ---- qmv_argmax without a workspace ---------------------------------------
 * For callers that cannot allocate device memory at all (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same result as qmv_argmax -- the same kernels, bit for bit -- with the
 * per-workgroup keys kept in a library-owned device array instead of a
 * workspace.  That array holds QMV_ARGMAX_SCRATCH_KEYS keys (16 KiB), the
 * most an argmax launch uses for any M and K; each GPU the library runs on
 * holds its own copy until the process ends, and its address is looked up
 * once per device on the first call there.  The call allocates nothing on
 * the device and needs nothing zeroed (every key the finalising kernel reads
 * is written by the same call); the array keeps the last call's keys.  All
 * calls on one GPU share the array: calls that overlap on one GPU (on
 * different streams without ordering between them) race.  Arguments,
 * limits and errors as qmv_argmax. */
#define QMV_ARGMAX_SCRATCH_KEYS 2048
qmv_status qmv_argmax_noalloc(qmv_type t, const void *blocks, int64_t M, int64_t K,
                              const float *x, int32_t *idx_out, float *max_out,
                              hipStream_t stream);

/* ---- sigmoid-routed top-k MoE FFN for one token ---------------------------
 * BebeLM page, section "核心算子" (MoE FFN): router scores are sigmoids
 * (not a softmax); the k experts with the largest score + bias are chosen
 * (the bias only ranks; ties go to the lower expert index); their weights are
 * the unbiased scores renormalised to sum 1; section "量化格式支持" keeps the
 * router and the expert bias in f32.  For each chosen expert e:
 *   g = Gate_e x, u = Up_e x, h = silu(g) * u, y_e = Down_e h;  y = sum w_e y_e.
 * x: f32[H].  router: f32[E][H] (row e scores expert e).  bias: f32[E].
 * gate_up: E stacked matrices of 2I rows x H columns in format gu_t (rows
 *   0..I-1 gate, I..2I-1 up).  down: E stacked matrices of H rows x I columns
 *   in format dn_t.
 * y: f32[H].  topk_idx: int32[k] and topk_w: f32[k], in rank order.
 * workspace: device, >= qmv_workspace_bytes(QMV_OP_MOE, H, I, E, k) bytes,
 *   16-byte aligned.  Layout after the call (for inspection): f32 logits[E]
 *   at byte 0; from byte 256 f32 gu[k][2I] (per slot: the I gate results,
 *   then the I up results); then f32 h[k][I] = silu(g) * u.
 * Constraints: 1 <= k <= E <= 64; H and I multiples of their formats' B;
 *   k * I <= QMV_MAX_K; with a 32-weight down format, I a multiple of 128.  Three launches; the selection never leaves the GPU. */
qmv_status moe_qmv_topk(const float *x, int64_t H, const float *router, const float *bias,
                        int32_t E, int32_t k, qmv_type gu_t, const void *gate_up,
                        qmv_type dn_t, const void *down, int64_t I, float *y,
                        int32_t *topk_idx, float *topk_w, void *workspace, size_t ws_bytes,
                        hipStream_t stream);

/* ---- small batch (speculative verify): Y[n][M] = X[n][K] . dequant(W)^T ----
 * FlareLLM page, section "推理层面的深度优化" (n-gram speculative decoding
 * checks several drafted tokens against the same weights).  X: f32 n x K
 * row-major, Y: f32 n x M row-major, 1 <= n <= QMV_MAX_N.  Formats Q8_0,
 * Q4_K, Q5_K, Q6_K.  Runs on the matrix
 * cores (bf16 MFMA on the exact integer codes, X split into bf16 hi + lo, f32
 * scales), within 1e-5 * sum_k |w_ik x_k| of the exact result like the
 * matvecs.  One launch when K <= 4096: a workgroup covers all of K for its
 * rows (its waves split K and add their partial products in a fixed order),
 * and the workspace size is 0.  Longer K is cut into slices of at most 4096
 * weights whose partial sums go to the workspace and are added in slice
 * order by a second launch.  workspace: device, >=
 * qmv_workspace_bytes(QMV_OP_GEMM_N, M, K, n, 0) bytes (NULL when that is
 * 0), 16-byte aligned, no initial contents needed.  Results are
 * deterministic; n <= 8 and 8 < n <= 16 use two operand layouts, so a
 * column's bits may differ between the two ranges (both within the bound). */
qmv_status qmv_gemm_n(qmv_type t, const void *blocks, int64_t M, int64_t K, int32_t n,
                      const float *X, float *Y, void *workspace, size_t ws_bytes,
                      hipStream_t stream);

/* ---- prefill-size product: Y[n][M] = X[n][K] . dequant(W)^T --------------
 * BebeLM page, section "性能表现" (prompt tokens are processed as a batch,
 * unlike the one-token decode).  X: f32 n x K row-major, Y: f32 n x M
 * row-major, 1 <= n <= QMV_MAX_PREFILL_N and n * K * 4 < 2^32.  Formats
 * Q8_0, Q4_K, Q5_K, Q6_K.  Same arithmetic as qmv_gemm_n (bf16 MFMA on the exact
 * codes, X as bf16 hi + lo, f32 scales per sub-block), so within 1e-5 *
 * sum_k |w_ik x_k| per output.  A workgroup covers up to 64 tokens by 128
 * or 256 rows; K is split into slices when rows and tokens alone give
 * fewer than 384 workgroups (1.5 per compute unit of a 256-CU part), and
 * the slices' partial sums are added in a fixed order, so results are
 * deterministic either way (the plan depends only on M, K and n).  A
 * first launch splits X once into the operand layout (bf16 hi + lo and
 * sub-block sums, 1088 bytes per 16 tokens and 256 values) in the
 * workspace, which every workgroup then copies instead of converting X.
 * workspace: device, >= qmv_workspace_bytes(QMV_OP_GEMM, M, K, n, 0) bytes
 * (always > 0: the split activations, plus the slices' partial sums when K
 * is split), 16-byte aligned, no initial contents needed; QMV_EWORKSPACE if
 * it is missing or too small. */
qmv_status qmv_gemm(qmv_type t, const void *blocks, int64_t M, int64_t K, int64_t n, const float *X,
                    float *Y, void *workspace, size_t ws_bytes, hipStream_t stream);

/* ---- dequantise to f32 (verification surface): w_out[M][K] --------------
 * BebeLM page, section "GGUF加载器" (the loader dequantises Q4_K, Q6_K, F16
 * and F32 tensors) and section "量化格式支持" (weights are dequantised at run
 * time, activations stay f32): w_out holds each weight's block decoding,
 * w = d*q (Q8_0), d*sc*q - dmin*m (Q4_K, one rounding), d*sc*(q - 32) (Q6_K)
 * and the layouts above for the other formats; every matvec above is defined
 * on these values.  w_out: f32 M x K row-major (device), 16-byte aligned;
 * one launch, bit-exact (no f32 rounding except Q4_K's single subtraction). */
qmv_status qmv_dequant(qmv_type t, const void *blocks, int64_t M, int64_t K, float *w_out,
                       hipStream_t stream);

/* ---- quantise f32 weights to blocks (weight preparation) -----------------
 * w: f32 M x K row-major; blocks_out: M*K/B blocks.  Plain min/max rules
 * (the pages give none): Q8_0 d = max|w|/127, q = round(w/d); Q4_K mins
 * first (dmin = max(-min)/62), then scales (d = max s/62, s = range/15);
 * Q6_K s = max|w|/31, d = max s/126; codes rounded half away from zero. */
qmv_status qmv_quantize(qmv_type t, const float *w, int64_t M, int64_t K, void *blocks_out,
                        hipStream_t stream);

/* ---- helpers -------------------------------------------------------------- */
/* Bytes of one row of K weights in format t; 0 if K is not a multiple of B. */
size_t qmv_row_bytes(qmv_type t, int64_t K);
/* Workspace an operation needs.  ARGMAX: (M, K, -, -); MOE: (H, I, E, k);
 * GEMM_N: (M, K, n, -); SHORT_CONV: (D, -, -, -). */
size_t qmv_workspace_bytes(qmv_op op, int64_t a, int64_t b, int32_t c, int32_t d);
/* Raw HIP error code of this thread's last QMV_EHIP (0 if none). */
int qmv_last_hip_error(void);
/* Static, human-readable name of a status. */
const char *qmv_status_str(qmv_status s);

/* ---- kernel timing hook (measurement only) --------------------------------
 * Arms this thread's next call: its main kernel (the matvec, argmax, MoE
 * expert or small-batch kernel) is launched with hipExtLaunchKernelGGL so that
 * the caller-created events `start` and `stop` carry that kernel's own
 * dispatch start and end timestamps -- no marker packets, no gaps counted.
 * Both events must be valid (created by the caller) or both NULL (disarm).
 * The hook is consumed by the next launching call on this thread. */
qmv_status qmv_time_next_launch(hipEvent_t start, hipEvent_t stop);

/* ---- bandwidth probe (measurement only) -----------------------------------
 * Streams `bytes` (a multiple of 16, buffer 16-byte aligned) in 4 KB chunks
 * per wave with 128-bit nontemporal loads, the fastest read pattern measured
 * on this device, and writes one u32 per workgroup into sink (>= 2048
 * entries); gives the achievable HBM read rate. */
qmv_status qmv_probe_stream_read(const void *buf, size_t bytes, uint32_t *sink,
                                 hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QMV_H */
