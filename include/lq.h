/*
 * lq.h -- C ABI of liblq.so: windowed INT8 recurrent-state decode for Gated
 * DeltaNet (scalar gate) and Kimi Delta Attention (per-key-channel gate) on
 * AMD Instinct MI355X (gfx950).
 *
 * What it computes.  The arXiv 2609.38166 abstract ("LeapQuant: Efficient
 * Linear Attention with Accurate Recurrent State Quantization", section
 * "Abstract (arXiv)" of the mlsanity.com paper page) describes per-window
 * quantization of the linear-attention recurrent state: the state is stored
 * in 8 bits and quantized only once at the end of a window of tokens; inside
 * the window each output comes from the fixed low-bit state plus
 * high-precision buffered updates; at quantization time the largest outlier
 * rows and columns are kept as a few high-precision Compensator Tokens that
 * share the real tokens' update path, and the residual is smoothed before
 * quantization.  The bedrocknews.com review of the paper adds that the state
 * goes from FP32 to INT8 and the compensators are kept in FP16/FP32.
 *
 * The recurrence (the pages name it but print no equation; this is the gated
 * delta rule of the cited Gated DeltaNet / Kimi Linear works): per unit
 * (one sequence x one value head) a d_v x d_k state S,
 *     S_t = S_{t-1} Diag(g_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t,
 * with g_t = alpha_t (one scalar per unit, gate_kind LQ_GATE_SCALAR) or
 * g_t = a_t in (0,1]^{d_k} (gate_kind LQ_GATE_CHANNEL).  Quantizer (readings,
 * the pages give no formula): line scores are squared L2 norms; the n_comp
 * highest-scoring rows/columns become fp32 compensator lines; the residual R
 * gets s_j = sqrt(max_i |R_ij|) per key channel and sigma_i =
 * max_j |R_ij / s_j| / 127 per row; codes = clamp(rne(R_ij/(sigma_i s_j)),
 * -127, 127).
 *
 * Conventions for every call:
 *  - pointers named in a call are DEVICE pointers the caller owns (for
 *    example torch tensors); `cfg`, `bytes`, `layout` and `flags` are host
 *    pointers;
 *  - `stream` is a hipStream_t (NULL = the default stream); every call except
 *    lq_read_status is asynchronous on it, launches nothing when it returns
 *    an error, and never allocates device memory; the library holds no
 *    global mutable state (each call derives its launch sizes afresh), so
 *    distinct state blobs may be used concurrently, from any host thread;
 *    calls on one blob must be ordered on one stream;
 *  - device pointers must be 16-byte aligned, the state blob 256-byte
 *    aligned (LQ_EINVAL otherwise);
 *  - errors found on the device (a decode step on a full window, a
 *    non-finite input or start state) never abort: they set sticky flags in
 *    the blob, read with lq_read_status and reset with lq_clear_status (and
 *    by lq_state_init / lq_prefill, which start a new state).
 *
 * Layouts (row-major, fp32 unless noted; unit u = s * n_v_heads + h; value
 * head h reads key head h / (n_v_heads / n_k_heads)):
 *   q, k    [n_seq][n_k_heads][d_k]      v, o   [n_seq][n_v_heads][d_v]
 *   beta    [n_seq][n_v_heads]           gate   [n_seq][n_v_heads] (scalar)
 *                                               [n_seq][n_v_heads][d_k] (channel)
 *   S0, S_out, S (fp32 state)            [n_seq][n_v_heads][d_v][d_k]
 * q and k are used as given: the caller L2-normalizes them and folds any
 * 1/sqrt(d_k) into q.
 */
#ifndef LQ_H
#define LQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP runtime's stream handle, declared exactly as <hip/hip_runtime_api.h>
 * declares it, so this header needs no HIP header. */
typedef struct ihipStream_t* hipStream_t;

/* return codes */
#define LQ_OK 0
#define LQ_EINVAL (-1)       /* NULL where not allowed, misaligned pointer, inconsistent sizes */
#define LQ_EUNSUPPORTED (-2) /* a configuration outside the supported set below */
#define LQ_EHIP (-3)         /* the HIP runtime reported an error (launch or copy) */
#define LQ_ESCRATCH (-4)     /* lq_window_flush_noalloc: more units than its scratch holds */

/* gate kinds */
#define LQ_GATE_SCALAR 0  /* Gated DeltaNet: one alpha per unit and token */
#define LQ_GATE_CHANNEL 1 /* Kimi Delta Attention: one gate per key channel */

/* state code formats (the 8-bit codes of the stored state) */
#define LQ_CODE_INT8 0 /* integers in [-127, 127] */
#define LQ_CODE_E4M3 1 /* 8-bit floats: OCP E4M3 without infinities, magnitudes up to 448 */

/* window-buffer formats (the buffered tokens' k and v) */
#define LQ_BUFFER_FP32 0 /* as given */
#define LQ_BUFFER_FP16 1 /* IEEE binary16, nearest-even, magnitudes above 65504 stored as 65504 */
#define LQ_BUFFER_NFORM 2 /* scalar gate, d = 128: each entry keeps k, the gate and, in place of v
                             and beta, the WY-form vector n (fp32), so the decode has no
                             sequential pass over the window and the boundary is one product */

/* how a decode step reads each unit's state and window (lq_config.load_policy):
   the bytes a step reads from a unit (its 8-bit tile, scales, compensator lines and
   buffered values) are read once per step, so streaming (non-temporal) loads keep
   them from displacing data that is read again (the keys that the value heads of
   one key head share, the lines the step writes); a state that stays in the
   last-level cache between steps is read faster with ordinary loads */
#define LQ_LOADS_AUTO 0   /* streaming loads in decode launches of more than 2,048 units */
#define LQ_LOADS_STREAM 1 /* always (a caller whose states do not stay in the cache) */
#define LQ_LOADS_CACHED 2 /* never */

/* sticky device flags (lq_read_status) */
#define LQ_DEV_WINDOW_OVERFLOW 0x1u /* lq_decode_step found a full window: that unit's o is NaN, nothing appended */
#define LQ_DEV_NONFINITE_INPUT 0x2u /* an input (decode token, prompt token, start state S0) was NaN or Inf */
#define LQ_DEV_BUFFER_SATURATED 0x4u /* binary16 buffer: a k or v magnitude above 65504 was stored as 65504 */

/*
 * Problem description.  Supported: d_k == d_v in {64, 128};
 * 1 <= window <= 256; 0 <= n_comp <= 16; n_seq, n_v_heads, n_k_heads >= 1;
 * n_v_heads % n_k_heads == 0; gate_kind in {LQ_GATE_SCALAR, LQ_GATE_CHANNEL};
 * code_format in {LQ_CODE_INT8, LQ_CODE_E4M3};
 * buffer_format in {LQ_BUFFER_FP32, LQ_BUFFER_FP16, LQ_BUFFER_NFORM} (NFORM with
 * gate_kind LQ_GATE_SCALAR and d_k = d_v = 128 only); flush_cus >= 0;
 * load_policy in {LQ_LOADS_AUTO, LQ_LOADS_STREAM, LQ_LOADS_CACHED};
 * the unit count n_seq * n_v_heads below 2^31.
 */
typedef struct lq_config {
    int32_t n_seq;
    int32_t n_v_heads;
    int32_t n_k_heads;
    int32_t d_k;
    int32_t d_v;
    int32_t window;   /* W: tokens per quantization window */
    int32_t n_comp;   /* compensator lines kept per unit */
    int32_t gate_kind;
    int32_t code_format; /* LQ_CODE_INT8 (the review's INT8) or LQ_CODE_E4M3 (the
                            abstract's "8-bit" read as a floating-point format): the
                            scales are chosen so the largest code is 127 or 448 */
    int32_t buffer_format; /* LQ_BUFFER_FP32, or LQ_BUFFER_FP16: each token's k and v
                              enter the window rounded to binary16 (half the buffer
                              bytes); the rounded token is then the token everywhere:
                              its own output, later replays, the window-end state */
    int32_t flush_cus; /* CUs' worth of workgroups in the persistent grid of the
                          window-boundary kernel (lq_window_flush and its
                          allocation-free form, lq_state_init, lq_prefill,
                          lq_dequant_state), which walks the units: at d = 128 a
                          workgroup fills a CU, so the kernel occupies at most this
                          many CUs wherever they are.  0, or a value above the
                          device's CU count: every CU.  A caller that runs a
                          layer's boundary on a second stream beside the next
                          layers' decode steps gives it part of the device.  The
                          results do not depend on it (each unit is computed the
                          same way wherever it runs) */
    int32_t load_policy; /* LQ_LOADS_*: the cache policy of lq_decode_step's state and
                            window reads; performance only, the results are the same
                            bit for bit */
} lq_config;

/*
 * Byte offsets of the sections of the state blob (each 256-byte aligned).
 * The blob is self-contained: copying it (with the lq_config) checkpoints
 * the whole decode state.
 *   status    uint32 sticky flags
 *   fill      int32 [units]            tokens buffered in the current window
 *   codes     8-bit [units][d_v][d_k]  the quantized state (int8, or E4M3 bytes)
 *   sigma     fp32  [units][d_v]       per-row scales
 *   smooth    fp32  [units][d_k]       per-key-channel smoothing factors
 *   comp_idx  int32 [units][n_comp]    c < d_v: row c; c >= d_v: column c - d_v
 *   comp_vec  fp32  [units][n_comp][max(d_k,d_v)]  row slot: the row (d_k);
 *                                      column slot: the column (d_v)
 *   buf_k     fp32 or fp16 [n_seq][n_k_heads][window][d_k]  (shared by a key head's value heads)
 *   buf_v     fp32 or fp16 [units][window][d_v]  (NFORM: the vectors n, fp32)
 *   buf_beta  fp32  [units][window]  (NFORM: not used; beta is inside n)
 *   buf_gate  fp32  [units][window] (scalar) or [units][window][d_k] (channel)
 *   work      int32 [1 + units]        scratch of lq_window_flush: count, then the
 *                                      units whose window is due
 */
typedef struct lq_layout {
    size_t total_bytes;
    size_t status, fill, codes, sigma, smooth, comp_idx, comp_vec;
    size_t buf_k, buf_v, buf_beta, buf_gate;
    size_t work;
} lq_layout;

/* Size in bytes of the state blob for cfg.  Host only, no HIP call. */
int32_t lq_state_bytes(const lq_config* cfg, size_t* bytes);

/* Section offsets of the blob for cfg.  Host only, no HIP call. */
int32_t lq_state_layout(const lq_config* cfg, lq_layout* layout);

/*
 * Quantize a start state into the blob: compensators, smoothing, scales and
 * codes of S0 (the abstract's window-end quantization with an empty window),
 * fill = 0, status = 0 (then LQ_DEV_NONFINITE_INPUT if S0 holds a NaN or Inf).
 * S0 may be NULL for the zero state.  Buffers are left as they are (never
 * read while fill = 0).
 */
int32_t lq_state_init(const lq_config* cfg, void* state, const float* S0, hipStream_t stream);

/*
 * One decode token for every sequence.  Per unit: append (k, v, beta, gate)
 * to the window buffer, then write o = S_j q where S_j is the stored
 * window-start state advanced through the buffered tokens (the current one
 * included): per the abstract, a token inside a window reads the 8-bit state
 * held since the window began plus the exactly kept tokens since.  The INT8
 * codes, scales, smoothing and compensators are read, never written.  A unit
 * whose window is already full (lq_window_flush was not called) gets o = NaN
 * and sets LQ_DEV_WINDOW_OVERFLOW.
 */
int32_t lq_decode_step(const lq_config* cfg, void* state, const float* q, const float* k,
                       const float* v, const float* beta, const float* gate, float* o,
                       hipStream_t stream);

/*
 * Window-boundary requantization: per the arXiv 2609.38166 abstract ("Abstract
 * (arXiv)" section, mlsanity.com paper page) the state goes through a whole
 * window of tokens unquantized and is requantized a single time when the
 * window closes, keeping the largest outliers
 * as Compensator Tokens and smoothing the residual before quantization; the
 * bedrocknews.com review adds that this happens at the window boundary instead
 * of after every update.  Every unit whose window is full (fill == window),
 * and every unit of a sequence s with force_mask[s] != 0 and fill > 0, is
 * advanced through its buffered tokens in FP64, gets new compensators,
 * smoothing, scales and codes, and fill = 0.  Other units are untouched.
 * force_mask: device uint8 [n_seq], or NULL.  Must be called between the
 * decode step that fills a window and the next decode step.  Uses the blob's
 * work section as scratch (the list of due units).
 */
int32_t lq_window_flush(const lq_config* cfg, void* state, const uint8_t* force_mask,
                        hipStream_t stream);

/*
 * lq_window_flush without the blob's work section: for callers that cannot
 * allocate device memory or must not have a call allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid it).  Same
 * arguments, semantics and results as lq_window_flush; the list of due units
 * is kept instead in a device array inside the library (one per GPU, 1 MiB,
 * held until the process ends), so the call allocates nothing.  At most
 * LQ_NOALLOC_MAX_UNITS units (n_seq * n_v_heads); more returns LQ_ESCRATCH
 * and launches nothing.  Every call on one GPU uses that GPU's array: calls
 * that overlap in time on one GPU (on different streams, or from different
 * host threads without ordering) race and must not be issued.
 */
#define LQ_NOALLOC_MAX_UNITS 262144
int32_t lq_window_flush_noalloc(const lq_config* cfg, void* state, const uint8_t* force_mask,
                                hipStream_t stream);

/*
 * Prefill: run a prompt of n_tok tokens (n_tok >= 0, the same for every
 * sequence) through the plain recurrence, from S0 (fp32 [n_seq][n_v_heads]
 * [d_v][d_k], or NULL for the zero state), and quantize the final state into
 * the blob as lq_state_init does (fill = 0, status = 0).  The arXiv abstract
 * ("Abstract (arXiv)" section, mlsanity.com paper page): the recurrent state
 * compresses the context; the prompt is that context, and the state is
 * quantized once, at its end.  Inside the prompt nothing is quantized: the
 * state is advanced 16 tokens at a time in FP64 on the matrix cores (the
 * chunked form of the delta rule, as in the window-end flush).
 * Inputs are token-major: q, k [n_tok][n_seq][n_k_heads][d_k]; v
 * [n_tok][n_seq][n_v_heads][d_v]; beta [n_tok][n_seq][n_v_heads]; gate
 * [n_tok][n_seq][n_v_heads] (scalar) or [n_tok][n_seq][n_v_heads][d_k]
 * (channel), all fp32, same conventions as lq_decode_step.  o (fp32
 * [n_tok][n_seq][n_v_heads][d_v], or NULL) receives o_t = S_t q_t for every
 * prompt token.  Pointers are device pointers owned by the caller, 16-byte
 * aligned (beta and a scalar gate 4-byte); errors as for lq_state_init (a
 * NaN or Inf in S0 or in a prompt token sets LQ_DEV_NONFINITE_INPUT).
 */
int32_t lq_prefill(const lq_config* cfg, void* state, const float* S0, int32_t n_tok,
                   const float* q, const float* k, const float* v, const float* beta,
                   const float* gate, float* o, hipStream_t stream);

/*
 * Dequantized state into S_out (fp32): the window-start state
 * Diag(sigma) Q Diag(s) + compensator lines -- the fixed low-bit state that
 * the arXiv 2609.38166 abstract ("Abstract (arXiv)" section, mlsanity.com
 * paper page) keeps for the whole window, with the Compensator Tokens added
 * back -- or, with include_buffer != 0, that state advanced through the
 * buffered tokens, i.e. what the last decode step read its output from (the
 * window-start state plus the exactly kept tokens since).
 * For inspection and checkpoint conversion.
 */
int32_t lq_dequant_state(const lq_config* cfg, const void* state, float* S_out,
                         int32_t include_buffer, hipStream_t stream);

/*
 * The FP32-state comparison step: S (fp32, in place) advanced by one token
 * and o = S_t q, with the same inputs and layouts as lq_decode_step.  This is
 * the FP32 baseline the pages measure against (bedrocknews.com review: the
 * comparison runs the same models with a 32-bit float state).
 */
int32_t lq_fp32_decode_step(const lq_config* cfg, float* S, const float* q, const float* k,
                            const float* v, const float* beta, const float* gate, float* o,
                            hipStream_t stream);

/*
 * Synchronizes `stream`, then returns the blob's sticky device flags
 * (LQ_DEV_*) in *flags (host pointer).  The flags stay set.
 */
int32_t lq_read_status(const lq_config* cfg, const void* state, uint32_t* flags,
                       hipStream_t stream);

/*
 * Resets the blob's sticky device flags to 0, asynchronously on `stream`
 * (ordered after the calls already queued there).
 */
int32_t lq_clear_status(const lq_config* cfg, void* state, hipStream_t stream);

/* Static description of a return code. */
const char* lq_strerror(int32_t code);

#ifdef __cplusplus
}
#endif

#endif /* LQ_H */
