/*
 * libgdr — gated delta rule kernels for AMD Instinct MI355X (gfx950).
 *
 * The operation (Gated Delta Rule-2; Gated DeltaNet-2 Q&A page "Gated
 * DeltaNet-2 — decoupling erase and write in linear attention", Q3, and
 * "Gated DeltaNet-2 Review" §3-1), per independent (batch, head) pair:
 *
 *     S_t = (I - k_t (b_t ⊙ k_t)^T) D_t S_{t-1} + k_t (w_t ⊙ v_t)^T
 *     D_t = diag(alpha_t),  alpha_t = exp(log_alpha_t)
 *     o_t = S_t^T q_t                  (read-out after the write; "Gated
 *                                       DeltaNet" explainer, mechanism)
 *
 * S_t is d_k x d_v.  b_t in R^{d_k} is the key-side erase gate, w_t in
 * R^{d_v} the value-side write gate.  Tying b = w = beta·1 gives KDA; also
 * making D_t = alpha_t·I gives Gated DeltaNet (Q&A page Q3).  Gates are
 * neither clamped nor assumed to lie in [0,1]; the expanded erase range
 * [0,2] ("Gated DeltaNet-2 Review" §5 ablation; sungsoo commentary, state
 * tracking) works unchanged.  No query scaling and no normalisation of q, k
 * is applied: that is the caller's job.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller.  The
 *   library never allocates device memory (scratch space is passed in as a
 *   caller-owned workspace), never frees caller memory, and keeps no state
 *   besides a lazily cached device-property record and, once the backward
 *   has run on a device, one extra stream and two events there (kept until
 *   the process ends).
 * - Execution is asynchronous on `stream` (a hipStream_t passed as void*;
 *   NULL is the default stream).  No call synchronises.
 * - Arguments are validated before any launch.  An invalid argument returns
 *   a status and launches nothing.  Launch failures return GDR_ERR_LAUNCH.
 *   No exception, abort or exit crosses the ABI.
 * - Layouts are contiguous row-major.  "act" is the activation dtype chosen
 *   by flags (bf16 bit patterns as uint16, or fp32).  Pointers must be
 *   16-byte aligned.
 * - Gate modes (flags): each of log_alpha, b, w is either per channel
 *   ([..., d_k] / [..., d_k] / [..., d_v]) or one scalar per token ([...]).
 *   Gated DeltaNet passes scalar log_alpha and the same scalar buffer as b
 *   and w; KDA passes channel log_alpha and one scalar buffer as b and w;
 *   the b-only / w-only ablations ("Gated DeltaNet-2 Review" §5 gate
 *   ablation) are mixed modes.
 * - Precision: with bf16 activations the dense chunk contractions run on
 *   MFMA with f16 operands and fp32 accumulation; the state, log-decay and
 *   the cumulative decay stay fp32 (the log-decay path runs in fp32:
 *   "Gated DeltaNet-2 Review" §3-2 item 2).  With fp32 activations every
 *   contraction runs on fp32 MFMA.  Erase gates up to 2 (the expanded range,
 *   "Gated DeltaNet-2 Review" §5) keep the bf16 accuracy for ordinary keys;
 *   one key repeated through a chunk with an erase gate near 2 makes the
 *   in-chunk solve cancel by about two orders of magnitude, and such inputs
 *   need fp32 activations.
 * - Decay range: every call returns values for any decay an fp32 log_alpha
 *   can express.  The forward with a workspace (fixed-length and packed)
 *   references each 16-token block's decay so that no operand factor leaves
 *   the f16 range.  The other chunk kernels reference a chunk's decay to its
 *   end; a (sequence, head) whose in-chunk decay leaves their operand range
 *   (about 10 nats per chunk with f16 operands) is recomputed token by token
 *   in fp32 by a follow-up kernel of the same call, which costs one small
 *   launch when no head needs it.  That recompute is sequential over a unit's
 *   tokens: a backward at B=1, H=32, T=16384, d=128 whose heads all leave the
 *   chunk-64 range takes about 240 ms instead of 2 ms.  Callers with such decay
 *   should pass chunk 16 to gdr_chunk_bwd (about 10 nats per 16 tokens stay in
 *   range; the same backward then takes about 13 ms).
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdr_status {
    GDR_OK = 0,
    GDR_ERR_INVALID_ARG = 1,     /* null pointer, bad size, misalignment, T % chunk != 0 */
    GDR_ERR_UNSUPPORTED = 2,     /* a valid request the library has no kernel for     */
    GDR_ERR_WORKSPACE = 3,       /* workspace pointer NULL or smaller than required   */
    GDR_ERR_LAUNCH = 4,          /* the HIP runtime rejected a launch                 */
    GDR_ERR_DEVICE = 5           /* no usable gfx950 device / device query failed     */
} gdr_status;

/* flags (bitwise OR) */
#define GDR_ACT_BF16      0x0u   /* q, k, v, b, w, dO are bf16 (uint16 bit patterns)  */
#define GDR_ACT_F32       0x1u   /* q, k, v, b, w, dO are fp32                        */
#define GDR_OUT_BF16      0x2u   /* o is bf16 (default fp32).  Forward/decode only.   */
#define GDR_ALPHA_SCALAR  0x4u   /* log_alpha is one fp32 per token                   */
#define GDR_B_SCALAR      0x8u   /* b is one value per token                          */
#define GDR_W_SCALAR      0x10u  /* w is one value per token                          */
#define GDR_FWD_GENERIC   0x20u  /* forward: use the single-role kernel even where the
                                    pipelined one applies (same results up to rounding
                                    order; for testing)                               */
#define GDR_FWD_SPLIT     0x80u  /* forward with a workspace: run the chunk producer and
                                    the state chains as two kernels, one after the
                                    other, instead of one persistent kernel (same
                                    results bit for bit; for testing)               */
#define GDR_GATE_LOGITS   0x40u  /* log_alpha, b and w hold logits: the kernels use
                                    log alpha = log(sigmoid(log_alpha)), b = sigmoid(b),
                                    w = sigmoid(w) in fp32 (the token mixer's gating,
                                    fused into the loads), and the backward returns the
                                    gradients of the logits.  Two-pass forward and
                                    backward (workspace, bf16, chunk 64) and decode only;
                                    GDR_ERR_UNSUPPORTED elsewhere.                      */

#define GDR_ABI_VERSION 2

int gdr_abi_version(void);
const char* gdr_status_string(gdr_status s);

/*
 * Chunkwise-parallel forward (the WY form: in-chunk cumulative log-decay is
 * absorbed into the rank-one erase factor, giving an asymmetric delta
 * recurrence solved per chunk; Q&A page Q4, "Gated DeltaNet-2 Review"
 * §3-2 item 5).
 *
 *   q, k       : act  [B, H, T, d_k]
 *   v          : act  [B, H, T, d_v]
 *   log_alpha  : fp32 [B, H, T, d_k]   or [B, H, T] with GDR_ALPHA_SCALAR
 *   b          : act  [B, H, T, d_k]   or [B, H, T] with GDR_B_SCALAR
 *   w          : act  [B, H, T, d_v]   or [B, H, T] with GDR_W_SCALAR
 *   S0         : fp32 [B, H, d_k, d_v] initial state; NULL means zeros
 *   o          : fp32 (or bf16 with GDR_OUT_BF16) [B, H, T, d_v], written
 *   S_final    : fp32 [B, H, d_k, d_v], written; NULL means not written.
 *                May alias S0 (each workgroup reads its block of S0 before
 *                writing the same block).  No other aliasing is allowed.
 *   chunk      : 16, 32 or 64; T must be a multiple of chunk.  The chunk is
 *                a blocking choice: results equal the token recurrence up to
 *                rounding for every chunk size.
 *   workspace  : optional device scratch owned by the caller, contents on
 *                entry ignored.  When it is non-NULL and
 *                gdr_chunk_fwd_workspace_bytes() is non-zero for the call, a
 *                persistent kernel runs (one workgroup per compute unit, after
 *                a small kernel that clears the call's flags): producer
 *                workgroups compute every chunk's state-independent operands
 *                into the workspace while per-head state chains consume them,
 *                each chunk handed over through a flag.  A chain waits for a
 *                flag with a bounded spin (seconds); if the call's producers
 *                cannot become resident meanwhile (another kernel holding the
 *                compute units for that long), the chain stops and its head's
 *                o and S_final are NaN.  workspace_bytes below the required
 *                size returns GDR_ERR_WORKSPACE.  With a NULL workspace (or a
 *                zero requirement) a single fused kernel runs.  Both paths
 *                give the same result up to rounding.
 * Supported: d_k, d_v in {16, 32, 64, 128}; B*H >= 1; T >= 0 (T == 0 copies
 * S0 to S_final).  Returns GDR_ERR_UNSUPPORTED for other head sizes.
 */
size_t gdr_chunk_fwd_workspace_bytes(int B, int H, int T, int d_k, int d_v,
                                     int chunk, uint32_t flags);

gdr_status gdr_chunk_fwd(const void* q, const void* k, const void* v,
                         const float* log_alpha, const void* b, const void* w,
                         const float* S0, void* o, float* S_final,
                         int B, int H, int T, int d_k, int d_v, int chunk,
                         uint32_t flags, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * gdr_chunk_fwd without a caller workspace and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Arguments and
 * results are those of gdr_chunk_fwd.  Where gdr_chunk_fwd would take a
 * workspace, this call uses a library-owned device array of
 * GDR_NOALLOC_SCRATCH_BYTES on the current GPU instead (each GPU the library
 * runs on holds its own copy until the process ends; it is looked up once per
 * device at the first call there).  A call whose
 * gdr_chunk_fwd_workspace_bytes() exceeds GDR_NOALLOC_SCRATCH_BYTES returns
 * GDR_ERR_WORKSPACE and launches nothing (at d_k = d_v = 128 the array holds
 * the operands of 900 chunks of 64 tokens, e.g. B*H = 16 heads of T = 3584).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (different streams, or different host threads) race and must be
 * ordered by the caller.  The array's contents between calls are never read
 * before being written.
 */
#define GDR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

gdr_status gdr_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                 const float* log_alpha, const void* b, const void* w,
                                 const float* S0, void* o, float* S_final,
                                 int B, int H, int T, int d_k, int d_v, int chunk,
                                 uint32_t flags, void* stream);

/*
 * The same forward over packed variable-length sequences: nseq sequences of
 * any lengths stored back to back (variable-length batches are the practical
 * extension the pages point to: "Gated DeltaNet study notes" §4-3).  Each
 * sequence runs its own recurrence from its own initial state; no state
 * crosses from one sequence to the next.
 *
 *   q, k       : act  [H, T, d_k]   (T = total tokens of all sequences)
 *   v          : act  [H, T, d_v]
 *   log_alpha  : fp32 [H, T, d_k]   or [H, T] with GDR_ALPHA_SCALAR
 *   b          : act  [H, T, d_k]   or [H, T] with GDR_B_SCALAR
 *   w          : act  [H, T, d_v]   or [H, T] with GDR_W_SCALAR
 *   cu_seqlens : int32 [nseq + 1], DEVICE memory: sequence s is tokens
 *                cu_seqlens[s] .. cu_seqlens[s+1]-1 of every head.  The
 *                caller guarantees cu_seqlens[0] = 0, non-decreasing values
 *                and cu_seqlens[nseq] = T (the library cannot check values in
 *                device memory).  Lengths need not be multiples of 64; a
 *                length of 0 copies that sequence's S0 to S_final.
 *   S0         : fp32 [nseq, H, d_k, d_v]; NULL means zeros
 *   o          : as gdr_chunk_fwd, [H, T, d_v]
 *   S_final    : fp32 [nseq, H, d_k, d_v]; NULL means not written; may alias S0
 *   workspace  : required, at least gdr_chunk_fwd_varlen_workspace_bytes()
 *                bytes (chunks of 64: a record per chunk for the producer and
 *                chain kernels of gdr_chunk_fwd, then the chunk tables; the
 *                tokens past a sequence's end in its last chunk are treated as
 *                absent).
 * Supported: bf16 activations, d_k and d_v in {64, 128}; nseq >= 1, H >= 1,
 * T >= 0.  Returns GDR_ERR_UNSUPPORTED otherwise.
 */
size_t gdr_chunk_fwd_varlen_workspace_bytes(int nseq, int H, int T, int d_k, int d_v,
                                            uint32_t flags);

gdr_status gdr_chunk_fwd_varlen(const void* q, const void* k, const void* v,
                                const float* log_alpha, const void* b, const void* w,
                                const float* S0, void* o, float* S_final,
                                const int* cu_seqlens, int nseq, int H, int T,
                                int d_k, int d_v, uint32_t flags, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * One recurrent decode step for N independent sequences (constant memory:
 * the state is updated in place; Q&A page introduction, "Gated DeltaNet-2
 * Review" §3-2 item 1).  Each (n, h) state is read once and written once.
 *
 *   q, k       : act  [N, H, d_k]
 *   v          : act  [N, H, d_v]
 *   log_alpha  : fp32 [N, H, d_k] or [N, H] with GDR_ALPHA_SCALAR
 *   b          : act  [N, H, d_k] or [N, H] with GDR_B_SCALAR
 *   w          : act  [N, H, d_v] or [N, H] with GDR_W_SCALAR
 *   S          : fp32 [N, H, d_k, d_v], read and overwritten with S_t
 *   o          : fp32 (or bf16) [N, H, d_v], written
 * Supported: d_k, d_v in {16, 32, 64, 128}.  All arithmetic is fp32.
 */
gdr_status gdr_decode_step(const void* q, const void* k, const void* v,
                           const float* log_alpha, const void* b, const void* w,
                           float* S, void* o, int N, int H, int d_k, int d_v,
                           uint32_t flags, void* stream);

/*
 * Gate-aware backward of gdr_chunk_fwd for the loss
 *     L = <dO, o> + <dS_final, S_final>,
 * with the erase-side gate gradient (db) and the write-side one (dw)
 * accumulated separately (Q&A page Q4).
 *
 *   inputs as gdr_chunk_fwd, plus
 *   dO         : act  [B, H, T, d_v]
 *   dS_final   : fp32 [B, H, d_k, d_v]; NULL means zero
 *   outputs (fp32, written, never accumulated into):
 *   dq, dk     : [B, H, T, d_k]       dv : [B, H, T, d_v]
 *   dlog_alpha : [B, H, T, d_k] (or [B, H, T] in scalar mode: the sum over
 *                channels)
 *   db         : [B, H, T, d_k] (or [B, H, T])   dw : [B, H, T, d_v] (or [B, H, T])
 *                When b and w are the same scalar buffer (tied gates), the
 *                gradient of that buffer is db + dw.
 *   dS0        : [B, H, d_k, d_v]; may be NULL when not needed.
 *   workspace  : device scratch of at least gdr_chunk_bwd_workspace_bytes()
 *                bytes, owned by the caller; contents on entry are ignored.
 * Part of the work may run on the library's second stream for the device; it
 * waits for the work queued on `stream` before the call and `stream` waits for
 * it before the call's last kernel (event fork and join), so every effect is
 * ordered on `stream` as if it ran there, also under graph capture.  Calls on
 * one device share that second stream.
 * Supported: bf16 or fp32 activations, d_k and d_v each in {16, 32, 64,
 * 128}, chunk 16, 32 or 64 (fp32 activations block with at most 32; results
 * do not depend on the blocking beyond rounding).  Returns
 * GDR_ERR_UNSUPPORTED otherwise.  GDR_GATE_LOGITS needs bf16 activations,
 * chunk 64 and d_k = d_v in {64, 128}.
 */
size_t gdr_chunk_bwd_workspace_bytes(int B, int H, int T, int d_k, int d_v,
                                     int chunk, uint32_t flags);

gdr_status gdr_chunk_bwd(const void* q, const void* k, const void* v,
                         const float* log_alpha, const void* b, const void* w,
                         const float* S0, const void* dO, const float* dS_final,
                         float* dq, float* dk, float* dv, float* dlog_alpha,
                         float* db, float* dw, float* dS0,
                         int B, int H, int T, int d_k, int d_v, int chunk,
                         uint32_t flags, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * The backward of gdr_chunk_fwd_varlen (packed variable-length sequences,
 * "Gated DeltaNet study notes" §4-3), for the same loss: every sequence's
 * gradients depend only on its own tokens, initial state and dS_final.
 *
 *   inputs as gdr_chunk_fwd_varlen ([H, T, ...] token streams, cu_seqlens in
 *   DEVICE memory with the same guarantees), plus
 *   dO         : act  [H, T, d_v]
 *   dS_final   : fp32 [nseq, H, d_k, d_v]; NULL means zero
 *   outputs (fp32, written, never accumulated into):
 *   dq, dk     : [H, T, d_k]       dv : [H, T, d_v]
 *   dlog_alpha, db, dw : [H, T, d_k] / [H, T, d_k] / [H, T, d_v], or [H, T]
 *                in the scalar modes (as gdr_chunk_bwd)
 *   dS0        : [nseq, H, d_k, d_v]; may be NULL.  A sequence of length 0
 *                gets dS0 = dS_final (zero when dS_final is NULL).
 *   workspace  : required, at least gdr_chunk_bwd_varlen_workspace_bytes()
 *                bytes, owned by the caller; contents on entry are ignored.
 * Uses the library's second stream as gdr_chunk_bwd does.
 * Supported: bf16 activations, d_k = d_v = 128 or 64 (chunks of 64).
 * Returns GDR_ERR_UNSUPPORTED otherwise.
 */
size_t gdr_chunk_bwd_varlen_workspace_bytes(int nseq, int H, int T, int d_k, int d_v,
                                            uint32_t flags);

gdr_status gdr_chunk_bwd_varlen(const void* q, const void* k, const void* v,
                                const float* log_alpha, const void* b, const void* w,
                                const float* S0, const void* dO, const float* dS_final,
                                float* dq, float* dk, float* dv, float* dlog_alpha,
                                float* db, float* dw, float* dS0,
                                const int* cu_seqlens, int nseq, int H, int T,
                                int d_k, int d_v, uint32_t flags, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Token-mixer prologue: the element-wise and short-window steps between the
 * caller's linear projections and the recurrence ("Gated DeltaNet study
 * notes" §2 token mixer block design; "Gated DeltaNet-2 Review" §4-3
 * engineering notes), in one pass:
 *   q = L2norm(SiLU(conv(q_pre))),  k = L2norm(SiLU(conv(k_pre))),
 *   v = SiLU(conv(v_pre)),  log_alpha = log(sigmoid(a_pre)) in fp32,
 *   b = sigmoid(b_pre),  w = sigmoid(w_pre).
 * conv is the depthwise causal convolution with 4 taps per channel, zero
 * before the first token of each sequence; L2norm(x) = x / sqrt(sum x^2 +
 * 1e-6) over the head's d_k channels.  All arithmetic is fp32.
 *
 *   q_pre, k_pre : bf16 [B, H, T, d_k]   v_pre : bf16 [B, H, T, d_v]
 *   conv_q, conv_k : fp32 [H, d_k, 4]    conv_v : fp32 [H, d_v, 4]
 *                  taps of channel c of head h: element j weights token t - j
 *   a_pre  : fp32 [B, H, T, d_k] (or [B, H, T] with GDR_ALPHA_SCALAR)
 *   b_pre  : bf16 [B, H, T, d_k] (or [B, H, T] with GDR_B_SCALAR)
 *   w_pre  : bf16 [B, H, T, d_v] (or [B, H, T] with GDR_W_SCALAR)
 *   outputs, written: q, k, v bf16 in the shapes of q_pre, k_pre, v_pre;
 *   log_alpha fp32 shaped as a_pre; b, w bf16 shaped as b_pre, w_pre.  These
 *   are exactly the inputs gdr_chunk_fwd takes with the same gate flags.
 * Outputs must not alias inputs.  Flags: the three gate modes only.
 * Supported: d_k, d_v in {64, 128}; GDR_ERR_UNSUPPORTED otherwise (also for
 * GDR_ACT_F32).
 */
gdr_status gdr_mixer_prologue(const void* q_pre, const void* k_pre, const void* v_pre,
                              const float* conv_q, const float* conv_k, const float* conv_v,
                              const float* a_pre, const void* b_pre, const void* w_pre,
                              void* q, void* k, void* v, float* log_alpha, void* b, void* w,
                              int B, int H, int T, int d_k, int d_v, uint32_t flags,
                              void* stream);

/*
 * Token-mixer epilogue: the recurrent output RMS-normalised and gated before
 * the caller's output projection ("Gated DeltaNet-2 Review" §4-3), per
 * (token, head):
 *   y = o / sqrt(mean(o^2) + 1e-6) * norm_weight * SiLU(g)
 * with the mean over the head's d_v channels, in fp32.
 *
 *   o           : fp32 [B, H, T, d_v] (gdr_chunk_fwd's output)
 *   g           : bf16 [B, H, T, d_v] output-gate logits
 *   norm_weight : fp32 [d_v], shared by the heads
 *   y           : bf16 [B, H, T, d_v], written; must not alias o or g
 * flags must be 0.  Supported: d_v in {64, 128}.
 */
gdr_status gdr_mixer_epilogue(const float* o, const void* g, const float* norm_weight, void* y,
                              int B, int H, int T, int d_v, uint32_t flags, void* stream);

/*
 * Backward of the token-mixer prologue's q, k and v paths and of the
 * epilogue, for training through the block.  (With GDR_GATE_LOGITS the
 * recurrence's backward already returns the gate logits' gradients, so the
 * gate paths need nothing here.)
 *
 * gdr_mixer_prologue_bwd: given dq, dk, dv (fp32 [B, H, T, d], the gradients
 * of the prologue's outputs, e.g. from gdr_chunk_bwd), writes the gradients
 * of the projection outputs dq_pre, dk_pre, dv_pre (fp32, shaped as q_pre,
 * k_pre, v_pre) and of the convolution taps dconv_q, dconv_k, dconv_v (fp32
 * [H, d, 4], summed over the batch and the tokens in a fixed order, so the
 * result is deterministic).  The forward's values are recomputed from q_pre,
 * k_pre, v_pre and the taps.
 * gdr_mixer_epilogue_bwd: given dy (fp32 [B, H, T, d_v]), writes d_o and dg
 * (fp32 [B, H, T, d_v]) and dnorm_weight (fp32 [d_v], summed over all rows
 * in a fixed order).
 * Both need a workspace of gdr_mixer_bwd_workspace_bytes() bytes (one buffer
 * serves both calls on one stream); outputs must not alias inputs; flags
 * must be 0.  Supported: d_k = d_v in {64, 128}, T >= 1.
 */
size_t gdr_mixer_bwd_workspace_bytes(int B, int H, int T, int d_k, int d_v);

gdr_status gdr_mixer_prologue_bwd(const void* q_pre, const void* k_pre, const void* v_pre,
                                  const float* conv_q, const float* conv_k, const float* conv_v,
                                  const float* dq, const float* dk, const float* dv,
                                  float* dq_pre, float* dk_pre, float* dv_pre,
                                  float* dconv_q, float* dconv_k, float* dconv_v,
                                  int B, int H, int T, int d_k, int d_v, uint32_t flags,
                                  void* workspace, size_t workspace_bytes, void* stream);

gdr_status gdr_mixer_epilogue_bwd(const float* o, const void* g, const float* norm_weight,
                                  const float* dy, float* d_o, float* dg, float* dnorm_weight,
                                  int B, int H, int T, int d_v, uint32_t flags,
                                  void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
