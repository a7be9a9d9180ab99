/*
 * lightning_attn.h -- C ABI of the MI355X (gfx950) lightning-attention library.
 *
 * What is computed.  The MiniMax-M1 fact sheet (archdb), "linear / SSM layer
 * configuration" field, describes the lightning layer as linear attention
 * with a fixed per-head exponential decay (ALiBi-style slopes) and a 128x128
 * state per head; its "positional scheme" field says the layer has no RoPE.
 * The CocoLoop explainer ("MiniMax-01 Lightning Attention", section "El
 * enfoque de Lightning Attention") calls it a linear-attention variant that
 * takes attention from O(n^2) to about O(n).  This library computes the
 * causal decayed form of it, per (batch b, head h), with lam = decay[h]:
 *
 *     S_{-1} = kv_in[b,h] (zero if kv_in is NULL)
 *     S_t    = lam * S_{t-1} + k_t^T v_t           (S is d x d, S[key][value])
 *     o_t    = q_t S_t
 *     kv_out[b,h] = S_{N-1}
 *
 * equivalently O = (Q K^T (.) M) V + diag(lam^(t+1)) Q S_{-1} with
 * M[i][j] = lam^(i-j) for i >= j and 0 otherwise (lam^0 = 1, also at lam = 0).
 * No 1/sqrt(d) scale and no normaliser are applied.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers, 16-byte aligned, contiguous.
 *    Q, K, V, O are row-major [B][H][N][d]; states are float32 [B][H][d][d]
 *    (row = key index, column = value index); decay is float32 [H], each
 *    value in [0, 1], shared by every batch entry.
 *  - bf16 means IEEE bfloat16 (1-8-7); results are rounded to nearest even.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls only enqueue work on it and return; there is no host
 *    synchronisation.  A kernel fault surfaces at the caller's next sync.
 *  - The caller owns every buffer.  The library never frees or retains
 *    caller memory.
 *  - kv_in may equal kv_out (in-place state update); otherwise the two must
 *    not overlap.  Every buffer a call writes (out, kv_out, a state pool, a
 *    caller's workspace) must not overlap any other argument; the one
 *    exception is the in-place state.  Overlaps are reported as
 *    LA_ERR_INVALID.
 *  - Arguments are validated before any HIP call, so validation errors are
 *    returned without touching the device.  Nothing is thrown across the ABI.
 *  - The library keeps no state between calls (except the per-device array
 *    of lightning_attn_fwd_noalloc): calls on different streams may run at
 *    once.  Given a caller workspace (or none needed, as in the decode steps,
 *    or the library's own array, as in lightning_attn_fwd_noalloc), a call
 *    allocates, frees, copies and synchronises nothing and issues no memset,
 *    so it can be captured in a HIP graph.
 *
 * Status codes: LA_OK, or one of the LA_ERR_* values below;
 * lightning_attn_strerror() names them.
 */
#ifndef LIGHTNING_ATTN_H
#define LIGHTNING_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LA_OK 0
#define LA_ERR_INVALID 1      /* NULL pointer, size <= 0, bad block/chunk, misaligned pointer, overlap */
#define LA_ERR_UNSUPPORTED 2  /* d not in {64, 128}; dtype/block combination not built; N > 2^24;
                                 B, H, B*H or num_slots*H >= 2^31; B*H*N > 2^48 */
#define LA_ERR_HIP 3          /* a HIP runtime call or kernel launch failed */
#define LA_ERR_NOMEM 4        /* the library's own workspace allocation failed */
#define LA_ERR_WORKSPACE 5    /* caller workspace too small */

#define LA_DTYPE_BF16 0
#define LA_DTYPE_F32 1

/* Flags of lightning_attn_fwd_ex, lightning_attn_fwd_slots, lightning_attn_bwd.
 * LA_FLAG_EXACT: every head by the exact chunked path (chunk aggregates, scan,
 * outputs from the chunk start states), never the warm start described at
 * lightning_attn_fwd (nor its check). */
#define LA_FLAG_EXACT 1u
/* LA_FLAG_SILU_QKV (lightning_attn_fwd_ex and lightning_attn_fwd_slots only):
 * q, k, v are the pre-activation projections; the kernels apply
 * SiLU(x) = x / (1 + e^-x) to every element as its tile arrives in on-chip
 * memory, rounded once to bf16, exactly as if lightning_attn_silu had been
 * run over q, k and v first (the MiniMax-M1 fact sheet, "linear / SSM layer
 * configuration" field: SiLU on Q, K, V), so the activations make no extra
 * pass through HBM and q, k, v are left unchanged.  bf16 inputs and block 64
 * only (LA_ERR_UNSUPPORTED otherwise).  SiLU and the sigmoid gate use the
 * hardware base-2 exponential and reciprocal (about 1 ulp each) in every
 * entry point. */
#define LA_FLAG_SILU_QKV 2u

/*
 * Prefill, bf16 Q/K/V/O, fp32 accumulation and fp32 state.
 *   q, k, v   : bf16 [B][H][N][d]            (read)
 *   decay     : float [H]                    (read)
 *   out       : bf16 [B][H][N][d]            (written)
 *   kv_in     : float [B][H][d][d] or NULL   (read; NULL = zero initial state)
 *   kv_out    : float [B][H][d][d] or NULL   (written; S after the last token)
 *   B, H, N   : >= 1;  d in {64, 128}
 *   block     : intra-block length of the blockwise algorithm, one of
 *               {64, 128, 256}.  The result does not depend on it beyond
 *               rounding (at 64 with the warm start and its check described
 *               below).  64 is the tuned path (the 64-token kernels with LDS
 *               DMA and the warm start); 128 and 256 run a general kernel
 *               that is several times slower.
 * Decays are meant to lie in [0, 1].  With bf16 inputs and block 64, a head
 * with span = ceil(30 ln 2 / -ln lam), rounded up to a multiple of 64, at
 * most half the warm-start chunk (lam^span <= 2^-30; the chunk is
 * lightning_attn_fwd_warm_chunk) is first computed per chunk of that length
 * from the state W_c that the span tokens before the chunk build from zero
 * (the warm start; c0 = the chunk's first token, the first chunk starts from
 * kv_in): the state X_c = S_(c0-span-1) from before those tokens is left
 * out, and it would enter token t of the chunk as lam^(t-c0+span+1) X_c,
 * beside the carried lam^(t-c0+1) W_c.  A check on the device then compares,
 * for every chunk, lam^span max|X_c| with 2^-24 max|W_c| (largest entries):
 * if any chunk exceeds it (a burst of large keys and values just before a
 * window, a window of zeros, NaN or inf), the head is computed again on the
 * exact path, so what is left out never exceeds the fp32 rounding bound of
 * the carried term.  On Gaussian inputs the ratio is about 2^-30 and no head
 * is recomputed; the check and the (then empty) recomputation launches add
 * a few microseconds.  Heads that do not decay within a warm-start chunk,
 * and every other dtype and block, take the exact path from the start.  The
 * _ex entry point with LA_FLAG_EXACT takes the exact path for every head.
 * The result does not depend on the path beyond rounding.
 * Non-finite inputs: a NaN or inf in token t of a head makes that head's
 * later state and output rows non-finite, as in the exact function (the check
 * above never lets the warm start drop such a state); rows of the same block
 * before t may come out non-finite too, as the blocked products meet the
 * value there (0 * NaN).
 * Scratch (decay-power table, per-chunk states and the check's slots, see
 * lightning_attn_fwd_workspace_bytes) is allocated stream-ordered with
 * hipMallocAsync/hipFreeAsync on `stream`.
 */
int lightning_attn_fwd(const void* q, const void* k, const void* v, const float* decay, void* out,
                       const float* kv_in, float* kv_out, int64_t B, int64_t H, int64_t N, int64_t d,
                       int64_t block, void* stream);

/* Same as lightning_attn_fwd with float32 q, k, v and out.  block 64 for d = 128;
 * {64, 128, 256} for d = 64. */
int lightning_attn_fwd_f32(const void* q, const void* k, const void* v, const float* decay, void* out,
                           const float* kv_in, float* kv_out, int64_t B, int64_t H, int64_t N, int64_t d,
                           int64_t block, void* stream);

/* Same as lightning_attn_fwd with bf16 q, k, v and a float32 out: the same
 * kernels as the bf16 path, storing the fp32 accumulator instead of rounding
 * it to bf16 (so bf16 out == RNE(fp32 out) for the same inputs). */
int lightning_attn_fwd_bf16_f32out(const void* q, const void* k, const void* v, const float* decay,
                                   void* out, const float* kv_in, float* kv_out, int64_t B, int64_t H,
                                   int64_t N, int64_t d, int64_t block, void* stream);

/*
 * General prefill entry point behind the three above.
 *   in_dtype, out_dtype : LA_DTYPE_BF16 / LA_DTYPE_F32 (f32 in requires f32 out)
 *   chunk     : tokens per chunk of the chunk-parallel scan; 0 picks the
 *               default (lightning_attn_fwd_chunk); otherwise a positive
 *               multiple of block.  The result does not depend on it beyond
 *               rounding.
 *   warm_chunk: tokens per chunk of the warm-start pass (bf16 inputs, block
 *               64): which heads decay within a chunk is judged against it,
 *               and those heads are computed chunk by chunk at this length;
 *               0 picks the default (lightning_attn_fwd_warm_chunk: with
 *               chunk 0, up to four times the default chunk; with an
 *               explicit chunk, that chunk); otherwise a multiple of 64, at
 *               least the scan's chunk.  Ignored by the other paths.
 *   flags     : 0, or LA_FLAG_EXACT and/or LA_FLAG_SILU_QKV
 *   workspace : device scratch of at least lightning_attn_fwd_workspace_bytes_ex()
 *               bytes, 256-byte aligned, owned by the caller and not used
 *               after the enqueued work completes; NULL = allocate
 *               stream-ordered as lightning_attn_fwd does.
 *   evt_begin, evt_end : optional hipEvent_t (as void*), recorded on `stream`
 *               immediately before and after the kernel that writes every
 *               output row (the dominant kernel): the warm-start pass with
 *               bf16 inputs and block 64, the output pass otherwise; for
 *               timing; NULL = not recorded.
 */
int lightning_attn_fwd_ex(const void* q, const void* k, const void* v, const float* decay, void* out,
                          const float* kv_in, float* kv_out, int64_t B, int64_t H, int64_t N, int64_t d,
                          int64_t block, int in_dtype, int out_dtype, int64_t chunk, int64_t warm_chunk,
                          unsigned int flags, void* workspace, size_t workspace_bytes, void* evt_begin, void* evt_end,
                          void* stream);

/*
 * Prefill with the lightning layer's output steps fused into the kernels
 * that write the output rows (no extra pass over HBM): the MiniMax-M1 fact
 * sheet puts an RMSNorm on the output (its "linear / SSM layer
 * configuration" field) and a sigmoid gate after that norm, before the
 * output projection (its "output gate" field).  Per token t and head h:
 *     o   = the prefill output of lightning_attn_fwd_ex (same arguments)
 *     out = o / sqrt(mean_j(o_j^2) + eps) * gamma[h] * sigmoid(gate_t)
 * the mean over the d features of the token's head row, every factor
 * optional; fp32 until the one rounding of out.
 *   q, k, v   : bf16 [B][H][N][d] (with LA_FLAG_SILU_QKV: pre-activations)
 *   gamma     : float [H][d] or NULL (no norm)
 *   eps       : in [0, 1] (the block norms use 1e-5)
 *   gate      : bf16 [B][H][N][d] or NULL (no gate); sigmoid(x) = 1 / (1 + e^-x)
 *   out       : out_dtype [B][H][N][d] (written; apart from every input)
 *   other arguments as lightning_attn_fwd_ex at block 64 (bf16 inputs)
 * kv_out is the recurrence's final state, as in lightning_attn_fwd_ex (the
 * epilogue touches the outputs only).
 */
int lightning_attn_fwd_fused(const void* q, const void* k, const void* v, const float* decay, const float* gamma,
                             float eps, const void* gate, void* out, const float* kv_in, float* kv_out, int64_t B,
                             int64_t H, int64_t N, int64_t d, int out_dtype, int64_t chunk, int64_t warm_chunk,
                             unsigned int flags, void* workspace, size_t workspace_bytes, void* evt_begin,
                             void* evt_end, void* stream);

/*
 * Prefill into a pool of states (serving: chunked prefill of several
 * requests into their existing states).  The same computation as
 * lightning_attn_fwd_ex with kv_in = kv_out, except that batch row b starts
 * from, and writes its final state back to, pool slot slots[b] (in place).
 *   states    : float [num_slots][H][d][d]           (read and written)
 *   slots     : int32 [B], device memory             (read)
 *   other arguments as lightning_attn_fwd_ex (default chunk, stream-ordered
 *   workspace allocation)
 * A row whose slot lies outside [0, num_slots) starts from a zero state and
 * keeps no final state.  Two rows naming the same slot race (undefined).
 */
int lightning_attn_fwd_slots(const void* q, const void* k, const void* v, const float* decay, void* out,
                             float* states, const int32_t* slots, int64_t B, int64_t H, int64_t N, int64_t d,
                             int64_t num_slots, int64_t block, int in_dtype, int out_dtype, unsigned int flags,
                             void* stream);

/*
 * Backward pass of the prefill: the gradients of a loss L given
 * dout = dL/dO and dkv_out = dL/d(kv_out).  This is the derivative of the
 * recurrence above (the pages print no backward pass).  With the adjoint
 * G_t = dL/dS_t = lam G_{t+1} + q_t^T dout_t, G_{N-1} = dkv_out + q_{N-1}^T dout_{N-1}:
 *     dq_t = dout_t S_t^T,  dk_t = v_t G_t^T,  dv_t = k_t G_t,  dkv_in = lam G_0.
 * Each of dq, dk, dv is computed as a prefill-shaped pass (dk and dv run the
 * tokens last first) with the kernels of lightning_attn_fwd_ex at block 64.
 * With bf16 inputs the heads that decay within a chunk take the warm start
 * and its check, as in lightning_attn_fwd, in every pass (for dk and dv on
 * the adjoint state); a head that fails the check in a pass is computed
 * again on the exact path for that pass.  With bf16 inputs the dk and dv
 * passes share their kernel launches (each keeps its own chunk states and
 * check slots in the workspace).
 *   q, k, v, dout : in_dtype [B][H][N][d]          (read)
 *   decay         : float [H]                      (read)
 *   kv_in         : float [B][H][d][d] or NULL     (read: the forward's initial state; NULL = zero)
 *   dkv_out       : float [B][H][d][d] or NULL     (read: dL/d(kv_out); NULL = zero)
 *   dq, dk, dv    : out_dtype [B][H][N][d]         (written)
 *   dkv_in        : float [B][H][d][d] or NULL     (written: dL/d(kv_in); may be dkv_out itself)
 *   B, H, N >= 1; d in {64, 128}; in_dtype / out_dtype as lightning_attn_fwd_ex
 *   (bf16 in: bf16 or fp32 out; fp32 in: fp32 out); flags: 0 or LA_FLAG_EXACT
 *   workspace     : device scratch of at least lightning_attn_bwd_workspace_bytes()
 *                   bytes, 256-byte aligned; NULL = allocated stream-ordered
 * Outputs may not overlap inputs or each other.
 */
int lightning_attn_bwd(const void* q, const void* k, const void* v, const float* decay, const void* dout,
                       const float* kv_in, const float* dkv_out, void* dq, void* dk, void* dv, float* dkv_in,
                       int64_t B, int64_t H, int64_t N, int64_t d, int in_dtype, int out_dtype, unsigned int flags,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of scratch lightning_attn_bwd needs for these sizes (0 on invalid
 * arguments): the decay table, two sets of chunk states (B*H*ceil(N/L) d x d
 * fp32 each, L the default chunk at block 64) and two B*H d x d fp32 states. */
size_t lightning_attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d);

/* Chunk length the library uses for (B, H, N, block) when `chunk` is 0, or
 * `chunk` itself when it is valid; -1 on invalid arguments.  The default
 * starts at 16384 tokens and halves while B*H*ceil(N/chunk) < 2048, down to
 * max(block, 256), then is capped at N rounded up to a whole block. */
int64_t lightning_attn_fwd_chunk(int64_t B, int64_t H, int64_t N, int64_t block, int64_t chunk);

/* Warm-start chunk the library uses for (B, H, N, block, chunk, warm_chunk)
 * (see lightning_attn_fwd_ex); -1 on invalid arguments.  The default with
 * chunk 0 doubles the default chunk, at most twice, while the warm-start pass
 * keeps at least 1024 workgroups (B*H*ceil(N/warm_chunk) >= 1024) and the
 * chunk fits in N rounded up to whole chunks: longer chunks let more heads
 * take the warm start and shorten its warm-up windows relative to the chunk,
 * while the exact path keeps the shorter chunks.  The pooled prefill and the
 * backward use the default. */
int64_t lightning_attn_fwd_warm_chunk(int64_t B, int64_t H, int64_t N, int64_t block, int64_t chunk,
                                      int64_t warm_chunk);

/* Bytes of scratch the prefill needs for these sizes at the default chunk
 * (lightning_attn_fwd, or lightning_attn_fwd_ex with chunk 0); 0 on invalid
 * arguments.  Layout, each part starting 256-byte aligned: the decay-power
 * table; B*H*ceil(N/chunk) float32 d x d chunk states; the warm-start check's
 * slots (8 floats per (b, h) and chunk); and, as the last B*H*4 bytes, one
 * int32 per (b, h), row-major: 1 when the check sent that head to the exact
 * path in the call, else 0 (written by every bf16 block-64 call without
 * LA_FLAG_EXACT). */
size_t lightning_attn_fwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int64_t block);

/* The same for lightning_attn_fwd_ex with an explicit chunk (0 = the
 * default, as above). */
size_t lightning_attn_fwd_workspace_bytes_ex(int64_t B, int64_t H, int64_t N, int64_t d, int64_t block,
                                             int64_t chunk);

/*
 * One decode step for B sequences (N = 1 of the recurrence above):
 *     S <- lam * S + k^T v ;   o = q S
 *   q, k, v   : bf16 [B][H][d]              (read)
 *   decay     : float [H]                   (read)
 *   out       : bf16 [B][H][d]              (written)
 *   kv_in     : float [B][H][d][d] or NULL  (read; NULL = zero state)
 *   kv_out    : float [B][H][d][d] or NULL  (written; may equal kv_in)
 *   B, H >= 1; d in {64, 128}
 */
int lightning_attn_decode_step(const void* q, const void* k, const void* v, const float* decay, void* out,
                               const float* kv_in, float* kv_out, int64_t B, int64_t H, int64_t d,
                               void* stream);

/*
 * Decode step over a pool of states (serving): the same step as
 * lightning_attn_decode_step, with batch row b reading and writing, in
 * place, the state of pool slot slots[b].  The recurrence has no position
 * term, so requests at different positions share one call.
 *   q, k, v   : bf16 [B][H][d]                       (read)
 *   decay     : float [H]                            (read)
 *   out       : bf16 [B][H][d]                       (written)
 *   states    : float [num_slots][H][d][d]           (read and written in place)
 *   slots     : int32 [B], device memory             (read)
 *   B, H, num_slots >= 1; d in {64, 128}
 * A row whose slot lies outside [0, num_slots) is idle: its output row is
 * written as zeros and no state is touched.  Two rows naming the same slot
 * race (undefined result).  Slots are device data, so their range is checked
 * by the kernel, not before the launch.
 */
int lightning_attn_decode_slots(const void* q, const void* k, const void* v, const float* decay, void* out,
                                float* states, const int32_t* slots, int64_t B, int64_t H, int64_t d,
                                int64_t num_slots, void* stream);

/*
 * The lightning layer's elementwise steps either side of the core (the
 * MiniMax-M1 fact sheet: SiLU on Q, K, V and an RMSNorm on the output, in its
 * "linear / SSM layer configuration" field; a sigmoid gate after that norm,
 * before the output projection, in its "output gate" field).  The norm is
 * taken per head over the d features of a token, o / sqrt(mean(o^2) + eps)
 * times gamma[h]; eps = 1e-5 matches the block norms.
 *
 * Decode step with them fused (no extra memory pass): the step of
 * lightning_attn_decode_slots (slots == NULL: row b uses state row b, and
 * num_slots >= B), with
 *   silu != 0 : q, k, v <- SiLU(q), SiLU(k), SiLU(v) as they are read
 *   gamma     : float [H][d] or NULL (no norm)
 *   gate      : bf16 [B][H][d] or NULL (no gate): o <- o * sigmoid(gate)
 *   eps       : in [0, 1]
 */
int lightning_attn_decode_fused(const void* q, const void* k, const void* v, const float* decay, void* out,
                                float* states, const int32_t* slots, int64_t num_slots, int silu,
                                const float* gamma, float eps, const void* gate, int64_t B, int64_t H, int64_t d,
                                void* stream);

/*
 * Decode over several layers' states in one launch (serving: the lightning
 * layers of a model, each with its own state pool; the MiniMax-01 abstract on
 * the aitopics.org "Zheng, Lin" page gives inference contexts of up to 4M
 * tokens, for which the per-layer recurrent states are the whole decode-time
 * working set).  Layer l steps its rows exactly as lightning_attn_decode_fused
 * would with that layer's tensors:
 *   q, k, v    : bf16 [num_layers][B][H][d]              (read)
 *   decay      : float [num_layers][H]                   (read)
 *   out        : bf16 [num_layers][B][H][d]              (written)
 *   states     : float [num_layers][num_slots][H][d][d]  (read and written in place)
 *   slots      : int32 [num_layers][B], device memory, or NULL: row b of
 *                layer l uses slot slots[l][b] of layer l's pool (out of
 *                range: idle row, zero output, no state touched; a layer
 *                with no ready token for a row marks it idle), or row b
 *                itself when NULL (then num_slots >= B)
 *   silu, eps  : as lightning_attn_decode_fused
 *   gamma      : float [num_layers][H][d] or NULL (no norm)
 *   gate       : bf16 [num_layers][B][H][d] or NULL (no gate)
 *   num_layers, B, H, num_slots >= 1; d in {64, 128}
 * Rows of different layers never share a state.  Two rows of one layer
 * naming the same slot race (undefined).
 */
int lightning_attn_decode_layers(const void* q, const void* k, const void* v, const float* decay, void* out,
                                 float* states, const int32_t* slots, int64_t num_layers, int64_t B, int64_t H,
                                 int64_t d, int64_t num_slots, int silu, const float* gamma, float eps,
                                 const void* gate, void* stream);

/*
 * Prefill epilogue as its own pass (the block-64 prefill kernel has no room
 * to take it in): out = RMSNorm_head(o) * gamma[h] * sigmoid(gate).
 *   o      : o_dtype (LA_DTYPE_BF16 or LA_DTYPE_F32) [B][H][N][d]   (read)
 *   gate   : bf16 [B][H][N][d] or NULL (no gate)                   (read)
 *   gamma  : float [H][d] or NULL (no norm)                        (read)
 *   out    : bf16 [B][H][N][d] (written; may be o itself when o is bf16)
 */
int lightning_attn_norm_gate(const void* o, int o_dtype, const void* gate, const float* gamma, float eps, void* out,
                             int64_t B, int64_t H, int64_t N, int64_t d, void* stream);

/* Prefill prologue as its own pass: x <- SiLU(x) over n bf16 elements in place
 * (apply to Q, K and V before lightning_attn_fwd).  0 <= n <= 2^44; n = 0 is
 * a no-op. */
int lightning_attn_silu(void* x, int64_t n, void* stream);

/*
 * Prefill that allocates nothing, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the computation of lightning_attn_fwd_ex at block 64,
 * with its workspace (decay table and chunk states) in a device array of
 * LA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends.  The caller passes inputs and outputs as for
 * lightning_attn_fwd_ex; `stream` must belong to the current device
 * (LA_ERR_INVALID otherwise).
 *   chunk      : 0 = the default chunk (lightning_attn_fwd_chunk at block 64),
 *                doubled until the chunk states fit the array; otherwise as in
 *                lightning_attn_fwd_ex
 *   warm_chunk : 0 = the default warm-start chunk of lightning_attn_fwd_ex
 *                (chunk 0), but at least the chunk; otherwise as there
 * Returns LA_ERR_WORKSPACE when the workspace for these sizes (see
 * lightning_attn_fwd_workspace_bytes_ex) exceeds LA_NOALLOC_SCRATCH_BYTES, with
 * nothing enqueued.  The array is shared by every call on a GPU and keeps the
 * last call's contents: calls that overlap in time on one GPU (two streams,
 * two threads) race and give undefined results; calls ordered on one stream
 * do not.  Every byte a call reads from the array it has written before.
 */
#define LA_NOALLOC_SCRATCH_BYTES (96u * 1024u * 1024u)
int lightning_attn_fwd_noalloc(const void* q, const void* k, const void* v, const float* decay, void* out,
                               const float* kv_in, float* kv_out, int64_t B, int64_t H, int64_t N, int64_t d,
                               int in_dtype, int out_dtype, int64_t chunk, int64_t warm_chunk, unsigned int flags,
                               void* stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* lightning_attn_strerror(int status);

/* HIP runtime version the library is running against (hipRuntimeGetVersion),
 * written to *version; returns LA_OK or LA_ERR_HIP / LA_ERR_INVALID. */
int lightning_attn_runtime_version(int* version);

#ifdef __cplusplus
}
#endif

#endif /* LIGHTNING_ATTN_H */
