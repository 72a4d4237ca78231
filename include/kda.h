/*
 * kda.h -- C ABI of the KDA (Kimi Delta Attention) library for MI355X (gfx950).
 *
 * The library runs the gated delta-rule recurrence of Kimi Delta Attention on
 * one GPU. Per sequence b and head h it keeps a fixed-size fp32 state S
 * (d_k x d_v) and, per token t:
 *
 *   short conv + SiLU:   x~ = SiLU(w0 x_{t-3} + w1 x_{t-2} + w2 x_{t-1} + w3 x_t)
 *                        for every channel of q, k and v (width-4, causal,
 *                        depthwise, no bias; a 3-token ring of raw inputs
 *                        carries the history between calls)
 *   L2 normalisation:    q^ = q~ / sqrt(|q~|^2 + 1e-6), same for k (per head,
 *                        over d_k); v^ = v~
 *   decay:               S' = Diag(exp(g_t)) S_{t-1}   (g: log decay per key channel)
 *   delta + rank-1:      S_t = S' + beta_t k^ (v^ - S'^T k^)^T
 *   readout:             o_t = S_t^T q^
 *
 * Sources: "KV缓存从11.25GB缩到0.21GB：WARP中Kimi Delta Attention线性注意力原理剖析",
 * section "KDA 递推公式先衰减再差分" (the three update steps, in-kernel L2
 * normalisation, the width-4 short convolution with its 3-token ring kept as
 * session state) and section "414MB 的 KDA 状态从哪来" (state size independent
 * of context length); "为什么 Kimi K3 敢把 KV Cache 扔掉？一篇讲透 GPT-2 到 K3 的架构
 * 进化", section 7 (the Kimi Linear update with Diag(alpha)) and section 5
 * (the chunkwise-parallel prefill).
 *
 * Conventions for every call:
 *  - Pointers named as device buffers are HIP device pointers, densely
 *    packed in the layouts given; the caller owns them. q, k, v, o and the
 *    ring need the alignment of their element type, g and beta 4 bytes;
 *    conv_w, S (s_mem), ring_mem and the prefill workspace 16 bytes.
 *  - Calls are asynchronous on the given stream (NULL = the default stream)
 *    and never synchronise the host. A kernel fault surfaces at the caller's
 *    next synchronisation.
 *  - Arguments are validated before anything is enqueued. On any error the
 *    call returns a negative kda_status, enqueues nothing and leaves the
 *    state untouched; kda_last_error() then describes the problem.
 *  - No C++ exception crosses this boundary.
 *  - A state handle must not be used from two streams at once.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID = -1,     /* bad argument: NULL pointer, size, alignment, flag */
  KDA_ERR_UNSUPPORTED = -2, /* valid but not built: e.g. d_k = 96 */
  KDA_ERR_HIP = -3,         /* a HIP runtime call failed (message has the HIP error) */
  KDA_ERR_OOM = -4          /* device allocation failed */
} kda_status;

/* Element type of the token inputs q, k, v, of the output o and of the conv
 * ring. The state S, g, beta and the conv weights are always fp32. */
typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

typedef struct {
  int32_t batch;      /* B: independent sequences, >= 1 */
  int32_t heads;      /* H, >= 1 */
  int32_t d_k;        /* key width per head: 16, 32, 64 or 128 */
  int32_t d_v;        /* value width per head: 16, 32, 64 or 128 */
  int32_t conv_width; /* must be 4 */
  int32_t io;         /* a kda_dtype value: dtype of q, k, v, o and the ring
                         (a plain integer so that any value a caller passes is
                         read and rejected as an error, not as an enum) */
} kda_dims;

/* Flags for kda_conv_prologue / kda_decode_step / kda_chunk_prefill. */
#define KDA_F_SKIP_CONV 1u /* q, k, v are already convolved and activated:
                              no conv, no SiLU, the ring is neither read nor written */
#define KDA_F_SKIP_L2 2u   /* q, k are already unit-normalised: no L2 step */
#define KDA_F_SCALAR_G 4u  /* kda_decode_step / kda_chunk_prefill only: g holds one
                              log-decay per (sequence, token, head), shared by every
                              key channel of the head (the scalar alpha of Gated
                              DeltaNet): g is [B][H] for a decode step and [B][T][H]
                              for a prefill. Source: "为什么 Kimi K3 敢把 KV Cache
                              扔掉？…", section 6 (Gated Delta Net: one decay per
                              token or head) and section 7 (KDA refines it to one
                              per channel). The result equals the per-channel call
                              with g repeated over d_k. */
#define KDA_F_RAW_GATES 8u /* kda_decode_step / kda_chunk_prefill only: g and beta hold
                              the raw gate projections a and b (any real values) and
                              the kernels form the decay g = log(sigmoid(a)) (alpha =
                              sigmoid(a) in (0, 1)) and beta = sigmoid(b) themselves.
                              Combines with KDA_F_SCALAR_G (then a is [B][T][H]).
                              Any a that is not NaN is accepted (a = -inf gives
                              g = -inf: the rows are cleared).
                              Source: "为什么 Kimi K3 敢把 KV Cache 扔掉？…", section 6:
                              the Alpha/Beta projection sets the forgetting and update
                              strengths, alpha in [0, 1]; the squashing by a sigmoid
                              is a reading (no formula is printed). */

/* Opaque per-layer session state: S and the conv ring for B sequences. */
typedef struct kda_state kda_state;

/* Channel count of the conv ring / weights: Ctot = H * (2*d_k + d_v).
 * Channel order is q | k | v, each head-major: q channel of (h, i) is
 * h*d_k + i, k channel is H*d_k + h*d_k + i, v channel is 2*H*d_k + h*d_v + j. */

/* Bytes of the recurrent state: B*H*d_k*d_v*4. If ring_bytes is not NULL it
 * receives the ring size B*3*Ctot*sizeof(io). Neither depends on the number
 * of tokens processed (the state has a fixed size whatever the context
 * length: section "Kimi Delta Attention 把注意力状态压成固定大小").
 * Returns 0 for invalid or unsupported dims. */
size_t kda_state_bytes(const kda_dims* dims, size_t* ring_bytes);

/* Creates a state handle for dims: the per-head state S and the conv ring,
 * the session state a decode step carries from token to token. Source: "KV缓存
 * 从11.25GB缩到0.21GB：…", section "Kimi Delta Attention 把注意力状态压成固定大小"
 * (a fixed-size state per head instead of a growing cache) and section "KDA
 * 递推公式先衰减再差分" (the 3-token ring of raw projections is kept as session
 * state between calls).
 *  s_mem:    device buffer of kda_state_bytes() bytes, layout S[B][H][d_k][d_v]
 *            fp32, or NULL to let the library allocate it (hipMalloc).
 *  ring_mem: device buffer of ring_bytes, layout ring[B][3][Ctot] in the io
 *            dtype (tap 0 = token t-3, tap 2 = token t-1), or NULL to allocate.
 * Caller-provided buffers are never freed by the library. The contents start
 * uninitialised: call kda_state_reset before the first token.
 * Errors: KDA_ERR_INVALID (NULL out, misaligned buffer), KDA_ERR_UNSUPPORTED
 * (dims), KDA_ERR_OOM. */
kda_status kda_state_alloc(const kda_dims* dims, void* s_mem, void* ring_mem,
                           kda_state** out);

/* Zeroes S and the ring of the listed sequences (a sequence start: an empty
 * state and no conv history; source: section "KDA 递推公式先衰减再差分", the
 * zero history before a sequence's first token).
 * seq_ids is a HOST array of n sequence indices in [0, B); seq_ids = NULL
 * resets all B sequences (n is then ignored). The zeroing is done by a fill
 * kernel on the stream (no hipMemsetAsync), so it may be graph-captured.
 * Errors: KDA_ERR_INVALID (NULL state, n < 0, index out of range). */
kda_status kda_state_reset(kda_state* st, const int32_t* seq_ids, int32_t n,
                           hipStream_t stream);

/* Frees the handle, and the buffers the library allocated for it (S and the
 * ring when it allocated them, its prefill workspace). NULL is a no-op. */
void kda_state_free(kda_state* st);

/* Device views of the state (for checkpointing: copy out to save, copy in
 * to restore; the ring belongs to the saved session as much as S, section
 * "KDA 递推公式先衰减再差分"). NULL for a NULL handle. */
float* kda_state_S(kda_state* st);
void* kda_state_ring(kda_state* st);
kda_status kda_state_get_dims(const kda_state* st, kda_dims* out);

/* The activations the recurrence consumes, for T tokens of B sequences.
 *  q, k:  [B][T][H][d_k] raw projections (io dtype); v: [B][T][H][d_v].
 *  conv_w: [Ctot][4] fp32, tap 3 multiplies the current token.
 *  ring:  [B][3][Ctot] io dtype, read as the history before token 0 and
 *         advanced to the last three raw tokens (in place).
 *  q_out, k_out: [B][T][H][d_k] fp32; v_out: [B][T][H][d_v] fp32.
 * Writes q^, k^ (conv, SiLU, L2) and v^ (conv, SiLU). With KDA_F_SKIP_CONV
 * the inputs are copied through (conv_w and ring may be NULL); with
 * KDA_F_SKIP_L2 q and k are not normalised; KDA_F_SCALAR_G (no g here) is
 * rejected with KDA_ERR_INVALID. T = 0 is a no-op.
 * Source: section "KDA 递推公式先衰减再差分" (short conv, SiLU, L2). */
kda_status kda_conv_prologue(const kda_dims* dims, int32_t T, const void* q,
                             const void* k, const void* v, const float* conv_w,
                             void* ring, float* q_out, float* k_out, float* v_out,
                             uint32_t flags, hipStream_t stream);

/* One decode token for all B sequences of the state, fused in one pass over S:
 * conv + SiLU + L2 on this token, decay, delta read, rank-1 write, readout.
 *  q, k: [B][H][d_k] raw projections (io dtype); v: [B][H][d_v].
 *  g:    [B][H][d_k] fp32 natural-log decay (-inf allowed: clears the rows);
 *        [B][H] with KDA_F_SCALAR_G.
 *  beta: [B][H] fp32.
 *  conv_w: [Ctot][4] fp32 (NULL allowed with KDA_F_SKIP_CONV).
 *  o:    [B][H][d_v] io dtype (written).
 * S and the ring are updated in place.
 * Source: section "KDA 递推公式先衰减再差分", steps (1)-(3). */
kda_status kda_decode_step(kda_state* st, const void* q, const void* k,
                           const void* v, const float* g, const float* beta,
                           const float* conv_w, void* o, uint32_t flags,
                           hipStream_t stream);

/* Device workspace that kda_chunk_prefill needs for `chunk` and T tokens of
 * this state's dims, or 0 if the arguments are invalid. Passing a smaller
 * (but non-zero) workspace makes the call process T in several segments. */
size_t kda_prefill_workspace_bytes(const kda_dims* dims, int32_t T, int32_t chunk);

/* T tokens for all B sequences, chunkwise-parallel, continuing from the
 * current S and ring and leaving them at token T (same result as T decode
 * steps up to rounding).
 *  q, k: [B][T][H][d_k] raw (io dtype); v: [B][T][H][d_v].
 *  g:    [B][T][H][d_k] fp32; precondition: g <= 0 and not NaN. Any such
 *        value is handled, -inf included (it clears the rows, as in a
 *        decode step): every decay factor the kernels form is the
 *        exponential of a sum of decays of one sign, bounded by 1, except
 *        the factored diagonal tiles of 16-token blocks whose decay stays
 *        within 64 on every key channel (others are formed term by term).
 *        [B][T][H] with KDA_F_SCALAR_G (same precondition).
 *  beta: [B][T][H] fp32.  conv_w: [Ctot][4] fp32.
 *  o:    [B][T][H][d_v] io dtype (written).
 *  chunk: 16, 32 or 64 (64 recommended). T need not be a multiple of chunk.
 *  workspace: device buffer of workspace_bytes, or NULL to use a buffer the
 *        state handle allocates on first use (and keeps until kda_state_free).
 *        With NULL the call allocates (hipMalloc) whenever the handle's buffer
 *        is smaller than the call needs (up to 2 GiB; then T runs in
 *        segments): the first such call, and any later one that needs more,
 *        frees the old buffer and allocates the new one, which synchronises
 *        the host with the device and cannot be captured in a HIP graph. Pass
 *        a workspace (or use kda_chunk_prefill_noalloc) to avoid both.
 * With io = bf16 the contractions run on bf16 MFMA with fp32 accumulation and
 * an fp32 state; with io = fp32 they run on fp32 MFMA.
 * Source: "为什么 Kimi K3 敢把 KV Cache 扔掉？…", section 5 (chunks with
 * attention-like work inside, the state handed from chunk to chunk, the WY
 * representation) and section 6 (cumulative in-chunk decay). */
kda_status kda_chunk_prefill(kda_state* st, int32_t T, const void* q,
                             const void* k, const void* v, const float* g,
                             const float* beta, const float* conv_w, void* o,
                             int32_t chunk, void* workspace, size_t workspace_bytes,
                             uint32_t flags, hipStream_t stream);

/* Size of the fixed device scratch of kda_chunk_prefill_noalloc (64 MiB). */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)

/* kda_chunk_prefill for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. Same arguments and results as kda_chunk_prefill, without the
 * workspace: the call neither allocates nor frees anything (no hipMalloc,
 * hipFree or allocating library routine). Its workspace is a fixed array of
 * KDA_NOALLOC_SCRATCH_BYTES in device memory, one per GPU, held by the
 * library from its first use on that GPU until the process ends; T is
 * processed in as many segments as that array needs (one chunk of all
 * B * H heads must fit: 74,240 bytes per head and sequence at chunk 64,
 * d_k = d_v = 128, bf16, i.e. up to 904 of them).
 * Every call on a GPU shares that GPU's array: calls that overlap on one
 * GPU (two streams, two threads) race and must not be issued. The array's
 * contents on entry do not matter. The stream must belong to the current
 * device.
 * Errors: as kda_chunk_prefill, plus KDA_ERR_UNSUPPORTED when one chunk of
 * the state's sequences and heads needs more than the array holds, and
 * KDA_ERR_INVALID when the stream belongs to another device. */
kda_status kda_chunk_prefill_noalloc(kda_state* st, int32_t T, const void* q, const void* k,
                                     const void* v, const float* g, const float* beta,
                                     const float* conv_w, void* o, int32_t chunk,
                                     uint32_t flags, hipStream_t stream);

/* Output gate after the readout: a gated RMSNorm of each (sequence, token,
 * head) row of d_v readout values,
 *   out = x / sqrt(mean over d_v of x^2 + eps) * norm_w * sigmoid(gate).
 *  x:      [B][T][H][d_v] io dtype (e.g. the o of kda_chunk_prefill).
 *  gate:   [B][T][H][d_v] io dtype, the gate pre-activations.
 *  norm_w: [d_v] fp32, one weight vector shared by all heads.
 *  eps:    finite and > 0.
 *  out:    [B][T][H][d_v] io dtype; may be x itself (in place), must not
 *          otherwise overlap x or gate.
 * x, gate, out and norm_w must be 16-byte aligned. T = 0 is a no-op. Only the
 * dims' batch, heads, d_v and io are used.
 * Source: the WARP engine lists a gated RMSNorm beside its KDA decode step
 * ("KV缓存从11.25GB缩到0.21GB：…", section "相关源码与文档导航"), and "为什么 Kimi
 * K3 敢把 KV Cache 扔掉？…" section 6 puts a gate on the output that rescales
 * features; neither prints the formula: this is the plain reading of the two
 * (per-head RMSNorm over d_v, sigmoid gate).
 * Errors: KDA_ERR_INVALID (NULL or misaligned pointer, T < 0, eps),
 * KDA_ERR_UNSUPPORTED (dims). */
kda_status kda_gated_rmsnorm(const kda_dims* dims, int32_t T, const void* x, const void* gate,
                             const float* norm_w, float eps, void* out, hipStream_t stream);

/* kda_decode_step with the output gate of kda_gated_rmsnorm fused into the
 * readout: o receives the gated RMSNorm of S^T q^ (computed from the fp32
 * readout, before any rounding to the io dtype).
 *  gate:   [B][H][d_v] io dtype; norm_w: [d_v] fp32; eps finite and > 0.
 * Everything else as kda_decode_step. */
kda_status kda_decode_step_gated(kda_state* st, const void* q, const void* k,
                                 const void* v, const float* g, const float* beta,
                                 const float* conv_w, const void* gate, const float* norm_w,
                                 float eps, void* o, uint32_t flags, hipStream_t stream);

/* Device workspace with which kda_chunk_backward takes all T tokens in one
 * pass (0 if the arguments are invalid): per (chunk, sequence, head) a
 * scratch block of the chunk's intermediate products, plus the entering
 * state and the leaving-state gradient of every chunk, all fp32. About
 * 3.5 GB for B = 1, T = 4096, 96 heads of 128 x 128, chunk 64 (and 451 GB
 * for 16 sequences of 32768 tokens: see kda_backward_workspace_min_bytes). */
size_t kda_backward_workspace_bytes(const kda_dims* dims, int32_t T, int32_t chunk);

/* The least workspace kda_chunk_backward accepts for T tokens and `chunk`
 * (0 if the arguments are invalid). With less than
 * kda_backward_workspace_bytes the call takes the chunks in ranges of L
 * (the longest that fits): L chunks' blocks, the fp32 state
 * [B][H][d_k][d_v] entering every range but the first, and one carried
 * state gradient, i.e. L * (one chunk's blocks) + ceil(nc / L) * (one
 * state) bytes for nc = ceil(T / chunk) chunks; this returns the least of
 * that over L. About 13.4 GB for 16 sequences of 32768 tokens, 96 heads
 * of 128 x 128, chunk 64 (L = 8). */
size_t kda_backward_workspace_min_bytes(const kda_dims* dims, int32_t T, int32_t chunk);

/* Gradient of the recurrence (decay, delta read, rank-1 write, readout) for
 * training, chunkwise: for the forward pass that kda_chunk_prefill runs with
 * KDA_F_SKIP_CONV | KDA_F_SKIP_L2 from the entering state S0, and the loss
 * gradients dO of its readouts and dST of its final state, returns the
 * gradients of its activations, decay, beta and entering state. The
 * prologue (conv, SiLU, L2) is not part of it.
 *  q, k:  [B][T][H][d_k] q^, k^ as the recurrence consumes them (io dtype);
 *  v:     [B][T][H][d_v] v^;
 *  g:     [B][T][H][d_k] fp32 log-decay, finite and <= 0 (any such value: a
 *         chunk whose decay exceeds 60 on some channel takes exponentials of
 *         non-positive differences, the others products of two factors
 *         within 1e+-26);
 *  beta:  [B][T][H] fp32;
 *  S0:    [B][H][d_k][d_v] fp32 entering state, or NULL for zero;
 *  dO:    [B][T][H][d_v] io dtype;  dST: [B][H][d_k][d_v] fp32, or NULL for zero;
 *  dq, dk: [B][T][H][d_k] io dtype; dv: [B][T][H][d_v] io dtype;
 *  dg:    [B][T][H][d_k] fp32;  dbeta: [B][T][H] fp32;
 *  dS0:   [B][H][d_k][d_v] fp32, or NULL (not written).
 * q, k, v, g, dO, S0, dST and dS0 must be 16-byte aligned (the other
 * pointers the alignment of their element type). workspace: device buffer of
 * workspace_bytes >= kda_backward_workspace_min_bytes (16-byte aligned,
 * contents on entry ignored). With kda_backward_workspace_bytes or more the
 * chunks are taken in one pass; with less, in ranges: a first pass over the
 * ranges keeps the state entering each (the forward part is then computed
 * twice per range but the last), then the ranges are taken from the last to
 * the first, each handing the gradient of its entering state to the one
 * before. The results are bitwise those of the one-pass call.
 * flags must be 0. chunk: 16, 32 or 64; T need not be a multiple of it.
 * T = 0 writes dS0 = dST (zero if dST is NULL). All arithmetic is fp32.
 * The forward pass is recomputed inside (the entering state of every chunk
 * is kept in the workspace), so the call needs no saved activations beyond
 * its inputs. Outputs must not overlap the inputs.
 * Source: "为什么 Kimi K3 敢把 KV Cache 扔掉？…", section 5: chunking is how
 * the recurrence is trained in parallel (the state handed from chunk to
 * chunk, the WY representation inside a chunk); section 6 (cumulative
 * in-chunk decay). The gradient formulas are derived by reverse-mode
 * differentiation of that chunked form; the pages print none.
 * Errors: KDA_ERR_INVALID (NULL or misaligned pointer, T < 0, flags, small
 * workspace), KDA_ERR_UNSUPPORTED (dims, chunk). */
kda_status kda_chunk_backward(const kda_dims* dims, int32_t T, const void* q,
                              const void* k, const void* v, const float* g,
                              const float* beta, const float* S0, const void* dO,
                              const float* dST, void* dq, void* dk, void* dv, float* dg,
                              float* dbeta, float* dS0, int32_t chunk, void* workspace,
                              size_t workspace_bytes, uint32_t flags, hipStream_t stream);

/* Device workspace that kda_prologue_backward needs: the per-32-token-segment
 * conv-weight gradients, B * ceil(T / 32) * Ctot * 16 bytes (0 for invalid
 * arguments; 0 for T = 0). */
size_t kda_prologue_backward_workspace_bytes(const kda_dims* dims, int32_t T);

/* Gradient of the prologue (the width-4 causal conv, SiLU, and the L2
 * normalisation of q and k, as kda_conv_prologue computes them) for
 * training: from the gradients of q^, k^, v^ (e.g. those kda_chunk_backward
 * returns) to those of the raw projections, the conv weights and the ring's
 * history. The ring that the forward writes (the last three raw tokens) is
 * not differentiated.
 *  q, k:  [B][T][H][d_k] raw projections (io dtype); v: [B][T][H][d_v];
 *  conv_w: [Ctot][4] fp32 (16-byte aligned);
 *  ring:  [B][3][Ctot] io dtype, the history read before token 0, or NULL
 *         for zeros;
 *  dq_hat, dk_hat: [B][T][H][d_k] io dtype; dv_hat: [B][T][H][d_v];
 *  dq, dk: [B][T][H][d_k] io dtype (written); dv: [B][T][H][d_v];
 *  dconv_w: [Ctot][4] fp32 (written, 16-byte aligned);
 *  dring: [B][3][Ctot] fp32 (written), or NULL.
 * q, k, v, ring, dq_hat, dk_hat and dv_hat must be 16-byte aligned (the
 * outputs dq, dk, dv the alignment of their element type).
 * workspace: kda_prologue_backward_workspace_bytes (16-byte aligned). flags
 * must be 0. All arithmetic is fp32; the weight gradient is summed in a
 * fixed order (bitwise reproducible). T = 0 writes zero dconv_w and dring.
 * Source: "KV缓存从11.25GB缩到0.21GB：…", section "KDA 递推公式先衰减再差分"
 * (the short conv with SiLU before q/k/v, the L2 normalisation of q and k);
 * the gradient is its reverse-mode derivative (no formula is printed).
 * Errors: KDA_ERR_INVALID (NULL or misaligned pointer, T < 0, flags, small
 * workspace), KDA_ERR_UNSUPPORTED (dims). */
kda_status kda_prologue_backward(const kda_dims* dims, int32_t T, const void* q,
                                 const void* k, const void* v, const float* conv_w,
                                 const void* ring, const void* dq_hat, const void* dk_hat,
                                 const void* dv_hat, void* dq, void* dk, void* dv,
                                 float* dconv_w, float* dring, void* workspace,
                                 size_t workspace_bytes, uint32_t flags, hipStream_t stream);

/* Measurement helper, not part of the recurrence: multiplies the fp32 values
 * of a device buffer in place by scale, with the memory pattern of the
 * decode step's state stream (16-byte non-temporal loads, then stores: every
 * byte read once and written once). Timing it gives the practical HBM
 * ceiling that the state stream is compared against.
 *  buf: device buffer, 16-byte aligned; bytes: a multiple of 16.
 * Errors: KDA_ERR_INVALID (NULL or misaligned buffer, bytes). */
kda_status kda_stream_rmw(void* buf, size_t bytes, float scale, hipStream_t stream);

/* Description of the last error on the calling thread ("" if none). */
const char* kda_last_error(void);

/* Library version string. */
const char* kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
