/*
 * ttt_mem.h -- C ABI of libttt_mem.so: the chunked test-time-training memory
 * forward pass on AMD Instinct MI355X (gfx950).
 *
 * What is computed (one independent problem per (batch, head) pair):
 *
 *   A d x d fast-weight memory M (with a momentum state S of the same shape)
 *   is trained inside the forward pass by gradient steps on the inner loss
 *   l_t(M) = 1/2 || M k_t - v_t ||^2, whose gradient is (M k_t - v_t) k_t^T
 *   ("Continual Learning: From Attention to Neural Memory", sections 3.2-3.3
 *   and 4.2).  For every token t, with per-token gates theta_t (learning rate),
 *   eta_t (momentum decay) and alpha_t (forgetting):
 *
 *       S_t = eta_t S_{t-1} - theta_t (M_c k_t - v_t) k_t^T
 *       M_t = (1 - alpha_t) M_{t-1} + S_t
 *       z_t = M_t q_t                       (read after the token's own write)
 *
 *   ("论文速览 | Titans", sections 3.4 and 3.7; "Continual Learning...",
 *   section 5.2).  M_c is the chunk-start memory: the sequence is cut into
 *   chunks of b tokens (the last one may be shorter) and every gradient in a
 *   chunk is taken at the memory left by the previous chunk (mini-batch TTT:
 *   "5.1.1 · TTT layers 与 fast weights", section 1.1, eq. (6); "论文速览 |
 *   Titans", section 4.2).  The library evaluates each chunk in its dual
 *   (matrix) form; it never forms the per-token d x d intermediates.
 *
 * Conventions shared by every entry point:
 *
 *   - All data pointers are DEVICE pointers on the current HIP device, owned
 *     by the caller.  The library keeps no state, so calls are re-entrant;
 *     they are enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*, NULL = the default stream).  It allocates nothing, except the
 *     deep-memory entry points when they are given no workspace (they then
 *     take one from the stream-ordered allocator on `stream`).
 *   - Layouts are dense row-major:
 *       q, k, v           [B, H, T, d]   (token rows, d contiguous)
 *       theta, eta, alpha [B, H, T]      float32
 *       M0, S0, M_T, S_T  [B, H, d, d]   float32, M[i*d + j] carries key
 *                                        coordinate j into value coordinate i
 *       z                 [B, H, T, d]   bf16 on ttt_mem_forward_bf16 and
 *                                        ttt_mem_mlp_forward_bf16 (rounded to
 *                                        nearest even), float32 everywhere else
 *   - M0 or S0 may be NULL, meaning zeros.  M_T or S_T may be NULL, meaning
 *     "do not write".  M_T may be the same pointer as M0 and S_T the same as
 *     S0 (in-place state carry); z must not overlap any input.
 *   - Alignment: q, k, v, z, M0, S0, M_T, S_T must be 16-byte aligned; the
 *     gate arrays 4-byte aligned.
 *   - Sizes: B, H, T >= 0 (B*H == 0 is a no-op; T == 0 copies the initial
 *     state to the final state), d in {16, 32, 64, 128}, 1 <= b <= 64.
 *   - Errors: every argument check happens before anything is enqueued; a
 *     rejected call returns a negative status and touches no memory.  A
 *     failed kernel launch returns TTT_ERR_HIP.  Errors raised later by the
 *     device surface on the stream, as for any HIP kernel.
 *   - Gates are used as given (no clamping).  Inputs that make the recurrence
 *     diverge (for instance theta_t ||k_t||^2 outside (0, 2) with no momentum,
 *     "Continual Learning...", section 3.3) diverge here too; NaN and Inf
 *     propagate.
 */
#ifndef TTT_MEM_H
#define TTT_MEM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum ttt_status {
    TTT_OK = 0,
    TTT_ERR_INVALID_ARG = -1, /* bad size, NULL required pointer, misalignment, aliasing */
    TTT_ERR_UNSUPPORTED = -2, /* valid request outside what the kernels implement (d, b, hidden) */
    TTT_ERR_HIP = -3,         /* the HIP runtime rejected a launch */
    TTT_ERR_DEVICE = -4       /* a deep-memory launch reported a failure on the device (ttt_mem_deep_status) */
};

/*
 * Linear memory, float32 inputs and outputs (float32 MFMA products, float32
 * accumulation and state).
 */
int ttt_mem_forward_f32(const float* q, const float* k, const float* v,
                        const float* theta, const float* eta, const float* alpha,
                        const float* M0, const float* S0,
                        float* z, float* M_T, float* S_T,
                        int B, int H, int T, int d, int b, void* stream);

/*
 * Linear memory, bfloat16 q, k, v and z (raw bf16 bit patterns, uint16_t per
 * element), float32 gates and state.  Matrix products run on fp16 MFMA
 * operands with float32 accumulation: q and k convert to fp16 exactly (fp16
 * normal range), the state, the residuals and the intra-chunk weights are
 * rounded to fp16 once per chunk where they enter a product.  z is computed in
 * float32 and rounded to bf16 (nearest even) when it is stored, so its error
 * includes up to half a bf16 ulp of each element.  Precondition: q, k, the
 * state and the residuals M k - v stay below 65504 in magnitude (beyond it
 * the result is Inf/NaN).
 */
int ttt_mem_forward_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const float* theta, const float* eta, const float* alpha,
                         const float* M0, const float* S0,
                         uint16_t* z, float* M_T, float* S_T,
                         int B, int H, int T, int d, int b, void* stream);

/* The same computation with z stored as float32 (no output rounding). */
int ttt_mem_forward_bf16_zf32(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const float* theta, const float* eta, const float* alpha,
                              const float* M0, const float* S0,
                              float* z, float* M_T, float* S_T,
                              int B, int H, int T, int d, int b, void* stream);

/*
 * Deep (two-layer MLP) memory, bfloat16 q, k, v and z (rounded to nearest
 * even from float32); float32 gates, weights and momenta.  The memory is
 * f(u) = u + SiLU(u W1) W2 in row-vector form (W1: d x hidden, W2: hidden x d,
 * no biases), written by gradient steps on 1/2 ||f(k_t) - v_t||^2 taken by
 * explicit backprop at the chunk-start weights; each tensor has its own
 * momentum (S1, S2) and both use the token's theta, eta, alpha with the same
 * recurrences as the linear memory ("论文速览 | Titans", sections 3.4, 3.7,
 * 3.9 and 4.2; "Continual Learning: From Attention to Neural Memory",
 * sections 4.2 and 5.1-5.2).  The read is z_t = f(q_t) with the weights after
 * token t's own write.
 *
 *   Layouts: q, k, v, z [B, H, T, d] as above; W1_0, S1_0, W1_T, S1_T
 *   [B, H, d, hidden] and W2_0, S2_0, W2_T, S2_T [B, H, hidden, d], float32
 *   row-major (W1[i*hidden + j] maps input coordinate i to hidden unit j).
 *   W1_0 and W2_0 are required; S1_0, S2_0 may be NULL (zeros); any output
 *   weight may be NULL (not written) or the same pointer as its own initial
 *   tensor (in-place carry).  Pointers to the weights must be 4-byte aligned;
 *   q, k, v, z 16-byte aligned.
 *   Sizes: d = 64 and hidden = 256, 1 <= b <= 16 (other sizes return
 *   TTT_ERR_UNSUPPORTED).
 *   Precision: matrix products on bf16 operands with float32 accumulation;
 *   every float32 operand is split into two bf16 parts (about 16 significant
 *   bits); SiLU uses the hardware exp2 and reciprocal.
 *   Execution: the hidden units are split over a group of 8 workgroups per
 *   (batch, head), which exchange partial products once per chunk through a
 *   workspace in device memory (see ttt_mem_deep_forward_bf16).  This entry
 *   point takes that workspace from the stream-ordered allocator of the
 *   call's device (hipMallocAsync / hipFreeAsync on `stream`); use
 *   ttt_mem_deep_forward_bf16 to pass one and to read the device status.
 */
int ttt_mem_mlp_forward_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const float* theta, const float* eta, const float* alpha,
                             const float* W1_0, const float* W2_0,
                             const float* S1_0, const float* S2_0,
                             uint16_t* z, float* W1_T, float* W2_T, float* S1_T, float* S2_T,
                             int B, int H, int T, int d, int hidden, int b, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation and arguments as ttt_mem_mlp_forward_bf16, with the exchange
 * workspace in a file-scope device array of the library (2.4 MB per GPU,
 * reserved when the library is loaded and held until the process ends)
 * instead of an allocation.  It runs at most 8 (batch, head) sequences at a
 * time (the array holds 8 groups), so larger batches take proportionally
 * longer; a call whose workspace would not fit the array returns
 * TTT_ERR_UNSUPPORTED.  Every call on one GPU uses the same array: calls that
 * overlap in time on one GPU (different streams, other threads) race and
 * give undefined results; calls in stream order are fine (each launch clears
 * the counters it needs).  No hipMalloc, hipFree or allocating library
 * routine is called.
 */
int ttt_mem_mlp_forward_bf16_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const float* theta, const float* eta, const float* alpha,
                                     const float* W1_0, const float* W2_0,
                                     const float* S1_0, const float* S2_0,
                                     uint16_t* z, float* W1_T, float* W2_T, float* S1_T, float* S2_T,
                                     int B, int H, int T, int d, int hidden, int b, void* stream);

/* The same computation with z stored as float32. */
int ttt_mem_mlp_forward_bf16_zf32(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  const float* theta, const float* eta, const float* alpha,
                                  const float* W1_0, const float* W2_0,
                                  const float* S1_0, const float* S2_0,
                                  float* z, float* W1_T, float* W2_T, float* S1_T, float* S2_T,
                                  int B, int H, int T, int d, int hidden, int b, void* stream);

/*
 * Deep memory of depth L = `depth` ("论文速览 | Titans", section 3.9: L linear
 * maps with a nonlinearity between them; section 8.5 compares depths 1-4):
 * f(u) = u + SiLU(...SiLU(u W_1)...) W_L in row-vector form, W_1: d x hidden,
 * W_l: hidden x hidden (1 < l < L), W_L: hidden x d, every layer with its own
 * momentum, trained exactly as the two-layer memory above (which is depth 2).
 *
 *   Parameters are packed per (batch, head): W0, S0, W_T, S_T are
 *   [B, H, P] float32 with P = ttt_mem_deep_param_count(d, hidden, depth);
 *   layer 1 starts at 0, layer l (1 < l <= L) at d*hidden + (l-2)*hidden*hidden,
 *   each row-major as above.  W0 is required; S0 may be NULL (zeros); W_T and
 *   S_T may be NULL or equal W0 / S0 (in-place carry).
 *   work: a caller-owned workspace of at least
 *   ttt_mem_deep_work_bytes(B, H, d, hidden, depth) bytes, 256-byte aligned
 *   (NULL: taken from the stream-ordered allocator as above).  Calls that
 *   share a workspace must not overlap in time.  The workgroups of a group
 *   exchange through it and wait for each other with bounded waits: a wait
 *   that runs out, or a workgroup that finds no place in a group of its XCD,
 *   records a failure in the workspace instead of hanging; the results are
 *   then undefined.  ttt_mem_deep_status(work, stream) synchronizes `stream`
 *   and returns TTT_OK, or TTT_ERR_DEVICE if the last launch on `work`
 *   recorded a failure.  A wait gives up after 2,000,000 polls of its
 *   counter; the environment variable TTT_MEM_DEEP_SPIN_LIMIT (read at each
 *   call of the deep-memory entry points) sets another limit, so that a test
 *   can drive that path (0: a wait gives up as soon as a poll finds the
 *   group incomplete).
 *   Sizes: d = 64, hidden = 256, depth in {2, 3, 4}, 1 <= b <= 16.
 */
size_t ttt_mem_deep_param_count(int d, int hidden, int depth);
size_t ttt_mem_deep_work_bytes(int B, int H, int d, int hidden, int depth);
int ttt_mem_deep_forward_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const float* theta, const float* eta, const float* alpha,
                              const float* W0, const float* S0,
                              uint16_t* z, float* W_T, float* S_T,
                              int B, int H, int T, int d, int hidden, int depth, int b,
                              void* work, size_t work_bytes, void* stream);
int ttt_mem_deep_status(const void* work, void* stream);

/*
 * Linear memory over packed variable-length documents: every document starts
 * from its own initial state, so nothing of one document leaks into the next
 * through the fast weights ("5.1.1 · TTT layers 与 fast weights", section 1.2,
 * the notes on packed documents: the state reset follows the document
 * boundaries, momentum included; "Continual Learning: From Attention to
 * Neural Memory", sections 4.6 and 4.8: every independent sequence begins
 * from its own starting point, the memory is reset per sequence).  Each
 * document is chunked
 * on its own (its first chunk starts at its first token) and computed exactly
 * as ttt_mem_forward_* computes one sequence.
 *
 *   cu_seqlens: DEVICE int32 [N + 1], non-decreasing, cu_seqlens[0] = 0,
 *     cu_seqlens[N] <= T; document s is tokens cu_seqlens[s] ..
 *     cu_seqlens[s+1]-1.  (The host cannot read it; the kernel clamps every
 *     offset into [0, T], so a malformed table gives wrong results, never an
 *     access outside the arrays.)  An empty document copies its initial state.
 *   Order: documents run longest first.  On the bf16 entry points at
 *     d >= 64, when the ranking fits the workgroup's LDS (up to 2048
 *     documents at d = 128 and b > 32, at least 680 in every configuration)
 *     and no workgroup lane takes more than 384 (document, head) pairs, the
 *     launch is persistent: about one workgroup per CU ranks the documents
 *     itself and walks its share of them, nothing is allocated.  Otherwise one
 *     workgroup runs per document, and above 128 documents a ranking pass on
 *     `stream` writes the order to N ints taken from the stream-ordered
 *     allocator (hipMallocAsync), returned with hipFreeAsync on the same
 *     stream after the launch; TTT_ERR_HIP if that allocation fails.  The
 *     training entry points below use the same forward; their backward pass
 *     always takes the second form.
 *   Layouts: q, k, v, z [H, T, d]; theta, eta, alpha [H, T]; M0, S0, M_T, S_T
 *     [N, H, d, d] (document-major).  Tokens outside every document are not
 *     read and their z is not written.
 *   Everything else (NULL states, aliasing, alignment, d, b, precision) as
 *   for ttt_mem_forward_f32 / ttt_mem_forward_bf16; cu_seqlens must not
 *   overlap z, M_T or S_T.
 */
int ttt_mem_forward_varlen_f32(const float* q, const float* k, const float* v,
                               const float* theta, const float* eta, const float* alpha,
                               const float* M0, const float* S0,
                               float* z, float* M_T, float* S_T,
                               const int* cu_seqlens, int N, int H, int T, int d, int b, void* stream);

int ttt_mem_forward_varlen_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const float* theta, const float* eta, const float* alpha,
                                const float* M0, const float* S0,
                                float* z, float* M_T, float* S_T,
                                const int* cu_seqlens, int N, int H, int T, int d, int b, void* stream);

/*
 * Linear memory, token by token (the primal form), for generation: every
 * token's gradient is taken at the memory the previous token left (chunks of
 * one token; "5.1.1 · TTT layers 与 fast weights", section 1.1, the
 * primal/dual comparison after eq. (9): prefill in the dual form, decode in
 * the primal form).  The result equals ttt_mem_forward_* with b = 1; the
 * intended use is T = 1 per call with the state carried in place
 * (M_T == M0, S_T == S0) from one generated token to the next
 * ("Continual Learning: From Attention to Neural Memory", section 4.8, the
 * note on streaming inference).  All arithmetic is float32; the bf16 entry
 * point widens q, k, v exactly.  Layouts, NULL states, aliasing and error
 * behaviour as above; alignment: M0, S0, M_T, S_T 16 bytes, q and k 16 bytes
 * (float32) or 8 bytes (bf16), v, z and the gates their element size.
 * Sizes: d in {16, 32, 64, 128}.  The state is read once and written once
 * per call; tokens are processed in order inside the call.
 */
int ttt_mem_decode_f32(const float* q, const float* k, const float* v,
                       const float* theta, const float* eta, const float* alpha,
                       const float* M0, const float* S0,
                       float* z, float* M_T, float* S_T,
                       int B, int H, int T, int d, void* stream);

int ttt_mem_decode_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const float* theta, const float* eta, const float* alpha,
                        const float* M0, const float* S0,
                        float* z, float* M_T, float* S_T,
                        int B, int H, int T, int d, void* stream);

/*
 * Training forward and backward pass of the linear memory.
 *
 * The outer loss of a model that contains the memory trains q, k, v, the gates
 * and the initial state through the inner updates: every write is ordinary
 * arithmetic, so its outer gradient is the chain rule applied backward through
 * the unrolled state transitions, with no gradient path detached
 * ("Continual Learning: From Attention to Neural Memory", section 4.5;
 * "5.1.1 · TTT layers 与 fast weights", section 1.2, eqs. (15)-(16): the
 * outer gradient of a key runs through the inner gradient it produced).
 * The backward walks the chunks in reverse order, as the forward walks them
 * forward; inside a chunk it uses the same matrix (dual) form
 * ("论文速览 | Titans", section 4.7: chunks pass the memory state, and the
 * backward differentiates the inner update).
 *
 * ttt_mem_forward_ckpt_*: the forward above, plus the state entering every
 * chunk, which the backward differentiates from:
 *     ckpt [B, H, NC, 2, d, d], NC = ceil(T / b);
 *     ckpt[b, h, c, 0] = M and ckpt[b, h, c, 1] = S before chunk c
 *     (c = 0: M0 and S0, zeros for NULL),
 * float32 for the _f32 entry points, IEEE fp16 (round to nearest even) for
 * the _bf16 ones, whose products round the state to fp16 anyway.  Its size
 * in bytes is ttt_mem_ckpt_bytes(B, H, T, d, b), resp. _bf16.  ckpt is
 * required (non-NULL, 16-byte aligned) and must not overlap any other
 * argument.
 *
 * ttt_mem_backward_*: given the derivatives of the outer loss with respect
 * to the forward's outputs,
 *     dz [B, H, T, d] float32, dM_T, dS_T [B, H, d, d] float32 (NULL: zero),
 * and the same q, k, v, theta, eta, alpha, B, H, T, d, b as the forward that
 * wrote ckpt, writes the derivatives with respect to its inputs:
 *     dq, dk, dv                 [B, H, T, d] float32 (both entry points),
 *     dtheta, deta, dalpha       [B, H, T]    float32,
 *     dM0, dS0                   [B, H, d, d] float32 (NULL: not written).
 * work is a caller-owned scratch buffer (the derivatives with respect to the
 * state leaving every chunk): for the _f32 entry points of the checkpoints'
 * type and size (ttt_mem_ckpt_bytes), for the _bf16 ones of
 * ttt_mem_backward_work_bytes_bf16 bytes (the fp16 checkpoints' size plus a
 * few floats per sequence); its contents on entry do not matter and on return
 * are unspecified.
 * The bf16 entry point takes q, k, v in bf16 and computes its matrix products
 * with fp16 operands and float32 accumulation, as the bf16 forward does; the
 * float32 one uses float32 products.
 * Cotangent range (bf16 entry points): dz, dM_T and dS_T may have any finite
 * float32 magnitude.  Each sequence's cotangents are multiplied by one power
 * of two that brings their largest magnitude into [1, 2) before they are
 * rounded to fp16, and every gradient is divided by it again (both exact), so
 * the small values of a mean-reduced loss (1e-6 .. 1e-9) keep fp16's relative
 * precision.  Entries below about 2^-14 of their sequence's largest magnitude
 * fall into fp16's subnormal range (absolute error up to 2^-25 of that
 * magnitude).  Non-finite cotangents propagate (no scaling is applied).
 * Argument rules as for the forward: sizes, alignment (16 bytes for every
 * array except the gate arrays and their gradients, 4 bytes), no overlap
 * between any output and any other argument (dM0 may not alias dM_T).
 * Two kernels run in order on `stream`: a reverse walk over the chunks per
 * row block of the state, then one workgroup per (batch, head, chunk).
 */
int ttt_mem_forward_ckpt_f32(const float* q, const float* k, const float* v,
                             const float* theta, const float* eta, const float* alpha,
                             const float* M0, const float* S0,
                             float* z, float* M_T, float* S_T, float* ckpt,
                             int B, int H, int T, int d, int b, void* stream);

int ttt_mem_forward_ckpt_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const float* theta, const float* eta, const float* alpha,
                              const float* M0, const float* S0,
                              float* z, float* M_T, float* S_T, uint16_t* ckpt,
                              int B, int H, int T, int d, int b, void* stream);

/* Bytes of ckpt for the _f32 and the _bf16 entry points (and of the _f32
 * backward's work buffer); 0 for negative sizes. */
size_t ttt_mem_ckpt_bytes(int B, int H, int T, int d, int b);
size_t ttt_mem_ckpt_bytes_bf16(int B, int H, int T, int d, int b);

/* Bytes of the work buffer of ttt_mem_backward_bf16 and ttt_mem_backward_cg_bf16
 * (16-byte aligned, as every array); 0 for negative sizes. */
size_t ttt_mem_backward_work_bytes_bf16(int B, int H, int T, int d, int b);

int ttt_mem_backward_f32(const float* q, const float* k, const float* v,
                         const float* theta, const float* eta, const float* alpha,
                         const float* ckpt, const float* dz, const float* dM_T, const float* dS_T,
                         float* dq, float* dk, float* dv,
                         float* dtheta, float* deta, float* dalpha,
                         float* dM0, float* dS0, float* work,
                         int B, int H, int T, int d, int b, void* stream);

int ttt_mem_backward_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          const float* theta, const float* eta, const float* alpha,
                          const uint16_t* ckpt, const float* dz, const float* dM_T, const float* dS_T,
                          float* dq, float* dk, float* dv,
                          float* dtheta, float* deta, float* dalpha,
                          float* dM0, float* dS0, uint16_t* work,
                          int B, int H, int T, int d, int b, void* stream);

/*
 * Chunk-shared gates ("论文速览 | Titans", section 4.6: a faster, less
 * expressive variant in which alpha, theta and eta do not depend on the
 * token but are shared by the tokens of a chunk, so that inside a chunk the
 * recurrence is linear and time-invariant).  Identical to the entry points
 * above except that theta, eta, alpha -- and, for the backward, dtheta,
 * deta, dalpha -- are [B, H, NC] float32 with NC = ceil(T / b): every token
 * of chunk c uses entry c, and the gradient of entry c is the sum over the
 * chunk's tokens.  ttt_mem_forward_cg_* takes an optional ckpt (NULL: not
 * written) for ttt_mem_backward_cg_*.
 */
int ttt_mem_forward_cg_f32(const float* q, const float* k, const float* v,
                           const float* theta, const float* eta, const float* alpha,
                           const float* M0, const float* S0,
                           float* z, float* M_T, float* S_T, float* ckpt,
                           int B, int H, int T, int d, int b, void* stream);

int ttt_mem_forward_cg_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const float* theta, const float* eta, const float* alpha,
                            const float* M0, const float* S0,
                            float* z, float* M_T, float* S_T, uint16_t* ckpt,
                            int B, int H, int T, int d, int b, void* stream);

int ttt_mem_backward_cg_f32(const float* q, const float* k, const float* v,
                            const float* theta, const float* eta, const float* alpha,
                            const float* ckpt, const float* dz, const float* dM_T, const float* dS_T,
                            float* dq, float* dk, float* dv,
                            float* dtheta, float* deta, float* dalpha,
                            float* dM0, float* dS0, float* work,
                            int B, int H, int T, int d, int b, void* stream);

int ttt_mem_backward_cg_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const float* theta, const float* eta, const float* alpha,
                             const uint16_t* ckpt, const float* dz, const float* dM_T, const float* dS_T,
                             float* dq, float* dk, float* dv,
                             float* dtheta, float* deta, float* dalpha,
                             float* dM0, float* dS0, uint16_t* work,
                             int B, int H, int T, int d, int b, void* stream);

/*
 * Training over packed variable-length documents: the forward that also keeps
 * every document's chunk-start states, and the backward pass from them.  Each
 * document is its own sequence with its own initial state (the forward's
 * packed-document entry points above), so its gradients are exactly those of
 * ttt_mem_backward_* on that document alone ("Continual Learning: From
 * Attention to Neural Memory", section 4.5: the outer gradient runs back
 * through the unrolled writes; "5.1.1 · TTT layers 与 fast weights", section
 * 1.2, the notes on packed documents: nothing flows across a document
 * boundary).
 *
 *   Checkpoints and work buffer: [H][ceil(T/b) + N][M | S][d][d], float32 on
 *     the f32 entry points and fp16 on the bf16 ones, of
 *     ttt_mem_ckpt_bytes_varlen / ttt_mem_ckpt_bytes_varlen_bf16 bytes, caller
 *     owned; the bf16 backward's work buffer takes
 *     ttt_mem_backward_work_bytes_varlen_bf16 bytes (the cotangent scaling is
 *     per document and head).  Document s of head h uses the slots from h * (ceil(T/b) + N) +
 *     (the chunks of documents 0..s-1) on; the rest are not written.  A
 *     table that is not non-decreasing can make documents overlap; results
 *     are then undefined, and a document whose chunks would pass the head's
 *     last slot is cut there, so no access leaves the caller's buffers.
 *   Layouts: q, k, v, dz, dq, dk, dv [H, T, d]; theta, eta, alpha and their
 *     gradients [H, T]; M0, S0, dM_T, dS_T, dM0, dS0 [N, H, d, d]; cu_seqlens as
 *     for ttt_mem_forward_varlen_*.  The gradients of tokens outside every
 *     document are not written.
 *   Everything else (NULL arguments, alignment, overlap and size checks,
 *   precision) as for ttt_mem_forward_ckpt_* and ttt_mem_backward_*.
 *   Chunk-shared gates are not supported here.  Returns TTT_ERR_INVALID_ARG
 *   for a NULL ckpt or cu_seqlens.
 */
size_t ttt_mem_ckpt_bytes_varlen(int N, int H, int T, int d, int b);
size_t ttt_mem_ckpt_bytes_varlen_bf16(int N, int H, int T, int d, int b);
size_t ttt_mem_backward_work_bytes_varlen_bf16(int N, int H, int T, int d, int b);

int ttt_mem_forward_varlen_ckpt_f32(const float* q, const float* k, const float* v,
                                    const float* theta, const float* eta, const float* alpha,
                                    const float* M0, const float* S0,
                                    float* z, float* M_T, float* S_T, float* ckpt,
                                    const int* cu_seqlens, int N, int H, int T, int d, int b, void* stream);

int ttt_mem_forward_varlen_ckpt_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const float* theta, const float* eta, const float* alpha,
                                     const float* M0, const float* S0,
                                     float* z, float* M_T, float* S_T, uint16_t* ckpt,
                                     const int* cu_seqlens, int N, int H, int T, int d, int b, void* stream);

int ttt_mem_backward_varlen_f32(const float* q, const float* k, const float* v,
                                const float* theta, const float* eta, const float* alpha,
                                const float* ckpt, const float* dz, const float* dM_T, const float* dS_T,
                                float* dq, float* dk, float* dv,
                                float* dtheta, float* deta, float* dalpha,
                                float* dM0, float* dS0, float* work,
                                const int* cu_seqlens, int N, int H, int T, int d, int b, void* stream);

int ttt_mem_backward_varlen_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const float* theta, const float* eta, const float* alpha,
                                 const uint16_t* ckpt, const float* dz, const float* dM_T, const float* dS_T,
                                 float* dq, float* dk, float* dv,
                                 float* dtheta, float* deta, float* dalpha,
                                 float* dM0, float* dS0, uint16_t* work,
                                 const int* cu_seqlens, int N, int H, int T, int d, int b, void* stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* ttt_mem_status_string(int status);

/* ABI version of this header: (major << 16) | minor. */
int ttt_mem_abi_version(void);

#define TTT_MEM_ABI_VERSION ((3 << 16) | 0)

#ifdef __cplusplus
}
#endif

#endif /* TTT_MEM_H */
