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
 *     by the caller.  The library allocates nothing and keeps no state, so
 *     calls are re-entrant; they are enqueued asynchronously on `stream`
 *     (a hipStream_t passed as void*, NULL = the default stream).
 *   - Layouts are dense row-major:
 *       q, k, v           [B, H, T, d]   (token rows, d contiguous)
 *       theta, eta, alpha [B, H, T]      float32
 *       M0, S0, M_T, S_T  [B, H, d, d]   float32, M[i*d + j] carries key
 *                                        coordinate j into value coordinate i
 *       z                 [B, H, T, d]   float32
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

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum ttt_status {
    TTT_OK = 0,
    TTT_ERR_INVALID_ARG = -1, /* bad size, NULL required pointer, misalignment, aliasing */
    TTT_ERR_UNSUPPORTED = -2, /* valid request outside what the kernels implement (d, b, hidden) */
    TTT_ERR_HIP = -3          /* the HIP runtime rejected a launch */
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
 * Linear memory, bfloat16 q, k, v (raw bf16 bit patterns, uint16_t per
 * element), float32 state and z.  Matrix products run on fp16 MFMA operands
 * with float32 accumulation: q and k convert to fp16 exactly (fp16 normal
 * range), the state, the residuals and the intra-chunk weights are rounded
 * to fp16 once per chunk where they enter a product.  Precondition: q, k,
 * the state and the residuals M k - v stay below 65504 in magnitude (beyond
 * it the result is Inf/NaN).  z is float32 because the bf16 rounding of the
 * output alone would use most of a 2e-2 max-error/RMS budget.
 */
int ttt_mem_forward_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const float* theta, const float* eta, const float* alpha,
                         const float* M0, const float* S0,
                         float* z, float* M_T, float* S_T,
                         int B, int H, int T, int d, int b, void* stream);

/*
 * Deep (two-layer MLP) memory, bfloat16 q, k, v; float32 gates, weights,
 * momenta and z.  The memory is f(u) = u + SiLU(u W1) W2 in row-vector form
 * (W1: d x hidden, W2: hidden x d, no biases), written by gradient steps on
 * 1/2 ||f(k_t) - v_t||^2 taken by explicit backprop at the chunk-start
 * weights; each tensor has its own momentum (S1, S2) and both use the token's
 * theta, eta, alpha with the same recurrences as the linear memory
 * ("论文速览 | Titans", sections 3.4, 3.7, 3.9 and 4.2; "Continual Learning:
 * From Attention to Neural Memory", sections 4.2 and 5.1-5.2).  The read is
 * z_t = f(q_t) with the weights after token t's own write.
 *
 *   Layouts: q, k, v, z [B, H, T, d] as above; W1_0, S1_0, W1_T, S1_T
 *   [B, H, d, hidden] and W2_0, S2_0, W2_T, S2_T [B, H, hidden, d], float32
 *   row-major (W1[i*hidden + j] maps input coordinate i to hidden unit j).
 *   W1_0 and W2_0 are required; S1_0, S2_0 may be NULL (zeros); any output
 *   weight may be NULL (not written) or the same pointer as its own initial
 *   tensor (in-place carry).  Pointers to the weights must be 4-byte aligned;
 *   q, k, v, z 16-byte aligned.
 *   Sizes: d = 64 and hidden = 256, 1 <= b <= 16 (other sizes return
 *   TTT_ERR_UNSUPPORTED).  Matrix products use fp16 operands with float32
 *   accumulation (same precondition as ttt_mem_forward_bf16); SiLU uses the
 *   hardware exp2 and reciprocal.
 */
int ttt_mem_mlp_forward_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const float* theta, const float* eta, const float* alpha,
                             const float* W1_0, const float* W2_0,
                             const float* S1_0, const float* S2_0,
                             float* z, float* W1_T, float* W2_T, float* S1_T, float* S2_T,
                             int B, int H, int T, int d, int hidden, int b, void* stream);

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

/* Human-readable name of a status code (static storage, never NULL). */
const char* ttt_mem_status_string(int status);

/* ABI version of this header: (major << 16) | minor. */
int ttt_mem_abi_version(void);

#define TTT_MEM_ABI_VERSION ((1 << 16) | 0)

#ifdef __cplusplus
}
#endif

#endif /* TTT_MEM_H */
