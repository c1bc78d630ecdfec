// Chunked TTT / Titans linear memory forward for gfx950 (MI355X), and its C ABI.
//
// One workgroup owns RB = 16*NW consecutive rows of one (batch, head) memory
// and walks that sequence chunk by chunk; each wave keeps a 16-row slice of M
// and of the momentum S in MFMA accumulator registers for the whole sequence,
// so the state never leaves the chip between chunks.  Rows of a linear memory
// evolve independently (row i only meets value coordinate i), so row blocks
// of one head need no communication.
//
// Per chunk of n <= b tokens (padded to NP rows, NP a multiple of 16/32):
//   1. the chunk's q, k (and a transposed copy of k), the workgroup's columns
//      of v and the gates are staged in LDS;
//   2. one wave runs the gate scans across its 64 lanes (lane = token):
//      A_i = prod_{l<=i} a_l (a = 1 - alpha), E_i = prod_{l<=i} eta_l,
//      c_i = a_i c_{i-1} + E_i, the chunk-end weights w^M, w^S, and the
//      helpers of the lower-triangular decay matrix gamma (below);
//   3. all waves form P = -(tril(Q K^T) .* theta_j gamma_ij) on MFMA;
//   4. each wave, on MFMA:  E = K M0^T - V              (residuals at chunk start)
//                           Z^T = A.(M0 Q^T) + c.(S0 Q^T) + E^T P^T
//                           M  <- A_n M0 + c_n S0 + (K^T (w^M . E))^T
//                           S  <- E_n S0 + (K^T (w^S . E))^T
//      with w^M_j = -theta_j gamma_{n-1,j} and w^S_j = -theta_j prod_{l>j} eta_l.
//      On the bf16-input path the matrix units take fp16 operands (same
//      rate as bf16 on gfx950, 3 more mantissa bits): bf16 q and k convert
//      to fp16 exactly in the fp16 normal range, and M0, S0, E and P are
//      rounded to fp16 once per chunk.  Operands must stay below 65504 in
//      magnitude; accumulation and the carried state are float32.
//
// These are the per-token recurrences S_t = eta_t S_{t-1} - theta_t grad,
// M_t = (1 - alpha_t) M_{t-1} + S_t, z_t = M_t q_t ("论文速览 | Titans",
// sections 3.4, 3.7) with every gradient of a chunk taken at the chunk-start
// memory (same page, section 4.2; "5.1.1 · TTT layers 与 fast weights",
// section 1.1, eq. (6)), unrolled over the chunk.  With alpha = eta = 0 this
// is the dual form of that page, eqs. (7)-(9); decay unrolling follows
// "论文速览 | Titans" sections 4.3-4.5.  Unlike a ratio of cumulative products
// (beta_t / beta_i there), every weight here is built from products and sums
// only, so gates equal to zero (eta = 0, alpha = 1) are exact.
//
// The decay matrix: gamma_ij = sum_{m=j..i} (prod_{l=m+1..i} a_l)(prod_{l=j+1..m} eta_l)
// for j <= i.  Per column j the pair (gamma_ij, p_ij = prod_{l=j+1..i} eta_l)
// follows the 2x2 linear map T_i = [[a_i, eta_i], [0, eta_i]] in i.  Diagonal
// 16x16 blocks run that recurrence directly (lane = column); a block below the
// diagonal uses the product of the T's from the end of the column's block to
// row i (a segmented lane scan plus at most two block products), applied to
// the column's state at the end of its own block.
//
// MFMA operand layout trick: an accumulator tile holds, in lane (n, g), rows
// 4g..4g+3 of column n.  Storing M transposed (tiles of M^T) puts in each lane
// four consecutive columns of one row of M, which is exactly a k-slot group of
// an MFMA A or B operand when the contraction runs over those columns.  So M,
// S and E feed the next products straight from registers; the operands read
// from LDS are stored with the matching permutation of the contraction index.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ttt_mem.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__host__ __device__ constexpr int round_up(int x, int m) { return (x + m - 1) / m * m; }

// ---------------------------------------------------------------------------
// MFMA operand traits.  A "k-group" is the contraction length of one operand
// fragment: 16 for float32 (four v_mfma_f32_16x16x4_f32, one slot each) and 32
// for fp16 (one v_mfma_f32_16x16x32_f16, eight slots).  In both, lane group g
// of a fragment for k-group s carries contraction indices
//   f32 : slot i      -> 16s + 4g + i
//   fp16: slot i < 4  -> 32s + 4g + i,   slot 4 + i -> 32s + 16 + 4g + i
// which is the accumulator's own row order, so accumulator tiles convert to
// fragments lane-locally.  LDS operands are stored permuted along the
// contraction index so that a lane's slots are 16 contiguous bytes.
// ---------------------------------------------------------------------------
template <typename T>
struct Op;

template <>
struct Op<float> {
    static constexpr int KG = 16;
    using frag = f32x4;
    __device__ static int perm(int x) { return x; }
    __device__ static f32x4 mma(f32x4 acc, const frag& a, const frag& b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
        return acc;
    }
    template <int NTILES>
    __device__ static frag from_acc(const f32x4* tiles, int s) { return tiles[s]; }
    __device__ static frag lds(const float* row, int s, int g) {
        return *reinterpret_cast<const f32x4*>(row + 16 * s + 4 * g);
    }
    // Store four consecutive contraction indices x..x+3 (x % 4 == 0).
    __device__ static void put4(float* row, int x, f32x4 v) {
        *reinterpret_cast<f32x4*>(row + perm(x)) = v;
    }
    __device__ static float to_f32(float x) { return x; }
};

template <>
struct Op<_Float16> {
    static constexpr int KG = 32;
    using frag = f16x8;
    // x = 32s + 16h + 4g + i  ->  32s + 8g + 4h + i
    __device__ static int perm(int x) {
        return (x & ~31) | (((x >> 2) & 3) << 3) | (((x >> 4) & 1) << 2) | (x & 3);
    }
    __device__ static f32x4 mma(f32x4 acc, const frag& a, const frag& b) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
    }
    template <int NTILES>
    __device__ static frag from_acc(const f32x4* tiles, int s) {
        const f32x4 lo = tiles[2 * s];
        const f32x4 hi = (2 * s + 1 < NTILES) ? tiles[2 * s + 1] : f32x4{0.f, 0.f, 0.f, 0.f};
        frag f;
        f[0] = (_Float16)lo[0]; f[1] = (_Float16)lo[1]; f[2] = (_Float16)lo[2]; f[3] = (_Float16)lo[3];
        f[4] = (_Float16)hi[0]; f[5] = (_Float16)hi[1]; f[6] = (_Float16)hi[2]; f[7] = (_Float16)hi[3];
        return f;
    }
    __device__ static frag lds(const _Float16* row, int s, int g) {
        return *reinterpret_cast<const f16x8*>(row + 32 * s + 8 * g);
    }
    __device__ static void put4(_Float16* row, int x, f32x4 v) {
        f16x4 h;
        h[0] = (_Float16)v[0]; h[1] = (_Float16)v[1]; h[2] = (_Float16)v[2]; h[3] = (_Float16)v[3];
        *reinterpret_cast<f16x4*>(row + perm(x)) = h;
    }
};

// Global-memory element types: float for the f32 path, raw bf16 bits for the
// bf16-input path (whose matrix operands are fp16).
template <typename T> struct GlobalOf;
template <> struct GlobalOf<float> { using type = float; };
template <> struct GlobalOf<_Float16> { using type = uint16_t; };

__device__ inline float g2f(float x) { return x; }
__device__ inline float g2f(uint16_t x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }

struct Params {
    const void* q;
    const void* k;
    const void* v;
    const float* theta;
    const float* eta;
    const float* alpha;
    const float* M0;
    const float* S0;
    float* z;
    float* MT;
    float* ST;
    int BH;
    int T;
    int b;
};

template <typename T, int D, int NW, int NP>
__global__ __launch_bounds__(kWave * NW) void linear_memory_fwd(const Params p) {
    using O = Op<T>;
    using G = typename GlobalOf<T>::type;
    constexpr int RB = 16 * NW;          // rows of M per workgroup
    constexpr int NRB = D / RB;          // workgroups per (batch, head)
    constexpr int NC = D / 16;           // 16-column tiles of M
    constexpr int NT = NP / 16;          // 16-token tiles of a chunk
    constexpr int KG = O::KG;
    constexpr int NKC = (D + KG - 1) / KG;     // k-groups over the key dimension
    constexpr int NKT = NP / KG;               // k-groups over the chunk's tokens
    constexpr int EPAD = 16 / sizeof(T);       // 16-byte row padding
    constexpr int LQ = round_up(D, KG) + EPAD; // row stride of sQ, sK
    constexpr int LKT = NP + EPAD;             // row stride of sKT
    constexpr int LP = NP + EPAD;              // row stride of sP
    constexpr int LV = NP + 4;                 // row stride of sVT (float)
    constexpr int VEC = 16 / sizeof(G);        // elements per 16-byte global load
    constexpr int NTHR = kWave * NW;
    static_assert(NP % KG == 0, "chunk padding must fill whole k-groups");
    static_assert(D % RB == 0, "row blocks must tile d");

    __shared__ __attribute__((aligned(16))) T sQ[NP * LQ];
    __shared__ __attribute__((aligned(16))) T sK[NP * LQ];
    __shared__ __attribute__((aligned(16))) T sKT[D * LKT];
    __shared__ __attribute__((aligned(16))) T sP[NP * LP];
    __shared__ __attribute__((aligned(16))) float sVT[RB * LV];
    __shared__ __attribute__((aligned(16))) float sGamD[NT * 256];
    __shared__ __attribute__((aligned(16))) float sPhi[NT * NP * 2];
    __shared__ __attribute__((aligned(16))) float sTh[NP], sEg[NP], sAg[NP];
    __shared__ __attribute__((aligned(16))) float sAv[NP], sCv[NP], sWM[NP], sWS[NP];
    __shared__ __attribute__((aligned(16))) float sGend[NP], sPend[NP];
    __shared__ float sScal[4];

    const int tid = threadIdx.x;
    const int w = tid / kWave;
    const int lane = tid % kWave;
    const int lr = lane & 15;   // MFMA row/column index within a 16-tile
    const int lg = lane >> 4;   // MFMA k-slot group

    // Workgroup -> (sequence, row block).  When the count allows, the row
    // blocks of one sequence get workgroup ids that are congruent mod 8, so
    // they run on one XCD and share its L2 for the q, k re-reads.
    const int nwg = gridDim.x;
    int lin = blockIdx.x;
    if ((p.BH % 8) == 0) lin = (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8;
    const int bh = lin / NRB;
    const int rb = lin % NRB;
    const int seqlen = p.T;
    const int b = p.b;
    const int row_wg = rb * RB;          // first row of M in this workgroup
    const int row_w = row_wg + 16 * w;   // first row of this wave's slice

    // Zero the staging tiles once: padding columns (d < 32 on the fp16 path) stay 0.
    for (int i = tid; i < NP * LQ; i += NTHR) { sQ[i] = T(0.f); sK[i] = T(0.f); }
    for (int i = tid; i < D * LKT; i += NTHR) sKT[i] = T(0.f);
    for (int i = tid; i < NP * LP; i += NTHR) sP[i] = T(0.f);

    // State slice: lane (lr, lg) of tile ct holds M[row_w + lr][16ct + 4lg + i].
    f32x4 Macc[NC], Sacc[NC];
    const size_t state_off = static_cast<size_t>(bh) * D * D + static_cast<size_t>(row_w + lr) * D;
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
        const int col = 16 * ct + 4 * lg;
        Macc[ct] = p.M0 ? *reinterpret_cast<const f32x4*>(p.M0 + state_off + col) : f32x4{0.f, 0.f, 0.f, 0.f};
        Sacc[ct] = p.S0 ? *reinterpret_cast<const f32x4*>(p.S0 + state_off + col) : f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const G* __restrict__ gq = static_cast<const G*>(p.q);
    const G* __restrict__ gk = static_cast<const G*>(p.k);
    const G* __restrict__ gv = static_cast<const G*>(p.v);
    const size_t seq_tok = static_cast<size_t>(bh) * seqlen;   // first token row of this sequence

    for (int c0 = 0; c0 < seqlen; c0 += b) {
        const int n = min(b, seqlen - c0);
        __syncthreads();   // the previous chunk is done with every LDS buffer

        // ---- 1. stage the chunk in LDS ------------------------------------
        for (int u = tid; u < NP * (D / VEC); u += NTHR) {
            const int t = u / (D / VEC);
            const int c = (u % (D / VEC)) * VEC;
            float qv[VEC], kv[VEC];
            if (t < n) {
                const size_t off = (seq_tok + c0 + t) * D + c;
                const uint4 rq = *reinterpret_cast<const uint4*>(gq + off);
                const uint4 rk = *reinterpret_cast<const uint4*>(gk + off);
                const G* eq = reinterpret_cast<const G*>(&rq);
                const G* ek = reinterpret_cast<const G*>(&rk);
#pragma unroll
                for (int e = 0; e < VEC; ++e) { qv[e] = g2f(eq[e]); kv[e] = g2f(ek[e]); }
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e) { qv[e] = 0.f; kv[e] = 0.f; }
            }
#pragma unroll
            for (int e = 0; e < VEC; e += 4) {
                O::put4(sQ + t * LQ, c + e, f32x4{qv[e], qv[e + 1], qv[e + 2], qv[e + 3]});
                O::put4(sK + t * LQ, c + e, f32x4{kv[e], kv[e + 1], kv[e + 2], kv[e + 3]});
            }
            const int pt = O::perm(t);
#pragma unroll
            for (int e = 0; e < VEC; ++e) sKT[(c + e) * LKT + pt] = T(kv[e]);
        }
        for (int u = tid; u < NP * (RB / VEC); u += NTHR) {
            const int t = u / (RB / VEC);
            const int r = (u % (RB / VEC)) * VEC;
            float vv[VEC];
            if (t < n) {
                const uint4 rv = *reinterpret_cast<const uint4*>(gv + (seq_tok + c0 + t) * D + row_wg + r);
                const G* ev = reinterpret_cast<const G*>(&rv);
#pragma unroll
                for (int e = 0; e < VEC; ++e) vv[e] = g2f(ev[e]);
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e) vv[e] = 0.f;
            }
#pragma unroll
            for (int e = 0; e < VEC; ++e) sVT[(r + e) * LV + t] = vv[e];
        }
        if (tid < NP) {
            const bool ok = tid < n;
            const size_t gi = seq_tok + c0 + tid;
            sTh[tid] = ok ? p.theta[gi] : 0.f;          // padded tokens write nothing
            sEg[tid] = ok ? p.eta[gi] : 1.f;            // and leave products unchanged
            sAg[tid] = ok ? 1.f - p.alpha[gi] : 1.f;
        }
        __syncthreads();

        // ---- 2. gate scans (wave 0, lane = token) --------------------------
        if (w == 0) {
            const int l = lane;
            const float th = l < NP ? sTh[l] : 0.f;
            const float et = l < NP ? sEg[l] : 1.f;
            const float a = l < NP ? sAg[l] : 1.f;
            // E_i: inclusive prefix product of eta.
            float E = et;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const float y = __shfl_up(E, o);
                if (l >= o) E *= y;
            }
            // (A_i, c_i): prefix composition of the affine maps x -> a_i x + E_i.
            float m = a, cc = E;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const float mp = __shfl_up(m, o);
                const float cp = __shfl_up(cc, o);
                if (l >= o) { cc = m * cp + cc; m = m * mp; }
            }
            // Exclusive suffix products of a and eta (padding lanes hold 1).
            float sa = a, se = et;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const float ya = __shfl_down(sa, o);
                const float ye = __shfl_down(se, o);
                if (l + o < kWave) { sa *= ya; se *= ye; }
            }
            float SA = __shfl_down(sa, 1);
            float SE = __shfl_down(se, 1);
            if (l == kWave - 1) { SA = 1.f; SE = 1.f; }
            // gamma_{n-1,j} = SA_j + eta_{j+1} gamma_{n-1,j+1}, zero past the last token:
            // suffix composition of x -> mu_j x + nu_j.
            const float et_next = __shfl_down(et, 1);
            float mu = (l < n - 1) ? et_next : 0.f;
            float nu = (l < n) ? SA : 0.f;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const float mq = __shfl_down(mu, o);
                const float nq = __shfl_down(nu, o);
                if (l + o < kWave) { nu = mu * nq + nu; mu = mu * mq; }
            }
            if (l < NP) {
                sAv[l] = m;
                sCv[l] = cc;
                sWM[l] = -th * nu;
                sWS[l] = -th * SE;
            }
            if (l == n - 1) { sScal[0] = m; sScal[1] = cc; sScal[2] = E; }

            // Diagonal 16x16 blocks of theta_j gamma_ij: lane = (block, column).
            const int qb = l >> 4, jj = l & 15;
            if (qb < NT) {
                const int j = 16 * qb + jj;
                const float thj = sTh[j];
                float pp = 0.f, gg = 0.f;
#pragma unroll
                for (int s = 0; s < 16; ++s) {
                    const int i = 16 * qb + s;
                    const float ai = sAg[i], ei = sEg[i];
                    if (s == jj) { pp = 1.f; gg = 1.f; }
                    else if (s > jj) { pp = ei * pp; gg = ai * gg + pp; }
                    sGamD[(qb * 16 + s) * 16 + jj] = thj * gg;
                }
                sGend[j] = thj * gg;
                sPend[j] = thj * pp;
            }

            // Transfer maps for rows below a block: Psi_i = T_i ... T_{16*blk(i)}
            // as (X, Y, W) = [[X, Y], [0, W]], then products with whole blocks.
            float X = a, Y = et, W = et;
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) {
                const float xp = __shfl_up(X, o), yp = __shfl_up(Y, o), wp = __shfl_up(W, o);
                if ((l & 15) >= o) { Y = X * yp + Y * wp; X = X * xp; W = W * wp; }
            }
            float BX[NT], BY[NT], BW[NT];
#pragma unroll
            for (int q = 0; q < NT; ++q) {
                BX[q] = __shfl(X, 16 * q + 15);
                BY[q] = __shfl(Y, 16 * q + 15);
                BW[q] = __shfl(W, 16 * q + 15);
            }
            if (l < NP) {
                const int pb = l >> 4;
                float cx = X, cy = Y, cw = W;
#pragma unroll
                for (int q = NT - 2; q >= 0; --q) {
                    if (q < pb) {
                        sPhi[(q * NP + l) * 2 + 0] = cx;
                        sPhi[(q * NP + l) * 2 + 1] = cy;
                        // extend the map over block q for the next block up
                        const float ny = cx * BY[q] + cy * BW[q];
                        cx = cx * BX[q];
                        cw = cw * BW[q];
                        cy = ny;
                    }
                }
            }
        }
        __syncthreads();

        // ---- 3. P = -(tril(Q K^T) .* theta_j gamma_ij), stored as B operand rows
        for (int u = w; u < NT * NT; u += NW) {
            const int pb = u / NT, qb = u % NT;
            const int i = 16 * pb + lr;
            if (pb < qb) {
                O::put4(sP + i * LP, 16 * qb + 4 * lg, f32x4{0.f, 0.f, 0.f, 0.f});
                continue;
            }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NKC; ++s)
                acc = O::mma(acc, O::lds(sK + (16 * qb + lr) * LQ, s, lg), O::lds(sQ + i * LQ, s, lg));
            // acc[e] = q_i . k_j for j = 16qb + 4lg + e
            f32x4 L;
            if (pb == qb) {
                L = *reinterpret_cast<const f32x4*>(sGamD + (qb * 16 + lr) * 16 + 4 * lg);
            } else {
                const float x = sPhi[(qb * NP + i) * 2 + 0];
                const float y = sPhi[(qb * NP + i) * 2 + 1];
                const f32x4 gv = *reinterpret_cast<const f32x4*>(sGend + 16 * qb + 4 * lg);
                const f32x4 pv = *reinterpret_cast<const f32x4*>(sPend + 16 * qb + 4 * lg);
                L = x * gv + y * pv;
            }
            O::put4(sP + i * LP, 16 * qb + 4 * lg, -(acc * L));
        }
        __syncthreads();

        // ---- 4. residuals, read-out and state update (per wave) ------------
        using F = typename O::frag;
        F MB[NKC], SB[NKC];
#pragma unroll
        for (int s = 0; s < NKC; ++s) {
            MB[s] = O::template from_acc<NC>(Macc, s);
            SB[s] = O::template from_acc<NC>(Sacc, s);
        }
        // E = K M0^T - V; lane (lr, lg) of tile tt holds E[16tt + 4lg + e][row_w + lr].
        f32x4 Eacc[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            Eacc[tt] = -*reinterpret_cast<const f32x4*>(sVT + (16 * w + lr) * LV + 16 * tt + 4 * lg);
#pragma unroll
            for (int s = 0; s < NKC; ++s)
                Eacc[tt] = O::mma(Eacc[tt], O::lds(sK + (16 * tt + lr) * LQ, s, lg), MB[s]);
        }
        // Z^T = A.(M0 Q^T) + c.(S0 Q^T) + E^T P^T; lane (lr, lg) of tile tt holds
        // z[token 16tt + lr][row_w + 4lg + e].
        F EB[NKT];
#pragma unroll
        for (int s = 0; s < NKT; ++s) EB[s] = O::template from_acc<NT>(Eacc, s);
        const size_t zrow0 = (seq_tok + c0) * D + row_w + 4 * lg;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            f32x4 za = {0.f, 0.f, 0.f, 0.f}, zc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NKC; ++s) {
                const F bq = O::lds(sQ + (16 * tt + lr) * LQ, s, lg);
                za = O::mma(za, MB[s], bq);
                zc = O::mma(zc, SB[s], bq);
            }
            const int t = 16 * tt + lr;
            f32x4 zt = sAv[t] * za + sCv[t] * zc;
#pragma unroll
            for (int s = 0; s < NKT; ++s)
                if (KG * s <= 16 * tt + 15) zt = O::mma(zt, EB[s], O::lds(sP + t * LP, s, lg));
            if (t < n) *reinterpret_cast<f32x4*>(p.z + zrow0 + static_cast<size_t>(t) * D) = zt;
        }
        // M <- A_n M0 + c_n S0 + (K^T (w^M . E))^T,  S <- E_n S0 + (K^T (w^S . E))^T
        f32x4 EM[NT], ES[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            EM[tt] = Eacc[tt] * *reinterpret_cast<const f32x4*>(sWM + 16 * tt + 4 * lg);
            ES[tt] = Eacc[tt] * *reinterpret_cast<const f32x4*>(sWS + 16 * tt + 4 * lg);
        }
        F WMB[NKT], WSB[NKT];
#pragma unroll
        for (int s = 0; s < NKT; ++s) {
            WMB[s] = O::template from_acc<NT>(EM, s);
            WSB[s] = O::template from_acc<NT>(ES, s);
        }
        const float An = sScal[0], Cn = sScal[1], En = sScal[2];
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
            Macc[ct] = An * Macc[ct] + Cn * Sacc[ct];
            Sacc[ct] = En * Sacc[ct];
#pragma unroll
            for (int s = 0; s < NKT; ++s) {
                const F a = O::lds(sKT + (16 * ct + lr) * LKT, s, lg);
                Macc[ct] = O::mma(Macc[ct], a, WMB[s]);
                Sacc[ct] = O::mma(Sacc[ct], a, WSB[s]);
            }
        }
    }

#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
        const int col = 16 * ct + 4 * lg;
        if (p.MT) *reinterpret_cast<f32x4*>(p.MT + state_off + col) = Macc[ct];
        if (p.ST) *reinterpret_cast<f32x4*>(p.ST + state_off + col) = Sacc[ct];
    }
}

// ---------------------------------------------------------------------------
// Host side: validation, instance selection, launch.
// ---------------------------------------------------------------------------
template <typename T, int D, int NW, int NP>
hipError_t launch(const Params& p, hipStream_t stream) {
    constexpr int RB = 16 * NW;
    const long long nwg = static_cast<long long>(p.BH) * (D / RB);
    hipLaunchKernelGGL((linear_memory_fwd<T, D, NW, NP>), dim3(static_cast<unsigned>(nwg)),
                       dim3(kWave * NW), 0, stream, p);
    return hipGetLastError();
}

template <typename T, int D, int NW>
hipError_t launch_np(const Params& p, int np, hipStream_t stream) {
    if constexpr (Op<T>::KG == 32) {
        return np <= 32 ? launch<T, D, NW, 32>(p, stream) : launch<T, D, NW, 64>(p, stream);
    } else {
        if (np <= 16) return launch<T, D, NW, 16>(p, stream);
        if (np <= 32) return launch<T, D, NW, 32>(p, stream);
        return launch<T, D, NW, 64>(p, stream);
    }
}

template <typename T, int D>
hipError_t launch_nw(const Params& p, int np, hipStream_t stream) {
    if constexpr (D >= 32) {
        // Two waves per workgroup when that still leaves >= 256 workgroups.
        const long long row_tiles = static_cast<long long>(p.BH) * (D / 16);
        if (row_tiles >= 512) return launch_np<T, D, 2>(p, np, stream);
    }
    return launch_np<T, D, 1>(p, np, stream);
}

template <typename T>
hipError_t dispatch(const Params& p, int d, hipStream_t stream) {
    const int np = round_up(p.b, 16);
    switch (d) {
        case 16: return launch_nw<T, 16>(p, np, stream);
        case 32: return launch_nw<T, 32>(p, np, stream);
        case 64: return launch_nw<T, 64>(p, np, stream);
        default: return launch_nw<T, 128>(p, np, stream);
    }
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

template <typename T>
int forward_impl(const void* q, const void* k, const void* v, const float* theta, const float* eta,
                 const float* alpha, const float* M0, const float* S0, float* z, float* M_T, float* S_T,
                 int B, int H, int Tlen, int d, int b, void* stream) {
    using G = typename GlobalOf<T>::type;
    if (B < 0 || H < 0 || Tlen < 0) return TTT_ERR_INVALID_ARG;
    if (b < 1) return TTT_ERR_INVALID_ARG;
    if (d != 16 && d != 32 && d != 64 && d != 128) return TTT_ERR_UNSUPPORTED;
    if (b > 64) return TTT_ERR_UNSUPPORTED;
    const long long BH = static_cast<long long>(B) * H;
    if (BH == 0) return TTT_OK;
    if (BH * (d / 16) > 0x7fffffffLL) return TTT_ERR_UNSUPPORTED;
    if (BH * static_cast<long long>(Tlen) > 0x7fffffffLL) return TTT_ERR_UNSUPPORTED;
    const size_t tok = static_cast<size_t>(BH) * static_cast<size_t>(Tlen);
    const size_t in_bytes = tok * d * sizeof(G);
    const size_t z_bytes = tok * d * sizeof(float);
    const size_t st_bytes = static_cast<size_t>(BH) * d * d * sizeof(float);
    if (Tlen > 0) {
        if (!q || !k || !v || !theta || !eta || !alpha || !z) return TTT_ERR_INVALID_ARG;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(z, 16)) return TTT_ERR_INVALID_ARG;
        if (!aligned(theta, 4) || !aligned(eta, 4) || !aligned(alpha, 4)) return TTT_ERR_INVALID_ARG;
        const void* ins[] = {q, k, v};
        for (const void* in : ins)
            if (overlaps(z, z_bytes, in, in_bytes)) return TTT_ERR_INVALID_ARG;
        const void* gates[] = {theta, eta, alpha};
        for (const void* g : gates)
            if (overlaps(z, z_bytes, g, tok * sizeof(float))) return TTT_ERR_INVALID_ARG;
        if (overlaps(z, z_bytes, M0, st_bytes) || overlaps(z, z_bytes, S0, st_bytes) ||
            overlaps(z, z_bytes, M_T, st_bytes) || overlaps(z, z_bytes, S_T, st_bytes))
            return TTT_ERR_INVALID_ARG;
    }
    const void* states[] = {M0, S0, M_T, S_T};
    for (const void* s : states)
        if (s && !aligned(s, 16)) return TTT_ERR_INVALID_ARG;
    // In-place carry is allowed only as exact aliasing (M_T == M0, S_T == S0).
    if (M_T && M_T != M0 && (overlaps(M_T, st_bytes, M0, st_bytes) || overlaps(M_T, st_bytes, S0, st_bytes)))
        return TTT_ERR_INVALID_ARG;
    if (S_T && S_T != S0 && (overlaps(S_T, st_bytes, S0, st_bytes) || overlaps(S_T, st_bytes, M0, st_bytes)))
        return TTT_ERR_INVALID_ARG;
    if (M_T && S_T && overlaps(M_T, st_bytes, S_T, st_bytes)) return TTT_ERR_INVALID_ARG;

    Params p{q, k, v, theta, eta, alpha, M0, S0, z, M_T, S_T, static_cast<int>(BH), Tlen, b};
    const hipError_t err = dispatch<T>(p, d, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

}  // namespace

extern "C" {

int ttt_mem_forward_f32(const float* q, const float* k, const float* v, const float* theta, const float* eta,
                        const float* alpha, const float* M0, const float* S0, float* z, float* M_T, float* S_T,
                        int B, int H, int T, int d, int b, void* stream) {
    return forward_impl<float>(q, k, v, theta, eta, alpha, M0, S0, z, M_T, S_T, B, H, T, d, b, stream);
}

int ttt_mem_forward_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* theta,
                         const float* eta, const float* alpha, const float* M0, const float* S0, float* z,
                         float* M_T, float* S_T, int B, int H, int T, int d, int b, void* stream) {
    return forward_impl<_Float16>(q, k, v, theta, eta, alpha, M0, S0, z, M_T, S_T, B, H, T, d, b, stream);
}

const char* ttt_mem_status_string(int status) {
    switch (status) {
        case TTT_OK: return "ok";
        case TTT_ERR_INVALID_ARG: return "invalid argument";
        case TTT_ERR_UNSUPPORTED: return "unsupported size";
        case TTT_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

int ttt_mem_abi_version(void) { return TTT_MEM_ABI_VERSION; }

}  // extern "C"
