// Chunked TTT deep (two-layer MLP) memory forward for gfx950 (MI355X), and its C ABI.
//
// The memory is f(u) = u + SiLU(u W1) W2 in row-vector form (W1: d x hid,
// W2: hid x d), trained inside the forward pass on 1/2 ||f(k_t) - v_t||^2 with
// the same chunked schedule as the linear memory: every gradient of a chunk
// is taken at the chunk-start weights, each tensor has its own momentum, and
// both use the token's theta, eta, alpha ("论文速览 | Titans", sections 3.4,
// 3.7, 3.9 and 4.2; "Continual Learning: From Attention to Neural Memory",
// sections 4.2 and 5.2).  Explicit backprop at the chunk-start weights, for the
// chunk's keys K, values V and queries Q (rows are tokens):
//
//   Hk = K W1,  Ak = SiLU(Hk),  R = K + Ak W2 - V,  dH = (R W2^T) .* SiLU'(Hk)
//   G1_j = k_j^T dH_j,  G2_j = Ak_j^T R_j
//
// Unrolling the per-token recurrences over the chunk as for the linear memory
// (decay matrix L_ij = theta_j gamma_ij, j <= i; chunk-end weights w^M, w^S):
//
//   Hq = diag(A) Q W1 + diag(c) Q S1 - (L .* Q K^T) dH,   Aq = SiLU(Hq)
//   Z  = Q + diag(A) Aq W2 + diag(c) Aq S2 - (L .* Aq Ak^T) R
//   W1 <- A_n W1 + c_n S1 - K^T diag(w^M) dH,  S1 <- E_n S1 - K^T diag(w^S) dH
//   W2 <- A_n W2 + c_n S2 - Ak^T diag(w^M) R,  S2 <- E_n S2 - Ak^T diag(w^S) R
//
// which is the dual form of "5.1.1 · TTT layers 与 fast weights" section 1.1
// (eqs. (7)-(9)) carried through a nonlinear inner model.
//
// One workgroup per (batch, head) sequence: the MLP couples all rows, so a
// sequence is not split.  NW = hid/32 waves each own 32 hidden units: columns
// of W1 and S1, rows of W2 and S2, kept in fp32 MFMA accumulators for the
// whole sequence.  Everything that contracts over the hidden dimension (R and
// the read Z, and Aq Ak^T) is a sum of per-wave partials reduced through LDS.
// Per chunk:
//   phase 1  all waves: Hk, Hk^T, SiLU, partial R^T; wave 0: P = -(L .* Q K^T)
//   phase 2  R = K - V + sum of partials (fp16 copies [t][d] and [d][t])
//   phase 3  all waves: dH, Hq^T, Aq^T, partial Z^T and (Aq Ak^T)^T, then the
//            update of the own slices of W1, S1, W2, S2
//   phase 4  waves 0..3: z, one 16-column tile each; then the waves stage
//            the next chunk (prefetched into registers in phase 1), and the
//            last wave its gates
//
// MFMA: v_mfma_f32_16x16x16_f16.  An accumulator tile holds rows 4g..4g+3 of
// column n in lane (n, g); an operand fragment holds k-slots 4g..4g+3 of row
// (or column) n.  So an accumulator tile Y converts lane-locally (fp32 ->
// fp16) into the B operand for Y or the A operand for Y^T, and every product
// below is oriented so that its operands come straight from accumulators or
// from row-major LDS rows; the two transposed operands (K^T and W2^T) use the
// gfx950 LDS transpose load.  Operands are fp16 with a power-of-two block
// scale per wave and tensor (weights, momenta, SiLU(Hk), dH), undone exactly
// on the fp32 results, so decayed weights far below fp16's normal range keep
// full relative precision; accumulation and the weights are fp32.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ttt_mem.h"
#include "gfx950.h"

namespace {

constexpr int kD = 64;          // model width d
constexpr int kHid = 256;       // hidden width
constexpr int kNP = 16;         // padded chunk length (b <= 16)
constexpr int kNW = kHid / 32;  // waves: 32 hidden units each
constexpr int kDT = kD / 16;    // 16-wide tiles of d
constexpr int kHT = 2;          // 16-wide hidden tiles per wave
constexpr int kThreads = kNW * 64;
constexpr int kLK = kD + 8;     // LDS row stride (halves) of K, Q, V, R rows: 16-byte aligned, staggered banks
constexpr int kLRT = kNP + 4;   // row stride (floats) of R^T rows
constexpr int kLW = 32 + 4;     // row stride (halves) of a wave's W2^T staging rows

__device__ __forceinline__ f32x4 mma16(f16x4 a, f16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 to_f32(f16x4 h) {
    return f32x4{static_cast<float>(h[0]), static_cast<float>(h[1]), static_cast<float>(h[2]), static_cast<float>(h[3])};
}
// x = hi + lo with both halves fp16 (about 22 significant bits together).
struct Split {
    f16x4 hi, lo;
};
__device__ __forceinline__ Split split(f32x4 x) {
    const f16x4 hi = cvt4(x);
    return Split{hi, cvt4(x - to_f32(hi))};
}
// Product of two split operands, dropping lo * lo.
__device__ __forceinline__ f32x4 mma3(const Split& a, const Split& b, f32x4 c) {
    c = mma16(a.hi, b.hi, c);
    c = mma16(a.hi, b.lo, c);
    return mma16(a.lo, b.hi, c);
}
// Product of an exact fp16 operand and a split one.
__device__ __forceinline__ f32x4 mma2(f16x4 a, const Split& b, f32x4 c) {
    return mma16(a, b.lo, mma16(a, b.hi, c));
}
__device__ __forceinline__ f32x4 mma2(const Split& a, f16x4 b, f32x4 c) {
    return mma16(a.lo, b, mma16(a.hi, b, c));
}

// SiLU and its derivative through the hardware exp2 and reciprocal.
__device__ __forceinline__ float sigm(float x) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.44269504088896341f * x));
}
__device__ __forceinline__ f32x4 silu4(f32x4 x) {
    f32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = x[e] * sigm(x[e]);
    return r;
}
// SiLU(x) and SiLU'(x) = s (1 + x (1 - s)).
__device__ __forceinline__ void silu_d4(f32x4 x, f32x4& y, f32x4& dy) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float s = sigm(x[e]);
        y[e] = x[e] * s;
        dy[e] = s * (1.f + x[e] * (1.f - s));
    }
}

// Largest |x| over the wave (every lane gets it).
__device__ __forceinline__ float wave_max(float m) {
    m = fmaxf(m, dpp_or<kRowShr1, 0xf>(0.f, m));
    m = fmaxf(m, dpp_or<kRowShr2, 0xf>(0.f, m));
    m = fmaxf(m, dpp_or<kRowShr4, 0xf>(0.f, m));
    m = fmaxf(m, dpp_or<kRowShr8, 0xf>(0.f, m));
    m = fmaxf(m, dpp_or<kRowBcast15, 0xa>(0.f, m));
    m = fmaxf(m, dpp_or<kRowBcast31, 0xc>(0.f, m));
    return readlane(m, 63);
}
// Power-of-two block scale: sc = 2^s with m * sc in [32, 64) (1 for m = 0 or
// not finite), inv = 1 / sc.  Operands scaled this way keep fp16's relative
// precision at any magnitude (weights that have decayed far below fp16's
// normal range included), and scaling by a power of two is exact.
struct Pow2 {
    float sc, inv;
};
__device__ __forceinline__ Pow2 pow2_scale(float m) {
    const int e = ((__float_as_int(m) >> 23) & 0xff) - 127;
    int s = 5 - e;
    s = max(-120, min(120, s));
    if (!(m > 0.f) || e == 128) s = 0;
    return Pow2{__int_as_float((127 + s) << 23), __int_as_float((127 - s) << 23)};
}
template <int N>
__device__ __forceinline__ float absmax(const f32x4* x) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(x[i][e]));
    return m;
}

struct MlpParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* theta;
    const float* eta;
    const float* alpha;
    const float* W1;
    const float* W2;
    const float* S1;
    const float* S2;
    void* z;      // float32, or bf16 bits (rounded to nearest even) when z_bf16
    float* W1T;
    float* W2T;
    float* S1T;
    float* S2T;
    int T;
    int b;
    int z_bf16;
};

// One chunk of staged inputs and its gate quantities (double-buffered).
struct ChunkBuf {
    alignas(16) _Float16 kh[kNP * kLK];   // K rows (bf16 -> fp16, exact)
    alignas(16) _Float16 qh[kNP * kLK];   // Q rows
    alignas(16) uint16_t vb[kNP * kLK];   // V rows, raw bf16
    alignas(16) float L[kNP * kNP];       // theta_j gamma_ij, row i, column j (0 above the diagonal)
    alignas(16) float A[kNP];             // A_t
    alignas(16) float C[kNP];             // c_t
    alignas(16) float wm[kNP];            // -w^M_j
    alignas(16) float ws[kNP];            // -w^S_j
    alignas(16) float scal[4];            // A_n, c_n, E_n
};

struct MlpSmem {
    ChunkBuf buf[2];
    alignas(16) f32x4 part[kNW][kDT + 1][64];   // per-wave partial tiles (accumulator layout)
    alignas(16) _Float16 rhi[kNP * kLK];        // R rows [t][d], hi part
    alignas(16) _Float16 rlo[kNP * kLK];        // R rows [t][d], lo part
    alignas(16) float rt[kD * kLRT];            // R^T rows [d][t], float32
    alignas(16) f16x4 pneg[64];                 // -(L .* Q K^T) as B fragments of P^T
    alignas(16) _Float16 w2hi[kNW][kD * kLW];   // each wave's W2^T rows [d][own hidden] (scaled), hi
    alignas(16) _Float16 w2lo[kNW][kD * kLW];   // lo
};

// Registers of one prefetched chunk: thread u (0..255) holds one 16-byte
// unit of K (u < 128) or Q (u >= 128): token (u % 128) / 8, columns
// 8 (u % 8)..+7; threads u < 128 also the same unit of V; the last wave the
// gates of the chunk's tokens (lanes < 16).
struct Prefetch {
    uint4 kq, v;
    float th, et, al;
};

static_assert(kNW >= kDT, "waves 0..3 stage the chunk and own one d-tile each in the reductions");
constexpr int kGateW = kNW - 1;   // gate wave

__device__ void prefetch(Prefetch& pf, const MlpParams& p, size_t seq_tok, int c, int w, int lane) {
    const int c0 = c * p.b;
    const int n = max(0, min(p.b, p.T - c0));
    const uint32_t nbytes = static_cast<uint32_t>(n) * kD * 2;
    const size_t off = (seq_tok + static_cast<size_t>(c0)) * kD;
    const bool kv = w < 2;   // waves 0, 1: K and V; waves 2, 3: Q
    const int u = (w & 1) * 64 + lane;
    const uint32_t boff = static_cast<uint32_t>((u >> 3) * kD + 8 * (u & 7)) * 2;
    if (w < 4) {
        pf.kq = buf_load16(make_rsrc((kv ? p.k : p.q) + off, nbytes), boff);
        if (kv) pf.v = buf_load16(make_rsrc(p.v + off, nbytes), boff);
    }
    if (w == kGateW) {
        const uint32_t gbytes = static_cast<uint32_t>(n) * 4;
        const size_t gi = seq_tok + static_cast<size_t>(c0);
        pf.th = buf_load4(make_rsrc(p.theta + gi, gbytes), lane * 4);
        pf.al = buf_load4(make_rsrc(p.alpha + gi, gbytes), lane * 4);
        pf.et = buf_load4(make_rsrc(p.eta + gi, gbytes), lane * 4);
    }
}

__device__ void stage(const Prefetch& pf, ChunkBuf& B, int w, int lane) {
    const bool kv = w < 2;
    const int u = (w & 1) * 64 + lane;
    const int t = u >> 3, col = 8 * (u & 7);
    f16x8 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t wd = (&pf.kq.x)[e];
        const f16x2 two = cvt2(bf16lo(wd), bf16hi(wd));
        h[2 * e] = two[0];
        h[2 * e + 1] = two[1];
    }
    *reinterpret_cast<f16x8*>((kv ? B.kh : B.qh) + t * kLK + col) = h;
    if (kv) *reinterpret_cast<uint4*>(B.vb + t * kLK + col) = pf.v;
}

// Gate quantities of one chunk, lanes j < 16 of the gate wave: A_j, c_j, the
// decay column j (gamma_ij, p_ij by the column recurrence p <- eta_i p +
// [i = j], gamma <- a_i gamma + p, zero above the diagonal) and the chunk-end
// weights.  Padding tokens read theta = alpha = 0; their eta is taken as 1.
__device__ void gates(const Prefetch& pf, ChunkBuf& B, int n, int lane) {
    const int j = lane;
    const float a = 1.f - pf.al, e = j < n ? pf.et : 1.f, th = pf.th;
    float Aj = 1.f, Ej = 1.f, cj = 0.f, g = 0.f, pe = 0.f, wm = 0.f, ws = 0.f;
    // Not unrolled: an unrolled loop would hoist sixteen per-lane masks out of
    // the chunk loop and keep them in registers for the whole sequence.
#pragma unroll 1
    for (int l = 0; l < kNP; ++l) {
        const float al = readlane(a, l), el = readlane(e, l);
        if (l <= j) {
            Aj *= al;
            Ej *= el;
            cj = al * cj + Ej;
        }
        pe = el * pe + (l == j ? 1.f : 0.f);
        g = al * g + pe;
        if (j < kNP) B.L[l * kNP + j] = th * g;
        if (l == n - 1) {
            wm = th * g;
            ws = th * pe;
        }
    }
    if (j < kNP) {
        B.A[j] = Aj;
        B.C[j] = cj;
        B.wm[j] = -wm;
        B.ws[j] = -ws;
    }
    const float An = readlane(Aj, n - 1), Cn = readlane(cj, n - 1), En = readlane(Ej, n - 1);
    if (j == 0) {
        B.scal[0] = An;
        B.scal[1] = Cn;
        B.scal[2] = En;
    }
}

__global__ __launch_bounds__(kThreads) void mlp_memory_fwd(const MlpParams p) {
    __shared__ MlpSmem sm;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
    const int lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    const int bh = blockIdx.x;
    const int T = p.T, b = p.b;
    const int nch = (T + b - 1) / b;
    const size_t seq_tok = static_cast<size_t>(bh) * T;
    const int h0 = 32 * w;
    auto chunk_n = [&](int c) { return min(b, T - c * b); };

    // ---- resident weights: own hidden columns of W1, S1 and rows of W2, S2 ----
    // W1t[dt][ht], lane (n, g): W1[16dt + 4g + e][h0 + 16ht + n]; W2t[ht][dt]: W2[h0 + 16ht + 4g + e][16dt + n].
    f32x4 W1t[kDT][kHT], S1t[kDT][kHT], W2t[kHT][kDT], S2t[kHT][kDT];
    {
        const size_t wo = static_cast<size_t>(bh) * kD * kHid;
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
            for (int ht = 0; ht < kHT; ++ht)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const size_t i1 = wo + static_cast<size_t>(16 * dt + 4 * lg + e) * kHid + h0 + 16 * ht + lr;
                    const size_t i2 = wo + static_cast<size_t>(h0 + 16 * ht + 4 * lg + e) * kD + 16 * dt + lr;
                    W1t[dt][ht][e] = p.W1[i1];
                    S1t[dt][ht][e] = p.S1 ? p.S1[i1] : 0.f;
                    W2t[ht][dt][e] = p.W2[i2];
                    S2t[ht][dt][e] = p.S2 ? p.S2[i2] : 0.f;
                }
    }

    // ---- zero staging memory, stage chunk 0 ----
    {
        uint32_t* words = reinterpret_cast<uint32_t*>(&sm);
        for (int i = tid; i < static_cast<int>(sizeof(sm) / 4); i += kThreads) words[i] = 0u;
    }
    __syncthreads();
    Prefetch pf;
    const bool stager = w < 4 || w == kGateW;
    if (stager) prefetch(pf, p, seq_tok, 0, w, lane);
    if (nch > 0) {
        if (w < 4) stage(pf, sm.buf[0], w, lane);
        if (w == kGateW) gates(pf, sm.buf[0], chunk_n(0), lane);
    }
    __syncthreads();

    for (int c = 0; c < nch; ++c) {
        const ChunkBuf& B = sm.buf[c & 1];
        const int n = chunk_n(c);
        if (stager) prefetch(pf, p, seq_tok, c + 1, w, lane);

        // ================= phase 1 =================
        // Gradient path at full split precision: Hk = K W1, Ak = SiLU(Hk),
        // partial R^T = W2^T Ak^T over own hidden units.
        const Pow2 g1 = pow2_scale(wave_max(absmax<kDT * kHT>(&W1t[0][0])));
        const Pow2 g2 = pow2_scale(wave_max(absmax<kDT * kHT>(&W2t[0][0])));
        Split Akh[kHT];     // SiLU(Hk) * g1.sc [t x h]
        f16x4 AkTh[kHT];    // SiLU(Hk^T) * g1.sc [h x t], hi part (read path)
        f32x4 dAk[kHT];     // SiLU'(Hk) [t x h]
        {
            f32x4 r[kDT];
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt) r[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ht = 0; ht < kHT; ++ht) {
                f32x4 hkt = {0.f, 0.f, 0.f, 0.f}, hk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int dt = 0; dt < kDT; ++dt) {
                    const f16x4 kf = *reinterpret_cast<const f16x4*>(B.kh + lr * kLK + 16 * dt + 4 * lg);
                    const Split w1 = split(W1t[dt][ht] * g1.sc);
                    hkt = mma2(w1, kf, hkt);   // (W1^T K^T)[h][t]
                    hk = mma2(kf, w1, hk);     // (K W1)[t][h]
                }
                const Split akt = split(silu4(hkt * g1.inv) * g1.sc);
                AkTh[ht] = akt.hi;
                f32x4 ak;
                silu_d4(hk * g1.inv, ak, dAk[ht]);
                Akh[ht] = split(ak * g1.sc);
#pragma unroll
                for (int dt = 0; dt < kDT; ++dt) {
                    const Split w2 = split(W2t[ht][dt] * g2.sc);
                    r[dt] = mma3(w2, akt, r[dt]);
                    // W2^T staging (scaled by g2) for the transpose loads of phase 3:
                    // row d = 16dt + lr, own hidden 16ht + 4g..+3.
                    const int o = (16 * dt + lr) * kLW + 16 * ht + 4 * lg;
                    *reinterpret_cast<f16x4*>(sm.w2hi[w] + o) = w2.hi;
                    *reinterpret_cast<f16x4*>(sm.w2lo[w] + o) = w2.lo;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            const float unscale = g1.inv * g2.inv;
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt) sm.part[w][dt][lane] = r[dt] * unscale;
        }
        if (w == 0) {
            // S = K Q^T [j x t]: lane (t, g) holds (Q K^T)[t][4g..+3]; P^T fragment = -(L .* that).
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt) {
                const f16x4 kf = *reinterpret_cast<const f16x4*>(B.kh + lr * kLK + 16 * dt + 4 * lg);
                const f16x4 qf = *reinterpret_cast<const f16x4*>(B.qh + lr * kLK + 16 * dt + 4 * lg);
                s = mma16(kf, qf, s);
            }
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(B.L + lr * kNP + 4 * lg);
            sm.pneg[lane] = cvt4(-(s * l4));
        }
        __syncthreads();

        // ================= phase 2: R = K - V + sum of partials =================
        if (w < kDT) {
            const int dt = w;
            f32x4 r = sm.part[0][dt][lane];
#pragma unroll
            for (int ww = 1; ww < kNW; ++ww) r += sm.part[ww][dt][lane];
            // r[e] = R^T[d = 16dt + 4lg + e][t = lr] partial; add K - V at (t, d).
            const int t = lr, d0 = 16 * dt + 4 * lg;
            const f16x4 k4 = *reinterpret_cast<const f16x4*>(B.kh + t * kLK + d0);
            const u32x2 v2 = *reinterpret_cast<const u32x2*>(B.vb + t * kLK + d0);
            r[0] += static_cast<float>(k4[0]) - bf16lo(v2[0]);
            r[1] += static_cast<float>(k4[1]) - bf16hi(v2[0]);
            r[2] += static_cast<float>(k4[2]) - bf16lo(v2[1]);
            r[3] += static_cast<float>(k4[3]) - bf16hi(v2[1]);
            const Split rs = split(r);
            *reinterpret_cast<f16x4*>(sm.rhi + t * kLK + d0) = rs.hi;
            *reinterpret_cast<f16x4*>(sm.rlo + t * kLK + d0) = rs.lo;
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.rt[(d0 + e) * kLRT + t] = r[e];
        }
        __syncthreads();

        // ================= phase 3 =================
        // Opaque to the compiler: fp16 copies of the weights made in phase 1
        // are recomputed here instead of being kept live across the phases.
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
            for (int ht = 0; ht < kHT; ++ht)
                asm volatile("" : "+v"(W1t[dt][ht]), "+v"(S1t[dt][ht]), "+v"(W2t[ht][dt]), "+v"(S2t[ht][dt]));
        {
            const float At = B.A[lr], Ct = B.C[lr];
            const Pow2 gs1 = pow2_scale(wave_max(absmax<kDT * kHT>(&S1t[0][0])));
            const Pow2 gs2 = pow2_scale(wave_max(absmax<kDT * kHT>(&S2t[0][0])));
            // dH [t x h] = R W2^T .* SiLU'(Hk) (split operands), then its own block scale gd.
            f32x4 dH[kHT];
#pragma unroll
            for (int ht = 0; ht < kHT; ++ht) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int dt = 0; dt < kDT; ++dt) {
                    const int ro = lr * kLK + 16 * dt + 4 * lg;
                    const Split rf{*reinterpret_cast<const f16x4*>(sm.rhi + ro), *reinterpret_cast<const f16x4*>(sm.rlo + ro)};
                    // B = W2^T (k = d, n = h): transpose loads of the wave's W2^T rows.
                    const int wo = (16 * dt + 4 * lg + (lr >> 2)) * kLW + 16 * ht + 4 * (lr & 3);
                    const Split wt{__builtin_bit_cast(f16x4, ds_read_tr16(sm.w2hi[w] + wo)),
                                   __builtin_bit_cast(f16x4, ds_read_tr16(sm.w2lo[w] + wo))};
                    acc = mma3(rf, wt, acc);
                }
                dH[ht] = acc * g2.inv * dAk[ht];
            }
            const Pow2 gd = pow2_scale(wave_max(absmax<kHT>(dH)));
            // Read path (single fp16 operands): Hq^T [h x t] = A_t W1^T Q^T + c_t S1^T Q^T + dH^T P^T.
            const f16x4 pn = sm.pneg[lane];
            f16x4 AqTh[kHT];
#pragma unroll
            for (int ht = 0; ht < kHT; ++ht) {
                f32x4 za = {0.f, 0.f, 0.f, 0.f}, zc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int dt = 0; dt < kDT; ++dt) {
                    const f16x4 qf = *reinterpret_cast<const f16x4*>(B.qh + lr * kLK + 16 * dt + 4 * lg);
                    za = mma16(cvt4(W1t[dt][ht] * g1.sc), qf, za);
                    zc = mma16(cvt4(S1t[dt][ht] * gs1.sc), qf, zc);
                }
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                const f32x4 intra = mma16(cvt4(dH[ht] * gd.sc), pn, zero);
                const f32x4 hq = (At * g1.inv) * za + (Ct * gs1.inv) * zc + gd.inv * intra;
                AqTh[ht] = cvt4(silu4(hq));
            }
            // Partial Z^T [d x t] = A_t W2^T Aq^T + c_t S2^T Aq^T over own hidden units.
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt) {
                f32x4 za = {0.f, 0.f, 0.f, 0.f}, zc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ht = 0; ht < kHT; ++ht) {
                    za = mma16(cvt4(W2t[ht][dt] * g2.sc), AqTh[ht], za);
                    zc = mma16(cvt4(S2t[ht][dt] * gs2.sc), AqTh[ht], zc);
                }
                sm.part[w][dt][lane] = (At * g2.inv) * za + (Ct * gs2.inv) * zc;
            }
            // Partial (Aq Ak^T)^T [j x i]: lane (i, g) holds (Aq Ak^T)[i][4g..+3].
            {
                f32x4 gacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ht = 0; ht < kHT; ++ht) gacc = mma16(AkTh[ht], AqTh[ht], gacc);
                sm.part[w][kDT][lane] = gacc * g1.inv;
            }
            __builtin_amdgcn_sched_barrier(0);
            // Carry (gradient path, split operands).  Token weights -w^M, -w^S
            // scale the k-slot rows t = 4g + e of the B operands.
            const float An = B.scal[0], Cn = B.scal[1], En = B.scal[2];
            const f32x4 wm4 = *reinterpret_cast<const f32x4*>(B.wm + 4 * lg);
            const f32x4 ws4 = *reinterpret_cast<const f32x4*>(B.ws + 4 * lg);
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            // R^T rows for the W2 carry: lane (d = 16dt + lr, g) holds R[4g..+3][d].
            f32x4 rt4[kDT];
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt) rt4[dt] = *reinterpret_cast<const f32x4*>(sm.rt + (16 * dt + lr) * kLRT + 4 * lg);
            const Pow2 gr = pow2_scale(wave_max(absmax<kDT>(rt4) * fmaxf(absmax<1>(&wm4), absmax<1>(&ws4))));
#pragma unroll
            for (int ht = 0; ht < kHT; ++ht) {
                const Split dm = split(dH[ht] * wm4 * gd.sc), ds = split(dH[ht] * ws4 * gd.sc);
#pragma unroll
                for (int dt = 0; dt < kDT; ++dt) {
                    // A = K^T (m = d, k = t) by transpose load of the K rows.
                    const f16x4 kt = __builtin_bit_cast(f16x4, ds_read_tr16(B.kh + (4 * lg + (lr >> 2)) * kLK + 16 * dt + 4 * (lr & 3)));
                    const f32x4 w1 = An * W1t[dt][ht] + Cn * S1t[dt][ht];
                    S1t[dt][ht] = En * S1t[dt][ht] + gd.inv * mma2(kt, ds, zero);
                    W1t[dt][ht] = w1 + gd.inv * mma2(kt, dm, zero);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt) {
                const Split rm = split(rt4[dt] * wm4 * gr.sc), rs = split(rt4[dt] * ws4 * gr.sc);
                const float unscale = g1.inv * gr.inv;
#pragma unroll
                for (int ht = 0; ht < kHT; ++ht) {
                    const f32x4 w2 = An * W2t[ht][dt] + Cn * S2t[ht][dt];
                    S2t[ht][dt] = En * S2t[ht][dt] + unscale * mma3(Akh[ht], rs, zero);
                    W2t[ht][dt] = w2 + unscale * mma3(Akh[ht], rm, zero);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __syncthreads();

        // ================= phase 4 =================
        const bool zb = p.z_bf16 != 0;
        const uint32_t zsz = zb ? 2u : 4u;
        const auto rz = make_rsrc(static_cast<char*>(p.z) + (seq_tok + static_cast<size_t>(c) * b) * kD * zsz,
                                  static_cast<uint32_t>(n) * kD * zsz);
        if (w < kDT) {
            // z^T tile dt = w [d x t] = Q^T + sum of partial Z^T + R^T (-(L .* Aq Ak^T))^T.
            const int dt = w;
            f32x4 g = sm.part[0][kDT][lane];
            f32x4 zt = sm.part[0][dt][lane];
#pragma unroll
            for (int ww = 1; ww < kNW; ++ww) {
                g += sm.part[ww][kDT][lane];
                zt += sm.part[ww][dt][lane];
            }
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(B.L + lr * kNP + 4 * lg);
            const f16x4 gb = cvt4(-(g * l4));   // B fragment: lane (t, g) holds -(L .* Aq Ak^T)[t][4g..+3]
            // A = R^T (m = d, k = j): lane (d, g) holds R[4g..+3][d].
            const f16x4 ra = cvt4(*reinterpret_cast<const f32x4*>(sm.rt + (16 * dt + lr) * kLRT + 4 * lg));
            zt = mma16(ra, gb, zt);
            // zt lane (t = lr, g) holds z^T[16dt + 4g + e][t]: add q and store the 4 columns of token t.
            const int t = lr, d0 = 16 * dt + 4 * lg;
            const f16x4 q4 = *reinterpret_cast<const f16x4*>(B.qh + t * kLK + d0);
            zt += to_f32(q4);
            store_out4(zt, rz, static_cast<uint32_t>(t * kD + d0), zb);
        }
        if (c + 1 < nch) {
            ChunkBuf& Bn = sm.buf[(c + 1) & 1];
            if (w < 4) stage(pf, Bn, w, lane);
            if (w == kGateW) gates(pf, Bn, chunk_n(c + 1), lane);
        }
        __syncthreads();
    }

    // ---- final weights ----
    {
        // Lane indices recomputed behind an opaque copy, so that the compiler
        // does not keep the prologue's per-element addresses alive (in
        // registers or spilled) for the whole sequence.
        int tid2 = threadIdx.x;
        asm volatile("" : "+v"(tid2));
        const int lr = tid2 & 15, lg = (tid2 >> 4) & 3;
        const size_t wo = static_cast<size_t>(bh) * kD * kHid;
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
            for (int ht = 0; ht < kHT; ++ht)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const size_t i1 = wo + static_cast<size_t>(16 * dt + 4 * lg + e) * kHid + h0 + 16 * ht + lr;
                    const size_t i2 = wo + static_cast<size_t>(h0 + 16 * ht + 4 * lg + e) * kD + 16 * dt + lr;
                    if (p.W1T) p.W1T[i1] = W1t[dt][ht][e];
                    if (p.S1T) p.S1T[i1] = S1t[dt][ht][e];
                    if (p.W2T) p.W2T[i2] = W2t[ht][dt][e];
                    if (p.S2T) p.S2T[i2] = S2t[ht][dt][e];
                }
    }
}

int mlp_forward_impl(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* theta, const float* eta,
                     const float* alpha, const float* W1_0, const float* W2_0, const float* S1_0, const float* S2_0,
                     void* z, float* W1_T, float* W2_T, float* S1_T, float* S2_T, int B, int H, int Tlen, int d,
                     int hidden, int b, void* stream, bool z_bf16) {
    if (B < 0 || H < 0 || Tlen < 0 || b < 1) return TTT_ERR_INVALID_ARG;
    if (d != kD || hidden != kHid || b > kNP) return TTT_ERR_UNSUPPORTED;
    const long long BH = static_cast<long long>(B) * H;
    if (BH == 0) return TTT_OK;
    if (BH > 0x7fffffffLL || BH * static_cast<long long>(Tlen) > 0x7fffffffLL) return TTT_ERR_UNSUPPORTED;
    if (!W1_0 || !W2_0) return TTT_ERR_INVALID_ARG;
    const size_t tok = static_cast<size_t>(BH) * static_cast<size_t>(Tlen);
    const size_t in_bytes = tok * kD * 2, z_bytes = tok * kD * (z_bf16 ? 2 : 4);
    const size_t w_bytes = static_cast<size_t>(BH) * kD * kHid * 4;
    if (Tlen > 0) {
        if (!q || !k || !v || !theta || !eta || !alpha || !z) return TTT_ERR_INVALID_ARG;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(z, 16)) return TTT_ERR_INVALID_ARG;
        if (!aligned(theta, 4) || !aligned(eta, 4) || !aligned(alpha, 4)) return TTT_ERR_INVALID_ARG;
        const void* ins[] = {q, k, v};
        for (const void* in : ins)
            if (overlaps(z, z_bytes, in, in_bytes)) return TTT_ERR_INVALID_ARG;
        const void* gs[] = {theta, eta, alpha};
        for (const void* g : gs)
            if (overlaps(z, z_bytes, g, tok * 4)) return TTT_ERR_INVALID_ARG;
        const void* ws[] = {W1_0, W2_0, S1_0, S2_0, W1_T, W2_T, S1_T, S2_T};
        for (const void* x : ws)
            if (overlaps(z, z_bytes, x, w_bytes)) return TTT_ERR_INVALID_ARG;
    }
    const void* all[] = {W1_0, W2_0, S1_0, S2_0, W1_T, W2_T, S1_T, S2_T};
    for (const void* x : all)
        if (x && !aligned(x, 4)) return TTT_ERR_INVALID_ARG;
    // Outputs may alias their own initial tensor (in-place carry) but nothing else.
    const void* outs[] = {W1_T, W2_T, S1_T, S2_T};
    const void* own[] = {W1_0, W2_0, S1_0, S2_0};
    for (int i = 0; i < 4; ++i) {
        if (!outs[i]) continue;
        for (int j = 0; j < 4; ++j) {
            if (own[j] && outs[i] != own[i] && overlaps(outs[i], w_bytes, own[j], w_bytes)) return TTT_ERR_INVALID_ARG;
            if (j != i && outs[j] && overlaps(outs[i], w_bytes, outs[j], w_bytes)) return TTT_ERR_INVALID_ARG;
            if (j != i && own[j] && outs[i] == own[i] && overlaps(outs[i], w_bytes, own[j], w_bytes))
                return TTT_ERR_INVALID_ARG;
        }
    }
    MlpParams p{q, k, v, theta, eta, alpha, W1_0, W2_0, S1_0, S2_0, z, W1_T, W2_T, S1_T, S2_T, Tlen, b, z_bf16 ? 1 : 0};
    hipLaunchKernelGGL(mlp_memory_fwd, dim3(static_cast<unsigned>(BH)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), p);
    return hipGetLastError() == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

}  // namespace

extern "C" int ttt_mem_mlp_forward_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* theta,
                                        const float* eta, const float* alpha, const float* W1_0, const float* W2_0,
                                        const float* S1_0, const float* S2_0, uint16_t* z, float* W1_T, float* W2_T,
                                        float* S1_T, float* S2_T, int B, int H, int T, int d, int hidden, int b,
                                        void* stream) {
    return mlp_forward_impl(q, k, v, theta, eta, alpha, W1_0, W2_0, S1_0, S2_0, z, W1_T, W2_T, S1_T, S2_T, B, H, T, d,
                            hidden, b, stream, true);
}

extern "C" int ttt_mem_mlp_forward_bf16_zf32(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                             const float* theta, const float* eta, const float* alpha,
                                             const float* W1_0, const float* W2_0, const float* S1_0,
                                             const float* S2_0, float* z, float* W1_T, float* W2_T, float* S1_T,
                                             float* S2_T, int B, int H, int T, int d, int hidden, int b,
                                             void* stream) {
    return mlp_forward_impl(q, k, v, theta, eta, alpha, W1_0, W2_0, S1_0, S2_0, z, W1_T, W2_T, S1_T, S2_T, B, H, T, d,
                            hidden, b, stream, false);
}
