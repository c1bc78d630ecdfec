// Chunked TTT / Titans linear memory forward for gfx950 (MI355X), and its C ABI.
//
// What one workgroup does.  It owns RB = 16*NS consecutive rows of the memory
// of one (batch, head) sequence and walks that sequence chunk by chunk.  Rows
// of a linear memory evolve independently (row i only ever meets value
// coordinate i), so the row blocks of one sequence never communicate.  The
// workgroup has two kinds of waves, each running its own loop (the loops
// execute the same barriers):
//
//   * NS state waves.  Each keeps a 16-row slice of M and of the momentum S in
//     MFMA accumulator registers for the whole sequence (the state never
//     leaves the chip between chunks) and, per chunk, runs the dual form:
//        E   = K M0^T - V                          (residuals at chunk start)
//        Z^T = A.(M0 Q^T) + c.(S0 Q^T) + E^T P^T   (reads of every token)
//        M   <- A_n M0 + c_n S0 + (K^T (w^M . E))^T
//        S   <- E_n S0 + (K^T (w^S . E))^T
//   * two producer waves, one chunk ahead of the state waves.  They prefetch
//     the next chunks' q, k, v and gates from HBM into registers, stage them
//     in double-buffered LDS as MFMA operands, scan the gates, and build the
//     intra-chunk weight matrix P = -(tril(Q K^T) .* theta_j gamma_ij)
//     together with the chunk-end weights w^M, w^S.
//
// Per token this is S_t = eta_t S_{t-1} - theta_t grad, M_t = (1 - alpha_t)
// M_{t-1} + S_t, z_t = M_t q_t ("论文速览 | Titans", sections 3.4 and 3.7), with
// every gradient of a chunk taken at the chunk-start memory (same page,
// section 4.2; "5.1.1 · TTT layers 与 fast weights", section 1.1, eq. (6)),
// unrolled over the chunk.  With alpha = eta = 0 it is the dual form of that
// page's eqs. (7)-(9); decay and momentum unrolling follow "论文速览 | Titans"
// sections 4.3-4.5.
//
// Gate algebra (a = 1 - alpha; within a chunk, tokens i = 0..n-1):
//   A_i = prod_{l<=i} a_l,  E_i = prod_{l<=i} eta_l,  c_i = a_i c_{i-1} + E_i,
//   gamma_ij = sum_{m=j..i} (prod_{l=m+1..i} a_l)(prod_{l=j+1..m} eta_l),
//   w^M_j = -theta_j gamma_{n-1,j},  w^S_j = -theta_j prod_{l=j+1..n-1} eta_l.
// All of them are entries of products of the 2x2 maps T_l = [[a_l, eta_l],
// [0, eta_l]]:  T_i...T_0 = [[A_i, c_i], [0, E_i]], and column j of gamma
// follows (gamma_ij, p_ij) = T_i...T_{j+1} (1, 1).  One DPP scan of these
// maps across the 64 lanes (lane = token) gives A, c, E and, after its first
// four steps, the maps from each 16-token block start; 16x16 blocks on the
// diagonal of gamma run the column recurrence directly and blocks below it
// apply block maps to the column states at the end of their own block.  Only
// products and sums appear -- no ratio of cumulative products (the pages'
// beta_t / beta_i) -- so gates equal to 0 (eta = 0, alpha = 1) are exact.
//
// MFMA operand layout.  An accumulator tile holds, in lane (n, g), rows
// 4g..4g+3 of column n.  Keeping M transposed (tiles of M^T) therefore puts in
// each lane four consecutive columns of one row of M -- a k-slot group of an
// MFMA operand when the contraction runs over those columns -- so M, S and E
// feed the next products straight from registers.  On the fp16 path a
// 32-wide k-group holds two 16-row tiles; tile 2s+h, row m stands for index
// 32s + 8(m/4) + 4h + m%4, so that lane group g of a fragment carries the
// eight consecutive indices 32s + 8g .. 32s + 8g + 7, and LDS operands are
// plain row-major tiles (XOR-swizzled in 16-byte chunks to avoid LDS bank
// conflicts).  Operands that are needed transposed (k for the state update,
// v for the residuals) are read with the gfx950 LDS transpose load
// (ds_read_b64_tr_b16), so no transposed copy is staged.
//
// Precision.  The float32 path uses float32 MFMA (v_mfma_f32_16x16x4_f32).
// The bf16-input path uses fp16 operands (v_mfma_f32_16x16x32_f16, same rate
// as bf16 on gfx950, 3 more mantissa bits): bf16 q and k convert to fp16
// exactly in the fp16 normal range, and M0, S0, E, P and the chunk weights are
// rounded to fp16 once per chunk where they enter a product; accumulation and
// the carried state are float32.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ttt_mem.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kProducers = 2;
constexpr int kLdsBytes = 160 * 1024;

__host__ __device__ constexpr int round_up(int x, int m) { return (x + m - 1) / m * m; }
__host__ __device__ constexpr int cdiv(int x, int m) { return (x + m - 1) / m; }
__host__ __device__ constexpr int cmax(int a, int b) { return a > b ? a : b; }

// 16-byte chunk swizzle of a row-major fp16 tile with NCH chunks per row:
// conflict-free for 16 lanes reading one chunk of 16 interleaved tile rows and
// for the transpose loads of the state update.
template <int NCH>
__device__ __forceinline__ int swz(int t) {
    if constexpr (NCH >= 16) {
        return ((t & 3) << 2) | ((t >> 3) & 3);
    } else if constexpr (NCH == 8) {
        return ((t >> 1) & 1) | (((t >> 3) & 1) << 1) | ((((t >> 1) ^ (t >> 4)) & 1) << 2);
    } else if constexpr (NCH == 4) {
        return (t >> 3) & 3;
    } else {
        return 0;
    }
}

// LDS transpose load of four 16-bit elements (gfx950).  Within each group of
// 16 lanes, lane i receives element i%4 of the chunk read by lane 4j + i/4 in
// slot j.
__device__ __forceinline__ i16x4 ds_read_tr16(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(reinterpret_cast<uintptr_t>(p)));
}

// ---------------------------------------------------------------------------
// MFMA operand traits.  A "k-group" is the contraction length of one operand
// fragment: 16 for float32 (four v_mfma_f32_16x16x4_f32, one slot each) and 32
// for fp16 (one v_mfma_f32_16x16x32_f16, eight slots).  tmap(tile, m) is the
// index (token or key column) that row m of a 16-row tile stands for; lane
// group g of the fragment for k-group s carries the indices tmap(tile, 4g+i)
// of the k-group's tiles in slot order, which is the accumulator's own row
// order, so accumulator tiles convert to fragments lane-locally.
// ---------------------------------------------------------------------------
template <typename T>
struct Op;

template <>
struct Op<float> {
    static constexpr int KG = 16;
    static constexpr bool kF16 = false;
    using frag = f32x4;
    __device__ static int tmap(int tile, int m) { return 16 * tile + m; }
    __device__ static f32x4 mma(f32x4 acc, const frag& a, const frag& b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
        return acc;
    }
    template <int NTILES>
    __device__ static frag from_acc(const f32x4* tiles, int s) { return tiles[s]; }
};

template <>
struct Op<_Float16> {
    static constexpr int KG = 32;
    static constexpr bool kF16 = true;
    using frag = f16x8;
    __device__ static int tmap(int tile, int m) {
        return 32 * (tile >> 1) + 8 * (m >> 2) + 4 * (tile & 1) + (m & 3);
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
};

// Global-memory element types: float for the f32 path, raw bf16 bits for the
// bf16-input path (whose matrix operands are fp16).
template <typename T> struct GlobalOf;
template <> struct GlobalOf<float> { using type = float; };
template <> struct GlobalOf<_Float16> { using type = uint16_t; };

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// DPP move with an identity for lanes that have no source (gfx9 controls).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or(float identity, float src) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, identity),
                                                                 __builtin_bit_cast(int, src), CTRL, ROW_MASK,
                                                                 0xf, false));
}
// One inclusive-scan step over 2x2 upper-triangular maps [[X, Y], [0, W]]:
// mine <- mine * earlier (the earlier map is applied first).
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ void tri_step(float& X, float& Y, float& W) {
    const float xs = dpp_or<CTRL, ROW_MASK>(1.f, X);
    const float ys = dpp_or<CTRL, ROW_MASK>(0.f, Y);
    const float ws = dpp_or<CTRL, ROW_MASK>(1.f, W);
    Y = X * ys + Y * ws;
    X = X * xs;
    W = W * ws;
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

__device__ __forceinline__ float readlane(float x, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

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

// Compile-time geometry of one kernel instance.
template <typename T, int D, int NS, int NP>
struct Geo {
    using O = Op<T>;
    using G = typename GlobalOf<T>::type;
    static constexpr bool F16 = O::kF16;
    static constexpr int KG = O::KG;
    static constexpr int DS = F16 ? cmax(D, 32) : D;  // stored key width (fp16: >= one k-group)
    static constexpr int RB = 16 * NS;                // rows of M per workgroup
    static constexpr int NRB = D / RB;                // workgroups per sequence
    static constexpr int NC = DS / 16;                // 16-column tiles of M (incl. padding)
    static constexpr int NT = NP / 16;                // 16-token tiles of a chunk
    static constexpr int NKC = DS / KG;               // k-groups over the key dimension
    static constexpr int NKT = NP / KG;               // k-groups over the chunk's tokens
    // LDS row strides in elements.  fp16: unpadded, 16-byte-chunk swizzled;
    // float32: padded by 16 bytes.
    static constexpr int LQ = F16 ? DS : DS + 4;
    static constexpr int LP = F16 ? NP : NP + 4;
    static constexpr int LKT = NP + 4;                // float32 only: k^T rows
    static constexpr int LV = F16 ? RB : NP + 4;      // fp16: raw bf16 v rows; float32: -v^T rows
    static constexpr int NCHQ = DS * 2 / 16;          // fp16 16-byte chunks per q/k row
    static constexpr int NCHP = NP * 2 / 16;          // fp16 16-byte chunks per P row
    static constexpr int CB = 16 / sizeof(G);         // elements per 16-byte global load
    static constexpr int NQU = NP * (D / CB);         // 16-byte units of q (and of k) per chunk
    static constexpr int NVU = NP * (RB / CB);        // 16-byte units of v per chunk
    static constexpr int QUL = cdiv(NQU, kProducers * kWave);
    static constexpr int VUL = cdiv(NVU, kWave);
    static constexpr int NWAVE = NS + kProducers;
    static constexpr int BUF_BYTES = (2 * NP * LQ + NP * LP + 2 * NP) * (int)sizeof(T) +
                                     (F16 ? NP * LV * 2 : (DS * LKT + RB * LV) * 4) + (2 * NP + 4) * 4;
    static constexpr int HELP_BYTES = (2 * NP + 2 * NT * 256 + NT * NP * 3 + 2 * NP) * 4;
    static constexpr int NBUF = (2 * BUF_BYTES + HELP_BYTES + 1024 <= kLdsBytes) ? 2 : 1;
    static_assert(NP % KG == 0, "chunk padding must fill whole k-groups");
    static_assert(D % RB == 0, "row blocks must tile d");
    static_assert(NBUF * BUF_BYTES + HELP_BYTES + 1024 <= kLdsBytes, "LDS budget");
};

template <typename T, int D, int NS, int NP>
struct Smem {
    using Gm = Geo<T, D, NS, NP>;
    static constexpr bool F16 = Gm::F16;
    struct Buf {
        alignas(16) T q[NP * Gm::LQ];                  // q rows (fp16: swizzled chunks)
        alignas(16) T k[NP * Gm::LQ];                  // k rows
        alignas(16) T p[NP * Gm::LP];                  // -P rows, token dim in fragment order
        alignas(16) T wm[NP];                          // w^M (fragment order = token order)
        alignas(16) T ws[NP];                          // w^S
        // fp16: raw bf16 v rows [token][row]; float32: k^T rows and -v^T rows.
        alignas(16) uint16_t vb[F16 ? NP * Gm::LV : 1];
        alignas(16) float kt[F16 ? 1 : D * Gm::LKT];
        alignas(16) float vn[F16 ? 1 : Gm::RB * Gm::LV];
        alignas(16) float av[NP];                      // A_i
        alignas(16) float cv[NP];                      // c_i
        alignas(16) float scal[4];                     // A_n, c_n, E_n
    };
    Buf buf[Gm::NBUF];
    alignas(16) float ga[NP];              // a of the chunk being prepared
    alignas(16) float ge[NP];              // eta of the chunk being prepared
    alignas(16) float gamd[Gm::NT * 256];  // theta_j gamma_ij on diagonal 16-blocks [blk][i][j]
    alignas(16) float gampd[Gm::NT * 256]; // theta_j p_ij on diagonal 16-blocks
    alignas(16) float phi[Gm::NT * NP * 3];  // maps from the end of block q to row i [q][i][X,Y,W]
    alignas(16) float gend[NP];            // theta_j gamma at the end of column j's block
    alignas(16) float pend[NP];            // theta_j p at the end of column j's block
};

template <typename T, int D, int NS, int NP>
struct Kernel {
    using Gm = Geo<T, D, NS, NP>;
    using O = Op<T>;
    using G = typename Gm::G;
    using F = typename O::frag;
    using S = Smem<T, D, NS, NP>;
    using Buf = typename S::Buf;
    static constexpr bool F16 = Gm::F16;
    static constexpr int NT = Gm::NT, NC = Gm::NC, KG = Gm::KG, NKC = Gm::NKC, NKT = Gm::NKT, DS = Gm::DS;
    static constexpr int LQ = Gm::LQ, LP = Gm::LP, LKT = Gm::LKT, LV = Gm::LV, CB = Gm::CB, RB = Gm::RB;
    static constexpr int NCHQ = Gm::NCHQ, NCHP = Gm::NCHP;
    static constexpr int TPB = KG / 16;   // 16-token tiles per k-group

    // ---- LDS operand access -------------------------------------------------
    // Fragment of k-group s from row t of a q/k tile, lane group g.
    __device__ static F frag_q(const T* base, int t, int s, int g) {
        if constexpr (F16) {
            const int ch = (4 * s + g) ^ swz<NCHQ>(t);
            return *reinterpret_cast<const f16x8*>(base + t * LQ + 8 * ch);
        } else {
            return *reinterpret_cast<const f32x4*>(base + t * LQ + 16 * s + 4 * g);
        }
    }
    __device__ static F frag_p(const T* base, int t, int s, int g) {
        if constexpr (F16) {
            const int ch = (4 * s + g) ^ swz<NCHP>(t);
            return *reinterpret_cast<const f16x8*>(base + t * LP + 8 * ch);
        } else {
            return *reinterpret_cast<const f32x4*>(base + t * LP + 16 * s + 4 * g);
        }
    }
    // Store indices x..x+3 (x % 4 == 0) of row t of a P tile.
    __device__ static void put_p(T* base, int t, int x, f32x4 v) {
        if constexpr (F16) {
            const int ch = (x >> 3) ^ swz<NCHP>(t);
            f16x4 h;
            h[0] = (_Float16)v[0]; h[1] = (_Float16)v[1]; h[2] = (_Float16)v[2]; h[3] = (_Float16)v[3];
            *reinterpret_cast<f16x4*>(base + t * LP + 8 * ch + (x & 4)) = h;
        } else {
            *reinterpret_cast<f32x4*>(base + t * LP + x) = v;
        }
    }
    __device__ static void put_w(T* w, int x, f32x4 v) {
        if constexpr (F16) {
            f16x4 h;
            h[0] = (_Float16)v[0]; h[1] = (_Float16)v[1]; h[2] = (_Float16)v[2]; h[3] = (_Float16)v[3];
            *reinterpret_cast<f16x4*>(w + x) = h;
        } else {
            *reinterpret_cast<f32x4*>(w + x) = v;
        }
    }
    __device__ static F frag_w(const T* w, int s, int g) {
        if constexpr (F16) return *reinterpret_cast<const f16x8*>(w + 32 * s + 8 * g);
        else return *reinterpret_cast<const f32x4*>(w + 16 * s + 4 * g);
    }

    // ---- producers ------------------------------------------------------------
    struct Prefetch {
        uint4 q[Gm::QUL];
        uint4 k[Gm::QUL];
        uint4 v[Gm::VUL];
        float th, et, al;
    };

    // Issue the global loads of chunk c into registers.
    __device__ static void issue(Prefetch& pf, const Params& p, const G* gq, const G* gk, const G* gv,
                                 size_t seq_tok, int row_wg, int c, int ptid, int pw, int lane) {
        const int c0 = c * p.b;
        const int n = min(p.b, p.T - c0);
#pragma unroll
        for (int kk = 0; kk < Gm::QUL; ++kk) {
            const int u = ptid + kProducers * kWave * kk;
            const int t = u / (D / CB), cb = u % (D / CB);
            if (u < Gm::NQU && t < n) {
                const size_t off = (seq_tok + c0 + t) * D + cb * CB;
                pf.q[kk] = *reinterpret_cast<const uint4*>(gq + off);
                pf.k[kk] = *reinterpret_cast<const uint4*>(gk + off);
            } else {
                pf.q[kk] = uint4{0u, 0u, 0u, 0u};
                pf.k[kk] = uint4{0u, 0u, 0u, 0u};
            }
        }
        if (pw == 1) {
#pragma unroll
            for (int kk = 0; kk < Gm::VUL; ++kk) {
                const int u = lane + kWave * kk;
                const int t = u / (RB / CB), rb = u % (RB / CB);
                if (u < Gm::NVU && t < n)
                    pf.v[kk] = *reinterpret_cast<const uint4*>(gv + (seq_tok + c0 + t) * D + row_wg + rb * CB);
                else
                    pf.v[kk] = uint4{0u, 0u, 0u, 0u};
            }
        } else {
            const bool ok = lane < n;
            const size_t gi = seq_tok + c0 + lane;
            pf.th = ok ? p.theta[gi] : 0.f;   // padding tokens write nothing
            pf.et = ok ? p.eta[gi] : 1.f;     // and leave products unchanged
            pf.al = ok ? p.alpha[gi] : 0.f;
        }
    }

    // Registers -> LDS chunk buffer.
    __device__ static void stage(const Prefetch& pf, Buf& B, int ptid, int pw, int lane) {
#pragma unroll
        for (int kk = 0; kk < Gm::QUL; ++kk) {
            const int u = ptid + kProducers * kWave * kk;
            if (u < Gm::NQU) {
                const int t = u / (D / CB), cb = u % (D / CB);
                if constexpr (F16) {
                    const int ch = cb ^ swz<NCHQ>(t);
                    const uint4 rq = pf.q[kk], rk = pf.k[kk];
                    f16x8 hq, hk;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t wq = (&rq.x)[e], wk = (&rk.x)[e];
                        hq[2 * e] = (_Float16)bf16lo(wq);
                        hq[2 * e + 1] = (_Float16)bf16hi(wq);
                        hk[2 * e] = (_Float16)bf16lo(wk);
                        hk[2 * e + 1] = (_Float16)bf16hi(wk);
                    }
                    *reinterpret_cast<f16x8*>(B.q + t * LQ + 8 * ch) = hq;
                    *reinterpret_cast<f16x8*>(B.k + t * LQ + 8 * ch) = hk;
                } else {
                    const int c = cb * CB;
                    *reinterpret_cast<uint4*>(B.q + t * LQ + c) = pf.q[kk];
                    *reinterpret_cast<uint4*>(B.k + t * LQ + c) = pf.k[kk];
                    const uint4 rk = pf.k[kk];
#pragma unroll
                    for (int e = 0; e < 4; ++e) B.kt[(c + e) * LKT + t] = __uint_as_float((&rk.x)[e]);
                }
            }
        }
        if (pw == 1) {
#pragma unroll
            for (int kk = 0; kk < Gm::VUL; ++kk) {
                const int u = lane + kWave * kk;
                if (u < Gm::NVU) {
                    const int t = u / (RB / CB), rb = u % (RB / CB);
                    if constexpr (F16) {
                        *reinterpret_cast<uint4*>(B.vb + t * LV + rb * CB) = pf.v[kk];
                    } else {
                        const uint4 rv = pf.v[kk];
#pragma unroll
                        for (int e = 0; e < 4; ++e) B.vn[(rb * CB + e) * LV + t] = -__uint_as_float((&rv.x)[e]);
                    }
                }
            }
        }
    }

    // Producer wave 0: gate scans and decay-matrix helpers.
    __device__ static void gates(const Prefetch& pf, S& sm, Buf& B, int n, int lane) {
        const int l = lane;
        const float th = pf.th, et = pf.et, a = 1.f - pf.al;
        if (l < NP) { sm.ga[l] = a; sm.ge[l] = et; }
        // Inclusive prefix of T_l within 16-lane rows: Psi_l = T_l ... T_{16*(l/16)}.
        float X = a, Y = et, W = et;
        tri_step<kRowShr1>(X, Y, W);
        tri_step<kRowShr2>(X, Y, W);
        tri_step<kRowShr4>(X, Y, W);
        tri_step<kRowShr8>(X, Y, W);
        const float px = X, py = Y, pwv = W;
        // Extend to the whole wave: T_l ... T_0 = [[A_l, c_l], [0, E_l]].
        tri_step<kRowBcast15, 0xa>(X, Y, W);
        tri_step<kRowBcast31, 0xc>(X, Y, W);
        if (l < NP) { B.av[l] = X; B.cv[l] = Y; }
        if (l == n - 1) { B.scal[0] = X; B.scal[1] = Y; B.scal[2] = W; }
        // Maps from the end of block q to row l, for every block q below l's block.
        float BX[NT], BY[NT], BW[NT];
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            BX[q] = readlane(px, 16 * q + 15);
            BY[q] = readlane(py, 16 * q + 15);
            BW[q] = readlane(pwv, 16 * q + 15);
        }
        if (l < NP) {
            const int pb = l >> 4;
            float cx = px, cy = py, cw = pwv;
#pragma unroll
            for (int q = NT - 2; q >= 0; --q) {
                if (q < pb) {
                    float* dst = sm.phi + (q * NP + l) * 3;
                    dst[0] = cx; dst[1] = cy; dst[2] = cw;
                    const float ny = cx * BY[q] + cy * BW[q];
                    cx *= BX[q];
                    cw *= BW[q];
                    cy = ny;
                }
            }
        }
        // Diagonal 16x16 blocks: lane = (block, column j), rows run in order.
        const int qb = l >> 4, jj = l & 15;
        if (qb < NT) {
            float pp = 0.f, gg = 0.f;
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int i = 16 * qb + s;
                const float ai = sm.ga[i], ei = sm.ge[i];
                if (s == jj) { pp = 1.f; gg = 1.f; }
                else if (s > jj) { pp = ei * pp; gg = ai * gg + pp; }
                sm.gamd[(qb * 16 + s) * 16 + jj] = th * gg;
                sm.gampd[(qb * 16 + s) * 16 + jj] = th * pp;
            }
            sm.gend[l] = th * gg;
            sm.pend[l] = th * pp;
        }
    }

    // Producers: P tiles and the chunk-end weights.  Tile (pb, qb) holds rows
    // i = tmap(pb, .) and columns j = tmap(qb, .); it is nonzero only when the
    // k-group of pb is not before that of qb.  Producer pw takes the row tiles
    // pb = pw, pw + 2, ...
    __device__ static void ptiles(S& sm, Buf& B, int n, int pw, int lr, int lg) {
        const int ilast = n - 1;
        for (int pb = pw; pb < NT; pb += kProducers) {
            const int i = O::tmap(pb, lr);
            F qf[NKC];
#pragma unroll
            for (int s = 0; s < NKC; ++s) qf[s] = frag_q(B.q, i, s, lg);
            const int bi = i >> 4;
            for (int qb = 0; qb < NT; ++qb) {
                const int jb = O::tmap(qb, 4 * lg);   // j = jb + e, e = 0..3, one 16-block
                if (qb / TPB > pb / TPB) {
                    // Columns never read for these rows; only the chunk-end row's weights.
                    if (i == ilast) {
                        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                        put_w(B.wm, jb, zero);
                        put_w(B.ws, jb, zero);
                    }
                    continue;
                }
                const int kr = O::tmap(qb, lr);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < NKC; ++s) acc = O::mma(acc, frag_q(B.k, kr, s, lg), qf[s]);
                // acc[e] = q_i . k_{jb+e}
                const int bj = jb >> 4;
                f32x4 L, LPe;
                if (bi == bj) {
                    L = *reinterpret_cast<const f32x4*>(sm.gamd + (bi * 16 + (i & 15)) * 16 + (jb & 15));
                    LPe = *reinterpret_cast<const f32x4*>(sm.gampd + (bi * 16 + (i & 15)) * 16 + (jb & 15));
                } else if (bi > bj) {
                    const float* ph = sm.phi + (bj * NP + i) * 3;
                    const f32x4 gv = *reinterpret_cast<const f32x4*>(sm.gend + jb);
                    const f32x4 pv = *reinterpret_cast<const f32x4*>(sm.pend + jb);
                    L = ph[0] * gv + ph[1] * pv;
                    LPe = ph[2] * pv;
                } else {
                    L = f32x4{0.f, 0.f, 0.f, 0.f};
                    LPe = L;
                }
                put_p(B.p, i, jb, -(acc * L));
                if (i == ilast) { put_w(B.wm, jb, -L); put_w(B.ws, jb, -LPe); }
            }
        }
    }

    // ---- state waves ------------------------------------------------------
    // -V for accumulator tile tt: lane (lr, lg) gets -v[tmap(tt, 4lg + e)][row lr of the wave].
    __device__ static f32x4 neg_v(const Buf& B, int tt, int w, int lr, int lg) {
        if constexpr (F16) {
            const int t = O::tmap(tt, 4 * lg + (lr >> 2));
            const i16x4 r = ds_read_tr16(B.vb + t * LV + 16 * w + 4 * (lr & 3));
            const u32x2 u = __builtin_bit_cast(u32x2, r);
            return f32x4{-bf16lo(u[0]), -bf16hi(u[0]), -bf16lo(u[1]), -bf16hi(u[1])};
        } else {
            return *reinterpret_cast<const f32x4*>(B.vn + (16 * w + lr) * LV + 16 * tt + 4 * lg);
        }
    }
    // A operand of the state update for column tile ct, token k-group s:
    // lane (m = lr, lg) holds k[tokens of the k-group's slots][column tmap(ct, lr)].
    __device__ static F kt_frag(const Buf& B, int ct, int s, int lr, int lg) {
        if constexpr (F16) {
            const int col = 32 * (ct >> 1) + 8 * (lr & 3) + 4 * (ct & 1);
            const int ch = col >> 3;
            const int t0 = 32 * s + 8 * lg + (lr >> 2);
            const int t1 = t0 + 4;
            const i16x4 lo = ds_read_tr16(B.k + t0 * LQ + 8 * (ch ^ swz<NCHQ>(t0)) + (col & 4));
            const i16x4 hi = ds_read_tr16(B.k + t1 * LQ + 8 * (ch ^ swz<NCHQ>(t1)) + (col & 4));
            F f;
            const f16x4 l4 = __builtin_bit_cast(f16x4, lo), h4 = __builtin_bit_cast(f16x4, hi);
            f[0] = l4[0]; f[1] = l4[1]; f[2] = l4[2]; f[3] = l4[3];
            f[4] = h4[0]; f[5] = h4[1]; f[6] = h4[2]; f[7] = h4[3];
            return f;
        } else {
            return *reinterpret_cast<const f32x4*>(B.kt + (16 * ct + lr) * LKT + 16 * s + 4 * lg);
        }
    }

    // Phase 1: residuals E and the reads z; returns E as MFMA fragments.
    __device__ static void phase1(const f32x4* Macc, const f32x4* Sacc, const Buf& B, F* EB, float* z,
                                  size_t zrow0, int n, int w, int lr, int lg) {
        F MB[NKC], SB[NKC];
#pragma unroll
        for (int s = 0; s < NKC; ++s) {
            MB[s] = O::template from_acc<NC>(Macc, s);
            SB[s] = O::template from_acc<NC>(Sacc, s);
        }
        f32x4 E[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            E[tt] = neg_v(B, tt, w, lr, lg);
            const int t = O::tmap(tt, lr);
#pragma unroll
            for (int s = 0; s < NKC; ++s) E[tt] = O::mma(E[tt], frag_q(B.k, t, s, lg), MB[s]);
        }
#pragma unroll
        for (int s = 0; s < NKT; ++s) EB[s] = O::template from_acc<NT>(E, s);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const int t = O::tmap(tt, lr);
            f32x4 za = {0.f, 0.f, 0.f, 0.f}, zc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NKC; ++s) {
                const F bq = frag_q(B.q, t, s, lg);
                za = O::mma(za, MB[s], bq);
                zc = O::mma(zc, SB[s], bq);
            }
            f32x4 zt = B.av[t] * za + B.cv[t] * zc;
#pragma unroll
            for (int s = 0; s < NKT; ++s)
                if (s <= tt / TPB) zt = O::mma(zt, EB[s], frag_p(B.p, t, s, lg));
            if (t < n) *reinterpret_cast<f32x4*>(z + zrow0 + static_cast<size_t>(t) * D) = zt;
        }
    }

    // Phase 2: state update from the residual fragments.
    __device__ static void phase2(f32x4* Macc, f32x4* Sacc, const Buf& B, const F* EB, int lr, int lg) {
        F WMB[NKT], WSB[NKT];
#pragma unroll
        for (int s = 0; s < NKT; ++s) {
            WMB[s] = EB[s] * frag_w(B.wm, s, lg);
            WSB[s] = EB[s] * frag_w(B.ws, s, lg);
        }
        const float An = B.scal[0], Cn = B.scal[1], En = B.scal[2];
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
            Macc[ct] = An * Macc[ct] + Cn * Sacc[ct];
            Sacc[ct] = En * Sacc[ct];
#pragma unroll
            for (int s = 0; s < NKT; ++s) {
                const F a = kt_frag(B, ct, s, lr, lg);
                Macc[ct] = O::mma(Macc[ct], a, WMB[s]);
                Sacc[ct] = O::mma(Sacc[ct], a, WSB[s]);
            }
        }
    }
};

template <typename T, int D, int NS, int NP>
__global__ __launch_bounds__(kWave * (NS + kProducers)) void linear_memory_fwd(const Params p) {
    using Gm = Geo<T, D, NS, NP>;
    using K = Kernel<T, D, NS, NP>;
    using O = Op<T>;
    using G = typename Gm::G;
    using F = typename O::frag;
    constexpr int NBUF = Gm::NBUF;
    constexpr int NC = Gm::NC;
    constexpr int RB = Gm::RB;

    __shared__ __attribute__((aligned(16))) typename K::S sm;

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
    const int bh = lin / Gm::NRB;
    const int rb = lin % Gm::NRB;
    const int seqlen = p.T;
    const int b = p.b;
    const int row_wg = rb * RB;
    const int nch = (seqlen + b - 1) / b;
    const size_t seq_tok = static_cast<size_t>(bh) * seqlen;
    auto chunk_n = [&](int c) { return min(b, seqlen - c * b); };

    // Zero all staging memory once: padded rows and columns stay 0.
    {
        uint32_t* words = reinterpret_cast<uint32_t*>(&sm);
        for (int i = tid; i < static_cast<int>(sizeof(sm) / 4); i += kWave * Gm::NWAVE) words[i] = 0u;
    }
    __syncthreads();

    if (w < NS) {
        // ===================== state wave =====================
        const int row_w = row_wg + 16 * w;
        // Tile ct, lane (lr, lg): M[row_w + lr][tmap(ct, 4lg + e)], e = 0..3.
        f32x4 Macc[NC], Sacc[NC];
        const size_t state_off = static_cast<size_t>(bh) * D * D + static_cast<size_t>(row_w + lr) * D;
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
            const int col = O::tmap(ct, 4 * lg);
            const bool ok = col < D;
            Macc[ct] = (p.M0 && ok) ? *reinterpret_cast<const f32x4*>(p.M0 + state_off + col) : f32x4{0.f, 0.f, 0.f, 0.f};
            Sacc[ct] = (p.S0 && ok) ? *reinterpret_cast<const f32x4*>(p.S0 + state_off + col) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        F EB[Gm::NKT];
        if constexpr (NBUF == 2) {
            __syncthreads();   // chunk 0 staged
            __syncthreads();   // chunk 0 P tiles
            for (int c = 0; c < nch; ++c) {
                const int bf = c & 1;
                const size_t zrow0 = (seq_tok + static_cast<size_t>(c) * b) * D + row_w + 4 * lg;
                K::phase1(Macc, Sacc, sm.buf[bf], EB, p.z, zrow0, chunk_n(c), w, lr, lg);
                __syncthreads();
                K::phase2(Macc, Sacc, sm.buf[bf], EB, lr, lg);
                __syncthreads();
            }
        } else {
            for (int c = 0; c < nch; ++c) {
                __syncthreads();   // chunk c staged
                __syncthreads();   // chunk c P tiles
                const size_t zrow0 = (seq_tok + static_cast<size_t>(c) * b) * D + row_w + 4 * lg;
                K::phase1(Macc, Sacc, sm.buf[0], EB, p.z, zrow0, chunk_n(c), w, lr, lg);
                K::phase2(Macc, Sacc, sm.buf[0], EB, lr, lg);
                __syncthreads();   // chunk c consumed
            }
        }
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
            const int col = O::tmap(ct, 4 * lg);
            if (col < D) {
                if (p.MT) *reinterpret_cast<f32x4*>(p.MT + state_off + col) = Macc[ct];
                if (p.ST) *reinterpret_cast<f32x4*>(p.ST + state_off + col) = Sacc[ct];
            }
        }
    } else {
        // ===================== producer wave =====================
        const int pw = w - NS;
        const int ptid = tid - NS * kWave;
        const G* __restrict__ gq = static_cast<const G*>(p.q);
        const G* __restrict__ gk = static_cast<const G*>(p.k);
        const G* __restrict__ gv = static_cast<const G*>(p.v);
        typename K::Prefetch pf;
        if constexpr (NBUF == 2) {
            if (nch > 0) {
                K::issue(pf, p, gq, gk, gv, seq_tok, row_wg, 0, ptid, pw, lane);
                K::stage(pf, sm.buf[0], ptid, pw, lane);
                if (pw == 0) K::gates(pf, sm, sm.buf[0], chunk_n(0), lane);
                if (nch > 1) K::issue(pf, p, gq, gk, gv, seq_tok, row_wg, 1, ptid, pw, lane);
            }
            __syncthreads();
            if (nch > 0) K::ptiles(sm, sm.buf[0], chunk_n(0), pw, lr, lg);
            __syncthreads();
            for (int c = 0; c < nch; ++c) {
                const int nb = (c & 1) ^ 1;
                if (c + 1 < nch) {
                    K::stage(pf, sm.buf[nb], ptid, pw, lane);
                    if (pw == 0) K::gates(pf, sm, sm.buf[nb], chunk_n(c + 1), lane);
                    if (c + 2 < nch) K::issue(pf, p, gq, gk, gv, seq_tok, row_wg, c + 2, ptid, pw, lane);
                }
                __syncthreads();
                if (c + 1 < nch) K::ptiles(sm, sm.buf[nb], chunk_n(c + 1), pw, lr, lg);
                __syncthreads();
            }
        } else {
            for (int c = 0; c < nch; ++c) {
                K::issue(pf, p, gq, gk, gv, seq_tok, row_wg, c, ptid, pw, lane);
                K::stage(pf, sm.buf[0], ptid, pw, lane);
                if (pw == 0) K::gates(pf, sm, sm.buf[0], chunk_n(c), lane);
                __syncthreads();
                K::ptiles(sm, sm.buf[0], chunk_n(c), pw, lr, lg);
                __syncthreads();
                __syncthreads();
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Host side: validation, instance selection, launch.
// ---------------------------------------------------------------------------
template <typename T, int D, int NS, int NP>
hipError_t launch(const Params& p, hipStream_t stream) {
    using Gm = Geo<T, D, NS, NP>;
    const long long nwg = static_cast<long long>(p.BH) * Gm::NRB;
    hipLaunchKernelGGL((linear_memory_fwd<T, D, NS, NP>), dim3(static_cast<unsigned>(nwg)),
                       dim3(kWave * Gm::NWAVE), 0, stream, p);
    return hipGetLastError();
}

template <typename T, int D, int NS>
hipError_t launch_np(const Params& p, int np, hipStream_t stream) {
    if constexpr (Op<T>::KG == 32) {
        return np <= 32 ? launch<T, D, NS, 32>(p, stream) : launch<T, D, NS, 64>(p, stream);
    } else {
        if (np <= 16) return launch<T, D, NS, 16>(p, stream);
        if (np <= 32) return launch<T, D, NS, 32>(p, stream);
        return launch<T, D, NS, 64>(p, stream);
    }
}

template <typename T, int D>
hipError_t launch_ns(const Params& p, int np, hipStream_t stream) {
    if constexpr (D >= 32) {
        // Two state waves (32 rows) per workgroup when that still leaves >= 256 workgroups.
        const long long row_tiles = static_cast<long long>(p.BH) * (D / 16);
        if (row_tiles >= 512) return launch_np<T, D, 2>(p, np, stream);
    }
    return launch_np<T, D, 1>(p, np, stream);
}

template <typename T>
hipError_t dispatch(const Params& p, int d, hipStream_t stream) {
    const int np = round_up(p.b, 16);
    switch (d) {
        case 16: return launch_ns<T, 16>(p, np, stream);
        case 32: return launch_ns<T, 32>(p, np, stream);
        case 64: return launch_ns<T, 64>(p, np, stream);
        default: return launch_ns<T, 128>(p, np, stream);
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
