// Backward pass of the chunked TTT / Titans linear memory for gfx950 (MI355X),
// and its C ABI.
//
// The outer gradient of the memory is the chain rule run backward through the
// unrolled writes ("Continual Learning: From Attention to Neural Memory",
// section 4.5; "5.1.1 · TTT layers 与 fast weights", section 1.2, eqs. (15)-(16)).
// Chunk by chunk the forward is an affine map of the state, so the backward
// is its transpose, walked from the last chunk to the first ("论文速览 |
// Titans", section 4.7).
//
// One chunk, tokens i = 0..n-1, start state (M0, S0), gates as in the forward
// (a = 1 - alpha):
//   A_i = prod_{l<=i} a_l,  E_i = prod_{l<=i} eta_l,  c_i = a_i c_{i-1} + E_i,
//   gamma_ij (j <= i): gamma_jj = 1, gamma_ij = a_i gamma_{i-1,j} + p_ij,
//                      p_jj = 1,     p_ij = eta_i p_{i-1,j},
//   L_ij = theta_j gamma_ij,  w^M_j = L_{n-1,j},  w^S_j = theta_j p_{n-1,j},
//   E  = K M0^T - V                              (residuals, row j = e_j)
//   Z  = diag(A) Q M0^T + diag(c) Q S0^T - P E,  P = (Q K^T) .* L (lower, diagonal included)
//   M' = A_{n-1} M0 + c_{n-1} S0 - E^T diag(w^M) K
//   S' = E_{n-1} S0 - E^T diag(w^S) K.
// Given dZ, dM', dS' (the derivatives of the outer loss):
//   dE  = -P^T dZ - diag(w^M) K dM'^T - diag(w^S) K dS'^T,   dV = -dE
//   dM0 = A_{n-1} dM' + dZ^T diag(A) Q + dE^T K
//   dS0 = c_{n-1} dM' + E_{n-1} dS' + dZ^T diag(c) Q
//   D   = dZ E^T,   DL = D .* L
//   dQ  = diag(A) dZ M0 + diag(c) dZ S0 - DL K
//   dK  = -DL^T Q + dE M0 - diag(w^M) E dM' - diag(w^S) E dS'
// and the gates through the scalar cotangents
//   dA_i = q_i . (M0^T dz_i),  dc_i = q_i . (S0^T dz_i)  (plus <dM',M0>, <dM',S0> at i = n-1),
//   dE_{n-1} = <dS',S0>,  dL_ij = -(q_i . k_j) D_ij (plus -e_j^T dM' k_j on row n-1),
//   dw^S_j = -e_j^T dS' k_j,
// run backward through the products and the column recurrences of gamma
// (division-free, so gates equal to 0 are exact).
//
// The (dM, dS) carry needs only q, k, dz and the gates; everything else of a
// chunk needs the chunk's own start state and end cotangent.  Hence two
// kernels:
//   * carry: one workgroup per (sequence, block of 16*NS rows of the state),
//     reverse walk over the chunks with dM, dS in MFMA accumulators (rows of
//     the memory never meet, as in the forward); writes dV and the cotangent
//     leaving every chunk to a work buffer.  Producer waves stage the next
//     chunks and build P, one and two chunks ahead.
//   * grads: one workgroup per (sequence, chunk), fully parallel; reads the
//     chunk-start state saved by the forward and the cotangent from the work
//     buffer; computes dQ, dK and the gate gradients with the whole feature
//     dimension on chip.
//
// Precision: as the forward.  The float32 path uses float32 MFMA; the bf16
// path uses fp16 operands (bf16 inputs convert exactly in the fp16 normal
// range; states, cotangents and P are rounded to fp16 where they enter a
// product) with float32 accumulation, float32 carried cotangents and float32
// gate arithmetic.
//
// The backward is linear in the cotangents (dz, dM', dS').  On the bf16 path a
// first kernel takes the largest magnitude of each sequence's cotangents, and
// both kernels multiply every cotangent they round to fp16 by a power of two
// that brings that magnitude into [1, 2), then divide every gradient they
// write by it: exact in float32, and small cotangents (a mean-reduced loss
// gives 1e-6 .. 1e-9) stay in fp16's normal range instead of its subnormals.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "ttt_mem.h"
#include "gfx950.h"

namespace {

constexpr int kW = 64;
constexpr int kLdsMax = 160 * 1024;
// Partial maxima of the cotangents' magnitude per sequence.
constexpr int kScaleParts = 16;

// Power of two that brings the largest cotangent magnitude of sequence g into
// [1, 2): the maximum over its kScaleParts partial maxima.  1 when
// there are none (NULL), when all are zero, or when one is not finite.
__device__ __forceinline__ float cot_scale(const float* smax, int g) {
    if (!smax) return 1.f;
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < kScaleParts; ++i) m = fmaxf(m, smax[static_cast<size_t>(g) * kScaleParts + i]);
    if (!(m > 0.f) || !(m <= 3.0e38f)) return 1.f;
    const int e = min(max(ilogbf(m), -126), 126);
    return ldexpf(1.f, -e);
}

// Partial maxima of |dz|, |dM_T|, |dS_T| per sequence g (dense: sequence bh,
// tokens g*T .. g*T+T-1; packed documents: document g / H of head g % H, its
// tokens of row h): workgroup (g, part) covers every kScaleParts-th 256-unit
// stretch of the sequence's dz and, for part 0, its d x d state cotangents,
// and writes one value.
__global__ __launch_bounds__(256) void cot_absmax(const float* __restrict__ dz, const float* __restrict__ dMT,
                                                  const float* __restrict__ dST, float* __restrict__ out, int T,
                                                  int d, const int* __restrict__ cu, int H) {
    const int g = blockIdx.x / kScaleParts, part = blockIdx.x % kScaleParts;
    size_t tok0 = static_cast<size_t>(g) * T;
    int len = T;
    if (cu) {
        int t0;
        len = doc_len(cu, g / H, T, t0);
        tok0 = static_cast<size_t>(g % H) * T + t0;
    }
    const float4* z4 = reinterpret_cast<const float4*>(dz + tok0 * d);
    const size_t nz4 = static_cast<size_t>(len) * d / 4;
    auto amax4 = [](float m, const float4 v) {
        return fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    };
    float m = 0.f;
    for (size_t u = static_cast<size_t>(part) * 256 + threadIdx.x; u < nz4; u += static_cast<size_t>(kScaleParts) * 256)
        m = amax4(m, z4[u]);
    if (part == 0) {
        const size_t dd4 = static_cast<size_t>(d) * d / 4, base = static_cast<size_t>(g) * d * d;
        for (size_t e = threadIdx.x; e < dd4; e += 256) {
            if (dMT) m = amax4(m, reinterpret_cast<const float4*>(dMT + base)[e]);
            if (dST) m = amax4(m, reinterpret_cast<const float4*>(dST + base)[e]);
        }
    }
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    __shared__ float wm[4];
    if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
}

__host__ __device__ constexpr int bmax(int a, int b) { return a > b ? a : b; }
__host__ __device__ constexpr int bmin(int a, int b) { return a < b ? a : b; }

// Earlier LDS accesses of this wave have completed (same-wave hand-over of
// LDS data between lanes).
__device__ __forceinline__ void wave_lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Fragment loads for the MFMA operand traits Op<T> (k-groups of KG, KS slots
// per lane: lane (lr, lg) holds k-slots KS*lg .. KS*lg + KS - 1).
template <typename T>
struct Fr {
    using O = Op<T>;
    using F = typename O::frag;
    static constexpr int KG = O::KG;
    static constexpr int KS = KG / 4;

    // Row-major LDS tile X (LD elements per row): lane (lr, lg) gets
    // X[row][k0 + KS*lg + s], s < KS (one 16-byte read).
    __device__ static F rm(const T* X, int LD, int row, int k0, int lg) {
        return *reinterpret_cast<const F*>(X + row * LD + k0 + KS * lg);
    }
    // Transposed read: lane (lr, lg) gets X[k0 + KS*lg + s][c0 + lr].
    __device__ static F cm(const T* X, int LD, int k0, int c0, int lr, int lg) {
        if constexpr (O::kF16) {
            return tr(X, LD, k0 + 8 * lg + (lr >> 2), c0 + 4 * (lr & 3));
        } else {
            const T* p = X + (k0 + 4 * lg) * LD + c0 + lr;
            return F{p[0], p[LD], p[2 * LD], p[3 * LD]};
        }
    }
    // Transposed read whose rows stand for the tmap order of column tile ct:
    // lane (lr, lg) gets X[k0 + KS*lg + s][tmap(ct, lr)].
    __device__ static F cm_t(const T* X, int LD, int k0, int ct, int lr, int lg) {
        if constexpr (O::kF16) {
            return tr(X, LD, k0 + 8 * lg + (lr >> 2), 32 * (ct >> 1) + 8 * (lr & 3) + 4 * (ct & 1));
        } else {
            return cm(X, LD, k0, 16 * ct, lr, lg);
        }
    }
    // Two LDS transpose loads: within each 16-lane group, lane i receives
    // column (its reader's base + i % 4) of rows row0 + 0..3 and row0 + 4..7.
    __device__ static F tr(const T* X, int LD, int row0, int col) {
        const i16x4 lo = ds_read_tr16(X + row0 * LD + col);
        const i16x4 hi = ds_read_tr16(X + (row0 + 4) * LD + col);
        const f16x4 a = __builtin_bit_cast(f16x4, lo), b = __builtin_bit_cast(f16x4, hi);
        return F{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
    // KS float32 values -> fragment (fp16: round to nearest even).
    __device__ static F from_f32(const float* x) {
        if constexpr (O::kF16) {
            const f16x4 a = cvt4(f32x4{x[0], x[1], x[2], x[3]}), b = cvt4(f32x4{x[4], x[5], x[6], x[7]});
            return F{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        } else {
            return F{x[0], x[1], x[2], x[3]};
        }
    }
    // Fragment times KS per-slot float32 factors.
    __device__ static F scale(const F& f, const float* w) {
        F r;
#pragma unroll
        for (int s = 0; s < KS; ++s) r[s] = static_cast<T>(static_cast<float>(f[s]) * w[s]);
        return r;
    }
};

// One 16-byte unit of a global input row (8 bf16 or 4 float32) -> LDS as T
// (zeros when !ok).
template <typename T>
__device__ __forceinline__ void stage_unit(T* dst, const typename GlobalOf<T>::type* src, bool ok) {
    const uint4 u = ok ? *reinterpret_cast<const uint4*>(src) : uint4{0u, 0u, 0u, 0u};
    if constexpr (Op<T>::kF16) {
        const f16x4 a = cvt4(f32x4{bf16lo(u.x), bf16hi(u.x), bf16lo(u.y), bf16hi(u.y)});
        const f16x4 b = cvt4(f32x4{bf16lo(u.z), bf16hi(u.z), bf16lo(u.w), bf16hi(u.w)});
        *reinterpret_cast<f16x8*>(dst) = f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    } else {
        *reinterpret_cast<uint4*>(dst) = u;
    }
}

// One 16-byte unit already in registers -> LDS as T.
template <typename T>
__device__ __forceinline__ void put_unit(T* dst, uint4 u) {
    if constexpr (Op<T>::kF16) {
        const f16x4 a = cvt4(f32x4{bf16lo(u.x), bf16hi(u.x), bf16lo(u.y), bf16hi(u.y)});
        const f16x4 b = cvt4(f32x4{bf16lo(u.z), bf16hi(u.z), bf16lo(u.w), bf16hi(u.w)});
        *reinterpret_cast<f16x8*>(dst) = f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    } else {
        *reinterpret_cast<uint4*>(dst) = u;
    }
}

// Four input elements (bf16 or float32) of a global row as float32.
template <typename T>
__device__ __forceinline__ f32x4 gload4(const typename GlobalOf<T>::type* src) {
    if constexpr (Op<T>::kF16) {
        const uint2 u = *reinterpret_cast<const uint2*>(src);
        return f32x4{bf16lo(u.x), bf16hi(u.x), bf16lo(u.y), bf16hi(u.y)};
    } else {
        return *reinterpret_cast<const f32x4*>(src);
    }
}

// 1.0 in lane i, 0.0 elsewhere: one select on a lane mask in scalar registers.
__device__ __forceinline__ float unit_at(int i) {
    float d;
    asm("v_cndmask_b32_e64 %0, 0, 1.0, %1" : "=v"(d) : "s"(1ull << i));
    return d;
}

// Column j = lane of the decay tables of a chunk: p_ij = eta_i p_{i-1,j} and
// gamma_ij = a_i gamma_{i-1,j} + p_ij below the diagonal, both 1 on it and 0
// above.  The two updates started from zero keep the zeros, and a unit added
// at i = j starts the column (no branches).  a and eta are read per four rows
// as LDS broadcasts; put(i, gamma_ij) stores row i; the values at row n - 1
// are returned in g_last, p_last (a full chunk, n = NP, needs no per-row
// selects for them).
template <int NP, bool FULL, typename Put>
__device__ __forceinline__ void gamma_columns_impl(const float* av, const float* et, int n, Put& put,
                                                   float& g_last, float& p_last) {
    float g = 0.f, pp = 0.f;
    g_last = 0.f;
    p_last = 0.f;
#pragma unroll
    for (int i0 = 0; i0 < NP; i0 += 4) {
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(av + i0);
        const f32x4 e4 = *reinterpret_cast<const f32x4*>(et + i0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = i0 + e;
            pp = __builtin_fmaf(e4[e], pp, unit_at(i));
            g = __builtin_fmaf(a4[e], g, pp);
            put(i, g);
            if constexpr (!FULL) {
                g_last = i == n - 1 ? g : g_last;
                p_last = i == n - 1 ? pp : p_last;
            }
        }
    }
    if constexpr (FULL) {
        g_last = g;
        p_last = pp;
    }
}
template <int NP, typename Put>
__device__ __forceinline__ void gamma_columns(const float* av, const float* et, int n, Put put, float& g_last,
                                              float& p_last) {
    if (n == NP) gamma_columns_impl<NP, true>(av, et, n, put, g_last, p_last);
    else gamma_columns_impl<NP, false>(av, et, n, put, g_last, p_last);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 1; m < kW; m <<= 1) x += __shfl_xor(x, m, kW);
    return x;
}

// Inclusive scan across the wave (lane order) of the maps [[X, Y], [0, W]]:
// lane l ends with T_l ... T_0 (T_0 applied first).
__device__ __forceinline__ void map_scan(float& X, float& Y, float& W) {
    tri_step<kRowShr1>(X, Y, W);
    tri_step<kRowShr2>(X, Y, W);
    tri_step<kRowShr4>(X, Y, W);
    tri_step<kRowShr8>(X, Y, W);
    tri_step<kRowBcast15, 0xa>(X, Y, W);
    tri_step<kRowBcast31, 0xc>(X, Y, W);
}

// Chunk gates of one wave (lane = token l of a chunk padded with theta = 0,
// eta = a = 1): T_l = [[a_l, eta_l], [0, eta_l]] composes to
// T_l ... T_0 = [[A_l, c_l], [0, E_l]].
__device__ __forceinline__ void gate_prefix(float my_a, float my_et, float& A, float& E, float& c) {
    float X = my_a, Y = my_et, W = my_et;
    map_scan(X, Y, W);
    A = X;
    c = Y;
    E = W;
}

// Reverse linear recurrence r_i = u_i + f_i r_{i+1} over i = NP-1 .. 0
// (lane i holds u_i and f_i; f_i multiplies the later value): the lanes are
// reversed, scanned as maps [[f, u], [0, 1]] and reversed back.
template <int NP>
__device__ __forceinline__ float reverse_recurrence(float u, float f, int lane) {
    const int src = NP - 1 - lane;
    const int from = src >= 0 ? src : lane;
    float X = __shfl(f, from, kW), Y = __shfl(u, from, kW), W = 1.f;
    if (src < 0) {
        X = 1.f;
        Y = 0.f;
    }
    map_scan(X, Y, W);
    return __shfl(Y, src >= 0 ? src : lane, kW);
}

// ===========================================================================
// Carry kernel: reverse walk over the chunks, (dM, dS) per row block.
// ===========================================================================
struct CarryParams {
    const void* q;
    const void* k;
    const float* dz;
    const float* theta;
    const float* eta;
    const float* alpha;
    const float* dMT;   // NULL: zero
    const float* dST;
    void* work;         // [BH][nch][dM | dS][D][D] (as the checkpoints): cotangent leaving each chunk
    float* dv;          // [BH][T][D]
    float* dM0;         // NULL: not written
    float* dS0;
    int BH;
    int T;
    int b;
    int nch;
    int chunk_gates;    // gates [BH][nch] shared by the tokens of a chunk
    // Packed documents (NULL: dense): sequence bh is document bh / H of head
    // bh % H at tokens cu[s] .. cu[s+1]-1 of the head's [T] rows; the work
    // buffer is [H][tcmax][dM | dS][D][D] with the document's chunks from slot
    // h * tcmax + (the chunks of documents 0..s-1).
    const int* cu;
    int H;
    int tcmax;
    // Partial maxima of the cotangents per sequence bh; NULL: no scaling.
    const float* smax;
    // Packed documents above kLptDocs: their longest-first order (NULL: packing order).
    const int* perm;
};

template <typename T, int D, int NS, int NP>
struct CarryGeo {
    using O = Op<T>;
    static constexpr int KG = O::KG;
    static constexpr int DS = bmax(D, KG);      // stored feature width (fp16: >= one k-group)
    static constexpr int RB = 16 * NS;          // rows of the state per workgroup
    static constexpr int NRB = D / RB;
    static constexpr int NT = NP / 16;
    static constexpr int NKD = DS / KG;
    static constexpr int NKT = NP / KG;
    static constexpr int NCT = DS / 16;         // 16-column tiles of the state
    static constexpr int PAD = 16 / (int)sizeof(T);
    static constexpr int LQ = DS + PAD;
    static constexpr int LZ = RB + PAD;
    static constexpr int LP = NP + PAD;
    static constexpr int LF = NP + 4;
    static constexpr int QSLOT = (2 * NP * LQ + NP * LZ) * (int)sizeof(T) + 3 * NP * 4;
    static constexpr int PSLOT = NP * LP * (int)sizeof(T) + 4 * NP * 4 + 16;
    static constexpr int LS = NP * LF * 4;
    // Packed documents on persistent workgroups: a table of up to KMAX units
    // (plus their cotangent scales) per workgroup.
    static constexpr int KMAX = 128;
    static constexpr int UNIT_BYTES = KMAX * (16 + 4) + 16;
    // Three staging slots (state waves, P builder and loader each on their
    // own chunk, one barrier per chunk) when they fit; else one slot and a
    // serial schedule.
    static constexpr int NQ = (3 * QSLOT + 2 * PSLOT + LS + UNIT_BYTES + 1024 <= kLdsMax) ? 3 : 1;
    // The persistent walk (three slots): documents it ranks in LDS, four ints
    // each plus KMAX in the last staging slot, borrowed before the walk.
    static constexpr bool PERSIST = NQ == 3;
    static constexpr int NMAX_DOCS = bmin(2048, (QSLOT / 4 - KMAX) / 4);
    static constexpr int NPR = NQ == 3 ? 2 : 1;
    static constexpr int NWAVE = NS + 3;            // state waves, two loaders, one builder
    static_assert(NQ * QSLOT + NPR * PSLOT + LS + UNIT_BYTES + 1024 <= kLdsMax, "LDS budget");
    static_assert(D % RB == 0 && NP % KG == 0, "tiling");
};

template <typename T, int D, int NS, int NP>
struct CarrySmem {
    using Gm = CarryGeo<T, D, NS, NP>;
    struct QSlot {
        alignas(16) T q[NP * Gm::LQ];
        alignas(16) T k[NP * Gm::LQ];
        alignas(16) T dz[NP * Gm::LZ];     // dz columns of the workgroup's rows
        alignas(16) float th[NP];
        alignas(16) float et[NP];
        alignas(16) float av[NP];
    };
    struct PSlot {
        alignas(16) T pt[NP * Gm::LP];     // P^T: row t holds P[i][t] over i
        alignas(16) float A[NP];
        alignas(16) float c[NP];
        alignas(16) float wm[NP];
        alignas(16) float ws[NP];
        alignas(16) float scal[4];         // A_{n-1}, c_{n-1}, E_{n-1}
    };
    QSlot qs[Gm::NQ];
    PSlot ps[Gm::NPR];
    alignas(16) float ls[NP * Gm::LF];     // L_ij = theta_j gamma_ij (builder only)
    // Persistent walk over packed documents: the workgroup's units, their
    // cotangent scales, and build_walk_table's counts (in this order).
    WalkUnit units[Gm::KMAX];
    float usc[Gm::KMAX];
    int nitems, nunits, nempty;
};

template <typename T, int D, int NS, int NP>
struct Carry {
    using Gm = CarryGeo<T, D, NS, NP>;
    using O = Op<T>;
    using R = Fr<T>;
    using F = typename O::frag;
    using G = typename GlobalOf<T>::type;
    using Sm = CarrySmem<T, D, NS, NP>;
    static constexpr int KG = Gm::KG, KS = R::KS, LQ = Gm::LQ, LZ = Gm::LZ, LP = Gm::LP, LF = Gm::LF;

    // Loader: a chunk's q, k rows (all features), dz columns row0..row0+RB-1
    // and gates are fetched into registers one step ahead (issue) and written
    // to a staging slot the next step (commit), so HBM latency overlaps a
    // whole chunk step.  Issue only requests (clamped addresses, always in
    // bounds); the ragged tail is zeroed at commit, when the data is there.
    static constexpr int CB = 16 / (int)sizeof(G);   // elements per 16-byte unit
    static constexpr int UR = Gm::DS / CB;           // q / k units per row
    static constexpr int NLW = 2;                    // loader waves
    static constexpr int NQU = (NP * UR + NLW * kW - 1) / (NLW * kW);
    static constexpr int UZ = Gm::RB / 4;            // dz units (4 floats) per row
    static constexpr int NZU = (NP * UZ + NLW * kW - 1) / (NLW * kW);
    struct Regs {
        uint4 q[NQU], k[NQU];
        f32x4 z[NZU];
        float th, et, al;
    };
    // Loader wave lw (0 or 1) handles units lw*kW + lane + i*NLW*kW; wave 0 also the gates.
    __device__ __forceinline__ static void issue(const CarryParams& p, Regs& r, size_t tok0, int n, int row0, int lane, int lw,
                                 size_t g0, int gs) {
        const G* q = static_cast<const G*>(p.q);
        const G* k = static_cast<const G*>(p.k);
#pragma unroll
        for (int i = 0; i < NQU; ++i) {
            const int u = lane + (lw + i * NLW) * kW;
            const int t = u / UR, col = (u % UR) * CB;
            const bool ok = u < NP * UR && t < n && col < D;
            const size_t g = ok ? (tok0 + t) * D + col : 0;   // clamped: every load is in bounds
            r.q[i] = *reinterpret_cast<const uint4*>(q + g);
            r.k[i] = *reinterpret_cast<const uint4*>(k + g);
        }
#pragma unroll
        for (int i = 0; i < NZU; ++i) {
            const int u = lane + (lw + i * NLW) * kW;
            const int t = u / UZ, col = (u % UZ) * 4;
            const bool ok = u < NP * UZ && t < n;
            r.z[i] = *reinterpret_cast<const f32x4*>(p.dz + (ok ? (tok0 + t) * D + row0 + col : 0));
        }
        const size_t gi = lane < n ? g0 + static_cast<size_t>(lane) * gs : 0;
        r.th = p.theta[gi];
        r.et = p.eta[gi];
        r.al = p.alpha[gi];
    }
    // n: the chunk's token count (positions at or past it are written as zero
    // and as the identity gates).
    __device__ __forceinline__ static void commit(const Regs& r, typename Sm::QSlot& s, int n, int lane, int lw, float sc) {
#pragma unroll
        for (int i = 0; i < NQU; ++i) {
            const int u = lane + (lw + i * NLW) * kW;
            if (u < NP * UR) {
                const int t = u / UR, col = (u % UR) * CB;
                const bool ok = t < n && col < D;
                put_unit<T>(s.q + t * LQ + col, ok ? r.q[i] : uint4{0u, 0u, 0u, 0u});
                put_unit<T>(s.k + t * LQ + col, ok ? r.k[i] : uint4{0u, 0u, 0u, 0u});
            }
        }
#pragma unroll
        for (int i = 0; i < NZU; ++i) {
            const int u = lane + (lw + i * NLW) * kW;
            if (u < NP * UZ) {
                const int t = u / UZ, col = (u % UZ) * 4;
                st4<T>(s.dz + t * LZ + col, t < n ? sc * r.z[i] : f32x4{0.f, 0.f, 0.f, 0.f});
            }
        }
        if (lw == 0 && lane < NP) {
            const bool ok = lane < n;
            s.th[lane] = ok ? r.th : 0.f;
            s.et[lane] = ok ? r.et : 1.f;
            s.av[lane] = ok ? 1.f - r.al : 1.f;
        }
    }

    // Serial schedule (one slot): load and stage directly.
    __device__ __forceinline__ static void load_direct(const CarryParams& p, typename Sm::QSlot& s, size_t tok0, int n, int row0,
                                       int lane, size_t g0, int gs, float sc) {
        const G* q = static_cast<const G*>(p.q);
        const G* k = static_cast<const G*>(p.k);
        for (int u = lane; u < NP * UR; u += kW) {
            const int t = u / UR, col = (u % UR) * CB;
            const bool ok = t < n && col < D;
            const size_t g = (tok0 + t) * D + col;
            stage_unit<T>(s.q + t * LQ + col, q + (ok ? g : 0), ok);
            stage_unit<T>(s.k + t * LQ + col, k + (ok ? g : 0), ok);
        }
        for (int u = lane; u < NP * UZ; u += kW) {
            const int t = u / UZ, col = (u % UZ) * 4;
            const f32x4 v = t < n ? *reinterpret_cast<const f32x4*>(p.dz + (tok0 + t) * D + row0 + col)
                                  : f32x4{0.f, 0.f, 0.f, 0.f};
            st4<T>(s.dz + t * LZ + col, sc * v);
        }
        for (int l = lane; l < NP; l += kW) {
            const bool ok = l < n;
            const size_t gi = g0 + static_cast<size_t>(l) * gs;
            s.th[l] = ok ? p.theta[gi] : 0.f;
            s.et[l] = ok ? p.eta[gi] : 1.f;
            s.av[l] = ok ? 1.f - p.alpha[gi] : 1.f;
        }
    }

    // Gates, decay matrix and P^T of one staged chunk.
    __device__ __forceinline__ static void build(const typename Sm::QSlot& s, typename Sm::PSlot& ps, float* ls, int n, int lane) {
        const int lr = lane & 15, lg = lane >> 4;
        const float my_th = s.th[lane % NP], my_et = s.et[lane % NP], my_a = s.av[lane % NP];
        float A, E, c;
        gate_prefix(my_a, my_et, A, E, c);
        if (lane < NP) {
            ps.A[lane] = A;
            ps.c[lane] = c;
        }
        const float An = readlane(A, n - 1), cn = readlane(c, n - 1), En = readlane(E, n - 1);
        if (lane == 0) {
            ps.scal[0] = An;
            ps.scal[1] = cn;
            ps.scal[2] = En;
        }
        // Column j = lane of gamma and p.
        float g_last, p_last;
        gamma_columns<NP>(s.av, s.et, n, [&](int i, float g) {
            if (lane < NP) ls[i * LF + lane] = my_th * g;
        }, g_last, p_last);
        if (lane < NP) {
            ps.wm[lane] = my_th * g_last;
            ps.ws[lane] = my_th * p_last;
        }
        wave_lds_fence();
        // P^T tiles: G[i][t] = q_i . k_t on the lower tiles, times L_it (L is
        // zero above the diagonal); upper tiles zero.  The q fragments of a
        // row tile are read once; each tile's k fragments and L values are
        // read together ahead of its products.
#pragma unroll
        for (int it = 0; it < Gm::NT; ++it) {
#pragma unroll
            for (int tt = it + 1; tt < Gm::NT; ++tt)
                st4<T>(ps.pt + (16 * tt + lr) * LP + 16 * it + 4 * lg, f32x4{0.f, 0.f, 0.f, 0.f});
        }
#pragma unroll
        for (int it = 0; it < Gm::NT; ++it) {
            F qf[Gm::NKD];
#pragma unroll
            for (int kk = 0; kk < Gm::NKD; ++kk) qf[kk] = R::rm(s.q, LQ, 16 * it + lr, kk * KG, lg);
#pragma unroll
            for (int tt = 0; tt <= it; ++tt) {
                const int t = 16 * tt + lr;
                F kf[Gm::NKD];
                float lv[4];
#pragma unroll
                for (int kk = 0; kk < Gm::NKD; ++kk) kf[kk] = R::rm(s.k, LQ, t, kk * KG, lg);
#pragma unroll
                for (int e = 0; e < 4; ++e) lv[e] = ls[(16 * it + 4 * lg + e) * LF + t];
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < Gm::NKD; ++kk) acc = O::mma(acc, qf[kk], kf[kk]);
                f32x4 pv;
#pragma unroll
                for (int e = 0; e < 4; ++e) pv[e] = t <= 16 * it + 4 * lg + e ? acc[e] * lv[e] : 0.f;
                st4<T>(ps.pt + t * LP + 16 * it + 4 * lg, pv);
            }
        }
    }
};

// One chunk step of a carry walk's state wave (rows r0 .. r0+15 of the
// cotangents dM, dS, as accumulator tiles of dM^T): store the cotangent
// leaving the chunk into work slot `slot`, write dv of the chunk's n tokens
// from token tok0, and carry dM, dS back to the chunk's start.  s and ps hold
// the chunk's staged inputs and gate quantities; isc undoes the cotangent
// scaling on dv.
template <typename T, int D, int NS, int NP>
__device__ __forceinline__ void carry_state_step(const CarryParams& p,
                                                 const typename CarrySmem<T, D, NS, NP>::QSlot& s,
                                                 const typename CarrySmem<T, D, NS, NP>::PSlot& ps, f32x4* dM,
                                                 f32x4* dS, int n, size_t tok0, size_t slot, int r0, int r0l, int lr,
                                                 int lg, float isc) {
    using Gm = CarryGeo<T, D, NS, NP>;
    using O = Op<T>;
    using R = Fr<T>;
    using F = typename O::frag;
    constexpr int KG = Gm::KG, KS = R::KS, NT = Gm::NT, NKD = Gm::NKD, NKT = Gm::NKT, NCT = Gm::NCT;
    // Cotangent of the state leaving chunk c.
    {
        T* base = static_cast<T*>(p.work) + slot * (2 * D * D) + static_cast<size_t>(r0 + lr) * D;
#pragma unroll
        for (int jt = 0; jt < NCT; ++jt) {
            const int col = O::tmap(jt, 4 * lg);
            if (col < D) {
                st4<T>(base + col, dM[jt]);
                st4<T>(base + D * D + col, dS[jt]);
            }
        }
    }
    F MB[NKD], SB[NKD], ZC[NKT];
#pragma unroll
    for (int kk = 0; kk < NKD; ++kk) {
        MB[kk] = O::template from_acc<NCT>(dM, kk);
        SB[kk] = O::template from_acc<NCT>(dS, kk);
    }
#pragma unroll
    for (int kk = 0; kk < NKT; ++kk) ZC[kk] = R::cm(s.dz, Gm::LZ, kk * KG, r0l, lr, lg);
    // dE (tokens x own rows): -w^M K dM^T - w^S K dS^T - P^T dZ.
    f32x4 dE[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        const int trow = O::tmap(tt, lr);
        f32x4 x1 = {0.f, 0.f, 0.f, 0.f}, x2 = x1, x3 = x1;
#pragma unroll
        for (int kk = 0; kk < NKD; ++kk) {
            const F kf = R::rm(s.k, Gm::LQ, trow, kk * KG, lg);
            x1 = O::mma(x1, kf, MB[kk]);
            x2 = O::mma(x2, kf, SB[kk]);
        }
#pragma unroll
        for (int kk = 0; kk < NKT; ++kk) x3 = O::mma(x3, R::rm(ps.pt, Gm::LP, trow, kk * KG, lg), ZC[kk]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = O::tmap(tt, 4 * lg + e);
            dE[tt][e] = -(ps.wm[t] * x1[e] + ps.ws[t] * x2[e] + x3[e]);
            if (t < n) p.dv[(tok0 + t) * D + r0 + lr] = -isc * dE[tt][e];
        }
    }
    // Carry: dM <- A dM + Q^T diag(A) dZ + K^T dE, dS <- c dM + E dS + Q^T diag(c) dZ.
    F DE[NKT], ZA[NKT], ZK[NKT];
#pragma unroll
    for (int kk = 0; kk < NKT; ++kk) {
        DE[kk] = O::template from_acc<NT>(dE, kk);
        float av[KS], cv[KS];
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
            av[s2] = ps.A[kk * KG + KS * lg + s2];
            cv[s2] = ps.c[kk * KG + KS * lg + s2];
        }
        ZA[kk] = R::scale(ZC[kk], av);
        ZK[kk] = R::scale(ZC[kk], cv);
    }
    const float An = ps.scal[0], cn = ps.scal[1], En = ps.scal[2];
#pragma unroll
    for (int jt = 0; jt < NCT; ++jt) {
        f32x4 nM = An * dM[jt];
        f32x4 nS = cn * dM[jt] + En * dS[jt];
#pragma unroll
        for (int kk = 0; kk < NKT; ++kk) {
            const F qf = R::cm_t(s.q, Gm::LQ, kk * KG, jt, lr, lg);
            const F kf = R::cm_t(s.k, Gm::LQ, kk * KG, jt, lr, lg);
            nM = O::mma(nM, qf, ZA[kk]);
            nM = O::mma(nM, kf, DE[kk]);
            nS = O::mma(nS, qf, ZK[kk]);
        }
        dM[jt] = nM;
        dS[jt] = nS;
    }
}

template <typename T, int D, int NS, int NP>
__global__ __launch_bounds__((kW * CarryGeo<T, D, NS, NP>::NWAVE)) void linear_memory_bwd_carry(const CarryParams p) {
    using Gm = CarryGeo<T, D, NS, NP>;
    using C = Carry<T, D, NS, NP>;
    using O = Op<T>;
    constexpr int NCT = Gm::NCT;

    __shared__ __attribute__((aligned(16))) typename C::Sm sm;

    const int w = threadIdx.x / kW;
    const int lane = threadIdx.x % kW;
    const int lr = lane & 15, lg = lane >> 4;
    const int nwg = gridDim.x;
    int lin = blockIdx.x;
    if ((p.BH % 8) == 0) lin = (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8;   // row blocks of a sequence on one XCD
    int bh = lin / Gm::NRB;
    int rb = lin % Gm::NRB;
    int nch = p.nch, seqlen = p.T;
    size_t seq_tok = static_cast<size_t>(bh) * p.T;
    size_t w_chunk0 = static_cast<size_t>(bh) * p.nch;   // work-buffer slot of chunk 0
    if (p.cu) {
        // Packed documents: units u = (rank, head), documents ranked longest
        // first and dealt round-robin to the XCDs (the row blocks of a unit on
        // one XCD), so the longest walks start first; sequence bh = document s
        // of head h (state slot s * H + h).
        int u = bh;
        if ((p.BH % 8) == 0) {
            const int x = blockIdx.x % 8, m = blockIdx.x / 8;
            rb = m % Gm::NRB;
            u = (m / Gm::NRB) * 8 + x;
        }
        const int s = doc_of_rank(p.cu, p.BH / p.H, p.T, u / p.H, lane, p.perm), h = u % p.H;
        bh = s * p.H + h;
        int t0;
        seqlen = doc_len(p.cu, s, p.T, t0);
        seq_tok = static_cast<size_t>(h) * p.T + t0;
        // Cut at the head's last slot, as the forward that wrote the
        // checkpoints does (only a table that is not non-decreasing gets there).
        const int pre = doc_chunk_prefix(p.cu, s, p.T, p.b, lane);
        seqlen = min(seqlen, max(p.tcmax - pre, 0) * p.b);
        nch = (seqlen + p.b - 1) / p.b;
        w_chunk0 = static_cast<size_t>(h) * p.tcmax + pre;
    }
    const int row_wg = rb * Gm::RB;
    // Every cotangent enters scaled by sc; dv, dM0, dS0 leave divided by it
    // (the work buffer keeps the scaled cotangents for the gradient kernel).
    const float sc = cot_scale(p.smax, bh);
    const float isc = 1.f / sc;
    auto chunk_of = [&](int u) { return nch - 1 - u; };
    auto chunk_n = [&](int c) { return min(p.b, seqlen - c * p.b); };
    // Gate entry of token 0 of chunk c, and the step between tokens.
    const int gstride = p.chunk_gates ? 0 : 1;
    auto gate0 = [&](int c) {
        return p.chunk_gates ? static_cast<size_t>(bh) * nch + c : seq_tok + static_cast<size_t>(c) * p.b;
    };

    const bool is_state = w < NS;   // the two waves after them load, the last one builds
    const bool is_builder = w == NS + 2;
    const int lw = w - NS;   // loader index

    typename C::Regs lr_regs;
    auto do_issue = [&](int u) {
        const int c = chunk_of(u);
        C::issue(p, lr_regs, seq_tok + static_cast<size_t>(c) * p.b, chunk_n(c), row_wg, lane, lw, gate0(c),
                 gstride);
    };
    auto do_commit = [&](int u) { C::commit(lr_regs, sm.qs[u % Gm::NQ], chunk_n(chunk_of(u)), lane, lw, sc); };
    auto do_build = [&](int u) {
        const int c = chunk_of(u);
        C::build(sm.qs[u % Gm::NQ], sm.ps[u % Gm::NPR], sm.ls, chunk_n(c), lane);
    };

    // State wave: rows r0 .. r0+15 of dM, dS as accumulator tiles of dM^T
    // (tile jt, row m -> column tmap(jt, m) of dM; lane column -> row r0 + lr).
    f32x4 dM[NCT], dS[NCT];
    const int r0l = 16 * w;
    const int r0 = row_wg + r0l;
    const size_t st_off = static_cast<size_t>(bh) * D * D + static_cast<size_t>(r0 + lr) * D;
    auto state_init = [&]() {
#pragma unroll
        for (int jt = 0; jt < NCT; ++jt) {
            const int col = O::tmap(jt, 4 * lg);
            const bool ok = col < D;
            dM[jt] = (p.dMT && ok) ? sc * *reinterpret_cast<const f32x4*>(p.dMT + st_off + col)
                                   : f32x4{0.f, 0.f, 0.f, 0.f};
            dS[jt] = (p.dST && ok) ? sc * *reinterpret_cast<const f32x4*>(p.dST + st_off + col)
                                   : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    auto state_final = [&]() {
#pragma unroll
        for (int jt = 0; jt < NCT; ++jt) {
            const int col = O::tmap(jt, 4 * lg);
            if (col < D) {
                if (p.dM0) *reinterpret_cast<f32x4*>(p.dM0 + st_off + col) = isc * dM[jt];
                if (p.dS0) *reinterpret_cast<f32x4*>(p.dS0 + st_off + col) = isc * dS[jt];
            }
        }
    };

    auto do_state = [&](int u) {
        const int c = chunk_of(u);
        carry_state_step<T, D, NS, NP>(p, sm.qs[u % Gm::NQ], sm.ps[u % Gm::NPR], dM, dS, chunk_n(c),
                                       seq_tok + static_cast<size_t>(c) * p.b, w_chunk0 + c, r0, r0l, lr, lg, isc);
    };

    // Each role runs its own loop; the loops execute the same barriers.
    if constexpr (Gm::NQ == 3) {
        // Step u: state waves on chunk u, builder on u + 1, loader commits
        // u + 2 and fetches u + 3.
        if (is_state) {
            state_init();
            __syncthreads();
            __syncthreads();
            for (int u = 0; u < nch; ++u) {
                do_state(u);
                __syncthreads();
            }
            state_final();
        } else if (is_builder) {
            __syncthreads();
            if (nch > 0) do_build(0);
            __syncthreads();
            for (int u = 0; u < nch; ++u) {
                if (u + 1 < nch) do_build(u + 1);
                __syncthreads();
            }
        } else {
            if (nch > 0) {
                do_issue(0);
                do_commit(0);
            }
            if (nch > 1) do_issue(1);
            __syncthreads();
            if (nch > 1) do_commit(1);
            if (nch > 2) do_issue(2);
            __syncthreads();
            for (int u = 0; u < nch; ++u) {
                if (u + 2 < nch) do_commit(u + 2);
                if (u + 3 < nch) do_issue(u + 3);
                __syncthreads();
            }
        }
    } else {
        if (is_state) state_init();
        for (int u = 0; u < nch; ++u) {
            if (w == NS) {
                const int c = chunk_of(u);
                C::load_direct(p, sm.qs[0], seq_tok + static_cast<size_t>(c) * p.b, chunk_n(c), row_wg, lane,
                               gate0(c), gstride, sc);
            }
            __syncthreads();
            if (is_builder) do_build(u);
            __syncthreads();
            if (is_state) do_state(u);
            __syncthreads();
        }
        if (is_state) state_final();
    }

}

// Packed documents on persistent workgroups: about one workgroup per CU walks
// its table of (document, head) units (build_walk_table: longest first,
// balanced over the workgroup lanes) as one stream of chunks, each document's
// chunks from its last to its first.  The loaders and the builder run ahead
// across document boundaries; the state waves write a document's dM0, dS0
// after its first chunk and take the next document's dM_T, dS_T before that
// document's last chunk.  Each document's gradients are those of a walk of its
// own (the classic kernel's per-chunk step on the same staged inputs).
template <typename T, int D, int NS, int NP>
__global__ __launch_bounds__((kW * CarryGeo<T, D, NS, NP>::NWAVE)) void linear_memory_bwd_carry_packed(
    const CarryParams p) {
    using Gm = CarryGeo<T, D, NS, NP>;
    using C = Carry<T, D, NS, NP>;
    using O = Op<T>;
    constexpr int NCT = Gm::NCT;
    constexpr int NTH = kW * Gm::NWAVE;
    static_assert(Gm::PERSIST, "persistent walk: three staging slots");

    __shared__ __attribute__((aligned(16))) typename C::Sm sm;

    const int tid = threadIdx.x;
    const int w = tid / kW;
    const int lane = tid % kW;
    const int lr = lane & 15, lg = lane >> 4;
    const int V = gridDim.x / (8 * Gm::NRB);
    const int x8 = blockIdx.x % 8, m = blockIdx.x / 8;
    const int rb = m % Gm::NRB, v = m / Gm::NRB;
    const int row_wg = rb * Gm::RB;
    const int N = p.BH / p.H, b = p.b;

    // The table (its scratch in the last staging slot), the units' cotangent
    // scales, and the empty documents: dM0 = dM_T, dS0 = dS_T on this row block.
    int* temp = reinterpret_cast<int*>(&sm.qs[Gm::NQ - 1]);
    build_walk_table<NTH, Gm::KMAX>(p.cu, N, p.H, p.T, b, true, p.tcmax, temp, sm.units, &sm.nitems, x8, v, V);
    {
        const int nu0 = sm.nunits;
        for (int kk = tid; kk < nu0; kk += NTH) sm.usc[kk] = cot_scale(p.smax, sm.units[kk].bh);
        const int empties = sm.nempty;
        const int* tempty = temp + 4 * N;
        if (p.dM0 || p.dS0) {
            constexpr int Q = D / 4;
            for (int e = 0; e < empties; ++e) {
                const size_t base = static_cast<size_t>(tempty[e]) * D * D + static_cast<size_t>(row_wg) * D;
                for (int i = tid; i < Gm::RB * Q; i += NTH) {
                    const size_t off = base + static_cast<size_t>(i / Q) * D + 4 * (i % Q);
                    const f32x4 zero{0.f, 0.f, 0.f, 0.f};
                    if (p.dM0) *reinterpret_cast<f32x4*>(p.dM0 + off) = p.dMT ? *reinterpret_cast<const f32x4*>(p.dMT + off) : zero;
                    if (p.dS0) *reinterpret_cast<f32x4*>(p.dS0 + off) = p.dST ? *reinterpret_cast<const f32x4*>(p.dST + off) : zero;
                }
            }
        }
        __syncthreads();
        for (int i = tid; i < 4 * N + Gm::KMAX; i += NTH) temp[i] = 0;
        __syncthreads();
    }
    const int nu = __builtin_amdgcn_readfirstlane(sm.nunits);
    const int J = __builtin_amdgcn_readfirstlane(sm.nitems);

    // Walk position: unit k, its chunk c (counting down from nch - 1); past the
    // last unit every chunk has no tokens.
    struct Walk {
        int k, c, len, tok0, ck0, bh;
        float sc;
    };
    auto at = [&](Walk& q, int k) {
        q.k = k;
        if (k < nu) {
            const WalkUnit u = sm.units[k];
            q.tok0 = __builtin_amdgcn_readfirstlane(u.tok0);
            q.len = __builtin_amdgcn_readfirstlane(u.len);
            q.ck0 = __builtin_amdgcn_readfirstlane(u.ck0);
            q.bh = __builtin_amdgcn_readfirstlane(u.bh);
            q.sc = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sm.usc[k])));
            q.c = (q.len + b - 1) / b - 1;
        } else {
            q.tok0 = q.len = q.ck0 = q.bh = q.c = 0;
            q.sc = 1.f;
        }
    };
    auto next = [&](Walk& q) {
        if (q.c > 0) --q.c;
        else at(q, q.k + 1);
    };
    auto n_of = [&](const Walk& q) { return max(0, min(b, q.len - q.c * b)); };
    auto tok_of = [&](const Walk& q) { return static_cast<size_t>(q.tok0) + static_cast<size_t>(q.c) * b; };

    if (w < NS) {
        // ===================== state waves =====================
        const int r0l = 16 * w;
        const int r0 = row_wg + r0l;
        f32x4 dM[NCT], dS[NCT];
        Walk q;
        at(q, 0);
        auto off_of = [&]() { return static_cast<size_t>(q.bh) * D * D + static_cast<size_t>(r0 + lr) * D; };
        // The document's dM_T, dS_T (scaled); the loads are waited for here, so
        // that the common path of the walk carries no wait on its own stores.
        auto init = [&]() {
            const f32x4 zero{0.f, 0.f, 0.f, 0.f};
            if (q.k < nu && (p.dMT || p.dST)) {
                const size_t so = off_of();
#pragma unroll
                for (int jt = 0; jt < NCT; ++jt) {
                    const int col = O::tmap(jt, 4 * lg);
                    const bool ok = col < D;
                    dM[jt] = (p.dMT && ok) ? q.sc * *reinterpret_cast<const f32x4*>(p.dMT + so + col) : zero;
                    dS[jt] = (p.dST && ok) ? q.sc * *reinterpret_cast<const f32x4*>(p.dST + so + col) : zero;
                }
                __builtin_amdgcn_s_waitcnt(kWaitVm0);
            } else {
#pragma unroll
                for (int jt = 0; jt < NCT; ++jt) {
                    dM[jt] = zero;
                    dS[jt] = zero;
                }
            }
        };
        auto final_ = [&]() {
            const size_t so = off_of();
            const float isc = 1.f / q.sc;
#pragma unroll
            for (int jt = 0; jt < NCT; ++jt) {
                const int col = O::tmap(jt, 4 * lg);
                if (col < D) {
                    if (p.dM0) *reinterpret_cast<f32x4*>(p.dM0 + so + col) = isc * dM[jt];
                    if (p.dS0) *reinterpret_cast<f32x4*>(p.dS0 + so + col) = isc * dS[jt];
                }
            }
        };
        init();
        __syncthreads();
        __syncthreads();
        for (int u = 0; u < J; ++u) {
            carry_state_step<T, D, NS, NP>(p, sm.qs[u % Gm::NQ], sm.ps[u % Gm::NPR], dM, dS, n_of(q), tok_of(q),
                                           static_cast<size_t>(q.ck0) + q.c, r0, r0l, lr, lg, 1.f / q.sc);
            if (q.c == 0) {
                final_();
                at(q, q.k + 1);
                init();
            } else {
                --q.c;
            }
            __syncthreads();
        }
    } else if (w == NS + 2) {
        // ===================== builder =====================
        Walk q;
        at(q, 0);
        auto build = [&](int u) { C::build(sm.qs[u % Gm::NQ], sm.ps[u % Gm::NPR], sm.ls, n_of(q), lane); };
        __syncthreads();
        if (J > 0) {
            build(0);
            next(q);
        }
        __syncthreads();
        for (int u = 0; u < J; ++u) {
            if (u + 1 < J) {
                build(u + 1);
                next(q);
            }
            __syncthreads();
        }
    } else {
        // ===================== loaders =====================
        // Items are requested in order (three steps ahead) and staged one step
        // later; the length and scale of the two not yet staged are kept by parity.
        const int lw = w - NS;
        typename C::Regs regs;
        Walk q;
        at(q, 0);
        int rn[2] = {0, 0};
        float rsc[2] = {1.f, 1.f};
        int ji = 0;
        auto issue = [&]() {
            const size_t t0 = tok_of(q);
            const int n = n_of(q);
            C::issue(p, regs, t0, n, row_wg, lane, lw, t0, 1);
            if (ji & 1) {
                rn[1] = n;
                rsc[1] = q.sc;
            } else {
                rn[0] = n;
                rsc[0] = q.sc;
            }
            ++ji;
            next(q);
        };
        auto commit = [&](int u) {
            const bool odd = u & 1;
            C::commit(regs, sm.qs[u % Gm::NQ], odd ? rn[1] : rn[0], lane, lw, odd ? rsc[1] : rsc[0]);
        };
        if (J > 0) {
            issue();
            commit(0);
        }
        if (J > 1) issue();
        __syncthreads();
        if (J > 1) commit(1);
        if (J > 2) issue();
        __syncthreads();
        for (int u = 0; u < J; ++u) {
            if (u + 2 < J) commit(u + 2);
            if (u + 3 < J) issue();
            __syncthreads();
        }
    }
}

// ===========================================================================
// Gradient kernel: one workgroup per (sequence, chunk).
// ===========================================================================
struct GradParams {
    const void* q;
    const void* k;
    const void* v;
    const float* theta;
    const float* eta;
    const float* alpha;
    const void* ckpt;    // [BH][nch][M | S][D][D]: state entering each chunk (float32 or fp16)
    const void* work;    // [BH][nch][dM | dS][D][D]: cotangent leaving each chunk (same type)
    const float* dz;
    const float* dv;
    float* dq;
    float* dk;
    float* dth;
    float* deta;
    float* dal;
    int BH;
    int T;
    int b;
    int nch;
    int chunk_gates;     // gates and their gradients [BH][nch]
    // Packed documents (NULL: dense): workgroup = (head h, chunk slot) of
    // the [H][tcmax] checkpoint and work layouts.
    const int* cu;
    int H;
    int tcmax;
    const float* smax;   // as for the carry
};

template <typename T, int D, int NP>
struct GradGeo {
    using O = Op<T>;
    static constexpr int KG = O::KG;
    static constexpr int KS = KG / 4;
    static constexpr int DS = bmax(D, KG);
    static constexpr int NF = D / 16;           // feature tiles
    static constexpr int FPW = 1; // feature tiles per wave (register budget)
    static constexpr int NWAVE = 1 + NF / FPW;  // plus the gate wave
    static constexpr int NT = NP / 16;
    static constexpr int NKD = DS / KG;
    static constexpr int NKT = NP / KG;
    static constexpr int PAD = 16 / (int)sizeof(T);
    static constexpr int LQ = DS + PAD;
    static constexpr int LPT = NP + PAD;
    static constexpr int LF = NP + 4;
    static constexpr int TILE = NP * LQ * (int)sizeof(T);
    static constexpr int BASE = 3 * TILE + NP * LPT * (int)sizeof(T) + 2 * NP * LF * 4 + 8 * NP * 4;
    // Per-wave partial sums (four token vectors and three dots), added by the
    // gate wave in wave order.
    static constexpr int PART = 4 * NP + 4;
    static_assert(NF * PART * 4 <= TILE, "partials fit the residual tile");
    // dz and -dv staged as operands too when they fit (else read from HBM / L2).
    static constexpr bool DZ_LDS = BASE + 2 * TILE + 1024 <= kLdsMax;
    // The gate wave's reverse pass runs over dL alone before the feature
    // waves' partial sums arrive (they enter as a closed-form correction)
    // when a second copy of the gamma table fits; else it runs after them.
    static constexpr bool SPLIT = BASE + (DZ_LDS ? 2 * TILE : 0) + NP * LF * 4 + 1024 <= kLdsMax;
    // The partial sums get a region of their own when it fits too (written as
    // soon as they are formed, one barrier fewer); else they reuse the
    // residual tile once it is consumed.
    static constexpr bool PART_OWN =
        SPLIT && BASE + (DZ_LDS ? 2 * TILE : 0) + NP * LF * 4 + NF * PART * 4 + 1024 <= kLdsMax;
    static_assert(BASE + 1024 <= kLdsMax, "LDS budget");
    static_assert(NP % KG == 0, "tiling");
};

template <typename T, int D, int NP>
struct GradSmem {
    using Gm = GradGeo<T, D, NP>;
    alignas(16) T q[NP * Gm::LQ];
    alignas(16) T k[NP * Gm::LQ];
    alignas(16) T ec[NP * Gm::LQ];               // residuals E at the chunk-start state
    alignas(16) T dz[Gm::DZ_LDS ? NP * Gm::LQ : 8];
    alignas(16) T de[Gm::DZ_LDS ? NP * Gm::LQ : 8];
    alignas(16) T dlt[NP * Gm::LPT];             // -(D .* L)^T
    alignas(16) float lm[NP * Gm::LF];           // gamma_ij; then the eta contributions
    alignas(16) float dl[NP * Gm::LF];           // dL_ij; then the a contributions
    alignas(16) float th[NP];
    alignas(16) float et[NP];
    alignas(16) float av[NP];
    alignas(16) float A[NP];
    alignas(16) float Ev[NP];
    alignas(16) float c[NP];
    alignas(16) float wm[NP];
    alignas(16) float ws[NP];
    alignas(16) float ce[Gm::SPLIT ? NP * Gm::LF : 4];   // the eta contributions (gamma kept in lm)
    alignas(16) float part[Gm::PART_OWN ? Gm::NF * Gm::PART : 4];
};

template <typename T, int D, int NP>
__global__ __launch_bounds__((kW * GradGeo<T, D, NP>::NWAVE)) void linear_memory_bwd_grads(const GradParams p) {
    using Gm = GradGeo<T, D, NP>;
    using O = Op<T>;
    using R = Fr<T>;
    using F = typename O::frag;
    using G = typename GlobalOf<T>::type;
    constexpr int KG = Gm::KG, KS = Gm::KS, NT = Gm::NT, NKD = Gm::NKD, NKT = Gm::NKT;
    constexpr int LQ = Gm::LQ, LPT = Gm::LPT, LF = Gm::LF;

    __shared__ __attribute__((aligned(16))) GradSmem<T, D, NP> sm;

    const int tid = threadIdx.x;
    const int w = tid / kW;
    const int lane = tid % kW;
    const int lr = lane & 15, lg = lane >> 4;
    int bh, c, n;
    size_t tok0, slot;
    if (p.cu) {
        // Packed documents: workgroup = (head h, chunk slot); the slots past
        // the head's last chunk have no work (the whole workgroup leaves).
        // The slot's document is found by the wave's lanes, 64 documents at a
        // time: each lane takes one document's chunk count, an inclusive
        // prefix sum over the lanes gives each document's slot range, and a
        // ballot picks the one holding the slot (empty documents own none).
        const int h = blockIdx.x / p.tcmax, cidx = blockIdx.x % p.tcmax;
        const int ndoc = p.BH / p.H;
        int s = -1, acc = 0, t0 = 0, len = 0;
        for (int base = 0, before = 0; base < ndoc; base += kW) {
            const int j = base + lane;
            int tj = 0, lj = 0;
            if (j < ndoc) lj = doc_len(p.cu, j, p.T, tj);
            const int nj = (lj + p.b - 1) / p.b;
            int incl = nj;
            for (int o = 1; o < kW; o <<= 1) {
                const int y = __shfl_up(incl, o, kW);
                incl += lane >= o ? y : 0;
            }
            const int first = before + incl - nj;
            const unsigned long long hit = __ballot(j < ndoc && cidx >= first && cidx < first + nj);
            if (hit) {
                const int l = __ffsll(static_cast<long long>(hit)) - 1;
                s = base + l;
                acc = __builtin_amdgcn_readfirstlane(__shfl(first, l, kW));
                t0 = __builtin_amdgcn_readfirstlane(__shfl(tj, l, kW));
                len = __builtin_amdgcn_readfirstlane(__shfl(lj, l, kW));
                break;
            }
            before += __shfl(incl, kW - 1, kW);
        }
        if (s < 0) return;
        c = cidx - acc;
        bh = s * p.H + h;
        n = min(p.b, len - c * p.b);
        tok0 = static_cast<size_t>(h) * p.T + t0 + static_cast<size_t>(c) * p.b;
        slot = static_cast<size_t>(h) * p.tcmax + cidx;
    } else {
        bh = blockIdx.x / p.nch;
        c = blockIdx.x % p.nch;
        n = min(p.b, p.T - c * p.b);
        tok0 = static_cast<size_t>(bh) * p.T + static_cast<size_t>(c) * p.b;
        slot = static_cast<size_t>(bh) * p.nch + c;
    }
    // Cotangents enter scaled by sc (the work buffer already is); every
    // gradient leaves divided by it.
    const float sc = cot_scale(p.smax, bh);
    const float isc = 1.f / sc;
    const T* Mc = static_cast<const T*>(p.ckpt) + slot * (2 * D * D);
    const T* Sc = Mc + D * D;
    const T* dMe = static_cast<const T*>(p.work) + slot * (2 * D * D);
    const T* dSe = dMe + D * D;

    // ---- stage q, k (and dz, -dv), raw gates; clear the accumulators ----
    {
        constexpr int CB = 16 / (int)sizeof(G);
        constexpr int UR = Gm::DS / CB;
        const G* q = static_cast<const G*>(p.q);
        const G* k = static_cast<const G*>(p.k);
        // All loads of a thread first (clamped, always in bounds), then the
        // LDS writes: one HBM latency for the whole staging.
        constexpr int NTH = kW * Gm::NWAVE;
        constexpr int NQU = (NP * UR + NTH - 1) / NTH;
        uint4 qa[NQU], ka[NQU];
#pragma unroll
        for (int i = 0; i < NQU; ++i) {
            const int u = tid + i * NTH;
            const int t = u / UR, col = (u % UR) * CB;
            const bool ok = u < NP * UR && t < n && col < D;
            const size_t g = ok ? (tok0 + t) * D + col : 0;
            const uint4 a = *reinterpret_cast<const uint4*>(q + g);
            const uint4 b = *reinterpret_cast<const uint4*>(k + g);
            qa[i] = ok ? a : uint4{0u, 0u, 0u, 0u};
            ka[i] = ok ? b : uint4{0u, 0u, 0u, 0u};
        }
        constexpr int U4 = Gm::DS / 4;
        constexpr int NZU = Gm::DZ_LDS ? (NP * U4 + NTH - 1) / NTH : 1;
        f32x4 za[NZU], va[NZU];
        if constexpr (Gm::DZ_LDS) {
#pragma unroll
            for (int i = 0; i < NZU; ++i) {
                const int u = tid + i * NTH;
                const int t = u / U4, col = (u % U4) * 4;
                const bool ok = u < NP * U4 && t < n && col < D;
                const size_t g = ok ? (tok0 + t) * D + col : 0;
                const f32x4 z4 = *reinterpret_cast<const f32x4*>(p.dz + g);
                const f32x4 v4 = *reinterpret_cast<const f32x4*>(p.dv + g);
                za[i] = ok ? sc * z4 : f32x4{0.f, 0.f, 0.f, 0.f};
                va[i] = ok ? -sc * v4 : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
#pragma unroll
        for (int i = 0; i < NQU; ++i) {
            const int u = tid + i * NTH;
            if (u < NP * UR) {
                const int t = u / UR, col = (u % UR) * CB;
                put_unit<T>(sm.q + t * LQ + col, qa[i]);
                put_unit<T>(sm.k + t * LQ + col, ka[i]);
                if constexpr (Gm::DS > D) put_unit<T>(sm.ec + t * LQ + col, uint4{0u, 0u, 0u, 0u});
            }
        }
        if constexpr (Gm::DZ_LDS) {
#pragma unroll
            for (int i = 0; i < NZU; ++i) {
                const int u = tid + i * NTH;
                if (u < NP * U4) {
                    const int t = u / U4, col = (u % U4) * 4;
                    st4<T>(sm.dz + t * LQ + col, za[i]);
                    st4<T>(sm.de + t * LQ + col, va[i]);
                }
            }
        }
        for (int l = tid; l < NP; l += kW * Gm::NWAVE) {
            const bool ok = l < n;
            const size_t gi = p.chunk_gates ? static_cast<size_t>(bh) * p.nch + c : tok0 + l;
            sm.th[l] = ok ? p.theta[gi] : 0.f;
            sm.et[l] = ok ? p.eta[gi] : 1.f;
            sm.av[l] = ok ? 1.f - p.alpha[gi] : 1.f;
        }
    }
    // Partial sums of feature wave f: [dA | dc | dw^M | dw^S][NP], then the three dots.
    float* const part = Gm::PART_OWN ? sm.part : reinterpret_cast<float*>(sm.ec);
    __syncthreads();

    // Row-major operand fragment of dz or -dv (token row t, k-group at k0).
    auto zfrag = [&](const T* lds, const float* glob, float sign, int t, int k0) -> F {
        if constexpr (Gm::DZ_LDS) {
            return R::rm(lds, LQ, t, k0, lg);
        } else {
            sign *= sc;
            float x[KS];
            const int col = k0 + KS * lg;
            const bool ok = t < n && col < D;
#pragma unroll
            for (int s = 0; s < KS; s += 4) {
                const f32x4 v4 = ok ? *reinterpret_cast<const f32x4*>(glob + (tok0 + t) * D + col + s) : f32x4{0.f, 0.f, 0.f, 0.f};
                x[s] = sign * v4[0];
                x[s + 1] = sign * v4[1];
                x[s + 2] = sign * v4[2];
                x[s + 3] = sign * v4[3];
            }
            return R::from_f32(x);
        }
    };

    // Lower tiles of G = Q K^T and D = dZ E^T: dL = -G .* D into dl and
    // -(D .* L)^T into dlt (upper tiles zero), shared out over all waves.
    auto tiles = [&]() {
#pragma unroll 1
        for (int idx = w; idx < NT * NT; idx += Gm::NWAVE) {
            const int it = idx / NT, jt = idx % NT;
            const int j = 16 * jt + lr;
            T* dst = sm.dlt + j * LPT + 16 * it + 4 * lg;
            if (jt > it) {
                st4<T>(dst, f32x4{0.f, 0.f, 0.f, 0.f});
                continue;
            }
            f32x4 gacc = {0.f, 0.f, 0.f, 0.f}, dacc = gacc;
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk) {
                gacc = O::mma(gacc, R::rm(sm.q, LQ, 16 * it + lr, kk * KG, lg), R::rm(sm.k, LQ, j, kk * KG, lg));
                dacc = O::mma(dacc, zfrag(sm.dz, p.dz, 1.f, 16 * it + lr, kk * KG), R::rm(sm.ec, LQ, j, kk * KG, lg));
            }
            f32x4 nd;
            const float thj = sm.th[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * it + 4 * lg + e;
                const bool ok = j <= i;
                const float gv = sm.lm[i * LF + j];   // unconditional read: a select, not a branch
                nd[e] = ok ? -dacc[e] * (thj * gv) : 0.f;
                sm.dl[i * LF + j] = ok ? -gacc[e] * dacc[e] : 0.f;
            }
            st4<T>(dst, nd);
        }
    };

    if (w == 0) {
        // ===================== gate wave =====================
        const int l = lane;
        const float my_th = sm.th[l % NP], my_et = sm.et[l % NP], my_a = sm.av[l % NP];
        float A, E, cc;
        gate_prefix(my_a, my_et, A, E, cc);
        if (l < NP) {
            sm.A[l] = A;
            sm.Ev[l] = E;
            sm.c[l] = cc;
        }
        float g_last, p_last;
        gamma_columns<NP>(sm.av, sm.et, n, [&](int i, float g) {
            if (l < NP) sm.lm[i * LF + l] = g;
        }, g_last, p_last);
        if (l < NP) {
            sm.wm[l] = my_th * g_last;
            sm.ws[l] = my_th * p_last;
        }
        __syncthreads();   // (1) gates and residual tiles ready

        tiles();
        __syncthreads();   // (1b) dL and -(D .* L)^T complete
        // Reverse through the column recurrences of gamma and p (lane = column j).
        // Row i reads gamma rows i, i-1 and dL row i; the loads for the next
        // row are issued one iteration ahead.  p comes back from gamma without
        // a division: p_ij = gamma_ij - a_i gamma_{i-1,j} (gamma_{j-1,j} = 0).
        // The contributions to a_i (into dl) and eta_i (into cedst) are summed
        // over each row afterwards.  WITH_LAST adds the cotangents of the
        // chunk-end weights (dwm_j, dws_j), which enter at row n - 1.
        const int lc = l < NP ? l : 0;
        float dth = 0.f;
        auto reverse_pass = [&](auto with_last, float dwm_j, float dws_j, float* cedst) {
            constexpr bool WITH_LAST = decltype(with_last)::value;
            float gg = 0.f, gp = 0.f;
            float g_i = sm.lm[(NP - 1) * LF + lc];
            float g_im1 = NP > 1 ? sm.lm[(NP - 2) * LF + lc] : 0.f;
            float d_i = sm.dl[(NP - 1) * LF + lc];
#pragma unroll
            for (int i = NP - 1; i >= 0; --i) {
                const float g_im2 = i >= 2 ? sm.lm[(i >= 2 ? i - 2 : 0) * LF + lc] : 0.f;
                const float d_im1 = i >= 1 ? sm.dl[(i >= 1 ? i - 1 : 0) * LF + lc] : 0.f;
                const bool act = i >= l && i < n;
                float dli = act ? d_i : 0.f;
                const float a_i = readlane(my_a, i);
                if constexpr (WITH_LAST) {
                    const bool last = act && i == n - 1;
                    if (last) dli += dwm_j;
                    gg += my_th * dli;
                    dth += dli * g_i;
                    if (last) {
                        gp += my_th * dws_j;
                        dth += dws_j * (g_i - a_i * g_im1);
                    }
                } else {
                    gg += my_th * dli;
                    dth += dli * g_i;
                }
                float ca = 0.f, ce = 0.f;
                if (i > 0 && i > l) {
                    const float a_im1 = readlane(my_a, i > 0 ? i - 1 : 0);
                    ca = gg * g_im1;
                    gp += gg;
                    ce = gp * (g_im1 - a_im1 * g_im2);
                    gg *= a_i;
                    gp *= readlane(my_et, i);
                }
                if (l < NP) {
                    sm.dl[i * LF + l] = ca;
                    cedst[i * LF + l] = ce;
                }
                g_i = g_im1;
                g_im1 = g_im2;
                d_i = d_im1;
                // Keep the running sums in registers row by row (the compiler
                // would otherwise defer them and hold every row's dL live).
                asm volatile("" : "+v"(dth), "+v"(gg), "+v"(gp));
                __builtin_amdgcn_sched_barrier(0);
            }
            wave_lds_fence();
        };
        // Row sums (lane = row i) of the a and eta contributions.
        float sa = 0.f, se = 0.f;
        auto row_sums = [&](const float* cesrc) {
            if (l < NP) {
#pragma unroll 2
                for (int j = 0; j < NP; j += 4) {
                    const f32x4 va = *reinterpret_cast<const f32x4*>(sm.dl + l * LF + j);
                    const f32x4 ve = *reinterpret_cast<const f32x4*>(cesrc + l * LF + j);
                    sa += (va[0] + va[1]) + (va[2] + va[3]);
                    se += (ve[0] + ve[1]) + (ve[2] + ve[3]);
                }
            }
        };
        if constexpr (Gm::SPLIT) {
            wave_lds_fence();
            reverse_pass(std::false_type{}, 0.f, 0.f, sm.ce);
            row_sums(sm.ce);
        }
        __syncthreads();   // (2) feature waves past their state products
        if constexpr (!Gm::PART_OWN) __syncthreads();   // (3) partial sums of the feature waves written
        // Scalar cotangents: partial sums added in wave order (deterministic).
        float dA_l = 0.f, dc_l = 0.f, dwm_j = 0.f, dws_j = 0.f, dot0 = 0.f, dot1 = 0.f, dEn = 0.f;
#pragma unroll
        for (int f = 0; f < Gm::NF; ++f) {
            const float* pf = part + f * Gm::PART;
            dA_l += pf[l % NP];
            dc_l += pf[NP + l % NP];
            dwm_j += pf[2 * NP + l % NP];
            dws_j += pf[3 * NP + l % NP];
            dot0 += pf[4 * NP];
            dot1 += pf[4 * NP + 1];
            dEn += pf[4 * NP + 2];
        }
        // g_i = u_i + f_i g_{i+1} with f_i = a_{i+1} (A, c and the a-suffix
        // products) or eta_{i+1} (E and the eta-suffix products).
        const float a_next = __shfl(my_a, l + 1 < kW ? l + 1 : l, kW);
        const float e_next = __shfl(my_et, l + 1 < kW ? l + 1 : l, kW);
        const float fa = l + 1 < NP ? a_next : 0.f, fe = l + 1 < NP ? e_next : 0.f;
        if constexpr (!Gm::SPLIT) {
            reverse_pass(std::true_type{}, dwm_j, dws_j, sm.lm);
            row_sums(sm.lm);
        } else {
            // The chunk-end weights' cotangents enter the reverse pass at row
            // n - 1 with gg = theta_j dwm_j =: u_j and gp = theta_j dws_j =: w_j.
            // The pass is linear, so their part follows in closed form: at row i
            // gg = u_j Ra_i and gp = w_j Re_i + u_j Qc_i, with the suffix products
            // Ra_i = a_{i+1} .. a_{n-1}, Re_i = eta_{i+1} .. eta_{n-1} and
            // Qc_i = Ra_i + eta_{i+1} Qc_{i+1}; summed over the columns j < i:
            //   a part:   Ra_i (Gamma u)_{i-1}
            //   eta part: Re_i (P w)_{i-1} + Qc_i (P u)_{i-1},
            // with (P x)_{i-1} = (Gamma x)_{i-1} - a_{i-1} (Gamma x)_{i-2}.
            const bool col_on = l < n;
            const float g_last = sm.lm[(n - 1) * LF + lc];
            const float g_prev = n >= 2 ? sm.lm[(n >= 2 ? n - 2 : 0) * LF + lc] : 0.f;
            const float a_last = readlane(my_a, n - 1);
            if (col_on) dth += dwm_j * g_last + dws_j * (g_last - a_last * g_prev);
            // u and w go through the (no longer read) weight vectors.
            if (l < NP) {
                sm.wm[l] = col_on ? my_th * dwm_j : 0.f;
                sm.ws[l] = col_on ? my_th * dws_j : 0.f;
            }
            wave_lds_fence();
            float gu = 0.f, gw = 0.f;   // (Gamma u)_r, (Gamma w)_r for r = lane
#pragma unroll 4
            for (int j = 0; j < NP; j += 4) {
                const f32x4 gr = *reinterpret_cast<const f32x4*>(sm.lm + lc * LF + j);
                const f32x4 uu = *reinterpret_cast<const f32x4*>(sm.wm + j);
                const f32x4 ww = *reinterpret_cast<const f32x4*>(sm.ws + j);
                gu += (gr[0] * uu[0] + gr[1] * uu[1]) + (gr[2] * uu[2] + gr[3] * uu[3]);
                gw += (gr[0] * ww[0] + gr[1] * ww[1]) + (gr[2] * ww[2] + gr[3] * ww[3]);
            }
            const float one_last = l == n - 1 ? 1.f : 0.f;
            const float Ra = reverse_recurrence<NP>(one_last, fa, l);
            const float Re = reverse_recurrence<NP>(one_last, fe, l);
            const float Qc = reverse_recurrence<NP>(Ra, fe, l);
            // Every lane takes part in the shuffles; the lanes with no row
            // i - 1 (or i - 2) mask the value afterwards.
            const int s1 = l >= 1 ? l - 1 : 0, s2 = l >= 2 ? l - 2 : 0;
            const float gu1r = __shfl(gu, s1, kW), gu2r = __shfl(gu, s2, kW);
            const float gw1r = __shfl(gw, s1, kW), gw2r = __shfl(gw, s2, kW);
            const float a_m1 = __shfl(my_a, s1, kW);
            const float gu1 = l >= 1 ? gu1r : 0.f, gu2 = l >= 2 ? gu2r : 0.f;
            const float gw1 = l >= 1 ? gw1r : 0.f, gw2 = l >= 2 ? gw2r : 0.f;
            if (l >= 1 && l < n) {
                sa += Ra * gu1;
                se += Re * (gw1 - a_m1 * gw2) + Qc * (gu1 - a_m1 * gu2);
            }
        }
        const float my_dA = dA_l + (l == n - 1 ? dot0 : 0.f);
        const float my_dc = dc_l + (l == n - 1 ? dot1 : 0.f);
        const float gA = reverse_recurrence<NP>(my_dA, fa, l);
        const float gc = reverse_recurrence<NP>(my_dc, fa, l);
        const float gE = reverse_recurrence<NP>(gc + (l == n - 1 ? dEn : 0.f), fe, l);
        const float A_prev = l > 0 ? sm.A[(l - 1) % NP] : 1.f;
        const float c_prev = l > 0 ? sm.c[(l - 1) % NP] : 0.f;
        const float E_prev = l > 0 ? sm.Ev[(l - 1) % NP] : 1.f;
        const float da = sa + gA * A_prev + gc * c_prev;
        const float de = se + gE * E_prev;
        if (p.chunk_gates) {
            // A gate shared by the chunk's tokens collects all of their gradients.
            const float st = wave_sum(l < n ? dth : 0.f), se2 = wave_sum(l < n ? de : 0.f);
            const float sa2 = wave_sum(l < n ? da : 0.f);
            if (l == 0) {
                const size_t gi = static_cast<size_t>(bh) * p.nch + c;
                p.dth[gi] = isc * st;
                p.deta[gi] = isc * se2;
                p.dal[gi] = -isc * sa2;
            }
        } else if (l < n) {
            p.dth[tok0 + l] = isc * dth;
            p.deta[tok0 + l] = isc * de;
            p.dal[tok0 + l] = -isc * da;
        }
    } else {
        // ===================== feature wave =====================
        // Feature tiles fw*FPW .. fw*FPW + FPW - 1, 16 rows (residuals) or
        // features (gradients) each.
        constexpr int FPW = Gm::FPW;
        const int fw = w - 1;
        // Columns f0 .. f0+15 of a state as an operand whose rows are those
        // columns (k = row of the state): raw loads, then conversion, so the
        // next state's loads are in flight while the current one is used.
        // Raw column values, two consecutive rows per 32-bit register.
        // fp16: one 32-bit word per register (two adjacent columns of row
        // r + (lr & 1)); lanes 2m and 2m + 1 then swap halves (one DPP move and
        // one byte permute) so that each holds rows r, r + 1 of its own column.
        // Buffer loads keep the state's base in scalar registers and the row
        // offsets as constants; rows at or past D read 0.
        using R2 = typename std::conditional<Op<T>::kF16, uint32_t, f32x2>::type;
        constexpr int NRAW = NKD * KS / 2;
        auto colload = [&](const T* X, int f0, R2* raw) {
            if constexpr (Op<T>::kF16) {
                const __amdgpu_buffer_rsrc_t rs = make_rsrc(X, D * D * sizeof(T));
                const uint32_t vo = static_cast<uint32_t>(((KS * lg + (lr & 1)) * D + f0 + (lr & ~1)) * sizeof(T));
#pragma unroll
                for (int kk = 0; kk < NKD; ++kk) {
#pragma unroll
                    for (int s2 = 0; s2 < KS; s2 += 2)
                        raw[(kk * KS + s2) / 2] = __builtin_bit_cast(
                            uint32_t, buf_load4(rs, vo + static_cast<uint32_t>((kk * KG + s2) * D * sizeof(T))));
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < NKD; ++kk) {
#pragma unroll
                    for (int s2 = 0; s2 < KS; s2 += 2) {
                        const int r = kk * KG + KS * lg + s2;
                        const size_t o = static_cast<size_t>(r < D ? r : 0) * D + f0 + lr;
                        raw[(kk * KS + s2) / 2] = R2{X[o], X[o + D]};
                    }
                }
            }
        };
        auto colcvt = [&](const R2* raw, F* out) {
            if constexpr (Op<T>::kF16) {
                // even lane: (own lo, partner lo); odd lane: (partner hi, own hi)
                const uint32_t sel = (lr & 1) ? 0x03020706u : 0x05040100u;
#pragma unroll
                for (int kk = 0; kk < NKD; ++kk) {
#pragma unroll
                    for (int s2 = 0; s2 < KS; s2 += 2) {
                        const uint32_t wv = raw[(kk * KS + s2) / 2];
                        const uint32_t pv = static_cast<uint32_t>(
                            __builtin_amdgcn_mov_dpp(static_cast<int>(wv), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
                        const f16x2 h = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(pv, wv, sel));
                        out[kk][s2] = h[0];
                        out[kk][s2 + 1] = h[1];
                    }
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < NKD; ++kk) {
#pragma unroll
                    for (int s2 = 0; s2 < KS; ++s2)
                        out[kk][s2] = kk * KG + KS * lg + s2 < D ? raw[(kk * KS + s2) / 2][s2 & 1] : static_cast<T>(0.f);
                }
            }
        };
        // Residual rows of E^T: E^T[r][t] = M0[r][:] . k_t - v_t[r].
        const G* vg = static_cast<const G*>(p.v);
#pragma unroll
        for (int ft = 0; ft < FPW; ++ft) {
            const int f0 = 16 * (fw * FPW + ft);
            F am[NKD];
            const size_t ro = static_cast<size_t>(f0 + lr) * D;
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk) {
                // KS consecutive elements of row f0 + lr: one 16-byte load.
                const int col = kk * KG + KS * lg;
                const bool ok = col < D;
                const F m = *reinterpret_cast<const F*>(Mc + ro + (ok ? col : 0));
                am[kk] = ok ? m : F{};
            }
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const int t = 16 * tt + lr;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < NKD; ++kk) acc = O::mma(acc, am[kk], R::rm(sm.k, LQ, t, kk * KG, lg));
                const f32x4 vv = t < n ? gload4<T>(vg + (tok0 + t) * D + f0 + 4 * lg) : f32x4{0.f, 0.f, 0.f, 0.f};
                st4<T>(sm.ec + t * LQ + f0 + 4 * lg, acc - vv);
            }
        }
        // The first state in flight is M0, whose rows the residual pass above
        // has just brought into the L2: its column slices are read from there.
        R2 raw[NRAW];
        colload(Mc, 16 * fw * FPW, raw);
        __syncthreads();   // (1)
        tiles();
        __syncthreads();   // (1b)

        // Products with features f0.. as rows and tokens as columns: lane
        // (lr, lg) holds features f0 + 4lg + e of token t = 16tt + lr.
        auto red = [&](float x) {
            x += __shfl_xor(x, 16, kW);
            x += __shfl_xor(x, 32, kW);
            return x;
        };
        auto rdot = [&](const f32x4& a, const f32x4& b) { return red((a[0] * b[0] + a[1] * b[1]) + (a[2] * b[2] + a[3] * b[3])); };
        // The three state dots over the wave's columns (every element of the
        // d x d states once over the feature waves), from the operand
        // fragments (the positions of two states' fragments coincide).
        auto fdot = [&](const F* a, const F* b) {
            float acc = 0.f;
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk)
#pragma unroll
                for (int s2 = 0; s2 < KS; ++s2) acc += static_cast<float>(a[kk][s2]) * static_cast<float>(b[kk][s2]);
            return acc;
        };
        float d1 = 0.f, d2 = 0.f, d3 = 0.f;
        f32x4 dQ[FPW][NT], dK[FPW][NT];
        float pa[FPW][NT], pc[FPW][NT], pwm[FPW][NT], pws[FPW][NT];
        // Partial j of the tile's token t: stored at once into its own region
        // (the four lane groups hold the same sum and store it together, no
        // branch), else kept until the residual tile is free.
        auto keep = [&](float (&arr)[FPW][NT], int ft, int tt, int j, float x) {
            if constexpr (Gm::PART_OWN) {
                part[(fw * FPW + ft) * Gm::PART + j * NP + 16 * tt + lr] = x;
            } else {
                arr[ft][tt] = x;
            }
        };
#pragma unroll
        for (int ft = 0; ft < FPW; ++ft) {
            const int f0 = 16 * (fw * FPW + ft);
            F fs[NKD], fo[NKD], fm[NKD];
            colcvt(raw, fm);                       // M0
            __builtin_amdgcn_sched_barrier(0);   // the next state's loads stay behind this point
            colload(dMe, f0, raw);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const int t = 16 * tt + lr;
                f32x4 X = {0.f, 0.f, 0.f, 0.f}, H = X;
#pragma unroll
                for (int kk = 0; kk < NKD; ++kk) {
                    X = O::mma(X, fm[kk], zfrag(sm.dz, p.dz, 1.f, t, kk * KG));
                    H = O::mma(H, fm[kk], zfrag(sm.de, p.dv, -1.f, t, kk * KG));
                }
                keep(pa, ft, tt, 0, rdot(ld4<T>(sm.q + t * LQ + f0 + 4 * lg), X));
                dQ[ft][tt] = sm.A[t] * X;
                dK[ft][tt] = H;
            }
            colcvt(raw, fo);                       // dM'
            d1 += fdot(fo, fm);
            __builtin_amdgcn_sched_barrier(0);   // the next state's loads stay behind this point
            colload(Sc, f0, raw);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const int t = 16 * tt + lr;
                f32x4 U = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < NKD; ++kk) U = O::mma(U, fo[kk], R::rm(sm.ec, LQ, t, kk * KG, lg));
                keep(pwm, ft, tt, 2, -rdot(ld4<T>(sm.k + t * LQ + f0 + 4 * lg), U));
                dK[ft][tt] -= sm.wm[t] * U;
            }
            colcvt(raw, fs);                       // S0
            d2 += fdot(fo, fs);
            __builtin_amdgcn_sched_barrier(0);   // the next state's loads stay behind this point
            colload(dSe, f0, raw);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const int t = 16 * tt + lr;
                f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < NKD; ++kk) Y = O::mma(Y, fs[kk], zfrag(sm.dz, p.dz, 1.f, t, kk * KG));
                keep(pc, ft, tt, 1, rdot(ld4<T>(sm.q + t * LQ + f0 + 4 * lg), Y));
                dQ[ft][tt] += sm.c[t] * Y;
            }
            colcvt(raw, fo);                       // dS'
            d3 += fdot(fo, fs);
            __builtin_amdgcn_sched_barrier(0);   // the next state's loads stay behind this point
            if (ft + 1 < FPW) colload(Mc, f0 + 16, raw);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const int t = 16 * tt + lr;
                f32x4 W = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < NKD; ++kk) W = O::mma(W, fo[kk], R::rm(sm.ec, LQ, t, kk * KG, lg));
                keep(pws, ft, tt, 3, -rdot(ld4<T>(sm.k + t * LQ + f0 + 4 * lg), W));
                dK[ft][tt] -= sm.ws[t] * W;
            }
        }
        d1 = wave_sum(d1);
        d2 = wave_sum(d2);
        d3 = wave_sum(d3);
        if constexpr (!Gm::PART_OWN) __syncthreads();   // (2) residual tile consumed
#pragma unroll
        for (int ft = 0; ft < FPW; ++ft) {
            float* pf = part + (fw * FPW + ft) * Gm::PART;
            if constexpr (!Gm::PART_OWN) {
                if (lg == 0) {
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) {
                        const int t = 16 * tt + lr;
                        pf[t] = pa[ft][tt];
                        pf[NP + t] = pc[ft][tt];
                        pf[2 * NP + t] = pwm[ft][tt];
                        pf[3 * NP + t] = pws[ft][tt];
                    }
                }
            }
            if (lane == 0) {
                pf[4 * NP] = ft == 0 ? d1 : 0.f;
                pf[4 * NP + 1] = ft == 0 ? d2 : 0.f;
                pf[4 * NP + 2] = ft == 0 ? d3 : 0.f;
            }
        }
        __syncthreads();   // (3); with a partial region of its own, also (2)

        // dQ -= (DL K)^T, dK -= (DL^T Q)^T  (dlt holds -DL^T).
#pragma unroll
        for (int ft = 0; ft < FPW; ++ft) {
            const int f0 = 16 * (fw * FPW + ft);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
                for (int kk = 0; kk < NKT; ++kk) {
                    dQ[ft][tt] = O::mma(dQ[ft][tt], R::cm(sm.k, LQ, kk * KG, f0, lr, lg),
                                        R::cm(sm.dlt, LPT, kk * KG, 16 * tt, lr, lg));
                    dK[ft][tt] = O::mma(dK[ft][tt], R::cm(sm.q, LQ, kk * KG, f0, lr, lg),
                                        R::rm(sm.dlt, LPT, 16 * tt + lr, kk * KG, lg));
                }
                const int t = 16 * tt + lr;
                if (t < n) {
                    *reinterpret_cast<f32x4*>(p.dq + (tok0 + t) * D + f0 + 4 * lg) = isc * dQ[ft][tt];
                    *reinterpret_cast<f32x4*>(p.dk + (tok0 + t) * D + f0 + 4 * lg) = isc * dK[ft][tt];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
// Workgroup lanes V of the persistent carry walk on the current device:
// resident workgroups (CUs x occupancy) / (8 XCD lanes x NRB row blocks),
// queried once per device and instance.
template <typename T, int D, int NS, int NP>
int carry_lanes() {
    using Gm = CarryGeo<T, D, NS, NP>;
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    std::atomic<int>& slot = cached[dev & 63];
    int v = slot.load(std::memory_order_relaxed);
    if (v > 0) return v;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, linear_memory_bwd_carry_packed<T, D, NS, NP>,
                                                     kW * Gm::NWAVE, 0) != hipSuccess || per_cu <= 0)
        per_cu = 1;
    v = bmax(1, cus * per_cu / (8 * Gm::NRB));
    slot.store(v, std::memory_order_relaxed);
    return v;
}

template <typename T, int D, int NS, int NP>
hipError_t launch_carry(const CarryParams& cp, hipStream_t s) {
    using Gm = CarryGeo<T, D, NS, NP>;
    if constexpr (Gm::PERSIST) {
        if (cp.cu) {
            // Packed documents: persistent workgroups when the documents fit the
            // in-LDS ranking and every workgroup's units fit its table.
            const int N = cp.BH / cp.H;
            const int V = bmax(1, bmin(carry_lanes<T, D, NS, NP>(), (cp.BH + 7) / 8));
            const long long kmax = (static_cast<long long>(cp.BH) + 8LL * V - 1) / (8LL * V);
            if (N <= Gm::NMAX_DOCS && kmax <= Gm::KMAX) {
                hipLaunchKernelGGL((linear_memory_bwd_carry_packed<T, D, NS, NP>), dim3(8 * Gm::NRB * V),
                                   dim3(kW * Gm::NWAVE), 0, s, cp);
                return hipGetLastError();
            }
        }
    }
    // One workgroup per (sequence or document, row block); packed documents
    // above the in-wave ranking's limit take their order from a pass before
    // the launch.
    CarryParams q = cp;
    int* perm = nullptr;
    if (cp.cu && cp.T > 0) {
        const hipError_t e = make_doc_order(cp.cu, cp.BH / cp.H, cp.T, s, &perm);
        if (e != hipSuccess) return e;
    }
    q.perm = perm;
    const long long nwg = static_cast<long long>(cp.BH) * Gm::NRB;
    hipLaunchKernelGGL((linear_memory_bwd_carry<T, D, NS, NP>), dim3(static_cast<unsigned>(nwg)),
                       dim3(kW * Gm::NWAVE), 0, s, q);
    const hipError_t err = hipGetLastError();
    if (perm) (void)hipFreeAsync(perm, s);
    return err;
}

template <typename T, int D, int NP>
hipError_t launch_grads(const GradParams& gp, hipStream_t s) {
    using Gm = GradGeo<T, D, NP>;
    const long long nwg = gp.cu ? static_cast<long long>(gp.H) * gp.tcmax : static_cast<long long>(gp.BH) * gp.nch;
    if (nwg == 0) return hipSuccess;
    hipLaunchKernelGGL((linear_memory_bwd_grads<T, D, NP>), dim3(static_cast<unsigned>(nwg)),
                       dim3(kW * Gm::NWAVE), 0, s, gp);
    return hipGetLastError();
}

template <typename T, int D, int NP>
hipError_t launch_bwd(const CarryParams& cp, const GradParams& gp, hipStream_t s) {
    constexpr int NS = D >= 32 ? 2 : 1;
    hipError_t err = launch_carry<T, D, NS, NP>(cp, s);
    if (err != hipSuccess) return err;
    return launch_grads<T, D, NP>(gp, s);
}

template <typename T, int D>
hipError_t launch_bwd_np(const CarryParams& cp, const GradParams& gp, int b, hipStream_t s) {
    if constexpr (Op<T>::KG == 32) {
        return b <= 32 ? launch_bwd<T, D, 32>(cp, gp, s) : launch_bwd<T, D, 64>(cp, gp, s);
    } else {
        if (b <= 16) return launch_bwd<T, D, 16>(cp, gp, s);
        if (b <= 32) return launch_bwd<T, D, 32>(cp, gp, s);
        return launch_bwd<T, D, 64>(cp, gp, s);
    }
}


// The bf16 entry points' work buffer: the cotangent slots (the checkpoints'
// size), then at the next 256-byte boundary kScaleParts floats per sequence
// (per document and head for packed documents).
size_t scale_offset(size_t ck_b) { return (ck_b + 255) / 256 * 256; }
size_t bwd_work_bytes_bf16(size_t ck_b, long long groups) {
    return scale_offset(ck_b) + static_cast<size_t>(groups) * kScaleParts * sizeof(float);
}

template <typename T>
int backward_impl(const void* q, const void* k, const void* v, const float* theta, const float* eta,
                  const float* alpha, const void* ckpt, const float* dz, const float* dMT, const float* dST,
                  float* dq, float* dk, float* dv, float* dth, float* deta, float* dal, float* dM0, float* dS0,
                  void* work, int B, int H, int Tlen, int d, int b, void* stream, bool chunk_gates = false,
                  const int* cu = nullptr) {
    // Dense: B sequences of T tokens per head.  Packed documents (cu set): B
    // is the document count N, the token arrays are [H, T] and the states
    // [N, H, d, d] (see the forward's packed-document entry points).
    using G = typename GlobalOf<T>::type;
    if (B < 0 || H < 0 || Tlen < 0) return TTT_ERR_INVALID_ARG;
    if (b < 1) return TTT_ERR_INVALID_ARG;
    if (d != 16 && d != 32 && d != 64 && d != 128) return TTT_ERR_UNSUPPORTED;
    if (b > 64) return TTT_ERR_UNSUPPORTED;
    const bool packed = cu != nullptr;
    if (packed && chunk_gates) return TTT_ERR_UNSUPPORTED;
    const long long BH = static_cast<long long>(B) * H;
    if (BH == 0) return TTT_OK;
    const long long nch = (static_cast<long long>(Tlen) + b - 1) / b;
    const long long tcmax = packed ? varlen_chunk_slots(B, Tlen, b) : 0;
    const long long seqs = packed ? H : BH;   // rows of Tlen tokens
    // Grids and int indices: the carry walk has BH * (d / 16) workgroups at
    // most; the gradient kernel BH * nch (dense) or H * tcmax (packed).
    if (seqs * static_cast<long long>(Tlen) > 0x7fffffffLL || BH * (d / 16) > 0x7fffffffLL ||
        (packed ? static_cast<long long>(H) * tcmax : BH * nch) > 0x7fffffffLL)
        return TTT_ERR_UNSUPPORTED;
    if (packed && !aligned(cu, 4)) return TTT_ERR_INVALID_ARG;
    const size_t tok = static_cast<size_t>(seqs) * static_cast<size_t>(Tlen);
    const size_t in_b = tok * d * sizeof(G), f_b = tok * d * 4;
    const size_t g_b = (chunk_gates ? static_cast<size_t>(BH) * static_cast<size_t>(nch) : tok) * 4;
    const size_t st_b = static_cast<size_t>(BH) * d * d * 4;
    const size_t ck_b = packed ? ckpt_bytes_varlen(B, H, Tlen, d, b, sizeof(T)) : ckpt_bytes(B, H, Tlen, d, b, sizeof(T));
    const size_t cu_b = packed ? (static_cast<size_t>(B) + 1) * sizeof(int) : 0;
    // fp16 operands: per-group power-of-two scaling of the cotangents.
    constexpr bool kScaled = !std::is_same<T, float>::value;
    const long long groups = BH;
    const size_t work_b = kScaled ? bwd_work_bytes_bf16(ck_b, groups) : ck_b;
    if (Tlen > 0) {
        const void* req[] = {q, k, v, theta, eta, alpha, ckpt, dz, dq, dk, dv, dth, deta, dal, work};
        for (const void* r : req)
            if (!r) return TTT_ERR_INVALID_ARG;
        const void* a16[] = {q, k, v, ckpt, dz, dq, dk, dv, work};
        for (const void* r : a16)
            if (!aligned(r, 16)) return TTT_ERR_INVALID_ARG;
        const void* a4[] = {theta, eta, alpha, dth, deta, dal};
        for (const void* r : a4)
            if (!aligned(r, 4)) return TTT_ERR_INVALID_ARG;
    }
    const void* st[] = {dMT, dST, dM0, dS0};
    for (const void* r : st)
        if (r && !aligned(r, 16)) return TTT_ERR_INVALID_ARG;
    // No output may overlap any input or another output.
    const Span ins[] = {{q, in_b}, {k, in_b}, {v, in_b}, {theta, g_b}, {eta, g_b}, {alpha, g_b},
                        {ckpt, ck_b}, {dz, f_b}, {dMT, st_b}, {dST, st_b}, {cu, cu_b}};
    const Span outs[] = {{dq, f_b}, {dk, f_b}, {dv, f_b}, {dth, g_b}, {deta, g_b}, {dal, g_b},
                         {dM0, st_b}, {dS0, st_b}, {work, work_b}};
    const int n_outs = static_cast<int>(sizeof(outs) / sizeof(outs[0]));
    for (int i = 0; i < n_outs; ++i) {
        if (outs[i].n == 0) continue;
        for (const Span& in : ins)
            if (in.n && overlaps(outs[i].p, outs[i].n, in.p, in.n)) return TTT_ERR_INVALID_ARG;
        for (int j = i + 1; j < n_outs; ++j)
            if (outs[j].n && overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return TTT_ERR_INVALID_ARG;
    }

    const int cg = chunk_gates ? 1 : 0;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    float* smax = nullptr;
    if (kScaled && Tlen > 0) {
        smax = reinterpret_cast<float*>(static_cast<char*>(work) + scale_offset(ck_b));
        hipLaunchKernelGGL(cot_absmax, dim3(static_cast<unsigned>(groups * kScaleParts)), dim3(256), 0, s, dz, dMT,
                           dST, smax, Tlen, d, cu, H);
        const hipError_t e0 = hipGetLastError();
        if (e0 != hipSuccess) return TTT_ERR_HIP;
    }
    const CarryParams cp{q, k, dz, theta, eta, alpha, dMT, dST, work, dv, dM0, dS0,
                         static_cast<int>(BH), Tlen, b, static_cast<int>(nch), cg, cu, H, static_cast<int>(tcmax), smax,
                         nullptr};
    const GradParams gp{q, k, v, theta, eta, alpha, ckpt, work, dz, dv, dq, dk, dth, deta, dal,
                        static_cast<int>(BH), Tlen, b, static_cast<int>(nch), cg, cu, H, static_cast<int>(tcmax), smax};
    hipError_t err;
    switch (d) {
        case 16: err = launch_bwd_np<T, 16>(cp, gp, b, s); break;
        case 32: err = launch_bwd_np<T, 32>(cp, gp, b, s); break;
        case 64: err = launch_bwd_np<T, 64>(cp, gp, b, s); break;
        default: err = launch_bwd_np<T, 128>(cp, gp, b, s); break;
    }
    return err == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

}  // namespace

extern "C" {

int ttt_mem_backward_f32(const float* q, const float* k, const float* v, const float* theta, const float* eta,
                         const float* alpha, const float* ckpt, const float* dz, const float* dM_T,
                         const float* dS_T, float* dq, float* dk, float* dv, float* dtheta, float* deta,
                         float* dalpha, float* dM0, float* dS0, float* work, int B, int H, int T, int d, int b,
                         void* stream) {
    return backward_impl<float>(q, k, v, theta, eta, alpha, ckpt, dz, dM_T, dS_T, dq, dk, dv, dtheta, deta, dalpha,
                                dM0, dS0, work, B, H, T, d, b, stream);
}

int ttt_mem_backward_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* theta,
                          const float* eta, const float* alpha, const uint16_t* ckpt, const float* dz,
                          const float* dM_T, const float* dS_T, float* dq, float* dk, float* dv, float* dtheta,
                          float* deta, float* dalpha, float* dM0, float* dS0, uint16_t* work, int B, int H, int T,
                          int d, int b, void* stream) {
    return backward_impl<_Float16>(q, k, v, theta, eta, alpha, ckpt, dz, dM_T, dS_T, dq, dk, dv, dtheta, deta,
                                   dalpha, dM0, dS0, work, B, H, T, d, b, stream);
}

size_t ttt_mem_backward_work_bytes_bf16(int B, int H, int T, int d, int b) {
    if (B < 0 || H < 0 || T < 0 || d < 1 || b < 1) return 0;
    return bwd_work_bytes_bf16(ckpt_bytes(B, H, T, d, b, 2), static_cast<long long>(B) * H);
}

size_t ttt_mem_backward_work_bytes_varlen_bf16(int N, int H, int T, int d, int b) {
    if (N < 0 || H < 0 || T < 0 || d < 1 || b < 1) return 0;
    return bwd_work_bytes_bf16(ckpt_bytes_varlen(N, H, T, d, b, 2), static_cast<long long>(N) * H);
}

int ttt_mem_backward_cg_f32(const float* q, const float* k, const float* v, const float* theta, const float* eta,
                            const float* alpha, const float* ckpt, const float* dz, const float* dM_T,
                            const float* dS_T, float* dq, float* dk, float* dv, float* dtheta, float* deta,
                            float* dalpha, float* dM0, float* dS0, float* work, int B, int H, int T, int d, int b,
                            void* stream) {
    return backward_impl<float>(q, k, v, theta, eta, alpha, ckpt, dz, dM_T, dS_T, dq, dk, dv, dtheta, deta, dalpha,
                                dM0, dS0, work, B, H, T, d, b, stream, true);
}

int ttt_mem_backward_cg_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* theta,
                             const float* eta, const float* alpha, const uint16_t* ckpt, const float* dz,
                             const float* dM_T, const float* dS_T, float* dq, float* dk, float* dv, float* dtheta,
                             float* deta, float* dalpha, float* dM0, float* dS0, uint16_t* work, int B, int H, int T,
                             int d, int b, void* stream) {
    return backward_impl<_Float16>(q, k, v, theta, eta, alpha, ckpt, dz, dM_T, dS_T, dq, dk, dv, dtheta, deta,
                                   dalpha, dM0, dS0, work, B, H, T, d, b, stream, true);
}

int ttt_mem_backward_varlen_f32(const float* q, const float* k, const float* v, const float* theta,
                                const float* eta, const float* alpha, const float* ckpt, const float* dz,
                                const float* dM_T, const float* dS_T, float* dq, float* dk, float* dv, float* dtheta,
                                float* deta, float* dalpha, float* dM0, float* dS0, float* work,
                                const int* cu_seqlens, int N, int H, int T, int d, int b, void* stream) {
    if (!cu_seqlens) return TTT_ERR_INVALID_ARG;
    return backward_impl<float>(q, k, v, theta, eta, alpha, ckpt, dz, dM_T, dS_T, dq, dk, dv, dtheta, deta, dalpha,
                                dM0, dS0, work, N, H, T, d, b, stream, false, cu_seqlens);
}

int ttt_mem_backward_varlen_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* theta,
                                 const float* eta, const float* alpha, const uint16_t* ckpt, const float* dz,
                                 const float* dM_T, const float* dS_T, float* dq, float* dk, float* dv,
                                 float* dtheta, float* deta, float* dalpha, float* dM0, float* dS0, uint16_t* work,
                                 const int* cu_seqlens, int N, int H, int T, int d, int b, void* stream) {
    if (!cu_seqlens) return TTT_ERR_INVALID_ARG;
    return backward_impl<_Float16>(q, k, v, theta, eta, alpha, ckpt, dz, dM_T, dS_T, dq, dk, dv, dtheta, deta,
                                   dalpha, dM0, dS0, work, N, H, T, d, b, stream, false, cu_seqlens);
}

}  // extern "C"
