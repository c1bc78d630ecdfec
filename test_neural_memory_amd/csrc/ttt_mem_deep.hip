// Chunked TTT deep memory (L = 2, 3 or 4 layers) forward for gfx950
// (MI355X): the hidden units of every layer are split over the workgroups of
// a group, and the groups exchange partial products through the L2 of their
// XCD once or a few times per chunk.
//
// The memory is f(u) = u + SiLU(...SiLU(u W_1)...) W_L in row-vector form
// (W_1: d x hid, W_l: hid x hid for 1 < l < L, W_L: hid x d, no biases),
// written by gradient steps on 1/2 ||f(k_t) - v_t||^2 with every gradient of
// a chunk taken at the chunk-start weights, one momentum per layer and the
// token's theta, eta, alpha for all of them ("论文速览 | Titans", sections
// 3.4, 3.7, 3.9 and 4.2; "Continual Learning: From Attention to Neural
// Memory", sections 4.2 and 5.2).  The chunk is unrolled in its dual form
// ("5.1.1 · TTT layers 与 fast weights", section 1.1, eqs. (7)-(9), carried
// through a nonlinear inner model): with keys K, values V, queries Q of the
// chunk (rows are tokens), the decay matrix L_ij = theta_j gamma_ij (j <= i),
// the gate products A_i, c_i, E_i and the chunk-end weights w^M, w^S,
//
//   keys     X_0 = K, H_l = X_{l-1} W_l, X_l = SiLU(H_l) (l < L),
//            R = K + X_{L-1} W_L - V
//   deltas   D_L = R, D_l = (D_{l+1} W_{l+1}^T) .* SiLU'(H_l)
//   reads    Y_0 = Q, Hq_l = diag(A) Y_{l-1} W_l + diag(c) Y_{l-1} S_l
//                          - (L .* Y_{l-1} X_{l-1}^T) D_l,  Y_l = SiLU(Hq_l),
//            Z = Q + Hq_L
//   carry    W_l <- A_n W_l + c_n S_l - X_{l-1}^T diag(w^M) D_l,
//            S_l <- E_n S_l - X_{l-1}^T diag(w^S) D_l
//
// Work split.  A group of G = 8 workgroups owns one (batch, head) sequence at
// a time; each workgroup has two waves and each wave owns 16 hidden units of
// every hidden layer: the columns of W_l (l < L) and the rows of W_L, with
// their momenta, in fp32 MFMA accumulators for the whole sequence.  What
// crosses waves is exchanged per chunk: R (a sum of per-wave partials of
// X_{L-1} W_L), the z partials, and for deeper memories the activations X_l,
// Y_l (gathered) and the partial products of D_l (summed).  The sixteen
// waves of a group exchange through a workspace in global memory: every
// workgroup writes its (two-wave) contribution, adds one to the group's
// counter, and waits until the counter shows all G contributions; the counter
// and the data live in the L2 of the XCD all G workgroups run on (workgroup
// ids congruent mod 8; checked at run time against the hardware XCC id), so
// the counter is polled with an atomic that executes in that L2 and the data
// is read with device-scope loads (served coherently at device scope, never
// from a line the CU's vector L1 kept), into registers where the registers
// allow, from slots that rotate through a short ring.  Every wait is bounded: a
// wait that runs out sets a status bit and the kernel finishes (with wrong
// results) instead of hanging.
//
// Precision.  MFMA operands are bf16 (v_mfma_f32_16x16x16_bf16): k, q and v
// are exact; every float32 operand (weights, momenta, activations, residuals,
// deltas) is split into bf16 hi + lo, and a product takes hi*hi + hi*lo +
// lo*hi (about 16 significant bits), accumulating in float32.  bf16 keeps
// float32's exponent range, so weights that decay far below the fp16 range
// need no scaling.

#include <cstdlib>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "ttt_mem.h"
#include "gfx950.h"

namespace {

constexpr int kD = 64;          // model width d
constexpr int kHid = 256;       // hidden width
constexpr int kNP = 16;         // padded chunk length (b <= 16)
constexpr int kG = 8;           // workgroups per group (one sequence at a time)
constexpr int kWaves = 2;       // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kDT = kD / 16;    // 16-wide tiles of d
constexpr int kHT = kHid / 16;  // 16-wide tiles of the hidden width (one per wave of a group)
constexpr int kKS = kD + 8;     // LDS row stride (bf16) of K, Q, V rows
constexpr int kRS = kD + 4;     // LDS row stride (floats) of R rows [t][d]
constexpr int kRTS = kNP + 4;   // LDS row stride (floats) of R^T rows [d][t]
constexpr int kLS = kNP + 4;    // LDS row stride (floats) of the decay matrix rows
constexpr int kWS = 16 + 4;     // LDS row stride (bf16) of a wave's staged W_L^T rows [d][h]
constexpr int kThreads2 = 256;         // deep_fwd2: two chain waves and two read waves
constexpr int kSlot = 3 * kNP * kD;   // floats per workgroup slot and exchange step: R, then the two read waves' z partials
// Exchange slots form a ring of steps per group.  A workgroup reads the
// slots of step e after the group counter shows every workgroup's signal of
// e, and its own signal of e + 1 follows the completion of those reads.  So
// once the counter shows step e + 1, nobody reads step e - 1 any more:
// deep_fwd3/4, which write the slot of step e + 1 only after that, need two
// steps; deep_fwd2 writes a z partial into the slot of step e + 2 before its
// wait for e + 1 and needs three.  The smaller the ring, the less of the XCD's
// L2 it takes from the hidden layers' weights and from the data streamed
// through it (lines evicted dirty are written back to HBM).
constexpr int kRing = 3;    // deep_fwd2
constexpr int kRingM = 2;   // deep_fwd3, deep_fwd4
// Cache policy of the slot copies: SC1 (device scope), so a copy is served
// coherently at device scope -- never from a line the CU's vector L1 kept from
// an earlier step -- and no L1 invalidation is needed.
constexpr int kSlotLoadPolicy = 16;
// Four floats at float offset `off` of a slot range, loaded with that policy.
__device__ __forceinline__ f32x4 slot_load(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off * 4, 0, kSlotLoadPolicy));
}
constexpr int kCtrStride = 64;        // ints between group counters (256 bytes)
constexpr int kHdrInts = 1024;        // status word, XCD ticket counters and padding before the group counters
constexpr int kTicketInts = 64;       // first XCD ticket counter (one per XCD, kCtrStride apart)
constexpr uint32_t kStatusTimeout = 1u, kStatusPlacement = 2u;

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// x = hi + lo, both bf16 (round to nearest even); together about 16 bits.
struct Sp {
    s16x4 hi, lo;
};
__device__ __forceinline__ s16x4 pack4(f32x4 v) { return __builtin_bit_cast(s16x4, pack_bf16x4(v)); }
__device__ __forceinline__ f32x4 unpack4(s16x4 h) {
    const u32x2 w = __builtin_bit_cast(u32x2, h);
    return f32x4{bf16lo(w[0]), bf16hi(w[0]), bf16lo(w[1]), bf16hi(w[1])};
}
__device__ __forceinline__ Sp split(f32x4 x) {
    const s16x4 hi = pack4(x);
    return Sp{hi, pack4(x - unpack4(hi))};
}
// Products of split operands, dropping lo * lo; with an exact bf16 operand.
__device__ __forceinline__ f32x4 mma3(const Sp& a, const Sp& b, f32x4 c) {
    c = mma(a.hi, b.hi, c);
    c = mma(a.hi, b.lo, c);
    return mma(a.lo, b.hi, c);
}
__device__ __forceinline__ f32x4 mma2(s16x4 a, const Sp& b, f32x4 c) { return mma(a, b.lo, mma(a, b.hi, c)); }
__device__ __forceinline__ f32x4 mma2(const Sp& a, s16x4 b, f32x4 c) { return mma(a.lo, b, mma(a.hi, b, c)); }

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
__device__ __forceinline__ void silu_d4(f32x4 x, f32x4& y, f32x4& dy) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float s = sigm(x[e]);
        y[e] = x[e] * s;
        dy[e] = s * (1.f + x[e] * (1.f - s));
    }
}

__device__ __forceinline__ int xcc_id() { return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xf; }

// Poll the group counter with an atomic add of 0 that returns the value; the
// atomic executes in the L2, where the other workgroups' increments are.  The
// wait for the result is in the same asm block.
__device__ __forceinline__ int l2_counter(int* p) {
    int c, zero = 0;
    asm volatile("global_atomic_add %0, %1, %2, off sc0\n\ts_waitcnt vmcnt(0)" : "=v"(c) : "v"(p), "v"(zero) : "memory");
    return c;
}

struct DeepParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* theta;
    const float* eta;
    const float* alpha;
    // Layer l (0-based) of sequence s: W0[l] + s * wstride[l] (row-major).
    const float* W0[4];
    const float* S0[4];
    float* WT[4];
    float* ST[4];
    long long wstride[4];
    void* z;         // float32, or bf16 bits (rounded to nearest even) when z_bf16
    int z_bf16;
    int BH;
    int T;
    int b;
    int ngroups;
    int nxcc;        // XCCs of the device (workgroup b is expected on XCC b % nxcc)
    int spin_limit;  // polls before a wait gives up
    int* work;       // [kHdrInts status][ngroups counters][exchange slots]
};

// One chunk of staged inputs and its gate quantities (double-buffered).
struct ChunkBuf {
    alignas(16) uint16_t kb[kNP * kKS];   // K rows [t][d], bf16
    alignas(16) uint16_t qb[kNP * kKS];   // Q rows
    alignas(16) uint16_t vb[kNP * kKS];   // V rows
    alignas(16) float L[kNP * kLS];       // theta_j gamma_ij, row i, column j (0 above the diagonal)
    alignas(16) float A[kNP];
    alignas(16) float C[kNP];
    alignas(16) float wm[kNP];            // -theta_j gamma_{n-1,j}
    alignas(16) float ws[kNP];            // -theta_j p_{n-1,j}
    alignas(16) float scal[4];            // A_n, c_n, E_n
};

struct DeepSmem {
    ChunkBuf buf[2];
    alignas(16) float R[kNP * kRS];              // R rows [t][d]
    alignas(16) float RT[2][kD * kRTS];          // R^T rows [d][t], by chunk parity (the read waves lag a chunk)
    alignas(16) uint16_t wst[kWaves][2][kD * kWS];   // per chain wave: its W_L rows staged as [d][h], hi and lo
    alignas(16) f32x4 xpart[kWaves][2][64];      // partner tiles for the two-wave pre-reduction of R
    // Per chain wave, for the read wave of the same units: SiLU(Hk)^T (bf16
    // hi / lo) and SiLU(Hk) (float32, K layout) by chunk parity, and dH
    // (float32, K layout) of the last chunk.
    struct {
        s16x4 akt[2][2][64];
        f32x4 ak[2][64];
        f32x4 dh[64];
    } act[kWaves];
    int bail, gid, part;
};

// Registers of one prefetched chunk: thread u (0..127) holds one 16-byte unit
// of K, Q and V each (token u / 8, columns 8 (u % 8)..+7); lanes < 16 of wave
// 1 the chunk's gates.
struct Prefetch {
    uint4 k, q, v;
    float th, et, al;
};

__device__ void prefetch(Prefetch& pf, const DeepParams& p, size_t seq_tok, int c, int tid) {
    const int c0 = c * p.b;
    const int n = max(0, min(p.b, p.T - c0));
    const uint32_t nbytes = static_cast<uint32_t>(n) * kD * 2;
    const size_t off = (seq_tok + static_cast<size_t>(c0)) * kD;
    const uint32_t boff = static_cast<uint32_t>((tid >> 3) * kD + 8 * (tid & 7)) * 2;
    pf.k = buf_load16(make_rsrc(p.k + off, nbytes), boff);
    pf.q = buf_load16(make_rsrc(p.q + off, nbytes), boff);
    pf.v = buf_load16(make_rsrc(p.v + off, nbytes), boff);
    if (tid >= 64) {
        const int lane = tid - 64;
        const uint32_t gbytes = static_cast<uint32_t>(n) * 4;
        const size_t gi = seq_tok + static_cast<size_t>(c0);
        pf.th = buf_load4(make_rsrc(p.theta + gi, gbytes), lane * 4);
        pf.al = buf_load4(make_rsrc(p.alpha + gi, gbytes), lane * 4);
        pf.et = buf_load4(make_rsrc(p.eta + gi, gbytes), lane * 4);
    }
}

__device__ void stage(const Prefetch& pf, ChunkBuf& B, int tid) {
    const int t = tid >> 3, col = 8 * (tid & 7);
    *reinterpret_cast<uint4*>(B.kb + t * kKS + col) = pf.k;
    *reinterpret_cast<uint4*>(B.qb + t * kKS + col) = pf.q;
    *reinterpret_cast<uint4*>(B.vb + t * kKS + col) = pf.v;
}

// row_newbcast:N -- every lane of a 16-lane row receives lane N of that row.
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + N, 0xf, 0xf, false));
}

// Gate quantities of one chunk, lanes j < 16 of one wave (token j): A_j, c_j
// by a DPP scan of the 2x2 maps [[a, eta], [0, eta]] (a = 1 - alpha), column j
// of the decay matrix by its recurrence p <- eta_i p + [i = j], gamma <- a_i
// gamma + p (zero above the diagonal; a_i, eta_i broadcast from lane i), and
// the chunk-end weights.  Padding tokens read theta = alpha = 0 and take
// eta = 1.  Only products and sums: eta = 0 and alpha = 1 are exact.
__device__ void gates(const Prefetch& pf, ChunkBuf& B, int n, int lane) {
    const int j = lane & 15;
    const float a = 1.f - pf.al, e = lane < n ? pf.et : 1.f, th = pf.th;
    float X = a, Y = e, W = e;   // -> A_j, c_j, E_j
    tri_step<kRowShr1>(X, Y, W);
    tri_step<kRowShr2>(X, Y, W);
    tri_step<kRowShr4>(X, Y, W);
    tri_step<kRowShr8>(X, Y, W);
    float ai[kNP], ei[kNP];
    ai[0] = row_bcast<0>(a); ei[0] = row_bcast<0>(e);
    ai[1] = row_bcast<1>(a); ei[1] = row_bcast<1>(e);
    ai[2] = row_bcast<2>(a); ei[2] = row_bcast<2>(e);
    ai[3] = row_bcast<3>(a); ei[3] = row_bcast<3>(e);
    ai[4] = row_bcast<4>(a); ei[4] = row_bcast<4>(e);
    ai[5] = row_bcast<5>(a); ei[5] = row_bcast<5>(e);
    ai[6] = row_bcast<6>(a); ei[6] = row_bcast<6>(e);
    ai[7] = row_bcast<7>(a); ei[7] = row_bcast<7>(e);
    ai[8] = row_bcast<8>(a); ei[8] = row_bcast<8>(e);
    ai[9] = row_bcast<9>(a); ei[9] = row_bcast<9>(e);
    ai[10] = row_bcast<10>(a); ei[10] = row_bcast<10>(e);
    ai[11] = row_bcast<11>(a); ei[11] = row_bcast<11>(e);
    ai[12] = row_bcast<12>(a); ei[12] = row_bcast<12>(e);
    ai[13] = row_bcast<13>(a); ei[13] = row_bcast<13>(e);
    ai[14] = row_bcast<14>(a); ei[14] = row_bcast<14>(e);
    ai[15] = row_bcast<15>(a); ei[15] = row_bcast<15>(e);
    float g = 0.f, pe = 0.f, wm = 0.f, ws = 0.f;
#pragma unroll
    for (int i = 0; i < kNP; ++i) {
        pe = i == j ? 1.f : ei[i] * pe;
        g = ai[i] * g + pe;
        if (lane < kNP) B.L[i * kLS + j] = th * g;
        if (i == n - 1) {
            wm = th * g;
            ws = th * pe;
        }
    }
    if (lane < kNP) {
        B.A[j] = X;
        B.C[j] = Y;
        B.wm[j] = -wm;
        B.ws[j] = -ws;
        if (lane == n - 1) {
            B.scal[0] = X;
            B.scal[1] = Y;
            B.scal[2] = W;
        }
    }
}

// 4 bf16 of an LDS row (8 bytes).
__device__ __forceinline__ s16x4 lds4(const uint16_t* p) { return *reinterpret_cast<const s16x4*>(p); }
// Transpose load: with row pointer base (row stride rs elements), lane L of
// 16-lane group g reads row 4g + L/4 at columns 4 (L % 4)..+3; lane i then
// holds column i of rows 4g..4g+3.
__device__ __forceinline__ s16x4 lds_tr4(const uint16_t* base, int rs, int lr, int lg) {
    return ds_read_tr16(base + (4 * lg + (lr >> 2)) * rs + 4 * (lr & 3));
}

// Two-layer deep memory.  Waves 0 and 1 (the chain waves) carry the
// dependent work of a chunk: keys, the R exchange, dH and the carry of the
// weights.  Waves 2 and 3 (the read waves, units of waves 0 and 1) read the
// previous chunk -- Hq, Aq and the z partial -- from their own copy of the
// weights one chunk behind, which they keep by applying the same carry to the
// same float32 inputs (so both copies hold identical values), sum the z of the
// chunk before and compute the gate quantities of the chunk the chain waves
// carry next.  Per chunk step the five barriers below are shared by all four
// waves; the read waves' work fills the chain's segments instead of
// lengthening them.
__global__ __launch_bounds__(kThreads2, 1) void deep_fwd2(const DeepParams p) {
    __shared__ DeepSmem sm;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool chain = w < 2;
    const int wp = w & 1;            // the chain wave whose units this wave holds
    const int lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    int* const status = p.work;

    // Group and part from the XCD the workgroup actually runs on: a ticket
    // from that XCD's counter (an atomic in its L2) numbers the workgroups
    // of the XCD; G consecutive tickets form a group.  The grid is a
    // multiple of 8 G, so round-robin dispatch gives every XCD whole groups;
    // a workgroup past its XCD's share flags the status and leaves.
    if (tid == 0) {
        const int x = xcc_id() % p.nxcc;
        const int t = __hip_atomic_fetch_add(p.work + kTicketInts + x * kCtrStride, 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        const int per_xcd = p.ngroups / p.nxcc;
        sm.bail = t >= per_xcd * kG ? 1 : 0;
        if (sm.bail)
            __hip_atomic_fetch_or(status, static_cast<int>(kStatusPlacement), __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_SYSTEM);
        sm.gid = x + p.nxcc * (t / kG);
        sm.part = t % kG;
    }
    __syncthreads();
    if (sm.bail) return;
    const int gi = __builtin_amdgcn_readfirstlane(sm.gid);
    const int part = __builtin_amdgcn_readfirstlane(sm.part);
    int* const ctr = p.work + kHdrInts + gi * kCtrStride;
    float* const xbase = reinterpret_cast<float*>(p.work + kHdrInts + p.ngroups * kCtrStride) +
                         static_cast<size_t>(gi) * kRing * kG * kSlot;
    const int hu = 32 * part + 16 * wp;   // first hidden unit of this wave
    int epoch = 0;                        // exchanges of this group so far

    // Group exchange in two halves: signal() after this workgroup's
    // contribution is written; wait() until all G have signalled.  Every
    // wave first waits until its own stores have completed (a completed store
    // sits in the L2 that the whole group shares), so the counter can only
    // show this workgroup once its slot data is there for the other
    // workgroups' device-scope copies.
    auto signal = [&]() {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __syncthreads();
        if (tid == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    // Only the chain waves, which read the slots, wait: lane 0 of each polls,
    // and the wave goes on when it returns (3.5 % faster than one poller and
    // a workgroup barrier; the deeper kernels, whose waves all read slots,
    // gain nothing from it).  The read waves' next work does not depend on
    // the exchange; a timeout is seen by every wave after the next workgroup
    // barrier (sm.bail).
    auto wait = [&]() {
        if (chain && lane == 0) {
            const int target = kG * (epoch + 1);
            int spins = 0;
            while (l2_counter(ctr) < target) {
                if (++spins > p.spin_limit) {
                    sm.bail = 1;
                    __hip_atomic_fetch_or(status, static_cast<int>(kStatusTimeout), __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_SYSTEM);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        ++epoch;
    };

    for (int s = gi; s < p.BH; s += p.ngroups) {
        const size_t seq_tok = static_cast<size_t>(s) * p.T;
        const int nch = (p.T + p.b - 1) / p.b;
        auto chunk_n = [&](int c) { return min(p.b, p.T - c * p.b); };

        // ---- weights: W1[dt] = W_1[16dt.., hu..] as [d][h]; W2[dt] = W_L[hu.., 16dt..] as [h][d] ----
        // (every wave: the chain waves' copy is current, the read waves' one chunk behind)
        f32x4 W1[kDT], S1[kDT], W2[kDT], S2[kDT];
        {
            const float* w1 = p.W0[0] + s * p.wstride[0];
            const float* s1 = p.S0[0] ? p.S0[0] + s * p.wstride[0] : nullptr;
            const float* w2 = p.W0[1] + s * p.wstride[1];
            const float* s2 = p.S0[1] ? p.S0[1] + s * p.wstride[1] : nullptr;
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i1 = (16 * dt + 4 * lg + e) * kHid + hu + lr;
                    const int i2 = (hu + 4 * lg + e) * kD + 16 * dt + lr;
                    W1[dt][e] = w1[i1];
                    S1[dt][e] = s1 ? s1[i1] : 0.f;
                    W2[dt][e] = w2[i2];
                    S2[dt][e] = s2 ? s2[i2] : 0.f;
                }
        }
        // Chain waves: W_L rows split into bf16 hi / lo (W2s, reused by the
        // products of the next chunk) and staged as [d][h] (for the
        // transposed operand of R W_L^T).
        Sp W2s[kDT];
        auto stage_w2 = [&]() {
            uint16_t* hi = sm.wst[wp][0];
            uint16_t* lo = sm.wst[wp][1];
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt) {
                W2s[dt] = split(W2[dt]);
                *reinterpret_cast<s16x4*>(hi + (16 * dt + lr) * kWS + 4 * lg) = W2s[dt].hi;
                *reinterpret_cast<s16x4*>(lo + (16 * dt + lr) * kWS + 4 * lg) = W2s[dt].lo;
            }
        };
        // The carry of one chunk (buffer Bc) from dH, SiLU(Hk) (K layout) and
        // R^T: the chain waves apply it to their weights, the read waves (a
        // chunk later) to theirs, from the same float32 values.
        auto carry = [&](const ChunkBuf& Bc, f32x4 dH, f32x4 Ak, const float* RTc) {
            const float An = Bc.scal[0], Cn = Bc.scal[1], En = Bc.scal[2];
            const f32x4 wm4 = *reinterpret_cast<const f32x4*>(Bc.wm + 4 * lg);
            const f32x4 ws4 = *reinterpret_cast<const f32x4*>(Bc.ws + 4 * lg);
            const Sp dm = split(dH * wm4), dsv = split(dH * ws4);   // B = (w .* dH)[t][h]
            // A = (Ak diag(w))^T[h][t]: the token weights ride on Ak.
            const Sp akm = split(Ak * wm4), aks = split(Ak * ws4);
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt) {
                const s16x4 kt = lds_tr4(Bc.kb + 16 * dt, kKS, lr, lg);   // A = K^T[d][t]
                const f32x4 w1 = An * W1[dt] + Cn * S1[dt];
                S1[dt] = mma2(kt, dsv, En * S1[dt]);
                W1[dt] = mma2(kt, dm, w1);
                // R[4lg..4lg+3][16dt + lr]: B = R[t][d] of the W_L carry.
                const Sp rs = split(*reinterpret_cast<const f32x4*>(RTc + (16 * dt + lr) * kRTS + 4 * lg));
                const f32x4 w2 = An * W2[dt] + Cn * S2[dt];
                S2[dt] = mma3(aks, rs, En * S2[dt]);
                W2[dt] = mma3(akm, rs, w2);
            }
        };
        if (chain) stage_w2();

        Prefetch pf;
        if (chain) prefetch(pf, p, seq_tok, 0, tid);
        __syncthreads();   // the previous sequence's last use of the chunk buffers
        if (chain && nch > 0) {
            stage(pf, sm.buf[0], tid);
            if (w == 1) gates(pf, sm.buf[0], chunk_n(0), lane);
        }
        __syncthreads();

        // Step c: the chain waves run chunk c (keys, exchange, dH, carry); the
        // read waves read chunk c - 1 and put its z partial in the slot of the
        // next step; after this step's exchange the z of chunk c - 2 is summed.
        // Two more steps finish the z of the last chunks.
        bool ok = true;
        const int iters = nch > 0 ? nch + 2 : 0;
        for (int c = 0; c < iters; ++c) {
            const bool keys = c < nch;
            const bool reads = c >= 1 && c <= nch;    // read waves: chunk c - 1
            const bool zout = c >= 2;                 // the z of chunk c - 2 leaves with this step
            ChunkBuf& B = sm.buf[c & 1];
            const ChunkBuf& Bp = sm.buf[(c + 1) & 1];  // chunk c - 1
            const float* RTp = sm.RT[(c + 1) & 1];
            const int n = keys ? chunk_n(c) : 0;
            Prefetch graw;   // read wave 0: raw gates of chunk c + 1
            float* slot = xbase + static_cast<size_t>((epoch % kRing) * kG + part) * kSlot;
            float* nslot = xbase + static_cast<size_t>(((epoch + 1) % kRing) * kG + part) * kSlot;

            // ================= segment 1: keys of chunk c | reads of chunk c - 1 =================
            f32x4 Ak = {0.f, 0.f, 0.f, 0.f}, dAk = Ak, rp[kDT];
            Sp aq{}, lgm{};
            float At = 0.f, Ct = 0.f;
            if (chain) {
                if (keys && c + 1 < nch) prefetch(pf, p, seq_tok, c + 1, tid);
                if (keys) {
                    f32x4 hk = {0.f, 0.f, 0.f, 0.f}, hkt = hk;
#pragma unroll
                    for (int dt = 0; dt < kDT; ++dt) {
                        const s16x4 kf = lds4(B.kb + lr * kKS + 16 * dt + 4 * lg);
                        const Sp w1s = split(W1[dt]);
                        hk = mma2(kf, w1s, hk);      // (K W_1)[t][h]
                        hkt = mma2(w1s, kf, hkt);    // (K W_1)^T[h][t]
                    }
                    silu_d4(hk, Ak, dAk);
                    const Sp akt = split(silu4(hkt));   // Ak^T[h][t]
                    sm.act[w].akt[c & 1][0][lane] = akt.hi;
                    sm.act[w].akt[c & 1][1][lane] = akt.lo;
                    sm.act[w].ak[c & 1][lane] = Ak;
                    // Partial R^T[d][t] over this wave's hidden units; two-wave pre-reduction.
#pragma unroll
                    for (int dt = 0; dt < kDT; ++dt) rp[dt] = mma3(W2s[dt], akt, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int k2 = 0; k2 < 2; ++k2) sm.xpart[1 - w][k2][lane] = w == 0 ? rp[2 + k2] : rp[k2];
                }
            } else if (reads) {
                At = Bp.A[lr];
                Ct = Bp.C[lr];
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(Bp.L + lr * kLS + 4 * lg);   // L[t][4lg..]
                f32x4 kq = {0.f, 0.f, 0.f, 0.f}, za = kq, zc = kq;
#pragma unroll
                for (int dt = 0; dt < kDT; ++dt) {
                    const s16x4 kf = lds4(Bp.kb + lr * kKS + 16 * dt + 4 * lg);
                    const s16x4 qf = lds4(Bp.qb + lr * kKS + 16 * dt + 4 * lg);
                    kq = mma(kf, qf, kq);                  // (K Q^T)[j][t]
                    za = mma2(split(W1[dt]), qf, za);     // (W_1^T Q^T)[h][t]
                    zc = mma2(split(S1[dt]), qf, zc);
                }
                const Sp pt = split(kq * l4);             // P^T[j][t] = (L .* Q K^T)[t][j]
                f32x4 hq = mma3(split(sm.act[wp].dh[lane]), pt, f32x4{0.f, 0.f, 0.f, 0.f});   // (dH^T P^T)[h][t]
                hq = At * za + Ct * zc - hq;
                aq = split(silu4(hq));                   // Aq^T[h][t]
                const Sp akt{sm.act[wp].akt[(c + 1) & 1][0][lane], sm.act[wp].akt[(c + 1) & 1][1][lane]};
                // (Ak Aq^T)[j][t] over this wave's hidden units, times L.
                lgm = split(mma3(akt, aq, f32x4{0.f, 0.f, 0.f, 0.f}) * l4);
            }
            __syncthreads();

            // ================= segment 2: R partial to the slot; signal =================
            if (chain && keys) {
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) {
                    const int dt = 2 * w + k2;
                    const f32x4 r = (w == 0 ? rp[k2] : rp[2 + k2]) + sm.xpart[w][k2][lane];
                    // lane (t = lr, lg) holds R^T[16dt + 4lg + e][t] = R[t][16dt + 4lg + e]
                    *reinterpret_cast<f32x4*>(slot + lr * kD + 16 * dt + 4 * lg) = r;
                }
            }
            signal();

            // ================= segment 3 (the wait): z partial of chunk c - 1 =================
            if (!chain && reads) {
                // z = q + the sum of the partials: read wave 0 of workgroup 0 adds q.
                float* zs = nslot + kNP * kD * (1 + wp) + lr * kD + 4 * lg;
#pragma unroll
                for (int dt = 0; dt < kDT; ++dt) {
                    const f32x4 a2 = mma3(split(W2[dt]), aq, f32x4{0.f, 0.f, 0.f, 0.f});
                    const f32x4 c2 = mma3(split(S2[dt]), aq, f32x4{0.f, 0.f, 0.f, 0.f});
                    const Sp rs = split(*reinterpret_cast<const f32x4*>(RTp + (16 * dt + lr) * kRTS + 4 * lg));
                    const f32x4 in = mma3(rs, lgm, f32x4{0.f, 0.f, 0.f, 0.f});   // (R^T (L .* G)^T)[d][t]
                    f32x4 zp = At * a2 + Ct * c2 - in;
                    if (part == 0 && wp == 0) zp += unpack4(lds4(Bp.qb + lr * kKS + 16 * dt + 4 * lg));
                    *reinterpret_cast<f32x4*>(zs + 16 * dt) = zp;
                }
            }
            wait();
            const float* rslot = xbase + static_cast<size_t>(((epoch - 1) % kRing) * kG) * kSlot;

            // ================= segment 4: partials in, R | the read waves' carry =================
            const bool zred = zout && part < kDT && w == 3;
            if (chain) {
                // The partials straight into registers (device-scope loads, all
                // in flight at once), summed in slot order.  Global-to-LDS
                // copies of the same tiles measured 1.84 against 1.60 ms per
                // launch: each lane needs only its own 16 bytes back.
                const auto rsl = make_rsrc(rslot, static_cast<uint32_t>(kG * kSlot * 4));
                f32x4 rpart[2][kG];
                if (keys) {
#pragma unroll
                    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
                        for (int g2 = 0; g2 < kG; ++g2)
                            rpart[k2][g2] = slot_load(rsl, g2 * kSlot + lr * kD + 16 * (2 * w + k2) + 4 * lg);
                }
                // R = K - V + sum of partials (rows [t][d] and R^T [d][t] of this chunk's parity).
                if (keys) {
                    float* RTc = sm.RT[c & 1];
#pragma unroll
                    for (int k2 = 0; k2 < 2; ++k2) {
                        const int dt = 2 * w + k2;
                        f32x4 r = unpack4(lds4(B.kb + lr * kKS + 16 * dt + 4 * lg)) - unpack4(lds4(B.vb + lr * kKS + 16 * dt + 4 * lg));
#pragma unroll
                        for (int g2 = 0; g2 < kG; ++g2) r += rpart[k2][g2];
                        if (lr >= n) r = f32x4{0.f, 0.f, 0.f, 0.f};   // padding tokens carry no residual
                        *reinterpret_cast<f32x4*>(sm.R + lr * kRS + 16 * dt + 4 * lg) = r;
#pragma unroll
                        for (int e = 0; e < 4; ++e) RTc[(16 * dt + 4 * lg + e) * kRTS + lr] = r[e];
                    }
                }
            } else {
                // Raw gates of chunk c + 1 into registers, for the gate pass of
                // read wave 0 in segment 5.
                if (w == 2 && keys && c + 1 < nch) {
                    const int n1 = chunk_n(c + 1);
                    const size_t gi = seq_tok + static_cast<size_t>(c + 1) * p.b;
                    const uint32_t gbytes = static_cast<uint32_t>(n1) * 4;
                    graw.th = buf_load4(make_rsrc(p.theta + gi, gbytes), lane * 4);
                    graw.al = buf_load4(make_rsrc(p.alpha + gi, gbytes), lane * 4);
                    graw.et = buf_load4(make_rsrc(p.eta + gi, gbytes), lane * 4);
                }
                // The carry of chunk c - 1 on the read waves' weights (needed
                // only while a later chunk remains to be read).
                if (reads && c < nch) carry(Bp, sm.act[wp].dh[lane], sm.act[wp].ak[(c + 1) & 1][lane], RTp);
            }
            __syncthreads();
            if (sm.bail) {
                ok = false;
                break;
            }
            // z of chunk c - 2 on read wave 1 (four workgroups, one d tile
            // each), while the chain waves run segment 5: the sum of the two
            // read waves' partials of every workgroup, in slot order (on chain
            // wave 0 it lengthened segment 4).
            if (zred) {
                const auto rsl = make_rsrc(rslot, static_cast<uint32_t>(kG * kSlot * 4));
                f32x4 zpart[2 * kG];
#pragma unroll
                for (int g2 = 0; g2 < kG; ++g2)
#pragma unroll
                    for (int r2 = 0; r2 < 2; ++r2)
                        zpart[2 * g2 + r2] = slot_load(rsl, g2 * kSlot + kNP * kD * (1 + r2) + lr * kD + 16 * part + 4 * lg);
                const int np = chunk_n(c - 2);
                f32x4 zt = zpart[0];
#pragma unroll
                for (int g2 = 1; g2 < 2 * kG; ++g2) zt += zpart[g2];
                const bool zb = p.z_bf16 != 0;
                const uint32_t zsz = zb ? 2u : 4u;
                const auto rz = make_rsrc(static_cast<char*>(p.z) + (seq_tok + static_cast<size_t>(c - 2) * p.b) * kD * zsz,
                                          static_cast<uint32_t>(np) * kD * zsz);
                store_out4(zt, rz, static_cast<uint32_t>(lr * kD + 16 * part + 4 * lg), zb);
            }
            if (!keys) continue;

            // ================= segment 5: dH and the carry of chunk c | z of chunk c - 2, gates of chunk c + 1 =================
            if (chain) {
                f32x4 dH = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int dt = 0; dt < kDT; ++dt) {
                    const Sp rf = split(*reinterpret_cast<const f32x4*>(sm.R + lr * kRS + 16 * dt + 4 * lg));
                    const Sp wt{lds_tr4(sm.wst[w][0] + 16 * dt * kWS, kWS, lr, lg), lds_tr4(sm.wst[w][1] + 16 * dt * kWS, kWS, lr, lg)};
                    dH = mma3(rf, wt, dH);   // [t][h]
                }
                dH *= dAk;
                sm.act[w].dh[lane] = dH;
                carry(B, dH, Ak, sm.RT[c & 1]);
                stage_w2();
                if (c + 1 < nch) {
                    ChunkBuf& Bn = sm.buf[(c + 1) & 1];
                    stage(pf, Bn, tid);
                }
            } else if (w == 2 && c + 1 < nch) {
                // Gate quantities of chunk c + 1, for the chain's carry in the
                // next step.  In segment 4 this pass made read wave 0 the
                // longest wave there; with it and the z sum moved here a launch
                // of 32 sequences x 4096 tokens takes 1.47-1.48 ms, not 1.58.
                gates(graw, sm.buf[(c + 1) & 1], chunk_n(c + 1), lane);
            }
            __syncthreads();
        }
        if (!ok) break;

        // ---- final weights (the chain waves' copy) ----
        if (chain) {
            float* w1 = p.WT[0] ? p.WT[0] + s * p.wstride[0] : nullptr;
            float* s1 = p.ST[0] ? p.ST[0] + s * p.wstride[0] : nullptr;
            float* w2 = p.WT[1] ? p.WT[1] + s * p.wstride[1] : nullptr;
            float* s2 = p.ST[1] ? p.ST[1] + s * p.wstride[1] : nullptr;
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i1 = (16 * dt + 4 * lg + e) * kHid + hu + lr;
                    const int i2 = (hu + 4 * lg + e) * kD + 16 * dt + lr;
                    if (w1) w1[i1] = W1[dt][e];
                    if (s1) s1[i1] = S1[dt][e];
                    if (w2) w2[i2] = W2[dt][e];
                    if (s2) s2[i2] = S2[dt][e];
                }
        }
    }
}

// ---------------------------------------------------------------------------
// Deeper memories: L = NM + 2 layers, NM hidden-to-hidden layers W_j
// (2 <= j <= L - 1, hid x hid).  The same group of G workgroups and the same
// exchange as deep_fwd2, with every crossing of the hidden units of a layer
// made explicit: each wave owns the columns of W_j for its 16 units of layer
// j (all hid rows, in registers) and the matching 16 x 16 tiles of its
// momentum (in the workspace, read and written only by the owning lanes).
// Per chunk, in order:
//   keys     X_1[:, U] = SiLU(K W_1[:, U]); for j = 2 .. L-1 gather X_{j-1}
//            (every wave's 16 columns to every workgroup) and form
//            X_j[:, U] = SiLU(X_{j-1} W_j[:, U]); the partial products
//            X_{L-1}[:, U] W_L[U, :] are summed into R (with the z partials
//            of the previous chunk) as in deep_fwd2.
//   deltas   D_{L-1}[:, U] = (R W_L[U, :]^T) .* SiLU'(H_{L-1}); for j = L-1
//            .. 2 the partial products D_j[:, U] W_j[:, U]^T over this
//            wave's units are summed across the group and every wave keeps
//            its own columns: D_{j-1}[:, U] = (sum) .* SiLU'(H_{j-1}).
//   reads    Y_1 as in deep_fwd2 from the chunk-start W_1, S_1; for j = 2 ..
//            L-1 gather Y_{j-1} and form Y_j[:, U] from W_j, S_j, D_j and
//            the decayed Gram (L .* Y_{j-1} X_{j-1}^T); the z partial from
//            Y_{L-1}[:, U], W_L[U, :], S_L[U, :], R.
//   carry    every layer at once, from the chunk-start weights.
// That is 3 L - 5 exchanges per chunk (the reads are not moved into a wait
// as in deep_fwd2: a stash of chunk-start hidden-to-hidden weights would not
// fit in LDS).
constexpr int kSlotM = kHT * 256;   // floats per workgroup slot: 16 delta partial tiles
constexpr int kBlk = 256;           // bf16 per plane of a 16 x 16 activation block

template <int NM>
struct MidSmem {
    // Gathered activations first (the unrolled tile loops address them with
    // immediate offsets from one base): block kt (units 16 kt .. 16 kt + 15)
    // as [hi | lo][token][unit] bf16.
    alignas(16) uint16_t xg[NM][kHT][2][kBlk];   // X_1 .. X_NM of the keys
    alignas(16) uint16_t yg[kHT][2][kBlk];       // Y_{j-1} of the queries, one layer at a time
    alignas(16) float scr[kWaves][16 * 17];       // per-wave 16 x 16 transposes
    alignas(16) uint16_t wtr[kWaves][8][2][16 * kWS];   // per-wave transposes of 8 weight tiles (hi, lo)
    ChunkBuf buf[2];
    alignas(16) float R[kNP * kRS];
    alignas(16) float RT[kD * kRTS];
    alignas(16) uint16_t wst[kWaves][2][kD * kWS];
    alignas(16) f32x4 xpart[kWaves][2][64];
    union {
        // This wave's two R tiles from every workgroup, copied from the slots
        // straight into LDS (at depth 4 the kernel has no registers to spare
        // for them).
        f32x4 dma[kWaves][2 * kG][64];
        f32x4 pred[kWaves][8][64];       // two-wave pre-reduction of delta partials
    } u;
    alignas(16) f32x4 dmaz[kG][64];      // the z tiles of the reducing workgroups
    int bail, gid, part;
};

__device__ __forceinline__ void wave_lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// f(std::integral_constant<int, I>{}) for I = B, B + S, ... while I != E:
// loops over layers whose index must be a compile-time constant (the
// resident weight arrays are indexed by it).
template <int B, int E, int S, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B != E) {
        f(std::integral_constant<int, B>{});
        static_for<B + S, E, S>(f);
    }
}

// The value itself, opaque to the compiler: a split of a resident weight tile
// is then recomputed where it is used instead of being kept live from an
// earlier use (which costs 4 registers per tile across the whole chunk).
__device__ __forceinline__ f32x4 fresh(f32x4 x) {
    asm volatile("" : "+v"(x));
    return x;
}

// 16 x 16 tile between the two accumulator layouts: lane (lr, lg) holds
// x[e] = M[4 lg + e][lr] and receives M[lr][4 lg + e] (wave-local scratch).
__device__ __forceinline__ f32x4 tr16(f32x4 x, float* scr, int lr, int lg) {
#pragma unroll
    for (int e = 0; e < 4; ++e) scr[(4 * lg + e) * 17 + lr] = x[e];
    wave_lds_wait();
    f32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = scr[lr * 17 + 4 * lg + e];
    wave_lds_wait();
    return y;
}

template <int NM>
__device__ __forceinline__ void deep_fwd_mid(const DeepParams& p) {
    constexpr int L = NM + 2;
    __shared__ MidSmem<NM> sm;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    int* const status = p.work;

    // Group and part from the XCD the workgroup runs on (as deep_fwd2).
    if (tid == 0) {
        const int x = xcc_id() % p.nxcc;
        const int t = __hip_atomic_fetch_add(p.work + kTicketInts + x * kCtrStride, 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        const int per_xcd = p.ngroups / p.nxcc;
        sm.bail = t >= per_xcd * kG ? 1 : 0;
        if (sm.bail)
            __hip_atomic_fetch_or(status, static_cast<int>(kStatusPlacement), __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_SYSTEM);
        sm.gid = x + p.nxcc * (t / kG);
        sm.part = t % kG;
    }
    __syncthreads();
    if (sm.bail) return;
    const int gi = __builtin_amdgcn_readfirstlane(sm.gid);
    const int part = __builtin_amdgcn_readfirstlane(sm.part);
    int* const ctr = p.work + kHdrInts + gi * kCtrStride;
    float* const xall = reinterpret_cast<float*>(p.work + kHdrInts + p.ngroups * kCtrStride);
    float* const xbase = xall + static_cast<size_t>(gi) * kRingM * kG * kSlotM;
    // Weights and momenta of the hidden-to-hidden layers, [group][layer][W | S][wave of the group][tile][lane]
    // (this wave's 16 columns as accumulator tiles; only the owning lanes touch them).
    f32x4* const sbase = reinterpret_cast<f32x4*>(xall + static_cast<size_t>(p.ngroups) * kRingM * kG * kSlotM) +
                         (static_cast<size_t>(gi) * NM * 2 * (kG * kWaves) + (2 * part + w)) * kHT * 64 + lane;
    // Tile addresses come from a base made opaque where they are used, so that
    // the compiler forms them there instead of keeping all of them live across
    // the chunk loop (two registers each).
    auto tbase = [&]() -> f32x4* {
        f32x4* b = sbase;
        asm volatile("" : "+v"(b));
        return b;
    };
    auto wmid_at = [](f32x4* b, int m, int kt) -> f32x4* { return b + (static_cast<size_t>(2 * m) * (kG * kWaves) * kHT + kt) * 64; };
    auto smom_at = [](f32x4* b, int m, int kt) -> f32x4* {
        return b + (static_cast<size_t>(2 * m + 1) * (kG * kWaves) * kHT + kt) * 64;
    };
    const int hu = 32 * part + 16 * w;   // first hidden unit of this wave (every hidden layer)
    const int own = 2 * part + w;        // its 16-unit block
    int epoch = 0;

    // As in deep_fwd2: each wave's stores complete before the counter moves.
    auto signal = [&]() {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __syncthreads();
        if (tid == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto wait = [&]() -> bool {
        if (tid == 0) {
            const int target = kG * (epoch + 1);
            int spins = 0;
            while (l2_counter(ctr) < target) {
                if (++spins > p.spin_limit) {
                    sm.bail = 1;
                    __hip_atomic_fetch_or(status, static_cast<int>(kStatusTimeout), __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_SYSTEM);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        __syncthreads();
        ++epoch;
        return sm.bail == 0;
    };
    auto my_slot = [&]() { return xbase + static_cast<size_t>((epoch % kRingM) * kG + part) * kSlotM; };
    auto step_slots = [&]() { return xbase + static_cast<size_t>(((epoch - 1) % kRingM) * kG) * kSlotM; };
    // Gather: this wave's block of an activation (T layout: lane (lr, lg) =
    // X[token lr][unit hu + 4 lg + j], split) into dst[kt] of every workgroup.
    auto gather = [&](const Sp& xt, uint16_t (*dst)[2][kBlk]) -> bool {
        uint16_t* s = reinterpret_cast<uint16_t*>(my_slot());
        *reinterpret_cast<s16x4*>(s + (2 * w) * kBlk + lr * 16 + 4 * lg) = xt.hi;
        *reinterpret_cast<s16x4*>(s + (2 * w + 1) * kBlk + lr * 16 + 4 * lg) = xt.lo;
        signal();
        if (!wait()) return false;
        // Each wave copies 1 KB of every workgroup's slot: device-scope loads
        // into registers, all in flight, then into the LDS blocks.
        const auto rsl = make_rsrc(step_slots(), static_cast<uint32_t>(kG * kSlotM * 4));
        f32x4 blk[kG];
#pragma unroll
        for (int g2 = 0; g2 < kG; ++g2) blk[g2] = slot_load(rsl, g2 * kSlotM + w * 256 + lane * 4);
#pragma unroll
        for (int g2 = 0; g2 < kG; ++g2)
            *reinterpret_cast<f32x4*>(reinterpret_cast<char*>(&dst[2 * g2][0][0]) + w * 1024 + lane * 16) = blk[g2];
        __syncthreads();
        return true;
    };
    // T-layout fragment of gathered block kt (A with m = token, or B with n = token).
    auto gfrag = [&](const uint16_t (*src)[2][kBlk], int kt) -> Sp {
        return Sp{lds4(&src[kt][0][lr * 16 + 4 * lg]), lds4(&src[kt][1][lr * 16 + 4 * lg])};
    };

    for (int s = gi; s < p.BH; s += p.ngroups) {
        const size_t seq_tok = static_cast<size_t>(s) * p.T;
        const int nch = (p.T + p.b - 1) / p.b;
        auto chunk_n = [&](int c) { return min(p.b, p.T - c * p.b); };

        // ---- resident weights ----
        f32x4 W1[kDT], S1[kDT], WL[kDT], SL[kDT];
        {
            const float* w1 = p.W0[0] + s * p.wstride[0];
            const float* s1 = p.S0[0] ? p.S0[0] + s * p.wstride[0] : nullptr;
            const float* wl = p.W0[L - 1] + s * p.wstride[L - 1];
            const float* sl = p.S0[L - 1] ? p.S0[L - 1] + s * p.wstride[L - 1] : nullptr;
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i1 = (16 * dt + 4 * lg + e) * kHid + hu + lr;
                    const int i2 = (hu + 4 * lg + e) * kD + 16 * dt + lr;
                    W1[dt][e] = w1[i1];
                    S1[dt][e] = s1 ? s1[i1] : 0.f;
                    WL[dt][e] = wl[i2];
                    SL[dt][e] = sl ? sl[i2] : 0.f;
                }
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const float* wm = p.W0[1 + m] + s * p.wstride[1 + m];
                const float* sm0 = p.S0[1 + m] ? p.S0[1 + m] + s * p.wstride[1 + m] : nullptr;
                f32x4* const tb = tbase();
#pragma unroll
                for (int kt = 0; kt < kHT; ++kt) {
                    f32x4 wv, sv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int ij = (16 * kt + 4 * lg + e) * kHid + hu + lr;
                        wv[e] = wm[ij];
                        sv[e] = sm0 ? sm0[ij] : 0.f;
                    }
                    *wmid_at(tb, m, kt) = wv;
                    *smom_at(tb, m, kt) = sv;
                }
            }
        }
        auto stage_wl = [&]() {
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt) {
                const Sp ws = split(WL[dt]);
                *reinterpret_cast<s16x4*>(sm.wst[w][0] + (16 * dt + lr) * kWS + 4 * lg) = ws.hi;
                *reinterpret_cast<s16x4*>(sm.wst[w][1] + (16 * dt + lr) * kWS + 4 * lg) = ws.lo;
            }
        };
        stage_wl();

        Prefetch pf;
        prefetch(pf, p, seq_tok, 0, tid);
        __syncthreads();
        if (nch > 0) {
            stage(pf, sm.buf[0], tid);
            if (w == 1) gates(pf, sm.buf[0], chunk_n(0), lane);
        }
        __syncthreads();

        f32x4 Zp[2] = {};   // this workgroup's z partial of the previous chunk (own two d tiles)
        bool ok = true;
        const int iters = nch > 0 ? nch + 1 : 0;
        for (int c = 0; c < iters && ok; ++c) {
            const bool keys = c < nch;
            const bool zout = c >= 1;
            const ChunkBuf& B = sm.buf[c & 1];
            const int n = keys ? chunk_n(c) : 0;
            if (keys && c + 1 < nch) prefetch(pf, p, seq_tok, c + 1, tid);

            // ================= keys forward =================
            f32x4 dX[L - 1], Dk[L - 1];   // SiLU'(H_j), D_j (K layout: lane (lr, lg) = [token 4lg+e][unit lr])
            f32x4 XLk = {0.f, 0.f, 0.f, 0.f};
            Sp xlt{};                      // X_{L-1} (T layout), split
            if (keys) {
                f32x4 hk = {0.f, 0.f, 0.f, 0.f}, hkt = hk;
#pragma unroll
                for (int dt = 0; dt < kDT; ++dt) {
                    const s16x4 kf = lds4(B.kb + lr * kKS + 16 * dt + 4 * lg);
                    const Sp w1s = split(fresh(W1[dt]));
                    hk = mma2(kf, w1s, hk);
                    hkt = mma2(w1s, kf, hkt);
                }
                f32x4 xk;
                silu_d4(hk, xk, dX[0]);
                f32x4 xt = silu4(hkt);
                static_for<2, L, 1>([&](auto J) {
                    constexpr int j = decltype(J)::value;
                    if (!ok) return;
                    if (!gather(split(xt), sm.xg[j - 2])) {
                        ok = false;
                        return;
                    }
                    f32x4 ht = {0.f, 0.f, 0.f, 0.f};   // H_j^T[unit][token]
                    f32x4* const tb = tbase();
#pragma unroll
                    for (int kt = 0; kt < kHT; ++kt) {
                        ht = mma3(split(*wmid_at(tb, j - 2, kt)), gfrag(sm.xg[j - 2], kt), ht);
                        if ((kt & 7) == 7) asm volatile("" ::: "memory");   // at most 8 tiles of loads in flight (registers)
                    }
                    silu_d4(tr16(ht, sm.scr[w], lr, lg), xk, dX[j - 1]);
                    xt = silu4(ht);
                });
                if (!ok) break;
                XLk = xk;
                xlt = split(xt);
                f32x4 rp[kDT];
#pragma unroll
                for (int dt = 0; dt < kDT; ++dt) rp[dt] = mma3(split(fresh(WL[dt])), xlt, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) sm.xpart[1 - w][k2][lane] = w == 0 ? rp[2 + k2] : rp[k2];   // no run-time index into a register array
                __syncthreads();
                float* slot = my_slot();
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) {
                    const int dt = 2 * w + k2;
                    const f32x4 r = (w == 0 ? rp[k2] : rp[2 + k2]) + sm.xpart[w][k2][lane];
                    *reinterpret_cast<f32x4*>(slot + lr * kD + 16 * dt + 4 * lg) = r;
                }
            }
            // ================= R (and the z of chunk c - 1) across the group =================
            // Depth 3 takes this wave's R tiles and the z tiles straight into
            // registers (5.97 against 6.17 ms per launch); depth 4 has no
            // registers to spare and copies them into LDS.
            constexpr bool kRegR = NM == 1;
            f32x4 rpart[kRegR ? 2 : 1][kRegR ? kG : 1];
            {
                float* slot = my_slot();
                if (zout) {
#pragma unroll
                    for (int k2 = 0; k2 < 2; ++k2)
                        *reinterpret_cast<f32x4*>(slot + kNP * kD + lr * kD + 16 * (2 * w + k2) + 4 * lg) = Zp[k2];
                }
                signal();
                if (w == 1 && keys && c + 1 < nch) gates(pf, sm.buf[(c + 1) & 1], chunk_n(c + 1), lane);
                if (!wait()) {
                    ok = false;
                    break;
                }
                const float* rslot = step_slots();
                const bool zred = zout && part < kDT && w == 0;
                f32x4 zt = {0.f, 0.f, 0.f, 0.f};
                if constexpr (kRegR) {
                    const auto rsl = make_rsrc(rslot, static_cast<uint32_t>(kG * kSlotM * 4));
                    f32x4 zpart[kG];
                    if (keys) {
#pragma unroll
                        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
                            for (int g2 = 0; g2 < kG; ++g2)
                                rpart[k2][g2] = slot_load(rsl, g2 * kSlotM + lr * kD + 16 * (2 * w + k2) + 4 * lg);
                    }
                    if (zred) {
#pragma unroll
                        for (int g2 = 0; g2 < kG; ++g2)
                            zpart[g2] = slot_load(rsl, g2 * kSlotM + kNP * kD + lr * kD + 16 * part + 4 * lg);
                        zt = zpart[0];
#pragma unroll
                        for (int g2 = 1; g2 < kG; ++g2) zt += zpart[g2];
                    }
                } else {
                    if (keys) {
#pragma unroll
                        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
                            for (int g2 = 0; g2 < kG; ++g2)
                                __builtin_amdgcn_global_load_lds(rslot + g2 * kSlotM + lr * kD + 16 * (2 * w + k2) + 4 * lg,
                                                                 &sm.u.dma[w][k2 * kG + g2][0], 16, 0, kSlotLoadPolicy);
                    }
                    if (zred) {
#pragma unroll
                        for (int g2 = 0; g2 < kG; ++g2)
                            __builtin_amdgcn_global_load_lds(rslot + g2 * kSlotM + kNP * kD + lr * kD + 16 * part + 4 * lg,
                                                             &sm.dmaz[g2][0], 16, 0, kSlotLoadPolicy);
                    }
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    if (zred) {
                        zt = sm.dmaz[0][lane];
#pragma unroll
                        for (int g2 = 1; g2 < kG; ++g2) zt += sm.dmaz[g2][lane];
                    }
                }
                if (zred) {
                    const int np = chunk_n(c - 1);
                    const bool zb = p.z_bf16 != 0;
                    const uint32_t zsz = zb ? 2u : 4u;
                    const auto rz = make_rsrc(static_cast<char*>(p.z) + (seq_tok + static_cast<size_t>(c - 1) * p.b) * kD * zsz,
                                              static_cast<uint32_t>(np) * kD * zsz);
                    store_out4(zt, rz, static_cast<uint32_t>(lr * kD + 16 * part + 4 * lg), zb);
                }
            }
            if (!keys) continue;
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const int dt = 2 * w + k2;
                f32x4 r = unpack4(lds4(B.kb + lr * kKS + 16 * dt + 4 * lg)) - unpack4(lds4(B.vb + lr * kKS + 16 * dt + 4 * lg));
#pragma unroll
                for (int g2 = 0; g2 < kG; ++g2) {
                    if constexpr (kRegR) r += rpart[k2][g2];
                    else r += sm.u.dma[w][k2 * kG + g2][lane];
                }
                if (lr >= n) r = f32x4{0.f, 0.f, 0.f, 0.f};
                *reinterpret_cast<f32x4*>(sm.R + lr * kRS + 16 * dt + 4 * lg) = r;
#pragma unroll
                for (int e = 0; e < 4; ++e) sm.RT[(16 * dt + 4 * lg + e) * kRTS + lr] = r[e];
            }
            __syncthreads();

            // ================= deltas =================
            {
                f32x4 dH = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int dt = 0; dt < kDT; ++dt) {
                    const Sp rf = split(*reinterpret_cast<const f32x4*>(sm.R + lr * kRS + 16 * dt + 4 * lg));
                    const Sp wt{lds_tr4(sm.wst[w][0] + 16 * dt * kWS, kWS, lr, lg),
                                lds_tr4(sm.wst[w][1] + 16 * dt * kWS, kWS, lr, lg)};
                    dH = mma3(rf, wt, dH);
                }
                Dk[L - 2] = dH * dX[L - 2];
            }
            static_for<L - 1, 1, -1>([&](auto J) {
                constexpr int j = decltype(J)::value;
                if (!ok) return;
                const Sp dT = split(tr16(Dk[j - 1], sm.scr[w], lr, lg));   // D_j[:, U] (T layout)
                f32x4* const tb = tbase();
                // Eight tiles kt = 8 h + i at a time: loads in flight together,
                // then the transposes through LDS with one wait.
                auto half = [&](int h, auto&& use) {
                    f32x4 wv[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) wv[i] = *wmid_at(tb, j - 2, 8 * h + i);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const Sp sp = split(wv[i]);
                        *reinterpret_cast<s16x4*>(sm.wtr[w][i][0] + lr * kWS + 4 * lg) = sp.hi;
                        *reinterpret_cast<s16x4*>(sm.wtr[w][i][1] + lr * kWS + 4 * lg) = sp.lo;
                    }
                    wave_lds_wait();
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const Sp t{lds_tr4(sm.wtr[w][i][0], kWS, lr, lg), lds_tr4(sm.wtr[w][i][1], kWS, lr, lg)};
                        use(i, mma3(dT, t, f32x4{0.f, 0.f, 0.f, 0.f}));
                    }
                    wave_lds_wait();
                };
                // Partials of D_{j-1} over this wave's units: tile kt = D_j[:, U] W_j[16kt.., U]^T (K layout).
                half(1 - w, [&](int i, f32x4 t) { sm.u.pred[w][i][lane] = t; });
                __syncthreads();
                float* slot = my_slot();
                half(w, [&](int i, f32x4 t) {
                    *reinterpret_cast<f32x4*>(slot + (8 * w + i) * 256 + lane * 4) = t + sm.u.pred[1 - w][i][lane];
                });
                signal();
                if (!wait()) {
                    ok = false;
                    return;
                }
                const auto rsl = make_rsrc(step_slots(), static_cast<uint32_t>(kG * kSlotM * 4));
                f32x4 dpart[kG];
#pragma unroll
                for (int g2 = 0; g2 < kG; ++g2) dpart[g2] = slot_load(rsl, g2 * kSlotM + own * 256 + lane * 4);
                f32x4 sum = dpart[0];
#pragma unroll
                for (int g2 = 1; g2 < kG; ++g2) sum += dpart[g2];
                Dk[j - 2] = sum * dX[j - 2];
            });
            if (!ok) break;

            // ================= reads of chunk c =================
            {
                const float At = B.A[lr], Ct = B.C[lr];
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(B.L + lr * kLS + 4 * lg);   // L[t][4lg..]
                f32x4 kq = {0.f, 0.f, 0.f, 0.f}, za = kq, zc = kq;
#pragma unroll
                for (int dt = 0; dt < kDT; ++dt) {
                    const s16x4 kf = lds4(B.kb + lr * kKS + 16 * dt + 4 * lg);
                    const s16x4 qf = lds4(B.qb + lr * kKS + 16 * dt + 4 * lg);
                    kq = mma(kf, qf, kq);
                    za = mma2(split(fresh(W1[dt])), qf, za);
                    zc = mma2(split(fresh(S1[dt])), qf, zc);
                }
                f32x4 hq = mma3(split(Dk[0]), split(kq * l4), f32x4{0.f, 0.f, 0.f, 0.f});
                hq = At * za + Ct * zc - hq;   // Hq_1^T[unit][token]
                static_for<2, L, 1>([&](auto J) {
                    constexpr int j = decltype(J)::value;
                    if (!ok) return;
                    if (!gather(split(silu4(hq)), sm.yg)) {
                        ok = false;
                        return;
                    }
                    f32x4 yw = {0.f, 0.f, 0.f, 0.f}, ys = yw, gt = yw;
                    f32x4* const tb = tbase();
#pragma unroll
                    for (int kt = 0; kt < kHT; ++kt) {
                        const Sp yf = gfrag(sm.yg, kt);
                        yw = mma3(split(*wmid_at(tb, j - 2, kt)), yf, yw);
                        ys = mma3(split(*smom_at(tb, j - 2, kt)), yf, ys);
                        gt = mma3(gfrag(sm.xg[j - 2], kt), yf, gt);   // (X_{j-1} Y_{j-1}^T)[j'][t]
                        if ((kt & 7) == 7) asm volatile("" ::: "memory");
                    }
                    hq = At * yw + Ct * ys - mma3(split(Dk[j - 1]), split(gt * l4), f32x4{0.f, 0.f, 0.f, 0.f});
                });
                if (!ok) break;
                // z partial: Y_{L-1}[:, U] through W_L, S_L and the decayed Gram with R.
                const Sp aq = split(silu4(hq));
                const Sp lgm = split(mma3(xlt, aq, f32x4{0.f, 0.f, 0.f, 0.f}) * l4);
                f32x4 zp[kDT];
#pragma unroll
                for (int dt = 0; dt < kDT; ++dt) {
                    const f32x4 a2 = mma3(split(fresh(WL[dt])), aq, f32x4{0.f, 0.f, 0.f, 0.f});
                    const f32x4 c2 = mma3(split(fresh(SL[dt])), aq, f32x4{0.f, 0.f, 0.f, 0.f});
                    const Sp rs = split(*reinterpret_cast<const f32x4*>(sm.RT + (16 * dt + lr) * kRTS + 4 * lg));
                    const f32x4 in = mma3(rs, lgm, f32x4{0.f, 0.f, 0.f, 0.f});
                    zp[dt] = At * a2 + Ct * c2 - in;
                }
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) sm.xpart[1 - w][k2][lane] = w == 0 ? zp[2 + k2] : zp[k2];
                __syncthreads();
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) {
                    const int dt = 2 * w + k2;
                    Zp[k2] = (w == 0 ? zp[k2] : zp[2 + k2]) + sm.xpart[w][k2][lane];
                    if (part == 0) Zp[k2] += unpack4(lds4(B.qb + lr * kKS + 16 * dt + 4 * lg));
                }
            }

            // ================= carry =================
            {
                const float An = B.scal[0], Cn = B.scal[1], En = B.scal[2];
                const f32x4 wm4 = *reinterpret_cast<const f32x4*>(B.wm + 4 * lg);
                const f32x4 ws4 = *reinterpret_cast<const f32x4*>(B.ws + 4 * lg);
                {
                    const Sp dm = split(Dk[0] * wm4), dsv = split(Dk[0] * ws4);
#pragma unroll
                    for (int dt = 0; dt < kDT; ++dt) {
                        const s16x4 kt = lds_tr4(B.kb + 16 * dt, kKS, lr, lg);
                        const f32x4 w1 = An * W1[dt] + Cn * S1[dt];
                        S1[dt] = mma2(kt, dsv, En * S1[dt]);
                        W1[dt] = mma2(kt, dm, w1);
                    }
                }
                static_for<2, L, 1>([&](auto J) {
                    constexpr int j = decltype(J)::value;
                    const Sp dm = split(Dk[j - 1] * wm4), dsv = split(Dk[j - 1] * ws4);
                    f32x4* const tb = tbase();
#pragma unroll
                    for (int kt = 0; kt < kHT; ++kt) {
                        // X_{j-1}^T rows 16kt.. (A = X_{j-1}[token][unit] read transposed).
                        const Sp xk{lds_tr4(&sm.xg[j - 2][kt][0][0], 16, lr, lg), lds_tr4(&sm.xg[j - 2][kt][1][0], 16, lr, lg)};
                        f32x4 sv = *smom_at(tb, j - 2, kt);
                        const f32x4 wn = An * *wmid_at(tb, j - 2, kt) + Cn * sv;
                        sv = mma3(xk, dsv, En * sv);
                        *wmid_at(tb, j - 2, kt) = mma3(xk, dm, wn);
                        *smom_at(tb, j - 2, kt) = sv;
                        if ((kt & 7) == 7) asm volatile("" ::: "memory");
                    }
                });
                {
                    const Sp akm = split(XLk * wm4), aks = split(XLk * ws4);
#pragma unroll
                    for (int dt = 0; dt < kDT; ++dt) {
                        const Sp rs = split(*reinterpret_cast<const f32x4*>(sm.RT + (16 * dt + lr) * kRTS + 4 * lg));
                        const f32x4 w2 = An * WL[dt] + Cn * SL[dt];
                        SL[dt] = mma3(aks, rs, En * SL[dt]);
                        WL[dt] = mma3(akm, rs, w2);
                    }
                }
                stage_wl();
            }
            if (c + 1 < nch) stage(pf, sm.buf[(c + 1) & 1], tid);
            __syncthreads();
        }
        if (!ok) break;

        // ---- final weights ----
        {
            // Lane coordinates recomputed here (opaque), not kept live from the initial loads.
            int ln = lane;
            asm volatile("" : "+v"(ln));
            const int lr = ln & 15, lg = ln >> 4;
            float* w1 = p.WT[0] ? p.WT[0] + s * p.wstride[0] : nullptr;
            float* s1 = p.ST[0] ? p.ST[0] + s * p.wstride[0] : nullptr;
            float* wl = p.WT[L - 1] ? p.WT[L - 1] + s * p.wstride[L - 1] : nullptr;
            float* sl = p.ST[L - 1] ? p.ST[L - 1] + s * p.wstride[L - 1] : nullptr;
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i1 = (16 * dt + 4 * lg + e) * kHid + hu + lr;
                    const int i2 = (hu + 4 * lg + e) * kD + 16 * dt + lr;
                    if (w1) w1[i1] = W1[dt][e];
                    if (s1) s1[i1] = S1[dt][e];
                    if (wl) wl[i2] = WL[dt][e];
                    if (sl) sl[i2] = SL[dt][e];
                }
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                float* wm = p.WT[1 + m] ? p.WT[1 + m] + s * p.wstride[1 + m] : nullptr;
                float* smt = p.ST[1 + m] ? p.ST[1 + m] + s * p.wstride[1 + m] : nullptr;
                f32x4* const tb = tbase();
#pragma unroll
                for (int kt = 0; kt < kHT; ++kt) {
                    const f32x4 wv = *wmid_at(tb, m, kt), sv = *smom_at(tb, m, kt);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int ij = (16 * kt + 4 * lg + e) * kHid + hu + lr;
                        if (wm) wm[ij] = wv[e];
                        if (smt) smt[ij] = sv[e];
                    }
                }
            }
        }
    }
}

__global__ __launch_bounds__(kThreads, 1) void deep_fwd3(const DeepParams p) { deep_fwd_mid<1>(p); }
__global__ __launch_bounds__(kThreads, 1) void deep_fwd4(const DeepParams p) { deep_fwd_mid<2>(p); }

// Zero the status word and the group counters before a launch.
__global__ void deep_init(int* work, int nints) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nints; i += gridDim.x * blockDim.x) work[i] = 0;
}

}  // namespace

namespace {

// Exchange workspace of the entry point that allocates nothing: a file-scope
// device array (one copy per GPU, held until the process ends).  It holds the
// header and kScratchGroups groups; larger batches run kScratchGroups groups
// at a time.  Host code never passes the array's name to a kernel: it takes
// the array's device address on each GPU once (scratch_ptr) and uses that.
constexpr int kScratchGroups = 8;
constexpr size_t kScratchBytes = (static_cast<size_t>(kHdrInts) + kScratchGroups * kCtrStride) * 4 +
                                 static_cast<size_t>(kScratchGroups) * kRing * kG * kSlot * 4;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mutex;

// Device address of `scratch` on the current device (hipGetSymbolAddress
// once per device, with that device current); NULL on failure.
void* scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch[dev] = ptr;
    }
    return g_scratch[dev];
}

// Polls before a wait gives up: 2,000,000 (seconds, far beyond any healthy
// exchange), or TTT_MEM_DEEP_SPIN_LIMIT from the environment (read at every
// call), with which a test drives the timeout path from the host.
int spin_limit() {
    const char* e = std::getenv("TTT_MEM_DEEP_SPIN_LIMIT");
    if (!e || !*e) return 2000000;
    char* end = nullptr;
    const long v = std::strtol(e, &end, 10);
    return (*end == '\0' && v >= 0 && v <= 2000000000L) ? static_cast<int>(v) : 2000000;
}

// Workspace of a launch with ngroups groups: the header and group counters,
// the exchange slots and, for depth > 2, the momenta of the hidden-to-hidden
// layers (16 tiles of 64 x 4 floats per wave and layer).
size_t deep_work_bytes_for(long long ngroups, int depth = 2) {
    const size_t hdr = (static_cast<size_t>(kHdrInts) + static_cast<size_t>(ngroups) * kCtrStride) * 4;
    if (depth <= 2) return hdr + static_cast<size_t>(ngroups) * kRing * kG * kSlot * 4;
    return hdr + static_cast<size_t>(ngroups) * kRingM * kG * kSlotM * 4 +
           static_cast<size_t>(ngroups) * (depth - 2) * 2 * (kG * kWaves) * kHT * 64 * 16;
}

// Groups for BH sequences: a multiple of 8 (one XCD each), at most BH rounded
// up, and at most what can be resident at once.
long long deep_groups(long long BH, int max_groups) {
    long long g = (BH + 7) / 8 * 8;
    return g < max_groups ? g : max_groups;
}

struct TensorSet {   // a weight tensor, its momentum and their outputs, as passed by the caller
    const void* W0;
    const void* S0;
    const void* WT;
    const void* ST;
    size_t bytes;
};

struct Layers {
    const float* W0[4];
    const float* S0[4];
    float* WT[4];
    float* ST[4];
    long long stride[4];
    TensorSet tensors[4];
    int ntensors;
};

int deep_forward_impl(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* theta, const float* eta,
                      const float* alpha, const Layers& ly, int depth, void* z, bool z_bf16, int B, int H, int Tlen,
                      int d, int hidden, int b, void* work, size_t work_bytes, void* stream_,
                      bool use_scratch = false) {
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    if (B < 0 || H < 0 || Tlen < 0 || b < 1) return TTT_ERR_INVALID_ARG;
    if (d != kD || hidden != kHid || b > kNP || depth < 2 || depth > 4) return TTT_ERR_UNSUPPORTED;
    if (use_scratch && depth != 2) return TTT_ERR_UNSUPPORTED;
    const long long BH = static_cast<long long>(B) * H;
    if (BH == 0) return TTT_OK;
    if (BH > 0x7fffffffLL || BH * static_cast<long long>(Tlen) > 0x7fffffffLL) return TTT_ERR_UNSUPPORTED;
    for (int l = 0; l < depth; ++l)
        if (!ly.W0[l]) return TTT_ERR_INVALID_ARG;
    const size_t tok = static_cast<size_t>(BH) * static_cast<size_t>(Tlen);
    const size_t in_bytes = tok * kD * 2, z_bytes = tok * kD * (z_bf16 ? 2 : 4);
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
    }
    // Weight tensors (as the caller passes them: one per layer, or one
    // packed tensor for all layers): 4-byte aligned; an output may be its own
    // initial tensor (in-place carry) and overlaps nothing else; z overlaps
    // none of them.
    for (int i = 0; i < ly.ntensors; ++i) {
        const TensorSet& t = ly.tensors[i];
        const void* all[] = {t.W0, t.S0, t.WT, t.ST};
        for (const void* x : all) {
            if (x && !aligned(x, 4)) return TTT_ERR_INVALID_ARG;
            if (x && Tlen > 0 && overlaps(z, z_bytes, x, t.bytes)) return TTT_ERR_INVALID_ARG;
        }
        const void* outs[] = {t.WT, t.ST};
        const void* own[] = {t.W0, t.S0};
        for (int o = 0; o < 2; ++o) {
            if (!outs[o]) continue;
            for (int j = 0; j < ly.ntensors; ++j) {
                const TensorSet& u = ly.tensors[j];
                const void* others[] = {u.W0, u.S0, u.WT, u.ST};
                for (int k2 = 0; k2 < 4; ++k2) {
                    if (!others[k2]) continue;
                    if (j == i && k2 == 2 + o) continue;                     // itself
                    if (j == i && k2 == o && own[o] == outs[o]) continue;    // in-place carry
                    if (overlaps(outs[o], t.bytes, others[k2], u.bytes)) return TTT_ERR_INVALID_ARG;
                }
            }
        }
    }

    int dev = 0, ncu = 0, nxcc = 1, occ = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TTT_ERR_HIP;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return TTT_ERR_HIP;
    if (hipDeviceGetAttribute(&nxcc, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || nxcc < 1) nxcc = 1;
    void (*const kfn)(const DeepParams) = depth == 2 ? deep_fwd2 : depth == 3 ? deep_fwd3 : deep_fwd4;
    const void* kern = reinterpret_cast<const void*>(kfn);
    const int threads = depth == 2 ? kThreads2 : kThreads;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, threads, 0) != hipSuccess) return TTT_ERR_HIP;
    int max_groups = (ncu * occ / kG) / 8 * 8;
    if (use_scratch && max_groups > kScratchGroups) max_groups = kScratchGroups;
    if (max_groups < 8) return TTT_ERR_UNSUPPORTED;
    const long long ngroups = deep_groups(BH, max_groups);
    const size_t need = deep_work_bytes_for(ngroups, depth);
    bool own_work = false;
    if (use_scratch) {
        // The file-scope scratch: no allocation; sizes past it are refused.
        if (need > kScratchBytes) return TTT_ERR_UNSUPPORTED;
        work = scratch_ptr();
        if (!work) return TTT_ERR_HIP;
    } else if (work) {
        if (!aligned(work, 256) || work_bytes < need) return TTT_ERR_INVALID_ARG;
    } else {
        if (hipMallocAsync(&work, need, stream) != hipSuccess) return TTT_ERR_HIP;
        own_work = true;
    }

    DeepParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.theta = theta;
    p.eta = eta;
    p.alpha = alpha;
    for (int l = 0; l < 4; ++l) {
        p.W0[l] = l < depth ? ly.W0[l] : nullptr;
        p.S0[l] = l < depth ? ly.S0[l] : nullptr;
        p.WT[l] = l < depth ? ly.WT[l] : nullptr;
        p.ST[l] = l < depth ? ly.ST[l] : nullptr;
        p.wstride[l] = l < depth ? ly.stride[l] : 0;
    }
    p.z = z;
    p.z_bf16 = z_bf16 ? 1 : 0;
    p.BH = static_cast<int>(BH);
    p.T = Tlen;
    p.b = b;
    p.ngroups = static_cast<int>(ngroups);
    p.nxcc = nxcc;
    p.spin_limit = spin_limit();
    p.work = static_cast<int*>(work);
    const int hdr = kHdrInts + static_cast<int>(ngroups) * kCtrStride;
    hipLaunchKernelGGL(deep_init, dim3(8), dim3(256), 0, stream, p.work, hdr);
    hipError_t err = hipGetLastError();
    if (err == hipSuccess) {
        void* args[] = {&p};
        err = hipLaunchCooperativeKernel(kern, dim3(static_cast<unsigned>(ngroups * kG)), dim3(threads), args, 0,
                                         stream);
    }
    if (own_work) (void)hipFreeAsync(work, stream);
    return err == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

}  // namespace

extern "C" {

size_t ttt_mem_deep_param_count(int d, int hidden, int depth) {
    if (d < 1 || hidden < 1 || depth < 2) return 0;
    return static_cast<size_t>(d) * hidden * 2 + static_cast<size_t>(depth - 2) * hidden * hidden;
}

size_t ttt_mem_deep_work_bytes(int B, int H, int d, int hidden, int depth) {
    if (B < 0 || H < 0 || d != kD || hidden != kHid || depth < 2 || depth > 4) return 0;
    const long long BH = static_cast<long long>(B) * H;
    return deep_work_bytes_for(deep_groups(BH, 1 << 30), depth);
}

int ttt_mem_deep_forward_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* theta,
                              const float* eta, const float* alpha, const float* W0, const float* S0, uint16_t* z,
                              float* W_T, float* S_T, int B, int H, int T, int d, int hidden, int depth, int b,
                              void* work, size_t work_bytes, void* stream) {
    if (depth < 2 || depth > 4) return TTT_ERR_UNSUPPORTED;
    const long long P = static_cast<long long>(ttt_mem_deep_param_count(d, hidden, depth));
    Layers ly{};
    for (int l = 0; l < depth; ++l) {
        const long long off = l == 0 ? 0 : static_cast<long long>(d) * hidden + static_cast<long long>(l - 1) * hidden * hidden;
        ly.W0[l] = W0 ? W0 + off : nullptr;
        ly.S0[l] = S0 ? S0 + off : nullptr;
        ly.WT[l] = W_T ? W_T + off : nullptr;
        ly.ST[l] = S_T ? S_T + off : nullptr;
        ly.stride[l] = P;
    }
    const size_t tb = static_cast<size_t>(B > 0 && H > 0 ? static_cast<long long>(B) * H : 0) * P * 4;
    ly.tensors[0] = TensorSet{W0, S0, W_T, S_T, tb};
    ly.ntensors = 1;
    if (!W0) return TTT_ERR_INVALID_ARG;
    return deep_forward_impl(q, k, v, theta, eta, alpha, ly, depth, z, true, B, H, T, d, hidden, b, work, work_bytes,
                             stream);
}

int ttt_mem_deep_status(const void* work, void* stream) {
    if (!work) return TTT_ERR_INVALID_ARG;
    int st = 0;
    if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return TTT_ERR_HIP;
    if (hipMemcpy(&st, work, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return TTT_ERR_HIP;
    return st == 0 ? TTT_OK : TTT_ERR_DEVICE;
}

int ttt_mem_mlp_forward_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* theta,
                             const float* eta, const float* alpha, const float* W1_0, const float* W2_0,
                             const float* S1_0, const float* S2_0, uint16_t* z, float* W1_T, float* W2_T, float* S1_T,
                             float* S2_T, int B, int H, int T, int d, int hidden, int b, void* stream) {
    const long long s1 = static_cast<long long>(d) * hidden;
    const size_t tb = static_cast<size_t>(B > 0 && H > 0 ? static_cast<long long>(B) * H : 0) * s1 * 4;
    const Layers ly{{W1_0, W2_0}, {S1_0, S2_0}, {W1_T, W2_T}, {S1_T, S2_T}, {s1, s1},
                    {{W1_0, S1_0, W1_T, S1_T, tb}, {W2_0, S2_0, W2_T, S2_T, tb}}, 2};
    return deep_forward_impl(q, k, v, theta, eta, alpha, ly, 2, z, true, B, H, T, d, hidden, b, nullptr, 0, stream);
}

int ttt_mem_mlp_forward_bf16_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* theta,
                                     const float* eta, const float* alpha, const float* W1_0, const float* W2_0,
                                     const float* S1_0, const float* S2_0, uint16_t* z, float* W1_T, float* W2_T,
                                     float* S1_T, float* S2_T, int B, int H, int T, int d, int hidden, int b,
                                     void* stream) {
    const long long s1 = static_cast<long long>(d) * hidden;
    const size_t tb = static_cast<size_t>(B > 0 && H > 0 ? static_cast<long long>(B) * H : 0) * s1 * 4;
    const Layers ly{{W1_0, W2_0}, {S1_0, S2_0}, {W1_T, W2_T}, {S1_T, S2_T}, {s1, s1},
                    {{W1_0, S1_0, W1_T, S1_T, tb}, {W2_0, S2_0, W2_T, S2_T, tb}}, 2};
    return deep_forward_impl(q, k, v, theta, eta, alpha, ly, 2, z, true, B, H, T, d, hidden, b, nullptr, 0, stream,
                             true);
}

int ttt_mem_mlp_forward_bf16_zf32(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* theta,
                                  const float* eta, const float* alpha, const float* W1_0, const float* W2_0,
                                  const float* S1_0, const float* S2_0, float* z, float* W1_T, float* W2_T,
                                  float* S1_T, float* S2_T, int B, int H, int T, int d, int hidden, int b,
                                  void* stream) {
    const long long s1 = static_cast<long long>(d) * hidden;
    const size_t tb = static_cast<size_t>(B > 0 && H > 0 ? static_cast<long long>(B) * H : 0) * s1 * 4;
    const Layers ly{{W1_0, W2_0}, {S1_0, S2_0}, {W1_T, W2_T}, {S1_T, S2_T}, {s1, s1},
                    {{W1_0, S1_0, W1_T, S1_T, tb}, {W2_0, S2_0, W2_T, S2_T, tb}}, 2};
    return deep_forward_impl(q, k, v, theta, eta, alpha, ly, 2, z, false, B, H, T, d, hidden, b, nullptr, 0, stream);
}

}  // extern "C"
