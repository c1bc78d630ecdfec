// Token-by-token (primal) linear memory for decoding on gfx950 (MI355X), and
// its C ABI.
//
// Prefill evaluates chunks in their dual (matrix) form; generation is serial
// anyway, one token at a time, and uses the primal form: every token's
// gradient is taken at the memory its predecessor left, i.e. chunks of one
// token ("5.1.1 · TTT layers 与 fast weights", section 1.1, the primal/dual
// comparison after eq. (9)), with the state carried from call to call
// ("Continual Learning: From Attention to Neural Memory", section 4.8, the
// note on streaming inference).  Per token t and memory row i:
//
//   e_i   = M[i,:] . k_t - v_t[i]
//   S[i,:] = eta_t S[i,:] - theta_t e_i k_t
//   M[i,:] = (1 - alpha_t) M[i,:] + S[i,:]
//   z_t[i] = M[i,:] . q_t
//
// ("论文速览 | Titans", sections 3.4 and 3.7).  Row i only ever meets value
// coordinate i, so rows are independent: a wave keeps LPR = d/4 lanes per
// row (four consecutive columns each, float32) for RPW = 64/LPR rows, holds
// those rows of M and S in registers for all of the call's tokens, and
// reduces the two dot products per token with butterfly shuffles inside each
// row's lane group.  Arithmetic is float32 throughout (bf16 inputs widen
// exactly).  One call touches the state once: read, T tokens, write -- for
// T = 1 the kernel is bound by HBM on the 4 d^2 floats of state traffic per
// (batch, head).

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ttt_mem.h"
#include "gfx950.h"

namespace {

constexpr int kDecWave = 64;
constexpr int kDecWaves = 4;   // waves per workgroup

struct DecParams {
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
};

template <bool BF16>
__device__ __forceinline__ f32x4 load4(const void* base, size_t elem) {
    if constexpr (BF16) {
        const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + elem);
        return f32x4{bf16lo(u.x), bf16hi(u.x), bf16lo(u.y), bf16hi(u.y)};
    } else {
        return *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + elem);
    }
}
template <bool BF16>
__device__ __forceinline__ float load1(const void* base, size_t elem) {
    if constexpr (BF16) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(base)[elem]) << 16);
    else return static_cast<const float*>(base)[elem];
}

// Sum over the LPR lanes of one row group (aligned, power of two); every lane
// of the group receives the total.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) x += __shfl_xor(x, m, kDecWave);
    return x;
}

template <bool BF16, int D>
__global__ __launch_bounds__(kDecWave * kDecWaves) void linear_memory_decode(const DecParams p) {
    constexpr int LPR = D / 4;                  // lanes per row
    constexpr int RPW = kDecWave / LPR;         // rows per wave
    constexpr int RPG = RPW * kDecWaves;        // rows per workgroup
    constexpr int WG_PER_SEQ = (D + RPG - 1) / RPG;
    const int lane = threadIdx.x % kDecWave;
    const int w = threadIdx.x / kDecWave;
    const int bh = blockIdx.x / WG_PER_SEQ;
    const int row = (blockIdx.x % WG_PER_SEQ) * RPG + w * RPW + lane / LPR;
    const int col = 4 * (lane % LPR);
    if (bh >= p.BH || row >= D) return;   // whole row groups leave together (LPR divides 64)

    const size_t st = (static_cast<size_t>(bh) * D + row) * D + col;
    f32x4 M = p.M0 ? *reinterpret_cast<const f32x4*>(p.M0 + st) : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 S = p.S0 ? *reinterpret_cast<const f32x4*>(p.S0 + st) : f32x4{0.f, 0.f, 0.f, 0.f};

    const size_t tok0 = static_cast<size_t>(bh) * p.T;
    for (int t = 0; t < p.T; ++t) {
        const size_t tk = tok0 + t;
        const f32x4 kk = load4<BF16>(p.k, tk * D + col);
        const f32x4 qq = load4<BF16>(p.q, tk * D + col);
        const float vi = load1<BF16>(p.v, tk * D + row);
        const float th = p.theta[tk], et = p.eta[tk], al = p.alpha[tk];
        const float e = group_sum<LPR>(M[0] * kk[0] + M[1] * kk[1] + M[2] * kk[2] + M[3] * kk[3]) - vi;
        const float te = th * e, a = 1.f - al;
        S = et * S - te * kk;
        M = a * M + S;
        const float zi = group_sum<LPR>(M[0] * qq[0] + M[1] * qq[1] + M[2] * qq[2] + M[3] * qq[3]);
        if (lane % LPR == 0) p.z[tk * D + row] = zi;
    }
    if (p.MT) *reinterpret_cast<f32x4*>(p.MT + st) = M;
    if (p.ST) *reinterpret_cast<f32x4*>(p.ST + st) = S;
}

template <bool BF16, int D>
hipError_t launch_decode(const DecParams& p, hipStream_t stream) {
    constexpr int RPG = (kDecWave / (D / 4)) * kDecWaves;
    constexpr int WG_PER_SEQ = (D + RPG - 1) / RPG;
    const dim3 grid(static_cast<unsigned>(p.BH) * WG_PER_SEQ);
    hipLaunchKernelGGL((linear_memory_decode<BF16, D>), grid, dim3(kDecWave * kDecWaves), 0, stream, p);
    return hipGetLastError();
}

template <bool BF16>
int decode_impl(const void* q, const void* k, const void* v, const float* theta, const float* eta,
                const float* alpha, const float* M0, const float* S0, float* z, float* M_T, float* S_T,
                int B, int H, int Tlen, int d, void* stream) {
    const size_t esz = BF16 ? 2 : 4;
    if (B < 0 || H < 0 || Tlen < 0) return TTT_ERR_INVALID_ARG;
    if (d != 16 && d != 32 && d != 64 && d != 128) return TTT_ERR_UNSUPPORTED;
    const long long BH = static_cast<long long>(B) * H;
    if (BH == 0) return TTT_OK;
    if (BH * d > 0x7fffffffLL || BH * static_cast<long long>(Tlen) > 0x7fffffffLL) return TTT_ERR_UNSUPPORTED;
    const size_t tok = static_cast<size_t>(BH) * static_cast<size_t>(Tlen);
    const size_t in_bytes = tok * d * esz;
    const size_t z_bytes = tok * d * sizeof(float);
    const size_t st_bytes = static_cast<size_t>(BH) * d * d * sizeof(float);
    if (Tlen > 0) {
        if (!q || !k || !v || !theta || !eta || !alpha || !z) return TTT_ERR_INVALID_ARG;
        const size_t a_in = BF16 ? 8 : 16;
        if (!aligned(q, a_in) || !aligned(k, a_in) || !aligned(v, esz) || !aligned(z, 4)) return TTT_ERR_INVALID_ARG;
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
    // In-place carry only as exact aliasing: every lane reads its own state
    // segment before it writes the same segment.
    if (M_T && M_T != M0 && (overlaps(M_T, st_bytes, M0, st_bytes) || overlaps(M_T, st_bytes, S0, st_bytes)))
        return TTT_ERR_INVALID_ARG;
    if (S_T && S_T != S0 && (overlaps(S_T, st_bytes, S0, st_bytes) || overlaps(S_T, st_bytes, M0, st_bytes)))
        return TTT_ERR_INVALID_ARG;
    if (M_T && S_T && overlaps(M_T, st_bytes, S_T, st_bytes)) return TTT_ERR_INVALID_ARG;

    const DecParams p{q, k, v, theta, eta, alpha, M0, S0, z, M_T, S_T, static_cast<int>(BH), Tlen};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    switch (d) {
        case 16: err = launch_decode<BF16, 16>(p, s); break;
        case 32: err = launch_decode<BF16, 32>(p, s); break;
        case 64: err = launch_decode<BF16, 64>(p, s); break;
        default: err = launch_decode<BF16, 128>(p, s); break;
    }
    return err == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

}  // namespace

extern "C" {

int ttt_mem_decode_f32(const float* q, const float* k, const float* v, const float* theta, const float* eta,
                       const float* alpha, const float* M0, const float* S0, float* z, float* M_T, float* S_T,
                       int B, int H, int T, int d, void* stream) {
    return decode_impl<false>(q, k, v, theta, eta, alpha, M0, S0, z, M_T, S_T, B, H, T, d, stream);
}

int ttt_mem_decode_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* theta,
                        const float* eta, const float* alpha, const float* M0, const float* S0, float* z,
                        float* M_T, float* S_T, int B, int H, int T, int d, void* stream) {
    return decode_impl<true>(q, k, v, theta, eta, alpha, M0, S0, z, M_T, S_T, B, H, T, d, stream);
}

}  // extern "C"
