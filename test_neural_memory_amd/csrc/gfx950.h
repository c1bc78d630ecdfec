// Small gfx950 device helpers shared by the memory kernels: vector types,
// fp32 -> fp16 packing, raw buffer descriptors (bounded loads and stores),
// the LDS transpose load, lane broadcasts, and host-side pointer checks.
#ifndef TTT_MEM_GFX950_H
#define TTT_MEM_GFX950_H

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats to two fp16, round to nearest even (one v_cvt_pk_f16_f32).
__device__ __forceinline__ f16x2 cvt2(float a, float b) { return __builtin_convertvector(f32x2{a, b}, f16x2); }
__device__ __forceinline__ f16x4 cvt4(f32x4 v) {
    const f16x2 lo = cvt2(v[0], v[1]), hi = cvt2(v[2], v[3]);
    return f16x4{lo[0], lo[1], hi[0], hi[1]};
}

// Four floats to four bf16, round to nearest even (two v_cvt_pk_bf16_f32),
// packed in two dwords in element order.
__device__ __forceinline__ u32x2 pack_bf16x4(f32x4 v) {
    const bf16x2 lo = __builtin_convertvector(f32x2{v[0], v[1]}, bf16x2);
    const bf16x2 hi = __builtin_convertvector(f32x2{v[2], v[3]}, bf16x2);
    return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// LDS transpose load of four 16-bit elements (gfx950).  Within each group of
// 16 lanes, lane i receives element i%4 of the chunk read by lane 4j + i/4 in
// slot j.
__device__ __forceinline__ i16x4 ds_read_tr16(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(reinterpret_cast<uintptr_t>(p)));
}

// LDS by 32-bit byte address.  lds_addr gives the address of a pointer into
// __shared__ memory; opaque() hides a value from the optimizer so that a base
// address computed once stays in one register and every access adds a
// compile-time offset (folded into the instruction's 16-bit offset field).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
}
template <typename V>
__device__ __forceinline__ V lds_load(uint32_t a) {
    return *(const __attribute__((address_space(3))) V*)(static_cast<uintptr_t>(a));
}
template <typename V>
__device__ __forceinline__ void lds_store(uint32_t a, V v) {
    *(__attribute__((address_space(3))) V*)(static_cast<uintptr_t>(a)) = v;
}
__device__ __forceinline__ i16x4 ds_read_tr16_at(uint32_t a) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(static_cast<uintptr_t>(a)));
}

// Raw buffer descriptor over nbytes at ptr: accesses at or past nbytes read 0
// and are not written, which bounds ragged chunks without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* ptr, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(ptr), (short)0, static_cast<int>(nbytes), 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store16(f32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
}

__device__ __forceinline__ void buf_store8(u32x2 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}
// Four consecutive elements of an output row: float32 (16 bytes) or, with bf,
// bf16 rounded to nearest even (8 bytes); off counts elements.  Stores at or
// past the descriptor's range are dropped.
__device__ __forceinline__ void store_out4(f32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off, bool bf) {
    if (bf) buf_store8(pack_bf16x4(v), r, off * 2);
    else buf_store16(v, r, off * 4);
}

__device__ __forceinline__ float readlane(float x, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

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
        const f16x4 a = cvt4(lo), b = cvt4(hi);
        return frag{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
};

// Global-memory element types: float for the f32 path, raw bf16 bits for the
// bf16-input path (whose matrix operands are fp16).
template <typename T> struct GlobalOf;
template <> struct GlobalOf<float> { using type = float; };
template <> struct GlobalOf<_Float16> { using type = uint16_t; };

// Four float32 values -> four elements of T at an address (LDS or global;
// 8 or 16 bytes), and back.
template <typename T>
__device__ __forceinline__ void st4(T* dst, f32x4 v) {
    if constexpr (Op<T>::kF16) {
        *reinterpret_cast<f16x4*>(dst) = cvt4(v);
    } else {
        *reinterpret_cast<f32x4*>(dst) = v;
    }
}
template <typename T>
__device__ __forceinline__ f32x4 ld4(const T* src) {
    if constexpr (Op<T>::kF16) {
        const f16x4 h = *reinterpret_cast<const f16x4*>(src);
        return f32x4{static_cast<float>(h[0]), static_cast<float>(h[1]), static_cast<float>(h[2]),
                     static_cast<float>(h[3])};
    } else {
        return *reinterpret_cast<const f32x4*>(src);
    }
}

// Host-side pointer checks.
bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// Bytes of the chunk-start state checkpoints of a dense [B, H, T] problem:
// [B*H][ceil(T/b)][M | S][d][d] elements of elem bytes (0 for sizes no entry
// point accepts).
[[maybe_unused]] size_t ckpt_bytes(int B, int H, int T, int d, int b, size_t elem = sizeof(float)) {
    if (B < 0 || H < 0 || T < 0 || d < 1 || b < 1) return 0;
    const size_t nch = (static_cast<size_t>(T) + b - 1) / b;
    return static_cast<size_t>(B) * H * nch * 2 * d * d * elem;
}

// A byte range of a buffer (argument overlap checks).
struct Span {
    const void* p;
    size_t n;
};

// Packed documents ([H, T] tokens, N documents): chunk slots per head.  A
// document of length l has ceil(l / b) chunks, so the N documents of a head
// have at most ceil(T / b) + N of them; document s of head h owns the slots
// h * slots + (chunks of documents 0..s-1) onward.
inline long long varlen_chunk_slots(int N, int T, int b) {
    return (static_cast<long long>(T) + b - 1) / b + N;
}
[[maybe_unused]] size_t ckpt_bytes_varlen(int N, int H, int T, int d, int b, size_t elem = sizeof(float)) {
    if (N < 0 || H < 0 || T < 0 || d < 1 || b < 1) return 0;
    return static_cast<size_t>(H) * static_cast<size_t>(varlen_chunk_slots(N, T, b)) * 2 * d * d * elem;
}
// Length of document s, its offsets clamped into [0, T] (a malformed table
// cannot reach outside the packed arrays).
__device__ __forceinline__ int doc_len(const int* cu, int s, int T, int& t0) {
    t0 = min(max(cu[s], 0), T);
    return min(max(cu[s + 1], t0), T) - t0;
}
// Chunks of documents 0 .. s-1 (the first chunk slot of document s).  Called
// by a whole 64-wide wave (lane = its lane index, s uniform): the lanes take
// 64 documents at a time and the wave sums their chunk counts.
__device__ __forceinline__ int doc_chunk_prefix(const int* cu, int s, int T, int b, int lane) {
    int acc = 0;
    for (int base = 0; base < s; base += 64) {
        const int j = base + lane;
        int nj = 0;
        if (j < s) {
            int t0;
            nj = (doc_len(cu, j, T, t0) + b - 1) / b;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) nj += __shfl_xor(nj, o, 64);
        acc += nj;
    }
    return __builtin_amdgcn_readfirstlane(acc);
}

// Packed documents: the document of rank r when the N documents are ordered
// by length, longest first (ties by index, so a permutation); lane is the
// lane index in a 64-wide wave.  Workgroups dispatched first then take the
// longest chains (longest processing time first), and the short ones fill in
// behind them.  Up to kLptDocs documents every wave computes it (lanes over
// candidate documents, the table read with uniform indices); above that the
// order comes from doc_rank_order (perm[r], written by a pass before the
// launch), or, with no such table, the packing order is kept.
constexpr int kLptDocs = 128;
__device__ __forceinline__ int doc_of_rank(const int* cu, int N, int T, int r, int lane, const int* perm = nullptr) {
    static_assert(kLptDocs <= 128, "two lengths per lane");
    if (N > kLptDocs) return perm ? perm[r] : r;
    // Lane l holds the lengths of documents l and 64 + l (-1 past N); the
    // rank loop reads them back with uniform lane reads, not memory loads.
    int len[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const int i = 64 * g + lane;
        int t0;
        len[g] = i < N ? doc_len(cu, i, T, t0) : -1;
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        if (64 * g >= N) break;
        const int i = 64 * g + lane;
        const int li = len[g];
        int rank = 0;
        for (int j = 0; j < min(N, 64); ++j) {
            const int lj = __builtin_amdgcn_readlane(len[0], j);
            rank += (lj > li || (lj == li && j < i)) ? 1 : 0;
        }
        for (int j = 64; j < N; ++j) {
            const int lj = __builtin_amdgcn_readlane(len[1], j - 64);
            rank += (lj > li || (lj == li && j < i)) ? 1 : 0;
        }
        const unsigned long long hit = __ballot(i < N && rank == r);
        if (hit) return 64 * g + __ffsll(static_cast<long long>(hit)) - 1;
    }
    return r;
}

// perm[rank(i)] = i for the same order (length descending, index ascending),
// any N: thread i counts the documents that come before document i, reading
// the lengths through LDS 256 at a time.  The ranks are distinct, so perm is
// a permutation of 0 .. N-1.  Launch: ceil(N / 256) workgroups of 256.
__global__ __launch_bounds__(256) void doc_rank_order(const int* __restrict__ cu, int N, int T, int* __restrict__ perm) {
    __shared__ int lens[256];
    const int i = blockIdx.x * 256 + threadIdx.x;
    int t0;
    const int li = i < N ? doc_len(cu, i, T, t0) : -1;
    int rank = 0;
    for (int base = 0; base < N; base += 256) {
        __syncthreads();
        const int j = base + threadIdx.x;
        lens[threadIdx.x] = j < N ? doc_len(cu, j, T, t0) : -1;
        __syncthreads();
        const int cnt = min(256, N - base);
        for (int jj = 0; jj < cnt; ++jj) {
            const int lj = lens[jj];
            rank += (lj > li || (lj == li && base + jj < i)) ? 1 : 0;
        }
    }
    if (i < N) perm[rank] = i;
}

// Host: the LPT order table for N packed documents when the in-kernel ranking
// does not cover them (N > kLptDocs): N ints from the stream-ordered
// allocator, filled by doc_rank_order on `stream`; NULL (and hipSuccess) when
// not needed.  The caller frees it with hipFreeAsync after its launches.
[[maybe_unused]] hipError_t make_doc_order(const int* cu, int N, int T, hipStream_t stream, int** perm) {
    *perm = nullptr;
    if (N <= kLptDocs) return hipSuccess;
    hipError_t err = hipMallocAsync(reinterpret_cast<void**>(perm), static_cast<size_t>(N) * sizeof(int), stream);
    if (err != hipSuccess) {
        *perm = nullptr;
        return err;
    }
    hipLaunchKernelGGL(doc_rank_order, dim3(static_cast<unsigned>((N + 255) / 256)), dim3(256), 0, stream, cu, N, T,
                       *perm);
    err = hipGetLastError();
    if (err != hipSuccess) {
        (void)hipFreeAsync(*perm, stream);
        *perm = nullptr;
    }
    return err;
}

}  // namespace

// ---------------------------------------------------------------------------
// Persistent walks over packed documents: each workgroup's table of units.
//
// Units u = (rank, head) in rank order (documents longest first, ties by
// index) go to workgroup lanes: a lane is the NRB row-block workgroups of one
// XCD slot, me = x8 + 8 v of G2 = 8 V, with x8 the workgroup id mod 8, so the
// row blocks of a unit share one L2.  Two steps, longest processing time
// first:
// - head: when the lengths are heavy-tailed (the longest unit at least a
//   quarter of a lane's average), the units of at least 1/16 of that average
//   go one by one to the least-loaded lane (ties by lane), kept as one load
//   per wave lane and found by a wave-wide minimum;
// - rest: the lanes still below the average take the remaining units in
//   boustrophedon order (round q deals one unit to each open lane, in lane
//   order for even q and in reverse for odd q), which a lane enumerates alone.
//   Without a head every lane is open.
// The documents' offsets, lengths, chunk prefixes (checkpoint slots, with
// `slots`) and ranks live in `temp` (4 N + KMAX ints) while the table is
// built; the ranks count the documents before each one in the order (longer,
// or as long with a smaller index), so they are a permutation.  Units that
// are empty (after the cut at a head's last slot) take no place in the table:
// their state slots are left at temp + 4 N for the caller.  Afterwards
// counts = {chunks in all, table entries, empty units}; the caller clears
// temp once it is done with the empty units.
// ---------------------------------------------------------------------------
struct WalkUnit {
    int tok0, len, ck0, bh;   // first token in the [H, T] rows, length, slot of its first chunk, state slot
};

// s_waitcnt immediate for vmcnt(0) alone (expcnt 7, lgkmcnt 15 left open).
constexpr int kWaitVm0 = 0x0F70;
// Minimum and maximum over a 64-wide wave (every lane gets a value; the
// result is exact in lane 63), with the row-shift / row-broadcast DPP steps
// of the gate scan.
__device__ __forceinline__ unsigned wave_min_u32(unsigned x) {
    auto step = [&](auto ctrl, auto rmask) {
        const unsigned y = static_cast<unsigned>(__builtin_amdgcn_update_dpp(
            static_cast<int>(0xffffffffu), static_cast<int>(x), decltype(ctrl)::value, decltype(rmask)::value, 0xf, false));
        x = min(x, y);
    };
    step(std::integral_constant<int, kRowShr1>{}, std::integral_constant<int, 0xf>{});
    step(std::integral_constant<int, kRowShr2>{}, std::integral_constant<int, 0xf>{});
    step(std::integral_constant<int, kRowShr4>{}, std::integral_constant<int, 0xf>{});
    step(std::integral_constant<int, kRowShr8>{}, std::integral_constant<int, 0xf>{});
    step(std::integral_constant<int, kRowBcast15>{}, std::integral_constant<int, 0xa>{});
    step(std::integral_constant<int, kRowBcast31>{}, std::integral_constant<int, 0xc>{});
    return static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}
__device__ __forceinline__ int wave_max_i32(int x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
    return x;
}


template <int NTH, int KMAX>
__device__ __forceinline__ void build_walk_table(const int* __restrict__ cu, int N, int H, int Tl, int b, bool slots,
                                                 int tcmax, int* temp, WalkUnit* units, int* counts, int x8, int v,
                                                 int V) {
    constexpr int kWave = 64;
    const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
    const int U_ = N * H;
    int* tlen = temp;
    int* tt0 = tlen + N;
    int* tpre = tt0 + N;
    int* tperm = tpre + N;
    int* tempty = tperm + N;
    for (int i = tid; i < N; i += NTH) {
        const int a = min(max(cu[i], 0), Tl);
        tt0[i] = a;
        tlen[i] = min(max(cu[i + 1], a), Tl) - a;
    }
    __syncthreads();
    if (w == 0 && slots) {
        // Checkpoint slots: chunks of the documents before each one, in document order.
        int carry = 0;
        for (int base = 0; base < N; base += kWave) {
            const int i = base + lane;
            const int cnt = i < N ? (tlen[i] + b - 1) / b : 0;
            int incl = cnt;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const int y = __shfl_up(incl, o, kWave);
                if (lane >= o) incl += y;
            }
            if (i < N) tpre[i] = carry + incl - cnt;
            carry += __shfl(incl, kWave - 1, kWave);
        }
    }
    for (int i = tid; i < N; i += NTH) {
        const int li = tlen[i];
        int r = 0;
        for (int j = 0; j < N; ++j) {
            const int lj = tlen[j];
            r += (lj > li || (lj == li && j < i)) ? 1 : 0;
        }
        tperm[r] = i;
    }
    __syncthreads();
    // Wave 0 builds this workgroup's table.  Workgroup lanes (one lane = the
    // NRB row-block workgroups of one XCD slot, me = x8 + 8 v of G2 = 8 V)
    // take units u = (rank, head) in rank order, longest processing time
    // first in two steps:
    // - head: when the lengths are heavy-tailed (the longest unit at least a
    //   quarter of a lane's average), the units of at least 1/16 of that
    //   average go one by one to the least-loaded lane (ties by lane), kept
    //   as one load per wave lane and found by a wave-wide minimum;
    // - rest: the lanes still below the average take the remaining units in
    //   boustrophedon order (round q deals one unit to each open lane, in
    //   lane order for even q and in reverse for odd q), which a lane
    //   enumerates alone.  Without a head every lane is open.
    // Empty units take no place in the walk; their owner copies the states.
    int empties = 0;
    if (w == 0) {
        const int me = x8 + 8 * v, G2 = 8 * V, U = U_;
        auto unit_len = [&](int r, int h, int& tok0, int& ck0, int& bh) {
            const int s = tperm[r];
            int len = tlen[s];
            ck0 = 0;
            if (slots) {
                // Overlapping documents (offsets not non-decreasing) are cut at the head's last slot.
                const int pre = tpre[s];
                len = min(len, max(tcmax - pre, 0) * b);
                ck0 = h * tcmax + pre;
            }
            tok0 = h * Tl + tt0[s];
            bh = s * H + h;
            return len;
        };
        auto chunks_of_rank = [&](int r) {
            int t0_, c0_, bh_;
            return (unit_len(r, 0, t0_, c0_, bh_) + b - 1) / b;
        };
        // Total chunks over all units (the heads of a rank share its length).
        long long tot = 0;
        for (int base = 0; base < N; base += kWave) {
            int c = base + lane < N ? chunks_of_rank(base + lane) : 0;
#pragma unroll
            for (int o = kWave / 2; o > 0; o >>= 1) c += __shfl_xor(c, o, kWave);
            tot += c;
        }
        tot *= H;
        int kept = 0, J = 0;
        int E = 0;            // units in the head
        int ld = 0, cnt = 0;  // this wave lane's workgroup lane: chunks and units from the head
        const bool skew = G2 <= kWave && N > 0 && 4LL * chunks_of_rank(0) * G2 >= tot && (tot << 6) < 0x7fffffffLL;
        if (skew) {
            for (int r = 0; r < N; ++r) {
                const int c = chunks_of_rank(r);
                if (16LL * c * G2 < tot) break;
                for (int h = 0; h < H; ++h) {
                    // key = load * 64 + lane (lanes >= G2 never win)
                    const unsigned key = lane < G2 ? static_cast<unsigned>(ld) * kWave + lane : 0xffffffffu;
                    const int win = static_cast<int>(wave_min_u32(key) & (kWave - 1));
                    if (lane == win) {
                        ld += c;
                        cnt += 1;
                    }
                    if (win == me) {
                        int tok0, ck0, bh;
                        const int len = unit_len(r, h, tok0, ck0, bh);
                        if (lane == 0 && kept < KMAX) units[kept] = {tok0, len, ck0, bh};
                        ++kept;
                        J += c;
                    }
                }
                E += H;
            }
        }
        // Open lanes: below the average load (tot / G2 chunks).
        // (When the head holds every chunk and leaves no lane below, all lanes stay open for the empty units.)
        const unsigned long long below_avg = __ballot(lane < G2 && static_cast<long long>(ld) * G2 < tot);
        const unsigned long long open = below_avg ? below_avg : __ballot(lane < G2);
        const int nopen = __popcll(open);
        const bool me_open = (open >> me) & 1ull;
        const int myidx = __popcll(open & ((1ull << me) - 1ull));
        const int rest = U - E;
        const int rounds = nopen > 0 ? (rest + nopen - 1) / nopen : 0;
        // Every lane's table must fit: the head counts are known per lane, the rest at most `rounds`.
        const int maxhead = __builtin_amdgcn_readfirstlane(wave_max_i32(lane < G2 ? cnt : 0));
        if (maxhead + rounds <= KMAX && me_open) {
            for (int base = 0; base < rounds; base += kWave) {
                const int q = base + lane;
                const int u = E + q * nopen + ((q & 1) ? nopen - 1 - myidx : myidx);
                int tok0 = 0, ck0 = 0, bh = 0, len = 0;
                const bool live = q < rounds && u < U;
                if (live) len = unit_len(u / H, u % H, tok0, ck0, bh);
                const unsigned long long full = __ballot(live && len > 0);
                const unsigned long long none = __ballot(live && len == 0);
                const unsigned long long below = (1ull << lane) - 1ull;
                if (live && len > 0) units[kept + __popcll(full & below)] = {tok0, len, ck0, bh};
                if (live && len == 0) tempty[empties + __popcll(none & below)] = bh;
                kept += __popcll(full);
                empties += __popcll(none);
                int c = len > 0 ? (len + b - 1) / b : 0;
#pragma unroll
                for (int o = kWave / 2; o > 0; o >>= 1) c += __shfl_xor(c, o, kWave);
                J += c;
            }
        } else if (maxhead + rounds > KMAX) {
            // Some lane's table would overflow: plain boustrophedon order over all lanes
            // (at most ceil(U / G2) units each, which the launch checked).
            kept = 0;
            J = 0;
            const int rr = (U + G2 - 1) / G2;
            for (int base = 0; base < rr; base += kWave) {
                const int q = base + lane;
                const int u = q * G2 + ((q & 1) ? G2 - 1 - me : me);
                int tok0 = 0, ck0 = 0, bh = 0, len = 0;
                const bool live = q < rr && u < U;
                if (live) len = unit_len(u / H, u % H, tok0, ck0, bh);
                const unsigned long long full = __ballot(live && len > 0);
                const unsigned long long none = __ballot(live && len == 0);
                const unsigned long long below = (1ull << lane) - 1ull;
                if (live && len > 0) units[kept + __popcll(full & below)] = {tok0, len, ck0, bh};
                if (live && len == 0) tempty[empties + __popcll(none & below)] = bh;
                kept += __popcll(full);
                empties += __popcll(none);
                int c = len > 0 ? (len + b - 1) / b : 0;
#pragma unroll
                for (int o = kWave / 2; o > 0; o >>= 1) c += __shfl_xor(c, o, kWave);
                J += c;
            }
        }
        if (lane == 0) {
            counts[0] = J;
            counts[1] = kept;
            counts[2] = empties;
        }
    }
    __syncthreads();
}

#endif  // TTT_MEM_GFX950_H
