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
//   * producer waves (two, or four with the column split below), one chunk
//     ahead of the state waves.  They prefetch the next chunks' q, k, v and
//     gates from HBM into registers, stage them in double-buffered LDS as
//     MFMA operands, scan the gates (one wave) and run the decay matrix's
//     diagonal blocks (another), then build the intra-chunk weight matrix
//     P = -(tril(Q K^T) .* theta_j gamma_ij) and the chunk-end weights w^M, w^S.
//
// Column split (fp16 path, d >= 64): each 16-row tile is held by two state
// waves, one per half of the key columns of M and S.  Per chunk each of them
// reads out half of the chunk's tokens over all columns, using the partner's
// fp16 fragments of M0 and S0 from LDS, and updates only its own columns,
// using the partner's residual tiles from LDS.  With two waves per SIMD the
// long latency chains of the state and producer work hide each other.
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

#include <atomic>
#include <type_traits>

#include "ttt_mem.h"
#include "gfx950.h"

namespace {


constexpr int kWave = 64;
constexpr int kGR = 16;             // row stride of a diagonal decay block (floats)
constexpr int kGB = 16 * kGR + 4;   // block stride (floats): offsets blocks by one 16-byte slot
constexpr int kLdsBytes = 160 * 1024;

__host__ __device__ constexpr int round_up(int x, int m) { return (x + m - 1) / m * m; }
__host__ __device__ constexpr int cdiv(int x, int m) { return (x + m - 1) / m; }
__host__ __device__ constexpr int cmax(int a, int b) { return a > b ? a : b; }
__host__ __device__ constexpr int cmin(int a, int b) { return a < b ? a : b; }

// LDS service on gfx950 (measured with the bank-conflict counter): 64 banks
// of 4 bytes.  A ds_read_b128 is served in four passes of 16 lanes -- lanes
// 0-31 split by the parity of lane bits 2, 3 and 4, and the same for lanes
// 32-63 -- and a pass is conflict-free when its 16 addresses hit distinct
// 16-byte slots of a 256-byte line.  A ds_write_b128 is served eight
// consecutive lanes at a time against 128 bytes.  The swizzles below permute
// the 16-byte chunks of each row of a row-major fp16 tile (NCH chunks per row)
// so that every MFMA fragment read of interleaved tile rows and every tile
// write is conflict-free.
//
// q and k tiles (also read by the transpose loads of the state update, which
// use half of each 16-byte slot and so run at half rate whatever the layout).
template <int NCH>
__device__ __forceinline__ int swz_qk(int t) {
    if constexpr (NCH >= 16) {
        return ((t & 3) << 1) | (t & 8);
    } else if constexpr (NCH == 8) {
        return (t & 2) | ((t >> 1) & 4);
    } else if constexpr (NCH == 4) {
        return (t >> 2) & 2;
    } else {
        return 0;
    }
}
// Intra-chunk weight tile P (rows of NP fp16).
template <int NCH>
__device__ __forceinline__ int swz_p(int t) {
    if constexpr (NCH == 8) {
        return (t & 3) | ((t >> 1) & 4);
    } else if constexpr (NCH == 4) {
        return ((t >> 1) & 1) | ((t >> 2) & 2);
    } else {
        return 0;
    }
}


// Dense decay matrix rows (NP floats = NP/4 16-byte chunks): the read of a
// P-tile lane (row i = tmap(pb, lr), four columns from tmap(qb, 4 lg)) and
// the build's row-block writes are conflict-free for 16-chunk rows.
template <int NP>
__device__ __forceinline__ int gam_swz(int i) {
    const int sw = (i & 0xb) | ((((i >> 1) ^ (i >> 2)) & 1) << 2);
    return sw & (NP / 4 - 1);
}




// row_newbcast:N -- every lane of a 16-lane row receives lane N of that row
// (every lane has a source, so the instruction needs no old value).
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + N, 0xf, 0xf, false));
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
    void* z;             // float32, or bf16 bits when z_bf16 (rounded to nearest even)
    float* MT;
    float* ST;
    int BH;
    int T;
    int b;
    // Packed variable-length documents (NULL: dense [B, H, T, d]): document s
    // of head h is tokens cu[s] .. cu[s+1]-1 of head h's [T, d] rows, and
    // its state is slot s * H + h.
    const int* cu;
    int H;
    // Chunk-start states for the backward pass (NULL: not written):
    // [B*H][ceil(T/b)][M | S][d][d] for dense sequences; for packed documents
    // [H][tcmax][M | S][d][d], document s of head h from slot h * tcmax + (the
    // chunks of documents 0..s-1).  float32 on the float32 path and fp16 on
    // the fp16-operand path (the precision every later use rounds them to).
    void* ckpt;
    // Gates shared by the tokens of a chunk (dense sequences only): theta,
    // eta, alpha are [B*H][ceil(T/b)] and every token of chunk c uses entry c.
    int chunk_gates;
    int tcmax;   // packed documents: chunk slots per head
    int z_bf16;  // z element type: 0 float32, 1 bf16
    const int* perm;   // packed documents above kLptDocs: their longest-first order (NULL: packing order)
};

// Compile-time geometry of one kernel instance: NS 16-row tiles per
// workgroup, each split over CS state waves by key columns.
template <typename T, int D, int NS, int CS, int NP>
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
    static constexpr int TPB = KG / 16;               // 16-tiles per k-group
    static constexpr int NCW = NC / CS;               // column tiles of one state wave
    static constexpr int NKCW = NKC / CS;             // column k-groups of one state wave
    static constexpr int NTW = NT / CS;               // token tiles read out by one state wave
    static constexpr int NPW = CS == 2 ? 8 : 2;       // producer waves
    static constexpr int NSW = NS * CS;               // state waves
    static constexpr int NWAVE = NSW + NPW;
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
    static constexpr int QUL = cdiv(NQU, NPW * kWave);
    static constexpr int VUL = cdiv(NVU, kWave);
    static constexpr int BUF_BYTES = (2 * NP * LQ + NP * LP + 2 * NP) * (int)sizeof(T) +
                                     (F16 ? NP * LV * 2 : (DS * LKT + RB * LV) * 4);
    static constexpr int XCH_BYTES = CS > 1 ? NS * (2 * NKC * kWave * 16 + NT * kWave * 8) : 0;
    static constexpr int GATE_BYTES = 2 * (2 * NT * kGB + NT * NP * 3 + 2 * NP) * 4 + 4 * (2 * NP + 4) * 4;
    // Packed documents on the pipelined instances run persistent workgroups
    // that walk a table of their (document, head) units, KMAX at most.
    static constexpr bool PIPE = F16 && CS == 2;
    static constexpr int KMAX = PIPE ? 384 : 0;
    static constexpr int UNIT_BYTES = PIPE ? KMAX * 16 + 16 : 0;
    static constexpr int HELP_BYTES = GATE_BYTES + XCH_BYTES + UNIT_BYTES;
    static constexpr int NBUF = (2 * BUF_BYTES + HELP_BYTES + 1024 <= kLdsBytes) ? 2 : 1;
    static constexpr bool PERSIST = PIPE && NBUF == 2;
    // Documents the persistent schedule ranks in LDS: four ints each, and one
    // per unit of the workgroup, in the second chunk buffer, which the
    // schedule borrows before the pipeline starts.
    static constexpr int NMAX_DOCS = cmin(2048, (BUF_BYTES / 4 - KMAX) / 4);
    // The dense decay matrix theta_j gamma_ij of one chunk, when it fits.
    static constexpr int GAM_BYTES = NP * NP * 4;
    static constexpr bool USE_GAM = NBUF * BUF_BYTES + HELP_BYTES + GAM_BYTES + 1024 <= kLdsBytes;
    static_assert(NP % KG == 0, "chunk padding must fill whole k-groups");
    static_assert(D % RB == 0, "row blocks must tile d");
    static_assert(CS == 1 || (F16 && NKC % CS == 0 && NT % CS == 0), "column split needs whole k-groups");
    static_assert(NBUF * BUF_BYTES + HELP_BYTES + 1024 <= kLdsBytes, "LDS budget");
};

template <typename T, int D, int NS, int CS, int NP>
struct Smem {
    using Gm = Geo<T, D, NS, CS, NP>;
    static constexpr bool F16 = Gm::F16;
    struct Buf {
        alignas(16) T q[NP * Gm::LQ];      // q rows (fp16: swizzled chunks)
        alignas(16) T k[NP * Gm::LQ];      // k rows
        alignas(16) T p[NP * Gm::LP];      // -P rows, token dim in fragment order
        alignas(16) T wm[NP];              // w^M (fragment order = token order)
        alignas(16) T ws[NP];              // w^S
        // fp16: raw bf16 v rows [token][row]; float32: k^T rows and -v^T rows.
        alignas(16) uint16_t vb[F16 ? NP * Gm::LV : 1];
        alignas(16) float kt[F16 ? 1 : D * Gm::LKT];
        alignas(16) float vn[F16 ? 1 : Gm::RB * Gm::LV];
    };
    Buf buf[Gm::NBUF];
    // Decay-matrix quantities of one chunk (producers only), double-buffered
    // by chunk parity: the gate waves run two chunks ahead of the state waves.
    struct GateSlot {
        // theta_j gamma_ij and theta_j p_ij on the diagonal 16-blocks, [blk][i][j]
        // with padded rows (kGR floats) and blocks (kGB floats): bank-conflict free.
        alignas(16) float gamd[Gm::NT * kGB];
        alignas(16) float gampd[Gm::NT * kGB];
        alignas(16) float phi[Gm::NT * NP * 3];  // maps from the end of block q to row i [q][i][X,Y,W]
        alignas(16) float gend[NP];              // theta_j gamma at the end of column j's block
        alignas(16) float pend[NP];              // theta_j p at the end of column j's block
    };
    GateSlot gs[2];
    // Gate quantities the state waves read, a ring over four chunks.
    struct ReadGates {
        alignas(16) float av[NP];    // A_i
        alignas(16) float cv[NP];    // c_i
        alignas(16) float scal[4];   // A_n, c_n, E_n
    };
    ReadGates rg[4];
    // Dense decay matrix of the chunk whose P tiles are being built: row i
    // (token) holds theta_j gamma_ij for every j, 16-byte chunks XOR-swizzled
    // by gam_swz(i); blocks above the diagonal stay zero.
    alignas(16) float gam[Gm::USE_GAM ? NP * NP : 4];
    // Column-split exchange between the state waves of one row tile: fp16
    // fragments of M0, S0 per key k-group, and fp16 residual tiles per token tile.
    alignas(16) f16x8 xm[CS > 1 ? NS * Gm::NKC * kWave : 1];
    alignas(16) f16x8 xs[CS > 1 ? NS * Gm::NKC * kWave : 1];
    alignas(16) f16x4 xe[CS > 1 ? NS * Gm::NT * kWave : 1];
    // Persistent packed documents: the workgroup's non-empty units in walk
    // order (first token in the [H, T] rows, length, checkpoint slot of its
    // first chunk, state slot s * H + h), their count, their chunks in all,
    // and the number of empty units.
    WalkUnit units[Gm::KMAX > 0 ? Gm::KMAX : 1];
    int nitems, nunits, nempty;   // build_walk_table's counts, in this order
};

template <typename T, int D, int NS, int CS, int NP>
struct Kernel {
    using Gm = Geo<T, D, NS, CS, NP>;
    using O = Op<T>;
    using G = typename Gm::G;
    using F = typename O::frag;
    using S = Smem<T, D, NS, CS, NP>;
    using Buf = typename S::Buf;
    using GateSlot = typename S::GateSlot;
    using ReadGates = typename S::ReadGates;
    static constexpr bool F16 = Gm::F16;
    static constexpr int NT = Gm::NT, NC = Gm::NC, KG = Gm::KG, NKC = Gm::NKC, NKT = Gm::NKT, DS = Gm::DS;
    static constexpr int LQ = Gm::LQ, LP = Gm::LP, LKT = Gm::LKT, LV = Gm::LV, CB = Gm::CB, RB = Gm::RB;
    static constexpr int NCHQ = Gm::NCHQ, NCHP = Gm::NCHP, TPB = Gm::TPB, NPW = Gm::NPW;
    static constexpr int NCW = Gm::NCW, NKCW = Gm::NKCW, NTW = Gm::NTW;

    // ---- LDS operand access -------------------------------------------------
    // Fragment of k-group s from row t of a q/k tile, lane group g.
    __device__ static F frag_q(const T* base, int t, int s, int g) {
        if constexpr (F16) {
            const int ch = (4 * s + g) ^ swz_qk<NCHQ>(t);
            return *reinterpret_cast<const f16x8*>(base + t * LQ + 8 * ch);
        } else {
            return *reinterpret_cast<const f32x4*>(base + t * LQ + 16 * s + 4 * g);
        }
    }
    __device__ static F frag_p(const T* base, int t, int s, int g) {
        if constexpr (F16) {
            const int ch = (4 * s + g) ^ swz_p<NCHP>(t);
            return *reinterpret_cast<const f16x8*>(base + t * LP + 8 * ch);
        } else {
            return *reinterpret_cast<const f32x4*>(base + t * LP + 16 * s + 4 * g);
        }
    }
    // Store indices x..x+3 (x % 4 == 0) of row t of a P tile (float32 path).
    __device__ static void put_p(T* base, int t, int x, f32x4 v) {
        *reinterpret_cast<f32x4*>(base + t * LP + x) = v;
    }
    // fp16 path: store indices x..x+7 (x % 8 == 0) of row t, one 16-byte chunk.
    __device__ static void put_p8(T* base, int t, int x, f32x4 lo, f32x4 hi) {
        const int ch = (x >> 3) ^ swz_p<NCHP>(t);
        const f16x4 l = cvt4(lo), h = cvt4(hi);
        *reinterpret_cast<f16x8*>(base + t * LP + 8 * ch) = f16x8{l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
    }
    __device__ static F frag_w(const T* w, int s, int g) {
        if constexpr (F16) return *reinterpret_cast<const f16x8*>(w + 32 * s + 8 * g);
        else return *reinterpret_cast<const f32x4*>(w + 16 * s + 4 * g);
    }

    // ---- producers ------------------------------------------------------------
    // Each producer wave PW owns a fixed share of the chunk's 16-byte q/k
    // units (the two gate waves take smaller shares), v rows (one wave), gate
    // work and P tiles, all known at compile time.
    static constexpr int WU = cdiv(Gm::NQU, kWave);   // q (or k) units per chunk in 64-lane rounds
    // q/k rounds of producer PW.  With eight producers the gate waves 0 and 1
    // stage nothing (they build the decay matrix and the chunk-end weights
    // meanwhile) and waves 2..7 split the rounds, the larger shares first;
    // with two, the rounds are halved.
    static constexpr int rounds(int pw) {
        if (NPW == 8) return pw < 2 ? 0 : WU / 6 + (pw - 2 < WU % 6 ? 1 : 0);
        return pw == 0 ? WU / 2 : WU - WU / 2;
    }
    static constexpr int first_round(int pw) { return pw == 0 ? 0 : first_round(pw - 1) + rounds(pw - 1); }
    // v rows: with eight producers split between waves 6 and 7 (which take
    // the smaller q/k shares); with two, on wave 1.
    static constexpr int vrounds(int pw) {
        if (NPW == 8) return pw == 6 ? Gm::VUL / 2 : pw == 7 ? Gm::VUL - Gm::VUL / 2 : 0;
        return pw == NPW - 1 ? Gm::VUL : 0;
    }
    static constexpr int vfirst_of(int pw) { return pw == 0 ? 0 : vfirst_of(pw - 1) + vrounds(pw - 1); }
    template <int PW>
    struct Share {
        static constexpr int first = first_round(PW);
        static constexpr int count = rounds(PW);
        static constexpr int vfirst = vfirst_of(PW);
        static constexpr int vcount = vrounds(PW);
        static constexpr bool has_v = vcount > 0;
    };
    // P tiles: with eight producers, the row tiles of each lower-triangular
    // tile-block pair (one row tile against the pair's column block) are dealt
    // to waves 2..7 and the chunk-end weights go to wave 0; otherwise whole
    // pairs are dealt round-robin and the weights go to the last wave.
    static constexpr int NPAIR = (NT / TPB) * (NT / TPB + 1) / 2;
    static constexpr int kWrowWave = NPW == 8 ? 0 : ((NPAIR % NPW) == 0 ? NPW - 1 : NPAIR % NPW);
    // Decay-matrix blocks of the two gate waves: the blocks below the
    // diagonal alternate, the diagonal copies go to wave 1 (wave 0 also
    // builds the chunk-end weights).
    static constexpr int gam_owner(int bi, int bj, int idx) { return bi == bj ? 1 : (idx & 1); }
    static constexpr int unit_owner(int pair, int hp) {
        return NPW == 8 ? 2 + (pair * TPB + hp) % (NPW - 2) : pair % NPW;
    }
    static constexpr int qumax(int pw) { return pw == NPW ? 0 : cmax(rounds(pw), qumax(pw + 1)); }
    static constexpr int QUMAX = qumax(0);
    struct Prefetch {
        uint4 q[QUMAX > 0 ? QUMAX : 1];
        uint4 k[QUMAX > 0 ? QUMAX : 1];
        uint4 v[Gm::VUL];
        float th, et, al;
    };

    // Issue the global loads of chunk c into registers; nothing here waits for
    // them.  Rows past the chunk's n tokens read as zeros through the bounds,
    // and a chunk past the end of the sequence has n = 0: its loads touch no
    // memory.  Issuing unconditionally keeps the number of loads in flight the
    // same on every path, so waits on an older prefetch set stay partial.
    template <int PW>
    __device__ static void issue(Prefetch& pf, const Params& p, const G* gq, const G* gk, const G* gv,
                                 size_t seq_tok, int seqlen, int row_wg, int c, int lane) {
        using Sh = Share<PW>;
        const int c0 = c * p.b;
        const int n = max(0, min(p.b, seqlen - c0));
        const size_t chunk_off = (seq_tok + c0) * D;
        const uint32_t nbytes = static_cast<uint32_t>(n) * D * sizeof(G);
        const auto rq = make_rsrc(gq + chunk_off, nbytes);
        const auto rk = make_rsrc(gk + chunk_off, nbytes);
#pragma unroll
        for (int kk = 0; kk < Sh::count; ++kk) {
            const int u = (Sh::first + kk) * kWave + lane;
            const int t = u / (D / CB), cb = u % (D / CB);
            const uint32_t off = (static_cast<uint32_t>(t) * D + cb * CB) * sizeof(G);
            pf.q[kk] = buf_load16(rq, off);
            pf.k[kk] = buf_load16(rk, off);
        }
        if constexpr (Sh::has_v) {
            const auto rv = make_rsrc(gv + chunk_off, nbytes);
#pragma unroll
            for (int kk = 0; kk < Sh::vcount; ++kk) {
                const int u = lane + kWave * (Sh::vfirst + kk);
                const int t = u / (RB / CB), rb = u % (RB / CB);
                pf.v[kk] = buf_load16(rv, (static_cast<uint32_t>(t) * D + row_wg + rb * CB) * sizeof(G));
            }
        }
        if constexpr (PW < 2) {
            // Padding tokens read theta = alpha = eta = 0; the gate work maps eta to 1.
            // Chunk-shared gates: every real token reads the chunk's entry.
            uint32_t gbytes = static_cast<uint32_t>(n) * 4, goff = lane * 4;
            size_t gi = seq_tok + c0;
            if (p.chunk_gates) {
                const int nchunks = (p.T + p.b - 1) / p.b;
                gi = (seq_tok / p.T) * nchunks + c0 / p.b;
                gbytes = 4;
                goff = lane < n ? 0u : 4u;
            }
            pf.th = buf_load4(make_rsrc(p.theta + gi, gbytes), goff);
            pf.al = buf_load4(make_rsrc(p.alpha + gi, gbytes), goff);
            pf.et = buf_load4(make_rsrc(p.eta + gi, gbytes), goff);
        }
    }

    // Registers -> LDS chunk buffer.
    template <int PW>
    __device__ static void stage(const Prefetch& pf, Buf& B, int lane) {
        using Sh = Share<PW>;
#pragma unroll
        for (int kk = 0; kk < Sh::count; ++kk) {
            const int u = (Sh::first + kk) * kWave + lane;
            if ((Gm::NQU % kWave) == 0 || u < Gm::NQU) {
                const int t = u / (D / CB), cb = u % (D / CB);
                if constexpr (F16) {
                    const int ch = cb ^ swz_qk<NCHQ>(t);
                    const uint4 rq = pf.q[kk], rk = pf.k[kk];
                    f16x8 hq, hk;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t wq = (&rq.x)[e], wk = (&rk.x)[e];
                        const f16x2 a = cvt2(bf16lo(wq), bf16hi(wq)), b = cvt2(bf16lo(wk), bf16hi(wk));
                        hq[2 * e] = a[0];
                        hq[2 * e + 1] = a[1];
                        hk[2 * e] = b[0];
                        hk[2 * e + 1] = b[1];
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
        if constexpr (Sh::has_v) {
#pragma unroll
            for (int kk = 0; kk < Sh::vcount; ++kk) {
                const int u = lane + kWave * (Sh::vfirst + kk);
                if ((Gm::NVU % kWave) == 0 || u < Gm::NVU) {
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

    // Producer wave 0: gate scan (A, c, E) and the block maps of the decay matrix.
    __device__ static void gate_scan(const Prefetch& pf, GateSlot& gs, ReadGates& rg, int n, int lane) {
        const int l = lane;
        const float et = l < n ? pf.et : 1.f, a = 1.f - pf.al;
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
        if (l < NP) { rg.av[l] = X; rg.cv[l] = Y; }
        if (l == n - 1) { rg.scal[0] = X; rg.scal[1] = Y; rg.scal[2] = W; }
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
                    float* dst = gs.phi + (q * NP + l) * 3;
                    dst[0] = cx; dst[1] = cy; dst[2] = cw;
                    const float ny = cx * BY[q] + cy * BW[q];
                    cx *= BX[q];
                    cw *= BW[q];
                    cy = ny;
                }
            }
        }
    }

    // Producer wave 1: diagonal 16x16 blocks of the decay matrix.  Lane =
    // (block, column j); row i = 16*block + s takes a_i, eta_i from lane s of
    // the same 16-lane row.  The column state starts at (gamma, p) = (1, 1) on
    // its own row: p <- eta_i p + [i == j], gamma <- a_i gamma + p, which is
    // zero above the diagonal (scaled by theta_j, below).
    __device__ static void gate_diag(const Prefetch& pf, GateSlot& gs, int n, int lane) {
        const int l = lane;
        const float th = pf.th, et = l < n ? pf.et : 1.f, a = 1.f - pf.al;
        const int qb = l >> 4, jj = l & 15;
        float ai[16], ei[16];
        ai[0] = row_bcast<0>(a); ei[0] = row_bcast<0>(et);
        ai[1] = row_bcast<1>(a); ei[1] = row_bcast<1>(et);
        ai[2] = row_bcast<2>(a); ei[2] = row_bcast<2>(et);
        ai[3] = row_bcast<3>(a); ei[3] = row_bcast<3>(et);
        ai[4] = row_bcast<4>(a); ei[4] = row_bcast<4>(et);
        ai[5] = row_bcast<5>(a); ei[5] = row_bcast<5>(et);
        ai[6] = row_bcast<6>(a); ei[6] = row_bcast<6>(et);
        ai[7] = row_bcast<7>(a); ei[7] = row_bcast<7>(et);
        ai[8] = row_bcast<8>(a); ei[8] = row_bcast<8>(et);
        ai[9] = row_bcast<9>(a); ei[9] = row_bcast<9>(et);
        ai[10] = row_bcast<10>(a); ei[10] = row_bcast<10>(et);
        ai[11] = row_bcast<11>(a); ei[11] = row_bcast<11>(et);
        ai[12] = row_bcast<12>(a); ei[12] = row_bcast<12>(et);
        ai[13] = row_bcast<13>(a); ei[13] = row_bcast<13>(et);
        ai[14] = row_bcast<14>(a); ei[14] = row_bcast<14>(et);
        ai[15] = row_bcast<15>(a); ei[15] = row_bcast<15>(et);
        if (qb < NT) {
            float* gd = gs.gamd + qb * kGB + jj;
            float* gpd = gs.gampd + qb * kGB + jj;
            // The recurrences are linear, so starting column j at theta_j
            // instead of 1 yields theta_j gamma_ij and theta_j p_ij directly.
            float pp = 0.f, gg = 0.f;
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                pp = s == jj ? th : ei[s] * pp;
                gg = ai[s] * gg + pp;
                gd[s * kGR] = gg;
                gpd[s * kGR] = pp;
            }
            gs.gend[l] = gg;
            gs.pend[l] = pp;
        }
    }

    // theta_j gamma_ij (and, with PE, theta_j p_ij) for 4 consecutive j =
    // jb..jb+3 of one 16-block.  Every candidate is loaded (all addresses are
    // in bounds) and the result selected without branches: lanes of one wave
    // mix diagonal, below-diagonal and above-diagonal blocks, and branches
    // around the loads would serialise their LDS latencies.
    template <bool PE>
    __device__ static void decay4(const GateSlot& sm, int i, int jb, f32x4& L, f32x4& LPe) {
        const int bi = i >> 4, bj = jb >> 4;
        f32x4 ld = *reinterpret_cast<const f32x4*>(sm.gamd + bi * kGB + (i & 15) * kGR + (jb & 15));
        f32x4 gv = *reinterpret_cast<const f32x4*>(sm.gend + jb);
        const float* ph = sm.phi + (bj * NP + i) * 3;   // in bounds for every bj < NT
        float x = ph[0], y = ph[1];
        f32x4 lpd, pv;
        float wv;
        pv = *reinterpret_cast<const f32x4*>(sm.pend + jb);
        if constexpr (PE) {
            lpd = *reinterpret_cast<const f32x4*>(sm.gampd + bi * kGB + (i & 15) * kGR + (jb & 15));
            wv = ph[2];
            asm volatile("" : "+v"(lpd), "+v"(wv));
        }
        asm volatile("" : "+v"(ld), "+v"(gv), "+v"(pv), "+v"(x), "+v"(y));
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const f32x4 lo = x * gv + y * pv;
        L = bi == bj ? ld : (bi > bj ? lo : zero);
        if constexpr (PE) {
            const f32x4 lpo = wv * pv;
            LPe = bi == bj ? lpd : (bi > bj ? lpo : zero);
        }
    }

    // Dense decay matrix from the gate data of one chunk, split over the two
    // gate waves by gam_owner (16x16 blocks on and below the diagonal).
    // Lane (r, c4) writes row 16 bi + r, columns 16 bj + 4 c4 .. + 3: on the
    // diagonal the block recurrence's values, below it the map from the end
    // of block bj to row i applied to the column states at that block end.
    template <int HALF>
    __device__ static void gamma_build(const GateSlot& gs, float* gam, int lane) {
        const int r = lane & 15, c4 = lane >> 4;
        int idx = 0;
#pragma unroll
        for (int bi = 0; bi < NT; ++bi) {
#pragma unroll
            for (int bj = 0; bj < bi; ++bj, ++idx) {
                if (gam_owner(bi, bj, idx) != HALF) continue;
                const int i = 16 * bi + r, j = 16 * bj + 4 * c4;
                const float* ph = gs.phi + (bj * NP + i) * 3;
                const f32x4 gv = *reinterpret_cast<const f32x4*>(gs.gend + j);
                const f32x4 pv = *reinterpret_cast<const f32x4*>(gs.pend + j);
                const f32x4 g = ph[0] * gv + ph[1] * pv;
                *reinterpret_cast<f32x4*>(gam + i * NP + 4 * ((j >> 2) ^ gam_swz<NP>(i))) = g;
            }
        }
#pragma unroll
        for (int bi = 0; bi < NT; ++bi) {
            if (gam_owner(bi, bi, 0) != HALF) continue;
            const int i = 16 * bi + r, j = 16 * bi + 4 * c4;
            const f32x4 g = *reinterpret_cast<const f32x4*>(gs.gamd + bi * kGB + r * kGR + 4 * c4);
            *reinterpret_cast<f32x4*>(gam + i * NP + 4 * ((j >> 2) ^ gam_swz<NP>(i))) = g;
        }
    }

    // Producers: P tiles.  Tile (pb, qb) holds rows i = tmap(pb, .) and
    // columns j = tmap(qb, .); only tiles whose column k-group is not after the
    // row's k-group are ever read.  Producer PW takes the tiles of row block
    // and column block (rbk, cbk) = kTiles[PW] (blocks of TPB tiles), so the q
    // and k fragments of a block are read once for all its tiles.
    template <int PW>
    __device__ static void ptiles(const GateSlot& sm, const float* gam, Buf& B, int lr, int lg) {
        constexpr int NB = NT / TPB;   // k-groups (tile blocks) per chunk
        // Lower-triangular (rbk, cbk) block pairs in order; row tile hp of a
        // pair belongs to producer unit_owner(pair, hp).
#pragma unroll
        for (int rbk = 0; rbk < NB; ++rbk) {
#pragma unroll
            for (int cbk = 0; cbk <= rbk; ++cbk) {
                const int pair = rbk * (rbk + 1) / 2 + cbk;
                bool any = false;
#pragma unroll
                for (int hp = 0; hp < TPB; ++hp) any = any || unit_owner(pair, hp) == PW;
                if (!any) continue;
                F kf[TPB][NKC];
#pragma unroll
                for (int h = 0; h < TPB; ++h)
#pragma unroll
                    for (int s = 0; s < NKC; ++s) kf[h][s] = frag_q(B.k, O::tmap(cbk * TPB + h, lr), s, lg);
#pragma unroll
                for (int hp = 0; hp < TPB; ++hp) {
                    if (unit_owner(pair, hp) != PW) continue;
                    const int pb = rbk * TPB + hp;
                    const int i = O::tmap(pb, lr);
                    F qf[NKC];
#pragma unroll
                    for (int s = 0; s < NKC; ++s) qf[s] = frag_q(B.q, i, s, lg);
                    f32x4 pv[TPB];
#pragma unroll
                    for (int hq = 0; hq < TPB; ++hq) {
                        const int qb = cbk * TPB + hq;
                        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int s = 0; s < NKC; ++s) acc = O::mma(acc, kf[hq][s], qf[s]);
                        const int jb = O::tmap(qb, 4 * lg);   // acc[e] = q_i . k_{jb+e}
                        f32x4 L, LPe;
                        if constexpr (Gm::USE_GAM) {
                            L = *reinterpret_cast<const f32x4*>(gam + i * NP + 4 * ((jb >> 2) ^ gam_swz<NP>(i)));
                        } else {
                            decay4<false>(sm, i, jb, L, LPe);
                        }
                        pv[hq] = -(acc * L);
                    }
                    // The TPB column tiles of a block hold consecutive token columns.
                    if constexpr (F16) put_p8(B.p, i, O::tmap(cbk * TPB, 4 * lg), pv[0], pv[1]);
                    else put_p(B.p, i, O::tmap(cbk * TPB, 4 * lg), pv[0]);
                }
            }
        }
    }
    // Chunk-end weights w^M_j = -theta_j gamma_{n-1,j}, w^S_j = -theta_j p_{n-1,j}; lane = 4 tokens.
    __device__ static void wrow(const GateSlot& sm, Buf& B, int n, int lane) {
        if (lane < NP / 4) {
            f32x4 L, LPe;
            decay4<true>(sm, n - 1, 4 * lane, L, LPe);
            if constexpr (F16) {
                *reinterpret_cast<f16x4*>(B.wm + 4 * lane) = cvt4(-L);
                *reinterpret_cast<f16x4*>(B.ws + 4 * lane) = cvt4(-LPe);
            } else {
                *reinterpret_cast<f32x4*>(B.wm + 4 * lane) = -L;
                *reinterpret_cast<f32x4*>(B.ws + 4 * lane) = -LPe;
            }
        }
    }

    // ---- state waves ------------------------------------------------------
    // -V for token tile tt: lane (lr, lg) gets -v[tmap(tt, 4lg + e)][row r0 + lr].
    __device__ static f32x4 neg_v(const Buf& B, int tt, int r0, int lr, int lg) {
        if constexpr (F16) {
            const int t = O::tmap(tt, 4 * lg + (lr >> 2));
            const i16x4 r = ds_read_tr16(B.vb + t * LV + r0 + 4 * (lr & 3));
            const u32x2 u = __builtin_bit_cast(u32x2, r);
            return f32x4{-bf16lo(u[0]), -bf16hi(u[0]), -bf16lo(u[1]), -bf16hi(u[1])};
        } else {
            return *reinterpret_cast<const f32x4*>(B.vn + (r0 + lr) * LV + 16 * tt + 4 * lg);
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
            const i16x4 lo = ds_read_tr16(B.k + t0 * LQ + 8 * (ch ^ swz_qk<NCHQ>(t0)) + (col & 4));
            const i16x4 hi = ds_read_tr16(B.k + t1 * LQ + 8 * (ch ^ swz_qk<NCHQ>(t1)) + (col & 4));
            const f16x4 l4 = __builtin_bit_cast(f16x4, lo), h4 = __builtin_bit_cast(f16x4, hi);
            return F{l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
        } else {
            return *reinterpret_cast<const f32x4*>(B.kt + (16 * ct + lr) * LKT + 16 * s + 4 * lg);
        }
    }

    // State wave (rho, chi): rows r0..r0+15 of the workgroup block, column
    // tiles chi*NCW.., token tiles chi*NTW.. .  MB/SB hold fp16 fragments of
    // M0, S0 for every key k-group (own ones from registers, the partner's
    // from the exchange).
    struct StateCtx {
        int rho, chi, r0, lr, lg;
    };

    // Phase A: residuals E and readouts (A.M0 q + c.S0 q) of the own token
    // tiles.  MB/SB hold the fp16 fragments of M0, S0 for the own key
    // k-groups; MP/SP receive the partner's from the exchange.
    __device__ static void phaseA(const StateCtx& x, const Buf& B, const ReadGates& rg, S& sm, const F* MB,
                                  const F* SB, f32x4* E,
                                  f32x4* Zp) {
        F MP[NKCW], SP[NKCW];
        const int pchi = x.chi ^ 1;
        if constexpr (CS > 1) {
#pragma unroll
            for (int sw = 0; sw < NKCW; ++sw) {
                const int s = pchi * NKCW + sw;
                MP[sw] = sm.xm[(x.rho * NKC + s) * kWave + x.lr + 16 * x.lg];
                SP[sw] = sm.xs[(x.rho * NKC + s) * kWave + x.lr + 16 * x.lg];
            }
        }
#pragma unroll
        for (int tw = 0; tw < NTW; ++tw) {
            const int tt = x.chi * NTW + tw;
            const int t = O::tmap(tt, x.lr);
            E[tw] = neg_v(B, tt, x.r0, x.lr, x.lg);
            f32x4 za = {0.f, 0.f, 0.f, 0.f}, zc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sw = 0; sw < NKCW; ++sw) {
                const int s = x.chi * NKCW + sw;   // own key k-group
                E[tw] = O::mma(E[tw], frag_q(B.k, t, s, x.lg), MB[sw]);
                const F bq = frag_q(B.q, t, s, x.lg);
                za = O::mma(za, MB[sw], bq);
                zc = O::mma(zc, SB[sw], bq);
            }
            if constexpr (CS > 1) {
#pragma unroll
                for (int sw = 0; sw < NKCW; ++sw) {
                    const int s = pchi * NKCW + sw;   // partner's key k-group
                    E[tw] = O::mma(E[tw], frag_q(B.k, t, s, x.lg), MP[sw]);
                    const F bq = frag_q(B.q, t, s, x.lg);
                    za = O::mma(za, MP[sw], bq);
                    zc = O::mma(zc, SP[sw], bq);
                }
            }
            Zp[tw] = rg.av[t] * za + rg.cv[t] * zc;
        }
        if constexpr (CS > 1) {
#pragma unroll
            for (int tw = 0; tw < NTW; ++tw) {
                const int tt = x.chi * NTW + tw;
                sm.xe[(x.rho * NT + tt) * kWave + x.lr + 16 * x.lg] = cvt4(E[tw]);
            }
        }
    }

    // Phase B: intra-chunk term and store of z for the own token tiles, then
    // the update of the own columns of M and S.
    __device__ static void phaseB(const StateCtx& x, const Buf& B, const ReadGates& rg, S& sm, f32x4* Macc,
                                  f32x4* Sacc, F* MB, F* SB,
                                  const f32x4* E, f32x4* Zp, __amdgpu_buffer_rsrc_t rz, uint32_t zcol, bool zb) {
        // (MB, SB: the own key k-groups, refreshed from the updated state at the end.)
        F EB[NKT];
        if constexpr (CS > 1) {
#pragma unroll
            for (int s = 0; s < NKT; ++s) {
                const f16x4 lo = sm.xe[(x.rho * NT + 2 * s) * kWave + x.lr + 16 * x.lg];
                const f16x4 hi = sm.xe[(x.rho * NT + 2 * s + 1) * kWave + x.lr + 16 * x.lg];
                EB[s] = F{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
        } else {
#pragma unroll
            for (int s = 0; s < NKT; ++s) EB[s] = O::template from_acc<NT>(E, s);
        }
#pragma unroll
        for (int tw = 0; tw < NTW; ++tw) {
            const int tt = x.chi * NTW + tw;
            const int t = O::tmap(tt, x.lr);
#pragma unroll
            for (int s = 0; s < NKT; ++s)
                if (s <= tt / TPB) Zp[tw] = O::mma(Zp[tw], EB[s], frag_p(B.p, t, s, x.lg));
            store_out4(Zp[tw], rz, static_cast<uint32_t>(t) * D + zcol, zb);   // rows >= n dropped
        }
        F WMB[NKT], WSB[NKT];
#pragma unroll
        for (int s = 0; s < NKT; ++s) {
            WMB[s] = EB[s] * frag_w(B.wm, s, x.lg);
            WSB[s] = EB[s] * frag_w(B.ws, s, x.lg);
        }
        const float An = rg.scal[0], Cn = rg.scal[1], En = rg.scal[2];
#pragma unroll
        for (int cw = 0; cw < NCW; ++cw) {
            const int ct = x.chi * NCW + cw;
            Macc[cw] = An * Macc[cw] + Cn * Sacc[cw];
            Sacc[cw] = En * Sacc[cw];
#pragma unroll
            for (int s = 0; s < NKT; ++s) {
                const F a = kt_frag(B, ct, s, x.lr, x.lg);
                Macc[cw] = O::mma(Macc[cw], a, WMB[s]);
                Sacc[cw] = O::mma(Sacc[cw], a, WSB[s]);
            }
        }
        own_frags(x, sm, Macc, Sacc, MB, SB);
    }

    // ---- column-split state waves (fp16): software-pipelined phases --------
    // Every LDS operand stream of a state wave has one per-lane base address,
    // computed once (buffer 0, the wave's first own token tile) and hidden
    // from the optimizer; each access adds a compile-time offset for the
    // buffer, the token tile, the k-group or the array.  The phases issue the
    // loads of the next k-group (column tile) before the products of the
    // current one, so LDS latency overlaps the matrix cores instead of
    // sitting between each load and its product.
    struct Lanes {
        uint32_t qk[NKC];              // q fragments, k-groups in processing order (own first)
        uint32_t kt[cmax(NCW / 2, 1)]; // transposed k reads, per pair of own column tiles
        uint32_t v;                    // transposed v reads
        uint32_t p[NKT];               // P fragments per token k-group
        uint32_t w;                    // w^M fragments (w^S at a fixed offset)
        uint32_t xp, xo;               // partner's / own M0 fragments in the exchange (S0 at a fixed offset)
        uint32_t xe, xeo;              // residual tiles: all of the row tile / own
        uint32_t g;                    // A_i of the wave's first token in gate slot 0 (c_i at a fixed offset)
    };
    static constexpr int rowoff(int tw) { return 32 * (tw >> 1) + 4 * (tw & 1); }
    static constexpr uint32_t kBufB = sizeof(Buf);
    static constexpr uint32_t kOffQ = offsetof(Buf, q), kOffK = offsetof(Buf, k), kOffP = offsetof(Buf, p);
    static constexpr uint32_t kOffWM = offsetof(Buf, wm), kOffWS = offsetof(Buf, ws), kOffV = offsetof(Buf, vb);
    static constexpr uint32_t kOffXS = offsetof(S, xs) - offsetof(S, xm);
    static constexpr uint32_t kGateB = sizeof(ReadGates);
    static constexpr uint32_t kOffCV = offsetof(ReadGates, cv) - offsetof(ReadGates, av);

    __device__ static Lanes lanes(const StateCtx& x, S& sm) {
        static_assert(F16 && CS == 2 && NTW <= 2 && NCW % 2 == 0 && NCHQ >= 8, "pipelined phases: fp16 column split");
        static_assert(kBufB + kOffK + 2 * 4 * LQ < 65536 && kBufB + 8 + 2 * (32 * (NKT - 1) + 4) * LQ < 65536,
                      "LDS offsets must fit 16 bits");
        static_assert(kBufB + kOffWS - kOffWM + 64 * NKT < 65536 && kBufB + 8 * LP < 65536, "LDS offsets");
        Lanes a;
        const int pchi = x.chi ^ 1;
        const int t = O::tmap(x.chi * NTW, x.lr);   // token of the wave's first own tile, row lr
        const uint32_t b0 = lds_addr(&sm.buf[0]);
#pragma unroll
        for (int j = 0; j < NKC; ++j) {
            const int s = j < NKCW ? x.chi * NKCW + j : pchi * NKCW + (j - NKCW);
            a.qk[j] = opaque(b0 + 2 * (t * LQ + 8 * ((4 * s + x.lg) ^ swz_qk<NCHQ>(t))));
        }
        const int tk = 8 * x.lg + (x.lr >> 2);
#pragma unroll
        for (int h = 0; h < NCW / 2; ++h) {
            const int ch = 4 * ((x.chi * NCW) / 2 + h) + (x.lr & 3);
            a.kt[h] = opaque(b0 + kOffK + 2 * (tk * LQ + 8 * (ch ^ swz_qk<NCHQ>(tk))));
        }
        const int tv = O::tmap(x.chi * NTW, 4 * x.lg + (x.lr >> 2));
        a.v = opaque(b0 + kOffV + 2 * (tv * LV + x.r0 + 4 * (x.lr & 3)));
#pragma unroll
        for (int s2 = 0; s2 < NKT; ++s2)
            a.p[s2] = opaque(b0 + kOffP + 2 * (t * LP + 8 * ((4 * s2 + x.lg) ^ swz_p<NCHP>(t))));
        a.w = opaque(b0 + kOffWM + 16 * x.lg);
        a.xp = opaque(lds_addr(&sm.xm[(x.rho * NKC + pchi * NKCW) * kWave + x.lr + 16 * x.lg]));
        a.xo = opaque(lds_addr(&sm.xm[(x.rho * NKC + x.chi * NKCW) * kWave + x.lr + 16 * x.lg]));
        a.xe = opaque(lds_addr(&sm.xe[x.rho * NT * kWave + x.lr + 16 * x.lg]));
        a.xeo = opaque(lds_addr(&sm.xe[(x.rho * NT + x.chi * NTW) * kWave + x.lr + 16 * x.lg]));
        a.g = opaque(lds_addr(&sm.rg[0].av[t]));
        return a;
    }

    // Phase A (pipelined): E = K M0^T - V and Z = A.(M0 Q^T) + c.(S0 Q^T) for
    // the own token tiles over all key k-groups (own fragments from registers,
    // the partner's from the exchange); the residual tiles go to the exchange.
    template <int BI>
    __device__ static void phaseA2(const Lanes& a, uint32_t gs, uint32_t gsc, const F* MB, const F* SB, f32x4* E,
                                   f32x4* Zp, f32x4* Macc, f32x4* Sacc) {
        constexpr uint32_t BO = BI * kBufB;
        F kf[2][NTW], qf[2][NTW], MP[NKCW], SP[NKCW];
        i16x4 vr[NTW];
        float av[NTW], cv[NTW];
        auto load = [&](int j, int slot) {
#pragma unroll
            for (int tw = 0; tw < NTW; ++tw) {
                kf[slot][tw] = lds_load<F>(a.qk[j] + BO + kOffK + 2 * rowoff(tw) * LQ);
                qf[slot][tw] = lds_load<F>(a.qk[j] + BO + kOffQ + 2 * rowoff(tw) * LQ);
            }
        };
#pragma unroll
        for (int tw = 0; tw < NTW; ++tw) vr[tw] = ds_read_tr16_at(a.v + BO + 2 * rowoff(tw) * LV);
        load(0, 0);
#pragma unroll
        for (int sw = 0; sw < NKCW; ++sw) {
            MP[sw] = lds_load<F>(a.xp + 16 * kWave * sw);
            SP[sw] = lds_load<F>(a.xp + kOffXS + 16 * kWave * sw);
        }
#pragma unroll
        for (int tw = 0; tw < NTW; ++tw) {
            av[tw] = lds_load<float>(gs + 4 * rowoff(tw));
            cv[tw] = lds_load<float>(gs + kOffCV + 4 * rowoff(tw));
        }
        f32x4 za[NTW], zc[NTW];
#pragma unroll
        for (int j = 0; j < NKC; ++j) {
            if (j + 1 < NKC) load(j + 1, (j + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
            if (j == 0) {
#pragma unroll
                for (int tw = 0; tw < NTW; ++tw) {
                    const u32x2 u = __builtin_bit_cast(u32x2, vr[tw]);
                    E[tw] = f32x4{-bf16lo(u[0]), -bf16hi(u[0]), -bf16lo(u[1]), -bf16hi(u[1])};
                    za[tw] = f32x4{0.f, 0.f, 0.f, 0.f};
                    zc[tw] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
            const F& Mj = j < NKCW ? MB[j] : MP[j - NKCW];
            const F& Sj = j < NKCW ? SB[j] : SP[j - NKCW];
#pragma unroll
            for (int tw = 0; tw < NTW; ++tw) {
                E[tw] = O::mma(E[tw], kf[j & 1][tw], Mj);
                za[tw] = O::mma(za[tw], Mj, qf[j & 1][tw]);
                zc[tw] = O::mma(zc[tw], Sj, qf[j & 1][tw]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int tw = 0; tw < NTW; ++tw) {
            Zp[tw] = av[tw] * za[tw] + cv[tw] * zc[tw];
            lds_store<f16x4>(a.xeo + 8 * kWave * tw, cvt4(E[tw]));
        }
        // Decay of the own state for the carry (M0, S0 entered the products
        // above through their fp16 fragments; this phase has slack).
        const f32x4 sc = lds_load<f32x4>(gsc);   // A_n, c_n, E_n (the same address in every lane)
#pragma unroll
        for (int cw = 0; cw < NCW; ++cw) {
            Macc[cw] = sc[0] * Macc[cw] + sc[1] * Sacc[cw];
            Sacc[cw] = sc[2] * Sacc[cw];
        }
    }

    // Phase B (pipelined): the intra-chunk term and the store of z for the own
    // token tiles, then the update of the own (already decayed) columns
    // with the transposed k reads of the next column tile in flight.  The
    // intra-chunk products run over every token k-group: the blocks of P
    // above its diagonal are never written and stay zero.
    // FRAGS: end with the next chunk's fragments (frags2); the persistent walk
    // calls frags2 itself, after any switch to the next document.
    template <int BI, bool FRAGS = true>
    __device__ static void phaseB2(const Lanes& a, f32x4* Macc, f32x4* Sacc, F* MB, F* SB, f32x4* Zp,
                                   __amdgpu_buffer_rsrc_t rz, uint32_t zoff, bool zb) {
        constexpr uint32_t BO = BI * kBufB;
        f16x4 eb[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) eb[tt] = lds_load<f16x4>(a.xe + 8 * kWave * tt);
        F pfr[NTW][NKT];
#pragma unroll
        for (int tw = 0; tw < NTW; ++tw)
#pragma unroll
            for (int s = 0; s < NKT; ++s) pfr[tw][s] = lds_load<F>(a.p[s] + BO + 2 * rowoff(tw) * LP);
        F wmf[NKT], wsf[NKT];
#pragma unroll
        for (int s = 0; s < NKT; ++s) {
            wmf[s] = lds_load<F>(a.w + BO + 64 * s);
            wsf[s] = lds_load<F>(a.w + BO + (kOffWS - kOffWM) + 64 * s);
        }
        F ktf[2][NKT];
        auto load_kt = [&](int cw, int slot) {
#pragma unroll
            for (int s = 0; s < NKT; ++s) {
                const uint32_t b = a.kt[cw >> 1] + BO + 8 * (cw & 1) + 2 * 32 * s * LQ;
                const i16x4 lo = ds_read_tr16_at(b);
                const i16x4 hi = ds_read_tr16_at(b + 2 * 4 * LQ);
                const f16x4 l4 = __builtin_bit_cast(f16x4, lo), h4 = __builtin_bit_cast(f16x4, hi);
                ktf[slot][s] = F{l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
            }
        };
        load_kt(0, 0);
        __builtin_amdgcn_sched_barrier(0);
        F EB[NKT];
#pragma unroll
        for (int s = 0; s < NKT; ++s) {
            const f16x4 lo = eb[2 * s], hi = eb[2 * s + 1];
            EB[s] = F{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int tw = 0; tw < NTW; ++tw) {
#pragma unroll
            for (int s = 0; s < NKT; ++s) Zp[tw] = O::mma(Zp[tw], EB[s], pfr[tw][s]);
        }
        F WMB[NKT], WSB[NKT];
#pragma unroll
        for (int s = 0; s < NKT; ++s) {
            WMB[s] = EB[s] * wmf[s];
            WSB[s] = EB[s] * wsf[s];
        }
#pragma unroll
        for (int tw = 0; tw < NTW; ++tw) store_out4(Zp[tw], rz, zoff + rowoff(tw) * D, zb);   // rows >= n dropped
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int cw = 0; cw < NCW; ++cw) {
            if (cw + 1 < NCW) load_kt(cw + 1, (cw + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < NKT; ++s) {
                Macc[cw] = O::mma(Macc[cw], ktf[cw & 1][s], WMB[s]);
                Sacc[cw] = O::mma(Sacc[cw], ktf[cw & 1][s], WSB[s]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (FRAGS) frags2(a, Macc, Sacc, MB, SB);
    }

    // fp16 fragments of the own columns of M, S for the next chunk, and their
    // copy in the exchange for the partner wave.
    __device__ static void frags2(const Lanes& a, const f32x4* Macc, const f32x4* Sacc, F* MB, F* SB) {
#pragma unroll
        for (int sw = 0; sw < NKCW; ++sw) {
            MB[sw] = O::template from_acc<NCW>(Macc, sw);
            SB[sw] = O::template from_acc<NCW>(Sacc, sw);
            lds_store<F>(a.xo + 16 * kWave * sw, MB[sw]);
            lds_store<F>(a.xo + kOffXS + 16 * kWave * sw, SB[sw]);
        }
    }

    // fp16 fragments of the own columns of M, S (and their copy for the partner).
    __device__ static void own_frags(const StateCtx& x, S& sm, const f32x4* Macc, const f32x4* Sacc, F* MB, F* SB) {
#pragma unroll
        for (int sw = 0; sw < NKCW; ++sw) {
            MB[sw] = O::template from_acc<NCW>(Macc, sw);
            SB[sw] = O::template from_acc<NCW>(Sacc, sw);
            if constexpr (CS > 1) {
                const int s = x.chi * NKCW + sw;
                sm.xm[(x.rho * NKC + s) * kWave + x.lr + 16 * x.lg] = MB[sw];
                sm.xs[(x.rho * NKC + s) * kWave + x.lr + 16 * x.lg] = SB[sw];
            }
        }
    }
};

// One producer wave's loop (role PW): the same barriers as the state waves.
template <typename T, int D, int NS, int CS, int NP, int PW>
__device__ __forceinline__ void producer_loop_impl(const Params& p, typename Kernel<T, D, NS, CS, NP>::S& sm,
                                                   size_t seq_tok, int seqlen, int row_wg, int nch, int lane) {
    using Gm = Geo<T, D, NS, CS, NP>;
    using K = Kernel<T, D, NS, CS, NP>;
    using G = typename Gm::G;
    const int lr = lane & 15, lg = lane >> 4;
    // Issue priority: the serial gate work first, then the state waves, then
    // the P tiles and staging (the state waves' priority is set in the kernel).
    __builtin_amdgcn_s_setprio(PW < 2 ? 3 : 1);
    const int b = p.b;
    auto chunk_n = [&](int c) { return min(b, seqlen - c * b); };
    const G* __restrict__ gq = static_cast<const G*>(p.q);
    const G* __restrict__ gk = static_cast<const G*>(p.k);
    const G* __restrict__ gv = static_cast<const G*>(p.v);
    auto prepare = [&](typename K::Buf& B, const typename K::Prefetch& pf) {   // stage a chunk
        K::template stage<PW>(pf, B, lane);
    };
    auto gates = [&](int c, const typename K::Prefetch& pf) {   // gate quantities of chunk c
        if constexpr (PW == 0) K::gate_scan(pf, sm.gs[c & 1], sm.rg[c & 3], chunk_n(c), lane);
        if constexpr (PW == 1) K::gate_diag(pf, sm.gs[c & 1], chunk_n(c), lane);
    };
    // Decay matrix and chunk-end weights of chunk c (from its gate data),
    // one phase before its P tiles.
    auto build = [&](int c, typename K::Buf& B) {
        if constexpr (Gm::USE_GAM) {
            if constexpr (PW == 0) K::template gamma_build<0>(sm.gs[c & 1], sm.gam, lane);
            if constexpr (PW == 1) K::template gamma_build<1>(sm.gs[c & 1], sm.gam, lane);
            if constexpr (PW == K::kWrowWave) K::wrow(sm.gs[c & 1], B, chunk_n(c), lane);
        }
    };
    auto finish = [&](int c, typename K::Buf& B) {    // P tiles of chunk c
        K::template ptiles<PW>(sm.gs[c & 1], sm.gam, B, lr, lg);
        if constexpr (!Gm::USE_GAM && PW == K::kWrowWave) K::wrow(sm.gs[c & 1], B, chunk_n(c), lane);
    };
    auto issue = [&](int c, typename K::Prefetch& pf) {
        K::template issue<PW>(pf, p, gq, gk, gv, seq_tok, seqlen, row_wg, c, lane);
    };
    if constexpr (Gm::NBUF == 2) {
        // Two register sets of prefetched chunks (even and odd chunks): the
        // loads of chunk c + 3 are issued while chunk c + 1 is staged, two
        // chunk periods before use.  The gate quantities run one chunk further
        // ahead, in the second phase, so that the serial gate work never sits
        // between the staging of a chunk and its P tiles.
        typename K::Prefetch pf0, pf1;
        issue(0, pf0);
        issue(1, pf1);
        if (nch > 0) {
            prepare(sm.buf[0], pf0);
            gates(0, pf0);
        }
        issue(2, pf0);
        __syncthreads();
        if (nch > 0) build(0, sm.buf[0]);
        if (nch > 1) gates(1, pf1);
        __syncthreads();
        if (nch > 0) finish(0, sm.buf[0]);
        __syncthreads();
        // Step c (the state waves consume chunk c): stage chunk c + 1 from cur
        // into B and build its decay matrix, then its P tiles and the gate
        // quantities of chunk c + 2 (held in nxt).
        auto step = [&](int c, typename K::Prefetch& cur, const typename K::Prefetch& nxt, typename K::Buf& B) {
            if (c + 1 < nch) {
                prepare(B, cur);
                build(c + 1, B);
            }
            issue(c + 3, cur);
            __syncthreads();
            if (c + 1 < nch) finish(c + 1, B);
            if (c + 2 < nch) gates(c + 2, nxt);
            __syncthreads();
        };
        for (int c = 0; c < nch; c += 2) {
            step(c, pf1, pf0, sm.buf[1]);
            if (c + 1 < nch) step(c + 1, pf0, pf1, sm.buf[0]);
        }
    } else {
        typename K::Prefetch pf;
        for (int c = 0; c < nch; ++c) {
            issue(c, pf);
            prepare(sm.buf[0], pf);
            gates(c, pf);
            __syncthreads();
            build(c, sm.buf[0]);
            __syncthreads();
            finish(c, sm.buf[0]);
            __syncthreads();
            __syncthreads();
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------------------
// Packed documents on persistent workgroups.
//
// One workgroup launch per (document, head, row block) pays the chunk
// pipeline's fill (loads, staging, gate scan, decay matrix and P tiles ahead
// of the first chunk) and its drain every time, several chunk periods for a
// document of a few chunks.  Here about one workgroup per CU walks many
// documents as one stream of chunks: the producers keep running ahead across
// document boundaries, and the state waves store a document's final state and
// take the next one's initial state between the update of its last chunk and
// the fragments of the next chunk.  Each document is still computed from its
// own state and chunked from its own first token ("5.1.1 · TTT layers 与 fast
// weights", section 1.2, packed documents: the state resets at every document
// boundary), exactly as one launch per document computes it.
//
// Units u = (rank, head), documents ranked longest first (ties by index), go
// to workgroup lanes: u = x + 8 (v + k V), k = 0, 1, ..., where x is the
// workgroup id mod 8 (its XCD) and the NRB row blocks of lane (x, v) are NRB
// workgroups of that XCD, so the row blocks of a unit share one L2.  Longest
// first and dealt round-robin, every workgroup gets a similar mix of lengths.
// ---------------------------------------------------------------------------
// A walk position: unit k of the workgroup's table, the first token of its
// current chunk in the [H, T] rows, the tokens left from there, the chunk's
// checkpoint slot and the unit's state slot.  Past the last unit rem = 0.
struct Cursor {
    int k, tok, rem, ck, bh;
};

template <typename Sm>
__device__ __forceinline__ void cursor_at(Cursor& q, const Sm& sm, int k, int nu) {
    q.k = k;
    if (k < nu) {
        const auto u = sm.units[k];
        q.tok = __builtin_amdgcn_readfirstlane(u.tok0);
        q.rem = __builtin_amdgcn_readfirstlane(u.len);
        q.ck = __builtin_amdgcn_readfirstlane(u.ck0);
        q.bh = __builtin_amdgcn_readfirstlane(u.bh);
    } else {
        q.tok = 0;
        q.rem = 0;
        q.ck = 0;
        q.bh = 0;
    }
}

// Next chunk: within the unit, or the next unit's first.
template <typename Sm>
__device__ __forceinline__ void cursor_next(Cursor& q, const Sm& sm, int nu, int b) {
    if (q.rem > b) {
        q.tok += b;
        q.rem -= b;
        q.ck += 1;
    } else {
        cursor_at(q, sm, q.k + 1, nu);
    }
}

// The workgroup's table of non-empty units (build_walk_table, with the second
// chunk buffer as its scratch) and its chunk count.  Empty documents get their
// final state (the initial one) here; the buffer is cleared again before the
// pipeline starts.
template <typename T, int D, int NS, int CS, int NP>
__device__ __forceinline__ int packed_schedule(const Params& p, typename Kernel<T, D, NS, CS, NP>::S& sm, int x8,
                                               int v, int V, int row_wg, int& nu) {
    using Gm = Geo<T, D, NS, CS, NP>;
    constexpr int NTH = kWave * Gm::NWAVE;
    const int tid = threadIdx.x;
    const int N = p.BH / p.H;
    int* temp = reinterpret_cast<int*>(&sm.buf[1]);
    build_walk_table<NTH, Gm::KMAX>(p.cu, N, p.H, p.T, p.b, p.ckpt != nullptr, p.tcmax, temp,
                                    sm.units, &sm.nitems, x8, v, V);
    const int empties = sm.nempty;
    const int* tempty = temp + 4 * N;
    // The final state of an empty document is its initial state (rows of this row block).
    if (empties > 0 && (p.MT || p.ST)) {
        constexpr int Q = D / 4;   // float4 per row
        for (int e = 0; e < empties; ++e) {
            const size_t base = static_cast<size_t>(tempty[e]) * D * D + static_cast<size_t>(row_wg) * D;
            for (int i = tid; i < Gm::RB * Q; i += NTH) {
                const size_t off = base + static_cast<size_t>(i / Q) * D + 4 * (i % Q);
                const f32x4 zero{0.f, 0.f, 0.f, 0.f};
                if (p.MT) *reinterpret_cast<f32x4*>(p.MT + off) = p.M0 ? *reinterpret_cast<const f32x4*>(p.M0 + off) : zero;
                if (p.ST) *reinterpret_cast<f32x4*>(p.ST + off) = p.S0 ? *reinterpret_cast<const f32x4*>(p.S0 + off) : zero;
            }
        }
        __syncthreads();
    }
    for (int i = tid; i < 4 * N + Gm::KMAX; i += NTH) temp[i] = 0;
    __syncthreads();
    nu = __builtin_amdgcn_readfirstlane(sm.nunits);
    return __builtin_amdgcn_readfirstlane(sm.nitems);
}

// One producer wave's walk over the workgroup's chunks (role PW): the chunk
// pipeline of producer_loop_impl with chunk c of a sequence replaced by item j
// of the stream.  The loads run three items ahead through a cursor; the
// lengths of the four newest items stay in one register (8 bits each).
template <typename T, int D, int NS, int CS, int NP, int PW>
__device__ __forceinline__ void producer_packed_impl(const Params& p, typename Kernel<T, D, NS, CS, NP>::S& sm,
                                                     int row_wg, int nu, int J, int lane) {
    using Gm = Geo<T, D, NS, CS, NP>;
    using K = Kernel<T, D, NS, CS, NP>;
    using G = typename Gm::G;
    static_assert(Gm::NBUF == 2, "pipelined instances only");
    const int lr = lane & 15, lg = lane >> 4;
    __builtin_amdgcn_s_setprio(PW < 2 ? 3 : 1);
    const int b = p.b;
    const G* __restrict__ gq = static_cast<const G*>(p.q);
    const G* __restrict__ gk = static_cast<const G*>(p.k);
    const G* __restrict__ gv = static_cast<const G*>(p.v);
    Cursor ci;
    cursor_at(ci, sm, 0, nu);
    uint32_t nring = 0;
    int ji = 0;
    // Items past the last one have n = 0: their loads touch no memory.
    auto issue = [&](typename K::Prefetch& pf) {
        K::template issue<PW>(pf, p, gq, gk, gv, static_cast<size_t>(ci.tok), ci.rem, row_wg, 0, lane);
        const uint32_t n = static_cast<uint32_t>(max(0, min(b, ci.rem)));
        const int sh = 8 * (ji & 3);
        nring = (nring & ~(0xffu << sh)) | (n << sh);
        ++ji;
        cursor_next(ci, sm, nu, b);
    };
    auto nof = [&](int j) { return static_cast<int>((nring >> (8 * (j & 3))) & 0xffu); };
    auto gates = [&](int j, const typename K::Prefetch& pf) {
        if constexpr (PW == 0) K::gate_scan(pf, sm.gs[j & 1], sm.rg[j & 3], nof(j), lane);
        if constexpr (PW == 1) K::gate_diag(pf, sm.gs[j & 1], nof(j), lane);
    };
    auto build = [&](int j, typename K::Buf& B) {
        if constexpr (Gm::USE_GAM) {
            if constexpr (PW == 0) K::template gamma_build<0>(sm.gs[j & 1], sm.gam, lane);
            if constexpr (PW == 1) K::template gamma_build<1>(sm.gs[j & 1], sm.gam, lane);
            if constexpr (PW == K::kWrowWave) K::wrow(sm.gs[j & 1], B, nof(j), lane);
        }
    };
    auto finish = [&](int j, typename K::Buf& B) {
        K::template ptiles<PW>(sm.gs[j & 1], sm.gam, B, lr, lg);
        if constexpr (!Gm::USE_GAM && PW == K::kWrowWave) K::wrow(sm.gs[j & 1], B, nof(j), lane);
    };
    typename K::Prefetch pf0, pf1;
    issue(pf0);
    issue(pf1);
    if (J > 0) {
        K::template stage<PW>(pf0, sm.buf[0], lane);
        gates(0, pf0);
    }
    issue(pf0);
    __syncthreads();
    if (J > 0) build(0, sm.buf[0]);
    if (J > 1) gates(1, pf1);
    __syncthreads();
    if (J > 0) finish(0, sm.buf[0]);
    __syncthreads();
    auto step = [&](int j, typename K::Prefetch& cur, const typename K::Prefetch& nxt, typename K::Buf& B) {
        if (j + 1 < J) {
            K::template stage<PW>(cur, B, lane);
            build(j + 1, B);
        }
        issue(cur);
        __syncthreads();
        if (j + 1 < J) finish(j + 1, B);
        if (j + 2 < J) gates(j + 2, nxt);
        __syncthreads();
    };
    for (int j = 0; j < J; j += 2) {
        step(j, pf1, pf0, sm.buf[1]);
        if (j + 1 < J) step(j + 1, pf0, pf1, sm.buf[0]);
    }
}

template <typename T, int D, int NS, int CS, int NP>
__global__ __launch_bounds__(kWave * (NS * CS + 8)) void linear_memory_fwd_packed(const Params p) {
    using Gm = Geo<T, D, NS, CS, NP>;
    using K = Kernel<T, D, NS, CS, NP>;
    using O = Op<T>;
    using F = typename O::frag;
    static_assert(Gm::PERSIST, "persistent walk: pipelined instances only");
    constexpr int NSW = Gm::NSW;

    __shared__ __attribute__((aligned(16))) typename K::S sm;

    const int tid = threadIdx.x;
    const int w = tid / kWave;
    const int lane = tid % kWave;
    const int lr = lane & 15;
    const int lg = lane >> 4;
    const int V = gridDim.x / (8 * Gm::NRB);
    const int x8 = blockIdx.x % 8, m = blockIdx.x / 8;
    const int rb = m % Gm::NRB, v = m / Gm::NRB;
    const int b = p.b;
    const int row_wg = rb * Gm::RB;

    {
        uint32_t* words = reinterpret_cast<uint32_t*>(&sm);
        for (int i = tid; i < static_cast<int>(sizeof(sm) / 4); i += kWave * Gm::NWAVE) words[i] = 0u;
    }
    __syncthreads();
    int nu = 0;
    const int J = packed_schedule<T, D, NS, CS, NP>(p, sm, x8, v, V, row_wg, nu);

    if (w < NSW) {
        // ===================== state wave =====================
        typename K::StateCtx x;
        __builtin_amdgcn_s_setprio(2);
        x.rho = w / CS;
        x.chi = w % CS;
        x.r0 = 16 * x.rho;
        x.lr = lr;
        x.lg = lg;
        const int row = row_wg + x.r0;
        f32x4 Macc[Gm::NCW], Sacc[Gm::NCW];
        Cursor cs;
        cursor_at(cs, sm, 0, nu);
        auto state_off = [&]() { return static_cast<size_t>(cs.bh) * D * D + static_cast<size_t>(row + lr) * D; };
        // The initial state of unit cs (zeros past the last unit).  The loads
        // are waited for here: a wait left for the fragments after the switch
        // would sit on every chunk's path and also wait for its z stores (the
        // vector-memory counter counts stores too).
        auto load_state = [&]() {
            const f32x4 zero{0.f, 0.f, 0.f, 0.f};
            if (cs.k < nu && (p.M0 || p.S0)) {
                const size_t so = state_off();
#pragma unroll
                for (int cw = 0; cw < Gm::NCW; ++cw) {
                    const int col = O::tmap(x.chi * Gm::NCW + cw, 4 * lg);
                    const bool ok = col < D;
                    Macc[cw] = (p.M0 && ok) ? *reinterpret_cast<const f32x4*>(p.M0 + so + col) : zero;
                    Sacc[cw] = (p.S0 && ok) ? *reinterpret_cast<const f32x4*>(p.S0 + so + col) : zero;
                }
                __builtin_amdgcn_s_waitcnt(kWaitVm0);
            } else {
#pragma unroll
                for (int cw = 0; cw < Gm::NCW; ++cw) {
                    Macc[cw] = zero;
                    Sacc[cw] = zero;
                }
            }
        };
        auto store_state = [&]() {
            const size_t so = state_off();
#pragma unroll
            for (int cw = 0; cw < Gm::NCW; ++cw) {
                const int col = O::tmap(x.chi * Gm::NCW + cw, 4 * lg);
                if (col < D) {
                    if (p.MT) *reinterpret_cast<f32x4*>(p.MT + so + col) = Macc[cw];
                    if (p.ST) *reinterpret_cast<f32x4*>(p.ST + so + col) = Sacc[cw];
                }
            }
        };
        load_state();
        F MB[Gm::NKCW], SB[Gm::NKCW];
        f32x4 E[Gm::NTW], Zp[Gm::NTW];
        K::own_frags(x, sm, Macc, Sacc, MB, SB);
        const uint32_t zcol = row + 4 * lg;
        const bool zb = p.z_bf16 != 0;
        const uint32_t zsz = zb ? 2u : 4u;
        __syncthreads();   // item 0 staged
        __syncthreads();   // item 0 decay matrix
        __syncthreads();   // item 0 P tiles
        const typename K::Lanes a = K::lanes(x, sm);
        const uint32_t zoff = opaque(O::tmap(x.chi * Gm::NTW, lr) * D + zcol);
        auto item = [&](int j, auto bi) {
            constexpr int BI = decltype(bi)::value;
            const auto rz = make_rsrc(static_cast<char*>(p.z) + static_cast<size_t>(cs.tok) * D * zsz,
                                      static_cast<uint32_t>(min(b, cs.rem)) * D * zsz);
            if (p.ckpt) {
                T* base = static_cast<T*>(p.ckpt) + static_cast<size_t>(cs.ck) * (2 * D * D) +
                          static_cast<size_t>(row + lr) * D;
#pragma unroll
                for (int cw = 0; cw < Gm::NCW; ++cw) {
                    const int col = O::tmap(x.chi * Gm::NCW + cw, 4 * lg);
                    if (col < D) {
                        st4<T>(base + col, Macc[cw]);
                        st4<T>(base + D * D + col, Sacc[cw]);
                    }
                }
            }
            const uint32_t gs = a.g + static_cast<uint32_t>(j & 3) * K::kGateB;
            const uint32_t gsc = lds_addr(&sm.rg[j & 3].scal[0]);
            K::template phaseA2<BI>(a, gs, gsc, MB, SB, E, Zp, Macc, Sacc);
            __syncthreads();
            K::template phaseB2<BI, false>(a, Macc, Sacc, MB, SB, Zp, rz, zoff, zb);
            if (cs.rem > b) {
                cs.tok += b;
                cs.rem -= b;
                cs.ck += 1;
            } else {
                // Last chunk of the document: its final state out, the next one's initial state in.
                store_state();
                cursor_at(cs, sm, cs.k + 1, nu);
                load_state();
            }
            K::frags2(a, Macc, Sacc, MB, SB);
            __syncthreads();
        };
        for (int j = 0; j < J; j += 2) {
            item(j, std::integral_constant<int, 0>{});
            if (j + 1 < J) item(j + 1, std::integral_constant<int, 1>{});
        }
    } else {
        // ===================== producer wave =====================
        switch (w - NSW) {
            case 0: producer_packed_impl<T, D, NS, CS, NP, 0>(p, sm, row_wg, nu, J, lane); break;
            case 1: producer_packed_impl<T, D, NS, CS, NP, 1>(p, sm, row_wg, nu, J, lane); break;
            case 2: producer_packed_impl<T, D, NS, CS, NP, 2>(p, sm, row_wg, nu, J, lane); break;
            case 3: producer_packed_impl<T, D, NS, CS, NP, 3>(p, sm, row_wg, nu, J, lane); break;
            case 4: producer_packed_impl<T, D, NS, CS, NP, 4>(p, sm, row_wg, nu, J, lane); break;
            case 5: producer_packed_impl<T, D, NS, CS, NP, 5>(p, sm, row_wg, nu, J, lane); break;
            case 6: producer_packed_impl<T, D, NS, CS, NP, 6>(p, sm, row_wg, nu, J, lane); break;
            default: producer_packed_impl<T, D, NS, CS, NP, 7>(p, sm, row_wg, nu, J, lane); break;
        }
    }
}

template <typename T, int D, int NS, int CS, int NP>
__global__ __launch_bounds__(kWave * (NS * CS + (CS == 2 ? 8 : 2))) void linear_memory_fwd(const Params p) {
    using Gm = Geo<T, D, NS, CS, NP>;
    using K = Kernel<T, D, NS, CS, NP>;
    using O = Op<T>;
    using F = typename O::frag;
    constexpr int NBUF = Gm::NBUF;
    constexpr int RB = Gm::RB;
    constexpr int NSW = Gm::NSW;

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
    int bh = lin / Gm::NRB;
    int rb = lin % Gm::NRB;
    int seqlen = p.T;
    size_t ck_chunk0 = 0;   // checkpoint slot of the sequence's chunk 0
    size_t seq_tok = static_cast<size_t>(bh) * p.T;
    if (p.cu) {
        // Packed documents: units u = (rank, head) in rank order, dealt
        // round-robin to the XCDs (the row blocks of a unit on one XCD), so
        // that dispatch order follows the ranking; then the real document.
        int u = bh;
        if ((p.BH % 8) == 0) {
            const int x = blockIdx.x % 8, m = blockIdx.x / 8;
            rb = m % Gm::NRB;
            u = (m / Gm::NRB) * 8 + x;
        }
        const int s = doc_of_rank(p.cu, p.BH / p.H, p.T, u / p.H, lane, p.perm), h = u % p.H;
        bh = s * p.H + h;
        // Offsets clamped into [0, T]: a malformed table cannot send any
        // access outside the packed arrays.
        const int t0 = min(max(p.cu[s], 0), p.T);
        seqlen = min(max(p.cu[s + 1], t0), p.T) - t0;
        seq_tok = static_cast<size_t>(h) * p.T + t0;
        if (p.ckpt) {
            // Non-overlapping documents fill at most the head's tcmax slots;
            // overlapping ones (a table that is not non-decreasing) are cut
            // at the head's last slot.
            const int pre = doc_chunk_prefix(p.cu, s, p.T, p.b, lane);
            ck_chunk0 = static_cast<size_t>(h) * p.tcmax + pre;
            seqlen = min(seqlen, max(p.tcmax - pre, 0) * p.b);
        }
    }
    const int b = p.b;
    const int row_wg = rb * RB;
    const int nch = (seqlen + b - 1) / b;
    auto chunk_n = [&](int c) { return min(b, seqlen - c * b); };
    if (!p.cu) ck_chunk0 = static_cast<size_t>(bh) * nch;

    // Zero all staging memory once: padded rows and columns stay 0.
    {
        uint32_t* words = reinterpret_cast<uint32_t*>(&sm);
        for (int i = tid; i < static_cast<int>(sizeof(sm) / 4); i += kWave * Gm::NWAVE) words[i] = 0u;
    }
    __syncthreads();

    if (w < NSW) {
        // ===================== state wave =====================
        typename K::StateCtx x;
        __builtin_amdgcn_s_setprio(2);
        x.rho = w / CS;
        x.chi = w % CS;
        x.r0 = 16 * x.rho;           // first row within the workgroup block
        x.lr = lr;
        x.lg = lg;
        const int row = row_wg + x.r0;
        // Own column tile cw, lane (lr, lg): M[row + lr][tmap(chi*NCW + cw, 4lg + e)], e = 0..3.
        f32x4 Macc[Gm::NCW], Sacc[Gm::NCW];
        const size_t state_off = static_cast<size_t>(bh) * D * D + static_cast<size_t>(row + lr) * D;
#pragma unroll
        for (int cw = 0; cw < Gm::NCW; ++cw) {
            const int col = O::tmap(x.chi * Gm::NCW + cw, 4 * lg);
            const bool ok = col < D;
            Macc[cw] = (p.M0 && ok) ? *reinterpret_cast<const f32x4*>(p.M0 + state_off + col) : f32x4{0.f, 0.f, 0.f, 0.f};
            Sacc[cw] = (p.S0 && ok) ? *reinterpret_cast<const f32x4*>(p.S0 + state_off + col) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // Checkpoint of the state entering chunk c (what the backward pass
        // differentiates from), in the layout of M_T / S_T.
        auto save = [&](int c) {
            if (p.ckpt) {
                T* base = static_cast<T*>(p.ckpt) + (ck_chunk0 + c) * (2 * D * D) +
                          static_cast<size_t>(row + lr) * D;
#pragma unroll
                for (int cw = 0; cw < Gm::NCW; ++cw) {
                    const int col = O::tmap(x.chi * Gm::NCW + cw, 4 * lg);
                    if (col < D) {
                        st4<T>(base + col, Macc[cw]);
                        st4<T>(base + D * D + col, Sacc[cw]);
                    }
                }
            }
        };
        F MB[Gm::NKCW], SB[Gm::NKCW];
        f32x4 E[Gm::NTW], Zp[Gm::NTW];
        K::own_frags(x, sm, Macc, Sacc, MB, SB);
        const uint32_t zcol = row + 4 * lg;
        // z of chunk c: its n rows of float32 or bf16 (stores past them are dropped).
        const bool zb = p.z_bf16 != 0;
        const uint32_t zsz = zb ? 2u : 4u;
        auto zchunk = [&](int c) {
            return make_rsrc(static_cast<char*>(p.z) + (seq_tok + static_cast<size_t>(c) * b) * D * zsz,
                             static_cast<uint32_t>(chunk_n(c)) * D * zsz);
        };
        if constexpr (NBUF == 2 && Gm::F16 && CS == 2) {
            __syncthreads();   // chunk 0 staged
            __syncthreads();   // chunk 0 decay matrix
            __syncthreads();   // chunk 0 P tiles
            const typename K::Lanes a = K::lanes(x, sm);
            const uint32_t zoff = opaque(O::tmap(x.chi * Gm::NTW, lr) * D + zcol);   // elements
            // Chunk c reads buffer c & 1 and gate slot c & 3.
            for (int c = 0; c < nch; c += 2) {
                {
                    const auto rz = zchunk(c);
                    const uint32_t gs = a.g + static_cast<uint32_t>(c & 3) * K::kGateB;
                    const uint32_t gsc = lds_addr(&sm.rg[c & 3].scal[0]);
                    save(c);
                    K::template phaseA2<0>(a, gs, gsc, MB, SB, E, Zp, Macc, Sacc);
                    __syncthreads();
                    K::template phaseB2<0>(a, Macc, Sacc, MB, SB, Zp, rz, zoff, zb);
                    __syncthreads();
                }
                if (c + 1 < nch) {
                    const auto rz = zchunk(c + 1);
                    const uint32_t gs = a.g + static_cast<uint32_t>((c + 1) & 3) * K::kGateB;
                    const uint32_t gsc = lds_addr(&sm.rg[(c + 1) & 3].scal[0]);
                    save(c + 1);
                    K::template phaseA2<1>(a, gs, gsc, MB, SB, E, Zp, Macc, Sacc);
                    __syncthreads();
                    K::template phaseB2<1>(a, Macc, Sacc, MB, SB, Zp, rz, zoff, zb);
                    __syncthreads();
                }
            }
        } else if constexpr (NBUF == 2) {
            __syncthreads();   // chunk 0 staged
            __syncthreads();   // chunk 0 decay matrix
            __syncthreads();   // chunk 0 P tiles
            // Chunk c reads buffer c & 1; the loop is unrolled by two so that
            // every LDS address is a compile-time offset from lane constants.
            auto chunk = [&](int c, const typename K::Buf& B) {
                const auto rz = zchunk(c);
                const typename K::ReadGates& rg = sm.rg[c & 3];
                save(c);
                K::phaseA(x, B, rg, sm, MB, SB, E, Zp);
                __syncthreads();
                K::phaseB(x, B, rg, sm, Macc, Sacc, MB, SB, E, Zp, rz, zcol, zb);
                __syncthreads();
            };
            for (int c = 0; c < nch; c += 2) {
                chunk(c, sm.buf[0]);
                if (c + 1 < nch) chunk(c + 1, sm.buf[1]);
            }
        } else {
            for (int c = 0; c < nch; ++c) {
                __syncthreads();   // chunk c staged
                __syncthreads();   // chunk c decay matrix
                __syncthreads();   // chunk c P tiles
                const auto rz = zchunk(c);
                save(c);
                K::phaseA(x, sm.buf[0], sm.rg[c & 3], sm, MB, SB, E, Zp);
                __syncthreads();
                K::phaseB(x, sm.buf[0], sm.rg[c & 3], sm, Macc, Sacc, MB, SB, E, Zp, rz, zcol, zb);
                __syncthreads();   // chunk c consumed
            }
        }
#pragma unroll
        for (int cw = 0; cw < Gm::NCW; ++cw) {
            const int col = O::tmap(x.chi * Gm::NCW + cw, 4 * lg);
            if (col < D) {
                if (p.MT) *reinterpret_cast<f32x4*>(p.MT + state_off + col) = Macc[cw];
                if (p.ST) *reinterpret_cast<f32x4*>(p.ST + state_off + col) = Sacc[cw];
            }
        }
    } else {
        // ===================== producer wave =====================
        const int pw = w - NSW;
        if (pw == 0) producer_loop_impl<T, D, NS, CS, NP, 0>(p, sm, seq_tok, seqlen, row_wg, nch, lane);
        else if (pw == 1) producer_loop_impl<T, D, NS, CS, NP, 1>(p, sm, seq_tok, seqlen, row_wg, nch, lane);
        else if constexpr (Gm::NPW == 8) {
            switch (pw) {
                case 2: producer_loop_impl<T, D, NS, CS, NP, 2>(p, sm, seq_tok, seqlen, row_wg, nch, lane); break;
                case 3: producer_loop_impl<T, D, NS, CS, NP, 3>(p, sm, seq_tok, seqlen, row_wg, nch, lane); break;
                case 4: producer_loop_impl<T, D, NS, CS, NP, 4>(p, sm, seq_tok, seqlen, row_wg, nch, lane); break;
                case 5: producer_loop_impl<T, D, NS, CS, NP, 5>(p, sm, seq_tok, seqlen, row_wg, nch, lane); break;
                case 6: producer_loop_impl<T, D, NS, CS, NP, 6>(p, sm, seq_tok, seqlen, row_wg, nch, lane); break;
                default: producer_loop_impl<T, D, NS, CS, NP, 7>(p, sm, seq_tok, seqlen, row_wg, nch, lane); break;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Host side: validation, instance selection, launch.
// ---------------------------------------------------------------------------
// Workgroup lanes V of the persistent packed walk on the current device:
// resident workgroups (CUs x occupancy) / (8 XCD lanes x NRB row blocks),
// queried once per device and instance.
template <typename T, int D, int NS, int CS, int NP>
int packed_lanes() {
    using Gm = Geo<T, D, NS, CS, NP>;
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    std::atomic<int>& slot = cached[dev & 63];
    int v = slot.load(std::memory_order_relaxed);
    if (v > 0) return v;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, linear_memory_fwd_packed<T, D, NS, CS, NP>,
                                                     kWave * Gm::NWAVE, 0) != hipSuccess || per_cu <= 0)
        per_cu = 1;
    v = cmax(1, cus * per_cu / (8 * Gm::NRB));
    slot.store(v, std::memory_order_relaxed);
    return v;
}

template <typename T, int D, int NS, int CS, int NP>
hipError_t launch(const Params& p, hipStream_t stream) {
    using Gm = Geo<T, D, NS, CS, NP>;
    if constexpr (Gm::PERSIST) {
        if (p.cu) {
            // Packed documents: persistent workgroups when the documents fit the
            // in-LDS ranking and every workgroup's units fit its table.
            const int N = p.BH / p.H;
            const int V = cmax(1, cmin(packed_lanes<T, D, NS, CS, NP>(), (p.BH + 7) / 8));
            const long long kmax = (static_cast<long long>(p.BH) + 8LL * V - 1) / (8LL * V);
            if (N <= Gm::NMAX_DOCS && kmax <= Gm::KMAX) {
                hipLaunchKernelGGL((linear_memory_fwd_packed<T, D, NS, CS, NP>), dim3(8 * Gm::NRB * V),
                                   dim3(kWave * Gm::NWAVE), 0, stream, p);
                return hipGetLastError();
            }
        }
    }
    // One workgroup per (sequence or document, row block).  Packed documents
    // above the in-wave ranking's limit take their order from a pass before
    // the launch.
    Params q = p;
    int* perm = nullptr;
    if (p.cu && p.T > 0) {
        const hipError_t e = make_doc_order(p.cu, p.BH / p.H, p.T, stream, &perm);
        if (e != hipSuccess) return e;
    }
    q.perm = perm;
    const long long nwg = static_cast<long long>(p.BH) * Gm::NRB;
    hipLaunchKernelGGL((linear_memory_fwd<T, D, NS, CS, NP>), dim3(static_cast<unsigned>(nwg)),
                       dim3(kWave * Gm::NWAVE), 0, stream, q);
    const hipError_t err = hipGetLastError();
    if (perm) (void)hipFreeAsync(perm, stream);
    return err;
}

template <typename T, int D, int NS>
hipError_t launch_np(const Params& p, int np, hipStream_t stream) {
    if constexpr (Op<T>::KG == 32) {
        // fp16: split the columns over two state waves when every half keeps
        // whole k-groups (d >= 64).
        constexpr int CS = D >= 64 ? 2 : 1;
        return np <= 32 ? launch<T, D, NS, CS, 32>(p, stream) : launch<T, D, NS, CS, 64>(p, stream);
    } else {
        if (np <= 16) return launch<T, D, NS, 1, 16>(p, stream);
        if (np <= 32) return launch<T, D, NS, 1, 32>(p, stream);
        return launch<T, D, NS, 1, 64>(p, stream);
    }
}

// Compute units of the current device, queried once per device.
int device_cus() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    std::atomic<int>& slot = cached[dev & 63];
    int v = slot.load(std::memory_order_relaxed);
    if (v > 0) return v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    slot.store(v, std::memory_order_relaxed);
    return v;
}

template <typename T, int D>
hipError_t launch_ns(const Params& p, int np, hipStream_t stream) {
    if constexpr (D >= 32) {
        // Two 16-row tiles per workgroup when there are more row tiles than
        // CUs: one-tile workgroups would then share CUs or run in a second
        // round, which costs more than the fewer, larger workgroups.
        const long long row_tiles = static_cast<long long>(p.BH) * (D / 16);
        if (row_tiles > device_cus()) return launch_np<T, D, 2>(p, np, stream);
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


template <typename T>
int forward_impl(const void* q, const void* k, const void* v, const float* theta, const float* eta,
                 const float* alpha, const float* M0, const float* S0, void* z, float* M_T, float* S_T,
                 void* ckpt, int B, int H, int Tlen, int d, int b, void* stream, bool chunk_gates = false,
                 bool z_bf16 = false) {
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
    const size_t z_bytes = tok * d * (z_bf16 ? 2 : sizeof(float));
    const size_t st_bytes = static_cast<size_t>(BH) * d * d * sizeof(float);
    // Gate entries: one per token, or one per chunk.
    const size_t g_count = chunk_gates ? static_cast<size_t>(BH) * ((static_cast<size_t>(Tlen) + b - 1) / b) : tok;
    if (Tlen > 0) {
        if (!q || !k || !v || !theta || !eta || !alpha || !z) return TTT_ERR_INVALID_ARG;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(z, 16)) return TTT_ERR_INVALID_ARG;
        if (!aligned(theta, 4) || !aligned(eta, 4) || !aligned(alpha, 4)) return TTT_ERR_INVALID_ARG;
        const void* ins[] = {q, k, v};
        for (const void* in : ins)
            if (overlaps(z, z_bytes, in, in_bytes)) return TTT_ERR_INVALID_ARG;
        const void* gates[] = {theta, eta, alpha};
        for (const void* g : gates)
            if (overlaps(z, z_bytes, g, g_count * sizeof(float))) return TTT_ERR_INVALID_ARG;
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
    if (ckpt) {
        // Written while the inputs are read and the outputs written: no overlap with any of them.
        const size_t ck_bytes = ckpt_bytes(B, H, Tlen, d, b, sizeof(T));
        if (!aligned(ckpt, 16)) return TTT_ERR_INVALID_ARG;
        const void* ins[] = {q, k, v};
        for (const void* in : ins)
            if (overlaps(ckpt, ck_bytes, in, in_bytes)) return TTT_ERR_INVALID_ARG;
        const void* gates[] = {theta, eta, alpha};
        for (const void* g : gates)
            if (overlaps(ckpt, ck_bytes, g, g_count * sizeof(float))) return TTT_ERR_INVALID_ARG;
        for (const void* s : states)
            if (overlaps(ckpt, ck_bytes, s, st_bytes)) return TTT_ERR_INVALID_ARG;
        if (overlaps(ckpt, ck_bytes, z, z_bytes)) return TTT_ERR_INVALID_ARG;
    }

    Params p{q, k, v, theta, eta, alpha, M0, S0, z, M_T, S_T, static_cast<int>(BH), Tlen, b, nullptr, H, ckpt,
             chunk_gates ? 1 : 0, 0, z_bf16 ? 1 : 0, nullptr};
    const hipError_t err = dispatch<T>(p, d, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

// Packed variable-length documents: q, k, v, z [H, T, d] and gates [H, T]
// with document s of head h at tokens cu[s] .. cu[s+1]-1; states [N, H, d, d].
template <typename T>
int forward_varlen_impl(const void* q, const void* k, const void* v, const float* theta, const float* eta,
                        const float* alpha, const float* M0, const float* S0, float* z, float* M_T, float* S_T,
                        const int* cu, int N, int H, int Tlen, int d, int b, void* stream, void* ckpt = nullptr) {
    using G = typename GlobalOf<T>::type;
    if (N < 0 || H < 0 || Tlen < 0) return TTT_ERR_INVALID_ARG;
    if (b < 1) return TTT_ERR_INVALID_ARG;
    if (d != 16 && d != 32 && d != 64 && d != 128) return TTT_ERR_UNSUPPORTED;
    if (b > 64) return TTT_ERR_UNSUPPORTED;
    const long long BH = static_cast<long long>(N) * H;
    if (BH == 0) return TTT_OK;
    if (!cu || !aligned(cu, 4)) return TTT_ERR_INVALID_ARG;
    if (BH * (d / 16) > 0x7fffffffLL) return TTT_ERR_UNSUPPORTED;
    if (static_cast<long long>(H) * Tlen > 0x7fffffffLL) return TTT_ERR_UNSUPPORTED;
    const size_t tok = static_cast<size_t>(H) * static_cast<size_t>(Tlen);
    const size_t in_bytes = tok * d * sizeof(G);
    const size_t z_bytes = tok * d * sizeof(float);
    const size_t st_bytes = static_cast<size_t>(BH) * d * d * sizeof(float);
    const size_t cu_bytes = (static_cast<size_t>(N) + 1) * sizeof(int);
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
            overlaps(z, z_bytes, M_T, st_bytes) || overlaps(z, z_bytes, S_T, st_bytes) ||
            overlaps(z, z_bytes, cu, cu_bytes))
            return TTT_ERR_INVALID_ARG;
    }
    const void* states[] = {M0, S0, M_T, S_T};
    for (const void* st : states)
        if (st && !aligned(st, 16)) return TTT_ERR_INVALID_ARG;
    if (M_T && M_T != M0 && (overlaps(M_T, st_bytes, M0, st_bytes) || overlaps(M_T, st_bytes, S0, st_bytes)))
        return TTT_ERR_INVALID_ARG;
    if (S_T && S_T != S0 && (overlaps(S_T, st_bytes, S0, st_bytes) || overlaps(S_T, st_bytes, M0, st_bytes)))
        return TTT_ERR_INVALID_ARG;
    if (M_T && S_T && overlaps(M_T, st_bytes, S_T, st_bytes)) return TTT_ERR_INVALID_ARG;
    if (overlaps(M_T, st_bytes, cu, cu_bytes) || overlaps(S_T, st_bytes, cu, cu_bytes)) return TTT_ERR_INVALID_ARG;
    const long long tcmax = varlen_chunk_slots(N, Tlen, b);
    if (ckpt) {
        // [H][tcmax][M | S][d][d]; the gradient pass launches H * tcmax workgroups.
        if (static_cast<long long>(H) * tcmax > 0x7fffffffLL) return TTT_ERR_UNSUPPORTED;
        if (!aligned(ckpt, 16)) return TTT_ERR_INVALID_ARG;
        const size_t ck_bytes = ckpt_bytes_varlen(N, H, Tlen, d, b, sizeof(T));
        const Span others[] = {{q, in_bytes}, {k, in_bytes}, {v, in_bytes}, {theta, tok * 4}, {eta, tok * 4},
                               {alpha, tok * 4}, {M0, st_bytes}, {S0, st_bytes}, {z, z_bytes}, {M_T, st_bytes},
                               {S_T, st_bytes}, {cu, cu_bytes}};
        for (const Span& o : others)
            if (o.p && overlaps(ckpt, ck_bytes, o.p, o.n)) return TTT_ERR_INVALID_ARG;
    }

    Params p{q, k, v, theta, eta, alpha, M0, S0, z, M_T, S_T, static_cast<int>(BH), Tlen, b, cu, H, ckpt, 0,
             static_cast<int>(tcmax), 0, nullptr};
    // More documents than the in-kernel ranking covers: a pass before the
    // launch writes their longest-first order to a stream-ordered table.
    const hipError_t err = dispatch<T>(p, d, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

}  // namespace

extern "C" {

int ttt_mem_forward_f32(const float* q, const float* k, const float* v, const float* theta, const float* eta,
                        const float* alpha, const float* M0, const float* S0, float* z, float* M_T, float* S_T,
                        int B, int H, int T, int d, int b, void* stream) {
    return forward_impl<float>(q, k, v, theta, eta, alpha, M0, S0, z, M_T, S_T, nullptr, B, H, T, d, b, stream);
}

int ttt_mem_forward_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* theta,
                         const float* eta, const float* alpha, const float* M0, const float* S0, uint16_t* z,
                         float* M_T, float* S_T, int B, int H, int T, int d, int b, void* stream) {
    return forward_impl<_Float16>(q, k, v, theta, eta, alpha, M0, S0, z, M_T, S_T, nullptr, B, H, T, d, b, stream,
                                  false, true);
}

int ttt_mem_forward_bf16_zf32(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* theta,
                              const float* eta, const float* alpha, const float* M0, const float* S0, float* z,
                              float* M_T, float* S_T, int B, int H, int T, int d, int b, void* stream) {
    return forward_impl<_Float16>(q, k, v, theta, eta, alpha, M0, S0, z, M_T, S_T, nullptr, B, H, T, d, b, stream);
}

int ttt_mem_forward_varlen_f32(const float* q, const float* k, const float* v, const float* theta, const float* eta,
                               const float* alpha, const float* M0, const float* S0, float* z, float* M_T,
                               float* S_T, const int* cu_seqlens, int N, int H, int T, int d, int b, void* stream) {
    return forward_varlen_impl<float>(q, k, v, theta, eta, alpha, M0, S0, z, M_T, S_T, cu_seqlens, N, H, T, d, b,
                                      stream);
}

int ttt_mem_forward_varlen_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* theta,
                                const float* eta, const float* alpha, const float* M0, const float* S0, float* z,
                                float* M_T, float* S_T, const int* cu_seqlens, int N, int H, int T, int d, int b,
                                void* stream) {
    return forward_varlen_impl<_Float16>(q, k, v, theta, eta, alpha, M0, S0, z, M_T, S_T, cu_seqlens, N, H, T, d, b,
                                         stream);
}

int ttt_mem_forward_ckpt_f32(const float* q, const float* k, const float* v, const float* theta, const float* eta,
                             const float* alpha, const float* M0, const float* S0, float* z, float* M_T, float* S_T,
                             float* ckpt, int B, int H, int T, int d, int b, void* stream) {
    if (!ckpt) return TTT_ERR_INVALID_ARG;
    return forward_impl<float>(q, k, v, theta, eta, alpha, M0, S0, z, M_T, S_T, ckpt, B, H, T, d, b, stream);
}

int ttt_mem_forward_ckpt_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* theta,
                              const float* eta, const float* alpha, const float* M0, const float* S0, float* z,
                              float* M_T, float* S_T, uint16_t* ckpt, int B, int H, int T, int d, int b,
                              void* stream) {
    if (!ckpt) return TTT_ERR_INVALID_ARG;
    return forward_impl<_Float16>(q, k, v, theta, eta, alpha, M0, S0, z, M_T, S_T, ckpt, B, H, T, d, b, stream);
}

size_t ttt_mem_ckpt_bytes(int B, int H, int T, int d, int b) { return ckpt_bytes(B, H, T, d, b, 4); }

size_t ttt_mem_ckpt_bytes_varlen(int N, int H, int T, int d, int b) { return ckpt_bytes_varlen(N, H, T, d, b, 4); }

size_t ttt_mem_ckpt_bytes_varlen_bf16(int N, int H, int T, int d, int b) {
    return ckpt_bytes_varlen(N, H, T, d, b, 2);
}

int ttt_mem_forward_varlen_ckpt_f32(const float* q, const float* k, const float* v, const float* theta,
                                    const float* eta, const float* alpha, const float* M0, const float* S0, float* z,
                                    float* M_T, float* S_T, float* ckpt, const int* cu_seqlens, int N, int H, int T,
                                    int d, int b, void* stream) {
    if (!ckpt) return TTT_ERR_INVALID_ARG;
    return forward_varlen_impl<float>(q, k, v, theta, eta, alpha, M0, S0, z, M_T, S_T, cu_seqlens, N, H, T, d, b,
                                      stream, ckpt);
}

int ttt_mem_forward_varlen_ckpt_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* theta,
                                     const float* eta, const float* alpha, const float* M0, const float* S0,
                                     float* z, float* M_T, float* S_T, uint16_t* ckpt, const int* cu_seqlens, int N,
                                     int H, int T, int d, int b, void* stream) {
    if (!ckpt) return TTT_ERR_INVALID_ARG;
    return forward_varlen_impl<_Float16>(q, k, v, theta, eta, alpha, M0, S0, z, M_T, S_T, cu_seqlens, N, H, T, d,
                                         b, stream, ckpt);
}

size_t ttt_mem_ckpt_bytes_bf16(int B, int H, int T, int d, int b) { return ckpt_bytes(B, H, T, d, b, 2); }

int ttt_mem_forward_cg_f32(const float* q, const float* k, const float* v, const float* theta, const float* eta,
                           const float* alpha, const float* M0, const float* S0, float* z, float* M_T, float* S_T,
                           float* ckpt, int B, int H, int T, int d, int b, void* stream) {
    return forward_impl<float>(q, k, v, theta, eta, alpha, M0, S0, z, M_T, S_T, ckpt, B, H, T, d, b, stream, true);
}

int ttt_mem_forward_cg_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* theta,
                            const float* eta, const float* alpha, const float* M0, const float* S0, float* z,
                            float* M_T, float* S_T, uint16_t* ckpt, int B, int H, int T, int d, int b,
                            void* stream) {
    return forward_impl<_Float16>(q, k, v, theta, eta, alpha, M0, S0, z, M_T, S_T, ckpt, B, H, T, d, b, stream,
                                  true);
}

const char* ttt_mem_status_string(int status) {
    switch (status) {
        case TTT_OK: return "ok";
        case TTT_ERR_INVALID_ARG: return "invalid argument";
        case TTT_ERR_UNSUPPORTED: return "unsupported size";
        case TTT_ERR_HIP: return "HIP launch failed";
        case TTT_ERR_DEVICE: return "device-side failure (deep-memory group exchange)";
        default: return "unknown status";
    }
}

int ttt_mem_abi_version(void) { return TTT_MEM_ABI_VERSION; }

}  // extern "C"
