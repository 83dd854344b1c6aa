// gemm_panel_ring.hip -- the f32-panel ring with K split over workgroups
// (KS=3 configurations with BK = 32), in both modes: the f32 panels of A and
// B reach shared memory through direct global->LDS copies into a ring of NS
// stages, as in the f32 ring kernel, so many panels are in flight per
// workgroup without holding them in registers; each fragment is read in f32
// and, in the f16r mode, rounded to binary16 (nearest even) in registers and
// multiplied on v_mfma_f32_16x16x32_f16, in the f32 mode multiplied as read on
// v_mfma_f32_16x16x4_f32, with f32 accumulation either way.  For up to a few
// hundred rows of C the call streams B once from memory and the matrix work is
// small, so what matters is keeping enough copies in flight to reach the
// memory roof; in f16r the packing pass of the packed path (read, round and
// write all of B, then read it again) and the one-panel-ahead register
// staging of the other KS=3 kernel both fall short of it there, in f32 the
// split-K tiles (KS=1: partial tiles summed by a second pass).
//
// Shapes: every operand layout with 16-byte aligned rows and K % 32 == 0;
// N % 4 == 0 where B is stored K x N and M % 4 == 0 where A is stored K x M
// (M and N need not be tile multiples: copies of rows past M or N read the
// last row, and of columns past them the tile's first column, values that
// only reach outputs the masked epilogue never stores).  K is split over
// blockIdx.y, the last workgroup of a tile adding the slices' partial tiles
// in slice order.
#include "f16_kernel.hpp"

// X(BM, BN, NS, WM, WN, GM): the compiled configurations of each mode.
#define G355_PANEL_RING_F16R_CONFIGS(X) \
    X(16, 128, 4, 1, 2, 8)              \
    X(32, 64, 4, 2, 1, 8)               \
    X(32, 128, 4, 2, 2, 8)              \
    X(64, 64, 4, 4, 1, 8)               \
    X(64, 128, 3, 2, 2, 8)              \
    X(128, 128, 3, 4, 2, 8)             \
    X(128, 256, 3, 2, 4, 8)             \
    X(256, 128, 3, 4, 2, 8)
#define G355_PANEL_RING_F32_CONFIGS(X) \
    X(16, 128, 4, 1, 2, 8)             \
    X(32, 64, 4, 2, 1, 8)              \
    X(32, 128, 4, 2, 2, 8)             \
    X(64, 64, 4, 4, 1, 8)              \
    X(64, 128, 3, 2, 2, 8)             \
    X(128, 128, 3, 4, 2, 8)

namespace g355 {
namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const f32x4v lds_f32x4c;
typedef __attribute__((address_space(3))) const float lds_f32c;

// A K slice of a split call: the workgroup stores its partial tile in P
// (slices x tiles x TILE_BYTES; within a tile, wave-major, block-major, lane
// by lane, 16 bytes each), and the last workgroup of the tile to arrive
// (counted in counts[tile]) adds the slices' partial tiles in slice order into
// acc and returns true; the others return false.  The counter is zero again
// when the last one leaves.  `flag` is 4 bytes of the workgroup's shared
// memory that no wave reads any more.
template <int GFM, int GFN, int TILE_BYTES>
__device__ __forceinline__ bool last_slice_adds(f32x4v (&acc)[GFM][GFN], const DirectArgs& p,
                                                int wave, int lane, unsigned char* flag_lds) {
    constexpr int kSC1 = 1 << 4;             // cache-policy bit of the buffer intrinsics
    constexpr int kRsrc = 0x00020000;        // raw buffer, 32-bit data format
    constexpr int NB = GFM * GFN;
    const int tiles = gridDim.x, slice = blockIdx.y;
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        p.P, (short)0, static_cast<int>((int64_t)p.slices * tiles * TILE_BYTES), kRsrc);
    auto at = [&](int z, int b) {
        return static_cast<int>(((int64_t)z * tiles + blockIdx.x) * TILE_BYTES +
                                ((wave * NB + b) * 64 + lane) * 16);
    };
#pragma unroll
    for (int b = 0; b < NB; ++b)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[b / GFN][b % GFN]), rp,
                                               at(slice, b), 0, kSC1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();   // every wave is past its last panel read and its stores are done
    unsigned* count = p.counts + blockIdx.x;
    int* flag = reinterpret_cast<int*>(flag_lds);
    if (threadIdx.x == 0)
        *flag = __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                static_cast<unsigned>(p.slices - 1);
    __syncthreads();
    if (!*flag) return false;
    if (threadIdx.x == 0) __hip_atomic_store(count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    constexpr int ZG = 4;
    for (int z0 = 0; z0 < p.slices; z0 += ZG) {
        f32x4v t[ZG][NB];
#pragma unroll
        for (int zz = 0; zz < ZG; ++zz) {
            const int z = min(z0 + zz, p.slices - 1);   // past the last slice: a reload, unused
#pragma unroll
            for (int b = 0; b < NB; ++b)
                t[zz][b] = __builtin_bit_cast(
                    f32x4v, __builtin_amdgcn_raw_buffer_load_b128(rp, at(z, b), 0, kSC1));
        }
#pragma unroll
        for (int zz = 0; zz < ZG; ++zz) {
            if (z0 + zz >= p.slices) break;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const f32x4v a = acc[b / GFN][b % GFN];
                acc[b / GFN][b % GFN] = z0 + zz == 0 ? t[zz][b] : a + t[zz][b];
            }
        }
    }
    return true;
}

// ---------------------------------------------------------------------------
// Panel layout (each operand copied along its stored rows and kept in that
// orientation):
//   A (as stored; B^T alike): BM rows of 128 bytes (eight 16-byte chunks of 4
//      k); chunk c of row r sits at position c ^ swz<64>(r) = c ^ ((r / 2) %
//      8), the key of the packed image's 128-byte rows; a copy instruction
//      fills 8 rows, lane l fetching the global chunk that belongs at its
//      position.  Measured (LdsBankConflict): no conflicts with this key or
//      with r % 8, while (r % 8) ^ ((r / 8) % 2) made every A fragment read a
//      two-way conflict (2-4% of the call's time at 256-512 rows).
//   B (as stored): 32 k-rows of BN floats, BN * 4 bytes apart; a copy
//      instruction fills 1024 / (4 BN) whole k-rows.
//   A^T (A stored K x M): 32 k-rows of BM floats in groups of 256 / BM k-rows
//      that one copy instruction fills, the groups 1 KB + PAD apart (KRowsPanel
//      below), so that the four k-rows the lane quarters read at once (4
//      apart) fall in four different quarters of the 64 banks.
// A panel's sum over its 32 k may run in any order, so lane quarter q takes
// k in {4q .. 4q + 3} and {16 + 4q .. 16 + 4q + 3}, for A and B alike: two
// 16-byte reads of a row (A, B^T), or eight single reads of k-rows (A^T).  In
// f16r these eight k are the lane's eight operands of one
// v_mfma_f32_16x16x32_f16; in f32, step t of eight v_mfma_f32_16x16x4_f32
// takes the t-th of them from every lane quarter, so each step sums four
// distinct k and the eight steps all 32.  Columns (B as stored): the wave
// tile's columns are dealt to its 16-column blocks four at a time -- lane
// column r16 of block 4g + jj is column 64g + 4 r16 + jj of the wave tile --
// so one 16-byte read of a B k-row gives a lane its value for four blocks
// (eight reads: four blocks' fragments, 16 lanes reading 256 contiguous
// bytes), and in the epilogue a lane holds four consecutive columns of a row,
// which it reads (beta != 0) and writes as one piece.  With B^T the columns
// are not dealt (lane column r16 of block j is column 16 j + r16, 16
// consecutive rows of the B^T panel, as the A reads) and the epilogue is the
// block layout's.
// ---------------------------------------------------------------------------

// The k-rows panel of A^T: 32 k-rows of EXT floats.  One 1 KB copy fills a
// group of RPI = 256 / EXT k-rows; groups lie GROUP bytes apart.  The lane
// quarters read k-rows 4q + t together (t fixed), 16 floats each, which must
// fall in four different quarters of the 64 banks.  Up to 4 k-rows a group,
// PAD does it (the k-rows of a group are contiguous, so rows 4 apart in one
// group sit a multiple of 128 floats apart); with 8 or 16 a group the slots
// are permuted, k-row r at slot Q (r % 4) + (r / 4) % Q (Q = RPI / 4), so
// that rows 4 apart land in slots that differ by one modulo Q: 32 banks
// apart for 128-byte k-rows (plus PAD across groups), 16 for 64-byte ones.
template <int EXT>
struct KRowsPanel {
    static_assert(EXT == 16 || EXT == 32 || EXT == 64 || EXT == 128 || EXT == 256, "panel extent");
    static constexpr int RPI = 256 / EXT;
    static constexpr int Q = RPI >= 8 ? RPI / 4 : 1;
    static constexpr int PAD = RPI == 1 ? 16 : RPI == 2 ? 32 : RPI == 16 ? 0 : 64;
    static constexpr int GROUP = 1024 + PAD;
    static constexpr int BYTES = (32 / RPI) * GROUP;
    __host__ __device__ static constexpr int slot(int r) { return RPI >= 8 ? Q * (r % 4) + (r / 4) % Q : r; }
    __host__ __device__ static constexpr int row_of_slot(int s) { return RPI >= 8 ? 4 * (s % Q) + s / Q : s; }
    // byte offset of float e of k-row kr
    __host__ __device__ static constexpr int at(int kr, int e) {
        return (kr / RPI) * GROUP + slot(kr % RPI) * EXT * 4 + 4 * e;
    }
};

template <int BM, int BN, int NS, int WM, int WN, bool TA, bool TB>
struct PanelRingShape {
    static constexpr int BK = 32;
    static constexpr int NW = WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int GFM = TM / 16, GFN = TN / 16;
    static constexpr int A_ROW = BK * 4;                       // rows layout
    static constexpr int A_BYTES = TA ? KRowsPanel<BM>::BYTES : BM * A_ROW;
    static constexpr int B_ROW = TB ? BK * 4 : BN * 4;         // a B^T row, or a k-row of B
    static constexpr int B_BYTES = TB ? BN * B_ROW : BK * B_ROW;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    // 1 KB copies per wave per panel (8 rows, or 1024 / (4 EXT) k-rows, each)
    static constexpr int A_INS = BM / 8 / NW;
    static constexpr int B_INS = BN / 8 / NW;
    static constexpr int FILLS = A_INS + B_INS;
    static_assert(BN == 64 || BN == 128 || BN == 256, "whole k-rows per copy instruction");
    static_assert(A_INS >= 1 && A_INS * NW * 8 == BM && B_INS >= 1 && B_INS * NW * 8 == BN,
                  "copies split evenly over the waves");
    static_assert(TM % 16 == 0 && TN % (TB ? 16 : 64) == 0,
                  "wave tile of 16-row blocks and (dealt) 64-column groups");
    static_assert(NS >= 3 && NS * STAGE <= 160 * 1024, "LDS budget of one CU");
    static_assert((NS - 2) * FILLS < 64, "vmcnt range");
};

__device__ __forceinline__ f16x8 rn8(f32x4v lo, f32x4v hi) {
    return f16x8{static_cast<_Float16>(lo[0]), static_cast<_Float16>(lo[1]),
                 static_cast<_Float16>(lo[2]), static_cast<_Float16>(lo[3]),
                 static_cast<_Float16>(hi[0]), static_cast<_Float16>(hi[1]),
                 static_cast<_Float16>(hi[2]), static_cast<_Float16>(hi[3])};
}

// Epilogue of the column-dealt blocks: element e of lane (q, r16) in block
// (i, 4g + jj) is C[row0 + 16 i + 4 q + e][col0 + 64 g + 4 r16 + jj].  The
// value is fma(alpha, acc, beta*c) as in every epilogue of the library (f32,
// or binary16 C widened and the result rounded once to nearest even); beta ==
// 0 never reads C.  When C's rows allow it (f32: 16-byte aligned, binary16:
// 8-byte aligned, ldc % 4 == 0) a lane's four columns are one access, and the
// C reads of a row of blocks are issued before the previous row's stores;
// otherwise element by element.  N % 4 == 0, so a lane's four columns are all
// inside or all past the edge.
template <int GFM, int GFN, bool MASKED, bool OUT16, typename CT>
__device__ __forceinline__ void store_tile_dealt(const f32x4v (&acc)[GFM][GFN], CT* __restrict__ C,
                                                 int64_t ldc, int row0, int col0, int M, int N,
                                                 float alpha, float beta, int lane) {
    constexpr int GG = GFN / 4;
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const int q = lane >> 4, r16 = lane & 15;
    auto row_of = [&](int i, int e) { return row0 + 16 * i + 4 * q + e; };
    auto col_of = [&](int g) { return col0 + 64 * g + 4 * r16; };
    auto inside = [&](int row, int col) { return !MASKED || (row < M && col < N); };
    auto h2f = [](uint32_t bits) {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
    };
    const bool vec = ldc % 4 == 0 && (reinterpret_cast<uintptr_t>(C) & (OUT16 ? 7 : 15)) == 0;
    if (!vec) {
#pragma unroll
        for (int i = 0; i < GFM; ++i)
#pragma unroll
            for (int g = 0; g < GG; ++g)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = row_of(i, e), col = col_of(g);
                    if (!inside(row, col)) continue;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        CT* at = C + (int64_t)row * ldc + col + jj;
                        const float a = acc[i][4 * g + jj][e];
                        if constexpr (OUT16) {
                            const float v = beta == 0.f ? alpha * a
                                                        : __builtin_fmaf(alpha, a, beta * h2f(*at));
                            *at = f32_to_f16_bits(v);
                        } else {
                            *at = beta == 0.f ? alpha * a : __builtin_fmaf(alpha, a, beta * *at);
                        }
                    }
                }
        return;
    }
    auto load4 = [&](int row, int col) -> f32x4v {
        if constexpr (OUT16) {
            const u32x2 w = *reinterpret_cast<const u32x2*>(C + (int64_t)row * ldc + col);
            return f32x4v{h2f(w[0] & 0xffffu), h2f(w[0] >> 16), h2f(w[1] & 0xffffu), h2f(w[1] >> 16)};
        } else {
            return __builtin_nontemporal_load(
                reinterpret_cast<const f32x4v*>(C + (int64_t)row * ldc + col));
        }
    };
    auto store4 = [&](int row, int col, f32x4v v) {
        if constexpr (OUT16) {
            u32x2 w;
            w[0] = uint32_t{f32_to_f16_bits(v[0])} | (uint32_t{f32_to_f16_bits(v[1])} << 16);
            w[1] = uint32_t{f32_to_f16_bits(v[2])} | (uint32_t{f32_to_f16_bits(v[3])} << 16);
            *reinterpret_cast<u32x2*>(C + (int64_t)row * ldc + col) = w;
        } else {
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4v*>(C + (int64_t)row * ldc + col));
        }
    };
    auto quad = [&](int i, int g, int e) {
        return f32x4v{acc[i][4 * g][e], acc[i][4 * g + 1][e], acc[i][4 * g + 2][e],
                      acc[i][4 * g + 3][e]};
    };
    if (beta == 0.f) {
#pragma unroll
        for (int i = 0; i < GFM; ++i)
#pragma unroll
            for (int g = 0; g < GG; ++g)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (inside(row_of(i, e), col_of(g))) store4(row_of(i, e), col_of(g), alpha * quad(i, g, e));
        return;
    }
    f32x4v old[2][GG * 4];
    auto load_row = [&](int i, f32x4v(&d)[GG * 4]) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < GG; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                d[g * 4 + e] = inside(row_of(i, e), col_of(g)) ? load4(row_of(i, e), col_of(g))
                                                               : f32x4v{0.f, 0.f, 0.f, 0.f};
    };
    load_row(0, old[0]);
#pragma unroll
    for (int i = 0; i < GFM; ++i) {
        if (i + 1 < GFM) load_row(i + 1, old[(i + 1) & 1]);
#pragma unroll
        for (int g = 0; g < GG; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (!inside(row_of(i, e), col_of(g))) continue;
                const f32x4v a = quad(i, g, e), c = old[i & 1][g * 4 + e];
                f32x4v out;
#pragma unroll
                for (int x = 0; x < 4; ++x) out[x] = __builtin_fmaf(alpha, a[x], beta * c[x]);
                store4(row_of(i, e), col_of(g), out);
            }
        asm volatile("" ::: "memory");
    }
}

// Epilogue of the 16 x 16 blocks into a C stored transposed (the few-columns
// form: this workgroup computes C^T): element e of lane (q, r16) in block
// (i, j) is C^T[row][col] with row = row0 + 16 i + 4 q + e, col = col0 + 16 j
// + r16, stored at C[col * ldc + row], so a lane's four elements of a block
// are four consecutive floats (binary16 values), one 16-byte (8-byte) access
// when the rows of C allow it and all four lie inside.  Same value as the
// other epilogues: fma(alpha, acc, beta*c), beta == 0 never reads C.
template <int GFM, int GFN, bool OUT16, typename CT>
__device__ __forceinline__ void store_tile_t(const f32x4v (&acc)[GFM][GFN], CT* __restrict__ C,
                                             int64_t ldc, int row0, int col0, int M, int N,
                                             float alpha, float beta, int lane) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const int q = lane >> 4, r16 = lane & 15;
    auto h2f = [](uint32_t bits) {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
    };
    const bool vec = ldc % 4 == 0 && (reinterpret_cast<uintptr_t>(C) & (OUT16 ? 7 : 15)) == 0;
#pragma unroll
    for (int i = 0; i < GFM; ++i)
#pragma unroll
        for (int j = 0; j < GFN; ++j) {
            const int row = row0 + 16 * i + 4 * q, col = col0 + 16 * j + r16;
            if (col >= N || row >= M) continue;
            CT* at = C + (int64_t)col * ldc + row;
            if (vec && row + 3 < M) {
                f32x4v old = f32x4v{0.f, 0.f, 0.f, 0.f};
                if (beta != 0.f) {
                    if constexpr (OUT16) {
                        const u32x2 w = *reinterpret_cast<const u32x2*>(at);
                        old = f32x4v{h2f(w[0] & 0xffffu), h2f(w[0] >> 16), h2f(w[1] & 0xffffu),
                                     h2f(w[1] >> 16)};
                    } else {
                        old = *reinterpret_cast<const f32x4v*>(at);
                    }
                }
                f32x4v out;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    out[e] = beta == 0.f ? alpha * acc[i][j][e]
                                         : __builtin_fmaf(alpha, acc[i][j][e], beta * old[e]);
                if constexpr (OUT16) {
                    u32x2 w;
                    w[0] = uint32_t{f32_to_f16_bits(out[0])} | (uint32_t{f32_to_f16_bits(out[1])} << 16);
                    w[1] = uint32_t{f32_to_f16_bits(out[2])} | (uint32_t{f32_to_f16_bits(out[3])} << 16);
                    *reinterpret_cast<u32x2*>(at) = w;
                } else {
                    *reinterpret_cast<f32x4v*>(at) = out;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (row + e >= M) break;
                    const float a = acc[i][j][e];
                    if constexpr (OUT16) {
                        const float v = beta == 0.f ? alpha * a
                                                    : __builtin_fmaf(alpha, a, beta * h2f(at[e]));
                        at[e] = f32_to_f16_bits(v);
                    } else {
                        at[e] = beta == 0.f ? alpha * a : __builtin_fmaf(alpha, a, beta * at[e]);
                    }
                }
            }
        }
}

// F16: round to binary16 and multiply on v_mfma_f32_16x16x32_f16 (f16r);
// otherwise multiply the f32 values on v_mfma_f32_16x16x4_f32, eight steps a
// panel, step s taking from lane quarter q the s-th of its eight k (so the
// same fragment reads serve both modes).  TA: A stored K x M; TB: B stored
// N x K.
template <int BM, int BN, int NS, int WM, int WN, int GM, bool MASKED, bool OUT16, bool F16, bool TA,
          bool TB>
__global__ __launch_bounds__(WM * WN * 64) void gemm_panel_ring_kernel(DirectArgs p) {
    using S = PanelRingShape<BM, BN, NS, WM, WN, TA, TB>;
    using KA = KRowsPanel<BM>;
    constexpr int GFM = S::GFM, GFN = S::GFN, GG = GFN / 4;
    __shared__ __attribute__((aligned(1024))) unsigned char ring[NS * S::STAGE];

    int tm, tn;
    tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, GM, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int k_lo = blockIdx.y * p.depth;
    const int k_hi = min(p.K, k_lo + p.depth);
    const int nk = (k_hi - k_lo) / S::BK;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave / WN, wc = wave % WN;

    // Copy sources.  Rows layout (A, B^T): copy j of this wave fills the panel
    // rows 8u .. 8u + 7, u = wave + NW j: lane l takes row 8u + l / 8 at
    // position l % 8, which holds global chunk (l % 8) ^ swz<64>(row); rows
    // past M (N) read row M - 1 (N - 1).  k-rows of A^T: copy j fills group u,
    // lane l the four floats 4 (l % LPR) .. of the k-row in slot l / LPR (LPR
    // lanes a k-row; columns past M read column m0).  B: copy j fills bytes
    // 1024u .. 1024u + 1023 of the B panel: lane l the four floats at byte
    // 1024u + 16l, i.e. k-row (1024u + 16l) / B_ROW from column ((1024u + 16l)
    // % B_ROW) / 4 on (columns past N read column n0); copy j is copy 0 moved
    // down 1024 NW / B_ROW k-rows.
    const float* a_src[S::A_INS];
#pragma unroll
    for (int j = 0; j < S::A_INS; ++j) {
        if constexpr (TA) {
            constexpr int LPR = 64 / KA::RPI;
            const int col = m0 + 4 * (lane % LPR);
            const int kr = KA::RPI * (wave + S::NW * j) + KA::row_of_slot(lane / LPR);
            a_src[j] = p.A + (int64_t)(k_lo + kr) * p.lda + (col < p.M ? col : m0);
        } else {
            const int row = 8 * (wave + S::NW * j) + (lane >> 3);
            const int chunk = (lane & 7) ^ swz<64>(row & 15);
            a_src[j] = p.A + (int64_t)min(m0 + row, p.M - 1) * p.lda + k_lo + chunk * 4;
        }
    }
    const int64_t a_panel = TA ? (int64_t)S::BK * p.lda : S::BK;
    constexpr int A_DST = TA ? KA::GROUP : 1024;   // LDS bytes between copies
    const float* b_src[TB ? S::B_INS : 1];
    int64_t b_step = 0, b_panel = S::BK;
    if constexpr (TB) {
#pragma unroll
        for (int j = 0; j < S::B_INS; ++j) {
            const int row = 8 * (wave + S::NW * j) + (lane >> 3);
            const int chunk = (lane & 7) ^ swz<64>(row & 15);
            b_src[j] = p.B + (int64_t)min(n0 + row, p.N - 1) * p.ldb + k_lo + chunk * 4;
        }
    } else {
        const int b_byte = 1024 * wave + 16 * lane;
        const int bcol = n0 + (b_byte % S::B_ROW) / 4;
        b_src[0] = p.B + (int64_t)(k_lo + b_byte / S::B_ROW) * p.ldb + (bcol < p.N ? bcol : n0);
        b_step = (int64_t)(1024 / S::B_ROW) * S::NW * p.ldb;
        b_panel = (int64_t)S::BK * p.ldb;
    }

    auto stage_of = [&](int i) __attribute__((always_inline)) -> unsigned char* {
        return ring + i * S::STAGE;
    };
    auto fill = [&](unsigned char* stage, int kt) __attribute__((always_inline)) {
        const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(stage));
#pragma unroll
        for (int j = 0; j < S::A_INS; ++j)
            lds_copy16(a_src[j] + kt * a_panel, base + (wave + S::NW * j) * A_DST);
#pragma unroll
        for (int j = 0; j < S::B_INS; ++j) {
            if constexpr (TB)
                lds_copy16(b_src[j] + kt * b_panel, base + S::A_BYTES + (wave + S::NW * j) * 1024);
            else
                lds_copy16(b_src[0] + j * b_step + kt * b_panel,
                           base + S::A_BYTES + (wave + S::NW * j) * 1024);
        }
    };

    // Fragment reads of lane (q, r16): a row r16 of a block at logical chunks
    // q and q + 4 (A; B^T at row r16 of a 16-column block); A^T k-rows 4q ..
    // 4q + 3 and 16 + 4q .. 16 + 4q + 3 at column r16 of a block; B k-rows
    // 4q .. 4q + 3 and 16 + 4q .. 16 + 4q + 3 at the lane's four columns of a
    // 64-column group.
    const int r16 = lane & 15, q = lane >> 4;
    const int a_row = (wr * S::TM + r16) * S::A_ROW;
    const int a_off0 = TA ? KA::at(4 * q, wr * S::TM + r16) : a_row + ((q ^ swz<64>(r16)) << 4);
    const int a_off1 = TA ? KA::at(16 + 4 * q, wr * S::TM + r16)
                          : a_row + (((q + 4) ^ swz<64>(r16)) << 4);
    const int b_row = S::A_BYTES + (wc * S::TN + r16) * S::B_ROW;   // B^T
    const int b_off = TB ? b_row + ((q ^ swz<64>(r16)) << 4)
                         : S::A_BYTES + 4 * q * S::B_ROW + (wc * S::TN + 4 * r16) * 4;
    const int b_off1 = b_row + (((q + 4) ^ swz<64>(r16)) << 4);

    f32x4v acc[GFM][GFN];
#pragma unroll
    for (int i = 0; i < GFM; ++i)
#pragma unroll
        for (int j = 0; j < GFN; ++j) acc[i][j] = f32x4v{0.f, 0.f, 0.f, 0.f};

    // Prologue: panels 0 .. NS - 2 (a short slice reloads its last panel, so
    // the count of copies in flight is the same every panel).
#pragma unroll
    for (int i = 0; i + 1 < NS; ++i) fill(stage_of(i), min(i, nk - 1));
    for (int kt = 0; kt < nk; ++kt) {
        // this wave's copies of panel kt have landed; after the barrier every
        // wave's have, and every wave is done reading the stage of panel kt - 1
        wait_vmcnt<(NS - 2) * S::FILLS>();
        ring_barrier();
        fill(stage_of((kt + NS - 1) % NS), min(kt + NS - 1, nk - 1));
        const lds_u8* st = (const lds_u8*)(stage_of(kt % NS));
        f32x4v a0[GFM], a1[GFM];
#pragma unroll
        for (int i = 0; i < GFM; ++i) {
            if constexpr (TA) {
                // k-row offsets relative to k-row 4q (16 + 4q): KA::at is
                // additive over whole multiples of RPI and 4q's own slot
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    a0[i][t] = *reinterpret_cast<lds_f32c*>(st + a_off0 + KA::at(t, 16 * i));
                    a1[i][t] = *reinterpret_cast<lds_f32c*>(st + a_off1 + KA::at(t, 16 * i));
                }
            } else {
                a0[i] = *reinterpret_cast<lds_f32x4c*>(st + a_off0 + i * 16 * S::A_ROW);
                a1[i] = *reinterpret_cast<lds_f32x4c*>(st + a_off1 + i * 16 * S::A_ROW);
            }
        }
        if constexpr (TB) {
            f32x4v b0[GFN], b1[GFN];
#pragma unroll
            for (int j = 0; j < GFN; ++j) {
                b0[j] = *reinterpret_cast<lds_f32x4c*>(st + b_off + j * 16 * S::B_ROW);
                b1[j] = *reinterpret_cast<lds_f32x4c*>(st + b_off1 + j * 16 * S::B_ROW);
            }
            if constexpr (F16) {
                f16x8 fa[GFM], fb[GFN];
#pragma unroll
                for (int i = 0; i < GFM; ++i) fa[i] = rn8(a0[i], a1[i]);
#pragma unroll
                for (int j = 0; j < GFN; ++j) fb[j] = rn8(b0[j], b1[j]);
#pragma unroll
                for (int i = 0; i < GFM; ++i)
#pragma unroll
                    for (int j = 0; j < GFN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
            } else {
#pragma unroll
                for (int t = 0; t < 8; ++t)
#pragma unroll
                    for (int i = 0; i < GFM; ++i)
#pragma unroll
                        for (int j = 0; j < GFN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                t < 4 ? a0[i][t] : a1[i][t - 4], t < 4 ? b0[j][t] : b1[j][t - 4],
                                acc[i][j], 0, 0, 0);
            }
        } else if constexpr (F16) {
            f16x8 fa[GFM], fb[GFN];
#pragma unroll
            for (int i = 0; i < GFM; ++i) fa[i] = rn8(a0[i], a1[i]);
#pragma unroll
            for (int g = 0; g < GG; ++g) {
                f32x4v v[8];
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    v[t] = *reinterpret_cast<lds_f32x4c*>(st + b_off + (t < 4 ? t : t + 12) * S::B_ROW +
                                                          g * 256);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    fb[4 * g + jj] = rn8(f32x4v{v[0][jj], v[1][jj], v[2][jj], v[3][jj]},
                                         f32x4v{v[4][jj], v[5][jj], v[6][jj], v[7][jj]});
            }
#pragma unroll
            for (int i = 0; i < GFM; ++i)
#pragma unroll
                for (int j = 0; j < GFN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        } else {
#pragma unroll
            for (int g = 0; g < GG; ++g) {
                f32x4v v[8];
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    v[t] = *reinterpret_cast<lds_f32x4c*>(st + b_off + (t < 4 ? t : t + 12) * S::B_ROW +
                                                          g * 256);
#pragma unroll
                for (int t = 0; t < 8; ++t)
#pragma unroll
                    for (int i = 0; i < GFM; ++i)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
                            acc[i][4 * g + jj] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                t < 4 ? a0[i][t] : a1[i][t - 4], v[t][jj], acc[i][4 * g + jj], 0, 0, 0);
            }
        }
    }
    wait_vmcnt<0>();   // no copy may still be landing in LDS when the workgroup ends

    if (p.slices > 1 && !last_slice_adds<GFM, GFN, BM * BN * 4>(acc, p, wave, lane, ring)) return;
    const int row0 = m0 + wr * S::TM, col0 = n0 + wc * S::TN;
    if constexpr (TB) {
        if (p.tc) {
            if constexpr (OUT16)
                store_tile_t<GFM, GFN, true>(acc, p.C16, p.ldc, row0, col0, p.M, p.N, p.alpha,
                                             p.beta, lane);
            else
                store_tile_t<GFM, GFN, false>(acc, p.C, p.ldc, row0, col0, p.M, p.N, p.alpha,
                                              p.beta, lane);
        } else if constexpr (OUT16) {
            store_tile_m16<GFM, GFN, MASKED, true>(acc, p.C16, p.ldc, row0, col0, p.M, p.N, p.alpha,
                                                   p.beta, lane);
        } else {
            store_tile_m16<GFM, GFN, MASKED, false>(acc, p.C, p.ldc, row0, col0, p.M, p.N, p.alpha,
                                                    p.beta, lane);
        }
    } else if constexpr (OUT16) {
        store_tile_dealt<GFM, GFN, MASKED, true>(acc, p.C16, p.ldc, row0, col0, p.M, p.N, p.alpha,
                                                 p.beta, lane);
    } else {
        store_tile_dealt<GFM, GFN, MASKED, false>(acc, p.C, p.ldc, row0, col0, p.M, p.N, p.alpha,
                                                  p.beta, lane);
    }
}

template <int BM, int BN, int NS, int WM, int WN, int GM, bool F16, bool TA, bool TB>
hipError_t launch_panel_ring_layout(const DirectArgs& a, bool masked, hipStream_t s) {
    const dim3 grid(a.tiles_m * a.tiles_n, a.slices), block(WM * WN * 64);
    const bool edge = masked || a.M % BM != 0 || a.N % BN != 0;
    if constexpr (F16) {
        if (a.C16) {
            if (edge)
                gemm_panel_ring_kernel<BM, BN, NS, WM, WN, GM, true, true, true, TA, TB><<<grid, block, 0, s>>>(a);
            else
                gemm_panel_ring_kernel<BM, BN, NS, WM, WN, GM, false, true, true, TA, TB><<<grid, block, 0, s>>>(a);
            return hipGetLastError();
        }
    }
    if (edge) gemm_panel_ring_kernel<BM, BN, NS, WM, WN, GM, true, false, F16, TA, TB><<<grid, block, 0, s>>>(a);
    else gemm_panel_ring_kernel<BM, BN, NS, WM, WN, GM, false, false, F16, TA, TB><<<grid, block, 0, s>>>(a);
    return hipGetLastError();
}

template <int BM, int BN, int NS, int WM, int WN, int GM, bool F16>
hipError_t launch_panel_ring(const DirectArgs& a, bool ta, bool tb, bool masked, hipStream_t s) {
    // the host hands only the shapes this kernel takes (panel_ring_takes)
    if ((!tb && a.N % 4 != 0) || (ta && a.M % 4 != 0) || a.K % 32 != 0 || a.depth % 32 != 0 ||
        a.K <= 0 || (!F16 && a.C16) || (a.tc && !tb))
        return hipErrorInvalidValue;
    if (ta && tb) return launch_panel_ring_layout<BM, BN, NS, WM, WN, GM, F16, true, true>(a, masked, s);
    if (ta) return launch_panel_ring_layout<BM, BN, NS, WM, WN, GM, F16, true, false>(a, masked, s);
    if (tb) return launch_panel_ring_layout<BM, BN, NS, WM, WN, GM, F16, false, true>(a, masked, s);
    return launch_panel_ring_layout<BM, BN, NS, WM, WN, GM, F16, false, false>(a, masked, s);
}

#define G355_PANEL_RING_F16R(BM, BN, NS, WM, WN, GM) \
    {{GEMM355_MODE_F16R, BM, BN, 32, NS, WM, WN, GM, 3}, &launch_panel_ring<BM, BN, NS, WM, WN, GM, true>},
#define G355_PANEL_RING_F32(BM, BN, NS, WM, WN, GM) \
    {{GEMM355_MODE_F32, BM, BN, 32, NS, WM, WN, GM, 3}, &launch_panel_ring<BM, BN, NS, WM, WN, GM, false>},

const DirectInstance kF16rInstances[] = {G355_PANEL_RING_F16R_CONFIGS(G355_PANEL_RING_F16R)};
const DirectInstance kF32Instances[] = {G355_PANEL_RING_F32_CONFIGS(G355_PANEL_RING_F32)};

}  // namespace

const DirectInstance* panel_ring_instances(int mode, int* count) {
    if (mode == GEMM355_MODE_F32) {
        *count = static_cast<int>(sizeof(kF32Instances) / sizeof(kF32Instances[0]));
        return kF32Instances;
    }
    *count = static_cast<int>(sizeof(kF16rInstances) / sizeof(kF16rInstances[0]));
    return kF16rInstances;
}

bool panel_ring_takes(bool ta, bool tb, const float* A, int64_t lda, const float* B, int64_t ldb,
                      int64_t M, int64_t N, int64_t K) {
    auto vec = [](const float* p, int64_t ld) {
        return ld % 4 == 0 && (reinterpret_cast<uintptr_t>(p) & 15) == 0;
    };
    return vec(A, lda) && vec(B, ldb) && (tb || N % 4 == 0) && (!ta || M % 4 == 0) && K % 32 == 0 &&
           K > 0;
}

}  // namespace g355
