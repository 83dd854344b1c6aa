// f16_kernel.hpp -- the f16 GEMM kernel templates of libgemm355 (the f16r
// mode on rounded, packed operands), shared by the translation unit of the
// f32 output (gemm_f16r.hip, which also holds the rounding/packing pass and
// the table of configurations) and that of the binary16 output
// (gemm_f16r_o16.hip).  Not part of the public ABI.
#pragma once

#include <type_traits>
#include <utility>

#include "internal.hpp"

namespace g355 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------------------
// Packed operand layout.  Rows (of A, or columns of B) are grouped in blocks
// of kPackRows, depth in blocks of D values (D = 64 or 32, the depth of the
// panel the GEMM configuration multiplies from).  Block (xb, kb) starts at
// element ((xb * nkb) + kb) * kPackRows * D.  Inside it, row r holds its D
// values as D/8 chunks of 8, logical chunk c at position c ^ swz(r):
//   D = 64 (128-byte rows): swz(r) = (r / 2) % 8
//   D = 32 ( 64-byte rows): swz(r) = (r / 2) % 4
// so that rows r and r + 2 never hold a logical chunk at the same position.
// A fragment read has 16 lanes take 16 consecutive rows at one logical chunk
// (ds_read_b128).  Measured on gfx950 (a probe timing 16-byte LDS reads of
// fixed lane patterns): both keys read at the full 16-byte rate; 64-byte rows
// keyed by (r / 4) % 4 -- distinct 16-byte slots within every 256 bytes, but
// rows r and r + 2 alike -- take two passes per read, as do unswizzled rows.
// ----------------------------------------------------------------------------
constexpr int kPackRows = 256;
constexpr int kPackK = 64;   // the padded depth is a multiple of this for every D

template <int D>
__device__ __forceinline__ int swz(int r) {
    static_assert(D == 32 || D == 64, "panel depth");
    return (r / 2) % (D / 8);
}

template <int D>
__device__ __forceinline__ int64_t packed_offset(int64_t x, int kb, int c, int64_t nkb) {
    const int64_t xb = x / kPackRows;
    const int r = static_cast<int>(x - xb * kPackRows);
    return ((xb * nkb + kb) * kPackRows + r) * D + ((c ^ swz<D>(r)) << 3);
}

// ----------------------------------------------------------------------------
// The f16 GEMM on the packed operands.
//
// A stage holds the BK = 64 deep panels of A (BM rows) and B (BN columns) of
// one k step, in the packed image: 128 bytes per row.  The stages form a ring
// of ST buffers in LDS, filled by direct global->LDS loads
// (global_load_lds_dwordx4): one wave instruction copies one contiguous
// kilobyte of a packed block into the same kilobyte of the stage without
// passing through registers.  Fills run ST-1 panels ahead of the panel being
// multiplied.  The K loop is unrolled by ST, so every stage is named
// statically (a fixed shared-memory address).
// ----------------------------------------------------------------------------
typedef __attribute__((address_space(3))) const f16x8 lds_f16x8;
typedef __attribute__((address_space(1))) void glb_void;

template <int BM, int BN, int ST, int WM, int WN>
struct F16Shape {
    static constexpr int BK = kPackK;
    static constexpr int NW = WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 32, FN = TN / 32;
    static constexpr int ROW = BK * 2;              // bytes per panel row
    static constexpr int KSTEPS = BK / 16;          // matrix instructions per block per panel
    static constexpr int A_BYTES = BM * ROW;
    static constexpr int STAGE = (BM + BN) * ROW;   // bytes per stage
    static constexpr int A_INS = A_BYTES / 1024 / NW;   // fill instructions per wave per stage
    static constexpr int B_INS = BN * ROW / 1024 / NW;
    static constexpr int FILLS = A_INS + B_INS;
    static_assert(ST >= 2 && ST <= 3, "2 or 3 stages");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(A_INS * 1024 * NW == A_BYTES && B_INS * 1024 * NW == BN * ROW,
                  "kilobytes of a panel split evenly over the waves");
    static_assert(kPackRows % BM == 0 && kPackRows % BN == 0, "tiles nest in packed blocks");
    static_assert(ST * STAGE <= 160 * 1024, "LDS budget of one CU");
};

// Word 3 of a raw buffer descriptor on gfx9-family GPUs: 32-bit data format
// (a zero format would make every load return zero), no swizzle, no index
// stride; bounds are checked against the record count in bytes.
constexpr int kBufferFlags = 0x00020000;

template <int BM, int BN, int ST, int WM, int WN, int GM, bool RS, bool MASKED, bool OUT16>
__global__ __launch_bounds__(WM * WN * 64) void gemm_f16_kernel(F16Args p) {
    using S = F16Shape<BM, BN, ST, WM, WN>;
    __shared__ __attribute__((aligned(1024))) unsigned char ring0[S::STAGE];
    __shared__ __attribute__((aligned(1024))) unsigned char ring1[S::STAGE];
    __shared__ __attribute__((aligned(1024))) unsigned char ring2[ST > 2 ? S::STAGE : 16];

    int tm, tn;
    tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, GM, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave / WN, wc = wave % WN;
    const int h = lane >> 5;
    const int r32 = lane & 31;
    const int64_t nkb = p.nkb;

    // Panel kt of this tile's A rows is the BM-row slice at row m0 % 256 of
    // packed block (m0 / 256, kt); consecutive kt are consecutive blocks.
    const unsigned char* a_tile = reinterpret_cast<const unsigned char*>(
        p.A16 + ((int64_t)(m0 / kPackRows) * nkb * kPackRows + m0 % kPackRows) * kPackK);
    const unsigned char* b_tile = reinterpret_cast<const unsigned char*>(
        p.B16t + ((int64_t)(n0 / kPackRows) * nkb * kPackRows + n0 % kPackRows) * kPackK);
    const int lane_ofs = wave * 1024 + lane * 16;
    const unsigned char* a_src = a_tile + lane_ofs;
    const unsigned char* b_src = b_tile + lane_ofs;
    constexpr int64_t kBlockBytes = int64_t{kPackRows} * kPackK * 2;

    auto fill = [&](unsigned char* stage, int kt) __attribute__((always_inline)) {
        const uint32_t as = __builtin_amdgcn_readfirstlane(lds_addr(stage) + wave * 1024);
        const uint32_t bs = as + S::A_BYTES;
        const int64_t kofs = (int64_t)kt * kBlockBytes;
#pragma unroll
        for (int j = 0; j < S::A_INS; ++j)
            lds_copy16(a_src + kofs + j * S::NW * 1024, as + j * S::NW * 1024);
#pragma unroll
        for (int j = 0; j < S::B_INS; ++j)
            lds_copy16(b_src + kofs + j * S::NW * 1024, bs + j * S::NW * 1024);
    };

    // Register-staged fills (RS): the same kilobytes go through VGPRs --
    // load(kt) issues the 16-byte loads of panel kt into `stg`, commit(stage)
    // writes them to the same offsets of the stage.  The loads are buffer
    // loads: the panel's base address lives in a scalar descriptor (rebuilt
    // per panel with scalar arithmetic) whose record count is exactly the
    // panel's bytes, and every load of the wave shares one 32-bit lane offset,
    // so no 64-bit vector address is formed per load.
    u32x4 stg[RS ? S::FILLS : 1];
    auto load = [&](int kt) __attribute__((always_inline)) {
        const int64_t kofs = (int64_t)kt * kBlockBytes;
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a_tile + kofs), (short)0, S::A_BYTES, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(b_tile + kofs), (short)0, BN * S::ROW, kBufferFlags);
#pragma unroll
        for (int j = 0; j < S::A_INS; ++j)
            stg[j] = __builtin_amdgcn_raw_buffer_load_b128(ra, lane_ofs, j * S::NW * 1024, 0);
#pragma unroll
        for (int j = 0; j < S::B_INS; ++j)
            stg[S::A_INS + j] = __builtin_amdgcn_raw_buffer_load_b128(rb, lane_ofs, j * S::NW * 1024, 0);
    };
    auto commit = [&](unsigned char* stage) __attribute__((always_inline)) {
        lds_u8* as = (lds_u8*)(stage) + wave * 1024 + lane * 16;
        lds_u8* bs = (lds_u8*)(stage) + S::A_BYTES + wave * 1024 + lane * 16;
#pragma unroll
        for (int j = 0; j < S::A_INS; ++j)
            *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(as + j * S::NW * 1024) =
                stg[j];
#pragma unroll
        for (int j = 0; j < S::B_INS; ++j)
            *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(bs + j * S::NW * 1024) =
                stg[S::A_INS + j];
    };

    // Fragment reads: lane (h, r32) of block i reads row r32 of the block at
    // logical chunk h*4 + ks (lane half h feeds k in [32h, 32h+32) of the
    // panel, 8 per instruction, to A and B alike).  Blocks start at multiples
    // of 32 rows (of 16 within the packed block), so the row's swizzle key is
    // swz(r32).
    const int sw = swz<kPackK>(r32);
    const int a_row0 = (wr * S::TM + r32) * S::ROW;
    const int b_row0 = S::A_BYTES + (wc * S::TN + r32) * S::ROW;
    auto frags = [&](const unsigned char* stage, int ks, f16x8 (&a)[S::FM], f16x8 (&b)[S::FN]) {
        const lds_u8* base = (const lds_u8*)(stage);
        const int chunk = ((h * S::KSTEPS + ks) ^ sw) << 4;
#pragma unroll
        for (int i = 0; i < S::FM; ++i)
            a[i] = *reinterpret_cast<lds_f16x8*>(base + a_row0 + i * 32 * S::ROW + chunk);
#pragma unroll
        for (int j = 0; j < S::FN; ++j)
            b[j] = *reinterpret_cast<lds_f16x8*>(base + b_row0 + j * 32 * S::ROW + chunk);
    };

    // The accumulators get their first value from the first matrix
    // instruction of the first panel, with an inline-constant zero as its
    // addend, so they are born in the accumulation registers instead of being
    // zeroed in general registers and copied over.
    f32x16 acc[S::FM][S::FN];
    using first_panel = std::true_type;
    using later_panel = std::false_type;

    constexpr int NMF = S::FM * S::FN;
    constexpr int NFR = S::FM + S::FN;
    const int nk = static_cast<int>(nkb);
    auto stage_of = [&](int i) __attribute__((always_inline)) -> unsigned char* { return i == 0 ? ring0 : i == 1 ? ring1 : ring2; };

    // Multiply one stage: fragments of step ks+1 are read while step ks
    // multiplies.
    auto multiply = [&](const unsigned char* cur, auto first) __attribute__((always_inline)) {
        f16x8 a[2][S::FM], b[2][S::FN];
        frags(cur, 0, a[0], b[0]);
        const f32x16 zero = {};
#pragma unroll
        for (int ks = 0; ks < S::KSTEPS; ++ks) {
            if (ks + 1 < S::KSTEPS) frags(cur, ks + 1, a[(ks + 1) & 1], b[(ks + 1) & 1]);
#pragma unroll
            for (int i = 0; i < S::FM; ++i)
#pragma unroll
                for (int j = 0; j < S::FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        a[ks & 1][i], b[ks & 1][j],
                        (decltype(first)::value && ks == 0) ? zero : acc[i][j], 0, 0, 0);
        }
    };

    if constexpr (!RS) {
        // One panel: fill panel kt+ST-1 into the stage freed by panel kt-1
        // (every wave passed the barrier after reading it), multiply the
        // current stage, then wait until panel kt+1 has landed -- the fills of
        // later panels may stay in flight -- and for every other wave.  Fills
        // past the last panel reload the last panel into a stage nobody reads
        // again, so the wave's count of outstanding fills is the same at every
        // step and the step is one basic block, which the group barriers below
        // order: fills, then the first fragments, then one matrix instruction
        // after another with the next step's fragment reads between them.
        auto panel = [&](const unsigned char* cur, unsigned char* freed, int kt_fill,
                         auto first) __attribute__((always_inline)) {
            fill(freed, kt_fill);
            multiply(cur, first);
            __builtin_amdgcn_sched_group_barrier(0x020, S::FILLS, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, NFR, 0);
#pragma unroll
            for (int ks = 0; ks < S::KSTEPS; ++ks) {
#pragma unroll
                for (int m = 0; m < NMF; ++m) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (ks + 1 < S::KSTEPS && m < NFR)
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            }
            wait_vmcnt<(ST - 2) * S::FILLS>();
            ring_barrier();
        };

        // Prologue: panels 0 .. ST-2 into stages 0 .. ST-2, then wait for panel 0.
#pragma unroll
        for (int i = 0; i + 1 < ST; ++i) fill(stage_of(i), min(i, nk - 1));
        wait_vmcnt<(ST - 2) * S::FILLS>();
        ring_barrier();

        panel(stage_of(0), stage_of(ST - 1), min(ST - 1, nk - 1), first_panel{});
#pragma unroll
        for (int u = 1; u < ST; ++u)
            if (u < nk) panel(stage_of(u), stage_of(u - 1), min(u + ST - 1, nk - 1), later_panel{});
        for (int kt = ST; kt < nk; kt += ST) {
#pragma unroll
            for (int u = 0; u < ST; ++u) {
                if (u == 0 || kt + u < nk)
                    panel(stage_of(u), stage_of((u + ST - 1) % ST), min(kt + u + ST - 1, nk - 1),
                          later_panel{});
            }
        }
        wait_vmcnt<0>();   // no fill may still be landing in LDS when the workgroup ends
    } else {
        // Register-staged ring of two stages: while stage kt%2 is multiplied,
        // panel kt+1 (loaded into registers during the previous panel) is
        // written to the other stage, then the loads of panel kt+2 are issued.
        // The group barriers spread the writes between the matrix
        // instructions of the first step and the loads between those of the
        // second, so the loads have most of a panel to arrive.
        static_assert(ST == 2, "the register-staged ring has two stages");
        auto panel = [&](const unsigned char* cur, unsigned char* next, int kt_load,
                         auto first) __attribute__((always_inline)) {
            multiply(cur, first);
            commit(next);
            load(kt_load);
            __builtin_amdgcn_sched_group_barrier(0x100, NFR, 0);
#pragma unroll
            for (int ks = 0; ks < S::KSTEPS; ++ks) {
#pragma unroll
                for (int m = 0; m < NMF; ++m) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (ks + 1 < S::KSTEPS && m < NFR)
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    if (ks == 0 && m < S::FILLS) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                    if (ks == 1 && m < S::FILLS) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
            }
            ring_barrier();
        };
        load(0);
        commit(ring0);
        load(min(1, nk - 1));
        ring_barrier();
        panel(ring0, ring1, min(2, nk - 1), first_panel{});
        if (1 < nk) panel(ring1, ring0, min(3, nk - 1), later_panel{});
        for (int kt = 2; kt < nk; kt += 2) {
            panel(ring0, ring1, min(kt + 2, nk - 1), later_panel{});
            if (kt + 1 < nk) panel(ring1, ring0, min(kt + 3, nk - 1), later_panel{});
        }
        wait_vmcnt<0>();
    }

    // Epilogue: C = alpha*acc + beta*C over this wave's part of the tile.
    if constexpr (OUT16)
        store_tile16<S::FM, S::FN, MASKED>(acc, p.C16, p.ldc, m0 + wr * S::TM, n0 + wc * S::TN,
                                           p.M, p.N, p.alpha, p.beta, lane);
    else
        store_tile<S::FM, S::FN, MASKED>(acc, p.C, p.ldc, m0 + wr * S::TM, n0 + wc * S::TN, p.M,
                                         p.N, p.alpha, p.beta, lane);
}

// ----------------------------------------------------------------------------
// The half-depth ring.  Panels are BK = 32 deep (64 bytes per row, packed
// blocks of depth 32), and NS of them (up to 5 x 32 KB for a 256 x 256 tile,
// all of a CU's shared memory) form a ring filled direct from the packed
// blocks, so NS - 1 panels -- up to two 64-deep steps of the full-depth ring
// -- are in flight while one is multiplied; the fills then have several
// microseconds to arrive from the memory-side cache when they miss in L2.
//
// The matrix instruction is v_mfma_f32_16x16x32_f16: one panel is one step of
// 32 k for every 16 x 16 block of the wave tile.  For the same flops it moves
// half the accumulator bytes of the 32x32x16 form through the register file
// per instruction, and on this GPU, whose f16 GEMMs run at the power limit,
// that measured about 4% faster at 8192^3.  The wave tile is GFM x GFN blocks;
// the A fragments of rows 0..H-1 (H = GFM/2) and all B fragments of a panel
// are read before it starts.  First half: rows 0..H-1 are multiplied while the
// A fragments of rows H.. are read and this wave's fills of the panel NS - 1
// ahead are issued.  Then the wave waits for its fills of the next panel and
// passes the barrier (every wave's fills of the next panel have landed, every
// wave has read all of this one).  Second half: rows H.. are multiplied while
// the next panel's B fragments (into the other of two buffers) and A rows
// 0..H-1 are read.  So the matrix instructions never wait for shared memory
// right after a barrier.
// ----------------------------------------------------------------------------
template <int BM, int BN, int NS, int WM, int WN>
struct RingShape {
    static constexpr int BK = 32;
    static constexpr int NW = WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int GFM = TM / 16, GFN = TN / 16;   // 16 x 16 blocks per wave
    static constexpr int H = GFM / 2;
    static constexpr int ROW = BK * 2;              // bytes per panel row
    static constexpr int A_BYTES = BM * ROW;
    static constexpr int STAGE = (BM + BN) * ROW;   // bytes per stage
    static constexpr int A_INS = A_BYTES / 1024 / NW;   // fill instructions per wave per panel
    static constexpr int B_INS = BN * ROW / 1024 / NW;
    static constexpr int FILLS = A_INS + B_INS;
    static_assert(NS >= 3 && NS <= 5, "3 to 5 stages");
    static_assert(TM % 32 == 0 && TN % 16 == 0, "wave tile must be an even number of block rows");
    static_assert(A_INS >= 1 && B_INS >= 1 && A_INS * 1024 * NW == A_BYTES &&
                      B_INS * 1024 * NW == BN * ROW,
                  "kilobytes of a panel split evenly over the waves");
    static_assert(kPackRows % BM == 0 && kPackRows % BN == 0, "tiles nest in packed blocks");
    static_assert(NS * STAGE <= 160 * 1024, "LDS budget of one CU");
    static_assert((NS - 2) * FILLS < 64, "vmcnt range");
};

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Epilogue of the 16 x 16 blocks: element e of lane l in block (i, j) sits at
// row 16 i + 4 (l / 16) + e, column 16 j + l % 16.  Same value as store_tile,
// fma(alpha, acc, beta*c), for f32 or binary16 C (read widened, rounded once
// to nearest even).  beta == 0 never reads C.  With beta != 0 the loads of a
// row of blocks are issued before the stores of the previous row.
template <int FM, int FN, bool MASKED, bool OUT16, typename CT>
__device__ __forceinline__ void store_tile_m16(const f32x4 (&acc)[FM][FN], CT* __restrict__ C,
                                               int64_t ldc, int row0, int col0, int M, int N,
                                               float alpha, float beta, int lane) {
    const int q = lane >> 4, r16 = lane & 15;
    auto row_of = [&](int i, int e) { return row0 + i * 16 + 4 * q + e; };
    auto col_of = [&](int j) { return col0 + j * 16 + r16; };
    auto inside = [&](int row, int col) { return !MASKED || (row < M && col < N); };
    auto ld = [&](int row, int col) -> float {
        if constexpr (OUT16)
            return static_cast<float>(__builtin_bit_cast(_Float16, C[(int64_t)row * ldc + col]));
        else
            return __builtin_nontemporal_load(C + (int64_t)row * ldc + col);
    };
    auto st = [&](int row, int col, float v) {
        if constexpr (OUT16)
            C[(int64_t)row * ldc + col] = f32_to_f16_bits(v);
        else
            __builtin_nontemporal_store(v, C + (int64_t)row * ldc + col);
    };
    if (beta == 0.f) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (inside(row_of(i, e), col_of(j)))
                        st(row_of(i, e), col_of(j), alpha * acc[i][j][e]);
        return;
    }
    float v[2][FN * 4];
    auto load_row = [&](int i, float(&d)[FN * 4]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                d[j * 4 + e] = inside(row_of(i, e), col_of(j)) ? ld(row_of(i, e), col_of(j)) : 0.f;
    };
    load_row(0, v[0]);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        if (i + 1 < FM) load_row(i + 1, v[(i + 1) & 1]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (inside(row_of(i, e), col_of(j)))
                    st(row_of(i, e), col_of(j),
                       __builtin_fmaf(alpha, acc[i][j][e], beta * v[i & 1][j * 4 + e]));
        asm volatile("" ::: "memory");
    }
}

// The staged epilogue's shared memory per wave: 16 rows of TN floats, rows
// TN + 4 floats apart (the four lane quarters of a block write four rows at
// once; the padding puts them in different banks).
template <int TN>
struct StagedRows {
    static constexpr int RS = TN + 4;
    static constexpr int BYTES = 16 * RS * 4;
};

// Epilogue through shared memory for a tile whose C rows allow vector
// accesses (f32: 16-byte aligned rows; binary16: 8-byte aligned): one 16-row
// band of the wave's tile at a time is written to the wave's own shared
// memory in the matrix-instruction layout and read back as four consecutive
// columns per lane, so C is read (beta != 0) and written in whole 128-byte
// row segments instead of the 64-byte (f32) or 32-byte (binary16) ones of the
// block layout.  The same value as store_tile / store_tile16: fma(alpha, acc,
// beta*c), binary16 C widened exactly and the result rounded once to nearest
// even.  A wave's shared-memory instructions complete in order, so no wait
// separates the write of a band, its read-back and the next band's write.
// MASKED (a tile of a ragged launch) skips rows >= M and columns >= N: a lane
// whose four columns all lie inside keeps its one access, the lane across the
// edge goes element by element.  Rows that do not allow vector accesses
// (!vec) are read back one column per lane instead, 64 lanes on 64
// consecutive columns of a row: single-element accesses, still whole row
// segments per instruction.
template <int FM, int FN, int TN, bool OUT16, bool MASKED, typename CT>
__device__ __forceinline__ void store_tile_m16_staged(const f32x4 (&acc)[FM][FN],
                                                      CT* __restrict__ C, int64_t ldc,
                                                      int row0, int col0, int M, int N, float alpha,
                                                      float beta, int lane, unsigned char* stage,
                                                      bool vec) {
    using R = StagedRows<TN>;
    static_assert(FN * 16 == TN, "a band is the wave tile's width");
    constexpr int LPR = TN / 4;        // lanes per staged row (four columns each)
    constexpr int RPI = 64 / LPR;      // rows per read-back instruction
    constexpr int IT = 16 / RPI;
    typedef __attribute__((address_space(3))) float lds_f32;
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    lds_f32* st = (lds_f32*)(stage);
    const int q = lane >> 4, r16 = lane & 15;
    const int rr0 = lane / LPR, c4 = lane % LPR;
    auto c_at = [&](int i, int it) {
        return C + (int64_t)(row0 + 16 * i + it * RPI + rr0) * ldc + col0 + 4 * c4;
    };
    // how many of the lane's four columns of staged row (i, it) are inside
    // C: 4 (one access), 1..3 (element by element) or 0
    auto inside = [&](int i, int it) -> int {
        if constexpr (!MASKED) return 4;
        const int row = row0 + 16 * i + it * RPI + rr0, col = col0 + 4 * c4;
        return row < M ? max(0, min(4, N - col)) : 0;
    };
    // binary16 C: four values as two 32-bit words (low half first)
    auto h2f = [](uint32_t bits) {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
    };
    auto load4 = [&](int i, int it) -> f32x4 {
        const int n = inside(i, it);
        if (n == 4) {
            if constexpr (OUT16) {
                const u32x2 w = *reinterpret_cast<const u32x2*>(c_at(i, it));
                return f32x4{h2f(w[0] & 0xffffu), h2f(w[0] >> 16), h2f(w[1] & 0xffffu),
                             h2f(w[1] >> 16)};
            } else {
                return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(c_at(i, it)));
            }
        }
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        for (int e = 0; e < n; ++e) {
            if constexpr (OUT16) v[e] = h2f(c_at(i, it)[e]);
            else v[e] = c_at(i, it)[e];
        }
        return v;
    };
    auto store4 = [&](int i, int it, f32x4 v) {
        const int n = inside(i, it);
        if (n == 4) {
            if constexpr (OUT16) {
                u32x2 w;
                w[0] = uint32_t{f32_to_f16_bits(v[0])} | (uint32_t{f32_to_f16_bits(v[1])} << 16);
                w[1] = uint32_t{f32_to_f16_bits(v[2])} | (uint32_t{f32_to_f16_bits(v[3])} << 16);
                *reinterpret_cast<u32x2*>(c_at(i, it)) = w;
            } else {
                __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(c_at(i, it)));
            }
            return;
        }
        for (int e = 0; e < n; ++e) {
            if constexpr (OUT16) c_at(i, it)[e] = f32_to_f16_bits(v[e]);
            else c_at(i, it)[e] = v[e];
        }
    };
    auto stage_band = [&](int i) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) st[(4 * q + e) * R::RS + 16 * j + r16] = acc[i][j][e];
    };
    auto staged = [&](int it) __attribute__((always_inline)) {
        return *(const lds_f32x4*)(st + (it * RPI + rr0) * R::RS + 4 * c4);
    };
    if (!vec) {
        // one column per lane: staged row rr, columns 64 h + lane
        constexpr int H = TN / 64;
        static_assert(TN % 64 == 0, "whole 64-column groups");
        auto at = [&](int i, int rr, int h) {
            return C + (int64_t)(row0 + 16 * i + rr) * ldc + col0 + 64 * h + lane;
        };
        auto in = [&](int i, int rr, int h) {
            return !MASKED || (row0 + 16 * i + rr < M && col0 + 64 * h + lane < N);
        };
        auto ld1 = [&](const CT* a) -> float {
            if constexpr (OUT16) return h2f(*a);
            else return __builtin_nontemporal_load(a);
        };
        auto st1 = [&](CT* a, float v) {
            if constexpr (OUT16) *a = f32_to_f16_bits(v);
            else __builtin_nontemporal_store(v, a);
        };
        // a band's staged values are all read back before its first store,
        // and its C values (beta != 0) all loaded, so each kind of access is
        // waited for once per band
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            stage_band(i);
            float v[16][H], c[16][H];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr)
#pragma unroll
                for (int h = 0; h < H; ++h) v[rr][h] = st[rr * R::RS + 64 * h + lane];
            if (beta != 0.f) {
#pragma unroll
                for (int rr = 0; rr < 16; ++rr)
#pragma unroll
                    for (int h = 0; h < H; ++h) c[rr][h] = in(i, rr, h) ? ld1(at(i, rr, h)) : 0.f;
#pragma unroll
                for (int rr = 0; rr < 16; ++rr)
#pragma unroll
                    for (int h = 0; h < H; ++h)
                        if (in(i, rr, h)) st1(at(i, rr, h), __builtin_fmaf(alpha, v[rr][h], beta * c[rr][h]));
            } else {
#pragma unroll
                for (int rr = 0; rr < 16; ++rr)
#pragma unroll
                    for (int h = 0; h < H; ++h)
                        if (in(i, rr, h)) st1(at(i, rr, h), alpha * v[rr][h]);
            }
        }
        return;
    }
    if (beta == 0.f) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            stage_band(i);
#pragma unroll
            for (int it = 0; it < IT; ++it) store4(i, it, alpha * staged(it));
        }
        return;
    }
    // the C loads of band i + 1 are issued before band i is written
    f32x4 old[2][IT];
    auto load_band = [&](int i, f32x4(&d)[IT]) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < IT; ++it) d[it] = load4(i, it);
    };
    load_band(0, old[0]);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        if (i + 1 < FM) load_band(i + 1, old[(i + 1) & 1]);
        stage_band(i);
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const f32x4 v = staged(it);
            f32x4 out;
#pragma unroll
            for (int x = 0; x < 4; ++x) out[x] = __builtin_fmaf(alpha, v[x], beta * old[i & 1][it][x]);
            store4(i, it, out);
        }
    }
}

// SK: a data-parallel + stream-K launch (p.sk_q > 0): the workgroups first
// take p.sk_dp whole rounds of tiles, then the (tile, panel) units of the
// remaining tiles, tile-major, in runs of sk_q (workgroups of one XCD get
// consecutive runs); a workgroup walks its run tile by tile, and a tile split
// over several workgroups is finished by the last of them to arrive, which
// adds the parts the others stored in P in k order.
// Four waves on a tile under 256 x 256 (wave tiles of 64 x 64) are held to
// two waves per SIMD, so two workgroups share a CU (their rings fit its
// shared memory): left alone the compiler spends accumulator registers and
// one workgroup runs per CU (2048^3 f16r 0.0582 -> 0.0550 ms measured).
template <int BM, int BN, int NS, int WM, int WN, int GM, bool MASKED, bool OUT16, bool SK>
__global__ __launch_bounds__(WM * WN * 64, (WM * WN == 4 && BM * BN < 256 * 256) ? 2 : 1)
void gemm_f16_ring_kernel(F16Args p) {
    using S = RingShape<BM, BN, NS, WM, WN>;
    static_assert(S::NW * StagedRows<S::TN>::BYTES <= NS * S::STAGE, "staged epilogue fits the ring");
    constexpr int D = S::BK;
    constexpr int GFM = S::GFM, GFN = S::GFN, H = S::H;
    constexpr int U = 2 * NS;   // panels per unrolled step: every stage, both B buffers
    __shared__ __attribute__((aligned(1024))) unsigned char ring[NS * S::STAGE];
    unsigned char* const st0 = ring;
    unsigned char* const st1 = ring + S::STAGE;
    unsigned char* const st2 = ring + 2 * S::STAGE;
    unsigned char* const st3 = ring + (NS > 3 ? 3 : 0) * S::STAGE;
    unsigned char* const st4 = ring + (NS > 4 ? 4 : 0) * S::STAGE;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave / WN, wc = wave % WN;
    const int nkt = static_cast<int>(p.nkb);   // panels of a whole tile
    const int dp_tiles = SK ? p.sk_dp * gridDim.x : 0;
    int g = 0, u = 0, u_end = 0, r = 0;
    if constexpr (SK) {
        const int G = gridDim.x, xcd = blockIdx.x & 7, q8 = G >> 3, r8 = G & 7;
        g = xcd * q8 + (xcd < r8 ? xcd : r8) + (blockIdx.x >> 3);
        u = g * p.sk_q;
        u_end = min((p.tiles_m * p.tiles_n - dp_tiles) * nkt, u + p.sk_q);
    }

    for (;;) {
        int tm, tn, kp0, nk;
        bool dp_item = false;
        if constexpr (!SK) {
            tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, GM, tm, tn);
            kp0 = 0;
            nk = nkt;
        } else if (r < p.sk_dp) {
            tile_of_block(r * gridDim.x + blockIdx.x, dp_tiles, p.tiles_m, p.tiles_n, GM, tm, tn);
            kp0 = 0;
            nk = nkt;
            dp_item = true;
        } else {
            if (u >= u_end) break;
            const int t = u / nkt;
            kp0 = u - t * nkt;
            nk = min(nkt - kp0, u_end - u);
            raster_tile(dp_tiles + t, p.tiles_m, p.tiles_n, GM, tm, tn);
        }
        const int m0 = tm * BM, n0 = tn * BN;

        // Panel kt of this tile's A rows is the BM-row slice at row m0 % 256 of
        // packed block (m0 / 256, kt); consecutive kt are consecutive blocks.
        constexpr int64_t kBlockBytes = int64_t{kPackRows} * D * 2;
        const int lane_ofs = wave * 1024 + lane * 16;
        const unsigned char* a_src = reinterpret_cast<const unsigned char*>(
            p.A16 + ((int64_t)(m0 / kPackRows) * p.nkb * kPackRows + m0 % kPackRows) * D) + lane_ofs +
            kp0 * kBlockBytes;
        const unsigned char* b_src = reinterpret_cast<const unsigned char*>(
            p.B16t + ((int64_t)(n0 / kPackRows) * p.nkb * kPackRows + n0 % kPackRows) * D) + lane_ofs +
            kp0 * kBlockBytes;

        auto stage_of = [&](int i) __attribute__((always_inline)) -> unsigned char* {
            return i == 0 ? st0 : i == 1 ? st1 : i == 2 ? st2 : i == 3 ? st3 : st4;
        };
        auto fill = [&](unsigned char* stage, int kt) __attribute__((always_inline)) {
            const uint32_t as = __builtin_amdgcn_readfirstlane(lds_addr(stage) + wave * 1024);
            const uint32_t bs = as + S::A_BYTES;
            const int64_t kofs = (int64_t)kt * kBlockBytes;
    #pragma unroll
            for (int j = 0; j < S::A_INS; ++j)
                lds_copy16(a_src + kofs + j * S::NW * 1024, as + j * S::NW * 1024);
    #pragma unroll
            for (int j = 0; j < S::B_INS; ++j)
                lds_copy16(b_src + kofs + j * S::NW * 1024, bs + j * S::NW * 1024);
        };

        // Fragment reads: lane (q, r16) reads row r16 of a 16-row block at logical
        // chunk q, the 8 k values [8q, 8q + 8) of the panel, to A and B alike.
        // Blocks start at multiples of 16 rows, whole swizzle periods, so the key
        // is swz(r16).
        const int r16 = lane & 15, q = lane >> 4;
        const int chunk = (q ^ swz<D>(r16)) << 4;
        const int a_row0 = (wr * S::TM + r16) * S::ROW + chunk;
        const int b_row0 = S::A_BYTES + (wc * S::TN + r16) * S::ROW + chunk;
        f16x8 fa[GFM], fb[2][GFN];
        auto read_a = [&](const unsigned char* stage, int i) __attribute__((always_inline)) {
            fa[i] = *reinterpret_cast<lds_f16x8*>((const lds_u8*)(stage) + a_row0 + i * 16 * S::ROW);
        };
        auto read_b = [&](const unsigned char* stage, int b, int j) __attribute__((always_inline)) {
            fb[b][j] = *reinterpret_cast<lds_f16x8*>((const lds_u8*)(stage) + b_row0 + j * 16 * S::ROW);
        };

        // The accumulators get their first value from the first matrix
        // instruction, with an inline-constant zero as its addend.
        f32x4 acc[GFM][GFN];
        auto mfma_rows = [&](int i0, int i1, int b, auto first) __attribute__((always_inline)) {
            const f32x4 zero = {};
    #pragma unroll
            for (int i = i0; i < i1; ++i)
    #pragma unroll
                for (int j = 0; j < GFN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        fa[i], fb[b][j], decltype(first)::value ? zero : acc[i][j], 0, 0, 0);
        };
        // one matrix instruction, then one fragment read, while reads remain
        auto interleave = [&](auto nmf_c, auto nrd_c) __attribute__((always_inline)) {
            constexpr int nmf = decltype(nmf_c)::value, nrd = decltype(nrd_c)::value;
    #pragma unroll
            for (int m = 0; m < nmf; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (m < nrd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        };

        // One panel in stage `cur`, its B fragments in fb[b]: fill panel kt_fill
        // into `freed` (the stage of the previous panel, which every wave finished
        // reading before the last barrier), then the two halves described above.
        // Fills past the last panel reload the last panel into a stage nobody
        // reads again, so the count of outstanding fills is the same every panel.
        auto panel = [&](const unsigned char* cur, unsigned char* freed, const unsigned char* next,
                         int kt_fill, auto b_c, auto first) __attribute__((always_inline)) {
            constexpr int b = decltype(b_c)::value;
            fill(freed, kt_fill);
    #pragma unroll
            for (int i = H; i < GFM; ++i) read_a(cur, i);
            mfma_rows(0, H, b, first);
            __builtin_amdgcn_sched_group_barrier(0x020, S::FILLS, 0);
            interleave(std::integral_constant<int, H * GFN>{}, std::integral_constant<int, GFM - H>{});
            // The first half's matrix instructions stay ahead of the wait and
            // the barrier: they touch no memory, so without this fence the
            // scheduler moves most of them past the barrier, and every panel
            // then waits for its last fragment reads and for the other waves
            // with almost no matrix work queued.
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt<(NS - 2) * S::FILLS>();
            ring_barrier();
    #pragma unroll
            for (int j = 0; j < GFN; ++j) read_b(next, b ^ 1, j);
    #pragma unroll
            for (int i = 0; i < H; ++i) read_a(next, i);
            mfma_rows(H, GFM, b, first);
            interleave(std::integral_constant<int, (GFM - H) * GFN>{},
                       std::integral_constant<int, GFN + H>{});
        };
        // Panel kt + u of an unrolled step: stage (kt + u) % NS with kt a multiple
        // of U, and the B buffer alternates with the panel's parity.
        auto step = [&](int kt, auto u_c, auto first) __attribute__((always_inline)) {
            constexpr int u = decltype(u_c)::value;
            panel(stage_of(u % NS), stage_of((u + NS - 1) % NS), stage_of((u + 1) % NS),
                  min(kt + u + NS - 1, nk - 1), std::integral_constant<int, u & 1>{}, first);
        };

        // Prologue: panels 0 .. NS-2 into stages 0 .. NS-2; wait for panel 0 and
        // read its first fragments.
    #pragma unroll
        for (int i = 0; i + 1 < NS; ++i) fill(stage_of(i), min(i, nk - 1));
        wait_vmcnt<(NS - 2) * S::FILLS>();
        ring_barrier();
    #pragma unroll
        for (int j = 0; j < GFN; ++j) read_b(stage_of(0), 0, j);
    #pragma unroll
        for (int i = 0; i < H; ++i) read_a(stage_of(0), i);

        step(0, std::integral_constant<int, 0>{}, std::true_type{});
        static_for<U - 1>([&](auto v_c) __attribute__((always_inline)) {
            constexpr int u = decltype(v_c)::value + 1;
            if (u < nk) step(0, std::integral_constant<int, u>{}, std::false_type{});
        });
        for (int kt = U; kt < nk; kt += U) {
            static_for<U>([&](auto u_c) __attribute__((always_inline)) {
                if (decltype(u_c)::value == 0 || kt + decltype(u_c)::value < nk)
                    step(kt, u_c, std::false_type{});
            });
        }
        wait_vmcnt<0>();   // no fill may still be landing in LDS when the tile's work ends

        bool finish = true;
        if (SK && nk < nkt) {
            // A part of the tile: store the accumulators in register order (one
            // 16-byte device-scope store per block and lane) in this workgroup's
            // slot for the tile (0: the tile its run starts in, 1: the one it ends
            // in), wait for them, pass a barrier and count in; the last workgroup
            // of the tile reads every part back in k order (part s comes from
            // workgroup g_first + s) and applies the epilogue.
            constexpr int kSC1 = 1 << 4;          // cache-policy bit of the buffer intrinsics
            constexpr int kRsrc = 0x00020000;     // raw buffer, 32-bit data format
            constexpr int NB = GFM * GFN;
            constexpr int TILE_BYTES = BM * BN * 4;
            const int t = u / nkt;
            const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
                p.P, (short)0, static_cast<int>((int64_t)gridDim.x * 2 * TILE_BYTES), kRsrc);
            auto at = [&](int wg, int b) {
                const int slot = (wg * p.sk_q) / nkt == t ? 0 : 1;
                return static_cast<int>(((int64_t)wg * 2 + slot) * TILE_BYTES +
                                        ((wave * NB + b) * 64 + lane) * 16);
            };
    #pragma unroll
            for (int b = 0; b < NB; ++b)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[b / GFN][b % GFN]),
                                                       rp, at(g, b), 0, kSC1);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();   // every wave is past its last fragment read and its stores are done
            const int g_first = (t * nkt) / p.sk_q;
            const int parts = (t * nkt + nkt - 1) / p.sk_q - g_first + 1;
            unsigned* count = p.counts + t;
            int* flag = reinterpret_cast<int*>(ring);
            if (threadIdx.x == 0)
                *flag = __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                        static_cast<unsigned>(parts - 1);
            __syncthreads();
            finish = *flag != 0;
            if (finish) {
                if (threadIdx.x == 0) __hip_atomic_store(count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                // four blocks at a time, the loads of up to four parts in
                // flight together, added in k order
                constexpr int CB = 4, ZG = 4;
                static_assert(NB % CB == 0, "blocks in chunks of four");
#pragma unroll
                for (int b0 = 0; b0 < NB; b0 += CB) {
                    for (int s0 = 0; s0 < parts; s0 += ZG) {
                        f32x4 tv[ZG][CB];
#pragma unroll
                        for (int ss = 0; ss < ZG; ++ss) {
                            const int wg = g_first + min(s0 + ss, parts - 1);   // past the last: unused reload
#pragma unroll
                            for (int c = 0; c < CB; ++c)
                                tv[ss][c] = __builtin_bit_cast(
                                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, at(wg, b0 + c), 0, kSC1));
                        }
#pragma unroll
                        for (int ss = 0; ss < ZG; ++ss) {
                            if (s0 + ss >= parts) break;
#pragma unroll
                            for (int c = 0; c < CB; ++c) {
                                const int b = b0 + c;
                                const f32x4 a = acc[b / GFN][b % GFN];
                                acc[b / GFN][b % GFN] = s0 + ss == 0 ? tv[ss][c] : a + tv[ss][c];
                            }
                        }
                    }
                }
            }
        }

    // vector rows of C: f32 16-byte aligned, binary16 8-byte aligned
        const uintptr_t c_addr = OUT16 ? reinterpret_cast<uintptr_t>(p.C16) : reinterpret_cast<uintptr_t>(p.C);
        const bool vec = p.ldc % 4 == 0 && (c_addr & (OUT16 ? 7 : 15)) == 0;
        if (!finish) {
            // another workgroup finishes this tile
        } else {
            // every wave is past its last fragment read once all have arrived here
            __syncthreads();
            unsigned char* mine = ring + wave * StagedRows<S::TN>::BYTES;
            if constexpr (OUT16)
                store_tile_m16_staged<GFM, GFN, S::TN, true, MASKED>(
                    acc, p.C16, p.ldc, m0 + wr * S::TM, n0 + wc * S::TN, p.M, p.N, p.alpha, p.beta,
                    lane, mine, vec);
            else
                store_tile_m16_staged<GFM, GFN, S::TN, false, MASKED>(
                    acc, p.C, p.ldc, m0 + wr * S::TM, n0 + wc * S::TN, p.M, p.N, p.alpha, p.beta,
                    lane, mine, vec);
        }
        if constexpr (!SK) break;
        if (dp_item) ++r;
        else u += nk;
        ring_barrier();   // every wave is done with the ring before the next tile refills it
    }
}

// Whether a half-depth ring configuration has a stream-K form: not for wave
// tiles of 128 x 128, whose 256 accumulator registers leave no room for the
// partial sums.  (The host's stream-K rule leaves them out too.)
constexpr bool ring_takes_sk(int bm, int bn, int wm, int wn) {
    return (bm / wm) * (bn / wn) < 128 * 128;
}

// One configuration, both masking variants, f32 (OUT16 false) or binary16 C.
template <int BM, int BN, int NS, int WM, int WN, int GM, bool OUT16>
hipError_t launch_f16_ring_out(const F16Args& a, hipStream_t s) {
    const dim3 block(WM * WN * 64);
    const bool masked = (a.M % BM) != 0 || (a.N % BN) != 0;
    if constexpr (!ring_takes_sk(BM, BN, WM, WN)) {
        if (a.sk_q > 0) return hipErrorInvalidValue;
    } else if (a.sk_q > 0) {
        const int grid = ring_sk_grid(int64_t{a.tiles_m} * a.tiles_n, a.nkb, a.sk_q, a.sk_dp,
                                      a.sk_grid, a.P, a.counts);
        if (grid <= 0) return hipErrorInvalidValue;
        // the stream-K form always guards its stores (whole tiles too): the
        // compiler keeps that variant's loop in registers better
        gemm_f16_ring_kernel<BM, BN, NS, WM, WN, GM, true, OUT16, true><<<dim3(grid), block, 0, s>>>(a);
        return hipGetLastError();
    }
    const dim3 grid(a.tiles_m * a.tiles_n);
    if (masked) gemm_f16_ring_kernel<BM, BN, NS, WM, WN, GM, true, OUT16, false><<<grid, block, 0, s>>>(a);
    else gemm_f16_ring_kernel<BM, BN, NS, WM, WN, GM, false, OUT16, false><<<grid, block, 0, s>>>(a);
    return hipGetLastError();
}

template <int BM, int BN, int ST, int WM, int WN, int GM, bool RS, bool OUT16>
hipError_t launch_f16_out(const F16Args& a, hipStream_t s) {
    const dim3 grid(a.tiles_m * a.tiles_n), block(WM * WN * 64);
    const bool masked = (a.M % BM) != 0 || (a.N % BN) != 0;
    if (masked) gemm_f16_kernel<BM, BN, ST, WM, WN, GM, RS, true, OUT16><<<grid, block, 0, s>>>(a);
    else gemm_f16_kernel<BM, BN, ST, WM, WN, GM, RS, false, OUT16><<<grid, block, 0, s>>>(a);
    return hipGetLastError();
}

// The binary16-output launches (defined in gemm_f16r_o16.hip).
template <int BM, int BN, int NS, int WM, int WN, int GM>
hipError_t launch_f16_ring_o16(const F16Args& a, hipStream_t s);
template <int BM, int BN, int ST, int WM, int WN, int GM, bool RS>
hipError_t launch_f16_o16(const F16Args& a, hipStream_t s);

// Compiled f16 configurations.  Half-depth rings: X(BM, BN, NS, WM, WN, GM),
// BK = 32, ST = NS stages.  Full-depth panels: Y(BM, BN, ST, WM, WN, GM),
// BK = 64; ST = 1 in a configuration names the register-staged two-stage
// ring (one stage in LDS is written from registers while the other is
// multiplied), ST = 2 or 3 the direct-to-LDS ring of that many stages.
#define G355_F16_RING_CONFIGS(X) \
    X(256, 256, 5, 4, 2, 8)      \
    X(256, 256, 5, 2, 4, 8)      \
    X(256, 256, 4, 4, 2, 8)      \
    X(256, 256, 4, 2, 4, 8)      \
    X(256, 256, 5, 2, 2, 8)      \
    X(128, 128, 5, 2, 2, 8)      \
    X(256, 128, 4, 4, 2, 8)      \
    X(128, 256, 4, 2, 4, 8)      \
    X(128, 128, 5, 4, 2, 8)
#define G355_F16_PANEL_CONFIGS(Y) \
    Y(256, 256, 1, 4, 2, 8)       \
    Y(256, 256, 1, 2, 4, 8)       \
    Y(128, 128, 1, 2, 2, 8)       \
    Y(256, 256, 2, 4, 2, 8)       \
    Y(256, 256, 2, 2, 4, 8)       \
    Y(256, 128, 3, 2, 2, 8)       \
    Y(256, 128, 2, 2, 2, 8)       \
    Y(256, 128, 3, 4, 2, 8)       \
    Y(128, 256, 3, 2, 2, 8)       \
    Y(128, 128, 2, 2, 2, 8)       \
    Y(128, 128, 3, 2, 2, 8)       \
    Y(128, 64, 2, 2, 2, 8)        \
    Y(64, 64, 2, 2, 2, 8)

}  // namespace g355
