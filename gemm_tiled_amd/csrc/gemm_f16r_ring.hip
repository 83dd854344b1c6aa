// gemm_f16r_ring.hip -- f16r with the operands rounded to binary16 as the
// matrix instruction's fragments are read (KS=3 configurations with BK = 16):
// the f32 panels reach shared memory through direct global->LDS copies into a
// ring of NS stages, as in the f32 ring kernel, so many panels are in flight
// per workgroup without holding them in registers; each fragment is read in
// f32, rounded to binary16 (nearest even) in registers and multiplied on
// v_mfma_f32_16x16x16_f16 with f32 accumulation.  For few rows of C the call
// streams B once from memory and the matrix work is small, so what matters is
// keeping enough copies in flight to reach the memory roof; the packing pass
// of the packed path (read, round and write all of B, then read it again) and
// the one-panel-ahead register staging of the other KS=3 kernel both fall
// short of it there.
//
// Panel layout (BK = 16 floats of k), as in the f32 ring but keyed for the
// 16-lane fragment reads of this instruction:
//   A: BM rows of 64 bytes (four 16-byte chunks of 4 k); chunk c of row r sits
//      at position c ^ ((r / 2) % 4); a copy instruction fills 16 rows, lane l
//      fetching the global chunk that belongs at its position.
//   B: 16 k-rows of BN = 256 floats, 1024 + 16 bytes apart.
// Fragments: lane (q, r16) takes row r16 of a 16-row A block at chunk q (one
// 16-byte read) and column r16 of a 16-column B block at k-rows 4q .. 4q + 3
// (four 4-byte reads); the four lane quarters read k-rows 4 apart, which the
// 16-byte row padding puts in different banks.
//
// Shapes: the plain layout with 16-byte aligned rows, N % 4 == 0 and
// K % 16 == 0 (M and N need not be tile multiples: copies of rows past M read
// row M - 1 and of columns past N column n0, values that only reach outputs
// the masked epilogue never stores).  K is split over blockIdx.y as in the
// other KS=3 kernel, the last workgroup of a tile adding the slices' partial
// tiles in slice order.
#include "f16_kernel.hpp"

// X(BM, BN, NS, WM, WN, GM): the compiled configurations.
#define G355_F16_FROM_F32_RING_CONFIGS(X) \
    X(64, 256, 3, 1, 4, 8)                \
    X(64, 256, 6, 1, 4, 8)                \
    X(32, 256, 6, 1, 2, 8)                \
    X(128, 256, 4, 2, 4, 8)

namespace g355 {
namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const f32x4v lds_f32x4c;
typedef __attribute__((address_space(3))) const float lds_f32c;

template <int BM, int BN, int NS, int WM, int WN>
struct F16RingShape {
    static constexpr int BK = 16;
    static constexpr int NW = WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int GFM = TM / 16, GFN = TN / 16;
    static constexpr int A_BYTES = BM * BK * 4;
    static constexpr int B_ROW = BN * 4 + 16;
    static constexpr int STAGE = A_BYTES + BK * B_ROW;
    static constexpr int A_INS = BM / 16 / NW;
    static constexpr int B_INS = BK / NW;
    static constexpr int FILLS = A_INS + B_INS;
    static_assert(BN == 256, "one k-row of B is one 1 KB copy");
    static_assert(A_INS >= 1 && A_INS * 16 * NW == BM && B_INS >= 1 && B_INS * NW == BK,
                  "copies split evenly over the waves");
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile of whole 16 x 16 blocks");
    static_assert(NS >= 3 && NS * STAGE <= 160 * 1024, "LDS budget of one CU");
    static_assert((NS - 2) * FILLS < 64, "vmcnt range");
};

__device__ __forceinline__ f16x4 rn4(f32x4v v) {
    return f16x4{static_cast<_Float16>(v[0]), static_cast<_Float16>(v[1]),
                 static_cast<_Float16>(v[2]), static_cast<_Float16>(v[3])};
}

template <int BM, int BN, int NS, int WM, int WN, int GM, bool MASKED, bool OUT16>
__global__ __launch_bounds__(WM * WN * 64) void gemm_f16_f32ring_kernel(DirectArgs p) {
    using S = F16RingShape<BM, BN, NS, WM, WN>;
    constexpr int GFM = S::GFM, GFN = S::GFN;
    __shared__ __attribute__((aligned(1024))) unsigned char ring[NS * S::STAGE];

    int tm, tn;
    tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, GM, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int slice = blockIdx.y;
    const int k_lo = slice * p.depth;
    const int k_hi = min(p.K, k_lo + p.depth);
    const int nk = (k_hi - k_lo) / S::BK;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave / WN, wc = wave % WN;

    // Copy sources.  A copy j of this wave fills panel rows 16 (wave + NW j)
    // .. +15; lane l takes row l / 4 of them at position l % 4, which holds
    // global chunk (l % 4) ^ ((row / 2) % 4) = (l % 4) ^ ((l / 8) % 4).  B copy
    // j fills k-row wave + NW j, lane l its floats 4l .. 4l + 3.
    const int arow = lane >> 2;
    const int achunk = (lane & 3) ^ ((lane >> 3) & 3);
    const float* a_src[S::A_INS];
#pragma unroll
    for (int j = 0; j < S::A_INS; ++j) {
        const int row = min(m0 + (wave + S::NW * j) * 16 + arow, p.M - 1);
        a_src[j] = p.A + (int64_t)row * p.lda + k_lo + achunk * 4;
    }
    const int bcol = n0 + lane * 4 < p.N ? n0 + lane * 4 : n0;
    const float* b_src = p.B + (int64_t)(k_lo + wave) * p.ldb + bcol;
    const int64_t b_step = (int64_t)S::NW * p.ldb;
    const int64_t b_panel = (int64_t)S::BK * p.ldb;

    auto stage_of = [&](int i) __attribute__((always_inline)) -> unsigned char* {
        return ring + i * S::STAGE;
    };
    auto fill = [&](unsigned char* stage, int kt) __attribute__((always_inline)) {
        const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(stage));
#pragma unroll
        for (int j = 0; j < S::A_INS; ++j)
            lds_copy16(a_src[j] + kt * S::BK, base + (wave + S::NW * j) * 1024);
#pragma unroll
        for (int j = 0; j < S::B_INS; ++j)
            lds_copy16(b_src + j * b_step + kt * b_panel,
                       base + S::A_BYTES + (wave + S::NW * j) * S::B_ROW);
    };

    const int r16 = lane & 15, q = lane >> 4;
    const int a_off = (wr * S::TM + r16) * 64 + ((q ^ ((r16 >> 1) & 3)) << 4);
    const int b_off = S::A_BYTES + (4 * q) * S::B_ROW + (wc * S::TN + r16) * 4;

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
        f16x4 fa[GFM], fb[GFN];
#pragma unroll
        for (int i = 0; i < GFM; ++i)
            fa[i] = rn4(*reinterpret_cast<lds_f32x4c*>(st + a_off + i * 16 * 64));
#pragma unroll
        for (int j = 0; j < GFN; ++j) {
            f32x4v v;
#pragma unroll
            for (int t = 0; t < 4; ++t)
                v[t] = *reinterpret_cast<lds_f32c*>(st + b_off + t * S::B_ROW + j * 16 * 4);
            fb[j] = rn4(v);
        }
#pragma unroll
        for (int i = 0; i < GFM; ++i)
#pragma unroll
            for (int j = 0; j < GFN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x16f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    wait_vmcnt<0>();   // no copy may still be landing in LDS when the workgroup ends

    const int row0 = m0 + wr * S::TM, col0 = n0 + wc * S::TN;
    if (p.slices > 1) {
        constexpr int kSC1 = 1 << 4;             // cache-policy bit of the buffer intrinsics
        constexpr int kRsrc = 0x00020000;        // raw buffer, 32-bit data format
        constexpr int NB = GFM * GFN;
        constexpr int TILE_BYTES = BM * BN * 4;
        const int tiles = gridDim.x;
        const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
            p.P, (short)0, static_cast<int>((int64_t)p.slices * tiles * TILE_BYTES), kRsrc);
        auto at = [&](int z, int b) {
            return static_cast<int>(((int64_t)z * tiles + blockIdx.x) * TILE_BYTES +
                                    ((wave * NB + b) * 64 + lane) * 16);
        };
#pragma unroll
        for (int b = 0; b < NB; ++b)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[b / GFN][b % GFN]),
                                                   rp, at(slice, b), 0, kSC1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();   // every wave is past its last panel read and its stores are done
        unsigned* count = p.counts + blockIdx.x;
        int* flag = reinterpret_cast<int*>(ring);
        if (threadIdx.x == 0)
            *flag = __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                    static_cast<unsigned>(p.slices - 1);
        __syncthreads();
        if (!*flag) return;
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
    }
    if constexpr (OUT16)
        store_tile_m16<GFM, GFN, MASKED, true>(acc, p.C16, p.ldc, row0, col0, p.M, p.N, p.alpha,
                                               p.beta, lane);
    else
        store_tile_m16<GFM, GFN, MASKED, false>(acc, p.C, p.ldc, row0, col0, p.M, p.N, p.alpha,
                                                p.beta, lane);
}

template <int BM, int BN, int NS, int WM, int WN, int GM>
hipError_t launch_f32ring(const DirectArgs& a, bool ta, bool tb, bool masked, hipStream_t s) {
    // the host hands only the shapes this kernel takes (f16_from_f32_ring_takes)
    if (ta || tb || a.N % 4 != 0 || a.K % 16 != 0 || a.depth % 16 != 0 || a.K <= 0)
        return hipErrorInvalidValue;
    const dim3 grid(a.tiles_m * a.tiles_n, a.slices), block(WM * WN * 64);
    const bool edge = masked || a.M % BM != 0 || a.N % BN != 0;
    if (a.C16) {
        if (edge) gemm_f16_f32ring_kernel<BM, BN, NS, WM, WN, GM, true, true><<<grid, block, 0, s>>>(a);
        else gemm_f16_f32ring_kernel<BM, BN, NS, WM, WN, GM, false, true><<<grid, block, 0, s>>>(a);
    } else {
        if (edge) gemm_f16_f32ring_kernel<BM, BN, NS, WM, WN, GM, true, false><<<grid, block, 0, s>>>(a);
        else gemm_f16_f32ring_kernel<BM, BN, NS, WM, WN, GM, false, false><<<grid, block, 0, s>>>(a);
    }
    return hipGetLastError();
}

#define G355_F32RING_INSTANCE(BM, BN, NS, WM, WN, GM) \
    {{GEMM355_MODE_F16R, BM, BN, 16, NS, WM, WN, GM, 3}, &launch_f32ring<BM, BN, NS, WM, WN, GM>},

const DirectInstance kF32RingInstances[] = {G355_F16_FROM_F32_RING_CONFIGS(G355_F32RING_INSTANCE)};

}  // namespace

const DirectInstance* f16_from_f32_ring_instances(int* count) {
    *count = static_cast<int>(sizeof(kF32RingInstances) / sizeof(kF32RingInstances[0]));
    return kF32RingInstances;
}

bool f16_from_f32_ring_takes(bool ta, bool tb, const float* A, int64_t lda, const float* B,
                             int64_t ldb, int64_t N, int64_t K) {
    auto vec = [](const float* p, int64_t ld) {
        return ld % 4 == 0 && (reinterpret_cast<uintptr_t>(p) & 15) == 0;
    };
    return !ta && !tb && vec(A, lda) && vec(B, ldb) && N % 4 == 0 && K % 16 == 0 && K > 0;
}

}  // namespace g355
