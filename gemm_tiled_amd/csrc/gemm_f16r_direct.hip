// gemm_f16r_direct.hip -- the f16r GEMM with the operands rounded to binary16
// as they are staged (KS=3 configurations): no packing pass, and K split over
// workgroups when the tiles alone would leave CUs idle.
//
// The computation is the one of the f16r mode (the lab's FP16 GEMM: A and B
// rounded to binary16 with round-to-nearest-even, products summed in f32,
// C = alpha*acc + beta*C in f32).  The packed path rounds both operands in a
// separate pass that reads and writes every element once more; for shapes
// with few rows of C that pass costs more than the product itself (B alone
// is read, rounded and written back, then read again).  Here each workgroup
// loads its f32 panels into registers, rounds them and writes the binary16
// panel image to shared memory, so B is read once, in f32, straight from its
// place in memory.
//
// Panels are 64 k deep.  In shared memory every row (of A, or column of B)
// holds its 64 values as eight 16-byte chunks, logical chunk c at position
// c ^ ((r / 2) % 8) -- the packed image of the packed path, read the same way
// (v_mfma_f32_16x16x32_f16: lane (q, r16) takes row r16 of a 16-row block at
// logical chunk 4s + q in step s of the panel).  Staging:
//   - an operand stored with k contiguous (A, or B stored N x K): a thread
//     loads 8 consecutive k of one row (two 16-byte loads), rounds them and
//     writes one 16-byte chunk;
//   - an operand stored with k as its row index (B, or A stored K x M): a
//     thread loads 4 consecutive columns of 8 consecutive k rows (eight
//     16-byte loads), rounds them and writes four 16-byte chunks, one per
//     column: the transpose happens in registers.
// Two stages: the loads of panel p + 1 are issued before the matrix work on
// panel p and written to the other stage after it, one barrier per panel.
//
// Split K: slice z = blockIdx.y covers k in [z*depth, min(K, (z+1)*depth)).
// With one slice the workgroup applies the epilogue itself.  With several,
// each stores its accumulators (in their register order, one 16-byte store per
// block and lane) to the partial buffer with device-scope (SC1) stores, waits
// for them, passes a barrier and counts itself in; the last workgroup of a
// tile to arrive reads all slices back in slice order, adds them and applies
// the epilogue, and resets the tile's counter.  The sum is the same, bit for
// bit, whichever workgroup arrives last.
#include "f16_kernel.hpp"

// X(BM, BN, WM, WN, GM): the compiled configurations.
#define G355_DIRECT_CONFIGS(X) \
    X(64, 64, 2, 2, 8)         \
    X(32, 64, 1, 4, 8)         \
    X(128, 128, 2, 2, 8)       \
    X(64, 256, 1, 4, 8)

namespace g355 {
namespace {

constexpr int kDBK = 64;      // k per panel
constexpr int kDRow = 128;    // bytes per panel row (64 binary16 values)

template <int BM, int BN, int WM, int WN>
struct DirectShape {
    static constexpr int NW = WM * WN, NT = NW * 64;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int GFM = TM / 16, GFN = TN / 16;   // 16 x 16 blocks per wave
    static constexpr int A_BYTES = BM * kDRow;
    static constexpr int STAGE = (BM + BN) * kDRow;
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile of whole 16 x 16 blocks");
    static_assert(BM % 4 == 0 && BN % 4 == 0, "column groups of four");
    static_assert(2 * STAGE <= 160 * 1024, "LDS budget of one CU");
};

__device__ __forceinline__ int dswz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ float comp(const float4& v, int j) {
    return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

__device__ __forceinline__ _Float16 rn(float x) { return static_cast<_Float16>(x); }

// 16 bytes of a row-major matrix X at (r, c) .. (r, c + 3).  MASKED: reads
// only inside rows x cols (zeros elsewhere) and needs only 4-byte alignment
// (a 16-byte global load needs no more on this GPU).
template <bool MASKED>
__device__ __forceinline__ float4 ld4(const float* __restrict__ X, int64_t ld, int r, int c,
                                      int rows, int cols) {
    if (!MASKED) return *reinterpret_cast<const float4*>(X + (int64_t)r * ld + c);
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < rows) {
        const float* p = X + (int64_t)r * ld + c;
        if (c + 3 < cols) {
            __builtin_memcpy(&v, p, sizeof v);
        } else {
            if (c + 0 < cols) v.x = p[0];
            if (c + 1 < cols) v.y = p[1];
            if (c + 2 < cols) v.z = p[2];
        }
    }
    return v;
}

typedef __attribute__((address_space(3))) f16x8 lds_f16x8_w;

// An operand stored with k contiguous: R rows x 64 k per panel, in units of
// one row's 8 consecutive k.
template <int R, int NT, bool MASKED>
struct KRows {
    static constexpr int UNITS = R * 8;
    static constexpr int U = (UNITS + NT - 1) / NT;
    float4 v[U][2];
    __device__ __forceinline__ void load(const float* __restrict__ X, int64_t ld, int x0, int xdim,
                                         int k0, int khi, int tid) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int w = tid + NT * u;
            if (UNITS % NT != 0 && w >= UNITS) continue;
            const int row = w >> 3, k = k0 + 8 * (w & 7);
            v[u][0] = ld4<MASKED>(X, ld, x0 + row, k, xdim, khi);
            v[u][1] = ld4<MASKED>(X, ld, x0 + row, k + 4, xdim, khi);
        }
    }
    __device__ __forceinline__ void store(lds_u8* base, int tid) const {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int w = tid + NT * u;
            if (UNITS % NT != 0 && w >= UNITS) continue;
            const int row = w >> 3, ch = w & 7;
            const f16x8 h = {rn(v[u][0].x), rn(v[u][0].y), rn(v[u][0].z), rn(v[u][0].w),
                             rn(v[u][1].x), rn(v[u][1].y), rn(v[u][1].z), rn(v[u][1].w)};
            *reinterpret_cast<lds_f16x8_w*>(base + row * kDRow + ((ch ^ dswz(row)) << 4)) = h;
        }
    }
};

// An operand stored with k as its row index (K x xdim): 64 k x R columns per
// panel, in units of 8 k rows x 4 columns, transposed in registers.  Unit w
// takes k group w % 8 of column group w / 8: the eight lanes of a column group
// write the eight chunks of its columns (128 contiguous bytes per column, so
// the writes of a wave spread over all banks), and each load instruction of a
// wave reads eight whole 128-byte lines.
template <int R, int NT, bool MASKED>
struct KCols {
    static constexpr int CG = R / 4;          // column groups
    static constexpr int UNITS = 8 * CG;
    static constexpr int U = (UNITS + NT - 1) / NT;
    float4 v[U][8];
    __device__ __forceinline__ void load(const float* __restrict__ X, int64_t ld, int x0, int xdim,
                                         int k0, int khi, int tid) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int w = tid + NT * u;
            if (UNITS % NT != 0 && w >= UNITS) continue;
            const int c = w >> 3, g = w & 7;
#pragma unroll
            for (int t = 0; t < 8; ++t)
                v[u][t] = ld4<MASKED>(X, ld, k0 + 8 * g + t, x0 + 4 * c, khi, xdim);
        }
    }
    __device__ __forceinline__ void store(lds_u8* base, int tid) const {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int w = tid + NT * u;
            if (UNITS % NT != 0 && w >= UNITS) continue;
            const int c = w >> 3, g = w & 7;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int x = 4 * c + j;
                const f16x8 h = {rn(comp(v[u][0], j)), rn(comp(v[u][1], j)), rn(comp(v[u][2], j)),
                                 rn(comp(v[u][3], j)), rn(comp(v[u][4], j)), rn(comp(v[u][5], j)),
                                 rn(comp(v[u][6], j)), rn(comp(v[u][7], j))};
                *reinterpret_cast<lds_f16x8_w*>(base + x * kDRow + ((g ^ dswz(x)) << 4)) = h;
            }
        }
    }
};

template <bool KCONTIG, int R, int NT, bool MASKED>
using Stager = std::conditional_t<KCONTIG, KRows<R, NT, MASKED>, KCols<R, NT, MASKED>>;

template <int BM, int BN, int WM, int WN, int GM, bool TA, bool TB, bool MASKED, bool OUT16>
__global__ __launch_bounds__(WM * WN * 64) void gemm_f16_direct_kernel(DirectArgs p) {
    using S = DirectShape<BM, BN, WM, WN>;
    constexpr int GFM = S::GFM, GFN = S::GFN;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * S::STAGE];

    int tm, tn;
    tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, GM, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int slice = blockIdx.y;
    const int k_lo = slice * p.depth;
    const int k_hi = min(p.K, k_lo + p.depth);
    const int np = (k_hi - k_lo + kDBK - 1) / kDBK;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave / WN, wc = wave % WN;

    // A is k-contiguous unless stored K x M; B is k-contiguous when stored N x K.
    Stager<!TA, BM, S::NT, MASKED> sa;
    Stager<TB, BN, S::NT, MASKED> sb;
    auto load = [&](int kp) __attribute__((always_inline)) {
        sa.load(p.A, p.lda, m0, p.M, kp, k_hi, tid);
        sb.load(p.B, p.ldb, n0, p.N, kp, k_hi, tid);
    };
    auto stage = [&](int i) __attribute__((always_inline)) -> lds_u8* {
        return (lds_u8*)(lds) + i * S::STAGE;
    };
    auto store = [&](lds_u8* st) __attribute__((always_inline)) {
        sa.store(st, tid);
        sb.store(st + S::A_BYTES, tid);
    };

    // Fragment reads: blocks start at multiples of 16 rows (whole swizzle
    // periods), so a lane's chunk position depends on r16 only.
    const int r16 = lane & 15, q = lane >> 4;
    const int a_row0 = (wr * S::TM + r16) * kDRow;
    const int b_row0 = S::A_BYTES + (wc * S::TN + r16) * kDRow;
    const int pos0 = ((q ^ dswz(r16)) << 4), pos1 = (((4 + q) ^ dswz(r16)) << 4);

    f32x4 acc[GFM][GFN];
#pragma unroll
    for (int i = 0; i < GFM; ++i)
#pragma unroll
        for (int j = 0; j < GFN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const lds_u8* st) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int pos = s == 0 ? pos0 : pos1;
            f16x8 fa[GFM], fb[GFN];
#pragma unroll
            for (int i = 0; i < GFM; ++i)
                fa[i] = *reinterpret_cast<const lds_f16x8*>(st + a_row0 + i * 16 * kDRow + pos);
#pragma unroll
            for (int j = 0; j < GFN; ++j)
                fb[j] = *reinterpret_cast<const lds_f16x8*>(st + b_row0 + j * 16 * kDRow + pos);
#pragma unroll
            for (int i = 0; i < GFM; ++i)
#pragma unroll
                for (int j = 0; j < GFN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
    };

    if (np > 0) {
        load(k_lo);
        store(stage(0));
        __syncthreads();
        for (int kp = 0; kp < np; ++kp) {
            const bool more = kp + 1 < np;
            if (more) load(k_lo + (kp + 1) * kDBK);
            compute(stage(kp & 1));
            if (more) store(stage((kp + 1) & 1));
            __syncthreads();
        }
    }

    const int row0 = m0 + wr * S::TM, col0 = n0 + wc * S::TN;
    if (p.slices > 1) {
        constexpr int kSC1 = 1 << 4;             // cache-policy bit of the buffer intrinsics
        constexpr int kRsrc = 0x00020000;        // raw buffer, 32-bit data format
        constexpr int TILE_BYTES = BM * BN * 4;
        const int tiles = gridDim.x;
        const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
            p.P, (short)0, static_cast<int>((int64_t)p.slices * tiles * TILE_BYTES), kRsrc);
        // this lane's 16 bytes of block b in slice z
        auto at = [&](int z, int b) {
            return static_cast<int>(((int64_t)z * tiles + blockIdx.x) * TILE_BYTES +
                                    ((wave * GFM * GFN + b) * 64 + lane) * 16);
        };
#pragma unroll
        for (int i = 0; i < GFM; ++i)
#pragma unroll
            for (int j = 0; j < GFN; ++j)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), rp,
                                                       at(slice, i * GFN + j), 0, kSC1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();   // every wave is past its last panel read, and its stores are done
        unsigned* count = p.counts + blockIdx.x;
        int* flag = reinterpret_cast<int*>(lds);
        if (tid == 0)
            *flag = __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                    static_cast<unsigned>(p.slices - 1);
        __syncthreads();
        if (!*flag) return;
        if (tid == 0) __hip_atomic_store(count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // Slices in groups of four: the loads of a group (every block) are
        // issued together, then added in slice order.
        constexpr int NB = GFM * GFN, ZG = 4;
        for (int z0 = 0; z0 < p.slices; z0 += ZG) {
            f32x4 t[ZG][NB];
#pragma unroll
            for (int zz = 0; zz < ZG; ++zz) {
                const int z = min(z0 + zz, p.slices - 1);   // past the last slice: a reload, unused
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    t[zz][b] = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, at(z, b), 0, kSC1));
            }
#pragma unroll
            for (int zz = 0; zz < ZG; ++zz) {
                if (z0 + zz >= p.slices) break;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    f32x4& a = acc[b / GFN][b % GFN];
                    a = z0 + zz == 0 ? t[zz][b] : a + t[zz][b];
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

template <int BM, int BN, int WM, int WN, int GM, bool TA, bool TB, bool OUT16>
hipError_t launch_layout(const DirectArgs& a, bool masked, hipStream_t s) {
    const dim3 grid(a.tiles_m * a.tiles_n, a.slices), block(WM * WN * 64);
    if (masked)
        gemm_f16_direct_kernel<BM, BN, WM, WN, GM, TA, TB, true, OUT16><<<grid, block, 0, s>>>(a);
    else
        gemm_f16_direct_kernel<BM, BN, WM, WN, GM, TA, TB, false, OUT16><<<grid, block, 0, s>>>(a);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int GM>
hipError_t launch_direct(const DirectArgs& a, bool ta, bool tb, bool masked, hipStream_t s) {
    const bool o16 = a.C16 != nullptr;
#define G355_DIRECT_CASE(TA, TB)                                                              \
    if (ta == TA && tb == TB)                                                                 \
        return o16 ? launch_layout<BM, BN, WM, WN, GM, TA, TB, true>(a, masked, s)           \
                   : launch_layout<BM, BN, WM, WN, GM, TA, TB, false>(a, masked, s);
    G355_DIRECT_CASE(false, false)
    G355_DIRECT_CASE(false, true)
    G355_DIRECT_CASE(true, false)
    G355_DIRECT_CASE(true, true)
#undef G355_DIRECT_CASE
    return hipErrorInvalidValue;
}

#define G355_DIRECT_INSTANCE(BM, BN, WM, WN, GM) \
    {{GEMM355_MODE_F16R, BM, BN, kDBK, 2, WM, WN, GM, 3}, &launch_direct<BM, BN, WM, WN, GM>},

const DirectInstance kDirectInstances[] = {G355_DIRECT_CONFIGS(G355_DIRECT_INSTANCE)};

}  // namespace

const DirectInstance* direct_instances(int* count) {
    *count = static_cast<int>(sizeof(kDirectInstances) / sizeof(kDirectInstances[0]));
    return kDirectInstances;
}

}  // namespace g355
