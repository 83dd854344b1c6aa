// f32_kernel.hpp -- the f32 GEMM kernel template of libgemm355, shared by the
// translation unit of the plain layout (gemm_f32.hip) and that of the
// transposed operand layouts (gemm_f32_t.hip).  Not part of the public ABI.
//
// The structure follows the phobos docs page "gemm, f32": one output tile per
// workgroup (section "One output tile per CTA"), a K loop over BK-deep panels
// of A and B staged in shared memory by all threads and double-buffered so the
// copy of the next pair overlaps the math on the current one (sections "The k
// loop" and "The attributes", @pipeline), and the alpha/beta epilogue over the
// same tile (section "The epilogue").  On gfx950 the tile is split over 64-lane
// wavefronts, each owning a grid of 32x32 accumulator blocks.
//
// Masked variant (the default of the page's kernel without @aligned, and the
// zero-fill rule of the Matrix Multiplication lab's shared-memory kernels):
// out-of-range elements of A and B are loaded as zeros and stores outside
// M x N are skipped.
//
// Operand layouts (the lab's Part 5 layout study; BLAS transa/transb): with TA
// the kernel reads op(A) = A^T from a K x M row-major array, with TB op(B) =
// B^T from an N x K row-major array.  A panel is always copied with 16-byte
// loads along the operand's contiguous dimension and stored in shared memory
// in that same orientation: k-contiguous panels are read by the matrix
// instructions four k at a time (16-byte reads), the others one k at a time.
#pragma once

#include <type_traits>

#include "internal.hpp"

namespace g355 {

// Compiled f32 tile configurations: X(BM, BN, BK, WM, WN, GM).
#define G355_F32_CONFIGS(X)   \
    X(256, 256, 16, 2, 2, 8)  \
    X(256, 128, 16, 2, 2, 8)  \
    X(128, 256, 16, 2, 2, 8)  \
    X(128, 128, 16, 2, 2, 8)  \
    X(128, 128, 32, 2, 2, 8)  \
    X(128, 64, 16, 2, 2, 8)   \
    X(64, 64, 16, 2, 2, 8)    \
    X(64, 64, 32, 2, 2, 8)

// The direct-to-LDS ring (f32_ring.hpp): X(BM, BN, NS, WM, WN, GM), BK = 16,
// NS stages, every operand layout (split-K slices and leading dimensions past
// its copies' offsets run the register-staged kernel with these tiles).
#define G355_F32_RING_CONFIGS(X) \
    X(256, 256, 3, 2, 4, 8)      \
    X(256, 256, 4, 2, 4, 8)      \
    X(256, 256, 4, 4, 2, 8)      \
    X(128, 256, 4, 2, 4, 8)      \
    X(128, 256, 6, 2, 4, 8)

template <int BM, int BN, int BK, int WM, int WN, bool TA, bool TB>
struct F32Shape {
    static constexpr int NT = WM * WN * 64;
    static constexpr int TM = BM / WM;   // rows of C per wave
    static constexpr int TN = BN / WN;   // cols of C per wave
    static constexpr int FM = TM / 32;   // 32x32 accumulator blocks per wave (rows)
    static constexpr int FN = TN / 32;   // (cols)
    static constexpr int KH = BK / 2;    // k values per lane half per panel
    // A panel in LDS: BM rows of BK floats (k contiguous), padded so that the
    // 16-byte reads of 8 consecutive rows hit distinct banks; with TA, BK rows
    // of BM floats (m contiguous), padded like the B panel.
    static constexpr int AS = TA ? BM + 4 : BK + 4;
    // B panel in LDS: BK rows of BN floats (n contiguous), padded so the two
    // lane halves of a 32-bit read land on different bank halves; with TB, BN
    // rows of BK floats (k contiguous), padded like the A panel.
    static constexpr int BS = TB ? BK + 4 : BN + 4;
    static constexpr int A_STAGE = (TA ? BK : BM) * AS;
    static constexpr int B_STAGE = (TB ? BN : BK) * BS;
    static constexpr int LDS_FLOATS = 2 * (A_STAGE + B_STAGE);
    static constexpr int A_LD = BM * BK / 4 / NT;  // float4 loads per thread per panel
    static constexpr int B_LD = BK * BN / 4 / NT;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(BK % 8 == 0, "BK must be a multiple of 8");
    static_assert((BM * BK / 4) % NT == 0 && (BK * BN / 4) % NT == 0, "panel split");
    static_assert(LDS_FLOATS * 4 <= 160 * 1024, "LDS budget of one CU");
};

// Load one float4 of a row-major matrix X at (r, c) .. (r, c+3); the masked
// form reads only inside rows x cols and fills the rest with zeros.  Without
// VEC (a leading dimension that is not a multiple of 4) a row may start at
// any 4-byte boundary; a 16-byte global load only needs 4-byte alignment on
// this GPU, so the copy through memcpy still compiles to one load.
template <bool MASKED, bool VEC>
__device__ __forceinline__ float4 load4(const float* __restrict__ X, int64_t ld, int r, int c,
                                        int rows, int cols) {
    if (!MASKED) {
        return *reinterpret_cast<const float4*>(X + (int64_t)r * ld + c);
    } else {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (r < rows) {
            const float* p = X + (int64_t)r * ld + c;
            if (c + 3 < cols) {
                if (VEC) v = *reinterpret_cast<const float4*>(p);
                else __builtin_memcpy(&v, p, sizeof v);
            } else {
                if (c + 0 < cols) v.x = p[0];
                if (c + 1 < cols) v.y = p[1];
                if (c + 2 < cols) v.z = p[2];
                if (c + 3 < cols) v.w = p[3];
            }
        }
        return v;
    }
}

// SPLIT: this workgroup covers the K slice blockIdx.y (see F32Args) and
// stores its raw partial tile.  R16: operands are rounded to binary16 (round
// to nearest even) as they are staged; the f32 matrix instruction then
// multiplies binary16 values exactly and accumulates in f32, which is the
// f16r mode's arithmetic.
template <int BM, int BN, int BK, int WM, int WN, int GM, bool MASKED, bool VEC, bool TA, bool TB,
          bool SPLIT = false, bool R16 = false>
__global__ __launch_bounds__(WM * WN * 64) void gemm_f32_kernel(F32Args p) {
    using S = F32Shape<BM, BN, BK, WM, WN, TA, TB>;
    __shared__ __attribute__((aligned(16))) float smem[S::LDS_FLOATS];
    float* const As = smem;                     // [2][A_STAGE]
    float* const Bs = smem + 2 * S::A_STAGE;    // [2][B_STAGE]

    int tm, tn;
    tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, GM, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wr = wave / WN, wc = wave % WN;
    const int h = lane >> 5;    // lane half: which k sub-range this lane feeds
    const int r32 = lane & 31;  // row (A) / column (B) of the 32x32 block

    // The tile's corner of each stored array: A (M x K) or A^T (K x M);
    // B (K x N) or B^T (N x K).
    const float* __restrict__ A = TA ? p.A + m0 : p.A + (int64_t)m0 * p.lda;
    const float* __restrict__ B = TB ? p.B + (int64_t)n0 * p.ldb : p.B + n0;
    const int rows_a = p.M - m0;   // valid rows of op(A) in this tile (masked variant)
    const int cols_b = p.N - n0;   // valid columns of op(B)
    // the K range of this workgroup: everything, or one slice
    const int k_lo = SPLIT ? static_cast<int>(blockIdx.y) * p.ksplit : 0;
    const int k_hi = SPLIT ? min(p.K, k_lo + p.ksplit) : p.K;

    float4 ra[S::A_LD], rb[S::B_LD];

    // Element (r, c) of a panel's float4 grid: r runs over the stored rows of
    // the panel, c over its contiguous dimension in steps of 4.
    auto load_panels = [&](int k0) {
#pragma unroll
        for (int i = 0; i < S::A_LD; ++i) {
            const int idx = tid + i * S::NT;
            if (!TA) {   // BM rows (m) of BK contiguous k
                const int r = idx / (BK / 4), c = (idx % (BK / 4)) * 4;
                ra[i] = load4<MASKED, VEC>(A, p.lda, r, k0 + c, rows_a, k_hi);
            } else {     // BK rows (k) of BM contiguous m
                const int r = idx / (BM / 4), c = (idx % (BM / 4)) * 4;
                ra[i] = load4<MASKED, VEC>(A, p.lda, k0 + r, c, k_hi, rows_a);
            }
        }
#pragma unroll
        for (int i = 0; i < S::B_LD; ++i) {
            const int idx = tid + i * S::NT;
            if (!TB) {   // BK rows (k) of BN contiguous n
                const int r = idx / (BN / 4), c = (idx % (BN / 4)) * 4;
                rb[i] = load4<MASKED, VEC>(B, p.ldb, k0 + r, c, k_hi, cols_b);
            } else {     // BN rows (n) of BK contiguous k
                const int r = idx / (BK / 4), c = (idx % (BK / 4)) * 4;
                rb[i] = load4<MASKED, VEC>(B, p.ldb, r, k0 + c, cols_b, k_hi);
            }
        }
    };
    auto round16 = [](float4& v) {
        if (R16) {
            v.x = static_cast<float>(static_cast<_Float16>(v.x));
            v.y = static_cast<float>(static_cast<_Float16>(v.y));
            v.z = static_cast<float>(static_cast<_Float16>(v.z));
            v.w = static_cast<float>(static_cast<_Float16>(v.w));
        }
    };
    auto store_panels = [&](int stage) {
        float* as = As + stage * S::A_STAGE;
        float* bs = Bs + stage * S::B_STAGE;
#pragma unroll
        for (int i = 0; i < S::A_LD; ++i) round16(ra[i]);
#pragma unroll
        for (int i = 0; i < S::B_LD; ++i) round16(rb[i]);
#pragma unroll
        for (int i = 0; i < S::A_LD; ++i) {
            const int idx = tid + i * S::NT;
            constexpr int W = TA ? BM : BK;
            const int r = idx / (W / 4), c = (idx % (W / 4)) * 4;
            *reinterpret_cast<float4*>(as + r * S::AS + c) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < S::B_LD; ++i) {
            const int idx = tid + i * S::NT;
            constexpr int W = TB ? BK : BN;
            const int r = idx / (W / 4), c = (idx % (W / 4)) * 4;
            *reinterpret_cast<float4*>(bs + r * S::BS + c) = rb[i];
        }
    };

    f32x16 acc[S::FM][S::FN];
#pragma unroll
    for (int i = 0; i < S::FM; ++i)
#pragma unroll
        for (int j = 0; j < S::FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int nk = (k_hi - k_lo + BK - 1) / BK;
    load_panels(k_lo);
    store_panels(0);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) load_panels(k_lo + (kt + 1) * BK);

        // The panel pair in LDS: lane half h supplies k in [h*KH, (h+1)*KH) of
        // the panel, one k per instruction, to both operands alike, so every
        // instruction sums matching k of A and B.
        const float* as = As + cur * S::A_STAGE;
        const float* bs = Bs + cur * S::B_STAGE;
        float a[S::FM][S::KH];
        float b[S::FN][S::KH];
#pragma unroll
        for (int i = 0; i < S::FM; ++i) {
            const int row = wr * S::TM + i * 32 + r32;
            if (!TA) {
                const float* src = as + row * S::AS + h * S::KH;
#pragma unroll
                for (int q = 0; q < S::KH / 4; ++q) {
                    const float4 v = *reinterpret_cast<const float4*>(src + 4 * q);
                    a[i][4 * q + 0] = v.x;
                    a[i][4 * q + 1] = v.y;
                    a[i][4 * q + 2] = v.z;
                    a[i][4 * q + 3] = v.w;
                }
            } else {
                const float* src = as + (h * S::KH) * S::AS + row;
#pragma unroll
                for (int s = 0; s < S::KH; ++s) a[i][s] = src[s * S::AS];
            }
        }
#pragma unroll
        for (int j = 0; j < S::FN; ++j) {
            const int col = wc * S::TN + j * 32 + r32;
            if (!TB) {
                const float* src = bs + (h * S::KH) * S::BS + col;
#pragma unroll
                for (int s = 0; s < S::KH; ++s) b[j][s] = src[s * S::BS];
            } else {
                const float* src = bs + col * S::BS + h * S::KH;
#pragma unroll
                for (int q = 0; q < S::KH / 4; ++q) {
                    const float4 v = *reinterpret_cast<const float4*>(src + 4 * q);
                    b[j][4 * q + 0] = v.x;
                    b[j][4 * q + 1] = v.y;
                    b[j][4 * q + 2] = v.z;
                    b[j][4 * q + 3] = v.w;
                }
            }
        }
#pragma unroll
        for (int s = 0; s < S::KH; ++s)
#pragma unroll
            for (int i = 0; i < S::FM; ++i)
#pragma unroll
                for (int j = 0; j < S::FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][s], b[j][s], acc[i][j],
                                                                      0, 0, 0);

        if (more) store_panels(cur ^ 1);
        __syncthreads();
    }

    if (SPLIT) {
        // the raw partial tile of this slice (1 * acc is exact; beta = 0 reads nothing)
        float* P = p.C + static_cast<int64_t>(blockIdx.y) * p.M * p.ldc;
        store_tile<S::FM, S::FN, MASKED>(acc, P, p.ldc, m0 + wr * S::TM, n0 + wc * S::TN, p.M,
                                         p.N, 1.0f, 0.0f, lane);
        return;
    }
    // Epilogue: C = alpha*acc + beta*C over this wave's part of the tile.
    store_tile<S::FM, S::FN, MASKED>(acc, p.C, p.ldc, m0 + wr * S::TM, n0 + wc * S::TN, p.M, p.N,
                                     p.alpha, p.beta, lane);
}

// One layout of one configuration: the aligned variant when every dimension
// is a tile multiple and rows are 16-byte aligned, else the masked variant
// with 16-byte or (odd leading dimensions) 4-byte loads.
template <int BM, int BN, int BK, int WM, int WN, int GM, bool TA, bool TB>
hipError_t launch_f32_layout(const F32Args& a, F32Variant v, hipStream_t s) {
    const dim3 grid(a.tiles_m * a.tiles_n), block(WM * WN * 64);
    if (!v.masked)
        gemm_f32_kernel<BM, BN, BK, WM, WN, GM, false, true, TA, TB><<<grid, block, 0, s>>>(a);
    else if (v.vec)
        gemm_f32_kernel<BM, BN, BK, WM, WN, GM, true, true, TA, TB><<<grid, block, 0, s>>>(a);
    else
        gemm_f32_kernel<BM, BN, BK, WM, WN, GM, true, false, TA, TB><<<grid, block, 0, s>>>(a);
    return hipGetLastError();
}

// The transposed layouts (defined in gemm_f32_t.hip).
template <int BM, int BN, int BK, int WM, int WN, int GM>
hipError_t launch_f32_transposed(const F32Args& a, F32Variant v, hipStream_t s);

// The ring configurations (defined in gemm_f32_ring.hip).
template <int BM, int BN, int NS, int WM, int WN, int GM>
hipError_t launch_f32_ring(const F32Args& a, F32Variant v, hipStream_t s);

}  // namespace g355
