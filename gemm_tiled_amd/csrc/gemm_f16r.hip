// gemm_f16r.hip -- the f16r mode: A and B rounded to binary16 (round to
// nearest even), products accumulated in f32 on the gfx950 matrix cores
// (v_mfma_f32_32x32x16_f16), then C = alpha*acc + beta*C in f32.
//
// The phobos docs page "gemm on tensor cores" (section "What changes") keeps
// the f32 kernel line for line and only moves dot onto the matrix units with
// operands rounded to f16.  Here the rounding is a pass of its own that also
// packs each operand panel-major: A, and B transposed (so both are k
// contiguous), are cut into blocks of 256 rows x 64 k, and each block is
// stored as one contiguous 32 KB run that is already the shared-memory image
// the GEMM kernel multiplies from.  Filling a panel is then a straight copy of
// contiguous kilobytes (one stream per panel instead of 256 rows scattered
// one row pitch apart), and the zero padding of partial blocks is the masked
// edge rule of the Matrix Multiplication lab's tiled kernels (out-of-range
// operands load as 0), so the GEMM loads carry no masks; only its epilogue is
// masked.
#include "f16_kernel.hpp"

namespace g355 {
namespace {

// Two f32 -> two binary16, round to nearest even (a C++ conversion to
// _Float16 is correctly rounded in the default rounding mode), packed.
__device__ __forceinline__ uint32_t pack_rn(float lo, float hi) {
    const f16x2 v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

// One operand of the packing pass: the packed image `dst` (rows x Kp, in
// blocks of 256 rows x D) is filled from the f32 array `src` with leading
// dimension `ld`, holding the operand either with k contiguous (`direct`: row
// x of the image is row x of src, as A is stored, or B^T) or with the rows of
// the image contiguous (transposing: row x of the image is column x of src,
// as B is stored, or A^T).
struct PackOperand {
    const float* src;
    int64_t ld;
    uint16_t* dst;
    int64_t rows_p;   // padded rows of the image (multiple of 256)
    int rows;         // logical rows (M for A, N for B)
    int blocks;       // workgroups of this operand
};

// Both operands are packed by one launch: the first a.blocks workgroups pack
// A, the rest B, so the two streams share the memory system and the tail of
// one overlaps the start of the other.
struct PackArgs {
    PackOperand a, b;
    int64_t nkb;   // depth blocks of D
    int K;
};

constexpr int kUnitsPerThread = 8;
constexpr int kUnitsPerBlock = 256 * kUnitsPerThread;
constexpr int kTB = 64;        // transpose block edge
constexpr int kTS = kTB + 2;   // LDS row stride in halves

// Direct packing.  One unit converts 8 consecutive k of one row into one
// 16-byte chunk of the packed image, and units are numbered in the order of
// the packed image, so consecutive threads write consecutive bytes (whole
// 128-byte lines) and the D/8 threads of one packed row read D consecutive
// floats of one source row.
template <int D, bool VEC>
__device__ __forceinline__ void pack_unit(const PackOperand& o, int64_t nkb, int K, int64_t u) {
    constexpr int cpr = D / 8;
    const int64_t q = u / cpr;                       // packed row: (block, row in block)
    const int pc = static_cast<int>(u - q * cpr);    // physical chunk
    const int64_t blk = q / kPackRows;
    const int rin = static_cast<int>(q - blk * kPackRows);
    const int64_t xb = blk / nkb;
    const int kb = static_cast<int>(blk - xb * nkb);
    const int64_t r = xb * kPackRows + rin;
    const int k = kb * D + ((pc ^ swz<D>(rin)) << 3);
    const float* X = o.src;
    float v[8];
    if (r < o.rows && VEC && k + 7 < K) {
        // the f32 source is read once: non-temporal, so it does not evict the
        // packed operands from the caches
        const f32x4* src = reinterpret_cast<const f32x4*>(X + r * o.ld + k);
        const f32x4 x = __builtin_nontemporal_load(src), y = __builtin_nontemporal_load(src + 1);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
        v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
    } else if (r < o.rows && k + 7 < K) {
        // a row that starts on any 4-byte boundary: 16-byte global loads
        // need only 4-byte alignment here
        __builtin_memcpy(v, X + r * o.ld + k, sizeof v);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (r < o.rows && k + e < K) ? X[r * o.ld + k + e] : 0.f;
    }
    uint4 w;
    w.x = pack_rn(v[0], v[1]);
    w.y = pack_rn(v[2], v[3]);
    w.z = pack_rn(v[4], v[5]);
    w.w = pack_rn(v[6], v[7]);
    *reinterpret_cast<uint4*>(o.dst + u * 8) = w;
}

template <int D, bool VEC>
__device__ __forceinline__ void pack_direct(const PackOperand& o, int64_t nkb, int K, int b) {
    const int64_t units = o.rows_p * nkb * (D / 8);
    const int64_t u0 = (int64_t)b * kUnitsPerBlock + threadIdx.x;
#pragma unroll
    for (int i = 0; i < kUnitsPerThread; ++i) {
        const int64_t u = u0 + i * 256;
        if (u < units) pack_unit<D, VEC>(o, nkb, K, u);
    }
}

// Transposing packing.  A 64 (k) x 64 (image rows) block of the source is read
// along its contiguous dimension (coalesced), rounded, transposed through LDS
// and written as 64 packed rows of the 64 / D depth blocks it covers.
template <int D, bool VEC>
__device__ __forceinline__ void pack_transpose(const PackOperand& o, int64_t nkb, int K, int b,
                                               uint16_t* t) {
    const int cols = static_cast<int>(o.rows_p / kTB);
    const int x0 = (b % cols) * kTB;
    const int kt = b / cols;
    const int k0 = kt * kTB;
    const int tid = threadIdx.x;
    const float* X = o.src;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + i * 256;
        const int kr = idx >> 4, xq = (idx & 15) * 4;
        const int k = k0 + kr, x = x0 + xq;
        float v[4];
        if (k < K && VEC && x + 3 < o.rows) {
            const f32x4 q =
                __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(X + (int64_t)k * o.ld + x));
            v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
        } else if (k < K && x + 3 < o.rows) {
            __builtin_memcpy(v, X + (int64_t)k * o.ld + x, sizeof v);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = (k < K && x + e < o.rows) ? X[(int64_t)k * o.ld + x + e] : 0.f;
        }
        const uint32_t p01 = pack_rn(v[0], v[1]);
        const uint32_t p23 = pack_rn(v[2], v[3]);
        uint16_t* row = t + kr * kTS + xq;
        row[0] = static_cast<uint16_t>(p01 & 0xffffu);
        row[1] = static_cast<uint16_t>(p01 >> 16);
        row[2] = static_cast<uint16_t>(p23 & 0xffffu);
        row[3] = static_cast<uint16_t>(p23 >> 16);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int u = tid + j * 256;
        const int x = u >> 3, c = u & 7;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = static_cast<uint32_t>(t[(c * 8 + 2 * e) * kTS + x]) |
                   (static_cast<uint32_t>(t[(c * 8 + 2 * e + 1) * kTS + x]) << 16);
        constexpr int cpr = D / 8;
        const int kb = kt * (kTB / D) + c / cpr;
        *reinterpret_cast<uint4*>(o.dst + packed_offset<D>(x0 + x, kb, c % cpr, nkb)) =
            make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// Workgroups an operand needs: direct units, or 64 x 64 transpose blocks.
inline int64_t pack_blocks(bool direct, int64_t rows_p, int64_t kp) {
    return direct ? (rows_p * (kp / 8) + kUnitsPerBlock - 1) / kUnitsPerBlock
                  : (rows_p / kTB) * (kp / kTB);
}

// DA / DB: the operand is packed directly (k contiguous in its source).
template <int D, bool DA, bool DB, bool VA, bool VB>
__global__ __launch_bounds__(256) void pack_kernel(PackArgs p) {
    __shared__ uint16_t t[kTB * kTS];   // transpose tile
    const int b = static_cast<int>(blockIdx.x);
    if (b < p.a.blocks) {
        if (DA) pack_direct<D, VA>(p.a, p.nkb, p.K, b);
        else pack_transpose<D, VA>(p.a, p.nkb, p.K, b, t);
    } else {
        if (DB) pack_direct<D, VB>(p.b, p.nkb, p.K, b - p.a.blocks);
        else pack_transpose<D, VB>(p.b, p.nkb, p.K, b - p.a.blocks, t);
    }
}

// f32 output here, binary16 output from gemm_f16r_o16.hip.
template <int BM, int BN, int NS, int WM, int WN, int GM>
hipError_t launch_f16_ring(const F16Args& a, hipStream_t s) {
    if (a.C16) return launch_f16_ring_o16<BM, BN, NS, WM, WN, GM>(a, s);
    return launch_f16_ring_out<BM, BN, NS, WM, WN, GM, false>(a, s);
}

template <int BM, int BN, int ST, int WM, int WN, int GM, bool RS>
hipError_t launch_f16(const F16Args& a, hipStream_t s) {
    if (a.C16) return launch_f16_o16<BM, BN, ST, WM, WN, GM, RS>(a, s);
    return launch_f16_out<BM, BN, ST, WM, WN, GM, RS, false>(a, s);
}

#define G355_F16_RING_INSTANCE(BM, BN, NS, WM, WN, GM) \
    {{GEMM355_MODE_F16R, BM, BN, 32, NS, WM, WN, GM}, &launch_f16_ring<BM, BN, NS, WM, WN, GM>},
#define G355_F16_PANEL_INSTANCE(BM, BN, ST, WM, WN, GM)    \
    {{GEMM355_MODE_F16R, BM, BN, kPackK, ST, WM, WN, GM}, \
     &launch_f16<BM, BN, (ST == 1 ? 2 : ST), WM, WN, GM, ST == 1>},

const F16Instance kF16Instances[] = {G355_F16_RING_CONFIGS(G355_F16_RING_INSTANCE)
                                         G355_F16_PANEL_CONFIGS(G355_F16_PANEL_INSTANCE)};

}  // namespace

const F16Instance* f16_instances(int* count) {
    *count = static_cast<int>(sizeof(kF16Instances) / sizeof(kF16Instances[0]));
    return kF16Instances;
}

hipError_t launch_pack(const float* A, int64_t lda, bool ta, const float* B, int64_t ldb,
                       bool tb, int M, int N, int K, uint16_t* A16, uint16_t* B16t, int64_t mp,
                       int64_t np, int64_t kp, int depth, hipStream_t s) {
    if ((depth != 32 && depth != 64) || kp % kPackK != 0 || mp % kPackRows != 0 ||
        np % kPackRows != 0)
        return hipErrorInvalidValue;
    // A (op(A) = A, k contiguous) packs directly, A^T transposes; B (K x N)
    // transposes, B^T (N x K, k contiguous) packs directly.
    const bool da = !ta, db = tb;
    PackArgs p;
    p.a = PackOperand{A, lda, A16, mp, M, 0};
    p.b = PackOperand{B, ldb, B16t, np, N, 0};
    p.nkb = kp / depth;
    p.K = K;
    const int64_t ab = pack_blocks(da, mp, kp), bb = pack_blocks(db, np, kp);
    if (ab + bb > 0x7fffffff) return hipErrorInvalidConfiguration;
    p.a.blocks = static_cast<int>(ab);
    p.b.blocks = static_cast<int>(bb);
    const bool va = (lda % 4 == 0) && ((reinterpret_cast<uintptr_t>(A) & 15) == 0);
    const bool vb = (ldb % 4 == 0) && ((reinterpret_cast<uintptr_t>(B) & 15) == 0);
    const dim3 grid(static_cast<unsigned>(ab + bb));
    auto go = [&](auto d, auto da_, auto db_) {
        constexpr int DD = decltype(d)::value;
        constexpr bool DA = decltype(da_)::value, DB = decltype(db_)::value;
        if (va && vb) pack_kernel<DD, DA, DB, true, true><<<grid, 256, 0, s>>>(p);
        else if (va) pack_kernel<DD, DA, DB, true, false><<<grid, 256, 0, s>>>(p);
        else if (vb) pack_kernel<DD, DA, DB, false, true><<<grid, 256, 0, s>>>(p);
        else pack_kernel<DD, DA, DB, false, false><<<grid, 256, 0, s>>>(p);
    };
    auto layouts = [&](auto d) {
        using T = std::true_type;
        using F = std::false_type;
        if (da && !db) go(d, T{}, F{});          // A, B (the plain layout)
        else if (!da && !db) go(d, F{}, F{});    // A^T, B
        else if (da && db) go(d, T{}, T{});      // A, B^T
        else go(d, F{}, T{});                    // A^T, B^T
    };
    if (depth == 32) layouts(std::integral_constant<int, 32>{});
    else layouts(std::integral_constant<int, 64>{});
    return hipGetLastError();
}

}  // namespace g355
