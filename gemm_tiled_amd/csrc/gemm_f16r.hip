// gemm_f16r.hip -- the f16r mode: A and B rounded to binary16 (round to
// nearest even), products accumulated in f32 on the gfx950 matrix cores
// (v_mfma_f32_32x32x16_f16), then C = alpha*acc + beta*C in f32.
//
// The phobos docs page "gemm on tensor cores" (section "What changes") keeps
// the f32 kernel line for line and only moves dot onto the matrix units with
// operands rounded to f16.  Here the rounding is a pass of its own: A is
// rounded into a row-major binary16 copy and B into a transposed binary16 copy
// (each row holds one column of B, k contiguous), both zero-padded to whole
// tiles.  The GEMM kernel then reads two k-contiguous operands with 16-byte
// loads, half the bytes of the f32 source, with no masks on its loads; only the
// epilogue is masked.  The zero padding is the masked-edge rule of the
// Matrix Multiplication lab's tiled kernels (out-of-range operands load as 0).
#include "internal.hpp"

namespace g355 {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Two f32 -> two binary16, round to nearest even (a C++ conversion to
// _Float16 is correctly rounded in the default rounding mode), packed.
__device__ __forceinline__ uint32_t pack_rn(float lo, float hi) {
    const f16x2 v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

// ----------------------------------------------------------------------------
// A -> A16: row-major, Mp x Kp, zero outside M x K.  One thread writes 8
// consecutive k of one row (16 bytes).
// ----------------------------------------------------------------------------
template <bool VEC>
__global__ __launch_bounds__(256) void round_a_kernel(const float* __restrict__ A, int64_t lda,
                                                      int M, int K, uint16_t* __restrict__ A16,
                                                      int64_t mp, int64_t kp) {
    const int64_t k8s = kp / 8;
    const int64_t units = mp * k8s;
    for (int64_t u = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; u < units;
         u += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = u / k8s;
        const int k = static_cast<int>(u - r * k8s) * 8;
        float v[8];
        if (r < M && VEC && k + 7 < K) {
            const float4* src = reinterpret_cast<const float4*>(A + r * lda + k);
            const float4 x = src[0], y = src[1];
            v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
            v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (r < M && k + e < K) ? A[r * lda + k + e] : 0.f;
        }
        uint4 o;
        o.x = pack_rn(v[0], v[1]);
        o.y = pack_rn(v[2], v[3]);
        o.z = pack_rn(v[4], v[5]);
        o.w = pack_rn(v[6], v[7]);
        *reinterpret_cast<uint4*>(A16 + r * kp + k) = o;
    }
}

// ----------------------------------------------------------------------------
// B -> B16t: B16t[n][k] = rn(B[k][n]), Np x Kp, zero outside.  A 64 x 64 block
// of B is read along n (coalesced), rounded, transposed through LDS and written
// along k (coalesced).
// ----------------------------------------------------------------------------
constexpr int kTB = 64;        // transpose block edge
constexpr int kTS = kTB + 2;   // LDS row stride in halves

template <bool VEC>
__global__ __launch_bounds__(256) void round_bt_kernel(const float* __restrict__ B, int64_t ldb,
                                                       int K, int N, uint16_t* __restrict__ B16t,
                                                       int64_t kp) {
    __shared__ uint16_t t[kTB * kTS];   // t[k][n]
    const int n0 = blockIdx.x * kTB;
    const int k0 = blockIdx.y * kTB;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + i * 256;
        const int kr = idx >> 4, nq = (idx & 15) * 4;
        const int k = k0 + kr, n = n0 + nq;
        float v[4];
        if (k < K && VEC && n + 3 < N) {
            const float4 x = *reinterpret_cast<const float4*>(B + (int64_t)k * ldb + n);
            v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = (k < K && n + e < N) ? B[(int64_t)k * ldb + n + e] : 0.f;
        }
        const uint32_t p01 = pack_rn(v[0], v[1]);
        const uint32_t p23 = pack_rn(v[2], v[3]);
        uint16_t* row = t + kr * kTS + nq;
        row[0] = static_cast<uint16_t>(p01 & 0xffffu);
        row[1] = static_cast<uint16_t>(p01 >> 16);
        row[2] = static_cast<uint16_t>(p23 & 0xffffu);
        row[3] = static_cast<uint16_t>(p23 >> 16);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int u = tid + j * 256;
        const int n = u >> 3, k8 = (u & 7) * 8;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = static_cast<uint32_t>(t[(k8 + 2 * e) * kTS + n]) |
                   (static_cast<uint32_t>(t[(k8 + 2 * e + 1) * kTS + n]) << 16);
        *reinterpret_cast<uint4*>(B16t + (int64_t)(n0 + n) * kp + k0 + k8) =
            make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// ----------------------------------------------------------------------------
// The f16 GEMM on the rounded operands.
// ----------------------------------------------------------------------------
template <int BM, int BN, int BK, int WM, int WN>
struct F16Shape {
    static constexpr int NT = WM * WN * 64;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 32, FN = TN / 32;
    static constexpr int KH = BK / 2;        // k per lane half per panel
    static constexpr int KSTEPS = BK / 16;   // matrix instructions per block per panel
    // Both panels are stored n- or m-major with k contiguous; rows padded by 8
    // halves so the 16-byte reads of 16 consecutive rows hit distinct banks.
    static constexpr int AS = BK + 8;
    static constexpr int A_STAGE = BM * AS;
    static constexpr int B_STAGE = BN * AS;
    static constexpr int LDS_HALVES = 2 * (A_STAGE + B_STAGE);
    static constexpr int A_LD = BM * BK / 8 / NT;   // 16-byte loads per thread per panel
    static constexpr int B_LD = BN * BK / 8 / NT;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(BK % 16 == 0 && 64 % BK == 0, "BK must be 16, 32 or 64");
    static_assert(256 % BM == 0 && 256 % BN == 0, "operands are padded to multiples of 256");
    static_assert((BM * BK / 8) % NT == 0 && (BN * BK / 8) % NT == 0, "panel split");
    static_assert(LDS_HALVES * 2 <= 160 * 1024, "LDS budget of one CU");
};

template <int BM, int BN, int BK, int WM, int WN, int GM, bool MASKED>
__global__ __launch_bounds__(WM * WN * 64) void gemm_f16_kernel(F16Args p) {
    using S = F16Shape<BM, BN, BK, WM, WN>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[S::LDS_HALVES];
    uint16_t* const As = smem;                    // [2][BM][AS]
    uint16_t* const Bs = smem + 2 * S::A_STAGE;   // [2][BN][AS]

    int tm, tn;
    tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, GM, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wr = wave / WN, wc = wave % WN;
    const int h = lane >> 5;
    const int r32 = lane & 31;

    const int64_t kp = p.kp;
    const uint16_t* __restrict__ A = p.A16 + (int64_t)m0 * kp;
    const uint16_t* __restrict__ B = p.B16t + (int64_t)n0 * kp;

    uint4 ra[S::A_LD], rb[S::B_LD];
    auto load_panels = [&](int k0) {
#pragma unroll
        for (int i = 0; i < S::A_LD; ++i) {
            const int idx = tid + i * S::NT;
            const int r = idx / (BK / 8), c = (idx % (BK / 8)) * 8;
            ra[i] = *reinterpret_cast<const uint4*>(A + (int64_t)r * kp + k0 + c);
        }
#pragma unroll
        for (int i = 0; i < S::B_LD; ++i) {
            const int idx = tid + i * S::NT;
            const int r = idx / (BK / 8), c = (idx % (BK / 8)) * 8;
            rb[i] = *reinterpret_cast<const uint4*>(B + (int64_t)r * kp + k0 + c);
        }
    };
    auto store_panels = [&](int stage) {
        uint16_t* as = As + stage * S::A_STAGE;
        uint16_t* bs = Bs + stage * S::B_STAGE;
#pragma unroll
        for (int i = 0; i < S::A_LD; ++i) {
            const int idx = tid + i * S::NT;
            const int r = idx / (BK / 8), c = (idx % (BK / 8)) * 8;
            *reinterpret_cast<uint4*>(as + r * S::AS + c) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < S::B_LD; ++i) {
            const int idx = tid + i * S::NT;
            const int r = idx / (BK / 8), c = (idx % (BK / 8)) * 8;
            *reinterpret_cast<uint4*>(bs + r * S::AS + c) = rb[i];
        }
    };

    f32x16 acc[S::FM][S::FN];
#pragma unroll
    for (int i = 0; i < S::FM; ++i)
#pragma unroll
        for (int j = 0; j < S::FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int nk = static_cast<int>(kp / BK);
    load_panels(0);
    store_panels(0);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) load_panels((kt + 1) * BK);

        // Lane half h feeds k in [h*KH, (h+1)*KH) of the panel, 8 per
        // instruction, to A and B alike.
        const uint16_t* as = As + cur * S::A_STAGE;
        const uint16_t* bs = Bs + cur * S::B_STAGE;
#pragma unroll
        for (int ks = 0; ks < S::KSTEPS; ++ks) {
            f16x8 a[S::FM], b[S::FN];
#pragma unroll
            for (int i = 0; i < S::FM; ++i)
                a[i] = *reinterpret_cast<const f16x8*>(
                    as + (wr * S::TM + i * 32 + r32) * S::AS + h * S::KH + ks * 8);
#pragma unroll
            for (int j = 0; j < S::FN; ++j)
                b[j] = *reinterpret_cast<const f16x8*>(
                    bs + (wc * S::TN + j * 32 + r32) * S::AS + h * S::KH + ks * 8);
#pragma unroll
            for (int i = 0; i < S::FM; ++i)
#pragma unroll
                for (int j = 0; j < S::FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0,
                                                                        0, 0);
        }

        if (more) store_panels(cur ^ 1);
        __syncthreads();
    }

    // Epilogue: C = alpha*acc + beta*C; element e of lane l of a 32x32 block
    // is row 8*(e/4) + 4*(l/32) + e%4, column l%32.
    const float alpha = p.alpha, beta = p.beta;
#pragma unroll
    for (int i = 0; i < S::FM; ++i) {
#pragma unroll
        for (int j = 0; j < S::FN; ++j) {
            const int col = n0 + wc * S::TN + j * 32 + r32;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + wr * S::TM + i * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                if (MASKED && (row >= p.M || col >= p.N)) continue;
                float* c = p.C + (int64_t)row * p.ldc + col;
                float v = alpha * acc[i][j][e];
                if (beta != 0.f) v += beta * *c;
                *c = v;
            }
        }
    }
}

template <int BM, int BN, int BK, int WM, int WN, int GM>
hipError_t launch_f16(const F16Args& a, hipStream_t s) {
    const dim3 grid(a.tiles_m * a.tiles_n), block(WM * WN * 64);
    const bool masked = (a.M % BM) != 0 || (a.N % BN) != 0;
    if (masked)
        gemm_f16_kernel<BM, BN, BK, WM, WN, GM, true><<<grid, block, 0, s>>>(a);
    else
        gemm_f16_kernel<BM, BN, BK, WM, WN, GM, false><<<grid, block, 0, s>>>(a);
    return hipGetLastError();
}

#define F16_INSTANCE(BM, BN, BK, WM, WN, GM) \
    {{GEMM355_MODE_F16R, BM, BN, BK, WM, WN, GM}, &launch_f16<BM, BN, BK, WM, WN, GM>}

const F16Instance kF16Instances[] = {
    F16_INSTANCE(256, 256, 64, 2, 2, 8),
    F16_INSTANCE(256, 256, 32, 2, 2, 8),
    F16_INSTANCE(256, 128, 64, 2, 2, 8),
    F16_INSTANCE(128, 256, 64, 2, 2, 8),
    F16_INSTANCE(128, 128, 64, 2, 2, 8),
    F16_INSTANCE(128, 128, 32, 2, 2, 8),
    F16_INSTANCE(128, 64, 64, 2, 2, 8),
    F16_INSTANCE(64, 64, 64, 2, 2, 8),
};

}  // namespace

const F16Instance* f16_instances(int* count) {
    *count = static_cast<int>(sizeof(kF16Instances) / sizeof(kF16Instances[0]));
    return kF16Instances;
}

hipError_t launch_round_a(const float* A, int64_t lda, int M, int K, uint16_t* A16, int64_t mp,
                          int64_t kp, hipStream_t s) {
    const int64_t units = mp * (kp / 8);
    const int64_t want = (units + 255) / 256;
    const int blocks = static_cast<int>(want < 8192 ? (want > 0 ? want : 1) : 8192);
    const bool vec = (lda % 4 == 0) && ((reinterpret_cast<uintptr_t>(A) & 15) == 0);
    if (vec)
        round_a_kernel<true><<<blocks, 256, 0, s>>>(A, lda, M, K, A16, mp, kp);
    else
        round_a_kernel<false><<<blocks, 256, 0, s>>>(A, lda, M, K, A16, mp, kp);
    return hipGetLastError();
}

hipError_t launch_round_bt(const float* B, int64_t ldb, int K, int N, uint16_t* B16t, int64_t np,
                           int64_t kp, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(np / kTB), static_cast<unsigned>(kp / kTB));
    const bool vec = (ldb % 4 == 0) && ((reinterpret_cast<uintptr_t>(B) & 15) == 0);
    if (vec)
        round_bt_kernel<true><<<grid, 256, 0, s>>>(B, ldb, K, N, B16t, kp);
    else
        round_bt_kernel<false><<<grid, 256, 0, s>>>(B, ldb, K, N, B16t, kp);
    return hipGetLastError();
}

}  // namespace g355
