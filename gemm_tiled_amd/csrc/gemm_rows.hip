// gemm_rows.hip -- the few-rows configuration (KS=2): C = alpha*op(A)@op(B) +
// beta*C when C has few rows, the lab's skinny shapes ("Part 5": M from 1 to a
// few dozen at K = N = 4096).  There the arithmetic intensity 2MNK /
// 4(MK + KN + MN) is far below the ridge: the call streams B from memory once
// and its time is B's bytes over the memory bandwidth.  So B goes straight
// from global memory into registers (16-byte loads, no shared-memory staging,
// every load of a 64-deep chunk in flight at once), and the multiply-adds run
// on the matrix unit, whose f32 rate consumes B about three times faster than
// the memory delivers it for up to 16 rows.
//
// Work: a workgroup of four waves owns 64 columns of C, one group of 16*MB
// rows and one slice of K; wave w takes a quarter of the slice.  The wave's
// 64 lanes hold, per 16-deep step, lane (q, c) = (l / 16, l % 16):
//   B rows kb + 4q + t (t = 0..3), columns n0 + 4c .. n0 + 4c + 3 (one float4
//   per t: component j is column n0 + 4c + j);
//   A rows m0 + 16 mb + c, columns kb + 4q + t.
// v_mfma_f32_16x16x4_f32 number (t, j) multiplies A[., k = kb + 4q + t] by
// B[k, n0 + 4c + j]: its k index is the lane quarter q, its row index c (A),
// its column index c (B), so block acc[mb][j] accumulates rows m0 + 16 mb ..
// +15 against columns {n0 + 4c + j}.  Lane l of that block holds rows
// 4q + e (e = 0..3), column n0 + 4c + j: the four blocks j give it the float4
// of columns n0 + 4c .. +3 of each of its rows.
//
// The four waves' sums are added in wave order through shared memory; one
// slice then applies the epilogue, more slices store dense partial tiles that
// the split-K reduction (aux_kernels.hip) adds in slice order.  In the f16r
// mode A and B are rounded to binary16 on load (RNE), which the f32 matrix
// instruction then multiplies exactly and accumulates in f32.
#include "internal.hpp"

namespace g355 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCols = 64;     // columns of C per workgroup
constexpr int kWaves = 4;     // waves per workgroup, each a quarter of the slice
constexpr int kChunk = 64;    // k per loop iteration of a wave (4 steps of 16)

struct RowsArgs {
    const float* A;
    const float* B;
    float* C;            // f32 C (unused when C16 is set)
    uint16_t* C16;       // binary16 C, or nullptr
    float* P;            // dense partial tiles of every slice (slices > 1)
    unsigned* counts;    // one arrival counter per (column group, row group), zero between calls
    int64_t lda, ldb, ldc;
    int M, N, K;
    float alpha, beta;
    int depth;           // k per slice, a multiple of kWaves * kChunk
    int slices;
    bool tc;             // C is stored transposed: element (row, col) at C[col * ldc + row]
};

__device__ __forceinline__ float rn16(float x) {
    return static_cast<float>(static_cast<_Float16>(x));
}

// How a chunk reads A: row-major four k at a time (lda % 4 == 0, A aligned,
// K % 4 == 0), row-major one value at a time, or stored K x M.
enum AMode { kAVec = 0, kARow = 1, kACol = 2 };

// Raw buffer descriptor flags of gfx9-family GPUs: 32-bit data format.  The
// loads below never leave their matrix (every offset is clamped), so the
// descriptor's range check is not relied upon.
constexpr int kRsrcFlags = 0x00020000;

// One 64-deep chunk of a wave, loaded through buffer descriptors with 32-bit
// byte offsets.  Every load is inside its matrix: rows of A past M are read
// as row M - 1 and columns of B past N as column N - 1 (or the last float4),
// which only feeds rows and columns of the accumulators that are never
// stored; a chunk that starts past K (fetched ahead, never multiplied) is
// read at K - 64.  k past K must contribute zero: with KTAIL (K not a
// multiple of the chunk) each row index is clamped and the A values past K
// are replaced by zero; without it every multiplied chunk lies inside K, the
// per-lane offsets are computed once per chunk and each load adds a uniform
// offset.  Nothing touches the loaded values before the matrix instructions,
// so a chunk's loads stay in flight together while the other chunk is
// multiplied.
//
// VR = 0: the matrix-instruction form above (lane row c of each 16-row block).
// VR > 0 (at most VR rows, one group; VR = 1 or 2): every lane holds A rows
// 0 .. VR-1 at its own k and multiplies with vector FMAs; 16-row matrix
// instructions would waste 15/16 of their work on a single row.
template <int MB, int AM, bool TB, bool KTAIL, int VR>
struct Chunk {
    static constexpr int NA = VR > 0 ? VR : MB;   // A registers per step
    // B: without TB bv[s][t] holds row kk + t, columns col .. col + 3; with
    // TB bv[s][j] holds column col + j, rows kk .. kk + 3 (as stored).
    f32x4 bv[4][4];
    f32x4 av[4][NA];   // rows of A, k = kk .. kk + 3

    __device__ __forceinline__ void load(const RowsArgs& p, __amdgpu_buffer_rsrc_t ra,
                                         __amdgpu_buffer_rsrc_t rb, int k, int col, int m0, int q,
                                         int c) {
        if (!KTAIL) k = min(k, p.K - kChunk);   // K % kChunk == 0
        const int kq = k + 4 * q;   // this lane's first k of step 0
        const int ldb4 = static_cast<int>(p.ldb) * 4, lda4 = static_cast<int>(p.lda) * 4;
        auto krow = [&](int kk) { return KTAIL ? min(kk, p.K - 1) : kk; };
        if constexpr (!TB) {
            const int cl = min(col, p.N - 4) * 4;   // N % 4 == 0
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const f32x4 v = KTAIL
                        ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                        rb, krow(kq + 16 * s + t) * ldb4 + cl, 0, 0))
                        : __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                        rb, kq * ldb4 + cl, (16 * s + t) * ldb4, 0));
                    bv[s][t] = v;
                }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int nb = min(col + j, p.N - 1) * ldb4;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    // K % 4 == 0: a float4 along k starting below K is inside K
                    const f32x4 v = KTAIL
                        ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                        rb, nb + min(kq + 16 * s, p.K - 4) * 4, 0, 0))
                        : __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                        rb, nb + kq * 4, 64 * s, 0));
                    bv[s][j] = v;
                }
            }
        }
#pragma unroll
        for (int mb = 0; mb < NA; ++mb) {
            const int rc = min(VR > 0 ? mb : m0 + 16 * mb + c, p.M - 1);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int kk = kq + 16 * s;
                f32x4 v;
                if constexpr (AM == kAVec) {
                    // K % 4 == 0 here too
                    v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      ra, rc * lda4 + (KTAIL ? min(kk, p.K - 4) : kk) * 4, 0, 0));
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int kr = krow(kk + t);
                        const int off = AM == kACol ? kr * lda4 + rc * 4 : rc * lda4 + kr * 4;
                        v[t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra, off, 0, 0));
                    }
                }
                if constexpr (KTAIL) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) v[t] = kk + t < p.K ? v[t] : 0.f;
                }
                av[s][mb] = v;
            }
        }
    }

    // vector form: accv[r] += A[r][k] * B[k][col .. col + 3] over the lane's k
    template <bool R16>
    __device__ __forceinline__ void multiply_rows(f32x4 (&accv)[NA]) const {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                f32x4 b;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float x = TB ? bv[s][j][t] : bv[s][t][j];
                    b[j] = R16 ? rn16(x) : x;
                }
#pragma unroll
                for (int r = 0; r < NA; ++r) {
                    const float a = R16 ? rn16(av[s][r][t]) : av[s][r][t];
#pragma unroll
                    for (int j = 0; j < 4; ++j) accv[r][j] = __builtin_fmaf(a, b[j], accv[r][j]);
                }
            }
    }

    template <bool R16>
    __device__ __forceinline__ void multiply(f32x4 (&acc)[MB][4]) const {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                f32x4 b;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float x = TB ? bv[s][j][t] : bv[s][t][j];
                    b[j] = R16 ? rn16(x) : x;
                }
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const float a = R16 ? rn16(av[s][mb][t]) : av[s][mb][t];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b[j], acc[mb][j], 0, 0, 0);
                }
            }
    }
};

template <int MB, int AM, bool TB, bool R16, bool KTAIL, int VR>
__global__ __launch_bounds__(kWaves * 64) void gemm_rows_kernel(RowsArgs p) {
    static_assert(VR == 0 || MB == 1, "the vector form covers one row group");
    // per-wave sums: [wave][row][column quad]; the vector form has one more
    // level, the lane quarter, whose k subsets are added too
    constexpr int RED_ROWS = VR > 0 ? 4 * VR : 16 * MB;
    __shared__ f32x4 red[kWaves][RED_ROWS][kCols / 4];
    __shared__ unsigned last;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q = lane >> 4, c = lane & 15;
    const int n0 = blockIdx.x * kCols;
    const int slice = blockIdx.y;
    const int m0 = blockIdx.z * 16 * MB;
    const int kw = p.depth / kWaves;
    const int k_lo = slice * p.depth + wave * kw;
    const int k_hi = min(k_lo + kw, p.K);
    const int col = n0 + 4 * c;              // first of this lane's four columns

    f32x4 acc[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 accv[VR > 0 ? VR : 1];
#pragma unroll
    for (int r = 0; r < (VR > 0 ? VR : 1); ++r) accv[r] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Buffer descriptors over A and B (their byte extents fit 32-bit offsets).
    const int64_t a_bytes = AM == kACol ? ((int64_t)(p.K - 1) * p.lda + p.M) * 4
                                        : ((int64_t)(p.M - 1) * p.lda + p.K) * 4;
    const int64_t b_bytes = TB ? ((int64_t)(p.N - 1) * p.ldb + p.K) * 4
                               : ((int64_t)(p.K - 1) * p.ldb + p.N) * 4;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.A), (short)0, static_cast<int>(a_bytes), kRsrcFlags);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.B), (short)0, static_cast<int>(b_bytes), kRsrcFlags);
    // Two chunks per pass, both fetched before either is multiplied (a chunk
    // starting past k_hi is fetched at a clamped place and not multiplied, so
    // the loads are unconditional).  The host picks the slice depth so that a
    // wave's range is usually exactly one pass (128 k): straight-line code,
    // every load in flight at once.  The scheduling barriers keep the
    // compiler from sinking each load next to its use.
    // With 32 or 64 rows (MB > 1) one chunk is in registers at a time, which
    // keeps two waves per SIMD (the other wave's loads cover the wait).
    if constexpr (MB > 1) {
        Chunk<MB, AM, TB, KTAIL, VR> x;
        for (int k = k_lo; k < k_hi; k += kChunk) {
            __builtin_amdgcn_sched_barrier(0);
            x.load(p, ra, rb, k, col, m0, q, c);
            __builtin_amdgcn_sched_barrier(0);
            x.template multiply<R16>(acc);
        }
    } else {
        Chunk<MB, AM, TB, KTAIL, VR> x, y;
        for (int k = k_lo; k < k_hi; k += 2 * kChunk) {
            __builtin_amdgcn_sched_barrier(0);
            x.load(p, ra, rb, k, col, m0, q, c);
            y.load(p, ra, rb, k + kChunk, col, m0, q, c);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (VR > 0) {
                x.template multiply_rows<R16>(accv);
                if (k + kChunk < k_hi) y.template multiply_rows<R16>(accv);
            } else {
                x.template multiply<R16>(acc);
                if (k + kChunk < k_hi) y.template multiply<R16>(acc);
            }
        }
    }

    // the four waves' sums (and, in the vector form, the four lane quarters'),
    // added in a fixed order
    const int t = threadIdx.x;
    const int c4 = t % (kCols / 4);
    const int cc = n0 + 4 * c4;
    f32x4 sum[MB];
    if constexpr (VR > 0) {
#pragma unroll
        for (int r = 0; r < VR; ++r) red[wave][4 * r + q][c] = accv[r];
        __syncthreads();
        const int rr = t / (kCols / 4);            // row (threads of rows >= VR idle)
        sum[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (rr < VR) {
            sum[0] = red[0][4 * rr][c4];
#pragma unroll
            for (int w = 0; w < kWaves; ++w)
#pragma unroll
                for (int qq = 0; qq < 4; ++qq)
                    if (w || qq) sum[0] += red[w][4 * rr + qq][c4];
        }
    } else {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                red[wave][16 * mb + 4 * q + e][c] =
                    f32x4{acc[mb][0][e], acc[mb][1][e], acc[mb][2][e], acc[mb][3][e]};
        __syncthreads();
#pragma unroll
        for (int r = 0; r < MB; ++r) {
            const int rr = t / (kCols / 4) + 16 * r;   // row within the group
            sum[r] = red[0][rr][c4];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) sum[r] += red[w][rr][c4];
        }
    }

    if (p.slices > 1) {
        // Store this slice's partial tile, then count the workgroup in; the
        // last workgroup of the column group to arrive adds all slices in
        // slice order.  The partial tiles are written and read with
        // device-scope (SC1) buffer accesses, which bypass the caches private
        // to one XCD, and each wave waits for its stores to complete before
        // the barrier that precedes the count: the last workgroup sees every
        // slice without a whole-cache write-back or invalidation.  Partial
        // rows are NP = N rounded up to 4 floats apart, so every access is a
        // 16-byte one (the padding columns hold values nobody reads).
        constexpr int kSC1 = 1 << 4;   // cache-policy bit of the buffer intrinsics
        const int np = (p.N + 3) & ~3;
        const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
            p.P, (short)0, static_cast<int>((int64_t)p.slices * p.M * np * 4), kRsrcFlags);
#pragma unroll
        for (int r = 0; r < MB; ++r) {
            const int row = m0 + t / (kCols / 4) + 16 * r;
            if (row < p.M && cc < p.N)
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(u32x4, sum[r]), rp,
                    static_cast<int>((((int64_t)slice * p.M + row) * np + cc) * 4), 0, kSC1);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        unsigned* count = p.counts + blockIdx.z * gridDim.x + blockIdx.x;
        if (t == 0)
            last = __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   static_cast<unsigned>(p.slices - 1);
        __syncthreads();
        if (!last) return;
        if (t == 0) __hip_atomic_store(count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int r = 0; r < MB; ++r) {
            const int row = m0 + t / (kCols / 4) + 16 * r;
            if (row >= p.M || cc >= p.N) continue;
            const int base = static_cast<int>(((int64_t)row * np + cc) * 4);
            const int stride = static_cast<int>((int64_t)p.M * np * 4);
            f32x4 v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, base, 0, kSC1));
            for (int z = 1; z < p.slices; ++z)
                v += __builtin_bit_cast(f32x4,
                                        __builtin_amdgcn_raw_buffer_load_b128(rp, base, z * stride, kSC1));
            sum[r] = v;
        }
    }

    // epilogue: C = alpha*sum + beta*C (beta == 0 does not read C)
#pragma unroll
    for (int r = 0; r < MB; ++r) {
        const int row = m0 + t / (kCols / 4) + 16 * r;
        if (row >= p.M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (cc + j >= p.N) continue;
            const int64_t at = p.tc ? (int64_t)(cc + j) * p.ldc + row : (int64_t)row * p.ldc + cc + j;
            if (p.C16) {
                const float old = p.beta == 0.f ? 0.f
                                                : static_cast<float>(__builtin_bit_cast(_Float16, p.C16[at]));
                const float v = p.beta == 0.f ? p.alpha * sum[r][j]
                                              : __builtin_fmaf(p.alpha, sum[r][j], p.beta * old);
                p.C16[at] = f32_to_f16_bits(v);
            } else {
                p.C[at] = p.beta == 0.f ? p.alpha * sum[r][j]
                                        : __builtin_fmaf(p.alpha, sum[r][j], p.beta * p.C[at]);
            }
        }
    }
}

template <int MB, bool KTAIL, int VR = 0>
hipError_t launch_mb(const RowsArgs& a, int am, bool tb, bool r16, dim3 grid, hipStream_t s) {
    const dim3 block(kWaves * 64);
#define G355_ROWS_LAUNCH(AM, TB, R16) gemm_rows_kernel<MB, AM, TB, R16, KTAIL, VR><<<grid, block, 0, s>>>(a)
#define G355_ROWS_AM(TB, R16)                                \
    do {                                                     \
        if (am == kAVec) G355_ROWS_LAUNCH(kAVec, TB, R16);   \
        else if (am == kARow) G355_ROWS_LAUNCH(kARow, TB, R16); \
        else G355_ROWS_LAUNCH(kACol, TB, R16);               \
    } while (0)
    if (r16) {
        if (tb) G355_ROWS_AM(true, true);
        else G355_ROWS_AM(false, true);
    } else {
        if (tb) G355_ROWS_AM(true, false);
        else G355_ROWS_AM(false, false);
    }
#undef G355_ROWS_AM
#undef G355_ROWS_LAUNCH
    return hipGetLastError();
}

}  // namespace

TileConfig rows_config(int mode) {
    TileConfig c{mode, 16, kCols, kChunk, 1, 1, kWaves, 1};
    c.ks = 2;
    return c;
}

int rows_depth_unit() { return kWaves * kChunk; }

int rows_group(int M) { return M <= 16 ? 16 : M <= 32 ? 32 : 64; }

bool rows_supported(bool ta, bool tb, const float* B, int64_t lda, int64_t ldb, int M, int N,
                    int K) {
    const bool aligned = (reinterpret_cast<uintptr_t>(B) & 15) == 0 && ldb % 4 == 0;
    // byte offsets of the buffer loads are 32-bit
    const int64_t a_bytes = ta ? ((int64_t)(K - 1) * lda + M) * 4 : ((int64_t)(M - 1) * lda + K) * 4;
    const int64_t b_bytes = tb ? ((int64_t)(N - 1) * ldb + K) * 4 : ((int64_t)(K - 1) * ldb + N) * 4;
    const int64_t limit = int64_t{1} << 31;
    return aligned && (tb ? K % 4 == 0 : N % 4 == 0) && a_bytes < limit && b_bytes < limit;
}

// C (f32) or C16 (binary16) receives the result (tc: stored transposed, the
// few-columns form: the caller passes the transposed problem C^T = op(B)^T
// op(A)^T).  depth is the k per slice
// (a multiple of rows_depth_unit()); with slices > 1, P holds slices x M x NP
// floats of partial tiles (NP = N rounded up to 4) and counts one zeroed
// counter per workgroup column
// (ceil(N/64) x row groups), which the kernel leaves zero again.
hipError_t launch_f32_rows(const float* A, int64_t lda, bool ta, const float* B, int64_t ldb,
                           bool tb, bool r16, float* C, uint16_t* C16, int64_t ldc, bool tc, int M,
                           int N, int K, float alpha, float beta, int depth, int slices, float* P,
                           unsigned* counts, hipStream_t s) {
    if (depth <= 0 || depth % rows_depth_unit() != 0) return hipErrorInvalidValue;
    if (!rows_supported(ta, tb, B, lda, ldb, M, N, K)) return hipErrorInvalidValue;
    if (slices > 1 && (!P || !counts)) return hipErrorInvalidValue;
    const RowsArgs a{A, B, C, C16, P, counts, lda, ldb, ldc, M, N, K, alpha, beta, depth, slices, tc};
    const int group = rows_group(M);
    const dim3 grid((N + kCols - 1) / kCols, slices, (M + group - 1) / group);
    const bool tail = K % kChunk != 0;
    const bool a_vec = !ta && lda % 4 == 0 && (reinterpret_cast<uintptr_t>(A) & 15) == 0 && K % 4 == 0;
    const int am = ta ? kACol : a_vec ? kAVec : kARow;
    // one or two rows (and K a whole number of chunks): the vector form
    if (M == 1 && !tail) return launch_mb<1, false, 1>(a, am, tb, r16, grid, s);
    if (M == 2 && !tail) return launch_mb<1, false, 2>(a, am, tb, r16, grid, s);
    if (group == 16) return tail ? launch_mb<1, true>(a, am, tb, r16, grid, s)
                                 : launch_mb<1, false>(a, am, tb, r16, grid, s);
    if (group == 32) return tail ? launch_mb<2, true>(a, am, tb, r16, grid, s)
                                 : launch_mb<2, false>(a, am, tb, r16, grid, s);
    return tail ? launch_mb<4, true>(a, am, tb, r16, grid, s)
                : launch_mb<4, false>(a, am, tb, r16, grid, s);
}

int rows_counters(int M, int N) { return ((N + kCols - 1) / kCols) * ((M + rows_group(M) - 1) / rows_group(M)); }

}  // namespace g355
