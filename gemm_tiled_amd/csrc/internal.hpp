// internal.hpp -- declarations shared by the kernels and the host side of
// libgemm355.  Not part of the public ABI (include/gemm355.h is).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gemm355.h"

namespace g355 {

// One tile configuration: the workgroup owns a BM x BN tile of C and walks K
// in steps of BK through a ring of ST shared-memory stages; its WM x WN
// wavefronts of 64 lanes split the tile; GM tile rows form one group of the
// rasterised tile order (L2 reuse).
// KS = 1 names the split-K configuration for few rows of C (the f32 kernel
// over slices of K, partial tiles summed by a second pass; in the f16r mode it
// rounds the operands as it loads them, with no packing pass); KS = 2 the
// few-rows configuration; KS = 3 the f16r configurations that round the
// operands as they stage them for the binary16 matrix instruction.
struct TileConfig {
    int mode;  // GEMM355_MODE_*
    int bm, bn, bk, st, wm, wn, gm;
    int ks = 0;
    int threads() const { return wm * wn * 64; }
    bool operator==(const TileConfig& o) const {
        return mode == o.mode && bm == o.bm && bn == o.bn && bk == o.bk && st == o.st &&
               wm == o.wm && wn == o.wn && gm == o.gm && ks == o.ks;
    }
};

// Arguments of one f32 GEMM launch.
// A and B as stored (see F32Variant::ta, tb).  In a split-K launch, slice z
// (blockIdx.y) of the K range [z*ksplit, (z+1)*ksplit) writes its partial
// product to C + z*M*ldc, and alpha, beta are applied by the reduction.
struct F32Args {
    const float* A;
    const float* B;
    float* C;
    int64_t lda, ldb, ldc;
    int M, N, K;
    float alpha, beta;
    int tiles_m, tiles_n;
    int ksplit = 0;   // k per slice (multiple of BK); 0 = no split
    // The f32 ring only (gemm_f32_ring.hip): with sk_q > 0 the launch is a
    // data-parallel + stream-K one.  Its G workgroups first take sk_dp whole
    // rounds of tiles (round r: the tile of block id r*G + blockIdx.x in the
    // usual order over the first sk_dp*G raster positions, G a multiple of
    // 8); the (tile, 16-deep panel) units of the remaining tiles, tile-major
    // in raster order, are then dealt in runs of sk_q.  A tile whose panels
    // span several runs is finished by the last of its workgroups to arrive
    // (counted in counts[tile - sk_dp*G], zero before and after the launch),
    // which adds the partial tiles the others stored in P (two BM x BN slots
    // per workgroup, G x 2 x BM x BN floats, below 2^31 bytes) in k order.
    // G = sk_grid.
    int sk_q = 0, sk_dp = 0, sk_grid = 0;
    float* P = nullptr;
    unsigned* counts = nullptr;
};

// Arguments of one f16 GEMM launch on rounded, packed operands: A16 holds A
// and B16t holds B transposed (k contiguous), both binary16 in the packed
// panel-major layout of gemm_f16r.hip (blocks of 256 rows x BK k, BK the
// configuration's panel depth, zero outside the logical matrices).
struct F16Args {
    const uint16_t* A16;
    const uint16_t* B16t;
    float* C;
    int64_t nkb;  // depth blocks of BK (padded K / BK)
    int64_t ldc;
    int M, N;
    float alpha, beta;
    int tiles_m, tiles_n;
    uint16_t* C16 = nullptr;   // binary16 output (then C is unused): the f16-output variant
    // The half-depth ring only: data-parallel rounds and stream-K runs as in
    // F32Args (P: gridDim.x x 2 x BM x BN floats; counts: one per tile).
    int sk_q = 0, sk_dp = 0, sk_grid = 0;
    float* P = nullptr;
    unsigned* counts = nullptr;
};

// Which variant of a compiled configuration a launch needs.
struct F32Variant {
    bool masked;  // some of M, N, K is not a tile multiple
    bool vec;     // 16-byte global loads are legal (lda, ldb % 4 == 0, aligned pointers)
    bool ta = false;   // op(A) = A^T: A is stored K x M
    bool tb = false;   // op(B) = B^T: B is stored N x K
    bool r16 = false;  // round A and B to binary16 (RNE) on load: the f16r mode
};

// The grid of a stream-K ring launch (F32Args / F16Args sk_*), checked: every
// unit of the tiles left after the data-parallel rounds lies in some run, the
// rounds use whole XCD groups of workgroups, the buffers are there.  0 when
// the arguments do not describe such a launch.
inline int ring_sk_grid(int64_t tiles, int64_t nkt, int q, int dp, int grid, const void* P,
                        const void* counts) {
    if (q <= 0 || dp < 0 || grid <= 0 || !P || !counts) return 0;
    if (dp > 0 && (grid % 8 != 0 || int64_t{dp} * grid > tiles)) return 0;
    const int64_t rest = (tiles - int64_t{dp} * grid) * nkt;
    if (tiles * nkt >= (int64_t{1} << 31) || rest > int64_t{grid} * q) return 0;
    return grid;
}

// Whether a call with ring configuration cfg runs the f32 ring (whole tiles
// of the plain layout, 16-byte aligned rows, K a multiple of 16, no split-K
// slices of the F32Args::ksplit kind); otherwise the register-staged kernel
// of the same tile runs it.
bool f32_ring_takes(const TileConfig& cfg, const F32Args& a, const F32Variant& v);

using F32Launch = hipError_t (*)(const F32Args&, F32Variant, hipStream_t);
using F16Launch = hipError_t (*)(const F16Args&, hipStream_t);

struct F32Instance {
    TileConfig cfg;
    F32Launch launch;
};
struct F16Instance {
    TileConfig cfg;
    F16Launch launch;
};

// Tables of compiled instances (defined in the kernel translation units).
const F32Instance* f32_instances(int* count);
const F16Instance* f16_instances(int* count);

// Rounding and packing pass of the f16r mode: op(A) (M x K) into Mp x Kp and
// op(B) (K x N) transposed into Np x Kp, Mp, Np multiples of 256, Kp of 64, in
// one launch, in depth blocks of `depth` (32 or 64) values.  ta: A is stored
// K x M (op(A) = A^T); tb: B is stored N x K (op(B) = B^T).
hipError_t launch_pack(const float* A, int64_t lda, bool ta, const float* B, int64_t ldb,
                       bool tb, int M, int N, int K, uint16_t* A16, uint16_t* B16t, int64_t mp,
                       int64_t np, int64_t kp, int depth, hipStream_t s);

// C = beta*C (beta == 0: C = 0 without reading it); C16: the same on binary16
// storage (rounded to nearest even).
hipError_t launch_scale_c(float* C, int64_t ldc, int M, int N, float beta, hipStream_t s);
hipError_t launch_scale_c16(uint16_t* C16, int64_t ldc, int M, int N, float beta, hipStream_t s);

// The split-K reduction: C = alpha * sum_{z < S} P[z] + beta * C, slices
// summed in order z = 0, 1, ... (P: S slices of M x N, dense).
hipError_t launch_splitk_reduce(const float* P, int S, int M, int N, float alpha, float beta,
                                float* C, int64_t ldc, hipStream_t s);
// The same into binary16 storage C16 (read as binary16 when beta != 0, the
// result rounded to nearest even).
hipError_t launch_splitk_reduce16(const float* P, int S, int M, int N, float alpha, float beta,
                                  uint16_t* C16, int64_t ldc, hipStream_t s);

// The split-K configuration of a mode (KS = 1) and its launch.
TileConfig splitk_config(int mode);
hipError_t launch_f32_splitk(const F32Args& a, F32Variant v, hipStream_t s);

// The few-rows configuration (KS=2, gemm_rows.hip): B streamed from memory
// into registers, k split within and across workgroups.  Needs 16-byte loads
// of B: B aligned, ldb % 4 == 0, and N % 4 == 0 (B is K x N) or K % 4 == 0
// (B stored N x K).  depth is the k per slice, a multiple of
// rows_depth_unit(); with slices > 1 the workgroups store partial tiles in P
// and the last one of each column of workgroups (counted in `counts`, zero
// before and after the launch) adds them in slice order and writes C.
TileConfig rows_config(int mode);
int rows_depth_unit();
int rows_group(int M);
bool rows_supported(bool ta, bool tb, const float* B, int64_t lda, int64_t ldb, int M, int N,
                    int K);
int rows_counters(int M, int N);
// tc: C is stored transposed (the few-columns form, run as the few-rows one
// on C^T = op(B)^T op(A)^T).
hipError_t launch_f32_rows(const float* A, int64_t lda, bool ta, const float* B, int64_t ldb,
                           bool tb, bool r16, float* C, uint16_t* C16, int64_t ldc, bool tc, int M,
                           int N, int K, float alpha, float beta, int depth, int slices, float* P,
                           unsigned* counts, hipStream_t s);

// The configurations that round the operands to binary16 as they stage them
// through registers (KS=3, BK=64, gemm_f16r_direct.hip): f16r only, no
// packing pass; K is split over blockIdx.y in slices of `depth` (a multiple
// of the panel depth) and, with slices > 1,
// the workgroups of a tile store their accumulators in P (slices x tiles x
// BM x BN floats, below 2^31 bytes) and the last one to arrive (counted in
// counts[tile], zero before and after the launch) adds them in slice order
// and writes C (f32) or C16 (binary16, when C16 is not null).
struct DirectArgs {
    const float* A;
    const float* B;
    float* C;
    uint16_t* C16;
    float* P;
    unsigned* counts;
    int64_t lda, ldb, ldc;
    int M, N, K;
    float alpha, beta;
    int tiles_m, tiles_n;
    int depth, slices;
    bool tc = false;   // C stored transposed: element (row, col) at C[col * ldc + row]
};
using DirectLaunch = hipError_t (*)(const DirectArgs&, bool ta, bool tb, bool masked, hipStream_t);
struct DirectInstance {
    TileConfig cfg;
    DirectLaunch launch;
};
const DirectInstance* direct_instances(int* count);
// The KS=3 configurations with BK = 32 (gemm_panel_ring.hip), in both modes:
// f32 panels in a ring of direct-to-LDS copies, each fragment read in f32 and
// multiplied on v_mfma_f32_16x16x4_f32 (f32) or rounded to binary16 for
// v_mfma_f32_16x16x32_f16 (f16r).  They take every operand layout with
// 16-byte aligned rows and K % 32 == 0, N % 4 == 0 where B is stored K x N
// and M % 4 == 0 where A is stored K x M (panel_ring_takes), slices of K a
// multiple of 32 deep; binary16 C in f16r only.
const DirectInstance* panel_ring_instances(int mode, int* count);
bool panel_ring_takes(bool ta, bool tb, const float* A, int64_t lda, const float* B, int64_t ldb,
                      int64_t M, int64_t N, int64_t K);

// Measurement kernels.
hipError_t launch_roof_mfma(int mode, int form, int64_t iters, int blocks, float* sink, double* flops,
                            hipStream_t s);
hipError_t launch_roof_fma(int64_t iters, int blocks, float* sink, double* flops, hipStream_t s);
hipError_t launch_roof_hbm(const void* buf, int64_t bytes, int blocks, float* sink,
                           hipStream_t s);
hipError_t launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s);
// p[0..n) = value on stream s (a kernel, never a memset).
hipError_t launch_fill_u32(unsigned* p, int64_t n, unsigned value, hipStream_t s);

// The workgroup -> tile mapping used by every GEMM kernel.  Consecutive
// workgroup ids are dealt to the 8 XCDs of the chip in turn; the remap gives
// each XCD one contiguous run of the rasterised order, so the tiles that
// share an XCD's L2 also share A rows and B columns.  Within the run, tiles
// go down GM tile rows before moving one tile column right.
// Position pos of the rasterised tile order: groups of gm tile rows, column
// by column inside a group.
__device__ __forceinline__ void raster_tile(int pos, int tiles_m, int tiles_n, int gm, int& tm,
                                            int& tn) {
    const int per_group = gm * tiles_n;
    const int group = pos / per_group;
    const int first_m = group * gm;
    const int rows = min(tiles_m - first_m, gm);
    const int in_group = pos - group * per_group;
    tm = first_m + in_group % rows;
    tn = in_group / rows;
}

__device__ __forceinline__ void tile_of_block(int g, int G, int tiles_m, int tiles_n, int gm,
                                              int& tm, int& tn) {
    const int xcd = g & 7;
    const int q = G >> 3, r = G & 7;
    const int gg = xcd * q + (xcd < r ? xcd : r) + (g >> 3);
    raster_tile(gg, tiles_m, tiles_n, gm, tm, tn);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// ----------------------------------------------------------------------------
// Shared-memory rings filled by direct global->LDS copies (the f16 ring and
// the f32 ring kernels).
// ----------------------------------------------------------------------------
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt vmcnt(N) with N a compile-time constant (at most 63).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for the panel ring.  __syncthreads() carries a workgroup
// fence, for which the compiler waits until every outstanding global->LDS fill
// of the wave has landed; that would cap the ring at one panel in flight.  The
// ring orders its fills itself (wait_vmcnt before this barrier), so a bare
// s_barrier suffices; this wave's own LDS reads are drained first so no other
// wave can refill a stage under them, and the asm is a compiler memory barrier.
__device__ __forceinline__ void ring_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One direct global->LDS copy of a wave: lane l copies the 16 bytes at `src`
// (its own address) to LDS byte address lds_base + 16 l.  Written as assembly
// so that the compiler does not track these copies: it cannot always tell
// which stage a shared-memory read may alias and would then wait for every
// copy in flight before the read, which serialises the ring.  The ring waits
// for its copies itself (wait_vmcnt before each barrier).  M0 carries the
// wave's LDS base (the compiler writes it before the statement); the copy
// needs one wait state after a write of M0.
__device__ __forceinline__ void lds_copy16(const void* src, uint32_t lds_base) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds_base)
                 : "memory");
}

// One masked direct copy of a wave, 4 bytes a lane: lane l copies the float at
// byte offset voff of the raw buffer `rsrc` to LDS byte address lds_base + 4 l.
// A lane whose offset lies past the buffer's record count (kLdsCopyOut) reads
// zero, which is how the copies zero-fill rows, columns and k past the edge
// of a matrix.  Untracked by the compiler for the reason given above.
typedef int i32x4_rsrc __attribute__((ext_vector_type(4)));
constexpr uint32_t kLdsCopyOut = 0x80000000u;
__device__ __forceinline__ i32x4_rsrc copy_rsrc(const float* base) {
    // raw buffer of 32-bit data, record count 2^31 - 1 (every offset the
    // copies use for a lane inside the matrix stays below 2^30)
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const i32x4_rsrc r = {static_cast<int>(static_cast<uint32_t>(a)), static_cast<int>((a >> 32) & 0xffff),
                          0x7fffffff, 0x00020000};
    return r;
}
__device__ __forceinline__ void lds_copy4_masked(i32x4_rsrc rsrc, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds" : : "v"(voff), "s"(rsrc), "{m0}"(lds_base)
                 : "memory");
}
// The same with 16 bytes a lane (lane l to lds_base + 16 l): for operands whose
// 16-byte chunks lie wholly inside or wholly outside the matrix.
__device__ __forceinline__ void lds_copy16_masked(i32x4_rsrc rsrc, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(rsrc), "{m0}"(lds_base)
                 : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const unsigned char* generic_lds_ptr) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_u8*)(generic_lds_ptr)));
}


// An f32 result rounded to binary16 (nearest even) as a step of its own: the
// empty asm makes the value opaque, so the compiler cannot fold the rounding
// into the multiply-add that produced it (a mixed-precision FMA rounds the
// exact result to binary16 once, which differs from rounding the f32 value
// when that value is a binary16 tie).  Every binary16 result of the library
// is the f32 result of the same call with f32 output, rounded once.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    asm volatile("" : "+v"(x));
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// Epilogue shared by the GEMM kernels (phobos docs, "gemm, f32", section "The
// epilogue": C = alpha*acc + beta*C over the tile, C read in place).  A wave
// holds FM x FN accumulator blocks of 32x32; element e of lane l in a block
// sits at row 8*(e/4) + 4*(l/32) + e%4, column l%32, so one store instruction
// writes two 128-byte row segments.  beta == 0 never reads C.  Otherwise the
// 16 loads of a block are issued together before its 16 stores, so a wave
// waits for memory once per block rather than once per element.  C is touched
// exactly once, so its loads and stores are non-temporal: they do not evict
// the operand panels other workgroups are still re-reading from the caches.
// MASKED guards every access with row < M and col < N.  The value is
// fma(alpha, acc, beta*c) (one rounding for alpha*acc + beta*c), written out
// so that every epilogue of the library computes the same f32 number.
template <int FM, int FN, bool MASKED>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[FM][FN], float* __restrict__ C,
                                           int64_t ldc, int row0, int col0, int M, int N,
                                           float alpha, float beta, int lane) {
    const int h = lane >> 5, r32 = lane & 31;
    auto row_of = [&](int i, int e) { return row0 + i * 32 + 8 * (e >> 2) + 4 * h + (e & 3); };
    auto col_of = [&](int j) { return col0 + j * 32 + r32; };
    auto inside = [&](int row, int col) { return !MASKED || (row < M && col < N); };
    if (beta == 0.f) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = row_of(i, e), col = col_of(j);
                    if (inside(row, col))
                        __builtin_nontemporal_store(alpha * acc[i][j][e], C + (int64_t)row * ldc + col);
                }
        return;
    }
#pragma unroll
    for (int b = 0; b < FM * FN; ++b) {
        const int i = b / FN, j = b % FN;
        float v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = row_of(i, e), col = col_of(j);
            v[e] = inside(row, col) ? __builtin_nontemporal_load(C + (int64_t)row * ldc + col) : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = row_of(i, e), col = col_of(j);
            if (inside(row, col))
                __builtin_nontemporal_store(__builtin_fmaf(alpha, acc[i][j][e], beta * v[e]),
                                            C + (int64_t)row * ldc + col);
        }
        // keep the compiler from hoisting every block's loads above the first
        // stores (that would need FM*FN*16 live registers)
        asm volatile("" ::: "memory");
    }
}

// The epilogue of the f16-output variant: C16 holds binary16 bit patterns;
// C = alpha*acc + beta*C is evaluated in f32 as in store_tile (C widened
// exactly) and rounded to binary16 once, to nearest even.  Same tile walk.
template <int FM, int FN, bool MASKED>
__device__ __forceinline__ void store_tile16(const f32x16 (&acc)[FM][FN], uint16_t* __restrict__ C,
                                             int64_t ldc, int row0, int col0, int M, int N,
                                             float alpha, float beta, int lane) {
    const int h = lane >> 5, r32 = lane & 31;
    auto row_of = [&](int i, int e) { return row0 + i * 32 + 8 * (e >> 2) + 4 * h + (e & 3); };
    auto col_of = [&](int j) { return col0 + j * 32 + r32; };
    auto inside = [&](int row, int col) { return !MASKED || (row < M && col < N); };
    auto to16 = [](float x) { return f32_to_f16_bits(x); };
    auto to32 = [](uint16_t b) { return static_cast<float>(__builtin_bit_cast(_Float16, b)); };
#pragma unroll
    for (int b = 0; b < FM * FN; ++b) {
        const int i = b / FN, j = b % FN;
        float v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = row_of(i, e), col = col_of(j);
            v[e] = (beta != 0.f && inside(row, col)) ? to32(C[(int64_t)row * ldc + col]) : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = row_of(i, e), col = col_of(j);
            if (inside(row, col))
                C[(int64_t)row * ldc + col] = to16(
                    beta == 0.f ? alpha * acc[i][j][e] : __builtin_fmaf(alpha, acc[i][j][e], beta * v[e]));
        }
        asm volatile("" ::: "memory");
    }
}

}  // namespace g355
