// gemm_f32_ring.hip -- the f32 GEMM on a ring of direct-to-LDS panels, for
// row-major A and B: whole tiles with 16-byte aligned rows, or (the masked
// form) any shape and any leading dimensions.
//
// Same computation as gemm_f32_kernel (the phobos "gemm, f32" page: one output
// tile per workgroup, a K loop over BK-deep panels staged in shared memory,
// the alpha/beta epilogue over the tile), on v_mfma_f32_32x32x2_f32 at full
// f32 precision.  What differs is how the panels reach shared memory: instead
// of every thread loading its part of the next panel into registers and
// storing it after the math of the current one (one panel ahead, a barrier
// per panel with the copy in between), each wave issues global->LDS copies
// (global_load_lds_dwordx4, 1 KB per instruction) into a ring of NS stages,
// NS - 1 panels ahead, as in the f16 ring kernel.
//
// Panel layout (BK = 16 floats of k):
//   A: BM rows of 64 bytes (four 16-byte chunks of 4 k); chunk c of row r sits
//      at position c ^ ((r / 4) % 4), so the 16 lanes that read one chunk of 16
//      consecutive rows hit 16 different bank groups.  A copy instruction
//      fills 16 rows; lane l fetches the global chunk that belongs at its
//      destination position.
//   B: 16 k-rows of BN = 256 floats (one copy instruction each), rows
//      1024 + 16 bytes apart: the two lane halves, which read rows 8 apart,
//      then fall in opposite halves of the 64 banks.
// The masked form copies 4 bytes a lane through buffer loads (256 bytes per
// instruction, four times the instructions, which the matrix work hides) into
// the same layout: A copy j of wave w fills the 4 rows of instruction index
// w + NW j, B copy j a quarter (256 bytes) of a k-row.  A lane whose element
// lies past M, N or K gets an out-of-range offset and writes a zero, so both
// operands are zero-filled at every edge and the epilogue masks its stores.
//
// Matrix instructions: lane (h, r32) feeds k = 8h + s in step s (s = 0..7) to
// A (row r32 of its block) and B (column r32) alike, so every instruction
// pairs matching k; its A values for steps 4q..4q+3 are one 16-byte read
// (chunk 2h + q), its B values single reads of four k-rows.
//
// Each panel is two halves of four steps with the barrier between them, as in
// the f16 ring: the first half multiplies fragments read before it while this
// wave reads the second half's and issues its copies; the wave waits for its
// copies of the next panel, passes the barrier, and the second half
// multiplies while the next panel's first fragments are read.
#include "f32_kernel.hpp"

namespace g355 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const f32x4 lds_f32x4c;
typedef __attribute__((address_space(3))) const float lds_f32c;

// NARROW: the masked copies of 4 bytes a lane (any shape and leading
// dimension); otherwise copies of 16 bytes a lane (whole tiles, or masked ones
// whose chunks of four lie wholly inside or outside the matrix).
template <int BM, int BN, int NS, int WM, int WN, bool NARROW>
struct F32RingShape {
    static constexpr int BK = 16;
    static constexpr int NW = WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 32, FN = TN / 32;
    static constexpr int A_BYTES = BM * BK * 4;      // rows of 64 bytes
    static constexpr int B_ROW = BN * 4 + 16;        // bytes per padded k-row
    static constexpr int STAGE = A_BYTES + BK * B_ROW;
    // copies per wave per panel: of 16 A rows and one B k-row (1 KB each), or
    // (masked) of 4 A rows and a quarter k-row (256 bytes each)
    static constexpr int A_INS = NARROW ? BM / 4 / NW : BM / 16 / NW;
    static constexpr int B_INS = NARROW ? 4 * BK / NW : BK / NW;
    static constexpr int FILLS = A_INS + B_INS;
    static_assert(BN == 256, "one k-row of B is 1 KB");
    static_assert(A_INS >= 1 && A_INS * NW * (NARROW ? 4 : 16) == BM &&
                      B_INS >= 1 && B_INS * NW == (NARROW ? 4 : 1) * BK,
                  "copies split evenly over the waves");
    static_assert(!NARROW || NW % 4 == 0, "masked copies: a wave's A swizzle and B quarter are fixed");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(NS >= 3 && NS * STAGE <= 160 * 1024, "LDS budget of one CU");
    static_assert((NS - 2) * FILLS < 64, "vmcnt range");
};

// MASKED with WIDE: 16-byte masked copies (16-byte aligned rows, N and K
// multiples of 4), which take a quarter of the 4-byte ones' instructions.
template <int BM, int BN, int NS, int WM, int WN, int GM, bool SK, bool MASKED, bool WIDE = false>
__global__ __launch_bounds__(WM * WN * 64) void gemm_f32_ring_kernel(F32Args p) {
    static_assert(!WIDE || MASKED, "16-byte masked copies are a masked form");
    using S = F32RingShape<BM, BN, NS, WM, WN, MASKED && !WIDE>;
    constexpr int FM = S::FM, FN = S::FN;
    __shared__ __attribute__((aligned(1024))) unsigned char ring[NS * S::STAGE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave / WN, wc = wave % WN;
    const int h = lane >> 5, r32 = lane & 31;
    const int nkt = (p.K + S::BK - 1) / S::BK;   // panels of a tile (the last one short when masked)

    // Work of this workgroup: one whole tile, or (stream-K) sk_dp whole tiles
    // and then the run of (tile, panel) units [u, u_end) of the remaining
    // tiles, workgroups numbered so that the runs of one XCD are consecutive.
    constexpr bool sk = SK;   // the host sets p.sk_q > 0 exactly for SK launches
    const int tiles = p.tiles_m * p.tiles_n;
    const int dp_tiles = sk ? p.sk_dp * gridDim.x : 0;
    int g = 0, u = 0, u_end = 0, r = 0;
    if constexpr (sk) {
        const int G = gridDim.x, xcd = blockIdx.x & 7, q8 = G >> 3, r8 = G & 7;
        g = xcd * q8 + (xcd < r8 ? xcd : r8) + (blockIdx.x >> 3);
        u = g * p.sk_q;
        u_end = min((tiles - dp_tiles) * nkt, u + p.sk_q);
    }

    auto stage_of = [&](int i) __attribute__((always_inline)) -> unsigned char* {
        return ring + i * S::STAGE;
    };
    const int sw = (r32 >> 2) & 3;
    const int a_off = (wr * S::TM + r32) * 64;
    const int b_off = S::A_BYTES + (8 * h) * S::B_ROW + (wc * S::TN + r32) * 4;
    const int arow = lane >> 2;
    const int achunk = (lane & 3) ^ ((arow >> 2) & 3);

    for (;;) {
        int tm, tn, kp0, nk;
        bool dp_item = false;
        if constexpr (!sk) {
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
        const int k_lo = kp0 * S::BK;

        // Copy sources.  A copy j of this wave fills panel rows 16 (wave + NW j)
        // .. +15 (bytes (wave + NW j) KB of the stage); lane l takes row l / 4
        // of them and position l % 4, which holds global chunk (l % 4) ^
        // swz(row); rows start at multiples of 16, so swz(row) = (l / 16) % 4.
        // B copy j fills k-row wave + NW j, lane l its floats 4l .. 4l + 3.
        const float* a_src = p.A + (int64_t)(m0 + wave * 16 + arow) * p.lda + k_lo + achunk * 4;
        const float* b_src = p.B + (int64_t)(k_lo + wave) * p.ldb + n0 + lane * 4;
        const int64_t a_step = (int64_t)S::NW * 16 * p.lda;   // next copy of this wave
        const int64_t b_step = (int64_t)S::NW * p.ldb;
        const int64_t b_panel = (int64_t)S::BK * p.ldb;
        // Masked copies: A copy j fills panel rows 4 (wave + NW j) .. +3, lane
        // l row 4 (wave + NW j) + l / 16 at word l % 16 of it, which holds k =
        // 4 ((l % 16) / 4 ^ swz) + l % 4 with swz = (wave + NW j) % 4 = wave % 4.
        // B copy j fills quarter wave % 4 of k-row wave / 4 + (NW / 4) j, lane
        // l its float 64 (wave % 4) + l.  Offsets are bytes from the panel's
        // first element (row m0, column n0, depth k of the panel).
        const int a_row = 4 * wave + (lane >> 4);
        const int a_kk = ((((lane & 15) >> 2) ^ (wave & 3)) << 2) | (lane & 3);
        const uint32_t a_voff = static_cast<uint32_t>(((int64_t)a_row * p.lda + a_kk) * 4);
        const uint32_t a_voff_step = static_cast<uint32_t>((int64_t)4 * S::NW * p.lda * 4);
        const int b_q = wave & 3, b_kr = wave >> 2;
        const bool b_col_in = n0 + 64 * b_q + lane < p.N;
        const uint32_t b_voff = static_cast<uint32_t>(((int64_t)b_kr * p.ldb + 64 * b_q + lane) * 4);
        const uint32_t b_voff_step = static_cast<uint32_t>((int64_t)(S::NW / 4) * p.ldb * 4);
        // 16-byte masked copies: the lanes and destinations of the unmasked
        // copies, a lane outside the matrix (row >= M, k >= K or columns >= N;
        // K and N multiples of 4, so a chunk is wholly in or out) reading zero.
        const uint32_t a16_voff = static_cast<uint32_t>(((int64_t)(wave * 16 + arow) * p.lda + achunk * 4) * 4);
        const uint32_t a16_step = static_cast<uint32_t>(a_step * 4);
        const bool b16_col_in = n0 + 4 * lane < p.N;
        const uint32_t b16_voff = static_cast<uint32_t>(((int64_t)wave * p.ldb + 4 * lane) * 4);
        const uint32_t b16_step = static_cast<uint32_t>(b_step * 4);
        auto fill = [&](unsigned char* stage, int kt) __attribute__((always_inline)) {
            const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(stage));
            if constexpr (WIDE) {
                const int kp = k_lo + kt * S::BK;
                const i32x4_rsrc ra = copy_rsrc(p.A + (int64_t)m0 * p.lda + kp);
                const bool a_k_in = kp + achunk * 4 < p.K;
#pragma unroll
                for (int j = 0; j < S::A_INS; ++j) {
                    const bool in = a_k_in && m0 + wave * 16 + arow + S::NW * 16 * j < p.M;
                    lds_copy16_masked(ra, in ? a16_voff + j * a16_step : kLdsCopyOut,
                                      base + (wave + S::NW * j) * 1024);
                }
                const i32x4_rsrc rb = copy_rsrc(p.B + (int64_t)kp * p.ldb + n0);
#pragma unroll
                for (int j = 0; j < S::B_INS; ++j) {
                    const bool in = b16_col_in && kp + wave + S::NW * j < p.K;
                    lds_copy16_masked(rb, in ? b16_voff + j * b16_step : kLdsCopyOut,
                                      base + S::A_BYTES + (wave + S::NW * j) * S::B_ROW);
                }
            } else if constexpr (MASKED) {
                const int kp = k_lo + kt * S::BK;
                const i32x4_rsrc ra = copy_rsrc(p.A + (int64_t)m0 * p.lda + kp);
                const bool a_k_in = kp + a_kk < p.K;
#pragma unroll
                for (int j = 0; j < S::A_INS; ++j) {
                    const bool in = a_k_in && m0 + a_row + 4 * S::NW * j < p.M;
                    lds_copy4_masked(ra, in ? a_voff + j * a_voff_step : kLdsCopyOut,
                                     base + (wave + S::NW * j) * 256);
                }
                const i32x4_rsrc rb = copy_rsrc(p.B + (int64_t)kp * p.ldb + n0);
#pragma unroll
                for (int j = 0; j < S::B_INS; ++j) {
                    const int kr = b_kr + (S::NW / 4) * j;
                    const bool in = b_col_in && kp + kr < p.K;
                    lds_copy4_masked(rb, in ? b_voff + j * b_voff_step : kLdsCopyOut,
                                     base + S::A_BYTES + kr * S::B_ROW + b_q * 256);
                }
            } else {
#pragma unroll
                for (int j = 0; j < S::A_INS; ++j)
                    lds_copy16(a_src + j * a_step + kt * S::BK, base + (wave + S::NW * j) * 1024);
#pragma unroll
                for (int j = 0; j < S::B_INS; ++j)
                    lds_copy16(b_src + j * b_step + kt * b_panel,
                               base + S::A_BYTES + (wave + S::NW * j) * S::B_ROW);
            }
        };

        // Fragments of half q (steps 4q .. 4q + 3): A block i one 16-byte read
        // at chunk 2h + q of its row; B block j four single reads at k-rows
        // 8h + 4q + t.
        f32x4 fa[2][FM];
        float fb[2][FN][4];
        auto frags = [&](const unsigned char* stage, int q) __attribute__((always_inline)) {
            const lds_u8* base = (const lds_u8*)(stage);
            const int chunk = ((2 * h + q) ^ sw) << 4;
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[q][i] = *reinterpret_cast<lds_f32x4c*>(base + a_off + i * 32 * 64 + chunk);
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    fb[q][j][t] = *reinterpret_cast<lds_f32c*>(base + b_off + (4 * q + t) * S::B_ROW +
                                                               j * 32 * 4);
        };

        f32x16 acc[FM][FN];
        auto mfmas = [&](int q, auto first) __attribute__((always_inline)) {
            const f32x16 zero = {};
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            fa[q][i][t], fb[q][j][t],
                            (decltype(first)::value && t == 0) ? zero : acc[i][j], 0, 0, 0);
        };
        constexpr int NMF = 4 * FM * FN;      // matrix instructions per half
        constexpr int NRD = FM + 4 * FN;      // fragment reads per half
        auto interleave = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int m = 0; m < NMF; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (m < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        };

        // One panel in `cur`: copy panel kt_fill into `freed` (the previous
        // panel's stage, which every wave finished reading before the last
        // barrier); first half beside the reads of the second half's
        // fragments; wait for this wave's copies of the next panel; barrier;
        // second half beside the reads of the next panel's first fragments.
        // Copies past the last panel reload the last one into a stage nobody
        // reads again, so the count of outstanding copies is the same every
        // panel.
        auto panel = [&](const unsigned char* cur, unsigned char* freed, const unsigned char* next,
                         int kt_fill, auto first) __attribute__((always_inline)) {
            fill(freed, kt_fill);
            frags(cur, 1);
            mfmas(0, first);
            __builtin_amdgcn_sched_group_barrier(0x020, S::FILLS, 0);
            interleave();
            wait_vmcnt<(NS - 2) * S::FILLS>();
            ring_barrier();
            frags(next, 0);
            mfmas(1, std::false_type{});
            interleave();
        };

#pragma unroll
        for (int i = 0; i + 1 < NS; ++i) fill(stage_of(i), min(i, nk - 1));
        wait_vmcnt<(NS - 2) * S::FILLS>();
        ring_barrier();
        frags(stage_of(0), 0);

        panel(stage_of(0), stage_of(NS - 1), stage_of(1), min(NS - 1, nk - 1), std::true_type{});
#pragma unroll
        for (int v = 1; v < NS; ++v)
            if (v < nk)
                panel(stage_of(v), stage_of(v - 1), stage_of((v + 1) % NS), min(v + NS - 1, nk - 1),
                      std::false_type{});
        for (int kt = NS; kt < nk; kt += NS) {
#pragma unroll
            for (int v = 0; v < NS; ++v)
                if (v == 0 || kt + v < nk)
                    panel(stage_of(v), stage_of((v + NS - 1) % NS), stage_of((v + 1) % NS),
                          min(kt + v + NS - 1, nk - 1), std::false_type{});
        }
        wait_vmcnt<0>();   // no copy may still be landing in LDS when the segment ends

        bool finish = true;
        if (sk && nk < nkt) {
            // A part of the tile: store the accumulators in register order
            // (16 floats per block and lane, four 16-byte device-scope
            // stores, each instruction of a wave one contiguous kilobyte) in
            // this workgroup's slot for the tile (0: the tile its run starts
            // in, 1: the tile it ends in), wait for them, pass a barrier and
            // count in.  The last workgroup of the tile to arrive reads every
            // part back and adds them in k order (part s comes from workgroup
            // g_first + s), so the sum does not depend on the arrival order.
            constexpr int kSC1 = 1 << 4;          // cache-policy bit of the buffer intrinsics
            constexpr int kRsrc = 0x00020000;     // raw buffer, 32-bit data format
            constexpr int NB = FM * FN;
            constexpr int TILE_BYTES = BM * BN * 4;
            const int t = u / nkt;
            const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
                p.P, (short)0, static_cast<int>((int64_t)gridDim.x * 2 * TILE_BYTES), kRsrc);
            auto slot_of = [&](int wg) { return (wg * p.sk_q) / nkt == t ? 0 : 1; };
            auto at = [&](int wg, int b, int q) {   // quarter q of block b of this lane
                return static_cast<int>(((int64_t)wg * 2 + slot_of(wg)) * TILE_BYTES +
                                        (((wave * NB + b) * 4 + q) * 64 + lane) * 16);
            };
            typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 v = {acc[b / FN][b % FN][4 * q], acc[b / FN][b % FN][4 * q + 1],
                                     acc[b / FN][b % FN][4 * q + 2], acc[b / FN][b % FN][4 * q + 3]};
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rp,
                                                           at(g, b, q), 0, kSC1);
                }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();   // every wave is past its last panel read and its stores are done
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
                // one block at a time, the loads of up to four parts (two for
                // the larger wave tiles, for registers) in flight together
                constexpr int ZG = NB >= 8 ? 2 : 4;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    for (int s0 = 0; s0 < parts; s0 += ZG) {
                        f32x4 tv[ZG][4];
#pragma unroll
                        for (int ss = 0; ss < ZG; ++ss) {
                            const int wg = g_first + min(s0 + ss, parts - 1);   // past the last: unused reload
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                tv[ss][q] = __builtin_bit_cast(
                                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, at(wg, b, q), 0, kSC1));
                        }
#pragma unroll
                        for (int ss = 0; ss < ZG; ++ss) {
                            if (s0 + ss >= parts) break;
#pragma unroll
                            for (int e = 0; e < 16; ++e) {
                                const float a = acc[b / FN][b % FN][e];
                                acc[b / FN][b % FN][e] =
                                    s0 + ss == 0 ? tv[ss][e / 4][e % 4] : a + tv[ss][e / 4][e % 4];
                            }
                        }
                    }
                }
            }
        }
        if (finish)
            store_tile<FM, FN, MASKED>(acc, p.C, p.ldc, m0 + wr * S::TM, n0 + wc * S::TN, p.M, p.N,
                                       p.alpha, p.beta, lane);
        if constexpr (!sk) break;
        if (dp_item) ++r;
        else u += nk;
        ring_barrier();   // every wave is done with the ring before the next run refills it
    }
}

}  // namespace

// The ring handles the plain layout: whole tiles with 16-byte aligned rows
// and K a multiple of 16 in the unmasked form, any other shape in the masked
// form while the copies' byte offsets within a panel (BM rows of A, 16
// k-rows of B) stay below 2^30; transposed operands and split-K slices run
// the register-staged kernel with the same BM x BN tile (BK = 16, 2 x 2
// waves).
namespace {
bool ring_plain(const F32Args& a, const F32Variant& v) {
    return !v.ta && !v.tb && a.ksplit == 0 && !v.r16 && a.M > 0 && a.N > 0 && a.K > 0;
}
bool ring_whole(int bm, int bn, const F32Args& a, const F32Variant& v) {
    return ring_plain(a, v) && !v.masked && v.vec && a.M % bm == 0 && a.N % bn == 0 &&
           a.K % 16 == 0;
}
bool ring_masked(int bm, const F32Args& a, const F32Variant& v) {
    return ring_plain(a, v) && int64_t{bm} * a.lda < (int64_t{1} << 28) &&
           int64_t{16} * a.ldb < (int64_t{1} << 28);
}
}  // namespace

bool f32_ring_takes(const TileConfig& cfg, const F32Args& a, const F32Variant& v) {
    return ring_whole(cfg.bm, cfg.bn, a, v) || ring_masked(cfg.bm, a, v);
}

template <int BM, int BN, int NS, int WM, int WN, int GM, bool MASKED, bool WIDE = false>
hipError_t launch_ring_form(const F32Args& a, hipStream_t s) {
    const dim3 block(WM * WN * 64);
    if (a.sk_q > 0) {
        const int grid = ring_sk_grid(int64_t{a.tiles_m} * a.tiles_n, (a.K + 15) / 16, a.sk_q,
                                      a.sk_dp, a.sk_grid, a.P, a.counts);
        if (grid <= 0) return hipErrorInvalidValue;
        gemm_f32_ring_kernel<BM, BN, NS, WM, WN, GM, true, MASKED, WIDE><<<dim3(grid), block, 0, s>>>(a);
    } else {
        gemm_f32_ring_kernel<BM, BN, NS, WM, WN, GM, false, MASKED, WIDE>
            <<<dim3(static_cast<unsigned>(a.tiles_m * a.tiles_n)), block, 0, s>>>(a);
    }
    return hipGetLastError();
}

template <int BM, int BN, int NS, int WM, int WN, int GM>
hipError_t launch_f32_ring(const F32Args& a, F32Variant v, hipStream_t s) {
    if (ring_whole(BM, BN, a, v)) return launch_ring_form<BM, BN, NS, WM, WN, GM, false>(a, s);
    if (ring_masked(BM, a, v)) {
        // 16-byte chunks lie wholly inside or outside the matrix
        if (v.vec && a.N % 4 == 0 && a.K % 4 == 0)
            return launch_ring_form<BM, BN, NS, WM, WN, GM, true, true>(a, s);
        return launch_ring_form<BM, BN, NS, WM, WN, GM, true>(a, s);
    }
    if (v.ta || v.tb) return launch_f32_transposed<BM, BN, 16, 2, 2, GM>(a, v, s);
    return launch_f32_layout<BM, BN, 16, 2, 2, GM, false, false>(a, v, s);
}

#define G355_F32_RING_INSTANTIATE(BM, BN, NS, WM, WN, GM) \
    template hipError_t launch_f32_ring<BM, BN, NS, WM, WN, GM>(const F32Args&, F32Variant, hipStream_t);
G355_F32_RING_CONFIGS(G355_F32_RING_INSTANTIATE)

}  // namespace g355
