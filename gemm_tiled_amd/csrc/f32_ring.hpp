// f32_ring.hpp -- the f32 GEMM on a ring of direct-to-LDS panels, in every
// operand layout: whole tiles with 16-byte aligned rows, or (the masked forms)
// any shape and any leading dimensions.  Shared by the translation units of
// the four layouts (gemm_f32_ring.hip for A and B as stored, and
// gemm_f32_ring_tn.hip, _nt.hip, _tt.hip); not part of the public ABI.
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
// A panel holds BK = 16 floats of k for the EXT elements of the tile's extent
// of its operand (EXT = BM rows of op(A), BN columns of op(B)), in one of two
// layouts, by the direction in which k runs in the operand's memory (the
// Matrix Multiplication lab's layout study: each operand copied along its
// contiguous dimension and kept in that orientation):
//   rows (k along the stored rows: A as stored, B transposed): EXT rows of 64
//      bytes (four 16-byte chunks of 4 k); chunk c of row r sits at position
//      c ^ ((r / 4) % 4), so the 16 lanes that read one chunk of 16
//      consecutive rows hit 16 different bank groups.  A copy instruction
//      fills 16 rows; lane l fetches the global chunk that belongs at its
//      destination position.  The matrix instructions take four k of a row
//      in one 16-byte read.
//   k-rows (k down the stored rows: B as stored, A transposed): 16 k-rows of
//      EXT floats.  A copy instruction fills 256 / EXT k-rows; such groups
//      lie 1 KB + PAD apart, PAD (16 bytes for groups of one k-row, 32 for
//      two) putting k-rows 8 apart, which the two lane halves read together,
//      in opposite halves of the 64 banks.  The matrix instructions take one
//      k per read.
// The masked forms copy 4 bytes a lane through buffer loads (256 bytes per
// instruction: 4 rows, or a quarter or half k-row; four times the
// instructions, which the matrix work hides) into the same layouts, or 16
// bytes a lane with the lanes and destinations of the whole-tile copies where
// every 16-byte chunk lies wholly inside or outside the matrix.  A lane whose
// element lies past M, N or K gets an out-of-range offset and writes a zero,
// so both operands are zero-filled at every edge and the epilogue masks its
// stores.
//
// Matrix instructions: lane (h, r32) feeds k = 8h + s in step s (s = 0..7) to
// A (row r32 of its block) and B (column r32) alike, so every instruction
// pairs matching k; its values for steps 4q..4q+3 come from one 16-byte read
// (rows layout, chunk 2h + q) or four single reads of k-rows 8h + 4q + t.
//
// Each panel is two halves of four steps with the barrier between them, as in
// the f16 ring: the first half multiplies fragments read before it while this
// wave reads the second half's and issues its copies; the wave waits for its
// copies of the next panel, passes the barrier, and the second half
// multiplies while the next panel's first fragments are read.
#pragma once

#include <type_traits>

#include "f32_kernel.hpp"

namespace g355 {

// How the ring takes a call: whole tiles with plain 16-byte copies, or the
// masked copies of 16 or 4 bytes a lane.
enum class RingForm { Whole, Wide, Narrow };

// One layout of one ring configuration (TA: op(A) = A^T, A stored K x M; TB:
// op(B) = B^T, B stored N x K), explicitly instantiated per layout.
template <int BM, int BN, int NS, int WM, int WN, int GM, bool TA, bool TB>
hipError_t launch_ring_layout(const F32Args& a, RingForm form, hipStream_t s);

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const f32x4 lds_f32x4c;
typedef __attribute__((address_space(3))) const float lds_f32c;

// One operand's panel in LDS: EXT elements of the tile's extent by 16 of k, in
// the rows layout (KROWS false) or the k-rows layout.
template <int EXT, bool KROWS>
struct RingPanel {
    static_assert(EXT == 128 || EXT == 256, "panel extent");
    static constexpr int RPI = KROWS ? 256 / EXT : 16;   // rows (k-rows) one 1 KB copy fills
    static constexpr int GROUP = KROWS ? (RPI == 1 ? 1024 + 16 : 1024 + 32) : 1024;
    static constexpr int BYTES = KROWS ? (16 / RPI) * GROUP : EXT * 64;
    static constexpr int PARTS = EXT / 64;               // 256-byte copies per k-row
    // byte offset of element e of k-row kr (k-rows layout)
    static constexpr int at(int kr, int e) {
        return (kr / RPI) * GROUP + (kr % RPI) * EXT * 4 + e * 4;
    }
};

template <int BM, int BN, int NS, int WM, int WN, bool NARROW, bool TA, bool TB>
struct F32RingShape {
    static constexpr int BK = 16;
    static constexpr int NW = WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 32, FN = TN / 32;
    using PA = RingPanel<BM, TA>;     // A in k-rows when transposed
    using PB = RingPanel<BN, !TB>;    // B in k-rows as stored
    static constexpr int A_BYTES = PA::BYTES;
    static constexpr int STAGE = PA::BYTES + PB::BYTES;
    // copies per wave per panel: of 1 KB (16 rows or 256 / EXT k-rows) or,
    // masked, of 256 bytes (4 rows or 64 floats of a k-row)
    static constexpr int A_INS = (NARROW ? BM / 4 : BM / 16) / NW;
    static constexpr int B_INS = (NARROW ? BN / 4 : BN / 16) / NW;
    static constexpr int FILLS = A_INS + B_INS;
    static_assert(A_INS >= 1 && A_INS * NW * (NARROW ? 4 : 16) == BM &&
                      B_INS >= 1 && B_INS * NW * (NARROW ? 4 : 16) == BN,
                  "copies split evenly over the waves");
    static_assert(!NARROW || NW % 4 == 0, "masked copies: a wave's swizzle and k-row part are fixed");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(NS >= 3 && NS * STAGE <= 160 * 1024, "LDS budget of one CU");
    static_assert((NS - 2) * FILLS < 64, "vmcnt range");
};

// Where copy j of a wave puts this lane's element: element e0 + j e_j of the
// extent at depth k0 + j k_j of the panel, the instruction's LDS destination
// dst0 + j dst_j bytes into the operand's part of the stage.
struct RingCopyLane {
    int e0, k0, e_j, k_j, dst0, dst_j;
};
template <int EXT, bool KROWS, int NW, bool NARROW>
__device__ __forceinline__ RingCopyLane ring_copy_lane(int wave, int lane) {
    using P = RingPanel<EXT, KROWS>;
    RingCopyLane c{};
    if constexpr (!KROWS && !NARROW) {
        // copy n = wave + NW j fills rows 16 n .. +15; lane l takes row l / 4
        // of them at position l % 4, which holds global chunk (l % 4) ^
        // swz(row); rows start at multiples of 16, so swz(row) = (l / 16) % 4
        c.e0 = 16 * wave + (lane >> 2);
        c.k0 = ((lane & 3) ^ ((lane >> 4) & 3)) << 2;
        c.e_j = 16 * NW;
        c.dst0 = wave * 1024;
        c.dst_j = NW * 1024;
    } else if constexpr (!KROWS) {
        // copy n fills rows 4 n .. +3: lane l row 4 n + l / 16 at word l % 16,
        // which holds k = 4 ((l % 16) / 4 ^ swz) + l % 4, swz = n % 4 = wave % 4
        c.e0 = 4 * wave + (lane >> 4);
        c.k0 = ((((lane & 15) >> 2) ^ (wave & 3)) << 2) | (lane & 3);
        c.e_j = 4 * NW;
        c.dst0 = wave * 256;
        c.dst_j = NW * 256;
    } else if constexpr (!NARROW) {
        // copy n fills k-rows RPI n .. +RPI-1, lane l floats 4 (l % LPR) .. +3
        // of k-row RPI n + l / LPR (LPR lanes a k-row)
        constexpr int LPR = 64 / P::RPI;
        c.e0 = 4 * (lane % LPR);
        c.k0 = P::RPI * wave + lane / LPR;
        c.k_j = P::RPI * NW;
        c.dst0 = wave * P::GROUP;
        c.dst_j = NW * P::GROUP;
    } else {
        // copy n fills part n % PARTS (64 floats) of k-row n / PARTS, lane l its
        // float 64 part + l; part = wave % PARTS
        constexpr int PARTS = P::PARTS;
        static_assert(NW % PARTS == 0 && (NW / PARTS) % P::RPI == 0, "a wave's part is fixed");
        const int part = wave % PARTS;
        c.e0 = 64 * part + lane;
        c.k0 = wave / PARTS;
        c.k_j = NW / PARTS;
        c.dst0 = P::at(wave / PARTS, 64 * part);
        c.dst_j = (NW / PARTS / P::RPI) * P::GROUP;
    }
    return c;
}

// MASKED with WIDE: 16-byte masked copies (16-byte aligned rows, and along
// each operand's contiguous dimension a multiple of 4 elements), which take a
// quarter of the 4-byte ones' instructions.
template <int BM, int BN, int NS, int WM, int WN, int GM, bool SK, bool MASKED, bool WIDE, bool TA,
          bool TB>
__global__ __launch_bounds__(WM * WN * 64) void gemm_f32_ring_kernel(F32Args p) {
    static_assert(!WIDE || MASKED, "16-byte masked copies are a masked form");
    constexpr bool NARROW = MASKED && !WIDE;
    using S = F32RingShape<BM, BN, NS, WM, WN, NARROW, TA, TB>;
    using PA = typename S::PA;
    using PB = typename S::PB;
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
    // Fragment reads: rows layout at row (wave's offset + r32) and chunk
    // 2h + q (swizzled by sw); k-rows layout at k-rows 8h + 4q + t.
    const int sw = (r32 >> 2) & 3;
    const int a_frag = TA ? h * (8 / PA::RPI) * PA::GROUP + (wr * S::TM + r32) * 4
                          : (wr * S::TM + r32) * 64;
    const int b_frag = S::A_BYTES + (TB ? (wc * S::TN + r32) * 64
                                        : h * (8 / PB::RPI) * PB::GROUP + (wc * S::TN + r32) * 4);
    // This lane's copies: element offsets from the panel's corner (the
    // operand's first element of the tile at the panel's depth) of copy 0,
    // and their advance per copy; stored A is A[e * lda + k] (rows) or A[k *
    // lda + e] (k-rows), B likewise with ldb.
    const RingCopyLane ca = ring_copy_lane<BM, TA, S::NW, NARROW>(wave, lane);
    const RingCopyLane cb = ring_copy_lane<BN, !TB, S::NW, NARROW>(wave, lane);
    const int64_t a_off = TA ? (int64_t)ca.k0 * p.lda + ca.e0 : (int64_t)ca.e0 * p.lda + ca.k0;
    const int64_t a_offj = TA ? (int64_t)ca.k_j * p.lda + ca.e_j : (int64_t)ca.e_j * p.lda + ca.k_j;
    const int64_t b_off = TB ? (int64_t)cb.e0 * p.ldb + cb.k0 : (int64_t)cb.k0 * p.ldb + cb.e0;
    const int64_t b_offj = TB ? (int64_t)cb.e_j * p.ldb + cb.k_j : (int64_t)cb.k_j * p.ldb + cb.e_j;
    // corner advance per panel (16 of k)
    const int64_t a_panel = TA ? (int64_t)S::BK * p.lda : S::BK;
    const int64_t b_panel = TB ? S::BK : (int64_t)S::BK * p.ldb;
    // masked copies: byte offsets (below 2^30: the host bounds the leading
    // dimensions)
    const uint32_t a_voff = static_cast<uint32_t>(a_off * 4), a_voffj = static_cast<uint32_t>(a_offj * 4);
    const uint32_t b_voff = static_cast<uint32_t>(b_off * 4), b_voffj = static_cast<uint32_t>(b_offj * 4);

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

        // the panels' corners at depth k_lo
        const float* a_corner = TA ? p.A + (int64_t)k_lo * p.lda + m0 : p.A + (int64_t)m0 * p.lda + k_lo;
        const float* b_corner = TB ? p.B + (int64_t)n0 * p.ldb + k_lo : p.B + (int64_t)k_lo * p.ldb + n0;
        const float* a_src = a_corner + a_off;
        const float* b_src = b_corner + b_off;
        auto fill = [&](unsigned char* stage, int kt) __attribute__((always_inline)) {
            const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(stage));
            if constexpr (MASKED) {
                const int kp = k_lo + kt * S::BK;
                const i32x4_rsrc ra = copy_rsrc(a_corner + kt * a_panel);
#pragma unroll
                for (int j = 0; j < S::A_INS; ++j) {
                    const bool in = m0 + ca.e0 + j * ca.e_j < p.M && kp + ca.k0 + j * ca.k_j < p.K;
                    const uint32_t voff = in ? a_voff + j * a_voffj : kLdsCopyOut;
                    if constexpr (WIDE) lds_copy16_masked(ra, voff, base + ca.dst0 + j * ca.dst_j);
                    else lds_copy4_masked(ra, voff, base + ca.dst0 + j * ca.dst_j);
                }
                const i32x4_rsrc rb = copy_rsrc(b_corner + kt * b_panel);
#pragma unroll
                for (int j = 0; j < S::B_INS; ++j) {
                    const bool in = n0 + cb.e0 + j * cb.e_j < p.N && kp + cb.k0 + j * cb.k_j < p.K;
                    const uint32_t voff = in ? b_voff + j * b_voffj : kLdsCopyOut;
                    const uint32_t dst = base + S::A_BYTES + cb.dst0 + j * cb.dst_j;
                    if constexpr (WIDE) lds_copy16_masked(rb, voff, dst);
                    else lds_copy4_masked(rb, voff, dst);
                }
            } else {
#pragma unroll
                for (int j = 0; j < S::A_INS; ++j)
                    lds_copy16(a_src + j * a_offj + kt * a_panel, base + ca.dst0 + j * ca.dst_j);
#pragma unroll
                for (int j = 0; j < S::B_INS; ++j)
                    lds_copy16(b_src + j * b_offj + kt * b_panel,
                               base + S::A_BYTES + cb.dst0 + j * cb.dst_j);
            }
        };

        // Fragments of half q (steps 4q .. 4q + 3) of each 32-block: one
        // 16-byte read (rows layout) or four single reads (k-rows layout).
        std::conditional_t<TA, float[4], f32x4> fa[2][FM];
        std::conditional_t<TB, f32x4, float[4]> fb[2][FN];
        auto frags = [&](const unsigned char* stage, int q) __attribute__((always_inline)) {
            const lds_u8* base = (const lds_u8*)(stage);
            const int chunk = ((2 * h + q) ^ sw) << 4;
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                if constexpr (TA) {
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        fa[q][i][t] = *reinterpret_cast<lds_f32c*>(base + a_frag + PA::at(4 * q + t, 32 * i));
                } else {
                    fa[q][i] = *reinterpret_cast<lds_f32x4c*>(base + a_frag + i * 32 * 64 + chunk);
                }
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                if constexpr (TB) {
                    fb[q][j] = *reinterpret_cast<lds_f32x4c*>(base + b_frag + j * 32 * 64 + chunk);
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        fb[q][j][t] = *reinterpret_cast<lds_f32c*>(base + b_frag + PB::at(4 * q + t, 32 * j));
                }
            }
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
        constexpr int NRD = (TA ? 4 * FM : FM) + (TB ? FN : 4 * FN);   // fragment reads per half
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

template <int BM, int BN, int NS, int WM, int WN, int GM, bool MASKED, bool WIDE, bool TA, bool TB>
hipError_t launch_ring_form(const F32Args& a, hipStream_t s) {
    const dim3 block(WM * WN * 64);
    if (a.sk_q > 0) {
        const int grid = ring_sk_grid(int64_t{a.tiles_m} * a.tiles_n, (a.K + 15) / 16, a.sk_q,
                                      a.sk_dp, a.sk_grid, a.P, a.counts);
        if (grid <= 0) return hipErrorInvalidValue;
        gemm_f32_ring_kernel<BM, BN, NS, WM, WN, GM, true, MASKED, WIDE, TA, TB>
            <<<dim3(grid), block, 0, s>>>(a);
    } else {
        gemm_f32_ring_kernel<BM, BN, NS, WM, WN, GM, false, MASKED, WIDE, TA, TB>
            <<<dim3(static_cast<unsigned>(a.tiles_m * a.tiles_n)), block, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace

template <int BM, int BN, int NS, int WM, int WN, int GM, bool TA, bool TB>
hipError_t launch_ring_layout(const F32Args& a, RingForm form, hipStream_t s) {
    switch (form) {
        case RingForm::Whole:
            return launch_ring_form<BM, BN, NS, WM, WN, GM, false, false, TA, TB>(a, s);
        case RingForm::Wide:
            return launch_ring_form<BM, BN, NS, WM, WN, GM, true, true, TA, TB>(a, s);
        case RingForm::Narrow:
            return launch_ring_form<BM, BN, NS, WM, WN, GM, true, false, TA, TB>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace g355
