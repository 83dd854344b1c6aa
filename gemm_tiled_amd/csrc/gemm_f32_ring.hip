// gemm_f32_ring.hip -- which calls the f32 ring takes, in which form, and the
// ring kernels of the plain layout (A and B as stored); the kernel itself is
// in f32_ring.hpp, the transposed layouts' instances in gemm_f32_ring_tn.hip,
// gemm_f32_ring_nt.hip and gemm_f32_ring_tt.hip.
#include "f32_ring.hpp"

namespace g355 {

// The ring takes a call in any operand layout: whole tiles with 16-byte
// aligned rows and K a multiple of 16 in the unmasked form, any other shape in
// the masked forms while the copies' byte offsets within a panel (BM or BN
// stored rows of the rows layout, 16 k-rows of the k-rows layout) stay below
// 2^30.  The 16-byte masked copies need 16-byte aligned rows and, along each
// operand's contiguous dimension, a multiple of 4 elements, so that every
// chunk lies wholly inside or outside the matrix.  Split-K slices and calls
// past those offsets run the register-staged kernel with the same BM x BN
// tile (BK = 16, 2 x 2 waves).
namespace {
bool ring_plain(const F32Args& a, const F32Variant& v) {
    return a.ksplit == 0 && !v.r16 && a.M > 0 && a.N > 0 && a.K > 0;
}
bool ring_whole(int bm, int bn, const F32Args& a, const F32Variant& v) {
    return ring_plain(a, v) && !v.masked && v.vec && a.M % bm == 0 && a.N % bn == 0 &&
           a.K % 16 == 0;
}
bool ring_masked(int bm, int bn, const F32Args& a, const F32Variant& v) {
    const int64_t a_rows = v.ta ? 16 : bm, b_rows = v.tb ? bn : 16;   // stored rows of a panel
    return ring_plain(a, v) && a_rows * a.lda < (int64_t{1} << 28) &&
           b_rows * a.ldb < (int64_t{1} << 28);
}
bool ring_wide(const F32Args& a, const F32Variant& v) {
    const int a_run = v.ta ? a.M : a.K, b_run = v.tb ? a.K : a.N;   // contiguous extents
    return v.vec && a_run % 4 == 0 && b_run % 4 == 0;
}
}  // namespace

bool f32_ring_takes(const TileConfig& cfg, const F32Args& a, const F32Variant& v) {
    return ring_whole(cfg.bm, cfg.bn, a, v) || ring_masked(cfg.bm, cfg.bn, a, v);
}

// the transposed layouts' instances live in their own translation units
#define G355_F32_RING_EXTERN_ONE(BM, BN, NS, WM, WN, GM, TA, TB) \
    extern template hipError_t launch_ring_layout<BM, BN, NS, WM, WN, GM, TA, TB>(const F32Args&, RingForm, hipStream_t);
#define G355_F32_RING_EXTERN(BM, BN, NS, WM, WN, GM)                 \
    G355_F32_RING_EXTERN_ONE(BM, BN, NS, WM, WN, GM, true, false)    \
    G355_F32_RING_EXTERN_ONE(BM, BN, NS, WM, WN, GM, false, true)    \
    G355_F32_RING_EXTERN_ONE(BM, BN, NS, WM, WN, GM, true, true)
G355_F32_RING_CONFIGS(G355_F32_RING_EXTERN)

template <int BM, int BN, int NS, int WM, int WN, int GM>
hipError_t launch_f32_ring(const F32Args& a, F32Variant v, hipStream_t s) {
    RingForm form;
    if (ring_whole(BM, BN, a, v)) form = RingForm::Whole;
    else if (ring_masked(BM, BN, a, v)) form = ring_wide(a, v) ? RingForm::Wide : RingForm::Narrow;
    else if (v.ta || v.tb) return launch_f32_transposed<BM, BN, 16, 2, 2, GM>(a, v, s);
    else return launch_f32_layout<BM, BN, 16, 2, 2, GM, false, false>(a, v, s);
    if (v.ta && v.tb) return launch_ring_layout<BM, BN, NS, WM, WN, GM, true, true>(a, form, s);
    if (v.ta) return launch_ring_layout<BM, BN, NS, WM, WN, GM, true, false>(a, form, s);
    if (v.tb) return launch_ring_layout<BM, BN, NS, WM, WN, GM, false, true>(a, form, s);
    return launch_ring_layout<BM, BN, NS, WM, WN, GM, false, false>(a, form, s);
}

#define G355_F32_RING_INSTANTIATE(BM, BN, NS, WM, WN, GM)                                          \
    template hipError_t launch_ring_layout<BM, BN, NS, WM, WN, GM, false, false>(const F32Args&,  \
                                                                                RingForm,         \
                                                                                hipStream_t);     \
    template hipError_t launch_f32_ring<BM, BN, NS, WM, WN, GM>(const F32Args&, F32Variant, hipStream_t);
G355_F32_RING_CONFIGS(G355_F32_RING_INSTANTIATE)

}  // namespace g355
