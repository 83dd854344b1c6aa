// gemm_splitk.hip -- the split-K configuration for few rows of C.
//
// With M small (the lab's skinny shapes, "Part 5": M from 1 to a few hundred
// at K = N = 4096) the tiles of C are too few to occupy 256 CUs and the time
// goes into streaming B from memory.  This configuration multiplies 32 x 128
// tiles, one 32 x 32 block per wave, over slices of K: slice z of every tile
// is its own workgroup (blockIdx.y = z) and stores its partial tile; a second
// pass adds the slices in order z = 0, 1, ... and applies alpha and beta, so
// the result does not depend on scheduling.  In the f16r mode the operands are
// rounded to binary16 as they are staged (no packing pass: B is read once).
#include "f32_kernel.hpp"

namespace g355 {
namespace {

constexpr int kBM = 32, kBN = 128, kBK = 32, kWM = 1, kWN = 4, kGM = 8;

template <bool SPLIT, bool R16, bool TA, bool TB>
hipError_t launch_layout(const F32Args& a, F32Variant v, hipStream_t s, dim3 grid) {
    const dim3 block(kWM * kWN * 64);
    if (!v.masked)
        gemm_f32_kernel<kBM, kBN, kBK, kWM, kWN, kGM, false, true, TA, TB, SPLIT, R16>
            <<<grid, block, 0, s>>>(a);
    else if (v.vec)
        gemm_f32_kernel<kBM, kBN, kBK, kWM, kWN, kGM, true, true, TA, TB, SPLIT, R16>
            <<<grid, block, 0, s>>>(a);
    else
        gemm_f32_kernel<kBM, kBN, kBK, kWM, kWN, kGM, true, false, TA, TB, SPLIT, R16>
            <<<grid, block, 0, s>>>(a);
    return hipGetLastError();
}

template <bool SPLIT, bool R16>
hipError_t launch_rounding(const F32Args& a, F32Variant v, hipStream_t s, dim3 grid) {
    if (v.ta && v.tb) return launch_layout<SPLIT, R16, true, true>(a, v, s, grid);
    if (v.ta) return launch_layout<SPLIT, R16, true, false>(a, v, s, grid);
    if (v.tb) return launch_layout<SPLIT, R16, false, true>(a, v, s, grid);
    return launch_layout<SPLIT, R16, false, false>(a, v, s, grid);
}

}  // namespace

TileConfig splitk_config(int mode) {
    TileConfig c{mode, kBM, kBN, kBK, 2, kWM, kWN, kGM};
    c.ks = 1;
    return c;
}

// a.ksplit == 0: one slice, the normal epilogue into C.  Otherwise the
// partial tiles of ceil(K / ksplit) slices go to a.C (dense M x N slices).
hipError_t launch_f32_splitk(const F32Args& a, F32Variant v, hipStream_t s) {
    const int slices = a.ksplit > 0 ? (a.K + a.ksplit - 1) / a.ksplit : 1;
    if (a.ksplit > 0 && a.ksplit % kBK != 0) return hipErrorInvalidValue;
    const dim3 grid(a.tiles_m * a.tiles_n, slices);
    if (a.ksplit > 0)
        return v.r16 ? launch_rounding<true, true>(a, v, s, grid)
                     : launch_rounding<true, false>(a, v, s, grid);
    return v.r16 ? launch_rounding<false, true>(a, v, s, grid)
                 : launch_rounding<false, false>(a, v, s, grid);
}

}  // namespace g355
