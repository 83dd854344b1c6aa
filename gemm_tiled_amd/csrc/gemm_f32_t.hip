// gemm_f32_t.hip -- the transposed operand layouts of the f32 GEMM (op(A) =
// A^T and/or op(B) = B^T, the BLAS transa/transb of the Matrix Multiplication
// lab's layout study), compiled apart from the plain layout so the two units
// build in parallel.
#include "f32_kernel.hpp"

namespace g355 {

template <int BM, int BN, int BK, int WM, int WN, int GM>
hipError_t launch_f32_transposed(const F32Args& a, F32Variant v, hipStream_t s) {
    if (v.ta && v.tb) return launch_f32_layout<BM, BN, BK, WM, WN, GM, true, true>(a, v, s);
    if (v.ta) return launch_f32_layout<BM, BN, BK, WM, WN, GM, true, false>(a, v, s);
    return launch_f32_layout<BM, BN, BK, WM, WN, GM, false, true>(a, v, s);
}

#define G355_F32_TRANSPOSED(BM, BN, BK, WM, WN, GM)                                     \
    template hipError_t launch_f32_transposed<BM, BN, BK, WM, WN, GM>(const F32Args&, \
                                                                     F32Variant, hipStream_t);
G355_F32_CONFIGS(G355_F32_TRANSPOSED)

}  // namespace g355
