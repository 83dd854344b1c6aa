// gemm_f32_ring_tt.hip -- the f32 ring kernels (f32_ring.hpp) of the TT
// operand layout: op(A) = A^T and op(B) = B^T.
#include "f32_ring.hpp"

namespace g355 {

#define G355_F32_RING_TT(BM, BN, NS, WM, WN, GM)                                      \
    template hipError_t launch_ring_layout<BM, BN, NS, WM, WN, GM, true, true>(const F32Args&, \
                                                                              RingForm,       \
                                                                              hipStream_t);
G355_F32_RING_CONFIGS(G355_F32_RING_TT)

}  // namespace g355
