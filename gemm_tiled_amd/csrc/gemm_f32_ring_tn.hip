// gemm_f32_ring_tn.hip -- the f32 ring kernels (f32_ring.hpp) of the TN
// operand layout: op(A) = A^T (A stored K x M), B as stored.
#include "f32_ring.hpp"

namespace g355 {

#define G355_F32_RING_TN(BM, BN, NS, WM, WN, GM)                                      \
    template hipError_t launch_ring_layout<BM, BN, NS, WM, WN, GM, true, false>(const F32Args&, \
                                                                              RingForm,       \
                                                                              hipStream_t);
G355_F32_RING_CONFIGS(G355_F32_RING_TN)

}  // namespace g355
