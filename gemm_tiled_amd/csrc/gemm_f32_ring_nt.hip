// gemm_f32_ring_nt.hip -- the f32 ring kernels (f32_ring.hpp) of the NT
// operand layout: A as stored, op(B) = B^T (B stored N x K).
#include "f32_ring.hpp"

namespace g355 {

#define G355_F32_RING_NT(BM, BN, NS, WM, WN, GM)                                      \
    template hipError_t launch_ring_layout<BM, BN, NS, WM, WN, GM, false, true>(const F32Args&, \
                                                                              RingForm,       \
                                                                              hipStream_t);
G355_F32_RING_CONFIGS(G355_F32_RING_NT)

}  // namespace g355
