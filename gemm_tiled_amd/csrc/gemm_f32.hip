// gemm_f32.hip -- C = alpha*op(A)@op(B) + beta*C on f32, contracted on the
// gfx950 matrix cores (v_mfma_f32_32x32x2_f32, full f32 precision).  The
// kernel template is in f32_kernel.hpp; this unit compiles the plain layout
// (op = identity) and holds the table of configurations, whose launches hand
// the transposed layouts to gemm_f32_t.hip.
#include "f32_kernel.hpp"

namespace g355 {
namespace {

template <int BM, int BN, int BK, int WM, int WN, int GM>
hipError_t launch_f32(const F32Args& a, F32Variant v, hipStream_t s) {
    if (v.ta || v.tb) return launch_f32_transposed<BM, BN, BK, WM, WN, GM>(a, v, s);
    return launch_f32_layout<BM, BN, BK, WM, WN, GM, false, false>(a, v, s);
}

#define G355_F32_INSTANCE(BM, BN, BK, WM, WN, GM) \
    {{GEMM355_MODE_F32, BM, BN, BK, 2, WM, WN, GM}, &launch_f32<BM, BN, BK, WM, WN, GM>},

#define G355_F32_RING_INSTANCE(BM, BN, NS, WM, WN, GM) \
    {{GEMM355_MODE_F32, BM, BN, 16, NS, WM, WN, GM}, &launch_f32_ring<BM, BN, NS, WM, WN, GM>},

// The rings come first: the heuristic takes the first of equally priced
// tiles, and a ring configuration runs the register-staged kernel of its tile
// wherever the ring does not apply.
const F32Instance kF32Instances[] = {G355_F32_RING_CONFIGS(G355_F32_RING_INSTANCE)
                                         G355_F32_CONFIGS(G355_F32_INSTANCE)};

}  // namespace

const F32Instance* f32_instances(int* count) {
    *count = static_cast<int>(sizeof(kF32Instances) / sizeof(kF32Instances[0]));
    return kF32Instances;
}

}  // namespace g355
