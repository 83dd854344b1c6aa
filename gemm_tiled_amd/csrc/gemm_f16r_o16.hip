// gemm_f16r_o16.hip -- the binary16-output launches of the f16 GEMM
// configurations (the f16-output variant of the f16r mode: C stored as
// binary16, the f32 epilogue value rounded to nearest even), compiled apart
// from the f32-output launches so the two units build in parallel.
#include "f16_kernel.hpp"

namespace g355 {

template <int BM, int BN, int NS, int WM, int WN, int GM>
hipError_t launch_f16_ring_o16(const F16Args& a, hipStream_t s) {
    return launch_f16_ring_out<BM, BN, NS, WM, WN, GM, true>(a, s);
}

template <int BM, int BN, int ST, int WM, int WN, int GM, bool RS>
hipError_t launch_f16_o16(const F16Args& a, hipStream_t s) {
    return launch_f16_out<BM, BN, ST, WM, WN, GM, RS, true>(a, s);
}

#define G355_F16_RING_O16(BM, BN, NS, WM, WN, GM) \
    template hipError_t launch_f16_ring_o16<BM, BN, NS, WM, WN, GM>(const F16Args&, hipStream_t);
#define G355_F16_PANEL_O16(BM, BN, ST, WM, WN, GM)                                          \
    template hipError_t launch_f16_o16<BM, BN, (ST == 1 ? 2 : ST), WM, WN, GM, ST == 1>( \
        const F16Args&, hipStream_t);
G355_F16_RING_CONFIGS(G355_F16_RING_O16)
G355_F16_PANEL_CONFIGS(G355_F16_PANEL_O16)

}  // namespace g355
