// GEMV kernel instances for the Mirai-M and Mirai-L weight formats, without and with the rotation
// prologue.
#include "gemv_kernel.h"

namespace qd {

hipError_t gemv_run_mirai_m(const GemvArgs& a, const Cfg& c, int xf, hipStream_t st) {
    return xf == 0 ? run_batch<4, 0, W_MIRAI_M>(a, c, st) : run_batch<4, 1, W_MIRAI_M>(a, c, st);
}

hipError_t gemv_run_mirai_l(const GemvArgs& a, const Cfg& c, int xf, hipStream_t st) {
    return xf == 0 ? run_batch<8, 0, W_MIRAI_L>(a, c, st) : run_batch<8, 1, W_MIRAI_L>(a, c, st);
}

}  // namespace qd
