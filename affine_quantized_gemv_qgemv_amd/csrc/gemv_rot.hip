// GEMV kernel instances for the Mirai formats behind the RMSNorm + block-32 Hadamard prologue.
#include "gemv_kernel.h"

namespace qd {

hipError_t gemv_run_rot(const GemvArgs& a, const Cfg& c, int fmt, hipStream_t st) {
    return fmt == W_MIRAI_M ? run_batch<4, 2, W_MIRAI_M>(a, c, st) : run_batch<8, 2, W_MIRAI_L>(a, c, st);
}

}  // namespace qd
