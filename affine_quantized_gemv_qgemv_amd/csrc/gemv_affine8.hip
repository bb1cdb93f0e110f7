// GEMV kernel instances for MLX affine 8-bit weights (the router).
#include "gemv_kernel.h"

namespace qd {

hipError_t gemv_run_affine8(const GemvArgs& a, const Cfg& c, int xf, hipStream_t st) {
    return xf == 0 ? run_batch<8, 0, W_AFFINE>(a, c, st) : run_batch<8, 1, W_AFFINE>(a, c, st);
}

}  // namespace qd
