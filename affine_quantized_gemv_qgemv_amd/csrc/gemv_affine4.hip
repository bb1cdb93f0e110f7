// GEMV kernel instances for MLX affine 4-bit weights (fp16 and fp32-staged activations).
#include "gemv_kernel.h"

namespace qd {

hipError_t gemv_run_affine4(const GemvArgs& a, const Cfg& c, int xf, hipStream_t st) {
    return xf == 0 ? run_batch<4, 0, W_AFFINE>(a, c, st) : run_batch<4, 1, W_AFFINE>(a, c, st);
}

}  // namespace qd
