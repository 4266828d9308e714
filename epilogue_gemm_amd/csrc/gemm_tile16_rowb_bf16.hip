// gemm_tile16_rowb_bf16.hip -- the 16x16x32 tile kernel with a row-major B
// (transposing LDS reads) for bf16 inputs, every output format.  A unit of
// its own because it is compiled with the generic machine scheduler
// (build.py): under the default one the accumulators of this kernel are
// shuffled through extra registers at every k-step.
#include "gemm_tile16.hpp"

namespace ge {

LaunchFn tile16_rowb_launcher_bf16(int out_dt, int la, int lb, int epi) {
  if (out_dt == GEMM_EPI_F32) return tile16::pick<bf16, float, true>(la, lb, epi);
  if (out_dt == GEMM_EPI_FP8_E4M3) return tile16::pick<bf16, fp8e4m3, true>(la, lb, epi);
  return tile16::pick<bf16, bf16, true>(la, lb, epi);
}

}  // namespace ge
