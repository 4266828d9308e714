// gemm_skinny_f16_fp8.hip -- decode-shape kernel instantiations for fp16 inputs and
// FP8 E4M3 output (one translation unit per format pair, so they compile in parallel).
#include "gemm_skinny.hpp"

namespace ge {

LaunchFn skinny_launcher_f16_fp8(int cfg, int epi) { return skinny_pick<f16, fp8e4m3>(cfg, epi); }

}  // namespace ge
