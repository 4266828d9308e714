// gemm_skinny_f16_f32.hip -- decode-shape kernel instantiations for fp16 inputs and
// fp32 output (one translation unit per format pair, so they compile in parallel).
#include "gemm_skinny.hpp"

namespace ge {

LaunchFn skinny_launcher_f16_f32(int cfg, int epi) { return skinny_pick<f16, float>(cfg, epi); }

}  // namespace ge
