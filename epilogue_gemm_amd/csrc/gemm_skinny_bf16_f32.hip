// gemm_skinny_bf16_f32.hip -- decode-shape kernel instantiations for bf16 inputs and
// fp32 output (one translation unit per format pair, so they compile in parallel).
#include "gemm_skinny.hpp"

namespace ge {

LaunchFn skinny_launcher_bf16_f32(int cfg, int epi) { return skinny_pick<bf16, float>(cfg, epi); }

}  // namespace ge
