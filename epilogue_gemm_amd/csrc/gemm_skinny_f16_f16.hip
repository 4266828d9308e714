// gemm_skinny_f16_f16.hip -- decode-shape kernel instantiations for fp16 inputs and
// fp16 output (one translation unit per format pair, so they compile in parallel).
#include "gemm_skinny.hpp"

namespace ge {

LaunchFn skinny_launcher_f16_f16(int cfg, int epi) { return skinny_pick<f16, f16>(cfg, epi); }

}  // namespace ge
