// gemm_tile_bf16_f32.hip -- tile-kernel instantiations for bf16 inputs and f32 output
// (one translation unit per format pair, so they compile in parallel).
#include "tile_dispatch.hpp"

namespace ge {

LaunchFn tile_launcher_bf16_f32(int cfg, int la, int lb, int epi) {
  return tile::pick_config<bf16, float>(cfg, la, lb, epi);
}

}  // namespace ge
