// gemm_tile_f16_f32.hip -- tile-kernel instantiations for f16 inputs and f32 output
// (one translation unit per format pair, so they compile in parallel).
#include "tile_dispatch.hpp"

namespace ge {

LaunchFn tile_launcher_f16_f32(int cfg, int la, int lb, int epi) {
  return tile::pick_config<f16, float>(cfg, la, lb, epi);
}

}  // namespace ge
