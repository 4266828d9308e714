// gemm_tile_f16_f16.hip -- tile-kernel instantiations for f16 inputs and f16 output
// (one translation unit per format pair, so they compile in parallel).
#include "tile_dispatch.hpp"

namespace ge {

LaunchFn tile_launcher_f16_f16(int cfg, int la, int lb, int epi) {
  return tile::pick_config<f16, f16>(cfg, la, lb, epi);
}

}  // namespace ge
