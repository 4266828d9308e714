// gemm_tile_bf16_fp8.hip -- tile-kernel instantiations for bf16 inputs and FP8 E4M3 output
// (one translation unit per format pair, so they compile in parallel).
#include "tile_dispatch.hpp"

namespace ge {

LaunchFn tile_launcher_bf16_fp8(int cfg, int la, int lb, int epi) {
  return tile::pick_config<bf16, fp8e4m3>(cfg, la, lb, epi);
}

}  // namespace ge
