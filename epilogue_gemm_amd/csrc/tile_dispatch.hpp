// tile_dispatch.hpp -- the two-stage tile configurations (0-4) of one input
// and output format, in the order of the host-side table (gemm_epi.cpp).
#pragma once

#include "gemm_tile.hpp"
#include "gemm_tile16.hpp"

namespace ge {
namespace tile {

template <typename TIn, typename TOut>
LaunchFn pick_config(int cfg, int la, int lb, int epi) {
  switch (cfg) {
    case 0: return pick_layout<256, 256, 4, TIn, TOut>(la, lb, epi);
    case 1: return pick_layout<128, 128, 4, TIn, TOut>(la, lb, epi);
    case 2: return pick_layout<64, 64, 4, TIn, TOut>(la, lb, epi);
    case 3: return pick_layout<256, 256, 8, TIn, TOut>(la, lb, epi);
    case 4: return tile16::pick<TIn, TOut, false>(la, lb, epi);
    // 5-7, the rings: gemm_ring_<in>_<out>.hip; 8, the row-major-B 16x16x32
    // kernel: gemm_tile16_rowb_*.hip
    default: return nullptr;
  }
}

}  // namespace tile
}  // namespace ge
