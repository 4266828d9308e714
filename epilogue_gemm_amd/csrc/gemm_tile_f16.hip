// gemm_tile_f16.hip -- f16-input instantiations of the tile kernel.
#include "gemm_tile.hpp"

namespace ge {

namespace {
template <int BM, int BN>
LaunchFn pick_out(int out_dt, int la, int lb) {
  if (out_dt == GEMM_EPI_F32) return tile::pick_layout<BM, BN, f16, float>(la, lb);
  return tile::pick_layout<BM, BN, f16, f16>(la, lb);
}
}  // namespace

LaunchFn tile_launcher_f16(int cfg, int out_dt, int la, int lb) {
  switch (cfg) {
    case 0: return pick_out<256, 256>(out_dt, la, lb);
    case 1: return pick_out<128, 128>(out_dt, la, lb);
    case 2: return pick_out<64, 64>(out_dt, la, lb);
    default: return nullptr;
  }
}

}  // namespace ge
