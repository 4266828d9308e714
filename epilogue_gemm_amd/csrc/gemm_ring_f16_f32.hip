// gemm_ring_f16_f32.hip -- ring tile kernel instantiations (configurations 5-7: eight,
// four and two slots) for fp16 inputs and fp32 output (one translation unit per
// format pair, so they compile in parallel).
#include "gemm_ring.hpp"

namespace ge {

LaunchFn ring_launcher_f16_f32(int cfg, int la, int lb, int epi) {
  switch (cfg) {
    case 5: return ring::pick<f16, float, 8>(la, lb, epi);
    case 6: return ring::pick<f16, float, 4>(la, lb, epi);
    case 7: return ring::pick<f16, float, 2>(la, lb, epi);
    default: return nullptr;
  }
}

}  // namespace ge
