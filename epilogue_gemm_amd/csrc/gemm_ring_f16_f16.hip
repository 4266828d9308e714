// gemm_ring_f16_f16.hip -- ring tile kernel instantiations (configurations 5-7: eight,
// four and two slots) for fp16 inputs and fp16 output (one translation unit per
// format pair, so they compile in parallel).
#include "gemm_ring.hpp"

namespace ge {

LaunchFn ring_launcher_f16_f16(int cfg, int la, int lb, int epi) {
  switch (cfg) {
    case 5: return ring::pick<f16, f16, 8>(la, lb, epi);
    case 6: return ring::pick<f16, f16, 4>(la, lb, epi);
    case 7: return ring::pick<f16, f16, 2>(la, lb, epi);
    default: return nullptr;
  }
}

}  // namespace ge
