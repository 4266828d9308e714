// gemm_ring_bf16_bf16.hip -- ring tile kernel instantiations (configurations 5-7: eight,
// four and two slots) for bf16 inputs and bf16 output (one translation unit per
// format pair, so they compile in parallel).
#include "gemm_ring.hpp"

namespace ge {

LaunchFn ring_launcher_bf16_bf16(int cfg, int la, int lb, int epi) {
  switch (cfg) {
    case 5: return ring::pick<bf16, bf16, 8>(la, lb, epi);
    case 6: return ring::pick<bf16, bf16, 4>(la, lb, epi);
    case 7: return ring::pick<bf16, bf16, 2>(la, lb, epi);
    default: return nullptr;
  }
}

}  // namespace ge
