// gemm_ring_bf16_fp8.hip -- ring tile kernel instantiations (configurations 5-7: eight,
// four and two slots) for bf16 inputs and FP8 E4M3 output (one translation unit per
// format pair, so they compile in parallel).
#include "gemm_ring.hpp"

namespace ge {

LaunchFn ring_launcher_bf16_fp8(int cfg, int la, int lb, int epi) {
  switch (cfg) {
    case 5: return ring::pick<bf16, fp8e4m3, 8>(la, lb, epi);
    case 6: return ring::pick<bf16, fp8e4m3, 4>(la, lb, epi);
    case 7: return ring::pick<bf16, fp8e4m3, 2>(la, lb, epi);
    default: return nullptr;
  }
}

}  // namespace ge
