// noalloc.hip -- gemm_epi_run_noalloc: gemm_epi_run_ws for callers that
// cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// The only kernel that needs memory beyond its inputs and outputs is the
// split-K skinny kernel (fp32 partial blocks and per-column-block arrival
// counters).  Here that workspace is a file-scope device array, `scratch`,
// of GEMM_EPI_NOALLOC_SCRATCH_BYTES: the runtime reserves one copy on each
// GPU when it loads the library's code object there, and it stays until the
// process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory, so
// its device address is looked up once per device with hipGetSymbolAddress
// (with that device current) and kept in `g_scratch`; only that address is
// ever passed to a kernel.
//
// Every call on a GPU shares that GPU's array and finds it as the last call
// left it, so a call that splits K first clears the part it will use with a
// small fill kernel (a kernel, not hipMemsetAsync, so that a captured graph
// holds kernel nodes only).  Calls that overlap in time on one GPU race on
// the array: order them on one stream or with events.
#include <mutex>

#include "kernels.hpp"

namespace ge {
namespace {

static_assert(GEMM_EPI_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");

static __device__ __align__(256) unsigned char scratch[GEMM_EPI_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device (nullptr: not looked up yet)
std::mutex g_scratch_mu;

// Device address of this device's `scratch`, looked up on first use.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

// Zero n16 16-byte words at p.
__global__ __launch_bounds__(256) void clear_kernel(u32x4* __restrict__ p, uint32_t n16) {
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n16; i += gridDim.x * 256u) p[i] = u32x4{0u, 0u, 0u, 0u};
}

}  // namespace
}  // namespace ge

extern "C" gemm_epi_status gemm_epi_run_noalloc(gemm_epi_plan_t plan, const void* A, const void* B,
                                                const void* bias, void* C, void* stream) {
  const gemm_epi_status chk = ge::check_run_args(plan, A, B, bias, C);
  if (chk != GEMM_EPI_OK) return chk;
  const size_t need = gemm_epi_workspace_size(plan);
  if (need == 0) return gemm_epi_run(plan, A, B, bias, C, stream);
  if (need > (size_t)GEMM_EPI_NOALLOC_SCRATCH_BYTES) return GEMM_EPI_ERR_UNSUPPORTED;
  void* ws = nullptr;
  hipError_t e = ge::scratch_address(&ws);
  if (e == hipSuccess) {
    // need is a multiple of 256 bytes (the counters' area is rounded up)
    const uint32_t n16 = (uint32_t)(need / 16);
    const uint32_t blocks = (n16 + 255u) / 256u < 256u ? (n16 + 255u) / 256u : 256u;
    hipLaunchKernelGGL(ge::clear_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (ge::u32x4*)ws, n16);
    e = hipGetLastError();
  }
  if (e != hipSuccess) {
    ge::set_last_hip_error((int)e);
    return GEMM_EPI_ERR_HIP;
  }
  return gemm_epi_run_ws(plan, A, B, bias, C, ws, (size_t)GEMM_EPI_NOALLOC_SCRATCH_BYTES, stream);
}
