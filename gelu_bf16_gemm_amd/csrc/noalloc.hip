// Device scratch of fusedops_linear_epilogue_noalloc: the FP8 row-rendezvous workspace kept in
// a library-owned device array instead of a caller-allocated buffer, for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ variable, so every GPU the library runs on holds its own
// copy, at its own address, from module load until the process ends. Host code never uses the
// array's name as an address (on the host it is only a stand-in for the symbol): the device
// address is looked up once per device with hipGetSymbolAddress, with that device current, and
// that pointer is what kernels and the clear launch receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/fusedops.h"
#include "kernels.h"

namespace fusedops {

static __device__ __align__(256) uint32_t scratch[FUSEDOPS_NOALLOC_SCRATCH_BYTES / 4];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Zero the words a quantised call needs at zero: the tile ticket counter (word 1) and the
// control lines of every 32-token block record (arrival counters and the release flag).
// Slots need no clearing (readers take only words the current call has written before the
// release), and the error word (word 0) stays sticky for fusedops_rendezvous_error. One
// workgroup per record; plain vector stores (a fill kernel rather than a memset, so the
// clear can sit inside a captured graph).
__global__ __launch_bounds__(256) void clear_rendezvous_kernel(uint32_t* ws, int ctl_words, int64_t record_words) {
  uint32_t* rec = ws + 32 + (int64_t)blockIdx.x * record_words;
  for (int i = threadIdx.x; i < ctl_words; i += blockDim.x) rec[i] = 0u;
  if (blockIdx.x == 0 && threadIdx.x == 1) ws[1] = 0u;
}

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

hipError_t launch_clear_rendezvous(void* ws, int64_t records, int ctl_words, int64_t record_words,
                                   hipStream_t stream) {
  if (records < 1 || records > (int64_t(1) << 30)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(clear_rendezvous_kernel, dim3((unsigned)records), dim3(256), 0, stream,
                     static_cast<uint32_t*>(ws), ctl_words, record_words);
  return hipGetLastError();
}

}  // namespace fusedops
