// fia_run_no_alloc: phase 2 for callers that cannot allocate device memory.
//
// The plan and the workspace of an executor live in `scratch`, a static
// device array of fixed size that every GPU the library runs on holds until
// the process ends.  Its device address on the current GPU is looked up once
// per device (hipGetSymbolAddress, with that device current) and kept; host
// code only ever uses that address, never the array's name.  Calls on one
// GPU share the array and keep the last call's contents: no kernel of the
// library expects zeroed scratch (every partial is written before it is
// read), and calls that overlap on one GPU race.
#include <mutex>
#include <string>

#include "fia.h"
#include "fia_internal.h"

namespace fia {
fia_status run_on_scratch(fia_executor* e, void* plan, size_t plan_cap, void* ws, size_t ws_cap,
                          void* stream);
void set_last_error(const char* msg);
}  // namespace fia

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // per GPU
constexpr size_t kPlanBytes = size_t(1) << 20;       // plan area at the start
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

extern "C" fia_status fia_run_no_alloc(fia_executor* executor, void* stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    fia::set_last_error("no usable current HIP device");
    return FIA_ERR_HIP;
  }
  void* base = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch_ptr[dev] == nullptr) {
      void* p = nullptr;
      const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (err != hipSuccess || p == nullptr) {
        fia::set_last_error((std::string("hipGetSymbolAddress of the scratch failed: ") +
                             hipGetErrorString(err)).c_str());
        return FIA_ERR_HIP;
      }
      g_scratch_ptr[dev] = p;
    }
    base = g_scratch_ptr[dev];
  }
  uint8_t* b = static_cast<uint8_t*>(base);
  return fia::run_on_scratch(executor, b, kPlanBytes, b + kPlanBytes, kScratchBytes - kPlanBytes,
                             stream);
}
