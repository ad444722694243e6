// ar_static.hip -- ar_sim_run_static: the persistent all-reduce simulator for
// callers that cannot allocate device memory (code under graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The receive buffers and the control block that ar_sim_run takes from the
// caller live here in one library-owned device array, `scratch`, of
// kStaticBytes bytes.  Each device the library runs on holds its own copy
// until the process ends.  In host code the array's name only stands for the
// device symbol, so the device address of this device's copy is looked up
// once per device (hipGetSymbolAddress, with that device current) and kept;
// every host-side use (kernel arguments, the fills) goes through that address.
//
// Every call clears what the protocols need cleared before the simulator
// runs: the control block to zero, and the receive buffers of the call's
// descriptor to zero (LL, LL128, barrier: a zero flag is "never written") or
// to the sentinel 0xFFFF (SENTINEL).  The clears are small fill kernels on
// the caller's stream (no memset nodes), so the call can be captured.  All
// calls on one device share the array: calls that overlap in time on one
// device (different streams without ordering between them) race.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <mutex>

#include "../../include/ar.h"
#include "ar_host.h"

namespace ar {

// control block first (ar_ctrl_bytes() rounded up to 256 bytes), then the
// receive buffers
constexpr int64_t kStaticCtrlBytes =
    ((int64_t)(kCtrlProgress + kCtrlMaxProgress) * 4 + 256 + 255) / 256 * 256;
constexpr int64_t kStaticBytes = kStaticCtrlBytes + (int64_t)AR_STATIC_SCRATCH_BYTES;
static_assert(kStaticBytes < (int64_t(1) << 31), "fill offsets stay 32-bit");

static __device__ __align__(256) uint8_t scratch[kStaticBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
uint8_t* g_static_base[kMaxDevices];   // device address of `scratch`, per device

// Device address of this device's `scratch` (looked up on the first call on
// the device, with the device current).
int static_base(uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return AR_ENODEV;
  std::lock_guard<std::mutex> lk(g_static_mu);
  if (!g_static_base[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return map_hip(e);
    if (!ptr) return map_hip(hipErrorInvalidSymbol);
    g_static_base[dev] = static_cast<uint8_t*>(ptr);
  }
  *out = g_static_base[dev];
  return AR_OK;
}

}  // namespace

// The status word of the control block, copied to the caller's output.
__global__ void k_static_status(const int* ctrl, int32_t* status) {
  if (threadIdx.x == 0)
    *status = __hip_atomic_load(ctrl + kCtrlStatus, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace ar

using namespace ar;

extern "C" int ar_sim_run_static(const ar_sim_params* p, int32_t* status, void* stream) {
  if (!p || !status) return AR_EINVAL;
  if (p->scratch || p->ctrl) return AR_EINVAL;       // the library's own buffers are used
  if (!aligned(status, 4)) return AR_EALIGN;
  int rc = check_desc(&p->desc);
  if (rc) return rc;
  const int64_t need = desc_scratch_bytes(&p->desc);
  if (need > (int64_t)AR_STATIC_SCRATCH_BYTES) return AR_ESIZE;
  uint8_t* base = nullptr;
  rc = static_base(&base);
  if (rc) return rc;
  ar_sim_params q = *p;
  q.ctrl = base;
  q.scratch = base + kStaticCtrlBytes;
  rc = sim_validate(&q);                 // every host-side check, nothing enqueued
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = map_hip(fill_words(base, kStaticCtrlBytes, 0u, s));
  if (rc) return rc;
  const uint32_t armed = p->desc.proto == kSentinel ? 0xFFFFFFFFu : 0u;
  rc = map_hip(fill_words(base + kStaticCtrlBytes, need, armed, s));
  if (rc) return rc;
  rc = ar_sim_run(&q, stream);
  if (rc) return rc;
  return map_hip(launch(k_static_status, dim3(1), dim3(64), s,
                        static_cast<const int*>(q.ctrl), status));
}
