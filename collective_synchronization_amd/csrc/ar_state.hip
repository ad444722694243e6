// ar_state.hip -- fill kernels that return buffers to their initial state,
// and ar_state_reset, which makes captured sequences of calls replayable.
//
// Every buffer the protocols share has one state in which any epoch may
// start: the control block zero, LL / LL128 / barrier receive buffers zero
// (a zero flag is "never written"), SENTINEL receive buffers all 0xFFFF
// ("Why Microseconds Matter in AI Infrastructure", section "Latency can
// matter more than bandwidth": the receive buffer starts as a negative NaN),
// and the work buffer of the linear-layer chain zero (its hand-off words are
// LL words).  A HIP graph replays the epochs its calls were captured with, so
// a replay is only sound from the state the capture started from; one
// ar_state_reset at the head of the captured sequence restores it on every
// replay.  The fills are kernels, not memset nodes.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "../../include/ar.h"
#include "ar_host.h"

namespace ar {

// Fill [0, bytes) of `base` with the 32-bit pattern `word`, 16 bytes a lane,
// with device-scope coherent stores (the protocols poll with such loads).
__global__ __launch_bounds__(kBlock) void k_fill_words(uint8_t* base, uint32_t bytes,
                                                       uint32_t word) {
  const rsrc_t rs = make_rsrc(base, bytes);
  const u32x4 v = u32x4{word, word, word, word};
  // 64-bit offsets, so that the last step cannot wrap below `bytes`
  const uint64_t step = (uint64_t)gridDim.x * kBlock * 16u;
  for (uint64_t off = ((uint64_t)blockIdx.x * kBlock + threadIdx.x) * 16u; off < bytes;
       off += step)
    st16(rs, (uint32_t)off, v);
}

hipError_t fill_words(void* base, int64_t bytes, uint32_t word, hipStream_t s) {
  if (bytes <= 0) return hipSuccess;
  int64_t blocks = ceil_div64(bytes, (int64_t)kBlock * 16);
  if (blocks > 4096) blocks = 4096;
  return launch(k_fill_words, dim3((unsigned)blocks), dim3(kBlock), s,
                static_cast<uint8_t*>(base), (uint32_t)bytes, word);
}

}  // namespace ar

using namespace ar;

extern "C" int ar_state_reset(const ar_desc* d, void* scratch, void* ctrl, void* work,
                              void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (!scratch && !ctrl && !work) return AR_EINVAL;
  const int64_t sbytes = desc_scratch_bytes(d);
  const int64_t wbytes = work ? ar_linear_work_bytes(d) : 0;
  if (wbytes < 0) return (int)wbytes;
  if (scratch && !aligned(scratch, 256)) return AR_EALIGN;
  if (ctrl && !aligned(ctrl, 256)) return AR_EALIGN;
  if (work && !aligned(work, 256)) return AR_EALIGN;
  // the fill kernel's offsets are 32-bit
  if ((scratch && sbytes >= (int64_t(1) << 32)) || (work && wbytes >= (int64_t(1) << 32)))
    return AR_ESIZE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (ctrl) {
    rc = map_hip(fill_words(ctrl, ar_ctrl_bytes(), 0u, s));
    if (rc) return rc;
  }
  if (scratch) {
    const uint32_t init = d->proto == AR_SENTINEL ? 0xFFFFFFFFu : 0u;
    rc = map_hip(fill_words(scratch, sbytes, init, s));
    if (rc) return rc;
  }
  if (work) {
    rc = map_hip(fill_words(work, wbytes, 0u, s));
    if (rc) return rc;
  }
  return AR_OK;
}
