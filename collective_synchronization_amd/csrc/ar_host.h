// ar_host.h -- host-side helpers shared by the library's translation units:
// device attributes, size arithmetic of the slot layouts, argument checks
// and typed kernel launches.  Internal; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <mutex>

#include "../../include/ar.h"
#include "../../include/ar_device.h"

namespace ar {

constexpr int kBlock = 256;              // 4 waves
constexpr int kWavesPerBlock = kBlock / kWave;

struct DeviceInfo {
  bool ok = false;
  int cus = 0;
  double wallclock_hz = 0.0;
  int coop = 0;
};

inline int device_info(DeviceInfo* out) {
  static std::mutex g_mu;
  static DeviceInfo g_info[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return AR_ENODEV;
  std::lock_guard<std::mutex> lk(g_mu);
  DeviceInfo& d = g_info[dev];
  if (!d.ok) {
    int cus = 0, khz = 0, coop = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return AR_ENODEV;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
      return AR_ENODEV;
    if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess)
      coop = 0;
    d.cus = cus;
    d.wallclock_hz = (double)khz * 1000.0;
    d.coop = coop;
    d.ok = true;
  }
  *out = d;
  return AR_OK;
}

// A poll deadline the library accepts (0 means the default of 1 s).
inline bool timeout_ok(uint64_t ns) { return ns <= AR_MAX_TIMEOUT_NS; }

inline uint64_t ns_to_ticks(uint64_t ns, double hz) {
  if (ns == 0) ns = 1000000000ull;
  const double t = (double)ns * hz * 1e-9;
  return t < 1.0 ? 1ull : (uint64_t)t;
}

inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int64_t encoded_bytes(int32_t proto, int64_t count) {
  if (count < 0) return AR_EINVAL;
  switch (proto) {
    case kLL: return 16 * ceil_div64(count, 4);
    case kLL128: return 128 * ceil_div64(count, 60);
    case kSentinel:
    case kBarrier: return 16 * ceil_div64(count, 8);
    default: return AR_EINVAL;
  }
}

inline int64_t slot_bytes_of(int32_t proto, int64_t count) {
  const int64_t E = encoded_bytes(proto, count);
  if (E < 0) return E;
  return ceil_div64(E, 128) * 128;
}

// Share width of a two-shot all-reduce: ceil(count / n) rounded up to a
// multiple of 8 elements (16 bytes), so every share starts 16-byte aligned.
inline int64_t share_width(int64_t count, int n) {
  return (ceil_div64(count, n) + 7) / 8 * 8;
}

inline void share_bounds(int64_t count, int n, int k, int64_t* lo, int64_t* hi) {
  const int64_t w = share_width(count, n);
  int64_t a = (int64_t)k * w;
  if (a > count) a = count;
  int64_t b = a + w;
  if (b > count) b = count;
  *lo = a;
  *hi = b;
}

inline int64_t desc_slot_bytes(const ar_desc* d) {
  if (d->collective == AR_TWOSHOT)
    return slot_bytes_of(d->proto, share_width(d->count, d->nranks));
  return slot_bytes_of(d->proto, d->count);
}

// Bytes of one region (all consumers, both parities, all sources).
inline int64_t desc_region_bytes(const ar_desc* d) {
  return (int64_t)d->nconsumers * 2 * d->nranks * desc_slot_bytes(d);
}

inline int64_t desc_scratch_bytes(const ar_desc* d) {
  return desc_region_bytes(d) * (d->collective == AR_TWOSHOT ? 2 : 1);
}

inline bool aligned(const void* p, uintptr_t a) {
  return ((uintptr_t)p & (a - 1)) == 0;
}

inline int check_desc(const ar_desc* d) {
  if (!d) return AR_EINVAL;
  if (d->nranks < 1 || d->nranks > AR_MAX_RANKS) return AR_EINVAL;
  if (d->nconsumers != 1 && d->nconsumers != d->nranks) return AR_EINVAL;
  if (d->count < 0) return AR_EINVAL;
  if (d->proto < 0 || d->proto > kBarrier) return AR_EINVAL;
  if (d->collective < AR_ALLREDUCE || d->collective > AR_TWOSHOT) return AR_EINVAL;
  if (d->collective == AR_TWOSHOT &&
      (d->nconsumers != d->nranks || d->proto == kBarrier))
    return AR_EINVAL;
  const int64_t slot = desc_slot_bytes(d);
  if (slot > (int64_t(1) << 30)) return AR_ESIZE;
  if (desc_scratch_bytes(d) >= (int64_t(1) << 32)) return AR_ESIZE;
  return AR_OK;
}

inline int check_rows(const void* p, int64_t stride, int64_t count) {
  if (count == 0) return AR_OK;
  if (!p) return AR_EINVAL;
  if (stride < count) return AR_EINVAL;
  if (!aligned(p, 16) || (stride % 8) != 0) return AR_EALIGN;
  if (stride >= (int64_t(1) << 30)) return AR_ESIZE;   // row byte offsets stay 32-bit
  return AR_OK;
}

// Launch choice without a flag.  A cooperative launch may fill the
// occupancy the runtime reports, an ordinary one keeps half; the
// cooperative launch costs a fixed ~15 us more per launch on MI355X (8 ranks
// [1,4096]: 23.4 against 6.8 us for one op, the same per-op time over 256
// ops).  It is taken when the device supports it, the launch holds at least
// kCoopMinOps ops, and its grid lets the waves walk fewer tiles in the same
// kernel, or run the workgroup kernel where the ordinary grid needs the
// one-wave kernel (or the ordinary grid does not fit at all).  (Taking every
// many-tile launch cooperatively, for the residency guarantee, was tried: the
// profiler's kernel trace of such launches then ends without its results, so
// those launches stay ordinary where the geometry is the same.)
constexpr int kCoopMinOps = 32;

inline bool coop_pays(int rc_ord, int tpw_ord, bool wide_ord, int tpw_co, bool wide_co) {
  if (rc_ord != AR_OK) return true;
  if (wide_co == wide_ord) return tpw_co < tpw_ord;
  return wide_co;
}

inline thread_local int g_last_hip_error = 0;

inline int map_hip(hipError_t e) {
  if (e == hipSuccess) return AR_OK;
  g_last_hip_error = (int)e;
  return AR_ELAUNCH;
}

// Launch with the runtime's own return code (not the sticky last error,
// which may hold an unrelated earlier failure of the calling thread).
template <typename... KArgs>
inline hipError_t launch_typed(void (*kernel)(KArgs...), dim3 grid, dim3 block,
                               hipStream_t s, KArgs... args) {
  void* argv[sizeof...(KArgs) + 1] = {static_cast<void*>(&args)..., nullptr};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block,
                         argv, 0, s);
}

// Every argument is converted to the kernel's own parameter type first.
template <typename... KArgs, typename... Args>
inline hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block,
                         hipStream_t s, Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel arity");
  return launch_typed<KArgs...>(kernel, grid, block, s, static_cast<KArgs>(args)...);
}


// Entry points of the other collectives (ar_collectives.hip).
int twoshot_pack(int32_t proto, const ar_desc* d, const void* in, int64_t in_stride,
                 void* scratch, ar_epoch e, hipStream_t s);
int twoshot_reduce(const ar_desc* d, void* scratch, void* out, int64_t out_stride,
                   ar_epoch e, void* ctrl, uint64_t timeout_ns, int32_t flags,
                   hipStream_t s);
int coll_sim_geometry(const ar_sim_params* p, int32_t* groups, int32_t* tiles,
                      int32_t* tiles_per_group, int32_t* blocks, int32_t* wide,
                      int32_t* cooperative);
int coll_sim_run(const ar_sim_params* p, hipStream_t s);
int chain_sim_geometry(const ar_sim_params* p, int32_t* blocks, int32_t* cooperative);
int chain_sim_run(const ar_sim_params* p, const float* scales, hipStream_t s);
// Every host-side check ar_sim_run makes, including the grid it would launch,
// without enqueuing anything (ar_kernels.hip).
int sim_validate(const ar_sim_params* p);
// Fill [0, bytes) of a device buffer with a 32-bit pattern: a kernel with
// device-scope coherent 16-byte stores, so it can be captured in a graph
// (ar_state.hip).  bytes: a multiple of 16, below 4 GiB.
hipError_t fill_words(void* base, int64_t bytes, uint32_t word, hipStream_t s);

}  // namespace ar
