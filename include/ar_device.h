// ar_device.h -- gfx950 device helpers for the self-synchronizing all-reduce.
//
// Memory-model notes (gfx94x/gfx950 family, one agent with 8 XCDs, each XCD
// with its own L2):
//  * A store or load with the sc1 cache-policy bit is coherent at device
//    (agent) scope: it is what the compiler emits for agent-scope relaxed
//    atomics, and it is how a value written on one XCD becomes visible to a
//    poll on another without a cache flush.
//  * An agent-scope release fence is buffer_wbl2 sc1 + a wait for all
//    outstanding memory operations; an acquire fence is buffer_inv sc1.
//  * Naturally aligned 8-byte accesses are single-copy atomic, which is the
//    property the LL word relies on.  A 16-byte access is used as two LL
//    words, each validated on its own.
//  * Raw buffer accesses carry a byte range: an access past it reads 0 and
//    a store past it is dropped, so a wrong offset into a receive buffer can
//    never touch other memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ar {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kWave = 64;
constexpr int kTileBytes = 1024;          // one wave x 16 bytes
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit format
constexpr int kCpAgent = 16;              // sc1: device-scope coherent access

// Protocol ids (same values as the public ar_proto enum).
constexpr int kLL = 0;
constexpr int kLL128 = 1;
constexpr int kSentinel = 2;
constexpr int kBarrier = 3;

// Status codes written by the device (same values as ar_status).
constexpr int kEtimeout = -5;
constexpr int kEcorrupt = -6;

// Control block words.
constexpr int kCtrlStatus = 0;
constexpr int kCtrlAbort = 1;
// One word per wave index from kCtrlProgress on: rank 0's progress in share
// mode, or the barrier baseline's arrival-and-completion counter.
constexpr int kCtrlProgress = 64;
constexpr int kCtrlMaxProgress = 4096;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)bytes, (int)kRsrcWord3);
}

__device__ __forceinline__ void compiler_barrier() {
  __asm__ __volatile__("" ::: "memory");
}

// Device-scope coherent 16/8-byte accesses (sc1).
__device__ __forceinline__ u32x4 ld16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpAgent);
}
__device__ __forceinline__ void st16(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCpAgent);
}
__device__ __forceinline__ u32x2 ld8(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCpAgent);
}
__device__ __forceinline__ void st8(rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kCpAgent);
}

// Ordering between device-scope coherent accesses.
//
// Every access that another XCD observes in this library (slots, flags,
// counters, progress words) is an sc1 access, which bypasses the per-XCD
// caches for coherence.  A full agent-scope fence adds an L2 writeback
// (release) or invalidate (acquire) of the whole XCD cache, which only
// matters for non-sc1 data; for sc1-only traffic what orders a later access
// after an earlier one is that the earlier one has completed, i.e. its
// acknowledgement has returned: s_waitcnt vmcnt(0).  The three orderings
// the protocols need -- data before flag (LL128, barrier), flag before data
// (LL128 consumer), re-arm before the next op's stores (sentinel dual
// buffer) -- are exercised across XCD pairs by ar_probe_litmus, which a GPU
// test runs.  AR_FORMAL_FENCES=1 selects the full agent-scope fences instead
// (the compiler's sequence, with the L2 writeback/invalidate).
#ifndef AR_FORMAL_FENCES
#define AR_FORMAL_FENCES 0
#endif

__device__ __forceinline__ void wait_vm() {
  compiler_barrier();
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), other counters untouched
  compiler_barrier();
}

__device__ __forceinline__ void fence_release() {
#if AR_FORMAL_FENCES
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
#else
  wait_vm();
#endif
}
__device__ __forceinline__ void fence_acquire() {
#if AR_FORMAL_FENCES
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#else
  wait_vm();
#endif
}
__device__ __forceinline__ void fence_acq_rel() {
#if AR_FORMAL_FENCES
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
#else
  wait_vm();
#endif
}

__device__ __forceinline__ uint32_t ld_agent_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t now_ticks() { return wall_clock64(); }

// ------------------------------------------------------------- epochs ---
// seq counts ops from 1 and skips 0 when the u32 wraps.
__device__ __forceinline__ uint32_t seq_next(uint32_t s) {
  return s == 0xFFFFFFFFu ? 1u : s + 1u;
}
__device__ __forceinline__ uint32_t seq_prev(uint32_t s) {
  return s == 1u ? 0xFFFFFFFFu : s - 1u;
}

// --------------------------------------------------------------- bf16 ---
__device__ __forceinline__ float bf_lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf_hi(uint32_t w) {
  return __uint_as_float(w & 0xFFFF0000u);
}
// binary32 -> bf16, nearest even, every NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? 0x7FC0u : r;
}
__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) {
  return (lo & 0xFFFFu) | (hi << 16);
}
// A bf16 pattern above 0xFF80 is a negative NaN; it leaves as 0x7FC0 so the
// sentinel 0xFFFF can never be sent.
__device__ __forceinline__ uint32_t canon_half(uint32_t h) {
  return h > 0xFF80u ? 0x7FC0u : h;
}
__device__ __forceinline__ uint32_t canon_word(uint32_t w) {
  return canon_half(w & 0xFFFFu) | (canon_half(w >> 16) << 16);
}
// A dword is delivered when neither bf16 half still holds the sentinel.
__device__ __forceinline__ bool word_delivered(uint32_t w) {
  return (w & 0xFFFFu) != 0xFFFFu && (w >> 16) != 0xFFFFu;
}

// ------------------------------------------------------------- status ---
__device__ __forceinline__ void report_error(int* ctrl, int code) {
  int expected = 0;
  __hip_atomic_compare_exchange_strong(ctrl + kCtrlStatus, &expected, code,
                                       __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(ctrl + kCtrlAbort, 1, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool aborted(const int* ctrl) {
  return __hip_atomic_load(ctrl + kCtrlAbort, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT) != 0;
}

// Bounded wait helper: returns false (and reports once per wave) when the
// deadline passes or another wave has aborted the kernel.
struct Waiter {
  uint64_t deadline;
  int* ctrl;
  uint32_t iter;
  __device__ __forceinline__ Waiter(uint64_t timeout_ticks, int* c)
      : deadline(now_ticks() + timeout_ticks), ctrl(c), iter(0) {}
  // Call after an unsuccessful poll.  true = keep polling.
  __device__ __forceinline__ bool again(int lane) {
    ++iter;
    __builtin_amdgcn_s_sleep(1);
    compiler_barrier();
    if ((iter & 7u) == 0u) {
      if (aborted(ctrl)) return false;
      if (now_ticks() > deadline) {
        if (lane == 0) report_error(ctrl, kEtimeout);
        return false;
      }
    }
    return true;
  }
};

}  // namespace ar
