// ar_protocols.h -- per-protocol encode (producer) and poll/validate/reduce
// (consumer) for one tile: 1 KiB of a receive slot, one wave, 16 bytes a lane.
//
// Lane -> element map of tile t (the slot layout is fixed by the encoding):
//   LL        4 elements at 256t + 4*lane       (two 8-byte words: data|flag)
//   SENTINEL  8 elements at 512t + 8*lane       (plain bf16, 0xFFFF = empty)
//   BARRIER   8 elements at 512t + 8*lane       (plain bf16)
//   LL128     line L = 8t + lane/8, chunk j = lane%8:
//             j < 7: 8 elements at 60L + 8j; j = 7: 4 elements at 60L + 56
//             followed by the line's u64 flag.
#pragma once

#include "ar_device.h"

namespace ar {

template <int P>
__device__ __forceinline__ void lane_elems(int tile, int lane, int64_t& first,
                                           int& n) {
  if (P == kLL) {
    first = (int64_t)tile * 256 + lane * 4;
    n = 4;
  } else if (P == kLL128) {
    const int64_t line = (int64_t)tile * 8 + (lane >> 3);
    const int j = lane & 7;
    first = 60 * line + 8 * j;
    n = (j == 7) ? 4 : 8;
  } else {
    first = (int64_t)tile * 512 + lane * 8;
    n = 8;
  }
}

// Load n (4 or 8) bf16 from row[first..] as packed dwords w[0..n/2), zero
// past `count`.  first is a multiple of 4, so 8-byte loads are aligned;
// 16-byte loads are used when first is a multiple of 8.
__device__ __forceinline__ void load_elems(const uint16_t* __restrict__ row,
                                           int64_t count, int64_t first, int n,
                                           uint32_t w[4]) {
  if (first + n <= count) {
    if (n == 8 && (first & 7) == 0) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(row + first);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
      const u32x2 a = *reinterpret_cast<const u32x2*>(row + first);
      w[0] = a.x; w[1] = a.y;
      if (n == 8) {
        const u32x2 b = *reinterpret_cast<const u32x2*>(row + first + 4);
        w[2] = b.x; w[3] = b.y;
      }
    }
  } else {
    for (int k = 0; k < n; k += 2) {
      const uint32_t lo = (first + k < count) ? row[first + k] : 0u;
      const uint32_t hi = (first + k + 1 < count) ? row[first + k + 1] : 0u;
      w[k >> 1] = pack2(lo, hi);
    }
  }
}

// Store n (4 or 8) bf16 packed in w to row[first..], only below `count`.
__device__ __forceinline__ void store_elems(uint16_t* __restrict__ row,
                                            int64_t count, int64_t first,
                                            int n, const uint32_t w[4]) {
  if (first + n <= count) {
    if (n == 8 && (first & 7) == 0) {
      u32x4 v;
      v.x = w[0]; v.y = w[1]; v.z = w[2]; v.w = w[3];
      *reinterpret_cast<u32x4*>(row + first) = v;
    } else {
      u32x2 a;
      a.x = w[0]; a.y = w[1];
      *reinterpret_cast<u32x2*>(row + first) = a;
      if (n == 8) {
        u32x2 b;
        b.x = w[2]; b.y = w[3];
        *reinterpret_cast<u32x2*>(row + first + 4) = b;
      }
    }
  } else {
    for (int k = 0; k < n; ++k) {
      if (first + k < count) {
        const uint32_t d = w[k >> 1];
        row[first + k] = (uint16_t)((k & 1) ? (d >> 16) : (d & 0xFFFFu));
      }
    }
  }
}

// ----------------------------------------------------------- producer ---

// Elements of the lane's chunk of tile `tile` that lie below `count`.
template <int P>
__device__ __forceinline__ int chunk_keep(int64_t count, int tile, int lane) {
  int64_t first;
  int n;
  lane_elems<P>(tile, lane, first, n);
  const int64_t left = count - first;
  return (int)(left < 0 ? 0 : (left < n ? left : n));
}

// The lane's raw input words (bf16 pairs) of tile `tile`.  Branch-free:
// every lane issues the same buffer loads through a resource whose range is
// the row (`row_bytes`; reads past it return 0).  The words are returned
// unmasked, so that a load issued for the next op can stay in flight across
// the op loop; mask_words(w, chunk_keep(...)) clears what lies past count.
template <int P>
__device__ __forceinline__ void load_chunk(const uint16_t* __restrict__ row,
                                           uint32_t row_bytes, int tile,
                                           int lane, uint32_t w[4]) {
  int64_t first;
  int n;
  lane_elems<P>(tile, lane, first, n);
  const rsrc_t rr = make_rsrc(row, row_bytes);
  const int64_t off64 = first * 2;
  const uint32_t off = off64 < (int64_t)row_bytes ? (uint32_t)off64 : row_bytes;
  if (P == kLL) {
    const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(rr, off, 0, 0);
    w[0] = a.x; w[1] = a.y; w[2] = 0u; w[3] = 0u;
  } else if (P == kLL128) {
    // 8-byte aligned only (60 elements per line): two 8-byte loads
    const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(rr, off, 0, 0);
    const u32x2 b = __builtin_amdgcn_raw_buffer_load_b64(rr, off + 8u, 0, 0);
    w[0] = a.x; w[1] = a.y; w[2] = b.x; w[3] = b.y;
  } else {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rr, off, 0, 0);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
}

// Keep the first `keep` bf16 halves of w, clear the rest.
__device__ __forceinline__ void mask_words(uint32_t w[4], int keep) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t lo_ok = (2 * d < keep) ? 0x0000FFFFu : 0u;
    const uint32_t hi_ok = (2 * d + 1 < keep) ? 0xFFFF0000u : 0u;
    w[d] &= (lo_ok | hi_ok);
  }
}

// The lane's 16 encoded bytes for epoch `seq` from its raw input words.
template <int P>
__device__ __forceinline__ u32x4 encode_words(const uint32_t w[4], int lane,
                                              uint32_t seq) {
  u32x4 v;
  if (P == kLL) {
    // two LL words: data then flag, each single-copy atomic on its own
    v.x = w[0]; v.y = seq; v.z = w[1]; v.w = seq;
  } else if (P == kLL128) {
    if ((lane & 7) == 7) {
      v.x = w[0]; v.y = w[1]; v.z = seq; v.w = 0u;   // last data + u64 flag
    } else {
      v.x = w[0]; v.y = w[1]; v.z = w[2]; v.w = w[3];
    }
  } else if (P == kSentinel) {
    v.x = canon_word(w[0]); v.y = canon_word(w[1]);
    v.z = canon_word(w[2]); v.w = canon_word(w[3]);
  } else {
    v.x = w[0]; v.y = w[1]; v.z = w[2]; v.w = w[3];
  }
  return v;
}

template <int P>
__device__ __forceinline__ u32x4 encode_chunk(const uint16_t* __restrict__ row,
                                              uint32_t row_bytes, int64_t count,
                                              int tile, int lane, uint32_t seq) {
  uint32_t w[4];
  load_chunk<P>(row, row_bytes, tile, lane, w);
  mask_words(w, chunk_keep<P>(count, tile, lane));
  return encode_words<P>(w, lane, seq);
}

// Store one encoded tile chunk into `ncons` receive buffers at slot offsets
// dst0, dst0 + cstride, ..., except buffer `skip` (the producer's own: its
// consumer takes the value from registers; -1 = none).  For LL128 only the
// data part is stored here; the flags follow an ordering point
// (produce_flags).  The data store still covers the whole 128-byte line: the
// flag field is written with the stale value of two ops before (seq - 2),
// which a consumer reads as "not yet", so the line goes out as two full
// 64-byte sectors; an 8-byte tail would be a second partial write of the
// sector that the flag store writes again.
template <int P>
__device__ __forceinline__ void store_chunk(rsrc_t rs, uint32_t dst0,
                                            uint32_t cstride, int ncons,
                                            int skip, int tile, uint32_t E,
                                            int lane, u32x4 v) {
  const uint32_t loff = (uint32_t)tile * kTileBytes + (uint32_t)lane * 16u;
  if (loff >= E) return;
  if (P == kLL128 && (lane & 7) == 7) {
    const u32x4 d = u32x4{v.x, v.y, seq_prev(seq_prev(v.z)), 0u};   // v.z = seq
    for (int c = 0; c < ncons; ++c)
      if (c != skip) st16(rs, dst0 + c * cstride + loff, d);
  } else {
    for (int c = 0; c < ncons; ++c)
      if (c != skip) st16(rs, dst0 + c * cstride + loff, v);
  }
}

template <int P>
__device__ __forceinline__ void produce_data(rsrc_t rs, uint32_t dst0,
                                             uint32_t cstride, int ncons,
                                             int skip,
                                             const uint16_t* __restrict__ row,
                                             uint32_t row_bytes, int64_t count,
                                             int tile, uint32_t E, uint32_t seq,
                                             int lane) {
  const uint32_t loff = (uint32_t)tile * kTileBytes + (uint32_t)lane * 16u;
  if (loff >= E) return;
  store_chunk<P>(rs, dst0, cstride, ncons, skip, tile, E, lane,
                 encode_chunk<P>(row, row_bytes, count, tile, lane, seq));
}

// LL128 second phase: the u64 line flags (lane 7 of each line).
__device__ __forceinline__ void produce_flags(rsrc_t rs, uint32_t dst0,
                                              uint32_t cstride, int ncons,
                                              int skip, int tile, uint32_t E,
                                              uint32_t seq, int lane) {
  const uint32_t loff = (uint32_t)tile * kTileBytes + (uint32_t)lane * 16u;
  if (loff >= E || (lane & 7) != 7) return;
  u32x2 f;
  f.x = seq; f.y = 0u;
  for (int c = 0; c < ncons; ++c)
    if (c != skip) st8(rs, dst0 + c * cstride + loff + 8u, f);
}

// ----------------------------------------------------------- consumer ---

// Per-lane readiness of one 16-byte chunk: ok = delivered for epoch seq;
// bad = holds a flag that is neither seq, the stale seq of two ops before,
// nor 0 (never written).
template <int P>
__device__ __forceinline__ void classify(const u32x4 v, uint32_t seq,
                                         uint32_t stale, bool& ok, bool& bad) {
  if (P == kLL) {
    ok = (v.y == seq) && (v.w == seq);
    const bool b1 = v.y != seq && v.y != stale && v.y != 0u;
    const bool b2 = v.w != seq && v.w != stale && v.w != 0u;
    bad = b1 || b2;
  } else if (P == kSentinel) {
    ok = word_delivered(v.x) && word_delivered(v.y) && word_delivered(v.z) &&
         word_delivered(v.w);
    bad = false;
  } else {
    ok = true;
    bad = false;
  }
}

// Poll and validate one tile of every rank's slot for one consumer, in
// whatever order the blocks arrive; the validated 16-byte chunks end in
// v[0..nranks).  `src0` is the byte offset of slot 0 of this consumer and
// parity; slot r is at src0 + r*slot_bytes.  Rank `own` (-1 = none) is not
// polled: its chunk is `own_v`, already in registers.  SENTINEL with `rearm`
// stores the sentinel back over every chunk it has read.  Returns 0,
// kEtimeout or kEcorrupt.
//
// Two phases.  (1) Probe: lane r polls one 16-byte probe of rank r -- the
// last chunk of the tile, which the producer wave writes in the same store
// instruction as the rest -- so one load per iteration watches every rank
// and the polling traffic stays off the lines still being written.
// (2) Read: once every probe holds readiness evidence, every pending rank's
// whole chunk is read and validated from its own evidence; chunks not yet
// complete are read again.  Correctness rests on phase 2 alone.
// LL128: the probe is the flag of the tile's last line; the producer stored
// every data byte of its wave (and waited for the stores to complete) before
// any flag, so phase 2 reads data issued after a flag was seen.
template <int P, int NMAX>
__device__ __forceinline__ int poll_tile(rsrc_t rs, uint32_t src0,
                                         uint32_t slot_bytes, int nranks,
                                         int tile, uint32_t E, uint32_t seq,
                                         uint32_t stale, bool rearm, int own,
                                         u32x4 own_v, int* ctrl,
                                         uint64_t timeout_ticks, int lane,
                                         u32x4 (&v)[NMAX]) {
  const uint32_t tile0 = (uint32_t)tile * kTileBytes;
  const uint32_t loff = tile0 + (uint32_t)lane * 16u;
  const bool active = loff < E;
  uint32_t pending = (1u << nranks) - 1u;   // wave-uniform set of ranks
#pragma unroll
  for (int r = 0; r < NMAX; ++r) {
    v[r] = u32x4{0u, 0u, 0u, 0u};
    if (r == own) {
      v[r] = own_v;
      pending &= ~(1u << r);
    }
  }
  if (pending == 0u) return 0;
  Waiter wt(timeout_ticks, ctrl);

  // ---- phase 1: one probe per rank, lane r watches rank r ----
  if (P != kBarrier) {
    const uint32_t tile_end = (tile0 + kTileBytes < E) ? tile0 + kTileBytes : E;
    const uint32_t probe = tile_end - 16u;   // last chunk of the tile
    uint32_t waiting = pending;
    while (true) {
      const bool mine = lane < nranks && ((waiting >> lane) & 1u);
      bool ok = true, bad = false;
      if (mine) {
        const uint32_t at = src0 + (uint32_t)lane * slot_bytes + probe;
        if (P == kLL128) {
          const u32x2 f = ld8(rs, at + 8u);
          ok = (f.x == seq) && (f.y == 0u);
          bad = !ok && !(f.y == 0u && (f.x == 0u || f.x == stale));
        } else {
          classify<P>(ld16(rs, at), seq, stale, ok, bad);
        }
      }
      if (__ballot(bad) != 0ull) {
        if (lane == 0) report_error(ctrl, kEcorrupt);
        return kEcorrupt;
      }
      waiting &= ~(uint32_t)__ballot(mine && ok);
      if (waiting == 0u) break;
      if (!wt.again(lane)) return kEtimeout;
    }
    if (P == kLL128) fence_acquire();
  }

  // ---- phase 2: read and validate every pending rank's whole chunk ----
  while (true) {
#pragma unroll
    for (int r = 0; r < NMAX; ++r)
      if (r < nranks && ((pending >> r) & 1u) && active)
        v[r] = ld16(rs, src0 + r * slot_bytes + loff);
    uint32_t fresh = 0u;
    bool corrupt = false;
#pragma unroll
    for (int r = 0; r < NMAX; ++r) {
      if (r < nranks && ((pending >> r) & 1u)) {
        bool ok = true, bad = false;
        if (active) {
          if (P == kLL128) {
            if ((lane & 7) == 7) {
              ok = (v[r].z == seq) && (v[r].w == 0u);
              bad = !ok && !(v[r].w == 0u && (v[r].z == 0u || v[r].z == stale));
            }
          } else {
            classify<P>(v[r], seq, stale, ok, bad);
          }
        }
        if (__ballot(bad) != 0ull) corrupt = true;
        if (__ballot(!ok) == 0ull) fresh |= 1u << r;
      }
    }
    if (corrupt) {
      if (lane == 0) report_error(ctrl, kEcorrupt);
      return kEcorrupt;
    }
    if (P == kSentinel && rearm && fresh != 0u) {
      const u32x4 armed = u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu,
                                0xFFFFFFFFu};
#pragma unroll
      for (int r = 0; r < NMAX; ++r)
        if (r < nranks && ((fresh >> r) & 1u) && active)
          st16(rs, src0 + r * slot_bytes + loff, armed);
    }
    pending &= ~fresh;
    if (pending == 0u) break;
    if (!wt.again(lane)) return kEtimeout;
  }
  return 0;
}

// Poll and validate one rank's chunk (the lane's 16 bytes at byte offset
// `at`) until the whole wave's chunk carries evidence for epoch `seq`.
// SENTINEL with `rearm` stores the sentinel back over it once read.
// Returns 0, kEtimeout or kEcorrupt; the chunk ends in `v`.
template <int P>
__device__ __forceinline__ int poll_chunk(rsrc_t rs, uint32_t at, bool active,
                                          uint32_t seq, uint32_t stale,
                                          bool rearm, int* ctrl,
                                          uint64_t timeout_ticks, int lane,
                                          u32x4& v) {
  v = u32x4{0u, 0u, 0u, 0u};
  Waiter wt(timeout_ticks, ctrl);
  if (P == kLL128) {
    // Flags first (lane 7 of each line), data only after a flag was seen:
    // the producer's data stores all completed before its first flag store.
    const bool flag_lane = active && (lane & 7) == 7;
    while (true) {
      bool ok = true, bad = false;
      if (flag_lane) {
        const u32x2 f = ld8(rs, at + 8u);
        ok = (f.x == seq) && (f.y == 0u);
        bad = !ok && !(f.y == 0u && (f.x == 0u || f.x == stale));
      }
      if (__ballot(bad) != 0ull) {
        if (lane == 0) report_error(ctrl, kEcorrupt);
        return kEcorrupt;
      }
      if (__ballot(!ok) == 0ull) break;
      if (!wt.again(lane)) return kEtimeout;
    }
    fence_acquire();
    if (active) v = ld16(rs, at);
    return 0;
  }
  while (true) {
    if (active) v = ld16(rs, at);
    bool ok = true, bad = false;
    if (active) classify<P>(v, seq, stale, ok, bad);
    if (__ballot(bad) != 0ull) {
      if (lane == 0) report_error(ctrl, kEcorrupt);
      return kEcorrupt;
    }
    if (__ballot(!ok) == 0ull) break;
    if (!wt.again(lane)) return kEtimeout;
  }
  if (P == kSentinel && rearm && active)
    st16(rs, at, u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu});
  return 0;
}

// Poll up to B chunks of one peer at once (nb <= B of them in use): every
// round issues the loads of all chunks still missing before waiting on any,
// so a wave that owns several tiles pays one poll latency, not one per tile.
// Same checks, order and re-arm as poll_chunk.
template <int P, int B>
__device__ __forceinline__ int poll_chunks(rsrc_t rs, const uint32_t (&at)[B],
                                           const bool (&active)[B], int nb,
                                           uint32_t seq, uint32_t stale,
                                           bool rearm, int* ctrl,
                                           uint64_t timeout_ticks, int lane,
                                           u32x4 (&v)[B]) {
  bool done[B];
#pragma unroll
  for (int j = 0; j < B; ++j) {
    v[j] = u32x4{0u, 0u, 0u, 0u};
    done[j] = j >= nb;                              // wave-uniform
  }
  Waiter wt(timeout_ticks, ctrl);
  if (P == kLL128) {
    const bool flag_lane = (lane & 7) == 7;
    u32x2 f[B];
    while (true) {
#pragma unroll
      for (int j = 0; j < B; ++j)
        if (!done[j] && flag_lane && active[j]) f[j] = ld8(rs, at[j] + 8u);
      bool all = true;
#pragma unroll
      for (int j = 0; j < B; ++j) {
        if (done[j]) continue;
        bool ok = true, bad = false;
        if (flag_lane && active[j]) {
          ok = (f[j].x == seq) && (f[j].y == 0u);
          bad = !ok && !(f[j].y == 0u && (f[j].x == 0u || f[j].x == stale));
        }
        if (__ballot(bad) != 0ull) {
          if (lane == 0) report_error(ctrl, kEcorrupt);
          return kEcorrupt;
        }
        if (__ballot(!ok) == 0ull) done[j] = true;
        else all = false;
      }
      if (all) break;
      if (!wt.again(lane)) return kEtimeout;
    }
    fence_acquire();
#pragma unroll
    for (int j = 0; j < B; ++j)
      if (j < nb && active[j]) v[j] = ld16(rs, at[j]);
    return 0;
  }
  while (true) {
#pragma unroll
    for (int j = 0; j < B; ++j)
      if (!done[j] && active[j]) v[j] = ld16(rs, at[j]);
    bool all = true;
#pragma unroll
    for (int j = 0; j < B; ++j) {
      if (done[j]) continue;
      bool ok = true, bad = false;
      if (active[j]) classify<P>(v[j], seq, stale, ok, bad);
      if (__ballot(bad) != 0ull) {
        if (lane == 0) report_error(ctrl, kEcorrupt);
        return kEcorrupt;
      }
      if (__ballot(!ok) == 0ull) done[j] = true;
      else all = false;
    }
    if (all) break;
    if (!wt.again(lane)) return kEtimeout;
  }
  if (P == kSentinel && rearm) {
#pragma unroll
    for (int j = 0; j < B; ++j)
      if (j < nb && active[j])
        st16(rs, at[j], u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu});
  }
  return 0;
}

// LL128, many tiles per wave: every data store of a producer wave in an op
// completes before the first of its flag stores, so one flag of that wave
// seen for epoch `seq` makes all its data of the op readable.  Lane r (<
// nranks, r != own) polls the last line flag of tile `tile` of rank r until
// it holds seq; the caller then reads data with read_tiles.  Returns 0,
// kEtimeout or kEcorrupt.
__device__ __forceinline__ int probe_line_flags(rsrc_t rs, uint32_t src0,
                                                uint32_t slot_bytes, int nranks,
                                                int tile, uint32_t E, uint32_t seq,
                                                uint32_t stale, int own, int* ctrl,
                                                uint64_t timeout_ticks, int lane) {
  const uint32_t tile0 = (uint32_t)tile * kTileBytes;
  const uint32_t tile_end = (tile0 + kTileBytes < E) ? tile0 + kTileBytes : E;
  const uint32_t flag_at = tile_end - 8u;      // u64 flag of the tile's last line
  uint32_t waiting = ((1u << nranks) - 1u) & ~(own >= 0 ? 1u << own : 0u);
  Waiter wt(timeout_ticks, ctrl);
  while (waiting != 0u) {
    const bool mine = lane < nranks && ((waiting >> lane) & 1u);
    bool ok = true, bad = false;
    if (mine) {
      const u32x2 f = ld8(rs, src0 + (uint32_t)lane * slot_bytes + flag_at);
      ok = (f.x == seq) && (f.y == 0u);
      bad = !ok && !(f.y == 0u && (f.x == 0u || f.x == stale));
    }
    if (__ballot(bad) != 0ull) {
      if (lane == 0) report_error(ctrl, kEcorrupt);
      return kEcorrupt;
    }
    waiting &= ~(uint32_t)__ballot(mine && ok);
    if (waiting == 0u) break;
    if (!wt.again(lane)) return kEtimeout;
  }
  fence_acquire();
  return 0;
}

// Read and validate tiles tile[0..nb) of every rank's slot at once, every
// chunk checked from its own evidence, for a wave that owns many tiles (the
// large-payload case).  All chunks of the batch are loaded in one round, so a
// batch whose data has already arrived costs one memory round trip; chunks
// not yet complete are read again.  Rank `own` (-1 = none) is not read: its
// chunks are own_v[j].  SENTINEL with `rearm` stores the sentinel back over
// every chunk once read.  LL128: call after probe_line_flags for the same
// producers; the line flags are then checked here as the readiness evidence.
// Returns 0, kEtimeout or kEcorrupt; chunk (j, r) ends in v[j][r].
template <int P, int NMAX, int CB>
__device__ __forceinline__ int read_tiles(rsrc_t rs, uint32_t src0, uint32_t slot_bytes,
                                          int nranks, const int (&tile)[CB], int nb,
                                          uint32_t E, uint32_t seq, uint32_t stale,
                                          bool rearm, int own, const u32x4 (&own_v)[CB],
                                          int* ctrl, uint64_t timeout_ticks, int lane,
                                          u32x4 (&v)[CB][NMAX]) {
  uint32_t pending[CB];
  uint32_t loff[CB];
  bool active[CB];
  const uint32_t all = ((1u << nranks) - 1u) & ~(own >= 0 ? 1u << own : 0u);
  bool any = false;
#pragma unroll
  for (int j = 0; j < CB; ++j) {
    loff[j] = (uint32_t)tile[j] * kTileBytes + (uint32_t)lane * 16u;
    active[j] = j < nb && loff[j] < E;
    pending[j] = j < nb ? all : 0u;
    any = any || pending[j] != 0u;
#pragma unroll
    for (int r = 0; r < NMAX; ++r)
      v[j][r] = (r == own) ? own_v[j] : u32x4{0u, 0u, 0u, 0u};
  }
  if (!any) return 0;
  Waiter wt(timeout_ticks, ctrl);
  while (true) {
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
      for (int r = 0; r < NMAX; ++r)
        if (r < nranks && ((pending[j] >> r) & 1u) && active[j])
          v[j][r] = ld16(rs, src0 + r * slot_bytes + loff[j]);
    bool corrupt = false, left = false;
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      uint32_t fresh = 0u;
#pragma unroll
      for (int r = 0; r < NMAX; ++r) {
        if (r < nranks && ((pending[j] >> r) & 1u)) {
          bool ok = true, bad = false;
          if (active[j]) {
            if (P == kLL128) {
              if ((lane & 7) == 7) {
                ok = (v[j][r].z == seq) && (v[j][r].w == 0u);
                bad = !ok && !(v[j][r].w == 0u && (v[j][r].z == 0u || v[j][r].z == stale));
              }
            } else {
              classify<P>(v[j][r], seq, stale, ok, bad);
            }
          }
          if (__ballot(bad) != 0ull) corrupt = true;
          if (__ballot(!ok) == 0ull) fresh |= 1u << r;
        }
      }
      if (P == kSentinel && rearm && fresh != 0u) {
#pragma unroll
        for (int r = 0; r < NMAX; ++r)
          if (r < nranks && ((fresh >> r) & 1u) && active[j])
            st16(rs, src0 + r * slot_bytes + loff[j],
                 u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu});
      }
      pending[j] &= ~fresh;
      left = left || pending[j] != 0u;
    }
    if (corrupt) {
      if (lane == 0) report_error(ctrl, kEcorrupt);
      return kEcorrupt;
    }
    if (!left) break;
    if (!wt.again(lane)) return kEtimeout;
  }
  return 0;
}

// Fixed rank order: start from rank 0, add ranks 1..N-1 one binary32
// addition at a time, round to bf16 (NaN -> 0x7FC0), store the lane's
// elements of tile `tile` below `count`.
template <int P, int NMAX>
__device__ __forceinline__ void reduce_words(const u32x4 (&v)[NMAX], int nranks,
                                             uint32_t o[4]) {
  float acc[8];
  {
    const u32x4 d = v[0];
    if (P == kLL) {
      acc[0] = bf_lo(d.x); acc[1] = bf_hi(d.x);
      acc[2] = bf_lo(d.z); acc[3] = bf_hi(d.z);
    } else {
      acc[0] = bf_lo(d.x); acc[1] = bf_hi(d.x);
      acc[2] = bf_lo(d.y); acc[3] = bf_hi(d.y);
      acc[4] = bf_lo(d.z); acc[5] = bf_hi(d.z);
      acc[6] = bf_lo(d.w); acc[7] = bf_hi(d.w);
    }
  }
#pragma unroll
  for (int r = 1; r < NMAX; ++r) {
    if (r < nranks) {
      const u32x4 d = v[r];
      if (P == kLL) {
        acc[0] += bf_lo(d.x); acc[1] += bf_hi(d.x);
        acc[2] += bf_lo(d.z); acc[3] += bf_hi(d.z);
      } else {
        acc[0] += bf_lo(d.x); acc[1] += bf_hi(d.x);
        acc[2] += bf_lo(d.y); acc[3] += bf_hi(d.y);
        acc[4] += bf_lo(d.z); acc[5] += bf_hi(d.z);
        acc[6] += bf_lo(d.w); acc[7] += bf_hi(d.w);
      }
    }
  }
  if (P == kLL) {
    o[0] = pack2(to_bf16(acc[0]), to_bf16(acc[1]));
    o[1] = pack2(to_bf16(acc[2]), to_bf16(acc[3]));
    o[2] = 0u; o[3] = 0u;
  } else {
    o[0] = pack2(to_bf16(acc[0]), to_bf16(acc[1]));
    o[1] = pack2(to_bf16(acc[2]), to_bf16(acc[3]));
    o[2] = pack2(to_bf16(acc[4]), to_bf16(acc[5]));
    o[3] = pack2(to_bf16(acc[6]), to_bf16(acc[7]));
  }
}

template <int P, int NMAX>
__device__ __forceinline__ void reduce_store_tile(const u32x4 (&v)[NMAX],
                                                  int nranks, int tile,
                                                  uint32_t E, int lane,
                                                  uint16_t* __restrict__ out_row,
                                                  int64_t count) {
  const uint32_t loff = (uint32_t)tile * kTileBytes + (uint32_t)lane * 16u;
  if (loff >= E) return;
  uint32_t o[4];
  reduce_words<P, NMAX>(v, nranks, o);
  int64_t first;
  int n;
  lane_elems<P>(tile, lane, first, n);
  store_elems(out_row, count, first, n, o);
}

// The data words of one validated 16-byte chunk (the inverse of
// encode_words up to the NaN canonicalization of SENTINEL).
template <int P>
__device__ __forceinline__ void chunk_words(const u32x4 v, uint32_t w[4]) {
  if (P == kLL) {
    w[0] = v.x; w[1] = v.z; w[2] = 0u; w[3] = 0u;
  } else {
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;   // LL128 lane 7: 4 elements
  }
}

// Decode one validated chunk of tile `tile` and store its elements below
// `count` into out_row (element 0 of the encoding at out_row[0]).
template <int P>
__device__ __forceinline__ void store_chunk_elems(uint16_t* __restrict__ out_row,
                                                  int64_t count, int tile,
                                                  uint32_t E, int lane, u32x4 v) {
  const uint32_t loff = (uint32_t)tile * kTileBytes + (uint32_t)lane * 16u;
  if (loff >= E) return;
  uint32_t w[4];
  chunk_words<P>(v, w);
  int64_t first;
  int n;
  lane_elems<P>(tile, lane, first, n);
  store_elems(out_row, count, first, n, w);
}

// Encoded bytes of `count` elements (the slot layout of ar_encoded_bytes).
template <int P>
__device__ __forceinline__ uint32_t enc_bytes(int64_t count) {
  if (P == kLL) return (uint32_t)(16 * ((count + 3) / 4));
  if (P == kLL128) return (uint32_t)(128 * ((count + 59) / 60));
  return (uint32_t)(16 * ((count + 7) / 8));
}

// Poll, validate and reduce one tile for one consumer (all ranks polled).
template <int P, int NMAX>
__device__ __forceinline__ int consume_tile(
    rsrc_t rs, uint32_t src0, uint32_t slot_bytes, int nranks, int tile,
    uint32_t E, uint32_t seq, uint32_t stale, bool rearm,
    uint16_t* __restrict__ out_row, int64_t count, int* ctrl,
    uint64_t timeout_ticks, int lane) {
  u32x4 v[NMAX];
  const int st = poll_tile<P, NMAX>(rs, src0, slot_bytes, nranks, tile, E, seq,
                                    stale, rearm, -1, u32x4{0u, 0u, 0u, 0u},
                                    ctrl, timeout_ticks, lane, v);
  if (st) return st;
  reduce_store_tile<P, NMAX>(v, nranks, tile, E, lane, out_row, count);
  return 0;
}

}  // namespace ar
