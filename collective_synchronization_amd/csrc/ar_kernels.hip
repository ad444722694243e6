// ar_kernels.hip -- HIP kernels (gfx950) and the C-ABI entry points of the
// self-synchronizing small-message one-shot bf16 all-reduce.
//
// Build: hipcc --offload-arch=gfx950 -O3 -fPIC -shared
//        -fno-gpu-flush-denormals-to-zero -ffp-contract=off
//        -Xclang -target-feature -Xclang -packed-fp32-ops
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "../../include/ar.h"
#include "../../include/ar_dev.h"
#include "ar_host.h"
#include "../../include/ar_protocols.h"

namespace ar {

// Waves per workgroup of the simulator.  One wave per workgroup spreads a
// rank's waves over as many CUs as possible: each CU's path to the L2 then
// carries one wave's write-through stores instead of four.
#ifndef AR_SIM_WAVES_PER_BLOCK
#define AR_SIM_WAVES_PER_BLOCK 1
#endif
constexpr int kSimWPB = AR_SIM_WAVES_PER_BLOCK;
constexpr int kSimBlock = kSimWPB * kWave;
constexpr int kSimWavesPerQ = 8 * kSimWPB;    // waves of one rank per Q step

// ================================================================ kernels ==

struct PackArgs {
  const uint16_t* in;
  int64_t in_stride;
  int64_t count;
  const uint8_t* scratch;
  uint32_t scratch_bytes;
  uint32_t E, slot_bytes;
  int32_t nranks, nconsumers, tiles;
  uint32_t seq, parity;
};

// One wave per (rank, tile): encode and broadcast to every consumer's buffer
// (the device-callable interface of ar_dev.h).
template <int P>
__global__ __launch_bounds__(kBlock) void k_pack(PackArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int r = gw / a.tiles;
  const int tile = gw - r * a.tiles;
  if (r >= a.nranks) return;
  const ar_dev::buffer b = ar_dev::make(a.scratch, a.scratch_bytes, a.slot_bytes, a.E,
                                      a.nranks, a.nconsumers, a.count, a.seq, a.parity);
  uint32_t w[4];
  load_chunk<P>(a.in + (int64_t)r * a.in_stride,
                (uint32_t)(((a.count * 2) + 15) & ~int64_t(15)), tile, lane, w);
  mask_words(w, chunk_keep<P>(a.count, tile, lane));
  ar_dev::broadcast<P>(b, r, tile, lane, w);
  if (P == kLL128) {
    ar_dev::fence();
    ar_dev::broadcast_flags(b, r, tile, lane);
  }
}

struct ReduceArgs {
  uint16_t* out;
  int64_t out_stride;
  int64_t count;
  const uint8_t* scratch;
  uint32_t scratch_bytes;
  uint32_t E, slot_bytes;
  int32_t nranks, nconsumers, tiles;
  uint32_t seq, parity;
  int* ctrl;
  uint64_t timeout_ticks;
  int32_t rearm;
};

// One wave per (consumer, tile): poll, validate, reduce in rank order.
template <int P, int NMAX>
__global__ __launch_bounds__(kBlock) void k_reduce(ReduceArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int c = gw / a.tiles;
  const int tile = gw - c * a.tiles;
  if (c >= a.nconsumers) return;
  const ar_dev::buffer b = ar_dev::make(a.scratch, a.scratch_bytes, a.slot_bytes, a.E,
                                      a.nranks, a.nconsumers, a.count, a.seq, a.parity);
  ar_dev::recv_reduce<P, NMAX>(b, c, tile, lane, a.rearm != 0, a.ctrl, a.timeout_ticks,
                               a.out + (int64_t)c * a.out_stride);
}

// Fill byte range [begin, begin+bytes) of the buffer with 0xFF, 16 bytes a
// lane, with device-scope coherent stores.
__global__ __launch_bounds__(kBlock) void k_arm(const uint8_t* scratch,
                                                uint32_t scratch_bytes,
                                                uint32_t region0,
                                                uint32_t region_stride,
                                                uint32_t region_bytes,
                                                int32_t nregions) {
  const rsrc_t rs = make_rsrc(scratch, scratch_bytes);
  const u32x4 armed = u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
  const uint64_t chunks = region_bytes / 16u;
  const uint64_t total = chunks * (uint64_t)nregions;
  for (uint64_t i = (uint64_t)blockIdx.x * kBlock + threadIdx.x; i < total;
       i += (uint64_t)gridDim.x * kBlock) {
    const uint32_t reg = (uint32_t)(i / chunks);
    const uint32_t k = (uint32_t)(i - (uint64_t)reg * chunks);
    st16(rs, region0 + reg * region_stride + k * 16u, armed);
  }
}

__global__ __launch_bounds__(kBlock) void k_fill_zero(uint32_t* p, uint32_t words) {
  for (uint32_t i = blockIdx.x * kBlock + threadIdx.x; i < words;
       i += gridDim.x * kBlock)
    __hip_atomic_store(p + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------- simulator --

// The barrier baseline's counter of wave index wr sits at progress word
// (wr % 128) * 32 + wr / 128, a permutation of the progress words.
static_assert(kCtrlMaxProgress == 128 * 32, "counter layout covers the progress words");

struct SimArgs {
  const uint16_t* in;
  int64_t in_stride;
  uint16_t* out;
  int64_t out_stride;
  const uint8_t* scratch;
  uint32_t scratch_bytes;
  int* ctrl;
  int64_t count;
  uint32_t E, slot_bytes;
  int32_t nranks, nconsumers, nops;
  int32_t W, Q, T, TPW;
  uint32_t seq0, parity0;
  uint64_t timeout_ticks;
  const uint32_t* delay;
  const uint16_t* order;
  uint64_t* trace;
};

__device__ __forceinline__ bool wait_geq(const uint32_t* p, uint32_t target,
                                         Waiter& wt, int lane) {
  while (ld_agent_u32(p) < target)
    if (!wt.again(lane)) return false;
  return true;
}

// Persistent role-split kernel.  Workgroups are dispatched round robin over
// the eight XCDs: workgroup b sits on XCD (s + b) % 8, with a start s that
// depends on earlier dispatches, so only b % 8 matters for which workgroups
// share an XCD.  Rank g owns Q workgroups per XCD; its wave index wr (0..W-1)
// is rotated by g so that the producer of a tile and the consumer that
// reads it sit on different XCDs, and the same wr owns the same tiles
// {wr, wr + W, ...} in every rank.
//
// A rank's own contribution never goes through memory: its consumer takes
// the encoded chunk from registers and its producer skips its own buffer.
// ONE: every wave owns at most one tile (the small-message case; not the
// barrier baseline).  The op loop is then software-pipelined: the next op's
// payload is loaded while this op is polled, and this op's output is stored
// after the next op's stores are out, so neither input load nor output store
// sits between one op's validation and the next op's transmission.
// Otherwise (many tiles per wave, the large-payload case) a wave sends all
// its tiles, then receives them kReadBatch at a time: every chunk of a batch
// is loaded in one round, so a batch whose data has arrived costs one memory
// round trip (LL128: plus one flag probe per op, see probe_line_flags).  The
// two variants are separate kernels so that neither carries the other's
// registers.
// EXTRAS: the launch uses producer delays, a tile order or a trace.  The
// variant without them drops those paths at compile time: less code and
// fewer scalar registers in the op loop (8 ranks [1,4096]: 4.5% faster per
// op in the workgroup kernel, 9% at 16 ranks).
template <int P, int NMAX, bool SHARE, bool EXTRAS, bool ONE>
__global__ __launch_bounds__(kSimBlock) void k_sim(SimArgs a) {
  constexpr bool kFast = ONE && P != kBarrier;
  // (Measured for the barrier baseline, not adopted: 4 tiles a round at 8
  // ranks, 4 MiB 93.8 -> 90.4 us per op, but 202 vector registers instead of
  // 109 halve the occupancy, so the launch turns cooperative, and one-tile
  // sizes lose 4.5 -> 5.6 us.)
  constexpr int kReadBatch = NMAX <= 4 ? 4 : (NMAX <= 8 ? 2 : 1);
  if constexpr (!EXTRAS) {
    a.delay = nullptr;
    a.order = nullptr;
    a.trace = nullptr;
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.x;
  const int x = b & 7;
  const int q = b >> 3;
  const int g = q / a.Q;
  const int qq = q - g * a.Q;
  if (g >= a.nranks) return;
  const int rot = SHARE ? (g == 0 ? 0 : 1 + (g - 1) % 7) : (g & 7);
  const int xr = (x - rot) & 7;
  const int wr = (qq * 8 + xr) * kSimWPB + wave;
  if (wr >= a.T) return;
  // tiles of this wave (1 in the one-tile variant: T <= W there)
  const int mine = kFast ? 1 : (a.T - 1 - wr) / a.W + 1;
  const bool consumer = SHARE ? (g == 0) : true;
  const int cself = SHARE ? 0 : g;
  const int skip = consumer ? cself : -1;       // own buffer, fed from registers

  const rsrc_t rs = make_rsrc(a.scratch, a.scratch_bytes);
  const uint32_t N = (uint32_t)a.nranks;
  const uint32_t cstride = 2u * N * a.slot_bytes;
  uint32_t* const progress = reinterpret_cast<uint32_t*>(a.ctrl) + kCtrlProgress;
  // Barrier baseline: one counter per wave index.  Waves wr of the N ranks
  // are the only producers of the tiles that waves wr of the consumers read
  // (the same tiles in every rank), so the top and bottom barriers are kept
  // among those waves: per op the counter takes N producer arrivals, then
  // the nconsumers completions (each waits for all N arrivals first, and the
  // next arrivals wait for all completions), so op i's arrivals are complete
  // at i*K + N and its completions at (i+1)*K.  (The progress words are
  // otherwise unused by this protocol; the control block is zero at launch.)
  // Counters of neighbouring wave indices sit 128 bytes apart (a line each
  // up to 128 indices): adjacent counters in one line made every group's
  // atomics and polls contend (measured, 8 ranks: 8 KiB 9.4 -> 4.5 us per
  // op, 4 MiB 121 -> 98 us).  wr < 4096, so the index stays below 4096.
  uint32_t* const bar = progress + ((wr & 127) * 32 + (wr >> 7));
  const uint32_t K = N + (uint32_t)a.nconsumers;
  const int tstride = 2 * a.nranks;
  const int64_t op_rows = a.nranks;

  if (a.trace && lane == 0)
    __hip_atomic_fetch_min(reinterpret_cast<unsigned long long*>(a.trace) +
                               (int64_t)a.nops * tstride,
                           (unsigned long long)now_ticks(), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);

  uint32_t wnext[4] = {0u, 0u, 0u, 0u};     // one-tile: next op's payload
  u32x4 v[NMAX];                            // one-tile: last validated op
  bool out_pending = false;
  const uint32_t row_bytes = (uint32_t)(((a.count * 2) + 15) & ~int64_t(15));
  const int keep = chunk_keep<P>(a.count, wr, lane);
  if (kFast) load_chunk<P>(a.in + (int64_t)g * a.in_stride, row_bytes, wr, lane, wnext);

  uint32_t seq = a.seq0;
  uint32_t par = a.parity0;
  for (int op = 0; op < a.nops; ++op) {
    const uint32_t stale = seq_prev(seq_prev(seq));
    const uint32_t pp = (P == kBarrier) ? 0u : par;

    // ---- licence to write this parity / bottom barrier of the baseline --
    if (P == kBarrier) {
      if (op >= 1) {
        Waiter wt(a.timeout_ticks, a.ctrl);
        if (!wait_geq(bar, (uint32_t)op * K, wt, lane)) return;
        fence_acquire();
      }
    } else if (SHARE && g != 0 && op >= 2) {
      // Rank 0's wave wr publishes seq when it starts an op, i.e. after it
      // finished reading (and re-arming) the parity this op overwrites.
      Waiter wt(a.timeout_ticks, a.ctrl);
      const uint32_t prev = seq_prev(seq);
      while (true) {
        const uint32_t pv = ld_agent_u32(progress + wr);
        if (pv == prev || pv == seq) break;
        if (!wt.again(lane)) return;
      }
      fence_acquire();
    }
    if (SHARE && g == 0 && P != kBarrier && lane == 0)
      st_agent_u32(progress + wr, seq);

    // ---- producer skew ----
    if (a.delay) {
      const uint32_t d = a.delay[(int64_t)op * a.nranks + g];
      if (d) {
        const uint64_t t0 = now_ticks();
        while (now_ticks() - t0 < (uint64_t)d) __builtin_amdgcn_s_sleep(2);
      }
    }

    // ---- produce(op): slot g of parity pp in every other consumer's buffer
    const uint16_t* row = a.in + ((int64_t)op * op_rows + g) * a.in_stride;
    const uint32_t dst0 = (pp * N + (uint32_t)g) * a.slot_bytes;
    u32x4 own_v = u32x4{0u, 0u, 0u, 0u};
    if constexpr (kFast) {
      mask_words(wnext, keep);
      own_v = encode_words<P>(wnext, lane, seq);
      store_chunk<P>(rs, dst0, cstride, a.nconsumers, skip, wr, a.E, lane, own_v);
      if (P == kLL128) {
        fence_release();
        produce_flags(rs, dst0, cstride, a.nconsumers, skip, wr, a.E, seq, lane);
      }
      if (out_pending) {   // previous op's output, now that this op is sent
        reduce_store_tile<P, NMAX>(
            v, a.nranks, wr, a.E, lane,
            a.out + ((int64_t)(op - 1) * a.nconsumers + cself) * a.out_stride, a.count);
        out_pending = false;
      }
      // unconditional: past the last op the range is empty and the load
      // reads nothing, so the loaded registers need no merge (and no wait)
      load_chunk<P>(row + op_rows * a.in_stride, op + 1 < a.nops ? row_bytes : 0u, wr, lane,
                    wnext);
    } else {
      const uint16_t* ord =
          a.order ? a.order + ((int64_t)op * a.nranks + g) * a.TPW : nullptr;
      // the loads of up to TB tiles in flight together, then their stores (a
      // tile past the payload reads nothing and stores nothing).  Measured:
      // 1-5% per op at 0.5-4 MiB for LL, LL128 and the sentinel; for the
      // barrier baseline, whose wave sends all its tiles between two
      // barriers, 4 tiles 4-6% and 8 tiles another 2-6% at 1-4 MiB (16 tiles
      // take more than 128 vector registers, which halves the occupancy).
      constexpr int TB = P == kBarrier ? 8 : 4;
      for (int j0 = 0; j0 < a.TPW; j0 += TB) {
        uint32_t wv[TB][4];
        int kk[TB];
#pragma unroll
        for (int i = 0; i < TB; ++i) {
          const int j = j0 + i;
          kk[i] = j < a.TPW ? (ord ? (int)ord[j] : j) : mine;
          load_chunk<P>(row, row_bytes, wr + kk[i] * a.W, lane, wv[i]);
        }
#pragma unroll
        for (int i = 0; i < TB; ++i) {
          if (kk[i] >= mine) continue;
          const int tile = wr + kk[i] * a.W;
          mask_words(wv[i], chunk_keep<P>(a.count, tile, lane));
          store_chunk<P>(rs, dst0, cstride, a.nconsumers, skip, tile, a.E, lane,
                         encode_words<P>(wv[i], lane, seq));
        }
      }
      if (P == kLL128) {
        fence_release();
        for (int k = 0; k < mine; ++k)
          produce_flags(rs, dst0, cstride, a.nconsumers, skip, wr + k * a.W, a.E,
                        seq, lane);
      }
      if (P == kBarrier) {
        fence_release();
        if (lane == 0)
          __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (a.trace) {
      fence_release();   // stores acknowledged before the timestamp
      if (lane == 0)
        __hip_atomic_fetch_max(
            reinterpret_cast<unsigned long long*>(a.trace) + (int64_t)op * tstride + g,
            (unsigned long long)now_ticks(), __ATOMIC_RELAXED,
            __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- consume(op) ----
    if (consumer) {
      const uint32_t src0 = ((uint32_t)cself * 2u + pp) * N * a.slot_bytes;
      if constexpr (kFast) {
        if (poll_tile<P, NMAX>(rs, src0, a.slot_bytes, a.nranks, wr, a.E, seq,
                               stale, true, g, own_v, a.ctrl, a.timeout_ticks,
                               lane, v) != 0)
          return;
        out_pending = true;
      } else {
        if (P == kBarrier) {
          Waiter wt(a.timeout_ticks, a.ctrl);
          if (!wait_geq(bar, (uint32_t)op * K + N, wt, lane)) return;
          fence_acquire();
        }
        uint16_t* orow = a.out + ((int64_t)op * a.nconsumers + cself) * a.out_stride;
        // Where an op's chunks fill half of the memory-side cache (the 256 MB
        // MALL) or more and a wave walks many tiles, read the tiles written
        // last first: they are the ones still cached.  Send order -> newest
        // first, us per op, one box: sentinel 8 ranks 4 MiB 132.8 -> 127.6,
        // 2 MiB 73.6 -> 68.1 (8 tiles a wave), 16 ranks 1 MiB 125.8 -> 121.9
        // (8), 512 KiB 64.9 -> 66.0 (4 tiles a wave); LL 8 ranks 4 MiB 209.3
        // -> 197.9 (32 tiles), 2 MiB 88.6 -> 88.3 (16), 16 ranks 1 MiB 200.7
        // -> 200.0 (16), 512 KiB 84.5 -> 86.4 (8); at 8 ranks 1 MiB (a
        // quarter of the cache) the send order is 1-1.5% faster.
        // (Not the barrier baseline, which reads only after the whole group's
        // sends: send order, 8 ranks 4 MiB 91.7 -> 91.0 us, 16 ranks 1 MiB
        // 90.6 -> 88.9.)
        const bool newest_first =
            P != kBarrier && a.TPW >= (P == kLL ? 16 : 8) &&
            (uint64_t)a.nconsumers * (uint64_t)a.nranks * a.E >= (uint64_t(128) << 20);
        // LL128: one flag per producer wave orders all of its data of the op
        if (P == kLL128 &&
            probe_line_flags(rs, src0, a.slot_bytes, a.nranks, wr, a.E, seq, stale, g,
                             a.ctrl, a.timeout_ticks, lane) != 0)
          return;
        for (int k0 = 0; k0 < mine; k0 += kReadBatch) {
          const int nb = (mine - k0) < kReadBatch ? (mine - k0) : kReadBatch;
          int tl[kReadBatch];
          uint32_t wv[kReadBatch][4];
          u32x4 ov[kReadBatch];
          // the rank's own chunks (input loads of the batch together)
#pragma unroll
          for (int j = 0; j < kReadBatch; ++j) {
            tl[j] = wr + (newest_first ? mine - 1 - (k0 + j) : k0 + j) * a.W;
            load_chunk<P>(row, j < nb ? row_bytes : 0u, tl[j], lane, wv[j]);
          }
#pragma unroll
          for (int j = 0; j < kReadBatch; ++j) {
            mask_words(wv[j], chunk_keep<P>(a.count, tl[j], lane));
            ov[j] = encode_words<P>(wv[j], lane, seq);
          }
          u32x4 vt[kReadBatch][NMAX];
          if (read_tiles<P, NMAX, kReadBatch>(rs, src0, a.slot_bytes, a.nranks, tl, nb, a.E,
                                              seq, stale, true, g, ov, a.ctrl,
                                              a.timeout_ticks, lane, vt) != 0)
            return;
#pragma unroll
          for (int j = 0; j < kReadBatch; ++j)
            if (j < nb)
              reduce_store_tile<P, NMAX>(vt[j], a.nranks, tl[j], a.E, lane, orow, a.count);
        }
        if (P == kBarrier) {
          fence_release();
          if (lane == 0)
            __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      // SENTINEL: the re-arm stores of this op complete before any store of
      // the next op (whose arrival licenses peers to refill this parity).
      // LL/LL128 read only: their loads have returned (the values were used).
      if (P == kSentinel) fence_release();
      if (a.trace && lane == 0)
        __hip_atomic_fetch_max(
            reinterpret_cast<unsigned long long*>(a.trace) + (int64_t)op * tstride +
                a.nranks + cself,
            (unsigned long long)now_ticks(), __ATOMIC_RELAXED,
            __HIP_MEMORY_SCOPE_AGENT);
    }
    seq = seq_next(seq);
    par ^= 1u;
  }
  if (out_pending)
    reduce_store_tile<P, NMAX>(
        v, a.nranks, wr, a.E, lane,
        a.out + ((int64_t)(a.nops - 1) * a.nconsumers + cself) * a.out_stride, a.count);
}

// Wide simulator for latency-bound sizes: one workgroup of nranks waves per
// (rank g, tile group tg); wave w is paired with peer w.  Wave w sends this
// rank's chunk to consumer w and, in a consumer, polls peer w's chunk, so
// every wave carries one store stream and one poll stream.  Per op, every
// wave first sends all tiles of its tile group, then the workgroup receives
// them tile by tile: validated chunks are staged in LDS (double-buffered by
// tile iteration) and, after one workgroup barrier, the wave of the rank
// itself (the "own" wave, whose contribution never leaves registers when
// the group holds one tile) reduces in fixed rank order.  With one tile per
// group in system mode, LL, a wave instead sends the next op right after its
// own receive, before that barrier (the first loop below).
// Sentinel: the wave that re-arms peer w's slot is the wave that next sends
// to peer w, so waiting for its own stores orders re-arm before refill.
// Share mode: only rank 0 consumes; a producer rank's workgroup keeps its
// wave 0, which takes the dual-buffer licence from rank 0's progress word.
// Placement: workgroup (g, tg) sits on XCD (s + tg + rot(g)) mod 8 as in k_sim.
// BATCH: tiles received per workgroup barrier (1 when every workgroup owns a
// single tile, 2 otherwise; the two chunks of a peer are polled together).
// EXTRAS: as for k_sim.
template <int P, int NMAX, bool SHARE, int BATCH, bool EXTRAS>
__global__ __launch_bounds__(1024) void k_sim_wide(SimArgs a) {
  if constexpr (!EXTRAS) {
    a.delay = nullptr;
    a.order = nullptr;
    a.trace = nullptr;
  }
  __shared__ u32x4 lds[2][BATCH][NMAX][kWave];
  __shared__ int lds_err;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x >> 6;
  const int b = blockIdx.x;
  const int x = b & 7;
  const int q = b >> 3;
  const int g = q / a.Q;
  const int qq = q - g * a.Q;
  if (g >= a.nranks) return;                       // whole workgroup
  const int rot = SHARE ? (g == 0 ? 0 : 1 + (g - 1) % 7) : (g & 7);
  const int tg = qq * 8 + ((x - rot) & 7);
  if (tg >= a.T) return;                           // whole workgroup
  const int G = a.W;
  // the one-tile variant is launched only when every group owns one tile
  const int mine = BATCH == 1 ? 1 : (a.T - 1 - tg) / G + 1;
  const bool consumer = SHARE ? (g == 0) : true;
  if (!consumer && w != 0) return;                 // producer-only rank: one wave
  const int cself = SHARE ? 0 : g;
  const bool sender = SHARE ? (g != 0) : (w != g);
  const int dst_c = SHARE ? 0 : w;
  const bool own = consumer && w == g;
  const bool poller = consumer && w != g;
  // The rank's own chunk is staged in LDS by the sender wave g+1, which
  // holds the same encoded chunk in registers, so that the own wave only
  // reduces and stays off the critical path.  Share mode and a single rank
  // have no sender wave in the consumer workgroup: there the own wave
  // stages it.
  const bool own_stages = SHARE || a.nranks == 1;
  const bool stager = own_stages ? own : (w == (g + 1) % a.nranks);

  const rsrc_t rs = make_rsrc(a.scratch, a.scratch_bytes);
  const uint32_t N = (uint32_t)a.nranks;
  uint32_t* const progress = reinterpret_cast<uint32_t*>(a.ctrl) + kCtrlProgress;
  const int tstride = 2 * a.nranks;
  const int64_t op_rows = a.nranks;
  const bool pipelined = BATCH == 1 || mine == 1;
  if (threadIdx.x == 0) lds_err = 0;
  if (consumer) __syncthreads();

  if (a.trace && lane == 0 && w == 0)
    __hip_atomic_fetch_min(reinterpret_cast<unsigned long long*>(a.trace) +
                               (int64_t)a.nops * tstride,
                           (unsigned long long)now_ticks(), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);

  uint32_t wnext[4] = {0u, 0u, 0u, 0u};
  const bool needs_input = sender || (own && own_stages);
  const uint32_t row_bytes = (uint32_t)(((a.count * 2) + 15) & ~int64_t(15));
  const int keep = chunk_keep<P>(a.count, tg, lane);
  if (pipelined && needs_input)
    load_chunk<P>(a.in + (int64_t)g * a.in_stride, row_bytes, tg, lane, wnext);

  // One tile per group in system mode, LL: wave w sends op i+1 to peer w as
  // soon as its own poll has validated peer w's op i, before the workgroup
  // barrier of op i.  Peer w sent op i only after it had consumed this
  // rank's op i-1, so the slot of op i+1's parity is free: the licence is
  // pairwise and needs no barrier, and the send overlaps the wait for the
  // other peers.  The sentinel and LL128 keep the general loop below: their
  // waits before a send (re-arm stores, data before flags) would then hold
  // every wave on its way to the barrier.  (A separate loop: folding this
  // order into the general one made the compiler spill scalar registers.)
  if constexpr (BATCH == 1 && !SHARE && P == kLL) {
    uint32_t seq = a.seq0;
    uint32_t par = a.parity0;
    int buf = 0;
    u32x4 own0 = u32x4{0u, 0u, 0u, 0u};   // encoded own chunk, for the stager
    // the send of op `opn` (epoch sq, buffer parity pr), then the load of
    // op opn+1's payload (an empty range past the last op)
    auto send_op = [&](int opn, uint32_t sq, uint32_t pr) {
      if (sender && a.delay) {
        const uint32_t d = a.delay[(int64_t)opn * a.nranks + g];
        if (d) {
          const uint64_t t0 = now_ticks();
          while (now_ticks() - t0 < (uint64_t)d) __builtin_amdgcn_s_sleep(2);
        }
      }
      if (!(sender || (own && own_stages))) return;
      mask_words(wnext, keep);
      own0 = encode_words<P>(wnext, lane, sq);
      if (sender) {
        const uint32_t dst0 = ((uint32_t)dst_c * 2u * N + pr * N + (uint32_t)g) * a.slot_bytes;
        store_chunk<P>(rs, dst0, 0u, 1, -1, tg, a.E, lane, own0);
        if (a.trace) {
          fence_release();
          if (lane == 0)
            __hip_atomic_fetch_max(
                reinterpret_cast<unsigned long long*>(a.trace) + (int64_t)opn * tstride + g,
                (unsigned long long)now_ticks(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      const uint16_t* next = a.in + ((int64_t)(opn + 1) * op_rows + g) * a.in_stride;
      load_chunk<P>(next, opn + 1 < a.nops ? row_bytes : 0u, tg, lane, wnext);
    };
    send_op(0, seq, par);
    for (int op = 0; op < a.nops; ++op) {
      const uint32_t stale = seq_prev(seq_prev(seq));
      const uint32_t src0 = ((uint32_t)cself * 2u * N + par * N) * a.slot_bytes;
      int st = 0;
      if (poller) {
        const uint32_t loff = (uint32_t)tg * kTileBytes + (uint32_t)lane * 16u;
        u32x4 got;
        st = poll_chunk<P>(rs, src0 + (uint32_t)w * a.slot_bytes + loff, loff < a.E, seq, stale,
                           true, a.ctrl, a.timeout_ticks, lane, got);
        if (st != 0) {
          if (lane == 0) lds_err = 1;
        } else {
          lds[buf][0][w][lane] = got;
        }
      }
      if (stager) lds[buf][0][g][lane] = own0;
      if (st == 0 && op + 1 < a.nops) send_op(op + 1, seq_next(seq), par ^ 1u);
      __syncthreads();
      if (lds_err) return;                         // whole workgroup
      if (own) {
        u32x4 v[NMAX];
#pragma unroll
        for (int r = 0; r < NMAX; ++r)
          v[r] = (r < a.nranks) ? lds[buf][0][r][lane] : u32x4{0u, 0u, 0u, 0u};
        reduce_store_tile<P, NMAX>(v, a.nranks, tg, a.E, lane,
                                   a.out + ((int64_t)op * a.nconsumers + cself) * a.out_stride,
                                   a.count);
        if (a.trace && lane == 0)
          __hip_atomic_fetch_max(
              reinterpret_cast<unsigned long long*>(a.trace) + (int64_t)op * tstride +
                  a.nranks + cself,
              (unsigned long long)now_ticks(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      buf ^= 1;
      seq = seq_next(seq);
      par ^= 1u;
    }
    return;
  }

  uint32_t seq = a.seq0;
  uint32_t par = a.parity0;
  int buf = 0;
  for (int op = 0; op < a.nops; ++op) {
    const uint32_t stale = seq_prev(seq_prev(seq));
    const uint32_t pp = par;
    const uint16_t* row = a.in + ((int64_t)op * op_rows + g) * a.in_stride;

    if (SHARE && !consumer && op >= 2) {
      Waiter wt(a.timeout_ticks, a.ctrl);
      const uint32_t prev = seq_prev(seq);
      while (true) {
        const uint32_t pv = ld_agent_u32(progress + tg);
        if (pv == prev || pv == seq) break;
        if (!wt.again(lane)) return;
      }
      fence_acquire();
    }
    if (SHARE && consumer && w == 0 && lane == 0 && op == 0) st_agent_u32(progress + tg, seq);
    if (sender && a.delay) {
      const uint32_t d = a.delay[(int64_t)op * a.nranks + g];
      if (d) {
        const uint64_t t0 = now_ticks();
        while (now_ticks() - t0 < (uint64_t)d) __builtin_amdgcn_s_sleep(2);
      }
    }
    // sentinel: this wave's re-arm stores of the previous op complete before
    // its next store to the same peer
    if (P == kSentinel && !SHARE && sender) fence_release();

    const uint32_t dst0 = ((uint32_t)dst_c * 2u * N + pp * N + (uint32_t)g) * a.slot_bytes;
    const uint32_t src0 = ((uint32_t)cself * 2u * N + pp * N) * a.slot_bytes;
    // ---- send every tile of this op first ----
    // own0 / own1: the encoded own chunks of the group's first two tiles,
    // kept by the stager for its LDS writes
    u32x4 own0 = u32x4{0u, 0u, 0u, 0u};
    u32x4 own1 = u32x4{0u, 0u, 0u, 0u};
    if (sender || (own && own_stages)) {
      auto send_tile = [&](int k) -> u32x4 {
        const int tile = tg + k * G;
        u32x4 mine_v;
        if (pipelined) {
          mask_words(wnext, keep);
          mine_v = encode_words<P>(wnext, lane, seq);
        } else {
          mine_v = encode_chunk<P>(row, row_bytes, a.count, tile, lane, seq);
        }
        if (sender) store_chunk<P>(rs, dst0, 0u, 1, -1, tile, a.E, lane, mine_v);
        return mine_v;
      };
      // senders take their tiles in the caller's order, if one is given (a
      // separate loop: the order's loads would otherwise make every send
      // wait for all of the wave's outstanding memory operations)
      if (sender && a.order) {
        const uint16_t* ord = a.order + ((int64_t)op * a.nranks + g) * a.TPW;
        for (int j = 0; j < a.TPW; ++j) {
          const int k = (int)ord[j];
          if (k < mine) {
            const u32x4 v = send_tile(k);
            if (k == 0) own0 = v;
            if (BATCH > 1 && k == 1) own1 = v;
          }
        }
      } else {
        // (one tile per group whenever BATCH is 1)
        own0 = send_tile(0);
        if (BATCH > 1 && mine > 1) own1 = send_tile(1);
        for (int k = BATCH > 1 ? 2 : 1; k < mine; ++k) send_tile(k);
      }
      if (sender && P == kLL128) {
        fence_release();
        for (int k = 0; k < mine; ++k)
          produce_flags(rs, dst0, 0u, 1, -1, tg + k * G, a.E, seq, lane);
      }
      if (sender && a.trace) {
        fence_release();
        if (lane == 0)
          __hip_atomic_fetch_max(
              reinterpret_cast<unsigned long long*>(a.trace) + (int64_t)op * tstride + g,
              (unsigned long long)now_ticks(), __ATOMIC_RELAXED,
              __HIP_MEMORY_SCOPE_AGENT);
      }
      // the next op's payload is loaded after this op's sends, so that no
      // wait for this wave's stores (the fences above) also waits for it
      // unconditional for the op: past the last op the range is empty and the
      // load reads nothing, so the loaded registers need no merge (and no wait)
      if (pipelined)
        load_chunk<P>(row + op_rows * a.in_stride, op + 1 < a.nops ? row_bytes : 0u, tg, lane,
                      wnext);
    }
    if (!consumer) {
      seq = seq_next(seq);
      par ^= 1u;
      continue;
    }
    // ---- then receive, BATCH tiles per workgroup barrier ----
    for (int k0 = 0; k0 < mine; k0 += BATCH) {
      const int nb = (mine - k0) < BATCH ? (mine - k0) : BATCH;
      if (poller) {
        uint32_t at[BATCH];
        bool active[BATCH];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
          const uint32_t loff = (uint32_t)(tg + (k0 + j) * G) * kTileBytes + (uint32_t)lane * 16u;
          at[j] = src0 + (uint32_t)w * a.slot_bytes + loff;
          active[j] = j < nb && loff < a.E;
        }
        u32x4 got[BATCH];
        int st;
        if constexpr (BATCH == 1)
          st = poll_chunk<P>(rs, at[0], active[0], seq, stale, true, a.ctrl,
                             a.timeout_ticks, lane, got[0]);
        else
          st = poll_chunks<P, BATCH>(rs, at, active, nb, seq, stale, true, a.ctrl,
                                     a.timeout_ticks, lane, got);
        if (st != 0) {
          if (lane == 0) lds_err = 1;
        } else {
          if (P == kSentinel && SHARE) fence_release();   // re-arm before the progress word
#pragma unroll
          for (int j = 0; j < BATCH; ++j)
            if (j < nb) lds[buf][j][w][lane] = got[j];
        }
      }
      if (stager) {
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
          const int k = k0 + j;
          if (j < nb)
            lds[buf][j][g][lane] =
                k == 0 ? own0
                       : (BATCH > 1 && k == 1)
                             ? own1
                             : encode_chunk<P>(row, row_bytes, a.count, tg + k * G, lane, seq);
        }
      }
      __syncthreads();
      if (lds_err) return;                         // whole workgroup
      // share mode: every slot of this op has been read and re-armed (the
      // pollers waited for their re-arm stores before the barrier), so rank
      // 0 publishes the next op as started now, not after its reduce: the
      // producers' licence for op+2 then reaches them one reduce earlier
      if (SHARE && w == 0 && lane == 0 && k0 + nb == mine)
        st_agent_u32(progress + tg, seq_next(seq));
      // ---- reduce in rank order (own wave) ----
      if (own) {
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
          if (j >= nb) break;
          u32x4 v[NMAX];
#pragma unroll
          for (int r = 0; r < NMAX; ++r)
            v[r] = (r < a.nranks) ? lds[buf][j][r][lane] : u32x4{0u, 0u, 0u, 0u};
          reduce_store_tile<P, NMAX>(
              v, a.nranks, tg + (k0 + j) * G, a.E, lane,
              a.out + ((int64_t)op * a.nconsumers + cself) * a.out_stride, a.count);
        }
        if (a.trace && lane == 0 && k0 + nb == mine)
          __hip_atomic_fetch_max(
              reinterpret_cast<unsigned long long*>(a.trace) + (int64_t)op * tstride +
                  a.nranks + cself,
              (unsigned long long)now_ticks(), __ATOMIC_RELAXED,
              __HIP_MEMORY_SCOPE_AGENT);
      }
      buf ^= 1;
    }
    seq = seq_next(seq);
    par ^= 1u;
  }
}

// ---------------------------------------------------------------- probes --

__device__ __forceinline__ uint32_t xcc_id() {
  // HW_REG_XCC_ID (id 20), bits [3:0]
  return (uint32_t)__builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11)) & 0xFu;
}

__global__ void k_pingpong(uint32_t* work, int32_t iters, int32_t xa,
                           int32_t xb, uint64_t* res, uint64_t timeout_ticks) {
  if (threadIdx.x != 0) return;
  uint32_t* fa = work;        // a -> b, own 128-byte line
  uint32_t* fb = work + 32;   // b -> a
  const int b = blockIdx.x;
  if (b == xa) {
    res[2] = xcc_id();
    const uint64_t deadline = now_ticks() + timeout_ticks;
    const uint64_t t0 = now_ticks();
    for (uint32_t k = 1; k <= (uint32_t)iters; ++k) {
      st_agent_u32(fa, k);
      while (ld_agent_u32(fb) != k) {
        if (now_ticks() > deadline) { res[4] = 1; return; }
      }
    }
    res[0] = now_ticks() - t0;
    res[1] = (uint64_t)iters;
  } else if (b == xb) {
    res[3] = xcc_id();
    const uint64_t deadline = now_ticks() + timeout_ticks;
    for (uint32_t k = 1; k <= (uint32_t)iters; ++k) {
      while (ld_agent_u32(fa) != k) {
        if (now_ticks() > deadline) { res[4] = 2; return; }
      }
      st_agent_u32(fb, k);
    }
  }
}

// Ordering litmus between a writer wave (block xa) and a reader wave (block
// xb); see ar_probe_litmus in ar.h for the three kinds.
__global__ void k_litmus(uint8_t* work, int32_t iters, int32_t xa, int32_t xb,
                         int32_t kind, uint64_t* res, uint64_t timeout_ticks) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  uint32_t* const flag = reinterpret_cast<uint32_t*>(work);         // line 0
  uint32_t* const ack = reinterpret_cast<uint32_t*>(work + 128);    // line 1
  uint32_t* const wrote = reinterpret_cast<uint32_t*>(work + 256);  // line 2
  const rsrc_t rs = make_rsrc(work, 4096);
  const uint32_t blk = 1024;                                        // 1 KiB block
  const uint64_t deadline = now_ticks() + timeout_ticks;
  if (b == xa) {
    if (lane == 0) res[2] = xcc_id();
    for (uint32_t k = 1; k <= (uint32_t)iters; ++k) {
      if (kind == 0) {
        st16(rs, blk + lane * 16u, u32x4{k, k, k, k});
        fence_release();
        if (lane == 0) st_agent_u32(flag, k);
      } else if (kind == 1) {
        st16(rs, blk + lane * 16u, u32x4{k, k, k, k});
      } else {
        if (lane == 0) {
          while (ld_agent_u32(ack) != k - 1u) {
            if (now_ticks() > deadline) { res[4] = 1; return; }
          }
          fence_acquire();
          __builtin_amdgcn_raw_buffer_store_b32(k, rs, blk, 0, kCpAgent);
          fence_release();
          st_agent_u32(wrote, k);
        }
      }
    }
  } else if (b == xb) {
    if (lane == 0) res[3] = xcc_id();
    uint64_t viol = 0, obs = 0, second = 0;
    uint32_t last = 0;
    if (kind == 0) {
      while (true) {
        const uint32_t f = ld_agent_u32(flag);
        fence_acquire();
        const u32x4 d = ld16(rs, blk + lane * 16u);
        const bool bad = d.x < f || d.y < f || d.z < f || d.w < f;
        viol += __popcll(__ballot(bad));
        ++obs;
        last = f;
        if (f == (uint32_t)iters) break;
        if (now_ticks() > deadline) { if (lane == 0) res[4] = 2; break; }
      }
    } else if (kind == 1) {
      while (true) {
        const u32x4 d = ld16(rs, blk + lane * 16u);
        viol += __popcll(__ballot(d.x != d.y || d.z != d.w));
        second += __popcll(__ballot(d.x != d.z));
        ++obs;
        last = d.x;
        if (__ballot(d.x != (uint32_t)iters || d.z != (uint32_t)iters) == 0ull) break;
        if (now_ticks() > deadline) { if (lane == 0) res[4] = 2; break; }
      }
    } else if (lane == 0) {
      for (uint32_t k = 1; k <= (uint32_t)iters; ++k) {
        while (ld_agent_u32(wrote) != k) {
          if (now_ticks() > deadline) { res[4] = 2; goto out; }
        }
        fence_acquire();
        const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(rs, blk, 0, kCpAgent);
        viol += (w != k);
        ++obs;
        last = w;
        __builtin_amdgcn_raw_buffer_store_b32(0u, rs, blk, 0, kCpAgent);   // re-arm
        fence_release();
        st_agent_u32(ack, k);
      }
    }
  out:
    if (lane == 0) {
      res[0] = viol;
      res[1] = obs;
      res[5] = last;
      res[6] = second;
    }
  }
}

__global__ __launch_bounds__(kBlock) void k_chain_init(uint32_t* work, uint32_t n,
                                                       uint32_t stride) {
  for (uint32_t i = blockIdx.x * kBlock + threadIdx.x; i < n; i += gridDim.x * kBlock)
    work[i] = (uint32_t)(((uint64_t)i + stride) & (uint64_t)(n - 1));
}

__global__ void k_chain(const uint32_t* work, uint32_t bytes, int32_t iters,
                        uint64_t* res) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  const rsrc_t rs = make_rsrc(work, bytes);
  uint32_t idx = 0;
  const uint64_t t0 = now_ticks();
  for (int i = 0; i < iters; ++i) {
    idx = __builtin_amdgcn_raw_buffer_load_b32(rs, idx * 4u, 0, kCpAgent);
    compiler_barrier();
  }
  res[0] = now_ticks() - t0;
  res[1] = (uint64_t)iters;
  res[2] = idx;
}

__global__ __launch_bounds__(kBlock) void k_copy(const u32x4* __restrict__ src,
                                                 u32x4* __restrict__ dst,
                                                 uint64_t n16) {
  for (uint64_t i = (uint64_t)blockIdx.x * kBlock + threadIdx.x; i < n16;
       i += (uint64_t)gridDim.x * kBlock)
    dst[i] = src[i];
}

__global__ void k_empty() {}

// Each workgroup records the XCD it runs on and holds its slot until every
// workgroup of the grid has arrived (a bounded wait), so that the recorded
// placement is that of a fully resident grid, as in the simulators.
__global__ void k_placement(int32_t* res, uint32_t* count, uint32_t blocks,
                            uint64_t timeout_ticks) {
  if (threadIdx.x != 0) return;
  res[blockIdx.x] = (int32_t)xcc_id();
  __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t deadline = now_ticks() + timeout_ticks;
  while (ld_agent_u32(count) < blocks) {
    if (now_ticks() > deadline) {
      res[blockIdx.x] = -1;
      return;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// ============================================================ host side ==

template <int P>
static hipError_t launch_pack(PackArgs a, int blocks, hipStream_t s) {
  return launch(k_pack<P>, dim3(blocks), dim3(kBlock), s, a);
}

static int pack_common(int32_t want_proto, const ar_desc* d, const void* in,
                       int64_t in_stride, void* scratch, ar_epoch e,
                       void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (d->proto != want_proto) return AR_EINVAL;
  if (e.parity > 1u || e.seq == 0u) return AR_EINVAL;
  rc = check_rows(in, in_stride, d->count);
  if (rc) return rc;
  if (d->count == 0) return AR_OK;
  if (!scratch) return AR_EINVAL;
  if (!aligned(scratch, 256)) return AR_EALIGN;
  if (d->collective == AR_TWOSHOT)
    return twoshot_pack(want_proto, d, in, in_stride, scratch, e,
                        static_cast<hipStream_t>(stream));
  PackArgs a;
  a.in = static_cast<const uint16_t*>(in);
  a.in_stride = in_stride;
  a.count = d->count;
  a.scratch = static_cast<const uint8_t*>(scratch);
  a.slot_bytes = (uint32_t)slot_bytes_of(d->proto, d->count);
  a.scratch_bytes = (uint32_t)((int64_t)d->nconsumers * 2 * d->nranks * a.slot_bytes);
  a.E = (uint32_t)encoded_bytes(d->proto, d->count);
  a.nranks = d->nranks;
  a.nconsumers = d->nconsumers;
  a.tiles = (int32_t)ceil_div64(a.E, kTileBytes);
  a.seq = e.seq;
  a.parity = e.parity;
  const int64_t waves = (int64_t)a.tiles * d->nranks;
  const int blocks = (int)ceil_div64(waves, kWavesPerBlock);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  switch (want_proto) {
    case kLL: err = launch_pack<kLL>(a, blocks, s); break;
    case kLL128: err = launch_pack<kLL128>(a, blocks, s); break;
    case kSentinel: err = launch_pack<kSentinel>(a, blocks, s); break;
    default: err = launch_pack<kBarrier>(a, blocks, s); break;
  }
  return map_hip(err);
}

template <int P, int NMAX>
static hipError_t launch_reduce(ReduceArgs a, int blocks, hipStream_t s) {
  return launch(k_reduce<P, NMAX>, dim3(blocks), dim3(kBlock), s, a);
}

template <int P>
static hipError_t launch_reduce_n(const ReduceArgs& a, int blocks, hipStream_t s) {
  if (a.nranks <= 4) return launch_reduce<P, 4>(a, blocks, s);
  if (a.nranks <= 8) return launch_reduce<P, 8>(a, blocks, s);
  return launch_reduce<P, 16>(a, blocks, s);
}

// The kernel variant: `one` = every wave or workgroup owns at most one tile
// (the narrow kernel's software-pipelined variant, the wide kernel's BATCH 1);
// otherwise the variant for many tiles.  The barrier baseline has only the
// latter.
template <int P, int NMAX, bool SHARE, bool EXTRAS>
static const void* sim_kernel(bool wide, bool one) {
  if (!wide) {
    if constexpr (P != kBarrier)
      if (one) return reinterpret_cast<const void*>(&k_sim<P, NMAX, SHARE, EXTRAS, true>);
    return reinterpret_cast<const void*>(&k_sim<P, NMAX, SHARE, EXTRAS, false>);
  }
  return one ? reinterpret_cast<const void*>(&k_sim_wide<P, NMAX, SHARE, 1, EXTRAS>)
             : reinterpret_cast<const void*>(&k_sim_wide<P, NMAX, SHARE, 2, EXTRAS>);
}

template <int P, int NMAX, bool SHARE>
static hipError_t launch_sim(const SimArgs& a, int blocks, bool coop, bool wide, bool one,
                             hipStream_t s) {
  SimArgs copy = a;
  void* args[] = {&copy};
  const bool extras = a.delay || a.order || a.trace;
  const void* fn = extras ? sim_kernel<P, NMAX, SHARE, true>(wide, one)
                          : sim_kernel<P, NMAX, SHARE, false>(wide, one);
  const dim3 block(wide ? kWave * a.nranks : kSimBlock);
  if (coop) return hipLaunchCooperativeKernel(fn, dim3(blocks), block, args, 0, s);
  return hipLaunchKernel(fn, dim3(blocks), block, args, 0, s);
}

// The smaller occupancy of the variant with and without the optional
// features (a launch's grid is sized before it is known which it takes).
template <int P, int NMAX, bool SHARE>
static int occupancy_of(bool wide, bool one, int nranks) {
  const void* fns[2] = {sim_kernel<P, NMAX, SHARE, false>(wide, one),
                        sim_kernel<P, NMAX, SHARE, true>(wide, one)};
  const int threads = wide ? kWave * nranks : kSimBlock;
  int occ = 0;
  for (int i = 0; i < 2; ++i) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fns[i], threads, 0) != hipSuccess)
      return 0;
    occ = (i == 0 || n < occ) ? n : occ;
  }
  return occ;
}

template <int P>
static hipError_t dispatch_sim_p(const SimArgs& a, bool share, int blocks, bool coop,
                                 bool wide, bool one, hipStream_t s) {
  if (a.nranks <= 4)
    return share ? launch_sim<P, 4, true>(a, blocks, coop, wide, one, s)
                 : launch_sim<P, 4, false>(a, blocks, coop, wide, one, s);
  if (a.nranks <= 8)
    return share ? launch_sim<P, 8, true>(a, blocks, coop, wide, one, s)
                 : launch_sim<P, 8, false>(a, blocks, coop, wide, one, s);
  return share ? launch_sim<P, 16, true>(a, blocks, coop, wide, one, s)
               : launch_sim<P, 16, false>(a, blocks, coop, wide, one, s);
}

template <int P>
static int occupancy_p(int nranks, bool share, bool wide, bool one) {
  if (nranks <= 4)
    return share ? occupancy_of<P, 4, true>(wide, one, nranks)
                 : occupancy_of<P, 4, false>(wide, one, nranks);
  if (nranks <= 8)
    return share ? occupancy_of<P, 8, true>(wide, one, nranks)
                 : occupancy_of<P, 8, false>(wide, one, nranks);
  return share ? occupancy_of<P, 16, true>(wide, one, nranks)
               : occupancy_of<P, 16, false>(wide, one, nranks);
}

static int sim_occupancy(int proto, int nranks, bool share, bool wide, bool one) {
  switch (proto) {
    case kLL: return occupancy_p<kLL>(nranks, share, wide, one);
    case kLL128: return occupancy_p<kLL128>(nranks, share, wide, one);
    case kSentinel: return occupancy_p<kSentinel>(nranks, share, wide, one);
    default: return occupancy_p<kBarrier>(nranks, share, wide, one);
  }
}

struct SimGeom {
  int32_t W, Q, T, TPW, blocks;
  bool wide;
  bool coop;                 // cooperative launch
  bool one;                  // the one-tile kernel variant (TPW <= 1)
};

// The wide kernel (a workgroup of one wave per peer) serves LL, LL128 and
// SENTINEL unless AR_SIM_NARROW asks for the one-wave-per-tile kernel; the
// barrier baseline always uses the latter.
static bool sim_is_wide(const ar_sim_params* p) {
  return p->desc.proto != kBarrier && (p->flags & AR_SIM_NARROW) == 0;
}
static bool sim_force_wide(const ar_sim_params* p) {
  return p->desc.proto != kBarrier && (p->flags & AR_SIM_WIDE) != 0;
}

// Grid for one kernel variant: Q workgroups (or waves) per rank and XCD
// within the residency the variant's occupancy allows.
static int sim_plan(const ar_sim_params* p, const DeviceInfo& di, bool wide, bool coop,
                    bool one, int64_t T, int64_t* Q_out) {
  const ar_desc* d = &p->desc;
  const bool share = d->nconsumers == 1 && d->nranks > 1;
  const int occ = sim_occupancy(d->proto, d->nranks, share, wide, one);
  if (occ <= 0) return AR_ELAUNCH;
  // Every workgroup waits on others, so the whole grid must be resident at
  // once.  An ordinary launch keeps the grid to half of what the occupancy
  // query reports (a margin for limits the query does not model); a
  // cooperative launch, whose residency the runtime checks, may fill it.
  // The one-wave kernel is held to 8 workgroups per CU: the large sizes that
  // use it are bound by memory bandwidth, which that many waves already
  // saturate.
  int64_t capacity = (int64_t)occ * di.cus / (coop ? 1 : 2);
  if (!wide && capacity > 8 * (int64_t)di.cus) capacity = 8 * (int64_t)di.cus;
  const int64_t qmax_dev = capacity / (8 * (int64_t)d->nranks);
  const int64_t per_q = wide ? 8 : kSimWavesPerQ;   // tile groups / waves per Q
  const int64_t qcap = kCtrlMaxProgress / per_q;
  const int64_t qmax = qmax_dev < qcap ? qmax_dev : qcap;
  if (qmax < 1) return AR_ECAPACITY;
  int64_t Q;
  if (p->waves_per_rank > 0) {
    if (p->waves_per_rank % per_q) return AR_EINVAL;
    Q = p->waves_per_rank / per_q;
    if (Q > qmax) return AR_ECAPACITY;
  } else {
    Q = ceil_div64(T, per_q);
    if (Q > qmax) Q = qmax;
    if (Q < 1) Q = 1;
  }
  *Q_out = Q;
  return AR_OK;
}

static int sim_geometry_as(const ar_sim_params* p, const DeviceInfo& di, bool wide,
                           bool coop, SimGeom* g) {
  const ar_desc* d = &p->desc;
  const int64_t E = encoded_bytes(d->proto, d->count);
  const int64_t T = ceil_div64(E, kTileBytes);
  if (T <= 0) {
    *g = SimGeom{0, 0, 0, 0, 0, wide, coop, false};
    return AR_OK;
  }
  if (T > (int64_t(1) << 24)) return AR_ESIZE;
  const int64_t per_q = wide ? 8 : kSimWavesPerQ;
  // the one-tile variant when its own residency gives every wave (or group)
  // at most one tile; otherwise the many-tile variant, sized by its own
  // (the variant launched is always the one whose occupancy sized the grid)
  int64_t Q = 0;
  bool one = false;
  if (wide || d->proto != kBarrier) {
    if (sim_plan(p, di, wide, coop, true, T, &Q) == AR_OK && T <= per_q * Q) one = true;
  }
  if (!one) {
    const int rc = sim_plan(p, di, wide, coop, false, T, &Q);
    if (rc) return rc;
  }
  const int64_t W = per_q * Q;
  g->W = (int32_t)W;
  g->Q = (int32_t)Q;
  g->T = (int32_t)T;
  g->TPW = (int32_t)ceil_div64(T, W);
  g->blocks = (int32_t)(8 * Q * d->nranks);
  g->wide = wide;
  g->coop = coop;
  g->one = one;
  return AR_OK;
}

// Kernel choice: the wide kernel while each of its workgroups walks at most
// 3 tiles (4 ranks) or 2 (8 and 16 ranks), or when AR_SIM_WIDE asks for it;
// otherwise, or with AR_SIM_NARROW, or for the barrier baseline, the
// one-wave-per-tile kernel.  From a sweep of both kernels on MI355X (4, 8
// and 16 ranks, 8-256 KiB per rank, 64 ops, ordinary and cooperative
// launches): with one tile the wide kernel wins everywhere (up to 3.2x);
// with two it wins everywhere (4 ranks 256 KiB sentinel: 3.11 vs 3.54 us;
// 16 ranks 8 KiB LL128: 4.71 vs 8.11 us); with three it still wins at 4
// ranks (256 KiB LL: 4.62 vs 4.73 us) but loses at 8 and 16 (8 ranks 64 KiB
// LL128: 6.13 vs 5.45 us); from four on, the one-wave kernel wins (8 ranks
// 128 KiB sentinel: 6.64 vs 5.05 us).
static int sim_kernel_choice(const ar_sim_params* p, const DeviceInfo& di, bool coop,
                             SimGeom* g) {
  if (sim_is_wide(p)) {
    SimGeom gw;
    const int rc = sim_geometry_as(p, di, true, coop, &gw);
    const int max_tiles = p->desc.nranks > 4 ? 2 : 3;
    if (rc == AR_OK && (gw.TPW <= max_tiles || sim_force_wide(p))) {
      *g = gw;
      return AR_OK;
    }
    if (sim_force_wide(p)) return rc;
    if (rc != AR_OK && rc != AR_ECAPACITY && rc != AR_EINVAL) return rc;
  }
  return sim_geometry_as(p, di, false, coop, g);
}

// Launch choice (coop_pays): measured, 64 ops, 16 ranks [1,4096] LL 4.19 ->
// 3.23 us per op (2 -> 1 tiles per workgroup), 16 ranks [8,4096] LL 15.8 ->
// 10.0 us, 4 ranks [1,131072] sentinel 3.53 -> 2.23 us (the workgroup kernel
// instead of the one-wave kernel).
static int sim_geometry(const ar_sim_params* p, const DeviceInfo& di, SimGeom* g) {
  if (p->flags & AR_SIM_COOPERATIVE) return sim_kernel_choice(p, di, true, g);
  const int rc = sim_kernel_choice(p, di, false, g);
  if ((p->flags & AR_SIM_ORDINARY) || !di.coop || p->nops < kCoopMinOps) return rc;
  if (rc != AR_OK && rc != AR_ECAPACITY) return rc;
  SimGeom gc;
  if (sim_kernel_choice(p, di, true, &gc) == AR_OK &&
      coop_pays(rc, g->TPW, g->wide, gc.TPW, gc.wide)) {
    *g = gc;
    return AR_OK;
  }
  return rc;
}

static int check_sim(const ar_sim_params* p) {
  if (!p) return AR_EINVAL;
  int rc = check_desc(&p->desc);
  if (rc) return rc;
  const ar_desc* d = &p->desc;
  if (p->nops < 1) return AR_EINVAL;
  if (p->waves_per_rank < 0) return AR_EINVAL;
  if ((p->flags & ~(AR_SIM_COOPERATIVE | AR_SIM_ORDINARY | AR_SIM_NARROW | AR_SIM_WIDE)) !=
          0 ||
      p->reserved != 0)
    return AR_EINVAL;
  if ((p->flags & AR_SIM_COOPERATIVE) && (p->flags & AR_SIM_ORDINARY)) return AR_EINVAL;
  if ((p->flags & AR_SIM_NARROW) && (p->flags & AR_SIM_WIDE)) return AR_EINVAL;
  if (p->epoch.parity > 1u || p->epoch.seq == 0u) return AR_EINVAL;
  if (!timeout_ok(p->timeout_ns)) return AR_EINVAL;
  rc = check_rows(p->in, p->in_stride, d->count);
  if (rc) return rc;
  rc = check_rows(p->out, p->out_stride, d->count);
  if (rc) return rc;
  if (!p->scratch || !p->ctrl) return AR_EINVAL;
  if (!aligned(p->scratch, 256) || !aligned(p->ctrl, 256)) return AR_EALIGN;
  if (p->trace && !aligned(p->trace, 8)) return AR_EALIGN;
  if (p->delay_ticks && !aligned(p->delay_ticks, 4)) return AR_EALIGN;
  if (p->tile_order && !aligned(p->tile_order, 2)) return AR_EALIGN;
  return AR_OK;
}

int sim_validate(const ar_sim_params* p) {
  int rc = check_sim(p);
  if (rc) return rc;
  const ar_desc* d = &p->desc;
  if (d->collective == AR_ALLGATHER && p->out_stride < (int64_t)d->nranks * ((d->count + 7) / 8 * 8))
    return AR_EINVAL;
  if (d->count == 0) return AR_OK;
  DeviceInfo di;
  rc = device_info(&di);
  if (rc) return rc;
  if ((p->flags & AR_SIM_COOPERATIVE) && !di.coop) return AR_ENODEV;
  return ar_sim_geometry(p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
}

}  // namespace ar

// ============================================================ C ABI ======

using namespace ar;

extern "C" {

const char* ar_status_string(int code) {
  switch (code) {
    case AR_OK: return "AR_OK";
    case AR_EINVAL: return "AR_EINVAL: invalid argument";
    case AR_EALIGN: return "AR_EALIGN: misaligned pointer or stride";
    case AR_ESIZE: return "AR_ESIZE: size limit exceeded";
    case AR_ELAUNCH: return "AR_ELAUNCH: HIP runtime error";
    case AR_ETIMEOUT: return "AR_ETIMEOUT: poll deadline passed";
    case AR_ECORRUPT: return "AR_ECORRUPT: impossible readiness flag";
    case AR_ENODEV: return "AR_ENODEV: no usable device";
    case AR_ECAPACITY: return "AR_ECAPACITY: grid cannot be co-resident";
    default: return "AR_UNKNOWN";
  }
}

int ar_abi_version(void) { return 7; }

int64_t ar_encoded_bytes(int32_t proto, int64_t count) {
  return encoded_bytes(proto, count);
}

int64_t ar_slot_bytes(int32_t proto, int64_t count) {
  return slot_bytes_of(proto, count);
}

int64_t ar_scratch_bytes(const ar_desc* d) {
  const int rc = check_desc(d);
  if (rc) return rc;
  return desc_scratch_bytes(d);
}

int64_t ar_desc_slot_bytes(const ar_desc* d) {
  const int rc = check_desc(d);
  if (rc) return rc;
  return desc_slot_bytes(d);
}

int ar_shard_bounds(int64_t count, int32_t nranks, int32_t k, int64_t* lo,
                    int64_t* hi) {
  if (!lo || !hi || count < 0 || nranks < 1 || nranks > AR_MAX_RANKS || k < 0 ||
      k >= nranks)
    return AR_EINVAL;
  share_bounds(count, nranks, k, lo, hi);
  return AR_OK;
}

int64_t ar_ctrl_bytes(void) {
  return (int64_t)(kCtrlProgress + kCtrlMaxProgress) * 4 + 256;
}

int ar_epoch_init(ar_epoch* e) {
  if (!e) return AR_EINVAL;
  e->seq = 1u;
  e->parity = 0u;
  return AR_OK;
}

int ar_epoch_flip(ar_epoch* e) {
  if (!e || e->parity > 1u || e->seq == 0u) return AR_EINVAL;
  e->seq = e->seq == 0xFFFFFFFFu ? 1u : e->seq + 1u;
  e->parity ^= 1u;
  return AR_OK;
}

int ar_epoch_advance(ar_epoch* e, uint64_t nops) {
  if (!e || e->parity > 1u || e->seq == 0u) return AR_EINVAL;
  // seq runs through 1..2^32-1 (period 2^32-1); parity has period 2
  const uint64_t period = 0xFFFFFFFFull;
  const uint64_t s = (uint64_t)(e->seq - 1u);
  e->seq = (uint32_t)((s + nops % period) % period) + 1u;
  e->parity ^= (uint32_t)(nops & 1u);
  return AR_OK;
}

int ar_ctrl_reset(void* ctrl, void* stream) {
  if (!ctrl) return AR_EINVAL;
  if (!aligned(ctrl, 256)) return AR_EALIGN;
  const uint32_t words = (uint32_t)(ar_ctrl_bytes() / 4);
  return map_hip(launch(k_fill_zero, dim3((words + kBlock - 1) / kBlock), dim3(kBlock),
                        static_cast<hipStream_t>(stream), static_cast<uint32_t*>(ctrl),
                        words));
}

int ar_pack_ll(const ar_desc* d, const void* in, int64_t in_stride,
               void* scratch, ar_epoch e, void* stream) {
  return pack_common(kLL, d, in, in_stride, scratch, e, stream);
}

int ar_pack_ll128(const ar_desc* d, const void* in, int64_t in_stride,
                  void* scratch, ar_epoch e, void* stream) {
  return pack_common(kLL128, d, in, in_stride, scratch, e, stream);
}

int ar_pack_sentinel(const ar_desc* d, const void* in, int64_t in_stride,
                     void* scratch, ar_epoch e, void* stream) {
  return pack_common(kSentinel, d, in, in_stride, scratch, e, stream);
}

int ar_pack_plain(const ar_desc* d, const void* in, int64_t in_stride,
                  void* scratch, ar_epoch e, void* stream) {
  return pack_common(kBarrier, d, in, in_stride, scratch, e, stream);
}

int ar_arm_sentinel(const ar_desc* d, void* scratch, int32_t parity,
                    void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (d->proto != kSentinel) return AR_EINVAL;
  if (parity < -1 || parity > 1) return AR_EINVAL;
  if (d->count == 0) return AR_OK;
  if (!scratch) return AR_EINVAL;
  if (!aligned(scratch, 256)) return AR_EALIGN;
  const uint32_t slot = (uint32_t)desc_slot_bytes(d);
  const uint32_t total = (uint32_t)desc_scratch_bytes(d);
  const uint32_t region = (uint32_t)d->nranks * slot;   // one parity of one consumer
  // consumer buffers in the scratch: one per consumer, twice for two-shot
  // (reduce-scatter region, then all-gather region, same layout)
  const int32_t nbuf = d->nconsumers * (d->collective == AR_TWOSHOT ? 2 : 1);
  uint32_t region0, stride;
  int32_t nregions;
  if (parity < 0) {
    region0 = 0;
    stride = region;
    nregions = 2 * nbuf;
  } else {
    region0 = (uint32_t)parity * region;
    stride = 2u * region;
    nregions = nbuf;
  }
  const uint64_t chunks = (uint64_t)(region / 16u) * (uint64_t)nregions;
  uint64_t blocks = (chunks + kBlock - 1) / kBlock;
  if (blocks > 4096) blocks = 4096;
  return map_hip(launch(k_arm, dim3((unsigned)blocks), dim3(kBlock),
                        static_cast<hipStream_t>(stream),
                        static_cast<const uint8_t*>(scratch), total, region0, stride,
                        region, nregions));
}

int ar_reduce_validate(const ar_desc* d, void* scratch, void* out,
                       int64_t out_stride, ar_epoch e, void* ctrl,
                       uint64_t timeout_ns, int32_t flags, void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (e.parity > 1u || e.seq == 0u) return AR_EINVAL;
  if (flags & ~AR_FLAG_REARM) return AR_EINVAL;
  if (!timeout_ok(timeout_ns)) return AR_EINVAL;
  if (d->collective == AR_ALLGATHER) return AR_EINVAL;
  rc = check_rows(out, out_stride, d->count);
  if (rc) return rc;
  if (d->count == 0) return AR_OK;
  if (!scratch || !ctrl) return AR_EINVAL;
  if (!aligned(scratch, 256) || !aligned(ctrl, 256)) return AR_EALIGN;
  if (d->collective == AR_TWOSHOT)
    return twoshot_reduce(d, scratch, out, out_stride, e, ctrl, timeout_ns, flags,
                          static_cast<hipStream_t>(stream));
  DeviceInfo di;
  rc = device_info(&di);
  if (rc) return rc;
  ReduceArgs a;
  a.out = static_cast<uint16_t*>(out);
  a.out_stride = out_stride;
  a.count = d->count;
  a.scratch = static_cast<const uint8_t*>(scratch);
  a.slot_bytes = (uint32_t)slot_bytes_of(d->proto, d->count);
  a.scratch_bytes = (uint32_t)((int64_t)d->nconsumers * 2 * d->nranks * a.slot_bytes);
  a.E = (uint32_t)encoded_bytes(d->proto, d->count);
  a.nranks = d->nranks;
  a.nconsumers = d->nconsumers;
  a.tiles = (int32_t)ceil_div64(a.E, kTileBytes);
  a.seq = e.seq;
  a.parity = e.parity;
  a.ctrl = static_cast<int*>(ctrl);
  a.timeout_ticks = ns_to_ticks(timeout_ns, di.wallclock_hz);
  a.rearm = (flags & AR_FLAG_REARM) && d->proto == kSentinel;
  const int64_t waves = (int64_t)a.tiles * d->nconsumers;
  const int blocks = (int)ceil_div64(waves, kWavesPerBlock);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  switch (d->proto) {
    case kLL: err = launch_reduce_n<kLL>(a, blocks, s); break;
    case kLL128: err = launch_reduce_n<kLL128>(a, blocks, s); break;
    case kSentinel: err = launch_reduce_n<kSentinel>(a, blocks, s); break;
    default: err = launch_reduce_n<kBarrier>(a, blocks, s); break;
  }
  return map_hip(err);
}

int ar_sim_geometry(const ar_sim_params* p, int32_t* waves_per_rank,
                    int32_t* tiles_per_rank, int32_t* tiles_per_wave,
                    int32_t* blocks, int32_t* wide, int32_t* cooperative) {
  if (!p) return AR_EINVAL;
  int rc = check_desc(&p->desc);
  if (rc) return rc;
  if (p->desc.collective != AR_ALLREDUCE)
    return coll_sim_geometry(p, waves_per_rank, tiles_per_rank, tiles_per_wave, blocks,
                             wide, cooperative);
  DeviceInfo di;
  rc = device_info(&di);
  if (rc) return rc;
  SimGeom g;
  rc = sim_geometry(p, di, &g);
  if (rc) return rc;
  if (waves_per_rank) *waves_per_rank = g.W;
  if (tiles_per_rank) *tiles_per_rank = g.T;
  if (tiles_per_wave) *tiles_per_wave = g.TPW;
  if (blocks) *blocks = g.blocks;
  if (wide) *wide = g.wide ? 1 : 0;
  if (cooperative) *cooperative = g.coop ? 1 : 0;
  return AR_OK;
}

static int sim_launch(const ar_sim_params* p, const DeviceInfo& di, const SimGeom& g,
                      hipStream_t s) {
  const ar_desc* d = &p->desc;
  const bool share = d->nconsumers == 1 && d->nranks > 1;
  SimArgs a;
  a.in = static_cast<const uint16_t*>(p->in);
  a.in_stride = p->in_stride;
  a.out = static_cast<uint16_t*>(p->out);
  a.out_stride = p->out_stride;
  a.scratch = static_cast<const uint8_t*>(p->scratch);
  a.slot_bytes = (uint32_t)slot_bytes_of(d->proto, d->count);
  a.scratch_bytes = (uint32_t)((int64_t)d->nconsumers * 2 * d->nranks * a.slot_bytes);
  a.ctrl = static_cast<int*>(p->ctrl);
  a.count = d->count;
  a.E = (uint32_t)encoded_bytes(d->proto, d->count);
  a.nranks = d->nranks;
  a.nconsumers = d->nconsumers;
  a.nops = p->nops;
  a.W = g.W;
  a.Q = g.Q;
  a.T = g.T;
  a.TPW = g.TPW;
  a.seq0 = p->epoch.seq;
  a.parity0 = p->epoch.parity;
  a.timeout_ticks = ns_to_ticks(p->timeout_ns, di.wallclock_hz);
  a.delay = p->delay_ticks;
  a.order = p->tile_order;
  a.trace = p->trace;
  // the barrier baseline's per-wave counter reaches (nranks + nconsumers) * nops
  if ((uint64_t)(d->nranks + d->nconsumers) * (uint64_t)(p->nops + 1) >= 0xFFFFFFFFull)
    return AR_ESIZE;
  if (g.W > kCtrlMaxProgress) return AR_ECAPACITY;   // one counter / progress word a wave
  hipError_t e;
  switch (d->proto) {
    case kLL: e = dispatch_sim_p<kLL>(a, share, g.blocks, g.coop, g.wide, g.one, s); break;
    case kLL128: e = dispatch_sim_p<kLL128>(a, share, g.blocks, g.coop, g.wide, g.one, s); break;
    case kSentinel:
      e = dispatch_sim_p<kSentinel>(a, share, g.blocks, g.coop, g.wide, g.one, s);
      break;
    default: e = dispatch_sim_p<kBarrier>(a, share, g.blocks, g.coop, g.wide, g.one, s); break;
  }
  return map_hip(e);
}

int ar_sim_chain_run(const ar_sim_params* p, const float* scales, void* stream) {
  const int rc = check_sim(p);
  if (rc) return rc;
  return chain_sim_run(p, scales, static_cast<hipStream_t>(stream));
}

int ar_sim_chain_geometry(const ar_sim_params* p, int32_t* blocks, int32_t* cooperative) {
  const int rc = check_sim(p);
  if (rc) return rc;
  return chain_sim_geometry(p, blocks, cooperative);
}

int ar_sim_run(const ar_sim_params* p, void* stream) {
  int rc = check_sim(p);
  if (rc) return rc;
  const ar_desc* d = &p->desc;
  if (d->collective != AR_ALLREDUCE)
    return coll_sim_run(p, static_cast<hipStream_t>(stream));
  if (d->count == 0) return AR_OK;
  DeviceInfo di;
  rc = device_info(&di);
  if (rc) return rc;
  if ((p->flags & AR_SIM_COOPERATIVE) && !di.coop) return AR_ENODEV;
  SimGeom g;
  rc = sim_geometry(p, di, &g);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = sim_launch(p, di, g, s);
  // A cooperative launch the library chose by itself that the runtime turns
  // down is retried as an ordinary launch (same kernel choice rule, half the
  // occupancy).  Not with a tile order: its shape follows the first geometry.
  if (rc == AR_ELAUNCH && g.coop && !(p->flags & AR_SIM_COOPERATIVE) && !p->tile_order) {
    (void)hipGetLastError();
    SimGeom go;
    if (sim_kernel_choice(p, di, false, &go) == AR_OK) rc = sim_launch(p, di, go, s);
  }
  return rc;
}

int ar_wallclock_hz(double* hz) {
  if (!hz) return AR_EINVAL;
  DeviceInfo di;
  const int rc = device_info(&di);
  if (rc) return rc;
  *hz = di.wallclock_hz;
  return AR_OK;
}

int ar_probe_pingpong(void* work, int32_t iters, int32_t xcd_a, int32_t xcd_b,
                      void* result, void* stream) {
  if (!work || !result || iters < 1) return AR_EINVAL;
  if (xcd_a < 0 || xcd_a > 7 || xcd_b < 0 || xcd_b > 7 || xcd_a == xcd_b) return AR_EINVAL;
  if (!aligned(work, 256) || !aligned(result, 8)) return AR_EALIGN;
  DeviceInfo di;
  int rc = device_info(&di);
  if (rc) return rc;
  uint32_t* w = static_cast<uint32_t*>(work);
  uint64_t* r = static_cast<uint64_t*>(result);
  const uint64_t to = ns_to_ticks(2000000000ull, di.wallclock_hz);
  // 8 one-wave workgroups, one per XCD: resident together on an idle device
  return map_hip(launch(k_pingpong, dim3(8), dim3(64), static_cast<hipStream_t>(stream),
                        w, iters, xcd_a, xcd_b, r, to));
}

int ar_probe_litmus(void* work, int32_t iters, int32_t xcd_a, int32_t xcd_b,
                    int32_t kind, void* result, void* stream) {
  if (!work || !result || iters < 1 || kind < 0 || kind > 2) return AR_EINVAL;
  if (xcd_a < 0 || xcd_a > 7 || xcd_b < 0 || xcd_b > 7 || xcd_a == xcd_b) return AR_EINVAL;
  if (!aligned(work, 256) || !aligned(result, 8)) return AR_EALIGN;
  DeviceInfo di;
  int rc = device_info(&di);
  if (rc) return rc;
  uint8_t* w = static_cast<uint8_t*>(work);
  uint64_t* r = static_cast<uint64_t*>(result);
  const uint64_t to = ns_to_ticks(5000000000ull, di.wallclock_hz);
  return map_hip(launch(k_litmus, dim3(8), dim3(64), static_cast<hipStream_t>(stream),
                        w, iters, xcd_a, xcd_b, kind, r, to));
}

int ar_probe_loadchain(void* work, int64_t bytes, int32_t iters, void* result,
                       void* stream) {
  if (!work || !result || iters < 1) return AR_EINVAL;
  if (bytes < 4096 || bytes > (int64_t(1) << 31) || (bytes & (bytes - 1))) return AR_EINVAL;
  if (!aligned(work, 256) || !aligned(result, 8)) return AR_EALIGN;
  const uint32_t n = (uint32_t)(bytes / 4);
  const uint32_t stride = 4099u;   // ~16 KiB hops, odd: one cycle through n
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc = map_hip(launch(k_chain_init, dim3(1024), dim3(kBlock), s,
                          static_cast<uint32_t*>(work), n, stride));
  if (rc) return rc;
  return map_hip(launch(k_chain, dim3(1), dim3(64), s,
                        static_cast<const uint32_t*>(work), (uint32_t)bytes, iters,
                        static_cast<uint64_t*>(result)));
}

int ar_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (!src || !dst || bytes < 0 || (bytes % 16)) return AR_EINVAL;
  if (!aligned(src, 16) || !aligned(dst, 16)) return AR_EALIGN;
  if (bytes == 0) return AR_OK;
  const uint64_t n16 = (uint64_t)bytes / 16;
  uint64_t blocks = (n16 + kBlock - 1) / kBlock;
  if (blocks > 8192) blocks = 8192;
  return map_hip(launch(k_copy, dim3((unsigned)blocks), dim3(kBlock),
                        static_cast<hipStream_t>(stream),
                        static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16));
}

int ar_probe_empty(void* stream) {
  return map_hip(launch(k_empty, dim3(1), dim3(64), static_cast<hipStream_t>(stream)));
}

int ar_probe_placement(int32_t blocks, int32_t threads, void* work, void* result,
                       void* stream) {
  if (!work || !result || blocks < 1 || threads < 1 || threads > 1024) return AR_EINVAL;
  if (!aligned(work, 256) || !aligned(result, 4)) return AR_EALIGN;
  DeviceInfo di;
  int rc = device_info(&di);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = map_hip(launch(k_fill_zero, dim3(1), dim3(kBlock), s, static_cast<uint32_t*>(work),
                      1u));
  if (rc) return rc;
  return map_hip(launch(k_placement, dim3((unsigned)blocks), dim3((unsigned)threads), s,
                        static_cast<int32_t*>(result), static_cast<uint32_t*>(work),
                        (uint32_t)blocks, ns_to_ticks(1000000000ull, di.wallclock_hz)));
}

int ar_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
