// ar_collectives.hip -- the standalone all-gather and the two-shot
// all-reduce on the same self-synchronizing transfers (gfx950).
//
// "flash-comm: Self-Synchronizing Collective Communication for LLM
// Decoding", abstract: the transfers that carry their own readiness evidence
// also serve a standalone all-gather.  "SiFAR: Synchronization-Free
// All-Reduce for Low-Latency LLM Inference", abstract: the two-shot form
// (reduce-scatter of shares, then all-gather of the reduced shares) is the
// one that scales to more GPUs.  Here each share and each reduced share
// travels with the one-shot encodings (LL, LL128, sentinel) and the same
// dual-buffered epochs; the two exchanges use two receive regions.
// "Why Microseconds Matter in AI Infrastructure", section "Communication is
// becoming part of GPU execution": the producer that sends from its own
// epilogue (a per-rank scale), and the chained simulator in which each
// all-reduce's result feeds that producer for the next one, in one launch.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "../../include/ar.h"
#include "../../include/ar_dev.h"
#include "ar_host.h"
#include "../../include/ar_protocols.h"

namespace ar {

// =========================================================== stream-ordered

struct GatherArgs {
  uint16_t* out;
  int64_t out_stride, row_stride, count;
  const uint8_t* scratch;
  uint32_t scratch_bytes;
  uint32_t E, slot_bytes;
  int32_t nranks, nconsumers, tiles;
  uint32_t seq, parity;
  int* ctrl;
  uint64_t timeout_ticks;
  int32_t rearm;
};

// One wave per (consumer, source rank, tile): poll, validate, decode into
// the source's output row.
template <int P>
__global__ __launch_bounds__(kBlock) void k_gather(GatherArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int per_c = a.nranks * a.tiles;
  const int c = gw / per_c;
  if (c >= a.nconsumers) return;
  const int rem = gw - c * per_c;
  const int r = rem / a.tiles;
  const int tile = rem - r * a.tiles;
  const ar_dev::buffer b = ar_dev::make(a.scratch, a.scratch_bytes, a.slot_bytes, a.E,
                                        a.nranks, a.nconsumers, a.count, a.seq, a.parity);
  uint32_t w[4];
  if (ar_dev::recv<P>(b, c, r, tile, lane, a.rearm != 0, a.ctrl, a.timeout_ticks, w) != 0)
    return;
  ar_dev::store_row<P>(a.out + (int64_t)c * a.out_stride + (int64_t)r * a.row_stride,
                       a.count, tile, lane, w);
}

// --------------------------------------------------- producer epilogue --

// y = bf16_rne(f32(x) * s) on the lane's data words (the producer whose
// epilogue sends; one binary32 multiplication per element).
__device__ __forceinline__ void scale_words(uint32_t w[4], float s) {
#pragma unroll
  for (int d = 0; d < 4; ++d)
    w[d] = pack2(to_bf16(bf_lo(w[d]) * s), to_bf16(bf_hi(w[d]) * s));
}

struct ScaleArgs {
  const uint16_t* in;
  int64_t in_stride;
  const float* scales;
  uint16_t* out;              // unfused producer only
  int64_t out_stride;
  ar_dev::buffer b;           // fused producer only
  int32_t nranks, tiles;
  int64_t count;
};

// Fused: one wave per (rank, tile) computes its scaled payload chunk and
// broadcasts it from registers with the device-callable interface.
template <int P>
__global__ __launch_bounds__(kBlock) void k_scale_send(ScaleArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int r = gw / a.tiles;
  if (r >= a.nranks) return;
  const int tile = gw - r * a.tiles;
  uint32_t w[4];
  load_chunk<P>(a.in + (int64_t)r * a.in_stride,
                (uint32_t)(((a.count * 2) + 15) & ~int64_t(15)), tile, lane, w);
  scale_words(w, a.scales[r]);
  mask_words(w, chunk_keep<P>(a.count, tile, lane));
  ar_dev::broadcast<P>(a.b, r, tile, lane, w);
  if (P == kLL128) {
    ar_dev::fence();
    ar_dev::broadcast_flags(a.b, r, tile, lane);
  }
}

// Unfused: the same producer writing its result to HBM (8 elements a lane).
__global__ __launch_bounds__(kBlock) void k_scale_rows(ScaleArgs a) {
  const int64_t per_row = (a.count + 7) / 8;
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t r = i / per_row;
  if (r >= a.nranks) return;
  const int64_t first = (i - r * per_row) * 8;
  uint32_t w[4];
  // 8 elements from a 16-byte aligned start; both helpers stop at count
  load_elems(a.in + r * a.in_stride, a.count, first, 8, w);
  scale_words(w, a.scales[r]);
  store_elems(a.out + r * a.out_stride, a.count, first, 8, w);
}

struct TsArgs {
  const uint16_t* in;      // pack only
  int64_t in_stride;
  uint16_t* out;           // reduce / gather
  int64_t out_stride, count, width;
  const uint8_t* scratch;
  uint32_t scratch_bytes, slot_bytes, ag0;   // ag0: byte offset of the all-gather region
  int32_t nranks, tiles;                     // tiles of one full share
  uint32_t seq, parity;
  int* ctrl;
  uint64_t timeout_ticks;
  int32_t rearm;
};

__device__ __forceinline__ void share_of(int64_t count, int64_t width, int k, int64_t& lo,
                                         int64_t& m) {
  int64_t a = (int64_t)k * width;
  if (a > count) a = count;
  int64_t b = a + width;
  if (b > count) b = count;
  lo = a;
  m = b - a;
}

// One wave per (rank r, consumer c, tile of share c): encode rank r's share c
// into the reduce-scatter slot r of consumer c.
template <int P>
__global__ __launch_bounds__(kBlock) void k_ts_pack(TsArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int per_r = a.nranks * a.tiles;
  const int r = gw / per_r;
  if (r >= a.nranks) return;
  const int rem = gw - r * per_r;
  const int c = rem / a.tiles;
  const int tile = rem - c * a.tiles;
  int64_t lo, m;
  share_of(a.count, a.width, c, lo, m);
  const uint32_t E = enc_bytes<P>(m);
  if ((uint32_t)tile * kTileBytes >= E) return;
  const rsrc_t rs = make_rsrc(a.scratch, a.scratch_bytes);
  const uint32_t dst0 =
      (((uint32_t)c * 2u + a.parity) * (uint32_t)a.nranks + (uint32_t)r) * a.slot_bytes;
  const uint16_t* row = a.in + (int64_t)r * a.in_stride + lo;
  produce_data<P>(rs, dst0, 0u, 1, -1, row, (uint32_t)((m * 2 + 15) & ~int64_t(15)), m,
                  tile, E, a.seq, lane);
  if (P == kLL128) {
    fence_release();
    produce_flags(rs, dst0, 0u, 1, -1, tile, E, a.seq, lane);
  }
}

// One wave per (consumer c, tile of share c): poll and validate share c of
// every rank, reduce in rank order, write it to consumer c's output and send
// it to every other consumer's all-gather slot c.
template <int P, int NMAX>
__global__ __launch_bounds__(kBlock) void k_ts_reduce(TsArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int c = gw / a.tiles;
  if (c >= a.nranks) return;
  const int tile = gw - c * a.tiles;
  int64_t lo, m;
  share_of(a.count, a.width, c, lo, m);
  const uint32_t E = enc_bytes<P>(m);
  if ((uint32_t)tile * kTileBytes >= E) return;
  const rsrc_t rs = make_rsrc(a.scratch, a.scratch_bytes);
  const uint32_t N = (uint32_t)a.nranks;
  const uint32_t src0 = ((uint32_t)c * 2u + a.parity) * N * a.slot_bytes;
  u32x4 v[NMAX];
  if (poll_tile<P, NMAX>(rs, src0, a.slot_bytes, a.nranks, tile, E, a.seq,
                         seq_prev(seq_prev(a.seq)), a.rearm != 0, -1,
                         u32x4{0u, 0u, 0u, 0u}, a.ctrl, a.timeout_ticks, lane, v) != 0)
    return;
  uint32_t o[4];
  reduce_words<P, NMAX>(v, a.nranks, o);
  mask_words(o, chunk_keep<P>(m, tile, lane));
  int64_t first;
  int n;
  lane_elems<P>(tile, lane, first, n);
  if ((uint32_t)tile * kTileBytes + (uint32_t)lane * 16u < E)
    store_elems(a.out + (int64_t)c * a.out_stride + lo, m, first, n, o);
  const u32x4 enc = encode_words<P>(o, lane, a.seq);
  const uint32_t dst0 = a.ag0 + (a.parity * N + (uint32_t)c) * a.slot_bytes;
  const uint32_t cstride = 2u * N * a.slot_bytes;
  store_chunk<P>(rs, dst0, cstride, a.nranks, c, tile, E, lane, enc);
  if (P == kLL128) {
    fence_release();
    produce_flags(rs, dst0, cstride, a.nranks, c, tile, E, a.seq, lane);
  }
}

// One wave per (consumer c, share k != c, tile of share k): poll, validate
// and decode the reduced share k into consumer c's output.
template <int P>
__global__ __launch_bounds__(kBlock) void k_ts_gather(TsArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int per_c = a.nranks * a.tiles;
  const int c = gw / per_c;
  if (c >= a.nranks) return;
  const int rem = gw - c * per_c;
  const int k = rem / a.tiles;
  const int tile = rem - k * a.tiles;
  if (k == c) return;
  int64_t lo, m;
  share_of(a.count, a.width, k, lo, m);
  const uint32_t E = enc_bytes<P>(m);
  if ((uint32_t)tile * kTileBytes >= E) return;
  const rsrc_t rs = make_rsrc(a.scratch, a.scratch_bytes);
  const uint32_t loff = (uint32_t)tile * kTileBytes + (uint32_t)lane * 16u;
  const uint32_t at =
      a.ag0 + (((uint32_t)c * 2u + a.parity) * (uint32_t)a.nranks + (uint32_t)k) * a.slot_bytes +
      loff;
  u32x4 v;
  if (poll_chunk<P>(rs, at, loff < E, a.seq, seq_prev(seq_prev(a.seq)), a.rearm != 0,
                    a.ctrl, a.timeout_ticks, lane, v) != 0)
    return;
  store_chunk_elems<P>(a.out + (int64_t)c * a.out_stride + lo, m, tile, E, lane, v);
}

// ================================================================ simulator

struct CollSimArgs {
  const uint16_t* in;
  int64_t in_stride;
  uint16_t* out;
  int64_t out_stride, row_stride, count, width;
  const uint8_t* scratch;
  uint32_t scratch_bytes, slot_bytes, ag0, E;
  int* ctrl;
  int32_t nranks, nops;
  int32_t W, Q, T, TPW;
  uint32_t seq0, parity0;
  uint64_t timeout_ticks;
  const uint32_t* delay;
  uint64_t* trace;
  const float* scales;        // chained simulator only
};

__device__ __forceinline__ void sim_delay(const CollSimArgs& a, int op, int g) {
  if (!a.delay) return;
  const uint32_t d = a.delay[(int64_t)op * a.nranks + g];
  if (d) {
    const uint64_t t0 = now_ticks();
    while (now_ticks() - t0 < (uint64_t)d) __builtin_amdgcn_s_sleep(2);
  }
}

__device__ __forceinline__ void trace_max(const CollSimArgs& a, int64_t idx) {
  __hip_atomic_fetch_max(reinterpret_cast<unsigned long long*>(a.trace) + idx,
                         (unsigned long long)now_ticks(), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup b -> (rank g, tile group tg) with the all-reduce simulator's
// XCD-aware placement: workgroup b runs on XCD (s + b) mod 8 (round-robin
// dispatch from a start s) and rank g's groups are rotated by g, so a
// producer and the consumer reading it sit on different XCDs.  Returns
// false for workgroups without work.
__device__ __forceinline__ bool sim_place(const CollSimArgs& a, int& g, int& tg) {
  const int b = blockIdx.x;
  const int x = b & 7;
  const int q = b >> 3;
  g = q / a.Q;
  const int qq = q - g * a.Q;
  if (g >= a.nranks) return false;
  tg = qq * 8 + ((x - (g & 7)) & 7);
  return tg < a.T;
}

// All-gather simulator: a workgroup of nranks waves per (rank g, tile group
// tg), wave w paired with peer w.  Per op, wave w sends rank g's tiles to
// consumer w, then polls peer w's tiles and decodes them straight into row
// w of rank g's output (no staging: nothing is reduced); the rank's own
// wave writes its own row.  One workgroup barrier per op: a rank starts op
// i+1 once it holds all of op i (LL with one tile per group: none, below).
// TB: tiles whose input loads overlap when a wave walks several (1: one
// load, then its stores, at a time).
template <int P, int NMAX, int TB, bool EXTRAS>
__global__ __launch_bounds__(1024) void k_sim_gather(CollSimArgs a) {
  if constexpr (!EXTRAS) {
    a.delay = nullptr;
    a.trace = nullptr;
  }
  __shared__ int lds_err;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x >> 6;
  int g, tg;
  if (!sim_place(a, g, tg)) return;                // whole workgroup
  const int G = a.W;
  const int mine = (a.T - 1 - tg) / G + 1;
  const bool own = w == g;
  const rsrc_t rs = make_rsrc(a.scratch, a.scratch_bytes);
  const uint32_t N = (uint32_t)a.nranks;
  const int tstride = 2 * a.nranks;
  const uint32_t row_bytes = (uint32_t)(((a.count * 2) + 15) & ~int64_t(15));
  // one tile per group: the next op's payload chunk is loaded while this op
  // is exchanged, so no input load sits between two ops' sends
  const bool pipelined = mine == 1;
  // LL, one tile per group, no delays or trace: no barrier at all.  Wave w
  // sends op i+1 to peer w once it holds peer w's op i, which peer w sent
  // after reading this rank's op i-1: the licence is pairwise, and each
  // wave goes at its own pace (a wave whose poll gives up just ends).
  const bool unpaced = !EXTRAS && P == kLL && pipelined;
  const int keep = chunk_keep<P>(a.count, tg, lane);
  uint32_t wnext[4] = {0u, 0u, 0u, 0u};
  if (pipelined) load_chunk<P>(a.in + (int64_t)g * a.in_stride, row_bytes, tg, lane, wnext);
  if (threadIdx.x == 0) lds_err = 0;
  __syncthreads();
  if (a.trace && lane == 0 && w == 0) {
    __hip_atomic_fetch_min(reinterpret_cast<unsigned long long*>(a.trace) +
                               (int64_t)a.nops * tstride,
                           (unsigned long long)now_ticks(), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  }
  uint32_t seq = a.seq0;
  uint32_t par = a.parity0;
  for (int op = 0; op < a.nops; ++op) {
    const uint32_t stale = seq_prev(seq_prev(seq));
    const uint16_t* row = a.in + ((int64_t)op * a.nranks + g) * a.in_stride;
    uint16_t* orow = a.out + ((int64_t)op * a.nranks + g) * a.out_stride;
    u32x4 mine_v = u32x4{0u, 0u, 0u, 0u};
    if (pipelined) {
      mask_words(wnext, keep);
      mine_v = encode_words<P>(wnext, lane, seq);
    }
    if (!own) {
      sim_delay(a, op, g);
      // this wave's earlier stores (sentinel re-arms) complete before it sends
      if (P == kSentinel) fence_release();
      const uint32_t dst0 = (((uint32_t)w * 2u + par) * N + (uint32_t)g) * a.slot_bytes;
      if (TB == 1) {
        if (pipelined)
          store_chunk<P>(rs, dst0, 0u, 1, -1, tg, a.E, lane, mine_v);
        else
          for (int k = 0; k < mine; ++k)
            produce_data<P>(rs, dst0, 0u, 1, -1, row, row_bytes, a.count, tg + k * G, a.E,
                            seq, lane);
      } else {
        // the loads of up to TB tiles in flight together, then their stores
        // (a tile past the payload reads nothing and stores nothing)
        for (int k0 = 0; k0 < mine; k0 += TB) {
          uint32_t wv[TB][4];
#pragma unroll
          for (int j = 0; j < TB; ++j) load_chunk<P>(row, row_bytes, tg + (k0 + j) * G, lane, wv[j]);
#pragma unroll
          for (int j = 0; j < TB; ++j) {
            if (k0 + j >= mine) break;
            const int tile = tg + (k0 + j) * G;
            mask_words(wv[j], chunk_keep<P>(a.count, tile, lane));
            store_chunk<P>(rs, dst0, 0u, 1, -1, tile, a.E, lane, encode_words<P>(wv[j], lane, seq));
          }
        }
      }
      if (P == kLL128) {
        fence_release();
        for (int k = 0; k < mine; ++k)
          produce_flags(rs, dst0, 0u, 1, -1, tg + k * G, a.E, seq, lane);
      }
      if (a.trace) {
        fence_release();
        if (lane == 0) trace_max(a, (int64_t)op * tstride + g);
      }
      // the next op's load goes out after this op's sends, so that no wait
      // for this wave's stores (the fences above) also waits for it
      if (pipelined && op + 1 < a.nops)
        load_chunk<P>(row + (int64_t)a.nranks * a.in_stride, row_bytes, tg, lane, wnext);
      const uint32_t src0 = (((uint32_t)g * 2u + par) * N + (uint32_t)w) * a.slot_bytes;
      for (int k = 0; k < mine; ++k) {
        const int tile = tg + k * G;
        const uint32_t loff = (uint32_t)tile * kTileBytes + (uint32_t)lane * 16u;
        u32x4 v;
        if (poll_chunk<P>(rs, src0 + loff, loff < a.E, seq, stale, true, a.ctrl,
                          a.timeout_ticks, lane, v) != 0) {
          if (lane == 0) lds_err = 1;
          if (unpaced) return;                     // no barrier to meet
          break;
        }
        store_chunk_elems<P>(orow + (int64_t)w * a.row_stride, a.count, tile, a.E, lane, v);
      }
    } else {
      if (TB == 1) {
        if (pipelined && op + 1 < a.nops)
          load_chunk<P>(row + (int64_t)a.nranks * a.in_stride, row_bytes, tg, lane, wnext);
        for (int k = 0; k < mine; ++k) {
          const int tile = tg + k * G;
          store_chunk_elems<P>(orow + (int64_t)g * a.row_stride, a.count, tile, a.E, lane,
                               pipelined ? mine_v
                                         : encode_chunk<P>(row, row_bytes, a.count, tile, lane,
                                                           seq));
        }
      } else {
        for (int k0 = 0; k0 < mine; k0 += TB) {
          uint32_t wv[TB][4];
#pragma unroll
          for (int j = 0; j < TB; ++j) load_chunk<P>(row, row_bytes, tg + (k0 + j) * G, lane, wv[j]);
#pragma unroll
          for (int j = 0; j < TB; ++j) {
            if (k0 + j >= mine) break;
            const int tile = tg + (k0 + j) * G;
            mask_words(wv[j], chunk_keep<P>(a.count, tile, lane));
            store_chunk_elems<P>(orow + (int64_t)g * a.row_stride, a.count, tile, a.E, lane,
                                 encode_words<P>(wv[j], lane, seq));
          }
        }
      }
    }
    if (!unpaced) {
      __syncthreads();
      if (lds_err) return;                         // whole workgroup
    }
    if (a.trace && own && lane == 0) trace_max(a, (int64_t)op * tstride + a.nranks + g);
    seq = seq_next(seq);
    par ^= 1u;
  }
}

// Two-shot simulator: a workgroup of nranks waves per (rank g, tile group tg
// of the share tiles), wave w paired with peer w.  Per op:
//  1. reduce-scatter: wave w sends every tile of the group of rank g's share
//     w to rank w;
//  2. per tile t: wave w polls tile t of rank w's share g and stages it in
//     LDS row w (the own wave stages its own share-g chunk); after a barrier
//     the own wave reduces the staged rows in rank order, writes the reduced
//     tile to rank g's output and stages it; after a second barrier wave w
//     sends the reduced tile to rank w (all-gather);
//  3. wave w polls every tile of rank w's reduced share w and decodes it
//     into rank g's output.
// No step waits on a peer's progress in the same op beyond the data it
// needs: every reduce-scatter chunk is out before any wave polls, and every
// reduced tile is sent before any wave polls the all-gather.
// A wave waits for its own earlier stores before each reduce-scatter send.
// Both slots of a parity are written again two ops later, and a peer gets
// there only after it has received this wave's reduce-scatter chunk of the
// op in between; so the sentinel re-arms of an op (the wave's own, of the
// slots it polled) complete before that licence is sent.
// BATCH: share tiles received, reduced and all-gathered per pair of
// workgroup barriers (1 when every workgroup owns one tile, 2 otherwise; a
// wave polls its peer's two chunks together).  LL with one tile per group
// takes one barrier per op instead (the pairwise loop below).
template <int P, int NMAX, int BATCH, bool EXTRAS>
__global__ __launch_bounds__(1024) void k_sim_twoshot(CollSimArgs a) {
  if constexpr (!EXTRAS) {
    a.delay = nullptr;
    a.trace = nullptr;
  }
  // the pairwise LL loop below stages op i's rows in buffer parity(i)
  constexpr bool kPairwise = BATCH == 1 && !EXTRAS && P == kLL;
  __shared__ u32x4 lds[kPairwise ? 2 : BATCH][NMAX][kWave];
  __shared__ u32x4 red[BATCH][kWave];
  __shared__ int lds_err;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x >> 6;
  int g, tg;
  if (!sim_place(a, g, tg)) return;                // whole workgroup
  const int G = a.W;
  const int mine = (a.T - 1 - tg) / G + 1;
  const bool own = w == g;
  const rsrc_t rs = make_rsrc(a.scratch, a.scratch_bytes);
  const uint32_t N = (uint32_t)a.nranks;
  const int tstride = 2 * a.nranks;
  int64_t lo_g, m_g, lo_w, m_w;
  share_of(a.count, a.width, g, lo_g, m_g);
  share_of(a.count, a.width, w, lo_w, m_w);
  const uint32_t E_g = enc_bytes<P>(m_g);
  const uint32_t E_w = enc_bytes<P>(m_w);
  const uint32_t rb_w = (uint32_t)((m_w * 2 + 15) & ~int64_t(15));
  const uint32_t rb_g = (uint32_t)((m_g * 2 + 15) & ~int64_t(15));
  // one share tile per group: the next op's chunk (share w for a sender,
  // share g for the own wave) is loaded while this op is exchanged
  const bool pipelined = mine == 1;
  const int64_t lo_mine = own ? lo_g : lo_w;
  const uint32_t rb_mine = own ? rb_g : rb_w;
  const int keep = chunk_keep<P>(own ? m_g : m_w, tg, lane);
  uint32_t wnext[4] = {0u, 0u, 0u, 0u};
  if (pipelined)
    load_chunk<P>(a.in + (int64_t)g * a.in_stride + lo_mine, rb_mine, tg, lane, wnext);
  if (threadIdx.x == 0) lds_err = 0;
  __syncthreads();
  if (a.trace && lane == 0 && w == 0) {
    __hip_atomic_fetch_min(reinterpret_cast<unsigned long long*>(a.trace) +
                               (int64_t)a.nops * tstride,
                           (unsigned long long)now_ticks(), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  }
  // One tile per group, LL: one workgroup barrier per op.  After it every
  // wave sums the staged rows itself (the same rank-order sum, so the same
  // bits) and wave w sends the reduced tile to peer w at once, then polls
  // peer w's reduced share and goes on to the next op without waiting for
  // the other waves.  Licences, pairwise: wave w sends op i+1's chunk to
  // peer w after it has received peer w's reduced share of op i, which peer
  // w sent after reading this rank's chunk of op i (and of op i-1 before
  // it), so the reduce-scatter slot of op i+1's parity is free; and it
  // sends op i+1's reduced tile after receiving peer w's chunk of op i+1,
  // which peer w sent after reading the reduced tile of op i-1.  Staging
  // rows alternate between two LDS buffers by parity: wave w writes its row
  // of op i+2 after it has passed the barrier of op i+1, which every wave
  // reaches only after it has read the rows of op i.
  if constexpr (kPairwise) {
    const uint32_t loff = (uint32_t)tg * kTileBytes + (uint32_t)lane * 16u;
    const int keep_g = chunk_keep<P>(m_g, tg, lane);
    int64_t first_g;
    int n_g;
    lane_elems<P>(tg, lane, first_g, n_g);
    uint32_t seq = a.seq0;
    uint32_t par = a.parity0;
    bool failed = false;                           // this wave's last poll gave up
    for (int op = 0; op < a.nops; ++op) {
      const uint32_t stale = seq_prev(seq_prev(seq));
      const uint16_t* row = a.in + ((int64_t)op * a.nranks + g) * a.in_stride;
      uint16_t* orow = a.out + ((int64_t)op * a.nranks + g) * a.out_stride;
      const uint32_t rs_dst = (((uint32_t)w * 2u + par) * N + (uint32_t)g) * a.slot_bytes;
      const uint32_t rs_src = (((uint32_t)g * 2u + par) * N + (uint32_t)w) * a.slot_bytes;
      mask_words(wnext, keep);
      const u32x4 mine_v = encode_words<P>(wnext, lane, seq);
      if (!own) store_chunk<P>(rs, rs_dst, 0u, 1, -1, tg, E_w, lane, mine_v);
      if (op + 1 < a.nops)
        load_chunk<P>(row + (int64_t)a.nranks * a.in_stride + lo_mine, rb_mine, tg, lane,
                      wnext);
      if (!own) {
        u32x4 got;
        if (failed || poll_chunk<P>(rs, rs_src + loff, loff < E_g, seq, stale, true,
                                    a.ctrl, a.timeout_ticks, lane, got) != 0) {
          if (lane == 0) lds_err = 1;
        } else {
          lds[par][w][lane] = got;
        }
      } else {
        lds[par][g][lane] = mine_v;
      }
      __syncthreads();
      if (lds_err) return;                         // whole workgroup
      u32x4 v[NMAX];
#pragma unroll
      for (int r = 0; r < NMAX; ++r)
        v[r] = (r < a.nranks) ? lds[par][r][lane] : u32x4{0u, 0u, 0u, 0u};
      uint32_t o[4];
      reduce_words<P, NMAX>(v, a.nranks, o);
      mask_words(o, keep_g);
      if (own) {
        if (loff < E_g) store_elems(orow + lo_g, m_g, first_g, n_g, o);
      } else {
        store_chunk<P>(rs, a.ag0 + rs_dst, 0u, 1, -1, tg, E_g, lane,
                       encode_words<P>(o, lane, seq));
        u32x4 got;
        if (poll_chunk<P>(rs, a.ag0 + rs_src + loff, loff < E_w, seq, stale, true, a.ctrl,
                          a.timeout_ticks, lane, got) != 0) {
          // the next op's barrier ends the workgroup (after the last op,
          // the status word holds the error)
          failed = true;
        } else {
          store_chunk_elems<P>(orow + lo_w, m_w, tg, E_w, lane, got);
        }
      }
      seq = seq_next(seq);
      par ^= 1u;
    }
    return;
  }
  uint32_t seq = a.seq0;
  uint32_t par = a.parity0;
  for (int op = 0; op < a.nops; ++op) {
    const uint32_t stale = seq_prev(seq_prev(seq));
    const uint16_t* row = a.in + ((int64_t)op * a.nranks + g) * a.in_stride;
    uint16_t* orow = a.out + ((int64_t)op * a.nranks + g) * a.out_stride;
    // reduce-scatter slots: to consumer w from g, and here (g) from w
    const uint32_t rs_dst = (((uint32_t)w * 2u + par) * N + (uint32_t)g) * a.slot_bytes;
    const uint32_t rs_src = (((uint32_t)g * 2u + par) * N + (uint32_t)w) * a.slot_bytes;
    const uint32_t ag_dst = a.ag0 + rs_dst;
    const uint32_t ag_src = a.ag0 + rs_src;
    if (!own) sim_delay(a, op, g);
    u32x4 mine_v = u32x4{0u, 0u, 0u, 0u};        // pipelined: this op's chunk
    if (pipelined) {
      mask_words(wnext, keep);
      mine_v = encode_words<P>(wnext, lane, seq);
    }
    // ---- 1. reduce-scatter sends: every tile of the group ----
    if (!own) {
      if (P == kSentinel) fence_release();
      if (pipelined) {
        store_chunk<P>(rs, rs_dst, 0u, 1, -1, tg, E_w, lane, mine_v);
      } else {
        // the loads of up to TB tiles in flight together, then their stores
        // (a tile past the share reads nothing and stores nothing); 16-wave
        // workgroups have 128 registers a lane, hence the smaller group
        constexpr int TB = NMAX >= 16 ? 2 : 4;
        for (int k0 = 0; k0 < mine; k0 += TB) {
          uint32_t wv[TB][4];
#pragma unroll
          for (int j = 0; j < TB; ++j)
            load_chunk<P>(row + lo_w, rb_w, tg + (k0 + j) * G, lane, wv[j]);
#pragma unroll
          for (int j = 0; j < TB; ++j) {
            if (k0 + j >= mine) break;
            const int tile = tg + (k0 + j) * G;
            mask_words(wv[j], chunk_keep<P>(m_w, tile, lane));
            store_chunk<P>(rs, rs_dst, 0u, 1, -1, tile, E_w, lane,
                           encode_words<P>(wv[j], lane, seq));
          }
        }
      }
      if (P == kLL128) {
        fence_release();
        for (int k = 0; k < mine; ++k)
          produce_flags(rs, rs_dst, 0u, 1, -1, tg + k * G, E_w, seq, lane);
      }
      if (a.trace) {
        fence_release();
        if (lane == 0) trace_max(a, (int64_t)op * tstride + g);
      }
    }
    // the next op's load goes out after this op's sends, so that no wait for
    // this wave's stores (the fences above) also waits for it
    if (pipelined && op + 1 < a.nops)
      load_chunk<P>(row + (int64_t)a.nranks * a.in_stride + lo_mine, rb_mine, tg, lane, wnext);
    // ---- 2. per BATCH tiles: receive share g, reduce, send reduced ----
    for (int k0 = 0; k0 < mine; k0 += BATCH) {
      const int nb = (mine - k0) < BATCH ? (mine - k0) : BATCH;
      if (!own) {
        u32x4 got[BATCH];
        int st;
        if constexpr (BATCH == 1) {
          const uint32_t loff = (uint32_t)(tg + k0 * G) * kTileBytes + (uint32_t)lane * 16u;
          st = poll_chunk<P>(rs, rs_src + loff, loff < E_g, seq, stale, true, a.ctrl,
                             a.timeout_ticks, lane, got[0]);
        } else {
          uint32_t at[BATCH];
          bool act[BATCH];
#pragma unroll
          for (int j = 0; j < BATCH; ++j) {
            const uint32_t loff =
                (uint32_t)(tg + (k0 + j) * G) * kTileBytes + (uint32_t)lane * 16u;
            at[j] = rs_src + loff;
            act[j] = j < nb && loff < E_g;
          }
          st = poll_chunks<P, BATCH>(rs, at, act, nb, seq, stale, true, a.ctrl,
                                     a.timeout_ticks, lane, got);
        }
        if (st != 0) {
          if (lane == 0) lds_err = 1;
        } else {
#pragma unroll
          for (int j = 0; j < BATCH; ++j)
            if (j < nb) lds[j][w][lane] = got[j];
        }
      } else {
#pragma unroll
        for (int j = 0; j < BATCH; ++j)
          if (j < nb)
            lds[j][g][lane] =
                pipelined ? mine_v
                          : encode_chunk<P>(row + lo_g, rb_g, m_g, tg + (k0 + j) * G, lane, seq);
      }
      __syncthreads();
      if (lds_err) return;                         // whole workgroup
      // fixed-order reduce of share g, tiles k0.. (own wave)
      if (own) {
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
          if (j >= nb) break;
          const int tile = tg + (k0 + j) * G;
          const uint32_t loff = (uint32_t)tile * kTileBytes + (uint32_t)lane * 16u;
          u32x4 v[NMAX];
#pragma unroll
          for (int r = 0; r < NMAX; ++r)
            v[r] = (r < a.nranks) ? lds[j][r][lane] : u32x4{0u, 0u, 0u, 0u};
          uint32_t o[4];
          reduce_words<P, NMAX>(v, a.nranks, o);
          mask_words(o, chunk_keep<P>(m_g, tile, lane));
          int64_t first;
          int n;
          lane_elems<P>(tile, lane, first, n);
          if (loff < E_g) store_elems(orow + lo_g, m_g, first, n, o);
          red[j][lane] = u32x4{o[0], o[1], o[2], o[3]};
        }
      }
      __syncthreads();
      if (!own) {
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
          if (j >= nb) break;
          const u32x4 r4 = red[j][lane];
          const uint32_t o[4] = {r4.x, r4.y, r4.z, r4.w};
          store_chunk<P>(rs, ag_dst, 0u, 1, -1, tg + (k0 + j) * G, E_g, lane,
                         encode_words<P>(o, lane, seq));
        }
        if (P == kLL128) {
          fence_release();
          for (int j = 0; j < nb; ++j)
            produce_flags(rs, ag_dst, 0u, 1, -1, tg + (k0 + j) * G, E_g, seq, lane);
        }
      }
    }
    // ---- 3. all-gather receive: every tile of peer w's reduced share ----
    if (!own) {
      for (int k = 0; k < mine; ++k) {
        const int tile = tg + k * G;
        const uint32_t loff = (uint32_t)tile * kTileBytes + (uint32_t)lane * 16u;
        u32x4 got;
        if (poll_chunk<P>(rs, ag_src + loff, loff < E_w, seq, stale, true, a.ctrl,
                          a.timeout_ticks, lane, got) != 0) {
          if (lane == 0) lds_err = 1;
          break;
        }
        store_chunk_elems<P>(orow + lo_w, m_w, tile, E_w, lane, got);
      }
    }
    __syncthreads();
    if (lds_err) return;
    if (a.trace && own && lane == 0) trace_max(a, (int64_t)op * tstride + a.nranks + g);
    seq = seq_next(seq);
    par ^= 1u;
  }
}

// Poll tile `tile` of the all-gather slots of every source but `skip`, each
// holding the reduced share of its source (so each source has its own
// encoded length), in whatever order they arrive; validate from the
// evidence and re-arm (SENTINEL).  LL128 first probes every source's last
// line flag (lane r watches source r), then reads after an acquire, as
// poll_tile does.  Returns 0, kEtimeout or kEcorrupt; chunks end in v.
template <int P, int NMAX>
__device__ __forceinline__ int poll_shares(rsrc_t rs, uint32_t src0, uint32_t slot_bytes,
                                           int nranks, int skip, int tile, int64_t count,
                                           int64_t width, uint32_t seq, uint32_t stale,
                                           int* ctrl, uint64_t timeout_ticks, int lane,
                                           u32x4 (&v)[NMAX]) {
  const uint32_t tile0 = (uint32_t)tile * kTileBytes;
  const uint32_t loff = tile0 + (uint32_t)lane * 16u;
  uint32_t pending = 0u;                           // wave-uniform
  uint32_t E[NMAX];
#pragma unroll
  for (int r = 0; r < NMAX; ++r) {
    v[r] = u32x4{0u, 0u, 0u, 0u};
    int64_t lo, m;
    share_of(count, width, r, lo, m);
    E[r] = enc_bytes<P>(m);
    if (r < nranks && r != skip && tile0 < E[r]) pending |= 1u << r;
  }
  if (pending == 0u) return 0;
  Waiter wt(timeout_ticks, ctrl);
  if (P == kLL128) {
    int64_t lo, m;
    share_of(count, width, lane, lo, m);
    const uint32_t El = enc_bytes<P>(m);
    const uint32_t tile_end = (tile0 + kTileBytes < El) ? tile0 + kTileBytes : El;
    uint32_t waiting = pending;
    while (true) {
      const bool mine = lane < nranks && ((waiting >> lane) & 1u);
      bool ok = true, bad = false;
      if (mine) {
        const u32x2 f = ld8(rs, src0 + (uint32_t)lane * slot_bytes + tile_end - 8u);
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
  }
  while (true) {
#pragma unroll
    for (int r = 0; r < NMAX; ++r)
      if (((pending >> r) & 1u) && loff < E[r]) v[r] = ld16(rs, src0 + r * slot_bytes + loff);
    uint32_t fresh = 0u;
    bool corrupt = false;
#pragma unroll
    for (int r = 0; r < NMAX; ++r) {
      if ((pending >> r) & 1u) {
        bool ok = true, bad = false;
        if (loff < E[r]) {
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
    if (P == kSentinel && fresh != 0u) {
      const u32x4 armed = u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
#pragma unroll
      for (int r = 0; r < NMAX; ++r)
        if (((fresh >> r) & 1u) && loff < E[r]) st16(rs, src0 + r * slot_bytes + loff, armed);
    }
    pending &= ~fresh;
    if (pending == 0u) break;
    if (!wt.again(lane)) return kEtimeout;
  }
  return 0;
}

// Two-shot simulator for larger shares: one wave per (rank g, share tile
// group), no workgroup barrier.  Per op and tile t the wave
//  1. sends tile t of each share w of rank g's payload to rank w;
//  2. polls tile t of share g from every other rank at once (its own share-g
//     chunk stays in registers), reduces in rank order and writes the
//     reduced tile to rank g's output;
//  3. sends the reduced tile to every other rank's all-gather slot g;
//  4. polls tile t of every other rank's reduced share at once and decodes
//     each into rank g's output.
// A wave talks only to the waves of the same tile group of the other ranks,
// so the dual-buffer licences of the wide two-shot kernel hold pairwise:
// each reduce-scatter send is preceded by a wait for the wave's own earlier
// stores (the sentinel re-arms among them).
template <int P, int NMAX, bool EXTRAS>
__global__ __launch_bounds__(kWave) void k_sim_twoshot_narrow(CollSimArgs a) {
  if constexpr (!EXTRAS) {
    a.delay = nullptr;
    a.trace = nullptr;
  }
  const int lane = threadIdx.x;
  int g, tg;
  if (!sim_place(a, g, tg)) return;
  const int G = a.W;
  const int mine = (a.T - 1 - tg) / G + 1;
  const rsrc_t rs = make_rsrc(a.scratch, a.scratch_bytes);
  const uint32_t N = (uint32_t)a.nranks;
  const int tstride = 2 * a.nranks;
  int64_t lo_g, m_g;
  share_of(a.count, a.width, g, lo_g, m_g);
  const uint32_t E_g = enc_bytes<P>(m_g);
  if (a.trace && lane == 0 && tg == 0)
    __hip_atomic_fetch_min(reinterpret_cast<unsigned long long*>(a.trace) +
                               (int64_t)a.nops * tstride,
                           (unsigned long long)now_ticks(), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  uint32_t seq = a.seq0;
  uint32_t par = a.parity0;
  for (int op = 0; op < a.nops; ++op) {
    const uint32_t stale = seq_prev(seq_prev(seq));
    const uint16_t* row = a.in + ((int64_t)op * a.nranks + g) * a.in_stride;
    uint16_t* orow = a.out + ((int64_t)op * a.nranks + g) * a.out_stride;
    const uint32_t rs_src = (((uint32_t)g * 2u + par) * N) * a.slot_bytes;   // slot 0 of g
    const uint32_t ag_src = a.ag0 + rs_src;
    sim_delay(a, op, g);
    for (int k = 0; k < mine; ++k) {
      const int tile = tg + k * G;
      const uint32_t loff = (uint32_t)tile * kTileBytes + (uint32_t)lane * 16u;
      // ---- 1. reduce-scatter sends ----
      // the tiles of up to 8 shares (the own one included) are loaded first,
      // all the loads in flight together, then encoded and sent share by
      // share; the own share's chunk stays in own_v
      constexpr int GB = NMAX < 8 ? NMAX : 8;
      if (P == kSentinel) fence_release();
      u32x4 own_v = u32x4{0u, 0u, 0u, 0u};
      for (int w0 = 0; w0 < (NMAX <= GB ? 1 : a.nranks); w0 += GB) {
        uint32_t wv[GB][4];
#pragma unroll
        for (int j = 0; j < GB; ++j) {
          // shares past nranks are empty: their loads read nothing and give 0
          int64_t lo_w, m_w;
          share_of(a.count, a.width, w0 + j, lo_w, m_w);
          load_chunk<P>(row + lo_w, (uint32_t)((m_w * 2 + 15) & ~int64_t(15)), tile, lane,
                        wv[j]);
        }
#pragma unroll
        for (int j = 0; j < GB; ++j) {
          const int w = w0 + j;
          if (w >= a.nranks) break;
          int64_t lo_w, m_w;
          share_of(a.count, a.width, w, lo_w, m_w);
          mask_words(wv[j], chunk_keep<P>(m_w, tile, lane));
          const u32x4 enc = encode_words<P>(wv[j], lane, seq);
          if (w == g) {
            own_v = enc;
            continue;
          }
          store_chunk<P>(rs, (((uint32_t)w * 2u + par) * N + (uint32_t)g) * a.slot_bytes, 0u,
                         1, -1, tile, enc_bytes<P>(m_w), lane, enc);
        }
      }
      if (P == kLL128) {
        fence_release();
        for (int w = 0; w < a.nranks; ++w) {
          if (w == g) continue;
          int64_t lo_w, m_w;
          share_of(a.count, a.width, w, lo_w, m_w);
          produce_flags(rs, (((uint32_t)w * 2u + par) * N + (uint32_t)g) * a.slot_bytes, 0u, 1,
                        -1, tile, enc_bytes<P>(m_w), seq, lane);
        }
      }
      if (a.trace && k == mine - 1) {
        fence_release();
        if (lane == 0) trace_max(a, (int64_t)op * tstride + g);
      }
      // ---- 2.-3. share g: receive, reduce, all-gather send ----
      if ((uint32_t)tile * kTileBytes < E_g) {
        u32x4 v[NMAX];
        if (poll_tile<P, NMAX>(rs, rs_src, a.slot_bytes, a.nranks, tile, E_g, seq, stale, true,
                               g, own_v, a.ctrl, a.timeout_ticks, lane, v) != 0)
          return;
        uint32_t o[4];
        reduce_words<P, NMAX>(v, a.nranks, o);
        mask_words(o, chunk_keep<P>(m_g, tile, lane));
        int64_t first;
        int n;
        lane_elems<P>(tile, lane, first, n);
        if (loff < E_g) store_elems(orow + lo_g, m_g, first, n, o);
        const u32x4 enc = encode_words<P>(o, lane, seq);
        store_chunk<P>(rs, a.ag0 + (par * N + (uint32_t)g) * a.slot_bytes,
                       2u * N * a.slot_bytes, a.nranks, g, tile, E_g, lane, enc);
        if (P == kLL128) {
          fence_release();
          produce_flags(rs, a.ag0 + (par * N + (uint32_t)g) * a.slot_bytes,
                        2u * N * a.slot_bytes, a.nranks, g, tile, E_g, seq, lane);
        }
      }
      // ---- 4. all-gather receive ----
      {
        u32x4 v[NMAX];
        if (poll_shares<P, NMAX>(rs, ag_src, a.slot_bytes, a.nranks, g, tile, a.count,
                                 a.width, seq, stale, a.ctrl, a.timeout_ticks, lane, v) != 0)
          return;
#pragma unroll
        for (int r = 0; r < NMAX; ++r) {
          if (r >= a.nranks || r == g) continue;
          int64_t lo_r, m_r;
          share_of(a.count, a.width, r, lo_r, m_r);
          store_chunk_elems<P>(orow + lo_r, m_r, tile, enc_bytes<P>(m_r), lane, v[r]);
        }
      }
    }
    if (a.trace && lane == 0 && tg == 0) trace_max(a, (int64_t)op * tstride + a.nranks + g);
    seq = seq_next(seq);
    par ^= 1u;
  }
}

// ------------------------------------------------- chained simulator --

// Chained all-reduce simulator: the decode pattern, in which each op's
// result feeds the next op's producer ("Why Microseconds Matter in AI
// Infrastructure", section "Communication is becoming part of GPU
// execution": the producing computation and the communication in one
// kernel).  Op 0's payload of rank r is its input row; op i+1's payload of
// rank r is rank r's own copy of op i's result, scaled by
// scales[(i+1)*nranks + r] (y = bf16_rne(f32(x) * s), the producer
// epilogue's arithmetic).  So no op can start before the previous one has
// been reduced, as in a decode step whose next layer consumes the sum.
// One workgroup of nranks waves per (rank g, tile), wave w paired with peer
// w, every workgroup holding one tile.  Per op: every wave but the own one
// encodes the rank's payload chunk, sends it to peer w and polls peer w's
// chunk into LDS; barrier; the own wave reduces in rank order, writes the
// output tile and, unless the op is the last, scales the result into the
// next payload chunk in LDS; barrier; every wave takes that chunk.  The
// second barrier also covers both LDS buffers' reuse, and each op's sends
// come after the op before it has been consumed (consume(i), then
// produce(i+1)), which is the dual-buffer licence.
// LL and LL128 up to 8 ranks take one barrier per op instead: every wave
// sums the staged rows itself (the same rank-order sum, so the same bits)
// and scales its own next payload chunk, and the staging rows alternate
// between two LDS buffers by parity (a wave stages op i+1 only after the
// barrier of op i, and its row of op i+2 only after that of op i+1, which
// every wave reaches after reading op i's rows).  At 16 ranks the sixteen
// copies of the sum cost more than the barrier saves, and the sentinel's
// wait for its re-arm stores before each send then falls on the path.
template <int P, int NMAX>
__global__ __launch_bounds__(1024) void k_sim_chain(CollSimArgs a) {
  constexpr bool kEach = P != kSentinel && NMAX <= 8;
  __shared__ u32x4 lds[kEach ? 2 : 1][NMAX][kWave];
  __shared__ u32x4 next[kWave];
  __shared__ int lds_err;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x >> 6;
  int g, tg;
  if (!sim_place(a, g, tg)) return;                // whole workgroup
  const bool own = w == g;
  // the rank's own chunk is staged by wave g+1 (by the own wave for one rank)
  const int stager = a.nranks == 1 ? g : (g + 1) % a.nranks;
  const rsrc_t rs = make_rsrc(a.scratch, a.scratch_bytes);
  const uint32_t N = (uint32_t)a.nranks;
  const uint32_t row_bytes = (uint32_t)(((a.count * 2) + 15) & ~int64_t(15));
  const int keep = chunk_keep<P>(a.count, tg, lane);
  const uint32_t loff = (uint32_t)tg * kTileBytes + (uint32_t)lane * 16u;
  uint32_t x[4];                                   // this op's payload chunk
  load_chunk<P>(a.in + (int64_t)g * a.in_stride, row_bytes, tg, lane, x);
  mask_words(x, keep);
  if (threadIdx.x == 0) lds_err = 0;
  __syncthreads();
  uint32_t seq = a.seq0;
  uint32_t par = a.parity0;
  for (int op = 0; op < a.nops; ++op) {
    const uint32_t stale = seq_prev(seq_prev(seq));
    const int b = kEach ? (int)par : 0;            // staging buffer of this op
    // every wave scales its own next chunk: the factor, loaded before this
    // op's exchange
    const float s_next =
        kEach && op + 1 < a.nops ? a.scales[(int64_t)(op + 1) * a.nranks + g] : 0.f;
    const u32x4 enc = encode_words<P>(x, lane, seq);
    if (!own) {
      // sentinel: this wave's re-arm stores of the previous op complete
      // before its next store to the same peer
      if (P == kSentinel) fence_release();
      const uint32_t dst0 = (((uint32_t)w * 2u + par) * N + (uint32_t)g) * a.slot_bytes;
      store_chunk<P>(rs, dst0, 0u, 1, -1, tg, a.E, lane, enc);
      if (P == kLL128) {
        fence_release();
        produce_flags(rs, dst0, 0u, 1, -1, tg, a.E, seq, lane);
      }
      const uint32_t src = (((uint32_t)g * 2u + par) * N + (uint32_t)w) * a.slot_bytes + loff;
      u32x4 got;
      if (poll_chunk<P>(rs, src, loff < a.E, seq, stale, true, a.ctrl, a.timeout_ticks, lane,
                        got) != 0) {
        if (lane == 0) lds_err = 1;
      } else {
        lds[b][w][lane] = got;
      }
    }
    if (w == stager) lds[b][g][lane] = enc;
    __syncthreads();
    if (lds_err) return;                           // whole workgroup
    if (kEach || own) {
      u32x4 v[NMAX];
#pragma unroll
      for (int r = 0; r < NMAX; ++r)
        v[r] = (r < a.nranks) ? lds[b][r][lane] : u32x4{0u, 0u, 0u, 0u};
      uint32_t o[4];
      reduce_words<P, NMAX>(v, a.nranks, o);
      mask_words(o, keep);
      if (own) {
        int64_t first;
        int n;
        lane_elems<P>(tg, lane, first, n);
        if (loff < a.E)
          store_elems(a.out + ((int64_t)op * a.nranks + g) * a.out_stride, a.count, first, n,
                      o);
      }
      if (op + 1 < a.nops) {
        scale_words(o, kEach ? s_next : a.scales[(int64_t)(op + 1) * a.nranks + g]);
        mask_words(o, keep);
        if constexpr (kEach) {
#pragma unroll
          for (int k = 0; k < 4; ++k) x[k] = o[k];
        } else {
          next[lane] = u32x4{o[0], o[1], o[2], o[3]};
        }
      }
    }
    if constexpr (!kEach) {
      __syncthreads();
      if (op + 1 < a.nops) {
        const u32x4 nx = next[lane];
        x[0] = nx.x;
        x[1] = nx.y;
        x[2] = nx.z;
        x[3] = nx.w;
      }
    }
    seq = seq_next(seq);
    par ^= 1u;
  }
}

// ================================================================ host side

// All-gather: with several tiles per wave, the sentinel kernel overlaps the
// input loads of 4 tiles (16 ranks, 256 KiB: 67.2 -> 58.5 us per op; 8
// ranks, 1 MiB: 56.7 -> 52.5 us); LL and LL128 measured no gain (LL: 8
// ranks, 1 MiB, 93 -> 106 us).  With one tile per wave the plain kernel is
// up to 7% faster.  The grid is sized by the smaller occupancy of the two.
// EXTRAS: the launch uses producer delays or a trace; the variant without
// them drops those paths at compile time (as for the all-reduce simulators).
template <int P, int NMAX, bool EXTRAS>
static const void* sim_fn_x(int collective, bool narrow, bool multi) {
  if (collective == AR_ALLGATHER) {
    if constexpr (P == kSentinel)
      if (multi) return reinterpret_cast<const void*>(&k_sim_gather<P, NMAX, 4, EXTRAS>);
    return reinterpret_cast<const void*>(&k_sim_gather<P, NMAX, 1, EXTRAS>);
  }
  if (narrow) return reinterpret_cast<const void*>(&k_sim_twoshot_narrow<P, NMAX, EXTRAS>);
  return multi ? reinterpret_cast<const void*>(&k_sim_twoshot<P, NMAX, 2, EXTRAS>)
               : reinterpret_cast<const void*>(&k_sim_twoshot<P, NMAX, 1, EXTRAS>);
}

template <int P, int NMAX>
static const void* sim_fn(int collective, bool narrow, bool multi, bool extras) {
  return extras ? sim_fn_x<P, NMAX, true>(collective, narrow, multi)
                : sim_fn_x<P, NMAX, false>(collective, narrow, multi);
}

template <int P>
static const void* sim_fn_n(int collective, int nranks, bool narrow, bool multi,
                            bool extras) {
  if (nranks <= 4) return sim_fn<P, 4>(collective, narrow, multi, extras);
  if (nranks <= 8) return sim_fn<P, 8>(collective, narrow, multi, extras);
  return sim_fn<P, 16>(collective, narrow, multi, extras);
}

static const void* coll_sim_fn(int proto, int collective, int nranks, bool narrow,
                               bool multi, bool extras) {
  switch (proto) {
    case kLL: return sim_fn_n<kLL>(collective, nranks, narrow, multi, extras);
    case kLL128: return sim_fn_n<kLL128>(collective, nranks, narrow, multi, extras);
    default: return sim_fn_n<kSentinel>(collective, nranks, narrow, multi, extras);
  }
}

// Two-shot kernel choice, from a sweep of both kernels on MI355X (4, 8 and 16
// ranks, 16 KiB .. 2 MiB per rank, every protocol).  The one-wave kernel
// serializes its N-1 sends and polls, which costs it a roughly fixed 6 / 9 /
// 16-22 us per op at 4 / 8 / 16 ranks (LL128: 11 / 18 / 33 us), while the
// workgroup kernel's time grows with the share tiles each workgroup walks.
// The workgroup kernel wins up to this many tiles:
//   4 ranks: 2 (2 tiles: 6.5 vs 7.1 us, LL, 512 KiB; 3 tiles: 9.0 vs
//     7.7 us, LL, 1 MiB);
//   8 ranks: 3 (3 tiles: 14.2 vs 19.1 us, LL128, 512 KiB; 4 tiles:
//     12.6 vs 10.7 us, LL, 512 KiB);
//   16 ranks: 5 (4 tiles: 18.3 vs 24.3 us, SENTINEL, 512 KiB; 8 tiles:
//     41.5 vs 29.2 us, SENTINEL, 1 MiB), and 9 for LL128 (9 tiles: 62.0 vs
//     70.9 us, 1 MiB; 18 tiles: 120 vs 109 us, 2 MiB).
static int twoshot_wide_max_tiles(int proto, int nranks) {
  if (nranks <= 4) return 2;
  if (nranks <= 8) return 3;
  return proto == kLL128 ? 9 : 5;
}

struct CollGeom {
  int32_t W, Q, T, TPW, blocks;
  bool narrow;                 // two-shot: one wave per tile group
  bool coop;                   // cooperative launch
};

static int coll_check(const ar_sim_params* p) {
  const ar_desc* d = &p->desc;
  if (d->nconsumers != d->nranks) return AR_EINVAL;
  if (d->proto == kBarrier) return AR_EINVAL;
  if (p->tile_order) return AR_EINVAL;
  const int kernel_flags = AR_SIM_NARROW | AR_SIM_WIDE;
  const int launch_flags = AR_SIM_COOPERATIVE | AR_SIM_ORDINARY;
  if (p->flags & ~(kernel_flags | launch_flags)) return AR_EINVAL;
  if ((p->flags & launch_flags) == launch_flags) return AR_EINVAL;
  if ((p->flags & kernel_flags) &&
      (d->collective != AR_TWOSHOT || (p->flags & kernel_flags) == kernel_flags))
    return AR_EINVAL;
  return AR_OK;
}

// Tiles of one rank's transfer: the whole payload (all-gather) or one full
// share (two-shot).  Grid: the all-reduce simulator's rule (the occupancy
// query's residency, halved for an ordinary launch; tile groups in
// multiples of 8 per rank).
static int coll_geometry_as(const ar_sim_params* p, const DeviceInfo& di, bool narrow,
                            bool coop, CollGeom* g) {
  const ar_desc* d = &p->desc;
  const int64_t n_el =
      d->collective == AR_TWOSHOT ? share_width(d->count, d->nranks) : d->count;
  const int64_t T = ceil_div64(encoded_bytes(d->proto, n_el), kTileBytes);
  if (T <= 0) {
    *g = CollGeom{0, 0, 0, 0, 0, narrow, coop};
    return AR_OK;
  }
  if (T > (int64_t(1) << 24)) return AR_ESIZE;
  // the smallest occupancy of the kernels the launch may pick (one tile per
  // wave or several, with or without delays and trace), so that any of them
  // is resident on this grid
  int occ = 0;
  for (int m = 0; m < 4; ++m) {
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &o, coll_sim_fn(d->proto, d->collective, d->nranks, narrow, (m & 1) != 0,
                            (m & 2) != 0),
            narrow ? kWave : kWave * d->nranks, 0) != hipSuccess ||
        o <= 0)
      return AR_ELAUNCH;
    occ = (m == 0 || o < occ) ? o : occ;
  }
  // whole grid resident: the occupancy query's figure (half of it for an
  // ordinary launch), and one-wave workgroups at most 8 per CU (as for the
  // all-reduce simulator)
  int64_t capacity = (int64_t)occ * di.cus / (coop ? 1 : 2);
  if (narrow && capacity > 8 * (int64_t)di.cus) capacity = 8 * (int64_t)di.cus;
  const int64_t qmax = capacity / (8 * (int64_t)d->nranks);
  if (qmax < 1) return AR_ECAPACITY;
  int64_t Q;
  if (p->waves_per_rank > 0) {
    if (p->waves_per_rank % 8) return AR_EINVAL;
    Q = p->waves_per_rank / 8;
    if (Q > qmax) return AR_ECAPACITY;
  } else {
    Q = ceil_div64(T, 8);
    if (Q > qmax) Q = qmax;
  }
  g->W = (int32_t)(8 * Q);
  g->Q = (int32_t)Q;
  g->T = (int32_t)T;
  g->TPW = (int32_t)ceil_div64(T, 8 * Q);
  g->blocks = (int32_t)(8 * Q * d->nranks);
  g->narrow = narrow;
  g->coop = coop;
  return AR_OK;
}

// Two-shot kernel choice: a workgroup of one wave per peer while each
// workgroup walks at most twoshot_wide_max_tiles share tiles, else (or with
// AR_SIM_NARROW) one wave per share tile group; AR_SIM_WIDE forces the
// former.
static int coll_kernel_choice(const ar_sim_params* p, const DeviceInfo& di, bool coop,
                              CollGeom* g) {
  if (p->desc.collective != AR_TWOSHOT) return coll_geometry_as(p, di, false, coop, g);
  if (p->flags & AR_SIM_NARROW) return coll_geometry_as(p, di, true, coop, g);
  const int rc = coll_geometry_as(p, di, false, coop, g);
  if (p->flags & AR_SIM_WIDE) return rc;
  if (rc == AR_OK && g->TPW <= twoshot_wide_max_tiles(p->desc.proto, p->desc.nranks))
    return AR_OK;
  return coll_geometry_as(p, di, true, coop, g);
}

// Launch choice: as for the all-reduce simulator (coop_pays).
static int coll_geometry(const ar_sim_params* p, const DeviceInfo& di, CollGeom* g) {
  if (p->flags & AR_SIM_COOPERATIVE) return coll_kernel_choice(p, di, true, g);
  const int rc = coll_kernel_choice(p, di, false, g);
  if ((p->flags & AR_SIM_ORDINARY) || !di.coop || p->nops < kCoopMinOps) return rc;
  if (rc != AR_OK && rc != AR_ECAPACITY) return rc;
  CollGeom gc;
  if (coll_kernel_choice(p, di, true, &gc) == AR_OK &&
      coop_pays(rc, g->TPW, !g->narrow, gc.TPW, !gc.narrow)) {
    *g = gc;
    return AR_OK;
  }
  return rc;
}

int coll_sim_geometry(const ar_sim_params* p, int32_t* groups, int32_t* tiles,
                      int32_t* tiles_per_group, int32_t* blocks, int32_t* wide,
                      int32_t* cooperative) {
  int rc = coll_check(p);
  if (rc) return rc;
  DeviceInfo di;
  rc = device_info(&di);
  if (rc) return rc;
  CollGeom g;
  rc = coll_geometry(p, di, &g);
  if (rc) return rc;
  if (groups) *groups = g.W;
  if (tiles) *tiles = g.T;
  if (tiles_per_group) *tiles_per_group = g.TPW;
  if (blocks) *blocks = g.blocks;
  if (wide) *wide = g.narrow ? 0 : 1;
  if (cooperative) *cooperative = g.coop ? 1 : 0;
  return AR_OK;
}

int coll_sim_run(const ar_sim_params* p, hipStream_t s) {
  int rc = coll_check(p);
  if (rc) return rc;
  const ar_desc* d = &p->desc;
  const int64_t R = (d->count + 7) / 8 * 8;
  if (d->collective == AR_ALLGATHER && p->out_stride < (int64_t)d->nranks * R)
    return AR_EINVAL;
  if (d->count == 0) return AR_OK;
  DeviceInfo di;
  rc = device_info(&di);
  if (rc) return rc;
  if ((p->flags & AR_SIM_COOPERATIVE) && !di.coop) return AR_ENODEV;
  CollGeom g;
  rc = coll_geometry(p, di, &g);
  if (rc) return rc;
  CollSimArgs a;
  a.in = static_cast<const uint16_t*>(p->in);
  a.in_stride = p->in_stride;
  a.out = static_cast<uint16_t*>(p->out);
  a.out_stride = p->out_stride;
  a.row_stride = R;
  a.count = d->count;
  a.width = share_width(d->count, d->nranks);
  a.scratch = static_cast<const uint8_t*>(p->scratch);
  a.scratch_bytes = (uint32_t)desc_scratch_bytes(d);
  a.slot_bytes = (uint32_t)desc_slot_bytes(d);
  a.ag0 = (uint32_t)desc_region_bytes(d);
  a.E = (uint32_t)encoded_bytes(d->proto, d->count);
  a.ctrl = static_cast<int*>(p->ctrl);
  a.nranks = d->nranks;
  a.nops = p->nops;
  a.W = g.W;
  a.Q = g.Q;
  a.T = g.T;
  a.TPW = g.TPW;
  a.seq0 = p->epoch.seq;
  a.parity0 = p->epoch.parity;
  a.timeout_ticks = ns_to_ticks(p->timeout_ns, di.wallclock_hz);
  a.delay = p->delay_ticks;
  a.trace = p->trace;
  a.scales = nullptr;
  void* args[] = {&a};
  const bool extras = a.delay || a.trace;
  const void* fn =
      coll_sim_fn(d->proto, d->collective, d->nranks, g.narrow, g.TPW > 1, extras);
  const dim3 block(g.narrow ? kWave : kWave * d->nranks);
  if (!g.coop) return map_hip(hipLaunchKernel(fn, dim3(g.blocks), block, args, 0, s));
  const hipError_t e = hipLaunchCooperativeKernel(fn, dim3(g.blocks), block, args, 0, s);
  if (e == hipSuccess || (p->flags & AR_SIM_COOPERATIVE)) return map_hip(e);
  // a cooperative launch the library chose by itself that the runtime turns
  // down is retried as an ordinary launch on the ordinary grid
  (void)hipGetLastError();
  CollGeom go;
  rc = coll_kernel_choice(p, di, false, &go);
  if (rc) return rc;
  a.W = go.W;
  a.Q = go.Q;
  a.T = go.T;
  a.TPW = go.TPW;
  const void* fo =
      coll_sim_fn(d->proto, d->collective, d->nranks, go.narrow, go.TPW > 1, extras);
  return map_hip(hipLaunchKernel(fo, dim3(go.blocks), dim3(go.narrow ? kWave : kWave * d->nranks),
                                 args, 0, s));
}

// --------------------------------------------------- chained simulator host

template <int P>
static const void* chain_fn_n(int nranks) {
  if (nranks <= 4) return reinterpret_cast<const void*>(&k_sim_chain<P, 4>);
  if (nranks <= 8) return reinterpret_cast<const void*>(&k_sim_chain<P, 8>);
  return reinterpret_cast<const void*>(&k_sim_chain<P, 16>);
}

static const void* chain_fn(int proto, int nranks) {
  switch (proto) {
    case kLL: return chain_fn_n<kLL>(nranks);
    case kLL128: return chain_fn_n<kLL128>(nranks);
    default: return chain_fn_n<kSentinel>(nranks);
  }
}

// Beyond the simulator's own checks: the one-shot all-reduce in system mode,
// LL / LL128 / SENTINEL, no tile order, delays or trace, and the library's
// own grid (launch flags only).
static int chain_check(const ar_sim_params* p) {
  const ar_desc* d = &p->desc;
  if (d->collective != AR_ALLREDUCE || d->nconsumers != d->nranks) return AR_EINVAL;
  if (d->proto == kBarrier) return AR_EINVAL;
  if (p->tile_order || p->delay_ticks || p->trace || p->waves_per_rank) return AR_EINVAL;
  if (p->flags & (AR_SIM_NARROW | AR_SIM_WIDE)) return AR_EINVAL;
  return AR_OK;
}

struct ChainGeom {
  int32_t Q, T, blocks;
  bool coop;
};

// One workgroup per (rank, tile) for every tile of the payload.  The grid
// must be resident: at most the occupancy query's figure, halved for an
// ordinary launch.  Without a launch flag: ordinary when the grid fits
// that, else cooperative where the device supports it.
static int chain_geometry(const ar_sim_params* p, const DeviceInfo& di, ChainGeom* g) {
  const ar_desc* d = &p->desc;
  const int64_t T = ceil_div64(encoded_bytes(d->proto, d->count), kTileBytes);
  if (T > (int64_t(1) << 24)) return AR_ESIZE;
  const int64_t Q = ceil_div64(T, 8);
  const int64_t blocks = 8 * Q * d->nranks;
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, chain_fn(d->proto, d->nranks),
                                                   kWave * d->nranks, 0) != hipSuccess ||
      occ <= 0)
    return AR_ELAUNCH;
  const int64_t full = (int64_t)occ * di.cus;
  bool coop;
  if (p->flags & AR_SIM_COOPERATIVE)
    coop = true;
  else if (p->flags & AR_SIM_ORDINARY)
    coop = false;
  else
    coop = blocks > full / 2 && di.coop;
  if (blocks > (coop ? full : full / 2)) return AR_ECAPACITY;
  g->Q = (int32_t)Q;
  g->T = (int32_t)T;
  g->blocks = (int32_t)blocks;
  g->coop = coop;
  return AR_OK;
}

int chain_sim_geometry(const ar_sim_params* p, int32_t* blocks, int32_t* cooperative) {
  int rc = chain_check(p);
  if (rc) return rc;
  DeviceInfo di;
  rc = device_info(&di);
  if (rc) return rc;
  ChainGeom g;
  rc = chain_geometry(p, di, &g);
  if (rc) return rc;
  if (blocks) *blocks = g.blocks;
  if (cooperative) *cooperative = g.coop ? 1 : 0;
  return AR_OK;
}

int chain_sim_run(const ar_sim_params* p, const float* scales, hipStream_t s) {
  int rc = chain_check(p);
  if (rc) return rc;
  if (!scales) return AR_EINVAL;
  if (!aligned(scales, 4)) return AR_EALIGN;
  const ar_desc* d = &p->desc;
  if (d->count == 0) return AR_OK;
  DeviceInfo di;
  rc = device_info(&di);
  if (rc) return rc;
  if ((p->flags & AR_SIM_COOPERATIVE) && !di.coop) return AR_ENODEV;
  ChainGeom g;
  rc = chain_geometry(p, di, &g);
  if (rc) return rc;
  CollSimArgs a{};
  a.in = static_cast<const uint16_t*>(p->in);
  a.in_stride = p->in_stride;
  a.out = static_cast<uint16_t*>(p->out);
  a.out_stride = p->out_stride;
  a.row_stride = (d->count + 7) / 8 * 8;
  a.count = d->count;
  a.width = d->count;
  a.scratch = static_cast<const uint8_t*>(p->scratch);
  a.scratch_bytes = (uint32_t)desc_scratch_bytes(d);
  a.slot_bytes = (uint32_t)desc_slot_bytes(d);
  a.ag0 = 0u;
  a.E = (uint32_t)encoded_bytes(d->proto, d->count);
  a.ctrl = static_cast<int*>(p->ctrl);
  a.nranks = d->nranks;
  a.nops = p->nops;
  a.W = 8 * g.Q;
  a.Q = g.Q;
  a.T = g.T;
  a.TPW = 1;
  a.seq0 = p->epoch.seq;
  a.parity0 = p->epoch.parity;
  a.timeout_ticks = ns_to_ticks(p->timeout_ns, di.wallclock_hz);
  a.delay = nullptr;
  a.trace = nullptr;
  a.scales = scales;
  void* args[] = {&a};
  const void* fn = chain_fn(d->proto, d->nranks);
  const dim3 block(kWave * d->nranks);
  // no ordinary fallback: an ordinary grid could not hold every tile
  if (g.coop) return map_hip(hipLaunchCooperativeKernel(fn, dim3(g.blocks), block, args, 0, s));
  return map_hip(hipLaunchKernel(fn, dim3(g.blocks), block, args, 0, s));
}

// ----------------------------------------------------- stream-ordered host

static TsArgs ts_args(const ar_desc* d, void* scratch, ar_epoch e) {
  TsArgs a{};
  a.count = d->count;
  a.width = share_width(d->count, d->nranks);
  a.scratch = static_cast<const uint8_t*>(scratch);
  a.scratch_bytes = (uint32_t)desc_scratch_bytes(d);
  a.slot_bytes = (uint32_t)desc_slot_bytes(d);
  a.ag0 = (uint32_t)desc_region_bytes(d);
  a.nranks = d->nranks;
  a.tiles = (int32_t)ceil_div64(encoded_bytes(d->proto, a.width), kTileBytes);
  a.seq = e.seq;
  a.parity = e.parity;
  return a;
}

int twoshot_pack(int32_t proto, const ar_desc* d, const void* in, int64_t in_stride,
                 void* scratch, ar_epoch e, hipStream_t s) {
  TsArgs a = ts_args(d, scratch, e);
  a.in = static_cast<const uint16_t*>(in);
  a.in_stride = in_stride;
  const int64_t waves = (int64_t)d->nranks * d->nranks * a.tiles;
  const dim3 grid((unsigned)ceil_div64(waves, kWavesPerBlock));
  switch (proto) {
    case kLL: return map_hip(launch(k_ts_pack<kLL>, grid, dim3(kBlock), s, a));
    case kLL128: return map_hip(launch(k_ts_pack<kLL128>, grid, dim3(kBlock), s, a));
    default: return map_hip(launch(k_ts_pack<kSentinel>, grid, dim3(kBlock), s, a));
  }
}

template <int P>
static hipError_t ts_reduce_p(const TsArgs& a, hipStream_t s) {
  const dim3 g1((unsigned)ceil_div64((int64_t)a.nranks * a.tiles, kWavesPerBlock));
  hipError_t e;
  if (a.nranks <= 4) e = launch(k_ts_reduce<P, 4>, g1, dim3(kBlock), s, a);
  else if (a.nranks <= 8) e = launch(k_ts_reduce<P, 8>, g1, dim3(kBlock), s, a);
  else e = launch(k_ts_reduce<P, 16>, g1, dim3(kBlock), s, a);
  if (e != hipSuccess) return e;
  const dim3 g2(
      (unsigned)ceil_div64((int64_t)a.nranks * a.nranks * a.tiles, kWavesPerBlock));
  return launch(k_ts_gather<P>, g2, dim3(kBlock), s, a);
}

int twoshot_reduce(const ar_desc* d, void* scratch, void* out, int64_t out_stride,
                   ar_epoch e, void* ctrl, uint64_t timeout_ns, int32_t flags,
                   hipStream_t s) {
  DeviceInfo di;
  int rc = device_info(&di);
  if (rc) return rc;
  TsArgs a = ts_args(d, scratch, e);
  a.out = static_cast<uint16_t*>(out);
  a.out_stride = out_stride;
  a.ctrl = static_cast<int*>(ctrl);
  a.timeout_ticks = ns_to_ticks(timeout_ns, di.wallclock_hz);
  a.rearm = (flags & AR_FLAG_REARM) && d->proto == kSentinel;
  switch (d->proto) {
    case kLL: return map_hip(ts_reduce_p<kLL>(a, s));
    case kLL128: return map_hip(ts_reduce_p<kLL128>(a, s));
    default: return map_hip(ts_reduce_p<kSentinel>(a, s));
  }
}

}  // namespace ar

// ================================================================== C ABI

using namespace ar;

extern "C" int ar_gather_validate(const ar_desc* d, void* scratch, void* out,
                                  int64_t out_stride, ar_epoch e, void* ctrl,
                                  uint64_t timeout_ns, int32_t flags, void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (d->collective != AR_ALLGATHER) return AR_EINVAL;
  if (e.parity > 1u || e.seq == 0u) return AR_EINVAL;
  if (flags & ~AR_FLAG_REARM) return AR_EINVAL;
  if (!timeout_ok(timeout_ns)) return AR_EINVAL;
  const int64_t R = (d->count + 7) / 8 * 8;
  rc = check_rows(out, out_stride, (int64_t)d->nranks * R);
  if (rc) return rc;
  if (d->count == 0) return AR_OK;
  if (!scratch || !ctrl) return AR_EINVAL;
  if (!aligned(scratch, 256) || !aligned(ctrl, 256)) return AR_EALIGN;
  DeviceInfo di;
  rc = device_info(&di);
  if (rc) return rc;
  GatherArgs a;
  a.out = static_cast<uint16_t*>(out);
  a.out_stride = out_stride;
  a.row_stride = R;
  a.count = d->count;
  a.scratch = static_cast<const uint8_t*>(scratch);
  a.scratch_bytes = (uint32_t)desc_scratch_bytes(d);
  a.slot_bytes = (uint32_t)desc_slot_bytes(d);
  a.E = (uint32_t)encoded_bytes(d->proto, d->count);
  a.nranks = d->nranks;
  a.nconsumers = d->nconsumers;
  a.tiles = (int32_t)ceil_div64(a.E, kTileBytes);
  a.seq = e.seq;
  a.parity = e.parity;
  a.ctrl = static_cast<int*>(ctrl);
  a.timeout_ticks = ns_to_ticks(timeout_ns, di.wallclock_hz);
  a.rearm = (flags & AR_FLAG_REARM) && d->proto == kSentinel;
  const int64_t waves = (int64_t)a.tiles * d->nranks * d->nconsumers;
  if (waves >= (int64_t(1) << 31)) return AR_ESIZE;
  const dim3 grid((unsigned)ceil_div64(waves, kWavesPerBlock));
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (d->proto) {
    case kLL: return map_hip(launch(k_gather<kLL>, grid, dim3(kBlock), s, a));
    case kLL128: return map_hip(launch(k_gather<kLL128>, grid, dim3(kBlock), s, a));
    case kSentinel: return map_hip(launch(k_gather<kSentinel>, grid, dim3(kBlock), s, a));
    default: return map_hip(launch(k_gather<kBarrier>, grid, dim3(kBlock), s, a));
  }
}

extern "C" int ar_scale_pack(const ar_desc* d, const void* in, int64_t in_stride,
                             const float* scales, void* scratch, ar_epoch e,
                             void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (d->collective == AR_TWOSHOT) return AR_EINVAL;
  if (e.parity > 1u || e.seq == 0u) return AR_EINVAL;
  rc = check_rows(in, in_stride, d->count);
  if (rc) return rc;
  if (d->count == 0) return AR_OK;
  if (!scratch || !scales) return AR_EINVAL;
  if (!aligned(scratch, 256) || !aligned(scales, 4)) return AR_EALIGN;
  ScaleArgs a{};
  a.in = static_cast<const uint16_t*>(in);
  a.in_stride = in_stride;
  a.scales = scales;
  a.count = d->count;
  a.nranks = d->nranks;
  const int64_t E = encoded_bytes(d->proto, d->count);
  a.tiles = (int32_t)ceil_div64(E, kTileBytes);
  a.b = ar_dev::make(scratch, (uint32_t)desc_scratch_bytes(d), (uint32_t)desc_slot_bytes(d),
                     (uint32_t)E, d->nranks, d->nconsumers, d->count, e.seq, e.parity);
  const dim3 grid((unsigned)ceil_div64((int64_t)a.tiles * d->nranks, kWavesPerBlock));
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (d->proto) {
    case kLL: return map_hip(launch(k_scale_send<kLL>, grid, dim3(kBlock), s, a));
    case kLL128: return map_hip(launch(k_scale_send<kLL128>, grid, dim3(kBlock), s, a));
    case kSentinel: return map_hip(launch(k_scale_send<kSentinel>, grid, dim3(kBlock), s, a));
    default: return map_hip(launch(k_scale_send<kBarrier>, grid, dim3(kBlock), s, a));
  }
}

extern "C" int ar_scale_rows(int32_t nranks, int64_t count, const void* in,
                             int64_t in_stride, const float* scales, void* out,
                             int64_t out_stride, void* stream) {
  if (nranks < 1 || nranks > AR_MAX_RANKS || count < 0) return AR_EINVAL;
  int rc = check_rows(in, in_stride, count);
  if (rc) return rc;
  rc = check_rows(out, out_stride, count);
  if (rc) return rc;
  if (count == 0) return AR_OK;
  if (!scales) return AR_EINVAL;
  if (!aligned(scales, 4)) return AR_EALIGN;
  ScaleArgs a{};
  a.in = static_cast<const uint16_t*>(in);
  a.in_stride = in_stride;
  a.scales = scales;
  a.out = static_cast<uint16_t*>(out);
  a.out_stride = out_stride;
  a.nranks = nranks;
  a.count = count;
  const int64_t threads = (int64_t)nranks * ((count + 7) / 8);
  return map_hip(launch(k_scale_rows, dim3((unsigned)ceil_div64(threads, kBlock)),
                        dim3(kBlock), static_cast<hipStream_t>(stream), a));
}
