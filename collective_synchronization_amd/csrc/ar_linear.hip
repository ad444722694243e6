// ar_linear.hip -- chained one-shot all-reduces whose producer is a
// row-parallel linear layer shard, in one persistent launch (gfx950).
//
// "SiFAR: Synchronization-Free All-Reduce for Low-Latency LLM Inference",
// abstract: communication and model execution are designed together, the
// all-reduce result being the input of the next layer (dual buffering takes
// the bottom barrier away).  "Why Microseconds Matter in AI
// Infrastructure", section "Communication is becoming part of GPU
// execution": the kernel that produces a payload sends it itself.  Here op
// i's producer on rank g is one decode token's row-parallel linear shard:
//     y_g[j] = bf16_rne( S(0, kr) ),  S = pairwise binary32 sum over k of
//              f32(z[g*kr + k]) * f32(W[layer][g][j][k]),
// z being op i-1's all-reduce result (op 0: rank g's input row), kr =
// count / nranks; the y_g are all-reduced with the one-shot protocols.
//
// Two kinds of workgroup share the launch:
//  * exchange workgroups, one per (rank g, 1 KiB tile t) as in the chained
//    all-reduce simulator: wave w sends rank g's chunk of tile t to
//    consumer w and polls peer w's chunk; the rank's own wave reduces in
//    rank order, writes the output and, for the part of tile t inside
//    rank g's input slice, publishes it for the next op;
//  * GEMV workers, spread over the rest of the chip: each wave computes a
//    block of RW output rows of one rank and publishes them.
// Both hand-offs inside the GPU (payload rows to the exchange workgroup,
// the reduced slice to the workers) use LL words -- 4 data bytes beside the
// op's epoch in one 8-byte store -- so no counter, reset or fence orders
// them: the words validate themselves, as the slots do.  A worker issues
// the loads of its next weight block before it waits for the op's input,
// so the weight stream of op i+1 overlaps op i's all-reduce.
//
// Dot products: lane l of a wave holds the KL = kr/64 products of inputs
// [l*KL, (l+1)*KL); it sums them pairwise in registers, then the wave adds
// lane partials level by level with partners l^1, l^2, ..., l^32, which
// joins contiguous halves: the pairwise tree of the whole row, whatever
// lane holds it (binary32 addition is commutative).  A wave sums a block of
// rows together, the lanes trading halves of their rows at the first
// levels, so one exchange serves several rows.
//
// Buffer reuse (two parities of every buffer): a rank's workers write its
// payload rows of op i+2 only after its input slice of op i+1 exists, which
// needs every rank's op i+1 payload for the tiles of that slice, which
// needs those ranks' slices of op i, which need this rank's op i payload of
// every tile -- each read before it was sent.  The same chain covers the
// slice buffer and, as in the chained simulator, the receive slots are
// licensed pairwise (a peer sends op i only after consuming op i-1).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "../../include/ar.h"
#include "ar_host.h"
#include "../../include/ar_protocols.h"

namespace ar {

struct LinArgs {
  const uint16_t* in;
  int64_t in_stride;
  const uint16_t* w;          // [layers][nranks][count][kr] bf16
  uint16_t* out;
  int64_t out_stride;
  const uint8_t* scratch;
  uint32_t scratch_bytes, slot_bytes, E;
  const uint8_t* work;        // payload words, then slice words
  uint32_t work_bytes, act0;  // act0: byte offset of the slice words
  int* ctrl;
  int64_t count;
  int32_t kr, layers, nranks, nops;
  int32_t Q, T, comm_blocks;  // exchange grid: 8*Q*nranks workgroups
  int32_t wpr, bpr;           // worker workgroups per rank, row blocks per rank
  uint32_t seq0, parity0;
  uint64_t timeout_ticks;
};

// An LL word's flag: ready for epoch seq, "not yet" (two ops before, or
// never written), or impossible.
__device__ __forceinline__ void ll_flag(uint32_t f, uint32_t seq, uint32_t stale, bool& ok,
                                        bool& bad) {
  ok = f == seq;
  bad = !ok && f != stale && f != 0u;
}

// The lane's KL weights of one row (KL/2 packed bf16 pairs): a buffer load
// through the (layer, rank) shard's resource, the row's byte offset in a
// scalar register and the lane's in a vector one.
template <int KL>
__device__ __forceinline__ void load_wrow(rsrc_t r, uint32_t lane_off, uint32_t row_off,
                                          uint32_t (&d)[KL / 2]) {
  if constexpr (KL == 4) {
    const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(r, lane_off, row_off, 0);
    d[0] = a.x;
    d[1] = a.y;
  } else {
#pragma unroll
    for (int q = 0; q < KL / 8; ++q) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, lane_off + 16u * q, row_off, 0);
      d[4 * q] = v.x;
      d[4 * q + 1] = v.y;
      d[4 * q + 2] = v.z;
      d[4 * q + 3] = v.w;
    }
  }
}

// Plain load of the lane's KL inputs (8-byte aligned).
template <int KL>
__device__ __forceinline__ void load_inputs(const uint16_t* __restrict__ p, uint32_t (&d)[KL / 2]) {
#pragma unroll
  for (int q = 0; q < KL / 4; ++q) {
    const u32x2 v = reinterpret_cast<const u32x2*>(p)[q];
    d[2 * q] = v.x;
    d[2 * q + 1] = v.y;
  }
}

// The lane's part of one row: its KL products summed pairwise (contiguous
// halves).
template <int KL>
__device__ __forceinline__ float lane_part(const float (&z)[KL], const uint32_t (&d)[KL / 2]) {
  float p[KL];
#pragma unroll
  for (int k = 0; k < KL / 2; ++k) {
    p[2 * k] = z[2 * k] * bf_lo(d[k]);
    p[2 * k + 1] = z[2 * k + 1] * bf_hi(d[k]);
  }
#pragma unroll
  for (int s = 1; s < KL; s <<= 1)
#pragma unroll
    for (int k = 0; k < KL; k += 2 * s) p[k] = p[k] + p[k + s];
  return p[0];
}

// The row whose sum rows_sum<R> leaves in a lane: bit s of the lane picks
// the upper half at level s, so row = sum over s of bit_s(lane) * R/2^(s+1)
// (every lane of an aligned block of R lanes holds a different row).
template <int R>
__device__ __forceinline__ int lane_row(int lane) {
  int r = 0;
#pragma unroll
  for (int s = 0; (R >> (s + 1)) > 0; ++s) r += ((lane >> s) & 1) * (R >> (s + 1));
  return r;
}

// Sums of R rows over the wave's lanes, v[u] holding the lane's part of row
// u.  Level s adds the partial sums of lane blocks l and l ^ 2^s (aligned
// blocks of 2^s lanes joined into blocks of 2^(s+1)), which is the pairwise
// tree over the lanes.  The first log2(R) levels halve the rows a lane
// carries (the lane keeps one half and sends its partner the other), the
// remaining ones are a plain butterfly.  Returns the sum of row
// lane_row<R>(lane).
template <int R>
__device__ __forceinline__ float rows_sum(float (&v)[R], int lane) {
#pragma unroll
  for (int s = 0; (R >> s) > 1; ++s) {
    const int c = R >> s;                                  // rows the lane carries
    const bool upper = (lane >> s) & 1;
#pragma unroll
    for (int i = 0; i < c / 2; ++i) {
      const float keep = upper ? v[c / 2 + i] : v[i];
      const float send = upper ? v[i] : v[c / 2 + i];
      v[i] = keep + __shfl_xor(send, 1 << s, kWave);
    }
  }
  float t = v[0];
#pragma unroll
  for (int m = R; m < kWave; m <<= 1) t = t + __shfl_xor(t, m, kWave);
  return t;
}

// Rows per wave and block (host and device): 32 bf16 of weights a lane
// for a block, except for slices of 2048 (KL = 32), whose block is the two
// rows a payload word holds.
__host__ __device__ constexpr int lin_rows_per_wave(int kl) { return kl <= 16 ? 32 / kl : 2; }
// Weight buffers of a worker wave (the ring of blocks in flight).
__host__ __device__ constexpr int lin_buffers(int kl) { return kl <= 16 ? 4 : 2; }

template <int NMAX, int KL>
struct LinSmem {
  static constexpr int kRw = lin_rows_per_wave(KL);
  static constexpr int kBufs = lin_buffers(KL);
  static constexpr int kComm = (NMAX + 1) * kWave * 16;     // peers' chunks + own payload
  static constexpr int kWork = 2 * 64 * KL * 4;             // the slice, two parities
  static constexpr int kBytes = kComm > kWork ? kComm : kWork;
};

template <int P, int NMAX, int KL>
__global__ __launch_bounds__(kWave * NMAX) void k_sim_linear(LinArgs a) {
  using S = LinSmem<NMAX, KL>;
  constexpr int RW = S::kRw;
  constexpr int NBUF = S::kBufs;
  static_assert(NBUF >= 2 && NBUF <= 4, "the worker's step loop serves 2 to 4 buffers");
  static_assert(RW >= 2 && (RW & (RW - 1)) == 0, "rows a block: a power of two >= 2");
  __shared__ __align__(16) uint8_t smem[S::kBytes];
  __shared__ int err;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x >> 6;
  const uint32_t N = (uint32_t)a.nranks;
  const rsrc_t ws = make_rsrc(a.work, a.work_bytes);
  const uint32_t half = (uint32_t)(a.count / 2);            // payload words per rank and parity
  const uint32_t khalf = (uint32_t)(a.kr / 2);              // slice words per rank and parity
  if (threadIdx.x == 0) err = 0;
  __syncthreads();

  if ((int)blockIdx.x >= a.comm_blocks) {
    // ---------------------------------------------------------- worker --
    const int hb = (int)blockIdx.x - a.comm_blocks;
    const int g = hb / a.wpr;
    const int b0 = hb - g * a.wpr;
    if (g >= a.nranks) return;                             // whole workgroup
    const int nblk = (a.bpr - 1 - b0) / a.wpr + 1;
    float* zf = reinterpret_cast<float*>(smem);            // [2][kr]
    const int64_t shard_elems = a.count * a.kr;           // one (layer, rank) shard
    const uint32_t shard_bytes = (uint32_t)(shard_elems * 2);
    const uint32_t lane_off = (uint32_t)lane * KL * 2u;
    auto shard = [&](int l) -> rsrc_t {
      return make_rsrc(a.w + ((int64_t)l * a.nranks + g) * shard_elems, shard_bytes);
    };
    auto row_of = [&](int j, int u) -> int {
      return (b0 + j * a.wpr) * (NMAX * RW) + w * RW + u;
    };
    uint32_t buf[NBUF][RW][KL / 2];
    auto load_block = [&](uint32_t (&d)[RW][KL / 2], rsrc_t wl, int j) {
#pragma unroll
      for (int u = 0; u < RW; ++u)
        load_wrow<KL>(wl, lane_off, (uint32_t)row_of(j, u) * (uint32_t)a.kr * 2u, d[u]);
    };
    const int myrow = lane_row<RW>(lane);
    // the block's RW sums, then its RW/2 payload words for the exchange
    // workgroup: lane l < RW holds row lane_row(l), and its partner l ^ RW/2
    // the next row, so the lanes with an even row write one word each
    auto compute_block = [&](const uint32_t (&d)[RW][KL / 2], const float (&z)[KL], int j,
                             uint32_t par, uint32_t seq) {
      float v[RW];
#pragma unroll
      for (int u = 0; u < RW; ++u) v[u] = lane_part<KL>(z, d[u]);
      const float t = rows_sum<RW>(v, lane);
      const float t1 = __shfl_xor(t, RW / 2, kWave);
      if (lane < RW && (myrow & 1) == 0) {
        const uint32_t row = (uint32_t)(row_of(j, 0) + myrow);
        st8(ws, ((uint32_t)g * 2u + par) * half * 8u + (row >> 1) * 8u,
            u32x2{pack2(to_bf16(t), to_bf16(t1)), seq});
      }
    };
    // op `op`'s layer input, the lane's KL elements of rank g's slice (op 0:
    // rank g's own input row; op i: op i-1's result, published as LL words)
    float z[KL];
    auto get_input = [&](int op, uint32_t seq, uint32_t par) -> bool {
      if (op == 0) {
        const uint16_t* row = a.in + (int64_t)g * a.in_stride + (int64_t)g * a.kr + lane * KL;
        uint32_t d[KL / 2];
        load_inputs<KL>(row, d);
#pragma unroll
        for (int k = 0; k < KL / 2; ++k) {
          z[2 * k] = bf_lo(d[k]);
          z[2 * k + 1] = bf_hi(d[k]);
        }
        return true;
      }
      const uint32_t pseq = seq_prev(seq);
      const uint32_t pstale = seq_prev(seq_prev(pseq));
      float* zb = zf + (par ^ 1u) * a.kr;
      if (w == 0) {
        const uint32_t base = a.act0 + ((uint32_t)g * 2u + (par ^ 1u)) * khalf * 8u;
        // probe first: lane t watches the last word of the t-th 64-word
        // part of the slice, then the whole slice is read and checked
        Waiter wt(a.timeout_ticks, a.ctrl);
        const int nprobe = (int)(khalf / 64u) > 0 ? (int)(khalf / 64u) : 1;
        int st = 0;
        while (true) {
          bool ok = true, bad = false;
          if (lane < nprobe) {
            const uint32_t word = ((uint32_t)lane + 1u) * (khalf / (uint32_t)nprobe) - 1u;
            const u32x2 v = ld8(ws, base + word * 8u);
            ll_flag(v.y, pseq, pstale, ok, bad);
          }
          if (__ballot(bad) != 0ull) {
            if (lane == 0) report_error(a.ctrl, kEcorrupt);
            st = kEcorrupt;
            break;
          }
          if (__ballot(!ok) == 0ull) break;
          if (!wt.again(lane)) {
            st = kEtimeout;
            break;
          }
        }
        while (st == 0) {
          bool ok = true, bad = false;
          uint32_t d[KL / 2];
#pragma unroll
          for (int q = 0; q < KL / 4; ++q) {
            // the lane's KL/2 words: KL/4 16-byte loads
            const u32x4 v = ld16(ws, base + ((uint32_t)lane * (KL / 2) + 2u * q) * 8u);
            bool o1, b1, o2, b2;
            ll_flag(v.y, pseq, pstale, o1, b1);
            ll_flag(v.w, pseq, pstale, o2, b2);
            ok = ok && o1 && o2;
            bad = bad || b1 || b2;
            d[2 * q] = v.x;
            d[2 * q + 1] = v.z;
          }
          if (__ballot(bad) != 0ull) {
            if (lane == 0) report_error(a.ctrl, kEcorrupt);
            st = kEcorrupt;
            break;
          }
          if (__ballot(!ok) == 0ull) {
#pragma unroll
            for (int k = 0; k < KL / 2; ++k) {
              zb[lane * KL + 2 * k] = bf_lo(d[k]);
              zb[lane * KL + 2 * k + 1] = bf_hi(d[k]);
            }
            break;
          }
          if (!wt.again(lane)) {
            st = kEtimeout;
            break;
          }
        }
        if (st != 0 && lane == 0) err = 1;
      }
      __syncthreads();
      if (err) return false;
#pragma unroll
      for (int k = 0; k < KL; ++k) z[k] = zb[lane * KL + k];
      return true;
    };
    // The wave's blocks in order over all ops, NBUF weight buffers in a
    // ring: before block q is summed, the buffer freed by block q-1 starts
    // loading block q + NBUF - 1 -- past the end of an op, the next op's
    // blocks (its layer), so that op's weights stream in while this op's
    // all-reduce runs and before its input exists.
    const int total = a.nops * nblk;
    int lq = 0, lj = 0, llayer = 0;                        // next block to load
    auto load_next = [&](uint32_t (&d)[RW][KL / 2]) {
      if (lq < total) {
        load_block(d, shard(llayer), lj);
        ++lq;
        if (++lj == nblk) {
          lj = 0;
          if (++llayer == a.layers) llayer = 0;
        }
      }
    };
    int cop = 0, cj = 0;                                   // next block to sum
    uint32_t seq = a.seq0;
    uint32_t par = a.parity0;
    // one step: refill the buffer block q-1 used, then sum block q
    auto step = [&](uint32_t (&d)[RW][KL / 2], uint32_t (&freed)[RW][KL / 2]) -> bool {
      load_next(freed);
      if (cj == 0 && !get_input(cop, seq, par)) return false;
      compute_block(d, z, cj, par, seq);
      if (++cj == nblk) {
        cj = 0;
        ++cop;
        seq = seq_next(seq);
        par ^= 1u;
      }
      return true;
    };
#pragma unroll
    for (int b = 0; b < NBUF - 1; ++b) load_next(buf[b]);
    for (int q = 0; q < total; q += NBUF) {
      if (!step(buf[0], buf[NBUF - 1])) return;            // whole workgroup
      if (q + 1 >= total) break;
      if (!step(buf[1], buf[0])) return;
      if constexpr (NBUF > 2) {
        if (q + 2 >= total) break;
        if (!step(buf[2], buf[1])) return;
      }
      if constexpr (NBUF > 3) {
        if (q + 3 >= total) break;
        if (!step(buf[3], buf[2])) return;
      }
    }
    return;
  }

  // ------------------------------------------------------------ exchange --
  const int b = blockIdx.x;
  const int x = b & 7;
  const int q = b >> 3;
  const int g = q / a.Q;
  const int qq = q - g * a.Q;
  if (g >= a.nranks) return;                               // whole workgroup
  // tile group: tiles tgrp, tgrp + 8Q, ... (one tile unless the grid needs
  // fewer exchange workgroups), taken in turn within each op
  const int tgrp = qq * 8 + ((x - (g & 7)) & 7);
  if (tgrp >= a.T) return;                                 // whole workgroup
  const int tstride = 8 * a.Q;
  u32x4* peers = reinterpret_cast<u32x4*>(smem);           // [NMAX][64]
  u32x4* mine = peers + NMAX * kWave;                      // [64]
  const bool role = w < a.nranks;
  const bool own = w == g;
  const int stager = a.nranks == 1 ? g : (g + 1) % a.nranks;
  const rsrc_t rs = make_rsrc(a.scratch, a.scratch_bytes);
  const int64_t slo = (int64_t)g * a.kr, shi = slo + a.kr;
  uint32_t seq = a.seq0;
  uint32_t par = a.parity0;
  for (int op = 0; op < a.nops; ++op) {
   const uint32_t stale = seq_prev(seq_prev(seq));
   for (int tg = tgrp; tg < a.T; tg += tstride) {
    const uint32_t loff = (uint32_t)tg * kTileBytes + (uint32_t)lane * 16u;
    const bool active = loff < a.E;
    int64_t first;
    int n;
    lane_elems<P>(tg, lane, first, n);
    const int keep = chunk_keep<P>(a.count, tg, lane);
    const int nwords = (keep + 1) >> 1;                    // payload words of the lane
    if (w == stager) {
      // the rank's payload words of this tile, as the workers publish them
      const uint32_t base = ((uint32_t)g * 2u + par) * half * 8u + (uint32_t)(first >> 1) * 8u;
      uint32_t d[4] = {0u, 0u, 0u, 0u};
      Waiter wt(a.timeout_ticks, a.ctrl);
      int st = 0;
      bool have = !(active && nwords > 0);
      while (true) {
        bool bad = false;
        if (!have) {
          bool ok = true;
          const u32x4 v0 = ld16(ws, base);
          bool o, bb;
          ll_flag(v0.y, seq, stale, o, bb);
          ok = ok && o;
          bad = bad || bb;
          if (nwords > 1) {
            ll_flag(v0.w, seq, stale, o, bb);
            ok = ok && o;
            bad = bad || bb;
          }
          d[0] = v0.x;
          d[1] = v0.z;
          if (nwords > 2) {
            const u32x4 v1 = ld16(ws, base + 16u);
            ll_flag(v1.y, seq, stale, o, bb);
            ok = ok && o;
            bad = bad || bb;
            if (nwords > 3) {
              ll_flag(v1.w, seq, stale, o, bb);
              ok = ok && o;
              bad = bad || bb;
            }
            d[2] = v1.x;
            d[3] = v1.z;
          }
          have = ok;
        }
        if (__ballot(bad) != 0ull) {
          if (lane == 0) report_error(a.ctrl, kEcorrupt);
          st = kEcorrupt;
          break;
        }
        if (__ballot(!have) == 0ull) break;
        if (!wt.again(lane)) {
          st = kEtimeout;
          break;
        }
      }
      mask_words(d, keep);
      mine[lane] = u32x4{d[0], d[1], d[2], d[3]};
      if (st != 0 && lane == 0) err = 1;
    }
    __syncthreads();
    if (err) return;                                       // whole workgroup
    if (role && !own) {
      const u32x4 m = mine[lane];
      const uint32_t d[4] = {m.x, m.y, m.z, m.w};
      const u32x4 enc = encode_words<P>(d, lane, seq);
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
      if (poll_chunk<P>(rs, src, active, seq, stale, true, a.ctrl, a.timeout_ticks, lane,
                        got) != 0) {
        if (lane == 0) err = 1;
      } else {
        peers[w * kWave + lane] = got;
      }
      if (w == stager) peers[g * kWave + lane] = enc;
    } else if (own && w == stager) {
      // one rank: the own wave stages its own chunk
      const u32x4 m = mine[lane];
      const uint32_t d[4] = {m.x, m.y, m.z, m.w};
      peers[g * kWave + lane] = encode_words<P>(d, lane, seq);
    }
    __syncthreads();
    if (err) return;                                       // whole workgroup
    if (own) {
      u32x4 v[NMAX];
#pragma unroll
      for (int r = 0; r < NMAX; ++r)
        v[r] = (r < a.nranks) ? peers[r * kWave + lane] : u32x4{0u, 0u, 0u, 0u};
      uint32_t o[4];
      reduce_words<P, NMAX>(v, a.nranks, o);
      mask_words(o, keep);
      if (active) store_elems(a.out + ((int64_t)op * a.nranks + g) * a.out_stride, a.count,
                              first, n, o);
      // the part of the result inside rank g's input slice, for the workers
      const uint32_t abase = a.act0 + ((uint32_t)g * 2u + par) * khalf * 8u;
#pragma unroll
      for (int qw = 0; qw < 4; ++qw) {
        const int64_t e = first + 2 * qw;
        if (active && qw < nwords && e >= slo && e < shi)
          st8(ws, abase + (uint32_t)((e - slo) >> 1) * 8u, u32x2{o[qw], seq});
      }
    }
   }
    seq = seq_next(seq);
    par ^= 1u;
  }
}

// ================================================================ host side

template <int P, int NMAX>
static const void* lin_fn_k(int kl) {
  switch (kl) {
    case 4: return reinterpret_cast<const void*>(&k_sim_linear<P, NMAX, 4>);
    case 8: return reinterpret_cast<const void*>(&k_sim_linear<P, NMAX, 8>);
    case 16: return reinterpret_cast<const void*>(&k_sim_linear<P, NMAX, 16>);
    default: return reinterpret_cast<const void*>(&k_sim_linear<P, NMAX, 32>);
  }
}

template <int P>
static const void* lin_fn_n(int nranks, int kl) {
  if (nranks <= 4) return lin_fn_k<P, 4>(kl);
  if (nranks <= 8) return lin_fn_k<P, 8>(kl);
  return lin_fn_k<P, 16>(kl);
}

static const void* lin_fn(int proto, int nranks, int kl) {
  switch (proto) {
    case kLL: return lin_fn_n<kLL>(nranks, kl);
    case kLL128: return lin_fn_n<kLL128>(nranks, kl);
    default: return lin_fn_n<kSentinel>(nranks, kl);
  }
}

static int lin_nmax(int nranks) { return nranks <= 4 ? 4 : (nranks <= 8 ? 8 : 16); }

// Work buffer: payload words [nranks][2][count/2], then slice words
// [nranks][2][kr/2].
static int64_t lin_payload_bytes(const ar_desc* d) { return 8 * (int64_t)d->nranks * d->count; }
static int64_t lin_slice_bytes(const ar_desc* d) { return 8 * (int64_t)d->count; }

int64_t linear_work_bytes(const ar_desc* d) {
  if (!d || d->nranks < 1 || d->nranks > AR_MAX_RANKS || d->count <= 0) return AR_EINVAL;
  const int64_t b = lin_payload_bytes(d) + lin_slice_bytes(d);
  return (b + 255) / 256 * 256;
}

// Beyond the generic checks: the one-shot all-reduce in system mode, LL /
// LL128 / SENTINEL, count = nranks * kr with kr in {256, 512, 1024, 2048},
// layers >= 1, 16-byte aligned weights, a 256-byte aligned work buffer, no
// delays, tile order or trace, the library's own grid.
static int lin_check(const ar_sim_params* p, const void* weights, int32_t layers,
                     const void* work) {
  if (!p) return AR_EINVAL;
  int rc = check_desc(&p->desc);
  if (rc) return rc;
  const ar_desc* d = &p->desc;
  if (d->collective != AR_ALLREDUCE || d->nconsumers != d->nranks) return AR_EINVAL;
  if (d->proto == kBarrier) return AR_EINVAL;
  if (p->nops < 1 || p->reserved != 0) return AR_EINVAL;
  if (p->tile_order || p->delay_ticks || p->trace || p->waves_per_rank) return AR_EINVAL;
  if (p->flags & ~(AR_SIM_COOPERATIVE | AR_SIM_ORDINARY)) return AR_EINVAL;
  if ((p->flags & AR_SIM_COOPERATIVE) && (p->flags & AR_SIM_ORDINARY)) return AR_EINVAL;
  if (p->epoch.parity > 1u || p->epoch.seq == 0u) return AR_EINVAL;
  if (!timeout_ok(p->timeout_ns)) return AR_EINVAL;
  if (d->count <= 0 || d->count % d->nranks != 0) return AR_EINVAL;
  const int64_t kr = d->count / d->nranks;
  if (kr != 256 && kr != 512 && kr != 1024 && kr != 2048) return AR_EINVAL;
  if (layers < 1 || !weights || !work) return AR_EINVAL;
  if (!aligned(weights, 16)) return AR_EALIGN;
  if (!aligned(work, 256)) return AR_EALIGN;
  rc = check_rows(p->in, p->in_stride, d->count);
  if (rc) return rc;
  rc = check_rows(p->out, p->out_stride, d->count);
  if (rc) return rc;
  if (!p->scratch || !p->ctrl) return AR_EINVAL;
  if (!aligned(p->scratch, 256) || !aligned(p->ctrl, 256)) return AR_EALIGN;
  if (linear_work_bytes(d) >= (int64_t(1) << 32)) return AR_ESIZE;
  return AR_OK;
}

struct LinGeom {
  int32_t Q, T, comm_blocks, wpr, bpr, blocks, kl;
  bool coop;
};

// Exchange workgroups: one per (rank, tile).  Workers: up to one per row
// block (nmax waves of RW rows), as many per rank as the resident grid
// holds beside the exchange workgroups -- the occupancy query's figure,
// halved for an ordinary launch -- each taking every wpr-th block.  Without
// a launch flag the launch is cooperative where the device supports it: the
// full resident grid has about twice the workers, whose weight buffers then
// hold more of the next op's layer while this op's all-reduce runs (8 ranks,
// hidden 4096, LL: 10.8 against 14.6 us per op in the first form of the
// workers).
static int lin_geometry(const ar_sim_params* p, const DeviceInfo& di, LinGeom* g) {
  const ar_desc* d = &p->desc;
  const int64_t kr = d->count / d->nranks;
  const int kl = (int)(kr / 64);
  const int nmax = lin_nmax(d->nranks);
  const int64_t T = ceil_div64(encoded_bytes(d->proto, d->count), kTileBytes);
  const int64_t rows_wg = (int64_t)nmax * lin_rows_per_wave(kl);
  if (d->count % rows_wg != 0) return AR_EINVAL;          // every row in a block
  const int64_t bpr = d->count / rows_wg;
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, lin_fn(d->proto, d->nranks, kl),
                                                   kWave * nmax, 0) != hipSuccess ||
      occ <= 0)
    return AR_ELAUNCH;
  const int64_t full = (int64_t)occ * di.cus;
  bool coop;
  if (p->flags & AR_SIM_COOPERATIVE)
    coop = true;
  else if (p->flags & AR_SIM_ORDINARY)
    coop = false;
  else
    coop = di.coop != 0;
  const int64_t cap = coop ? full : full / 2;
  // exchange workgroups: one per tile where that leaves room for a worker
  // workgroup per rank, else each takes several tiles in turn
  int64_t Q = ceil_div64(T, 8), comm = 8 * Q * d->nranks;
  while (Q > 1 && comm + d->nranks > cap) {
    --Q;
    comm = 8 * Q * d->nranks;
  }
  int64_t wpr = (cap - comm) / d->nranks;
  if (wpr > bpr) wpr = bpr;
  if (wpr < 1) return AR_ECAPACITY;
  // an even share of blocks per worker workgroup
  const int64_t per = ceil_div64(bpr, wpr);
  wpr = ceil_div64(bpr, per);
  if ((int64_t)p->nops * per >= (int64_t(1) << 31)) return AR_ESIZE;   // worker block count
  g->Q = (int32_t)Q;
  g->T = (int32_t)T;
  g->comm_blocks = (int32_t)comm;
  g->wpr = (int32_t)wpr;
  g->bpr = (int32_t)bpr;
  g->blocks = (int32_t)(comm + wpr * d->nranks);
  g->kl = kl;
  g->coop = coop;
  return AR_OK;
}

int linear_sim_geometry(const ar_sim_params* p, const void* weights, int32_t layers,
                        const void* work, int32_t* blocks, int32_t* workers,
                        int32_t* cooperative) {
  int rc = lin_check(p, weights, layers, work);
  if (rc) return rc;
  DeviceInfo di;
  rc = device_info(&di);
  if (rc) return rc;
  if ((p->flags & AR_SIM_COOPERATIVE) && !di.coop) return AR_ENODEV;
  LinGeom g;
  rc = lin_geometry(p, di, &g);
  if (rc) return rc;
  if (blocks) *blocks = g.blocks;
  if (workers) *workers = g.wpr * p->desc.nranks;
  if (cooperative) *cooperative = g.coop ? 1 : 0;
  return AR_OK;
}

int linear_sim_run(const ar_sim_params* p, const void* weights, int32_t layers, void* work,
                   hipStream_t s) {
  int rc = lin_check(p, weights, layers, work);
  if (rc) return rc;
  const ar_desc* d = &p->desc;
  DeviceInfo di;
  rc = device_info(&di);
  if (rc) return rc;
  if ((p->flags & AR_SIM_COOPERATIVE) && !di.coop) return AR_ENODEV;
  LinGeom g;
  rc = lin_geometry(p, di, &g);
  if (rc) return rc;
  LinArgs a{};
  a.in = static_cast<const uint16_t*>(p->in);
  a.in_stride = p->in_stride;
  a.w = static_cast<const uint16_t*>(weights);
  a.out = static_cast<uint16_t*>(p->out);
  a.out_stride = p->out_stride;
  a.scratch = static_cast<const uint8_t*>(p->scratch);
  a.scratch_bytes = (uint32_t)desc_scratch_bytes(d);
  a.slot_bytes = (uint32_t)desc_slot_bytes(d);
  a.E = (uint32_t)encoded_bytes(d->proto, d->count);
  a.work = static_cast<const uint8_t*>(work);
  a.work_bytes = (uint32_t)linear_work_bytes(d);
  a.act0 = (uint32_t)lin_payload_bytes(d);
  a.ctrl = static_cast<int*>(p->ctrl);
  a.count = d->count;
  a.kr = (int32_t)(d->count / d->nranks);
  a.layers = layers;
  a.nranks = d->nranks;
  a.nops = p->nops;
  a.Q = g.Q;
  a.T = g.T;
  a.comm_blocks = g.comm_blocks;
  a.wpr = g.wpr;
  a.bpr = g.bpr;
  a.seq0 = p->epoch.seq;
  a.parity0 = p->epoch.parity;
  a.timeout_ticks = ns_to_ticks(p->timeout_ns, di.wallclock_hz);
  void* args[] = {&a};
  const void* fn = lin_fn(d->proto, d->nranks, g.kl);
  const dim3 block(kWave * lin_nmax(d->nranks));
  if (g.coop) {
    const hipError_t e = hipLaunchCooperativeKernel(fn, dim3(g.blocks), block, args, 0, s);
    if (e == hipSuccess || (p->flags & AR_SIM_COOPERATIVE)) return map_hip(e);
    // the runtime refused the library's own choice: the ordinary grid
    ar_sim_params q = *p;
    q.flags = AR_SIM_ORDINARY;
    rc = lin_geometry(&q, di, &g);
    if (rc) return rc;
    a.comm_blocks = g.comm_blocks;
    a.wpr = g.wpr;
  }
  return map_hip(hipLaunchKernel(fn, dim3(g.blocks), block, args, 0, s));
}

}  // namespace ar

using namespace ar;

extern "C" {

int64_t ar_linear_work_bytes(const ar_desc* d) {
  if (!d) return AR_EINVAL;
  const int rc = check_desc(d);
  if (rc) return rc;
  return linear_work_bytes(d);
}

int ar_sim_linear_run(const ar_sim_params* p, const void* weights, int32_t layers, void* work,
                      void* stream) {
  return linear_sim_run(p, weights, layers, work, static_cast<hipStream_t>(stream));
}

int ar_sim_linear_geometry(const ar_sim_params* p, const void* weights, int32_t layers,
                           const void* work, int32_t* blocks, int32_t* workers,
                           int32_t* cooperative) {
  return linear_sim_geometry(p, weights, layers, work, blocks, workers, cooperative);
}

}  // extern "C"
