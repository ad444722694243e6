/*
 * ar_dev.h -- device-callable send / receive / reduce / broadcast on the
 * self-synchronizing receive buffers of ar.h, for use inside HIP kernels
 * (gfx950).
 *
 * "Why Microseconds Matter in AI Infrastructure", section "Communication is
 * becoming part of GPU execution": low-latency send, receive, reduction and
 * broadcast become calls made from inside kernels, so that the kernel that
 * produces a payload can send it from its epilogue (no separate launch, no
 * extra pass over HBM) and the kernel that needs a result can receive and
 * reduce it in place.  This header is that interface; the library's own
 * stream-ordered kernels (ar_pack_*, ar_reduce_validate, ar_gather_validate,
 * ar_scale_pack) are written with it.
 *
 * Model.  A buffer set (ar_dev::buffer) is one descriptor's receive buffers
 * for one op: the scratch of ar.h, its epoch (seq, parity) and sizes.  Work
 * is done per wave and per tile: a tile is 1 KiB of a slot, 16 bytes per
 * lane, and lane l of tile t carries elements [first, first + n) of the
 * payload as given by lane_elements<P>(t, l):
 *     LL        4 elements at 256t + 4l
 *     SENTINEL  8 elements at 512t + 8l          (BARRIER: the same)
 *     LL128     8 elements at 60L + 8j, L = 8t + l/8, j = l%8 < 7;
 *               4 elements at 60L + 56 for j = 7 (the line's flag follows)
 * Data words w[0..3] hold those elements as bf16 pairs, element `first` in
 * the low half of w[0]; words past n/2 are ignored.  Every call must be
 * made by all 64 lanes of a wave together (the polls vote with ballots).
 *
 * Ordering.  Stores and polls are device-scope coherent (sc1) 16-byte
 * buffer accesses.  LL128: send the data of a wave's tiles, call fence(),
 * then send the flags.  A SENTINEL consumer that re-arms (rearm = true) must
 * call fence() before its wave sends anything that licenses the refill of
 * the same slot (dual buffering: the same parity two ops later).
 *
 * Errors.  recv / recv_reduce return 0, AR_ETIMEOUT or AR_ECORRUPT and
 * record the first error in the control block (ar.h); nothing is written
 * for a failed tile.
 */
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "ar.h"
#include "ar_protocols.h"

namespace ar_dev {

using ar::u32x4;

struct buffer {
    uint8_t* scratch;        /* ar.h receive buffers, 256-byte aligned */
    uint32_t scratch_bytes;  /* ar_scratch_bytes(desc) */
    uint32_t slot_bytes;     /* ar_desc_slot_bytes(desc) */
    uint32_t E;              /* ar_encoded_bytes(proto, count) */
    int32_t nranks;
    int32_t nconsumers;
    int64_t count;           /* elements per payload */
    uint32_t seq;            /* epoch of this op */
    uint32_t parity;
};

/* The buffer set from its parts (host or device). */
__host__ __device__ inline buffer make(const void* scratch, uint32_t scratch_bytes,
                                       uint32_t slot_bytes, uint32_t E, int32_t nranks,
                                       int32_t nconsumers, int64_t count, uint32_t seq,
                                       uint32_t parity) {
    buffer b;
    b.scratch = static_cast<uint8_t*>(const_cast<void*>(scratch));
    b.scratch_bytes = scratch_bytes;
    b.slot_bytes = slot_bytes;
    b.E = E;
    b.nranks = nranks;
    b.nconsumers = nconsumers;
    b.count = count;
    b.seq = seq;
    b.parity = parity;
    return b;
}

/* Host: the buffer set of descriptor d for epoch e (sizes from the library). */
inline int make_buffer(const ar_desc* d, void* scratch, ar_epoch e, buffer* b) {
    const int64_t sb = ar_scratch_bytes(d);
    if (sb < 0) return (int)sb;
    const int64_t slot = ar_desc_slot_bytes(d);
    if (slot < 0) return (int)slot;
    b->scratch = static_cast<uint8_t*>(scratch);
    b->scratch_bytes = (uint32_t)sb;
    b->slot_bytes = (uint32_t)slot;
    b->E = (uint32_t)ar_encoded_bytes(d->proto, d->count);
    b->nranks = d->nranks;
    b->nconsumers = d->nconsumers;
    b->count = d->count;
    b->seq = e.seq;
    b->parity = e.parity;
    return AR_OK;
}

/* Tiles of one slot. */
__device__ __forceinline__ int tiles(const buffer& b) {
    return (int)((b.E + ar::kTileBytes - 1) / ar::kTileBytes);
}

template <int P>
__device__ __forceinline__ void lane_elements(int tile, int lane, int64_t* first, int* n) {
    int64_t f;
    int k;
    ar::lane_elems<P>(tile, lane, f, k);
    *first = f;
    *n = k;
}

/* Byte offset of slot `rank` of consumer `c` in this op's parity. */
__device__ __forceinline__ uint32_t slot_offset(const buffer& b, int c, int rank) {
    return (((uint32_t)c * 2u + b.parity) * (uint32_t)b.nranks + (uint32_t)rank) * b.slot_bytes;
}

/* Wait until this wave's earlier stores have completed. */
__device__ __forceinline__ void fence() { ar::fence_release(); }

/* Encode the lane's data words for this op (elements past count must be 0). */
template <int P>
__device__ __forceinline__ u32x4 encode(const buffer& b, int lane, const uint32_t w[4]) {
    return ar::encode_words<P>(w, lane, b.seq);
}

/* Send: the lane's encoded tile chunk of rank `rank` to consumer c. */
template <int P>
__device__ __forceinline__ void send(const buffer& b, int c, int rank, int tile, int lane,
                                     const uint32_t w[4]) {
    const ar::rsrc_t rs = ar::make_rsrc(b.scratch, b.scratch_bytes);
    ar::store_chunk<P>(rs, slot_offset(b, c, rank), 0u, 1, -1, tile, b.E, lane,
                       encode<P>(b, lane, w));
}

/* Broadcast: the same to every consumer except `skip` (-1 = none). */
template <int P>
__device__ __forceinline__ void broadcast(const buffer& b, int rank, int tile, int lane,
                                          const uint32_t w[4], int skip = -1) {
    const ar::rsrc_t rs = ar::make_rsrc(b.scratch, b.scratch_bytes);
    ar::store_chunk<P>(rs, slot_offset(b, 0, rank),
                       2u * (uint32_t)b.nranks * b.slot_bytes, b.nconsumers, skip, tile,
                       b.E, lane, encode<P>(b, lane, w));
}

/* LL128 flags of a tile already sent (after fence()), to consumer c or all. */
__device__ __forceinline__ void send_flags(const buffer& b, int c, int rank, int tile,
                                           int lane) {
    const ar::rsrc_t rs = ar::make_rsrc(b.scratch, b.scratch_bytes);
    ar::produce_flags(rs, slot_offset(b, c, rank), 0u, 1, -1, tile, b.E, b.seq, lane);
}
__device__ __forceinline__ void broadcast_flags(const buffer& b, int rank, int tile,
                                                int lane, int skip = -1) {
    const ar::rsrc_t rs = ar::make_rsrc(b.scratch, b.scratch_bytes);
    ar::produce_flags(rs, slot_offset(b, 0, rank), 2u * (uint32_t)b.nranks * b.slot_bytes,
                      b.nconsumers, skip, tile, b.E, b.seq, lane);
}

/* Receive: poll the lane's chunk of tile `tile` in slot `rank` of consumer c
 * until it holds evidence for this op, validate it and return its data words
 * in w (0 on error). */
template <int P>
__device__ __forceinline__ int recv(const buffer& b, int c, int rank, int tile, int lane,
                                    bool rearm, int* ctrl, uint64_t timeout_ticks,
                                    uint32_t w[4]) {
    const ar::rsrc_t rs = ar::make_rsrc(b.scratch, b.scratch_bytes);
    const uint32_t loff = (uint32_t)tile * ar::kTileBytes + (uint32_t)lane * 16u;
    u32x4 v;
    const int st = ar::poll_chunk<P>(rs, slot_offset(b, c, rank) + loff, loff < b.E, b.seq,
                                     ar::seq_prev(ar::seq_prev(b.seq)), rearm, ctrl,
                                     timeout_ticks, lane, v);
    if (st != 0) v = u32x4{0u, 0u, 0u, 0u};
    ar::chunk_words<P>(v, w);
    return st;
}

/* Receive tile `tile` of every rank for consumer c, in any arrival order,
 * reduce in rank order (binary32, then bf16 to nearest even) and store the
 * lane's elements below count into out_row. */
template <int P, int NMAX>
__device__ __forceinline__ int recv_reduce(const buffer& b, int c, int tile, int lane,
                                           bool rearm, int* ctrl, uint64_t timeout_ticks,
                                           uint16_t* out_row) {
    const ar::rsrc_t rs = ar::make_rsrc(b.scratch, b.scratch_bytes);
    return ar::consume_tile<P, NMAX>(rs, slot_offset(b, c, 0), b.slot_bytes, b.nranks, tile,
                                     b.E, b.seq, ar::seq_prev(ar::seq_prev(b.seq)), rearm,
                                     out_row, b.count, ctrl, timeout_ticks, lane);
}

/* Store the lane's data words of tile `tile` into a bf16 row (elements below
 * count). */
template <int P>
__device__ __forceinline__ void store_row(uint16_t* row, int64_t count, int tile, int lane,
                                          const uint32_t w[4]) {
    int64_t first;
    int n;
    ar::lane_elems<P>(tile, lane, first, n);
    ar::store_elems(row, count, first, n, w);
}

}  // namespace ar_dev
