/*
 * ar.h -- C ABI of the self-synchronizing small-message one-shot bf16
 * all-reduce for MI355X (gfx950).
 *
 * The operation ("SiFAR: Synchronization-Free All-Reduce for Low-Latency LLM
 * Inference", abstract; "flash-comm: Self-Synchronizing Collective
 * Communication for LLM Decoding", abstract): every rank r contributes a bf16
 * payload x_r[0..count); every receiving rank obtains
 *     out[j] = bf16_rne(((f32(x_0[j]) + f32(x_1[j])) + ...) + f32(x_{N-1}[j]))
 * with each '+' one binary32 round-to-nearest-even addition in fixed rank
 * order 0..N-1 (independent of the order in which payloads arrive) and any
 * NaN result written as 0x7FC0.  Each payload travels with its own readiness
 * evidence ("Why Microseconds Matter in AI Infrastructure", section "Latency
 * can matter more than bandwidth"): an LL flag in the same 8-byte store as
 * 4 bytes of data, an LL128-style flag per 128-byte line, or a receive buffer
 * armed with the negative-NaN sentinel 0xFFFF and polled until overwritten.
 * Two buffer parities alternate by epoch (the same section's double
 * buffering; SiFAR's dual buffering), which removes the bottom barrier.
 *
 * On one GPU, N ranks are simulated: rank r's producer writes slot r of a
 * receive buffer, and a consumer polls, validates and reduces.  A receive
 * buffer belongs to one consumer rank; "nconsumers = 1" simulates one rank's
 * share (the receive side of rank 0), "nconsumers = nranks" every rank.
 *
 * Conventions for every call:
 *  - Device pointers are plain device addresses (for example from
 *    hipMalloc or a framework allocator).  The caller owns every buffer; the
 *    library allocates no device memory and keeps no global mutable state
 *    apart from a per-device cache of occupancy figures.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Device work is enqueued asynchronously; AR_OK means "enqueued".
 *  - Return codes: AR_OK (0) or a negative ar_status.  Host-detected errors
 *    are returned before anything is enqueued.  Errors detected on the
 *    device (timeouts, corrupt flags) are written to the status word of the
 *    caller's control block (first error wins) and are read by the caller
 *    after synchronizing.
 *  - bf16 values are passed as raw 16-bit patterns (uint16_t), rows are
 *    row-major, `*_stride` is the distance between rows in elements.
 */
#ifndef AR_H_
#define AR_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------- status --- */
typedef enum {
    AR_OK = 0,
    AR_EINVAL = -1,     /* null pointer, rank count outside 1..16, count < 0,
                           unknown protocol, reserved field not 0 */
    AR_EALIGN = -2,     /* in/out not 16-byte aligned, stride not a multiple
                           of 8 elements, scratch/ctrl not 256-byte aligned */
    AR_ESIZE = -3,      /* a size limit is exceeded (slot > 1 GiB, too many
                           ops, buffer offsets beyond 32 bits) */
    AR_ELAUNCH = -4,    /* a HIP runtime call failed */
    AR_ETIMEOUT = -5,   /* device: a poll passed its deadline */
    AR_ECORRUPT = -6,   /* device: a readiness flag that can never be legal */
    AR_ENODEV = -7,     /* no device, or cooperative launch unsupported */
    AR_ECAPACITY = -8   /* the simulator grid cannot be co-resident */
} ar_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* ar_status_string(int code);

/* ----------------------------------------------------------- protocols --- */
typedef enum {
    AR_LL = 0,        /* 8-byte words: u32 data (2 bf16) | u32 flag = seq     */
    AR_LL128 = 1,     /* 128-byte lines: 60 bf16 (120 B) | u64 flag = seq      */
    AR_SENTINEL = 2,  /* bf16 copy, negative NaNs sent as 0x7FC0, buffer armed
                         with 0xFFFF and polled until overwritten            */
    AR_BARRIER = 3,   /* plain copy; readiness from counters (baseline)       */
    AR_AUTO = 4       /* only for ar_select_protocol                          */
} ar_proto;

#define AR_MAX_RANKS 16

/* Largest poll deadline (timeout_ns) any call accepts: 60 s.  A larger value
 * is rejected with AR_EINVAL, so that every wait stays bounded. */
#define AR_MAX_TIMEOUT_NS 60000000000ull

/*
 * Encoded bytes E of one rank's payload of `count` elements:
 *   LL 16*ceil(count/4), LL128 128*ceil(count/60), SENTINEL and BARRIER
 *   16*ceil(count/8).  Bytes past `count` are zero (LL pad words carry the
 *   flag).  Returns a negative ar_status for a bad protocol or count < 0.
 */
int64_t ar_encoded_bytes(int32_t proto, int64_t count);

/* One slot = E rounded up to 128 bytes (one line). */
int64_t ar_slot_bytes(int32_t proto, int64_t count);

/* ------------------------------------------------------------ epochs --- */
/*
 * Epoch of one op.  seq is the flag value written by LL and LL128 producers
 * (a u32 that starts at 1 and skips 0 on wrap); parity selects one of the two
 * receive-buffer halves and toggles every op.  A buffer half can only hold
 * the current seq, the seq of two ops before (same parity), or 0 (never
 * written); any other flag value is corruption.  The caller owns the epoch
 * and must advance it by one flip per op issued on a receive buffer.
 */
typedef struct {
    uint32_t seq;
    uint32_t parity;
} ar_epoch;

int ar_epoch_init(ar_epoch* e);                      /* {seq 1, parity 0} */
/* Next op ("Why Microseconds Matter in AI Infrastructure", "Latency can
 * matter more than bandwidth": reuse of the other buffer is licensed by the
 * exchange itself).  seq = seq+1 (0 skipped), parity ^= 1. */
int ar_epoch_flip(ar_epoch* e);
int ar_epoch_advance(ar_epoch* e, uint64_t nops);    /* nops flips */

/* -------------------------------------------------------- descriptors --- */
/*
 * Collectives carried by the same self-synchronizing transfers:
 *   AR_ALLREDUCE  one-shot all-reduce: every rank sends its whole payload to
 *                 every consumer, which reduces all of them ("SiFAR" and
 *                 "flash-comm" abstracts; "Why Microseconds Matter in AI
 *                 Infrastructure", "Latency can matter more than bandwidth");
 *   AR_ALLGATHER  standalone all-gather: every consumer receives every
 *                 rank's payload unreduced ("flash-comm", abstract);
 *   AR_TWOSHOT    two-shot all-reduce ("SiFAR", abstract): rank k owns share
 *                 k of the elements (ar_shard_bounds); a reduce-scatter sends
 *                 share k of every payload to rank k, which reduces it in
 *                 rank order, and an all-gather sends each reduced share to
 *                 every rank.  Every rank is a consumer (nconsumers ==
 *                 nranks); LL, LL128 and SENTINEL only.
 * All three give bit-identical results on every consumer, and the two
 * all-reduces give the same bits.
 */
typedef enum {
    AR_ALLREDUCE = 0,
    AR_ALLGATHER = 1,
    AR_TWOSHOT = 2
} ar_collective;

typedef struct {
    int32_t nranks;      /* N simulated ranks, 1..AR_MAX_RANKS              */
    int32_t nconsumers;  /* receive buffers: 1 (rank 0's share) or nranks    */
    int64_t count;       /* bf16 elements per rank payload, >= 0             */
    int32_t proto;       /* AR_LL, AR_LL128, AR_SENTINEL or AR_BARRIER       */
    int32_t collective;  /* ar_collective (0 = one-shot all-reduce)          */
} ar_desc;

/*
 * Share k of a two-shot all-reduce: elements [lo, hi) with width
 * C = ceil(count / nranks) rounded up to a multiple of 8, lo = min(k*C,
 * count), hi = min(lo + C, count); trailing shares may be empty.  Host only.
 */
int ar_shard_bounds(int64_t count, int32_t nranks, int32_t k, int64_t* lo,
                    int64_t* hi);

/*
 * Slot bytes of a descriptor: ar_slot_bytes(proto, count) for AR_ALLREDUCE
 * and AR_ALLGATHER, ar_slot_bytes(proto, C) for AR_TWOSHOT (one share).
 */
int64_t ar_desc_slot_bytes(const ar_desc* d);

/*
 * Receive-buffer ("scratch") layout, caller-owned, 256-byte aligned:
 *   scratch[consumer c][parity p][source rank r][slot_bytes]
 * at byte offset ((c*2 + p)*nranks + r) * slot_bytes.  AR_TWOSHOT has two
 * such regions, each slot holding one share: the reduce-scatter region
 * first (slot r of consumer c: share c of rank r's payload), then, at byte
 * nconsumers*2*nranks*slot_bytes, the all-gather region (slot k of consumer
 * c: share k reduced by rank k).  LL and LL128 scratch must be zero-filled
 * once before first use (a zero flag is "never written"); SENTINEL scratch
 * must be armed with ar_arm_sentinel.
 */
int64_t ar_scratch_bytes(const ar_desc* d);

/*
 * Control block, caller-owned device memory of ar_ctrl_bytes() bytes,
 * 256-byte aligned, zero-filled before first use and after any error:
 *   int32 word 0 = status (0 or a negative ar_status, first error wins),
 *   word 1 = abort flag, words 64.. = one word per simulator wave (rank 0's
 *   progress in share mode, the barrier baseline's counter).
 */
int64_t ar_ctrl_bytes(void);
/* Zero the control block with a small fill kernel (safe inside graphs). */
int ar_ctrl_reset(void* ctrl, void* stream);

/* ------------------------------------------------------- graph capture --- */
/*
 * Every device call of this library is one or more kernel launches on
 * `stream` -- no memset or copy nodes, no host waits -- so a sequence of
 * calls can be captured in a HIP graph (hipStreamBeginCapture, or a
 * framework's graph capture) and replayed; cooperative launches are captured
 * as cooperative kernel nodes.  A replay repeats the epochs its calls were
 * captured with, so flags left by the previous replay would look current (or
 * corrupt) to it.  Start the captured sequence with ar_state_reset of every
 * buffer the sequence uses: each replay then begins from the initial state,
 * in which any epoch is valid.  (ar_sim_run_static clears its own buffers.)
 *
 * ar_state_reset -- returns the buffers of descriptor d to their initial
 * state with fill kernels on `stream`:
 *   ctrl:    ar_ctrl_bytes() bytes, to zero;
 *   scratch: ar_scratch_bytes(d) bytes, to zero (LL, LL128, BARRIER: a zero
 *            flag is "never written"), or every element to 0xFFFF for
 *            AR_SENTINEL (both parities; both regions of AR_TWOSHOT);
 *   work:    ar_linear_work_bytes(d) bytes (the work buffer of
 *            ar_sim_linear_run), to zero.
 * Each may be NULL (left alone), but not all three (AR_EINVAL); each other
 * one 256-byte aligned (AR_EALIGN); a buffer of 4 GiB or more: AR_ESIZE.
 * After a replay the buffers hold what the captured calls left, as after
 * the same calls made eagerly: an eager call on them next takes the epoch
 * that followed the last captured call, or comes after an ar_state_reset.
 */
int ar_state_reset(const ar_desc* d, void* scratch, void* ctrl, void* work, void* stream);

/* ------------------------------------------------------------ producer --- */
/*
 * Producers: encode every simulated rank's payload for epoch `e` into slot r
 * of parity e.parity of every consumer's receive buffer.  AR_TWOSHOT: rank
 * r's share c (encoded on its own, element lo_c first) into the
 * reduce-scatter slot r of consumer c.
 *   in:   device, rank r's payload at in + r*in_stride (elements), bf16.
 *         16-byte aligned, in_stride a multiple of 8 and >= count.  Each
 *         row is read up to the 16-byte boundary after element count-1
 *         (never past in_stride); elements at or past count are ignored.
 *   scratch: device, ar_scratch_bytes(d) bytes (layout above).
 * Stores use device-scope coherent (sc1) 16-byte accesses.
 *
 * ar_pack_ll -- LL: each 8-byte word holds 4 data bytes and the u32 flag
 * seq, written by one store, so a reader that sees the flag sees the data
 * ("Why Microseconds Matter in AI Infrastructure", "Latency can matter more
 * than bandwidth": data and readiness flag in one atomic store).
 */
int ar_pack_ll(const ar_desc* d, const void* in, int64_t in_stride,
               void* scratch, ar_epoch e, void* stream);

/*
 * ar_pack_ll128 -- LL128-style: 120 data bytes then a u64 flag per 128-byte
 * line (same section names an LL128 atomic design).  gfx950 documents no
 * 128-byte store atomicity, so each wave stores the data, issues a
 * device-scope release fence, then stores the flags.
 */
int ar_pack_ll128(const ar_desc* d, const void* in, int64_t in_stride,
                  void* scratch, ar_epoch e, void* stream);

/*
 * ar_pack_sentinel -- copy with every negative NaN replaced by 0x7FC0, so the
 * armed value 0xFFFF is never transmitted (same section: the sentinel must
 * not appear in transmitted data).
 */
int ar_pack_sentinel(const ar_desc* d, const void* in, int64_t in_stride,
                     void* scratch, ar_epoch e, void* stream);

/* ar_pack_plain -- raw copy for the plain-barrier baseline (SiFAR abstract:
 * the one-shot baseline separates data from its top and bottom barriers). */
int ar_pack_plain(const ar_desc* d, const void* in, int64_t in_stride,
                  void* scratch, ar_epoch e, void* stream);

/*
 * ar_arm_sentinel -- fill the SENTINEL slots of parity `parity` (0 or 1; -1 =
 * both) of every consumer with 0xFFFF ("Why Microseconds Matter in AI
 * Infrastructure", "Latency can matter more than bandwidth": the receive
 * buffer is initialized to a negative NaN).  A fill kernel, not a memset.
 * AR_TWOSHOT: both regions.
 */
int ar_arm_sentinel(const ar_desc* d, void* scratch, int32_t parity,
                    void* stream);

/* ------------------------------------------------------------ consumer --- */
#define AR_FLAG_REARM 1   /* SENTINEL: re-arm each slot chunk after reading */

/*
 * ar_reduce_validate -- every consumer c polls its receive buffer (parity
 * e.parity) with device-scope coherent 16-byte loads, validates each block
 * from its own evidence in whatever order blocks arrive, and reduces the N
 * rank rows in fixed rank order ("flash-comm", abstract: receivers validate
 * the blocks they need; reduction order is decoupled from transport order).
 *   out: device, consumer c's result at out + c*out_stride, 16-byte aligned,
 *        out_stride a multiple of 8 and >= count.
 *   ctrl: device control block; a poll that passes timeout_ns writes
 *        AR_ETIMEOUT, an impossible LL/LL128 flag writes AR_ECORRUPT (the
 *        output of that tile is then not written).  timeout_ns 0 = 1 s;
 *        above AR_MAX_TIMEOUT_NS: AR_EINVAL.
 *   flags: AR_FLAG_REARM (SENTINEL only) re-arms what was read, so the same
 *        parity is ready for the op two epochs later.
 * BARRIER payloads carry no evidence: this call then trusts stream order
 * (the kernel boundary after ar_pack_plain is the barrier).
 */
int ar_reduce_validate(const ar_desc* d, void* scratch, void* out,
                       int64_t out_stride, ar_epoch e, void* ctrl,
                       uint64_t timeout_ns, int32_t flags, void* stream);
/*
 * With d->collective == AR_TWOSHOT, ar_reduce_validate runs both steps after
 * the ar_pack_* of the shares: consumer c polls and validates share c of
 * every rank, reduces it in rank order, writes it to its output and sends it
 * (encoded for epoch e) to every other consumer's all-gather slot c; then
 * every consumer polls, validates and decodes the other shares into its
 * output.  Same arguments and errors; AR_FLAG_REARM re-arms both regions.
 * AR_ALLGATHER descriptors are rejected (AR_EINVAL): use ar_gather_validate.
 */

/*
 * ar_gather_validate -- standalone all-gather ("flash-comm", abstract: the
 * same self-synchronizing transfers support all-gather).  d->collective must
 * be AR_ALLGATHER.  After ar_pack_* (which is the same as for the one-shot
 * all-reduce), every consumer c polls and validates slot r of every rank in
 * any arrival order and writes the decoded payload (SENTINEL: negative NaNs
 * arrive as 0x7FC0) to row r of its output:
 *   out: device, consumer c's row r at out + c*out_stride + r*R elements,
 *        R = count rounded up to a multiple of 8; 16-byte aligned,
 *        out_stride a multiple of 8 and >= nranks*R.  Elements of a row at
 *        or past count are not written.
 * ctrl, timeout_ns, flags and errors as for ar_reduce_validate.
 */
int ar_gather_validate(const ar_desc* d, void* scratch, void* out,
                       int64_t out_stride, ar_epoch e, void* ctrl,
                       uint64_t timeout_ns, int32_t flags, void* stream);

/* ------------------------------------------------- producer epilogue --- */
/*
 * In-kernel sending ("Why Microseconds Matter in AI Infrastructure",
 * "Communication is becoming part of GPU execution": send, receive, reduce
 * and broadcast called from inside kernels).  The device-callable interface
 * is include/ar_dev.h; these two entry points compare a producer that sends
 * from its epilogue with one that writes its result for a separate pack.
 * The producer is a per-rank scale: y_r = bf16_rne(f32(x_r) * scales[r]),
 * one binary32 multiplication per element (NaN -> 0x7FC0).
 *
 * ar_scale_pack -- fused: computes y_r and encodes it for epoch e straight
 * into slot r of every consumer (the ar_pack_* layout and encoding of
 * d->proto; AR_ALLREDUCE and AR_ALLGATHER descriptors).  in as for ar_pack_*;
 * scales: device float[nranks], 4-byte aligned.
 */
int ar_scale_pack(const ar_desc* d, const void* in, int64_t in_stride,
                  const float* scales, void* scratch, ar_epoch e, void* stream);

/*
 * ar_scale_rows -- unfused: writes y_r to out + r*out_stride (elements below
 * count only; rows as for ar_pack_*), for a later ar_pack_*.
 */
int ar_scale_rows(int32_t nranks, int64_t count, const void* in, int64_t in_stride,
                  const float* scales, void* out, int64_t out_stride, void* stream);

/* ------------------------------------------------------------ simulator --- */
/*
 * ar_sim_run -- `nops` back-to-back one-shot all-reduces in one persistent
 * cooperative kernel: N simulated ranks as groups of waves placed on
 * different XCDs, producers and consumers running concurrently with no top
 * barrier (consumers start polling at once: "SiFAR", abstract, speculative
 * reduction validated by the readiness evidence) and no bottom barrier
 * (dual-buffered epochs).  Each rank runs consume(i) -> produce(i+1), so a
 * buffer half is reused only after the exchange that licenses it ("Why
 * Microseconds Matter in AI Infrastructure", "Latency can matter more than
 * bandwidth").  With nconsumers = 1 the producers of ranks 1..N-1 take that
 * license from rank 0's block of the previous op.  AR_BARRIER runs the plain
 * baseline instead: one buffer, a top barrier (all N producers arrived) and a
 * bottom barrier (all consumers done) per op, kept by one counter for each
 * wave index: the waves with index w in every rank exchange the same tiles,
 * so each such group is its own barrier domain, as the blocks of a rank with
 * the same index would be across GPUs.
 *
 * Every wave of the grid must be resident at once (waves wait on each
 * other).  A cooperative launch (hipLaunchCooperativeKernel) has the runtime
 * guarantee it, and its grid may fill the occupancy the runtime reports for
 * the kernel on the whole device.  An ordinary launch keeps the grid to half
 * of that and needs the device to be free of other work for the duration
 * (otherwise waits end in AR_ETIMEOUT, never in a hang).  A cooperative
 * launch costs about 15 us more, once per launch, on MI355X.  Launch mode:
 *   AR_SIM_COOPERATIVE: cooperative (AR_ENODEV where unsupported);
 *   AR_SIM_ORDINARY: ordinary;
 *   neither: cooperative where the device supports it, nops >= 32 and its
 *        larger grid lets each wave or workgroup walk fewer tiles or run the
 *        workgroup kernel; ordinary otherwise.  If the runtime refuses such
 *        a cooperative launch, the op runs as an ordinary launch instead
 *        (not with a tile_order, whose shape follows the first geometry:
 *        then the error is returned).
 *
 * Buffers (device):
 *   in:  op i, rank r at in + (i*nranks + r)*in_stride elements.
 *   out: op i, consumer c at out + (i*nconsumers + c)*out_stride elements.
 *   scratch, ctrl: as above; for AR_BARRIER only parity 0 is used and the
 *        control block must be zero at launch (ar_ctrl_reset).
 *   delay_ticks (optional, NULL = none): uint32 [nops][nranks] wall-clock
 *        ticks (ar_wallclock_hz) that each wave of rank r waits before
 *        producing op i.
 *   tile_order (optional): uint16 [nops][nranks][tiles_per_wave] giving, per
 *        op and rank, the order in which each wave writes its own tiles
 *        (a permutation of 0..tiles_per_wave-1; see ar_sim_geometry).
 *   trace (optional): uint64 [nops*2*nranks + 1]; element i*2N + r = latest
 *        wall clock after rank r's last store of op i, element i*2N + N + c
 *        = latest completion of op i at consumer c, last element = earliest
 *        start.  Must be zero-filled, and the last element set to all ones,
 *        by the caller.
 *
 * Other collectives (desc.collective), system mode only (nconsumers ==
 * nranks), LL / LL128 / SENTINEL, no tile_order:
 *   AR_ALLGATHER: op i's output at consumer c is the all-gather layout of
 *        ar_gather_validate at out + (i*nranks + c)*out_stride.  A rank
 *        starts op i+1 once it holds all of op i (one workgroup barrier per
 *        op), as a rank whose next payload depends on this result would;
 *        with LL and one tile per workgroup, each pair of ranks licenses
 *        its own next op instead (no barrier).
 *        One kernel (a workgroup of one wave per peer); AR_SIM_NARROW and
 *        AR_SIM_WIDE are rejected.
 *   AR_TWOSHOT: per op and tile of a share, the reduce-scatter exchange, the
 *        share owner's fixed-order reduce, then the all-gather exchange of
 *        the reduced share; output as for AR_ALLREDUCE.  The trace's
 *        "last store" is that of the reduce-scatter.  Two kernels: a
 *        workgroup of one wave per peer (AR_SIM_WIDE) or one wave per share
 *        tile group serving every peer (AR_SIM_NARROW); without either flag
 *        the library picks by rank count, protocol and share tiles per
 *        workgroup.
 * SENTINEL: every wave waits for its own earlier stores (its re-arms among
 * them) before the first send of each op, so every slot this wave re-armed
 * in op i is armed again before any peer can get to op i+2 and write it.
 * LL and LL128 consumers only read their slots and need no such wait.
 */
#define AR_SIM_COOPERATIVE 1   /* launch with hipLaunchCooperativeKernel */
#define AR_SIM_ORDINARY 8      /* an ordinary launch (never cooperative) */
#define AR_SIM_NARROW 2        /* one wave per tile serving every peer, instead
                                  of a workgroup of one wave per peer */
#define AR_SIM_WIDE 4          /* the workgroup-of-one-wave-per-peer kernel even
                                  when its workgroups must walk several tiles */

typedef struct {
    ar_desc desc;
    int32_t nops;               /* >= 1 */
    int32_t waves_per_rank;     /* tile groups (wide) or waves (narrow) per
                                   rank, a multiple of 8; 0 = library choice */
    int32_t flags;              /* AR_SIM_COOPERATIVE or AR_SIM_ORDINARY,
                                   | AR_SIM_NARROW or AR_SIM_WIDE; 0 =
                                   library choice of both */
    int32_t reserved;           /* must be 0 */
    const void* in;
    int64_t in_stride;
    void* out;
    int64_t out_stride;
    void* scratch;
    void* ctrl;
    ar_epoch epoch;             /* epoch of op 0 */
    uint64_t timeout_ns;        /* per poll; 0 = 1 s; at most
                                   AR_MAX_TIMEOUT_NS (else AR_EINVAL) */
    const uint32_t* delay_ticks;
    const uint16_t* tile_order;
    uint64_t* trace;
} ar_sim_params;

int ar_sim_run(const ar_sim_params* p, void* stream);

/*
 * ar_sim_run_static -- ar_sim_run for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the receive buffers and the control block come from a
 * library-owned device array of AR_STATIC_SCRATCH_BYTES (64 MiB) of receive
 * buffers plus one control block, one copy per device, held until the
 * process ends.  The call allocates nothing.
 *   p: as for ar_sim_run, with p->scratch and p->ctrl NULL (else AR_EINVAL);
 *      ar_scratch_bytes(&p->desc) above AR_STATIC_SCRATCH_BYTES: AR_ESIZE.
 *      Every call clears the control block and the receive buffers it uses
 *      (zero, or the sentinel for AR_SENTINEL) with fill kernels on
 *      `stream` first, so p->epoch need not carry over between calls.
 *   status: device int32, written after the simulator (stream-ordered)
 *      with the control block's status word: 0, AR_ETIMEOUT or AR_ECORRUPT.
 *      Not written when the call returns an error.
 * All calls on one device share the array and leave their contents in it:
 * calls that overlap in time on one device (streams not ordered against
 * each other) race.  Errors otherwise as for ar_sim_run.
 */
#define AR_STATIC_SCRATCH_BYTES (64ll << 20)
int ar_sim_run_static(const ar_sim_params* p, int32_t* status, void* stream);

/*
 * Geometry ar_sim_run will use for these parameters: tile groups per rank
 * (a wave each in the narrow kernel, a workgroup each in the wide kernel),
 * tiles per rank (1 KiB of slot each), tiles per group, total workgroups,
 * the kernel (1 = wide: a workgroup of one wave per peer; 0 = narrow: one
 * wave per tile serving every peer) and the launch (1 = cooperative, 0 =
 * ordinary).  Any output pointer may be NULL.
 */
int ar_sim_geometry(const ar_sim_params* p, int32_t* waves_per_rank,
                    int32_t* tiles_per_rank, int32_t* tiles_per_wave,
                    int32_t* blocks, int32_t* wide, int32_t* cooperative);

/*
 * ar_sim_chain_run -- `nops` one-shot all-reduces in one persistent kernel
 * where each op's result feeds the next op's producer, the dependency of a
 * decode step whose next layer consumes the sum ("Why Microseconds Matter
 * in AI Infrastructure", section "Communication is becoming part of GPU
 * execution": the producing computation and the communication fused into
 * one kernel).  Op 0's payload of rank r is row r of `in` (in +
 * r*in_stride); op i+1's payload of rank r is rank r's own copy of op i's
 * result scaled by scales[(i+1)*nranks + r]: y = bf16_rne(f32(x) * s), one
 * binary32 multiplication per element (NaN -> 0x7FC0), the arithmetic of
 * ar_scale_pack.  Every rank's output of op i at out + (i*nranks + r) *
 * out_stride, as for ar_sim_run.
 *   p: as for ar_sim_run, restricted to desc.collective = AR_ALLREDUCE,
 *      nconsumers = nranks, proto AR_LL / AR_LL128 / AR_SENTINEL,
 *      waves_per_rank = 0, no tile_order, delay_ticks or trace, flags
 *      AR_SIM_COOPERATIVE or AR_SIM_ORDINARY or 0.  Only op 0's input rows
 *      are read.
 *   scales: device, float[nops * nranks], 4-byte aligned; entries of op 0
 *      are not read.
 * One workgroup per (rank, tile) holds every 1 KiB tile of a rank's slot,
 * so the grid must be resident at once: without a launch flag the launch
 * is ordinary when half the occupancy holds it, else cooperative.
 * AR_ECAPACITY when no resident grid holds every tile (payloads above a
 * few tens of KiB per rank at 16 ranks).  Per op: the sends, the polls,
 * one workgroup barrier, the rank-order reduce and the scaling, a second
 * barrier (LL and LL128 up to 8 ranks: every wave reduces and scales
 * itself, and the second barrier goes).  Errors as for ar_sim_run.
 */
int ar_sim_chain_run(const ar_sim_params* p, const float* scales, void* stream);

/* Launch ar_sim_chain_run would make for these parameters: total
 * workgroups and 1 for a cooperative launch.  Either output may be NULL. */
int ar_sim_chain_geometry(const ar_sim_params* p, int32_t* blocks, int32_t* cooperative);

/*
 * ar_sim_linear_run -- `nops` chained one-shot all-reduces in one persistent
 * kernel whose producer is one decode token's row-parallel linear layer
 * shard ("SiFAR: Synchronization-Free All-Reduce for Low-Latency LLM
 * Inference", abstract: communication and model execution designed
 * together, the all-reduce result being the next layer's input; "Why
 * Microseconds Matter in AI Infrastructure", section "Communication is
 * becoming part of GPU execution": the producing kernel sends its payload).
 * With kr = count / nranks, op i's payload of rank r is
 *     y_r[j] = bf16_rne( S(0, kr) )   for j < count,
 * S(a, b) the pairwise binary32 sum of f32(z[r*kr + k]) * f32(W[l][r][j][k])
 * over k in [a, b) (S(a, b) = S(a, m) + S(m, b), m = a + (b - a) / 2; every
 * product and every sum one binary32 operation, nearest even; NaN ->
 * 0x7FC0), l = i mod layers, z = op i-1's result (op 0: row r of `in`, of
 * which only elements [r*kr, (r+1)*kr) are read).  The payloads are
 * all-reduced as by ar_sim_run; every rank's output of op i at out +
 * (i*nranks + r)*out_stride.
 *   p: as for ar_sim_run, restricted to desc.collective = AR_ALLREDUCE,
 *      nconsumers = nranks, proto AR_LL / AR_LL128 / AR_SENTINEL, count =
 *      nranks * kr with kr one of 256, 512, 1024, 2048; waves_per_rank = 0,
 *      no tile_order, delay_ticks or trace; flags AR_SIM_COOPERATIVE,
 *      AR_SIM_ORDINARY or 0 (0: cooperative where the device supports it,
 *      for its larger resident grid; if the runtime refuses that launch, the
 *      ordinary grid).
 *   weights: device, bf16 [layers][nranks][count][kr], 16-byte aligned;
 *      W[l][r][j] is output j's row of weights over rank r's input slice.
 *   layers: >= 1.
 *   work: device, ar_linear_work_bytes(&p->desc) bytes, 256-byte aligned,
 *      caller-owned: zero-filled when allocated and then used only with the
 *      epochs of the scratch it goes with (like the scratch, it holds
 *      epoch-tagged words between launches).  It carries the payload rows
 *      from the GEMV workgroups to the exchange workgroups, which send each
 *      tile whole, and each rank's reduced input slice back to the workers,
 *      as LL words.
 * Exchange workgroups (one per rank and 1 KiB tile, or per group of tiles
 * taken in turn where one per tile would leave no room for a worker per
 * rank) and GEMV worker workgroups beside them must all be resident: the
 * worker count fills what the occupancy query leaves (halved for an ordinary
 * launch); AR_ECAPACITY when not even one worker workgroup per rank fits.  Errors as for ar_sim_run
 * (AR_EINVAL for the restrictions above, AR_EALIGN for alignment).
 */
int ar_sim_linear_run(const ar_sim_params* p, const void* weights, int32_t layers, void* work,
                      void* stream);

/* Bytes of the work buffer of ar_sim_linear_run for descriptor d (a
 * multiple of 256): 8*nranks*count (payload rows, as LL words, two
 * parities) + 8*count (each rank's reduced input slice, as LL words, two
 * parities); < 0 on a bad descriptor. */
int64_t ar_linear_work_bytes(const ar_desc* d);

/* Launch ar_sim_linear_run would make: total workgroups, GEMV worker
 * workgroups among them, and whether it is cooperative.  Any output pointer
 * may be NULL. */
int ar_sim_linear_geometry(const ar_sim_params* p, const void* weights, int32_t layers,
                           const void* work, int32_t* blocks, int32_t* workers,
                           int32_t* cooperative);

/* Wall-clock counter frequency of the current device in Hz. */
int ar_wallclock_hz(double* hz);

/* ------------------------------------------------------------- selector --- */
/*
 * Cost-guided protocol selector ("flash-comm", abstract: the readiness
 * encoding is chosen by message size and number of GPUs, trading
 * synchronization cost against extra bytes; "Why Microseconds Matter in AI
 * Infrastructure", "What I learned from it": selection from measurements).
 * Model per protocol p, rank count and size range:
 *   T_p(S) = alpha_us[p] + beta_us_per_byte[p] * S,
 * with S = 2*count payload bytes per rank.  The entries with the nearest
 * nranks are used (ties: the smaller).  Among them, the entry whose range
 * holds S: the smallest max_bytes >= S, where max_bytes <= 0 means no upper
 * bound; if every range ends below S, the one that ends last.  Several
 * entries per rank count give a piecewise model (the kernels change regime
 * with size; the committed table has one range per interval between two
 * measured sizes, each line through those two measurements).  alpha_us and
 * beta_us_per_byte may be negative; a protocol whose alpha_us or
 * beta_us_per_byte is not a finite number (NaN marks it) is unavailable.
 * Ties go to the lower protocol id (LL < LL128 < SENTINEL < BARRIER).  Host only; writes the
 * chosen id and, if non-NULL, its predicted time.  AR_EINVAL for a NULL
 * table or proto_out, nentries < 1, S < 0, nranks outside 1..16, or no
 * available protocol in the chosen entry.
 *
 * Each entry models one collective (ar_collective): the one-shot all-reduce
 * (0), the all-gather or the two-shot all-reduce.  ar_select_protocol uses
 * the one-shot entries only.
 */
typedef struct {
    int32_t nranks;
    int32_t collective;         /* ar_collective the entry models */
    int64_t max_bytes;          /* inclusive upper end of the range; <= 0: none */
    double alpha_us[4];
    double beta_us_per_byte[4];
} ar_cost_entry;

int ar_select_protocol(const ar_cost_entry* table, int32_t nentries,
                       int64_t payload_bytes, int32_t nranks,
                       int32_t* proto_out, double* predicted_us);

/* The same choice among the entries of one collective; AR_EINVAL when the
 * table has none for it. */
int ar_select_collective(const ar_cost_entry* table, int32_t nentries,
                         int32_t collective, int64_t payload_bytes, int32_t nranks,
                         int32_t* proto_out, double* predicted_us);

/*
 * All-reduce algorithm and protocol: the one-shot choice and the two-shot
 * choice are each made as above from their own entries, and the one with the
 * lower predicted time wins (ties: one-shot; no two-shot entries: one-shot).
 * The pages' reason for both forms ("SiFAR", abstract): one-shot scales
 * poorly with the number of GPUs, two-shot does better at higher degrees.
 * Writes AR_ALLREDUCE or AR_TWOSHOT and the protocol.
 */
int ar_select_allreduce(const ar_cost_entry* table, int32_t nentries,
                        int64_t payload_bytes, int32_t nranks,
                        int32_t* collective_out, int32_t* proto_out,
                        double* predicted_us);

/* -------------------------------------------------------- floor probes --- */
/*
 * Probes for the one-chip floor, the analogue of the speed-of-light bound of
 * "Why Microseconds Matter in AI Infrastructure", section "Defining the
 * physical lower bound" (two round trips to the coherent cache level plus
 * one remote store).
 *
 * ar_probe_pingpong: two single-lane waves on the XCDs `xcd_a` != `xcd_b`
 *   (workgroups are placed round-robin over the 8 XCDs) bounce a flag
 *   `iters` times with device-scope coherent stores and polls.
 *   work: device, >= 512 bytes, zeroed.  result: device uint64[6] =
 *   {total ticks at a, iters, XCC id of a, XCC id of b, status, 0}.
 * ar_probe_loadchain: one lane follows `iters` dependent device-scope
 *   coherent loads through `bytes` of `work` (initialized by the probe).
 *   result: device uint64[2] = {ticks, iters}.
 * ar_probe_copy: streaming 16-byte copy of `bytes` (multiple of 16).
 * ar_probe_empty: an empty kernel (launch floor).
 */
int ar_probe_pingpong(void* work, int32_t iters, int32_t xcd_a, int32_t xcd_b,
                      void* result, void* stream);
int ar_probe_loadchain(void* work, int64_t bytes, int32_t iters, void* result,
                       void* stream);
int ar_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);
int ar_probe_empty(void* stream);

/*
 * ar_probe_placement: the XCD each workgroup of a `blocks` x `threads` grid
 * runs on (the XCC_ID hardware register), taken while the whole grid is
 * resident (each workgroup waits, bounded to 1 s, for all to arrive; one
 * that gives up records -1).  The simulators assume round-robin dispatch
 * over the eight XCDs of one partition: workgroup b on XCD (s + b) mod 8,
 * s depending on earlier dispatches; this checks it.  work: device,
 * 256-byte aligned, >= 4 bytes (zeroed by the call); result: device
 * int32[blocks].
 */
int ar_probe_placement(int32_t blocks, int32_t threads, void* work, void* result,
                       void* stream);

/*
 * ar_probe_litmus: ordering evidence for the coherent accesses the protocols
 * rely on, between one writer wave on XCD `xcd_a` and one reader wave on XCD
 * `xcd_b`, `iters` rounds (work: >= 4096 bytes, zeroed; result: device
 * uint64[8] = {violations, observations, XCC a, XCC b, status, last value,
 * secondary count, 0}).
 *   kind 0, message passing: the writer stores k into a 1 KiB block
 *     (16 bytes a lane), orders, then stores flag k; the reader loads the
 *     flag, orders, loads the block; a violation is a block value older
 *     than the flag it followed.
 *   kind 1, LL word tear: the writer stores 16-byte {k,k,k,k} chunks; the
 *     reader checks that each 8-byte half is self-consistent (violation) and
 *     counts 16-byte chunks whose halves differ (secondary count).
 *   kind 2, re-arm ordering (the dual-buffer chain): the reader re-arms
 *     (stores 0) a word after reading value k, orders, then publishes k; the
 *     writer waits for k, then stores k+1 into the same word; a violation
 *     is the reader finding 0 where k+1 must have landed after its re-arm.
 */
int ar_probe_litmus(void* work, int32_t iters, int32_t xcd_a, int32_t xcd_b,
                    int32_t kind, void* result, void* stream);

/* Library ABI version (bumped when an existing signature or struct changes;
 * entry points may be added between bumps). */
int ar_abi_version(void);

/* hipError_t code of the last HIP call that made an entry point return
 * AR_ELAUNCH on the calling thread (0 if none). */
int ar_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* AR_H_ */
