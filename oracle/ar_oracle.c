/*
 * ar_oracle.c -- plain CPU oracle for the self-synchronizing one-shot bf16
 * all-reduce.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only tests/, __graft_entry__.smoke() and the cpu_baseline
 * leg of bench.py use it.  It shares no code, header, table or constant
 * generator with the HIP library under collective_synchronization_amd/csrc.
 *
 * It is deliberately slow and literal: one element at a time, one rank at a
 * time, no SIMD, no threads, no blocking.  Build with
 *     gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared
 * and never with -ffast-math (that would flush denormals and reassociate).
 *
 * Sources (the pages are cited by title and section):
 *  [LvB]  "Why Microseconds Matter in AI Infrastructure", section "Latency can
 *         matter more than bandwidth": the low-latency (LL) protocol puts the
 *         data and a readiness flag into one atomic store; LL128 is named as
 *         an atomic line design; the sentinel method arms the receive buffer
 *         with a value such as a negative NaN, polls until it changes, never
 *         transmits that value and must reset the buffer; double buffering
 *         lets the exchange itself license reuse of the other buffer.
 *  [FC]   "flash-comm: Self-Synchronizing Collective Communication for LLM
 *         Decoding", abstract: every block carries evidence of its own
 *         readiness, receivers validate the blocks they need, and the
 *         reduction order is fixed independently of the transport order so
 *         all GPUs get the same result.
 *  [SiFAR] "SiFAR: Synchronization-Free All-Reduce for Low-Latency LLM
 *         Inference", abstract: one-shot all-reduce, dual buffering removes
 *         the bottom (write-after-write) barrier.
 *
 * Readings taken where the pages are silent:
 *  - result: out[j] = bf16_rne(((f32(x0[j]) + f32(x1[j])) + ...) + f32(x_{N-1}[j]))
 *    with every '+' one IEEE binary32 round-to-nearest-even addition, in rank
 *    order 0..N-1, starting from x0 (not from +0.0), denormals kept.
 *  - any NaN result becomes the canonical bf16 quiet NaN 0x7FC0.
 *  - LL word (8 bytes, little endian): bytes 0-3 = x[2k] | x[2k+1] << 16,
 *    bytes 4-7 = u32 flag = seq.  The word count is padded to an even number
 *    (a 16-byte boundary); pad halves are 0 and pad words carry the flag.
 *  - LL128 line (128 bytes): bytes 0-119 = 60 bf16 x[60L .. 60L+59] (0 past
 *    the end), bytes 120-127 = u64 flag = seq.
 *  - sentinel: bf16 0xFFFF (a negative quiet NaN whose two bytes are 0xFF);
 *    every negative-NaN input is canonicalized to 0x7FC0 before transmission;
 *    the slot is padded with zeros to a 16-byte boundary.
 *  - barrier baseline: the raw bf16 payload, zero padded to 16 bytes.
 *  - seq is a u32 epoch counter starting at 1 that skips 0 on wrap; the value
 *    a buffer half can legitimately hold from earlier use is the seq of two
 *    ops before (same parity) or 0 (never written).
 */
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

#define O_LL 0
#define O_LL128 1
#define O_SENTINEL 2
#define O_BARRIER 3

#define O_READY 0
#define O_NOT_READY 1
#define O_CORRUPT 2

#define O_SENTINEL_BITS 0xFFFFu
#define O_CANON_NAN 0x7FC0u

/* ---------------------------------------------------------------- bf16 --- */

/* bf16 -> binary32: a bf16 is the upper half of a binary32, so this is exact. */
float o_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t f32_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

static int f32_is_nan(uint32_t u)
{
    return (u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0;
}

/*
 * binary32 -> bf16, round to nearest, ties to even (IEEE default rounding),
 * written from the definition on the sign-magnitude encoding: keep the upper
 * 16 bits, look at the discarded lower 16 bits, and step the magnitude up by
 * one bf16 unit when the discarded part is more than half a unit, or exactly
 * half a unit and the kept part is odd.  A carry out of the mantissa moves
 * into the exponent, which is the correct next value (and gives infinity on
 * overflow).  NaN -> 0x7FC0 (reading: canonical quiet NaN).
 */
uint16_t o_bf16_rne(float f)
{
    uint32_t u = f32_bits(f);
    if (f32_is_nan(u))
        return (uint16_t)O_CANON_NAN;
    uint32_t kept = u >> 16;            /* sign | exponent | 7-bit mantissa */
    uint32_t discarded = u & 0xFFFFu;   /* fraction below the bf16 unit     */
    const uint32_t half = 0x8000u;
    int up;
    if (discarded > half)
        up = 1;
    else if (discarded < half)
        up = 0;
    else
        up = (int)(kept & 1u);          /* tie: go to the even neighbour    */
    return (uint16_t)(kept + (uint32_t)up);
}

/*
 * Sentinel protocol input canonicalization ([LvB]: the sentinel value must
 * never be transmitted).  Reading: every negative NaN (sign 1, exponent all
 * ones, mantissa non-zero) becomes 0x7FC0; everything else is unchanged.
 */
uint16_t o_canon_in(uint16_t b)
{
    int neg = (b & 0x8000u) != 0;
    int exp_all_ones = (b & 0x7F80u) == 0x7F80u;
    int mant_nonzero = (b & 0x007Fu) != 0;
    if (neg && exp_all_ones && mant_nonzero)
        return (uint16_t)O_CANON_NAN;
    return b;
}

/* ----------------------------------------------------------------- epochs --- */

/* Dual-buffered epochs ([LvB] double buffering, [SiFAR] dual buffering). */
uint32_t o_epoch_next(uint32_t seq)
{
    return seq == 0xFFFFFFFFu ? 1u : seq + 1u;
}

uint32_t o_epoch_prev(uint32_t seq)
{
    return seq == 1u ? 0xFFFFFFFFu : seq - 1u;
}

/* ------------------------------------------------------------- encodings --- */

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* Bytes the encoding of `count` bf16 elements occupies (E). */
int64_t o_encoded_bytes(int proto, int64_t count)
{
    if (count < 0)
        return -1;
    switch (proto) {
    case O_LL:       return 16 * ceil_div(count, 4);    /* 2 words per 16 B   */
    case O_LL128:    return 128 * ceil_div(count, 60);  /* 60 elements a line */
    case O_SENTINEL:
    case O_BARRIER:  return 16 * ceil_div(count, 8);
    default:         return -1;
    }
}

static uint16_t elem_or_zero(const uint16_t* x, int64_t count, int64_t j)
{
    return j < count ? x[j] : (uint16_t)0;
}

static void put_u16(uint8_t* p, uint16_t v)
{
    p[0] = (uint8_t)(v & 0xFF);
    p[1] = (uint8_t)(v >> 8);
}

static void put_u32(uint8_t* p, uint32_t v)
{
    for (int i = 0; i < 4; ++i)
        p[i] = (uint8_t)(v >> (8 * i));
}

static void put_u64(uint8_t* p, uint64_t v)
{
    for (int i = 0; i < 8; ++i)
        p[i] = (uint8_t)(v >> (8 * i));
}

static uint16_t get_u16(const uint8_t* p)
{
    return (uint16_t)(p[0] | (p[1] << 8));
}

static uint32_t get_u32(const uint8_t* p)
{
    uint32_t v = 0;
    for (int i = 0; i < 4; ++i)
        v |= (uint32_t)p[i] << (8 * i);
    return v;
}

static uint64_t get_u64(const uint8_t* p)
{
    uint64_t v = 0;
    for (int i = 0; i < 8; ++i)
        v |= (uint64_t)p[i] << (8 * i);
    return v;
}

/*
 * Encode one rank's payload x[0..count) for epoch `seq` into out[0..E).
 * LL ([LvB]): data and flag share one 8-byte word.
 * LL128 ([LvB]): one flag per 128-byte line.
 * Sentinel ([LvB]): canonicalized copy.
 * Barrier: raw copy.
 * Returns E, or -1 for a bad protocol.
 */
int64_t o_encode(int proto, const uint16_t* x, int64_t count, uint32_t seq,
                 uint8_t* out)
{
    int64_t E = o_encoded_bytes(proto, count);
    if (E < 0)
        return -1;
    if (proto == O_LL) {
        int64_t nwords = E / 8;
        for (int64_t k = 0; k < nwords; ++k) {
            uint32_t lo = elem_or_zero(x, count, 2 * k);
            uint32_t hi = elem_or_zero(x, count, 2 * k + 1);
            uint8_t* w = out + 8 * k;
            put_u32(w, lo | (hi << 16));
            put_u32(w + 4, seq);
        }
    } else if (proto == O_LL128) {
        int64_t nlines = E / 128;
        for (int64_t L = 0; L < nlines; ++L) {
            uint8_t* line = out + 128 * L;
            for (int i = 0; i < 60; ++i)
                put_u16(line + 2 * i, elem_or_zero(x, count, 60 * L + i));
            put_u64(line + 120, (uint64_t)seq);
        }
    } else if (proto == O_SENTINEL) {
        int64_t nelem = E / 2;
        for (int64_t j = 0; j < nelem; ++j)
            put_u16(out + 2 * j, o_canon_in(elem_or_zero(x, count, j)));
    } else {
        int64_t nelem = E / 2;
        for (int64_t j = 0; j < nelem; ++j)
            put_u16(out + 2 * j, elem_or_zero(x, count, j));
    }
    return E;
}

/* A flag value other than the current seq: stale (seq of two ops before, or
 * 0 = never written) means "not yet"; anything else means corruption. */
static int classify_flag(uint64_t flag, uint32_t seq)
{
    if (flag == (uint64_t)seq)
        return O_READY;
    uint32_t stale = o_epoch_prev(o_epoch_prev(seq));
    if (flag == 0 || flag == (uint64_t)stale)
        return O_NOT_READY;
    return O_CORRUPT;
}

/*
 * Validate and decode one received slot ([FC]: the receiver validates each
 * block from the evidence it carries).  Writes y[0..count) and returns
 * O_READY, O_NOT_READY or O_CORRUPT (corruption wins over not-ready).
 * y is written even when not ready (callers must not use it then).
 */
int o_decode(int proto, const uint8_t* in, int64_t count, uint32_t seq,
             uint16_t* y)
{
    int64_t E = o_encoded_bytes(proto, count);
    if (E < 0)
        return O_CORRUPT;
    int status = O_READY;
    if (proto == O_LL) {
        int64_t nwords = E / 8;
        for (int64_t k = 0; k < nwords; ++k) {
            const uint8_t* w = in + 8 * k;
            int c = classify_flag(get_u32(w + 4), seq);
            if (c > status)
                status = c;
            uint32_t data = get_u32(w);
            if (2 * k < count)
                y[2 * k] = (uint16_t)(data & 0xFFFFu);
            if (2 * k + 1 < count)
                y[2 * k + 1] = (uint16_t)(data >> 16);
        }
    } else if (proto == O_LL128) {
        int64_t nlines = E / 128;
        for (int64_t L = 0; L < nlines; ++L) {
            const uint8_t* line = in + 128 * L;
            int c = classify_flag(get_u64(line + 120), seq);
            if (c > status)
                status = c;
            for (int i = 0; i < 60; ++i)
                if (60 * L + i < count)
                    y[60 * L + i] = get_u16(line + 2 * i);
        }
    } else if (proto == O_SENTINEL) {
        /* Ready only when no element still holds the sentinel ([LvB]). */
        int64_t nelem = E / 2;
        for (int64_t j = 0; j < nelem; ++j) {
            uint16_t v = get_u16(in + 2 * j);
            if (v == O_SENTINEL_BITS && status == O_READY)
                status = O_NOT_READY;
            if (j < count)
                y[j] = v;
        }
    } else {
        /* Barrier baseline: readiness comes from the barrier, not the data. */
        for (int64_t j = 0; j < count; ++j)
            y[j] = get_u16(in + 2 * j);
    }
    return status;
}

/* ------------------------------------------------------------- reduction --- */

/*
 * Fixed-order reduction ([FC]: reduction order is independent of arrival
 * order).  y holds n rank rows of `count` bf16 (row r at y + r*count).
 * Each element: start from rank 0, add ranks 1..n-1 one binary32 addition
 * at a time, then round to bf16.
 */
void o_reduce(int n, const uint16_t* y, int64_t count, uint16_t* out)
{
    for (int64_t j = 0; j < count; ++j) {
        float acc = o_bf16_to_f32(y[j]);
        for (int r = 1; r < n; ++r) {
            float term = o_bf16_to_f32(y[(int64_t)r * count + j]);
            acc = acc + term;
        }
        out[j] = o_bf16_rne(acc);
    }
}

/*
 * One complete one-shot all-reduce as seen by one receiving rank:
 * every rank's payload x[r] is encoded for epoch seq, "delivered" in the
 * order given by perm (a permutation of 0..n-1; NULL = rank order),
 * validated and decoded into row r, then reduced in rank order.
 * x is n rows of `count` bf16 (row r at x + r*count).
 * Returns O_READY on success, or the worst decode status.
 */
int o_allreduce(int n, const uint16_t* x, int64_t count, int proto,
                uint32_t seq, const int32_t* perm, uint16_t* out)
{
    if (n < 1 || count < 0)
        return O_CORRUPT;
    int64_t E = o_encoded_bytes(proto, count);
    if (E < 0)
        return O_CORRUPT;
    uint8_t* wire = (uint8_t*)malloc((size_t)(E > 0 ? E : 1));
    uint16_t* y = (uint16_t*)malloc((size_t)(n * count > 0 ? n * count : 1) * 2);
    int* seen = (int*)calloc((size_t)n, sizeof(int));
    if (!wire || !y || !seen) {
        free(wire); free(y); free(seen);
        return O_CORRUPT;
    }
    int status = O_READY;
    for (int i = 0; i < n; ++i) {
        int r = perm ? perm[i] : i;
        if (r < 0 || r >= n || seen[r]) {
            status = O_CORRUPT;
            break;
        }
        seen[r] = 1;
        o_encode(proto, x + (int64_t)r * count, count, seq, wire);
        int c = o_decode(proto, wire, count, seq, y + (int64_t)r * count);
        if (c > status)
            status = c;
    }
    if (status == O_READY)
        o_reduce(n, y, count, out);
    free(wire);
    free(y);
    free(seen);
    return status;
}

/* Array helpers for the tests (element-wise wrappers, nothing more). */
void o_bf16_rne_array(const float* f, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = o_bf16_rne(f[i]);
}

void o_canon_in_array(const uint16_t* b, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = o_canon_in(b[i]);
}

/* ------------------------------------------------ all-gather, two-shot --- */
/*
 * [FC] abstract: the same self-synchronizing transfer also carries a
 * standalone all-gather.  [SiFAR] abstract: the two-shot all-reduce (a
 * reduce-scatter, each rank reducing one share, then an all-gather of the
 * reduced shares) is the form that scales to more GPUs.
 *
 * Readings:
 *  - shares: rank k owns elements [lo_k, hi_k) with width C = ceil(count/n)
 *    rounded up to a multiple of 8 elements (16 bytes), lo_k = min(k*C,
 *    count), hi_k = min(lo_k + C, count); trailing shares may be empty.
 *  - each share travels with the same encodings as a whole payload, encoded
 *    on its own (element 0 of the share is element 0 of the encoding).
 *  - all-gather output: n rows, row r = rank r's payload as decoded (the
 *    sentinel protocol delivers canon_in(x)).
 */
void o_shard_bounds(int64_t count, int n, int k, int64_t* lo, int64_t* hi)
{
    int64_t w = (count + n - 1) / n;
    w = (w + 7) / 8 * 8;
    int64_t a = (int64_t)k * w;
    if (a > count)
        a = count;
    int64_t b = a + w;
    if (b > count)
        b = count;
    *lo = a;
    *hi = b;
}

/*
 * All-gather as seen by one receiving rank: every rank's payload is encoded
 * for epoch seq, delivered in perm order (NULL = rank order), validated and
 * decoded into row r of out (n rows of `count`).  Returns the worst status.
 */
int o_allgather(int n, const uint16_t* x, int64_t count, int proto,
                uint32_t seq, const int32_t* perm, uint16_t* out)
{
    if (n < 1 || count < 0)
        return O_CORRUPT;
    int64_t E = o_encoded_bytes(proto, count);
    if (E < 0)
        return O_CORRUPT;
    uint8_t* wire = (uint8_t*)malloc((size_t)(E > 0 ? E : 1));
    int* seen = (int*)calloc((size_t)n, sizeof(int));
    if (!wire || !seen) {
        free(wire); free(seen);
        return O_CORRUPT;
    }
    int status = O_READY;
    for (int i = 0; i < n; ++i) {
        int r = perm ? perm[i] : i;
        if (r < 0 || r >= n || seen[r]) {
            status = O_CORRUPT;
            break;
        }
        seen[r] = 1;
        o_encode(proto, x + (int64_t)r * count, count, seq, wire);
        int c = o_decode(proto, wire, count, seq, out + (int64_t)r * count);
        if (c > status)
            status = c;
    }
    free(wire);
    free(seen);
    return status;
}

/*
 * Two-shot all-reduce, every step in order:
 *  1. reduce-scatter: for each share k, every rank r's elements [lo_k, hi_k)
 *     are encoded for epoch seq, delivered to rank k, validated and decoded;
 *     rank k reduces them in rank order (o_reduce) into its reduced share;
 *  2. all-gather: each reduced share is encoded for epoch seq, delivered to
 *     every rank, validated, decoded and written to out[lo_k, hi_k).
 * x: n rows of `count`; out: `count`.  Returns the worst status.
 */
int o_twoshot(int n, const uint16_t* x, int64_t count, int proto,
              uint32_t seq, uint16_t* out)
{
    if (n < 1 || count < 0)
        return O_CORRUPT;
    int64_t lo0, w;
    o_shard_bounds(count, n, 0, &lo0, &w);          /* w = width of share 0 */
    w -= lo0;
    int64_t Emax = o_encoded_bytes(proto, w > 0 ? w : 1);
    uint8_t* wire = (uint8_t*)malloc((size_t)(Emax > 0 ? Emax : 1));
    uint16_t* y = (uint16_t*)malloc((size_t)(n * (w > 0 ? w : 1)) * 2);
    uint16_t* red = (uint16_t*)malloc((size_t)(w > 0 ? w : 1) * 2);
    if (!wire || !y || !red) {
        free(wire); free(y); free(red);
        return O_CORRUPT;
    }
    int status = O_READY;
    for (int k = 0; k < n; ++k) {
        int64_t lo, hi;
        o_shard_bounds(count, n, k, &lo, &hi);
        int64_t m = hi - lo;
        if (m == 0)
            continue;
        for (int r = 0; r < n; ++r) {                /* step 1 */
            o_encode(proto, x + (int64_t)r * count + lo, m, seq, wire);
            int c = o_decode(proto, wire, m, seq, y + (int64_t)r * m);
            if (c > status)
                status = c;
        }
        o_reduce(n, y, m, red);
        o_encode(proto, red, m, seq, wire);           /* step 2 */
        int c = o_decode(proto, wire, m, seq, out + lo);
        if (c > status)
            status = c;
    }
    free(wire);
    free(y);
    free(red);
    return status;
}

/* ------------------------------------------------ producer epilogue --- */
/*
 * "Why Microseconds Matter in AI Infrastructure", section "Communication is
 * becoming part of GPU execution": send, receive and reduce become callable
 * from inside the kernels that produce the data.  The producer used to
 * exercise that path is a per-rank scaling epilogue (a reading: the pages
 * name no producer):
 *     y[j] = bf16_rne( f32(x[j]) * s )
 * one binary32 multiplication, round to nearest even, then the bf16
 * rounding of o_bf16_rne (NaN -> 0x7FC0).
 */
void o_scale(const uint16_t* x, int64_t count, float s, uint16_t* out)
{
    for (int64_t j = 0; j < count; ++j) {
        float p = o_bf16_to_f32(x[j]) * s;
        out[j] = o_bf16_rne(p);
    }
}

/* --------------------------------------- row-parallel linear producer --- */
/*
 * "SiFAR: Synchronization-Free All-Reduce for Low-Latency LLM Inference",
 * abstract: communication and model execution are designed together, the
 * all-reduce's result being the next layer's input; "Why Microseconds
 * Matter in AI Infrastructure", section "Communication is becoming part of
 * GPU execution": the kernel that produces a payload sends it itself.  The
 * producer here is one decode token's row-parallel linear layer shard (a
 * reading: the pages name the pattern, not a layer).  Rank g holds the
 * inputs v[0..kr) (elements [g*kr, (g+1)*kr) of the layer's input row) and,
 * for every output j, the weight row wt[j][0..kr) of its input slice; its
 * partial output is
 *     y[j] = bf16_rne( S(0, kr) )
 *     S(a, b) = f32(v[a]) * f32(wt[j][a])                        if b - a == 1
 *             = S(a, m) + S(m, b),  m = a + (b - a) / 2          otherwise
 * every product one binary32 multiplication and every '+' one binary32
 * addition, round to nearest even, denormals kept: the textbook pairwise
 * (recursive halving) summation of the kr products.
 */
static float pairwise_dot(const uint16_t* v, const uint16_t* w, int64_t a, int64_t b)
{
    if (b - a == 1)
        return o_bf16_to_f32(v[a]) * o_bf16_to_f32(w[a]);
    int64_t m = a + (b - a) / 2;
    float left = pairwise_dot(v, w, a, m);
    float right = pairwise_dot(v, w, m, b);
    return left + right;
}

/* The binary32 sum S(0, kr) for one weight row (kr >= 1). */
float o_linear_dot(const uint16_t* v, const uint16_t* w, int64_t kr)
{
    if (kr < 1)
        return 0.0f;
    return pairwise_dot(v, w, 0, kr);
}

/* One rank's partial output: wt is `count` rows of kr bf16 (row j at
 * wt + j*kr); out[j] = bf16_rne(S(0, kr)) of row j. */
void o_linear_shard(const uint16_t* v, int64_t kr, const uint16_t* wt, int64_t count,
                    uint16_t* out)
{
    for (int64_t j = 0; j < count; ++j)
        out[j] = o_bf16_rne(o_linear_dot(v, wt + j * kr, kr));
}
