/*
 * Host-side sanitizer driver for the C oracle (oracle/ar_oracle.c).
 *
 * Built by tests/test_host_sanitize.py with gcc's AddressSanitizer and
 * UndefinedBehaviorSanitizer (no recovery): every oracle entry point runs on
 * small, ragged and degenerate shapes, every protocol, with inputs that mix
 * random bf16 with the special values the protocols treat specially.  Every
 * buffer is a heap block of exactly the size the oracle may touch, so an
 * access one element past it is reported.  Besides memory safety it checks
 * facts of the oracle's contract: an encode then decode returns the payload
 * (canonicalized for the sentinel), a corrupted LL / LL128 flag is reported
 * as corrupt, and the two-shot result equals the one-shot result bit for
 * bit (the same rank-order sum per element).
 *
 * Exit status 0 when every check held; the sanitizers abort on any error.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#include <float.h>

/* the oracle's exported functions (oracle/ar_oracle.c) */
float o_bf16_to_f32(uint16_t b);
uint16_t o_bf16_rne(float f);
uint16_t o_canon_in(uint16_t b);
uint32_t o_epoch_next(uint32_t seq);
uint32_t o_epoch_prev(uint32_t seq);
int64_t o_encoded_bytes(int proto, int64_t count);
int64_t o_encode(int proto, const uint16_t* x, int64_t count, uint32_t seq, uint8_t* out);
int o_decode(int proto, const uint8_t* in, int64_t count, uint32_t seq, uint16_t* y);
void o_reduce(int n, const uint16_t* y, int64_t count, uint16_t* out);
int o_allreduce(int n, const uint16_t* x, int64_t count, int proto, uint32_t seq,
                const int32_t* perm, uint16_t* out);
void o_bf16_rne_array(const float* f, int64_t n, uint16_t* out);
void o_canon_in_array(const uint16_t* b, int64_t n, uint16_t* out);
void o_shard_bounds(int64_t count, int n, int k, int64_t* lo, int64_t* hi);
int o_allgather(int n, const uint16_t* x, int64_t count, int proto, uint32_t seq,
                const int32_t* perm, uint16_t* out);
int o_twoshot(int n, const uint16_t* x, int64_t count, int proto, uint32_t seq,
              uint16_t* out);
void o_scale(const uint16_t* x, int64_t count, float s, uint16_t* out);

enum { LL = 0, LL128 = 1, SENTINEL = 2, BARRIER = 3 };
enum { READY = 0, NOT_READY = 1, CORRUPT = 2 };

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void)
{
    /* xorshift64* (Vigna, "An experimental exploration of Marsaglia's
     * xorshift generators, scrambled") */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 0x2545F4914F6CDD1Dull;
}

static const uint16_t SPECIALS[] = {0xFFFF, 0xFFC0, 0xFF81, 0x7FC0, 0x7F80,
                                    0xFF80, 0x8000, 0x0000, 0x0001, 0x8001};

static uint16_t* payload(int n, int64_t count)
{
    size_t m = (size_t)n * (size_t)count;
    uint16_t* x = (uint16_t*)malloc(m ? m * 2 : 1);
    for (size_t i = 0; i < m; ++i) {
        uint64_t r = next_u64();
        x[i] = (r & 15u) == 0 ? SPECIALS[(r >> 8) % (sizeof SPECIALS / 2)]
                              : (uint16_t)(r >> 32);
    }
    return x;
}

static int failures = 0;
#define CHECK(cond, ...)                                      \
    do {                                                      \
        if (!(cond)) {                                        \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                     \
            fprintf(stderr, "\n");                            \
            ++failures;                                       \
        }                                                     \
    } while (0)

static void round_trip(int proto, const uint16_t* x, int64_t count, uint32_t seq)
{
    int64_t E = o_encoded_bytes(proto, count);
    CHECK(E >= 0, "encoded bytes proto %d count %lld", proto, (long long)count);
    uint8_t* wire = (uint8_t*)malloc(E ? (size_t)E : 1);
    uint16_t* y = (uint16_t*)malloc(count ? (size_t)count * 2 : 1);
    CHECK(o_encode(proto, x, count, seq, wire) == E, "encode length");
    CHECK(o_decode(proto, wire, count, seq, y) == READY, "decode proto %d count %lld",
          proto, (long long)count);
    for (int64_t j = 0; j < count; ++j) {
        uint16_t want = proto == SENTINEL ? o_canon_in(x[j]) : x[j];
        if (y[j] != want) {
            CHECK(0, "round trip proto %d count %lld at %lld", proto, (long long)count,
                  (long long)j);
            break;
        }
    }
    /* the epoch two ahead reads this wire as stale (LL, LL128), never as data */
    const uint32_t ahead = o_epoch_next(o_epoch_next(seq));
    int st = o_decode(proto, wire, count, ahead, y);
    if (proto == LL || proto == LL128)
        CHECK(count == 0 || st == NOT_READY, "stale wire proto %d: %d", proto, st);
    /* an impossible flag value is corruption */
    if ((proto == LL || proto == LL128) && E > 0) {
        const int64_t at = proto == LL ? E - 4 : E - 8;   /* last flag word */
        const uint32_t bad = 0xDEADBEEFu;
        memcpy(wire + at, &bad, 4);
        CHECK(o_decode(proto, wire, count, seq, y) == CORRUPT, "corrupt flag proto %d",
              proto);
    }
    free(wire);
    free(y);
}

static void collectives(int n, int64_t count, int proto, uint32_t seq)
{
    uint16_t* x = payload(n, count);
    for (int r = 0; r < n; ++r)
        round_trip(proto, x + (int64_t)r * count, count, seq);
    int32_t* perm = (int32_t*)malloc((size_t)n * sizeof(int32_t));
    for (int i = 0; i < n; ++i)
        perm[i] = n - 1 - i;
    size_t c2 = count ? (size_t)count * 2 : 1;
    uint16_t* one = (uint16_t*)malloc(c2);
    uint16_t* two = (uint16_t*)malloc(c2);
    uint16_t* all = (uint16_t*)malloc(count ? (size_t)n * c2 : 1);
    CHECK(o_allreduce(n, x, count, proto, seq, perm, one) == READY, "allreduce");
    CHECK(o_twoshot(n, x, count, proto, seq, two) == READY, "twoshot");
    CHECK(count == 0 || memcmp(one, two, (size_t)count * 2) == 0,
          "two-shot != one-shot, n %d count %lld proto %d", n, (long long)count, proto);
    CHECK(o_allgather(n, x, count, proto, seq, perm, all) == READY, "allgather");
    for (int64_t j = 0; j < (int64_t)n * count; ++j) {
        uint16_t want = proto == SENTINEL ? o_canon_in(x[j]) : x[j];
        if (all[j] != want) {
            CHECK(0, "allgather row data n %d count %lld", n, (long long)count);
            break;
        }
    }
    /* a repeated rank in the delivery order is rejected */
    if (n > 1) {
        perm[1] = perm[0];
        CHECK(o_allreduce(n, x, count, proto, seq, perm, one) == CORRUPT, "bad perm");
    }
    o_scale(x, count, -3.5f, one);
    o_scale(x, count, 1e30f, one);
    o_scale(x, count, 1e-30f, one);
    o_canon_in_array(x, count, one);
    free(x);
    free(perm);
    free(one);
    free(two);
    free(all);
}

int main(void)
{
    static const int64_t counts[] = {0, 1, 2, 7, 8, 9, 59, 60, 61, 119, 120, 121,
                                     511, 512, 513, 1000, 4099};
    static const int ranks[] = {1, 2, 3, 5, 8, 16};
    static const uint32_t seqs[] = {1u, 2u, 0xFFFFFFFEu, 0xFFFFFFFFu};
    int cases = 0;
    for (size_t ci = 0; ci < sizeof counts / sizeof counts[0]; ++ci)
        for (size_t ri = 0; ri < sizeof ranks / sizeof ranks[0]; ++ri)
            for (int proto = LL; proto <= BARRIER; ++proto) {
                const uint32_t seq = seqs[(ci + ri + (size_t)proto) % 4];
                collectives(ranks[ri], counts[ci], proto, seq);
                ++cases;
            }
    /* epochs skip 0 on wrap, both ways */
    CHECK(o_epoch_next(0xFFFFFFFFu) == 1u, "epoch wrap");
    CHECK(o_epoch_prev(1u) == 0xFFFFFFFFu, "epoch wrap back");
    /* shard bounds tile [0, count) in order for every rank count */
    for (int64_t count = 0; count <= 300; ++count)
        for (int n = 1; n <= 16; ++n) {
            int64_t end = 0;
            for (int k = 0; k < n; ++k) {
                int64_t lo, hi;
                o_shard_bounds(count, n, k, &lo, &hi);
                CHECK(lo == end && lo <= hi && hi <= count, "shards %lld/%d/%d",
                      (long long)count, n, k);
                end = hi;
            }
            CHECK(end == count, "shards cover %lld/%d", (long long)count, n);
        }
    /* rounding on the float specials */
    const float specials[] = {0.0f, -0.0f, INFINITY, -INFINITY, NAN, -NAN, FLT_MAX,
                              -FLT_MAX, FLT_MIN, FLT_TRUE_MIN, -FLT_TRUE_MIN, 1.0f,
                              1.00390625f, 1.01171875f, 3.3895314e38f};
    const int64_t ns = (int64_t)(sizeof specials / sizeof specials[0]);
    uint16_t* r = (uint16_t*)malloc((size_t)ns * 2);
    o_bf16_rne_array(specials, ns, r);
    CHECK(r[4] == 0x7FC0 && r[5] == 0x7FC0, "NaN rounds to 0x7FC0");
    CHECK(r[2] == 0x7F80 && r[3] == 0xFF80, "infinities keep");
    CHECK(r[6] == 0x7F80, "FLT_MAX rounds up to infinity");
    for (int64_t i = 0; i < ns; ++i)
        CHECK(r[i] == o_bf16_rne(specials[i]), "array and scalar rounding agree");
    free(r);
    printf("%d cases, %d failures\n", cases, failures);
    return failures ? 1 : 0;
}
