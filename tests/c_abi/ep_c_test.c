/*
 * A C caller of libepget: the hot path driven through the C ABI alone
 * (include/ep_get.h, HIP runtime for memory), with no Python in between,
 * checked against the CPU oracle (oracle/ep_oracle.c, linked in as the
 * reference).  TEST INFRASTRUCTURE: built by __graft_entry__.build(), run by
 * tests/test_c_abi.py on a GPU.
 *
 * Two problems: one of two layout chunks (the separate layout, dispatch and
 * combine calls) and one of a single chunk (also the one-call layout and
 * dispatch).  Layout outputs, slots and dispatched rows must equal the
 * oracle's bit for bit; the combine within 1e-3 + 1e-2 |ref|.
 * Exit status 0 on success.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ep_get.h"

/* the oracle's entry points (oracle/ep_oracle.c) */
int oracle_layout(int32_t T, int32_t K, int32_t E, int32_t R, int32_t G, int32_t A, int64_t S,
                  const int32_t *topk_idx, int32_t *expert_count, int32_t *expert_offset,
                  int32_t *rank_row_count, int32_t *rank_token_count, int32_t *group_token_count,
                  uint8_t *is_token_in_rank, int32_t *token_slot);
void oracle_dispatch(int32_t T, int32_t H, int32_t K, int64_t num_rows, const uint16_t *x,
                     const float *topk_weights, const int32_t *token_slot, uint16_t *recv_x,
                     int32_t *recv_src_token, float *recv_weight);
void oracle_combine(int32_t T, int32_t H, int32_t K, int64_t num_rows, const uint16_t *y,
                    const int32_t *token_slot, const float *topk_weights, uint16_t *out);
void oracle_bf16_to_double(int64_t n, const uint16_t *in, double *out);

#define CHECK_HIP(call)                                                            \
    do {                                                                           \
        hipError_t e_ = (call);                                                    \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #call,          \
                    hipGetErrorString(e_));                                        \
            exit(2);                                                               \
        }                                                                          \
    } while (0)
#define CHECK_EP(call)                                                             \
    do {                                                                           \
        int r_ = (call);                                                           \
        if (r_ != EP_OK) {                                                         \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #call,          \
                    ep_error_string(r_));                                          \
            exit(3);                                                               \
        }                                                                          \
    } while (0)

/* splitmix64: seeded input bits only */
static uint64_t rng_state;
static uint64_t next_u64(void) {
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static float next_unit(void) { return (float)(next_u64() >> 40) / 16777216.0f; }

static void *dev_alloc(size_t bytes) {
    void *p = NULL;
    CHECK_HIP(hipMalloc(&p, bytes > 0 ? bytes : 1));
    return p;
}
static void to_dev(void *d, const void *h, size_t bytes) { CHECK_HIP(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice)); }
static void to_host(void *h, const void *d, size_t bytes) { CHECK_HIP(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost)); }

static int fail(const char *what, long at) {
    fprintf(stderr, "mismatch in %s at %ld\n", what, at);
    return 1;
}
static int same_i32(const char *what, const int32_t *a, const int32_t *b, long n) {
    for (long i = 0; i < n; ++i)
        if (a[i] != b[i]) return fail(what, i);
    return 0;
}

/* Layout outputs on the device. */
typedef struct {
    int32_t *count, *offset, *rank_rows, *rank_tokens, *group_tokens, *slot;
    uint8_t *map;
    void *ws;
    size_t ws_bytes;
} dev_layout;

static dev_layout alloc_layout(const ep_problem *p) {
    dev_layout d;
    d.count = dev_alloc(4 * (size_t)p->num_experts);
    d.offset = dev_alloc(4 * (size_t)p->num_experts);
    d.rank_rows = dev_alloc(4 * (size_t)p->num_ranks);
    d.rank_tokens = dev_alloc(4 * (size_t)p->num_ranks);
    d.group_tokens = dev_alloc(4 * (size_t)p->num_groups);
    d.slot = dev_alloc(4 * (size_t)p->num_tokens * p->num_topk);
    d.map = dev_alloc((size_t)p->num_tokens * p->num_ranks);
    d.ws_bytes = ep_workspace_bytes(p);
    d.ws = dev_alloc(d.ws_bytes);
    return d;
}

static int check_layout(const ep_problem *p, const dev_layout *d, int status, int ref_status,
                        const int32_t *cnt, const int32_t *off, const int32_t *rrc, const int32_t *rtc,
                        const int32_t *gtc, const uint8_t *map, const int32_t *slot) {
    const int E = p->num_experts, R = p->num_ranks, G = p->num_groups;
    const long TK = (long)p->num_tokens * p->num_topk, TR = (long)p->num_tokens * R;
    int32_t *g = malloc(4 * (size_t)(TK > E ? TK : E) + 16);
    uint8_t *gm = malloc((size_t)TR + 1);
    int bad = status != ref_status ? fail("status", status) : 0;
    to_host(g, d->count, 4 * (size_t)E);
    bad |= same_i32("expert_count", g, cnt, E);
    to_host(g, d->offset, 4 * (size_t)E);
    bad |= same_i32("expert_offset", g, off, E);
    to_host(g, d->rank_rows, 4 * (size_t)R);
    bad |= same_i32("rank_row_count", g, rrc, R);
    to_host(g, d->rank_tokens, 4 * (size_t)R);
    bad |= same_i32("rank_token_count", g, rtc, R);
    to_host(g, d->group_tokens, 4 * (size_t)G);
    bad |= same_i32("group_token_count", g, gtc, G);
    to_host(g, d->slot, 4 * (size_t)TK);
    bad |= same_i32("token_slot", g, slot, TK);
    to_host(gm, d->map, (size_t)TR);
    if (memcmp(gm, map, (size_t)TR) != 0) bad |= fail("is_token_in_rank", 0);
    free(g);
    free(gm);
    return bad;
}

static int run_problem(int32_t T, int32_t H, int32_t E, int32_t K, int32_t R, int32_t G, uint64_t seed) {
    ep_problem p = {T, H, E, K, R, G, 1, 0, 0};
    p.rank_stride_rows = ep_rank_stride_hint(&p);
    const int64_t S = p.rank_stride_rows, rows = S * R;
    const long TK = (long)T * K;
    rng_state = seed;

    /* inputs: K distinct experts per token, weights in [0,1), x finite bf16 */
    int32_t *idx = malloc(4 * (size_t)TK);
    float *w = malloc(4 * (size_t)TK);
    uint16_t *x = malloc(2 * (size_t)T * H);
    for (int32_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < K; ++j) {
            int32_t e, dup;
            do {
                e = (int32_t)(next_u64() % (uint64_t)E);
                dup = 0;
                for (int32_t i = 0; i < j; ++i) dup |= idx[(long)t * K + i] == e;
            } while (dup);
            idx[(long)t * K + j] = e;
            w[(long)t * K + j] = next_unit();
        }
    }
    for (long i = 0; i < (long)T * H; ++i) {
        float f = next_unit() * 4.0f - 2.0f;
        uint32_t u;
        memcpy(&u, &f, 4);
        x[i] = (uint16_t)(u >> 16);
    }

    /* the oracle */
    int32_t *cnt = malloc(4 * (size_t)E), *off = malloc(4 * (size_t)E);
    int32_t *rrc = malloc(4 * (size_t)R), *rtc = malloc(4 * (size_t)R), *gtc = malloc(4 * (size_t)G);
    uint8_t *map = malloc((size_t)T * R + 1);
    int32_t *slot = malloc(4 * (size_t)TK);
    const int ref_status = oracle_layout(T, K, E, R, G, 1, S, idx, cnt, off, rrc, rtc, gtc, map, slot);
    uint16_t *ref_recv = calloc((size_t)rows * H, 2);
    int32_t *ref_src = malloc(4 * (size_t)rows);
    float *ref_rw = malloc(4 * (size_t)rows);
    oracle_dispatch(T, H, K, rows, x, w, slot, ref_recv, ref_src, ref_rw);
    uint16_t *ref_out = malloc(2 * (size_t)T * H);
    oracle_combine(T, H, K, rows, ref_recv, slot, w, ref_out);

    /* the library: separate calls on the legacy default stream */
    int32_t *d_idx = dev_alloc(4 * (size_t)TK);
    float *d_w = dev_alloc(4 * (size_t)TK);
    uint16_t *d_x = dev_alloc(2 * (size_t)T * H);
    uint16_t *d_recv = dev_alloc(2 * (size_t)rows * H);
    int32_t *d_src = dev_alloc(4 * (size_t)rows);
    float *d_rw = dev_alloc(4 * (size_t)rows);
    uint16_t *d_out = dev_alloc(2 * (size_t)T * H);
    to_dev(d_idx, idx, 4 * (size_t)TK);
    to_dev(d_w, w, 4 * (size_t)TK);
    to_dev(d_x, x, 2 * (size_t)T * H);
    dev_layout a = alloc_layout(&p), b = alloc_layout(&p);
    CHECK_EP(ep_get_layout(&p, d_idx, a.count, a.offset, a.rank_rows, a.rank_tokens, a.group_tokens,
                           a.map, a.slot, NULL, a.ws, a.ws_bytes, NULL));
    CHECK_EP(ep_dispatch(&p, d_x, d_w, a.slot, d_recv, d_src, d_rw, NULL));
    CHECK_EP(ep_combine(&p, d_recv, a.slot, d_w, d_out, NULL));
    int bad = check_layout(&p, &a, ep_read_status(a.ws, NULL), ref_status == 0 ? EP_OK : ref_status,
                           cnt, off, rrc, rtc, gtc, map, slot);

    uint16_t *got = malloc(2 * (size_t)rows * H);
    int32_t *gsrc = malloc(4 * (size_t)rows);
    float *grw = malloc(4 * (size_t)rows);
    to_host(got, d_recv, 2 * (size_t)rows * H);
    to_host(gsrc, d_src, 4 * (size_t)rows);
    to_host(grw, d_rw, 4 * (size_t)rows);
    for (long i = 0; i < TK && !bad; ++i) {
        const int64_t s = slot[i];
        if (s < 0) continue;
        if (memcmp(got + s * H, ref_recv + s * H, 2 * (size_t)H) != 0) bad |= fail("recv_x row", (long)s);
        if (gsrc[s] != ref_src[s]) bad |= fail("recv_src_token", (long)s);
        if (memcmp(&grw[s], &ref_rw[s], 4) != 0) bad |= fail("recv_weight", (long)s);
    }
    uint16_t *gout = malloc(2 * (size_t)T * H);
    double *g64 = malloc(8 * (size_t)T * H), *r64 = malloc(8 * (size_t)T * H);
    to_host(gout, d_out, 2 * (size_t)T * H);
    oracle_bf16_to_double((int64_t)T * H, gout, g64);
    oracle_bf16_to_double((int64_t)T * H, ref_out, r64);
    for (long i = 0; i < (long)T * H && !bad; ++i)
        if (!(fabs(g64[i] - r64[i]) <= 1e-3 + 1e-2 * fabs(r64[i]))) bad |= fail("combine", i);

    /* the one-call layout and dispatch into fresh buffers */
    CHECK_HIP(hipMemset(d_recv, 0, 2 * (size_t)rows * H));
    CHECK_EP(ep_layout_dispatch(&p, d_idx, b.count, b.offset, b.rank_rows, b.rank_tokens, b.group_tokens,
                                b.map, b.slot, NULL, b.ws, b.ws_bytes, d_x, d_w, d_recv, NULL, NULL,
                                NULL));
    bad |= check_layout(&p, &b, ep_read_status(b.ws, NULL), ref_status == 0 ? EP_OK : ref_status,
                        cnt, off, rrc, rtc, gtc, map, slot);
    to_host(got, d_recv, 2 * (size_t)rows * H);
    for (long i = 0; i < TK && !bad; ++i) {
        const int64_t s = slot[i];
        if (s >= 0 && memcmp(got + s * H, ref_recv + s * H, 2 * (size_t)H) != 0)
            bad |= fail("one-call recv_x row", (long)s);
    }

    printf("T=%d H=%d E=%d K=%d R=%d G=%d S=%lld: %s\n", T, H, E, K, R, G, (long long)S,
           bad ? "MISMATCH" : "ok");
    fflush(stdout);
    return bad;
}

int main(void) {
    int bad = 0;
    bad |= run_problem(300, 1024, 64, 6, 8, 2, 1);  /* two layout chunks */
    bad |= run_problem(100, 7168, 256, 8, 8, 1, 2); /* one chunk: one-kernel layout and dispatch */
    return bad;
}
