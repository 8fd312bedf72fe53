/*
 * Drives every function of the C oracle (oracle/ep_oracle.c) over random
 * small problems -- empty batches, -1 and out-of-range ids, duplicates,
 * alignment, slices too small, groups -- with every array allocated at
 * exactly the size its documentation states.  Built with AddressSanitizer
 * and UndefinedBehaviorSanitizer by tests/test_oracle_sanitized.py, so that
 * any read or write past an array, any signed overflow or any misaligned
 * access in the oracle aborts the run.  Also checks a few invariants of the
 * layout.  Exit status 0 when every case passes.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_layout(int32_t T, int32_t K, int32_t E, int32_t R, int32_t G, int32_t A, int64_t S,
                  const int32_t *topk_idx, int32_t *expert_count, int32_t *expert_offset,
                  int32_t *rank_row_count, int32_t *rank_token_count, int32_t *group_token_count,
                  uint8_t *is_token_in_rank, int32_t *token_slot);
void oracle_dispatch(int32_t T, int32_t H, int32_t K, int64_t num_rows, const uint16_t *x,
                     const float *topk_weights, const int32_t *token_slot, uint16_t *recv_x,
                     int32_t *recv_src_token, float *recv_weight);
void oracle_combine(int32_t T, int32_t H, int32_t K, int64_t num_rows, const uint16_t *y,
                    const int32_t *token_slot, const float *topk_weights, uint16_t *out);
void oracle_combine_topk_weights(int32_t T, int32_t K, int64_t num_rows, const float *recv_weight,
                                 const int32_t *token_slot, float *combined_topk_weights);
void oracle_quantize_fp8(int32_t T, int32_t H, const uint16_t *x, uint8_t *q, float *sf);
void oracle_dispatch_fp8(int32_t T, int32_t H, int32_t K, int64_t num_rows, const uint8_t *q,
                         const float *sf, const float *topk_weights, const int32_t *token_slot,
                         uint8_t *recv_q, float *recv_sf, int64_t sf_token_stride,
                         int64_t sf_hidden_stride, int32_t *recv_src_token, float *recv_weight);
int oracle_group_layout(int32_t T, int32_t R, int32_t G, int64_t SG,
                        const uint8_t *is_token_in_rank, int32_t *group_slot);
void oracle_dispatch_hier(int32_t T, int32_t H, int32_t K, int32_t R, int32_t G, int64_t S,
                          int64_t SG, const uint16_t *x, const float *topk_weights,
                          const int32_t *group_slot, const int32_t *token_slot,
                          uint16_t *group_buf, uint16_t *recv_x, int32_t *recv_src_token,
                          float *recv_weight);
void oracle_combine_hier(int32_t T, int32_t H, int32_t K, int32_t R, int32_t G, int64_t S,
                         int64_t SG, const uint16_t *y, const int32_t *token_slot,
                         const float *topk_weights, const int32_t *group_slot,
                         uint16_t *group_buf, uint16_t *out);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {  /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static int32_t pick(int32_t lo, int32_t hi) { return lo + (int32_t)(next_u32() % (uint32_t)(hi - lo + 1)); }

/* exact-size allocation (at least one byte, so that a zero-length array is
 * still a distinct block whose every access is out of bounds) */
static void *alloc(size_t n, size_t size) {
    void *p = malloc(n * size > 0 ? n * size : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    memset(p, 0x5A, n * size > 0 ? n * size : 1);
    return p;
}

static int fail(const char *what, int it) {
    fprintf(stderr, "case %d: %s\n", it, what);
    return 1;
}

int main(void) {
    const int iters = 400;
    for (int it = 0; it < iters; ++it) {
        const int32_t R = 1 << pick(0, 2), L = pick(1, 4), E = R * L;
        const int32_t G = 1 << pick(0, (R == 1) ? 0 : (R == 2 ? 1 : 2));
        const int32_t K = pick(1, 6), A = pick(1, 3);
        const int32_t T = pick(0, 40), H = 128 * pick(1, 2);
        const int64_t S = pick(1, T * K + E * A + 1);
        const int64_t rows = (int64_t)R * S;
        const int64_t SG = pick(1, T + 1);
        const int32_t nsf = H / 128;

        int32_t *idx = alloc((size_t)T * K, sizeof *idx);
        for (int64_t i = 0; i < (int64_t)T * K; ++i) idx[i] = pick(-1, E + 1);
        uint16_t *x = alloc((size_t)T * H, sizeof *x);
        for (int64_t i = 0; i < (int64_t)T * H; ++i) x[i] = (uint16_t)(next_u32() & 0x7F7F);
        float *w = alloc((size_t)T * K, sizeof *w);
        for (int64_t i = 0; i < (int64_t)T * K; ++i) w[i] = (float)pick(-100, 100) / 64.0f;

        int32_t *cnt = alloc(E, 4), *off = alloc(E, 4), *rrc = alloc(R, 4), *rtc = alloc(R, 4);
        int32_t *gtc = alloc(G, 4), *slot = alloc((size_t)T * K, 4);
        uint8_t *map = alloc((size_t)T * R, 1);
        const int status = oracle_layout(T, K, E, R, G, A, S, idx, cnt, off, rrc, rtc, gtc, map, slot);

        /* invariants: counts add up to the valid ids; slots are distinct
         * rows of the buffer; a bad id is reported */
        int64_t valid = 0, sum = 0, bad = 0;
        for (int64_t i = 0; i < (int64_t)T * K; ++i) {
            valid += idx[i] >= 0 && idx[i] < E;
            bad += idx[i] < -1 || idx[i] >= E;
        }
        for (int32_t e = 0; e < E; ++e) sum += cnt[e];
        if (sum != valid) return fail("expert counts", it);
        if (bad && status == 0) return fail("bad id not reported", it);
        uint8_t *seen = alloc((size_t)rows, 1);
        memset(seen, 0, (size_t)rows);
        for (int64_t i = 0; i < (int64_t)T * K; ++i) {
            const int32_t s = slot[i];
            if (s < 0) continue;
            if (s >= rows || seen[s]) return fail("slot out of range or repeated", it);
            seen[s] = 1;
        }

        uint16_t *recv = alloc((size_t)rows * H, 2);
        int32_t *src = alloc((size_t)rows, 4);
        float *rw = alloc((size_t)rows, 4);
        oracle_dispatch(T, H, K, rows, x, w, slot, recv, src, rw);
        for (int64_t i = 0; i < (int64_t)T * K; ++i)
            if (slot[i] >= 0 && src[slot[i]] != i / K) return fail("source index", it);
        uint16_t *out = alloc((size_t)T * H, 2);
        oracle_combine(T, H, K, rows, recv, slot, w, out);
        oracle_combine(T, H, K, rows, recv, slot, NULL, out);
        float *cw = alloc((size_t)T * K, 4);
        oracle_combine_topk_weights(T, K, rows, rw, slot, cw);

        uint8_t *q = alloc((size_t)T * H, 1);
        float *sf = alloc((size_t)T * nsf, 4);
        oracle_quantize_fp8(T, H, x, q, sf);
        uint8_t *rq = alloc((size_t)rows * H, 1);
        float *rsf = alloc((size_t)rows * nsf, 4);
        oracle_dispatch_fp8(T, H, K, rows, q, sf, w, slot, rq, rsf, nsf, 1, src, rw);
        oracle_dispatch_fp8(T, H, K, rows, q, sf, NULL, slot, rq, rsf, 1, rows, NULL, NULL);

        int32_t *gslot = alloc((size_t)T * G, 4);
        (void)oracle_group_layout(T, R, G, SG, map, gslot);
        uint16_t *gbuf = alloc((size_t)G * SG * H, 2);
        oracle_dispatch_hier(T, H, K, R, G, S, SG, x, w, gslot, slot, gbuf, recv, src, rw);
        oracle_dispatch_hier(T, H, K, R, G, S, SG, x, NULL, gslot, slot, gbuf, recv, NULL, NULL);
        oracle_combine_hier(T, H, K, R, G, S, SG, recv, slot, w, gslot, gbuf, out);

        free(idx); free(x); free(w); free(cnt); free(off); free(rrc); free(rtc); free(gtc);
        free(slot); free(map); free(seen); free(recv); free(src); free(rw); free(out); free(cw);
        free(q); free(sf); free(rq); free(rsf); free(gslot); free(gbuf);
    }
    printf("%d cases passed\n", iters);
    return 0;
}
