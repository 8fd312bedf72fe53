/*
 * CPU oracle for MoE token layout, dispatch and combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg load this library; the HIP product path
 * never calls it, and the two share no code, headers or constants.
 *
 * It is the plain definition of what the hot path computes, written as
 * single-threaded loops in the pages' order, with no blocking or fusion.
 *
 * Pages cited (by title):
 *   [SYM] "DeepEP Symmetric Memory 全面架构分析"
 *         (DeepEP symmetric memory: full architecture analysis)
 *   [V2]  "DeepEP V2 ElasticBuffer 架构深度分析"
 *         (DeepEP V2 ElasticBuffer architecture in depth; it has no section
 *         headings, so its code blocks are cited by what they show)
 *   [V1]  "第 3 章 V1：Buffer 初始化与通信域建立"
 *         (chapter 3, V1 buffer initialisation and communicator set-up)
 *
 * Notation: T tokens, H hidden (bf16 elements per row), E experts, K top-k,
 * R destination ranks, L = E/R local experts per rank, G scale-out groups,
 * A expert alignment, S rows per rank slice.  rank(e) = e / L.
 *
 * Error statuses (the oracle's own numbering):
 *   ORACLE_OK           0
 *   ORACLE_CAPACITY    -3   some rank's aligned rows exceed S
 *   ORACLE_BAD_EXPERT  -4   an id outside [0,E) other than -1; reported in
 *                           preference to a capacity overflow
 * An id of -1 marks an empty top-k entry and is not an error.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_CAPACITY (-3)
#define ORACLE_BAD_EXPERT (-4)

static int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

static int valid_expert(int32_t e, int32_t E) { return e >= 0 && e < E; }

/*
 * Routing layout for one source rank.
 *
 * [SYM] §6.1 lists what dispatch derives from topk_idx: per-scale-up-rank and
 * per-expert prefix sums, the unaligned per-expert receive counts, the
 * expert_alignment, and a destination buffer slot per (token, top-k) entry.
 * [SYM] §7.3 reads back, per scale-up rank, the received token count and, per
 * local expert, a count whose sum is the expanded (token, expert) row count.
 * [V1] §3.2 groups ranks by eight (rdma_rank = rank / 8); with G groups the
 * group of rank r is r / (R/G).
 *
 * Outputs (all caller-allocated):
 *   expert_count[E]      rows routed to each expert (unaligned count)
 *   expert_offset[E]     first row of expert e's segment inside its rank's
 *                        slice: the sum of align_up(count, A) over the lower
 *                        local experts of the same rank
 *   rank_row_count[R]    expanded rows per rank (sum of its experts' counts)
 *   rank_token_count[R]  tokens with at least one entry on the rank
 *   group_token_count[G] tokens with at least one entry in the group (NULL ok)
 *   is_token_in_rank[T*R] 1 if the token has an entry on the rank, else 0
 *   token_slot[T*K]      rank(e)*S + expert_offset[e] + pos, where pos counts
 *                        the earlier entries (token-major, then top-k order)
 *                        that name the same expert; -1 for empty or bad ids
 *                        and for rows at or beyond S inside their slice
 */
int oracle_layout(int32_t T, int32_t K, int32_t E, int32_t R, int32_t G, int32_t A,
                  int64_t S, const int32_t *topk_idx, int32_t *expert_count,
                  int32_t *expert_offset, int32_t *rank_row_count,
                  int32_t *rank_token_count, int32_t *group_token_count,
                  uint8_t *is_token_in_rank, int32_t *token_slot)
{
    const int32_t L = E / R;
    const int32_t ranks_per_group = R / G;
    int bad = 0, over = 0;

    /* expert histogram */
    for (int32_t e = 0; e < E; ++e) expert_count[e] = 0;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < K; ++j) {
            int32_t e = topk_idx[t * K + j];
            if (e == -1) continue;
            if (!valid_expert(e, E)) { bad = 1; continue; }
            expert_count[e] += 1;
        }
    }

    /* per-rank rows and within-slice expert offsets (exclusive scan over the
     * rank's local experts of the aligned counts) */
    for (int32_t r = 0; r < R; ++r) {
        int64_t run = 0, rows = 0;
        for (int32_t l = 0; l < L; ++l) {
            int32_t e = r * L + l;
            expert_offset[e] = (int32_t)run;
            run += align_up(expert_count[e], A);
            rows += expert_count[e];
        }
        rank_row_count[r] = (int32_t)rows;
        if (run > S) over = 1;
    }

    /* token-to-rank map and unique-token counts per rank and per group */
    for (int32_t r = 0; r < R; ++r) rank_token_count[r] = 0;
    if (group_token_count)
        for (int32_t g = 0; g < G; ++g) group_token_count[g] = 0;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t r = 0; r < R; ++r) {
            uint8_t in = 0;
            for (int32_t j = 0; j < K; ++j) {
                int32_t e = topk_idx[t * K + j];
                if (valid_expert(e, E) && e / L == r) in = 1;
            }
            is_token_in_rank[t * R + r] = in;
            rank_token_count[r] += in;
        }
        if (group_token_count) {
            for (int32_t g = 0; g < G; ++g) {
                int in = 0;
                for (int32_t r = g * ranks_per_group; r < (g + 1) * ranks_per_group; ++r)
                    if (is_token_in_rank[t * R + r]) in = 1;
                group_token_count[g] += in;
            }
        }
    }

    /* slots: a counting sort over the (token, top-k) entries in token-major
     * order, so each expert segment holds its rows in ascending source token
     * (then ascending top-k position) */
    int64_t *cursor = (int64_t *)calloc((size_t)(E > 0 ? E : 1), sizeof(int64_t));
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < K; ++j) {
            int32_t e = topk_idx[t * K + j];
            if (!valid_expert(e, E)) { token_slot[t * K + j] = -1; continue; }
            int64_t off = expert_offset[e] + cursor[e];
            cursor[e] += 1;
            token_slot[t * K + j] = off < S ? (int32_t)((int64_t)(e / L) * S + off) : -1;
        }
    }
    free(cursor);

    if (bad) return ORACLE_BAD_EXPERT;
    if (over) return ORACLE_CAPACITY;
    return ORACLE_OK;
}

/*
 * Dispatch: copy each token's hidden row to every destination slot it was
 * given, with its source token index and its top-k weight.
 *
 * [SYM] §6.1 passes x, topk_weights and the destination slot array to the
 * dispatch kernel; [V2] TokenLayout block: a received record holds the hidden
 * row, the top-k weights and the source token index.  [SYM] §9.2: dispatch
 * returns recv_x and the received weights.
 *
 * Slots < 0 or >= num_rows are skipped.  recv_src_token and recv_weight may
 * be NULL (not written).  With topk_weights NULL every weight is 1.
 */
void oracle_dispatch(int32_t T, int32_t H, int32_t K, int64_t num_rows,
                     const uint16_t *x, const float *topk_weights,
                     const int32_t *token_slot, uint16_t *recv_x,
                     int32_t *recv_src_token, float *recv_weight)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < K; ++j) {
            int64_t s = token_slot[t * K + j];
            if (s < 0 || s >= num_rows) continue;
            memcpy(recv_x + s * H, x + t * H, (size_t)H * sizeof(uint16_t));
            if (recv_src_token) recv_src_token[s] = (int32_t)t;
            if (recv_weight) recv_weight[s] = topk_weights ? topk_weights[t * K + j] : 1.0f;
        }
    }
}

/*
 * Hierarchical (two-level) path.  "DeepEP V2 ElasticBuffer 架构深度分析"
 * (dispatch launch block, hybrid_dispatch_impl; logical topology block) and
 * [V1] §3.2 show a dispatch that, when ranks form several scale-out groups,
 * sends each token once to every group it needs and expands it inside the
 * group.  No kernel body is printed; the reading taken here:
 *
 *   group layout: group_slot[t,g] = g*SG + (number of earlier tokens with an
 *     entry in group g) for a token with an entry in group g, else -1 (also
 *     -1 past the group capacity SG, and the status is then ORACLE_CAPACITY);
 *   dispatch: x[t] -> group_buf[group_slot[t,g]], then each entry's row is
 *     copied from its group's row: recv_x[token_slot[t,j]] =
 *     group_buf[group_slot[t, group of token_slot[t,j]]]; the received row
 *     carries source token t and weight w[t,j], or -1 and 0 when its group
 *     row was dropped for capacity (the row itself is then not written);
 *   combine: per (t,g) a partial sum over the entries in group g, folded in
 *     fp32 with fused multiply-add in ascending j and rounded to bf16 in
 *     group_buf (the value that would cross the scale-out link), then
 *     out[t] = bf16(sum over groups of the partials).
 *
 * The partial is rounded to bf16, a quantisation that decides the result, so
 * it is computed in the kernel's precision (fp32 FMA); the final sum over
 * groups is in double.
 */
int oracle_group_layout(int32_t T, int32_t R, int32_t G, int64_t SG,
                        const uint8_t *is_token_in_rank, int32_t *group_slot)
{
    const int32_t rpg = R / G;
    int over = 0;
    for (int32_t g = 0; g < G; ++g) {
        int64_t pos = 0;
        for (int64_t t = 0; t < T; ++t) {
            int in = 0;
            for (int32_t r = g * rpg; r < (g + 1) * rpg; ++r)
                if (is_token_in_rank[t * R + r]) in = 1;
            if (!in) { group_slot[t * G + g] = -1; continue; }
            group_slot[t * G + g] = pos < SG ? (int32_t)(g * SG + pos) : -1;
            pos += 1;
        }
        if (pos > SG) over = 1;
    }
    return over ? ORACLE_CAPACITY : ORACLE_OK;
}

/* group of a valid slot: rank = slot / S, group = rank / (R/G) */
static int32_t slot_group(int64_t s, int64_t S, int32_t R, int32_t G) { return (int32_t)((s / S) / (R / G)); }

void oracle_dispatch_hier(int32_t T, int32_t H, int32_t K, int32_t R, int32_t G, int64_t S,
                          int64_t SG, const uint16_t *x, const float *topk_weights,
                          const int32_t *group_slot, const int32_t *token_slot,
                          uint16_t *group_buf, uint16_t *recv_x, int32_t *recv_src_token,
                          float *recv_weight)
{
    const int64_t num_rows = (int64_t)R * S, group_rows = (int64_t)G * SG;
    for (int64_t t = 0; t < T; ++t)
        for (int32_t g = 0; g < G; ++g) {
            int64_t gs = group_slot[t * G + g];
            if (gs >= 0 && gs < group_rows) memcpy(group_buf + gs * H, x + t * H, (size_t)H * 2);
        }
    for (int64_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < K; ++j) {
            int64_t s = token_slot[t * K + j];
            if (s < 0 || s >= num_rows) continue;
            int64_t gs = group_slot[t * G + slot_group(s, S, R, G)];
            int kept = gs >= 0 && gs < group_rows;
            if (recv_src_token) recv_src_token[s] = kept ? (int32_t)t : -1;
            if (recv_weight)
                recv_weight[s] = !kept ? 0.0f : topk_weights ? topk_weights[t * K + j] : 1.0f;
            if (kept) memcpy(recv_x + s * H, group_buf + gs * H, (size_t)H * 2);
        }
}

static float bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint16_t double_to_bf16(double v);

void oracle_combine_hier(int32_t T, int32_t H, int32_t K, int32_t R, int32_t G, int64_t S,
                         int64_t SG, const uint16_t *y, const int32_t *token_slot,
                         const float *topk_weights, const int32_t *group_slot,
                         uint16_t *group_buf, uint16_t *out)
{
    const int64_t num_rows = (int64_t)R * S, group_rows = (int64_t)G * SG;
    for (int64_t t = 0; t < T; ++t)
        for (int32_t g = 0; g < G; ++g) {
            int64_t gs = group_slot[t * G + g];
            if (gs < 0 || gs >= group_rows) continue;
            for (int64_t h = 0; h < H; ++h) {
                float acc = 0.0f;
                for (int32_t j = 0; j < K; ++j) {
                    int64_t s = token_slot[t * K + j];
                    if (s < 0 || s >= num_rows || slot_group(s, S, R, G) != g) continue;
                    float w = topk_weights ? topk_weights[t * K + j] : 1.0f;
                    acc = fmaf(w, bf16_to_float(y[s * H + h]), acc);
                }
                group_buf[gs * H + h] = double_to_bf16((double)acc);
            }
        }
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int32_t g = 0; g < G; ++g) {
                int64_t gs = group_slot[t * G + g];
                if (gs < 0 || gs >= group_rows) continue;
                acc += (double)bf16_to_float(group_buf[gs * H + h]);
            }
            out[t * H + h] = double_to_bf16(acc);
        }
}

/*
 * Combined top-k weights: the weight carried by each dispatched row, read
 * back into token order ([SYM] §9.2: combine returns combined_topk_weights
 * beside combined_x).  Slots < 0 or >= num_rows give 0.
 */
void oracle_combine_topk_weights(int32_t T, int32_t K, int64_t num_rows,
                                 const float *recv_weight, const int32_t *token_slot,
                                 float *combined_topk_weights)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < K; ++j) {
            int64_t s = token_slot[t * K + j];
            combined_topk_weights[t * K + j] = (s < 0 || s >= num_rows) ? 0.0f : recv_weight[s];
        }
    }
}

/* bf16 bit pattern -> value (exact). */
static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Round a double to the nearest bf16 (8 significant bits, float's exponent
 * range, gradual underflow), ties to even, overflow to infinity.
 *
 * For |v| = m * 2^e with m in [0.5, 1), the bf16 quantum at that magnitude is
 * 2^(e-8), but never below the subnormal quantum 2^-133.  Scaling by a power
 * of two is exact, and rint() rounds half to even in the default mode.
 */
static uint16_t double_to_bf16(double v)
{
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isinf(a)) return sign | 0x7F80;
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);
    int qexp = e - 8;
    if (qexp < -133) qexp = -133;
    double r = ldexp(rint(ldexp(a, -qexp)), qexp);
    if (r >= ldexp(1.0, 128)) return sign | 0x7F80;
    float f = (float)r; /* exact: r is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

/*
 * Combine: gather the K expert-output rows of each token from the slots that
 * dispatch used, weight them by the token's top-k weights and sum.
 *
 * [SYM] §9.2: combine takes the expert outputs, the dispatch handle and
 * topk_weights and returns tokens in their original order.  The sum is taken
 * in double precision over j = 0..K-1 and rounded once to bf16.  Slots < 0 or
 * >= num_rows contribute nothing; topk_weights NULL means unit weights.
 */
void oracle_combine(int32_t T, int32_t H, int32_t K, int64_t num_rows,
                    const uint16_t *y, const int32_t *token_slot,
                    const float *topk_weights, uint16_t *out)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int32_t j = 0; j < K; ++j) {
                int64_t s = token_slot[t * K + j];
                if (s < 0 || s >= num_rows) continue;
                double w = topk_weights ? (double)topk_weights[t * K + j] : 1.0;
                acc += w * bf16_to_double(y[s * H + h]);
            }
            out[t * H + h] = double_to_bf16(acc);
        }
    }
}

/*
 * FP8 (e4m3, the OCP "fn" variant: 4 exponent bits with bias 7, 3 mantissa
 * bits, no infinities, 0x7F/0xFF NaN, largest finite 448) dispatch support.
 *
 * The pages show that dispatch can move FP8 rows with scale factors ([SYM]
 * §6.1: sf, num_sf_packs, sf_token_stride, sf_hidden_stride; §9.2:
 * use_fp8_dispatch; [V2] elastic.py block: a TMA-aligned column-major scale
 * layout with sf_token_stride = 1 and sf_hidden_stride = the aligned token
 * count) but not the quantisation rule.  The reading taken: one fp32 scale
 * per token and block of 128 channels, sf = amax / 448, codes = the nearest
 * e4m3 value (ties to even, magnitudes above 448 saturate) of
 * x * (448 / amax), everything in fp32; an all-zero block gets sf = 0 and
 * zero codes.
 */

/* The e4m3 value of a non-negative code c < 0x7F. */
static float e4m3_magnitude(int c)
{
    int e = c >> 3, m = c & 7;
    if (e == 0) return ldexpf((float)m, -9);          /* subnormal: m * 2^-9 */
    return ldexpf((float)(8 + m), e - 10);             /* (1 + m/8) * 2^(e-7) */
}

/* The 127 finite magnitudes, codes 0..0x7E, filled on first use. */
static float e4m3_table[0x7F];
static int e4m3_table_ready = 0;

static float e4m3_mag(int c)
{
    if (!e4m3_table_ready) {
        for (int k = 0; k < 0x7F; ++k) e4m3_table[k] = e4m3_magnitude(k);
        e4m3_table_ready = 1;
    }
    return e4m3_table[c];
}

/* Nearest e4m3 code, ties to the even code; magnitudes above 448 saturate,
 * NaN maps to 0x7F.  The finite magnitudes increase with the code, so a
 * binary search finds the two neighbours of |v|. */
static uint8_t float_to_e4m3(float v)
{
    if (isnan(v)) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0;
    float a = fabsf(v);
    if (a >= 448.0f) return sign | 0x7E;
    int lo = 0, hi = 0x7E;           /* magnitude(lo) <= a < magnitude(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (e4m3_mag(mid) <= a) lo = mid; else hi = mid;
    }
    float dlo = a - e4m3_mag(lo), dhi = e4m3_mag(hi) - a;
    int best = dlo < dhi ? lo : (dhi < dlo ? hi : ((lo & 1) == 0 ? lo : hi));
    return sign | (uint8_t)best;
}

void oracle_float_to_e4m3(int64_t n, const float *in, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = float_to_e4m3(in[i]);
}

void oracle_e4m3_to_float(int64_t n, const uint8_t *in, float *out)
{
    for (int64_t i = 0; i < n; ++i) {
        int c = in[i] & 0x7F;
        float m = c == 0x7F ? NAN : e4m3_magnitude(c);
        out[i] = (in[i] & 0x80) ? -m : m;
    }
}

/* Per-token, per-128-channel quantisation of bf16 rows [T,H] (H % 128 == 0)
 * into e4m3 codes [T,H] and fp32 scales [T, H/128] (token-major). */
void oracle_quantize_fp8(int32_t T, int32_t H, const uint16_t *x, uint8_t *q, float *sf)
{
    const int32_t nb = H / 128;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t b = 0; b < nb; ++b) {
            const uint16_t *xb = x + t * H + (int64_t)b * 128;
            float amax = 0.0f;
            for (int i = 0; i < 128; ++i) {
                uint32_t u = (uint32_t)xb[i] << 16;
                float f;
                memcpy(&f, &u, sizeof f);
                if (fabsf(f) > amax) amax = fabsf(f);
            }
            const float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
            for (int i = 0; i < 128; ++i) {
                uint32_t u = (uint32_t)xb[i] << 16;
                float f;
                memcpy(&f, &u, sizeof f);
                q[t * H + (int64_t)b * 128 + i] = float_to_e4m3(f * inv);
            }
            sf[t * nb + b] = amax / 448.0f;
        }
    }
}

/* FP8 dispatch: rows of H code bytes go where dispatch sends bf16 rows, and
 * each received row's H/128 scales go to recv_sf[row * sf_token_stride +
 * b * sf_hidden_stride] (token-major: strides (H/128, 1); the TMA-aligned
 * column-major layout: (1, aligned row count)).  Source index and weight as
 * in oracle_dispatch. */
void oracle_dispatch_fp8(int32_t T, int32_t H, int32_t K, int64_t num_rows,
                         const uint8_t *q, const float *sf, const float *topk_weights,
                         const int32_t *token_slot, uint8_t *recv_q, float *recv_sf,
                         int64_t sf_token_stride, int64_t sf_hidden_stride,
                         int32_t *recv_src_token, float *recv_weight)
{
    const int32_t nb = H / 128;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < K; ++j) {
            int64_t s = token_slot[t * K + j];
            if (s < 0 || s >= num_rows) continue;
            memcpy(recv_q + s * H, q + t * H, (size_t)H);
            for (int32_t b = 0; b < nb; ++b)
                recv_sf[s * sf_token_stride + b * sf_hidden_stride] = sf[t * nb + b];
            if (recv_src_token) recv_src_token[s] = (int32_t)t;
            if (recv_weight) recv_weight[s] = topk_weights ? topk_weights[t * K + j] : 1.0f;
        }
    }
}

/* Element-wise conversions, exported so the tests can pin them. */
void oracle_double_to_bf16(int64_t n, const double *in, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = double_to_bf16(in[i]);
}

void oracle_bf16_to_double(int64_t n, const uint16_t *in, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_to_double(in[i]);
}
