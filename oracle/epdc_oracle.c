/*
 * CPU oracle for MoE expert-parallel dispatch/combine -- TEST INFRASTRUCTURE.
 *
 * Plain, slow, obviously-correct reference for what the HIP path computes.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library; the product path never calls it.  It shares no code,
 * header, table or constant with the HIP library.
 *
 * What is computed, and where the MORI pages say so:
 *  - dispatch(input, weights, scales, indices) -> (output, weights, scales,
 *    indices, recv_count): MORI "Communication APIs" page, MORI-EP section,
 *    EpDispatchCombineOp methods table.  Here every (token, k) pair is one
 *    received row; rows are grouped by expert, experts in ascending order, and
 *    destination rank r owns experts [r*E/R, (r+1)*E/R) -- a contiguous
 *    segment of one receive buffer.  Inside an expert, rows are ordered by the
 *    pair index p = t*K + k (stable by source token).
 *  - recv_count: produced by dispatch itself, zero for ranks that receive
 *    nothing ("AsyncLL v2 SDMA overlap" section of the same page: a peer's
 *    count arrives even when it is zero, and it is computed by the dispatch
 *    kernels rather than reset by the host).
 *  - get_dispatch_src_token_pos(): per received row, the pair index p it came
 *    from (same methods table).
 *  - combine(input, weights, indices) -> (output, weights): gather combine with
 *    BF16 data and FP32 accumulation ("Choosing an EP API and backend" page,
 *    "EP paths" table, HIP row).
 *  - FP8 is OCP E4M3 on gfx950, FP4 is produced by gfx950's pair-at-a-time
 *    scaled convert family ("Choosing an EP API and backend" page, EPv2
 *    restrictions list).  Block sizes: 128 elements per fp32 scale for FP8,
 *    32 elements per E8M0 scale for MXFP4 (OCP Microscaling v1.0).
 *
 *  - the rank-deduplicated dispatch and the standard-MoE conversion: see the
 *    section of that name below.
 *
 * Where the pages are silent this file takes these readings: an expert
 * index outside [0,E) gives its pair no row (slot -1) and is counted; an
 * all-zero FP8 block has scale 0 and codes 0x00; the MXFP4 shared exponent is
 * floor(log2(amax)) - 2 clamped to [-127,127] (-127 for amax == 0); combine
 * accumulates k = 0..K-1 with a separate fp32 multiply and add, starting from
 * +0.0f, then rounds to bf16 to nearest even.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -shared -fPIC (no fast-math).
 * A second build of the same source adds -fopenmp: the loops over tokens
 * marked "omp parallel for" below then run on all host cores.  Each token's
 * iteration writes only its own rows (distinct slots; the routing's cursor
 * loop stays serial), so both builds give identical results.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the token loops use: 1 in the plain build. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- bfloat16: the top 16 bits of an IEEE binary32 ---------------------- */

static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a finite float to the nearest bfloat16, ties to the even pattern. */
static uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t lo = (uint16_t)(u >> 16);          /* truncation: toward zero */
    if ((u & 0xFFFFu) == 0)
        return lo;                               /* exactly representable */
    uint16_t hi = (uint16_t)(lo + 1);           /* next bf16 away from zero */
    double a = fabs((double)f);
    double dlo = a - fabs((double)bf16_to_f32(lo));
    /* IEEE 754 rounding measures the step past the largest finite value as
     * if the exponent range were unbounded: that step is 2^128, not inf. */
    double hi_mag = ((hi & 0x7F80u) == 0x7F80u) ? ldexp(1.0, 128)
                                                 : fabs((double)bf16_to_f32(hi));
    double dhi = hi_mag - a;
    if (dlo < dhi)
        return lo;
    if (dhi < dlo)
        return hi;
    return (lo & 1u) ? hi : lo;
}

/* ---- OCP E4M3 (FN): bias 7, 3 mantissa bits, max 448, no infinities ------ */

/* Nearest E4M3 value to v, ties to even mantissa, magnitudes above 448 give
 * 448.  Works in double, where a/q is exact for the float inputs used. */
uint8_t oracle_e4m3_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    double q;                                    /* spacing in a's binade */
    if (a < ldexp(1.0, -6)) {
        q = ldexp(1.0, -9);                      /* subnormal spacing */
    } else {
        int ex;
        frexp(a, &ex);                           /* a in [2^(ex-1), 2^ex) */
        q = ldexp(1.0, ex - 1 - 3);
    }
    double r = nearbyint(a / q) * q;             /* default mode: ties-to-even */
    if (r > 448.0)
        r = 448.0;
    if (r == 0.0)
        return sign;
    if (r < ldexp(1.0, -6))
        return (uint8_t)(sign | (uint8_t)(r / ldexp(1.0, -9)));
    int ex;
    double m = frexp(r, &ex);                    /* r = m * 2^ex, m in [0.5,1) */
    int e_field = (ex - 1) + 7;
    int mant = (int)((m * 2.0 - 1.0) * 8.0);
    return (uint8_t)(sign | (e_field << 3) | mant);
}

/* ---- OCP E2M1 (FP4): bias 1, 1 mantissa bit: 0,.5,1,1.5,2,3,4,6 --------- */

uint8_t oracle_e2m1_encode(double v)
{
    uint8_t sign = signbit(v) ? 0x8 : 0x0;
    double a = fabs(v);
    double q = (a < 2.0) ? 0.5 : (a < 4.0 ? 1.0 : 2.0);
    double r = nearbyint(a / q) * q;
    if (r > 6.0)
        r = 6.0;
    uint8_t code;
    if (r == 0.0)
        code = 0;
    else if (r < 1.0)
        code = 1;                                /* 0.5, the one subnormal */
    else if (r < 2.0)
        code = (uint8_t)((1 << 1) | (int)((r - 1.0) * 2.0));
    else if (r < 4.0)
        code = (uint8_t)((2 << 1) | (int)((r / 2.0 - 1.0) * 2.0));
    else
        code = (uint8_t)((3 << 1) | (int)((r / 4.0 - 1.0) * 2.0));
    return (uint8_t)(sign | code);
}

/* ---- Routing: histogram, exclusive scan, stable slots -------------------- */

/*
 * indices [T*K] (row-major [T,K]).  Outputs: cnt[E], expert_off[E+1],
 * rank_off[R+1], recv_count[R], slot_of[T*K] (-1 for an invalid index) and
 * src_token_pos[n_valid].  Returns the number of invalid pairs, or -1 on bad
 * arguments.
 */
int oracle_route(int T, int K, int E, int R, const int32_t *indices,
                 int32_t *cnt, int32_t *expert_off, int32_t *rank_off,
                 int32_t *recv_count, int32_t *slot_of, int32_t *src_token_pos)
{
    if (T < 0 || K <= 0 || E <= 0 || R <= 0 || E % R != 0)
        return -1;
    long n = (long)T * K;
    int invalid = 0;

    for (int e = 0; e < E; ++e)
        cnt[e] = 0;
    for (long p = 0; p < n; ++p) {
        int32_t e = indices[p];
        if (e < 0 || e >= E)
            ++invalid;
        else
            ++cnt[e];
    }

    expert_off[0] = 0;
    for (int e = 0; e < E; ++e)
        expert_off[e + 1] = expert_off[e] + cnt[e];

    int per_rank = E / R;
    for (int r = 0; r < R; ++r)
        rank_off[r] = expert_off[r * per_rank];
    rank_off[R] = expert_off[E];
    for (int r = 0; r < R; ++r)
        recv_count[r] = rank_off[r + 1] - rank_off[r];

    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    if (!cursor)
        return -1;
    for (int e = 0; e < E; ++e)
        cursor[e] = expert_off[e];
    for (long p = 0; p < n; ++p) {
        int32_t e = indices[p];
        if (e < 0 || e >= E) {
            slot_of[p] = -1;
            continue;
        }
        int32_t s = cursor[e]++;
        slot_of[p] = s;
        src_token_pos[s] = (int32_t)p;
    }
    free(cursor);
    return invalid;
}

/* ---- Row copy (bf16 or pre-quantized bytes) to the rows of a token's pairs */

/* dst[slot_of[t*K+k]] = src[t] for every valid pair; row_bytes per row. */
void oracle_scatter_rows(int T, int K, const int32_t *slot_of,
                         const uint8_t *src, long row_bytes, uint8_t *dst)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            int32_t s = slot_of[(long)t * K + k];
            if (s < 0)
                continue;
            memcpy(dst + (long)s * row_bytes, src + (long)t * row_bytes,
                   (size_t)row_bytes);
        }
}

/* ---- FP8 E4M3 with one fp32 scale per 128 elements ---------------------- */

/* x [T,H] bf16 bits -> q [T,H] E4M3 codes, scales [T,H/128] fp32. */
int oracle_quant_fp8(int T, int H, const uint16_t *x, uint8_t *q, float *scales)
{
    const int B = 128;
    if (H % B != 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < H / B; ++j) {
            const uint16_t *xb = x + (long)t * H + (long)j * B;
            uint8_t *qb = q + (long)t * H + (long)j * B;
            float amax = 0.0f;
            for (int i = 0; i < B; ++i) {
                float a = fabsf(bf16_to_f32(xb[i]));
                if (a > amax)
                    amax = a;
            }
            float s = 0.0f;
            if (amax == 0.0f) {
                for (int i = 0; i < B; ++i)
                    qb[i] = 0x00;
            } else {
                s = amax / 448.0f;                       /* fp32, RN */
                for (int i = 0; i < B; ++i) {
                    float y = bf16_to_f32(xb[i]) / s;    /* fp32, RN */
                    qb[i] = oracle_e4m3_encode(y);
                }
            }
            scales[(long)t * (H / B) + j] = s;
        }
    return 0;
}

/* ---- MXFP4: E2M1 codes two per byte, one E8M0 scale per 32 ---------------- */

/* x [T,H] bf16 bits -> q [T,H/2] (element 2m in the low nibble of byte m),
 * scales [T,H/32] E8M0 bytes (biased exponent, bias 127). */
int oracle_quant_mxfp4(int T, int H, const uint16_t *x, uint8_t *q, uint8_t *scales)
{
    const int B = 32;
    if (H % B != 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < H / B; ++j) {
            const uint16_t *xb = x + (long)t * H + (long)j * B;
            uint8_t *qb = q + ((long)t * H + (long)j * B) / 2;
            float amax = 0.0f;
            for (int i = 0; i < B; ++i) {
                float a = fabsf(bf16_to_f32(xb[i]));
                if (a > amax)
                    amax = a;
            }
            int e;
            if (amax == 0.0f) {
                e = -127;
            } else {
                int ex;
                frexp((double)amax, &ex);        /* floor(log2(amax)) = ex-1 */
                e = (ex - 1) - 2;                /* emax of E2M1 is 2 */
                if (e < -127)
                    e = -127;
                if (e > 127)
                    e = 127;
            }
            scales[(long)t * (H / B) + j] = (uint8_t)(e + 127);
            for (int i = 0; i < B; i += 2) {
                uint8_t lo = oracle_e2m1_encode(ldexp((double)bf16_to_f32(xb[i]), -e));
                uint8_t hi = oracle_e2m1_encode(ldexp((double)bf16_to_f32(xb[i + 1]), -e));
                qb[i / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    return 0;
}

/* ---- Gather combine: fp32 accumulation, bf16 output ---------------------- */

/*
 * in [N_cap,H] bf16 bits in the received layout, weights [N_cap,K] fp32 in the
 * received layout or NULL (then every weight is 1).  For token t and pair k
 * the weight is weights[slot][k] with slot = slot_of[t*K+k].  Pairs with no
 * slot contribute nothing and report weight 0.  out [T,H] bf16 bits,
 * out_weights [T,K] or NULL.
 */
void oracle_combine(int T, int H, int K, const int32_t *slot_of,
                    const uint16_t *in, const float *weights,
                    uint16_t *out, float *out_weights)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        float *w = (float *)malloc(sizeof(float) * (size_t)K);
        for (int k = 0; k < K; ++k) {
            int32_t s = slot_of[(long)t * K + k];
            w[k] = (s < 0) ? 0.0f : (weights ? weights[(long)s * K + k] : 1.0f);
            if (out_weights)
                out_weights[(long)t * K + k] = w[k];
        }
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                int32_t s = slot_of[(long)t * K + k];
                if (s < 0)
                    continue;
                float prod = w[k] * bf16_to_f32(in[(long)s * H + h]);
                acc = acc + prod;
            }
            out[(long)t * H + h] = f32_to_bf16_rne(acc);
        }
        free(w);
    }
}

/* ---- scatter combine: experts push, the token side reduces -------------- */

/*
 * The pages list a scatter combine next to the gather combine ("Choosing an
 * EP API and backend" page, "EP paths" table, FlyDSL row) without defining
 * it.  Reading: the expert side pushes each received row, multiplied by its
 * weight in fp32, to a staging row of the token it came from (one staging row
 * per pair, so no two pushes meet), and the token side adds its K staging
 * rows in k order.  Step 1: staging[src_token_pos[s]] = w(s) * f32(in[s]) for
 * each received row s < n_rows, w(s) = weights[s][k] with k the pair's k (1
 * when weights is NULL).  Step 2: out[t] = bf16_rne(sum over k = 0..K-1 with
 * slot_of[t*K+k] >= 0 of staging[t*K+k]) from +0.0f; out_weights as in
 * oracle_combine.
 */
void oracle_combine_push(int n_rows, int T, int H, int K, const int32_t *src_token_pos,
                         const int32_t *slot_of, const uint16_t *in, const float *weights,
                         float *staging, uint16_t *out, float *out_weights)
{
    for (int s = 0; s < n_rows; ++s) {
        long p = src_token_pos[s];
        int k = (int)(p % K);
        float w = weights ? weights[(long)s * K + k] : 1.0f;
        for (int h = 0; h < H; ++h)
            staging[p * H + h] = w * bf16_to_f32(in[(long)s * H + h]);
    }
    for (int t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) {
            int32_t s = slot_of[(long)t * K + k];
            if (out_weights)
                out_weights[(long)t * K + k] =
                    s < 0 ? 0.0f : (weights ? weights[(long)s * K + k] : 1.0f);
        }
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                long p = (long)t * K + k;
                if (slot_of[p] < 0)
                    continue;
                acc = acc + staging[p * H + h];
            }
            out[(long)t * H + h] = f32_to_bf16_rne(acc);
        }
    }
}

/* ---- rank-deduplicated dispatch and the standard-MoE conversion --------- */

/*
 * MORI names a "standard-MoE conversion" for its intra-node path ("Choosing
 * an EP API and backend" page, "EP paths" table) and an intra-node kernel
 * type ("Communication APIs" page, kernel types table) without defining
 * either.  Reading used here: the dispatch sends each token once per
 * destination rank that hosts at least one of its valid experts (a "unit"
 * (t, r)); rank r's units are contiguous and ordered by token; the
 * conversion then expands a rank's units into the expert-contiguous rows of
 * the pair dispatch above, and on the way back sums the weighted expert
 * outputs of each unit into one bf16 row that the combine adds up per token.
 *
 * Units: pair p = t*K + k with a valid expert e belongs to rank e / (E/R); the
 * pair with the smallest k among the token's pairs on that rank opens the
 * unit.  unit_cnt[R], unit_off[R+1] (exclusive scan), unit_of[T*K] (the unit
 * row of each pair, -1 for an invalid expert) and unit_src[U] (the token of
 * each unit row).  Returns U, or -1 on bad arguments.
 */
int oracle_route_units(int T, int K, int E, int R, const int32_t *indices,
                       int32_t *unit_cnt, int32_t *unit_off, int32_t *unit_of,
                       int32_t *unit_src)
{
    if (T < 0 || K <= 0 || E <= 0 || R <= 0 || E % R != 0)
        return -1;
    const int per_rank = E / R;
    int32_t *open = (int32_t *)malloc(sizeof(int32_t) * (size_t)R);
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)R);
    if (!open || !cursor) {
        free(open);
        free(cursor);
        return -1;
    }

    /* count: one unit per (token, rank) that any valid pair of the token hits */
    for (int r = 0; r < R; ++r)
        unit_cnt[r] = 0;
    for (int t = 0; t < T; ++t) {
        for (int r = 0; r < R; ++r)
            open[r] = 0;
        for (int k = 0; k < K; ++k) {
            int32_t e = indices[(long)t * K + k];
            if (e < 0 || e >= E)
                continue;
            int r = e / per_rank;
            if (!open[r]) {
                open[r] = 1;
                ++unit_cnt[r];
            }
        }
    }
    unit_off[0] = 0;
    for (int r = 0; r < R; ++r)
        unit_off[r + 1] = unit_off[r] + unit_cnt[r];

    /* place: tokens in ascending order take the next row of each rank they hit */
    for (int r = 0; r < R; ++r)
        cursor[r] = unit_off[r];
    for (int t = 0; t < T; ++t) {
        for (int r = 0; r < R; ++r)
            open[r] = -1;
        for (int k = 0; k < K; ++k) {
            long p = (long)t * K + k;
            int32_t e = indices[p];
            if (e < 0 || e >= E) {
                unit_of[p] = -1;
                continue;
            }
            int r = e / per_rank;
            if (open[r] < 0) {
                open[r] = cursor[r]++;
                unit_src[open[r]] = t;
            }
            unit_of[p] = open[r];
        }
    }
    int U = unit_off[R];
    free(open);
    free(cursor);
    return U;
}

/* dst[u] = src[unit_src[u]] for u < U: each token's row, once per unit. */
void oracle_gather_rows(int U, const int32_t *unit_src, const uint8_t *src,
                        long row_bytes, uint8_t *dst)
{
    for (int u = 0; u < U; ++u)
        memcpy(dst + (long)u * row_bytes, src + (long)unit_src[u] * row_bytes,
               (size_t)row_bytes);
}

/* Standard-MoE conversion, dispatch direction: dst[slot_of[p]] =
 * src[unit_of[p]] for every valid pair (a unit row goes to each of its
 * expert rows). */
void oracle_units_to_experts(long n_pairs, const int32_t *slot_of, const int32_t *unit_of,
                             const uint8_t *src, long row_bytes, uint8_t *dst)
{
    for (long p = 0; p < n_pairs; ++p) {
        if (slot_of[p] < 0 || unit_of[p] < 0)
            continue;
        memcpy(dst + (long)slot_of[p] * row_bytes, src + (long)unit_of[p] * row_bytes,
               (size_t)row_bytes);
    }
}

/*
 * Standard-MoE conversion, combine direction: for unit u of token t,
 * partial[u] = bf16_rne(sum over k = 0..K-1 with unit_of[t*K+k] == u of
 * w(t,k) * in[slot_of[t*K+k]]), fp32 separate multiply and add from +0.0f;
 * w(t,k) = weights[slot][k] with slot = slot_of[t*K+k], or 1 when weights is
 * NULL (the weighting of the gather combine, applied on the expert side).
 */
void oracle_experts_to_units(int U, int H, int K, const int32_t *unit_src,
                             const int32_t *unit_of, const int32_t *slot_of,
                             const uint16_t *in, const float *weights, uint16_t *partial)
{
    for (int u = 0; u < U; ++u) {
        long t = unit_src[u];
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                long p = t * K + k;
                int32_t s = slot_of[p];
                if (unit_of[p] != u || s < 0)
                    continue;
                float w = weights ? weights[(long)s * K + k] : 1.0f;
                float prod = w * bf16_to_f32(in[(long)s * H + h]);
                acc = acc + prod;
            }
            partial[(long)u * H + h] = f32_to_bf16_rne(acc);
        }
    }
}

/*
 * Combine of unit rows: out[t] = bf16_rne(sum of f32(partial[u]) over the
 * token's distinct units in ascending row order, i.e. ascending rank), from
 * +0.0f; +0 for a token with no unit.  out_weights[t][k] =
 * unit_weights[unit_of[t*K+k]][k] (1 when unit_weights is NULL), 0 for a pair
 * with no unit.
 */
void oracle_combine_units(int T, int H, int K, const int32_t *unit_of,
                          const uint16_t *partial, const float *unit_weights,
                          uint16_t *out, float *out_weights)
{
    int32_t *units = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
    for (int t = 0; t < T; ++t) {
        /* the token's distinct units, ascending (insertion sort of <= K ids) */
        int n = 0;
        for (int k = 0; k < K; ++k) {
            long p = (long)t * K + k;
            int32_t u = unit_of[p];
            if (out_weights)
                out_weights[p] = u < 0 ? 0.0f : (unit_weights ? unit_weights[(long)u * K + k] : 1.0f);
            if (u < 0)
                continue;
            int seen = 0;
            for (int i = 0; i < n; ++i)
                seen |= units[i] == u;
            if (seen)
                continue;
            int i = n++;
            while (i > 0 && units[i - 1] > u) {
                units[i] = units[i - 1];
                --i;
            }
            units[i] = u;
        }
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int i = 0; i < n; ++i)
                acc = acc + bf16_to_f32(partial[(long)units[i] * H + h]);
            out[(long)t * H + h] = f32_to_bf16_rne(acc);
        }
    }
    free(units);
}

/* Exposed for the oracle's own pins (bf16 rounding). */
uint16_t oracle_f32_to_bf16(float f) { return f32_to_bf16_rne(f); }

/* Array forms of the scalar encoders, for the oracle's own pins. */
void oracle_e4m3_encode_array(long n, const float *v, uint8_t *out)
{
    for (long i = 0; i < n; ++i)
        out[i] = oracle_e4m3_encode(v[i]);
}

void oracle_e2m1_encode_array(long n, const double *v, uint8_t *out)
{
    for (long i = 0; i < n; ++i)
        out[i] = oracle_e2m1_encode(v[i]);
}

void oracle_f32_to_bf16_array(long n, const float *v, uint16_t *out)
{
    for (long i = 0; i < n; ++i)
        out[i] = f32_to_bf16_rne(v[i]);
}
