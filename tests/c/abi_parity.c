/*
 * A C99 program that uses the library through its C ABI alone (include/epdc.h
 * and the HIP runtime's C API for device memory; no Python, no torch), and
 * checks every output byte for byte against the CPU oracle, which it links
 * directly (test infrastructure: oracle/epdc_oracle.c).
 *
 *   abi_parity --cpu   host-only checks (no GPU call): sizes, argument errors
 *   abi_parity         the host checks, then dispatch + combine on the GPU for
 *                      several configurations, each compared with the oracle
 *
 * Inputs come from a fixed xorshift generator: finite bf16 rows, K distinct
 * experts per token with a few invalid ids, positive weights.  Exit status 0
 * when everything matches.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "epdc.h"

/* The oracle's entry points used here (oracle/epdc_oracle.c). */
int oracle_route(int T, int K, int E, int R, const int32_t *indices, int32_t *cnt,
                 int32_t *expert_off, int32_t *rank_off, int32_t *recv_count, int32_t *slot_of,
                 int32_t *src_token_pos);
void oracle_scatter_rows(int T, int K, const int32_t *slot_of, const uint8_t *src,
                         long row_bytes, uint8_t *dst);
int oracle_quant_fp8(int T, int H, const uint16_t *x, uint8_t *q, float *scales);
void oracle_combine(int T, int H, int K, const int32_t *slot_of, const uint16_t *in,
                    const float *weights, uint16_t *out, float *out_weights);

static uint64_t g_rng = 0x9E3779B97F4A7C15ull;

static uint32_t rnd(void)
{
    g_rng ^= g_rng << 13;
    g_rng ^= g_rng >> 7;
    g_rng ^= g_rng << 17;
    return (uint32_t)(g_rng >> 16);
}

/* A finite bf16 value in about [2^-7, 2^8) of either sign. */
static uint16_t rnd_bf16(void)
{
    const uint32_t r = rnd();
    const uint16_t sign = (uint16_t)((r & 1u) << 15);
    const uint16_t exp = (uint16_t)(120 + (r >> 1) % 15);
    const uint16_t man = (uint16_t)((r >> 8) & 0x7F);
    return (uint16_t)(sign | (exp << 7) | man);
}

#define FAIL(...)                                                                      \
    do {                                                                               \
        fprintf(stderr, __VA_ARGS__);                                                  \
        fprintf(stderr, "\n");                                                         \
        return 1;                                                                      \
    } while (0)

#define HIP(x)                                                                         \
    do {                                                                               \
        hipError_t e_ = (x);                                                           \
        if (e_ != hipSuccess)                                                          \
            FAIL("%s: %s", #x, hipGetErrorString(e_));                                 \
    } while (0)

#define EPDC(x)                                                                        \
    do {                                                                               \
        epdc_status s_ = (x);                                                          \
        if (s_ != EPDC_SUCCESS)                                                        \
            FAIL("%s: status %d (%s)", #x, (int)s_, epdc_last_error());                \
    } while (0)

static int host_checks(void)
{
    epdc_config c;
    memset(&c, 0, sizeof c);
    c.max_tokens = 4096;
    c.hidden = 7168;
    c.topk = 8;
    c.num_experts = 256;
    c.num_ranks = 8;
    c.input_kind = EPDC_IN_BF16;
    size_t ws = 0, payload = 0, scale = 0;
    EPDC(epdc_workspace_bytes(&c, &ws));
    if (ws == 0)
        FAIL("workspace bytes are 0");
    EPDC(epdc_row_bytes(&c, &payload, &scale));
    if (payload != 2 * 7168 || scale != 0)
        FAIL("bf16 row bytes %zu / %zu", payload, scale);
    c.quant = EPDC_QUANT_FP8_E4M3_B128;
    EPDC(epdc_row_bytes(&c, &payload, &scale));
    if (payload != 7168 || scale != 4 * 56)
        FAIL("FP8 row bytes %zu / %zu", payload, scale);
    c.quant = EPDC_QUANT_MXFP4_B32;
    EPDC(epdc_row_bytes(&c, &payload, &scale));
    if (payload != 3584 || scale != 224)
        FAIL("MXFP4 row bytes %zu / %zu", payload, scale);
    /* argument errors come back as statuses with a message */
    c.hidden = 7;
    if (epdc_workspace_bytes(&c, &ws) != EPDC_ERR_INVALID_ARGS || !*epdc_last_error())
        FAIL("hidden 7 accepted");
    if (epdc_create(NULL, NULL, 0, NULL) != EPDC_ERR_INVALID_ARGS)
        FAIL("NULL create accepted");
    if (epdc_combine(NULL, NULL, NULL, NULL, NULL, NULL, NULL) != EPDC_ERR_INVALID_ARGS)
        FAIL("NULL combine accepted");
    if (!epdc_kernel_name(EPDC_KERNEL_COMBINE) ||
        strcmp(epdc_kernel_name(EPDC_KERNEL_COMBINE), "k_combine") != 0 ||
        epdc_kernel_name(EPDC_NUM_KERNELS) != NULL)
        FAIL("kernel names");
    printf("host checks ok\n");
    return 0;
}

typedef struct {
    const char *name;
    int T, H, K, E, R, quant, invalid, independent;
} Case;

static int run_case(const Case *c)
{
    const int T = c->T, H = c->H, K = c->K, E = c->E, R = c->R;
    const long N = (long)T * K;
    printf("case %s: T=%d H=%d K=%d E=%d R=%d\n", c->name, T, H, K, E, R);
    fflush(stdout);

    /* host inputs */
    uint16_t *x = malloc(sizeof(uint16_t) * (size_t)T * H);
    int32_t *idx = malloc(sizeof(int32_t) * (size_t)N);
    float *w = malloc(sizeof(float) * (size_t)N);
    uint16_t *cin = c->independent ? malloc(sizeof(uint16_t) * (size_t)N * H) : NULL;
    if (!x || !idx || !w || (c->independent && !cin))
        FAIL("host allocation");
    for (long i = 0; i < (long)T * H; ++i)
        x[i] = rnd_bf16();
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            int e, dup;
            do {
                e = (int)(rnd() % (uint32_t)E);
                dup = 0;
                for (int j = 0; j < k; ++j)
                    dup |= idx[(long)t * K + j] == e;
            } while (dup);
            idx[(long)t * K + k] = e;
            w[(long)t * K + k] = (float)(rnd() % 1000 + 1) / 1000.0f;
        }
    for (int i = 0; i < c->invalid; ++i)
        idx[(long)(rnd() % (uint32_t)T) * K + i % K] = (i & 1) ? -1 - i : E + i;
    if (cin)
        for (long i = 0; i < N * H; ++i)
            cin[i] = rnd_bf16();

    epdc_config cfg;
    memset(&cfg, 0, sizeof cfg);
    cfg.max_tokens = T;
    cfg.hidden = H;
    cfg.topk = K;
    cfg.num_experts = E;
    cfg.num_ranks = R;
    cfg.input_kind = EPDC_IN_BF16;
    cfg.quant = c->quant;
    size_t ws_bytes = 0, payload = 0, scale = 0;
    EPDC(epdc_workspace_bytes(&cfg, &ws_bytes));
    EPDC(epdc_row_bytes(&cfg, &payload, &scale));

    /* device buffers */
    void *d_x, *d_w, *d_idx, *d_ws, *d_out, *d_outw, *d_outs, *d_outi, *d_recv, *d_y, *d_yw;
    void *d_cin = NULL;
    HIP(hipMalloc(&d_x, sizeof(uint16_t) * (size_t)T * H));
    HIP(hipMalloc(&d_w, sizeof(float) * (size_t)N));
    HIP(hipMalloc(&d_idx, sizeof(int32_t) * (size_t)N));
    HIP(hipMalloc(&d_ws, ws_bytes));
    HIP(hipMalloc(&d_out, payload * (size_t)N));
    HIP(hipMalloc(&d_outw, sizeof(float) * (size_t)N * K));
    HIP(hipMalloc(&d_outs, (scale ? scale : 4) * (size_t)N));
    HIP(hipMalloc(&d_outi, sizeof(int32_t) * (size_t)N * K));
    HIP(hipMalloc(&d_recv, sizeof(int32_t) * (size_t)R));
    HIP(hipMalloc(&d_y, sizeof(uint16_t) * (size_t)T * H));
    HIP(hipMalloc(&d_yw, sizeof(float) * (size_t)N));
    HIP(hipMemcpy(d_x, x, sizeof(uint16_t) * (size_t)T * H, hipMemcpyHostToDevice));
    HIP(hipMemcpy(d_w, w, sizeof(float) * (size_t)N, hipMemcpyHostToDevice));
    HIP(hipMemcpy(d_idx, idx, sizeof(int32_t) * (size_t)N, hipMemcpyHostToDevice));
    if (cin) {
        HIP(hipMalloc(&d_cin, sizeof(uint16_t) * (size_t)N * H));
        HIP(hipMemcpy(d_cin, cin, sizeof(uint16_t) * (size_t)N * H, hipMemcpyHostToDevice));
    }

    epdc_op *op = NULL;
    EPDC(epdc_create(&cfg, d_ws, ws_bytes, &op));
    if (!c->independent)
        EPDC(epdc_set_combine_hint(op, EPDC_COMBINE_INPUT_RECENT));
    EPDC(epdc_dispatch(op, NULL, T, d_x, (const float *)d_w, NULL, (const int32_t *)d_idx,
                       d_out, (float *)d_outw, c->quant ? d_outs : NULL, (int32_t *)d_outi,
                       (int32_t *)d_recv));
    EPDC(epdc_combine(op, NULL, c->independent ? d_cin : d_out, (const float *)d_outw,
                      (const int32_t *)d_outi, d_y, (float *)d_yw));
    HIP(hipDeviceSynchronize());

    /* results */
    const int32_t *d_eo, *d_ro, *d_so, *d_sp;
    int32_t count = 0;
    EPDC(epdc_get_routing(op, &d_eo, &d_ro, &d_so));
    EPDC(epdc_get_dispatch_src_token_pos(op, &d_sp, &count));
    if (count != N)
        FAIL("src_token_pos count %d, expected %ld", count, N);
    int32_t *g_recv = malloc(sizeof(int32_t) * (size_t)R), *g_eo = malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *g_ro = malloc(sizeof(int32_t) * (size_t)(R + 1)), *g_so = malloc(sizeof(int32_t) * (size_t)N);
    int32_t *g_sp = malloc(sizeof(int32_t) * (size_t)N);
    uint8_t *g_out = malloc(payload * (size_t)N), *g_outs = malloc((scale ? scale : 4) * (size_t)N);
    float *g_outw = malloc(sizeof(float) * (size_t)N * K), *g_yw = malloc(sizeof(float) * (size_t)N);
    int32_t *g_outi = malloc(sizeof(int32_t) * (size_t)N * K);
    uint16_t *g_y = malloc(sizeof(uint16_t) * (size_t)T * H);
    HIP(hipMemcpy(g_recv, d_recv, sizeof(int32_t) * (size_t)R, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(g_eo, d_eo, sizeof(int32_t) * (size_t)(E + 1), hipMemcpyDeviceToHost));
    HIP(hipMemcpy(g_ro, d_ro, sizeof(int32_t) * (size_t)(R + 1), hipMemcpyDeviceToHost));
    HIP(hipMemcpy(g_so, d_so, sizeof(int32_t) * (size_t)N, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(g_sp, d_sp, sizeof(int32_t) * (size_t)N, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(g_out, d_out, payload * (size_t)N, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(g_outs, d_outs, (scale ? scale : 4) * (size_t)N, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(g_outw, d_outw, sizeof(float) * (size_t)N * K, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(g_outi, d_outi, sizeof(int32_t) * (size_t)N * K, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(g_y, d_y, sizeof(uint16_t) * (size_t)T * H, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(g_yw, d_yw, sizeof(float) * (size_t)N, hipMemcpyDeviceToHost));
    int32_t flag = -1;
    EPDC(epdc_get_device_error(op, NULL, &flag));

    /* the oracle on the same inputs */
    int32_t *cnt = malloc(sizeof(int32_t) * (size_t)E), *eo = malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *ro = malloc(sizeof(int32_t) * (size_t)(R + 1)), *recv = malloc(sizeof(int32_t) * (size_t)R);
    int32_t *so = malloc(sizeof(int32_t) * (size_t)N), *sp = malloc(sizeof(int32_t) * (size_t)N);
    const int invalid = oracle_route(T, K, E, R, idx, cnt, eo, ro, recv, so, sp);
    if (invalid < 0)
        FAIL("oracle_route refused the arguments");
    const long nv = eo[E];
    uint8_t *out = calloc((size_t)nv ? (size_t)nv : 1, payload);
    uint8_t *outs = calloc((size_t)nv ? (size_t)nv : 1, scale ? scale : 4);
    if (c->quant == EPDC_QUANT_FP8_E4M3_B128) {
        uint8_t *q = malloc((size_t)T * H);
        float *sc = malloc(sizeof(float) * (size_t)T * (H / 128));
        if (oracle_quant_fp8(T, H, x, q, sc) != 0)
            FAIL("oracle_quant_fp8 failed");
        oracle_scatter_rows(T, K, so, q, H, out);
        oracle_scatter_rows(T, K, so, (const uint8_t *)sc, (long)scale, outs);
        free(q);
        free(sc);
    } else {
        oracle_scatter_rows(T, K, so, (const uint8_t *)x, 2L * H, out);
    }
    /* the carried rows: slot s of pair p = t*K+k holds token t's weights and ids */
    float *outw = calloc((size_t)nv ? (size_t)nv * K : 1, sizeof(float));
    int32_t *outi = calloc((size_t)nv ? (size_t)nv * K : 1, sizeof(int32_t));
    for (long p = 0; p < N; ++p)
        if (so[p] >= 0) {
            memcpy(outw + (long)so[p] * K, w + (p / K) * K, sizeof(float) * (size_t)K);
            memcpy(outi + (long)so[p] * K, idx + (p / K) * K, sizeof(int32_t) * (size_t)K);
        }
    uint16_t *y = malloc(sizeof(uint16_t) * (size_t)T * H);
    float *yw = malloc(sizeof(float) * (size_t)N);
    oracle_combine(T, H, K, so, c->independent ? cin : (const uint16_t *)out, outw, y, yw);

    if (memcmp(g_recv, recv, sizeof(int32_t) * (size_t)R))
        FAIL("%s: recv_count differs", c->name);
    if (memcmp(g_eo, eo, sizeof(int32_t) * (size_t)(E + 1)))
        FAIL("%s: expert_off differs", c->name);
    if (memcmp(g_ro, ro, sizeof(int32_t) * (size_t)(R + 1)))
        FAIL("%s: rank_off differs", c->name);
    if (memcmp(g_so, so, sizeof(int32_t) * (size_t)N))
        FAIL("%s: slot_of differs", c->name);
    if (memcmp(g_sp, sp, sizeof(int32_t) * (size_t)nv))
        FAIL("%s: src_token_pos differs", c->name);
    if (memcmp(g_out, out, payload * (size_t)nv))
        FAIL("%s: payload rows differ", c->name);
    if (scale && memcmp(g_outs, outs, scale * (size_t)nv))
        FAIL("%s: scale rows differ", c->name);
    if (memcmp(g_outw, outw, sizeof(float) * (size_t)nv * K))
        FAIL("%s: carried weights differ", c->name);
    if (memcmp(g_outi, outi, sizeof(int32_t) * (size_t)nv * K))
        FAIL("%s: carried indices differ", c->name);
    if (memcmp(g_y, y, sizeof(uint16_t) * (size_t)T * H))
        FAIL("%s: combine output differs", c->name);
    if (memcmp(g_yw, yw, sizeof(float) * (size_t)N))
        FAIL("%s: combine weights differ", c->name);
    if (flag != (invalid > 0 ? 1 : 0))
        FAIL("%s: device error flag %d with %d invalid ids", c->name, flag, invalid);
    printf("case %s ok: %ld received rows, %d invalid ids, bit-exact\n", c->name, nv, invalid);
    fflush(stdout);

    EPDC(epdc_destroy(op));
    void *dev[] = {d_x, d_w, d_idx, d_ws, d_out, d_outw, d_outs, d_outi, d_recv, d_y, d_yw, d_cin};
    for (size_t i = 0; i < sizeof dev / sizeof dev[0]; ++i)
        if (dev[i])
            HIP(hipFree(dev[i]));
    void *host[] = {x, idx, w, cin, g_recv, g_eo, g_ro, g_so, g_sp, g_out, g_outs, g_outw, g_yw,
                    g_outi, g_y, cnt, eo, ro, recv, so, sp, out, outs, outw, outi, y, yw};
    for (size_t i = 0; i < sizeof host / sizeof host[0]; ++i)
        free(host[i]);
    return 0;
}

int main(int argc, char **argv)
{
    if (host_checks())
        return 1;
    if (argc > 1 && strcmp(argv[1], "--cpu") == 0)
        return 0;
    const Case cases[] = {
        /* one routing tile: the single-launch dispatch */
        {"decode_bf16", 128, 7168, 8, 256, 8, EPDC_QUANT_NONE, 0, 0},
        /* several tiles, the scan in the scatter blocks; staged cold combine */
        {"bf16_tiles", 1000, 7168, 8, 256, 8, EPDC_QUANT_NONE, 5, 1},
        /* FP8: the last rank block scans the table */
        {"fp8_tiles", 3000, 2048, 8, 512, 8, EPDC_QUANT_FP8_E4M3_B128, 3, 1},
        /* generic K and a power-of-two row */
        {"k3", 700, 512, 3, 12, 3, EPDC_QUANT_NONE, 2, 0},
    };
    for (size_t i = 0; i < sizeof cases / sizeof cases[0]; ++i)
        if (run_case(&cases[i]))
            return 1;
    printf("all cases bit-exact\n");
    return 0;
}
