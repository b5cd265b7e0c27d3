/*
 * oracle.c -- plain, slow fp64 CPU reference for the MXFP4 MoE expert layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the HIP library, and the HIP library never calls it.
 *
 * What it computes, and where each step comes from:
 *
 *  - The pages (bjdmk.com.cn news page, section on the road to 1000 tokens/s;
 *    tilert.ai blog, section on the second leap) say the MoE expert weights
 *    are stored as MXFP4, 4 bits per parameter, and that everything else stays
 *    at higher precision.  MXFP4 is the OCP Microscaling format: blocks of 32
 *    E2M1 elements sharing one E8M0 power-of-two scale.  The element and scale
 *    codes are decoded by their definitions below (exact in fp64).
 *  - The same page says each expert is active on only a small fraction of the
 *    tokens: tokens are routed to k experts.  The pages do not define the
 *    router or the expert FFN; the plainest standard reading is taken:
 *    softmax over the router logits, keep the top k, renormalise; each expert
 *    computes SiLU(gate) * up, then the down projection; the k expert outputs
 *    are summed with the routing weights.
 *  - The prefill workload feeds the GEMMs MXFP8 (E4M3 elements, E8M0 block
 *    scales) activations: x is encoded per token along H and the intermediate
 *    h per assignment along I, by the same block rule as the weights.
 *  - The pages keep the parts of the model other than the MoE experts at FP8
 *    (bjdmk.com.cn news page, co-design section; yifor-blog digest, on
 *    selective FP4 quantisation).  The optional shared expert is read that
 *    way: one SiLU-gated FFN of the routed experts' shape, applied to every
 *    token with weight 1 and added to the routed sum, whose weights are
 *    MXFP8 (E4M3 elements, one E8M0 scale per 32 along the reduction
 *    dimension: the OCP MX block structure of the experts, with 8-bit
 *    elements).
 *
 * Rounding: the only rounding is the encoding step itself (round to nearest,
 * ties to the even code, saturating at the largest finite element).  All
 * products and sums are fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_EINVAL -1
#define OR_EMISSING -2

/* ------------------------------------------------------------------ */
/* element and scale codes                                              */
/* ------------------------------------------------------------------ */

/* E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit, no inf/NaN.
 * Exponent field 0 is subnormal: 0.m * 2^(1-1).  Otherwise 1.m * 2^(e-1). */
double oracle_e2m1_value(int code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* E4M3 (OCP "FN" variant): 1 sign, 4 exponent bits (bias 7), 3 mantissa
 * bits; no infinities; S.1111.111 is NaN; exponent field 0 is subnormal. */
double oracle_e4m3_value(int code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp(m / 8.0, 1 - 7);
    else mag = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* E8M0: an unsigned biased exponent, value 2^(u-127); 0xFF is NaN. */
double oracle_e8m0_value(int code) {
    if (code == 255) return NAN;
    return ldexp(1.0, code - 127);
}

/* ------------------------------------------------------------------ */
/* encoding of one block of 32 values                                   */
/* ------------------------------------------------------------------ */

/* floor(log2(a)) for finite a > 0, read from the binary exponent (frexp),
 * which is exact; log2() can round up just below a power of two. */
static int floor_log2(double a) {
    int e;
    frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
    return e - 1;
}

/* Nearest element of a format to v (|v| already divided by the scale),
 * searching the format's non-negative codes 0..max_code, whose values
 * increase with the code.  Ties go to the even code.  Values beyond the
 * largest finite element saturate to it. */
static int nearest_code(double mag, const double* table, int max_code) {
    if (mag >= table[max_code]) return max_code;
    int lo = 0;
    while (lo + 1 <= max_code && table[lo + 1] <= mag) lo++;
    if (table[lo] == mag) return lo;
    double dlo = mag - table[lo], dhi = table[lo + 1] - mag;
    if (dlo < dhi) return lo;
    if (dhi < dlo) return lo + 1;
    return (lo % 2 == 0) ? lo : lo + 1;
}

/* One MX block: scale X = 2^(floor(log2 amax) - emax_elem), the exponent
 * clamped to [-127, 127] so it fits E8M0; elements = nearest(v / X).
 * amax == 0 gives scale code 0 and all elements +0.  A block holding any
 * non-finite element (NaN or infinity, wherever it sits) gives scale code
 * 0xFF (NaN) and element codes 0. */
static void encode_block(const double* v, int n, int emax_elem, const double* table,
                         int max_code, int sign_bit, uint8_t* codes, uint8_t* scale) {
    double amax = 0.0;
    int finite = 1;
    for (int i = 0; i < n; i++) {
        double a = fabs(v[i]);
        if (!isfinite(a)) finite = 0; /* NaN or infinity anywhere in the block */
        else if (a > amax) amax = a;
    }
    if (!finite) {
        *scale = 255;
        for (int i = 0; i < n; i++) codes[i] = 0;
        return;
    }
    int se;
    if (amax == 0.0) se = -127;
    else se = floor_log2(amax) - emax_elem;
    if (se < -127) se = -127;
    if (se > 127) se = 127;
    *scale = (uint8_t)(se + 127);
    for (int i = 0; i < n; i++) {
        double q = ldexp(v[i], -se); /* exact: division by a power of two */
        int c = nearest_code(fabs(q), table, max_code);
        if (signbit(q)) c |= sign_bit;
        codes[i] = (uint8_t)c;
    }
}

static double E2M1_POS[8];
static double E4M3_POS[127];
static int tables_ready = 0;

static void init_tables(void) {
    if (tables_ready) return;
    for (int c = 0; c < 8; c++) E2M1_POS[c] = oracle_e2m1_value(c);
    for (int c = 0; c < 127; c++) E4M3_POS[c] = oracle_e4m3_value(c);
    tables_ready = 1;
}

/* MXFP4 encoding of a row-major float32 matrix [rows, cols] along cols.
 * packed [rows, cols/2]: element k of a row in byte k/2, even k in the low
 * nibble.  scales [rows, cols/32] E8M0.  cols must be a multiple of 32. */
int oracle_quantize_mxfp4(const float* w, int64_t rows, int64_t cols,
                          uint8_t* packed, uint8_t* scales) {
    if (cols % 32 != 0 || rows < 0) return OR_EINVAL;
    init_tables();
    int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        double v[32];
        uint8_t codes[32];
        for (int64_t b = 0; b < nb; b++) {
            for (int i = 0; i < 32; i++) v[i] = (double)w[r * cols + b * 32 + i];
            encode_block(v, 32, 2, E2M1_POS, 7, 8, codes, &scales[r * nb + b]);
            for (int i = 0; i < 16; i++)
                packed[r * (cols / 2) + b * 16 + i] =
                    (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
        }
    }
    return OR_OK;
}

/* MXFP8 (E4M3) encoding of fp64 values [rows, cols] along cols.
 * codes [rows, cols], scales [rows, cols/32]. */
int oracle_quantize_mxfp8(const double* v, int64_t rows, int64_t cols,
                          uint8_t* codes, uint8_t* scales) {
    if (cols % 32 != 0 || rows < 0) return OR_EINVAL;
    init_tables();
    int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++)
            encode_block(&v[r * cols + b * 32], 32, 8, E4M3_POS, 126, 0x80,
                         &codes[r * cols + b * 32], &scales[r * nb + b]);
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* routing                                                              */
/* ------------------------------------------------------------------ */

typedef struct { float logit; int idx; } cand_t;

/* (logit desc, index asc); logits are compared as the fp32 values given */
static int cand_cmp(const void* a, const void* b) {
    const cand_t* x = (const cand_t*)a;
    const cand_t* y = (const cand_t*)b;
    if (x->logit > y->logit) return -1;
    if (x->logit < y->logit) return 1;
    return (x->idx < y->idx) ? -1 : (x->idx > y->idx);
}

/* Top-k routing.  ids [T,k]: the k experts with the largest logits, ordered
 * by (logit desc, index asc).  w [T,k]: the softmax over all E logits
 * restricted to the chosen k and renormalised, which equals
 * exp(l_j - l_1) / sum_i exp(l_i - l_1) over the chosen i.
 * counts [E], offsets [E+1] (exclusive prefix sum), sorted [T*k]: the flat
 * slots t*k+j grouped by expert, ascending within an expert; pos [T*k] is
 * the inverse (position of slot t*k+j in sorted).  Any output may be NULL. */
int oracle_route(const float* logits, int64_t T, int64_t E, int k,
                 int32_t* ids, double* w, int32_t* counts, int32_t* offsets,
                 int32_t* sorted, int32_t* pos) {
    if (T < 0 || E <= 0 || k < 1 || k > E) return OR_EINVAL;
    int32_t* my_ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * k + 1));
    cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)E);
    if (!my_ids || !c) { free(my_ids); free(c); return OR_EINVAL; }
    for (int64_t t = 0; t < T; t++) {
        for (int64_t e = 0; e < E; e++) { c[e].logit = logits[t * E + e]; c[e].idx = (int)e; }
        qsort(c, (size_t)E, sizeof(cand_t), cand_cmp);
        double l1 = (double)c[0].logit, den = 0.0;
        for (int j = 0; j < k; j++) den += exp((double)c[j].logit - l1);
        for (int j = 0; j < k; j++) {
            my_ids[t * k + j] = c[j].idx;
            if (w) w[t * k + j] = exp((double)c[j].logit - l1) / den;
        }
    }
    if (ids) memcpy(ids, my_ids, sizeof(int32_t) * (size_t)(T * k));
    int64_t n = 0;
    for (int64_t e = 0; e < E; e++) {
        if (offsets) offsets[e] = (int32_t)n;
        int64_t cnt = 0;
        for (int64_t s = 0; s < T * k; s++) {
            if (my_ids[s] == e) {
                if (sorted) sorted[n] = (int32_t)s;
                if (pos) pos[s] = (int32_t)n;
                n++;
                cnt++;
            }
        }
        if (counts) counts[e] = (int32_t)cnt;
    }
    if (offsets) offsets[E] = (int32_t)n;
    free(my_ids);
    free(c);
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* expert FFN and combine                                               */
/* ------------------------------------------------------------------ */

static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* decoded weight W[n][kk] of an MXFP4 matrix with K columns */
static double mxfp4_weight(const uint8_t* packed, const uint8_t* scales, int64_t K,
                           int64_t n, int64_t kk) {
    uint8_t byte = packed[n * (K / 2) + kk / 2];
    int code = (kk % 2 == 0) ? (byte & 15) : (byte >> 4);
    return oracle_e2m1_value(code) * oracle_e8m0_value(scales[n * (K / 32) + kk / 32]);
}

/* y[n] = sum_kk W[n][kk] * v[kk] for n in [0, N) */
static void mxfp4_matvec(const uint8_t* packed, const uint8_t* scales, int64_t N, int64_t K,
                         const double* v, double* y) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        double acc = 0.0;
        for (int64_t kk = 0; kk < K; kk++) acc += mxfp4_weight(packed, scales, K, n, kk) * v[kk];
        y[n] = acc;
    }
}

/* decoded weight W[n][kk] of an MXFP8 matrix with K columns: codes [N, K]
 * E4M3, scales [N, K/32] E8M0 */
static double mxfp8_weight(const uint8_t* codes, const uint8_t* scales, int64_t K, int64_t n,
                           int64_t kk) {
    return oracle_e4m3_value(codes[n * K + kk]) * oracle_e8m0_value(scales[n * (K / 32) + kk / 32]);
}

/* y[n] = sum_kk W[n][kk] * v[kk] for n in [0, N), W in MXFP8 */
static void mxfp8_matvec(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K,
                         const double* v, double* y) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        double acc = 0.0;
        for (int64_t kk = 0; kk < K; kk++) acc += mxfp8_weight(codes, scales, K, n, kk) * v[kk];
        y[n] = acc;
    }
}

/* replace v[0..n) by its MXFP8 (E4M3) encode-then-decode */
static void mxfp8_roundtrip(double* v, int64_t n) {
    uint8_t codes[32], sc;
    init_tables();
    for (int64_t b = 0; b < n / 32; b++) {
        encode_block(&v[b * 32], 32, 8, E4M3_POS, 126, 0x80, codes, &sc);
        for (int i = 0; i < 32; i++)
            v[b * 32 + i] = oracle_e4m3_value(codes[i]) * oracle_e8m0_value(sc);
    }
}

/* The layer output for the tokens listed in `tokens` (n_tok of them):
 *   out[i][:] = sum_j w[t][j] * W_down[e_j] ( silu(W_gate[e_j] x_t) * (W_up[e_j] x_t) )
 *             + Ws_down ( silu(Ws_gate x_t) * (Ws_up x_t) )     (shared expert, if given)
 * with t = tokens[i], (e_j, w[t][j]) from oracle_route over all T tokens.
 * x [T,H] bf16 bits; logits [T,E] fp32.  Expert e's matrices come through
 * the per-expert pointer arrays: gu_packed[e] [2I, H/2], gu_scales[e]
 * [2I, H/32], dn_packed[e] [H, I/2], dn_scales[e] [H, I/32].  Pointers of
 * experts that no listed token uses may be NULL; a NULL that is needed
 * returns OR_EMISSING.  The shared expert is MXFP8: sh_gu [2I, H] E4M3
 * codes (rows 0..I-1 gate, I..2I-1 up), sh_gus [2I, H/32], sh_dn [H, I],
 * sh_dns [H, I/32]; all four NULL = no shared expert.  act_mxfp8 != 0
 * encodes x_t (along H) and every h (along I) to MXFP8 before the products
 * that consume them.  out [n_tok, H] fp64. */
int oracle_forward_ex(const uint16_t* x, const float* logits, int64_t T, int64_t E,
                      int64_t H, int64_t I, int k,
                      const uint8_t* const* gu_packed, const uint8_t* const* gu_scales,
                      const uint8_t* const* dn_packed, const uint8_t* const* dn_scales,
                      const uint8_t* sh_gu, const uint8_t* sh_gus, const uint8_t* sh_dn,
                      const uint8_t* sh_dns, int act_mxfp8, const int32_t* tokens,
                      int64_t n_tok, double* out) {
    if (T < 0 || E <= 0 || H <= 0 || I <= 0 || H % 32 || I % 32 || k < 1 || k > E)
        return OR_EINVAL;
    const int shared = sh_gu || sh_gus || sh_dn || sh_dns;
    if (shared && !(sh_gu && sh_gus && sh_dn && sh_dns)) return OR_EMISSING;
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * k + 1));
    double* w = (double*)malloc(sizeof(double) * (size_t)(T * k + 1));
    double* xt = (double*)malloc(sizeof(double) * (size_t)H);
    double* gu = (double*)malloc(sizeof(double) * (size_t)(2 * I));
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
    double* y = (double*)malloc(sizeof(double) * (size_t)H);
    int rc = OR_OK;
    if (!ids || !w || !xt || !gu || !h || !y) { rc = OR_EINVAL; goto done; }
    rc = oracle_route(logits, T, E, k, ids, w, NULL, NULL, NULL, NULL);
    if (rc) goto done;
    for (int64_t i = 0; i < n_tok; i++) {
        int64_t t = tokens[i];
        if (t < 0 || t >= T) { rc = OR_EINVAL; goto done; }
        for (int64_t kk = 0; kk < H; kk++) xt[kk] = bf16_to_double(x[t * H + kk]);
        if (act_mxfp8) mxfp8_roundtrip(xt, H);
        for (int64_t n = 0; n < H; n++) out[i * H + n] = 0.0;
        for (int j = 0; j < k; j++) {
            int e = ids[t * k + j];
            if (!gu_packed[e] || !gu_scales[e] || !dn_packed[e] || !dn_scales[e]) {
                rc = OR_EMISSING;
                goto done;
            }
            /* gate rows 0..I-1, up rows I..2I-1 of the fused matrix */
            mxfp4_matvec(gu_packed[e], gu_scales[e], 2 * I, H, xt, gu);
            for (int64_t n = 0; n < I; n++) {
                double g = gu[n], u = gu[I + n];
                h[n] = g / (1.0 + exp(-g)) * u; /* SiLU(g) * u */
            }
            if (act_mxfp8) mxfp8_roundtrip(h, I);
            mxfp4_matvec(dn_packed[e], dn_scales[e], H, I, h, y);
            for (int64_t n = 0; n < H; n++) out[i * H + n] += w[t * k + j] * y[n];
        }
        if (shared) { /* the same FFN with MXFP8 weights, weight 1 */
            mxfp8_matvec(sh_gu, sh_gus, 2 * I, H, xt, gu);
            for (int64_t n = 0; n < I; n++) {
                double g = gu[n], u = gu[I + n];
                h[n] = g / (1.0 + exp(-g)) * u;
            }
            if (act_mxfp8) mxfp8_roundtrip(h, I);
            mxfp8_matvec(sh_dn, sh_dns, H, I, h, y);
            for (int64_t n = 0; n < H; n++) out[i * H + n] += y[n];
        }
    }
done:
    free(ids); free(w); free(xt); free(gu); free(h); free(y);
    return rc;
}

/* oracle_forward_ex without a shared expert */
int oracle_forward(const uint16_t* x, const float* logits, int64_t T, int64_t E,
                   int64_t H, int64_t I, int k,
                   const uint8_t* const* gu_packed, const uint8_t* const* gu_scales,
                   const uint8_t* const* dn_packed, const uint8_t* const* dn_scales,
                   int act_mxfp8, const int32_t* tokens, int64_t n_tok, double* out) {
    return oracle_forward_ex(x, logits, T, E, H, I, k, gu_packed, gu_scales, dn_packed,
                             dn_scales, NULL, NULL, NULL, NULL, act_mxfp8, tokens, n_tok, out);
}
