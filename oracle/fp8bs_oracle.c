/*
 * fp8bs_oracle.c -- plain CPU oracle for the FP8 block-scaled linear-layer path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or constant generator with the HIP library: everything here is written
 * from the definitions below, in the slowest obvious way.
 *
 * What it computes.  The Puro-2B technical report (lkr-homepage blog, section 2
 * "FP8") runs the matmuls of the main linear layers in FP8 with DeepSeek-V3's
 * fine-grained block quantization and keeps numerically sensitive work in
 * BF16/FP32.  The concrete reading implemented here:
 *   - FP8 format: OCP E4M3FN (bias 7, 3 mantissa bits, no infinities,
 *     NaN = S.1111.111, largest finite 448).
 *   - A tile is 1x128 consecutive elements along the contraction axis for
 *     activations and gradients, 128x128 for weights.  Each tile has one FP32
 *     scale: a = max(amax, 2^-100), s = a/448, inv = 448/a (two correctly
 *     rounded FP32 divisions), code = E4M3_RNE(clamp(x*inv, -448, 448)).
 *   - The GEMM sums, per output element and per 128-wide contraction block kb,
 *     the exact integer product sum of the codes (in units of 2^-9 each), turns
 *     it into FP32 (one rounding), multiplies by the FP32 product of the two
 *     operands' scales, and adds it to an FP32 accumulator, kb ascending.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC.
 * Every output element is produced by one thread in a fixed order, so results
 * do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORACLE_OK 0
#define ORACLE_ERR_SHAPE (-1)
#define ORACLE_ERR_NONFINITE (-2)
#define ORACLE_ERR_ARG (-3)
#define ORACLE_ERR_NOMEM (-4)

#define TILE 128
#define E4M3_MAX 448.0f
#define AMAX_FLOOR 0x1p-100f

int oracle_version(void) { return 1; }

/* ------------------------------------------------------------------------- */
/* E4M3FN decode (OCP 8-bit floating point specification, E4M3 column).      */
/* sign = bit 7, E = bits 6..3, m = bits 2..0.                                 */
/* E == 0: (-1)^sign * m * 2^-9 (subnormal); otherwise                         */
/* (-1)^sign * (1 + m/8) * 2^(E-7).  S.1111.111 is NaN.                        */
/* ------------------------------------------------------------------------- */
double oracle_e4m3_value(uint8_t c) {
    int sign = c >> 7, E = (c >> 3) & 15, m = c & 7;
    if (E == 15 && m == 7) return NAN;
    double mag = (E == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, E - 7);
    return sign ? -mag : mag;
}

/* Same value as an integer count of 2^-9 units (exact; |result| <= 229376).
 * Returns INT32_MIN for the two NaN codes. */
int32_t oracle_e4m3_units(uint8_t c) {
    double v = oracle_e4m3_value(c);
    if (isnan(v)) return INT32_MIN;
    return (int32_t)ldexp(v, 9); /* exact: every finite E4M3 value is a multiple of 2^-9 */
}

/* Sorted magnitudes of the non-negative finite codes 0x00..0x7E. */
static double g_mag[127];
static int32_t g_units[256];

__attribute__((constructor)) static void oracle_build_tables(void) {
    for (int c = 0; c < 127; ++c) g_mag[c] = oracle_e4m3_value((uint8_t)c);
    for (int c = 0; c < 256; ++c) g_units[c] = oracle_e4m3_units((uint8_t)c);
}

/* E4M3 encode with round-to-nearest, ties to even, by searching the table of
 * representable magnitudes.  Finite magnitudes above 448 saturate to 448 (the
 * quantizer clamps before it encodes, so this never decides a result there).
 * The sign bit is copied from v, so -0.0 and negative values that round to
 * zero encode as 0x80.  NaN encodes as 0x7F. */
uint8_t oracle_e4m3_encode(float v) {
    if (isnan(v)) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= g_mag[126]) return sign | 126;
    /* largest code lo with g_mag[lo] <= a (binary search over 127 entries) */
    int lo = 0, hi = 126;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (g_mag[mid] <= a) lo = mid; else hi = mid;
    }
    if (g_mag[lo] == a) return sign | (uint8_t)lo;
    /* a lies strictly between g_mag[lo] and g_mag[lo+1]; the midpoint of two
     * adjacent E4M3 magnitudes is exact in double. */
    double midpoint = 0.5 * (g_mag[lo] + g_mag[lo + 1]);
    int code;
    if (a < midpoint) code = lo;
    else if (a > midpoint) code = lo + 1;
    else code = (lo % 2 == 0) ? lo : lo + 1; /* tie: the even code */
    return sign | (uint8_t)code;
}

void oracle_e4m3_encode_array(const float* v, int64_t n, uint8_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(v[i]);
}

/* BF16 bits -> FP32 is exact: the BF16 pattern is the top half of the FP32 one. */
static float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* FP32 -> BF16 with round to nearest, ties to even (NaN stays NaN). */
uint16_t oracle_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lower = u & 0xFFFFu;
    uint32_t upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
    return (uint16_t)upper;
}

void oracle_f32_to_bf16_array(const float* v, int64_t n, uint16_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(v[i]);
}

/* ------------------------------------------------------------------------- */
/* One tile: amax, scale, codes.  vals holds the tile's n decoded elements.    */
/* Returns ORACLE_ERR_NONFINITE if any element is Inf or NaN.                  */
/* ------------------------------------------------------------------------- */
static int quantize_tile(const float* vals, int64_t n, uint8_t* codes, float* scale) {
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        if (!isfinite(vals[i])) return ORACLE_ERR_NONFINITE;
        float m = fabsf(vals[i]);
        if (m > amax) amax = m;
    }
    float a = amax > AMAX_FLOOR ? amax : AMAX_FLOOR;
    float s = a / E4M3_MAX;
    float inv = E4M3_MAX / a;
    for (int64_t i = 0; i < n; ++i) {
        float p = vals[i] * inv;
        if (p > E4M3_MAX) p = E4M3_MAX;
        if (p < -E4M3_MAX) p = -E4M3_MAX;
        codes[i] = oracle_e4m3_encode(p);
    }
    *scale = s;
    return ORACLE_OK;
}

/* Threads: 0 means every core OpenMP sees. */
static void set_threads(int threads) {
    if (threads > 0) omp_set_num_threads(threads);
    else omp_set_num_threads(omp_get_num_procs());
}

/* Row-tile quantizer: x bf16 [M,K] -> q [M,K], s [M, K/128].
 * s[r][j] covers x[r][128j .. 128j+127]. */
int oracle_quantize_rowtile(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s,
                            int threads) {
    if (M < 0 || K < 0 || K % TILE) return ORACLE_ERR_SHAPE;
    int64_t kt = K / TILE, ntiles = M * kt;
    int status = ORACLE_OK;
    set_threads(threads);
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < ntiles; ++t) {
        int64_t r = t / kt, j = t % kt;
        float vals[TILE];
        uint8_t codes[TILE];
        for (int c = 0; c < TILE; ++c) vals[c] = bf16_to_f32(x[r * K + j * TILE + c]);
        float sc;
        if (quantize_tile(vals, TILE, codes, &sc) != ORACLE_OK) {
            #pragma omp atomic write
            status = ORACLE_ERR_NONFINITE;
            continue;
        }
        memcpy(q + r * K + j * TILE, codes, TILE);
        s[r * kt + j] = sc;
    }
    return status;
}

/* Block quantizer: w bf16 [N,K] -> q [N,K], optional q_t [K,N] (q_t[k][n] = q[n][k]),
 * s [N/128, K/128].  s[i][j] covers rows 128i.. and columns 128j.. . */
int oracle_quantize_block(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, uint8_t* q_t,
                          float* s, int threads) {
    if (N < 0 || K < 0 || N % TILE || K % TILE) return ORACLE_ERR_SHAPE;
    int64_t nb = N / TILE, kbn = K / TILE, nblocks = nb * kbn;
    int status = ORACLE_OK;
    set_threads(threads);
    #pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblocks; ++b) {
        int64_t bi = b / kbn, bj = b % kbn;
        float* vals = (float*)malloc(sizeof(float) * TILE * TILE);
        uint8_t* codes = (uint8_t*)malloc(TILE * TILE);
        if (!vals || !codes) {
            free(vals); free(codes);
            #pragma omp atomic write
            status = ORACLE_ERR_NOMEM;
            continue;
        }
        for (int r = 0; r < TILE; ++r)
            for (int c = 0; c < TILE; ++c)
                vals[r * TILE + c] = bf16_to_f32(w[(bi * TILE + r) * K + bj * TILE + c]);
        float sc;
        if (quantize_tile(vals, TILE * TILE, codes, &sc) != ORACLE_OK) {
            #pragma omp atomic write
            status = ORACLE_ERR_NONFINITE;
        } else {
            for (int r = 0; r < TILE; ++r)
                for (int c = 0; c < TILE; ++c) {
                    int64_t n = bi * TILE + r, k = bj * TILE + c;
                    q[n * K + k] = codes[r * TILE + c];
                    if (q_t) q_t[k * N + n] = codes[r * TILE + c];
                }
            s[bi * kbn + bj] = sc;
        }
        free(vals);
        free(codes);
    }
    return status;
}

/* Transposed (token-axis) quantizer: x bf16 [M,C] -> qt [C,M], st [C, M/128].
 * The tile for (c, mb) is x[128mb .. 128mb+127][c]: 128 consecutive tokens of
 * one channel, i.e. the row-tile quantizer applied to x transposed. */
int oracle_quantize_transposed(const uint16_t* x, int64_t M, int64_t C, uint8_t* qt, float* st,
                               int threads) {
    if (M < 0 || C < 0 || M % TILE) return ORACLE_ERR_SHAPE;
    int64_t mbn = M / TILE, ntiles = C * mbn;
    int status = ORACLE_OK;
    set_threads(threads);
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < ntiles; ++t) {
        int64_t c = t / mbn, mb = t % mbn;
        float vals[TILE];
        uint8_t codes[TILE];
        for (int i = 0; i < TILE; ++i) vals[i] = bf16_to_f32(x[(mb * TILE + i) * C + c]);
        float sc;
        if (quantize_tile(vals, TILE, codes, &sc) != ORACLE_OK) {
            #pragma omp atomic write
            status = ORACLE_ERR_NONFINITE;
            continue;
        }
        memcpy(qt + c * M + mb * TILE, codes, TILE);
        st[c * mbn + mb] = sc;
    }
    return status;
}

/* ------------------------------------------------------------------------- */
/* Block-scaled GEMM, "TN" form: out[i][j] = sum over contraction blocks kb of  */
/*   sA(i,kb) * sB(j,kb) * sum_{k in kb} dec(A[i][k]) * dec(B[j][k]).           */
/* A [I,Kc] and B [J,Kc] hold E4M3 codes, contraction index contiguous.        */
/* sA(i,kb) = sA[i*(Kc/128) + kb] (one scale per row and block).                */
/* sB depends on the mode:                                                      */
/*   0 BLOCK    sB(j,kb) = sB[(j/128)*(Kc/128) + kb]  (weights, fprop)          */
/*   1 BLOCK_T  sB(j,kb) = sB[kb*ceil(J/128) + j/128] (weight scales read        */
/*              transposed, dgrad)                                              */
/*   2 ROW      sB(j,kb) = sB[j*(Kc/128) + kb]         (token-axis tiles, wgrad)   */
/* rows (nullable) lists the output rows to compute; out is [nrows][J].          */
/* ------------------------------------------------------------------------- */
int oracle_gemm(int mode, const uint8_t* A, const float* sA, const uint8_t* B, const float* sB,
                int64_t I, int64_t J, int64_t Kc, const int64_t* rows, int64_t nrows, float* out,
                int threads) {
    if (I < 0 || J < 0 || Kc < 0 || Kc % TILE) return ORACLE_ERR_SHAPE;
    if (mode < 0 || mode > 2) return ORACLE_ERR_ARG;
    if (!rows) nrows = I;
    for (int64_t r = 0; rows && r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= I) return ORACLE_ERR_ARG;
    int64_t kbn = Kc / TILE, jb = (J + TILE - 1) / TILE;

    /* Decode B once to exact integer units; reject NaN codes. */
    int32_t* Bu = (int32_t*)malloc(sizeof(int32_t) * (size_t)(J * Kc > 0 ? J * Kc : 1));
    if (!Bu) return ORACLE_ERR_NOMEM;
    int bad = 0;
    for (int64_t e = 0; e < J * Kc; ++e) {
        Bu[e] = g_units[B[e]];
        if (Bu[e] == INT32_MIN) bad = 1;
    }
    if (bad) { free(Bu); return ORACLE_ERR_NONFINITE; }

    int status = ORACLE_OK;
    set_threads(threads);
    #pragma omp parallel
    {
        int32_t* Au = (int32_t*)malloc(sizeof(int32_t) * (size_t)(Kc > 0 ? Kc : 1));
        #pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t i = rows ? rows[r] : r;
            int row_bad = 0;
            for (int64_t k = 0; k < Kc; ++k) {
                Au[k] = g_units[A[i * Kc + k]];
                if (Au[k] == INT32_MIN) row_bad = 1;
            }
            if (row_bad) {
                #pragma omp atomic write
                status = ORACLE_ERR_NONFINITE;
                continue;
            }
            for (int64_t j = 0; j < J; ++j) {
                float acc = 0.0f;
                for (int64_t kb = 0; kb < kbn; ++kb) {
                    int64_t P = 0; /* exact: |P| < 128 * 229376^2 < 2^43 */
                    const int32_t* a = Au + kb * TILE;
                    const int32_t* b = Bu + j * Kc + kb * TILE;
                    for (int k = 0; k < TILE; ++k) P += (int64_t)a[k] * (int64_t)b[k];
                    float t = (float)P * 0x1p-18f; /* one rounding, then an exact 2^-18 */
                    float sa = sA[i * kbn + kb];
                    float sb;
                    if (mode == 0) sb = sB[(j / TILE) * kbn + kb];
                    else if (mode == 1) sb = sB[kb * jb + j / TILE];
                    else sb = sB[j * kbn + kb];
                    float c = sa * sb;
                    float term = t * c;
                    acc = acc + term;
                }
                out[r * J + j] = acc;
            }
        }
        free(Au);
    }
    free(Bu);
    return status;
}

/* ------------------------------------------------------------------------- */
/* SwiGLU, the BF16 elementwise op of the MLP that produces the input H of     */
/* the down projection (the report keeps such numerically sensitive work in   */
/* BF16/FP32 and runs only the main linear matmuls in FP8):                   */
/*     h[m][f] = silu(g) * u,   silu(g) = g / (1 + e^(-g)),                     */
/* with the gate g = gu[m][f] (the first F columns of the gate/up projection's */
/* output [M, 2F]) and the up value u = gu[m][F + f] (the last F).  Evaluated */
/* in double (exp from libm) and rounded once to BF16, ties to even.          */
/* ------------------------------------------------------------------------- */
/* double -> BF16 bits with one rounding, to nearest, ties to even: a normal   */
/* BF16 value has 8 significant bits, so the rounding unit of |v| in           */
/* [2^(e-1), 2^e) is 2^(e-8); below 2^-126 the unit is fixed at 2^-133 (BF16   */
/* subnormals).  A result of 2^128 or more is infinity.                        */
static uint16_t f64_to_bf16(double v) {
    if (isnan(v)) return 0x7FC0u;
    const uint16_t sign = signbit(v) ? 0x8000u : 0u;
    const double a = fabs(v);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                                   /* a = m 2^e, m in [0.5, 1) */
    int unit = e - 8;
    if (unit < -133) unit = -133;
    const double r = ldexp(nearbyint(ldexp(a, -unit)), unit);   /* default mode: ties to even */
    const float f = (float)r;                       /* exact, or infinity past FP32's range */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFFu));
}

int oracle_swiglu_bf16(const uint16_t* gu, int64_t M, int64_t F, uint16_t* h, int threads) {
    if (M < 0 || F < 0) return ORACLE_ERR_SHAPE;
    if ((M > 0 && F > 0) && (!gu || !h)) return ORACLE_ERR_ARG;
    for (int64_t e = 0; e < M * 2 * F; ++e)
        if (!isfinite(bf16_to_f32(gu[e]))) return ORACLE_ERR_NONFINITE;
    set_threads(threads);
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t f = 0; f < F; ++f) {
            const double g = (double)bf16_to_f32(gu[m * 2 * F + f]);
            const double u = (double)bf16_to_f32(gu[m * 2 * F + F + f]);
            const double silu = g / (1.0 + exp(-g));
            h[m * F + f] = f64_to_bf16(silu * u);
        }
    }
    return ORACLE_OK;
}

/* SwiGLU backward: from the gradient dh of H = silu(g) * u,                  */
/*     d_gate = dh * u * silu'(g),  silu'(g) = s (1 + g (1 - s)),  s = 1/(1+e^-g) */
/*     d_up   = dh * silu(g),                                                  */
/* written as the gradient of the gate/up output [M, 2F] (d_gate in columns   */
/* 0..F-1, d_up in F..2F-1).  Double, one rounding to BF16 per element.       */
int oracle_swiglu_backward_bf16(const uint16_t* dh, const uint16_t* gu, int64_t M, int64_t F,
                                uint16_t* dgu, int threads) {
    if (M < 0 || F < 0) return ORACLE_ERR_SHAPE;
    if ((M > 0 && F > 0) && (!dh || !gu || !dgu)) return ORACLE_ERR_ARG;
    for (int64_t e = 0; e < M * F; ++e)
        if (!isfinite(bf16_to_f32(dh[e]))) return ORACLE_ERR_NONFINITE;
    for (int64_t e = 0; e < M * 2 * F; ++e)
        if (!isfinite(bf16_to_f32(gu[e]))) return ORACLE_ERR_NONFINITE;
    set_threads(threads);
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t f = 0; f < F; ++f) {
            const double d = (double)bf16_to_f32(dh[m * F + f]);
            const double g = (double)bf16_to_f32(gu[m * 2 * F + f]);
            const double u = (double)bf16_to_f32(gu[m * 2 * F + F + f]);
            const double sig = 1.0 / (1.0 + exp(-g));
            dgu[m * 2 * F + f] = f64_to_bf16(d * u * (sig * (1.0 + g * (1.0 - sig))));
            dgu[m * 2 * F + F + f] = f64_to_bf16(d * (g * sig));
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------- */
/* RMSNorm, the BF16 op in front of the attention and MLP input projections:  */
/*     y[m][c] = x[m][c] * r[m] * gamma[c],  r[m] = 1 / sqrt(mean_c x^2 + eps). */
/* Double, one rounding of y to BF16; r is returned rounded to FP32.          */
/* ------------------------------------------------------------------------- */
int oracle_rmsnorm_bf16(const uint16_t* x, const uint16_t* gamma, double eps, int64_t M,
                        int64_t C, uint16_t* y, float* rstd, int threads) {
    if (M < 0 || C <= 0 || !(eps >= 0.0)) return ORACLE_ERR_SHAPE;
    if (M > 0 && (!x || !gamma || !y || !rstd)) return ORACLE_ERR_ARG;
    for (int64_t e = 0; e < M * C; ++e)
        if (!isfinite(bf16_to_f32(x[e]))) return ORACLE_ERR_NONFINITE;
    for (int64_t c = 0; c < C; ++c)
        if (!isfinite(bf16_to_f32(gamma[c]))) return ORACLE_ERR_NONFINITE;
    set_threads(threads);
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        double ss = 0.0;
        for (int64_t c = 0; c < C; ++c) {
            const double v = (double)bf16_to_f32(x[m * C + c]);
            ss += v * v;
        }
        const double r = 1.0 / sqrt(ss / (double)C + eps);
        rstd[m] = (float)r;
        for (int64_t c = 0; c < C; ++c)
            y[m * C + c] = f64_to_bf16((double)bf16_to_f32(x[m * C + c]) * r *
                                       (double)bf16_to_f32(gamma[c]));
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------- */
/* BF16 GEMM, the unquantized comparator of the FP8 path (the report weighs   */
/* its FP8 training against BF16 training of the same model):                 */
/*     out[i][j] = sum_k a(i,k) * b(j,k),  a = A [I,K], b = B [J,K] BF16 bits. */
/* A product of two BF16 values has at most 16 significant bits and is exact  */
/* in double; the sum runs in double, k ascending, and is rounded once to     */
/* FP32.  rows (nullable) lists the output rows; out is [nrows][J].            */
/* ------------------------------------------------------------------------- */
int oracle_gemm_bf16(const uint16_t* A, const uint16_t* B, int64_t I, int64_t J, int64_t K,
                     const int64_t* rows, int64_t nrows, float* out, int threads) {
    if (I < 0 || J < 0 || K < 0) return ORACLE_ERR_SHAPE;
    if (!rows) nrows = I;
    for (int64_t r = 0; rows && r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= I) return ORACLE_ERR_ARG;
    for (int64_t e = 0; e < J * K; ++e)
        if (!isfinite(bf16_to_f32(B[e]))) return ORACLE_ERR_NONFINITE;
    int status = ORACLE_OK;
    set_threads(threads);
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t i = rows ? rows[r] : r;
        int row_bad = 0;
        for (int64_t k = 0; k < K; ++k)
            if (!isfinite(bf16_to_f32(A[i * K + k]))) row_bad = 1;
        if (row_bad) {
            #pragma omp atomic write
            status = ORACLE_ERR_NONFINITE;
            continue;
        }
        for (int64_t j = 0; j < J; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += (double)bf16_to_f32(A[i * K + k]) * (double)bf16_to_f32(B[j * K + k]);
            out[r * J + j] = (float)acc;
        }
    }
    return status;
}
