/*
 * Plain CPU oracle for the MiniMax-H3 AdaLN-modulated projection stages.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests, the package smoke check and the benchmark's CPU
 * baseline may load this library.  It shares no code with the HIP path.
 *
 * What it follows (FlashInfer diffusion_ops pages):
 *  - "minimax_h3_mlp_fp8_sm120", the printed per-row formula block: RMSNorm with an FP32
 *    sum of squares and rsqrt, indexed AdaLN with its device-side guard, per-token e4m3
 *    quantisation, FC1 with FP32 accumulation, SwiGLU, FC2, gated residual.
 *  - "minimax_h3_bf16_pre_attention", description and Parameters (qkv_weight row order,
 *    q/k_norm_weight, rope_cos_sin, rope_positions, out, eps, qk_eps): the same pre-norm
 *    and AdaLN, QKV projection, per-head Q/K RMSNorm, split-half NeoX RoPE on dims [0,96),
 *    destination-major pack.
 *  - "minimax_h3_nvfp4_out_proj", description: out = BF16(residual + BF16(gate[gate_index]*o)),
 *    gate 0 for indices outside [0, rows); and, not on the pages, its MXFP4 (OCP
 *    Microscaling) W4A4 counterpart (see the MXFP4 section).
 *
 * Arithmetic: every value between two rounding points the pages print is carried in
 * IEEE double; each bf16(...), e4m3(...) or RN(...) on the page is one round-to-nearest-even
 * of that double value.  Products of bf16 or e4m3 values are exact in double.
 *
 * Readings where the pages are silent (all also listed with the design notes):
 *  - RMSNorm divides the sum of squares by the row width and adds eps inside the root.
 *  - n = bf16(x * r * w) is a single rounding.
 *  - The QKV output is rounded to bf16 before the per-head Q/K RMSNorm; V is bf16(acc).
 *  - RoPE pairs dimension j with j+48 (j < 48), cos from column j and sin from column 48+j
 *    of the cache row; o_j = u_j c - u_{j+48} s, o_{j+48} = u_{j+48} c + u_j s, each rounded
 *    once; dims [96,128) pass through.
 *  - Out-proj rounds o = bf16(acc) before the gate multiply, as the MLP's o does.
 *  - e4m3 means OCP float8_e4m3fn, round-to-nearest-even, saturating at +-448; a row whose
 *    amax is 0 gets scale 0 and all-zero codes.
 *  - scales are applied left to right: (acc * s_row) * s_col.
 *
 * Every function works on caller-owned host arrays: bf16 values as uint16 bit patterns,
 * e4m3 as uint8 codes.  Rows are independent; callers may split rows over threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define HID 5376
#define NHEAD 56
#define HDIM 128
#define QKVN (3 * NHEAD * HDIM)
#define ATTW (NHEAD * HDIM)
#define NROT 96
#define NFREQ 48
#define INTER 14336

/* ---- number formats ---------------------------------------------------------------- */

double oracle_bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Nearest bf16 (8 significant bits, fp32 exponent range), ties to even.  v finite. */
uint16_t oracle_round_bf16(double v) {
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                          /* a = f * 2^e, f in [0.5, 1) */
    int qexp = (e - 1 >= -126) ? e - 8 : -133;   /* quantum of the binade (or subnormal) */
    double r = ldexp(nearbyint(ldexp(a, -qexp)), qexp);
    if (r >= 0x1.0p128) return sign | 0x7F80u;   /* overflow to infinity */
    float rf = (float)r;                   /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &rf, 4);
    return (uint16_t)(sign | (u >> 16));
}

double oracle_e4m3_value(uint8_t c) {
    int s = c >> 7, ex = (c >> 3) & 15, m = c & 7;
    double v;
    if (ex == 15 && m == 7) return NAN;
    if (ex == 0) v = ldexp((double)m, -9);
    else v = ldexp(1.0 + m / 8.0, ex - 7);
    return s ? -v : v;
}

/* Nearest float8_e4m3fn (4 significant bits, min normal 2^-6, subnormal quantum 2^-9),
 * ties to even, magnitudes beyond 448 saturate to 448.  v finite. */
uint8_t oracle_round_e4m3(double v) {
    uint8_t sign = signbit(v) ? 0x80u : 0u;
    double a = fabs(v);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);
    int qexp = (e - 1 >= -6) ? e - 4 : -9;
    double r = ldexp(nearbyint(ldexp(a, -qexp)), qexp);
    if (r > 448.0) r = 448.0;
    if (r == 0.0) return sign;
    int e2;
    frexp(r, &e2);
    int E = e2 - 1;                        /* r = 1.mmm * 2^E */
    if (E >= -6) {
        int mant = (int)(ldexp(r, -E) * 8.0 - 8.0);
        return (uint8_t)(sign | ((E + 7) << 3) | mant);
    }
    return (uint8_t)(sign | (int)ldexp(r, 9));
}

/* fp32 rounding of a double (C conversion is round-to-nearest-even). */
static double fl32(double v) { return (double)(float)v; }

static double bf(uint16_t b) { return oracle_bf16_value(b); }

/* ---- shared row steps: RMSNorm + indexed AdaLN ------------------------------------- */

/* n = bf16(rmsnorm(x, eps) * w); a = bf16(shift[i] + n * bf16(1 + scale[i])), or a = +0 for
 * the whole row when i is outside [0, rows).  Returns 1 when the row is valid. */
static int norm_adaln_row(const uint16_t* x, const uint16_t* w, const uint16_t* scale,
                          const uint16_t* shift, int64_t rows, int64_t ld, int64_t i, double eps,
                          uint16_t* a_out) {
    int valid = (i >= 0 && i < rows);
    if (!valid) {
        for (int k = 0; k < HID; k++) a_out[k] = 0;
        return 0;
    }
    double ss = 0.0;
    for (int k = 0; k < HID; k++) {
        double v = bf(x[k]);
        ss += v * v;
    }
    double r = 1.0 / sqrt(ss / HID + eps);
    const uint16_t* sc = scale + i * ld;
    const uint16_t* sh = shift + i * ld;
    for (int k = 0; k < HID; k++) {
        double n = bf(oracle_round_bf16(bf(x[k]) * r * bf(w[k])));
        double s1 = bf(oracle_round_bf16(1.0 + bf(sc[k])));
        a_out[k] = oracle_round_bf16(bf(sh[k]) + n * s1);
    }
    return 1;
}

/* ---- bf16 pre-attention --------------------------------------------------------------- */

/* The epilogue of one row: qkv[21504] (bf16, rows [q | k | v] x 56 heads x 128) -> the packed
 * out row [56][3][128] (P = 1): per-head Q/K RMSNorm, RoPE at cache row clamp(p), V as is. */
static void qkv_epilogue_row(const uint16_t* qkv, int64_t p, const uint16_t* qw, const uint16_t* kw,
                             const uint16_t* cs, int64_t S, double qk_eps, uint16_t* orow) {
    if (p < 0) p = 0;
    if (p > S - 1) p = S - 1;
    const uint16_t* crow = cs + p * NROT;
    for (int kind = 0; kind < 3; kind++) {
        for (int h = 0; h < NHEAD; h++) {
            const uint16_t* v = qkv + kind * ATTW + h * HDIM;
            uint16_t* o = orow + (h * 3 + kind) * HDIM;
            if (kind == 2) {            /* V: bf16(acc) only */
                for (int d = 0; d < HDIM; d++) o[d] = v[d];
                continue;
            }
            const uint16_t* nw = kind == 0 ? qw : kw;
            double ss = 0.0;
            for (int d = 0; d < HDIM; d++) ss += bf(v[d]) * bf(v[d]);
            double r2 = 1.0 / sqrt(ss / HDIM + qk_eps);
            double u[HDIM];
            for (int d = 0; d < HDIM; d++) u[d] = bf(oracle_round_bf16(bf(v[d]) * r2 * bf(nw[d])));
            for (int j = 0; j < NFREQ; j++) {
                double c = bf(crow[j]), sn = bf(crow[NFREQ + j]);
                o[j] = oracle_round_bf16(u[j] * c - u[j + NFREQ] * sn);
                o[j + NFREQ] = oracle_round_bf16(u[j + NFREQ] * c + u[j] * sn);
            }
            for (int d = NROT; d < HDIM; d++) o[d] = oracle_round_bf16(u[d]);
        }
    }
}

/* Rows [m0, m1) of the workspace alone: ws[m] = a of row m (the first launch of the stage). */
void oracle_norm_adaln(int64_t m0, int64_t m1, const uint16_t* x, const uint16_t* xw, const uint16_t* scale,
                       const uint16_t* shift, int64_t rows, int64_t ld, const int64_t* idx, double eps,
                       uint16_t* ws) {
    for (int64_t m = m0; m < m1; m++)
        norm_adaln_row(x + m * HID, xw, scale, shift, rows, ld, idx[m], eps, ws + m * HID);
}

/*
 * Rows [m0, m1) of the pre-attention stage.
 *   x[M][5376], xw[5376]; scale/shift: row i at scale + i*ld (ld >= 5376); idx[M] int64;
 *   W[21504][5376] rows [q heads | k heads | v heads], each 56 x 128;
 *   qw/kw[128]; cs[S][96]; pos[M] int64 cache rows (clamped to [0,S)); pass the row
 *   numbers themselves for identity positions.
 *   ws[M][5376] receives a; out[M][56][3][128] receives the packed q/k/v (P = 1).
 */
void oracle_pre_attn(int64_t m0, int64_t m1, const uint16_t* x, const uint16_t* xw,
                     const uint16_t* scale, const uint16_t* shift, int64_t rows, int64_t ld,
                     const int64_t* idx, const uint16_t* W, const uint16_t* qw, const uint16_t* kw,
                     const uint16_t* cs, int64_t S, const int64_t* pos, double eps, double qk_eps,
                     uint16_t* ws, uint16_t* out) {
    double* a = (double*)malloc(sizeof(double) * HID);
    uint16_t* qkv = (uint16_t*)malloc(sizeof(uint16_t) * QKVN);
    for (int64_t m = m0; m < m1; m++) {
        uint16_t* arow = ws + m * HID;
        norm_adaln_row(x + m * HID, xw, scale, shift, rows, ld, idx[m], eps, arow);
        for (int k = 0; k < HID; k++) a[k] = bf(arow[k]);
        /* QKV projection, one bf16 rounding per output */
        for (int n = 0; n < QKVN; n++) {
            const uint16_t* wr = W + (int64_t)n * HID;
            double acc = 0.0;
            for (int k = 0; k < HID; k++) acc += a[k] * bf(wr[k]);
            qkv[n] = oracle_round_bf16(acc);
        }
        qkv_epilogue_row(qkv, pos[m], qw, kw, cs, S, qk_eps, out + m * NHEAD * 3 * HDIM);
    }
    free(a);
    free(qkv);
}

/* ---- bf16 out-projection with gated residual ------------------------------------------- */

/* out[m][n] = bf16(res + bf16(g * o)) for one row given o (already bf16); g = gate[i][n] when
 * 0 <= i < rows, else 0. */
static void gated_row(const double* o, int64_t i, const uint16_t* gate, int64_t rows, int64_t ld,
                      const uint16_t* res, uint16_t* out) {
    int valid = (i >= 0 && i < rows);
    for (int n = 0; n < HID; n++) {
        double g = valid ? bf(gate[i * ld + n]) : 0.0;
        double go = bf(oracle_round_bf16(g * o[n]));
        out[n] = oracle_round_bf16(bf(res[n]) + go);
    }
}

/*
 * Rows [m0, m1): o = bf16(attn[m] . Wo[n]); g = gate[gi[m]][n] if 0 <= gi[m] < rows else 0;
 * out = bf16(res + bf16(g * o)).  attn[M][7168], Wo[5376][7168], gate row i at gate + i*ld.
 */
void oracle_out_proj(int64_t m0, int64_t m1, const uint16_t* attn, const uint16_t* Wo,
                     const uint16_t* gate, int64_t rows, int64_t ld, const int32_t* gi,
                     const uint16_t* res, uint16_t* out) {
    double* a = (double*)malloc(sizeof(double) * ATTW);
    double* o = (double*)malloc(sizeof(double) * HID);
    for (int64_t m = m0; m < m1; m++) {
        for (int k = 0; k < ATTW; k++) a[k] = bf(attn[m * ATTW + k]);
        for (int n = 0; n < HID; n++) {
            const uint16_t* wr = Wo + (int64_t)n * ATTW;
            double acc = 0.0;
            for (int k = 0; k < ATTW; k++) acc += a[k] * bf(wr[k]);
            o[n] = bf(oracle_round_bf16(acc));
        }
        gated_row(o, gi[m], gate, rows, ld, res + m * HID, out + m * HID);
    }
    free(o);
    free(a);
}

/* ---- MXFP4 (OCP Microscaling): E2M1 elements, one E8M0 scale per 32 along K --------------
 * Not on the pages.  The gfx950-native counterpart of the NVFP4 W4A4 out-projection
 * ("minimax_h3_nvfp4_out_proj": block-16 E2M1 with UE4M3 block scales and a global scale)
 * in the format the hardware scales natively, OCP Microscaling Formats (MX) v1.0, MXFP4:
 *  - a block is 32 consecutive values of a row along K; its scale is X = 2^(E - 127), stored
 *    as the E8M0 byte E;
 *  - E is the MX conversion's shared exponent: floor(log2(amax)) - 2 (2 is the largest E2M1
 *    exponent), biased by 127 and clamped to [0, 254]; an all-zero block gets E = 0;
 *  - each element is the E2M1 value nearest v / X (exact: X is a power of two), ties to the
 *    even significand, magnitudes beyond 6 saturating to 6, the sign kept (so -0 is code 8);
 *  - codes pack two per byte along K, element 2j in the low nibble of byte j.
 */
static const double e2m1_mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oracle_e2m1_value(uint8_t c) {
    double v = e2m1_mag[c & 7];
    return (c & 8) ? -v : v;
}

uint8_t oracle_round_e2m1(double v) {
    uint8_t sign = signbit(v) ? 8u : 0u;
    double a = fabs(v);
    if (a >= 6.0) return (uint8_t)(sign | 7);     /* saturate (for huge a the distances below tie) */
    int best = 0;
    for (int c = 1; c < 8; c++) {
        double d = fabs(a - e2m1_mag[c]), db = fabs(a - e2m1_mag[best]);
        if (d < db || (d == db && (c & 1) == 0)) best = c;   /* the code's last bit is the significand */
    }
    return (uint8_t)(sign | best);
}

int oracle_mx_scale_exp(double amax) {
    if (amax == 0.0) return 0;
    int e;
    frexp(amax, &e);                       /* amax = f 2^e, f in [0.5, 1): floor(log2) = e - 1 */
    int E = (e - 1) - 2 + 127;
    return E < 0 ? 0 : (E > 254 ? 254 : E);
}

/* x[R][K] bf16 -> codes[R][K/2], scales[R][K/32] (row-major E8M0 bytes).  K % 32 == 0. */
void oracle_mx_quant_fp4(const uint16_t* x, int64_t R, int64_t K, uint8_t* codes, uint8_t* scales) {
    for (int64_t r = 0; r < R; r++) {
        for (int64_t b = 0; b < K / 32; b++) {
            const uint16_t* v = x + r * K + b * 32;
            double amax = 0.0;
            for (int k = 0; k < 32; k++) {
                double t = fabs(bf(v[k]));
                if (t > amax) amax = t;
            }
            int E = oracle_mx_scale_exp(amax);
            scales[r * (K / 32) + b] = (uint8_t)E;
            for (int k = 0; k < 32; k += 2) {
                uint8_t lo = oracle_round_e2m1(ldexp(bf(v[k]), 127 - E));
                uint8_t hi = oracle_round_e2m1(ldexp(bf(v[k + 1]), 127 - E));
                codes[r * (K / 2) + b * 16 + k / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
}

/* the values of one MXFP4 row of n elements (n % 32 == 0) */
static void mx_row_values(const uint8_t* codes, const uint8_t* scales, int64_t n, double* v) {
    for (int64_t b = 0; b < n / 32; b++) {
        const double X = ldexp(1.0, (int)scales[b] - 127);
        for (int64_t k = 32 * b; k < 32 * b + 32; k++) {
            uint8_t c = (codes[k / 2] >> (4 * (k & 1))) & 15;
            v[k] = oracle_e2m1_value(c) * X;
        }
    }
}

/*
 * Rows [m0, m1) of the MXFP4 W4A4 out-projection: o = bf16(A[m] . W[n]) with A and W the
 * values of their MXFP4 codes and scales (exact products, exact double sum of 7168 terms up to
 * rounding far below a bf16 ulp), then the gated residual of oracle_out_proj.
 * a_codes[M][3584], a_scales[M][224], w_codes[5376][3584], w_scales[5376][224] (row-major).
 */
void oracle_out_proj_mxfp4(int64_t m0, int64_t m1, const uint8_t* a_codes, const uint8_t* a_scales,
                           const uint8_t* w_codes, const uint8_t* w_scales, const uint16_t* gate,
                           int64_t rows, int64_t ld, const int32_t* gi, const uint16_t* res, uint16_t* out) {
    double* a = (double*)malloc(sizeof(double) * ATTW);
    double* w = (double*)malloc(sizeof(double) * ATTW * HID);    /* all of W's values, 308 MB */
    double* o = (double*)malloc(sizeof(double) * HID);
    for (int n = 0; n < HID; n++)
        mx_row_values(w_codes + (int64_t)n * (ATTW / 2), w_scales + (int64_t)n * (ATTW / 32), ATTW,
                      w + (int64_t)n * ATTW);
    for (int64_t m = m0; m < m1; m++) {
        mx_row_values(a_codes + m * (ATTW / 2), a_scales + m * (ATTW / 32), ATTW, a);
        for (int n = 0; n < HID; n++) {
            const double* wr = w + (int64_t)n * ATTW;
            double acc = 0.0;
            for (int k = 0; k < ATTW; k++) acc += a[k] * wr[k];
            o[n] = bf(oracle_round_bf16(acc));
        }
        gated_row(o, gi[m], gate, rows, ld, res + m * HID, out + m * HID);
    }
    free(o);
    free(w);
    free(a);
}

/*
 * Rows [m0, m1) of the MXFP4 W4A4 pre-attention GEMM and epilogue (not on the pages; the
 * MXFP4 counterpart of the NVFP4 pre-attention, whose activation is the quantised workspace):
 * qkv = bf16(A[m] . W[n]) with A the values of the workspace's MXFP4 codes/scales
 * (ws_codes[M][2688], ws_scales[M][168], row-major) and W those of the weight
 * (w_codes[21504][2688], w_scales[21504][168]); then the bf16 pre-attention's epilogue.
 * pos[M] cache rows (the row numbers for identity positions); out[M][56][3][128].
 */
void oracle_qkv_mxfp4(int64_t m0, int64_t m1, const uint8_t* ws_codes, const uint8_t* ws_scales,
                      const uint8_t* w_codes, const uint8_t* w_scales, const uint16_t* qw, const uint16_t* kw,
                      const uint16_t* cs, int64_t S, const int64_t* pos, double qk_eps, uint16_t* out) {
    double* a = (double*)malloc(sizeof(double) * HID);
    double* w = (double*)malloc(sizeof(double) * HID);
    uint16_t* qkv = (uint16_t*)malloc(sizeof(uint16_t) * QKVN);
    for (int64_t m = m0; m < m1; m++) {
        mx_row_values(ws_codes + m * (HID / 2), ws_scales + m * (HID / 32), HID, a);
        for (int n = 0; n < QKVN; n++) {
            mx_row_values(w_codes + (int64_t)n * (HID / 2), w_scales + (int64_t)n * (HID / 32), HID, w);
            double acc = 0.0;
            for (int k = 0; k < HID; k++) acc += a[k] * w[k];
            qkv[n] = oracle_round_bf16(acc);
        }
        qkv_epilogue_row(qkv, pos[m], qw, kw, cs, S, qk_eps, out + m * NHEAD * 3 * HDIM);
    }
    free(qkv);
    free(w);
    free(a);
}

/* ---- per-token e4m3 quantisation ---------------------------------------------------------- */

/* s = RN(amax(|v|) / 448) in fp32; code[k] = e4m3(fl32(v[k] / s)); amax 0 -> s 0, codes 0. */
static float quant_row(const uint16_t* v, int n, uint8_t* code) {
    double amax = 0.0;
    for (int k = 0; k < n; k++) {
        double t = fabs(bf(v[k]));
        if (t > amax) amax = t;
    }
    double s = fl32(amax / 448.0);
    for (int k = 0; k < n; k++) code[k] = (s == 0.0) ? 0 : oracle_round_e4m3(fl32(bf(v[k]) / s));
    return (float)s;
}

/* ---- e4m3 output mode of the pre-attention ------------------------------------------------
 * "minimax_h3_nvfp4_pre_attention", Parameters (out_mode "e4m3" with per-tensor q/k/v
 * dequantization scales; its quantisation page is missing, so the plainest reading): each
 * element v of the bf16 output becomes code = e4m3(fl32(v / descale)), saturating at 448, with
 * descale the scale of the element's kind.  In the packed output [..., 3, 128] the kind of
 * element e is (e / 128) mod 3.  fl32 of the fp64 quotient is the correctly rounded fp32
 * quotient (53 >= 2 * 24 + 2 bits). */
void oracle_quant_out_e4m3(const uint16_t* v, int64_t n, double dq, double dk, double dv, uint8_t* code) {
    for (int64_t e = 0; e < n; e++) {
        const int kind = (int)((e / HDIM) % 3);
        const double d = kind == 0 ? dq : (kind == 1 ? dk : dv);
        code[e] = oracle_round_e4m3(fl32(bf(v[e]) / d));
    }
}

/* ---- FP8 W8A8 MLP ------------------------------------------------------------------------ */

/* value of every e4m3 code, filled from oracle_e4m3_value (a lookup, not a second decoder) */
static double e4m3_tab[256];
static int e4m3_tab_ready = 0;
static void e4m3_tab_init(void) {
    if (e4m3_tab_ready) return;
    for (int c = 0; c < 256; c++) e4m3_tab[c] = oracle_e4m3_value((uint8_t)c);
    e4m3_tab_ready = 1;
}

/*
 * Rows [m0, m1) of the MLP block.  Tables: row i of scale/shift/gate at base + i*ld.
 * W1q[28672][5376] e4m3 with per-row w1s[28672] (rows [0,14336) gate, [14336,28672) up);
 * W2q[5376][14336] e4m3 with per-row w2s[5376].  Writes a_q[M][5376], a_s[M], y[M][14336],
 * y_q[M][14336], y_s[M] and out[M][5376].  out may alias res or x only when each row is
 * processed before the next reads it (this routine reads the row first).
 */
/* FC2 and the gated residual of one row from its codes y_q and scale s_y (the MLP page's formula
   block, last two lines): o = bf16(acc * s_y * w2s[n]) with acc the exact code dot product,
   out = bf16(res + bf16(g * o)), g = 0 for a guarded row.  yq is scratch for INTER values. */
static void fc2_gated_row(const uint8_t* yq_codes, float sy, int valid, const uint16_t* gate_row,
                          const uint8_t* W2q, const float* w2s, const uint16_t* res_row, double* yq,
                          uint16_t* out_row) {
    for (int k = 0; k < INTER; k++) yq[k] = oracle_e4m3_value(yq_codes[k]);
    for (int n = 0; n < HID; n++) {
        const uint8_t* wr = W2q + (int64_t)n * INTER;
        double acc = 0.0;
        for (int k = 0; k < INTER; k++) acc += yq[k] * e4m3_tab[wr[k]];
        double o = bf(oracle_round_bf16(acc * (double)sy * (double)w2s[n]));
        double g = valid ? bf(gate_row[n]) : 0.0;
        double go = bf(oracle_round_bf16(g * o));
        out_row[n] = oracle_round_bf16(bf(res_row[n]) + go);
    }
}

/* The FC2 + gated residual stage alone, on given y_q [R, 14336] and s_y [R] (rows m0 .. m1 of
   them, with their idx and res rows): the reference for that stage on another path's own y_q. */
void oracle_mlp_fc2(int64_t m0, int64_t m1, const uint8_t* y_q, const float* y_s, const uint16_t* gate,
                    int64_t rows, int64_t ld, const int64_t* idx, const uint16_t* res, const uint8_t* W2q,
                    const float* w2s, uint16_t* out) {
    double* yq = (double*)malloc(sizeof(double) * INTER);
    e4m3_tab_init();
    for (int64_t m = m0; m < m1; m++) {
        int64_t i = idx[m];
        int valid = i >= 0 && i < rows;
        fc2_gated_row(y_q + m * INTER, y_s[m], valid, valid ? gate + i * ld : gate, W2q, w2s, res + m * HID, yq,
                      out + m * HID);
    }
    free(yq);
}

void oracle_mlp(int64_t m0, int64_t m1, const uint16_t* x, const uint16_t* xw,
                const uint16_t* scale, const uint16_t* shift, const uint16_t* gate, int64_t rows,
                int64_t ld, const int64_t* idx, const uint16_t* res, const uint8_t* W1q,
                const float* w1s, const uint8_t* W2q, const float* w2s, double eps,
                uint8_t* a_q, float* a_s, uint16_t* y, uint8_t* y_q, float* y_s, uint16_t* out) {
    uint16_t* a = (uint16_t*)malloc(sizeof(uint16_t) * HID);
    double* aq = (double*)malloc(sizeof(double) * HID);
    double* yq = (double*)malloc(sizeof(double) * INTER);
    double* h = (double*)malloc(sizeof(double) * 2 * INTER);
    e4m3_tab_init();
    for (int64_t m = m0; m < m1; m++) {
        int64_t i = idx[m];
        int valid = norm_adaln_row(x + m * HID, xw, scale, shift, rows, ld, i, eps, a);
        float sa = quant_row(a, HID, a_q + m * HID);
        a_s[m] = sa;
        for (int k = 0; k < HID; k++) aq[k] = oracle_e4m3_value(a_q[m * HID + k]);
        /* FC1: h = bf16(acc * s_a * w1s[n]) */
        for (int n = 0; n < 2 * INTER; n++) {
            const uint8_t* wr = W1q + (int64_t)n * HID;
            double acc = 0.0;
            for (int k = 0; k < HID; k++) acc += aq[k] * e4m3_tab[wr[k]];
            h[n] = bf(oracle_round_bf16(acc * (double)sa * (double)w1s[n]));
        }
        /* SwiGLU: y = bf16(bf16(silu(h_gate)) * h_up) */
        uint16_t* yrow = y + m * INTER;
        for (int j = 0; j < INTER; j++) {
            double t = h[j];
            double sl = bf(oracle_round_bf16(t / (1.0 + exp(-t))));
            yrow[j] = oracle_round_bf16(sl * h[INTER + j]);
        }
        float sy = quant_row(yrow, INTER, y_q + m * INTER);
        y_s[m] = sy;
        fc2_gated_row(y_q + m * INTER, sy, valid, valid ? gate + i * ld : gate, W2q, w2s, res + m * HID, yq,
                      out + m * HID);
    }
    free(a);
    free(aq);
    free(yq);
    free(h);
}
