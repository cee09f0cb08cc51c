/*
 * lq_oracle.c -- plain, slow FP64 CPU oracle for windowed INT8 recurrent-state
 * decode of Gated DeltaNet (scalar gate) and Kimi Delta Attention (channel gate).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is compiled into liboracle.so and is
 * loaded by the test-suite, by the package smoke check and by the CPU-baseline
 * leg of bench.py.  The GPU library never links, loads or calls it, and it
 * shares no source with the GPU library.
 *
 * Sources (web pages about arXiv 2609.38166, "LeapQuant: Efficient Linear
 * Attention with Accurate Recurrent State Quantization"):
 *   [ABS]  the arXiv abstract, as reproduced on the mlsanity.com paper page,
 *          section "Abstract (arXiv)";
 *   [REV]  the bedrocknews.com review article of arXiv 2609.38166 (single body
 *          paragraph);
 *   [IDX]  the paperaft.vercel.app index.json record, field "summary".
 * The pages print no equation.  Where they are silent this file takes one
 * reading and says so with the tag READING; every such reading is listed in
 * the repository's design notes.
 *
 * Notation (READING, fixed by the two delta-rule invariants "beta = 0 with
 * gate = 1 keeps the state" and "beta = 1 with a unit key gives S k = v"):
 *   S      d_v x d_k state, maps keys to values, row-major S[i*dk + j];
 *   A_t    = Diag(g_t) (I - beta_t k_t k_t^T), g_t = alpha_t * 1 for GDN
 *          (scalar gate) and g_t = a_t in (0,1]^{d_k} for KDA (gate on the key
 *          channels);
 *   S_t    = S_{t-1} A_t + beta_t v_t k_t^T;      o_t = S_t q_t  (post-update).
 *
 * Everything is FP64.  Inputs are FP32 (they are what the library receives),
 * quantizer outputs are rounded to their storage types (fp32 scales, smoothing
 * and compensators; int8 codes) exactly where the stored state holds them.
 * Units (one sequence x value head) are independent; OpenMP only splits the
 * outer loop over units and never changes the arithmetic inside one unit.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_GATE_SCALAR 0 /* GDN: one alpha per (token, unit)             */
#define ORC_GATE_CHANNEL 1 /* KDA: one a-vector of d_k per (token, unit)  */

#define ORC_FMT_INT8 0 /* codes are integers in [-127, 127]             */
#define ORC_FMT_E4M3 1 /* codes are 8-bit floats, E4M3 (no infinities)  */

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* The two 8-bit code formats                                               */
/* ------------------------------------------------------------------------ */
/*
 * [ABS] says the state is kept in 8 bits; [REV] says INT8.  READING: INT8 is
 * the main format; an 8-bit floating-point variant is the alternative the
 * word "8-bit" also allows.  It is the E4M3 format of the OCP 8-bit floating
 * point specification (the "FN" flavour, no infinities): one sign bit, four
 * exponent bits with bias 7, three mantissa bits.  Exponent field 0 holds the
 * subnormals m/8 * 2^-6; exponent field 15 with mantissa 7 is NaN, so the
 * largest finite magnitude is (1 + 6/8) * 2^8 = 448.  The quantizer is the
 * same in both formats (compensators, smoothing, per-row scale); only the
 * code grid and its largest magnitude (127 or 448) differ.
 */
double orc_e4m3_value(int code) {
    const int c = code & 0xFF;
    const double sign = (c & 0x80) ? -1.0 : 1.0;
    const int e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) return sign * ldexp((double)m / 8.0, -6);
    return sign * ldexp(1.0 + (double)m / 8.0, e - 7);
}

/*
 * Nearest E4M3 value, ties to the even mantissa, magnitudes above 448 taken
 * as 448.  Around a magnitude a the representable values are spaced
 * 2^(E-3) with E = max(floor(log2 a), -6); a / 2^(E-3) rounded to an
 * integer k gives k = m (subnormal), 8 + m (normal) or 16 (the next binade).
 * READING: zero (also a negative value that rounds to zero) is the code 0x00.
 */
int orc_e4m3_encode(double x) {
    double a = fabs(x);
    if (a > 448.0) a = 448.0;
    if (a == 0.0) return 0;
    int ex;
    frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1): floor(log2 a) = ex - 1 */
    int E = ex - 1;
    if (E < -6) E = -6;
    const double k = nearbyint(ldexp(a, 3 - E)); /* exact scaling, then ties-to-even */
    if (k == 0.0) return 0;
    int e, m;
    if (k < 8.0) {
        e = 0;
        m = (int)k;
    } else if (k == 16.0) {
        e = E + 8;
        m = 0;
    } else {
        e = E + 7;
        m = (int)k - 8;
    }
    return (x < 0.0 ? 0x80 : 0) | (e << 3) | m;
}

/* ------------------------------------------------------------------------ */
/* Buffer precision                                                          */
/* ------------------------------------------------------------------------ */
/*
 * [ABS]: inside a window the outputs use high-precision buffered updates.
 * READING: the buffer holds each token's k and v either in fp32 (as given)
 * or in IEEE binary16 (1 sign bit, 5 exponent bits with bias 15, 10 mantissa
 * bits; subnormals m/1024 * 2^-14; largest finite 65504), the buffered token
 * then being the rounded one everywhere (its own output, later replays and
 * the window-end state).  Rounding is to nearest, ties to the even mantissa;
 * magnitudes above 65504 are stored as 65504 (saturation, READING) and NaN
 * stays NaN.  Around a magnitude a the binary16 values are spaced 2^(E-10),
 * E = max(floor(log2 a), -14).
 */
float orc_fp16_round(float xf) {
    const double x = (double)xf;
    if (isnan(x)) return xf;
    double a = fabs(x);
    if (a > 65504.0) a = 65504.0;
    if (a == 0.0) return xf;
    int ex;
    frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1) */
    int E = ex - 1;
    if (E < -14) E = -14;
    const double r = ldexp(nearbyint(ldexp(a, 10 - E)), E - 10);
    return (float)(x < 0.0 ? -r : r);
}

void orc_fp16_round_array(long n, const float* in, float* out) {
    for (long i = 0; i < n; ++i) out[i] = orc_fp16_round(in[i]);
}

static double code_value(int fmt, int8_t c) {
    return fmt == ORC_FMT_E4M3 ? orc_e4m3_value((uint8_t)c) : (double)c;
}

static double code_max(int fmt) { return fmt == ORC_FMT_E4M3 ? 448.0 : 127.0; }

/* The code of an unrounded value x = R / (sigma s), |x| <= code_max up to
 * the rounding of sigma. */
static int8_t code_round(int fmt, double x) {
    if (fmt == ORC_FMT_E4M3) return (int8_t)(uint8_t)orc_e4m3_encode(x);
    double c = nearbyint(x); /* default rounding mode: nearest, ties to even */
    if (c > 127.0) c = 127.0;
    if (c < -127.0) c = -127.0;
    return (int8_t)c;
}

/* ------------------------------------------------------------------------ */
/* O1: one step of the plain delta-rule recurrence on one unit.              */
/* ------------------------------------------------------------------------ */
/*
 * S <- S A_t + beta v k^T with A_t = Diag(g)(I - beta k k^T), written out as
 *   M = S Diag(g)                      (gate the key channels: READING, gate
 *                                       applied before the delta correction)
 *   S = M - beta (M k) k^T + beta v k^T
 * and, when o is given, o = S q with the updated S (READING: output after the
 * update, so a token sees its own write).
 *
 * [ABS]: GDN and KDA hold everything seen so far in a recurrent state whose
 * size does not grow with the context; every token reads and updates it.  The recurrence itself is not
 * printed on the pages; this is the gated delta rule of the works the pages
 * cite ("Gated Delta Networks: Improving Mamba2 with Delta Rule"; "Kimi
 * Linear"), in the orientation the invariants above fix.
 */
static void step_one(int dk, int dv, int gate_kind, double* S, const float* q,
                     const float* k, const float* v, float beta, const float* g,
                     double* o, double* Mk /* scratch, dv */) {
    for (int i = 0; i < dv; ++i) {
        for (int j = 0; j < dk; ++j) {
            double gj = (gate_kind == ORC_GATE_SCALAR) ? (double)g[0] : (double)g[j];
            S[(size_t)i * dk + j] *= gj; /* S now holds M = S Diag(g) */
        }
    }
    for (int i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * (double)k[j];
        Mk[i] = acc;
    }
    for (int i = 0; i < dv; ++i) {
        for (int j = 0; j < dk; ++j) {
            S[(size_t)i * dk + j] = S[(size_t)i * dk + j] - (double)beta * Mk[i] * (double)k[j] +
                                    (double)beta * (double)v[i] * (double)k[j];
        }
    }
    if (o) {
        for (int i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * (double)q[j];
            o[i] = acc;
        }
    }
}

/*
 * O1 over n_tok tokens for n_units independent units.
 *   S     [n_units][dv][dk]  in/out
 *   q, k  [n_tok][n_units][dk]
 *   v     [n_tok][n_units][dv]
 *   beta  [n_tok][n_units]
 *   gate  [n_tok][n_units] (scalar) or [n_tok][n_units][dk] (channel)
 *   o     [n_tok][n_units][dv] or NULL
 */
int orc_recurrence(int n_units, int dk, int dv, int n_tok, int gate_kind, double* S,
                   const float* q, const float* k, const float* v, const float* beta,
                   const float* gate, double* o) {
    if (n_units < 0 || dk <= 0 || dv <= 0 || n_tok < 0) return -1;
    const int gstride = (gate_kind == ORC_GATE_SCALAR) ? 1 : dk;
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < n_units; ++u) {
        double* Mk = (double*)malloc(sizeof(double) * (size_t)dv);
        double* Su = S + (size_t)u * dv * dk;
        for (int t = 0; t < n_tok; ++t) {
            size_t tu = (size_t)t * n_units + u;
            step_one(dk, dv, gate_kind, Su, q ? q + tu * dk : NULL, k + tu * dk, v + tu * dv,
                     beta[tu], gate + tu * gstride, (o && q) ? o + tu * dv : NULL, Mk);
        }
        free(Mk);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Qz: compensator extraction, smoothing and 8-bit requantization.           */
/* ------------------------------------------------------------------------ */
/*
 * [ABS]: the state's largest outliers are kept as a few high-precision
 * Compensator Tokens, the remaining residual is smoothed, then quantized to
 * 8 bits.  [REV]: the biggest outlier rows and columns are pulled out of the
 * state matrix and kept in FP16/FP32; the state goes from FP32 to INT8.
 *
 * READINGS (the pages give no formula):
 *  - a line's outlier score is its squared L2 norm, taken on the full state;
 *  - candidates are rows 0..dv-1 then columns dv..dv+dk-1, one top-n_c over
 *    all of them, equal scores going to the lower candidate index;
 *  - a selected row is taken whole (v_c = e_row, k_c = S[row,:]); a selected
 *    column is taken with the entries of selected rows set to zero
 *    (v_c = that column, k_c = e_col); each is one compensator token, kept in
 *    fp32; slots hold rows ascending, then columns ascending;
 *  - residual R = S with the selected lines zeroed;
 *  - smoothing per key channel: s_j = sqrt(max_i |R[i,j]|), 1 when that is 0
 *    (SmoothQuant's migration strength 0.5; SmoothQuant is among the cited
 *    works); rounded to fp32;
 *  - scale per row: sigma_i = max_j |R[i,j] / s_j| / qmax, rounded to fp32,
 *    with qmax = 127 (INT8) or 448 (E4M3);
 *  - code of x = R[i,j] / (sigma_i s_j), with the fp32-rounded sigma and s:
 *    INT8 clamp(round-half-even(x), -127, 127); E4M3 the nearest E4M3 value,
 *    ties to the even mantissa; rows with sigma_i = 0 get code 0.
 *
 * Outputs per unit u:
 *   codes    [dv][dk] 8-bit codes (int8 values, or E4M3 bytes)
 *   sigma    [dv] fp32, smooth [dk] fp32
 *   comp_idx [n_c] int32 (c < dv: row c; c >= dv: column c - dv)
 *   comp_vec [n_c][D] fp32, D = max(dk, dv); a row slot holds k_c (dk values),
 *            a column slot holds v_c (dv values), the rest is 0
 *   x_out    [dv][dk] fp64 unrounded code values (0 where sigma_i = 0), or NULL
 *   scores   [dv + dk] fp64 line scores, or NULL
 * force_sel [n_units][n_c] (ascending candidate indices) replaces the top-n_c
 * choice when given.  smooth_enable = 0 fixes s = 1 (used by the per-token
 * ablation only).
 */
static void select_topn(int n_cand, int n_c, const double* score, int* sel, unsigned char* taken) {
    memset(taken, 0, (size_t)n_cand);
    for (int r = 0; r < n_c; ++r) {
        int best = -1;
        for (int c = 0; c < n_cand; ++c) {
            if (taken[c]) continue;
            if (best < 0 || score[c] > score[best]) best = c; /* strict: ties keep lower index */
        }
        taken[best] = 1;
        sel[r] = best;
    }
    /* ascending order: rows first (indices < dv), then columns */
    for (int a = 1; a < n_c; ++a)
        for (int b = a; b > 0 && sel[b - 1] > sel[b]; --b) {
            int t = sel[b];
            sel[b] = sel[b - 1];
            sel[b - 1] = t;
        }
}

/* One unit; all pointers already offset to unit u except that element
 * offsets below still use u = 0. */
static void qz_unit(int fmt, int dk, int dv, int n_c, int smooth_enable, const double* Su,
                    const int* force_sel_u, int8_t* codes, float* sigma, float* smooth,
                    int* comp_idx, float* comp_vec, double* x_out, double* scores_out) {
    const int D = dk > dv ? dk : dv;
    const int n_cand = dv + dk;
    const size_t u = 0;
    {
        double* R = (double*)malloc(sizeof(double) * (size_t)dv * dk);
        double* score = (double*)malloc(sizeof(double) * (size_t)n_cand);
        unsigned char* taken = (unsigned char*)malloc((size_t)n_cand);
        unsigned char* row_sel = (unsigned char*)calloc((size_t)dv, 1);
        unsigned char* col_sel = (unsigned char*)calloc((size_t)dk, 1);
        int* sel = (int*)malloc(sizeof(int) * (size_t)(n_c > 0 ? n_c : 1));
        double* sj = (double*)malloc(sizeof(double) * (size_t)dk);

        /* 1. line scores: squared L2 norms of rows, then of columns */
        for (int i = 0; i < dv; ++i) {
            double a = 0.0;
            for (int j = 0; j < dk; ++j) a += Su[(size_t)i * dk + j] * Su[(size_t)i * dk + j];
            score[i] = a;
        }
        for (int j = 0; j < dk; ++j) {
            double a = 0.0;
            for (int i = 0; i < dv; ++i) a += Su[(size_t)i * dk + j] * Su[(size_t)i * dk + j];
            score[dv + j] = a;
        }
        if (scores_out) memcpy(scores_out + (size_t)u * n_cand, score, sizeof(double) * n_cand);

        /* 2. selection */
        if (force_sel_u) {
            for (int r = 0; r < n_c; ++r) sel[r] = force_sel_u[r];
        } else {
            select_topn(n_cand, n_c, score, sel, taken);
        }
        for (int r = 0; r < n_c; ++r) {
            if (sel[r] < dv) row_sel[sel[r]] = 1;
            else col_sel[sel[r] - dv] = 1;
        }

        /* 3. extraction into compensator slots (fp32), 4. residual */
        memcpy(R, Su, sizeof(double) * (size_t)dv * dk);
        float* cv = comp_vec + (size_t)u * n_c * D;
        for (int r = 0; r < n_c; ++r) {
            comp_idx[(size_t)u * n_c + r] = sel[r];
            for (int e = 0; e < D; ++e) cv[(size_t)r * D + e] = 0.0f;
            if (sel[r] < dv) {
                int row = sel[r];
                for (int j = 0; j < dk; ++j) cv[(size_t)r * D + j] = (float)Su[(size_t)row * dk + j];
            } else {
                int col = sel[r] - dv;
                for (int i = 0; i < dv; ++i)
                    cv[(size_t)r * D + i] = row_sel[i] ? 0.0f : (float)Su[(size_t)i * dk + col];
            }
        }
        for (int i = 0; i < dv; ++i)
            for (int j = 0; j < dk; ++j)
                if (row_sel[i] || col_sel[j]) R[(size_t)i * dk + j] = 0.0;

        /* 5. smoothing per key channel */
        for (int j = 0; j < dk; ++j) {
            double a = 0.0;
            for (int i = 0; i < dv; ++i) {
                double m = fabs(R[(size_t)i * dk + j]);
                if (m > a) a = m;
            }
            float s = 1.0f;
            if (smooth_enable && a > 0.0) s = (float)sqrt(a);
            smooth[(size_t)u * dk + j] = s;
            sj[j] = (double)s;
        }

        /* 6. per-row scale, 7. codes */
        for (int i = 0; i < dv; ++i) {
            double m = 0.0;
            for (int j = 0; j < dk; ++j) {
                double a = fabs(R[(size_t)i * dk + j] / sj[j]);
                if (a > m) m = a;
            }
            float sg = (float)(m / code_max(fmt));
            sigma[(size_t)u * dv + i] = sg;
            for (int j = 0; j < dk; ++j) {
                size_t e = (size_t)u * dv * dk + (size_t)i * dk + j;
                if (sg == 0.0f) {
                    codes[e] = 0;
                    if (x_out) x_out[e] = 0.0;
                    continue;
                }
                double x = R[(size_t)i * dk + j] / ((double)sg * sj[j]);
                if (x_out) x_out[e] = x;
                codes[e] = code_round(fmt, x);
            }
        }
        free(R);
        free(score);
        free(taken);
        free(row_sel);
        free(col_sel);
        free(sel);
        free(sj);
    }
}

int orc_qz(int fmt, int n_units, int dk, int dv, int n_c, int smooth_enable, const double* S,
           const int* force_sel, int8_t* codes, float* sigma, float* smooth, int* comp_idx,
           float* comp_vec, double* x_out, double* scores_out) {
    if (n_units < 0 || dk <= 0 || dv <= 0 || n_c < 0 || n_c > dk + dv) return -1;
    if (fmt != ORC_FMT_INT8 && fmt != ORC_FMT_E4M3) return -1;
    const int D = dk > dv ? dk : dv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < n_units; ++u) {
        size_t e = (size_t)u * dv * dk;
        qz_unit(fmt, dk, dv, n_c, smooth_enable, S + e, force_sel ? force_sel + (size_t)u * n_c : NULL,
                codes + e, sigma + (size_t)u * dv, smooth + (size_t)u * dk,
                comp_idx + (size_t)u * n_c, comp_vec + (size_t)u * n_c * D,
                x_out ? x_out + e : NULL, scores_out ? scores_out + (size_t)u * (dv + dk) : NULL);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Dequantization: S_hat = Diag(sigma) Q Diag(s) + sum_c v_c k_c^T           */
/* ------------------------------------------------------------------------ */
/*
 * [ABS]: within a window the fixed low-bit state stands for the state at the
 * window start; the compensator tokens are part of it.  A row slot adds
 * e_row k_c^T, a column slot adds v_c e_col^T.
 */
static void dequant_unit(int fmt, int dk, int dv, int n_c, const int8_t* codes, const float* sigma,
                         const float* smooth, const int* comp_idx, const float* comp_vec,
                         double* Su) {
    const int D = dk > dv ? dk : dv;
    const size_t u = 0;
    {
        for (int i = 0; i < dv; ++i)
            for (int j = 0; j < dk; ++j)
                Su[(size_t)i * dk + j] = (double)sigma[(size_t)u * dv + i] *
                                         code_value(fmt, codes[(size_t)u * dv * dk + (size_t)i * dk + j]) *
                                         (double)smooth[(size_t)u * dk + j];
        for (int r = 0; r < n_c; ++r) {
            int c = comp_idx[(size_t)u * n_c + r];
            const float* cv = comp_vec + ((size_t)u * n_c + r) * D;
            if (c < dv) {
                for (int j = 0; j < dk; ++j) Su[(size_t)c * dk + j] += (double)cv[j];
            } else {
                for (int i = 0; i < dv; ++i) Su[(size_t)i * dk + (c - dv)] += (double)cv[i];
            }
        }
    }
}

int orc_dequant(int fmt, int n_units, int dk, int dv, int n_c, const int8_t* codes, const float* sigma,
                const float* smooth, const int* comp_idx, const float* comp_vec, double* S) {
    if (n_units < 0 || dk <= 0 || dv <= 0 || n_c < 0) return -1;
    if (fmt != ORC_FMT_INT8 && fmt != ORC_FMT_E4M3) return -1;
    const int D = dk > dv ? dk : dv;
#pragma omp parallel for schedule(static)
    for (int u = 0; u < n_units; ++u) {
        dequant_unit(fmt, dk, dv, n_c, codes + (size_t)u * dv * dk, sigma + (size_t)u * dv,
                     smooth + (size_t)u * dk, comp_idx + (size_t)u * n_c,
                     comp_vec + (size_t)u * n_c * D, S + (size_t)u * dv * dk);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O3: output from the fixed low-bit state plus the buffered window.         */
/* ------------------------------------------------------------------------ */
/*
 * [ABS]: inside a window a token's output is formed from the 8-bit state,
 * which stays unchanged until the window closes, plus the window's tokens
 * kept at full precision.  [REV]: the price is recomputing the
 * contributions of the buffered tokens.
 *
 * With the window-start state S_hat and buffered tokens 1..n (the current
 * token is entry n), the state after token n is
 *   S_n = S_hat A_1...A_n + sum_i beta_i v_i k_i^T A_{i+1}...A_n,
 * so o = S_n q = S_hat r + acc with r = A_1...A_n q and
 *   acc = sum_i beta_i v_i (k_i . A_{i+1}...A_n q).
 * Both come from one backward pass over the buffer: r = q, then for
 * i = n..1: c = k_i . r; acc += beta_i c v_i; r = A_i r = g_i * (r - beta_i c k_i).
 * S_hat r is taken from the stored pieces: Diag(sigma) Q Diag(s) r plus, per
 * compensator token, v_c (k_c . r) -- the compensators are transformed by the
 * window's A_i exactly like the state they were taken from ([ABS]: they share
 * the update path of real tokens).
 *
 * Per unit u, entries are stored entry-major: bk [n_units][n_ent][dk],
 * bv [n_units][n_ent][dv], bb [n_units][n_ent], bg [n_units][n_ent] or
 * [n_units][n_ent][dk]; q [n_units][dk]; o [n_units][dv].
 */
int orc_replay_output(int fmt, int n_units, int dk, int dv, int n_c, int gate_kind, int n_ent,
                      const int8_t* codes, const float* sigma, const float* smooth,
                      const int* comp_idx, const float* comp_vec, const float* bk,
                      const float* bv, const float* bb, const float* bg, const float* q,
                      double* o) {
    if (n_units < 0 || dk <= 0 || dv <= 0 || n_c < 0 || n_ent < 0) return -1;
    if (fmt != ORC_FMT_INT8 && fmt != ORC_FMT_E4M3) return -1;
    const int D = dk > dv ? dk : dv;
    const int gstride = (gate_kind == ORC_GATE_SCALAR) ? 1 : dk;
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < n_units; ++u) {
        double* r = (double*)malloc(sizeof(double) * (size_t)dk);
        double* acc = (double*)calloc((size_t)dv, sizeof(double));
        for (int j = 0; j < dk; ++j) r[j] = (double)q[(size_t)u * dk + j];
        for (int i = n_ent - 1; i >= 0; --i) {
            const float* ki = bk + ((size_t)u * n_ent + i) * dk;
            const float* vi = bv + ((size_t)u * n_ent + i) * dv;
            const float* gi = bg + ((size_t)u * n_ent + i) * gstride;
            double b = (double)bb[(size_t)u * n_ent + i];
            double c = 0.0;
            for (int j = 0; j < dk; ++j) c += (double)ki[j] * r[j];
            for (int e = 0; e < dv; ++e) acc[e] += b * c * (double)vi[e];
            for (int j = 0; j < dk; ++j) {
                double gj = (gate_kind == ORC_GATE_SCALAR) ? (double)gi[0] : (double)gi[j];
                r[j] = gj * (r[j] - b * c * (double)ki[j]);
            }
        }
        double* ou = o + (size_t)u * dv;
        for (int i = 0; i < dv; ++i) {
            double a = 0.0;
            for (int j = 0; j < dk; ++j)
                a += code_value(fmt, codes[(size_t)u * dv * dk + (size_t)i * dk + j]) *
                     (double)smooth[(size_t)u * dk + j] * r[j];
            ou[i] = (double)sigma[(size_t)u * dv + i] * a + acc[i];
        }
        for (int s = 0; s < n_c; ++s) {
            int c = comp_idx[(size_t)u * n_c + s];
            const float* cv = comp_vec + ((size_t)u * n_c + s) * D;
            if (c < dv) {
                double a = 0.0;
                for (int j = 0; j < dk; ++j) a += (double)cv[j] * r[j];
                ou[c] += a;
            } else {
                for (int i = 0; i < dv; ++i) ou[i] += (double)cv[i] * r[c - dv];
            }
        }
        free(r);
        free(acc);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O2: the windowed scheme, definitional ("fake-quant") form, end to end.    */
/* ------------------------------------------------------------------------ */
/*
 * [ABS]: the state runs unquantized through a whole window and is quantized
 * a single time, when the window closes.  [REV]: the state is quantized once at the
 * window boundary instead of after every update.
 *
 * Start: (codes, sigma, s, comps) = Qz(S0) and S_hat = their dequantization.
 * Each token: S_hat <- S_hat A_t + beta v k^T in FP64 (never quantized inside
 * the window) and o_t = S_hat q_t.  After the token that fills the window
 * (fill == W), or after token force_at[u] (a forced partial flush; -1 = none),
 * the state is requantized: S_hat <- dequant(Qz(S_hat)), fill = 0.
 *
 * W = 1, n_c = 0, smooth_enable = 0 is the naive per-token quantization the
 * [REV] page compares against.
 *
 *   S0       [n_units][dv][dk] fp64 (the unquantized start state)
 *   inputs   token-major, as for orc_recurrence
 *   force_at [n_units] or NULL
 *   o        [n_tok][n_units][dv]
 *   S_out    [n_units][dv][dk] final S_hat, or NULL
 */
int orc_windowed_run(int fmt, int buf_fp16, int n_units, int dk, int dv, int n_tok, int gate_kind, int W, int n_c,
                     int smooth_enable, const double* S0, const float* q, const float* k,
                     const float* v, const float* beta, const float* gate, const int* force_at,
                     double* o, double* S_out) {
    if (n_units < 0 || dk <= 0 || dv <= 0 || n_tok < 0 || W < 1 || n_c < 0) return -1;
    if (fmt != ORC_FMT_INT8 && fmt != ORC_FMT_E4M3) return -1;
    const int D = dk > dv ? dk : dv;
    const int gstride = (gate_kind == ORC_GATE_SCALAR) ? 1 : dk;
    int rc = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < n_units; ++u) {
        double* S = (double*)malloc(sizeof(double) * (size_t)dv * dk);
        double* Mk = (double*)malloc(sizeof(double) * (size_t)dv);
        int8_t* cq = (int8_t*)malloc((size_t)dv * dk);
        float* sg = (float*)malloc(sizeof(float) * (size_t)dv);
        float* sm = (float*)malloc(sizeof(float) * (size_t)dk);
        int* ci = (int*)malloc(sizeof(int) * (size_t)(n_c > 0 ? n_c : 1));
        float* cv = (float*)malloc(sizeof(float) * (size_t)(n_c > 0 ? n_c : 1) * D);
        float* kr = (float*)malloc(sizeof(float) * (size_t)dk);
        float* vr = (float*)malloc(sizeof(float) * (size_t)dv);
        memcpy(S, S0 + (size_t)u * dv * dk, sizeof(double) * (size_t)dv * dk);
        qz_unit(fmt, dk, dv, n_c, smooth_enable, S, NULL, cq, sg, sm, ci, cv, NULL, NULL);
        dequant_unit(fmt, dk, dv, n_c, cq, sg, sm, ci, cv, S);
        int fill = 0;
        for (int t = 0; t < n_tok; ++t) {
            size_t tu = (size_t)t * n_units + u;
            const float* kt = k + tu * dk;
            const float* vt = v + tu * dv;
            if (buf_fp16) { /* the window holds the token as rounded into the buffer */
                for (int j = 0; j < dk; ++j) kr[j] = orc_fp16_round(kt[j]);
                for (int i = 0; i < dv; ++i) vr[i] = orc_fp16_round(vt[i]);
                kt = kr;
                vt = vr;
            }
            step_one(dk, dv, gate_kind, S, q + tu * dk, kt, vt, beta[tu], gate + tu * gstride,
                     o + tu * dv, Mk);
            fill += 1;
            int forced = force_at && force_at[u] == t;
            if (fill == W || forced) {
                qz_unit(fmt, dk, dv, n_c, smooth_enable, S, NULL, cq, sg, sm, ci, cv, NULL, NULL);
                dequant_unit(fmt, dk, dv, n_c, cq, sg, sm, ci, cv, S);
                fill = 0;
            }
        }
        if (S_out) memcpy(S_out + (size_t)u * dv * dk, S, sizeof(double) * (size_t)dv * dk);
        free(S);
        free(Mk);
        free(cq);
        free(sg);
        free(sm);
        free(ci);
        free(cv);
        free(kr);
        free(vr);
    }
    return rc;
}
