/*
 * nh_oracle.c -- plain, slow CPU oracle for the Nemotron-H Mamba2 mixer block.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the GPU library; the two meet only on the
 * seeded inputs drawn by the `synth` package.
 *
 * Sources.  The block's constants come from the issue page "feat(nemotron_
 * voicechat): load the VoiceChat checkpoint and run offline duplex inference
 * ... #1374", section "config.json" (text_config: hidden 4480, 128 Mamba heads
 * of 80, state 128, 8 groups, conv kernel 4 with bias, no projection bias,
 * eps 1e-5, the hybrid_override_pattern) and the 4-bit group-64 quantization of
 * the mixer projections (same section; docs page "Nemotron VoiceChat", intro).
 * The conv weight layout [channels][4] is from the issue page, "Network 2".
 * The pages give no mixer equations; those are the standard Mamba2 mixer
 * (Dao & Gu 2024, "Transformers are SSMs", the selective SSM recurrence):
 *   out = x + out_proj(RMSNormGated(SSM(conv(in_proj(RMSNorm(x)))), z)).
 * The docs page, section "Offline timeline", states that the full-history
 * recompute and the cached per-position mode give the same result; here both
 * modes are the same plain recurrence.
 *
 * Arithmetic: every value is a double.  In CONTRACT mode the values that the
 * GPU path stores in bf16 (u, zxbcdt, xc, y, o) are rounded to bf16 (nearest,
 * ties to even) at the same points, and the SSM state is rounded to float32
 * where it is stored between calls.  EXACT mode rounds nothing.
 *
 * Parity pins live in tests/test_oracle_*.py; every function below is pinned
 * by at least one closed form, invariant, special case, brute-force sum or
 * independent library composition there.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define NHO_EXACT 0
#define NHO_CONTRACT 1

/* ------------------------------------------------------------------ bf16 */

/* bf16 is the upper half of an IEEE float32. */
double nho_bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round a double to the nearest bf16 (8 significant bits), ties to even.
 * Finite inputs only; magnitudes beyond the bf16 range are not produced by
 * the block.  Values below the smallest normal are rounded on the subnormal
 * grid (spacing 2^-133). */
uint16_t nho_double_to_bf16(double v)
{
    double r;
    if (v == 0.0) {
        r = v;
    } else if (fabs(v) < ldexp(1.0, -126)) {
        r = rint(v * ldexp(1.0, 133)) * ldexp(1.0, -133);
    } else {
        int e;
        double m = frexp(v, &e);          /* v = m * 2^e, 0.5 <= |m| < 1 */
        r = ldexp(rint(ldexp(m, 8)), e - 8); /* keep 8 significant bits; rint = ties-to-even */
    }
    float f = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static double round_bf16(double v) { return nho_bf16_to_double(nho_double_to_bf16(v)); }

void nho_double_to_bf16_array(const double *in, uint16_t *out, long n)
{
    for (long i = 0; i < n; ++i) out[i] = nho_double_to_bf16(in[i]);
}

/* ------------------------------------------------------------ scalar maps */

double nho_silu(double v) { return v / (1.0 + exp(-v)); }

/* softplus(v) = ln(1 + e^v), written without overflow. */
double nho_softplus(double v) { return fmax(v, 0.0) + log1p(exp(-fabs(v))); }

/* ------------------------------------------------------------- layer map */

/* hybrid_override_pattern as printed in text_config (issue page, section
 * "config.json"): M = Mamba2 mixer, * = attention, - = MLP. */
static const char NHO_PATTERN[] = "M-M-M-MM-M-M-M*-M-M-M*-M-M-M-M*-M-M-M-M*-M-MM-M-M-M-M-M-";

const char *nho_hybrid_pattern(void) { return NHO_PATTERN; }

/* Writes the indices of the layers marked c; returns how many there are. */
int nho_layers_of_kind(char c, int *idx, int cap)
{
    int n = 0;
    for (int i = 0; NHO_PATTERN[i]; ++i)
        if (NHO_PATTERN[i] == c) {
            if (idx && n < cap) idx[n] = i;
            ++n;
        }
    return n;
}

/* ------------------------------------------------------------------- W4 */

/* Affine 4-bit weights, MLX layout (issue page, "config.json": group_size 64,
 * bits 4; the quantized linear is recognised by its .scales key).  Nibble k of
 * a row sits in word k/8 at bits 4*(k%8), lowest nibble first.
 *   W[n][k] = scales[n][k/gs] * q[n][k] + biases[n][k/gs]. */
int nho_w4_nibble(const uint32_t *qrow, int k) { return (int)((qrow[k / 8] >> (4 * (k % 8))) & 0xFu); }

void nho_w4_dequant_row(const uint32_t *qw, const uint16_t *sc, const uint16_t *bi,
                        int k, int gs, double *out)
{
    for (int j = 0; j < k; ++j) {
        double s = nho_bf16_to_double(sc[j / gs]);
        double b = nho_bf16_to_double(bi[j / gs]);
        out[j] = s * (double)nho_w4_nibble(qw, j) + b;
    }
}

void nho_w4_dequant(const uint32_t *qw, const uint16_t *sc, const uint16_t *bi,
                    int n, int k, int gs, double *W)
{
    for (int r = 0; r < n; ++r)
        nho_w4_dequant_row(qw + (long)r * (k / 8), sc + (long)r * (k / gs),
                           bi + (long)r * (k / gs), k, gs, W + (long)r * k);
}

/* y[m][r] = sum_k W[r][k] * x[m][k] over all n rows of W, for m input rows. */
void nho_w4_matvec(const uint32_t *qw, const uint16_t *sc, const uint16_t *bi,
                   int n, int k, int gs, const double *x, int m, double *y, int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
        double *row = (double *)malloc(sizeof(double) * (size_t)k);
#pragma omp for schedule(static)
        for (int r = 0; r < n; ++r) {
            nho_w4_dequant_row(qw + (long)r * (k / 8), sc + (long)r * (k / gs),
                               bi + (long)r * (k / gs), k, gs, row);
            for (int i = 0; i < m; ++i) {
                const double *xi = x + (long)i * k;
                double acc = 0.0;
                for (int j = 0; j < k; ++j) acc += row[j] * xi[j];
                y[(long)i * n + r] = acc;
            }
        }
        free(row);
    }
}

/* ---------------------------------------------------------------- norms */

/* RMSNorm with a plain weight (eps inside the square root), one row of d. */
static void rmsnorm_row(const double *x, int d, const uint16_t *w, double eps, double *out)
{
    double ss = 0.0;
    for (int i = 0; i < d; ++i) ss += x[i] * x[i];
    double r = 1.0 / sqrt(ss / d + eps);
    for (int i = 0; i < d; ++i) out[i] = x[i] * r * nho_bf16_to_double(w[i]);
}

void nho_rmsnorm(const double *x, int rows, int d, const uint16_t *w, double eps, double *out)
{
    for (int r = 0; r < rows; ++r) rmsnorm_row(x + (long)r * d, d, w, eps, out + (long)r * d);
}

/* Gated RMSNorm over groups: g = y * silu(z); each block of `group` channels
 * is normalised by its own RMS and multiplied by its slice of the weight. */
void nho_rmsnorm_gated(const double *y, const double *z, int rows, int d, int group,
                       const uint16_t *w, double eps, double *out)
{
    double *g = (double *)malloc(sizeof(double) * (size_t)group);
    for (int r = 0; r < rows; ++r)
        for (int j = 0; j < d / group; ++j) {
            const double *yr = y + (long)r * d + (long)j * group;
            const double *zr = z + (long)r * d + (long)j * group;
            for (int i = 0; i < group; ++i) g[i] = yr[i] * nho_silu(zr[i]);
            rmsnorm_row(g, group, w + (long)j * group, eps, out + (long)r * d + (long)j * group);
        }
    free(g);
}

/* ----------------------------------------------------------------- conv */

/* Causal depthwise conv1d of kernel K with bias, followed by SiLU (the
 * conv1d of the Mamba2 mixer; weight [channels][K] as in the issue page,
 * "Network 2").  Cross-correlation with K-1 positions of left context:
 *   out[t][c] = silu(b[c] + sum_{j<K} w[c][j] * in[t-(K-1)+j][c]),
 * so tap K-1 multiplies the newest input.  Inputs before position 0 come
 * from state_in (row r holds position r-(K-1), row 0 oldest), or are zero
 * when state_in is NULL.  state_out receives the last K-1 pre-conv rows.
 * xbc row t starts at xbc + t*ld. */
void nho_conv1d(const double *xbc, long ld, int T, int C, int K, const double *state_in,
                const uint16_t *w, const uint16_t *b, double *out, double *state_out)
{
    for (int c = 0; c < C; ++c) {
        for (int t = 0; t < T; ++t) {
            double acc = nho_bf16_to_double(b[c]);
            for (int j = 0; j < K; ++j) {
                int tau = t - (K - 1) + j;
                double v;
                if (tau >= 0)
                    v = xbc[(long)tau * ld + c];
                else
                    v = state_in ? state_in[(long)(tau + K - 1) * C + c] : 0.0;
                acc += nho_bf16_to_double(w[(long)c * K + j]) * v;
            }
            out[(long)t * C + c] = nho_silu(acc);
        }
        if (state_out) {
            /* new row r holds position T-(K-1)+r */
            double tmp[16];
            for (int r = 0; r < K - 1; ++r) {
                int tau = T - (K - 1) + r;
                if (tau >= 0)
                    tmp[r] = xbc[(long)tau * ld + c];
                else
                    tmp[r] = state_in ? state_in[(long)(tau + K - 1) * C + c] : 0.0;
            }
            for (int r = 0; r < K - 1; ++r) state_out[(long)r * C + c] = tmp[r];
        }
    }
}

/* ------------------------------------------------------ discretisation */

/* dt[t][h] = softplus(dt_raw[t][h] + dt_bias[h]);  A[h] = -exp(A_log[h]). */
void nho_discretize(const double *dt_raw, long ld, int T, int H, const float *dt_bias,
                    const float *A_log, double *dt, double *A)
{
    for (int t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h)
            dt[(long)t * H + h] = nho_softplus(dt_raw[(long)t * ld + h] + (double)dt_bias[h]);
    if (A)
        for (int h = 0; h < H; ++h) A[h] = -exp((double)A_log[h]);
}

/* ------------------------------------------------------------- SSM scan */

/* The selective state-space recurrence of Mamba2, position by position.
 * Head h reads group g = h / (H/G) of B and C.  For every position t:
 *   S[h][p][n] <- exp(dt[t][h]*A[h]) * S[h][p][n] + dt[t][h] * x[t][h*P+p] * B[t][g*N+n]
 *   y[t][h*P+p] = sum_n C[t][g*N+n] * S[h][p][n] + D[h] * x[t][h*P+p]
 * x, B, C rows start at base + t*ld.  S ([H][P][N]) is updated in place.
 * With round_state_f32 the state is rounded to float32 after every position
 * (the state's storage format between per-position calls). */
void nho_ssm_recurrence(int T, int H, int P, int N, int G,
                        const double *x, long ldx, const double *Bm, long ldb,
                        const double *Cm, long ldc, const double *dt, const double *A,
                        const float *D, double *S, double *y, int round_state_f32, int nthreads)
{
    const int hpg = H / G;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel for schedule(static)
    for (int h = 0; h < H; ++h) {
        const int g = h / hpg;
        double *Sh = S + (long)h * P * N;
        for (int t = 0; t < T; ++t) {
            const double dth = dt[(long)t * H + h];
            const double dA = exp(dth * A[h]);
            const double *xt = x + (long)t * ldx + (long)h * P;
            const double *Bt = Bm + (long)t * ldb + (long)g * N;
            const double *Ct = Cm + (long)t * ldc + (long)g * N;
            for (int p = 0; p < P; ++p) {
                double *row = Sh + (long)p * N;
                double acc = 0.0;
                for (int n = 0; n < N; ++n) {
                    double s = dA * row[n] + dth * xt[p] * Bt[n];
                    if (round_state_f32) s = (double)(float)s;
                    row[n] = s;
                    acc += Ct[n] * s;
                }
                y[(long)t * H * P + (long)h * P + p] = acc + (double)D[h] * xt[p];
            }
        }
    }
}

/* ------------------------------------------------------------- the block */

typedef struct {
    int hidden, n_heads, head_dim, d_state, n_groups, conv_k, group_size;
    double eps;
} nho_dims;

typedef struct {
    const uint16_t *norm_w;                                   /* [hidden] */
    const uint32_t *in_q; const uint16_t *in_s, *in_b;        /* [in_out][hidden] */
    const uint16_t *conv_w, *conv_b;                          /* [conv_dim][K], [conv_dim] */
    const float *dt_bias, *A_log, *D;                         /* [H] */
    const uint16_t *gnorm_w;                                  /* [d_inner] */
    const uint32_t *out_q; const uint16_t *out_s, *out_b;     /* [hidden][d_inner] */
} nho_weights;

/* Optional intermediates, each [B][T][width] (NULL to skip). */
typedef struct {
    double *u, *zxbcdt, *xc, *dt, *y, *o, *m;
} nho_debug;

static void maybe_round(double *v, long n, int mode)
{
    if (mode == NHO_CONTRACT)
        for (long i = 0; i < n; ++i) v[i] = round_bf16(v[i]);
}

/* One Mamba2 mixer block with pre-norm and residual over T positions of B
 * independent sequences:
 *   u  = RMSNorm(x) * norm_w                         (bf16 in CONTRACT)
 *   zxbcdt = W_in u, split z | x | B | C | dt_raw    (bf16)
 *   xc = silu(conv1d(x|B|C) + bias)                  (bf16)
 *   dt = softplus(dt_raw + dt_bias), A = -exp(A_log)
 *   y  = SSM recurrence over (xc_x, xc_B, xc_C, dt)  (bf16)
 *   o  = RMSNormGated(y, z) over groups of d_inner/n_groups (bf16)
 *   out = x + W_out o
 * x: [B][T][hidden] doubles (the caller widens bf16 or float32 input).
 * conv_state: [B][K-1][conv_dim] in/out, NULL means zero initial state and no
 * write-back.  ssm_state: [B][H][P][N] in/out (required).
 * out: [B][T][hidden] doubles, before any output rounding.
 * stepwise: in CONTRACT mode, round the SSM state to float32 after every
 * position (the per-position call stores it between positions). */
int nho_block(const nho_dims *d, const nho_weights *w, int B, int T, const double *x,
              double *conv_state, double *ssm_state, double *out, int mode, int stepwise,
              int nthreads, const nho_debug *dbg)
{
    const int Hd = d->hidden, H = d->n_heads, P = d->head_dim, N = d->d_state, G = d->n_groups;
    const int K = d->conv_k, gs = d->group_size;
    const int DI = H * P, CD = DI + 2 * G * N, NI = 2 * DI + 2 * G * N + H;
    if (T <= 0 || B <= 0) return -1;

    double *u = (double *)malloc(sizeof(double) * (size_t)T * Hd);
    double *zx = (double *)malloc(sizeof(double) * (size_t)T * NI);
    double *xc = (double *)malloc(sizeof(double) * (size_t)T * CD);
    double *dt = (double *)malloc(sizeof(double) * (size_t)T * H);
    double *A = (double *)malloc(sizeof(double) * (size_t)H);
    double *y = (double *)malloc(sizeof(double) * (size_t)T * DI);
    double *z = (double *)malloc(sizeof(double) * (size_t)T * DI);
    double *o = (double *)malloc(sizeof(double) * (size_t)T * DI);
    double *m = (double *)malloc(sizeof(double) * (size_t)T * Hd);
    double *cs_new = (double *)malloc(sizeof(double) * (size_t)(K - 1) * CD);

    for (int b = 0; b < B; ++b) {
        const double *xb = x + (long)b * T * Hd;
        double *cs = conv_state ? conv_state + (long)b * (K - 1) * CD : NULL;
        double *S = ssm_state + (long)b * H * P * N;

        nho_rmsnorm(xb, T, Hd, w->norm_w, d->eps, u);
        maybe_round(u, (long)T * Hd, mode);

        nho_w4_matvec(w->in_q, w->in_s, w->in_b, NI, Hd, gs, u, T, zx, nthreads);
        maybe_round(zx, (long)T * NI, mode);

        /* split: z [0,DI), xBC [DI, DI+CD), dt_raw [DI+CD, NI) */
        nho_conv1d(zx + DI, NI, T, CD, K, cs, w->conv_w, w->conv_b, xc, cs_new);
        maybe_round(xc, (long)T * CD, mode);
        if (cs) memcpy(cs, cs_new, sizeof(double) * (size_t)(K - 1) * CD);

        nho_discretize(zx + DI + CD, NI, T, H, w->dt_bias, w->A_log, dt, A);

        nho_ssm_recurrence(T, H, P, N, G, xc, CD, xc + DI, CD, xc + DI + G * N, CD, dt, A,
                           w->D, S, y, mode == NHO_CONTRACT && stepwise, nthreads);
        maybe_round(y, (long)T * DI, mode);
        if (mode == NHO_CONTRACT && !stepwise)
            for (long i = 0; i < (long)H * P * N; ++i) S[i] = (double)(float)S[i];

        for (int t = 0; t < T; ++t) memcpy(z + (long)t * DI, zx + (long)t * NI, sizeof(double) * DI);
        nho_rmsnorm_gated(y, z, T, DI, DI / G, w->gnorm_w, d->eps, o);
        maybe_round(o, (long)T * DI, mode);

        nho_w4_matvec(w->out_q, w->out_s, w->out_b, Hd, DI, gs, o, T, m, nthreads);
        for (long i = 0; i < (long)T * Hd; ++i) out[(long)b * T * Hd + i] = xb[i] + m[i];

        if (dbg) {
#define DUMP(field, src, width) \
    if (dbg->field) memcpy(dbg->field + (long)b * T * (width), src, sizeof(double) * (size_t)T * (width))
            DUMP(u, u, Hd);
            DUMP(zxbcdt, zx, NI);
            DUMP(xc, xc, CD);
            DUMP(dt, dt, H);
            DUMP(y, y, DI);
            DUMP(o, o, DI);
            DUMP(m, m, Hd);
#undef DUMP
        }
    }
    free(u); free(zx); free(xc); free(dt); free(A); free(y); free(z); free(o); free(m); free(cs_new);
    return 0;
}

int nho_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
