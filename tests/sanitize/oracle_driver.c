/*
 * oracle_driver.c -- runs the float64 (and float32) CPU oracle over the
 * shapes its pins use, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py).  Every call must
 * return 0 and every output must be finite; the sanitizers report any
 * out-of-bounds access, leak or undefined operation and abort the run.
 * Test infrastructure: it declares the oracle's exported functions itself
 * and shares nothing with the GPU library.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int srwm_oracle_forward(const double* x, const double* W0, double* y, double* W_T, long B, long T, long H,
                        int d_in, int d_out, int n_lr, int apply_input_softmax, int w0_per_sequence,
                        long reset_interval, int nthreads);
int srwm_oracle_f32_forward(const float* x, const float* W0, float* y, float* W_T, long B, long T, long H,
                            int d_in, int d_out, int n_lr, int apply_input_softmax, int w0_per_sequence,
                            long reset_interval, int nthreads);
void srwm_oracle_step(double* W, int d_in, int d_out, int n_lr, const double* x_t, int apply_input_softmax,
                      double* y_t, double* u_out, double* z_out, double* kh_out, double* qh_out, double* g_out,
                      double* v_out, double* vb_out);
void srwm_oracle_delta_update(double* W, int rows, int d_in, const double* kh, const double* qh,
                              const double* eta, double* v_out, double* vb_out);
void srwm_oracle_fast_step(double* F, int d_key, int d_v, const double* p, double* y, double* kh_out,
                           double* qh_out, double* g_out, double* vb_out);
int srwm_oracle_deltanet_forward(const double* x, const double* Wslow, const double* F0, double* y,
                                 double* F_T, long B, long T, long H, int d_in, int d_key, int d_v,
                                 int nthreads);
int srwm_oracle_srdeltanet_forward(const double* x, const double* W0, const double* F0, double* y,
                                   double* W_T, double* F_T, long B, long T, long H, int d_in, int d_key,
                                   int d_v, int n_lr, int apply_input_softmax, int nthreads);

static unsigned long long rng_state = 0x9E3779B97F4A7C15ull;

static double uniform_pm1(void)
{
    /* xorshift64*: inputs only, no part of the method */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 2685821657736338717ull) >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

/* exactly n doubles on the heap (so an access past the end is caught) */
static double* fill(size_t n, double scale)
{
    double* p = (double*)malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = scale * uniform_pm1();
    return p;
}

static int failures = 0;

static void check_finite(const char* what, const double* p, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) {
            fprintf(stderr, "%s: non-finite value at %zu\n", what, i);
            ++failures;
            return;
        }
}

static void run_forward(long B, long T, long H, int d_in, int d_out, int n_lr, int flag, int per_seq,
                        long reset, int threads)
{
    const int m = d_out + 2 * d_in + n_lr;
    const size_t nx = (size_t)B * T * H * d_in, ny = (size_t)B * T * H * d_out;
    const size_t nw0 = (size_t)(per_seq ? B * H : H) * m * d_in, nst = (size_t)B * H * m * d_in;
    double* x = fill(nx, 2.0);
    double* W0 = fill(nw0, 1.0 / sqrt((double)d_in));
    double* y = fill(ny, 0.0);
    double* WT = fill(nst, 0.0);
    if (srwm_oracle_forward(x, W0, y, WT, B, T, H, d_in, d_out, n_lr, flag, per_seq, reset, threads) != 0) {
        fprintf(stderr, "forward rejected a valid call\n");
        ++failures;
    }
    check_finite("y", y, ny);
    check_finite("W_T", WT, nst);
    /* the float32 evaluation of the same definition */
    float* xf = (float*)malloc((nx ? nx : 1) * sizeof(float));
    float* wf = (float*)malloc((nw0 ? nw0 : 1) * sizeof(float));
    float* yf = (float*)malloc((ny ? ny : 1) * sizeof(float));
    float* tf = (float*)malloc((nst ? nst : 1) * sizeof(float));
    for (size_t i = 0; i < nx; ++i) xf[i] = (float)x[i];
    for (size_t i = 0; i < nw0; ++i) wf[i] = (float)W0[i];
    if (srwm_oracle_f32_forward(xf, wf, yf, tf, B, T, H, d_in, d_out, n_lr, flag, per_seq, reset, threads) != 0)
        ++failures;
    free(xf), free(wf), free(yf), free(tf);
    free(x), free(W0), free(y), free(WT);
}

int main(void)
{
    /* the pins' shapes: d = 1, 2, (3, 5), 8, 16, 64, 128; T = 0, 1, 3, 17; both
       flags, both rate counts, per-sequence initial states, resets */
    static const int dims[][2] = {{1, 1}, {2, 2}, {3, 5}, {2, 1}, {8, 8}, {8, 16}, {16, 8}, {16, 16},
                                  {64, 64}, {128, 128}};
    static const long Ts[] = {0, 1, 3, 17};
    for (size_t i = 0; i < sizeof(dims) / sizeof(dims[0]); ++i)
        for (size_t j = 0; j < sizeof(Ts) / sizeof(Ts[0]); ++j)
            for (int flag = 0; flag < 2; ++flag)
                for (int lr = 0; lr < 2; ++lr) {
                    const int d_in = dims[i][0], d_out = dims[i][1];
                    const long T = dims[i][0] >= 64 ? (Ts[j] > 3 ? 3 : Ts[j]) : Ts[j];
                    run_forward(2, T, 3, d_in, d_out, lr ? 1 : 4, flag, 0, 0, 1 + (int)(j % 3));
                    run_forward(2, T, 2, d_in, d_out, lr ? 1 : 4, flag, 1, 2, 2);
                }
    /* invalid arguments are refused, not read */
    if (srwm_oracle_forward(NULL, NULL, NULL, NULL, -1, 1, 1, 2, 2, 4, 0, 0, 0, 1) == 0) ++failures;
    if (srwm_oracle_forward(NULL, NULL, NULL, NULL, 1, 1, 1, 2, 2, 3, 0, 0, 0, 1) == 0) ++failures;

    /* one step with every intermediate, and the given-address update */
    {
        const int d_in = 5, d_out = 3, n_lr = 4, m = d_out + 2 * d_in + n_lr;
        double* W = fill((size_t)m * d_in, 0.5);
        double* x = fill(d_in, 1.0);
        double *y = fill(d_out, 0), *u = fill(d_in, 0), *z = fill(m, 0), *kh = fill(d_in, 0);
        double *qh = fill(d_in, 0), *g = fill(n_lr, 0), *v = fill(m, 0), *vb = fill(m, 0);
        srwm_oracle_step(W, d_in, d_out, n_lr, x, 1, y, u, z, kh, qh, g, v, vb);
        check_finite("step", W, (size_t)m * d_in);
        double* eta = fill(m, 0.5);
        srwm_oracle_delta_update(W, m, d_in, kh, qh, eta, v, vb);
        srwm_oracle_delta_update(W, m, d_in, kh, qh, eta, NULL, NULL);
        check_finite("delta_update", W, (size_t)m * d_in);
        free(W), free(x), free(y), free(u), free(z), free(kh), free(qh), free(g), free(v), free(vb), free(eta);
    }
    /* DeltaNet and SR-DeltaNet */
    {
        const long B = 2, T = 9, H = 2;
        const int d_in = 4, d_key = 3, d_v = 5, P = d_v + 2 * d_key + 1;
        double* x = fill((size_t)B * T * H * d_in, 1.0);
        double* Ws = fill((size_t)H * P * H * d_in, 0.5);
        double* F0 = fill((size_t)B * H * d_v * d_key, 0.5);
        double* y = fill((size_t)B * T * H * d_v, 0);
        double* FT = fill((size_t)B * H * d_v * d_key, 0);
        if (srwm_oracle_deltanet_forward(x, Ws, F0, y, FT, B, T, H, d_in, d_key, d_v, 2) != 0) ++failures;
        if (srwm_oracle_deltanet_forward(x, Ws, NULL, y, NULL, B, T, H, d_in, d_key, d_v, 3) != 0) ++failures;
        check_finite("deltanet y", y, (size_t)B * T * H * d_v);
        for (int n_lr = 1; n_lr <= 4; n_lr += 3) {
            const int m = P + 2 * d_in + n_lr;
            double* W0 = fill((size_t)H * m * d_in, 0.5);
            double* WT = fill((size_t)B * H * m * d_in, 0);
            if (srwm_oracle_srdeltanet_forward(x, W0, F0, y, WT, FT, B, T, H, d_in, d_key, d_v, n_lr, 1, 2) != 0)
                ++failures;
            if (srwm_oracle_srdeltanet_forward(x, W0, NULL, y, NULL, NULL, B, T, H, d_in, d_key, d_v, n_lr, 0, 1) != 0)
                ++failures;
            check_finite("srdeltanet y", y, (size_t)B * T * H * d_v);
            free(W0), free(WT);
        }
        double* p = fill(P, 1.0);
        double *yv = fill(d_v, 0), *kh = fill(d_key, 0), *qh = fill(d_key, 0), *g = fill(1, 0), *vb = fill(d_v, 0);
        double* F = fill((size_t)d_v * d_key, 0.5);
        srwm_oracle_fast_step(F, d_key, d_v, p, yv, kh, qh, g, vb);
        srwm_oracle_fast_step(F, d_key, d_v, p, yv, NULL, NULL, NULL, NULL);
        check_finite("fast_step", F, (size_t)d_v * d_key);
        free(p), free(yv), free(kh), free(qh), free(g), free(vb), free(F);
        free(x), free(Ws), free(F0), free(y), free(FT);
    }
    if (failures) {
        fprintf(stderr, "oracle_driver: %d failures\n", failures);
        return 1;
    }
    printf("oracle_driver: ok\n");
    return 0;
}
