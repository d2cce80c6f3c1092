/*
 * srwm_oracle.c -- plain CPU oracle of the SRWM forward recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the independent checker of the GPU
 * library; it shares no code, header, table or helper with it.  Only tests/,
 * __graft_entry__.smoke() and bench.py's cpu_baseline leg may load it.  The
 * product path never calls it and has no CPU fallback.
 *
 * What it computes (the plain definition, evaluated with one scalar loop per
 * formula, in float64):
 *
 *   Self-referential weight matrix, 4-learning-rate, multi-head.
 *   Source pages:
 *   [ACL]  "Metalearning Continual Learning Algorithms -- part 2/5",
 *          Sec. 2.3 SRWM dynamics, Eq. (1)-(3), and the paragraph
 *          "4-learning-rate version", Eq. (4)-(5).
 *   [SRWM] review page "SRWM: 让权重矩阵学习修改自身" of Irie et al.,
 *          "A Modern Self-Referential Weight Matrix That Learns to Modify
 *          Itself" (ICML 2022): Sec. 2.2 (symbol table, output timing),
 *          Sec. 2.3 (delta-rule intuition, worked example),
 *          Sec. 2.4 (four row blocks, multi-head, input activation),
 *          Sec. 2.5 (W0 is the trained initial program).
 *
 *   Per (sequence b, head h) the state W is an m x d_in matrix,
 *   m = d_out + 2*d_in + 4 (4 learning rates), with row blocks [W^y; W^k; W^q; W^beta]
 *   ([ACL] 4-lr paragraph; [SRWM] Sec. 2.4).  Every unit starts from the
 *   shared W0[h] ([ACL] after Eq. (3); [SRWM] Sec. 2.5).  For t = 1..T:
 *
 *     u      = x_t, or softmax(x_t) when the input activation is on
 *              ([ACL] after Eq. (3); [SRWM] Sec. 2.4 last paragraph)
 *     z      = W u = [y_t, k_t, q_t, beta_t]          [ACL] Eq. (1)
 *     y_t    = z[0:d_out], taken from W_{t-1}         [SRWM] Sec. 2.2
 *     kh, qh = softmax(k_t), softmax(q_t)             [ACL] Eq. (2), phi
 *     g      = sigmoid(beta_t), beta_t in R^4          [ACL] Eq. (4)-(5)
 *     v      = W qh,  vb = W kh  (both with W_{t-1})  [ACL] Eq. (2), (4)
 *     W     += eta_i (v_i - vb_i) kh^T, eta_i = g[block(i)]
 *                                                     [ACL] Eq. (3), (5)
 *
 *   The block order of the gate vector is (y, k, q, beta) as the 4-lr
 *   paragraph lists the sub-blocks.  Eq. (3) as extracted has its bracket
 *   pair swapped ("sigma( CLOSE ... OPEN beta_t )"); it is read as
 *   sigma(beta_t) (v_t - vb_t) outer phi(k_t), the only reading whose
 *   shapes agree, and the one the [SRWM] Sec. 2.1 prose spells out.
 *
 *   With one learning rate ([ACL] Eq. (1)-(3) as first written,
 *   m = d_out + 2*d_in + 1) the single sigmoid(beta_t) gates every row.
 *
 *   Options beyond the shared-W0 forward ([SRWM] Sec. 3.3 and 4.5: the RL
 *   state persists across truncation windows, and resetting it every 50
 *   steps is the ablation that loses the benefit):
 *     - a per-sequence initial state W0[b][h] instead of the shared W0[h];
 *     - reset_interval R > 0: at every step t > 0 with t % R == 0 the state
 *       returns to the initial matrix before the step is taken.
 *
 * Also here: DeltaNet and SR-DeltaNet ([SRWM] Sec. 2.1 and Appendix C.1),
 * stated with their readings at the end of the file.
 *
 * softmax(s)_j = exp(s_j - max s) / sum_l exp(s_l - max s);
 * sigmoid(z)   = 1/(1+exp(-z)) for z >= 0, exp(z)/(1+exp(z)) otherwise.
 * Neither page fixes a temperature or scale; none is applied.
 *
 * Pins (tests/test_oracle_pins.py): the worked example of [SRWM] Sec. 2.3,
 * the W0 = 0 fixed point of [SRWM] Sec. 2.5, the reread identity of
 * [SRWM] Sec. 2.3, the address-norm bounds of [SRWM] Sec. 2.3, an
 * independent d = 2 closed-form expansion, and derived invariants.  No
 * function here is "parity unpinned".
 *
 * Built twice from this one source: REAL = double (the oracle, symbols
 * srwm_oracle_*) and REAL = float (symbols srwm_oracle_f32_*), the latter
 * only to measure how far any float32 evaluation drifts from float64.
 * Compile with -ffp-contract=off so that no multiply-add is fused.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef ORACLE_FLOAT
typedef float real;
#define FN(name) srwm_oracle_f32_##name
#define EXP expf
#else
typedef double real;
#define FN(name) srwm_oracle_##name
#define EXP exp
#endif

/* softmax over n entries: exp(s_j - max) / sum exp(s_l - max). */
static void softmax(const real* s, int n, real* out)
{
    real mx = s[0];
    for (int j = 1; j < n; ++j)
        if (s[j] > mx) mx = s[j];
    real sum = 0;
    for (int j = 0; j < n; ++j) {
        out[j] = EXP(s[j] - mx);
        sum += out[j];
    }
    for (int j = 0; j < n; ++j) out[j] = out[j] / sum;
}

static real sigmoid(real z)
{
    if (z >= 0) return (real)1 / ((real)1 + EXP(-z));
    real e = EXP(z);
    return e / ((real)1 + e);
}

/* Block of row i in the 4-lr split [y | k | q | beta]: 0, 1, 2 or 3. */
static int row_block(int i, int d_in, int d_out)
{
    if (i < d_out) return 0;
    if (i < d_out + d_in) return 1;
    if (i < d_out + 2 * d_in) return 2;
    return 3;
}

/* Learning-rate index of row i: its block with four rates, 0 with one. */
static int rate_of_row(int i, int d_in, int d_out, int n_lr)
{
    return n_lr == 1 ? 0 : row_block(i, d_in, d_out);
}

/*
 * Delta-rule self-update with the addresses given ([ACL] Eq. (2)-(3) and
 * (4)-(5); [SRWM] Sec. 2.3):
 *   v  = W qh,  vb = W kh       (reads of the current W)
 *   W  = W + eta_i (v_i - vb_i) kh_j    for every row i and column j
 * W is rows x d_in, row-major.  eta holds one learning rate per row.
 * v_out / vb_out (length rows) receive the two reads when non-NULL.
 */
void FN(delta_update)(real* W, int rows, int d_in, const real* kh,
                      const real* qh, const real* eta, real* v_out,
                      real* vb_out)
{
    for (int i = 0; i < rows; ++i) {
        real* w = W + (size_t)i * d_in;
        real v = 0, vb = 0;
        for (int j = 0; j < d_in; ++j) v += w[j] * qh[j];
        for (int j = 0; j < d_in; ++j) vb += w[j] * kh[j];
        if (v_out) v_out[i] = v;
        if (vb_out) vb_out[i] = vb;
        real a = eta[i] * (v - vb);
        for (int j = 0; j < d_in; ++j) w[j] = w[j] + a * kh[j];
    }
}

/*
 * One step of the recurrence on one unit.  W (m x d_in, m = d_out + 2*d_in +
 * n_lr, n_lr = 4 or 1) is updated in place from W_{t-1} to W_t.  x_t has d_in
 * entries; y_t receives d_out entries.  Every other pointer may be NULL; when
 * given it receives the step's intermediate: u (d_in), z (m), kh, qh (d_in),
 * g (n_lr), v, vb (m).
 */
void FN(step)(real* W, int d_in, int d_out, int n_lr, const real* x_t,
              int apply_input_softmax, real* y_t, real* u_out, real* z_out,
              real* kh_out, real* qh_out, real* g_out, real* v_out,
              real* vb_out)
{
    const int m = d_out + 2 * d_in + n_lr;
    real* buf = (real*)malloc(sizeof(real) * (size_t)(3 * d_in + 2 * m + 4));
    real* u = buf;
    real* kh = u + d_in;
    real* qh = kh + d_in;
    real* z = qh + d_in;
    real* eta = z + m;
    real* g = eta + m;

    /* Input of Eq. (1): x_t itself, or softmax(x_t) in the RL variant. */
    if (apply_input_softmax)
        softmax(x_t, d_in, u);
    else
        for (int j = 0; j < d_in; ++j) u[j] = x_t[j];

    /* Eq. (1): [y_t, k_t, q_t, beta_t] = W_{t-1} u. */
    for (int i = 0; i < m; ++i) {
        real s = 0;
        for (int j = 0; j < d_in; ++j) s += W[(size_t)i * d_in + j] * u[j];
        z[i] = s;
    }
    /* The output comes from W_{t-1}, before the self-update. */
    for (int i = 0; i < d_out; ++i) y_t[i] = z[i];

    /* phi = softmax on key and query; sigma on the rate logit(s). */
    softmax(z + d_out, d_in, kh);
    softmax(z + d_out + d_in, d_in, qh);
    for (int c = 0; c < n_lr; ++c) g[c] = sigmoid(z[m - n_lr + c]);

    /* Eq. (5): every row block uses its own learning rate (Eq. (3): one). */
    for (int i = 0; i < m; ++i) eta[i] = g[rate_of_row(i, d_in, d_out, n_lr)];

    /* Eq. (2) reads and Eq. (3) rank-one delta update. */
    FN(delta_update)(W, m, d_in, kh, qh, eta, v_out, vb_out);

    if (u_out) memcpy(u_out, u, sizeof(real) * (size_t)d_in);
    if (z_out) memcpy(z_out, z, sizeof(real) * (size_t)m);
    if (kh_out) memcpy(kh_out, kh, sizeof(real) * (size_t)d_in);
    if (qh_out) memcpy(qh_out, qh, sizeof(real) * (size_t)d_in);
    if (g_out) memcpy(g_out, g, sizeof(real) * (size_t)n_lr);
    free(buf);
}

/*
 * Whole sequence for one unit.  x: T rows of d_in at row stride x_ld;
 * y: T rows of d_out at row stride y_ld; W0 and W_T: m x d_in (W_T may be
 * NULL).  T = 0 leaves y untouched and copies W0 to W_T.  reset_interval
 * R > 0 returns the state to W0 before every step t > 0 with t % R == 0.
 */
void FN(unit)(const real* x, ptrdiff_t x_ld, const real* W0, real* y,
              ptrdiff_t y_ld, real* W_T, long T, int d_in, int d_out,
              int n_lr, int apply_input_softmax, long reset_interval)
{
    const int m = d_out + 2 * d_in + n_lr;
    const size_t n = (size_t)m * d_in;
    real* W = (real*)malloc(sizeof(real) * n);
    memcpy(W, W0, sizeof(real) * n);
    for (long t = 0; t < T; ++t) {
        if (reset_interval > 0 && t > 0 && t % reset_interval == 0)
            memcpy(W, W0, sizeof(real) * n);
        FN(step)(W, d_in, d_out, n_lr, x + t * x_ld, apply_input_softmax,
                 y + t * y_ld, NULL, NULL, NULL, NULL, NULL, NULL, NULL);
    }
    if (W_T) memcpy(W_T, W, sizeof(real) * n);
    free(W);
}

/* Batched forward: x[B][T][H][d_in], W0[H][m][d_in] (or W0[B][H][m][d_in]
 * with w0_per_sequence), y[B][T][H][d_out], W_T[B][H][m][d_in] (or NULL).
 * The (b, h) units are independent ([SRWM] Sec. 2.4: each head runs on its
 * own); they are spread over nthreads POSIX threads, each unit evaluated
 * sequentially in t. */
typedef struct {
    const real* x;
    const real* W0;
    real* y;
    real* W_T;
    long B, T, H;
    int d_in, d_out, n_lr, flag, w0_per_seq;
    long reset_interval;
    long first, stride;
} job_t;

static void* run_job(void* p)
{
    const job_t* jb = (const job_t*)p;
    const long m = jb->d_out + 2L * jb->d_in + jb->n_lr;
    for (long u = jb->first; u < jb->B * jb->H; u += jb->stride) {
        const long b = u / jb->H, h = u % jb->H;
        const real* x = jb->x + (b * jb->T * jb->H + h) * jb->d_in;
        real* y = jb->y + (b * jb->T * jb->H + h) * jb->d_out;
        real* wt = jb->W_T ? jb->W_T + (b * jb->H + h) * m * jb->d_in : NULL;
        const real* w0 = jb->W0 + (jb->w0_per_seq ? u : h) * m * jb->d_in;
        FN(unit)(x, jb->H * jb->d_in, w0, y, jb->H * jb->d_out, wt, jb->T,
                 jb->d_in, jb->d_out, jb->n_lr, jb->flag, jb->reset_interval);
    }
    return NULL;
}

int FN(forward)(const real* x, const real* W0, real* y, real* W_T, long B,
                long T, long H, int d_in, int d_out, int n_lr,
                int apply_input_softmax, int w0_per_sequence,
                long reset_interval, int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || d_in < 1 || d_out < 1) return -1;
    if (n_lr != 1 && n_lr != 4) return -1;
    if (reset_interval < 0) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    job_t jobs[256];
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = (job_t){x, W0, y, W_T, B, T, H, d_in, d_out, n_lr,
                          apply_input_softmax, w0_per_sequence,
                          reset_interval, i, nthreads};
    }
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, run_job, &jobs[i]) != 0) break;
        started = i;
    }
    run_job(&jobs[0]);
    for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
    /* Threads that could not start: run their share here. */
    for (int i = started + 1; i < nthreads; ++i) run_job(&jobs[i]);
    return 0;
}

/* ------------------------------------------------------------------------
 * DeltaNet and SR-DeltaNet.
 *
 * DeltaNet ([SRWM] Sec. 2.1, the page's Eq. (1)-(4)): a slow matrix maps the
 * input to a key, a value, a query and a rate logit; a separate fast matrix
 * F (d_v x d_key per head, usually starting from zero) gets a delta write at
 * the key and is then queried.  Per step, with the projection
 * p = [k (d_key); v (d_v); q (d_key); beta (1)] (the order the page names
 * them in):
 *   kh = softmax(k), qh = softmax(q), g = sigmoid(beta)
 *   vb = F kh                       what the key address holds now
 *   F  = F + g (v - vb) kh^T        the delta write
 *   y  = F qh                       the query reads the matrix AFTER the write
 * (the page stresses that DeltaNet queries the updated matrix, while the
 * SRWM's output comes from the matrix before its update).  The slow
 * projection is full width: p for head h is rows [h*P, (h+1)*P) of
 * Wslow[H*P][D] times the whole input x_t (D = H*d_in), P = d_v + 2*d_key + 1
 * (the page contrasts DeltaNet's (D, D) key projection with the SRWM's
 * per-head (H, d, d)).
 *
 * SR-DeltaNet ([SRWM] Appendix C.1): the slow projection is replaced by an
 * SRWM (per head, d_out = P output rows, its own self-modification as
 * above), and the fast matrix is kept: the SRWM's output y^SR_t, taken from
 * its matrix before its update, is the projection p of the fast step.
 * ------------------------------------------------------------------------ */

/* One fast-matrix step.  F (d_v x d_key, row-major) is updated in place; y
 * (d_v) receives the query after the write.  kh_out, qh_out (d_key), g_out
 * (1) and vb_out (d_v) receive the step's intermediates when non-NULL. */
void FN(fast_step)(real* F, int d_key, int d_v, const real* p, real* y,
                   real* kh_out, real* qh_out, real* g_out, real* vb_out)
{
    real* buf = (real*)malloc(sizeof(real) * (size_t)(2 * d_key + d_v));
    real* kh = buf;
    real* qh = kh + d_key;
    real* vb = qh + d_key;
    const real* k = p;
    const real* v = p + d_key;
    const real* q = p + d_key + d_v;
    softmax(k, d_key, kh);
    softmax(q, d_key, qh);
    const real g = sigmoid(p[2 * d_key + d_v]);
    /* read at the key address */
    for (int i = 0; i < d_v; ++i) {
        real s = 0;
        for (int j = 0; j < d_key; ++j) s += F[(size_t)i * d_key + j] * kh[j];
        vb[i] = s;
    }
    /* delta write */
    for (int i = 0; i < d_v; ++i) {
        const real a = g * (v[i] - vb[i]);
        for (int j = 0; j < d_key; ++j) F[(size_t)i * d_key + j] = F[(size_t)i * d_key + j] + a * kh[j];
    }
    /* query the updated matrix */
    for (int i = 0; i < d_v; ++i) {
        real s = 0;
        for (int j = 0; j < d_key; ++j) s += F[(size_t)i * d_key + j] * qh[j];
        y[i] = s;
    }
    if (kh_out) memcpy(kh_out, kh, sizeof(real) * (size_t)d_key);
    if (qh_out) memcpy(qh_out, qh, sizeof(real) * (size_t)d_key);
    if (g_out) g_out[0] = g;
    if (vb_out) memcpy(vb_out, vb, sizeof(real) * (size_t)d_v);
    free(buf);
}

typedef struct {
    int kind; /* 0 DeltaNet, 1 SR-DeltaNet */
    const real* x;
    const real* Wp; /* DeltaNet: Wslow[H*P][D]; SR-DeltaNet: W0[H][m][d_in] */
    const real* F0; /* NULL (zero) or [B][H][d_v][d_key] */
    real* y;
    real* W_T; /* SR-DeltaNet only, or NULL */
    real* F_T;
    long B, T, H;
    int d_in, d_key, d_v, n_lr, flag;
    long first, stride;
} fjob_t;

static void* run_fjob(void* pv)
{
    const fjob_t* jb = (const fjob_t*)pv;
    const int P = jb->d_v + 2 * jb->d_key + 1;
    const long D = jb->H * jb->d_in;
    const size_t nf = (size_t)jb->d_v * jb->d_key;
    const int m = P + 2 * jb->d_in + jb->n_lr;
    real* F = (real*)malloc(sizeof(real) * nf);
    real* p = (real*)malloc(sizeof(real) * (size_t)P);
    real* W = jb->kind == 1 ? (real*)malloc(sizeof(real) * (size_t)m * jb->d_in) : NULL;
    for (long u = jb->first; u < jb->B * jb->H; u += jb->stride) {
        const long b = u / jb->H, h = u % jb->H;
        if (jb->F0)
            memcpy(F, jb->F0 + u * nf, sizeof(real) * nf);
        else
            memset(F, 0, sizeof(real) * nf);
        if (W) memcpy(W, jb->Wp + h * (long)m * jb->d_in, sizeof(real) * (size_t)m * jb->d_in);
        for (long t = 0; t < jb->T; ++t) {
            const real* xt = jb->x + (b * jb->T + t) * D; /* x[b][t][:][:] */
            if (jb->kind == 0) {
                /* slow projection of the whole input onto head h's rows */
                const real* ws = jb->Wp + h * (long)P * D;
                for (int i = 0; i < P; ++i) {
                    real s = 0;
                    for (long j = 0; j < D; ++j) s += ws[i * D + j] * xt[j];
                    p[i] = s;
                }
            } else {
                /* the SRWM of head h produces the projection and modifies itself */
                FN(step)(W, jb->d_in, P, jb->n_lr, xt + h * jb->d_in, jb->flag, p,
                         NULL, NULL, NULL, NULL, NULL, NULL, NULL);
            }
            FN(fast_step)(F, jb->d_key, jb->d_v, p, jb->y + ((b * jb->T + t) * jb->H + h) * jb->d_v,
                          NULL, NULL, NULL, NULL);
        }
        if (jb->F_T) memcpy(jb->F_T + u * nf, F, sizeof(real) * nf);
        if (W && jb->W_T) memcpy(jb->W_T + u * (long)m * jb->d_in, W, sizeof(real) * (size_t)m * jb->d_in);
    }
    free(F);
    free(p);
    free(W);
    return NULL;
}

static int run_fjobs(fjob_t base, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    fjob_t jobs[256];
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = base;
        jobs[i].first = i;
        jobs[i].stride = nthreads;
    }
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, run_fjob, &jobs[i]) != 0) break;
        started = i;
    }
    run_fjob(&jobs[0]);
    for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
    for (int i = started + 1; i < nthreads; ++i) run_fjob(&jobs[i]);
    return 0;
}

/* DeltaNet forward: x[B][T][H][d_in], Wslow[H*P][H*d_in], F0 NULL or
 * [B][H][d_v][d_key], y[B][T][H][d_v], F_T NULL or [B][H][d_v][d_key]. */
int FN(deltanet_forward)(const real* x, const real* Wslow, const real* F0, real* y, real* F_T,
                         long B, long T, long H, int d_in, int d_key, int d_v, int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || d_in < 1 || d_key < 1 || d_v < 1) return -1;
    fjob_t base = {0, x, Wslow, F0, y, NULL, F_T, B, T, H, d_in, d_key, d_v, 4, 0, 0, 1};
    return run_fjobs(base, nthreads);
}

/* SR-DeltaNet forward: the SRWM W0[H][m][d_in], m = P + 2*d_in + n_lr,
 * P = d_v + 2*d_key + 1; W_T NULL or [B][H][m][d_in]; the rest as DeltaNet. */
int FN(srdeltanet_forward)(const real* x, const real* W0, const real* F0, real* y, real* W_T,
                           real* F_T, long B, long T, long H, int d_in, int d_key, int d_v,
                           int n_lr, int apply_input_softmax, int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || d_in < 1 || d_key < 1 || d_v < 1) return -1;
    if (n_lr != 1 && n_lr != 4) return -1;
    fjob_t base = {1, x, W0, F0, y, W_T, F_T, B, T, H, d_in, d_key, d_v, n_lr, apply_input_softmax, 0, 1};
    return run_fjobs(base, nthreads);
}
