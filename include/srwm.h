/*
 * srwm.h -- C ABI of libsrwm on AMD Instinct MI355X (gfx950): the forward
 * recurrence of the multi-head self-referential weight matrix (SRWM), its
 * backward pass (memory-efficient BPTT), and the DeltaNet / SR-DeltaNet
 * fast-weight programmers (declared further down).
 *
 * The operation (sources: "Metalearning Continual Learning Algorithms --
 * part 2/5", Sec. 2.3 Eq. (1)-(3) and the "4-learning-rate version"
 * paragraph, Eq. (4)-(5); review page "SRWM: 让权重矩阵学习修改自身" of
 * "A Modern Self-Referential Weight Matrix That Learns to Modify Itself",
 * Sec. 2.2-2.5, 3.3, 4.5):
 *
 *   Every (sequence b, head h) is an independent unit with an m x d_in state
 *   W, m = d_out + 2*d_in + n_lr, row blocks [W^y; W^k; W^q; W^beta] with
 *   n_lr = 4 rate rows (Eq. (4)-(5)) or 1 (Eq. (1)-(3)).  All units start
 *   from the initial matrix W0[h] (shared over b), or W0[b][h].  For t = 0..T-1:
 *     u     = x[b,t,h,:]            (softmax(x[b,t,h,:]) if apply_input_softmax)
 *     z     = W u = [y_t, k_t, q_t, beta_t]                      Eq. (1)
 *     y[b,t,h,:] = z[0:d_out]        (from W before this step's update)
 *     kh    = softmax(k_t), qh = softmax(q_t), g = sigmoid(beta_t)
 *     W[i,:] += g[rate(i)] * ((W qh)_i - (W kh)_i) * kh      Eq. (2)-(5)
 *   with rate(i) = 0, 1, 2, 3 for the y, k, q, beta rows (always 0 when
 *   n_lr = 1).  W_T[b,h] = W after step T-1.
 *
 * Conventions shared by every entry point:
 *   - Layout: dense, row-major, contiguous.  x[B][T][H][d_in],
 *     W0[H][m][d_in] (or [B][H][m][d_in]), y[B][T][H][d_out],
 *     W_T[B][H][m][d_in].
 *   - Dtypes: x and y share io_dtype (SRWM_IO_F32 = float32, SRWM_IO_BF16 =
 *     bfloat16 bits in uint16).  W0 and W_T are always float32; the state and
 *     all arithmetic are float32.  bf16 x is widened exactly; y is rounded to
 *     bf16 with round-to-nearest-even.
 *   - Memory: every pointer is a device pointer (hipMalloc'd or equivalent),
 *     16-byte aligned (SRWM_ERR_ARG otherwise) and owned by the caller.  The
 *     library allocates no memory, frees nothing, keeps no pointer after the
 *     call returns and holds no mutable global state: concurrent calls on
 *     different streams are safe.  (An SR-DeltaNet call given a second stream
 *     creates and destroys a HIP event; see there.  srwm_backward_noalloc
 *     uses a scratch array the library holds per GPU; see there.)
 *   - Execution: asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  The return code covers argument validation and the launch
 *     only; a fault during execution surfaces at the next synchronisation.
 *   - Plain C types at the boundary: every `int io_dtype` holds a
 *     srwm_io_dtype_t value and every `void* stream` (and `aux_stream`) is a
 *     hipStream_t passed as a pointer, so this header needs no HIP header and
 *     a caller that has none (ctypes, another language's FFI) can still call
 *     it.  The ABI is the same as with the enum and hipStream_t spelled out.
 *   - Alignment: the kernels move 16-byte pieces, so every buffer must start
 *     on a 16-byte boundary.  A hipMalloc'd pointer always does; a view at an
 *     odd offset into a larger buffer may not, and is refused with
 *     SRWM_ERR_ARG (the Python binding names the offending tensor).
 *   - Errors: negative codes below; srwm_strerror() names them.  Validation
 *     happens before any HIP call, so an invalid call touches no device.
 */
#ifndef SRWM_H
#define SRWM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SRWM_VERSION_MAJOR 0
#define SRWM_VERSION_MINOR 8
#define SRWM_VERSION_PATCH 0

typedef enum { SRWM_IO_F32 = 0, SRWM_IO_BF16 = 1 } srwm_io_dtype_t;

enum {
    SRWM_OK = 0,
    SRWM_ERR_NULL = -1,        /* a required pointer is NULL                       */
    SRWM_ERR_SHAPE = -2,       /* negative size, m != d_out+2*d_in+n_lr, overflow   */
    SRWM_ERR_UNSUPPORTED = -3, /* no kernel built for (d_in, d_out, io_dtype, n_lr) */
    SRWM_ERR_ALIAS = -4,       /* an output overlaps an input or the other output  */
    SRWM_ERR_HIP = -5,         /* the HIP runtime rejected the launch               */
    SRWM_ERR_ARG = -6,         /* other invalid argument (io_dtype, flag, n_lr,
                                  reset interval, variant, a pointer not 16-byte
                                  aligned)                                          */
    SRWM_ERR_SCRATCH = -7      /* srwm_backward_noalloc: one sequence's per-unit
                                  gradients exceed the library's scratch array   */
};

/*
 * srwm_forward -- run the whole recurrence for all B*H units, four learning
 * rates, shared W0.
 *
 *   x       [B][T][H][d_in]   io_dtype, device, read only
 *   W0      [H][m][d_in]      float32, device, read only, shared over b
 *   y       [B][T][H][d_out]  io_dtype, device, written (not read)
 *   W_T     [B][H][m][d_in]   float32, device, written; may be NULL
 *   m       must equal d_out + 2*d_in + 4 (checked)
 *   apply_input_softmax  0: Eq. (1) sees x_t (supervised/few-shot variant);
 *                        1: it sees softmax(x_t) (RL variant)
 *   stream  hipStream_t, or NULL
 *
 * Edge cases: B*H == 0 is a no-op returning SRWM_OK.  T == 0 leaves y
 * untouched and writes W_T[b,h] = W0[h].  NaN/Inf in x or W0 propagate; they
 * are not checked.  Outputs must not overlap inputs or each other
 * (SRWM_ERR_ALIAS).  Pointers may be NULL only when the tensor they address
 * is empty.  One step's row of x, H*d_in elements, may span at most 64 MiB
 * (SRWM_ERR_SHAPE beyond).  Returns SRWM_OK or a negative error code.
 */
int srwm_forward(const void* x, const float* W0, void* y, float* W_T,
                 int64_t B, int64_t T, int64_t H, int64_t d_in, int64_t d_out,
                 int64_t m, int io_dtype, int apply_input_softmax,
                 void* stream);

/*
 * srwm_forward_variant -- srwm_forward with an explicit kernel variant, for
 * tuning and for testing every variant against the same definition.
 * variant = -1 makes the automatic choice (identical to srwm_forward).
 * Otherwise `variant` indexes the list srwm_variant_info() reports; a
 * variant whose shape does not match the call gives SRWM_ERR_ARG.  Every
 * variant computes the same function; they differ in how a unit's state is
 * spread over lanes and in the order of the per-step passes.
 */
int srwm_forward_variant(const void* x, const float* W0, void* y, float* W_T,
                         int64_t B, int64_t T, int64_t H, int64_t d_in,
                         int64_t d_out, int64_t m, int io_dtype,
                         int apply_input_softmax, void* stream, int variant);

/*
 * Full argument set of srwm_forward_ex.  Fields as in srwm_forward, plus:
 *   n_lr             4: one learning rate per row block (Eq. (4)-(5));
 *                    1: one learning rate for every row (Eq. (1)-(3)).
 *                    m must equal d_out + 2*d_in + n_lr.
 *   w0_per_sequence  0: W0 is [H][m][d_in], shared over the batch;
 *                    1: W0 is [B][H][m][d_in], one initial state per unit
 *                    (for example the W_T of an earlier call: the state carry
 *                    across truncation windows of the review page, Sec. 3.3).
 *   reset_interval   0: never; R > 0: the state returns to the unit's initial
 *                    matrix before every step t > 0 with t % R == 0 (the
 *                    reset ablation of the review page, Sec. 4.5).  At most
 *                    INT32_MAX.
 *   variant          -1 for the automatic choice, else a srwm_variant_info
 *                    index.
 *   tape             NULL, or the backward tape (see srwm_backward).
 *   window_states    with a tape and R > 0: the state of each unit at the end
 *                    of every window but the last (the last one's is W_T),
 *                    [B][H][n_resets][m][d_in] float32 (out), n_resets =
 *                    (T - 1) / R, the number of resets the run performs
 *                    (0 when T <= R; then it may be NULL).  The backward pass
 *                    restarts each earlier window from it: a window's start is
 *                    the initial matrix, not the previous window's end, so
 *                    undoing updates cannot cross a reset.  Ignored otherwise.
 *   t_stride         0: x and y are [B][T][H][*]; S >= T: they are the steps
 *                    [t0, t0+T) of longer sequences laid out [B][S][H][*]
 *                    (x and y point at step t0 of sequence 0), so a run can
 *                    continue over time slices of one buffer without copies.
 *                    0 < S < T gives SRWM_ERR_SHAPE.  The tape and the window
 *                    states keep their own [B][H][T] layout.
 */
typedef struct srwm_forward_args {
    const void* x;
    const float* W0;
    void* y;
    float* W_T;
    int64_t B, T, H, d_in, d_out, m;
    int io_dtype;
    int apply_input_softmax;
    int n_lr;
    int w0_per_sequence;
    int64_t reset_interval;
    int variant;
    void* stream;
    float* tape;   /* NULL, or [B][H][T][srwm_tape_row()] float32 (out): the
                      record srwm_backward needs (see there) */
    float* window_states;
    int64_t t_stride;
} srwm_forward_args_t;

/* srwm_forward_ex -- the forward pass with every option.  Same edge cases,
 * ownership and error behaviour as srwm_forward; args == NULL gives
 * SRWM_ERR_NULL. */
int srwm_forward_ex(const srwm_forward_args_t* args);

/* Number of built kernel variants. */
int srwm_variant_count(void);

/* Description of one kernel variant. */
typedef struct srwm_variant_info {
    int d_in, d_out, io_dtype, n_lr;
    int waves;          /* waves per workgroup; one workgroup per unit          */
    int lanes_per_row;  /* lanes that share one row of W                        */
    int waves_per_simd; /* waves per SIMD its register use allows               */
    int schedule;       /* 0: projection, addresses, read, update in turn;
                           1: the read of step t and the projection of step t+1
                              share one pass over W, the projection corrected by
                              the rank-one update of Eq. (3)                   */
    int supports_reset; /* built with the reset ablation (reset_interval > 0)  */
    int writes_tape;    /* writes the backward tape (used when args.tape != NULL) */
    int is_auto;        /* may the automatic choice pick it                     */
} srwm_variant_info_t;

/* srwm_variant_info -- fill *info for variant `i` (0 <= i <
 * srwm_variant_count()).  Returns SRWM_OK, SRWM_ERR_ARG (bad index) or
 * SRWM_ERR_NULL (info == NULL). */
int srwm_variant_info(int i, srwm_variant_info_t* info);

/*
 * srwm_select_variant -- the variant index the automatic choice uses for
 * (d_in, d_out, io_dtype, n_lr), a reset interval (0: none) and `units` =
 * B*H: among the eligible variants, the fewest waves per unit for which
 * units*waves gives every SIMD of the chip two waves (>= 2048 waves), or else
 * the most waves per unit.  Returns a negative error code (SRWM_ERR_SHAPE,
 * SRWM_ERR_ARG, SRWM_ERR_UNSUPPORTED) when there is none.
 */
int srwm_select_variant(int64_t d_in, int64_t d_out, int io_dtype, int n_lr,
                        int64_t reset_interval, int64_t units);

/* Resources of one compiled kernel, as the HIP runtime reports them on the
 * current device (hipFuncGetAttributes, and
 * hipOccupancyMaxActiveBlocksPerMultiprocessor for its launch size). */
typedef struct srwm_kernel_resources {
    int vgprs;             /* vector registers per lane                        */
    int lds_bytes;         /* static LDS per workgroup                         */
    int scratch_bytes;     /* private (spill) memory per lane                  */
    int threads;           /* threads per workgroup of its launches            */
    int workgroups_per_cu; /* workgroups one CU holds at once                  */
    int waves_per_simd;    /* workgroups_per_cu * threads / 64 / 4 SIMDs       */
} srwm_kernel_resources_t;

/* srwm_variant_resources -- *out for forward variant `i`.  SRWM_ERR_ARG (bad
 * index) and SRWM_ERR_NULL (out == NULL) come before any HIP call;
 * SRWM_ERR_HIP if a runtime query fails (no GPU, say). */
int srwm_variant_resources(int i, srwm_kernel_resources_t* out);

/* srwm_backward_resources -- *out for the kernel srwm_backward launches for
 * (d_in, d_out, n_lr), without (reset == 0) or with resets, and units = B*H
 * (it takes, among the kernels for the shape, the fewest waves per unit that
 * still give every SIMD two waves, else the most); errors as
 * srwm_variant_resources, SRWM_ERR_SHAPE for units < 0, and
 * SRWM_ERR_UNSUPPORTED when there is none. */
int srwm_backward_resources(int64_t d_in, int64_t d_out, int n_lr, int reset, int64_t units,
                            srwm_kernel_resources_t* out);

/*
 * Backward pass (memory-efficient backpropagation through time: the pages
 * train W0 by backpropagating through the unrolled self-modification,
 * "Metalearning Continual Learning Algorithms" after Eq. (6) and the review
 * page Sec. 2.5).
 *
 * The forward pass run with args.tape != NULL records, per unit and step, a
 * row of srwm_tape_row() floats at tape[b][h][t][...]: with
 * K = round_up(m, 4),
 *   [0, m)            a_t, the row factor of the step's rank-one update
 *   [K, K+d_in)       phi(k_t)
 *   [K+d_in, K+2d_in) phi(q_t) - phi(k_t), rounded as the forward pass used it
 *   [K+2d_in, +4)     the learning rates sigma(beta_t) (n_lr of them, the
 *                     rest zero)
 *   [K+2d_in+4, +d_in) u_t, the step's input as the projection used it (x_t
 *                     widened to float32, softmax-ed when the input softmax
 *                     is on)
 * ([m, K) is padding: written as zeros or left as it was).  From the final state W_T,
 * srwm_backward walks t = T-1..0, undoes each update (W_{t-1} = W_t -
 * a_t phi(k_t)^T) and accumulates the adjoint; no projection and no input
 * softmax is recomputed.
 * With L = sum_t <gy[t], y_t> + <gW_T, W_T> it writes
 *   dx       [B][T][H][d_in]   dL/dx, float32 (also for bf16 x)
 *   dW_init  [B][H][m][d_in]   dL/d(initial state of each unit)
 *   dW0      [H][m][d_in]      sum over b of dW_init (the gradient of an
 *                              initial matrix shared over the batch), or NULL
 * Inputs: W_T as the forward pass wrote it, the tape, gy [B][T][H][d_out]
 * float32, gW_T [B][H][m][d_in] float32 or NULL (zero).  x is not read (the
 * tape holds u_t) and may be NULL; io_dtype must still name x's dtype, and
 * apply_input_softmax must be the forward pass's flag (it selects the
 * softmax's backward for dx).
 * With B == 0 a given dW0 is filled with zeros (one kernel launch); with
 * H == 0 nothing is launched.
 * The reset ablation: reset_interval R > 0 as in the forward pass, with the
 * forward pass's window_states.  Walking back into window w-1 at the reset
 * before step wR, the kernel adds the adjoint of the state entering step wR
 * (window w's share of dL/d(initial state)) to dW_init, sets the adjoint to
 * zero (the discarded end state of window w-1 affects nothing) and restarts
 * from window w-1's recorded end state.  dW_init is the sum of the windows'
 * shares, taken from the last window to the first.  Same
 * conventions as the forward: device pointers, 16-byte aligned, nothing
 * allocated, asynchronous on `stream`; errors as there (SRWM_ERR_UNSUPPORTED
 * when srwm_backward_supported() is 0).
 */
typedef struct srwm_backward_args {
    const void* x;                /* not read; kept for the layout of 0.4 */
    const float* W_T;
    const float* tape;
    const float* gy;
    const float* gW_T;
    float* dx;
    float* dW_init;
    float* dW0;
    int64_t B, T, H, d_in, d_out, m;
    int io_dtype;
    int apply_input_softmax;
    int n_lr;
    void* stream;
    int64_t reset_interval;       /* 0, or R > 0 as in the forward pass */
    const float* window_states;   /* the forward pass's, with R > 0 and T > R */
} srwm_backward_args_t;

int srwm_backward(const srwm_backward_args_t* args);

/*
 * srwm_backward_noalloc -- srwm_backward for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving or training
 * loops, harnesses that forbid hipMalloc) and want only the gradient of a
 * shared initial matrix: the per-unit gradients srwm_backward writes to the
 * caller's dW_init live instead in a scratch array the library holds on each
 * GPU (a file-scope device array of srwm_backward_noalloc_scratch_bytes()
 * bytes, 32 MiB, one copy per GPU, held until the process ends).
 *
 *   args->dW_init must be NULL (SRWM_ERR_ARG otherwise); args->dW0 [H][m][d_in]
 *   is required when H*m*d_in > 0 (SRWM_ERR_NULL); everything else as in
 *   srwm_backward, whose kernels it runs.  dx and dW0 are bit-identical to
 *   srwm_backward's for the same arguments.
 *   The batch runs in slices of whole sequences that fit the scratch, each
 *   slice's gradients summed into dW0 in order; a call whose single sequence
 *   needs more (H*m*d_in*4 bytes > the scratch) returns SRWM_ERR_SCRATCH.
 *   The scratch used is the current device's: `stream` (if not NULL) must
 *   belong to the current device (SRWM_ERR_ARG otherwise).  The first call on
 *   a device looks the array's address up (a HIP call, no allocation); no
 *   call allocates or frees memory.
 *   Calls on one GPU share its scratch and it keeps the last call's
 *   contents (every element a call reads it has written first): two calls
 *   that overlap in time on one GPU, on any streams, race and give wrong
 *   results; serialise them.
 */
int srwm_backward_noalloc(const srwm_backward_args_t* args);

/* Size in bytes of srwm_backward_noalloc's scratch array (per GPU). */
int64_t srwm_backward_noalloc_scratch_bytes(void);

/* Floats per step in the tape: round_up(m, 4) + 3*d_in + 4, or SRWM_ERR_SHAPE. */
int64_t srwm_tape_row(int64_t d_in, int64_t d_out, int n_lr);

/* 1 if srwm_backward has a kernel for (d_in, d_out, io_dtype, n_lr), else 0.
 * (d_in = d_out = 128 has one without resets only: with reset_interval > 0
 * srwm_backward returns SRWM_ERR_UNSUPPORTED there.  That kernel keeps the
 * adjoint in dW_init while it runs.) */
int srwm_backward_supported(int64_t d_in, int64_t d_out, int io_dtype, int n_lr);

/*
 * DeltaNet and SR-DeltaNet forward (review page Sec. 2.1 and Appendix C.1):
 * fast-weight programmers with a separate fast matrix F (d_v x d_key per
 * (sequence, head) unit).  Per step, with the projection
 * p_t = [k (d_key); v (d_v); q (d_key); beta (1)], P = d_v + 2*d_key + 1:
 *   kh = softmax(k), qh = softmax(q), g = sigmoid(beta)
 *   F += g (v - F kh) kh^T;   y_t = F qh   (queried after the write)
 * DeltaNet: p_t for head h = rows [h*P, (h+1)*P) of W_slow times the whole
 * input x_t (all heads, D = H*d_in: a full-width slow projection).
 * SR-DeltaNet: p_t is the output of an SRWM per head (d_out = P, its own
 * self-modification, as srwm_forward_ex with that W0, n_lr and input flag).
 *
 * All buffers are float32 device pointers, 16-byte aligned, caller-owned:
 *   x      [B][T][H][d_in]
 *   W_slow [H*P][H*d_in]          (DeltaNet; H*d_in must be a multiple of 4)
 *   W0     [H][m][d_in], m = P + 2*d_in + n_lr   (SR-DeltaNet's SRWM)
 *   F0     [B][H][d_v][d_key] or NULL (the fast matrix starts at zero)
 *   z      [B][T][H][P] (out): the projections of every step (work space the
 *          caller provides; it holds p_t afterwards)
 *   y      [B][T][H][d_v] (out)
 *   W_T    [B][H][m][d_in] or NULL (out, SR-DeltaNet: the SRWM's final state)
 *   F_T    [B][H][d_v][d_key] or NULL (out)
 * Nothing is allocated; asynchronous on `stream`; SRWM_ERR_UNSUPPORTED when
 * no kernel exists for (d_key, d_v) (srwm_fwp_supported) or, for SR-DeltaNet,
 * for the SRWM shape (srwm_supported(d_in, P, SRWM_IO_F32, n_lr)); other
 * errors as for srwm_forward (outputs overlapping any buffer: SRWM_ERR_ALIAS).
 */
typedef struct srwm_deltanet_args {
    const float* x;
    const float* W_slow;
    const float* F0;
    float* z;
    float* y;
    float* F_T;
    int64_t B, T, H, d_in, d_key, d_v;
    void* stream;
} srwm_deltanet_args_t;

int srwm_deltanet_forward(const srwm_deltanet_args_t* args);

/* The projection alone: z = the slow projection of every step (the same
 * arguments; F0, y and F_T are ignored and may be NULL). */
int srwm_deltanet_project(const srwm_deltanet_args_t* args);

/* The fast-matrix recurrence alone, from given projections z[B][T][H][P]
 * (P = d_v + 2*d_key + 1, rows [k; v; q; beta]): y[B][T][H][d_v] and F_T
 * (NULL allowed), starting from F0 (NULL: zero).  The second half of both
 * srwm_deltanet_forward and srwm_srdeltanet_forward.  t_stride as in
 * srwm_forward_args_t: 0, or S >= T when z and y are the steps [t0, t0+T) of
 * [B][S][H][*] buffers. */
typedef struct srwm_fast_args {
    const float* z;
    const float* F0;
    float* y;
    float* F_T;
    int64_t B, T, H, d_key, d_v;
    void* stream;
    int64_t t_stride;
} srwm_fast_args_t;

int srwm_fast_forward(const srwm_fast_args_t* args);

/*
 * SR-DeltaNet's two halves can overlap in time: the projection of steps
 * [t0+C, t0+2C) needs nothing from the fast matrix, so it runs on `stream`
 * while the fast-matrix recurrence of steps [t0, t0+C) runs on `aux_stream`.
 *   aux_stream   a second hipStream_t of the caller's, or NULL.
 *   chunk_steps  C: 0 picks a length for the shape; C >= T runs unchunked.
 * The overlap needs aux_stream, W_T and F_T (the carried states of both
 * halves live there between chunks); without any of them, or with C >= T, the
 * call runs the two halves one after the other on `stream`.  The results are
 * the same bits either way.  An overlapped call creates and destroys HIP
 * events, makes aux_stream wait for `stream`'s earlier work and makes
 * `stream` wait for all of it, so work queued on `stream` afterwards sees
 * every output.  Overlapping calls that share an aux_stream are serialised
 * on it, not wrong.  Under HIP graph capture of `stream`, aux_stream joins
 * the capture through the first event and is joined back by the last, so
 * the captured graph holds both halves (aux_stream must not be capturing
 * anything else).
 */
typedef struct srwm_srdeltanet_args {
    const float* x;
    const float* W0;
    const float* F0;
    float* z;
    float* y;
    float* W_T;
    float* F_T;
    int64_t B, T, H, d_in, d_key, d_v;
    int n_lr;
    int apply_input_softmax;
    void* stream;
    void* aux_stream;
    int64_t chunk_steps;
} srwm_srdeltanet_args_t;

int srwm_srdeltanet_forward(const srwm_srdeltanet_args_t* args);

/* The chunk length srwm_srdeltanet_forward takes for chunk_steps == 0 with
 * these sizes: about T/8 in whole 32-step pieces, at least 256, when the
 * projection's waves over all units leave room beside it (at most two per
 * SIMD of the chip), else T (no overlap).  Negative error code for sizes or
 * an n_lr that srwm_srdeltanet_forward would reject. */
int64_t srwm_srdeltanet_chunk_steps(int64_t B, int64_t T, int64_t H, int64_t d_in, int64_t d_key, int64_t d_v,
                                    int n_lr);

/* 1 if the fast-matrix kernel exists for (d_key, d_v), else 0. */
int srwm_fwp_supported(int64_t d_key, int64_t d_v);

/* 1 if a kernel exists for (d_in, d_out, io_dtype, n_lr), else 0. */
int srwm_supported(int64_t d_in, int64_t d_out, int io_dtype, int n_lr);

/*
 * Measurement aid (not part of the method): srwm_valu_probe launches
 * `workgroups` workgroups of 256 threads that each run `iters` rounds of 16
 * steps of 8 independent single-lane FP32 FMA chains and write one float per
 * thread to out[workgroups*256] (device, 16-byte aligned).  Timing it gives the
 * chip's scalar FP32 FMA rate, the ceiling of kernels built without packed
 * FP32; srwm_valu_probe_flop returns the FLOP (2 per FMA) of one launch.
 */
int srwm_valu_probe(float* out, int64_t workgroups, int iters, void* stream);
int64_t srwm_valu_probe_flop(int64_t workgroups, int iters);

/*
 * Measurement aid (not part of the method): srwm_lds_probe launches
 * `workgroups` workgroups of 256 threads that each fill a 32 KB LDS array and
 * then run `iters` rounds of 16 conflict-free 16-byte LDS reads per lane
 * (ds_read_b128; a wave's lanes read one contiguous 1 KB span), folding the
 * values into one word per thread written to out[workgroups*256] (device,
 * 16-byte aligned).  Timing it gives the chip's LDS read bandwidth, the roof
 * the kernels' LDS traffic is compared with; srwm_lds_probe_bytes returns the
 * LDS bytes one launch reads.  Errors: SRWM_ERR_NULL (out), SRWM_ERR_SHAPE
 * (workgroups or iters < 1), SRWM_ERR_ARG (alignment), SRWM_ERR_HIP (launch).
 */
int srwm_lds_probe(unsigned* out, int64_t workgroups, int iters, void* stream);
int64_t srwm_lds_probe_bytes(int64_t workgroups, int iters);

/* Static string naming an error code (never NULL). */
const char* srwm_strerror(int code);

/* Version as MAJOR*10000 + MINOR*100 + PATCH. */
int srwm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SRWM_H */
