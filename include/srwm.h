/*
 * srwm.h -- C ABI of libsrwm: forward recurrence of the multi-head,
 * 4-learning-rate self-referential weight matrix (SRWM) on AMD Instinct
 * MI355X (gfx950).
 *
 * The operation (sources: "Metalearning Continual Learning Algorithms --
 * part 2/5", Sec. 2.3 Eq. (1)-(3) and the "4-learning-rate version"
 * paragraph, Eq. (4)-(5); review page "SRWM: 让权重矩阵学习修改自身" of
 * "A Modern Self-Referential Weight Matrix That Learns to Modify Itself",
 * Sec. 2.2-2.5):
 *
 *   Every (sequence b, head h) is an independent unit with an m x d_in state
 *   W, m = d_out + 2*d_in + 4, row blocks [W^y; W^k; W^q; W^beta].  All units
 *   start from the shared initial matrix W0[h].  For t = 0..T-1:
 *     u     = x[b,t,h,:]            (softmax(x[b,t,h,:]) if apply_input_softmax)
 *     z     = W u = [y_t, k_t, q_t, beta_t]                      Eq. (1)
 *     y[b,t,h,:] = z[0:d_out]        (from W before this step's update)
 *     kh    = softmax(k_t), qh = softmax(q_t), g = sigmoid(beta_t) in R^4
 *     W[i,:] += g[block(i)] * ((W qh)_i - (W kh)_i) * kh     Eq. (2)-(5)
 *   with block(i) = 0, 1, 2, 3 for the y, k, q, beta rows.
 *   W_T[b,h] = W after step T-1.
 *
 * Conventions shared by every entry point:
 *   - Layout: dense, row-major, contiguous.  x[B][T][H][d_in],
 *     W0[H][m][d_in], y[B][T][H][d_out], W_T[B][H][m][d_in].
 *   - Dtypes: x and y share io_dtype (SRWM_IO_F32 = float32, SRWM_IO_BF16 =
 *     bfloat16 bits in uint16).  W0 and W_T are always float32; the state and
 *     all arithmetic are float32.  bf16 x is widened exactly; y is rounded to
 *     bf16 with round-to-nearest-even.
 *   - Memory: every pointer is a device pointer (hipMalloc'd or equivalent),
 *     16-byte aligned (SRWM_ERR_ARG otherwise) and owned by the caller.  The
 *     library allocates nothing, frees nothing, keeps no pointer after the
 *     call returns and holds no mutable global state: concurrent calls on
 *     different streams are safe.
 *   - Execution: asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  The return code covers argument validation and the launch
 *     only; a fault during execution surfaces at the next synchronisation.
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
#define SRWM_VERSION_MINOR 1
#define SRWM_VERSION_PATCH 0

typedef enum { SRWM_IO_F32 = 0, SRWM_IO_BF16 = 1 } srwm_io_dtype_t;

enum {
    SRWM_OK = 0,
    SRWM_ERR_NULL = -1,        /* a required pointer is NULL                      */
    SRWM_ERR_SHAPE = -2,       /* negative size, m != d_out+2*d_in+4, overflow     */
    SRWM_ERR_UNSUPPORTED = -3, /* no kernel built for (d_in, d_out, io_dtype)      */
    SRWM_ERR_ALIAS = -4,       /* an output overlaps an input or the other output */
    SRWM_ERR_HIP = -5,         /* the HIP runtime rejected the launch              */
    SRWM_ERR_ARG = -6          /* other invalid argument (io_dtype, flag, variant,
                                  a pointer not 16-byte aligned)                  */
};

/*
 * srwm_forward -- run the whole recurrence for all B*H units.
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
 * are not checked.  x/y and W0/W_T must not overlap (SRWM_ERR_ALIAS).
 * Pointers may be NULL only when the tensor they address is empty.
 * Returns SRWM_OK or a negative error code.
 */
int srwm_forward(const void* x, const float* W0, void* y, float* W_T,
                 int64_t B, int64_t T, int64_t H, int64_t d_in, int64_t d_out,
                 int64_t m, int io_dtype, int apply_input_softmax,
                 void* stream);

/*
 * srwm_forward_variant -- srwm_forward with an explicit kernel variant, for
 * tuning and for testing every variant against the same definition.
 * variant = -1 makes the automatic choice (identical to srwm_forward): among
 * the eligible variants of (d_in, d_out, io_dtype), the fewest waves per
 * unit for which B*H*waves gives every SIMD of the chip two waves (>= 2048
 * waves), or else the most waves per unit.  Otherwise `variant` indexes the list that
 * srwm_variant_info() reports; a variant whose (d_in, d_out, io_dtype) does
 * not match the call gives SRWM_ERR_ARG.  Every variant computes the same
 * function; they differ in how a unit's state is spread over lanes.
 */
int srwm_forward_variant(const void* x, const float* W0, void* y, float* W_T,
                         int64_t B, int64_t T, int64_t H, int64_t d_in,
                         int64_t d_out, int64_t m, int io_dtype,
                         int apply_input_softmax, void* stream, int variant);

/* Number of built kernel variants. */
int srwm_variant_count(void);

/*
 * srwm_variant_info -- describe variant `i` (0 <= i < srwm_variant_count()):
 * d_in, d_out, io_dtype, waves per workgroup (one workgroup per unit), lanes
 * sharing one row of W, waves per SIMD its register use allows, its step
 * schedule (0: projection, addresses, read, update in turn; 1: the read of
 * step t and the projection of step t+1 share one pass over W, with the
 * rank-one correction of Eq. (3) applied to the projection), and whether the
 * automatic choice may pick it.  Any output pointer may be NULL.
 * Returns SRWM_OK or SRWM_ERR_ARG.
 */
int srwm_variant_info(int i, int* d_in, int* d_out, int* io_dtype, int* waves,
                      int* lanes_per_row, int* waves_per_simd, int* schedule,
                      int* is_auto);

/*
 * srwm_select_variant -- the variant index srwm_forward would use for
 * (d_in, d_out, io_dtype) and `units` = B*H (>= 0), or a negative error code
 * (SRWM_ERR_SHAPE, SRWM_ERR_ARG, SRWM_ERR_UNSUPPORTED).
 */
int srwm_select_variant(int64_t d_in, int64_t d_out, int io_dtype, int64_t units);

/* 1 if a kernel exists for (d_in, d_out, io_dtype), else 0. */
int srwm_supported(int64_t d_in, int64_t d_out, int io_dtype);

/* Static string naming an error code (never NULL). */
const char* srwm_strerror(int code);

/* Version as MAJOR*10000 + MINOR*100 + PATCH. */
int srwm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SRWM_H */
