// srwm_fwd.hip -- C ABI of libsrwm's forward pass (the kernels are in
// srwm_fwd_kernels.h, instantiated by the variant table's parts).
//
// Forward recurrence of the multi-head, 4-learning-rate self-referential
// weight matrix ("Metalearning Continual Learning Algorithms -- part 2/5",
// Sec. 2.3 Eq. (1)-(3) and the 4-learning-rate paragraph, Eq. (4)-(5);
// review page "SRWM: 让权重矩阵学习修改自身", Sec. 2.2-2.5).
//
// Design (one workgroup per (sequence, head) unit, state resident on chip):
//   * The m x d_in state W of a unit lives in VGPRs for all T steps.  Lane
//     (rg, p) of the workgroup, rg = tid / P and p = tid % P, holds rows
//     rg + G*r (r = 0..R-1, G = threads / P) and columns [p*L, p*L + L),
//     L = d_in / P.  The P lanes that share a row are adjacent in one DPP
//     row, so a row's dot product is P partial sums joined by log2(P) DPP
//     adds and every one of the P lanes ends with the same bits.
//   * Strided rows (row = rg + G*r) put register r of every lane in one row
//     block (y, k, q or beta) whenever G divides d_in and d_out, so the
//     learning rate of register r is known at compile time.  The four beta
//     rows take a last register row whose other G-4 rows are zero padding:
//     zero rows read zero and stay zero.
//   * Per step: (A) z = W u from the lane's columns of u (staged in LDS),
//     reduced across P lanes, written to LDS; (B) one or two waves form
//     softmax(k), softmax(q), sigmoid(beta) and store y_t = z[0:d_out];
//     (C) r = W (qh - kh) -- the two reads v - vb of Eq. (2) fused into one
//     pass over W, reduced across P lanes, times the row block's gate;
//     (D) W += a kh^T in place.  Two workgroup barriers per step.
//   * x is staged S steps at a time into a double-buffered LDS tile: the
//     global loads of chunk c+1 are issued a whole chunk ahead, then widened
//     (bf16 -> f32 is exact), optionally softmax-ed per step row, and stored.
//
// Arithmetic is float32 throughout.  Packed FP32 instructions are disabled
// at build time; every FMA is a scalar v_fma_f32.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "srwm.h"
#include "srwm_device.h"
#include "srwm_fwd_table.h"

namespace {

using namespace srwm;

// ----------------------------------------------------------------------------
// The variant table: its parts (each instantiated in its own translation
// unit) indexed as one table, in this order.
VariantPart (*const kFwdParts[])() = {fwd_variants_small, fwd_variants_d64, fwd_variants_misc, fwd_variants_tape};

struct Table {
    const Variant* v[512];
    int n = 0;
    Table()
    {
        for (auto part : kFwdParts) {
            const VariantPart p = part();
            for (int i = 0; i < p.n && n < 512; ++i) v[n++] = &p.v[i];
        }
    }
};

const Table& table()
{
    static const Table t;
    return t;
}

// Two waves per SIMD of the chip (256 CUs x 4 SIMDs x 2): enough waves to
// hide one wave's latency behind another's arithmetic.
constexpr int64_t kChipWaveSlots = 2048;

bool variant_matches(const Variant& v, int64_t d_in, int64_t d_out, int io, int nlr, bool reset, bool tape)
{
    return v.d_in == d_in && v.d_out == d_out && v.io == io && v.nlr == nlr && (!reset || v.reset) &&
           (v.tape == (tape ? 1 : 0));
}

// Automatic choice among the eligible variants: the fewest waves per unit
// that still fill the chip -- two waves per SIMD for one-wave units (units >=
// 2048), four for multi-wave units (units * waves >= 4096: they spend part of
// each step in barriers and LDS round trips that a second pair of waves
// hides; at d = 64 and 512 units eight waves per unit take 0.49 ms against
// 0.51 ms for four); if none does, the most waves per unit.  Variants whose reset support
// matches the request come first: a variant built with the reset ablation
// serves a plain request only for a shape that has no plain variant.
int find_variant(int64_t d_in, int64_t d_out, int io, int nlr, bool reset, bool tape, int requested,
                 int64_t units)
{
    if (requested >= 0) {
        if (requested >= table().n) return -1;
        return variant_matches(*table().v[requested], d_in, d_out, io, nlr, reset, tape) ? requested : -1;
    }
    for (int pass = 0; pass < 2; ++pass) {
        int best_fill = -1, best_any = -1;
        for (int i = 0; i < table().n; ++i) {
            const Variant& v = *table().v[i];
            if (!variant_matches(v, d_in, d_out, io, nlr, reset, tape) || !v.is_auto) continue;
            if (pass == 0 && (v.reset != 0) != reset) continue;
            const int64_t fill = v.nw == 1 ? kChipWaveSlots : 2 * kChipWaveSlots;
            if (units * v.nw >= fill && (best_fill < 0 || v.nw < table().v[best_fill]->nw)) best_fill = i;
            if (best_any < 0 || v.nw > table().v[best_any]->nw) best_any = i;
        }
        if (best_fill >= 0 || best_any >= 0) return best_fill >= 0 ? best_fill : best_any;
    }
    // a shape whose only variants are not marked eligible (or all fused, with reset)
    for (int i = 0; i < table().n; ++i)
        if (variant_matches(*table().v[i], d_in, d_out, io, nlr, reset, tape)) return i;
    return -1;
}

}  // namespace

namespace srwm {

int forward_check(const srwm_forward_args_t* a, FwdPlan* plan)
{
    if (a == nullptr) return SRWM_ERR_NULL;
    const int64_t B = a->B, T = a->T, H = a->H, d_in = a->d_in, d_out = a->d_out, m = a->m;
    if (B < 0 || T < 0 || H < 0 || d_in < 1 || d_out < 1) return SRWM_ERR_SHAPE;
    if (a->t_stride < 0 || (a->t_stride > 0 && a->t_stride < T)) return SRWM_ERR_SHAPE;
    const int64_t S = a->t_stride > 0 ? a->t_stride : T;
    if (a->n_lr != 1 && a->n_lr != 4) return SRWM_ERR_ARG;
    if (m != d_out + 2 * d_in + a->n_lr) return SRWM_ERR_SHAPE;
    if (a->io_dtype != SRWM_IO_F32 && a->io_dtype != SRWM_IO_BF16) return SRWM_ERR_ARG;
    if (a->apply_input_softmax != 0 && a->apply_input_softmax != 1) return SRWM_ERR_ARG;
    if (a->w0_per_sequence != 0 && a->w0_per_sequence != 1) return SRWM_ERR_ARG;
    if (a->reset_interval < 0 || a->reset_interval > INT32_MAX) return SRWM_ERR_ARG;
    if (a->variant < -1) return SRWM_ERR_ARG;
    const bool reset = a->reset_interval > 0;
    const bool want_tape = a->tape != nullptr;
    const int64_t units_hint = (B > 0 && H > INT64_MAX / B) ? INT64_MAX : B * H;
    const int vi = find_variant(d_in, d_out, a->io_dtype, a->n_lr, reset, want_tape, a->variant, units_hint);
    if (vi < 0) return a->variant >= 0 ? SRWM_ERR_ARG : SRWM_ERR_UNSUPPORTED;
    const int64_t es = a->io_dtype == SRWM_IO_BF16 ? 2 : 4;
    int64_t units, steps, span, nx, ny, nw0, nwt, ntape, nws;
    // with a tape and resets: the end states of all windows but the last
    const int64_t nres = (reset && want_tape && T > 0) ? (T - 1) / a->reset_interval : 0;
    // x and y cover (B-1)*S + T steps of each head (all of them when S == T)
    if (!mul_ok(B > 0 ? B - 1 : 0, S, &span) || span > INT64_MAX - T) return SRWM_ERR_SHAPE;
    span = (B > 0 && T > 0) ? span + T : 0;
    if (!mul_ok(B, H, &units) || !mul_ok(units, T, &steps) || !mul_ok(span, H * d_in * es, &nx) ||
        !mul_ok(span, H * d_out * es, &ny) || !mul_ok(a->w0_per_sequence ? units : H, m * d_in * 4, &nw0) ||
        !mul_ok(units, m * d_in * 4, &nwt) || !mul_ok(steps, tape_row(d_in, d_out, a->n_lr) * 4, &ntape) ||
        !mul_ok(nwt, nres, &nws))
        return SRWM_ERR_SHAPE;
    if (!want_tape) ntape = 0;
    if (units > INT32_MAX || S > INT32_MAX || H > INT32_MAX) return SRWM_ERR_SHAPE;
    // the kernels address a chunk of up to 32 steps of x with a lane's 32-bit
    // offset from the chunk's first row: one step's row (H*d_in elements) may
    // span at most 64 MiB
    if (H * d_in * es > (INT64_C(1) << 26)) return SRWM_ERR_SHAPE;
    const void* x = a->x;
    const float* W0 = a->W0;
    void* y = a->y;
    float* W_T = a->W_T;
    float* tape = a->tape;
    float* wstates = nws > 0 ? a->window_states : nullptr;
    if ((nx > 0 && x == nullptr) || (ny > 0 && y == nullptr) || (nw0 > 0 && units > 0 && W0 == nullptr) ||
        (nws > 0 && wstates == nullptr))
        return SRWM_ERR_NULL;
    // The kernels move 16-byte pieces: every buffer must be 16-byte aligned.
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(W0) |
         reinterpret_cast<uintptr_t>(y) | reinterpret_cast<uintptr_t>(W_T) |
         reinterpret_cast<uintptr_t>(tape) | reinterpret_cast<uintptr_t>(wstates)) & 15u)
        return SRWM_ERR_ARG;
    plan->vi = vi;
    plan->waves = table().v[vi]->nw;
    plan->units = units;
    plan->wstates = wstates;
    plan->run = false;
    if (units == 0) return SRWM_OK;
    if (W_T == nullptr) nwt = 0;
    if (ranges_overlap(x, nx, y, ny) || ranges_overlap(W0, nw0, W_T, nwt) ||
        ranges_overlap(x, nx, W_T, nwt) || ranges_overlap(W0, nw0, y, ny) ||
        ranges_overlap(y, ny, W_T, nwt) || ranges_overlap(tape, ntape, x, nx) ||
        ranges_overlap(tape, ntape, W0, nw0) || ranges_overlap(tape, ntape, y, ny) ||
        ranges_overlap(tape, ntape, W_T, nwt) || ranges_overlap(wstates, nws, x, nx) ||
        ranges_overlap(wstates, nws, W0, nw0) || ranges_overlap(wstates, nws, y, ny) ||
        ranges_overlap(wstates, nws, W_T, nwt) || ranges_overlap(wstates, nws, tape, ntape))
        return SRWM_ERR_ALIAS;
    plan->run = !(T == 0 && W_T == nullptr);
    return SRWM_OK;
}

int forward_launch(const FwdPlan& plan, const srwm_forward_args_t* a)
{
    const Variant& v = *table().v[plan.vi];
    const void* x = a->x;
    const float* W0 = a->W0;
    void* y = a->y;
    float* W_T = a->W_T;
    float* tape = a->tape;
    float* wstates = plan.wstates;
    int Ti = static_cast<int>(a->T), Si = static_cast<int>(a->t_stride > 0 ? a->t_stride : a->T);
    int Hi = static_cast<int>(a->H), fl = a->apply_input_softmax;
    int per_seq = a->w0_per_sequence, rst = static_cast<int>(a->reset_interval);
    void* args[] = {const_cast<void**>(&x), const_cast<float**>(&W0), &y, &W_T, &tape, &wstates, &Ti, &Si, &Hi, &fl,
                    &per_seq, &rst};
    const hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(v.fn),
                                           dim3(static_cast<unsigned>(plan.units)), dim3(v.nw * kWave),
                                           args, 0, static_cast<hipStream_t>(a->stream));
    return err == hipSuccess ? SRWM_OK : SRWM_ERR_HIP;
}

}  // namespace srwm

namespace {

int forward_impl(const srwm_forward_args_t* a)
{
    FwdPlan plan;
    const int rc = forward_check(a, &plan);
    if (rc != SRWM_OK || !plan.run) return rc;
    return forward_launch(plan, a);
}

srwm_forward_args_t basic_args(const void* x, const float* W0, void* y, float* W_T, int64_t B, int64_t T,
                               int64_t H, int64_t d_in, int64_t d_out, int64_t m, int io_dtype,
                               int apply_input_softmax, void* stream, int variant)
{
    srwm_forward_args_t a;
    a.x = x;
    a.W0 = W0;
    a.y = y;
    a.W_T = W_T;
    a.B = B;
    a.T = T;
    a.H = H;
    a.d_in = d_in;
    a.d_out = d_out;
    a.m = m;
    a.io_dtype = io_dtype;
    a.apply_input_softmax = apply_input_softmax;
    a.n_lr = 4;
    a.w0_per_sequence = 0;
    a.reset_interval = 0;
    a.variant = variant;
    a.stream = stream;
    a.tape = nullptr;
    a.window_states = nullptr;
    a.t_stride = 0;
    return a;
}

}  // namespace

extern "C" {

int srwm_forward(const void* x, const float* W0, void* y, float* W_T, int64_t B, int64_t T,
                 int64_t H, int64_t d_in, int64_t d_out, int64_t m, int io_dtype,
                 int apply_input_softmax, void* stream)
{
    const srwm_forward_args_t a =
        basic_args(x, W0, y, W_T, B, T, H, d_in, d_out, m, io_dtype, apply_input_softmax, stream, -1);
    return forward_impl(&a);
}

int srwm_forward_variant(const void* x, const float* W0, void* y, float* W_T, int64_t B,
                         int64_t T, int64_t H, int64_t d_in, int64_t d_out, int64_t m,
                         int io_dtype, int apply_input_softmax, void* stream, int variant)
{
    const srwm_forward_args_t a =
        basic_args(x, W0, y, W_T, B, T, H, d_in, d_out, m, io_dtype, apply_input_softmax, stream, variant);
    return forward_impl(&a);
}

int srwm_forward_ex(const srwm_forward_args_t* args) { return forward_impl(args); }

int64_t srwm_tape_row(int64_t d_in, int64_t d_out, int n_lr)
{
    if (d_in < 1 || d_out < 1 || (n_lr != 1 && n_lr != 4)) return SRWM_ERR_SHAPE;
    return tape_row(d_in, d_out, n_lr);
}

int srwm_variant_count(void) { return table().n; }

int srwm_variant_info(int i, srwm_variant_info_t* info)
{
    if (i < 0 || i >= table().n) return SRWM_ERR_ARG;
    if (info == nullptr) return SRWM_ERR_NULL;
    const Variant& v = *table().v[i];
    info->d_in = v.d_in;
    info->d_out = v.d_out;
    info->io_dtype = v.io;
    info->n_lr = v.nlr;
    info->waves = v.nw;
    info->lanes_per_row = v.p;
    info->waves_per_simd = v.wpe;
    info->schedule = v.fused;
    info->supports_reset = v.reset;
    info->writes_tape = v.tape;
    info->is_auto = v.is_auto;
    return SRWM_OK;
}

int srwm_variant_resources(int i, srwm_kernel_resources_t* out)
{
    if (i < 0 || i >= table().n) return SRWM_ERR_ARG;
    if (out == nullptr) return SRWM_ERR_NULL;
    return kernel_resources(reinterpret_cast<const void*>(table().v[i]->fn), table().v[i]->nw * kWave, out);
}

int srwm_select_variant(int64_t d_in, int64_t d_out, int io_dtype, int n_lr, int64_t reset_interval,
                        int64_t units)
{
    if (d_in < 1 || d_out < 1 || units < 0 || reset_interval < 0) return SRWM_ERR_SHAPE;
    if (io_dtype != SRWM_IO_F32 && io_dtype != SRWM_IO_BF16) return SRWM_ERR_ARG;
    if (n_lr != 1 && n_lr != 4) return SRWM_ERR_ARG;
    const int vi = find_variant(d_in, d_out, io_dtype, n_lr, reset_interval > 0, false, -1, units);
    return vi >= 0 ? vi : SRWM_ERR_UNSUPPORTED;
}

int srwm_supported(int64_t d_in, int64_t d_out, int io_dtype, int n_lr)
{
    return find_variant(d_in, d_out, io_dtype, n_lr, false, false, -1, 1) >= 0 ? 1 : 0;
}

const char* srwm_strerror(int code)
{
    switch (code) {
    case SRWM_OK: return "SRWM_OK: success";
    case SRWM_ERR_NULL: return "SRWM_ERR_NULL: a required pointer is NULL";
    case SRWM_ERR_SHAPE: return "SRWM_ERR_SHAPE: invalid sizes (negative, m != d_out+2*d_in+n_lr, or overflow)";
    case SRWM_ERR_UNSUPPORTED: return "SRWM_ERR_UNSUPPORTED: no kernel built for this (d_in, d_out, io_dtype, n_lr)";
    case SRWM_ERR_ALIAS: return "SRWM_ERR_ALIAS: an output buffer overlaps another buffer";
    case SRWM_ERR_HIP: return "SRWM_ERR_HIP: the HIP runtime rejected the launch";
    case SRWM_ERR_ARG: return "SRWM_ERR_ARG: invalid io_dtype, flag, n_lr, reset interval, variant or alignment";
    case SRWM_ERR_SCRATCH:
        return "SRWM_ERR_SCRATCH: one sequence's per-unit gradients (H*m*d_in floats) exceed the no-allocation "
               "backward's scratch array";
    default: return "unknown srwm error code";
    }
}

int srwm_version(void)
{
    return SRWM_VERSION_MAJOR * 10000 + SRWM_VERSION_MINOR * 100 + SRWM_VERSION_PATCH;
}

}  // extern "C"
