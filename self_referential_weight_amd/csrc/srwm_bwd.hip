// srwm_bwd.hip -- gfx950 backward pass of the SRWM recurrence and its C ABI
// (srwm_backward): gradients of a loss on y_1..y_T and W_T with respect to x
// and the initial state, from the tape the forward pass records.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "srwm.h"
#include "srwm_device.h"
#include "srwm_bwd_kernels.h"

namespace {

using namespace srwm;

// Backward kernels: (d_in, d_out, waves per unit, lanes per row, learning
// rates).  They read u_t from the tape, never x, so one kernel serves both
// I/O dtypes of the forward pass.
using BwdFn = void (*)(const float*, const float*, const float*, const float*, float*, float*, int, int,
                       int, int, const float*);
struct BwdVariant {
    int d_in, d_out, nlr, nw, reset;
    BwdFn fn;
};
// Without and with the reset ablation's window restarts.
#define SRWM_BWD(DI, DO, NW, P, NLR)                                                     \
    BwdVariant{DI, DO, NLR, NW, 0, &srwm_bwd_kernel<DI, DO, NW, P, NLR, false>},        \
        BwdVariant{DI, DO, NLR, NW, 1, &srwm_bwd_kernel<DI, DO, NW, P, NLR, true>}
// d = 128: the wide kernel (W in registers, the adjoint in dW_init; no resets).
#define SRWM_BWD_WIDE(DI, DO, NW, P, NLR) \
    BwdVariant{DI, DO, NLR, NW, 0, &srwm_bwd_wide_kernel<DI, DO, NW, P, NLR, false>}
const BwdVariant kBwdVariants[] = {
    SRWM_BWD(8, 8, 1, 8, 4), SRWM_BWD(16, 16, 1, 4, 4), SRWM_BWD(64, 64, 4, 16, 4), SRWM_BWD(64, 64, 8, 16, 4),
    SRWM_BWD(8, 8, 1, 8, 1), SRWM_BWD(16, 16, 1, 4, 1), SRWM_BWD(64, 64, 4, 16, 1), SRWM_BWD(64, 64, 8, 16, 1),
    SRWM_BWD_WIDE(128, 128, 8, 16, 4), SRWM_BWD_WIDE(128, 128, 8, 16, 1),
};
constexpr int kNumBwdVariants = sizeof(kBwdVariants) / sizeof(kBwdVariants[0]);

// Among the kernels for (d_in, d_out, n_lr, reset): the fewest waves per unit
// for which units * waves gives every SIMD of the chip two waves (>= 2048), or
// else the most waves per unit (as the forward pass chooses); -1 if none.
int find_bwd(int64_t d_in, int64_t d_out, int nlr, int reset, int64_t units)
{
    int enough = -1, most = -1;
    for (int i = 0; i < kNumBwdVariants; ++i) {
        const BwdVariant& v = kBwdVariants[i];
        if (v.d_in != d_in || v.d_out != d_out || v.nlr != nlr || v.reset != reset) continue;
        if (units >= (2048 + v.nw - 1) / v.nw && (enough < 0 || v.nw < kBwdVariants[enough].nw)) enough = i;
        if (most < 0 || v.nw > kBwdVariants[most].nw) most = i;
    }
    return enough >= 0 ? enough : most;
}

// A validated backward call: the kernel, the unit count, the byte sizes.
struct BwdPlan {
    int vi;
    int64_t units, per_b, nres;
};

// Validation shared by srwm_backward and srwm_backward_noalloc (which brings
// no dW_init of its own: own_dwinit = false).  No HIP call.
int backward_check(const srwm_backward_args_t* a, bool own_dwinit, BwdPlan* plan)
{
    if (a == nullptr) return SRWM_ERR_NULL;
    const int64_t B = a->B, T = a->T, H = a->H, d_in = a->d_in, d_out = a->d_out, m = a->m;
    if (B < 0 || T < 0 || H < 0 || d_in < 1 || d_out < 1) return SRWM_ERR_SHAPE;
    if (a->n_lr != 1 && a->n_lr != 4) return SRWM_ERR_ARG;
    if (m != d_out + 2 * d_in + a->n_lr) return SRWM_ERR_SHAPE;
    if (a->io_dtype != SRWM_IO_F32 && a->io_dtype != SRWM_IO_BF16) return SRWM_ERR_ARG;
    if (a->apply_input_softmax != 0 && a->apply_input_softmax != 1) return SRWM_ERR_ARG;
    if (a->reset_interval < 0 || a->reset_interval > INT32_MAX) return SRWM_ERR_ARG;
    if (!own_dwinit && a->dW_init != nullptr) return SRWM_ERR_ARG;
    const int want_reset = a->reset_interval > 0 ? 1 : 0;
    int64_t units, steps, ndx, ngy, nst, ntape, nw0, nws;
    if (!mul_ok(B, H, &units)) return SRWM_ERR_SHAPE;
    const int vi = find_bwd(d_in, d_out, a->n_lr, want_reset, units);
    if (vi < 0) return SRWM_ERR_UNSUPPORTED;
    // the forward pass's end states of all windows but the last
    const int64_t nres = (a->reset_interval > 0 && T > 0) ? (T - 1) / a->reset_interval : 0;
    if (!mul_ok(units, T, &steps) || !mul_ok(steps, d_in * 4, &ndx) || !mul_ok(steps, d_out * 4, &ngy) ||
        !mul_ok(units, m * d_in * 4, &nst) || !mul_ok(steps, tape_row(d_in, d_out, a->n_lr) * 4, &ntape) ||
        !mul_ok(H, m * d_in * 4, &nw0) || !mul_ok(nst, nres, &nws))
        return SRWM_ERR_SHAPE;
    if (units > INT32_MAX || T > INT32_MAX || H > INT32_MAX) return SRWM_ERR_SHAPE;
    if ((nst > 0 && (a->W_T == nullptr || (own_dwinit && a->dW_init == nullptr))) ||
        (ntape > 0 && a->tape == nullptr) || (ndx > 0 && a->dx == nullptr) || (ngy > 0 && a->gy == nullptr) ||
        (nws > 0 && a->window_states == nullptr) || (!own_dwinit && nw0 > 0 && a->dW0 == nullptr))
        return SRWM_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(a->W_T) |
         reinterpret_cast<uintptr_t>(a->tape) | reinterpret_cast<uintptr_t>(a->gy) |
         reinterpret_cast<uintptr_t>(a->gW_T) | reinterpret_cast<uintptr_t>(a->dx) |
         reinterpret_cast<uintptr_t>(a->dW_init) | reinterpret_cast<uintptr_t>(a->dW0) |
         reinterpret_cast<uintptr_t>(nws > 0 ? a->window_states : nullptr)) & 15u)
        return SRWM_ERR_ARG;
    plan->vi = vi;
    plan->units = units;
    plan->per_b = H * m * d_in;
    plan->nres = nres;
    if (units == 0) return SRWM_OK;
    const void* ins[] = {a->W_T, a->tape, a->gy, a->gW_T, nws > 0 ? a->window_states : nullptr};
    const int64_t nins[] = {nst, ntape, ngy, a->gW_T ? nst : 0, nws};
    void* outs[] = {a->dx, a->dW_init, a->dW0};
    const int64_t nouts[] = {ndx, own_dwinit ? nst : 0, a->dW0 ? nw0 : 0};
    for (int o = 0; o < 3; ++o) {
        for (int i = 0; i < 5; ++i)
            if (ranges_overlap(outs[o], nouts[o], ins[i], nins[i])) return SRWM_ERR_ALIAS;
        for (int o2 = o + 1; o2 < 3; ++o2)
            if (ranges_overlap(outs[o], nouts[o], outs[o2], nouts[o2])) return SRWM_ERR_ALIAS;
    }
    return SRWM_OK;
}

// dW0 = sum over the B sequences of dWi (accumulate: dW0 + that sum, added
// in the same order, so a batch summed in slices gives the same bits).
int launch_batch_sum(const float* dWi, float* dW0, int64_t B, int64_t per_b, int accumulate, hipStream_t st)
{
    if (dW0 == nullptr || per_b == 0) return SRWM_OK;
    int64_t Bv = B, pb = per_b;
    void* args[] = {const_cast<float**>(&dWi), &dW0, &Bv, &pb, &accumulate};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&srwm_sum_over_batch_kernel),
                                         dim3(static_cast<unsigned>((per_b + 255) / 256)), dim3(256), args, 0, st);
    return e == hipSuccess ? SRWM_OK : SRWM_ERR_HIP;
}

// The backward kernel of `plan` over sequences [b0, b0 + Bc) of the call,
// writing their per-unit gradients to dWi (Bc*H units: every buffer is
// batch-major, so a slice of the batch is an offset into each).
int launch_backward(const BwdPlan& plan, const srwm_backward_args_t* a, int64_t b0, int64_t Bc, float* dWi)
{
    const BwdVariant& v = kBwdVariants[plan.vi];
    const int64_t H = a->H, T = a->T, md = a->m * a->d_in;
    const int64_t row = tape_row(a->d_in, a->d_out, a->n_lr);
    const float* WTp = a->W_T + b0 * H * md;
    const float* tape = a->tape + b0 * H * T * row;
    const float* gy = a->gy + b0 * T * H * a->d_out;
    const float* gWT = a->gW_T ? a->gW_T + b0 * H * md : nullptr;
    float* dx = a->dx + b0 * T * H * a->d_in;
    const float* wstates = plan.nres > 0 ? a->window_states + b0 * H * plan.nres * md : nullptr;
    int Ti = static_cast<int>(T), Hi = static_cast<int>(H), fl = a->apply_input_softmax;
    int rst = static_cast<int>(a->reset_interval);
    void* args[] = {const_cast<float**>(&WTp), const_cast<float**>(&tape),
                    const_cast<float**>(&gy), const_cast<float**>(&gWT), &dx, &dWi, &Ti, &Hi, &fl, &rst,
                    const_cast<float**>(&wstates)};
    const hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(v.fn),
                                           dim3(static_cast<unsigned>(Bc * H)), dim3(v.nw * kWave), args, 0,
                                           static_cast<hipStream_t>(a->stream));
    return err == hipSuccess ? SRWM_OK : SRWM_ERR_HIP;
}

int backward_impl(const srwm_backward_args_t* a)
{
    BwdPlan plan;
    const int rc = backward_check(a, true, &plan);
    if (rc != SRWM_OK) return rc;
    const hipStream_t st = static_cast<hipStream_t>(a->stream);
    if (plan.units == 0) return launch_batch_sum(nullptr, a->dW0, 0, plan.per_b, 0, st);
    const int rk = launch_backward(plan, a, 0, a->B, a->dW_init);
    if (rk != SRWM_OK) return rk;
    return launch_batch_sum(a->dW_init, a->dW0, a->B, plan.per_b, 0, st);
}

// ----------------------------------------------------------------------------
// The no-allocation backward pass (srwm_backward_noalloc): the per-unit
// gradients that srwm_backward writes to the caller's dW_init live instead in
// `scratch`, a file-scope device array of kScratchFloats floats (one copy per
// GPU, held until the process ends).  Its device address is looked up once
// per device, with that device current, at the entry point's first call on
// it; host code passes that address, never the array's name, to kernels.
constexpr int64_t kScratchFloats = int64_t(8) << 20;  // 32 MiB
constexpr int kMaxDevices = 64;

__device__ __align__(256) float scratch[kScratchFloats];

std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices] = {};

int scratch_address(hipStream_t stream, float** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SRWM_ERR_HIP;
    if (stream != nullptr) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return SRWM_ERR_HIP;
        if (sdev != dev) return SRWM_ERR_ARG;  // the scratch used is the current device's
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return SRWM_ERR_HIP;
        g_scratch[dev] = static_cast<float*>(ptr);
    }
    *out = g_scratch[dev];
    return SRWM_OK;
}

int backward_noalloc_impl(const srwm_backward_args_t* a)
{
    BwdPlan plan;
    int rc = backward_check(a, false, &plan);
    if (rc != SRWM_OK) return rc;
    const hipStream_t st = static_cast<hipStream_t>(a->stream);
    if (plan.per_b == 0) return SRWM_OK;  // H == 0
    if (plan.per_b > kScratchFloats) return SRWM_ERR_SCRATCH;  // one sequence's gradients do not fit
    if (plan.units == 0) return launch_batch_sum(nullptr, a->dW0, 0, plan.per_b, 0, st);
    float* dwi = nullptr;
    rc = scratch_address(st, &dwi);
    if (rc != SRWM_OK) return rc;
    // Slices of whole sequences, as even as the scratch allows; the kernel is
    // the one srwm_backward takes for the whole batch, and the batch sum
    // continues from slice to slice in order, so dx and dW0 are bit-identical
    // to srwm_backward's.
    const int64_t bmax = kScratchFloats / plan.per_b;
    const int64_t nslices = (a->B + bmax - 1) / bmax;
    const int64_t bs = (a->B + nslices - 1) / nslices;
    for (int64_t b0 = 0; b0 < a->B; b0 += bs) {
        const int64_t n = (a->B - b0) < bs ? (a->B - b0) : bs;
        rc = launch_backward(plan, a, b0, n, dwi);
        if (rc != SRWM_OK) return rc;
        rc = launch_batch_sum(dwi, a->dW0, n, plan.per_b, b0 > 0 ? 1 : 0, st);
        if (rc != SRWM_OK) return rc;
    }
    return SRWM_OK;
}

}  // namespace

extern "C" {

int srwm_backward(const srwm_backward_args_t* args) { return backward_impl(args); }

int srwm_backward_noalloc(const srwm_backward_args_t* args) { return backward_noalloc_impl(args); }

int64_t srwm_backward_noalloc_scratch_bytes(void) { return kScratchFloats * 4; }

int srwm_backward_resources(int64_t d_in, int64_t d_out, int n_lr, int reset, int64_t units,
                            srwm_kernel_resources_t* out)
{
    if (n_lr != 1 && n_lr != 4) return SRWM_ERR_ARG;
    if (units < 0) return SRWM_ERR_SHAPE;
    if (out == nullptr) return SRWM_ERR_NULL;
    const int vi = find_bwd(d_in, d_out, n_lr, reset ? 1 : 0, units);
    if (vi < 0) return SRWM_ERR_UNSUPPORTED;
    return kernel_resources(reinterpret_cast<const void*>(kBwdVariants[vi].fn), kBwdVariants[vi].nw * kWave, out);
}

int srwm_backward_supported(int64_t d_in, int64_t d_out, int io_dtype, int n_lr)
{
    if (io_dtype != SRWM_IO_F32 && io_dtype != SRWM_IO_BF16) return 0;
    for (int i = 0; i < kNumBwdVariants; ++i) {
        const BwdVariant& v = kBwdVariants[i];
        if (v.d_in == d_in && v.d_out == d_out && v.nlr == n_lr) return 1;
    }
    return 0;
}

}  // extern "C"
