// srwm_bwd.hip -- gfx950 backward pass of the SRWM recurrence and its C ABI
// (srwm_backward): gradients of a loss on y_1..y_T and W_T with respect to x
// and the initial state, from the tape the forward pass records.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

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

int backward_impl(const srwm_backward_args_t* a)
{
    if (a == nullptr) return SRWM_ERR_NULL;
    const int64_t B = a->B, T = a->T, H = a->H, d_in = a->d_in, d_out = a->d_out, m = a->m;
    if (B < 0 || T < 0 || H < 0 || d_in < 1 || d_out < 1) return SRWM_ERR_SHAPE;
    if (a->n_lr != 1 && a->n_lr != 4) return SRWM_ERR_ARG;
    if (m != d_out + 2 * d_in + a->n_lr) return SRWM_ERR_SHAPE;
    if (a->io_dtype != SRWM_IO_F32 && a->io_dtype != SRWM_IO_BF16) return SRWM_ERR_ARG;
    if (a->apply_input_softmax != 0 && a->apply_input_softmax != 1) return SRWM_ERR_ARG;
    if (a->reset_interval < 0 || a->reset_interval > INT32_MAX) return SRWM_ERR_ARG;
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
    if ((nst > 0 && (a->W_T == nullptr || a->dW_init == nullptr)) || (ntape > 0 && a->tape == nullptr) ||
        (ndx > 0 && a->dx == nullptr) || (ngy > 0 && a->gy == nullptr) ||
        (nws > 0 && a->window_states == nullptr))
        return SRWM_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(a->W_T) |
         reinterpret_cast<uintptr_t>(a->tape) | reinterpret_cast<uintptr_t>(a->gy) |
         reinterpret_cast<uintptr_t>(a->gW_T) | reinterpret_cast<uintptr_t>(a->dx) |
         reinterpret_cast<uintptr_t>(a->dW_init) | reinterpret_cast<uintptr_t>(a->dW0) |
         reinterpret_cast<uintptr_t>(nws > 0 ? a->window_states : nullptr)) & 15u)
        return SRWM_ERR_ARG;
    hipStream_t st = static_cast<hipStream_t>(a->stream);
    auto sum_over_batch = [&]() -> int {
        // dW0 = sum over b of dW_init (zero when B == 0)
        const int64_t per_b = H * m * d_in;
        if (a->dW0 == nullptr || per_b == 0) return SRWM_OK;
        const float* dWi = a->dW_init;
        float* dW0 = a->dW0;
        int64_t Bv = B, pb = per_b;
        void* args2[] = {const_cast<float**>(&dWi), &dW0, &Bv, &pb};
        const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&srwm_sum_over_batch_kernel),
                                             dim3(static_cast<unsigned>((per_b + 255) / 256)), dim3(256),
                                             args2, 0, st);
        return e == hipSuccess ? SRWM_OK : SRWM_ERR_HIP;
    };
    if (units == 0) return sum_over_batch();
    const float* wstates = nws > 0 ? a->window_states : nullptr;
    const void* ins[] = {a->W_T, a->tape, a->gy, a->gW_T, wstates};
    const int64_t nins[] = {nst, ntape, ngy, a->gW_T ? nst : 0, nws};
    void* outs[] = {a->dx, a->dW_init, a->dW0};
    const int64_t nouts[] = {ndx, nst, a->dW0 ? nw0 : 0};
    for (int o = 0; o < 3; ++o) {
        for (int i = 0; i < 5; ++i)
            if (ranges_overlap(outs[o], nouts[o], ins[i], nins[i])) return SRWM_ERR_ALIAS;
        for (int o2 = o + 1; o2 < 3; ++o2)
            if (ranges_overlap(outs[o], nouts[o], outs[o2], nouts[o2])) return SRWM_ERR_ALIAS;
    }
    const BwdVariant& v = kBwdVariants[vi];
    const float* WTp = a->W_T;
    const float* tape = a->tape;
    const float* gy = a->gy;
    const float* gWT = a->gW_T;
    float* dx = a->dx;
    float* dWi = a->dW_init;
    int Ti = static_cast<int>(T), Hi = static_cast<int>(H), fl = a->apply_input_softmax;
    int rst = static_cast<int>(a->reset_interval);
    void* args[] = {const_cast<float**>(&WTp), const_cast<float**>(&tape),
                    const_cast<float**>(&gy), const_cast<float**>(&gWT), &dx, &dWi, &Ti, &Hi, &fl, &rst,
                    const_cast<float**>(&wstates)};
    const hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(v.fn),
                                           dim3(static_cast<unsigned>(units)), dim3(v.nw * kWave), args, 0, st);
    if (err != hipSuccess) return SRWM_ERR_HIP;
    return sum_over_batch();
}

}  // namespace

extern "C" {

int srwm_backward(const srwm_backward_args_t* args) { return backward_impl(args); }

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
