// srwm_calib.hip -- measurement aid: the chip's scalar FP32 FMA rate, against
// which the kernels' executed arithmetic is compared (the peak the product
// kernels can reach: packed FP32 instructions are disabled at build time, so
// every FMA is a single-lane v_fma_f32 / v_fmac_f32).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "srwm.h"

namespace {

constexpr int kChains = 8;  // independent FMA chains per lane: enough to cover the FMA latency

__global__ __launch_bounds__(256) void srwm_valu_probe_kernel(float* __restrict__ out, int iters, float b,
                                                              float c)
{
    float a[kChains];
#pragma unroll
    for (int i = 0; i < kChains; ++i) a[i] = static_cast<float>(threadIdx.x + i) * 1e-3f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 16; ++u)
#pragma unroll
            for (int i = 0; i < kChains; ++i) a[i] = fmaf(a[i], b, c);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kChains; ++i) s += a[i];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

int srwm_valu_probe(float* out, int64_t workgroups, int iters, void* stream)
{
    if (out == nullptr) return SRWM_ERR_NULL;
    if (workgroups < 1 || workgroups > INT32_MAX || iters < 1) return SRWM_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(out) & 15u) return SRWM_ERR_ARG;
    int it = iters;
    float b = 0.999f, c = 1e-3f;
    void* args[] = {&out, &it, &b, &c};
    const hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(&srwm_valu_probe_kernel),
                                           dim3(static_cast<unsigned>(workgroups)), dim3(256), args, 0,
                                           static_cast<hipStream_t>(stream));
    return err == hipSuccess ? SRWM_OK : SRWM_ERR_HIP;
}

int64_t srwm_valu_probe_flop(int64_t workgroups, int iters)
{
    return workgroups * 256 * static_cast<int64_t>(iters) * 16 * kChains * 2;
}

}  // extern "C"
