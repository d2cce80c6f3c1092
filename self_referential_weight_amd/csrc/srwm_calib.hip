// srwm_calib.hip -- measurement aids: the chip's scalar FP32 FMA rate, against
// which the kernels' executed arithmetic is compared (the peak the product
// kernels can reach: packed FP32 instructions are disabled at build time, so
// every FMA is a single-lane v_fma_f32 / v_fmac_f32), and its LDS read
// bandwidth, against which the kernels' LDS traffic is compared.
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

// LDS read bandwidth: every lane reads 16-byte pieces (ds_read_b128) from a
// 32 KB LDS array, a wave's 64 lanes one contiguous 1 KB span (no bank
// conflicts).  Per iteration the 16 reads of a lane sit 1 KB apart from one
// base (immediate offsets: no address arithmetic per read), and the base moves
// by 13 entries per iteration, so no read can be hoisted out of the loop or
// merged with the last iteration's.  The values are folded with three-input
// integer adds (two VALU instructions per 16-byte read: a wave's 1 KB read
// costs 8 SIMD cycles of issue, so the VALU could keep up with 512 B per
// clock per CU), and the reads set the pace.  Four waves per workgroup, several workgroups
// per CU.
constexpr int kLdsVec = 2048;  // float4 entries of the array (32 KB)
constexpr int kLdsUnroll = 16;

__global__ __launch_bounds__(256) void srwm_lds_probe_kernel(unsigned* __restrict__ out, int iters)
{
    __shared__ uint4 buf[kLdsVec];
    const int t = threadIdx.x;
    for (int i = t; i < kLdsVec; i += 256)
        buf[i] = make_uint4(i * 2654435761u, i ^ 0x9e3779b9u, i + 7u, ~i);
    __syncthreads();
    unsigned a = t, b = t * 3u;
    for (int it = 0; it < iters; ++it) {
        const uint4* __restrict__ base = buf + ((t + 13 * it) & 1023);  // + 15 KB stays inside the array
#pragma unroll
        for (int u = 0; u < kLdsUnroll; ++u) {
            const uint4 v = base[64 * u];
            a = a + v.x + v.y;  // v_add3_u32
            b = b + v.z + v.w;
        }
    }
    out[blockIdx.x * blockDim.x + t] = a + b;
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

int srwm_lds_probe(unsigned* out, int64_t workgroups, int iters, void* stream)
{
    if (out == nullptr) return SRWM_ERR_NULL;
    if (workgroups < 1 || workgroups > INT32_MAX || iters < 1) return SRWM_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(out) & 15u) return SRWM_ERR_ARG;
    int it = iters;
    void* args[] = {&out, &it};
    const hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(&srwm_lds_probe_kernel),
                                           dim3(static_cast<unsigned>(workgroups)), dim3(256), args, 0,
                                           static_cast<hipStream_t>(stream));
    return err == hipSuccess ? SRWM_OK : SRWM_ERR_HIP;
}

int64_t srwm_lds_probe_bytes(int64_t workgroups, int iters)
{
    return workgroups * 256 * static_cast<int64_t>(iters) * kLdsUnroll * 16;
}

}  // extern "C"
