// srwm_device.h -- device helpers shared by the forward and backward kernels
// of libsrwm (gfx950): cross-lane reductions on DPP, the hardware exp2 and
// reciprocal, bf16 conversion, 16-byte vector moves; and the host-side
// argument checks both entry points use.
#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "srwm.h"

namespace srwm {

constexpr int kWave = 64;

// ----------------------------------------------------------------------------
// Cross-lane helpers (GFX9 DPP encodings).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within 16

// bound_ctrl is set: every source lane the DPP patterns used here read
// (quad_perm, row mirrors and rotations, row_newbcast) is valid, so the old
// value is never used, and the compiler need not write it to the
// destination before each move.
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of P adjacent lanes (P | 16); every lane of the
// group gets the same bits (fp addition is commutative).
template <int P>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert(P == 1 || P == 2 || P == 4 || P == 8 || P == 16, "P");
    if constexpr (P >= 2) v += dpp<kDppXor1>(v);
    if constexpr (P >= 4) v += dpp<kDppXor2>(v);
    if constexpr (P >= 8) v += dpp<kDppHalfMirror>(v);
    if constexpr (P >= 16) v += dpp<kDppMirror>(v);
    return v;
}

// Lane c of this lane's 16-lane DPP row (row_newbcast:c); k must fold to a
// constant.
__device__ __forceinline__ float row_bcast(float v, int k)
{
    switch (k) {
    case 0: return dpp<0x150>(v);
    case 1: return dpp<0x151>(v);
    case 2: return dpp<0x152>(v);
    case 3: return dpp<0x153>(v);
    case 4: return dpp<0x154>(v);
    case 5: return dpp<0x155>(v);
    case 6: return dpp<0x156>(v);
    case 7: return dpp<0x157>(v);
    case 8: return dpp<0x158>(v);
    case 9: return dpp<0x159>(v);
    case 10: return dpp<0x15A>(v);
    case 11: return dpp<0x15B>(v);
    case 12: return dpp<0x15C>(v);
    case 13: return dpp<0x15D>(v);
    case 14: return dpp<0x15E>(v);
    default: return dpp<0x15F>(v);
    }
}

// max(a, b) for finite or infinite operands: the median of {a, b, +inf}, one
// v_med3_f32 (a compare and select would need a VCC hazard wait between them;
// a NaN operand is dropped here and still reaches the softmax through exp).
__device__ __forceinline__ float fmax2(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, INFINITY); }

// Order-preserving map of a float to a signed int (an involution): positive
// floats keep their bits, negative ones flip their magnitude bits, so signed
// integer max equals float max (integer max fuses with DPP; float max would
// need NaN canonicalisation of both operands).
__device__ __forceinline__ int order_key(float f)
{
    const int b = __float_as_int(f);
    return b ^ static_cast<int>(static_cast<unsigned>(b >> 31) >> 1);
}

__device__ __forceinline__ float from_order_key(int k)
{
    return __int_as_float(k ^ static_cast<int>(static_cast<unsigned>(k >> 31) >> 1));
}

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}


template <int P>
__device__ __forceinline__ float group_max(float v)
{
    int k = order_key(v);
    if constexpr (P >= 2) k = max(k, dpp_i<kDppXor1>(k));
    if constexpr (P >= 4) k = max(k, dpp_i<kDppXor2>(k));
    if constexpr (P >= 8) k = max(k, dpp_i<kDppHalfMirror>(k));
    if constexpr (P >= 16) k = max(k, dpp_i<kDppMirror>(k));
    return from_order_key(k);
}

__device__ __forceinline__ float readlane(float v, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Wave-uniform max / sum over all 64 lanes (the cross-row step runs on the
// scalar unit for the max).
__device__ __forceinline__ float wave_max(float v)
{
    int k = order_key(v);
    k = max(k, dpp_i<kDppXor1>(k));
    k = max(k, dpp_i<kDppXor2>(k));
    k = max(k, dpp_i<kDppHalfMirror>(k));
    k = max(k, dpp_i<kDppMirror>(k));
    const int m = max(max(__builtin_amdgcn_readlane(k, 0), __builtin_amdgcn_readlane(k, 16)),
                      max(__builtin_amdgcn_readlane(k, 32), __builtin_amdgcn_readlane(k, 48)));
    return from_order_key(m);
}

__device__ __forceinline__ float wave_sum(float v)
{
    v = group_sum<16>(v);
    return (readlane(v, 0) + readlane(v, 16)) + (readlane(v, 32) + readlane(v, 48));
}

// Lane-row exchanges of gfx950: v_permlane32_swap swaps DPP rows 2-3 of its
// first operand with rows 0-1 of its second; v_permlane16_swap swaps the odd
// rows of the first with the even rows of the second (a row is 16 lanes).
__device__ __forceinline__ void swap32(float& x, float& y)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    x = __uint_as_float(r[0]);
    y = __uint_as_float(r[1]);
}

__device__ __forceinline__ void swap16(float& x, float& y)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    x = __uint_as_float(r[0]);
    y = __uint_as_float(r[1]);
}

// Sum of v over the lane pair that differs in lane bit B (B = 3, 4 or 5).
template <int B>
__device__ __forceinline__ float pair_sum(float v)
{
    static_assert(B >= 3 && B <= 5, "lane bit");
    if constexpr (B == 3) {
        return v + dpp<0x128>(v);  // row_ror:8 -- lane i+8 mod 16, i.e. i ^ 8
    } else {
        float x = v, y = v;
        if constexpr (B == 4) swap16(x, y);
        else swap32(x, y);
        return x + y;
    }
}

// Sum over all 64 lanes, the same bits in every lane.
__device__ __forceinline__ float wave_total(float v)
{
    v = group_sum<16>(v);
    return pair_sum<5>(pair_sum<4>(v));
}

// Max over all 64 lanes of two values at once, the same bits in every lane:
// the 16-lane DPP trees, then one lane-row swap pairs the two values' row
// results (rows 0, 2 carry a's pairs, rows 1, 3 b's), a second joins the two
// halves and a third hands every row both totals.  Seven instructions after
// the trees instead of two readlane chains, and no scalar-register hazards.
__device__ __forceinline__ void wave_max2(float& a, float& b)
{
    int ka = order_key(a), kb = order_key(b);
    ka = max(ka, dpp_i<kDppXor1>(ka));
    kb = max(kb, dpp_i<kDppXor1>(kb));
    ka = max(ka, dpp_i<kDppXor2>(ka));
    kb = max(kb, dpp_i<kDppXor2>(kb));
    ka = max(ka, dpp_i<kDppHalfMirror>(ka));
    kb = max(kb, dpp_i<kDppHalfMirror>(kb));
    ka = max(ka, dpp_i<kDppMirror>(ka));
    kb = max(kb, dpp_i<kDppMirror>(kb));
    // rows (0,1) of a meet in row 0, of b in row 1; rows (2,3) in rows 2 / 3
    auto r = __builtin_amdgcn_permlane16_swap(static_cast<unsigned>(ka), static_cast<unsigned>(kb), false, false);
    const int t = max(static_cast<int>(r[0]), static_cast<int>(r[1]));
    r = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(t), static_cast<unsigned>(t), false, false);
    const int u = max(static_cast<int>(r[0]), static_cast<int>(r[1]));  // rows 0, 2: a; rows 1, 3: b
    r = __builtin_amdgcn_permlane16_swap(static_cast<unsigned>(u), static_cast<unsigned>(u), false, false);
    a = from_order_key(static_cast<int>(r[0]));
    b = from_order_key(static_cast<int>(r[1]));
}

// Sum over all 64 lanes of two values at once (the same pairing as wave_max2).
__device__ __forceinline__ void wave_sum2(float& a, float& b)
{
    a = group_sum<16>(a);
    b = group_sum<16>(b);
    float x = a, y = b;
    swap16(x, y);
    float t = x + y, t2 = t;
    swap32(t, t2);
    float u = t + t2, u2 = u;
    swap16(u, u2);
    a = u;
    b = u2;
}

// Max / sum over each half-wave (lanes 0-31 and 32-63 separately): the DPP
// tree inside 16-lane rows, then rows 0+1 and 2+3 joined by one lane-row
// swap.  Every lane of a half ends with the same bits.
__device__ __forceinline__ float half_max(float v)
{
    int k = order_key(v);
    k = max(k, dpp_i<kDppXor1>(k));
    k = max(k, dpp_i<kDppXor2>(k));
    k = max(k, dpp_i<kDppHalfMirror>(k));
    k = max(k, dpp_i<kDppMirror>(k));
    const auto r = __builtin_amdgcn_permlane16_swap(static_cast<unsigned>(k), static_cast<unsigned>(k), false, false);
    return from_order_key(max(static_cast<int>(r[0]), static_cast<int>(r[1])));
}

// half_max as float max with DPP operands, written out: the compiler cannot
// fuse a DPP move into v_max_f32 itself (IEEE mode makes it canonicalise both
// operands first), so the order-preserving integer form above costs six
// conversions that this form does not.  Each DPP read follows its operand's
// write by two wait states (s_nop 1), and a trailing s_nop 1 covers a
// consumer placed right after the block.  NaN operands are dropped, as by
// fmax2.  Faster where several waves share a SIMD; one-wave units, which
// interleave the integer form with other work, keep that.
__device__ __forceinline__ float half_max_f(float v)
{
    float r = v, t;
    asm("s_nop 1\n\t"
        "v_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "s_nop 1\n\t"
        "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "s_nop 1\n\t"
        "v_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "s_nop 1\n\t"
        "v_max_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_mov_b32 %1, %0\n\t"
        "s_nop 1\n\t"
        "v_permlane16_swap_b32 %0, %1\n\t"
        "s_nop 1\n\t"
        "v_max_f32 %0, %0, %1\n\t"
        "s_nop 1"
        : "+v"(r), "=&v"(t));
    return r;
}

__device__ __forceinline__ float half_sum(float v)
{
    return pair_sum<4>(group_sum<16>(v));
}

// e^x as 2^(x log2 e) on the hardware exp2 (v_exp_f32).
__device__ __forceinline__ float exp_f32(float x)
{
    return __builtin_amdgcn_exp2f(x * 1.44269504088896340736f);
}

// e^(x - m) given ms = m log2(e): 2^(x log2 e - ms), the shift and the scale
// in one multiply-add.
__device__ __forceinline__ float exp_shifted(float x, float ms)
{
    return __builtin_amdgcn_exp2f(fmaf(x, 1.44269504088896340736f, -ms));
}

__device__ __forceinline__ float log2e_scaled(float m) { return m * 1.44269504088896340736f; }

// 1/x on the hardware reciprocal (v_rcp_f32, 1 ulp).
__device__ __forceinline__ float rcp_f32(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ float sigmoid_f32(float z)
{
    return rcp_f32(1.0f + exp_f32(-z));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h)
{
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float32 -> bfloat16, round to nearest, ties to even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two floats to bf16 in one conversion (round to nearest even, as
// f32_to_bf16): a in the low half, b in the high half.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Load N consecutive floats (16-byte aligned when N % 4 == 0).
template <int N>
__device__ __forceinline__ void load_f32(const float* __restrict__ src, float (&dst)[N])
{
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const float4 v = reinterpret_cast<const float4*>(src)[i];
            dst[4 * i + 0] = v.x;
            dst[4 * i + 1] = v.y;
            dst[4 * i + 2] = v.z;
            dst[4 * i + 3] = v.w;
        }
    } else if constexpr (N % 2 == 0) {
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            const float2 v = reinterpret_cast<const float2*>(src)[i];
            dst[2 * i + 0] = v.x;
            dst[2 * i + 1] = v.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) dst[i] = src[i];
    }
}

template <int N>
__device__ __forceinline__ void store_f32(float* __restrict__ dst, const float (&src)[N])
{
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N / 4; ++i)
            reinterpret_cast<float4*>(dst)[i] =
                make_float4(src[4 * i], src[4 * i + 1], src[4 * i + 2], src[4 * i + 3]);
    } else if constexpr (N % 2 == 0) {
#pragma unroll
        for (int i = 0; i < N / 2; ++i)
            reinterpret_cast<float2*>(dst)[i] = make_float2(src[2 * i], src[2 * i + 1]);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) dst[i] = src[i];
    }
}


// Make this wave's LDS stores visible to its own later LDS loads from other
// lanes (DS operations of one wave complete in order; this orders them in the
// compiler and waits for the stores).
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Asynchronous copy of one dword per active lane from a buffer straight into
// LDS (gfx950 buffer_load_dword ... lds): lane i of the wave reads the dword
// at byte voff + soff of the buffer described by rsrc and writes lds_base[i],
// lds_base uniform over the wave.  voff is the lane's own byte offset, soff a
// wave-uniform one; a read past the resource's num_records yields zero.  The
// copy is tracked by vmcnt: wait_vmem() before the workgroup barrier after
// which the LDS words are read.
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ void copy_dword_to_lds(__amdgpu_buffer_rsrc_t rsrc, int voff, int soff, float* lds_base)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(lds_base), 4, voff, soff, 0, 0);
}

// The same copy, 16 bytes per active lane (gfx950 buffer_load_dwordx4 ...
// lds): lane i writes the 16 bytes at lds_base + 16 i.
__device__ __forceinline__ void copy_x4_to_lds(__amdgpu_buffer_rsrc_t rsrc, int voff, int soff, void* lds_base)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(lds_base), 16, voff, soff, 0, 0);
}

// Buffer resource over n floats at base (raw buffer, bounds-checked against
// n * 4 bytes): its four dwords are wave-uniform, so they live in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t float_rsrc(const float* base, int n)
{
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, n * 4, 0x00020000);
}

// The lane's index in its wave, computed afresh at each call (two VALU
// instructions with no register inputs; volatile, so never hoisted): for a
// lane-constant LDS address used once per loop iteration in a kernel whose
// registers are full, cheaper than holding the address live across the loop,
// which there means a spill and a scratch reload with a wait on every
// outstanding vector-memory operation.
__device__ __forceinline__ int lane_now()
{
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// s_waitcnt vmcnt(0): every vector memory operation of this wave has completed
// (expcnt and lgkmcnt left at their maxima).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Keep v materialised in every lane at this point: a value that only some
// lanes store afterwards would otherwise have its last reduction step sunk
// into the store's branch, where the DPP add can no longer be fused (an extra
// move and a separate add per value).  Emits no instruction.
__device__ __forceinline__ void keep(float& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ float uniform(float v)
{
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// ----------------------------------------------------------------------------
// The backward tape: one float32 row per (unit, step), written by the forward
// pass and read by the backward pass.
//   [0, m)                a_t, the row factor of the step's rank-one update
//   [m, KH_OFF)           padding to a 16-byte boundary (zeros, or not written)
//   [KH_OFF, E_OFF)       phi(k_t)
//   [E_OFF, G_OFF)        phi(q_t) - phi(k_t), as the forward pass rounded it
//   [G_OFF, U_OFF)        the learning rates sigma(beta_t) (n_lr of them, rest zero)
//   [U_OFF, ROW)          u_t, the step's input as the projection used it (x_t
//                         widened, softmax-ed when the input softmax is on)
template <int M, int D_IN>
struct TapeLayout {
    static constexpr int KH_OFF = (M + 3) & ~3;
    static constexpr int E_OFF = KH_OFF + D_IN;
    static constexpr int G_OFF = E_OFF + D_IN;
    static constexpr int U_OFF = G_OFF + 4;
    static constexpr int ROW = U_OFF + D_IN;
};

inline int64_t tape_row(int64_t d_in, int64_t d_out, int64_t n_lr)
{
    return ((d_out + 2 * d_in + n_lr + 3) & ~int64_t(3)) + 3 * d_in + 4;
}

// ----------------------------------------------------------------------------
// Host-side helpers.

// A kernel's registers, LDS, scratch and occupancy for `threads` threads per
// workgroup, from the runtime's view of the loaded code object.
inline int kernel_resources(const void* fn, int threads, srwm_kernel_resources_t* out)
{
    hipFuncAttributes fa;
    if (hipFuncGetAttributes(&fa, fn) != hipSuccess) return SRWM_ERR_HIP;
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, threads, 0) != hipSuccess) return SRWM_ERR_HIP;
    out->vgprs = fa.numRegs;
    out->lds_bytes = static_cast<int>(fa.sharedSizeBytes);
    out->scratch_bytes = static_cast<int>(fa.localSizeBytes);
    out->threads = threads;
    out->workgroups_per_cu = blocks;
    out->waves_per_simd = blocks * (threads / kWave) / 4;
    return SRWM_OK;
}

inline bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb)
{
    if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

inline bool mul_ok(int64_t a, int64_t b, int64_t* out)
{
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

// A validated forward call: the variant, the units and the window-state
// buffer its kernel gets, and whether any kernel runs.  forward_check
// validates exactly as srwm_forward_ex; forward_launch launches the kernel of
// a plan with the buffers, T and t_stride of `a` and checks nothing (the
// chunks of a validated call may read their initial state from W_T in place:
// every lane loads its own state elements before it writes them back).
struct FwdPlan {
    int vi;
    int waves;  // of the variant's workgroup
    int64_t units;
    float* wstates;
    bool run;
};
int forward_check(const srwm_forward_args_t* a, FwdPlan* plan);
int forward_launch(const FwdPlan& plan, const srwm_forward_args_t* a);

}  // namespace srwm
