// srwm_fwd.hip -- gfx950 kernels and C ABI of libsrwm.
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

#include <type_traits>

#include "srwm.h"

namespace {

constexpr int kWave = 64;

// ----------------------------------------------------------------------------
// Cross-lane helpers (GFX9 DPP encodings).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within 16

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
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

// max(a, b) for finite or infinite operands (no NaN canonicalisation).
__device__ __forceinline__ float fmax2(float a, float b) { return a > b ? a : b; }

template <int P>
__device__ __forceinline__ float group_max(float v)
{
    if constexpr (P >= 2) v = fmax2(v, dpp<kDppXor1>(v));
    if constexpr (P >= 4) v = fmax2(v, dpp<kDppXor2>(v));
    if constexpr (P >= 8) v = fmax2(v, dpp<kDppHalfMirror>(v));
    if constexpr (P >= 16) v = fmax2(v, dpp<kDppMirror>(v));
    return v;
}

__device__ __forceinline__ float readlane(float v, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Wave-uniform max / sum over all 64 lanes.
__device__ __forceinline__ float wave_max(float v)
{
    v = group_max<16>(v);
    return fmax2(fmax2(readlane(v, 0), readlane(v, 16)), fmax2(readlane(v, 32), readlane(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v)
{
    v = group_sum<16>(v);
    return (readlane(v, 0) + readlane(v, 16)) + (readlane(v, 32) + readlane(v, 48));
}

// e^x as 2^(x log2 e) on the hardware exp2 (v_exp_f32).
__device__ __forceinline__ float exp_f32(float x)
{
    return __builtin_amdgcn_exp2f(x * 1.44269504088896340736f);
}

__device__ __forceinline__ float sigmoid_f32(float z)
{
    return 1.0f / (1.0f + exp_f32(-z));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h)
{
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float32 -> bfloat16, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
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

// ----------------------------------------------------------------------------
// Compile-time geometry of one kernel variant.
//
// Main rows (the y, k and q blocks, MAIN = d_out + 2*d_in rows) use the
// strided lane layout described at the top of the file.  The four beta rows
// use one of two layouts:
//   BETA_SEP (d_in % 16 == 0): wave 0 holds them, DPP row i (lanes 16i..16i+15)
//     holding beta row i, LB = d_in/16 consecutive columns per lane; a beta
//     row's dot product is then a 16-lane DPP sum inside one DPP row, and the
//     lanes that need its learning-rate term are the ones that computed it.
//   otherwise: they are appended to the main rows (one extra register row,
//     zero padded), which only the small test shapes use.
template <int D_IN, int D_OUT, int NW, int P>
struct Geom {
    static constexpr int NT = NW * kWave;          // threads per unit
    static constexpr int M = D_OUT + 2 * D_IN + 4; // rows of W
    static constexpr int MAIN = D_OUT + 2 * D_IN;  // y, k, q rows
    static constexpr bool BETA_SEP = (D_IN % 16 == 0);
    static constexpr int ROWS = BETA_SEP ? MAIN : M; // rows in the strided layout
    static constexpr int L = D_IN / P;             // columns per lane
    static constexpr int G = NT / P;               // row groups
    static constexpr int R = (ROWS + G - 1) / G;   // rows per lane
    static constexpr bool ALIGNED = (D_IN % G == 0) && (D_OUT % G == 0);
    static constexpr int LB = BETA_SEP ? D_IN / 16 : 0; // beta columns per lane
    // x staging: E consecutive elements per lane, LR lanes per step row.
    // Aim for 32 step rows per chunk (8 for one-wave units, whose registers
    // are scarcer) with every lane loading, at most 16 and at least d_in/16
    // elements per lane (so a row spans <= 16 lanes).
    static constexpr int E_TARGET = ((NW == 1 ? 8 : 32) * D_IN) / NT;
    static constexpr int E_LO = D_IN / 16 > E_TARGET ? D_IN / 16 : E_TARGET;
    static constexpr int E = D_IN < 16 ? D_IN : (E_LO < 16 ? (E_LO < 1 ? 1 : E_LO) : 16);
    static constexpr int LR = D_IN / E;
    static constexpr int S_FULL = NT / LR;
    static constexpr int S = S_FULL < 32 ? S_FULL : 32; // steps per chunk
    static_assert(D_IN % P == 0, "P must divide d_in");
    static_assert(D_IN % E == 0, "E must divide d_in");
    static_assert(LR <= 16 && (LR & (LR - 1)) == 0, "row lanes");
    static_assert(G >= 4, "need at least four row groups");
    // Row block (0 y, 1 k, 2 q, 3 beta) of register r when ALIGNED.
    static constexpr int block_of_reg(int r)
    {
        const int row = G * r;
        return row < D_OUT ? 0 : row < D_OUT + D_IN ? 1 : row < D_OUT + 2 * D_IN ? 2 : 3;
    }
};

__device__ __forceinline__ int block_of_row(int row, int d_in, int d_out)
{
    return row < d_out ? 0 : row < d_out + d_in ? 1 : row < d_out + 2 * d_in ? 2 : 3;
}

// phi(k) and phi(q) by one wave: k and q are d-vectors in LDS; lanes take
// entries lane, lane+64, ...  Writes kh = softmax(k) and e = softmax(q) - kh,
// the difference the fused read of Eq. (2) needs.  The two reductions are
// interleaved for ILP.
template <int D>
__device__ __forceinline__ void wave_addresses(const float* __restrict__ k, const float* __restrict__ q,
                                               float* __restrict__ kh_out, float* __restrict__ e_out,
                                               int lane)
{
    constexpr int EPL = (D + 63) / 64;
    float a[EPL], b[EPL];
    float ma = -INFINITY, mb = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int j = lane + 64 * i;
        a[i] = (j < D) ? k[j] : -INFINITY;
        b[i] = (j < D) ? q[j] : -INFINITY;
        ma = fmax2(ma, a[i]);
        mb = fmax2(mb, b[i]);
    }
    ma = wave_max(ma);
    mb = wave_max(mb);
    float sa = 0.f, sb = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int j = lane + 64 * i;
        a[i] = (j < D) ? exp_f32(a[i] - ma) : 0.f;
        b[i] = (j < D) ? exp_f32(b[i] - mb) : 0.f;
        sa += a[i];
        sb += b[i];
    }
    const float ia = 1.0f / wave_sum(sa);
    const float ib = 1.0f / wave_sum(sb);
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int j = lane + 64 * i;
        if (j < D) {
            // Both probabilities are rounded before the difference (no fused
            // multiply-subtract), so k_t == q_t gives e == 0 exactly.
#pragma clang fp contract(off)
            const float kh = a[i] * ia;
            const float qh = b[i] * ib;
            kh_out[j] = kh;
            e_out[j] = qh - kh;
        }
    }
}

// Width of the LDS vector pieces streamed through the FMA loops.
template <int N>
struct Piece {
    static constexpr int W = N % 4 == 0 ? 4 : N % 2 == 0 ? 2 : 1;
};

// Stream src[0..N) from LDS in pieces of Piece<N>::W floats through
// body(c, value), double-buffered: piece k+1 is requested before piece k is
// consumed, and a scheduling barrier after each piece keeps the compiler from
// hoisting later pieces (which would hold the whole vector in VGPRs).
template <int N, class F>
__device__ __forceinline__ void stream_lds(const float* __restrict__ src, F&& body)
{
    constexpr int VW = Piece<N>::W;
    constexpr int NPC = N / VW;
    float cur[VW];
    load_f32<VW>(src, cur);
#pragma unroll
    for (int k = 0; k < NPC; ++k) {
        float nxt[VW];
        if (k + 1 < NPC) load_f32<VW>(src + (k + 1) * VW, nxt);
#pragma unroll
        for (int c = 0; c < VW; ++c) body(k * VW + c, cur[c]);
        __builtin_amdgcn_sched_barrier(0);
        if (k + 1 < NPC) {
#pragma unroll
            for (int c = 0; c < VW; ++c) cur[c] = nxt[c];
        }
    }
}

__device__ __forceinline__ float uniform(float v)
{
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// ----------------------------------------------------------------------------
// The kernel: grid = B*H workgroups (unit = b*H + h), NW*64 threads each.
// WPE is the occupancy (waves per SIMD) the register allocation must allow.
template <int D_IN, int D_OUT, int NW, int P, int WPE, bool BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * kWave, NW * kWave),
                          amdgpu_waves_per_eu(WPE)))
void srwm_fwd_kernel(const void* __restrict__ xv, const float* __restrict__ W0,
                     void* __restrict__ yv, float* __restrict__ WT, int T, int H, int in_softmax)
{
    using Gm = Geom<D_IN, D_OUT, NW, P>;
    constexpr int M = Gm::M, MAIN = Gm::MAIN, ROWS = Gm::ROWS;
    constexpr int L = Gm::L, G = Gm::G, R = Gm::R, LB = Gm::LB;
    constexpr int E = Gm::E, LR = Gm::LR, S = Gm::S;
    constexpr bool BETA_SEP = Gm::BETA_SEP;

    __shared__ __attribute__((aligned(16))) float s_x[2][S][D_IN];
    __shared__ __attribute__((aligned(16))) float s_z[R * G + 4];
    __shared__ __attribute__((aligned(16))) float s_kh[D_IN]; // phi(k_t)
    __shared__ __attribute__((aligned(16))) float s_e[D_IN];  // phi(q_t) - phi(k_t)
    __shared__ __attribute__((aligned(16))) float s_g[4];     // sigma(beta_t)

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = NW == 1 ? 0 : tid / kWave;
    const int p = tid % P;
    const int rg = tid / P;
    const int unit = blockIdx.x;
    const int b = unit / H;
    const int h = unit - b * H;

    // Element offsets.  x[b][t][h][:] = x0 + t*x_step.
    const int64_t x_step = (int64_t)H * D_IN;
    const int64_t y_step = (int64_t)H * D_OUT;
    const int64_t x0 = ((int64_t)b * T * H + h) * D_IN;
    const int64_t y0 = ((int64_t)b * T * H + h) * D_OUT;
    const float* __restrict__ w0h = W0 + (int64_t)h * M * D_IN;

    // ---- a0: W <- W0[h] into registers.
    float w[R][L];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = rg + G * r;
        if (row < ROWS) {
            load_f32<L>(w0h + (int64_t)row * D_IN + p * L, w[r]);
        } else {
#pragma unroll
            for (int c = 0; c < L; ++c) w[r][c] = 0.f;
        }
    }
    // beta rows (BETA_SEP): wave 0, lane -> row MAIN + lane/16, cols bcol..bcol+LB
    const int bcol = (lane & 15) * (LB > 0 ? LB : 1);
    const int brow = lane >> 4;
    float wb[LB > 0 ? LB : 1];
    if constexpr (BETA_SEP) {
        if (wave == 0) load_f32<LB>(w0h + (int64_t)(MAIN + brow) * D_IN + bcol, wb);
    }

    // ---- x staging: lane tid < S*LR loads E elements of step row tid/LR.
    const int xs_row = tid / LR;
    const int xs_col = (tid % LR) * E;
    const bool xs_active = tid < S * LR;
    constexpr int XR = BF16 ? (E + 1) / 2 : E; // registers held per lane
    uint32_t xr[XR];

    auto load_chunk = [&](int c0) {
        const int t = c0 + xs_row;
        if (xs_active && t < T) {
            if constexpr (BF16) {
                const uint16_t* src = reinterpret_cast<const uint16_t*>(xv) + x0 + (int64_t)t * x_step + xs_col;
                if constexpr (E % 8 == 0) {
#pragma unroll
                    for (int i = 0; i < E / 8; ++i) {
                        const uint4 v = reinterpret_cast<const uint4*>(src)[i];
                        xr[4 * i + 0] = v.x;
                        xr[4 * i + 1] = v.y;
                        xr[4 * i + 2] = v.z;
                        xr[4 * i + 3] = v.w;
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < XR; ++i) {
                        const uint32_t lo = src[2 * i];
                        const uint32_t hi = (2 * i + 1 < E) ? src[2 * i + 1] : 0u;
                        xr[i] = lo | (hi << 16);
                    }
                }
            } else {
                const float* src = reinterpret_cast<const float*>(xv) + x0 + (int64_t)t * x_step + xs_col;
                float tmp[E];
                load_f32<E>(src, tmp);
#pragma unroll
                for (int i = 0; i < E; ++i) xr[i] = __float_as_uint(tmp[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < XR; ++i) xr[i] = 0u;
        }
    };

    // Widen, apply the optional input softmax per step row, write to LDS.
    auto stage_chunk = [&](float (*dst)[D_IN]) {
        float v[E];
#pragma unroll
        for (int i = 0; i < E; ++i) {
            if constexpr (BF16)
                v[i] = __uint_as_float((i & 1) ? (xr[i >> 1] & 0xffff0000u) : (xr[i >> 1] << 16));
            else
                v[i] = __uint_as_float(xr[i]);
        }
        if (in_softmax) {
            float mx = v[0];
#pragma unroll
            for (int i = 1; i < E; ++i) mx = fmax2(mx, v[i]);
            mx = group_max<LR>(mx);
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < E; ++i) {
                v[i] = exp_f32(v[i] - mx);
                s += v[i];
            }
            const float inv = 1.0f / group_sum<LR>(s);
#pragma unroll
            for (int i = 0; i < E; ++i) v[i] *= inv;
        }
        if (xs_active) store_f32<E>(&dst[xs_row][xs_col], v);
    };

    // Phase B roles: wave 0 forms the addresses; WAVE_AUX the gates and y_t.
    constexpr int WAVE_AUX = NW >= 2 ? 1 : 0;

    if (T > 0) {
        load_chunk(0);
        stage_chunk(s_x[0]);
        if (T > S) load_chunk(S);
        __syncthreads();

        int chunk = 0;
        for (int c0 = 0; c0 < T; c0 += S, ++chunk) {
            const int n = (T - c0) < S ? (T - c0) : S;
            const float* sxc = &s_x[chunk & 1][0][0];
            for (int s = 0; s < n; ++s) {
                const int t = c0 + s;
                const float* __restrict__ urow = sxc + s * D_IN;
                // ---- (A) Eq. (1): z = W u.
                float acc[R];
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r] = 0.f;
                stream_lds<L>(urow + p * L, [&](int c, float uc) {
#pragma unroll
                    for (int r = 0; r < R; ++r) acc[r] = fmaf(w[r][c], uc, acc[r]);
                });
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r] = group_sum<P>(acc[r]);
                // All P lanes of a row group hold the same sums; lane p stores
                // registers r = p, p+P, ... (one LDS store per P registers).
#pragma unroll
                for (int r0 = 0; r0 < R; r0 += P) {
                    float v = acc[r0];
#pragma unroll
                    for (int q = 1; q < P && r0 + q < R; ++q) v = (p == q) ? acc[r0 + q] : v;
                    const int row = rg + G * (r0 + p);
                    if ((r0 + P <= R || r0 + p < R) && (Gm::ALIGNED || row < ROWS)) s_z[row] = v;
                }
                if constexpr (BETA_SEP) {
                    if (wave == 0) {
                        float accb = 0.f;
                        stream_lds<LB>(urow + bcol, [&](int c, float uc) { accb = fmaf(wb[c], uc, accb); });
                        accb = group_sum<16>(accb);
                        if ((lane & 15) == 0) s_z[MAIN + brow] = accb;
                    }
                }
                __syncthreads();

                // ---- (B) phi(k), phi(q), sigma(beta); y_t from W_{t-1}.
                if (wave == 0) wave_addresses<D_IN>(s_z + D_OUT, s_z + D_OUT + D_IN, s_kh, s_e, lane);
                if (wave == WAVE_AUX) {
                    if (lane < 4) s_g[lane] = sigmoid_f32(s_z[MAIN + lane]);
#pragma unroll
                    for (int j0 = 0; j0 < D_OUT; j0 += kWave) {
                        const int j = j0 + lane;
                        if (j < D_OUT) {
                            const float zy = s_z[j];
                            if constexpr (BF16)
                                reinterpret_cast<uint16_t*>(yv)[y0 + (int64_t)t * y_step + j] = f32_to_bf16(zy);
                            else
                                reinterpret_cast<float*>(yv)[y0 + (int64_t)t * y_step + j] = zy;
                        }
                    }
                }
                __syncthreads();

                // ---- (C) Eq. (2)/(4) fused: W (qh - kh) = v - vb, times the gate.
                const float g0 = uniform(s_g[0]), g1 = uniform(s_g[1]);
                const float g2 = uniform(s_g[2]), g3 = uniform(s_g[3]);
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r] = 0.f;
                stream_lds<L>(s_e + p * L, [&](int c, float ec) {
#pragma unroll
                    for (int r = 0; r < R; ++r) acc[r] = fmaf(w[r][c], ec, acc[r]);
                });
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float gate;
                    if constexpr (Gm::ALIGNED) {
                        const int bk = Gm::block_of_reg(r);
                        gate = bk == 0 ? g0 : bk == 1 ? g1 : bk == 2 ? g2 : g3;
                    } else {
                        const int bk = block_of_row(rg + G * r, D_IN, D_OUT);
                        gate = bk == 0 ? g0 : bk == 1 ? g1 : bk == 2 ? g2 : g3;
                    }
                    acc[r] = gate * group_sum<P>(acc[r]);
                }
                float accb = 0.f;
                if constexpr (BETA_SEP) {
                    if (wave == 0) {
                        stream_lds<LB>(s_e + bcol, [&](int c, float ec) { accb = fmaf(wb[c], ec, accb); });
                        accb = g3 * group_sum<16>(accb);
                    }
                }
                // ---- (D) Eq. (3)/(5): W += a kh^T, in place.
                stream_lds<L>(s_kh + p * L, [&](int c, float kc) {
#pragma unroll
                    for (int r = 0; r < R; ++r) w[r][c] = fmaf(acc[r], kc, w[r][c]);
                });
                if constexpr (BETA_SEP) {
                    if (wave == 0)
                        stream_lds<LB>(s_kh + bcol, [&](int c, float kc) { wb[c] = fmaf(accb, kc, wb[c]); });
                }
            }
            if (c0 + S < T) {
                stage_chunk(s_x[(chunk + 1) & 1]);
                if (c0 + 2 * S < T) load_chunk(c0 + 2 * S);
                __syncthreads();
            }
        }
    }

    // ---- a7: W_T[b,h] <- W.
    if (WT != nullptr) {
        float* __restrict__ wdst = WT + (int64_t)unit * M * D_IN;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = rg + G * r;
            if (row < ROWS) store_f32<L>(wdst + (int64_t)row * D_IN + p * L, w[r]);
        }
        if constexpr (BETA_SEP) {
            if (wave == 0) store_f32<LB>(wdst + (int64_t)(MAIN + brow) * D_IN + bcol, wb);
        }
    }
}

// ----------------------------------------------------------------------------
// Variant table.
using KernelFn = void (*)(const void*, const float*, void*, float*, int, int, int);

struct Variant {
    int d_in, d_out, io, nw, p, wpe, is_auto;
    KernelFn fn;
};

template <int D_IN, int D_OUT, int NW, int P, int WPE, bool BF16>
constexpr Variant make_variant(int is_auto)
{
    return Variant{D_IN, D_OUT, BF16 ? SRWM_IO_BF16 : SRWM_IO_F32, NW, P, WPE, is_auto,
                   &srwm_fwd_kernel<D_IN, D_OUT, NW, P, WPE, BF16>};
}

#define SRWM_BOTH_IO(DI, DO, NW, P, WPE, AUTO) \
    make_variant<DI, DO, NW, P, WPE, false>(AUTO), make_variant<DI, DO, NW, P, WPE, true>(AUTO)

// (d_in, d_out, waves per unit, lanes per row, waves per SIMD the registers
// allow, eligible for the automatic choice).
const Variant kVariants[] = {
    SRWM_BOTH_IO(2, 2, 1, 2, 1, 1),
    SRWM_BOTH_IO(3, 5, 1, 1, 1, 1),
    SRWM_BOTH_IO(8, 8, 1, 8, 1, 1),
    SRWM_BOTH_IO(8, 16, 1, 8, 1, 1),
    SRWM_BOTH_IO(16, 8, 1, 8, 1, 1),
    SRWM_BOTH_IO(16, 16, 1, 4, 1, 1),
    SRWM_BOTH_IO(32, 32, 1, 4, 1, 1),
    SRWM_BOTH_IO(64, 64, 1, 4, 2, 1),
    SRWM_BOTH_IO(64, 64, 2, 8, 2, 1),
    SRWM_BOTH_IO(64, 64, 4, 8, 1, 1),
    SRWM_BOTH_IO(64, 64, 1, 4, 1, 0),
    SRWM_BOTH_IO(64, 64, 4, 16, 1, 0),
    SRWM_BOTH_IO(128, 128, 8, 16, 1, 1),
    SRWM_BOTH_IO(128, 128, 16, 16, 1, 1),
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

// One wave per SIMD of the chip (256 CUs x 4 SIMDs).
constexpr int64_t kChipSimds = 1024;

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb)
{
    if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out)
{
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

// Automatic choice among the eligible variants of (d_in, d_out, io): the
// fewest waves per unit that still give every SIMD of the chip a wave
// (units * waves >= 1024); if none does, the most waves per unit.
int find_variant(int64_t d_in, int64_t d_out, int io, int requested, int64_t units)
{
    if (requested >= 0) {
        if (requested >= kNumVariants) return -1;
        const Variant& v = kVariants[requested];
        return (v.d_in == d_in && v.d_out == d_out && v.io == io) ? requested : -1;
    }
    int best_fill = -1, best_any = -1;
    for (int i = 0; i < kNumVariants; ++i) {
        const Variant& v = kVariants[i];
        if (v.d_in != d_in || v.d_out != d_out || v.io != io || !v.is_auto) continue;
        if (units * v.nw >= kChipSimds && (best_fill < 0 || v.nw < kVariants[best_fill].nw)) best_fill = i;
        if (best_any < 0 || v.nw > kVariants[best_any].nw) best_any = i;
    }
    return best_fill >= 0 ? best_fill : best_any;
}

int forward_impl(const void* x, const float* W0, void* y, float* W_T, int64_t B, int64_t T,
                 int64_t H, int64_t d_in, int64_t d_out, int64_t m, int io_dtype,
                 int apply_input_softmax, void* stream, int variant)
{
    if (B < 0 || T < 0 || H < 0 || d_in < 1 || d_out < 1) return SRWM_ERR_SHAPE;
    if (m != d_out + 2 * d_in + 4) return SRWM_ERR_SHAPE;
    if (io_dtype != SRWM_IO_F32 && io_dtype != SRWM_IO_BF16) return SRWM_ERR_ARG;
    if (apply_input_softmax != 0 && apply_input_softmax != 1) return SRWM_ERR_ARG;
    if (variant < -1) return SRWM_ERR_ARG;
    const int64_t units_hint = (B > 0 && H > INT64_MAX / B) ? INT64_MAX : B * H;
    const int vi = find_variant(d_in, d_out, io_dtype, variant, units_hint);
    if (vi < 0) return variant >= 0 ? SRWM_ERR_ARG : SRWM_ERR_UNSUPPORTED;
    const int64_t es = io_dtype == SRWM_IO_BF16 ? 2 : 4;
    int64_t units, steps, nx, ny, nw0, nwt;
    if (!mul_ok(B, H, &units) || !mul_ok(units, T, &steps) || !mul_ok(steps, d_in * es, &nx) ||
        !mul_ok(steps, d_out * es, &ny) || !mul_ok(H, m * d_in * 4, &nw0) ||
        !mul_ok(units, m * d_in * 4, &nwt))
        return SRWM_ERR_SHAPE;
    if (units > INT32_MAX || T > INT32_MAX || H > INT32_MAX) return SRWM_ERR_SHAPE;
    if ((nx > 0 && x == nullptr) || (ny > 0 && y == nullptr) || (nw0 > 0 && units > 0 && W0 == nullptr))
        return SRWM_ERR_NULL;
    // The kernels move 16-byte pieces: every buffer must be 16-byte aligned.
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(W0) |
         reinterpret_cast<uintptr_t>(y) | reinterpret_cast<uintptr_t>(W_T)) & 15u)
        return SRWM_ERR_ARG;
    if (units == 0) return SRWM_OK;
    if (W_T == nullptr) nwt = 0;
    if (ranges_overlap(x, nx, y, ny) || ranges_overlap(W0, nw0, W_T, nwt) ||
        ranges_overlap(x, nx, W_T, nwt) || ranges_overlap(W0, nw0, y, ny) ||
        ranges_overlap(y, ny, W_T, nwt))
        return SRWM_ERR_ALIAS;
    if (T == 0 && W_T == nullptr) return SRWM_OK;

    const Variant& v = kVariants[vi];
    int Ti = static_cast<int>(T), Hi = static_cast<int>(H), fl = apply_input_softmax;
    void* args[] = {&x, &W0, &y, &W_T, &Ti, &Hi, &fl};
    const hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(v.fn),
                                           dim3(static_cast<unsigned>(units)), dim3(v.nw * kWave),
                                           args, 0, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? SRWM_OK : SRWM_ERR_HIP;
}

}  // namespace

extern "C" {

int srwm_forward(const void* x, const float* W0, void* y, float* W_T, int64_t B, int64_t T,
                 int64_t H, int64_t d_in, int64_t d_out, int64_t m, int io_dtype,
                 int apply_input_softmax, void* stream)
{
    return forward_impl(x, W0, y, W_T, B, T, H, d_in, d_out, m, io_dtype, apply_input_softmax,
                        stream, -1);
}

int srwm_forward_variant(const void* x, const float* W0, void* y, float* W_T, int64_t B,
                         int64_t T, int64_t H, int64_t d_in, int64_t d_out, int64_t m,
                         int io_dtype, int apply_input_softmax, void* stream, int variant)
{
    return forward_impl(x, W0, y, W_T, B, T, H, d_in, d_out, m, io_dtype, apply_input_softmax,
                        stream, variant);
}

int srwm_variant_count(void) { return kNumVariants; }

int srwm_variant_info(int i, int* d_in, int* d_out, int* io_dtype, int* waves, int* lanes_per_row,
                      int* waves_per_simd, int* is_auto)
{
    if (i < 0 || i >= kNumVariants) return SRWM_ERR_ARG;
    const Variant& v = kVariants[i];
    if (d_in) *d_in = v.d_in;
    if (d_out) *d_out = v.d_out;
    if (io_dtype) *io_dtype = v.io;
    if (waves) *waves = v.nw;
    if (lanes_per_row) *lanes_per_row = v.p;
    if (waves_per_simd) *waves_per_simd = v.wpe;
    if (is_auto) *is_auto = v.is_auto;
    return SRWM_OK;
}

int srwm_supported(int64_t d_in, int64_t d_out, int io_dtype)
{
    return find_variant(d_in, d_out, io_dtype, -1, 1) >= 0 ? 1 : 0;
}

const char* srwm_strerror(int code)
{
    switch (code) {
    case SRWM_OK: return "SRWM_OK: success";
    case SRWM_ERR_NULL: return "SRWM_ERR_NULL: a required pointer is NULL";
    case SRWM_ERR_SHAPE: return "SRWM_ERR_SHAPE: invalid sizes (negative, m != d_out+2*d_in+4, or overflow)";
    case SRWM_ERR_UNSUPPORTED: return "SRWM_ERR_UNSUPPORTED: no kernel built for this (d_in, d_out, io_dtype)";
    case SRWM_ERR_ALIAS: return "SRWM_ERR_ALIAS: an output buffer overlaps another buffer";
    case SRWM_ERR_HIP: return "SRWM_ERR_HIP: the HIP runtime rejected the launch";
    case SRWM_ERR_ARG: return "SRWM_ERR_ARG: invalid io_dtype, flag or variant";
    default: return "unknown srwm error code";
    }
}

int srwm_version(void)
{
    return SRWM_VERSION_MAJOR * 10000 + SRWM_VERSION_MINOR * 100 + SRWM_VERSION_PATCH;
}

}  // extern "C"
