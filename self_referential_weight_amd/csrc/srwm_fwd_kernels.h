// srwm_fwd_kernels.h -- the forward kernels of libsrwm (device code only):
// the phased and the fused-schedule SRWM recurrence and the geometry and
// staging helpers they use.  Included by srwm_fwd.hip, which holds the
// variant table and the C ABI.  The design notes are at the top of that file.
#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "srwm_device.h"

namespace srwm {

// ----------------------------------------------------------------------------
// Compile-time geometry of one kernel variant.
//
// Main rows (the y, k and q blocks, MAIN = d_out + 2*d_in rows) use the
// strided lane layout described at the top of the file.  The NLR rate rows
// (four, or one in the one-rate form) use one of two layouts:
//   BETA_SEP (d_in % 16 == 0): wave 0 holds them, DPP row i (lanes 16i..16i+15)
//     holding rate row i, LB = d_in/16 consecutive columns per lane; a rate
//     row's dot product is then a 16-lane DPP sum inside one DPP row, and the
//     lanes that need its learning-rate term are the ones that computed it.
//     With one rate, DPP rows 1-3 hold zeros and store nothing.
//   otherwise: they are appended to the main rows (one extra register row,
//     zero padded), which only the small test shapes use.
template <int D_IN, int D_OUT, int NW, int P, int NLR = 4, bool LONG = false>
struct Geom {
    static_assert(NLR == 1 || NLR == 4, "one or four learning rates");
    static constexpr int NT = NW * kWave;            // threads per unit
    static constexpr int M = D_OUT + 2 * D_IN + NLR; // rows of W
    static constexpr int MAIN = D_OUT + 2 * D_IN;  // y, k, q rows
    static constexpr bool BETA_SEP = (D_IN % 16 == 0);
    static constexpr int ROWS = BETA_SEP ? MAIN : M; // rows in the strided layout
    static constexpr int L = D_IN / P;             // columns per lane
    static constexpr int G = NT / P;               // row groups
    static constexpr int R = (ROWS + G - 1) / G;   // rows per lane
    static constexpr bool ALIGNED = (D_IN % G == 0) && (D_OUT % G == 0);
    static constexpr int LB = BETA_SEP ? D_IN / 16 : 0; // beta columns per lane
    // x staging: E consecutive elements per lane, LR lanes per step row.
    // Aim for 32 step rows per chunk with every lane loading, at most 16 and
    // at least d_in/16 elements per lane (so a row spans <= 16 lanes).  One-wave
    // units have scarcer registers: 8 rows, or 16 with LONG (the tape-writing
    // forward at d_in = 64: 2.4% faster than 8; the plain forward would gain
    // 0.6% but spill 14 more registers, whose write-backs add 7.7% to its HBM
    // traffic).
    static constexpr int E_TARGET = ((NW == 1 ? (LONG ? 16 : 8) : 32) * D_IN) / NT;
    static constexpr int E_LO = D_IN / 16 > E_TARGET ? D_IN / 16 : E_TARGET;
    static constexpr int E = D_IN < 16 ? D_IN : (E_LO < 16 ? (E_LO < 1 ? 1 : E_LO) : 16);
    static constexpr int LR = D_IN / E;
    static constexpr int S_FULL = NT / LR;
    static constexpr int S = S_FULL < 32 ? S_FULL : 32; // steps per chunk
    static_assert(D_IN % P == 0, "P must divide d_in");
    static_assert(D_IN % E == 0, "E must divide d_in");
    static_assert(LR <= 16 && (LR & (LR - 1)) == 0, "row lanes");
    static_assert(G >= 4, "need at least four row groups");
    // Learning-rate index of register r when ALIGNED: the row block (0 y,
    // 1 k, 2 q, 3 beta) with four rates, 0 with one.
    static constexpr int rate_of_reg(int r)
    {
        const int row = G * r;
        if (NLR == 1) return 0;
        return row < D_OUT ? 0 : row < D_OUT + D_IN ? 1 : row < D_OUT + 2 * D_IN ? 2 : 3;
    }
};

template <int NLR>
__device__ __forceinline__ int rate_of_row(int row, int d_in, int d_out)
{
    if (NLR == 1) return 0;
    return row < d_out ? 0 : row < d_out + d_in ? 1 : row < d_out + 2 * d_in ? 2 : 3;
}

// phi(k) and phi(q) by one wave: k and q are d-vectors in LDS.  The lower
// half-wave takes k, the upper half q (lane hl of a half holds entries hl,
// hl + 32, ...: consecutive lanes, consecutive LDS words), so both softmaxes
// share every reduction step.  Then phi(k) and phi(q) entries meet in one
// lane: a lane-row swap of two entries i, i+1 leaves the lower half with
// (phi(k), phi(q)) of entry i and the upper half with those of entry i+1, so
// every lane writes one kh = softmax(k) entry and e = softmax(q) - kh, the
// difference the fused read of Eq. (2) needs (with one entry per lane, the
// lower half alone writes).  FMAX picks the float form of the half-wave max
// (multi-wave units) over the integer one.
template <int D, bool FMAX = false>
__device__ __forceinline__ void wave_addresses(const float* __restrict__ k, const float* __restrict__ q,
                                               float* __restrict__ kh_out, float* __restrict__ e_out, int lane,
                                               float* kh_lane = nullptr, float* e_lane = nullptr)
{
    constexpr int EPH = (D + 31) / 32;
    const bool upper = lane >= 32;
    const int hl = lane & 31;
    const float* __restrict__ src = upper ? q : k;
    float v[EPH];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPH; ++i) {
        const int j = hl + 32 * i;
        v[i] = (j < D) ? src[j] : -INFINITY;
        mx = fmax2(mx, v[i]);
    }
    const float ms = log2e_scaled(FMAX ? half_max_f(mx) : half_max(mx));
#pragma unroll
    for (int i = 0; i < EPH; ++i) {
        const int j = hl + 32 * i;
        v[i] = (j < D) ? exp_shifted(v[i], ms) : 0.f;
    }
    float s = v[0];  // (not 0 + v[0]: the compiler keeps that add, as -0 + 0 = +0)
#pragma unroll
    for (int i = 1; i < EPH; ++i) s += v[i];
    const float inv = rcp_f32(half_sum(s));
    // Both probabilities are rounded before the difference (no fused
    // multiply-subtract), so k_t == q_t gives e == 0 exactly: the two halves
    // run the same instructions on the same values.
    if constexpr (EPH % 2 == 0) {
#pragma unroll
        for (int i = 0; i < EPH; i += 2) {
#pragma clang fp contract(off)
            float pk = v[i] * inv, pq = v[i + 1] * inv;
            swap32(pk, pq);  // lower: (phi(k), phi(q)) of entry i; upper: of entry i+1
            const int j = hl + 32 * (upper ? i + 1 : i);
            kh_out[j] = pk;
            e_out[j] = pq - pk;
            if (kh_lane != nullptr && i == (EPH == 2 ? 0 : -1)) {
                // with two entries per lane (D = 64) entry j is this lane's own: j == lane
                *kh_lane = pk;
                *e_lane = pq - pk;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < EPH; ++i) {
#pragma clang fp contract(off)
            float p = v[i] * inv, pq = p;
            swap32(p, pq);  // lower half: p = phi(k) entry, pq = the matching phi(q) entry
            const int j = hl + 32 * i;
            if (!upper && j < D) {
                kh_out[j] = p;
                e_out[j] = pq - p;
            }
            if (kh_lane != nullptr && i == 0) {
                // one entry per lane (D <= 32): lane j < D holds entry j
                *kh_lane = p;
                *e_lane = pq - p;
            }
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

// x staging.  S step rows of x for one unit are loaded one chunk ahead into
// registers (lane tid < S*LR takes E consecutive elements of row tid/LR), then
// widened (bf16 -> f32 is exact), optionally softmax-ed per row, and written
// to an LDS tile.
//
// One-wave tape-writing units whose x rows are whole 16-byte pieces (DMA)
// fetch the raw chunk straight into a second LDS buffer instead (buffer_load_dwordx4 ...
// lds, 1 KB per instruction: lane i takes piece i mod LPR of row i / LPR of
// the instruction's rows), and stage() reads each lane's E elements from
// there.  No register then holds x across the chunk: in the registers of a
// one-wave unit such a prefetch was spilled, its loads waited for at once.
// The lane's offsets are recomputed from the lane index at each use.
template <int D_IN, int D_OUT, int NW, int P, bool BF16, bool LONG = false>
struct XStage {
    using Gm = Geom<D_IN, D_OUT, NW, P, 4, LONG>;
    static constexpr int E = Gm::E, LR = Gm::LR, S = Gm::S;
    static constexpr int XR = BF16 ? (E + 1) / 2 : E; // registers held per lane
    using XT = typename std::conditional<BF16, uint16_t, float>::type;
    static constexpr int RB = D_IN * (int)sizeof(XT);  // bytes per step row
    static constexpr int LPR = RB / 16;                 // DMA lanes per row
    static constexpr bool DMA = LONG && NW == 1 && RB % 16 == 0 && LPR <= kWave && kWave % LPR == 0 &&
                                (E * (int)sizeof(XT)) % 4 == 0;
    static constexpr int RPI = DMA ? kWave / LPR : 1;  // rows per DMA instruction
    static constexpr int NI = (S + RPI - 1) / RPI;      // DMA instructions per chunk
    static constexpr int RAW_WORDS = DMA ? NI * kWave * 4 : 4;  // the raw chunk buffer (uint32)
    uint32_t xr[XR];
    int row, col;
    uint32_t lane_off;  // element offset of this lane's piece within a chunk
    bool active;
    const XT* __restrict__ xu;  // x[b][0][h][0] (wave-uniform)
    int64_t x_step;
    int T;
    uint32_t* raw;  // DMA: the raw chunk in LDS, RAW_WORDS words

    __device__ __forceinline__ XStage(int tid, const void* __restrict__ xv_, int64_t x0_, int64_t x_step_, int T_,
                                      uint32_t* raw_ = nullptr)
        : row(tid / LR), col((tid % LR) * E), active(tid < S * LR),
          xu(reinterpret_cast<const XT*>(xv_) + x0_), x_step(x_step_), T(T_), raw(raw_)
    {
        lane_off = static_cast<uint32_t>(row * x_step + col);
    }

    // Issue the global loads of the chunk that starts at step c0.
    __device__ __forceinline__ void load(int c0)
    {
        if constexpr (DMA) {
            // The resource ends with the unit's last step row in the chunk, and
            // lanes of rows past it copy nothing.  The host bounds a step's row
            // to 64 MiB, so every offset here is below 2^31.
            const int l = lane_now();
            const int r0 = l / LPR;
            const int xsb = static_cast<int>(x_step * (int64_t)sizeof(XT));
            const int last = (T - 1 - c0) < (S - 1) ? (T - 1 - c0) : (S - 1);
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(xu + (int64_t)c0 * x_step), (short)0, last * xsb + RB, 0x00020000);
            const int voff = r0 * xsb + (l % LPR) * 16;
#pragma unroll
            for (int k = 0; k < NI; ++k) {
                const int rk = k * RPI + r0;
                if ((NI * RPI == S || rk < S) && c0 + rk < T)
                    copy_x4_to_lds(rs, voff, k * RPI * xsb, raw + k * kWave * 4);
            }
            return;
        }
        const int t = c0 + row;
        if (active && t < T) {
            const XT* src = xu + (int64_t)c0 * x_step + lane_off;
            if constexpr (BF16) {
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
                float tmp[E];
                load_f32<E>(src, tmp);
#pragma unroll
                for (int i = 0; i < E; ++i) xr[i] = __float_as_uint(tmp[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < XR; ++i) xr[i] = 0u;
        }
    }

    // Widen, apply the optional input softmax per step row, write to LDS.
    __device__ __forceinline__ void stage(float (*dst)[D_IN], int in_softmax)
    {
        if constexpr (DMA) {
            wait_vmem();  // the chunk's copies (and every earlier store) have landed
            const int l = lane_now();
            // lanes past the chunk's S rows (l >= S*LR) read nothing
            const int lr = l < S * LR ? l : 0;
            const uint32_t* src = raw + ((lr / LR) * RB + (lr % LR) * E * (int)sizeof(XT)) / 4;
#pragma unroll
            for (int i = 0; i < XR; ++i) xr[i] = src[i];
        }
        const int srow = DMA ? lane_now() / LR : row;
        const int scol = DMA ? (lane_now() % LR) * E : col;
        const bool sact = DMA ? lane_now() < S * LR : active;
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
            const float ms = log2e_scaled(group_max<LR>(mx));
            float sum = 0.f;
#pragma unroll
            for (int i = 0; i < E; ++i) {
                v[i] = exp_shifted(v[i], ms);
                sum += v[i];
            }
            const float inv = rcp_f32(group_sum<LR>(sum));
#pragma unroll
            for (int i = 0; i < E; ++i) v[i] *= inv;
        }
        if (sact) store_f32<E>(&dst[srow][scol], v);
    }
};

// Store y_t = z[0:d_out] (one wave; lanes take consecutive entries).
template <int D_OUT, bool BF16>
__device__ __forceinline__ void store_y(void* __restrict__ yv, int64_t off, const float* __restrict__ z, int lane)
{
#pragma unroll
    for (int j0 = 0; j0 < D_OUT; j0 += kWave) {
        const int j = j0 + lane;
        if (j < D_OUT) {
            if constexpr (BF16)
                reinterpret_cast<uint16_t*>(yv)[off + j] = f32_to_bf16(z[j]);
            else
                reinterpret_cast<float*>(yv)[off + j] = z[j];
        }
    }
}

// ----------------------------------------------------------------------------
// The kernel: grid = B*H workgroups (unit = b*H + h), NW*64 threads each.
// WPE is the occupancy (waves per SIMD) the register allocation must allow.
template <int D_IN, int D_OUT, int NW, int P, int WPE, int NLR, bool RESET, bool TAPE, bool BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * kWave, NW * kWave),
                          amdgpu_waves_per_eu(WPE)))
void srwm_fwd_kernel(const void* __restrict__ xv, const float* __restrict__ W0,
                     void* __restrict__ yv, float* __restrict__ WT, float* __restrict__ tape,
                     float* __restrict__ wstates, int T, int t_stride, int H, int in_softmax,
                     int w0_per_seq, int reset_interval)
{
    using Gm = Geom<D_IN, D_OUT, NW, P, NLR, TAPE>;
    constexpr int M = Gm::M, MAIN = Gm::MAIN, ROWS = Gm::ROWS;
    constexpr int L = Gm::L, G = Gm::G, R = Gm::R, LB = Gm::LB;
    constexpr int S = Gm::S;
    constexpr bool BETA_SEP = Gm::BETA_SEP;
    // Row sums held complete in every lane before the stores that only some
    // lanes make (keep()): measured faster for multi-wave d <= 64 units,
    // slower at d = 128 and without the registers to spare in one-wave units.
    constexpr bool KEEP_SUMS = NW > 1 && D_IN <= 64;

    __shared__ __attribute__((aligned(16))) float s_x[2][S][D_IN];
    using XS = XStage<D_IN, D_OUT, NW, P, BF16, TAPE>;
    __shared__ __attribute__((aligned(16))) uint32_t s_xraw[XS::RAW_WORDS];
    // z_t, double-buffered by step parity so one barrier per step suffices.
    __shared__ __attribute__((aligned(16))) float s_z[2][R * G + 4];
    using TL = TapeLayout<M, D_IN>;
    // The tape is written with buffer stores straight from the registers that
    // hold each entry (d_in <= 64: one entry of phi(k_t), e_t and u_t per
    // lane): the row's address is a uniform descriptor per step (SGPRs; its
    // record count is one tape row, so no store leaves the row), each lane's
    // offset a constant.  Every wave stores its a_t rows, wave 0 the rest.
    // (One-wave units used to assemble the row in LDS and copy it out with
    // 16-byte stores, 2.3% slower: with every register in use, the copy's two
    // pieces per lane each waited for its LDS read before its store; wave 0 of
    // multi-wave units read the vectors back from LDS, 2.3% slower on the
    // few-shot taped forward.)  At d_in = 128 wave 0 copies the vectors from
    // LDS and every wave stores its a_t rows through plain pointers.
    constexpr bool TAPE_BUF = TAPE && D_IN <= kWave;
    static_assert(!(TAPE && NW == 1) || D_IN <= kWave, "one tape entry per lane of phi(k_t), e_t and u_t");
    // Each wave forms phi(k_t) and phi(q_t) - phi(k_t) itself, in its own slice.
    __shared__ __attribute__((aligned(16))) float s_kh[NW][D_IN];
    __shared__ __attribute__((aligned(16))) float s_e[NW][D_IN];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = NW == 1 ? 0 : tid / kWave;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // the same, known uniform
    const int p = tid % P;
    const int rg = tid / P;
    const int unit = blockIdx.x;
    const int b = unit / H;
    const int h = unit - b * H;

    // Element offsets.  x[b][t][h][:] = x0 + t*x_step; sequences lie t_stride
    // (>= T) steps apart, so x and y may be time slices of longer sequences.
    const int64_t x_step = (int64_t)H * D_IN;
    const int64_t y_step = (int64_t)H * D_OUT;
    const int64_t x0 = ((int64_t)b * t_stride * H + h) * D_IN;
    const int64_t y0 = ((int64_t)b * t_stride * H + h) * D_OUT;
    const float* __restrict__ w0h = W0 + (int64_t)(w0_per_seq ? unit : h) * M * D_IN;

    // ---- a0: W <- W0 into registers (again at each reset of the ablation).
    float w[R][L];
    const int bcol = (lane & 15) * (LB > 0 ? LB : 1);
    const int brow = lane >> 4;
    float wb[LB > 0 ? LB : 1];
    auto load_w0 = [&]() {
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
        if constexpr (BETA_SEP) {
            if (wave == 0) {
                if (brow < NLR) {
                    load_f32<LB>(w0h + (int64_t)(MAIN + brow) * D_IN + bcol, wb);
                } else {
#pragma unroll
                    for (int c = 0; c < LB; ++c) wb[c] = 0.f;
                }
            }
        }
    };
    load_w0();
    // W -> dst[m][d_in] (W_T, or with the tape and resets the end state of a window).
    auto store_w = [&](float* __restrict__ wdst) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = rg + G * r;
            if (row < ROWS) store_f32<L>(wdst + (int64_t)row * D_IN + p * L, w[r]);
        }
        if constexpr (BETA_SEP) {
            if (wave == 0 && brow < NLR) store_f32<LB>(wdst + (int64_t)(MAIN + brow) * D_IN + bcol, wb);
        }
    };

    XS xs(tid, xv, x0, x_step, T, s_xraw);
    // The unit's barrier.  With the x chunk copied straight into LDS (one
    // wave) a wave-scope fence suffices, and a workgroup-scope one would also
    // wait for those copies in flight (they are LDS writes), which stage()
    // waits for when it needs them.  (For the other one-wave units the
    // wave-scope fence measured 0.3% slower.)
    auto unit_sync = [] {
        if constexpr (XS::DMA)
            wave_sync();
        else
            __syncthreads();
    };
    float* const khs = s_kh[wave];
    float* const es = s_e[wave];

    // The wave that stores y_t.
    constexpr int WAVE_AUX = NW >= 2 ? 1 : 0;
    // One-wave units take y_t and the learning rates straight from the
    // registers of the projection: every lane holds whole row sums of the y
    // rows (registers r < D_OUT / G) and DPP row i of the rate rows holds rate
    // row i's sum, so neither goes through LDS.
    constexpr bool Y_REG = NW == 1 && Gm::ALIGNED;
    constexpr bool G_REG = NW == 1 && BETA_SEP;
    constexpr int RY = D_OUT / G;  // y registers (Y_REG)

    int until_reset = reset_interval;  // steps left before the next reset
    (void)until_reset;

    // One step t, reading u_t at urow; PAR = t & 1 picks the z buffer (the
    // chunk length is even, so it is the parity of the step within its chunk).
    // Multi-wave units have registers to spare: they read a lane's columns of
    // a vector at once rather than in pieces, read q^ - k^ and k^ together (so
    // the update does not wait for its own LDS read), and the first step of
    // each pair also reads the second step's u (its row is in the same tile).
    // (Units holding more than 48 state floats per lane keep the piecewise
    // reads and the single copy of the step below: with them the two-wave
    // d = 64 units spill.)
    constexpr bool SPARE = NW > 1 && R * L <= 48;
    constexpr bool PREF = SPARE && L <= 8;
    // a straight-line copy of the step per wave role (the chunk loop below)
    constexpr bool ROLES = NW > 1 && D_IN <= 64 && Gm::ALIGNED && SPARE;
    float u_next[PREF ? L : 1];

    auto step = [&](const int t, const float* __restrict__ urow, auto par, auto role) {
        constexpr int PAR = decltype(par)::value;
        // role 0: wave 0 (the rate rows, the tape's vectors); 1: the wave that
        // stores y_t; 2: the others; 3: any wave (decided at run time)
        constexpr int ROLE = decltype(role)::value;
        const bool W0 = ROLE == 3 ? wave == 0 : ROLE == 0;
        const bool AUX = NW == 1 || (ROLE == 3 ? wave == WAVE_AUX : ROLE == 1);
        if constexpr (RESET) {
            // Reset ablation of the review page (Sec. 4.5): before every
            // step t > 0 with t % R == 0 the state returns to W0.
            if (reset_interval > 0) {
                if (until_reset == 0) {
                    if constexpr (TAPE) {
                        // the backward pass restarts window t/R - 1 from its end state
                        const int nres = (T - 1) / reset_interval;
                        store_w(wstates + ((int64_t)unit * nres + (t / reset_interval - 1)) * M * D_IN);
                    }
                    load_w0();
                    until_reset = reset_interval;
                }
                --until_reset;
            }
        }
        // ---- (A) Eq. (1): z = W u.
        float* __restrict__ zt = s_z[PAR];
        // TAPE_BUF: one word of this step's tape row, through the row as a
        // buffer resource (uniform, the same for every store of the step), at
        // a lane-constant byte offset vb (VGPR) plus a compile-time one cb
        // (the store's scalar offset)
        auto tstore = [&](float v, int vb, int cb) {
            const __amdgpu_buffer_rsrc_t row = __builtin_amdgcn_make_buffer_rsrc(
                tape + ((int64_t)unit * T + t) * TL::ROW, (short)0, TL::ROW * 4, 0x00020000);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), row, vb, cb, 0);
        };
        // Multi-wave units with a copy of the step per role: wave 0 reads its
        // rate-row columns of u, q^ - k^ and k^ together with the other
        // vectors, not right before use -- the rate rows are its extra work,
        // and every other wave waits for it at the barrier (few-shot taped
        // forward 0.79 -> 0.745 ms).  Where the role is decided at run time
        // (d = 128, d_out = 193) the loads sit behind a branch and cost more
        // than they save (wide 11.06 -> 11.79 ms).
        constexpr bool BPREF = BETA_SEP && ROLES;
        float ubv[BPREF ? LB : 1];
        if constexpr (BPREF) {
            if (W0) load_f32<LB>(urow + bcol, ubv);
        }
        // With the prefetch, wave 0 forms its rate rows' sums and gates first:
        // the chain (row sum over 16 lanes, exp, reciprocal) then overlaps
        // its main rows instead of ending its pass before the barrier.
        float gz = 0.f;
        if constexpr (BPREF) {
            if (W0) {
                float accb = 0.f;
#pragma unroll
                for (int c = 0; c < LB; ++c) accb = fmaf(wb[c], ubv[c], accb);
                gz = sigmoid_f32(group_sum<16>(accb));
            }
        }
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.f;
        if constexpr (PREF) {
            float uv[L];
            if constexpr (PAR == 0) {
                load_f32<L>(urow + p * L, uv);
                load_f32<L>(urow + D_IN + p * L, u_next);  // row s + 1 <= S - 1 of the tile
            } else {
#pragma unroll
                for (int c = 0; c < L; ++c) uv[c] = u_next[c];
            }
#pragma unroll
            for (int c = 0; c < L; ++c)
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r] = fmaf(w[r][c], uv[c], acc[r]);
        } else {
            stream_lds<L>(urow + p * L, [&](int c, float uc) {
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r] = fmaf(w[r][c], uc, acc[r]);
            });
        }
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = group_sum<P>(acc[r]);
        if constexpr (KEEP_SUMS) {
#pragma unroll
            for (int r = 0; r < R; ++r) keep(acc[r]);
        }
        // All P lanes of a row group hold the same sums and every one
        // stores them (the same word from P lanes): stores at constant
        // offsets from one address, no per-lane selection of a register.
#pragma unroll
        for (int r = (Y_REG ? RY : 0); r < R; ++r) {
            const int row = rg + G * r;
            if (Gm::ALIGNED || row < ROWS) zt[row] = acc[r];
        }
        if constexpr (Y_REG) {
            // y_t rows rg + G*r, r < RY, from every lane of the row group
            const int64_t yo = y0 + (int64_t)t * y_step + rg;
            if constexpr (BF16) {
                uint16_t* __restrict__ yb = reinterpret_cast<uint16_t*>(yv) + yo;
#pragma unroll
                for (int r = 0; r + 1 < RY; r += 2) {
                    const uint32_t pk = f32x2_to_bf16x2(acc[r], acc[r + 1]);
                    yb[G * r] = static_cast<uint16_t>(pk);
                    yb[G * (r + 1)] = static_cast<uint16_t>(pk >> 16);
                }
                if constexpr (RY % 2 == 1) yb[G * (RY - 1)] = f32_to_bf16(acc[RY - 1]);
            } else {
                float* __restrict__ yf = reinterpret_cast<float*>(yv) + yo;
#pragma unroll
                for (int r = 0; r < RY; ++r) yf[G * r] = acc[r];
            }
        }
        float gb = 0.f;  // G_REG: the gate of rate row brow, in DPP row brow
        if constexpr (BETA_SEP) {
            if (BPREF && W0) {
                if constexpr (KEEP_SUMS) keep(gz);
                if ((lane & 15) == 0 && brow < NLR) zt[MAIN + brow] = gz;
            } else if (W0) {
                float accb = 0.f;
                stream_lds<LB>(urow + bcol, [&](int c, float uc) { accb = fmaf(wb[c], uc, accb); });
                accb = group_sum<16>(accb);
                if constexpr (G_REG) {
                    gb = sigmoid_f32(accb);
                    if constexpr (TAPE_BUF) {
                        tstore(brow < NLR ? gb : 0.f, 4 * brow, 4 * TL::G_OFF);  // the same word from the 16 lanes
                    }
                } else {
                    // the other waves read the gates themselves
                    accb = sigmoid_f32(accb);
                    if constexpr (KEEP_SUMS) keep(accb);
                    if ((lane & 15) == 0 && brow < NLR) zt[MAIN + brow] = accb;
                }
            }
        }
        unit_sync();

        // ---- (B) phi(k), phi(q), sigma(beta), computed by every wave for
        // itself (identical bits in every wave); y_t from W_{t-1}.
        if constexpr (TAPE_BUF) {
            float khl = 0.f, el = 0.f;
            wave_addresses<D_IN, (NW > 1)>(zt + D_OUT, zt + D_OUT + D_IN, khs, es, lane, &khl, &el);
            if (W0 && lane < D_IN) {  // (every wave forms them; wave 0 stores them)
                tstore(khl, 4 * lane, 4 * TL::KH_OFF);
                tstore(el, 4 * lane, 4 * TL::E_OFF);
            }
        } else {
            wave_addresses<D_IN, (NW > 1)>(zt + D_OUT, zt + D_OUT + D_IN, khs, es, lane);
        }
        float gl = 0.f, g0, g1, g2, g3;
        if constexpr (G_REG) {
            g0 = readlane(gb, 0);
            if constexpr (NLR == 4) {
                g1 = readlane(gb, 16);
                g2 = readlane(gb, 32);
                g3 = readlane(gb, 48);
            } else {
                g1 = g2 = g3 = g0;
            }
        } else if constexpr (BETA_SEP) {
            // wave 0 stored the gates (one sigmoid per unit instead of one per wave)
            g0 = zt[MAIN];
            if constexpr (NLR == 4) {
                g1 = zt[MAIN + 1];
                g2 = zt[MAIN + 2];
                g3 = zt[MAIN + 3];
            } else {
                g1 = g2 = g3 = g0;
            }
            if constexpr (TAPE) gl = zt[MAIN + (NLR == 4 ? (lane & 3) : 0)];
        } else {
            gl = sigmoid_f32(zt[MAIN + (NLR == 4 ? (lane & 3) : 0)]);
            g0 = readlane(gl, 0);
            g1 = readlane(gl, 1);
            g2 = readlane(gl, 2);
            g3 = readlane(gl, 3);
        }
        if constexpr (!Y_REG) {
            if (AUX) store_y<D_OUT, BF16>(yv, y0 + (int64_t)t * y_step, zt, lane);
        }
        wave_sync();
        const float* __restrict__ khw = khs;
        const float* __restrict__ ew = es;

        // ---- (C) Eq. (2)/(4) fused: W (qh - kh) = v - vb, times the gate.
        float ebv[BPREF ? LB : 1], kbv[BPREF ? LB : 1];
        if constexpr (BPREF) {
            if (W0) {
                load_f32<LB>(ew + bcol, ebv);
                load_f32<LB>(khw + bcol, kbv);
            }
        }
        float kv[PREF ? L : 1];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.f;
        if constexpr (PREF) {
            float ev[L];
            load_f32<L>(ew + p * L, ev);
            load_f32<L>(khw + p * L, kv);
#pragma unroll
            for (int c = 0; c < L; ++c)
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r] = fmaf(w[r][c], ev[c], acc[r]);
        } else {
            stream_lds<L>(ew + p * L, [&](int c, float ec) {
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r] = fmaf(w[r][c], ec, acc[r]);
            });
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float gate;
            if constexpr (Gm::ALIGNED) {
                const int bk = Gm::rate_of_reg(r);
                gate = bk == 0 ? g0 : bk == 1 ? g1 : bk == 2 ? g2 : g3;
            } else {
                const int bk = rate_of_row<NLR>(rg + G * r, D_IN, D_OUT);
                gate = bk == 0 ? g0 : bk == 1 ? g1 : bk == 2 ? g2 : g3;
            }
            acc[r] = gate * group_sum<P>(acc[r]);
        }
        if constexpr (KEEP_SUMS) {
#pragma unroll
            for (int r = 0; r < R; ++r) keep(acc[r]);
        }
        float accb = 0.f;
        if constexpr (BETA_SEP) {
            if (W0) {
                if constexpr (BPREF) {
#pragma unroll
                    for (int c = 0; c < LB; ++c) accb = fmaf(wb[c], ebv[c], accb);
                } else {
                    stream_lds<LB>(ew + bcol, [&](int c, float ec) { accb = fmaf(wb[c], ec, accb); });
                }
                accb = g3 * group_sum<16>(accb);
            }
        }
        if constexpr (TAPE) {
            // Tape for the backward pass: a_t, phi(k_t) (enough to undo the
            // update, W_{t-1} = W_t - a_t phi(k_t)^T), phi(q_t) - phi(k_t), the
            // learning rates and u_t (so the backward needs no projection and
            // no input softmax).
            float* __restrict__ tp = tape + ((int64_t)unit * T + t) * TL::ROW;
            if constexpr (TAPE_BUF) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int row = rg + G * r;
                    // (rows past ROWS are padding: their words would land on phi(k_t))
                    if (R * G == ROWS || row < ROWS) tstore(acc[r], 4 * rg, 4 * G * r);  // the same word from all P lanes of the row
                }
                if constexpr (BETA_SEP && NW > 1) {
                    if (W0) keep(accb);  // (its last DPP level not sunk into the branch below)
                }
                if (W0) {
                    if constexpr (BETA_SEP) {
                        // every lane of DPP row brow holds rate row brow's a (zero past n_lr: the row padding)
                        tstore(brow < NLR ? accb : 0.f, 4 * brow, 4 * MAIN);
                    }
                    // the rates: from the gate registers (one wave), else lanes 0..3 hold them
                    if (NW > 1 || !BETA_SEP) {
                        if (lane < 4) tstore(lane < NLR ? gl : 0.f, 4 * lane, 4 * TL::G_OFF);
                    }
                    if (lane < D_IN) tstore(urow[lane], 4 * lane, 4 * TL::U_OFF);
                }
            } else {
                // (where every register row is a real row, no branch: it would
                // split the last DPP level of each row sum into a move before
                // it and an add after it -- few-shot taped forward 0.749 ->
                // 0.728 ms)
                constexpr bool ALL_REAL = R * G == ROWS;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int row = rg + G * r;
                    if (ALL_REAL || row < ROWS) tp[row] = acc[r];  // the same word from all P lanes of the row
                }
                if constexpr (BETA_SEP) {
                    if (W0) keep(accb);
                    if (W0 && (lane & 15) == 0 && brow < NLR) tp[MAIN + brow] = accb;
                }
                if (W0) {
#pragma unroll
                    for (int j0 = 0; j0 < D_IN; j0 += kWave) {
                        if (j0 + lane < D_IN) {
                            tp[TL::KH_OFF + j0 + lane] = khw[j0 + lane];
                            tp[TL::E_OFF + j0 + lane] = ew[j0 + lane];
                            tp[TL::U_OFF + j0 + lane] = urow[j0 + lane];
                        }
                    }
                    if (lane < 4) tp[TL::G_OFF + lane] = lane < NLR ? gl : 0.f;
                }
            }
        }
        // ---- (D) Eq. (3)/(5): W += a kh^T, in place.
        if constexpr (PREF) {
#pragma unroll
            for (int c = 0; c < L; ++c)
#pragma unroll
                for (int r = 0; r < R; ++r) w[r][c] = fmaf(acc[r], kv[c], w[r][c]);
        } else {
            stream_lds<L>(khw + p * L, [&](int c, float kc) {
#pragma unroll
                for (int r = 0; r < R; ++r) w[r][c] = fmaf(acc[r], kc, w[r][c]);
            });
        }
        if constexpr (BETA_SEP) {
            if (W0) {
                if constexpr (BPREF) {
#pragma unroll
                    for (int c = 0; c < LB; ++c) wb[c] = fmaf(accb, kbv[c], wb[c]);
                } else {
                    stream_lds<LB>(khw + bcol, [&](int c, float kc) { wb[c] = fmaf(accb, kc, wb[c]); });
                }
            }
        }
    };

    if (T > 0) {
        xs.load(0);
        xs.stage(s_x[0], in_softmax);
        if (T > S) xs.load(S);
        unit_sync();

        static_assert(S % 2 == 0, "chunks start at even steps");
        int chunk = 0;
        for (int c0 = 0; c0 < T; c0 += S, ++chunk) {
            const int n = (T - c0) < S ? (T - c0) : S;
            const float* sxc = &s_x[chunk & 1][0][0];
            // two steps per iteration, so the z buffer of each is a constant
            auto run = [&](auto role) {
                for (int s = 0; s < n; s += 2) {
                    step(c0 + s, sxc + s * D_IN, std::integral_constant<int, 0>{}, role);
                    if (s + 1 < n) step(c0 + s + 1, sxc + (s + 1) * D_IN, std::integral_constant<int, 1>{}, role);
                }
            };
            // Each wave role runs its own straight-line copy of the step (a
            // scalar branch per chunk), so wave 0's rate-row work interleaves
            // with its main rows instead of sitting behind exec-mask branches.
            // At d = 128 the three copies cost registers (spills around the
            // chunk loop) and time (11.2 vs 11.0 ms on the wide workload), and
            // in SR-DeltaNet's projection (d_out = 193) they take registers
            // that the fast-matrix kernel running beside it needs (4.54 vs
            // 4.38 ms per step), so one copy decides at run time there.
            if constexpr (NW > 1 && !ROLES) {
                run(std::integral_constant<int, 3>{});
            } else if constexpr (NW == 1) {
                for (int s = 0; s < n; s += 2) {
                    step(c0 + s, sxc + s * D_IN, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
                    if (s + 1 < n)
                        step(c0 + s + 1, sxc + (s + 1) * D_IN, std::integral_constant<int, 1>{},
                             std::integral_constant<int, 0>{});
                }
            } else if (wave_u == 0) {
                run(std::integral_constant<int, 0>{});
            } else if (wave_u == WAVE_AUX) {
                run(std::integral_constant<int, 1>{});
            } else {
                run(std::integral_constant<int, 2>{});
            }
            if (c0 + S < T) {
                xs.stage(s_x[(chunk + 1) & 1], in_softmax);
                if (c0 + 2 * S < T) xs.load(c0 + 2 * S);
                unit_sync();
            }
        }
    }

    // ---- a7: W_T[b,h] <- W.
    if (WT != nullptr) store_w(WT + (int64_t)unit * M * D_IN);
}

// ----------------------------------------------------------------------------
// Fused-schedule kernel for units spread over several waves (latency-bound
// shapes).  It computes the same recurrence with a shorter serial chain per
// step.  The projection of step t+1 is formed from W_{t-1}, in the same pass
// over W as the read of step t, and corrected by the rank-one update of step t:
//     W_t u_{t+1} = W_{t-1} u_{t+1} + a_t (kh_t . u_{t+1}),   a_t = g (W_{t-1}(qh_t - kh_t)),
// which is Eq. (3) applied to the vector u_{t+1}.  The update of W itself is
// deferred to the next iteration, where it runs between the barrier and the
// fused pass and fills the latency of the softmax chain.  One workgroup
// barrier per step.
template <int D_IN, int D_OUT, int NW, int P, int WPE, int NLR, bool BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * kWave, NW * kWave),
                          amdgpu_waves_per_eu(WPE)))
void srwm_fwd_fused_kernel(const void* __restrict__ xv, const float* __restrict__ W0,
                           void* __restrict__ yv, float* __restrict__ WT, float* /*tape: not written*/,
                           float* /*window states: not written*/, int T, int t_stride, int H, int in_softmax,
                           int w0_per_seq, int /*reset_interval: not supported by this schedule*/)
{
    using Gm = Geom<D_IN, D_OUT, NW, P, NLR>;
    constexpr int M = Gm::M, MAIN = Gm::MAIN, ROWS = Gm::ROWS;
    constexpr int L = Gm::L, G = Gm::G, R = Gm::R, LB = Gm::LB;
    constexpr int S = Gm::S;
    constexpr bool BETA_SEP = Gm::BETA_SEP;
    static_assert(NW >= 2, "fused schedule is for multi-wave units");

    __shared__ __attribute__((aligned(16))) float s_x[2][S][D_IN];
    __shared__ __attribute__((aligned(16))) float s_z[2][R * G + 4];
    // phi(k_t) and phi(q_t) - phi(k_t), per wave and by step parity (the
    // update of step t-1 still reads phi(k_{t-1}) while step t's are written).
    __shared__ __attribute__((aligned(16))) float s_kh[2][NW][D_IN];
    __shared__ __attribute__((aligned(16))) float s_e[NW][D_IN];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int p = tid % P;
    const int rg = tid / P;
    const int unit = blockIdx.x;
    const int b = unit / H;
    const int h = unit - b * H;
    const int64_t x_step = (int64_t)H * D_IN;
    const int64_t y_step = (int64_t)H * D_OUT;
    const int64_t x0 = ((int64_t)b * t_stride * H + h) * D_IN;
    const int64_t y0 = ((int64_t)b * t_stride * H + h) * D_OUT;
    const float* __restrict__ w0h = W0 + (int64_t)(w0_per_seq ? unit : h) * M * D_IN;

    // ---- a0: W <- W0[h].
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
    const int bcol = (lane & 15) * (LB > 0 ? LB : 1);
    const int brow = lane >> 4;
    float wb[LB > 0 ? LB : 1];
    if constexpr (BETA_SEP) {
        if (wave == 0) {
            if (brow < NLR) {
                load_f32<LB>(w0h + (int64_t)(MAIN + brow) * D_IN + bcol, wb);
            } else {
#pragma unroll
                for (int c = 0; c < LB; ++c) wb[c] = 0.f;
            }
        }
    }
    float gate_of[R];  // filled per step: the learning rate of register r

    if (T > 0) {
        XStage<D_IN, D_OUT, NW, P, BF16> xs(tid, xv, x0, x_step, T);
        xs.load(0);
        xs.stage(s_x[0], in_softmax);
        if (T > S) xs.load(S);
        __syncthreads();

        // ---- prologue: z_0 = W_0 u_0.
        {
            const float* __restrict__ u0 = &s_x[0][0][0];
            float acc[R];
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = 0.f;
            stream_lds<L>(u0 + p * L, [&](int c, float uc) {
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r] = fmaf(w[r][c], uc, acc[r]);
            });
#pragma unroll
            for (int r = 0; r < R; ++r) {
                acc[r] = group_sum<P>(acc[r]);
                const int row = rg + G * r;
                if (p == 0 && (Gm::ALIGNED || row < ROWS)) s_z[0][row] = acc[r];
            }
            if constexpr (BETA_SEP) {
                if (wave == 0) {
                    float accb = 0.f;
                    stream_lds<LB>(u0 + bcol, [&](int c, float uc) { accb = fmaf(wb[c], uc, accb); });
                    accb = group_sum<16>(accb);
                    if ((lane & 15) == 0 && brow < NLR) s_z[0][MAIN + brow] = accb;
                }
            }
        }

        float a_prev[R];   // a_{t-1}, applied at the start of iteration t
        float ab_prev = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) a_prev[r] = 0.f;

        for (int t = 0; t < T; ++t) {
            const bool has_next = t + 1 < T;
            // chunk holding step t+1 must be in LDS before this barrier
            if (has_next && ((t + 1) % S) == 0) {
                xs.stage(s_x[((t + 1) / S) & 1], in_softmax);
                if (t + 1 + S < T) xs.load(t + 1 + S);
            }
            __syncthreads();
            const float* __restrict__ zt = s_z[t & 1];

            // ---- (B) addresses and gates of step t (every wave), y_t.
            float* __restrict__ khw = s_kh[t & 1][wave];
            float* __restrict__ ew = s_e[wave];
            wave_addresses<D_IN, true>(zt + D_OUT, zt + D_OUT + D_IN, khw, ew, lane);
            const float gl = sigmoid_f32(zt[MAIN + (NLR == 4 ? (lane & 3) : 0)]);
            const float g0 = readlane(gl, 0), g1 = readlane(gl, 1), g2 = readlane(gl, 2), g3 = readlane(gl, 3);
            if (wave == 1) store_y<D_OUT, BF16>(yv, y0 + (int64_t)t * y_step, zt, lane);

            // ---- (D) of step t-1: W_{t-2} -> W_{t-1} (overlaps the chain above).
            if (t > 0) {
                const float* __restrict__ khp = s_kh[(t - 1) & 1][wave];
                float kv[L];
                load_f32<L>(khp + p * L, kv);
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int c = 0; c < L; ++c) w[r][c] = fmaf(a_prev[r], kv[c], w[r][c]);
                if constexpr (BETA_SEP) {
                    if (wave == 0) {
                        float kb[LB];
                        load_f32<LB>(khp + bcol, kb);
#pragma unroll
                        for (int c = 0; c < LB; ++c) wb[c] = fmaf(ab_prev, kb[c], wb[c]);
                    }
                }
            }
            wave_sync();

#pragma unroll
            for (int r = 0; r < R; ++r) {
                if constexpr (Gm::ALIGNED) {
                    const int bk = Gm::rate_of_reg(r);
                    gate_of[r] = bk == 0 ? g0 : bk == 1 ? g1 : bk == 2 ? g2 : g3;
                } else {
                    const int bk = rate_of_row<NLR>(rg + G * r, D_IN, D_OUT);
                    gate_of[r] = bk == 0 ? g0 : bk == 1 ? g1 : bk == 2 ? g2 : g3;
                }
            }

            // ---- fused pass over W_{t-1}: read (e_t) and next projection (u_{t+1}).
            const int tn = has_next ? t + 1 : t;
            const float* __restrict__ un = &s_x[(tn / S) & 1][tn % S][0];
            float accr[R], accz[R];
            float cpart = 0.f;  // kh_t . u_{t+1}, this lane's columns
#pragma unroll
            for (int r = 0; r < R; ++r) {
                accr[r] = 0.f;
                accz[r] = 0.f;
            }
            {
                float ev[L], uv[L], kv[L];
                load_f32<L>(ew + p * L, ev);
                load_f32<L>(un + p * L, uv);
                load_f32<L>(khw + p * L, kv);
#pragma unroll
                for (int c = 0; c < L; ++c) {
                    cpart = fmaf(kv[c], uv[c], cpart);
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        accr[r] = fmaf(w[r][c], ev[c], accr[r]);
                        accz[r] = fmaf(w[r][c], uv[c], accz[r]);
                    }
                }
            }
            const float ct = group_sum<P>(cpart);
            float* __restrict__ zn = s_z[(t + 1) & 1];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float a = gate_of[r] * group_sum<P>(accr[r]);
                a_prev[r] = a;
                if (has_next) {
                    float z = fmaf(a, ct, group_sum<P>(accz[r]));
                    if constexpr (D_IN <= 64) keep(z);  // as KEEP_SUMS of the phased kernel
                    const int row = rg + G * r;
                    if (p == 0 && (Gm::ALIGNED || row < ROWS)) zn[row] = z;
                }
            }
            if constexpr (BETA_SEP) {
                if (wave == 0) {
                    float eb[LB], ub[LB];
                    load_f32<LB>(ew + bcol, eb);
                    load_f32<LB>(un + bcol, ub);
                    float br = 0.f, bz = 0.f;
#pragma unroll
                    for (int c = 0; c < LB; ++c) {
                        br = fmaf(wb[c], eb[c], br);
                        bz = fmaf(wb[c], ub[c], bz);
                    }
                    ab_prev = g3 * group_sum<16>(br);
                    if (has_next) {
                        float z = fmaf(ab_prev, ct, group_sum<16>(bz));
                        if constexpr (D_IN <= 64) keep(z);
                        if ((lane & 15) == 0 && brow < NLR) zn[MAIN + brow] = z;
                    }
                }
            }
        }

        // ---- (D) of the last step.
        {
            const float* __restrict__ khp = s_kh[(T - 1) & 1][wave];
            float kv[L];
            load_f32<L>(khp + p * L, kv);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int c = 0; c < L; ++c) w[r][c] = fmaf(a_prev[r], kv[c], w[r][c]);
            if constexpr (BETA_SEP) {
                if (wave == 0) {
                    float kb[LB];
                    load_f32<LB>(khp + bcol, kb);
#pragma unroll
                    for (int c = 0; c < LB; ++c) wb[c] = fmaf(ab_prev, kb[c], wb[c]);
                }
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
            if (wave == 0 && brow < NLR) store_f32<LB>(wdst + (int64_t)(MAIN + brow) * D_IN + bcol, wb);
        }
    }
}


}  // namespace srwm
