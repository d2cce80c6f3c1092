// srwm_bwd_kernels.h -- the backward kernel of libsrwm (device code only),
// included by srwm_bwd.hip, which holds the variant table and the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "srwm_device.h"

namespace srwm {

// ----------------------------------------------------------------------------
// Backward pass (memory-efficient BPTT).
//
// The pages train W0 by backpropagation through the unrolled self-modification
// ("Metalearning Continual Learning Algorithms", after Eq. (6): memory-efficient
// BPTT; review page Sec. 2.5).  The forward pass run with a tape stores, per
// step, a_t = g (.) W_{t-1}(qh_t - kh_t), kh_t, e_t = qh_t - kh_t and the
// rates g_t.  From W_T the kernel walks t backwards: it undoes the update,
// W_{t-1} = W_t - a_t kh_t^T (no projection is recomputed: the tape holds
// everything the step's adjoint needs), and carries Wh = dL/dW_t:
//     ah    = Wh kh_t                 khh  = Wh^T a_t
//     rh    = g (.) ah                betah_c = (1 - g_c) sum_{rate(i)=c} ah_i a_i
//     eh    = W^T rh                  (khh -= eh, qhh = eh)
//     kbar  = kh (.) (khh - <khh,kh>) qbar = qh (.) (qhh - <qhh,qh>)
//     zh    = [gy_t; kbar; qbar; betah]
//     uh    = W^T zh                  dx_t = uh, or the softmax backward of it
//     Wh   += rh e^T + zh u^T
// after which Wh = dL/dW_{t-1}.
//
// Layout: lane (rg, p), rg = tid / P, p = tid % P, holds G-th rows (rows
// rg + G*r, or with P = 16 runs of consecutive rows in a lane-dependent slot
// order, below) and columns [p*L, p*L + L) of both W and Wh in registers.
// Row sums (ah) are P lanes joined by DPP.  Column sums (khh, eh, uh) are over all G row groups:
// inside a wave they are reduce-scattered over the row-group lane bits (the
// lane-row swaps v_permlane32_swap / v_permlane16_swap halve the columns a
// lane carries, 1 swap + 1 add per pair; a DPP rotation adds the remaining
// bit), then the NW wave partials meet in LDS, where lane j of every wave
// reads column j.  uh of step t is reduced together with khh and eh of step
// t-1, so each step has a single workgroup barrier: step inputs are staged in
// a triple-buffered LDS ring and the exchange area is double-buffered.
// How the column sums over the row-group lane bits are split: halving on
// lane bit 5, then on bit 4, while the lane still carries >= 2 columns; the
// remaining row-group bits are summed in place.  After the exchange a lane
// carries LC consecutive columns starting at col0().
template <int P, int L>
struct ColExchange {
    static constexpr int LOGP = P == 1 ? 0 : P == 2 ? 1 : P == 4 ? 2 : P == 8 ? 3 : 4;
    static_assert(P == 4 || P == 8 || P == 16, "lanes per row");
    static constexpr bool H5 = L >= 2;
    static constexpr int L1 = H5 ? L / 2 : L;
    static constexpr bool H4 = L1 >= 2;
    static constexpr int LC = H4 ? L1 / 2 : L1;
    // row-group bits summed in place: bits LOGP..3, plus 4 and 5 when not halved
    static constexpr int KEEP_MASK = ((1 << 4) - (1 << LOGP)) | (H4 ? 0 : 16) | (H5 ? 0 : 32);

    template <int N>
    __device__ __forceinline__ static void run(float (&v)[N][L])
    {
        if constexpr (H5) {
#pragma unroll
            for (int a = 0; a < N; ++a)
#pragma unroll
                for (int c = 0; c < L / 2; ++c) {
                    float x = v[a][c], y = v[a][c + L / 2];
                    swap32(x, y);
                    v[a][c] = x + y;
                }
        }
        if constexpr (H4) {
#pragma unroll
            for (int a = 0; a < N; ++a)
#pragma unroll
                for (int c = 0; c < L1 / 2; ++c) {
                    float x = v[a][c], y = v[a][c + L1 / 2];
                    swap16(x, y);
                    v[a][c] = x + y;
                }
        }
#pragma unroll
        for (int a = 0; a < N; ++a)
#pragma unroll
            for (int c = 0; c < LC; ++c) v[a][c] = keep_sum(v[a][c]);
    }

    __device__ __forceinline__ static float keep_sum(float x)
    {
        if constexpr (LOGP == 2) {
            x += dpp<0x128>(x);  // bit 3 (row_ror:8)
            x += dpp<0x124>(x);  // then bit 2 (row_ror:4): the four lanes i + 4k of a DPP row
        } else if constexpr (LOGP == 3) {
            x = pair_sum<3>(x);
        }
        if constexpr (!H4) x = pair_sum<4>(x);
        if constexpr (!H5) x = pair_sum<5>(x);
        return x;
    }

    __device__ __forceinline__ static int col0(int lane)
    {
        const int p = lane % P;
        return p * L + (H5 ? ((lane >> 5) & 1) * (L / 2) : 0) + (H4 ? ((lane >> 4) & 1) * (L1 / 2) : 0);
    }
    __device__ __forceinline__ static bool writer(int lane) { return (lane & KEEP_MASK) == 0; }
};

// Row sums over the 16 lanes of a DPP row for a run of SW register rows held
// swizzled: slot s of lane p holds the run's row s ^ (p mod SW).  Lane p and
// lane p ^ 1 hold each row in opposite slots of a pair, so one DPP add per
// pair joins two lanes of two rows at once; after log2(SW) such levels lane p
// holds row p mod SW summed over its SW-lane group, and two rotations finish
// the 16 lanes.
template <int SW>
struct RunSum {
    static_assert(SW == 1 || SW == 2 || SW == 4, "run length");
    __device__ __forceinline__ static float total(const float* v)
    {
        if constexpr (SW == 1) return group_sum<16>(v[0]);
        float u = v[0] + dpp<kDppXor1>(v[1]);
        if constexpr (SW == 4) {
            const float x = v[2] + dpp<kDppXor1>(v[3]);
            u += dpp<kDppXor2>(x);
        } else {
            u += dpp<kDppXor2>(u);
        }
        u += dpp<0x124>(u);  // row_ror:4
        u += dpp<0x128>(u);  // row_ror:8
        return u;
    }
    // Slot s of the run from the per-lane value of row p mod SW (slot 0):
    // slot s holds row s ^ (p mod SW), which lane p ^ s of the quad has.
    __device__ __forceinline__ static float slot(int s, float v)
    {
        if constexpr (SW == 1) return v;
        switch (s) {
        case 0: return v;
        case 1: return dpp<kDppXor1>(v);
        case 2: return dpp<kDppXor2>(v);
        default: return dpp<0x1B>(v);  // quad_perm [3,2,1,0]
        }
    }
    // Sum over the SW lanes that hold the run's SW different rows.
    __device__ __forceinline__ static float quad_sum(float v)
    {
        if constexpr (SW == 1) return v;
        v += dpp<kDppXor1>(v);
        if constexpr (SW == 4) v += dpp<kDppXor2>(v);
        return v;
    }
};

template <int D_IN, int D_OUT, int NW, int P, int NLR, bool RESET>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * kWave, NW * kWave), amdgpu_waves_per_eu(2)))
void srwm_bwd_kernel(const float* __restrict__ WTin,
                     const float* __restrict__ tape, const float* __restrict__ gy,
                     const float* __restrict__ gWT, float* __restrict__ dx,
                     float* __restrict__ dWinit, int T, int H, int in_softmax, int reset_interval,
                     const float* __restrict__ wstates)
{
    constexpr int NT = NW * kWave;
    constexpr int M = D_OUT + 2 * D_IN + NLR;
    constexpr int MAIN = D_OUT + 2 * D_IN;
    constexpr int L = D_IN / P;
    constexpr int G = NT / P;
    constexpr int R = (M + G - 1) / G;
    using TL = TapeLayout<M, D_IN>;
    using CX = ColExchange<P, L>;
    constexpr int TW = TL::ROW;
    constexpr int TPL = (TW + NT - 1) / NT;
    static_assert(D_IN % P == 0 && D_IN % G == 0 && D_OUT % G == 0, "row blocks must align with row groups");
    static_assert(D_IN <= kWave && D_OUT <= NT, "one lane per column, one thread per output");
    static_assert(D_IN % 4 == 0, "16-byte tape pieces");
    static_assert((NW & (NW - 1)) == 0, "power-of-two waves");

    // the step-input ring: a slot holds the tape row, then gy_t (one slot
    // offset serves both)
    constexpr int RW = TW + D_OUT;
    static_assert(TW % 4 == 0, "16-byte ring slots");
    __shared__ __attribute__((aligned(16))) float s_ring[3][RW];
    // khh, eh, uh column partials per wave, one float array per quantity so that
    // the writers (8 column slices 32 floats apart) and the readers (lane j,
    // column j) both meet at most two-way bank conflicts
    __shared__ __attribute__((aligned(16))) float s_red[2][NW][3][D_IN];
    __shared__ __attribute__((aligned(16))) float s_bred[2][NW][4];     // betah partials per wave
    // The per-column phase (lane <-> column jc).  With P = 16 and d_in = 64
    // the columns are dealt: lane 16q + k of wave w takes column
    // q + 4((w + k / KR) mod NW) + G (k mod KR).  The exchange's LDS slots
    // follow the dealing (col_slot below).  Unswizzled rows (SW = 1) would
    // then find the kbar and qbar entries of every K and Q row they hold in
    // their own DPP row (the lanes of row group rg = 4w + q hold columns
    // q + 4w + G k of those blocks, one row_newbcast each); the swizzled runs
    // take them through LDS (ZLDS).  Otherwise lane j takes column j and the
    // zh rows go through LDS.
    constexpr bool BCAST = P == 16 && D_IN == kWave && 16 % NW == 0;
    constexpr int KR = D_IN / G;  // register rows per K or Q block
    // Rows of the main blocks are held swizzled (with P = 16): in each run of
    // SW register rows of one block, slot s of lane p holds the run's row
    // s ^ (p mod SW).  A run's row sums then take a butterfly (RunSum below):
    // 5 DPP adds for 4 rows instead of 16, ending with the total of row
    // p mod SW in lane p, from which the run's other slots come back by
    // quad_perm.  The kbar and qbar entries of the K and Q rows then go
    // through LDS (the dealt columns sit one per lane, not one per slot).
    constexpr int YR = D_OUT / G;  // register rows of the y block
    constexpr int SW = P != 16 ? 1 : (KR % 4 == 0 && YR % 4 == 0) ? 4 : (KR % 2 == 0 && YR % 2 == 0) ? 2 : 1;
    constexpr int RS = MAIN / G;   // register rows of the main blocks
    constexpr bool ZLDS = !BCAST || SW > 1;
    static_assert(SW == 1 || BCAST, "swizzled rows take the per-lane beta row");
    __shared__ __attribute__((aligned(16))) float s_zh[ZLDS ? NW : 1][ZLDS ? M : 1];  // each wave's own zh rows

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = NW == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid / kWave);
    const int p = tid % P;
    const int rg = tid / P;
    // The last register row holds rows G(R-1) + rg; in a wave whose row groups
    // all land past M (the beta block is short) it is only padding, and the
    // wave skips it (W and Wh stay zero there).
    const bool last_empty = NW > 1 && wave * (kWave / P) + G * (R - 1) >= M;
    const int unit = blockIdx.x;
    const int b = unit / H;
    const int h = unit - b * H;
    int jc = lane;
    if constexpr (BCAST) {
        const int kq = lane & 15;
        jc = (lane >> 4) + 4 * ((wave + kq / KR) & (NW - 1)) + G * (kq % KR);
    }
    // Where the exchange puts column c in every wave's array.  With the
    // columns dealt, slot 16 (c mod 4) + c / 4: the 32 lanes of a half-wave
    // then write (column 4p + 2 b5 + b4 from lane (b5, b4, p)) and read
    // (column jc) 32 distinct consecutive slots, with no bank conflict.
    auto col_slot = [](int c) {
        if constexpr (BCAST) return 16 * (c & 3) + (c >> 2);
        else return c;
    };
    const int jslot = col_slot(jc);
    const int64_t x_step = (int64_t)H * D_IN;
    const int64_t y_step = (int64_t)H * D_OUT;
    const int64_t x0 = ((int64_t)b * T * H + h) * D_IN;
    const int64_t y0 = ((int64_t)b * T * H + h) * D_OUT;
    const float* __restrict__ tp0 = tape + (int64_t)unit * T * TW;

    // Register rows r with G*(r+1) <= M hold real rows in every lane; the last
    // one may be partial: its reads clamp the address and select 0 (no branch).
    auto row_ok = [](int r, int row) { return G * (r + 1) <= M || row < M; };
    auto row_at = [](int r, int row) { return G * (r + 1) <= M ? row : (row < M ? row : M - 1); };
    // The row register r of this lane holds (see the swizzle above).  With
    // SW > 1 the rows of run j of a block are SW consecutive rows,
    // SW (G j + rg) + (0 .. SW-1) past the block's first row, so that the
    // lanes of a half-wave read the tape and zh entries of their slots from
    // consecutive LDS words (no bank conflict).
    const int sw_e = lane & (SW - 1);
    int so[SW];
#pragma unroll
    for (int s = 0; s < SW; ++s) so[s] = SW == 1 ? rg : SW * rg + (s ^ sw_e);
    auto srow = [&](int r) {
        if (r >= RS) return rg + G * r;
        if constexpr (SW == 1) return rg + G * r;
        const int rb = r < YR ? 0 : r < YR + KR ? YR : YR + KR;            // the block's first register
        const int b0 = r < YR ? 0 : r < YR + KR ? D_OUT : D_OUT + D_IN;    // and its first row
        return b0 + SW * G * ((r - rb) / SW) + so[r % SW];
    };

    // Learning-rate index of register r (the row block; 0 with one rate).
    auto rate = [](int r) constexpr {
        const int row = G * r;
        return NLR == 1 ? 0 : row < D_OUT ? 0 : row < D_OUT + D_IN ? 1 : row < MAIN ? 2 : 3;
    };

    // W <- W_T, Wh <- dL/dW_T (or 0)
    float w[R][L], wh[R][L];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = srow(r);
        if (row < M) {
            load_f32<L>(WTin + ((int64_t)unit * M + row) * D_IN + p * L, w[r]);
            if (gWT != nullptr) {
                load_f32<L>(gWT + ((int64_t)unit * M + row) * D_IN + p * L, wh[r]);
            } else {
#pragma unroll
                for (int c = 0; c < L; ++c) wh[r][c] = 0.f;
            }
        } else {
#pragma unroll
            for (int c = 0; c < L; ++c) w[r][c] = wh[r][c] = 0.f;
        }
    }

    // Step inputs are fetched two steps ahead into registers and staged one
    // step ahead into the LDS ring: the tape row (which holds u_t) and gy_t,
    // whose entries every GS-th thread takes (spread over all waves).
    constexpr int GS = NT / D_OUT;
    static_assert(NT % D_OUT == 0, "gy entries spread over the threads");
    const bool g_mine = tid % GS == 0;
    const int g_idx = tid / GS;
    // Each row is read through a buffer resource made per step (SGPRs; its
    // record count is the row, so the entries past it read as zero) with the
    // thread's byte offset as the only per-lane operand.
    float tnext[TPL];
    float gnext = 0.f;
    const int tid4 = 4 * tid;
    auto fetch = [&](int t) {
        const __amdgpu_buffer_rsrc_t trow = float_rsrc(tp0 + (int64_t)t * TW, TW);
#pragma unroll
        for (int i = 0; i < TPL; ++i)
            tnext[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(trow, tid4, 4 * NT * i, 0));
        if (g_mine)
            gnext = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(float_rsrc(gy + y0 + (int64_t)t * y_step, D_OUT),
                                                                        4 * g_idx, 0, 0));
    };
    auto stage = [&](int slot) {
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const int j = tid + NT * i;
            if (j < TW) s_ring[slot][j] = tnext[i];
        }
        if (g_mine) s_ring[slot][TW + g_idx] = gnext;
    };

    // The exchange: this lane's column partials of khh, eh and uh (and the
    // betah partials) -> LDS area `par`.
    float part[3][L];
    auto exchange = [&](int par, float (&bp)[4]) {
        CX::run(part);
        if (CX::writer(lane)) {
            const int c0 = CX::col0(lane);
            static_assert(!BCAST || CX::LC == 1, "one column per writer when the columns are dealt");
#pragma unroll
            for (int a = 0; a < 3; ++a) {
                if constexpr (BCAST) {
                    s_red[par][wave][a][col_slot(c0)] = part[a][0];
                } else if constexpr (CX::LC % 2 == 0) {
#pragma unroll
                    for (int c = 0; c < CX::LC; c += 2)
                        *reinterpret_cast<float2*>(&s_red[par][wave][a][c0 + c]) = make_float2(part[a][c], part[a][c + 1]);
                } else {
#pragma unroll
                    for (int c = 0; c < CX::LC; ++c) s_red[par][wave][a][c0 + c] = part[a][c];
                }
            }
        }
        // The P lanes of a row group hold the same betah partials; sum them
        // over the row-group bits below 4 in place, then over bits 5 and 4
        // (one copy per row group): with four rates as a reduce-scatter (rate
        // c ends in lane 16c).
#pragma unroll
        for (int c = 0; c < NLR; ++c) {
            if constexpr (P == 4) {
                bp[c] += dpp<0x128>(bp[c]);
                bp[c] += dpp<0x124>(bp[c]);
            } else if constexpr (P == 8) {
                bp[c] = pair_sum<3>(bp[c]);
            }
        }
        if constexpr (NLR == 4) {
            swap32(bp[0], bp[2]);
            swap32(bp[1], bp[3]);
            float lo = bp[0] + bp[2], hi = bp[1] + bp[3];  // rows 0-1: rates 0, 1; rows 2-3: 2, 3
            swap16(lo, hi);
            const float tot = lo + hi;  // row q of the wave holds rate q
            if ((lane & 15) == 0) s_bred[par][wave][lane >> 4] = tot;
        } else {
            const float tot = pair_sum<5>(pair_sum<4>(bp[0]));
            if (lane == 0) s_bred[par][wave][0] = tot;
        }
    };
    // Column j's totals over the unit (lane j of every wave).
    auto gather = [&](int par, float& khh_j, float& eh_j, float& uh_j) {
        khh_j = eh_j = uh_j = 0.f;
        if (lane < D_IN) {
            khh_j = s_red[par][0][0][jslot];
            eh_j = s_red[par][0][1][jslot];
            uh_j = s_red[par][0][2][jslot];
#pragma unroll
            for (int wv = 1; wv < NW; ++wv) {
                khh_j += s_red[par][wv][0][jslot];
                eh_j += s_red[par][wv][1][jslot];
                uh_j += s_red[par][wv][2][jslot];
            }
        }
    };
    // dx of a step from its uh (column j in lane j) and u_j.
    auto store_dx = [&](int t, float uh_j, float u_j) {
        float d = uh_j;
        if (in_softmax) {
            const float du = wave_total(lane < D_IN ? uh_j * u_j : 0.f);
            d = u_j * (uh_j - du);
        }
        if (lane < D_IN)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(d), float_rsrc(dx + x0 + (int64_t)t * x_step, D_IN),
                                                  4 * jc, 0, 0);
    };

#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int c = 0; c < L; ++c) part[a][c] = 0.f;
    float u_next = 0.f;  // u_{t+1}[lane]

    // Reset ablation (built only into the RESET variants): the windows' shares
    // of dL/d(initial state) are summed into this unit's dWinit, from the last
    // window to the first, onto zeros written first; each thread adds to its
    // own elements, so each load follows the same thread's store.
    const int n_resets = (RESET && reset_interval > 0 && T > 0) ? (T - 1) / reset_interval : 0;
    int next_reset = n_resets * reset_interval;  // the latest step that starts a window, or 0
    float* __restrict__ dwi_unit = dWinit + (int64_t)unit * M * D_IN;
    auto add_share = [&]() {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = srow(r);
            if (row < M) {
                float prev[L];
                load_f32<L>(dwi_unit + row * D_IN + p * L, prev);
#pragma unroll
                for (int c = 0; c < L; ++c) prev[c] += wh[r][c];
                store_f32<L>(dwi_unit + row * D_IN + p * L, prev);
            }
        }
    };
    if (n_resets > 0) {
        float zero[L];
#pragma unroll
        for (int c = 0; c < L; ++c) zero[c] = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = srow(r);
            if (row < M) store_f32<L>(dwi_unit + row * D_IN + p * L, zero);
        }
    }

    if (T > 0) {
        fetch(T - 1);
        stage((T - 1) % 3);
        if (T > 1) fetch(T - 2);
        __syncthreads();
    }

    // One step t of the walk.  The input ring slot is t mod 3 and the
    // exchange area t mod 2: in the loop six steps at a time both are
    // constants, so every LDS address is a lane-constant base plus an
    // immediate offset (no per-step slot arithmetic).
    auto bstep = [&](const int t, auto slot_v, auto par_v) {
            const int slot = slot_v, par = par_v;  // (compile-time constants in the unrolled loop below)
            const float* __restrict__ tt = s_ring[slot];
            const float* __restrict__ us = tt + TL::U_OFF;
            const float* __restrict__ gs = tt + TW;

            // ---- (A) undo the update of step t; ah, khh, rh, eh.
            float a[R], kt[L];
    #pragma unroll
            for (int r = 0; r < R; ++r) {
                const int row = srow(r);
                const float av = tt[row_at(r, row)];
                a[r] = row_ok(r, row) ? av : 0.f;
            }
            load_f32<L>(tt + TL::KH_OFF + p * L, kt);
            const float4 gv = *reinterpret_cast<const float4*>(tt + TL::G_OFF);
            const float gate[4] = {gv.x, gv.y, gv.z, gv.w};

            // ah of the rows: per register row with SW = 1 (and for the beta
            // row); with swizzled runs, ar[j] is the total of row p mod SW of run j
            float khh[L], ah[R], pr[R], ar[RS / SW];
    #pragma unroll
            for (int c = 0; c < L; ++c) khh[c] = 0.f;
    #pragma unroll
            for (int r = 0; r < R; ++r) {
                if (r == R - 1 && last_empty) {
                    ah[r] = 0.f;
                    continue;
                }
                float as = 0.f;
    #pragma unroll
                for (int c = 0; c < L; ++c) {
                    w[r][c] = fmaf(-a[r], kt[c], w[r][c]);
                    as = fmaf(wh[r][c], kt[c], as);
                    khh[c] = fmaf(wh[r][c], a[r], khh[c]);
                }
                if (SW > 1 && r < RS) {
                    pr[r] = as;
                    if (r % SW == SW - 1) {
                        ar[r / SW] = RunSum<SW>::total(&pr[r + 1 - SW]);
                        keep(ar[r / SW]);  // (as below: no DPP level split over the branch)
                    }
                } else {
                    ah[r] = group_sum<P>(as);
                    // complete in every lane here: otherwise the last DPP level of
                    // each sum is split into a move before the last row's branch and
                    // an add after it (12 extra instructions per step)
                    keep(ah[r]);
                }
            }
            float bp[4] = {0.f, 0.f, 0.f, 0.f};
            float rh[R], eh[L];
    #pragma unroll
            for (int c = 0; c < L; ++c) eh[c] = 0.f;
    #pragma unroll
            for (int r = 0; r < R; ++r) {
                if (SW > 1 && r < RS) {
                    // the run's rates from its one total: rh by quad_perm; the
                    // betah partial sum_i ah_i a_i over the run's rows by a quad sum
                    // (slot 0 holds row p mod SW, the one whose total this lane has)
                    const int s = r % SW, j = r / SW;
                    rh[r] = RunSum<SW>::slot(s, gate[rate(r)] * ar[j]);
                    if (s == 0) {
                        float pb = ar[j] * a[r];
                        keep(pb);  // (a multiply, not folded into the first add: that add takes the DPP)
                        pb = RunSum<SW>::quad_sum(pb);
                        keep(pb);
                        bp[rate(r)] += pb;
                    }
                } else {
                    // (a skipped last row has ah = 0 and W = 0: no branch here)
                    rh[r] = gate[rate(r)] * ah[r];
                    bp[rate(r)] = fmaf(ah[r], a[r], bp[rate(r)]);
                }
    #pragma unroll
                for (int c = 0; c < L; ++c) eh[c] = fmaf(w[r][c], rh[r], eh[c]);
            }
            // (every lane of a row group holds the same bp: the exchange sums them
            // over the row-group lane bits only, and one lane per DPP row writes)
            // part[2] holds uh of step t+1 (zero before the first step)
    #pragma unroll
            for (int c = 0; c < L; ++c) {
                part[0][c] = khh[c];
                part[1][c] = eh[c];
            }
            exchange(par, bp);

            // stage the inputs of step t-1 (two slots away from anything in use)
            const int slot_prev = slot == 0 ? 2 : slot - 1;
            if (t > 0) {
                stage(slot_prev);
                if (t > 1) fetch(t - 2);
            }
            __syncthreads();

            // ---- (B) per column (lane j): totals, dx of step t+1, kbar, qbar, betah.
            float khh_j, eh_j, uh1_j;
            gather(par, khh_j, eh_j, uh1_j);
            if (t + 1 < T && wave == ((t + 1) & (NW - 1))) store_dx(t + 1, uh1_j, u_next);
            u_next = lane < D_IN ? us[jc] : 0.f;
            float kbar_v = 0.f, qbar_v = 0.f, zb = 0.f;  // BCAST: this lane's column of kbar, qbar; its beta row
            {
                // betah totals (with dealt columns each lane of the wave that
                // holds the beta rows sums its own row's, below)
                float bt[4] = {0.f, 0.f, 0.f, 0.f};
                if constexpr (!BCAST) {
    #pragma unroll
                    for (int c = 0; c < NLR; ++c) bt[c] = s_bred[par][0][c];
    #pragma unroll
                    for (int wv = 1; wv < NW; ++wv)
    #pragma unroll
                        for (int c = 0; c < NLR; ++c) bt[c] += s_bred[par][wv][c];
                }
                const float kh_j = lane < D_IN ? tt[TL::KH_OFF + jc] : 0.f;
                const float e_j = lane < D_IN ? tt[TL::E_OFF + jc] : 0.f;
                const float qh_j = kh_j + e_j;
                const float kb = khh_j - eh_j;
                // <kb, kh> and <eh, qh> over the 64 columns with one reduction: the
                // lower half-wave sums the first, the upper the second (columns j
                // and j +/- 32 joined by a lane-row swap), then a swap hands each
                // half the other's total.
                float pk = kb * kh_j, pq = eh_j * qh_j;
                swap32(pk, pq);                       // lower: kb kh of j, j+32; upper: eh qh of j-32, j
                float dk = half_sum(pk + pq);         // lower half: <kb, kh>; upper half: <eh, qh>
                float dq = dk;
                swap32(dk, dq);                       // every lane: dk = lower's total, dq = upper's
                if constexpr (BCAST) {
                    kbar_v = kh_j * (kb - dk);
                    qbar_v = qh_j * (eh_j - dq);
                    if constexpr (ZLDS) {
                        // column jc of this wave's dealt columns (all 64 in every wave)
                        s_zh[wave][D_OUT + jc] = kbar_v;
                        s_zh[wave][D_OUT + D_IN + jc] = qbar_v;
                    }
                    if (!last_empty) {
                        // this lane's beta row rg (rows past M hold zb = 0)
                        const int c = rg < NLR ? rg : 0;
                        float bsum = s_bred[par][0][c];
    #pragma unroll
                        for (int wv = 1; wv < NW; ++wv) bsum += s_bred[par][wv][c];
                        zb = rg < NLR ? (1.f - tt[TL::G_OFF + c]) * bsum : 0.f;
                    }
                } else {
                    if (lane < D_IN) {
                        s_zh[wave][D_OUT + lane] = kh_j * (kb - dk);
                        s_zh[wave][D_OUT + D_IN + lane] = qh_j * (eh_j - dq);
                    }
                    if (lane < NLR) {
                        const float bv = lane == 0 ? bt[0] : lane == 1 ? bt[1] : lane == 2 ? bt[2] : bt[3];
                        const float gl = lane == 0 ? gate[0] : lane == 1 ? gate[1] : lane == 2 ? gate[2] : gate[3];
                        s_zh[wave][MAIN + lane] = (1.f - gl) * bv;
                    }
                }
            }
            if constexpr (ZLDS) wave_sync();

            // ---- (C) uh of step t (column partials, reduced with step t-1); Wh update.
            float ev[L], uv[L];
            load_f32<L>(tt + TL::E_OFF + p * L, ev);
            load_f32<L>(us + p * L, uv);
    #pragma unroll
            for (int c = 0; c < L; ++c) part[2][c] = 0.f;
    #pragma unroll
            for (int r = 0; r < R; ++r) {
                if (r == R - 1 && last_empty) continue;
                const int row = srow(r);
                float zr;
                if (G * r < D_OUT) zr = gs[row];
                else if constexpr (BCAST) {
                    // rows of the beta block past M hold zb = 0
                    if (r >= RS) zr = zb;
                    else if constexpr (ZLDS) zr = s_zh[wave][row];
                    else zr = G * r < D_OUT + D_IN ? row_bcast(kbar_v, r - D_OUT / G)
                                                   : row_bcast(qbar_v, r - (D_OUT + D_IN) / G);
                } else {
                    const float zv = s_zh[wave][row_at(r, row)];
                    zr = row_ok(r, row) ? zv : 0.f;
                }
    #pragma unroll
                for (int c = 0; c < L; ++c) {
                    part[2][c] = fmaf(w[r][c], zr, part[2][c]);
                    wh[r][c] = fmaf(rh[r], ev[c], fmaf(zr, uv[c], wh[r][c]));
                }
            }

            // Reset ablation: step t = wR started window w from the initial state.
            // The adjoint now held is window w's share of dL/d(initial state); the
            // end state of window w-1, which the reset discarded, has a zero adjoint,
            // and the walk continues from that end state as the forward pass
            // recorded it (undoing updates cannot cross the reset).
            if (RESET && t == next_reset && t > 0) {
                add_share();
    #pragma unroll
                for (int r = 0; r < R; ++r)
    #pragma unroll
                    for (int c = 0; c < L; ++c) wh[r][c] = 0.f;
                const float* __restrict__ ws = wstates + ((int64_t)unit * n_resets + (t / reset_interval - 1)) * M * D_IN;
    #pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int row = srow(r);
                    if (row < M) load_f32<L>(ws + row * D_IN + p * L, w[r]);
                }
                next_reset -= reset_interval;
            }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    int t = T - 1;
    for (; t >= 0 && t % 6 != 5; --t) bstep(t, t % 3, t & 1);  // down to a step t = 5 (mod 6)
    for (; t >= 5; t -= 6) {
        bstep(t, I2{}, I1{});
        bstep(t - 1, I1{}, I0{});
        bstep(t - 2, I0{}, I1{});
        bstep(t - 3, I2{}, I0{});
        bstep(t - 4, I1{}, I1{});
        bstep(t - 5, I0{}, I0{});
    }

    if (T > 0) {
        // uh of step 0: one more exchange (no khh, eh, betah)
        float bp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < L; ++c) part[0][c] = part[1][c] = 0.f;
        exchange(1, bp);
        __syncthreads();
        float khh_j, eh_j, uh0_j;
        gather(1, khh_j, eh_j, uh0_j);
        if (wave == 0) store_dx(0, uh0_j, u_next);
    }

    // dL/d(initial state of this unit): with resets, the first window's share
    // added to the later windows' sum
    if (n_resets > 0) {
        add_share();
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = srow(r);
            if (row < M) store_f32<L>(dwi_unit + row * D_IN + p * L, wh[r]);
        }
    }
}

// ----------------------------------------------------------------------------
// Backward pass for units whose W and adjoint Wh do not both fit in the
// registers of one workgroup with room for the step's vectors (d = 128:
// 2 x 49,664 floats).  The same step as srwm_bwd_kernel, with these
// differences:
//   * the main rows (y, k, q: MAIN = d_out + 2 d_in of them, RM register rows
//     of G) are spread as in srwm_bwd_kernel: lane (rg, p) holds rows
//     rg + G*r, columns [p*L, p*L+L).  W stays in registers; of Wh, register
//     rows r < RL live in LDS and the rest in registers beside W.  The rate
//     rows (n_lr of them) sit in LDS, W and Wh, and are processed by wave 0,
//     whose lanes rg < n_lr take them as a last row (rows MAIN + rg): no
//     wave carries padding rows.  Every LDS element of the state is read and
//     written only by the lane that owns it, so every load follows that
//     thread's own store.  Nothing of the state leaves the chip during the
//     walk; dWinit is written once at the end.
//   * each pass over the rows takes a row's inputs (a_t entry, zh entry, Wh
//     row) as it reaches the row, so the step's vectors stay few;
//   * the per-column phase gives each lane CPL = D_IN / 64 columns
//     (j = lane + 64 c); each wave keeps only the zh entries of its own rows;
//   * gy_t is staged one entry per thread.
// No reset ablation (Wh has no second buffer to gather the windows' shares).
template <int D_IN, int D_OUT, int NW, int P, int NLR, bool RESET>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * kWave, NW * kWave), amdgpu_waves_per_eu(2)))
void srwm_bwd_wide_kernel(const float* __restrict__ WTin,
                          const float* __restrict__ tape, const float* __restrict__ gy,
                          const float* __restrict__ gWT, float* __restrict__ dx,
                          float* __restrict__ dWinit, int T, int H, int in_softmax, int /*reset_interval*/,
                          const float* __restrict__ /*wstates*/)
{
    static_assert(!RESET, "the wide backward has no reset variant");
    constexpr int NT = NW * kWave;
    constexpr int M = D_OUT + 2 * D_IN + NLR;
    constexpr int MAIN = D_OUT + 2 * D_IN;
    constexpr int L = D_IN / P;
    constexpr int G = NT / P;
    constexpr int RM = MAIN / G;       // register rows of the main rows
    constexpr int RG = kWave / P;      // row groups per wave
    constexpr int CPL = D_IN / kWave;  // columns per lane in the per-column phase
    using TL = TapeLayout<M, D_IN>;
    using CX = ColExchange<P, L>;
    constexpr int TW = TL::ROW;
    static_assert(D_IN % kWave == 0 && D_OUT % kWave == 0, "whole columns per lane");
    static_assert(D_IN % P == 0 && D_IN % G == 0 && D_OUT % G == 0 && MAIN % G == 0,
                  "row blocks must align with row groups");
    static_assert(D_OUT <= NT, "one thread per output");
    static_assert(L % 4 == 0, "16-byte pieces of Wh");
    static_assert((NW & (NW - 1)) == 0, "power-of-two waves");
    static_assert(RG >= 4, "wave 0 holds the rate rows as its row groups 0..n_lr-1");
    // register rows of Wh kept in LDS: as many as fit beside the staging
    // buffers; the other RM - RL rows are registers
    constexpr int RL = 7;
    constexpr int RR = RM - RL;
    static_assert(RL <= RM, "LDS rows");
    // zh entries a wave reads: its rows rg + G r for r >= D_OUT / G (the k, q
    // rows), RG per register row, and for wave 0 the n_lr rate rows
    constexpr int RZ0 = D_OUT / G;
    constexpr int NZ = (RM - RZ0) * RG + 4;

    __shared__ __attribute__((aligned(16))) float s_tape[3][TW];
    __shared__ __attribute__((aligned(16))) float s_gy[3][D_OUT];
    __shared__ __attribute__((aligned(16))) float s_red[2][NW][3][D_IN];
    __shared__ __attribute__((aligned(16))) float s_bred[2][NW][4];
    __shared__ __attribute__((aligned(16))) float s_zh[NW][NZ];
    __shared__ __attribute__((aligned(16))) float s_wh[RL][G][D_IN];
    __shared__ __attribute__((aligned(16))) float s_wb[2][4][D_IN];  // rate rows: [0] W, [1] Wh
    static_assert(sizeof(float) * (3 * TW + 3 * D_OUT + 2 * NW * 3 * D_IN + 2 * NW * 4 + NW * NZ +
                                   RL * G * D_IN + 8 * D_IN) <= 160 * 1024, "LDS");

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
    const int64_t x0 = ((int64_t)b * T * H + h) * D_IN;
    const int64_t y0 = ((int64_t)b * T * H + h) * D_OUT;
    const float* __restrict__ tp0 = tape + (int64_t)unit * T * TW;
    float* __restrict__ whu = dWinit + (int64_t)unit * M * D_IN;  // this unit's Wh at the end
    const float* __restrict__ wtu = WTin + (int64_t)unit * M * D_IN;
    const int rgw = rg - RG * wave;  // row group within the wave
    // the rate row of this lane when wave == 0 (rows >= n_lr: zero rows)
    const bool brow = wave == 0 && rg < NLR;

    // Wh register rows RL..RM-1
    float whr[RR > 0 ? RR : 1][L];
    // A lane's L floats of an LDS row are stored as L/4 16-byte pieces, piece
    // q of lane p at 16-byte slot q*P + p of the row group's D_IN floats: the
    // P lanes of a row group read or write one contiguous span per piece (no
    // bank conflicts), not pieces 4*L bytes apart.
    static_assert(L % 4 == 0 && D_IN == P * L, "16-byte pieces");
    auto lds_get = [&](const float* __restrict__ seg, float (&v)[L]) {
#pragma unroll
        for (int q = 0; q < L / 4; ++q) {
            const float4 f = *reinterpret_cast<const float4*>(seg + 4 * (q * P + p));
            v[4 * q] = f.x;
            v[4 * q + 1] = f.y;
            v[4 * q + 2] = f.z;
            v[4 * q + 3] = f.w;
        }
    };
    auto lds_put = [&](float* __restrict__ seg, const float (&v)[L]) {
#pragma unroll
        for (int q = 0; q < L / 4; ++q)
            *reinterpret_cast<float4*>(seg + 4 * (q * P + p)) = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    };
    auto load_wh = [&](int r, float (&v)[L]) {
        if (r < RL) {
            lds_get(&s_wh[r < RL ? r : 0][rg][0], v);
        } else {
#pragma unroll
            for (int c = 0; c < L; ++c) v[c] = whr[r < RL ? 0 : r - RL][c];
        }
    };
    auto store_wh = [&](int r, const float (&v)[L]) {
        if (r < RL) {
            lds_put(&s_wh[r < RL ? r : 0][rg][0], v);
        } else {
#pragma unroll
            for (int c = 0; c < L; ++c) whr[r < RL ? 0 : r - RL][c] = v[c];
        }
    };

    auto rate = [](int r) constexpr {
        const int row = G * r;
        return NLR == 1 ? 0 : row < D_OUT ? 0 : row < D_OUT + D_IN ? 1 : 2;
    };
    constexpr int RATE_B = NLR == 1 ? 0 : 3;

    // W <- W_T; Wh <- dL/dW_T (or 0).
    float w[RM][L];
#pragma unroll
    for (int r = 0; r < RM; ++r) {
        const int row = rg + G * r;
        float v[L];
        load_f32<L>(wtu + row * D_IN + p * L, w[r]);
        if (gWT != nullptr) {
            load_f32<L>(gWT + (int64_t)unit * M * D_IN + row * D_IN + p * L, v);
        } else {
#pragma unroll
            for (int c = 0; c < L; ++c) v[c] = 0.f;
        }
        store_wh(r, v);
    }
    if (wave == 0) {
        float wv[L], hv[L];
#pragma unroll
        for (int c = 0; c < L; ++c) wv[c] = hv[c] = 0.f;
        if (rg < NLR) {
            load_f32<L>(wtu + (MAIN + rg) * D_IN + p * L, wv);
            if (gWT != nullptr) load_f32<L>(gWT + (int64_t)unit * M * D_IN + (MAIN + rg) * D_IN + p * L, hv);
        }
        lds_put(&s_wb[0][rg][0], wv);
        lds_put(&s_wb[1][rg][0], hv);
    }

    // Step inputs (the tape row, which holds u_t, and gy_t) are copied two
    // steps ahead straight from global memory into the LDS ring (no
    // registers): the rows in 64-dword pieces, piece k by wave k mod NW (gy's
    // two pieces by the waves with fewest tape pieces), each lane one dword.
    constexpr int NPC = (TW + kWave - 1) / kWave;  // pieces of a tape row
    constexpr int NGC = D_OUT / kWave;             // pieces of a gy row
    static_assert(NPC <= 2 * NW && NPC % NW + NGC <= NW, "one or two tape pieces and at most one gy piece per wave");
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    // one buffer resource per row (wave-uniform, SGPRs) and the lane's byte
    // offset as the only per-lane operand: no 64-bit lane addresses held
    const int lane4 = 4 * lane;
    auto fetch = [&](int t, int slot) {
        const __amdgpu_buffer_rsrc_t trow = float_rsrc(tp0 + (int64_t)t * TW, TW);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int k = wu + NW * i;
            if (k < NPC && kWave * k + lane < TW) copy_dword_to_lds(trow, lane4, 4 * kWave * k, &s_tape[slot][kWave * k]);
        }
        const int kg = wu - NPC % NW;  // gy piece of the waves after those with two tape pieces
        if (kg >= 0 && kg < NGC)
            copy_dword_to_lds(float_rsrc(gy + y0 + (int64_t)t * y_step, D_OUT), lane4, 4 * kWave * kg, &s_gy[slot][kWave * kg]);
    };

    float part[3][L];
    auto exchange = [&](int par, float (&bp)[4]) {
        CX::run(part);
        if (CX::writer(lane)) {
            const int c0 = CX::col0(lane);
#pragma unroll
            for (int a = 0; a < 3; ++a) {
                if constexpr (CX::LC % 2 == 0) {
#pragma unroll
                    for (int c = 0; c < CX::LC; c += 2)
                        *reinterpret_cast<float2*>(&s_red[par][wave][a][c0 + c]) = make_float2(part[a][c], part[a][c + 1]);
                } else {
#pragma unroll
                    for (int c = 0; c < CX::LC; ++c) s_red[par][wave][a][c0 + c] = part[a][c];
                }
            }
        }
#pragma unroll
        for (int c = 0; c < NLR; ++c) {
            if constexpr (P == 4) {
                bp[c] += dpp<0x128>(bp[c]);
                bp[c] += dpp<0x124>(bp[c]);
            } else if constexpr (P == 8) {
                bp[c] = pair_sum<3>(bp[c]);
            }
        }
        if constexpr (NLR == 4) {
            swap32(bp[0], bp[2]);
            swap32(bp[1], bp[3]);
            float lo = bp[0] + bp[2], hi = bp[1] + bp[3];
            swap16(lo, hi);
            const float tot = lo + hi;
            if ((lane & 15) == 0) s_bred[par][wave][lane_now() >> 4] = tot;
        } else {
            const float tot = pair_sum<5>(pair_sum<4>(bp[0]));
            if (lane == 0) s_bred[par][wave][0] = tot;
        }
    };
    auto gather = [&](int par, float (&khh_j)[CPL], float (&eh_j)[CPL], float (&uh_j)[CPL]) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int j = lane + kWave * c;
            khh_j[c] = eh_j[c] = uh_j[c] = 0.f;
#pragma unroll
            for (int wv = 0; wv < NW; ++wv) {
                khh_j[c] += s_red[par][wv][0][j];
                eh_j[c] += s_red[par][wv][1][j];
                uh_j[c] += s_red[par][wv][2][j];
            }
        }
    };
    auto store_dx = [&](int t, const float (&uh_j)[CPL], const float (&u_j)[CPL]) {
        float d[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) d[c] = uh_j[c];
        if (in_softmax) {
            float s = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) s = fmaf(uh_j[c], u_j[c], s);
            const float du = wave_total(s);
#pragma unroll
            for (int c = 0; c < CPL; ++c) d[c] = u_j[c] * (uh_j[c] - du);
        }
        const __amdgpu_buffer_rsrc_t xrow = float_rsrc(dx + x0 + (int64_t)t * x_step, D_IN);
#pragma unroll
        for (int c = 0; c < CPL; ++c) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(d[c]), xrow, lane4, 4 * kWave * c, 0);
    };

#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int c = 0; c < L; ++c) part[a][c] = 0.f;
    float u_next[CPL];  // u_{t+1}, columns lane + 64 c
#pragma unroll
    for (int c = 0; c < CPL; ++c) u_next[c] = 0.f;

    if (T > 0) {
        fetch(T - 1, (T - 1) % 3);
        if (T > 1) fetch(T - 2, (T - 2) % 3);
        wait_vmem();
        __syncthreads();
    }

    int slot = (T - 1) % 3;
    for (int t = T - 1; t >= 0; --t) {
        const float* __restrict__ tt = s_tape[slot];
        const float* __restrict__ us = tt + TL::U_OFF;
        const float* __restrict__ gs = s_gy[slot];
        const int par = t & 1;

        // ---- (A) row by row: undo the update of step t; ah (row sums of
        // Wh kh) and rh = g ah; khh = Wh^T a, eh = W^T rh (column partials).
        float kt[L];
        load_f32<L>(tt + TL::KH_OFF + p * L, kt);
        const float4 gv = *reinterpret_cast<const float4*>(tt + TL::G_OFF);
        const float gate[4] = {gv.x, gv.y, gv.z, gv.w};
        float khh[L], eh[L], rh[RM];
        float rhb = 0.f;  // the rate row's rh (wave 0)
        float bp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < L; ++c) khh[c] = eh[c] = 0.f;
        // (A1) per row: undo, the row's partial of ah, khh; the next row's
        // Wh and a_t entry are requested before this row is processed, and a
        // scheduling fence per row keeps the loads from running further ahead
        // (each would hold a row of registers).
        {
            float whn[L];
            load_wh(0, whn);
            float an = tt[rg];
#pragma unroll
            for (int r = 0; r < RM; ++r) {
                float wh[L];
#pragma unroll
                for (int c = 0; c < L; ++c) wh[c] = whn[c];
                const float ar = an;
                if (r + 1 < RM) {
                    load_wh(r + 1, whn);
                    an = tt[rg + G * (r + 1)];
                }
                float as = 0.f;
#pragma unroll
                for (int c = 0; c < L; ++c) {
                    w[r][c] = fmaf(-ar, kt[c], w[r][c]);
                    as = fmaf(wh[c], kt[c], as);
                    khh[c] = fmaf(wh[c], ar, khh[c]);
                }
                rh[r] = as;
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // (A2) the row sums, all rows' DPP chains side by side; rh = g ah
        // (a_t entries read again from LDS rather than held in registers)
#pragma unroll
        for (int r = 0; r < RM; ++r) {
            const float ah = group_sum<P>(rh[r]);
            rh[r] = gate[rate(r)] * ah;
            bp[rate(r)] = fmaf(ah, tt[rg + G * r], bp[rate(r)]);
        }
        // (A3) eh = W^T rh (W after the undo)
#pragma unroll
        for (int r = 0; r < RM; ++r)
#pragma unroll
            for (int c = 0; c < L; ++c) eh[c] = fmaf(w[r][c], rh[r], eh[c]);
        if (wave == 0) {
            // the rate rows (zero rows for rg >= n_lr)
            const float av = tt[MAIN + (rg < NLR ? rg : 0)];
            const float ar = rg < NLR ? av : 0.f;
            float wv[L], wh[L];
            lds_get(&s_wb[0][rg][0], wv);
            lds_get(&s_wb[1][rg][0], wh);
            float as = 0.f;
#pragma unroll
            for (int c = 0; c < L; ++c) {
                wv[c] = fmaf(-ar, kt[c], wv[c]);
                as = fmaf(wh[c], kt[c], as);
                khh[c] = fmaf(wh[c], ar, khh[c]);
            }
            lds_put(&s_wb[0][rg][0], wv);
            const float ah = group_sum<P>(as);
            rhb = gate[RATE_B] * ah;
            bp[RATE_B] = fmaf(ah, ar, bp[RATE_B]);
#pragma unroll
            for (int c = 0; c < L; ++c) eh[c] = fmaf(wv[c], rhb, eh[c]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) bp[c] = p == 0 ? bp[c] : 0.f;
#pragma unroll
        for (int c = 0; c < L; ++c) {
            part[0][c] = khh[c];
            part[1][c] = eh[c];
        }
        exchange(par, bp);

        const int slot_prev = slot == 0 ? 2 : slot - 1;
        // step t-1's inputs (copied during step t+1) are in LDS for every wave
        // after this barrier; then step t-2's are requested into the slot step
        // t+1 used
        wait_vmem();
        __syncthreads();
        if (t > 1) fetch(t - 2, slot_prev == 0 ? 2 : slot_prev - 1);

        // ---- (B) per column (lane j = lane + 64 c): totals, dx of step t+1,
        // kbar, qbar, betah; each wave keeps the zh entries of its own rows.
        {
            float khh_j[CPL], eh_j[CPL], uh1_j[CPL];
            gather(par, khh_j, eh_j, uh1_j);
            if (t + 1 < T && wave == ((t + 1) & (NW - 1))) store_dx(t + 1, uh1_j, u_next);
#pragma unroll
            for (int c = 0; c < CPL; ++c) u_next[c] = us[lane + kWave * c];
            float bt[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) bt[c] = c < NLR ? s_bred[par][0][c] : 0.f;
#pragma unroll
            for (int wv = 1; wv < NW; ++wv)
#pragma unroll
                for (int c = 0; c < NLR; ++c) bt[c] += s_bred[par][wv][c];
            float kh_j[CPL], qh_j[CPL], kb[CPL];
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int j = lane + kWave * c;
                kh_j[c] = tt[TL::KH_OFF + j];
                qh_j[c] = kh_j[c] + tt[TL::E_OFF + j];
                kb[c] = khh_j[c] - eh_j[c];
                sk = fmaf(kb[c], kh_j[c], sk);
                sq = fmaf(eh_j[c], qh_j[c], sq);
            }
            wave_sum2(sk, sq);  // <kb, kh> and <eh, qh> over all D_IN columns
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int j = lane + kWave * c;
                // rows D_OUT + j (kbar) and D_OUT + D_IN + j (qbar): row group
                // j mod G, register rows RZ0 + j / G and RZ0 + (D_IN + j) / G
                const int jg = j % G;
                if (jg / RG == wave) {
                    s_zh[wave][(j / G) * RG + jg % RG] = kh_j[c] * (kb[c] - sk);
                    s_zh[wave][((D_IN + j) / G) * RG + jg % RG] = qh_j[c] * (eh_j[c] - sq);
                }
            }
            if (wave == 0 && lane < NLR) {
                const float bv = lane == 0 ? bt[0] : lane == 1 ? bt[1] : lane == 2 ? bt[2] : bt[3];
                const float gl = lane == 0 ? gate[0] : lane == 1 ? gate[1] : lane == 2 ? gate[2] : gate[3];
                s_zh[0][NZ - 4 + lane_now()] = (1.f - gl) * bv;
            }
        }
        wave_sync();

        // ---- (C) row by row: uh of step t (column partials, reduced with
        // step t-1); Wh += rh e^T + zh u^T.
        float ev[L], uv[L];
        load_f32<L>(tt + TL::E_OFF + p * L, ev);
        load_f32<L>(us + p * L, uv);
#pragma unroll
        for (int c = 0; c < L; ++c) part[2][c] = 0.f;
        {
            // per row, with the next row's Wh requested first (fenced as in A1)
            float whn[L];
            load_wh(0, whn);
#pragma unroll
            for (int r = 0; r < RM; ++r) {
                const int row = rg + G * r;
                const float zr = r < RZ0 ? gs[row] : s_zh[wave][(r < RZ0 ? 0 : r - RZ0) * RG + rgw];
                float wh[L];
#pragma unroll
                for (int c = 0; c < L; ++c) wh[c] = whn[c];
                if (r + 1 < RM) load_wh(r + 1, whn);
#pragma unroll
                for (int c = 0; c < L; ++c) part[2][c] = fmaf(w[r][c], zr, part[2][c]);
#pragma unroll
                for (int c = 0; c < L; ++c) wh[c] = fmaf(rh[r], ev[c], fmaf(zr, uv[c], wh[c]));
                store_wh(r, wh);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (wave == 0) {
            const int rg0 = lane_now() / P;  // rg of wave 0's lanes
            const float zv = s_zh[0][NZ - 4 + (rg0 < NLR ? rg0 : 0)];
            const float zr = rg < NLR ? zv : 0.f;
            float wv[L], wh[L];
            lds_get(&s_wb[0][rg][0], wv);
            lds_get(&s_wb[1][rg][0], wh);
#pragma unroll
            for (int c = 0; c < L; ++c) part[2][c] = fmaf(wv[c], zr, part[2][c]);
#pragma unroll
            for (int c = 0; c < L; ++c) wh[c] = fmaf(rhb, ev[c], fmaf(zr, uv[c], wh[c]));
            lds_put(&s_wb[1][rg][0], wh);
        }
        slot = slot_prev;
    }

    if (T > 0) {
        // uh of step 0: one more exchange (no khh, eh, betah)
        float bp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < L; ++c) part[0][c] = part[1][c] = 0.f;
        exchange(1, bp);
        __syncthreads();
        float khh_j[CPL], eh_j[CPL], uh0_j[CPL];
        gather(1, khh_j, eh_j, uh0_j);
        if (wave == 0) store_dx(0, uh0_j, u_next);
    }
    // dWinit <- Wh = dL/d(initial state of this unit).
#pragma unroll
    for (int r = 0; r < RM; ++r) {
        const int row = rg + G * r;
        float v[L];
        load_wh(r, v);
        store_f32<L>(whu + row * D_IN + p * L, v);
    }
    if (brow) {
        float v[L];
        lds_get(&s_wb[1][rg][0], v);
        store_f32<L>(whu + (MAIN + rg) * D_IN + p * L, v);
    }
}

// dW0[h] = sum_b dWinit[b][h] (the gradient of the initial matrix shared over
// the batch), summed in a fixed order b = 0, 1, ...; with `accumulate` the sum
// continues from dW0's value (a batch summed in slices, in order).
__global__ __launch_bounds__(256) void srwm_sum_over_batch_kernel(const float* __restrict__ dWinit,
                                                                  float* __restrict__ dW0, int64_t B,
                                                                  int64_t per_b, int accumulate)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= per_b) return;
    float s = accumulate ? dW0[i] : 0.f;
    for (int64_t b = 0; b < B; ++b) s += dWinit[b * per_b + i];
    dW0[i] = s;
}

}  // namespace srwm
