// srwm_fwp.hip -- gfx950 kernels and C ABI of the fast-weight programmers the
// SRWM is compared with and built into: DeltaNet and SR-DeltaNet.
//
// DeltaNet (review page "SRWM: 让权重矩阵学习修改自身", Sec. 2.1): a slow
// matrix maps the input x_t to [k; v; q; beta] (in the order the page names
// them), and a separate fast matrix F (d_v x d_key per head, zero at the start
// unless a state is carried in) gets a delta write at the key and is then
// queried:
//     kh = softmax(k), qh = softmax(q), g = sigmoid(beta)
//     vb = F kh;   F += g (v - vb) kh^T;   y_t = F qh    (F after the write)
// The slow projection is full width: head h's rows of W_slow[H*P][H*d_in]
// read the whole x_t (the page contrasts DeltaNet's (D, D) projection with
// the SRWM's per-head one).  P = d_v + 2*d_key + 1.
//
// SR-DeltaNet (same page, Appendix C.1): an SRWM (per head, d_out = P)
// replaces the slow projection; its output y^SR_t, which it takes from its
// matrix before its own update, is the fast step's projection.
//
// Layout of the work:
//   * The projection of every step is independent of F, so it is computed
//     for all (b, t) first: for DeltaNet one dense GEMM, Z = X W_slow^T, on
//     the fp32 matrix cores (v_mfma_f32_16x16x4_f32); for SR-DeltaNet the SRWM
//     kernel of srwm_fwd.hip with y = Z.  Z[B][T][H][P] is a caller-provided
//     float32 buffer.
//   * The fast-matrix recurrence: one workgroup per (b, h) unit, the rows of
//     F split over its waves and held in registers.  The softmaxes depend
//     only on Z, so they are formed a chunk of steps ahead, off the serial
//     chain; per step the chain is two row reductions and the write.
//     y_t = F_{t-1} qh + a (kh . qh) with a = g (v - vb): the query of the
//     written matrix without a second pass over it.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "srwm.h"
#include "srwm_device.h"

namespace {

using namespace srwm;

typedef float v4f __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------------------
// Z[n][c] = sum_k X[n][k] W[c][k]: n < N (= B*T rows of x), c < C (= H*P),
// k < K (= H*d_in, K % 4 == 0).  Workgroup tile 64 x 128, four waves of
// 32 x 64 (2 x 4 MFMA tiles of 16 x 16), K staged through LDS 32 at a time.
// MFMA 16x16x4 f32 operand layout: lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; accumulator register r of lane l is D[4 (l / 16) + r][l % 16].
constexpr int kGM = 64, kGN = 128, kGK = 32, kGPad = 4;
static_assert(kGK == 32, "one chunk of K: eight MFMA steps of four lane groups");
// A remainder of at most kGX columns past the last whole column tile is
// taken by that tile as one more 16-column MFMA block (each wave computes one
// 16 x 16 piece of it), instead of a tile of its own that would be nearly all
// padding: DeltaNet's C = 2 x 193 = 386 would otherwise spend a quarter of
// its MFMAs on a tile with 2 real columns.
constexpr int kGX = 16;
__host__ __device__ constexpr int64_t gemm_col_tiles(int64_t C)
{
    return (C > kGN && C % kGN != 0 && C % kGN <= kGX) ? C / kGN : (C + kGN - 1) / kGN;
}

// Workgroups are dispatched to the 8 XCDs round-robin (workgroup i on XCD
// i % 8), each XCD with its own L2.  The 1-D grid is renumbered so that the
// column tiles of one row tile are consecutive on one XCD: the x rows are
// fetched from HBM once and re-read from that XCD's L2.
constexpr int kXcds = 8;

__global__ __launch_bounds__(256) void srwm_proj_gemm_kernel(const float* __restrict__ X,
                                                             const float* __restrict__ W,
                                                             float* __restrict__ Z, int64_t N, int C,
                                                             int K)
{
    __shared__ __attribute__((aligned(16))) float sX[kGM][kGK + kGPad];
    __shared__ __attribute__((aligned(16))) float sW[kGN + kGX][kGK + kGPad];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t ctiles = gemm_col_tiles(C);
    const int64_t tiles = ((N + kGM - 1) / kGM) * ctiles;
    const int64_t per_xcd = (int64_t)gridDim.x / kXcds;  // grid is a multiple of kXcds
    const int64_t g = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (g >= tiles) return;  // padding workgroups (whole workgroup, before any barrier)
    const int64_t n0 = (g / ctiles) * kGM;
    const int c0 = static_cast<int>(g % ctiles) * kGN;
    const int wm = (wave >> 1) * 32, wn = (wave & 1) * 64;
    const bool wodd = __builtin_amdgcn_readfirstlane(wave) & 1;  // uniform
    const int lr = tid >> 3, lc = (tid & 7) * 4;  // loader: rows lr, lr + 32; columns lc..lc+3
    // The tile's corner in X, W and Z (uniform): inside a tile every element
    // is a 32-bit offset from it.
    const float* __restrict__ Xt = X + n0 * K;
    const float* __restrict__ Wt = W + (int64_t)c0 * K;
    float* __restrict__ Zt = Z + n0 * C + c0;

    // FULL: every row, column and K chunk of the tile exists (all but the
    // edge tiles), so loads and stores need no bounds checks.  EXTRA: the
    // last column tile with the remainder columns (checked: only C - c0 - kGN
    // of its 16 are real).
    auto run = [&](auto full, auto extra) {
        constexpr bool FULL = decltype(full)::value;
        constexpr bool EXTRA = decltype(extra)::value;
        v4f c00 = {0.f, 0.f, 0.f, 0.f}, c01 = c00, c02 = c00, c03 = c00;
        v4f c10 = c00, c11 = c00, c12 = c00, c13 = c00, cx = c00;
        // K chunk k0's X pieces (rows lr, lr + 32) and W pieces (rows lr +
        // 32 i) of this thread; with EXTRA, threads < 128 also row kGN + lr of W
        float4 px0, px1, pw0, pw1, pw2, pw3, pwx = make_float4(0.f, 0.f, 0.f, 0.f);
        auto piece = [&](const float* __restrict__ base, int row0, int lim, int r, int gk) {
            if constexpr (FULL) {
                return *reinterpret_cast<const float4*>(base + static_cast<uint32_t>(r * K + gk));
            } else {
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (row0 + r < lim && gk < K) v = *reinterpret_cast<const float4*>(base + static_cast<int64_t>(r) * K + gk);
                return v;
            }
        };
        const int nl = N - n0 < kGM ? static_cast<int>(N - n0) : kGM;  // rows of the tile that exist
        auto fetch = [&](int k0) {
            px0 = piece(Xt, 0, nl, lr, k0 + lc);
            px1 = piece(Xt, 0, nl, lr + 32, k0 + lc);
            pw0 = piece(Wt, c0, C, lr, k0 + lc);
            pw1 = piece(Wt, c0, C, lr + 32, k0 + lc);
            pw2 = piece(Wt, c0, C, lr + 64, k0 + lc);
            pw3 = piece(Wt, c0, C, lr + 96, k0 + lc);
            if constexpr (EXTRA) {
                // rows kGN .. kGN + 15 of the tile, bounds-checked against C
                pwx = make_float4(0.f, 0.f, 0.f, 0.f);
                if (tid < 8 * kGX && c0 + kGN + lr < C && k0 + lc < K)
                    pwx = *reinterpret_cast<const float4*>(Wt + static_cast<int64_t>(kGN + lr) * K + k0 + lc);
            }
        };
        fetch(0);
        for (int k0 = 0; k0 < K; k0 += kGK) {
            *reinterpret_cast<float4*>(&sX[lr][lc]) = px0;
            *reinterpret_cast<float4*>(&sX[lr + 32][lc]) = px1;
            *reinterpret_cast<float4*>(&sW[lr][lc]) = pw0;
            *reinterpret_cast<float4*>(&sW[lr + 32][lc]) = pw1;
            *reinterpret_cast<float4*>(&sW[lr + 64][lc]) = pw2;
            *reinterpret_cast<float4*>(&sW[lr + 96][lc]) = pw3;
            if constexpr (EXTRA) {
                if (tid < 8 * kGX) *reinterpret_cast<float4*>(&sW[kGN + lr][lc]) = pwx;
            }
            __syncthreads();
            // the next chunk's loads are in flight while this one's MFMAs run
            if (k0 + kGK < K) fetch(k0 + kGK);
            // The sum over k is order-free, so in MFMA step s of the chunk lane
            // group j = lane / 16 supplies k = 8 j + s: its operands for all eight
            // steps are 8 consecutive floats of one row, one 16-byte LDS read per
            // half of four steps.
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int kb = 8 * (lane >> 4) + 4 * hf;
                const int ra = wm + (lane & 15), rb = wn + (lane & 15);
                const float4 a0 = *reinterpret_cast<const float4*>(&sX[ra][kb]);
                const float4 a1 = *reinterpret_cast<const float4*>(&sX[ra + 16][kb]);
                const float4 b0 = *reinterpret_cast<const float4*>(&sW[rb][kb]);
                const float4 b1 = *reinterpret_cast<const float4*>(&sW[rb + 16][kb]);
                const float4 b2 = *reinterpret_cast<const float4*>(&sW[rb + 32][kb]);
                const float4 b3 = *reinterpret_cast<const float4*>(&sW[rb + 48][kb]);
                const float av0[4] = {a0.x, a0.y, a0.z, a0.w}, av1[4] = {a1.x, a1.y, a1.z, a1.w};
                const float bv0[4] = {b0.x, b0.y, b0.z, b0.w}, bv1[4] = {b1.x, b1.y, b1.z, b1.w};
                const float bv2[4] = {b2.x, b2.y, b2.z, b2.w}, bv3[4] = {b3.x, b3.y, b3.z, b3.w};
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    c00 = __builtin_amdgcn_mfma_f32_16x16x4f32(av0[st], bv0[st], c00, 0, 0, 0);
                    c01 = __builtin_amdgcn_mfma_f32_16x16x4f32(av0[st], bv1[st], c01, 0, 0, 0);
                    c02 = __builtin_amdgcn_mfma_f32_16x16x4f32(av0[st], bv2[st], c02, 0, 0, 0);
                    c03 = __builtin_amdgcn_mfma_f32_16x16x4f32(av0[st], bv3[st], c03, 0, 0, 0);
                    c10 = __builtin_amdgcn_mfma_f32_16x16x4f32(av1[st], bv0[st], c10, 0, 0, 0);
                    c11 = __builtin_amdgcn_mfma_f32_16x16x4f32(av1[st], bv1[st], c11, 0, 0, 0);
                    c12 = __builtin_amdgcn_mfma_f32_16x16x4f32(av1[st], bv2[st], c12, 0, 0, 0);
                    c13 = __builtin_amdgcn_mfma_f32_16x16x4f32(av1[st], bv3[st], c13, 0, 0, 0);
                }
                if constexpr (EXTRA) {
                    // this wave's piece of the extra block: rows 16 wave .. +15,
                    // which are the rows of its A operand av0 (even waves) or
                    // av1 (odd waves), already in registers
                    const float4 bx = *reinterpret_cast<const float4*>(&sW[kGN + (lane & 15)][kb]);
                    const float bxv[4] = {bx.x, bx.y, bx.z, bx.w};
#pragma unroll
                    for (int st = 0; st < 4; ++st)
                        cx = __builtin_amdgcn_mfma_f32_16x16x4f32(wodd ? av1[st] : av0[st], bxv[st], cx, 0, 0, 0);
                }
            }
            __syncthreads();
        }
        const v4f acc[2][4] = {{c00, c01, c02, c03}, {c10, c11, c12, c13}};
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = wn + 16 * j + (lane & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = wm + 16 * i + 4 * (lane >> 4) + r;
                    if constexpr (FULL) {
                        Zt[static_cast<uint32_t>(row * C + col)] = acc[i][j][r];
                    } else {
                        if (n0 + row < N && c0 + col < C) Zt[static_cast<int64_t>(row) * C + col] = acc[i][j][r];
                    }
                }
            }
        if constexpr (EXTRA) {
            const int col = kGN + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * wave + 4 * (lane >> 4) + r;
                if ((FULL || n0 + row < N) && c0 + col < C) Zt[static_cast<int64_t>(row) * C + col] = cx[r];
            }
        }
    };
    // (the 32-bit offsets: rows * K and rows * C within a tile stay below 2^31)
    const bool full = n0 + kGM <= N && c0 + kGN <= C && K % kGK == 0 && K <= INT32_MAX / (kGN + kGX) &&
                      C <= INT32_MAX / kGM;
    const bool extra = c0 + kGN < C && g % ctiles == ctiles - 1;  // the last tile, with the remainder
    if (full) {
        if (extra) run(std::true_type{}, std::true_type{});
        else run(std::true_type{}, std::false_type{});
    } else {
        if (extra) run(std::false_type{}, std::true_type{});
        else run(std::false_type{}, std::false_type{});
    }
}

// ----------------------------------------------------------------------------
// The fast-matrix recurrence.  Z[b][t][h][0..PR) holds the projection
// [k; v; q; beta] of step t.  One workgroup of NW waves per unit; the rows of
// F are independent of each other (each row's write and query need only kh,
// qh, g and its own value), so wave w owns rows [w*RW, (w+1)*RW), RW = d_v/NW,
// and lane (rg, p) of the wave holds rows rg + G*r and columns [p*L, p*L+L).
// Steps are handled S at a time: the softmaxes, values and gates of chunk c+1
// are formed (wave w takes steps w, w+NW, ... of the chunk, from registers
// loaded a chunk earlier) into one half of a double-buffered LDS area while
// the matrix work of chunk c runs from the other half; one workgroup barrier
// per chunk.  With NPW > 0 the preparation is left to NPW extra waves, which
// form chunk c+1 while the NW row-holding waves work through chunk c (the
// recurrence is bound by its per-step dependency chain, so the preparation
// fills issue slots the recurrence leaves idle).
template <int D_KEY, int D_V, int NW, int P, int S, int NPW = 0>
__global__ __launch_bounds__((NW + NPW) * 64) void srwm_fast_kernel(const float* __restrict__ Z,
                                                            const float* __restrict__ F0,
                                                            float* __restrict__ y, float* __restrict__ FT,
                                                            int T, int t_stride, int H)
{
    constexpr int PR = D_V + 2 * D_KEY + 1;
    constexpr int L = D_KEY / P;
    constexpr int G = kWave / P;
    constexpr int RW = D_V / NW;             // rows per wave
    constexpr int R = (RW + G - 1) / G;      // rows per lane
    constexpr int EZ = (PR + kWave - 1) / kWave;
    constexpr int V0 = D_KEY, Q0 = D_KEY + D_V, BETA = PR - 1;
    constexpr int NPREP = NPW > 0 ? NPW : NW;  // waves that prepare a chunk
    constexpr int SW = S / NPREP;              // steps each of them prepares per chunk
    // prepared step: kh [0, D_KEY), qh [D_KEY, 2 D_KEY), v [2 D_KEY, +D_V), g
    constexpr int KQ = 2 * D_KEY, GO = KQ + D_V, KP = (GO + 2 + 3) & ~3;
    // <kh, qh> of a step is formed once, by the wave that prepares the step,
    // when lane j holds key column j and query column j of the raw projection
    // (stored at GO + 1); otherwise every wave forms it per step.
    constexpr bool KQ_PREP = D_KEY <= kWave && Q0 % kWave == 0;
    static_assert(D_KEY % P == 0 && D_V % NW == 0 && S % NPREP == 0, "shapes");
    static_assert(D_KEY % 4 == 0 && D_V % 4 == 0, "16-byte sections");

    __shared__ __attribute__((aligned(16))) float s_p[2][S][KP];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = NW + NPW == 1 ? 0 : tid / kWave;
    const bool rec = NPW == 0 || wave < NW;      // holds rows of F
    const bool preps = NPW == 0 || wave >= NW;   // prepares steps
    const int pw = NPW > 0 ? wave - NW : wave;   // index among the preparing waves
    const int p = lane % P;
    const int rg = lane / P;
    const int row0 = wave * RW;
    const int unit = blockIdx.x;
    const int b = unit / H;
    const int h = unit - b * H;
    const int64_t z_step = (int64_t)H * PR;
    const int64_t z0 = ((int64_t)b * t_stride * H + h) * PR;  // sequences t_stride (>= T) steps apart
    const int64_t y_step = (int64_t)H * D_V;
    const int64_t y0 = ((int64_t)b * t_stride * H + h) * D_V;

    float F[R][L];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int lr = rg + G * r;
        if (F0 != nullptr && lr < RW && rec) {
            load_f32<L>(F0 + ((int64_t)unit * D_V + row0 + lr) * D_KEY + p * L, F[r]);
        } else {
#pragma unroll
            for (int c = 0; c < L; ++c) F[r][c] = 0.f;
        }
    }

    // This wave's share of a chunk's raw projections: steps c0 + pw + NPREP*j.
    float zr[SW][EZ];
    auto load_chunk = [&](int c0) {
#pragma unroll
        for (int j = 0; j < SW; ++j) {
            const int t = c0 + pw + NPREP * j;
            // one row address per step; its EZ pieces are constant offsets from it
            const float* __restrict__ zrow = Z + z0 + (int64_t)t * z_step + lane;
#pragma unroll
            for (int i = 0; i < EZ; ++i) {
                const int e = lane + kWave * i;
                zr[j][i] = (t < T && e < PR) ? zrow[kWave * i] : 0.f;
            }
        }
    };
    // Softmaxes, values and gates of this wave's steps of a chunk.
    auto prep_chunk = [&](int buf) {
#pragma unroll
        for (int j = 0; j < SW; ++j) {
            const int s = pw + NPREP * j;
            float mk = -INFINITY, mq = -INFINITY;
#pragma unroll
            for (int i = 0; i < EZ; ++i) {
                const int e = lane + kWave * i;
                if (e < V0) mk = fmax2(mk, zr[j][i]);
                else if (e >= Q0 && e < BETA) mq = fmax2(mq, zr[j][i]);
            }
            wave_max2(mk, mq);
            float ex[EZ];
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int i = 0; i < EZ; ++i) {
                const int e = lane + kWave * i;
                const bool isk = e < V0, isq = e >= Q0 && e < BETA;
                ex[i] = isk ? exp_f32(zr[j][i] - mk) : isq ? exp_f32(zr[j][i] - mq) : 0.f;
                if (isk) sk += ex[i];
                if (isq) sq += ex[i];
            }
            wave_sum2(sk, sq);
            const float ik = rcp_f32(sk), iq = rcp_f32(sq);
            if constexpr (KQ_PREP) {
                const float kq = wave_total(lane < D_KEY ? ex[0] * ex[Q0 / kWave] : 0.f) * (ik * iq);
                if (lane == 0) s_p[buf][s][GO + 1] = kq;
            }
#pragma unroll
            for (int i = 0; i < EZ; ++i) {
                const int e = lane + kWave * i;
                if (e < V0) s_p[buf][s][e] = ex[i] * ik;
                else if (e < Q0) s_p[buf][s][KQ + e - V0] = zr[j][i];
                else if (e < BETA) s_p[buf][s][D_KEY + e - Q0] = ex[i] * iq;
                else if (e == BETA) s_p[buf][s][GO] = sigmoid_f32(zr[j][i]);
            }
        }
    };

    if (T > 0) {
        if (preps) {
            load_chunk(0);
            prep_chunk(0);
            if (T > S) load_chunk(S);
        }
        __syncthreads();
    }
    for (int c0 = 0, chunk = 0; c0 < T; c0 += S, ++chunk) {
        const int buf = chunk & 1;
        if (preps && c0 + S < T) {
            prep_chunk(buf ^ 1);
            if (c0 + 2 * S < T) load_chunk(c0 + 2 * S);
        }
        const int n = !rec ? 0 : (T - c0) < S ? (T - c0) : S;
        // step c0 + s of the chunk (in a full chunk every s is a constant:
        // the prepared vectors' LDS addresses and y's offset are immediates)
        auto fstep = [&](const int s) {
            const float* __restrict__ ps = s_p[buf][s];
            float kh[L], qh[L];
            load_f32<L>(ps + p * L, kh);
            load_f32<L>(ps + D_KEY + p * L, qh);
            const float g = ps[GO];
            float kq = 0.f;
            if constexpr (KQ_PREP) {
                kq = ps[GO + 1];
            } else {
#pragma unroll
                for (int c = 0; c < L; ++c) kq = fmaf(kh[c], qh[c], kq);
                kq = group_sum<P>(kq);
            }
            const int64_t yt = y0 + (int64_t)(c0 + s) * y_step + row0;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int lr = rg + G * r;
                float s1 = 0.f, s2 = 0.f;
#pragma unroll
                for (int c = 0; c < L; ++c) {
                    s1 = fmaf(F[r][c], kh[c], s1);
                    s2 = fmaf(F[r][c], qh[c], s2);
                }
                s1 = group_sum<P>(s1);  // vb: the key address's content
                s2 = group_sum<P>(s2);  // F_{t-1} qh
                const float v = lr < RW ? ps[KQ + row0 + lr] : 0.f;
                const float a = g * (v - s1);
#pragma unroll
                for (int c = 0; c < L; ++c) F[r][c] = fmaf(a, kh[c], F[r][c]);
                // y formed in every lane before the store's branch: otherwise the
                // last DPP level of s2 sinks into the branch as a move and an add
                float yv = fmaf(a, kq, s2);
                asm volatile("" : "+v"(yv));
                if (p == 0 && lr < RW) y[yt + lr] = yv;
            }
        };
        if (n == S) {
#pragma unroll
            for (int s = 0; s < S; ++s) fstep(s);
        } else {
            for (int s = 0; s < n; ++s) fstep(s);
        }
        __syncthreads();
    }

    if (FT != nullptr && rec) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int lr = rg + G * r;
            if (lr < RW) store_f32<L>(FT + ((int64_t)unit * D_V + row0 + lr) * D_KEY + p * L, F[r]);
        }
    }
}

// ----------------------------------------------------------------------------
// Variants: (d_key, d_v, lanes per row).
using FastFn = void (*)(const float*, const float*, float*, float*, int, int, int);
struct FastVariant {
    int d_key, d_v, nw, npw;  // row-holding waves, preparing waves
    FastFn fn;
};
// (d_key, d_v, waves per unit, lanes per row, steps per chunk, preparing waves)
const FastVariant kFastVariants[] = {
    {8, 8, 1, 0, &srwm_fast_kernel<8, 8, 1, 8, 16>},
    {16, 16, 1, 0, &srwm_fast_kernel<16, 16, 1, 4, 16>},
    {64, 64, 4, 4, &srwm_fast_kernel<64, 64, 4, 4, 16, 4>},
    {64, 64, 8, 4, &srwm_fast_kernel<64, 64, 8, 8, 16, 4>},
};
constexpr int kNumFastVariants = sizeof(kFastVariants) / sizeof(kFastVariants[0]);

// The most row-holding waves per unit that keep units * nw within four waves
// per SIMD of the chip (4096); else the fewest.  The bound counts the
// row-holding waves only: the preparing waves sit beside them (512 units of
// the 8 + 4 variant launch 6144 waves), which measured faster than the
// 4 + 4 variant at 512 units.
int find_fast(int64_t d_key, int64_t d_v, int64_t units = 1)
{
    int best = -1, fewest = -1;
    for (int i = 0; i < kNumFastVariants; ++i) {
        const FastVariant& v = kFastVariants[i];
        if (v.d_key != d_key || v.d_v != d_v) continue;
        if (fewest < 0 || v.nw < kFastVariants[fewest].nw) fewest = i;
        if (units * v.nw <= 4096 && (best < 0 || v.nw > kFastVariants[best].nw)) best = i;
    }
    return best >= 0 ? best : fewest;
}

// Byte sizes shared by both entry points: x, z, y and one fast state per unit.
struct FwpSizes {
    int64_t units, steps, nx, nz, ny, nf;
};

int fwp_sizes(int64_t B, int64_t T, int64_t H, int64_t d_in, int64_t d_key, int64_t d_v, FwpSizes* s)
{
    if (B < 0 || T < 0 || H < 0 || d_in < 1 || d_key < 1 || d_v < 1) return SRWM_ERR_SHAPE;
    const int64_t P = d_v + 2 * d_key + 1;
    if (!mul_ok(B, H, &s->units) || !mul_ok(s->units, T, &s->steps) || !mul_ok(s->steps, d_in * 4, &s->nx) ||
        !mul_ok(s->steps, P * 4, &s->nz) || !mul_ok(s->steps, d_v * 4, &s->ny) ||
        !mul_ok(s->units, d_v * d_key * 4, &s->nf))
        return SRWM_ERR_SHAPE;
    if (s->units > INT32_MAX || T > INT32_MAX || H > INT32_MAX) return SRWM_ERR_SHAPE;
    return SRWM_OK;
}

// Steps of each head that buffers of T steps per sequence, sequences
// t_stride (0: T) apart, cover: (B-1)*t_stride + T, or 0 when empty.
int time_span(int64_t B, int64_t T, int64_t t_stride, int64_t* span)
{
    if (t_stride < 0 || (t_stride > 0 && t_stride < T)) return SRWM_ERR_SHAPE;
    const int64_t S = t_stride > 0 ? t_stride : T;
    if (S > INT32_MAX || !mul_ok(B > 0 ? B - 1 : 0, S, span) || *span > INT64_MAX - T) return SRWM_ERR_SHAPE;
    *span = (B > 0 && T > 0) ? *span + T : 0;
    return SRWM_OK;
}

int launch_fast(int vi, const float* z, const float* F0, float* y, float* FT, int64_t units, int64_t T,
                int64_t t_stride, int64_t H, void* stream)
{
    int Ti = static_cast<int>(T), Si = static_cast<int>(t_stride > 0 ? t_stride : T), Hi = static_cast<int>(H);
    void* args[] = {const_cast<float**>(&z), const_cast<float**>(&F0), &y, &FT, &Ti, &Si, &Hi};
    const hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(kFastVariants[vi].fn),
                                           dim3(static_cast<unsigned>(units)), dim3((kFastVariants[vi].nw + kFastVariants[vi].npw) * kWave), args, 0,
                                           static_cast<hipStream_t>(stream));
    return err == hipSuccess ? SRWM_OK : SRWM_ERR_HIP;
}

// The checks of a DeltaNet call; `project_only` skips the fast-matrix buffers.
int deltanet_check(const srwm_deltanet_args_t* a, bool project_only, int* vi, int64_t* K, int64_t* C)
{
    if (a == nullptr) return SRWM_ERR_NULL;
    FwpSizes s;
    int rc = fwp_sizes(a->B, a->T, a->H, a->d_in, a->d_key, a->d_v, &s);
    if (rc != SRWM_OK) return rc;
    *vi = find_fast(a->d_key, a->d_v, s.units);
    if (*vi < 0 && !project_only) return SRWM_ERR_UNSUPPORTED;
    const int64_t P = a->d_v + 2 * a->d_key + 1;
    int64_t nw;
    if (!mul_ok(a->H, a->d_in, K) || !mul_ok(a->H, P, C) || !mul_ok(*C, *K * 4, &nw)) return SRWM_ERR_SHAPE;
    if (*K % 4 != 0) return SRWM_ERR_SHAPE;  // 16-byte rows of x and W_slow
    if (*K > INT32_MAX || *C > INT32_MAX) return SRWM_ERR_SHAPE;
    if (s.units == 0) return SRWM_OK;
    if (s.nx > 0 && (a->x == nullptr || a->W_slow == nullptr || a->z == nullptr || (!project_only && a->y == nullptr)))
        return SRWM_ERR_NULL;
    const float* F0 = project_only ? nullptr : a->F0;
    float* y = project_only ? nullptr : a->y;
    float* FT = project_only ? nullptr : a->F_T;
    if ((reinterpret_cast<uintptr_t>(a->x) | reinterpret_cast<uintptr_t>(a->W_slow) |
         reinterpret_cast<uintptr_t>(F0) | reinterpret_cast<uintptr_t>(a->z) |
         reinterpret_cast<uintptr_t>(y) | reinterpret_cast<uintptr_t>(FT)) & 15u)
        return SRWM_ERR_ARG;
    const void* ins[] = {a->x, a->W_slow, F0};
    const int64_t nins[] = {s.nx, nw, F0 ? s.nf : 0};
    void* outs[] = {a->z, y, FT};
    const int64_t nouts[] = {s.nz, y ? s.ny : 0, FT ? s.nf : 0};
    for (int o = 0; o < 3; ++o) {
        for (int i = 0; i < 3; ++i)
            if (ranges_overlap(outs[o], nouts[o], ins[i], nins[i])) return SRWM_ERR_ALIAS;
        for (int o2 = o + 1; o2 < 3; ++o2)
            if (ranges_overlap(outs[o], nouts[o], outs[o2], nouts[o2])) return SRWM_ERR_ALIAS;
    }
    return SRWM_OK;
}

int launch_projection(const srwm_deltanet_args_t* a, int64_t K, int64_t C)
{
    const int64_t N = a->B * a->T;
    if (N == 0 || a->H == 0) return SRWM_OK;
    const float* X = a->x;
    const float* Wp = a->W_slow;
    float* Zp = a->z;
    int Ci = static_cast<int>(C), Ki = static_cast<int>(K);
    int64_t Nv = N;
    void* args[] = {const_cast<float**>(&X), const_cast<float**>(&Wp), &Zp, &Nv, &Ci, &Ki};
    const int64_t tiles = ((N + kGM - 1) / kGM) * gemm_col_tiles(C);
    const int64_t grid = (tiles + kXcds - 1) / kXcds * kXcds;
    if (grid > INT32_MAX) return SRWM_ERR_SHAPE;
    const hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(&srwm_proj_gemm_kernel),
                                           dim3(static_cast<unsigned>(grid)), dim3(256), args, 0,
                                           static_cast<hipStream_t>(a->stream));
    return err == hipSuccess ? SRWM_OK : SRWM_ERR_HIP;
}

int deltanet_impl(const srwm_deltanet_args_t* a, bool project_only)
{
    int vi;
    int64_t K, C;
    const int rc = deltanet_check(a, project_only, &vi, &K, &C);
    if (rc != SRWM_OK) return rc;
    if (a->B * a->H == 0) return SRWM_OK;
    const int rp = launch_projection(a, K, C);
    if (rp != SRWM_OK || project_only) return rp;
    return launch_fast(vi, a->z, a->F0, a->y, a->F_T, a->B * a->H, a->T, 0, a->H, a->stream);
}

int fast_impl(const srwm_fast_args_t* a)
{
    if (a == nullptr) return SRWM_ERR_NULL;
    FwpSizes s;
    int rc = fwp_sizes(a->B, a->T, a->H, 1, a->d_key, a->d_v, &s);
    if (rc != SRWM_OK) return rc;
    const int vi = find_fast(a->d_key, a->d_v, s.units);
    if (vi < 0) return SRWM_ERR_UNSUPPORTED;
    int64_t span;
    rc = time_span(a->B, a->T, a->t_stride, &span);
    if (rc != SRWM_OK) return rc;
    const int64_t P = a->d_v + 2 * a->d_key + 1;
    if (!mul_ok(span * a->H, P * 4, &s.nz) || !mul_ok(span * a->H, a->d_v * 4, &s.ny)) return SRWM_ERR_SHAPE;
    if (s.units == 0) return SRWM_OK;
    if (s.steps > 0 && (a->z == nullptr || a->y == nullptr)) return SRWM_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(a->F0) | reinterpret_cast<uintptr_t>(a->y) |
         reinterpret_cast<uintptr_t>(a->F_T)) & 15u)
        return SRWM_ERR_ARG;
    const void* ins[] = {a->z, a->F0};
    const int64_t nins[] = {s.nz, a->F0 ? s.nf : 0};
    void* outs[] = {a->y, a->F_T};
    const int64_t nouts[] = {s.ny, a->F_T ? s.nf : 0};
    for (int o = 0; o < 2; ++o)
        for (int i = 0; i < 2; ++i)
            if (ranges_overlap(outs[o], nouts[o], ins[i], nins[i])) return SRWM_ERR_ALIAS;
    if (ranges_overlap(a->y, s.ny, a->F_T, a->F_T ? s.nf : 0)) return SRWM_ERR_ALIAS;
    return launch_fast(vi, a->z, a->F0, a->y, a->F_T, s.units, a->T, a->t_stride, a->H, a->stream);
}

// Steps per chunk when SR-DeltaNet's halves overlap: about an eighth of the
// sequence, whole 32-step pieces, at least 256 steps (the fast matrix's last
// chunk is the part that cannot overlap; each chunk adds a state store and
// reload and a launch).  Only when the projection leaves room on the chip (at
// most two of its waves per SIMD over all units); else unchunked.
int64_t auto_chunk_steps(int64_t T, int64_t units, int proj_waves)
{
    if (units * proj_waves > 2048) return T;
    int64_t C = (T + 7) / 8;
    C = (C + 31) / 32 * 32;
    return C < 256 ? 256 : C;
}

// The two halves over chunks of C steps: the projection of chunk c on
// `stream`, then (after an event) the fast matrix of chunk c on aux.  The
// states carried between chunks live in W_T and F_T, read and rewritten in
// place by each chunk's kernel.
int srdeltanet_overlapped(const srwm_srdeltanet_args_t* a, const FwdPlan& plan, const srwm_forward_args_t& f,
                          int vi, int64_t units, int64_t C)
{
    const hipStream_t main_s = static_cast<hipStream_t>(a->stream);
    const hipStream_t aux_s = static_cast<hipStream_t>(a->aux_stream);
    const int64_t P = a->d_v + 2 * a->d_key + 1;
    // One event, recorded once per chunk on the caller's stream (a wait takes
    // the record made before it) and once at the end on aux.
    hipEvent_t ev;
    if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) return SRWM_ERR_HIP;
    int rc = SRWM_OK;
    bool aux_used = false;
    for (int64_t t0 = 0; t0 < a->T && rc == SRWM_OK; t0 += C) {
        const int64_t n = (a->T - t0) < C ? (a->T - t0) : C;
        srwm_forward_args_t fc = f;
        fc.x = a->x + t0 * a->H * a->d_in;
        fc.y = a->z + t0 * a->H * P;
        fc.T = n;
        fc.t_stride = a->T;
        fc.W0 = t0 == 0 ? a->W0 : a->W_T;
        fc.w0_per_sequence = t0 == 0 ? 0 : 1;
        rc = forward_launch(plan, &fc);
        if (rc != SRWM_OK) break;
        if (hipEventRecord(ev, main_s) != hipSuccess || hipStreamWaitEvent(aux_s, ev, 0) != hipSuccess) {
            rc = SRWM_ERR_HIP;
            break;
        }
        aux_used = true;
        rc = launch_fast(vi, a->z + t0 * a->H * P, t0 == 0 ? a->F0 : a->F_T, a->y + t0 * a->H * a->d_v, a->F_T,
                         units, n, a->T, a->H, a->aux_stream);
    }
    // The caller's stream waits for everything queued on aux, also after an
    // error (best effort), so no fast-matrix chunk outlives the call's stream
    // order and a captured aux stream is always joined back.
    if (aux_used) {
        const bool ok = hipEventRecord(ev, aux_s) == hipSuccess && hipStreamWaitEvent(main_s, ev, 0) == hipSuccess;
        if (!ok && rc == SRWM_OK) rc = SRWM_ERR_HIP;
    }
    (void)hipEventDestroy(ev);
    return rc;
}

int srdeltanet_impl(const srwm_srdeltanet_args_t* a)
{
    if (a == nullptr) return SRWM_ERR_NULL;
    FwpSizes s;
    int rc = fwp_sizes(a->B, a->T, a->H, a->d_in, a->d_key, a->d_v, &s);
    if (rc != SRWM_OK) return rc;
    const int vi = find_fast(a->d_key, a->d_v, s.units);
    if (vi < 0) return SRWM_ERR_UNSUPPORTED;
    const int64_t P = a->d_v + 2 * a->d_key + 1;
    if (a->n_lr != 1 && a->n_lr != 4) return SRWM_ERR_ARG;
    if (a->chunk_steps < 0) return SRWM_ERR_ARG;
    const int64_t m = P + 2 * a->d_in + a->n_lr;
    int64_t nst, nw0;
    if (!mul_ok(s.units, m * a->d_in * 4, &nst) || !mul_ok(a->H, m * a->d_in * 4, &nw0)) return SRWM_ERR_SHAPE;
    if (srwm_supported(a->d_in, P, SRWM_IO_F32, a->n_lr) != 1) return SRWM_ERR_UNSUPPORTED;
    if (s.units == 0) return SRWM_OK;
    if ((reinterpret_cast<uintptr_t>(a->F0) | reinterpret_cast<uintptr_t>(a->y) |
         reinterpret_cast<uintptr_t>(a->F_T)) & 15u)
        return SRWM_ERR_ARG;
    if (s.ny > 0 && a->y == nullptr) return SRWM_ERR_NULL;
    // the fast memory's buffers against everything else
    const void* others[] = {a->x, a->W0, a->z, a->W_T};
    const int64_t nothers[] = {s.nx, nw0, s.nz, a->W_T ? nst : 0};
    void* outs[] = {a->y, a->F_T};
    const int64_t nouts[] = {s.ny, a->F_T ? s.nf : 0};
    for (int o = 0; o < 2; ++o) {
        for (int i = 0; i < 4; ++i)
            if (ranges_overlap(outs[o], nouts[o], others[i], nothers[i])) return SRWM_ERR_ALIAS;
        if (ranges_overlap(outs[o], nouts[o], a->F0, a->F0 ? s.nf : 0)) return SRWM_ERR_ALIAS;
    }
    if (ranges_overlap(a->y, s.ny, a->F_T, a->F_T ? s.nf : 0)) return SRWM_ERR_ALIAS;
    // the SRWM half writes z and W_T before the fast matrix reads F0
    if (ranges_overlap(a->F0, a->F0 ? s.nf : 0, a->z, s.nz) ||
        ranges_overlap(a->F0, a->F0 ? s.nf : 0, a->W_T, a->W_T ? nst : 0))
        return SRWM_ERR_ALIAS;
    // the projection: the SRWM with d_out = P writes its outputs into z
    srwm_forward_args_t f;
    f.x = a->x;
    f.W0 = a->W0;
    f.y = a->z;
    f.W_T = a->W_T;
    f.B = a->B;
    f.T = a->T;
    f.H = a->H;
    f.d_in = a->d_in;
    f.d_out = P;
    f.m = m;
    f.io_dtype = SRWM_IO_F32;
    f.apply_input_softmax = a->apply_input_softmax;
    f.n_lr = a->n_lr;
    f.w0_per_sequence = 0;
    f.reset_interval = 0;
    f.variant = -1;
    f.stream = a->stream;
    f.tape = nullptr;
    f.window_states = nullptr;
    f.t_stride = 0;
    FwdPlan plan;
    rc = forward_check(&f, &plan);
    if (rc != SRWM_OK) return rc;
    const int64_t C = a->chunk_steps > 0 ? a->chunk_steps : auto_chunk_steps(a->T, s.units, plan.waves);
    if (C < a->T && a->aux_stream != nullptr && a->aux_stream != a->stream && a->W_T != nullptr &&
        a->F_T != nullptr)
        return srdeltanet_overlapped(a, plan, f, vi, s.units, C);
    if (plan.run) {
        rc = forward_launch(plan, &f);
        if (rc != SRWM_OK) return rc;
    }
    if (a->T == 0 && a->F_T == nullptr) return SRWM_OK;
    return launch_fast(vi, a->z, a->F0, a->y, a->F_T, s.units, a->T, 0, a->H, a->stream);
}

}  // namespace

extern "C" {

int srwm_deltanet_forward(const srwm_deltanet_args_t* args) { return deltanet_impl(args, false); }

int srwm_deltanet_project(const srwm_deltanet_args_t* args) { return deltanet_impl(args, true); }

int srwm_fast_forward(const srwm_fast_args_t* args) { return fast_impl(args); }

int srwm_srdeltanet_forward(const srwm_srdeltanet_args_t* args) { return srdeltanet_impl(args); }

int srwm_fwp_supported(int64_t d_key, int64_t d_v) { return find_fast(d_key, d_v) >= 0 ? 1 : 0; }

int64_t srwm_srdeltanet_chunk_steps(int64_t B, int64_t T, int64_t H, int64_t d_in, int64_t d_key, int64_t d_v,
                                    int n_lr)
{
    FwpSizes s;
    const int rc = fwp_sizes(B, T, H, d_in, d_key, d_v, &s);
    if (rc != SRWM_OK) return rc;
    if (n_lr != 1 && n_lr != 4) return SRWM_ERR_ARG;
    if (find_fast(d_key, d_v, s.units) < 0) return SRWM_ERR_UNSUPPORTED;
    const int vi = srwm_select_variant(d_in, d_v + 2 * d_key + 1, SRWM_IO_F32, n_lr, 0, s.units);
    if (vi < 0) return vi;
    srwm_variant_info_t info;
    if (srwm_variant_info(vi, &info) != SRWM_OK) return SRWM_ERR_UNSUPPORTED;
    return auto_chunk_steps(T, s.units, info.waves);
}

}  // extern "C"
