// srwm_fwd_table.h -- the forward kernel variant table of libsrwm.  The
// table is split into parts, each instantiated in its own translation unit
// (srwm_fwd_small.hip, srwm_fwd_d64.hip, srwm_fwd_misc.hip,
// srwm_fwd_tape.hip) so they compile in parallel; srwm_fwd.hip indexes them
// as one table, parts in the order kFwdParts lists them.
#pragma once

#include <hip/hip_runtime.h>

#include "srwm.h"
#include "srwm_fwd_kernels.h"

namespace srwm {

using KernelFn = void (*)(const void*, const float*, void*, float*, float*, float*, int, int, int, int, int, int);

struct Variant {
    int d_in, d_out, io, nw, p, wpe, nlr, fused, reset, tape, is_auto;
    KernelFn fn;
};

// SCHED: 0 phased, 1 phased with the reset ablation, 2 fused, 3 phased
// writing the backward tape, 4 phased with the reset ablation writing the
// backward tape (and the windows' end states).
template <int D_IN, int D_OUT, int NW, int P, int WPE, int NLR, int SCHED, bool BF16>
constexpr Variant make_variant(int is_auto)
{
    constexpr int io = BF16 ? SRWM_IO_BF16 : SRWM_IO_F32;
    if constexpr (SCHED == 2)
        return Variant{D_IN, D_OUT, io, NW, P, WPE, NLR, 1, 0, 0, is_auto,
                       &srwm_fwd_fused_kernel<D_IN, D_OUT, NW, P, WPE, NLR, BF16>};
    else
        return Variant{D_IN, D_OUT, io, NW, P, WPE, NLR, 0, SCHED == 1 || SCHED == 4, SCHED == 3 || SCHED == 4,
                       is_auto,
                       &srwm_fwd_kernel<D_IN, D_OUT, NW, P, WPE, NLR, SCHED == 1 || SCHED == 4,
                                        SCHED == 3 || SCHED == 4, BF16>};
}

// Both I/O dtypes of one geometry: (d_in, d_out, waves per unit, lanes per
// row, waves per SIMD the registers allow, learning rates, eligible for the
// automatic choice).  _RESET variants also implement the reset ablation.
#define SRWM_BOTH_IO(DI, DO, NW, P, WPE, NLR, AUTO)                   \
    make_variant<DI, DO, NW, P, WPE, NLR, 0, false>(AUTO),             \
        make_variant<DI, DO, NW, P, WPE, NLR, 0, true>(AUTO)
#define SRWM_BOTH_IO_RESET(DI, DO, NW, P, WPE, NLR, AUTO)             \
    make_variant<DI, DO, NW, P, WPE, NLR, 1, false>(AUTO),             \
        make_variant<DI, DO, NW, P, WPE, NLR, 1, true>(AUTO)
#define SRWM_BOTH_IO_FUSED(DI, DO, NW, P, WPE, NLR, AUTO)             \
    make_variant<DI, DO, NW, P, WPE, NLR, 2, false>(AUTO),             \
        make_variant<DI, DO, NW, P, WPE, NLR, 2, true>(AUTO)
#define SRWM_BOTH_IO_TAPE(DI, DO, NW, P, WPE, NLR, AUTO)              \
    make_variant<DI, DO, NW, P, WPE, NLR, 3, false>(AUTO),             \
        make_variant<DI, DO, NW, P, WPE, NLR, 3, true>(AUTO)
#define SRWM_BOTH_IO_TAPE_RESET(DI, DO, NW, P, WPE, NLR, AUTO)        \
    make_variant<DI, DO, NW, P, WPE, NLR, 4, false>(AUTO),             \
        make_variant<DI, DO, NW, P, WPE, NLR, 4, true>(AUTO)

// One part of the table: its variants and how many.
struct VariantPart {
    const Variant* v;
    int n;
};

VariantPart fwd_variants_small();  // d_in <= 32 (tests, latency-bound workloads)
VariantPart fwd_variants_d64();    // d_in = 64 and 128, four learning rates
VariantPart fwd_variants_misc();   // one learning rate; SR-DeltaNet's projection
VariantPart fwd_variants_tape();   // forward passes that write the backward tape

}  // namespace srwm
