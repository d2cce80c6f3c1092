// srwm_fwd_misc.hip -- part of libsrwm's forward variant table:
// one learning rate, and SR-DeltaNet's projection (d_out = d_v + 2*d_key + 1).
// The kernels are in srwm_fwd_kernels.h; srwm_fwd.hip holds the C ABI and
// indexes the parts as one table.
#include "srwm_fwd_table.h"

namespace srwm {

namespace {
const Variant kPart[] = {
    // one learning rate
    SRWM_BOTH_IO_RESET(2, 2, 1, 2, 1, 1, 1),
    SRWM_BOTH_IO_RESET(8, 8, 1, 8, 1, 1, 1),
    SRWM_BOTH_IO_RESET(16, 16, 1, 4, 1, 1, 1),
    SRWM_BOTH_IO(64, 64, 1, 2, 2, 1, 1),
    SRWM_BOTH_IO_RESET(64, 64, 2, 8, 2, 1, 1),
    SRWM_BOTH_IO(64, 64, 4, 4, 1, 1, 1),
    SRWM_BOTH_IO(64, 64, 8, 8, 1, 1, 1),
    SRWM_BOTH_IO_FUSED(64, 64, 8, 8, 1, 1, 0),
    SRWM_BOTH_IO(128, 128, 8, 4, 1, 1, 1),
    SRWM_BOTH_IO_FUSED(128, 128, 8, 8, 1, 1, 0),
    SRWM_BOTH_IO_RESET(128, 128, 8, 4, 1, 1, 1),
    // SR-DeltaNet's projection: d_out = d_v + 2*d_key + 1 (float32 I/O)
    make_variant<8, 25, 1, 8, 1, 4, 1, false>(1),
    make_variant<8, 25, 1, 8, 1, 1, 1, false>(1),
    make_variant<16, 49, 1, 4, 1, 4, 1, false>(1),
    make_variant<16, 49, 1, 4, 1, 1, 1, false>(1),
    make_variant<64, 193, 4, 4, 1, 4, 1, false>(1),
    make_variant<64, 193, 4, 4, 1, 1, 1, false>(1),
    make_variant<64, 193, 8, 4, 1, 4, 0, false>(1),
    make_variant<64, 193, 8, 4, 1, 1, 0, false>(1),
    make_variant<64, 193, 8, 8, 1, 4, 0, false>(0),
    make_variant<64, 193, 8, 8, 1, 4, 2, false>(0),
};
}  // namespace

VariantPart fwd_variants_misc() { return VariantPart{kPart, static_cast<int>(sizeof(kPart) / sizeof(kPart[0]))}; }

}  // namespace srwm
