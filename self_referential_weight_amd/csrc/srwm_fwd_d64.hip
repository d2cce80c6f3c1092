// srwm_fwd_d64.hip -- part of libsrwm's forward variant table:
// d_in = 64 and 128 with four learning rates.
// The kernels are in srwm_fwd_kernels.h; srwm_fwd.hip holds the C ABI and
// indexes the parts as one table.
#include "srwm_fwd_table.h"

namespace srwm {

namespace {
const Variant kPart[] = {
    // d = 64: one wave per unit for many units, up to eight for few
    SRWM_BOTH_IO(64, 64, 1, 2, 2, 4, 1),
    SRWM_BOTH_IO(64, 64, 2, 8, 2, 4, 0),
    SRWM_BOTH_IO_FUSED(64, 64, 4, 8, 1, 4, 0),
    SRWM_BOTH_IO_FUSED(64, 64, 8, 8, 1, 4, 0),
    SRWM_BOTH_IO(64, 64, 1, 4, 2, 4, 0),
    SRWM_BOTH_IO(64, 64, 1, 4, 1, 4, 0),
    SRWM_BOTH_IO(64, 64, 4, 8, 1, 4, 0),
    SRWM_BOTH_IO(64, 64, 4, 16, 1, 4, 0),
    SRWM_BOTH_IO(64, 64, 4, 4, 1, 4, 1),
    SRWM_BOTH_IO(64, 64, 8, 8, 1, 4, 1),
    SRWM_BOTH_IO_FUSED(64, 64, 4, 4, 1, 4, 0),
    SRWM_BOTH_IO_RESET(64, 64, 2, 8, 2, 4, 1),
    // d = 128
    SRWM_BOTH_IO(128, 128, 8, 4, 1, 4, 1),
    SRWM_BOTH_IO(128, 128, 8, 8, 1, 4, 0),
    SRWM_BOTH_IO_FUSED(128, 128, 8, 8, 1, 4, 0),
    SRWM_BOTH_IO_FUSED(128, 128, 8, 16, 1, 4, 0),
    SRWM_BOTH_IO_FUSED(128, 128, 16, 16, 1, 4, 0),
    SRWM_BOTH_IO(128, 128, 8, 16, 1, 4, 0),
    SRWM_BOTH_IO(128, 128, 16, 16, 1, 4, 0),
    SRWM_BOTH_IO(128, 128, 16, 8, 1, 4, 0),
    SRWM_BOTH_IO_RESET(128, 128, 8, 4, 1, 4, 1),
};
}  // namespace

VariantPart fwd_variants_d64() { return VariantPart{kPart, static_cast<int>(sizeof(kPart) / sizeof(kPart[0]))}; }

}  // namespace srwm
