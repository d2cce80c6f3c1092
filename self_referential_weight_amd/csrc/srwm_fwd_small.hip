// srwm_fwd_small.hip -- part of libsrwm's forward variant table:
// d_in <= 32 (the test shapes and the latency-bound small workloads).
// The kernels are in srwm_fwd_kernels.h; srwm_fwd.hip holds the C ABI and
// indexes the parts as one table.
#include "srwm_fwd_table.h"

namespace srwm {

namespace {
const Variant kPart[] = {
    // small shapes (tests, latency-bound workloads)
    SRWM_BOTH_IO_RESET(2, 2, 1, 2, 1, 4, 1),
    SRWM_BOTH_IO_RESET(3, 5, 1, 1, 1, 4, 1),
    SRWM_BOTH_IO_RESET(8, 8, 1, 8, 1, 4, 1),
    SRWM_BOTH_IO_RESET(8, 16, 1, 8, 1, 4, 1),
    SRWM_BOTH_IO_RESET(16, 8, 1, 8, 1, 4, 1),
    SRWM_BOTH_IO_RESET(16, 16, 1, 4, 1, 4, 1),
    SRWM_BOTH_IO_FUSED(16, 16, 2, 4, 1, 4, 0),
    SRWM_BOTH_IO_RESET(32, 32, 1, 4, 1, 4, 1),
};
}  // namespace

VariantPart fwd_variants_small() { return VariantPart{kPart, static_cast<int>(sizeof(kPart) / sizeof(kPart[0]))}; }

}  // namespace srwm
