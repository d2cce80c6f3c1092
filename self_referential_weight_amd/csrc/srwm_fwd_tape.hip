// srwm_fwd_tape.hip -- part of libsrwm's forward variant table:
// forward passes that also write the backward tape.
// The kernels are in srwm_fwd_kernels.h; srwm_fwd.hip holds the C ABI and
// indexes the parts as one table.
#include "srwm_fwd_table.h"

namespace srwm {

namespace {
const Variant kPart[] = {
    // forward passes that also write the backward tape
    SRWM_BOTH_IO_TAPE(8, 8, 1, 8, 1, 4, 1),
    SRWM_BOTH_IO_TAPE(16, 16, 1, 4, 1, 4, 1),
    SRWM_BOTH_IO_TAPE(64, 64, 1, 2, 2, 4, 1),
    SRWM_BOTH_IO_TAPE(64, 64, 2, 8, 2, 4, 0),
    SRWM_BOTH_IO_TAPE(64, 64, 4, 8, 1, 4, 0),
    SRWM_BOTH_IO_TAPE(64, 64, 4, 4, 1, 4, 1),
    SRWM_BOTH_IO_TAPE(64, 64, 8, 8, 1, 4, 1),
    SRWM_BOTH_IO_TAPE(8, 8, 1, 8, 1, 1, 1),
    SRWM_BOTH_IO_TAPE(16, 16, 1, 4, 1, 1, 1),
    SRWM_BOTH_IO_TAPE(64, 64, 1, 2, 2, 1, 1),
    SRWM_BOTH_IO_TAPE(64, 64, 2, 8, 2, 1, 0),
    SRWM_BOTH_IO_TAPE(64, 64, 4, 8, 1, 1, 0),
    SRWM_BOTH_IO_TAPE(64, 64, 4, 4, 1, 1, 1),
    SRWM_BOTH_IO_TAPE(64, 64, 8, 8, 1, 1, 1),
    SRWM_BOTH_IO_TAPE(128, 128, 8, 4, 1, 4, 1),
    SRWM_BOTH_IO_TAPE(128, 128, 8, 4, 1, 1, 1),
    // ... with the reset ablation (they also record each window's end state)
    SRWM_BOTH_IO_TAPE_RESET(8, 8, 1, 8, 1, 4, 1),
    SRWM_BOTH_IO_TAPE_RESET(16, 16, 1, 4, 1, 4, 1),
    SRWM_BOTH_IO_TAPE_RESET(64, 64, 1, 4, 2, 4, 1),
    SRWM_BOTH_IO_TAPE_RESET(64, 64, 4, 4, 1, 4, 1),
    SRWM_BOTH_IO_TAPE_RESET(64, 64, 8, 8, 1, 4, 1),
    SRWM_BOTH_IO_TAPE_RESET(8, 8, 1, 8, 1, 1, 1),
    SRWM_BOTH_IO_TAPE_RESET(16, 16, 1, 4, 1, 1, 1),
    SRWM_BOTH_IO_TAPE_RESET(64, 64, 1, 4, 2, 1, 1),
    SRWM_BOTH_IO_TAPE_RESET(64, 64, 4, 4, 1, 1, 1),
    SRWM_BOTH_IO_TAPE_RESET(64, 64, 8, 8, 1, 1, 1),
};
}  // namespace

VariantPart fwd_variants_tape() { return VariantPart{kPart, static_cast<int>(sizeof(kPart) / sizeof(kPart[0]))}; }

}  // namespace srwm
