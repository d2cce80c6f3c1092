/*
 * abi_driver.c -- drives every error path of libsrwm's C ABI that is decided
 * before any HIP call (NULL pointers, sizes, size overflow, unsupported
 * shapes, aliasing, alignment, flags), plus the empty problems that return
 * without a launch, against a host-only build of the library under
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py).
 * No call reaches the GPU: the pointers are never dereferenced.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "srwm.h"

static int failures = 0;

#define EXPECT(call, code)                                                                  \
    do {                                                                                    \
        const long long got_ = (long long)(call);                                           \
        if (got_ != (long long)(code)) {                                                    \
            fprintf(stderr, "%s:%d: %s returned %lld, expected %lld\n", __FILE__, __LINE__, #call, \
                    got_, (long long)(code));                                               \
            ++failures;                                                                     \
        }                                                                                   \
    } while (0)

#define P(a) ((void*)(uintptr_t)(a))
#define F(a) ((float*)(uintptr_t)(a))
static const uintptr_t X = 0x10000000, W0 = 0x20000000, Y = 0x30000000, WT = 0x40000000, TP = 0x50000000,
                       GY = 0x60000000, DX = 0x70000000, DWI = 0x80000000, DW0 = 0x90000000, Z = 0xA0000000,
                       WS = 0xB0000000;

static srwm_forward_args_t fwd_args(void)
{
    srwm_forward_args_t a;
    memset(&a, 0, sizeof a);
    a.x = P(X), a.W0 = F(W0), a.y = P(Y), a.W_T = F(WT);
    a.B = 2, a.T = 3, a.H = 2, a.d_in = 16, a.d_out = 16, a.m = 52;
    a.io_dtype = SRWM_IO_F32, a.n_lr = 4, a.variant = -1;
    return a;
}

static srwm_backward_args_t bwd_args(void)
{
    srwm_backward_args_t a;
    memset(&a, 0, sizeof a);
    a.x = P(X), a.W_T = F(WT), a.tape = F(TP), a.gy = F(GY), a.dx = F(DX), a.dW_init = F(DWI), a.dW0 = F(DW0);
    a.B = 2, a.T = 3, a.H = 2, a.d_in = 16, a.d_out = 16, a.m = 52, a.n_lr = 4;
    return a;
}

static srwm_deltanet_args_t dn_args(void)
{
    srwm_deltanet_args_t a;
    memset(&a, 0, sizeof a);
    a.x = F(X), a.W_slow = F(W0), a.z = F(Z), a.y = F(Y);
    a.B = 2, a.T = 3, a.H = 2, a.d_in = 16, a.d_key = 16, a.d_v = 16;
    return a;
}

static srwm_srdeltanet_args_t sdn_args(void)
{
    srwm_srdeltanet_args_t a;
    memset(&a, 0, sizeof a);
    a.x = F(X), a.W0 = F(W0), a.z = F(Z), a.y = F(Y);
    a.B = 2, a.T = 3, a.H = 2, a.d_in = 16, a.d_key = 16, a.d_v = 16, a.n_lr = 4;
    return a;
}

static srwm_fast_args_t fast_args(void)
{
    srwm_fast_args_t a;
    memset(&a, 0, sizeof a);
    a.z = F(Z), a.y = F(Y);
    a.B = 2, a.T = 3, a.H = 2, a.d_key = 16, a.d_v = 16;
    return a;
}

int main(void)
{
    /* srwm_forward */
    EXPECT(srwm_forward(P(X), F(W0), P(Y), F(WT), 2, 3, 2, 16, 16, 51, 0, 0, NULL), SRWM_ERR_SHAPE);
    EXPECT(srwm_forward(P(X), F(W0), P(Y), F(WT), -1, 3, 2, 16, 16, 52, 0, 0, NULL), SRWM_ERR_SHAPE);
    EXPECT(srwm_forward(P(X), F(W0), P(Y), F(WT), 2, 3, 2, 7, 7, 25, 0, 0, NULL), SRWM_ERR_UNSUPPORTED);
    EXPECT(srwm_forward(P(X), F(W0), P(Y), F(WT), 2, 3, 2, 16, 16, 52, 2, 0, NULL), SRWM_ERR_ARG);
    EXPECT(srwm_forward(P(X), F(W0), P(Y), F(WT), 2, 3, 2, 16, 16, 52, 0, 2, NULL), SRWM_ERR_ARG);
    EXPECT(srwm_forward(NULL, F(W0), P(Y), F(WT), 2, 3, 2, 16, 16, 52, 0, 0, NULL), SRWM_ERR_NULL);
    EXPECT(srwm_forward(P(X), F(W0), P(X + 64), F(WT), 2, 3, 2, 16, 16, 52, 0, 0, NULL), SRWM_ERR_ALIAS);
    EXPECT(srwm_forward(P(X), F(W0), P(Y), F(Y + 16), 2, 3, 2, 16, 16, 52, 0, 0, NULL), SRWM_ERR_ALIAS);
    EXPECT(srwm_forward(P(X + 4), F(W0), P(Y), F(WT), 2, 3, 2, 16, 16, 52, 0, 0, NULL), SRWM_ERR_ARG);
    EXPECT(srwm_forward(P(X), F(W0), P(Y), F(WT), (int64_t)1 << 40, (int64_t)1 << 40, 2, 16, 16, 52, 0, 0, NULL),
           SRWM_ERR_SHAPE);
    EXPECT(srwm_forward(P(X), F(W0), P(Y), F(WT), 1, (int64_t)1 << 31, 1, 16, 16, 52, 0, 0, NULL), SRWM_ERR_SHAPE);
    EXPECT(srwm_forward(P(X), F(W0), P(Y), F(WT), INT64_MAX, INT64_MAX, INT64_MAX, 16, 16, 52, 0, 0, NULL),
           SRWM_ERR_SHAPE);
    EXPECT(srwm_forward_variant(P(X), F(W0), P(Y), F(WT), 2, 3, 2, 16, 16, 52, 0, 0, NULL, -2), SRWM_ERR_ARG);
    EXPECT(srwm_forward_variant(P(X), F(W0), P(Y), F(WT), 2, 3, 2, 16, 16, 52, 0, 0, NULL, 1000000), SRWM_ERR_ARG);
    /* empty problems return before any HIP call */
    EXPECT(srwm_forward(NULL, F(W0), NULL, NULL, 0, 3, 2, 16, 16, 52, 0, 0, NULL), SRWM_OK);
    EXPECT(srwm_forward(NULL, NULL, NULL, NULL, 2, 3, 0, 16, 16, 52, 0, 0, NULL), SRWM_OK);
    EXPECT(srwm_forward(NULL, F(W0), NULL, NULL, 2, 0, 2, 16, 16, 52, 0, 0, NULL), SRWM_OK);

    /* srwm_forward_ex */
    EXPECT(srwm_forward_ex(NULL), SRWM_ERR_NULL);
    {
        srwm_forward_args_t a = fwd_args();
        a.t_stride = 2;
        EXPECT(srwm_forward_ex(&a), SRWM_ERR_SHAPE);
        a = fwd_args(), a.t_stride = 1000, a.y = P(X + 65536);
        EXPECT(srwm_forward_ex(&a), SRWM_ERR_ALIAS);
        a = fwd_args(), a.n_lr = 2;
        EXPECT(srwm_forward_ex(&a), SRWM_ERR_ARG);
        a = fwd_args(), a.n_lr = 1;
        EXPECT(srwm_forward_ex(&a), SRWM_ERR_SHAPE);
        a = fwd_args(), a.reset_interval = (int64_t)1 << 40;
        EXPECT(srwm_forward_ex(&a), SRWM_ERR_ARG);
        a = fwd_args(), a.W0 = NULL, a.w0_per_sequence = 1;
        EXPECT(srwm_forward_ex(&a), SRWM_ERR_NULL);
        a = fwd_args(), a.W_T = F(W0 + 8192), a.w0_per_sequence = 1;
        EXPECT(srwm_forward_ex(&a), SRWM_ERR_ALIAS);
        a = fwd_args(), a.tape = F(TP), a.reset_interval = 1;
        EXPECT(srwm_forward_ex(&a), SRWM_ERR_NULL);
        a.window_states = F(WS + 4);
        EXPECT(srwm_forward_ex(&a), SRWM_ERR_ARG);
        a.window_states = F(TP + 64);
        EXPECT(srwm_forward_ex(&a), SRWM_ERR_ALIAS);
        a = fwd_args(), a.tape = F(X + 16);
        EXPECT(srwm_forward_ex(&a), SRWM_ERR_ALIAS);
        a = fwd_args(), a.B = (int64_t)1 << 16, a.H = (int64_t)1 << 16, a.T = 1;
        EXPECT(srwm_forward_ex(&a), SRWM_ERR_SHAPE);
        a = fwd_args(), a.tape = F(TP), a.T = INT64_MAX / 2;
        EXPECT(srwm_forward_ex(&a), SRWM_ERR_SHAPE);
    }

    /* srwm_backward */
    EXPECT(srwm_backward(NULL), SRWM_ERR_NULL);
    {
        srwm_backward_args_t a = bwd_args();
        a.n_lr = 2;
        EXPECT(srwm_backward(&a), SRWM_ERR_ARG);
        a = bwd_args(), a.m = 51;
        EXPECT(srwm_backward(&a), SRWM_ERR_SHAPE);
        a = bwd_args(), a.d_in = 32, a.d_out = 32, a.m = 100;
        EXPECT(srwm_backward(&a), SRWM_ERR_UNSUPPORTED);
        a = bwd_args(), a.dW_init = NULL;
        EXPECT(srwm_backward(&a), SRWM_ERR_NULL);
        a = bwd_args(), a.dx = F(DX + 8);
        EXPECT(srwm_backward(&a), SRWM_ERR_ARG);
        a = bwd_args(), a.dx = F(GY);
        EXPECT(srwm_backward(&a), SRWM_ERR_ALIAS);
        a = bwd_args(), a.dW0 = F(DWI + 16);
        EXPECT(srwm_backward(&a), SRWM_ERR_ALIAS);
        a = bwd_args(), a.reset_interval = 1;
        EXPECT(srwm_backward(&a), SRWM_ERR_NULL);
        a.window_states = F(DWI);
        EXPECT(srwm_backward(&a), SRWM_ERR_ALIAS);
        a = bwd_args(), a.B = (int64_t)1 << 31, a.H = 1, a.T = 1;
        EXPECT(srwm_backward(&a), SRWM_ERR_SHAPE);
        a = bwd_args(), a.T = INT64_MAX / 3;
        EXPECT(srwm_backward(&a), SRWM_ERR_SHAPE);
        /* empty: no launch when there is no dW0 to clear */
        a = bwd_args(), a.B = 0, a.x = NULL, a.W_T = NULL, a.tape = NULL, a.gy = NULL, a.dx = NULL,
        a.dW_init = NULL, a.dW0 = NULL;
        EXPECT(srwm_backward(&a), SRWM_OK);
    }

    /* srwm_backward_noalloc: validation before any HIP call */
    {
        srwm_backward_args_t a = bwd_args();
        a.dW_init = NULL;
        EXPECT(srwm_backward_noalloc(NULL), SRWM_ERR_NULL);
        a.dW_init = F(DWI);
        EXPECT(srwm_backward_noalloc(&a), SRWM_ERR_ARG);
        a.dW_init = NULL, a.dW0 = NULL;
        EXPECT(srwm_backward_noalloc(&a), SRWM_ERR_NULL);
        a = bwd_args(), a.dW_init = NULL, a.H = 170, a.d_in = 128, a.d_out = 128, a.m = 388;
        EXPECT(srwm_backward_noalloc(&a), SRWM_ERR_SCRATCH);
        a = bwd_args(), a.dW_init = NULL, a.B = INT64_MAX / 2;
        EXPECT(srwm_backward_noalloc(&a), SRWM_ERR_SHAPE);
        a = bwd_args(), a.dW_init = NULL, a.H = 0;
        EXPECT(srwm_backward_noalloc(&a), SRWM_OK);
        EXPECT(srwm_backward_noalloc_scratch_bytes(), (int64_t)32 << 20);
    }

    /* DeltaNet, SR-DeltaNet, the fast matrix alone */
    {
        srwm_deltanet_args_t a = dn_args();
        EXPECT(srwm_deltanet_forward(NULL), SRWM_ERR_NULL);
        a.d_key = 7, a.d_v = 7;
        EXPECT(srwm_deltanet_forward(&a), SRWM_ERR_UNSUPPORTED);
        a = dn_args(), a.H = 1, a.d_in = 3;
        EXPECT(srwm_deltanet_forward(&a), SRWM_ERR_SHAPE);
        a = dn_args(), a.z = NULL;
        EXPECT(srwm_deltanet_forward(&a), SRWM_ERR_NULL);
        a = dn_args(), a.y = F(Y + 4);
        EXPECT(srwm_deltanet_forward(&a), SRWM_ERR_ARG);
        a = dn_args(), a.z = F(X + 16);
        EXPECT(srwm_deltanet_forward(&a), SRWM_ERR_ALIAS);
        a = dn_args(), a.B = (int64_t)1 << 31, a.H = 1;
        EXPECT(srwm_deltanet_forward(&a), SRWM_ERR_SHAPE);
        a = dn_args(), a.z = NULL;
        EXPECT(srwm_deltanet_project(&a), SRWM_ERR_NULL);
        a = dn_args(), a.z = F(W0 + 16);
        EXPECT(srwm_deltanet_project(&a), SRWM_ERR_ALIAS);
        a = dn_args(), a.B = 0, a.x = NULL, a.z = NULL, a.y = NULL;
        EXPECT(srwm_deltanet_forward(&a), SRWM_OK);
    }
    {
        srwm_srdeltanet_args_t a = sdn_args();
        EXPECT(srwm_srdeltanet_forward(NULL), SRWM_ERR_NULL);
        a.n_lr = 2;
        EXPECT(srwm_srdeltanet_forward(&a), SRWM_ERR_ARG);
        a = sdn_args(), a.d_in = 8;
        EXPECT(srwm_srdeltanet_forward(&a), SRWM_ERR_UNSUPPORTED);
        a = sdn_args(), a.y = F(Z + 64);
        EXPECT(srwm_srdeltanet_forward(&a), SRWM_ERR_ALIAS);
        a = sdn_args(), a.F0 = F(Z + 16);
        EXPECT(srwm_srdeltanet_forward(&a), SRWM_ERR_ALIAS);
        a = sdn_args(), a.F0 = F(WT), a.W_T = F(WT);
        EXPECT(srwm_srdeltanet_forward(&a), SRWM_ERR_ALIAS);
        a = sdn_args(), a.chunk_steps = -1;
        EXPECT(srwm_srdeltanet_forward(&a), SRWM_ERR_ARG);
        a = sdn_args(), a.H = 0, a.x = NULL, a.z = NULL, a.y = NULL, a.W0 = NULL;
        EXPECT(srwm_srdeltanet_forward(&a), SRWM_OK);
        EXPECT(srwm_srdeltanet_chunk_steps(128, 4096, 2, 64, 64, 64, 4), 512);
        EXPECT(srwm_srdeltanet_chunk_steps(2, 3, 2, 16, 16, 16, 2), SRWM_ERR_ARG);
        EXPECT(srwm_srdeltanet_chunk_steps(-1, 3, 2, 16, 16, 16, 4), SRWM_ERR_SHAPE);
        EXPECT(srwm_srdeltanet_chunk_steps(INT64_MAX, INT64_MAX, 2, 16, 16, 16, 4), SRWM_ERR_SHAPE);
    }
    {
        srwm_fast_args_t a = fast_args();
        EXPECT(srwm_fast_forward(NULL), SRWM_ERR_NULL);
        a.y = F(Z + 32);
        EXPECT(srwm_fast_forward(&a), SRWM_ERR_ALIAS);
        a = fast_args(), a.t_stride = 1000, a.y = F(Z + 65536);
        EXPECT(srwm_fast_forward(&a), SRWM_ERR_ALIAS);
        a = fast_args(), a.T = (int64_t)1 << 31, a.B = 1, a.H = 1;
        EXPECT(srwm_fast_forward(&a), SRWM_ERR_SHAPE);
        a = fast_args(), a.d_key = 7;
        EXPECT(srwm_fast_forward(&a), SRWM_ERR_UNSUPPORTED);
    }

    /* queries */
    {
        const int n = srwm_variant_count();
        srwm_variant_info_t info;
        srwm_kernel_resources_t r;
        if (n < 1) ++failures;
        for (int i = 0; i < n; ++i) EXPECT(srwm_variant_info(i, &info), SRWM_OK);
        EXPECT(srwm_variant_info(n, &info), SRWM_ERR_ARG);
        EXPECT(srwm_variant_info(0, NULL), SRWM_ERR_NULL);
        EXPECT(srwm_variant_resources(-1, &r), SRWM_ERR_ARG);
        EXPECT(srwm_variant_resources(0, NULL), SRWM_ERR_NULL);
        EXPECT(srwm_backward_resources(64, 64, 2, 0, 1, &r), SRWM_ERR_ARG);
        EXPECT(srwm_backward_resources(32, 32, 4, 0, 1, &r), SRWM_ERR_UNSUPPORTED);
        EXPECT(srwm_select_variant(7, 7, 0, 4, 0, 4), SRWM_ERR_UNSUPPORTED);
        EXPECT(srwm_select_variant(0, 64, 0, 4, 0, 4), SRWM_ERR_SHAPE);
        EXPECT(srwm_supported(64, 64, SRWM_IO_BF16, 4), 1);
        EXPECT(srwm_backward_supported(32, 32, 0, 4), 0);
        EXPECT(srwm_fwp_supported(7, 7), 0);
        EXPECT(srwm_tape_row(0, 8, 4), SRWM_ERR_SHAPE);
        EXPECT(srwm_tape_row(64, 64, 4), 196 + 3 * 64 + 4);
        EXPECT(srwm_valu_probe(NULL, 4, 1, NULL), SRWM_ERR_NULL);
        EXPECT(srwm_lds_probe(NULL, 4, 1, NULL), SRWM_ERR_NULL);
        EXPECT(srwm_lds_probe((unsigned*)(uintptr_t)(Y + 4), 4, 1, NULL), SRWM_ERR_ARG);
        for (int c = 0; c >= -9; --c)
            if (srwm_strerror(c) == NULL) ++failures;
        if (srwm_version() <= 0) ++failures;
    }
    if (failures) {
        fprintf(stderr, "abi_driver: %d failures\n", failures);
        return 1;
    }
    printf("abi_driver: ok\n");
    return 0;
}
