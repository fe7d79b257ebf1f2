/* A plain C99 client of the library's C ABI: includes the public header,
 * links libadaln.so and calls its host-only entry points (no GPU needed).
 * Prints one line per check; exits non-zero on the first failure. */
#include <stdio.h>
#include <string.h>

#include "adaln.h"

#define CHECK(cond)                                          \
    do {                                                     \
        if (!(cond)) {                                       \
            fprintf(stderr, "failed: %s (line %d)\n", #cond, \
                    __LINE__);                               \
            return 1;                                        \
        }                                                    \
        printf("ok: %s\n", #cond);                           \
    } while (0)

int main(void)
{
    /* bucket rule of the mixed schedule (hand-evaluated values) */
    CHECK(adaln_bshape(1560, 131072, 2200000000LL, 2) == 84);
    CHECK(adaln_bshape(32760, 131072, 2200000000LL, 2) == 2);
    CHECK(adaln_bshape(0, 1, 1, 1) == ADALN_ERR_INVALID);
    CHECK(adaln_bshape_real(16380, 131072, 8.0 * 16380.0 * 16380.0, 2.0) == 8);

    /* cost model: exact samples of t = 1 + 2e-9 * B * S^2 */
    {
        double B[6] = {1, 2, 4, 1, 2, 4};
        double S[6] = {1000, 1000, 1000, 4000, 4000, 4000};
        double t[6], out[4];
        int i;
        for (i = 0; i < 6; ++i)
            t[i] = 1.0 + 2e-9 * B[i] * S[i] * S[i];
        CHECK(adaln_costfit(B, S, t, 6, 0.5, 3.0, out) == ADALN_OK);
        CHECK(out[2] > 2.0 - 1e-6 && out[2] < 2.0 + 1e-6);
        CHECK(adaln_costfit(B, S, t, 2, 0.5, 3.0, out) == ADALN_ERR_INVALID);
    }

    /* limits, errors, workspace sizes */
    CHECK(adaln_max_d(ADALN_BF16) == 32768);
    CHECK(adaln_max_d(ADALN_F32) == 16384);
    CHECK(strlen(adaln_strerror(ADALN_ERR_ALIGN)) > 0);
    CHECK(adaln_bwd_workspace_bytes(1, 75600, 5120, ADALN_BF16) > 0);
    CHECK(adaln_bwd_workspace_bytes(2, 3, 60, ADALN_BF16) == 0);
    {
        int64_t plan[4];
        CHECK(adaln_bwd_fused_plan(1, 75600, 2048, ADALN_BF16, plan) == ADALN_OK);
        CHECK(plan[1] == 1 && plan[3] > 0);
        CHECK(adaln_bwd_fused_plan(1, 75600, 5120, ADALN_BF16, plan) == ADALN_OK);
        CHECK(plan[1] == 2 && plan[3] > 0);
        CHECK(adaln_bwd_fused_plan(1, 1000, 8192, ADALN_BF16, plan) == ADALN_OK);
        CHECK(plan[1] == 2);
    }
    {
        int64_t p[7];
        CHECK(adaln_plan(0, 1, 75600, 5120, ADALN_BF16, p) == ADALN_OK);
        CHECK(p[1] == 1 && p[2] == 75600 / 4 && p[3] == 0 && p[5] == 4 && p[6] == 0);
        CHECK(adaln_plan(1, 1, 75600, 5120, ADALN_BF16, p) == ADALN_OK);
        CHECK(p[1] == 2 && p[5] == 2);
        CHECK(adaln_plan(1, 16, 1560, 1536, ADALN_BF16, p) == ADALN_OK);
        CHECK(p[1] == 1 && p[6] == 97);
        CHECK(adaln_plan(2, 1, 75600, 5120, ADALN_BF16, p) == ADALN_OK);
        CHECK(p[0] == 32 && p[5] == 511 && p[4] == p[1] * p[2] * 64);
        CHECK(adaln_plan(3, 1, 75600, 5120, ADALN_BF16, p) == ADALN_OK);
        CHECK(p[0] == 10 && p[3] == p[0] * p[2] && p[1] * p[2] >= 75600);
        CHECK(adaln_plan(4, 1, 75600, 5120, ADALN_BF16, p) == ADALN_ERR_INVALID);
    }
    /* an invalid call enqueues nothing and explains itself */
    CHECK(adaln_fwd(NULL, NULL, NULL, NULL, NULL, NULL, 1, 1, 64, 9, NULL) ==
          ADALN_ERR_DTYPE);
    CHECK(strstr(adaln_last_error(), "dtype") != NULL);
    return 0;
}
