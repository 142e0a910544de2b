/* A C99 program against include/ngv.h and libngv.so: the header compiles as
 * C, the entry points link, and calls that need no device (the workspace
 * size, status strings, argument checks) behave as documented. */
#include <stdio.h>
#include <string.h>

#include "ngv.h"

int main(void) {
    ngv_dims d = {8, 8, 8}, bad = {8, 0, 8};
    ngv_xform xf;
    size_t ws = ngv_workspace_bytes(32, 9);
    int fails = 0;
    memset(&xf, 0, sizeof xf);
    if (ws == 0 || ws % 256 != 0 || ws != ngv_workspace_bytes(32, 0)) {
        printf("workspace size %zu\n", ws);
        ++fails;
    }
    if (strcmp(ngv_status_str(NGV_OK), "ok") != 0) ++fails;
    /* argument checks come before any device work */
    if (ngv_warp_fwd(NULL, &d, NULL, NULL, &d, &xf, NULL, 0, NULL) != NGV_EINVAL) ++fails;
    if (ngv_mse_loss_fwd_bwd((const float *)16, (const float *)16, &bad, 1.0f, (double *)16, NULL, 0, NULL, 0,
                             NULL) != NGV_EINVAL)
        ++fails;
    if (ngv_adam_step((float *)16, (const float *)16, (float *)16, (float *)16, &d, 0, NULL, 0.1f, 0.9f, 0.999f,
                      1e-8f, 0.0f, NULL, 0, NULL) != NGV_EINVAL)
        ++fails;
    printf(fails ? "abi check FAILED (%d)\n" : "abi check ok\n", fails);
    return fails ? 1 : 0;
}
