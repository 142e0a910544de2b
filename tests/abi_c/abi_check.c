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
    /* LNCC windows 13..31 need the larger workspace; the slab backward with
     * the MI gradient needs F and the stored W */
    if (ngv_lncc_loss_fwd_bwd((const float *)16, (const float *)16, &d, 13, 1e-5f, 1.0f, (double *)16, NULL, 0,
                              (void *)256, ws, NULL) != NGV_EWORKSPACE)
        ++fails;
    if (ngv_workspace_bytes(0, 31) <= ngv_workspace_bytes(0, 13)) ++fails;
    if (ngv_warp_bwd_adam_slab_mi(NULL, &d, NULL, NULL, &d, &xf, NULL, NULL, NULL, 32, 0.0f, 1.0f, 0.0f, 1.0f, 1.0f,
                                  NULL, NULL, NULL, 1, NULL, 0.1f, 0.9f, 0.999f, 1e-8f, NULL, NULL, 0, NULL, 0,
                                  NULL) != NGV_EINVAL)
        ++fails;
    /* every entry point of the header links */
    {
        typedef void (*entry_fn)(void);
        const entry_fn entry[] = {
            (entry_fn)ngv_workspace_bytes,
            (entry_fn)ngv_status_str,
            (entry_fn)ngv_warp_fwd,
            (entry_fn)ngv_warp_fwd_slab,
            (entry_fn)ngv_warp_bwd,
            (entry_fn)ngv_mi_loss_fwd_bwd,
            (entry_fn)ngv_mi_loss_fwd_bwd_noalloc,
            (entry_fn)ngv_mi_loss_fwd_bwd_order,
            (entry_fn)ngv_lncc_loss_fwd_bwd,
            (entry_fn)ngv_adam_step,
            (entry_fn)ngv_warp_bwd_adam,
            (entry_fn)ngv_warp_bwd_adam_slab,
            (entry_fn)ngv_warp_bwd_adam_slab_mi,
            (entry_fn)ngv_warp_bwd_adam_mi,
            (entry_fn)ngv_warp_fwd_mi,
            (entry_fn)ngv_warp_lncc_mi_bwd,
            (entry_fn)ngv_mi_grad,
            (entry_fn)ngv_warp_zrange,
            (entry_fn)ngv_mse_loss_fwd_bwd,
            (entry_fn)ngv_warp_compose};
        for (size_t i = 0; i < sizeof entry / sizeof entry[0]; ++i)
            if (!entry[i]) ++fails;
    }
    printf(fails ? "abi check FAILED (%d)\n" : "abi check ok\n", fails);
    return fails ? 1 : 0;
}
