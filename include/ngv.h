/*
 * ngv.h -- C ABI of libngv.so: one optimisation step of affine + deformable
 * image registration on one AMD Instinct MI355X (gfx950), as HIP kernels.
 *
 * The operations follow the papernotes.org summary page "A Scalable
 * Distributed Framework for Multimodal GigaVoxel Image Registration"
 * (ICLR 2026): the objective L(phi) = C(F, M o phi) + R(phi) with
 * phi(x) = A x + t + u(x) (section "Background"), the composite implicit grid
 * sampler (Key design 1), the Parzen-window Mattes MI and the fused LNCC
 * (Key design 2), partial-sum interpolation over image shards (Key design 4)
 * and the optimiser step with states m1, m2 (method overview).
 *
 * Conventions for every call
 *   - Volumes are fp32, dense, x fastest: index (z*ny + y)*nx + x.
 *   - Vector fields (u, gu) are three such volumes back to back: components
 *     x, y, z, each of nx*ny*nz floats (structure of arrays).
 *   - Coordinates are normalised per axis to [-1, 1], with the centres of the
 *     end voxels at -1 and +1 (align_corners=True). A acts on (x, y, z).
 *   - Every pointer named as device memory is caller-owned device memory on
 *     the current HIP device; structs are host memory read during the call.
 *     The library keeps no pointer after a call returns.
 *   - stream: a hipStream_t (NULL: the null stream). Calls only enqueue work;
 *     results (including the fp64 scalars) are ready when the stream is.
 *   - accumulate = 0 overwrites the outputs, 1 adds to them.
 *   - Workspace: device memory of at least ngv_workspace_bytes(bins, win)
 *     bytes, aligned to 256 bytes, whose size does not depend on the volume
 *     size (the page's O(1) extra memory). A workspace may be reused by
 *     calls that run in order on one stream, never by concurrent calls.
 *   - Errors: arguments are checked before any work is enqueued. On failure a
 *     negative NGV_E* code is returned and nothing is written. A HIP launch
 *     error returns NGV_EHIP; ngv_status_str gives the text.
 */
#ifndef NGV_H
#define NGV_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define NGV_API __attribute__((visibility("default")))
#else
#define NGV_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Grid size: x fastest, z slowest. Every extent must be >= 1 (and at most
 * 2^31, with at most 2^62 voxels; else NGV_EINVAL). Calls that run the
 * sampler (every ngv_warp_* call) take extents of at most 2^30 in both grids
 * and moving-image planes (md->nx * md->ny) of fewer than 2^31 voxels, and
 * return NGV_EUNSUPPORTED beyond that: their index arithmetic is 32-bit. */
typedef struct ngv_dims {
    int64_t nx, ny, nz;
} ngv_dims;

/* Parameters of the composite map p(x) = A x + t + S u(x) (Key design 1).
 * A, S: row-major 3x3; t: 3; the output grid is the implicit identity grid
 * with x_bounds = (xmin, xmax) per axis, i.e. output voxel i sits at
 * x_k = xmin_k + i_k (xmax_k - xmin_k) / (n_k - 1). S rescales u into the
 * frame of the image (identity for a whole image). */
typedef struct ngv_xform {
    float A[9];
    float t[3];
    float S[9];
    float xmin[3];
    float xmax[3];
} ngv_xform;

/* Planes [z0, z0 + nz) of the moving image held by a buffer (Key design 4:
 * a shard contributes the interpolation corners it holds, zero for the rest;
 * summing the partial results over shards that cover the volume gives the
 * whole). {0, md->nz} is the whole image.
 * zrange: NULL, or a device pointer to two doubles [lo, hi] bounding the
 * z-component of S u in M's voxel units over the output grid, as written by
 * ngv_warp_zrange for the same u, md and xf. With it a call skips the output
 * voxels whose sample provably has no corner in the slab (they contribute
 * zero); the result is the same. A bound that does not hold gives wrong
 * results: compute it from the u the call reads. */
typedef struct ngv_slab {
    int64_t z0, nz;
    const double *zrange;
} ngv_slab;

enum {
    NGV_OK = 0,
    NGV_EINVAL = -1,      /* bad argument: null pointer, size, window, bins, slab */
    NGV_EWORKSPACE = -2,  /* workspace missing, too small or misaligned */
    NGV_EHIP = -3,        /* HIP runtime or launch error */
    NGV_EUNSUPPORTED = -4 /* valid request outside what the kernels implement */
};

/* Workspace bytes for calls with these MI bins and LNCC window (either may be
 * 0 when unused). The same for every volume size: about 0.3 MB for windows
 * up to 11; windows 13..31 add per-block state that grows with the window
 * (about 36 MB at 13, 155 MB at 31). */
NGV_API size_t ngv_workspace_bytes(int bins, int win);

/* Composite implicit grid sampler, forward (Key design 1; partial sums, Key
 * design 4): W(i) = sum over the 8 trilinear corners c of w_c(p) M[c], with
 * p the sample position of A x_i + t + S u(i) in M's voxel grid, corners
 * outside the moving grid or outside the slab counted as zero.
 *   M   device, md->nx * md->ny * slab->nz floats: planes [z0, z0+nz) of M
 *   md  full moving grid size;  slab NULL = whole image
 *   u   device, 3 * od volume floats (normalised units)
 *   od  output grid size;  xf host parameters
 *   W   device, od volume floats (written, or added to with accumulate = 1)
 * No workspace. */
NGV_API int ngv_warp_fwd(const float *M, const ngv_dims *md, const ngv_slab *slab, const float *u,
                 const ngv_dims *od, const ngv_xform *xf, float *W, int accumulate, void *stream);

/* The sampler forward for a moving image held in z-slabs, as a sequence of
 * calls (Key design 4: the partial sums of the shards add up to the whole).
 * Call it once per slab, in increasing z, the slabs covering [0, md->nz)
 * without gaps, each call with the same u, xf and z-range bound
 * (slab->zrange from ngv_warp_zrange, required). The first slab that reaches
 * an output voxel writes its part of W, later slabs add theirs, and the top
 * slab's call writes zero to the voxels that no slab reaches. After the last
 * call W is, bit for bit, what zeroing W and calling ngv_warp_fwd with
 * accumulate = 1 on every slab gives, without the zeroing pass (where a
 * voxel's sum starts, what W held is read and discarded).
 *   M, md, slab, u, od, xf  as in ngv_warp_fwd
 *   W   device, od volume floats: no initialisation needed before the first
 *       call; complete after the last
 * The z-range bound decides which slabs reach a voxel (conservatively), the
 * same way in every call. No workspace. */
NGV_API int ngv_warp_fwd_slab(const float *M, const ngv_dims *md, const ngv_slab *slab, const float *u,
                              const ngv_dims *od, const ngv_xform *xf, float *W, void *stream);

/* Sampler backward (Key design 1: gradients to u and to the affine part; none
 * to M). With gW = dL/dW and g_p = dL/dp:
 *   gu = S^T g_p (3 fields),  gA9[j*3+k] = sum_i g_p,j(i) x_k(i),  gt3 = sum_i g_p(i).
 * The derivative of the trilinear form is taken in the floor cell of p (a
 * forward difference at exact lattice positions).
 *   gW  device, od volume floats;  gu device, 3 * od volume floats
 *   gA9 device, 9 doubles;  gt3 device, 3 doubles (fp64 sums)
 * Slab and accumulate as in ngv_warp_fwd; summing over slabs gives the whole. */
NGV_API int ngv_warp_bwd(const float *M, const ngv_dims *md, const ngv_slab *slab, const float *u,
                 const ngv_dims *od, const ngv_xform *xf, const float *gW, float *gu, double *gA9,
                 double *gt3, int accumulate, void *ws, size_t ws_bytes, void *stream);

/* Mattes MI loss and gradient (Key design 2; shard merge, Key design 5).
 * Parzen estimate with the cubic B-spline kernel on bins x bins joint bins:
 * intensities are clamped to [fmin, fmax] / [wmin, wmax] and mapped to bin
 * coordinate 2 + (v - vmin)(bins - 5)/(vmax - vmin), so that the kernel mass of
 * every sample lies inside the bins. p = H / N, marginals are row and column
 * sums, MI = sum_{p>0} p ln(p / (p_F p_W)).
 *   loss  device, 1 double: weight * (-MI)
 *   gW    device, volume floats, d loss / d W (NULL: loss only; the
 *         log-ratio table stays in the workspace for ngv_mi_grad or
 *         ngv_warp_bwd_adam_mi); the clamp passes the gradient for
 *         wmin <= W <= wmax, zero outside
 *   bins  8..256 (NGV_EINVAL outside).
 * Volume: fewer than 2^32 voxels, else NGV_EUNSUPPORTED (the histogram holds
 * each bin in 32.32 fixed point in 64 bits, and its entries sum to N * 2^32).
 * Precision: each GPU lane first sums the 4 x 4 weight blocks of up to 64 of
 * its samples in fp32 registers; these partial sums are rounded to 32.32
 * fixed point (or, where a wave's lanes share their bins, summed over the
 * wave's 64 lanes in fp32 first), and everything after that is exact integer
 * addition. So a histogram entry carries the rounding of at most 4096 fp32
 * additions, and the result is bitwise the same on every run for a given
 * device and volume shape, whatever the order of the merges. */
NGV_API int ngv_mi_loss_fwd_bwd(const float *F, const float *W, const ngv_dims *d, int bins, float fmin,
                        float fmax, float wmin, float wmax, float weight, double *loss, float *gW,
                        int accumulate, void *ws, size_t ws_bytes, void *stream);

/* ngv_mi_loss_fwd_bwd without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. The call itself allocates and frees nothing. Its
 * scratch (the joint histogram and the log-ratio table) is a fixed array of
 * 196608 bytes in the library's device memory, one copy per GPU, created with
 * the library's code object and held until the process ends.
 *   bins  8..128 (NGV_EUNSUPPORTED above 128, NGV_EINVAL outside 8..256);
 *         every other argument and result as in ngv_mi_loss_fwd_bwd.
 * Every call on one GPU uses that GPU's one copy, which keeps the last call's
 * contents (the histogram is cleared at the start of each call): calls on one
 * GPU must run in order (one stream, or streams ordered by events); calls
 * that overlap on one GPU race and give wrong results. The log-ratio table it
 * leaves is in that array, not in any workspace, so ngv_mi_grad and
 * ngv_warp_bwd_adam_mi cannot follow it. */
NGV_API int ngv_mi_loss_fwd_bwd_noalloc(const float *F, const float *W, const ngv_dims *d, int bins, float fmin,
                                        float fmax, float wmin, float wmax, float weight, double *loss, float *gW,
                                        int accumulate, void *stream);

/* The same MI with a choice of the fixed image's Parzen kernel (section
 * "Background and motivation": Mattes mutual information): fixed_order = 3 is
 * ngv_mi_loss_fwd_bwd (one cubic B-spline for both images); fixed_order = 0
 * is the pair of Mattes et al.'s original estimator, the zero-order (box)
 * kernel on F and the cubic B-spline on W: each sample falls with weight 1 in
 * the one F bin a with a - c in (-1/2, 1/2], i.e. floor(c + 1/2) of its bin
 * coordinate c, so a sample exactly half way between two bin centres goes to
 * the upper one. The kernels form c in fp32 (within about 5e-6 bin of its
 * exact value), so a sample that close to such an edge may fall on either
 * side. The gradient still flows only through W's cubic kernel. Other
 * orders: NGV_EINVAL. Arguments otherwise as in ngv_mi_loss_fwd_bwd. */
NGV_API int ngv_mi_loss_fwd_bwd_order(const float *F, const float *W, const ngv_dims *d, int bins,
                                      int fixed_order, float fmin, float fmax, float wmin, float wmax,
                                      float weight, double *loss, float *gW, int accumulate, void *ws,
                                      size_t ws_bytes, void *stream);

/* LNCC loss and gradient (Key design 2): window sums s_F, s_W, s_FF, s_WW,
 * s_FW of the five moment images over the win^3 cube centred on each voxel
 * (zero padding, n = win^3), cross = s_FW - s_F s_W / n, v_F = s_FF - s_F^2/n,
 * v_W = s_WW - s_W^2/n, cc = cross^2 / (v_F v_W + eps),
 *   loss = weight * (-(1/N) sum_x cc(x)),  gW = d loss / d W.
 * Window sums are fp64. For windows 3..11 all intermediates stay on chip;
 * for 13..31 (a tile halo too wide for one block's registers and LDS) a
 * slower kernel keeps its running sums in the workspace, whose size depends
 * on the window but not on the volume: O(1) extra memory either way.
 *   win  odd, 3..31 (NGV_EINVAL otherwise)
 *   loss device 1 double;  gW device volume floats (NULL: loss only).
 *   ws   at least ngv_workspace_bytes(0, win) (or any bins) */
NGV_API int ngv_lncc_loss_fwd_bwd(const float *F, const float *W, const ngv_dims *d, int win, float eps,
                          float weight, double *loss, float *gW, int accumulate, void *ws,
                          size_t ws_bytes, void *stream);

/* Optimiser step on the displacement field (method overview: states m1, m2,
 * a gradient step after Sobolev smoothing). g = gu, or, with
 * smooth_sigma > 0, gu smoothed by the normalised Gaussian of that standard
 * deviation (voxels; taps -R..R, R = ceil(3 sigma) <= 4, zero padding), then
 * Adam with bias correction at step >= 1:
 *   m1 = b1 m1 + (1-b1) g,  m2 = b2 m2 + (1-b2) g^2,
 *   u -= lr (m1 / (1-b1^step)) / (sqrt(m2 / (1-b2^step)) + eps).
 *   u, m1, m2 device, 3 * d volume floats (updated in place); gu device.
 *   step_dev  NULL (the step number is `step`), or a device int32 holding it
 *             (read when the call's kernels run; `step` is then ignored and
 *             values below 1 count as 1), so that a captured graph can
 *             replay the update with the step advanced on the device. The
 *             bias corrections are formed the same way either way (fp64,
 *             rounded to fp32); with step_dev a one-thread kernel forms them
 *             into the workspace, which this call then requires. */
NGV_API int ngv_adam_step(float *u, const float *gu, float *m1, float *m2, const ngv_dims *d, int step,
                  const int32_t *step_dev, float lr, float beta1, float beta2, float eps, float smooth_sigma,
                  void *ws, size_t ws_bytes, void *stream);

/* The sampler backward fused with the optimiser step, for an update without
 * smoothing (Key design 1 backward; method overview: gradient step with
 * states m1, m2). The u-gradient of this call is formed as in ngv_warp_bwd,
 * gu_partial is added to it (the gradient accumulated by earlier slabs with
 * ngv_warp_bwd; NULL: none), and the Adam step of ngv_adam_step with
 * smooth_sigma = 0 is applied to u, m1, m2 in place. The gradient itself is
 * not stored. Each voxel's u is read and rewritten by the same thread only,
 * so u is both the sampler's displacement and the updated state.
 *   u, m1, m2  device, 3 * od volume floats (updated);  gW device, od volume
 *   gA9, gt3   as in ngv_warp_bwd, added to with accumulate_affine = 1
 *   step, step_dev  as in ngv_adam_step
 * Same result as ngv_warp_bwd followed by ngv_adam_step, without writing and
 * re-reading gu. */
NGV_API int ngv_warp_bwd_adam(const float *M, const ngv_dims *md, const ngv_slab *slab, float *u,
                              const ngv_dims *od, const ngv_xform *xf, const float *gW,
                              const float *gu_partial, float *m1, float *m2, int step,
                              const int32_t *step_dev, float lr, float beta1, float beta2, float eps,
                              double *gA9, double *gt3, int accumulate_affine, void *ws, size_t ws_bytes,
                              void *stream);

/* The sampler backward fused with the optimiser step for a moving image held
 * in z-slabs (Key design 1 backward; Key design 4 partial sums; method
 * overview: gradient step with states m1, m2). Call it once per slab, in
 * increasing z, the slabs covering [0, md->nz) without gaps, each call with
 * the same u, xf and z-range bound (slab->zrange from ngv_warp_zrange,
 * required). A voxel's u-gradient is the sum of its slabs' parts in slab
 * order: the first slab that reaches it starts the sum, later ones add to it
 * in gu, and the last one that reaches it (no later slab can) applies the
 * Adam step of ngv_adam_step (smooth_sigma = 0) to u, m1, m2 with that sum,
 * without storing it; the top slab's call also steps the voxels that no slab
 * reaches, with a zero gradient. After the last call every voxel has had one
 * step, bit for bit as after ngv_warp_bwd on every slab and
 * ngv_warp_bwd_adam's update, without zeroing gu or a second pass over it.
 *   u    device, updated in place: a call writes only the voxels it
 *        completes, and no later call of the sequence reads them, so every
 *        sample is taken at the u of the sequence's start (which the z-range
 *        bound must describe)
 *   gu   device, 3 * od volume floats: scratch for the partial sums between
 *        the calls (no initialisation needed; its contents are unspecified
 *        afterwards)
 *   gA9, gt3  as in ngv_warp_bwd_adam (accumulate_affine = 1 after the first)
 *   step, step_dev  as in ngv_adam_step
 * The z-range bound decides which slabs reach a voxel (conservatively), the
 * same way in every call. */
NGV_API int ngv_warp_bwd_adam_slab(const float *M, const ngv_dims *md, const ngv_slab *slab, float *u,
                                   const ngv_dims *od, const ngv_xform *xf, const float *gW, float *gu, float *m1,
                                   float *m2, int step, const int32_t *step_dev, float lr, float beta1,
                                   float beta2, float eps, double *gA9, double *gt3, int accumulate_affine,
                                   void *ws, size_t ws_bytes, void *stream);

/* One call of the backward slab sequence of ngv_warp_bwd_adam_slab that also
 * forms the MI term's gradient (Key design 2, the MI gradient in the
 * backward; Key design 4, slabs): at each voxel it adds to gW's value the
 * MI gradient that ngv_mi_grad would add, from F, the stored W and the
 * log-ratio table that the latest MI forward left in this workspace. With
 * the moving image in slabs no one call sees W whole, so W is the stored
 * result of the forward slab sequence (the recomputing ngv_warp_bwd_adam_mi
 * needs the whole moving image). The same u, m1, m2 and gu, bit for bit, as
 * ngv_mi_grad adding to gW and then ngv_warp_bwd_adam_slab.
 *   gW      device, od volume floats: the other terms' gradient (NULL: none)
 *   F, W    device, od volume floats: the fixed image and the stored W
 *   bins, fmin, fmax, wmin, wmax, weight_mi  as in ngv_mi_loss_fwd_bwd; the
 *           table is held in LDS: bins above 128, or 2^32 voxels or more,
 *           return NGV_EUNSUPPORTED
 *   other arguments as in ngv_warp_bwd_adam_slab;
 *   ws      at least ngv_workspace_bytes(bins, 0) */
NGV_API int ngv_warp_bwd_adam_slab_mi(const float *M, const ngv_dims *md, const ngv_slab *slab, float *u,
                                      const ngv_dims *od, const ngv_xform *xf, const float *gW, const float *F,
                                      const float *W, int bins, float fmin, float fmax, float wmin, float wmax,
                                      float weight_mi, float *gu, float *m1, float *m2, int step,
                                      const int32_t *step_dev, float lr, float beta1, float beta2, float eps,
                                      double *gA9, double *gt3, int accumulate_affine, void *ws, size_t ws_bytes,
                                      void *stream);

/* The sampler backward fused with the MI gradient and the optimiser step:
 * the second sweep of a fused step (Key design 1 backward, Key design 2 MI
 * gradient, method overview gradient step). Per output voxel the call forms
 * W from the corners that the backward gathers anyway (the sampler forward's
 * value, bit for bit), the MI gradient from F and that W with the log-ratio
 * table that the latest MI forward left in this workspace (as ngv_mi_grad:
 * the cubic kernel on both images, the same F, bins, ranges and weight),
 * adds gW (the other terms' gradient, e.g. the LNCC call's, which then
 * overwrites rather than accumulates; NULL: none), and continues as
 * ngv_warp_bwd_adam. Same results, bit for bit, as ngv_mi_grad into gW (or
 * into a zeroed buffer when gW is NULL) followed by ngv_warp_bwd_adam, without
 * writing or re-reading the MI gradient or reading W.
 * Whole moving image only (no slab): W must be the sampler of all of M.
 *   M, md, u, od, xf  as in ngv_warp_bwd_adam (u updated in place)
 *   F     device, od volume floats (the fixed image on the output grid)
 *   gW    device, od volume floats, or NULL
 *   bins, fmin, fmax, wmin, wmax, weight  as in ngv_mi_loss_fwd_bwd
 *   m1, m2, step, step_dev, lr, beta1, beta2, eps, gA9, gt3,
 *   accumulate_affine  as in ngv_warp_bwd_adam
 *   ws    the workspace of the MI forward, at least ngv_workspace_bytes(bins, 0)
 * The table is held in LDS: bins above 128, or a volume of 2^32 voxels or
 * more, return NGV_EUNSUPPORTED (use ngv_mi_loss_fwd_bwd's gradient and
 * ngv_warp_bwd_adam instead). */
NGV_API int ngv_warp_bwd_adam_mi(const float *M, const ngv_dims *md, float *u, const ngv_dims *od,
                                 const ngv_xform *xf, const float *F, const float *gW, int bins, float fmin,
                                 float fmax, float wmin, float wmax, float weight, float *m1, float *m2, int step,
                                 const int32_t *step_dev, float lr, float beta1, float beta2, float eps,
                                 double *gA9, double *gt3, int accumulate_affine, void *ws, size_t ws_bytes,
                                 void *stream);

/* The sampler forward with the MI forward in the same sweep (the first sweep
 * of a fused step; Key design 1 and Key design 2): W (+)= the sampler exactly
 * as ngv_warp_fwd, and the joint Parzen histogram of (F, W) over the output
 * grid is built from the final W values as the sweep produces them, then
 * finalised as in ngv_mi_loss_fwd_bwd: loss (+)= weight * (-MI)
 * (accumulate_loss), and the log-ratio table stays in the workspace for
 * ngv_mi_grad. W must be complete after this call: the whole image, or the
 * last slab with accumulate = 1 (every output voxel is visited; a z-range
 * bound only skips the gathers this slab cannot need). W = NULL: the
 * samples feed the histogram and are not stored (one call over the whole
 * moving image, accumulate = 0: the first sweep of a fused step).
 *   F     device, od volume floats (the fixed image on the output grid)
 *   bins, fmin, fmax, wmin, wmax, weight  as in ngv_mi_loss_fwd_bwd
 *   loss  device, 1 double
 * The block histograms are held in LDS: bins above 128, or a volume of 2^32
 * voxels or more, return NGV_EUNSUPPORTED. */
NGV_API int ngv_warp_fwd_mi(const float *M, const ngv_dims *md, const ngv_slab *slab, const float *u,
                            const ngv_dims *od, const ngv_xform *xf, float *W, int accumulate, const float *F,
                            int bins, float fmin, float fmax, float wmin, float wmax, float weight, double *loss,
                            int accumulate_loss, void *ws, size_t ws_bytes, void *stream);

/* The second sweep of a fused step, LNCC and MI together (Key design 1:
 * the composite sampler recomputes each sample instead of storing W; Key
 * design 2: the fused LNCC and the MI gradient). For every voxel the call
 * needs, W is the sampler of M at A x + t + S u(x), evaluated again (bit for
 * bit ngv_warp_fwd's value) rather than read; the LNCC loss and gradient are
 * those of ngv_lncc_loss_fwd_bwd on that W, the MI gradient (bins > 0) that
 * of ngv_mi_grad from the log-ratio table that the latest MI forward left in
 * this workspace (ngv_warp_fwd_mi with W = NULL, or ngv_mi_loss_fwd_bwd), and
 * their sum (the LNCC term as the LNCC call would store it, plus the MI term)
 * feeds the sampler backward at each output voxel as in ngv_warp_bwd: gu is
 * written, dA and dt summed. Neither W nor dL/dW is stored anywhere; gu is,
 * for an optimiser step that may smooth it (ngv_adam_step).
 *   M, md, u, od, xf  as in ngv_warp_bwd, whole moving image (no slab)
 *   F       device, od volume floats (the fixed image on the output grid)
 *   win, eps, weight_lncc  as in ngv_lncc_loss_fwd_bwd, but win 3..11 only (this is
 *           the small-window kernel; 13..31 return NGV_EUNSUPPORTED);
 *           loss_lncc device, 1 double
 *   bins    0 (no MI term) or as in ngv_mi_loss_fwd_bwd, with fmin, fmax,
 *           wmin, wmax, weight_mi
 *   gu      device, 3 * od volume floats, written; must not overlap u
 *   gA9, gt3, accumulate_affine  as in ngv_warp_bwd_adam
 *   ws      at least ngv_workspace_bytes(bins, 0)
 * Same gu, bit for bit, as ngv_warp_fwd, ngv_lncc_loss_fwd_bwd writing gW,
 * ngv_mi_grad adding to it and ngv_warp_bwd on the sum; the same LNCC loss. */
NGV_API int ngv_warp_lncc_mi_bwd(const float *M, const ngv_dims *md, const float *u, const ngv_dims *od,
                                 const ngv_xform *xf, const float *F, int win, float eps, float weight_lncc,
                                 double *loss_lncc, int bins, float fmin, float fmax, float wmin, float wmax,
                                 float weight_mi, float *gu, double *gA9, double *gt3, int accumulate_affine, void *ws,
                                 size_t ws_bytes, void *stream);

/* The MI gradient sweep (Key design 2) from the log-ratio table that the
 * latest MI forward left in this workspace (ngv_warp_fwd_mi, or
 * ngv_mi_loss_fwd_bwd; the cubic kernel on both images) for the same F, W,
 * bins, ranges and weight:
 * gW (+)= d loss / d W, as in ngv_mi_loss_fwd_bwd. F, W, gW 16-byte aligned.
 * Bins 8..256, fewer than 2^32 voxels (else NGV_EUNSUPPORTED). */
NGV_API int ngv_mi_grad(const float *F, const float *W, const ngv_dims *d, int bins, float fmin, float fmax,
                        float wmin, float wmax, float weight, float *gW, int accumulate, void *ws,
                        size_t ws_bytes, void *stream);

/* The range of the z-component of the displacement S u, in the voxel units of
 * the moving grid md, over the output grid od: zrange[0] = min, zrange[1] =
 * max over all output voxels (fp64). It lets slab calls (ngv_slab.zrange)
 * visit only the output voxels whose samples can reach their slab (Key
 * design 4: a shard's partial sum is zero outside the region it maps to).
 *   u       device, 3 * od volume floats;  md, xf as for the sampler
 *   zrange  device, 2 doubles (written) */
NGV_API int ngv_warp_zrange(const float *u, const ngv_dims *od, const ngv_dims *md, const ngv_xform *xf,
                            double *zrange, void *ws, size_t ws_bytes, void *stream);

/* Mean squared error as the similarity term, with its gradient (section
 * "Background and motivation": MSE among the similarity terms; Key design 5:
 * a per-voxel loss, so shard values merge by their N_h / N weighted sum):
 *   loss = weight * (1/N) sum_x (W(x) - F(x))^2,  gW = 2 weight (W - F) / N.
 * The squares are summed in fp64 from exact fp64 differences; the order of
 * the sum is fixed for a device, so the loss is the same on every run.
 *   F, W  device, d volume floats, 16-byte aligned
 *   loss  device, 1 double;  gW device, d volume floats, 16-byte aligned
 *         (NULL: loss only). Workspace: ngv_workspace_bytes(0, 0). */
NGV_API int ngv_mse_loss_fwd_bwd(const float *F, const float *W, const ngv_dims *d, float weight, double *loss,
                                 float *gW, int accumulate, void *ws, size_t ws_bytes, void *stream);

/* Warp composition with the composite sampler (section "Background and
 * motivation": warp composition is one of the profiled memory bottlenecks;
 * Key design 1). With p(i) = A x_i + t + S v(i) as in ngv_warp_fwd, per
 * component c = x, y, z:
 *   w_c(i) = v_c(i) + U~_c(p(i)),
 * U~_c the trilinear, zero-padded interpolation of component c of the field U
 * on its own grid ud, whose end voxels sit at -1 and +1. With
 * phi_v(x) = A x + t + S v(x) and phi_U(y) = y + S U(y) this is
 * phi_U(phi_v(x)) = A x + t + S w(x).
 *   uf  device, 3 * ud volume floats (U, components x, y, z)
 *   v   device, 3 * vd volume floats;  w device, 3 * vd volume floats
 *   w may be v itself (in place); it must not overlap uf (NGV_EINVAL).
 * No workspace, no slab: the whole of U is held. */
NGV_API int ngv_warp_compose(const float *uf, const ngv_dims *ud, const float *v, const ngv_dims *vd,
                             const ngv_xform *xf, float *w, void *stream);

/* Text for a status code; for NGV_EHIP it includes the last HIP error. The
 * returned string is owned by the library (thread-local, valid until the next
 * call from the same thread). */
NGV_API const char *ngv_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* NGV_H */
