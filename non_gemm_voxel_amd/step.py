"""One optimisation step of affine + deformable registration on one GPU, as
the sequence of C-ABI calls the objective L(phi) = C(F, M o phi) + R(phi)
implies ("A Scalable Distributed Framework for Multimodal GigaVoxel Image
Registration", Background and method overview):

  W  = sampler(M; A, t, u)                    ngv_warp_fwd  (per z-slab of M: ngv_warp_fwd_slab; with
                                              fused_mi the last is ngv_warp_fwd_mi, the
                                              MI forward in the same sweep -- slower on
                                              MI355X than the separate calls, so off)
  gW = dC/dW  for C = -MI and/or -mean(cc)    ngv_mi_grad (or ngv_mi_loss_fwd_bwd), ngv_lncc_loss_fwd_bwd
  gu, dA, dt = sampler backward               ngv_warp_bwd  (per z-slab of M)
  u  = Adam(u, smooth(gu))                    ngv_adam_step

Without smoothing the last two are one call, ngv_warp_bwd_adam (the last
slab's backward feeds the update directly; gu is not written), unless
fused=False. With MI (mi_in_backward, the default) the MI call only builds
the histogram, the loss and the log-ratio table, the LNCC call writes gW
rather than adding to it, and the backward forms the MI gradient itself:
with the whole moving image in one piece that call is ngv_warp_bwd_adam_mi,
from F and the W it recomputes from its own gathers (the second sweep of a
fused step); with the moving image in z-slabs each slab call is
ngv_warp_bwd_adam_slab_mi, from F and the stored W. The results are bit for
bit those of the separate calls. With several z-slabs, ngv_warp_zrange first
bounds the z-displacement so that each slab call visits only the output
voxels that can sample its planes. All buffers are device tensors allocated
once; the step itself allocates nothing. Calls are enqueued on the current
stream.

The Adam step number lives on the device (step_dev, advanced by a one-element
kernel each step), so a whole step can be captured once as a HIP graph
(capture()) and replayed: for volumes small enough that launches dominate.
"""
import torch

from . import ngv


class RegistrationStep:
    def __init__(self, F, M, A, t, bins=None, win=None, smooth_sigma=0.0, lr=1e-3, slabs=1, S=None,
                 eps_lncc=1e-5, betas=(0.9, 0.999), eps_adam=1e-8, fused=True, fused_mi=False,
                 mi_in_backward=True, fused_step=False):
        if bins is None and win is None:
            raise ValueError("at least one similarity term (bins for MI, win for LNCC)")
        dev = F.device
        shape = tuple(F.shape)
        self.shape = shape
        self.F, self.M = F, M
        self.bins, self.win = bins, win
        self.smooth_sigma, self.lr = smooth_sigma, lr
        self.betas, self.eps_adam, self.eps_lncc = betas, eps_adam, eps_lncc
        self.xf = ngv.make_xform(A, t, S)
        vec = (3,) + shape
        self.u = torch.zeros(vec, dtype=torch.float32, device=dev)
        self.m1 = torch.zeros(vec, dtype=torch.float32, device=dev)
        self.m2 = torch.zeros(vec, dtype=torch.float32, device=dev)
        self.gu = torch.empty(vec, dtype=torch.float32, device=dev)
        self.W = torch.empty(shape, dtype=torch.float32, device=dev)
        self.gW = torch.empty(shape, dtype=torch.float32, device=dev)
        self.loss = torch.zeros(2, dtype=torch.float64, device=dev)  # [MI term, LNCC term]
        self.gA = torch.zeros(9, dtype=torch.float64, device=dev)
        self.gt = torch.zeros(3, dtype=torch.float64, device=dev)
        self.ws = ngv.workspace(dev, bins or 32, win or 9)
        nz = shape[0]
        bounds = [round(h * nz / slabs) for h in range(slabs + 1)]
        self.slabs = [(bounds[h], bounds[h + 1] - bounds[h]) for h in range(slabs)]
        self.M_views = [M[z0:z0 + n] for z0, n in self.slabs]
        self.zrange = torch.zeros(2, dtype=torch.float64, device=dev) if slabs > 1 else None
        self.slab_args = [(z0, n, self.zrange) for z0, n in self.slabs]
        self.t = 0
        self.step_dev = torch.zeros(1, dtype=torch.int32, device=dev)  # the Adam step number, on the device
        self.fused = fused and smooth_sigma == 0.0
        # the sweeps that hold the MI histogram or table in LDS take at most 128 bins
        lds_bins = bins is not None and bins <= 128
        self.fused_mi = fused_mi and lds_bins
        # the MI gradient formed in the fused backward: MI, no smoothing; with
        # one slab from the W the backward recomputes, with several from the
        # stored W (no one slab call sees W whole)
        self.mi_bwd = mi_in_backward and lds_bins and self.fused
        # the two-sweep fused step: sweep 1 the MI forward on samples that are
        # not stored, sweep 2 the LNCC (and MI) gradient on samples taken
        # again, into the sampler backward; then the optimiser step on gu
        # (the fused second sweep is the small-window LNCC kernel: w <= 11)
        self.fused_step = fused_step and win is not None and win <= 11 and slabs == 1 and (bins is None or lds_bins)

    def warp(self):
        """W from the current u (slab by slab, after bounding the displacement);
        with fused_mi the last slab's sweep also does the MI forward."""
        if self.zrange is not None:
            ngv.ngv_warp_zrange(self.u, self.xf, self.zrange, self.shape, ws=self.ws)
        last = len(self.slab_args) - 1
        for h, sl in enumerate(self.slab_args):
            if h == last and self.fused_mi:
                ngv.ngv_warp_fwd_mi(self.M_views[h], self.u, self.xf, self.W, self.F, self.loss[0:1], bins=self.bins,
                                    mdims=self.shape, slab=sl, accumulate=h > 0, ws=self.ws)
            elif self.zrange is not None and not self.fused_mi:
                ngv.ngv_warp_fwd_slab(self.M_views[h], self.u, self.xf, self.W, sl, mdims=self.shape)
            else:
                ngv.ngv_warp_fwd(self.M_views[h], self.u, self.xf, self.W, mdims=self.shape, slab=sl,
                                 accumulate=h > 0)

    def mi(self):
        """The MI loss (unless the sweep did it) and its gradient into gW; with
        mi_in_backward only the loss and the log-ratio table (the backward
        forms the gradient)."""
        if self.fused_mi:
            if not self.mi_bwd:
                ngv.ngv_mi_grad(self.F, self.W, self.gW, bins=self.bins, ws=self.ws)
        else:
            ngv.ngv_mi_loss_fwd_bwd(self.F, self.W, self.loss[0:1], None if self.mi_bwd else self.gW,
                                    bins=self.bins, ws=self.ws)

    def lncc(self):
        """The LNCC loss and its gradient, added to gW after MI (written when
        it is the only term in gW). The call adds to both its outputs when it
        accumulates, so the loss slot is cleared first (a fill kernel) to hold
        this step's value alone."""
        acc = self.bins is not None and not self.mi_bwd
        if acc:
            self.loss[1:2].zero_()
        ngv.ngv_lncc_loss_fwd_bwd(self.F, self.W, self.loss[1:2], self.gW, win=self.win, eps=self.eps_lncc,
                                  accumulate=acc, ws=self.ws)

    def losses(self):
        """The losses and gW."""
        if self.bins:
            self.mi()
        if self.win:
            self.lncc()

    def forward(self):
        """W, the losses and gW."""
        self.warp()
        self.losses()

    def backward(self):
        """gu, dA, dt (unfused path)."""
        for h, sl in enumerate(self.slab_args):
            ngv.ngv_warp_bwd(self.M_views[h], self.u, self.xf, self.gW, self.gu, self.gA, self.gt,
                             mdims=self.shape, slab=sl, accumulate=h > 0, ws=self.ws)

    def _advance(self):
        self.t += 1
        self.step_dev.add_(1)

    def update(self):
        self._advance()
        ngv.ngv_adam_step(self.u, self.gu, self.m1, self.m2, self.t, self.lr, self.betas[0], self.betas[1],
                          self.eps_adam, self.smooth_sigma, ws=self.ws, step_dev=self.step_dev)

    def forward_backward(self):
        self.forward()
        self.backward()

    def backward_update(self):
        """The sampler backward fused with the update. With several slabs each
        slab's call adds its part of the gradient and steps the voxels that no
        later slab reaches (gu holds the partial sums in between)."""
        self._advance()
        if self.zrange is not None:
            for h, sl in enumerate(self.slab_args):
                kw = dict(beta1=self.betas[0], beta2=self.betas[1], eps=self.eps_adam, mdims=self.shape,
                          accumulate_affine=h > 0, ws=self.ws, step_dev=self.step_dev)
                if self.mi_bwd:
                    ngv.ngv_warp_bwd_adam_slab_mi(self.M_views[h], self.u, self.xf, self.gW if self.win else None,
                                                  self.F, self.W, self.gu, self.m1, self.m2, self.t, self.lr, self.gA,
                                                  self.gt, sl, bins=self.bins, **kw)
                else:
                    ngv.ngv_warp_bwd_adam_slab(self.M_views[h], self.u, self.xf, self.gW, self.gu, self.m1, self.m2,
                                               self.t, self.lr, self.gA, self.gt, sl, **kw)
            return
        if self.mi_bwd:
            ngv.ngv_warp_bwd_adam_mi(self.M, self.u, self.xf, self.F, self.gW if self.win else None, self.m1,
                                     self.m2, self.t, self.lr, self.gA, self.gt, bins=self.bins,
                                     beta1=self.betas[0], beta2=self.betas[1], eps=self.eps_adam, ws=self.ws,
                                     step_dev=self.step_dev)
            return
        last = len(self.slabs) - 1
        for h, sl in enumerate(self.slab_args[:-1]):
            ngv.ngv_warp_bwd(self.M_views[h], self.u, self.xf, self.gW, self.gu, self.gA, self.gt,
                             mdims=self.shape, slab=sl, accumulate=h > 0, ws=self.ws)
        ngv.ngv_warp_bwd_adam(self.M_views[last], self.u, self.xf, self.gW, self.m1, self.m2, self.t, self.lr,
                              self.gA, self.gt, gu_partial=self.gu if last > 0 else None, beta1=self.betas[0],
                              beta2=self.betas[1], eps=self.eps_adam, mdims=self.shape, slab=self.slab_args[last],
                              accumulate_affine=last > 0, ws=self.ws, step_dev=self.step_dev)

    def mi_sweep(self):
        """Sweep 1 of the fused step: the MI loss and log-ratio table from
        samples that are not stored."""
        ngv.ngv_warp_fwd_mi(self.M, self.u, self.xf, None, self.F, self.loss[0:1], bins=self.bins, ws=self.ws)

    def gradient_sweep(self):
        """Sweep 2 of the fused step: the LNCC loss and the gradient of both
        terms into gu, dA, dt, on samples taken again."""
        ngv.ngv_warp_lncc_mi_bwd(self.M, self.u, self.xf, self.F, self.loss[1:2], self.gu, self.gA, self.gt,
                                 win=self.win, eps=self.eps_lncc, bins=self.bins, ws=self.ws)

    def fused_sweeps(self):
        """Both sweeps of the fused step; neither W nor gW is written."""
        if self.bins:
            self.mi_sweep()
        self.gradient_sweep()

    def step(self):
        if self.fused_step:
            self.fused_sweeps()
            self.update()
            return
        self.forward()
        if self.fused:
            self.backward_update()
        else:
            self.backward()
            self.update()

    def capture(self):
        """One whole step recorded as a HIP graph (nothing runs while it is
        recorded); each replay is one more step, with the step number advanced
        on the device, bit for bit as step(). Replays read and write this
        object's tensors in place and continue from whatever state the eager
        calls left. The caller synchronises as for any stream work."""
        dev = self.F.device
        t = self.t
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            self.step()
        torch.cuda.current_stream(dev).wait_stream(side)
        self.t = t  # recording ran no step
        return graph
