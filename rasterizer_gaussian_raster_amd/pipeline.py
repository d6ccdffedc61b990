"""Buffers and call sequence for rendering and fitting with libgi.

Torch provides device memory and the stream; every step below is one call of
the C ABI (through :mod:`.gi`):

  render : gi_render_image (preprocess, binning and the forward in one call; same results as
           gi_preprocess_bin_sort -> gi_render_fwd)
  fit (sum mode)   : gi_fit_step_sum, one call per step: binning -> the fused per-tile forward, L2
                     gradient and backward -> Adam with the gathered gradient, which also sets up the
                     updated parameters for the next step's binning (and reduces the loss); with the
                     SSIM loss gi_fit_step_sum_ssim, whose raster pass is forward -> gi_loss_ssim ->
                     backward
  fit (alpha mode) : render -> gi_loss_l2 -> gi_render_bwd -> gi_adam_step (gradients cleared)

Fitter.capture() records the sum-mode step as HIP graphs (torch.cuda.CUDAGraph over the same
calls on the capture stream); step() then replays one graph per step: a single launch instead of a
dozen, so the host no longer paces the GPU.  Adam then reads its step count from device memory.

uint32/uint16 device arrays are held in int32/int16 tensors (same bytes).
"""
from __future__ import annotations

import math

import torch

from . import gi

# Default per-slot learning rates (pixels for the mean and the Cholesky factor,
# colour units for the colours).
DEFAULT_LR = (0.05, 0.05, 0.01, 0.01, 0.01, 0.005, 0.005, 0.005)

# Up to this many tiles the raster kernels take the tiles in gi_bin_sort's
# tile_order (ranked by list length, dealt to the CUs in serpentine layers): the
# whole grid is then resident on the chip at once and the order is what balances
# the CUs.  Larger grids balance themselves.  The order is a schedule, not data:
# one from an earlier binning is as valid, so a fit refreshes it every
# ORDER_EVERY steps only.
ORDER_MAX_TILES = 8192
ORDER_EVERY = 16

# The fitters read the pair count back (one host wait) every CAPACITY_EVERY steps and grow the pair
# buffers when it comes within 80 % of capacity: a binning that overflows renders nothing and
# gives a zero gradient for that step, so growth must come before the count gets there.
CAPACITY_EVERY = 16


class Raster:
    """Device buffers for one (W, H, n, mode) problem."""

    def __init__(self, width, height, n, mode=gi.MODE_SUM, capacity=None, device="cuda"):
        self.W, self.H, self.n, self.mode = int(width), int(height), int(n), int(mode)
        self.desc = gi.desc(self.W, self.H, self.mode)
        self.T = gi.num_tiles(self.desc)
        self.device = device
        alpha = self.mode == gi.MODE_ALPHA
        dev = torch.device(device)
        self.records = torch.empty((max(self.n, 1), 8), dtype=torch.float32, device=dev)
        self.opacity = torch.empty(max(self.n, 1), dtype=torch.float32, device=dev) if alpha else None
        self.pixbox = torch.empty((max(self.n, 1), 4), dtype=torch.int16, device=dev)
        self.counts = torch.empty(max(self.n, 1), dtype=torch.int32, device=dev)
        self.offsets = torch.empty(self.n + 1, dtype=torch.int32, device=dev)
        self.ranges = torch.empty((max(self.T, 1), 2), dtype=torch.int32, device=dev)
        self.d_num = torch.zeros(2, dtype=torch.int32, device=dev)   # M of the last binning; running max
        self.image = torch.empty((3, self.H, self.W), dtype=torch.float32, device=dev)
        self.t_final = torch.empty((self.H, self.W), dtype=torch.float32, device=dev) if alpha else None
        self.last = torch.empty((self.H, self.W), dtype=torch.int32, device=dev) if alpha else None
        self.loss_partials = torch.empty(max(self.T, 1), dtype=torch.float32, device=dev)
        self.order = (torch.empty(max(self.T, 1), dtype=torch.int32, device=dev)
                      if self.T <= ORDER_MAX_TILES else None)
        self.has_order = False          # an order has been written (by any earlier binning)
        self.capacity = 0
        self.keys = self.vals = self.ws = self.bwd_ws = None
        self.M = None
        if capacity is not None:
            self.set_capacity(capacity)

    def set_capacity(self, capacity):
        capacity = int(capacity)
        dev = torch.device(self.device)
        self.capacity = capacity
        self.keys = torch.empty(max(capacity, 1), dtype=torch.int32, device=dev)
        self.vals = torch.empty(max(capacity, 1), dtype=torch.int32, device=dev)
        nbytes = gi.gi_bin_sort_workspace_bytes(self.desc, self.n, capacity)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.bwd_ws = None                      # sized on first backward (capacity-dependent)

    # -- steps ---------------------------------------------------------------------------------
    def _order(self):
        return self.order if self.has_order else None

    def preprocess(self, params, logit=None, stream=None):
        gi.gi_preprocess(self.desc, self.n, params, logit, self.records, self.opacity, self.pixbox, self.counts,
                         stream)

    def _bin_call(self, sync, stream, tile_order, params, logit):
        if params is None:
            return gi.gi_bin_sort(self.desc, self.n, self.pixbox, self.counts, self.offsets, self.keys, self.vals,
                                  self.ranges, self.capacity, self.d_num, self.ws, sync_count=sync, stream=stream,
                                  tile_order=tile_order)
        return gi.gi_preprocess_bin_sort(self.desc, self.n, params, logit, self.records, self.opacity, self.pixbox,
                                         self.counts, self.offsets, self.keys, self.vals, self.ranges,
                                         self.capacity, self.d_num, self.ws, sync_count=sync, stream=stream,
                                         tile_order=tile_order)

    def bin(self, sync=False, slack=1.25, stream=None, order=None, params=None, logit=None):
        """Bin and sort.  sync: read M back (one host wait) and grow the buffers if needed.
        order: also (re)write the tile order; default: only when none has been written yet.
        params (and logit in alpha mode): preprocess them first, in the same call."""
        if order is None:
            order = not self.has_order
        tile_order = self.order if order else None
        if tile_order is not None:
            self.has_order = True
        if self.keys is None:
            self.set_capacity(max(1024, 4 * self.n))
            sync = True
        if not sync:
            self._bin_call(False, stream, tile_order, params, logit)
            return None
        try:
            M = self._bin_call(True, stream, tile_order, params, logit)
        except gi.GiError as e:
            if e.status != gi.GI_ERR_CAPACITY:
                raise
            M = int(self.d_num[0].item()) & 0xFFFFFFFF
            self.set_capacity(int(M * slack) + 1024)
            M = self._bin_call(True, stream, tile_order, None, None)     # preprocess outputs are in place
        self.M = M
        return M

    def forward(self, background=None, stream=None):
        gi.gi_render_fwd(self.desc, self.n, self.records, self.opacity, self.pixbox, self.ranges, self.vals,
                         background, self.image, self.t_final, self.last, stream, tile_order=self._order())
        return self.image

    def forward_l2(self, target, dL_dimage, stream=None):
        gi.gi_render_fwd_l2(self.desc, self.n, self.records, self.pixbox, self.ranges, self.vals, target, self.image,
                            dL_dimage, self.loss_partials, stream, tile_order=self._order())
        return self.image

    def backward(self, dL_dimage, dparams, logit=None, background=None, dlogit=None, dbackground=None,
                 stream=None, d_loss=None):
        """dparams=None (sum mode): leave the per-pair gradients in the workspace for adam_pairs.
        d_loss (sum mode, after forward_l2): also reduce the loss partials into it, in the same launch."""
        if self.bwd_ws is None:
            nbytes = gi.gi_render_bwd_workspace_bytes(self.desc, self.n, self.capacity)
            self.bwd_ws = torch.empty(nbytes, dtype=torch.uint8, device=torch.device(self.device))
        gi.gi_render_bwd(self.desc, self.n, self.records, self.opacity, logit, self.pixbox, self.offsets,
                         self.ranges, self.vals, self.capacity, background, self.t_final, self.last, dL_dimage,
                         dparams, dlogit, dbackground, self.bwd_ws, stream, tile_order=self._order(),
                         loss_partials=self.loss_partials if d_loss is not None else None,
                         loss_count=3 * self.W * self.H, d_loss=d_loss)

    def backward_absgrad(self, dL_dimage, dparams, dabs, stream=None):
        """Sum mode: backward with the gather into dparams (+=), and each Gaussian's absgrad into
        dabs [n,2] (+=)."""
        if self.bwd_ws is None:
            nbytes = gi.gi_render_bwd_workspace_bytes(self.desc, self.n, self.capacity)
            self.bwd_ws = torch.empty(nbytes, dtype=torch.uint8, device=torch.device(self.device))
        gi.gi_render_bwd_absgrad(self.desc, self.n, self.records, self.pixbox, self.offsets, self.ranges, self.vals,
                                 self.capacity, dL_dimage, dparams, dabs, self.bwd_ws, stream,
                                 tile_order=self._order())

    def forward_backward_l2(self, target, dL_dimage=None, stream=None):
        """Sum mode: forward_l2 then backward(dL, None) in one launch (pair gradients in bwd_ws)."""
        if self.bwd_ws is None:
            nbytes = gi.gi_render_bwd_workspace_bytes(self.desc, self.n, self.capacity)
            self.bwd_ws = torch.empty(nbytes, dtype=torch.uint8, device=torch.device(self.device))
        gi.gi_render_fwd_bwd_l2(self.desc, self.n, self.records, self.pixbox, self.offsets, self.ranges, self.vals,
                                self.capacity, target, self.image, dL_dimage, self.loss_partials, self.bwd_ws,
                                stream, tile_order=self._order())
        return self.image

    def render(self, params, logit=None, background=None, sync=True, stream=None):
        """Preprocess, bin and render in one gi_render_image call.  sync: read M back (one host wait)
        and grow the buffers (and render again) if needed."""
        if self.keys is None:
            self.set_capacity(max(1024, 4 * self.n))
            sync = True
        flags = 0
        if self.order is not None:
            flags |= gi.FIT_USE_ORDER if self.has_order else gi.FIT_ORDER
        call = lambda sc, fl: gi.gi_render_image(self.desc, self.n, params, logit, background, self.records,
                                                 self.opacity, self.pixbox, self.counts, self.offsets, self.keys,
                                                 self.vals, self.ranges, self.order, fl, self.capacity, self.d_num,
                                                 self.ws, self.image, self.t_final, self.last, sync_count=sc,
                                                 stream=stream)
        if not sync:
            call(False, flags)
        else:
            try:
                self.M = call(True, flags)
            except gi.GiError as e:
                if e.status != gi.GI_ERR_CAPACITY:
                    raise
                M = int(self.d_num[0].item()) & 0xFFFFFFFF
                self.set_capacity(int(M * 1.25) + 1024)
                self.M = call(True, flags)
        if flags & gi.FIT_ORDER:
            self.has_order = True
        return self.image


DEFAULT_LR_RS = (0.05, 0.05, 0.01, 0.01, 0.01, 0.005, 0.005, 0.005)   # mu, mu, sx, sy, theta, colour


def cholesky_params(params, kind=gi.PARAMS_RS, fx=1.0, fy=1.0, out=None, stream=None):
    """Cholesky-form params of Gaussians given in form `kind`, with the image plane scaled by
    (fx, fy) (to render at another size: fx = W'/W, fy = H'/H)."""
    if out is None:
        out = torch.empty_like(params)
    gi.gi_params_to_cholesky(kind, params.shape[0], params, fx, fy, out, stream)
    return out


def merge_to(params, width, height, target, stream=None):
    """Merge a Cholesky-form set [n,8] down to `target` Gaussians (gi_merge_to: rounds of mutual
    cheapest pairs under the moment-matching cost); returns the new set [m,8] (m > target only when
    no two Gaussians left in neighbouring cells pick each other) and the number of rounds."""
    n = params.shape[0]
    d = gi.desc(width, height)
    ws = torch.empty(gi.gi_merge_workspace_bytes(d, n), dtype=torch.uint8, device=params.device)
    out = torch.empty((max(n, 1), 8), dtype=torch.float32, device=params.device)
    m, rounds = gi.gi_merge_to(d, n, params.contiguous(), target, out, ws, stream)
    return out[:m].clone(), rounds


class FitterRS:
    """Fits rotation-scale Gaussians (mux, muy, sx, sy, theta, cr, cg, cb) with L2 loss and Adam
    (sum mode).  A step: gi_fit_step_sum with GI_FIT_NO_UPDATE on their Cholesky form (preprocess,
    binning, the fused forward / L2 / backward raster, leaving the pair slots in the workspace),
    then gi_adam_step_pairs_rs (gather of the slots, their map to the rotation-scale gradient,
    Adam on the rotation-scale parameters, the loss, and the Cholesky form for the next step).
    Every CAPACITY_EVERY steps the pair count is read back and the buffers grown if needed."""

    def __init__(self, target, params_rs, lr=DEFAULT_LR_RS, betas=(0.9, 0.999), eps=1e-8, capacity_slack=1.5):
        self.target = target.contiguous()
        _, H, W = self.target.shape
        self.params = params_rs.contiguous().clone()
        self.n = self.params.shape[0]
        self.raster = Raster(W, H, self.n, device=self.params.device)
        self.chol = torch.empty_like(self.params)
        self.gchol = torch.zeros_like(self.params)
        self.grad = torch.zeros_like(self.params)
        self.m = torch.zeros_like(self.params)
        self.v = torch.zeros_like(self.params)
        self.dL = torch.empty_like(self.target)
        self.loss = torch.zeros(1, dtype=torch.float32, device=self.params.device)
        self.lr, self.betas, self.eps = tuple(lr), betas, eps
        self._hp = gi.adam_hparams(self.lr, betas[0], betas[1], eps)
        self.step_count = 0
        self.slack = capacity_slack
        cholesky_params(self.params, out=self.chol)
        self.raster.preprocess(self.chol)
        M = self.raster.bin(sync=True)
        self.raster.set_capacity(int(M * capacity_slack) + 4096)

    def check_capacity(self):
        """Host wait: grow the pair buffers when the last binning came near (or over) capacity."""
        M = int(self.raster.d_num[0].item()) & 0xFFFFFFFF
        if M > 0.8 * self.raster.capacity:
            self.raster.set_capacity(int(M * self.slack) + 4096)
            return True
        return False

    def step(self):
        self._step()
        if self.step_count % CAPACITY_EVERY == 0:
            self.check_capacity()

    def _step(self):
        """The Cholesky form of the current params is in self.chol: written by the previous step's
        gi_adam_step_pairs_rs (or by __init__ / step_separate).  Binning and the fused raster run as
        gi_fit_step_sum with GI_FIT_NO_UPDATE (so the raster's workgroups finish the sort where the
        buckets are small), then gi_adam_step_pairs_rs updates the rotation-scale params."""
        r, n = self.raster, self.n
        if r.bwd_ws is None:
            r.bwd_ws = torch.empty(gi.gi_render_bwd_workspace_bytes(r.desc, n, r.capacity), dtype=torch.uint8,
                                   device=self.params.device)
        fb = gi.fit_buffers(self.chol, None, None, self.target, r.image, r.loss_partials, None, r.records, r.pixbox,
                            r.counts, r.offsets, r.keys, r.vals, r.ranges, r.order, r.d_num, r.capacity, r.ws,
                            r.bwd_ws)
        flags = gi.FIT_NO_UPDATE
        if r.order is not None:
            if r.has_order:
                flags |= gi.FIT_USE_ORDER
            if self.step_count % ORDER_EVERY == 0 or not r.has_order:
                flags |= gi.FIT_ORDER
                r.has_order = True
        gi.gi_fit_step_sum(r.desc, n, fb, self._hp, 1, flags=flags)
        self.step_count += 1
        b1, b2 = self.betas
        gi.gi_adam_step_pairs_rs(r.desc, n, r.offsets, r.capacity, r.bwd_ws, self.params, self.m, self.v, self.lr,
                                 b1, b2, self.eps, self.step_count, loss_partials=r.loss_partials,
                                 loss_count=3 * r.W * r.H, d_loss=self.loss, chol_out=self.chol)

    def step_separate(self):
        """The same step from the separate calls (forward + L2, backward to the pair slots, the gather
        to the rotation-scale gradient, Adam): a cross-check of the fused one."""
        r, n = self.raster, self.n
        cholesky_params(self.params, out=self.chol)
        r.bin(sync=False, order=self.step_count % ORDER_EVERY == 0, params=self.chol)
        r.forward_l2(self.target, self.dL)
        r.backward(self.dL, None, d_loss=self.loss)
        self.grad.zero_()
        gi.gi_grad_gather(r.desc, gi.PARAMS_RS, n, self.params, 1.0, 1.0, r.records, r.offsets, r.capacity,
                          r.bwd_ws, self.grad)
        self.step_count += 1
        b1, b2 = self.betas
        gi.gi_adam_step(n, 8, self.params, self.grad, self.m, self.v, self.lr, b1, b2, self.eps, self.step_count, 0)
        cholesky_params(self.params, out=self.chol)


class Fitter:
    """Fits Gaussians to a target image with L2 loss and Adam (all steps in libgi)."""

    def __init__(self, target, params, logit=None, background=None, lr=DEFAULT_LR, lr_logit=0.05, lr_bg=0.01,
                 betas=(0.9, 0.999), eps=1e-8, capacity_slack=1.5, loss=None):
        """loss: None for the L2 loss, or weights (w1, w2, ws) of w1 L1 + w2 L2 + ws (1 - SSIM)
        (gi_loss_ssim; the sum mode then takes the separate forward / loss / backward / Adam launches)."""
        self.target = target.contiguous()
        _, H, W = self.target.shape
        self.params = params.contiguous().clone()
        self.n = self.params.shape[0]
        alpha = logit is not None
        self.raster = Raster(W, H, self.n, gi.MODE_ALPHA if alpha else gi.MODE_SUM, device=self.params.device)
        dev = self.params.device
        self.grad = torch.zeros_like(self.params)
        self.m = torch.zeros_like(self.params)
        self.v = torch.zeros_like(self.params)
        self.logit = logit.contiguous().clone() if alpha else None
        self.bg = background.contiguous().clone() if alpha else None
        if alpha:
            self.g_logit, self.m_logit, self.v_logit = (torch.zeros_like(self.logit) for _ in range(3))
            self.g_bg, self.m_bg, self.v_bg = (torch.zeros(4, dtype=torch.float32, device=dev) for _ in range(3))
            self.bg4 = torch.zeros(4, dtype=torch.float32, device=dev)
            self.bg4[:3] = self.bg
        self.lr, self.lr_logit, self.lr_bg = tuple(lr), lr_logit, lr_bg
        self.betas, self.eps = betas, eps
        self.dL = torch.empty_like(self.target)
        self.loss = torch.zeros(1, dtype=torch.float32, device=dev)
        self.loss_ws = torch.empty(gi.gi_loss_workspace_bytes(self.target.numel()), dtype=torch.uint8, device=dev)
        self.loss_w = None if loss is None else tuple(float(v) for v in loss)
        if self.loss_w is not None:             # the target's SSIM statistics, formed once for the fit
            self.ssim_ws = torch.empty(gi.gi_loss_ssim_workspace_bytes(W, H), dtype=torch.uint8, device=dev)
            gi.gi_loss_ssim_target(W, H, self.target, self.ssim_ws)
        self.step_count = 0
        self.graphs = None
        self.d_step = None
        self.slack = capacity_slack
        self.prepared = False           # the last fit step left the set-up of the current params
        self.track_max = False          # steps also raise raster.d_num[1] to their pair count
        self._fb = None                 # gi_fit_buffers over the current buffers
        self._hp = gi.adam_hparams(self.lr, betas[0], betas[1], eps)
        # size the tile-pair buffers once, with room for the Gaussians to spread
        self.raster.preprocess(self.params, self.logit)
        M = self.raster.bin(sync=True)
        self.raster.set_capacity(int(M * capacity_slack) + 4096)
        self.raster.bwd_ws = torch.empty(gi.gi_render_bwd_workspace_bytes(self.raster.desc, self.n,
                                                                          self.raster.capacity),
                                         dtype=torch.uint8, device=dev)

    def _state(self):
        """The tensors a step updates (parameters and Adam moments, and in alpha mode the logits and
        background with theirs)."""
        t = [self.params, self.m, self.v]
        if self.logit is not None:
            t += [self.logit, self.m_logit, self.v_logit, self.bg4, self.m_bg, self.v_bg]
        return t

    def guarded_steps(self, k, spike=10.0):
        """k training steps with divergence recovery ("FlashImgs", Training features: a loss spike is
        rolled back).  After the k steps the loss is read (one host wait); when it is not finite or
        above spike x the loss of the last good check, the parameters and Adam state go back to that
        check (the k steps are dropped; step counter too) and False is returned; otherwise this state
        becomes the good check and True is returned.  The first call checks against its own start."""
        if getattr(self, "_good", None) is None:
            self._good = [t.clone() for t in self._state()]
            self._good_step, self._good_loss = self.step_count, None
        for _ in range(k):
            self.step()
        loss = float(self.loss.item())
        if not math.isfinite(loss) or (self._good_loss is not None and loss > spike * self._good_loss):
            for t, g in zip(self._state(), self._good):
                t.copy_(g)
            self.step_count = self._good_step
            self.prepared = False           # the set-up in the raster's buffers is of the dropped steps
            self.graphs = None              # captured steps carry that set-up's flag
            return False
        for t, g in zip(self._state(), self._good):
            g.copy_(t)
        self._good_step, self._good_loss = self.step_count, loss
        return True

    def densify(self, s0=1.5):
        """One adaptive-density-control pass (gi_adc, sum mode): dead, out-of-bounds and bloated
        Gaussians are moved to the pixels of largest error of the last rendered image (their Adam
        moments cleared).  Returns a device tensor with the number moved.  The next step sets up
        the binning afresh."""
        if self.logit is not None:
            raise ValueError("density control is for the sum mode")
        r = self.raster
        if getattr(self, "_adc_ws", None) is None:
            self._adc_ws = torch.empty(gi.gi_adc_workspace_bytes(r.desc, self.n), dtype=torch.uint8,
                                       device=self.params.device)
            self._adc_moved = torch.zeros(1, dtype=torch.int32, device=self.params.device)
        gi.gi_adc(r.desc, self.n, self.params, self.m, self.v, r.image, self.target, s0, None, self._adc_moved,
                  self._adc_ws)
        self.prepared = False
        return self._adc_moved

    def check_capacity(self):
        """Host wait: grow the pair buffers when the last binning came near (or over) capacity."""
        M = int(self.raster.d_num[0].item()) & 0xFFFFFFFF
        if M > 0.8 * self.raster.capacity:
            self.graphs = None              # the captured graphs hold the old buffers: capture() again
            self.prepared = False           # the new bin workspace holds no set-up
            self._fb = None
            self.raster.set_capacity(int(M * self.slack) + 4096)
            self.raster.bwd_ws = torch.empty(gi.gi_render_bwd_workspace_bytes(self.raster.desc, self.n,
                                                                              self.raster.capacity),
                                             dtype=torch.uint8, device=self.params.device)
            return True
        return False

    def _sum_step(self, order, d_step=None):
        """The sum-mode step: one gi_fit_step_sum call (binning, fused raster, Adam + the set-up of the
        updated parameters for the next call), or gi_fit_step_sum_ssim with the SSIM loss (the raster
        pass is then forward, loss, backward).  d_step: device step counter, advanced here (graph mode)."""
        r = self.raster
        if self._fb is None:
            self._fb = gi.fit_buffers(self.params, self.m, self.v, self.target, r.image, r.loss_partials, self.loss,
                                      r.records, r.pixbox, r.counts, r.offsets, r.keys, r.vals, r.ranges, r.order,
                                      r.d_num, r.capacity, r.ws, r.bwd_ws)
        flags = gi.FIT_PREPARED if self.prepared else 0
        if self.track_max:
            flags |= gi.FIT_TRACK_MAX
        if r.order is not None:
            if r.has_order:                 # written by an earlier call (any permutation is valid)
                flags |= gi.FIT_USE_ORDER
            if order or not r.has_order:
                flags |= gi.FIT_ORDER
                r.has_order = True
        if d_step is not None:
            d_step.add_(1)
        if self.loss_w is None:
            gi.gi_fit_step_sum(r.desc, self.n, self._fb, self._hp, self.step_count + 1, d_step=d_step, flags=flags)
        else:
            gi.gi_fit_step_sum_ssim(r.desc, self.n, self._fb, self._hp, *self.loss_w, self.dL, self.ssim_ws,
                                    self.step_count + 1, d_step=d_step, flags=flags)
        self.prepared = True

    def capture(self, warmup=2):
        """Record the sum-mode step as two HIP graphs (with and without the tile-order refresh).  The
        `warmup` steps run first (real steps) on a side stream, as graph capture asks."""
        if self.logit is not None or self.loss_w is not None:
            raise ValueError("graph capture is for the sum mode with the L2 loss")
        dev = self.params.device
        self.d_step = torch.full((1,), self.step_count, dtype=torch.int32, device=dev)
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            for _ in range(warmup):
                self._sum_step(self.step_count % ORDER_EVERY == 0, d_step=self.d_step)
                self.step_count += 1
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize(dev)
        graphs = {}
        for order in (False, True):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self._sum_step(order, d_step=self.d_step)
            graphs[order] = g
        torch.cuda.synchronize(dev)
        self.graphs = graphs

    def step(self):
        """One training step.  In sum mode the raster's records / boxes describe the updated parameters
        afterwards and its tile ranges are cleared (the next step's binning starts from them).  Every
        CAPACITY_EVERY steps the pair count is read back and the buffers grown if it nears capacity
        (captured graphs are then recorded again)."""
        self._step()
        if self.step_count % CAPACITY_EVERY == 0:
            had_graphs = self.graphs is not None
            if self.check_capacity() and had_graphs:
                self.capture()

    def _step(self):
        if self.graphs is not None:
            self.graphs[self.step_count % ORDER_EVERY == 0].replay()
            self.step_count += 1
            return
        r = self.raster
        if self.logit is None:
            self._sum_step(self.step_count % ORDER_EVERY == 0)
            self.step_count += 1
            return
        if self.loss_w is None:             # alpha mode, L2: forward with the loss gradient, one update pass
            bg = self.bg4
            r.bin(sync=False, order=self.step_count % ORDER_EVERY == 0, params=self.params, logit=self.logit)
            gi.gi_render_fwd_alpha_l2(r.desc, self.n, r.records, r.opacity, r.pixbox, r.ranges, r.vals, bg,
                                      self.target, r.image, r.t_final, r.last, self.dL, r.loss_partials,
                                      tile_order=r._order())
            r.backward(self.dL, None, logit=self.logit, background=bg)
            self.step_count += 1
            b1, b2 = self.betas
            gi.gi_adam_step_pairs_alpha(r.desc, self.n, r.offsets, r.capacity, r.bwd_ws, self.params, self.m,
                                        self.v, self.lr, self.logit, self.m_logit, self.v_logit, self.lr_logit,
                                        self.bg4, self.m_bg, self.v_bg, self.lr_bg, b1, b2, self.eps,
                                        self.step_count, loss_partials=r.loss_partials,
                                        loss_count=self.target.numel(), d_loss=self.loss)
            return
        self.step_separate()

    def step_separate(self):
        """The step from separate calls: forward, the loss (L2 or SSIM), backward with the gather, and
        Adam (in the alpha mode with L2 a cross-check of the fused step)."""
        r = self.raster
        bg = self.bg4 if self.logit is not None else None
        r.bin(sync=False, order=self.step_count % ORDER_EVERY == 0, params=self.params, logit=self.logit)
        r.forward(bg)
        if self.loss_w is None:
            gi.gi_loss_l2(self.target.numel(), r.image, self.target, self.dL, self.loss, self.loss_ws)
        else:
            _, H, W = self.target.shape
            gi.gi_loss_ssim(W, H, r.image, self.target, *self.loss_w, self.dL, self.loss, self.ssim_ws,
                            flags=gi.SSIM_TARGET_PREPARED)
        if self.logit is None:
            r.backward(self.dL, self.grad)
            self.step_count += 1
            b1, b2 = self.betas
            gi.gi_adam_step(self.n, 8, self.params, self.grad, self.m, self.v, self.lr, b1, b2, self.eps,
                            self.step_count, 1)
            return
        r.backward(self.dL, self.grad, logit=self.logit, background=bg, dlogit=self.g_logit,
                   dbackground=self.g_bg)
        self.step_count += 1
        b1, b2 = self.betas
        gi.gi_adam_step(self.n, 8, self.params, self.grad, self.m, self.v, self.lr, b1, b2, self.eps,
                        self.step_count, 1)
        gi.gi_adam_step(self.n, 1, self.logit, self.g_logit, self.m_logit, self.v_logit, [self.lr_logit],
                        b1, b2, self.eps, self.step_count, 1)
        gi.gi_adam_step(1, 4, self.bg4, self.g_bg, self.m_bg, self.v_bg, [self.lr_bg] * 3 + [0.0],
                        b1, b2, self.eps, self.step_count, 1)
