"""FP8 linear layer as a torch autograd op, built only from the C-ABI entry points.

Forward (Jet-RL pages, paper.rainbus.top summary, "方法步骤详情" steps 1-3):
X is quantised 1x128 (or taken already quantised from ``rmsnorm_quant``), W
128x128, Y = FProp; the FP8 X (codes + scales) and FP8 W are what is saved for
backward -- no bf16 copy of X is kept.

Backward (step 4): dY stays bf16 between layers and is quantised 1x128 for
DGrad (dX = dY W, the weight blocks used transposed) and, after the 128x1
requantisation of both saved operands, WGrad (dW = dY^T X).

Every arithmetic step runs in libjetfp8.so; this module only orders the calls
and allocates outputs through torch.  The token count M must be a multiple of
128 for the backward (128-token groups of the requantisation).

Optionally the weight gradient is kept in fp32 (``gemm_wgrad_f32``): each
backward adds its dW to an fp32 buffer, so the gradients of several
micro-batches are summed before any rounding to bf16.

The modules quantise their weight once per weight version (the unified flow of
the pages' "核心方法" section: one FP8 weight per update, shared by every
forward, rollout or training, and by the backward's DGrad): ``WeightCache``
keeps the 128x128 FP8 form and re-quantises only when the parameter's storage
or its in-place version counter changes.

Rollout: a forward that builds no autograd graph (``torch.no_grad()``, or
neither input nor weight requiring grad) over at most 256 rows runs
``gemm_fprop_packed`` on the cached weight's rollout-packed copy
(``pack_weight_rollout``, made once per weight version).  Its output is bitwise
the training forward's: same codes, scales and fold.
"""

import torch

from . import _lib

# widest row the RMSNorm backward kernel takes (rmsnorm_backward_workspace_bytes)
RMSNORM_BACKWARD_MAX_K = 24576
# most rows gemm_fprop_packed takes
ROLLOUT_MAX_ROWS = 256


def rollout_path(x2, w):
    """True when a forward of x2 [M, K] against w [N, K] needs no autograd graph and
    fits gemm_fprop_packed (M <= 256, 32-bit byte offsets): the rollout path."""
    if torch.is_grad_enabled() and (x2.requires_grad or w.requires_grad):
        return False
    M, K = x2.shape
    N = w.shape[0]
    return M <= ROLLOUT_MAX_ROWS and N * K < 2 ** 31 and M * K < 2 ** 31


class WeightCache:
    """The FP8 form (quantize_weight_128x128) of one bf16 weight, kept until the
    weight changes: its storage (a new tensor), shape or version counter (any
    in-place update, e.g. an optimizer step).  ``quantizations`` counts the calls
    to the quantiser."""

    def __init__(self):
        self.key = None
        self.q = self.s = None
        self.quantizations = 0
        self.packed_key = None
        self.packed = None
        self.packs = 0

    def get(self, w):
        key = (w.data_ptr(), tuple(w.shape), w.device, w._version)
        if key != self.key:
            self.q, self.s = _lib.quantize_weight_128x128(w.detach().contiguous())
            self.quantizations += 1
            self.key = key
        return self.q, self.s

    def get_packed(self, w):
        """(rollout-packed codes, scales) of the current FP8 weight: pack_weight_rollout
        of ``get(w)``'s codes, made once per weight version (``packs`` counts them)."""
        q, s = self.get(w)
        if self.packed_key != self.key:
            self.packed = _lib.pack_weight_rollout(q)
            self.packs += 1
            self.packed_key = self.key
        return self.packed, s


class FP8LinearFunction(torch.autograd.Function):
    """y = x w^T with the mixed-granularity FP8 recipe.  x bf16 [M, K], w bf16 [N, K].

    With ``dw_fp32`` (a float32 [N, K] buffer) the backward adds the weight
    gradient to that buffer in fp32 and returns no gradient for ``w``.  With a
    ``WeightCache`` the weight is quantised only when it has changed."""

    @staticmethod
    def forward(ctx, x, w, dw_fp32=None, wcache=None):
        qx, sx = _lib.quantize_act_1x128(x.contiguous())
        if wcache is not None:
            qw, sw = wcache.get(w)
        else:
            qw, sw = _lib.quantize_weight_128x128(w.contiguous())
        y = _lib.gemm_fprop(qx, sx, qw, sw)
        ctx.save_for_backward(qx, sx, qw, sw)
        ctx.dw_fp32 = dw_fp32
        return y

    @staticmethod
    def backward(ctx, dy):
        qx, sx, qw, sw = ctx.saved_tensors
        dx, dw = fp8_linear_backward(dy, qx, sx, qw, sw, dw_fp32=ctx.dw_fp32)
        return dx, dw, None, None


def fp8_linear_backward(dy, qx, sx, qw, sw, dw_fp32=None):
    """(dx bf16 [M, K], dw bf16 [N, K]) from bf16 dY [M, N] and the saved FP8 operands.
    With ``dw_fp32`` given, dW is added to it in fp32 instead and None is returned for dw."""
    M = dy.shape[0]
    if M % 128:
        raise ValueError(f"FP8 linear backward needs M % 128 == 0 (128-token groups), got M={M}")
    qdy, sdy = _lib.quantize_act_1x128(dy.contiguous())
    dx = _lib.gemm_dgrad(qdy, sdy, qw, sw)
    qxt, sxt = _lib.requant_transpose_128x1(qx, sx)
    qdyt, sdyt = _lib.requant_transpose_128x1(qdy, sdy)
    if dw_fp32 is not None:
        _lib.gemm_wgrad_f32(qdyt, sdyt, qxt, sxt, dw=dw_fp32, accumulate=True)
        return dx, None
    dw = _lib.gemm_wgrad(qdyt, sdyt, qxt, sxt)
    return dx, dw


def fp8_linear(x, w, dw_fp32=None, wcache=None):
    """Functional form of :class:`FP8LinearFunction`."""
    return FP8LinearFunction.apply(x, w, dw_fp32, wcache)


class FP8Linear(torch.nn.Module):
    """A bias-free linear layer with a bf16 master weight [out, in] whose forward
    and backward GEMMs run in FP8 (the unified precision flow: rollout calls the
    same forward).

    ``fp32_grad_accum=True`` keeps the weight gradient in an fp32 buffer
    ``main_grad`` instead of ``weight.grad``: every backward adds to it (summing
    micro-batches before any bf16 rounding); ``zero_main_grad()`` clears it."""

    def __init__(self, in_features, out_features, device=None, fp32_grad_accum=False):
        super().__init__()
        if in_features % 128 or out_features % 128:
            raise ValueError("in_features and out_features must be multiples of 128")
        self.weight = torch.nn.Parameter(
            torch.empty(out_features, in_features, dtype=torch.bfloat16, device=device))
        torch.nn.init.normal_(self.weight, std=0.02)
        self.register_buffer(
            "main_grad",
            torch.zeros(out_features, in_features, dtype=torch.float32, device=device)
            if fp32_grad_accum else None,
            persistent=False)
        self.wcache = WeightCache()

    def zero_main_grad(self):
        if self.main_grad is not None:
            self.main_grad.zero_()

    def forward(self, x):
        shape = x.shape
        x2 = x.reshape(-1, shape[-1])
        if rollout_path(x2, self.weight):
            qx, sx = _lib.quantize_act_1x128(x2.contiguous())
            y = _lib.gemm_fprop_packed(qx, sx, *self.wcache.get_packed(self.weight))
        else:
            y = fp8_linear(x2, self.weight, self.main_grad, self.wcache)
        return y.reshape(*shape[:-1], self.weight.shape[0])


class RMSNormFP8LinearFunction(torch.autograd.Function):
    """y = FP8Linear(RMSNorm(x; gamma, eps); w) with the norm fused into the
    quantisation (rmsnorm_quant_rstd): the normalised activation exists only as
    its FP8 codes and scales.  Saved for backward: bf16 x and the per-row rstd
    (for the norm's gradients) and the FP8 operands of the GEMMs."""

    @staticmethod
    def forward(ctx, x, gamma, w, eps, wcache=None):
        x = x.contiguous()
        qx, sx, rstd = _lib.rmsnorm_quant_rstd(x, gamma.contiguous(), eps)
        qw, sw = wcache.get(w) if wcache is not None else _lib.quantize_weight_128x128(w.contiguous())
        y = _lib.gemm_fprop(qx, sx, qw, sw)
        ctx.save_for_backward(x, gamma, rstd, qx, sx, qw, sw)
        return y

    @staticmethod
    def backward(ctx, dy):
        x, gamma, rstd, qx, sx, qw, sw = ctx.saved_tensors
        dxn, dw = fp8_linear_backward(dy, qx, sx, qw, sw)
        dx, dgamma = _lib.rmsnorm_backward(x, gamma.contiguous(), rstd, dxn)
        # gamma's gradient is computed in fp32; the parameter's dtype is bf16
        return dx, dgamma.to(gamma.dtype), dw, None, None


class RMSNormFP8Linear(torch.nn.Module):
    """RMSNorm (bf16 gamma, initialised to 1) followed by a bias-free FP8 linear
    layer; forward and backward run through the library's kernels."""

    def __init__(self, in_features, out_features, eps=1e-6, device=None):
        super().__init__()
        if in_features % 128 or out_features % 128:
            raise ValueError("in_features and out_features must be multiples of 128")
        if in_features > RMSNORM_BACKWARD_MAX_K:
            raise ValueError(f"in_features={in_features}: the RMSNorm backward takes rows of at most "
                             f"{RMSNORM_BACKWARD_MAX_K} elements")
        self.eps = float(eps)
        self.gamma = torch.nn.Parameter(torch.ones(in_features, dtype=torch.bfloat16, device=device))
        self.weight = torch.nn.Parameter(
            torch.empty(out_features, in_features, dtype=torch.bfloat16, device=device))
        torch.nn.init.normal_(self.weight, std=0.02)
        self.wcache = WeightCache()

    def forward(self, x):
        shape = x.shape
        x2 = x.reshape(-1, shape[-1])
        if rollout_path(x2, self.weight) and not (torch.is_grad_enabled() and self.gamma.requires_grad):
            qx, sx = _lib.rmsnorm_quant(x2.contiguous(), self.gamma.contiguous(), self.eps)
            y = _lib.gemm_fprop_packed(qx, sx, *self.wcache.get_packed(self.weight))
        else:
            y = RMSNormFP8LinearFunction.apply(x2, self.gamma, self.weight, self.eps, self.wcache)
        return y.reshape(*shape[:-1], self.weight.shape[0])


class FP8Stack(torch.nn.Module):
    """A stack of RMSNormFP8Linear layers (for example the four projections of a
    transformer layer's MLP path at the 8B shapes), every GEMM, quantisation and
    normalisation in FP8 through the library.  No activation function between
    the layers: the pages do not define one for this path."""

    def __init__(self, dims, eps=1e-6, device=None):
        super().__init__()
        if len(dims) < 2:
            raise ValueError("dims needs at least an input and an output size")
        self.layers = torch.nn.ModuleList(
            RMSNormFP8Linear(dims[i], dims[i + 1], eps=eps, device=device) for i in range(len(dims) - 1))

    def forward(self, x):
        for layer in self.layers:
            x = layer(x)
        return x
