"""PyTorch integration of the FP8 scaled linear layer and the GradScaler step,
over the C-ABI library: every FP8 cast, GEMM, unscale, check and scale update
runs in libfp8sg's kernels; this module only allocates buffers, wires
autograd and walks module trees.

  - Float8Linear / _Fp8LinearFn ["FP8训练：量化、自动微分、Torchao", §6: one
    autograd node per linear; the forward takes and returns plain bf16, FP8
    never leaves it; what is saved for the backward pass is the FP8 operands
    and their inverse scales, not the bf16 inputs; §1 for row-wise scaling].
  - convert_to_float8_training [same page, §8: post-order walk over the module
    tree, nn.Linear children replaced in place when module_filter_fn(module,
    fully qualified name) allows, the new module reusing the original weight
    tensor].
  - GradScaler ["第20章 量化与混合精度训练", §20.2.2 and §20.5.33;
    "AMP：Automatic Mixed Precision 技术笔记", §4 and §6]: scale the loss,
    unscale fp16 gradients in place with the non-finite check, skip the
    optimizer step on inf/NaN, update the scale on the device.

Dynamic scaling runs through two registered operators, fp8sg::scaled_linear_fwd
and fp8sg::scaled_linear_bwd (torch.library custom ops with shape-only fake
implementations and an autograd formula), so torch.compile keeps each FP8 linear
as one opaque call in its graph (the same page, §7: the compiler sees the FP8
linear as an opaque call and optimises around it) instead of tracing into the
library calls.  Delayed and row-wise scaling use an autograd.Function in eager
mode; a module keeps its backward scratch (the quantized gradient) across steps.

An fp16 model under loss scaling [PT-CH20 §20.2.2] uses fp16 layers
(Float8Linear with an fp16 weight): fp16 inputs are cast by the fp16-input
kernels, outputs and gradients are fp16, and with a GradScaler attached the
weight gradient leaves the wgrad GEMM unscaled and checked (the scaler's
unscale_ then skips it); the input gradient keeps the loss scale for the layers
below.

Limits of this layer: inputs and weights are bf16 or fp16; Float8Linear has no bias (the method's linear has none; the default
filter leaves biased layers alone); leading dimensions of the input are
flattened into M; M, N, K must be multiples of 16.
"""
from typing import Callable, Optional

import torch
from torch import nn

from . import (E4M3FN, E5M2, LinearBwdWs, LinearBwdWsRW, LinearSaved, LinearSavedRW, OUT_BF16,
               OUT_F16, SCALE_REC_BYTES, ScaleRec,
               amp_norm_workspace_len, amp_unscale_check, amp_unscale_check_norm,
               amp_update_scale, fp8_amax, fp8_amax_f16, fp8_gemm, fp8_gemm_kmajor,
               fp8_gemm_kmajor_unscale, fp8_linear_copies,
               fp8_quantize_f16, fp8_scaled_linear_bwd, fp8_scaled_linear_bwd_delayed,
               fp8_scaled_linear_bwd_rowwise, fp8_scaled_linear_fwd, fp8_scaled_linear_fwd_delayed,
               fp8_scaled_linear_fwd_rowwise)

SCALINGS = ("dynamic", "delayed", "rowwise")


def _seed_history(hist: torch.Tensor, x: torch.Tensor):
    """Delayed scaling needs a history before its first step: its first entry
    becomes max |x| of the first tensor seen (one amax pass)."""
    rec = ScaleRec(device=x.device)
    fp8_amax(x, rec)
    hist.zero_()
    hist[:1].copy_(rec.buf[0:4].view(torch.float32))  # the record's amax field


# ---------------------------------------------------------------- custom ops
# The dynamic-scaling linear as two operators.  The forward returns y and the
# state the backward needs (codes, transposed codes, the two scale records),
# all fresh outputs; nothing is mutated.  Which transposed copies are made
# follows fp8_linear_copies (the fastest backward on this device); a copy not
# made travels as an empty tensor.

def _present(t):
    return t if t is not None and t.numel() > 0 else None


@torch.library.custom_op("fp8sg::scaled_linear_fwd", mutates_args=())
def _op_fwd(x: torch.Tensor, w: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor,
                                                         torch.Tensor, torch.Tensor, torch.Tensor]:
    M, K = x.shape
    N = w.shape[0]
    xt, wt, _ = fp8_linear_copies(M, N, K)
    u8 = dict(dtype=torch.uint8, device=x.device)
    # uninitialised records: the forward writes every field the backward reads
    # (a zero fill would cost one more kernel launch per call)
    saved = LinearSaved(M, N, K, tensors=(
        torch.empty((M, K), **u8), torch.empty((K, M), **u8) if xt else None,
        torch.empty((N, K), **u8), torch.empty((K, N), **u8) if wt else None,
        torch.empty((2, SCALE_REC_BYTES), **u8)))
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    fp8_scaled_linear_fwd(x, w, saved, y, OUT_BF16)
    empty = torch.empty(0, dtype=torch.uint8, device=x.device)
    return (y, saved.x_q, saved.x_qT if xt else empty, saved.w_q, saved.w_qT if wt else empty.clone(),
            saved.recs)


@_op_fwd.register_fake
def _op_fwd_fake(x, w):
    M, K = x.shape
    N = w.shape[0]
    xt, wt, _ = fp8_linear_copies(M, N, K)
    u8 = dict(dtype=torch.uint8, device=x.device)
    return (x.new_empty((M, N), dtype=torch.bfloat16), x.new_empty((M, K), **u8),
            x.new_empty((K, M) if xt else (0,), **u8), x.new_empty((N, K), **u8),
            x.new_empty((K, N) if wt else (0,), **u8), x.new_empty((2, SCALE_REC_BYTES), **u8))


@torch.library.custom_op("fp8sg::scaled_linear_bwd", mutates_args=())
def _op_bwd(gy: torch.Tensor, x_q: torch.Tensor, x_qT: torch.Tensor, w_q: torch.Tensor,
            w_qT: torch.Tensor, recs: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    M, N = gy.shape
    K = x_q.shape[1]
    saved = LinearSaved(M, N, K, tensors=(x_q, _present(x_qT), w_q, _present(w_qT), recs))
    gx = torch.empty((M, K), dtype=torch.bfloat16, device=gy.device)
    gw = torch.empty((N, K), dtype=torch.bfloat16, device=gy.device)
    # the backward writes gy's record before it reads it: no zero fill needed
    rec = ScaleRec(buf=torch.empty(SCALE_REC_BYTES, dtype=torch.uint8, device=gy.device))
    ws = LinearBwdWs(M, N, device=gy.device, transposed=fp8_linear_copies(M, N, K)[2], gy_sc=rec)
    fp8_scaled_linear_bwd(gy, saved, ws, gx, gw, OUT_BF16)
    return gx, gw


@_op_bwd.register_fake
def _op_bwd_fake(gy, x_q, x_qT, w_q, w_qT, recs):
    M, N = gy.shape
    K = x_q.shape[1]
    return (gy.new_empty((M, K), dtype=torch.bfloat16), gy.new_empty((N, K), dtype=torch.bfloat16))


def _op_setup(ctx, inputs, output):
    ctx.save_for_backward(*output[1:])
    # the codes and records are state, not differentiable outputs: without
    # this, autograd passes the backward a zero-filled "gradient" of each (one
    # fill kernel per code tensor, up to 117 MB each in the MLP block)
    ctx.set_materialize_grads(False)


def _op_backward(ctx, gy, *_unused):
    if gy is None:  # y took no part in the loss
        return None, None
    if gy.dtype != torch.bfloat16:
        raise TypeError(f"Float8Linear expects bf16 output gradients, got {gy.dtype}")
    gx, gw = torch.ops.fp8sg.scaled_linear_bwd(gy.contiguous(), *ctx.saved_tensors)
    return gx, gw


_op_fwd.register_autograd(_op_backward, setup_context=_op_setup)


class _Fp8LinearFn(torch.autograd.Function):
    """y = x W^T through the FP8 path with delayed or row-wise scaling; saves
    the FP8 codes (row-major and transposed) and the scale records (delayed) or
    scale vectors (row-wise) for the backward pass."""

    @staticmethod
    def forward(ctx, x2d: torch.Tensor, weight: torch.Tensor, mod: "Float8Linear"):
        M, K = x2d.shape
        N = weight.shape[0]
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x2d.device)
        ctx.mod = mod
        ctx.dims = (M, N, K)
        if mod.scaling == "rowwise":
            saved = LinearSavedRW(M, N, K, device=x2d.device)
            fp8_scaled_linear_fwd_rowwise(x2d, weight, saved, y, OUT_BF16)
            ctx.save_for_backward(*saved.tensors())
            return y
        xt, wt, _ = fp8_linear_copies(M, N, K)
        saved = LinearSaved(M, N, K, device=x2d.device, x_transposed=xt, w_transposed=wt)
        if mod.scaling == "delayed":
            if not mod._seeded_fwd:
                _seed_history(mod.hist_x, x2d)
                _seed_history(mod.hist_w, weight)
                mod._seeded_fwd = True
            fp8_scaled_linear_fwd_delayed(x2d, weight, saved, mod.hist_x, mod.hist_w, y, OUT_BF16)
        else:
            fp8_scaled_linear_fwd(x2d, weight, saved, y, OUT_BF16)
        ctx.save_for_backward(*saved.tensors())
        return y

    @staticmethod
    def backward(ctx, gy: torch.Tensor):
        M, N, K = ctx.dims
        mod = ctx.mod
        if gy.dtype != torch.bfloat16:
            raise TypeError(f"Float8Linear expects bf16 output gradients, got {gy.dtype}")
        gy = gy.contiguous()
        gx = torch.empty((M, K), dtype=torch.bfloat16, device=gy.device)
        gw = torch.empty((N, K), dtype=torch.bfloat16, device=gy.device)
        if mod.scaling == "rowwise":
            saved = LinearSavedRW(M, N, K, tensors=ctx.saved_tensors)
            fp8_scaled_linear_bwd_rowwise(gy, saved, mod._bwd_scratch(M, N, gy.device, True), gx,
                                          gw, OUT_BF16)
            return gx, gw, None
        saved = LinearSaved(M, N, K, tensors=ctx.saved_tensors)
        ws = mod._bwd_scratch(M, N, gy.device, False, fp8_linear_copies(M, N, K)[2])
        if mod.scaling == "delayed":
            if not mod._seeded_bwd:
                _seed_history(mod.hist_gy, gy)
                mod._seeded_bwd = True
            fp8_scaled_linear_bwd_delayed(gy, saved, ws, mod.hist_gy, gx, gw, OUT_BF16)
        else:
            fp8_scaled_linear_bwd(gy, saved, ws, gx, gw, OUT_BF16)
        return gx, gw, None


class _Fp8LinearF16Fn(torch.autograd.Function):
    """y = x W^T for an fp16 model under loss scaling [PT-CH20 §20.2.2; FP8-TRAIN
    §2, §4]: fp16 x and W cast to e4m3, the GEMMs in FP8, fp16 y and
    gradients.  The output gradient carries the loss scale; the input gradient
    keeps it (it flows to the layers below), the weight gradient leaves the
    wgrad GEMM unscaled and checked when a GradScaler is attached (its scale and
    non-finite flag), and the scaler then skips that gradient in unscale_."""

    @staticmethod
    def forward(ctx, x2d: torch.Tensor, weight: torch.Tensor, mod: "Float8Linear"):
        M, K = x2d.shape
        N = weight.shape[0]
        xt, wt, _ = fp8_linear_copies(M, N, K)
        saved = LinearSaved(M, N, K, device=x2d.device, x_transposed=xt, w_transposed=wt)
        fp8_amax_f16(x2d, saved.x_sc)
        fp8_quantize_f16(x2d, E4M3FN, saved.x_sc, saved.x_q, saved.x_qT)
        fp8_amax_f16(weight, saved.w_sc)
        fp8_quantize_f16(weight, E4M3FN, saved.w_sc, saved.w_q, saved.w_qT)
        y = torch.empty((M, N), dtype=torch.float16, device=x2d.device)
        fp8_gemm(saved.x_q, E4M3FN, saved.w_q, E4M3FN, saved.x_sc.inv_ptr(), saved.w_sc.inv_ptr(), y,
                 OUT_F16)
        ctx.mod = mod
        ctx.dims = (M, N, K)
        ctx.save_for_backward(*saved.tensors())
        return y

    @staticmethod
    def backward(ctx, gy: torch.Tensor):
        M, N, K = ctx.dims
        mod = ctx.mod
        if gy.dtype != torch.float16:
            raise TypeError(f"an fp16 Float8Linear expects fp16 output gradients, got {gy.dtype}")
        gy = gy.contiguous()
        saved = LinearSaved(M, N, K, tensors=ctx.saved_tensors)
        ws = mod._bwd_scratch(M, N, gy.device, False, fp8_linear_copies(M, N, K)[2])
        fp8_amax_f16(gy, ws.gy_sc)
        fp8_quantize_f16(gy, E5M2, ws.gy_sc, ws.gy_q, ws.gy_qT)
        # an operand without its transposed copy is read contraction-major
        wk, gk, xk = saved.w_qT is None, ws.gy_qT is None, saved.x_qT is None
        gx = torch.empty((M, K), dtype=torch.float16, device=gy.device)
        fp8_gemm_kmajor(ws.gy_q, E5M2, False, saved.w_q if wk else saved.w_qT, E4M3FN, wk,
                        ws.gy_sc.inv_ptr(), saved.w_sc.inv_ptr(), gx, OUT_F16)
        gw = torch.empty((N, K), dtype=torch.float16, device=gy.device)
        a, b = (ws.gy_q if gk else ws.gy_qT), (saved.x_q if xk else saved.x_qT)
        scaler = mod.grad_scaler
        if scaler is not None:
            fp8_gemm_kmajor_unscale(a, E5M2, gk, b, E4M3FN, xk, ws.gy_sc.inv_ptr(),
                                    saved.x_sc.inv_ptr(), scaler._scale, scaler._found, gw)
            scaler._mark_unscaled(mod.weight)
        else:
            fp8_gemm_kmajor(a, E5M2, gk, b, E4M3FN, xk, ws.gy_sc.inv_ptr(), saved.x_sc.inv_ptr(),
                            gw, OUT_F16)
        return gx, gw, None


class Float8Linear(nn.Module):
    """nn.Linear (no bias) whose forward and backward GEMMs run in FP8 with
    per-tensor scaling, "dynamic" (scale from the current tensor) or
    "delayed" (scale from an amax history of history_len earlier steps), or
    with "rowwise" scaling (one scale per row of every operand along the
    dimension its GEMM does not contract).

    dtype torch.float16 makes an fp16 layer for an fp16 model under loss
    scaling (dynamic scaling): fp16 inputs, weight, output and gradients; with
    attach_grad_scaler(scaler), its weight gradient is unscaled and checked in
    the wgrad GEMM's epilogue."""

    def __init__(self, in_features: int, out_features: int, scaling: str = "dynamic",
                 history_len: int = 16, device=None, dtype=torch.bfloat16):
        super().__init__()
        if scaling not in SCALINGS:
            raise ValueError(f"scaling must be one of {SCALINGS}, not {scaling!r}")
        if dtype not in (torch.bfloat16, torch.float16):
            raise TypeError(f"Float8Linear takes bf16 or fp16, not {dtype}")
        if dtype == torch.float16 and scaling != "dynamic":
            raise ValueError("an fp16 Float8Linear uses dynamic scaling")
        self.in_features, self.out_features = in_features, out_features
        self.scaling = scaling
        self.grad_scaler = None
        self.weight = nn.Parameter(torch.empty((out_features, in_features), dtype=dtype,
                                               device=device))
        if scaling == "delayed":
            for name in ("hist_x", "hist_w", "hist_gy"):
                self.register_buffer(name, torch.zeros(history_len, dtype=torch.float32,
                                                       device=device))
        self._seeded_fwd = self._seeded_bwd = False
        self._ws = None

    def _bwd_scratch(self, M, N, device, rowwise, transposed=True):
        """The quantized gradient of the backward pass, kept across steps (its
        contents are written and consumed inside one backward call on the
        current stream, so calls on one stream can share it)."""
        key = (M, N, str(device), rowwise, transposed)
        if self._ws is None or self._ws[0] != key:
            ws = LinearBwdWsRW(M, N, device=device) if rowwise else \
                LinearBwdWs(M, N, device=device, transposed=transposed)
            self._ws = (key, ws)
        return self._ws[1]

    def attach_grad_scaler(self, scaler: "GradScaler") -> "Float8Linear":
        """fp16 layers: unscale and check the weight gradient in the wgrad GEMM
        with this scaler's scale and flag (the scaler's unscale_ then skips it)."""
        if self.weight.dtype != torch.float16:
            raise TypeError("the fused unscale serves fp16 layers (fp16 gradients)")
        self.grad_scaler = scaler
        return self

    @classmethod
    def from_float(cls, lin: nn.Linear, scaling: str = "dynamic",
                   history_len: int = 16) -> "Float8Linear":
        """A Float8Linear sharing lin's weight tensor (no copy); an fp16 weight
        makes an fp16 layer."""
        if lin.bias is not None:
            raise ValueError("Float8Linear has no bias")
        if lin.weight.dtype not in (torch.bfloat16, torch.float16):
            raise TypeError(f"Float8Linear needs a bf16 or fp16 weight, got {lin.weight.dtype}")
        with torch.device("meta"):
            new = cls(lin.in_features, lin.out_features, scaling, history_len,
                      dtype=lin.weight.dtype)
        new.weight = lin.weight
        new._ws = None
        if scaling == "delayed":
            for name in ("hist_x", "hist_w", "hist_gy"):
                setattr(new, name, torch.zeros(history_len, dtype=torch.float32,
                                               device=lin.weight.device))
        return new

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.dtype != self.weight.dtype:
            raise TypeError(f"Float8Linear takes inputs of its weight's dtype {self.weight.dtype}")
        lead = x.shape[:-1]
        x2d = x.reshape(-1, self.in_features).contiguous()
        if self.weight.dtype == torch.float16:
            y = _Fp8LinearF16Fn.apply(x2d, self.weight, self)
        elif self.scaling == "dynamic":
            y = torch.ops.fp8sg.scaled_linear_fwd(x2d, self.weight)[0]
        else:
            y = _Fp8LinearFn.apply(x2d, self.weight, self)
        return y.reshape(*lead, self.out_features)

    def extra_repr(self):
        return f"in_features={self.in_features}, out_features={self.out_features}, " \
               f"scaling={self.scaling}"


# Layers kept in high precision by name [FP8-TRAIN §8: the output head and the
# MoE router, where FP8 costs more convergence than it saves time]: the last
# component of the fully qualified name.
HIGH_PRECISION_NAMES = ("lm_head", "output", "router")


def default_module_filter(mod: nn.Linear, fqn: str) -> bool:
    """Convert a linear layer when the FP8 path can take it (bf16 weight, no
    bias, in and out features multiples of 16) and its name does not mark it as
    the output head or a MoE router."""
    last = fqn.rsplit(".", 1)[-1]
    return (mod.bias is None and mod.weight.dtype in (torch.bfloat16, torch.float16) and
            mod.in_features % 16 == 0 and mod.out_features % 16 == 0 and
            last not in HIGH_PRECISION_NAMES)


def convert_to_float8_training(model: nn.Module,
                               module_filter_fn: Optional[Callable[[nn.Module, str], bool]] = None,
                               scaling: str = "dynamic", history_len: int = 16,
                               grad_scaler: Optional["GradScaler"] = None) -> nn.Module:
    """Replace, in place and post-order, every nn.Linear child that
    module_filter_fn(child, fully_qualified_name) accepts (default:
    default_module_filter) with a Float8Linear sharing its weight.  With
    grad_scaler, the fp16 layers unscale and check their weight gradients in
    the wgrad GEMM's epilogue with that scaler."""
    accept = module_filter_fn or default_module_filter
    # every (parent, attribute, module, dotted path) below the root, each
    # module after all of its own descendants; the swaps are made after the
    # walk, so it never iterates over a tree it is changing
    edges = list(_descendants_post_order(model, ()))
    for parent, attr, child, path in edges:
        if type(child) is nn.Linear and accept(child, ".".join(path)):
            new = Float8Linear.from_float(child, scaling, history_len)
            if grad_scaler is not None and new.weight.dtype == torch.float16:
                new.attach_grad_scaler(grad_scaler)
            setattr(parent, attr, new)
    return model


def _descendants_post_order(mod: nn.Module, path: tuple):
    for attr, child in mod.named_children():
        yield from _descendants_post_order(child, path + (attr,))
        yield mod, attr, child, path + (attr,)


class GradScaler:
    """Dynamic loss scaling for fp16 gradients with the scale, growth tracker
    and non-finite flag kept on the device.  scale(loss) multiplies by the
    current scale; unscale_(optimizer) unscales the optimizer's gradients in
    place and checks them (optionally also returning their global 2-norm, for
    clipping); step(optimizer) runs optimizer.step() unless a gradient was
    inf/NaN (this reads the flag: one host synchronisation, as in PyTorch's
    GradScaler); update() applies the halve-on-inf / grow-after-interval rule
    and clears the flag."""

    def __init__(self, init_scale: float = 2.0 ** 16, growth_factor: float = 2.0,
                 backoff_factor: float = 0.5, growth_interval: int = 2000, device="cuda"):
        self._scale = torch.tensor([init_scale], dtype=torch.float32, device=device)
        self._tracker = torch.zeros(1, dtype=torch.int32, device=device)
        self._found = torch.zeros(1, dtype=torch.int32, device=device)
        self.growth_factor, self.backoff_factor = growth_factor, backoff_factor
        self.growth_interval = growth_interval
        self._unscaled = set()
        self._pre_unscaled = set()  # parameters whose gradient a layer unscaled this step

    def scale(self, loss: torch.Tensor) -> torch.Tensor:
        # a 0-dim fp32 factor: torch's promotion keeps the loss's own dtype
        # unless it is lower, as PyTorch's GradScaler does
        return loss * self._scale.view(())

    def _mark_unscaled(self, param):
        """An fp16 Float8Linear wrote param's gradient already unscaled and
        checked (wgrad epilogue): unscale_ leaves it alone this step."""
        self._pre_unscaled.add(id(param))

    def _grads(self, optimizer):
        gs = []
        for group in optimizer.param_groups:
            for p in group["params"]:
                if p.grad is None or id(p) in self._pre_unscaled:
                    continue
                if p.grad.dtype != torch.float16 or not p.grad.is_contiguous():
                    raise TypeError("GradScaler unscales contiguous fp16 gradients only")
                gs.append(p.grad)
        return gs

    def unscale_(self, optimizer, with_norm: bool = False):
        """Unscale and check the optimizer's gradients once per step.  With
        with_norm, returns a device float32[2]: (sum of squares, 2-norm) of the
        unscaled gradients taken together."""
        if id(optimizer) in self._unscaled:
            raise RuntimeError("unscale_() has already been called on this optimizer this step")
        grads = self._grads(optimizer)
        self._unscaled.add(id(optimizer))
        if not with_norm:
            amp_unscale_check(grads, self._scale, self._found)
            return None
        ws = torch.empty(amp_norm_workspace_len([g.numel() for g in grads]), dtype=torch.float32,
                         device=self._scale.device)
        out = torch.empty(2, dtype=torch.float32, device=self._scale.device)
        amp_unscale_check_norm(grads, self._scale, self._found, ws, out)
        return out

    def step(self, optimizer, *args, **kwargs):
        if id(optimizer) not in self._unscaled:
            self.unscale_(optimizer)
        if int(self._found.item()) == 0:
            return optimizer.step(*args, **kwargs)
        return None

    def update(self):
        amp_update_scale(self._scale, self._tracker, self._found, self.growth_factor,
                         self.backoff_factor, self.growth_interval)
        self._unscaled.clear()
        self._pre_unscaled.clear()

    def get_scale(self) -> float:
        return float(self._scale.item())

    def state(self):
        """(scale, growth tracker, non-finite flag), read from the device."""
        return self.get_scale(), int(self._tracker.item()), int(self._found.item())
