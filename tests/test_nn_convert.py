"""convert_to_float8_training's module surgery ["FP8训练：量化、自动微分、
Torchao", §8]: post-order walk, nn.Linear children replaced in place when the
filter accepts (module, fully qualified name), the replacement sharing the
original weight tensor.  Pure module-tree logic: no kernels run."""
import torch
from torch import nn

from fp8_scaled_gemm_amd.nn import Float8Linear, convert_to_float8_training, default_module_filter


def lin(i, o, bias=False):
    return nn.Linear(i, o, bias=bias, dtype=torch.bfloat16)


class Block(nn.Module):
    def __init__(self):
        super().__init__()
        self.gate, self.up, self.down = lin(64, 128), lin(64, 128), lin(128, 64)
        self.router = lin(64, 16)
        self.norm = nn.LayerNorm(64)


class Model(nn.Module):
    def __init__(self):
        super().__init__()
        self.embed = nn.Embedding(100, 64)
        self.blocks = nn.ModuleList([Block(), Block()])
        self.proj = lin(64, 64, bias=True)     # biased: the default filter leaves it
        self.lm_head = lin(64, 100)            # 100 outputs: not a multiple of 16


def test_default_filter_converts_what_the_path_takes():
    m = Model()
    w = {n: p for n, p in m.named_parameters()}
    convert_to_float8_training(m)
    for b in m.blocks:
        for name in ("gate", "up", "down"):
            assert isinstance(getattr(b, name), Float8Linear)
        # a MoE router stays in high precision by name (the page's section 8)
        assert type(b.router) is nn.Linear
        assert isinstance(b.norm, nn.LayerNorm)
    assert type(m.proj) is nn.Linear and type(m.lm_head) is nn.Linear
    # the weights are the original tensors, not copies
    assert m.blocks[1].down.weight is w["blocks.1.down.weight"]
    assert m.blocks[0].gate.weight.data_ptr() == w["blocks.0.gate.weight"].data_ptr()


def test_filter_sees_fully_qualified_names_post_order():
    m = Model()
    seen = []

    def keep_router_out(mod, fqn):
        seen.append(fqn)
        return default_module_filter(mod, fqn) and not fqn.endswith("router")

    convert_to_float8_training(m, keep_router_out)
    assert seen == ["blocks.0.gate", "blocks.0.up", "blocks.0.down", "blocks.0.router",
                    "blocks.1.gate", "blocks.1.up", "blocks.1.down", "blocks.1.router",
                    "proj", "lm_head"]
    assert type(m.blocks[0].router) is nn.Linear and isinstance(m.blocks[0].gate, Float8Linear)


def test_delayed_modules_carry_histories():
    m = Block()
    convert_to_float8_training(m, scaling="delayed", history_len=8)
    for name in ("gate", "up", "down"):
        f = getattr(m, name)
        assert f.scaling == "delayed"
        assert all(getattr(f, h).shape == (8,) and getattr(f, h).dtype == torch.float32
                   for h in ("hist_x", "hist_w", "hist_gy"))
    assert set(dict(m.named_buffers())) >= {"gate.hist_x", "down.hist_gy"}


def test_default_filter_keeps_output_head_and_router_by_name():
    # sizes the path takes, names that mark the layers kept in high precision
    assert default_module_filter(lin(64, 128), "blocks.3.mlp.up")
    assert not default_module_filter(lin(64, 128), "lm_head")
    assert not default_module_filter(lin(64, 128), "model.output")
    assert not default_module_filter(lin(64, 16), "layers.2.moe.router")
    assert default_module_filter(lin(64, 16), "layers.2.router_proj.weight_like")  # last part only


def test_from_float_refuses_what_the_path_cannot_take():
    import pytest
    with pytest.raises(ValueError):
        Float8Linear.from_float(lin(32, 32, bias=True))
    with pytest.raises(TypeError):
        Float8Linear.from_float(nn.Linear(32, 32, bias=False))  # fp32 weight


def test_scaling_modes():
    for scaling in ("dynamic", "delayed", "rowwise"):
        m = convert_to_float8_training(Model(), scaling=scaling)
        assert m.blocks[0].gate.scaling == scaling
        assert hasattr(m.blocks[0].gate, "hist_x") == (scaling == "delayed")
    try:
        Float8Linear(16, 16, scaling="blockwise")
    except ValueError:
        pass
    else:
        raise AssertionError("unknown scaling accepted")


def test_dynamo_captures_the_fp8_linear_as_one_op():
    """torch.compile with fullgraph traces a converted MLP without a graph
    break; the captured graph holds the fp8sg::scaled_linear_fwd operator (an
    opaque call) for each linear.  Tracing only: the backend records the graph
    and never runs it (no GPU here)."""
    graphs = []

    def record(gm, example_inputs):
        graphs.append(gm)
        return lambda *args: (torch.zeros(32, 64, dtype=torch.bfloat16),)

    class Mlp(nn.Module):
        def __init__(self):
            super().__init__()
            self.up, self.down = lin(64, 128), lin(128, 64)

        def forward(self, x):
            return self.down(torch.relu(self.up(x)))

    m = convert_to_float8_training(Mlp())
    torch._dynamo.reset()
    torch.compile(m, backend=record, fullgraph=True)(torch.empty(32, 64, dtype=torch.bfloat16))
    assert len(graphs) == 1
    targets = [str(n.target) for n in graphs[0].graph.nodes if n.op == "call_function"]
    assert sum("fp8sg.scaled_linear_fwd" in t for t in targets) == 2, targets


def test_backward_gets_no_zero_filled_code_gradients():
    """The dynamic-scaling op returns y plus the codes and records the
    backward needs.  Those are state, not differentiable outputs: the autograd
    setup turns off gradient materialization, so the backward receives None
    for them rather than a zero-filled tensor of each code's size (one fill
    kernel per tensor, up to 117 MB each in the MLP block).  A backward whose
    y took no part in the loss returns no gradients.  Host logic only: a
    recording context stands in for autograd's."""
    import fp8_scaled_gemm_amd.nn as FN

    class Ctx:
        def __init__(self):
            self.saved, self.materialize = None, True

        def save_for_backward(self, *t):
            self.saved = t

        def set_materialize_grads(self, v):
            self.materialize = v

    ctx = Ctx()
    outs = (torch.empty(32, 64, dtype=torch.bfloat16),) + tuple(
        torch.empty(n, dtype=torch.uint8) for n in (2048, 0, 4096, 0, 8))
    FN._op_setup(ctx, (None, None), outs)
    assert ctx.materialize is False
    assert len(ctx.saved) == 5 and all(a is b for a, b in zip(ctx.saved, outs[1:]))
    assert FN._op_backward(ctx, None, None, None, None, None, None) == (None, None)
