"""The layer oracle against its pins, and planted mistakes in copies of it
that the pins must catch. Runs without a GPU."""
import os
import types

import pytest

import layer_pins
import oracle
from oracle import layer as oracle_layer

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCE = os.path.join(ROOT, "oracle", "layer.py")


@pytest.mark.parametrize("pin", layer_pins.ALL_LAYER_PINS, ids=lambda p: p.__name__)
def test_layer_pin(pin):
    pin(oracle_layer)


MUTANTS = {
    "offsets_viewed_levels_first": (
        ".astype(np.float32).reshape(so)",
        ".astype(np.float32).reshape(B, Nq, L, M, K, 2).transpose(0, 1, 3, 2, 4, 5).copy()"),
    "logits_without_bias": ('linear_forward(query, p["w_attn"], p["b_attn"])',
                            'linear_forward(query, p["w_attn"], None)'),
    "value_weight_transposed": ('value = linear_forward(inp, p["w_value"], p["b_value"])',
                                'value = linear_forward(inp, p["w_value"].T, p["b_value"])'),
    "query_grad_drops_logit_head": ('g["query"] = gq1 + gq2', 'g["query"] = gq1'),
    "output_bias_grad_from_core_grad": ('dcore, g["w_out"], g["b_out"] = linear_backward(core, p["w_out"], gy)',
                                        'dcore, g["w_out"], _ = linear_backward(core, p["w_out"], gy)\n'
                                        '    g["b_out"] = dcore.reshape(-1, C).sum(0)'),
    "weight_grad_transposed_operands": ("gw = g2.T @ x2", "gw = (x2.T @ g2).T * 0 + g2.T @ x2[::-1]"),
    "input_grad_uses_weight_transpose": ("gx = (g2 @ w).reshape(x.shape)",
                                         "gx = (g2 @ w[::-1]).reshape(x.shape)"),
    "bias_grad_mean": ("gb = g2.sum(0)", "gb = g2.mean(0)"),
}


def _mutant_module(old, new):
    src = open(SOURCE).read()
    assert old in src, "mutation site not found"
    src = src.replace(old, new).replace("from . import backward_fused, forward_fused",
                                        "from oracle import backward_fused, forward_fused")
    mod = types.ModuleType("oracle_layer_mutant")
    exec(compile(src, "oracle_layer_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_layer_pins_catch_mutant(name):
    mod = _mutant_module(*MUTANTS[name])
    caught = None
    for pin in layer_pins.ALL_LAYER_PINS:
        try:
            pin(mod)
        except Exception as e:   # any failure of a pin counts as caught
            caught = (pin.__name__, type(e).__name__)
            break
    assert caught is not None, f"mutant {name} survived every layer pin"


def test_oracle_package_is_importable():
    assert callable(oracle.forward_fused)
