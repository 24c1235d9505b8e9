"""MoeLayer validates every tensor it is given before anything is enqueued
(CPU only).  The library loader is replaced by one that fails the test, so
an argument that slipped past the checks would show up as that failure
rather than as a device call."""
import pytest
import torch

import mxfp4_grouped_expert_amd as moe
from mxfp4_grouped_expert_amd import binding as B
from mxfp4_grouped_expert_amd.layer import MoeLayer

E, H, I, K = 4, 64, 96, 2


@pytest.fixture(autouse=True)
def _no_library_calls(monkeypatch):
    def fail():
        raise AssertionError("the library was called with an invalid argument")
    monkeypatch.setattr(B, "load", fail)


def _weights(**over):
    w = dict(w_router=torch.zeros(E, H, dtype=torch.float32), bias=None,
             w13_q=torch.zeros(E, 2 * I, H // 2, dtype=torch.uint8),
             w13_s=torch.zeros(E, 2 * I, H // 32, dtype=torch.uint8),
             w2_q=torch.zeros(E, H, I // 2, dtype=torch.uint8),
             w2_s=torch.zeros(E, H, I // 32, dtype=torch.uint8))
    w.update(over)
    return w


def _make(**over):
    w = _weights(**over)
    return MoeLayer(w["w_router"], w["bias"], w["w13_q"], w["w13_s"], w["w2_q"], w["w2_s"], K,
                    layout="canonical")


@pytest.mark.parametrize("over,msg", [
    (dict(w_router=torch.zeros(E, H + 32, dtype=torch.float32)), "w_router has shape"),
    (dict(w_router=torch.zeros(E, H, dtype=torch.float64)), "w_router has dtype"),
    (dict(w_router=torch.zeros(H, E, dtype=torch.float32).t()), "contiguous"),
    (dict(bias=torch.zeros(E + 1, dtype=torch.float32)), "device tensor"),  # w_router first
    (dict(w13_s=torch.zeros(E, 2 * I, H // 16, dtype=torch.uint8)), "device tensor"),
])
def test_constructor_rejects_bad_weights(over, msg):
    with pytest.raises(ValueError, match=msg):
        _make(**over)


def test_constructor_rejects_bad_k_and_dims():
    w = _weights()
    with pytest.raises(ValueError, match="k must"):
        MoeLayer(w["w_router"], None, w["w13_q"], w["w13_s"], w["w2_q"], w["w2_s"], E + 1)
    with pytest.raises(ValueError, match="multiples of 32"):
        MoeLayer(w["w_router"], None, torch.zeros(E, 2 * 40, H // 2, dtype=torch.uint8),
                 w["w13_s"], w["w2_q"], w["w2_s"], K)
    with pytest.raises(ValueError, match="w13_q"):
        MoeLayer(w["w_router"], None, torch.zeros(E, H, dtype=torch.uint8), w["w13_s"],
                 w["w2_q"], w["w2_s"], K)


def _bare_layer():
    # a layer whose weights were accepted (the device check is what a CPU
    # tensor fails, so the rest of the state is filled in by hand)
    layer = MoeLayer.__new__(MoeLayer)
    layer.E, layer.H, layer.I, layer.k = E, H, I, K
    layer.device = torch.device("cuda:0")
    layer.T = None
    return layer


@pytest.mark.parametrize("x,msg", [
    (torch.zeros(3, H - 32, dtype=torch.bfloat16), "x has shape"),       # too narrow: read past x
    (torch.zeros(3, H, dtype=torch.float32), "x has dtype"),
    (torch.zeros(H, 3, dtype=torch.bfloat16).t(), "contiguous"),      # a transposed view
    (torch.zeros(3, 2 * H, dtype=torch.bfloat16)[:, ::2], "contiguous"),
    (torch.zeros(3, H, 1, dtype=torch.bfloat16), "bf16 tensor"),
    (torch.zeros(3, H, dtype=torch.bfloat16), "device tensor"),
])
def test_call_rejects_malformed_x_before_enqueueing(x, msg):
    layer = _bare_layer()
    with pytest.raises(ValueError, match=msg):
        layer(x)
    with pytest.raises(ValueError, match=msg):
        layer.route_only(x)
    assert layer.T is None  # nothing was planned either


def test_int16_bits_pass_the_dtype_check():
    layer = _bare_layer()
    with pytest.raises(ValueError, match="device tensor"):  # dtype and shape accepted
        layer(torch.zeros(2, H, dtype=torch.int16))


def test_package_exports_the_layer():
    assert moe.MoeLayer is MoeLayer
