"""The torch layer rejects mismatched tensors before the library is called (CPU only).

The device check and the library calls are replaced by stubs, so CPU tensors
stand in for device tensors and any call that reached the library would fail
the test.
"""
import pytest
import torch

from exact_attention_forward_amd import api


@pytest.fixture
def stubbed(monkeypatch):
    calls = []
    monkeypatch.setattr(api, "_on_device", lambda t: True)
    monkeypatch.setattr(api, "_stream", lambda dev: None)
    monkeypatch.setattr(api._b, "fa_forward", lambda *a: calls.append("fwd") or 0)
    monkeypatch.setattr(api._b, "fa_backward", lambda *a: calls.append("bwd") or 0)
    return calls


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def test_well_formed_calls_reach_the_library(stubbed):
    q, k, v, do = (t(1, 8, 2, 64) for _ in range(4))
    o, lse = api.forward(q, k, v)
    assert o.dtype == torch.float32 and o.shape == (1, 8, 2, 64) and lse.shape == (1, 2, 8)
    api.backward(q, k, v, o, lse, do)
    assert stubbed == ["fwd", "bwd"]


@pytest.mark.parametrize("which", [1, 2])
def test_forward_dtype_mismatch(stubbed, which):
    args = [t(1, 8, 2, 64) for _ in range(3)]
    args[which] = t(1, 8, 2, 64, dtype=torch.float32)
    with pytest.raises(TypeError):
        api.forward(*args)
    assert stubbed == []


def test_forward_shape_and_layout(stubbed):
    with pytest.raises(ValueError):
        api.forward(t(1, 8, 2, 64), t(1, 8, 2, 64), t(1, 9, 2, 64))
    with pytest.raises(ValueError):
        api.forward(t(1, 8, 2, 64), t(1, 8, 2, 64), t(1, 2, 8, 64).transpose(1, 2))
    with pytest.raises(ValueError):
        api.forward(t(8, 2, 64), t(8, 2, 64), t(8, 2, 64))
    with pytest.raises(TypeError):
        api.forward(*(t(1, 8, 2, 64, dtype=torch.float64) for _ in range(3)))
    assert stubbed == []


def test_backward_checks_do_o_and_lse(stubbed):
    q, k, v = (t(1, 8, 2, 64) for _ in range(3))
    o, lse = t(1, 8, 2, 64, dtype=torch.float32), t(1, 2, 8, dtype=torch.float32)
    with pytest.raises(TypeError):  # dO of another dtype
        api.backward(q, k, v, o, lse, t(1, 8, 2, 64, dtype=torch.float16))
    with pytest.raises(TypeError):  # o not float32
        api.backward(q, k, v, t(1, 8, 2, 64), lse, t(1, 8, 2, 64))
    with pytest.raises(ValueError):  # o of another shape
        api.backward(q, k, v, t(1, 8, 2, 32, dtype=torch.float32), lse, t(1, 8, 2, 64))
    with pytest.raises(ValueError):  # lse laid out [B, T, H]
        api.backward(q, k, v, o, t(1, 8, 2, dtype=torch.float32), t(1, 8, 2, 64))
    with pytest.raises(TypeError):  # lse not float32
        api.backward(q, k, v, o, t(1, 2, 8), t(1, 8, 2, 64))
    with pytest.raises(ValueError):  # lse not contiguous
        api.backward(q, k, v, o, t(1, 8, 2, dtype=torch.float32).transpose(1, 2), t(1, 8, 2, 64))
    assert stubbed == []


def test_device_tensors_required():
    with pytest.raises(ValueError):
        api.forward(*(t(1, 8, 2, 64) for _ in range(3)))


def test_attention_runs_forward_then_backward_with_the_saved_outputs(stubbed):
    q, k, v = (t(1, 8, 2, 64).requires_grad_() for _ in range(3))
    o = api.attention(q, k, v)
    assert stubbed == ["fwd"] and o.dtype == torch.float32 and o.requires_grad
    o.backward(torch.ones_like(o))
    assert stubbed == ["fwd", "bwd"]
    for x in (q, k, v):
        assert x.grad is not None and x.grad.dtype == torch.bfloat16 and x.grad.shape == x.shape
