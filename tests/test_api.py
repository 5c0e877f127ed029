"""Host-side checks of the rwkv-ops-shaped entry points
(rwkv_linear_attention_amd/api.py): they refuse what they do not serve
before any library call, and the aliases the pages list are the same
functions."""
import pytest

torch = pytest.importorskip("torch")

import rwkv_linear_attention_amd as m  # noqa: E402


def cpu(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def test_aliases():
    assert m.rwkv7_op is m.generalized_delta_rule


def test_cpu_tensors_are_refused():
    x = cpu(1, 16, 1, 64)
    with pytest.raises(ValueError, match="GPU only"):
        m.generalized_delta_rule(x, x, x, x, x, x)
    g = cpu(1, 16, 1)
    with pytest.raises(ValueError, match="GPU only"):
        m.gated_delta_net(x, x, x, g, g)
    with pytest.raises(ValueError, match="GPU only"):
        m.rwkv7_op_rnn(*(cpu(1, 1, 1, 64),) * 6)


def test_head_first_is_refused():
    x = cpu(1, 16, 1, 64)
    with pytest.raises(NotImplementedError):
        m.generalized_delta_rule(x, x, x, x, x, x, head_first=True)
    with pytest.raises(NotImplementedError):
        m.gated_delta_net_recurrent(x, x, x, cpu(1, 16, 1), cpu(1, 16, 1), head_first=True)
    y = cpu(1, 1, 64)
    with pytest.raises(NotImplementedError):
        m.gated_delta_net_recurrent_single_step(y, y, y, cpu(1, 1), cpu(1, 1), head_first=False)


def test_chunk_size_must_divide_T():
    x = cpu(1, 40, 1, 64)
    with pytest.raises(ValueError, match="divide"):
        m.gated_delta_net_chunk(x, x, x, cpu(1, 40, 1), cpu(1, 40, 1), chunk_size=16)
