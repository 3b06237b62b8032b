"""State initialisation through the C ABI: W0, b0 (and W1, b1, W2, b2) tiled
over the batch, gradients zeroed, offset reset, by one launch of the
multi-segment fill kernel.  A copy, so the check is bit-exact.  Sources that
are 16-byte aligned take the float4 path, sources one float off it the scalar
path."""
import pytest
import torch

from test_rnn_layers_amd import libttt

pytestmark = pytest.mark.gpu

D, F = 64, 256


def _src(shape, offset, gen):
    """A contiguous tensor of `shape` that starts `offset` floats into a fresh allocation."""
    n = 1
    for s in shape:
        n *= s
    base = torch.randn(n + 4, generator=gen).cuda()
    t = base[offset:offset + n].view(*shape)
    assert (t.data_ptr() % 16 == 0) == (offset % 4 == 0)
    return t


@pytest.mark.parametrize("offset", [0, 1])
def test_linear_state_init(offset):
    B, H = 3, 5
    gen = torch.Generator().manual_seed(7 + offset)
    W0, b0 = _src((H, D, D), offset, gen), _src((H, D), offset, gen)
    cfg = libttt.linear_cfg(B, H)
    st = libttt.LinearState.empty(B, H, D)
    for t in (st.W, st.b, st.W_grad, st.b_grad):
        t.fill_(float("nan"))
    libttt.ttt_linear_state_init(cfg, W0, b0, st)
    torch.cuda.synchronize()
    assert torch.equal(st.W, W0.unsqueeze(0).expand(B, H, D, D))
    assert torch.equal(st.b, b0.unsqueeze(0).expand(B, H, D))
    assert not st.W_grad.any() and not st.b_grad.any() and not torch.isnan(st.W_grad).any()
    assert st.offset == 0


@pytest.mark.parametrize("offset", [0, 1])
def test_mlp_state_init(offset):
    B, H = 2, 3
    gen = torch.Generator().manual_seed(11 + offset)
    W1, b1 = _src((H, D, F), offset, gen), _src((H, F), offset, gen)
    W2, b2 = _src((H, F, D), offset, gen), _src((H, D), offset, gen)
    cfg = libttt.mlp_cfg(B, H)
    st = libttt.MlpState.empty(B, H, D, F)
    for t in st.tensors:
        t.fill_(float("nan"))
    libttt.ttt_mlp_state_init(cfg, W1, b1, W2, b2, st)
    torch.cuda.synchronize()
    for got, want in ((st.W1, W1), (st.b1, b1), (st.W2, W2), (st.b2, b2)):
        assert torch.equal(got, want.unsqueeze(0).expand(B, *want.shape))
    for g in (st.W1_grad, st.b1_grad, st.W2_grad, st.b2_grad):
        assert not g.any() and not torch.isnan(g).any()
    assert st.offset == 0
