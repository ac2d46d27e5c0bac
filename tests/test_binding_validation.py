"""The Python binding rejects mismatched shapes and dtypes before any pointer
reaches the C ABI (which cannot see sizes behind raw pointers). CPU only: the
checks run before the device check, so host tensors with bad shapes exercise
them without a GPU."""
from __future__ import annotations

import pytest
import torch

import test_layer_amd as tla

H, D, M = 4, 64, 128
N = 96


def _tok(n=N, c=H * D, dtype=torch.bfloat16):
    return torch.zeros((n, c), dtype=dtype)


def _theta(h=H, dtype=torch.float32):
    return torch.zeros((h, 3 * D * M), dtype=dtype)


@pytest.mark.parametrize("fn", ["write", "grad", "partials"])
def test_write_family_rejects_mismatched_operands(fn):
    def call(K, Vp, theta, **kw):
        if fn == "write":
            return tla.ttt_write(K, Vp, theta, 0.1, 2, H, **kw)
        if fn == "grad":
            return tla.ttt_grad(K, Vp, theta, H, **kw)
        return tla.ttt_grad_partials(K, Vp, theta, H, workspace=torch.zeros(16, dtype=torch.uint8))

    with pytest.raises(ValueError, match="Vp"):
        call(_tok(), _tok(n=N + 1), _theta())
    with pytest.raises(ValueError, match="Vp"):
        call(_tok(), _tok(dtype=torch.float32), _theta())
    with pytest.raises(ValueError, match="theta"):
        call(_tok(), _tok(), _theta(dtype=torch.float64))
    with pytest.raises(ValueError, match="theta"):
        call(_tok(), _tok(), torch.zeros((H, 3 * D * M + 1)), d_hidden=M) if fn != "partials" else \
            tla.ttt_grad_partials(_tok(), _tok(), torch.zeros((H, 3 * D * M + 1)), H,
                                  workspace=torch.zeros(16, dtype=torch.uint8), d_hidden=M)
    with pytest.raises(ValueError, match="2-D"):
        call(_tok().view(N, H, D), _tok().view(N, H, D), _theta())


def test_loss_and_grad_outputs_are_sized():
    with pytest.raises(ValueError, match="loss_out"):
        tla.ttt_write(_tok(), _tok(), _theta(), 0.1, 2, H, loss_out=torch.zeros(2 * H - 1))
    with pytest.raises(ValueError, match="loss_out"):
        tla.ttt_write(_tok(), _tok(), _theta(), 0.1, 2, H, loss_out=torch.zeros(2 * H, dtype=torch.float64))
    with pytest.raises(ValueError, match="loss_out"):
        tla.ttt_grad(_tok(), _tok(), _theta(), H, loss_out=torch.zeros(H - 1))
    with pytest.raises(ValueError, match="grad"):
        tla.ttt_grad(_tok(), _tok(), _theta(), H, grad=torch.zeros(H * 3 * D * M - 1))
    with pytest.raises(ValueError, match="grad"):
        tla.ttt_apply(_theta(), torch.zeros(H * 3 * D * M, dtype=torch.float16), 0.1, H, D, M)
    with pytest.raises(ValueError, match="theta"):
        tla.ttt_apply(_theta(h=H - 1), torch.zeros(H * 3 * D * M), 0.1, H, D, M)
    with pytest.raises(ValueError, match="grad"):
        tla.ttt_muon_apply(_theta(), torch.zeros(3), 0.1, H, D, M)
    with pytest.raises(ValueError, match="dst"):
        tla.ttt_reduce(torch.zeros(16, dtype=torch.uint8), N, H, D, M, tla.BF16, tla.REDUCE_STORE,
                       torch.zeros(5))


def test_read_rejects_mismatched_output_and_theta():
    with pytest.raises(ValueError, match="out"):
        tla.ttt_read(_tok(), _theta(), H, out=_tok(n=N - 1))
    with pytest.raises(ValueError, match="out"):
        tla.ttt_read(_tok(), _theta(), H, out=_tok(dtype=torch.float32))
    with pytest.raises(ValueError, match="theta"):
        tla.ttt_read(_tok(), _theta(h=H + 1), H, d_hidden=M)


def test_shortconv_rejects_layout_mismatch():
    n_views, gh, gw, ns = 2, 4, 5, 1
    n = n_views * (ns + gh * gw)
    w = torch.zeros((H * D, 3, 3))
    with pytest.raises(ValueError, match="tokens"):
        tla.shortconv(_tok(n=n + 1), w, n_views, gh, gw, ns)
    with pytest.raises(ValueError, match="channels"):
        tla.shortconv(_tok(n=n), torch.zeros((H * D - 8, 3, 3)), n_views, gh, gw, ns)
    with pytest.raises(ValueError, match="out"):
        tla.shortconv(_tok(n=n), w, n_views, gh, gw, ns, out=_tok(n=n - 1))
    with pytest.raises(TypeError):
        tla.shortconv(_tok(n=n), torch.zeros((H * D, 3, 3), dtype=torch.float64), n_views, gh, gw, ns)


def test_streamed_calls_reject_mismatched_operands():
    with pytest.raises(ValueError, match="Vp_host"):
        tla.ttt_write_streamed(_tok(), _tok(n=N - 1), _theta(), 0.1, 1, H, 32)
    with pytest.raises(ValueError, match="theta"):
        tla.ttt_write_streamed(_tok(), _tok(), _theta(h=1), 0.1, 1, H, 32, d_hidden=M)
    with pytest.raises(ValueError, match="out"):
        tla.ttt_read_streamed(_tok(), _theta(), H, 32, out=_tok(n=N + 3))


def test_well_formed_host_tensors_reach_the_device_check():
    """With consistent shapes the only complaint left for host tensors is that
    they are not on the GPU."""
    with pytest.raises(ValueError, match="GPU"):
        tla.ttt_write(_tok(), _tok(), _theta(), 0.1, 2, H, loss_out=torch.zeros(2 * H))
    with pytest.raises(ValueError, match="GPU"):
        tla.ttt_read(_tok(), _theta(), H, out=_tok())
