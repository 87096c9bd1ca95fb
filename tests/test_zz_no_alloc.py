"""The no-allocation batch-1 entry point against the handle path and the oracle.

sffn_forward_sparse_noalloc keeps the gate -> down unit products in a static
device array of the library; two calls in a row (the second on a smaller
problem) must each match sffn_forward_sparse on the same inputs.
"""
import numpy as np
import pytest
import torch

from activation_sparse_gated_amd import inputs as gen
from activation_sparse_gated_amd import sffn
from oracle import reference as ref

import parity as P

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def _run_pair(D, H, T, s, act, cfg):
    x = gen.tokens(D, T, cfg=cfg, dtype="bf16")
    w = gen.standard_weights(D, H, s, cfg=cfg, dtype="bf16")
    dx = _dev(x)
    dW = {k: _dev(w[k]) for k in ("W1", "W3", "W2T")}
    y_na = torch.full((T, D), float("nan"), dtype=torch.float32, device="cuda")
    y_h = torch.empty(T, D, dtype=torch.float32, device="cuda")
    print(f"no-alloc call D={D} H={H} T={T} act={act}", flush=True)
    sffn.sffn_forward_sparse_noalloc(dx, dW["W1"], dW["W3"], dW["W2T"], y_na, D, H, T, act)
    with sffn.Handle(D, H, 0, T, act, sffn.SFFN_BF16) as h:
        sffn.sffn_forward_sparse(h.ptr, dx, dW["W1"], dW["W3"], dW["W2T"], y_h, T,
                                 sffn.SFFN_MODE_PER_TOKEN)
    torch.cuda.synchronize()
    assert torch.isfinite(y_na).all()
    # against the existing entry point: same kernels, so the same result up to the
    # order of the down pass's fp32 additions
    P.check_y(y_na, y_h.cpu().numpy().astype(np.float64), "no-alloc vs handle")
    o = ref.ffn_standard(x, w["W1"], w["W3"], w["W2T"], act=act)
    P.check_y(y_na, o["y"], "no-alloc vs oracle")


def test_noalloc_matches_handle_path_twice_second_smaller():
    sffn.load()
    _run_pair(2560, 7168, 3, 0.9, sffn.SFFN_ACT_RSPLUS, cfg=2)
    _run_pair(512, 1408, 2, 0.9, sffn.SFFN_ACT_RELU, cfg=1)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    sffn.load()
    D, H = 256, 16385
    buf = torch.zeros(4 * H * D, dtype=torch.int16, device="cuda")
    y = torch.zeros(1, D, dtype=torch.float32, device="cuda")
    st = sffn.sffn_forward_sparse_noalloc(buf, buf, buf, buf, y, D, H, 1, sffn.SFFN_ACT_RELU,
                                          check=False)
    assert st == sffn.SFFN_INVALID_ARGUMENT
    assert "16384" in sffn.sffn_last_error(None)
    st = sffn.sffn_forward_sparse_noalloc(buf, buf, buf, buf, y, 8192, 16, 1, sffn.SFFN_ACT_RELU,
                                          check=False)
    assert st == sffn.SFFN_INVALID_ARGUMENT
