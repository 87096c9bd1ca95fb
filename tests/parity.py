"""Helpers of the GPU parity tests: stage generated inputs on the device, run
the HIP path through the C ABI, and compare with the fp64 oracle."""
import numpy as np
import torch

from activation_sparse_gated_amd import inputs as gen
from activation_sparse_gated_amd import sffn

# tolerances of the contract: live sets exact except units with |z| < 1e-3;
# y within relative L2 5e-3 and max-abs 2e-2 * max|y| (bf16 weights, fp32 accumulate)
Z_BAND = 1e-3
REL_L2 = 5e-3
MAX_ABS_FRAC = 2e-2

DT = {"bf16": sffn.SFFN_BF16, "f32": sffn.SFFN_F32}


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def run_sparse(h, x, w, T, mode, want_live=True):
    D, H = h.D, h.H
    y = torch.full((T, D), float("nan"), dtype=torch.float32, device="cuda")
    cnt = torch.full((T,), -1, dtype=torch.int32, device="cuda") if want_live else None
    idx = torch.full((T, H), -1, dtype=torch.int32, device="cuda") if want_live else None
    sffn.sffn_forward_sparse(h.ptr, dev(x), dev(w["W1"]), dev(w["W3"]), dev(w["W2T"]), y, T, mode,
                             cnt, idx)
    torch.cuda.synchronize()
    return y, cnt, idx


def run_lopa(h, x, w, T, mode, want_live=True):
    D, H = h.D, h.H
    y = torch.full((T, D), float("nan"), dtype=torch.float32, device="cuda")
    cnt = torch.full((T,), -1, dtype=torch.int32, device="cuda") if want_live else None
    idx = torch.full((T, H), -1, dtype=torch.int32, device="cuda") if want_live else None
    sffn.sffn_forward_lopa(h.ptr, dev(x), dev(w["V"]), dev(w["U"]), dev(w["W3"]), dev(w["W2T"]), y,
                           T, mode, cnt, idx)
    torch.cuda.synchronize()
    return y, cnt, idx


def run_dense(h, x, w, T):
    y = torch.full((T, h.D), float("nan"), dtype=torch.float32, device="cuda")
    sffn.sffn_forward_dense(h.ptr, dev(x), dev(w["W1"]), dev(w["W3"]), dev(w["W2T"]), y, T)
    torch.cuda.synchronize()
    return y


def y_errors(y_gpu, y_ref):
    yg = y_gpu.detach().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(yg)), "non-finite output"
    diff = yg - y_ref
    nref = np.linalg.norm(y_ref)
    rel = np.linalg.norm(diff) / nref if nref > 0 else np.linalg.norm(diff)
    mx = np.max(np.abs(y_ref)) if y_ref.size else 0.0
    mabs = np.max(np.abs(diff)) if diff.size else 0.0
    return rel, mabs, mx


def check_y(y_gpu, y_ref, label=""):
    """Per-token check of the output tolerance."""
    yg = y_gpu.detach().cpu().numpy()
    for t in range(y_ref.shape[0]):
        rel, mabs, mx = y_errors(torch.from_numpy(yg[t:t + 1]), y_ref[t:t + 1])
        assert rel <= REL_L2, f"{label} token {t}: relative L2 {rel:.3e}"
        assert mabs <= MAX_ABS_FRAC * mx + 1e-30, f"{label} token {t}: max abs {mabs:.3e} vs {mx:.3e}"


def check_live(cnt, idx, oracle, label=""):
    c = cnt.cpu().numpy()
    ix = idx.cpu().numpy()
    for t in range(len(oracle["live"])):
        k = int(c[t])
        assert 0 <= k <= ix.shape[1], f"{label} token {t}: count {k}"
        got = ix[t, :k]
        assert len(set(got.tolist())) == k, f"{label} token {t}: repeated indices"
        assert np.all(np.diff(got) > 0), f"{label} token {t}: list not ascending"
        want = set(oracle["live"][t].tolist())
        diff = set(got.tolist()) ^ want
        bad = [i for i in diff if abs(oracle["z"][t][i]) >= Z_BAND]
        assert not bad, f"{label} token {t}: live sets differ at {bad[:8]} (z={[oracle['z'][t][i] for i in bad[:4]]})"


def tokens_stack(D, T, cfg, dtype, layer=0, replica=0):
    return gen.tokens(D, T, cfg=cfg, layer=layer, replica=replica, dtype=dtype)


def run_i8(h, x, w, T, mode=sffn.SFFN_MODE_PER_TOKEN, dense=False, want_live=True):
    """int8 weights (w: W1/W3/W2T int8 and *_scale fp32) through the _i8 forward calls."""
    D, H = h.D, h.H
    dv = {k: torch.from_numpy(np.ascontiguousarray(w[k])).cuda()
          for k in ("W1", "W3", "W2T", "W1_scale", "W3_scale", "W2T_scale")}
    y = torch.full((T, D), float("nan"), dtype=torch.float32, device="cuda")
    if dense:
        sffn.sffn_forward_dense_i8(h.ptr, dev(x), dv["W1"], dv["W1_scale"], dv["W3"],
                                   dv["W3_scale"], dv["W2T"], dv["W2T_scale"], y, T)
        torch.cuda.synchronize()
        return y, None, None
    cnt = torch.full((T,), -1, dtype=torch.int32, device="cuda") if want_live else None
    idx = torch.full((T, H), -1, dtype=torch.int32, device="cuda") if want_live else None
    sffn.sffn_forward_sparse_i8(h.ptr, dev(x), dv["W1"], dv["W1_scale"], dv["W3"], dv["W3_scale"],
                                dv["W2T"], dv["W2T_scale"], y, T, mode, cnt, idx)
    torch.cuda.synchronize()
    return y, cnt, idx


def run_lopa_i8(h, x, w, T, mode=sffn.SFFN_MODE_PER_TOKEN, want_live=True):
    """int8 LoPA weights (V/U/W3/W2T int8 and *_scale fp32) through sffn_forward_lopa_i8."""
    D, H = h.D, h.H
    dv = {k: torch.from_numpy(np.ascontiguousarray(w[k])).cuda()
          for k in ("V", "U", "W3", "W2T", "V_scale", "U_scale", "W3_scale", "W2T_scale")}
    y = torch.full((T, D), float("nan"), dtype=torch.float32, device="cuda")
    cnt = torch.full((T,), -1, dtype=torch.int32, device="cuda") if want_live else None
    idx = torch.full((T, H), -1, dtype=torch.int32, device="cuda") if want_live else None
    sffn.sffn_forward_lopa_i8(h.ptr, dev(x), dv["V"], dv["V_scale"], dv["U"], dv["U_scale"],
                              dv["W3"], dv["W3_scale"], dv["W2T"], dv["W2T_scale"], y, T, mode,
                              cnt, idx)
    torch.cuda.synchronize()
    return y, cnt, idx


def run_lopa_i4(h, x, w, T, mode=sffn.SFFN_MODE_PER_TOKEN, want_live=True):
    """int4 LoPA weights (V/U int8 rows, W3/W2T packed int4 with group scales) through
    sffn_forward_lopa_i4."""
    D, H = h.D, h.H
    dv = {k: torch.from_numpy(np.ascontiguousarray(w[k])).cuda()
          for k in ("V", "U", "W3", "W2T", "V_scale", "U_scale", "W3_scale", "W2T_scale")}
    y = torch.full((T, D), float("nan"), dtype=torch.float32, device="cuda")
    cnt = torch.full((T,), -1, dtype=torch.int32, device="cuda") if want_live else None
    idx = torch.full((T, H), -1, dtype=torch.int32, device="cuda") if want_live else None
    sffn.sffn_forward_lopa_i4(h.ptr, dev(x), dv["V"], dv["V_scale"], dv["U"], dv["U_scale"],
                              dv["W3"], dv["W3_scale"], dv["W2T"], dv["W2T_scale"], y, T, mode,
                              cnt, idx)
    torch.cuda.synchronize()
    return y, cnt, idx


def run_i4(h, x, w, T, mode=sffn.SFFN_MODE_PER_TOKEN, dense=False, want_live=True):
    """group-scaled int4 weights (W1/W3/W2T packed, *_scale fp32 [H, D/128])."""
    D, H = h.D, h.H
    dv = {k: torch.from_numpy(np.ascontiguousarray(w[k])).cuda()
          for k in ("W1", "W3", "W2T", "W1_scale", "W3_scale", "W2T_scale")}
    y = torch.full((T, D), float("nan"), dtype=torch.float32, device="cuda")
    if dense:
        sffn.sffn_forward_dense_i4(h.ptr, dev(x), dv["W1"], dv["W1_scale"], dv["W3"],
                                   dv["W3_scale"], dv["W2T"], dv["W2T_scale"], y, T)
        torch.cuda.synchronize()
        return y, None, None
    cnt = torch.full((T,), -1, dtype=torch.int32, device="cuda") if want_live else None
    idx = torch.full((T, H), -1, dtype=torch.int32, device="cuda") if want_live else None
    sffn.sffn_forward_sparse_i4(h.ptr, dev(x), dv["W1"], dv["W1_scale"], dv["W3"], dv["W3_scale"],
                                dv["W2T"], dv["W2T_scale"], y, T, mode, cnt, idx)
    torch.cuda.synchronize()
    return y, cnt, idx
