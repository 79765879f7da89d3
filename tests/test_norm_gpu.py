"""GPU parity of the output-gate sigmoid RMSNorm against the fp64 oracle.

Bar, from the arithmetic: the kernel works in fp32 (a 128-term sum of squares, one
rsqrt, sigmoid and three products: at most ~2e-5 relative before rounding), then
rounds y to bf16 (half an ulp, 2^-8 relative), so each element must satisfy
|y - y_ref| <= (2^-8 + 3e-5) |y_ref|, and rstd must match to 2e-5 relative.
"""

import numpy as np
import pytest
import torch

from linear_attention_rule_amd import gated_rmsnorm
from linear_attention_rule_amd import workloads as W
from oracle import kda_oracle as O

pytestmark = pytest.mark.gpu
Y_REL = 2.0 ** -8 + 3e-5
RSTD_REL = 2e-5


def _check(x, gate, weight, eps, y, rstd, rows=None):
    f = W.to_f64
    xs, gs = f(x), f(gate)
    if rows is not None:
        xs, gs = xs.reshape(-1, 128)[rows], gs.reshape(-1, 128)[rows]
    y_ref, r_ref = O.gated_rmsnorm(xs, gs, weight.numpy(), eps)
    yg = y.to(torch.float64).cpu().numpy()
    if rows is not None:
        yg = yg.reshape(-1, 128)[rows]
    err = np.abs(yg - y_ref)
    assert np.all(err <= Y_REL * np.abs(y_ref) + 1e-30), float((err / (np.abs(y_ref) + 1e-30)).max())
    if rstd is not None:
        rg = rstd.cpu().numpy().astype(np.float64)
        if rows is not None:
            rg = rg.reshape(-1)[rows]
        assert np.all(np.abs(rg - r_ref) <= RSTD_REL * r_ref)


@pytest.mark.parametrize("T,H", [(1, 1), (5, 3), (37, 16), (1000, 2), (3, 70)])
def test_norm_small_shapes(T, H):
    d = W.make_norm(W.NormCase(f"n_{T}x{H}", T, H, seed=4100 + T + H))
    x, g, w = d["x"].cuda(), d["gate"].cuda(), d["weight"].cuda()
    y, rstd = gated_rmsnorm(x, g, w, d["eps"])
    torch.cuda.synchronize()
    _check(d["x"], d["gate"], d["weight"], d["eps"], y, rstd)


def test_norm_strided_views_in_place_and_no_rstd():
    T, H = 300, 4
    d = W.make_norm(W.NormCase("n_fused", T, H, seed=4200))
    fused = torch.zeros((T, 3, H, 128), dtype=torch.bfloat16)   # [x | gate | other] per token
    fused[:, 0] = d["x"]
    fused[:, 1] = d["gate"]
    fused = fused.cuda()
    x, g, w = fused[:, 0], fused[:, 1], d["weight"].cuda()
    y_dense, _ = gated_rmsnorm(d["x"].cuda(), d["gate"].cuda(), w, d["eps"])
    y, rstd = gated_rmsnorm(x, g, w, d["eps"], out=x, want_rstd=False)   # in place, strided
    torch.cuda.synchronize()
    assert rstd is None
    assert torch.equal(y.contiguous().view(torch.int16).cpu(), y_dense.view(torch.int16).cpu())
    assert torch.equal(fused[:, 1].cpu(), d["gate"])                  # gate untouched
    assert bool((fused[:, 2].float() == 0).all())
    _check(d["x"], d["gate"], d["weight"], d["eps"], y_dense, None)


def test_norm_zero_rows():
    T, H, eps = 8, 2, 1e-5
    d = W.make_norm(W.NormCase("n_zero", T, H, eps=eps, seed=4300))
    d["x"][3] = 0
    y, rstd = gated_rmsnorm(d["x"].cuda(), d["gate"].cuda(), d["weight"].cuda(), eps)
    torch.cuda.synchronize()
    assert bool((y[3].float() == 0).all())
    assert np.allclose(rstd[3].cpu().numpy(), 1.0 / np.sqrt(eps), rtol=RSTD_REL)
    _check(d["x"], d["gate"], d["weight"], eps, y, rstd)


def test_norm_full_size_sampled():
    case = W.NORM
    print(f"case {case.name} seed {case.seed}", flush=True)
    d = W.make_norm(case)
    y, rstd = gated_rmsnorm(d["x"].cuda(), d["gate"].cuda(), d["weight"].cuda(), d["eps"])
    torch.cuda.synchronize()
    rows = np.arange(0, case.tokens * case.heads, 97)
    _check(d["x"], d["gate"], d["weight"], d["eps"], y, rstd, rows=rows)
