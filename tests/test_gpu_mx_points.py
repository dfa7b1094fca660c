"""GPU checks of where the MXFP8 layer quantises, on the crafted layers of tests/mx_cases.py.

Each crafted layer makes "quantised along the right axis, from fp32" an exact statement about
one output (a column that must be exactly zero, a ratio or value that must hold exactly), so
these checks see what a relative-Frobenius tolerance cannot: a wrong blocking axis, a skipped
quantisation point, a lost per-expert padding, or a BF16 rounding before quantising. The same
statements are pinned on the oracle in tests/test_oracle_mx_points.py; here every output is also
compared with the oracle at the MXFP8 tolerance. Staged and fused forward paths both run.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from oracle import moe_oracle as mo
from tests import mx_cases as mc
from tests._gpu import MX_TOL, ArrayCase, frob_rel_err

PATHS = ["staged", "fused"]


def _run(c: mc.Crafted, path: str):
    case = ArrayCase(c.x, c.dout, c.logits, c.wg, c.wu, c.wd, c.K, fused=(path == "fused"))
    got = case.run()
    W = mo.Weights(c.wg, c.wu, c.wd, "mxfp8")
    fw = mo.forward(lambda r: c.x[r], c.logits, W, c.K, 0, c.wg.shape[0], 64, row_align=32)
    bw = mo.backward(fw, lambda r: c.dout[r], W, c.K, 0, c.wg.shape[0], c.E)
    ref = dict(out=fw.out, dx=bw.dx, dwg=bw.dwg, dwu=bw.dwu, dwd=bw.dwd)
    errs = {k: frob_rel_err(got[k], ref[k]) for k in ref if np.linalg.norm(ref[k]) > 0}
    print(f"  rel. Frobenius error vs oracle: {errs}")
    assert all(v <= MX_TOL for v in errs.values()), errs
    return got, fw, bw


@pytest.mark.parametrize("path", PATHS)
def test_gpu_dispatch_quantises_x_along_h(path):
    got, _, _ = _run(mc.dispatch_x_along_h(), path)
    assert (got["out"][:, 1] == 0).all() and (got["out"][:, 0] != 0).all()


@pytest.mark.parametrize("path", PATHS)
def test_gpu_swiglu_quantises_h_along_i(path):
    got, _, _ = _run(mc.swiglu_h_along_i(), path)
    assert (got["out"][:, 1] == 0).all() and (got["out"][:, 0] != 0).all()


@pytest.mark.parametrize("path", PATHS)
def test_gpu_backward_quantises_dout_along_h(path):
    got, _, _ = _run(mc.backward_d_along_h(), path)
    assert (got["dx"][:, 2] == 0).all() and (got["dx"][:, 3] != 0).all()


@pytest.mark.parametrize("path", PATHS)
def test_gpu_dx_gemm_quantises_dg_du_along_i(path):
    got, _, _ = _run(mc.backward_dgdu_along_i(), path)
    assert (got["dx"][:, 1] == 0).all() and (got["dx"][:, 0] != 0).all()


@pytest.mark.parametrize("path", PATHS)
def test_gpu_wgrad_quantises_x_along_tokens(path):
    c = mc.wgrad_x_along_tokens()
    got, _, _ = _run(c, path)
    n_even = c.N // 2
    for k in ("dwg", "dwu"):
        dw = got[k][0]
        assert (dw[:, 32] != 0).all()
        assert np.array_equal(dw[:, 0] * c.N, dw[:, 32] * n_even), k


@pytest.mark.parametrize("path", PATHS)
def test_gpu_wgrad_quantises_h_along_tokens(path):
    c = mc.wgrad_h_along_tokens()
    got, fw, bw = _run(c, path)
    assert got["dwd"][0, 0, 1] == bw.dwd[0, 0, 1] == (c.N // 2) * fw.h[0, 1]


@pytest.mark.parametrize("path", PATHS)
def test_gpu_wgrad_quantises_dg_du_pd_along_tokens_per_expert(path):
    got_t, _, _ = _run(mc.wgrad_dgdu_pd_along_tokens(odd_scale=mc.TINY), path)
    got_z, _, _ = _run(mc.wgrad_dgdu_pd_along_tokens(odd_scale=0.0), path)
    for k in ("dwg", "dwu", "dwd"):
        assert np.array_equal(got_t[k], got_z[k]), k
    assert not np.array_equal(got_t["dx"], got_z["dx"])
    got_s, _, _ = _run(mc.wgrad_dgdu_pd_along_tokens(odd_scale=mc.TINY, split_experts=True), path)
    for k in ("dwg", "dwu", "dwd"):
        assert (got_s[k][0] != 0).any() and (got_s[k][1] != 0).any(), k


@pytest.mark.parametrize("path", PATHS)
def test_gpu_quantised_operands_come_from_fp32_values(path):
    got, _, _ = _run(mc.precision_ties(), path)
    assert (got["dwd"][0][0:2] == 216.0).all() and (got["dwd"][0][2:] == 0).all()
    assert (got["dwu"][0][:, 0] == 36.0).all()
    assert (got["dwg"][1][:, 0] == 36.0).all()
    assert (got["dx"][:, 7] == 72.0).all() and (got["dx"][:, 9] == 72.0).all()
