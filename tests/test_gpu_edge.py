"""GPU edge cases of the whole layer (fused forward through the ring, then the backward), each
against the CPU oracle and against the staged forward: no local pairs, one token and one
expert, every expert selected, the largest top-k and local-expert counts, and ragged token
counts."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import datagen
from oracle import moe_oracle as mo

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from tests._gpu import BF16_TOL, MX_TOL, BwdCase, frob_rel_err, host_u16, max_rel_err


def _check_against_oracle(case, tol_fn, tol):
    cfg = case.cfg
    fw, bw = case.oracle_backward()
    tok = fw.sched.touched
    idx = case.layer.idx.cpu().numpy().reshape(-1, cfg.K)
    assert np.array_equal(idx, fw.idx)
    if len(tok):
        assert tol_fn(case.out_rows(tok), fw.out) <= tol
        assert tol_fn(mo.decode_bf16(host_u16(case.dx)[tok]), bw.dx) <= tol
        dp = case.dp.cpu().numpy().reshape(cfg.N, cfg.K)
        local = (fw.idx >= cfg.e0) & (fw.idx < cfg.e0 + cfg.E_loc)
        assert tol_fn(dp[local], bw.dp[local]) <= tol
        for name in ("dwg", "dwu", "dwd"):
            assert tol_fn(getattr(case, name).cpu().numpy().astype(np.float64), getattr(bw, name)) <= tol
    if case.dlogits is not None:
        got = case.dlogits.cpu().numpy().astype(np.float64)
        if np.abs(bw.dlogits).max() > 0:
            assert tol_fn(got, bw.dlogits) <= tol
        else:
            assert np.abs(got).max() <= 1e-6
    return fw


def _run_both(case):
    """Fused forward + backward, then staged forward + backward: bit-identical results."""
    case.run(fused=True)
    fused = case.grads() + [case.out.clone()]
    case.out.zero_()
    case.run(fused=False)
    staged = case.grads() + [case.out.clone()]
    names = ["dx", "dp", "dwg", "dwu", "dwd"] + (["dlogits"] if case.dlogits is not None else []) + ["out"]
    for name, a, b in zip(names, fused, staged):
        assert torch.equal(a, b), f"{name}: {int((a != b).sum())} elements differ"


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8"])
def test_no_local_pairs(dtype):
    """No token routes to a local expert: the persistent forward has no tiles and must still
    drain; nothing is written to out or dX, dp stays zero and dW is overwritten with zeros."""
    cfg = datagen.CONFIGS["tiny"].replace(e0=6, E_loc=2, dtype=dtype, M=32)
    logits = np.zeros((cfg.N, cfg.E), np.float32)
    logits[:, :2] = 5.0
    case = BwdCase(cfg, fused=True, logits=logits)
    for t in (case.dwg, case.dwu, case.dwd):
        t.fill_(7.0)
    case.run(fused=True)
    assert int(case.layer.header()[0]) == 0
    assert not case.out.any() and not case.dx.any() and not case.dp.any()
    for t in (case.dwg, case.dwu, case.dwd):
        assert not t.any()


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8"])
def test_one_token_one_expert(dtype):
    cfg = datagen.CONFIGS["tiny"].replace(S=1, T=1, E=1, K=1, e0=0, E_loc=1, H=128, I=128,
                                          dtype=dtype, M=32 if dtype == "mxfp8" else 16,
                                          x_std=1.0)
    case = BwdCase(cfg, fused=True)
    _run_both(case)
    tol_fn, tol = (max_rel_err, BF16_TOL) if dtype == "bf16" else (frob_rel_err, MX_TOL)
    _check_against_oracle(case, tol_fn, tol)


def test_every_expert_selected():
    """K = E: every token uses every expert (a dense softmax mixture); dlogits complete."""
    cfg = datagen.CONFIGS["tiny"].replace(E=4, K=4, e0=0, E_loc=4, x_std=1.0)
    case = BwdCase(cfg, fused=True)
    _run_both(case)
    _check_against_oracle(case, max_rel_err, BF16_TOL)


def test_largest_topk_and_local_experts():
    """top-16 over 1024 experts with 64 local experts (the library's maxima)."""
    cfg = datagen.CONFIGS["tiny"].replace(S=1, T=512, E=1024, K=16, e0=0, E_loc=64, H=128,
                                          I=128, M=256, x_std=1.0)
    case = BwdCase(cfg, fused=True)
    _run_both(case)
    fw = _check_against_oracle(case, max_rel_err, BF16_TOL)
    assert fw.sched.P > 0


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8"])
def test_ragged_token_counts(dtype):
    """Segments of 100 tokens, hidden 256, intermediate 384 (a partial 256-column tile)."""
    cfg = datagen.CONFIGS["tiny"].replace(S=3, T=100, H=256, E=12, K=3, I=384, e0=2, E_loc=5,
                                          dtype=dtype, M=64, x_std=1.0, ring_bytes=32 << 20)
    case = BwdCase(cfg, fused=True)
    _run_both(case)
    tol_fn, tol = (max_rel_err, BF16_TOL) if dtype == "bf16" else (frob_rel_err, MX_TOL)
    _check_against_oracle(case, tol_fn, tol)
