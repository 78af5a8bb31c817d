"""GPU parity of dsv_draft_features against the oracle: the top logit and the 15 gaps to
ranks 2-16 bit-exact (both sides round the exact difference once to fp32), the top token's
log-probability and the entropy within 1e-4 * max(1, |value|) -- the kernels accumulate the
softmax sums in fp32 over up to ~1000 terms per lane plus a merge tree, a relative error of at
most ~1000 * 2^-24 = 6e-5 on the sum, and the oracle in fp64."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads as wl  # noqa: E402
from gpu_util import DEV, to_dev  # noqa: E402
import block_verification_attention_amd as dsv  # noqa: E402

TOL = 1e-4


def _gpu(x):
    st = dsv.new_status(DEV)
    f = dsv.draft_features(to_dev(np.ascontiguousarray(x, np.float32)), st)
    torch.cuda.synchronize()
    return f.cpu().numpy(), int(st.item())


def _check(x, tag):
    ref = oracle.draft_features(x)
    got, st = _gpu(x)
    assert st == 0, tag
    assert np.array_equal(got[..., :16], ref[..., :16]), f"{tag}: top / gaps"
    for c in (16, 17):
        err = np.abs(got[..., c].astype(np.float64) - ref[..., c])
        assert np.all(err <= TOL * np.maximum(1.0, np.abs(ref[..., c]))), f"{tag}: feature {c}, max err {err.max()}"
    return got, ref


@pytest.mark.parametrize("vocab", [16, 17, 1000, 4099, 32768, 151936])
def test_features_random(vocab):
    rng = np.random.default_rng(vocab)
    rows = 37 if vocab < 100000 else 9
    x = (rng.standard_normal((rows, vocab)) * rng.uniform(0.2, 6.0, (rows, 1))).astype(np.float32)
    # planted structure: a dominant token, repeated maxima, quantised rows with many ties,
    # -inf entries (zero probability), fewer than 16 finite entries
    x[0, vocab // 2] += 30.0
    x[1, :4] = x[1].max() + 1.0
    x[2] = np.round(x[2])
    x[3, : vocab // 2] = -np.inf
    x[4, :] = -np.inf
    x[4, [1, 5, 9]] = [0.5, 2.0, -1.0]
    _check(x, f"vocab {vocab}")


def test_features_draft_workload():
    # the drafter workload: 32 requests x 15 positions over a 248,320-token vocabulary
    c = wl.config4(with_draft_logits=True)
    got, ref = _check(c["draft_logits"], "config 4 draft logits")
    assert got.shape == (32, 15, 18)


def test_features_bad_rows():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((6, 2048)).astype(np.float32)
    x[1, 100] = np.nan
    x[3, 7] = np.inf
    x[4] = -np.inf
    got, st = _gpu(x)
    assert st & dsv.STATUS_NAN
    for r in (1, 3, 4):
        assert np.all(np.isnan(got[r]))
    good = [0, 2, 5]
    ref = oracle.draft_features(x[good])
    assert np.array_equal(got[good][:, :16], ref[:, :16])


def test_features_bad_rows_long():
    # rows of many blocks: a NaN before a larger maximum that rescales the running sums, a
    # NaN among -inf only, a NaN as the last logit; the good rows around them are unaffected
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 100_000)).astype(np.float32)
    x[1, 3] = np.nan
    x[1, 95_000] = 50.0
    x[2] = -np.inf
    x[2, 40_000] = np.nan
    x[3, -1] = np.nan
    got, st = _gpu(x)
    assert st & dsv.STATUS_NAN
    for r in (1, 2, 3):
        assert np.all(np.isnan(got[r])), r
    good = [0, 4, 5]
    ref = oracle.draft_features(x[good])
    assert np.array_equal(got[good][:, :16], ref[:, :16])


def test_features_host_errors():
    st = dsv.new_status(DEV)
    with pytest.raises(dsv.DsvError):
        dsv.draft_features(torch.zeros((2, 15), dtype=torch.float32, device=DEV), st)
