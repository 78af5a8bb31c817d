"""GPU parity of dsv_accept against the oracle: bit-exact argmax, accepted lengths, bonus,
progress, output tokens and draft margins."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads as wl  # noqa: E402
from gpu_util import DEV, oracle_pack, to_dev  # noqa: E402
import block_verification_attention_amd as dsv  # noqa: E402


def _gpu_accept(logits, slot_tok, offsets, k, W, draft=None, logits_dev=None):
    st = dsv.new_status(DEV)
    o = dsv.accept(n_bs=len(k), W=W, status=st,
                   target_logits=logits_dev if logits_dev is not None else (to_dev(logits) if logits is not None else None),
                   slot_tok=to_dev(np.asarray(slot_tok, np.int32)) if slot_tok is not None else None,
                   offsets=to_dev(np.asarray(offsets, np.int32)) if offsets is not None else None,
                   k=to_dev(np.asarray(k, np.int32)),
                   draft_logits=to_dev(draft) if draft is not None else None)
    torch.cuda.synchronize()
    return {key: v.cpu().numpy() for key, v in o.items()}, int(st.item())


def _check_target(c_logits, slot_tok, offsets, k, W, tag):
    ref = oracle.accept(c_logits, slot_tok, offsets, k, W)
    got, st = _gpu_accept(c_logits, slot_tok, offsets, k, W)
    assert st == 0, tag
    for key in ("slot_argmax", "accepted", "bonus", "progress", "out_tokens"):
        assert np.array_equal(got[key], ref[key]), f"{tag}: {key}\n{got[key]}\n{ref[key]}"
    return got, ref


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_accept_configs(cfg):
    c = {1: wl.config1, 2: lambda: wl.config2()[1], 3: wl.config3}[cfg]()
    p = oracle_pack(c)
    got, _ = _check_target(c["logits"], p["slot_tok"], p["offsets"], c["k"], c["W"], f"cfg{cfg}")
    assert np.array_equal(got["accepted"], c["planted_accepted"])


def test_accept_ties_zero_sign_and_small_vocab():
    r = np.random.default_rng(9)
    for vocab in (1, 2, 3, 5, 1001, 4099):
        for trial in range(6):
            n, W = int(r.integers(1, 9)), int(r.integers(1, 17))
            k = r.integers(0, W + 1, size=n).astype(np.int32)
            m_bs = int(k.sum()) + int(r.integers(0, 5))
            x = r.integers(-2, 3, size=(max(m_bs, 1), vocab)).astype(np.float32)[:m_bs]  # many ties
            x[x == 0] = np.where(r.random(np.count_nonzero(x == 0)) < 0.5, -0.0, 0.0)
            tok = r.integers(0, vocab, size=(n, W)).astype(np.int32)
            p = oracle.pack(k, np.zeros(n, np.int32), np.zeros(n, np.int64), tok, W, m_bs)
            if m_bs == 0:
                continue
            _check_target(x, p["slot_tok"], p["offsets"], k, W, f"vocab {vocab} trial {trial}")


def test_accept_nan_row_and_bad_request():
    x = np.random.default_rng(2).standard_normal((6, 300)).astype(np.float32)
    x[1, 17] = np.nan
    k = np.array([3, 3], np.int32)
    tok = np.zeros((2, 16), np.int32)
    p = oracle.pack(k, [0, 0], [0, 0], tok, 16, 6)
    got, st = _gpu_accept(x, p["slot_tok"], p["offsets"], k, 16)
    assert st & dsv.STATUS_NAN
    assert got["slot_argmax"][1] == -1
    assert got["slot_argmax"][0] == np.argmax(x[0]) and got["slot_argmax"][3] == np.argmax(x[3])
    # request with k > W
    k_bad = np.array([3, 17], np.int32)
    got, st = _gpu_accept(x[:, :200].copy(), p["slot_tok"], [0, 3, 20], k_bad, 16)
    assert st & dsv.STATUS_BAD_REQUEST
    assert got["accepted"][1] == -1 and got["bonus"][1] == -1 and got["progress"][1] == 0
    assert np.all(got["out_tokens"][1] == -1)


def test_accept_unaligned_rows():
    """vocab not a multiple of 4: the scalar path."""
    r = np.random.default_rng(5)
    x = r.standard_normal((40, 32003)).astype(np.float32)
    k = np.array([16, 9, 0, 15], np.int32)
    tok = r.integers(0, 32003, size=(4, 16)).astype(np.int32)
    p = oracle.pack(k, np.zeros(4, np.int32), np.zeros(4, np.int64), tok, 16, 40)
    _check_target(x, p["slot_tok"], p["offsets"], k, 16, "unaligned")


def _check_margin(draft, tag):
    n, n_pos, _ = draft.shape
    ref_m, ref_t = oracle.top2_margin(draft)
    got, st = _gpu_accept(None, None, None, np.zeros(n, np.int32), 16, draft=draft)
    assert st == 0, tag
    assert np.array_equal(got["margin"].view(np.uint32), ref_m.view(np.uint32)), tag
    assert np.array_equal(got["draft_top1"], ref_t), tag


def test_margin_small_and_duplicates():
    r = np.random.default_rng(11)
    for vocab in (2, 3, 17, 1024, 5001):
        x = r.integers(-3, 4, size=(3, 15, vocab)).astype(np.float32)  # duplicated maxima
        _check_margin(x, f"dup vocab {vocab}")
        y = r.standard_normal((3, 15, vocab)).astype(np.float32)
        _check_margin(y, f"normal vocab {vocab}")


def test_margin_config4_full():
    c = wl.config4()
    _check_margin(c["draft_logits"], "cfg4")


def test_margin_nan():
    x = np.random.default_rng(3).standard_normal((2, 15, 999)).astype(np.float32)
    x[1, 4, 500] = np.nan
    got, st = _gpu_accept(None, None, None, np.zeros(2, np.int32), 16, draft=x)
    assert st & dsv.STATUS_NAN
    assert np.isnan(got["margin"][1, 4]) and got["draft_top1"][1, 4] == -1
    ref_m, ref_t = oracle.top2_margin(x[0])
    assert np.array_equal(got["margin"][0], ref_m) and np.array_equal(got["draft_top1"][0], ref_t)
