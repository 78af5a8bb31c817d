"""Logits sweeps over matrices past 2^31 elements (32-bit element offsets would wrap), drawn
on the device from seeded generators.  The greedy accept step: 900 requests x 16 slots over a
151,936-token vocabulary, 14,400 x 151,936 fp32 (8.75 GB); requests on both sides of the
2^31-element boundary (and the one that straddles it) get planted accepted prefixes, and the
oracle runs on copies of their rows and decides every per-slot argmax and per-request result
of those requests.  The draft features: 8,700 positions x 248,320 tokens (8.6 GB), rows on both
sides of the boundary and the row across it against the oracle.  The sampling verifier: the
accept step's shape with boosted drafts, requests on both sides of the boundary and across it
against the oracle on the same seeded uniforms."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from gpu_util import DEV, to_dev  # noqa: E402
import block_verification_attention_amd as dsv  # noqa: E402

N_BS, W, VOCAB = 900, 16, 151_936


def test_accept_past_2_31_logits():
    m_bs = N_BS * W
    assert m_bs * VOCAB > 1 << 31
    straddle = (1 << 31) // VOCAB // W  # the request whose rows cross element 2^31
    sample = {0: 3, straddle: 7, N_BS - 3: 15, N_BS - 2: 0, N_BS - 1: 10}  # request -> planted length
    rng = np.random.default_rng(7200)
    k = np.full(N_BS, W, np.int32)
    tokens = rng.integers(0, VOCAB, (N_BS, W)).astype(np.int32)
    ref_pack = oracle.pack(k, np.zeros(N_BS, np.int32), np.zeros(N_BS, np.int64), tokens, W, m_bs)
    slot_tok = ref_pack["slot_tok"]
    offs = ref_pack["offsets"]

    g = torch.Generator(device=DEV)
    g.manual_seed(7201)
    logits = torch.empty((m_bs, VOCAB), dtype=torch.float32, device=DEV)
    for r0 in range(0, m_bs, 2048):
        logits[r0:r0 + 2048].normal_(generator=g)
    # planted prefixes: row j of request i predicts the draft at slot j + 1 for j < length
    rows, cols = [], []
    for i, a in sample.items():
        for j in range(a):
            rows.append(int(offs[i]) + j)
            cols.append(int(slot_tok[int(offs[i]) + j + 1]))
    logits[torch.as_tensor(rows, device=DEV), torch.as_tensor(cols, device=DEV)] = 100.0

    st = dsv.new_status(DEV)
    got = dsv.accept(n_bs=N_BS, W=W, status=st, target_logits=logits, slot_tok=to_dev(slot_tok),
                     offsets=to_dev(offs), k=to_dev(k))
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    g_arg = got["slot_argmax"].cpu().numpy()
    for i, a in sample.items():
        sl = slice(int(offs[i]), int(offs[i]) + W)
        ref = oracle.accept(logits[sl].cpu().numpy(), slot_tok[sl], np.array([0, W], np.int32),
                            np.array([W], np.int32), W)
        assert np.array_equal(g_arg[sl], ref["slot_argmax"]), i
        for key in ("accepted", "bonus", "progress"):
            assert int(got[key][i].item()) == int(ref[key][0]), (i, key)
        assert np.array_equal(got["out_tokens"][i].cpu().numpy(), ref["out_tokens"][0]), i
        assert int(ref["accepted"][0]) >= a, (i, a)  # the planted prefix is accepted
    del logits
    torch.cuda.empty_cache()


def test_draft_features_past_2_31_logits():
    # 8,700 draft positions x 248,320 tokens (2.16e9 fp32): rows on both sides of element 2^31
    # and the row across it, checked against the oracle on copies of those rows
    rows_n, vocab = 8_700, 248_320
    assert rows_n * vocab > 1 << 31
    across = (1 << 31) // vocab
    sample = [0, across - 1, across, across + 1, rows_n - 1]
    g = torch.Generator(device=DEV)
    g.manual_seed(7202)
    x = torch.empty((rows_n, vocab), dtype=torch.float32, device=DEV)
    for r0 in range(0, rows_n, 1024):
        x[r0:r0 + 1024].normal_(generator=g)
    st = dsv.new_status(DEV)
    f = dsv.draft_features(x, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    got = f[torch.as_tensor(sample, device=DEV)].cpu().numpy()
    ref = oracle.draft_features(x[torch.as_tensor(sample, device=DEV)].cpu().numpy())
    assert np.array_equal(got[:, :16], ref[:, :16])
    for c in (16, 17):
        err = np.abs(got[:, c].astype(np.float64) - ref[:, c])
        assert np.all(err <= 1e-4 * np.maximum(1.0, np.abs(ref[:, c]))), (c, err.max())
    del x
    torch.cuda.empty_cache()


def test_accept_sample_past_2_31_logits():
    # the sampling verifier over the accept step's matrix shape: drafts raised to the row
    # maximum + U(8, 12) before the temperature, seeded uniforms shared with the oracle
    m_bs = N_BS * W
    T = 0.9
    straddle = (1 << 31) // VOCAB // W
    sample = [0, straddle, N_BS - 2, N_BS - 1]
    rng = np.random.default_rng(7203)
    k = np.full(N_BS, W, np.int32)
    tokens = rng.integers(0, VOCAB, (N_BS, W)).astype(np.int32)
    ref_pack = oracle.pack(k, np.zeros(N_BS, np.int32), np.zeros(N_BS, np.int64), tokens, W, m_bs)
    slot_tok, offs = ref_pack["slot_tok"], ref_pack["offsets"]
    u_acc = rng.random(m_bs, dtype=np.float32)
    u_draw = rng.random(N_BS, dtype=np.float32)

    g = torch.Generator(device=DEV)
    g.manual_seed(7204)
    logits = torch.empty((m_bs, VOCAB), dtype=torch.float32, device=DEV)
    for r0 in range(0, m_bs, 2048):
        logits[r0:r0 + 2048].normal_(generator=g)
    rows, cols = [], []
    for i in sample:
        for j in range(W - 1):
            rows.append(int(offs[i]) + j)
            cols.append(int(slot_tok[int(offs[i]) + j + 1]))
    rows_t = torch.as_tensor(rows, device=DEV)
    boost = torch.as_tensor(rng.uniform(8.0, 12.0, len(rows)).astype(np.float32), device=DEV)
    logits[rows_t, torch.as_tensor(cols, device=DEV)] = logits[rows_t].max(dim=1).values + boost

    st = dsv.new_status(DEV)
    got = dsv.accept_sample(n_bs=N_BS, W=W, status=st, target_logits=logits, temperature=T,
                            slot_tok=to_dev(slot_tok), offsets=to_dev(offs), k=to_dev(k),
                            u_accept=to_dev(u_acc), u_draw=to_dev(u_draw))
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    n_acc = 0
    for i in sample:
        sl = slice(int(offs[i]), int(offs[i]) + W)
        ref = oracle.accept_sample(logits[sl].cpu().numpy(), slot_tok[sl], np.array([0, W], np.int32),
                                   np.array([W], np.int32), W, T, u_acc[sl], u_draw[i:i + 1])
        am = ref["acc_margin"][~np.isnan(ref["acc_margin"])]
        dm = ref["draw_margin"][~np.isnan(ref["draw_margin"])]
        assert am.size == 0 or am.min() > 1e-5, "fixture has an accept decision at its threshold"
        assert dm.size == 0 or dm.min() > 1e-9, "fixture has a draw at a boundary"
        for key in ("accepted", "bonus", "progress"):
            assert int(got[key][i].item()) == int(ref[key][0]), (i, key)
        assert np.array_equal(got["out_tokens"][i].cpu().numpy(), ref["out_tokens"][0]), i
        n_acc += int(ref["accepted"][0])
    assert 0 < n_acc < len(sample) * (W - 1)
    del logits
    torch.cuda.empty_cache()
