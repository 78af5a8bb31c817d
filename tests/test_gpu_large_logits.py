"""The greedy accept step over a logits matrix past 2^31 elements (32-bit element offsets
would wrap): 900 requests x 16 slots over a 151,936-token vocabulary, 14,400 x 151,936 fp32
(8.75 GB), drawn on the device from a seeded generator.  Requests on both sides of the
2^31-element boundary (and the one that straddles it) get planted accepted prefixes; the
oracle runs on copies of their rows and decides every per-slot argmax and per-request result
of those requests."""
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
