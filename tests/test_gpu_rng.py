"""GPU parity of dsv_philox_uniforms against the oracle's Philox4x64-10 (bit for bit: both
take the top 24 bits of each 64-bit word), and the sampling verifier run end to end on
uniforms generated on the device, against the oracle run on the oracle's uniforms."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads as wl  # noqa: E402
from gpu_util import DEV, to_dev  # noqa: E402
import block_verification_attention_amd as dsv  # noqa: E402


@pytest.mark.parametrize("key,counter,n", [(0, 0, 1), (1, 0, 4), (12345, 7, 1001),
                                           ((3 << 64) + 99, 2**64 - 2, 4096 + 3),
                                           (2**128 - 1, 2**128 - 64, 250), (5, 2**128 - 8, 101),
                                           (77, 5, 1 << 20)])
def test_uniforms_bit_exact(key, counter, n):
    got = dsv.philox_uniforms(key, counter, n, device=DEV)
    torch.cuda.synchronize()
    ref = oracle.philox_uniforms(key, counter, n)
    assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_uniforms_unaligned_output_and_zero_length():
    buf = torch.full((1 + 1003,), -1.0, dtype=torch.float32, device=DEV)
    dsv.philox_uniforms(9, 3, 1002, out=buf[1:])  # 4-byte aligned only: the scalar stores
    dsv.philox_uniforms(9, 3, 0, out=buf[1:])
    torch.cuda.synchronize()
    h = buf.cpu().numpy()
    assert h[0] == -1.0 and h[-1] == -1.0
    assert np.array_equal(h[1:1003].view(np.uint32), oracle.philox_uniforms(9, 3, 1002).view(np.uint32))


def test_sampling_verifier_on_device_uniforms():
    # 20 requests x 16 slots over a 32,768-token vocabulary; the accept uniforms take counter
    # blocks [0, 80) of the key and the successor draws the blocks after them
    g = np.random.default_rng(404)
    n_bs, W, vocab, T = 20, 16, 32768, 0.9
    k = g.integers(0, W + 1, n_bs).astype(np.int32)
    m_bs = int(k.sum()) + 3
    bt = g.integers(0, vocab, (n_bs, W)).astype(np.int32)
    logits, bt = wl.sampling_logits(g, k, vocab, m_bs, bt, boost=(0.0, 8.0), p_random=0.2, W=W)
    p = oracle.pack(k, np.zeros(n_bs, np.int32), np.zeros(n_bs, np.int64), bt, W, m_bs)
    key = 0xC0FFEE
    c_draw = (m_bs + 3) // 4
    ua = dsv.philox_uniforms(key, 0, m_bs, device=DEV)
    ud = dsv.philox_uniforms(key, c_draw, n_bs, device=DEV)
    ref = oracle.accept_sample(logits, p["slot_tok"], p["offsets"], k, W, T,
                               oracle.philox_uniforms(key, 0, m_bs), oracle.philox_uniforms(key, c_draw, n_bs))
    am = ref["acc_margin"][~np.isnan(ref["acc_margin"])]
    dm = ref["draw_margin"][~np.isnan(ref["draw_margin"])]
    assert am.size == 0 or am.min() > 1e-5, "fixture has an accept decision at its threshold"
    assert dm.size == 0 or dm.min() > 1e-9, "fixture has a draw at a boundary"
    st = dsv.new_status(DEV)
    got = dsv.accept_sample(n_bs=n_bs, W=W, status=st, target_logits=to_dev(logits), temperature=T,
                            slot_tok=to_dev(p["slot_tok"]), offsets=to_dev(p["offsets"]), k=to_dev(k),
                            u_accept=ua, u_draw=ud)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for key_ in ("accepted", "bonus", "progress", "out_tokens"):
        assert np.array_equal(got[key_].cpu().numpy(), ref[key_]), key_
    assert 0 < ref["accepted"].sum() < int(np.maximum(k - 1, 0).sum())
