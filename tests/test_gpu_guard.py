"""Guard bands around every buffer the library writes: each output (and the KV pools, which take
the candidate writes, the workspaces and the status word) is the middle of a larger allocation
whose 4 KB before and after hold a byte pattern; after the call the pattern must be intact, so
a write past either end of any buffer fails the test.  Covered: the packer, the allocator, the
verification call with and without its prefill set (head dims 64, 128, 256; splits forced), the
fused packer call, the no-allocation entry point, the fp32 path, greedy and sampling
acceptance, the draft features and the counter-based uniforms."""
import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import workloads as wl  # noqa: E402
from gpu_util import DEV, to_dev  # noqa: E402
import block_verification_attention_amd as dsv  # noqa: E402

GUARD = 4096   # bytes on each side (keeps the 256-byte alignment of the middle)
PATTERN = 0x5A


class Guards:
    """Allocates guarded buffers and checks their guard bands."""

    def __init__(self):
        self.bufs = []

    def empty(self, name, shape, dtype, fill=None):
        n = math.prod(shape) if shape else 1
        esz = torch.empty((), dtype=dtype).element_size()
        raw = torch.full((2 * GUARD + n * esz,), PATTERN, dtype=torch.uint8, device=DEV)
        mid = raw[GUARD:GUARD + n * esz].view(dtype).view(shape)
        if fill is not None:
            mid.copy_(fill if isinstance(fill, torch.Tensor) else torch.full_like(mid, fill))
        self.bufs.append((name, raw))
        return mid

    def like(self, name, t, fill=None):
        return self.empty(name, tuple(t.shape), t.dtype, t if fill is None else fill)

    def check(self, tag):
        torch.cuda.synchronize()
        for name, raw in self.bufs:
            head, tail = raw[:GUARD], raw[-GUARD:]
            assert bool((head == PATTERN).all()) and bool((tail == PATTERN).all()), (tag, name)


def _pack_out(g, n_bs, m_bs, pre):
    return dict(offsets=g.empty(pre + "offsets", (n_bs + 1,), torch.int32),
                slot_req=g.empty(pre + "slot_req", (m_bs,), torch.int32),
                slot_tok=g.empty(pre + "slot_tok", (m_bs,), torch.int32),
                slot_pos=g.empty(pre + "slot_pos", (m_bs,), torch.int32),
                slot_cache_loc=g.empty(pre + "slot_cache_loc", (m_bs,), torch.int64))


@pytest.mark.parametrize("d_head,hq,hkv", [(128, 8, 2), (256, 12, 2), (64, 4, 1)])
@pytest.mark.parametrize("with_prefill", [False, True])
def test_guard_verification_calls(d_head, hq, hkv, with_prefill):
    c = wl.make_mixed_case(70 + d_head, hq=hq, hkv=hkv, d=d_head, k=[16, 5, 0, 11, 1, 16, 3],
                           ctx_len=[700, 0, 40, 63, 1000, 129, 2], m_bs=56,
                           pf_q_len=[257, 40] if with_prefill else [1], pf_ctx=[0, 30] if with_prefill else [0])
    g = Guards()
    st = g.empty("status", (1,), torch.int32, 0)
    kp = g.like("k_pool", to_dev(c["k_pool"]))
    vp = g.like("v_pool", to_dev(c["v_pool"]))
    k, ctx, base, tok = (to_dev(c[x]) for x in ("k", "ctx_len", "kv_base", "block_tokens"))
    q, kn, vn = to_dev(c["q"]), to_dev(c["k_new"]), to_dev(c["v_new"])
    packed = dsv.pack_slots(k, ctx, base, tok, c["m_bs"], st, out=_pack_out(g, c["n_bs"], c["m_bs"], "pack."))
    out = g.like("out", q, float("nan"))
    lse = g.empty("lse", (c["m_bs"], hq), torch.float32, float("nan"))
    prefill = None
    if with_prefill:
        pf = c["prefill"]
        pq = to_dev(pf["q"])
        prefill = dsv.Prefill(q_start=to_dev(pf["q_start"]), q_len=to_dev(pf["q_len"]),
                              ctx_len=to_dev(pf["ctx_len"]), kv_base=to_dev(pf["kv_base"]), q=pq,
                              out=g.like("pf_out", pq, float("nan")), max_len=int(pf["max_len"]),
                              lse=g.empty("pf_lse", (pq.shape[0], hq), torch.float32, float("nan")))
    max_ctx = int(c["ctx_len"].max())
    a = dsv.attn_args(q, kp, vp, packed["offsets"], k, ctx, base, W=c["W"], max_ctx=max_ctx, out=out,
                      status=st, lse=lse, k_new=kn, v_new=vn, slot_cache_loc=packed["slot_cache_loc"],
                      kv_chunk=64, prefill=prefill)
    need = dsv.verify_attn_workspace_bytes(a)
    assert need > 0  # 64-row splits: the merge runs
    ws = g.empty("workspace", (need,), torch.uint8, 0)
    a.workspace, a.workspace_bytes = ws.data_ptr(), need
    dsv.verify_attn_call(a)
    g.check(f"verify d{d_head}")
    # the packer fused into the launch, and the no-allocation entry point, on the same buffers
    fused = _pack_out(g, c["n_bs"], c["m_bs"], "fused.")
    dsv.pack_verify_attn(a, tok, out=fused)
    g.check(f"pack_verify d{d_head}")
    dsv.verify_attn_noalloc_call(a)
    g.check(f"noalloc d{d_head}")
    assert int(st.item()) == 0


def test_guard_fp32_verification():
    c = wl.config1()
    g = Guards()
    st = g.empty("status", (1,), torch.int32, 0)
    kp = g.like("k_pool", to_dev(c["k_pool"]))
    vp = g.like("v_pool", to_dev(c["v_pool"]))
    k, ctx, base, tok = (to_dev(c[x]) for x in ("k", "ctx_len", "kv_base", "block_tokens"))
    q, kn, vn = to_dev(c["q"]), to_dev(c["k_new"]), to_dev(c["v_new"])
    packed = dsv.pack_slots(k, ctx, base, tok, c["m_bs"], st, out=_pack_out(g, c["n_bs"], c["m_bs"], ""))
    out = g.like("out", q, float("nan"))
    lse = g.empty("lse", (c["m_bs"], c["hq"]), torch.float32, float("nan"))
    dsv.verify_attn(q, kp, vp, packed["offsets"], k, ctx, base, W=c["W"], max_ctx=int(c["ctx_len"].max()),
                    status=st, out=out, lse=lse, k_new=kn, v_new=vn, slot_cache_loc=packed["slot_cache_loc"])
    g.check("fp32 verify")
    assert int(st.item()) == 0


def test_guard_allocator():
    rng = np.random.default_rng(73)
    n_bs, W, m_bs = 12, 16, 96
    g = Guards()
    st = g.empty("status", (1,), torch.int32, 0)
    scores = to_dev(rng.uniform(0.05, 0.95, size=(n_bs, W - 1)).astype(np.float32))
    ctx = to_dev(rng.integers(0, 500, size=n_bs).astype(np.int32))
    base = to_dev((np.arange(n_bs) * 600).astype(np.int64))
    tok = to_dev(rng.integers(0, 32000, size=(n_bs, W)).astype(np.int32))
    out = dict(k=g.empty("k", (n_bs,), torch.int32), k0=g.empty("k0", (n_bs,), torch.int32),
               **_pack_out(g, n_bs, m_bs, ""))
    dsv.allocate_pack(scores, n_bs, 80, ctx, base, tok, m_bs, st, out=out)
    g.check("allocate_pack")
    assert int(st.item()) == 0


def test_guard_accept_sample_features_uniforms():
    rng = np.random.default_rng(74)
    n_bs, W, vocab = 5, 16, 3001
    k = np.array([16, 3, 0, 9, 1], np.int32)
    offsets = np.concatenate([[0], np.cumsum(k)]).astype(np.int32)
    m_bs = int(offsets[-1]) + 3
    logits = to_dev(rng.normal(0, 2, size=(m_bs, vocab)).astype(np.float32))
    slot_tok = to_dev(rng.integers(0, vocab, size=m_bs).astype(np.int32))
    draft = to_dev(rng.normal(0, 2, size=(n_bs, 15, 2003)).astype(np.float32))
    kd, od = to_dev(k), to_dev(offsets)
    g = Guards()
    st = g.empty("status", (1,), torch.int32, 0)
    out = dict(slot_argmax=g.empty("slot_argmax", (m_bs,), torch.int32),
               accepted=g.empty("accepted", (n_bs,), torch.int32),
               bonus=g.empty("bonus", (n_bs,), torch.int32),
               progress=g.empty("progress", (n_bs,), torch.int32),
               out_tokens=g.empty("out_tokens", (n_bs, W), torch.int32),
               margin=g.empty("margin", (n_bs, 15), torch.float32),
               draft_top1=g.empty("draft_top1", (n_bs, 15), torch.int32))
    need = dsv.accept_workspace_bytes(m_bs, vocab, n_bs, 15, 2003)
    ws = g.empty("accept.workspace", (max(need, 1),), torch.uint8, 0)
    dsv.accept(n_bs=n_bs, W=W, status=st, target_logits=logits, slot_tok=slot_tok, offsets=od, k=kd,
               draft_logits=draft, out=out, workspace=ws)
    g.check("accept")
    ua = g.empty("u_accept", (m_bs,), torch.float32, 0.0)
    ud = g.empty("u_draw", (n_bs,), torch.float32, 0.0)
    dsv.philox_uniforms(5, 0, m_bs, out=ua)
    dsv.philox_uniforms(5, 1 << 40, n_bs, out=ud)
    g.check("philox")
    sout = dict(accepted=g.empty("s.accepted", (n_bs,), torch.int32),
                bonus=g.empty("s.bonus", (n_bs,), torch.int32),
                progress=g.empty("s.progress", (n_bs,), torch.int32),
                out_tokens=g.empty("s.out_tokens", (n_bs, W), torch.int32),
                p_cand=g.empty("s.p_cand", (m_bs,), torch.float32, float("nan")))
    need = dsv.accept_sample_workspace_bytes(n_bs, m_bs, vocab)
    sws = g.empty("sample.workspace", (max(need, 1),), torch.uint8, 0)
    dsv.accept_sample(n_bs=n_bs, W=W, status=st, target_logits=logits, temperature=0.8, slot_tok=slot_tok,
                      offsets=od, k=kd, u_accept=ua, u_draw=ud, out=sout, workspace=sws)
    g.check("accept_sample")
    fo = g.empty("features", (n_bs, 15, 18), torch.float32, float("nan"))
    need = dsv.draft_features_workspace_bytes(n_bs * 15, 2003)
    fws = g.empty("features.workspace", (max(need, 1),), torch.uint8, 0)
    dsv.draft_features(draft, st, out=fo, workspace=fws)
    g.check("draft_features")
    assert int(st.item()) == 0


def test_guard_cache_map():
    """The token-granular cache map: pool rows in a random order, the candidates written
    through the map's rows for this step's positions."""
    c = wl.make_case(75, dtype="bf16", hq=8, hkv=2, d=128, k=np.array([16, 5, 0, 11], np.int32),
                     ctx_len=np.array([300, 0, 40, 129], np.int32), m_bs=36)
    rng = np.random.default_rng(75)
    rows = c["k_pool"].shape[1]
    perm = rng.permutation(rows)
    kph, vph = np.empty_like(c["k_pool"]), np.empty_like(c["v_pool"])
    kph[:, perm], vph[:, perm] = c["k_pool"], c["v_pool"]
    stride = int((c["ctx_len"] + c["W"]).max()) + 3
    idx = np.full((c["n_bs"], stride), -7, np.int32)
    for i in range(c["n_bs"]):
        n = int(c["ctx_len"][i] + c["k"][i])
        idx[i, :n] = perm[int(c["kv_base"][i]) + np.arange(n)]
    g = Guards()
    st = g.empty("status", (1,), torch.int32, 0)
    kp, vp = g.like("k_pool", to_dev(kph)), g.like("v_pool", to_dev(vph))
    kv_index = g.like("kv_index", to_dev(idx))
    k, ctx, base, tok = (to_dev(c[x]) for x in ("k", "ctx_len", "kv_base", "block_tokens"))
    packed = dsv.pack_slots(k, ctx, base, tok, c["m_bs"], st, out=_pack_out(g, c["n_bs"], c["m_bs"], ""))
    off = packed["offsets"].cpu().numpy()
    loc = np.full(c["m_bs"], -1, np.int64)
    for i in range(c["n_bs"]):
        for j in range(int(c["k"][i])):
            loc[off[i] + j] = idx[i, int(c["ctx_len"][i]) + j]
    q = to_dev(c["q"])
    out = g.like("out", q, float("nan"))
    lse = g.empty("lse", (c["m_bs"], c["hq"]), torch.float32, float("nan"))
    dsv.verify_attn(q, kp, vp, packed["offsets"], k, ctx, base, W=c["W"], max_ctx=int(c["ctx_len"].max()),
                    status=st, out=out, lse=lse, k_new=to_dev(c["k_new"]), v_new=to_dev(c["v_new"]),
                    slot_cache_loc=to_dev(loc), kv_chunk=64, kv_index=kv_index,
                    workspace=g.empty("workspace", (1 << 20,), torch.uint8, 0))
    g.check("cache map")
    assert int(st.item()) == 0
