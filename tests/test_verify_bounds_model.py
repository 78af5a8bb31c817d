"""Host-side model of the addressing of the head_dim-256 bf16 verification kernel
(`attn_bf16_kernel<256, 4, false, 32, 1, false>` in
block_verification_attention_amd/csrc/dsv_attn.hip), run on the CPU.

For every workgroup of the grid the host plans, every wave and every lane, the model forms
the kernel's own index expressions: the work-unit decode (KV-head walk, request rotation
per split, head groups), the head packing of (query head, row) pairs into 16-column tiles,
the query-fragment loads, the staged K/V tile loads with the clamp of boundary tiles to
t_hi - 1, the candidate block, the output and split-partial stores, the zeroed tail rows,
and every LDS byte range (tile stores with their XOR swizzles, the candidate stage, the K
operand reads and the transposing V reads).  Each is checked against the size of the
tensor it addresses and the 64 KiB of dynamic LDS of the launch.

The groupings covered are one to twelve query heads per KV head.  One and two heads per KV
head run on the same 4-wave kernel as three and four, with the waves past the request's
(head, row) pairs holding no heads (they only move tile loads).  The shapes are those of
the GPU parity tests (ragged prefixes and contexts, zero-context requests, k_i = 0), with
the automatic split plan and forced splits of 64 and 256 rows."""
import sys

import numpy as np
import pytest

import workloads as wl

# kernel constants of the instantiation
D, NW, TILE, HV = 256, 4, 32, 1
RPC = 1024 // (2 * D)             # rows per 1 KB wave load
NCK = TILE // RPC                 # wave loads per tensor per tile
NP = 2 * NCK * HV                 # wave loads per stage
QPW = (NP + NW - 1) // NW         # wave loads per wave per stage
EVEN = NCK % NW == 0
SUB_BYTES = 2 * TILE * D * 2
STAGE_BYTES = HV * SUB_BYTES
SHM = 2 * STAGE_BYTES             # two LDS stages
DB, KS = D // 16, D // 32
KB, KK = TILE // 16, TILE // 32
CPH = 2 * 16 * (D // 8)
CPB = (CPH + NW * 64 - 1) // (NW * 64)
K_TILE_KV = 64                    # split granularity
XCDS = 8
WIDE_HEADS_PER_WG = 4


def ctrunc(a, b):
    """C integer division (truncation toward zero)."""
    q = abs(a) // abs(b)
    return q if (a >= 0) == (b > 0) else -q


def k_slot(row, slot):
    sw = min(D // 8, 16)
    return slot ^ (row & (sw - 1))


def v_slot(row, slot):
    m = min(D // 16, 8)
    return slot ^ (2 * (row & (m - 1)))


def heads_per_wg(G):
    groups = (G + WIDE_HEADS_PER_WG - 1) // WIDE_HEADS_PER_WG
    return (G + groups - 1) // groups


def plan(n_bs, hkv, G, max_ctx, W, kv_chunk, cus=256):
    """The host's split plan at head_dim 256: (chunk, n_splits)."""
    rows = max_ctx + W
    chunk = kv_chunk
    if chunk <= 0:
        hg = (G + heads_per_wg(G) - 1) // heads_per_wg(G)
        units = n_bs * hkv * hg
        wgs = (6 if hg > 1 or hkv < XCDS else 10) * cus
        target = min(max((wgs + units - 1) // units, 1), 64)
        chunk = max(rows // target // K_TILE_KV * K_TILE_KV, K_TILE_KV)
        if units >= wgs and chunk > 4096:
            chunk = 4096
    return chunk, max(rows // chunk, 1)


class Bounds:
    def __init__(self):
        self.n = 0

    def check(self, ok, what):
        self.n += 1
        assert bool(np.all(ok)), what


# per (wave, lane, piece): the staged piece's tile-of-stage, K or V, row in its tile, slot
_W, _L, _U = np.meshgrid(np.arange(NW), np.arange(64), np.arange(QPW), indexing="ij")
if EVEN:
    P_SUB = _U // (2 * NCK // NW)
    P_ISV = _U % (2 * NCK // NW) >= NCK // NW
    P_EXISTS = np.ones_like(_U, bool)
else:
    P_SUB = (_W + _U * NW) // (2 * NCK)
    P_ISV = (_W + _U * NW) % (2 * NCK) >= NCK
    P_EXISTS = _W + _U * NW < NP
P_ROW = ((_W + _U * NW) % NCK) * RPC + _L // (D // 8)
P_SLOT = _L % (D // 8)


def check_lds(b):
    """Every LDS byte range of the kernel (independent of the shape): tile stores into both
    stages, the candidate block in stage 1 and its zeroed V rows, K operand reads and the
    transposing V reads of both stages."""
    ks_ = np.vectorize(k_slot)
    vs_ = np.vectorize(v_slot)
    loff = (P_SUB * SUB_BYTES + np.where(P_ISV, TILE * D * 2, 0) + P_ROW * (2 * D)
            + 16 * np.where(P_ISV, vs_(P_ROW, P_SLOT), ks_(P_ROW, P_SLOT)))
    for stage in (0, 1):
        a = stage * STAGE_BYTES + loff[P_EXISTS]
        b.check((a >= 0) & (a + 16 <= SHM), ("lds store", stage))
    e = np.arange(CPB * NW * 64)
    e = e[e < CPH]
    isv, row, slot = e // (16 * (D // 8)), (e // (D // 8)) % 16, e % (D // 8)
    a = (STAGE_BYTES + np.where(isv == 1, TILE * D * 2, 0) + row * (2 * D)
         + 16 * np.where(isv == 1, vs_(row, slot), ks_(row, slot)))
    b.check(a + 16 <= SHM, "candidate lds")
    e = np.arange(16 * (D // 8))
    row, slot = 16 + e // (D // 8), e % (D // 8)
    b.check(STAGE_BYTES + TILE * D * 2 + row * (2 * D) + 16 * vs_(row, slot) + 16 <= SHM, "candidate v zero")
    lane = np.arange(64)
    lq, lg = lane & 15, lane >> 4
    for stage in (0, 1):
        for ks in range(KS):
            koff = lq * (2 * D) + ks_(lq, 4 * ks + lg) * 16
            for kbk in range(KB):
                a = koff + stage * STAGE_BYTES + 16 * kbk * (2 * D)
                b.check((a >= 0) & (a + 16 <= SHM), ("lds k read", stage, ks, kbk))
        vrow = 4 * lg + (lq >> 2)
        for db in range(DB):
            voff = TILE * D * 2 + vrow * (2 * D) + vs_(vrow, 2 * db + ((lq & 3) >> 1)) * 16 + 8 * (lq & 1)
            for kk in range(KK):
                v0 = voff + stage * STAGE_BYTES + 32 * kk * (2 * D)
                b.check((v0 >= 0) & (v0 + 16 * (2 * D) + 8 <= SHM), ("lds v read", stage, db, kk))


def model_launch(case, kv_chunk, b):
    """Every global access of one launch over `case` (see the module docstring)."""
    n_bs, hq, hkv, W = case["n_bs"], case["hq"], case["hkv"], case["W"]
    G = hq // hkv
    GW = heads_per_wg(G)
    HG = (G + GW - 1) // GW
    k, ctx, kv_base = case["k"], case["ctx_len"], case["kv_base"]
    m_bs, pool_rows = case["m_bs"], case["pool_rows"]
    offsets = np.concatenate([[0], np.cumsum(k)]).astype(np.int64)
    end = int(offsets[-1])
    chunk, n_splits = plan(n_bs, hkv, G, int(ctx.max()), W, kv_chunk)
    grid = n_splits * n_bs * hkv * HG
    xcd_sib = HG > 1 and grid % (XCDS * HG) == 0
    q_elems = m_bs * hq * D
    knew_elems = m_bs * hkv * D
    ws_o_elems = n_splits * m_bs * hq * D
    ws_lse_elems = n_splits * m_bs * hq
    seen = set()
    lane = np.arange(64)
    lq, lg = lane & 15, lane >> 4
    w = np.arange(NW)[:, None]

    def unit_kv_head(u):
        return (u % hkv + u // XCDS) % hkv if XCDS % hkv == 0 else u % hkv

    for bid in range(grid):
        if xcd_sib:
            slot = bid // XCDS
            hg = slot % HG
            u = (slot // HG) * XCDS + bid % XCDS
            g = unit_kv_head(u)
            t0 = u // hkv
        else:
            g = unit_kv_head(bid)
            t0 = bid // hkv
            hg = t0 % HG
            t0 //= HG
        split = t0 // n_bs
        i = (t0 % n_bs + split) % n_bs if hkv < XCDS else t0 % n_bs
        seen.add((split, i, g, hg))
        b.check(0 <= i < n_bs and 0 <= g < hkv and 0 <= hg < HG and 0 <= split < n_splits,
                ("unit", bid, split, i, g, hg))
        h0 = g * G + hg * GW
        ki, off, c, kb = int(k[i]), int(offsets[i]), int(ctx[i]), int(kv_base[i])
        if i == 0 and split == 0:  # tail rows [end, m_bs) of this head group zeroed
            nh = min(GW, G - hg * GW)
            b.check(nh >= 1 and 0 <= h0 and h0 + nh <= hq and 0 <= end <= m_bs, ("zero rows", bid))
        b.check(0 <= ki <= W and off + ki <= m_bs and kb + c + ki <= pool_rows, ("request", i))
        n_vis = c + ki
        n_splits_i = min(max(n_vis // chunk, 1), n_splits)
        if ki == 0 or split >= n_splits_i:
            continue
        shift = K_TILE_KV if (n_splits_i >= 2 and n_vis - (n_splits_i - 1) * chunk >= 2 * K_TILE_KV + ki) else 0
        r_lo = split * chunk + (shift if split == n_splits_i - 1 else 0)
        r_hi = n_vis if split == n_splits_i - 1 else r_lo + chunk + (shift if split == n_splits_i - 2 else 0)
        pairs = G * ki
        pb, pe = 0, pairs
        if HG > 1:
            cap = NW * 16
            hgr = (pairs + cap - 1) // cap
            if hg >= hgr:
                continue
            per = (pairs + hgr - 1) // hgr
            pb = hg * per
            pe = min(pairs, pb + per)
        has_cand = r_hi > c
        t_hi = c if has_cand else r_hi
        n_tiles = ctrunc(t_hi - r_lo + HV * TILE - 1, HV * TILE)
        # head packing, per (wave, lane)
        pr = pb + w * 16 + lq[None, :]
        col_ok = pr < pe
        col_row = np.where(col_ok, pr % ki, 0)
        h = g * G + np.where(col_ok, pr // ki, 0)
        wave_has_heads = (pb + w * 16 < pe) & np.ones_like(col_ok)
        b.check((h >= g * G) & (h < g * G + G) & (h < hq), ("head", bid))
        # query fragment (loaded where the lane's (head, row) exists)
        qrow = off + col_row
        for ks in range(KS):
            e0 = (qrow * hq + h) * D + 8 * lg[None, :] + 32 * ks
            b.check(~col_ok | ((e0 >= 0) & (e0 + 8 <= q_elems)), ("q", bid, ks))
        # staged tiles: every stage the loop loads, boundary tiles clamped to t_hi - 1
        if n_tiles > 0:
            tile_base = r_lo + np.arange(n_tiles) * HV * TILE
            interior = (tile_base + HV * TILE <= t_hi)[:, None, None, None]
            pos = tile_base[:, None, None, None] + P_SUB[None] * TILE + P_ROW[None]
            pos = np.where(interior, pos, np.minimum(pos, t_hi - 1))
            pos = pos[:, P_EXISTS]
            b.check((pos >= 0) & (pos < t_hi) & (kb + pos < pool_rows), ("tile rows", bid))
        # output or split partials of each live lane's (head, row)
        live = wave_has_heads & col_ok
        orow = off + col_row
        b.check(~live | ((orow >= off) & (orow < off + ki)), ("out row", bid))
        for db in range(DB):
            d0 = 16 * db + 4 * lg[None, :]
            if n_splits_i == 1:
                e0 = (orow * hq + h) * D + d0
                b.check(~live | ((e0 >= 0) & (e0 + 4 <= q_elems)), ("out", bid))
            else:
                e0 = ((split * m_bs + orow) * hq + h) * D + d0
                b.check(~live | ((e0 >= 0) & (e0 + 4 <= ws_o_elems)), ("partial", bid))
        if n_splits_i == 1:
            b.check(~live | (orow * hq + h < m_bs * hq), ("lse", bid))
        else:
            b.check(~live | ((split * m_bs + orow) * hq + h < ws_lse_elems), ("partial lse", bid))
        # candidate block: rows 0 .. k_i - 1 of k_new / v_new
        if has_cand:
            e = np.arange(CPB * NW * 64)
            row, slot = (e // (D // 8)) % 16, e % (D // 8)
            used = (e < CPH) & (row < ki)
            e0 = ((off + row) * hkv + g) * D + 8 * slot
            b.check(~used | ((e0 >= 0) & (e0 + 8 <= knew_elems)), ("candidate load", bid))
    # every (split, request, KV head, head group) is one workgroup
    assert len(seen) == grid == n_splits * n_bs * hkv * HG


def _case(hq, hkv, k, ctx, W=16, extra_tail=4):
    k = np.asarray(k, np.int32)
    ctx = np.asarray(ctx, np.int32)
    kv_base, pool_rows = wl.segments(ctx, W)
    return {"n_bs": len(k), "hq": hq, "hkv": hkv, "W": W, "k": k, "ctx_len": ctx,
            "kv_base": kv_base, "pool_rows": pool_rows, "m_bs": int(k.sum()) + extra_tail}


RAGGED = ((16, 5, 0, 11, 1, 16, 3), (700, 0, 40, 63, 64, 1000, 129))


@pytest.mark.parametrize("hq,hkv", [(4, 4), (2, 1), (8, 4), (3, 1), (6, 2), (4, 1), (24, 2), (12, 1),
                                     (8, 8), (32, 8)])
@pytest.mark.parametrize("kv_chunk", [0, 64, 256])
def test_head_dim_256_addresses_in_bounds(hq, hkv, kv_chunk):
    b = Bounds()
    check_lds(b)
    model_launch(_case(hq, hkv, *RAGGED), kv_chunk, b)
    # zero-context requests, single anchors and an all-empty request
    model_launch(_case(hq, hkv, (1, 16, 0, 3), (0, 0, 0, 5)), kv_chunk, b)
    # long contexts that split, a request ending exactly on a tile and on a split boundary
    model_launch(_case(hq, hkv, (16, 1, 7), (2048 - 16, 4064, 1537)), kv_chunk, b)
    assert b.n > 0


def test_model_checks_bite(monkeypatch):
    """The checks are not vacuous: one LDS granule less than the launch's 64 KiB, or a pool
    one row too short for the last request, fails them."""
    case = _case(2, 1, (16, 1), (40, 0))
    model_launch(case, 0, Bounds())
    short = dict(case, pool_rows=case["pool_rows"] - 16 - 1)  # the last segment's spare rows and one
    with pytest.raises(AssertionError):
        model_launch(short, 0, Bounds())
    check_lds(Bounds())
    monkeypatch.setattr(sys.modules[__name__], "SHM", SHM - 16)
    with pytest.raises(AssertionError):
        check_lds(Bounds())
