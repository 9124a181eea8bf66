"""Pins of the CPU oracle against facts other than its own formulas (CPU only).

Each test fixes a piece of the oracle with something independent: a closed form,
a special case that reduces to a textbook or library routine, explicit scalar
loops on tiny inputs, an invariant of the mathematics, finite differences, or a
value the handbook "Context parallelism: Ring Attention and Ulysses" fixes
(tests/golden/handbook_p4.json).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import cp_inputs
import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "handbook_p4.json")))


def rnd(*shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- attention values

def test_hand_worked_two_token_example():
    # Two tokens, D=2, causal.  Row 0 sees key 0 only; row 1 sees both.
    q = np.array([[[[1.0, 0.0]], [[0.0, 1.0]]]])       # [1,2,1,2]
    k = np.array([[[[1.0, 0.0]], [[1.0, 1.0]]]])
    v = np.array([[[[1.0, 2.0]], [[3.0, 4.0]]]])
    out, lse = oracle.attn_fwd(q, k, v)
    c = 1 / math.sqrt(2)
    assert lse[0, 0, 0] == pytest.approx(c, abs=1e-15)
    assert out[0, 0, 0] == pytest.approx([1.0, 2.0], abs=1e-15)
    # row 1: scores (0, c)
    z = 1 + math.exp(c)
    assert lse[0, 0, 1] == pytest.approx(math.log(z), abs=1e-15)
    w = math.exp(c) / z
    assert out[0, 1, 0] == pytest.approx([(1 - w) * 1 + w * 3, (1 - w) * 2 + w * 4], abs=1e-14)


@pytest.mark.parametrize("case", ["causal", "offset", "zigzag", "packed", "window", "window_noncausal"])
def test_zero_query_closed_form(case):
    # q = 0 makes every visible score 0: lse = log(#visible), out = mean of visible v.
    S, H, D = 24, 2, 3
    k, v = rnd(1, S, H, D, seed=1), rnd(1, S, H, D, seed=2)
    q = np.zeros((1, S, H, D))
    kw, counts, firsts = {}, None, None
    i = np.arange(S)
    if case == "causal":
        counts, firsts = i + 1, np.zeros(S, int)
    elif case == "offset":
        # queries at global 100.., keys at 96..: query i sees keys j <= i + 4
        kw = dict(q_offset=100, k_offset=96)
        counts, firsts = np.minimum(i + 5, S), np.zeros(S, int)
    elif case == "zigzag":
        qpos = np.array(list(range(0, 4)) + list(range(40, 60)))   # 24 increasing positions
        kpos = np.arange(30, 54)
        kw = dict(q_pos=qpos, k_pos=kpos)
        counts = np.array([max(0, min(S, p - 30 + 1)) for p in qpos])
        firsts = np.zeros(S, int)
    elif case == "packed":
        lens = [5, 9, 10]
        seg = np.repeat(np.arange(3), lens)[None]
        starts = np.repeat(np.cumsum([0] + lens[:-1]), lens)
        kw = dict(q_seg=seg, k_seg=seg)
        counts, firsts = i - starts + 1, starts
    else:
        # the window: keys at positions i - W + 1 .. i, with or without the causal flag
        W = 5
        kw = dict(window=W, causal=case == "window")
        counts, firsts = np.minimum(i + 1, W), np.maximum(0, i - W + 1)
    out, lse = oracle.attn_fwd(q, k, v, **kw)
    for h in range(H):
        for r in range(S):
            if counts[r] == 0:
                assert lse[0, h, r] == -np.inf and np.all(out[0, r, h] == 0)
                continue
            assert lse[0, h, r] == pytest.approx(math.log(counts[r]), abs=1e-13)
            if case == "zigzag":
                sel = np.arange(S)[np.arange(30, 54) <= qpos[r]]
            elif case == "offset":
                sel = np.arange(counts[r])
            else:
                sel = np.arange(firsts[r], firsts[r] + counts[r])
            np.testing.assert_allclose(out[0, r, h], v[0, sel, h].mean(axis=0), atol=1e-13)


def test_first_row_and_window_one():
    S, H, D = 9, 3, 4
    q, k, v = rnd(2, S, H, D, seed=3), rnd(2, S, H, D, seed=4), rnd(2, S, H, D, seed=5)
    out, lse = oracle.attn_fwd(q, k, v)
    np.testing.assert_allclose(out[:, 0], v[:, 0], atol=1e-14)
    np.testing.assert_allclose(lse[:, :, 0], (q[:, 0] * k[:, 0]).sum(-1) / 2.0, atol=1e-14)
    out1, lse1 = oracle.attn_fwd(q, k, v, window=1)      # each query sees only itself
    np.testing.assert_allclose(out1, v, atol=1e-14)
    np.testing.assert_allclose(lse1, np.transpose((q * k).sum(-1), (0, 2, 1)) / 2.0, atol=1e-14)
    outw, lsew = oracle.attn_fwd(q, k, v, window=S)       # window >= S is plain causal
    np.testing.assert_array_equal(outw, out)
    np.testing.assert_array_equal(lsew, lse)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa(causal):
    B, S, H, D = 2, 33, 3, 8
    q, k, v = rnd(B, S, H, D, seed=6), rnd(B, S, H, D, seed=7), rnd(B, S, H, D, seed=8)
    out, _ = oracle.attn_fwd(q, k, v, causal=causal)
    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)  # [B,H,S,D]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal)
    np.testing.assert_allclose(out, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12)


def test_matches_torch_sdpa_masked_gqa():
    # boolean mask (packed + window + offsets) and grouped heads through sdpa's own mask path
    B, Sq, Sk, Hq, Hkv, D = 1, 20, 28, 4, 2, 5
    q, k, v = rnd(B, Sq, Hq, D, seed=9), rnd(B, Sk, Hkv, D, seed=10), rnd(B, Sk, Hkv, D, seed=11)
    qpos, kpos = np.arange(8, 28), np.arange(Sk)
    seg = np.repeat([0, 1, 2], [10, 9, 9])
    mask = oracle.visible_mask(qpos, kpos, True, seg[qpos], seg[kpos], 7)
    assert mask.any(axis=1).all()
    out, _ = oracle.attn_fwd(q, k, v, q_pos=qpos, k_pos=kpos, q_seg=seg[qpos][None],
                             k_seg=seg[kpos][None], window=7)
    rep = lambda x: torch.from_numpy(np.repeat(x, Hq // Hkv, axis=2)).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(0, 2, 1, 3), rep(k), rep(v), attn_mask=torch.from_numpy(mask))
    np.testing.assert_allclose(out, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12)


def _brute(q, k, v, qpos, kpos, qseg, kseg, causal, window, G):
    B, Sq, Hq, D = q.shape
    out = np.zeros(q.shape)
    lse = np.full((B, Hq, Sq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            for i in range(Sq):
                sc = []
                for j in range(k.shape[1]):
                    if causal and kpos[j] > qpos[i]:
                        continue
                    if qseg is not None and qseg[b][i] != kseg[b][j]:
                        continue
                    # the window: the `window` most recent positions up to the query's own
                    if window and not 0 <= qpos[i] - kpos[j] < window:
                        continue
                    s = sum(q[b, i, h, d] * k[b, j, h // G, d] for d in range(D)) / math.sqrt(D)
                    sc.append((s, j))
                if not sc:
                    continue
                m = max(s for s, _ in sc)
                tot = sum(math.exp(s - m) for s, _ in sc)
                lse[b, h, i] = m + math.log(tot)
                for s, j in sc:
                    out[b, i, h] += math.exp(s - lse[b, h, i]) * v[b, j, h // G]
    return out, lse


@pytest.mark.parametrize("causal,window,packed", [(True, 0, False), (True, 3, True), (False, 0, True),
                                                   (False, 3, False), (False, 2, True)])
def test_brute_force_loops(causal, window, packed):
    B, Sq, Sk, Hq, Hkv, D = 2, 7, 9, 4, 2, 3
    q, k, v = rnd(B, Sq, Hq, D, seed=12), rnd(B, Sk, Hkv, D, seed=13), rnd(B, Sk, Hkv, D, seed=14)
    qpos = np.array([3, 4, 5, 9, 10, 11, 12])
    kpos = np.arange(2, 11)
    qseg = kseg = None
    if packed:
        qseg = np.array([[0, 0, 1, 1, 1, 2, 2], [0, 0, 0, 0, 1, 1, 1]])
        kseg = np.array([[0, 0, 0, 1, 1, 1, 1, 2, 2], [0, 0, 0, 0, 0, 0, 1, 1, 1]])
    out, lse = oracle.attn_fwd(q, k, v, q_pos=qpos, k_pos=kpos, q_seg=qseg, k_seg=kseg,
                               causal=causal, window=window)
    ref_o, ref_l = _brute(q, k, v, qpos, kpos, qseg, kseg, causal, window, Hq // Hkv)
    np.testing.assert_allclose(out, ref_o, atol=1e-13)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(ref_l))
    np.testing.assert_allclose(lse[np.isfinite(lse)], ref_l[np.isfinite(ref_l)], atol=1e-13)


def test_gqa_equals_repeated_mha():
    B, S, Hq, Hkv, D = 1, 16, 8, 2, 4
    q, k, v = rnd(B, S, Hq, D, seed=15), rnd(B, S, Hkv, D, seed=16), rnd(B, S, Hkv, D, seed=17)
    o1, l1 = oracle.attn_fwd(q, k, v)
    o2, l2 = oracle.attn_fwd(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2))
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)


def test_packed_equals_per_document():
    lens = [3, 8, 5, 6]
    S, H, D = sum(lens), 2, 4
    q, k, v = rnd(1, S, H, D, seed=18), rnd(1, S, H, D, seed=19), rnd(1, S, H, D, seed=20)
    seg = np.repeat(np.arange(len(lens)), lens)[None]
    out, lse = oracle.attn_fwd(q, k, v, q_seg=seg, k_seg=seg)
    s0 = 0
    for n in lens:
        o, l = oracle.attn_fwd(q[:, s0:s0 + n], k[:, s0:s0 + n], v[:, s0:s0 + n])
        np.testing.assert_allclose(out[:, s0:s0 + n], o, atol=1e-14)
        np.testing.assert_allclose(lse[:, :, s0:s0 + n], l, atol=1e-14)
        s0 += n


# ---------------------------------------------------------------- merge

@pytest.mark.parametrize("split", [1, 7, 13])
def test_merge_of_key_halves_is_full_attention(split):
    B, Sq, Sk, H, D = 1, 10, 16, 2, 4
    q, k, v = rnd(B, Sq, H, D, seed=21), rnd(B, Sk, H, D, seed=22), rnd(B, Sk, H, D, seed=23)
    kw = dict(q_offset=6)
    full_o, full_l = oracle.attn_fwd(q, k, v, **kw)
    a = oracle.attn_fwd(q, k[:, :split], v[:, :split], **kw)
    b = oracle.attn_fwd(q, k[:, split:], v[:, split:], k_offset=split, **kw)
    for x, y in ((a, b), (b, a)):
        o, l = oracle.lse_merge(*x, *y)
        np.testing.assert_allclose(o, full_o, atol=1e-13)
        np.testing.assert_allclose(l, full_l, atol=1e-13)


def test_merge_identity_and_empty():
    o = rnd(1, 3, 2, 4, seed=24)
    l = rnd(1, 2, 3, seed=25)
    zero, ninf = np.zeros_like(o), np.full_like(l, -np.inf)
    mo, ml = oracle.lse_merge(o, l, zero, ninf)
    np.testing.assert_array_equal(mo, o)
    np.testing.assert_array_equal(ml, l)
    mo, ml = oracle.lse_merge(zero, ninf, zero, ninf)
    assert np.all(mo == 0) and np.all(ml == -np.inf)


# ---------------------------------------------------------------- zigzag, ring, Ulysses

def test_zigzag_work_matches_handbook():
    g = GOLDEN["zigzag_work"]
    P = g["P"]
    assert [oracle.work(oracle.rank_chunks(r, P, "contiguous")) for r in range(P)] == g["contiguous"]
    assert [oracle.work(oracle.rank_chunks(r, P, "zigzag")) for r in range(P)] == g["zigzag"]
    assert oracle.chunk_order(P) == GOLDEN["zigzag_chunk_order"]["order"]


@pytest.mark.parametrize("S,P", [(32, 4), (1024, 16), (96, 3)])
def test_zigzag_exact_pairs_every_rank_every_step(S, P):
    c = S // (2 * P)
    total = 0
    for r in range(P):
        qpos = oracle.rank_positions(r, P, S, "zigzag")
        for s in range(P):
            kpos = oracle.rank_positions((r - s) % P, P, S, "zigzag")
            n = oracle.visible_pairs(qpos, kpos)
            assert n == (2 * c * c + c if s == 0 else 2 * c * c)
            total += n
    assert total == S * (S + 1) // 2


def test_reorder_roundtrip_and_layout():
    x = np.arange(2 * 48 * 3).reshape(2, 48, 3)
    y = oracle.reorder(x, 4)
    np.testing.assert_array_equal(oracle.reorder_inv(y, 4), x)
    # a contiguous 4-way split of the reordered sequence gives every rank its zigzag chunks
    for r in range(4):
        np.testing.assert_array_equal(y[:, 12 * r:12 * (r + 1), 0] // 3,
                                      np.broadcast_to(oracle.rank_positions(r, 4, 48, "zigzag"), (2, 12)) + 48 * np.arange(2)[:, None])
    with pytest.raises(ValueError):
        oracle.reorder(np.zeros((1, 30)), 4)


def test_striped_layout_and_roundtrip():
    S, P = 48, 4
    x = np.arange(2 * S * 3).reshape(2, S, 3)
    y = oracle.reorder_striped(x, P)
    np.testing.assert_array_equal(oracle.reorder_striped_inv(y, P), x)
    c = S // P
    seen = []
    for r in range(P):
        pos = y[0, c * r:c * (r + 1), 0] // 3        # the tokens a contiguous split hands rank r
        assert np.all(np.diff(pos) == P) and pos[0] == r   # striped: stride P from r
        np.testing.assert_array_equal(pos, oracle.rank_positions(r, P, S, "striped"))
        seen.extend(pos)
    assert sorted(seen) == list(range(S))             # every token exactly once
    with pytest.raises(ValueError):
        oracle.reorder_striped(np.zeros((1, 30)), 4)


@pytest.mark.parametrize("S,P", [(32, 4), (1024, 16), (96, 3)])
def test_striped_exact_pairs_every_rank_every_step(S, P):
    # query i of rank r sits at r + P*i, key j of block src at src + P*j: visible iff
    # j < i, or j == i and src <= r
    c = S // P
    total = 0
    for r in range(P):
        qpos = oracle.rank_positions(r, P, S, "striped")
        per_rank = 0
        for s in range(P):
            src = (r - s) % P
            n = oracle.visible_pairs(qpos, oracle.rank_positions(src, P, S, "striped"))
            assert n == c * (c - 1) // 2 + (c if src <= r else 0)
            per_rank += n
        assert per_rank == P * c * (c - 1) // 2 + c * (r + 1)
        total += per_rank
    assert total == S * (S + 1) // 2


def test_ring_counts_match_handbook():
    g = GOLDEN["ring_block_counts"]
    assert oracle.ring_block_counts(g["P"], g["S"], "contiguous") == g["counts"]
    # zigzag: every step of every rank holds visible pairs
    assert oracle.ring_block_counts(g["P"], g["S"], "zigzag") == [g["P"]] * g["P"]


@pytest.mark.parametrize("layout", ["contiguous", "zigzag", "striped"])
def test_ring_equals_full_attention_toy(layout):
    q, k, v = cp_inputs.toy_qkv()
    ref_o, ref_l = oracle.attn_fwd(q, k, v)
    for qpos, o, l in oracle.ring_fwd(q, k, v, 4, layout):
        np.testing.assert_allclose(o, ref_o[:, qpos], atol=1e-12)
        np.testing.assert_allclose(l, ref_l[:, :, qpos], atol=1e-12)


@pytest.mark.parametrize("layout", ["zigzag", "striped"])
def test_ring_packed_window_gqa_equals_full(layout):
    S, Hq, Hkv, D, P = 48, 4, 2, 4, 3
    q, k, v = rnd(1, S, Hq, D, seed=26), rnd(1, S, Hkv, D, seed=27), rnd(1, S, Hkv, D, seed=28)
    seg = np.repeat([0, 1, 2, 3], [5, 20, 9, 14])[None]
    ref_o, ref_l = oracle.attn_fwd(q, k, v, q_seg=seg, k_seg=seg, window=6)
    for qpos, o, l in oracle.ring_fwd(q, k, v, P, layout, seg=seg, window=6):
        np.testing.assert_allclose(o, ref_o[:, qpos], atol=1e-12)
        np.testing.assert_allclose(l, ref_l[:, :, qpos], atol=1e-12)


def test_ulysses_shapes_roundtrip_and_full():
    g = GOLDEN["ulysses_shapes"]
    q, k, v = (t.numpy().astype(np.float64) for t in cp_inputs.toy_qkv())
    P = g["P"]
    S = q.shape[1]
    xs = [q[:, r * S // P:(r + 1) * S // P] for r in range(P)]
    assert list(xs[0].shape[1:]) == g["input"]
    ys = oracle.seq_to_head(xs)
    assert list(ys[0].shape[1:]) == g["attention"]
    back = oracle.head_to_seq(ys)
    for a, b in zip(back, xs):
        np.testing.assert_array_equal(a, b)
    # rank p's heads are [2p, 2p+2) of the whole sequence
    np.testing.assert_array_equal(ys[1], q[:, :, 2:4])
    ref_o, ref_l = oracle.attn_fwd(q, k, v)
    out, lse, _ = oracle.ulysses_attn(q, k, v, P)
    np.testing.assert_allclose(out, ref_o, atol=1e-12)
    np.testing.assert_allclose(lse, ref_l, atol=1e-12)


def test_ulysses_stack_roundtrip_and_gqa_limit():
    P, B, S, H, D = 4, 2, 16, 8, 3
    st = rnd(P, B, S // P, H, D, seed=29)
    out = oracle.ulysses_relayout(st)
    assert out.shape == (P, B, S, H // P, D)
    np.testing.assert_array_equal(oracle.ulysses_relayout_inv(out), st)
    # explicit element map: out[p][b][s*S/P+i][hh] = in[s][b][i][p*H/P+hh]
    for p in range(P):
        for s in range(P):
            np.testing.assert_array_equal(out[p, :, s * 4:(s + 1) * 4], st[s, :, :, 2 * p:2 * p + 2])
    q, k, v = rnd(1, 16, 8, 4, seed=30), rnd(1, 16, 2, 4, seed=31), rnd(1, 16, 2, 4, seed=32)
    oracle.ulysses_attn(q, k, v, 2)
    with pytest.raises(ValueError):
        oracle.ulysses_attn(q, k, v, 4)  # degree above the kv head count


# ---------------------------------------------------------------- backward

def _loss(q, k, v, dout, kw):
    o, _ = oracle.attn_fwd(q, k, v, **kw)
    return float((o * dout).sum())


@pytest.mark.parametrize("kw", [dict(), dict(q_offset=3, k_offset=1), dict(window=2),
                                dict(q_seg=np.array([[0, 0, 1, 1, 1, 2]]), k_seg=np.array([[0, 0, 1, 1, 1, 2]]))])
def test_backward_finite_differences(kw):
    B, S, Hq, Hkv, D = 1, 6, 4, 2, 3
    q, k, v = rnd(B, S, Hq, D, seed=33), rnd(B, S, Hkv, D, seed=34), rnd(B, S, Hkv, D, seed=35)
    dout = rnd(B, S, Hq, D, seed=36)
    out, lse = oracle.attn_fwd(q, k, v, **kw)
    dq, dk, dv = oracle.attn_bwd(q, k, v, out, lse, dout, **kw)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + eps
            fp = _loss(q, k, v, dout, kw)
            x[idx] = old - eps
            fm = _loss(q, k, v, dout, kw)
            x[idx] = old
            num[idx] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(g, num, atol=1e-8)


def test_backward_invariants():
    B, S, Hq, Hkv, D = 2, 12, 4, 2, 5
    q, k, v = rnd(B, S, Hq, D, seed=37), rnd(B, S, Hkv, D, seed=38), rnd(B, S, Hkv, D, seed=39)
    dout = rnd(B, S, Hq, D, seed=40)
    out, lse = oracle.attn_fwd(q, k, v)
    dq, dk, dv = oracle.attn_bwd(q, k, v, out, lse, dout)
    np.testing.assert_allclose(dk.sum(axis=1), 0, atol=1e-12)          # shift invariance
    np.testing.assert_allclose(dv.sum(axis=1), dout.reshape(B, S, Hkv, 2, D).sum(axis=(1, 3)), atol=1e-12)


@pytest.mark.parametrize("Hq,Hkv,P,rep", [(8, 2, 4, 2), (8, 2, 8, 4), (8, 4, 8, 2)])
@pytest.mark.parametrize("masks", ["causal", "packed_window"])
def test_ulysses_beyond_kv_heads_equals_full(Hq, Hkv, P, rep, masks):
    """Degree P > kv heads with each kv head replicated rep times by group (handbook
    exercise): forward and all three gradients equal full attention's."""
    S, D = 32, 4
    q, k, v, do = (rnd(1, S, h, D, seed=60 + i) for i, h in enumerate((Hq, Hkv, Hkv, Hq)))
    m = {} if masks == "causal" else dict(q_seg=np.repeat([0, 1, 2], [9, 13, 10])[None],
                                          k_seg=np.repeat([0, 1, 2], [9, 13, 10])[None], window=5)
    ro, rl = oracle.attn_fwd(q, k, v, **m)
    with pytest.raises(ValueError):
        oracle.ulysses_attn(q, k, v, P, **m)           # not without replication
    o, l, _ = oracle.ulysses_attn(q, k, v, P, kv_rep=rep, **m)
    np.testing.assert_allclose(o, ro, atol=1e-12)
    np.testing.assert_allclose(l, rl, atol=1e-12)
    ref = oracle.attn_bwd(q, k, v, ro, rl, do, **m)
    got = oracle.ulysses_attn_bwd(q, k, v, do, P, kv_rep=rep, **m)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, atol=1e-12)


def test_replicate_and_sum_replicas():
    x = rnd(2, 3, 4, 5, seed=70)
    y = oracle.replicate_heads(x, 3)
    assert y.shape == (2, 3, 12, 5)
    for j in range(12):
        np.testing.assert_array_equal(y[:, :, j], x[:, :, j // 3])   # head j is kv head j // rep
    np.testing.assert_allclose(oracle.sum_replicas(y, 3), 3 * x)
    st = rnd(4, 1, 8, 2, 3, seed=71)                                  # [P][B][S/P][H][D]
    out = oracle.ulysses_relayout_rep(st, 2)                          # 4 heads over 4 ranks
    assert out.shape == (4, 1, 32, 1, 3)
    np.testing.assert_allclose(oracle.ulysses_relayout_inv_sum(out, 2), 2 * st)


@pytest.mark.parametrize("Pr,Pu,rep,masks", [(2, 2, 1, "causal"), (2, 4, 2, "causal"), (4, 2, 1, "packed_window"),
                                             (2, 2, 1, "noncausal")])
def test_usp_equals_full(Pr, Pu, rep, masks):
    """Ulysses within groups x zigzag ring across groups (USP) equals full attention."""
    S, Hq, Hkv, D = 32, 8, 2 if rep > 1 else 4, 4
    q, k, v = rnd(1, S, Hq, D, seed=72), rnd(1, S, Hkv, D, seed=73), rnd(1, S, Hkv, D, seed=74)
    m = dict(causal=masks != "noncausal")
    seg = None
    if masks == "packed_window":
        seg = np.repeat([0, 1, 2], [11, 7, 14])[None]
        m.update(window=6)
    ro, rl = oracle.attn_fwd(q, k, v, q_seg=seg, k_seg=seg, **m)
    o, l = oracle.usp_attn(q, k, v, Pr, Pu, kv_rep=rep, seg=seg, **m)
    np.testing.assert_allclose(o, ro, atol=1e-12)
    np.testing.assert_allclose(l, rl, atol=1e-12)
    st = rnd(Pr, Pu, 1, S // (Pr * Pu), Hq, D, seed=75)
    np.testing.assert_array_equal(oracle.usp_relayout_inv(oracle.usp_relayout(st)), st)


@pytest.mark.parametrize("layout", ["contiguous", "zigzag", "striped"])
def test_ring_backward_equals_full(layout):
    S, Hq, Hkv, D, P = 32, 4, 2, 4, 4
    q, k, v = rnd(1, S, Hq, D, seed=41), rnd(1, S, Hkv, D, seed=42), rnd(1, S, Hkv, D, seed=43)
    dout = rnd(1, S, Hq, D, seed=44)
    seg = np.repeat([0, 1, 2], [7, 15, 10])[None]
    kw = dict(q_seg=seg, k_seg=seg)
    out, lse = oracle.attn_fwd(q, k, v, **kw)
    ref = oracle.attn_bwd(q, k, v, out, lse, dout, **kw)
    finals = oracle.ring_fwd(q, k, v, P, layout, seg=seg)
    got = oracle.ring_bwd(q, k, v, dout, P, layout, finals, seg=seg)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, atol=1e-12)


def test_inputs_recipe():
    q, k, v = cp_inputs.toy_qkv()
    assert q.shape == (1, 32, 8, 16) and q.dtype == torch.float32
    lens = cp_inputs.doc_lengths(8192)
    assert sum(lens) == 8192 and all(256 <= n <= 4096 for n in lens[:-1])


# ---------------------------------------------------------------- padding to a multiple of P

@pytest.mark.parametrize("masks", ["causal", "noncausal", "packed_window"])
def test_end_padding_leaves_real_rows_unchanged(masks):
    """Padding at the end (zeros, positions continuing, pads in a segment of their own)
    changes no real row: plain attention, zigzag ring and Ulysses on the padded
    sequence equal unpadded full attention on the real rows."""
    S, Hq, Hkv, D, P = 29, 4, 2, 4, 4
    q, k, v = rnd(1, S, Hq, D, seed=80), rnd(1, S, Hkv, D, seed=81), rnd(1, S, Hkv, D, seed=82)
    m = dict(causal=masks != "noncausal")
    seg = np.repeat([0, 1, 2], [8, 12, 9])[None] if masks == "packed_window" else None
    if masks == "packed_window":
        m["window"] = 5
    ro, rl = oracle.attn_fwd(q, k, v, q_seg=seg, k_seg=seg, **m)
    Sp = oracle.padded_length(S, 2 * P)
    assert Sp == 32
    qp, kp, vp = (oracle.pad_rows(t, Sp) for t in (q, k, v))
    assert np.all(qp[:, S:] == 0) and np.array_equal(qp[:, :S], q)
    segp = oracle.pad_segments(seg if seg is not None else np.zeros((1, S), np.int64), Sp)
    assert np.all(segp[:, S:] == segp[:, :S].max() + 1)
    sm = dict(q_seg=segp, k_seg=segp) if (seg is not None or not m["causal"]) else {}
    o, l = oracle.attn_fwd(qp, kp, vp, **sm, **m)
    np.testing.assert_allclose(o[:, :S], ro, atol=1e-12)
    np.testing.assert_allclose(l[:, :, :S], rl, atol=1e-12)
    for qpos, o, l in oracle.ring_fwd(qp, kp, vp, P, "zigzag", seg=sm.get("q_seg"), **m):
        real = qpos < S
        np.testing.assert_allclose(o[:, real], ro[:, qpos[real]], atol=1e-12)
        np.testing.assert_allclose(l[:, :, real], rl[:, :, qpos[real]], atol=1e-12)
    if not sm:
        o, l, _ = oracle.ulysses_attn(qp, kp, vp, 2, **m)
        np.testing.assert_allclose(o[:, :S], ro, atol=1e-12)
    np.testing.assert_array_equal(oracle.pad_rows(qp, S), q)   # truncation undoes it
