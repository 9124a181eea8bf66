"""Kernel-level parity of the HIP path against the CPU oracle (GPU only).

Sizes span several tiles and a ragged tail; every mask kind, offsets, positions,
grouped heads and fully masked rows are covered.  Bars: permutations bit-exact;
attention float32 max-abs 1e-5 (out and lse); bf16 out 1e-2 and lse 1e-3; gradients
1e-2 * max(1, max|ref|) (bf16) and 1e-5 * max(1, max|ref|) (float32).
"""

import math
import os

import numpy as np
import pytest
import torch

import cp_inputs
import oracle

pytestmark = pytest.mark.gpu

TOL = {torch.float32: dict(out=1e-5, lse=1e-5, grad=1e-5), torch.bfloat16: dict(out=1e-2, lse=1e-3, grad=1e-2)}


@pytest.fixture(scope="module")
def cp():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import context_cp_attn_amd as cp
    cp.load_library()
    return cp


def say(*a):
    print(*a, flush=True)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bits of a CPU tensor as an integer numpy array (bf16 -> int16)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    return t.numpy()


def f64(t):
    return t.detach().cpu().double().numpy()


def check_lse(got, ref, tol):
    got = f64(got)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), "-inf pattern differs"
    fin = np.isfinite(ref)
    if fin.any():
        err = np.abs(got[fin] - ref[fin]).max()
        assert err <= tol, f"lse max-abs {err} > {tol}"


def check_close(got, ref, tol, what):
    err = np.abs(f64(got) - ref).max() if ref.size else 0.0
    assert err <= tol, f"{what} max-abs {err} > {tol}"


# --------------------------------------------------------------------- permutations

@pytest.mark.parametrize("P,B,S,H,D,dtype", [
    (4, 1, 32, 8, 16, torch.float32),      # toy
    (4, 2, 24, 8, 24, torch.bfloat16),     # 96-byte runs
    (3, 1, 15, 6, 7, torch.float32),       # 56-byte runs
    (2, 3, 10, 2, 3, torch.bfloat16),      # 6-byte runs
    (16, 1, 4096, 32, 128, torch.bfloat16),
    (1, 2, 9, 3, 5, torch.float32),         # degree 1: a plain copy
])
def test_ulysses_relayout_bit_exact(cp, P, B, S, H, D, dtype):
    say(f"relayout P={P} B={B} S={S} H={H} D={D} {dtype}")
    torch.manual_seed(1)
    x = torch.randn(P, B, S // P, H, D).to(dtype).cuda()
    y = cp.ulysses_relayout(x, P)
    np.testing.assert_array_equal(bits(y), oracle.ulysses_relayout(bits(x)))
    if P == 1:
        assert torch.equal(y, x)
    z = cp.ulysses_relayout_inv(y, P)
    assert torch.equal(z, x)
    np.testing.assert_array_equal(bits(z), oracle.ulysses_relayout_inv(bits(y)))


@pytest.mark.parametrize("G,P,B,S,H,D,dtype,rep", [
    (1, 4, 1, 64, 2, 128, torch.bfloat16, 2),     # kv heads replicated 2x (degree 2x the kv heads)
    (1, 8, 2, 64, 2, 64, torch.bfloat16, 4),
    (3, 2, 1, 32, 4, 16, torch.float32, 1),      # USP groups
    (2, 4, 1, 128, 2, 128, torch.bfloat16, 2),   # groups and replication
    (1, 3, 1, 12, 1, 7, torch.float32, 3),       # odd head size: 4-byte vectors
])
def test_relayout_ex(cp, G, P, B, S, H, D, dtype, rep):
    say(f"relayout_ex G={G} P={P} B={B} S={S} H={H} D={D} {dtype} rep={rep}")
    torch.manual_seed(2)
    x = torch.randn(G, P, B, S // P, H, D).to(dtype).cuda()
    y = cp.ulysses_relayout_ex(x, P, groups=G, rep=rep)
    ref = np.stack([oracle.ulysses_relayout_rep(bits(x[g]), rep) for g in range(G)])
    np.testing.assert_array_equal(bits(y), ref)
    if rep == 1:
        z = cp.ulysses_relayout_ex(y, P, groups=G, inverse=True)
        assert torch.equal(z, x)
        np.testing.assert_array_equal(bits(z), oracle.usp_relayout_inv(bits(y)))
    # inverse with copies summed (float32 gradients)
    g32 = torch.randn(y.shape, generator=torch.Generator().manual_seed(3)).cuda()
    z = cp.ulysses_relayout_ex(g32, P, groups=G, rep=rep, inverse=True)
    ref = np.stack([oracle.ulysses_relayout_inv_sum(f64(g32[g]), rep) for g in range(G)])
    check_close(z, ref, 1e-5 * max(1.0, np.abs(ref).max()), "inverse sum")


@pytest.mark.parametrize("Hq,Hkv,P", [(8, 2, 4), (8, 2, 8)])
def test_ulysses_beyond_kv_heads(cp, Hq, Hkv, P):
    """Degree P above the kv head count by replicating kv heads: out, lse and all
    gradients against the oracle's full attention."""
    S, D, rep = 512, 128, P // Hkv
    say(f"ulysses Hq={Hq} Hkv={Hkv} P={P} rep={rep}")
    q, k, v, do = cp_inputs.normal_tensors([(1, S, Hq, D), (1, S, Hkv, D), (1, S, Hkv, D), (1, S, Hq, D)], seed=11)
    st = lambda t: t.reshape(P, 1, S // P, t.shape[2], D).cuda()
    out, lse, rel = cp.drivers.ulysses_forward(st(q), st(k), st(v), P, kv_rep=rep)
    ro, rl = oracle.attn_fwd(q, k, v)
    check_close(out.reshape(1, S, Hq, D), ro, 1e-2, "out")
    check_lse(torch.cat(list(lse), dim=1), rl, 1e-3)
    dq, dk, dv = cp.drivers.ulysses_backward(rel, lse, st(do), P, kv_rep=rep)
    refs = oracle.attn_bwd(q, k, v, ro, rl, do)
    for got, ref, nm in zip((dq, dk, dv), refs, ("dq", "dk", "dv")):
        check_close(got.reshape(ref.shape), ref, 1e-2 * max(1.0, np.abs(ref).max()), nm)


@pytest.mark.parametrize("Pr,Pu,Hkv,masks,dtype", [
    (2, 4, 2, "causal", torch.bfloat16),          # kv heads replicated inside the groups
    (4, 2, 2, "packed_window", torch.bfloat16),
    (2, 2, 8, "causal", torch.float32),
])
def test_usp_forward(cp, Pr, Pu, Hkv, masks, dtype):
    """Ulysses within groups x zigzag ring across groups against full attention."""
    S, Hq = 1024, 8
    D = 128 if dtype == torch.bfloat16 else 32
    rep = max(1, Pu // Hkv)
    say(f"usp Pr={Pr} Pu={Pu} Hkv={Hkv} rep={rep} {masks} {dtype}")
    q, k, v = cp_inputs.normal_tensors([(1, S, Hq, D), (1, S, Hkv, D), (1, S, Hkv, D)], seed=12, dtype=dtype)
    seg, window = None, 0
    if masks == "packed_window":
        seg = cp_inputs.random_segment_ids(S, 40, 300, seed=13)
        window = 100
    out, _ = cp.drivers.usp_forward(q.cuda(), k.cuda(), v.cuda(), Pr, Pu, kv_rep=rep,
                                    seg=None if seg is None else seg.cuda(), window=window)
    sm = {} if seg is None else dict(q_seg=seg.numpy(), k_seg=seg.numpy())
    ro, rl = oracle.attn_fwd(q, k, v, window=window, **sm)
    check_close(out, ro, TOL[dtype]["out"], "usp out")


@pytest.mark.parametrize("Pr,Pu,Hkv,masks,dtype", [
    (2, 4, 2, "causal", torch.bfloat16),          # kv heads replicated inside the groups
    (4, 2, 2, "packed_window", torch.bfloat16),
    (2, 2, 8, "causal", torch.float32),
    (2, 8, 8, "causal", torch.bfloat16),          # the degree-16 split of the pages' exercise: Ulysses 8 x ring 2
])
def test_usp_backward(cp, Pr, Pu, Hkv, masks, dtype):
    """Gradients through Ulysses within groups x zigzag ring across groups against
    the oracle's gradients of full attention (dq, dk, dv on every element)."""
    S, Hq = 1024, 8 if Pu < 8 else 32
    D = 128 if dtype == torch.bfloat16 else 32
    rep = max(1, Pu // Hkv)
    say(f"usp bwd Pr={Pr} Pu={Pu} Hkv={Hkv} rep={rep} {masks} {dtype}")
    q, k, v, do = cp_inputs.normal_tensors([(1, S, Hq, D), (1, S, Hkv, D), (1, S, Hkv, D), (1, S, Hq, D)],
                                           seed=14, dtype=dtype)
    seg, window = None, 0
    if masks == "packed_window":
        seg = cp_inputs.random_segment_ids(S, 40, 300, seed=13)
        window = 100
    out, lse, state = cp.drivers.usp_forward(q.cuda(), k.cuda(), v.cuda(), Pr, Pu, kv_rep=rep,
                                             seg=None if seg is None else seg.cuda(), window=window, keep=True)
    dq, dk, dv = cp.drivers.usp_backward(state, lse, do.cuda())
    sm = {} if seg is None else dict(q_seg=seg.numpy(), k_seg=seg.numpy())
    ro, rl = oracle.attn_fwd(q, k, v, window=window, **sm)
    check_close(out, ro, TOL[dtype]["out"], "usp out")
    refs = oracle.attn_bwd(q, k, v, ro, rl, do, window=window, **sm)
    for got, ref, nm in zip((dq, dk, dv), refs, ("dq", "dk", "dv")):
        check_close(got, ref, TOL[dtype]["grad"] * max(1.0, np.abs(ref).max()), f"usp {nm}")


@pytest.mark.parametrize("shape,S_out,fill,dtype", [
    ((1, 1001, 32, 128), 1008, 0, torch.bfloat16),
    ((2, 37), 40, 7, torch.int32),          # segment ids: pads get id 7
    ((3, 10, 5), 16, 0, torch.uint8),
    ((1, 1008, 8), 1001, 0, torch.float32),  # truncation removes padding
])
def test_pad_rows(cp, shape, S_out, fill, dtype):
    say(f"pad_rows {shape} -> {S_out} fill={fill} {dtype}")
    n = int(np.prod(shape))
    x = (torch.arange(n, dtype=torch.int64) % 251).to(dtype).reshape(shape) if dtype in (torch.int32, torch.uint8) \
        else torch.randn(shape).to(dtype)
    y = cp.pad_rows(x.cuda(), S_out, fill=fill)
    np.testing.assert_array_equal(bits(y), oracle.pad_rows(bits(x), S_out, fill=fill))


@pytest.mark.parametrize("scheme,causal", [("ring", True), ("ring", False), ("ulysses", True)])
def test_padded_sequence_attention(cp, scheme, causal):
    """A sequence no CP degree divides, padded at its end: the real rows of the ring
    (zigzag) or Ulysses result equal unpadded full attention's."""
    S, Hq, Hkv, D, P = 1001, 4, 4, 128, 4
    say(f"padded {scheme} causal={causal} S={S} P={P}")
    q, k, v = cp_inputs.normal_tensors([(1, S, Hq, D), (1, S, Hkv, D), (1, S, Hkv, D)], seed=14)
    ro, rl = oracle.attn_fwd(q, k, v, causal=causal)
    mult = 2 * P if scheme == "ring" else P
    (qp, S0), (kp, _), (vp, _) = (cp.drivers.pad_sequence(t.cuda(), mult) for t in (q, k, v))
    Sp = qp.shape[1]
    assert S0 == S and Sp % mult == 0
    if scheme == "ring":
        seg = None
        if not causal:   # pads in a segment of their own
            seg = cp.drivers.pad_segments(torch.zeros(1, S, dtype=torch.int32, device="cuda"), mult, pad_id=1)
            seg = cp.zigzag_reorder(seg, P)
        qz, kz, vz = (cp.zigzag_reorder(t, P) for t in (qp, kp, vp))
        for r in range(P):
            acc, lse = cp.drivers.RingShare(qz, kz, vz, P, r, seg=seg, causal=causal).forward()
            pos = oracle.rank_positions(r, P, Sp, "zigzag")
            real = pos < S
            check_close(acc[:, real], ro[:, pos[real]], 1e-2, f"rank {r} out")
            check_lse(lse[:, :, real], rl[:, :, pos[real]], 1e-3)
    else:
        st = lambda t: t.reshape(P, 1, Sp // P, t.shape[2], D)
        out, lse, _ = cp.drivers.ulysses_forward(st(qp), st(kp), st(vp), P)
        check_close(out.reshape(1, Sp, Hq, D)[:, :S], ro, 1e-2, "out")
        check_lse(torch.cat(list(lse), dim=1)[:, :, :S], rl, 1e-3)


@pytest.mark.parametrize("strategy", [0, 1])
@pytest.mark.parametrize("shape,P,dtype", [
    ((1, 65536), 4, torch.int32),
    ((2, 48, 3, 5), 3, torch.bfloat16),
    ((1, 32, 8, 16), 4, torch.float32),
    ((3, 40, 7), 5, torch.uint8),
    ((1, 4096, 4096), 4, torch.bfloat16),
    ((2, 30, 3), 5, torch.int32),
    ((2, 6, 3), 1, torch.float32),          # one rank: the identity
])
def test_reorder_bit_exact(cp, shape, P, dtype, strategy):
    """strategy 0 = dual-chunk-swap (zigzag), 1 = striped."""
    if strategy == 0 and shape[1] % (2 * P):
        pytest.skip("dual-chunk-swap needs S divisible by 2P")
    say(f"reorder {shape} P={P} {dtype} strategy={strategy}")
    n = int(np.prod(shape))
    x = (torch.arange(n, dtype=torch.int64) * 2654435761 % 251).to(dtype).reshape(shape).cuda() \
        if dtype in (torch.int32, torch.uint8) else torch.randn(shape).to(dtype).cuda()
    fwd, inv = ((oracle.reorder, oracle.reorder_inv) if strategy == 0
                else (oracle.reorder_striped, oracle.reorder_striped_inv))
    y = cp.zigzag_reorder(x, P, strategy=strategy)
    np.testing.assert_array_equal(bits(y), fwd(bits(x), P))
    if P == 1:
        assert torch.equal(y, x)
    z = cp.zigzag_reorder(y, P, inverse=True, strategy=strategy)
    np.testing.assert_array_equal(bits(z), inv(bits(y), P))
    assert torch.equal(z, x)


# --------------------------------------------------------------------- merge

@pytest.mark.parametrize("blk_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [16, 128])
def test_lse_merge(cp, blk_dtype, D):
    say(f"merge D={D} {blk_dtype}")
    B, S, H = 2, 37, 3
    g = torch.Generator().manual_seed(2)
    o1 = torch.randn(B, S, H, D, generator=g)
    o2 = torch.randn(B, S, H, D, generator=g).to(blk_dtype)
    l1 = torch.randn(B, H, S, generator=g) * 3
    l2 = torch.randn(B, H, S, generator=g) * 3
    l1[0, 0, :5] = -float("inf")
    l2[0, 0, 3:8] = -float("inf")   # rows 3,4: both empty
    l2[1, 2, 10:] = -float("inf")
    acc, lacc = o1.cuda(), l1.cuda()
    cp.lse_merge(acc, lacc, o2.cuda(), l2.cuda())
    ref_o, ref_l = oracle.lse_merge(f64(o1), f64(l1), f64(o2), f64(l2))
    check_lse(lacc, ref_l, 1e-5)
    check_close(acc, ref_o, 1e-5, "merged out")


# --------------------------------------------------------------------- attention

CASES = {
    # name: (B, Sq, Sk, Hq, Hkv, mask kwargs builder)
    "causal_square": (1, 300, 300, 4, 2, lambda Sq, Sk: dict()),
    "noncausal": (2, 200, 333, 2, 2, lambda Sq, Sk: dict(causal=False)),
    "offsets": (1, 160, 410, 4, 1, lambda Sq, Sk: dict(q_offset=250, k_offset=0)),
    "zigzag_pos": (1, 256, 256, 2, 2, lambda Sq, Sk: dict(
        q_pos=np.r_[np.arange(0, 128), np.arange(896, 1024)], k_pos=np.r_[np.arange(384, 512), np.arange(512, 640)])),
    "packed_window": (1, 520, 520, 4, 2, lambda Sq, Sk: dict(seg=[37, 150, 90, 243], window=64)),
    "empty_rows": (1, 130, 190, 2, 1, lambda Sq, Sk: dict(q_offset=0, k_offset=64)),
    # a window with the causal flag off: the window bounds qpos - kpos on both sides
    # (0 <= qpos - kpos < 37), so later keys stay hidden
    "noncausal_window": (1, 210, 260, 2, 1, lambda Sq, Sk: dict(causal=False, window=37, q_offset=40)),
    # a window of 1: each row sees only the key at its own position
    "window_1": (1, 150, 150, 2, 2, lambda Sq, Sk: dict(window=1)),
    # offsets and a window that leaves the first rows with no visible key
    "offset_window": (1, 140, 300, 2, 1, lambda Sq, Sk: dict(q_offset=20, k_offset=100, window=50)),
    # three query heads per kv head: the backward splits the group's heads into
    # uneven halves (1 + 2)
    "gqa3": (1, 200, 330, 6, 2, lambda Sq, Sk: dict(q_offset=130)),
    # one query head per kv head and positions from offsets: the backward's paired
    # dK / dV role (96-row query tiles: ragged, offsets, rows that see no key, batch 2)
    "mha_ragged": (2, 301, 301, 2, 2, lambda Sq, Sk: dict()),
    "mha_offsets": (1, 170, 430, 3, 3, lambda Sq, Sk: dict(q_offset=260, k_offset=0)),
    "mha_empty_rows": (1, 200, 290, 2, 2, lambda Sq, Sk: dict(q_offset=0, k_offset=97)),
}


def make_case(name, D, dtype, seed=0):
    B, Sq, Sk, Hq, Hkv, mk = CASES[name]
    q, k, v, do = cp_inputs.normal_tensors([(B, Sq, Hq, D), (B, Sk, Hkv, D), (B, Sk, Hkv, D), (B, Sq, Hq, D)],
                                           seed=seed, dtype=dtype)
    m = mk(Sq, Sk)
    if "seg" in m:
        seg = cp_inputs.segment_ids(m.pop("seg"), batch=B)
        m["q_seg"] = seg
        m["k_seg"] = seg
    return (q, k, v, do), m


def to_dev(m):
    out = {}
    for key, val in m.items():
        if isinstance(val, np.ndarray):
            val = torch.from_numpy(val.astype(np.int32))
        if isinstance(val, torch.Tensor):
            val = val.to(torch.int32).contiguous().cuda()
        out[key] = val
    return out


def oracle_mask(m):
    return {k: (v.numpy() if isinstance(v, torch.Tensor) else v) for k, v in m.items()}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("dtype,D", [(torch.float32, 16), (torch.float32, 128), (torch.bfloat16, 32),
                                     (torch.bfloat16, 64), (torch.bfloat16, 128),
                                     (torch.bfloat16, 16), (torch.bfloat16, 96)])  # row-per-wavefront bf16
def test_attn_fwd(cp, name, dtype, D):
    say(f"attn_fwd {name} D={D} {dtype}")
    (q, k, v, _), m = make_case(name, D, dtype)
    out, lse = cp.attn_fwd(q.cuda(), k.cuda(), v.cuda(), **to_dev(m))
    ref_o, ref_l = oracle.attn_fwd(q, k, v, **oracle_mask(m))
    check_lse(lse, ref_l, TOL[dtype]["lse"])
    check_close(out, ref_o, TOL[dtype]["out"], "out")
    empty = np.isneginf(ref_l)
    if empty.any():  # rows with no visible key are exactly zero
        o = f64(out).transpose(0, 2, 1, 3)
        assert np.all(o[empty] == 0)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("dtype,D", [(torch.float32, 16), (torch.float32, 128), (torch.bfloat16, 32),
                                     (torch.bfloat16, 128), (torch.bfloat16, 16)])
def test_attn_fwd_merge(cp, name, dtype, D):
    """Fused ring step = the oracle's merge of the oracle's block attention into a
    running (acc, lse) that has -inf rows, finite rows and rows that stay empty."""
    say(f"attn_fwd_merge {name} D={D} {dtype}")
    (q, k, v, _), m = make_case(name, D, dtype, seed=6)
    B, Sq, Hq, _ = q.shape
    g = torch.Generator().manual_seed(7)
    acc0 = torch.randn(B, Sq, Hq, D, generator=g)
    lse0 = torch.randn(B, Hq, Sq, generator=g) * 2 + 3
    lse0[..., ::5] = -float("inf")
    acc0[lse0.transpose(1, 2) == -float("inf")] = 0.0   # a ring starts from acc = 0, lse = -inf
    acc, lacc = acc0.cuda(), lse0.cuda()
    cp.attn_fwd_merge(q.cuda(), k.cuda(), v.cuda(), acc, lacc, **to_dev(m))
    blk_o, blk_l = oracle.attn_fwd(q, k, v, **oracle_mask(m))
    ref_o, ref_l = oracle.lse_merge(f64(acc0), f64(lse0), blk_o, blk_l)
    check_lse(lacc, ref_l, TOL[dtype]["lse"])
    check_close(acc, ref_o, TOL[dtype]["out"], "merged out")
    # and the unfused pair gives the same result within the bar
    acc2, lacc2 = acc0.cuda(), lse0.cuda()
    o, l = cp.attn_fwd(q.cuda(), k.cuda(), v.cuda(), **to_dev(m))
    cp.lse_merge(acc2, lacc2, o, l)
    check_close(acc, f64(acc2), TOL[dtype]["out"], "fused vs unfused")



@pytest.mark.parametrize("case", ["64_tiles", "64_tiles_and_1_key", "65_tiles", "causal_straddle"])
@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.bfloat16, 32),
                                     (torch.float32, 128)])
def test_attn_fwd_merge_group_sync_boundary(cp, case, dtype, D):
    """The fused ring step on a grid of few query tiles walks each tile's keys with two
    key groups of one workgroup.  Each group waits only for its own waves after a key
    tile when the workgroup's live keys span at most 64 tiles of 64 keys, and for the
    whole workgroup otherwise.  Both sides of that limit against the oracle: 4096 keys
    (64 tiles), 4097 (a 65th tile of one key), 4160 (65 full tiles), and a causal
    problem whose first query tile sees exactly 64 tiles and whose second sees 66."""
    Sq, Hq, Hkv = 256, 2, 1
    Sk, m = {"64_tiles": (4096, dict(causal=False)), "64_tiles_and_1_key": (4097, dict(causal=False)),
             "65_tiles": (4160, dict(causal=False)),
             "causal_straddle": (4300, dict(q_offset=4096 - 128, k_offset=0))}[case]
    say(f"attn_fwd_merge group-sync boundary {case} D={D} {dtype}")
    q, k, v = cp_inputs.normal_tensors([(1, Sq, Hq, D), (1, Sk, Hkv, D), (1, Sk, Hkv, D)], seed=41, dtype=dtype)
    g = torch.Generator().manual_seed(42)
    acc0 = torch.randn(1, Sq, Hq, D, generator=g)
    lse0 = torch.randn(1, Hq, Sq, generator=g) + 4
    acc, lacc = acc0.cuda(), lse0.cuda()
    cp.attn_fwd_merge(q.cuda(), k.cuda(), v.cuda(), acc, lacc, **to_dev(m))
    blk_o, blk_l = oracle.attn_fwd(q, k, v, **oracle_mask(m))
    ref_o, ref_l = oracle.lse_merge(f64(acc0), f64(lse0), blk_o, blk_l)
    check_lse(lacc, ref_l, TOL[dtype]["lse"])
    check_close(acc, ref_o, TOL[dtype]["out"], "merged out")

@pytest.mark.parametrize("name", ["causal_square", "offsets", "zigzag_pos", "packed_window", "empty_rows",
                                  "noncausal_window", "window_1", "offset_window", "gqa3", "noncausal",
                                  "mha_ragged", "mha_offsets", "mha_empty_rows"])
@pytest.mark.parametrize("dtype,D", [(torch.float32, 16), (torch.float32, 128), (torch.bfloat16, 64),
                                     (torch.bfloat16, 128), (torch.bfloat16, 16)])
def test_attn_bwd(cp, name, dtype, D):
    say(f"attn_bwd {name} D={D} {dtype}")
    (q, k, v, do), m = make_case(name, D, dtype, seed=3)
    dm = to_dev(m)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    out, lse = cp.attn_fwd(qd, kd, vd, **dm)
    dq, dk, dv = cp.attn_bwd(qd, kd, vd, out, lse, dod, **dm)
    om = oracle_mask(m)
    ref_o, ref_l = oracle.attn_fwd(q, k, v, **om)
    refs = oracle.attn_bwd(q, k, v, ref_o, ref_l, do, **om)
    for got, ref, nm in zip((dq, dk, dv), refs, ("dq", "dk", "dv")):
        check_close(got, ref, TOL[dtype]["grad"] * max(1.0, np.abs(ref).max()), nm)
    # accumulate adds onto what is there
    dq2, dk2, dv2 = cp.attn_bwd(qd, kd, vd, out, lse, dod, dq=dq.clone(), dk=dk.clone(), dv=dv.clone(),
                                accumulate=True, **dm)
    for a, b in ((dq2, dq), (dk2, dk), (dv2, dv)):
        torch.testing.assert_close(a, 2 * b, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 16)])
def test_attn_bwd_rows_ready(cp, dtype, D):
    """cp_attn_bwd_rows_ready: a second kv block's gradients with the per-row values
    the first call left in the workspace equal a fresh call's, bit for bit."""
    say(f"attn_bwd rows_ready D={D} {dtype}")
    Sq, Sk, Hq, Hkv = 300, 260, 4, 2
    q, k, v, k2, v2, do = (t.cuda() for t in cp_inputs.normal_tensors(
        [(1, Sq, Hq, D), (1, Sk, Hkv, D), (1, Sk, Hkv, D), (1, Sk, Hkv, D), (1, Sk, Hkv, D), (1, Sq, Hq, D)],
        seed=17, dtype=dtype))
    m = dict(q_offset=Sk)
    out, lse = cp.attn_fwd(q, k, v, **m)
    ws = cp.bwd_workspace(q, k, **m)
    cp.attn_bwd(q, k, v, out, lse, do, workspace=ws, **m)
    got = cp.attn_bwd(q, k2, v2, out, lse, do, workspace=ws, rows_ready=True, **m)
    ref = cp.attn_bwd(q, k2, v2, out, lse, do, **m)
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
    with pytest.raises(ValueError):
        cp.attn_bwd(q, k2, v2, out, lse, do, rows_ready=True, **m)


@pytest.mark.parametrize("masks", ["long_docs", "long_window"])
def test_attn_long_masked_ranges(cp, masks):
    """Segmented or windowed problems whose workgroups see more than 64 tiles: the
    kernels classify ranges of up to 64 tiles at once (one per lane) and walk longer
    ones tile by tile.  Documents of 400 and 8600 tokens put both kinds in one
    launch of the forward (64-key tiles: up to 134 in a range) and of the backward
    (128-row tiles: up to 68); a 7000-token window without segment ids gives the
    forward up to 110.  Forward through the two-workgroup split (workspace), the
    in-workgroup split (none) and the fused ring step; backward; all against the
    oracle, bf16, D=128."""
    S, Hq, Hkv, D = 9000, 2, 1, 128
    say(f"attn long masked ranges {masks}")
    q, k, v, do = cp_inputs.normal_tensors([(1, S, Hq, D), (1, S, Hkv, D), (1, S, Hkv, D), (1, S, Hq, D)],
                                           seed=31, dtype=torch.bfloat16)
    if masks == "long_docs":
        seg = cp_inputs.segment_ids([400, 8600], batch=1)
        m = dict(q_seg=seg, k_seg=seg)
    else:
        m = dict(window=7000)
    dm = to_dev(m)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    ws = cp.fwd_workspace(qd, kd, **dm)
    assert ws is not None
    out, lse = cp.attn_fwd(qd, kd, vd, workspace=ws, **dm)
    out1, lse1 = cp.attn_fwd(qd, kd, vd, workspace=False, **dm)
    acc = torch.zeros(1, S, Hq, D, device="cuda")
    lacc = torch.full((1, Hq, S), float("-inf"), device="cuda")
    cp.attn_fwd_merge(qd, kd, vd, acc, lacc, **dm)
    dq, dk, dv = cp.attn_bwd(qd, kd, vd, out, lse, dod, **dm)
    om = oracle_mask(m)
    ref_o, ref_l = oracle.attn_fwd(q, k, v, **om)
    for o_, l_, nm in ((out, lse, "split"), (out1, lse1, "unsplit"), (acc, lacc, "fused")):
        check_lse(l_, ref_l, 1e-3)
        check_close(o_, ref_o, 1e-2, f"{nm} out")
    refs = oracle.attn_bwd(q, k, v, ref_o, ref_l, do, **om)
    for got, ref, nm in zip((dq, dk, dv), refs, ("dq", "dk", "dv")):
        check_close(got, ref, TOL[torch.bfloat16]["grad"] * max(1.0, np.abs(ref).max()), nm)


def _expected_flags(B, qp, kp, qs, ks):
    """The rules of cp_attn_check_args written with numpy."""
    f = 0
    for bit, pos in ((1, qp), (2, kp)):
        if pos is not None and ((np.diff(pos) <= 0).any() or (pos < 0).any()):
            f |= bit
    for bit, seg in ((4, qs), (8, ks)):
        if seg is not None and (np.diff(seg.reshape(B, -1), axis=1) < 0).any():
            f |= bit
    return f


def test_check_attn_args(cp, monkeypatch):
    """Violation bits of the device check equal the numpy rules, bit for bit; the
    CP_ATTN_DEBUG mode raises before launching on a violation."""
    say("check_attn_args")
    from context_cp_attn_amd import ops
    B, Sq, Sk = 2, 700, 515
    q = torch.zeros(B, Sq, 2, 16, device="cuda")
    k = torch.zeros(B, Sk, 1, 16, device="cuda")
    rng = np.random.default_rng(11)
    seen = set()
    for trial in range(40):
        # strictly increasing positions / non-decreasing ids (each row of the segment
        # ids restarts, which is allowed), then up to one planted defect per array
        qp = np.cumsum(rng.integers(1, 4, Sq)) - 1
        kp = np.cumsum(rng.integers(1, 4, Sk)) + 7
        qs = np.concatenate([np.sort(rng.integers(0, 5, Sq)) for _ in range(B)])
        ks = np.concatenate([np.sort(rng.integers(0, 5, Sk)) for _ in range(B)])
        for arr in (qp, kp, qs, ks):
            kind = rng.integers(0, 4)
            i = int(rng.integers(0, arr.size - 1))
            if kind == 1:
                arr[i + 1] = arr[i]            # a repeat: breaks strictness only
            elif kind == 2:
                arr[i + 1] = arr[i] - 1        # a step down
            elif kind == 3:
                arr[0] = -1 - int(rng.integers(0, 3))   # a negative first entry
        want = _expected_flags(B, qp, kp, qs, ks)
        seen.add(want)
        t = lambda x: torch.from_numpy(x.astype(np.int32)).cuda()
        msgs = cp.check_attn_args(q, k, q_pos=t(qp), k_pos=t(kp), q_seg=t(qs), k_seg=t(ks))
        got = sum(bit for bit, msg in ops._CHECK_BITS.items() if msg in msgs)
        assert got == want, (trial, got, want)
    assert 0 in seen and len(seen) > 4
    # NULL arrays are skipped
    assert cp.check_attn_args(q, k) == []
    # debug mode: a violation raises before any launch; valid arrays run normally
    monkeypatch.setattr(ops, "DEBUG", True)
    v = torch.zeros_like(k)
    bad = torch.arange(Sq, dtype=torch.int32, device="cuda").flip(0).contiguous()
    with pytest.raises(ValueError, match="q_pos"):
        cp.attn_fwd(q, k, v, q_pos=bad)
    out, lse = cp.attn_fwd(q, k, v, q_pos=torch.arange(Sq, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all()


@pytest.mark.parametrize("many_tiles", [False, True])
@pytest.mark.parametrize("masks", ["causal_offset", "packed_window"])
def test_attn_fwd_grid_variants(cp, many_tiles, masks):
    """The forward splits each query tile's keys over two wavefront groups of one
    workgroup when the grid has fewer than 4 query tiles (of 128 rows) per CU, and
    runs whole tiles otherwise; both variants against the oracle, plain (with and
    without a workspace: with 1000 keys cp_attn_fwd_ws does not split) and
    fused-merge, D=128."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    S, Hq, Hkv, D = 1000, 8, 2, 128
    tiles_per_batch = ((S + 127) // 128) * Hq
    B = -(-4 * cus // tiles_per_batch) if many_tiles else 1   # >= 4 tiles per CU, or far fewer
    say(f"attn_fwd grid variant many_tiles={many_tiles} B={B} {masks}")
    q, k, v = cp_inputs.normal_tensors([(B, S, Hq, D), (B, S, Hkv, D), (B, S, Hkv, D)], seed=8)
    if masks == "causal_offset":
        m = dict(q_offset=S // 3, k_offset=0)
    else:
        seg = cp_inputs.random_segment_ids(S, 60, 400, seed=9, batch=B)
        m = dict(q_seg=seg, k_seg=seg, window=150)
    dm = to_dev(m)
    out, lse = cp.attn_fwd(q.cuda(), k.cuda(), v.cuda(), **dm)                      # workspace path
    out1, lse1 = cp.attn_fwd(q.cuda(), k.cuda(), v.cuda(), workspace=False, **dm)   # cp_attn_fwd
    acc = torch.zeros(B, S, Hq, D, device="cuda")
    lacc = torch.full((B, Hq, S), float("-inf"), device="cuda")
    cp.attn_fwd_merge(q.cuda(), k.cuda(), v.cuda(), acc, lacc, **dm)
    # the oracle on a sample of batches (every batch element runs the same code)
    bs = sorted({0, B - 1})
    om = oracle_mask({k_: (v_[bs] if k_ in ("q_seg", "k_seg") else v_) for k_, v_ in m.items()})
    ref_o, ref_l = oracle.attn_fwd(q[bs], k[bs], v[bs], **om)
    check_lse(lse[bs], ref_l, 1e-3)
    check_close(out[bs], ref_o, 1e-2, "out")
    check_lse(lse1[bs], ref_l, 1e-3)
    check_close(out1[bs], ref_o, 1e-2, "out without workspace")
    check_lse(lacc[bs], ref_l, 1e-3)
    check_close(acc[bs], ref_o, 1e-2, "fused out")


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("masks", ["causal_offset", "empty_rows", "packed_window", "batch2"])
def test_attn_fwd_split(cp, D, masks):
    """cp_attn_fwd_ws on a grid small enough to split the keys of every query tile
    over two workgroups (>= 8192 keys, a ragged last key tile): the combined result
    against the oracle, and against cp_attn_fwd (no workspace)."""
    Sq, Sk, Hq, Hkv = 300, 8400, 4, 2
    B = 2 if masks == "batch2" else 1
    say(f"attn_fwd split D={D} {masks}")
    q, k, v = cp_inputs.normal_tensors([(B, Sq, Hq, D), (B, Sk, Hkv, D), (B, Sk, Hkv, D)], seed=12)
    if masks in ("causal_offset", "batch2"):   # the last rows see every key
        m = dict(q_offset=Sk - 150, k_offset=0)
    elif masks == "empty_rows":       # rows 0..99 precede every key
        m = dict(q_offset=0, k_offset=100)
    else:                             # queries at positions 8000.. inside packed documents
        kseg = cp_inputs.random_segment_ids(Sk, 500, 3000, seed=13)
        qpos = np.arange(8000, 8000 + Sq)
        m = dict(q_pos=qpos, k_pos=np.arange(Sk), q_seg=kseg[:, 8000:8000 + Sq].contiguous(), k_seg=kseg,
                 window=2500)
    dm = to_dev(m)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    ws = cp.fwd_workspace(qd, kd, **dm)
    assert ws is not None
    out, lse = cp.attn_fwd(qd, kd, vd, workspace=ws, **dm)
    out1, lse1 = cp.attn_fwd(qd, kd, vd, workspace=False, **dm)
    ref_o, ref_l = oracle.attn_fwd(q, k, v, **oracle_mask(m))
    check_lse(lse, ref_l, 1e-3)
    check_close(out, ref_o, 1e-2, "split out")
    empty = np.isneginf(ref_l)
    if empty.any():
        assert np.all(f64(out).transpose(0, 2, 1, 3)[empty] == 0)
    check_close(out, f64(out1), 1e-2, "split vs unsplit")


@pytest.mark.parametrize("Sq,Sk", [(1, 1), (1, 300), (300, 1), (33, 65), (1, 8193)])
@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.bfloat16, 16),
                                     (torch.float32, 16)])
@pytest.mark.parametrize("causal", [True, False])
def test_attn_tiny_and_ragged(cp, Sq, Sk, dtype, D, causal):
    """Degenerate shapes: one query row, one key, lengths one past a tile, and a
    single row against 8193 keys (the split forward with one ragged key tile);
    forward (with and without a workspace) and backward against the oracle.  With
    causal masking and q_offset = Sk - Sq (>= 0) every row sees a key."""
    say(f"attn tiny Sq={Sq} Sk={Sk} D={D} {dtype} causal={causal}")
    q, k, v, do = cp_inputs.normal_tensors([(1, Sq, 2, D), (1, Sk, 1, D), (1, Sk, 1, D), (1, Sq, 2, D)],
                                           seed=21, dtype=dtype)
    m = dict(causal=causal, q_offset=max(Sk - Sq, 0))
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    out, lse = cp.attn_fwd(qd, kd, vd, **m)
    out1, lse1 = cp.attn_fwd(qd, kd, vd, workspace=False, **m)
    dq, dk, dv = cp.attn_bwd(qd, kd, vd, out, lse, dod, **m)
    ref_o, ref_l = oracle.attn_fwd(q, k, v, **m)
    refs = oracle.attn_bwd(q, k, v, ref_o, ref_l, do, **m)
    for o_, l_, nm in ((out, lse, "ws"), (out1, lse1, "no ws")):
        check_lse(l_, ref_l, TOL[dtype]["lse"])
        check_close(o_, ref_o, TOL[dtype]["out"], f"out ({nm})")
    for got, ref, nm in zip((dq, dk, dv), refs, ("dq", "dk", "dv")):
        check_close(got, ref, TOL[dtype]["grad"] * max(1.0, np.abs(ref).max()), nm)


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_deterministic(cp, dtype, D):
    say(f"determinism {dtype} D={D}")
    (q, k, v, do), m = make_case("packed_window", D, dtype, seed=4)
    dm = to_dev(m)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    r1 = cp.attn_fwd(qd, kd, vd, **dm)
    r2 = cp.attn_fwd(qd, kd, vd, **dm)
    assert all(torch.equal(a, b) for a, b in zip(r1, r2))
    g1 = cp.attn_bwd(qd, kd, vd, *r1, dod, **dm)
    g2 = cp.attn_bwd(qd, kd, vd, *r1, dod, **dm)
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))


def test_single_token_and_gqa_8(cp):
    say("attn single token / GQA 8")
    q, k, v = cp_inputs.normal_tensors([(1, 1, 8, 128), (1, 1, 1, 128), (1, 1, 1, 128)], seed=5)
    out, lse = cp.attn_fwd(q.cuda(), k.cuda(), v.cuda())
    ref_o, ref_l = oracle.attn_fwd(q, k, v)
    check_lse(lse, ref_l, 1e-3)
    check_close(out, ref_o, 1e-2, "out")


def _random_problem(seed):
    """A seeded random attention block: shapes, grouped heads, head dim and a mask
    drawn from offsets, non-causal, windows, segment ids and position arrays (alone
    and combined), as ring and packed shares produce them."""
    rng = np.random.default_rng(1000 + seed)
    D = int(rng.choice([32, 64, 128]))
    B = int(rng.choice([1, 2]))
    Hkv = int(rng.choice([1, 2, 4]))
    Hq = Hkv * int(rng.choice([1, 2, 3, 4]))
    Sq, Sk = int(rng.integers(1, 401)), int(rng.integers(1, 521))
    kind = ["offsets", "noncausal", "window", "segments", "positions", "positions_segments_window"][seed % 6]
    m = {}
    if kind in ("offsets", "window"):
        m.update(q_offset=int(rng.integers(0, 400)), k_offset=int(rng.integers(0, 400)))
    if kind == "noncausal":
        m.update(causal=False)
    if "window" in kind:
        m.update(window=int(rng.integers(1, 300)))
    if "positions" in kind:
        # strictly increasing global positions, as a zigzag or striped share holds them
        m.update(q_pos=np.sort(rng.choice(4 * max(Sq, Sk), Sq, replace=False)),
                 k_pos=np.sort(rng.choice(4 * max(Sq, Sk), Sk, replace=False)))
    if "segments" in kind:
        # non-decreasing document ids of each batch row, over a shared range of ids
        nd = int(rng.integers(1, 8))
        m.update(q_seg=torch.from_numpy(np.sort(rng.integers(0, nd, (B, Sq)), axis=1).astype(np.int32)),
                 k_seg=torch.from_numpy(np.sort(rng.integers(0, nd, (B, Sk)), axis=1).astype(np.int32)))
    return (B, Sq, Sk, Hq, Hkv, D), kind, m


# seeds of the random-block sweep (CP_RANDOM_BLOCKS widens it; 300 pass)
RANDOM_BLOCKS = int(os.environ.get("CP_RANDOM_BLOCKS", "48"))


@pytest.mark.parametrize("seed", range(RANDOM_BLOCKS))
def test_attn_random_blocks(cp, seed):
    """Seeded random blocks (bf16, matrix-core head dims): forward with and without a
    workspace, the fused ring step from a running result, and the backward, each
    against the oracle."""
    (B, Sq, Sk, Hq, Hkv, D), kind, m = _random_problem(seed)
    say(f"attn random seed={seed} B={B} Sq={Sq} Sk={Sk} Hq={Hq} Hkv={Hkv} D={D} {kind}")
    q, k, v, do = cp_inputs.normal_tensors([(B, Sq, Hq, D), (B, Sk, Hkv, D), (B, Sk, Hkv, D), (B, Sq, Hq, D)],
                                           seed=50 + seed, dtype=torch.bfloat16)
    dm = to_dev(m)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    out, lse = cp.attn_fwd(qd, kd, vd, **dm)
    out1, lse1 = cp.attn_fwd(qd, kd, vd, workspace=False, **dm)
    g = torch.Generator().manual_seed(seed)
    acc0 = torch.randn(B, Sq, Hq, D, generator=g)
    lse0 = torch.randn(B, Hq, Sq, generator=g) + 2
    lse0[..., ::7] = -float("inf")
    acc0[lse0.transpose(1, 2) == -float("inf")] = 0.0
    acc, lacc = acc0.cuda(), lse0.cuda()
    cp.attn_fwd_merge(qd, kd, vd, acc, lacc, **dm)
    dq, dk, dv = cp.attn_bwd(qd, kd, vd, out, lse, dod, **dm)
    om = oracle_mask(m)
    ref_o, ref_l = oracle.attn_fwd(q, k, v, **om)
    tol = TOL[torch.bfloat16]
    for o_, l_, nm in ((out, lse, "ws"), (out1, lse1, "no ws")):
        check_lse(l_, ref_l, tol["lse"])
        check_close(o_, ref_o, tol["out"], f"out ({nm})")
    mo, ml = oracle.lse_merge(f64(acc0), f64(lse0), ref_o, ref_l)
    check_lse(lacc, ml, tol["lse"])
    check_close(acc, mo, tol["out"], "merged out")
    refs = oracle.attn_bwd(q, k, v, ref_o, ref_l, do, **om)
    for got, ref, nm in zip((dq, dk, dv), refs, ("dq", "dk", "dv")):
        check_close(got, ref, tol["grad"] * max(1.0, np.abs(ref).max()), nm)


def _random_rows(rng, shape, dtype):
    if dtype in (torch.int32, torch.uint8):
        hi = 251 if dtype == torch.uint8 else 1 << 30
        return torch.from_numpy(rng.integers(0, hi, shape).astype(np.int64)).to(dtype)
    return torch.from_numpy(rng.standard_normal(shape)).to(dtype)


@pytest.mark.parametrize("seed", range(32))
def test_permutations_random(cp, seed):
    """Seeded random shapes for the data-movement kernels, bit for bit against the
    oracle: the grouped / replicated Ulysses relayout and its inverse, both reorder
    strategies and their inverses, and end padding / truncation.  Element sizes 1, 2
    and 4 bytes, odd row sizes, degrees 1-8."""
    rng = np.random.default_rng(2000 + seed)
    dtype = [torch.bfloat16, torch.float32, torch.int32, torch.uint8][seed % 4]
    say(f"permutations random seed={seed} {dtype}")
    # relayout (element sizes 2 and 4)
    if dtype != torch.uint8:
        G, P, B = int(rng.integers(1, 4)), int(rng.integers(1, 9)), int(rng.integers(1, 3))
        rep = int(rng.choice([1, 1, 2, 4]))
        H = P * int(rng.integers(1, 4))
        if rep > 1 and P % rep == 0 and rng.random() < 0.5:
            H = (P // rep) * int(rng.integers(1, 3))   # fewer heads than the degree
        D = int(rng.integers(1, 70))
        S = P * int(rng.integers(1, 40))
        x = _random_rows(rng, (G, P, B, S // P, H, D), dtype).cuda()
        y = cp.ulysses_relayout_ex(x, P, groups=G, rep=rep)
        ref = np.stack([oracle.ulysses_relayout_rep(bits(x[g]), rep) for g in range(G)])
        np.testing.assert_array_equal(bits(y), ref)
        if rep == 1:
            z = cp.ulysses_relayout_ex(y, P, groups=G, inverse=True)
            np.testing.assert_array_equal(bits(z), oracle.usp_relayout_inv(bits(y)))
            assert torch.equal(z, x)
    # reorders
    P = int(rng.integers(1, 9))
    B = int(rng.integers(1, 4))
    tail = tuple(int(t) for t in rng.integers(1, 12, int(rng.integers(0, 3))))
    for strategy, unit in ((0, 2 * P), (1, P)):
        S = unit * int(rng.integers(1, 30))
        x = _random_rows(rng, (B, S) + tail, dtype).cuda()
        fwd, inv = ((oracle.reorder, oracle.reorder_inv) if strategy == 0
                    else (oracle.reorder_striped, oracle.reorder_striped_inv))
        y = cp.zigzag_reorder(x, P, strategy=strategy)
        np.testing.assert_array_equal(bits(y), fwd(bits(x), P))
        z = cp.zigzag_reorder(y, P, inverse=True, strategy=strategy)
        np.testing.assert_array_equal(bits(z), inv(bits(y), P))
    # padding and truncation
    S = int(rng.integers(1, 300))
    S_out = max(1, S + int(rng.integers(-S // 2, 40)))
    x = _random_rows(rng, (B, S) + tail, dtype)
    row_bytes = int(np.prod(tail, dtype=np.int64)) * x.element_size()
    fill = int(rng.integers(1, 1000)) if dtype == torch.int32 and row_bytes % 4 == 0 and seed % 2 else 0
    y = cp.pad_rows(x.cuda(), S_out, fill=fill)
    np.testing.assert_array_equal(bits(y), oracle.pad_rows(bits(x), S_out, fill=fill))


@pytest.mark.parametrize("seed", range(12))
def test_ulysses_random(cp, seed):
    """Seeded random Ulysses passes through the driver: degree 1-8 (kv heads
    replicated where the degree exceeds them), grouped heads, D 64 or 128, causal or
    not, windows and packed documents; out, lse, dq, dk, dv against the oracle's
    attention over the whole sequence."""
    rng = np.random.default_rng(4000 + seed)
    P = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4]))
    while (Hkv * G) % P:
        G *= 2
    Hq = Hkv * G
    rep = P // math.gcd(P, Hkv)
    D = int(rng.choice([64, 128]))
    S = P * int(rng.integers(4, 80))
    m = {}
    kind = seed % 4
    if kind == 1:
        m["causal"] = False
    elif kind == 2:
        m["window"] = int(rng.integers(1, S))
    elif kind == 3:
        seg = cp_inputs.random_segment_ids(S, 1, max(2, S // 2), seed=seed)
        m.update(q_seg=seg, k_seg=seg)
    say(f"ulysses random seed={seed} P={P} Hq={Hq} Hkv={Hkv} rep={rep} D={D} S={S} {sorted(m)}")
    q, k, v, do = cp_inputs.normal_tensors([(1, S, Hq, D), (1, S, Hkv, D), (1, S, Hkv, D), (1, S, Hq, D)],
                                           seed=90 + seed)
    st = lambda t: t.reshape(P, 1, S // P, t.shape[2], D).cuda()
    dm = to_dev(m)
    out, lse, rel = cp.drivers.ulysses_forward(st(q), st(k), st(v), P, kv_rep=rep, **dm)
    om = oracle_mask(m)
    ro, rl = oracle.attn_fwd(q, k, v, **om)
    check_close(out.reshape(1, S, Hq, D), ro, 1e-2, "out")
    check_lse(torch.cat(list(lse), dim=1), rl, 1e-3)
    dq, dk, dv = cp.drivers.ulysses_backward(rel, lse, st(do), P, kv_rep=rep, **dm)
    refs = oracle.attn_bwd(q, k, v, ro, rl, do, **om)
    for got, ref, nm in zip((dq, dk, dv), refs, ("dq", "dk", "dv")):
        check_close(got.reshape(ref.shape), ref, 1e-2 * max(1.0, np.abs(ref).max()), nm)


@pytest.mark.parametrize("seed", range(8))
def test_usp_random(cp, seed):
    """Seeded random Ulysses x ring (USP) passes: Pr ring groups of Pu Ulysses ranks
    (kv heads replicated where Pu exceeds them), grouped heads, causal, windows and
    packed documents; out, dq, dk, dv against the oracle's full attention."""
    rng = np.random.default_rng(5000 + seed)
    Pr, Pu = int(rng.choice([2, 3, 4])), int(rng.choice([1, 2, 4]))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4]))
    while (Hkv * G) % Pu:
        G *= 2
    Hq = Hkv * G
    rep = Pu // math.gcd(Pu, Hkv)
    D = int(rng.choice([64, 128]))
    S = 2 * Pr * Pu * int(rng.integers(4, 40))
    seg = cp_inputs.random_segment_ids(S, 1, max(2, S // 3), seed=seed) if seed % 2 else None
    window = int(rng.integers(1, S)) if seed % 4 >= 2 else 0
    say(f"usp random seed={seed} Pr={Pr} Pu={Pu} Hq={Hq} Hkv={Hkv} rep={rep} D={D} S={S} "
        f"seg={seg is not None} window={window}")
    q, k, v, do = cp_inputs.normal_tensors([(1, S, Hq, D), (1, S, Hkv, D), (1, S, Hkv, D), (1, S, Hq, D)],
                                           seed=110 + seed)
    out, lse, state = cp.drivers.usp_forward(q.cuda(), k.cuda(), v.cuda(), Pr, Pu, kv_rep=rep,
                                             seg=None if seg is None else seg.cuda(), window=window, keep=True)
    dq, dk, dv = cp.drivers.usp_backward(state, lse, do.cuda())
    sm = {} if seg is None else dict(q_seg=seg.numpy(), k_seg=seg.numpy())
    ro, rl = oracle.attn_fwd(q, k, v, window=window, **sm)
    check_close(out, ro, 1e-2, "usp out")
    refs = oracle.attn_bwd(q, k, v, ro, rl, do, window=window, **sm)
    for got, ref, nm in zip((dq, dk, dv), refs, ("dq", "dk", "dv")):
        check_close(got, ref, 1e-2 * max(1.0, np.abs(ref).max()), f"usp {nm}")


@pytest.mark.parametrize("seed", range(16))
def test_attn_random_blocks_rowwise(cp, seed):
    """The random blocks of test_attn_random_blocks on the row-per-wavefront kernels:
    float32 (any D up to 128) and bf16 head dims without a matrix-core kernel; forward,
    fused ring step and backward against the oracle at their own bars."""
    (B, Sq, Sk, Hq, Hkv, _), kind, m = _random_problem(seed)
    rng = np.random.default_rng(6000 + seed)
    dtype = torch.float32 if seed % 2 == 0 else torch.bfloat16
    D = int(rng.integers(1, 129)) if dtype == torch.float32 else int(rng.choice([8, 16, 24, 48, 80, 96, 112]))
    Sq, Sk = min(Sq, 160), min(Sk, 200)    # one wavefront per row: kept small
    if "q_pos" in m:
        m["q_pos"], m["k_pos"] = m["q_pos"][:Sq], m["k_pos"][:Sk]
    if "q_seg" in m:
        m["q_seg"], m["k_seg"] = m["q_seg"][:, :Sq].contiguous(), m["k_seg"][:, :Sk].contiguous()
    say(f"attn random rowwise seed={seed} B={B} Sq={Sq} Sk={Sk} Hq={Hq} Hkv={Hkv} D={D} {dtype} {kind}")
    q, k, v, do = cp_inputs.normal_tensors([(B, Sq, Hq, D), (B, Sk, Hkv, D), (B, Sk, Hkv, D), (B, Sq, Hq, D)],
                                           seed=150 + seed, dtype=dtype)
    dm = to_dev(m)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    out, lse = cp.attn_fwd(qd, kd, vd, **dm)
    g = torch.Generator().manual_seed(seed)
    acc0 = torch.randn(B, Sq, Hq, D, generator=g)
    lse0 = torch.randn(B, Hq, Sq, generator=g) + 2
    acc, lacc = acc0.cuda(), lse0.cuda()
    cp.attn_fwd_merge(qd, kd, vd, acc, lacc, **dm)
    dq, dk, dv = cp.attn_bwd(qd, kd, vd, out, lse, dod, **dm)
    om = oracle_mask(m)
    ref_o, ref_l = oracle.attn_fwd(q, k, v, **om)
    tol = TOL[dtype]
    check_lse(lse, ref_l, tol["lse"])
    check_close(out, ref_o, tol["out"], "out")
    mo, ml = oracle.lse_merge(f64(acc0), f64(lse0), ref_o, ref_l)
    check_lse(lacc, ml, tol["lse"])
    check_close(acc, mo, tol["out"], "merged out")
    # the backward's rows are the GPU forward's (bf16 out rounded): the oracle takes
    # its own exact forward, within the gradient bar
    refs = oracle.attn_bwd(q, k, v, ref_o, ref_l, do, **om)
    for got, ref, nm in zip((dq, dk, dv), refs, ("dq", "dk", "dv")):
        check_close(got, ref, tol["grad"] * max(1.0, np.abs(ref).max()), nm)
