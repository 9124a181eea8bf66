"""Parity of the five workloads, end to end through the drivers (GPU only).

Toy: every output element against the oracle.  Full-size workloads run in the
launch configuration bench.py times; outputs the oracle can compute one by one
(sampled query rows, the keys at the end of the sequence) are compared element
by element, the rest through exact properties that hold at any size.
"""

import numpy as np
import pytest
import torch

import cp_inputs
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cp():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import context_cp_attn_amd as cp
    cp.load_library()
    return cp


def say(*a):
    print(*a, flush=True)


def bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.numpy()


def bf16_bits_to_f64(b):
    return (b.astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64(t):
    return t.detach().cpu().double().numpy()


def max_err(a, b):
    return float(np.abs(a - b).max())


def check_rows(out, lse, ref_o, ref_l, tol_o, tol_l):
    assert np.array_equal(np.isneginf(lse), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    assert max_err(lse[fin], ref_l[fin]) <= tol_l
    assert max_err(out, ref_o) <= tol_o


def grad_tol(ref):
    return 1e-2 * max(1.0, float(np.abs(ref).max()))


def causal_band_grads(qs, ks, vs, gs, j0, j1):
    """Oracle dK, dV of keys [j0, j1) of a causal problem: only the rows at or after
    j0 see them, each through its full-row (out, lse), so the oracle runs those rows'
    forward against every key and their backward against the band's keys (the
    blockwise form of the gradient, the oracle's ring backward)."""
    rows = np.arange(j0, qs.shape[1])
    ro, rl = oracle.attn_fwd(qs[:, rows], ks, vs, q_pos=rows)
    _, bk, bv = oracle.attn_bwd(qs[:, rows], ks[:, j0:j1], vs[:, j0:j1], ro, rl, gs[:, rows], q_pos=rows,
                                k_offset=j0)
    return bk, bv


# ------------------------------------------------------------------ toy (fp32)

def test_toy_full_ring_ulysses_reorder(cp):
    say("toy: full attention, ring (contiguous, zigzag), Ulysses, reorder")
    q, k, v = cp_inputs.toy_qkv()
    P, S = 4, 32
    ref_o, ref_l = oracle.attn_fwd(q, k, v)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o, l = cp.attn_fwd(qd, kd, vd)
    check_rows(f64(o), f64(l), ref_o, ref_l, 1e-5, 1e-5)
    # ring, both partitions
    for layout in ("contiguous", "zigzag", "striped"):
        st = {"zigzag": 0, "striped": 1}.get(layout)
        src = [cp.zigzag_reorder(t, P, strategy=st) for t in (qd, kd, vd)] if st is not None else [qd, kd, vd]
        for r in range(P):
            acc, lse = cp.drivers.RingShare(*src, P, r, layout).forward()
            pos = oracle.rank_positions(r, P, S, layout)
            check_rows(f64(acc), f64(lse), ref_o[:, pos], ref_l[:, :, pos], 1e-5, 1e-5)
    # Ulysses: 2 heads per rank
    stack = [t.reshape(P, 1, S // P, 8, 16).cuda() for t in (q, k, v)]
    out_stack, lses, (ql, kl, vl, _) = cp.drivers.ulysses_forward(*stack, P)
    np.testing.assert_array_equal(bits(ql), oracle.ulysses_relayout(bits(stack[0])))
    assert tuple(ql.shape[2:]) == (32, 2, 16)
    assert max_err(f64(out_stack).reshape(1, S, 8, 16), ref_o) <= 1e-5
    assert max_err(np.concatenate([f64(x) for x in lses], axis=1), ref_l) <= 1e-5
    # reorder into 2P = 8 chunks
    y = cp.zigzag_reorder(qd, P)
    np.testing.assert_array_equal(bits(y), oracle.reorder(bits(q), P))


@pytest.mark.parametrize("layout", ["contiguous", "zigzag", "striped"])
def test_toy_ring_backward(cp, layout):
    say(f"toy ring backward {layout}")
    q, k, v = cp_inputs.toy_qkv()
    (do,) = cp_inputs.normal_tensors([(1, 32, 8, 16)], seed=9, scale=1.0, dtype=torch.float32)
    P, S = 4, 32
    ref_o, ref_l = oracle.attn_fwd(q, k, v)
    rq, rk, rv = oracle.attn_bwd(q, k, v, ref_o, ref_l, do)
    dev = [t.cuda() for t in (q, k, v, do)]
    st = {"zigzag": 0, "striped": 1}.get(layout)
    if st is not None:
        dev = [cp.zigzag_reorder(t, P, strategy=st) for t in dev]
    qd, kd, vd, dd = dev
    dk, dv = torch.zeros_like(kd), torch.zeros_like(vd)
    dq = torch.zeros_like(qd)
    C = S // P
    for r in range(P):
        sh = cp.drivers.RingShare(qd, kd, vd, P, r, layout)
        o, l = sh.forward()
        sh.backward(o, l, dd[:, r * C:(r + 1) * C], dq[:, r * C:(r + 1) * C], dk, dv)
    if st is not None:
        dq, dk, dv = (cp.zigzag_reorder(t, P, inverse=True, strategy=st) for t in (dq, dk, dv))
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        assert max_err(f64(got), ref) <= 1e-5 * max(1.0, np.abs(ref).max())


# ------------------------------------------------------------------ Ulysses llama2-7b, 32K, cp=16

@pytest.mark.timeout(600)
def test_ulysses_llama2_7b_32k(cp):
    P, S, H, D = 16, 32768, 32, 128
    say("ulysses llama2-7b: inputs")
    q, k, v, do = cp_inputs.normal_tensors([(1, S, H, D)] * 4, seed=0)
    stack = [t.reshape(P, 1, S // P, H, D) for t in (q, k, v, do)]
    dev = [t.cuda() for t in stack]
    say("ulysses llama2-7b: relayout bit-exact")
    ql = cp.ulysses_relayout(dev[0], P)
    ref_ql = oracle.ulysses_relayout(bits(stack[0]))
    np.testing.assert_array_equal(bits(ql), ref_ql)
    back = cp.ulysses_relayout_inv(ql, P)
    assert torch.equal(back, dev[0])
    kl, vl, gl = (cp.ulysses_relayout(t, P) for t in dev[1:])
    # rank 0's share in the launch shape the benchmark uses
    o, l = cp.attn_fwd(ql[0], kl[0], vl[0])
    dq, dk, dv = cp.attn_bwd(ql[0], kl[0], vl[0], o, l, gl[0])
    torch.cuda.synchronize()
    say("ulysses llama2-7b: oracle on sampled rows")
    # the oracle's own rank-0 share (relayout of the input bits)
    share = [bf16_bits_to_f64(oracle.ulysses_relayout(bits(t))[0]) for t in stack[1:3]]
    qs = bf16_bits_to_f64(ref_ql[0])
    gs = bf16_bits_to_f64(oracle.ulysses_relayout(bits(stack[3]))[0])
    ks, vs = share
    rows = np.unique(np.r_[0, 1, 127, 128, 129, 4095, 4096, 20000, S - 129, S - 128, np.arange(S - 64, S)])
    ro, rl = oracle.attn_fwd(qs[:, rows], ks, vs, q_pos=rows)
    check_rows(f64(o)[:, rows], f64(l)[:, :, rows], ro, rl, 1e-2, 1e-3)
    rq, _, _ = oracle.attn_bwd(qs[:, rows], ks, vs, ro, rl, gs[:, rows], q_pos=rows)
    assert max_err(f64(dq)[:, rows], rq) <= 1e-2 * max(1.0, np.abs(rq).max())
    # keys at the end are seen only by the last queries: exact dk/dv there
    tail = np.arange(S - 256, S)
    to, tl = oracle.attn_fwd(qs[:, tail], ks, vs, q_pos=tail)
    _, tk, tv = oracle.attn_bwd(qs[:, tail], ks, vs, to, tl, gs[:, tail], q_pos=tail)
    assert max_err(f64(dk)[:, tail], tk[:, tail]) <= 1e-2 * max(1.0, np.abs(tk[:, tail]).max())
    assert max_err(f64(dv)[:, tail], tv[:, tail]) <= 1e-2 * max(1.0, np.abs(tv[:, tail]).max())
    # an interior band of keys, seen by the second half of the rows
    say("ulysses llama2-7b: dk/dv of keys [16384, 16512)")
    bk, bv = causal_band_grads(qs, ks, vs, gs, 16384, 16512)
    assert max_err(f64(dk)[:, 16384:16512], bk) <= grad_tol(bk)
    assert max_err(f64(dv)[:, 16384:16512], bv) <= grad_tol(bv)
    # every row's P sums to one: sum_j dV_j = sum_i dO_i
    sdv = f64(dv).sum(axis=1)
    sdo = gs.sum(axis=1)
    assert max_err(sdv, sdo) <= 1e-2 * max(1.0, np.abs(sdo).max())


@pytest.mark.timeout(600)
def test_ulysses_step_all_ranks(cp):
    """The benchmark's timed step (drivers.UlyssesStep: q, k, v relayouted together,
    buffers reused): all 16 ranks' outputs and gradients after the inverse relayouts,
    in the global sequence layout,
    on sampled query rows (out, lse, dq, all 32 heads) and on the last 256 keys (dk,
    dv, all heads), and sum_j dV_j = sum_i dO_i on every head."""
    P, S, H, D = 16, 32768, 32, 128
    say("ulysses step: inputs")
    q, k, v, do = cp_inputs.normal_tensors([(1, S, H, D)] * 4, seed=0)
    qkv = torch.stack([t.reshape(P, 1, S // P, H, D) for t in (q, k, v)]).cuda()
    step = cp.drivers.UlyssesStep(qkv, do.reshape(P, 1, S // P, H, D).cuda(), P)
    step.run()
    step.run()   # the second pass reuses every buffer of the first
    torch.cuda.synchronize()
    # the grouped relayout of q, k, v is the three single ones, bit for bit
    np.testing.assert_array_equal(bits(step.qkvl[1]), oracle.ulysses_relayout(bits(k.reshape(P, 1, S // P, H, D))))
    out = f64(step.out).reshape(1, S, H, D)
    dq, dk, dv = (f64(t).reshape(1, S, H, D) for t in step.dqkv)
    lse = f64(step.lse)   # [P][1][H/P][S]: rank p holds heads [2p, 2p + 2)
    lse = lse.transpose(1, 0, 2, 3).reshape(1, H, S)
    qf, kf, vf, gf = (f64(t) for t in (q, k, v, do))
    say("ulysses step: oracle on sampled rows, all heads")
    rows = np.unique(np.r_[0, 1, 2047, 2048, 2049, 9000, 16383, 16384, 30000, np.arange(S - 8, S)])
    ro, rl = oracle.attn_fwd(qf[:, rows], kf, vf, q_pos=rows)
    check_rows(out[:, rows], lse[:, :, rows], ro, rl, 1e-2, 1e-3)
    rq, _, _ = oracle.attn_bwd(qf[:, rows], kf, vf, ro, rl, gf[:, rows], q_pos=rows)
    assert max_err(dq[:, rows], rq) <= grad_tol(rq)
    say("ulysses step: dk/dv of the last 256 keys, all heads")
    tail = np.arange(S - 256, S)
    to, tl = oracle.attn_fwd(qf[:, tail], kf, vf, q_pos=tail)
    _, tk, tv = oracle.attn_bwd(qf[:, tail], kf[:, tail], vf[:, tail], to, tl, gf[:, tail], q_pos=tail,
                                k_offset=S - 256)
    assert max_err(dk[:, tail], tk) <= grad_tol(tk)
    assert max_err(dv[:, tail], tv) <= grad_tol(tv)
    sdo = gf.sum(axis=1)
    assert max_err(dv.sum(axis=1), sdo) <= grad_tol(sdo)


# ------------------------------------------------------------------ ring llama2-7b, 32K, cp=16

def test_ring_llama2_7b_32k_zigzag(cp):
    P, S, H, D = 16, 32768, 32, 128
    say("ring llama2-7b: inputs + zigzag reorder")
    q, k, v = cp_inputs.normal_tensors([(1, S, H, D)] * 3, seed=0)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    qz = cp.zigzag_reorder(qd, P)
    np.testing.assert_array_equal(bits(qz), oracle.reorder(bits(q), P))
    kz, vz = cp.zigzag_reorder(kd, P), cp.zigzag_reorder(vd, P)
    qf, kf, vf = (f64(t) for t in (q, k, v))
    for r in (0, 7, 15):
        say(f"ring llama2-7b: rank {r}")
        acc, lse = cp.drivers.RingShare(qz, kz, vz, P, r).forward()
        pos = oracle.rank_positions(r, P, S, "zigzag")
        pick = np.r_[0, 1, 511, 1023, 1024, 1025, 1500, 2047]
        ro, rl = oracle.attn_fwd(qf[:, pos[pick]], kf, vf, q_pos=pos[pick])
        check_rows(f64(acc)[:, pick], f64(lse)[:, :, pick], ro, rl, 1e-2, 1e-3)


def test_ring_and_usp_long_blocks(cp):
    """Blocks of 8192 keys on a small grid: the drivers run attn_fwd with its
    two-workgroup key split + lse_merge instead of the fused step (their default
    choice there).  Ring ranks (automatic and forced fused) and a Ulysses-2 x ring-2
    forward, sampled rows against the oracle's full attention, bf16, 16K tokens."""
    S, Hq, Hkv, D = 16384, 4, 2, 128
    q, k, v = cp_inputs.normal_tensors([(1, S, Hq, D), (1, S, Hkv, D), (1, S, Hkv, D)], seed=5)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    qf, kf, vf = (f64(t) for t in (q, k, v))
    P = 2
    qz, kz, vz = (cp.zigzag_reorder(t, P) for t in (qd, kd, vd))
    assert cp.drivers.split_workspace(qz[:, :S // P], kz[:, :S // P]) is not False
    pick = np.r_[0, 1, 4095, 4096, 6000, 8191]
    for r in range(P):
        pos = oracle.rank_positions(r, P, S, "zigzag")
        ro, rl = oracle.attn_fwd(qf[:, pos[pick]], kf, vf, q_pos=pos[pick])
        for fused in (None, True):
            say(f"ring long blocks: rank {r} fused={fused}")
            acc, lse = cp.drivers.RingShare(qz, kz, vz, P, r, fused=fused).forward()
            check_rows(f64(acc)[:, pick], f64(lse)[:, :, pick], ro, rl, 1e-2, 1e-3)
    say("usp long blocks: Ulysses 2 x ring 2")
    out, _ = cp.drivers.usp_forward(qd, kd, vd, 2, 2)
    rows = np.r_[0, 2047, 4096, 8191, 12000, 16383]
    ro, rl = oracle.attn_fwd(qf[:, rows], kf, vf, q_pos=rows)
    assert max_err(f64(out)[:, rows], ro) <= 1e-2


# ------------------------------------------------------------------ Ulysses llama3.1-8b GQA, 64K, cp=4

@pytest.mark.timeout(600)
def test_ulysses_llama31_8b_64k_gqa(cp):
    P, S, Hq, Hkv, D = 4, 65536, 32, 8, 128
    say("ulysses llama3.1-8b: inputs")
    q, k, v, do = cp_inputs.normal_tensors([(1, S, Hq, D), (1, S, Hkv, D), (1, S, Hkv, D), (1, S, Hq, D)], seed=0)
    say("ulysses llama3.1-8b: relayout")
    ql = cp.ulysses_relayout(q.reshape(P, 1, S // P, Hq, D).cuda(), P)[0]   # 8 q heads
    kl = cp.ulysses_relayout(k.reshape(P, 1, S // P, Hkv, D).cuda(), P)[0]  # 2 kv heads
    vl = cp.ulysses_relayout(v.reshape(P, 1, S // P, Hkv, D).cuda(), P)[0]
    gl = cp.ulysses_relayout(do.reshape(P, 1, S // P, Hq, D).cuda(), P)[0]
    assert ql.shape == (1, S, 8, D) and kl.shape == (1, S, 2, D)
    o, l = cp.attn_fwd(ql, kl, vl)
    dq, dk, dv = cp.attn_bwd(ql, kl, vl, o, l, gl)
    torch.cuda.synchronize()
    say("ulysses llama3.1-8b: oracle on sampled rows")
    qs, gs = f64(q[:, :, 0:8]), f64(do[:, :, 0:8])      # rank 0 = heads [0, 8) and kv heads [0, 2)
    ks, vs = f64(k[:, :, 0:2]), f64(v[:, :, 0:2])
    np.testing.assert_array_equal(bits(ql), bits(q[:, :, 0:8].contiguous()))
    rows = np.r_[0, 63, 64, 65, 32767, 40000, np.arange(S - 32, S)]
    ro, rl = oracle.attn_fwd(qs[:, rows], ks, vs, q_pos=rows)
    check_rows(f64(o)[:, rows], f64(l)[:, :, rows], ro, rl, 1e-2, 1e-3)
    rq, _, _ = oracle.attn_bwd(qs[:, rows], ks, vs, ro, rl, gs[:, rows], q_pos=rows)
    assert max_err(f64(dq)[:, rows], rq) <= 1e-2 * max(1.0, np.abs(rq).max())
    tail = np.arange(S - 128, S)
    to, tl = oracle.attn_fwd(qs[:, tail], ks, vs, q_pos=tail)
    _, tk, tv = oracle.attn_bwd(qs[:, tail], ks, vs, to, tl, gs[:, tail], q_pos=tail)
    assert max_err(f64(dk)[:, tail], tk[:, tail]) <= 1e-2 * max(1.0, np.abs(tk[:, tail]).max())
    assert max_err(f64(dv)[:, tail], tv[:, tail]) <= 1e-2 * max(1.0, np.abs(tv[:, tail]).max())
    # group sums: sum_j dV[j, g] = sum over the group's 4 heads of sum_i dO
    sdo = gs.reshape(1, S, 2, 4, D).sum(axis=(1, 3))
    assert max_err(f64(dv).sum(axis=1), sdo) <= 1e-2 * max(1.0, np.abs(sdo).max())
    # an interior band of keys of kv head 0 (its group: query heads 0-3)
    say("ulysses llama3.1-8b: dk/dv of keys [57344, 57472), kv head 0")
    bk, bv = causal_band_grads(qs[:, :, 0:4], ks[:, :, 0:1], vs[:, :, 0:1], gs[:, :, 0:4], 57344, 57472)
    assert max_err(f64(dk)[:, 57344:57472, 0:1], bk) <= grad_tol(bk)
    assert max_err(f64(dv)[:, 57344:57472, 0:1], bv) <= grad_tol(bv)
    say("ulysses llama3.1-8b: dual-chunk-swap reorder of 64K tokens")
    ids = torch.arange(S, dtype=torch.int32)[None].cuda()
    z = cp.zigzag_reorder(ids, P)
    np.testing.assert_array_equal(bits(z), oracle.reorder(bits(ids), P))
    x = torch.randn(1, S, 4096).bfloat16().cuda()
    y = cp.zigzag_reorder(x, P)
    np.testing.assert_array_equal(bits(y), oracle.reorder(bits(x), P))   # all 512 MiB
    assert torch.equal(cp.zigzag_reorder(y, P, inverse=True), x)


# ------------------------------------------------------------------ packed + windowed ring, 8K, cp=4

def _packed_ring(cp, S, Hq, Hkv, D, P, W, lens, strategy=0):
    q, k, v, do = cp_inputs.normal_tensors([(1, S, Hq, D), (1, S, Hkv, D), (1, S, Hkv, D), (1, S, Hq, D)], seed=0)
    seg = cp_inputs.segment_ids(lens)
    layout = cp.drivers.LAYOUT_OF_STRATEGY[strategy]
    dev = [cp.zigzag_reorder(t.cuda(), P, strategy=strategy) for t in (q, k, v, do, seg)]
    qz, kz, vz, dz, sz = dev
    C = S // P
    outs, lses = [], []
    dq = torch.zeros(qz.shape, device="cuda")
    dk, dv = torch.zeros(kz.shape, device="cuda"), torch.zeros(vz.shape, device="cuda")
    for r in range(P):
        sh = cp.drivers.RingShare(qz, kz, vz, P, r, layout=layout, seg=sz, window=W)
        o, l = sh.forward()
        outs.append(o)
        lses.append(l)
        sh.backward(o.bfloat16(), l, dz[:, r * C:(r + 1) * C], dq[:, r * C:(r + 1) * C], dk, dv)
    grads = [cp.zigzag_reorder(t, P, inverse=True, strategy=strategy) for t in (dq, dk, dv)]
    return (q, k, v, do, seg), outs, lses, grads


@pytest.mark.parametrize("strategy", ["dual_chunk_swap", "auto"])
def test_packed_window_small_all_elements(cp, strategy):
    S, Hq, Hkv, D, P, W = 2048, 4, 2, 128, 4, 512
    lens = cp_inputs.doc_lengths(S, 64, 1024, seed=1)
    st = cp.drivers.auto_strategy(packed=True) if strategy == "auto" else 0
    layout = cp.drivers.LAYOUT_OF_STRATEGY[st]
    say(f"packed+window small ({strategy} -> {layout}): docs {lens}")
    (q, k, v, do, seg), outs, lses, grads = _packed_ring(cp, S, Hq, Hkv, D, P, W, lens, strategy=st)
    m = dict(q_seg=seg, k_seg=seg, window=W)
    ro, rl = oracle.attn_fwd(q, k, v, **m)
    for r in range(P):
        pos = oracle.rank_positions(r, P, S, layout)
        check_rows(f64(outs[r]), f64(lses[r]), ro[:, pos], rl[:, :, pos], 1e-2, 1e-3)
    refs = oracle.attn_bwd(q, k, v, ro, rl, do, **m)
    for got, ref in zip(grads, refs):
        assert max_err(f64(got), ref) <= 1e-2 * max(1.0, np.abs(ref).max())


@pytest.mark.timeout(600)
def test_packed_window_8k(cp):
    """The packed + windowed workload at its full size, all 4 ranks: every output row
    and every element of dq, dk and dv against the oracle.  Documents never see each
    other, so the oracle runs per document (the oracle's packed = per-document
    property)."""
    S, Hq, Hkv, D, P, W = 8192, 32, 8, 128, 4, 4096
    lens = cp_inputs.doc_lengths(S)
    say(f"packed+window 8K: docs {lens}")
    (q, k, v, do, seg), outs, lses, grads = _packed_ring(cp, S, Hq, Hkv, D, P, W, lens)
    qf, kf, vf, gf = (f64(t) for t in (q, k, v, do))
    ro, rl = np.zeros(qf.shape), np.full((1, Hq, S), -np.inf)
    rdq, rdk, rdv = np.zeros(qf.shape), np.zeros(kf.shape), np.zeros(vf.shape)
    s0 = 0
    for n in lens:
        d = slice(s0, s0 + n)
        o, l = oracle.attn_fwd(qf[:, d], kf[:, d], vf[:, d], q_offset=s0, k_offset=s0, window=W)
        ro[:, d], rl[:, :, d] = o, l
        rdq[:, d], rdk[:, d], rdv[:, d] = oracle.attn_bwd(qf[:, d], kf[:, d], vf[:, d], o, l, gf[:, d],
                                                           q_offset=s0, k_offset=s0, window=W)
        s0 += n
    say("packed+window 8K: oracle done")
    for r in range(P):
        pos = oracle.rank_positions(r, P, S, "zigzag")
        check_rows(f64(outs[r]), f64(lses[r]), ro[:, pos], rl[:, :, pos], 1e-2, 1e-3)
    for got, ref in zip(grads, (rdq, rdk, rdv)):
        assert max_err(f64(got), ref) <= grad_tol(ref)


# ------------------------------------------------------------------ the step's kernels, every element

@pytest.mark.timeout(600)
def test_dense_causal_multiblock_all_elements(cp):
    """The kernel instances of the Ulysses step (one query head per kv head, causal,
    no window or segment ids; the forward's two-workgroup key split) on a smaller
    sequence: 8192 tokens = 32 key blocks of the backward, 64 query tiles of the
    forward per head; out, lse, dq, dk, dv compared on every element."""
    S, H, D = 8192, 2, 128
    q, k, v, do = cp_inputs.normal_tensors([(1, S, H, D)] * 4, seed=11)
    qd, kd, vd, gd = (t.cuda() for t in (q, k, v, do))
    assert cp.fwd_workspace(qd, kd) is not None    # the split forward runs here
    o, l = cp.attn_fwd(qd, kd, vd)
    dq, dk, dv = cp.attn_bwd(qd, kd, vd, o, l, gd)
    torch.cuda.synchronize()
    say("dense 8K: oracle")
    ro, rl = oracle.attn_fwd(q, k, v)
    check_rows(f64(o), f64(l), ro, rl, 1e-2, 1e-3)
    refs = oracle.attn_bwd(q, k, v, ro, rl, do)
    for got, ref in zip((dq, dk, dv), refs):
        assert max_err(f64(got), ref) <= grad_tol(ref)


# ------------------------------------------------------------------ ring pass as a HIP graph

@pytest.mark.parametrize("fused", [True, False])
def test_ring_forward_graph_replays(cp, fused):
    """A rank's ring forward captured as one HIP graph: every replay, with eager
    passes and synchronisations between the replays, equals the eager pass bit for
    bit, and the result matches the oracle on sampled rows."""
    P, S, H, D, r = 8, 4096, 4, 128, 3
    say(f"ring graph: P={P} S={S} H={H} rank {r} fused={fused}")
    q, k, v = cp_inputs.normal_tensors([(1, S, H, D)] * 3, seed=11)
    qz, kz, vz = (cp.zigzag_reorder(t.cuda(), P) for t in (q, k, v))
    ring = cp.drivers.RingShare(qz, kz, vz, P, r, fused=fused)
    ref_o, ref_l = (t.clone() for t in ring.forward())
    replay, go, gl = ring.forward_graph()
    for rep in range(4):
        go.fill_(float("nan"))
        replay()
        torch.cuda.synchronize()
        assert torch.equal(go, ref_o) and torch.equal(gl, ref_l), f"replay {rep}"
        eo, el = ring.forward()
        torch.cuda.synchronize()
        assert torch.equal(eo, ref_o) and torch.equal(el, ref_l), f"eager pass after replay {rep}"
    pos = oracle.rank_positions(r, P, S, "zigzag")
    pick = np.r_[0, 1, 255, 256, 300, 511]
    qf, kf, vf = (f64(t) for t in (q, k, v))
    ro, rl = oracle.attn_fwd(qf[:, pos[pick]], kf, vf, q_pos=pos[pick])
    check_rows(f64(go)[:, pick], f64(gl)[:, :, pick], ro, rl, 1e-2, 1e-3)


# ------------------------------------------------------------------ random ring shares

@pytest.mark.parametrize("seed", range(16))
def test_ring_random_shares(cp, seed):
    """Seeded random ring passes through the driver: degree 2-4, contiguous / zigzag /
    striped partition, grouped heads, D 64 or 128, packed documents and a window
    (alone or together), the fused or the unfused step; every rank's out and lse, and
    dq, dk, dv of the whole sequence after all ranks' backward passes, against the
    oracle's attention over the whole sequence."""
    rng = np.random.default_rng(3000 + seed)
    P = int(rng.integers(2, 5))
    S = 2 * P * int(rng.integers(8, 97))
    Hkv = int(rng.choice([1, 2]))
    Hq = Hkv * int(rng.choice([1, 2, 4]))
    D = int(rng.choice([64, 128]))
    layout = ["zigzag", "striped", "contiguous"][seed % 3]
    use_seg, window = bool(rng.integers(0, 2)), int(rng.choice([0, 0, int(rng.integers(1, S))]))
    fused = [None, True, False][(seed // 3) % 3]
    say(f"ring random seed={seed} P={P} S={S} Hq={Hq} Hkv={Hkv} D={D} {layout} seg={use_seg} "
        f"window={window} fused={fused}")
    q, k, v, do = cp_inputs.normal_tensors([(1, S, Hq, D), (1, S, Hkv, D), (1, S, Hkv, D), (1, S, Hq, D)],
                                           seed=70 + seed)
    seg = cp_inputs.random_segment_ids(S, 1, max(2, S // 3), seed=seed) if use_seg else None
    mask = dict(window=window)
    if seg is not None:
        mask.update(q_seg=seg.numpy(), k_seg=seg.numpy())
    ro, rl = oracle.attn_fwd(q, k, v, **mask)
    rq, rk, rv = oracle.attn_bwd(q, k, v, ro, rl, do, **mask)
    st = {"zigzag": 0, "striped": 1}.get(layout)
    dev = [t.cuda() for t in (q, k, v, do)] + ([seg.cuda()] if seg is not None else [])
    if st is not None:
        dev = [cp.zigzag_reorder(t, P, strategy=st) for t in dev]
    qd, kd, vd, dd = dev[:4]
    sd = dev[4] if seg is not None else None
    C = S // P
    dk, dv = torch.zeros(kd.shape, device="cuda"), torch.zeros(vd.shape, device="cuda")
    for r in range(P):
        sh = cp.drivers.RingShare(qd, kd, vd, P, r, layout, seg=sd, window=window, fused=fused)
        acc, lse = sh.forward()
        pos = oracle.rank_positions(r, P, S, layout)
        check_rows(f64(acc), f64(lse), ro[:, pos], rl[:, :, pos], 1e-2, 1e-3)
        dq = torch.zeros(acc.shape, device="cuda")
        sh.backward(acc.bfloat16(), lse, dd[:, r * C:(r + 1) * C], dq, dk, dv)
        assert max_err(f64(dq), rq[:, pos]) <= grad_tol(rq), f"rank {r} dq"
    if st is not None:
        dk, dv = (cp.zigzag_reorder(t, P, inverse=True, strategy=st) for t in (dk, dv))
    assert max_err(f64(dk), rk) <= grad_tol(rk), "dk"
    assert max_err(f64(dv), rv) <= grad_tol(rv), "dv"
