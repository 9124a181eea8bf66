"""Benchmark of the context-parallel attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-legs]
    python bench.py --leg {ring,reorder,gqa64k,packed,usp}   (one leg alone, for profilers)

Workload (one "step"): the Ulysses share of llama2-7b (MHA, 32 heads, D=128) at
32K context with cp=16, every simulated rank on this one GPU:

  forward:  relayout q, k, v  [16][1,2048,32,128] -> [16][1,32768,2,128]  (bf16)
            16 x attention fwd, one launch per rank at its real shape
            (q/k/v [1,32768,2,128], causal)
            inverse relayout of the output
  backward: relayout dout; 16 x attention bwd (fp32 gradients);
            inverse relayout of dq, dk, dv (fp32)

value = algorithmic attention FLOPs of the step (fwd 4*D and bwd 8*D per visible
(query, key, head) triple) / step time, in TFLOP/s.  Inputs are resident in HBM
before the timed region.  The relayout bandwidth is reported beside it.

Legs timed in the same run (not part of value): the ring share of llama2-7b
(2048 queries x 32 heads vs 16 zigzag KV blocks: the fused step with the merge in
the attention epilogue, and the unfused fwd + merge pair), the 64K-token
dual-chunk-swap reorder, the Ulysses rank share of llama3.1-8b at 64K with cp=4
(q [1,65536,8,128] on k/v [1,65536,2,128], fwd + bwd), the packed + windowed 8K ring
share (4 ranks x 4
steps, fused fwd + merge, bwd; striped as chosen automatically for packed
sequences, and dual-chunk-swap; the whole pass, and each rank's share alone, the
slowest of which sets a 4-GPU step), and llama3.1-8b at 16K on 16 ranks beyond its 8 kv
heads (Ulysses 8 x ring 2, and Ulysses 16 with kv heads replicated).  The CPU oracle
is timed on a bounded sample of the step's attention rows (cpu_baseline).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal attn fwd+bwd TFLOP/s and % bf16 MFMA peak; relayout GB/s on 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E (published)


def pairs_causal(S: int) -> int:
    return S * (S + 1) // 2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    ap.add_argument("--no-legs", action="store_true", help="skip the ring / reorder / packed legs")
    ap.add_argument("--leg", choices=["ring", "reorder", "gqa64k", "packed", "usp"],
                    help="run only this leg and print its JSON (for profilers; no step, no value)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-relayout", action="store_true", help="skip the per-direction relayout timings")
    ap.add_argument("--profile-copy", action="store_true",
                    help="after the timed steps, run one plain 1 GiB device copy (read 1 GiB + write 1 GiB) "
                         "that calibrates the FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


# every file the backward kernel is built from: the committed counter profile is used
# only while its recorded hash of these still matches
BWD_SOURCES = [os.path.join(ROOT, "context_cp_attn_amd", *p) for p in (
    ("csrc", "attn_bwd_mfma.hip"), ("csrc", "mfma_common.h"), ("csrc", "common.h"), ("csrc", "launch.h"),
    ("build.py",))]


def sha_of(*paths):
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


class StepWorkload:
    """The step's inputs, resident in HBM, and the drivers' preallocated Ulysses pass
    (context_cp_attn_amd.drivers.UlyssesStep) over them."""

    P, S, H, D = 16, 32768, 32, 128

    def __init__(self, torch, cp, cp_inputs):
        P, S, H, D = self.P, self.S, self.H, self.D
        q, k, v, do = cp_inputs.normal_tensors([(1, S, H, D)] * 4, seed=0)
        # the global [1,S,H,D] sequence split into P contiguous slices = [P][1][S/P][H][D];
        # q, k, v held together in one [3][P][1][S/P][H][D] buffer (a fused QKV projection's output)
        qkv = torch.stack([t.reshape(P, 1, S // P, H, D) for t in (q, k, v)]).to("cuda")
        self.step = cp.drivers.UlyssesStep(qkv, do.reshape(P, 1, S // P, H, D).to("cuda"), P)
        hp = H // P
        self.flops_fwd_rank = 4 * D * hp * pairs_causal(S)
        self.flops_bwd_rank = 8 * D * hp * pairs_causal(S)
        self.flops = P * (self.flops_fwd_rank + self.flops_bwd_rank)
        # bytes moved by the relayouts of one step: one read + one write each
        bf_bytes = S * H * D * 2  # one whole [P][1][S/P][H][D] bf16 tensor
        self.relayout_bytes = 5 * 2 * bf_bytes + 3 * 2 * 2 * bf_bytes

    def run(self):
        self.step.run()


def timed(torch, fn, reps):
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def frac(x, peak):
    return round(x / peak, 4)


def relayout_directions(torch, cp, step, cp_inputs, reps=20):
    """Each relayout direction alone: one launch per rep, the 256 MB last-level cache
    flushed before it by writing a 1 GiB buffer, HIP events around the launch on the
    launch stream; median and min over the reps.  Bytes = one read + one write of
    the tensor."""
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    us = step.step

    def one(fn, nbytes):
        ts = []
        for _ in range(reps):
            flush.fill_(1)
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            fn()
            e.record()
            torch.cuda.synchronize()
            ts.append(s.elapsed_time(e))
        ts.sort()
        med, mn = ts[len(ts) // 2], ts[0]
        gb_med, gb_max = nbytes / (med * 1e-3) / 1e9, nbytes / (mn * 1e-3) / 1e9
        return {"bytes": nbytes, "median_us": round(med * 1e3, 2), "min_us": round(mn * 1e3, 2),
                "gbps_median": round(gb_med, 1), "gbps_best": round(gb_max, 1),
                "frac_median": frac(gb_med, PEAK_HBM_GBPS), "frac_best": frac(gb_max, PEAK_HBM_GBPS)}

    P = step.P
    qs = us.qkv[0]
    out = {
        # one tensor [16][1,2048,32,128] -> [16][1,32768,2,128] per launch
        "seq_to_head_bf16_llama2_7b_cp16": one(lambda: cp.ulysses_relayout(qs, P, out=us.qkvl[0]),
                                               2 * qs.numel() * 2),
        "head_to_seq_bf16_llama2_7b_cp16": one(lambda: cp.ulysses_relayout_inv(us.ol, P, out=us.out),
                                               2 * us.ol.numel() * 2),
        "head_to_seq_f32_llama2_7b_cp16": one(lambda: cp.ulysses_relayout_inv(us.dqkvl[0], P, out=us.dqkv[0]),
                                              2 * us.dqkvl[0].numel() * 4),
        # q, k and v in one launch, as the step runs them (three groups of the general relayout)
        "seq_to_head_bf16_qkv_llama2_7b_cp16": one(
            lambda: cp.ulysses_relayout_ex(us.qkv, P, groups=3, out=us.qkvl), 2 * us.qkv.numel() * 2),
        "head_to_seq_f32_dqkv_llama2_7b_cp16": one(
            lambda: cp.ulysses_relayout_ex(us.dqkvl, P, groups=3, inverse=True, out=us.dqkv),
            2 * us.dqkvl.numel() * 4),
    }
    # the llama3.1-8b 64K Ulysses share (cp=4): q [4][1,16384,32,128] -> [4][1,65536,8,128],
    # k [4][1,16384,8,128] -> [4][1,65536,2,128]
    S, P4, D = 65536, 4, 128
    for name, H in (("q", 32), ("kv", 8)):
        (x,) = cp_inputs.normal_tensors([(P4, 1, S // P4, H, D)], seed=1)
        x = x.cuda()
        y = torch.empty(P4, 1, S, H // P4, D, device="cuda", dtype=x.dtype)
        out[f"seq_to_head_bf16_llama31_8b_64k_cp4_{name}"] = one(lambda: cp.ulysses_relayout(x, P4, out=y),
                                                                 2 * x.numel() * 2)
        del x, y
    del flush
    return out


def packed_work(seg, P, layout, window, D):
    """Visible (query, key) pairs per head of a causal packed + windowed sequence
    (counted from the segment ids: a query sees the keys of its own document no
    further back than the window), and the fraction of the forward's query-tile x
    key-tile blocks that hold no visible pair over all P ranks' P ring steps, and the
    visible pairs per head of each rank's queries."""
    import numpy as np
    S = seg.shape[0]
    start = np.zeros(S, dtype=np.int64)
    for t in range(1, S):
        start[t] = start[t - 1] if seg[t] == seg[t - 1] else t
    i = np.arange(S)
    pairs = int(np.sum(np.minimum(i - start + 1, window)))
    # the kernel's tiles: 128 query rows x 64 keys of one rank pair
    C = S // P
    if layout == "striped":
        pos = [np.arange(r, S, P) for r in range(P)]
    else:
        c = S // (2 * P)
        pos = [np.r_[np.arange(r * c, (r + 1) * c), np.arange((2 * P - 1 - r) * c, (2 * P - r) * c)] for r in range(P)]
    empty = total = 0
    rank_pairs = []
    for r in range(P):
        rank_pairs.append(0)
        for src in range(P):
            qp, kp = pos[r], pos[src]
            vis = (kp[None, :] <= qp[:, None]) & (seg[qp][:, None] == seg[kp][None, :]) & \
                  (qp[:, None] - kp[None, :] < window)
            rank_pairs[-1] += int(vis.sum())
            blk = vis.reshape(C // 128, 128, C // 64, 64).any(axis=(1, 3))
            empty += int((~blk).sum())
            total += blk.size
    assert sum(rank_pairs) == pairs
    return pairs, empty / total, rank_pairs


def legs(torch, cp, cp_inputs, only=None):
    """Ring share (llama2-7b, cp=16), 64K reorder, the llama3.1-8b 64K rank share (fwd + bwd),
    the packed + windowed ring, and Ulysses beyond the kv head count; ``only`` names
    one of them (ring, reorder, gqa64k, packed, usp) to run that alone."""
    out = {}
    D = 128
    if only in (None, 'ring'):
        # ring share of llama2-7b: rank 0, 16 zigzag steps of fwd + merge
        S, H, D, P = 32768, 32, 128, 16
        q, k, v = (t.cuda() for t in cp_inputs.normal_tensors([(1, S, H, D)] * 3, seed=0))
        qz, kz, vz = (cp.zigzag_reorder(t, P) for t in (q, k, v))
        del q, k, v
        fl = 4 * D * H * (2 * P * (S // (2 * P)) ** 2 + S // (2 * P))
        merge_bytes = (S // P) * H * D * (4 + 2 + 4) + 3 * (S // P) * H * 4
        # unfused: attn_fwd writes (out bf16, lse), lse_merge folds them into (acc, lse_acc)
        # (pass times untraced: the per-launch events of the kernel trace add several
        # microseconds to each of these 50-60 us steps; the per-kernel averages come
        # from a second, traced run)
        ring = cp.drivers.RingShare(qz, kz, vz, P, 0, fused=False)
        for _ in range(4):
            ring.forward()
        ms = timed(torch, ring.forward, 10)
        with cp._lib.KernelTrace() as tr:
            timed(torch, ring.forward, 5)
        fwd_ms, n_fwd = tr.results.get("attn_fwd_mfma", (0.0, 1))
        mg_ms, n_mg = tr.results.get("lse_merge", (0.0, 1))
        # fused: the merge runs in the attention epilogue
        ring_f = cp.drivers.RingShare(qz, kz, vz, P, 0, fused=True)
        for _ in range(4):
            ring_f.forward()
        ms_f = timed(torch, ring_f.forward, 10)
        with cp._lib.KernelTrace() as tr:
            timed(torch, ring_f.forward, 5)
        fm_ms, n_fm = tr.results.get("attn_fwd_merge_mfma", (0.0, 1))
        fm_tf = fl / P / (fm_ms / n_fm) / 1e9    # one step's pairs: the pass's over P steps
        mg_gb = merge_bytes / (mg_ms / n_mg) / 1e6
        out["ring_llama2_7b_32k_cp16_rank0"] = {
            "fused_ms_per_pass": round(ms_f, 4), "fused_tflops": round(fl / ms_f / 1e9, 2),
            "fused_frac": frac(fl / ms_f / 1e9, PEAK_BF16_TFLOPS),
            "attn_fwd_merge_mfma_avg_ms": round(fm_ms / n_fm, 5),
            "attn_fwd_merge_mfma_tflops": round(fm_tf, 2), "attn_fwd_merge_mfma_frac": frac(fm_tf, PEAK_BF16_TFLOPS),
            "kernel_time_frac_of_pass": round(fm_ms / 5 / ms_f, 4),
            "unfused_ms_per_pass": round(ms, 4), "unfused_tflops": round(fl / ms / 1e9, 2),
            "unfused_frac": frac(fl / ms / 1e9, PEAK_BF16_TFLOPS),
            "attn_fwd_mfma_avg_ms": round(fwd_ms / n_fwd, 5),
            "lse_merge_avg_ms": round(mg_ms / n_mg, 5),
            "lse_merge_gbps": round(mg_gb, 1), "lse_merge_frac": frac(mg_gb, PEAK_HBM_GBPS),
            "flop_per_pass": f"4*D*H*(2*P*c^2 + c), c = S/(2P): {fl:.4e}"}
        del qz, kz, vz, ring, ring_f
    if only in (None, 'reorder'):
        # dual-chunk-swap reorder of 64K tokens into 8 chunks: [1,65536,4096] bf16 (512 MiB)
        x = torch.randn(1, 65536, 4096, device="cuda").bfloat16()
        y = torch.empty_like(x)
        cp.zigzag_reorder(x, 4, out=y)
        with cp._lib.KernelTrace() as tr:
            timed(torch, lambda: cp.zigzag_reorder(x, 4, out=y), 10)
        zms, zn = tr.results["zigzag_reorder"]
        zgb = 2 * x.numel() * 2 / (zms / zn) / 1e6
        out["reorder_64k_4096_bf16_cp4"] = {"avg_ms": round(zms / zn, 5), "gbps": round(zgb, 1),
                                            "frac": frac(zgb, PEAK_HBM_GBPS)}
        del x, y
    if only in (None, 'gqa64k'):
        # Ulysses rank share of llama3.1-8b at 64K (cp=4): q [1,65536,8,128], k/v [1,65536,2,128]
        # (8 query heads on 2 kv heads), causal, one forward and one backward per pass
        S, Hq, Hkv = 65536, 8, 2
        q, k, v, do = (t.cuda() for t in cp_inputs.normal_tensors([(1, S, Hq, D), (1, S, Hkv, D), (1, S, Hkv, D),
                                                                   (1, S, Hq, D)], seed=0))
        o, l = cp.attn_fwd(q, k, v)
        bws = cp.bwd_workspace(q, k)
        gq, gk, gv = (torch.empty(t.shape, device="cuda") for t in (q, k, v))

        def gqa_pass():
            cp.attn_fwd(q, k, v, out=o, lse=l)
            cp.attn_bwd(q, k, v, o, l, do, dq=gq, dk=gk, dv=gv, workspace=bws)

        gqa_pass()
        with cp._lib.KernelTrace() as tr:
            ms = timed(torch, gqa_pass, 3)
        ff = 4 * D * Hq * pairs_causal(S)
        f_ms = tr.results["attn_fwd_mfma"][0] / tr.results["attn_fwd_mfma"][1]
        b_ms = tr.results["attn_bwd_mfma"][0] / tr.results["attn_bwd_mfma"][1]
        out["ulysses_llama31_8b_64k_cp4_rank_fwd_bwd"] = {
            "ms_per_pass": round(ms, 3), "tflops": round(3 * ff / ms / 1e9, 2),
            "frac": frac(3 * ff / ms / 1e9, PEAK_BF16_TFLOPS),
            "fwd_avg_ms": round(f_ms, 4), "fwd_tflops": round(ff / f_ms / 1e9, 2),
            "fwd_frac": frac(ff / f_ms / 1e9, PEAK_BF16_TFLOPS),
            "bwd_avg_ms": round(b_ms, 4), "bwd_tflops": round(2 * ff / b_ms / 1e9, 2),
            "bwd_frac": frac(2 * ff / b_ms / 1e9, PEAK_BF16_TFLOPS)}
        del q, k, v, do, o, l, bws, gq, gk, gv
    if only in (None, 'packed'):
        # packed + windowed ring share: 8K, 32 q / 8 kv heads, docs 256..4096, window 4096, cp=4,
        # with the automatic strategy (striped for packed sequences) and with dual-chunk-swap
        S, Hq, Hkv, P = 8192, 32, 8, 4
        q, k, v, do = (t.cuda() for t in cp_inputs.normal_tensors([(1, S, Hq, D), (1, S, Hkv, D), (1, S, Hkv, D),
                                                                   (1, S, Hq, D)], seed=0))
        seg = cp_inputs.segment_ids(cp_inputs.doc_lengths(S)).cuda()
        C = S // P
        for name, st in (("auto", cp.drivers.auto_strategy(packed=True)), ("dual_chunk_swap", 0)):
            layout = cp.drivers.LAYOUT_OF_STRATEGY[st]
            qz, kz, vz, dz, sz = (cp.zigzag_reorder(t, P, strategy=st) for t in (q, k, v, do, seg))
            shares = [cp.drivers.RingShare(qz, kz, vz, P, r, layout=layout, seg=sz, window=4096) for r in range(P)]

            dk = torch.zeros(kz.shape, device="cuda")
            dv = torch.zeros(vz.shape, device="cuda")

            def rank_pass(r):
                o, l = shares[r].forward()
                ob = o.bfloat16()
                dq = torch.zeros(1, C, Hq, D, device="cuda")
                shares[r].backward(ob, l, dz[:, r * C:(r + 1) * C], dq, dk, dv)

            def packed_pass():
                dk.zero_()
                dv.zero_()
                for r in range(P):
                    rank_pass(r)

            packed_pass()
            ms = timed(torch, packed_pass, 3)
            # each rank's share alone: on P GPUs the ranks run at once and the step
            # lasts as long as the slowest of them
            rank_ms = [timed(torch, lambda: rank_pass(r), 3) for r in range(P)]
            pairs, skipped, rank_pairs = packed_work(seg[0].cpu().numpy(), P, layout, 4096, D)
            fl = 12 * D * Hq * pairs  # forward 4*D + backward 8*D per visible pair and head
            slow = max(rank_ms)
            out[f"packed_window_8k_cp4_all_ranks_{name}"] = {
                "strategy": layout, "ms_per_pass": round(ms, 3), "visible_pairs_per_head": pairs,
                "tflops": round(fl / ms / 1e9, 2), "frac": frac(fl / ms / 1e9, PEAK_BF16_TFLOPS),
                "fwd_tiles_skipped_frac": round(skipped, 4),
                "rank_ms": [round(x, 3) for x in rank_ms], "rank_visible_pairs_per_head": rank_pairs,
                "slowest_rank_ms": round(slow, 3),
                "per_gpu_tflops_at_slowest_rank": round(fl / P / slow / 1e9, 2),
                "per_gpu_frac_at_slowest_rank": frac(fl / P / slow / 1e9, PEAK_BF16_TFLOPS)}
    if only in (None, 'usp'):
        # beyond the kv head count, llama3.1-8b (32 q / 8 kv heads) at 16K tokens on 16 ranks:
        # Ulysses 8 within groups x ring 2 across them (USP), and Ulysses 16 with kv heads
        # replicated 2x; forward of all ranks, algorithmic causal FLOPs of the whole sequence
        S, Hq, Hkv = 16384, 32, 8
        q, k, v = (t.cuda() for t in cp_inputs.normal_tensors([(1, S, Hq, D), (1, S, Hkv, D), (1, S, Hkv, D)], seed=0))
        fl = 4 * D * Hq * S * (S + 1) / 2
        usp = lambda: cp.drivers.usp_forward(q, k, v, 2, 8)
        usp()
        ms = timed(torch, usp, 3)
        out["usp_llama31_8b_16k_ulysses8_ring2_fwd"] = {"ms_per_pass": round(ms, 3), "tflops": round(fl / ms / 1e9, 2),
                                                         "frac": frac(fl / ms / 1e9, PEAK_BF16_TFLOPS)}
        P = 16
        st = lambda t: t.reshape(P, 1, S // P, t.shape[2], D)
        uly = lambda: cp.drivers.ulysses_forward(st(q), st(k), st(v), P, kv_rep=2)
        uly()
        ms = timed(torch, uly, 3)
        out["ulysses16_kv_rep2_llama31_8b_16k_fwd"] = {"ms_per_pass": round(ms, 3), "tflops": round(fl / ms / 1e9, 2),
                                                        "frac": frac(fl / ms / 1e9, PEAK_BF16_TFLOPS)}
    return out


def cpu_baseline(torch, cp_inputs, budget_s):
    """The oracle (numpy float64) on a bounded sample of the step's attention rows."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    S, H, D = 32768, 2, 128
    q, k, v, do = (t.float().numpy().astype(np.float64)
                   for t in cp_inputs.normal_tensors([(1, S, H, D)] * 4, seed=7))
    stride = 3  # every 3rd row: about 15 s of float64 work on 16 host cores
    rows = np.arange(S - 1, -1, -stride)  # spread over the sequence, heaviest first
    t0 = time.perf_counter()
    done_pairs, n = 0, 0
    for i0 in range(0, len(rows), 64):
        r = np.sort(rows[i0:i0 + 64])
        qr, gr = q[:, r], do[:, r]
        o, l = oracle.attn_fwd(qr, k, v, q_pos=r)
        oracle.attn_bwd(qr, k, v, o, l, gr, q_pos=r)
        done_pairs += int((r + 1).sum()) * H
        n += len(r)
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    flops = done_pairs * 12 * D
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} query rows x {H} heads (one row in {stride} of S=32768, from the end, causal) fwd+bwd in float64 "
                      f"against all keys, {dt:.1f} s"}


def traffic_from_profiles(kernel_sha):
    """HBM bytes per launch from committed rocprofv3 counters, if they match the source."""
    p = os.path.join(ROOT, "profiles", "attn_bwd_mfma_ulysses_llama2_7b_32k_counters.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_source_sha") != kernel_sha:
        return None
    return d.get("hbm_bytes_per_launch")


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {a.gpus} is not supported (every simulated "
              "context-parallel rank runs on the one GPU)", file=sys.stderr)
        sys.exit(2)
    import torch
    import cp_inputs
    import context_cp_attn_amd as cp
    cp.load_library()
    torch.cuda.set_device(0)
    if a.leg:
        print(json.dumps({"leg": a.leg, "legs": legs(torch, cp, cp_inputs, only=a.leg)}), flush=True)
        return

    step = StepWorkload(torch, cp, cp_inputs)
    for _ in range(a.warmup):
        step.run()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with cp._lib.KernelTrace() as tr:
        torch.cuda.synchronize()
        s.record()
        for _ in range(a.steps):
            step.run()
        e.record()
        torch.cuda.synchronize()
    ms = s.elapsed_time(e) / a.steps
    value = step.flops / (ms * 1e-3) / 1e12
    kern = {k_: {"avg_ms": round(t / n, 5), "launches": n} for k_, (t, n) in tr.results.items()}
    # dominant kernel: the most total time
    dom = max(tr.results.items(), key=lambda kv: kv[1][0])[0]
    bwd_ms = tr.results["attn_bwd_mfma"][0] / tr.results["attn_bwd_mfma"][1]
    fwd_ms = tr.results["attn_fwd_mfma"][0] / tr.results["attn_fwd_mfma"][1]
    rel_t = sum(tr.results[k_][0] for k_ in ("ulysses_relayout", "ulysses_relayout_inv")) / a.steps
    bwd_sha = sha_of(*BWD_SOURCES)
    if dom == "attn_bwd_mfma":
        ach = step.flops_bwd_rank / (bwd_ms * 1e-3) / 1e12
        roof = {"kernel": "attn_bwd_mfma", "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_from_profiles(bwd_sha), "avg_launch_ms": round(bwd_ms, 4),
                "algorithmic_per_launch": f"8*D*Hq*S(S+1)/2 = {step.flops_bwd_rank:.4e} FLOP"}
    else:
        ach = step.flops_fwd_rank / (fwd_ms * 1e-3) / 1e12
        roof = {"kernel": "attn_fwd_mfma", "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "avg_launch_ms": round(fwd_ms, 4),
                "algorithmic_per_launch": f"4*D*Hq*S(S+1)/2 = {step.flops_fwd_rank:.4e} FLOP"}
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "ulysses_llama2_7b_32k_cp16", "global_batch": 1, "seq_len": 32768,
                   "heads": 32, "head_dim": 128, "cp": 16,
                   "parallelism": "cp16 Ulysses, all 16 ranks simulated on 1 GPU",
                   "step": "relayout q,k,v; 16x fwd; relayout_inv out; relayout dout; 16x bwd; "
                           "relayout_inv dq,dk,dv"},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(step.flops_fwd_rank / (fwd_ms * 1e-3) / 1e12, 2),
        "bwd_tflops": round(step.flops_bwd_rank / (bwd_ms * 1e-3) / 1e12, 2),
        # the FlashAttention papers count the backward as 10*D per pair (QK^T recomputed);
        # printed for comparison only, never used in value or roofline
        "bwd_tflops_fa_convention_10D": round(step.flops_bwd_rank * 10 / 8 / (bwd_ms * 1e-3) / 1e12, 2),
        "relayout_gbps": round(step.relayout_bytes / (rel_t * 1e-3) / 1e9, 1),
        "relayout_pct_hbm_peak": round(100 * step.relayout_bytes / (rel_t * 1e-3) / 1e9 / PEAK_HBM_GBPS, 1),
        "fwd_frac": frac(step.flops_fwd_rank / (fwd_ms * 1e-3) / 1e12, PEAK_BF16_TFLOPS),
        "bwd_frac": frac(step.flops_bwd_rank / (bwd_ms * 1e-3) / 1e12, PEAK_BF16_TFLOPS),
        "roofline": roof,
        "kernels": kern,
    }
    if a.profile_copy:
        src_buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst_buf = torch.empty_like(src_buf)
        torch.cuda.synchronize()
        dst_buf.copy_(src_buf)
        torch.cuda.synchronize()
        del src_buf, dst_buf
    if not a.no_relayout:
        res["relayout_directions"] = relayout_directions(torch, cp, step, cp_inputs)
    if not a.no_legs:
        res["legs"] = legs(torch, cp, cp_inputs)
    res["cpu_baseline"] = None if a.no_cpu else cpu_baseline(torch, cp_inputs, a.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
