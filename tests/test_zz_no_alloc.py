"""cp_attn_bwd_noalloc (the backward with the library's own device scratch) against
cp_attn_bwd with a caller-owned workspace, through the C ABI (GPU only).

Two calls in a row on the same device, the second smaller, each compared with the
existing entry point on every element: the kernels are the same and deterministic,
so the gradients agree bit for bit (stricter than the gradient bar).  The first call
uses the scratch's head-split partials as well as its row arrays.
"""

import pytest
import torch

import cp_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cp():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import context_cp_attn_amd as cp
    cp.load_library()
    return cp


def _case(cp, B, Sq, Sk, Hq, Hkv, D, seed, **mask):
    q, k, v, do = (t.cuda() for t in cp_inputs.normal_tensors(
        [(B, Sq, Hq, D), (B, Sk, Hkv, D), (B, Sk, Hkv, D), (B, Sq, Hq, D)], seed=seed))
    o, l = cp.attn_fwd(q, k, v, **mask)
    return q, k, v, o, l, do


@pytest.mark.parametrize("accumulate", [False, True])
def test_noalloc_matches_workspace_backward(cp, accumulate):
    from context_cp_attn_amd import _lib
    from context_cp_attn_amd.ops import make_args
    import ctypes
    lib = _lib.load()
    # 1) a packed ring step of the 8K workload's shape (grouped heads: the key side is
    #    split over head halves, whose partials live in the scratch); 2) a smaller
    #    dense causal block
    seg = cp_inputs.segment_ids([300, 900, 848]).cuda()
    cases = [
        dict(shape=(1, 2048, 2048, 32, 8, 128), seed=3,
             mask=dict(q_seg=seg, k_seg=seg, window=1024, q_offset=0, k_offset=0)),
        dict(shape=(1, 700, 700, 2, 2, 128), seed=4, mask=dict()),
    ]
    for c in cases:
        q, k, v, o, l, do = _case(cp, *c["shape"], c["seed"], **c["mask"])
        need = lib.cp_attn_bwd_workspace_size(ctypes.byref(make_args(q, k, **c["mask"])))
        print(f"noalloc shape={c['shape']} workspace={need} accumulate={accumulate}", flush=True)
        assert 0 < need <= _lib.CP_ATTN_BWD_NOALLOC_MAX_BYTES
        g = torch.Generator().manual_seed(c["seed"] + 100)
        init = [torch.randn(t.shape, generator=g).cuda() if accumulate else torch.zeros(t.shape, device="cuda")
                for t in (q, k, v)]
        ref = [t.clone() for t in init]
        cp.attn_bwd(q, k, v, o, l, do, dq=ref[0], dk=ref[1], dv=ref[2], accumulate=accumulate, **c["mask"])
        got = [t.clone() for t in init]
        cp.attn_bwd_noalloc(q, k, v, o, l, do, *got, accumulate=accumulate, **c["mask"])
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), f"{name} differs (max {float((a - b).abs().max())})"
