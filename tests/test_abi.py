"""The C ABI without a GPU: the library loads, exports what include/*.h declares,
and rejects invalid arguments with the documented status codes before touching
device memory (fake, never-dereferenced pointers are passed)."""

import ctypes
import glob
import os
import re

import pytest

from context_cp_attn_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE_A, FAKE_B, FAKE_C = 1 << 32, 1 << 36, 1 << 40   # 16-byte aligned, far apart
INVALID, UNSUPPORTED, ALIAS = _lib.CP_ERR_INVALID, _lib.CP_ERR_UNSUPPORTED, _lib.CP_ERR_ALIAS


def declared_symbols():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(cp_[a-z0-9_]+)\s*\(", text))
    return names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_symbols()
    assert {"cp_attn_fwd", "cp_attn_bwd", "cp_lse_merge", "cp_ulysses_relayout",
            "cp_ulysses_relayout_inv", "cp_zigzag_reorder"} <= names
    for n in names:
        assert hasattr(lib, n), n
    assert set(_lib.SIGNATURES) == names


def test_status_strings():
    lib = _lib.load()
    assert [lib.cp_status_string(i).decode() for i in range(5)] == [
        "CP_OK", "CP_ERR_INVALID", "CP_ERR_UNSUPPORTED", "CP_ERR_ALIAS", "CP_ERR_HIP"]


def args(**kw):
    a = dict(batch=1, seqlen_q=64, seqlen_k=64, heads_q=4, heads_kv=2, head_dim=128, dtype=0,
             causal=1, q_offset=0, k_offset=0, q_pos=None, k_pos=None, q_seg=None, k_seg=None,
             window=0, softmax_scale=0.0)
    a.update(kw)
    return _lib.AttnArgs(**a)


def fwd(a, q=FAKE_A, k=FAKE_B, v=FAKE_C, out=1 << 44, lse=1 << 45):
    lib = _lib.load()
    return lib.cp_attn_fwd(ctypes.byref(a), q, k, v, out, lse, None), lib.cp_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(batch=0), INVALID, "sizes must be >= 1"),
    (dict(seqlen_q=-3), INVALID, "sizes must be >= 1"),
    (dict(heads_q=6, heads_kv=4), INVALID, "not a multiple"),
    (dict(dtype=7), INVALID, "unknown dtype"),
    (dict(causal=2), INVALID, "causal"),
    (dict(window=-1), INVALID, "window"),
    (dict(q_seg=FAKE_A), INVALID, "both"),
    (dict(softmax_scale=-1.0), INVALID, "softmax_scale"),
    (dict(q_offset=-5), INVALID, "q_offset"),
    # the last position would pass 2^31 (and q_offset + seqlen_q would pass 2^63)
    (dict(q_offset=(1 << 31) - 64), INVALID, "q_offset"),
    (dict(q_offset=(1 << 63) - 8), INVALID, "q_offset"),
    (dict(k_offset=(1 << 63) - 8), INVALID, "k_offset"),
    (dict(head_dim=256), UNSUPPORTED, "head_dim"),
    (dict(head_dim=256, dtype=1), UNSUPPORTED, "head_dim"),
    # bounded before the byte-size test multiplies by it
    (dict(head_dim=1 << 40), UNSUPPORTED, "head_dim"),
    # 2^31 or more rows over batches and heads: the 32-bit grid indices would wrap
    (dict(batch=65535, heads_q=65535, heads_kv=1, seqlen_q=1, seqlen_k=1, head_dim=16), UNSUPPORTED, "rows"),
    (dict(batch=2, heads_q=1 << 15, heads_kv=1, seqlen_q=1, seqlen_k=1 << 15, head_dim=16), UNSUPPORTED, "rows"),
])
def test_attn_fwd_rejects(kw, code, msg):
    st, err = fwd(args(**kw))
    assert st == code and msg in err


def test_attn_fwd_alias_and_alignment():
    st, err = fwd(args(), out=FAKE_A)       # out == q
    assert st == ALIAS
    st, err = fwd(args(), lse=FAKE_C + 64)  # lse inside v
    assert st == ALIAS
    st, err = fwd(args(), q=FAKE_A + 2)     # bf16 operands must be 16-byte aligned
    assert st == INVALID and "aligned" in err
    # head dims without a matrix-core kernel only need element alignment
    st, err = fwd(args(head_dim=16), q=FAKE_A + 1)
    assert st == INVALID and "aligned" in err
    st, err = fwd(args(head_dim=16), out=(1 << 44) + 1)
    assert st == INVALID and "misaligned" in err


def test_attn_fwd_workspace_rules():
    lib = _lib.load()
    size = lambda a: lib.cp_attn_fwd_workspace_size(ctypes.byref(a))
    small = args(seqlen_k=8192)                      # 4 query tiles, 8192 keys: the split applies
    rows = 1 * 64 * 4
    assert size(args(seqlen_k=8191)) == 0            # too few keys to pay for the combine
    assert size(small) >= 2 * rows * 128 * 4 + 2 * rows * 4 and size(small) % 256 == 0
    assert size(args(dtype=1)) == 0                  # float32: row-per-wavefront path
    assert size(args(head_dim=16)) == 0              # bf16 without a matrix-core kernel
    assert size(args(seqlen_q=1 << 17, heads_q=16, heads_kv=2)) == 0   # fills the device
    assert size(args(batch=0)) == 0
    # shapes the call itself refuses get no workspace size either
    assert size(args(batch=65535, heads_q=65535, heads_kv=1, seqlen_q=1 << 30, seqlen_k=1 << 30)) == 0
    assert size(args(seqlen_k=8192, q_offset=-1)) == 0
    assert size(args(seqlen_k=8192, heads_q=6, heads_kv=4)) == 0

    def call(a, ws, nbytes):
        st = lib.cp_attn_fwd_ws(ctypes.byref(a), FAKE_A, FAKE_B, FAKE_C, 1 << 44, 1 << 45, ws, nbytes, None)
        return st, lib.cp_last_error().decode()

    need = size(small)
    ws = 1 << 46
    st, err = call(small, ws, need - 1)
    assert st == INVALID and "workspace" in err
    st, err = call(small, 0, need)
    assert st == INVALID and "workspace" in err
    st, err = call(small, ws + 8, need)
    assert st == INVALID and "aligned" in err
    st, err = call(small, FAKE_B - 256, need)        # over k
    assert st == ALIAS
    assert call(args(batch=0), ws, need)[0] == INVALID   # shared validation


def test_attn_check_args_rejects():
    lib = _lib.load()

    def call(a, flags=1 << 44):
        st = lib.cp_attn_check_args(None if a is None else ctypes.byref(a), flags, None)
        return st, lib.cp_last_error().decode()

    assert call(None)[0] == INVALID
    st, err = call(args(), flags=0)
    assert st == INVALID and "flags" in err
    st, err = call(args(), flags=(1 << 44) + 2)
    assert st == INVALID and "aligned" in err
    assert call(args(seqlen_k=0))[0] == INVALID
    st, err = call(args(k_seg=FAKE_A))
    assert st == INVALID and "both" in err


def test_attn_fwd_merge_rejects():
    lib = _lib.load()

    def call(a, acc=1 << 44, lacc=1 << 45, q=FAKE_A):
        st = lib.cp_attn_fwd_merge(ctypes.byref(a), q, FAKE_B, FAKE_C, acc, lacc, None)
        return st, lib.cp_last_error().decode()

    assert call(args(batch=0))[0] == INVALID        # shared validation with cp_attn_fwd
    st, err = call(args(), acc=0)
    assert st == INVALID and "non-NULL" in err
    st, err = call(args(), acc=(1 << 44) + 4)        # float32 accumulator read as 16-byte vectors
    assert st == INVALID and "aligned" in err
    assert call(args(), acc=FAKE_B)[0] == ALIAS      # accumulator over k
    assert call(args(), lacc=(1 << 44) + 256)[0] == ALIAS  # lse_acc inside the accumulator


def test_attn_bwd_workspace_and_alias():
    lib = _lib.load()
    a = args()
    need = lib.cp_attn_bwd_workspace_size(ctypes.byref(a))
    assert need >= 4 * 4 * 64 and need % 256 == 0
    # grouped heads (4 q / 2 kv) on a grid of few workgroups: each key-side item is
    # split over the group's heads and the workspace adds the float32 dK and dV
    # partials [2][B,Sk,Hkv,D]; not for one q head per kv head, nor for arguments the
    # call would reject
    rows_only = lib.cp_attn_bwd_workspace_size(ctypes.byref(args(heads_kv=4)))
    assert need == rows_only + 2 * 64 * 2 * 128 * 4
    assert lib.cp_attn_bwd_workspace_size(ctypes.byref(args(window=100))) == need
    assert lib.cp_attn_bwd_workspace_size(ctypes.byref(args(heads_kv=3))) == rows_only
    # sizes whose row count overflows int64 ask for nothing (the call itself rejects them)
    assert lib.cp_attn_bwd_workspace_size(ctypes.byref(args(batch=1 << 40, seqlen_q=1 << 40))) == 0
    base = [FAKE_A, FAKE_B, FAKE_C, 1 << 41, 1 << 42, 1 << 43, 1 << 44, 1 << 45, 1 << 46]
    st = lib.cp_attn_bwd(ctypes.byref(a), *base, 0, 1 << 47, need - 1, None)
    assert st == INVALID and "workspace" in lib.cp_last_error().decode()
    st = lib.cp_attn_bwd(ctypes.byref(a), *base, 2, 1 << 47, need, None)
    assert st == INVALID
    bad = list(base)
    bad[6] = FAKE_A  # dq over q
    st = lib.cp_attn_bwd(ctypes.byref(a), *bad, 0, 1 << 47, need, None)
    assert st == ALIAS


def test_attn_bwd_noalloc_rejects():
    """Host-side checks of the allocation-free backward: argument errors as
    cp_attn_bwd, and problems whose workspace exceeds the scratch the library holds
    (the llama3.1-8b 64K share with its head-split partials) are refused before any
    device work."""
    lib = _lib.load()
    base = [FAKE_A, FAKE_B, FAKE_C, 1 << 41, 1 << 42, 1 << 43, 1 << 44, 1 << 45, 1 << 46]
    assert lib.cp_attn_bwd_noalloc(ctypes.byref(args(heads_kv=3)), *base, 0, None) == INVALID
    big = args(seqlen_q=65536, seqlen_k=65536, heads_q=8, heads_kv=2, head_dim=128)
    assert lib.cp_attn_bwd_workspace_size(ctypes.byref(big)) > _lib.CP_ATTN_BWD_NOALLOC_MAX_BYTES
    assert lib.cp_attn_bwd_noalloc(ctypes.byref(big), *base, 0, None) == UNSUPPORTED
    assert "scratch" in lib.cp_last_error().decode()


def test_relayout_rejects():
    lib = _lib.load()
    f = lib.cp_ulysses_relayout
    assert f(FAKE_A, FAKE_B, 16, 1, 32768, 8, 128, 2, None) == INVALID          # degree > kv heads
    assert "cannot exceed" in lib.cp_last_error().decode()
    assert f(FAKE_A, FAKE_B, 4, 1, 30, 8, 16, 4, None) == INVALID               # S % P
    assert f(FAKE_A, FAKE_B, 4, 1, 32, 8, 16, 3, None) == INVALID               # elem bytes
    assert f(FAKE_A, FAKE_A + 64, 4, 1, 32, 8, 16, 4, None) == ALIAS            # overlap
    assert lib.cp_ulysses_relayout_inv(FAKE_A, FAKE_B, 0, 1, 32, 8, 16, 4, None) == INVALID


def test_reorder_rejects():
    lib = _lib.load()
    f = lib.cp_zigzag_reorder
    assert f(FAKE_A, FAKE_B, 1, 30, 4, 4, 0, 0, None) == INVALID     # S % 2P
    assert f(FAKE_A, FAKE_B, 1, 30, 4, 4, 1, 0, None) == INVALID     # striped: S % P
    assert f(FAKE_A, FAKE_A + 8, 1, 32, 4, 4, 1, 0, None) == ALIAS   # striped: overlap
    assert f(FAKE_A, FAKE_B, 1, 32, 4, 4, 5, 0, None) == INVALID     # unknown strategy
    assert f(FAKE_A, FAKE_B, 1, 32, 4, 4, 0, 3, None) == INVALID     # inverse flag
    assert f(FAKE_A, FAKE_A, 1, 32, 4, 4, 0, 0, None) == ALIAS
    # sizes whose byte count overflows int64: rejected before any other arithmetic
    assert f(FAKE_A, FAKE_B, 1 << 40, 1 << 40, 16, 4, 0, 0, None) == INVALID
    assert "2^62" in lib.cp_last_error().decode()


def test_merge_rejects():
    lib = _lib.load()
    f = lib.cp_lse_merge
    assert f(1, 8, 2, 128, FAKE_A, FAKE_B, FAKE_C, 1 << 41, 9, None) == INVALID
    assert f(1, 8, 2, 12, FAKE_A, FAKE_B, FAKE_C, 1 << 41, 1, None) == UNSUPPORTED
    assert f(1, 8, 2, 128, FAKE_A, FAKE_B, FAKE_A, 1 << 41, 1, None) == ALIAS        # out_acc / out_blk
    # every pair of a written buffer (out_acc, lse_acc) with another buffer is refused
    assert f(1, 8, 2, 128, FAKE_A, FAKE_B, FAKE_C, FAKE_A + 256, 1, None) == ALIAS  # out_acc / lse_blk
    assert f(1, 8, 2, 128, FAKE_A, FAKE_C + 64, FAKE_C, 1 << 41, 1, None) == ALIAS   # lse_acc / out_blk
    assert f(1, 8, 2, 128, FAKE_A, FAKE_B, FAKE_C, FAKE_B + 16, 1, None) == ALIAS   # lse_acc / lse_blk
    assert f(1, 8, 2, 128, FAKE_A, FAKE_A + 4096, FAKE_C, 1 << 41, 1, None) == ALIAS  # out_acc / lse_acc
    # 32 GiB of accumulator and beyond: 32-bit vector indices would overflow
    assert f(1, 1 << 21, 32, 128, FAKE_A, FAKE_B, FAKE_C, 1 << 41, 1, None) == UNSUPPORTED
    assert "32 GiB" in lib.cp_last_error().decode()
    assert f(1 << 30, 1 << 30, 1 << 20, 128, FAKE_A, FAKE_B, FAKE_C, 1 << 41, 1, None) == INVALID
    assert "2^62" in lib.cp_last_error().decode()


def test_relayout_ex_rejects():
    lib = _lib.load()

    def call(inp=FAKE_A, out=FAKE_B, **kw):
        a = dict(groups=1, P=4, batch=1, seqlen=32, heads=8, head_dim=16, elem_bytes=2, rep=1, inverse=0)
        a.update(kw)
        st = lib.cp_ulysses_relayout_ex(ctypes.byref(_lib.RelayoutArgs(**a)), inp, out, None)
        return st, lib.cp_last_error().decode()

    assert call(groups=0)[0] == INVALID
    assert call(rep=0)[0] == INVALID
    assert call(seqlen=30)[0] == INVALID                          # S % P
    st, err = call(heads=2, P=4)                                    # 2 heads over 4 ranks, no replication
    assert st == INVALID and "replicated" in err
    assert call(heads=2, P=4, rep=2, inverse=1)[0] == INVALID       # replica sums need float32
    assert call(elem_bytes=3)[0] == INVALID
    assert call(inverse=2)[0] == INVALID
    assert call(groups=70000)[0] == UNSUPPORTED
    st, err = call(batch=1 << 40, seqlen=1 << 32, P=4)               # bytes overflow int64
    assert st == INVALID and "2^62" in err
    # the head side is rep times the sequence side: an output just past the input's
    # end still overlaps when it is the larger side
    assert call(out=FAKE_A + 32 * 8 * 16 * 2 - 16)[0] == ALIAS
    assert lib.cp_ulysses_relayout_ex(None, FAKE_A, FAKE_B, None) == INVALID


def test_pad_rows_rejects():
    lib = _lib.load()
    f = lib.cp_pad_rows
    assert f(FAKE_A, FAKE_B, 0, 8, 16, 4, 0, None) == INVALID          # batch
    assert f(FAKE_A, FAKE_B, 1, 8, 16, 6, 7, None) == INVALID          # fill word needs 4-byte rows
    assert f(FAKE_A, FAKE_A + 16, 1, 8, 16, 4, 0, None) == ALIAS
    assert f(0, FAKE_B, 1, 8, 16, 4, 0, None) == INVALID
    assert f(FAKE_A, FAKE_B, 1 << 40, 8, 1 << 40, 4, 0, None) == INVALID   # bytes overflow int64


def test_python_errors_are_valueerrors():
    with pytest.raises(ValueError):
        _lib.check(INVALID)
