"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects bad arguments before it
launches anything.  No GPU is needed (and none is touched)."""
import ctypes

import numpy as np
import os
import re
import subprocess

import pytest
import torch

import block_sparse_attention_select_amd as msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")

# The argument checks below pass made-up device addresses that must never be
# dereferenced; keep them off machines with a GPU.
no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="uses fake device pointers; CPU-only host checks")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = msa.load()
    names = declared_functions()
    assert set(names) == set(msa.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", msa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (msa_\w+)", out))
    assert set(names) <= exported
    assert lib.msa_version() >= 100


def test_status_strings():
    for st in (0, -1, -2, -3, -4):
        s = msa.status_string(st)
        assert s.startswith("MSA_")
    assert "unknown" in msa.status_string(7)


def dims(**kw):
    base = dict(total_tokens=16384, num_seqs=3, max_seqlen=7122, num_q_heads=16, num_kv_heads=1)
    base.update(kw)
    return msa.make_dims(**base)


def test_workspace_sizes_are_positive_and_monotone():
    small = {op: msa.msa_workspace_size(dims(total_tokens=1024, num_seqs=1, max_seqlen=1024), op)
             for op in (msa.MSA_OP_SELECT, msa.MSA_OP_FWD, msa.MSA_OP_BWD)}
    big = {op: msa.msa_workspace_size(dims(), op) for op in (msa.MSA_OP_SELECT, msa.MSA_OP_FWD, msa.MSA_OP_BWD)}
    for op in small:
        assert 0 < small[op] < big[op]
        assert big[op] % 256 == 0
    assert msa.msa_workspace_size(dims(total_tokens=0, num_seqs=0, max_seqlen=0), msa.MSA_OP_BWD) == 0
    # without the stored dS the unsharded 32k layer stays within a few GiB of scratch
    layer = dims(total_tokens=32768, num_seqs=1, max_seqlen=32768, num_q_heads=64, num_kv_heads=4)
    assert msa.msa_workspace_size(layer, msa.MSA_OP_BWD_RECOMPUTE) < 3 << 30


@pytest.mark.parametrize("T,S,L,hk", [(16384, 3, 7122, 1), (32768, 1, 32768, 4), (65536, 2, 65536, 4),
                                      (131072, 1, 131072, 2), (131072, 1, 131072, 4)])
def test_backward_workspace_stored_ds_tail(T, S, L, hk):
    """The backward workspace ends with 64 KB of stored dS per (token, KV head) while that tail stays within
    16 GiB (T * Hk <= 262144); beyond it the backward recomputes and needs no tail."""
    d = dims(total_tokens=T, num_seqs=S, max_seqlen=L, num_q_heads=16 * hk, num_kv_heads=hk)
    full = msa.msa_workspace_size(d, msa.MSA_OP_BWD)
    lean = msa.msa_workspace_size(d, msa.MSA_OP_BWD_RECOMPUTE)
    tail = T * hk * 65536 if T * hk <= 262144 else 0
    assert full == lean + tail


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), msa.MSA_ERR_UNSUPPORTED),
    (dict(block_size=64), msa.MSA_ERR_UNSUPPORTED),
    (dict(topk_blocks=8), msa.MSA_ERR_UNSUPPORTED),
    (dict(num_q_heads=8), msa.MSA_ERR_UNSUPPORTED),
    (dict(num_q_heads=32, num_kv_heads=1), msa.MSA_ERR_UNSUPPORTED),
    (dict(max_seqlen=200000, total_tokens=300000), msa.MSA_ERR_UNSUPPORTED),
    (dict(total_tokens=-1), msa.MSA_ERR_INVALID_ARG),
    (dict(num_seqs=0), msa.MSA_ERR_INVALID_ARG),
    (dict(max_seqlen=0), msa.MSA_ERR_INVALID_ARG),
    (dict(max_seqlen=20000), msa.MSA_ERR_INVALID_ARG),
])
def test_workspace_size_rejects_bad_dims(kw, status):
    n = ctypes.c_size_t(0)
    d = dims(**kw)
    assert msa.load().msa_workspace_size(ctypes.byref(d), msa.MSA_OP_FWD, ctypes.byref(n)) == status


FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced


def _fwd(lib, d, q=FAKE, q_st=2048, q_sh=128, k=FAKE, v=FAKE, blk=FAKE, cu=FAKE, scale=0.088, o=FAKE,
         o_st=2048, o_sh=128, lse=FAKE, ws=FAKE, nbytes=1 << 40):
    return lib.msa_attn_fwd(ctypes.byref(d), q, q_st, q_sh, k, 128, 128, v, 128, 128, blk, cu, scale,
                            o, o_st, o_sh, lse, ws, nbytes, None)


@no_gpu
def test_fwd_argument_errors_launch_nothing():
    lib = msa.load()
    d = dims()
    assert _fwd(lib, d, q=None) == msa.MSA_ERR_INVALID_ARG
    assert _fwd(lib, d, q=FAKE + 2) == msa.MSA_ERR_INVALID_ARG       # misaligned
    assert _fwd(lib, d, q_st=2047) == msa.MSA_ERR_INVALID_ARG         # stride not a multiple of 8
    assert _fwd(lib, d, o_sh=0) == msa.MSA_ERR_INVALID_ARG            # broadcast output
    assert _fwd(lib, d, blk=None) == msa.MSA_ERR_INVALID_ARG
    assert _fwd(lib, d, lse=FAKE + 4) == msa.MSA_ERR_INVALID_ARG
    assert _fwd(lib, d, scale=0.0) == msa.MSA_ERR_INVALID_ARG
    assert _fwd(lib, d, scale=float("nan")) == msa.MSA_ERR_INVALID_ARG
    assert _fwd(lib, d, ws=None) == msa.MSA_ERR_WORKSPACE
    assert _fwd(lib, d, ws=FAKE + 16) == msa.MSA_ERR_WORKSPACE        # not 256-byte aligned
    need = msa.msa_workspace_size(d, msa.MSA_OP_FWD)
    assert _fwd(lib, d, nbytes=need - 1) == msa.MSA_ERR_WORKSPACE
    # empty pack: a no-op that touches nothing
    assert _fwd(lib, dims(total_tokens=0, num_seqs=0, max_seqlen=0), q=None, ws=None) == msa.MSA_OK


@no_gpu
def test_qk_norm_argument_errors_launch_nothing():
    lib = msa.load()
    d = dims()
    fwd = lambda **kw: lib.msa_qk_norm_rope_fwd(
        ctypes.byref(d), kw.get("q", FAKE), 2048, 128, FAKE, 128, 128, FAKE, FAKE, 1e-6, 1e7, kw.get("rope", 64),
        FAKE, FAKE, 2048, kw.get("qo_sh", 128), FAKE, 128, 128, None)
    assert fwd(rope=32) == msa.MSA_ERR_UNSUPPORTED
    assert fwd(q=None) == msa.MSA_ERR_INVALID_ARG
    assert fwd(qo_sh=0) == msa.MSA_ERR_INVALID_ARG      # broadcast output
    bwd = lambda **kw: lib.msa_qk_norm_rope_bwd(
        ctypes.byref(d), FAKE, 2048, 128, FAKE, 128, 128, FAKE, FAKE, 1e-6, 1e7, 64, FAKE, FAKE, 2048, 128,
        FAKE, 128, 128, FAKE, 2048, 128, FAKE, 128, 128, kw.get("dw", FAKE), FAKE, FAKE, kw.get("n", 1 << 40), None)
    assert bwd(dw=None) == msa.MSA_ERR_INVALID_ARG
    assert bwd(n=msa.msa_workspace_size(d, msa.MSA_OP_QKNORM_BWD) - 256) == msa.MSA_ERR_WORKSPACE


@no_gpu
def test_select_and_bwd_argument_errors_launch_nothing():
    lib = msa.load()
    d = dims()
    sel = lambda **kw: lib.msa_index_select(
        ctypes.byref(kw.get("d", d)), kw.get("iq", FAKE), 128, 128, FAKE, 128, kw.get("sk_h", 128), FAKE, FAKE,
        1e-6, kw.get("base", 1e7), kw.get("rope", 64), FAKE, kw.get("blk", FAKE), kw.get("ws", FAKE),
        kw.get("n", 1 << 40), None)
    assert sel(rope=32) == msa.MSA_ERR_UNSUPPORTED
    assert sel(base=1.0) == msa.MSA_ERR_INVALID_ARG
    assert sel(iq=None) == msa.MSA_ERR_INVALID_ARG
    assert sel(blk=FAKE + 4) == msa.MSA_ERR_INVALID_ARG
    assert sel(n=0) == msa.MSA_ERR_WORKSPACE
    assert sel(d=dims(total_tokens=0, num_seqs=0, max_seqlen=0), iq=None, ws=None) == msa.MSA_OK

    sel_ex = lambda flags, **kw: lib.msa_index_select_ex(
        ctypes.byref(d), FAKE, 128, 128, FAKE, 128, 128, FAKE, FAKE, 1e-6, 1e7, 64, flags, FAKE, FAKE, FAKE,
        kw.get("n", 1 << 40), None)
    assert sel_ex(2) == msa.MSA_ERR_INVALID_ARG            # unknown flag bit
    assert sel_ex(0x80000000) == msa.MSA_ERR_INVALID_ARG
    assert sel_ex(msa.MSA_SELECT_FORCE_INIT, n=0) == msa.MSA_ERR_WORKSPACE

    def bwd(dv_sh=128, ws=FAKE, n=1 << 40, lse=FAKE):
        return lib.msa_attn_bwd(ctypes.byref(d), FAKE, 2048, 128, FAKE, 128, 128, FAKE, 128, 128, FAKE, 2048, 128,
                                lse, FAKE, 2048, 128, FAKE, FAKE, 0.088, FAKE, 2048, 128, FAKE, 128, 128,
                                FAKE, 128, dv_sh, ws, n, None)
    assert bwd(dv_sh=0) == msa.MSA_ERR_INVALID_ARG
    assert bwd(lse=None) == msa.MSA_ERR_INVALID_ARG
    assert bwd(n=msa.msa_workspace_size(d, msa.MSA_OP_BWD) - 256) == msa.MSA_ERR_WORKSPACE


def qsa_dims(**kw):
    base = dict(total_tokens=16384, num_seqs=3, max_seqlen=7122, num_q_heads=12, num_kv_heads=1, head_dim=256,
                block_size=4, topk_blocks=512)
    base.update(kw)
    return msa.make_dims(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(), msa.MSA_OK),
    (dict(head_dim=128), msa.MSA_ERR_UNSUPPORTED),
    (dict(block_size=128), msa.MSA_ERR_UNSUPPORTED),
    (dict(topk_blocks=1025), msa.MSA_ERR_UNSUPPORTED),
    (dict(topk_blocks=0), msa.MSA_ERR_INVALID_ARG),
    (dict(num_q_heads=16), msa.MSA_ERR_UNSUPPORTED),
    (dict(max_seqlen=40000, total_tokens=50000), msa.MSA_ERR_UNSUPPORTED),
    (dict(num_seqs=0), msa.MSA_ERR_INVALID_ARG),
])
def test_qsa_workspace_dims(kw, status):
    """The narrow-block entry points validate their own dims (D 256, block 4, 12 q / kv, K <= 1024)."""
    n = ctypes.c_size_t(0)
    d = qsa_dims(**kw)
    for op in (msa.MSA_OP_QSA_FWD, msa.MSA_OP_QSA_BWD):
        assert msa.load().msa_workspace_size(ctypes.byref(d), op, ctypes.byref(n)) == status
        if status == msa.MSA_OK:
            assert n.value > 0 and n.value % 256 == 0
    # the wide dims are not narrow dims and vice versa
    assert msa.load().msa_workspace_size(ctypes.byref(dims()), msa.MSA_OP_QSA_FWD, ctypes.byref(n)) == \
        msa.MSA_ERR_UNSUPPORTED
    assert msa.load().msa_workspace_size(ctypes.byref(qsa_dims()), msa.MSA_OP_FWD, ctypes.byref(n)) == \
        msa.MSA_ERR_UNSUPPORTED


def _dslines(lengths):
    """dS lines of the narrow backward per (KV head, query head): one per (token, causal 64-key tile)."""
    return sum(p // 64 + 1 for L in lengths for p in range(L))


@pytest.mark.parametrize("T,M,S,hk", [(16384, 7122, 3, 1), (5000, 5000, 1, 2), (4097, 64, 65, 1), (3000, 1100, 3, 1),
                                      (200, 7, 40, 1)])
def test_qsa_backward_workspace_holds_every_dslines_mix(T, M, S, hk):
    """The narrow backward workspace covers the dS lines of the worst pack its dims allow (sequences as long as
    max_seqlen, the rest in one), by brute force over the lines."""
    n_b = ctypes.c_size_t(0)
    d = qsa_dims(total_tokens=T, num_seqs=S, max_seqlen=M, num_q_heads=12 * hk, num_kv_heads=hk)
    assert msa.load().msa_workspace_size(ctypes.byref(d), msa.MSA_OP_QSA_BWD, ctypes.byref(n_b)) == msa.MSA_OK
    worst = [M] * (T // M) + ([T % M] if T % M else [])
    lines = _dslines(worst) * hk * 12
    assert n_b.value >= lines * 128
    # any other mix of lengths up to M summing to T needs no more lines
    rng = np.random.default_rng(T)
    for _ in range(20):
        left, mix = T, []
        while left > 0:
            L = int(rng.integers(1, min(M, left) + 1))
            mix.append(L)
            left -= L
        assert _dslines(mix) * hk * 12 <= lines


@no_gpu
def test_qsa_argument_errors_launch_nothing():
    lib = msa.load()
    d = qsa_dims()

    def fwd(q=FAKE, o_sh=256, blk=FAKE, scale=0.0625, ws=FAKE, n=1 << 40, dd=d):
        return lib.msa_qsa_attn_fwd(ctypes.byref(dd), q, 3072, 256, FAKE, 256, 256, FAKE, 256, 256, blk, FAKE, scale,
                                    FAKE, 3072, o_sh, FAKE, ws, n, None)
    assert fwd(q=None) == msa.MSA_ERR_INVALID_ARG
    assert fwd(o_sh=0) == msa.MSA_ERR_INVALID_ARG
    assert fwd(blk=None) == msa.MSA_ERR_INVALID_ARG
    assert fwd(scale=-1.0) == msa.MSA_ERR_INVALID_ARG
    assert fwd(ws=None) == msa.MSA_ERR_WORKSPACE
    assert fwd(n=msa.msa_workspace_size(d, msa.MSA_OP_QSA_FWD) - 256) == msa.MSA_ERR_WORKSPACE
    assert fwd(dd=dims()) == msa.MSA_ERR_UNSUPPORTED
    assert fwd(dd=qsa_dims(total_tokens=0, num_seqs=0, max_seqlen=0), q=None, ws=None) == msa.MSA_OK

    def bwd(dv_sh=256, lse=FAKE, n=1 << 40):
        return lib.msa_qsa_attn_bwd(ctypes.byref(d), FAKE, 3072, 256, FAKE, 256, 256, FAKE, 256, 256, FAKE, 3072,
                                    256, lse, FAKE, 3072, 256, FAKE, FAKE, 0.0625, FAKE, 3072, 256, FAKE, 256, 256,
                                    FAKE, 256, dv_sh, FAKE, n, None)
    assert bwd(dv_sh=0) == msa.MSA_ERR_INVALID_ARG
    assert bwd(lse=None) == msa.MSA_ERR_INVALID_ARG
    assert bwd(n=msa.msa_workspace_size(d, msa.MSA_OP_QSA_BWD) - 256) == msa.MSA_ERR_WORKSPACE


# ---------------------------------------------------------------- binding argument checks
# The binding validates every tensor the kernels read as a plain array before
# it calls into the library.  Dtype, shape and layout are checked before the
# device, so these rejections show on a CPU too.
CPU = torch.device("cpu")


def test_binding_rejects_bad_cu_seqlens():
    for bad in (torch.zeros(4, dtype=torch.int64), torch.zeros(2, 2, dtype=torch.int32),
                torch.zeros(0, dtype=torch.int32), torch.zeros(4, dtype=torch.float32), [0, 5]):
        with pytest.raises(ValueError, match="cu_seqlens"):
            msa._cu_seqlens(bad, CPU)
    with pytest.raises(ValueError, match="cu_seqlens"):              # host memory: never handed to a kernel
        msa._cu_seqlens(torch.zeros(4, dtype=torch.int32), torch.device("cuda", 0))


def test_binding_rejects_bad_norm_weights():
    for bad in (torch.zeros(128, dtype=torch.float32), torch.zeros(64, dtype=torch.bfloat16),
                torch.zeros(2, 128, dtype=torch.bfloat16)):
        with pytest.raises(ValueError, match="w_q"):
            msa._weight(bad, "w_q", CPU)


def test_binding_weight_copy_is_kept_for_the_call():
    """A strided weight comes back as a contiguous copy the caller holds (not a
    temporary whose memory could be reused by the next copy before the launch)."""
    w = torch.arange(256, dtype=torch.float32).bfloat16()[::2]
    with pytest.raises(ValueError):
        msa._weight(w, "w_q", torch.device("cuda", 0))                # device check comes after the layout
    src = open(os.path.join(ROOT, "block_sparse_attention_select_amd", "__init__.py")).read()
    assert "_ptr(w_q.contiguous())" not in src and "_ptr(w_k.contiguous())" not in src


def test_binding_rejects_bad_block_lists_and_lse():
    with pytest.raises(ValueError, match="blk_idx"):
        msa._int32_rows(torch.zeros(10, 1, 16, dtype=torch.int64), "blk_idx", 10, 1, CPU, 16)
    with pytest.raises(ValueError, match="blk_idx"):
        msa._int32_rows(torch.zeros(10, 2, 16, dtype=torch.int32), "blk_idx", 10, 1, CPU, 16)
    with pytest.raises(ValueError, match="blk_idx"):
        msa._int32_rows(torch.zeros(10, 1, 8, dtype=torch.int32), "blk_idx", 10, 1, CPU, 16)
    with pytest.raises(ValueError, match="blk_idx"):
        msa._int32_rows(torch.zeros(10, 16, 1, dtype=torch.int32).transpose(1, 2), "blk_idx", 10, 1, CPU, 16)
    with pytest.raises(ValueError, match="lse"):
        msa._lse_rows(torch.zeros(10, 16, dtype=torch.float64), "lse", 10, 16, CPU)
    with pytest.raises(ValueError, match="lse"):
        msa._lse_rows(torch.zeros(10, 8, dtype=torch.float32), "lse", 10, 16, CPU)
    with pytest.raises(ValueError, match="lse"):
        msa._lse_rows(torch.zeros(16, 10, dtype=torch.float32).t(), "lse", 10, 16, CPU)


def test_binding_rejects_mismatched_shapes():
    k = torch.zeros(10, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        msa._bf16_view(k, "k", (10, 1, 128))
    with pytest.raises(ValueError):
        msa._bf16_view(torch.zeros(10, 1, 128, dtype=torch.float16), "k")


def test_noalloc_forward_rejects_oversize_before_anything():
    """The allocation-free forward checks the workspace it would need against its
    static scratch first: a pack beyond it returns MSA_ERR_WORKSPACE with no
    pointer read, no HIP call and no launch (null pointers here)."""
    d = msa.make_dims(131072, 1, 131072, 32, 2)
    assert msa.msa_workspace_size(d, msa.MSA_OP_FWD) > msa.MSA_NOALLOC_SCRATCH_BYTES
    st = msa.load().msa_attn_fwd_noalloc(d, None, 0, 0, None, 0, 0, None, 0, 0, None, None, 0.1, None, 0, 0,
                                         None, None)
    assert st == msa.MSA_ERR_WORKSPACE
    assert msa.msa_workspace_size(dims(), msa.MSA_OP_FWD) <= msa.MSA_NOALLOC_SCRATCH_BYTES
    big = msa.make_dims(32768, 1, 32768, 64, 4)                  # the unsharded 32k layer fits
    assert msa.msa_workspace_size(big, msa.MSA_OP_FWD) <= msa.MSA_NOALLOC_SCRATCH_BYTES
