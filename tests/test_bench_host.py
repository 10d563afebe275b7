"""Host-side logic of bench.py (no GPU): the kernel-code hash that keys the
committed traffic counters, the profiler kernel-name mapping and the counted
(query head, selected causal key) pairs behind every FLOP figure."""
import os
import shutil

import numpy as np

import bench


def test_code_text_drops_comments_but_keeps_string_literals():
    src = ('int a;  // trailing\n'
           '/* block\n   comment */  int   b = 1;\n'
           'const char* s = "x // kept  /* kept */";\n'
           'asm volatile("s_waitcnt vmcnt(12)" ::: "memory");\n')
    assert bench.code_text(src) == ('int a; int b = 1; const char* s = "x // kept  /* kept */"; '
                                    'asm volatile("s_waitcnt vmcnt(12)" ::: "memory");')


def test_source_hash_ignores_comments_and_layout_not_code(tmp_path, monkeypatch):
    csrc = tmp_path / "csrc"
    shutil.copytree(bench.CSRC, csrc, ignore=shutil.ignore_patterns("*.o", "*.so"))
    monkeypatch.setattr(bench, "CSRC", str(csrc))
    base = bench.kernel_source_hash()
    f = csrc / "attn_fwd.hip"
    text = f.read_text()
    f.write_text("// a new comment line\n" + text.replace("\n\n", "\n\n\n", 3))
    assert bench.kernel_source_hash() == base
    f.write_text(text.replace("kRescaleSlack = 8.f", "kRescaleSlack = 7.f", 1))
    assert bench.kernel_source_hash() != base


def test_kernel_key_names_every_instance():
    k = bench.kernel_key
    assert k("void msa::(anonymous namespace)::attn_fwd_kernel<false, false>(unsigned short const*)") == \
        "attn_fwd_kernel"
    assert k("msa::(anonymous namespace)::attn_fwd_kernel<false, true>(int)") == "attn_fwd_qknorm_kernel"
    assert k("msa::(anonymous namespace)::attn_fwd_kernel<true, false>(int)") == "attn_fwd_dense_kernel"
    assert k("msa::(anonymous namespace)::block_prep_kernel<true>(int)") == "block_prep_qknorm_kernel"
    assert k("msa::(anonymous namespace)::qsa_prep_kernel<true>(int)") == "qsa_prep_swizzled_kernel"
    assert k("msa::(anonymous namespace)::attn_bwd_dkdv_kernel<false, true>(int)") == "attn_bwd_dkdv_kernel"
    assert k("msa::(anonymous namespace)::attn_bwd_dkdv_kernel<false, false>(int)") == \
        "attn_bwd_dkdv_recompute_kernel"
    assert k("msa::(anonymous namespace)::attn_bwd_dq_ds_kernel(int)") == "attn_bwd_dq_kernel"
    assert k("msa::(anonymous namespace)::attn_bwd_dq_kernel<false, false>(int)") == "attn_bwd_dq_recompute_kernel"
    assert k("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_selected_keys_matches_brute_force():
    rng = np.random.default_rng(3)
    lengths = [300, 1, 129, 520]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T, hk, block = int(cu[-1]), 2, 128
    blk = np.full((T, hk, 4), -1, np.int32)
    for s, L in enumerate(lengths):
        for p in range(L):
            b = p // block
            for h in range(hk):
                ids = rng.choice(b + 2, size=min(4, b + 2), replace=False)  # may list b + 1 (ignored)
                blk[cu[s] + p, h, :len(ids)] = ids
    want = 0
    for s, L in enumerate(lengths):
        for p in range(L):
            for h in range(hk):
                for c in blk[cu[s] + p, h]:
                    if 0 <= c <= p // block:
                        want += sum(1 for j in range(block * c, block * c + block) if j <= p)
    assert bench.selected_keys(blk, cu, block) == want
