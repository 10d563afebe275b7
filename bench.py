#!/usr/bin/env python3
"""Benchmark of the MSA hot path on one MI355X: index-select + block-sparse
attention forward + backward over one 16384-token THD pack.

A step is one pass of the whole path over one pack already resident in HBM:
msa_index_select, then msa_attn_fwd on its block ids, then msa_attn_bwd.
Prints ONE JSON line.  ``value`` is milliseconds per pack (select + fwd +
bwd; lower is better); the line also carries the split, the counted-FLOP
throughput of fwd+bwd against the bf16 MFMA peak, the roofline of the
dominant kernel (HIP-event timed on its launch stream) and the CPU oracle
timed on a bounded sample of the same pack.
"""
from __future__ import annotations

import argparse
import re
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "MSA fwd+bwd ms & select ms per 16k-token THD pack; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
D = 128

# Algorithmic (counted) work per unit, for the roofline of each kernel.  The
# counted fwd+bwd work is 14*D FLOP per (query head, selected causal key): the
# forward's S and PV, and the backward's S recompute, dP, dV, dK and dQ.  The
# backward runs in two passes that both need S and dP; the dK/dV pass is
# charged S, dP, dV and dK, the dQ pass only dQ, so the per-kernel figures sum
# to the counted total:
#   select_scores: 2*D FLOP per causal (query, key) pair per index head;
#   attn_fwd:      4*D FLOP per (query head, selected causal key)   [S, PV];
#   attn_bwd_dq:   2*D FLOP per (query head, selected causal key)   [dQ];
#   attn_bwd_dkdv: 8*D FLOP per (query head, selected causal key)   [S, dP, dV, dK].
FLOP_PER_KEY = {"attn_fwd": 4 * D, "attn_bwd_dq": 2 * D, "attn_bwd_dkdv": 8 * D}
# What the kernels execute.  With the stored dS (the default whenever its buffer
# fits) the dQ pass is one product, 14*D in all; when the dQ pass recomputes S
# and dP (MSA_ATTN_RECOMPUTE, or packs too large for the stored dS), 18*D.
EXEC_FLOP_PER_KEY = {"attn_fwd": 4 * D, "attn_bwd_dq": 2 * D, "attn_bwd_dkdv": 8 * D}
EXEC_FLOP_PER_KEY_RECOMPUTE = {"attn_fwd": 4 * D, "attn_bwd_dq": 6 * D, "attn_bwd_dkdv": 8 * D}


def selected_keys(blk: np.ndarray, cu: np.ndarray, block: int = 128) -> int:
    """Sum over (token, kv head) of the causal keys in the listed blocks (ids distinct per row)."""
    T = blk.shape[0]
    pos = np.empty(T, np.int64)
    for s in range(len(cu) - 1):
        pos[cu[s]:cu[s + 1]] = np.arange(cu[s + 1] - cu[s])
    b = pos // block
    valid = (blk >= 0) & (blk <= b[:, None, None])
    full = (blk < b[:, None, None]) & valid
    own = (blk == b[:, None, None])
    n = full.sum(axis=2) * block + own.sum(axis=2) * (pos % block + 1)[:, None]
    return int(n.sum())


def causal_pairs(lengths) -> int:
    return int(sum(L * (L + 1) // 2 for L in lengths))


CSRC = os.path.join(ROOT, "block_sparse_attention_select_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


# a C++ comment or string literal (strings kept as written, comments dropped)
_CPP_TOKEN = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'', re.S)


def code_text(src: str) -> str:
    """The source without its comments, whitespace runs outside string literals collapsed to one space."""
    out, code, pos = [], [], 0
    for m in _CPP_TOKEN.finditer(src):
        code.append(src[pos:m.start()])
        if m.group().startswith("/"):
            code.append(" ")
        else:
            out.append(re.sub(r"\s+", " ", "".join(code)))
            out.append(m.group())
            code = []
        pos = m.end()
    code.append(src[pos:])
    out.append(re.sub(r"\s+", " ", "".join(code)))
    return "".join(out).strip()


def kernel_source_hash() -> str:
    """Hash of the code of every HIP/C++ source of the library (comments and layout ignored): counters
    taken on other code are stale."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*"))):
        with open(f, encoding="utf-8") as fh:
            h.update(os.path.basename(f).encode())
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def traffic_file(config: str) -> str:
    return os.path.join(PROFILES, f"traffic_{config}.json")


# template flags of the library's kernel instances, in order; kernels not listed take (dense, qknorm)
KERNEL_FLAGS = {"block_prep_kernel": ("qknorm",), "bwd_block_prep_kernel": ("qknorm",),
                "qsa_prep_kernel": ("swizzled",)}
# instances named outright: the backward's stored-dS kernels carry the names of the library's timers (what
# the bench step runs); the sparse recompute instances (MSA_ATTN_RECOMPUTE, or packs too large for the
# stored dS) get a _recompute suffix
KERNEL_NAMES = {"attn_bwd_dkdv_kernel<false, true>": "attn_bwd_dkdv_kernel",
                "attn_bwd_dkdv_kernel<false, false>": "attn_bwd_dkdv_recompute_kernel",
                "attn_bwd_dkdv_kernel<true, false>": "attn_bwd_dkdv_dense_kernel",
                "attn_bwd_dq_ds_kernel": "attn_bwd_dq_kernel",
                "attn_bwd_dq_kernel<false, false>": "attn_bwd_dq_recompute_kernel",
                "qsa_dq_ds_kernel": "qsa_dq_kernel"}


def kernel_key(raw: str) -> str:
    """Library kernel name of a profiler record: `attn_fwd_kernel<false, true>(...)` -> `attn_fwd_qknorm_kernel`:
    each template flag that is set adds its name (KERNEL_FLAGS: `_dense` for the dense instances, `_qknorm`
    for the fused q/k norm ones, `_swizzled` for the narrow variant's dQ-stage copy); other kernels keep their
    name."""
    n = raw.replace("(anonymous namespace)::", "").split("(")[0].replace("msa::", "").strip()
    if n.startswith("void "):
        n = n[len("void "):]
    if n in KERNEL_NAMES:
        return KERNEL_NAMES[n]
    m = re.search(r"<([^<>]*)>$", n)
    flags = [a.strip() for a in m.group(1).split(",")] if m else []
    n = re.sub(r"<[^<>]*>$", "", n)
    names = KERNEL_FLAGS.get(n, ("dense", "qknorm"))
    suffix = "".join("_" + nm for nm, f in zip(names, flags) if f == "true")
    if suffix and n.endswith("_kernel"):
        n = n[:-len("_kernel")] + suffix + "_kernel"
    return n


def summarize_pmc(dirs, config: str, copy_mib: int) -> dict:
    """Per-kernel HBM bytes per dispatch from rocprofv3 --pmc CSVs (FETCH_SIZE and
    WRITE_SIZE, in KiB), each scaled by what the same counter reads for the plain
    copy of `copy_mib` MiB that --calibrate-copy runs."""
    acc = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] not in ("FETCH_SIZE", "WRITE_SIZE"):
                    continue
                name = kernel_key(r["Kernel_Name"])
                e = acc.setdefault(name, {}).setdefault(r["Counter_Name"], {})
                e[r["Dispatch_Id"]] = e.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    avg = {k: {c: sum(v.values()) / len(v) for c, v in d.items()} for k, d in acc.items()}
    # the calibration kernel: the library-external kernel that both read and
    # wrote the most (the streaming pass --calibrate-copy runs)
    copies = [d for k, d in avg.items() if not k.endswith("_kernel") and "FETCH_SIZE" in d and "WRITE_SIZE" in d]
    if not copies:
        raise SystemExit("no calibration kernel with FETCH_SIZE and WRITE_SIZE in the PMC runs (use --calibrate-copy)")
    cp = max(copies, key=lambda d: min(d["FETCH_SIZE"], d["WRITE_SIZE"]))
    nbytes = copy_mib * 2**20
    f_fetch = nbytes / (cp["FETCH_SIZE"] * 1024)
    f_write = nbytes / (cp["WRITE_SIZE"] * 1024)
    out = {"config": config, "source_hash": kernel_source_hash(), "copy_mib": copy_mib,
           "copy_factor_fetch": round(f_fetch, 4), "copy_factor_write": round(f_write, 4), "kernels": {}}
    for k, d in avg.items():
        if k.endswith("_kernel") and "FETCH_SIZE" in d and "WRITE_SIZE" in d:
            fb = d["FETCH_SIZE"] * 1024 * f_fetch
            wb = d["WRITE_SIZE"] * 1024 * f_write
            out["kernels"][k[:-len("_kernel")]] = {"fetch_bytes": int(fb), "write_bytes": int(wb),
                                                   "hbm_bytes": int(fb + wb)}
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def measured_peaks(dev) -> dict:
    """What this GPU reaches on two plain library kernels: a large bf16 GEMM
    (torch.matmul, hipBLASLt) and a streaming pass over 1 GiB (torch.neg: read
    n and write n bytes).  Reported beside the spec peaks, not instead of them."""
    n = 8192
    a = torch.randn(n, n, device=dev).bfloat16()
    b = torch.randn(n, n, device=dev).bfloat16()
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    gemm_tflops = 2 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    src = torch.zeros(2 ** 28, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    e0.record()
    for _ in range(reps):
        torch.neg(src, out=dst)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() * 4 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return {"bf16_gemm_tflops": round(gemm_tflops, 1), "bf16_gemm": f"torch.matmul {n}x{n}x{n}",
            "copy_gbs": round(copy_gbs, 1), "copy": "torch.neg over 1 GiB int32 (read + write)"}


def select_parity(p, blk_np) -> dict:
    """The GPU selection against the oracle's on every row: rows whose 16th/17th
    oracle scores are within 1e-3 relative are near ties; mismatches are counted
    inside and outside them."""
    import oracle as O
    f = lambda t: t.float().numpy()
    res = O.index_select(f(p.idx_q), f(p.idx_k), f(p.w_q), f(p.w_k), p.cu_seqlens.numpy())
    diff = (blk_np != res.blk_idx).any(axis=2)
    tie = res.near_tie(1e-3)
    return {"rows": int(diff.size), "near_tie_rows": int(tie.sum()),
            "mismatch_in_near_ties": int((diff & tie).sum()), "mismatch_outside": int((diff & ~tie).sum())}, res


def cpu_baseline(p, stride: int):
    """The oracle as it stands, on this host: select on the whole pack, fwd+bwd on
    every `stride`-th token, scaled to the full pack."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    f = lambda t: t.float().numpy()
    cu = p.cu_seqlens.numpy()
    t0 = time.perf_counter()
    res = O.index_select(f(p.idx_q), f(p.idx_k), f(p.w_q), f(p.w_k), cu)
    t_sel = time.perf_counter() - t0
    rows = np.arange(0, p.total, stride)
    q, k, v, do = f(p.q), f(p.k), f(p.v), f(p.do)
    t0 = time.perf_counter()
    O.attention_forward(q, k, v, res.blk_idx, cu, p.softmax_scale, rows=rows)
    O.attention_backward(q, k, v, do, res.blk_idx, cu, p.softmax_scale, rows=rows)
    t_att = time.perf_counter() - t0
    est_ms = (t_sel + t_att * p.total / len(rows)) * 1e3
    return {"value": round(est_ms, 1), "unit": "ms", "cores": int(threads), "kind": "oracle",
            "sample": f"select on all {p.total} tokens ({t_sel:.1f} s); fwd+bwd on every {stride}th token "
                      f"({len(rows)} rows, {t_att:.1f} s) scaled x{p.total / len(rows):.0f}",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def seed_leg(msa, config: str, seed: int, steps: int, warmup: int) -> dict:
    """The bench step (select -> forward on its ids -> backward) on another seed's pack of the same config:
    wall time per step, the select / forward / backward split from events between the calls, and the counted
    fwd+bwd rate."""
    p = synth.make_pack(config, seed)
    dev = torch.device("cuda:0")
    g = lambda t: t.to(dev)
    cu = g(p.cu_seqlens)
    q, k, v, do = g(p.q), g(p.k), g(p.v), g(p.do)
    iq, ik, wq, wk = g(p.idx_q), g(p.idx_k), g(p.w_q), g(p.w_k)
    T, Hq, Hk = p.total, p.num_q_heads, p.num_kv_heads
    dims = msa.make_dims(T, len(p.lengths), p.max_seqlen, Hq, Hk)
    ws = {op: torch.empty(max(msa.msa_workspace_size(dims, op), 1), dtype=torch.uint8, device=dev)
          for op in (msa.MSA_OP_SELECT, msa.MSA_OP_FWD, msa.MSA_OP_BWD)}
    blk = torch.empty(T, Hk, 16, dtype=torch.int32, device=dev)
    o, lse = torch.empty_like(q), torch.empty(T, Hq, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        msa.msa_index_select(iq, ik, wq, wk, cu, p.max_seqlen, out=blk, workspace=ws[msa.MSA_OP_SELECT])
        if ev is not None:
            ev[1].record()
        msa.msa_attn_fwd(q, k, v, blk, cu, p.max_seqlen, out=o, lse=lse, workspace=ws[msa.MSA_OP_FWD])
        if ev is not None:
            ev[2].record()
        msa.msa_attn_bwd(q, k, v, o, lse, do, blk, cu, p.max_seqlen, dq=dq, dk=dk, dv=dv,
                         workspace=ws[msa.MSA_OP_BWD])
        if ev is not None:
            ev[3].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    split = [float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i in range(3)]
    per_qhead = selected_keys(blk.cpu().numpy(), p.cu_seqlens.numpy()) * (Hq // Hk)
    fb_ms = split[1] + split[2]
    return {"seed": seed, "lengths": p.lengths, "step_ms": round(wall_ms, 4), "select_ms": round(split[0], 4),
            "fwd_ms": round(split[1], 4), "bwd_ms": round(split[2], 4), "fwd_bwd_ms": round(fb_ms, 4),
            "fwd_bwd_mfma_frac": round(14 * D * per_qhead / (fb_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def qsa_leg(msa, seed: int, steps: int, warmup: int) -> dict:
    """Narrow-block variant (msa_qsa_attn_*) on the qsa16k pack: 12 q / 1 kv heads, D 256,
    4-token blocks, 512 seeded block ids per query (synth.random_block_lists)."""
    p = synth.make_pack("qsa16k", seed)
    dev = torch.device("cuda:0")
    g = lambda t: t.to(dev)
    cu_np = p.cu_seqlens.numpy()
    blk_np = synth.random_block_lists(cu_np, p.num_kv_heads, 4, p.topk_blocks, seed)
    cu, q, k, v, do = g(p.cu_seqlens), g(p.q), g(p.k), g(p.v), g(p.do)
    blk = g(torch.from_numpy(blk_np))
    T, Hq, Hk, Dn = p.total, p.num_q_heads, p.num_kv_heads, p.head_dim
    dims = msa.make_dims(T, len(p.lengths), p.max_seqlen, Hq, Hk, head_dim=Dn, block_size=4,
                         topk_blocks=p.topk_blocks)
    ws = {op: torch.empty(max(msa.msa_workspace_size(dims, op), 1), dtype=torch.uint8, device=dev)
          for op in (msa.MSA_OP_QSA_FWD, msa.MSA_OP_QSA_BWD)}
    o, lse = torch.empty_like(q), torch.empty(T, Hq, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        msa.msa_qsa_attn_fwd(q, k, v, blk, cu, p.max_seqlen, out=o, lse=lse, workspace=ws[msa.MSA_OP_QSA_FWD])
        if ev is not None:
            ev[1].record()
        msa.msa_qsa_attn_bwd(q, k, v, o, lse, do, blk, cu, p.max_seqlen, dq=dq, dk=dk, dv=dv,
                             workspace=ws[msa.MSA_OP_QSA_BWD])
        if ev is not None:
            ev[2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    msa.msa_timing_collect()
    msa.msa_timing_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kt = msa.msa_timing_collect()
    msa.msa_timing_enable(False)
    per_qhead = selected_keys(blk_np, cu_np, 4) * (Hq // Hk)
    fb_flop = 14 * Dn * per_qhead
    fb_ms = fwd_ms + bwd_ms
    tflops = fb_flop / (fb_ms * 1e-3) / 1e12
    return {
        "workload": f"qsa16k: {T}-token THD pack, seed {seed}, lengths {p.lengths}, {Hq} q / {Hk} kv heads, "
                    f"D {Dn}, 4-token blocks, {p.topk_blocks} listed per query (seeded)",
        "fwd_ms": round(fwd_ms, 4),
        "bwd_ms": round(bwd_ms, 4),
        "fwd_bwd_ms": round(fb_ms, 4),
        "fwd_bwd_counted_gflop": round(fb_flop / 1e9, 1),
        "fwd_bwd_tflops": round(tflops, 2),
        "fwd_bwd_mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "kernels_avg_ms": {name: round(ms / n, 4) for name, (n, ms) in kt.items()},
        "context_gb300_ms": {"fwd_bwd": 16.4, "note": "pages' GB300 figure for qwen3.8-next on unpublished 16k packs"},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)  # the clocks settle over the first tens of steps
    ap.add_argument("--config", default="pack16k", choices=sorted(c for c in synth.CONFIGS if c != "qsa16k"))
    ap.add_argument("--no-qsa", action="store_true", help="skip the narrow-block (qsa16k) leg")
    ap.add_argument("--no-seeds", action="store_true", help="skip the step timing on the other two seeds' packs")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-stride", type=int, default=3, help="oracle fwd+bwd sample: every n-th token")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle (timing and selection parity)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured GEMM and copy peaks")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="after timing, copy MIB MiB device-to-device (a PMC calibration kernel)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR",
                    help="write profiles/traffic_<config>.json from rocprofv3 --pmc output dirs and exit")
    ap.add_argument("--copy-mib", type=int, default=1024, help="size of the calibration copy in those runs")
    args = ap.parse_args()

    if args.summarize_pmc:
        out = summarize_pmc(args.summarize_pmc, args.config, args.copy_mib)
        os.makedirs(PROFILES, exist_ok=True)
        with open(traffic_file(args.config), "w") as f:
            json.dump(out, f, indent=1)
        print(json.dumps(out))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the MSA path shards by KV head with no exchange step, "
              "so only --gpus 1 is run here", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        sys.exit(2)

    import block_sparse_attention_select_amd as msa
    msa.load()

    p = synth.make_pack(args.config, args.seed)
    dev = torch.device("cuda:0")
    g = lambda t: t.to(dev)
    cu = g(p.cu_seqlens)
    q, k, v, do = g(p.q), g(p.k), g(p.v), g(p.do)
    iq, ik, wq, wk = g(p.idx_q), g(p.idx_k), g(p.w_q), g(p.w_k)
    T, Hq, Hk = p.total, p.num_q_heads, p.num_kv_heads
    dims = msa.make_dims(T, len(p.lengths), p.max_seqlen, Hq, Hk)
    ws = {op: torch.empty(max(msa.msa_workspace_size(dims, op), 1), dtype=torch.uint8, device=dev)
          for op in (msa.MSA_OP_SELECT, msa.MSA_OP_FWD, msa.MSA_OP_BWD)}
    blk = torch.empty(T, Hk, 16, dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty(T, Hq, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        msa.msa_index_select(iq, ik, wq, wk, cu, p.max_seqlen, out=blk, workspace=ws[msa.MSA_OP_SELECT])
        if ev is not None:
            ev[1].record()
        msa.msa_attn_fwd(q, k, v, blk, cu, p.max_seqlen, out=o, lse=lse, workspace=ws[msa.MSA_OP_FWD])
        if ev is not None:
            ev[2].record()
        msa.msa_attn_bwd(q, k, v, o, lse, do, blk, cu, p.max_seqlen, dq=dq, dk=dk, dv=dv,
                         workspace=ws[msa.MSA_OP_BWD])
        if ev is not None:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the timed steps carry no events (event records between the calls add
    # time of their own); the select / fwd / bwd split is taken in a separate
    # pass of the same steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    sel_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    fwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    bwd_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))

    # the forced-initial-block selection variant on the same pack (not part of the step)
    blk_init = torch.empty_like(blk)
    ei = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for _ in range(2):
        msa.msa_index_select(iq, ik, wq, wk, cu, p.max_seqlen, force_init=True, out=blk_init,
                             workspace=ws[msa.MSA_OP_SELECT])
    ei[0].record()
    for _ in range(args.steps):
        msa.msa_index_select(iq, ik, wq, wk, cu, p.max_seqlen, force_init=True, out=blk_init,
                             workspace=ws[msa.MSA_OP_SELECT])
    ei[1].record()
    torch.cuda.synchronize()
    sel_init_ms = ei[0].elapsed_time(ei[1]) / args.steps

    # attention-side q/k norm + partial RoPE, forward and backward, on this pack (not part of the step)
    gw = torch.Generator().manual_seed(args.seed + 77)
    wq_a = (0.1 * torch.randn(128, generator=gw)).bfloat16().to(dev)
    wk_a = (0.1 * torch.randn(128, generator=gw)).bfloat16().to(dev)
    qh, kh = torch.empty_like(q), torch.empty_like(k)
    ws_qk = torch.empty(max(msa.msa_workspace_size(dims, msa.MSA_OP_QKNORM_BWD), 1), dtype=torch.uint8, device=dev)
    qk_fwd = lambda: msa.msa_qk_norm_rope_fwd(q, k, wq_a, wk_a, cu, p.max_seqlen, q_out=qh, k_out=kh)
    qk_bwd = lambda: msa.msa_qk_norm_rope_bwd(q, k, wq_a, wk_a, cu, p.max_seqlen, dq, dk, workspace=ws_qk)
    # the attention with that norm fused in (msa_attn_fwd_qknorm / _bwd_qknorm) on the raw q, k, against the
    # separate passes (norm forward + attention forward; attention backward + norm backward)
    ws_fq = torch.empty(max(msa.msa_workspace_size(dims, msa.MSA_OP_BWD_QKNORM), 1), dtype=torch.uint8, device=dev)
    fo, flse = torch.empty_like(q), torch.empty_like(lse)
    fused_fwd = lambda: msa.msa_attn_fwd_qknorm(q, k, v, wq_a, wk_a, blk, cu, p.max_seqlen, out=fo, lse=flse,
                                                workspace=ws[msa.MSA_OP_FWD])
    fused_bwd = lambda: msa.msa_attn_bwd_qknorm(q, k, v, wq_a, wk_a, fo, flse, do, blk, cu, p.max_seqlen,
                                                workspace=ws_fq)

    def sep_fwd():
        qk_fwd()
        msa.msa_attn_fwd(qh, kh, v, blk, cu, p.max_seqlen, out=fo, lse=flse, workspace=ws[msa.MSA_OP_FWD])
    # the low-memory backward (MSA_ATTN_RECOMPUTE: dQ recomputes S and dP, no stored dS) on the step's inputs
    rdq, rdk, rdv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    rc_bwd = lambda: msa.msa_attn_bwd(q, k, v, o, lse, do, blk, cu, p.max_seqlen, dq=rdq, dk=rdk, dv=rdv,
                                      workspace=ws[msa.MSA_OP_BWD], recompute=True)
    qk_ms = {}
    for name, fn in (("fwd", qk_fwd), ("bwd", qk_bwd), ("fused_fwd", fused_fwd), ("fused_bwd", fused_bwd),
                     ("sep_fwd", sep_fwd), ("recompute_bwd", rc_bwd)):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        qk_ms[name] = e0.elapsed_time(e1) / args.steps
    qk_elems = q.numel() + k.numel()
    qk_bytes = {"fwd": 2 * qk_elems * 2, "bwd": 3 * qk_elems * 2}  # bf16 in + out (bwd: x and dz in, dx out)

    # per-kernel durations: HIP event pairs recorded by the library on the launch stream
    msa.msa_timing_collect()
    msa.msa_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = msa.msa_timing_collect()
    msa.msa_timing_enable(False)
    kernels = {name: round(ms / n, 4) for name, (n, ms) in kt.items()}

    # counted work
    blk_np = blk.cpu().numpy()
    cu_np = p.cu_seqlens.numpy()
    nkeys = selected_keys(blk_np, cu_np)              # (token, kv head, key) triples
    per_qhead = nkeys * (Hq // Hk)                    # (token, q head, key)
    fwd_flop = 4 * D * per_qhead
    fb_flop = 14 * D * per_qhead
    sel_flop = 2 * D * causal_pairs(p.lengths) * Hk
    sel_bytes = 2 * T * Hk * D * 2 + T * Hk * 16 * 4
    fb_ms = fwd_ms + bwd_ms
    fb_tflops = fb_flop / (fb_ms * 1e-3) / 1e12

    # the backward stores dS (and its dQ pass executes one product) when its workspace carries the dS tail
    stored_ds = msa.msa_workspace_size(dims, msa.MSA_OP_BWD) > msa.msa_workspace_size(dims, msa.MSA_OP_BWD_RECOMPUTE)
    exec_fpk = EXEC_FLOP_PER_KEY if stored_ds else EXEC_FLOP_PER_KEY_RECOMPUTE
    dom = max(kt.items(), key=lambda kv: kv[1][1])[0]
    dom_ms = kt[dom][1] / kt[dom][0]
    dom_exec = None
    if dom in FLOP_PER_KEY:
        dom_flop = FLOP_PER_KEY[dom] * per_qhead
        dom_exec = exec_fpk[dom] * per_qhead
    elif dom == "select_scores":
        dom_flop = sel_flop
    else:
        dom_flop = None
    traffic = None
    tf = traffic_file(args.config)
    if os.path.exists(tf):
        rec = json.load(open(tf))
        if rec.get("source_hash") == kernel_source_hash() and dom in rec.get("kernels", {}):
            traffic = rec["kernels"][dom]["hbm_bytes"]
    roofline = None
    if dom_flop is not None:
        ach = dom_flop / (dom_ms * 1e-3) / 1e12
        roofline = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                    "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                    "avg_launch_ms": round(dom_ms, 4), "algorithmic_flop_per_launch": int(dom_flop)}
        if dom_exec is not None:
            roofline["executed_flop_per_launch"] = int(dom_exec)
            roofline["executed_tflops"] = round(dom_exec / (dom_ms * 1e-3) / 1e12, 2)
        if dom == "attn_bwd_dkdv":
            # what the pass must move once: q and dO of every (token, q head), K and V, the per-row
            # -LSE log2(e) and Delta ([T][Hk][16] fp32) and the block lists in; dK and dV (bf16) out,
            # and with the stored dS its bf16 dS, 2 B per (query head, selected causal key)
            alg = (2 * T * Hq * D * 2 + 2 * T * Hk * D * 2 + 3 * T * Hk * 16 * 4 + 2 * T * Hk * D * 2
                   + (2 * per_qhead if stored_ds else 0))
            roofline["algorithmic_bytes_per_launch"] = int(alg)
            if traffic is not None:
                roofline["traffic_over_algorithmic"] = round(traffic / alg, 2)
    per_kernel = {}
    for name, fpk in FLOP_PER_KEY.items():
        if name in kt:
            ms = kt[name][1] / kt[name][0]
            per_kernel[name] = {"ms": round(ms, 4),
                                "counted_tflops": round(fpk * per_qhead / (ms * 1e-3) / 1e12, 1),
                                "executed_tflops": round(exec_fpk[name] * per_qhead / (ms * 1e-3) / 1e12, 1)}

    line = {
        "metric": METRIC,
        "value": round(wall_ms, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: {p.total}-token THD pack, seed {args.seed}, lengths {p.lengths}, "
                               f"{Hq} q / {Hk} kv / {Hk} index heads, D 128, block 128, top-16",
                   "seq_lens": p.lengths, "num_q_heads": Hq, "num_kv_heads": Hk, "head_dim": D,
                   "block_size": 128, "topk_blocks": 16, "parallelism": "none (1 GPU)"},
        "select_ms": round(sel_ms, 4),
        "select_force_init_ms": round(sel_init_ms, 4),
        "qk_norm_rope_fwd_ms": round(qk_ms["fwd"], 4),
        "qk_norm_rope_bwd_ms": round(qk_ms["bwd"], 4),
        "qk_norm_rope_fwd_hbm_frac": round(qk_bytes["fwd"] / (qk_ms["fwd"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "attn_qknorm_fused_fwd_ms": round(qk_ms["fused_fwd"], 4),
        "attn_qknorm_separate_fwd_ms": round(qk_ms["sep_fwd"], 4),
        "attn_qknorm_fused_bwd_ms": round(qk_ms["fused_bwd"], 4),
        "qk_norm_rope_bwd_hbm_frac": round(qk_bytes["bwd"] / (qk_ms["bwd"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "fwd_ms": round(fwd_ms, 4),
        "bwd_ms": round(bwd_ms, 4),
        "bwd_recompute_ms": round(qk_ms["recompute_bwd"], 4),
        "bwd_workspace_mb": round(msa.msa_workspace_size(dims, msa.MSA_OP_BWD) / 2**20, 1),
        "bwd_recompute_workspace_mb": round(msa.msa_workspace_size(dims, msa.MSA_OP_BWD_RECOMPUTE) / 2**20, 1),
        "fwd_bwd_ms": round(fb_ms, 4),
        "fwd_bwd_counted_gflop": round(fb_flop / 1e9, 1),
        "fwd_bwd_tflops": round(fb_tflops, 2),
        "fwd_bwd_mfma_frac": round(fb_tflops / PEAK_BF16_TFLOPS, 4),
        "fwd_tflops": round(fwd_flop / (fwd_ms * 1e-3) / 1e12, 2),
        "select_gflop": round(sel_flop / 1e9, 2),
        "select_algorithmic_mb": round(sel_bytes / 1e6, 2),
        "select_hbm_gbs": round(sel_bytes / (sel_ms * 1e-3) / 1e9, 1),
        "select_hbm_frac": round(sel_bytes / (sel_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "select_binding_frac": round(max(sel_bytes / (PEAK_HBM_GBS * 1e9), sel_flop / (PEAK_BF16_TFLOPS * 1e12))
                                     / (sel_ms * 1e-3), 4),
        "kernels_avg_ms": kernels,
        "kernel_rates": per_kernel,
        "fwd_bwd_executed_tflops": round(sum(exec_fpk.values()) * per_qhead / (fb_ms * 1e-3) / 1e12, 2),
        "bwd_stored_ds": bool(stored_ds),
        "roofline": roofline,
        "context_gb300_ms": {"fwd_bwd": 6.7, "select": 0.62, "note": "pages' GB300 figures on unpublished 16k packs"},
    }
    if not args.no_seeds:
        # the same config's packs for two more seeds (other lengths and data): the step time per seed and the
        # mean over the three
        legs = [{"seed": args.seed, "lengths": p.lengths, "step_ms": round(wall_ms, 4), "select_ms": round(sel_ms, 4),
                 "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4), "fwd_bwd_ms": round(fb_ms, 4),
                 "fwd_bwd_mfma_frac": round(fb_tflops / PEAK_BF16_TFLOPS, 4)}]
        for sd in (args.seed + 1, args.seed + 2):
            legs.append(seed_leg(msa, args.config, sd, max(10, args.steps // 2), min(args.warmup, 20)))
        line["seeds"] = {"per_seed": legs,
                         "mean_step_ms": round(float(np.mean([x["step_ms"] for x in legs])), 4),
                         "mean_fwd_bwd_ms": round(float(np.mean([x["fwd_bwd_ms"] for x in legs])), 4),
                         "mean_fwd_bwd_mfma_frac": round(float(np.mean([x["fwd_bwd_mfma_frac"] for x in legs])), 4)}
    if not args.no_qsa:
        line["qsa16k"] = qsa_leg(msa, args.seed, args.steps, args.warmup)
    if args.calibrate_copy > 0:
        # a plain streaming kernel of known traffic (read n, write n bytes); a
        # tensor copy would go to the DMA engines and leave no kernel to count
        src = torch.zeros(args.calibrate_copy * 2**20 // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_peaks:
        pk = measured_peaks(dev)
        pk["fwd_bwd_frac_of_gemm"] = round(fb_tflops / pk["bf16_gemm_tflops"], 4)
        line["measured_peaks"] = pk
    if not args.no_cpu_baseline:
        line["select_parity"], _ = select_parity(p, blk_np)
        line["cpu_baseline"] = cpu_baseline(p, args.cpu_stride)
    else:
        line["select_parity"] = None
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
