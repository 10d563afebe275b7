"""Builds the planted-selection inputs described in tests/golden/planted_select.json.

Only input construction lives here (no arithmetic of the method): both the
oracle pins and the GPU parity tests consume the same tensors.
"""
import json
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "planted_select.json")


def load_planted():
    with open(GOLDEN) as f:
        spec = json.load(f)
    B = spec["block_size"]
    D = spec["head_dim"]
    lengths = [s["length"] for s in spec["sequences"]]
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    idx_q = torch.zeros(T, 1, D, dtype=torch.float32)
    idx_k = torch.zeros(T, 1, D, dtype=torch.float32)
    idx_q[:, 0, 64] = 1.0
    idx_k[:, 0, 64] = spec["background_x"]
    idx_k[:, 0, 65] = 1.0
    for s, seq in enumerate(spec["sequences"]):
        for c, x in enumerate(seq["peak_x"]):
            if x is None:
                continue
            p = c * B + spec["peak_offset"]
            assert p < seq["length"]
            idx_k[int(cu[s]) + p, 0, 64] = x
    w = torch.zeros(D, dtype=torch.float32)
    def cases(key):
        out = []
        for e in spec[key]:
            t = int(cu[e["seq"]]) + e["pos"]
            ids = list(e["ids"]) + [-1] * (spec["topk"] - len(e["ids"]))
            out.append((t, ids, e["why"]))
        return out
    return dict(idx_q=idx_q.to(torch.bfloat16), idx_k=idx_k.to(torch.bfloat16),
                w_q=w.to(torch.bfloat16), w_k=w.to(torch.bfloat16), cu_seqlens=cu,
                lengths=lengths, block=B, topk=spec["topk"], expected=cases("expected"),
                expected_force_init=cases("expected_force_init"))
