"""Write SHA-256 digests of the oracle's full selections and tile unions at the measured sizes.

    python tests/golden/make_selection_digests.py [workload ...]

The GPU tests check the library's selections and unions on EVERY row of these workloads by
hashing its outputs chunk by chunk and comparing against the digests stored here. This script
calls only ``datagen`` (the seeded indexer inputs, drawn on the CPU, so they are the same on every
machine) and ``oracle`` (compress -> per-row top-k -> union); nothing here touches the HIP library.

Digest layout (one JSON file per workload, ``selection_<workload>.json``):
  inputs_sha256   sha256 of the raw bytes of qi, ki (bf16 bits) and w (fp32)
  kbar_sha256     sha256 of the oracle's block keys [N//B][dI] (bf16 bits)
  topk_sha256     [G][n_chunks] first 16 hex digits of sha256 of topk[g, r0:r0+rows_per_chunk]
                  (int32, ascending ids, -1 padding)
  umask_sha256    [G] sha256 of umask[g] [T][W] (uint32), only for workloads with a union
  ucount_sha256   [G] sha256 of ucount[g] [T] (int32)
"""
from __future__ import annotations

import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import datagen  # noqa: E402
import oracle  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
ROWS_PER_CHUNK = 4096

# Workloads whose selections are digested, and whether their tile union is too.
DIGESTED = {
    "prefill_32k": True,
    "prefill_32k_iid": True,
    "long_prefill_128k": True,
    "ablation_32k_b1_k2048": False,
}


def sha(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def input_digests(x: dict) -> dict:
    return {"qi": sha(bits(x["qi"])), "ki": sha(bits(x["ki"])), "w": sha(x["w"].numpy().astype(np.float32))}


def path_of(name: str) -> str:
    return os.path.join(HERE, f"selection_{name}.json")


def make(name: str) -> dict:
    wl = datagen.WORKLOADS[name]
    t0 = time.time()
    x = datagen.index_inputs(wl)
    qi, ki, w = bits(x["qi"]), bits(x["ki"]), x["w"].numpy().astype(np.float32)
    kbar = oracle.compress(ki, wl.block)
    N, G, kb = wl.n_tokens, wl.n_kv_heads, wl.kb
    topk = np.empty((G, N, kb), dtype=np.int32)
    for r0 in range(0, N, ROWS_PER_CHUNK):
        rows = np.arange(r0, min(N, r0 + ROWS_PER_CHUNK), dtype=np.int32)
        topk[:, rows] = oracle.index_topk(qi, w, kbar, wl.block, kb, rows=rows)
        print(f"[{name}] rows {r0}..{rows[-1]} done at {time.time() - t0:.0f}s", flush=True)
    d = {
        "workload": name,
        "generated_by": "tests/golden/make_selection_digests.py (datagen indexer inputs + oracle only)",
        "n_tokens": N, "n_kv_heads": G, "block": wl.block, "topk_tokens": wl.topk_tokens,
        "union_tile": wl.union_tile,
        "inputs_sha256": input_digests(x),
        "kbar_sha256": sha(kbar),
        "rows_per_chunk": ROWS_PER_CHUNK,
        "topk_sha256": [[sha(topk[g, r0:r0 + ROWS_PER_CHUNK])[:16] for r0 in range(0, N, ROWS_PER_CHUNK)]
                        for g in range(G)],
    }
    if DIGESTED[name]:
        umask, ucount = oracle.union(topk, N, wl.block, wl.union_tile)
        d["umask_sha256"] = [sha(umask[g]) for g in range(G)]
        d["ucount_sha256"] = [sha(ucount[g]) for g in range(G)]
        d["mean_union_blocks"] = float(ucount.mean())
    d["oracle_seconds"] = round(time.time() - t0, 1)
    return d


def main(names) -> None:
    for name in names:
        d = make(name)
        with open(path_of(name), "w") as f:
            json.dump(d, f, indent=1)
            f.write("\n")
        print(f"[{name}] wrote {path_of(name)}", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or list(DIGESTED))
