"""GPU parity at the measured sizes, in the launch configuration bench.py times.

Selections and unions are checked on EVERY row and tile: the library's outputs are hashed chunk by
chunk and compared with digests of the oracle's full selections (``tests/golden/selection_*.json``,
written by ``tests/golden/make_selection_digests.py`` from the same CPU-drawn indexer inputs and
the oracle only). On a mismatch the oracle is run on the failing chunk to name the first wrong row.
Attention is checked on sampled query rows (the oracle cannot finish the whole workload), decode on
all 32 sequences, and every output against properties that hold at any size.
"""
import hashlib
import json
import os

import numpy as np
import pytest
import torch

import datagen
import oracle
from tests.gpu_common import OracleChain, assert_close_attention, bits, params_of, say

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def sg():
    import block_sparse_long_sgqa_amd as sg

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sg.lib()
    return sg


def sha(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def load_digests(name: str) -> dict:
    with open(os.path.join(GOLDEN, f"selection_{name}.json")) as f:
        return json.load(f)


def check_inputs(d: dict, x: dict) -> None:
    """The indexer inputs are the ones the digests were made from (CPU draws are portable)."""
    got = {"qi": sha(bits(x["qi"])), "ki": sha(bits(x["ki"])),
           "w": sha(x["w"].cpu().numpy().astype(np.float32))}
    assert got == d["inputs_sha256"], f"indexer inputs differ from the digested ones: {got}"


def check_topk_digests(d: dict, topk: np.ndarray, ch: OracleChain) -> None:
    """Every row of topk [G][N][KB] against the oracle's digests; localise a mismatch with the oracle."""
    rpc = d["rows_per_chunk"]
    G, N, _ = topk.shape
    bad = [(g, c) for g in range(G) for c, r0 in enumerate(range(0, N, rpc))
           if sha(topk[g, r0:r0 + rpc])[:16] != d["topk_sha256"][g][c]]
    if not bad:
        say(f"{d['workload']}: all {G * N} selections match the oracle")
        return
    g, c = bad[0]
    r0 = c * rpc
    rows = np.arange(r0, min(N, r0 + rpc), dtype=np.int32)
    say(f"{d['workload']}: {len(bad)} (group, chunk) digests differ; oracle on group {g} rows {r0}..{rows[-1]}")
    want = ch.topk(rows)[g]
    diff = np.nonzero((want != topk[g, rows]).any(axis=1))[0]
    i = int(rows[diff[0]]) if len(diff) else -1
    raise AssertionError(f"{d['workload']}: selection differs from the oracle in {len(bad)} chunks; "
                         f"first: group {g} row {i}")


def check_union_digests(d: dict, umask: np.ndarray, ucount: np.ndarray, what: str) -> None:
    G = umask.shape[0]
    for g in range(G):
        assert sha(umask[g]) == d["umask_sha256"][g], f"{what}: union mask of group {g} differs from the oracle"
        assert sha(ucount[g]) == d["ucount_sha256"][g], f"{what}: union count of group {g} differs from the oracle"
    say(f"{what}: all {G * umask.shape[1]} tile unions match the oracle")


def run_prefill_full(sg, wl, tiles_sample, attn_rows_per_tile):
    p = params_of(wl)
    d = load_digests(wl.name)
    say(f"full-size {wl.name}: drawing inputs (indexer inputs on the CPU)")
    x = datagen.prefill_inputs(wl, device="cuda")
    host = {k: x[k].cpu() for k in ("qi", "ki", "w")}
    check_inputs(d, host)
    o = sg.alloc_prefill_outputs(p)
    say(f"full-size {wl.name}: compress/index_topk/union/attend")
    sg.sgqa_compress(p, x["ki"], o["blk_k"])
    sg.sgqa_index_topk(p, x["qi"], x["w"], o["blk_k"], o["topk"])
    sg.sgqa_union(p, o["topk"], o["umask"], o["ucount"])
    sg.sgqa_attend(p, x["q"], x["k"], x["v"], o["umask"], o["ucount"], o["out"])
    torch.cuda.synchronize()
    say(f"full-size {wl.name}: fused index_union")
    fm = torch.empty_like(o["umask"])
    fc = torch.empty_like(o["ucount"])
    sg.sgqa_index_union(p, x["qi"], x["w"], o["blk_k"], fm, fc)
    say(f"full-size {wl.name}: sgqa_prefill")
    out2 = torch.empty_like(o["out"])
    ws = sg.workspace(p, sg.SGQA_OP_PREFILL)
    sg.sgqa_prefill(p, x["q"], x["k"], x["v"], x["qi"], x["w"], x["ki"], out2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), o["out"].view(torch.int16)), "prefill != single calls"
    del ws, out2

    ch = OracleChain(host, p)
    assert sha(bits(o["blk_k"])) == d["kbar_sha256"], "block keys differ from the oracle"
    np.testing.assert_array_equal(bits(o["blk_k"]), ch.kbar)

    say(f"full-size {wl.name}: hashing every selection row")
    topk = o["topk"].cpu().numpy()
    check_topk_digests(d, topk, ch)
    del topk
    umask = o["umask"].cpu().numpy().view(np.uint32)
    ucount = o["ucount"].cpu().numpy()
    check_union_digests(d, umask, ucount, f"{wl.name} union")
    check_union_digests(d, fm.cpu().numpy().view(np.uint32), fc.cpu().numpy(), f"{wl.name} fused index_union")

    rng = np.random.default_rng(7)
    tiles = np.unique(np.concatenate([[0, p.n_tiles - 1], rng.integers(0, p.n_tiles, tiles_sample)]))
    say(f"full-size {wl.name}: oracle union and attention on tiles {tiles.tolist()}")
    om, oc, _, _ = ch.union_of_tiles(tiles)
    np.testing.assert_array_equal(umask[:, tiles], om[:, tiles])
    np.testing.assert_array_equal(ucount[:, tiles], oc[:, tiles])
    arows = np.concatenate([rng.choice(ch.tile_rows(int(t)), size=min(attn_rows_per_tile, len(ch.tile_rows(int(t)))),
                                       replace=False) for t in tiles]).astype(np.int32)
    want = oracle.attend(bits(x["q"]), bits(x["k"]), bits(x["v"]), om, p.block, p.union_tile, rows=arows)
    got = o["out"][torch.from_numpy(arows).long().cuda()]
    assert_close_attention(got, want, f"{wl.name} attention")
    assert torch.isfinite(o["out"].float()).all()


def test_prefill_32k_full_size(sg):
    run_prefill_full(sg, datagen.PREFILL, tiles_sample=3, attn_rows_per_tile=8)


def test_long_prefill_128k_full_size(sg):
    run_prefill_full(sg, datagen.LONG_PREFILL, tiles_sample=2, attn_rows_per_tile=4)


def test_prefill_32k_iid_stress(sg):
    run_prefill_full(sg, datagen.PREFILL_IID, tiles_sample=2, attn_rows_per_tile=4)


def test_ablation_block1_k2048_selection(sg):
    wl = datagen.ABLATION_B1
    p = params_of(wl)
    d = load_digests(wl.name)
    say("ablation B=1 k=2048 at 32k: drawing inputs")
    x = datagen.prefill_inputs(wl, device="cuda")
    host = {k: x[k].cpu() for k in ("qi", "ki", "w")}
    check_inputs(d, host)
    blk = torch.empty((p.n_tokens, 64), dtype=torch.bfloat16, device="cuda")
    topk = torch.empty((p.n_kv_heads, p.n_tokens, p.kb), dtype=torch.int32, device="cuda")
    sg.sgqa_compress(p, x["ki"], blk)
    sg.sgqa_index_topk(p, x["qi"], x["w"], blk, topk)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(blk), bits(x["ki"]))  # B = 1: block keys are the keys
    assert sha(bits(blk)) == d["kbar_sha256"]
    say("ablation B=1: hashing every selection row")
    check_topk_digests(d, topk.cpu().numpy(), OracleChain(host, p))


def test_decode_256k_full_size(sg):
    """All 32 sequences: block keys, selection and output against the oracle."""
    wl = datagen.DECODE
    p = params_of(wl)
    say("decode 32 x 262144: drawing caches on the GPU")
    y = datagen.decode_inputs(wl, device="cuda")
    blk = torch.empty((p.n_seqs, p.n_tokens // p.block, 64), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((p.n_seqs, p.n_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    topk = torch.empty((p.n_seqs, p.n_kv_heads, p.kb), dtype=torch.int32, device="cuda")
    ws = sg.workspace(p, sg.SGQA_OP_DECODE)
    say("decode 32 x 262144: compress + decode")
    sg.sgqa_compress(p, y["ki_cache"], blk)
    sg.sgqa_decode(p, y["q"], y["k_cache"], y["v_cache"], blk, y["qi"], y["w"], out, ws, topk_out=topk)
    torch.cuda.synchronize()
    out2 = torch.empty_like(out)
    sg.sgqa_decode(p, y["q"], y["k_cache"], y["v_cache"], blk, y["qi"], y["w"], out2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), "decode is not deterministic"
    t = topk.cpu().numpy()
    for s in range(p.n_seqs):
        sl = slice(s, s + 1)
        kbar = oracle.compress(bits(y["ki_cache"][sl]), p.block)
        np.testing.assert_array_equal(bits(blk[sl]), kbar)
        sel, want = oracle.decode(y["q"][sl], y["k_cache"][sl], y["v_cache"][sl], kbar, y["qi"][sl], y["w"],
                                  p.block, p.kb)
        np.testing.assert_array_equal(t[s:s + 1], sel, err_msg=f"decode selection of sequence {s}")
        assert_close_attention(out[sl], want, f"decode seq {s}")
