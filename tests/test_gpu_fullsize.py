"""GPU parity at the measured sizes, in the launch configuration bench.py times.

The oracle cannot finish these workloads whole, so it checks sampled outputs one by one (rows of
the selection, whole union tiles, query rows of the attention, whole decode sequences); every
output is also checked against properties that hold at any size.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from tests.gpu_common import OracleChain, assert_close_attention, bits, params_of, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sg():
    import block_sparse_long_sgqa_amd as sg

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sg.lib()
    return sg


def check_topk_properties(topk: np.ndarray, block: int, kb: int, rows: np.ndarray) -> None:
    """Every row: ascending ids < c(i), exactly min(kb, c(i)) of them, then -1."""
    for g in range(topk.shape[0]):
        for i in rows:
            c = int(i) // block
            r = topk[g, i]
            m = min(kb, c)
            assert (r[m:] == -1).all(), (g, i)
            v = r[:m]
            assert (v >= 0).all() and (v < max(c, 1)).all(), (g, i)
            assert (np.diff(v) > 0).all(), (g, i)


def run_prefill_full(sg, wl, n_rows_sample, tiles_sample, attn_rows_per_tile):
    p = params_of(wl)
    say(f"full-size {wl.name}: drawing inputs on the GPU")
    x = datagen.prefill_inputs(wl, device="cuda")
    o = sg.alloc_prefill_outputs(p)
    say(f"full-size {wl.name}: compress/index_topk/union/attend")
    sg.sgqa_compress(p, x["ki"], o["blk_k"])
    sg.sgqa_index_topk(p, x["qi"], x["w"], o["blk_k"], o["topk"])
    sg.sgqa_union(p, o["topk"], o["umask"], o["ucount"])
    sg.sgqa_attend(p, x["q"], x["k"], x["v"], o["umask"], o["ucount"], o["out"])
    torch.cuda.synchronize()
    say(f"full-size {wl.name}: sgqa_prefill")
    out2 = torch.empty_like(o["out"])
    ws = sg.workspace(p, sg.SGQA_OP_PREFILL)
    sg.sgqa_prefill(p, x["q"], x["k"], x["v"], x["qi"], x["w"], x["ki"], out2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), o["out"].view(torch.int16)), "prefill != single calls"
    del ws, out2

    host = {k: x[k].cpu() for k in ("qi", "ki", "w")}
    ch = OracleChain(host, p)
    np.testing.assert_array_equal(bits(o["blk_k"]), ch.kbar)

    topk = o["topk"].cpu().numpy()
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 1, p.block * p.kb - 1, p.block * p.kb, p.n_tokens - 1],
                                     rng.integers(0, p.n_tokens, n_rows_sample)])).astype(np.int32)
    say(f"full-size {wl.name}: oracle top-k on {len(rows)} sampled rows")
    np.testing.assert_array_equal(topk[:, rows], ch.topk(rows))
    check_topk_properties(topk, p.block, p.kb, rng.integers(0, p.n_tokens, 2000))

    umask = o["umask"].cpu().numpy().view(np.uint32)
    ucount = o["ucount"].cpu().numpy()
    pc = np.unpackbits(umask.view(np.uint8), axis=-1).sum(axis=-1)
    np.testing.assert_array_equal(pc, ucount)                     # count = popcount, every tile
    tiles = np.unique(np.concatenate([[0, p.n_tiles - 1], rng.integers(0, p.n_tiles, tiles_sample)]))
    say(f"full-size {wl.name}: oracle union on tiles {tiles.tolist()}")
    om, oc, _, _ = ch.union_of_tiles(tiles)
    np.testing.assert_array_equal(umask[:, tiles], om[:, tiles])
    np.testing.assert_array_equal(ucount[:, tiles], oc[:, tiles])

    arows = np.concatenate([rng.choice(ch.tile_rows(int(t)), size=min(attn_rows_per_tile, len(ch.tile_rows(int(t)))),
                                       replace=False) for t in tiles]).astype(np.int32)
    say(f"full-size {wl.name}: oracle attention on {len(arows)} rows")
    want = oracle.attend(bits(x["q"]), bits(x["k"]), bits(x["v"]), om, p.block, p.union_tile, rows=arows)
    got = o["out"][torch.from_numpy(arows).long().cuda()]
    assert_close_attention(got, want, f"{wl.name} attention")
    assert torch.isfinite(o["out"].float()).all()


def test_prefill_32k_full_size(sg):
    run_prefill_full(sg, datagen.PREFILL, n_rows_sample=48, tiles_sample=3, attn_rows_per_tile=8)


def test_long_prefill_128k_full_size(sg):
    run_prefill_full(sg, datagen.LONG_PREFILL, n_rows_sample=24, tiles_sample=2, attn_rows_per_tile=4)


def test_prefill_32k_iid_stress(sg):
    # rho = 1: neighbouring queries are unrelated, unions are nearly dense.
    wl = datagen.PREFILL.replace(name="prefill_32k_iid", rho=1.0)
    run_prefill_full(sg, wl, n_rows_sample=16, tiles_sample=2, attn_rows_per_tile=4)


def test_ablation_block1_k2048_selection(sg):
    wl = datagen.ABLATION_B1
    p = params_of(wl)
    say("ablation B=1 k=2048 at 32k: drawing inputs")
    x = datagen.prefill_inputs(wl, device="cuda")
    blk = torch.empty((p.n_tokens, 64), dtype=torch.bfloat16, device="cuda")
    topk = torch.empty((p.n_kv_heads, p.n_tokens, p.kb), dtype=torch.int32, device="cuda")
    sg.sgqa_compress(p, x["ki"], blk)
    sg.sgqa_index_topk(p, x["qi"], x["w"], blk, topk)
    torch.cuda.synchronize()
    ch = OracleChain({k: x[k].cpu() for k in ("qi", "ki", "w")}, p)
    np.testing.assert_array_equal(bits(blk), bits(x["ki"]))  # B = 1: block keys are the keys
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[p.kb, p.kb + 1, p.n_tokens - 1], rng.integers(0, p.n_tokens, 16)]))
    say("ablation B=1: oracle rows")
    t = topk.cpu().numpy()
    np.testing.assert_array_equal(t[:, rows], ch.topk(rows.astype(np.int32)))
    check_topk_properties(t, 1, p.kb, rng.integers(0, p.n_tokens, 500))


def test_decode_256k_full_size(sg):
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
    c = (p.n_tokens - 1) // p.block
    assert (t >= 0).all() and (t < c).all() and (np.diff(t, axis=-1) > 0).all()
    for s in (0, 21):
        say(f"decode: oracle on sequence {s}")
        sl = slice(s, s + 1)
        kbar = oracle.compress(bits(y["ki_cache"][sl]), p.block)
        np.testing.assert_array_equal(bits(blk[sl]), kbar)
        sel, want = oracle.decode(y["q"][sl], y["k_cache"][sl], y["v_cache"][sl], kbar, y["qi"][sl], y["w"],
                                  p.block, p.kb)
        np.testing.assert_array_equal(t[s:s + 1], sel)
        assert_close_attention(out[sl], want, f"decode seq {s}")
