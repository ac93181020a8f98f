"""GPU parity where the tile unions outgrow the attention kernels' LDS block-list window.

The prefill attention and its dq backward hold a window of a tile's ascending block list in LDS
(16384 and 12288 entries) and move it along the chunks when the union is longer. Two workloads
reach that regime:
  * B = 1 at N = 20037 with unrelated queries and k = 2048: the late tiles' unions hold nearly every
    one of their ~20000 blocks, so both windows move several times per tile (small heads, so the
    oracle stays quick);
  * B = 8 at N = 1048571 (just under 2^20 tokens, the context the pages' architecture section aims
    at) with 2 KV groups of 4 heads and k = 4096: the selection runs with 32-bit block ids
    (131072 blocks) and the prefill accepts the full length.
Selections, unions and attention are compared with the oracle on sampled tiles and rows; the
fused prefill must equal the single calls bit for bit.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from tests.gpu_common import OracleChain, assert_close_attention, bf16_to_f64, bits, params_of, say

pytestmark = pytest.mark.gpu

WINDOW_B1 = datagen.PREFILL.replace(name="window_b1_20k", n_tokens=20037, n_q_heads=8, n_kv_heads=1, block=1,
                                    topk_tokens=2048, union_tile=64, qi_mode="iid")
LONG_1M = datagen.PREFILL.replace(name="prefill_1m_g2", n_tokens=(1 << 20) - 5, n_q_heads=8, n_kv_heads=2,
                                  union_tile=128)


@pytest.fixture(scope="module")
def sg():
    import block_sparse_long_sgqa_amd as sg

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sg.lib()
    return sg


def run_chain(sg, wl):
    """Single calls (topk kept for the checks) and the fused prefill on device inputs."""
    p = params_of(wl)
    say(f"{wl.name}: drawing inputs N={p.n_tokens} B={p.block} G={p.n_kv_heads} Hq={p.n_q_heads}")
    x = datagen.prefill_inputs(wl, device="cuda")
    o = sg.alloc_prefill_outputs(p)
    say(f"{wl.name}: compress / index_topk / union / attend")
    sg.sgqa_compress(p, x["ki"], o["blk_k"])
    sg.sgqa_index_topk(p, x["qi"], x["w"], o["blk_k"], o["topk"])
    sg.sgqa_union(p, o["topk"], o["umask"], o["ucount"])
    sg.sgqa_attend(p, x["q"], x["k"], x["v"], o["umask"], o["ucount"], o["out"])
    torch.cuda.synchronize()
    say(f"{wl.name}: sgqa_prefill")
    out2 = torch.empty_like(o["out"])
    ws = sg.workspace(p, sg.SGQA_OP_PREFILL)
    sg.sgqa_prefill(p, x["q"], x["k"], x["v"], x["qi"], x["w"], x["ki"], out2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), o["out"].view(torch.int16)), "prefill != single calls"
    assert torch.isfinite(o["out"].float()).all()
    del ws, out2
    return p, x, o


def check_tiles(wl, p, x, o, tiles, rows_per_tile, rng):
    """Selections and unions of the sampled tiles, then attention on sampled rows of them."""
    ch = OracleChain({k: x[k].cpu() for k in ("qi", "ki", "w")}, p)
    np.testing.assert_array_equal(bits(o["blk_k"]), ch.kbar)
    say(f"{wl.name}: oracle selections and unions of tiles {tiles.tolist()}")
    om, oc, sel, rows = ch.union_of_tiles(tiles)
    got_sel = o["topk"][:, torch.from_numpy(rows).long().cuda()].cpu().numpy()
    np.testing.assert_array_equal(got_sel, sel)
    umask = o["umask"][:, torch.from_numpy(tiles).long().cuda()].cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(umask, om[:, tiles])
    np.testing.assert_array_equal(o["ucount"][:, torch.from_numpy(tiles).long().cuda()].cpu().numpy(), oc[:, tiles])
    say(f"{wl.name}: union sizes of the sampled tiles {oc[:, tiles].tolist()}")
    arows = np.concatenate([rng.choice(ch.tile_rows(int(t)), size=min(rows_per_tile, len(ch.tile_rows(int(t)))),
                                       replace=False) for t in tiles]).astype(np.int32)
    arows = np.unique(np.concatenate([arows, [p.n_tokens - 1]])).astype(np.int32)
    want = oracle.attend(bits(x["q"]), bits(x["k"]), bits(x["v"]), om, p.block, p.union_tile, rows=arows)
    got = o["out"][torch.from_numpy(arows).long().cuda()]
    assert_close_attention(got, want, f"{wl.name} attention")
    return om, arows


def assert_close_grad(got_bf16, want, what):
    # The backward tests' bar: relative to the largest |reference| of the compared values.
    got = bf16_to_f64(bits(got_bf16)).reshape(want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite"
    scale = max(1e-6, float(np.abs(want).max()))
    err = np.abs(got - want)
    say(f"{what}: scale={scale:.3e} max_rel={err.max() / scale:.3e} mean_rel={err.mean() / scale:.3e}")
    assert err.max() <= 2e-2 * scale, f"{what}: max error {err.max()} (scale {scale})"
    assert err.mean() <= 2e-3 * scale, f"{what}: mean error {err.mean()} (scale {scale})"


def test_window_b1_dense_unions(sg):
    wl = WINDOW_B1
    p, x, o = run_chain(sg, wl)
    ucount = o["ucount"].cpu().numpy()
    assert ucount.max() > 16384, f"the test needs unions past the LDS window (largest {ucount.max()})"
    rng = np.random.default_rng(5)
    big = np.nonzero(ucount[0] > 16384)[0]
    N = p.n_tokens
    key_lo, key_hi = N - 80, N  # dk/dv checked on these keys: every row attending them is in the last tiles
    tail = np.arange(key_lo // p.union_tile, p.n_tiles)
    tiles = np.unique(np.concatenate([[0], tail, rng.choice(big, size=3, replace=False)]))
    om, arows = check_tiles(wl, p, x, o, tiles, rows_per_tile=6, rng=rng)

    # Backward: dq on the sampled rows (dq's window is 12288 entries), dk/dv of the last 80 keys.
    say(f"{wl.name}: forward with lse and backward")
    Hq, G, D = p.n_q_heads, p.n_kv_heads, p.head_dim
    gen = torch.Generator(device="cuda")
    gen.manual_seed(13)
    dout = torch.randn((N, Hq, D), generator=gen, device="cuda").to(torch.bfloat16)
    out = torch.empty_like(o["out"])
    lse = torch.empty((N, Hq), dtype=torch.float32, device="cuda")
    sg.sgqa_attend_fwd(p, x["q"], x["k"], x["v"], o["umask"], o["ucount"], out, lse)
    dq = torch.empty_like(out)
    dk = torch.empty((G, N, D), dtype=torch.bfloat16, device="cuda")
    dv = torch.empty_like(dk)
    ws = sg.workspace(p, sg.SGQA_OP_ATTEND_BWD)
    sg.sgqa_attend_bwd(p, x["q"], x["k"], x["v"], o["umask"], o["ucount"], out, lse, dout, dq, dk, dv, ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), o["out"].view(torch.int16))
    say(f"{wl.name}: oracle gradient on {len(arows)} rows and keys {key_lo}..{key_hi - 1}")
    pq, pk, pv = oracle.attend_bwd_part(bits(x["q"]), bits(x["k"]), bits(x["v"]), om, bits(dout), p.block,
                                        p.union_tile, arows, 0, key_lo, key_hi)
    assert_close_grad(dq[torch.from_numpy(arows).long().cuda()], pq, f"{wl.name} dq rows")
    assert_close_grad(dk[0, key_lo:key_hi], pk, f"{wl.name} dk keys")
    assert_close_grad(dv[0, key_lo:key_hi], pv, f"{wl.name} dv keys")


def test_prefill_1m_block8(sg):
    wl = LONG_1M
    p, x, o = run_chain(sg, wl)
    assert p.n_tokens // p.block > 65536  # 32-bit block ids in the selection
    rng = np.random.default_rng(9)
    tiles = np.unique(np.concatenate([[0, p.n_tiles - 1], rng.integers(p.n_tiles // 2, p.n_tiles, 2)]))
    check_tiles(wl, p, x, o, tiles, rows_per_tile=4, rng=rng)
