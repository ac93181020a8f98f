"""GPU parity on seeded random shapes, end to end through the C ABI against the oracle.

The fixed cases elsewhere list chosen shapes; here sequence length, query and KV head counts, block
size, k and union tile are drawn together (fixed seeds), so combinations none of them lists meet the
oracle: ragged last blocks, chunks and tiles at once, K_B that is not a multiple of a chunk's
blocks, K_B above or below the candidate count, one or several KV groups, head ratios from 1 to 8.
Selections (top-k and the fused tile union) must be bit-exact; attention outputs within the
attention tolerance; gradients within the relative gradient bar of the backward tests. Every draw
is sized so that the fp64 oracle takes seconds.
"""
import os

import numpy as np
import pytest
import torch

import datagen
import oracle
from tests.gpu_common import OracleChain, assert_close_attention, bits, params_of, say, to_dev
from tests.test_gpu_bwd import assert_close_grad, run_fwd_bwd

pytestmark = pytest.mark.gpu

N_PREFILL = 40
N_DECODE = 20


@pytest.fixture(scope="module")
def sg():
    import block_sparse_long_sgqa_amd as sg

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sg.lib()
    return sg


def draw_prefill(seed: int) -> datagen.Workload:
    rng = np.random.default_rng(7000 + seed)
    B = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
    G = int(rng.choice([1, 2, 3, 4]))
    r = int(rng.choice([1, 2, 4, 8]))
    N = int(rng.integers(2 * B, 2600))  # sequences shorter than a block are covered by the fixed cases
    kb = int(rng.integers(1, 260 if B > 1 else 700))
    tile = int(rng.choice([1, 7, 16, 33, 64, 128]))
    qi_mode = str(rng.choice(["iid", "corr"]))
    return datagen.PREFILL.replace(name=f"rand_prefill_{seed}", n_tokens=N, n_q_heads=G * r, n_kv_heads=G,
                                   block=B, topk_tokens=kb * B, union_tile=tile, qi_mode=qi_mode)


def describe(wl: datagen.Workload) -> str:
    return (f"N={wl.n_tokens} Hq={wl.n_q_heads} G={wl.n_kv_heads} B={wl.block} K_B={wl.kb} "
            f"Tq={wl.union_tile} qi={wl.qi_mode}")


@pytest.mark.parametrize("seed", range(N_PREFILL))
def test_random_prefill(sg, seed):
    wl = draw_prefill(seed)
    p = params_of(wl)
    x = datagen.prefill_inputs(wl)
    ch = OracleChain(x, p)
    sel = ch.topk()
    want_mask, want_cnt = oracle.union(sel, p.n_tokens, p.block, p.union_tile)
    want = oracle.attend(bits(x["q"]), bits(x["k"]), bits(x["v"]), want_mask, p.block, p.union_tile)
    say(f"random prefill {seed}: {describe(wl)}")
    xd = to_dev(x)
    G, N = p.n_kv_heads, p.n_tokens
    kbar = torch.from_numpy(ch.kbar.view(np.int16)).view(torch.bfloat16).cuda().reshape(-1, p.idx_dim)
    blk = torch.empty((N // p.block, p.idx_dim), dtype=torch.bfloat16, device="cuda")
    if N // p.block > 0:
        sg.sgqa_compress(p, xd["ki"], blk)
    topk = torch.empty((G, N, p.kb), dtype=torch.int32, device="cuda")
    sg.sgqa_index_topk(p, xd["qi"], xd["w"], kbar, topk)
    umask = torch.empty((G, p.n_tiles, p.n_words), dtype=torch.int32, device="cuda")
    ucount = torch.empty((G, p.n_tiles), dtype=torch.int32, device="cuda")
    sg.sgqa_index_union(p, xd["qi"], xd["w"], kbar, umask, ucount)
    out = torch.empty((N, p.n_q_heads, p.head_dim), dtype=torch.bfloat16, device="cuda")
    sg.sgqa_prefill(p, xd["q"], xd["k"], xd["v"], xd["qi"], xd["w"], xd["ki"], out,
                    sg.workspace(p, sg.SGQA_OP_PREFILL))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(blk), ch.kbar)
    np.testing.assert_array_equal(topk.cpu().numpy(), sel)
    np.testing.assert_array_equal(umask.cpu().numpy().view(np.uint32), want_mask)
    np.testing.assert_array_equal(ucount.cpu().numpy(), want_cnt)
    assert_close_attention(out, want, f"random prefill {seed}")


@pytest.mark.parametrize("seed", [s for s in range(N_PREFILL) if draw_prefill(s).n_tokens <= 1600])
def test_random_backward(sg, seed):
    wl = draw_prefill(seed)
    p = params_of(wl)
    x = datagen.prefill_inputs(wl)
    ch = OracleChain(x, p)
    umask, ucount = oracle.union(ch.topk(), p.n_tokens, p.block, p.union_tile)
    g = torch.Generator().manual_seed(31 + seed)
    dout = torch.randn((p.n_tokens, p.n_q_heads, p.head_dim), generator=g).to(torch.bfloat16)
    want_dq, want_dk, want_dv = oracle.attend_bwd(bits(x["q"]), bits(x["k"]), bits(x["v"]), umask, bits(dout),
                                                  p.block, p.union_tile)
    say(f"random backward {seed}: {describe(wl)}")
    xd = to_dev(x)
    um = torch.from_numpy(umask.view(np.int32)).cuda()
    uc = torch.from_numpy(ucount).cuda()
    _, _, dq, dk, dv = run_fwd_bwd(sg, p, xd, um, uc, dout.cuda())
    assert_close_grad(dq, want_dq, f"dq random {seed}")
    assert_close_grad(dk, want_dk, f"dk random {seed}")
    assert_close_grad(dv, want_dv, f"dv random {seed}")
    # Again with the smallest batches the plan allows (many batches, the partial-row buffers
    # alternating and each batch's tile-order sum on the second stream). The batches are runs of
    # whole tiles summed in tile order, so while the tile-major design runs the gradients are the
    # same bits; past its batch limit the key-major design runs and is held to the oracle instead.
    deltas = (p.n_tokens * p.n_q_heads * 4 + 255) // 256 * 256
    tile_major = sg.workspace_size(p, sg.SGQA_OP_ATTEND_BWD) > deltas
    os.environ["SGQA_BWD_BATCH_ROWS"] = "1"
    try:
        batched_tile_major = sg.workspace_size(p, sg.SGQA_OP_ATTEND_BWD) > deltas
        _, _, dq2, dk2, dv2 = run_fwd_bwd(sg, p, xd, um, uc, dout.cuda())
    finally:
        os.environ.pop("SGQA_BWD_BATCH_ROWS", None)
    if tile_major and batched_tile_major:
        for a, b, n in ((dq, dq2, "dq"), (dk, dk2, "dk"), (dv, dv2, "dv")):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{n} random {seed}: batched run differs"
    else:
        assert_close_grad(dq2, want_dq, f"dq random {seed} batched")
        assert_close_grad(dk2, want_dk, f"dk random {seed} batched")
        assert_close_grad(dv2, want_dv, f"dv random {seed} batched")


def draw_decode(seed: int) -> datagen.Workload:
    rng = np.random.default_rng(9100 + seed)
    B = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
    G = int(rng.choice([1, 2, 3, 5, 8]))
    S = int(rng.integers(1, 5))
    L = int(rng.integers(2 * B, 40000))
    kb = int(rng.integers(1, 1500))
    return datagen.DECODE.replace(name=f"rand_decode_{seed}", n_tokens=L, n_seqs=S, n_q_heads=8 * G, n_kv_heads=G,
                                  topk_tokens=kb * B, block=B)


@pytest.mark.parametrize("seed", range(N_DECODE))
def test_random_decode(sg, seed):
    wl = draw_decode(seed)
    p = params_of(wl)
    S, L, G, B = wl.n_seqs, wl.n_tokens, wl.n_kv_heads, wl.block
    x = datagen.decode_inputs(wl)
    kbar = oracle.compress(bits(x["ki_cache"]), B)
    want_sel, want_out = oracle.decode(x["q"], x["k_cache"], x["v_cache"], kbar, x["qi"], x["w"], B, p.kb)
    say(f"random decode {seed}: L={L} S={S} G={G} B={B} K_B={p.kb}")
    xd = to_dev(x)
    blk = torch.empty((S, L // B, 64), dtype=torch.bfloat16, device="cuda")
    if L // B > 0:
        sg.sgqa_compress(p, xd["ki_cache"], blk)
    out = torch.empty((S, p.n_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    topk = torch.empty((S, G, p.kb), dtype=torch.int32, device="cuda")
    sg.sgqa_decode(p, xd["q"], xd["k_cache"], xd["v_cache"], blk, xd["qi"], xd["w"], out, sg.workspace(p, sg.SGQA_OP_DECODE),
                   topk_out=topk)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(blk), kbar.reshape(bits(blk).shape))
    np.testing.assert_array_equal(topk.cpu().numpy(), want_sel)
    assert_close_attention(out, want_out, f"random decode {seed}")


# ---------------------------------------------------------------- variants

def masked_fits(B: int, r: int) -> bool:
    """The masked-union kernel's per-chunk membership table (64 / B block entries times one word per
    32 queries of a 256-row workgroup) must fit its 64 words."""
    span = -(-256 // r) + 1
    return (64 // B) * ((span + 31) // 32) <= 64


def draw_masked(seed: int) -> datagen.Workload:
    rng = np.random.default_rng(8300 + seed)
    while True:
        B = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
        r = int(rng.choice([1, 2, 4, 8, 16]))
        if masked_fits(B, r):
            break
    G = int(rng.choice([1, 2]))
    N = int(rng.integers(2 * B, 1800))
    kb = int(rng.integers(1, 200 if B > 1 else 500))
    tile = int(rng.choice([1, 5, 16, 48, 64, 128]))
    return datagen.PREFILL.replace(name=f"rand_masked_{seed}", n_tokens=N, n_q_heads=G * r, n_kv_heads=G,
                                   block=B, topk_tokens=kb * B, union_tile=tile, qi_mode="iid")


@pytest.mark.parametrize("seed", range(12))
def test_random_prefill_masked(sg, seed):
    wl = draw_masked(seed)
    p = params_of(wl)
    x = datagen.prefill_inputs(wl)
    ch = OracleChain(x, p)
    want = oracle.attend_sel(bits(x["q"]), bits(x["k"]), bits(x["v"]), ch.topk(), p.block)
    say(f"random masked prefill {seed}: {describe(wl)}")
    xd = to_dev(x)
    out = torch.empty((p.n_tokens, p.n_q_heads, p.head_dim), dtype=torch.bfloat16, device="cuda")
    sg.sgqa_prefill_masked(p, xd["q"], xd["k"], xd["v"], xd["qi"], xd["w"], xd["ki"], out,
                           sg.workspace(p, sg.SGQA_OP_PREFILL_MASKED))
    torch.cuda.synchronize()
    assert_close_attention(out, want, f"random masked prefill {seed}")


def draw_varlen(seed: int):
    rng = np.random.default_rng(9700 + seed)
    B = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
    G = int(rng.choice([1, 2, 3]))
    S = int(rng.integers(1, 6))
    C = int(rng.integers(2 * B, 6000))
    kb = int(rng.integers(1, 600))
    page = int(rng.choice([p for p in (1, 2, 4, 8, 16, 32, 64, 128, 256) if p >= B]))
    lens = [int(v) for v in rng.integers(1, C + 1, size=S)]
    wl = datagen.DECODE.replace(name=f"rand_varlen_{seed}", n_tokens=C, n_seqs=S, n_q_heads=8 * G, n_kv_heads=G,
                                topk_tokens=kb * B, block=B)
    return wl, page, lens


def oracle_prefix(x, s, L, B, kb, caches=None):
    """The oracle's decode of sequence s over the first L positions of its caches."""
    sl = slice(s, s + 1)
    kbar = oracle.compress(bits(x["ki_cache"][sl, :L]), B)
    if caches is None:
        return oracle.decode(x["q"][sl], x["k_cache"][sl, :, :L].contiguous(), x["v_cache"][sl, :, :L].contiguous(),
                             kbar, x["qi"][sl], x["w"], B, kb)
    return oracle.decode_fp8(x["q"][sl], caches["k8"][sl, :, :L].contiguous(), caches["v8"][sl, :, :L].contiguous(),
                             caches["kv_scale"][sl], kbar, x["qi"][sl], x["w"], B, kb)


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("fp8", [False, True])
def test_random_varlen_paged_decode(sg, seed, fp8):
    from tests.test_gpu_incremental import to_pages

    wl, page, lens = draw_varlen(seed)
    p = params_of(wl)
    S, C, G, B = wl.n_seqs, wl.n_tokens, wl.n_kv_heads, wl.block
    x = datagen.decode_inputs(wl)
    f = datagen.fp8_caches(wl) if fp8 else None
    say(f"random varlen decode {seed} fp8={fp8}: C={C} S={S} G={G} B={B} K_B={p.kb} page={page} lens={lens}")
    xd = to_dev(x)
    blk = torch.empty((S, C // B, 64), dtype=torch.bfloat16, device="cuda")
    sg.sgqa_compress(p, xd["ki_cache"], blk)
    ws = sg.workspace(p, sg.SGQA_OP_DECODE)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    kc, vc = (f["k8"].cuda(), f["v8"].cuda()) if fp8 else (xd["k_cache"], xd["v_cache"])

    def run(k_cache, v_cache, pages=None):
        out = torch.empty((S, p.n_q_heads, 128), dtype=torch.bfloat16, device="cuda")
        topk = torch.empty((S, G, p.kb), dtype=torch.int32, device="cuda")
        if fp8:
            sg.sgqa_decode_fp8(p, xd["q"], k_cache, v_cache, f["kv_scale"].cuda(), blk, xd["qi"], xd["w"], out, ws,
                               seq_lens=sl, pages=pages, topk_out=topk)
        else:
            sg.sgqa_decode_varlen(p, xd["q"], k_cache, v_cache, blk, xd["qi"], xd["w"], sl, out, ws, pages=pages,
                                  topk_out=topk)
        torch.cuda.synchronize()
        return out, topk

    out, topk = run(kc, vc)
    for s, L in enumerate(lens):
        sel, want = oracle_prefix(x, s, L, B, p.kb, f)
        np.testing.assert_array_equal(topk[s:s + 1].cpu().numpy(), sel)
        assert_close_attention(out[s:s + 1], want, f"random varlen {seed} fp8={fp8} seq {s} L={L}")
    table, kpool, n_pages = to_pages(sg, kc, page, 100 + seed)
    _, vpool, _ = to_pages(sg, vc, page, 100 + seed)
    out_p, topk_p = run(kpool, vpool, sg.Pages(table, page, n_pages))
    assert torch.equal(topk_p, topk)
    assert torch.equal(out_p.view(torch.int16), out.view(torch.int16))
