"""Incremental / varlen / paged decode on the GPU (sgqa_decode_varlen, sgqa_append) against the oracle.

The oracle needs nothing new: a sequence of length L_s is sgqa_decode's problem on the first L_s
positions of its caches, and a block key written by sgqa_append is the block compression of the
index keys it closes. Every check here compares with the oracle on those prefixes (selections
bit-exact, outputs within the attention tolerance), and paged runs with dense runs bit-exactly.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from tests.gpu_common import assert_close_attention, bits, params_of, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sg():
    import block_sparse_long_sgqa_amd as sg

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sg.lib()
    return sg


def small_decode(S=3, C=1200, G=2, k=256, B=8, name="varlen"):
    wl = datagen.DECODE.replace(name=f"dec_{name}_{C}_{S}_{G}", n_tokens=C, n_seqs=S, n_q_heads=8 * G,
                                n_kv_heads=G, topk_tokens=k, block=B)
    return wl, params_of(wl), datagen.decode_inputs(wl)


def oracle_seq(x, s, L, B, kb):
    """The oracle's decode of sequence s at context length L (its first L positions)."""
    sl = slice(s, s + 1)
    kbar = oracle.compress(bits(x["ki_cache"][sl, :L]), B)
    sel, out = oracle.decode(x["q"][sl], x["k_cache"][sl, :, :L].contiguous(), x["v_cache"][sl, :, :L].contiguous(),
                             kbar, x["qi"][sl], x["w"], B, kb)
    return sel, out


def to_pages(sg, cache, page_tokens, seed):
    """Scatter dense caches [S][G][C][D] into a pool of pages under a random page table."""
    S, G, C, D = cache.shape
    per = (C + page_tokens - 1) // page_tokens
    n_pages = S * per + 5
    rng = np.random.default_rng(seed)
    table = rng.permutation(n_pages)[:S * per].reshape(S, per).astype(np.int32)
    pool = torch.zeros((n_pages, G, page_tokens, D), dtype=cache.dtype, device=cache.device)
    for s in range(S):
        for pg in range(per):
            t0, t1 = pg * page_tokens, min(C, (pg + 1) * page_tokens)
            pool[int(table[s, pg]), :, : t1 - t0] = cache[s, :, t0:t1]
    return torch.from_numpy(table).cuda(), pool, n_pages


def test_varlen_decode_matches_oracle_and_dense_paged_agree(sg):
    wl, p, x = small_decode(S=4)
    S, C, B = p.n_seqs, p.n_tokens, p.block
    lens = [C, 777, 9, 1]
    say(f"varlen decode S={S} C={C} lens={lens}")
    xd = {k: v.cuda() for k, v in x.items()}
    blk = torch.empty((S, C // B, 64), dtype=torch.bfloat16, device="cuda")
    sg.sgqa_compress(p, xd["ki_cache"], blk)
    ws = sg.workspace(p, sg.SGQA_OP_DECODE)
    out = torch.empty((S, p.n_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    topk = torch.empty((S, p.n_kv_heads, p.kb), dtype=torch.int32, device="cuda")
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    sg.sgqa_decode_varlen(p, xd["q"], xd["k_cache"], xd["v_cache"], blk, xd["qi"], xd["w"], sl, out, ws,
                          topk_out=topk)
    torch.cuda.synchronize()
    for s, L in enumerate(lens):
        sel, want = oracle_seq(x, s, L, B, p.kb)
        np.testing.assert_array_equal(topk[s:s + 1].cpu().numpy(), sel)
        assert_close_attention(out[s:s + 1], want, f"varlen seq {s} L={L}")
    # Paged pools under a random page table give the same bits.
    table, kpool, n_pages = to_pages(sg, xd["k_cache"], 64, 1)
    _, vpool, _ = to_pages(sg, xd["v_cache"], 64, 1)
    pages = sg.Pages(table, 64, n_pages)
    out_p = torch.empty_like(out)
    sg.sgqa_decode_varlen(p, xd["q"], kpool, vpool, blk, xd["qi"], xd["w"], sl, out_p, ws, pages=pages)
    torch.cuda.synchronize()
    assert torch.equal(out_p.view(torch.int16), out.view(torch.int16))
    # All lengths at capacity: identical to sgqa_decode.
    full = torch.full((S,), C, dtype=torch.int32, device="cuda")
    out_v = torch.empty_like(out)
    out_d = torch.empty_like(out)
    sg.sgqa_decode_varlen(p, xd["q"], xd["k_cache"], xd["v_cache"], blk, xd["qi"], xd["w"], full, out_v, ws)
    sg.sgqa_decode(p, xd["q"], xd["k_cache"], xd["v_cache"], blk, xd["qi"], xd["w"], out_d, ws)
    torch.cuda.synchronize()
    assert torch.equal(out_v.view(torch.int16), out_d.view(torch.int16))


def test_varlen_lengths_are_clamped(sg):
    # Lengths outside [1, C] are clamped: 0 behaves as 1 and C + 50 as C.
    wl, p, x = small_decode(S=2, C=300, name="clamp")
    S, C, B = p.n_seqs, p.n_tokens, p.block
    xd = {k: v.cuda() for k, v in x.items()}
    blk = torch.empty((S, C // B, 64), dtype=torch.bfloat16, device="cuda")
    sg.sgqa_compress(p, xd["ki_cache"], blk)
    ws = sg.workspace(p, sg.SGQA_OP_DECODE)
    outs = []
    for lens in ([0, C + 50], [1, C]):
        out = torch.empty((S, p.n_q_heads, 128), dtype=torch.bfloat16, device="cuda")
        sg.sgqa_decode_varlen(p, xd["q"], xd["k_cache"], xd["v_cache"], blk, xd["qi"], xd["w"],
                              torch.tensor(lens, dtype=torch.int32, device="cuda"), out, ws)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


@pytest.mark.parametrize("paged", [False, True])
def test_append_then_decode_step_by_step(sg, paged):
    S, C, B, T = 3, 400, 8, 12
    wl, p, x = small_decode(S=S, C=C, name="append")
    G = p.n_kv_heads
    L0 = [5, 63, 300]
    say(f"append loop paged={paged} L0={L0} T={T}")
    xd = {k: v.cuda() for k, v in x.items()}
    # Caches hold only the first L0[s] positions (and the block keys of the complete blocks there).
    kc = torch.zeros_like(xd["k_cache"])
    vc = torch.zeros_like(xd["v_cache"])
    ic = torch.zeros_like(xd["ki_cache"])
    blk = torch.zeros((S, C // B, 64), dtype=torch.bfloat16, device="cuda")
    for s, L in enumerate(L0):
        kc[s, :, :L] = xd["k_cache"][s, :, :L]
        vc[s, :, :L] = xd["v_cache"][s, :, :L]
        ic[s, :L] = xd["ki_cache"][s, :L]
        nb = L // B
        if nb:
            blk[s, :nb] = torch.from_numpy(oracle.compress(bits(x["ki_cache"][s:s + 1, :L]), B)[0].view(np.int16)) \
                .view(torch.bfloat16).cuda()
    pages = None
    if paged:
        table, kc, n_pages = to_pages(sg, kc, 64, 7)
        _, vc, _ = to_pages(sg, vc, 64, 7)
        pages = sg.Pages(table, 64, n_pages)
    ws = sg.workspace(p, sg.SGQA_OP_DECODE)
    out = torch.empty((S, p.n_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    topk = torch.empty((S, G, p.kb), dtype=torch.int32, device="cuda")
    for t in range(T):
        pos = [L + t for L in L0]
        posd = torch.tensor(pos, dtype=torch.int32, device="cuda")
        idx = torch.arange(S, device="cuda")
        pd = torch.tensor(pos, device="cuda", dtype=torch.long)
        k_new = xd["k_cache"][idx, :, pd].contiguous()          # [S][G][D]
        v_new = xd["v_cache"][idx, :, pd].contiguous()
        i_new = xd["ki_cache"][idx, pd].contiguous()            # [S][dI]
        sg.sgqa_append(p, k_new, v_new, i_new, posd, kc, vc, ic, blk, pages=pages)
        lens = torch.tensor([q + 1 for q in pos], dtype=torch.int32, device="cuda")
        sg.sgqa_decode_varlen(p, xd["q"], kc, vc, blk, xd["qi"], xd["w"], lens, out, ws, pages=pages, topk_out=topk)
        torch.cuda.synchronize()
        for s in range(S):
            L = pos[s] + 1
            nb = L // B
            want_blk = oracle.compress(bits(x["ki_cache"][s:s + 1, :L]), B)
            np.testing.assert_array_equal(bits(blk[s:s + 1, :nb]), want_blk)
            sel, want = oracle_seq(x, s, L, B, p.kb)
            np.testing.assert_array_equal(topk[s:s + 1].cpu().numpy(), sel)
            assert_close_attention(out[s:s + 1], want, f"append step {t} seq {s} L={L}")
    np.testing.assert_array_equal(bits(ic[0, :L0[0] + T]), bits(x["ki_cache"][0, :L0[0] + T]))


def test_append_skips_out_of_range_positions(sg):
    S, C = 2, 64
    wl, p, x = small_decode(S=S, C=C, name="skip")
    xd = {k: v.cuda() for k, v in x.items()}
    kc = torch.zeros_like(xd["k_cache"])
    vc = torch.zeros_like(xd["v_cache"])
    ic = torch.zeros_like(xd["ki_cache"])
    blk = torch.zeros((S, C // p.block, 64), dtype=torch.bfloat16, device="cuda")
    k_new = torch.ones((S, p.n_kv_heads, 128), dtype=torch.bfloat16, device="cuda")
    i_new = torch.ones((S, 64), dtype=torch.bfloat16, device="cuda")
    pos = torch.tensor([-1, C], dtype=torch.int32, device="cuda")
    sg.sgqa_append(p, k_new, k_new, i_new, pos, kc, vc, ic, blk)
    torch.cuda.synchronize()
    assert not kc.any() and not vc.any() and not ic.any() and not blk.any()
