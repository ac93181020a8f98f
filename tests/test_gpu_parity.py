"""GPU parity of every C-ABI call against the CPU oracle, at sizes the oracle finishes in seconds.

Bar: block keys, selections and unions bit-exact (integer-valued indexer inputs make fp32 scores
exact); attention within max-abs 1e-2 and mean-abs 1e-3 of the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from tests.gpu_common import (OracleChain, assert_close_attention, bits, params_of, say, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sg():
    import block_sparse_long_sgqa_amd as sg

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sg.lib()
    return sg


# Small workloads: several tiles, ragged tails, every block size of interest.
SMALL = {
    "tiny": datagen.TINY,
    "gqa_ragged": datagen.PREFILL.replace(name="gqa_ragged", n_tokens=3000 + 5, topk_tokens=512, union_tile=64),
    "b4_tile24": datagen.PREFILL.replace(name="b4_tile24", n_tokens=1531, n_q_heads=16, n_kv_heads=2, block=4,
                                         topk_tokens=256, union_tile=24),
    "b1_token": datagen.PREFILL.replace(name="b1_token", n_tokens=1100, n_q_heads=8, n_kv_heads=1, block=1,
                                        topk_tokens=200, union_tile=16),
    "b16_iid": datagen.PREFILL.replace(name="b16_iid", n_tokens=2048 + 17, n_q_heads=32, n_kv_heads=4, block=16,
                                       topk_tokens=512, union_tile=32, qi_mode="iid"),
    "tile1": datagen.PREFILL.replace(name="tile1", n_tokens=700, n_q_heads=8, n_kv_heads=1, topk_tokens=128,
                                     union_tile=1),
    "b64_r4": datagen.PREFILL.replace(name="b64_r4", n_tokens=4096 + 64 + 3, n_q_heads=16, n_kv_heads=4, block=64,
                                      topk_tokens=1024, union_tile=128),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_compress_bit_exact(sg, name):
    wl = SMALL[name]
    p = params_of(wl)
    say(f"compress {name} N={p.n_tokens} B={p.block}")
    x = datagen.prefill_inputs(wl)
    want = oracle.compress(bits(x["ki"]), p.block)
    ki = x["ki"].cuda()
    out = torch.empty((max(p.n_tokens // p.block, 1), p.idx_dim), dtype=torch.bfloat16, device="cuda")
    sg.sgqa_compress(p, ki, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out)[: p.n_tokens // p.block], want)


def test_compress_multi_sequence_and_normal_data(sg):
    # S sequences at once (the decode cache build) on N(0,1) keys: bit-exact (both sides sum in fp64
    # in ascending position and round once).
    S, N, B = 3, 4096 + 24, 8
    g = torch.Generator().manual_seed(5)
    ki = torch.randn((S, N, 64), generator=g).to(torch.bfloat16)
    want = oracle.compress(bits(ki), B)
    p = sg.Params(n_tokens=N, n_q_heads=8, n_kv_heads=1, block=B, n_seqs=S)
    out = torch.empty((S, N // B, 64), dtype=torch.bfloat16, device="cuda")
    say("compress S=3 normal data")
    sg.sgqa_compress(p, ki.cuda(), out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out), want)


@pytest.mark.parametrize("B", [1, 2, 8, 32])
def test_compress_bit_exact_any_bf16(sg, B):
    """Arbitrary finite bf16 keys: subnormals, exponents spread over the whole range inside one
    block, infinities and exact rounding ties (pairs one bf16 ulp apart average to a tie)."""
    rng = np.random.default_rng(100 + B)
    S, N = 2, 96 * B + max(B - 1, 1) // 2
    raw = rng.integers(0, 0x7F80, size=(S, N, 64), dtype=np.uint16)        # finite magnitudes
    raw |= (rng.integers(0, 2, size=raw.shape, dtype=np.uint16) << 15)    # signs
    nb = N // B
    sub = rng.integers(0, 0x0080, size=(S, N, 64), dtype=np.uint16)       # subnormal magnitudes
    raw[:, : (nb // 4) * B] = sub[:, : (nb // 4) * B]
    if B >= 2:
        lo = rng.integers(0x3F00, 0x4100, size=(S, N // 2, 64), dtype=np.uint16) & 0xFFFE
        ties = np.stack([lo, lo + 1], axis=2).reshape(S, -1, 64)         # x and x + 1 ulp
        r0 = (nb // 4) * B
        r1 = min(N, r0 + (nb // 4) * B)
        raw[:, r0:r1] = ties[:, r0:r1]
    raw[0, 5, 3] = 0x7F80                                                  # +inf
    raw[1, 7, 9] = 0xFF80                                                  # -inf
    want = oracle.compress(raw, B)
    ki = torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16).cuda()
    p = sg.Params(n_tokens=N, n_q_heads=8, n_kv_heads=1, block=B, n_seqs=S)
    out = torch.empty((S, nb, 64), dtype=torch.bfloat16, device="cuda")
    say(f"compress arbitrary bf16 B={B} N={N}")
    sg.sgqa_compress(p, ki, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out), want)


def run_topk(sg, p, xd, kbar_dev):
    topk = torch.empty((p.n_kv_heads, p.n_tokens, p.kb), dtype=torch.int32, device="cuda")
    sg.sgqa_index_topk(p, xd["qi"], xd["w"], kbar_dev, topk)
    return topk


# Selection-only cases: K_B = 576 makes the per-row buffer exactly K_B + one chunk, so cuts in the
# middle of the stream take their smallest room (independent queries: many of them).
TOPK_EXTRA = {
    "kb576_room": datagen.PREFILL.replace(name="kb576_room", n_tokens=8192 + 5, n_q_heads=16, n_kv_heads=2,
                                          topk_tokens=4608, union_tile=64, qi_mode="iid"),
}


@pytest.mark.parametrize("name", list(SMALL) + list(TOPK_EXTRA))
def test_index_topk_bit_exact(sg, name):
    wl = SMALL[name] if name in SMALL else TOPK_EXTRA[name]
    p = params_of(wl)
    x = datagen.prefill_inputs(wl)
    ch = OracleChain(x, p)
    say(f"index_topk {name} N={p.n_tokens} G={p.n_kv_heads} B={p.block} kb={p.kb}")
    xd = to_dev(x)
    kbar = torch.from_numpy(ch.kbar.view(np.int16)).view(torch.bfloat16).cuda()
    topk = run_topk(sg, p, xd, kbar)
    torch.cuda.synchronize()
    want = ch.topk()
    np.testing.assert_array_equal(topk.cpu().numpy(), want)


@pytest.mark.parametrize("case", ["zero_queries", "dense_k", "negative_weights", "all_equal_keys",
                                  "strided_outliers", "sample_sees_only_the_top"])
def test_index_topk_degenerate_cases(sg, case):
    wl = datagen.PREFILL.replace(name=f"deg_{case}", n_tokens=2500, n_q_heads=16, n_kv_heads=2, topk_tokens=400,
                                 union_tile=32)
    if case == "dense_k":
        wl = wl.replace(topk_tokens=4096)
    if case == "strided_outliers":
        # Every 4th block scores far above the rest and the others tie in small groups: a strided
        # sample of the candidates is unrepresentative (the kernel must still be exact).
        wl = wl.replace(n_tokens=4096, topk_tokens=128)
    if case == "sample_sees_only_the_top":
        # Odd blocks score above zero, even blocks exactly zero. Rows with 641..1152 candidates
        # take their threshold from a stride-2 sample of the odd blocks only, which sets it above
        # the true K_B-th score in most rows: those rows must take every candidate in a second
        # pass (the kernel must still be exact).
        wl = wl.replace(n_tokens=8192 + 5, topk_tokens=256)
    x = datagen.prefill_inputs(wl)
    if case == "zero_queries":
        x["qi"] = torch.zeros_like(x["qi"])
    if case == "negative_weights":
        x["w"] = -x["w"]          # every score <= 0; -0 and +0 must tie
    if case == "all_equal_keys":
        x["ki"] = torch.ones_like(x["ki"])
    if case == "strided_outliers":
        ki = torch.randint(-1, 2, x["ki"].shape, generator=torch.Generator().manual_seed(11)).float()
        blocks = torch.arange(wl.n_tokens) // wl.block
        for res in (1, 2):
            sel = (blocks % 4 == res)
            ki[sel] = 4.0 if res == 2 else 3.0
        x["ki"] = ki.to(torch.bfloat16)
        x["qi"] = x["qi"].abs()
    if case == "sample_sees_only_the_top":
        gen = torch.Generator().manual_seed(12)
        blocks = torch.arange(wl.n_tokens) // wl.block
        mag = torch.randint(1, 5, x["ki"].shape, generator=gen).float()
        sign = torch.where(blocks % 2 == 1, 1.0, -1.0).unsqueeze(1)
        x["ki"] = (mag * sign).to(torch.bfloat16)
        x["qi"] = x["qi"].abs()
        x["w"] = x["w"].abs()
    p = params_of(wl)
    ch = OracleChain(x, p)
    say(f"index_topk degenerate {case}")
    xd = to_dev(x)
    kbar = torch.from_numpy(ch.kbar.view(np.int16)).view(torch.bfloat16).cuda()
    topk = run_topk(sg, p, xd, kbar)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(topk.cpu().numpy(), ch.topk())


@pytest.mark.parametrize("name", ["tiny", "gqa_ragged", "b4_tile24", "b1_token", "tile1"])
def test_union_bit_exact(sg, name):
    wl = SMALL[name]
    p = params_of(wl)
    x = datagen.prefill_inputs(wl)
    ch = OracleChain(x, p)
    sel = ch.topk()
    want_mask, want_cnt = oracle.union(sel, p.n_tokens, p.block, p.union_tile)
    say(f"union {name} T={p.n_tiles} W={p.n_words}")
    umask = torch.empty((p.n_kv_heads, p.n_tiles, p.n_words), dtype=torch.int32, device="cuda")
    ucount = torch.empty((p.n_kv_heads, p.n_tiles), dtype=torch.int32, device="cuda")
    sg.sgqa_union(p, torch.from_numpy(sel).cuda(), umask, ucount)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(umask.cpu().numpy().view(np.uint32), want_mask)
    np.testing.assert_array_equal(ucount.cpu().numpy(), want_cnt)


@pytest.mark.parametrize("name", list(SMALL) + ["zero_queries", "negative_weights"])
def test_index_union_fused_bit_exact(sg, name):
    # The fused selection -> union path never writes topk; its mask must be the oracle's union of the
    # oracle's selections (and so equal to sgqa_index_topk + sgqa_union).
    wl = SMALL.get(name, SMALL["gqa_ragged"].replace(name=f"fused_{name}"))
    x = datagen.prefill_inputs(wl)
    if name == "zero_queries":
        x["qi"] = torch.zeros_like(x["qi"])
    if name == "negative_weights":
        x["w"] = -x["w"]
    p = params_of(wl)
    ch = OracleChain(x, p)
    want_mask, want_cnt = oracle.union(ch.topk(), p.n_tokens, p.block, p.union_tile)
    say(f"index_union {name} N={p.n_tokens} B={p.block} Tq={p.union_tile}")
    xd = to_dev(x)
    kbar = torch.from_numpy(ch.kbar.view(np.int16)).view(torch.bfloat16).cuda()
    umask = torch.full((p.n_kv_heads, p.n_tiles, p.n_words), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    ucount = torch.full((p.n_kv_heads, p.n_tiles), -7, dtype=torch.int32, device="cuda")
    sg.sgqa_index_union(p, xd["qi"], xd["w"], kbar, umask, ucount)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(umask.cpu().numpy().view(np.uint32), want_mask)
    np.testing.assert_array_equal(ucount.cpu().numpy(), want_cnt)


@pytest.mark.parametrize("name", list(SMALL))
def test_attend_within_tolerance(sg, name):
    wl = SMALL[name]
    p = params_of(wl)
    x = datagen.prefill_inputs(wl)
    ch = OracleChain(x, p)
    umask, ucount = oracle.union(ch.topk(), p.n_tokens, p.block, p.union_tile)
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([np.arange(0, 40), np.arange(p.n_tokens - 40, p.n_tokens),
                                     rng.integers(0, p.n_tokens, 300)])).astype(np.int32)
    want = oracle.attend(bits(x["q"]), bits(x["k"]), bits(x["v"]), umask, p.block, p.union_tile, rows=rows)
    say(f"attend {name} N={p.n_tokens} Hq={p.n_q_heads} G={p.n_kv_heads} B={p.block} Tq={p.union_tile}")
    xd = to_dev(x)
    out = torch.empty((p.n_tokens, p.n_q_heads, p.head_dim), dtype=torch.bfloat16, device="cuda")
    sg.sgqa_attend(p, xd["q"], xd["k"], xd["v"], torch.from_numpy(umask.view(np.int32)).cuda(),
                   torch.from_numpy(ucount).cuda(), out)
    torch.cuda.synchronize()
    assert_close_attention(out[torch.from_numpy(rows).long().cuda()], want, f"attend {name}")


@pytest.mark.parametrize("name", ["tiny", "gqa_ragged", "b4_tile24", "b16_iid", "tile1", "b64_r4"])
def test_attend_masked_within_tolerance(sg, name):
    # Masked-union variant: the union only decides what is gathered; each Q row attends its own
    # query's selection and own block (oracle: attend_sel, with no union at all).
    wl = SMALL[name]
    p = params_of(wl)
    x = datagen.prefill_inputs(wl)
    ch = OracleChain(x, p)
    sel = ch.topk()
    umask, ucount = oracle.union(sel, p.n_tokens, p.block, p.union_tile)
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([np.arange(0, 40), np.arange(p.n_tokens - 40, p.n_tokens),
                                     rng.integers(0, p.n_tokens, 300)])).astype(np.int32)
    want = oracle.attend_sel(bits(x["q"]), bits(x["k"]), bits(x["v"]), sel, p.block, rows=rows)
    say(f"attend_masked {name} N={p.n_tokens} Hq={p.n_q_heads} G={p.n_kv_heads} B={p.block} Tq={p.union_tile}")
    xd = to_dev(x)
    out = torch.empty((p.n_tokens, p.n_q_heads, p.head_dim), dtype=torch.bfloat16, device="cuda")
    ws = sg.workspace(p, sg.SGQA_OP_ATTEND_MASKED)
    sg.sgqa_attend_masked(p, xd["q"], xd["k"], xd["v"], torch.from_numpy(sel).cuda(),
                          torch.from_numpy(umask.view(np.int32)).cuda(), torch.from_numpy(ucount).cuda(), out, ws)
    torch.cuda.synchronize()
    assert_close_attention(out[torch.from_numpy(rows).long().cuda()], want, f"attend_masked {name}")
    if p.union_tile == 1:
        # One query per tile: the union is the query's own set, so both readings give the same bits.
        out1 = torch.empty_like(out)
        sg.sgqa_attend(p, xd["q"], xd["k"], xd["v"], torch.from_numpy(umask.view(np.int32)).cuda(),
                       torch.from_numpy(ucount).cuda(), out1)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), out1.view(torch.int16))


@pytest.mark.parametrize("name", ["gqa_ragged", "b4_tile24"])
def test_prefill_masked_end_to_end(sg, name):
    wl = SMALL[name]
    p = params_of(wl)
    x = datagen.prefill_inputs(wl)
    ch = OracleChain(x, p)
    want = oracle.attend_sel(bits(x["q"]), bits(x["k"]), bits(x["v"]), ch.topk(), p.block)
    say(f"prefill_masked {name}")
    xd = to_dev(x)
    out = torch.empty((p.n_tokens, p.n_q_heads, p.head_dim), dtype=torch.bfloat16, device="cuda")
    ws = sg.workspace(p, sg.SGQA_OP_PREFILL_MASKED)
    sg.sgqa_prefill_masked(p, xd["q"], xd["k"], xd["v"], xd["qi"], xd["w"], xd["ki"], out, ws)
    torch.cuda.synchronize()
    assert_close_attention(out, want, f"prefill_masked {name}")
    # The union reading of the same inputs differs (it attends extra blocks).
    out_u = torch.empty_like(out)
    sg.sgqa_prefill(p, xd["q"], xd["k"], xd["v"], xd["qi"], xd["w"], xd["ki"], out_u, sg.workspace(p, sg.SGQA_OP_PREFILL))
    torch.cuda.synchronize()
    assert (out_u.float() - out.float()).abs().max().item() > 1e-2


@pytest.mark.parametrize("name", ["tiny", "gqa_ragged", "b4_tile24", "b1_token"])
def test_prefill_end_to_end(sg, name):
    wl = SMALL[name]
    p = params_of(wl)
    x = datagen.prefill_inputs(wl)
    ch = OracleChain(x, p)
    umask, _ = oracle.union(ch.topk(), p.n_tokens, p.block, p.union_tile)
    want = oracle.attend(bits(x["q"]), bits(x["k"]), bits(x["v"]), umask, p.block, p.union_tile)
    say(f"prefill {name}")
    xd = to_dev(x)
    out = torch.empty((p.n_tokens, p.n_q_heads, p.head_dim), dtype=torch.bfloat16, device="cuda")
    ws = sg.workspace(p, sg.SGQA_OP_PREFILL)
    sg.sgqa_prefill(p, xd["q"], xd["k"], xd["v"], xd["qi"], xd["w"], xd["ki"], out, ws)
    torch.cuda.synchronize()
    assert_close_attention(out, want, f"prefill {name}")
    # Determinism: a second run gives the same bits.
    out2 = torch.empty_like(out)
    sg.sgqa_prefill(p, xd["q"], xd["k"], xd["v"], xd["qi"], xd["w"], xd["ki"], out2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("n", [1, 5, 8, 9, 63, 65, 130])
def test_prefill_short_sequences(sg, n):
    # Sequences shorter than one block up to a few chunks: no complete block at all (N < B, nothing
    # to compress or select), single-chunk unions, ragged last blocks and tiles, queries with no
    # candidate block (i < B).
    wl = datagen.PREFILL.replace(name=f"short_{n}", n_tokens=n, n_q_heads=16, n_kv_heads=2, block=8,
                                 topk_tokens=64, union_tile=16)
    p = params_of(wl)
    x = datagen.prefill_inputs(wl)
    ch = OracleChain(x, p)
    umask, _ = oracle.union(ch.topk(), p.n_tokens, p.block, p.union_tile)
    want = oracle.attend(bits(x["q"]), bits(x["k"]), bits(x["v"]), umask, p.block, p.union_tile)
    say(f"prefill short N={n}")
    xd = to_dev(x)
    out = torch.empty((p.n_tokens, p.n_q_heads, p.head_dim), dtype=torch.bfloat16, device="cuda")
    ws = sg.workspace(p, sg.SGQA_OP_PREFILL)
    sg.sgqa_prefill(p, xd["q"], xd["k"], xd["v"], xd["qi"], xd["w"], xd["ki"], out, ws)
    torch.cuda.synchronize()
    assert_close_attention(out, want, f"prefill short N={n}")
    # The masked-union reading of the same inputs: each row its own selection and own block.
    want_sel = oracle.attend_sel(bits(x["q"]), bits(x["k"]), bits(x["v"]), ch.topk(), p.block)
    out_m = torch.empty_like(out)
    sg.sgqa_prefill_masked(p, xd["q"], xd["k"], xd["v"], xd["qi"], xd["w"], xd["ki"], out_m,
                           sg.workspace(p, sg.SGQA_OP_PREFILL_MASKED))
    torch.cuda.synchronize()
    assert_close_attention(out_m, want_sel, f"prefill_masked short N={n}")


def test_prefill_dense_when_k_covers_context(sg):
    # k >= N: selection is everything, the path is dense causal GQA attention (oracle pinned to SDPA).
    wl = datagen.PREFILL.replace(name="dense_e2e", n_tokens=1024 + 8, n_q_heads=16, n_kv_heads=2,
                                 topk_tokens=2048, union_tile=64)
    p = params_of(wl)
    x = datagen.prefill_inputs(wl)
    full = np.full((2, p.n_tokens, p.kb), -1, np.int32)
    for i in range(p.n_tokens):
        c = i // p.block
        full[:, i, :c] = np.arange(c)
    umask, _ = oracle.union(full, p.n_tokens, p.block, p.union_tile)
    want = oracle.attend(bits(x["q"]), bits(x["k"]), bits(x["v"]), umask, p.block, p.union_tile)
    say("prefill dense")
    xd = to_dev(x)
    out = torch.empty((p.n_tokens, p.n_q_heads, p.head_dim), dtype=torch.bfloat16, device="cuda")
    ws = sg.workspace(p, sg.SGQA_OP_PREFILL)
    sg.sgqa_prefill(p, xd["q"], xd["k"], xd["v"], xd["qi"], xd["w"], xd["ki"], out, ws)
    torch.cuda.synchronize()
    assert_close_attention(out, want, "prefill dense")


@pytest.mark.parametrize("L,S,G,kb_tokens,B", [
    (203, 3, 2, 48, 8), (4096 + 5, 4, 8, 4096, 8), (9000, 2, 8, 2048, 8), (3000, 2, 1, 256, 4),
    (5, 2, 2, 48, 8),          # L < B: no candidate block, only the own block's tokens
    (9, 1, 2, 48, 8),          # exactly one candidate block
    (12 * 8 + 1, 2, 10, 4096, 8),  # K_B > c: every candidate selected; G = 10 is not a multiple of 8
    (150001, 1, 2, 1024, 1),   # c > 32768: the selection is reduced over segments, then picked again
    (20000, 1, 2, 2048, 1),    # K_B = 2048 > 1024 threads: no per-thread-maximum bound
])
def test_decode_matches_oracle(sg, L, S, G, kb_tokens, B):
    wl = datagen.DECODE.replace(name=f"dec_{L}_{S}_{G}", n_tokens=L, n_seqs=S, n_q_heads=8 * G, n_kv_heads=G,
                                topk_tokens=kb_tokens, block=B)
    p = params_of(wl)
    x = datagen.decode_inputs(wl)
    kbar = oracle.compress(bits(x["ki_cache"]), B)
    want_sel, want_out = oracle.decode(x["q"], x["k_cache"], x["v_cache"], kbar, x["qi"], x["w"], B, p.kb)
    say(f"decode L={L} S={S} G={G} kb={p.kb} B={B}")
    xd = to_dev(x)
    blk = torch.empty((S, L // B, 64), dtype=torch.bfloat16, device="cuda")
    sg.sgqa_compress(p, xd["ki_cache"], blk)
    out = torch.empty((S, p.n_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    topk = torch.empty((S, G, p.kb), dtype=torch.int32, device="cuda")
    ws = sg.workspace(p, sg.SGQA_OP_DECODE)
    sg.sgqa_decode(p, xd["q"], xd["k_cache"], xd["v_cache"], blk, xd["qi"], xd["w"], out, ws, topk_out=topk)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(blk), kbar)
    np.testing.assert_array_equal(topk.cpu().numpy(), want_sel)
    assert_close_attention(out, want_out, f"decode L={L}")


def test_decode_all_scores_tied(sg):
    # Zero indexer queries: every candidate scores 0, so the selection is the K_B lowest block ids
    # and the keys above the search's lower bound are far too many to compact.
    L, S, G, B = 40000, 2, 2, 8
    wl = datagen.DECODE.replace(name="dec_tied", n_tokens=L, n_seqs=S, n_q_heads=8 * G, n_kv_heads=G,
                                topk_tokens=4096, block=B)
    p = params_of(wl)
    x = datagen.decode_inputs(wl)
    x["qi"] = torch.zeros_like(x["qi"])
    kbar = oracle.compress(bits(x["ki_cache"]), B)
    want_sel, want_out = oracle.decode(x["q"], x["k_cache"], x["v_cache"], kbar, x["qi"], x["w"], B, p.kb)
    assert (want_sel == np.arange(p.kb, dtype=np.int32)).all()
    say("decode with every score tied")
    xd = to_dev(x)
    blk = torch.empty((S, L // B, 64), dtype=torch.bfloat16, device="cuda")
    sg.sgqa_compress(p, xd["ki_cache"], blk)
    out = torch.empty((S, p.n_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    topk = torch.empty((S, G, p.kb), dtype=torch.int32, device="cuda")
    ws = sg.workspace(p, sg.SGQA_OP_DECODE)
    sg.sgqa_decode(p, xd["q"], xd["k_cache"], xd["v_cache"], blk, xd["qi"], xd["w"], out, ws, topk_out=topk)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(topk.cpu().numpy(), want_sel)
    assert_close_attention(out, want_out, "decode tied")
