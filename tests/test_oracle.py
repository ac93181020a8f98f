"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Every check uses an independent route: the pages' printed figures, a hand-worked example, a
library routine (torch's bf16 rounding and scaled-dot-product attention), closed forms, invariants
of the definitions, or a brute force written here in numpy / plain Python.
Source of the definitions: "Inside Step 5 Preview", section "Sparse GQA" (paragraphs "Reducing
indexer's cost", "Efficient implementation of sparse attention", "Trade-off between top-k and
block size") and Figure 3.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import datagen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_bf16_bits_torch(x32: np.ndarray) -> np.ndarray:
    return bits(torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16))


# ------------------------------------------------------------------------------------ bf16 rounding

def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(4000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),   # binary32 subnormals
        (rng.standard_normal(2000) * 1e37).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, 3.4e38, -3.4e38, 1e-45], dtype=np.float32),
    ])
    # halfway cases: exactly between two bf16 neighbours (upper 16 bits + 0x8000)
    half = (rng.integers(0x0080, 0x7F00, 2000).astype(np.uint32) << 16 | 0x8000).view(np.float32)
    vals = np.concatenate([vals, half, -half])
    want = to_bf16_bits_torch(vals)
    got = np.array([orc.f64_to_bf16(float(x)) for x in vals], dtype=np.uint16)
    np.testing.assert_array_equal(got, want)


def test_bf16_rounding_hand_cases(orc):
    assert orc.f64_to_bf16(1.0) == 0x3F80
    assert orc.f64_to_bf16(1 + 2 ** -8) == 0x3F80           # tie -> even (1.0)
    assert orc.f64_to_bf16(1 + 3 * 2 ** -8) == 0x3F82       # tie -> even (1 + 2^-6)
    assert orc.f64_to_bf16(1 + 2 ** -8 + 2 ** -20) == 0x3F81  # above the tie
    assert orc.f64_to_bf16(-2.5) == 0xC020
    assert orc.f64_to_bf16(1e39) == 0x7F80
    assert orc.bf16_to_f64(0x4049) == 3.140625


# ------------------------------------------------------------------------------------ compress

def test_compress_hand_worked_example(orc):
    ex = json.load(open(os.path.join(GOLDEN, "hand_worked_example.json")))
    ki = to_bf16_bits_torch(np.array(ex["idx_k"], dtype=np.float32))
    kbar = orc.compress(ki, ex["block"])
    np.testing.assert_array_equal(f64(kbar), np.array(ex["block_keys"], dtype=np.float64))


def test_compress_block1_is_identity(orc):
    x = datagen.prefill_inputs(datagen.TINY.replace(n_tokens=300))
    ki = bits(x["ki"])
    np.testing.assert_array_equal(orc.compress(ki, 1), ki)


@pytest.mark.parametrize("B", [2, 4, 8, 16])
def test_compress_matches_numpy_mean(orc, B):
    rng = np.random.default_rng(B)
    N, dI = 8 * 37 + 5, 64   # a ragged tail that must not be compressed
    ki32 = rng.standard_normal((2, N, dI)).astype(np.float32)
    ki = to_bf16_bits_torch(ki32)
    got = orc.compress(ki, B)
    assert got.shape == (2, N // B, dI)
    vals = f64(ki)[:, : (N // B) * B].reshape(2, N // B, B, dI)
    mean = vals.sum(axis=2) / B                       # exact in fp64 for B <= 16 bf16 addends here
    m32 = mean.astype(np.float32)
    exact = m32.astype(np.float64) == mean           # skip the rare means that need > 24 bits
    want = to_bf16_bits_torch(m32)
    assert exact.mean() > 0.99
    np.testing.assert_array_equal(got[exact], want[exact])


def test_compress_integer_means_are_exact(orc):
    # Integer keys in [-4, 4]: every block mean m/B has at most 6 significant bits -> exact in bf16.
    x = datagen.prefill_inputs(datagen.TINY)
    ki = bits(x["ki"])
    got = f64(orc.compress(ki, 8))
    want = f64(ki).reshape(-1, 8, 64).mean(axis=1)
    np.testing.assert_array_equal(got, want)


# ------------------------------------------------------------------------------------ scores / top-k

def brute_scores(qi_row: np.ndarray, w_row: np.ndarray, kbar: np.ndarray, nc: int) -> np.ndarray:
    """Independent score: numpy matrix product in fp64, ReLU, weighted head sum."""
    dots = f64(qi_row) @ f64(kbar[:nc]).T            # [HI][nc]
    return (np.maximum(dots, 0.0) * w_row.astype(np.float64)[:, None]).sum(axis=0)


def brute_select(scores, kb: int) -> np.ndarray:
    order = sorted(range(len(scores)), key=lambda b: (-scores[b], b))
    chosen = sorted(order[:kb])
    return np.array(chosen + [-1] * (kb - len(chosen)), dtype=np.int32)


def test_topk_hand_worked_example(orc):
    ex = json.load(open(os.path.join(GOLDEN, "hand_worked_example.json")))
    B, kb = ex["block"], ex["topk_tokens"] // ex["block"]
    ki = to_bf16_bits_torch(np.array(ex["idx_k"], dtype=np.float32))
    qi = to_bf16_bits_torch(np.array(ex["idx_q"], dtype=np.float32)).reshape(8, 1, 1, 2)
    w = np.array(ex["idx_w"], dtype=np.float32)
    sel = orc.index_topk(qi, w, orc.compress(ki, B), B, kb)
    np.testing.assert_array_equal(sel[0], np.array(ex["topk"], dtype=np.int32))
    umask, ucount = orc.union(sel, 8, B, ex["union_tile"])
    for t, want_bits in enumerate(ex["union_mask_bits"]):
        assert [b for b in range(4) if (umask[0, t, 0] >> b) & 1] == want_bits
    np.testing.assert_array_equal(ucount[0], ex["union_count"])


@pytest.mark.parametrize("B,k", [(1, 16), (2, 8), (4, 32), (8, 64), (8, 8)])
def test_topk_matches_brute_force(orc, B, k):
    wl = datagen.Workload("bf", 160, 4, 2, 128, 4, 64, B, k, 4, weights="12", qi_mode="corr", rho=0.5)
    x = datagen.prefill_inputs(wl)
    qi, ki, w = bits(x["qi"]), bits(x["ki"]), x["w"].numpy()
    kbar = orc.compress(ki, B)
    kb = k // B
    sel = orc.index_topk(qi, w, kbar, B, kb)
    for g in range(2):
        for i in range(160):
            nc = i // B
            s = brute_scores(qi[i, g], w[g], kbar, nc)
            np.testing.assert_array_equal(sel[g, i], brute_select(list(s), kb), err_msg=f"g={g} i={i}")


def test_scores_match_brute_force_exactly(orc):
    x = datagen.prefill_inputs(datagen.TINY.replace(n_tokens=512))
    qi, ki, w = bits(x["qi"]), bits(x["ki"]), x["w"].numpy()
    kbar = orc.compress(ki, 8)
    s = orc.block_scores(qi[511, 0], w[0], kbar, 63)
    np.testing.assert_array_equal(s, brute_scores(qi[511, 0], w[0], kbar, 63))


def test_topk_zero_queries_pick_lowest_ids(orc):
    # All scores are +0 -> ties everywhere -> the K_B lowest block ids.
    N, B, kb = 256, 8, 5
    qi = np.zeros((N, 1, 4, 64), dtype=np.uint16)
    ki = bits(datagen.prefill_inputs(datagen.TINY.replace(n_tokens=N))["ki"])
    sel = orc.index_topk(qi, np.ones((1, 4), np.float32), orc.compress(ki, B), B, kb)
    for i in range(N):
        m = min(kb, i // B)
        np.testing.assert_array_equal(sel[0, i, :m], np.arange(m))
        assert (sel[0, i, m:] == -1).all()


def test_topk_all_negative_dots_pick_lowest_ids(orc):
    N, B, kb = 128, 4, 3
    ki = to_bf16_bits_torch(np.ones((N, 64), np.float32))
    qi = to_bf16_bits_torch(-np.ones((N, 1, 4, 64), np.float32))
    sel = orc.index_topk(qi, np.ones((1, 4), np.float32), orc.compress(ki, B), B, kb)
    np.testing.assert_array_equal(sel[0, -1], np.arange(kb))


def test_topk_k_at_least_context_selects_everything(orc):
    wl = datagen.TINY.replace(n_tokens=200, topk_tokens=256)
    x = datagen.prefill_inputs(wl)
    sel = orc.index_topk(bits(x["qi"]), x["w"].numpy(), orc.compress(bits(x["ki"]), 8), 8, 32)
    for i in range(200):
        c = i // 8
        np.testing.assert_array_equal(sel[0, i, :c], np.arange(c))
        assert (sel[0, i, c:] == -1).all()


def test_topk_invariant_to_head_permutation_and_weight_scale(orc):
    wl = datagen.PREFILL.replace(n_tokens=600, n_q_heads=16, n_kv_heads=2, topk_tokens=128)
    x = datagen.prefill_inputs(wl)
    qi, ki, w = bits(x["qi"]), bits(x["ki"]), x["w"].numpy()
    kbar = orc.compress(ki, 8)
    base = orc.index_topk(qi, w, kbar, 8, 16)
    perm = [2, 0, 3, 1]
    np.testing.assert_array_equal(orc.index_topk(np.ascontiguousarray(qi[:, :, perm]),
                                                 np.ascontiguousarray(w[:, perm]), kbar, 8, 16), base)
    np.testing.assert_array_equal(orc.index_topk(qi, w * 2, kbar, 8, 16), base)


def test_block1_reduces_to_token_topk(orc):
    # With B = 1 the block keys are the index keys and candidates are the tokens j < i.
    wl = datagen.PREFILL.replace(n_tokens=300, n_q_heads=8, n_kv_heads=1, block=1, topk_tokens=20)
    x = datagen.prefill_inputs(wl)
    qi, ki, w = bits(x["qi"]), bits(x["ki"]), x["w"].numpy()
    sel = orc.index_topk(qi, w, orc.compress(ki, 1), 1, 20)
    for i in range(300):
        dots = f64(qi[i, 0]) @ f64(ki[:i]).T
        s = (np.maximum(dots, 0) * w[0][:, None]).sum(axis=0)
        np.testing.assert_array_equal(sel[0, i], brute_select(list(s), 20))


def test_scored_pairs_closed_form_and_pages_ratio(orc):
    figs = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))
    B = figs["block_size"]["value"]
    for N, Bx in [(1, 8), (7, 8), (8, 8), (1000, 8), (32768, 8), (32768, 1), (131072, 8)]:
        q, r = divmod(N, Bx)
        assert orc.scored_pairs(N, Bx) == Bx * q * (q - 1) // 2 + r * q
    ratio = orc.scored_pairs(32768, 1) / orc.scored_pairs(32768, B)
    assert abs(ratio - figs["indexer_topk_cost_reduction"]["value"]) < 0.01   # 8.0017
    assert figs["topk_tokens"]["value"] // B == figs["topk_blocks"]["value"]


# ------------------------------------------------------------------------------------ union

def test_union_matches_brute_force_sets(orc):
    wl = datagen.PREFILL.replace(n_tokens=777, n_q_heads=16, n_kv_heads=2, topk_tokens=96, union_tile=24)
    x = datagen.prefill_inputs(wl)
    B, kb, Tq, N = 8, 12, 24, 777
    sel = orc.index_topk(bits(x["qi"]), x["w"].numpy(), orc.compress(bits(x["ki"]), B), B, kb)
    umask, ucount = orc.union(sel, N, B, Tq)
    T = (N + Tq - 1) // Tq
    assert umask.shape == (2, T, ((N + B - 1) // B + 31) // 32)
    for g in range(2):
        for t in range(T):
            want = set()
            for i in range(t * Tq, min(N, (t + 1) * Tq)):
                want |= {int(b) for b in sel[g, i] if b >= 0} | {i // B}
            got = {b for b in range(umask.shape[2] * 32) if (umask[g, t, b // 32] >> (b % 32)) & 1}
            assert got == want
            assert ucount[g, t] == len(want)


def test_union_tile1_is_selection_plus_own_block(orc):
    wl = datagen.TINY.replace(n_tokens=256, topk_tokens=40)
    x = datagen.prefill_inputs(wl)
    sel = orc.index_topk(bits(x["qi"]), x["w"].numpy(), orc.compress(bits(x["ki"]), 8), 8, 5)
    umask, ucount = orc.union(sel, 256, 8, 1)
    for i in range(256):
        want = {int(b) for b in sel[0, i] if b >= 0} | {i // 8}
        got = {b for b in range(32) if (umask[0, i, 0] >> b) & 1}
        assert got == want and ucount[0, i] == len(want)


# ------------------------------------------------------------------------------------ attention

def _small_prefill(N=96, Hq=4, G=2, B=4, k=16, Tq=8, seed_name="att"):
    wl = datagen.PREFILL.replace(name=seed_name, n_tokens=N, n_q_heads=Hq, n_kv_heads=G, block=B,
                                 topk_tokens=k, union_tile=Tq, rho=0.5)
    return wl, datagen.prefill_inputs(wl)


def brute_attention(q, k, v, allowed, scale):
    """q [Hq][D], k/v [N][D] of the head's group, allowed [N] bool -> [Hq][D] (numpy fp64)."""
    lg = scale * (f64(q) @ f64(k).T)
    lg = np.where(allowed[None, :], lg, -np.inf)
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return p @ f64(v)


def test_attend_matches_explicit_mask(orc):
    wl, x = _small_prefill()
    N, B, Tq, kb, r = 96, 4, 8, 4, 2
    q, k, v = bits(x["q"]), bits(x["k"]), bits(x["v"])
    sel = orc.index_topk(bits(x["qi"]), x["w"].numpy(), orc.compress(bits(x["ki"]), B), B, kb)
    umask, _ = orc.union(sel, N, B, Tq)
    out = orc.attend(q, k, v, umask, B, Tq)
    scale = 1 / math.sqrt(128)
    for i in range(N):
        t = i // Tq
        for g in range(2):
            blocks = {b for b in range(N // B) if (umask[g, t, b // 32] >> (b % 32)) & 1}
            allowed = np.array([(j <= i) and (j // B in blocks) for j in range(N)])
            want = brute_attention(q[i, g * r:(g + 1) * r], k[g], v[g], allowed, scale)
            np.testing.assert_allclose(out[i, g * r:(g + 1) * r], want, rtol=1e-12, atol=1e-12)


def test_attend_dense_when_k_covers_context_equals_sdpa(orc):
    # k >= N: every candidate is selected, so the path is dense causal GQA attention.
    wl, x = _small_prefill(N=64, Hq=4, G=2, B=8, k=64, Tq=16, seed_name="dense")
    q, k, v = bits(x["q"]), bits(x["k"]), bits(x["v"])
    sel = orc.index_topk(bits(x["qi"]), x["w"].numpy(), orc.compress(bits(x["ki"]), 8), 8, 8)
    umask, _ = orc.union(sel, 64, 8, 16)
    out = orc.attend(q, k, v, umask, 8, 16)
    qt = torch.from_numpy(f64(q)).permute(1, 0, 2)                 # [Hq][N][D]
    kt = torch.from_numpy(f64(k)).repeat_interleave(2, dim=0)      # [Hq][N][D]
    vt = torch.from_numpy(f64(v)).repeat_interleave(2, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True).permute(1, 0, 2)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_attend_zero_query_is_mean_of_visible_values_and_first_row_is_v0(orc):
    wl, x = _small_prefill(N=80, seed_name="zeroq")
    N, B, Tq = 80, 4, 8
    q = np.zeros((N, 4, 128), dtype=np.uint16)
    k, v = bits(x["k"]), bits(x["v"])
    sel = orc.index_topk(bits(x["qi"]), x["w"].numpy(), orc.compress(bits(x["ki"]), B), B, 4)
    umask, _ = orc.union(sel, N, B, Tq)
    out = orc.attend(q, k, v, umask, B, Tq)
    for i in [0, 7, 33, 79]:
        for g in range(2):
            t = i // Tq
            toks = [j for j in range(i + 1) if (umask[g, t, (j // B) // 32] >> ((j // B) % 32)) & 1]
            want = f64(v[g][toks]).mean(axis=0)
            np.testing.assert_allclose(out[i, 2 * g], want, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(out[0, :2], np.repeat(f64(v[0][:1]), 2, axis=0), atol=0)


def test_attend_sel_matches_brute_force_per_query_sets(orc):
    # Each query over Sel(i,g) and its own block, from an explicit numpy mask built from the
    # selection (no union at all); a larger union tile must not change anything.
    wl, x = _small_prefill(seed_name="attsel")
    N, B, kb, r = 96, 4, 4, 2
    q, k, v = bits(x["q"]), bits(x["k"]), bits(x["v"])
    sel = orc.index_topk(bits(x["qi"]), x["w"].numpy(), orc.compress(bits(x["ki"]), B), B, kb)
    out = orc.attend_sel(q, k, v, sel, B)
    scale = 1 / math.sqrt(128)
    for i in range(N):
        for g in range(2):
            blocks = {int(b) for b in sel[g, i] if b >= 0} | {i // B}
            allowed = np.array([(j <= i) and (j // B in blocks) for j in range(N)])
            want = brute_attention(q[i, g * r:(g + 1) * r], k[g], v[g], allowed, scale)
            np.testing.assert_allclose(out[i, g * r:(g + 1) * r], want, rtol=1e-12, atol=1e-12)


def test_attend_sel_is_union_attention_at_tile_1_and_differs_at_larger_tiles(orc):
    # With one query per tile the union is Sel(i,g) plus the own block, so both readings agree; with
    # a larger tile the union reading attends extra blocks (the two readings differ).
    wl, x = _small_prefill(N=128, seed_name="attsel2")
    N, B, kb = 128, 4, 4
    q, k, v = bits(x["q"]), bits(x["k"]), bits(x["v"])
    sel = orc.index_topk(bits(x["qi"]), x["w"].numpy(), orc.compress(bits(x["ki"]), B), B, kb)
    out = orc.attend_sel(q, k, v, sel, B)
    m1, _ = orc.union(sel, N, B, 1)
    np.testing.assert_allclose(out, orc.attend(q, k, v, m1, B, 1), rtol=1e-12, atol=1e-13)
    m8, _ = orc.union(sel, N, B, 8)
    assert np.abs(out - orc.attend(q, k, v, m8, B, 8)).max() > 1e-3


def test_attend_sel_dense_when_k_covers_context_equals_sdpa(orc):
    wl, x = _small_prefill(N=64, Hq=4, G=2, B=8, k=64, Tq=16, seed_name="densesel")
    q, k, v = bits(x["q"]), bits(x["k"]), bits(x["v"])
    sel = orc.index_topk(bits(x["qi"]), x["w"].numpy(), orc.compress(bits(x["ki"]), 8), 8, 8)
    out = orc.attend_sel(q, k, v, sel, 8)
    qt = torch.from_numpy(f64(q)).permute(1, 0, 2)
    kt = torch.from_numpy(f64(k)).repeat_interleave(2, dim=0)
    vt = torch.from_numpy(f64(v)).repeat_interleave(2, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True).permute(1, 0, 2)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-10, atol=1e-12)


def _torch_attention_grads(q, k, v, dout, allowed, r, scale):
    """fp64 autograd of softmax attention with a boolean mask [N][N] per group (allowed[g]);
    q/dout [N][Hq][D], k/v [G][N][D] (bf16 bits) -> dq, dk, dv as numpy fp64."""
    qt = torch.from_numpy(f64(q)).permute(1, 0, 2).clone().requires_grad_(True)   # [Hq][N][D]
    kt = torch.from_numpy(f64(k)).clone().requires_grad_(True)                    # [G][N][D]
    vt = torch.from_numpy(f64(v)).clone().requires_grad_(True)
    mask = torch.from_numpy(np.repeat(allowed, r, axis=0))                        # [Hq][N][N]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt.repeat_interleave(r, dim=0),
                                                         vt.repeat_interleave(r, dim=0), attn_mask=mask, scale=scale)
    o.backward(torch.from_numpy(f64(dout)).permute(1, 0, 2))
    return qt.grad.permute(1, 0, 2).numpy(), kt.grad.numpy(), vt.grad.numpy()


def test_attend_bwd_matches_torch_autograd_on_union_masks(orc):
    wl, x = _small_prefill(seed_name="bwd")
    N, B, Tq, kb, r, G = 96, 4, 8, 4, 2, 2
    q, k, v = bits(x["q"]), bits(x["k"]), bits(x["v"])
    dout = bits(torch.randn((N, 4, 128), generator=torch.Generator().manual_seed(3)).to(torch.bfloat16))
    sel = orc.index_topk(bits(x["qi"]), x["w"].numpy(), orc.compress(bits(x["ki"]), B), B, kb)
    umask, _ = orc.union(sel, N, B, Tq)
    dq, dk, dv = orc.attend_bwd(q, k, v, umask, dout, B, Tq)
    allowed = np.zeros((G, N, N), dtype=bool)
    for g in range(G):
        for i in range(N):
            t = i // Tq
            for j in range(i + 1):
                allowed[g, i, j] = (umask[g, t, (j // B) // 32] >> ((j // B) % 32)) & 1
    tq, tk, tv = _torch_attention_grads(q, k, v, dout, allowed, r, 1 / math.sqrt(128))
    np.testing.assert_allclose(dq, tq, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dk, tk, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dv, tv, rtol=1e-9, atol=1e-11)
    # A key block outside every union that could see it gets no gradient at all.
    seen = np.zeros((G, N), dtype=bool)
    for g in range(G):
        seen[g] = allowed[g].any(axis=0)
    assert (dk[~seen] == 0).all() and (dv[~seen] == 0).all()


def test_attend_bwd_part_equals_the_whole_gradient(orc):
    # The subset form (sampled dq rows, one group's key range) is the full gradient's arithmetic
    # term for term, so it must reproduce the full result exactly, for every group and for key
    # ranges that start and end inside blocks.
    wl, x = _small_prefill(seed_name="bwd")
    N, B, Tq, kb = 96, 4, 8, 4
    q, k, v = bits(x["q"]), bits(x["k"]), bits(x["v"])
    dout = bits(torch.randn((N, 4, 128), generator=torch.Generator().manual_seed(3)).to(torch.bfloat16))
    sel = orc.index_topk(bits(x["qi"]), x["w"].numpy(), orc.compress(bits(x["ki"]), B), B, kb)
    umask, _ = orc.union(sel, N, B, Tq)
    dq, dk, dv = orc.attend_bwd(q, k, v, umask, dout, B, Tq)
    rows = np.array([0, 5, 17, 63, N - 1], dtype=np.int32)
    for g0, lo, hi in ((0, 0, N), (1, 37, 59), (1, N - 3, N), (0, 20, 20)):
        pq, pk, pv = orc.attend_bwd_part(q, k, v, umask, dout, B, Tq, rows, g0, lo, hi)
        np.testing.assert_array_equal(pq, dq[rows])
        np.testing.assert_array_equal(pk, dk[g0, lo:hi])
        np.testing.assert_array_equal(pv, dv[g0, lo:hi])


def test_attend_bwd_dense_equals_causal_sdpa_autograd(orc):
    wl, x = _small_prefill(N=64, Hq=4, G=2, B=8, k=64, Tq=16, seed_name="bwddense")
    q, k, v = bits(x["q"]), bits(x["k"]), bits(x["v"])
    dout = bits(torch.randn((64, 4, 128), generator=torch.Generator().manual_seed(4)).to(torch.bfloat16))
    sel = orc.index_topk(bits(x["qi"]), x["w"].numpy(), orc.compress(bits(x["ki"]), 8), 8, 8)
    umask, _ = orc.union(sel, 64, 8, 16)
    dq, dk, dv = orc.attend_bwd(q, k, v, umask, dout, 8, 16)
    causal = np.tril(np.ones((64, 64), dtype=bool))
    tq, tk, tv = _torch_attention_grads(q, k, v, dout, np.stack([causal, causal]), 2, 1 / math.sqrt(128))
    np.testing.assert_allclose(dq, tq, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dk, tk, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dv, tv, rtol=1e-9, atol=1e-11)


# ------------------------------------------------------------------------------------ decode

def test_decode_equals_prefill_last_row_without_union(orc):
    L, B, k = 203, 8, 48
    wl = datagen.DECODE.replace(name="dec_small", n_tokens=L, n_seqs=3, n_q_heads=8, n_kv_heads=2,
                                topk_tokens=k)
    x = datagen.decode_inputs(wl)
    kbar = orc.compress(bits(x["ki_cache"]), B)
    topk, out = orc.decode(x["q"], x["k_cache"], x["v_cache"], kbar, x["qi"], x["w"], B, k // B)
    for s in range(3):
        # The same sequence as a prefill whose last query is the decode query; Tq = 1.
        qi = np.zeros((L, 2, 4, 64), dtype=np.uint16)
        qi[L - 1] = bits(x["qi"][s])
        q = np.zeros((L, 8, 128), dtype=np.uint16)
        q[L - 1] = bits(x["q"][s])
        sel = orc.index_topk(qi, x["w"], kbar[s], B, k // B, rows=[L - 1])
        np.testing.assert_array_equal(topk[s], sel[:, 0])
        full = np.full((2, L, k // B), -1, dtype=np.int32)
        full[:, L - 1] = sel[:, 0]
        umask, _ = orc.union(full, L, B, 1)
        ref = orc.attend(q, bits(x["k_cache"][s]), bits(x["v_cache"][s]), umask, B, 1, rows=[L - 1])
        np.testing.assert_allclose(out[s], ref[0], rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------------------------ coverage

def test_coverage_hand_example(orc):
    # G = 1, N = 4, B = 2, rows i >= 2 only.
    sel1 = np.array([[[-1], [0], [1], [2]]], dtype=np.int32)
    sel1[0, 3, 0] = 0
    selb = np.array([[[-1], [-1], [-1], [0]]], dtype=np.int32)
    # i=2: T1={1,2}, TB = own-block tokens {2} -> 0.5 ; i=3: T1={0,3}, TB={0,1,2,3} -> 1.0
    assert orc.coverage(sel1, selb, 2, i_min=2) == pytest.approx(0.75)


def test_coverage_brute_force_and_dense_case(orc):
    wl = datagen.PREFILL.replace(n_tokens=256, n_q_heads=8, n_kv_heads=1)
    x = datagen.prefill_inputs(wl)
    qi, ki, w = bits(x["qi"]), bits(x["ki"]), x["w"].numpy()
    s1 = orc.index_topk(qi, w, orc.compress(ki, 1), 1, 24)
    s8 = orc.index_topk(qi, w, orc.compress(ki, 8), 8, 6)
    want = []
    for i in range(40, 256):
        t1 = {int(j) for j in s1[0, i] if j >= 0} | {i}
        tb = {int(b) * 8 + j for b in s8[0, i] if b >= 0 for j in range(8)} | set(range((i // 8) * 8, i + 1))
        want.append(len(t1 & tb) / len(t1))
    assert orc.coverage(s1, s8, 8, i_min=40) == pytest.approx(float(np.mean(want)), abs=1e-12)
    # Both selections dense (k >= context): everything is covered.
    d1 = orc.index_topk(qi, w, orc.compress(ki, 1), 1, 256)
    d8 = orc.index_topk(qi, w, orc.compress(ki, 8), 8, 32)
    assert orc.coverage(d1, d8, 8) == 1.0


# ------------------------------------------------------------------------------------ FP8 K/V decode

def test_fp8_e4m3_codes(orc):
    # Hand values from the format's definition, then all 256 codes against torch's float8_e4m3fn.
    assert orc.fp8_e4m3_to_f64(0x38) == 1.0
    assert orc.fp8_e4m3_to_f64(0x7E) == 448.0
    assert orc.fp8_e4m3_to_f64(0x01) == 2.0 ** -9
    assert orc.fp8_e4m3_to_f64(0x08) == 2.0 ** -6
    assert orc.fp8_e4m3_to_f64(0xC4) == -3.0
    z = orc.fp8_e4m3_to_f64(0x80)
    assert z == 0.0 and np.signbit(z)
    assert np.isnan(orc.fp8_e4m3_to_f64(0x7F)) and np.isnan(orc.fp8_e4m3_to_f64(0xFF))
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([orc.fp8_e4m3_to_f64(c) for c in range(256)])
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])


def _fp8_exact_case(seed=11):
    """Small decode inputs whose K/V are FP8 codes; returns codes and their bf16 image (exact)."""
    wl = datagen.DECODE.replace(name="orc_fp8", n_tokens=300, n_seqs=2, n_q_heads=16, n_kv_heads=2,
                                topk_tokens=64, block=8)
    x = datagen.decode_inputs(wl)
    g = torch.Generator().manual_seed(seed)
    # codes with exponent fields 1..13 (normal, |v| <= 240): exactly representable in bf16
    def codes(shape):
        e = torch.randint(1, 14, shape, generator=g)
        m = torch.randint(0, 8, shape, generator=g)
        sg = torch.randint(0, 2, shape, generator=g)
        return (sg * 128 + e * 8 + m).to(torch.uint8)
    k8 = codes(x["k_cache"].shape)
    v8 = codes(x["v_cache"].shape)
    return wl, x, k8, v8


def test_decode_fp8_reduces_to_bf16_decode(orc):
    # Power-of-two scales keep code * scale exact in bf16, so orc_decode_f8 must equal orc_decode on
    # the dequantized caches. Different key and value scales catch a swapped scale.
    wl, x, k8, v8 = _fp8_exact_case()
    S, G = wl.n_seqs, wl.n_kv_heads
    kv_scale = torch.tensor([[[0.5, 4.0], [2.0, 0.25]]] * S, dtype=torch.float32)[:, :G]
    kb16 = (k8.view(torch.float8_e4m3fn).float() * kv_scale[:, :, 0, None, None]).to(torch.bfloat16)
    vb16 = (v8.view(torch.float8_e4m3fn).float() * kv_scale[:, :, 1, None, None]).to(torch.bfloat16)
    assert torch.equal(kb16.float(), k8.view(torch.float8_e4m3fn).float() * kv_scale[:, :, 0, None, None])
    kbar = orc.compress(bits(x["ki_cache"]), wl.block)
    kb = wl.topk_tokens // wl.block
    sel8, out8 = orc.decode_fp8(x["q"], k8, v8, kv_scale, kbar, x["qi"], x["w"], wl.block, kb)
    sel, out = orc.decode(x["q"], kb16, vb16, kbar, x["qi"], x["w"], wl.block, kb)
    np.testing.assert_array_equal(sel8, sel)
    np.testing.assert_allclose(out8, out, rtol=0, atol=1e-12)
