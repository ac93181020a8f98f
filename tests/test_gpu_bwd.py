"""Attention gradient on the GPU (sgqa_attend_fwd + sgqa_attend_bwd) against the oracle's attend_bwd.

Bar: the gradients are sums of many bf16-rounded products (P and dS enter the matrix cores as
bf16, as do q, k, v, dout), so they are compared relative to each tensor's scale: with s = the
largest |reference| of the tensor, max |got - ref| <= 2e-2 s and mean |got - ref| <= 2e-3 s.
A bf16 operand carries a relative rounding error of at most 2^-9 ~ 2e-3; a sum of n such terms with
cancellation (the dS of a row sum to 0) keeps its absolute error near 2^-9 * sqrt(n) * term size,
well inside 2e-2 s for the sizes here. Full-size runs check exact invariants instead.
"""
import os

import numpy as np
import pytest
import torch

import datagen
import oracle
from tests.gpu_common import OracleChain, bits, bf16_to_f64, params_of, say, to_dev

pytestmark = pytest.mark.gpu

MAX_REL = 2e-2
MEAN_REL = 2e-3


# Backward cases: several tiles and ragged tails for every block size of interest, sized so that
# the fp64 oracle gradient takes seconds.
BWD = {
    "tiny": datagen.TINY,
    "g2_b8": datagen.PREFILL.replace(name="bwd_g2_b8", n_tokens=1200 + 5, n_q_heads=16, n_kv_heads=2,
                                     topk_tokens=256, union_tile=64),
    "b4_tile24": datagen.PREFILL.replace(name="bwd_b4", n_tokens=900, n_q_heads=16, n_kv_heads=2, block=4,
                                         topk_tokens=128, union_tile=24),
    "b1_token": datagen.PREFILL.replace(name="bwd_b1", n_tokens=600, n_q_heads=8, n_kv_heads=1, block=1,
                                        topk_tokens=64, union_tile=16),
    "b16_iid": datagen.PREFILL.replace(name="bwd_b16", n_tokens=1000 + 17, n_q_heads=32, n_kv_heads=4, block=16,
                                       topk_tokens=256, union_tile=32, qi_mode="iid"),
    "tile1": datagen.PREFILL.replace(name="bwd_t1", n_tokens=500, n_q_heads=8, n_kv_heads=1, topk_tokens=64,
                                     union_tile=1),
    "b64_r4": datagen.PREFILL.replace(name="bwd_b64", n_tokens=1100 + 3, n_q_heads=16, n_kv_heads=4, block=64,
                                      topk_tokens=256, union_tile=128),
    # Shorter than one block, and one key past a chunk.
    "short_5": datagen.PREFILL.replace(name="bwd_short5", n_tokens=5, n_q_heads=16, n_kv_heads=2,
                                       topk_tokens=64, union_tile=16),
    "short_65": datagen.PREFILL.replace(name="bwd_short65", n_tokens=65, n_q_heads=16, n_kv_heads=2,
                                        topk_tokens=64, union_tile=16),
}


@pytest.fixture(scope="module")
def sg():
    import block_sparse_long_sgqa_amd as sg

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sg.lib()
    return sg


def assert_close_grad(got_bf16, want, what):
    got = bf16_to_f64(bits(got_bf16)).reshape(want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite"
    scale = max(1e-6, float(np.abs(want).max()))
    err = np.abs(got - want)
    say(f"{what}: scale={scale:.3e} max_rel={err.max() / scale:.3e} mean_rel={err.mean() / scale:.3e}")
    assert err.max() <= MAX_REL * scale, f"{what}: max error {err.max()} (scale {scale})"
    assert err.mean() <= MEAN_REL * scale, f"{what}: mean error {err.mean()} (scale {scale})"


def run_fwd_bwd(sg, p, xd, umask, ucount, dout):
    N, Hq, G, D = p.n_tokens, p.n_q_heads, p.n_kv_heads, p.head_dim
    out = torch.empty((N, Hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((N, Hq), dtype=torch.float32, device="cuda")
    sg.sgqa_attend_fwd(p, xd["q"], xd["k"], xd["v"], umask, ucount, out, lse)
    dq = torch.empty((N, Hq, D), dtype=torch.bfloat16, device="cuda")
    dk = torch.empty((G, N, D), dtype=torch.bfloat16, device="cuda")
    dv = torch.empty((G, N, D), dtype=torch.bfloat16, device="cuda")
    ws = sg.workspace(p, sg.SGQA_OP_ATTEND_BWD)
    sg.sgqa_attend_bwd(p, xd["q"], xd["k"], xd["v"], umask, ucount, out, lse, dout, dq, dk, dv, ws)
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


# The two dk/dv designs: tile-major (per-tile partial rows summed in tile order; the default where
# its batches stay few), the same with the smallest batches the plan allows (many batches, so the
# ordered sum runs across batch boundaries), and key-major (the fallback for the longest contexts).
MODES = {"tile": {}, "tile_batched": {"SGQA_BWD_BATCH_ROWS": "1"}, "key": {"SGQA_BWD_PATH": "key"}}


class bwd_mode:
    """Sets the library's backward-path environment variables for the duration of a block."""

    def __init__(self, mode):
        self.env = MODES[mode]

    def __enter__(self):
        for k in ("SGQA_BWD_PATH", "SGQA_BWD_BATCH_ROWS"):
            os.environ.pop(k, None)
        os.environ.update(self.env)

    def __exit__(self, *a):
        for k in self.env:
            os.environ.pop(k, None)


@pytest.mark.parametrize("name", list(BWD))
def test_attend_bwd_matches_oracle(sg, name):
    wl = BWD[name]
    p = params_of(wl)
    x = datagen.prefill_inputs(wl)
    ch = OracleChain(x, p)
    umask, ucount = oracle.union(ch.topk(), p.n_tokens, p.block, p.union_tile)
    g = torch.Generator().manual_seed(7)
    dout = torch.randn((p.n_tokens, p.n_q_heads, p.head_dim), generator=g).to(torch.bfloat16)
    say(f"attend_bwd {name} N={p.n_tokens} Hq={p.n_q_heads} G={p.n_kv_heads} B={p.block} Tq={p.union_tile}")
    want_dq, want_dk, want_dv = oracle.attend_bwd(bits(x["q"]), bits(x["k"]), bits(x["v"]), umask, bits(dout),
                                                  p.block, p.union_tile)
    xd = to_dev(x)
    um = torch.from_numpy(umask.view(np.int32)).cuda()
    uc = torch.from_numpy(ucount).cuda()
    for mode in MODES:
        say(f"attend_bwd {name}: dk/dv mode {mode}")
        with bwd_mode(mode):
            out, lse, dq, dk, dv = run_fwd_bwd(sg, p, xd, um, uc, dout.cuda())
            # The forward with lse is the forward.
            ref = torch.empty_like(out)
            sg.sgqa_attend(p, xd["q"], xd["k"], xd["v"], um, uc, ref)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
            assert_close_grad(dq, want_dq, f"dq {name} {mode}")
            assert_close_grad(dk, want_dk, f"dk {name} {mode}")
            assert_close_grad(dv, want_dv, f"dv {name} {mode}")
            # Deterministic: a second run gives the same bits.
            _, _, dq2, dk2, dv2 = run_fwd_bwd(sg, p, xd, um, uc, dout.cuda())
            for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
                assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# Full-size checks: key ranges near the end (their rows span many tiles, so the dk/dv kernel walks
# long tile lists) and sampled dq rows, against the oracle's gradient on that subset.
FULL_KEYS = {"prefill_32k": 4096 - 3, "long_prefill_128k": 2048 - 3}


@pytest.mark.parametrize("name", ["prefill_32k", "long_prefill_128k"])
def test_attend_bwd_full_size(sg, name):
    wl = datagen.WORKLOADS[name]
    p = params_of(wl)
    N, Hq, G, D, Tq = p.n_tokens, p.n_q_heads, p.n_kv_heads, p.head_dim, p.union_tile
    x = datagen.prefill_inputs(wl, device="cuda")
    say(f"attend_bwd {name}: selection and union")
    umask = torch.empty((G, p.n_tiles, p.n_words), dtype=torch.int32, device="cuda")
    ucount = torch.empty((G, p.n_tiles), dtype=torch.int32, device="cuda")
    blk = torch.empty((N // p.block, p.idx_dim), dtype=torch.bfloat16, device="cuda")
    sg.sgqa_compress(p, x["ki"], blk)
    sg.sgqa_index_union(p, x["qi"], x["w"], blk, umask, ucount)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    dout = torch.randn((N, Hq, D), generator=gen, device="cuda").to(torch.bfloat16)
    say(f"attend_bwd {name}: forward + backward")
    out, lse, dq, dk, dv = run_fwd_bwd(sg, p, x, umask, ucount, dout)
    # The key-major design on the same inputs: every key's gradient agrees with the tile-major
    # one (both sum the same products in fp32, in different orders).
    with bwd_mode("key"):
        say(f"attend_bwd {name}: key-major dk/dv")
        _, _, dq_k, dk_k, dv_k = run_fwd_bwd(sg, p, x, umask, ucount, dout)
    assert torch.equal(dq.view(torch.int16), dq_k.view(torch.int16))
    for a, b, what in ((dk, dk_k, "dk"), (dv, dv_k, "dv")):
        scale = a.float().abs().max().item()
        err = (a.float() - b.float()).abs()
        say(f"{what} tile-major vs key-major: max {err.max().item() / scale:.3e} mean {err.mean().item() / scale:.3e}")
        assert err.max().item() <= 1e-2 * scale and err.mean().item() <= 1e-4 * scale
    del dq_k, dk_k, dv_k

    # Invariants over every key: sum_j dv[g][j] = sum over the group's rows of dout (each row's p
    # sums to 1), and sum_j dk[g][j] = 0 (each row's dS sums to 0), to within the bf16 rounding.
    r = Hq // G
    want_dv = dout.float().view(N, G, r, D).sum(dim=(0, 2))  # [G][D]
    got_dv = dv.float().sum(dim=1)
    dv_scale = dv.float().abs().max().item()
    err = (got_dv - want_dv).abs().max().item()
    say(f"sum dv error {err:.3e} (|dv| max {dv_scale:.3e})")
    assert err <= 2e-3 * dv_scale * N ** 0.5
    got_dk = dk.float().sum(dim=1)
    dk_scale = dk.float().abs().max().item()
    err = got_dk.abs().max().item()
    say(f"sum dk {err:.3e} (|dk| max {dk_scale:.3e})")
    assert err <= 2e-3 * dk_scale * N ** 0.5
    assert torch.isfinite(dq.float()).all()

    # The oracle on a subset: the union of every tile the key range's rows live in, plus two early
    # tiles for dq rows; group g0's keys key_lo .. key_lo + 63.
    rng = np.random.default_rng(17)
    key_lo = N - FULL_KEYS[name]
    key_hi = key_lo + 64
    g0 = 3
    tiles = np.unique(np.concatenate([np.arange(key_lo // Tq, p.n_tiles), rng.integers(0, key_lo // Tq, 2)]))
    say(f"attend_bwd {name}: oracle unions of {len(tiles)} tiles")
    ch = OracleChain({k: x[k].cpu() for k in ("qi", "ki", "w")}, p)
    om, _, _, _ = ch.union_of_tiles(tiles)
    np.testing.assert_array_equal(umask[:, torch.from_numpy(tiles).long().cuda()].cpu().numpy().view(np.uint32),
                                  om[:, tiles])
    rows = np.unique(np.concatenate([rng.choice(ch.tile_rows(int(t)), 2, replace=False) for t in tiles[::4]]
                                    + [[N - 1]])).astype(np.int32)
    say(f"attend_bwd {name}: oracle dq on {len(rows)} rows, dk/dv of group {g0} keys {key_lo}..{key_hi - 1}")
    pq, pk, pv = oracle.attend_bwd_part(bits(x["q"]), bits(x["k"]), bits(x["v"]), om, bits(dout), p.block, Tq,
                                        rows, g0, key_lo, key_hi)
    assert_close_grad(dq[torch.from_numpy(rows).long().cuda()], pq, f"dq {name} sampled rows")
    assert_close_grad(dk[g0, key_lo:key_hi], pk, f"dk {name} keys")
    assert_close_grad(dv[g0, key_lo:key_hi], pv, f"dv {name} keys")


def test_attend_bwd_stream_order(sg):
    """The tile-order sums of each dk/dv batch run on the library's own second stream; the results
    must still be ordered on the caller's stream. With many small batches (the event hand-offs
    between the two streams at every batch): two calls back to back on a caller-made stream, sharing
    one workspace and read on that stream without a host wait in between, and two host threads
    calling at once on two streams, all give the bits of a call on the default stream."""
    import threading

    wl = datagen.PREFILL.replace(name="bwd_streams", n_tokens=8192, n_q_heads=16, n_kv_heads=2,
                                 topk_tokens=512, union_tile=64)
    p = params_of(wl)
    N, Hq, G, D = p.n_tokens, p.n_q_heads, p.n_kv_heads, p.head_dim
    x = datagen.prefill_inputs(wl, device="cuda")
    umask = torch.empty((G, p.n_tiles, p.n_words), dtype=torch.int32, device="cuda")
    ucount = torch.empty((G, p.n_tiles), dtype=torch.int32, device="cuda")
    blk = torch.empty((N // p.block, p.idx_dim), dtype=torch.bfloat16, device="cuda")
    sg.sgqa_compress(p, x["ki"], blk)
    sg.sgqa_index_union(p, x["qi"], x["w"], blk, umask, ucount)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    dout = torch.randn((N, Hq, D), generator=gen, device="cuda").to(torch.bfloat16)
    with bwd_mode("tile_batched"):
        # The tile-major design runs (its workspace holds more than the deltas).
        assert sg.workspace_size(p, sg.SGQA_OP_ATTEND_BWD) > N * Hq * 4 + 256
        out, lse, dq0, dk0, dv0 = run_fwd_bwd(sg, p, x, umask, ucount, dout)

        def grads():
            return (torch.empty_like(dq0), torch.empty_like(dk0), torch.empty_like(dv0))

        def same(got, what):
            for a, b, n in zip(got, (dq0, dk0, dv0), ("dq", "dk", "dv")):
                assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{what}: {n} differs"

        s = torch.cuda.Stream()
        ws = sg.workspace(p, sg.SGQA_OP_ATTEND_BWD)
        g1, g2 = grads(), grads()
        torch.cuda.synchronize()
        say("attend_bwd streams: two calls back to back on a caller stream")
        with torch.cuda.stream(s):
            for g in (g1, g2):
                sg.sgqa_attend_bwd(p, x["q"], x["k"], x["v"], umask, ucount, out, lse, dout, *g, ws, stream=s)
            copies = [tuple(t.clone() for t in g) for g in (g1, g2)]
        s.synchronize()
        for c, what in zip(copies, ("first call", "second call")):
            same(c, what)

        say("attend_bwd streams: two host threads on two streams")
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        wss = [sg.workspace(p, sg.SGQA_OP_ATTEND_BWD) for _ in streams]
        outs = [grads(), grads()]
        torch.cuda.synchronize()
        errors = []

        def work(t):
            try:
                st = streams[t]
                with torch.cuda.stream(st):
                    for _ in range(2):
                        sg.sgqa_attend_bwd(p, x["q"], x["k"], x["v"], umask, ucount, out, lse, dout, *outs[t],
                                           wss[t], stream=st)
                st.synchronize()
            except Exception as e:  # reported on the main thread
                errors.append(e)

        threads = [threading.Thread(target=work, args=(t,)) for t in range(2)]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        assert not errors, errors
        for t in range(2):
            same(outs[t], f"thread {t}")
