"""FP8 E4M3 K/V cache decode on the GPU (sgqa_decode_fp8) against the oracle's decode_fp8.

The selection reads only the bf16 index side, so it must equal the oracle's bit for bit (and the
bf16 decode's); the output is compared with the oracle's fp64 attention over code value * scale
within the attention tolerance. Paged pools must give the dense result's bits.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from tests.gpu_common import assert_close_attention, bits, params_of, say
from tests.test_gpu_incremental import to_pages

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sg():
    import block_sparse_long_sgqa_amd as sg

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sg.lib()
    return sg


def fp8_case(S=3, C=1200, G=2, k=256, B=8, name="fp8"):
    wl = datagen.DECODE.replace(name=f"dec_{name}_{C}_{S}_{G}_{B}", n_tokens=C, n_seqs=S, n_q_heads=8 * G,
                                n_kv_heads=G, topk_tokens=k, block=B)
    return wl, params_of(wl), datagen.decode_inputs(wl), datagen.fp8_caches(wl)


def oracle_fp8(x, f, s, L, B, kb):
    """The oracle's FP8 decode of sequence s at context length L (its first L positions)."""
    sl = slice(s, s + 1)
    kbar = oracle.compress(bits(x["ki_cache"][sl, :L]), B)
    return oracle.decode_fp8(x["q"][sl], f["k8"][sl, :, :L].contiguous(), f["v8"][sl, :, :L].contiguous(),
                             f["kv_scale"][sl], kbar, x["qi"][sl], x["w"], B, kb)


def run_fp8(sg, p, xd, fd, blk, lens=None, pages=None, kc=None, vc=None):
    S = p.n_seqs
    out = torch.empty((S, p.n_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    topk = torch.empty((S, p.n_kv_heads, p.kb), dtype=torch.int32, device="cuda")
    ws = sg.workspace(p, sg.SGQA_OP_DECODE)
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    sg.sgqa_decode_fp8(p, xd["q"], fd["k8"] if kc is None else kc, fd["v8"] if vc is None else vc,
                       fd["kv_scale"], blk, xd["qi"], xd["w"], out, ws, seq_lens=sl, pages=pages, topk_out=topk)
    torch.cuda.synchronize()
    return out, topk


@pytest.mark.parametrize("C,k,B,G", [(1200, 256, 8, 2), (4096, 2048, 8, 1), (3000, 1024, 64, 2), (5000, 512, 1, 1)])
def test_fp8_decode_matches_oracle(sg, C, k, B, G):
    wl, p, x, f = fp8_case(S=2, C=C, G=G, k=k, B=B)
    say(f"fp8 decode S=2 C={C} k={k} B={B} G={G}")
    xd = {n: v.cuda() for n, v in x.items()}
    fd = {n: v.cuda() for n, v in f.items()}
    blk = torch.empty((p.n_seqs, max(C // B, 1), 64), dtype=torch.bfloat16, device="cuda")
    sg.sgqa_compress(p, xd["ki_cache"], blk)
    out, topk = run_fp8(sg, p, xd, fd, blk)
    # The selection is the bf16 decode's.
    ws = sg.workspace(p, sg.SGQA_OP_DECODE)
    out_bf = torch.empty_like(out)
    topk_bf = torch.empty_like(topk)
    sg.sgqa_decode(p, xd["q"], xd["k_cache"], xd["v_cache"], blk, xd["qi"], xd["w"], out_bf, ws, topk_out=topk_bf)
    torch.cuda.synchronize()
    assert torch.equal(topk, topk_bf)
    for s in range(p.n_seqs):
        sel, want = oracle_fp8(x, f, s, C, B, p.kb)
        np.testing.assert_array_equal(topk[s:s + 1].cpu().numpy(), sel)
        assert_close_attention(out[s:s + 1], want, f"fp8 seq {s}")


def test_fp8_varlen_and_paged(sg):
    wl, p, x, f = fp8_case(S=4, C=1200, G=2, k=256, B=8, name="fp8v")
    S, C, B = p.n_seqs, p.n_tokens, p.block
    lens = [C, 777, 9, 1]
    say(f"fp8 varlen decode lens={lens}")
    xd = {n: v.cuda() for n, v in x.items()}
    fd = {n: v.cuda() for n, v in f.items()}
    blk = torch.empty((S, C // B, 64), dtype=torch.bfloat16, device="cuda")
    sg.sgqa_compress(p, xd["ki_cache"], blk)
    out, topk = run_fp8(sg, p, xd, fd, blk, lens=lens)
    for s, L in enumerate(lens):
        sel, want = oracle_fp8(x, f, s, L, B, p.kb)
        np.testing.assert_array_equal(topk[s:s + 1].cpu().numpy(), sel)
        assert_close_attention(out[s:s + 1], want, f"fp8 varlen seq {s} L={L}")
    say("fp8 paged decode (page 64)")
    table, kpool, n_pages = to_pages(sg, fd["k8"], 64, 3)
    _, vpool, _ = to_pages(sg, fd["v8"], 64, 3)
    pages = sg.Pages(table, 64, n_pages)
    out_p, topk_p = run_fp8(sg, p, xd, fd, blk, lens=lens, pages=pages, kc=kpool, vc=vpool)
    assert torch.equal(topk_p, topk)
    assert torch.equal(out_p.view(torch.int16), out.view(torch.int16))
    # float8_e4m3fn tensors are taken as their codes.
    out_f, _ = run_fp8(sg, p, xd, fd, blk, lens=lens, kc=fd["k8"].view(torch.float8_e4m3fn),
                       vc=fd["v8"].view(torch.float8_e4m3fn))
    assert torch.equal(out_f.view(torch.int16), out.view(torch.int16))


def test_fp8_decode_256k_full_size(sg):
    wl = datagen.DECODE
    p = params_of(wl)
    say("fp8 decode 32 x 262144: drawing caches on the GPU")
    y = datagen.decode_inputs(wl, device="cuda")
    del y["k_cache"], y["v_cache"]
    f = datagen.fp8_caches(wl, device="cuda")
    blk = torch.empty((p.n_seqs, p.n_tokens // p.block, 64), dtype=torch.bfloat16, device="cuda")
    sg.sgqa_compress(p, y["ki_cache"], blk)
    say("fp8 decode 32 x 262144: decode")
    out, topk = run_fp8(sg, p, y, f, blk)
    out2, _ = run_fp8(sg, p, y, f, blk)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), "decode is not deterministic"
    t = topk.cpu().numpy()
    c = (p.n_tokens - 1) // p.block
    assert (t >= 0).all() and (t < c).all() and (np.diff(t, axis=-1) > 0).all()
    for s in (0, 21):
        say(f"fp8 decode: oracle on sequence {s}")
        sl = slice(s, s + 1)
        kbar = oracle.compress(bits(y["ki_cache"][sl]), p.block)
        sel, want = oracle.decode_fp8(y["q"][sl], f["k8"][sl], f["v8"][sl], f["kv_scale"][sl], kbar, y["qi"][sl],
                                      y["w"], p.block, p.kb)
        np.testing.assert_array_equal(t[s:s + 1], sel)
        assert_close_attention(out[sl], want, f"fp8 decode seq {s}")
