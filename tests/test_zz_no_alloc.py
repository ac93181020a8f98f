"""sgqa_decode_noalloc (the decode for callers that cannot allocate) against sgqa_decode.

Two calls in a row through the C ABI, the second with a smaller input, so the library's static
per-GPU scratch still holds the first call's larger contents when the second runs: each output and
selection must be bit-identical to sgqa_decode's (same kernels, caller workspace) and within the
attention tolerance of the oracle. The first call's context is long enough (more than 32768
candidate blocks) that the selection goes through the segment lists, which also live in the scratch.
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


def run_pair(sg, wl):
    p = params_of(wl)
    say(f"noalloc decode {wl.name}: S={p.n_seqs} L={p.n_tokens} G={p.n_kv_heads} Hq={p.n_q_heads} kb={p.kb}")
    y = datagen.decode_inputs(wl, device="cuda")
    blk = torch.empty((p.n_seqs, p.n_tokens // p.block, 64), dtype=torch.bfloat16, device="cuda")
    sg.sgqa_compress(p, y["ki_cache"], blk)
    assert sg.workspace_size(p, sg.SGQA_OP_DECODE) <= sg.NOALLOC_SCRATCH_BYTES
    ws = sg.workspace(p, sg.SGQA_OP_DECODE)
    ref = torch.empty((p.n_seqs, p.n_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    ref_topk = torch.empty((p.n_seqs, p.n_kv_heads, p.kb), dtype=torch.int32, device="cuda")
    sg.sgqa_decode(p, y["q"], y["k_cache"], y["v_cache"], blk, y["qi"], y["w"], ref, ws, topk_out=ref_topk)
    out = torch.full_like(ref, 7.0)
    topk = torch.full_like(ref_topk, -7)
    sg.sgqa_decode_noalloc(p, y["q"], y["k_cache"], y["v_cache"], blk, y["qi"], y["w"], out, topk_out=topk)
    torch.cuda.synchronize()
    assert torch.equal(topk, ref_topk), "noalloc selection differs from sgqa_decode"
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "noalloc output differs from sgqa_decode"
    for s in (0, p.n_seqs - 1):
        sl = slice(s, s + 1)
        kbar = oracle.compress(bits(y["ki_cache"][sl]), p.block)
        sel, want = oracle.decode(y["q"][sl], y["k_cache"][sl], y["v_cache"][sl], kbar, y["qi"][sl], y["w"],
                                  p.block, p.kb)
        np.testing.assert_array_equal(topk[sl].cpu().numpy(), sel)
        assert_close_attention(out[sl], want, f"noalloc decode {wl.name} seq {s}")


def test_noalloc_decode_two_calls_second_smaller(sg):
    big = datagen.DECODE.replace(name="noalloc_big", n_tokens=8 * (32768 + 600) + 3, n_seqs=2, n_q_heads=16,
                                 n_kv_heads=2)
    small = datagen.DECODE.replace(name="noalloc_small", n_tokens=4101, n_seqs=3, n_q_heads=16, n_kv_heads=2,
                                   topk_tokens=1024)
    run_pair(sg, big)
    run_pair(sg, small)


def test_noalloc_decode_rejects_sizes_beyond_the_scratch(sg):
    p = sg.Params(n_tokens=1 << 20, n_seqs=64, n_q_heads=64, n_kv_heads=8, block=8, topk_tokens=4096, union_tile=1)
    assert sg.workspace_size(p, sg.SGQA_OP_DECODE) > sg.NOALLOC_SCRATCH_BYTES
    t = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    st = sg.lib().sgqa_decode_noalloc(p.c(), *([t.data_ptr()] * 6), None, t.data_ptr(), None)
    assert st == sg.SGQA_ERR_SCRATCH, sg.status_string(st)
