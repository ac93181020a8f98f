"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every function that include/sgqa.h declares, report its version and
status texts, size workspaces on the host, and reject bad arguments with the documented status
before touching the device.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgqa.h")


@pytest.fixture(scope="module")
def sg():
    import block_sparse_long_sgqa_amd as sg

    if not os.path.exists(sg.LIB_PATH):
        from block_sparse_long_sgqa_amd import build

        build.build()
    sg.lib()
    return sg


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(sgqa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_calls():
    names = declared_functions()
    for n in ("sgqa_compress", "sgqa_index_topk", "sgqa_union", "sgqa_attend", "sgqa_prefill", "sgqa_decode",
              "sgqa_workspace_size", "sgqa_status_string", "sgqa_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(sg):
    lib = ctypes.CDLL(sg.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(sg.EXPORTED)


def test_abi_version_and_status_strings(sg):
    assert sg.lib().sgqa_abi_version() == 1
    for code in range(8):
        assert len(sg.status_string(code)) > 0
    assert sg.status_string(0) == "ok"
    assert sg.status_string(99) == "unknown status"


def _p(**kw):
    import block_sparse_long_sgqa_amd as sg

    base = dict(n_tokens=32768, n_q_heads=64, n_kv_heads=8, block=8, topk_tokens=4096, union_tile=64)
    base.update(kw)
    return sg.Params(**base)


def test_workspace_sizes_match_layout(sg):
    p = _p()
    assert sg.workspace_size(p, sg.SGQA_OP_COMPRESS) == 0
    assert sg.workspace_size(p, sg.SGQA_OP_INDEX_TOPK) == 0
    assert sg.workspace_size(p, sg.SGQA_OP_ATTEND) == 0
    r = lambda x: (x + 255) // 256 * 256  # noqa: E731
    N, G, kb, T, W = 32768, 8, 512, 512, 128
    want = r(N // 8 * 64 * 2) + r(G * T * W * 4) + r(G * T * 4)  # the fused path keeps no topk
    assert sg.workspace_size(p, sg.SGQA_OP_PREFILL) == want
    d = _p(n_tokens=262144, n_seqs=32, union_tile=1)
    assert sg.workspace_size(d, sg.SGQA_OP_DECODE) > 32 * 8 * 512 * 4


@pytest.mark.parametrize("kw", [
    dict(head_dim=64), dict(idx_heads=3), dict(idx_dim=32), dict(block=3), dict(block=128),
    dict(topk_tokens=100), dict(topk_tokens=0), dict(topk_tokens=8 * 4096), dict(n_q_heads=60),
    dict(union_tile=0), dict(n_tokens=0), dict(n_seqs=2), dict(n_kv_heads=0),
    dict(n_q_heads=8 * 32, n_kv_heads=8),
])
def test_bad_shapes_are_rejected_before_any_launch(sg, kw):
    p = _p(**kw)
    out = ctypes.c_size_t(0)
    st = sg.lib().sgqa_workspace_size(ctypes.byref(p.c()), sg.SGQA_OP_PREFILL, ctypes.byref(out))
    assert st == sg.SGQA_ERR_SHAPE
    nul = ctypes.c_void_p(0)
    buf = (ctypes.c_uint8 * 64)()
    a = ctypes.c_void_p((ctypes.addressof(buf) + 15) // 16 * 16)
    st = sg.lib().sgqa_prefill(ctypes.byref(p.c()), a, a, a, a, a, a, a, a, 1 << 40, nul)
    assert st == sg.SGQA_ERR_SHAPE


def bwd_workspace(N, Hq, G, B, Tq, batch_rows=1 << 21, max_batches=2048):
    """The backward's workspace as its header states it: the deltas (N Hq fp32), and for the
    tile-major dk/dv (when its batches of partial rows number at most max_batches) the fp32
    accumulator (G N rows of 1 KiB), nblk / ebase / ipref per pair, the batch starts, the word
    prefixes (pairs x mask words), the work items (8 B) and the 1-KiB partial rows: one batch, or two
    buffers of a batch each when there are several batches (one is reduced while the other fills)."""
    r = lambda x: (x + 255) // 256 * 256  # noqa: E731
    delta = r(N * Hq * 4)
    T, nbc = -(-N // Tq), -(-N // B)
    W, nbi = -(-nbc // 32), 128 // B
    nb = [-(-min(N, (t + 1) * Tq) // B) for t in range(T)]
    rows = G * sum(n * B for n in nb)
    items = G * sum(-(-n // nbi) for n in nb)
    unit = nbc * B
    cap = max(min(batch_rows, 1 << 21), 2 * unit)
    if cap >= rows:
        cap, n_b = rows, 1
    else:
        n_b = (rows - 1) // (cap - unit) + 1
    P = T * G
    if n_b > max_batches:
        return delta
    return (delta + r(G * N * 1024) + r(P * 4) + r((P + 1) * 8) + r((P + 1) * 4) + r((n_b + 1) * 4)
            + r(P * W * 4) + r(items * 8) + r((2 if n_b > 1 else 1) * cap * 1024))


@pytest.mark.parametrize("shape", [(131072, 64, 8, 8, 128), (32768, 64, 8, 8, 64), (20037, 8, 1, 1, 64),
                                   (1205, 16, 2, 8, 64), (5, 16, 2, 8, 16),
                                   # either side of the batch limit: 1898 batches (tile-major), 2837 (key-major)
                                   (327680, 64, 8, 8, 128), (393216, 64, 8, 8, 128)])
def test_backward_workspace(sg, shape, monkeypatch):
    N, Hq, G, B, Tq = shape
    p = _p(n_tokens=N, n_q_heads=Hq, n_kv_heads=G, block=B, topk_tokens=max(B, 64), union_tile=Tq)
    monkeypatch.delenv("SGQA_BWD_PATH", raising=False)
    monkeypatch.delenv("SGQA_BWD_BATCH_ROWS", raising=False)
    assert sg.workspace_size(p, sg.SGQA_OP_ATTEND_BWD) == bwd_workspace(N, Hq, G, B, Tq)
    deltas = (N * Hq * 4 + 255) // 256 * 256
    if N == 327680:
        assert bwd_workspace(N, Hq, G, B, Tq) > deltas  # the tile-major design
    if N == 393216:
        assert bwd_workspace(N, Hq, G, B, Tq) == deltas  # too many batches: key-major
    monkeypatch.setenv("SGQA_BWD_BATCH_ROWS", "1")
    assert sg.workspace_size(p, sg.SGQA_OP_ATTEND_BWD) == bwd_workspace(N, Hq, G, B, Tq, batch_rows=1)
    monkeypatch.setenv("SGQA_BWD_PATH", "key")
    assert sg.workspace_size(p, sg.SGQA_OP_ATTEND_BWD) == (N * Hq * 4 + 255) // 256 * 256


@pytest.mark.parametrize("n_tokens", [262144 + 8, 1 << 20])
def test_long_context_prefill_is_accepted(sg, n_tokens):
    # The attention kernels walk a tile's block list in fixed-size LDS segments, so no sequence
    # length is refused for the list; the prefill workspace is the layout at that length.
    p = _p(n_tokens=n_tokens, union_tile=128)
    r = lambda x: (x + 255) // 256 * 256  # noqa: E731
    N, G = n_tokens, 8
    T, W = (N + 127) // 128, ((N + 7) // 8 + 31) // 32
    assert sg.workspace_size(p, sg.SGQA_OP_PREFILL) == r(N // 8 * 64 * 2) + r(G * T * W * 4) + r(G * T * 4)
    assert sg.workspace_size(p, sg.SGQA_OP_ATTEND) == 0
    assert sg.workspace_size(p, sg.SGQA_OP_ATTEND_BWD) == bwd_workspace(N, 64, G, 8, 128)
    assert sg.workspace_size(p, sg.SGQA_OP_INDEX_TOPK) == 0


def test_null_and_alignment_errors(sg):
    lib = sg.lib()
    p = _p()
    nul = ctypes.c_void_p(0)
    assert lib.sgqa_workspace_size(None, 0, ctypes.byref(ctypes.c_size_t())) == sg.SGQA_ERR_NULL
    assert lib.sgqa_compress(None, nul, nul, nul) == sg.SGQA_ERR_NULL
    assert lib.sgqa_compress(ctypes.byref(p.c()), nul, nul, nul) == sg.SGQA_ERR_NULL
    buf = (ctypes.c_uint8 * 64)()
    a = ctypes.c_void_p((ctypes.addressof(buf) + 15) // 16 * 16)
    mis = ctypes.c_void_p(a.value + 4)
    assert lib.sgqa_compress(ctypes.byref(p.c()), mis, a, nul) == sg.SGQA_ERR_ALIGN
    assert lib.sgqa_union(ctypes.byref(p.c()), a, mis, a, nul) == sg.SGQA_ERR_ALIGN
    assert lib.sgqa_attend(ctypes.byref(p.c()), a, a, a, a, a, nul, nul, 0, nul) == sg.SGQA_ERR_NULL
    # workspace too small is reported before the device is queried
    assert lib.sgqa_prefill(ctypes.byref(p.c()), a, a, a, a, a, a, a, a, 16, nul) == sg.SGQA_ERR_WORKSPACE
    d = _p(n_tokens=4096, n_seqs=4, union_tile=1)
    assert lib.sgqa_decode(ctypes.byref(d.c()), a, a, a, a, a, a, nul, a, a, 16, nul) == sg.SGQA_ERR_WORKSPACE


def test_binding_refuses_host_tensors(sg):
    import torch

    p = _p(n_tokens=64, n_q_heads=8, n_kv_heads=1, topk_tokens=64, union_tile=16)
    ki = torch.zeros((64, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sg.sgqa_compress(p, ki, torch.zeros((8, 64), dtype=torch.bfloat16))


def test_varlen_decode_and_append_validation(sg):
    lib = sg.lib()
    nul = ctypes.c_void_p(0)
    buf = (ctypes.c_uint8 * 64)()
    a = ctypes.c_void_p((ctypes.addressof(buf) + 15) // 16 * 16)
    d = _p(n_tokens=4096, n_seqs=4, union_tile=1)
    dp = ctypes.byref(d.c())
    # seq_lens is required by the varlen call
    assert lib.sgqa_decode_varlen(dp, a, a, a, None, a, a, a, nul, nul, a, a, 1 << 40, nul) == sg.SGQA_ERR_NULL

    def pages(table, max_pages, page_tokens, n_pages):
        return ctypes.byref(sg.sgqa_pages(table.value, max_pages, page_tokens, n_pages))

    def varlen(pg):
        return lib.sgqa_decode_varlen(dp, a, a, a, pg, a, a, a, a, nul, a, a, 1 << 40, nul)

    assert varlen(pages(nul, 64, 64, 100)) == sg.SGQA_ERR_NULL                 # no table
    assert varlen(pages(a, 64, 48, 100)) == sg.SGQA_ERR_SHAPE                  # page not a power of two
    assert varlen(pages(a, 64, 4, 100)) == sg.SGQA_ERR_SHAPE                   # page smaller than B = 8
    assert varlen(pages(a, 63, 64, 100)) == sg.SGQA_ERR_SHAPE                  # max_pages * page < capacity
    assert varlen(pages(a, 64, 64, 0)) == sg.SGQA_ERR_SHAPE                    # empty pool
    # a valid descriptor gets as far as the workspace check
    assert lib.sgqa_decode_varlen(dp, a, a, a, pages(a, 64, 64, 100), a, a, a, a, nul, a, a, 16, nul) \
        == sg.SGQA_ERR_WORKSPACE

    def append(pg, pos=a, idx_cache=a):
        return lib.sgqa_append(dp, a, a, a, pos, a, a, pg, idx_cache, a, nul)

    assert append(None, pos=nul) == sg.SGQA_ERR_NULL
    assert append(None, idx_cache=nul) == sg.SGQA_ERR_NULL
    assert append(None, pos=ctypes.c_void_p(a.value + 4)) == sg.SGQA_ERR_ALIGN
    assert append(pages(a, 64, 12, 100)) == sg.SGQA_ERR_SHAPE
    bad_dim = _p(n_tokens=4096, n_seqs=4, union_tile=1, head_dim=64)
    assert lib.sgqa_append(ctypes.byref(bad_dim.c()), a, a, a, a, a, a, None, a, a, nul) == sg.SGQA_ERR_SHAPE


def test_fp8_decode_validation(sg):
    lib = sg.lib()
    nul = ctypes.c_void_p(0)
    buf = (ctypes.c_uint8 * 64)()
    a = ctypes.c_void_p((ctypes.addressof(buf) + 15) // 16 * 16)
    d = _p(n_tokens=4096, n_seqs=4, union_tile=1)
    dp = ctypes.byref(d.c())

    def fp8(scale=a, lens=nul, pg=None, ws_bytes=1 << 40, q=a):
        return lib.sgqa_decode_fp8(dp, q, a, a, scale, pg, a, a, a, lens, nul, a, a, ws_bytes, nul)

    assert fp8(scale=nul) == sg.SGQA_ERR_NULL                                   # kv_scale is required
    assert fp8(q=nul) == sg.SGQA_ERR_NULL
    assert fp8(scale=ctypes.c_void_p(a.value + 4)) == sg.SGQA_ERR_ALIGN
    bad = ctypes.byref(sg.sgqa_pages(a.value, 64, 48, 100))
    assert fp8(pg=bad) == sg.SGQA_ERR_SHAPE
    # dense and varlen descriptors get as far as the workspace check
    assert fp8(ws_bytes=16) == sg.SGQA_ERR_WORKSPACE
    assert fp8(lens=a, ws_bytes=16) == sg.SGQA_ERR_WORKSPACE


def test_masked_variant_shapes_and_workspace(sg):
    r = lambda x: (x + 255) // 256 * 256  # noqa: E731
    p = _p()  # N 32768, G 8, B 8, r 8
    W = (32768 // 8 + 31) // 32
    assert sg.workspace_size(p, sg.SGQA_OP_ATTEND_MASKED) == r(8 * 32768 * W * 4)
    assert sg.workspace_size(p, sg.SGQA_OP_PREFILL_MASKED) == \
        sg.workspace_size(p, sg.SGQA_OP_PREFILL) + r(8 * 32768 * 512 * 4) + r(8 * 32768 * W * 4)
    # B = 1 with r = 8: 64 block entries x 2 words per chunk do not fit the membership table.
    bad = _p(block=1, topk_tokens=512)
    out = ctypes.c_size_t(0)
    assert sg.lib().sgqa_workspace_size(ctypes.byref(bad.c()), sg.SGQA_OP_ATTEND_MASKED, ctypes.byref(out)) \
        == sg.SGQA_ERR_SHAPE
    nul = ctypes.c_void_p(0)
    buf = (ctypes.c_uint8 * 64)()
    a = ctypes.c_void_p((ctypes.addressof(buf) + 15) // 16 * 16)
    assert sg.lib().sgqa_attend_masked(ctypes.byref(bad.c()), a, a, a, a, a, a, a, a, 1 << 40, nul) == sg.SGQA_ERR_SHAPE
    assert sg.lib().sgqa_attend_masked(ctypes.byref(p.c()), a, a, a, nul, a, a, a, a, 1 << 40, nul) == sg.SGQA_ERR_NULL
    assert sg.lib().sgqa_attend_masked(ctypes.byref(p.c()), a, a, a, a, a, a, a, a, 16, nul) == sg.SGQA_ERR_WORKSPACE


def test_noalloc_decode_rejects_oversized_calls_on_the_host(sg):
    """Sizes whose decode scratch exceeds the library's static buffer fail before any device work."""
    p = _p(n_tokens=1 << 20, n_seqs=64, union_tile=1)
    assert sg.workspace_size(p, sg.SGQA_OP_DECODE) > sg.NOALLOC_SCRATCH_BYTES
    fake = 1 << 20  # never dereferenced: the size check comes first
    st = sg.lib().sgqa_decode_noalloc(p.c(), *([fake] * 6), None, fake, None)
    assert st == sg.SGQA_ERR_SCRATCH, sg.status_string(st)
    assert "scratch" in sg.status_string(st)
