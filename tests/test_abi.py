"""C-ABI surface checks that need no GPU: exports, host-side argument validation, workspace sizes."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")
LIB = os.path.join(ROOT, "sparse_attention_fp4_csa2_amd", "libcsa2.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from sparse_attention_fp4_csa2_amd import build
        build.build()
    from sparse_attention_fp4_csa2_amd import _lib
    return _lib.load(LIB)


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("csa2_append_fp4", "csa2_index_topk", "csa2_sparse_attn", "csa2_swa_merge"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    assert lib.csa2_status_str(0) == b"ok"
    assert lib.csa2_status_str(-3) == b"workspace too small"
    assert lib.csa2_version() == 10000


def test_host_validation_rejects_before_launch(lib):
    P = ctypes.c_void_p
    fake = P(4096)            # never dereferenced: every call below fails its host checks
    # null pointers
    assert lib.csa2_append_fp4(None, None, fake, 1, 1, 8, fake, None, None, None) == -1
    # cap not a multiple of 8
    assert lib.csa2_append_fp4(fake, None, fake, 1, 1, 12, fake, None, None, None) == -1
    # group sums need keys; cap % 512 for group sums
    assert lib.csa2_append_fp4(fake, None, fake, 1, 1, 8, fake, None, fake, None) == -1
    assert lib.csa2_append_fp4(fake, fake, fake, 1, 1, 520, fake, fake, fake, None) == -2
    # misaligned latent
    assert lib.csa2_append_fp4(P(4097), None, fake, 1, 1, 8, fake, None, None, None) == -1
    # top_k larger than the number of blocks
    assert lib.csa2_index_topk(fake, fake, fake, None, fake, None, 1, 1, 4, 64, 9, 0,
                               fake, fake, fake, 1 << 20, None) == -1
    # too many indexer heads
    assert lib.csa2_index_topk(fake, fake, fake, None, fake, None, 1, 1, 17, 64, 4, 0,
                               fake, fake, fake, 1 << 20, None) == -2
    # workspace too small
    assert lib.csa2_index_topk(fake, fake, fake, None, fake, None, 1, 1, 4, 2048, 32, 0,
                               fake, fake, fake, 16, None) == -3
    # two-level without group sums / with query positions
    ws = lib.csa2_index_topk_ws(1, 1, 4096, 4)
    assert lib.csa2_index_topk(fake, fake, fake, None, fake, None, 1, 1, 4, 4096, 32, 4,
                               fake, fake, fake, ws, None) == -2
    assert lib.csa2_index_topk(fake, fake, fake, fake, fake, fake, 1, 1, 4, 4096, 32, 4,
                               fake, fake, fake, ws, None) == -2
    # attention: heads beyond the maximum, bad scale
    assert lib.csa2_sparse_attn(fake, fake, fake, fake, fake, None, 1, 1, 129, 64, 4, 0.04,
                                fake, fake, fake, 1 << 30, None) == -2
    assert lib.csa2_sparse_attn(fake, fake, fake, fake, fake, None, 1, 1, 16, 64, 4, -1.0,
                                fake, fake, fake, 1 << 30, None) == -1
    # attention workspace too small
    need = lib.csa2_sparse_attn_ws(1, 1, 64, 2048)
    assert need > 0
    assert lib.csa2_sparse_attn(fake, fake, fake, fake, fake, None, 1, 1, 64, 32768, 2048, 0.04,
                                fake, fake, fake, need - 1, None) == -3
    # window merge
    assert lib.csa2_swa_merge(fake, fake, fake, None, None, 1, 1, 16, 0, 8, 0.04,
                              fake, fake, fake, fake, fake, 1 << 20, None) == -1
    assert lib.csa2_topk(fake, 1, 70000, 4, fake, fake, None) == -2
    # one-call layer and its two phases: null window, workspace too small
    need = lib.csa2_attend_layer_ws(2, 1, 64, 2048, 512)
    assert need > 0
    assert lib.csa2_attend_layer(fake, fake, fake, fake, fake, None, None, fake, None, 2, 1, 64, 32768,
                                 2048, 512, 512, 0.04, fake, fake, fake, need, None) == -1
    assert lib.csa2_attend_layer(fake, fake, fake, fake, fake, None, fake, fake, None, 2, 1, 64, 32768,
                                 2048, 512, 512, 0.04, fake, fake, fake, need - 1, None) == -3
    assert lib.csa2_attend_layer_window(fake, fake, fake, None, None, 2, 1, 64, 2048, 512, 512, 0.04,
                                        fake, need - 1, None) == -3
    assert lib.csa2_attend_layer_window(fake, None, fake, None, None, 2, 1, 64, 2048, 512, 512, 0.04,
                                        fake, need, None) == -1
    assert lib.csa2_attend_layer_sparse(fake, fake, fake, fake, fake, None, 2, 1, 64, 32768, 2048, 512,
                                        0.04, fake, fake, fake, need - 1, None) == -3
    assert lib.csa2_attend_layer_sparse(fake, fake, fake, fake, fake, None, 2, 1, 129, 32768, 2048, 512,
                                        0.04, fake, fake, fake, need, None) == -2


def test_workspace_sizes_are_pure_and_monotone(lib):
    a = lib.csa2_index_topk_ws(32, 1, 32768, 0)
    assert a >= 32 * 4096 * 4
    b = lib.csa2_index_topk_ws(8, 1, 524288, 256)
    # block scores over the kept groups, the group scores, the kept group ids and their counts
    assert b >= 8 * 256 * 64 * 4 + 8 * 1024 * 4 + 8 * 256 * 4 + 8 * 4
    assert lib.csa2_swa_merge_ws(32, 1, 64, 512) >= lib.csa2_swa_merge_ws(1, 1, 64, 512)
    assert lib.csa2_index_topk_ws(0, 1, 8, 0) == 0


def test_layer_plan_with_row_tiles(lib):
    # host-side plan of a layer call (no GPU).  With 16 or fewer heads and
    # several rows per sequence, rows share attention tiles: a 4096-row
    # prefill chunk then runs one split per two-row tile with the window on the
    # same tiles, so its layer is one launch, as at 64 heads; 4 draft rows per
    # sequence need split-K and a combine (two launches), as do Q = 1 decode
    # rows, which keep one row per tile
    B, K, W = 1, 2048, 512
    assert lib.csa2_attend_layer_launches(B, 4096, 64, K, W) == 1
    assert lib.csa2_attend_layer_launches(B, 4096, 16, K, W) == 1
    assert lib.csa2_attend_layer_launches(32, 4, 16, K, W) == 2
    assert lib.csa2_attend_layer_launches(32, 1, 16, K, W) == 2
    # a one-split call needs no workspace; a split one does
    assert lib.csa2_sparse_attn_ws(B, 4096, 16, K) == 0
    assert lib.csa2_sparse_attn_ws(32, 4, 16, K) > 0
