"""The C-ABI library loads, exports every entry point include/dl.h declares, and rejects bad arguments on the
host (before any GPU work).  Runs on the CPU: no call here reaches a kernel."""
import ctypes as C
import os
import re

import pytest

import sparse_attention_moe_amd as dl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared(headers=None):
    inc = os.path.join(ROOT, "include")
    names = set()
    for h in headers or sorted(f for f in os.listdir(inc) if f.endswith(".h")):
        src = open(os.path.join(inc, h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(dl_[a-z_0-9]+)\s*\(", src))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dl.LIB_PATH):
        pytest.fail("libdl.so is not built: run __graft_entry__.build()")
    return dl.load(require_gpu=False)


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(dl.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.dl_abi_version() == dl.ABI_VERSION


def test_method_header_declares_no_measurement_aid():
    # dl.h holds the decode step and its workspace queries; probes and phase events live in dl_measure.h
    step = _declared(["dl.h"])
    assert not [n for n in step if n.startswith(("dl_probe", "dl_profile"))]
    assert set(_declared(["dl_measure.h"])) == {"dl_probe_read", "dl_probe_null", "dl_profile_enable",
                                                 "dl_profile_read", "dl_profile_ffn_fused"}


def test_version_guards(lib):
    # the ABI version is checked at load; the HIP major version the library was built against must match the
    # runtime torch brings (the library runs on it)
    import torch
    hv = lib.dl_hip_version()
    assert hv // 10_000_000 >= 6
    dl.check_hip_version(hv, f"{hv // 10_000_000}.0.51831")  # same major, other minor: accepted
    with pytest.raises(ImportError, match="major"):
        dl.check_hip_version(hv, f"{hv // 10_000_000 - 1}.4.0")
    with pytest.raises(ImportError, match="ROCm"):
        dl.check_hip_version(hv, None)
    if torch.version.hip:
        dl.check_hip_version(hv, torch.version.hip)  # this process's torch


def test_indexer_rejects_bad_arguments(lib):
    P = dl.Pages(2, 64, 4, 0x1000, 0x2000)  # fake device pointers: validation fails before any use
    ws = C.c_void_p(0x10000)
    rc = lib.dl_indexer_topk(None, 1, 1, 16, 128, 2048, 1, None, ws, 1 << 30, None)
    assert rc == -1 and b"pages" in lib.dl_last_error()
    rc = lib.dl_indexer_topk(C.byref(P), None, 1, 16, 128, 2048, 1, None, ws, 1 << 30, None)
    assert rc == -1
    assert lib.dl_indexer_topk(C.byref(P), 1, 1, 65, 128, 2048, 1, None, ws, 1 << 30, None) == -4
    assert lib.dl_indexer_topk(C.byref(P), 1, 1, 16, 100, 2048, 1, None, ws, 1 << 30, None) == -4
    assert lib.dl_indexer_topk(C.byref(P), 1, 1, 16, 128, 0, 1, None, ws, 1 << 30, None) == -2
    bad = dl.Pages(2, 48, 4, 0x1000, 0x2000)  # page size not a power of two
    assert lib.dl_indexer_topk(C.byref(bad), 1, 1, 16, 128, 2048, 1, None, ws, 1 << 30, None) == -2
    assert lib.dl_indexer_topk(C.byref(P), 1, 1, 16, 128, 2048, 1, None, ws, 16, None) == -5
    assert lib.dl_indexer_topk(C.byref(P), 1, 1, 16, 128, 2048, 1, None, C.c_void_p(0x10001), 1 << 30, None) == -5
    need = lib.dl_indexer_topk_workspace(C.byref(P))
    assert need >= 2 * 256 * 4  # at least the score rows


def test_ffn_and_route_reject_bad_arguments(lib):
    wg = dl.Mat(1, 1, dl.DL_FP8_E4M3, 9, 2048, 6144)
    wd = dl.Mat(1, 1, dl.DL_FP8_E4M3, 9, 6144, 2048)
    ws = C.c_void_p(0x10000)
    ok = lib.dl_moe_ffn_workspace(8, 6144, 2048, 2, 8, 1)
    # expert top_k above the routed count
    assert lib.dl_moe_ffn(1, 8, 6144, 2048, 1, 1, 9, C.byref(wg), C.byref(wg), C.byref(wd), 8, 1, None, 1,
                          dl.DL_BF16, ws, ok, None) == -2
    # FP8 weights without scales
    ns = dl.Mat(1, None, dl.DL_FP8_E4M3, 9, 2048, 6144)
    assert lib.dl_moe_ffn(1, 8, 6144, 2048, 1, 1, 2, C.byref(ns), C.byref(wg), C.byref(wd), 8, 1, None, 1,
                          dl.DL_BF16, ws, ok, None) == -1
    # FP8 weights with columns that are not whole 128-blocks
    odd = dl.Mat(1, 1, dl.DL_FP8_E4M3, 9, 2048, 6100)
    assert lib.dl_moe_ffn(1, 8, 6100, 2048, 1, 1, 2, C.byref(odd), C.byref(odd), C.byref(wd), 8, 1, None, 1,
                          dl.DL_BF16, ws, ok, None) in (-2, -4)
    # unsupported output dtype
    assert lib.dl_moe_ffn(1, 8, 6144, 2048, 1, 1, 2, C.byref(wg), C.byref(wg), C.byref(wd), 8, 1, None, 1,
                          dl.DL_I8, ws, ok, None) == -3
    assert lib.dl_moe_route(1, 4, 64, 1, None, 8, 9, 1, 1, None, ws, 1 << 20, None) == -2
    assert lib.dl_moe_route(None, 4, 64, 1, None, 8, 2, 1, 1, None, ws, 1 << 20, None) == -1
    assert lib.dl_moe_route(1, 4, 64, 1, None, 8, 2, 1, 1, None, None, 0, None) == -5


def test_attention_rejects_bad_arguments(lib):
    P = dl.Pages(2, 64, 4, 0x1000, 0x2000)
    ws = C.c_void_p(0x10000)
    # FP8 KV without scales
    assert lib.dl_sparse_attn_decode(C.byref(P), 1, dl.DL_BF16, 1, None, dl.DL_FP8_E4M3, 64, 576, 512, 0.04, 1, 2048,
                                     None, None, None, 0, 1, ws, 1 << 30, None) == -1
    # value wider than the latent
    assert lib.dl_sparse_attn_decode(C.byref(P), 1, dl.DL_BF16, 1, 1, dl.DL_FP8_E4M3, 64, 576, 640, 0.04, 1, 2048,
                                     None, None, None, 0, 1, ws, 1 << 30, None) == -2
    # W_O without a residual
    wo = dl.Mat(1, 1, dl.DL_FP8_E4M3, 1, 6144, 64 * 512)
    assert lib.dl_sparse_attn_decode(C.byref(P), 1, dl.DL_BF16, 1, 1, dl.DL_FP8_E4M3, 64, 576, 512, 0.04, 1, 2048,
                                     None, C.byref(wo), None, 0, 1, ws, 1 << 30, None) == -1


def test_ffn_rejects_sizes_beyond_the_chunk_limits(lib):
    ws = C.c_void_p(0x10000)
    # inter above 16384 (the down projection streams its K in one chunk of at most 128 blocks)
    wg = dl.Mat(1, 1, dl.DL_FP8_E4M3, 9, 16512, 256)
    wd = dl.Mat(1, 1, dl.DL_FP8_E4M3, 9, 256, 16512)
    assert lib.dl_moe_ffn(1, 8, 256, 16512, 1, 1, 2, C.byref(wg), C.byref(wg), C.byref(wd), 8, 1, None, 1,
                          dl.DL_BF16, ws, 1 << 40, None) == -4
    # hidden size above 65536
    wg = dl.Mat(1, 1, dl.DL_FP8_E4M3, 9, 256, 65664)
    wd = dl.Mat(1, 1, dl.DL_FP8_E4M3, 9, 65664, 256)
    assert lib.dl_moe_ffn(1, 8, 65664, 256, 1, 1, 2, C.byref(wg), C.byref(wg), C.byref(wd), 8, 1, None, 1,
                          dl.DL_BF16, ws, 1 << 40, None) == -4
    assert b"65536" in lib.dl_last_error()


def test_kv_append_rejects_bad_arguments(lib):
    P = dl.Pages(2, 64, 4, 0x1000, 0x2000)
    F32, BF16 = dl.DL_F32, dl.DL_BF16
    # NULL pages, NULL latent, NULL key with a key width
    assert lib.dl_kv_append(None, 1, F32, 576, 1, F32, 128, 1.0, 1, 1, 1, None) == -1
    assert lib.dl_kv_append(C.byref(P), None, F32, 576, 1, F32, 128, 1.0, 1, 1, 1, None) == -1
    assert lib.dl_kv_append(C.byref(P), 1, F32, 576, None, F32, 128, 1.0, 1, 1, 1, None) == -1
    # widths out of range
    assert lib.dl_kv_append(C.byref(P), 1, F32, 0, 1, F32, 128, 1.0, 1, 1, 1, None) == -2
    assert lib.dl_kv_append(C.byref(P), 1, F32, 2048, 1, F32, 128, 1.0, 1, 1, 1, None) == -2
    assert lib.dl_kv_append(C.byref(P), 1, F32, 576, 1, F32, 1025, 1.0, 1, 1, 1, None) == -2
    # dtypes other than fp32 / bf16
    assert lib.dl_kv_append(C.byref(P), 1, dl.DL_I8, 576, 1, F32, 128, 1.0, 1, 1, 1, None) == -3
    assert lib.dl_kv_append(C.byref(P), 1, BF16, 576, 1, dl.DL_FP8_E4M3, 128, 1.0, 1, 1, 1, None) == -3
    # key scale not finite and positive
    for ks in (0.0, -1.0, float("inf"), float("nan")):
        assert lib.dl_kv_append(C.byref(P), 1, F32, 576, 1, F32, 128, ks, 1, 1, 1, None) == -2, ks
    assert b"key_scale" in lib.dl_last_error()


def test_pooled_selection_rejects_bad_pools(lib):
    P = dl.Pages(2, 64, 4, 0x1000, 0x2000)
    ws = C.c_void_p(0x10000)
    for pool in (0, 3, 128):  # not a power of two, or wider than a page
        assert lib.dl_indexer_topk_pooled_workspace(C.byref(P), pool) == 0
        assert lib.dl_indexer_topk_pooled(C.byref(P), pool, 1, 1, 16, 128, 512, 1, None, ws, 1 << 30, None) == -4
        assert b"pool" in lib.dl_last_error()
        assert lib.dl_layer_workspace_pooled(C.byref(dl.LayerDesc()), C.byref(P), pool) == 0
    assert lib.dl_indexer_topk_pooled_workspace(C.byref(P), 4) > 0
    # top_pools * pool beyond the selection limit
    assert lib.dl_indexer_topk_pooled(C.byref(P), 64, 1, 1, 16, 128, 2048, 1, None, ws, 1 << 30, None) == -2
    assert lib.dl_layer_step_pooled(C.byref(dl.LayerDesc()), None, 4, ws, 1 << 30, None) == -1


def test_probe_null_rejects_bad_counts(lib):
    assert lib.dl_probe_null(0, 1, None) == -2
    assert lib.dl_probe_null(1025, 1, None) == -2
    assert lib.dl_probe_null(4, 0, None) == -2
    assert lib.dl_probe_null(4, 65537, None) == -2


def test_ffn_ep_rejects_bad_arguments(lib):
    wg = dl.Mat(1, 1, dl.DL_FP8_E4M3, 33, 2048, 6144)
    wd = dl.Mat(1, 1, dl.DL_FP8_E4M3, 33, 6144, 2048)
    ws = C.c_void_p(0x10000)
    need = lib.dl_moe_ffn_workspace(8, 6144, 2048, 8, 32, 1)
    # a negative first expert, no local routed expert, a stack that does not hold n_local + n_shared matrices
    assert lib.dl_moe_ffn_ep(1, 8, 6144, 2048, 1, 1, 8, -1, C.byref(wg), C.byref(wg), C.byref(wd), 32, 1, None, 1,
                             dl.DL_BF16, ws, need, None) == -2
    assert lib.dl_moe_ffn_ep(1, 8, 6144, 2048, 1, 1, 8, 0, C.byref(wg), C.byref(wg), C.byref(wd), 0, 1, None, 1,
                             dl.DL_BF16, ws, need, None) == -2
    assert lib.dl_moe_ffn_ep(1, 8, 6144, 2048, 1, 1, 8, 32, C.byref(wg), C.byref(wg), C.byref(wd), 31, 1, None, 1,
                             dl.DL_BF16, ws, need, None) == -2
    assert b"w_gate" in lib.dl_last_error()


def test_index_key_tiles_reject_bad_shapes(lib):
    ws = C.c_void_p(0x10000)
    # the tiling entry point: NULL, items not a multiple of 16, dim not a multiple of 64 (or out of range), overlap
    assert lib.dl_tile_index_keys(None, 0x2000, 64, 128, None) == -1
    assert lib.dl_tile_index_keys(0x1000, 0x100000, 40, 128, None) == -2
    assert lib.dl_tile_index_keys(0x1000, 0x100000, 64, 48, None) == -2
    assert lib.dl_tile_index_keys(0x1000, 0x100000, 64, 320, None) == -2
    assert lib.dl_tile_index_keys(0x1000, 0x1800, 64, 128, None) == -2
    assert b"overlap" in lib.dl_last_error()
    # an unknown layout, tiles with a key width that is not whole 64-byte chunks, pages of fewer than 16 items
    bad = dl.Pages(2, 64, 4, 0x1000, 0x2000, 7)
    assert lib.dl_indexer_topk(C.byref(bad), 1, 1, 16, 128, 2048, 1, None, ws, 1 << 30, None) == -2
    T = dl.Pages(2, 64, 4, 0x1000, 0x2000, dl.DL_LAYOUT_TILES)
    assert lib.dl_indexer_topk(C.byref(T), 1, 1, 16, 48, 2048, 1, None, ws, 1 << 30, None) == -4
    assert b"tiled" in lib.dl_last_error()
    T8 = dl.Pages(2, 8, 64, 0x1000, 0x2000, dl.DL_LAYOUT_TILES)
    assert lib.dl_indexer_topk(C.byref(T8), 1, 1, 16, 128, 256, 1, None, ws, 1 << 30, None) == -4
    # pools of 8 positions leave 8 pool keys per 64-position page
    assert lib.dl_indexer_topk_pooled(C.byref(T), 8, 1, 1, 16, 128, 64, 1, None, ws, 1 << 30, None) == -4
    assert lib.dl_kv_append(C.byref(T), 1, dl.DL_F32, 576, 1, dl.DL_F32, 48, 1.0, 1, 1, 1, None) == -4
