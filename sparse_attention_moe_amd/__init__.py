"""Python binding of libdl.so, the gfx950 sparse-attention MoE decode layer step.

Argument marshalling only: torch tensors supply device pointers and the current HIP stream; every step
runs in the library's kernels.  Importing works without a GPU (so the C ABI can be inspected), but every
compute call requires the built library and a visible GPU and raises otherwise — there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdl.so")
ABI_VERSION = 3

DL_F32, DL_BF16, DL_FP8_E4M3, DL_I8, DL_I32 = 0, 1, 2, 3, 4
STATUS = {0: "DL_OK", -1: "DL_ERR_NULL", -2: "DL_ERR_SHAPE", -3: "DL_ERR_DTYPE", -4: "DL_ERR_UNSUPPORTED",
          -5: "DL_ERR_WORKSPACE", -6: "DL_ERR_HIP"}

EXPORTS = ["dl_abi_version", "dl_hip_version", "dl_last_error", "dl_pack_weights", "dl_kv_append", "dl_indexer_topk_workspace", "dl_indexer_topk",
           "dl_indexer_topk_rows_workspace", "dl_indexer_topk_rows", "dl_indexer_topk_pooled_workspace",
           "dl_indexer_topk_pooled", "dl_layer_workspace_rows", "dl_layer_step_rows",
           "dl_layer_workspace_pooled", "dl_layer_step_pooled", "dl_indexer_topk_rows_pooled_workspace",
           "dl_indexer_topk_rows_pooled", "dl_layer_workspace_rows_pooled", "dl_layer_step_rows_pooled",
           "dl_sparse_attn_workspace", "dl_sparse_attn_decode", "dl_moe_route_workspace", "dl_moe_route", "dl_moe_route_noalloc",
           "dl_moe_ffn_workspace", "dl_moe_ffn", "dl_moe_ffn_ep", "dl_layer_workspace", "dl_layer_step", "dl_profile_enable",
           "dl_profile_read", "dl_profile_ffn_fused", "dl_probe_read", "dl_probe_null", "dl_tile_index_keys"]
N_PHASES = 9
PHASES = ["indexer_topk", "attention", "projection", "router", "plan_split_h", "expert_gate_up", "split_z",
          "expert_down", "combine"]


class DLError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class Pages(C.Structure):
    _fields_ = [("batch", C.c_int32), ("page_size", C.c_int32), ("max_pages_per_seq", C.c_int32),
                ("seq_lens", C.c_void_p), ("page_table", C.c_void_p), ("key_layout", C.c_int32)]


DL_LAYOUT_ROWS, DL_LAYOUT_TILES = 0, 1


class Mat(C.Structure):
    _fields_ = [("w", C.c_void_p), ("scale", C.c_void_p), ("dtype", C.c_int32), ("count", C.c_int32),
                ("rows", C.c_int32), ("cols", C.c_int32), ("layout", C.c_int32)]


class LayerDesc(C.Structure):
    _fields_ = [("D", C.c_int32), ("n_heads", C.c_int32), ("d_c", C.c_int32), ("d_v", C.c_int32),
                ("idx_heads", C.c_int32), ("idx_dim", C.c_int32), ("top_k", C.c_int32), ("n_routed", C.c_int32),
                ("n_shared", C.c_int32), ("expert_top_k", C.c_int32), ("inter", C.c_int32), ("sm_scale", C.c_float),
                ("q_dt", C.c_int32), ("kv_dt", C.c_int32), ("out_dt", C.c_int32), ("w_uv", Mat), ("w_o", Mat),
                ("w_r", C.c_void_p), ("r_bias", C.c_void_p), ("w_gate", Mat), ("w_up", Mat), ("w_down", Mat)]


class LayerIO(C.Structure):
    _fields_ = [("pages", Pages), ("x", C.c_void_p), ("q", C.c_void_p), ("q_idx", C.c_void_p),
                ("kv_pool", C.c_void_p), ("kv_scale", C.c_void_p), ("k_pool", C.c_void_p), ("y", C.c_void_p),
                ("sel", C.c_void_p), ("h", C.c_void_p), ("experts", C.c_void_p), ("gates", C.c_void_p),
                ("o", C.c_void_p), ("y32", C.c_void_p), ("logits", C.c_void_p)]


_lib = None


def load(require_gpu: bool = True):
    """Load libdl.so (raises if it is missing or its ABI differs)."""
    global _lib
    if require_gpu and not torch.cuda.is_available():
        raise RuntimeError("sparse_attention_moe_amd needs a ROCm GPU (gfx950); none is visible")
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        L = C.CDLL(LIB_PATH)
        P, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
        L.dl_abi_version.restype = C.c_int
        L.dl_hip_version.restype = C.c_int
        L.dl_pack_weights.argtypes = [C.POINTER(Mat), P, P]
        L.dl_last_error.restype = C.c_char_p
        L.dl_kv_append.argtypes = [C.POINTER(Pages), P, i32, i32, P, i32, i32, C.c_float, P, P, P, P]
        L.dl_indexer_topk_pooled_workspace.restype = sz
        L.dl_indexer_topk_pooled_workspace.argtypes = [C.POINTER(Pages), i32]
        L.dl_indexer_topk_pooled.argtypes = [C.POINTER(Pages), i32, P, P, i32, i32, i32, P, P, P, sz, P]
        L.dl_indexer_topk_rows_workspace.restype = sz
        L.dl_indexer_topk_rows_workspace.argtypes = [C.POINTER(Pages), i32]
        L.dl_indexer_topk_rows.argtypes = [C.POINTER(Pages), i32, P, P, i32, i32, i32, P, P, P, sz, P]
        L.dl_layer_workspace_rows.restype = sz
        L.dl_layer_workspace_rows.argtypes = [C.POINTER(LayerDesc), C.POINTER(Pages), i32]
        L.dl_layer_step_rows.argtypes = [C.POINTER(LayerDesc), C.POINTER(LayerIO), i32, P, sz, P]
        L.dl_layer_workspace_pooled.restype = sz
        L.dl_layer_workspace_pooled.argtypes = [C.POINTER(LayerDesc), C.POINTER(Pages), i32]
        L.dl_layer_step_pooled.argtypes = [C.POINTER(LayerDesc), C.POINTER(LayerIO), i32, P, sz, P]
        L.dl_indexer_topk_rows_pooled_workspace.restype = sz
        L.dl_indexer_topk_rows_pooled_workspace.argtypes = [C.POINTER(Pages), i32, i32]
        L.dl_indexer_topk_rows_pooled.argtypes = [C.POINTER(Pages), i32, i32, P, P, i32, i32, i32, P, P, P, sz, P]
        L.dl_layer_workspace_rows_pooled.restype = sz
        L.dl_layer_workspace_rows_pooled.argtypes = [C.POINTER(LayerDesc), C.POINTER(Pages), i32, i32]
        L.dl_layer_step_rows_pooled.argtypes = [C.POINTER(LayerDesc), C.POINTER(LayerIO), i32, i32, P, sz, P]
        L.dl_indexer_topk_workspace.restype = sz
        L.dl_indexer_topk_workspace.argtypes = [C.POINTER(Pages)]
        L.dl_indexer_topk.argtypes = [C.POINTER(Pages), P, P, i32, i32, i32, P, P, P, sz, P]
        L.dl_sparse_attn_workspace.restype = sz
        L.dl_sparse_attn_workspace.argtypes = [i32, i32, i32, i32, C.POINTER(Mat), C.POINTER(Mat)]
        L.dl_sparse_attn_decode.argtypes = [C.POINTER(Pages), P, i32, P, P, i32, i32, i32, i32, C.c_float, P, i32,
                                            C.POINTER(Mat), C.POINTER(Mat), P, i32, P, P, sz, P]
        L.dl_moe_route_workspace.restype = sz
        L.dl_moe_route_workspace.argtypes = [i32, i32, i32]
        L.dl_moe_route.argtypes = [P, i32, i32, P, P, i32, i32, P, P, P, P, sz, P]
        L.dl_moe_route_noalloc.argtypes = [P, i32, i32, P, P, i32, i32, P, P, P, P]
        L.dl_moe_ffn_workspace.restype = sz
        L.dl_moe_ffn_workspace.argtypes = [i32, i32, i32, i32, i32, i32]
        L.dl_moe_ffn.argtypes = [P, i32, i32, i32, P, P, i32, C.POINTER(Mat), C.POINTER(Mat), C.POINTER(Mat), i32,
                                 i32, P, P, i32, P, sz, P]
        L.dl_moe_ffn_ep.argtypes = [P, i32, i32, i32, P, P, i32, i32, C.POINTER(Mat), C.POINTER(Mat), C.POINTER(Mat),
                                    i32, i32, P, P, i32, P, sz, P]
        L.dl_layer_workspace.restype = sz
        L.dl_layer_workspace.argtypes = [C.POINTER(LayerDesc), C.POINTER(Pages)]
        L.dl_layer_step.argtypes = [C.POINTER(LayerDesc), C.POINTER(LayerIO), P, sz, P]
        L.dl_profile_enable.argtypes = [C.c_int]
        L.dl_profile_read.argtypes = [C.POINTER(C.c_double), C.POINTER(C.c_int64)]
        L.dl_profile_ffn_fused.argtypes = []
        L.dl_profile_ffn_fused.restype = C.c_int
        L.dl_probe_read.argtypes = [P, sz, C.POINTER(sz), P]
        L.dl_probe_null.argtypes = [i32, i32, P]
        L.dl_tile_index_keys.argtypes = [P, P, C.c_int64, i32, P]
        if L.dl_abi_version() != ABI_VERSION:
            raise ImportError(f"libdl ABI {L.dl_abi_version()} != {ABI_VERSION}")
        check_hip_version(L.dl_hip_version(), torch.version.hip)
        _lib = L
    return _lib


def check_hip_version(lib_hip: int, torch_hip: Optional[str]):
    """Refuse a library built against another HIP major version than the runtime torch brings into the process
    (the library then runs on that runtime: the one loaded first wins).  lib_hip is HIP_VERSION as the library
    reports it (major * 10^7 + minor * 10^5 + patch); torch_hip is torch.version.hip ("7.0.51831")."""
    if not torch_hip:
        raise ImportError("torch is not a ROCm build (torch.version.hip is empty): libdl needs HIP")
    lib_major = lib_hip // 10_000_000
    torch_major = int(str(torch_hip).split(".")[0])
    if lib_major != torch_major:
        raise ImportError(f"libdl was built against HIP {lib_major}.{lib_hip // 100_000 % 100}, torch runs HIP "
                          f"{torch_hip}: major versions differ")


def _check(rc: int):
    if rc != 0:
        raise DLError(rc, _lib.dl_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    assert t.is_contiguous(), "tensors must be contiguous"
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _dt(t: torch.Tensor) -> int:
    return {torch.float32: DL_F32, torch.bfloat16: DL_BF16, torch.uint8: DL_FP8_E4M3,
            torch.float8_e4m3fn: DL_FP8_E4M3, torch.int8: DL_I8, torch.int32: DL_I32}[t.dtype]


def workspace(nbytes: int, device) -> torch.Tensor:
    """A 256-byte-aligned device buffer (torch's allocator aligns to at least 512 bytes)."""
    t = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    assert t.data_ptr() % 256 == 0
    return t


def pages(seq_lens: torch.Tensor, page_table: torch.Tensor, page_size: int, key_layout: int = DL_LAYOUT_ROWS) -> Pages:
    """dl_pages of a batch; key_layout is the layout of the index-key cache read or written with these pages."""
    return Pages(seq_lens.numel(), page_size, page_table.shape[1], _ptr(seq_lens), _ptr(page_table), key_layout)


def key_tiles_ok(dim: int, items_per_page: int) -> bool:
    """Whether an index-key cache of this shape can be held in DL_LAYOUT_TILES."""
    return dim % 64 == 0 and 64 <= dim <= 256 and items_per_page % 16 == 0


def tile_index_keys(keys: torch.Tensor, stream=None) -> torch.Tensor:
    """DL_LAYOUT_TILES copy of a row-major int8 index-key cache [..., dim]; same shape and bytes."""
    L = load()
    dst = torch.empty_like(keys)
    _check(L.dl_tile_index_keys(_ptr(keys), _ptr(dst), keys.numel() // keys.shape[-1], keys.shape[-1],
                                _stream(stream)))
    return dst


def mat(w: Optional[torch.Tensor], scale: Optional[torch.Tensor] = None, layout: int = DL_LAYOUT_ROWS) -> Mat:
    """dl_mat over a [count, rows, cols] (or [rows, cols]) weight tensor; tiled tensors keep that shape."""
    if w is None:
        return Mat(None, None, 0, 0, 0, 0, 0)
    w3 = w if w.dim() == 3 else w.unsqueeze(0)
    dt = DL_FP8_E4M3 if w.dtype in (torch.uint8, torch.float8_e4m3fn) else DL_F32
    return Mat(_ptr(w), _ptr(scale), dt, w3.shape[0], w3.shape[1], w3.shape[2], layout)


def pack_weights(w: torch.Tensor, scale: torch.Tensor, stream=None) -> torch.Tensor:
    """Tiled copy (DL_LAYOUT_TILES) of a row-major FP8 weight tensor; same shape and bytes."""
    L = load()
    dst = torch.empty_like(w)
    _check(L.dl_pack_weights(C.byref(mat(w, scale)), _ptr(dst), _stream(stream)))
    return dst


# ---------------------------------------------------------------- stage calls
def kv_append(pg: Pages, latent, key, key_scale: float, kv_pool, kv_scale, k_pool, stream=None):
    """Quantise each row's new token into its cache slot (position seq_lens[b] - 1); pools are updated in place."""
    L = load()
    DI = key.shape[-1] if key is not None else 0
    _check(L.dl_kv_append(C.byref(pg), _ptr(latent), _dt(latent), latent.shape[-1], _ptr(key),
                          _dt(key) if key is not None else DL_F32, DI, float(key_scale), _ptr(kv_pool),
                          _ptr(kv_scale), _ptr(k_pool), _stream(stream)))


def indexer_topk(pg: Pages, q_idx, k_pool, top_k: int, sel, sel_score=None, ws=None, stream=None,
                 rows_per_seq: int = 1):
    L = load()
    need = L.dl_indexer_topk_rows_workspace(C.byref(pg), rows_per_seq)
    if ws is None:
        ws = workspace(need, q_idx.device)
    _check(L.dl_indexer_topk_rows(C.byref(pg), rows_per_seq, _ptr(q_idx), _ptr(k_pool), q_idx.shape[1],
                                  q_idx.shape[2], top_k, _ptr(sel), _ptr(sel_score), _ptr(ws), ws.numel(),
                                  _stream(stream)))
    return sel


def indexer_topk_pooled(pg: Pages, pool: int, q_idx, pool_keys, top_pools: int, sel, pool_score=None, ws=None,
                        stream=None, rows_per_seq: int = 1):
    """Pool-granular selection: sel [B * rows_per_seq, top_pools * pool] positions of the kept pools (see dl.h)."""
    L = load()
    if rows_per_seq == 1:
        if ws is None:
            ws = workspace(L.dl_indexer_topk_pooled_workspace(C.byref(pg), pool), q_idx.device)
        _check(L.dl_indexer_topk_pooled(C.byref(pg), pool, _ptr(q_idx), _ptr(pool_keys), q_idx.shape[1],
                                        q_idx.shape[2], top_pools, _ptr(sel), _ptr(pool_score), _ptr(ws), ws.numel(),
                                        _stream(stream)))
        return sel
    if ws is None:
        ws = workspace(L.dl_indexer_topk_rows_pooled_workspace(C.byref(pg), rows_per_seq, pool), q_idx.device)
    _check(L.dl_indexer_topk_rows_pooled(C.byref(pg), rows_per_seq, pool, _ptr(q_idx), _ptr(pool_keys),
                                         q_idx.shape[1], q_idx.shape[2], top_pools, _ptr(sel), _ptr(pool_score),
                                         _ptr(ws), ws.numel(), _stream(stream)))
    return sel


def sparse_attn_decode(pg: Pages, q, kv_pool, kv_scale, n_heads, d_c, d_v, sm_scale, sel, top_k, out,
                       w_uv: Optional[Mat] = None, w_o: Optional[Mat] = None, residual=None, ws=None, stream=None):
    L = load()
    puv = C.byref(w_uv) if w_uv is not None else None
    po = C.byref(w_o) if w_o is not None else None
    need = L.dl_sparse_attn_workspace(pg.batch, n_heads, d_v, top_k, puv, po)
    if ws is None:
        ws = workspace(need, q.device)
    kv_dt = DL_F32 if kv_pool.dtype == torch.float32 else DL_FP8_E4M3
    res_dt = _dt(residual) if residual is not None else 0
    _check(L.dl_sparse_attn_decode(C.byref(pg), _ptr(q), _dt(q), _ptr(kv_pool), _ptr(kv_scale), kv_dt, n_heads, d_c,
                                   d_v, float(sm_scale), _ptr(sel), top_k, puv, po, _ptr(residual), res_dt, _ptr(out),
                                   _ptr(ws), ws.numel(), _stream(stream)))
    return out


def moe_route(h, w_r, bias, top_k, experts, gates, logits=None, ws=None, stream=None):
    L = load()
    B, D = h.shape
    E = w_r.shape[0]
    if ws is None:
        ws = workspace(L.dl_moe_route_workspace(B, D, E), h.device)
    _check(L.dl_moe_route(_ptr(h), B, D, _ptr(w_r), _ptr(bias), E, top_k, _ptr(experts), _ptr(gates), _ptr(logits),
                          _ptr(ws), ws.numel(), _stream(stream)))
    return experts, gates


def moe_route_noalloc(h, w_r, bias, top_k, experts, gates, logits=None, stream=None):
    """dl_moe_route_noalloc: the router with the library's own static device scratch (no workspace, no
    allocation); calls that overlap on one GPU race."""
    L = load()
    B, D = h.shape
    E = w_r.shape[0]
    _check(L.dl_moe_route_noalloc(_ptr(h), B, D, _ptr(w_r), _ptr(bias), E, top_k, _ptr(experts), _ptr(gates),
                                  _ptr(logits), _stream(stream)))
    return experts, gates


def moe_ffn(h, experts, gates, w_gate: Mat, w_up: Mat, w_down: Mat, n_routed, n_shared, out, residual=None,
            ws=None, stream=None):
    L = load()
    B, D = h.shape
    ke = experts.shape[1]
    inter = w_gate.rows
    if ws is None:
        ws = workspace(L.dl_moe_ffn_workspace(B, D, inter, ke, n_routed, n_shared), h.device)
    _check(L.dl_moe_ffn(_ptr(h), B, D, inter, _ptr(experts), _ptr(gates), ke, C.byref(w_gate), C.byref(w_up),
                        C.byref(w_down), n_routed, n_shared, _ptr(residual), _ptr(out), _dt(out), _ptr(ws), ws.numel(),
                        _stream(stream)))
    return out


def moe_ffn_ep(h, experts, gates, expert_lo: int, w_gate: Mat, w_up: Mat, w_down: Mat, n_local, n_shared, out,
               residual=None, ws=None, stream=None):
    """dl_moe_ffn_ep: the FFN share of the experts [expert_lo, expert_lo + n_local) (+ n_shared shared experts)."""
    L = load()
    B, D = h.shape
    ke = experts.shape[1]
    inter = w_gate.rows
    if ws is None:
        ws = workspace(L.dl_moe_ffn_workspace(B, D, inter, ke, n_local, n_shared), h.device)
    _check(L.dl_moe_ffn_ep(_ptr(h), B, D, inter, _ptr(experts), _ptr(gates), ke, expert_lo, C.byref(w_gate),
                           C.byref(w_up), C.byref(w_down), n_local, n_shared, _ptr(residual), _ptr(out), _dt(out),
                           _ptr(ws), ws.numel(), _stream(stream)))
    return out


def profile_ffn_fused() -> int:
    """1 if the most recent expert FFN ran as one kernel, 0 if as three, -1 before the first (measurement aid)."""
    return int(load().dl_profile_ffn_fused())


def probe_read(buf: torch.Tensor, stream=None) -> int:
    """Enqueue one streaming read of buf (measurement aid); returns the number of bytes it reads."""
    L = load()
    n = C.c_size_t(0)
    _check(L.dl_probe_read(_ptr(buf), buf.numel() * buf.element_size(), C.byref(n), _stream(stream)))
    return n.value


def probe_null(n_kernels: int, blocks: int, stream=None):
    """Enqueue n_kernels dependent launches of an empty kernel of `blocks` workgroups (measurement aid)."""
    _check(load().dl_probe_null(n_kernels, blocks, _stream(stream)))


def profile_enable(on: bool):
    _check(load().dl_profile_enable(1 if on else 0))


def profile_read():
    """-> (dict phase -> summed ms, number of steps) for the steps recorded since the last read."""
    arr = (C.c_double * N_PHASES)()
    n = C.c_int64()
    _check(load().dl_profile_read(arr, C.byref(n)))
    return {PHASES[i]: arr[i] for i in range(N_PHASES)}, n.value


# ---------------------------------------------------------------- whole step
class LayerStep:
    """dl_layer_step over one layer instance given as a dict of device tensors (names as synth.make_layer).

    Holds the descriptor, the io struct and the workspace, so repeated calls only enqueue."""

    def __init__(self, spec, t: Dict[str, torch.Tensor], debug: bool = False, tiles: bool = True,
                 drop_rows: bool = False):
        """tiles: FP8 weights are re-tiled once (dl_pack_weights) and the step streams the tiles.
        drop_rows: afterwards drop the row-major weights from `t` (saves memory when nothing else needs them)."""
        L = load()
        self.spec, self.t = spec, t
        dev = t["x"].device
        self.R = getattr(spec, "R", 1)
        self.pool = getattr(spec, "pool", 1)  # > 1: pool-granular selection over t["pool_keys"]
        B = spec.B * self.R  # rows
        self.keep = []
        # the index keys in DL_LAYOUT_TILES where their shape allows (the scoring kernel's loads are then 1 KB
        # contiguous); the step reads them through the pages' key_layout
        key_name = "pool_keys" if self.pool > 1 else "k_pool"
        keys = t[key_name]
        self.key_layout = DL_LAYOUT_ROWS
        if tiles and keys is not None and keys.dtype == torch.int8 and key_tiles_ok(spec.DI, spec.page_size // self.pool):
            keys = tile_index_keys(keys)
            self.key_layout = DL_LAYOUT_TILES
        self.keys = keys
        self.pg = pages(t["seq_lens"], t["page_table"], spec.page_size, self.key_layout)
        d = LayerDesc()
        d.D, d.n_heads, d.d_c, d.d_v = spec.D, spec.H, spec.Dc, spec.Dv
        d.idx_heads, d.idx_dim, d.top_k = spec.HI, spec.DI, spec.topk
        d.n_routed, d.n_shared, d.expert_top_k, d.inter = spec.E, spec.n_shared, spec.ke, spec.I
        d.sm_scale = spec.scale
        self.w = {}
        for name in ("w_uv", "w_o", "w_gate", "w_up", "w_down"):
            w = t.get(name)
            lay = DL_LAYOUT_ROWS
            if w is not None and tiles and w.dtype == torch.uint8:
                w = pack_weights(w, t[name + "_scale"])
                lay = DL_LAYOUT_TILES
                if drop_rows:
                    t[name] = None
            self.w[name] = (w, t.get(name + "_scale"), lay)
        d.q_dt = _dt(t["x"])
        d.kv_dt = DL_F32 if t["kv"].dtype == torch.float32 else DL_FP8_E4M3
        d.out_dt = DL_BF16 if spec.fp8 else DL_F32
        d.w_uv = self.mat("w_uv")
        d.w_o = self.mat("w_o")
        d.w_r = _ptr(t["w_r"])
        d.r_bias = _ptr(t["r_bias"])
        d.w_gate = self.mat("w_gate")
        d.w_up = self.mat("w_up")
        d.w_down = self.mat("w_down")
        self.desc = d
        self.y = torch.empty(B, spec.D, dtype=torch.bfloat16 if spec.fp8 else torch.float32, device=dev)
        io = LayerIO()
        io.pages = self.pg
        io.x, io.q, io.q_idx = _ptr(t["x"]), _ptr(t["q"]), _ptr(t["q_idx"])
        io.kv_pool, io.kv_scale, io.k_pool = _ptr(t["kv"]), _ptr(t.get("kv_scale")), _ptr(self.keys)
        io.y = _ptr(self.y)
        self.dbg = {}
        if debug:
            self.dbg = dict(sel=torch.empty(B, spec.topk, dtype=torch.int32, device=dev),
                            h=torch.empty(B, spec.D, dtype=torch.float32, device=dev),
                            experts=torch.empty(B, spec.ke, dtype=torch.int32, device=dev),
                            gates=torch.empty(B, spec.ke, dtype=torch.float32, device=dev),
                            o=torch.empty(B, spec.H, spec.Dv, dtype=torch.float32, device=dev),
                            y32=torch.empty(B, spec.D, dtype=torch.float32, device=dev),
                            logits=torch.empty(B, spec.E, dtype=torch.float32, device=dev))
        self.io = io
        self.debug_outputs(debug)
        if self.R > 1 and self.pool > 1:
            n = L.dl_layer_workspace_rows_pooled(C.byref(d), C.byref(self.pg), self.R, self.pool)
        elif self.pool > 1:
            n = L.dl_layer_workspace_pooled(C.byref(d), C.byref(self.pg), self.pool)
        else:
            n = L.dl_layer_workspace_rows(C.byref(d), C.byref(self.pg), self.R)
        if n == 0:
            raise ValueError(f"layer workspace: unsupported shape (R={self.R}, pool={self.pool})")
        self.ws = workspace(n, dev)

    def mat(self, name: str) -> Mat:
        w, sc, lay = self.w[name]
        return mat(w, sc, lay)

    def debug_outputs(self, on: bool):
        """Point the step's optional debug outputs at self.dbg (on) or pass NULL for them (off: the production
        step, which writes only y)."""
        for k, v in self.dbg.items():
            setattr(self.io, k, _ptr(v) if on else None)

    def __call__(self, stream=None):
        if self.R > 1 and self.pool > 1:
            _check(load().dl_layer_step_rows_pooled(C.byref(self.desc), C.byref(self.io), self.R, self.pool,
                                                    _ptr(self.ws), self.ws.numel(), _stream(stream)))
        elif self.pool > 1:
            _check(load().dl_layer_step_pooled(C.byref(self.desc), C.byref(self.io), self.pool, _ptr(self.ws),
                                               self.ws.numel(), _stream(stream)))
        else:
            _check(load().dl_layer_step_rows(C.byref(self.desc), C.byref(self.io), self.R, _ptr(self.ws),
                                             self.ws.numel(), _stream(stream)))
        return self.y
