"""CPU oracle for the sparse-attention MoE decode layer step (ctypes over oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline use it; the product path never does.  It shares no code with the HIP
library.  All arithmetic is in oracle.c (fp64, plain loops); this module only
moves numpy arrays in and out.  Every function follows the passage cited at the
matching C function.

Parity pins live in tests/test_oracle_pins.py.  Pinned: FP8/bf16 decode and
rounding, indexer, top-k, attention, projection, router, FFN, the current-token
append (closed forms, brute force, invariants, library special cases).  None is
"parity unpinned".
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

O_F32, O_BF16, O_FP8 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile oracle.c (gcc -O2, no fast-math, OpenMP) into liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Mat(C.Structure):
    _fields_ = [("w", C.c_void_p), ("scale", C.c_void_p), ("dtype", C.c_int32),
                ("count", C.c_int32), ("rows", C.c_int32), ("cols", C.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = C.CDLL(_LIB_PATH)
        P = C.c_void_p
        i32 = C.c_int32
        L.o_fp8_e4m3fn.restype = C.c_double
        L.o_fp8_e4m3fn.argtypes = [C.c_uint8]
        L.o_bf16_round.restype = C.c_uint16
        L.o_bf16_round.argtypes = [C.c_double]
        L.o_bf16_to_double.restype = C.c_double
        L.o_bf16_to_double.argtypes = [C.c_uint16]
        L.o_indexer_scores.argtypes = [P, P, P, i32, i32, i32, i32, P]
        L.o_topk.argtypes = [P, i32, i32, P]
        L.o_sparse_attention.argtypes = [P, i32, P, i32, P, P, i32, i32, i32, i32, C.c_double, P, i32, P, P]
        L.o_out_proj.argtypes = [P, i32, i32, C.POINTER(_Mat), C.POINTER(_Mat), P, i32, i32, P]
        L.o_router.argtypes = [P, P, P, i32, i32, i32, P, P, P]
        L.o_ffn.argtypes = [P, P, P, i32, C.POINTER(_Mat), C.POINTER(_Mat), C.POINTER(_Mat), i32, i32, i32, i32, P]
        L.o_round_out.argtypes = [P, C.c_long, i32, P]
        L.o_fp8_round.restype = C.c_uint8
        L.o_fp8_round.argtypes = [C.c_double]
        L.o_kv_append_row.argtypes = [P, i32, i32, P, i32, i32, C.c_float, P, P, P]
        L.o_threads.restype = C.c_int
        L.o_init()
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _act(a: np.ndarray):
    """(contiguous array, dtype code) for an activation given as fp32 or bf16 bit patterns."""
    if a.dtype == np.uint16:
        return _c(a, np.uint16), O_BF16
    return _c(a, np.float32), O_F32


# ------------------------------------------------------------------ decoding
def threads() -> int:
    """OpenMP threads the oracle's loops use."""
    return int(lib().o_threads())


def fp8_decode(codes) -> np.ndarray:
    L = lib()
    c = np.asarray(codes, dtype=np.uint8).ravel()
    return np.array([L.o_fp8_e4m3fn(int(v)) for v in c]).reshape(np.shape(codes))


def fp8_round(x) -> np.ndarray:
    """Real values -> e4m3fn codes (uint8): nearest, ties to even, saturating at 448."""
    L = lib()
    v = np.asarray(x, dtype=np.float64)
    return np.array([L.o_fp8_round(float(t)) for t in v.ravel()], dtype=np.uint8).reshape(v.shape)


def bf16_round(x) -> np.ndarray:
    """fp64 values -> bf16 bit patterns (uint16), round to nearest even."""
    L = lib()
    x = _c(x, np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    L.o_round_out(_p(x), x.size, O_BF16, _p(out))
    return out


def bf16_to_f64(b) -> np.ndarray:
    L = lib()
    return np.array([L.o_bf16_to_double(int(v)) for v in np.asarray(b).ravel()]).reshape(np.shape(b))


# ------------------------------------------------------------------- stages
def kv_append_row(latent: np.ndarray, key: np.ndarray, key_scale: float):
    """One row of the current-token append: (latent codes uint8 [Dc], block scales fp32 [ceil(Dc/128)],
    indexer key int8 [DI]) for a latent and key given as fp32 or bf16 bit patterns."""
    L = lib()
    lat, lat_dt = _act(np.ravel(latent))
    k, k_dt = _act(np.ravel(key))
    Dc, DI = lat.size, k.size
    codes = np.empty(Dc, dtype=np.uint8)
    scales = np.empty((Dc + 127) // 128, dtype=np.float32)
    kout = np.empty(DI, dtype=np.int8)
    if L.o_kv_append_row(_p(lat), lat_dt, Dc, _p(k), k_dt, DI, float(key_scale), _p(codes), _p(scales), _p(kout)):
        raise ValueError("kv_append_row: bad arguments")
    return codes, scales, kout



def indexer_scores(q_idx: np.ndarray, k_pool: np.ndarray, page_table_row: np.ndarray, L: int) -> np.ndarray:
    """q_idx int8 [HI, DI]; k_pool int8 [P, page, DI]; -> int32 [L]."""
    q = _c(q_idx, np.int8)
    kp = _c(k_pool, np.int8)
    pt = _c(page_table_row, np.int32)
    HI, DI = q.shape
    out = np.zeros(max(L, 1), dtype=np.int32)
    if L > 0:
        rc = lib().o_indexer_scores(_p(q), _p(kp), _p(pt), L, kp.shape[1], HI, DI, _p(out))
        if rc != 0:
            raise OverflowError("indexer score exceeds int32")
    return out[:L]


def topk(scores: np.ndarray, k: int) -> np.ndarray:
    s = _c(scores, np.int32)
    sel = np.empty(k, dtype=np.int32)
    if lib().o_topk(_p(s), s.size, k, _p(sel)) != 0:
        raise MemoryError
    return sel


def pooled_topk(q_idx: np.ndarray, pool_keys: np.ndarray, page_table_row: np.ndarray, L: int, pool: int,
                top_pools: int):
    """Pool-granular selection (Kiln: a separate pool-key cache, "What moved the number ..."; decode gathers
    the selected pools, "The decode kernels, and why they are opt-in").  Reading: pool p covers positions
    [p pool, (p + 1) pool); its key is entry p of the pool-key cache (pool_keys [pages, page / pool, DI], paged
    like the position keys); the ceil(L / pool) pools are scored like positions and the top pools kept under the
    same order; each kept pool, in ascending order, contributes its positions below L.  Returns (sel positions
    [top_pools * pool] with -1 padding, pool scores [ceil(L / pool)], kept pools [top_pools])."""
    Lp = (L + pool - 1) // pool
    scores = indexer_scores(q_idx, pool_keys, page_table_row, Lp)
    pools = topk(scores, top_pools)
    sel = np.full(top_pools * pool, -1, dtype=np.int32)
    for k, pl in enumerate(pools):
        if pl < 0:
            break
        for j in range(pool):
            p = int(pl) * pool + j
            sel[k * pool + j] = p if p < L else -1
    return sel, scores, pools


def attention(q_b: np.ndarray, kv: np.ndarray, kv_scale: Optional[np.ndarray], page_table_row: np.ndarray,
              sel: np.ndarray, sm_scale: float, Dv: int, want_p: bool = False):
    """q_b [H, Dc] (fp32 or bf16 bits); kv [P, page, Dc] uint8 codes or fp32; -> o fp64 [H, Dv]."""
    q, qdt = _act(q_b)
    H, Dc = q.shape
    if kv.dtype == np.uint8:
        kvc, kdt = _c(kv, np.uint8), O_FP8
        ks = _c(kv_scale, np.float32)
    else:
        kvc, kdt, ks = _c(kv, np.float32), O_F32, None
    pt = _c(page_table_row, np.int32)
    s = _c(sel, np.int32)
    o = np.empty((H, Dv), dtype=np.float64)
    p = np.empty((H, s.size), dtype=np.float64) if want_p else None
    rc = lib().o_sparse_attention(_p(q), qdt, _p(kvc), kdt, _p(ks), _p(pt), kvc.shape[1], H, Dc, Dv,
                                  float(sm_scale), _p(s), s.size, _p(o), _p(p))
    if rc != 0:
        raise MemoryError
    return (o, p) if want_p else o


def _mat(w: np.ndarray, scale: Optional[np.ndarray], keep: list):
    if w.ndim == 2:
        w = w[None]
    if w.dtype == np.uint8:
        wc, dt = _c(w, np.uint8), O_FP8
        sc = _c(scale, np.float32)
    else:
        wc, dt, sc = _c(w, np.float32), O_F32, None
    keep += [wc, sc]
    m = _Mat(wc.ctypes.data, None if sc is None else sc.ctypes.data, dt, wc.shape[0], wc.shape[1], wc.shape[2])
    return m


def out_proj(o: np.ndarray, w_uv, w_uv_scale, w_o, w_o_scale, x_b: np.ndarray) -> np.ndarray:
    """o fp64 [H, Dv] -> h fp64 [D] = x + W_O concat_h(W_UV[h] o[h])."""
    keep: list = []
    oc = _c(o, np.float64)
    H, Dv = oc.shape
    muv = _mat(w_uv, w_uv_scale, keep) if w_uv is not None else None
    mo = _mat(w_o, w_o_scale, keep)
    x, xdt = _act(x_b)
    D = x.size
    h = np.empty(D, dtype=np.float64)
    rc = lib().o_out_proj(_p(oc), H, Dv, C.byref(muv) if muv is not None else None, C.byref(mo),
                          _p(x), xdt, D, _p(h))
    if rc != 0:
        raise MemoryError
    return h


def router(h: np.ndarray, w_r: np.ndarray, bias: Optional[np.ndarray], ke: int):
    """-> (logits fp64 [E], experts int32 [ke], gates fp64 [ke])."""
    hc = _c(h, np.float64)
    wr = _c(w_r, np.float32)
    E, D = wr.shape
    b = None if bias is None else _c(bias, np.float32)
    lg = np.empty(E, dtype=np.float64)
    ex = np.empty(ke, dtype=np.int32)
    g = np.empty(ke, dtype=np.float64)
    if lib().o_router(_p(hc), _p(wr), _p(b), E, D, ke, _p(lg), _p(ex), _p(g)) != 0:
        raise MemoryError
    return lg, ex, g


def ffn(h: np.ndarray, experts: Sequence[int], gates: Sequence[float], expert_weights, n_routed: int,
        n_shared: int) -> np.ndarray:
    """Dense per-token expert loop.  expert_weights(e) -> (wg, sg, wu, su, wd, sd) numpy for expert e
    (scales None for fp32).  Returns y fp64 [D] (unrounded): h + sum over slots of gate * expert output + the
    shared experts.  A negative expert id marks a slot computed elsewhere (an expert held by another GPU in an
    expert-parallel layout): it adds nothing."""
    ids = [int(e) for e in experts if int(e) >= 0] + [n_routed + s for s in range(n_shared)]
    if not ids:
        return _c(h, np.float64).copy()
    uniq = sorted(set(ids))
    loc = {e: i for i, e in enumerate(uniq)}
    parts = [expert_weights(e) for e in uniq]
    wg = np.stack([p[0] for p in parts]); wu = np.stack([p[2] for p in parts]); wd = np.stack([p[4] for p in parts])
    f8 = wg.dtype == np.uint8
    sg = np.stack([p[1] for p in parts]) if f8 else None
    su = np.stack([p[3] for p in parts]) if f8 else None
    sd = np.stack([p[5] for p in parts]) if f8 else None
    keep: list = []
    mg, mu, md = _mat(wg, sg, keep), _mat(wu, su, keep), _mat(wd, sd, keep)
    # local numbering: routed ids map into the compact stack; the shared experts are the last entries
    ke = len(experts)
    lex = np.array([loc[int(e)] if int(e) >= 0 else -1 for e in experts], dtype=np.int32)
    # place shared experts at local index n_routed_local + s by building an order where they come last
    n_loc_routed = len(uniq) - n_shared
    assert all(loc[n_routed + s] == n_loc_routed + s for s in range(n_shared))
    g = _c(gates, np.float64)
    hc = _c(h, np.float64)
    D = hc.size
    I = wg.shape[1]
    y = np.empty(D, dtype=np.float64)
    if lib().o_ffn(_p(hc), _p(lex), _p(g), ke, C.byref(mg), C.byref(mu), C.byref(md), n_loc_routed, n_shared,
                   D, I, _p(y)) != 0:
        raise MemoryError
    return y


def round_out(y: np.ndarray, bf16: bool) -> np.ndarray:
    yc = _c(y, np.float64)
    if bf16:
        out = np.empty(yc.shape, dtype=np.uint16)
        lib().o_round_out(_p(yc), yc.size, O_BF16, _p(out))
    else:
        out = np.empty(yc.shape, dtype=np.float32)
        lib().o_round_out(_p(yc), yc.size, O_F32, _p(out))
    return out


# ------------------------------------------------------------ whole layer
def _np(t):
    """torch tensor (any device) or numpy -> host numpy; bf16 -> uint16 bit patterns."""
    if isinstance(t, np.ndarray):
        return t
    import torch
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class LayerOracle:
    """Runs the oracle on chosen rows of one generated layer (dict of tensors from synth.make_layer).

    Host copies of big tensors are made lazily; expert weights are fetched per expert, so a full-size
    layer can be checked on sampled rows without copying every expert to the host.
    """

    def __init__(self, spec, t: Dict):
        self.spec, self.t = spec, t
        self._cache: Dict[str, np.ndarray] = {}
        self._exp: Dict[int, tuple] = {}

    def a(self, name):
        if name not in self._cache:
            v = self.t.get(name)
            self._cache[name] = None if v is None else _np(v)
        return self._cache[name]

    def expert(self, e: int):
        if e not in self._exp:
            t = self.t
            f8 = self.spec.fp8
            g = lambda n: _np(t[n][e])
            self._exp[e] = (g("w_gate"), g("w_gate_scale") if f8 else None, g("w_up"),
                            g("w_up_scale") if f8 else None, g("w_down"), g("w_down_scale") if f8 else None)
        return self._exp[e]

    def row(self, b: int, stages=("sel", "o", "h", "route", "y")) -> Dict[str, np.ndarray]:
        """Row b of the step.  With R = spec.R query rows per sequence (multi-row decode: the verification of
        multi-token-prediction drafts, TileRT "Running the Generation Example with Multi-Token Prediction
        (MTP)" and Kiln "What did we measure that did not pay?"), row b is the token at position
        seq_lens[b // R] - R + b % R of sequence b // R and sees the positions up to its own (reading: causal
        among the R rows, like any decode token); everything after the visible length is per row."""
        sp = self.spec
        R = getattr(sp, "R", 1)
        seq, rr = b // R, b % R
        L = max(0, int(self.a("seq_lens")[seq]) - (R - 1 - rr))
        pt = self.a("page_table")[seq]
        r: Dict[str, np.ndarray] = {}
        pool = getattr(sp, "pool", 1)
        if pool > 1:  # pool-granular selection: top_k positions are top_k / pool whole pools
            r["sel"], r["scores"], r["pools"] = pooled_topk(self.a("q_idx")[b], self.a("pool_keys"), pt, L, pool,
                                                            sp.topk // pool)
        else:
            r["scores"] = indexer_scores(self.a("q_idx")[b], self.a("k_pool"), pt, L)
            r["sel"] = topk(r["scores"], sp.topk)
        if "o" not in stages:
            return r
        r["o"] = attention(self.a("q")[b], self.a("kv"), self.a("kv_scale"), pt, r["sel"], sp.scale, sp.Dv)
        if "h" not in stages:
            return r
        r["h"] = out_proj(r["o"], self.a("w_uv"), self.a("w_uv_scale"), self.a("w_o"), self.a("w_o_scale"),
                          self.a("x")[b])
        if "route" not in stages:
            return r
        r["logits"], r["experts"], r["gates"] = router(r["h"], self.a("w_r"), self.a("r_bias"), sp.ke)
        if "y" not in stages:
            return r
        r["y64"] = ffn(r["h"], r["experts"], r["gates"], self.expert, sp.E, sp.n_shared)
        r["y"] = round_out(r["y64"], sp.fp8)
        return r
