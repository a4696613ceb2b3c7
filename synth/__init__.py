"""Seeded synthetic inputs for the sparse-attention MoE decode layer step.

This module only draws random numbers and lays them out.  It holds none of the
method's arithmetic: no scoring, selection, attention, routing or FFN.  Both the
CPU oracle (through the tests) and the HIP library consume the tensors it
returns, so the two sides always read the same bytes.

Random numbers come from torch's Philox generator on the device the tensors are
made on, one generator per tensor name (seeded from ``seed``, ``instance`` and a
CRC32 of the name).  Big configurations are generated on the GPU; small ones on
the CPU.  Either way the tensors are materialised once and then handed to both
sides.

Encoding to FP8 (OCP e4m3fn) uses torch's float8 conversion (round to nearest
even, clamped to +-448) with block scale = amax/448, which is how the cached
latents and the expert weights of the model on the pages are stored ("FP8
weights with 128 x 128 block scales", Introducing Kiln, section "How was Kiln
measured against vLLM on H200?").  The scale layout is the plain one: one fp32
per 128 x 128 weight block, one fp32 per (token, 128-feature block) of the
latent cache.
"""
from __future__ import annotations

import dataclasses
import math
import zlib
from typing import Dict, List, Optional

import torch

FP8_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    """Shapes and value distributions of one decode layer-step workload."""

    name: str
    B: int                      # batch rows (sequences)
    D: int                      # hidden size
    H: int                      # query heads
    Dc: int                     # latent (key) width, shared by all heads
    Dv: int                     # value width: the first Dv latent features
    head_dim: int               # per-head output of W_UV (0: no W_UV)
    HI: int                     # indexer heads
    DI: int                     # indexer dim
    topk: int                   # positions kept per sequence
    E: int                      # routed experts
    ke: int                     # experts per token
    n_shared: int               # shared experts (gate 1)
    I: int                      # SwiGLU intermediate size
    seq_lens: tuple             # cached positions per row (0 = padding row)
    page_size: int = 64
    fp8: bool = True            # FP8 KV + FP8 weights + bf16 activations, else all fp32
    router_std: Optional[float] = None   # None -> 1/sqrt(D)
    zipf_s: float = 0.0         # >0: router bias ln p_e, p_e ~ rank^-s (skewed popularity)
    permute_pages: bool = False
    extra_pages: int = 0        # pool pages nobody references (catch stray reads)
    key_values: str = "uniform"  # indexer q/k: "uniform" in [-127,127] or "ternary" {-1,0,1}
    dup_router_rows: bool = False  # make expert 1 a copy of expert 0 (exact router ties)
    sm_scale: Optional[float] = None     # None -> 1/sqrt(Dc)
    R: int = 1                  # query rows per sequence (multi-row decode); per-row tensors have B * R rows
    pool: int = 1               # >1: also a pool-key cache, one indexer key per pool of `pool` positions

    @property
    def wo_in(self) -> int:
        return self.H * (self.head_dim if self.head_dim else self.Dv)

    @property
    def max_pages(self) -> int:
        return max(1, max((l + self.page_size - 1) // self.page_size for l in self.seq_lens))

    @property
    def scale(self) -> float:
        return self.sm_scale if self.sm_scale is not None else 1.0 / math.sqrt(self.Dc)

    @property
    def n_kv_blocks(self) -> int:
        return (self.Dc + 127) // 128


def _ragged_lens(seed: int, B: int, lo: int, hi: int) -> tuple:
    g = torch.Generator().manual_seed(seed * 1000003 + 17)
    return tuple(int(v) for v in torch.randint(lo, hi + 1, (B,), generator=g))


def config(n: int) -> LayerSpec:
    """The five named workloads (1 = tiny fp32 layer ... 5 = batch 64 at 8K)."""
    big = dict(D=6144, H=64, Dc=576, Dv=512, head_dim=128, HI=16, DI=128, topk=2048,
               E=256, ke=8, n_shared=1, I=2048, fp8=True)
    if n == 1:
        return LayerSpec("tiny-fp32-b1-4k", B=1, D=512, H=8, Dc=64, Dv=64, head_dim=0, HI=1, DI=32,
                         topk=256, E=8, ke=2, n_shared=0, I=256, seq_lens=(4096,), fp8=False,
                         router_std=1.0)
    if n == 2:
        return LayerSpec("b8-128k", B=8, seq_lens=(131072,) * 8, **big)
    if n == 3:
        return LayerSpec("b1-1m", B=1, seq_lens=(1048576,), **big)
    if n == 4:
        return LayerSpec("b12-ragged-64k-256k-zipf", B=12, seq_lens=_ragged_lens(0, 12, 65536, 262144),
                         permute_pages=True, zipf_s=1.1, **big)
    if n == 5:
        return LayerSpec("b64-8k", B=64, seq_lens=(8192,) * 64, **big)
    raise ValueError(f"no config {n}")


def _gen(device, seed: int, instance: int, name: str) -> torch.Generator:
    h = zlib.crc32(name.encode()) & 0xFFFFFFFF
    g = torch.Generator(device=device)
    g.manual_seed((seed * 0x9E3779B1 + instance * 0x85EBCA77 + h) & 0x7FFFFFFFFFFFFFFF)
    return g


def _randn(shape, device, seed, inst, name, std=1.0) -> torch.Tensor:
    t = torch.randn(shape, generator=_gen(device, seed, inst, name), device=device, dtype=torch.float32)
    return t * std if std != 1.0 else t


def quant_fp8_blocks(w: torch.Tensor, br: int, bc: int):
    """w [..., R, C] fp32 -> (codes uint8 [..., R, C], scale fp32 [..., ceil(R/br), ceil(C/bc)]).

    scale = amax over the block / 448 (1 if the block is all zero);
    code = e4m3fn(clamp(w / scale, +-448)), round to nearest even.
    """
    *lead, R, C = w.shape
    nbr, nbc = (R + br - 1) // br, (C + bc - 1) // bc
    pad = torch.zeros(*lead, nbr * br, nbc * bc, dtype=torch.float32, device=w.device)
    pad[..., :R, :C] = w
    blk = pad.reshape(*lead, nbr, br, nbc, bc)
    amax = blk.abs().amax(dim=(-3, -1))                       # [..., nbr, nbc]
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    q = (blk / scale[..., :, None, :, None]).clamp_(-FP8_MAX, FP8_MAX)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(*lead, nbr * br, nbc * bc)[..., :R, :C]
    return codes.contiguous(), scale.contiguous()


def _int8_uniform(shape, device, seed, inst, name, kind):
    g = _gen(device, seed, inst, name)
    if kind == "ternary":
        return torch.randint(-1, 2, shape, generator=g, device=device, dtype=torch.int8)
    return torch.randint(-127, 128, shape, generator=g, device=device, dtype=torch.int8)


def make_layer(spec: LayerSpec, seed: int = 0, device="cpu", instance: int = 0,
               weights: bool = True) -> Dict[str, torch.Tensor]:
    """All tensors of one layer instance and one decode step, on ``device``.

    Returned keys (dtype, shape):
      seq_lens int32 [B]; page_table int32 [B, max_pages]; n_pages
      x   act [B*R, D]          (bf16, or fp32 when not spec.fp8; R = spec.R query rows per sequence)
      q   act [B*R, H, Dc]
      q_idx int8 [B*R, HI, DI];  k_pool int8 [P, page, DI]
      kv  uint8/fp32 [P, page, Dc];  kv_scale fp32 [P, page, ceil(Dc/128)] (fp8 only)
      w_uv (fp8 only) uint8 [H, head_dim, Dv] + w_uv_scale [H, head_dim/128, Dv/128]
      w_o  [D, wo_in] (+ w_o_scale);  w_r fp32 [E, D];  r_bias fp32 [E]
      w_gate, w_up [E+S, I, D]; w_down [E+S, D, I] (+ *_scale)
    """
    B, ps = spec.B, spec.page_size
    dev = torch.device(device)
    out: Dict[str, torch.Tensor] = {}
    lens = torch.tensor(spec.seq_lens, dtype=torch.int32)
    pages_per = [(l + ps - 1) // ps for l in spec.seq_lens]
    n_pages = sum(pages_per) + spec.extra_pages
    n_pages = max(n_pages, 1)
    mp = spec.max_pages
    pt = torch.zeros(B, mp, dtype=torch.int32)
    if spec.permute_pages:
        perm = torch.randperm(n_pages, generator=_gen("cpu", seed, instance, "page_perm"))
    else:
        perm = torch.arange(n_pages)
    at = 0
    for b, n in enumerate(pages_per):
        pt[b, :n] = perm[at:at + n].to(torch.int32)
        at += n
    out["seq_lens"] = lens.to(dev)
    out["page_table"] = pt.to(dev)
    out["n_pages"] = torch.tensor(n_pages)
    act_dt = torch.bfloat16 if spec.fp8 else torch.float32

    rows = B * spec.R
    out["x"] = _randn((rows, spec.D), dev, seed, instance, "x").to(act_dt)
    out["q"] = _randn((rows, spec.H, spec.Dc), dev, seed, instance, "q").to(act_dt)
    out["q_idx"] = _int8_uniform((rows, spec.HI, spec.DI), dev, seed, instance, "q_idx", spec.key_values)
    out["k_pool"] = _int8_uniform((n_pages, ps, spec.DI), dev, seed, instance, "k_pool", spec.key_values)
    if spec.pool > 1:
        out["pool_keys"] = _int8_uniform((n_pages, ps // spec.pool, spec.DI), dev, seed, instance, "pool_keys",
                                         spec.key_values)
    lat = _randn((n_pages, ps, spec.Dc), dev, seed, instance, "kv")
    if spec.fp8:
        codes, sc = quant_fp8_blocks(lat.reshape(n_pages * ps, 1, spec.Dc), 1, 128)
        out["kv"] = codes.reshape(n_pages, ps, spec.Dc)
        out["kv_scale"] = sc.reshape(n_pages, ps, spec.n_kv_blocks)
    else:
        out["kv"] = lat
    del lat
    if not weights:
        return out

    def wmat(name, shape, std):
        w = _randn(shape, dev, seed, instance, name, std)
        if not spec.fp8:
            return w, None
        return quant_fp8_blocks(w, 128, 128)

    if spec.head_dim:
        out["w_uv"], out["w_uv_scale"] = wmat("w_uv", (spec.H, spec.head_dim, spec.Dv), 0.02)
    w, s = wmat("w_o", (spec.D, spec.wo_in), 0.02)
    out["w_o"] = w
    if s is not None:
        out["w_o_scale"] = s
    rstd = spec.router_std if spec.router_std is not None else 1.0 / math.sqrt(spec.D)
    wr = _randn((spec.E, spec.D), dev, seed, instance, "w_r", rstd)
    if spec.dup_router_rows and spec.E >= 2:
        wr[1] = wr[0]
    out["w_r"] = wr
    bias = torch.zeros(spec.E, dtype=torch.float32)
    if spec.zipf_s > 0:
        rank = torch.randperm(spec.E, generator=_gen("cpu", seed, instance, "zipf_rank")) + 1
        p = rank.double() ** (-spec.zipf_s)
        p = p / p.sum()
        bias = torch.log(p).float()
    out["r_bias"] = bias.to(dev)

    NE = spec.E + spec.n_shared
    f8 = spec.fp8
    wg = torch.empty((NE, spec.I, spec.D), dtype=torch.uint8 if f8 else torch.float32, device=dev)
    wu = torch.empty_like(wg)
    wd = torch.empty((NE, spec.D, spec.I), dtype=wg.dtype, device=dev)
    if f8:
        sg = torch.empty((NE, (spec.I + 127) // 128, (spec.D + 127) // 128), dtype=torch.float32, device=dev)
        su = torch.empty_like(sg)
        sd = torch.empty((NE, (spec.D + 127) // 128, (spec.I + 127) // 128), dtype=torch.float32, device=dev)
    for e in range(NE):
        for name, dst, shape, sdst in (("w_gate", wg, (spec.I, spec.D), sg if f8 else None),
                                       ("w_up", wu, (spec.I, spec.D), su if f8 else None),
                                       ("w_down", wd, (spec.D, spec.I), sd if f8 else None)):
            w, s = wmat(f"{name}/{e}", shape, 0.02)
            dst[e] = w
            if f8:
                sdst[e] = s
    out["w_gate"], out["w_up"], out["w_down"] = wg, wu, wd
    if f8:
        out["w_gate_scale"], out["w_up_scale"], out["w_down_scale"] = sg, su, sd
    return out


def small_fp8_spec(name="small-fp8", B=None, seq_lens=(3000, 700, 0), D=1024, H=16, Dc=576, Dv=512,
                   head_dim=128, HI=16, DI=128, topk=512, E=16, ke=4, n_shared=1, I=512, **kw) -> LayerSpec:
    """A reduced FP8 layer with the big configurations' structure (several tiles, ragged tail,
    a padding row) that the oracle finishes in seconds."""
    if B is None:
        B = len(seq_lens)
    assert B == len(seq_lens), "one length per row"
    return LayerSpec(name, B=B, D=D, H=H, Dc=Dc, Dv=Dv, head_dim=head_dim, HI=HI, DI=DI, topk=topk,
                     E=E, ke=ke, n_shared=n_shared, I=I, seq_lens=tuple(seq_lens), fp8=True, **kw)


def spec_replace(spec: LayerSpec, **kw) -> LayerSpec:
    return dataclasses.replace(spec, **kw)


def to_numpy(t: torch.Tensor):
    """Host numpy view of a generated tensor (bf16 as uint16 bit patterns)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()


def make_append(seed: int = 0, B: int = 9, Dc: int = 576, DI: int = 128, page_size: int = 64,
                max_pages: int = 4, bf16: bool = False, device="cpu") -> Dict[str, torch.Tensor]:
    """Inputs of the current-token append, on ``device``: B rows' new-token latents [B, Dc] and indexer keys
    [B, DI] (fp32, or bf16 when ``bf16``), a key scale, the cache geometry, and pools pre-filled with random
    bytes so that bytes the append must leave alone can be checked.

    Row 3 is padding (length 0).  Rows 5 and 7 address the same physical slot.  Row 4's first two latent
    blocks contain the value 448 (so that their block scale is exactly 1) and otherwise midpoints between
    neighbouring e4m3 values (normal and subnormal), i.e. exact rounding ties; row 2 has an all-zero block.
    The keys include exact halves of the key scale (ties) and values far outside the int8 range."""
    assert B >= 8 and Dc >= 256
    n_pages = B * max_pages + 3
    g = _gen("cpu", seed, 0, "append-geom")
    perm = torch.randperm(n_pages, generator=g)[: B * max_pages].to(torch.int32)
    page_table = perm.reshape(B, max_pages).clone()
    cap = max_pages * page_size
    lens = torch.randint(1, cap + 1, (B,), generator=g, dtype=torch.int32)
    lens[0], lens[1], lens[2], lens[3] = 1, page_size, page_size + 1, 0
    lens[5] = lens[7] = cap - page_size + 7
    page_table[7, max_pages - 1] = page_table[5, max_pages - 1]      # same physical slot as row 5
    lat = _randn((B, Dc), "cpu", seed, 0, "append-latent", std=3.0)
    lat[2, 128:256] = 0.0
    lat[6, :128] *= 1e-3
    grid = torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32)
    mids = (grid[:-1] + grid[1:]) / 2                                   # 126 exact ties
    signs = torch.where(torch.arange(126) % 2 == 0, 1.0, -1.0)
    lat[4, :128] = torch.cat([torch.tensor([448.0]), mids * signs, torch.zeros(1)])
    lat[4, 128:256] = torch.cat([torch.tensor([-448.0]), (mids[:16] * signs[:16]).repeat(8)[:127]])
    gk = _gen("cpu", seed, 0, "append-key")
    key = (torch.rand((B, DI), generator=gk) * 400.0 - 200.0)
    key_scale = 0.5
    n_tie = min(DI, 16)
    key[:, :n_tie] = (torch.arange(n_tie, dtype=torch.float32) - 8.0 + 0.5) * key_scale
    key[:, n_tie:n_tie + 2] = torch.tensor([1000.0, -1000.0])[: max(0, min(2, DI - n_tie))]
    dt = torch.bfloat16 if bf16 else torch.float32
    nb = (Dc + 127) // 128
    gp = _gen("cpu", seed, 0, "append-pools")
    return {
        "seq_lens": lens.to(device), "page_table": page_table.to(device),
        "latent": lat.to(dt).to(device), "key": key.to(dt).to(device), "key_scale": torch.tensor(key_scale),
        "kv_pool": torch.randint(0, 256, (n_pages, page_size, Dc), generator=gp, dtype=torch.uint8).to(device),
        "kv_scale": torch.rand((n_pages, page_size, nb), generator=gp).to(device),
        "k_pool": torch.randint(-128, 128, (n_pages, page_size, DI), generator=gp, dtype=torch.int8).to(device),
    }


def ep_slice(t: Dict[str, torch.Tensor], spec: LayerSpec, g: int, n: int, shared: bool = True) -> Dict[str, torch.Tensor]:
    """Expert weights held by GPU g of n in an expert-parallel layout: routed experts [g E/n, (g+1) E/n), then
    (shared=True) the shared experts, with their block scales.  Pure copying: no arithmetic."""
    E = spec.E
    assert E % n == 0, "whole experts per GPU"
    e0, e1 = g * E // n, (g + 1) * E // n
    names = ["w_gate", "w_up", "w_down"] + (["w_gate_scale", "w_up_scale", "w_down_scale"] if spec.fp8 else [])
    out = {}
    for k in names:
        parts = [t[k][e0:e1]] + ([t[k][E:E + spec.n_shared]] if shared and spec.n_shared else [])
        out[k] = torch.cat(parts).contiguous()
    return out


def tp_slice(t: Dict[str, torch.Tensor], spec: LayerSpec, s: int, n: int) -> Dict[str, torch.Tensor]:
    """Expert weights of tensor-parallel slice s of n: intermediate rows [s I/n, (s+1) I/n) of every expert's gate
    and up matrices and the same columns of its down matrix, with their block scales (I/n must be a multiple of
    128 so that slices hold whole scale blocks).  Pure slicing: no arithmetic.  The slices' FFN contributions add
    up to the whole FFN because SwiGLU acts on each intermediate row separately."""
    I = spec.I
    assert I % n == 0 and (I // n) % 128 == 0, "slices of whole 128-row scale blocks"
    r0, r1 = s * I // n, (s + 1) * I // n
    b0, b1 = r0 // 128, r1 // 128
    out = {
        "w_gate": t["w_gate"][:, r0:r1].contiguous(), "w_up": t["w_up"][:, r0:r1].contiguous(),
        "w_down": t["w_down"][:, :, r0:r1].contiguous(),
    }
    if spec.fp8:
        out["w_gate_scale"] = t["w_gate_scale"][:, b0:b1].contiguous()
        out["w_up_scale"] = t["w_up_scale"][:, b0:b1].contiguous()
        out["w_down_scale"] = t["w_down_scale"][:, :, b0:b1].contiguous()
    return out
