"""GPU parity: the HIP library (through the C ABI) against the CPU oracle on seeded synthetic layers.

Bit-exact: kept positions (and their scores), expert choices (up to oracle logits within 1e-6).
Floating point: max |err| <= 2e-2 * max |oracle| for o, h - x, y - h and y, each against its own maximum."""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_moe_amd as dl
import synth
from parity import FP_TOL, assert_close, check_rows, expert_mismatch, host, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _layer(spec, seed=0, weights=True):
    say(f"[gen] {spec.name} B={spec.B} lens={spec.seq_lens[:4]} seed={seed}")
    return synth.make_layer(spec, seed=seed, device=DEV, weights=weights)


def untile_keys(a: np.ndarray) -> np.ndarray:
    """Row-major view of an index-key cache [..., items, dim] held in DL_LAYOUT_TILES: per 16 consecutive items,
    byte kc*1024 + g*256 + p*16 + j is key byte kc*64 + g*16 + j of item p (the layout dl.h documents)."""
    dim = a.shape[-1]
    g = a.reshape(-1, dim // 64, 4, 16, 16)          # [group, kc, g, item, j]
    return g.transpose(0, 3, 1, 2, 4).reshape(a.shape)


def _topk(spec, t, tiled=False):
    sel = torch.empty(spec.B, spec.topk, dtype=torch.int32, device=DEV)
    ss = torch.empty_like(sel)
    keys = dl.tile_index_keys(t["k_pool"]) if tiled else t["k_pool"]
    pg = dl.pages(t["seq_lens"], t["page_table"], spec.page_size, dl.DL_LAYOUT_TILES if tiled else dl.DL_LAYOUT_ROWS)
    say(f"[gpu] indexer_topk {spec.name} HI={spec.HI} DI={spec.DI} k={spec.topk} tiled={tiled}")
    dl.indexer_topk(pg, t["q_idx"], keys, spec.topk, sel, ss)
    torch.cuda.synchronize()
    if tiled:
        assert np.array_equal(untile_keys(host(keys)), host(t["k_pool"]))
    return host(sel), host(ss)


def _check_topk(spec, t, rows=None, tiled=False):
    sel, ss = _topk(spec, t, tiled)
    orc = oracle.LayerOracle(spec, t)
    for b in (rows if rows is not None else range(spec.B)):
        r = orc.row(b, stages=("sel",))
        assert np.array_equal(sel[b], r["sel"]), f"{spec.name} row {b}: first diff at " \
            f"{np.nonzero(sel[b] != r['sel'])[0][:5]}"
        n = int((r["sel"] >= 0).sum())
        assert np.array_equal(ss[b][:n], r["scores"][r["sel"][:n]])
        assert np.all(ss[b][n:] == 0)


SMALL = {
    "tiny-fp32": synth.config(1),
    "fp8-ragged": synth.small_fp8_spec(),
    "fp8-ternary-ties": synth.small_fp8_spec(name="ternary", key_values="ternary", seq_lens=(5000, 2049, 2048, 17)),
    "fp8-permuted": synth.small_fp8_spec(name="perm", permute_pages=True, extra_pages=5, seq_lens=(4100, 64, 1)),
    "page16": synth.small_fp8_spec(name="page16", page_size=16, seq_lens=(3001, 512)),
    "heads4-dim64": synth.small_fp8_spec(name="hi4di64", HI=4, DI=64, seq_lens=(2500, 1300)),
    "heads20-dim48": synth.small_fp8_spec(name="hi20di48", HI=20, DI=48, seq_lens=(2600,), B=1),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_indexer_topk_small(name):
    spec = SMALL[name]
    t = _layer(spec, seed=1, weights=False)
    _check_topk(spec, t)


@pytest.mark.parametrize("name", [n for n, sp in SMALL.items() if sp.fp8 and sp.DI % 64 == 0 and sp.page_size % 16 == 0])
def test_indexer_topk_tiled_keys(name):
    # the same selections from the key cache in DL_LAYOUT_TILES (and the tiling itself against the documented
    # byte order)
    spec = SMALL[name]
    t = _layer(spec, seed=1, weights=False)
    _check_topk(spec, t, tiled=True)


def test_indexer_topk_reused_workspace():
    # the scoring kernel clears the histograms itself: a workspace of garbage bytes (every flag word all ones), the
    # same workspace again after a selection over other queries (its flags then hold the earlier launch's stamp),
    # and a third call, all give the oracle's selection bit for bit
    spec = synth.small_fp8_spec(name="reuse", seq_lens=(5000, 2049, 17, 3000))
    t = _layer(spec, seed=3, weights=False)
    t2 = _layer(spec, seed=4, weights=False)
    pg = dl.pages(t["seq_lens"], t["page_table"], spec.page_size)
    ws = dl.workspace(dl.load().dl_indexer_topk_rows_workspace(dl.C.byref(pg), 1), DEV)
    ws.fill_(0xFF)
    orc = oracle.LayerOracle(spec, t)
    want = [orc.row(b, stages=("sel",))["sel"] for b in range(spec.B)]
    for call, q in enumerate((t["q_idx"], t2["q_idx"], t["q_idx"], t["q_idx"])):
        sel = torch.empty(spec.B, spec.topk, dtype=torch.int32, device=DEV)
        say(f"[gpu] indexer_topk on a reused workspace, call {call}")
        dl.indexer_topk(pg, q, t["k_pool"], spec.topk, sel, ws=ws)
        torch.cuda.synchronize()
        if q is t["q_idx"]:
            got = host(sel)
            for b in range(spec.B):
                assert np.array_equal(got[b], want[b]), f"call {call} row {b}"


def test_indexer_topk_k_above_length_and_empty_rows():
    spec = synth.small_fp8_spec(name="short", seq_lens=(100, 0, 511, 512, 513), B=5, topk=512)
    t = _layer(spec, seed=2, weights=False)
    _check_topk(spec, t)


def test_indexer_topk_all_equal_scores():
    # every item is a candidate: 6,000 and 3,000 are selected among in LDS, 20,000 from the workspace
    spec = synth.small_fp8_spec(name="flat", seq_lens=(6000, 3000, 20000), B=3)
    t = _layer(spec, seed=3, weights=False)
    t["q_idx"].zero_()  # every score is 0: the lowest positions win
    sel, _ = _topk(spec, t)
    for b in range(spec.B):
        assert np.array_equal(sel[b], np.arange(spec.topk))


def _bin1(s: int) -> int:
    # the scoring kernel's log-linear histogram bin: exact below 256, then 128 bins per binade
    if s < 256:
        return s
    n = s.bit_length() - 1
    return 256 + (n - 8) * 128 + ((s >> (n - 7)) & 127)


def test_indexer_topk_many_candidates_in_the_threshold_bin():
    # Scores packed densely around 14,000 (head 0 only: 127 k0 + k1 with k0 in [120, 127]), so the histogram bin
    # holding the k-th score contains many items with distinct scores: the 50,000-item row selects among a few
    # thousand of them in LDS, the 600,000-item row among more than 4,096, read back from the workspace.
    spec = synth.small_fp8_spec(name="dense-bin", seq_lens=(50000, 600000), B=2, topk=512)
    t = _layer(spec, seed=12, weights=False)
    g = torch.Generator(device="cpu").manual_seed(12)
    kp = torch.zeros_like(t["k_pool"], device="cpu")
    kp[..., 0] = torch.randint(120, 128, kp.shape[:-1], generator=g, dtype=torch.int8)
    kp[..., 1] = torch.randint(-128, 128, kp.shape[:-1], generator=g, dtype=torch.int8)
    t["k_pool"] = kp.to(DEV)
    q = torch.zeros_like(t["q_idx"], device="cpu")
    q[:, 0, 0], q[:, 0, 1] = 127, 1
    t["q_idx"] = q.to(DEV)
    orc = oracle.LayerOracle(spec, t)
    cands = []
    for b in range(spec.B):
        sc = orc.row(b, stages=("sel",))["scores"]
        bins = np.array([_bin1(int(x)) for x in sc])
        cands.append(int((bins == np.sort(bins)[::-1][spec.topk - 1]).sum()))
    say(f"[cpu] candidates in the threshold bin: {cands}")
    assert 256 < cands[0] <= 4096 < cands[1]
    _check_topk(spec, t)


LAYERS = {
    # value and head widths of the attention merge + W_UV kernels other than the named workloads' 512 / 128, at two
    # rows (one workgroup per row and head) and at ten (one per head and block of rows, on the matrix cores)
    **{f"fp8-dv{dv}-hd{hd}-b{b}": synth.small_fp8_spec(name=f"dv{dv}hd{hd}b{b}", Dc=dc, Dv=dv, head_dim=hd,
                                                        seq_lens=tuple(lens[i % 2] + 37 * i for i in range(b)), B=b)
       for dc, dv, hd, lens in ((256, 128, 128, (1900, 300)), (256, 256, 128, (1200, 2100)),
                                (128, 128, 256, (2500, 64)), (512, 256, 256, (700, 3000)))
       for b in (2, 10)},
    "tiny-fp32": synth.config(1),
    "fp8-ragged-pad": synth.small_fp8_spec(),
    "fp8-zipf-perm": synth.small_fp8_spec(name="zipf", zipf_s=1.1, permute_pages=True, B=4,
                                          seq_lens=(2500, 4096, 1000, 3333)),
    "fp8-dup-router": synth.small_fp8_spec(name="dup", dup_router_rows=True, seq_lens=(1500, 2600), B=2),
    "fp8-ke1-noshared": synth.small_fp8_spec(name="ke1", ke=1, n_shared=0, seq_lens=(900, 3000), B=2),
    "fp8-b20": synth.small_fp8_spec(name="b20", B=20, seq_lens=tuple(600 + 97 * i for i in range(20)), topk=256),
}


@pytest.mark.parametrize("name", list(LAYERS))
def test_layer_step_small(name):
    spec = LAYERS[name]
    t = _layer(spec, seed=4)
    step = dl.LayerStep(spec, t, debug=True)
    say(f"[gpu] layer_step {spec.name}")
    y = step()
    torch.cuda.synchronize()
    w = check_rows(spec, t, step.dbg, y, list(range(spec.B)))
    say(f"{name}: {w}")


@pytest.mark.parametrize("lens", [(3000, 700, 0), tuple(300 + 211 * i for i in range(10))])
def test_fused_equals_unfused_and_replays(lens):
    # the fused step reads tiled weights, the separate calls row-major ones; 3 and 10 rows take the two forms of
    # the attention merge + W_UV kernel
    spec = synth.small_fp8_spec(name="fused", B=len(lens), seq_lens=lens)
    t = _layer(spec, seed=5)
    step = dl.LayerStep(spec, t, debug=True)
    say("[gpu] fused step + 4 separate calls")
    y = step().clone()
    ref = {k: v.clone() for k, v in step.dbg.items()}
    B = spec.B
    pg = dl.pages(t["seq_lens"], t["page_table"], spec.page_size)
    sel = torch.empty(B, spec.topk, dtype=torch.int32, device=DEV)
    dl.indexer_topk(pg, t["q_idx"], t["k_pool"], spec.topk, sel)
    h = torch.empty(B, spec.D, dtype=torch.float32, device=DEV)
    dl.sparse_attn_decode(pg, t["q"], t["kv"], t.get("kv_scale"), spec.H, spec.Dc, spec.Dv, spec.scale, sel,
                          spec.topk, h, w_uv=dl.mat(t["w_uv"], t["w_uv_scale"]), w_o=dl.mat(t["w_o"], t["w_o_scale"]),
                          residual=t["x"])
    ex = torch.empty(B, spec.ke, dtype=torch.int32, device=DEV)
    g = torch.empty(B, spec.ke, dtype=torch.float32, device=DEV)
    dl.moe_route(h, t["w_r"], t["r_bias"], spec.ke, ex, g)
    y2 = torch.empty_like(y)
    dl.moe_ffn(h, ex, g, dl.mat(t["w_gate"], t["w_gate_scale"]), dl.mat(t["w_up"], t["w_up_scale"]),
               dl.mat(t["w_down"], t["w_down_scale"]), spec.E, spec.n_shared, y2, residual=h)
    torch.cuda.synchronize()
    assert torch.equal(sel, ref["sel"]) and torch.equal(h, ref["h"])
    assert torch.equal(ex, ref["experts"]) and torch.equal(g, ref["gates"])
    assert torch.equal(y2, y)
    say("[gpu] 50 replays")
    for i in range(50):
        yi = step()
        if i % 10 == 9:
            torch.cuda.synchronize()
            assert torch.equal(yi, y)
            for k, v in step.dbg.items():
                assert torch.equal(v, ref[k]), k


def test_attention_only_matches_oracle():
    spec = synth.small_fp8_spec(name="attn", B=2, seq_lens=(2600, 333))
    t = _layer(spec, seed=6, weights=False)
    sel, _ = _topk(spec, t)
    pg = dl.pages(t["seq_lens"], t["page_table"], spec.page_size)
    o = torch.empty(spec.B, spec.H, spec.Dv, dtype=torch.float32, device=DEV)
    dl.sparse_attn_decode(pg, t["q"], t["kv"], t["kv_scale"], spec.H, spec.Dc, spec.Dv, spec.scale,
                          torch.from_numpy(sel).to(DEV), spec.topk, o)
    torch.cuda.synchronize()
    orc = oracle.LayerOracle(spec, t)
    for b in range(spec.B):
        ref = oracle.attention(orc.a("q")[b], orc.a("kv"), orc.a("kv_scale"), orc.a("page_table")[b], sel[b],
                               spec.scale, spec.Dv)
        assert_close(f"o row {b}", host(o)[b], ref)


@pytest.mark.parametrize("B,E,ke,D,dup", [(40, 256, 8, 6144, False), (70, 300, 6, 1000, False),
                                          (9, 1024, 32, 2048, True), (3, 64, 1, 512, True)])
def test_route_standalone(B, E, ke, D, dup):
    """dl_moe_route against the oracle: several token blocks, more than 256 experts, a ragged last hidden
    chunk, and (dup) two pairs of identical router rows forced to the top, an exact tie the lower id wins."""
    g = torch.Generator().manual_seed(11 + B)
    h = torch.randn(B, D, generator=g)
    w_r = torch.randn(E, D, generator=g) / math.sqrt(D)
    bias = torch.randn(E, generator=g) * 0.1
    if dup:
        w_r[1], w_r[5] = w_r[0], w_r[4]
        bias[0] = bias[1] = 10.0
        bias[4] = bias[5] = 9.0
    ex = torch.empty(B, ke, dtype=torch.int32, device=DEV)
    gt = torch.empty(B, ke, dtype=torch.float32, device=DEV)
    lg = torch.empty(B, E, dtype=torch.float32, device=DEV)
    say(f"[gpu] moe_route B={B} E={E} ke={ke} D={D} dup={dup}")
    dl.moe_route(h.to(DEV), w_r.to(DEV), bias.to(DEV), ke, ex, gt, logits=lg)
    torch.cuda.synchronize()
    ex, gt, lg = host(ex), host(gt), host(lg)
    near = 0
    for b in range(B):
        ol, oe, og = oracle.router(h[b].double().numpy(), w_r.numpy(), bias.numpy(), ke)
        m = expert_mismatch(ex[b], oe, ol)
        assert m in (None, "near-tie"), f"row {b}: {m}"
        near += m is not None
        if m is None:
            assert np.allclose(gt[b], og, rtol=0, atol=1e-6), f"row {b} gates"
        assert np.allclose(lg[b], ol, rtol=0, atol=1e-6 * max(1.0, float(np.abs(ol).max()))), f"row {b} logits"
        if dup:  # of two exactly tied experts the lower id is picked first, and right before the other
            lst = [int(v) for v in ex[b]]
            for lo, hi in ((0, 1), (4, 5)):
                if hi in lst:
                    assert lo in lst and lst.index(hi) == lst.index(lo) + 1, f"row {b}: {lst}"
    say(f"near ties: {near}")


# ------------------------------------------------------------------ the five named workloads
@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_config(cfg, seed):
    """The fused step at full size, in the launch configuration the benchmark times (tiled weights and keys),
    against the oracle on every row: kept positions bit-exact (and, from the indexer entry point on the same
    keys, their scores), experts bit-exact up to oracle logits within 1e-6, o, h - x, y - h, y and the gates
    within the floating-point bar; router logits compared to the oracle's fp64 ones."""
    spec = synth.config(cfg)
    t = _layer(spec, seed=seed)
    step = dl.LayerStep(spec, t, debug=True)
    say(f"[gpu] layer_step {spec.name}")
    y = step()
    torch.cuda.synchronize()
    # the scores of the kept positions, from the indexer entry point on the tiled keys the step read
    sel2 = torch.empty(spec.B, spec.topk, dtype=torch.int32, device=DEV)
    ss = torch.empty_like(sel2)
    dl.indexer_topk(step.pg, t["q_idx"], step.keys, spec.topk, sel2, ss)
    torch.cuda.synchronize()
    assert torch.equal(sel2, step.dbg["sel"])
    rows = list(range(spec.B))
    say(f"[cpu] oracle rows {rows}")
    w = check_rows(spec, t, step.dbg, y, rows)
    orc = oracle.LayerOracle(spec, t)
    ss = host(ss)
    for b in rows:
        r = orc.row(b, stages=("sel",))
        n = int((r["sel"] >= 0).sum())
        assert np.array_equal(ss[b][:n], r["scores"][r["sel"][:n]]), f"row {b}: kept scores differ"
        assert np.all(ss[b][n:] == 0)
    say(f"cfg{cfg} seed {seed}: {w}")
    assert w["logit_abs"] < 1e-4
    del step, t
    torch.cuda.empty_cache()


def test_tiny_config_full_oracle():
    spec = synth.config(1)
    t = _layer(spec, seed=0)
    step = dl.LayerStep(spec, t, debug=True)
    y = step()
    torch.cuda.synchronize()
    w = check_rows(spec, t, step.dbg, y, [0])
    assert w["y"] <= FP_TOL


def test_pack_weights_layout():
    """dl_pack_weights follows the tile layout stated in dl.h (checked against a numpy re-tiling)."""
    g = torch.Generator(device=DEV).manual_seed(7)
    w = torch.randint(0, 126, (3, 64, 384), generator=g, device=DEV, dtype=torch.uint8)
    sc = torch.ones(3, 1, 3, device=DEV)
    tiled = dl.pack_weights(w, sc)
    torch.cuda.synchronize()
    src = w.cpu().numpy()
    got = tiled.cpu().numpy().reshape(-1)
    count, rows, cols = src.shape
    ref = np.empty_like(got)
    o = 0
    for m in range(count):
        for t in range(rows // 16):
            for kb in range(cols // 128):
                for h in range(2):
                    for l in range(64):
                        r, c = t * 16 + l % 16, kb * 128 + h * 64 + (l // 16) * 16
                        ref[o:o + 16] = src[m, r, c:c + 16]
                        o += 16
    assert np.array_equal(got, ref)


def test_rows_and_tiles_layouts_agree():
    spec = synth.small_fp8_spec(name="layouts", B=2, seq_lens=(1700, 900))
    t = _layer(spec, seed=8)
    y_rows = dl.LayerStep(spec, t, debug=True, tiles=False)().clone()
    y_tiles = dl.LayerStep(spec, t, debug=True, tiles=True)()
    torch.cuda.synchronize()
    assert torch.equal(y_rows, y_tiles)


# ------------------------------------------------------------- current-token append
@pytest.mark.parametrize("bf16,tiled", [(False, False), (True, False), (True, True)])
def test_kv_append_bit_exact(bf16, tiled):
    t = synth.make_append(seed=3, bf16=bf16, device=DEV)
    h = {k: synth.to_numpy(v) for k, v in t.items()}  # the caches as generated, row-major
    if tiled:
        t["k_pool"] = dl.tile_index_keys(t["k_pool"])
    lens, pt, ps = h["seq_lens"], h["page_table"], 64
    kv, kvs, kp = h["kv_pool"].copy(), h["kv_scale"].copy(), h["k_pool"].copy()
    Dc, DI = kv.shape[2], kp.shape[2]
    written = set()
    for b in range(lens.shape[0]):                    # expected: the oracle's row, at the lowest row's slot
        if lens[b] <= 0:
            continue
        p = int(lens[b]) - 1
        page, slot = int(pt[b, p // ps]), p % ps
        if (page, slot) in written:
            continue
        written.add((page, slot))
        codes, scales, k8 = oracle.kv_append_row(h["latent"][b], h["key"][b], float(h["key_scale"]))
        kv[page, slot], kvs[page, slot], kp[page, slot] = codes, scales, k8
    assert len(written) == lens.shape[0] - 2          # one padding row, one row sharing a slot
    say(f"[gpu] kv_append bf16={bf16} tiled={tiled} B={lens.shape[0]} Dc={Dc} DI={DI}")
    pg = dl.pages(t["seq_lens"], t["page_table"], ps, dl.DL_LAYOUT_TILES if tiled else dl.DL_LAYOUT_ROWS)
    dl.kv_append(pg, t["latent"], t["key"], float(h["key_scale"]), t["kv_pool"], t["kv_scale"], t["k_pool"])
    torch.cuda.synchronize()
    got_kv, got_s, got_k = host(t["kv_pool"]), host(t["kv_scale"]), host(t["k_pool"])
    if tiled:
        got_k = untile_keys(got_k)
    bad = np.argwhere(got_kv != kv)
    assert bad.size == 0, f"{len(bad)} latent bytes differ, first {bad[:3].tolist()}: {got_kv[tuple(bad[0])]} vs {kv[tuple(bad[0])]}"
    assert np.array_equal(got_s.view(np.uint32), kvs.view(np.uint32))
    assert np.array_equal(got_k, kp)


# ------------------------------------------------------------- multi-row decode (R query rows per sequence)
@pytest.mark.parametrize("R", [2, 3, 4])
def test_indexer_rows_bit_exact(R):
    # ragged: a long sequence spanning many score blocks, one shorter than R (its first rows see nothing), a
    # padding sequence, one with an exact multiple of the page size
    spec = synth.spec_replace(synth.small_fp8_spec(name=f"rows{R}", seq_lens=(5000, 2, 0, 1024, 777), topk=512), R=R)
    t = _layer(spec, seed=20 + R, weights=False)
    rows = spec.B * R
    sel = torch.empty(rows, spec.topk, dtype=torch.int32, device=DEV)
    ss = torch.empty_like(sel)
    pg = dl.pages(t["seq_lens"], t["page_table"], spec.page_size)
    say(f"[gpu] indexer_topk rows R={R} B={spec.B} lens={spec.seq_lens}")
    dl.indexer_topk(pg, t["q_idx"], t["k_pool"], spec.topk, sel, ss, rows_per_seq=R)
    torch.cuda.synchronize()
    sel, ss = host(sel), host(ss)
    orc = oracle.LayerOracle(spec, t)
    for i in range(rows):
        r = orc.row(i, stages=("sel",))
        assert np.array_equal(sel[i], r["sel"]), f"row {i}: first diff at {np.nonzero(sel[i] != r['sel'])[0][:5]}"
        n = int((r["sel"] >= 0).sum())
        assert np.array_equal(ss[i][:n], r["scores"][r["sel"][:n]])
        assert np.all(ss[i][n:] == 0)


@pytest.mark.parametrize("R", [2, 3, 4])
def test_layer_step_rows(R):
    spec = synth.spec_replace(synth.small_fp8_spec(name=f"step-rows{R}", seq_lens=(3000, 2, 700), B=3), R=R)
    t = _layer(spec, seed=30 + R)
    step = dl.LayerStep(spec, t, debug=True)
    say(f"[gpu] layer_step rows R={R} lens={spec.seq_lens}")
    y = step()
    torch.cuda.synchronize()
    w = check_rows(spec, t, step.dbg, y, list(range(spec.B * R)))
    say(f"rows R={R}: {w}")


def _ffn_mats(w, tiled):
    """dl_mat views of an FFN's gate, up and down stacks: row-major (the three-launch path), or re-tiled
    (DL_LAYOUT_TILES: the fused FFN kernel); returns the views and the tensors they point into."""
    keep, mats = [], []
    for k in ("w_gate", "w_up", "w_down"):
        wk, sk = w[k], w[k + "_scale"]
        if tiled:
            wk = dl.pack_weights(wk, sk)
        keep.append(wk)
        mats.append(dl.mat(wk, sk, dl.DL_LAYOUT_TILES if tiled else dl.DL_LAYOUT_ROWS))
    return mats, keep


def _check_ffn_path(tiled):
    # FP8 weights in tiles run the fused FFN kernel, row-major ones the three launches
    assert dl.profile_ffn_fused() == (1 if tiled else 0)


# ------------------------------------------------------------- one GPU's tensor-parallel share of the FFN
@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("n", [2, 4])
def test_ffn_tensor_parallel_slices_sum_to_whole(n, tiled):
    # Each of n GPUs would hold I/n intermediate rows of every expert; here the n shares run one after the other
    # on one GPU.  Their outputs (the residual added by share 0 only) must add up to the oracle's whole FFN.
    spec = synth.small_fp8_spec(name=f"tp{n}", B=4, seq_lens=(900, 600, 300, 1), I=512)
    t = _layer(spec, seed=40 + n)
    B = spec.B
    h = (torch.randn(B, spec.D, generator=torch.Generator().manual_seed(7)) * 0.5).to(DEV)
    ex = torch.empty(B, spec.ke, dtype=torch.int32, device=DEV)
    g = torch.empty(B, spec.ke, dtype=torch.float32, device=DEV)
    dl.moe_route(h, t["w_r"], t["r_bias"], spec.ke, ex, g)
    total = torch.zeros(B, spec.D, dtype=torch.float32, device=DEV)
    for s_ in range(n):
        w = synth.tp_slice(t, spec, s_, n)
        part = torch.empty(B, spec.D, dtype=torch.float32, device=DEV)
        say(f"[gpu] moe_ffn tensor-parallel share {s_}/{n} inter={spec.I // n} tiled={tiled}")
        (wg, wu, wd), keep = _ffn_mats(w, tiled)
        dl.moe_ffn(h, ex, g, wg, wu, wd, spec.E, spec.n_shared, part, residual=h if s_ == 0 else None)
        _check_ffn_path(tiled)
        total += part
    torch.cuda.synchronize()
    orc = oracle.LayerOracle(spec, t)
    hh = host(h).astype(np.float64)
    exh, gh = host(ex), host(g)
    got = host(total).astype(np.float64)
    for b in range(B):
        y64 = oracle.ffn(hh[b], exh[b], gh[b].astype(np.float64), orc.expert, spec.E, spec.n_shared)
        assert_close(f"tp{n} row {b} y-h", got[b] - hh[b], y64 - hh[b])


# ------------------------------------------------------------- pool-granular selection
@pytest.mark.parametrize("pool,offset,tiled", [(2, 0, False), (4, 0, False), (16, 0, False), (4, 1, False),
                                               (2, 0, True), (4, 0, True)])
def test_indexer_pooled_bit_exact(pool, offset, tiled):
    # offset 1: the output starts 4 bytes past a 16-byte boundary, which takes the one-position-at-a-time stores
    top_pools = 512 // pool
    spec = synth.spec_replace(synth.small_fp8_spec(name=f"pool{pool}", seq_lens=(9001, 3, 0, 4096, 777), topk=512),
                              pool=pool)
    t = _layer(spec, seed=50 + pool, weights=False)
    B = spec.B
    buf = torch.empty(B * top_pools * pool + offset, dtype=torch.int32, device=DEV)
    sel = buf[offset:].view(B, top_pools * pool)
    ps = torch.empty(B, top_pools, dtype=torch.int32, device=DEV)
    pg = dl.pages(t["seq_lens"], t["page_table"], spec.page_size, dl.DL_LAYOUT_TILES if tiled else dl.DL_LAYOUT_ROWS)
    keys = dl.tile_index_keys(t["pool_keys"]) if tiled else t["pool_keys"]
    say(f"[gpu] indexer_topk_pooled pool={pool} top_pools={top_pools} offset={offset} tiled={tiled} lens={spec.seq_lens}")
    dl.indexer_topk_pooled(pg, pool, t["q_idx"], keys, top_pools, sel, ps)
    torch.cuda.synchronize()
    sel, ps = host(sel), host(ps)
    qh, pth, pkh = host(t["q_idx"]), host(t["page_table"]), host(t["pool_keys"])
    for b in range(B):
        want, sc, pools = oracle.pooled_topk(qh[b], pkh, pth[b], spec.seq_lens[b], pool, top_pools)
        assert np.array_equal(sel[b], want), f"row {b}: first diff at {np.nonzero(sel[b] != want)[0][:5]}"
        n = int((pools >= 0).sum())
        assert np.array_equal(ps[b][:n], sc[pools[:n]]) and np.all(ps[b][n:] == 0)


@pytest.mark.parametrize("pool", [2, 4, 16])
def test_layer_step_pooled(pool):
    # The whole step with pool-granular selection: positions come from whole pools, the rest as in dl_layer_step.
    spec = synth.spec_replace(synth.small_fp8_spec(name=f"step-pool{pool}", seq_lens=(3001, 5, 0, 700), B=4),
                              pool=pool)
    t = _layer(spec, seed=60 + pool)
    step = dl.LayerStep(spec, t, debug=True)
    say(f"[gpu] layer_step pooled pool={pool} lens={spec.seq_lens}")
    y = step()
    torch.cuda.synchronize()
    w = check_rows(spec, t, step.dbg, y, list(range(spec.B)))
    say(f"pooled pool={pool}: {w}")


@pytest.mark.parametrize("R,pool", [(2, 4), (4, 2), (3, 16)])
def test_indexer_rows_pooled_bit_exact(R, pool):
    # several rows per sequence, each selecting whole pools over its own visible length: a long sequence, one
    # shorter than R (its first rows see nothing), a padding sequence, lengths that are not multiples of the pool
    top_pools = 512 // pool
    spec = synth.spec_replace(synth.small_fp8_spec(name=f"rows{R}-pool{pool}", seq_lens=(9001, 2, 0, 4096, 777),
                                                   topk=512), R=R, pool=pool)
    t = _layer(spec, seed=80 + R * pool, weights=False)
    rows = spec.B * R
    sel = torch.empty(rows, top_pools * pool, dtype=torch.int32, device=DEV)
    ps = torch.empty(rows, top_pools, dtype=torch.int32, device=DEV)
    pg = dl.pages(t["seq_lens"], t["page_table"], spec.page_size)
    say(f"[gpu] indexer_topk rows+pools R={R} pool={pool} lens={spec.seq_lens}")
    dl.indexer_topk_pooled(pg, pool, t["q_idx"], t["pool_keys"], top_pools, sel, ps, rows_per_seq=R)
    torch.cuda.synchronize()
    sel, ps = host(sel), host(ps)
    orc = oracle.LayerOracle(spec, t)
    for i in range(rows):
        r = orc.row(i, stages=("sel",))
        assert np.array_equal(sel[i], r["sel"]), f"row {i}: first diff at {np.nonzero(sel[i] != r['sel'])[0][:5]}"
        n = int((r["pools"] >= 0).sum())
        assert np.array_equal(ps[i][:n], r["scores"][r["pools"][:n]]) and np.all(ps[i][n:] == 0)


@pytest.mark.parametrize("R,pool", [(2, 4), (4, 2)])
def test_layer_step_rows_pooled(R, pool):
    # the multi-token-prediction verification step reading the pool-key cache: every row against the oracle
    spec = synth.spec_replace(synth.small_fp8_spec(name=f"step-rows{R}-pool{pool}", seq_lens=(3001, 2, 700), B=3),
                              R=R, pool=pool)
    t = _layer(spec, seed=90 + R * pool)
    step = dl.LayerStep(spec, t, debug=True)
    say(f"[gpu] layer_step rows+pools R={R} pool={pool} lens={spec.seq_lens}")
    y = step()
    torch.cuda.synchronize()
    w = check_rows(spec, t, step.dbg, y, list(range(spec.B * R)))
    say(f"rows+pools R={R} pool={pool}: {w}")


# ------------------------------------------------------------- one GPU's expert-parallel share of the FFN
@pytest.mark.parametrize("n", [2, 4, 8])
@pytest.mark.parametrize("tiled", [False, True])
def test_ffn_expert_parallel_shares_sum_to_whole(n, tiled):
    # GPU g of n holds routed experts [g E/n, (g+1) E/n); each share applies only its picks (with n = 8 a token picks
    # more experts than a GPU holds).  The shares, run one after the other on one GPU, with the shared expert and
    # the residual on share 0, must add up to the oracle's whole FFN.
    spec = synth.small_fp8_spec(name=f"ep{n}", B=4, seq_lens=(900, 600, 300, 1), I=512)
    t = _layer(spec, seed=70 + n)
    B, per = spec.B, spec.E // n
    h = (torch.randn(B, spec.D, generator=torch.Generator().manual_seed(9)) * 0.5).to(DEV)
    ex = torch.empty(B, spec.ke, dtype=torch.int32, device=DEV)
    g = torch.empty(B, spec.ke, dtype=torch.float32, device=DEV)
    dl.moe_route(h, t["w_r"], t["r_bias"], spec.ke, ex, g)
    total = torch.zeros(B, spec.D, dtype=torch.float32, device=DEV)
    for s_ in range(n):
        w = synth.ep_slice(t, spec, s_, n, shared=s_ == 0)
        part = torch.empty(B, spec.D, dtype=torch.float32, device=DEV)
        ns = spec.n_shared if s_ == 0 else 0
        say(f"[gpu] moe_ffn_ep share {s_}/{n} experts [{s_ * per}, {(s_ + 1) * per}) shared={ns} tiled={tiled}")
        (wg, wu, wd), keep = _ffn_mats(w, tiled)
        dl.moe_ffn_ep(h, ex, g, s_ * per, wg, wu, wd, per, ns, part, residual=h if s_ == 0 else None)
        _check_ffn_path(tiled)
        total += part
    torch.cuda.synchronize()
    orc = oracle.LayerOracle(spec, t)
    hh = host(h).astype(np.float64)
    exh, gh = host(ex), host(g)
    got = host(total).astype(np.float64)
    for b in range(B):
        y64 = oracle.ffn(hh[b], exh[b], gh[b].astype(np.float64), orc.expert, spec.E, spec.n_shared)
        assert_close(f"ep{n} row {b} y-h", got[b] - hh[b], y64 - hh[b])


@pytest.mark.parametrize("tiled", [False, True])
def test_ffn_expert_parallel_share_without_picks(tiled):
    # a share holding none of the picked experts and no shared expert has no active slot at all: its output is
    # exactly the residual it is given (zero without one), whatever the other shares compute
    spec = synth.small_fp8_spec(name="ep-empty", B=4, seq_lens=(900, 600, 300, 1), I=512)
    t = _layer(spec, seed=79)
    B, n = spec.B, 2
    per = spec.E // n
    h = (torch.randn(B, spec.D, generator=torch.Generator().manual_seed(13)) * 0.5).to(DEV)
    # every token picks among the first half of the experts
    ex = torch.tensor([[(b * spec.ke + j) % per for j in range(spec.ke)] for b in range(B)], dtype=torch.int32,
                      device=DEV)
    g = torch.full((B, spec.ke), 1.0 / spec.ke, dtype=torch.float32, device=DEV)
    w = synth.ep_slice(t, spec, 1, n, shared=False)
    (wg, wu, wd), keep = _ffn_mats(w, tiled)
    for resid in (None, h):
        part = torch.full((B, spec.D), float("nan"), dtype=torch.float32, device=DEV)
        say(f"[gpu] moe_ffn_ep share 1/{n} with no picks residual={resid is not None} tiled={tiled}")
        dl.moe_ffn_ep(h, ex, g, per, wg, wu, wd, per, 0, part, residual=resid)
        _check_ffn_path(tiled)
        torch.cuda.synchronize()
        assert torch.equal(part, h if resid is not None else torch.zeros_like(h))


@pytest.mark.parametrize("tiled", [False, True])
def test_ffn_skips_negative_expert_ids(tiled):
    # dl_moe_ffn with some slots marked -1 (applied elsewhere) against the oracle, which skips them too; one token
    # has every slot elsewhere, so its output is the residual plus the shared expert
    spec = synth.small_fp8_spec(name="skip", B=4, seq_lens=(900, 600, 300, 1), I=512)
    t = _layer(spec, seed=77)
    B = spec.B
    h = (torch.randn(B, spec.D, generator=torch.Generator().manual_seed(10)) * 0.5).to(DEV)
    ex = torch.empty(B, spec.ke, dtype=torch.int32, device=DEV)
    g = torch.empty(B, spec.ke, dtype=torch.float32, device=DEV)
    dl.moe_route(h, t["w_r"], t["r_bias"], spec.ke, ex, g)
    exs = ex.clone()
    exs[0, 1] = -1
    exs[1, 0] = -1
    exs[1, 3] = -1
    exs[2, :] = -1
    y = torch.empty(B, spec.D, dtype=torch.float32, device=DEV)
    say(f"[gpu] moe_ffn with skipped slots tiled={tiled}")
    (wg, wu, wd), keep = _ffn_mats(t, tiled)
    dl.moe_ffn(h, exs, g, wg, wu, wd, spec.E, spec.n_shared, y, residual=h)
    _check_ffn_path(tiled)
    torch.cuda.synchronize()
    orc = oracle.LayerOracle(spec, t)
    hh = host(h).astype(np.float64)
    exh, gh = host(exs), host(g)
    got = host(y).astype(np.float64)
    for b in range(B):
        y64 = oracle.ffn(hh[b], exh[b], gh[b].astype(np.float64), orc.expert, spec.E, spec.n_shared)
        assert_close(f"skip row {b} y-h", got[b] - hh[b], y64 - hh[b])


@pytest.mark.parametrize("tiled", [False, True])
def test_ffn_repeated_expert_in_a_token(tiled):
    # caller-given picks may name one expert in two slots of a token: each slot is its own pair (its own gate),
    # ranked after the token's earlier picks; the oracle applies the expert once per slot as well
    spec = synth.small_fp8_spec(name="rep", B=4, seq_lens=(900, 600, 300, 1), I=512)
    t = _layer(spec, seed=78)
    B = spec.B
    h = (torch.randn(B, spec.D, generator=torch.Generator().manual_seed(12)) * 0.5).to(DEV)
    ex = torch.empty(B, spec.ke, dtype=torch.int32, device=DEV)
    g = torch.empty(B, spec.ke, dtype=torch.float32, device=DEV)
    dl.moe_route(h, t["w_r"], t["r_bias"], spec.ke, ex, g)
    exr = ex.clone()
    exr[1, 2] = exr[1, 0]
    exr[3, spec.ke - 1] = exr[3, 1]
    exr[3, 0] = exr[3, 1]
    y = torch.empty(B, spec.D, dtype=torch.float32, device=DEV)
    say(f"[gpu] moe_ffn with a repeated expert tiled={tiled}")
    (wg, wu, wd), keep = _ffn_mats(t, tiled)
    dl.moe_ffn(h, exr, g, wg, wu, wd, spec.E, spec.n_shared, y, residual=h)
    _check_ffn_path(tiled)
    torch.cuda.synchronize()
    orc = oracle.LayerOracle(spec, t)
    hh = host(h).astype(np.float64)
    exh, gh = host(exr), host(g)
    assert len(set(exh[3].tolist())) == spec.ke - 2
    got = host(y).astype(np.float64)
    for b in range(B):
        y64 = oracle.ffn(hh[b], exh[b], gh[b].astype(np.float64), orc.expert, spec.E, spec.n_shared)
        assert_close(f"rep row {b} y-h", got[b] - hh[b], y64 - hh[b])


@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("D,I,E,ke,B", [(128, 128, 8, 2, 3), (384, 384, 16, 4, 5), (2048, 256, 64, 6, 40)])
def test_ffn_work_queue_shapes(D, I, E, ke, B, tiled):
    # the expert GEMVs' work queues over K ranges of one 128-block (a single piece per unit), of three blocks
    # (pieces of two and one), and a batch above 16 tokens with 40 x 6 picks over 64 experts (several token
    # groups per expert); two calls in a row give bit-identical outputs whichever waves took which pieces
    spec = synth.small_fp8_spec(name=f"q{D}", B=B, seq_lens=tuple(500 + 37 * i for i in range(B)), D=D, I=I, E=E,
                                ke=ke, topk=256)
    t = _layer(spec, seed=90 + D)
    h = (torch.randn(B, D, generator=torch.Generator().manual_seed(D)) * 0.5).to(DEV)
    ex = torch.empty(B, ke, dtype=torch.int32, device=DEV)
    g = torch.empty(B, ke, dtype=torch.float32, device=DEV)
    dl.moe_route(h, t["w_r"], t["r_bias"], ke, ex, g)
    ys = []
    say(f"[gpu] moe_ffn queue shapes D={D} I={I} E={E} ke={ke} B={B} tiled={tiled}")
    (wg, wu, wd), keep = _ffn_mats(t, tiled)
    for _ in range(2):
        y = torch.empty(B, D, dtype=torch.float32, device=DEV)
        dl.moe_ffn(h, ex, g, wg, wu, wd, E, spec.n_shared, y, residual=h)
        _check_ffn_path(tiled)
        ys.append(y)
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1])
    orc = oracle.LayerOracle(spec, t)
    hh = host(h).astype(np.float64)
    exh, gh = host(ex), host(g)
    got = host(ys[0]).astype(np.float64)
    for b in range(B):
        y64 = oracle.ffn(hh[b], exh[b], gh[b].astype(np.float64), orc.expert, E, spec.n_shared)
        assert_close(f"q{D} row {b} y-h", got[b] - hh[b], y64 - hh[b])
