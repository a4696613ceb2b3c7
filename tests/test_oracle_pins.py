"""Pins of the CPU oracle to facts other than itself: closed forms, hand-worked values, brute force on tiny
inputs, invariants, and special cases that reduce to a library routine (torch / numpy).  Runs on the CPU."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


# --------------------------------------------------------------- decoding
def test_fp8_hand_values():
    g = json.load(open(os.path.join(GOLD, "fp8_e4m3fn_hand.json")))
    for code, val in g["codes"].items():
        got = oracle.fp8_decode([int(code, 16)])[0]
        assert got == val, code
        assert math.copysign(1.0, got) == math.copysign(1.0, val), code


def test_fp8_all_codes_vs_library_and_order():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.fp8_decode(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.all(np.isnan(ours[nan]))
    assert np.array_equal(ours[~nan], lib[~nan])
    pos = ours[:0x7F]
    assert np.all(np.diff(pos) > 0)              # codes 0..0x7E increase strictly
    assert np.array_equal(ours[0x80:0xFF], -pos)  # sign bit mirrors


def test_bf16_rne_equals_veltkamp_split():
    # Introducing Kiln, "The hyper-connection arithmetic was what spilled": in fp32, c = 65537 x and
    # hi = c - (c - x) is exactly the round-to-nearest-even bf16 value (checked there on 100,000 values).
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100_000) * np.exp2(rng.integers(-60, 60, 100_000))).astype(np.float32)
    base = torch.from_numpy(x).to(torch.bfloat16).float().numpy().view(np.uint32)
    ties = (base | np.uint32(0x8000)).view(np.float32)[:2000]     # exact half-way cases
    x = np.concatenate([x, ties])
    c = (x * np.float32(65537)).astype(np.float32)
    hi = (c - (c - x)).astype(np.float32)
    ours = oracle.bf16_round(x.astype(np.float64))
    ours_f = (ours.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(ours_f, hi)
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, lib)


def test_bf16_round_ties_to_even_hand():
    assert list(oracle.bf16_round([1.0, 1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 0.0, -0.0])) == \
        [0x3F80, 0x3F80, 0x3F82, 0xBF80, 0x0000, 0x8000]


# ---------------------------------------------------------------- indexer
def _pool(P, ps, DI, rng, lo=-127, hi=127):
    return rng.integers(lo, hi + 1, (P, ps, DI)).astype(np.int8)


def test_indexer_unit_query_picks_coordinate():
    rng = np.random.default_rng(2)
    kp = _pool(5, 8, 16, rng)
    pt = np.array([3, 0, 4, 1, 2], dtype=np.int32)
    for d in (0, 7, 15):
        q = np.zeros((1, 16), np.int8)
        q[0, d] = 1
        s = oracle.indexer_scores(q, kp, pt, 37)
        for p in range(37):
            assert s[p] == max(0, int(kp[pt[p // 8], p % 8, d]))


def test_indexer_closed_forms_and_int32_bound():
    kp = np.ones((2, 64, 128), np.int8)
    q = np.ones((16, 128), np.int8)
    assert np.all(oracle.indexer_scores(q, kp, np.array([0, 1], np.int32), 100) == 16 * 128)
    s = oracle.indexer_scores(np.full((16, 128), 127, np.int8), np.full((1, 64, 128), 127, np.int8),
                              np.array([0], np.int32), 64)
    assert np.all(s == 16 * 128 * 127 * 127) and 16 * 128 * 127 * 127 == 33_032_192
    # an all-negative head contributes nothing
    q2 = np.ones((2, 128), np.int8)
    q2[1] = -1
    assert np.all(oracle.indexer_scores(q2, kp, np.array([0, 1], np.int32), 128) == 128)


def test_indexer_relu_pair_gives_abs_dot():
    rng = np.random.default_rng(3)
    kp = _pool(4, 16, 32, rng)
    v = rng.integers(-127, 128, 32).astype(np.int8)
    q = np.stack([v, -v.astype(np.int16)]).astype(np.int8)    # relu(x) + relu(-x) = |x|
    pt = np.array([2, 0, 3, 1], np.int32)
    s = oracle.indexer_scores(q, kp, pt, 60)
    keys = kp[pt].reshape(-1, 32)[:60].astype(np.int64)
    assert np.array_equal(s, np.abs(keys @ v.astype(np.int64)))


def test_indexer_page_table_indirection():
    ps = 8
    P = 6
    kp = np.zeros((P, ps, 4), np.int8)
    for pg in range(P):
        for sl in range(ps):
            kp[pg, sl, 0], kp[pg, sl, 1] = pg, sl
    q = np.zeros((2, 4), np.int8)
    q[0, 0] = 1
    q[1, 1] = 1
    pt = np.array([5, 2, 0, 4], np.int32)
    s = oracle.indexer_scores(q, kp, pt, 29)
    assert [int(v) for v in s] == [int(pt[p // ps]) + p % ps for p in range(29)]


# ------------------------------------------------------------------ top-k
def _brute_topk(s, k):
    """Position p is kept iff fewer than k positions beat it under (score desc, position asc)."""
    L = len(s)
    keep = [p for p in range(L) if sum(1 for r in range(L) if s[r] > s[p] or (s[r] == s[p] and r < p)) < k]
    return keep + [-1] * (k - len(keep))


def test_topk_hand_cases():
    g = json.load(open(os.path.join(GOLD, "topk_hand.json")))
    for c in g["cases"]:
        assert list(oracle.topk(np.array(c["scores"], np.int32), c["k"])) == c["sel"]


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 200))
    k = int(rng.integers(1, 260))
    s = rng.integers(0, 6 if seed % 2 else 10**6, L).astype(np.int32)   # odd seeds: tie-heavy
    assert list(oracle.topk(s, k)) == _brute_topk(list(s), k)


def test_topk_threshold_characterisation():
    rng = np.random.default_rng(9)
    s = rng.integers(0, 50, 4000).astype(np.int32)
    k = 256
    sel = oracle.topk(s, k)
    assert np.all(np.diff(sel) > 0) and len(sel) == k
    T = np.sort(s)[::-1][k - 1]
    gt = np.nonzero(s > T)[0]
    eq = np.nonzero(s == T)[0][: k - len(gt)]
    assert np.array_equal(sel, np.sort(np.concatenate([gt, eq])))


def test_topk_k_at_least_L_and_all_equal():
    s = np.arange(10, dtype=np.int32)[::-1].copy()
    assert list(oracle.topk(s, 12)) == list(range(10)) + [-1, -1]
    assert list(oracle.topk(np.full(100, 7, np.int32), 5)) == [0, 1, 2, 3, 4]


# -------------------------------------------------------------- attention
def _fp8_lib(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _latents_lib(kv, ks, pt, ps, positions):
    """Decoded latents of positions through torch's FP8 decode (independent of the oracle's)."""
    out = []
    for p in positions:
        pg, sl = pt[p // ps], p % ps
        if kv.dtype == np.uint8:
            c = _fp8_lib(kv[pg, sl]) * np.repeat(ks[pg, sl].astype(np.float64), 128)[: kv.shape[2]]
        else:
            c = kv[pg, sl].astype(np.float64)
        out.append(c)
    return np.array(out)


def _small_attn_inputs(seed, fp8=True, P=6, ps=16, H=4, Dc=192, L=80):
    rng = np.random.default_rng(seed)
    lat = torch.from_numpy(rng.standard_normal((P * ps, 1, Dc)).astype(np.float32))
    if fp8:
        codes, sc = synth.quant_fp8_blocks(lat, 1, 128)
        kv = codes.reshape(P, ps, Dc).numpy()
        ks = sc.reshape(P, ps, -1).numpy()
    else:
        kv, ks = lat.reshape(P, ps, Dc).numpy(), None
    q = rng.standard_normal((H, Dc)).astype(np.float32)
    pt = rng.permutation(P).astype(np.int32)
    return q, kv, ks, pt, ps, L


@pytest.mark.parametrize("fp8", [True, False])
def test_attention_all_positions_is_full_attention(fp8):
    q, kv, ks, pt, ps, L = _small_attn_inputs(4, fp8)
    sel = np.arange(L, dtype=np.int32)
    Dv = 128
    o, p = oracle.attention(q, kv, ks, pt, sel, 0.125, Dv, want_p=True)
    C = torch.from_numpy(_latents_lib(kv, ks, pt, ps, range(L)))
    Q = torch.from_numpy(q.astype(np.float64))
    ref = torch.softmax(0.125 * Q @ C.T, dim=-1) @ C[:, :Dv]
    assert np.allclose(o, ref.numpy(), rtol=1e-12, atol=1e-13)
    assert np.all(np.abs(p.sum(1) - 1.0) < 1e-12)


def test_attention_special_cases():
    q, kv, ks, pt, ps, L = _small_attn_inputs(5)
    Dv = 160
    # a single selected position returns its value part exactly
    sel = np.array([-1, 17, -1, -1], np.int32)
    o = oracle.attention(q, kv, ks, pt, sel, 0.1, Dv)
    c17 = _latents_lib(kv, ks, pt, ps, [17])[0][:Dv]
    assert np.array_equal(o, np.tile(c17, (q.shape[0], 1)))
    # q = 0 gives the mean of the selected values
    sel = np.array([3, 9, 40, 77, -1], np.int32)
    o0 = oracle.attention(np.zeros_like(q), kv, ks, pt, sel, 0.1, Dv)
    mean = _latents_lib(kv, ks, pt, ps, [3, 9, 40, 77])[:, :Dv].mean(0)
    assert np.allclose(o0, np.tile(mean, (q.shape[0], 1)), rtol=0, atol=1e-14)
    # order of the selected list does not matter
    o1 = oracle.attention(q, kv, ks, pt, sel, 0.1, Dv)
    o2 = oracle.attention(q, kv, ks, pt, sel[[4, 2, 0, 3, 1]], 0.1, Dv)
    assert np.allclose(o1, o2, rtol=1e-13, atol=1e-15)
    # no selected entry (empty sequence) -> zeros
    assert np.all(oracle.attention(q, kv, ks, pt, np.full(4, -1, np.int32), 0.1, Dv) == 0)


def test_attention_identical_latents():
    q, kv, ks, pt, ps, L = _small_attn_inputs(6)
    kv[:] = kv[0, 0]
    ks[:] = ks[0, 0]
    o = oracle.attention(q, kv, ks, pt, np.arange(0, 60, 3, dtype=np.int32), 0.3, 192)
    c = _latents_lib(kv, ks, pt, ps, [0])[0]
    assert np.allclose(o, np.tile(c, (q.shape[0], 1)), rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------- projection
def _dec_mat(w, s):
    """Decode block-scaled FP8 [..., R, C] through torch (library) for a dense reference."""
    v = _fp8_lib(w)
    R, Cc = w.shape[-2:]
    sc = np.repeat(np.repeat(s.astype(np.float64), 128, axis=-2), 128, axis=-1)[..., :R, :Cc]
    return v * sc


def test_out_proj_identity_and_library():
    rng = np.random.default_rng(7)
    H, Dv = 4, 16
    o = rng.standard_normal((H, Dv))
    x = rng.standard_normal(H * Dv).astype(np.float32)
    h = oracle.out_proj(o, None, None, np.eye(H * Dv, dtype=np.float32), None, x)
    assert np.array_equal(h, x.astype(np.float64) + o.ravel())
    # FP8 block-scaled W_UV and W_O against a dense numpy product of torch-decoded weights
    H, Dv, hd, D = 3, 256, 128, 384
    o = rng.standard_normal((H, Dv))
    wuv, suv = synth.quant_fp8_blocks(torch.from_numpy(rng.standard_normal((H, hd, Dv)).astype(np.float32) * .02),
                                      128, 128)
    wo, so = synth.quant_fp8_blocks(torch.from_numpy(rng.standard_normal((D, H * hd)).astype(np.float32) * .02),
                                    128, 128)
    xb = torch.from_numpy(rng.standard_normal(D).astype(np.float32)).to(torch.bfloat16)
    xbits = xb.view(torch.int16).numpy().view(np.uint16)
    h = oracle.out_proj(o, wuv.numpy(), suv.numpy(), wo.numpy(), so.numpy(), xbits)
    Wuv = _dec_mat(wuv.numpy(), suv.numpy())
    Wo = _dec_mat(wo.numpy(), so.numpy())
    u = np.einsum("hrv,hv->hr", Wuv, o).ravel()
    ref = xb.double().numpy() + Wo @ u
    assert np.allclose(h, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- router
def test_router_brute_force_and_gates():
    rng = np.random.default_rng(8)
    E, D, ke = 12, 40, 3
    h = rng.standard_normal(D)
    wr = (rng.standard_normal((E, D)) / np.sqrt(D)).astype(np.float32)
    wr[5] = wr[2]                                        # exact tie: expert 2 must win over 5
    bias = np.zeros(E, np.float32)
    lg, ex, g = oracle.router(h, wr, bias, ke)
    assert np.allclose(lg, wr.astype(np.float64) @ h, rtol=1e-13, atol=1e-13)
    order = sorted(range(E), key=lambda e: (-lg[e], e))
    assert list(ex) == order[:ke]
    assert abs(g.sum() - 1) < 1e-15 and np.all(np.diff(g) <= 0)
    ref = torch.softmax(torch.tensor(lg[ex]), 0).numpy()
    assert np.allclose(g, ref, rtol=1e-14)
    # one-hot router rows read h directly; ke = 1 gives gate 1
    wr1 = np.eye(D, dtype=np.float32)[:E]
    lg1, ex1, g1 = oracle.router(h, wr1, None, 1)
    assert np.array_equal(lg1, h[:E]) and ex1[0] == int(np.argmax(h[:E])) and g1[0] == 1.0
    # tie between duplicated rows resolves to the lower id on both sides of the boundary
    wr2 = np.zeros((4, D), np.float32)
    lg2, ex2, _ = oracle.router(h, wr2, np.array([0, 1, 1, 0], np.float32), 2)
    assert list(ex2) == [1, 2]


# ------------------------------------------------------------------- FFN
def _expert_bank(rng, n, D, I, fp8):
    bank = {}
    for e in range(n):
        ws = [rng.standard_normal(s).astype(np.float32) * 0.05 for s in ((I, D), (I, D), (D, I))]
        if fp8:
            parts = []
            for w in ws:
                c, s = synth.quant_fp8_blocks(torch.from_numpy(w), 128, 128)
                parts += [c.numpy(), s.numpy()]
            bank[e] = tuple(parts)
        else:
            bank[e] = (ws[0], None, ws[1], None, ws[2], None)
    return bank


@pytest.mark.parametrize("fp8", [True, False])
def test_ffn_single_expert_is_dense_swiglu(fp8):
    rng = np.random.default_rng(10)
    D, I = 256, 384
    bank = _expert_bank(rng, 3, D, I, fp8)
    h = rng.standard_normal(D)
    y = oracle.ffn(h, [1], [1.0], bank.__getitem__, 3, 0)
    wg, sg, wu, su, wd, sd = bank[1]
    dec = (lambda w, s: _dec_mat(w, s)) if fp8 else (lambda w, s: w.astype(np.float64))
    Wg, Wu, Wd = (torch.from_numpy(dec(w, s)) for w, s in ((wg, sg), (wu, su), (wd, sd)))
    ht = torch.from_numpy(h)
    ref = ht + Wd @ (torch.nn.functional.silu(Wg @ ht) * (Wu @ ht))
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_ffn_structure():
    rng = np.random.default_rng(11)
    D, I = 128, 128
    bank = _expert_bank(rng, 5, D, I, False)          # experts 0..3 routed, 4 shared
    h = rng.standard_normal(D)
    y_sh = oracle.ffn(h, [2, 0], [0.75, 0.25], bank.__getitem__, 4, 1)
    y_no = oracle.ffn(h, [2, 0], [0.75, 0.25], lambda e: bank[e], 4, 0)
    f_sh = oracle.ffn(h, [4], [1.0], bank.__getitem__, 5, 0) - h       # shared expert alone, gate 1
    assert np.allclose(y_sh - y_no, f_sh, rtol=1e-12, atol=1e-13)
    y2 = oracle.ffn(h, [2, 0], [1.5, 0.5], bank.__getitem__, 4, 0)      # linear in the gates
    assert np.allclose(y2 - h, 2 * (y_no - h), rtol=1e-13, atol=1e-14)
    zero = {e: (w[0], None, w[2], None, np.zeros_like(w[4]), None) for e, w in bank.items()}
    assert np.array_equal(oracle.ffn(h, [1, 3], [0.5, 0.5], zero.__getitem__, 4, 1), h)   # W_down = 0


# ------------------------------------------------------------ whole rows
def test_layer_rows_tiny_fp8():
    spec = synth.small_fp8_spec(B=2, seq_lens=(700, 0), D=256, H=4, head_dim=128, topk=256, E=6, ke=2, I=256)
    t = synth.make_layer(spec, seed=3)
    orc = oracle.LayerOracle(spec, t)
    r0 = orc.row(0)
    assert np.all(np.diff(r0["sel"]) > 0) and r0["sel"].min() >= 0
    assert len(set(r0["experts"])) == spec.ke and abs(r0["gates"].sum() - 1) < 1e-14
    r1 = orc.row(1)                                   # padding row: nothing selected, o = 0, h = x
    assert np.all(r1["sel"] == -1) and np.all(r1["o"] == 0)
    assert np.array_equal(r1["h"], oracle.bf16_to_f64(t["x"][1].view(torch.int16).numpy().view(np.uint16)))


# ------------------------------------------------------------- current-token append
def _torch_fp8_codes(x32: np.ndarray) -> np.ndarray:
    """torch's own float32 -> e4m3fn conversion (nearest, ties to even), as codes."""
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_round_hand_values():
    # ties go to the even code; the format saturates at 448; the sign of a zero result is kept
    cases = {1.0625: 0x38, 1.1875: 0x3A, 2.0 ** -10: 0x00, 3 * 2.0 ** -11: 0x01, 2.0 ** -9: 0x01,
             448.0: 0x7E, 1000.0: 0x7E, -1000.0: 0xFE, -1e-4: 0x80, 0.0: 0x00, 240.0: 0x77, 248.0: 0x78}
    for x, code in cases.items():
        assert int(oracle.fp8_round([x])[0]) == code, x


def test_fp8_round_vs_library():
    # every code, every midpoint between neighbouring codes (exact in fp32), and random values from the
    # subnormal range up to just below 448, both signs: the same codes as torch's conversion
    dec = oracle.fp8_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (dec[:-1] + dec[1:]) / 2
    rng = np.random.default_rng(5)
    rand = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(447.0), 20000))
    x = np.concatenate([dec, mids, rand]).astype(np.float32)
    x = np.concatenate([x, -x])
    assert np.array_equal(oracle.fp8_round(x.astype(np.float64)), _torch_fp8_codes(x))
    # round trip of every finite code
    assert np.array_equal(oracle.fp8_round(dec), np.arange(0x7F, dtype=np.uint8))


@pytest.mark.parametrize("Dc,bf16", [(576, False), (576, True), (64, False), (200, True)])
def test_kv_append_row(Dc, bf16):
    rng = np.random.default_rng(Dc + bf16)
    lat = rng.standard_normal(Dc).astype(np.float32) * np.float32(3.0)
    lat[: min(128, Dc)] *= np.float32(1e-3)           # a block of small values
    if Dc > 256:
        lat[128:256] = 0.0                             # an all-zero block
    key = np.concatenate([rng.uniform(-200, 200, 100), [0.5, 1.5, 2.5, -0.5, -2.5, 127.5, -127.5, 1e6]])
    key = key.astype(np.float32)
    if bf16:
        lat_in = torch.from_numpy(lat).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        key_in = torch.from_numpy(key).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        lat = torch.from_numpy(lat).to(torch.bfloat16).float().numpy()
        key = torch.from_numpy(key).to(torch.bfloat16).float().numpy()
    else:
        lat_in, key_in = lat, key
    ks = np.float32(0.75)
    codes, scales, k8 = oracle.kv_append_row(lat_in, key_in, ks)
    nb = (Dc + 127) // 128
    assert scales.shape == (nb,) and codes.shape == (Dc,)
    for j in range(nb):
        blk = lat[j * 128:(j + 1) * 128]
        amax = np.float32(np.max(np.abs(blk)))
        if amax == 0:
            assert scales[j] == 0 and not codes[j * 128:(j + 1) * 128].any()
            continue
        q = blk / scales[j]                            # fp32 quotient
        # the codes are torch's rounding of the quotient, the largest element maps to +-448, and the decoded
        # value is within half a code spacing of the quotient
        assert np.array_equal(codes[j * 128:(j + 1) * 128], _torch_fp8_codes(q))
        big = int(np.argmax(np.abs(blk)))
        assert codes[j * 128 + big] in (0x7E, 0xFE)
        dq = oracle.fp8_decode(codes[j * 128:(j + 1) * 128])
        spacing = np.where(np.abs(q) < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(q), 1e-30))) - 3))
        assert np.all(np.abs(dq - q) <= spacing / 2 + 1e-12)
        assert abs(scales[j] * 448.0 - amax) <= amax * 2.0 ** -23
    # keys: numpy's round-half-even of the fp32 quotient, clamped to +-127
    want = np.clip(np.rint(key / ks), -127, 127).astype(np.int8)
    assert np.array_equal(k8, want)
    assert list(k8[-8:]) == [1, 2, 3, -1, -3, 127, -127, 127] or bf16
    # exact halves with a unit scale: ties to even
    _, _, kt = oracle.kv_append_row(np.zeros(64, np.float32), np.array([0.5, 1.5, 2.5, -0.5, -2.5, 126.5], np.float32), 1.0)
    assert list(kt) == [0, 2, 2, 0, -2, 126]


# ------------------------------------------------------------- multi-row decode (R query rows per sequence)
def test_multirow_last_row_is_single_row_decode_and_rows_are_causal():
    # R = 3 rows per sequence: the last row of a sequence sees every cached position, so it is exactly the
    # single-row decode of its inputs; row r sees L - (R - 1 - r) positions, so its scores are the prefix of the
    # scores its query gets over the whole sequence, and its selection never reaches beyond its own position.
    R = 3
    spec = synth.spec_replace(synth.config(1), R=R, seq_lens=(700,), topk=256)
    t = synth.make_layer(spec, seed=9)
    multi = oracle.LayerOracle(spec, t)
    single_spec = synth.spec_replace(spec, R=1)
    for r in range(R):
        one = {k: v for k, v in t.items()}
        for name in ("x", "q", "q_idx"):
            one[name] = t[name][r:r + 1]
        full = oracle.LayerOracle(single_spec, one).row(0, stages=("sel",))
        got = multi.row(r, stages=("sel",) if r < R - 1 else ("sel", "o", "h", "route", "y"))
        vis = 700 - (R - 1 - r)
        assert len(got["scores"]) == vis
        assert np.array_equal(got["scores"], full["scores"][:vis])
        kept = got["sel"][got["sel"] >= 0]
        assert kept.size == min(spec.topk, vis) and kept.max() < vis
        if r == R - 1:
            ref = oracle.LayerOracle(single_spec, one).row(0)
            assert np.array_equal(got["sel"], ref["sel"])
            assert np.array_equal(got["y"], ref["y"])


def test_multirow_short_sequence_rows_are_padding():
    # a sequence holding fewer positions than rows: its first rows see nothing (all -1), the rest see 1, 2, ...
    spec = synth.spec_replace(synth.config(1), R=4, seq_lens=(2,), topk=8)
    t = synth.make_layer(spec, seed=2)
    orc = oracle.LayerOracle(spec, t)
    vis = [len(orc.row(r, stages=("sel",))["scores"]) for r in range(4)]
    assert vis == [0, 0, 1, 2]
    assert np.all(orc.row(1, stages=("sel",))["sel"] == -1)


def test_ffn_tensor_parallel_slices_add_up():
    # splitting every expert's intermediate rows (gate/up rows, down columns) into slices splits the FFN output
    # into a sum: SwiGLU acts on each intermediate row on its own, so sum_s f_s(h) = f(h)
    spec = synth.config(1)
    t = synth.make_layer(spec, seed=3)
    orc = oracle.LayerOracle(spec, t)
    r = orc.row(0)
    h, ex, g = r["h"], r["experts"], r["gates"]
    n = 2
    total = np.zeros_like(h)
    for s_ in range(n):
        sub = dict(t)
        sub.update(synth.tp_slice(t, spec, s_, n))
        so = oracle.LayerOracle(synth.spec_replace(spec, I=spec.I // n), sub)
        total += oracle.ffn(h, ex, g, so.expert, spec.E, spec.n_shared) - h
    np.testing.assert_allclose(total + h, r["y64"], rtol=0, atol=1e-12 * max(1.0, float(np.abs(r["y64"]).max())))


# ------------------------------------------------------------- pool-granular selection
def test_pooled_selection_pool1_is_per_position_and_expansion():
    spec = synth.spec_replace(synth.config(1), pool=4, seq_lens=(1001,), topk=64)
    t = synth.make_layer(spec, seed=11)
    q, pt = synth.to_numpy(t["q_idx"])[0], synth.to_numpy(t["page_table"])[0]
    kp = synth.to_numpy(t["k_pool"])
    # pool = 1 over the position keys is exactly the per-position selection
    sel1, _, _ = oracle.pooled_topk(q, kp, pt, 1001, 1, 64)
    assert np.array_equal(sel1, oracle.topk(oracle.indexer_scores(q, kp, pt, 1001), 64))
    # pool = 4: 251 pools (the last holds one position); the kept pools are the top ones by (score, pool) found by
    # plain sorting, expanded to their positions below L, ascending, -1 after
    pk = synth.to_numpy(t["pool_keys"])
    sel, sc, pools = oracle.pooled_topk(q, pk, pt, 1001, 4, 40)
    assert sc.size == 251
    want = sorted(sorted(range(251), key=lambda p: (-int(sc[p]), p))[:40])
    assert list(pools) == want
    valid = sel[sel >= 0]
    assert np.all(np.diff(valid) > 0) and np.all(sel[valid.size:] == -1) and valid.max() < 1001
    assert set(valid // 4) == set(want)
    assert valid.size == 40 * 4 - (3 if 250 in want else 0)


# ------------------------------------------------------------- one GPU's expert-parallel share of the FFN
def test_ffn_expert_parallel_groups_add_up_and_skipped_slot_is_a_zero_gate():
    # a negative expert id marks a slot whose expert another GPU holds: it must add exactly what a zero gate adds
    # (nothing), and splitting the experts into groups (each group's FFN with the other groups' slots skipped, the
    # shared expert and the residual counted once) must sum to the whole FFN
    spec = synth.small_fp8_spec(name="ep-pin", seq_lens=(300,), E=16, ke=4, n_shared=1, I=256, D=512)
    t = synth.make_layer(spec, seed=6)
    orc = oracle.LayerOracle(spec, t)
    r = orc.row(0)
    h, ex, g = r["h"], np.asarray(r["experts"]), np.asarray(r["gates"], dtype=np.float64)
    for j in range(spec.ke):
        e2, g0 = ex.copy(), g.copy()
        e2[j], g0[j] = -1, 0.0
        assert np.array_equal(oracle.ffn(h, e2, g, orc.expert, spec.E, spec.n_shared),
                              oracle.ffn(h, ex, g0, orc.expert, spec.E, spec.n_shared))
    n, per = 4, spec.E // 4
    total = np.zeros_like(r["y64"])
    for grp in range(n):
        mine = np.where((ex >= grp * per) & (ex < (grp + 1) * per), ex, -1)
        total += oracle.ffn(h, mine, g, orc.expert, spec.E, spec.n_shared if grp == 0 else 0) - h
    np.testing.assert_allclose(total + h, r["y64"], rtol=0, atol=1e-12 * max(1.0, float(np.abs(r["y64"]).max())))
    # every slot elsewhere and no shared expert: the output is the residual, exactly
    assert np.array_equal(oracle.ffn(h, np.full(spec.ke, -1), g, orc.expert, spec.E, 0), np.asarray(h, np.float64))
