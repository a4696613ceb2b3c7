"""The GPU parity checker itself, run on the CPU with oracle results standing in for the GPU's: it must compare
every stage, accept the oracle's own outputs and reject planted mistakes."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import check_rows


@pytest.fixture(scope="module")
def case():
    oracle.build(force=False)
    spec = synth.small_fp8_spec(name="harness", B=2, seq_lens=(900, 0), D=256, H=4, E=6, ke=2, I=256, topk=256)
    t = synth.make_layer(spec, seed=11)
    orc = oracle.LayerOracle(spec, t)
    rows = [orc.row(b) for b in range(spec.B)]
    dbg = {"sel": torch.from_numpy(np.stack([r["sel"] for r in rows])),
           "o": torch.from_numpy(np.stack([r["o"] for r in rows]).astype(np.float32)),
           "h": torch.from_numpy(np.stack([r["h"] for r in rows]).astype(np.float32)),
           "experts": torch.from_numpy(np.stack([r["experts"] for r in rows])),
           "gates": torch.from_numpy(np.stack([r["gates"] for r in rows]).astype(np.float32)),
           "y32": torch.from_numpy(np.stack([r["y64"] for r in rows]).astype(np.float32))}
    y = torch.from_numpy(np.stack([r["y"] for r in rows]).view(np.int16)).view(torch.bfloat16)
    return spec, t, dbg, y


def test_accepts_oracle_outputs_on_every_stage(case):
    spec, t, dbg, y = case
    w = check_rows(spec, t, dbg, y, [0, 1])
    assert w["rows"] == 2 and w["near_ties"] == 0
    assert w["o"] < 1e-6 and w["gates"] < 1e-6 and w["y-h"] < 1e-5 and w["y"] == 0.0


@pytest.mark.parametrize("what", ["sel", "o", "h", "experts", "gates", "y32", "y"])
def test_rejects_planted_mistakes(case, what):
    spec, t, dbg, y = case
    d = {k: v.clone() for k, v in dbg.items()}
    yy = y.clone()
    if what == "sel":
        d["sel"][0, 3] += 1
    elif what == "o":
        d["o"][0, 1, 5] += 0.05 * float(d["o"][0].abs().max())
    elif what == "h":
        d["h"][0, 7] += 0.05 * float((d["h"][0] - t["x"][0].float()).abs().max())
    elif what == "experts":
        d["experts"][0] = torch.flip(d["experts"][0], [0])
    elif what == "gates":
        d["gates"][0] = torch.flip(d["gates"][0], [0])
    elif what == "y32":
        d["y32"][0, 9] += 0.05 * float((d["y32"][0] - d["h"][0]).abs().max())
    else:
        yy[0, 9] = (yy[0, 9].float() + 1.0).to(torch.bfloat16)
    with pytest.raises(AssertionError):
        check_rows(spec, t, d, yy, [0, 1])
