"""The byte model behind bench.py's roofline figures, checked against hand counts of what one step must read.
Runs on the CPU."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_expert_bytes_are_fp8_weights_plus_block_scales():
    s = synth.config(2)
    # gate and up: 2 x [2048, 6144] FP8 codes + 2 x (16 x 48) fp32 scales; down: [6144, 2048] + 48 x 16 scales
    gu = 2 * 2048 * 6144 + 2 * 16 * 48 * 4
    dn = 6144 * 2048 + 48 * 16 * 4
    assert bench.EXPERT_BYTES_GATE_UP(s) == gu
    assert bench.EXPERT_BYTES_DOWN(s) == dn
    assert gu + dn == 37_757_952  # one touched expert


def test_step_bytes_at_batch_8_and_128k():
    s = synth.config(2)
    b = bench.algorithmic_bytes(s, s.seq_lens, 59)
    assert b["indexer_keys"] == 8 * 131072 * 128            # every cached key once, int8 [128]
    assert b["selected_kv"] == 8 * 2048 * (576 + 5 * 4)      # kept latents: FP8 codes + 5 fp32 block scales
    assert b["w_o"] == 6144 * 8192 + 48 * 64 * 4             # W_O [6144, 64 x 128] FP8 + block scales
    assert b["w_uv"] == 64 * 128 * 512 + 64 * 1 * 4 * 4      # W_UV per head [128, 512] FP8 + block scales
    assert b["w_r"] == 256 * 6144 * 4                        # router weights fp32
    assert b["expert_gate_up"] + b["expert_down"] == 59 * 37_757_952
    assert b["total"] == sum(v for k, v in b.items() if k != "total")


def test_short_rows_pools_and_multi_row_counts():
    s = synth.spec_replace(synth.config(2), seq_lens=(1000, 5000, 0) + (131072,) * 5)
    b = bench.algorithmic_bytes(s, s.seq_lens, 1)
    assert b["selected_kv"] == (1000 + 2048 + 0 + 5 * 2048) * 596  # a short row keeps all of its positions
    p = synth.spec_replace(s, pool=4)
    bp = bench.algorithmic_bytes(p, p.seq_lens, 1)
    assert bp["indexer_keys"] == (250 + 1250 + 0 + 5 * 32768) * 128  # one key per pool of 4 positions
    r = synth.spec_replace(synth.config(2), R=2, seq_lens=(2048, 1) + (131072,) * 6)
    br = bench.algorithmic_bytes(r, r.seq_lens, 1)
    # row r of a sequence sees seq_len - (R - 1 - r) positions: 2047 + 2048, 0 + 1, then 2 x 2048 for the rest
    assert br["selected_kv"] == (2047 + 2048 + 0 + 1 + 6 * 2 * 2048) * 596


def test_bench_refuses_more_than_one_gpu():
    """The build measures one GPU: asked for more, bench.py exits with status 2 and says so, before touching a GPU."""
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""
