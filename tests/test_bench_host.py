"""Host-side logic of bench.py (no GPU): the one-GPU contract, the pair counts behind the FLOP figures, and the
staleness rule of the committed traffic summaries."""
import json
import os
import shutil
import subprocess
import sys
import types

import numpy as np
import pytest

import bench
import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


@pytest.mark.parametrize("W,C,rank", [(2, 3, 0), (2, 3, 1), (4, 5, 2), (8, 2, 7)])
def test_ring_pair_counts_match_the_oracle_masks(W, C, rank):
    """bench.py's closed forms per ring step against counts of the oracle's causal mask on zigzag positions."""
    cfg = types.SimpleNamespace(kind="ring", W=W, C=C, B=1, H=1, rank=rank)
    got = bench.pairs_per_launch(cfg, None)
    S = 2 * W * C
    pq = oracle.zigzag_positions(S, W, rank)
    want = []
    for t in range(W):
        src = oracle.ring_source(rank, t, W)
        pk = oracle.zigzag_positions(S, W, src)
        want.append(int(oracle.allowed_mask(pq, pk, True).sum()))
    assert got == want


def test_dense_pair_count_and_flops():
    cfg = synth.get("t")
    n = bench.pairs_per_launch(cfg, None)[0]
    assert n == cfg.S * (cfg.S + 1) // 2 * cfg.H
    small = types.SimpleNamespace(kind="dense", S=77, B=2, H=3)
    assert bench.pairs_per_launch(small, None)[0] == int(oracle.allowed_mask(np.arange(77), np.arange(77), True).sum()) * 6
    assert cfg.flops()["total"] == 14 * cfg.D * n


def _tree(tmp_path):
    root = tmp_path / "repo"
    shutil.copytree(os.path.join(ROOT, "long_context_causal_ea_amd", "csrc"),
                    root / "long_context_causal_ea_amd" / "csrc")
    (root / "profiles").mkdir()
    return root


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    root = _tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(root))
    h0 = {k: bench.source_hash(k) for k in ("fwd", "bwd_dkdv", "xent")}
    f = root / "long_context_causal_ea_amd" / "csrc" / "fwd.hip"
    f.write_text(f.read_text() + "\n// a new comment\n/* and a block\n   comment */\n")
    assert bench.source_hash("fwd") == h0["fwd"]
    f.write_text(f.read_text() + "\nstatic int unused_marker = 1;\n")
    assert bench.source_hash("fwd") != h0["fwd"]
    assert bench.source_hash("bwd_dkdv") == h0["bwd_dkdv"] and bench.source_hash("xent") == h0["xent"]


def test_traffic_counts_only_while_the_kernel_is_unchanged(tmp_path, monkeypatch):
    root = _tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(root))
    prof = root / "profiles" / "traffic_xent_xent.txt"
    prof.write_text("header line\n\nkernel: xent\nhbm_bytes_per_launch: 8.4e9\n"
                    f"source_hash: {bench.source_hash('xent')}\n")
    assert bench.load_traffic("xent", "xent") == pytest.approx(8.4e9)
    assert bench.load_traffic("xent", "other") is None
    f = root / "long_context_causal_ea_amd" / "csrc" / "xent.hip"
    f.write_text(f.read_text() + "\nstatic int changed = 2;\n")
    assert bench.load_traffic("xent", "xent") is None


def test_rotary_bytes():
    b = bench.rope_bytes(65536, 32, 128)
    n = 65536 * 32 * 128
    assert b["fwd"] == 2 * n * 4 and b["inv"] == 2 * n * 8


def test_compulsory_bytes_count_each_tensor_once():
    """Per-launch minimum HBM bytes, tallied tensor by tensor at the 64K-token layer (B1 H32 D128, RoPE) and for a
    ring step (C3: 2C = 65536 local rows and a 65536-key share per launch, 7 of 8 forwards merging)."""
    n = 65536 * 32 * 128                 # elements of one [S, H, D] tensor
    r = 65536 * 32                       # (row, head) pairs
    bf16, f32 = 2 * n, 4 * n
    t = synth.get("t")
    assert bench.compulsory_bytes("fwd", t) == 3 * bf16 + f32 + 4 * r + bf16          # Q K V in, O LSE out, turned Q
    assert bench.compulsory_bytes("bwd_dkdv", t) == 4 * bf16 + 2 * 4 * r + 2 * 2 * f32   # dK dV read and written
    assert bench.compulsory_bytes("bwd_dq", t) == 4 * bf16 + 2 * 4 * r + 2 * f32
    assert bench.compulsory_bytes("bwd_delta", t) == f32 + bf16 + 4 * r
    c3 = synth.get("c3")
    assert bench.compulsory_bytes("fwd", c3) == pytest.approx(3 * bf16 + f32 + 4 * r + (f32 + 4 * r) * 7 / 8)
    assert bench.compulsory_bytes("bwd_dkdv", c3) == bench.compulsory_bytes("bwd_dkdv", t)
