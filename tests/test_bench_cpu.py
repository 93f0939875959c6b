"""Host-side logic of bench.py that needs no GPU: the one-GPU refusal, the
algorithmic byte accounting behind `value`, and the gate that reports the
measured HBM traffic only for the kernel sources it was measured on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused_before_touching_a_device():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert out["n_gpus"] == 2 and "one GPU" in out["error"]


def _kept_tokens(T, b, n):
    """Tokens in the last n blocks of a T-token sequence (the last block is
    always kept; it may be partial), counted block by block."""
    NB = (T + b - 1) // b
    return sum(min(b, T - j * b) for j in range(NB - n, NB))


@pytest.mark.parametrize("name", ["qwen3_4b_32k", "batched_64k_gate", "long_512k", "resa_ragged"])
@pytest.mark.parametrize("T_off", [0, 1, 37])
def test_kv_bytes_counts_descriptors_and_kept_tokens(name, T_off):
    w = W.get(name)
    T = w.T0[-1] + T_off
    NB = (T + w.block - 1) // w.block
    es = 2 if w.dtype == "bf16" else 4
    for n in (1, 2, NB // 10 + 1, NB):
        desc, kv = bench.kv_bytes(w, T, n)
        per_block = (2 * w.d * es) if w.desc_kind == W.DESC_MINMAX else (w.d * 4)
        assert desc == w.Hkv * NB * per_block
        assert kv == w.Hkv * _kept_tokens(T, w.block, n) * 2 * w.d * es


def test_headline_bytes_per_step():
    """long_512k at p = 0.9 after one append: 8193 blocks per KV head, 820
    kept (the last holding one token): 33.6 MB of descriptors and 214.7 MB
    of K and V per layer-step."""
    w = W.get("long_512k")
    T = w.T0[0] + 1
    NB = (T + w.block - 1) // w.block
    assert NB == 8193
    n = -(-(10000 - 9000) * NB // 10000)
    assert n == 820
    desc, kv = bench.kv_bytes(w, T, n)
    assert desc == 8 * 8193 * 512
    assert kv == 8 * (819 * 64 + 1) * 512
    assert round((desc + kv) / 1e6, 1) == 248.3


def test_code_only_ignores_comments_and_blank_lines():
    a = "int x = 1;  // one\n\n// note\nint y = 2;\n"
    b = "int x = 1;\nint y = 2;"
    assert bench.code_only(a) == bench.code_only(b)
    assert bench.code_only(a) != bench.code_only("int x = 2;\nint y = 2;")


def test_traffic_is_reported_only_for_the_measured_sources(monkeypatch, tmp_path):
    t = bench.measured_traffic("long_512k", 9000)
    assert isinstance(t, int)
    # about the algorithmic bytes of one call (no re-reads)
    w = W.get("long_512k")
    _, kv = bench.kv_bytes(w, w.T0[0] + 1, 820)
    assert 1.0 <= t / kv < 1.02
    assert bench.measured_traffic("long_512k", 9500) is None
    assert bench.measured_traffic("qwen3_4b_32k", 0) is None
    # a changed kernel source no longer matches the recorded hash
    src = os.path.join(ROOT, bench.TRAFFIC_SOURCES[0])
    changed = tmp_path / "decode.hip"
    changed.write_text(open(src).read() + "\nint one_more_line;\n")
    monkeypatch.setattr(bench, "TRAFFIC_SOURCES", (str(changed),) + bench.TRAFFIC_SOURCES[1:])
    assert bench.measured_traffic("long_512k", 9000) is None


class _FakeRun:
    """The parts of a benchmark run the count check reads."""
    def __init__(self, w, bp):
        import block_sparse_attention_build_amd as bsa
        self.w, self.bsa = w, bsa
        self.P = bsa.SelectParams(budget_tokens=w.budget_tokens, sparsity_bp=bp,
                                  n_local=w.n_local, n_min=w.n_min)


def test_kept_counts_are_checked_against_the_closed_form():
    import numpy as np
    w = W.get("resa_ragged")
    run = _FakeRun(w, w.sparsity_bp)
    lens = [t + 5 for t in w.T0]
    exp = bench.expected_counts(run, lens)
    # 16K: n_min = 16 binds; the others ceil(0.05 * NB)
    assert exp == [16, 39, 77, 103]
    good = [np.tile(np.array(exp)[:, None], (1, w.Hkv)) for _ in range(3)]
    assert bench.check_counts(good, exp) == 3 * w.B * w.Hkv
    bad = [g.copy() for g in good]
    bad[2][1, 4] += 1
    with pytest.raises(RuntimeError, match="layer 2, sequence 1"):
        bench.check_counts(bad, exp)
