"""The benchmark's host-side bookkeeping, without a GPU: the algorithmic byte
counts its rooflines divide by, the source digest that decides whether a
committed counter summary still describes the kernels, and the one-GPU
guard."""
import os
import subprocess
import sys

import numpy as np

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_decode_bytes_per_launch():
    # wkv 20480 x 6144 bf16 + 24 blocks of 84 B + kv 20480 bf16 + rows 6144 bf16
    # + both layers' 48 row ids + token id, map entry and 4 history entries
    w = synth.DECODE_Q2K
    want = 20480 * 6144 * 2 + 24 * 84 + 20480 * 2 + 6144 * 2 + 2 * 24 * 8 + 4 + 8 + 8 * 4
    assert bench.decode_bytes(w) == want == 251_713_932
    # wkv as Q2_K blocks: 20480 rows of 24 blocks of 84 B instead of the bf16 matrix
    wq = synth.DECODE_WKVQ2K
    assert bench.decode_q2kw_bytes(wq) == want - 20480 * 6144 * 2 + 20480 * 24 * 84 == 41_343_372


def test_source_digest_ignores_comments_only(tmp_path, monkeypatch):
    csrc = tmp_path / "csrc"
    csrc.mkdir()
    (csrc / "k.hip").write_text('#include "h.h"\nint f() { return 1; }  // one\n')
    (csrc / "h.h").write_text("int g();\n")
    monkeypatch.setattr(bench, "CSRC", str(csrc))
    d0 = bench.source_digest("k.hip")
    (csrc / "k.hip").write_text('#include "h.h"\n// a new comment\n\nint f() { return 1; }\n')
    assert bench.source_digest("k.hip") == d0
    (csrc / "h.h").write_text("int g(int);\n")          # an included header's code counts
    assert bench.source_digest("k.hip") != d0


def test_counter_traffic_needs_the_current_digest(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    digest = bench.source_digest("decode.hip")
    (tmp_path / "cur.md").write_text(
        f"source_sha256_16: {digest}\nhbm_bytes_per_launch: 252040986\n")
    (tmp_path / "old.md").write_text(
        "source_sha256_16: 0000000000000000\nhbm_bytes_per_launch: 252040986\n")
    assert bench.counter_traffic("cur.md", "decode.hip") == 252040986.0
    assert bench.counter_traffic("old.md", "decode.hip") is None
    assert bench.counter_traffic("missing.md", "decode.hip") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2 and "single MI355X" in r.stderr


def test_cpu_baseline_runs_its_own_stream():
    """The oracle leg draws its own prompt + max_steps token ids and per-step
    highways, so it never runs out of tokens whatever --steps/--warmup the GPU
    legs used (the driver's --steps 20 --warmup 5 gave those legs an 82-token
    stream, and the leg once hashed an empty slice at its 51st step)."""
    from synth import generate as G
    w = synth.ODD_Q2K
    ht = G.hash_tables(w)
    host = [G.layer_inputs(w, ht, l) for l in range(w.n_layers)]
    r = bench.cpu_baseline(w, ht, host, budget_s=120.0, max_steps=96, threads=2)
    assert r["steps"] == 96 and r["kind"] == "oracle" and r["cores"] == 2
    assert r["value"] > 0 and "96 single-token decode steps" in r["sample"]
    # a tiny budget stops after the first step, never before it
    r = bench.cpu_baseline(w, ht, host, budget_s=0.0, max_steps=96, threads=1)
    assert r["steps"] == 1


def test_cpu_baseline_gates_the_workload_highway(monkeypatch):
    """Each step gates that step's highway from the workload's decode stream
    (G.highway(w, n, decode=True)[step]), as the GPU decode leg does."""
    import oracle
    from synth import generate as G
    w = synth.ODD_Q2K
    ht = G.hash_tables(w)
    host = [G.layer_inputs(w, ht, l) for l in range(w.n_layers)]
    seen = []
    real = oracle.gate_and_add

    def spy(h, *a, **k):
        seen.append(np.array(h, copy=True))
        return real(h, *a, **k)

    monkeypatch.setattr(oracle, "gate_and_add", spy)
    bench.cpu_baseline(w, ht, host, budget_s=120.0, max_steps=3, threads=1)
    hw = G.highway(w, 3, decode=True)
    for step in range(3):
        np.testing.assert_array_equal(seen[step * w.n_layers], hw[step:step + 1])


def test_cpu_baseline_prefill_sample():
    from synth import generate as G
    w = synth.ODD_E4M3
    ht = G.hash_tables(w)
    host = [G.layer_inputs(w, ht, l) for l in range(w.n_layers)]
    r = bench.cpu_baseline_prefill(w, ht, host, sample_tokens=8, threads=2)
    assert r["tokens"] == 8 and r["cores"] == 2 and r["kind"] == "oracle"
    assert r["value"] > 0 and "first 8 of the" in r["sample"]


def test_oracle_threads_respects_omp_cap(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    assert 1 <= bench.oracle_threads() <= 3


def test_q2kw_valu_roofline_needs_the_current_digest(tmp_path, monkeypatch):
    """The Q2_K-wkv decode kernel's VALU roofline: instructions per launch
    from a counter summary taken on the current source, over the live launch
    time, against 1024 SIMDs x 2.4 GHz / 4 cycles a wave64 instruction."""
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    w = synth.DECODE_WKVQ2K
    (tmp_path / "decode_q2kw_counters.md").write_text(
        f"source_sha256_16: {bench.source_digest('decode.hip')}\n"
        "valu_instructions_per_launch: 9830400\nhbm_bytes_per_launch: 1\n")
    r = bench.q2kw_valu_roofline(0.02, w)
    assert r["bound"] == "alu" and abs(r["peak"] - 614.4) < 1e-9
    assert abs(r["achieved"] - 9830400 / 0.02e-3 / 1e9) < 1e-6
    assert abs(r["frac"] - 9830400 / 0.02e-3 / (1024 * 2.4e9 / 4)) < 1e-12
    assert abs(r["lane_instructions_per_weight"] - 9830400 * 64 / (20480 * 6144)) < 1e-12
    (tmp_path / "decode_q2kw_counters.md").write_text(
        "source_sha256_16: 0000000000000000\nvalu_instructions_per_launch: 9830400\n")
    assert bench.q2kw_valu_roofline(0.02, w) is None


def test_run_leg_reports_a_failing_leg(capsys):
    """A secondary leg that raises leaves an error entry (and its traceback
    on stderr) instead of ending the run; a leg that works returns its result."""
    assert bench.run_leg("ok", lambda: {"value": 1.0}) == {"value": 1.0}

    def boom():
        raise AssertionError("in_f")
    r = bench.run_leg("cpu baseline", boom)
    assert bench.failed(r) and r["error"] == "AssertionError: in_f"
    err = capsys.readouterr().err
    assert "cpu baseline: failed: AssertionError: in_f" in err and "Traceback" in err
    assert not bench.failed({"value": 1.0}) and not bench.failed(None)
