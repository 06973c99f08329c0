"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the readers of
the committed rocprofv3 summaries, and that those summaries were taken on
the kernel sources now in the tree (otherwise bench.py reports null for
their figures)."""
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("argv, env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                       (["--gpus", "1"], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True,
                       text=True, env=e, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _summary(tmp_path, body, sources=()):
    p = tmp_path / "summary.txt"
    p.write_text("# header: ignored\n" + body + "source_sha256: %s\n" % bench.source_digest(sources))
    return str(p)


def test_profile_fields_keep_the_first_value_of_a_repeated_field(tmp_path):
    p = _summary(tmp_path, "workload: first\nmfma_busy_frac: 0.5\n\nworkload: second\nmfma_busy_frac: 0.3\n")
    vals = bench.profile_fields(p, ())
    assert vals["workload"] == "first" and vals["mfma_busy_frac"] == "0.5"
    assert bench.mfma_counters(p, ()) == {"mfma_busy_frac": 0.5}


def test_summaries_of_other_sources_are_not_used(tmp_path):
    p = _summary(tmp_path, "traffic_bytes_per_launch: 123\n", sources=bench.PREFILL_SOURCES)
    assert bench.pmc_traffic(p, bench.PREFILL_SOURCES) == 123.0
    assert bench.pmc_traffic(p, bench.DECODE_SOURCES) is None
    assert bench.profile_fields(os.path.join(str(tmp_path), "missing.txt"), ()) is None


@pytest.mark.parametrize("summary, sources", [
    (bench.DECODE_PMC, bench.DECODE_SOURCES),
    (bench.PREFILL_PMC, bench.PREFILL_SOURCES),
    (bench.PREFILL_MFMA, bench.PREFILL_SOURCES),
    ("profiles/decode_bf16_B32_Hq64_Hkv8_d128_L4096.kernel_trace.txt", bench.DECODE_SOURCES),
    ("profiles/prefill_bf16_B2_P4096_Hq32_Hkv8_d128_causal.kernel_trace.txt", bench.PREFILL_SOURCES),
    ("profiles/decode_ex_B32_Hq64_Hkv8_d128_L4096.kernel_trace.txt", bench.EXT_SOURCES),
])
def test_committed_summaries_match_the_kernel_sources(summary, sources):
    assert bench.profile_fields(summary, sources) is not None, (
        "%s was taken on other kernel sources: profile again" % summary)


def test_committed_counters_read_back():
    # decode: every cached byte fetched once (calibrated FETCH + WRITE)
    t = bench.pmc_traffic(bench.DECODE_PMC, bench.DECODE_SOURCES)
    assert abs(t / 537919488 - 1.0) < 0.01
    # prefill: the causal leg is the one read, not the windowed one listed after it
    m = bench.mfma_counters(bench.PREFILL_MFMA, bench.PREFILL_SOURCES)
    assert m["algorithmic_flop_per_launch"] == 274945015808
    assert 0.0 < m["mfma_busy_frac"] < 1.0 and 1.0 < m["shader_clock_ghz"] < 2.5


def test_clock_reader_parses_the_amd_smi_layout(monkeypatch):
    body = {"gpu_data": [{"gpu": 0, "clock": dict(
        {"gfx_%d" % x: {"clk": {"value": 2000 + x, "unit": "MHz"}, "max_clk": {"value": 2400, "unit": "MHz"}}
         for x in range(8)},
        mem_0={"clk": {"value": 2000, "unit": "MHz"}}, fclk_0="N/A")}]}
    out = "WARNING: some notice\n" + json.dumps(body)
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: subprocess.CompletedProcess(a, 0, out, ""))
    c = bench.smi_clocks()
    assert c["gfx_mhz_per_xcd"] == [2000.0 + x for x in range(8)]
    assert c["gfx_mhz_mean"] == 2003.5 and c["mem_mhz"] == 2000.0
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: subprocess.CompletedProcess(a, 1, "", "no GPU"))
    assert bench.smi_clocks() is None
