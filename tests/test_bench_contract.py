"""CPU checks of the benchmark's contract: it refuses more than one GPU with a message and a
non-zero exit, and the counter profiles it reads its per-kernel figures from (VALU instructions
per element of the stochastic-rounding quantizers, HBM bytes of the GEMM launches) were taken on
the kernel sources as they stand, so that the figures it reports are not stale."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
    assert not r.stdout.strip().startswith("{")          # no result line


def test_valu_profile_matches_the_quantizer_sources():
    rec = bench.valu_per_element()
    assert set(rec) == {"k_dual_quant<SR>", "k_mx_quant_dual<SR>"}, (
        "profiles/ffn_pair_step_quantizer_valu_counters.md was taken on other quantizer sources")
    assert all(20 < v < 80 for v in rec.values())


def test_traffic_profile_matches_the_gemm_sources():
    t = bench.gemm_traffic()
    assert t is not None, "profiles/ffn_pair_step_hbm_traffic.md was taken on other GEMM sources"
    # at least the algorithmic bytes of the six GEMMs (operands once, outputs once), at most 10x
    assert 3.5e9 < t < 4e10


def test_profiles_name_their_commands():
    for name in os.listdir(os.path.join(ROOT, "profiles")):
        text = open(os.path.join(ROOT, "profiles", name)).read()
        assert "rocprofv3" in text, name
