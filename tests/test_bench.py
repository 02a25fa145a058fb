"""Host-side checks of bench.py (no GPU): the one-GPU contract, the roofline
denominators, and the stored HBM traffic records against the sources they
were measured on and the profiles that hold them."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from blocked_local_self_amd import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode != 0
    assert "exactly one GPU" in res.stderr


# Algorithmic bytes and flops per launch, counted independently of the code:
# bytes = 2 bytes x d x B x heads x (2 H W + 2 (H/s)(W/s)) (k and v read
# once, q read at the query pixels, out written once); flops = 4 d r^2 per
# (query, head) over the full window (QK^T and PV).
@pytest.mark.parametrize("name,alg_bytes,flops", [
    ("early_stage_bf16_64x64_d16_b8h3", 134_217_728, 13_153_337_344),
    ("mid_stage_bf16_32x32_d32_b8h3", 134_217_728, 13_153_337_344),
    ("strided_bf16_64x64_d16_b8h3_s2", 83_886_080, 3_288_334_336),
    ("large_bf16_128x128_d32_b12h3", 268_435_456, 43_486_543_872),
])
def test_roofline_denominators(name, alg_bytes, flops):
    wl = workloads.get(name)
    assert wl.alg_bytes == alg_bytes
    assert wl.flops == flops


def test_headline_is_the_largest_single_gpu_workload():
    stage = [workloads.get(n) for n in workloads.STAGE_WORKLOADS]
    assert workloads.BENCH_WORKLOAD == max(stage, key=lambda w: w.alg_bytes).name


def _records():
    for which, recs in bench.MEASURED_TRAFFIC.items():
        for key, rec in recs.items():
            yield which, key, rec


@pytest.mark.parametrize("which,key,rec", list(_records()), ids=lambda x: x if isinstance(x, str) else "")
def test_traffic_record_matches_sources_and_a_profile(which, key, rec):
    assert rec["bytes_per_launch"] == rec["read"] + rec["write"]
    src = bench.kernel_source_hash(f"{which}:{rec['kernel']}")
    # a kernel change voids the record (the bench then reports traffic as
    # null); the committed records are all for the committed sources
    assert rec["sources"] == src, f"{which} {key}: re-measure FETCH_SIZE / WRITE_SIZE"
    workload = key.split("/")[0]
    holders = [p for p in glob.glob(os.path.join(ROOT, "profiles", "*.txt"))
               if workload in os.path.basename(p) and src in open(p).read()]
    assert holders, f"no profile under profiles/ names {workload} and sources {src}"
