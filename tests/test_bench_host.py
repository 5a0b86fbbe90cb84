"""Host-side parts of bench.py that run without a GPU: the one-GPU refusal,
the oracle baseline leg, and the keys of the measured-traffic table."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_cpu_baseline_fields():
    import bench
    from mla_synth import WORKLOADS

    res = bench.cpu_baseline(WORKLOADS["tiny_f32"], 0.5)
    assert res["kind"] == "oracle" and res["unit"] == "tokens/s"
    assert res["value"] > 0 and res["cores"] >= 1 and res["seconds"] > 0
    assert res["fp64_gflop"] > 0
    assert "1 of 1 sequences" in res["sample"]


def test_traffic_table_keys():
    """Every measured-traffic entry names a bench workload and a 16-digit
    source hash; entries of the current sources carry both byte counts."""
    import bench
    from mla_synth import WORKLOADS

    for (h, name), v in bench.MEASURED_TRAFFIC.items():
        assert len(h) == 16 and int(h, 16) >= 0
        assert name in WORKLOADS
        assert v["fetch_bytes"] > 0 and v["write_bytes"] > 0
    sid = bench.splitkv_source_id()
    assert len(sid) == 16
    assert sid == bench.splitkv_source_id()


@pytest.mark.parametrize("name", ["dsv2_b32_ctx4096", "llama2_7b_mla_b64_ctx8192"])
def test_measured_fetch_covers_the_cache(name):
    """Where the table has an entry for the current sources, the split-KV
    launch fetched at least the latent cache it reads (1,152 bytes a token)
    and at most 10% more."""
    import bench
    from mla_synth import WORKLOADS

    v = bench.MEASURED_TRAFFIC.get((bench.splitkv_source_id(), name))
    if v is None:
        pytest.skip("no counters for the current attention sources")
    wl = WORKLOADS[name]
    latent = int(wl.seq_lens().astype("int64").sum()) * (wl.shape.d_c + wl.shape.d_rope) * 2
    assert latent <= v["fetch_bytes"] <= 1.10 * latent
