"""bench.py's host-side rules, without a GPU: which committed counter summary
(profiles/hbm_traffic_*.json) a bench line may report as `roofline.traffic`."""
import importlib.util
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("workload,m,kernels", [
    ("llama2_7b", 10, ["step_fused"]),
    ("llama2_13b", 37, ["compress", "adamstats_apply"]),
    ("llama2_13b", 20, ["compress", "adamstats_apply"]),
])
def test_committed_counter_summaries(workload, m, kernels):
    # each summary names the kernels it measured, with positive byte counts; it
    # is used exactly when it was taken on the kernel source as it is now
    b = _bench()
    rec = json.load(open(os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}_m{m}.json")))
    assert rec["workload"] == workload and rec["m"] == m and set(rec["kernels"]) == set(kernels)
    for k in rec["kernels"].values():
        assert k["fetch_bytes"] > 0 and k["write_bytes"] > 0 and k["launches_per_step"] >= 1
    t = b.load_traffic(workload, m, False, kernels)
    assert (t is not None) == (rec["kernel_source_sha256"] == b.kernel_source_sha())


def test_counters_apply_only_to_the_default_step_and_its_kernels():
    b = _bench()
    # a variant (decay, bf16, global quantizer, forced dense) never reports them
    assert b.load_traffic("llama2_7b", 10, True, ["step_fused"]) is None
    # nor a run whose kernels differ from the measured ones
    assert b.load_traffic("llama2_7b", 10, False, ["compress", "adamstats_apply"]) is None
    assert b.load_traffic("llama2_7b", 10, False, ["step_fused", "compress"]) is None
    # nor a configuration without a summary
    assert b.load_traffic("bert_base", 10, False, ["step_fused"]) is None


def test_counters_are_dropped_when_the_kernel_source_changes(tmp_path, monkeypatch):
    b = _bench()
    src = tmp_path / "kernels.hpp"
    src.write_text(open(b.KERNEL_SRC).read() + "\n// changed\n")
    monkeypatch.setattr(b, "KERNEL_SRC", str(src))
    assert b.load_traffic("llama2_7b", 10, False, ["step_fused"]) is None
