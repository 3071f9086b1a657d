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


def _summaries():
    d = os.path.join(ROOT, "profiles")
    return sorted(f for f in os.listdir(d) if f.startswith("hbm_traffic_") and f.endswith(".json"))


def test_every_configuration_has_a_summary():
    # the default line's headline and every entry of its configs array
    want = {"hbm_traffic_llama2_7b_m10.json", "hbm_traffic_tiny_m10.json", "hbm_traffic_bert_base_m10.json",
            "hbm_traffic_opt_1_3b_m10.json"} | {f"hbm_traffic_llama2_13b_m{m}.json" for m in (1, 10, 20, 37)}
    assert want <= set(_summaries())


@pytest.mark.parametrize("name", _summaries())
def test_committed_counter_summaries(name):
    # each summary names the kernels it measured, with positive byte counts (the
    # fused step at least; a partial last block adds the two general kernels);
    # it is used exactly when it was taken on the kernel source as it is now
    b = _bench()
    rec = json.load(open(os.path.join(ROOT, "profiles", name)))
    workload, m, kernels = rec["workload"], rec["m"], sorted(rec["kernels"])
    assert name == f"hbm_traffic_{workload}_m{m}.json"
    assert "step_fused" in kernels and set(kernels) <= {"step_fused", "compress", "adamstats_apply"}
    k = rec["kernels"]["step_fused"]
    assert k["fetch_bytes"] > 0 and k["write_bytes"] > 0 and k["launches_per_step"] >= 1
    assert rec["fetch_scale"] > 0 and rec["write_scale"] > 0
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
    assert b.load_traffic("llama2_13b", 30, False, ["step_fused"]) is None


@pytest.mark.parametrize("which", [0, 1])
def test_counters_are_dropped_when_the_kernel_source_changes(tmp_path, monkeypatch, which):
    # a change to the kernels or to the host code that launches them
    b = _bench()
    srcs = list(b.KERNEL_SRCS)
    changed = tmp_path / os.path.basename(srcs[which])
    changed.write_text(open(srcs[which]).read() + "\n// changed\n")
    before = b.kernel_source_sha()
    srcs[which] = str(changed)
    monkeypatch.setattr(b, "KERNEL_SRCS", srcs)
    assert b.kernel_source_sha() != before
    assert b.load_traffic("llama2_7b", 10, False, ["step_fused"]) is None
