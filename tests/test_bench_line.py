"""The final line of bench.py (the JSON contract) stays compact and carries
the fields the measurement needs, whatever the detail run holds."""

import json

import bench


def test_contract_line_is_compact_and_complete():
    per_m = {M: 100.0 + M / 7.0 for M in bench.MS}
    roof = {"bound": "mfma", "achieved": 1234.56789, "peak": bench.PEAK_F16_TFLOPS,
            "unit": "TFLOP/s", "frac": 0.490123456, "traffic": 512345678.0,
            "launch_us": 501.23456,
            "kernel": "mlp_chain_kernel cfg 12: 256x192x64 tile, 512 threads, rowsync "
                      "(M=2048, one launch per call)"}
    cpu = {"value": 0.01234567, "unit": "TFLOP/s", "cores": 16, "kind": "oracle",
           "sample": "x" * 160, "seconds": {"mlp_M%d" % M: 3.21 for M in bench.MS},
           "host_cpus": 256, "affinity_cpus": 16}
    cpu["seconds"].update({"tiny_mlp": 0.01, "conv_32x56x56x64": 1.5, "attn_B1_S512": 2.2})
    vs = {str(M): {"policy": "tilesync", "chain_us": 123.4, "serial_us": 134.5,
                   "speedup": 1.09, "sentinel_us": 140.1, "sentinel_ring_us": 130.2}
          for M in bench.MS}
    line = bench.contract_line(1002.5, 1.3912345, 20, 5, per_m, roof, cpu, vs)
    assert "\n" not in line
    assert len(line.encode()) < bench.LINE_LIMIT
    d = json.loads(line)
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["metric"] == bench.METRIC
    assert set(d["roofline"]) >= {"bound", "achieved", "peak", "unit", "frac", "traffic"}
    assert d["cpu_baseline"]["cores"] == 16 and d["cpu_baseline"]["kind"] == "oracle"
    assert d["config"]["workload"]
    # no per-policy detail tree on the line
    assert "detail" not in d


def test_contract_line_without_detail_or_baseline():
    per_m = {M: 100.0 for M in bench.MS}
    roof = {"bound": "mfma", "achieved": 1.0, "peak": 2.0, "unit": "TFLOP/s", "frac": 0.5,
            "traffic": None}
    d = json.loads(bench.contract_line(1.0, 1.0, 1, 0, per_m, roof, None, None))
    assert d["cpu_baseline"] is None and "vs_serial" not in d


def test_vs_serial_summary_carries_config5():
    def pol(us):
        return {"mean_us": us, "median_us": us - 4}
    rows = [{"M": 256, "step_policy": "tilesync", "serial": pol(150.0), "tilesync": pol(140.0)},
            {"M": 512, "step_policy": "tilesync", "serial": pol(220.0), "tilesync": pol(210.0),
             "sentinel": pol(225.0), "sentinel_ring": pol(214.0)}]
    v = bench.vs_serial_summary(rows)
    assert v["256"] == {"policy": "tilesync", "chain_us": 140.0, "serial_us": 150.0,
                        "speedup": round(150.0 / 140.0, 3)}
    assert v["512"]["sentinel_us"] == 225.0 and v["512"]["sentinel_ring_us"] == 214.0
