"""Host logic of bench.py (CPU only): work accounting matches the oracle's counts,
and multi-GPU requests are refused."""
import itertools

import attn_inputs as A
import bench
import oracle


def test_visible_pairs_closed_form_matches_oracle_count():
    for nq, n in itertools.product(range(0, 40), range(0, 40)):
        for causal in (False, True):
            assert bench.visible_pairs(nq, n, causal) == oracle.visible_pairs(nq, n, causal), (nq, n, causal)
    for nq, n in [(4096, 4096), (23400, 23400), (1, 32768), (100, 32768), (5000, 300)]:
        assert bench.visible_pairs(nq, n, True) == oracle.visible_pairs(nq, n, True)


def test_workload_figures():
    assert bench.prefill_flops(A.CONFIGS[2]) == 4 * 128 * 128 * 4096 * 4097 // 2
    assert abs(bench.prefill_flops(A.CONFIGS[4]) - 8.796e12) / 8.796e12 < 1e-3
    cfg = A.CONFIGS[5]
    assert bench.decode_kv_bytes(cfg, [32768] * 64) == 4 * 2 ** 30
    assert bench.prefill_bytes(A.CONFIGS[2]) == 4 * 4 * 32 * 4096 * 128 * 2


def test_multi_gpu_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_every_workload_has_a_config_and_is_timed_by_default():
    assert set(bench.DEFAULT_ORDER) == set(bench.WORKLOADS)
    assert bench.DEFAULT_ORDER[0] == "prefill_c4"          # the largest single-GPU prefill workload
    for name, (cid, desc) in bench.WORKLOADS.items():
        assert cid in A.CONFIGS and desc


def test_traffic_reduction_from_counter_csvs(tmp_path, monkeypatch):
    """--traffic-from: per-dispatch counters (median per kernel, summed over a
    step's kernels) scaled by the copy calibration."""
    header = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n"

    def write(folder, rows):
        d = tmp_path / folder / "host"
        d.mkdir(parents=True)
        (d / "run_counter_collection.csv").write_text(header + "".join(
            f"{i},\"{k}\",X,{v}\n" for i, (k, v) in enumerate(rows)))

    write("copy_FETCH_SIZE", [("__amd_rocclr_copyBuffer", 524288.0)] * 3)
    write("copy_WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1048576.0)] * 3)
    write("prefill_c2_FETCH_SIZE", [("void attn::(anonymous namespace)::prefill16_kernel<a, b>(int)", 1000.0),
                                    ("void attn::(anonymous namespace)::prefill16_kernel<a, b>(int)", 3000.0),
                                    ("void at::native::elementwise_kernel<x>(y)", 1e9)])
    write("prefill_c2_WRITE_SIZE", [("void attn::(anonymous namespace)::prefill16_kernel<a, b>(int)", 500.0)])
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    out = bench.traffic_from(str(tmp_path))
    rec = out["workloads"]["prefill_c2"]
    assert out["calibration"]["fetch_scale"] == 2.0 and out["calibration"]["write_scale"] == 1.0
    assert rec["bytes_per_step"] == (2000.0 * 2.0 + 500.0) * 1024
    assert set(out["workloads"]) == {"prefill_c2"}
