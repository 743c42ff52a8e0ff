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


def test_multi_gpu_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
