"""Graph capture: attn_decode_fwd_noalloc (the entry point for callers that
cannot allocate, such as code under graph capture) and attn_prefill_fwd
recorded into one HIP graph through torch.cuda.graph, replayed several times
with new inputs copied in eagerly between the replays; every replay must give
the same bits as the same calls made eagerly (MI355X only)."""
import sys

import numpy as np
import pytest
import torch

import attn_inputs as A
import exact_attention_31_amd as E
from gpu_helpers import to_device

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def test_decode_noalloc_and_prefill_replay_in_a_graph():
    _announce("graph: decode (no workspace) + prefill, 4 replays")
    B, Hq, Hkv, N, d = 4, 16, 2, 3000, 128
    k = to_device(A.random_tensor((B, Hkv, N, d), 801, "bf16"), "bf16")
    v = to_device(A.random_tensor((B, Hkv, N, d), 802, "bf16"), "bf16")
    lens = torch.tensor([3000, 17, 1999, 2500], dtype=torch.int32, device="cuda")
    qd = torch.empty((B, Hq, 1, d), dtype=torch.bfloat16, device="cuda")
    od = torch.empty_like(qd)
    lsed = torch.empty((B, Hq, 1), dtype=torch.float32, device="cuda")
    Bp, Hp, Np, dp = 1, 4, 700, 128
    qp = torch.empty((Bp, Hp, Np, dp), dtype=torch.bfloat16, device="cuda")
    kp = to_device(A.random_tensor((Bp, Hp, Np, dp), 803, "bf16"), "bf16")
    vp = to_device(A.random_tensor((Bp, Hp, Np, dp), 804, "bf16"), "bf16")

    def inputs(i):
        return (to_device(A.random_tensor((B, Hq, 1, d), 810 + i, "bf16"), "bf16"),
                to_device(A.random_tensor((Bp, Hp, Np, dp), 820 + i, "bf16"), "bf16"))

    def step():
        E.attn_decode_fwd_noalloc(qd, k, v, od, kv_lens=lens, lse=lsed)
        return E.attn_prefill_fwd(qp, kp, vp, causal=True)

    # warm-up on a side stream (first calls set up the library's per-device state)
    q0, p0 = inputs(0)
    qd.copy_(q0)
    qp.copy_(p0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        op = step()
    torch.cuda.synchronize()

    for i in range(1, 5):
        qi, pi = inputs(i)
        qd.copy_(qi)
        qp.copy_(pi)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_o, got_lse, got_p = od.clone(), lsed.clone(), op.clone()
        # the same calls, eagerly, into fresh outputs
        oe = torch.empty_like(qd)
        lse_e = torch.empty_like(lsed)
        E.attn_decode_fwd_noalloc(qd, k, v, oe, kv_lens=lens, lse=lse_e)
        pe = E.attn_prefill_fwd(qp, kp, vp, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(got_o, oe), f"replay {i}: decode output differs"
        assert torch.equal(got_lse, lse_e), f"replay {i}: decode lse differs"
        assert torch.equal(got_p, pe), f"replay {i}: prefill output differs"
        assert np.isfinite(got_o.float().cpu().numpy()).all()
        print(f"  replay {i} ok", flush=True)
