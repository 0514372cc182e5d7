"""The library under HIP graph capture (through PyTorch's graph API): it allocates nothing,
never synchronises and enqueues only kernels on the caller's stream, so a whole step can be
captured once and replayed.  Each replay is compared bit for bit with the eager results,
with eager work and synchronisations between replays."""

from __future__ import annotations

import pytest
import torch

import transformer_attention_07_amd as gqa
from synth import DecodeWorkload, Workload, make_decode_inputs, make_fp8_inputs, make_inputs

pytestmark = pytest.mark.gpu


def _replay_and_compare(graph, outs, want, n=3):
    for r in range(n):
        for t in outs:
            t.fill_(float("nan")) if t.is_floating_point() else t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, exp in zip(("out%d" % i for i in range(len(outs))), outs, want):
            assert torch.equal(got, exp), f"replay {r}: {name} differs from the eager result"
        # eager work between replays
        torch.randn(1 << 16, device="cuda").sum().item()


def test_fwd_bwd_step_in_a_graph():
    w = Workload("graph", B=2, H=8, G=2, S=777, window=200, num_sinks=16, direction="fwd+bwd", seed=8100)
    q, k, v, do = (t.cuda() for t in make_inputs(w))
    kw = dict(window=w.window, num_sinks=w.num_sinks)
    o, lse, o_lo = torch.empty_like(q), torch.empty(q.shape[:3], device="cuda"), torch.empty_like(q)
    dq, dk, dv = (torch.empty(t.shape, dtype=torch.float32, device="cuda") for t in (q, k, k))
    ws = torch.empty(gqa.gqa_attn_bwd_workspace_bytes(q, k, **kw), dtype=torch.uint8, device="cuda")

    def step():
        gqa.gqa_attn_fwd(q, k, v, out=o, lse=lse, o_lo=o_lo, **kw)
        gqa.gqa_attn_bwd(q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws, o_lo=o_lo, **kw)

    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (o, lse, dq, dk, dv)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    _replay_and_compare(g, [o, lse, dq, dk, dv], want)


def test_decode_rope_and_fp8_in_a_graph():
    dw = DecodeWorkload("graph_dec", B=1, H=16, G=2, Sq=4, Skv=5000, window=1024, num_sinks=32, seed=8200)
    dq_, dk_, dv_ = (t.cuda() for t in make_decode_inputs(dw))
    fw = Workload("graph_fp8", B=1, H=8, G=2, S=600, window=128, num_sinks=8, seed=8300)
    q8, k8, v8, sc = make_fp8_inputs(fw)
    q8, k8, v8 = q8.cuda(), k8.cuda(), v8.cuda()
    rw = Workload("graph_rope", B=1, H=8, G=2, S=500, seed=8400)
    rq, rk, rv, _ = (t.cuda() if t is not None else None for t in make_inputs(rw))

    do_ = torch.empty_like(dq_)
    dl = torch.empty(dq_.shape[:3], device="cuda")
    dws = torch.empty(gqa.gqa_attn_decode_workspace_bytes(dq_, dk_, dw.window, dw.num_sinks), dtype=torch.uint8,
                      device="cuda")
    fo = torch.empty(q8.shape, dtype=torch.bfloat16, device="cuda")
    fl = torch.empty(q8.shape[:3], device="cuda")
    fws = torch.empty(gqa.gqa_attn_fwd_fp8_workspace_bytes(q8, k8, window=fw.window, num_sinks=fw.num_sinks),
                      dtype=torch.uint8, device="cuda")
    ro, rl = torch.empty_like(rq), torch.empty(rq.shape[:3], device="cuda")
    rqr, rkr = torch.empty_like(rq), torch.empty_like(rk)

    def calls():
        gqa.gqa_attn_decode(dq_, dk_, dv_, window=dw.window, num_sinks=dw.num_sinks, out=do_, lse=dl, workspace=dws)
        gqa.gqa_attn_fwd_fp8(q8, k8, v8, *sc, window=fw.window, num_sinks=fw.num_sinks, out=fo, lse=fl, workspace=fws)
        gqa.gqa_attn_fwd_rope(rq, rk, rv, out=ro, lse=rl, q_rot=rqr, k_rot=rkr)

    calls()
    torch.cuda.synchronize()
    outs = [do_, dl, fo, fl, ro, rl, rqr, rkr]
    want = [t.clone() for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            calls()
    torch.cuda.synchronize()
    _replay_and_compare(g, outs, want)
