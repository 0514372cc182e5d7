"""Calls on different streams at once.  The library keeps no state between calls, so two
problems enqueued on two streams, overlapping in time, give bit for bit the results each
gives alone."""

from __future__ import annotations

import pytest
import torch

import transformer_attention_07_amd as gqa
from synth import DecodeWorkload, Workload, make_decode_inputs, make_inputs

pytestmark = pytest.mark.gpu


def _step(q, k, v, do, kw, stream):
    o, lse, o_lo = gqa.gqa_attn_fwd(q, k, v, keep_residual=True, stream=stream, **kw)
    return (o, lse) + gqa.gqa_attn_bwd(q, k, v, o, lse, do, o_lo=o_lo, stream=stream, **kw)


def test_two_streams_match_one_at_a_time():
    wa = Workload("sa", B=2, H=16, G=4, S=1500, window=300, num_sinks=40, direction="fwd+bwd", seed=9100)
    wb = Workload("sb", B=1, H=32, G=8, S=2100, direction="fwd+bwd", seed=9200)
    wd = DecodeWorkload("sd", B=2, H=32, G=4, Sq=3, Skv=20000, window=4096, num_sinks=64, seed=9300)
    a = [t.cuda() for t in make_inputs(wa)]
    b = [t.cuda() for t in make_inputs(wb)]
    d = [t.cuda() for t in make_decode_inputs(wd)]
    ka = dict(window=wa.window, num_sinks=wa.num_sinks)
    kd = dict(window=wd.window, num_sinks=wd.num_sinks)
    main = torch.cuda.current_stream()
    # one at a time
    want_a = _step(*a, ka, main)
    want_b = _step(*b, {}, main)
    want_d = gqa.gqa_attn_decode(*d, stream=main, **kd)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        s1.wait_stream(main)
        s2.wait_stream(main)
        with torch.cuda.stream(s1):
            got_a = _step(*a, ka, s1)
            got_d = gqa.gqa_attn_decode(*d, stream=s1, **kd)
        with torch.cuda.stream(s2):
            got_b = _step(*b, {}, s2)
        torch.cuda.synchronize()
        print(f"[streams] repetition {rep}", flush=True)
        for name, got, want in (("a", got_a, want_a), ("b", got_b, want_b), ("decode", got_d, want_d)):
            for i, (x, y) in enumerate(zip(got, want)):
                assert torch.equal(x, y), f"repetition {rep}: problem {name}, output {i} differs"
