"""GPU parity for the single-pass skip rule (KVQ_SKIP_RUNNING): the fused
kernel against the oracle's attend_running with the kernel's own split size
and 64-position blocks. Masks are compared outside the band around the
threshold of the running weight; outputs, counts and kept mass as for the
exact rule. Every case prints its name before touching the GPU."""
import dataclasses

import numpy as np
import pytest

import synth
from gpu_helpers import compare, run_gpu, say
from oracle import attend as A
from oracle import formats as F

pytestmark = pytest.mark.gpu


def _positions_per_split(ctx, splits):
    """The plan's split size for an explicit split count: ceil(ctx / splits)
    rounded up to 64 positions."""
    p = -(-ctx // splits)
    return -(-p // 64) * 64


def _run(name, splits, threshold=None, **kw):
    w = synth.resized(synth.workload(name), **kw) if kw else synth.workload(name)
    inp = synth.generate(w)
    tau = w.threshold if threshold is None else threshold
    g = run_gpu(inp, tau, splits=splits, running=True)
    P = _positions_per_split(w.ctx, splits)
    assert g["splits"] == -(-w.ctx // P)
    kc, ks = F.pack(w.fmt, inp.k)
    vc, vs = F.pack(w.fmt, inp.v)
    r, p_run = A.attend_running(inp.q, kc, ks, vc, vs, fmt=w.fmt, dim=w.dim, v_dim=w.v_dim, ctx_len=w.ctx,
                                sigma=w.sigma, threshold=tau, positions_per_split=P, block=64)
    # the band around the threshold is taken on the weight the decision uses
    compare(inp, tau, g, dataclasses.replace(r, p=p_run), dict(kc=kc, ks=ks, vc=vc, vs=vs))
    exact = A.attend(inp.q, kc, ks, vc, vs, fmt=w.fmt, dim=w.dim, v_dim=w.v_dim, ctx_len=w.ctx, sigma=w.sigma,
                     threshold=tau)
    say(f"  running rule: {r.rows_fetched} rows ({r.kept_pairs} pairs) vs exact {exact.rows_fetched} "
        f"({exact.kept_pairs}); gpu rows {g['stats']['rows_fetched']}")
    return g, r, exact


@pytest.mark.parametrize("splits", [1, 4, 16])
def test_running_tiny_q8_0(splits):
    say("case running tiny q8_0 splits", splits)
    _run("tiny", splits)


@pytest.mark.parametrize("fmt,splits", [("q4_0", 8), ("q4_0", 32), ("q8_0", 32), ("lut3", 16)])
def test_running_grouped_formats(fmt, splits):
    say("case running", fmt, "B2 32/4 ctx 4096 splits", splits)
    g, r, exact = _run("long", splits, fmt=fmt, batch=2, ctx=4096, hot=8)
    assert r.rows_fetched >= exact.rows_fetched


def test_running_long_full_size():
    say("case running long q4_0 ctx 32768, 64 splits (the default plan)")
    g, r, exact = _run("long", 64)
    assert g["splits"] == 64


def test_running_stress_many_kept():
    say("case running stress q4_0 (logit std 4.5), 64 splits")
    _run("stress", 64)


def test_running_ragged_and_threshold_zero():
    say("case running ragged ctx 3001 q4_0, 8 splits, tau 1e-6 and 0")
    _run("long", 8, batch=1, ctx=3001, hot=4)
    _run("long", 8, threshold=0.0, batch=1, ctx=3001, hot=4)
