"""mla_decode_step_noalloc (workspaces in the library's fixed scratch array) against
mla_decode_step (caller workspaces), through the C ABI (needs gfx950).

Each case makes two calls in a row on one device, the second with a smaller input (fewer
sequences, shorter contexts, chunks with no token), so what the first call left in the
shared scratch must not reach the second's results.  Both entry points run the same kernels
on the same inputs, so out and lse must be bitwise equal; the existing entry point's
workspaces are filled with NaN first, so it cannot pass by reading stale zeros.  The smaller
call is also held to the oracle's bar on every output.
"""
import numpy as np
import pytest
import torch

import head_latent_attention_02_amd as mla
from oracle import mla as ref
from workloads import get_config, make_inputs
from workloads.device import DeviceInputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def announce(msg):
    print(msg, flush=True)


def both_steps(d):
    """(out, lse) of mla_decode_step with NaN-filled workspaces, then of the allocation-free
    entry point, on the same device inputs."""
    for t in (d.q_abs, d.o_part, d.lse_part, d.o_lat, d.out, d.lse):
        t.fill_(float("nan"))
    mla.mla_decode_step(d.shape, d.q, d.w_uk, d.w_uv, d.pool, d.page_table, d.ctx_lens,
                        d.q_abs, d.o_part, d.lse_part, d.o_lat, d.out, d.lse)
    torch.cuda.synchronize()
    want = (d.out.clone(), d.lse.clone())
    out = torch.full_like(d.out, float("nan"))
    lse = torch.full_like(d.lse, float("nan"))
    mla.mla_decode_step_noalloc(d.shape, d.q, d.w_uk, d.w_uv, d.pool, d.page_table,
                                d.ctx_lens, out, lse)
    torch.cuda.synchronize()
    return want, (out, lse)


def check_against_oracle(inp, out, lse):
    c = inp.cfg
    w_out, w_lse = ref.mla_decode_naive(inp.q, inp.pool_view(), inp.page_table, inp.ctx_lens,
                                        inp.w_uk, inp.w_uv, c.scale, c.page_size, c.d_c)
    got = out.cpu().numpy().astype(np.float64)
    err = float(np.max(np.abs(got - w_out)) / np.max(np.abs(w_out)))
    lerr = float(np.max(np.abs(lse.cpu().numpy() - w_lse)) / np.max(np.abs(w_lse)))
    announce(f"  oracle rel err out {err:.3e} lse {lerr:.3e} (bar {TOL[c.dtype]})")
    assert err <= TOL[c.dtype] and lerr <= TOL[c.dtype]


CASES = {
    # first (larger) call, then the smaller one
    "bf16": (("dsv2-b16-t4096", dict(batch=8, ctx=("list", [4096, 3000, 2100, 700, 64, 1,
                                                           4095, 129]))),
             ("dsv2-b16-t4096", dict(batch=2, ctx=("list", [300, 129])))),
    "bf16-long-then-small": (("long-b4-t131072", {}),
                             ("dsv2-b16-t4096", dict(batch=3, ctx=("list", [1000, 65, 2])))),
    "f32": (("tiny-f32", dict(batch=4, ctx=("list", [500, 333, 64, 7]))),
            ("tiny-f32", dict(batch=2, ctx=("list", [40, 1])))),
    # the largest 128-head, 32-split step the scratch holds (7 sequences: 61.7 of 64 MiB),
    # so the workspaces reach the end of the array
    "bf16-max-scratch": (("dsv2-b16-t4096", dict(batch=7, n_splits=32,
                                                 ctx=("list", [4096, 2048, 700, 64, 1, 4000, 130]))),
                         ("dsv2-b16-t4096", dict(batch=2, ctx=("list", [300, 129])))),
    "gqla-mtp": (("gqla-mtp-b32-t65536", dict(batch=6, ctx=("list", [9000, 4097, 3000, 64,
                                                                      700, 2]))),
                 ("gqla-mtp-b32-t65536", dict(batch=2, ctx=("list", [513, 2])))),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_noalloc_step_matches_step_on_two_calls(case):
    for i, (name, over) in enumerate(CASES[case]):
        cfg = get_config(name, **over)
        inp = make_inputs(cfg)
        d = DeviceInputs(inp)
        announce(f"noalloc {case} call {i}: {name} B={cfg.batch} s_q={cfg.s_q} "
                 f"ctx={list(inp.ctx_lens)[:8]} S={d.shape.n_splits}")
        (w_out, w_lse), (out, lse) = both_steps(d)
        assert torch.isfinite(w_out).all() and torch.isfinite(w_lse).all()
        assert torch.equal(out, w_out), "out differs from mla_decode_step"
        assert torch.equal(lse, w_lse), "lse differs from mla_decode_step"
        if i == 1:
            check_against_oracle(inp, out, lse)
        del d


def test_noalloc_step_replays_under_graph_capture():
    """The allocation-free step is capturable in a HIP graph (no allocation, no memset in
    it): five replays, each followed by an eager step, all bitwise equal to the eager
    result, and the eager step matches the oracle."""
    cfg = get_config("dsv2-b16-t4096", batch=3, ctx=("list", [2100, 700, 5]))
    inp = make_inputs(cfg, seed=5)
    d = DeviceInputs(inp)
    announce(f"noalloc graph capture: {cfg.name} B={cfg.batch} ctx={list(inp.ctx_lens)}")

    def step():
        mla.mla_decode_step_noalloc(d.shape, d.q, d.w_uk, d.w_uv, d.pool, d.page_table,
                                    d.ctx_lens, d.out, d.lse)

    step()
    torch.cuda.synchronize()
    want = (d.out.clone(), d.lse.clone())
    check_against_oracle(inp, want[0], want[1])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(5):
        d.out.fill_(float("nan"))
        d.lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d.out, want[0]) and torch.equal(d.lse, want[1]), f"replay {r}"
        step()
        torch.cuda.synchronize()
        assert torch.equal(d.out, want[0]), f"eager step after replay {r}"
