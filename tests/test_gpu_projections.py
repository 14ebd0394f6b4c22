"""GPU parity of the projections around the path, unfolded and folded offline, against
oracle/projections.py (float64), through the C ABI.  Bar: 2e-2 relative (bf16 weights and
hidden states, fp32 accumulate; q, q_abs and the folded weights are rounded to bf16 once).
The whole-step cases run hidden state in, hidden state out: the folded chain (folded query
projection -> absorbed decode -> merge -> folded output projection) and the unfolded one
(query projection -> mla_decode_step -> output projection) against the naive decode between
the oracle's unfolded projections."""
import numpy as np
import pytest
import torch

import head_latent_attention_02_amd as mla
from oracle import mla as ref
from oracle import projections as pj
from workloads import get_config, make_inputs, make_projection_inputs
from workloads.device import DeviceInputs, to_dev
from workloads.gen import bf16_round

pytestmark = pytest.mark.gpu

TOL = 2e-2
ROPE_BASE = 10000.0


def rel_err(got, want):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    assert got.shape == want.shape and np.all(np.isfinite(got))
    return float(np.max(np.abs(got - want)) / np.max(np.abs(want)))


def setup(name, d_model, **kw):
    cfg = get_config(name, **kw)
    inp = make_inputs(cfg, seed=41)
    pr = make_projection_inputs(cfg, d_model, seed=41)
    d = DeviceInputs(inp)
    dev = dict(x=to_dev(pr.x, "bf16"), w_q=to_dev(pr.w_q, "bf16"), w_o=to_dev(pr.w_o, "bf16"))
    return cfg, inp, pr, d, dev


CASES = [("dsv2-b16-t4096", 512, dict(batch=2, ctx=("list", [300, 129]))),
         ("gqla-b32-t8192", 512, dict(batch=3, ctx=("list", [700, 65, 1]))),
         ("mtp-b64-ragged", 256, dict(batch=2, ctx=("list", [130, 64])))]
# more tokens than one matrix-core block of 32: 80 tokens (three blocks, the last partial)
# and 140 tokens (a second workgroup of token blocks, 12 tokens in it)
MANY = [("mtp-b64-ragged", 256, dict(batch=40, ctx=("list", [130 + 7 * i for i in range(40)]))),
        ("dsv2-b16-t4096", 256, dict(batch=140, ctx=("list", [64 + i for i in range(140)])))]


@pytest.mark.parametrize("name,d_model,kw", CASES + MANY)
def test_query_projection_unfolded_and_folded(name, d_model, kw):
    cfg, inp, pr, d, dev = setup(name, d_model, **kw)
    print(f"case {name} d_model={d_model} B={cfg.batch} s_q={cfg.s_q}", flush=True)
    B, s_q, H = cfg.batch, cfg.s_q, cfg.n_heads
    q = torch.empty(B, s_q, H, cfg.d_nope + cfg.d_rope, dtype=torch.bfloat16, device="cuda")
    mla.mla_project_q(d.shape, d_model, ROPE_BASE, dev["x"], dev["w_q"], d.ctx_lens, q)
    wqf = torch.empty(H, cfg.D, d_model, dtype=torch.bfloat16, device="cuda")
    mla.mla_fold_q_weights(d.shape, d_model, dev["w_q"], d.w_uk, wqf)
    q_abs = torch.empty(B, s_q, H, cfg.D, dtype=torch.bfloat16, device="cuda")
    mla.mla_project_q_folded(d.shape, d_model, ROPE_BASE, dev["x"], wqf, d.ctx_lens, q_abs)
    torch.cuda.synchronize()
    want_q = pj.project_query(pr.x, pr.w_q, inp.ctx_lens, s_q, cfg.d_nope)
    want_w = pj.fold_query_weights(pr.w_q, inp.w_uk, cfg.d_nope)
    e_q = rel_err(q.float().cpu().numpy(), want_q)
    e_w = rel_err(wqf.float().cpu().numpy(), want_w)
    # the folded projection against the oracle over the same bf16-rounded folded weights,
    # and against the unfolded definition (projection then absorption)
    got_abs = q_abs.float().cpu().numpy()
    wqf_np = wqf.float().cpu().numpy()
    e_abs = rel_err(got_abs, pj.project_query_folded(pr.x, wqf_np, inp.ctx_lens, s_q, cfg.d_c))
    e_def = rel_err(got_abs, ref.absorb_query(want_q, inp.w_uk, cfg.d_nope))
    print(f"  q {e_q:.3e}  folded weights {e_w:.3e}  q_abs {e_abs:.3e} (definition "
          f"{e_def:.3e})", flush=True)
    assert max(e_q, e_w, e_abs, e_def) <= TOL


@pytest.mark.parametrize("name,d_model,kw", CASES + MANY)
def test_output_projection_unfolded_and_folded(name, d_model, kw):
    cfg, inp, pr, d, dev = setup(name, d_model, **kw)
    B, s_q, H = cfg.batch, cfg.s_q, cfg.n_heads
    rng = np.random.default_rng(5)
    o_lat_np = rng.standard_normal((B, s_q, H, cfg.d_c)).astype(np.float32)
    out_np = rng.standard_normal((B, s_q, H, cfg.d_v)).astype(np.float32)
    o_lat, out = torch.from_numpy(o_lat_np).cuda(), torch.from_numpy(out_np).cuda()
    y = torch.empty(B, s_q, d_model, dtype=torch.float32, device="cuda")
    mla.mla_out_project(d.shape, d_model, out, dev["w_o"], y)
    torch.cuda.synchronize()
    e_y = rel_err(y.cpu().numpy(), pj.output_projection(out_np, pr.w_o))
    wof = torch.empty(d_model, H * cfg.d_c, dtype=torch.bfloat16, device="cuda")
    mla.mla_fold_o_weights(d.shape, d_model, dev["w_o"], d.w_uv, wof)
    y2 = torch.empty_like(y)
    mla.mla_out_project_folded(d.shape, d_model, o_lat, wof, y2)
    torch.cuda.synchronize()
    want_w = pj.fold_output_weights(pr.w_o, inp.w_uv, H)
    e_w = rel_err(wof.float().cpu().numpy(), want_w)
    e_y2 = rel_err(y2.cpu().numpy(), pj.output_projection(ref.up_project_values(o_lat_np,
                                                                                inp.w_uv),
                                                          pr.w_o))
    print(f"  y {e_y:.3e}  folded weights {e_w:.3e}  folded y {e_y2:.3e}", flush=True)
    assert max(e_y, e_w, e_y2) <= TOL


@pytest.mark.parametrize("name,d_model,kw", CASES)
def test_whole_step_hidden_in_hidden_out(name, d_model, kw):
    cfg, inp, pr, d, dev = setup(name, d_model, **kw)
    B, s_q, H = cfg.batch, cfg.s_q, cfg.n_heads
    # oracle: unfolded projections around the naive decode
    q_ref = pj.project_query(pr.x, pr.w_q, inp.ctx_lens, s_q, cfg.d_nope)
    out_ref, _ = ref.mla_decode_naive(q_ref, inp.pool_view(), inp.page_table, inp.ctx_lens,
                                      inp.w_uk, inp.w_uv, cfg.scale, cfg.page_size, cfg.d_c)
    want = pj.output_projection(out_ref, pr.w_o)
    # folded chain on the GPU
    wqf = torch.empty(H, cfg.D, d_model, dtype=torch.bfloat16, device="cuda")
    wof = torch.empty(d_model, H * cfg.d_c, dtype=torch.bfloat16, device="cuda")
    mla.mla_fold_q_weights(d.shape, d_model, dev["w_q"], d.w_uk, wqf)
    mla.mla_fold_o_weights(d.shape, d_model, dev["w_o"], d.w_uv, wof)
    op = d.o_part_view(cfg.d_c)
    y_f = torch.empty(B, s_q, d_model, dtype=torch.float32, device="cuda")
    mla.mla_project_q_folded(d.shape, d_model, ROPE_BASE, dev["x"], wqf, d.ctx_lens, d.q_abs)
    mla.mla_decode_absorbed(d.shape, d.q_abs, d.pool, d.page_table, d.ctx_lens, op,
                            d.lse_part)
    mla.mla_splitkv_combine(d.shape, cfg.d_c, op, d.lse_part, d.o_lat, d.lse)
    mla.mla_out_project_folded(d.shape, d_model, d.o_lat, wof, y_f)
    # unfolded chain on the GPU
    q = torch.empty(B, s_q, H, cfg.d_nope + cfg.d_rope, dtype=torch.bfloat16, device="cuda")
    y_u = torch.empty_like(y_f)
    mla.mla_project_q(d.shape, d_model, ROPE_BASE, dev["x"], dev["w_q"], d.ctx_lens, q)
    mla.mla_decode_step(d.shape, q, d.w_uk, d.w_uv, d.pool, d.page_table, d.ctx_lens, d.q_abs,
                        d.o_part, d.lse_part, d.o_lat, d.out, d.lse)
    mla.mla_out_project(d.shape, d_model, d.out, dev["w_o"], y_u)
    torch.cuda.synchronize()
    e_f = rel_err(y_f.cpu().numpy(), want)
    e_u = rel_err(y_u.cpu().numpy(), want)
    print(f"  whole step: folded {e_f:.3e}  unfolded {e_u:.3e}", flush=True)
    assert e_f <= TOL and e_u <= TOL


def test_full_size_projections_long_b4():
    """The long-context workload's shapes at d_model 5120 (128 heads): every projection at
    full size, the folded weights checked on sampled heads."""
    cfg, inp, pr, d, dev = setup("long-b4-t131072", 5120, ctx=("list", [131072, 64, 7, 5000]))
    B, s_q, H = cfg.batch, cfg.s_q, cfg.n_heads
    q = torch.empty(B, s_q, H, cfg.d_nope + cfg.d_rope, dtype=torch.bfloat16, device="cuda")
    mla.mla_project_q(d.shape, 5120, ROPE_BASE, dev["x"], dev["w_q"], d.ctx_lens, q)
    wqf = torch.empty(H, cfg.D, 5120, dtype=torch.bfloat16, device="cuda")
    mla.mla_fold_q_weights(d.shape, 5120, dev["w_q"], d.w_uk, wqf)
    q_abs = torch.empty(B, s_q, H, cfg.D, dtype=torch.bfloat16, device="cuda")
    mla.mla_project_q_folded(d.shape, 5120, ROPE_BASE, dev["x"], wqf, d.ctx_lens, q_abs)
    wof = torch.empty(5120, H * cfg.d_c, dtype=torch.bfloat16, device="cuda")
    mla.mla_fold_o_weights(d.shape, 5120, dev["w_o"], d.w_uv, wof)
    rng = np.random.default_rng(6)
    o_lat_np = rng.standard_normal((B, s_q, H, cfg.d_c)).astype(np.float32)
    out_np = rng.standard_normal((B, s_q, H, cfg.d_v)).astype(np.float32)
    y = torch.empty(B, s_q, 5120, dtype=torch.float32, device="cuda")
    y2 = torch.empty_like(y)
    mla.mla_out_project(d.shape, 5120, torch.from_numpy(out_np).cuda(), dev["w_o"], y)
    mla.mla_out_project_folded(d.shape, 5120, torch.from_numpy(o_lat_np).cuda(), wof, y2)
    torch.cuda.synchronize()
    heads = [0, 77, 127]
    want_q = pj.project_query(pr.x, pr.w_q, inp.ctx_lens, s_q, cfg.d_nope)
    want_wf = pj.fold_query_weights(pr.w_q[heads], inp.w_uk[heads], cfg.d_nope)
    errs = dict(
        q=rel_err(q.float().cpu().numpy(), want_q),
        wq_folded=rel_err(wqf.float().cpu().numpy()[heads], want_wf),
        q_abs=rel_err(q_abs.float().cpu().numpy(),
                      ref.absorb_query(want_q, inp.w_uk, cfg.d_nope)),
        y=rel_err(y.cpu().numpy(), pj.output_projection(out_np, pr.w_o)),
        y_folded=rel_err(y2.cpu().numpy(), pj.output_projection(
            ref.up_project_values(o_lat_np, inp.w_uv), pr.w_o)))
    print(f"  full-size projection errors {errs}", flush=True)
    assert max(errs.values()) <= TOL
