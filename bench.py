#!/usr/bin/env python3
"""Throughput of single-step absorbed MLA decode on one MI355X.

One step = the whole absorbed path on one batch: query absorption -> split-KV decode
over the paged latent cache -> split combine -> value up-projection, all through the C
ABI of libmla.so on one HIP stream.  The workload (default: batch 4 x 131072-token
contexts, 128 heads, latent 512 + RoPE 64, bf16, split-KV over 32 chunks) is seeded and
synthetic and is resident in HBM before timing starts.

K timed steps run the whole step through one library call (`mla_decode_step`, four
kernels) with HIP events on the launch stream around it only: ms_per_step is their median
step time (p10/p90 beside it).  Interleaved with them run K instrumented steps through
the four separate entry points with an event between kernels; they give the per-kernel
times (`kernel_ms`) and the decode kernel's launch time that `roofline` uses.  A 1 GiB
read (a sum over a 1 GiB buffer) before every step, outside the events, evicts the 256 MB
last-level cache so every step reads the cache from HBM; it leaves only clean lines
behind (`--flush write` fills the buffer instead; see _flusher).

Prints ONE JSON line.  `value` is cached-latent-tokens/s of the whole step.
`roofline` describes the decode kernel (the dominant one): algorithmic bytes (every
cached token's 576 bf16 once) / its median launch time from those events; `traffic`
comes from the committed rocprofv3 counter summary when it was taken on the current
kernel source, else null.  `cpu_baseline` times the float64 CPU oracle (naive,
non-absorbed MLA) on a bounded sample of the same workload.  `--path gqa` times the
GQLA per-group path instead (decode + combine on the expanded cache).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, published
KERNEL_SRC = os.path.join(ROOT, "head_latent_attention_02_amd", "csrc", "decode_mfma.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_absorbed_long_b4_t131072_traffic.json")


def kernel_hash():
    """Hash of the decode kernel's source code with comments and blank lines removed, so
    that a counter summary stays valid across comment-only edits."""
    code = []
    with open(KERNEL_SRC) as f:
        for line in f:
            line = line.split("//", 1)[0].strip()
            if line:
                code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the GPU reaches its steady clocks after about a second of continuous work (measured:
    # 5 warmup steps leave the step ~11 % slower and 3x noisier than 2000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default="long-b4-t131072")
    ap.add_argument("--splits", type=int, default=None, help="override n_splits")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--extra", action="store_true",
                    help="also time the other workloads (stderr lines)")
    ap.add_argument("--path", choices=("absorbed", "gqa", "expand", "projections",
                                       "moving-reference"),
                    default="absorbed",
                    help="absorbed MLA step (default), the GQLA per-group GQA path, or the "
                         "GQA path's cache expansion alone (a stderr-style JSON line)")
    ap.add_argument("--no-flush", action="store_true",
                    help="do not flush the last-level cache between steps")
    ap.add_argument("--flush", choices=("read", "write"), default="read",
                    help="how the last-level cache is flushed between steps (read: sum a "
                         "1 GiB buffer; write: fill it)")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the measured HBM-read and MFMA peaks (libmla_calib.so)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration)")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 28   # 1 GiB of fp32
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n}))


def measured_peaks():
    """The machine's own roofline denominators from libmla_calib.so: a pure HBM read stream
    (every workgroup its own contiguous span, 1 KB per load instruction, non-temporal; the
    best of 5 launches over a 604 MB buffer) and a dense bf16 v_mfma_f32_32x32x16 loop (the
    best of 5), both timed with HIP events on the launch stream."""
    import ctypes
    import torch
    from head_latent_attention_02_amd.build import CALIB_LIB_PATH
    if not os.path.exists(CALIB_LIB_PATH):
        return None
    lib = ctypes.CDLL(CALIB_LIB_PATH)
    lib.calib_hbm_read_bytes.restype = ctypes.c_int64
    lib.calib_hbm_read_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.calib_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_void_p, ctypes.c_void_p]
    lib.calib_mfma_bf16_flops.restype = ctypes.c_int64
    lib.calib_mfma_bf16_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.calib_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                    ctypes.c_void_p]
    st = torch.cuda.current_stream()
    n_wg, tiles = 256, 64
    nbytes = lib.calib_hbm_read_bytes(n_wg, tiles)
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty(n_wg * 256, dtype=torch.int32, device="cuda")
    flush = _flusher()

    def best_ms(launch, reps=5):
        out = []
        for _ in range(reps + 1):
            flush()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            if launch() != 0:
                raise RuntimeError("calibration launch failed")
            b.record(st)
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b))
        return min(out[1:])

    hbm_ms = best_ms(lambda: lib.calib_hbm_read(buf.data_ptr(), n_wg, tiles, sink.data_ptr(),
                                                st.cuda_stream))
    del buf
    m_wg, iters = 512, 20000
    fsink = torch.empty(m_wg * 256, dtype=torch.float32, device="cuda")
    mfma_ms = best_ms(lambda: lib.calib_mfma_bf16(m_wg, iters, fsink.data_ptr(),
                                                  st.cuda_stream))
    return {"hbm_read_GBs": nbytes / (hbm_ms * 1e-3) / 1e9,
            "mfma_bf16_TFLOPs": lib.calib_mfma_bf16_flops(m_wg, iters) / (mfma_ms * 1e-3) / 1e12,
            "source": "libmla_calib.so (calib/calib.hip): 604 MB non-temporal read stream, "
                      "dense 32x32x16 bf16 MFMA loop; best of 5 launches each"}


def host_info():
    """CPU model and the BLAS library numpy uses, for the CPU baseline's record."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:
        pass
    return model, blas


def cpu_baseline(inp, seconds):
    """Time the oracle on whole (sequence, head) rows of the workload until ~seconds."""
    import numpy as np
    from oracle import mla as ref
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count()
    c = inp.cfg
    pool = inp.pool_view()
    done, t0 = 0, time.perf_counter()
    h = 0
    while True:
        ref.mla_decode_naive(inp.q, pool, inp.page_table, inp.ctx_lens, inp.w_uk, inp.w_uv,
                             c.scale, c.page_size, c.d_c, batches=[0], heads=[h])
        done += 1
        h = (h + 1) % c.n_heads
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    per_row = el / done                     # one (sequence, head) row over T_0 tokens
    step_s = per_row * c.batch * c.n_heads * float(np.mean(inp.ctx_lens)) / float(inp.ctx_lens[0])
    model, blas = host_info()
    return {"value": inp.total_tokens / step_s, "unit": "cached-latent-tokens/s",
            "cores": int(cores), "kind": "oracle", "cpu_model": model, "blas": blas,
            "sample": f"{done} (sequence 0, head) rows of {int(inp.ctx_lens[0])} tokens in "
                      f"{el:.1f} s, scaled to all {c.batch}x{c.n_heads} rows"}


FLUSH_BYTES = 1 << 30   # > the 256 MB Infinity Cache: every step starts from HBM
FLUSH_KIND = "read"     # set from --flush


def _flusher():
    """Evict the last-level cache between steps.  "read" sums a 1 GiB buffer: the cache then
    holds clean lines only.  "write" fills it instead, which leaves the cache full of dirty
    lines whose write-back lands inside the next timed step (measured: +0.41 ms on the
    8.9 GB GQA-path decode, 1.78 vs 1.37 ms)."""
    import torch
    buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    if FLUSH_KIND == "write":
        return lambda: buf.fill_(1.0)
    out = torch.empty((), dtype=torch.float32, device="cuda")
    return lambda: torch.sum(buf, dim=0, out=out)


def _stats(ms):
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return float(np.median(a)), float(np.percentile(a, 10)), float(np.percentile(a, 90))


def time_workload(name, steps, warmup, splits=None, flush=True):
    """Absorbed step a1 -> a2 -> a3 -> a4; HIP events between the kernels of every step,
    with the last-level cache flushed between steps (outside the events)."""
    import torch
    import head_latent_attention_02_amd as mla
    from workloads import get_config, make_inputs
    from workloads.device import DeviceInputs

    cfg = get_config(name)
    if splits:
        cfg = cfg.with_(n_splits=splits)
    inp = make_inputs(cfg)
    d = DeviceInputs(inp)
    sh = d.shape
    op = d.o_part_view(cfg.d_c)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    fl = _flusher() if flush else (lambda: None)

    def whole_step():
        mla.mla_decode_step(sh, d.q, d.w_uk, d.w_uv, d.pool, d.page_table, d.ctx_lens,
                            d.q_abs, op, d.lse_part, d.o_lat, d.out, d.lse, stream=sp)

    def split_step(ev):
        ev[0].record(stream)
        mla.mla_absorb_q(sh, d.q, d.w_uk, d.q_abs, stream=sp)
        ev[1].record(stream)
        mla.mla_decode_absorbed(sh, d.q_abs, d.pool, d.page_table, d.ctx_lens, op,
                                d.lse_part, stream=sp)
        ev[2].record(stream)
        mla.mla_splitkv_combine(sh, cfg.d_c, op, d.lse_part, d.o_lat, d.lse, stream=sp)
        ev[3].record(stream)
        mla.mla_out_uv(sh, d.o_lat, d.w_uv, d.out, stream=sp)
        ev[4].record(stream)

    for _ in range(warmup):
        fl()
        whole_step()
    # The whole step (one library call, four kernels) with events only around it, and,
    # interleaved with it so both see the same clocks, the same step through the four
    # entry points with an event between kernels.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    evk = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fl()
        evs[i][0].record(stream)
        whole_step()
        evs[i][1].record(stream)
        fl()
        split_step(evk[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {"step": [e[0].elapsed_time(e[1]) for e in evs]}
    ms.update({"step_with_kernel_events": [e[0].elapsed_time(e[4]) for e in evk],
               "absorb_q": [e[0].elapsed_time(e[1]) for e in evk],
               "decode": [e[1].elapsed_time(e[2]) for e in evk],
               "combine": [e[2].elapsed_time(e[3]) for e in evk],
               "out_uv": [e[3].elapsed_time(e[4]) for e in evk]})
    return inp, d, ms, wall / steps * 1e3


def time_gqa_path(name, steps, warmup, flush=True):
    """GQA path on the expanded per-group cache: a5 -> a3 (a6 runs once, untimed)."""
    import torch
    import head_latent_attention_02_amd as mla
    from workloads import get_config, make_inputs
    from workloads.device import DeviceInputs

    cfg = get_config(name)
    inp = make_inputs(cfg)
    d = DeviceInputs(inp)
    sh = d.shape
    n = inp.num_pages
    k = torch.empty(n, cfg.page_size, cfg.n_wheads, cfg.d_nope, dtype=torch.bfloat16,
                    device="cuda")
    v = torch.empty(n, cfg.page_size, cfg.n_wheads, cfg.d_v, dtype=torch.bfloat16,
                    device="cuda")
    kr = torch.empty(n, cfg.page_size, cfg.d_rope, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    mla.gqla_expand_cache(sh, d.pool, d.w_uk, d.w_uv, k, v, kr, stream=sp)
    del d.pool
    op = d.o_part_view(cfg.d_v)
    fl = _flusher() if flush else (lambda: None)

    def split_step(ev):
        ev[0].record(stream)
        mla.gqla_decode_gqa(sh, d.q, k, v, kr, d.page_table, d.ctx_lens, op, d.lse_part,
                            stream=sp)
        ev[1].record(stream)
        mla.mla_splitkv_combine(sh, cfg.d_v, op, d.lse_part, d.out, d.lse, stream=sp)
        ev[2].record(stream)

    def whole_step(ev):
        ev[0].record(stream)
        mla.gqla_decode_step(sh, d.q, k, v, kr, d.page_table, d.ctx_lens, op, d.lse_part,
                             d.out, d.lse, stream=sp)
        ev[1].record(stream)

    for _ in range(warmup):
        fl()
        whole_step([torch.cuda.Event(), torch.cuda.Event()])
    # The whole step with events only around it, interleaved with the same step with an
    # event between its kernels (the decode kernel's time for the roofline).
    whole = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        fl()
        whole_step(whole[i])
        fl()
        split_step(evs[i])
    torch.cuda.synchronize()
    dec = _stats([e[0].elapsed_time(e[1]) for e in evs])[0]
    core, p10, p90 = _stats([e[0].elapsed_time(e[1]) for e in whole])
    bpt = mla.gqla_cache_scalars_per_token(sh) * 2
    return {"workload": name, "path": "gqa", "decode_ms": dec, "core_ms": core,
            "core_ms_p10_p90": [p10, p90],
            "tokens_per_s": inp.total_tokens / (core * 1e-3),
            "tokens": inp.total_tokens, "bytes_per_token": bpt,
            "decode_GBs": inp.total_tokens * bpt / (dec * 1e-3) / 1e9,
            "kernel": "mfma" if mla.gqla_decode_kernel_kind(sh) == 1 else "generic"}


def time_moving_reference(name, steps, warmup, flush=True):
    """The decode kernel's worst case: scores that climb on every tile of every chunk, so
    every row's softmax reference moves on every tile (workloads.gen.growing_score_inputs),
    timed beside the same kernel on the benign seeded workload."""
    import torch
    import head_latent_attention_02_amd as mla
    from workloads import get_config, make_inputs
    from workloads.device import DeviceInputs
    from workloads.gen import growing_score_inputs

    cfg = get_config(name)
    res = {"workload": name, "path": "absorbed decode, reference moving on every tile"}
    stream = torch.cuda.current_stream()
    fl = _flusher() if flush else (lambda: None)
    T = None
    for kind in ("benign", "moving"):
        if kind == "benign":
            inp = make_inputs(cfg)
        else:
            per_split = -(-T // cfg.n_splits)                     # ceil(T / S)
            chunk = -(-per_split // cfg.page_size) * cfg.page_size  # page-aligned chunk
            inp = growing_score_inputs(cfg, period_tokens=chunk)
        T = int(inp.ctx_lens[0])
        d = DeviceInputs(inp)
        op = d.o_part_view(cfg.d_c)
        mla.mla_absorb_q(d.shape, d.q, d.w_uk, d.q_abs)

        def run():
            mla.mla_decode_absorbed(d.shape, d.q_abs, d.pool, d.page_table, d.ctx_lens, op,
                                    d.lse_part, stream=stream.cuda_stream)
        for _ in range(warmup):
            fl()
            run()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            fl()
            evs[i][0].record(stream)
            run()
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        res[kind + "_decode_ms"] = _stats([e[0].elapsed_time(e[1]) for e in evs])[0]
        del d
        torch.cuda.empty_cache()
    res["ratio"] = res["moving_decode_ms"] / res["benign_decode_ms"]
    return res


def time_expand(name, steps, warmup, flush=True):
    """a6, the GQA path's set-up: the per-group K, V and shared RoPE-key cache built from the
    latent cache (every pool row, padding included), timed alone with events around it."""
    import torch
    import head_latent_attention_02_amd as mla
    from workloads import get_config, make_inputs
    from workloads.device import DeviceInputs

    cfg = get_config(name)
    inp = make_inputs(cfg)
    d = DeviceInputs(inp)
    n = inp.num_pages
    k = torch.empty(n, cfg.page_size, cfg.n_wheads, cfg.d_nope, dtype=torch.bfloat16,
                    device="cuda")
    v = torch.empty(n, cfg.page_size, cfg.n_wheads, cfg.d_v, dtype=torch.bfloat16,
                    device="cuda")
    kr = torch.empty(n, cfg.page_size, cfg.d_rope, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    fl = _flusher() if flush else (lambda: None)

    def step():
        mla.gqla_expand_cache(d.shape, d.pool, d.w_uk, d.w_uv, k, v, kr,
                              stream=stream.cuda_stream)

    for _ in range(warmup):
        fl()
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        fl()
        evs[i][0].record(stream)
        step()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    ms, p10, p90 = _stats([e[0].elapsed_time(e[1]) for e in evs])
    rows = n * cfg.page_size
    wbytes = rows * (cfg.n_wheads * (cfg.d_nope + cfg.d_v) + cfg.d_rope) * 2
    rbytes = rows * cfg.D * 2
    flops = 2.0 * rows * cfg.n_wheads * (cfg.d_nope + cfg.d_v) * cfg.d_c
    return {"workload": name, "path": "expand", "ms": ms, "ms_p10_p90": [p10, p90],
            "rows": rows, "bytes_written": wbytes, "bytes_read": rbytes,
            "write_GBs": wbytes / (ms * 1e-3) / 1e9,
            "hbm_GBs": (wbytes + rbytes) / (ms * 1e-3) / 1e9,
            "mfma_TFLOPs": flops / (ms * 1e-3) / 1e12}


def time_projections(name, steps, warmup, d_model=5120, flush=True):
    """Offline absorption measured against the runtime steps it replaces, on the workload's
    batch: the query side as projection + a1 (W^Q then W_UK) versus the folded projection
    (W~^Q, no a1), and the output side as a4 + projection (W_UV then W^O) versus the folded
    projection (W~^O, no a4).  Each leg alone, events around it, cache flushed before it."""
    import torch
    import head_latent_attention_02_amd as mla
    from workloads import get_config, make_inputs, make_projection_inputs
    from workloads.device import DeviceInputs, to_dev

    cfg = get_config(name, ctx=("list", [64] * get_config(name).batch))
    inp = make_inputs(cfg)
    pr = make_projection_inputs(cfg, d_model)
    d = DeviceInputs(inp)
    sh = d.shape
    B, s_q, H = cfg.batch, cfg.s_q, cfg.n_heads
    x, w_q, w_o = (to_dev(a, "bf16") for a in (pr.x, pr.w_q, pr.w_o))
    bf = dict(dtype=torch.bfloat16, device="cuda")
    q = torch.empty(B, s_q, H, cfg.d_nope + cfg.d_rope, **bf)
    wqf = torch.empty(H, cfg.D, d_model, **bf)
    wof = torch.empty(d_model, H * cfg.d_c, **bf)
    y = torch.empty(B, s_q, d_model, dtype=torch.float32, device="cuda")
    d.o_lat.normal_()
    mla.mla_fold_q_weights(sh, d_model, w_q, d.w_uk, wqf)
    mla.mla_fold_o_weights(sh, d_model, w_o, d.w_uv, wof)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    fl = _flusher() if flush else (lambda: None)
    legs = {
        "q_unfolded": lambda: (mla.mla_project_q(sh, d_model, 1e4, x, w_q, d.ctx_lens, q,
                                                 stream=sp),
                               mla.mla_absorb_q(sh, q, d.w_uk, d.q_abs, stream=sp)),
        "q_folded": lambda: mla.mla_project_q_folded(sh, d_model, 1e4, x, wqf, d.ctx_lens,
                                                     d.q_abs, stream=sp),
        "o_unfolded": lambda: (mla.mla_out_uv(sh, d.o_lat, d.w_uv, d.out, stream=sp),
                               mla.mla_out_project(sh, d_model, d.out, w_o, y, stream=sp)),
        "o_folded": lambda: mla.mla_out_project_folded(sh, d_model, d.o_lat, wof, y,
                                                       stream=sp),
    }
    wbytes = {"q_unfolded": (w_q.numel() + d.w_uk.numel()) * 2, "q_folded": wqf.numel() * 2,
              "o_unfolded": (d.w_uv.numel() + w_o.numel()) * 2, "o_folded": wof.numel() * 2}
    res = {"workload": name, "path": "projections", "d_model": d_model, "tokens": B * s_q}
    for k, fn in legs.items():
        for _ in range(warmup):
            fl()
            fn()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            fl()
            evs[i][0].record(stream)
            fn()
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        ms = _stats([e[0].elapsed_time(e[1]) for e in evs])[0]
        res[k] = {"ms": ms, "weight_MB": wbytes[k] / 1e6,
                  "weight_GBs": wbytes[k] / (ms * 1e-3) / 1e9}
    return res


def time_append(name, steps, warmup, d_model=5120, flush=True):
    """Cache-append step (write side): the step's new tokens projected, rotated and
    written into the paged cache."""
    import torch
    import head_latent_attention_02_amd as mla
    from workloads import get_config, make_inputs, make_append_inputs
    from workloads.device import DeviceInputs, to_dev

    cfg = get_config(name)
    inp = make_inputs(cfg)
    ap = make_append_inputs(cfg, d_model=d_model)
    d = DeviceInputs(inp)
    h, w_dkv, w_kr = (to_dev(x, cfg.dtype) for x in (ap.h, ap.w_dkv, ap.w_kr))
    stream = torch.cuda.current_stream()
    fl = _flusher() if flush else (lambda: None)

    def step():
        mla.mla_cache_append(d.shape, d_model, 10000.0, h, w_dkv, w_kr, d.page_table,
                             d.ctx_lens, d.pool, stream=stream.cuda_stream)

    for _ in range(warmup):
        fl()
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        fl()
        evs[i][0].record(stream)
        step()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    ms = _stats([e[0].elapsed_time(e[1]) for e in evs])[0]
    wbytes = (cfg.d_c + cfg.d_rope) * d_model * (2 if cfg.dtype == "bf16" else 4)
    return {"workload": name, "path": "append", "d_model": d_model,
            "new_tokens": cfg.batch * cfg.s_q, "ms": ms,
            "weight_GBs": wbytes / (ms * 1e-3) / 1e9}


def main():
    args = parse()
    global FLUSH_KIND
    FLUSH_KIND = args.flush
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the "
              "decode path has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import head_latent_attention_02_amd as mla

    if args.path == "expand":
        name = args.workload if args.workload.startswith("gqla") else "gqla-b32-t65536"
        print(json.dumps(time_expand(name, args.steps, min(args.warmup, 20),
                                     flush=not args.no_flush)), flush=True)
        return
    if args.path == "moving-reference":
        for name in ("long-b4-t131072", "gqla-b32-t8192"):
            print(json.dumps(time_moving_reference(name, args.steps, min(args.warmup, 200),
                                                   flush=not args.no_flush)), flush=True)
        return
    if args.path == "projections":
        for name in ("long-b4-t131072", "dsv2-b16-t4096", "mtp-b64-ragged"):
            print(json.dumps(time_projections(name, args.steps, min(args.warmup, 20),
                                              flush=not args.no_flush)), flush=True)
        return
    if args.path == "gqa":
        g = time_gqa_path(args.workload, args.steps, args.warmup, flush=not args.no_flush)
        ach = g["decode_GBs"]
        print(json.dumps({
            "metric": "GQLA GQA-path decode cached tokens/s (expanded per-group cache), 1 GPU",
            "value": g["tokens_per_s"], "unit": "cached-tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": g["core_ms"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) latents expanded on the GPU, permuted page table)",
            "config": {"workload": args.workload, "path": "gqa", "kernel": g["kernel"],
                       "llc_flush_between_steps": not args.no_flush,
                       "llc_flush": args.flush},
            "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": ach / HBM_PEAK_GBS, "traffic": None,
                         "kernel": "gqla_decode_gqa", "kernel_ms": g["decode_ms"]}}),
              flush=True)
        return

    inp, d, ms, wall_ms = time_workload(args.workload, args.steps, args.warmup, args.splits,
                                        flush=not args.no_flush)
    ms_step, p10, p90 = _stats(ms["step"])
    dec_ms = _stats(ms["decode"])[0]
    c = inp.cfg
    tokens = inp.total_tokens
    dec_bytes = tokens * c.D * 2                                  # algorithmic cache bytes
    dec_flops = tokens * c.s_q * c.n_heads * (2 * c.D + 2 * c.d_c)
    achieved = dec_bytes / (dec_ms * 1e-3) / 1e9
    traffic, traffic_source = None, None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_sha") == kernel_hash() and tr.get("workload") == args.workload:
            traffic = tr.get("hbm_bytes_per_launch")
            # not measured in this run: read from the committed counter record, which holds
            # rocprofv3 FETCH_SIZE / WRITE_SIZE of the same kernel source on this workload
            traffic_source = (os.path.relpath(TRAFFIC_FILE, ROOT) + " (rocprofv3 FETCH_SIZE "
                              "and WRITE_SIZE taken on kernel source " + tr["kernel_sha"] + ")")
    peaks = None if args.no_calibration else measured_peaks()
    line = {
        "metric": "MLA decode cached-latent-tokens/s; % HBM-BW and % bf16 MFMA peak, 1 GPU",
        "value": tokens / (ms_step * 1e-3),
        "unit": "cached-latent-tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) latents, permuted page table)",
        "config": {"workload": args.workload, "batch": c.batch, "ctx": int(inp.ctx_lens[0]),
                   "s_q": c.s_q, "heads": c.n_heads, "d_c": c.d_c, "d_rope": c.d_rope,
                   "n_splits": d.shape.n_splits, "page_size": c.page_size,
                   "path": "absorbed", "kernel": "mfma" if mla.mla_decode_kernel_kind(d.shape)
                   == 1 else "generic", "llc_flush_between_steps": not args.no_flush,
                   "llc_flush": args.flush},
        "step_ms_p10_p90": [p10, p90],
        "kernel_ms": {k: _stats(v)[0] for k, v in ms.items() if k != "step"},
        # decode + combine from the pass with events between kernels
        "core_ms": _stats([a + b for a, b in zip(ms["decode"], ms["combine"])])[0],
        "wall_ms_per_step_incl_flushes_and_kernel_pass": wall_ms,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "traffic_source": traffic_source,
                     "kernel": "mla_decode_absorbed", "kernel_ms": dec_ms,
                     "mfma_tflops": dec_flops / (dec_ms * 1e-3) / 1e12,
                     "mfma_frac": dec_flops / (dec_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
    }
    if peaks:
        line["roofline"]["measured_peak"] = peaks
        line["roofline"]["frac_of_measured_hbm"] = achieved / peaks["hbm_read_GBs"]
        line["roofline"]["mfma_frac_of_measured"] = (
            dec_flops / (dec_ms * 1e-3) / 1e12 / peaks["mfma_bf16_TFLOPs"])
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    if args.extra:
        del d
        for name in ("dsv2-b16-t4096", "mtp-b64-ragged", "gqla-b32-t65536",
                     "gqla-mtp-b32-t65536"):
            i2, d2, ms2, _ = time_workload(name, args.steps, args.warmup,
                                           flush=not args.no_flush)
            st2, dm2 = _stats(ms2["step"])[0], _stats(ms2["decode"])[0]
            b2 = i2.total_tokens * i2.cfg.D * 2
            print(json.dumps({"workload": name, "path": "absorbed", "ms_per_step": st2,
                              "decode_ms": dm2,
                              "kernel_ms": {k: _stats(v)[0] for k, v in ms2.items()},
                              "tokens_per_s": i2.total_tokens / (st2 * 1e-3),
                              "decode_GBs": b2 / (dm2 * 1e-3) / 1e9}), file=sys.stderr,
                  flush=True)
            del d2
        for name in ("gqla-b32-t8192", "gqla-b32-t65536", "gqla-mtp-b32-t65536",
                     "gqla-shard-b32-t65536"):
            print(json.dumps(time_gqa_path(name, args.steps, args.warmup,
                                           flush=not args.no_flush)),
                  file=sys.stderr, flush=True)
        print(json.dumps(time_expand("gqla-b32-t65536", args.steps, min(args.warmup, 20),
                                     flush=not args.no_flush)), file=sys.stderr, flush=True)
        for name in ("long-b4-t131072", "gqla-b32-t8192"):
            print(json.dumps(time_moving_reference(name, args.steps, min(args.warmup, 200),
                                                   flush=not args.no_flush)),
                  file=sys.stderr, flush=True)
        for name in ("long-b4-t131072", "dsv2-b16-t4096"):
            print(json.dumps(time_projections(name, args.steps, min(args.warmup, 20),
                                              flush=not args.no_flush)), file=sys.stderr,
                  flush=True)
        for name in ("long-b4-t131072", "mtp-b64-ragged"):
            print(json.dumps(time_append(name, args.steps, args.warmup,
                                         flush=not args.no_flush)),
                  file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()
