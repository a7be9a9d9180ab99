"""Benchmark: lightning-attention prefill at a million tokens, plus decode.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one prefill of the million-token workload (B=1, H=64,
N=1,048,576, d=128, bf16 inputs and output, block 64, fp32 state), i.e. all
of its kernels: decay-power table, chunk aggregates and chunk scan of the
heads that do not decay within a chunk, one output launch for every head
(the warm-start pass of the decaying heads beside the other heads' pass from
their chunk start states), and the decaying heads' final states copied out.  Inputs are synthetic (seeded,
generated on the device) and resident in HBM before timing starts.  Prints
ONE JSON line:

  value          whole-job prefill tokens/s (B*N / step time)
  roofline       the kernel that writes every output row (the dominant one;
                 all 64 heads of this workload take its warm-start part):
                 algorithmic bytes per launch (1024 B per head-token: q, k, v
                 read + o written, bf16) over its mean
                 duration from HIP events recorded around it on its own
                 stream, against 8 TB/s
  cpu_baseline   the fp64 oracle (plain-C recurrence) on a bounded sample of
                 the same workload, on this host's cores
  exact_path     the same step with every head on the exact chunked path
                 (LA_FLAG_EXACT: no warm start)
  depth_scaled   the same step with the decays of layers 0, 23, 46 and 69 of
                 a 70-layer stack (slopes scaled down linearly with depth):
                 deeper layers decay more slowly, so fewer heads take the
                 warm start
  backward       the backward pass of the same layer (dq, dk, dv from dout)
  epilogue_prologue  per-head RMSNorm + sigmoid gate of the output and SiLU
                 on one input, as their own passes over the same layer; the
                 prefill step with SiLU on q, k, v fused into its tile loads
                 (LA_FLAG_SILU_QKV) beside the step plus three SiLU passes;
                 and the step with the norm and gate fused into its output
                 kernels (lightning_attn_fwd_fused), with and without SiLU,
                 beside the same work as separate passes
  decode         256 sequences x 64 heads x d=128 decode step, 1000 in-place
                 steps timed as a whole: GB/s of state + token traffic; and
                 the same rows through a slot table over a 512-slot pool, and
                 those with SiLU, per-head RMSNorm and gate fused; and one
                 step of all 70 lightning layers of a model in one launch
                 (each layer its own state pool) against 70 launches, at 256
                 and 8 sequences per layer
  mfma           algorithmic MFMA fraction (2*b*d + 4*d^2 flop per
                 head-token at the block run) and the executed one (SQ_INSTS_MFMA
                 from the committed counter run, over this run's kernel time)

Only one GPU is used; --gpus > 1 exits with a message.
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

_ROOT = os.path.dirname(os.path.abspath(__file__))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
BYTES_PER_HT = 1024            # q, k, v read + o written, bf16, d = 128
FLOP_PER_MFMA = 32768          # one v_mfma_f32_32x32x16_bf16: 32 x 32 x 16 multiply-adds
COUNTERS_FILE = os.path.join(_ROOT, "profiles", "prefill_counters.json")


def flop_per_ht(block, d=128):
    """Algorithmic flops per head-token of the blockwise form at this block
    length: the causal half of the intra-block Q K^T and P V products (b d
    each) plus the inter-block Q S and the state update (2 d^2 each)."""
    return 2 * block * d + 4 * d * d


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def _hip():
    import torch
    lib = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


def decaying_heads(lam, chunk):
    """Which heads the library puts through its warm-start pass (bf16 inputs,
    block 64): those whose chunk-start state weighs at most 2^-30 of itself
    (lam^(r+1)) from row r = carry span on, with the span rounded up to whole
    64-token sub-tiles and at most half the chunk.  The kernels' rule,
    restated here for the byte count only."""
    out = []
    for x in lam:
        x = float(x)
        if x == 0.0:
            span = 0
        elif not (0.0 < x < 1.0):
            span = None
        else:
            t = 20.79441541679836 / -math.log(x)  # 30 ln 2 / -ln lam
            span = None if not t < 1e9 else ((math.ceil(t) + 63) // 64) * 64
        out.append(span is not None and 2 * span <= chunk)
    return out


def _code_text(path):
    """A source file without its comments, trailing blanks and empty lines."""
    s = open(path).read()
    s = re.sub(r"/\*.*?\*/", "", s, flags=re.S)
    s = re.sub(r"//[^\n]*", "", s)
    return "\n".join(l.rstrip() for l in s.splitlines() if l.strip())


def _src_hash():
    """Hash of the prefill kernels' code (comments left out): the committed
    counter record is used only while it matches."""
    h = hashlib.sha256()
    for name in ("la_output.hip", "la_state.hip", "la_device.h"):
        h.update(_code_text(os.path.join(_ROOT, "long_context_decayed_amd", "csrc", name)).encode())
    return h.hexdigest()[:16]


def _counters():
    """The committed rocprofv3 counter record of the prefill kernels, or None
    when it is absent or the kernel sources changed since it was taken."""
    try:
        rec = json.load(open(COUNTERS_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16") != _src_hash():
        log("counter record is stale (kernels changed since the counters were taken): traffic and "
            "executed-MFMA figures are null")
        return None
    return rec


def _device_info(dev):
    """What the numbers were measured on."""
    import torch
    import long_context_decayed_amd as la
    p = torch.cuda.get_device_properties(dev)
    return dict(name=p.name, arch=getattr(p, "gcnArchName", None), compute_units=p.multi_processor_count,
                memory_gib=round(p.total_memory / 2 ** 30, 1), hip_runtime=la.runtime_version(),
                torch=torch.__version__, torch_hip=torch.version.hip)


def bench_prefill(args, dev):
    import torch
    import long_context_decayed_amd as la
    from long_context_decayed_amd.inputs import decay_lambdas, decay_lambdas_depth, qkv_device

    B, H, N, d, block = 1, 64, args.tokens, 128, args.block
    log("generating inputs B=%d H=%d N=%d d=%d bf16 (seed 3)" % (B, H, N, d))
    q, k, v = qkv_device(B, H, N, d, seed=3, device=dev, slice_tokens=65536)
    lam = torch.from_numpy(decay_lambdas(H)).to(dev)
    out = torch.empty_like(q)
    kv_out = torch.empty((B, H, d, d), device=dev, dtype=torch.float32)
    chunk = la.chunk_for(B, H, N, block)
    warm_chunk = la.warm_chunk_for(B, H, N, block)
    ws = torch.empty(la.workspace_bytes(B, H, N, d, block), device=dev, dtype=torch.uint8)
    torch.cuda.synchronize()

    hip = _hip()
    evs = []
    for _ in range(2 * args.steps):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e)

    def step(i=None):
        ev = None if i is None else (evs[2 * i].value, evs[2 * i + 1].value)
        la.fwd(q, k, v, lam, kv_out=kv_out, block=block, out=out, workspace=ws, events=ev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("timing %d steps" % args.steps)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    kern = []
    for i in range(args.steps):
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), evs[2 * i], evs[2 * i + 1]) == 0
        kern.append(ms.value)
    for e in evs:
        hip.hipEventDestroy(e)
    kern_ms = sum(kern) / len(kern)
    ht = B * H * N
    fast = sum(decaying_heads(decay_lambdas(H), warm_chunk)) if block == 64 else H
    alg_bytes = BYTES_PER_HT * ht  # the timed kernel reads q, k, v and writes o of every head
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    rec = _counters() if block == 64 else None  # the counters were taken at block 64
    launch = (rec or {}).get("output_launch") or {}
    fpt = flop_per_ht(block, d)
    # Executed MFMA: the instructions the counter run saw per launch of the
    # same kernel (SQ_INSTS_MFMA, summed over waves) times the flops of one
    # 32x32x16 bf16 MFMA, over this run's own kernel time.
    exec_flop = launch.get("sq_insts_mfma") * FLOP_PER_MFMA if launch.get("sq_insts_mfma") else None
    mfma = dict(
        alg_flop_per_head_token=fpt,
        alg_flop_per_step=fpt * ht,
        alg_frac_of_step=fpt * ht / (ms_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        alg_frac_of_output_launch=fpt * ht / (kern_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        exec_flop_per_output_launch=exec_flop,
        exec_frac_of_output_launch=(exec_flop / (kern_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS) if exec_flop else None,
        shader_clock_ghz_under_load=launch.get("shader_clock_ghz"),
        peak_tflops=BF16_PEAK_TFLOPS,
        source="algorithmic: 2*b*d + 4*d^2 flop per head-token at the block run; executed: SQ_INSTS_MFMA x "
               "%d flop per launch from %s (null when stale)" % (FLOP_PER_MFMA, os.path.relpath(COUNTERS_FILE, _ROOT)),
    )
    res = dict(
        B=B, H=H, N=N, d=d, block=block, chunk=chunk, warm_chunk=warm_chunk, warm_start_heads=fast,
        ms_per_step=ms_step,
        tokens_per_s=B * N / (ms_step * 1e-3),
        output_kernel_ms=kern_ms,
        roofline=dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=achieved / HBM_PEAK_GBS, traffic=launch.get("bytes_per_launch")),
        step_hbm_frac=BYTES_PER_HT * ht / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        mfma_alg_frac=mfma["alg_frac_of_step"],
        mfma=mfma,
    )
    # What this GPU streams for the same traffic mix (3 reads + 1 write of
    # the layer's bf16 tensors, 1024 B per head-token) with a plain
    # elementwise kernel: torch.addcmul(q, k, v, out=o).  The 8 TB/s
    # datasheet figure is not reached by such a mix; this is the practical
    # ceiling the output launch is compared with beside the datasheet one.
    ms_mix = _time_ms(lambda: torch.addcmul(q, k, v, out=out), 3)
    mix_gbs = alg_bytes / (ms_mix * 1e-3) / 1e9
    res["stream_ceiling"] = dict(probe="torch.addcmul(q, k, v, out=o) over the layer's bf16 tensors",
                                 ms=ms_mix, achieved=mix_gbs, unit="GB/s",
                                 output_launch_frac_of_it=achieved / mix_gbs)
    if args.exact:
        # The same step with every head on the exact chunked path (LA_FLAG_EXACT:
        # chunk aggregates, scan, outputs from the chunk start states).  Its
        # roofline is taken over the whole step: the algorithmic bytes are the
        # same 1024 B per head-token; the aggregate pass's second read of k and
        # v shows up in `traffic` (all of the step's kernels, from the counters).
        ms_exact = _time_ms(lambda: la.fwd(q, k, v, lam, kv_out=kv_out, block=block, out=out, workspace=ws,
                                           exact=True), max(1, args.steps // 2))
        ach_x = alg_bytes / (ms_exact * 1e-3) / 1e9
        ex = (rec or {}).get("exact_step") or {}
        res["exact"] = dict(ms_per_step=ms_exact, tokens_per_s=B * N / (ms_exact * 1e-3),
                            roofline=dict(bound="hbm", achieved=ach_x, peak=HBM_PEAK_GBS, unit="GB/s",
                                          frac=ach_x / HBM_PEAK_GBS, traffic=ex.get("bytes_per_step"),
                                          scope="whole step (aggregate pass, scan, output pass)"))
    if args.depth:
        rows = []
        for layer in (0, 23, 46, 69):
            lam_np = decay_lambdas_depth(H, layer, 70)
            lam_l = torch.from_numpy(lam_np).to(dev)
            ms_l = _time_ms(lambda: la.fwd(q, k, v, lam_l, kv_out=kv_out, block=block, out=out, workspace=ws),
                            max(1, args.steps // 3))
            rows.append(dict(layer=layer, warm_start_heads=sum(decaying_heads(lam_np, warm_chunk)) if block == 64 else 0,
                             ms_per_step=ms_l, tokens_per_s=B * N / (ms_l * 1e-3)))
        res["depth_scaled"] = dict(n_layers=70, layers=rows,
                                   mean_ms_over_sampled_layers=sum(r["ms_per_step"] for r in rows) / len(rows))
    ms_silu = ms_norm_gate_fused = ms_layer_fused = None
    if args.fused and block == 64:
        # the same step on pre-activations, SiLU applied to the tiles as they load
        ms_silu = _time_ms(lambda: la.fwd(q, k, v, lam, kv_out=kv_out, block=block, out=out, workspace=ws,
                                          silu=True), max(1, args.steps // 2))
        # the output's per-head RMSNorm and sigmoid gate in the kernels that write
        # the output rows: core -> norm -> gate, and SiLU -> core -> norm -> gate
        gate = qkv_device(B, H, N, d, seed=6, device=dev, slice_tokens=65536)[0]
        gamma = torch.ones((H, d), device=dev, dtype=torch.float32)
        reps = max(1, args.steps // 2)
        ms_norm_gate_fused = _time_ms(lambda: la.fwd_fused(q, k, v, lam, gamma=gamma, gate=gate, kv_out=kv_out,
                                                           out=out, workspace=ws), reps)
        ms_layer_fused = _time_ms(lambda: la.fwd_fused(q, k, v, lam, gamma=gamma, gate=gate, kv_out=kv_out, out=out,
                                                       workspace=ws, silu=True), reps)
        del gate
    del ws
    if args.fused:
        ep = bench_norm_gate_silu(args, dev, out)
        if ms_silu is not None:
            ep["prefill_silu_fused_ms"] = ms_silu
            ep["prefill_plus_silu_passes_ms"] = ms_step + 3 * ep["silu_ms_per_tensor"]
            ep["prefill_norm_gate_fused_ms"] = ms_norm_gate_fused
            ep["prefill_plus_norm_gate_pass_ms"] = ms_step + ep["norm_gate_ms"]
            ep["layer_silu_core_norm_gate_fused_ms"] = ms_layer_fused
            ep["layer_silu_fused_core_plus_norm_gate_pass_ms"] = ms_silu + ep["norm_gate_ms"]
            ep["layer_all_separate_passes_ms"] = ms_step + 3 * ep["silu_ms_per_tensor"] + ep["norm_gate_ms"]
        res["epilogue_prologue"] = ep
    del out
    if args.backward:
        res["backward"] = bench_backward(args, dev, q, k, v, lam)
    sample = None
    if args.cpu_baseline:
        sample = (q, k, v, decay_lambdas(H))
    else:
        del q, k, v
    return res, sample


def _time_ms(fn, reps):
    import torch
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def bench_norm_gate_silu(args, dev, out):
    """The layer's elementwise steps either side of the core as the prefill's
    own passes, on the million-token output: per-head RMSNorm + sigmoid gate
    (o and gate read, y written) and SiLU in place on one input tensor."""
    import torch
    import long_context_decayed_amd as la
    from long_context_decayed_amd.inputs import qkv_device

    B, H, N, d = out.shape
    log("epilogue (norm + gate) and prologue (SiLU) passes on [%d, %d, %d, %d] bf16" % (B, H, N, d))
    gate = qkv_device(B, H, N, d, seed=6, device=dev, slice_tokens=65536)[0]
    gamma = torch.ones((H, d), device=dev, dtype=torch.float32)
    y = torch.empty_like(out)
    ms_ng = _time_ms(lambda: la.norm_gate(out, gamma=gamma, gate=gate, out=y), 5)
    ms_si = _time_ms(lambda: la.silu_(gate), 5)
    nbytes = out.numel() * 2
    del gate, y
    return dict(norm_gate_ms=ms_ng, norm_gate_gb_per_s=3 * nbytes / (ms_ng * 1e-3) / 1e9,
                silu_ms_per_tensor=ms_si, silu_gb_per_s=2 * nbytes / (ms_si * 1e-3) / 1e9)


def bench_backward(args, dev, q, k, v, lam):
    """The backward pass of the same layer (dq, dk, dv from dout; three
    prefill-shaped passes), timed with events on the current stream."""
    import torch
    import long_context_decayed_amd as la
    from long_context_decayed_amd.inputs import qkv_device

    B, H, N, d = q.shape
    log("backward: B=%d H=%d N=%d d=%d bf16" % (B, H, N, d))
    g = qkv_device(B, H, N, d, seed=5, device=dev, slice_tokens=65536)[0]
    ws = torch.empty(la.lib_bwd_workspace_bytes(B, H, N, d), device=dev, dtype=torch.uint8)
    outs = None
    for _ in range(max(1, args.warmup)):
        outs = la.bwd(q, k, v, lam, g, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    steps = max(1, args.steps // 2)
    e0.record()
    for _ in range(steps):
        outs = la.bwd(q, k, v, lam, g, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del outs, g, ws
    ht = B * H * N
    min_bytes = 7 * 2 * d * ht     # q, k, v, dout read + dq, dk, dv written, bf16
    gbs = min_bytes / (ms * 1e-3) / 1e9
    return dict(workload="backward of the same layer: dq, dk, dv (bf16) from dout, zero initial state and "
                         "final-state gradient", steps=steps, ms_per_step=ms, tokens_per_s=B * N / (ms * 1e-3),
                min_bytes_per_step=min_bytes, gb_per_s_vs_min_bytes=gbs, frac_hbm=gbs / HBM_PEAK_GBS)


def bench_decode(args, dev):
    import torch
    import long_context_decayed_amd as la
    from long_context_decayed_amd.inputs import decay_lambdas, qkv_device, state_device

    B, H, d, steps = 256, 64, 128, args.decode_steps
    log("decode: %d sequences x %d heads, d=%d, %d steps" % (B, H, d, steps))
    q, k, v = (t[:, :, 0].contiguous() for t in qkv_device(B, H, 1, d, seed=4, device=dev))
    s = state_device(B, H, d, seed=4, device=dev)
    lam = torch.from_numpy(decay_lambdas(H)).to(dev)
    o = torch.empty_like(q)
    for _ in range(10):
        la.decode_step(q, k, v, lam, kv_in=s, kv_out=s, out=o)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        la.decode_step(q, k, v, lam, kv_in=s, kv_out=s, out=o)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    per_step_bytes = 2 * B * H * d * d * 4 + 4 * B * H * d * 2
    gbs = per_step_bytes * steps / (ms * 1e-3) / 1e9
    res = dict(workload="decode 256 seq x H=64 x d=128, fp32 state, bf16 q/k/v/o", steps=steps,
               us_per_step=ms * 1e3 / steps, bytes_per_step=per_step_bytes, gb_per_s=gbs,
               frac_hbm=gbs / HBM_PEAK_GBS)
    # The same 1 GiB state swept in place by a plain elementwise kernel (read
    # and written once, as the decode step does): what this GPU streams for
    # that traffic, beside the datasheet's 8 TB/s.
    us_mix = _time_ms(lambda: s.mul_(1.0), 50) * 1e3
    mix_gbs = 2 * B * H * d * d * 4 / (us_mix * 1e-6) / 1e9
    res["stream_ceiling"] = dict(probe="torch: state.mul_(1.0) in place over the same fp32 state", us=us_mix,
                                 achieved=mix_gbs, unit="GB/s", decode_frac_of_it=gbs / mix_gbs)
    del s
    # Serving form: the same 256 rows over a pool of 512 state slots, through a
    # seeded random slot table (each row its own slot).
    pool = state_device(2 * B, H, d, seed=9, device=dev)
    g = torch.Generator().manual_seed(9)
    slots = torch.randperm(2 * B, generator=g)[:B].to(torch.int32).to(dev)
    for _ in range(10):
        la.decode_slots(q, k, v, lam, pool, slots, out=o)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        la.decode_slots(q, k, v, lam, pool, slots, out=o)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    gbs = (per_step_bytes + B * 4) * steps / (ms * 1e-3) / 1e9
    res["slots"] = dict(workload="the same 256 rows over a 512-slot state pool (seeded random slot table)",
                        us_per_step=ms * 1e3 / steps, gb_per_s=gbs, frac_hbm=gbs / HBM_PEAK_GBS)
    if args.fused:
        # the same, with SiLU on q, k, v, the per-head RMSNorm and the sigmoid gate fused in
        gate = q.clone()
        gamma = torch.ones((H, d), device=dev, dtype=torch.float32)
        ms = _time_ms(lambda: la.decode_fused(q, k, v, lam, pool, slots, silu=True, gamma=gamma, gate=gate, out=o),
                      steps)
        gbs = (per_step_bytes + B * 4 + B * H * d * 2) / (ms * 1e-3) / 1e9
        res["fused"] = dict(workload="the slot-table rows with SiLU on q, k, v, per-head RMSNorm and sigmoid gate "
                                     "fused", us_per_step=ms * 1e3, gb_per_s=gbs, frac_hbm=gbs / HBM_PEAK_GBS)
    return res


def bench_decode_layers(args, dev):
    """Decode over the 70 lightning layers of a model in one launch
    (lightning_attn_decode_layers: each layer its own state pool and the
    decays of its depth) against 70 single-layer launches of the same rows,
    at 256 and at 8 sequences per layer."""
    import torch
    import long_context_decayed_amd as la
    from long_context_decayed_amd.inputs import decay_lambdas_depth, qkv_device

    L, H, d = 70, 64, 128
    lam = torch.from_numpy(np.stack([decay_lambdas_depth(H, l, L) for l in range(L)]).astype(np.float32)).to(dev)
    rows = []
    for B in (256, 8):
        log("decode over %d layers x %d sequences x %d heads in one launch" % (L, B, H))
        q, k, v = (t.reshape(L, B, H, d).contiguous() for t in qkv_device(L * B, H, 1, d, seed=7, device=dev))
        states = torch.empty((L, B, H, d, d), device=dev, dtype=torch.float32)
        g = torch.Generator(device=dev).manual_seed(7)
        for l in range(L):  # N(0, 0.1^2) states, one layer at a time (a single draw would need 2x the memory)
            states[l].normal_(0.0, 0.1, generator=g)
        o = torch.empty_like(q)
        reps = max(3, args.decode_steps // 50)
        ms_one = _time_ms(lambda: la.decode_layers(q, k, v, lam, states, out=o), reps)
        lam_l = [lam[l].contiguous() for l in range(L)]

        def per_layer():
            for l in range(L):
                la.decode_fused(q[l], k[l], v[l], lam_l[l], states[l], silu=False, out=o[l])

        ms_sep = _time_ms(per_layer, reps)
        nbytes = L * (2 * B * H * d * d * 4 + 4 * B * H * d * 2)
        rows.append(dict(sequences_per_layer=B, layers=L, steps=reps, bytes_per_step=nbytes,
                         one_launch_us=ms_one * 1e3, one_launch_gb_per_s=nbytes / (ms_one * 1e-3) / 1e9,
                         one_launch_frac_hbm=nbytes / (ms_one * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         per_layer_launches_us=ms_sep * 1e3,
                         per_layer_launches_gb_per_s=nbytes / (ms_sep * 1e-3) / 1e9))
        del q, k, v, states, o
        torch.cuda.empty_cache()
    return dict(workload="one decode step of every lightning layer of a 70-layer stack (64 heads, d=128, fp32 "
                         "states, decays scaled down with depth), one launch vs 70 launches", rows=rows)


def cpu_baseline(sample, args):
    """The fp64 oracle recurrence, untouched, on a bounded sample of the
    workload: the first `heads` heads x first `tokens` tokens."""
    import numpy as np
    from oracle import crec

    q, k, v, lam = sample
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    threads = max(1, min(16, cores))
    heads = min(q.shape[1], 2 * threads)
    tokens = min(args.cpu_tokens, q.shape[2])
    hs = lambda t: t[0, :heads, :tokens].float().cpu().numpy()
    qs, ks, vs = hs(q), hs(k), hs(v)
    log("cpu baseline: oracle on %d heads x %d tokens, %d threads" % (heads, tokens, threads))
    t0 = time.perf_counter()
    crec.recurrent(qs, ks, vs, lam[:heads].astype(np.float64), o_range=(tokens, tokens), threads=threads,
                   want_state=False)
    dt = time.perf_counter() - t0
    ht_per_s = heads * tokens / dt
    return dict(value=ht_per_s / q.shape[1], unit="tokens/s", cores=threads, kind="oracle",
                sample="fp64 C recurrence over %d heads x %d tokens of the million-token workload "
                       "(%.1f s wall); value = head-tokens/s divided by the workload's 64 heads" % (
                           heads, tokens, dt))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--tokens", type=int, default=1 << 20)
    ap.add_argument("--block", type=int, default=64, choices=[64, 128, 256])
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-decode", dest="decode", action="store_false")
    ap.add_argument("--no-decode-layers", dest="decode_layers", action="store_false",
                    help="skip the 70-layer decode (one launch against one launch per layer)")
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--no-backward", dest="backward", action="store_false")
    ap.add_argument("--no-exact", dest="exact", action="store_false",
                    help="skip the step timed with every head on the exact chunked path")
    ap.add_argument("--no-depth", dest="depth", action="store_false",
                    help="skip the steps timed with the decays of deeper layers")
    ap.add_argument("--no-fused", dest="fused", action="store_false",
                    help="skip the SiLU / RMSNorm / gate measurements")
    ap.add_argument("--cpu-tokens", type=int, default=1 << 20)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB (a known-size "
                         "reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(sharding by sequence, head and batch is designed but not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: %d bytes read, %d bytes written" % (n, n))
        del src, dst
    prefill, sample = bench_prefill(args, dev)
    dec = bench_decode(args, dev) if args.decode else None
    if dec is not None and args.decode_layers:
        dec["layers"] = bench_decode_layers(args, dev)
    cpu = cpu_baseline(sample, args) if args.cpu_baseline else None
    line = {
        "metric": "lightning-attn fwd tokens/s + % bf16 MFMA peak at N=1M; decode GB/s % HBM peak",
        "value": prefill["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": prefill["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded device Gaussians / sqrt(d); per-head decays exp(-2^(-(8/H)(h+1))))",
        "config": {"workload": "lightning-attention prefill, one million-token layer: B=1 H=64 N=%d d=128 "
                               "bf16 in/out, block %d, chunk %d (warm start %d)" % (prefill["N"], prefill["block"],
                                                                                     prefill["chunk"], prefill["warm_chunk"]),
                   "batch": prefill["B"], "heads": prefill["H"], "seq_len": prefill["N"], "head_dim": 128,
                   "block": prefill["block"], "chunk": prefill["chunk"], "warm_chunk": prefill["warm_chunk"]},
        "roofline": prefill["roofline"],
        "stream_ceiling": prefill["stream_ceiling"],
        "output_kernel_ms": prefill["output_kernel_ms"],
        "warm_start_heads": prefill["warm_start_heads"],
        "step_hbm_frac": prefill["step_hbm_frac"],
        "mfma_alg_frac": prefill["mfma_alg_frac"],
        "mfma": prefill["mfma"],
        "exact_path": prefill.get("exact"),
        "depth_scaled": prefill.get("depth_scaled"),
        "backward": prefill.get("backward"),
        "epilogue_prologue": prefill.get("epilogue_prologue"),
        "cpu_baseline": cpu,
        "decode": dec,
        "device": _device_info(dev),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
