"""Benchmark of the gated causal GQA attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  1. prefill: the 32768-token causal prompt of the 27B shape (batch 1, 24 query heads over
     4 KV heads, head_dim 256, bf16, gated) in query blocks of q_block rows: kv_append of the
     block's K/V, then the block's attn_prefill, issued as its two launches (the main pass by
     attn_prefill_partials, then attn_merge when the keys are split) on one stream, so that
     events can bracket the main pass alone;
  2. decode: one decode row of the 35B-A3B shape (batch 2, 16 query heads over 2 KV heads)
     appended at KV offset 32768: kv_append, then attn_decode (split-KV pass + merge), on a
     cache chosen round-robin from enough distinct caches that the 256 MB Infinity Cache
     cannot hold them (cold KV reads);
  3. verify: 32 verify rows of the same shape at offset 32768 with a broadcast additive tree
     mask (the head-chunked verify): kv_append, then attn_decode.
Inputs are resident in HBM before timing starts.  Events on the stream the kernels run on
bracket each part of every step; torch's spin kernel holds the stream before the timed steps
so that the host is ahead of the device when they start.  A decode or verify call takes the
host (Python, ctypes) longer to issue than the GPU takes to run it, so their figures come from
a second measurement after the step loop: the spin kernel holds the stream while the host
enqueues 48 calls back to back (rotating over the cold caches), and events around those calls
time the device alone.  The same prompt is also run in query blocks of 128 (kv_append +
attn_prefill per block, enqueued under a hold, events around the loop) and reported beside the
512-row figure with its workspace bytes, and through the composed (materialised-score) route
at both block sizes for comparison (prefill_composed: time and transient workspace bytes).

value = prefill attention TFLOP/s over the 32k prompt (algorithmic flops: 4 * 256 per
admissible (head, row, key) triple: 4*256*24*32768*32769/2 = 1.3195e13 per prompt).
decode.value = KV GB/s of the one-row decode (K and V bytes read once per KV group + Q,
gate and out) over the device time of attn_decode (main pass + merge).  roofline = the dominant kernel, the main pass of a prefill block (event-timed
on its stream, averaged over the 64 blocks), against the dense bf16 MFMA peak;
decode.roofline = the decode call against HBM bandwidth.
cpu_baseline = the float64 oracle on a bounded sample of the same prompt, on the host cores.

`--copy-calibration BYTES` only copies a BYTES-sized device buffer once (for calibrating the
FETCH_SIZE / WRITE_SIZE counters against a known byte count) and exits.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)
MALL_BYTES = 256 << 20      # Infinity Cache


def _up(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def prefill_flops(Hq, N):
    return 4.0 * 256 * Hq * N * (N + 1) / 2


def measured_traffic():
    """Calibrated FETCH_SIZE + WRITE_SIZE bytes per prefill call and per decode call, from the
    counter record under profiles/, or None when the kernel sources have changed since."""
    path = os.path.join(ROOT, "profiles", "traffic_counters.json")
    try:
        rec = json.load(open(path))
        h = hashlib.sha256()
        for f in rec["sources"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
    except (OSError, KeyError, ValueError):
        return None
    return rec if h.hexdigest() == rec["sha256"] else None


def copy_calibration(nbytes):
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize(dev)
    dst.copy_(src)
    torch.cuda.synchronize(dev)
    print(json.dumps({"copy_calibration_bytes": int(nbytes)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--q-block", type=int, default=512)
    ap.add_argument("--seq", type=int, default=32768)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=480)
    ap.add_argument("--copy-calibration", type=int, default=0)
    ap.add_argument("--no-composed", action="store_true", help="skip the composed-route comparison")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the path has no multi-GPU part"}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import gqa_causal_attention_attn_amd as ga
    from synth import inputs as syn

    dev = torch.device("cuda:0")
    ga.lib()
    torch.cuda.set_device(dev)

    # ---- prompt inputs (27B shape)
    B, Hq, Hkv, N, qL = 1, 24, 4, args.seq, args.q_block
    rng = syn.streams(1003)
    t0 = time.time()
    host = {name: syn.normal_bits(rng[name], (B, H, N, 256))
            for name, H in (("q", Hq), ("k", Hkv), ("v", Hkv), ("gate", Hq))}
    q, k, v, g = (_up(host[name], dev) for name in ("q", "k", "v", "gate"))
    kc = torch.empty((B, Hkv, N, 256), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    out = torch.empty_like(q)
    ws_need = 0
    for s in range(0, N, qL):
        a = ga.plan_args(B=B, Hq=Hq, Hkv=Hkv, rows=min(qL, N - s), kv_offset=s, capacity=N)
        ws_need = max(ws_need, ga.workspace_bytes(a, 0))
    ws = torch.empty(max(ws_need, 16), dtype=torch.uint8, device=dev)
    plans = [ga.describe_plan(ga.plan_args(B=B, Hq=Hq, Hkv=Hkv, rows=min(qL, N - s), kv_offset=s, capacity=N), 0)
             for s in range(0, N, qL)]

    # ---- decode / verify inputs (35B-A3B shape at offset 32768)
    vB, vHq, vHkv, voff, vrows = 2, 16, 2, 32768, 32
    vrng = syn.streams(1004)
    vcap = voff + vrows
    cache_bytes = 2 * vB * vHkv * vcap * 256 * 2
    n_rot = max(2, int(np.ceil(4 * MALL_BYTES / cache_bytes)))  # >= 1 GiB of distinct caches
    kbits = syn.normal_bits(vrng["k"], (vB, vHkv, vcap, 256))
    vbits = syn.normal_bits(vrng["v"], (vB, vHkv, vcap, 256))
    caches = [(_up(kbits, dev), _up(vbits, dev)) for _ in range(n_rot)]
    k_new = caches[0][0][:, :, voff:].clone()
    v_new = caches[0][1][:, :, voff:].clone()
    dq = _up(syn.normal_bits(vrng["q"], (vB, vHq, 1, 256)), dev)
    dg = _up(syn.normal_bits(vrng["gate"], (vB, vHq, 1, 256)), dev)
    dout = torch.empty_like(dq)
    da = ga.plan_args(B=vB, Hq=vHq, Hkv=vHkv, rows=1, kv_offset=voff, capacity=vcap)
    dws = torch.empty(max(ga.workspace_bytes(da, 1), 16), dtype=torch.uint8, device=dev)
    dplan = ga.describe_plan(da, 1)
    vq = _up(syn.normal_bits(vrng["q"], (vB, vHq, vrows, 256)), dev)
    vg = _up(syn.normal_bits(vrng["gate"], (vB, vHq, vrows, 256)), dev)
    vmask = _up(syn.verify_mask(vrng["mask"], rows=vrows, kv_offset=voff, heads=1, kind="add"), dev)
    vout = torch.empty_like(vq)
    va = ga.plan_args(B=vB, Hq=vHq, Hkv=vHkv, rows=vrows, kv_offset=voff, capacity=vcap, mask_kind=2)
    vws = torch.empty(max(ga.workspace_bytes(va, 1), 16), dtype=torch.uint8, device=dev)
    vplan = ga.describe_plan(va, 1)
    torch.cuda.synchronize(dev)
    gen_s = time.time() - t0

    stream = torch.cuda.current_stream(dev)

    def prefill_pass(per_call=None):
        for i, s in enumerate(range(0, N, qL)):
            e = min(s + qL, N)
            ga.kv_append(k[:, :, s:e], v[:, :, s:e], kc, vc, kv_offset=s)
            if per_call is not None:
                per_call[i][0].record(stream)
            _, parts = ga.prefill_partials(q[:, :, s:e], kc, vc, g[:, :, s:e], kv_offset=s, kv_len=e,
                                           out=out[:, :, s:e], workspace=ws)
            if per_call is not None:
                per_call[i][1].record(stream)
            if parts is not None:
                ga.merge(parts[0], parts[1], g[:, :, s:e], out=out[:, :, s:e])

    def decode_pass(it, evs=None):
        kk_, vv_ = caches[it % n_rot]
        ga.kv_append(k_new[:, :, :1], v_new[:, :, :1], kk_, vv_, kv_offset=voff)
        if evs is not None:
            evs[0].record(stream)
        ga.decode(dq, kk_, vv_, dg, kv_offset=voff, out=dout, workspace=dws)
        if evs is not None:
            evs[1].record(stream)

    def verify_pass(it, evs=None):
        kk_, vv_ = caches[(it + n_rot // 2) % n_rot]
        ga.kv_append(k_new, v_new, kk_, vv_, kv_offset=voff)
        if evs is not None:
            evs[0].record(stream)
        ga.decode(vq, kk_, vv_, vg, kv_offset=voff, mask=vmask, out=vout, workspace=vws)
        if evs is not None:
            evs[1].record(stream)

    for w in range(args.warmup):
        prefill_pass()
        decode_pass(w)
        verify_pass(w)
    torch.cuda.synchronize(dev)

    # torch's spin kernel: cycles per millisecond, and the host time of one step, so that a hold
    # of the stream can let the host get ahead of the device before a timed region starts
    E = torch.cuda.Event
    c0_, c1_ = E(enable_timing=True), E(enable_timing=True)
    c0_.record(stream)
    torch.cuda._sleep(1_000_000)
    c1_.record(stream)
    torch.cuda.synchronize(dev)
    cyc_per_ms = 1_000_000 / c0_.elapsed_time(c1_)
    t0 = time.perf_counter()
    prefill_pass()
    decode_pass(0)
    verify_pass(0)
    step_host_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize(dev)

    K = args.steps
    ev = [[E(enable_timing=True) for _ in range(4)] for _ in range(K)]
    dec_ev = [[E(enable_timing=True), E(enable_timing=True)] for _ in range(K)]
    ver_ev = [[E(enable_timing=True), E(enable_timing=True)] for _ in range(K)]
    n_calls = len(plans)
    per_call = [[[E(enable_timing=True), E(enable_timing=True)] for _ in range(n_calls)] for _ in range(K)]
    torch.cuda.synchronize(dev)
    start = E(enable_timing=True)
    end = E(enable_timing=True)
    torch.cuda._sleep(int(min(step_host_ms * K, 2000.0) * cyc_per_ms))  # the host gets ahead
    start.record(stream)
    for it in range(K):
        ev[it][0].record(stream)
        prefill_pass(per_call[it])
        ev[it][1].record(stream)
        decode_pass(it, dec_ev[it])
        ev[it][2].record(stream)
        verify_pass(it, ver_ev[it])
        ev[it][3].record(stream)
    end.record(stream)
    torch.cuda.synchronize(dev)

    # Device time of the decode and verify calls.  One call through the Python binding costs the
    # host more than the GPU needs to run it, so events around single calls in the step loop
    # time the host.  Here a spin kernel holds the stream while the host enqueues n_dev calls
    # back to back, and events around them time the device alone.
    n_dev = 48
    held = [True]  # every timed batch was enqueued while the spin kernel still held the stream

    def device_timed(fn):
        t0 = time.perf_counter()
        fn(0)
        torch.cuda.synchronize(dev)
        host_s = (time.perf_counter() - t0)
        hold_ms = max(20.0, 3e3 * host_s * n_dev)
        out_us = []
        while len(out_us) < 3:
            torch.cuda._sleep(int(hold_ms * cyc_per_ms))
            s_, e_ = E(enable_timing=True), E(enable_timing=True)
            t1 = time.perf_counter()
            s_.record(stream)
            for i in range(n_dev):
                fn(i)
            e_.record(stream)
            enq_ms = (time.perf_counter() - t1) * 1e3
            torch.cuda.synchronize(dev)
            if enq_ms >= hold_ms and hold_ms < 2000.0:  # the host caught up: hold longer, time again
                hold_ms *= 4
                continue
            # (under a profiler that serialises dispatches the host always catches up; such a run
            # is flagged in device_timed and its figures are not device times)
            held[0] = held[0] and enq_ms < hold_ms
            out_us.append(s_.elapsed_time(e_) / n_dev * 1e3)
        return float(np.median(out_us))

    def dec_call(i, cold=True):
        kk_, vv_ = caches[i % n_rot] if cold else caches[0]
        ga.decode(dq, kk_, vv_, dg, kv_offset=voff, out=dout, workspace=dws)

    def dec_step(i):
        kk_, vv_ = caches[i % n_rot]
        ga.kv_append(k_new[:, :, :1], v_new[:, :, :1], kk_, vv_, kv_offset=voff)
        ga.decode(dq, kk_, vv_, dg, kv_offset=voff, out=dout, workspace=dws)

    def ver_call(i):
        kk_, vv_ = caches[i % n_rot]
        ga.decode(vq, kk_, vv_, vg, kv_offset=voff, mask=vmask, out=vout, workspace=vws)

    # the same 32k prompt in query blocks of the other size (qL 128 when the step uses 512):
    # kv_append + attn_prefill per block, events around the whole loop
    qL2 = 128 if qL != 128 else 512
    ws2_need = max(ga.workspace_bytes(ga.plan_args(B=B, Hq=Hq, Hkv=Hkv, rows=min(qL2, N - s), kv_offset=s, capacity=N),
                                      0) for s in range(0, N, qL2))
    ws2 = torch.empty(max(ws2_need, 16), dtype=torch.uint8, device=dev)

    def prefill_pass2():
        for s in range(0, N, qL2):
            e = min(s + qL2, N)
            ga.kv_append(k[:, :, s:e], v[:, :, s:e], kc, vc, kv_offset=s)
            ga.prefill(q[:, :, s:e], kc, vc, g[:, :, s:e], kv_offset=s, kv_len=e, out=out[:, :, s:e], workspace=ws2)

    t0 = time.perf_counter()
    prefill_pass2()
    torch.cuda.synchronize(dev)
    hold2_ms = max(20.0, 2e3 * (time.perf_counter() - t0))
    p2_ms = []
    while len(p2_ms) < max(2, K // 2):
        torch.cuda._sleep(int(hold2_ms * cyc_per_ms))  # the host enqueues the loop while the stream is held
        a2, b2 = E(enable_timing=True), E(enable_timing=True)
        t1 = time.perf_counter()
        a2.record(stream)
        prefill_pass2()
        b2.record(stream)
        enq_ms = (time.perf_counter() - t1) * 1e3
        torch.cuda.synchronize(dev)
        if enq_ms >= hold2_ms and hold2_ms < 2000.0:
            hold2_ms *= 4
            continue
        held[0] = held[0] and enq_ms < hold2_ms
        p2_ms.append(a2.elapsed_time(b2))

    # the composed (materialised-score) route on the same prompt, at both block sizes: the
    # comparison arm, kv_append + attn_prefill_composed per block, enqueued under a hold
    comp = {}
    if not args.no_composed:
        for qb_ in (512, 128):
            need = max(ga.workspace_bytes(ga.plan_args(B=B, Hq=Hq, Hkv=Hkv, rows=min(qb_, N - s), kv_offset=s,
                                                       capacity=N), 2) for s in range(0, N, qb_))
            wsc = torch.empty(need, dtype=torch.uint8, device=dev)

            def comp_pass():
                for s in range(0, N, qb_):
                    e = min(s + qb_, N)
                    ga.kv_append(k[:, :, s:e], v[:, :, s:e], kc, vc, kv_offset=s)
                    ga.prefill_composed(q[:, :, s:e], kc, vc, g[:, :, s:e], kv_offset=s, kv_len=e,
                                        out=out[:, :, s:e], workspace=wsc)

            comp_pass()
            torch.cuda.synchronize(dev)
            cms = []
            for _ in range(2):
                torch.cuda._sleep(int(50.0 * cyc_per_ms))
                a3, b3 = E(enable_timing=True), E(enable_timing=True)
                a3.record(stream)
                comp_pass()
                b3.record(stream)
                torch.cuda.synchronize(dev)
                cms.append(a3.elapsed_time(b3))
            # HBM bytes the route must move: per (head, row, key of the block's range, rounded
            # up to 32) the fp32 score written once and read twice and the 16-bit weight written
            # and read once (16 B), plus Q, gate and out (3 x 512 B per (head, row)) and K/V of
            # the range once per KV head
            cbytes = 0.0
            for s in range(0, N, qb_):
                e = min(s + qb_, N)
                kvp = -(-e // 32) * 32
                cbytes += B * Hq * (e - s) * (kvp * 16.0 + 3 * 512) + 2.0 * B * Hkv * e * 512
            cgbs = cbytes / (np.median(cms) * 1e-3) / 1e9
            comp[qb_] = {"ms": round(float(np.median(cms)), 3),
                         "tflops": round(float(prefill_flops(Hq, N) / (np.median(cms) * 1e-3) / 1e12), 2),
                         "workspace_bytes": int(need), "calls": len(range(0, N, qb_)),
                         "roofline": {"bound": "hbm", "achieved": round(float(cgbs), 1), "peak": PEAK_HBM_GBS,
                                      "unit": "GB/s", "frac": round(float(cgbs) / PEAK_HBM_GBS, 4),
                                      "bytes": int(cbytes)}}
            del wsc
            torch.cuda.empty_cache()

    # head dims 64 and 128 (their own fused pass, keys split where its grid is small): the same
    # 32k prompt shape in blocks of 512 rows, kv_append + attn_prefill, enqueued under a hold
    small = {}
    if not args.no_composed:
        for D_ in (128, 64):
            srng = syn.streams(1005 + D_)
            sq, sk, sv, sg = (_up(syn.normal_bits(srng[nm], (B, H, N, D_)), dev)
                              for nm, H in (("q", Hq), ("k", Hkv), ("v", Hkv), ("gate", Hq)))
            skc = torch.empty((B, Hkv, N, D_), dtype=torch.bfloat16, device=dev)
            svc = torch.empty_like(skc)
            sout = torch.empty_like(sq)
            sneed = max(ga.workspace_bytes(ga.plan_args(B=B, Hq=Hq, Hkv=Hkv, rows=min(qL, N - s), kv_offset=s, D=D_))
                        for s in range(0, N, qL))
            sws = torch.empty(max(sneed, 16), dtype=torch.uint8, device=dev)

            def small_pass():
                for s in range(0, N, qL):
                    e = min(s + qL, N)
                    ga.kv_append(sk[:, :, s:e], sv[:, :, s:e], skc, svc, kv_offset=s)
                    ga.prefill(sq[:, :, s:e], skc, svc, sg[:, :, s:e], kv_offset=s, kv_len=e, out=sout[:, :, s:e],
                               workspace=sws)

            small_pass()
            torch.cuda.synchronize(dev)
            sms = []
            for _ in range(2):
                torch.cuda._sleep(int(50.0 * cyc_per_ms))
                a4, b4 = E(enable_timing=True), E(enable_timing=True)
                a4.record(stream)
                small_pass()
                b4.record(stream)
                torch.cuda.synchronize(dev)
                sms.append(a4.elapsed_time(b4))
            sflops = 4.0 * D_ * Hq * N * (N + 1) / 2
            stf = sflops / (np.median(sms) * 1e-3) / 1e12
            small[D_] = {"ms": round(float(np.median(sms)), 3), "tflops": round(float(stf), 2),
                         "frac_of_peak": round(float(stf) / PEAK_BF16_TFLOPS, 4)}
            del sq, sk, sv, sg, skc, svc, sout, sws
            torch.cuda.empty_cache()

    dec_dev_us = device_timed(dec_call)
    warm_dev_us = device_timed(lambda i: dec_call(i, cold=False))
    dec_step_us = device_timed(dec_step)
    ver_dev_us = device_timed(ver_call)

    total_ms = start.elapsed_time(end)
    pre_ms = [e[0].elapsed_time(e[1]) for e in ev]
    call_ms = np.array([[pc[0].elapsed_time(pc[1]) for pc in step] for step in per_call])
    dec_us = np.array([e[0].elapsed_time(e[1]) for e in dec_ev]) * 1e3
    ver_us = np.array([e[0].elapsed_time(e[1]) for e in ver_ev]) * 1e3

    flops = prefill_flops(Hq, N)
    pre_tflops = flops / (np.mean(pre_ms) * 1e-3) / 1e12
    call_flops = np.array([4.0 * 256 * Hq * sum(range(s + 1, min(s + qL, N) + 1)) for s in range(0, N, qL)])
    call_mean_ms = call_ms.mean(axis=0)
    achieved_tflops = float(call_flops.sum() / (call_mean_ms.sum() * 1e-3) / 1e12)

    kv_len = voff + vrows  # the verify rows see the whole cache; the decode row reads voff + 1 keys
    dec_bytes = 2.0 * vB * vHkv * (voff + 1) * 256 * 2 + 3.0 * vB * vHq * 1 * 256 * 2
    dec_gbs = dec_bytes / (dec_dev_us * 1e-6) / 1e9
    warm_gbs = dec_bytes / (warm_dev_us * 1e-6) / 1e9
    ver_bytes = 2.0 * vB * vHkv * kv_len * 256 * 2 + 3.0 * vB * vHq * vrows * 256 * 2 + vrows * kv_len * 2
    ver_flops = 4.0 * 256 * vB * vHq * vrows * kv_len  # upper bound: every key admissible
    traffic = measured_traffic() if (N, qL) == (32768, 512) else None
    result = {
        "metric": "prefill attention TFLOP/s @32k (D256 GQA 24/4, bf16, gated); decode KV GB/s in 'decode'",
        "value": round(float(pre_tflops), 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 at the 27B and 35B-A3B attention shapes)",
        "config": {"workload": f"27B-shape causal prefill, batch 1, 24/4 heads, head_dim 256, {N} tokens in "
                               f"query blocks of {qL}; 35B-A3B-shape decode (1 row) and head-chunked verify "
                               f"(32 rows, broadcast additive mask), batch 2, 16/2 heads, at KV offset 32768",
                   "seq_len": N, "q_block": qL, "global_batch": B},
        "prefill": {"ms": round(float(np.mean(pre_ms)), 4), "tflops": round(float(pre_tflops), 2),
                    "frac_of_peak": round(float(pre_tflops) / PEAK_BF16_TFLOPS, 4), "calls": n_calls,
                    "workspace_bytes": int(ws_need),
                    "plan_last_block": {kk: plans[-1][kk] for kk in ("variant_name", "n_splits", "keys_per_split",
                                                                     "n_row_tiles", "grid_blocks")}},
        f"prefill_q_block_{qL2}": {"ms": round(float(np.median(p2_ms)), 4),
                                   "tflops": round(float(prefill_flops(Hq, N) / (np.median(p2_ms) * 1e-3) / 1e12), 2),
                                   "calls": len(range(0, N, qL2)), "workspace_bytes": int(ws2_need),
                                   "timing": "events around the block loop (kv_append + attn_prefill per block)"},
        "prefill_composed": {"route": "materialised scores: fp32 Q K^T, row softmax to 16-bit weights, P V + gate "
                                      "(attn_prefill_composed), kv_append per block; events around the block loop",
                             **{f"q_block_{kk}": vv for kk, vv in comp.items()}},
        "prefill_small_head_dims": {"route": "fused pass for head dims 64 and 128 (one wavefront per 32 rows of a "
                                             "head, two heads of a group sharing K/V tiles, keys split when "
                                             "the grid is small, then the merge), "
                                             "24/4 heads, same prompt and blocks",
                                    **{f"head_dim_{kk}": vv for kk, vv in small.items()}},
        "decode": {"metric": "decode KV GB/s (35B-A3B shape, batch 2, 1 row at offset 32768, cold KV; "
                             "device time of attn_decode: main pass + merge)",
                   "value": round(float(dec_gbs), 1), "unit": "GB/s", "us": round(dec_dev_us, 2),
                   "bytes": int(dec_bytes), "distinct_caches": n_rot,
                   "step_with_append_us": round(dec_step_us, 2), "device_timed": held[0],
                   "host_bound_call_us": round(float(np.median(dec_us)), 2),
                   "mall_warm_gbs": round(float(warm_gbs), 1), "mall_warm_us": round(warm_dev_us, 2),
                   "roofline": {"bound": "hbm", "achieved": round(float(dec_gbs), 1), "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": round(float(dec_gbs) / PEAK_HBM_GBS, 4),
                                "traffic": traffic and traffic["decode_call_bytes"]},
                   "plan": {kk: dplan[kk] for kk in ("variant_name", "n_splits", "keys_per_split", "n_head_chunks",
                                                     "grid_blocks")}},
        "verify": {"metric": "head-chunked verify, 32 rows at offset 32768, additive mask (cold KV; device "
                             "time of attn_decode)",
                   "us": round(ver_dev_us, 2), "host_bound_call_us": round(float(np.median(ver_us)), 2),
                   "gbs": round(float(ver_bytes / (ver_dev_us * 1e-6) / 1e9), 1),
                   "tflops_upper": round(float(ver_flops / (ver_dev_us * 1e-6) / 1e12), 1),
                   "plan": {kk: vplan[kk] for kk in ("variant_name", "n_splits", "keys_per_split", "n_head_chunks",
                                                     "grid_blocks")}},
        "roofline": {"bound": "mfma", "achieved": round(achieved_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic and traffic.get("prefill_main_bytes"),
                     "kernel": "attn_fwd_kernel (main pass of a prefill block)",
                     "avg_launch_us": round(float(call_mean_ms.mean()) * 1e3, 2)},
        "setup_s": round(gen_s, 1),
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(host, args.cpu_sample_rows, N)
    print(json.dumps(result), flush=True)


def cpu_baseline(host, n_rows, N):
    """The float64 oracle on a bounded sample of the same prompt: n_rows query rows spread
    over the prompt, all 24 heads, each against its causal prefix; scaled to TFLOP/s."""
    from oracle import reference
    from synth import inputs as syn

    Hq, Hkv = 24, 4
    qb, kb, vb, gb = host["q"], host["k"], host["v"], host["gate"]
    rows = np.linspace(N // n_rows, N - 1, n_rows).astype(np.int64)
    k64, v64 = syn.widen(kb), syn.widen(vb)
    t0 = time.time()
    for r in rows:
        reference.attention(syn.widen(qb[:, :, r:r + 1]), k64, v64, syn.widen(gb[:, :, r:r + 1]), n_kv_heads=Hkv,
                            kv_offset=int(r), kv_len=int(r) + 1)
    dt = time.time() - t0
    flops = float(sum(4.0 * 256 * Hq * (int(r) + 1) for r in rows))
    cores = None
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads") or 0) for i in threadpool_info()) or None
    except Exception:  # threadpoolctl missing: fall back to the affinity mask
        pass
    if not cores:
        cores = len(os.sched_getaffinity(0))
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_rows} query rows x 24 heads of the 32768-token prompt, each against its causal prefix "
                      f"(float64 NumPy/BLAS), {dt:.1f} s"}


if __name__ == "__main__":
    main()
