"""Benchmark of the gated causal GQA attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  1. the 32768-token causal prompt of the 27B shape (batch 1, 24 query heads over 4 KV
     heads, head_dim 256, bf16, gated) in query blocks of q_block rows: kv_append of the
     block's K/V, then attn_prefill of the block;
  2. one head-chunked verify step of the 35B-A3B shape (batch 2, 16 query heads over 2 KV
     heads, 32 rows appended at KV offset 32768 with a broadcast additive tree mask):
     kv_append, then attn_decode (split-KV pass + merge).
Inputs are resident in HBM before timing starts.  Events on the stream the kernels run on
bracket the timed region; the prefill and decode parts of every step are timed separately.

value = prefill attention TFLOP/s over the 32k prompt (algorithmic flops: 4 * 256 per
admissible (head, row, key) triple, i.e. 4*256*24*32768*32769/2 = 1.3195e13 per prompt).
decode.value = KV GB/s of the verify step (K+V bytes read once per KV group + Q, gate,
out and mask bytes).  roofline = the attn_prefill pass (split kernel + merge) against the
dense bf16 MFMA peak.  cpu_baseline = the float64 oracle on a bounded sample of the same
prompt, on the host cores.
"""

import argparse
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


def _up(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def prefill_flops(Hq, N):
    return 4.0 * 256 * Hq * N * (N + 1) / 2


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--q-block", type=int, default=512)
    ap.add_argument("--seq", type=int, default=32768)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=96)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the path has no multi-GPU part"}))
        sys.exit(2)

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

    # ---- verify inputs (35B-A3B shape, 32 rows at offset 32768, broadcast additive mask)
    vB, vHq, vHkv, voff, vrows = 2, 16, 2, 32768, 32
    vrng = syn.streams(1004)
    vcap = voff + vrows
    vk = _up(syn.normal_bits(vrng["k"], (vB, vHkv, vcap, 256)), dev)
    vv = _up(syn.normal_bits(vrng["v"], (vB, vHkv, vcap, 256)), dev)
    vq = _up(syn.normal_bits(vrng["q"], (vB, vHq, vrows, 256)), dev)
    vg = _up(syn.normal_bits(vrng["gate"], (vB, vHq, vrows, 256)), dev)
    vmask = _up(syn.verify_mask(vrng["mask"], rows=vrows, kv_offset=voff, heads=1, kind="add"), dev)
    vk_new = vk[:, :, voff:].clone()
    vv_new = vv[:, :, voff:].clone()
    vout = torch.empty_like(vq)
    va = ga.plan_args(B=vB, Hq=vHq, Hkv=vHkv, rows=vrows, kv_offset=voff, mask_kind=2)
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
            ga.prefill(q[:, :, s:e], kc, vc, g[:, :, s:e], kv_offset=s, kv_len=e, out=out[:, :, s:e], workspace=ws)
            if per_call is not None:
                per_call[i][1].record(stream)

    def verify_pass():
        ga.kv_append(vk_new, vv_new, vk, vv, kv_offset=voff)
        ga.decode(vq, vk, vv, vg, kv_offset=voff, mask=vmask, out=vout, workspace=vws)

    for _ in range(args.warmup):
        prefill_pass()
        verify_pass()
    torch.cuda.synchronize(dev)

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    n_calls = len(plans)
    per_call = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(n_calls)]
                for _ in range(K)]
    torch.cuda.synchronize(dev)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for it in range(K):
        ev[it][0].record(stream)
        prefill_pass(per_call[it])
        ev[it][1].record(stream)
        verify_pass()
        ev[it][2].record(stream)
    end.record(stream)
    torch.cuda.synchronize(dev)
    total_ms = start.elapsed_time(end)
    pre_ms = [e[0].elapsed_time(e[1]) for e in ev]
    ver_ms = [e[1].elapsed_time(e[2]) for e in ev]
    call_ms = np.array([[pc[0].elapsed_time(pc[1]) for pc in step] for step in per_call])

    flops = prefill_flops(Hq, N)
    pre_tflops = flops / (np.mean(pre_ms) * 1e-3) / 1e12
    # per call: algorithmic flops of block i = 4*256*Hq*sum over its rows of (position + 1)
    call_flops = np.array([4.0 * 256 * Hq * sum(range(s + 1, min(s + qL, N) + 1)) for s in range(0, N, qL)])
    call_mean_ms = call_ms.mean(axis=0)
    achieved_tflops = float(call_flops.sum() / (call_mean_ms.sum() * 1e-3) / 1e12)

    kv_bytes = 2.0 * vB * vHkv * (voff + vrows) * 256 * 2
    io_bytes = 3.0 * vB * vHq * vrows * 256 * 2 + vrows * (voff + vrows) * 2
    ver_gbs = (kv_bytes + io_bytes) / (np.mean(ver_ms) * 1e-3) / 1e9

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
                               f"query blocks of {qL}; plus 35B-A3B-shape verify, batch 2, 16/2 heads, 32 rows at "
                               f"offset 32768, broadcast additive mask",
                   "seq_len": N, "q_block": qL, "global_batch": B},
        "prefill": {"ms": round(float(np.mean(pre_ms)), 4), "tflops": round(float(pre_tflops), 2),
                    "frac_of_peak": round(float(pre_tflops) / PEAK_BF16_TFLOPS, 4), "calls": n_calls,
                    "workspace_bytes": int(ws_need),
                    "plan_last_block": {kk: plans[-1][kk] for kk in ("variant_name", "n_splits", "keys_per_split",
                                                                     "n_row_tiles", "grid_blocks")}},
        "decode": {"metric": "verify KV GB/s (35B-A3B shape, 32 rows at offset 32768, MALL-warm)",
                   "value": round(float(ver_gbs), 1), "unit": "GB/s", "us": round(float(np.mean(ver_ms)) * 1e3, 2),
                   "frac_of_peak": round(float(ver_gbs) / PEAK_HBM_GBS, 4), "bytes": int(kv_bytes + io_bytes),
                   "plan": {kk: vplan[kk] for kk in ("variant_name", "n_splits", "keys_per_split", "n_head_chunks",
                                                     "grid_blocks")}},
        "roofline": {"bound": "mfma", "achieved": round(achieved_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved_tflops / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "attn_prefill pass (attn_fwd_kernel + merge_kernel when split)",
                     "avg_call_us": round(float(call_mean_ms.mean()) * 1e3, 2)},
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
