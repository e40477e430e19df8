"""Benchmark of the gated causal GQA attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  1. prefill: the 32768-token causal prompt of the 27B shape (batch 1, 24 query heads over
     4 KV heads, head_dim 256, bf16, gated) in query blocks of q_block rows: kv_append of the
     first block's K/V, then per block its attn_prefill, issued as its two launches (the main
     pass by attn_prefill_partials, then attn_merge when the keys are split, carrying the next
     block's kv_append in the same launch; a kv_append of its own otherwise) on one stream, so
     that events can bracket the main pass alone;
  2. decode: the head-chunked verify workload of the 35B-A3B shape (batch 2, 16 query heads
     over 2 KV heads) at KV offset 32768 with one row and its broadcast additive mask holding
     -Inf entries: kv_append, then attn_decode, on a cache chosen round-robin from enough
     distinct caches that the 256 MB Infinity Cache cannot hold them (cold KV reads);
  3. verify: 32 rows of the same workload: kv_append, then attn_decode.
Inputs are resident in HBM before timing starts.  Events on the stream the kernels run on
bracket each part of every step; torch's spin kernel holds the stream before the timed steps
so that the host is ahead of the device when they start.

Beside the step (each figure enqueued while a spin kernel holds the stream, so events time the
device, not the host): the decode workload at rows 1, 4 and 32, offsets 32768 and 4097, bf16 and
fp16, cold and MALL-warm; the 27B decode at 4096 (rows 1 and 4); the 35B-A3B 8192-token prompt
with 10% near-tie rows; the 32k prompt in query blocks of 128, 1024 and 2048 (time, workspace
bytes, torch allocator peak); the composed (materialised-score) route at qL 512 and 128; head
dims 128 and 64 at qL 512 and 128; and two achievable-peak probes (libgqa_probes.so): a dense
bf16 MFMA loop with the shader clock it ran at, and a streaming HBM read.

Every sample's requested plan (rows, head chunks, splits, dtype, mask) is recorded beside the
plan the library resolved (attn_describe_plan); a resolved plan that differs from the request
stops the benchmark ("perf(qwen36): qualify M4 head-256 attention", review of the scheduler
benchmark: the effective attention policy and block size are recorded and checked).

value = prefill attention TFLOP/s over the 32k prompt (algorithmic flops: 4 * 256 per
admissible (head, row, key) triple: 4*256*24*32768*32769/2 = 1.3195e13 per prompt).
decode.value = KV GB/s of the one-row masked decode (K and V read once per KV group + Q, gate,
out and the mask row) over the device time of attn_decode (main pass + merge).
roofline = the dominant kernel, the main pass of a prefill block (event-timed on its stream,
averaged over the 64 blocks), against the dense bf16 MFMA peak; decode.roofline = the decode
call against HBM bandwidth.  cpu_baseline = the float64 oracle on a bounded sample of the same
prompt, on the host cores.

Modes: `--only NAME` runs one workload `--steps` times and prints a short line (for profiler
runs); `--probes` runs only the two probes; `--copy-calibration BYTES` copies a BYTES-sized device
buffer once (for calibrating FETCH_SIZE / WRITE_SIZE against a known byte count).
"""

import argparse
import ctypes as C
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
ONLY = ("prefill", "decode", "verify", "decode_f16", "verify_f16", "decode_27b", "prefill_8k", "prefill_d128",
        "prefill_d64")


def _up(bits, dev, dtype="bf16"):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)


def prefill_flops(Hq, N, D=256):
    return 4.0 * D * Hq * N * (N + 1) / 2


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


class Timer:
    """Device time of enqueued work: a spin kernel holds the stream while the host enqueues the
    calls, so events around them time the device alone (a call through the Python binding can
    take the host longer than the GPU needs for it)."""

    def __init__(self, dev):
        self.dev = dev
        self.stream = torch.cuda.current_stream(dev)
        E = torch.cuda.Event
        a, b = E(enable_timing=True), E(enable_timing=True)
        a.record(self.stream)
        torch.cuda._sleep(1_000_000)
        b.record(self.stream)
        torch.cuda.synchronize(dev)
        self.cyc_per_ms = 1_000_000 / a.elapsed_time(b)
        self.held = True  # every timed batch was enqueued while the spin kernel still held the stream

    def hold(self, ms):
        torch.cuda._sleep(int(ms * self.cyc_per_ms))

    def time(self, fn, n_inner=1, reps=3):
        """Median device ms of one fn(i) over reps batches of n_inner back-to-back calls."""
        t0 = time.perf_counter()
        for i in range(n_inner):
            fn(i)
        torch.cuda.synchronize(self.dev)
        hold_ms = max(20.0, 3e3 * (time.perf_counter() - t0))
        out = []
        while len(out) < reps:
            self.hold(hold_ms)
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t1 = time.perf_counter()
            s.record(self.stream)
            for i in range(n_inner):
                fn(i)
            e.record(self.stream)
            enq_ms = (time.perf_counter() - t1) * 1e3
            torch.cuda.synchronize(self.dev)
            if enq_ms >= hold_ms and hold_ms < 4000.0:  # the host caught up: hold longer, time again
                hold_ms *= 4
                continue
            # (under a profiler that serialises dispatches the host always catches up; such a run
            # is flagged in device_timed and its figures are not device times)
            self.held = self.held and enq_ms < hold_ms
            out.append(s.elapsed_time(e) / n_inner)
        return float(np.median(out))


class Plans:
    """Requested plan beside the resolved one for every sample; a mismatch stops the run."""

    KEYS = ("variant_name", "n_splits", "partial_kind", "keys_per_split", "n_head_chunks", "chunk_sizes",
            "waves_per_block", "n_row_tiles", "grid_blocks", "carry_blocks", "workspace_bytes")

    def __init__(self, ga):
        self.ga = ga
        self.samples = []

    def check(self, name, *, op, B, Hq, Hkv, rows, kv_offset, D=256, dtype="bf16", mask_kind=0, head_chunk=0,
              n_splits=0, workspace=None, Hm=1):
        ga = self.ga
        a = ga.plan_args(B=B, Hq=Hq, Hkv=Hkv, rows=rows, kv_offset=kv_offset, D=D, dtype=dtype, mask_kind=mask_kind,
                         head_chunk=head_chunk, n_splits=n_splits, Hm=Hm)
        d = ga.describe_plan(a, op)
        req = {"op": {0: "prefill", 1: "decode"}[op], "B": B, "Hq": Hq, "Hkv": Hkv, "rows": rows,
               "kv_offset": kv_offset, "head_dim": D, "dtype": dtype,
               "mask": {0: "none", 1: "bool", 2: "add16", 3: "add32"}[mask_kind], "mask_heads": Hm,
               "head_chunk": "policy" if head_chunk == 0 else head_chunk,
               "n_splits": "auto" if n_splits == 0 else n_splits}
        res = {k: d[k] for k in self.KEYS}
        G = Hq // Hkv
        problems = []
        name_v = d["variant_name"]
        if f"_{dtype}_" not in name_v + "_":
            problems.append("dtype")
        want_mask = {0: None, 1: "maskbool", 2: "maskadd", 3: "maskf32"}[mask_kind]
        if (want_mask is None) != ("mask" not in name_v) or (want_mask and want_mask not in name_v):
            problems.append("mask kind")
        want_chunks = ga.head_chunk_plan(rows, Hq, Hkv) if head_chunk == 0 else (
            [head_chunk] * (G // head_chunk) + ([G % head_chunk] if G % head_chunk else []))
        if d["chunk_sizes"] != want_chunks:
            problems.append("head chunks")
        if (name_v.rsplit("_", 1)[-1] == f"d{D}") != (D != 256) or d["keys_per_tile"] != 8192 // D:
            problems.append("head dim route")
        if n_splits and d["n_splits"] > n_splits:
            problems.append("splits")
        kv_hi = kv_offset + rows
        if d["n_splits"] * d["keys_per_split"] < kv_hi or (d["n_splits"] - 1) * d["keys_per_split"] >= kv_hi:
            problems.append("key coverage")
        if d["workspace_bytes"] != ga.workspace_bytes(a, op):
            problems.append("workspace")
        if workspace is not None and d["workspace_bytes"] > workspace:
            problems.append("workspace allocated")
        if problems:
            print(json.dumps({"error": f"plan of {name} differs from the request: {problems}", "requested": req,
                              "resolved": res}), flush=True)
            sys.exit(3)
        self.samples.append({"sample": name, "requested": req, "resolved": res})
        return res


def probes(dev, timer):
    """Dense bf16 MFMA rate (and the shader clock it ran at) and a streaming HBM read."""
    from gqa_causal_attention_attn_amd import build as gbuild

    lib = C.CDLL(gbuild.PROBES_LIB)
    lib.gqa_probe_mfma.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p]
    lib.gqa_probe_read.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int, C.c_void_p]
    s = C.c_void_p(timer.stream.cuda_stream)
    res = {}
    # MFMA: 256 workgroups of 8 wavefronts (two a SIMD), 8 independent chains each
    blocks, waves, iters = 256, 8, 4000
    out = torch.empty(blocks * waves * 64, dtype=torch.float32, device=dev)
    clk = torch.empty(blocks * waves * 2, dtype=torch.int64, device=dev)
    assert lib.gqa_probe_mfma(out.data_ptr(), clk.data_ptr(), blocks, waves, iters, s) == 0
    ms = timer.time(lambda i: lib.gqa_probe_mfma(out.data_ptr(), clk.data_ptr(), blocks, waves, iters, s), 1, 5)
    flops = blocks * waves * iters * 8 * 32.0 * 32 * 16 * 2
    c = clk.view(-1, 2).cpu().numpy().astype(np.float64)
    ghz = float(np.median(c[:, 0] / c[:, 1]) * 0.1)
    tf = flops / (ms * 1e-3) / 1e12
    res["mfma_bf16"] = {"tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                        "shader_clock_ghz": round(ghz, 3),
                        "peak_at_that_clock_tflops": round(PEAK_BF16_TFLOPS * ghz / 2.4, 1),
                        "kernel": "8 chains of v_mfma_f32_32x32x16_bf16 per wavefront, 8 wavefronts x 256 workgroups"}
    # the same instruction with VALU work beside it (two wavefronts a SIMD, as in the main pass)
    lib.gqa_probe_mfma_mix.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_void_p]
    mix = {}
    for chains, nv, ex in ((1, 0, 0), (4, 0, 0), (1, 2, 0), (1, 4, 0), (4, 4, 0), (1, 1, 1), (1, 2, 1)):
        it = 2000
        fn = (lambda i: lib.gqa_probe_mfma_mix(out.data_ptr(), blocks, it, chains, nv, ex, s))
        assert fn(0) == 0
        ms = timer.time(fn, 1, 5)
        tf = blocks * 8 * it * 16 * 32768.0 / (ms * 1e-3) / 1e12
        mix[f"chains{chains}_{nv}{'exp' if ex else 'fma'}"] = round(tf, 1)
    res["mfma_bf16_with_valu"] = {"tflops": mix, "kernel": "16 v_mfma_f32_32x32x16_bf16 per round on 1 (dependent) or "
                                  "4 accumulators, each followed by 0-4 independent FMAs or v_exp_f32; 8 wavefronts x 256 "
                                  "workgroups"}
    # LDS read rate of the two read forms of the main pass, in bytes per CU per shader clock
    lib.gqa_probe_lds.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p]
    lds = {}
    for kind, name, per in ((0, "ds_read_b128", 1024), (1, "ds_read_b64_tr_b16 (V-operand lanes)", 512)):
        it = 20000
        fn = (lambda i: lib.gqa_probe_lds(out.data_ptr(), blocks, it, kind, s))
        assert fn(0) == 0
        ms = timer.time(fn, 1, 5)
        nbytes = blocks * 8 * 8 * it * per
        lds[name] = {"tbps": round(nbytes / (ms * 1e-3) / 1e12, 2),
                     "bytes_per_cu_per_clock": round(nbytes / blocks / (ms * 1e-3) / (ghz * 1e9), 1)}
    res["lds_read"] = {**lds, "clock_ghz_used": round(ghz, 3)}
    # streaming read, cold: the decode workload's bytes (134 MB, rotating over 8 distinct buffers
    # so the 256 MB Infinity Cache cannot hold them) and one 1 GiB buffer; 2048 workgroups
    sink = torch.empty(2048 * 256, dtype=torch.int32, device=dev)
    for label, nbytes, n_buf in (("134MB", 134_270_976 // 16 * 16, 8), ("1GiB", 1 << 30, 1)):
        srcs = [torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev) for _ in range(n_buf)]
        fn = (lambda i: lib.gqa_probe_read(srcs[i % n_buf].data_ptr(), nbytes, sink.data_ptr(), 2048, s))
        assert fn(0) == 0
        ms = timer.time(fn, n_buf, 5)
        res[f"hbm_read_{label}"] = {"gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                                    "frac_of_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                    "us": round(ms * 1e3, 2), "distinct_buffers": n_buf}
        del srcs
    # the decode main pass's key stream without its compute: one workgroup of four wavefronts
    # per CU, 32 KiB tiles, three in flight; the main pass's buffer-to-LDS loads with its
    # per-tile wait and barrier, without the barrier, and the same loads into registers
    lib.gqa_probe_tile_stream.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int, C.c_int, C.c_void_p]
    nbytes, n_buf = 134_270_976 // 16 * 16, 8
    srcs = [torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev) for _ in range(n_buf)]
    tiles = {}
    for blocks_ in (244, 256):
        for mode, name in ((0, "lds_dma_barrier"), (1, "lds_dma"), (2, "registers")):
            fn = (lambda i: lib.gqa_probe_tile_stream(srcs[i % n_buf].data_ptr(), nbytes, sink.data_ptr(), blocks_,
                                                      mode, s))
            assert fn(0) == 0
            ms = timer.time(fn, n_buf, 5)
            tiles[f"{name}_{blocks_}wg"] = {"gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "us": round(ms * 1e3, 2)}
    res["tile_stream_134MB"] = {**tiles, "kernel": "one 4-wavefront workgroup per CU streams its slice in 32 KiB "
                                "tiles, 3 in flight (8 distinct buffers, cold)"}
    del srcs
    del sink
    torch.cuda.empty_cache()
    return res


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
    ap.add_argument("--no-extras", action="store_true", help="the timed step only (no side figures)")
    ap.add_argument("--only", choices=ONLY, help="run one workload --steps times (profiler runs)")
    ap.add_argument("--probes", action="store_true", help="run the achievable-peak probes only")
    ap.add_argument("--q-block-sweep", action="store_true",
                    help="fused prompt time per query block, head dim, shape and prompt length only")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the path has no multi-GPU part "
                                   "(see the sharding notes of the design)"}), flush=True)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import gqa_causal_attention_attn_amd as ga
    from gqa_causal_attention_attn_amd import _abi
    from synth import inputs as syn

    dev = torch.device("cuda:0")
    ga.lib()
    torch.cuda.set_device(dev)
    timer = Timer(dev)
    stream = timer.stream
    E = torch.cuda.Event
    plans = Plans(ga)

    if args.probes:
        print(json.dumps({"probes": probes(dev, timer)}), flush=True)
        return
    if args.q_block_sweep:
        print(json.dumps({"q_block_sweep": q_block_sweep(ga, syn, dev, timer, plans)}), flush=True)
        return

    t_setup = time.time()
    # ---- the 32k prompt (27B shape)
    B, Hq, Hkv, N, qL = 1, 24, 4, args.seq, args.q_block
    need_prompt = args.only in (None, "prefill")
    if need_prompt:
        rng = syn.streams(1003)
        host = {name: syn.normal_bits(rng[name], (B, H, N, 256))
                for name, H in (("q", Hq), ("k", Hkv), ("v", Hkv), ("gate", Hq))}
        q, k, v, g = (_up(host[name], dev) for name in ("q", "k", "v", "gate"))
        kc = torch.empty((B, Hkv, N, 256), dtype=torch.bfloat16, device=dev)
        vc = torch.empty_like(kc)
        out = torch.empty_like(q)
        ws_need = max(ga.workspace_bytes(ga.plan_args(B=B, Hq=Hq, Hkv=Hkv, rows=min(qL, N - s), kv_offset=s,
                                                      capacity=N), 0) for s in range(0, N, qL))
        ws = torch.empty(max(ws_need, 16), dtype=torch.uint8, device=dev)
        block_plans = [plans.check(f"prefill_32k_qL{qL}_block{i}", op=0, B=B, Hq=Hq, Hkv=Hkv, rows=min(qL, N - s),
                                   kv_offset=s, workspace=ws.numel())
                       for i, s in enumerate(range(0, N, qL))]

    # ---- the decode / verify workload (35B-A3B shape, batch 2, 16/2 heads, masked) at offset off
    class DecodeSet:
        """Distinct caches (>= 1 GiB together, so the 256 MB Infinity Cache cannot hold them) and
        the inputs of the rows 1..32 of this workload."""

        def __init__(self, seed, B_, Hq_, Hkv_, off, rows_max, dtype, masked, mask_heads=1, mask_kind="add"):
            r = syn.streams(seed)
            self.B, self.Hq, self.Hkv, self.off, self.dtype, self.masked = B_, Hq_, Hkv_, off, dtype, masked
            self.mask_heads, self.mask_kind = mask_heads, mask_kind
            self.tag = "" if not masked or (mask_heads == 1 and mask_kind == "add") else (
                ("_full_head" if mask_heads > 1 else "") + ("_bool" if mask_kind == "bool" else ""))
            cap = off + rows_max
            cache_bytes = 2 * B_ * Hkv_ * cap * 256 * 2
            self.n_rot = max(2, int(np.ceil(4 * MALL_BYTES / cache_bytes)))
            kb = syn.normal_bits(r["k"], (B_, Hkv_, cap, 256), dtype)
            vb = syn.normal_bits(r["v"], (B_, Hkv_, cap, 256), dtype)
            self.caches = [(_up(kb, dev, dtype), _up(vb, dev, dtype)) for _ in range(self.n_rot)]
            self.k_new = self.caches[0][0][:, :, off:].clone()
            self.v_new = self.caches[0][1][:, :, off:].clone()
            self.q = _up(syn.normal_bits(r["q"], (B_, Hq_, rows_max, 256), dtype), dev, dtype)
            self.g = _up(syn.normal_bits(r["gate"], (B_, Hq_, rows_max, 256), dtype), dev, dtype)
            self.mask = {}
            self.out = {}
            self.ws = {}
            self.plans = {}
            self.mrng = r["mask"]

        def prep(self, rows, name):
            if rows in self.out:
                return self.plans[rows]
            if self.masked:
                mb = syn.verify_mask(self.mrng, rows=rows, kv_offset=self.off, heads=self.mask_heads,
                                     kind=self.mask_kind, dtype=self.dtype)
                self.mask[rows] = (_up(mb, dev, self.dtype) if self.mask_kind == "add"
                                   else torch.from_numpy(mb).to(dev))
            self.out[rows] = torch.empty((self.B, self.Hq, rows, 256), dtype=self.q.dtype, device=dev)
            mk = 0 if not self.masked else 2 if self.mask_kind == "add" else 1
            res = plans.check(name, op=1, B=self.B, Hq=self.Hq, Hkv=self.Hkv, rows=rows, kv_offset=self.off,
                              dtype=self.dtype, mask_kind=mk, Hm=self.mask_heads)
            self.ws[rows] = torch.empty(max(res["workspace_bytes"], 16), dtype=torch.uint8, device=dev)
            self.plans[rows] = res
            return res

        def call(self, rows, i, cold=True, append=False):
            kk_, vv_ = self.caches[i % self.n_rot] if cold else self.caches[0]
            if append:
                ga.kv_append(self.k_new[:, :, :rows], self.v_new[:, :, :rows], kk_, vv_, kv_offset=self.off)
            ga.decode(self.q[:, :, :rows], kk_, vv_, self.g[:, :, :rows], kv_offset=self.off,
                      mask=self.mask.get(rows), out=self.out[rows], workspace=self.ws[rows])

        def bytes(self, rows):
            kv = self.off + rows
            mask = self.mask_heads * rows * kv * (2 if self.mask_kind == "add" else 1) if self.masked else 0
            return 2.0 * self.B * self.Hkv * kv * 256 * 2 + 3.0 * self.B * self.Hq * rows * 256 * 2 + mask

    need_dec = args.only in (None, "decode", "verify")
    if need_dec:
        dset = DecodeSet(1004, 2, 16, 2, 32768, 32, "bf16", True)
        dplan = dset.prep(1, "decode_35b_off32768_rows1_bf16")
        vplan = dset.prep(32, "verify_35b_off32768_rows32_bf16")
    setup_s = time.time() - t_setup

    spaces = [ws, torch.empty_like(ws)] if need_prompt else None

    def prefill_pass(per_call=None):
        ga.kv_append(k[:, :, :min(qL, N)], v[:, :, :min(qL, N)], kc, vc, kv_offset=0)
        pending = None  # a block's partials, gate and out, merged by the next block's call
        for i, s in enumerate(range(0, N, qL)):
            e = min(s + qL, N)
            e2 = min(e + qL, N)
            nxt = (k[:, :, e:e2], v[:, :, e:e2], kc, vc, e) if e < N else None
            # a block whose main pass carries work (its plan's carry_blocks) takes the previous
            # block's merge and the next block's append in its own launch; the others merge
            # themselves, the next block's append riding on that merge
            carries = block_plans[i]["carry_blocks"] > 0
            if not carries and pending is not None:
                ga.merge(pending[0], pending[1], pending[3], out=pending[4], partial_exp=pending[2])
                pending = None
            if per_call is not None:
                per_call[i][0].record(stream)
            _, parts = ga.prefill_partials(q[:, :, s:e], kc, vc, g[:, :, s:e], kv_offset=s, kv_len=e,
                                           out=out[:, :, s:e], workspace=spaces[i % 2],
                                           append=nxt if carries else None, carry=pending if carries else None)
            if per_call is not None:
                per_call[i][1].record(stream)
            if carries:
                pending = (*parts, g[:, :, s:e], out[:, :, s:e])
            elif parts is not None:
                ga.merge(parts[0], parts[1], g[:, :, s:e], out=out[:, :, s:e], partial_exp=parts[2], append=nxt)
            elif nxt is not None:
                ga.kv_append(*nxt[:4], kv_offset=e)
        if pending is not None:
            ga.merge(pending[0], pending[1], pending[3], out=pending[4], partial_exp=pending[2])

    # ---- profiler mode: one workload, --steps times
    if args.only:
        if args.only == "prefill":
            fn = (lambda i: prefill_pass())
        elif args.only in ("decode", "verify"):
            rows = 1 if args.only == "decode" else 32
            fn = (lambda i: dset.call(rows, i))
        elif args.only in ("decode_f16", "verify_f16"):
            fset = DecodeSet(1014, 2, 16, 2, 32768, 32, "f16", True)
            rows = 1 if args.only == "decode_f16" else 32
            fset.prep(rows, args.only)
            fn = (lambda i: fset.call(rows, i))
        elif args.only == "decode_27b":
            kset = DecodeSet(1001, 1, 24, 4, 4096, 4, "bf16", False)
            kset.prep(1, "decode_27b")
            fn = (lambda i: kset.call(1, i))
        elif args.only == "prefill_8k":
            pr = _prompt_8k(ga, syn, dev, plans)
            fn = (lambda i: pr["run"]())
        else:
            Dp = int(args.only[len("prefill_d"):])
            pq, pk, pv, pg, pkc, pvc, pout = _prompt_inputs(syn, dev, B, Hq, Hkv, N, Dp)
            need = 16
            for i, s in enumerate(range(0, N, qL)):
                need = max(need, plans.check(f"prefill_32k_D{Dp}_qL{qL}_block{i}", op=0, B=B, Hq=Hq, Hkv=Hkv,
                                             rows=min(qL, N - s), kv_offset=s, D=Dp)["workspace_bytes"])
            wsp = torch.empty(need, dtype=torch.uint8, device=dev)
            fn = (lambda i: ga.prompt_prefill(pq, pk, pv, pg, pkc, pvc, q_block=qL, out=pout, workspace=wsp))
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        for i in range(args.steps):
            fn(i)
        torch.cuda.synchronize(dev)
        print(json.dumps({"only": args.only, "steps": args.steps,
                          "wall_ms_per_step": round((time.perf_counter() - t0) * 1e3 / args.steps, 3)}), flush=True)
        return

    def decode_step(it, evs=None, rows=1):
        kk_, vv_ = dset.caches[(it + (0 if rows == 1 else dset.n_rot // 2)) % dset.n_rot]
        ga.kv_append(dset.k_new[:, :, :rows], dset.v_new[:, :, :rows], kk_, vv_, kv_offset=dset.off)
        if evs is not None:
            evs[0].record(stream)
        ga.decode(dset.q[:, :, :rows], kk_, vv_, dset.g[:, :, :rows], kv_offset=dset.off, mask=dset.mask[rows],
                  out=dset.out[rows], workspace=dset.ws[rows])
        if evs is not None:
            evs[1].record(stream)

    for w in range(args.warmup):
        prefill_pass()
        decode_step(w)
        decode_step(w, rows=32)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    prefill_pass()
    decode_step(0)
    decode_step(0, rows=32)
    step_host_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize(dev)

    # ---- the timed steps
    K = args.steps
    ev = [[E(enable_timing=True) for _ in range(4)] for _ in range(K)]
    dec_ev = [[E(enable_timing=True), E(enable_timing=True)] for _ in range(K)]
    ver_ev = [[E(enable_timing=True), E(enable_timing=True)] for _ in range(K)]
    n_calls = len(block_plans)
    per_call = [[[E(enable_timing=True), E(enable_timing=True)] for _ in range(n_calls)] for _ in range(K)]
    torch.cuda.synchronize(dev)
    start, end = E(enable_timing=True), E(enable_timing=True)
    timer.hold(min(step_host_ms * K, 2000.0))  # the host gets ahead
    start.record(stream)
    for it in range(K):
        ev[it][0].record(stream)
        prefill_pass(per_call[it])
        ev[it][1].record(stream)
        decode_step(it, dec_ev[it])
        ev[it][2].record(stream)
        decode_step(it, ver_ev[it], rows=32)
        ev[it][3].record(stream)
    end.record(stream)
    torch.cuda.synchronize(dev)
    total_ms = start.elapsed_time(end)
    pre_ms = [e[0].elapsed_time(e[1]) for e in ev]
    call_ms = np.array([[pc[0].elapsed_time(pc[1]) for pc in step] for step in per_call])
    dec_host_us = np.array([e[0].elapsed_time(e[1]) for e in dec_ev]) * 1e3
    ver_host_us = np.array([e[0].elapsed_time(e[1]) for e in ver_ev]) * 1e3

    flops = prefill_flops(Hq, N)
    pre_tflops = flops / (np.mean(pre_ms) * 1e-3) / 1e12
    call_flops = np.array([4.0 * 256 * Hq * sum(range(s + 1, min(s + qL, N) + 1)) for s in range(0, N, qL)])
    call_mean_ms = call_ms.mean(axis=0)
    achieved_tflops = float(call_flops.sum() / (call_mean_ms.sum() * 1e-3) / 1e12)

    # ---- the decode workload, device-timed (48 calls a batch), cold and MALL-warm
    def dec_figures(ds, rows, warm=True, append=True):
        plan = ds.prep(rows, f"decode_{ds.B}x{ds.Hq}/{ds.Hkv}_off{ds.off}_rows{rows}_{ds.dtype}{ds.tag}")
        cold_ms = timer.time(lambda i: ds.call(rows, i), 48)
        r = {"us": round(cold_ms * 1e3, 2), "gbs": round(ds.bytes(rows) / (cold_ms * 1e-3) / 1e9, 1),
             "frac_of_hbm": round(ds.bytes(rows) / (cold_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
             "bytes": int(ds.bytes(rows)), "tflops_upper": round(
                 4.0 * 256 * ds.B * ds.Hq * rows * (ds.off + rows) / (cold_ms * 1e-3) / 1e12, 1),
             "plan": {kk: plan[kk] for kk in ("variant_name", "n_splits", "n_head_chunks", "grid_blocks")}}
        if warm:
            warm_ms = timer.time(lambda i: ds.call(rows, i, cold=False), 48)
            r["mall_warm_us"] = round(warm_ms * 1e3, 2)
            r["mall_warm_gbs"] = round(ds.bytes(rows) / (warm_ms * 1e-3) / 1e9, 1)
        if append:
            r["with_append_us"] = round(timer.time(lambda i: ds.call(rows, i, append=True), 48) * 1e3, 2)
        return r

    dec_matrix = {"bf16": {}, "f16": {}}
    for rows in (1, 4, 32):
        dec_matrix["bf16"][f"rows_{rows}"] = dec_figures(dset, rows)
    head = dec_matrix["bf16"]["rows_1"]
    extras = {}
    if not args.no_extras:
        fset = DecodeSet(1014, 2, 16, 2, 32768, 32, "f16", True)
        for rows in (1, 4, 32):
            dec_matrix["f16"][f"rows_{rows}"] = dec_figures(fset, rows, warm=False, append=False)
        del fset
        oset = DecodeSet(1024, 2, 16, 2, 4097, 32, "bf16", True)
        dec_matrix["bf16_offset_4097"] = {f"rows_{rows}": dec_figures(oset, rows, warm=False, append=False)
                                          for rows in (1, 32)}
        del oset
        # the same workload under a full-head additive mask [1, 16, rows, kv] and a bool mask
        hset = DecodeSet(1034, 2, 16, 2, 32768, 32, "bf16", True, mask_heads=16)
        dec_matrix["bf16_full_head_mask"] = {f"rows_{rows}": dec_figures(hset, rows, warm=False, append=False)
                                             for rows in (1, 4, 32)}
        del hset
        bset = DecodeSet(1044, 2, 16, 2, 32768, 32, "bf16", True, mask_kind="bool")
        dec_matrix["bf16_bool_mask"] = {f"rows_{rows}": dec_figures(bset, rows, warm=False, append=False)
                                        for rows in (1, 32)}
        del bset
        # [1] the 27B decode at 4096: rows 1 and 4, no mask, cold and MALL-warm
        kset = DecodeSet(1001, 1, 24, 4, 4096, 4, "bf16", False)
        extras["decode_27b_off4096"] = {f"rows_{rows}": dec_figures(kset, rows) for rows in (1, 4)}
        del kset
        torch.cuda.empty_cache()

    # ---- the same 32k prompt in other query blocks (time, workspace, torch allocator peak)
    def prompt_figures(qb_, composed=False, D=256):
        if D == 256:
            pq, pk, pv, pg, pkc, pvc, pout = q, k, v, g, kc, vc, out
        else:
            pq, pk, pv, pg, pkc, pvc, pout = _prompt_inputs(syn, dev, B, Hq, Hkv, N, D)
        op = 2 if composed else 0
        need = max(ga.workspace_bytes(ga.plan_args(B=B, Hq=Hq, Hkv=Hkv, rows=min(qb_, N - s), kv_offset=s,
                                                   capacity=N, D=D), op) for s in range(0, N, qb_))
        if not composed:
            for i, s in enumerate(range(0, N, qb_)):
                plans.check(f"prefill_32k_D{D}_qL{qb_}_block{i}", op=0, B=B, Hq=Hq, Hkv=Hkv, rows=min(qb_, N - s),
                            kv_offset=s, D=D)
        wsp = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

        def run(i=0):
            ga.prompt_prefill(pq, pk, pv, pg, pkc, pvc, q_block=qb_, out=pout, workspace=wsp, composed=composed)

        run()
        torch.cuda.synchronize(dev)
        ms = timer.time(run, 1, 2 if composed else 3)
        # torch allocator peak over one pass that allocates its workspace through torch
        del wsp
        torch.cuda.synchronize(dev)
        torch.cuda.reset_peak_memory_stats(dev)
        base = torch.cuda.memory_allocated(dev)
        ga.prompt_prefill(pq, pk, pv, pg, pkc, pvc, q_block=qb_, out=pout, composed=composed)
        torch.cuda.synchronize(dev)
        peak = torch.cuda.max_memory_allocated(dev) - base
        tf = prefill_flops(Hq, N, D) / (ms * 1e-3) / 1e12
        return {"ms": round(ms, 3), "tflops": round(tf, 2), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                "calls": len(range(0, N, qb_)), "workspace_bytes": int(need), "torch_peak_delta_bytes": int(peak)}

    q_blocks, composed_fig, small = {}, {}, {}
    if not args.no_extras:
        for qb_ in (128, 1024, 2048):
            q_blocks[f"q_block_{qb_}"] = prompt_figures(qb_)
        for qb_ in (512, 128):
            f = prompt_figures(qb_, composed=True)
            cbytes = 0.0
            for s in range(0, N, qb_):
                e = min(s + qb_, N)
                kvp = -(-e // 32) * 32
                cbytes += B * Hq * (e - s) * (kvp * 16.0 + 3 * 512) + 2.0 * B * Hkv * e * 512
            f["roofline"] = {"bound": "hbm", "achieved": round(cbytes / (f["ms"] * 1e-3) / 1e9, 1),
                             "peak": PEAK_HBM_GBS, "unit": "GB/s", "bytes": int(cbytes),
                             "frac": round(cbytes / (f["ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
            composed_fig[f"q_block_{qb_}"] = f
            torch.cuda.empty_cache()
        for D_ in (128, 64):
            small[f"head_dim_{D_}"] = {f"q_block_{qb_}": prompt_figures(qb_, D=D_) for qb_ in (512, 128, 1024, 2048)}
            for qb_ in (512, 128):
                small[f"head_dim_{D_}"][f"composed_q_block_{qb_}"] = prompt_figures(qb_, composed=True, D=D_)
                torch.cuda.empty_cache()
            torch.cuda.empty_cache()
        # the prompt policy (attn_prompt_policy) on this device for the same prompt at each head dim
        policy = {}
        for D_ in (256, 128, 64):
            pol = ga.prompt_policy(D=D_, B=B, Hq=Hq, Hkv=Hkv, n_tokens=N)
            policy[f"head_dim_{D_}"] = {"choice": pol, **prompt_figures(pol["q_block"], D=D_)}
            torch.cuda.empty_cache()
        extras["prefill_policy"] = {"route": "the block size and route attn_prompt_policy picks for this device",
                                    "device_key": dict(zip(("gfx", "n_cus"), ga.device_key())), **policy}
        pr = _prompt_8k(ga, syn, dev, plans)
        pr["run"]()
        torch.cuda.synchronize(dev)
        ms8 = timer.time(lambda i: pr["run"](), 1, 5)
        tf8 = prefill_flops(16, 8192) / (ms8 * 1e-3) / 1e12
        extras["prefill_35b_8192_near_ties"] = {
            "ms": round(ms8, 4), "tflops": round(tf8, 2), "frac_of_peak": round(tf8 / PEAK_BF16_TFLOPS, 4),
            "q_block": 512, "near_tie_rows": pr["tie_rows"], "calls": 16,
            "plan_last_block": {kk: pr["last_plan"][kk] for kk in ("variant_name", "n_splits", "n_row_tiles",
                                                                   "grid_blocks")}}
        del pr
        torch.cuda.empty_cache()
        extras["probes"] = probes(dev, timer)

    # the main prompt's own allocator peak at qL 512 (its workspace through torch)
    torch.cuda.synchronize(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    ga.prompt_prefill(q, k, v, g, kc, vc, q_block=qL, out=out)
    torch.cuda.synchronize(dev)
    peak512 = torch.cuda.max_memory_allocated(dev) - base

    traffic = measured_traffic() if (N, qL) == (32768, 512) else None
    dec_bytes = dset.bytes(1)
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
                               f"query blocks of {qL}; 35B-A3B-shape head-chunked verify workload (batch 2, 16/2 "
                               f"heads, KV offset 32768, broadcast additive mask with -Inf entries): 1 decode row "
                               f"and 32 verify rows",
                   "seq_len": N, "q_block": qL, "global_batch": B},
        "prefill": {"ms": round(float(np.mean(pre_ms)), 4), "tflops": round(float(pre_tflops), 2),
                    "frac_of_peak": round(float(pre_tflops) / PEAK_BF16_TFLOPS, 4), "calls": n_calls,
                    "workspace_bytes": int(ws_need), "torch_peak_delta_bytes": int(peak512),
                    "plan_last_block": {kk: block_plans[-1][kk] for kk in ("variant_name", "n_splits",
                                                                           "keys_per_split", "n_row_tiles",
                                                                           "grid_blocks")}},
        "prefill_q_blocks": q_blocks,
        "prefill_composed": {"route": "materialised scores: fp32 Q K^T, row softmax to 16-bit weights, P V + gate "
                                      "(attn_prefill_composed), kv_append per block", **composed_fig},
        "prefill_small_head_dims": {"route": "the main pass at head dims 64 and 128, 24/4 heads, the same prompt "
                                             "length", **small},
        "decode": {"metric": "decode KV GB/s (35B-A3B shape, batch 2, 16/2 heads, 1 row at offset 32768 with its "
                             "broadcast additive mask, cold KV; device time of attn_decode: main pass + merge)",
                   "value": head["gbs"], "unit": "GB/s", "us": head["us"], "bytes": int(dec_bytes),
                   "distinct_caches": dset.n_rot, "device_timed": timer.held,
                   "host_bound_call_us": round(float(np.median(dec_host_us)), 2),
                   "mall_warm_gbs": head["mall_warm_gbs"], "mall_warm_us": head["mall_warm_us"],
                   "with_append_us": head["with_append_us"],
                   "roofline": {"bound": "hbm", "achieved": head["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(head["gbs"] / PEAK_HBM_GBS, 4),
                                "traffic": traffic and traffic.get("decode_call_bytes")},
                   "plan": {kk: dplan[kk] for kk in ("variant_name", "n_splits", "keys_per_split", "n_head_chunks",
                                                     "grid_blocks")},
                   "rows": dec_matrix},
        "verify": {"metric": "head-chunked verify, 32 rows at offset 32768, broadcast additive mask (cold KV; "
                             "device time of attn_decode)",
                   "us": dec_matrix["bf16"]["rows_32"]["us"], "gbs": dec_matrix["bf16"]["rows_32"]["gbs"],
                   "tflops_upper": dec_matrix["bf16"]["rows_32"]["tflops_upper"],
                   "host_bound_call_us": round(float(np.median(ver_host_us)), 2),
                   "plan": {kk: vplan[kk] for kk in ("variant_name", "n_splits", "keys_per_split", "n_head_chunks",
                                                     "grid_blocks")}},
        **extras,
        "roofline": {"bound": "mfma", "achieved": round(achieved_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic and traffic.get("prefill_main_bytes"),
                     "kernel": "attn_fwd_kernel (main pass of a prefill block; where the block's plan has "
                               "carry_blocks, the launch also runs the previous block's merge and the next "
                               "block's append on the CUs the main pass leaves idle)",
                     "avg_launch_us": round(float(call_mean_ms.mean()) * 1e3, 2)},
        "plans": {"validated": len(plans.samples), "samples": [s for s in plans.samples
                                                               if "block" not in s["sample"]
                                                               or s["sample"].endswith(("_block0", "_block63"))]},
        "setup_s": round(setup_s, 1),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(host, args.cpu_sample_rows, N)
    print(json.dumps(result), flush=True)


SWEEP_Q_BLOCKS = (128, 256, 512, 1024, 2048, 4096, 8192, 32768)


def q_block_sweep(ga, syn, dev, timer, plans):
    """Device time of a whole causal prompt on the fused route (kv_append + attn_prefill per
    query block) for every query-block size up to the prompt length, at head dims 256, 128 and
    64, the 24/4 and 16/2 head shapes and prompts of 2048, 8192 and 32768 tokens: the
    measurements behind the prompt policy (attn_prompt_policy).  One line per case as it ends."""
    out = []
    for D in (256, 128, 64):
        for Hq, Hkv in ((24, 4), (16, 2)):
            for N in (2048, 8192, 32768):
                pq, pk, pv, pg, pkc, pvc, pout = _prompt_inputs(syn, dev, 1, Hq, Hkv, N, D)
                row = {"head_dim": D, "Hq": Hq, "Hkv": Hkv, "n_tokens": N, "ms": {}, "workspace_bytes": {}}
                for qL in SWEEP_Q_BLOCKS:
                    if qL > N:
                        continue
                    need = 16
                    for i, s in enumerate(range(0, N, qL)):
                        need = max(need, plans.check(f"sweep_D{D}_{Hq}x{Hkv}_N{N}_qL{qL}_block{i}", op=0, B=1,
                                                     Hq=Hq, Hkv=Hkv, rows=min(qL, N - s), kv_offset=s,
                                                     D=D)["workspace_bytes"])
                    wsp = torch.empty(need, dtype=torch.uint8, device=dev)

                    def run(i=0):
                        ga.prompt_prefill(pq, pk, pv, pg, pkc, pvc, q_block=qL, out=pout, workspace=wsp)

                    run()
                    torch.cuda.synchronize(dev)
                    row["ms"][str(qL)] = round(timer.time(run, 1, 3), 4)
                    row["workspace_bytes"][str(qL)] = int(need)
                    del wsp
                best = min(row["ms"], key=lambda k: row["ms"][k])
                row["fastest_q_block"] = int(best)
                row["tflops_at_fastest"] = round(prefill_flops(Hq, N, D) / (row["ms"][best] * 1e-3) / 1e12, 1)
                print(json.dumps(row), flush=True)
                out.append(row)
                del pq, pk, pv, pg, pkc, pvc, pout
                torch.cuda.empty_cache()
    return out


def _prompt_inputs(syn, dev, B, Hq, Hkv, N, D):
    """A seeded prompt at head dim D: q, k, v, gate, empty K/V caches and the output."""
    r = syn.streams(1005 + D)
    q, k, v, g = (_up(syn.normal_bits(r[nm], (B, H, N, D)), dev)
                  for nm, H in (("q", Hq), ("k", Hkv), ("v", Hkv), ("gate", Hq)))
    kc = torch.empty((B, Hkv, N, D), dtype=torch.bfloat16, device=dev)
    return q, k, v, g, kc, torch.empty_like(kc), torch.empty_like(q)


def _prompt_8k(ga, syn, dev, plans):
    """The 35B-A3B prompt: batch 1, 16/2 heads, 8192 tokens in 512-row blocks, 10% of rows with two
    near-tied top scores (within two bf16 steps) in every head."""
    B, Hq, Hkv, N, qL = 1, 16, 2, 8192, 512
    r = syn.streams(1002)
    qb = syn.normal_bits(r["q"], (B, Hq, N, 256))
    kb = syn.normal_bits(r["k"], (B, Hkv, N, 256))
    vb = syn.normal_bits(r["v"], (B, Hkv, N, 256))
    gb = syn.normal_bits(r["gate"], (B, Hq, N, 256))
    qb, rec = syn.plant_near_ties(qb, kb, n_kv_heads=Hkv, rng=r["plant"])
    q, k, v, g = (_up(x, dev) for x in (qb, kb, vb, gb))
    kc = torch.empty((B, Hkv, N, 256), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    out = torch.empty_like(q)
    last = None
    for i, s in enumerate(range(0, N, qL)):
        last = plans.check(f"prefill_35b_8192_block{i}", op=0, B=B, Hq=Hq, Hkv=Hkv, rows=qL, kv_offset=s)
    need = max(ga.workspace_bytes(ga.plan_args(B=B, Hq=Hq, Hkv=Hkv, rows=qL, kv_offset=s), 0)
               for s in range(0, N, qL))
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

    def run():
        ga.prompt_prefill(q, k, v, g, kc, vc, q_block=qL, out=out, workspace=ws)

    return {"run": run, "tie_rows": int(np.unique(rec[:, 2]).size), "last_plan": last}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(host, n_rows, N):
    """The float64 oracle on a bounded sample of the same prompt: n_rows query rows spread over
    the prompt, all 24 heads, each against its causal prefix, in one process with the BLAS
    threads numpy was given; scaled to TFLOP/s and extrapolated to the whole prompt."""
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
    threads, api = None, None
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            threads = max(i.get("num_threads") or 0 for i in infos) or None
            api = infos[0].get("internal_api")
    except Exception:  # threadpoolctl missing: fall back to the affinity mask
        pass
    if not threads:
        threads = len(os.sched_getaffinity(0))
    tfs = flops / dt / 1e12
    return {"value": round(tfs, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_rows} query rows x 24 heads of the 32768-token prompt, each against its causal prefix "
                      f"(float64 NumPy/BLAS, one process), {dt:.1f} s; the whole prompt (1.3195e13 flop) would take "
                      f"about {prefill_flops(Hq, N) / (tfs * 1e12):.0f} s at this rate (extrapolated, not run)",
            "cpu_model": _cpu_model(), "blas": api, "blas_threads": threads,
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
