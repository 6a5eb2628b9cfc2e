#!/usr/bin/env python3
"""Benchmark of the compressed KV-cache codec on one MI355X.

One step = one pass of the whole hot path over the Llama-3-8B-shaped 4K
shared cache (32 layers x 8 kv-heads x 4096 tokens x head_dim 128, bf16 K/V,
Student-t(5) values with log-normal channel scales):
  kvpool_encode   K+V -> pool                        (PolyKV 2.B)
  kvpool_decode   pool -> bf16 K/V of 15 agents       (PolyKV 2.A fan-out)
  cachecard_pack  K+V -> CacheCard, per-token widths  (QKVShare item 2)
  cachecard_unpack card -> bf16 K/V                   (QKVShare item 3)
Inputs are generated on the GPU before timing. The JSON line reports
whole-step throughput in algorithmic GB/s (bytes each op must read and write
once), the per-op figures (back to back as in the step, and again with the
caches flushed by a 1 GiB write before each call), streaming ceilings from
probe kernels (read-only, write-only, copy), the roofline of the dominant
op (HIP events on the stream it runs on; the mean, as the profiler's kernel
statistics report means), and the CPU oracle timed on the same workload
together with its parity report against the GPU's outputs.
"""

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
FANOUT_MIN_AGENTS = 8  # the library decodes into this many agents or more as decode + fan-out copy
METRIC = "KV codec encode/decode GB/s and % of HBM peak, Llama-3-8B shape 4K tok"
FLUSH_BYTES = 1 << 30  # written, then another buffer read, before each cache-flushed call (4x the 256 MB
#                        Infinity Cache): the caches then hold clean lines of neither the op's inputs nor
#                        outputs, and no write-back of the flush's own data falls into the op's time
PROBE_BYTES = 2 << 30  # buffers of the streaming ceilings
OPS = ["encode", "decode", "pack", "unpack"]
CARD_MODEL_ID = b"llama-3-8b"  # the step's card metadata (position offset 0)
# kernels of each op, in launch order (the single-pass encode applies to
# this workload: a round of whole layers fits the GPU's LDS; pack and unpack
# scan the record offsets inside their own grid at 4096 tokens)
OP_KERNELS = {"encode": ["pool_encode_fused_kernel"],
              "decode": ["pool_decode_kernel<128, true>", "fanout_copy_kernel"],
              "pack": ["card_pack_kernel"],
              "unpack": ["card_unpack_kernel"]}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--agents", type=int, default=15)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--other-configs", action="store_true",
                    help="instead of the step: one JSON line per op for the tiny, SmolLM2 2K, 8K card and 32K "
                         "workloads (reported, not the benchmark line)")
    ap.add_argument("--cpu-layers", type=int, default=32, help="layers of the workload in the CPU oracle sample")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM bytes per dispatch (from rocprofv3 counters)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, copy a 1 GiB device buffer 3 times (the reference dispatches "
                         "that scale the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="only parse two rocprofv3 --pmc output folders (FETCH_SIZE, WRITE_SIZE) of a "
                         "--calibrate-copy run, write --traffic and print a summary table")
    ap.add_argument("--traffic-runs", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="only print FETCH_SIZE / WRITE_SIZE per dispatch for each run of consecutive dispatches of "
                         "one codec kernel with one grid size (e.g. of an --other-configs --calibrate-copy run)")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR",
                    help="only parse the kernel trace of a profiled bench run (rocprofv3 --kernel-trace, csv): "
                         "per-kernel durations over the step's timed dispatches, the op sums and the roofline "
                         "fraction they give, beside the bench line given by --bench-json")
    ap.add_argument("--bench-json", help="with --trace-summary: the JSON line the profiled run printed")
    return ap.parse_args()


def pool_payload_bytes(L, H, T, d):
    """Bytes of the pool's sections without header or padding."""
    vecs = L * H * T
    return 4 * L + vecs * d + 2 * vecs + vecs * 3 * d // 8


# ------------------------------------------------------------------ probes

def probe_lib():
    """libkvprobe.so: streaming copy / fill / read kernels (16 bytes per lane)."""
    import torch  # noqa: F401  (loaded first: the probes bind to torch's HIP runtime)
    path = os.path.join(ROOT, "agent_handoff_amd", "libkvprobe.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    p, sz, i32, u32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint32
    for name, args in (("kvp_copy", [p, p, sz, i32, p]), ("kvp_fill", [p, sz, u32, i32, p]),
                       ("kvp_read", [p, sz, p, i32, p])):
        f = getattr(lib, name)
        f.restype = i32
        f.argtypes = args
    return lib


class Probes:
    """The probe kernels on one stream. Variants: 0/1 one 16-byte unit per
    thread (plain / non-temporal stores), 2/3 four units per thread."""

    def __init__(self, stream):
        import torch
        self.lib = probe_lib()
        self.s = ctypes.c_void_p(stream.cuda_stream)
        self.sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    @staticmethod
    def _p(t):
        return ctypes.c_void_p(t.data_ptr())

    def fill(self, t, variant=2, value=0):
        rc = self.lib.kvp_fill(self._p(t), t.numel() * t.element_size(), value, variant, self.s)
        assert rc == 0, f"kvp_fill: {rc}"

    def copy(self, src, dst, variant=2):
        rc = self.lib.kvp_copy(self._p(src), self._p(dst), src.numel() * src.element_size(), variant, self.s)
        assert rc == 0, f"kvp_copy: {rc}"

    def read(self, src, variant=2):
        rc = self.lib.kvp_read(self._p(src), src.numel() * src.element_size(), self._p(self.sink), variant, self.s)
        assert rc == 0, f"kvp_read: {rc}"


# ------------------------------------------------------------------ the step

def main():
    args = parse()
    if args.traffic_from:
        traffic_from_counters(args.traffic_from[0], args.traffic_from[1], args.traffic, args.agents)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary, args.bench_json, args.warmup, args.steps)
        return
    if args.traffic_runs:
        traffic_runs(*args.traffic_runs)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (this codec is measured on "
              "one GPU's share; the multi-GPU handoff is a design note, not a benchmark)", file=sys.stderr)
        sys.exit(2)
    if args.other_configs:
        other_configs(args)
        return

    import numpy as np
    import torch

    from agent_handoff_amd import kvcodec as kv
    from agent_handoff_amd import synth

    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[3]
    L, H, T, d = shape = w.shape
    A = args.agents
    kv_bytes = L * H * T * d * 2

    log(f"generating {w.name} inputs on the GPU")
    k, v = synth.kv_tensors_torch(w, args.seed, dev)
    widths_np = synth.card_widths(synth.WORKLOADS[4], args.seed, T=T)
    widths = torch.from_numpy(widths_np).to(dev)

    pool = torch.empty(kv.kvpool_bytes(shape), dtype=torch.uint8, device=dev)
    ws = torch.zeros(kv.kvpool_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    k_out = [torch.empty_like(k) for _ in range(A)]
    v_out = [torch.empty_like(v) for _ in range(A)]
    card_n = kv.cachecard_bytes_host(shape, widths_np)
    card = torch.empty(card_n, dtype=torch.uint8, device=dev)
    cws = torch.empty(kv.cachecard_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    k_rt = torch.empty_like(k)
    v_rt = torch.empty_like(v)
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    torch.cuda.synchronize()  # inputs and buffers ready before the codec stream starts
    stream = torch.cuda.Stream()
    probes = Probes(stream)

    def op_call(o, agents=A):
        if o == "encode":
            kv.kvpool_encode(shape, k, v, pool, ws, status, stream=stream)
        elif o == "decode":
            kv.kvpool_decode(shape, pool, 0, L, k_out[:agents], v_out[:agents], status, stream=stream)
        elif o == "pack":
            kv.cachecard_pack(shape, k, v, widths, card, cws, CARD_MODEL_ID, 0, None, status, stream=stream)
        else:
            kv.cachecard_unpack(shape, card, k_rt, v_rt, cws, card_n, status, stream=stream)

    def step(ev=None):
        for j, o in enumerate(OPS):
            if ev is not None:
                ev[j].record(stream)
            op_call(o)
        if ev is not None:
            ev[len(OPS)].record(stream)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "device status set"

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(OPS) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert int(status.item()) == 0, "device status set during the timed steps"
    per_op = {o: [] for o in OPS}
    for ev in events:
        for j, o in enumerate(OPS):
            per_op[o].append(ev[j].elapsed_time(ev[j + 1]) * 1e-3)
    step_s = [sum(per_op[o][i] for o in OPS) for i in range(args.steps)]
    ms_per_step = wall / args.steps * 1e3

    # the step's outputs, for the oracle's parity report
    snap = None
    if not args.no_cpu_baseline:
        def bits(t):
            return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        snap = {"pool": pool.cpu().numpy(), "card": card.cpu().numpy(), "k_dec": bits(k_out[0]),
                "v_dec": bits(v_out[0]), "k_unp": bits(k_rt), "v_unp": bits(v_rt)}

    pool_b = pool_payload_bytes(*shape)
    alg = {"encode": 2 * kv_bytes + pool_b, "decode": pool_b + A * 2 * kv_bytes,
           "pack": 2 * kv_bytes + card_n, "unpack": card_n + 2 * kv_bytes}
    # bytes read and written once (the mix of each op's traffic)
    mix = {"encode": (2 * kv_bytes, pool_b), "decode": (pool_b, A * 2 * kv_bytes),
           "pack": (2 * kv_bytes, card_n), "unpack": (card_n, 2 * kv_bytes),
           "decode_1_agent": (pool_b, 2 * kv_bytes)}
    total_bytes = sum(alg.values())
    value = total_bytes / (wall / args.steps) / 1e9

    def med(x):
        return float(np.median(np.asarray(x)))

    def timed_list(fn, reps, flush=None):
        """Event durations (s) of reps calls of fn on the codec stream; with
        flush, a 1 GiB write runs before each call (outside its events)."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            if flush is not None:
                flush()
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e-3 for a, b in ev]

    def timed(fn, reps, flush=None):
        return med(timed_list(fn, reps, flush))

    # ---- streaming ceilings from the probe kernels (best variant of each)
    log("streaming ceilings")
    pa = torch.empty(PROBE_BYTES, dtype=torch.uint8, device=dev)
    pb = torch.empty(PROBE_BYTES, dtype=torch.uint8, device=dev)
    probes.fill(pa, 2, 0x3C3C3C3C)
    probes.fill(pb, 2, 0)
    rates = {"read": {}, "write": {}, "copy": {}}
    for var in range(4):
        rates["read"][var] = PROBE_BYTES / timed(lambda: probes.read(pa, var), 10) / 1e9
        rates["write"][var] = PROBE_BYTES / timed(lambda: probes.fill(pb, var), 10) / 1e9
        rates["copy"][var] = 2 * PROBE_BYTES / timed(lambda: probes.copy(pa, pb, var), 10) / 1e9
    del pa, pb
    best = {kind: max(r.values()) for kind, r in rates.items()}
    # a copy of the decode's byte count (half read, half written)
    half = alg["decode"] // 2 // 16 * 16
    cs = torch.empty(half, dtype=torch.uint8, device=dev)
    cd = torch.empty_like(cs)
    probes.fill(cs, 2, 0x5A5A5A5A)
    cvar = max(rates["copy"], key=rates["copy"].get)
    tc = timed(lambda: probes.copy(cs, cd, cvar), 5)
    del cs, cd
    torch.cuda.empty_cache()

    def mix_ceiling_us(o):
        r, wr = mix[o]
        return (r / (best["read"] * 1e9) + wr / (best["write"] * 1e9)) * 1e6

    ops_out = {}
    for o in OPS:
        t, tm = med(per_op[o]), float(np.mean(per_op[o]))
        gbs = alg[o] / t / 1e9
        p10, p90 = (float(np.percentile(np.asarray(per_op[o]), q)) for q in (10, 90))
        ops_out[o] = {"us": round(t * 1e6, 2), "us_mean": round(tm * 1e6, 2), "us_p10": round(p10 * 1e6, 2),
                      "us_p90": round(p90 * 1e6, 2), "bytes": alg[o], "GB/s": round(gbs, 1),
                      "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                      "mix_ceiling_us": round(mix_ceiling_us(o), 2),
                      "frac_of_mix_ceiling": round(mix_ceiling_us(o) / (t * 1e6), 4)}

    # ---- each op again with the caches flushed before every call
    log("cache-flushed calls")
    flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    flush_rd = torch.zeros(FLUSH_BYTES, dtype=torch.uint8, device=dev)

    def flush():
        probes.fill(flush_buf, 2, 0)
        probes.read(flush_rd, 0)

    for o in OPS:
        tf = timed(lambda: op_call(o), 10, flush)
        ops_out[o]["flushed_us"] = round(tf * 1e6, 2)
        ops_out[o]["flushed_frac_hbm_peak"] = round(alg[o] / tf / 1e9 / HBM_PEAK_GBS, 4)
    b1 = pool_b + 2 * kv_bytes
    t1 = timed(lambda: op_call("decode", 1), 10)
    t1f = timed(lambda: op_call("decode", 1), 10, flush)
    ops_out["decode_1_agent"] = {"us": round(t1 * 1e6, 2), "bytes": b1, "GB/s": round(b1 / t1 / 1e9, 1),
                                 "frac_hbm_peak": round(b1 / t1 / 1e9 / HBM_PEAK_GBS, 4),
                                 "flushed_us": round(t1f * 1e6, 2),
                                 "flushed_frac_hbm_peak": round(b1 / t1f / 1e9 / HBM_PEAK_GBS, 4),
                                 "mix_ceiling_us": round(mix_ceiling_us("decode_1_agent"), 2),
                                 "frac_of_mix_ceiling": round(mix_ceiling_us("decode_1_agent") / (t1 * 1e6), 4)}
    del flush_buf, flush_rd
    torch.cuda.empty_cache()
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "device status set in the flushed calls"

    # ---- beside the step
    # one hop of a card chain: the step's card re-encoded at the next agent's widths
    w_next_np = synth.card_widths(synth.WORKLOADS[4], args.seed + 1, T=T)
    w_next = torch.from_numpy(w_next_np).to(dev)
    card2_n = kv.cachecard_bytes_host(shape, w_next_np)
    card2 = torch.empty(card2_n, dtype=torch.uint8, device=dev)
    tws = torch.empty(kv.cachecard_transcode_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    tt = timed(lambda: kv.cachecard_transcode(shape, card, w_next, card2, tws, card_in_bytes=card_n, dev_status=status,
                                              stream=stream), 10)
    bt = card_n + card2_n
    ops_out["transcode"] = {"us": round(tt * 1e6, 2), "bytes": bt, "GB/s": round(bt / tt / 1e9, 1),
                            "frac_hbm_peak": round(bt / tt / 1e9 / HBM_PEAK_GBS, 4)}
    # key position re-alignment of the shared keys by 4096 positions (rotary
    # frequencies of the Llama-3 family: base 500000 over d channels)
    inv_freq = (500000.0 ** (-np.arange(d // 2, dtype=np.float64) * 2.0 / d)).astype(np.float32)
    tr = timed(lambda: kv.kvc_realign_keys(shape, k, k_rt, 4096, inv_freq, stream=stream), 10)
    ops_out["realign_keys"] = {"us": round(tr * 1e6, 2), "bytes": 2 * kv_bytes, "GB/s": round(2 * kv_bytes / tr / 1e9, 1),
                               "frac_hbm_peak": round(2 * kv_bytes / tr / 1e9 / HBM_PEAK_GBS, 4)}
    # low-rank anchor materialisation (KVCMAS defaults: V = 10 anchors of
    # rank 32) of the K and the V cache, one launch per tensor over its layers
    n_anc, rank = 10, 32
    fk = synth.anchor_factors_torch(args.seed, 6, L, n_anc, T, H * d, rank, device=dev)
    fv = synth.anchor_factors_torch(args.seed + 1, 6, L, n_anc, T, H * d, rank, device=dev)
    torch.cuda.synchronize()

    def lowrank():
        kv.kvc_lowrank_materialize(shape, rank, n_anc, k, *fk, k_rt, stream=stream)
        kv.kvc_lowrank_materialize(shape, rank, n_anc, v, *fv, v_rt, stream=stream)

    tl = timed(lowrank, 10)
    bl = 2 * (2 * kv_bytes + sum(t.numel() * t.element_size() for t in fk))
    fl = 2 * (2.0 * L * n_anc * T * H * d * rank)
    ops_out["lowrank_materialize"] = {"us": round(tl * 1e6, 2), "bytes": bl, "GB/s": round(bl / tl / 1e9, 1),
                                      "frac_hbm_peak": round(bl / tl / 1e9 / HBM_PEAK_GBS, 4),
                                      "TFLOP/s": round(fl / tl / 1e12, 1),
                                      "frac_mfma_bf16_peak": round(fl / tl / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                                      "anchors": n_anc, "rank": rank}
    del fk, fv
    # the write-once side of the anchors: the rank-32 truncated SVD of the K
    # cache (32 layers of 4096 x 1024), randomized on a 48-column sketch
    om = torch.from_numpy(synth.sketch(args.seed, 7, H * d)).to(dev)
    fa = torch.empty((L, T, rank), dtype=torch.bfloat16, device=dev)
    fr = torch.empty((L, H * d, rank), dtype=torch.bfloat16, device=dev)
    fws = torch.empty(kv.kvc_lowrank_factor_workspace_bytes(shape, rank), dtype=torch.uint8, device=dev)
    tf = timed(lambda: kv.kvc_lowrank_factor(shape, rank, k, om, fa, fr, fws, stream=stream), 5)
    ff = 4 * 2.0 * L * T * H * d * kv.LOWRANK_SKETCH
    ops_out["lowrank_factor"] = {"us": round(tf * 1e6, 2), "bytes": 4 * kv_bytes, "GB/s": round(4 * kv_bytes / tf / 1e9, 1),
                                 "TFLOP/s": round(ff / tf / 1e12, 2), "rank": rank, "sketch": kv.LOWRANK_SKETCH,
                                 "note": "Z read four times (two products with Z, two with Z^T)"}
    del fa, fr, fws
    drift = hop_drift(kv, synth, k, v, shape, widths_np, args.seed, stream, dev)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "device status set beside the step"

    ceilings = {"read_GB/s": round(best["read"], 1), "write_GB/s": round(best["write"], 1),
                "copy_GB/s": round(best["copy"], 1),
                "by_variant": {kind: {str(v_): round(x, 1) for v_, x in r.items()} for kind, r in rates.items()},
                "copy_decode_bytes": {"bytes": 2 * half, "us": round(tc * 1e6, 2),
                                      "GB/s": round(2 * half / tc / 1e9, 1),
                                      "decode_frac_of_copy": round(alg["decode"] / med(per_op["decode"]) /
                                                                   (2 * half / tc), 4)},
                "note": "probe kernels, 16-byte accesses per lane, 2 GiB buffers; mix ceiling of an op = "
                        "bytes read / read rate + bytes written / write rate"}

    # dominant op: the most time per step. Its kernels (the decode into many
    # agents is the decode kernel for agent 0, then the fan-out copy kernel)
    # are timed together by the op's events; the mean over the timed steps,
    # as the profiler's kernel statistics report means.
    dom = max(OPS, key=lambda o: float(np.mean(per_op[o])))
    kernel_names = dict(OP_KERNELS)
    if A < FANOUT_MIN_AGENTS:
        kernel_names["decode"] = ["pool_decode_kernel<128, false>"]
    traffic = None
    if os.path.exists(args.traffic):
        with open(args.traffic) as f:
            tr_ = json.load(f)
        entries = [tr_.get(kname.split("<")[0]) for kname in kernel_names[dom]]
        sha = _lib_sha(kv.LIB_PATH)
        if all(e and e.get("library_sha") == sha and e.get("agents") == A for e in entries):
            traffic = sum(e["bytes_per_dispatch"] for e in entries)
    t_dom = float(np.mean(per_op[dom]))
    ach = alg[dom] / t_dom / 1e9
    roofline = {"bound": "hbm", "op": dom, "kernel": " + ".join(kernel_names[dom]), "achieved": round(ach, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                "us_mean": round(t_dom * 1e6, 2), "bytes": alg[dom],
                "frac_of_mix_ceiling": round(mix_ceiling_us(dom) / (t_dom * 1e6), 4)}

    if args.calibrate_copy:
        calibration_copies(dev, stream)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(k, v, widths_np, shape, args.cpu_layers, A, snap)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "layers": L, "kv_heads": H, "tokens": T, "head_dim": d, "agents": A,
                   "values": "student-t(5) x log-normal channel scales",
                   "card_widths": "runs of geometric length, mean 16, widths 2/4/8/16 at .4/.3/.2/.1"},
        "ops": ops_out,
        "step_ms_events": round(med(step_s) * 1e3, 4),
        "ceilings": ceilings,
        "hop_drift": drift,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def trace_summary(trace_dir, bench_json, warmup, steps):
    """Per-kernel durations of the step's timed dispatches from the kernel
    trace of a profiled bench run. The step runs before anything else in the
    bench uses these kernels, so an op kernel's first warmup + steps
    dispatches are the step's (the card scan: two per step), the last
    `steps` of them the timed ones."""
    import csv
    import glob

    import numpy as np
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one kernel_trace.csv under {trace_dir}, found {files}")
    with open(files[0]) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))

    def durs(name, per_step=1):
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3 for r in rows
             if r["Kernel_Name"].startswith(("void kvc::(anonymous namespace)::" + name,
                                             "kvc::(anonymous namespace)::" + name))]
        n = (warmup + steps) * per_step
        if len(d) < n:
            raise SystemExit(f"{name}: {len(d)} dispatches, expected at least {n}")
        return d[warmup * per_step:n], d

    table = ["| kernel | op | dispatches (all) | mean, timed steps (us) | median, timed steps (us) | "
             "mean, all dispatches (us) |", "|---|---|---|---|---|---|"]
    op_mean = {}
    for o in OPS:
        total = 0.0
        for kname in OP_KERNELS[o]:
            t, allv = durs(kname)
            total += float(np.mean(t))
            table.append(f"| {kname} | {o} | {len(allv)} | {np.mean(t):.1f} | {np.median(t):.1f} | "
                         f"{np.mean(allv):.1f} |")
        op_mean[o] = total
    print("\n".join(table))
    line = None
    if bench_json:
        with open(bench_json) as f:
            line = json.loads([ln for ln in f.read().splitlines() if ln.startswith("{")][-1])
    print()
    print("| op | sum of kernel means (us) | bench event mean (us) | frac of 8 TB/s from the trace | "
          "from the events |")
    print("|---|---|---|---|---|")
    for o in OPS:
        ev = line["ops"][o]["us_mean"] if line else float("nan")
        nbytes = line["ops"][o]["bytes"] if line else float("nan")
        print(f"| {o} | {op_mean[o]:.1f} | {ev:.1f} | {nbytes / op_mean[o] / 1e3 / HBM_PEAK_GBS:.4f} | "
              f"{nbytes / ev / 1e3 / HBM_PEAK_GBS:.4f} |")


def hop_drift(kv, synth, k, v, shape, widths_np, seed, stream, dev, hops=5):
    """Reconstruction error of a card passed along a chain of agents, each
    re-encoding it at its own widths (cachecard_transcode, then unpack to
    measure): sum of squared errors over sum of squares of the original K
    and V, after 0..hops hops, for uniform 4-bit, for one fixed mix of
    widths, and for a mix redrawn at every hop."""
    import numpy as np
    import torch
    L, H, T, d = shape
    ref = torch.stack([k.float(), v.float()])
    den = float((ref * ref).sum())
    card_cap = kv.cachecard_max_bytes(shape)
    cards = [torch.empty(card_cap, dtype=torch.uint8, device=dev) for _ in range(2)]
    cws = torch.empty(kv.cachecard_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    tws = torch.empty(kv.cachecard_transcode_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    ko, vo = torch.empty_like(k), torch.empty_like(v)
    schemes = {"uniform_4": lambda h: np.full(T, 4, np.uint8),
               "mixed_fixed": lambda h: widths_np,
               "mixed_redrawn": lambda h: synth.card_widths(synth.WORKLOADS[4], seed + 100 + h, T=T)}
    out = {}
    with torch.cuda.stream(stream):
        for name, wf in schemes.items():
            errs = []
            for h in range(hops + 1):
                w_np = wf(h)
                w = torch.from_numpy(w_np).to(dev)
                n = kv.cachecard_bytes_host(shape, w_np)
                cur, prev = cards[h % 2], cards[(h + 1) % 2]
                if h == 0:
                    kv.cachecard_pack(shape, k, v, w, cur, cws, b"chain", 0, stream=stream)
                else:
                    kv.cachecard_transcode(shape, prev, w, cur, tws, card_in_bytes=prev_n, stream=stream)
                kv.cachecard_unpack(shape, cur, ko, vo, cws, card_bytes=n, stream=stream)
                diff = torch.stack([ko.float(), vo.float()]) - ref
                errs.append(float((diff * diff).sum()) / den)
                prev_n = n
            out[name] = [float(f"{e:.4e}") for e in errs]
    return {"metric": "relative reconstruction MSE after 0..5 hops", **out}


CALIBRATION_BYTES = 1 << 30


def calibration_copies(dev, stream):
    """Three device copies of CALIBRATION_BYTES, whose FETCH_SIZE and
    WRITE_SIZE readings scale those counters to bytes."""
    import torch
    src = torch.empty(CALIBRATION_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    with torch.cuda.stream(stream):
        for _ in range(3):
            dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
CODEC_KERNELS = ["pool_decode_kernel", "fanout_copy_kernel", "pool_encode_fused_kernel", "pool_encode_layered_kernel",
                 "card_pack_kernel", "card_unpack_kernel", "card_scan_kernel",
                 "card_transcode_kernel", "realign_keys_kernel", "lowrank_materialize_kernel",
                 "fac_zx_kernel", "fac_ztq_kernel"]
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _counter_rows(folder, counter):
    """(kernel name, value) per dispatch, in dispatch order, from the
    counter_collection.csv rocprofv3 wrote under folder."""
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one counter_collection.csv under {folder}, found {files}")
    rows = []
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return [(n, v) for _, n, v in rows]


def other_configs(args):
    """Encode / decode (or pack / unpack) of the workloads other than the
    headline one, each timed alone (median of HIP events over repeated calls
    on one stream, inputs resident): the tiny pool, the SmolLM2-1.7B 2K pool
    (decode into one agent), the Llama-3-8B 32K pool (encode of the whole
    pool in one call, then the decode streamed one layer per call, the 32
    calls timed as one sequence, and the whole pool decoded in one call)
    and the Llama-3.1-8B 8K card."""
    import torch

    from agent_handoff_amd import kvcodec as kv
    from agent_handoff_amd import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def timed(fn, reps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        fn()
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) * 1e-3 for a, b in ev)
        return t[len(t) // 2]

    def emit(w, op, t, nbytes, **extra):
        gbs = nbytes / t / 1e9
        print(json.dumps({"workload": w.name, "op": op, "us": round(t * 1e6, 2), "bytes": int(nbytes),
                          "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), **extra}), flush=True)

    for cfg in (1, 2, 5):
        w = synth.WORKLOADS[cfg]
        L, H, T, d = shape = w.shape
        log(f"generating {w.name} inputs on the GPU")
        k, v = synth.kv_tensors_torch(w, args.seed, dev)
        kv_bytes = L * H * T * d * 2
        pool_b = pool_payload_bytes(*shape)
        pool = torch.empty(kv.kvpool_bytes(shape), dtype=torch.uint8, device=dev)
        ws = torch.zeros(kv.kvpool_workspace_bytes(shape), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        reps = 20 if cfg != 5 else 8
        te = timed(lambda: kv.kvpool_encode(shape, k, v, pool, ws, stream=stream), reps)
        emit(w, "encode", te, 2 * kv_bytes + pool_b,
             path="single pass" if cfg != 5 else "layered (a layer exceeds one round)")
        if cfg == 5:
            ko = torch.empty((1, H, T, d), dtype=torch.bfloat16, device=dev)
            vo = torch.empty_like(ko)

            def dec():
                for l in range(L):
                    kv.kvpool_decode(shape, pool, l, l + 1, [ko], [vo], status, stream=stream)
            td = timed(dec, reps)
            emit(w, "decode, one layer per call (32 calls)", td, pool_b + 2 * kv_bytes)
            del ko, vo
            # and the whole pool in one call (4.3 GB of bf16 out)
            ko, vo = torch.empty_like(k), torch.empty_like(v)
            td = timed(lambda: kv.kvpool_decode(shape, pool, 0, L, [ko], [vo], status, stream=stream), reps)
            emit(w, "decode, one agent, all layers in one call", td, pool_b + 2 * kv_bytes)
            del ko, vo
        else:
            ko, vo = torch.empty_like(k), torch.empty_like(v)
            td = timed(lambda: kv.kvpool_decode(shape, pool, 0, L, [ko], [vo], status, stream=stream), reps)
            emit(w, "decode, one agent", td, pool_b + 2 * kv_bytes)
            del ko, vo
        del k, v, pool, ws
        torch.cuda.empty_cache()

    w = synth.WORKLOADS[4]
    L, H, T, d = shape = w.shape
    log(f"generating {w.name} inputs on the GPU")
    k, v = synth.kv_tensors_torch(w, args.seed, dev)
    kv_bytes = L * H * T * d * 2
    widths_np = synth.card_widths(w, args.seed, T=T)
    widths = torch.from_numpy(widths_np).to(dev)
    card_n = kv.cachecard_bytes_host(shape, widths_np)
    card = torch.empty(card_n, dtype=torch.uint8, device=dev)
    cws = torch.empty(kv.cachecard_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    ko, vo = torch.empty_like(k), torch.empty_like(v)
    torch.cuda.synchronize()
    tp = timed(lambda: kv.cachecard_pack(shape, k, v, widths, card, cws, b"llama-3.1-8b", 0, None, status,
                                         stream=stream), 20)
    emit(w, "card pack", tp, 2 * kv_bytes + card_n, card_bytes=card_n)
    tu = timed(lambda: kv.cachecard_unpack(shape, card, ko, vo, cws, card_n, status, stream=stream), 20)
    emit(w, "card unpack", tu, card_n + 2 * kv_bytes, card_bytes=card_n)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "device status set"
    del k, v, card, ko, vo
    torch.cuda.empty_cache()
    if args.calibrate_copy:
        calibration_copies(dev, stream)


def traffic_from_counters(fetch_dir, write_dir, out_path, agents):
    """HBM bytes per dispatch of each codec kernel: the FETCH_SIZE and
    WRITE_SIZE counters (KiB per dispatch, separate runs), each scaled by
    known bytes / counter reading of the last three calibration copies."""
    import numpy as np

    from agent_handoff_amd import kvcodec as kv
    res = {}
    factors = {}
    for counter, folder in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(folder, counter)
        copies = [v for n, v in rows if n.startswith(COPY_KERNEL)][-3:]
        if len(copies) != 3:
            raise SystemExit(f"{counter}: calibration copies not found")
        kib = float(np.median(copies))
        factors[counter] = CALIBRATION_BYTES / (kib * 1024.0)
        for k in CODEC_KERNELS:
            vals = [v for n, v in rows if k + "<" in n or k + "(" in n]
            if vals:
                res.setdefault(k, {})[counter] = {"kib_per_dispatch": float(np.median(vals)), "dispatches": len(vals)}
    sha = _lib_sha(kv.LIB_PATH)
    out = {"_calibration": {"copy_bytes": CALIBRATION_BYTES, "copy_kernel": COPY_KERNEL,
                            "factor": {c: round(f, 5) for c, f in factors.items()}}}
    lines = ["| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled HBM bytes / dispatch |",
             "|---|---|---|---|---|"]
    for k, e in res.items():
        if "FETCH_SIZE" not in e or "WRITE_SIZE" not in e:
            continue
        fb = e["FETCH_SIZE"]["kib_per_dispatch"] * 1024.0 * factors["FETCH_SIZE"]
        wb = e["WRITE_SIZE"]["kib_per_dispatch"] * 1024.0 * factors["WRITE_SIZE"]
        out[k] = {"library_sha": sha, "agents": agents, "fetch_bytes": round(fb), "write_bytes": round(wb),
                  "bytes_per_dispatch": round(fb + wb),
                  "fetch_kib_raw": e["FETCH_SIZE"]["kib_per_dispatch"],
                  "write_kib_raw": e["WRITE_SIZE"]["kib_per_dispatch"]}
        lines.append(f"| {k} | {e['FETCH_SIZE']['dispatches']} | {e['FETCH_SIZE']['kib_per_dispatch']:.0f} | "
                     f"{e['WRITE_SIZE']['kib_per_dispatch']:.0f} | {fb + wb:.4g} |")
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    print("\n".join(lines))
    print(f"copy factors: {factors}; library sha {sha}")


def traffic_runs(fetch_dir, write_dir):
    """FETCH_SIZE and WRITE_SIZE per dispatch (medians, scaled to bytes as in
    traffic_from_counters) for each run of consecutive dispatches of one
    codec kernel with one grid size: the workloads of an --other-configs run
    call the same kernels in turn."""
    import csv
    import glob
    import re

    import numpy as np
    runs = {}
    factors = {}
    for counter, folder in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
        if len(files) != 1:
            raise SystemExit(f"expected one counter_collection.csv under {folder}, found {files}")
        with open(files[0]) as f:
            rows = sorted((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"]))
                          for r in csv.DictReader(f) if r["Counter_Name"] == counter)
        copies = [v for _, n, _, v in rows if n.startswith(COPY_KERNEL)][-3:]
        if len(copies) != 3:
            raise SystemExit(f"{counter}: calibration copies not found")
        factors[counter] = CALIBRATION_BYTES / (float(np.median(copies)) * 1024.0)
        seq = []
        for _, n, g, v in rows:
            k = next((k for k in CODEC_KERNELS if k + "<" in n or k + "(" in n), None)
            if k is None:
                continue
            m = re.search(re.escape(k) + r"(<[^>]*>)?", n)
            name = m.group(0)
            if seq and seq[-1][0] == (name, g):
                seq[-1][1].append(v)
            else:
                seq.append(((name, g), [v]))
        runs[counter] = seq
    print("| kernel | grid (threads) | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | bytes read | bytes written |")
    print("|---|---|---|---|---|---|---|")
    for (key, fv), (key2, wv) in zip(runs["FETCH_SIZE"], runs["WRITE_SIZE"]):
        if key != key2:
            raise SystemExit("the two runs dispatched different kernels")
        fk, wk = float(np.median(fv)), float(np.median(wv))
        print(f"| {key[0]} | {key[1]} | {len(fv)} | {fk:.0f} | {wk:.0f} | {fk * 1024 * factors['FETCH_SIZE']:.4g} | "
              f"{wk * 1024 * factors['WRITE_SIZE']:.4g} |")
    print(f"copy factors: {factors}; library sha {_lib_sha(os.path.join(ROOT, 'agent_handoff_amd', 'libkvcodec.so'))}")


def _lib_sha(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _oracle_pass(kb, vb, widths_np, sub, agents, keep=False):
    """encode, decode (+ copies to the other agents' buffers), card pack and
    unpack with the CPU oracle; returns (seconds per op, card bytes,
    outputs if keep)."""
    import numpy as np

    import oracle
    t0 = time.perf_counter()
    pool = oracle.pool_encode(kb, vb)
    t1 = time.perf_counter()
    dk, dv = oracle.pool_decode(pool, sub)
    # one decode serves every agent; the other agents' buffers are filled by copies
    ck, cv = np.empty_like(dk), np.empty_like(dv)
    for _ in range(agents - 1):
        np.copyto(ck, dk)
        np.copyto(cv, dv)
    t2 = time.perf_counter()
    card = oracle.card_pack(kb, vb, widths_np, CARD_MODEL_ID, 0)
    t3 = time.perf_counter()
    uk, uv = oracle.card_unpack(card, sub)
    t4 = time.perf_counter()
    out = {"pool": pool, "k_dec": dk, "v_dec": dv, "card": card, "k_unp": uk, "v_unp": uv} if keep else None
    return {"encode": t1 - t0, "decode": t2 - t1, "pack": t3 - t2, "unpack": t4 - t3}, card.size, out


def parity_report(kb, vb, ref, snap):
    """The GPU step's outputs against the oracle's on the whole workload:
    mismatching pool and card bytes, the encoder's near-boundary counts
    (within 1e-5 of a decision), decoded values by bf16 ulp distance and the
    per-head reconstruction MSE (relative to the input's energy) of the GPU
    and the oracle decode."""
    import numpy as np

    import oracle
    from agent_handoff_amd.synth import bf16_bits_to_f32

    def ordered(b):
        b = b.astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)

    def ulp(a, b):
        d = np.abs(ordered(a) - ordered(b))
        return int(d.max()), int(np.count_nonzero(d == 1))

    def head_mse(x_bits, y_bits):
        L, H = x_bits.shape[:2]
        out = np.empty((L, H))
        for l in range(L):
            x = bf16_bits_to_f32(x_bits[l]).astype(np.float64)
            y = bf16_bits_to_f32(y_bits[l]).astype(np.float64)
            out[l] = np.sum((x - y) ** 2, axis=(1, 2)) / np.maximum(np.sum(x * x, axis=(1, 2)), 1e-300)
        return out

    nk, nv = oracle.pool_near_boundary(kb, vb, 1e-5)
    rep = {"pool_bytes_mismatched": int(np.count_nonzero(snap["pool"] != ref["pool"])),
           "card_bytes_mismatched": int(np.count_nonzero(snap["card"] != ref["card"])),
           "near_boundary_keys": nk, "near_boundary_value_coords": nv, "values": int(2 * kb.size)}
    for what, g, r in (("decode_k", snap["k_dec"], ref["k_dec"]), ("decode_v", snap["v_dec"], ref["v_dec"]),
                       ("unpack_k", snap["k_unp"], ref["k_unp"]), ("unpack_v", snap["v_unp"], ref["v_unp"])):
        worst, at1 = ulp(g, r)
        rep[what + "_max_ulp"] = worst
        rep[what + "_at_1_ulp"] = at1
    rel = 0.0
    for x, g, r in ((kb, snap["k_dec"], ref["k_dec"]), (vb, snap["v_dec"], ref["v_dec"])):
        mg, mr = head_mse(x, g), head_mse(x, r)
        rel = max(rel, float(np.max(np.abs(mg - mr) / np.maximum(mr, 1e-300))))
    rep["per_head_mse_max_rel_diff"] = float(f"{rel:.3e}")
    return rep


def cpu_baseline(k, v, widths_np, shape, layers, agents, snap=None):
    """The CPU oracle on the first `layers` layers of the same workload with
    every host thread, and on one layer with a single thread; the same
    algorithmic byte accounting as the GPU step. With the GPU step's outputs
    (snap) and the whole workload, also the parity report."""
    import numpy as np
    import torch

    import oracle
    L, H, T, d = shape

    def bits(t, n):
        return t[:n].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    def gbs(n, secs, card_bytes):
        kv_bytes = n * H * T * d * 2
        pool_b = pool_payload_bytes(n, H, T, d)
        nbytes = (2 * kv_bytes + pool_b) + (pool_b + agents * 2 * kv_bytes) + 2 * (2 * kv_bytes + card_bytes)
        return nbytes / secs / 1e9

    oracle.lib()
    threads = oracle.max_threads()
    kb, vb = bits(k, layers), bits(v, layers)
    # whole passes, repeated until about 10 s of CPU work; per-pass mean
    passes = []
    ref = None
    while not passes or (sum(sum(p.values()) for p in passes) < 10.0 and len(passes) < 50):
        secs, card_bytes, out = _oracle_pass(kb, vb, widths_np, (layers, H, T, d), agents, keep=not passes)
        ref = out if out is not None else ref
        passes.append(secs)
    secs = {o: sum(p[o] for p in passes) / len(passes) for o in passes[0]}
    total = sum(secs.values())
    oracle.set_threads(1)
    try:
        s1, c1, _ = _oracle_pass(kb[:1].copy(), vb[:1].copy(), widths_np, (1, H, T, d), agents)
    finally:
        oracle.set_threads(threads)
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    res = {"value": round(gbs(layers, total, card_bytes), 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "cpu": cpu_model,
           "sample": f"layers 0..{layers - 1} of {L} of the same workload: encode, decode + copies to "
                     f"{agents} agents, card pack, unpack; mean of {len(passes)} passes of {total:.2f} s",
           "seconds": {o: round(t, 3) for o, t in secs.items()},
           "single_thread": {"value": round(gbs(1, sum(s1.values()), c1), 3), "unit": "GB/s", "cores": 1,
                             "sample": f"layer 0 ({sum(s1.values()):.1f} s)"}}
    if snap is not None and layers == L:
        log("parity report: GPU step outputs against the oracle's")
        res["parity"] = parity_report(kb, vb, ref, snap)
    return res


if __name__ == "__main__":
    main()
