"""Benchmark of the MoE FFN layer forward pass on one MI355X.

A step is one full layer forward (router -> top-k -> dispatch -> experts +
shared expert -> combine) over one batch of seeded synthetic inputs already
resident in HBM, through the C ABI (hy_moe_forward_ex, automatic path choice,
caller workspace). Default workload: the Hy4-shape decode layer (T=32 tokens,
d=6144, 256 routed experts top-8 + 1 shared, I=2048, bf16), which is bound by
streaming every touched expert's weights from HBM. The same run also measures
the prefill layer (T=8192), bound by bf16 MFMA, because the headline metric
names both.

Prints one JSON line. Per-kernel durations come from HIP events the library
records on its stream around each kernel (stage_events), over the timed steps.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; %bf16 MFMA peak (T=8192), %HBM BW (T=32)"
PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E
PEAK_BF16 = 2.5e15         # flop/s, MI355X dense bf16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Events:
    """hipEvent_t handles from the HIP runtime torch loaded (same process runtime)."""

    def __init__(self, n):
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.handles = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.rt.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.handles.append(h.value)

    def array(self, i, m):
        return (ctypes.c_void_p * m)(*self.handles[i * m:(i + 1) * m])

    def ms(self, a, b):
        out = ctypes.c_float()
        if self.rt.hipEventElapsedTime(ctypes.byref(out), self.handles[a], self.handles[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def close(self):
        for h in self.handles:
            self.rt.hipEventDestroy(h)


def source_digest(path):
    """sha256 (first 16 hex digits) of a C/HIP source with comments and whitespace
    removed: the code that the counters were taken on, not its commentary."""
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256("".join(text.split()).encode()).hexdigest()[:16]


def traffic_for(kernel_key, units):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when
    absent or taken on a different version of the kernel's source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        rec = json.load(open(TRAFFIC_FILE)).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec:
        return None
    src = os.path.join(ROOT, rec["source"])
    if not os.path.exists(src) or source_digest(src) != rec["source_sha256_16"]:
        return None
    return rec["bytes_per_launch"]


WARMUP_MIN_S = 0.5  # default warm-up length: the shader clock climbs for ~60 ms of load after idle


def time_layer(hm, torch, inp, k, ws, steps, warmup, dominant):
    """Times `steps` forwards after `warmup` untimed ones (None: at least 5 steps and
    WARMUP_MIN_S seconds of them). Returns (total ms by the host clock around the syncs,
    mean ms of kernel `dominant` from events recorded around it in those same steps,
    mean ms per kernel from a separate pass of stage events after the timed region,
    warm-up steps run). Only the dominant kernel's two events are recorded while timing:
    an event between every kernel would add its own gaps to the step."""
    nk = len(hm.KERNELS)
    done = 0
    t_w = time.perf_counter()
    if warmup is not None:
        for _ in range(warmup):
            hm.forward_layer(inp, k, workspace=ws)
        done = warmup
    else:
        while done < 5 or time.perf_counter() - t_w < WARMUP_MIN_S:
            for _ in range(5):
                hm.forward_layer(inp, k, workspace=ws)
            done += 5
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = Events(2 * steps)
    arrays = []
    for i in range(steps):
        arr = (ctypes.c_void_p * (nk + 1))()
        arr[dominant] = ev.handles[2 * i]
        arr[dominant + 1] = ev.handles[2 * i + 1]
        arrays.append(arr)
    t0 = time.perf_counter()
    for i in range(steps):
        hm.forward_layer(inp, k, workspace=ws, stage_events=arrays[i])
    torch.cuda.synchronize()
    total_ms = (time.perf_counter() - t0) * 1e3
    dom_ms = sum(ev.ms(2 * i, 2 * i + 1) for i in range(steps)) / steps
    ev.close()
    # per-kernel breakdown (untimed)
    nb = min(steps, 20)
    ev = Events((nk + 1) * nb)
    for i in range(nb):
        hm.forward_layer(inp, k, workspace=ws, stage_events=ev.array(i, nk + 1))
    torch.cuda.synchronize()
    per = [0.0] * nk
    for i in range(nb):
        for j in range(nk):
            per[j] += ev.ms(i * (nk + 1) + j, i * (nk + 1) + j + 1) / nb
    ev.close()
    return total_ms, dom_ms, dict(zip(hm.KERNELS, per)), done


def stream_work(cfg, touched):
    """Algorithmic HBM bytes of a decode-size layer on the streaming path with `touched`
    routed experts: the dominant gate/up launch (one unit per touched routed expert,
    plus the shared expert) and the whole layer (every touched expert's weights once,
    the router, x and the output)."""
    d, I = cfg.d, cfg.I
    if cfg.ternary:
        unit = 2 * I * (d // 128 * 5 * 4) + 2 * I * 2    # packed codes + bf16 row scales
        shared = 2 * I * d * 2
        alg = touched * unit + shared
        per_unit = f"{unit} B packed gate+up codes and scales per touched routed expert, plus {shared} B bf16 shared"
        layer_bytes = touched * (3 * I * (d // 128 * 5 * 4) + 2 * I * 2 + d * 2) + 3 * I * d * 2
    elif cfg.fp8:
        unit = 2 * I * d + 2 * I * 4                    # E4M3 codes + fp32 row scales
        shared = 2 * I * d * 2
        alg = touched * unit + shared
        per_unit = f"{unit} B of E4M3 gate+up codes and scales per touched routed expert, plus {shared} B bf16 shared"
        layer_bytes = touched * (3 * I * d + (2 * I + d) * 4) + 3 * I * d * 2
    else:
        unit = 2 * I * d * 2
        alg = (touched + 1) * unit
        per_unit = f"{unit} B of bf16 gate+up weights per touched expert (routed + shared)"
        layer_bytes = (touched + 1) * 3 * I * d * 2
    layer_bytes += cfg.E * d * 2 + 2 * cfg.T * d * 2
    # ternary weights with d and I multiples of 512 run in the LDS-staged kernel
    tern_lds = cfg.ternary and d % 512 == 0 and I % 512 == 0
    kernel = ("tern_lds_kernel<2>" if tern_lds else "stream_gateup_kernel<2> (FP8 routed experts)" if cfg.fp8
              else "stream_gateup_kernel")
    return {"unit": unit, "alg": alg, "per_unit": per_unit, "layer_bytes": layer_bytes,
            "key": "ternary_gateup" if tern_lds else "stream_gateup", "kernel": kernel}


def gemm_work(cfg):
    """Algorithmic flops of a layer on the grouped path: the dominant gate/up stage
    (4 d I per dispatched row, routed and shared) and the whole layer (router + all
    three expert products)."""
    d, I = cfg.d, cfg.I
    rows = cfg.T * cfg.k + cfg.T
    kernel = ("grouped_gemm_kernel<true, 0, 1> (ternary routed tiles) + grouped_gemm_kernel<true, 0, 0> "
              "(bf16 shared tiles): one timed stage" if cfg.ternary else
              "grouped_gemm_kernel<true, 0, 2> (FP8 routed tiles) + grouped_gemm_kernel<true, 0, 0> "
              "(bf16 shared tiles): one timed stage" if cfg.fp8 else "grouped_gemm_kernel<true, 0, 0>")
    return {"rows": rows, "alg": 4 * rows * d * I, "layer_flop": 2 * cfg.T * d * cfg.E + 6 * rows * d * I,
            "per_unit": f"{4 * d * I} flop per dispatched row (gate and up: 2*d*I each)", "kernel": kernel}


def run_config(name, args, hi, hm, torch, weights=None):
    cfg = hi.CONFIGS[name]
    dev = "cuda:0"
    if weights is None:
        log(f"[bench] generating inputs for {name} on the GPU")
        inp = hi.dev_layer(cfg, device=dev)
    else:
        inp = dict(weights)
        inp["x"] = weights["x"][: cfg.T].contiguous()
        b = hi.host_bias(cfg)
        inp["bias"] = None if b is None else torch.from_numpy(b).to(dev)
    fmt = hm.WEIGHTS_SHERRY_TERNARY if cfg.ternary else hm.WEIGHTS_FP8_E4M3 if cfg.fp8 else hm.WEIGHTS_BF16
    ws = hm.alloc_workspace(cfg.T, cfg.d, cfg.E, cfg.k, cfg.I, fmt, device=dev)
    steps = args.steps
    dominant = hm.KERNELS.index("expert_gateup")
    total_ms, dom_ms, kern, warmup_done = time_layer(hm, torch, inp, cfg.k, ws, steps, args.warmup, dominant)
    ms = total_ms / steps
    routing = hm.forward_layer(inp, cfg.k, want_routing=True, workspace=ws)
    torch.cuda.synchronize()
    counts = routing["counts"].cpu()
    touched = int((counts > 0).sum())
    stream_path = cfg.T * cfg.k <= 16 * cfg.E  # the library's automatic path choice
    kernel_file = "sparse_moe_transformer_route_amd/csrc/" + ("moe_stream.hip" if stream_path else "moe_gemm.hip")
    if stream_path:
        w = stream_work(cfg, touched)
        sec = dom_ms * 1e-3
        alg = w["alg"]
        roof = {"bound": "hbm", "achieved": alg / sec / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                "frac": alg / sec / PEAK_HBM, "traffic": traffic_for(f"{w['key']}/{name}", touched + 1),
                "kernel": w["kernel"], "per_unit": w["per_unit"], "units_per_launch": touched + 1, "kernel_ms": dom_ms}
        layer = {"bytes": w["layer_bytes"], "hbm_frac": w["layer_bytes"] / (ms * 1e-3) / PEAK_HBM}
    else:
        w = gemm_work(cfg)
        rows, alg = w["rows"], w["alg"]
        sec = dom_ms * 1e-3
        roof = {"bound": "mfma", "achieved": alg / sec / 1e12, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                "frac": alg / sec / PEAK_BF16, "traffic": traffic_for(f"grouped_gemm_gateup/{name}", rows),
                "kernel": w["kernel"], "per_unit": w["per_unit"], "units_per_launch": rows, "kernel_ms": dom_ms}
        layer = {"flop": w["layer_flop"], "mfma_frac": w["layer_flop"] / (ms * 1e-3) / PEAK_BF16}
    roof["kernel_source_sha256_16"] = source_digest(os.path.join(ROOT, kernel_file))
    return {"cfg": cfg, "inp": inp, "ms": ms, "tokens_per_s": cfg.T / (ms * 1e-3), "kernels_ms": kern,
            "roofline": roof, "layer": layer, "touched": touched, "counts": counts, "routing": routing,
            "warmup": warmup_done}


def cpu_baseline(cfg, hi, torch, inp, routing, budget_s):
    """The oracle timed on this host's cores on the first tokens of the same batch.
    Expert weights are copied from the device tensors (generator output, never
    the HIP path's results); only the oracle's calls are timed."""
    import numpy as np

    import oracle
    nthreads = max(1, min(16, os.cpu_count() or 1))

    def bits(t):
        return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    x = bits(inp["x"])
    wr = bits(inp["router"])
    bias = None if inp.get("bias") is None else inp["bias"].cpu().numpy()
    sh = {key: bits(v) for key, v in inp["shared"].items()}
    sets_all = routing["topk_idx"].cpu().numpy()
    cache = {}

    def expert(e):
        # bf16 weights of routed expert e; Sherry and FP8 codes are decoded by the
        # oracle here, outside the timed region (weight materialisation)
        if e not in cache:
            if "fgate" in inp:
                cache[e] = tuple(oracle.fp8_decode(inp[q][e].cpu().numpy(), inp[s][e].cpu().numpy())
                                 for q, s in (("fgate", "fsgate"), ("fup", "fsup"), ("fdown", "fsdown")))
            elif "qgate" in inp:
                cache[e] = tuple(oracle.sherry_decode(inp[q][e].cpu().numpy().view(np.uint32), bits(inp[s][e]))[1]
                                 for q, s in (("qgate", "sgate"), ("qup", "sup"), ("qdown", "sdown")))
            else:
                cache[e] = tuple(bits(inp[key][e]) for key in ("gate", "up", "down"))
        return cache[e]

    def oracle_tokens(tok):
        for t in tok:
            for e in sets_all[t]:
                expert(int(e))
        t0 = time.perf_counter()
        lg = oracle.logits(x[tok], wr, bias, nthreads=nthreads)
        sets, _ = oracle.select(lg, cfg.k)
        w = oracle.weights(lg, sets)
        ys = oracle.ffn(x[tok], sh["gate"], sh["up"], sh["down"], nthreads=nthreads)
        yr = np.zeros((len(tok), cfg.k, cfg.d))
        for i in range(len(tok)):
            for j, e in enumerate(sets[i]):
                g, u, dn = expert(int(e))
                ffn = oracle.ffn_w64 if "fgate" in inp else oracle.ffn
                yr[i, j] = ffn(x[tok[i]:tok[i] + 1], g, u, dn, nthreads=nthreads)[0]
        oracle.combine(ys, yr, w)
        return time.perf_counter() - t0

    first = oracle_tokens([0])
    n = max(1, min(cfg.T, int(budget_s / max(first, 1e-3))))
    if n < cfg.T:
        tok = list(range(1, 1 + n))
        el = oracle_tokens(tok)
        done, what = len(tok), f"{len(tok)} of the {cfg.T} tokens of the same batch"
    else:
        # the whole batch is cheaper than the budget: repeat full passes over it
        tok = list(range(cfg.T))
        el, passes = 0.0, 0
        while passes == 0 or el < budget_s:
            el += oracle_tokens(tok)
            passes += 1
        done, what = passes * cfg.T, f"{passes} passes over all {cfg.T} tokens of the same batch"
    return {"value": done / el, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{what} (full fp64 layer per token: router over {cfg.E} experts, top-{cfg.k}, "
                      f"{cfg.k} routed + 1 shared SwiGLU experts, combine); {el:.1f} s on {nthreads} threads"}


def run_indexer(args, hi, hm, torch):
    """The sparse-attention indexer of one full layer over B decoding sequences: every
    query scores its sequence's S keys and keeps the top K (hy_indexer_topk)."""
    import numpy as np
    cfg = hi.INDEXER_CONFIGS[args.config]
    log(f"[bench] generating the indexer inputs (B={cfg.B}, S={cfg.S}) on the GPU")
    inp = hi.dev_indexer(cfg, device="cuda:0")
    ws = torch.empty(hm.lib().hy_indexer_workspace_size(cfg.B, cfg.S), dtype=torch.uint8, device="cuda:0")
    torch.cuda.synchronize()

    def call(ev=None):
        return hm.indexer_topk(inp["q"], inp["w"], inp["keys"], cfg.K, workspace=ws, stage_events=ev)

    done, t_w = 0, time.perf_counter()
    while (args.warmup is None and (done < 5 or time.perf_counter() - t_w < WARMUP_MIN_S)) or \
            (args.warmup is not None and done < args.warmup):
        call()
        done += 1
        if done % 5 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    steps = args.steps
    ev = Events(3 * steps)
    arrays = [ev.array(i, 3) for i in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        idx, _ = call(arrays[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    score_ms = sum(ev.ms(3 * i, 3 * i + 1) for i in range(steps)) / steps
    select_ms = sum(ev.ms(3 * i + 1, 3 * i + 2) for i in range(steps)) / steps
    ev.close()
    B, S, H, D = cfg.B, cfg.S, cfg.H, cfg.D
    unit = S * D * 2 + S * 4            # keys read + scores written per query
    alg = B * unit + B * H * D * 2 + B * H * 4
    roof = {"bound": "hbm", "achieved": alg / (score_ms * 1e-3) / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
            "frac": alg / (score_ms * 1e-3) / PEAK_HBM, "traffic": traffic_for(f"indexer_scores/{cfg.name}", B),
            "kernel": "indexer_scores_kernel<128>", "per_unit": f"{unit} B per query (its {S} keys of {D} bf16, its "
            f"{S} fp32 scores), plus the queries and head weights", "units_per_launch": B, "kernel_ms": score_ms,
            "kernel_source_sha256_16": source_digest(os.path.join(ROOT, "sparse_moe_transformer_route_amd/csrc/"
                                                                  "hy_indexer.hip"))}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("[bench] timing the oracle on the host")
        q, w = hi.host_indexer_queries(cfg)
        el, nq = 0.0, 0
        while nq == 0 or (el < args.cpu_seconds and nq < B):
            keys = hi.host_indexer_keys(cfg, nq)   # generation is not timed
            t1 = time.perf_counter()
            sc = oracle.indexer_scores(q[nq:nq + 1], w[nq:nq + 1], keys[None])
            oracle.topk_indices(sc, cfg.K)
            el += time.perf_counter() - t1
            nq += 1
        cpu = {"value": nq / el, "unit": "queries/s", "cores": 1, "kind": "oracle",
               "sample": f"{nq} of the {B} queries (fp64 scores of all {S} keys and the top-{cfg.K} sort each); "
                         f"{el:.1f} s on 1 thread"}
    log(f"[bench] {cfg.name}: {ms:.3f} ms/step, {B / (ms * 1e-3):.0f} queries/s, scoring {score_ms:.4f} ms, "
        f"selection {select_ms:.4f} ms")
    line = {
        "metric": "sparse-attention indexer throughput (one full indexer layer)", "value": B / (ms * 1e-3),
        "unit": "queries/s", "n_gpus": 1, "steps": steps, "warmup": done, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: B={B} sequences x S={S} keys, H={H} heads, D={D}, top-{cfg.K}",
                   "B": B, "S": S, "H": H, "D": D, "K": cfg.K, "seed": cfg.seed},
        "roofline": roof, "kernels_ms": {"indexer_scores": score_ms, "indexer_topk": select_ms},
        "indexcache": {"layers": 78, "full_layers": 21, "ms_per_step_all_layers": 21 * ms,
                       "note": "57 of 78 layers reuse the previous layer's selection and run no indexer kernel"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default: at least 5 and %.1f s of them)" % WARMUP_MIN_S)
    ap.add_argument("--config", default="decode", choices=["tiny", "decode", "prefill", "skewed", "ternary",
                                                                 "ternary_prefill", "fp8", "fp8_prefill",
                                                                 "indexer_tiny", "indexer_decode"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the T=8192 measurement")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy-gib", type=float, default=0.0,
                    help="only run 3 device-to-device copies of this many GiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the layer has no multi-GPU "
              f"path: sharding by expert is designed, not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch

    import hy_inputs as hi
    import sparse_moe_transformer_route_amd as hm
    torch.cuda.set_device(0)
    if args.calibrate_copy_gib > 0:
        n = int(args.calibrate_copy_gib * 2 ** 30)
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read_per_copy": n, "bytes_written_per_copy": n}))
        return

    if args.config.startswith("indexer"):
        run_indexer(args, hi, hm, torch)
        return
    cfg = hi.CONFIGS[args.config]
    shared_weights = None
    if not cfg.ternary and not cfg.fp8 and cfg.d == 6144:
        log("[bench] generating the Hy4-shape bf16 layer (19.3 GB of expert weights) on the GPU")
        shared_weights = hi.dev_layer(hi.CONFIGS["prefill"], device="cuda:0")
        torch.cuda.synchronize()
    main_res = run_config(args.config, args, hi, hm, torch, shared_weights)
    log(f"[bench] {args.config}: {main_res['ms']:.3f} ms/step, {main_res['tokens_per_s']:.1f} tokens/s, "
        f"kernels {json.dumps({k: round(v, 4) for k, v in main_res['kernels_ms'].items()})}")

    extra = {}
    if args.config == "decode" and not args.no_prefill:
        pre_args = argparse.Namespace(**vars(args))
        pre_args.steps = min(args.steps, 10)
        pre = run_config("prefill", pre_args, hi, hm, torch, shared_weights)
        log(f"[bench] prefill: {pre['ms']:.3f} ms/step, {pre['tokens_per_s']:.0f} tokens/s")
        extra["prefill"] = {"workload": "prefill T=8192 d=6144 E=256 k=8 I=2048 bf16", "ms_per_step": pre["ms"],
                            "steps": pre_args.steps, "warmup": pre["warmup"],
                            "tokens_per_s": pre["tokens_per_s"], "layer_mfma_frac": pre["layer"]["mfma_frac"],
                            "roofline": pre["roofline"], "kernels_ms": pre["kernels_ms"]}
        del pre
        torch.cuda.empty_cache()

    # measured peaks next to the published ones: bf16 MFMA on random operand bits (the
    # power-capped clock depends on operand activity) and one streaming read of HBM
    gen = torch.Generator(device="cuda:0").manual_seed(0)
    ops = torch.randn(hm.PROBE_OPERAND_BYTES // 2, generator=gen, device="cuda:0").to(torch.bfloat16)
    read_buf = shared_weights["gate"] if shared_weights is not None else torch.empty(4 << 30, dtype=torch.uint8,
                                                                                     device="cuda:0")
    peaks = {"mfma_bf16_tflops": hm.probe_mfma_bf16(ops), "hbm_read_gbs": hm.probe_hbm_read(read_buf),
             "hbm_read_bytes": read_buf.numel() * read_buf.element_size(),
             "how": "hy_moe_probe_mfma_bf16 (32x32x16 bf16 MFMAs, 4 workgroups per CU, random N(0,1) operands, "
                    "~40 ms) and hy_moe_probe_hbm_read (best of three timed streaming passes of 16-byte loads after "
                    "an untimed one)"}
    del read_buf
    log(f"[bench] measured peaks: {peaks['mfma_bf16_tflops']:.0f} TFLOP/s bf16 MFMA, "
        f"{peaks['hbm_read_gbs']:.0f} GB/s HBM read")
    roof = main_res["roofline"]
    meas = peaks["hbm_read_gbs"] if roof["unit"] == "GB/s" else peaks["mfma_bf16_tflops"]
    roof["frac_of_measured_peak"] = roof["achieved"] / meas
    if "prefill" in extra:
        extra["prefill"]["roofline"]["frac_of_measured_peak"] = (extra["prefill"]["roofline"]["achieved"]
                                                                 / peaks["mfma_bf16_tflops"])

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host")
        cpu = cpu_baseline(cfg, hi, torch, main_res["inp"], main_res["routing"], args.cpu_seconds)

    c = main_res["cfg"]
    line = {
        "metric": METRIC, "value": main_res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": main_res["warmup"], "ms_per_step": main_res["ms"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "sherry-ternary+bf16" if c.ternary else "fp8-e4m3+bf16" if c.fp8 else "bf16", "data": "synthetic",
        "config": {"workload": f"{c.name} MoE FFN layer T={c.T} d={c.d} E={c.E} top-{c.k} + 1 shared I={c.I}"
                               + (" Sherry-ternary routed experts" if c.ternary else " bf16")
                               + (" Zipf(1.2) router bias" if c.zipf_s else ""),
                   "T": c.T, "d": c.d, "E": c.E, "k": c.k, "I": c.I, "seed": c.seed,
                   "touched_experts": main_res["touched"]},
        "roofline": main_res["roofline"],
        "layer": main_res["layer"],
        "kernels_ms": main_res["kernels_ms"],
        "measured_peak": peaks,
        "cpu_baseline": cpu,
    }
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
