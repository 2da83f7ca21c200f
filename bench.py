"""Benchmark of the MoE FFN layer forward pass on one MI355X.

A step is one full layer forward (router -> top-k -> dispatch -> experts +
shared expert -> combine) over one batch of seeded synthetic inputs already
resident in HBM, through the C ABI (hy_moe_forward_ex, automatic path choice,
caller workspace). The headline workload is the Hy4-shape decode layer (T=32
tokens, d=6144, 256 routed experts top-8 + 1 shared, I=2048, bf16), bound by
streaming every touched expert's weights from HBM. The default run also times
the layer's other workloads, each as an object of the same JSON line: the tiny
layer, the prefill layer (T=8192, bound by bf16 MFMA), the skewed-routing
prefill (T=4096, Zipf router bias) and the Sherry-ternary decode layer.

Per workload: W untimed warm-up steps, then K timed steps; ms_per_step is the
host clock around the K steps (synchronised on both sides); the per-step median
and p10/p90 come from HIP events recorded on the library's stream at each
step's first and last kernel; the dominant kernel's time from events around it
in the same steps. Before the first workload the machine-peak probes run, which
also brings the shader clock up from idle. Prints one JSON line.
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
PEAK_FP8 = 5.0e15          # flop/s, MI355X dense fp8 MFMA
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


def _pct(vals, q):
    v = sorted(vals)
    if not v:
        return None
    pos = (len(v) - 1) * q
    lo, hi = int(math.floor(pos)), int(math.ceil(pos))
    return v[lo] + (v[hi] - v[lo]) * (pos - lo)


def step_stats(vals):
    return {"median": _pct(vals, 0.5), "p10": _pct(vals, 0.1), "p90": _pct(vals, 0.9), "n": len(vals)}


def time_layer(hm, torch, inp, k, ws, steps, warmup, dominant, flush=None, fwd_kw=None):
    """Times `steps` forwards after `warmup` untimed ones (None: at least 5 steps and
    WARMUP_MIN_S seconds of them). Returns dict(total_ms by the host clock around the
    synchronised steps, step_ms (per step, from events at the first and last kernel of
    the step), dom_ms (per step, events around kernel `dominant`), kernels (mean ms per
    kernel from a separate pass of stage events after the timed region), warmup (steps
    run), cold_ms (per step with `flush` run between steps outside the events, or None)).
    Only the step's two ends and the dominant kernel's two ends are recorded while
    timing: an event between every kernel would add its own gaps to the step.
    fwd_kw: extra keyword arguments of every forward_layer call."""
    nk = len(hm.KERNELS)
    kw = dict(fwd_kw or {})
    done = 0
    t_w = time.perf_counter()
    if warmup is not None:
        for _ in range(warmup):
            hm.forward_layer(inp, k, workspace=ws, **kw)
        done = warmup
    else:
        while done < 5 or time.perf_counter() - t_w < WARMUP_MIN_S:
            for _ in range(5):
                hm.forward_layer(inp, k, workspace=ws, **kw)
            done += 5
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = Events(4 * steps)
    arrays = []
    for i in range(steps):
        arr = (ctypes.c_void_p * (nk + 1))()
        arr[0] = ev.handles[4 * i]
        arr[nk] = ev.handles[4 * i + 1]
        arr[dominant] = ev.handles[4 * i + 2] if dominant > 0 else arr[0]
        arr[dominant + 1] = ev.handles[4 * i + 3] if dominant + 1 < nk else arr[nk]
        arrays.append(arr)
    t0 = time.perf_counter()
    for i in range(steps):
        hm.forward_layer(inp, k, workspace=ws, stage_events=arrays[i], **kw)
    torch.cuda.synchronize()
    total_ms = (time.perf_counter() - t0) * 1e3
    step_ms = [ev.ms(4 * i, 4 * i + 1) for i in range(steps)]
    da = (lambda i: 4 * i + 2) if dominant > 0 else (lambda i: 4 * i)
    db = (lambda i: 4 * i + 3) if dominant + 1 < nk else (lambda i: 4 * i + 1)
    dom_ms = [ev.ms(da(i), db(i)) for i in range(steps)]
    cold = None
    if flush is not None:
        # the same steps with a cache-flushing write between them (outside the events)
        cold = []
        for i in range(steps):
            flush()
            hm.forward_layer(inp, k, workspace=ws, stage_events=arrays[i], **kw)
        torch.cuda.synchronize()
        cold = [ev.ms(4 * i, 4 * i + 1) for i in range(steps)]
        cold_dom = [ev.ms(da(i), db(i)) for i in range(steps)]
    ev.close()
    # per-kernel breakdown (untimed)
    nb = min(steps, 20)
    ev = Events((nk + 1) * nb)
    for i in range(nb):
        hm.forward_layer(inp, k, workspace=ws, stage_events=ev.array(i, nk + 1), **kw)
    torch.cuda.synchronize()
    per = [0.0] * nk
    for i in range(nb):
        for j in range(nk):
            per[j] += ev.ms(i * (nk + 1) + j, i * (nk + 1) + j + 1) / nb
    ev.close()
    return {"total_ms": total_ms, "step_ms": step_ms, "dom_ms": dom_ms, "kernels": dict(zip(hm.KERNELS, per)),
            "warmup": done, "cold_ms": cold, "cold_dom_ms": cold_dom if cold is not None else None}


def stream_work(cfg, touched, blocked=False):
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
    kernel = (("tern_lds_kernel<2, true> (blocked Sherry codes)" if blocked else "tern_lds_kernel<2, false>")
              if tern_lds else "stream_gateup_kernel<2> (FP8 routed experts)" if cfg.fp8
              else "stream_gateup_kernel<3> (blocked bf16 weights)" if blocked else "stream_gateup_kernel<0>")
    return {"unit": unit, "alg": alg, "per_unit": per_unit, "layer_bytes": layer_bytes,
            "key": "ternary_gateup" if tern_lds else "stream_gateup", "kernel": kernel}


def gemm_work(cfg, blocked=False):
    """Algorithmic flops of a layer on the grouped path: the dominant gate/up stage
    (4 d I per dispatched row, routed and shared) and the whole layer (router + all
    three expert products)."""
    d, I = cfg.d, cfg.I
    rows = cfg.T * cfg.k + cfg.T
    kernel = (f"grouped_gemm_kernel<true, 0, {5 if blocked else 1}> (ternary routed tiles"
              f"{', blocked Sherry codes' if blocked else ''}) + grouped_gemm_kernel<true, 0, 0> "
              "(bf16 shared tiles): one timed stage" if cfg.ternary else
              "mx_quantize_kernel (token rows to MXFP8) + grouped_gemm_kernel<true, 0, 3> (FP8 MFMAs on the W8A8 "
              "routed tiles) + grouped_gemm_kernel<true, 0, 0> (bf16 shared tiles): one timed stage" if cfg.a8 else
              "grouped_gemm_kernel<true, 0, 2> (FP8 routed tiles) + grouped_gemm_kernel<true, 0, 0> "
              "(bf16 shared tiles): one timed stage" if cfg.fp8 else
              "grouped_gemm_kernel<true, 0, 4> (blocked bf16 weights)" if blocked else "grouped_gemm_kernel<true, 0, 0>")
    # W8A8: the routed rows run on FP8 MFMAs and the shared rows on bf16 ones, so the
    # stage's peak is the time both take at their own peaks
    routed, shared = cfg.T * cfg.k, cfg.T
    peak = rows / (routed / PEAK_FP8 + shared / PEAK_BF16) if cfg.a8 else PEAK_BF16
    layer_peak = ((2 * cfg.T * d * cfg.E + 6 * rows * d * I) /
                  ((2 * cfg.T * d * cfg.E + 6 * shared * d * I) / PEAK_BF16 + 6 * routed * d * I / PEAK_FP8)
                  if cfg.a8 else PEAK_BF16)
    return {"rows": rows, "alg": 4 * rows * d * I, "layer_flop": 2 * cfg.T * d * cfg.E + 6 * rows * d * I,
            "per_unit": f"{4 * d * I} flop per dispatched row (gate and up: 2*d*I each)", "kernel": kernel,
            "peak": peak, "layer_peak": layer_peak,
            "peak_how": (f"{routed} routed rows at the FP8 dense peak ({PEAK_FP8 / 1e15:.1f} PFLOP/s) and {shared} "
                         f"shared rows at the bf16 one ({PEAK_BF16 / 1e15:.1f}): total flops / the time both take "
                         f"at their peaks" if cfg.a8 else "bf16 dense MFMA peak")}


def measured_peak_of(roof, peaks):
    """The rate this GPU measured for a roofline's bound: HBM read for bytes, the bf16
    MFMA probe for flops, and for a W8A8 stage its rows at the FP8 and bf16 probes'
    rates combined as the published peaks are."""
    if roof["unit"] == "GB/s":
        return peaks["hbm_read_gbs"]
    mix = roof.get("peak_mix")
    if mix is None:
        return peaks["mfma_bf16_tflops"]
    return (mix["fp8_rows"] + mix["bf16_rows"]) / (mix["fp8_rows"] / peaks["mfma_fp8_tflops"] +
                                                   mix["bf16_rows"] / peaks["mfma_bf16_tflops"])


def input_digest(inp, torch):
    """sha256 (first 16 hex digits) of the step's inputs that are not regenerated by
    stream id alone: x, the router weights and the bias, plus the first routed expert's
    and the shared expert's weights as a check of the generator."""
    h = hashlib.sha256()
    keys = [k for k in ("x", "router", "bias") if inp.get(k) is not None]
    first = [k for k in ("gate", "qgate", "fgate") if k in inp][0]
    for t in [inp[k] for k in keys] + [inp[first][0]] + [inp["shared"][k] for k in ("gate", "up", "down")]:
        h.update(t.detach().contiguous().view(torch.uint8).cpu().numpy().tobytes())
    return h.hexdigest()[:16]


def run_config(name, args, hi, hm, torch, weights=None, steps=None, flush=None, blocked=False, rm_weights=None):
    """Times workload `name`. weights: a bf16 layer dict to take the expert weights from
    (already in the blocked layout when blocked is set; rm_weights then holds the same
    weights row-major). blocked: the blocked layout of bf16 weights
    (HY_MOE_WEIGHTS_BF16_BLOCKED) or of Sherry codes (HY_MOE_WEIGHTS_SHERRY_BLOCKED, d and I
    multiples of 512), converted once before anything is timed; FP8 workloads ignore it.
    res["inp_rm"] is the input set with row-major weights (what the oracle reads)."""
    cfg = hi.CONFIGS[name]
    dev = "cuda:0"
    bf16 = not cfg.ternary and not cfg.fp8
    blocked = blocked and (bf16 or (cfg.ternary and cfg.d % 512 == 0 and cfg.I % 512 == 0))

    def with_x(wts):
        d = dict(wts)
        d["x"] = wts["x"][: cfg.T].contiguous()
        b = hi.host_bias(cfg)
        d["bias"] = None if b is None else torch.from_numpy(b).to(dev)
        return d
    if weights is None:
        log(f"[bench] generating inputs for {name} on the GPU")
        inp_rm = hi.dev_layer(cfg, device=dev)
        inp = hm.block_layer(inp_rm) if blocked else inp_rm
    else:
        inp = with_x(weights)
        inp_rm = with_x(rm_weights) if blocked else inp
    fmt = ((hm.WEIGHTS_SHERRY_BLOCKED if blocked else hm.WEIGHTS_SHERRY_TERNARY) if cfg.ternary else
           hm.WEIGHTS_FP8_W8A8 if cfg.a8 else
           hm.WEIGHTS_FP8_E4M3 if cfg.fp8 else hm.WEIGHTS_BF16_BLOCKED if blocked else hm.WEIGHTS_BF16)
    fwd_kw = {"fp8_activations": True} if cfg.a8 else {"weights_blocked": True} if blocked else {}
    ws = hm.alloc_workspace(cfg.T, cfg.d, cfg.E, cfg.k, cfg.I, fmt, device=dev)
    steps = args.steps if steps is None else steps
    dominant = hm.KERNELS.index("expert_gateup")
    r = time_layer(hm, torch, inp, cfg.k, ws, steps, args.warmup, dominant, flush=flush, fwd_kw=fwd_kw)
    ms = r["total_ms"] / steps
    dom_ms = sum(r["dom_ms"]) / steps
    routing = hm.forward_layer(inp, cfg.k, want_routing=True, workspace=ws, **fwd_kw)
    torch.cuda.synchronize()
    counts = routing["counts"].cpu()
    touched = int((counts > 0).sum())
    near = int((routing["margin"] <= 1e-4).sum().item())
    stream_path = cfg.T * cfg.k <= 16 * cfg.E and not cfg.a8  # the library's automatic path choice
    kernel_file = "sparse_moe_transformer_route_amd/csrc/" + ("moe_stream.hip" if stream_path else "moe_gemm.hip")
    # algorithmic bytes and flops of the whole layer (both reported for every workload)
    lw = stream_work(cfg, touched, blocked)
    gw = gemm_work(cfg, blocked)
    layer = {"bytes": lw["layer_bytes"], "flop": gw["layer_flop"],
             "hbm_frac": lw["layer_bytes"] / (ms * 1e-3) / PEAK_HBM,
             "mfma_frac": gw["layer_flop"] / (ms * 1e-3) / gw["layer_peak"]}
    sec = dom_ms * 1e-3
    if stream_path:
        alg = lw["alg"]
        roof = {"bound": "hbm", "achieved": alg / sec / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                "frac": alg / sec / PEAK_HBM, "traffic": traffic_for(f"{lw['key']}/{name}", touched + 1),
                "kernel": lw["kernel"], "per_unit": lw["per_unit"], "units_per_launch": touched + 1,
                "kernel_ms": dom_ms}
    else:
        rows, alg = gw["rows"], gw["alg"]
        roof = {"bound": "mfma", "achieved": alg / sec / 1e12, "peak": gw["peak"] / 1e12, "unit": "TFLOP/s",
                "frac": alg / sec / gw["peak"], "traffic": traffic_for(f"grouped_gemm_gateup/{name}", rows),
                "kernel": gw["kernel"], "per_unit": gw["per_unit"], "units_per_launch": rows, "kernel_ms": dom_ms,
                "peak_how": gw["peak_how"]}
        if cfg.a8:
            roof["peak_mix"] = {"fp8_rows": cfg.T * cfg.k, "bf16_rows": cfg.T}
    roof["kernel_source_sha256_16"] = source_digest(os.path.join(ROOT, kernel_file))
    res = {"cfg": cfg, "inp": inp, "inp_rm": inp_rm, "blocked": blocked, "ms": ms, "tokens_per_s": cfg.T / (ms * 1e-3),
           "kernels_ms": r["kernels"],
           "roofline": roof, "layer": layer, "touched": touched, "counts": counts, "routing": routing,
           "warmup": r["warmup"], "steps": steps, "step_ms": step_stats(r["step_ms"]),
           "kernel_step_ms": step_stats(r["dom_ms"]), "near_ties": near,
           "input_sha256_16": input_digest(inp_rm, torch)}
    if r["cold_ms"] is not None:
        cold = step_stats(r["cold_ms"])
        cold_dom = sum(r["cold_dom_ms"]) / steps * 1e-3
        res["cold"] = {"step_ms": cold, "tokens_per_s_at_median": cfg.T / (cold["median"] * 1e-3),
                       "layer_hbm_frac_at_median": lw["layer_bytes"] / (cold["median"] * 1e-3) / PEAK_HBM,
                       "kernel_ms": cold_dom * 1e3,
                       "kernel_frac": (lw["alg"] if stream_path else gw["alg"]) / cold_dom /
                       (PEAK_HBM if stream_path else gw["peak"]),
                       "how": "a 512 MiB write between steps (outside the events) evicts the 256 MB last-level cache"}
    return res


def workload_object(res, extra=None):
    """The JSON object of one workload (the headline one is the top level)."""
    c = res["cfg"]
    o = {"workload": workload_name(c), "T": c.T, "weights_layout": layout_name(res), "ms_per_step": res["ms"],
         "steps": res["steps"],
         "warmup": res["warmup"], "step_ms": res["step_ms"], "tokens_per_s": res["tokens_per_s"],
         "roofline": res["roofline"], "layer": res["layer"], "kernels_ms": res["kernels_ms"],
         "touched_experts": res["touched"], "near_tie_tokens": res["near_ties"],
         "input_sha256_16": res["input_sha256_16"]}
    if "cold" in res:
        o["cold"] = res["cold"]
    if extra:
        o.update(extra)
    return o


def layout_name(res):
    c = res["cfg"]
    if c.ternary:
        return ("Sherry-packed routed experts in the blocked layout (16 rows x 512 weights per 1280 B block, "
                "hy_moe_block_sherry, converted once before timing), row-major bf16 shared expert" if res["blocked"]
                else "Sherry-packed routed experts (row-major codes), row-major bf16 shared expert")
    if c.fp8:
        return "row-major E4M3 routed experts, row-major bf16 shared expert"
    return ("blocked bf16 (16 rows x 64 columns per 2 KB block, hy_moe_block_bf16, converted once before timing)"
            if res["blocked"] else "row-major bf16")


def dtype_name(c):
    return ("sherry-ternary+bf16" if c.ternary else "fp8-e4m3+mxfp8-activations+bf16" if c.a8 else
            "fp8-e4m3+bf16" if c.fp8 else "bf16")


def workload_name(c):
    return (f"{c.name} MoE FFN layer T={c.T} d={c.d} E={c.E} top-{c.k} + 1 shared I={c.I}"
            + (" Sherry-ternary routed experts" if c.ternary else
               " FP8-E4M3 routed experts with MXFP8 activations (W8A8)" if c.a8 else
               " FP8-E4M3 routed experts" if c.fp8 else " bf16")
            + (" Zipf(1.2) router bias" if c.zipf_s else ""))


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
                ffn = oracle.ffn_w8a8 if cfg.a8 else oracle.ffn_w64 if "fgate" in inp else oracle.ffn
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
                      f"{cfg.k} routed + 1 shared SwiGLU experts, combine); {el:.1f} s on {nthreads} threads",
            "host": host_info(), "tiny_1thread": tiny_one_thread(hi)}


def host_info():
    """CPU model and core counts of this host."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


def tiny_one_thread(hi, budget_s=1.0):
    """The oracle's whole tiny layer (T=64, d=256, E=16, top-2, I=128) on one thread,
    repeated for about budget_s; host-generated inputs, generation not timed."""
    import oracle
    cfg = hi.CONFIGS["tiny"]
    L = hi.host_layer(cfg)
    el, passes = 0.0, 0
    while passes == 0 or el < budget_s:
        t0 = time.perf_counter()
        oracle.forward(L["x"], L["router"], L["bias"], L["gate"], L["up"], L["down"], L["shared"]["gate"],
                       L["shared"]["up"], L["shared"]["down"], cfg.k, nthreads=1)
        el += time.perf_counter() - t0
        passes += 1
    return {"value": passes * cfg.T / el, "unit": "tokens/s", "cores": 1,
            "sample": f"{passes} passes of the whole tiny layer (T={cfg.T}), {el:.2f} s"}


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


def library_batched_gemm_reference(torch, seconds=0.5):
    """torch.bmm (hipBLASLt) on 256 batched bf16 GEMMs of 288 x 6144 @ 6144 x 4096: the prefill
    gate/up work (73728 rows in all) with one weight matrix per expert, 12.9 GB of distinct
    weights as in the layer, but equal batches, contiguous rows and no gather."""
    g = torch.Generator(device="cuda:0").manual_seed(2)
    a = torch.randn(256, 288, 6144, generator=g, device="cuda:0", dtype=torch.bfloat16)
    b = (torch.randn(256, 6144, 4096, generator=g, device="cuda:0", dtype=torch.bfloat16) / 78.0).contiguous()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        torch.bmm(a, b)
        torch.cuda.synchronize()
    n = 10
    t0 = time.perf_counter()
    for _ in range(n):
        torch.bmm(a, b)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / n
    del a, b
    torch.cuda.empty_cache()
    return {"tflops": 2 * 73728 * 6144 * 4096 / dt / 1e12, "ms": dt * 1e3,
            "how": "torch.bmm bf16 [256 x 288 x 6144] @ [256 x 6144 x 4096] (hipBLASLt; one weight matrix per "
                   "batch, 12.9 GB), mean of 10 after 0.5 s warm"}


def library_gemm_reference(torch, seconds=0.5):
    """torch.matmul (hipBLASLt) on one dense bf16 GEMM of the prefill gate/up shape
    (73728 x 6144 @ 6144 x 4096, N(0,1)-like operands): what AMD's GEMM library reaches on
    this part for the same arithmetic without routing, gathering or ragged experts."""
    g = torch.Generator(device="cuda:0").manual_seed(1)
    a = torch.randn(73728, 6144, generator=g, device="cuda:0").to(torch.bfloat16)
    b = (torch.randn(6144, 4096, generator=g, device="cuda:0") / 78.0).to(torch.bfloat16).contiguous()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        torch.matmul(a, b)
        torch.cuda.synchronize()
    n = 10
    t0 = time.perf_counter()
    for _ in range(n):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / n
    del a, b
    torch.cuda.empty_cache()
    return {"tflops": 2 * 73728 * 6144 * 4096 / dt / 1e12, "ms": dt * 1e3,
            "how": "torch.matmul bf16 [73728 x 6144] @ [6144 x 4096] (hipBLASLt), mean of 10 after 0.5 s warm"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default: at least 5 and %.1f s of them)" % WARMUP_MIN_S)
    ap.add_argument("--config", default="decode", choices=["tiny", "decode", "prefill", "skewed", "ternary",
                                                                 "ternary_prefill", "fp8", "fp8_prefill",
                                                                 "fp8_w8a8_prefill",
                                                                 "indexer_tiny", "indexer_decode"])
    ap.add_argument("--only", action="store_true",
                    help="time --config alone (no other workloads, probes or oracle): for profiler runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    full = args.config == "decode" and not args.only
    bf16_hy4 = not cfg.ternary and not cfg.fp8 and cfg.d == 6144
    shared_weights = None
    if bf16_hy4 or full:
        log("[bench] generating the Hy4-shape bf16 layer (19.3 GB of expert weights) on the GPU")
        shared_weights = hi.dev_layer(hi.CONFIGS["prefill"], device="cuda:0")
        torch.cuda.synchronize()

    # measured peaks next to the published ones (these also bring the shader clock up
    # from idle before the first timed workload): bf16 MFMA on random operand bits (the
    # power-capped clock depends on operand activity), one streaming read of HBM, and
    # hipBLASLt's dense GEMM of the prefill gate/up shape
    peaks = None
    if not args.only:
        gen = torch.Generator(device="cuda:0").manual_seed(0)
        ops = torch.randn(hm.PROBE_OPERAND_BYTES // 2, generator=gen, device="cuda:0").to(torch.bfloat16)
        read_buf = shared_weights["gate"] if shared_weights is not None else torch.empty(
            4 << 30, dtype=torch.uint8, device="cuda:0")
        codes = ops.float().to(torch.float8_e4m3fn).view(torch.uint8)
        codes = torch.cat([codes, codes])  # E4M3 codes of the same values: PROBE_OPERAND_BYTES of them
        peaks = {"mfma_bf16_tflops": hm.probe_mfma_bf16(ops), "mfma_fp8_tflops": hm.probe_mfma_fp8(codes),
                 "hbm_read_gbs": hm.probe_hbm_read(read_buf),
                 "hbm_read_bytes": read_buf.numel() * read_buf.element_size(),
                 "how": "hy_moe_probe_mfma_bf16 (32x32x16 bf16 MFMAs, 4 workgroups per CU, random N(0,1) operands, "
                        "~40 ms), hy_moe_probe_mfma_fp8 (32x32x64 E4M3 MFMAs with unit block scales on the same "
                        "values as E4M3 codes, ~40 ms) and hy_moe_probe_hbm_read (best of three timed streaming passes of "
                        "non-temporal 16-byte loads, 1 KB in order per wave instruction, after an untimed one)"}
        del read_buf
        if full:
            peaks["library_gemm_bf16"] = library_gemm_reference(torch)
            peaks["library_batched_gemm_bf16"] = library_batched_gemm_reference(torch)
        log(f"[bench] measured peaks: {peaks['mfma_bf16_tflops']:.0f} TFLOP/s bf16 MFMA, "
            f"{peaks['hbm_read_gbs']:.0f} GB/s HBM read"
            + (f", hipBLASLt dense GEMM {peaks['library_gemm_bf16']['tflops']:.0f} TFLOP/s, batched per-expert GEMM "
               f"{peaks['library_batched_gemm_bf16']['tflops']:.0f} TFLOP/s" if full else ""))
        # back to load right away: the clock drops when the GPU idles
        hm.probe_mfma_bf16(ops)

    def report(res):
        log(f"[bench] {res['cfg'].name}: {res['ms']:.3f} ms/step (median {res['step_ms']['median']:.3f}, "
            f"p10 {res['step_ms']['p10']:.3f}, p90 {res['step_ms']['p90']:.3f}), {res['tokens_per_s']:.1f} tokens/s, "
            f"kernels {json.dumps({k: round(v, 4) for k, v in res['kernels_ms'].items()})}")

    # bf16 and ternary workloads run on the blocked layout of the same weights (one
    # conversion, outside every timed region); the headline is timed on row-major
    # weights as well
    blocked_weights = hm.block_layer(shared_weights) if shared_weights is not None else None
    torch.cuda.synchronize()
    extra = {}
    if full:
        t = run_config("tiny", args, hi, hm, torch, blocked=True)
        report(t)
        extra["tiny"] = workload_object(t, {"us_per_step": t["ms"] * 1e3})
        del t
    # the headline decode run also times the same steps with a 512 MiB write between
    # them (its "cold" object): each step streams 12 GB of weights, so the 256 MB
    # last-level cache holds none of the next step's first weights either way
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    n_flush = [0]

    def flush():
        n_flush[0] += 1
        flush_buf.fill_(n_flush[0] & 0xFF)
    main_res = run_config(args.config, args, hi, hm, torch, blocked_weights if bf16_hy4 or full else None,
                          flush=flush if full else None, blocked=True, rm_weights=shared_weights)
    report(main_res)
    if full:
        rm = run_config(args.config, args, hi, hm, torch, shared_weights)
        report(rm)
        extra["row_major_weights"] = {"weights_layout": layout_name(rm), "ms_per_step": rm["ms"],
                                      "tokens_per_s": rm["tokens_per_s"], "step_ms": rm["step_ms"],
                                      "roofline_frac": rm["roofline"]["frac"], "kernels_ms": rm["kernels_ms"],
                                      "note": "the same weights in row-major order (HY_MOE_WEIGHTS_BF16)"}
        del rm
    if full:
        pre = run_config("prefill", args, hi, hm, torch, blocked_weights, blocked=True, rm_weights=shared_weights)
        report(pre)
        extra["prefill"] = workload_object(pre)
        del pre
        sk = run_config("skewed", args, hi, hm, torch, blocked_weights, blocked=True, rm_weights=shared_weights)
        report(sk)
        cnt = sk["counts"]
        extra["skewed"] = workload_object(sk, {"hottest_expert_rows": int(cnt.max()),
                                               "empty_experts": int((cnt == 0).sum())})
        del sk
        torch.cuda.empty_cache()
        tn = run_config("ternary", args, hi, hm, torch, flush=flush, blocked=True)
        report(tn)
        extra["ternary"] = workload_object(tn)
        del tn
        torch.cuda.empty_cache()
        w8 = run_config("fp8_w8a8_prefill", args, hi, hm, torch)
        report(w8)
        extra["fp8_w8a8_prefill"] = workload_object(w8)
        del w8
        torch.cuda.empty_cache()

    roof = main_res["roofline"]
    if peaks is not None:
        for r in [roof] + [o["roofline"] for o in extra.values() if "roofline" in o]:
            r["frac_of_measured_peak"] = r["achieved"] / measured_peak_of(r, peaks)
            if r["unit"] == "TFLOP/s" and "library_gemm_bf16" in peaks:
                r["frac_of_library_dense_gemm"] = r["achieved"] / peaks["library_gemm_bf16"]["tflops"]
            if r["unit"] == "TFLOP/s" and "library_batched_gemm_bf16" in peaks:
                r["frac_of_library_batched_gemm"] = r["achieved"] / peaks["library_batched_gemm_bf16"]["tflops"]

    cpu = None
    if not args.no_cpu_baseline and not args.only:
        log("[bench] timing the oracle on the host")
        # the oracle takes row-major weights
        cpu = cpu_baseline(cfg, hi, torch, main_res["inp_rm"], main_res["routing"], args.cpu_seconds)

    c = main_res["cfg"]
    line = {
        "metric": METRIC, "value": main_res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": main_res["steps"], "warmup": main_res["warmup"], "ms_per_step": main_res["ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype_name(c), "data": "synthetic",
        "config": {"workload": workload_name(c), "weights_layout": layout_name(main_res),
                   "T": c.T, "d": c.d, "E": c.E, "k": c.k, "I": c.I, "seed": c.seed,
                   "touched_experts": main_res["touched"]},
        "step_ms": main_res["step_ms"],
        "roofline": main_res["roofline"],
        "layer": main_res["layer"],
        "kernels_ms": main_res["kernels_ms"],
        "near_tie_tokens": main_res["near_ties"],
        "input_sha256_16": main_res["input_sha256_16"],
        "measured_peak": peaks,
        "cpu_baseline": cpu,
    }
    if "cold" in main_res:
        line["cold"] = main_res["cold"]
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
