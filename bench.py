"""Benchmark of the FP8 linear layer hot path on one MI355X.

One step is one forward + backward pass of the Qwen3-8B MLP up-projection
linear (M = 8192 tokens, K = 4096, N = 12288) through every kernel of the path:

    rmsnorm_quant(X, gamma)        -> QX, SX      fused RMSNorm + 1x128 quantisation
    quantize_weight_128x128(W)     -> QW, SW      once per weight update
    gemm_fprop(QX, SX, QW, SW)     -> Y           FProp  (1x128)x(128x128)
    quantize_act_1x128(dY)         -> QdY, SdY    BF16 gradient -> FP8
    gemm_dgrad(QdY, SdY, QW, SW)   -> dX          DGrad, weight blocks transposed
    requant_transpose_128x1(QX)    -> QXt, SXt    saved FP8 activation -> 128x1
    requant_transpose_128x1(QdY)   -> QdYt, SdYt
    gemm_wgrad(QdYt, SdYt, QXt, SXt) -> dW        WGrad  (1x128)x(128x1)

Inputs are seeded synthetic bf16 tensors (X ~ N(0,1) with 4 outlier channels
x50, W ~ N(0, 0.02), dY ~ N(0, 1e-3), gamma ~ N(1, 0.05)), resident in HBM
before the timed region.  ``value`` is the step's GEMM work (3 x 2MNK FLOP)
divided by the step time.  Per-kernel times come from HIP events recorded on
the launch stream around every kernel of the timed steps; the ``roofline``
object describes the slowest GEMM against the dense FP8 MFMA peak.  The
``cpu_baseline`` runs the CPU oracle on a 256-token slice of the same step.

``--workload decode_8b`` instead times the rollout decode path at M tokens
(``--decode-m``, default 16): RMSNorm+quant, FProp against the FP8 QKV and
gate+up weights, the fused SwiGLU + 1x128 quantisation of the gate+up output
(the down projection's input) and the down FProp (weights quantised once,
outside the timed region).  Up to 256 tokens the weights are held in the
rollout-packed order (pack_weight_rollout, outside the timed region) and the
FProps go through gemm_fprop_packed; larger batches (or ``--decode-rowmajor``)
use the row-major codes and gemm_fprop_splitk, which splits K across
workgroups for the shapes with fewer output tiles than CUs (its workspace is
allocated before the timed region).  Decode is bound by streaming
the FP8 weights, so its kernels also report weight GB/s.  Beside it the bench
times the same step in BF16 through torch (``bf16_reference``: hipBLASLt GEMMs
over bf16 weights rotated the same way), the FP8-against-BF16 rollout
comparison of the pages, unless ``--no-bf16-reference``.

``--workload llama_layer`` times the forward + backward of the four linears
of one Llama-3.1-8B layer (QKV, O, gate+up, down) at M = 16384 tokens, and
``--workload qwen32b_half_mlp`` that of one GPU's half of a Qwen3-32B MLP
(gate+up 5120 -> 25600, down 12800 -> 5120) at M = 8192: per linear the same
kernels as the default step (1x128 quantisation of X, weight quantisation,
FProp, dY quantisation, DGrad, both requants, WGrad).  They report every
GEMM's rate; ``value`` is again all GEMM work over the step time.

``--workload llama_mlp`` times the forward of a Llama-3.1-8B MLP at M = 16384
as one chain (RMSNorm+quant, the gate+up FProp with SwiGLU and the 1x128
quantisation in its epilogue, down FProp), and for comparison the same chain
with swiglu_quant as a separate kernel and with the SwiGLU unfused.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--workload linear_8b_up|decode_8b|llama_layer|qwen32b_half_mlp|llama_mlp]
                       [--decode-m M] [--decode-rowmajor] [--no-bf16-reference]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "block-scaled FP8 GEMM TFLOP/s (FProp/DGrad/WGrad) + % of FP8 MFMA peak"
MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 (E4M3) MFMA
HBM_PEAK_GBS = 8000.0

M, K, N = 8192, 4096, 12288
KERNELS_TIMING = ("HIP events recorded after every kernel of the second timed pass; each interval also "
                  "holds one launch gap of about 5 us, which matters for the short memory-bound kernels "
                  "(device durations from rocprofv3 are in profiles/)")
EPS = 1e-6
DECODE_WEIGHT_SETS = 4
ROOT = os.path.dirname(os.path.abspath(__file__))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # untimed steps after the settle period (which covers the power-management
    # transient; see settle())
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="linear_8b_up",
                    choices=["linear_8b_up", "decode_8b", "llama_layer", "qwen32b_half_mlp", "llama_mlp"])
    ap.add_argument("--decode-m", type=int, default=16)
    ap.add_argument("--decode-rowmajor", action="store_true",
                    help="decode_8b: row-major weights and gemm_fprop_splitk at every batch size")
    ap.add_argument("--no-bf16-reference", action="store_true",
                    help="decode_8b: skip timing the same step in BF16 through torch")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy (torch copy_), whose HBM counters "
                         "calibrate FETCH_SIZE / WRITE_SIZE")
    return ap.parse_args()


def kernel_work():
    """Algorithmic FLOPs (GEMMs) or bytes (memory-bound kernels) per launch."""
    g = 2.0 * M * N * K
    act = lambda r, c: r * c * (2 + 1) + 4 * r * c // 128            # bf16 in, u8 + f32 scales out
    req = lambda r, c: 2 * (r * c + 4 * r * c // 128)                # u8 + scales in, same out
    return {
        "rmsnorm_quant": ("GB/s", act(M, K) + 2 * K),
        "quantize_weight_128x128": ("GB/s", N * K * 3 + 4 * N * K // (128 * 128)),
        "gemm_fprop": ("TFLOP/s", g),
        "quantize_act_1x128": ("GB/s", act(M, N)),
        "gemm_dgrad": ("TFLOP/s", g),
        "requant_x": ("GB/s", req(M, K)),
        "requant_dy": ("GB/s", req(M, N)),
        "gemm_wgrad": ("TFLOP/s", g),
    }


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "qwen3_8b_up_step_hbm_traffic.md")


def measured_traffic(kernel):
    """HBM-side bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary (calibrated against a plain copy), or None when that record was
    taken on a different GEMM source than the one built here."""
    import hashlib
    try:
        lines = open(TRAFFIC_RECORD).read().splitlines()
    except OSError:
        return None
    want, table = None, {}
    for ln in lines:
        f = ln.split()
        if len(f) == 3 and f[0] == "source_sha256":
            want = (f[1], f[2])
        elif len(f) == 3 and f[0] == "traffic_bytes":
            table[f[1]] = int(f[2])
    if want is None or kernel not in table:
        return None
    with open(os.path.join(ROOT, want[0]), "rb") as fh:
        if hashlib.sha256(fh.read()).hexdigest() != want[1]:
            return None
    return table[kernel]


def cpu_baseline(d, gamma):
    """The oracle on a 256-token slice of the step (all rows of the path)."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        blas_threads = None
    ms = 256
    x, dy = d["x"][:ms], d["dy"][:ms]
    t0 = time.perf_counter()
    qx, sx = oracle.rmsnorm_quant(x, gamma, EPS)
    qw, sw = oracle.quant_weight_128x128(d["w"])
    oracle.gemm_fprop_ref(qx, sx, qw, sw)
    qdy, sdy = oracle.quant_act_1x128(dy)
    oracle.gemm_dgrad_ref(qdy, sdy, qw, sw)
    qxt, sxt = oracle.requant_transpose_128x1(qx, sx)
    qdyt, sdyt = oracle.requant_transpose_128x1(qdy, sdy)
    oracle.gemm_wgrad_ref(qdyt, sdyt, qxt, sxt)
    dt = time.perf_counter() - t0
    flops = 3 * 2.0 * ms * N * K
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "blas_threads": blas_threads, "kind": "oracle",
            "sample": f"one step on a {ms}-token slice (M={ms}, K={K}, N={N}): rmsnorm_quant, "
                      f"full weight quantisation, quant dY, requant x2, fp64 FProp/DGrad/WGrad; "
                      f"{dt:.2f} s; quantisers single-threaded numpy, GEMMs numpy BLAS "
                      f"({blas_threads} threads) on the {cores} cores of the affinity mask"}


SETTLE_S = 0.15


def settle(torch, steps, seconds=SETTLE_S):
    """Run the step back to back for `seconds` before the warm-up steps.

    After an idle period the chip's power management takes some 20-30 ms of
    sustained load to settle: measured on the 8B step, the first 20 steps after
    0.3-0.5 s of idle averaged 1.28-1.48 ms (single steps up to 1.6 ms) against
    1.13 ms later, whether or not the buffers had been used before, while after
    0.28 s of unrelated bf16 matmul load the first steps already ran at 1.13-1.16
    ms.  A training job runs its steps back to back, so the timed steps start
    from that sustained state.  Returns the number of steps run."""
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _, fn in steps:
            fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def settle_info(n):
    return {"seconds": SETTLE_S, "steps": n,
            "why": "before the warm-up steps, the step runs back to back for this long: after an idle "
                   "period the chip's power management needs about 20-30 ms of sustained load to settle "
                   "(first steps up to 35 % slower, independent of buffer first-touch)"}


def time_steps(torch, steps, n_steps, n_warmup, dev):
    """Run the settle period and the warm-up steps, then two timed passes of n_steps steps on the launch
    stream.  Pass 1 records a HIP event only at step boundaries: it gives the
    step times and the wall time.  Pass 2 records an event after every kernel:
    it gives the per-kernel times (those events put a small gap between the
    kernels, so pass 2's steps run slightly longer than pass 1's).  Returns
    (per-kernel ms lists, per-step ms list, wall seconds of pass 1, settle steps)."""
    n_settle = settle(torch, steps)
    for _ in range(n_warmup):
        for _, fn in steps:
            fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(n_steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    bounds[0].record(stream)
    for s in range(n_steps):
        for _, fn in steps:
            fn()
        bounds[s + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [bounds[s].elapsed_time(bounds[s + 1]) for s in range(n_steps)]

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(steps) + 1)] for _ in range(n_steps)]
    torch.cuda.synchronize()
    for s in range(n_steps):
        ev[s][0].record(stream)
        for i, (_, fn) in enumerate(steps):
            fn()
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    per = {name: [] for name, _ in steps}
    for s in range(n_steps):
        for i, (name, _) in enumerate(steps):
            per[name].append(ev[s][i].elapsed_time(ev[s][i + 1]))
    return per, step_ms, wall, n_settle


def read_sclk_mhz():
    """Current shader clock from the driver's DPM table (the line marked '*'), or None."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as fh:
                for line in fh:
                    if line.rstrip().endswith("*"):
                        return int(line.split(":")[1].strip().lower().split("mhz")[0])
        except (OSError, ValueError, IndexError):
            continue
    return None


def sustained_sclk(torch, steps, seconds=0.6):
    """Shader clock under load: run the step back to back for `seconds` while a
    thread samples the DPM table every 20 ms (samples from the first 0.1 s are
    dropped).  Returns a dict, or None where the table is unreadable."""
    import threading
    if read_sclk_mhz() is None:
        return None
    samples, stop = [], threading.Event()

    def sampler():
        t0 = time.perf_counter()
        while not stop.is_set():
            v = read_sclk_mhz()
            if v is not None and time.perf_counter() - t0 > 0.1:
                samples.append(v)
            time.sleep(0.02)

    th = threading.Thread(target=sampler)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            for _, fn in steps:
                fn()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    if not samples:
        return None
    return {"median": float(np.median(samples)), "min": min(samples), "max": max(samples),
            "samples": len(samples),
            "source": f"pp_dpm_sclk sampled every 20 ms over {seconds} s of back-to-back steps after the timed passes"}


def bench_decode(args):
    import torch
    import quantized_rl_amd as jet
    from quantized_rl_amd import synth

    dev = torch.device("cuda:0")
    m = args.decode_m
    d = synth.decode_8b(m)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    x, gamma = bf16(d["x"]), bf16(d["gamma"])
    wq = {k: jet.quantize_weight_128x128(bf16(d[k])) for k in ("w_qkv", "w_gu", "w_down")}
    # The three FP8 weights total 176 MB, which the 256 MB MALL could hold from one
    # step to the next; consecutive steps therefore rotate over DECODE_WEIGHT_SETS
    # copies (704 MB), so every step streams its weights from HBM.
    sets = [wq] + [{k: (q.clone(), s.clone()) for k, (q, s) in wq.items()} for _ in range(DECODE_WEIGHT_SETS - 1)]
    # Up to 256 tokens the rollout engine keeps its weight copy in the packed order
    # (pack_weight_rollout, once per weight update: outside the timed region) and
    # runs gemm_fprop_packed; larger batches use the row-major codes and
    # gemm_fprop_splitk, which splits K for the shapes with fewer output tiles
    # than CUs through this workspace (allocated once, untimed).
    packed = m <= 256 and not args.decode_rowmajor
    if packed:
        sets = [{k: (jet.pack_weight_rollout(q), s) for k, (q, s) in st.items()} for st in sets]
    torch.cuda.synchronize()
    qx, sx = jet.rmsnorm_quant(x, gamma, d["eps"])
    y = {k: torch.empty((m, wq[k][0].shape[0]), dtype=torch.bfloat16, device=dev) for k in wq}
    inter = wq["w_down"][0].shape[1]  # 12288: the down projection's input width
    qh = torch.empty((m, inter), dtype=torch.uint8, device=dev)
    sh = torch.empty((inter // 128, m), dtype=torch.float32, device=dev)
    need = max(jet.gemm_fprop_splitk_workspace_bytes(m, q.shape[0], q.shape[1]) for q, _ in wq.values())
    ws = torch.empty((max(need, 4) // 4,), dtype=torch.float32, device=dev)

    def fprop(qa, sa, qb, sb, out, work):
        if packed:
            return jet.gemm_fprop_packed(qa, sa, qb, sb, out)
        return jet.gemm_fprop_splitk(qa, sa, qb, sb, out, work)
    cur = [0]

    def norm():
        cur[0] = (cur[0] + 1) % len(sets)
        jet.rmsnorm_quant(x, gamma, d["eps"], qx, sx)

    steps = [
        ("rmsnorm_quant", norm),
        ("gemm_fprop_qkv", lambda: fprop(qx, sx, *sets[cur[0]]["w_qkv"], y["w_qkv"], ws)),
        ("gemm_fprop_gate_up", lambda: fprop(qx, sx, *sets[cur[0]]["w_gu"], y["w_gu"], ws)),
        ("swiglu_quant", lambda: jet.swiglu_quant(y["w_gu"], qh, sh)),
        ("gemm_fprop_down", lambda: fprop(qh, sh, *sets[cur[0]]["w_down"], y["w_down"], ws)),
    ]
    per, step_ms, wall, n_settle = time_steps(torch, steps, args.steps, args.warmup, dev)
    ms_per_step = float(np.mean(step_ms))
    ref = None if args.no_bf16_reference else decode_bf16_reference(torch, d, bf16, args)
    if ref is not None:
        ref["speedup_fp8_over_bf16"] = round(ref["ms_per_step"] / ms_per_step, 3)
    shapes = {"gemm_fprop_qkv": (6144, 4096), "gemm_fprop_gate_up": (24576, 4096), "gemm_fprop_down": (4096, 12288)}
    flops = sum(2.0 * m * n * k for n, k in shapes.values())
    kernels = {}
    for name in per:
        avg_ms = float(np.mean(per[name]))
        if name in shapes:
            n, k = shapes[name]
            wbytes = n * k + 4 * (n // 128) * (k // 128) + m * k + 2 * m * n
            kernels[name] = {"avg_us": round(avg_ms * 1e3, 2), "weight_GBps": round(wbytes / (avg_ms * 1e-3) / 1e9, 1),
                             "frac_hbm": round(wbytes / (avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                             "TFLOPs": round(2.0 * m * n * k / (avg_ms * 1e-3) / 1e12, 2)}
        else:
            kernels[name] = {"avg_us": round(avg_ms * 1e3, 2)}
    dom = max(shapes, key=lambda k: kernels[k]["avg_us"])
    out = {
        "metric": METRIC, "value": round(flops / (ms_per_step * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": {"workload": "qwen3_8b_decode", "M": m, "K": 4096,
                   "weights": "qkv 6144x4096, gate_up 24576x4096, down 4096x12288", "seed": 2,
                   "weight_sets_rotated": DECODE_WEIGHT_SETS,
                   "weight_layout": "rollout-packed" if packed else "row-major",
                   "fprop": "gemm_fprop_packed" if packed else "gemm_fprop_splitk"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": kernels[dom]["weight_GBps"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": kernels[dom]["frac_hbm"], "traffic": None},
        "kernels": kernels,
        "kernels_timing": KERNELS_TIMING,
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "settle": settle_info(n_settle),
    }
    if ref is not None:
        out["bf16_reference"] = ref
    print(json.dumps(out), flush=True)


def decode_bf16_reference(torch, d, bf16, args):
    """The decode step in BF16 through torch, timed like the FP8 step: RMSNorm in fp32
    arithmetic rounded to bf16, the three projections as bf16 GEMMs (torch.matmul:
    hipBLASLt) against weights stored transposed and contiguous, SwiGLU in fp32
    rounded to bf16; the weights rotate over the same number of copies, so each
    step streams them from HBM.  The rollout comparison the pages report (FP8
    against BF16 rollout) on this GPU; a reference only, none of it is the FP8 path."""
    m = args.decode_m
    x, gamma = bf16(d["x"]), bf16(d["gamma"]).float()
    eps = d["eps"]
    w0 = {k: bf16(d[k]).t().contiguous() for k in ("w_qkv", "w_gu", "w_down")}  # [K, N]
    sets = [w0] + [{k: v.clone() for k, v in w0.items()} for _ in range(DECODE_WEIGHT_SETS - 1)]
    inter = w0["w_down"].shape[0]
    h = torch.empty_like(x)
    cur = [0]
    out = {}

    def norm():
        cur[0] = (cur[0] + 1) % len(sets)
        xf = x.float()
        h.copy_(xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + eps) * gamma)

    def qkv():
        out["qkv"] = torch.matmul(h, sets[cur[0]]["w_qkv"])

    def gate_up():
        out["gu"] = torch.matmul(h, sets[cur[0]]["w_gu"])

    def swiglu():
        gu = out["gu"].float()
        out["a"] = (torch.nn.functional.silu(gu[:, :inter]) * gu[:, inter:]).to(torch.bfloat16)

    def down():
        out["y"] = torch.matmul(out["a"], sets[cur[0]]["w_down"])

    steps = [("rmsnorm", norm), ("matmul_qkv", qkv), ("matmul_gate_up", gate_up), ("swiglu", swiglu),
             ("matmul_down", down)]
    per, step_ms, _, _ = time_steps(torch, steps, args.steps, args.warmup, torch.device("cuda:0"))
    return {"what": "the same decode step in BF16 through torch (hipBLASLt GEMMs, fp32 RMSNorm and SwiGLU)",
            "ms_per_step": round(float(np.mean(step_ms)), 4),
            "kernels_us": {k: round(float(np.mean(v)) * 1e3, 2) for k, v in per.items()}}


def bench_mlp(args):
    """Forward of a Llama-3.1-8B MLP at M = 16384 tokens as one chain:
    rmsnorm_quant -> gemm_fprop_swiglu_quant (gate+up FProp, 4096 -> 28672, whose
    epilogue applies SwiGLU and the 1x128 quantisation) -> FProp down (14336 ->
    4096), weights quantised once outside the timed region.  Timed beside it:
    the same chain with the gate+up output written in bf16 and swiglu_quant as a
    kernel of its own, and with the SwiGLU unfused (torch's silu and multiply
    writing a bf16 h, then quantize_act_1x128).  ``value`` is the fused chain's
    GEMM work over its step time."""
    import torch
    import quantized_rl_amd as jet
    from quantized_rl_amd import synth

    dev = torch.device("cuda:0")

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    m = 16384
    dgu, ddn = synth.llama_layer(0, "gate_up", m=m), synth.llama_layer(0, "down", m=m)
    x = bf16(dgu["x"])
    gamma = bf16(synth.decode_8b(16)["gamma"])  # N(1, 0.05) over 4096 channels
    qwg, swg = jet.quantize_weight_128x128(bf16(dgu["w"]))
    qwd, swd = jet.quantize_weight_128x128(bf16(ddn["w"]))
    del dgu, ddn
    n_gu, k = qwg.shape
    n_dn, inter = qwd.shape
    u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
    qx, sx = torch.empty((m, k), dtype=u8, device=dev), torch.empty((k // 128, m), dtype=f32, device=dev)
    ygu = torch.empty((m, n_gu), dtype=bf, device=dev)
    qh, sh = torch.empty((m, inter), dtype=u8, device=dev), torch.empty((inter // 128, m), dtype=f32, device=dev)
    ydn = torch.empty((m, n_dn), dtype=bf, device=dev)
    hbuf = torch.empty((m, inter), dtype=bf, device=dev)

    def silu_mul():
        torch.mul(torch.nn.functional.silu(ygu[:, :inter]), ygu[:, inter:], out=hbuf)

    norm = [("rmsnorm_quant", lambda: jet.rmsnorm_quant(x, gamma, EPS, qx, sx))]
    head = norm + [("gemm_fprop_gate_up", lambda: jet.gemm_fprop(qx, sx, qwg, swg, ygu))]
    tail = [("gemm_fprop_down", lambda: jet.gemm_fprop(qh, sh, qwd, swd, ydn))]
    # the gate+up FProp's epilogue applies SwiGLU and quantises: no bf16 gate+up output
    fused = norm + [("gemm_fprop_swiglu_quant", lambda: jet.gemm_fprop_swiglu_quant(qx, sx, qwg, swg, qh, sh))] + tail
    two_kernel = head + [("swiglu_quant", lambda: jet.swiglu_quant(ygu, qh, sh))] + tail
    unfused = head + [("torch_silu_mul", silu_mul),
                      ("quantize_act_1x128", lambda: jet.quantize_act_1x128(hbuf, qh, sh))] + tail
    flops = 2.0 * m * n_gu * k + 2.0 * m * n_dn * inter
    per, step_ms, wall, n_settle = time_steps(torch, fused, args.steps, args.warmup, dev)
    per_t, step_t, _, _ = time_steps(torch, two_kernel, args.steps, args.warmup, dev)
    per_u, step_u, _, _ = time_steps(torch, unfused, args.steps, args.warmup, dev)
    ms_per_step, ms_two, ms_unfused = float(np.mean(step_ms)), float(np.mean(step_t)), float(np.mean(step_u))
    act = lambda r, c: r * c * 3 + 4 * r * c // 128  # noqa: E731
    work = {"rmsnorm_quant": ("GB/s", act(m, k) + 2 * k), "gemm_fprop_gate_up": ("TFLOP/s", 2.0 * m * n_gu * k),
            "gemm_fprop_swiglu_quant": ("TFLOP/s", 2.0 * m * n_gu * k),
            "swiglu_quant": ("GB/s", m * inter * 5 + 4 * m * inter // 128),
            "gemm_fprop_down": ("TFLOP/s", 2.0 * m * n_dn * inter),
            # silu reads gate and writes a bf16 temporary, mul reads it and up and writes h
            "torch_silu_mul": ("GB/s", m * inter * 10), "quantize_act_1x128": ("GB/s", act(m, inter))}

    def rates(p):
        out = {}
        for name in p:
            unit, amount = work[name]
            avg_ms = float(np.mean(p[name]))
            rate = amount / (avg_ms * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
            peak = MFMA_FP8_PEAK_TFLOPS if unit == "TFLOP/s" else HBM_PEAK_GBS
            out[name] = {"avg_us": round(avg_ms * 1e3, 2), "rate": round(rate, 1), "unit": unit,
                         "frac": round(rate / peak, 4)}
        return out

    kernels = rates(per)
    dom = max(("gemm_fprop_swiglu_quant", "gemm_fprop_down"), key=lambda n: kernels[n]["avg_us"])
    out = {
        "metric": METRIC, "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": {"workload": "llama31_8b_mlp_fwd", "M": m, "K": k, "gate_up_N": n_gu, "down_K": inter,
                   "down_N": n_dn, "seed": 3},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": kernels[dom]["rate"],
                     "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(kernels[dom]["rate"] / MFMA_FP8_PEAK_TFLOPS, 4), "traffic": None},
        "kernels": kernels,
        "gate_up_output_bytes_not_written": 2 * m * n_gu,
        "two_kernel_swiglu": {"ms_per_step": round(ms_two, 4), "kernels": rates(per_t),
                              "bytes_moved_between_the_gemms": 2 * m * n_gu + work["swiglu_quant"][1]},
        "unfused_swiglu": {"ms_per_step": round(ms_unfused, 4), "kernels": rates(per_u),
                           "bytes_moved_between_the_gemms": 2 * m * n_gu + work["torch_silu_mul"][1]
                           + work["quantize_act_1x128"][1]},
        "kernels_timing": KERNELS_TIMING,
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "settle": settle_info(n_settle),
    }
    print(json.dumps(out), flush=True)


def bench_layers(args):
    """Forward + backward of several linears back to back (one training step of
    a layer's linears); every GEMM is reported against the FP8 MFMA peak."""
    import torch
    import quantized_rl_amd as jet
    from quantized_rl_amd import synth

    dev = torch.device("cuda:0")

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    if args.workload == "llama_layer":
        m, seed = 16384, 3
        linears = []
        for name in synth.LLAMA_LINEARS:
            d = synth.llama_layer(0, name, m=m)
            linears.append((name, bf16(d["x"]), bf16(d["w"]), bf16(d["dy"])))
            del d
        cfg = {"workload": "llama31_8b_layer_linears_fwd_bwd", "M": m, "layer": 0,
               "linears": {k: {"N": n, "K": kk} for k, (n, kk) in synth.LLAMA_LINEARS.items()}, "seed": seed}
    else:
        m, seed = 8192, 4
        d = synth.qwen32b_half_mlp(m)
        linears = [("gate_up", bf16(d["x"]), bf16(d["w_gu"]), bf16(d["dy_gu"])),
                   ("down", bf16(d["down_in"]), bf16(d["w_down"]), bf16(d["dy_down"]))]
        del d
        cfg = {"workload": "qwen3_32b_half_mlp_fwd_bwd", "M": m,
               "linears": {"gate_up": {"N": 25600, "K": 5120}, "down": {"N": 5120, "K": 12800}}, "seed": seed}
    u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
    steps, work = [], {}
    total_flops = 0.0
    for name, x, w, dy in linears:
        n, k = w.shape
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)  # noqa: E731
        b = dict(qx=e((m, k), u8), sx=e((k // 128, m), f32), qw=e((n, k), u8),
                 sw=e((n // 128, k // 128), f32), qdy=e((m, n), u8), sdy=e((n // 128, m), f32),
                 qxt=e((k, m), u8), sxt=e((m // 128, k), f32), qdyt=e((n, m), u8),
                 sdyt=e((m // 128, n), f32), y=e((m, n), bf), dx=e((m, k), bf), dw=e((n, k), bf))
        g = 2.0 * m * n * k
        total_flops += 3 * g
        steps += [
            (f"{name}.quantize_act_x", lambda x=x, b=b: jet.quantize_act_1x128(x, b["qx"], b["sx"])),
            (f"{name}.quantize_weight", lambda w=w, b=b: jet.quantize_weight_128x128(w, b["qw"], b["sw"])),
            (f"{name}.gemm_fprop", lambda b=b: jet.gemm_fprop(b["qx"], b["sx"], b["qw"], b["sw"], b["y"])),
            (f"{name}.quantize_act_dy", lambda dy=dy, b=b: jet.quantize_act_1x128(dy, b["qdy"], b["sdy"])),
            (f"{name}.gemm_dgrad", lambda b=b: jet.gemm_dgrad(b["qdy"], b["sdy"], b["qw"], b["sw"], b["dx"])),
            (f"{name}.requant_x", lambda b=b: jet.requant_transpose_128x1(b["qx"], b["sx"], b["qxt"], b["sxt"])),
            (f"{name}.requant_dy", lambda b=b: jet.requant_transpose_128x1(b["qdy"], b["sdy"], b["qdyt"], b["sdyt"])),
            (f"{name}.gemm_wgrad", lambda b=b: jet.gemm_wgrad(b["qdyt"], b["sdyt"], b["qxt"], b["sxt"], b["dw"])),
        ]
        act = m * k * 3 + 4 * m * k // 128
        work.update({
            f"{name}.quantize_act_x": ("GB/s", act),
            f"{name}.quantize_weight": ("GB/s", n * k * 3 + 4 * n * k // (128 * 128)),
            f"{name}.gemm_fprop": ("TFLOP/s", g),
            f"{name}.quantize_act_dy": ("GB/s", m * n * 3 + 4 * m * n // 128),
            f"{name}.gemm_dgrad": ("TFLOP/s", g),
            f"{name}.requant_x": ("GB/s", 2 * (m * k + 4 * m * k // 128)),
            f"{name}.requant_dy": ("GB/s", 2 * (m * n + 4 * m * n // 128)),
            f"{name}.gemm_wgrad": ("TFLOP/s", g),
        })
    torch.cuda.synchronize()
    per, step_ms, wall, n_settle = time_steps(torch, steps, args.steps, args.warmup, dev)
    ms_per_step = float(np.mean(step_ms))
    kernels = {}
    for name, (unit, amount) in work.items():
        avg_ms = float(np.mean(per[name]))
        rate = amount / (avg_ms * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
        peak = MFMA_FP8_PEAK_TFLOPS if unit == "TFLOP/s" else HBM_PEAK_GBS
        kernels[name] = {"avg_us": round(avg_ms * 1e3, 2), "rate": round(rate, 1), "unit": unit,
                         "frac": round(rate / peak, 4)}
    gemms = [k for k in kernels if ".gemm_" in k]
    dom = max(gemms, key=lambda k: kernels[k]["avg_us"])
    gemm_ms = sum(kernels[k]["avg_us"] for k in gemms) * 1e-3
    out = {
        "metric": METRIC, "value": round(total_flops / (ms_per_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3",
        "data": "synthetic", "config": cfg,
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": kernels[dom]["rate"],
                     "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(kernels[dom]["rate"] / MFMA_FP8_PEAK_TFLOPS, 4), "traffic": None},
        "gemm_only_TFLOPs": round(total_flops / (gemm_ms * 1e-3) / 1e12, 1),
        "kernels": kernels,
        "kernels_timing": KERNELS_TIMING,
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "settle": settle_info(n_settle),
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU: it times one GPU's share of the data-parallel layer, "
              f"whose only collective would be the weight-gradient all-reduce; --gpus {args.gpus} is not "
              f"supported", file=sys.stderr)
        sys.exit(2)
    if args.workload == "decode_8b":
        sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
        bench_decode(args)
        return
    if args.workload == "llama_mlp":
        sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
        bench_mlp(args)
        return
    if args.workload in ("llama_layer", "qwen32b_half_mlp"):
        sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
        bench_layers(args)
        return
    import torch
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import quantized_rl_amd as jet
    from quantized_rl_amd import synth

    dev = torch.device("cuda:0")
    d = synth.linear_8b_up(m=M, n=N, k=K)
    g_host = synth.decode_8b(16)["gamma"]  # gamma ~ N(1, 0.05), [4096]

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    x, w, dy, gamma = bf16(d["x"]), bf16(d["w"]), bf16(d["dy"]), bf16(g_host)
    u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
    qx, sx = torch.empty((M, K), dtype=u8, device=dev), torch.empty((K // 128, M), dtype=f32, device=dev)
    qw, sw = torch.empty((N, K), dtype=u8, device=dev), torch.empty((N // 128, K // 128), dtype=f32, device=dev)
    qdy, sdy = torch.empty((M, N), dtype=u8, device=dev), torch.empty((N // 128, M), dtype=f32, device=dev)
    qxt, sxt = torch.empty((K, M), dtype=u8, device=dev), torch.empty((M // 128, K), dtype=f32, device=dev)
    qdyt, sdyt = torch.empty((N, M), dtype=u8, device=dev), torch.empty((M // 128, N), dtype=f32, device=dev)
    y = torch.empty((M, N), dtype=bf, device=dev)
    dx = torch.empty((M, K), dtype=bf, device=dev)
    dw = torch.empty((N, K), dtype=bf, device=dev)

    steps = [
        ("rmsnorm_quant", lambda: jet.rmsnorm_quant(x, gamma, EPS, qx, sx)),
        ("quantize_weight_128x128", lambda: jet.quantize_weight_128x128(w, qw, sw)),
        ("gemm_fprop", lambda: jet.gemm_fprop(qx, sx, qw, sw, y)),
        ("quantize_act_1x128", lambda: jet.quantize_act_1x128(dy, qdy, sdy)),
        ("gemm_dgrad", lambda: jet.gemm_dgrad(qdy, sdy, qw, sw, dx)),
        ("requant_x", lambda: jet.requant_transpose_128x1(qx, sx, qxt, sxt)),
        ("requant_dy", lambda: jet.requant_transpose_128x1(qdy, sdy, qdyt, sdyt)),
        ("gemm_wgrad", lambda: jet.gemm_wgrad(qdyt, sdyt, qxt, sxt, dw)),
    ]

    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    per, step_ms, wall, n_settle = time_steps(torch, steps, args.steps, args.warmup, dev)
    ms_per_step = float(np.mean(step_ms))
    work = kernel_work()
    gemm_flops = 3 * 2.0 * M * N * K
    value = gemm_flops / (ms_per_step * 1e-3) / 1e12

    kernels = {}
    for name, (unit, amount) in work.items():
        avg_ms = float(np.mean(per[name]))
        rate = amount / (avg_ms * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
        peak = MFMA_FP8_PEAK_TFLOPS if unit == "TFLOP/s" else HBM_PEAK_GBS
        kernels[name] = {"avg_us": round(avg_ms * 1e3, 2), "rate": round(rate, 1), "unit": unit,
                         "frac": round(rate / peak, 4)}
    dom = max(("gemm_fprop", "gemm_dgrad", "gemm_wgrad"), key=lambda k: kernels[k]["avg_us"])
    roof = {"bound": "mfma", "kernel": dom, "achieved": kernels[dom]["rate"],
            "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(kernels[dom]["rate"] / MFMA_FP8_PEAK_TFLOPS, 4), "traffic": measured_traffic(dom)}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": {"workload": "qwen3_8b_mlp_up_proj_fwd_bwd", "M": M, "K": K, "N": N,
                   "x_quant": "rmsnorm_quant", "seed": 1},
        "roofline": roof,
        "kernels": kernels,
        "kernels_timing": KERNELS_TIMING,
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "settle": settle_info(n_settle),
    }
    out["sclk_mhz"] = sustained_sclk(torch, steps)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(d, g_host)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
