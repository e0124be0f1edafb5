"""Single-GPU benchmark of the MoE feed-forward layer through libmoe's C ABI.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--train]

One step = one whole layer pass over one batch: moe_route, moe_permute,
moe_grouped_gate_up, moe_grouped_down, moe_combine, all enqueued on one HIP
stream with the inputs and weights already resident in HBM.  W untimed steps,
then K timed steps between two device synchronisations.  Prints one JSON line:
tokens/s of the layer, plus

  roofline      the dominant kernel (the gate/up grouped GEMM with its SwiGLU
                epilogue): algorithmic bytes (or FLOPs) per launch divided by the
                mean duration of its launches in the timed steps, each bracketed
                by HIP events recorded on the stream it runs on, against the
                MI355X peak that bounds it;
  grouped_ffn   the two grouped GEMMs together (gate/up + down), priced the same
                way: MFMA share of the bf16 peak, and HBM share for the bytes;
  cpu_baseline  the CPU oracle (fp64 NumPy, self-contained routing) timed on the
                host cores on the same workload.

Run with no --workload (the driver's invocation), the line also carries
`train`: the layer's training pass (below) on the padded XS.2 batch, 40 steps
measured after the forward line's timed region, with its weight-gradient
roofline.

Before the W warmup steps an untimed settle phase runs steps until at least
40 of them and 100 ms of device time have passed (the clocks take some tens of
milliseconds of load to settle); its length is reported as `settle`.

With --train, one step is the training pass instead (forward keeping the
activations the backward needs, then every gradient), on the padded XS.2
training batch by default; its roofline entry is the weight-gradient kernel.

Synthetic seeded inputs; random-init weights of the layer's shape.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from mixture_experts_transformer_moe_amd import configs  # noqa: E402

METRIC = "MoE-layer tokens/s at 1 MI355X; % of bf16 MFMA peak (prefill) / HBM GB/s (decode)"
EV_EVERY = 4
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3

# HBM bytes of one gate/up launch as read by rocprofv3 (FETCH_SIZE and WRITE_SIZE,
# KiB per dispatch, one counter per run of this script with --copy-mib 256),
# each scaled by what the same counter reads for a plain 256 MiB device copy
# (FETCH_SIZE reads half of the copy's bytes, WRITE_SIZE all of them).  A record
# holds only for the kernel sources it was taken on: after any change to them
# the traffic is reported as null until the counters are taken again.
FETCH_FACTOR = 2.0
WRITE_FACTOR = 1.0
GEMM_SOURCES = ("grouped_gemm.hip", "grouped_gemm_lds.hip", "grouped_gemm.h", "mma_stream.h", "lds_dma.h",
                "moe_internal.h")
TRAFFIC = {
    # workload: (FETCH_SIZE KiB, WRITE_SIZE KiB, sha256 of GEMM_SOURCES)
    "prefill_outlier_bf16_t32768_d2048": (2220334.4, 296593.7,
                                          "7a444bd95cd2e0f0d71c371dd3d20d23890a983b340c180b63e9797b254bd5ef"),
    "xs2_bf16_t4096_d2048": (657312.4, 36864.3,
                             "7a444bd95cd2e0f0d71c371dd3d20d23890a983b340c180b63e9797b254bd5ef"),
    "m1_bf16_t8192_d4096": (3305043.9, 147597.8,
                            "7a444bd95cd2e0f0d71c371dd3d20d23890a983b340c180b63e9797b254bd5ef"),
    "m1_top16_bf16_t8192_d4096": (5444833.1, 278859.4,
                                  "7a444bd95cd2e0f0d71c371dd3d20d23890a983b340c180b63e9797b254bd5ef"),
    "decode_zipf_bf16_t32_d4096": (493915.0, 576.0,
                                   "7a444bd95cd2e0f0d71c371dd3d20d23890a983b340c180b63e9797b254bd5ef"),
}


# The same for one launch of the weight-gradient kernel in the training pass.
WGRAD_SOURCES = ("wgrad.hip", "lds_dma.h", "moe_internal.h")
WGRAD_TRAFFIC = {
    "xs2_train_bf16_t4096_d2048": (250806.5, 1581073.2,
                                   "ec40073f6eb5ff1c325864b70a7ecb9ecbf6943d6d6224261cb66c932b35412f"),
}


def sources_sha256(files=GEMM_SOURCES) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "mixture_experts_transformer_moe_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, table=TRAFFIC, files=GEMM_SOURCES):
    rec = table.get(workload)
    if rec is None or rec[2] != sources_sha256(files):
        return None
    return (rec[0] * FETCH_FACTOR + rec[1] * WRITE_FACTOR) * 1024.0


def gate_up_work(s: configs.MoEShape, n_touched: int, fp8: bool = False, shared: bool = True):
    """Algorithmic FLOPs and HBM bytes of one gate/up grouped-GEMM launch.

    bytes = weights of the touched routed experts (2F x D each) + shared weights
            (1 byte per weight and a 4-byte scale per row with FP8 weights)
          + A rows read (k*T routed rows and T shared rows of width D)
          + h written ((k*T*F + T*Fs) elements).
    shared=False: a launch over the routed experts only (the shared expert runs
    in moe_shared_ffn).
    """
    if not shared:
        s = configs.variant(s, Fs=0)
    el = 2 if s.dtype == "bf16" else 4
    flops = 4.0 * s.S * s.D * s.F + 4.0 * s.T * s.D * s.Fs
    if fp8:
        w = (n_touched * 2 * s.F + 2 * s.Fs) * (s.D + 4)
    else:
        w = (n_touched * 2 * s.F * s.D + 2 * s.Fs * s.D) * el
    a = (s.S + (s.T if s.Fs else 0)) * s.D * el
    h = (s.S * s.F + s.T * s.Fs) * el
    return flops, float(w + a + h)


def down_work(s: configs.MoEShape, n_touched: int, fp8: bool = False, shared: bool = True):
    """Algorithmic FLOPs and HBM bytes of one down grouped-GEMM launch:
    weights of the touched routed experts (D x F each) + shared weights (1 byte
    per weight and a 4-byte scale per row with FP8 weights) + h rows read
    ((k*T*F + T*Fs) elements) + y rows written ((k*T + T) rows of width D)."""
    if not shared:
        s = configs.variant(s, Fs=0)
    el = 2 if s.dtype == "bf16" else 4
    flops = 2.0 * s.S * s.D * s.F + 2.0 * s.T * s.D * s.Fs
    if fp8:
        w = (n_touched * s.D + (s.D if s.Fs else 0)) * 4 + (n_touched * s.D * s.F + s.D * s.Fs)
    else:
        w = (n_touched * s.D * s.F + s.D * s.Fs) * el
    h = (s.S * s.F + s.T * s.Fs) * el
    y = (s.S + (s.T if s.Fs else 0)) * s.D * el
    return flops, float(w + h + y)


def settle(step, min_steps: int = 40, min_ms: float = 100.0):
    """Untimed steps until at least min_steps of them and min_ms of wall time
    (with the device synchronised after each step) have passed."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while n < min_steps or (time.perf_counter() - t0) * 1e3 < min_ms:
        step()
        torch.cuda.synchronize()
        n += 1
    return {"steps": n, "ms": round((time.perf_counter() - t0) * 1e3, 1)}


def cpu_oracle_baseline(s, inp_host, target_s: float = 12.0, fp8: bool = False, gpu_topk=None):
    """Times the CPU oracle (self-contained fp64 forward) on host cores (with FP8
    weights: the oracle's FP8 reading of every expert, quantised as it goes).
    With gpu_topk ([T, k] expert ids from the GPU's fp32 logits) it also counts
    the sampled tokens whose self-contained fp64 routing selects another set of
    experts (near-ties between fp32 and fp64 logits; expected 0)."""
    from oracle import moe_oracle as O
    from oracle import fp8_oracle as F8
    wrap = F8.Fp8Weights if fp8 else (lambda inputs: inputs)
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1

    class Sub:
        def __init__(self, n):
            self.x = inp_host["x"][:n]
            self.w_router = inp_host["w_router"]
            self.bias = inp_host["bias"]

        def expert(self, e):
            return inp_host["wgu"][e], inp_host["wd"][e]

        def shared(self):
            return inp_host["shared"]

    # probe on a small slice, then size the sample to about target_s seconds
    n0 = min(s.T, 256)
    t0 = time.perf_counter()
    O.forward(wrap(Sub(n0)), s.alpha, s.k)
    probe = time.perf_counter() - t0
    n = s.T if probe * s.T / n0 <= target_s * 1.5 else max(n0, int(n0 * target_s / probe))
    n = min(n, s.T)
    passes, tokens, t0 = 0, 0, time.perf_counter()
    while True:
        _, routing = O.forward(wrap(Sub(n)), s.alpha, s.k)
        passes += 1
        tokens += n
        el = time.perf_counter() - t0
        if el >= min(target_s, 10.0) or passes >= 8:
            break
    sample = (f"self-contained fp64 oracle forward{' with FP8 weights' if fp8 else ''} over the first {n} of {s.T} tokens "
              f"(all experts they select), {passes} pass(es), weights already in host memory")
    res = {"value": tokens / el, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
           "sample": sample, "seconds": round(el, 3)}
    if gpu_topk is not None:
        cpu_sets = np.sort(np.asarray(routing.topk_idx)[:n], axis=1)
        gpu_sets = np.sort(np.asarray(gpu_topk)[:n], axis=1)
        res["routing_compared"] = int(n)
        res["routing_differs"] = int(np.count_nonzero((cpu_sets != gpu_sets).any(axis=1)))
    return res


def wgrad_work(s: configs.MoEShape, routed_rows: int):
    """Algorithmic FLOPs and HBM bytes of one weight-gradient launch
    (moe_weight_grads): every gradient written once (bf16 experts, fp32
    router) and every input tensor read once (x, [dg | du], dy, dout, h and the
    bf16 logit gradient; R = routed rows, T = tokens)."""
    R, T, D, F, Fs, E = routed_rows, s.T, s.D, s.F, s.Fs, s.E
    flops = 2.0 * R * (2 * F * D + D * F) + 2.0 * T * (2 * Fs * D + D * Fs) + 2.0 * T * E * D
    out = (E * (2 * F * D + D * F) + (2 * Fs * D + D * Fs)) * 2 + E * D * 4
    inp = (T * D + (R * 2 * F + T * 2 * Fs) + R * D + T * D + (R * F + T * Fs) + T * 256) * 2
    return flops, float(out + inp)


def train_flops(s: configs.MoEShape, routed_rows: int) -> float:
    """FLOPs of one training pass: the forward (router, both expert GEMMs,
    shared expert) and, for each of its products, the two backward products."""
    R, T = routed_rows, s.T
    fwd = 2.0 * T * s.D * s.E + 6.0 * R * s.D * s.F + 6.0 * T * s.D * s.Fs
    return 3.0 * fwd


def cpu_train_baseline(s, inp_host, mask, dout, target_s: float = 12.0):
    """Times the training oracle (fp64 forward + backward) on a token sample."""
    from oracle import moe_oracle as O
    from oracle import train_oracle as TR
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1

    class Sub:
        def __init__(self, n):
            self.x = inp_host["x"][:n]
            self.w_router = inp_host["w_router"]
            self.bias = inp_host["bias"]

        def expert(self, e):
            return inp_host["wgu"][e], inp_host["wd"][e]

        def shared(self):
            return inp_host["shared"]

    def one(n):
        sub = Sub(n)
        out, r = TR.forward(sub, s.alpha, s.k, mask[:n])
        TR.backward(sub, s.alpha, r, dout[:n], s.aux_coef)

    n0 = min(s.T, 128)
    t0 = time.perf_counter()
    one(n0)
    probe = time.perf_counter() - t0
    n = min(s.T, max(n0, int(n0 * target_s / probe)))
    passes, tokens, t0 = 0, 0, time.perf_counter()
    while True:
        one(n)
        passes += 1
        tokens += n
        el = time.perf_counter() - t0
        if el >= min(target_s, 10.0) or passes >= 8:
            break
    sample = (f"fp64 training oracle (masked forward with its own routing, then the backward of every "
              f"expert touched, shared expert and router) over the first {n} of {s.T} tokens, "
              f"{passes} pass(es), weights already in host memory")
    return {"value": tokens / el, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": sample, "seconds": round(el, 3)}


def copy_calibration(mib: int, dev) -> None:
    """Three device-to-device copies of a buffer of known size (for HBM counters)."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def vendor_gemm(s: configs.MoEShape) -> None:
    """The vendor library (torch.bmm / torch.mm, bf16) on the layer's expert
    products with every expert given the mean rows per expert (k T / E): the
    routed gate/up [E, M, D] x [E, D, 2F], down [E, M, F] x [E, F, D], and the
    shared expert's two products.  Context only: uniform shapes, no gather, no
    SwiGLU, no tile table; prints one JSON line."""
    import torch
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(0)
    M = max(1, s.S // s.E)

    def timed(f, n=20):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.2:          # clocks settle under load
            f()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            f()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    out = {"workload": s.name, "rows_per_expert": M}
    for name, (bt, m, k, n) in {"gate_up": (s.E, M, s.D, 2 * s.F), "down": (s.E, M, s.F, s.D),
                                "shared_gate_up": (1, s.T, s.D, 2 * s.Fs),
                                "shared_down": (1, s.T, s.Fs, s.D)}.items():
        if n == 0 or k == 0:
            continue
        a = torch.randn(bt, m, k, device=dev, dtype=torch.bfloat16, generator=g)
        w = torch.randn(bt, k, n, device=dev, dtype=torch.bfloat16, generator=g).contiguous()
        ms = timed(lambda: torch.bmm(a, w)) if bt > 1 else timed(lambda: torch.mm(a[0], w[0]))
        fl = 2.0 * bt * m * n * k
        out[name] = {"shape": [bt, m, k, n], "us": round(ms * 1e3, 1),
                     "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                     "mfma_frac": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del a, w
    print(json.dumps(out), flush=True)


def train_main(args):
    """Prints the training pass's JSON line (see train_measure)."""
    print(json.dumps(train_measure(args)), flush=True)


def train_measure(args) -> dict:
    """One step = the training pass: masked route, permute, load statistics,
    gate/up keeping the pre-activations, down, combine; then the combine
    backward, dh and SwiGLU backward, dx, weight and bias gradients."""
    import torch
    from mixture_experts_transformer_moe_amd import binding
    from mixture_experts_transformer_moe_amd.inputs import LayerInputs, dout_encoded, token_mask

    s = configs.get(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = LayerInputs(s)
    wgu, wd = inp.all_experts()
    host = {"x": inp.x, "w_router": inp.w_router, "bias": inp.bias, "wgu": wgu, "wd": wd,
            "shared": inp.shared()}
    w = binding.upload_train_weights(s, inp.w_router, inp.bias, wgu, wd, host["shared"], dev)
    x = binding.to_device(inp.x, s, dev)
    mask_h, dout_h = token_mask(s), dout_encoded(s)
    mask = torch.from_numpy(mask_h).to(dev)
    dout = binding.to_device(dout_h, s, dev)
    b = binding.alloc_train_buffers(s, mask, dev, with_x_perm=args.x_perm)
    c = binding.make_shape(s)
    stream = torch.cuda.current_stream(dev)
    fb = b.fwd

    def step(ev=None):
        binding.train_forward(s, x, w, b, s.aux_coef, None, stream)
        binding.moe_combine_backward(c, dout, fb.y_perm, fb.slot_of, fb.topk_idx, fb.topk_w, fb.logits,
                                     b.aux_coef, b.dy_perm, b.dz, b.dz16, stream)
        binding.moe_grouped_backward_h(c, b.dy_perm, dout, fb.offsets, w.w_down_t, w.ws_down_t, b.gu,
                                       b.dh, b.dgu, stream)
        binding.moe_grouped_backward_x(c, b.dgu, fb.offsets, w.w_gate_up_t, w.ws_gate_up_t, b.dz16,
                                       w.w_router_t, fb.slot_of, b.dx_perm, b.dx_shared, b.dx_router,
                                       b.dx, stream)
        if ev is not None:
            ev[0].record(stream)
        binding.moe_weight_grads(c, x, fb.sorted_token, fb.x_perm, fb.offsets, b.dgu, b.dy_perm, dout,
                                 fb.h, b.dz16, b.dw_gate_up, b.dw_down, b.dws_gate_up, b.dws_down,
                                 b.dw_router, stream)
        if ev is not None:
            ev[1].record(stream)
        binding.moe_bias_grad(c, b.dz, b.dbias, b.train_ws, stream)

    settled = settle(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timed = list(range(0, args.steps, EV_EVERY))
    evs = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for i in timed}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs.get(i))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    wg_ms = float(np.mean([a.elapsed_time(z) for a, z in evs.values()]))
    if args.copy_mib > 0:
        copy_calibration(args.copy_mib, dev)

    routed_rows = int(fb.offsets[-1].item())
    flops, nbytes = wgrad_work(s, routed_rows)
    achieved = nbytes / (wg_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(s.name, WGRAD_TRAFFIC, WGRAD_SOURCES),
            "kernel": "wgrad_kernel (moe_weight_grads)", "kernel_ms": round(wg_ms, 4),
            "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
            "mfma_tflops": round(flops / (wg_ms * 1e-3) / 1e12, 1)}
    ms = elapsed * 1e3 / args.steps
    cpu = None if args.no_cpu_baseline else cpu_train_baseline(s, host, mask_h, dout_h)
    line = {
        "metric": "MoE-layer training tokens/s (forward + backward) at 1 MI355X",
        "value": round(s.T * args.steps / elapsed, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle": settled, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": s.dtype,
        "data": "synthetic",
        "config": {"workload": s.name, "tokens": s.T, "routed_tokens": routed_rows // s.k,
                   "d_model": s.D, "experts": s.E, "top_k": s.k, "expert_width": s.F,
                   "shared_width": s.Fs, "alpha": s.alpha, "aux_coef": s.aux_coef,
                   "a_rows": "x_perm" if args.x_perm else "gather", "parallelism": "single-gpu"},
        "train_tflops": round(train_flops(s, routed_rows) / (ms * 1e-3) / 1e12, 1),
        "aux_loss": float(b.aux_loss.item()),
        "roofline": roof, "cpu_baseline": cpu,
    }
    return line


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # (an untimed settle phase runs before these: at least 40 steps and 100 ms)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, choices=sorted(configs.WORKLOADS),
                    help=f"default {configs.BENCH_WORKLOAD} (with the training summary)")
    ap.add_argument("--split-shared", action="store_true",
                    help="run the shared expert on a second stream beside the router and the "
                         "permutation (moe_shared_ffn), the grouped GEMMs over the routed experts only")
    ap.add_argument("--x-perm", action="store_true",
                    help="materialise x_perm in moe_permute and read it in the first GEMM "
                         "(default: the first GEMM gathers token rows through sorted_token)")
    ap.add_argument("--fp8-weights", action="store_true",
                    help="expert weights in FP8 (E4M3, per-row scales; moe_quantize_weights_fp8) "
                         "and the FP8 grouped GEMMs")
    ap.add_argument("--train", action="store_true",
                    help="time the training pass (forward keeping activations, then the backward "
                         "and every gradient) on the training workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed steps, copy a buffer of this many MiB device to device "
                         "three times (a plain copy of known size, to calibrate HBM byte counters)")
    ap.add_argument("--no-train-summary", action="store_true",
                    help="skip the short training-pass measurement whose summary the default forward "
                         "line carries (it is taken only when --workload is not given)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="instead of the layer: time the vendor library's batched bf16 GEMM (torch.bmm) "
                         "on the workload's expert products at uniform rows per expert, as context for "
                         "the grouped GEMMs' MFMA fraction")
    args = ap.parse_args()
    train_summary = args.workload is None and not args.no_train_summary and not args.train
    if args.workload is None:
        args.workload = configs.BENCH_WORKLOAD
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the layer's "
              "multi-GPU sharding is a design note, not a measured path.", file=sys.stderr)
        sys.exit(2)

    if args.vendor_gemm:
        vendor_gemm(configs.get(args.workload))
        return
    if args.train:
        if args.workload == configs.BENCH_WORKLOAD:
            args.workload = configs.XS2_TRAIN_T4096.name
        train_main(args)
        return

    import torch
    from mixture_experts_transformer_moe_amd import binding
    from mixture_experts_transformer_moe_amd.inputs import LayerInputs

    s = configs.get(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = LayerInputs(s)
    wgu, wd = inp.all_experts()
    host = {"x": inp.x, "w_router": inp.w_router, "bias": inp.bias, "wgu": wgu, "wd": wd,
            "shared": inp.shared()}
    # expert weights are packed once into MFMA fragment order (moe_pack_weights)
    w = binding.upload_weights(s, inp.w_router, inp.bias, wgu, wd, host["shared"], dev,
                               fp8=args.fp8_weights)
    x = binding.to_device(inp.x, s, dev)
    b = binding.alloc_buffers(s, dev, with_x_perm=args.x_perm)
    c = binding.make_shape(s)
    stream = torch.cuda.current_stream(dev)

    split = args.split_shared and not w.fp8 and s.Fs > 0 and s.dtype == "bf16"
    if split:
        side = torch.cuda.Stream(device=dev)
        ev_shared, ev_done = torch.cuda.Event(), torch.cuda.Event()
        ev_done.record(stream)
        h_shared = b.h[s.T * s.k * s.F:]

    def step(ev=None, marks=None):
        def mark(i):
            if marks is not None:
                marks[i].record(stream)
        if split:
            # the shared expert on a second stream, beside the router and the
            # permutation; it rewrites y_shared once the previous combine is done
            side.wait_event(ev_done)
            binding.moe_shared_ffn(c, x, w.ws_gate_up, w.ws_down, h_shared, b.y_shared, side)
            ev_shared.record(side)
        mark(0)
        binding.moe_route(c, x, w.w_router, w.bias, b.logits, b.topk_idx, b.topk_w, stream)
        mark(1)
        binding.moe_permute(c, b.topk_idx, x, b.counts, b.offsets, b.sorted_token, b.slot_of,
                            b.x_perm, b.workspace, stream)
        mark(2)
        if ev is not None:
            ev[0].record(stream)
        if w.fp8:
            binding.moe_grouped_gate_up_fp8(c, b.x_perm, b.sorted_token, x, b.offsets, w.w_gate_up,
                                            w.w_gate_up_scale, w.ws_gate_up, w.ws_gate_up_scale,
                                            b.h, stream)
        else:
            binding.moe_grouped_gate_up(c, b.x_perm, b.sorted_token, x, b.offsets, w.w_gate_up,
                                        None if split else w.ws_gate_up, b.h, stream)
        if ev is not None:
            ev[1].record(stream)
        mark(3)
        if ev is not None:
            ev[2].record(stream)
        if w.fp8:
            binding.moe_grouped_down_fp8(c, b.h, b.offsets, w.w_down, w.w_down_scale, w.ws_down,
                                         w.ws_down_scale, b.y_perm, b.y_shared, stream)
        else:
            binding.moe_grouped_down(c, b.h, b.offsets, w.w_down, None if split else w.ws_down,
                                     b.y_perm, b.y_shared, stream)
        if ev is not None:
            ev[3].record(stream)
        mark(4)
        if split:
            stream.wait_event(ev_shared)
        binding.moe_combine(c, b.y_perm, b.y_shared, b.slot_of, b.topk_w, b.out, stream)
        mark(5)
        if split:
            ev_done.record(stream)

    settled = settle(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # every timed step brackets its gate/up and down launches with HIP events
    # on their stream (each event costs the stream a few microseconds)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gu_times = [e[0].elapsed_time(e[1]) for e in evs]
    dn_times = [e[2].elapsed_time(e[3]) for e in evs]
    gate_up_ms = float(np.mean(gu_times))
    down_ms = float(np.mean(dn_times))

    # per-call medians (untimed pass after the timed steps: events between the
    # calls on the layer's stream, 20 steps after 5 warmup ones)
    calls = ("route", "permute", "gate_up", "down", "combine")
    per_call = {n: [] for n in calls}
    for i in range(25):
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        step(marks=marks)
        torch.cuda.synchronize()
        if i >= 5:
            for j, n in enumerate(calls):
                per_call[n].append(marks[j].elapsed_time(marks[j + 1]))
    calls_ms = {n: round(float(np.median(v)), 4) for n, v in per_call.items()}

    if args.copy_mib > 0:
        copy_calibration(args.copy_mib, dev)

    counts = b.counts.cpu().numpy()
    n_touched = int(np.count_nonzero(counts))
    flops, nbytes = gate_up_work(s, n_touched, args.fp8_weights, shared=not split)
    dflops, dbytes = down_work(s, n_touched, args.fp8_weights, shared=not split)
    intensity = flops / nbytes
    peak_flops = PEAK_BF16_TFLOPS if s.dtype == "bf16" else PEAK_F32_TFLOPS
    ridge = peak_flops * 1e12 / (PEAK_HBM_GBS * 1e9)
    if intensity < ridge:
        achieved = nbytes / (gate_up_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = flops / (gate_up_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak_flops,
                "unit": "TFLOP/s", "frac": round(achieved / peak_flops, 4)}
    traffic = None if (args.fp8_weights or split) else measured_traffic(s.name)
    kname = ("grouped_gemm_kernel<gate_up, FP8 weights> (moe_grouped_gate_up_fp8)" if args.fp8_weights
             else "gate/up grouped GEMM (moe_grouped_gate_up, routed experts only)" if split
             else "gate/up grouped GEMM (moe_grouped_gate_up)")
    roof.update({"traffic": traffic, "kernel": kname,
                 "kernel_ms": round(gate_up_ms, 4), "kernel_ms_median": round(float(np.median(gu_times)), 4),
                 "launches": len(gu_times), "algorithmic_bytes": nbytes,
                 "algorithmic_flops": flops,
                 "mfma_tflops": round(flops / (gate_up_ms * 1e-3) / 1e12, 1)})
    # the grouped FFN (a6 + a7) as a whole, from the same timed launches
    ffn_ms = gate_up_ms + down_ms
    ffn = {"gate_up_ms": round(gate_up_ms, 4), "down_ms": round(down_ms, 4),
           "flops": flops + dflops, "bytes": nbytes + dbytes,
           "mfma_tflops": round((flops + dflops) / (ffn_ms * 1e-3) / 1e12, 1),
           "mfma_frac": round((flops + dflops) / (ffn_ms * 1e-3) / 1e12 / peak_flops, 4),
           "hbm_gbs": round((nbytes + dbytes) / (ffn_ms * 1e-3) / 1e9, 1),
           "hbm_frac": round((nbytes + dbytes) / (ffn_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "graded_on": "mfma" if intensity >= ridge else "hbm"}

    ms = elapsed * 1e3 / args.steps
    tokens_per_s = s.T * args.steps / elapsed
    layer_tflops = s.flops() / (ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_oracle_baseline(s, host, fp8=args.fp8_weights, gpu_topk=b.topk_idx.cpu().numpy())
    line = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle": settled, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": s.dtype,
        "data": "synthetic",
        "config": {"workload": s.name, "tokens": s.T, "d_model": s.D, "experts": s.E,
                   "top_k": s.k, "expert_width": s.F, "shared_width": s.Fs, "alpha": s.alpha,
                   "a_rows": "x_perm" if args.x_perm else "gather",
                   "expert_weights": "fp8-e4m3-row-scaled" if args.fp8_weights else "bf16",
                   "parallelism": "single-gpu"},
        "layer_tflops": round(layer_tflops, 1),
        "experts_touched": n_touched, "rows_per_expert_max": int(counts.max()),
        "calls_median_ms": calls_ms,
        "tokens_per_s_from_call_medians": round(s.T / (sum(calls_ms.values()) * 1e-3), 1),
        "roofline": roof, "grouped_ffn": ffn, "cpu_baseline": cpu,
    }
    if train_summary:
        # the layer's training pass on its own workload (the padded XS.2
        # batch), measured after the forward line's timed region, with no CPU
        # leg; its full line comes from --train
        targs = argparse.Namespace(workload=configs.XS2_TRAIN_T4096.name, steps=40, warmup=5,
                                   no_cpu_baseline=True, x_perm=False, copy_mib=0)
        t = train_measure(targs)
        line["train"] = {"workload": t["config"]["workload"], "tokens_per_s": t["value"],
                         "ms_per_step": t["ms_per_step"], "steps": t["steps"], "settle": t["settle"],
                         "train_tflops": t["train_tflops"],
                         "wgrad_roofline": {k: t["roofline"][k] for k in ("bound", "achieved", "peak", "unit",
                                                                          "frac", "kernel_ms")}}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
