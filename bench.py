#!/usr/bin/env python
"""Throughput of the grouped fake-quant expert layer, forward + backward, on one MI355X.

One step = fq_grouped_expert_fwd + fq_grouped_expert_bwd over one batch of
synthetic input: routing, weight fake-quant of both stacks, permute + A1, fc1,
SwiGLU + A2, fc2, combine, then the straight-through backward down to the
weight- and activation-scale gradients, dX and d topk_w.  Inputs are resident
in HBM before the timed region.  Per-stage times come from hipEvents the
library records on its stream at stage boundaries.

Default workload: the Qwen3-30B-A3B-shaped NVFP4 (W4A4) layer, 128 experts,
hidden 2048, expert intermediate 768, top-8 over 16384 tokens (seq 2048 x
micro-batch 8) with Zipf(1.1) expert load.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload qwen3]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA

WORKLOADS = {
    # name: (synth case, format, description, backward to dX and d topk_w)
    "qwen3": ("qwen3", "nvfp4", "Qwen3-30B-A3B-shaped MoE layer nvfp4 W4A4, E=128 H=2048 I=768 top-8, "
                                 "T=16384, Zipf(1.1) load", True),
    # forward + weight-scale gradients only: no dX, so no fc1 data gradient or
    # A1 backward (the A1 quantiser is dynamic and has no parameter)
    "qwen3_w8a8": ("qwen3u", "w8a8", "same layer w8a8, T=16384, uniform routing, fwd + weight-scale grads",
                   False),
    "qwen3_w4afp8": ("qwen3l", "w4afp8", "same layer w4afp8, T=32768, Zipf(1.1) load", True),
    "qwen3_fp8": ("qwen3l", "fp8", "same layer fp8, T=32768, Zipf(1.1) load", True),
}
# stages that do no work when the backward stops at the weight-scale gradients
DX_STAGES = ("fc1_dgrad", "unpermute_a1", "a1_sum")


def _scale_elems(q, rows, cols):
    """Scale elements one [rows, cols] matrix reads under descriptor q (along cols)."""
    from scale_only_quantization_amd import fqlib as F
    if q.kind == F.FQ_NONE or q.source == F.FQ_DYNAMIC:
        return 0
    if q.kind == F.FQ_NVFP4:
        return rows * (cols // 16)
    if q.gran == F.FQ_PER_GROUP:
        return rows * (cols // q.group)
    return rows if q.gran == F.FQ_PER_ROW else 1


def _scale_grad_fused(q):
    """True where the weight-gradient GEMM's epilogue writes the scale gradient
    itself (NVFP4 blocks, INT groups of 16), so no reduction stage follows."""
    from scale_only_quantization_amd import fqlib as F
    return q.kind == F.FQ_NVFP4 or (q.gran == F.FQ_PER_GROUP and q.group == 16)


def stage_work(dims, descs, full_bwd=True):
    """Algorithmic bytes (HBM kernels) or FLOPs (GEMMs) of each stage per launch,
    for layer sizes `dims` (E, H, I, T, k) and quantiser descriptors
    (w1, w2, a1, a2); without the full backward, permute_dy forms no d topk_w
    (no read of Y_r)."""
    E, H, I, T, k = dims.E, dims.H, dims.I, dims.T, dims.k
    w1q, w2q = descs[0], descs[1]
    R = T * k
    bf, f4 = 2, 4
    sw1 = E * _scale_elems(w1q, 2 * I, H) * f4
    sw2 = E * _scale_elems(w2q, H, I) * f4
    W1, W2 = E * 2 * I * H * bf, E * H * I * bf
    fwd = {
        "route": ("hbm", R * 4 * 3),
        "w1_fq": ("hbm", 2 * W1 + sw1),
        "w2_fq": ("hbm", 2 * W2 + sw2),
        "permute_a1": ("hbm", T * H * bf + R * H * bf),
        "fc1": ("mfma", 2.0 * R * 2 * I * H),
        "swiglu_a2": ("hbm", R * 2 * I * bf + R * I * bf),
        "fc2": ("mfma", 2.0 * R * H * I),
        "combine": ("hbm", R * H * bf + T * H * bf + R * 4),
    }
    bwd = {
        "permute_dy": ("hbm", T * H * bf + R * H * bf + (R * H * bf if full_bwd else 0)),
        "fc2_dgrad": ("mfma", 2.0 * R * H * I),
        "fc2_wgrad": ("mfma", 2.0 * R * H * I),
        "swiglu_bwd": ("hbm", 2 * R * 2 * I * bf + R * I * bf),
        "a2_sum": ("hbm", R * 4),
        "fc1_dgrad": ("mfma", 2.0 * R * 2 * I * H),
        "fc1_wgrad": ("mfma", 2.0 * R * 2 * I * H),
        "unpermute_a1": ("hbm", 2 * T * H * bf + R * H * bf),
        "a1_sum": ("hbm", R * 4),
        # the weight-scale gradients: formed in the weight-gradient GEMM's
        # epilogue for NVFP4 blocks and INT groups of 16 (nothing left for this
        # stage), else summed from its per-32-column partials
        "w1_scale_grad": ("hbm", 0 if _scale_grad_fused(w1q) else W1 // 2 * 4 // 32 + sw1),
        "w2_scale_grad": ("hbm", 0 if _scale_grad_fused(w2q) else W2 // 2 * 4 // 32 + sw2),
    }
    return fwd, bwd


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch loaded (the one libfq uses)."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            h = ctypes.c_void_p()
            assert self.rt.hipEventCreate(ctypes.byref(h)) == 0
            out.append(h.value)
        return out

    def record(self, e, stream=None):
        assert self.rt.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream)) == 0

    def sync(self, e):
        assert self.rt.hipEventSynchronize(ctypes.c_void_p(e)) == 0

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.rt.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return ms.value


# Stages grouped by the kernel that runs them, with the sources that kernel is
# built from (a counter summary is valid only for those sources).
KERNELS = {
    "gemm_fwd": (("fc1", "fc2"), ("fq_gemm.hip",)),
    "gemm_dgrad": (("fc2_dgrad", "fc1_dgrad"), ("fq_gemm.hip",)),
    "gemm_wgrad": (("fc2_wgrad", "fc1_wgrad"), ("fq_gemm.hip",)),
    "tensor_fwd": (("w1_fq", "w2_fq"), ("fq_tensor.hip",)),
    # nvfp4: nothing (formed in gemm_wgrad's epilogue); INT/FP8: sums of its partials
    "weight_scale_grad": (("w1_scale_grad", "w2_scale_grad"), ("fq_gemm.hip", "fq_tensor.hip")),
    "route": (("route",), ("fq_layer.hip",)),
    "permute_a1": (("permute_a1",), ("fq_layer.hip",)),
    "swiglu_a2": (("swiglu_a2",), ("fq_layer.hip",)),
    "combine": (("combine",), ("fq_layer.hip",)),
    "permute_dy": (("permute_dy",), ("fq_layer.hip",)),
    "swiglu_bwd": (("swiglu_bwd",), ("fq_layer.hip",)),
    "segment_sum": (("a2_sum", "a1_sum"), ("fq_layer.hip",)),
    "unpermute_a1": (("unpermute_a1",), ("fq_layer.hip",)),
}
COMMON_SOURCES = ("fq_common.h", "fq_internal.h")


def traffic_from_profiles(kernel, workload):
    """HBM bytes per launch of `kernel` from a committed counter summary, if it
    was taken on the current sources of that kernel; else None."""
    path = os.path.join(ROOT, "profiles", f"counters_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k_, v = line.split(":", 1)
            kv[k_.strip()] = v.strip()
    if kv.get("sources_sha") != sources_sha(kernel):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def sources_sha(kernel):
    h = hashlib.sha256()
    d = os.path.join(ROOT, "scale_only_quantization_amd", "csrc")
    for n in sorted(KERNELS[kernel][1] + COMMON_SOURCES):
        h.update(open(os.path.join(d, n), "rb").read())
    return h.hexdigest()[:16]


def scale_adamw_step(ev, F, dl, reps=20, warmup=3):
    """The scale optimiser step (fq_scale_adamw) over the layer's learnable
    scales with the gradients of the last backward: NVFP4 block scales of both
    stacks (projected against their tensor scales) and the activation tensor
    scales.  Algorithmic bytes: the norm pass reads g (4 B per element), the
    update reads p, g, m, v and writes p, m, v (28 B)."""
    import torch
    params, keep, count = [], [], 0
    for n, q in dl.q.items():
        g = dl.g.get("ds_" + n)
        if g is None:
            continue
        p = dl.d["s_" + n]
        m, v = torch.zeros_like(p), torch.zeros_like(p)
        # NVFP4 weight block scales are projected against their tensor scale
        t = dl.d.get("t_" + n) if n.startswith("w") and q.kind == F.FQ_NVFP4 else None
        per = p.numel() // t.numel() if t is not None else 1
        keep += [m, v]
        params.append(F.scale_param(p, g, m, v, t, per))
        count += p.numel()
    if not params:
        return None
    ws = torch.empty(F.scale_adamw_workspace_size(params) // 4 + 1, dtype=torch.float32, device="cuda")
    hp = F.adamw_defaults()
    for i in range(warmup):
        F.scale_adamw(params, hp, 1 + i, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = ev.create(2)
    ev.record(e0)
    for i in range(reps):
        F.scale_adamw(params, hp, 1 + warmup + i, workspace=ws)
    ev.record(e1)
    ev.sync(e1)
    ms = ev.elapsed_ms(e0, e1) / reps
    alg = 32 * count
    gbs = alg / (ms * 1e-3) / 1e9
    return dict(ms=round(ms, 4), gbs=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 3), bytes=alg,
                elements=count, tensors=len(params))


def distill_logits(ev, F, T=16384, V=151936, k=64, reps=5, warmup=2):
    """The distillation loss and its gradient on one batch of logits shaped like
    the pages' Qwen3 runs (seq 2048 x micro-batch 8 tokens, the Qwen3
    vocabulary), student and teacher bf16, seeded on the device.  Algorithmic
    bytes: each logit read once and the bf16 gradient written once (6 B per
    element with the full teacher, 4 B with its top-k)."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(2024)
    zs = (torch.randn((T, V), generator=g, device="cuda") * 2.0).to(torch.bfloat16)
    zt = (zs.float() * 1.3 + torch.randn((T, V), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    labels = torch.randint(0, V, (T,), generator=g, device="cuda", dtype=torch.int32)
    tv, ti = torch.topk(zt.float(), k, dim=-1)
    ti = ti.to(torch.int32).contiguous()
    grad = torch.empty_like(zs)
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(F.lib().fq_distill_workspace_size(T) // 4, dtype=torch.float32, device="cuda")
    out = {}
    for kind, kk, kw, per in (("cakld", 0, dict(teacher=zt), 6), ("topk_kl", k, dict(top_v=tv, top_i=ti), 4)):
        d = F.distill_desc(kind, topk=kk)

        def fn():
            F.distill_loss(d, zs, loss, labels=labels, grad=grad, workspace=ws, **kw)
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = ev.create(2)
        ev.record(e0)
        for _ in range(reps):
            fn()
        ev.record(e1)
        ev.sync(e1)
        ms = ev.elapsed_ms(e0, e1) / reps
        alg = per * T * V
        gbs = alg / (ms * 1e-3) / 1e9
        out[kind] = dict(ms=round(ms, 4), gbs=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 3), bytes=alg)
    out["shape"] = [T, V]
    out["topk"] = k
    del zs, zt, grad, tv, ti
    torch.cuda.empty_cache()
    return out


def fake_quant_stack(ev, F, reps=20, warmup=3):
    """Standalone fq_tensor on the weight-only microbench stack: 128 expert
    matrices 768 x 2048 bf16 N(0, 0.02) with 0.1% outliers x 20, NVFP4 block-16
    and INT4 group-128 with learnable fp32 scales (the weight quantisers of the
    library's nvfp4 and w4a16 presets); forward (y), then the straight-through
    scale gradient from an fp32 upstream gradient.  Per call: average over
    `reps` back-to-back calls between two events."""
    import torch

    import synth
    from scale_only_quantization_amd.layer import bf16_to_device
    W, G = synth.make_weight_stack()
    E, N, K = W.shape
    n = W.size
    x = bf16_to_device(W)
    g = torch.from_numpy(G).cuda()
    del G
    y = torch.empty_like(x)
    out = {}
    for name, fmt, kind in (("nvfp4", "nvfp4", "nvfp4"), ("int4_g128", "w4a16", "int4_g")):
        qd = F.preset(fmt)[0]
        c = synth.calibrate_weight(kind, W, group=qd.group)
        s = torch.from_numpy(c["s"]).cuda()
        t = torch.from_numpy(c["t"]).cuda() if "t" in c else None
        ds = torch.empty_like(s)
        nscale = s.numel() * 4
        e0, e1 = ev.create(2)
        res = {}
        for pass_, fn, alg in (
                ("fwd", lambda: F.fq_tensor(qd, x, s, t, y=y), 4 * n + nscale),
                ("bwd", lambda: F.fq_tensor(qd, x, s, t, grad_y=g, grad_scale=ds), 6 * n + 2 * nscale)):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            ev.record(e0)
            for _ in range(reps):
                fn()
            ev.record(e1)
            ev.sync(e1)
            ms = ev.elapsed_ms(e0, e1) / reps
            gbs = alg / (ms * 1e-3) / 1e9
            res[pass_] = dict(ms=round(ms, 4), gbs=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 3),
                              bytes=alg)
        out[name] = res
    out["shape"] = [E, N, K]
    return out


def host_environment():
    """The host CPU: its model, usable cores, numpy and its BLAS."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = {}
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        blas = dict(name=b.get("name"), version=b.get("version"), config=b.get("openblas configuration"))
    except Exception:
        pass
    threads = None
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            threads = max(i.get("num_threads", 1) for i in info)
            blas["runtime"] = f"{info[0].get('internal_api')} {info[0].get('version')}"
    except Exception:
        pass
    return dict(cpu_model=model, affinity_cores=len(os.sched_getaffinity(0)), blas_threads=threads,
                numpy=np.__version__, blas=blas)


def cpu_baseline(data, P, fmt, quantiles=tuple(np.linspace(0.02, 0.98, 25))):
    """Time the oracle (numpy, float64 GEMMs) on a bounded sample: the full forward
    and backward of a few experts, i.e. every routed row of those experts, as a
    sub-layer with one routing slot per row."""
    from oracle import layer as OL
    from oracle import presets as OP
    env = host_environment()
    cores = env["blas_threads"] or env["affinity_cores"]
    case = data["case"]
    ids, w = data["ids"], data["w"]
    counts = np.bincount(ids.ravel(), minlength=case.E)
    order = np.argsort(counts, kind="stable")
    picks = [int(order[int(q * (case.E - 1))]) for q in quantiles]
    tsel, jsel, esel = [], [], []
    for new_e, e in enumerate(picks):
        t, j = np.nonzero(ids == e)
        tsel.append(t)
        jsel.append(j)
        esel.append(np.full(t.size, new_e))
    t = np.concatenate(tsel)
    j = np.concatenate(jsel)
    sub_ids = np.concatenate(esel)[:, None].astype(np.int32)
    Es = len(picks)
    w1, w2, a1, a2 = OP.PRESETS[fmt]
    Ls = OL.LayerSpec(Es, case.H, case.I, t.size, 1, w1, w2, a1, a2)

    def pick(v, idx):
        return None if v is None else np.asarray(v)[idx]
    Ps = dict(W1=data["W1"][picks], W2=data["W2"][picks], s_w1=pick(P["s_w1"], picks),
              t_w1=pick(P["t_w1"], picks), s_w2=pick(P["s_w2"], picks), t_w2=pick(P["t_w2"], picks),
              s_a1=pick(P["s_a1"], picks), s_a2=pick(P["s_a2"], picks))
    X = data["X"][t]
    dY = data["dY"][t]
    ws = w[t, j][:, None]
    t0 = time.perf_counter()
    S = OL.forward(Ls, Ps, X, sub_ids, ws)
    OL.backward(Ls, Ps, S, dY, ws)
    dt = time.perf_counter() - t0
    tokens = t.size / case.k
    return dict(value=tokens / dt, unit="tokens/s", cores=int(cores), kind="oracle", host=env,
                sample=(f"full fwd+bwd of experts {picks} (rows {[int(counts[e]) for e in picks]}, "
                        f"{t.size} routed rows = {tokens:.0f} token-equivalents at top-{case.k}) "
                        f"in {dt:.1f} s"))


def run_layer(name, F, ev, steps, warmup, data=None):
    """One layer workload: seeded inputs, the device layer built from the
    library's preset of its format, `warmup` untimed and `steps` timed
    forward + backward steps, per-stage times and the dominant kernel's
    roofline.  Returns (result, layer, data, params)."""
    import torch

    import synth
    from scale_only_quantization_amd.layer import ExpertLayer, LayerDims

    case_name, fmt, desc, full_bwd = WORKLOADS[name]
    case = synth.CASES[case_name]
    t_gen = time.perf_counter()
    if data is None:
        data = synth.make_layer(case)
    P = synth.layer_params(data, fmt)
    print(f"[bench] inputs for {name} ready in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr,
          flush=True)
    dims = LayerDims(case.E, case.H, case.I, case.T, case.k)
    dl = ExpertLayer(dims, fmt, data["W1"], data["W2"], data["X"], data["ids"], data["w"], data["dY"], P)
    nf, nb = len(F.FWD_STAGES) + 1, len(F.BWD_STAGES) + 1
    evf = [ev.create(nf) for _ in range(steps)]
    evb = [ev.create(nb) for _ in range(steps)]

    def step(i=None):
        dl.forward(events=None if i is None else evf[i])
        dl.backward(dx=full_bwd, dw=full_bwd, events=None if i is None else evb[i])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed * 1e3 / steps
    value = case.T / (ms / 1e3)

    # per-stage durations (ms), averaged over the timed steps
    dur = {}
    for stages_, evs in ((F.FWD_STAGES, evf), (F.BWD_STAGES, evb)):
        for si, n in enumerate(stages_):
            dur[n] = float(np.mean([ev.elapsed_ms(e[si], e[si + 1]) for e in evs]))
    work_f, work_b = stage_work(dims, tuple(dl.q[n] for n in ("w1", "w2", "a1", "a2")), full_bwd)
    work = {**work_f, **work_b}
    if not full_bwd:
        for n in DX_STAGES:
            dur.pop(n)
    stages = {}
    for n, d in dur.items():
        kind, amount = work[n]
        if kind == "mfma":
            ach = amount / (d * 1e-3) / 1e12
            stages[n] = dict(ms=round(d, 4), tflops=round(ach, 1), frac=round(ach / BF16_PEAK_TFLOPS, 3))
        else:
            ach = amount / (d * 1e-3) / 1e9
            stages[n] = dict(ms=round(d, 4), gbs=round(ach, 1), frac=round(ach / HBM_PEAK_GBS, 3))
    # the dominant kernel: the one with the most time per step over its launches
    per_kernel = {kn: sum(dur[n] for n in st if n in dur) for kn, (st, _) in KERNELS.items()}
    dom = max(per_kernel, key=per_kernel.get)
    launches = tuple(n for n in KERNELS[dom][0] if n in dur)
    kind = work[launches[0]][0]
    amount = sum(work[n][1] for n in launches) / len(launches)      # per launch
    avg_ms = per_kernel[dom] / len(launches)
    if kind == "mfma":
        ach = amount / (avg_ms * 1e-3) / 1e12
        peak, unit = BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        ach = amount / (avg_ms * 1e-3) / 1e9
        peak, unit = HBM_PEAK_GBS, "GB/s"
    roof = dict(bound="mfma" if kind == "mfma" else "hbm", achieved=round(ach, 1), peak=peak, unit=unit,
                frac=round(ach / peak, 4), traffic=traffic_from_profiles(dom, name),
                kernel=dom, launches=list(launches), avg_launch_ms=round(avg_ms, 4),
                work_per_launch=amount)
    config = {"workload": desc, "format": fmt, "experts": case.E, "hidden": case.H,
              "intermediate": case.I, "tokens": case.T, "topk": case.k, "routing": case.routing,
              "backward": "full: dX, d topk_w and every scale gradient" if full_bwd
              else "weight-scale gradients only"}
    res = dict(ms_per_step=round(ms, 4), value=round(value, 1), steps=steps, warmup=warmup, config=config,
               roofline=roof, stages=stages)
    return res, dl, data, P


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the w8a8, w4afp8 and fp8 layers after the headline nvfp4 layer")
    ap.add_argument("--stages", action="store_true", help="print per-stage times to stderr")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: the library runs on one GPU; the expert-parallel path over several GPUs "
              "is designed but not built, so --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from scale_only_quantization_amd import fqlib as F

    ev = HipEvents()
    res, dl, data, P = run_layer(args.workload, F, ev, args.steps, args.warmup)
    if args.stages:
        for n in F.FWD_STAGES + F.BWD_STAGES:
            print(f"[bench] {n:14s} {res['stages'].get(n, 'not run')}", file=sys.stderr)

    out = {
        "metric": "expert-layer fwd+bwd tokens/s",
        "value": res["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": res["config"],
        "roofline": res["roofline"],
        "stages": res["stages"],
    }
    out["scale_adamw"] = scale_adamw_step(ev, F, dl)
    if args.stages:
        print(f"[bench] scale_adamw {out['scale_adamw']}", file=sys.stderr)
    del dl
    torch.cuda.empty_cache()
    if args.workload == "qwen3" and not args.no_workloads:
        # the other layer workloads, each in its own format; T = 32768 inputs
        # are drawn once for w4afp8 and fp8
        out["workloads"] = {}
        shared = None
        for name in ("qwen3_w8a8", "qwen3_w4afp8", "qwen3_fp8"):
            r, wl, d, _ = run_layer(name, F, ev, min(args.steps, 10), min(args.warmup, 3),
                                    data=shared if WORKLOADS[name][0] == "qwen3l" else None)
            shared = d if WORKLOADS[name][0] == "qwen3l" else shared
            out["workloads"][name] = dict(
                ms_per_step=r["ms_per_step"], value=r["value"], unit="tokens/s", steps=r["steps"],
                tokens=r["config"]["tokens"], format=r["config"]["format"], roofline=r["roofline"],
                stages={n: s["frac"] for n, s in r["stages"].items()})
            print(f"[bench] {name}: {r['ms_per_step']:.3f} ms/step, {r['value'] / 1e6:.3f} M tokens/s",
                  file=sys.stderr, flush=True)
            del wl, d
            torch.cuda.empty_cache()
        del shared
    print("[bench] weight-only fake-quant microbench ...", file=sys.stderr, flush=True)
    out["fake_quant"] = fake_quant_stack(ev, F)
    if args.stages:
        print(f"[bench] fake_quant {out['fake_quant']}", file=sys.stderr)
    print("[bench] distillation loss on a Qwen3-sized batch of logits ...", file=sys.stderr, flush=True)
    out["distill"] = distill_logits(ev, F)
    if args.stages:
        print(f"[bench] distill {out['distill']}", file=sys.stderr)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU baseline on a bounded sample ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(data, P, WORKLOADS[args.workload][1])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
