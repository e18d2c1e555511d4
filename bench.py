#!/usr/bin/env python3
"""Benchmark of the SERQ quantized linear layer on one MI355X.

One step is one pass of the online hot path over one batch of synthetic
input: per-token activation quantization (serq_quant_act) followed by the
fused SERQ linear (serq_linear) -- the pure 4-bit GEMM, the salient-row
residual and the dequantizing epilogue. Calibration is offline and not timed.

Headline workload: the LLaMA-3-8B MLP's gate and up projections as the one
4096 -> 2 x 14336 layer they form (they share their input, so they are
calibrated together), r = 128, W4A4, bf16 activations and output, at
M = 4096 tokens: the largest layer of the five layer workloads within the
metric's 1..4096-token range. Inputs are seeded synthetic data (Gaussian
activations with 1 % outlier channels x50, Gaussian weights), calibrated by
the library, resident in HBM before the timed region. The weights and
activations are rotated through enough copies (>= 768 MiB) that every step
reads them from HBM rather than from the 256 MB last-level cache.

The K timed steps are captured once into a HIP graph (the library's kernels
are enqueued on torch's capture stream) and replayed once between two device
synchronizations, so the measurement is not bound by Python launch overhead.

Prints one JSON line. `value` is whole-job throughput in TOP/s:
2 * M * N * (K + r) integer operations per step / measured step time.
`roofline` is the dominant kernel (serq_linear) against the dense int8 MFMA
or the HBM peak, with the counter-measured bytes per launch when they were
taken on the current kernel sources. Beside the headline: "configs" (every
layer and token count of the five workloads -- tiny, q_proj, the 8B MLP in
W4A4 and W4A8, the 70B-shaped layers -- each calibrated, with its kernel
times and its own roofline entry), "mlp_activation"
(serq_silu_mul_quant_act on bf16 gate/up outputs of the 8B and 70B MLP
widths, with the unfused pair for comparison), "mlp_step" (the whole 8B MLP:
quant_act, gate/up, the fused activation, down; at 4096 tokens also on the
bf6 route, its output compared bit for bit), "bf6_route" (the same
linear on the scaled FP6 MFMA with int4 codes re-encoded as E3M2, against
serq_linear on the same codes, for prefill-sized layers), "mxfp4" (the
MXFP4 variant of the layer, serq_quant_act_mx + serq_linear_mx, against the
FP4 peak or HBM) and "cpu_baseline" (the oracle on a bounded row sample).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "serq_linear TOPS & HBM GB/s (% roofline) at M=1..4096, LLaMA-shaped K×N"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA (no sparsity)
ROTATE_BYTES = 768 << 20

WORKLOADS = {
    # name: (synth workload, layer, r, a_bits, default M, token counts, workload number)
    "tiny": ("tiny", "tiny", 8, 4, 16, (16,), 1),
    "q_proj": ("q_proj", "q_proj", 64, 4, 2048, (1, 16, 256, 2048), 2),
    "gate_up": ("mlp8b", "gate_up", 128, 4, 4096, (1, 32, 4096), 3),
    "down": ("mlp8b", "down", 128, 4, 4096, (1, 32, 4096), 3),
    "gate_up_w4a8": ("mlp8b_w4a8", "gate_up", 128, 8, 2048, (2048,), 4),
    "down_w4a8": ("mlp8b_w4a8", "down", 128, 8, 2048, (2048,), 4),
    "up70": ("l70b", "up70", 256, 4, 8192, (1, 8192), 5),
    "down70": ("l70b", "down70", 256, 4, 8192, (1, 8192), 5),
}
HEADLINE = "gate_up"


def linear_bytes(M, K, N, r, a_bits, y_bytes=2):
    return M * K * a_bits // 8 + K * N // 2 + r * N // 2 + 4 * (M + 2 * N) + M * N * y_bytes


def quant_bytes(M, K, a_bits, x_bytes=2):
    return M * K * x_bytes + 4 * K + M * K * a_bits // 8 + 4 * M


def act_bytes(M, K, a_bits):
    """serq_silu_mul_quant_act: g and u (bf16), s_hat_inv, codes, scales."""
    return M * K * 4 + 4 * K + M * K * a_bits // 8 + 4 * M


def linear_ops(M, K, N, r):
    return 2 * M * N * (K + r)


def kernel_src_sha():
    """Hash of serq_linear's kernel sources: stored HBM-traffic counters are
    used only while it matches the sources they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "w4a4_linear_layers_amd", "csrc")
    for f in ("serq_gemm.hip", "serq_internal.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


class Setup:
    """Device buffers for one layer: C rotated copies of weights and inputs."""

    def __init__(self, workload, M_max, seed=0):
        import numpy as np
        import torch

        import w4a4_linear_layers_amd as S
        from synth import workload_layer

        wl, layer, r, a_bits, _, _, _ = WORKLOADS[workload]
        t0 = time.time()
        li = workload_layer(wl, layer, M_max=M_max, seed=seed)
        self.gen_s = time.time() - t0
        self.K, self.N, self.r, self.a_bits = li.K, li.N, r, a_bits
        self.bf16 = li.dtype == "bf16"
        W = li.W_bits if self.bf16 else li.W
        if "W_up" in li.meta:          # gate and up share the input: calibrate them as one
            W = np.concatenate([W, li.meta["W_up_bits" if self.bf16 else "W_up"]], axis=1)
            self.N = W.shape[1]
        t0 = time.time()
        L = S.calibrate(W, li.act_absmax, r=r)
        self.calib_s = time.time() - t0
        self.li, self.L = li, L
        dev = torch.device("cuda")
        if self.bf16:
            x = torch.from_numpy(np.ascontiguousarray(li.X_bits[:, L.perm]).view(np.int16)).to(dev)
            x = x.view(torch.bfloat16)
        else:
            x = torch.from_numpy(np.ascontiguousarray(li.X[:, L.perm])).to(dev)
        self.x_bytes = x.element_size()
        self.ydt = torch.bfloat16 if self.bf16 else torch.float32
        per = x.numel() * self.x_bytes + L.Wq.nbytes + L.Rq.nbytes + 8 * self.N
        self.copies = max(2, math.ceil(ROTATE_BYTES / per))
        base = L.to(dev)
        self.layers, self.xs = [], []
        for _ in range(self.copies):
            self.layers.append(S.DeviceLayer(K=L.K, N=self.N, r=r, perm=base.perm, s_hat_inv=base.s_hat_inv,
                                             Wq=base.Wq.clone(), sw=base.sw.clone(), Rq=base.Rq.clone(),
                                             sr=base.sr.clone()))
            self.xs.append(x.clone())
        self.xq = torch.empty((M_max, self.K // 2 if a_bits == 4 else self.K),
                              dtype=torch.uint8 if a_bits == 4 else torch.int8, device=dev)
        self.sx = torch.empty(M_max, dtype=torch.float32, device=dev)
        self.y = torch.empty((M_max, self.N), dtype=self.ydt, device=dev)
        torch.cuda.synchronize()

    def free(self):
        import torch
        self.layers, self.xs = [], []
        self.xq = self.sx = self.y = None
        self.li = None
        torch.cuda.empty_cache()

    def step(self, i, M):
        import w4a4_linear_layers_amd as S
        c = i % self.copies
        L = self.layers[c]
        xq, sx = S.quant_act(self.xs[c][:M], L, a_bits=self.a_bits, out=(self.xq[:M], self.sx[:M]))
        S.linear(xq, sx, L, a_bits=self.a_bits, out_dtype=self.ydt, out=self.y[:M])

    def graph(self, fn, n):
        """Capture n calls fn(i) into one HIP graph (the kernels are enqueued on
        torch's capture stream), so that replays are not bound by Python
        launch overhead."""
        import torch
        fn(0)                 # one eager call: the kernels' code is loaded before the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        g.replay()            # upload + one untimed pass
        torch.cuda.synchronize()
        return g

    def time_kernels(self, M, n):
        """Average duration of each kernel alone: n back-to-back launches in
        one graph, bracketed by events on the replay stream."""
        import torch

        import w4a4_linear_layers_amd as S
        xq, sx = self.xq[:M], self.sx[:M]

        def q(i):
            c = i % self.copies
            S.quant_act(self.xs[c][:M], self.layers[c], a_bits=self.a_bits, out=(xq, sx))

        def lin(i):
            S.linear(xq, sx, self.layers[i % self.copies], a_bits=self.a_bits, out_dtype=self.ydt, out=self.y[:M])

        out = []
        for fn in (q, lin):
            g = self.graph(fn, n)
            st = torch.cuda.current_stream()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            g.replay()
            e1.record(st)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) * 1e3 / n)
        return tuple(out)


def time_mlp_act(K, Ms, n=100, a_bits=4, seed=0):
    """The MLP step before down, alone: silu(g) * u -> down's codes and
    scales, reading g and u in place from a gate/up output (bf16, M x 2K,
    ld = 2K) as serq_silu_mul_quant_act does in a LLaMA MLP with the
    intermediate width K. Each launch reads its own copy of the output (the
    copies span >= 768 MiB, beyond the last-level cache); n launches are
    captured in one graph and timed with events on the replay stream.
    For comparison, the same step unfused: torch's silu(g) * u written to
    HBM as bf16 (two elementwise kernels), then serq_quant_act on it (timing
    only; torch's silu is not the fixed recipe)."""
    import torch

    import w4a4_linear_layers_amd as S
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    sinv = torch.exp(torch.rand(K, device=dev, generator=gen) * 3 - 2)
    out = []
    for M in Ms:
        per = M * 2 * K * 2
        copies = max(2, math.ceil(ROTATE_BYTES / per))
        y = torch.randn((copies, M, 2 * K), device=dev, generator=gen).mul_(2).to(torch.bfloat16)
        xq = torch.empty((M, K // 2 if a_bits == 4 else K), dtype=torch.uint8 if a_bits == 4 else torch.int8,
                         device=dev)
        sx = torch.empty(M, dtype=torch.float32, device=dev)

        h = torch.empty((M, K), dtype=torch.bfloat16, device=dev)

        def act(i):
            yc = y[i % copies]
            S.silu_mul_quant_act(yc[:, :K], yc[:, K:], sinv, a_bits=a_bits, out=(xq, sx))

        def unfused(i):
            yc = y[i % copies]
            torch.mul(torch.nn.functional.silu(yc[:, :K]), yc[:, K:], out=h)
            S.quant_act(h, sinv, a_bits=a_bits, out=(xq, sx))

        times = []
        for fn in (act, unfused):
            fn(0)                      # one eager call before the capture
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n):
                    fn(i)
            g.replay()
            torch.cuda.synchronize()
            st = torch.cuda.current_stream()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            g.replay()
            e1.record(st)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3 / n)
            del g
        us = times[0]
        gbs = act_bytes(M, K, a_bits) / (us * 1e-6) / 1e9
        out.append(dict(K=K, M=M, us=round(us, 2), HBM_GBs=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 3),
                        unfused_us=round(times[1], 2)))
        del y, h
    return out


def time_mlp_step(Ms, n=50, seed=0):
    """The whole LLaMA-3-8B MLP on the path, per step: quant_act of x ->
    gate/up as one 4096 -> 2 x 14336 layer whose output channels carry
    down's input order (serq_permute_outputs) -> serq_silu_mul_quant_act on
    its bf16 output read in place -> down 14336 -> 4096. W4A4, r = 128,
    seeded synthetic weights, the layer pair rotated over >= 768 MiB of
    copies; n steps captured in one graph, timed with events."""
    import numpy as np
    import torch

    import w4a4_linear_layers_amd as S
    from synth import workload_layer

    M_max = max(Ms)
    gu = workload_layer("mlp8b", "gate_up", M_max=M_max, seed=seed)
    dn = workload_layer("mlp8b", "down", M_max=1, seed=seed, draw_x=False)
    Ni = gu.N
    Lg = S.calibrate(np.concatenate([gu.W_bits, gu.meta["W_up_bits"]], axis=1), gu.act_absmax, r=128)
    Ld = S.calibrate(dn.W_bits, dn.act_absmax, r=128)
    S.permute_outputs(Lg, np.concatenate([Ld.perm, Ni + Ld.perm]))
    dev = torch.device("cuda")
    per = Lg.Wq.nbytes + Lg.Rq.nbytes + Ld.Wq.nbytes + Ld.Rq.nbytes
    copies = max(2, math.ceil(ROTATE_BYTES / per))
    G0, D0 = Lg.to(dev), Ld.to(dev)

    def clone(L):
        return S.DeviceLayer(K=L.K, N=L.N, r=L.r, perm=L.perm, s_hat_inv=L.s_hat_inv, Wq=L.Wq.clone(),
                             sw=L.sw.clone(), Rq=L.Rq.clone(), sr=L.sr.clone())

    pairs = [(clone(G0), clone(D0)) for _ in range(copies)]
    bf6_pairs = []
    x = torch.from_numpy(np.ascontiguousarray(gu.X_bits[:, Lg.perm]).view(np.int16)).to(dev).view(torch.bfloat16)
    out = []
    for M in Ms:
        xq = torch.empty((M, gu.K // 2), dtype=torch.uint8, device=dev)
        sx = torch.empty(M, dtype=torch.float32, device=dev)
        y = torch.empty((M, 2 * Ni), dtype=torch.bfloat16, device=dev)
        hq = torch.empty((M, Ni // 2), dtype=torch.uint8, device=dev)
        hs = torch.empty(M, dtype=torch.float32, device=dev)
        yd = torch.empty((M, dn.N), dtype=torch.bfloat16, device=dev)
        parts = {
            "quant_act": lambda i: S.quant_act(x[:M], pairs[i % copies][0], out=(xq, sx)),
            "gate_up": lambda i: S.linear(xq, sx, pairs[i % copies][0], out=y),
            "silu_mul_quant_act": lambda i: S.silu_mul_quant_act(y[:, :Ni], y[:, Ni:], pairs[i % copies][1],
                                                                 out=(hq, hs)),
            "down": lambda i: S.linear(hq, hs, pairs[i % copies][1], out=yd),
        }

        def step(i):
            for f in parts.values():
                f(i)

        def timed(fn):
            fn(0)                      # one eager call before the capture
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n):
                    fn(i)
            g.replay()
            torch.cuda.synchronize()
            st = torch.cuda.current_stream()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            g.replay()
            e1.record(st)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / n

        step_us = timed(step)
        e = dict(M=M, step_us=round(step_us, 2))
        for k, f in parts.items():
            step(0)                    # the buffers every part reads hold one real step's data
            e[k + "_us"] = round(timed(f), 2)
        e["kernels"] = [S.kernel_name(M, gu.K, 2 * Ni, 128), S.kernel_name(M, Ni, dn.N, 128)]
        if M >= 4096:
            # the same step on the bf6 route: both layers' codes re-encoded
            # (activations on the device), the output compared bit for bit
            if not bf6_pairs:
                Bg, Bd = S.prepack_bf6(Lg).to(dev), S.prepack_bf6(Ld).to(dev)
                cl6 = lambda B: S.Bf6Layer(K=B.K, N=B.N, r=B.r, W6=B.W6.clone(), sw=B.sw, R6=B.R6, sr=B.sr)  # noqa: E731
                bf6_pairs.extend((cl6(Bg), cl6(Bd)) for _ in range(copies))
            x6 = torch.empty(S.bf6_bytes(M, gu.K), dtype=torch.uint8, device=dev)
            h6 = torch.empty(S.bf6_bytes(M, Ni), dtype=torch.uint8, device=dev)
            yd6 = torch.empty_like(yd)
            parts6 = [
                lambda i: S.quant_act(x[:M], pairs[i % copies][0], out=(xq, sx)),
                lambda i: S.act_bf6(xq, gu.K, out=x6),
                lambda i: S.linear_bf6(x6, sx, bf6_pairs[i % copies][0], out=y),
                lambda i: S.silu_mul_quant_act(y[:, :Ni], y[:, Ni:], pairs[i % copies][1], out=(hq, hs)),
                lambda i: S.act_bf6(hq, Ni, out=h6),
                lambda i: S.linear_bf6(h6, hs, bf6_pairs[i % copies][1], out=yd6),
            ]

            def step6(i):
                for f in parts6:
                    f(i)
            step(0)
            torch.cuda.synchronize()
            ref = yd.clone()
            step6(0)
            torch.cuda.synchronize()
            e["bf6_route_step_us"] = round(timed(step6), 2)
            e["bf6_route_identical"] = bool(torch.equal(yd6.view(torch.int16), ref.view(torch.int16)))
            e["bf6_route_kernels"] = [S.bf6_kernel_name(M, 2 * Ni, 128), S.bf6_kernel_name(M, dn.N, 128)]
        out.append(e)
    return out


def cpu_baseline(setup, M, rows=None, budget_s=20.0):
    """The CPU oracle as it stands, on a bounded row sample of the workload:
    activation quantization + int64 matmuls + fp64 epilogue. Rows are
    independent, so throughput scales exactly with the row count."""
    import numpy as np

    from oracle import serq_oracle as O
    li, L = setup.li, setup.L
    K, N, r = setup.K, setup.N, setup.r
    Wc = O.unpack_int4(L.Wq).T.copy()
    Rc = O.unpack_int4(np.ascontiguousarray(L.Rq[:, : r // 2])).T.copy() if r else np.zeros((0, N), np.int8)
    layer = dict(r=r, Wq_codes=Wc, Rq_codes=Rc, sw=L.sw, sr=L.sr)
    n = 8 if rows is None else rows
    X = li.X[:, L.perm]
    while True:
        t0 = time.perf_counter()
        q = O.quant_act(X[:n], L.s_hat_inv, setup.a_bits)
        O.linear(q, layer, out="bf16" if setup.bf16 else "f32")
        dt = time.perf_counter() - t0
        if rows is not None or dt > budget_s / 4 or n >= M:
            break
        n = min(M, max(n + 1, int(n * min(8.0, (budget_s / 2) / max(dt, 1e-3)))))
    ops = linear_ops(n, K, N, r)
    return dict(value=ops / dt / 1e12, unit="TOP/s", cores=1, kind="oracle",
                sample=f"{n} of {M} rows of the same workload (quant_act + int64 matmuls + fp64 epilogue), "
                       f"{dt:.1f} s; numpy integer matmul runs on one thread",
                seconds=round(dt, 2), rows=n, host_cpu=cpu_model(),
                affinity_cpus=len(os.sched_getaffinity(0)))


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


WORKLOAD_TITLES = {
    "tiny": "tiny layer",
    "q_proj": "LLaMA-2-7B q_proj",
    "gate_up": "LLaMA-3-8B MLP gate and up as one layer",
    "down": "LLaMA-3-8B MLP down",
    "gate_up_w4a8": "LLaMA-3-8B MLP gate and up as one layer, W4A8",
    "down_w4a8": "LLaMA-3-8B MLP down, W4A8",
    "up70": "LLaMA-2-70B-shaped up layer",
    "down70": "LLaMA-2-70B-shaped down layer",
}


def config_lines(setup, name, reps=50):
    """One entry per token count of a layer workload: kernel times (graph
    replays, events), throughput and the serq_linear roofline entry."""
    import w4a4_linear_layers_amd as S
    _, _, r, a_bits, _, token_counts, number = WORKLOADS[name]
    K, N = setup.K, setup.N
    y_bytes = 2 if setup.bf16 else 4
    out = []
    for m in token_counts:
        qu, lu = setup.time_kernels(m, reps)
        e = roofline_entry(m, K, N, r, a_bits, lu, None, y_bytes)
        tops = linear_ops(m, K, N, r) / (lu * 1e-6) / 1e12
        gbs = linear_bytes(m, K, N, r, a_bits, y_bytes) / (lu * 1e-6) / 1e9
        out.append(dict(workload=number, layer=name, title=WORKLOAD_TITLES[name], M=m, K=K, N=N, r=r,
                        a_bits=a_bits, kernel=S.kernel_name(m, K, N, r, a_bits), linear_us=round(lu, 2),
                        quant_act_us=round(qu, 2), step_us=round(qu + lu, 2), TOPS=round(tops, 2),
                        HBM_GBs=round(gbs, 1),
                        quant_act_GBs=round(quant_bytes(m, K, a_bits, setup.x_bytes) / (qu * 1e-6) / 1e9, 1),
                        roofline=dict(bound=e["bound"], achieved=e["achieved"], peak=e["peak"], unit=e["unit"],
                                      frac=e["frac"])))
        print(f"# {name} M={m}: linear {lu:.2f} us ({out[-1]['kernel']}) {tops:.1f} TOP/s {gbs:.0f} GB/s "
              f"({e['bound']} frac {e['frac']:.3f}); quant_act {qu:.2f} us", file=sys.stderr, flush=True)
    return out


def roofline_entry(M, K, N, r, a_bits, us, traffic, y_bytes=2):
    ops = linear_ops(M, K, N, r)
    byts = linear_bytes(M, K, N, r, a_bits, y_bytes)
    if ops / byts > INT8_PEAK_TOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        ach = ops / (us * 1e-6) / 1e12
        return dict(bound="mfma", achieved=round(ach, 1), peak=INT8_PEAK_TOPS, unit="TOP/s",
                    frac=round(ach / INT8_PEAK_TOPS, 4), traffic=traffic, kernel="serq_linear",
                    algorithmic_ops=ops, algorithmic_bytes=byts)
    ach = byts / (us * 1e-6) / 1e9
    return dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(ach / HBM_PEAK_GBS, 4), traffic=traffic, kernel="serq_linear",
                algorithmic_ops=ops, algorithmic_bytes=byts)


def load_traffic(workload, M):
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_M{M}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_src_sha") != kernel_src_sha():
        return None
    return t.get("bytes_per_launch")


def copy_probe(mib, reps=10):
    """Device-to-device copies of a known size: a reference for the HBM
    byte counters (each copy reads and writes mib MiB)."""
    import torch
    torch.cuda.set_device(0)
    a = torch.ones(mib << 19, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": mib << 20, "copies": reps}))
    return 0


FP6_PEAK_TOPS = 10100.0        # MI355X dense FP6/FP4 MFMA (no sparsity)
BF6_SHAPES = (                 # (M, K, N, r): q_proj, 8B gate/up and down, 70B up and down
    (2048, 4096, 4096, 64), (4096, 4096, 28672, 128), (4096, 14336, 4096, 128),
    (8192, 8192, 28672, 256), (8192, 28672, 8192, 256))


def time_bf6_route(shapes=BF6_SHAPES, reps=20):
    """The bf6 route (serq_act_bf6 + serq_linear_bf6) against serq_linear on
    the same random W4A4 codes: per-kernel times from graph replays, weights
    rotated over copies beyond the last-level cache, and whether the outputs
    are bit-identical."""
    import numpy as np
    import torch
    import w4a4_linear_layers_amd as S
    out = []
    for (M, K, N, r) in shapes:
        rng = np.random.default_rng(M + K + N + r)
        Wp = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
        Rp = np.zeros((N, S.rq_row_bytes(r)), np.uint8)
        Rp[:, : r // 2] = rng.integers(0, 256, (N, r // 2), dtype=np.uint8)
        W6 = torch.from_numpy(S._prepack(Wp, N, K, K // 2)).cuda()
        R6 = torch.from_numpy(S._prepack(Rp, N, r, S.rq_row_bytes(r))).cuda()
        copies = int(min(8, max(2, ROTATE_BYTES // (W6.numel() + M * K))))
        sw = torch.rand(N, device="cuda") * 0.01
        sr = torch.rand(N, device="cuda") * 0.001
        sx = torch.rand(M, device="cuda")
        L6 = [S.Bf6Layer(K=K, N=N, r=r, W6=W6.clone() if c else W6, sw=sw, R6=R6, sr=sr) for c in range(copies)]
        Wd, Rd = torch.from_numpy(Wp).cuda(), torch.from_numpy(Rp).cuda()
        L4 = [S.DeviceLayer(K=K, N=N, r=r, perm=None, s_hat_inv=None, Wq=Wd.clone() if c else Wd, sw=sw, Rq=Rd,
                            sr=sr) for c in range(copies)]
        Xs = [torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, device="cuda") for _ in range(copies)]
        X6s = [S.act_bf6(x, K) for x in Xs]
        y6 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        y4 = torch.empty_like(y6)
        S.linear_bf6(X6s[0], sx, L6[0], out=y6)
        S.linear(Xs[0], sx, L4[0], a_bits=4, out=y4)
        torch.cuda.synchronize()
        same = bool(torch.equal(y6.view(torch.int16), y4.view(torch.int16)))

        def timed(fn):
            g = _graph_of(fn, reps)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / reps

        t6 = timed(lambda i: S.linear_bf6(X6s[i % copies], sx, L6[i % copies], out=y6))
        t4 = timed(lambda i: S.linear(Xs[i % copies], sx, L4[i % copies], a_bits=4, out=y4))
        x6o = torch.empty_like(X6s[0])
        ta = timed(lambda i: S.act_bf6(Xs[i % copies], K, out=x6o))
        ops = linear_ops(M, K, N, r)
        out.append(dict(M=M, K=K, N=N, r=r, kernel=S.bf6_kernel_name(M, N, r), bit_identical=same,
                        linear_bf6_us=round(t6, 2), act_bf6_us=round(ta, 2), serq_linear_us=round(t4, 2),
                        TOPS=round(ops / t6 / 1e6, 1), frac_fp6_peak=round(ops / t6 / 1e6 / FP6_PEAK_TOPS, 4),
                        speedup_vs_int8_path=round(t4 / t6, 3)))
        del L6, L4, Xs, X6s, W6, R6, Wd, Rd
        torch.cuda.empty_cache()
    return out


FP4_PEAK_TOPS = 10100.0        # MI355X dense FP4 MFMA (no sparsity)
MX_SHAPES = (                  # (M, K, N, r): decode and prefill on the five layer shapes
    (1, 4096, 4096, 64), (16, 4096, 4096, 64), (2048, 4096, 4096, 64), (4096, 4096, 28672, 128),
    (4096, 14336, 4096, 128), (8192, 8192, 28672, 256), (8192, 28672, 8192, 256))


def mx_bytes(M, K, N, r, y_bytes=2):
    """Algorithmic bytes of serq_linear_mx: FP4 codes (1/2 byte) and E8M0
    bytes (1/32 byte) per element of X, W and R, plus Y."""
    return (M * K + K * N + r * N) * 17 // 32 + M * N * y_bytes


def time_mx_route(shapes=MX_SHAPES, reps=20):
    """The MXFP4 layer: serq_quant_act_mx and serq_linear_mx on random FP4
    codes and exponents (weights rotated over copies beyond the last-level
    cache), per-kernel times from graph replays, TOPS against the FP4 peak or
    GB/s against HBM by the layer's arithmetic intensity."""
    import numpy as np
    import torch
    import w4a4_linear_layers_amd as S
    out = []
    for (M, K, N, r) in shapes:
        rng = np.random.default_rng(M + K + N + r)
        Wq = torch.from_numpy(rng.integers(0, 256, (N, K // 2), dtype=np.uint8)).cuda()
        Wsc = torch.from_numpy(rng.integers(120, 130, (N, K // 32), dtype=np.uint8)).cuda()
        Rq = torch.from_numpy(rng.integers(0, 256, (N, r // 2), dtype=np.uint8)).cuda()
        Rsc = torch.from_numpy(rng.integers(115, 125, (N, r // 32), dtype=np.uint8)).cuda()
        copies = int(min(8, max(2, ROTATE_BYTES // (Wq.numel() + M * K))))
        Ls = [S.MxLayer(K=K, N=N, r=r, perm=None, s_hat_inv=None, Wq=Wq.clone() if c else Wq, Wsc=Wsc, Rq=Rq,
                        Rsc=Rsc) for c in range(copies)]
        X = [torch.randn((M, K), device="cuda").to(torch.bfloat16) for _ in range(copies)]
        sinv = torch.ones(K, device="cuda")
        xq = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
        xsc = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

        def timed(fn):
            g = _graph_of(fn, reps)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / reps

        tq = timed(lambda i: S.quant_act_mx(X[i % copies], sinv, out=(xq, xsc)))
        tl = timed(lambda i: S.linear_mx(xq, xsc, Ls[i % copies], out=y))
        ops = linear_ops(M, K, N, r)
        byts = mx_bytes(M, K, N, r)
        if ops / byts > FP4_PEAK_TOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
            roof = dict(bound="mfma", achieved=round(ops / tl / 1e6, 1), peak=FP4_PEAK_TOPS, unit="TOP/s",
                        frac=round(ops / tl / 1e6 / FP4_PEAK_TOPS, 4))
        else:
            roof = dict(bound="hbm", achieved=round(byts / tl / 1e3, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                        frac=round(byts / tl / 1e3 / HBM_PEAK_GBS, 4))
        out.append(dict(M=M, K=K, N=N, r=r, linear_mx_us=round(tl, 2), quant_act_mx_us=round(tq, 2),
                        TOPS=round(ops / tl / 1e6, 1), roofline=roof))
        del Ls, X, Wq, Rq
        torch.cuda.empty_cache()
    return out


def _graph_of(fn, reps):
    import torch
    for i in range(2):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    return g


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--M", type=int, default=None, help="tokens per step (default: the workload's)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the other workloads and token counts, the MLP and the bf6 lines")
    ap.add_argument("--configs", default=None, metavar="NAME[,NAME...]",
                    help="workloads for the per-config lines besides the headline's (default: all)")
    ap.add_argument("--no-mlp-act", action="store_true", help="skip the MLP activation timing")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-bf6", action="store_true", help="skip the bf6 route timings")
    ap.add_argument("--no-mx", action="store_true", help="skip the MXFP4 layer timings")
    ap.add_argument("--mx", default=None, metavar="M:K:N:r[,...]",
                    help="only time the MXFP4 layer on the given shapes (one JSON line each), then exit")
    ap.add_argument("--bf6", default=None, metavar="M:K:N:r[,...]",
                    help="only time the bf6 route on the given shapes (one JSON line each), then exit")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run device-to-device copies of MIB MiB (a reference kernel of known "
                         "traffic for scaling HBM byte counters), then exit")
    ap.add_argument("--mlp-act", default=None, metavar="K:M[,M...]",
                    help="only time serq_silu_mul_quant_act at intermediate width K for the given token "
                         "counts (one JSON line each), then exit")
    args = ap.parse_args(argv)
    if args.copy_probe:
        return copy_probe(args.copy_probe)
    if args.mlp_act:
        k_s, m_s = args.mlp_act.split(":")
        for e in time_mlp_act(int(k_s), [int(m) for m in m_s.split(",")], n=max(args.steps, 20)):
            print(json.dumps(dict(kernel="serq_silu_mul_quant_act", **e)), flush=True)
        return 0
    if args.mx:
        shapes = [tuple(int(v) for v in sh.split(":")) for sh in args.mx.split(",")]
        for e in time_mx_route(shapes, reps=max(args.steps, 5) if args.steps != 200 else 20):
            print(json.dumps(dict(route="mxfp4", **e)), flush=True)
        return 0
    if args.bf6:
        shapes = [tuple(int(v) for v in sh.split(":")) for sh in args.bf6.split(",")]
        for e in time_bf6_route(shapes, reps=max(args.steps, 5) if args.steps != 200 else 20):
            print(json.dumps(dict(route="bf6", **e)), flush=True)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the library has no "
              f"multi-GPU path)", file=sys.stderr)
        return 2

    import torch
    import w4a4_linear_layers_amd as S

    torch.cuda.set_device(0)
    wl, layer, r, a_bits, M_def, token_counts, _ = WORKLOADS[args.workload]
    M = args.M or M_def
    setup = Setup(args.workload, max([M] + list(token_counts)))
    K, N = setup.K, setup.N
    print(f"# setup: {args.workload} K={K} N={N} r={r} a_bits={a_bits} copies={setup.copies} "
          f"generate {setup.gen_s:.1f}s calibrate {setup.calib_s:.1f}s", file=sys.stderr, flush=True)

    for i in range(args.warmup):
        setup.step(i, M)
    torch.cuda.synchronize()
    # the K timed steps are captured once as a HIP graph and replayed once
    g = setup.graph(lambda i: setup.step(i, M), args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    del g
    ms_per_step = dt * 1e3 / args.steps
    ops = linear_ops(M, K, N, r)
    value = ops * args.steps / dt / 1e12
    y_bytes = 2 if setup.bf16 else 4

    q_us, l_us = setup.time_kernels(M, max(args.steps, 50))
    traffic = load_traffic(args.workload, M)
    roof = roofline_entry(M, K, N, r, a_bits, l_us, traffic, y_bytes)
    print(f"# step {ms_per_step * 1e3:.2f} us; quant_act {q_us:.2f} us, serq_linear {l_us:.2f} us "
          f"({S.kernel_name(M, K, N, r, a_bits)})", file=sys.stderr, flush=True)

    mx = []
    if not args.no_sweep and not args.no_mx:
        mx = time_mx_route()
        for e in mx:
            print(f"# mxfp4 M={e['M']} K={e['K']} N={e['N']}: linear_mx {e['linear_mx_us']:.1f} us ({e['TOPS']:.0f} "
                  f"TOP/s, {e['roofline']['bound']} frac {e['roofline']['frac']:.3f}); quant_act_mx "
                  f"{e['quant_act_mx_us']:.1f} us", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(setup, M)
        print(f"# cpu oracle: {cpu['value']:.4f} TOP/s on {cpu['rows']} rows", file=sys.stderr, flush=True)

    configs = []
    if not args.no_sweep:
        names = [n for n in WORKLOADS if n != args.workload] if args.configs is None else args.configs.split(",")
        configs.extend(config_lines(setup, args.workload))
        setup.free()
        for name in names:
            st = Setup(name, max(WORKLOADS[name][5]))
            print(f"# setup: {name} generate {st.gen_s:.1f}s calibrate {st.calib_s:.1f}s copies {st.copies}",
                  file=sys.stderr, flush=True)
            configs.extend(config_lines(st, name))
            st.free()
            del st
    else:
        setup.free()

    mlp_act = []
    if not args.no_sweep and not args.no_mlp_act:
        for k_int in (14336, 28672):
            for e in time_mlp_act(k_int, (1, 16, 256, 4096)):
                mlp_act.append(e)
                print(f"# silu_mul_quant_act K={e['K']} M={e['M']}: {e['us']:.2f} us {e['HBM_GBs']:.0f} GB/s "
                      f"(unfused {e['unfused_us']:.2f} us)", file=sys.stderr, flush=True)

    mlp_step = []
    if not args.no_sweep and not args.no_mlp_act:
        mlp_step = time_mlp_step((1, 16, 256, 4096))
        for e in mlp_step:
            print(f"# mlp step M={e['M']}: {e['step_us']:.1f} us (quant_act {e['quant_act_us']:.1f}, gate/up "
                  f"{e['gate_up_us']:.1f}, silu_mul_quant_act {e['silu_mul_quant_act_us']:.1f}, down "
                  f"{e['down_us']:.1f})" + (f"; bf6 route {e['bf6_route_step_us']:.1f} us, identical "
                                            f"{e['bf6_route_identical']}" if "bf6_route_step_us" in e else ""),
                  file=sys.stderr, flush=True)

    bf6 = []
    if not args.no_sweep and not args.no_bf6:
        bf6 = time_bf6_route()
        for e in bf6:
            print(f"# bf6 route M={e['M']} K={e['K']} N={e['N']}: linear_bf6 {e['linear_bf6_us']:.1f} us "
                  f"({e['kernel']}, {e['TOPS']:.0f} TOP/s) vs serq_linear {e['serq_linear_us']:.1f} us; "
                  f"act_bf6 {e['act_bf6_us']:.1f} us; bit-identical {e['bit_identical']}",
                  file=sys.stderr, flush=True)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int4" if a_bits == 4 else "int8xint4",
        "data": "synthetic",
        "config": {"workload": f"{WORKLOAD_TITLES[args.workload]}: SERQ linear K={K} N={N} r={r} "
                               f"{'W4A4' if a_bits == 4 else 'W4A8'}, "
                               f"{'bf16' if setup.bf16 else 'fp32'} in/out, M={M} tokens per step, calibrated",
                   "M": M, "K": K, "N": N, "r": r, "a_bits": a_bits,
                   "kernel": S.kernel_name(M, K, N, r, a_bits), "rotated_copies": setup.copies},
        "kernels_us": {"serq_quant_act": round(q_us, 3), "serq_linear": round(l_us, 3)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "configs": configs,
        "mlp_activation": mlp_act,
        "mlp_step": mlp_step,
        "bf6_route": bf6,
        "mxfp4": mx,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
