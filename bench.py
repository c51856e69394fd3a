"""Benchmark: one training step of the blockwise-FP8 linear stack of a Qwen3-1.7B-shaped model.

A step = 28 layers x 4 linear GEMM groups (qkv 2048->4096, o 2048->2048, gate_up 2048->12288,
down 6144->2048) at M = 8192 tokens (2 sequences of 4096):
  forward  (layer 0..27): quant_w_128x128_group(the layer's four W), then per linear
                         (qkv..down): quant_dual_1x128(X), fp8_gemm_fwd
  backward (layer 27..0, down..qkv): quant_dual_1x128(dY), fp8_gemm_dgrad, fp8_gemm_wgrad
quant_dual_1x128 writes both 1x128 orientations from one read: X's transposed copy is made in
the forward pass and kept for the weight gradient. With --unfused the step instead runs
quant_act_1x128(X) forward and quant_act_1x128(dY), quant_transpose(dY), quant_transpose(X)
backward (same results, 2 more bytes read per element of X and dY). With --pow2 every quantiser
and GEMM is the library's power-of-two-scale (E8M0) variant.
Every layer has its own seeded bf16 X, W, dY and fp32 dW buffers resident in HBM (~26 GB), so
the 256 MB last-level cache cannot serve one layer's data to the next.

Prints one JSON line: whole-step tokens/s, per-kernel times from HIP events recorded around
every launch on the launch stream inside the timed region, the dominant kernel's roofline
fraction, and the CPU oracle timed on a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("blockwise-FP8 GEMM TFLOP/s (% of FP8 peak); quant GB/s; linear-stack tokens/s")
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
M_TOKENS = 8192

# algorithmic bytes per element of the quantisers: 2 B bf16 read + 1 B E4M3 write (per copy) +
# scale share
B_ACT = 2 + 1 + 4 / 128
B_W = 2 + 1 + 4 / (128 * 128)
B_DUAL = 2 + 2 * (1 + 4 / 128)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--layers", type=int, default=28, help=argparse.SUPPRESS)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true",
                   help="time eager launches instead of one captured HIP graph per step")
    p.add_argument("--unfused", action="store_true",
                   help="separate quantiser launches per orientation instead of quant_dual_1x128")
    p.add_argument("--pow2", action="store_true",
                   help="power-of-two (E8M0) scales applied by the matrix cores: the library's "
                        "_pow2 variant of every quantiser and GEMM")
    order = p.add_mutually_exclusive_group()
    order.add_argument("--overlap", action="store_true",
                       help="time the step in the two-stream order (weight quantisation and wgrad "
                            "on a side stream; measured 0-0.3 % faster than the serial order on MI355X)")
    order.add_argument("--no-overlap", action="store_true",
                       help="time the step in the serial order on one stream (the default)")
    p.add_argument("--no-optim", action="store_true",
                   help="skip the optimizer-step measurement")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    p.add_argument("--config", choices=("c1", "c2", "c3", "all"), default=None,
                   help="measure a single-layer configuration instead of the 28-layer step "
                        "(c1: layer forward at M=4096; c2: layer fwd+bwd at M=16384; c3: down "
                        "projection outlier stress; all: c1, c2, c3), one JSON line each")
    p.add_argument("--no-copy-ceiling", action="store_true",
                   help="skip the same-run copy ceiling and per-shape quantiser/copy rates")
    p.add_argument("--ceiling", action="store_true",
                   help="only run the matrix-core microbenchmark (libpuro_probe.so): the MFMA "
                        "instruction's rate on register operands, without and with the GEMMs' "
                        "promotion, on zero, random and quantised-data codes, and the shader clock")
    return p.parse_args()


class Op:
    """One launch of the step: its class (kind[shape]), the kernel function it runs,
    algorithmic flops / bytes, the call bound to the main stream (serial order) and the call
    bound to its stream in the overlapped order, with the events it waits for before launching
    and records after."""

    def __init__(self, cls, flops, nbytes, serial, par=None, side=False, waits=(), record=None,
                 fn=None, traffic=None):
        self.cls, self.flops, self.bytes = cls, flops, nbytes
        self.fn = fn or cls.split("[")[0]  # the kernel function the launch runs
        # the HBM bytes the launch must move at least (operands, scales and output once)
        self.traffic = nbytes if traffic is None else traffic
        self.serial, self.par = serial, par or serial
        self.side, self.waits, self.record = side, tuple(waits), record


class Stack:
    """Device buffers and pre-marshalled launches of the whole step.

    Two launch orders over the same kernels and buffers:
      serial   every launch on one stream, in the step's order (the kernel timing pass);
      overlap  the critical chain on the main stream and, on a side stream, the work nothing
               later in the step waits for: each layer's weight quantisation (needed only by
               that layer's forward GEMMs) runs ahead, and each weight-gradient GEMM (whose dW
               feeds only the optimizer) runs beside the next linear's gradient quantisation
               and data-gradient GEMM. Events carry every real dependency: a forward GEMM
               waits for its layer's weights; a wgrad waits for the quantisation of its dY;
               a gradient quantisation that reuses a transposed-copy buffer waits for the
               wgrad that last read it; the step ends when both streams are done.
    """

    def __init__(self, layers: int, M: int, fused: bool = True, pow2: bool = False):
        import torch
        from blockwise_fp8_gemm_x128_amd import binding as B
        from blockwise_fp8_gemm_x128_amd import synth

        dev = torch.device("cuda:0")
        self.stream = torch.cuda.current_stream(dev)  # the main stream
        self.side = torch.cuda.Stream(dev)
        shared = {}
        self.shared = shared  # intermediates reused across layers: keep them allocated

        sfx = "_pow2" if pow2 else ""

        def prep(name, *args, side=False):
            serial = B.prepare(name + sfx, *args, stream=self.stream)
            par = B.prepare(name + sfx, *args, stream=self.side) if side else serial
            return serial, par

        def buf(key, shape, dtype):
            if key not in shared:
                shared[key] = torch.empty(shape, dtype=dtype, device=dev)
            return shared[key]

        self.persist = []
        self.weights = []
        self.linears = []  # per (layer, linear): its name, sizes and per-layer tensors
        wq_ops, fwd, bwd = [], [], []
        for layer in range(layers):
            group_w, group_q, group_s = [], [], []
            lf = []
            for li, (name, K, N) in enumerate(synth.LINEARS):
                s = lambda kind: synth.stack_seed(layer, li, kind)  # noqa: E731
                x = synth.randn_bf16((M, K), synth.X_STD, s(synth.KIND_X), dev)
                w = synth.randn_bf16((N, K), synth.W_STD, s(synth.KIND_W), dev)
                dy = synth.randn_bf16((M, N), synth.DY_STD, s(synth.KIND_DY), dev)
                wq = torch.empty((N, K), dtype=torch.uint8, device=dev)
                sw = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
                dw = torch.empty((N, K), dtype=torch.float32, device=dev)
                xq = buf(("xq", M, K), (M, K), torch.uint8)
                sx = buf(("sx", M, K), (K // 128, M), torch.float32)
                y = buf(("y", M, N), (M, N), torch.bfloat16)
                dyq = buf(("dyq", M, N), (M, N), torch.uint8)
                sdy = buf(("sdy", M, N), (N // 128, M), torch.float32)
                dx = buf(("dx", M, K), (M, K), torch.bfloat16)
                # one transposed-copy buffer per linear slot (shared across layers)
                dytq = buf(("dytq", li), (N, M), torch.uint8)
                sdyt = buf(("sdyt", li), (M // 128, N), torch.float32)
                self.persist += [x, w, dy, wq, sw, dw]
                self.weights.append((w, dw))  # bf16 copy of the master, and its gradient
                rec = {"layer": layer, "li": li, "name": name, "K": K, "N": N, "x": x, "w": w,
                       "dy": dy, "wq": wq, "sw": sw, "dw": dw}
                self.linears.append(rec)
                f = 2.0 * M * N * K
                # least HBM bytes of each GEMM: e4m3 operands and fp32 scales read once, the
                # output (bf16 Y / dX, fp32 dW) written once
                t_fwd = M * K + 4 * M * K / 128 + N * K + 4 * N * K / 16384 + 2 * M * N
                t_dgrad = M * N + 4 * M * N / 128 + N * K + 4 * N * K / 16384 + 2 * M * K
                t_wgrad = N * M + 4 * N * M / 128 + K * M + 4 * K * M / 128 + 4 * N * K
                group_w.append(w)
                group_q.append(wq)
                group_s.append(sw)
                g_fwd = Op(f"gemm_fwd{sfx}[{name}]", f, 0.0,
                           *prep("puro_fp8_gemm_fwd", xq, sx, wq, sw, y, M, N, K),
                           waits=(f"wq{layer}",) if li == 0 else (),
                           fn=B.puro_gemm_kernel_name("fwd", M, N, K, pow2), traffic=t_fwd)
                g_dgrad = Op(f"gemm_dgrad{sfx}[{name}]", f, 0.0,
                             *prep("puro_fp8_gemm_dgrad", dyq, sdy, wq, sw, dx, M, N, K),
                             fn=B.puro_gemm_kernel_name("dgrad", M, N, K, pow2),
                             traffic=t_dgrad)
                fn_wgrad = B.puro_gemm_kernel_name("wgrad", M, N, K, pow2)
                qsfx = "[pow2]" if pow2 else ""
                fn_dual = "quant_dual_1x128_kernel" + qsfx
                # the gradient quantisation that overwrites slot li's transposed copy waits for
                # the wgrad of the layer above (issued earlier) to have read it
                reuse = (f"wg{li}",) if layer < layers - 1 else ()
                if fused:
                    # X's transposed copy lives from this layer's forward to its backward
                    xtq = torch.empty((K, M), dtype=torch.uint8, device=dev)
                    sxt = torch.empty((M // 128, K), dtype=torch.float32, device=dev)
                    self.persist += [xtq, sxt]
                    rec.update(xtq=xtq, sxt=sxt)
                    lf += [Op(f"quant_dual_1x128{sfx}[{M}x{K}]", 0.0, M * K * B_DUAL,
                              *prep("puro_quant_dual_1x128", x, M, K, xq, sx, xtq, sxt),
                              fn=fn_dual),
                           g_fwd]
                    bwd.append([
                        Op(f"quant_dual_1x128{sfx}[{M}x{N}]", 0.0, M * N * B_DUAL,
                           *prep("puro_quant_dual_1x128", dy, M, N, dyq, sdy, dytq, sdyt),
                           waits=reuse, record=f"dual{li}", fn=fn_dual),
                        g_dgrad,
                        Op(f"gemm_wgrad{sfx}[{name}]", f, 0.0,
                           *prep("puro_fp8_gemm_wgrad", dytq, sdyt, xtq, sxt, dw, M, N, K, 0,
                                 side=True),
                           side=True, waits=(f"dual{li}",), record=f"wg{li}", fn=fn_wgrad,
                           traffic=t_wgrad),
                    ])
                else:
                    xtq = buf(("xtq", M, K), (K, M), torch.uint8)
                    sxt = buf(("sxt", M, K), (M // 128, K), torch.float32)
                    fn_act = "quant_act_1x128_kernel" + qsfx
                    fn_tr = "quant_dual_1x128_kernel(columns only)" + qsfx
                    lf += [Op(f"quant_act_1x128{sfx}[{M}x{K}]", 0.0, M * K * B_ACT,
                              *prep("puro_quant_act_1x128", x, M, K, xq, sx), fn=fn_act),
                           g_fwd]
                    bwd.append([
                        Op(f"quant_act_1x128{sfx}[{M}x{N}]", 0.0, M * N * B_ACT,
                           *prep("puro_quant_act_1x128", dy, M, N, dyq, sdy), fn=fn_act),
                        g_dgrad,
                        # the transposed copies and wgrad only feed dW: all on the side stream,
                        # whose own order protects the buffers it reuses
                        Op(f"quant_transpose{sfx}[{M}x{N}]", 0.0, M * N * B_ACT,
                           *prep("puro_quant_transpose", dy, M, N, dytq, sdyt, side=True),
                           side=True, fn=fn_tr),
                        Op(f"quant_transpose{sfx}[{M}x{K}]", 0.0, M * K * B_ACT,
                           *prep("puro_quant_transpose", x, M, K, xtq, sxt, side=True),
                           side=True, fn=fn_tr),
                        Op(f"gemm_wgrad{sfx}[{name}]", f, 0.0,
                           *prep("puro_fp8_gemm_wgrad", dytq, sdyt, xtq, sxt, dw, M, N, K, 0,
                                 side=True),
                           side=True, fn=fn_wgrad, traffic=t_wgrad),
                    ])
            # all four weights of the layer in one grouped launch
            items = B.w_group_items(group_w, group_q, group_s)
            wq_op = Op("quant_w_128x128" + sfx, 0.0,
                       sum(w.shape[0] * w.shape[1] for w in group_w) * B_W,
                       *prep("puro_quant_w_128x128_group", items, len(group_w), side=True),
                       side=True, record=f"wq{layer}",
                       fn="quant_w_128x128_group_kernel" + ("[pow2]" if pow2 else ""))
            wq_ops.append(wq_op)
            fwd += [wq_op] + lf
        bwd_flat = [op for grp in reversed(bwd) for op in grp]
        # serial order: the step as one stream runs it
        self.launches = fwd + bwd_flat
        # overlapped issue order: the side stream's weight quantisations first (they record
        # the events the forward GEMMs wait for), then the forward and backward in step order
        self.par_order = wq_ops + [op for op in fwd if op not in wq_ops] + bwd_flat
        self.events = {}
        for op in self.launches:
            for e in op.waits + ((op.record,) if op.record else ()):
                self.events.setdefault(e, torch.cuda.Event())
        self.fork, self.join = torch.cuda.Event(), torch.cuda.Event()
        self.graph = None
        self.flops = sum(op.flops for op in self.launches)
        self.bytes = sum(op.bytes for op in self.launches)

    def run(self, events=None, overlap=False):
        """One step. `events` (serial only): a (start, end) event pair per launch, recorded
        around it on the main stream."""
        if not overlap:
            if events is None:
                for op in self.launches:
                    op.serial()
            else:
                for op, (e0, e1) in zip(self.launches, events):
                    e0.record(self.stream)
                    op.serial()
                    e1.record(self.stream)
            return
        assert events is None
        self.fork.record(self.stream)
        self.side.wait_event(self.fork)
        for op in self.par_order:
            st = self.side if op.side else self.stream
            for e in op.waits:
                st.wait_event(self.events[e])
            op.par()
            if op.record:
                self.events[op.record].record(st)
        self.join.record(self.side)
        self.stream.wait_event(self.join)

    def capture(self, overlap=False):
        """Capture one whole step (all its launches) as a HIP graph on the main stream (the
        side stream joins the capture through the fork event)."""
        import torch
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph, stream=self.stream):
            self.run(overlap=overlap)

    def replay(self):
        self.graph.replay()


def cpu_baseline(M: int, layers: int, rows_fwd: int = 512, rows_wgrad: int = 512,
                 pow2: bool = False):
    """The oracle on the host cores, on a bounded sample of one step: every quantiser of one
    layer at full size, and each GEMM of that layer on a seeded sample of output rows (all
    columns), extrapolated linearly to all rows and then to all layers."""
    import numpy as np

    import oracle
    from blockwise_fp8_gemm_x128_amd import synth

    def u16(t):
        return t.contiguous().view(__import__("torch").int16).numpy().view(np.uint16)

    t_quant = t_gemm = 0.0
    rng = np.random.default_rng(0)
    for li, (name, K, N) in enumerate(synth.LINEARS):
        x = u16(synth.randn_bf16((M, K), synth.X_STD, synth.stack_seed(0, li, synth.KIND_X)))
        w = u16(synth.randn_bf16((N, K), synth.W_STD, synth.stack_seed(0, li, synth.KIND_W)))
        dy = u16(synth.randn_bf16((M, N), synth.DY_STD, synth.stack_seed(0, li, synth.KIND_DY)))
        t0 = time.perf_counter()
        wq, sw = oracle.quant_w_128x128(w, pow2=pow2)
        xq, sx = oracle.quant_act_1x128(x, pow2=pow2)
        dyq, sdy = oracle.quant_act_1x128(dy, pow2=pow2)
        dytq, sdyt = oracle.quant_transpose(dy, pow2=pow2)
        xtq, sxt = oracle.quant_transpose(x, pow2=pow2)
        t1 = time.perf_counter()
        t_quant += t1 - t0
        rf = np.sort(rng.choice(M, rows_fwd, replace=False))
        rw = np.sort(rng.choice(N, rows_wgrad, replace=False))
        t0 = time.perf_counter()
        oracle.gemm_fwd(xq, sx, wq, sw, rows=rf)
        t1 = time.perf_counter()
        oracle.gemm_dgrad(dyq, sdy, wq, sw, rows=rf)
        t2 = time.perf_counter()
        oracle.gemm_wgrad(dytq, sdyt, xtq, sxt, rows=rw)
        t3 = time.perf_counter()
        t_gemm += (t1 - t0) * M / rows_fwd + (t2 - t1) * M / rows_fwd + (t3 - t2) * N / rows_wgrad
    step_s = layers * (t_quant + t_gemm)
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")),
                             None)
    except OSError:
        pass
    return {
        "value": M / step_s,
        "unit": "tokens/s",
        "cores": oracle.num_threads(),
        "cpu_model": cpu_model,
        "kind": "oracle",
        "sample": (f"layer 0 of the step: all 5 quantiser passes per linear at full size "
                   f"(timed), each GEMM on {rows_fwd} sampled output rows (fwd, dgrad) or "
                   f"{rows_wgrad} rows (wgrad) of all columns, extrapolated linearly to all rows "
                   f"and x{layers} layers"),
        "step_s_extrapolated": step_s,
        "quant_s_per_layer": t_quant,
        "gemm_s_per_layer_extrapolated": t_gemm,
    }


# algorithmic bytes per element of the optimizer kernels
B_HYPERBALL = 4 + 4 + 4 + 4 + 4 + 2   # read w, u; write v; read v; write w, w_bf16
B_ADAMW = 4 * 4 + 3 * 4                # read p, g, m, v; write p, m, v
ADAMW_STANDIN = 1 << 26                # elements of the AdamW measurement (stated size)


def optimizer_bench(stack, steps: int):
    """Optimizer step over the stack's 112 linear matrices, timed apart from the training step
    (it runs once per global batch, not per micro-batch): fp32 masters made from the bf16
    weights, their initial Frobenius radii, and each matrix's dW from the stack as the update
    direction; each projected step also rewrites the bf16 weight the quantiser reads. Plus
    AdamW on a stand-in fp32 parameter vector of ADAMW_STANDIN elements."""
    import ctypes

    import torch
    from blockwise_fp8_gemm_x128_amd import binding as B

    dev = torch.device("cuda:0")
    ws = B.optim_workspace(dev)
    masters, calls, numel = [], [], 0
    for w, dw in stack.weights:
        m = w.float()
        r = B.puro_frobenius_norm(m, workspace=ws)
        masters.append((m, r))
        calls.append(B.prepare("puro_hyperball_step", m, dw, m.numel(), 1e-3, r, w, ws))
        numel += m.numel()
    torch.cuda.synchronize()
    for call in calls:  # warm-up
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for e0, e1 in ev:
        e0.record(stack.stream)
        for call in calls:
            call()
        e1.record(stack.stream)
    torch.cuda.synchronize()
    ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / steps
    gbps = numel * B_HYPERBALL / (ms * 1e-3) / 1e9

    n = ADAMW_STANDIN
    p, g, mm, vv = (torch.randn(n, device=dev) * 0.02 for _ in range(4))
    vv = vv.abs()
    call = B.prepare("puro_adamw_step", p, g, mm, vv, n,
                     ctypes.byref(B.adamw_params(1e-3, 0.9, 0.95, 1e-8, 0.1, 1)),
                     None)
    call()
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(stack.stream)
    for _ in range(steps):
        call()
    a1.record(stack.stream)
    torch.cuda.synchronize()
    ams = a0.elapsed_time(a1) / steps
    agbps = n * B_ADAMW / (ams * 1e-3) / 1e9
    del masters
    return {
        "projected_step": {"matrices": len(calls), "elements": numel,
                           "ms_per_optimizer_step": ms, "gbps": gbps,
                           "frac_hbm_peak": gbps / PEAK_HBM_GBPS,
                           "bytes_per_element": B_HYPERBALL,
                           "direction": "the stack's dW (the pages do not give MuonH's)"},
        "adamw": {"elements": n, "ms_per_call": ams, "gbps": agbps,
                  "frac_hbm_peak": agbps / PEAK_HBM_GBPS, "bytes_per_element": B_ADAMW,
                  "inputs": "stand-in fp32 vector (the pages do not size the non-matrix "
                            "parameters)"},
        "timing": "HIP events around the whole set of calls on the launch stream, eager",
    }


def copy_calibration():
    """A plain streaming kernel of known size -- torch's elementwise negation over 2^28 fp32
    (reads 1 GiB, writes 1 GiB) -- the reference against which the FETCH_SIZE / WRITE_SIZE
    counters are scaled."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n}))


def source_digest(fn: str) -> str:
    """Digest of the sources of a kernel function, to tell whether stored counters still apply
    (GEMM functions: gemm.hip and its DMA offsets; quantiser functions: quant.hip; both with
    common.hpp)."""
    import hashlib
    h = hashlib.sha256()
    files = (("gemm.hip", "dma_offsets.hpp") if fn.startswith("gemm") else ("quant.hip",))
    for f in files + ("common.hpp",):
        with open(os.path.join(ROOT, "blockwise_fp8_gemm_x128_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic_qwen3_1p7b_linear_stack_M8192.txt")


def stored_traffic(fn: str):
    """Average HBM bytes per launch of a kernel function in the step, from the committed
    FETCH_SIZE / WRITE_SIZE summary (its `traffic-record:` lines, counters already scaled by the
    copy-kernel factors), or None if there is none or the function's sources changed since the
    counters were taken."""
    try:
        with open(TRAFFIC_SUMMARY) as fh:
            recs = [json.loads(l.split(":", 1)[1]) for l in fh if l.startswith("traffic-record:")]
    except (OSError, ValueError):
        return None
    for t in recs:
        if t.get("function") == fn and t.get("source_digest") == source_digest(fn):
            return 1024.0 * (t["fetch_kib_per_launch"] * t["fetch_factor"] +
                             t["write_kib_per_launch"] * t["write_factor"])
    return None


def _loop_us(call, reps: int, stream) -> float:
    """Average duration in us of `reps` back-to-back calls (call(i) launches rep i), from one
    HIP event pair on the launch stream around the whole loop."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(2):
        call(i)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(reps):
        call(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return 1e3 * e0.elapsed_time(e1) / reps


def copy_ceiling(reps: int = 10):
    """Plain streaming ceiling measured in the same run: torch's elementwise negation of a
    256 Mi-element bf16 tensor (512 MiB read, 512 MiB written, twice the 256 MB memory-side
    cache), `reps` times back to back."""
    import torch
    st = torch.cuda.current_stream()
    n = 1 << 28
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    us = _loop_us(lambda i: torch.neg(src, out=dst), reps, st)
    del src, dst
    return {"gbps": 4.0 * n / (us * 1e-6) / 1e9, "bytes_per_call": 4 * n,
            "kernel": "torch.neg on bf16 (2 B read + 2 B written per element)"}


def quant_vs_copy(shapes, reps: int = 30, pow2: bool = False):
    """Per quantiser shape of the step: the two-orientation quantiser and a plain copy of the
    same bf16 input (torch.neg, 2 B read + 2 B written per element), each timed as `reps`
    back-to-back launches rotating over enough input copies (> 1 GB) that the memory-side cache
    cannot serve them; GB/s by each one's own bytes."""
    import torch
    from blockwise_fp8_gemm_x128_amd import binding as B
    st = torch.cuda.current_stream()
    out = {}
    for rows, cols in shapes:
        n = rows * cols
        nc = max(2, -(-(1 << 30) // (2 * n)))
        xs = [torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda").normal_()
              for _ in range(nc)]
        q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
        qt = torch.empty((cols, rows), dtype=torch.uint8, device="cuda")
        s = torch.empty((cols // 128, rows), dtype=torch.float32, device="cuda")
        sT = torch.empty((rows // 128, cols), dtype=torch.float32, device="cuda")
        dst = torch.empty_like(xs[0])
        name = "puro_quant_dual_1x128" + ("_pow2" if pow2 else "")
        calls = [B.prepare(name, x, rows, cols, q, s, qt, sT, stream=st) for x in xs]
        uq = _loop_us(lambda i: calls[i % nc](), reps, st)
        uc = _loop_us(lambda i: torch.neg(xs[i % nc], out=dst), reps, st)
        gq = n * B_DUAL / (uq * 1e-6) / 1e9
        gc = 4.0 * n / (uc * 1e-6) / 1e9
        out[f"{rows}x{cols}"] = {"quant_us": uq, "quant_gbps": gq, "copy_us": uc,
                                 "copy_gbps": gc, "quant_over_copy": gq / gc}
        del xs, calls, q, qt, s, sT, dst
    return out


# Single-layer configurations measured by `--config` (the default run is the 28-layer step):
#   c1  one layer forward at M = 4096: quantise X per 1x128 group, W per 128x128 block, Y = X W^T
#   c2  the same four linears, forward + data gradient + weight gradient at M = 16384, with the
#       two-orientation quantiser for X and dY
#   c3  the down projection's outlier stress inputs at M = 16384, forward + both gradients
CONFIGS = {
    "c1": {"M": 4096, "seed": 1, "linears": (0, 1, 2, 3), "backward": False,
           "workload": "one Qwen3-1.7B-shaped layer forward (qkv, o, gate_up, down), M = 4096"},
    "c2": {"M": 16384, "seed": 2, "linears": (0, 1, 2, 3), "backward": True,
           "workload": "the four linears of one layer, fwd + dgrad + wgrad, M = 16384"},
    "c3": {"M": 16384, "seed": 3, "linears": (3,), "backward": True, "outlier": True,
           "workload": "down projection outlier stress (1% channels x100, 0.1% zero tiles, "
                       "one 128x128 W block x50), fwd + dgrad + wgrad, M = 16384"},
}


def run_config(name: str, reps: int, cpu: bool):
    """One JSON line for a single-layer configuration: every GEMM's TFLOP/s and every
    quantiser's GB/s (each timed as `reps` back-to-back launches with one HIP event pair;
    quantisers rotate over input copies totalling > 1 GB, GEMMs reuse one set of operands) with
    their fractions of the 5.0 PFLOP/s and 8 TB/s peaks and the roofline times; and the oracle
    on the host cores (full size for c1 and c3, 512 sampled output rows per GEMM for c2)."""
    import numpy as np
    import torch
    from blockwise_fp8_gemm_x128_amd import binding as B
    from blockwise_fp8_gemm_x128_amd import synth

    cfg = CONFIGS[name]
    M = cfg["M"]
    st = torch.cuda.current_stream()
    gemms, quants = {}, {}
    host = []  # bf16 inputs per linear, for the oracle
    for li in cfg["linears"]:
        lname, K, N = synth.LINEARS[li]
        if cfg.get("outlier"):
            x, w, dy, _ = synth.outlier_inputs(M=M, K=K, N=N, config=cfg["seed"], linear=li)
        else:
            x, w, dy = synth.linear_inputs(cfg["seed"], li, M, K, N)
        host.append((lname, K, N, x, w, dy))
        nc = max(2, -(-(1 << 30) // (2 * M * max(K, N))))
        xs = [x.cuda() for _ in range(nc)]
        dys = [dy.cuda() for _ in range(nc)] if cfg["backward"] else []
        wd = w.cuda()
        f = 2.0 * M * N * K
        wq, sw = B.puro_quant_w_128x128(wd)
        P = B.prepare
        c = P("puro_quant_w_128x128", wd, N, K, wq, sw, stream=st)
        quants[f"quant_w_128x128[{lname} {N}x{K}]"] = {"us": _loop_us(lambda i: c(), reps, st),
                                                       "bytes": N * K * B_W}
        if not cfg["backward"]:
            xq, sx = B.puro_quant_act_1x128(xs[0])
            cs = [P("puro_quant_act_1x128", xx, M, K, xq, sx, stream=st) for xx in xs]
            us = _loop_us(lambda i: cs[i % nc](), reps, st)
            quants[f"quant_act_1x128[{lname} X {M}x{K}]"] = {"us": us, "bytes": M * K * B_ACT}
            y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            c = P("puro_fp8_gemm_fwd", xq, sx, wq, sw, y, M, N, K, stream=st)
            gemms[f"fwd[{lname}]"] = {"us": _loop_us(lambda i: c(), reps, st), "flops": f,
                                      "kernel": B.puro_gemm_kernel_name("fwd", M, N, K)}
            del xs
            continue
        xq, sx, xtq, sxt = B.puro_quant_dual_1x128(xs[0])
        cs = [P("puro_quant_dual_1x128", xx, M, K, xq, sx, xtq, sxt, stream=st) for xx in xs]
        us = _loop_us(lambda i: cs[i % nc](), reps, st)
        quants[f"quant_dual_1x128[{lname} X {M}x{K}]"] = {"us": us, "bytes": M * K * B_DUAL}
        dyq, sdy, dytq, sdyt = B.puro_quant_dual_1x128(dys[0])
        cs = [P("puro_quant_dual_1x128", dd, M, N, dyq, sdy, dytq, sdyt, stream=st) for dd in dys]
        us = _loop_us(lambda i: cs[i % nc](), reps, st)
        quants[f"quant_dual_1x128[{lname} dY {M}x{N}]"] = {"us": us, "bytes": M * N * B_DUAL}
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        dx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
        dw = torch.empty((N, K), dtype=torch.float32, device="cuda")
        for op, c in (("fwd", P("puro_fp8_gemm_fwd", xq, sx, wq, sw, y, M, N, K, stream=st)),
                      ("dgrad", P("puro_fp8_gemm_dgrad", dyq, sdy, wq, sw, dx, M, N, K,
                                  stream=st)),
                      ("wgrad", P("puro_fp8_gemm_wgrad", dytq, sdyt, xtq, sxt, dw, M, N, K, 0,
                                  stream=st))):
            gemms[f"{op}[{lname}]"] = {"us": _loop_us(lambda i: c(), reps, st), "flops": f,
                                       "kernel": B.puro_gemm_kernel_name(op, M, N, K)}
        del xs, dys
    for d in gemms.values():
        d["tflops"] = d["flops"] / (d["us"] * 1e-6) / 1e12
        d["frac_fp8_peak"] = d["tflops"] / PEAK_FP8_TFLOPS
        d["roofline_us"] = d["flops"] / (PEAK_FP8_TFLOPS * 1e12) * 1e6
    for d in quants.values():
        d["gbps"] = d["bytes"] / (d["us"] * 1e-6) / 1e9
        d["frac_hbm_peak"] = d["gbps"] / PEAK_HBM_GBPS
        d["roofline_us"] = d["bytes"] / (PEAK_HBM_GBPS * 1e9) * 1e6
    g_us = sum(d["us"] for d in gemms.values())
    q_us = sum(d["us"] for d in quants.values())
    g_fl = sum(d["flops"] for d in gemms.values())
    q_by = sum(d["bytes"] for d in quants.values())
    out = {
        "metric": METRIC,
        "value": g_fl / (g_us * 1e-6) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": reps, "warmup": 2, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic (seeded N(0,1) X, N(0,0.02^2) W, N(0,1e-3^2) dY, bf16)",
        "config": {"workload": cfg["workload"], "name": name, "tokens": M},
        "gemm_tflops": g_fl / (g_us * 1e-6) / 1e12,
        "gemm_frac_fp8_peak": g_fl / (g_us * 1e-6) / 1e12 / PEAK_FP8_TFLOPS,
        "gemm_us": g_us, "gemm_roofline_us": g_fl / (PEAK_FP8_TFLOPS * 1e12) * 1e6,
        "quant_gbps": q_by / (q_us * 1e-6) / 1e9,
        "quant_frac_hbm_peak": q_by / (q_us * 1e-6) / 1e9 / PEAK_HBM_GBPS,
        "quant_us": q_us, "quant_roofline_us": q_by / (PEAK_HBM_GBPS * 1e9) * 1e6,
        "gemms": gemms, "quantisers": quants,
        "timing": ("HIP event pair around reps back-to-back launches on the launch stream; "
                   "quantisers rotate over input copies totalling > 1 GB; GEMMs reuse one set "
                   "of operands"),
    }
    if cpu:
        out["cpu_baseline"] = config_cpu_baseline(name, host, M, cfg["backward"])
    return out


def config_cpu_baseline(name, host, M, backward):
    """The oracle on the host cores for one configuration: every quantiser at full size; the
    GEMMs at full size (c1, c3) or on 512 seeded sampled output rows each, extrapolated linearly
    (c2)."""
    import numpy as np

    import oracle
    rows_n = None if name in ("c1", "c3") else 512
    rng = np.random.default_rng(0)
    t_q = t_g = 0.0
    flops = 0.0

    def u16(t):
        return t.contiguous().view(__import__("torch").int16).numpy().view(np.uint16)

    for lname, K, N, x, w, dy in host:
        t0 = time.perf_counter()
        wq, sw = oracle.quant_w_128x128(u16(w))
        xq, sx = oracle.quant_act_1x128(u16(x))
        if backward:
            dyq, sdy = oracle.quant_act_1x128(u16(dy))
            dytq, sdyt = oracle.quant_transpose(u16(dy))
            xtq, sxt = oracle.quant_transpose(u16(x))
        t_q += time.perf_counter() - t0
        rm = None if rows_n is None else np.sort(rng.choice(M, rows_n, replace=False))
        rw = None if rows_n is None else np.sort(rng.choice(N, min(rows_n, N), replace=False))
        sc_m = 1.0 if rm is None else M / len(rm)
        sc_n = 1.0 if rw is None else N / len(rw)
        t0 = time.perf_counter()
        oracle.gemm_fwd(xq, sx, wq, sw, rows=rm)
        t_g += (time.perf_counter() - t0) * sc_m
        flops += 2.0 * M * N * K
        if backward:
            t0 = time.perf_counter()
            oracle.gemm_dgrad(dyq, sdy, wq, sw, rows=rm)
            t_g += (time.perf_counter() - t0) * sc_m
            t0 = time.perf_counter()
            oracle.gemm_wgrad(dytq, sdyt, xtq, sxt, rows=rw)
            t_g += (time.perf_counter() - t0) * sc_n
            flops += 4.0 * M * N * K
    return {"value": flops / t_g / 1e9, "unit": "GFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "gemm_s": t_g, "quant_s": t_q,
            "sample": ("every GEMM at full size" if rows_n is None else
                       f"each GEMM on {rows_n} sampled output rows (all columns), extrapolated "
                       f"linearly to all rows") + "; every quantiser at full size (timed apart)"}


def mfma_ceiling(iters: int = 100000):
    """Register-only rate of the GEMMs' instruction (v_mfma_f32_16x16x128_f8f6f4), from the
    microbenchmark in csrc/ceiling.hip: 8 independent products per round on operands loaded
    once, in three modes (0: accumulate in the matrix core; 1: + 4 FMAs per product, the
    forward/data-gradient promotion; 2: + 4 multiplies and 4 FMAs, the weight-gradient one), at
    2 and 4 waves per SIMD (256 or 512 blocks of 8 waves), on three operand patterns. The rate
    is flops over the launch's HIP-event duration; the clock is the median wave's shader-clock
    cycles (s_memtime) over the same duration, and `ticks_mhz` the constant-rate counter's
    (s_memrealtime) rate as a check on the timing."""
    import ctypes

    import torch
    from blockwise_fp8_gemm_x128_amd import binding as B
    from blockwise_fp8_gemm_x128_amd.build import PROBE_PATH

    if not os.path.exists(PROBE_PATH):
        raise SystemExit(f"{PROBE_PATH} is missing: build first (python -c 'import "
                         "__graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(PROBE_PATH)
    fn = lib.puro_probe_mfma
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                   ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.c_void_p]
    st = torch.cuda.current_stream()
    nbytes = 1 << 20
    g = torch.Generator().manual_seed(7)
    rnd = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g)
    rnd[(rnd & 0x7F) == 0x7F] = 0x7E  # no NaN codes (S.1111.111)
    x = (torch.randn((nbytes // 128, 128), generator=g) * 1.0).to(torch.bfloat16).cuda()
    xq, _ = B.puro_quant_act_1x128(x)
    patterns = {"zero": torch.zeros(nbytes, dtype=torch.uint8, device="cuda"),
                "random E4M3 codes": rnd.cuda(),
                "quantised N(0,1) bf16": xq.reshape(-1).contiguous()}
    modes = {0: "MFMA chain", 1: "+ 4 FMAs per product", 2: "+ 4 multiplies + 4 FMAs"}
    out = {}
    for pname, codes in patterns.items():
        for wps in (2, 4):
            blocks = 256 * wps // 2
            waves = blocks * 8
            cyc = torch.zeros(waves, dtype=torch.int64, device="cuda")
            tck = torch.zeros(waves, dtype=torch.int64, device="cuda")
            sink = torch.zeros(waves * 64, dtype=torch.float32, device="cuda")
            for mode, mname in modes.items():
                def launch(n):
                    rc = fn(codes.data_ptr(), nbytes, blocks, 8, n, mode, cyc.data_ptr(),
                            tck.data_ptr(), sink.data_ptr(), ctypes.c_void_p(st.cuda_stream))
                    if rc != 0:
                        raise RuntimeError(f"puro_probe_mfma returned {rc}")
                launch(iters // 10)
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(st)
                launch(iters)
                e1.record(st)
                torch.cuda.synchronize()
                sec = e0.elapsed_time(e1) * 1e-3
                flops = waves * iters * 8 * 2.0 * 16 * 16 * 128
                clk = float(cyc.double().median()) / sec / 1e9
                pf = flops / sec / 1e15
                out[f"{pname} | {wps} waves/SIMD | {mname}"] = {
                    "pflops": pf, "frac_of_5pf": pf / 5.0, "ms": sec * 1e3,
                    "clock_ghz": clk, "frac_at_that_clock": pf / (5.0 * clk / 2.4),
                    "ticks_mhz": float(tck.double().median()) / sec / 1e6}
    print(json.dumps({"mfma_ceiling": out, "iters": iters,
                      "instruction": "v_mfma_f32_16x16x128_f8f6f4 (E4M3 x E4M3, fp32)",
                      "peak_assumed": "5.0 PFLOP/s dense FP8 at 2.4 GHz"}), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.ceiling:
        mfma_ceiling()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(multi-GPU runs are out of scope: the path shards by data parallelism, see the "
              "design notes)", file=sys.stderr)
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    if args.config:
        for name in (("c1", "c2", "c3") if args.config == "all" else (args.config,)):
            print(json.dumps(run_config(name, max(args.steps, 5), not args.no_cpu_baseline)),
                  flush=True)
        return
    M = M_TOKENS
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):  # every launch is bound to this stream when prepared
        stack = Stack(args.layers, M, fused=not args.unfused, pow2=args.pow2)
    torch.cuda.synchronize()
    overlap = args.overlap
    with torch.cuda.stream(side):
        for _ in range(args.warmup):
            stack.run(overlap=overlap)
    torch.cuda.synchronize()
    use_graph = not args.no_graph
    if use_graph:
        stack.capture(overlap=overlap)
        stack.replay()  # one untimed replay
        torch.cuda.synchronize()

    # Timed region: K whole steps (one graph replay each, or eager launches).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(side):
        for _ in range(args.steps):
            if use_graph:
                stack.replay()
            else:
                stack.run(overlap=overlap)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    # Kernel timing pass: the same K steps launched eagerly, in the serial order on the main
    # stream, with a HIP event pair around every launch (events cannot be placed inside the
    # replayed graph; the serial order gives each kernel's own duration, not a share of the
    # chip it had while overlapping another).
    ev_sets = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in stack.launches] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    with torch.cuda.stream(side):
        for k in range(args.steps):
            stack.run(ev_sets[k])
    torch.cuda.synchronize()
    eager_ms_per_step = (time.perf_counter() - t1) * 1e3 / args.steps

    per_class = {}
    if True:
        for evs in ev_sets:
            for op, (e0, e1) in zip(stack.launches, evs):
                cls, fl, by = op.cls, op.flops, op.bytes
                d = per_class.setdefault(cls, {"ms": 0.0, "launches": 0, "flops": 0.0,
                                               "bytes": 0.0})
                d["ms"] += e0.elapsed_time(e1)
                d["launches"] += 1
                d["flops"] += fl
                d["bytes"] += by
    kernels = {}
    for cls, d in per_class.items():
        n = args.steps
        ent = {"ms_per_step": d["ms"] / n, "launches_per_step": d["launches"] // n,
               "avg_launch_us": 1e3 * d["ms"] / d["launches"]}
        if d["flops"]:
            tf = d["flops"] / (d["ms"] * 1e-3) / 1e12
            ent.update({"tflops": tf, "frac_fp8_peak": tf / PEAK_FP8_TFLOPS})
        else:
            gb = d["bytes"] / (d["ms"] * 1e-3) / 1e9
            ent.update({"gbps": gb, "frac_hbm_peak": gb / PEAK_HBM_GBPS})
        kernels[cls] = ent
    by_kind = {}
    for c, v in kernels.items():
        kind = c.split("[")[0]
        e = by_kind.setdefault(kind, {"ms_per_step": 0.0, "launches_per_step": 0})
        e["ms_per_step"] += v["ms_per_step"]
        e["launches_per_step"] += v["launches_per_step"]
    for kind, e in by_kind.items():
        fl = sum(op.flops for op in stack.launches if op.cls.split("[")[0] == kind)
        by = sum(op.bytes for op in stack.launches if op.cls.split("[")[0] == kind)
        secs = e["ms_per_step"] * 1e-3
        e["avg_launch_us"] = 1e3 * e["ms_per_step"] / e["launches_per_step"]
        if fl:
            e["tflops"] = fl / secs / 1e12
            e["frac_fp8_peak"] = e["tflops"] / PEAK_FP8_TFLOPS
        else:
            e["gbps"] = by / secs / 1e9
            e["frac_hbm_peak"] = e["gbps"] / PEAK_HBM_GBPS
    # Per kernel function: the launches that run the same compiled kernel (one function can
    # serve several shapes; one launch kind can use several functions).
    by_fn = {}
    for evs in ev_sets:
        for op, (e0, e1) in zip(stack.launches, evs):
            d = by_fn.setdefault(op.fn, {"ms": 0.0, "launches": 0, "flops": 0.0, "bytes": 0.0,
                                         "traffic": 0.0, "classes": set()})
            d["ms"] += e0.elapsed_time(e1)
            d["launches"] += 1
            d["flops"] += op.flops
            d["bytes"] += op.bytes
            d["traffic"] += op.traffic
            d["classes"].add(op.cls)
    kernels_by_fn = {}
    for fn, d in by_fn.items():
        secs = d["ms"] * 1e-3
        ent = {"ms_per_step": d["ms"] / args.steps,
               "launches_per_step": d["launches"] // args.steps,
               "avg_launch_us": 1e3 * d["ms"] / d["launches"],
               "work_per_launch": (d["flops"] or d["bytes"]) / d["launches"],
               "traffic_bytes_per_launch": d["traffic"] / d["launches"],
               "classes": sorted(d["classes"])}
        if d["flops"]:
            ent["tflops"] = d["flops"] / secs / 1e12
            ent["frac_fp8_peak"] = ent["tflops"] / PEAK_FP8_TFLOPS
        else:
            ent["gbps"] = d["bytes"] / secs / 1e9
            ent["frac_hbm_peak"] = ent["gbps"] / PEAK_HBM_GBPS
        kernels_by_fn[fn] = ent
    # Dominant kernel: the kernel function with the most time per step. achieved = its
    # algorithmic work per launch, averaged over its launches (flops or bytes of all its
    # launches / their number), / its average launch duration (HIP events on the launch stream).
    roofline = None
    if kernels_by_fn:
        dom = max(kernels_by_fn, key=lambda c: kernels_by_fn[c]["ms_per_step"])
        k = kernels_by_fn[dom]
        common = {"traffic": stored_traffic(dom),
                  "traffic_unit": "HBM bytes per launch, averaged over the function's launches "
                                  "(rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a plain copy "
                                  "kernel)",
                  "kernel": dom, "avg_launch_us": k["avg_launch_us"],
                  "launches_per_step": k["launches_per_step"],
                  "work_per_launch": (by_fn[dom]["flops"] or by_fn[dom]["bytes"]) /
                                     by_fn[dom]["launches"],
                  "source_digest": source_digest(dom)}
        if "tflops" in k:
            roofline = {"bound": "mfma", "achieved": k["tflops"], "peak": PEAK_FP8_TFLOPS,
                        "unit": "TFLOP/s", "frac": k["frac_fp8_peak"], **common}
        else:
            roofline = {"bound": "hbm", "achieved": k["gbps"], "peak": PEAK_HBM_GBPS,
                        "unit": "GB/s", "frac": k["frac_hbm_peak"], **common}
    gemm_ms = sum(v["ms_per_step"] for c, v in kernels.items() if c.startswith("gemm"))
    quant_ms = sum(v["ms_per_step"] for c, v in kernels.items() if c.startswith("quant"))
    gemm_flops = sum(op.flops for op in stack.launches)
    quant_bytes = sum(op.bytes for op in stack.launches)
    roof_ms = (gemm_flops / (PEAK_FP8_TFLOPS * 1e12) + quant_bytes / (PEAK_HBM_GBPS * 1e9)) * 1e3

    out = {
        "metric": METRIC,
        "value": M / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic (seeded N(0,1) X, N(0,0.02^2) W, N(0,1e-3^2) dY, bf16)",
        "config": {"workload": "Qwen3-1.7B-shaped linear stack step: 28 layers x "
                               "{qkv 2048->4096, o 2048->2048, gate_up 2048->12288, "
                               "down 6144->2048}, fwd + dgrad + wgrad + all quantisers",
                   "tokens_per_step": M, "seqs": M // 4096, "seq_len": 4096,
                   "layers": args.layers, "parallelism": "single GPU",
                   "quantisers": ("separate per orientation" if args.unfused else
                                  "fused two-orientation 1x128 for X and dY"),
                   "scales": ("power of two (E8M0), applied by the matrix cores" if args.pow2
                              else "fp32 amax/448, promoted in fp32 per 128-chunk")},
        "gemm_tflops": gemm_flops / (gemm_ms * 1e-3) / 1e12 if gemm_ms else None,
        "gemm_frac_fp8_peak": (gemm_flops / (gemm_ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS
                               if gemm_ms else None),
        "quant_gbps": quant_bytes / (quant_ms * 1e-3) / 1e9 if quant_ms else None,
        "quant_frac_hbm_peak": (quant_bytes / (quant_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS
                                if quant_ms else None),
        "roofline_step_ms": roof_ms,
        "step_frac_of_roofline": roof_ms / ms_per_step,
        "kernel_event_sum_ms_per_step": gemm_ms + quant_ms,
        "timed_region": ("one captured HIP graph replay per step" if use_graph
                         else "eager launches"),
        "launch_order": ("overlapped: critical chain on the main stream; weight quantisation "
                         "and weight-gradient GEMMs on a side stream, joined by events"
                         if overlap else "serial, one stream"),
        "kernel_timing": "HIP event pair per launch, serial order on one stream",
        "kernel_timing_pass_ms_per_step": eager_ms_per_step,
        "kernels_by_function": kernels_by_fn,
        "kernels_by_kind": by_kind,
        "kernels": kernels,
        "roofline": roofline,
    }
    if not args.no_optim:
        with torch.cuda.stream(side):
            out["optimizer"] = optimizer_bench(stack, args.steps)
    if not args.no_copy_ceiling:
        del stack
        torch.cuda.empty_cache()
        out["copy_ceiling"] = copy_ceiling()
        out["quant_vs_copy"] = quant_vs_copy(
            sorted({(M, n) for n in (2048, 4096, 6144, 12288)}), pow2=args.pow2)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(M, args.layers, pow2=args.pow2)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
