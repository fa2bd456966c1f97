"""Benchmark of the FP8 linear layer hot path on one MI355X.

A step is one pass of the layer over one batch of synthetic input, inputs
resident in HBM: quantize the activation and the weight (amax -> scale ->
saturating cast; rowwise, both tensors in one launch since they share K) and
run the scaled FP8 GEMM. The default workload is the
Llama3-8B FFN up-projection, rowwise e4m3: X bf16 [8192 x 4096] (Student-t,
unit variance), W bf16 [14336 x 4096] ~ N(0, 0.02^2), bf16 output.

Prints one JSON line: value = 2*M*N*K / (time per step) in TFLOP/s including
the quantizers; per-kernel durations come from HIP events recorded on the
stream the kernels run on; `roofline` is for the GEMM (the dominant kernel)
against MI355X's dense FP8 peak; `quantizers` gives each quantizer's
algorithmic GB/s (2 B read + 1 B written per element + 4 B per scale) against
8 TB/s; `cpu_baseline` times the CPU oracle on a bounded sample of the same
workload on this host's cores; `cold` repeats the step after evicting the
caches (a 1 GiB read before each step, outside the step's events) and gives
the median and minimum of every call. Before the W warmup steps, untimed
steps run for --settle-seconds (reported as `settle`), so that the timed
steps see the clock the device holds under sustained load.

Other workloads (--workload c1|c3|c4|c4b|c4mx|c5) print the same line for the
other shapes (c3 tensorwise delayed, c4 MoE grouped GEMM, c4b the MoE expert
layer's backward, c4mx c4 with MXFP8 block-32 E8M0 scales, c5 hybrid
backward, c6 the DeepSeek-V3 MoE layer forward: route, permute + cast,
gate|up grouped GEMM, SwiGLU + cast, down grouped GEMM, weighted combine;
c2bw c2's tensors with the blockwise recipe: 1 x 128 activation blocks,
128 x 128 weight tiles, power-of-two scales, the product on the MX kernel).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 scaled-GEMM TFLOP/s incl. quantize; quantizer GB/s; % of MI355X peak"
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 matrix throughput (no sparsity)
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
EVICT_BYTES = 1 << 30         # > 8 x 4 MB of L2 and the 256 MB last-level cache


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=100,
                   help="untimed steps first: the clock settles over the first few tens of ms of load")
    p.add_argument("--workload", default="c2", choices=["c1", "c2", "c2bw", "c3", "c4", "c4b", "c4mx", "c5", "c6"])
    p.add_argument("--cpu-seconds", type=float, default=20.0, help="target length of the CPU-oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--settle-seconds", type=float, default=1.0,
                   help="untimed steps for this long before the warmup steps (the clock ramps up over the first "
                        "tens of ms of load on a fresh device)")
    p.add_argument("--cold-steps", type=int, default=10,
                   help="steps timed after evicting the caches (0: skip the cold-cache leg)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="time a plain 1 GiB copy kernel instead (for scaling rocprofv3 byte counters)")
    return p.parse_args()


def bf16_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


class Step:
    """Holds device buffers of one workload and enqueues one step, recording an
    event after each kernel-level call."""

    def __init__(self, name):
        import torch

        import fp8_scaled_gemm_amax_amd as fp8
        import workloads
        self.fp8, self.torch, self.name = fp8, torch, name
        dev = "cuda:0"
        E = torch.empty
        if name in ("c1", "c2"):
            w = workloads.c1() if name == "c1" else workloads.c2()
            self.x, self.w = bf16_dev(w["x"]), bf16_dev(w["w"])
            self.cpu_sample = (w["x"], 0, w["w"], 0)
            m, k = self.x.shape
            n = self.w.shape[0]
            self.qx, self.qw = E((m, k), dtype=torch.uint8, device=dev), E((n, k), dtype=torch.uint8, device=dev)
            self.sx, self.sw = E(m, device=dev), E(n, device=dev)
            self.d = E((m, n), dtype=torch.bfloat16, device=dev)
            self.mnk = [(m, n, k)]
            # X and W share K: one rowwise-cast launch for both
            self.calls = [("quantize_row X+W (one launch)", m * k + n * k, m + n), ("gemm", None, 0)]
            self.desc = {"c1": "rowwise FP8 linear Y = X W^T, X bf16 [256x512] N(0,1) with 2 rows x50, "
                               "W bf16 [512x512] N(0,0.02^2); e4m3 rowwise both operands; bf16 out",
                         "c2": "Llama3-8B FFN up-proj rowwise FP8: X bf16 [8192x4096] Student-t(4)/sqrt(2), "
                               "W bf16 [14336x4096] N(0,0.02^2); e4m3 row/col scales; bf16 out"}[name]
            self.scales = {"recipe": "rowwise", "format": "e4m3"}
        elif name == "c2bw":
            w = workloads.c2()
            self.x, self.w = bf16_dev(w["x"]), bf16_dev(w["w"])
            self.cpu_sample = (w["x"], 0, w["w"], 0)
            self.cpu_kind = "blockwise"
            m, k = self.x.shape
            n = self.w.shape[0]
            self.qx, self.qw = E((m, k), dtype=torch.uint8, device=dev), E((n, k), dtype=torch.uint8, device=dev)
            self.sx, self.sw = fp8.mx_scale_records(m, k), fp8.mx_scale_records(n, k)
            self.d = E((m, n), dtype=torch.bfloat16, device=dev)
            self.mnk = [(m, n, k)]
            # (4-byte scale records: one per row per 128 columns)
            self.calls = [("blockwise_quantize_act X", m * k, m * k // 128),
                          ("blockwise_quantize_weight W", n * k, n * k // 128), ("gemm_mx", None, 0)]
            self.desc = ("Llama3-8B FFN up-proj, blockwise FP8: c2's X bf16 [8192x4096] and W bf16 [14336x4096]; "
                         "e4m3, 1x128 activation blocks, 128x128 weight tiles, power-of-two scales; bf16 out")
            self.scales = {"recipe": "blockwise", "format": "e4m3"}
        elif name == "c3":
            w = workloads.c3()
            self.w = bf16_dev(w["w"])
            _, xb = next(w["x_steps"]())
            self.x = bf16_dev(xb)
            self.cpu_sample = (xb, 0, w["w"], 0)
            self.cpu_kind = "tensor"
            m, k = self.x.shape
            n = self.w.shape[0]
            self.qx, self.qw = E((m, k), dtype=torch.uint8, device=dev), E((n, k), dtype=torch.uint8, device=dev)
            self.six, self.siw = E(1, device=dev), E(1, device=dev)
            self.hist = torch.zeros((2, 1024), device=dev)
            self.head = torch.zeros(1, dtype=torch.int32, device=dev)
            self.scale = torch.ones(2, device=dev)
            self.scale_inv = torch.ones(2, device=dev)
            self.cur = torch.zeros(2, device=dev)
            self.d = E((m, n), dtype=torch.bfloat16, device=dev)
            self.mnk = [(m, n, k)]
            # X and W share K: one delayed tensorwise cast launch for both
            self.calls = [("quantize_tensor X+W (delayed, one launch)", m * k + n * k, 2), ("gemm", None, 0),
                          ("delayed_scale_update", 0, 0)]
            self.desc = ("Flux-12B MLP linear, tensorwise delayed scaling: X bf16 [4608x3072] N(0,1), "
                         "W bf16 [12288x3072] N(0,0.02^2); history 1024, algo max, margin 0; bf16 out")
            self.scales = {"recipe": "delayed", "format": "e4m3"}
        elif name == "c4":
            w = workloads.c4()
            g, n, k = w["w"].shape
            self.x = bf16_dev(w["x"])
            self.w = bf16_dev(w["w"].reshape(g * n, k))
            self.offsets = torch.from_numpy(w["offsets"]).to(dev)
            self.cpu_sample = (w["x"], 0, w["w"][0], 0)
            m = self.x.shape[0]
            self.g, self.n, self.k = g, n, k
            self.qx, self.qw = E((m, k), dtype=torch.uint8, device=dev), E((g * n, k), dtype=torch.uint8, device=dev)
            self.sx, self.sw = E(m, device=dev), E(g * n, device=dev)
            self.d = E((m, n), dtype=torch.bfloat16, device=dev)
            self.mnk = [(m, n, k)]
            # tokens and expert weights share K: one rowwise-cast launch for both
            self.calls = [("quantize_row tokens+expert W (one launch)", m * k + g * n * k, m + g * n),
                          ("grouped_gemm", None, 0)]
            self.desc = ("DeepSeek-V3 MoE grouped GEMM, one GPU's share: 32 experts Zipf(1.1) counts (3 empty), "
                         "tokens bf16 [16384x7168] N(0,1), W_e bf16 [2048x7168] N(0,0.006^2); e4m3 rowwise; bf16 out")
            self.scales = {"recipe": "rowwise", "format": "e4m3"}
        elif name == "c4mx":
            w = workloads.c4()
            g, n, k = w["w"].shape
            self.x = bf16_dev(w["x"])
            self.w = bf16_dev(w["w"].reshape(g * n, k))
            self.offsets = torch.from_numpy(w["offsets"]).to(dev)
            self.cpu_sample = (w["x"], 0, w["w"][0], 0)
            self.cpu_kind = "mx"
            m = self.x.shape[0]
            self.g, self.n, self.k = g, n, k
            self.qx, self.qw = E((m, k), dtype=torch.uint8, device=dev), E((g * n, k), dtype=torch.uint8, device=dev)
            self.sx, self.sw = fp8.mx_scale_records(m, k), fp8.mx_scale_records(g * n, k)
            self.d = E((m, n), dtype=torch.bfloat16, device=dev)
            self.mnk = [(m, n, k)]
            # (4-byte scale records: k / 128 per row)
            self.calls = [("mx_quantize_row tokens", m * k, m * k // 512),
                          ("mx_quantize_row expert W", g * n * k, g * n * k // 512), ("grouped_gemm_mx", None, 0)]
            self.desc = ("DeepSeek-V3 MoE grouped GEMM, one GPU's share, MXFP8: c4's experts and tokens; e4m3 "
                         "elements with E8M0 scales per 32 elements along K (tokens and expert weights); bf16 out")
            self.scales = {"recipe": "mxfp8", "format": "e4m3"}
        elif name == "c6":
            w = workloads.c6()
            T, H = w["x"].shape
            nexp, I2, _ = w["w1"].shape
            k = w["idx"].shape[1]
            P, inter = T * k, I2 // 2
            self.T, self.H, self.E, self.I2, self.k, self.P, self.inter = T, H, nexp, I2, k, P, inter
            self.x = bf16_dev(w["x"])
            self.idx = torch.from_numpy(w["idx"]).to(dev)
            self.wts = torch.from_numpy(w["weights"]).to(dev)
            self.w1 = bf16_dev(w["w1"].reshape(nexp * I2, H))
            self.w2 = bf16_dev(w["w2"].reshape(nexp * H, inter))
            self.cpu_sample = w
            self.cpu_kind = "moe_layer"
            self.off = E(nexp + 1, dtype=torch.int64, device=dev)
            self.dest = E((T, k), dtype=torch.int32, device=dev)
            self.xq, self.xs = E((P, H), dtype=torch.uint8, device=dev), E(P, device=dev)
            self.w1q, self.w1s = E((nexp * I2, H), dtype=torch.uint8, device=dev), E(nexp * I2, device=dev)
            self.h = E((P, I2), dtype=torch.bfloat16, device=dev)
            self.aq, self.asi = E((P, inter), dtype=torch.uint8, device=dev), E(P, device=dev)
            self.w2q, self.w2s = E((nexp * H, inter), dtype=torch.uint8, device=dev), E(nexp * H, device=dev)
            self.y = E((P, H), dtype=torch.bfloat16, device=dev)
            self.out = E((T, H), dtype=torch.bfloat16, device=dev)
            self.mnk = [(P, I2, H), (P, H, inter)]
            # (name, elements, scales[, algorithmic bytes])
            self.calls = [("moe_route", 0, 0, 8 * T * k + 8 * (nexp + 1)),
                          ("moe_permute_quantize tokens", T * H, P, 2 * T * H + P * H + 4 * P),
                          ("quantize_row W1 (gate|up)", nexp * I2 * H, nexp * I2),
                          ("grouped_gemm gate|up", None, 0),
                          ("swiglu_quantize", P * inter, P, 4 * P * inter + P * inter + 4 * P),
                          ("quantize_row W2 (down)", nexp * H * inter, nexp * H),
                          ("grouped_gemm down", None, 0),
                          ("moe_unpermute_combine", 0, 0, 2 * P * H + 2 * T * H + 8 * T * k)]
            self.desc = ("DeepSeek-V3 MoE layer forward, one GPU's share: 2048 tokens [2048x7168] N(0,1), top-8 of "
                         "32 experts (Zipf(1.1) popularity, softmax weights), SwiGLU experts gate|up W1 "
                         "[32x4096x7168], down W2 [32x7168x2048] N(0,0.006^2); e4m3 rowwise, weights quantized "
                         "every step; bf16 out")
            self.scales = {"recipe": "rowwise", "format": "e4m3"}
        elif name == "c4b":
            w = workloads.c4b()
            g, n, k = w["w"].shape
            t = w["x"].shape[0]
            self.g, self.n, self.k, self.t = g, n, k, t
            self.x, self.dy = bf16_dev(w["x"]), bf16_dev(w["dy"])
            self.w = bf16_dev(w["w"].reshape(g * n, k))
            self.offsets = torch.from_numpy(w["offsets"]).to(dev)
            woff = np.arange(g + 1, dtype=np.int64) * n
            self.woffsets = torch.from_numpy(woff).to(dev)
            self.cpu_sample = (w["dy"], 1, np.ascontiguousarray(w["w"][0].T), 0)   # dgrad: dY rows, W_0^T rows
            L = fp8.grouped_layout_width(t, g)
            self.dyq, self.dys = E((t, n), dtype=torch.uint8, device=dev), E(t, device=dev)
            self.wt = E((k, g * n), dtype=torch.uint8, device=dev)
            self.wts, self.wta = E((g, k), device=dev), E((g, k), device=dev)
            self.dx = E((t, k), dtype=torch.bfloat16, device=dev)
            self.dyt = torch.zeros((n, L), dtype=torch.uint8, device=dev)
            self.xt = torch.zeros((k, L), dtype=torch.uint8, device=dev)
            self.dyts, self.dyta = E((g, n), device=dev), E((g, n), device=dev)
            self.xts, self.xta = E((g, k), device=dev), E((g, k), device=dev)
            self.dw = E((g, n, k), dtype=torch.bfloat16, device=dev)
            # the forward's rowwise cast of the tokens X and the expert weights W
            # left their per-group column amax as side outputs (token groups,
            # and each expert's n weight rows): the backward's grouped colwise
            # casts of X^T and W^T take them as ready
            qx, qw = E((t, k), dtype=torch.uint8, device=dev), E((g * n, k), dtype=torch.uint8, device=dev)
            fp8.fp8_quantize_row_batch([self.x, self.w], fp8.E4M3, 0, [qx, qw], [E(t, device=dev), E(g * n, device=dev)],
                                       None, [self.xta, self.wta], [self.offsets, self.woffsets])
            torch.cuda.synchronize()
            del qx, qw
            self.mnk = [(t, k, n), (n, k, t)]
            # dY^T right after dY's row cast (dY still in the last-level cache),
            # each product right after the casts it reads
            self.calls = [("quantize_row dY e5m2 with per-expert column amax (clear + one pass)", t * n, t,
                           3.0 * t * n + 4.0 * t + 4.0 * g * n),
                          ("grouped_quantize_col dY^T e5m2 (column amax from the row cast)", t * n, g * n,
                           3.0 * t * n + 8.0 * g * n),
                          ("grouped_quantize_col W^T e4m3 (column amax from the forward)", g * n * k, g * k,
                           3.0 * g * n * k + 8.0 * g * k),
                          ("grouped_gemm dgrad", None, 0),
                          ("grouped_quantize_col X^T e4m3 (column amax from the forward)", t * k, g * k,
                           3.0 * t * k + 8.0 * g * k),
                          ("grouped_gemm_ragged_k wgrad", None, 0)]
            self.desc = ("DeepSeek-V3 MoE expert layer backward, one GPU's share: c4's experts and tokens, "
                         "dY bf16 [16384x2048] N(0,1e-3^2) e5m2; dgrad dX_g = dY_g W_g (grouped GEMM), "
                         "wgrad dW_g = dY_g^T X_g over each expert's tokens (ragged-K grouped GEMM); per-expert "
                         "column amax of X and W from the forward cast's side outputs, of dY from its row cast; "
                         "bf16 out")
            self.scales = {"recipe": "rowwise+grouped colwise", "format": "e5m2 x e4m3"}
        else:
            w = workloads.c5()
            self.x, self.w, self.dy = bf16_dev(w["x"]), bf16_dev(w["w"]), bf16_dev(w["dy"])
            self.cpu_sample = (w["dy"], 1, np.ascontiguousarray(w["w"].T), 0)   # dgrad: dY rows, W^T rows
            m, k = self.x.shape
            n = self.w.shape[0]
            self.qdy, self.sdy = E((m, n), dtype=torch.uint8, device=dev), E(m, device=dev)
            self.cady = E(n, device=dev)
            self.qdyt, self.sdyt = E((n, m), dtype=torch.uint8, device=dev), E(n, device=dev)
            self.qwt, self.swt, self.caw = E((k, n), dtype=torch.uint8, device=dev), E(k, device=dev), E(k, device=dev)
            self.qxt, self.sxt, self.cax = E((k, m), dtype=torch.uint8, device=dev), E(k, device=dev), E(k, device=dev)
            self.dx = E((m, k), dtype=torch.bfloat16, device=dev)
            self.dw = E((n, k), dtype=torch.bfloat16, device=dev)
            # the forward's rowwise cast of X and W left their column amax as side
            # outputs (fp8_quantize_row_batch with col_amax_out): the backward's
            # colwise casts of X^T and W^T take them as ready
            qx, qw = E((m, k), dtype=torch.uint8, device=dev), E((n, k), dtype=torch.uint8, device=dev)
            fp8.fp8_quantize_row_batch([self.x, self.w], fp8.E4M3, 0, [qx, qw], [E(m, device=dev), E(n, device=dev)],
                                       None, [self.cax, self.caw])
            torch.cuda.synchronize()
            del qx, qw
            self.mnk = [(m, k, n), (n, k, m)]
            # each product right after the casts it reads, so that their codes are
            # still in the last-level cache (and no other cast's dirty codes are)
            self.ady = E(m, device=dev)
            self.calls = [("quantize_rowcol dY e5m2 (row codes + col codes transposed, two passes)", 2 * m * n,
                           m + n, 6.0 * m * n + 4.0 * (m + n)),
                          ("quantize_col W^T e4m3 (col amax from the forward)", n * k, k),
                          ("gemm dgrad", None, 0),
                          ("quantize_col X^T e4m3 (col amax from the forward)", m * k, k),
                          ("gemm wgrad", None, 0)]
            self.desc = ("hybrid backward of the Llama3-8B up-proj: dY bf16 [8192x14336] N(0,1e-3^2) e5m2; "
                         "dgrad dX = dY W, wgrad dW = dY^T X with colwise token scales (X and W column amax "
                         "from the forward cast's side outputs); bf16 out")
            self.scales = {"recipe": "rowwise+colwise", "format": "e5m2 x e4m3"}
        self.flops = sum(2.0 * m * n * k for m, n, k in self.mnk)

    def extra(self, reps=50):
        """Measurements beside the step. Llama3-8B up-projection: the forward
        cast of X and W with their column amax as side outputs (what a training
        step's forward does so that the backward's colwise casts of X^T and W^T
        need no amax pass), algorithmic bytes 2 + 1 per element, 4 per row scale
        and 4 per column amax."""
        if self.name != "c2":
            return {}
        torch, f = self.torch, self.fp8
        m, k = self.x.shape
        n = self.w.shape[0]
        cx, cw = torch.empty(k, device="cuda:0"), torch.empty(k, device="cuda:0")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

        def cast():
            f.fp8_quantize_row_batch([self.x, self.w], f.E4M3, 0, [self.qx, self.qw], [self.sx, self.sw], None,
                                     [cx, cw])
        for _ in range(10):
            cast()
        e0.record()
        for _ in range(reps):
            cast()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nbytes = 3.0 * (m + n) * k + 4.0 * (m + n) + 8.0 * k
        return {"forward_cast_with_col_amax": {
            "kernel": "quantize_row X+W with column amax side outputs (clear + one pass)", "avg_ms": round(ms, 5),
            "algorithmic_bytes": nbytes, "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4), "reps": reps}}

    def run(self, ev):
        """Enqueue one step; ev[i] is recorded after call i (ev[0] before the first)."""
        f = self.fp8
        ev[0].record()
        if self.name in ("c1", "c2"):
            f.fp8_quantize_row_batch([self.x, self.w], f.E4M3, 0, [self.qx, self.qw], [self.sx, self.sw])
            ev[1].record()
            f.fp8_gemm_scaled(self.qx, f.E4M3, self.qw, f.E4M3, self.sx, f.SCALE_VECTOR, self.sw, f.SCALE_VECTOR,
                              self.d)
            ev[2].record()
        elif self.name == "c2bw":
            f.fp8_blockwise_quantize_act(self.x, f.E4M3, self.qx, self.sx)
            ev[1].record()
            f.fp8_blockwise_quantize_weight(self.w, f.E4M3, self.qw, self.sw)
            ev[2].record()
            f.fp8_gemm_mx(self.qx, f.E4M3, self.sx, self.qw, f.E4M3, self.sw, self.d)
            ev[3].record()
        elif self.name == "c3":
            f.fp8_quantize_tensor_batch([self.x, self.w], f.E4M3, [self.scale[0:1], self.scale[1:2]],
                                        [self.qx, self.qw], [self.six, self.siw], [self.cur[0:1], self.cur[1:2]])
            ev[1].record()
            f.fp8_gemm_scaled(self.qx, f.E4M3, self.qw, f.E4M3, self.six, f.SCALE_TENSOR, self.siw, f.SCALE_TENSOR,
                              self.d)
            ev[2].record()
            f.fp8_delayed_scale_update(self.cur, self.hist, self.head, f.AMAX_MAX, 0, f.E4M3, self.scale,
                                       self.scale_inv)
            ev[3].record()
        elif self.name == "c4":
            f.fp8_quantize_row_batch([self.x, self.w], f.E4M3, 0, [self.qx, self.qw], [self.sx, self.sw])
            ev[1].record()
            f.fp8_grouped_gemm_scaled(self.qx, f.E4M3, self.qw.view(self.g, self.n, self.k), f.E4M3, self.offsets,
                                      self.sx, self.sw.view(self.g, self.n), self.d)
            ev[2].record()
        elif self.name == "c4mx":
            g, n, k = self.g, self.n, self.k
            f.fp8_mx_quantize_row(self.x, f.E4M3, self.qx, self.sx)
            ev[1].record()
            f.fp8_mx_quantize_row(self.w, f.E4M3, self.qw, self.sw)
            ev[2].record()
            # expert e's weight records: rows e*n .. e*n+n-1 of the stacked records
            sw = self.torch.as_strided(self.sw, (g, k // 128, n, 4), (4 * n, 4 * g * n, 4, 1))
            f.fp8_grouped_gemm_mx(self.qx, f.E4M3, self.sx, self.qw.view(g, n, k), f.E4M3, sw, self.offsets, self.d)
            ev[3].record()
        elif self.name == "c6":
            E, I2, H, inter = self.E, self.I2, self.H, self.inter
            f.fp8_moe_route(self.idx, E, self.off, self.dest)
            ev[1].record()
            f.fp8_moe_permute_quantize_row(self.x, self.dest, f.E4M3, 0, self.xq, self.xs)
            ev[2].record()
            f.fp8_quantize_row(self.w1, f.E4M3, 0, self.w1q, self.w1s)
            ev[3].record()
            f.fp8_grouped_gemm_scaled(self.xq, f.E4M3, self.w1q.view(E, I2, H), f.E4M3, self.off, self.xs,
                                      self.w1s.view(E, I2), self.h)
            ev[4].record()
            f.fp8_swiglu_quantize_row(self.h, f.E4M3, 0, self.aq, self.asi)
            ev[5].record()
            f.fp8_quantize_row(self.w2, f.E4M3, 0, self.w2q, self.w2s)
            ev[6].record()
            f.fp8_grouped_gemm_scaled(self.aq, f.E4M3, self.w2q.view(E, H, inter), f.E4M3, self.off, self.asi,
                                      self.w2s.view(E, H), self.y)
            ev[7].record()
            f.fp8_moe_unpermute_combine(self.y, self.dest, self.wts, self.out)
            ev[8].record()
        elif self.name == "c4b":
            g, n, k = self.g, self.n, self.k
            f.fp8_quantize_row_batch([self.dy], f.E5M2, 0, [self.dyq], [self.dys], None, [self.dyta], [self.offsets])
            ev[1].record()
            f.fp8_grouped_quantize_col(self.dy, f.E5M2, 0, self.offsets, self.dyt, self.dyts, self.dyta,
                                       col_amax_ready=True)
            ev[2].record()
            f.fp8_grouped_quantize_col(self.w, f.E4M3, 0, self.woffsets, self.wt, self.wts, self.wta,
                                       col_amax_ready=True)
            ev[3].record()
            b_view = self.torch.as_strided(self.wt, (g, k, n), (n, g * n, 1))   # expert g: columns g*n.. of W^T
            f.fp8_grouped_gemm_scaled(self.dyq, f.E5M2, b_view, f.E4M3, self.offsets, self.dys, self.wts, self.dx)
            ev[4].record()
            f.fp8_grouped_quantize_col(self.x, f.E4M3, 0, self.offsets, self.xt, self.xts, self.xta,
                                       col_amax_ready=True)
            ev[5].record()
            f.fp8_grouped_gemm_ragged_k(self.dyt, f.E5M2, self.xt, f.E4M3, self.offsets, self.t, self.dyts, self.xts,
                                        self.dw)
            ev[6].record()
        else:
            f.fp8_quantize_rowcol(self.dy, f.E5M2, 0, self.qdy, self.sdy, self.ady, self.qdyt, self.sdyt, self.cady)
            ev[1].record()
            f.fp8_quantize_col(self.w, f.E4M3, 0, self.qwt, self.swt, self.caw, col_amax_ready=True)
            ev[2].record()
            f.fp8_gemm_scaled(self.qdy, f.E5M2, self.qwt, f.E4M3, self.sdy, f.SCALE_VECTOR, self.swt, f.SCALE_VECTOR,
                              self.dx)
            ev[3].record()
            f.fp8_quantize_col(self.x, f.E4M3, 0, self.qxt, self.sxt, self.cax, col_amax_ready=True)
            ev[4].record()
            f.fp8_gemm_scaled(self.qdyt, f.E5M2, self.qxt, f.E4M3, self.sdyt, f.SCALE_VECTOR, self.sxt,
                              f.SCALE_VECTOR, self.dw)
            ev[5].record()


def measured_traffic(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; otherwise None."""
    from fp8_scaled_gemm_amax_amd.profiling import source_digest
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        table = json.load(f)
    rec = table.get(kernel_key)
    if not rec or rec.get("source_digest") != source_digest(rec.get("sources", [])):
        return None
    return rec.get("bytes_per_launch")


COPY_BYTES = 1 << 30


def copy_calibration(args):
    """A plain copy kernel of known size for scaling the HBM byte counters:
    y = x * 1 over 2^28 fp32 values (reads and writes exactly COPY_BYTES each).
    Also prints the copy's own bandwidth, the practical HBM ceiling."""
    import torch
    n = COPY_BYTES // 4
    x = torch.rand(n, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(args.warmup):
        torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        torch.mul(x, 1.0, out=y)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    print(json.dumps({"calibration": "copy y = x * 1 (fp32)", "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                      "avg_ms": round(ms, 5), "gbps": round(2 * COPY_BYTES / (ms * 1e-3) / 1e9, 1),
                      "steps": args.steps}), flush=True)


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(sample, target_s, kind="rowwise"):
    """The CPU oracle on a bounded sample of the workload's own tensors: the
    first ms rows of the activation and the first ns rows of the weight
    (K-contiguous) quantized rowwise (kind "mx": MX block-32; "blockwise";
    "tensor": one scale per tensor, the delayed recipe's cast given the scale
    its state holds, here the tensor's current one), then the oracle's fp64
    dequantize-and-matmul of the sample. Reported as 2*ms*ns*K / time in
    TFLOP/s."""
    from oracle import oracle as orc
    act, fa, wgt, fw = sample
    k = act.shape[1]
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))

    def run(ms, ns):
        t0 = time.perf_counter()
        if kind == "mx":
            qx, sx = orc.mx_quantize_row(act[:ms], fa)
            qw, sw = orc.mx_quantize_row(wgt[:ns], fw)
            orc.mx_gemm(qx, fa, sx, qw, fw, sw)
        elif kind == "blockwise":
            qx, ex = orc.blockwise_quantize_act(act[:ms], fa)
            qw, ew = orc.blockwise_quantize_weight(wgt[:ns], fw)
            orc.blockwise_gemm(qx, fa, ex, qw, fw, ew)
        elif kind == "tensor":
            qx, sx, _ = orc.quantize_tensor_current(act[:ms], fa)
            qw, sw, _ = orc.quantize_tensor_current(wgt[:ns], fw)
            orc.gemm(qx, fa, qw, fw, sx, sw, with_bound=False)
        else:
            qx, sx, _ = orc.quantize_row(act[:ms], fa)
            qw, sw, _ = orc.quantize_row(wgt[:ns], fw)
            orc.gemm(qx, fa, qw, fw, sx, sw, with_bound=False)
        return time.perf_counter() - t0

    ms, ns = min(act.shape[0], 1024), min(wgt.shape[0], 512)
    t = run(ms, ns)
    if t < 0.5 * target_s:                 # scale the sample up to about target_s (weight rows first)
        pairs = ms * ns * target_s / t
        ns = int(min(wgt.shape[0], max(ns, pairs / ms)))
        ms = int(min(act.shape[0], max(ms, pairs / ns)))
        t = run(ms, ns)
    if t < 0.5 * target_s and ms < act.shape[0]:     # (per-row costs dominate: grow the activation rows)
        ms = int(min(act.shape[0], ms * target_s / t))
        t = run(ms, ns)
    return {"value": round(2.0 * ms * ns * k / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{ms} activation rows x {ns} weight rows x K={k} of the workload's tensors: "
                      f"{ {'mx': 'MX block-32', 'blockwise': 'blockwise', 'tensor': 'tensorwise'}.get(kind, 'rowwise') } quantize of both "
                      f"(oracle) + fp64 "
                      f"dequantize-and-matmul, {t:.1f} s on {threads} threads"}


def cpu_baseline_moe(w, target_s):
    """The oracle's MoE layer forward on the workload's first ts tokens (all
    their entries, every expert's weights quantized): route, permute + cast,
    gate|up grouped product, SwiGLU + cast, down grouped product, combine.
    Reported as 6 * (ts * topk) * hidden * inter / time in TFLOP/s."""
    from oracle import oracle as orc
    x, idx, wts, w1, w2 = w["x"], w["idx"], w["weights"], w["w1"], w["w2"]
    nexp, I2, H = w1.shape
    inter = I2 // 2
    k = idx.shape[1]
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))

    def run(ts):
        t0 = time.perf_counter()
        off, dest = orc.moe_route(idx[:ts], nexp)
        xq, xs = orc.moe_permute_quantize_row(x[:ts], dest, 0)
        w1q, w1s, _ = orc.quantize_row(w1.reshape(nexp * I2, H), 0)
        h, _ = orc.grouped_gemm(xq, 0, w1q.reshape(nexp, I2, H), 0, off, xs, w1s.reshape(nexp, I2))
        aq, asi, _ = orc.swiglu_quantize_row(orc.bf16_round(h), 0)
        w2q, w2s, _ = orc.quantize_row(w2.reshape(nexp * H, inter), 0)
        y, _ = orc.grouped_gemm(aq, 0, w2q.reshape(nexp, H, inter), 0, off, asi, w2s.reshape(nexp, H))
        orc.moe_unpermute_combine(orc.bf16_round(y), dest, wts[:ts])
        return time.perf_counter() - t0

    ts = 16
    t = run(ts)
    if t < 0.5 * target_s:
        ts = int(min(x.shape[0], ts * target_s / t))
        t = run(ts)
    return {"value": round(6.0 * ts * k * H * inter / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"the layer forward on the first {ts} tokens (x{k} expert entries) with all {nexp} experts' "
                      f"weights quantized, oracle steps incl. fp64 grouped products, {t:.1f} s on {threads} threads"}


def cold_leg(step, steps, wev):
    """Steps timed one at a time after a read of EVICT_BYTES, which pushes the
    inputs out of the 4 MB L2s and the 256 MB last-level cache: each step then
    starts from HBM as the first use of freshly loaded tensors would. A read
    leaves clean lines behind (a write of the same size leaves dirty ones,
    whose write-back the step's kernels would then pay for). The read is
    enqueued before the step's first event, so no kernel of the step is
    charged for it. Reports the median and minimum of each call and of the
    whole step over these steps."""
    import torch
    buf = torch.ones(EVICT_BYTES // 4, dtype=torch.float32, device="cuda:0")
    ncalls = len(step.calls)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(ncalls + 1)] for _ in range(steps)]
    for _ in range(3):                                   # code objects loaded, clocks up
        step.run(wev)
    for i in range(steps):
        buf.sum()
        step.run(ev[i])
    torch.cuda.synchronize()
    call_ms = np.array([[ev[i][c].elapsed_time(ev[i][c + 1]) for c in range(ncalls)] for i in range(steps)])
    step_ms = np.array([ev[i][0].elapsed_time(ev[i][ncalls]) for i in range(steps)])
    del buf
    return {"steps": steps, "evict_bytes": EVICT_BYTES,
            "ms_per_step_median": round(float(np.median(step_ms)), 5),
            "ms_per_step_min": round(float(step_ms.min()), 5),
            "value_median": round(step.flops / (float(np.median(step_ms)) * 1e-3) / 1e12, 2),
            "calls": [{"kernel": step.calls[c][0], "median_ms": round(float(np.median(call_ms[:, c])), 5),
                       "min_ms": round(float(call_ms[:, c].min()), 5)} for c in range(ncalls)]}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration(args)
        return
    step = Step(args.workload)
    ncalls = len(step.calls)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(ncalls + 1)] for _ in range(args.steps)]
    wev = [torch.cuda.Event(enable_timing=True) for _ in range(ncalls + 1)]
    # the cold-cache leg runs first, so the warm timed steps are the last calls
    # of every kernel in a trace of this process
    cold = cold_leg(step, args.cold_steps, wev) if args.cold_steps > 0 else None
    settle_steps, t_settle = 0, time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_seconds:
        for _ in range(10):
            step.run(wev)
        torch.cuda.synchronize()
        settle_steps += 10
    settle_s = time.perf_counter() - t_settle
    for _ in range(args.warmup):
        step.run(wev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step.run(ev[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per_call_ms = [float(np.mean([ev[i][c].elapsed_time(ev[i][c + 1]) for i in range(args.steps)]))
                   for c in range(ncalls)]
    ms_step = elapsed / args.steps * 1e3
    value = step.flops / (ms_step * 1e-3) / 1e12

    gemm_idx = [i for i, call in enumerate(step.calls) if "gemm" in call[0]]
    g = gemm_idx[0]
    gemm_flops = 2.0 * np.prod(step.mnk[0])
    gemm_tflops = gemm_flops / (per_call_ms[g] * 1e-3) / 1e12
    kernel_key = {"c4": "grouped_gemm", "c4b": "grouped_gemm", "c4mx": "grouped_gemm_mx",
                  "c6": "grouped_gemm", "c2bw": "gemm_mx"}.get(args.workload, "gemm")
    traffic = measured_traffic(f"{kernel_key}:{args.workload}")
    roofline = {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4), "traffic": traffic,
                "kernel": step.calls[g][0], "avg_ms": round(per_call_ms[g], 5),
                "flops_per_launch": gemm_flops}
    quant, other = [], []
    for i, call in enumerate(step.calls):
        nm, elems, nscales = call[:3]
        nbytes = float(call[3]) if len(call) > 3 else (3.0 * elems + 4.0 * nscales if elems else 0.0)
        if nbytes:
            gbps = nbytes / (per_call_ms[i] * 1e-3) / 1e9
            rec = {"kernel": nm, "avg_ms": round(per_call_ms[i], 5), "algorithmic_bytes": nbytes,
                   "gbps": round(gbps, 1), "frac_of_hbm": round(gbps / PEAK_HBM_GBPS, 4)}
            (quant if "quant" in nm else other).append(rec)
        elif "gemm" in nm and i != g:
            m, n, k = step.mnk[1]
            other.append({"kernel": nm, "avg_ms": round(per_call_ms[i], 5),
                          "tflops": round(2.0 * m * n * k / (per_call_ms[i] * 1e-3) / 1e12, 2)})
        elif i != g:
            other.append({"kernel": nm, "avg_ms": round(per_call_ms[i], 5)})
    m, n, k = step.mnk[0]
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3" if args.workload not in ("c4b", "c5") else "fp8_e5m2xe4m3",
        "data": "synthetic",
        "config": {"workload": step.desc, "m": m, "n": n, "k": k, **step.scales, "out": "bf16",
                   "flops_per_step": step.flops},
        "roofline": roofline, "quantizers": quant, "other_kernels": other, "cold": cold,
        "settle": {"seconds": round(settle_s, 3), "steps": settle_steps},
        **step.extra(),
        "cpu_baseline": None if args.no_cpu_baseline else (
            cpu_baseline_moe(step.cpu_sample, args.cpu_seconds) if getattr(step, "cpu_kind", "") == "moe_layer"
            else cpu_baseline(step.cpu_sample, args.cpu_seconds, getattr(step, "cpu_kind", "rowwise"))),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
