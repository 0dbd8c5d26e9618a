"""Benchmark of the residue-compensated NVFP4/MXFP4 linear on one MI355X.

A step is one pass of the whole hot path over one synthetic batch: activation
quantize + residue and the compensated linear, as the library's one-call entry
runs them (weights are prepacked once, offline, as the method prescribes):
the quantize kernel followed by the linear, or, for few rows to quantize, one
launch of the linear that quantizes its rows in every workgroup.  The headline
workload is the large-MLP projection: NVFP4, M = 8 token rows, K = 8192,
N = 28672, x in bf16 (the HBM-bound decode shape).  Steps rotate over distinct
weight copies (> 2x the 256 MB Infinity Cache) so every step streams its
weights from HBM, and are replayed from a HIP graph so host launch cost does
not enter the timing.  Every figure is the median of five timed replays of its
graph (the headline also gives their minimum and maximum); by default the
headline step is also timed in three fresh processes before this one starts,
with their median and spread.

Prints ONE JSON line.  Beside the headline: the roofline of its dominant
kernel (the linear) against the nominal 8 TB/s and against the streaming-read
rate of the same byte count measured with the library's read kernel, the
uncompensated (plain W4A4) step and the compensation overhead, per-kernel
averages, NMSE against the binary64 product of the bf16 activations and fp32
weights, the oracle timed on the host cores (one thread and all threads), and
a sweep over every workload (each with its NMSE, read ceiling and, from 64
rows, its fraction of the matrix-core peak); then selective compensation
(K-Ext) at rho = 0.125 / 0.25 / 0.5 on the prefill-sized operands, compensated
decode attention (ResAttn) at decode shapes of the page's Figure 10, and the
grouped (mixture of experts) linear.
"""
import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = {0: 2500.0, 1: 10100.0}   # dense: f16 (NVFP4 runs exact f16 products), FP4 (MXFP4)
ROTATE_BYTES = 512 << 20       # distinct weight bytes per timed loop (2x the MALL)

HEADLINE_M = 8                 # token rows of the headline (large-MLP shape)
METRIC = "compensated FP4 linear µs/call + HBM GB/s (% of peak) at M=1–8, K,N≥4096"

# HBM traffic of the dominant kernel (compensated NVFP4 linear at the headline
# shape), from rocprofv3 FETCH_SIZE / WRITE_SIZE passes over `bench.py
# --pmc-launches`, per launch, already multiplied by the copy-kernel
# calibration factors (FETCH_SIZE x2.0, WRITE_SIZE x1.0).  Valid only for the
# kernel sources whose hash is recorded; reported as null otherwise.
TRAFFIC = {
    "sources_sha256": "e54e314917d3683aae23ffaa095f514c7c41689daaa49c5cd8c7edcaf5ad3e73",
    "fetch_bytes": 132855467,     # 2.0 x 64,870.83 KiB (mean of three launches)
    "write_bytes": 917504,        # 1.0 x 896 KiB
}
KERNEL_SOURCES = ["gemm.hip", "layout.h", "codec.h", "fp4_frag.h", "quant_row.h", "kernels.h"]


def kernel_sources_sha256():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_scaled_fp4_act_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def blk(fmt):
    return 16 if fmt == 0 else 32


def gemm_bytes(fmt, M, N, K, comp):
    """Algorithmic bytes of one linear launch: packed weights (codes, block
    scales, NVFP4 tensor scale) + the activation records it reads + fp32 y."""
    B = 2 * M if comp else M
    w = N * K // 2 + N * K // blk(fmt) + (4 if fmt == 0 else 0)
    a = B * (K // 2 + K // blk(fmt) + (4 if fmt == 0 else 0))
    return w + a + M * N * 4


def quant_bytes(fmt, M, K, comp, x_elem):
    B = 2 * M if comp else M
    return M * K * x_elem + B * (K // 2 + K // blk(fmt) + (4 if fmt == 0 else 0))


def step_bytes(fmt, M, N, K, comp, x_elem):
    """Whole step: x read once, activation records written then read, packed
    weights read once, y written."""
    return quant_bytes(fmt, M, K, comp, x_elem) + gemm_bytes(fmt, M, N, K, comp)


class Setup:
    """Device buffers for one workload: R rotated weight copies and inputs."""

    def __init__(self, rs, torch, fmt, M, N, K, x_np, W_dev, bf16=True):
        self.rs, self.torch = rs, torch
        self.fmt, self.M, self.N, self.K = fmt, M, N, K
        blob = rs.prepack_weights(W_dev, fmt)
        wbytes = blob.numel()
        self.R = max(2, int(math.ceil(ROTATE_BYTES / wbytes)))
        self.blobs = [blob] + [blob.clone() for _ in range(self.R - 1)]
        x = torch.from_numpy(x_np).cuda()
        if bf16:
            x = x.to(torch.bfloat16)
        self.xs = [x.clone() for _ in range(self.R)]
        nb = rs.packed_act_bytes(fmt, M, K, True)
        self.acts = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(self.R)]
        self.ys = [torch.empty((M, N), dtype=torch.float32, device="cuda") for _ in range(self.R)]

    def quant(self, i, comp):
        r = i % self.R
        self.rs.quantize_act_with_residue(self.xs[r], self.fmt, comp, out=self.acts[r])

    def gemm(self, i, comp):
        r = i % self.R
        f = self.rs.fp4_linear_compensated if comp else self.rs.fp4_linear
        f(self.acts[r], self.blobs[r], self.M, self.N, self.K, self.fmt, out=self.ys[r])

    def two_launch(self, i, comp):
        self.quant(i, comp)
        self.gemm(i, comp)

    def step(self, i, comp):
        r = i % self.R
        self.rs.fp4_linear_from_x(self.xs[r], self.blobs[r], self.N, self.fmt, comp, out=self.ys[r],
                                  act=self.acts[r])


class KextSetup:
    """Selective compensation (K-Ext) buffers: masks from an on-device
    calibration pass, R rotated [W | W_S] blobs of width K_eff, inputs."""

    def __init__(self, rs, torch, fmt, M, N, K, k, x_np, W_dev, x_cal_np):
        self.rs, self.torch = rs, torch
        self.fmt, self.M, self.N, self.K, self.k = fmt, M, N, K, k
        self.KE = rs.kext_dim(K, k)
        xc = torch.from_numpy(x_cal_np).cuda().to(torch.bfloat16)
        self.masks = rs.kext_select(rs.channel_abs_sum(xc), k)
        blob = rs.prepack_weights_kext(W_dev, fmt, self.masks, k)
        self.R = max(2, int(math.ceil(ROTATE_BYTES / blob.numel())))
        self.blobs = [blob] + [blob.clone() for _ in range(self.R - 1)]
        x = torch.from_numpy(x_np).cuda().to(torch.bfloat16)
        self.xs = [x.clone() for _ in range(self.R)]
        nb = rs.packed_act_bytes(fmt, M, self.KE, False)
        self.acts = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(self.R)]
        self.ys = [torch.empty((M, N), dtype=torch.float32, device="cuda") for _ in range(self.R)]

    def quant(self, i):
        r = i % self.R
        self.rs.quantize_act_kext(self.xs[r], self.fmt, self.masks, self.k, out=self.acts[r])

    def gemm(self, i):
        r = i % self.R
        self.rs.fp4_linear(self.acts[r], self.blobs[r], self.M, self.N, self.KE, self.fmt, out=self.ys[r])

    def step(self, i):
        self.quant(i)
        self.gemm(i)


def run_kext(rs, torch, wl, M, ks, steps, warmup):
    """K-Ext steps (quantize + one plain product over K_eff) at each k in ks,
    beside the plain and full-residue steps of the same workload."""
    from block_scaled_fp4_act_amd import inputs
    fmt = 0 if wl.fmt == "nvfp4" else 1
    base, S, x = run_workload(rs, torch, wl, M, steps, warmup, want_plain=True, want_kernels=False,
                              want_nmse=False)
    del S
    torch.cuda.empty_cache()
    gen = torch.Generator(device="cuda").manual_seed(wl.w_seed)
    W_dev = torch.randn((wl.N, wl.K), generator=gen, device="cuda", dtype=torch.float32) * 0.02
    xcal = inputs.calibration_rows(wl)
    out = {"workload": wl.name, "format": wl.fmt, "M": M, "K": wl.K, "N": wl.N,
           "plain_us_per_call": round(base["plain_us_per_call"], 3),
           "full_us_per_call": round(base["us_per_call"], 3), "kext": []}
    for k in ks:
        S = KextSetup(rs, torch, fmt, M, wl.N, wl.K, k, x, W_dev, xcal)
        t = time_graph(torch, lambda i: S.step(i), steps, warmup)
        tg = time_graph(torch, lambda i: S.gemm(i), steps, warmup)
        tq = time_graph(torch, lambda i: S.quant(i), steps, warmup)
        out["kext"].append({
            "rho": k / 8.0, "K_eff": S.KE, "us_per_call": round(t * 1e3, 3), "gemm_us": round(tg * 1e3, 3),
            "quant_us": round(tq * 1e3, 3), "vs_plain": round(t * 1e3 / base["plain_us_per_call"], 4),
            "vs_full": round(t * 1e3 / base["us_per_call"], 4),
            "gemm_TFLOPs": round(2.0 * M * wl.N * S.KE / (tg * 1e-3) / 1e12, 2)})
        del S
        torch.cuda.empty_cache()
    del W_dev
    torch.cuda.empty_cache()
    return out


def paper_numerics_step(rs, torch, S, steps, warmup):
    """The headline step with the page's operator numerics: the tensor scale
    alpha computed once from the batch (calibration-like, outside the timing),
    the shared-alpha multiplier-scale quantizer and the compensated linear with
    bf16 output."""
    alpha = rs.nvfp4_tensor_alpha(S.xs[0])
    ys = [torch.empty((S.M, S.N), dtype=torch.bfloat16, device="cuda") for _ in range(S.R)]

    def quant(i):
        r = i % S.R
        rs.nvfp4_quantize_act_alpha(S.xs[r], alpha, True, out=S.acts[r])

    def step(i):
        r = i % S.R
        quant(i)
        rs.fp4_linear_compensated_bf16(S.acts[r], S.blobs[r], S.M, S.N, S.K, 0, out=ys[r])

    t = time_graph(torch, step, steps, warmup)
    tq = time_graph(torch, quant, steps, warmup)
    step(0)
    y = ys[0].double()
    e = float(((y - S.ref) ** 2).sum()) / float((S.ref * S.ref).sum())
    return {"us_per_call": round(t * 1e3, 3), "quant_us": round(tq * 1e3, 3),
            "nmse_comp_bf16": round(e, 6), "alpha": float(alpha.item()),
            "what": "shared tensor scale alpha, multiplier-scale quantizer, bf16 output"}


ATTN_CASES = [  # (name, H_q, H_kv, D, B, L): decode shapes of the page's Figure 10
    ("D128_GQA8", 64, 8, 128, 1, 8192), ("D128_GQA8", 64, 8, 128, 1, 32768), ("D128_GQA8", 64, 8, 128, 1, 131072),
    ("D128_GQA8", 64, 8, 128, 8, 8192), ("D128_GQA8", 64, 8, 128, 8, 32768), ("D128_GQA8", 64, 8, 128, 32, 8192),
    ("D128_GQA4", 32, 8, 128, 8, 32768), ("D256_GQA6", 24, 4, 256, 8, 32768),
]


GROUPED_CASES = [  # (format, experts, rows per expert, N, K): synthetic mixture-of-experts decode
    (0, 8, 2, 2048, 4096), (1, 8, 2, 2048, 4096), (0, 16, 1, 2048, 4096),
]


def run_grouped(rs, torch, case, steps, warmup):
    """Grouped (mixture of experts) compensated linear: E experts' stacked
    weights (N(0, 0.02^2), rotated over >= 512 MB so each step streams them
    from HBM), rows per expert of one quantized activation buffer; one launch
    beside E ordinary linear launches on the same data."""
    fmt, E, rows, N, K = case
    M_total = E * rows
    gen = torch.Generator(device="cuda").manual_seed(11)
    blobs = [rs.prepack_weights(torch.randn((N, K), generator=gen, device="cuda") * 0.02, fmt) for _ in range(E)]
    stacked = torch.cat(blobs)
    del blobs
    R = max(2, int(math.ceil(ROTATE_BYTES / stacked.numel())))
    stacks = [stacked] + [stacked.clone() for _ in range(R - 1)]
    stride = rs.packed_weight_bytes(fmt, N, K)
    x = (torch.randn((M_total, K), generator=gen, device="cuda")).to(torch.bfloat16)
    act = rs.quantize_act_with_residue(x, fmt, True)
    acts_e = [rs.quantize_act_with_residue(x[e * rows:(e + 1) * rows].contiguous(), fmt, True) for e in range(E)]
    offs = torch.arange(0, M_total + 1, rows, dtype=torch.int32, device="cuda")
    y = torch.zeros((M_total, N), dtype=torch.float32, device="cuda")
    ys = [y[e * rows:(e + 1) * rows] for e in range(E)]
    f = rs.fp4_linear_compensated

    def grouped(i):
        rs.fp4_grouped_linear(act, stacks[i % R], M_total, E, offs, rows, N, K, fmt, True, out=y)

    def separate(i):
        st = stacks[i % R]
        for e in range(E):
            f(acts_e[e], st[e * stride:(e + 1) * stride], rows, N, K, fmt, out=ys[e])

    t_g = time_graph(torch, grouped, steps, warmup)
    t_s = time_graph(torch, separate, steps, warmup)
    wbytes = E * (stride - 256)
    del stacks, stacked
    torch.cuda.empty_cache()
    return {"format": "nvfp4" if fmt == 0 else "mxfp4", "experts": E, "rows_per_expert": rows, "N": N, "K": K,
            "grouped_us": round(t_g * 1e3, 3), "separate_launches_us": round(t_s * 1e3, 3),
            "weights_GBps": round(wbytes / (t_g * 1e-3) / 1e9, 1),
            "weights_hbm_frac": round(wbytes / (t_g * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def attn_kv_bytes(B, L, H_kv, D):
    """K and V codes plus their block scales of every cached token read once."""
    return 2 * B * L * H_kv * (D // 2 + D // 16)


def run_attn(rs, torch, case, steps, warmup):
    """Decode attention step (query quantize + compensated attention over the
    paged NVFP4 cache), beside the plain-query step.  The cache is filled with
    random bytes (every byte decodes to a finite value); R disjoint copies of
    the sequences' pages rotate so each step reads its KV from HBM."""
    import math
    name, H_q, H_kv, D, B, L = case
    pb = rs.kv_page_bytes(H_kv, D)
    pages_per_seq = (L + 31) // 32
    step_bytes = B * pages_per_seq * pb
    R = max(2, int(math.ceil(ROTATE_BYTES / step_bytes)))
    total_pages = R * B * pages_per_seq
    g = torch.Generator(device="cuda").manual_seed(7)
    cache = torch.randint(0, 256, (total_pages * pb,), dtype=torch.uint8, device="cuda", generator=g)
    perm = torch.randperm(total_pages, device="cuda", generator=g).to(torch.int32)
    tables = [perm[r * B * pages_per_seq:(r + 1) * B * pages_per_seq].view(B, pages_per_seq).contiguous()
              for r in range(R)]
    seq = torch.full((B,), L, dtype=torch.int32, device="cuda")
    q = (torch.randn((B * H_q, D), device="cuda", generator=g)).to(torch.bfloat16)
    splits = rs.resattn_splits(B, H_kv, L)
    ws = torch.empty(max(1, int(rs.lib().rsfp4_resattn_workspace_bytes(B, H_q, D, splits))), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((B, H_q, D), dtype=torch.bfloat16, device="cuda")
    acts = {c: rs.quantize_act_with_residue(q, 0, c) for c in (True, False)}

    def step(i, comp):
        rs.quantize_act_with_residue(q, 0, comp, out=acts[comp])
        rs.resattn_decode(acts[comp], cache, tables[i % R], seq, L, B, H_q, H_kv, D, compensated=comp,
                          splits=splits, out=out, out_bf16=True, ws=ws)

    t_c = time_graph(torch, lambda i: step(i, True), steps, warmup)
    t_p = time_graph(torch, lambda i: step(i, False), steps, warmup)
    kvb = attn_kv_bytes(B, L, H_kv, D)
    del cache
    torch.cuda.empty_cache()
    return {"config": name, "B": B, "L": L, "H_q": H_q, "H_kv": H_kv, "D": D, "splits": splits,
            "us_per_call": round(t_c * 1e3, 3), "plain_us_per_call": round(t_p * 1e3, 3),
            "comp_overhead": round(t_c / t_p - 1.0, 4), "kv_GBps": round(kvb / (t_c * 1e-3) / 1e9, 1),
            "kv_hbm_frac": round(kvb / (t_c * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


REPLAYS = 5


def time_graph(torch, fn, steps, warmup, stats=None):
    """Run `warmup` eager iterations, capture `steps` iterations in one HIP
    graph, replay it once untimed, then time REPLAYS replays, each with HIP
    events on the capturing stream.  Returns the median ms per iteration; with
    `stats` (a dict), also the minimum and maximum over the replays."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                fn(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(REPLAYS)]
    with torch.cuda.stream(s):
        for e0, e1 in ev:
            e0.record(s)
            g.replay()
            e1.record(s)
    torch.cuda.synchronize()
    per = sorted(e0.elapsed_time(e1) / steps for e0, e1 in ev)
    if stats is not None:
        stats.update(min=per[0], max=per[-1], replays=REPLAYS)
    return per[len(per) // 2]


_READ_PEAK = {}


def read_peak_gbps(rs, torch, nbytes, steps=20, warmup=3):
    """Streaming-read rate (GB/s) of the library's read kernel at a byte
    count, over rotated buffers (>= 512 MB in all) as the linear's weights."""
    if nbytes in _READ_PEAK:
        return _READ_PEAK[nbytes]
    nb = (nbytes + 255) // 256 * 256
    nread = (nbytes + 15) // 16 * 16       # the kernel reads whole 16-byte groups
    R = max(2, int(math.ceil(ROTATE_BYTES / nb)))
    buf = torch.empty(R * nb, dtype=torch.uint8, device="cuda")
    buf.fill_(0x5A)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    parts = [buf[r * nb: r * nb + nread] for r in range(R)]
    t = time_graph(torch, lambda i: rs.stream_read(parts[i % R], sink), steps, warmup)
    del buf, parts
    torch.cuda.empty_cache()
    _READ_PEAK[nbytes] = nread / (t * 1e-3) / 1e9
    return _READ_PEAK[nbytes]


def weight_bytes(fmt, N, K):
    return N * K // 2 + N * K // blk(fmt) + (4 if fmt == 0 else 0)


def run_workload(rs, torch, wl, M, steps, warmup, want_plain=True, want_kernels=True, want_nmse=True):
    """One workload at M rows: the whole step (one call from x), the linear and
    the quantizer alone, the plain step, NMSE against the binary64 product of
    the (bf16) activations and the fp32 weights, the streaming-read rate at
    the weight bytes and, from 64 rows, the linear's fraction of the matrix-
    core peak.  W ~ N(0, 0.02^2) is drawn on the device (seeded)."""
    fmt = 0 if wl.fmt == "nvfp4" else 1
    wlm = wl.with_m(M)
    x = wlm.draw_x()
    gen = torch.Generator(device="cuda").manual_seed(wl.w_seed)
    W_dev = torch.randn((wl.N, wl.K), generator=gen, device="cuda", dtype=torch.float32) * 0.02
    S = Setup(rs, torch, fmt, M, wl.N, wl.K, x, W_dev, bf16=wl.bf16)
    nm = {}
    if want_nmse:
        xd = S.xs[0].double()
        ref = xd @ W_dev.double().T
        den = float((ref * ref).sum())
        for comp in (True, False):
            rs.quantize_act_with_residue(S.xs[0], fmt, comp, out=S.acts[0])
            f = rs.fp4_linear_compensated if comp else rs.fp4_linear
            y = f(S.acts[0], S.blobs[0], M, wl.N, wl.K, fmt).double()
            nm["nmse_comp" if comp else "nmse_plain"] = float(((y - ref) ** 2).sum()) / den
        S.ref = ref
        del xd, y
    del W_dev
    out = {"workload": wl.name, "format": wl.fmt, "M": M, "K": wl.K, "N": wl.N, "rotation": S.R}
    sb = step_bytes(fmt, M, wl.N, wl.K, True, 2 if wl.bf16 else 4)
    st = {}
    t_comp = time_graph(torch, lambda i: S.step(i, True), steps, warmup, stats=st)
    out["us_per_call"] = t_comp * 1e3
    out["us_per_call_replay_spread"] = [round(st["min"] * 1e3, 3), round(st["max"] * 1e3, 3)]
    out["GBps"] = sb / (t_comp * 1e-3) / 1e9
    out["launches"] = rs.from_x_launches(fmt, M, wl.N, wl.K, True)
    if out["launches"] == 1:   # the two-launch step beside the one-launch one
        out["two_launch_us_per_call"] = time_graph(torch, lambda i: S.two_launch(i, True), steps, warmup) * 1e3
    if want_kernels:
        t_g = time_graph(torch, lambda i: S.gemm(i, True), steps, warmup)
        t_q = time_graph(torch, lambda i: S.quant(i, True), steps, warmup)
        gb = gemm_bytes(fmt, M, wl.N, wl.K, True)
        out["gemm_us"] = t_g * 1e3
        out["quant_us"] = t_q * 1e3
        out["gemm_GBps"] = gb / (t_g * 1e-3) / 1e9
        out["gemm_hbm_frac"] = out["gemm_GBps"] / HBM_PEAK_GBS
        out["gemm_TFLOPs"] = 2.0 * 2 * M * wl.N * wl.K / (t_g * 1e-3) / 1e12
    if want_plain:
        t_plain = time_graph(torch, lambda i: S.step(i, False), steps, warmup)
        out["plain_us_per_call"] = t_plain * 1e3
        out["comp_overhead"] = t_comp / t_plain - 1.0
        out["plain_launches"] = rs.from_x_launches(fmt, M, wl.N, wl.K, False)
        if out["plain_launches"] != out["launches"]:
            # the same two-launch form on both sides (quantizer + linear)
            t_c2 = out.get("two_launch_us_per_call", t_comp * 1e3) * 1e-3
            t_p2 = time_graph(torch, lambda i: S.two_launch(i, False), steps, warmup)
            out["plain_two_launch_us_per_call"] = t_p2 * 1e3
            out["comp_overhead_two_launch"] = t_c2 / t_p2 - 1.0
        if want_kernels:
            t_gp = time_graph(torch, lambda i: S.gemm(i, False), steps, warmup)
            out["plain_gemm_us"] = t_gp * 1e3
    out["step_GBps_frac"] = out["GBps"] / HBM_PEAK_GBS
    out.update(nm)
    if want_kernels:
        rp = read_peak_gbps(rs, torch, weight_bytes(fmt, wl.N, wl.K))
        out["read_peak_GBps"] = rp
        out["gemm_frac_of_read_peak"] = out["gemm_GBps"] / rp
        if M >= 64:
            out["mfma_frac"] = out["gemm_TFLOPs"] / MFMA_PEAK_TFLOPS[fmt]
            out["mfma_peak_TFLOPs"] = MFMA_PEAK_TFLOPS[fmt]
    return out, S, x


def host_info():
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu": model, "nproc": os.cpu_count()}


def pmc_launches(rs, torch):
    """Eager launches for hardware-counter passes (no graphs): a 256 MiB device
    copy three times (calibration: known bytes read and written), then, for
    each narrow workload (the attention projection, the MLP pair, the
    large-MLP shape and the MXFP4 shape, all compensated, M = 4 or 8), three
    quantize launches and three linear launches over distinct weight copies.
    Each case prints its algorithmic bytes before its launches."""
    from block_scaled_fp4_act_amd import inputs
    a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    print(json.dumps({"pmc_launches": "copy", "copy_bytes": 256 << 20, "launches": 3}), flush=True)
    cases = [(inputs.ATTN, inputs.ATTN.M), (inputs.MLP_UP, 8), (inputs.MLP_DOWN, 8),
             (inputs.LARGE_MLP, HEADLINE_M), (inputs.MX, 8)]
    for wl, M in cases:
        fmt = 0 if wl.fmt == "nvfp4" else 1
        gen = torch.Generator(device="cuda").manual_seed(wl.w_seed)
        W_dev = torch.randn((wl.N, wl.K), generator=gen, device="cuda", dtype=torch.float32) * 0.02
        S = Setup(rs, torch, fmt, M, wl.N, wl.K, wl.with_m(M).draw_x(), W_dev, bf16=wl.bf16)
        del W_dev
        torch.cuda.synchronize()
        print(json.dumps({"pmc_launches": wl.name, "M": M, "format": wl.fmt, "launches": "3 quantize, 3 linear",
                          "linear_algorithmic_bytes": gemm_bytes(fmt, M, wl.N, wl.K, True)}), flush=True)
        for i in range(3):
            S.quant(i, True)
        torch.cuda.synchronize()
        for i in range(3):
            S.gemm(i, True)
        torch.cuda.synchronize()
        del S
        torch.cuda.empty_cache()


def pmc_paths(rs, torch):
    """Eager launches for counter passes over every kernel path: the narrow
    linear at the headline and the large-MLP shape (M = 8), the tiled linear
    at the large-MLP shape (M = 128, NVFP4) and the MXFP4 shape (M = 256), all
    compensated, then decode attention (D = 128, GQA 8, B = 8, 32K tokens);
    three launches each, over distinct weight copies or cache pages."""
    from block_scaled_fp4_act_amd import inputs
    cases = [(inputs.ATTN, inputs.ATTN.M), (inputs.LARGE_MLP, 8), (inputs.LARGE_MLP, 128), (inputs.MX, 256)]
    for wl, M in cases:
        fmt = 0 if wl.fmt == "nvfp4" else 1
        gen = torch.Generator(device="cuda").manual_seed(wl.w_seed)
        W_dev = torch.randn((wl.N, wl.K), generator=gen, device="cuda", dtype=torch.float32) * 0.02
        S = Setup(rs, torch, fmt, M, wl.N, wl.K, wl.with_m(M).draw_x(), W_dev)
        del W_dev
        for i in range(3):
            S.quant(i, True)
        torch.cuda.synchronize()
        for i in range(3):
            S.gemm(i, True)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_paths": wl.name, "M": M, "format": wl.fmt,
                          "linear_algorithmic_bytes": gemm_bytes(fmt, M, wl.N, wl.K, True),
                          "linear_flops": 2 * 2 * M * wl.N * wl.K}), flush=True)
        del S
        torch.cuda.empty_cache()
    name, H_q, H_kv, D, B, L = ATTN_CASES[4]
    pb = rs.kv_page_bytes(H_kv, D)
    npg = (L + 31) // 32
    g = torch.Generator(device="cuda").manual_seed(7)
    cache = torch.randint(0, 256, (3 * B * npg * pb,), dtype=torch.uint8, device="cuda", generator=g)
    perm = torch.randperm(3 * B * npg, device="cuda", generator=g).to(torch.int32)
    seq = torch.full((B,), L, dtype=torch.int32, device="cuda")
    q = torch.randn((B * H_q, D), device="cuda", generator=g).to(torch.bfloat16)
    act = rs.quantize_act_with_residue(q, 0, True)
    out = torch.empty((B, H_q, D), dtype=torch.bfloat16, device="cuda")
    for r in range(3):
        table = perm[r * B * npg:(r + 1) * B * npg].view(B, npg).contiguous()
        rs.resattn_decode(act, cache, table, seq, L, B, H_q, H_kv, D, compensated=True, out=out, out_bf16=True)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_paths": "resattn " + name, "B": B, "L": L, "kv_bytes": attn_kv_bytes(B, L, H_kv, D)}),
          flush=True)


GCC_FLAGS = "gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math (-fopenmp for the all-threads build)"
CPU_SLICE = 1024        # output channels of the one-thread sample (extrapolated to N)


def _cpu_call_time(oracle, x, dw, fmt, M, comp, threads, min_s=0.5, max_calls=50):
    """Median seconds of the oracle's two parts of one call -- quantize the
    rows, then the compensated linear over the pre-quantized weights dw --
    over repeated calls.  Returns (quantize s, linear s, calls)."""
    tq, tl = [], []
    t_all = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        q = oracle.quantize_act(x, fmt, comp)
        t1 = time.perf_counter()
        oracle.linear(q["deq"], dw, M, comp, want_beta=False, threads=threads)
        tq.append(t1 - t0)
        tl.append(time.perf_counter() - t1)
        if (time.perf_counter() - t_all >= min_s and len(tq) >= 3) or len(tq) >= max_calls:
            break
    tq.sort()
    tl.sort()
    return tq[len(tq) // 2], tl[len(tl) // 2], len(tq)


def cpu_baseline(cases):
    """The oracle (plain C, binary64 accumulation, -O2 without contraction)
    timed on the host: activation quantize + compensated linear per call,
    weights quantized beforehand as on the GPU.  Two legs per workload: all
    threads of the OpenMP timing build (the full call where M <= 8; else the
    quantize in full and the linear over a CPU_SLICE-channel slice, scaled to
    N), and one thread (the quantize in full and the linear over the slice,
    scaled to N).  cases: [(workload, [M, ...])].  Returns the per-workload
    table and the seconds it took."""
    import oracle
    from block_scaled_fp4_act_amd import inputs
    oracle.build()
    nthr = oracle.threads()
    rows = []
    t_start = time.perf_counter()
    for wl, ms in cases:
        fmt = 0 if wl.fmt == "nvfp4" else 1
        W = inputs.weights(wl.N, wl.K, wl.w_seed)
        sl = np.arange(min(CPU_SLICE, wl.N))
        full_needed = any(m <= 8 for m in ms)
        w = oracle.quantize_weight(W, fmt, rows=None if full_needed else sl, threads=True)
        del W
        dw_all = w["deq"] if full_needed else None
        dw_sl = np.ascontiguousarray(w["deq"][sl]) if full_needed else w["deq"]
        del w
        x_all = wl.with_m(max(ms)).draw_x()
        for M in ms:
            x = np.ascontiguousarray(x_all[:M])
            if M <= 8:
                q_all, l_all, n_all = _cpu_call_time(oracle, x, dw_all, fmt, M, True, True)
                t_all = q_all + l_all
                all_label = "full call"
            else:
                q_all, l_sl, n_all = _cpu_call_time(oracle, x, dw_sl, fmt, M, True, True)
                t_all = q_all + l_sl * wl.N / len(sl)
                all_label = f"quantize in full, linear over {len(sl)} channels extrapolated to N = {wl.N}"
            q_one, l_one, n_one = _cpu_call_time(oracle, x, dw_sl, fmt, M, True, False, min_s=0.3, max_calls=10)
            t_one = q_one + l_one * wl.N / len(sl)
            sb = step_bytes(fmt, M, wl.N, wl.K, True, 2 if wl.bf16 else 4)
            rows.append({"workload": wl.name, "format": wl.fmt, "M": M, "K": wl.K, "N": wl.N,
                         "all_threads": {"us_per_call": round(t_all * 1e6, 1), "GBps": round(sb / t_all / 1e9, 4),
                                         "threads": nthr, "sample": f"{all_label}, median of {n_all} calls"},
                         "one_thread": {"us_per_call": round(t_one * 1e6, 1), "GBps": round(sb / t_one / 1e9, 4),
                                        "threads": 1, "sample": f"quantize in full, linear over {len(sl)} channels "
                                                                f"extrapolated to N = {wl.N}, median of {n_one} "
                                                                "calls"}})
            print(f"oracle timing {wl.name} M={M}: {t_all * 1e6:.0f} us ({nthr} threads), "
                  f"{t_one * 1e6:.0f} us (1 thread)", file=sys.stderr, flush=True)
        del dw_all, dw_sl
    return rows, time.perf_counter() - t_start


def cross_process(n, steps, warmup):
    """The headline step measured again in n fresh processes, one after the
    other (started before this process touches the GPU): their per-call
    medians, the median across them and the spread."""
    import statistics
    import subprocess
    vals = []
    for k in range(n):
        cmd = [sys.executable, "-u", os.path.abspath(__file__), "--only-headline", "--no-cpu-baseline",
               "--processes", "1", "--steps", str(steps), "--warmup", str(warmup)]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        if r.returncode != 0:
            raise RuntimeError(f"headline process {k} failed ({r.returncode}): {r.stderr[-2000:]}")
        line = [ln for ln in r.stdout.splitlines() if ln.startswith("{")][-1]
        vals.append(json.loads(line)["us_per_call"])
        print(f"headline process {k + 1}/{n}: {vals[-1]:.3f} us per call", file=sys.stderr, flush=True)
    return {"processes": n, "us_per_call": vals, "median_us": round(statistics.median(vals), 3),
            "min_us": round(min(vals), 3), "max_us": round(max(vals), 3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-headline", action="store_true", help="skip plain/kernels/sweep (profiling runs)")
    ap.add_argument("--pmc-launches", action="store_true",
                    help="only eager launches for counter passes (copy calibration + headline linear)")
    ap.add_argument("--pmc-paths", action="store_true",
                    help="only eager launches of every kernel path for counter passes")
    ap.add_argument("--processes", type=int, default=3,
                    help="also time the headline step in this many fresh processes (1: only this one)")
    ap.add_argument("--cases", default=None,
                    help="only these sweep cases, e.g. 'large_mlp:128,mx:256' (no headline, no oracle timing)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path is single-GPU; see the design notes for how it shards)", file=sys.stderr)
        sys.exit(2)

    procs = None
    if args.processes > 1 and not (args.pmc_launches or args.pmc_paths or args.cases or args.only_headline):
        procs = cross_process(args.processes, args.steps, args.warmup)

    import torch
    import block_scaled_fp4_act_amd as rs
    from block_scaled_fp4_act_amd import inputs
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    rs.lib()
    if args.pmc_launches:
        pmc_launches(rs, torch)
        return
    if args.pmc_paths:
        pmc_paths(rs, torch)
        return
    if args.cases:
        named = {"attn": inputs.ATTN, "mlp_up": inputs.MLP_UP, "mlp_down": inputs.MLP_DOWN,
                 "large_mlp": inputs.LARGE_MLP, "mx": inputs.MX, "small": inputs.SMALL}
        for item in args.cases.split(","):
            parts = item.split(":")
            if parts[0] == "grouped":   # grouped:<index into GROUPED_CASES> or grouped:all
                idx = range(len(GROUPED_CASES)) if parts[1] == "all" else [int(parts[1])]
                for ci in idx:
                    print(json.dumps(run_grouped(rs, torch, GROUPED_CASES[ci], min(args.steps, 100),
                                                 min(args.warmup, 10))), flush=True)
                continue
            if parts[0] == "resattn":   # resattn:<index into ATTN_CASES> or resattn:all
                idx = range(len(ATTN_CASES)) if parts[1] == "all" else [int(parts[1])]
                for ci in idx:
                    print(json.dumps(run_attn(rs, torch, ATTN_CASES[ci], min(args.steps, 50), min(args.warmup, 5))),
                          flush=True)
                continue
            name, m = parts[0], int(parts[1])
            if len(parts) > 2:      # name:M:k1/k2/..  -> selective compensation at those k
                ks = [int(v) for v in parts[2].split("/")]
                r = run_kext(rs, torch, named[name], m, ks, min(args.steps, 100), min(args.warmup, 10))
                print(json.dumps(r), flush=True)
                continue
            r, S2, _ = run_workload(rs, torch, named[name], m, min(args.steps, 100), min(args.warmup, 10))
            del S2
            torch.cuda.empty_cache()
            print(json.dumps({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}), flush=True)
        return

    wl = inputs.LARGE_MLP.with_m(HEADLINE_M)
    fmt = 0
    lite = args.only_headline
    head, S, x = run_workload(rs, torch, wl, wl.M, args.steps, args.warmup,
                              want_plain=not lite, want_kernels=not lite, want_nmse=not lite)
    if not lite:
        head["paper_numerics"] = paper_numerics_step(rs, torch, S, args.steps, args.warmup)
    del S
    torch.cuda.empty_cache()

    # roofline of the dominant kernel of the step: the compensated linear
    roof = None
    if "gemm_us" in head:
        gb = gemm_bytes(fmt, wl.M, wl.N, wl.K, True)
        ach = gb / (head["gemm_us"] * 1e-6) / 1e9
        traffic = None
        if TRAFFIC["sources_sha256"] is not None and TRAFFIC["sources_sha256"] == kernel_sources_sha256():
            traffic = TRAFFIC["fetch_bytes"] + TRAFFIC["write_bytes"]
        rp = head["read_peak_GBps"]
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "gemm_small_kernel (compensated NVFP4 linear)",
                "algorithmic_bytes_per_launch": gb,
                "measured_read_peak": round(rp, 1),
                "measured_read_peak_by": (f"stream_read_kernel over {weight_bytes(fmt, wl.N, wl.K)} bytes "
                                          "(the weight bytes), rotated buffers, HIP graph"),
                "frac_of_measured_read_peak": round(ach / rp, 4)}

    sweep, grouped, kext, attn = [], [], [], []
    if not args.no_sweep and not lite:
        cases = [(inputs.SMALL, 1), (inputs.ATTN, inputs.ATTN.M), (inputs.MLP_UP, 8), (inputs.MLP_DOWN, 8)]
        cases += [(inputs.LARGE_MLP, m) for m in inputs.LARGE_MLP_M]
        cases += [(inputs.MX, m) for m in inputs.MX_M]
        for w, m in cases:
            if w is inputs.LARGE_MLP and m == HEADLINE_M:
                r = head
            else:
                r, S2, _ = run_workload(rs, torch, w, m, min(args.steps, 100), min(args.warmup, 10))
                del S2
                torch.cuda.empty_cache()
            sweep.append({k: (round(v, 6) if isinstance(v, float) else v) for k, v in r.items()
                          if k != "paper_numerics"})
            print(f"sweep {w.name} M={m}: {r['us_per_call']:.2f} us", file=sys.stderr, flush=True)
        attn = [run_attn(rs, torch, c, min(args.steps, 50), min(args.warmup, 5)) for c in ATTN_CASES]
        grouped = [run_grouped(rs, torch, c, min(args.steps, 100), min(args.warmup, 10)) for c in GROUPED_CASES]
        # selective compensation (prefill-sized operands): rho = 0.125, 0.25, 0.5
        for w, m in ((inputs.LARGE_MLP, 128), (inputs.MX, 256)):
            kext.append(run_kext(rs, torch, w, m, inputs.KEXT_K, min(args.steps, 100), min(args.warmup, 10)))

    cpu = None
    if not args.no_cpu_baseline:
        cases = [(wl, [HEADLINE_M])]
        if not args.no_sweep and not lite:
            cases = [(inputs.SMALL, [1]), (inputs.ATTN, [inputs.ATTN.M]), (inputs.MLP_UP, [8]),
                     (inputs.MLP_DOWN, [8]), (inputs.LARGE_MLP, list(inputs.LARGE_MLP_M)),
                     (inputs.MX, list(inputs.MX_M))]
        table, secs = cpu_baseline(cases)
        hrow = [r for r in table if r["workload"] == wl.name and r["M"] == HEADLINE_M][0]
        cpu = {"value": hrow["all_threads"]["GBps"], "unit": "GB/s", "cores": hrow["all_threads"]["threads"],
               "kind": "oracle",
               "sample": (f"{wl.name} M={HEADLINE_M}: {hrow['all_threads']['sample']} (activation quantize + "
                          "compensated linear over pre-quantized weights), OpenMP timing build"),
               "us_per_call": hrow["all_threads"]["us_per_call"],
               "one_thread": hrow["one_thread"],
               "host": host_info(), "gcc": GCC_FLAGS,
               "per_workload": table, "seconds": round(secs, 1)}

    line = {
        "metric": METRIC,
        "value": round(head["GBps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["us_per_call"] / 1e3,
        "us_per_call": round(head["us_per_call"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4-e2m1/f32-acc",
        "data": "synthetic",
        "config": {"workload": wl.name, "format": "nvfp4", "M": wl.M, "K": wl.K, "N": wl.N,
                   "compensated": True, "x_dtype": "bf16", "w": "N(0,0.02^2) fp32, prepacked",
                   "timing": f"HIP graph of {args.steps} steps over {head['rotation']} rotated weight copies",
                   "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    line["us_per_call_replay_spread"] = head["us_per_call_replay_spread"]
    line["replays"] = REPLAYS
    if procs is not None:
        line["headline_processes"] = procs
    for k in ("launches", "plain_launches", "plain_us_per_call", "comp_overhead", "plain_two_launch_us_per_call",
              "comp_overhead_two_launch", "gemm_us", "plain_gemm_us", "quant_us", "gemm_GBps",
              "read_peak_GBps", "gemm_frac_of_read_peak", "nmse_comp", "nmse_plain", "paper_numerics"):
        if k in head:
            line[k] = round(head[k], 6) if isinstance(head[k], float) else head[k]
    line["step_hbm_frac"] = round(head["GBps"] / HBM_PEAK_GBS, 4)
    if sweep:
        line["sweep"] = sweep
        line["kext"] = kext
        line["attention"] = attn
        line["grouped"] = grouped
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
