#!/usr/bin/env python3
"""Benchmark of the QLoRA hot path on one MI355X.

Timed step (the headline number): one pass of the whole path over the
LLaMA-7B MLP pair at M = 4096 tokens, r = 64 --
  for the up-projection (4096 -> 11008) and the down-projection (11008 -> 4096):
  NF4 encode + double quantization of the frozen weight, forward, backward
  (dX, dL1, dL2).
value = algorithmic fwd+bwd FLOPs of both linears (4MKN + 6Mr(K+N) each; the
encode adds no FLOPs) / time per step, in TFLOP/s.

Also reported (not part of `value`):
  * per-kernel roofline of the fused quantized GEMMs (forward and dX), timed with
    HIP events on the stream they run on;
  * decode: packed-weight GB/s of the M = 1 forward kernel at 4096 -> 11008,
    rotating over 24 copies of the packed layer (> 512 MB) so that every call
    streams from HBM rather than the 256 MB Infinity Cache; M = 4 and 16 too;
    and the rate of a plain streaming read of the same number of bytes (the
    read ceiling the packed-weight rate is also compared with);
  * encode throughput over the 7 linears of one LLaMA-65B block (809.5 M weights);
  * the CPU oracle timed on a bounded sample of the headline step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "qlora_linear fwd+bwd TFLOP/s at M=4096; packed-weight HBM GB/s at M=1"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--step-only", action="store_true",
                    help="only the timed headline steps (for kernel traces of the step)")
    ap.add_argument("--roofline-only", action="store_true",
                    help="only the per-kernel roofline timings (fused GEMMs and the decode forward), printed as "
                         "one JSON line: the run that the committed kernel trace profiles")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="only launch each fused GEMM a few times on the headline shapes, then a plain "
                         "512 MiB device copy (the reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


def layer_flops(M, K, N, r):
    return 4 * M * K * N + 6 * M * r * (K + N)


class Linear:
    """Device buffers of one linear: weights, adapters, activations and outputs,
    all allocated before timing so the timed region allocates nothing."""

    def __init__(self, inp, dev):
        import torch
        import bit_quantized_lora_blockwise_amd as q
        self.q = q
        self.W = inp["W"].to(dev)
        self.N, self.K = self.W.shape
        self.X, self.L1, self.L2, self.dY = (inp[k].to(dev) for k in ("X", "L1", "L2", "dY"))
        self.M = self.X.shape[0]
        self.r = self.L1.shape[1]
        E = self.N * self.K
        u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
        self.codes = torch.empty((self.N, self.K // 2), dtype=u8, device=dev)
        self.absmax = torch.empty((E // 64,), dtype=f32, device=dev)
        self.c2 = torch.empty((E // 64,), dtype=u8, device=dev)
        self.c1 = torch.empty(((E // 64 + 255) // 256,), dtype=f32, device=dev)
        self.Y = torch.empty((self.M, self.N), dtype=bf, device=dev)
        self.T = torch.empty((self.M, self.r), dtype=bf, device=dev)
        self.G = torch.empty((self.M, self.r), dtype=bf, device=dev)
        self.dX = torch.empty((self.M, self.K), dtype=bf, device=dev)
        self.dL1 = torch.empty((self.K, self.r), dtype=f32, device=dev)
        self.dL2 = torch.empty((self.r, self.N), dtype=f32, device=dev)
        self.ws_f = torch.empty((max(16, q.qlora_linear_fwd_workspace(self.M, self.K, self.N, self.r)),),
                                dtype=u8, device=dev)
        self.ws_b = torch.empty((max(16, q.qlora_linear_bwd_workspace(self.M, self.K, self.N, self.r)),),
                                dtype=u8, device=dev)

    def encode(self):
        self.q.nf4_quantize_dq(self.W, codes=self.codes, c2=self.c2, c1=self.c1)

    def forward(self):
        self.q.qlora_linear_fwd(self.X, self.codes, self.c2, self.c1, self.N, self.L1, self.L2, 1.0, Y=self.Y,
                                T_out=self.T, workspace=self.ws_f)

    def backward(self):
        self.q.qlora_linear_bwd(self.X, self.dY, self.codes, self.c2, self.c1, self.L1, self.L2, 1.0, T=self.T,
                                dX=self.dX, dL1=self.dL1, dL2=self.dL2, workspace=self.ws_b)

    def step(self):
        self.encode()
        self.forward()
        self.backward()

    def flops(self):
        return layer_flops(self.M, self.K, self.N, self.r)


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "traffic_qgemm_llama7b_m4096.md")
GEMM_SOURCE = os.path.join(ROOT, "bit_quantized_lora_blockwise_amd", "csrc", "gemm_big.hip")
DECODE_SOURCE = os.path.join(ROOT, "bit_quantized_lora_blockwise_amd", "csrc", "decode.hip")


def code_digest(path):
    """sha256 of a source file with its comments and white space taken out: the
    digest changes with the code, not with its comments or layout."""
    import hashlib
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


def recorded_traffic(kernel, source=GEMM_SOURCE):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE / WRITE_SIZE
    summary, or None when the kernel's source code has changed since those
    counters were taken (the summary records each source's code digest)."""
    try:
        text = open(TRAFFIC_PROFILE).read()
        digest = code_digest(source)
    except OSError:
        return None
    if f"{os.path.basename(source)} code sha256 {digest}" not in text:
        return None
    for line in text.splitlines():
        parts = line.split()
        if len(parts) == 3 and parts[0] == "traffic_bytes_per_launch" and parts[1] == kernel:
            return float(parts[2])
    return None


def time_launches(fn, reps):
    """Average duration (ms) of `fn` over `reps` back-to-back calls, HIP events on the current stream."""
    import torch
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def time_queued_launches(fn, calls, reps=3):
    """Average duration (ms) of one `fn` call on the GPU when `calls` calls are
    issued one by one behind a long GPU job on the same stream (so the host has
    queued them all before the GPU reaches the first): HIP events around the
    calls only, best of `reps`."""
    import torch
    dev = torch.cuda.current_device()
    big = torch.randn((8192, 8192), dtype=torch.bfloat16, device=dev)
    fn()
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(1 + calls // 16):            # a few ms of GEMMs ahead of the calls
            torch.mm(big, big)
        a.record()
        for _ in range(calls):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / calls
        best = ms if best is None else min(best, ms)
    del big
    return best


def time_graph_launches(fn, calls, reps):
    """Average duration (ms) of one `fn` call when `calls` calls are captured in
    a HIP graph and the graph is replayed `reps` times (HIP events on the
    current stream): back-to-back launches without the host in between."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) / (reps * calls)


def kernel_rooflines(lins, reps, warm_launches=60):
    """Fused forward GEMM and fused dX GEMM, each launched alone (stage entry
    points).  The core clock settles over the first tens of milliseconds of
    sustained MFMA work, so `warm_launches` launches of both kernels run first;
    then each shape alone and both shapes back to back are timed with HIP
    events (avg_ms: the back-to-back average per launch)."""
    q = lins[0].q
    out = {}
    for L in lins:
        q.qlora_lora_grad_in(L.dY, L.L2, 1.0, G=L.G)
    fwd_fns = [lambda L=L: q.qlora_linear_fwd_t(L.X, L.codes, L.c2, L.c1, L.N, L.T, L.L2, 1.0, Y=L.Y)
               for L in lins]
    dx_fns = [lambda L=L: q.qlora_linear_dx(L.dY, L.codes, L.c2, L.c1, L.K, L.G, L.L1, dX=L.dX) for L in lins]

    def both(fns):
        def run():
            for f in fns:
                f()
        return run

    for _ in range(warm_launches // (2 * len(lins))):
        both(fwd_fns)()
        both(dx_fns)()
    for name, fns, flops in (
            ("k_qgemm_fwd", fwd_fns, [2 * L.M * L.K * L.N + 2 * L.M * L.r * L.N for L in lins]),
            ("k_qgemm_dx", dx_fns, [2 * L.M * L.K * L.N + 2 * L.M * L.r * L.K for L in lins])):
        per_shape = {}
        for L, f, fl in zip(lins, fns, flops):
            sms = time_launches(f, reps)
            per_shape[f"{L.K}->{L.N}"] = {"ms": sms, "tflops": fl / (sms * 1e-3) / 1e12}
        ms = time_launches(both(fns), reps) / len(fns)       # average per launch over the shape mix
        avg_flops = sum(flops) / len(flops)
        tf = avg_flops / (ms * 1e-3) / 1e12
        out[name] = {"avg_ms": ms, "flops_per_launch": avg_flops, "tflops": tf, "per_shape": per_shape}
    return out


def comparators(lins, reps):
    """The same fwd + bwd of both linears by other strategies, for context (the
    headline is the fused 4-bit path):
      lora_bf16_base: LoRA over a bf16 base (the dequantised weights kept in HBM)
        with this library's own GEMM kernels (lora_linear_fwd / lora_linear_bwd);
      dequant_then_gemm: the 4-bit base dequantised to bf16 in HBM each step
        (nf4_dequantize), then the same bf16-base kernels;
      *_hipblaslt: the same two with torch's bf16 GEMMs (hipBLASLt) for the base
        products and this library's adapter products.
    Also the bf16-weight GEMM kernels alone (kernels_bf16), to set against the
    fused 4-bit GEMMs (the cost of the on-the-fly dequantisation)."""
    import torch
    q = lins[0].q
    prep = []
    for L in lins:
        Wd = q.nf4_dequantize(L.codes, L.c2, L.c1, L.N, L.K)           # [N, K] bf16
        prep.append({"L": L, "W": Wd, "Wbuf": torch.empty_like(Wd)})

    def own_step(p, dequant):
        L = p["L"]
        W = p["Wbuf"] if dequant else p["W"]
        if dequant:
            q.nf4_dequantize(L.codes, L.c2, L.c1, L.N, L.K, out=W)
        q.lora_linear_fwd(L.X, W, L.L1, L.L2, 1.0, Y=L.Y, T_out=L.T, workspace=L.ws_f)
        q.lora_linear_bwd(L.X, L.dY, W, L.L1, L.L2, 1.0, T=L.T, dX=L.dX, dL1=L.dL1, dL2=L.dL2, workspace=L.ws_b)

    def torch_step(p, dequant):
        L = p["L"]
        W = p["Wbuf"] if dequant else p["W"]
        if dequant:
            q.nf4_dequantize(L.codes, L.c2, L.c1, L.N, L.K, out=W)
        # two-dimensional products only (transposed operands are plain views)
        T = q.qlora_lora_down(L.X, L.L1, T=L.T)
        Y = torch.mm(L.X, W.t())
        Y.add_(torch.mm(T, L.L2))
        G = q.qlora_lora_grad_in(L.dY, L.L2, 1.0, G=L.G)
        dX = torch.mm(L.dY, W)
        dX.add_(torch.mm(G, L.L1.t()))
        torch.mm(L.X.t(), G)                                             # dL1
        torch.mm(T.t(), L.dY)                                            # dL2

    out = {}
    flops = sum(L.flops() for L in lins)
    for name, fn, dq in (("lora_bf16_base", own_step, False), ("dequant_then_gemm", own_step, True),
                         ("lora_bf16_base_hipblaslt", torch_step, False),
                         ("dequant_then_gemm_hipblaslt", torch_step, True)):
        ms = time_launches(lambda: [fn(p, dq) for p in prep], reps)
        out[name] = {"ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}
    kb = {}
    for kind in ("fwd", "dx"):
        per = {}
        for p in prep:
            L = p["L"]
            if kind == "fwd":
                fl = 2 * L.M * L.K * L.N + 2 * L.M * L.r * L.N
                f = lambda L=L, W=p["W"]: q.lora_linear_fwd_t(L.X, W, L.T, L.L2, 1.0, Y=L.Y)
            else:
                fl = 2 * L.M * L.K * L.N + 2 * L.M * L.r * L.K
                f = lambda L=L, W=p["W"]: q.lora_linear_dx(L.dY, W, L.G, L.L1, dX=L.dX)
            ms = time_launches(f, reps)
            per[f"{L.K}->{L.N}"] = {"ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 1)}
        kb["k_bgemm_" + kind] = per
    out["kernels_bf16"] = kb
    del prep
    torch.cuda.empty_cache()
    return out


def decode_stacked_bench(dev, reps=200):
    """Stacked linears at decode size (M = 1): LLaMA-7B q|k|v (3 x 4096->4096) and
    gate|up (2 x 4096->11008) as one qlora_group_fwd call (one T-slice launch for
    every adapter, one decode launch over the stacked rows) against the same
    segments as separate qlora_linear_fwd calls; graph-replayed over rotated
    weight copies like decode_bench."""
    import torch
    import bit_quantized_lora_blockwise_amd as q
    import workloads as WL
    res = {}
    K, r, M = 4096, 64, 1
    for name, G, N in (("qkv", 3, 4096), ("gate_up", 2, 11008)):
        W = WL.normal((G * N, K), 0.02, 9100 + G, device=dev).to(torch.bfloat16)
        codes, absmax = q.nf4_quantize(W)
        c2, c1 = q.nf4_double_quant(absmax)
        del W, absmax
        packed = codes.numel() + c2.numel() + c1.numel() * 4
        copies = max(8, (600 << 20) // packed + 1)
        layers = [(codes.clone(), c2.clone(), c1.clone()) for _ in range(copies)]
        L1 = WL.normal((G, K, r), 1.0 / K, 9200 + G, device=dev).to(torch.bfloat16)
        L2 = WL.normal((G, r, N), 0.01, 9300 + G, device=dev).to(torch.bfloat16)
        X = WL.normal((M, K), 1.0, 9400 + G, device=dev).to(torch.bfloat16)
        Y = torch.empty((M, G * N), dtype=torch.bfloat16, device=dev)
        T = torch.empty((G, M, r), dtype=torch.bfloat16, device=dev)
        wsg = torch.empty((int(q.lib().qlora_group_fwd_workspace(M, K, N, G, r)),), dtype=torch.uint8, device=dev)
        wss = torch.empty((q.qlora_linear_fwd_workspace(M, K, N, r),), dtype=torch.uint8, device=dev)
        Ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(G)]
        nb = N * K // 64
        it = [0]

        def stacked():
            cd, cc2, cc1 = layers[it[0] % copies]
            it[0] += 1
            q.qlora_group_fwd(X, cd, cc2, cc1, N, G, L1, L2, 1.0, Y=Y, T_out=T, workspace=wsg)

        def separate():
            cd, cc2, cc1 = layers[it[0] % copies]
            it[0] += 1
            for g in range(G):
                q.qlora_linear_fwd(X, cd.view(-1)[g * N * K // 2:(g + 1) * N * K // 2], cc2.view(-1)[g * nb:(g + 1) * nb],
                                   cc1.view(-1)[g * nb // 256:(g + 1) * nb // 256], N, L1[g], L2[g], 1.0, Y=Ys[g],
                                   T_out=T[g], workspace=wss)

        sms = time_graph_launches(stacked, copies * 2, max(4, reps // (copies * 2)))
        pms = time_graph_launches(separate, copies * 2, max(4, reps // (copies * 2)))
        res[name] = {"G": G, "N": N, "K": K, "M": M, "packed_bytes": packed, "stacked_us": sms * 1e3,
                     "stacked_packed_gbps": packed / (sms * 1e-3) / 1e9, "separate_us": pms * 1e3,
                     "separate_packed_gbps": packed / (pms * 1e-3) / 1e9}
        del layers
        torch.cuda.empty_cache()
    return res


def decode_bench(dev, reps=200):
    import torch
    import bit_quantized_lora_blockwise_amd as q
    import workloads as WL
    res = {}
    inp = WL.config2(16)
    W = inp["W"].to(dev)
    N, K = W.shape
    codes, absmax = q.nf4_quantize(W)
    c2, c1 = q.nf4_double_quant(absmax)
    packed = codes.numel() + c2.numel() + c1.numel() * 4
    copies = max(24, (600 << 20) // packed + 1)
    layers = [(codes.clone(), c2.clone(), c1.clone()) for _ in range(copies)]
    del W, absmax
    L1, L2 = inp["L1"].to(dev), inp["L2"].to(dev)
    r = L1.shape[1]
    for M in (1, 4, 16):
        X = inp["X"][:M].contiguous().to(dev)
        T = q.qlora_lora_down(X, L1)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty((q.qlora_linear_fwd_workspace(M, K, N, r),), dtype=torch.uint8, device=dev)
        it = [0]

        def kern():
            cd, cc2, cc1 = layers[it[0] % copies]
            it[0] += 1
            q.qlora_linear_fwd_t(X, cd, cc2, cc1, N, T, L2, 1.0, Y=Y)

        def full():
            cd, cc2, cc1 = layers[it[0] % copies]
            it[0] += 1
            q.qlora_linear_fwd(X, cd, cc2, cc1, N, L1, L2, 1.0, Y=Y, T_out=T, workspace=ws)

        # calls queued behind a long GPU job (the copies rotate), so that the
        # events time the GPU alone (a captured graph would take the full call's
        # replay-safe two-launch path, timed beside as full_call_graph_us); and
        # the same calls issued one by one from Python for comparison
        kms = time_queued_launches(kern, copies * 2)
        fms = time_queued_launches(full, copies * 2)
        fms_graph = time_graph_launches(full, copies * 2, max(4, reps // (copies * 2)))
        kms_eager = time_launches(kern, reps)
        fms_eager = time_launches(full, reps)
        alg = packed + r * N * 2 + M * K * 2 + M * r * 2 + M * N * 2
        res[f"M{M}"] = {"kernel_us": kms * 1e3, "packed_gbps": packed / (kms * 1e-3) / 1e9,
                        "alg_gbps": alg / (kms * 1e-3) / 1e9, "full_call_us": fms * 1e3,
                        "full_call_packed_gbps": packed / (fms * 1e-3) / 1e9,
                        "full_call_alg_gbps": (alg + K * r * 2) / (fms * 1e-3) / 1e9,
                        "full_call_graph_us": fms_graph * 1e3,
                        "eager_kernel_us": kms_eager * 1e3, "eager_full_call_us": fms_eager * 1e3}
    res["packed_bytes"] = packed
    res["copies_rotated"] = copies
    del layers
    # the read ceiling: one plain streaming read of the same number of bytes per
    # call, over as many rotated copies, graph-replayed like the kernel timing;
    # every load depth of the probe is tried and the fastest is the ceiling
    import bit_quantized_lora_blockwise_amd.probe as P
    nbytes = (packed + 15) // 16 * 16
    bufs = [torch.empty((nbytes,), dtype=torch.uint8, device=dev) for _ in range(copies)]
    for b in bufs:
        b.fill_(1)
    sink = torch.zeros((1,), dtype=torch.int32, device=dev)
    by_loads = {}
    for loads in (1, 2, 4, 8, 16):
        it = [0]

        def probe(loads=loads):
            P.read_probe(bufs[it[0] % copies], sink, loads)
            it[0] += 1

        by_loads[loads] = time_graph_launches(probe, copies * 2, max(4, reps // (copies * 2))) * 1e3
    best = min(by_loads, key=by_loads.get)
    pus = by_loads[best]
    # the floor of an empty grid as large as the M = 1 decode kernel's (16 rows
    # of W per work group of 512 threads)
    groups = (N + 15) // 16
    eus = time_graph_launches(lambda: P.empty_probe(groups, 512), copies * 2,
                              max(4, reps // (copies * 2))) * 1e3
    res["read_ceiling"] = {"us": pus, "gbps": nbytes / (pus * 1e-6) / 1e9, "bytes": nbytes,
                           "loads_per_thread": best, "us_by_loads": {str(k): round(v, 3) for k, v in by_loads.items()},
                           "kernel": "k_read_probe (libqlprobe.so ql_read_probe)"}
    res["empty_grid_floor"] = {"us": eus, "groups": groups, "threads": 512,
                               "kernel": "k_empty_probe (libqlprobe.so ql_empty_probe)"}
    del bufs
    torch.cuda.empty_cache()
    return res


def encode_bench(dev, reps=3):
    import torch
    import bit_quantized_lora_blockwise_amd as q
    import workloads as WL
    mats = []
    for name in WL.LLAMA65B_BLOCK:
        W = WL.config5_weight(0, name, "gauss", device=dev)
        N, K = W.shape
        E = N * K
        bufs = (torch.empty((N, K // 2), dtype=torch.uint8, device=dev),
                torch.empty((E // 64,), dtype=torch.float32, device=dev),
                torch.empty((E // 64,), dtype=torch.uint8, device=dev),
                torch.empty(((E // 64 + 255) // 256,), dtype=torch.float32, device=dev))
        mats.append((W, bufs))

    def run():
        for W, (cd, am, c2, c1) in mats:
            q.nf4_quantize(W, cd, am)
            q.nf4_double_quant(am, c2, c1)

    def run_fused():
        for W, (cd, am, c2, c1) in mats:
            q.nf4_quantize_dq(W, codes=cd, c2=c2, c1=c1)

    ms_two = time_launches(run, reps)
    ms = time_launches(run_fused, reps)
    weights = sum(W.numel() for W, _ in mats)
    alg_bytes = weights * (2 + 0.5 + 4 / 64 + 4 / 64 + 1 / 64) + 4 * weights / 16384
    alg_bytes_fused = weights * (2 + 0.5 + 1 / 64) + 4 * weights / 16384
    res = {"block_weights": weights, "ms_per_block": ms, "weights_per_s": weights / (ms * 1e-3),
           "alg_gbps": alg_bytes_fused / (ms * 1e-3) / 1e9,
           "kernel": "k_nf4_encode_dq (one pass)", "ms_per_block_two_calls": ms_two,
           "alg_gbps_two_calls": alg_bytes / (ms_two * 1e-3) / 1e9}
    del mats
    torch.cuda.empty_cache()
    return res


def encode_model_bench(dev, layers=80):
    """The encoding workload of a whole LLaMA-65B-shaped model: the seven linear
    weights of each of `layers` blocks (64.76e9 weights at 80), drawn on the GPU
    with each layer's seeds in both weight distributions (N(0, 0.02) and
    0.02 * t_5).  For each distribution every weight is resident in HBM (129.5 GB
    of bf16) and every output buffer too (codes, c2, c1: 33.4 GB) before the
    timed region, which runs the one-pass encoder over all 7 * layers matrices
    back to back.  The codes of layers 0, 1, 40 and 79 of both distributions are
    compared with the CPU oracle bit for bit by the GPU test suite
    (test_gpu_encoder.py, test_fused_encoder_llama65b_layers), from the same
    generators and seeds."""
    import torch
    import bit_quantized_lora_blockwise_amd as q
    import workloads as WL
    names = list(WL.LLAMA65B_BLOCK)
    mats = []
    for layer in range(layers):
        for name in names:
            N, K = WL.LLAMA65B_BLOCK[name]
            nb = N * K // 64
            mats.append((layer, name, torch.empty((N, K), dtype=torch.bfloat16, device=dev),
                         torch.empty((N, K // 2), dtype=torch.uint8, device=dev),
                         torch.empty((nb,), dtype=torch.uint8, device=dev),
                         torch.empty(((nb + 255) // 256,), dtype=torch.float32, device=dev)))
    weights = sum(m[2].numel() for m in mats)
    alg_bytes = weights * (2 + 0.5 + 1 / 64) + 4 * sum(m[5].numel() for m in mats)
    out = {"layers": layers, "matrices": len(mats), "weights": weights, "alg_bytes": alg_bytes,
           "kernel": "k_nf4_encode_dq (nf4_quantize_dq)",
           "bitexact_vs_oracle": "layers 0, 1, 40, 79 x both distributions: tests/test_gpu_encoder.py"}
    for variant in ("gauss", "t5"):
        g0 = time.perf_counter()
        for layer, name, W, _, _, _ in mats:
            W.copy_(WL.config5_weight(layer, name, variant, device=dev))
        torch.cuda.synchronize()
        gen_s = time.perf_counter() - g0

        def run():
            for _, _, W, cd, c2, c1 in mats:
                q.nf4_quantize_dq(W, codes=cd, c2=c2, c1=c1)

        run()                                   # warm-up pass over every matrix
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        gbps = alg_bytes / (ms * 1e-3) / 1e9
        out[variant] = {"ms": round(ms, 3), "weights_per_s": weights / (ms * 1e-3), "alg_gbps": round(gbps, 1),
                        "frac_of_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4), "generate_s": round(gen_s, 2)}
    del mats
    torch.cuda.empty_cache()
    return out


def merge_bench(dev, reps=20):
    """Adapter merge (W' + s (L1 L2)^T to bf16) of the LLaMA-7B up and down
    projections at r = 64: one launch per matrix, HBM-bound."""
    import torch
    import bit_quantized_lora_blockwise_amd as q
    import workloads as WL
    mats = []
    for i, (N, K) in enumerate((WL.LLAMA7B_UP, WL.LLAMA7B_DOWN)):
        codes, absmax = q.nf4_quantize(WL.weight_gaussian(N, K, 0.02, 90 + 10 * i, device=dev))
        c2, c1 = q.nf4_double_quant(absmax)
        L1, L2 = (t.to(dev) for t in WL.lora_pair(K, N, 64, 91 + 10 * i, 92 + 10 * i, 0.01))
        out = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        mats.append((codes, c2, c1, N, K, L1, L2, out))

    def run():
        for codes, c2, c1, N, K, L1, L2, out in mats:
            q.qlora_merge(codes, c2, c1, N, K, L1, L2, 2.0, out=out)

    ms = time_launches(run, reps)
    elems = sum(m[3] * m[4] for m in mats)
    alg_bytes = sum(N * K * (0.5 + 2 + 1 / 64) + 4 * (N * K // 16384) + 2 * 64 * (N + K)
                    for _, _, _, N, K, _, _, _ in mats)
    gbps = alg_bytes / (ms * 1e-3) / 1e9
    del mats
    torch.cuda.empty_cache()
    return {"kernel": "k_merge", "weights": elems, "ms_two_launches": ms, "alg_bytes": alg_bytes,
            "alg_gbps": gbps, "frac_of_hbm_peak": gbps / PEAK_HBM_GBPS}


def quant_study(dev, n=4096, reps=10):
    """Quantization error of the 4-bit formats the pages rank (NF4 with double
    quantization against a 4-bit float and 4-bit integers) under the four ways
    of coding the block scales, on n x n N(0, 1) and Student-t (5 d.o.f.)
    weights: normalised MSE sum (W' - W)^2 / sum W^2 and the entropy of the code
    histogram, plus the time of the table encoder and dequantizer."""
    import torch
    import bit_quantized_lora_blockwise_amd as q
    g = torch.Generator(device=dev).manual_seed(1234)
    mats = {"normal": torch.randn((n, n), generator=g, device=dev)}
    z = torch.randn((n, n), generator=g, device=dev)
    chi = sum(torch.randn((n, n), generator=g, device=dev) ** 2 for _ in range(5))
    mats["t5"] = z / torch.sqrt(chi / 5)
    del z, chi
    out = {"weights": n * n, "nmse": {}, "code_entropy_bits": {}}
    for dist, W in mats.items():
        Wb = W.to(torch.bfloat16)
        Wf = Wb.float()
        den = (Wf.double() ** 2).sum()
        for book in ("nf4", "fp4", "int4"):
            codes, absmax = q.q4_quantize(Wb, book)
            h = torch.bincount(torch.cat([(codes & 15).flatten(), (codes >> 4).flatten()]).long(), minlength=16)
            p = h.double() / h.sum()
            p = p[p > 0]
            out["code_entropy_bits"][f"{dist}/{book}"] = round(float(-(p * torch.log2(p)).sum()), 4)
            for sc in ("absmax", "groupmax", "fullrange", "mean"):
                if sc == "absmax":
                    Wd = q.q4_dequantize(codes, n, n, book, sc, absmax=absmax)
                else:
                    c2, c1, mu = q.q4_double_quant(absmax, sc)
                    Wd = q.q4_dequantize(codes, n, n, book, sc, c2=c2, c1=c1, mu=mu)
                out["nmse"][f"{dist}/{book}/{sc}"] = round(float(((Wd.float() - Wf).double() ** 2).sum() / den), 6)
    Wb = mats["normal"].to(torch.bfloat16)
    codes, absmax = q.q4_quantize(Wb, "fp4")
    c2, c1, mu = q.q4_double_quant(absmax, "mean")
    Wd = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
    t_enc = time_launches(lambda: q.q4_quantize(Wb, "fp4", codes=codes, absmax=absmax), reps)
    t_nf4 = time_launches(lambda: q.nf4_quantize(Wb, codes=codes, absmax=absmax), reps)
    t_deq = time_launches(lambda: q.q4_dequantize(codes, n, n, "fp4", "mean", c2=c2, c1=c1, mu=mu, out=Wd), reps)
    e = n * n
    out["encode_table_us"] = round(t_enc * 1e3, 2)
    out["encode_table_gbps"] = round(e * (2 + 0.5 + 4 / 64) / (t_enc * 1e-3) / 1e9, 1)
    out["encode_nf4_bucketed_us"] = round(t_nf4 * 1e3, 2)
    out["dequant_mean_us"] = round(t_deq * 1e3, 2)
    out["dequant_mean_gbps"] = round(e * (0.5 + 1 / 64 + 2) / (t_deq * 1e-3) / 1e9, 1)
    del mats
    torch.cuda.empty_cache()
    return out


BLOCK_GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))


class BlockPipe:
    """One LLaMA-65B Transformer block's seven quantized LoRA linears at M tokens,
    trained one step: forward and backward of every linear, then one AdamW step
    over all adapters held in one flat buffer.  stacked=True runs q|k|v and
    gate|up as stacked matrices (4 layer calls), False the seven separate layers.
    The packed bases are built once (the base is frozen); everything the timed
    step touches is allocated here."""

    def __init__(self, dev, M, stacked, r=64):
        import torch
        import bit_quantized_lora_blockwise_amd as q
        import workloads as WL
        self.q, self.stacked, self.M, self.r = q, stacked, M, r
        f32, bf, u8 = torch.float32, torch.bfloat16, torch.uint8
        self.groups = []
        sizes = 0
        for gi, grp in enumerate(BLOCK_GROUPS):
            N, K = WL.LLAMA65B_BLOCK[grp[0]]
            G = len(grp)
            sizes += G * (K * r + r * N)
        self.master = torch.empty(sizes, dtype=f32, device=dev)
        self.grad = torch.zeros(sizes, dtype=f32, device=dev)
        self.m = torch.zeros(sizes, dtype=f32, device=dev)
        self.v = torch.zeros(sizes, dtype=f32, device=dev)
        self.pb = torch.empty(sizes, dtype=bf, device=dev)
        off = 0
        for gi, grp in enumerate(BLOCK_GROUPS):
            N, K = WL.LLAMA65B_BLOCK[grp[0]]
            G = len(grp)
            Ws, L1s, L2s = [], [], []
            for name in grp:
                i = list(WL.LLAMA65B_BLOCK).index(name)
                base = 100 * (i + 1)
                Ws.append(WL.weight_row_std(N, K, 0.01, 0.05, base, torch.bfloat16, dev))
                L1s.append(WL.normal((K, r), 1.0 / K, base + 1, device=dev))
                L2s.append(WL.normal((r, N), 0.01, base + 2, device=dev))
            codes, absmax = q.nf4_quantize(torch.cat(Ws))
            c2, c1 = q.nf4_double_quant(absmax)
            del Ws, absmax
            a, b = G * K * r, G * r * N
            self.master[off:off + a] = torch.stack(L1s).float().flatten()
            self.master[off + a:off + a + b] = torch.stack(L2s).float().flatten()
            gr = {"names": grp, "N": N, "K": K, "G": G, "codes": codes, "c2": c2, "c1": c1,
                  "L1": self.pb[off:off + a].view(G, K, r), "L2": self.pb[off + a:off + a + b].view(G, r, N),
                  "dL1": self.grad[off:off + a].view(G, K, r), "dL2": self.grad[off + a:off + a + b].view(G, r, N),
                  "X": WL.normal((M, K), 1.0, 1000 + gi, device=dev)}
            off += a + b
            dY = WL.normal((M, G * N), 1e-2, 1100 + gi, device=dev)
            nb = N * K // 64
            if stacked:
                gr["dY"] = dY
                gr["Y"] = torch.empty((M, G * N), dtype=bf, device=dev)
                gr["T"] = torch.empty((G, M, r), dtype=bf, device=dev)
                gr["dX"] = torch.empty((M, K), dtype=bf, device=dev)
                gr["ws_f"] = torch.empty(max(16, q.lib().qlora_group_fwd_workspace(M, K, N, G, r)), dtype=u8,
                                         device=dev)
                gr["ws_b"] = torch.empty(max(16, q.lib().qlora_group_bwd_workspace(M, K, N, G, r)), dtype=u8,
                                         device=dev)
            else:
                gr["seg"] = []
                for g in range(G):
                    gr["seg"].append({
                        "codes": codes[g * N:(g + 1) * N], "c2": c2[g * nb:(g + 1) * nb],
                        "c1": c1[g * nb // 256:(g + 1) * nb // 256], "dY": dY[:, g * N:(g + 1) * N].contiguous(),
                        "Y": torch.empty((M, N), dtype=bf, device=dev), "T": torch.empty((M, r), dtype=bf, device=dev),
                        "dX": torch.empty((M, K), dtype=bf, device=dev)})
                gr["ws_f"] = torch.empty(max(16, q.qlora_linear_fwd_workspace(M, K, N, r)), dtype=u8, device=dev)
                gr["ws_b"] = torch.empty(max(16, q.qlora_linear_bwd_workspace(M, K, N, r)), dtype=u8, device=dev)
                del dY
            self.groups.append(gr)
        self.pb.copy_(self.master)
        self.n_adapter = sizes
        self.t = 0

    def fwd_bwd(self):
        q = self.q
        for gr in self.groups:
            if self.stacked:
                q.qlora_group_fwd(gr["X"], gr["codes"], gr["c2"], gr["c1"], gr["N"], gr["G"], gr["L1"], gr["L2"],
                                  1.0, Y=gr["Y"], T_out=gr["T"], workspace=gr["ws_f"])
                q.qlora_group_bwd(gr["X"], gr["dY"], gr["codes"], gr["c2"], gr["c1"], gr["G"], gr["L1"], gr["L2"],
                                  1.0, T=gr["T"], dX=gr["dX"], dL1=gr["dL1"], dL2=gr["dL2"], workspace=gr["ws_b"])
            else:
                for g, sg in enumerate(gr["seg"]):
                    q.qlora_linear_fwd(gr["X"], sg["codes"], sg["c2"], sg["c1"], gr["N"], gr["L1"][g], gr["L2"][g],
                                       1.0, Y=sg["Y"], T_out=sg["T"], workspace=gr["ws_f"])
                    q.qlora_linear_bwd(gr["X"], sg["dY"], sg["codes"], sg["c2"], sg["c1"], gr["L1"][g],
                                       gr["L2"][g], 1.0, T=sg["T"], dX=sg["dX"], dL1=gr["dL1"][g],
                                       dL2=gr["dL2"][g], workspace=gr["ws_b"])

    def optimizer(self):
        self.t += 1
        self.q.qlora_adamw_step(self.master, self.m, self.v, self.grad, self.t, 1e-4, weight_decay=0.0,
                                param_bf16=self.pb)

    def step(self):
        self.fwd_bwd()
        self.optimizer()


def block_bench(dev, reps=5, M=2048):
    """LLaMA-65B block (7 linears, r = 64, M = 2048 tokens): fwd + bwd of every
    linear and one AdamW step over all adapters, stacked and separate."""
    import torch
    import workloads as WL
    flops = sum(layer_flops(M, K, N, 64) for N, K in WL.LLAMA65B_BLOCK.values())
    out = {"workload": "llama65b block: q,k,v,o 8192x8192, gate,up 8192->22016, down 22016->8192, r=64, M=2048",
           "flops_per_step": flops}
    for stacked in (True, False):
        pipe = BlockPipe(dev, M, stacked)
        key = "stacked" if stacked else "separate"
        ms = time_launches(pipe.step, reps)
        ms_fb = time_launches(pipe.fwd_bwd, reps)
        ms_opt = time_launches(pipe.optimizer, reps)
        out[key] = {"step_ms": round(ms, 4), "fwd_bwd_ms": round(ms_fb, 4), "adamw_ms": round(ms_opt, 4),
                    "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                    "adamw_gbps": round(pipe.n_adapter * 30 / (ms_opt * 1e-3) / 1e9, 1)}
        out["adapter_params"] = pipe.n_adapter
        del pipe
        torch.cuda.empty_cache()
    out["frac_of_bf16_peak"] = round(out["stacked"]["tflops"] / PEAK_BF16_TFLOPS, 4)
    return out


def cpu_baseline(min_seconds=10.0, max_passes=4):
    """The CPU oracle on a bounded sample of the headline workload: whole steps
    (both linears, 4096 -> 11008 and 11008 -> 4096, r = 64, M = 4096 tokens:
    encode, double quant, dequant, forward and backward in float64 NumPy),
    repeated until at least `min_seconds` of CPU time have been measured (at
    most `max_passes` steps)."""
    import numpy as np
    import torch
    import oracle as O
    import workloads as WL
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    b = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    c3 = WL.config3()
    lins = []
    for name in ("up", "down"):
        inp = c3[name]
        lins.append((inp["W"].float().numpy(), b(inp["X"]), b(inp["L1"]), b(inp["L2"]), b(inp["dY"])))
    del c3
    flops_step = sum(layer_flops(X.shape[0], W.shape[1], W.shape[0], 64) for W, X, _, _, _ in lins)
    passes, dt = 0, 0.0
    while passes < max_passes and (passes == 0 or dt < min_seconds):
        t0 = time.perf_counter()
        for W, X, L1, L2, dY in lins:
            N, K = W.shape
            codes, absmax = O.nf4_quantize(W)
            c2, c1 = O.nf4_double_quant(absmax)
            Wq = O.nf4_dequantize(codes, c2, c1, N, K)
            Y, T = O.qlora_forward(X, Wq, L1, L2, 1.0)
            O.qlora_backward(X, dY, Wq, L1, L2, 1.0, T=T)
        dt += time.perf_counter() - t0
        passes += 1
    return {"value": flops_step * passes / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model(),
            "seconds": round(dt, 3), "steps": passes,
            "sample": f"{passes} whole step(s) of the headline workload (llama7b MLP up + down, M=4096, r=64): "
                      "encode + double quant + dequant + fwd + bwd, float64 NumPy oracle on the host"}


def cpu_model():
    """Model name of the host CPU (from /proc/cpuinfo), with the number of
    logical CPUs this process may run on."""
    name = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                name = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return f"{name} ({len(os.sched_getaffinity(0))} logical CPUs available)"


def pmc_probe(lins, reps=3):
    """Launches for hardware-counter runs: fused forward and dX GEMMs of both
    headline linears, the M = 1 decode forward at 4096 -> 11008 (the full
    qlora_linear_fwd call: one launch that also forms T), the
    one-pass encoder of both weights, then one copy of 512 MiB (bytes read =
    bytes written = 2^29), the known-size reference for the traffic counters."""
    import torch
    q = lins[0].q
    for L in lins:
        q.qlora_lora_down(L.X, L.L1, T=L.T)
        q.qlora_lora_grad_in(L.dY, L.L2, 1.0, G=L.G)
    for _ in range(reps):
        for L in lins:
            q.qlora_linear_fwd_t(L.X, L.codes, L.c2, L.c1, L.N, L.T, L.L2, 1.0, Y=L.Y)
            q.qlora_linear_dx(L.dY, L.codes, L.c2, L.c1, L.K, L.G, L.L1, dX=L.dX)
    up = lins[0]
    X1 = up.X[:1].contiguous()
    Y1 = torch.empty((1, up.N), dtype=torch.bfloat16, device=X1.device)
    for _ in range(reps):
        q.qlora_linear_fwd(X1, up.codes, up.c2, up.c1, up.N, up.L1, up.L2, 1.0, Y=Y1)
    for _ in range(reps):
        for L in lins:
            L.encode()
    torch.cuda.synchronize()
    src = torch.empty((1 << 28,), dtype=torch.int16, device=lins[0].X.device).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_probe": "done", "gemm_launches_per_kind": reps * len(lins), "decode_launches": reps,
                      "encoder_launches": reps * len(lins), "copy_bytes": 1 << 29}))


def decode_roofline(dec):
    """The M = 1 decode forward at 4096 -> 11008 against 8 TB/s: the full
    qlora_linear_fwd call (one launch of k_qgemv_fwd that also forms T = X L1
    in its first work groups; algorithmic bytes include L1), and beside it the
    decode kernel alone at the stage entry point (T given)."""
    m1 = dec["M1"]
    ceil = dec["read_ceiling"]
    return {"kernel": "k_qgemv_fwd", "call": "qlora_linear_fwd (one launch, T formed in it)",
            "bound": "hbm", "achieved": m1["full_call_alg_gbps"], "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": m1["full_call_alg_gbps"] / PEAK_HBM_GBPS,
            "traffic": recorded_traffic("k_qgemv_fwd", DECODE_SOURCE),
            "avg_launch_us": m1["full_call_us"], "read_ceiling_gbps": ceil["gbps"],
            "packed_frac_of_read_ceiling": m1["full_call_packed_gbps"] / ceil["gbps"],
            "stage_kernel_us": m1["kernel_us"], "stage_frac": m1["alg_gbps"] / PEAK_HBM_GBPS,
            "empty_grid_floor_us": dec["empty_grid_floor"]["us"]}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as WL
    import bit_quantized_lora_blockwise_amd as q
    q.lib()
    dev = "cuda:0"
    torch.cuda.set_device(0)

    c3 = WL.config3()
    lins = [Linear(c3["up"], dev), Linear(c3["down"], dev)]
    del c3
    if args.pmc_probe:
        for L in lins:
            L.encode()
        pmc_probe(lins)
        return
    if args.roofline_only:
        for L in lins:
            L.encode()
        kern = kernel_rooflines(lins, args.kernel_reps)
        dom = max(kern, key=lambda k: kern[k]["avg_ms"])
        del lins
        torch.cuda.empty_cache()
        dec = decode_bench(dev)
        print(json.dumps({"roofline_only": True, "kernels": kern, "dominant": dom,
                          "roofline_decode": decode_roofline(dec), "decode": dec}))
        return

    def step():
        for L in lins:
            L.step()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    for _ in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    flops = sum(L.flops() for L in lins)
    value = flops / (ms_step * 1e-3) / 1e12
    if args.step_only:
        print(json.dumps({"step_only": True, "value": round(value, 3), "ms_per_step": round(ms_step, 4),
                          "steps": args.steps, "warmup": args.warmup}))
        return

    # phases of the step, each timed alone
    phases = {}
    for name, fn in (("encode", lambda: [L.encode() for L in lins]),
                     ("forward", lambda: [L.forward() for L in lins]),
                     ("backward", lambda: [L.backward() for L in lins])):
        phases[name + "_ms"] = time_launches(fn, max(3, args.kernel_reps // 4))
    fb_ms = phases["forward_ms"] + phases["backward_ms"]

    kern = kernel_rooflines(lins, args.kernel_reps)
    dom = max(kern, key=lambda k: kern[k]["avg_ms"])
    roof = {"kernel": dom, "bound": "mfma", "achieved": kern[dom]["tflops"], "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": kern[dom]["tflops"] / PEAK_BF16_TFLOPS, "traffic": recorded_traffic(dom),
            "avg_launch_ms": kern[dom]["avg_ms"], "flops_per_launch": kern[dom]["flops_per_launch"]}
    comp = comparators(lins, max(3, args.kernel_reps // 4))
    del lins
    torch.cuda.empty_cache()

    dec = decode_bench(dev)
    dec_roof = decode_roofline(dec)
    dec["stacked_m1"] = decode_stacked_bench(dev)
    enc = encode_bench(dev)
    enc["model_80_layers"] = encode_model_bench(dev)
    mrg = merge_bench(dev)
    study = quant_study(dev)
    blk = block_bench(dev)

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama7b MLP up 4096->11008 + down 11008->4096, M=4096 tokens, r=64: "
                               "encode + double quant + fwd + bwd per step",
                   "global_batch": 4096, "seq_len": 4096, "parallelism": "none (1 GPU)"},
        "fwd_bwd_only": {"ms": round(fb_ms, 4), "tflops": round(flops / (fb_ms * 1e-3) / 1e12, 3)},
        "phases_ms": {k: round(v, 4) for k, v in phases.items()},
        "comparators": comp,
        "roofline": roof,
        "kernels": kern,
        "decode_m1_packed_gbps": round(dec["M1"]["packed_gbps"], 1),
        "decode": dec,
        "roofline_decode": dec_roof,
        "encode": enc,
        "merge": mrg,
        "quant_study": study,
        "block": blk,
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
