"""GPU parity of the quantized LoRA linear (forward and backward) against the
CPU oracle: small and ragged shapes, the decode-sized workloads and the
training-sized LLaMA-7B and LLaMA-65B linears, every output compared element by
element (the large weights go through the oracle's encoder in worker processes,
on group-aligned row slabs).

Tolerance (Y, dX, dL1, dL2 and T): relative L2 <= 2e-3 and
max |err| <= 1e-2 * max |ref|, with the oracle rounding T, Y, G and dX to bf16
at the same points as the kernels."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
import oracle_pool
from gpu_util import assert_bitexact, assert_close, bits, f32np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def qlib():
    import bit_quantized_lora_blockwise_amd as q
    return q


def quantize_both(W_cpu):
    """Quantize on the GPU (kept on device) and, independently, with the oracle."""
    q = qlib()
    codes, absmax = q.nf4_quantize(W_cpu.to(DEV))
    c2, c1 = q.nf4_double_quant(absmax)
    Wn = W_cpu.float().numpy()
    rc, ra = O.nf4_quantize(Wn)
    rc2, rc1 = O.nf4_double_quant(ra)
    return (codes, c2, c1), (rc, rc2, rc1)


def run_gpu(inp, s=1.0, quant=None, keep_T=True):
    q = qlib()
    W = inp["W"]
    N, K = W.shape
    (codes, c2, c1) = quant
    X, L1, L2, dY = (inp[k].to(DEV) for k in ("X", "L1", "L2", "dY"))
    Y, T = q.qlora_linear_fwd(X, codes, c2, c1, N, L1, L2, s, T_out=True)
    dX, dL1, dL2 = q.qlora_linear_bwd(X, dY, codes, c2, c1, L1, L2, s, T=T if keep_T else None)
    torch.cuda.synchronize()
    return {"Y": Y, "T": T, "dX": dX, "dL1": dL1, "dL2": dL2}


def full_case(inp, s=1.0, name=""):
    N, K = inp["W"].shape
    M = inp["X"].shape[0]
    r = inp["L1"].shape[1]
    print(f"[layer] {name} M={M} K={K} N={N} r={r} s={s}", flush=True)
    gq, rq = quantize_both(inp["W"])
    g = run_gpu(inp, s, gq)
    Wq = O.nf4_dequantize(*rq, N, K)
    X, L1, L2, dY = (bits(inp[k]) for k in ("X", "L1", "L2", "dY"))
    Y, T = O.qlora_forward(X, Wq, L1, L2, s)
    dX, dL1, dL2, G, _ = O.qlora_backward(X, dY, Wq, L1, L2, s, T=T)
    assert_close(bits(g["T"]), T, f"{name} T")
    assert_close(bits(g["Y"]), Y, f"{name} Y")
    assert_close(bits(g["dX"]), dX, f"{name} dX")
    assert_close(f32np(g["dL1"]), dL1, f"{name} dL1")
    assert_close(f32np(g["dL2"]), dL2, f"{name} dL2")
    return g


def test_config1_full():
    full_case(WL.config1(), 1.0, "512x512 r=8 M=32")


RAGGED = [
    (37, 192, 200, 5), (17, 64, 33, 1), (130, 256, 136, 16), (64, 320, 96, 64), (200, 128, 260, 24),
    (1, 128, 50, 3), (2, 64, 8, 64), (3, 192, 77, 7), (4, 256, 130, 12), (16, 512, 260, 64), (15, 64, 129, 33),
    (257, 320, 300, 64), (300, 1088, 520, 13),
]


@pytest.mark.parametrize("M,K,N,r", RAGGED)
def test_ragged_shapes(M, K, N, r):
    inp = WL.layer_inputs(N, K, M, r, seed_base=M * 7919 + K * 31 + N + r, l2_std=0.3)
    full_case(inp, 0.75, "ragged")


@pytest.mark.parametrize("M", [32, 4])
def test_lora_isolation_zero_base(M):
    """W == 0: every code is 7 and every scale 0, so Y = bf16(s T L2) and dX = bf16(G L1^T);
    with L2 ~ N(0, 1) the LoRA epilogues are checked on their own."""
    inp = WL.layer_inputs(384, 256, M, 16, seed_base=500 + M, l2_std=1.0)
    inp["W"] = torch.zeros_like(inp["W"])
    full_case(inp, 1.5, "W=0")


def test_zero_upstream_gradient():
    inp = WL.layer_inputs(192, 128, 40, 8, seed_base=900)
    inp["dY"] = torch.zeros_like(inp["dY"])
    gq, _ = quantize_both(inp["W"])
    g = run_gpu(inp, 1.0, gq)
    assert not torch.any(g["dX"].float() != 0) and not torch.any(g["dL1"] != 0) and not torch.any(g["dL2"] != 0)


def test_recompute_T_and_skip_dX_match():
    q = qlib()
    inp = WL.layer_inputs(320, 192, 48, 12, seed_base=1234)
    gq, _ = quantize_both(inp["W"])
    a = run_gpu(inp, 1.0, gq, keep_T=True)
    b = run_gpu(inp, 1.0, gq, keep_T=False)
    assert torch.equal(a["dX"], b["dX"]) and torch.equal(a["dL1"], b["dL1"]) and torch.equal(a["dL2"], b["dL2"])
    X, L1, L2, dY = (inp[k].to(DEV) for k in ("X", "L1", "L2", "dY"))
    codes, c2, c1 = gq
    dX, dL1, dL2 = q.qlora_linear_bwd(X, dY, codes, c2, c1, L1, L2, 1.0, T=a["T"], dX=None)
    torch.cuda.synchronize()
    assert dX is None and torch.equal(dL1, a["dL1"]) and torch.equal(dL2, a["dL2"])


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_llama7b_up_full(M):
    """Decode-sized forward at the full 4096 -> 11008 shape, every output compared."""
    inp = WL.config2(M)
    N, K = inp["W"].shape
    print(f"[decode] M={M} K={K} N={N}", flush=True)
    q = qlib()
    gq, rq = quantize_both(inp["W"])
    X, L1, L2 = (inp[k].to(DEV) for k in ("X", "L1", "L2"))
    Y, T = q.qlora_linear_fwd(X, *gq, N, L1, L2, 1.0, T_out=True)
    torch.cuda.synchronize()
    Wq = O.nf4_dequantize(*rq, N, K)
    rY, rT = O.qlora_forward(bits(inp["X"]), Wq, bits(inp["L1"]), bits(inp["L2"]), 1.0)
    assert_close(bits(T), rT, f"decode M={M} T")
    assert_close(bits(Y), rY, f"decode M={M} Y")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_llama7b_down_full(M):
    """Decode-sized forward at the 11008 -> 4096 shape (few work groups, so the
    kernel splits K over more waves; X staged in LDS per work group at M = 1, once
    per CU by the persistent kernel at M = 4, slice by slice at M = 16), every
    output compared."""
    inp = WL.layer_inputs(4096, 11008, M, 64, seed_base=7100 + M)
    print(f"[decode] M={M} K=11008 N=4096", flush=True)
    q = qlib()
    gq, rq = quantize_both(inp["W"])
    X, L1, L2 = (inp[k].to(DEV) for k in ("X", "L1", "L2"))
    Y, T = q.qlora_linear_fwd(X, *gq, 4096, L1, L2, 1.0, T_out=True)
    torch.cuda.synchronize()
    Wq = O.nf4_dequantize(*rq, 4096, 11008)
    rY, rT = O.qlora_forward(bits(inp["X"]), Wq, bits(inp["L1"]), bits(inp["L2"]), 1.0)
    assert_close(bits(T), rT, f"decode down M={M} T")
    assert_close(bits(Y), rY, f"decode down M={M} Y")


def test_decode_graph_replay_matches_eager():
    """The decode forward captured in a HIP graph (as the decode timing runs it):
    every replay, with eager work and synchronisations in between, gives the
    eager call's Y and T bit for bit."""
    q = qlib()
    inp = WL.layer_inputs(4096, 2048, 4, 64, seed_base=4242)
    gq, _ = quantize_both(inp["W"])
    X, L1, L2 = (inp[k].to(DEV) for k in ("X", "L1", "L2"))
    Y0, T0 = q.qlora_linear_fwd(X, *gq, 4096, L1, L2, 1.0, T_out=True)
    Y = torch.empty_like(Y0)
    T = torch.empty_like(T0)
    ws = torch.empty((q.qlora_linear_fwd_workspace(4, 2048, 4096, 64),), dtype=torch.uint8, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q.qlora_linear_fwd(X, *gq, 4096, L1, L2, 1.0, Y=Y, T_out=T, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.qlora_linear_fwd(X, *gq, 4096, L1, L2, 1.0, Y=Y, T_out=T, workspace=ws)
    for rep in range(4):
        Y.fill_(0)
        T.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), Y0.view(torch.int16)), rep
        assert torch.equal(T.view(torch.int16), T0.view(torch.int16)), rep
        q.nf4_dequantize(*gq, 4096, 2048)                  # eager work between replays
    del g


# decode shapes whose step counts do not divide evenly over the waves: 8-wave
# work groups (over 384 of them) and 16-wave ones, X in LDS per work group, and
# the persistent kernel (M = 9 and 12: X of 32-128 KB; at K = 1600 nine of its
# sixteen waves have no steps)
DECODE_SPLIT = [(3, 2880, 6200, 8), (2, 2368, 100, 64), (9, 4160, 6500, 16), (12, 1600, 40, 20)]


@pytest.mark.parametrize("M,K,N,r", DECODE_SPLIT)
def test_decode_uneven_wave_split(M, K, N, r):
    inp = WL.layer_inputs(N, K, M, r, seed_base=M * 131 + K + N + r, l2_std=0.3)
    full_case(inp, 1.25, "decode split")


# the persistent decode kernel (X of 32-128 KB) with T formed elsewhere: a rank
# that is not a multiple of 4 (T by the separate product and its reduce), and T
# handed to the stage entry point
DECODE_PERSIST_GIVEN_T = [(9, 4160, 6500, 7), (16, 2048, 1000, 33), (5, 6400, 300, 64)]


@pytest.mark.parametrize("M,K,N,r", DECODE_PERSIST_GIVEN_T)
def test_decode_persistent_given_T(M, K, N, r):
    inp = WL.layer_inputs(N, K, M, r, seed_base=M * 17 + K + N * 3 + r, l2_std=0.3)
    full_case(inp, 0.8, "decode persistent")
    q = qlib()
    gq, rq = quantize_both(inp["W"])
    X, L1, L2 = (inp[k].to(DEV) for k in ("X", "L1", "L2"))
    T = q.qlora_lora_down(X, L1)
    Y = q.qlora_linear_fwd_t(X, *gq, N, T, L2, 0.8)
    torch.cuda.synchronize()
    Wq = O.nf4_dequantize(*rq, N, K)
    rY, rT = O.qlora_forward(bits(inp["X"]), Wq, bits(inp["L1"]), bits(inp["L2"]), 0.8)
    assert_close(bits(T), rT, f"decode persistent given T: T M={M} K={K} r={r}")
    assert_close(bits(Y), rY, f"decode persistent given T: Y M={M} K={K} r={r}")


# the slice-staged decode kernel (X above 128 KB, at most one 16-row tile per CU):
# M odd, N not a multiple of 16, a rank that is not a multiple of 4, a last slice
# of 128 columns; and three full slices
# one tile per work group; then more 16-row tiles than the 256 CUs of an MI355X,
# so that each work group keeps 2, 3 or 5 tiles' sums across the slices (the
# last slice 256, 2304, 4096 or 64 columns wide)
DECODE_SLICES = [(11, 8320, 1000, 13), (16, 12288, 2048, 64),
                 (16, 4352, 12000, 64), (11, 6400, 9000, 13), (6, 12288, 4200, 16), (16, 4160, 16400, 64)]


@pytest.mark.parametrize("M,K,N,r", DECODE_SLICES)
def test_decode_slices(M, K, N, r):
    assert M * K * 2 > 131072
    inp = WL.layer_inputs(N, K, M, r, seed_base=M * 23 + K + N * 5 + r, l2_std=0.3)
    full_case(inp, 0.9, "decode slices")
    q = qlib()
    gq, rq = quantize_both(inp["W"])
    X, L1, L2 = (inp[k].to(DEV) for k in ("X", "L1", "L2"))
    T = q.qlora_lora_down(X, L1)
    Y = q.qlora_linear_fwd_t(X, *gq, N, T, L2, 0.9)
    torch.cuda.synchronize()
    Wq = O.nf4_dequantize(*rq, N, K)
    rY, rT = O.qlora_forward(bits(inp["X"]), Wq, bits(inp["L1"]), bits(inp["L2"]), 0.9)
    assert_close(bits(T), rT, f"decode slices given T: T M={M} K={K} r={r}")
    assert_close(bits(Y), rY, f"decode slices given T: Y M={M} K={K} r={r}")


def _big_case(inp, name):
    """Full-size check, every output element compared: the GPU encoder's codes,
    absmax, c2 and c1 bit-exact against the oracle's (computed on group-aligned
    row slabs in worker processes), then T, Y, dX, dL1 and dL2 of the layer
    against the oracle's float64 layer on the oracle's own dequantized weight."""
    q = qlib()
    N, K = inp["W"].shape
    M = inp["X"].shape[0]
    print(f"[layer full] {name} M={M} K={K} N={N}", flush=True)
    W = inp["W"].to(DEV)
    codes, absmax = q.nf4_quantize(W)
    c2, c1 = q.nf4_double_quant(absmax)
    g = run_gpu(inp, 1.0, (codes, c2, c1))
    rc, ra, rc2, rc1, Wq = oracle_pool.quantize(bits(inp["W"]))
    assert_bitexact(codes.cpu().numpy().reshape(-1), rc.reshape(-1), f"{name} codes")
    assert_bitexact(absmax.cpu().numpy().view(np.uint32), ra.view(np.uint32), f"{name} absmax")
    assert_bitexact(c2.cpu().numpy(), rc2, f"{name} c2")
    assert_bitexact(c1.cpu().numpy().view(np.uint32), rc1.view(np.uint32), f"{name} c1")
    X, L1, L2, dY = (bits(inp[k]) for k in ("X", "L1", "L2", "dY"))
    Y, T = O.qlora_forward(X, Wq, L1, L2, 1.0)
    assert_close(bits(g["T"]), T, f"{name} T")
    assert_close(bits(g["Y"]), Y, f"{name} Y")
    del Y
    dX, dL1, dL2, _, _ = O.qlora_backward(X, dY, Wq, L1, L2, 1.0, T=T)
    assert_close(bits(g["dX"]), dX, f"{name} dX")
    assert_close(f32np(g["dL1"]), dL1, f"{name} dL1")
    assert_close(f32np(g["dL2"]), dL2, f"{name} dL2")


@pytest.mark.parametrize("which", ["up", "down"])
def test_llama7b_mlp_m4096_full(which):
    c = WL.config3()[which]
    _big_case(c, f"llama7b {which} M=4096")


@pytest.mark.parametrize("name", ["q", "gate", "down"])
def test_llama65b_block_linear_full(name):
    """One linear of each distinct shape of the 65B block (k, v, o share q's shape,
    up shares gate's) at M = 2048, every output compared."""
    _big_case(WL.config4_linear(name), f"llama65b {name} M=2048")


@pytest.mark.parametrize("M,K,N,r", [(300, 4160, 1000, 24), (1000, 640, 2048, 64), (130, 8192, 512, 8)])
def test_streaming_lora_products_partial_steps(M, K, N, r):
    """Shapes that take the streaming skinny kernel (reduction, row stride and r
    multiples of 8) with a partial last 64-column step, a partial last group of
    four steps, ragged 64-row tiles and a rank that leaves an MFMA column tile
    partly empty; every output of the layer against the oracle."""
    full_case(WL.layer_inputs(N, K, M, r, seed_base=777 + M + r, l2_std=0.1), 0.75, "streaming lora")


@pytest.mark.parametrize("M", [8, 96])
def test_stage_entry_points_match_fused_calls(M):
    """lora_down + fwd_t == fwd; grad_in + dx == the dX of bwd (same kernels, bitwise)."""
    q = qlib()
    inp = WL.layer_inputs(200, 256, M, 24, seed_base=4321 + M, l2_std=0.2)
    gq, _ = quantize_both(inp["W"])
    a = run_gpu(inp, 0.5, gq)
    X, L1, L2, dY = (inp[k].to(DEV) for k in ("X", "L1", "L2", "dY"))
    T = q.qlora_lora_down(X, L1)
    Y = q.qlora_linear_fwd_t(X, *gq, 200, T, L2, 0.5)
    G = q.qlora_lora_grad_in(dY, L2, 0.5)
    dX = q.qlora_linear_dx(dY, *gq, 256, G, L1)
    torch.cuda.synchronize()
    assert torch.equal(T, a["T"]) and torch.equal(Y, a["Y"]) and torch.equal(dX, a["dX"])


@pytest.mark.parametrize("loads", [1, 2, 4, 8, 16])
def test_read_probe_runs(loads):
    """The read-bandwidth probe (a measurement helper in its own library) reads a
    buffer whose XOR is not its trigger word, so the sink keeps its value; a
    ragged tail is accepted; the empty grid runs."""
    import bit_quantized_lora_blockwise_amd.probe as P
    buf = torch.zeros((1 << 20) + 48, dtype=torch.uint8, device=DEV)
    sink = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    P.read_probe(buf, sink, loads)
    P.empty_probe(1024, 256)
    torch.cuda.synchronize()
    assert int(sink.item()) == 7


def _partial_round_K(M):
    """A K whose dX product [M, K] (256 x 256 tiles) leaves the last round of its
    persistent grid (the CU count rounded down to a multiple of 8) partly empty."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grid = cus // 8 * 8
    rows = (M + 255) // 256
    cols = grid // rows + 1
    assert rows * cols > grid and (rows * cols) % grid != 0
    return 256 * cols


def test_backward_second_stream_matches_one_stream():
    """The dL1 / dL2 products run on the library's second stream when the dX
    product leaves a partial last round: same bits as the one-stream order
    (dX = None keeps them on the caller's stream) and as the dX stage entry
    point, and work the caller enqueues on its stream after the call sees the
    finished gradients."""
    q = qlib()
    M, N, r = 512, 256, 16
    K = _partial_round_K(M)
    inp = WL.layer_inputs(N, K, M, r, seed_base=9100, l2_std=0.1)
    gq, _ = quantize_both(inp["W"])
    X, L1, L2, dY = (inp[k].to(DEV) for k in ("X", "L1", "L2", "dY"))
    T = q.qlora_lora_down(X, L1)
    ref_dX = q.qlora_linear_dx(dY, *gq, K, q.qlora_lora_grad_in(dY, L2, 0.5), L1)
    _, ref_dL1, ref_dL2 = q.qlora_linear_bwd(X, dY, *gq, L1, L2, 0.5, T=T, dX=None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(2):
        with torch.cuda.stream(side):
            dX, dL1, dL2 = q.qlora_linear_bwd(X, dY, *gq, L1, L2, 0.5, T=T)
            copies = (dX.clone(), dL1.clone(), dL2.clone())
        side.synchronize()
        assert torch.equal(copies[0], ref_dX)
        assert torch.equal(copies[1], ref_dL1) and torch.equal(copies[2], ref_dL2)


def test_group_backward_second_stream_matches_segments():
    """Stacked backward (G = 2) with a partial last dX round: every segment's
    dL1 / dL2 equal qlora_linear_bwd of that segment bit for bit."""
    q = qlib()
    M, N, r, G = 512, 256, 16, 2
    K = _partial_round_K(M)
    segs = [WL.layer_inputs(N, K, M, r, seed_base=9200 + 10 * g, l2_std=0.1) for g in range(G)]
    X = segs[0]["X"].to(DEV)
    W = torch.cat([s["W"] for s in segs], 0).to(DEV)
    codes, c2, c1, _ = q.nf4_quantize_dq(W)
    L1 = torch.stack([s["L1"] for s in segs], 0).to(DEV)
    L2 = torch.stack([s["L2"] for s in segs], 0).to(DEV)
    dY = torch.cat([s["dY"] for s in segs], 1).to(DEV)
    _, gdL1, gdL2 = q.qlora_group_bwd(X, dY, codes, c2, c1, G, L1, L2, 0.5)
    torch.cuda.synchronize()
    cg = codes.view(G, N, K // 2)
    nb = N * K // 64
    for g in range(G):
        sg = (cg[g], c2.view(-1)[g * nb:(g + 1) * nb], c1.view(-1)[g * nb // 256:(g + 1) * nb // 256])
        _, dL1, dL2 = q.qlora_linear_bwd(X, dY[:, g * N:(g + 1) * N].contiguous(), *sg, L1[g], L2[g], 0.5, dX=None)
        torch.cuda.synchronize()
        assert torch.equal(gdL1.view(G, K, r)[g], dL1) and torch.equal(gdL2.view(G, r, N)[g], dL2)


# the decode forward at small X forms T's slices in the first work groups of its
# own launch; a tile's waves wait for them (bounded) or form them themselves.
# QLORA_DECODE_T_SPINS=0 cuts every wait to one poll, so that waves take their
# own path whenever the slices are not yet there: Y and T must be the same bits
# either way, and the same bits as T by the stand-alone product + Y by the stage
# entry point.  Ranks 8 (half of one column tile), 20 (a partial second tile)
# and 64; M = 1, 3 and 8; K down to one slice; ragged N.
DECODE_FUSED_T = [(1, 4096, 11008, 64), (3, 2880, 620, 8), (8, 2048, 1000, 20), (1, 448, 33, 64),
                  (4, 4096, 4096, 64)]


@pytest.mark.parametrize("M,K,N,r", DECODE_FUSED_T)
def test_decode_fused_T_own_path_same_bits(M, K, N, r, monkeypatch):
    import os
    q = qlib()
    print(f"[layer] decode fused T M={M} K={K} N={N} r={r}", flush=True)
    inp = WL.layer_inputs(N, K, M, r, seed_base=M * 7 + K + N + r, l2_std=0.3)
    gq, rq = quantize_both(inp["W"])
    X, L1, L2 = (inp[k].to(DEV) for k in ("X", "L1", "L2"))
    Ya, Ta = q.qlora_linear_fwd(X, *gq, N, L1, L2, 0.7, T_out=True)
    torch.cuda.synchronize()
    outs = []
    monkeypatch.setenv("QLORA_DECODE_T_SPINS", "0")
    for _ in range(3):
        Yb, Tb = q.qlora_linear_fwd(X, *gq, N, L1, L2, 0.7, T_out=True)
        torch.cuda.synchronize()
        outs.append((Yb, Tb))
    monkeypatch.delenv("QLORA_DECODE_T_SPINS")
    Ts = q.qlora_lora_down(X, L1)
    Ys = q.qlora_linear_fwd_t(X, *gq, N, Ts, L2, 0.7)
    torch.cuda.synchronize()
    for Yb, Tb in outs:
        assert_bitexact(bits(Tb), bits(Ta), "T, own path vs waited")
        assert_bitexact(bits(Yb), bits(Ya), "Y, own path vs waited")
    assert_bitexact(bits(Ta), bits(Ts), "T, in-launch slices vs stand-alone product")
    assert_bitexact(bits(Ya), bits(Ys), "Y, one launch vs stage entry point")
    Wq = O.nf4_dequantize(*rq, N, K)
    rY, rT = O.qlora_forward(bits(inp["X"]), Wq, bits(inp["L1"]), bits(inp["L2"]), 0.7)
    assert_close(bits(Ta), rT, f"decode fused T: T M={M} K={K} r={r}")
    assert_close(bits(Ya), rY, f"decode fused T: Y M={M} K={K} r={r}")


def test_decode_graph_replay_follows_new_inputs():
    """A decode forward captured once and replayed after X and L1 change in place
    (as a serving loop does) gives the eager call's Y and T on the new inputs,
    bit for bit, on every replay."""
    q = qlib()
    M, K, N, r = 1, 4096, 2000, 64
    inp = WL.layer_inputs(N, K, M, r, seed_base=777)
    gq, _ = quantize_both(inp["W"])
    X, L1, L2 = (inp[k].to(DEV) for k in ("X", "L1", "L2"))
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    T = torch.empty((M, r), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty((q.qlora_linear_fwd_workspace(M, K, N, r),), dtype=torch.uint8, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q.qlora_linear_fwd(X, *gq, N, L1, L2, 1.0, Y=Y, T_out=T, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.qlora_linear_fwd(X, *gq, N, L1, L2, 1.0, Y=Y, T_out=T, workspace=ws)
    gen = torch.Generator().manual_seed(99)
    for rep in range(4):
        X.copy_(torch.randn((M, K), generator=gen).to(torch.bfloat16))
        if rep % 2:
            L1.copy_((torch.randn((K, r), generator=gen) / 64).to(torch.bfloat16))
        torch.cuda.synchronize()
        Ye, Te = q.qlora_linear_fwd(X, *gq, N, L1, L2, 1.0, T_out=True)     # eager (one launch)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(T.view(torch.int16), Te.view(torch.int16)), rep
        assert torch.equal(Y.view(torch.int16), Ye.view(torch.int16)), rep
    del g
