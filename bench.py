"""Throughput of the W4A16 hot path on one MI355X.

One step = one pass of every stage of the path over synthetic inputs shaped
like the gate projection of a Qwen2.5-3B decoder layer (K = 2048, N = 11008,
group 64):

  pack     aq_quantize_pack of the bf16 weight                   (quantize + pack)
           and its symmetric variant aq_quantize_pack_sym
  gemv     aq_w4a16_gemv at M = 1, once on each of 40 distinct   (decode; 40 copies =
           packed weight copies, so every launch reads HBM         520 MB > the 256 MB MALL)
           and at M = 16 over the same copies (batched decode,
           the matrix-core kernel)
  gemm     aq_w4a16_gemm at M = 4096                             (prefill, bf16 MFMA; staged
           path: weights dequantized into a workspace, then the GEMM)
  absmean  aq_act_absmean over 65536 x 2048 calibration tokens   (AWQ statistic)
  search   aq_awq_search, 4096 tokens, 20 alphas, final pack     (AWQ search)
  fp4      aq_fp4_gemm at M = 1 (12 rotating copies of the 33 MB (FP4 decode)
           operands, graph-replayed) and M = 2048 on W[14336, 4096],
           and aq_fp4_quantize of an fp32 W[14336, 4096]          (FP4 encode)
  int8     aq_quantize_pack8, aq_w8a16_gemv at M = 1 (24          (8-bit variant)
           rotating copies, graph-replayed), aq_w8a16_gemm at
           M = 4096 (staged)
  layer    a whole Qwen2.5-3B decoder layer: norm-group AWQ of    (module-level path)
           q|k|v and gate|up (joint search, 65536-token abs-mean,
           4096-token search) plus plain packing of o and down;
           and the layer's decode GEMVs at M = 1 (q|k|v and
           gate|up fused: four launches per layer), averaged over
           a graph-replayed stack of 12 layers (536 MB)

Launches are bracketed by HIP events on the stream they run on (torch's current
stream, which the binding passes to the library): one event pair per launch (five
back-to-back calls for the short single-kernel rows: pack, pack_sym, pack8,
absmean, fp4_encode, averaged per call),
except the decode GEMV batches (INT4, INT8, FP4, the layer stack), which are
captured once in a HIP graph and replayed back to back between one pair (as a
decode loop does; eager Python launches would measure the binding's per-call
overhead instead of the kernel) and are averaged per launch.  The headline value is
the decode GEMV's HBM throughput (algorithmic bytes / average launch duration);
the GEMM's TFLOP/s and the other stages are reported beside it, and, as context
only, torch's dense bf16 matmul (the vendor BLAS) on the unquantized prefill
weight (`context_torch_bf16_mm_m4096`).

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A16 GEMV GB/s (M=1) + GEMM TFLOP/s (M=4096), K=2048 N=11008 g=64"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
K_, N_, G_ = 2048, 11008, 64
M_GEMM = 4096
N_COPIES = 40
FP4_N, FP4_K, FP4_M = 14336, 4096, 2048
CAL_T, CAL_SUB = 65536, 4096
LAYER_STACK = 12
N8_COPIES = 24
FP4_COPIES = 12


def gemv_bytes(m, n, k, g):
    return n * k // 2 + (n * k // g) * 5 + 2 * m * k + 4 * m * n


def pack_bytes(n, k, g):
    return 2 * n * k + n * k // 2 + (n * k // g) * 5


def fp4_bytes(m, n, k):
    return n * k // 2 + n * k // 16 + 2 * m * k + 4 * m * n


def _source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(kernel_key, files, launches_bytes):
    """HBM bytes per launch from the committed counter summary, if it matches the current source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(kernel_key)
    if not ent or ent.get("source_hash") != _source_hash(files):
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(budget_s=12.0):
    """The CPU oracle, untuned, on a bounded sample of the same workload (decode GEMV at M = 1)."""
    from oracle import int4
    from weight_only_bit_group_amd import synth
    try:
        import threadpoolctl
        threads = max(i["num_threads"] for i in threadpoolctl.threadpool_info()) or 1
    except Exception:  # pragma: no cover
        threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    wb = synth.layer_weight_bf16(1, "gate_proj")
    w = synth.bf16_bits_to_f32(wb)
    p, s, z = int4.quantize_pack(w, G_)
    x = synth.bf16_bits_to_f32(synth.layer_activations_bf16(1, 1, K_))
    calls, t0 = 0, time.perf_counter()
    while True:
        int4.forward(x, p, s, z, G_)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s or calls >= 200:
            break
    gbs = calls * gemv_bytes(1, N_, K_, G_) / el / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"oracle.int4.forward (fp64 dequantize + matvec) on the gate shape at M=1, "
                      f"{calls} calls in {el:.1f} s on {len(os.sched_getaffinity(0))} visible host cores "
                      f"(numpy elementwise single-threaded, BLAS {threads} threads)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the W4A16 path has no multi-GPU mode here (asked for --gpus {args.gpus}); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from weight_only_bit_group_amd import binding as B
    from weight_only_bit_group_amd import layer as L
    from weight_only_bit_group_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    print("[bench] setup", file=sys.stderr, flush=True)

    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)

    def weight_bf16(n, k):
        w = torch.randn((n, k), generator=gen, device=dev, dtype=torch.float32) * 0.02
        idx = torch.randint(0, n * k, (max(1, n * k // 1000),), generator=gen, device=dev)
        w.view(-1)[idx] *= 10.0
        return w.to(torch.bfloat16)

    def acts_bf16(m, k, outlier_ch, scale=20.0):
        x = torch.randn((m, k), generator=gen, device=dev, dtype=torch.float32)
        ch = torch.randperm(k, generator=gen, device=dev)[:outlier_ch]
        x[:, ch] *= scale
        return x.to(torch.bfloat16)

    # weights: the gate projection and 40 distinct packed copies for the rotating GEMV
    w_gate = weight_bf16(N_, K_)
    copies = []
    for i in range(N_COPIES):
        copies.append(B.aq_quantize_pack(w_gate if i == 0 else weight_bf16(N_, K_), G_))
    torch.cuda.synchronize()
    x1 = acts_bf16(1, K_, round(0.01 * K_))
    y1 = torch.empty((1, N_), dtype=torch.float32, device=dev)
    xg = acts_bf16(M_GEMM, K_, round(0.01 * K_))
    yg = torch.empty((M_GEMM, N_), dtype=torch.float32, device=dev)
    pk = [torch.empty_like(t) for t in copies[0]]
    # calibration activations: z * c_k, c_k = exp(1.5 N(0,1))
    ck = torch.exp(1.5 * torch.randn(K_, generator=gen, device=dev))
    xcal = (torch.randn((CAL_T, K_), generator=gen, device=dev) * ck).to(torch.bfloat16)
    sum_abs = torch.zeros(K_, dtype=torch.float64, device=dev)
    mean = torch.empty(K_, dtype=torch.float32, device=dev)
    ws_abs = torch.empty(B.aq_act_absmean_workspace(CAL_T, K_), dtype=torch.uint8, device=dev)
    B.aq_act_absmean(xcal, sum_abs, CAL_T, mean, ws_abs)
    absmean_host = mean.cpu().numpy().copy()
    xsub = xcal[:CAL_SUB].contiguous()
    ws_search = torch.empty(B.aq_awq_search_workspace(CAL_SUB, N_, K_, G_, 20), dtype=torch.uint8, device=dev)
    codes_np, bsc_np, ts = synth.random_fp4_operands(5, FP4_N, FP4_K)
    codes = torch.from_numpy(codes_np).to(dev)
    bsc = torch.from_numpy(bsc_np).to(dev)
    # FP4 decode: 12 distinct operand copies (12 x 33 MB > the 256 MB MALL), graph-replayed
    fp4_copies = [(codes, bsc)] + [tuple(torch.from_numpy(a).to(dev) for a in
                                         synth.random_fp4_operands(5 + i, FP4_N, FP4_K)[:2])
                                   for i in range(1, FP4_COPIES)]
    xf1 = acts_bf16(1, FP4_K, round(0.01 * FP4_K))
    xf2 = acts_bf16(FP4_M, FP4_K, round(0.01 * FP4_K))
    yf1 = torch.empty((1, FP4_N), dtype=torch.float32, device=dev)
    yf2 = torch.empty((FP4_M, FP4_N), dtype=torch.float32, device=dev)
    ws_gemm = torch.empty(B.aq_w4a16_gemm_workspace(M_GEMM, N_, K_, G_), dtype=torch.uint8, device=dev)
    ws_fp4 = torch.empty(B.aq_fp4_gemm_workspace(FP4_M, FP4_N, FP4_K), dtype=torch.uint8, device=dev)
    # FP4 encoder input: an fp32 weight of the FP4 shape, and its preallocated outputs
    w_fp4 = torch.randn((FP4_N, FP4_K), generator=gen, device=dev, dtype=torch.float32) * 0.02
    enc_out = dict(codes=torch.empty((FP4_N, FP4_K // 2), dtype=torch.uint8, device=dev),
                   block_scales=torch.empty((FP4_N, FP4_K // 16), dtype=torch.uint8, device=dev),
                   tensor_scale=torch.empty(1, dtype=torch.float32, device=dev),
                   workspace=torch.empty(B.aq_fp4_quantize_workspace(FP4_N, FP4_K), dtype=torch.uint8, device=dev))
    # a whole decoder layer: the seven linears as bf16 nn.Linear, RMSNorm weights, and its
    # quantized form (norm-group AWQ for q|k|v and gate|up, plain packing of o and down)
    layer_lin = {}
    for name, n, k in synth.LAYER_LINEARS:
        m = torch.nn.Linear(k, n, bias=False, device=dev, dtype=torch.bfloat16)
        with torch.no_grad():
            m.weight.copy_(weight_bf16(n, k))
        layer_lin[name] = m
    ln_w = torch.ones(K_, dtype=torch.float32, device=dev)

    def layer_awq():
        out = {}
        _, mods, _ = L.norm_group_awq(ln_w, [layer_lin[n] for n in ("q_proj", "k_proj", "v_proj")], xcal, G_, 20,
                                      CAL_SUB)
        out.update(zip(("q_proj", "k_proj", "v_proj"), mods))
        _, mods, _ = L.norm_group_awq(ln_w, [layer_lin[n] for n in ("gate_proj", "up_proj")], xcal, G_, 20,
                                      CAL_SUB)
        out.update(zip(("gate_proj", "up_proj"), mods))
        out["o_proj"] = L.quantize_linear(layer_lin["o_proj"], G_)
        out["down_proj"] = L.quantize_linear(layer_lin["down_proj"], G_)
        return out

    qlayer = layer_awq()
    # decode through a stack of LAYER_STACK layers (the AWQ-quantized layer first, then
    # plainly packed ones; 536 MB of packed weights, so every launch reads HBM), each as the
    # four GEMVs of its fused modules: q|k|v and gate|up (the consumers of one norm, stacked
    # with W4A16Linear.concat), o and down
    fused_groups = (("q_proj", "k_proj", "v_proj"), ("o_proj",), ("gate_proj", "up_proj"), ("down_proj",))
    k_in = {name: k for name, n, k in synth.LAYER_LINEARS}

    def fuse(mods):
        return [L.W4A16Linear.concat([mods[n] for n in names]) for names in fused_groups]

    stack = [fuse(qlayer)]
    for _ in range(LAYER_STACK - 1):
        stack.append(fuse({name: L.W4A16Linear(*B.aq_quantize_pack(weight_bf16(n, k), G_), G_)
                           for name, n, k in synth.LAYER_LINEARS}))
    x_in = [acts_bf16(1, k_in[names[0]], round(0.01 * k_in[names[0]])) for names in fused_groups]
    y_out = [torch.empty((1, f.out_features), dtype=torch.float32, device=dev) for f in stack[0]]

    def layer_decode():
        for lay in stack:
            for i, f in enumerate(lay):
                B.aq_w4a16_gemv(x_in[i], f.packed, f.scales, f.zeros, G_, out=y_out[i])

    side2 = torch.cuda.Stream()
    side2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side2):
        layer_decode()
    torch.cuda.current_stream().wait_stream(side2)
    torch.cuda.synchronize()
    layer_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(layer_graph):
        layer_decode()
    torch.cuda.synchronize()
    torch.cuda.synchronize()

    # context, not part of the path: torch's dense bf16 matmul (the vendor BLAS) on the prefill
    # shape with the unquantized bf16 weight, fp32 output like the W4A16 GEMM
    w_gate_t = w_gate.t()
    events = {k: [] for k in ("ref_mm", "pack", "pack_sym", "pack8", "gemv8", "gemm8", "gemv", "gemv16", "gemm", "absmean", "search", "fp4_gemv", "fp4_gemm", "fp4_encode",
                              "layer_awq", "layer_gemv")}

    # Short single-kernel rows run REPEAT identical calls back to back between one event
    # pair (the host enqueues a call faster than the kernel runs, so the launches follow
    # each other on the GPU) and report the average per call: one event pair around one
    # ~20 us kernel would add the events' own overhead (several us) to it.
    REPEAT = 5
    repeated = ("pack", "pack_sym", "pack8", "absmean", "fp4_encode")

    def timed(name, record, fn):
        reps = REPEAT if name in repeated else 1
        if record:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            events[name].append((a, b))
        else:
            fn()

    # The decode GEMVs run back to back over the rotating copies, captured once in a HIP
    # graph (as a decode loop does): replaying it launches the 40 kernels without the
    # Python binding's per-call overhead (several microseconds, more than a launch), so the
    # event pair around the replay measures the GPU, not the interpreter.
    def gemv_batch():
        for (p, s, z) in copies:
            B.aq_w4a16_gemv(x1, p, s, z, G_, out=y1)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gemv_batch()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gemv_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gemv_graph):
        gemv_batch()
    torch.cuda.synchronize()

    # batched decode: the same 40 copies at M = 16 activation rows (the matrix-core path)
    x16 = acts_bf16(16, K_, round(0.01 * K_))
    y16 = torch.empty((16, N_), dtype=torch.float32, device=dev)

    def gemv16_batch():
        for (p, s, z) in copies:
            B.aq_w4a16_gemv(x16, p, s, z, G_, out=y16)

    side5 = torch.cuda.Stream()
    side5.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side5):
        gemv16_batch()
    torch.cuda.current_stream().wait_stream(side5)
    torch.cuda.synchronize()
    gemv16_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gemv16_graph):
        gemv16_batch()
    torch.cuda.synchronize()

    # INT8: the gate weight's 8-bit codes, 24 distinct copies for the rotating decode GEMV
    # (24 x 22.9 MB = 549 MB > 2 x the MALL), captured in a graph like the INT4 batch
    pk8 = B.aq_quantize_pack8(w_gate, G_)
    copies8 = [pk8] + [B.aq_quantize_pack8(weight_bf16(N_, K_), G_) for _ in range(N8_COPIES - 1)]
    ws8 = torch.empty(B.aq_w8a16_gemm_workspace(M_GEMM, N_, K_, G_), dtype=torch.uint8, device=dev)

    def gemv8_batch():
        for (c, s8, z8) in copies8:
            B.aq_w8a16_gemv(x1, c, s8, z8, G_, out=y1)

    side3 = torch.cuda.Stream()
    side3.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side3):
        gemv8_batch()
    torch.cuda.current_stream().wait_stream(side3)
    torch.cuda.synchronize()
    gemv8_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gemv8_graph):
        gemv8_batch()
    torch.cuda.synchronize()

    def fp4_gemv_batch():
        for (c4, b4) in fp4_copies:
            B.aq_fp4_gemm(xf1, c4, b4, ts, out=yf1)

    side4 = torch.cuda.Stream()
    side4.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side4):
        fp4_gemv_batch()
    torch.cuda.current_stream().wait_stream(side4)
    torch.cuda.synchronize()
    fp4_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(fp4_graph):
        fp4_gemv_batch()
    torch.cuda.synchronize()

    def step(record):
        timed("pack", record, lambda: B.aq_quantize_pack(w_gate, G_, packed=pk[0], scales=pk[1], zeros=pk[2]))
        timed("pack_sym", record, lambda: B.aq_quantize_pack(w_gate, G_, packed=pk[0], scales=pk[1], zeros=pk[2],
                                                             sym=True))
        timed("gemv", record, gemv_graph.replay)
        timed("gemv16", record, gemv16_graph.replay)
        timed("ref_mm", record, lambda: torch.mm(xg, w_gate_t, out_dtype=torch.float32))
        timed("pack8", record, lambda: B.aq_quantize_pack8(w_gate, G_, codes=pk8[0], scales=pk8[1], zeros=pk8[2]))
        timed("gemv8", record, gemv8_graph.replay)
        timed("gemm8", record, lambda: B.aq_w8a16_gemm(xg, *pk8, G_, out=yg, workspace=ws8))
        p, s, z = copies[0]
        timed("gemm", record, lambda: B.aq_w4a16_gemm(xg, p, s, z, G_, out=yg, workspace=ws_gemm))
        sum_abs.zero_()
        timed("absmean", record, lambda: B.aq_act_absmean(xcal, sum_abs, CAL_T, mean, ws_abs))
        timed("search", record, lambda: B.aq_awq_search(xsub, absmean_host, w_gate, G_, 20, ws_search))
        timed("fp4_gemv", record, fp4_graph.replay)
        timed("fp4_gemm", record, lambda: B.aq_fp4_gemm(xf2, codes, bsc, ts, out=yf2, workspace=ws_fp4))
        timed("fp4_encode", record, lambda: B.aq_fp4_quantize(w_fp4, **enc_out))
        timed("layer_awq", record, layer_awq)
        timed("layer_gemv", record, layer_graph.replay)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print("[bench] timed region done", file=sys.stderr, flush=True)

    ms = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in events.items()}
    for k in repeated:
        ms[k] /= REPEAT
    ms["gemv"] /= N_COPIES
    ms["gemv16"] /= N_COPIES
    ms["gemv8"] /= N8_COPIES
    ms["fp4_gemv"] /= FP4_COPIES
    ms["layer_gemv"] /= LAYER_STACK
    gemv_b = gemv_bytes(1, N_, K_, G_)
    gemv_gbs = gemv_b / (ms["gemv"] * 1e-3) / 1e9
    gemm_flop = 2.0 * M_GEMM * N_ * K_
    gemm_tf = gemm_flop / (ms["gemm"] * 1e-3) / 1e12
    search_flop = 20 * 2.0 * CAL_SUB * N_ * K_
    rows = {
        "pack": {"us": ms["pack"] * 1e3, "GB/s": pack_bytes(N_, K_, G_) / (ms["pack"] * 1e-3) / 1e9},
        "pack_sym": {"us": ms["pack_sym"] * 1e3, "GB/s": pack_bytes(N_, K_, G_) / (ms["pack_sym"] * 1e-3) / 1e9},
        "gemv_m1": {"us": ms["gemv"] * 1e3, "GB/s": gemv_gbs},
        "gemv_m16": {"us": ms["gemv16"] * 1e3,
                     "GB/s": gemv_bytes(16, N_, K_, G_) / (ms["gemv16"] * 1e-3) / 1e9},
        "gemm_m4096": {"us": ms["gemm"] * 1e3, "TFLOP/s": gemm_tf},
        "context_torch_bf16_mm_m4096": {"us": ms["ref_mm"] * 1e3,
                                        "TFLOP/s": gemm_flop / (ms["ref_mm"] * 1e-3) / 1e12},
        "pack8": {"us": ms["pack8"] * 1e3,
                  "GB/s": (2 * N_ * K_ + N_ * K_ + (N_ * K_ // G_) * 5) / (ms["pack8"] * 1e-3) / 1e9},
        "gemv8_m1": {"us": ms["gemv8"] * 1e3,
                     "GB/s": (N_ * K_ + (N_ * K_ // G_) * 5 + 2 * K_ + 4 * N_) / (ms["gemv8"] * 1e-3) / 1e9},
        "gemm8_m4096": {"us": ms["gemm8"] * 1e3, "TFLOP/s": gemm_flop / (ms["gemm8"] * 1e-3) / 1e12},
        "absmean": {"us": ms["absmean"] * 1e3, "GB/s": 2.0 * CAL_T * K_ / (ms["absmean"] * 1e-3) / 1e9},
        "awq_search": {"ms": ms["search"], "TFLOP/s": search_flop / (ms["search"] * 1e-3) / 1e12},
        "fp4_gemv_m1": {"us": ms["fp4_gemv"] * 1e3,
                        "GB/s": fp4_bytes(1, FP4_N, FP4_K) / (ms["fp4_gemv"] * 1e-3) / 1e9},
        "fp4_encode": {"us": ms["fp4_encode"] * 1e3,
                       "GB/s": (4 * FP4_N * FP4_K + FP4_N * FP4_K // 2 + FP4_N * FP4_K // 16)
                       / (ms["fp4_encode"] * 1e-3) / 1e9},
        "layer_awq": {"ms": ms["layer_awq"]},
        "layer_gemv_m1": {"us": ms["layer_gemv"] * 1e3,
                          "GB/s": sum(gemv_bytes(1, n, k, G_) for _, n, k in synth.LAYER_LINEARS)
                          / (ms["layer_gemv"] * 1e-3) / 1e9},
        "fp4_gemm_m2048": {"us": ms["fp4_gemm"] * 1e3,
                           "TFLOP/s": 2.0 * FP4_M * FP4_N * FP4_K / (ms["fp4_gemm"] * 1e-3) / 1e12},
    }
    rows = {k: {kk: round(vv, 3) for kk, vv in v.items()} for k, v in rows.items()}
    gemv_src = ["weight_only_bit_group_amd/csrc/w4a16_gemv.hip", "weight_only_bit_group_amd/csrc/aq_device.h"]
    gemm_src = ["weight_only_bit_group_amd/csrc/mfma_gemm.hip", "weight_only_bit_group_amd/csrc/aq_device.h"]
    out = {
        "metric": METRIC,
        "value": round(gemv_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Qwen2.5-3B gate_proj W4A16: K=2048 N=11008 g=64; GEMV M=1 over 40 rotating "
                               "packed copies, GEMM M=4096, abs-mean 65536x2048, AWQ search T=4096 x 20 alphas, "
                               "FP4 [14336,4096] M=1 (12 rotating copies) / M=2048",
                   "K": K_, "N": N_, "group": G_, "gemv_M": 1, "gemm_M": M_GEMM, "rotating_copies": N_COPIES},
        "roofline": {"bound": "hbm", "achieved": round(gemv_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gemv_gbs / HBM_PEAK_GBS, 4),
                     "traffic": _traffic("w4a16_gemv_m1", gemv_src, gemv_b)},
        "gemm": {"value": round(gemm_tf, 2), "unit": "TFLOP/s",
                 "roofline": {"bound": "mfma", "achieved": round(gemm_tf, 2), "peak": BF16_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(gemm_tf / BF16_PEAK_TFLOPS, 4),
                              "traffic": _traffic("w4a16_gemm_m4096", gemm_src, None)}},
        "rows": rows,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
