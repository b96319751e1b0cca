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

  widen    the configurations around the headline shape: decode at M = 4 and at group
           128 (M = 1, 4, 16); the prefill GEMM at M = 512 (gate and q shapes); a
           36-layer stream of all seven linears (random weights packed on the device,
           1.6 GB) at M = 512 and M = 4096; FP4 on the [4096, 14336] (K = 14336) shape

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

Beside the path (outside the timed steps) the run measures the ceilings the roofline
fractions are also stated against (libaq_probe.so): an empty kernel, a pure streaming
read of exactly the decode GEMV's bytes at its launch shape and at the best of a few
shapes, and MFMA-only loops.  Every row reports the mean over the timed steps and the
10th / 50th / 90th percentiles of the per-step values.

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
PRE_LAYERS = 36
PRE_M = (512, 4096)


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


def _timeit(fn, budget_s, max_calls=1000):
    """(calls, seconds) of fn repeated until budget_s has passed (at least once)."""
    calls, t0 = 0, time.perf_counter()
    while True:
        fn()
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s or calls >= max_calls:
            return calls, el


def cpu_baseline(budget_s=6.0):
    """The CPU oracle, untuned, timed on this host on bounded samples of the same workloads.

    `value` is the headline's decode GEMV (gate shape, M = 1); `items` holds the other
    configurations, each with the sample it ran and, where only part of the workload ran,
    the stated extrapolation to the whole.
    """
    from oracle import awq, fp4, int4, stats
    from weight_only_bit_group_amd import synth
    try:
        import threadpoolctl
        threads = max(i["num_threads"] for i in threadpoolctl.threadpool_info()) or 1
    except Exception:  # pragma: no cover
        threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    cores = len(os.sched_getaffinity(0))
    items = {}
    w = {name: synth.bf16_bits_to_f32(synth.layer_weight_bf16(1, name)) for name, _, _ in synth.LAYER_LINEARS}
    packs = {name: int4.quantize_pack(w[name], G_) for name in w}

    # C2 headline: decode GEMV, gate shape, M = 1
    p, s_, z = packs["gate_proj"]
    x = synth.bf16_bits_to_f32(synth.layer_activations_bf16(1, 1, K_))
    calls, el = _timeit(lambda: int4.forward(x, p, s_, z, G_), budget_s, 200)
    gbs = calls * gemv_bytes(1, N_, K_, G_) / el / 1e9

    # C1: the 256 x 256 fp32 single linear, pack + M = 8 product
    c1 = synth.single_linear(0)
    xc1 = synth.bf16_bits_to_f32(c1["X"])
    calls1, el1 = _timeit(lambda: int4.forward(xc1, *int4.quantize_pack(c1["W"], 128), 128), 1.0)
    items["c1_pack_and_gemm"] = {"ms": round(el1 / calls1 * 1e3, 3), "sample": "full (W 256x256 fp32, X 8x256)"}

    # C2: pack of the gate weight, and the seven linears of one layer at M = 1
    t0 = time.perf_counter()
    int4.quantize_pack(w["gate_proj"], G_)
    el_pack = time.perf_counter() - t0
    items["c2_pack_gate"] = {"ms": round(el_pack * 1e3, 1),
                             "GB/s": round(pack_bytes(N_, K_, G_) / el_pack / 1e9, 4), "sample": "full, one call"}
    xs = {k: synth.bf16_bits_to_f32(synth.layer_activations_bf16(1, 1, k)) for k in (2048, 11008)}
    t0 = time.perf_counter()
    for name, n, k in synth.LAYER_LINEARS:
        int4.forward(xs[k], *packs[name], G_)
    el_layer = time.perf_counter() - t0
    lb = sum(gemv_bytes(1, n, k, G_) for _, n, k in synth.LAYER_LINEARS)
    items["c2_layer_gemv_m1"] = {"ms": round(el_layer * 1e3, 1), "GB/s": round(lb / el_layer / 1e9, 4),
                                 "sample": "full: the 7 linears of one layer at M = 1, g = 64"}

    # C3: prefill GEMM at M = 4096 on the gate linear (one of the 7 x 36 linears)
    x3 = synth.bf16_bits_to_f32(synth.layer_activations_bf16(3, 4096, K_))
    t0 = time.perf_counter()
    int4.forward(x3, p, s_, z, G_)
    el3 = time.perf_counter() - t0
    items["c3_gemm_gate_m4096"] = {"ms": round(el3 * 1e3, 1),
                                   "GFLOP/s": round(2.0 * 4096 * N_ * K_ / el3 / 1e9, 2),
                                   "sample": "stated subset: the gate linear only (1 of 252 in the 36-layer stream)"}

    # C4: abs-mean statistic (exact fsum per channel) and the alpha search
    xcal = synth.bf16_bits_to_f32(synth.calibration_rows_bf16(4, 8192, K_))
    t0 = time.perf_counter()
    stats.absmean(xcal)
    el4 = time.perf_counter() - t0
    items["c4_absmean"] = {"ms_extrapolated": round(el4 * 8 * 1e3, 1),
                           "GB/s": round(2.0 * 8192 * K_ / el4 / 1e9, 4),
                           "sample": "8192 of the 65536 tokens (x8 extrapolated to the whole)"}
    xsub = xcal[:4096]
    m = stats.absmean(xsub)
    for tag, name in (("q", "q_proj"), ("gate", "gate_proj")):
        # one candidate of the grid (alpha = 0.35): scales, qdq error matrix, output MSE
        t0 = time.perf_counter()
        awq.output_mse(xsub, awq.error_matrix(w[name], G_, awq.candidate_scale(m, 0.35)))
        el_a = time.perf_counter() - t0
        n_, k_ = synth.LINEAR_SHAPES[name]
        items[f"c4_search_{tag}"] = {"ms_extrapolated": round(el_a * 20 * 1e3, 1),
                                     "sample": f"{name} [{n_}, {k_}], T = 4096: one of the 20 alphas timed, "
                                               f"x20 extrapolated to the grid"}

    # C5: FP4 decode at M = 1 on both MLP shapes, M = 2048 on 256 output rows
    for tag, (n5, k5) in (("up", (FP4_N, FP4_K)), ("down", (FP4_K, FP4_N))):
        c5, b5, t5 = synth.random_fp4_operands(5, n5, k5)
        x5 = synth.bf16_bits_to_f32(synth.layer_activations_bf16(5, 1, k5))
        t0 = time.perf_counter()
        fp4.forward(x5, c5, b5, t5)
        el5 = time.perf_counter() - t0
        items[f"c5_fp4_gemv_m1_{tag}"] = {"ms": round(el5 * 1e3, 1),
                                          "GB/s": round(fp4_bytes(1, n5, k5) / el5 / 1e9, 4),
                                          "sample": f"full: W [{n5}, {k5}] (N, K), M = 1"}
    c5, b5, t5 = synth.random_fp4_operands(5, FP4_N, FP4_K)
    x5 = synth.bf16_bits_to_f32(synth.layer_activations_bf16(5, 2048, FP4_K))
    t0 = time.perf_counter()
    fp4.forward(x5, c5[:256], b5[:256], t5)
    el5 = time.perf_counter() - t0
    items["c5_fp4_gemm_m2048"] = {"GFLOP/s": round(2.0 * 2048 * 256 * FP4_K / el5 / 1e9, 2),
                                  "sample": "stated subset: 256 of the 14336 output rows at M = 2048"}
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"oracle.int4.forward (fp64 dequantize + matvec) on the gate shape at M=1, "
                      f"{calls} calls in {el:.1f} s on {cores} visible host cores "
                      f"(numpy elementwise single-threaded, BLAS {threads} threads)",
            "host_cores_visible": cores, "blas_threads": int(threads), "items": items}


def _graph(fn):
    """fn captured once in a HIP graph (after one eager run on a side stream)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_us(graph, launches, reps=20):
    """Per-launch microseconds of a graph of `launches` back-to-back kernels (median of reps)."""
    import torch
    vals = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        b.synchronize()
        vals.append(a.elapsed_time(b) * 1e3 / launches)
    return float(np.median(vals))


def ceilings(dev):
    """Measured ceilings (libaq_probe.so), outside the timed steps."""
    import torch
    from weight_only_bit_group_amd import probe
    stream = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(256, dtype=torch.float32, device=dev)
    out = {}
    g = _graph(lambda: [probe.empty(1, 64, torch.cuda.current_stream().cuda_stream) for _ in range(N_COPIES)])
    out["empty_kernel_us"] = round(_replay_us(g, N_COPIES), 3)
    gemv_grid = ((N_ + 3) // 4 + 3) // 4     # the M = 1 gate GEMV: four rows per wave, four waves per block
    g = _graph(lambda: [probe.empty(gemv_grid, 256, torch.cuda.current_stream().cuda_stream)
                        for _ in range(N_COPIES)])
    out["empty_kernel_gemv_grid_us"] = round(_replay_us(g, N_COPIES), 3)
    nbytes = gemv_bytes(1, N_, K_, G_)
    stride = (nbytes + 255) // 256 * 256
    buf = torch.randint(0, 255, (N_COPIES * stride,), dtype=torch.uint8, device=dev)
    units = nbytes // 16

    def read_graph(blocks, unroll):
        return _graph(lambda: [probe.stream_read(buf.data_ptr() + i * stride, nbytes, blocks, unroll, sink.data_ptr(),
                                                 torch.cuda.current_stream().cuda_stream)
                               for i in range(N_COPIES)])

    sweep = {}
    for blocks in (256, 512, gemv_grid, 1024, 2048):
        need = -(-units // (blocks * 256))
        unroll = next((u for u in (1, 2, 4, 5, 8) if u >= need), 8)
        sweep[f"{blocks}x256_u{unroll}"] = round(_replay_us(read_graph(blocks, unroll), N_COPIES), 3)
    at_shape = sweep[f"{gemv_grid}x256_u{next(u for u in (1, 2, 4, 5, 8) if u >= -(-units // (gemv_grid * 256)))}"]
    best = min(sweep.values())
    out["stream_read_bytes"] = nbytes
    out["stream_read_us"] = sweep
    out["stream_read_gemv_shape_us"] = at_shape
    out["stream_read_gemv_shape_GBs"] = round(nbytes / (at_shape * 1e-6) / 1e9, 1)
    out["stream_read_best_us"] = best
    out["stream_read_best_GBs"] = round(nbytes / (best * 1e-6) / 1e9, 1)
    del buf
    # a large streaming read (HBM bandwidth with the launch amortised): 4 GiB in one launch
    big = torch.empty(1 << 32, dtype=torch.uint8, device=dev)
    big.fill_(1)
    torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        probe.stream_read(big.data_ptr(), big.numel(), 4096, 8, sink.data_ptr(), stream)
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3)
    out["stream_read_4GiB_GBs"] = round(big.numel() / float(np.median(ts)) / 1e9, 1)
    del big
    # MFMA-only loops: 2 and 4 waves per SIMD (512 / 1024 blocks of 4 waves on 256 CUs)
    for big_tile, name, accs in ((True, "32x32x16", 4), (False, "16x16x32", 8)):
        flop_per = 2 * 32 * 32 * 16 if big_tile else 2 * 16 * 16 * 32
        for blocks in (512, 1024):
            iters = 4096
            ts = []
            for _ in range(4):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                probe.mfma_loop(big_tile, blocks, iters, sink.data_ptr(), stream)
                b.record()
                b.synchronize()
                ts.append(a.elapsed_time(b) * 1e-3)
            flops = blocks * 4 * iters * accs * flop_per
            out[f"mfma_{name}_{blocks // 256}w_TFLOPs"] = round(flops / float(np.median(ts)) / 1e12, 1)
    out["mfma_best_TFLOPs"] = max(v for k, v in out.items() if k.startswith("mfma_"))
    return out


def _pct(vals):
    v = np.asarray(vals, dtype=np.float64)
    return float(v.mean()), float(np.percentile(v, 10)), float(np.percentile(v, 50)), float(np.percentile(v, 90))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true")
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

    def acts_bf16(m, k, outlier_ch=None, scale=20.0):
        x = torch.randn((m, k), generator=gen, device=dev, dtype=torch.float32)
        ch = torch.randperm(k, generator=gen, device=dev)[:round(0.01 * k) if outlier_ch is None else outlier_ch]
        x[:, ch] *= scale
        return x.to(torch.bfloat16)

    # weights: the gate projection and 40 distinct packed copies for the rotating GEMV, at
    # group 64 and (other weights) at group 128
    w_gate = weight_bf16(N_, K_)
    copies = [B.aq_quantize_pack(w_gate if i == 0 else weight_bf16(N_, K_), G_) for i in range(N_COPIES)]
    copies128 = [B.aq_quantize_pack(weight_bf16(N_, K_), 128) for _ in range(N_COPIES)]
    torch.cuda.synchronize()
    x1 = acts_bf16(1, K_)
    y1 = torch.empty((1, N_), dtype=torch.float32, device=dev)
    xg = acts_bf16(M_GEMM, K_)
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
    # FP4 on both MLP shapes: [14336, 4096] ("up", the headline FP4 shape) and [4096, 14336]
    # ("down", K = 14336); 12 distinct operand copies each (12 x 33 MB > the 256 MB MALL)
    fp4_ops = {}
    for tag, (n5, k5) in (("up", (FP4_N, FP4_K)), ("down", (FP4_K, FP4_N))):
        ops = [tuple(torch.from_numpy(a).to(dev) for a in synth.random_fp4_operands(5 + i, n5, k5)[:2])
               for i in range(FP4_COPIES)]
        fp4_ops[tag] = dict(n=n5, k=k5, ops=ops, x1=acts_bf16(1, k5), xm=acts_bf16(FP4_M, k5),
                            y1=torch.empty((1, n5), dtype=torch.float32, device=dev),
                            ym=torch.empty((FP4_M, n5), dtype=torch.float32, device=dev),
                            ws=torch.empty(B.aq_fp4_gemm_workspace(FP4_M, n5, k5), dtype=torch.uint8, device=dev))
    ts = float(synth.random_fp4_operands(5, FP4_N, FP4_K)[2])
    ws_gemm = torch.empty(B.aq_w4a16_gemm_workspace(M_GEMM, N_, K_, G_), dtype=torch.uint8, device=dev)
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
    x_in = [acts_bf16(1, k_in[names[0]]) for names in fused_groups]
    y_out = [torch.empty((1, f.out_features), dtype=torch.float32, device=dev) for f in stack[0]]

    def layer_decode():
        for lay in stack:
            for i, f in enumerate(lay):
                B.aq_w4a16_gemv(x_in[i], f.packed, f.scales, f.zeros, G_, out=y_out[i])

    layer_graph = _graph(layer_decode)

    # the prefill stream: 36 layers x 7 linears of random bf16 weights, packed on the device
    # (1.6 GB of packed triples), run at M = 512 and M = 4096 (staged path, one shared
    # staging workspace sized for the largest linear)
    pre_stack = []
    for _ in range(PRE_LAYERS):
        lay = []
        for name, n, k in synth.LAYER_LINEARS:
            wl = weight_bf16(n, k)
            lay.append(B.aq_quantize_pack(wl, G_))
            del wl
        pre_stack.append(lay)
    # The same stream in the module-swap form: q|k|v and gate|up each one stacked linear (the
    # packed triples concatenated along N, as W4A16Linear.concat does), four GEMM launches per
    # layer instead of seven, the same FLOPs
    def _cat(trips):
        return tuple(torch.cat([t[i] for t in trips]) for i in range(3))

    pre_fused = [[_cat(lay[0:3]), lay[3], _cat(lay[4:6]), lay[6]] for lay in pre_stack]
    fused_linears = ((2560, 2048), (2048, 2048), (22016, 2048), (2048, 11008))
    # staging matrix (M = 4096) and K-slice partials (the few-tile shapes), the largest of every call
    ws_pre = torch.empty(max(B.aq_w4a16_gemm_workspace(mm, n, k, G_) for mm in PRE_M
                             for n, k in [(n, k) for _, n, k in synth.LAYER_LINEARS] + list(fused_linears)),
                         dtype=torch.uint8, device=dev)
    pre_x = {mm: {k: acts_bf16(mm, k) for k in (2048, 11008)} for mm in PRE_M}
    pre_y = {mm: {n: torch.empty((mm, n), dtype=torch.float32, device=dev) for n in (2048, 256, 11008, 2560, 22016)}
             for mm in PRE_M}

    def prefill(mm):
        def run():
            for lay in pre_stack:
                for (name, n, k), trip in zip(synth.LAYER_LINEARS, lay):
                    B.aq_w4a16_gemm(pre_x[mm][k], *trip, G_, out=pre_y[mm][n], workspace=ws_pre)
        return run

    def prefill_fused(mm):
        def run():
            for lay in pre_fused:
                for (n, k), trip in zip(fused_linears, lay):
                    B.aq_w4a16_gemm(pre_x[mm][k], *trip, G_, out=pre_y[mm][n], workspace=ws_pre)
        return run

    pre_graphs = {mm: _graph(prefill(mm)) for mm in PRE_M}
    pre_fused_graphs = {mm: _graph(prefill_fused(mm)) for mm in PRE_M}
    pre_flop = {mm: 2.0 * mm * PRE_LAYERS * sum(n * k for _, n, k in synth.LAYER_LINEARS) for mm in PRE_M}
    torch.cuda.synchronize()

    # context, not part of the path: torch's dense bf16 matmul (the vendor BLAS) on the prefill
    # shape with the unquantized bf16 weight, fp32 output like the W4A16 GEMM
    w_gate_t = w_gate.t()
    samples = {}

    # Short single-kernel rows run REPEAT identical calls back to back between one event
    # pair (the host enqueues a call faster than the kernel runs, so the launches follow
    # each other on the GPU) and report the average per call: one event pair around one
    # ~20 us kernel would add the events' own overhead (several us) to it.
    REPEAT = 5
    repeated = ("pack", "pack_sym", "pack8", "absmean", "fp4_encode", "gemm_m512", "gemm_m512_q")
    per_call = {}   # row -> launches per timed unit (graph batches)

    def timed(name, record, fn, launches=1):
        reps = REPEAT if name in repeated else 1
        if record:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            samples.setdefault(name, []).append((a, b))
            per_call[name] = reps * launches
        else:
            fn()

    # The decode GEMVs run back to back over the rotating copies, captured once in a HIP
    # graph (as a decode loop does): replaying it launches the kernels without the Python
    # binding's per-call overhead (several microseconds, more than a launch), so the event
    # pair around the replay measures the GPU, not the interpreter.
    def gemv_graph(xm, cps, g):
        y = torch.empty((xm.shape[0], N_), dtype=torch.float32, device=dev)
        return _graph(lambda: [B.aq_w4a16_gemv(xm, p, s, z, g, out=y) for (p, s, z) in cps])

    x4 = acts_bf16(4, K_)
    x16 = acts_bf16(16, K_)
    decode_graphs = {"gemv": gemv_graph(x1, copies, G_), "gemv_m4": gemv_graph(x4, copies, G_),
                     "gemv16": gemv_graph(x16, copies, G_), "gemv_m1_g128": gemv_graph(x1, copies128, 128),
                     "gemv_m4_g128": gemv_graph(x4, copies128, 128), "gemv_m16_g128": gemv_graph(x16, copies128, 128)}

    # INT8: the gate weight's 8-bit codes, 24 distinct copies for the rotating decode GEMV
    # (24 x 22.9 MB = 549 MB > 2 x the MALL), captured in a graph like the INT4 batch
    pk8 = B.aq_quantize_pack8(w_gate, G_)
    copies8 = [pk8] + [B.aq_quantize_pack8(weight_bf16(N_, K_), G_) for _ in range(N8_COPIES - 1)]
    ws8 = torch.empty(B.aq_w8a16_gemm_workspace(M_GEMM, N_, K_, G_), dtype=torch.uint8, device=dev)
    gemv8_graph = _graph(lambda: [B.aq_w8a16_gemv(x1, c, s8, z8, G_, out=y1) for (c, s8, z8) in copies8])
    fp4_graphs = {tag: _graph(lambda f=f: [B.aq_fp4_gemm(f["x1"], c4, b4, ts, out=f["y1"]) for (c4, b4) in f["ops"]])
                  for tag, f in fp4_ops.items()}
    x512 = acts_bf16(512, K_)
    ws512 = torch.empty(B.aq_w4a16_gemm_workspace(512, N_, K_, G_), dtype=torch.uint8, device=dev)
    ws512q = torch.empty(B.aq_w4a16_gemm_workspace(512, 2048, 2048, G_), dtype=torch.uint8, device=dev)
    y512 = torch.empty((512, N_), dtype=torch.float32, device=dev)
    y512q = torch.empty((512, 2048), dtype=torch.float32, device=dev)
    q_pack = pre_stack[0][0]

    def step(record):
        timed("pack", record, lambda: B.aq_quantize_pack(w_gate, G_, packed=pk[0], scales=pk[1], zeros=pk[2]))
        timed("pack_sym", record, lambda: B.aq_quantize_pack(w_gate, G_, packed=pk[0], scales=pk[1], zeros=pk[2],
                                                             sym=True))
        for name, gr in decode_graphs.items():
            timed(name, record, gr.replay, N_COPIES)
        timed("ref_mm", record, lambda: torch.mm(xg, w_gate_t, out_dtype=torch.float32))
        timed("pack8", record, lambda: B.aq_quantize_pack8(w_gate, G_, codes=pk8[0], scales=pk8[1], zeros=pk8[2]))
        timed("gemv8", record, gemv8_graph.replay, N8_COPIES)
        timed("gemm8", record, lambda: B.aq_w8a16_gemm(xg, *pk8, G_, out=yg, workspace=ws8))
        p, s, z = copies[0]
        timed("gemm", record, lambda: B.aq_w4a16_gemm(xg, p, s, z, G_, out=yg, workspace=ws_gemm))
        timed("gemm_m512", record, lambda: B.aq_w4a16_gemm(x512, p, s, z, G_, out=y512, workspace=ws512))
        timed("gemm_m512_q", record, lambda: B.aq_w4a16_gemm(x512, *q_pack, G_, out=y512q, workspace=ws512q))
        sum_abs.zero_()
        timed("absmean", record, lambda: B.aq_act_absmean(xcal, sum_abs, CAL_T, mean, ws_abs))
        timed("search", record, lambda: B.aq_awq_search(xsub, absmean_host, w_gate, G_, 20, ws_search))
        for tag, f in fp4_ops.items():
            timed(f"fp4_gemv_{tag}", record, fp4_graphs[tag].replay, FP4_COPIES)
            timed(f"fp4_gemm_{tag}", record, lambda f=f: B.aq_fp4_gemm(f["xm"], *f["ops"][0], ts, out=f["ym"],
                                                                      workspace=f["ws"]))
        timed("fp4_encode", record, lambda: B.aq_fp4_quantize(w_fp4, **enc_out))
        timed("layer_awq", record, layer_awq)
        timed("layer_gemv", record, layer_graph.replay, LAYER_STACK)
        for mm in PRE_M:
            timed(f"prefill_m{mm}", record, pre_graphs[mm].replay, PRE_LAYERS)
            timed(f"prefill_fused_m{mm}", record, pre_fused_graphs[mm].replay, PRE_LAYERS)

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

    # per-launch (per-call, per-layer for the stacks) milliseconds of every step
    per = {k: [a.elapsed_time(b) / per_call[k] for a, b in v] for k, v in samples.items()}
    ms = {k: float(np.mean(v)) for k, v in per.items()}

    def row(name, work=None, unit=None, scale=1.0):
        mean_, p10, p50, p90 = _pct(per[name])
        r = {"us": mean_ * 1e3, "p10_us": p10 * 1e3, "p50_us": p50 * 1e3, "p90_us": p90 * 1e3}
        if work is not None:
            r[unit] = work / (mean_ * 1e-3) / scale
        return r

    gemv_b = gemv_bytes(1, N_, K_, G_)
    gemv_gbs = gemv_b / (ms["gemv"] * 1e-3) / 1e9
    gemm_flop = 2.0 * M_GEMM * N_ * K_
    gemm_tf = gemm_flop / (ms["gemm"] * 1e-3) / 1e12
    # the search scores each candidate through the Gram matrix (T > K): K^2 N multiply-adds per
    # candidate plus T K^2 once for H = X^T X (the direct form would be T K N per candidate)
    search_flop = 20 * 2.0 * N_ * K_ * K_ + 2.0 * CAL_SUB * K_ * K_
    layer_b = sum(gemv_bytes(1, n, k, G_) for _, n, k in synth.LAYER_LINEARS)
    rows = {
        "pack": row("pack", pack_bytes(N_, K_, G_), "GB/s", 1e9),
        "pack_sym": row("pack_sym", pack_bytes(N_, K_, G_), "GB/s", 1e9),
        "gemv_m1": row("gemv", gemv_b, "GB/s", 1e9),
        "gemv_m4": row("gemv_m4", gemv_bytes(4, N_, K_, G_), "GB/s", 1e9),
        "gemv_m16": row("gemv16", gemv_bytes(16, N_, K_, G_), "GB/s", 1e9),
        "gemv_m1_g128": row("gemv_m1_g128", gemv_bytes(1, N_, K_, 128), "GB/s", 1e9),
        "gemv_m4_g128": row("gemv_m4_g128", gemv_bytes(4, N_, K_, 128), "GB/s", 1e9),
        "gemv_m16_g128": row("gemv_m16_g128", gemv_bytes(16, N_, K_, 128), "GB/s", 1e9),
        "gemm_m4096": row("gemm", gemm_flop, "TFLOP/s", 1e12),
        "gemm_m512": row("gemm_m512", 2.0 * 512 * N_ * K_, "TFLOP/s", 1e12),
        "gemm_m512_q": row("gemm_m512_q", 2.0 * 512 * 2048 * 2048, "TFLOP/s", 1e12),
        "context_torch_bf16_mm_m4096": row("ref_mm", gemm_flop, "TFLOP/s", 1e12),
        "pack8": row("pack8", 2 * N_ * K_ + N_ * K_ + (N_ * K_ // G_) * 5, "GB/s", 1e9),
        "gemv8_m1": row("gemv8", N_ * K_ + (N_ * K_ // G_) * 5 + 2 * K_ + 4 * N_, "GB/s", 1e9),
        "gemm8_m4096": row("gemm8", gemm_flop, "TFLOP/s", 1e12),
        "absmean": row("absmean", 2.0 * CAL_T * K_, "GB/s", 1e9),
        "awq_search": dict(row("search", search_flop, "TFLOP/s", 1e12), form="gram",
                           direct_form_equiv_TFLOP_s=20 * 2.0 * CAL_SUB * N_ * K_ / (ms["search"] * 1e-3) / 1e12),
        "fp4_gemv_m1": row("fp4_gemv_up", fp4_bytes(1, FP4_N, FP4_K), "GB/s", 1e9),
        "fp4_gemv_m1_k14336": row("fp4_gemv_down", fp4_bytes(1, FP4_K, FP4_N), "GB/s", 1e9),
        "fp4_gemm_m2048": row("fp4_gemm_up", 2.0 * FP4_M * FP4_N * FP4_K, "TFLOP/s", 1e12),
        "fp4_gemm_m2048_k14336": row("fp4_gemm_down", 2.0 * FP4_M * FP4_N * FP4_K, "TFLOP/s", 1e12),
        "fp4_encode": row("fp4_encode", 4 * FP4_N * FP4_K + FP4_N * FP4_K // 2 + FP4_N * FP4_K // 16, "GB/s", 1e9),
        "layer_awq": row("layer_awq"),
        "layer_gemv_m1": row("layer_gemv", layer_b, "GB/s", 1e9),
    }
    for mm in PRE_M:
        rows[f"prefill_36x7_m{mm}"] = row(f"prefill_m{mm}", pre_flop[mm] / PRE_LAYERS, "TFLOP/s", 1e12)
        rows[f"prefill_36x7_m{mm}"]["ms_36_layers"] = ms[f"prefill_m{mm}"] * PRE_LAYERS
        rows[f"prefill_36x4_m{mm}"] = row(f"prefill_fused_m{mm}", pre_flop[mm] / PRE_LAYERS, "TFLOP/s", 1e12)
        rows[f"prefill_36x4_m{mm}"]["ms_36_layers"] = ms[f"prefill_fused_m{mm}"] * PRE_LAYERS
    rows = {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()} for k, v in rows.items()}
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
    if not args.no_ceilings:
        print("[bench] ceilings (empty kernel, streaming read, MFMA loop)", file=sys.stderr, flush=True)
        c = ceilings(dev)
        out["ceilings"] = c
        floor = c["stream_read_gemv_shape_GBs"]
        out["roofline"].update({"measured_peak": floor, "frac_measured": round(gemv_gbs / floor, 4),
                                "measured_peak_best_shape": c["stream_read_best_GBs"],
                                "frac_measured_best_shape": round(gemv_gbs / c["stream_read_best_GBs"], 4),
                                "measured_by": "pure streaming read of the same bytes at the GEMV's launch "
                                               "shape, 40 rotating buffers, graph-replayed"})
        out["gemm"]["roofline"].update({"measured_peak": c["mfma_best_TFLOPs"],
                                        "frac_measured": round(gemm_tf / c["mfma_best_TFLOPs"], 4),
                                        "measured_by": "bf16 MFMA-only loop (best of 32x32x16 / 16x16x32 at "
                                                       "2 and 4 waves per SIMD)"})
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
