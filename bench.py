#!/usr/bin/env python3
"""Throughput of the TTT-Linear scan on one MI355X.

One step is one call of ``ttt_linear_forward`` over the whole workload (every
(batch, head) scan over the full sequence), with the inputs already resident
in device memory.  With ``--pass train`` a step is one training pass instead:
the recording forward (``ttt_linear_forward_record``) followed by the backward
(``ttt_linear_backward``) from a fixed seeded dL/dout and dL/dW_final; the
roofline is then that of the backward kernel.  With ``--pass project`` a step
is the layer's input projections (``ttt_linear_project``, from a seeded bf16 x
[B,T,H*d] and stacked weights) followed by the scan; the roofline is the
projection kernel's (bf16 MFMA).  With ``--mlp`` a step is one call of
``ttt_mlp_forward``: the same scan with the two-layer inner model
W2 silu(W1 x) (W2 is the workload's W0; W1 is drawn from the workload's seed).  W warm-up steps run untimed; then exactly K steps are
timed between two device synchronisations, and each launch is also bracketed
by events on its stream for the per-kernel duration.  Rank 0 prints one JSON
line.

The default workload is the 256-scan per-token scan with bf16 inputs
(B=16, H=16, T=4096, d=64, hidden 1024).  The float64 CPU oracle is timed on
a bounded sample of the same workload (a subset of the scans at full length,
split over worker processes) as a reported baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from test_rnn_layer_ttt_amd.inputs import WORKLOADS, make_inputs  # noqa: E402

METRIC = "TTT-Linear scan token-heads/s at d=64 + % of HBM/FP32 roofline, 1 MI355X"
METRIC_PROJECT = ("TTT-Linear layer (input projections + scan) token-heads/s at d=64 "
                  "+ % of bf16 MFMA roofline of the projection kernel, 1 MI355X")
METRIC_TRAIN = ("TTT-Linear training pass (recording forward + backward) token-heads/s at d=64 "
                "+ % of HBM roofline of the backward kernel, 1 MI355X")
METRIC_MLP = ("TTT-MLP scan (two-layer inner model) token-heads/s at d=64 "
              "+ % of FP32/MFMA roofline, 1 MI355X")
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
FP32_VECTOR_PEAK_TFLOPS = 157.3  # 256 CU x 2.4 GHz x 256 flop/clk (packed FMA), published
FP32_MATRIX_PEAK_TFLOPS = 157.3  # MFMA fp32, published
BF16_MATRIX_PEAK_TFLOPS = 2500.0  # dense MFMA bf16, published


def algorithmic_work(x, mask=None):
    """Compulsory HBM bytes and flops of one launch (counted per token-head).

    With a SKIP/UPDATE mask a skipped chunk's tokens need only q and gate in
    and out written (2 d^2 flops for W_c q); the mask itself is read once."""
    B, H, T, d = x.q.shape
    n = B * H * T
    s_in = 2 if x.in_bf16 else 4
    per_tok_bytes = (4 * d + 1) * s_in + 4 * d        # q,k,v,gate,eta in; out fp32
    per_tok_flops = 6 * d * d + (4 * x.chunk * d if x.dual else 0)
    n_skip, extra = 0, 0
    if mask is not None:
        skip_tok = np.repeat(mask == 0, x.chunk, axis=-1)[..., :T]
        n_skip = int(skip_tok.sum())
        extra = mask.size
    skip_bytes = 2 * d * s_in + 4 * d
    nbytes = ((n - n_skip) * per_tok_bytes + n_skip * skip_bytes + B * H * 8 * d * d + H * 8 * d
              + extra)
    flops = (n - n_skip) * per_tok_flops + n_skip * 2 * d * d
    return n, nbytes, flops


def mlp_work(x):
    """Compulsory HBM bytes and flops of one two-layer launch (per token-head).

    Bytes: those of the linear scan, with two d x d weights in and out per
    scan.  Flops: seven d x d products per token (P1 k, P2 a, P2^T delta, the
    two rank-one updates, W1 q and W2 silu(W1 q)), 14 d^2; the dual form adds
    the in-chunk causal terms (the Gram matrices k.q and a.aq and their
    corrections, 8 chunk d)."""
    B, H, T, d = x.q.shape
    n = B * H * T
    s_in = 2 if x.in_bf16 else 4
    per_tok_bytes = (4 * d + 1) * s_in + 4 * d
    nbytes = n * per_tok_bytes + B * H * 16 * d * d + H * 8 * d
    flops = n * (14 * d * d + (8 * x.chunk * d if x.dual else 0))
    return n, nbytes, flops


def backward_work(x):
    """Compulsory HBM bytes and flops of one backward launch (per token-head).

    Bytes: q, k, v, gate, eta in their input type; dL/dout and the recorded
    delta_t in fp32; the recorded W at every 16-token tile start (4 d^2 bytes
    per tile, d^2/4 per token); dq, dk, dv, dgate (fp32) and deta out; per
    scan dL/dW_final in and dW0 out; per head gamma, beta in and their
    gradients out.  Flops: the 12 d^2 of the per-token gradient algebra
    (G_t k_t, G_t^T delta_t, W_{t-1}^T dz_t, W_t^T dy_t and the two rank-one
    updates of G); the replays of W a backward kernel makes from the record
    are its own choice and not counted.
    """
    B, H, T, d = x.q.shape
    n = B * H * T
    s_in = 2 if x.in_bf16 else 4
    per_tok_bytes = (4 * d + 1) * s_in + 4 * d + 4 * d + (d * d) // 4 + 16 * d + 4
    nbytes = n * per_tok_bytes + B * H * 8 * d * d + H * 16 * d
    return n, nbytes, n * 12 * d * d


def kernel_name(x, force_valu=False):
    """Which kernel family runs this workload."""
    import test_rnn_layer_ttt_amd as ttt
    d = x.q.shape[-1]
    return ttt.ttt_linear_kernel(d, ttt.mode_bits(x.ln, x.dual, x.in_bf16,
                                                  force_valu=force_valu), x.chunk)


def precision(x, kernel):
    """What the arithmetic of a forward launch is, in words."""
    if kernel == "scan_valu":
        return ("bf16 inputs widened to fp32; " if x.in_bf16 else "fp32 inputs; ") + \
            "fp32 vector-ALU arithmetic, fp32 state and output"
    if x.in_bf16:
        return ("bf16 inputs; d x d products on bf16 MFMA (16x16x32, 16x16x16) with the fp32 "
                "operands (W, delta, eta-scaled Gram entries) split into bf16 hi + lo and only "
                "the lo*lo term (~2^-17 relative) dropped; fp32 accumulation, fp32 LayerNorm "
                "pass, fp32 state and output")
    return ("fp32 inputs; d x d products on fp32 MFMA (16x16x4); fp32 LayerNorm pass, "
            "fp32 state and output")


def mlp_precision(x, kernel):
    """What the arithmetic of a two-layer launch is, in words."""
    if kernel == "mlp_valu":
        return ("bf16 inputs widened to fp32; " if x.in_bf16 else "fp32 inputs; ") + \
            "fp32 vector-ALU arithmetic, fp32 weights and output"
    return ("bf16 inputs; d x d products on bf16 MFMA with the fp32 operands (weights, "
            "activations, errors) split into bf16 hi + lo, the lo*lo term dropped in the "
            "64-deep contractions and kept in the 16-deep ones; fp32 accumulation, fp32 "
            "LayerNorm, fp32 weights and output")


def projection_work(x):
    """Flops and compulsory HBM bytes of one projection launch: x [B,T,hidden]
    and the weights [H,4d+1,hidden] in bf16, the five results out in the
    scan's input type; 2 flops per product of hidden = H d terms."""
    B, H, T, d = x.q.shape
    hidden, rows = H * d, H * (4 * d + 1)
    out_size = 2 if x.in_bf16 else 4
    nbytes = B * T * hidden * 2 + rows * hidden * 2 + B * T * rows * out_size
    return B * H * T, nbytes, 2 * B * T * hidden * rows


def measure_peaks(stream, launches=5):
    """Measured compute ceilings on this GPU, TFLOP/s (median of ``launches``):
    fp32 fused multiply-adds on the vector ALUs, compiled like the scan kernels
    (no packed-FP32 instructions), and the bf16 MFMA in its 16x16x32 and
    32x32x16 shapes (``bf16_mfma``: the faster).  None when the probe library
    is not built."""
    import ctypes

    import torch

    from test_rnn_layer_ttt_amd.build import PEAKS_LIB
    if not os.path.exists(PEAKS_LIB):
        return None
    lib = ctypes.CDLL(PEAKS_LIB)
    out = torch.empty(1024 * 256, dtype=torch.float32, device=stream.device)
    res = {}
    for name, fn, flops_fn, iters in (("fp32_vector", lib.ttt_peak_fp32, lib.ttt_peak_fp32_flops,
                                       20000),
                                      ("bf16_mfma_16x16x32", lib.ttt_peak_bf16_mfma,
                                       lib.ttt_peak_bf16_mfma_flops, 4000),
                                      ("bf16_mfma_32x32x16", lib.ttt_peak_bf16_mfma32,
                                       lib.ttt_peak_bf16_mfma32_flops, 4000)):
        fn.restype = ctypes.c_int32
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
        flops_fn.restype = ctypes.c_double
        flops_fn.argtypes = [ctypes.c_int32, ctypes.c_int32]
        blocks = 1024                     # 16 waves per CU on 256 CUs
        ms = []
        for i in range(launches + 1):
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            if fn(out.data_ptr(), blocks, iters, stream.cuda_stream) != 0:
                raise RuntimeError(f"peak probe {name} failed to launch")
            b_.record(stream)
            b_.synchronize()
            if i > 0:
                ms.append(a_.elapsed_time(b_))
        res[name] = round(flops_fn(blocks, iters) / (float(np.median(ms)) / 1e3) / 1e12, 1)
    res["bf16_mfma"] = max(res["bf16_mfma_16x16x32"], res["bf16_mfma_32x32x16"])
    return res


def roofline(x, kernel_ms, traffic, train=False, mask=None, project=False,
             hbm_measured_gbs=None, kernel=None, mlp=False, peaks=None):
    """Both ceilings of one launch and the fraction of the binding one.

    t_hbm = algorithmic bytes / the HBM peak and t_compute = algorithmic flops /
    the compute peak of that arithmetic: fp32 (157.3 TFLOP/s) for the per-token
    scan and the backward, whose flops are fp32 arithmetic; dense bf16 MFMA for
    the dual form's chunk contractions and the projections.  The binding roof
    is the one with the larger time; ``frac`` is measured against it, and
    ``frac_hbm`` / ``frac_compute`` give both.  With ``hbm_measured_gbs`` (a
    device copy timed in the same run) the HBM fraction is also given against
    that measured ceiling."""
    if project:
        n, nbytes, flops = projection_work(x)
        name, cbound, cpeak = "proj_mfma", "mfma", BF16_MATRIX_PEAK_TFLOPS
    elif mlp:
        n, nbytes, flops = mlp_work(x)
        name = kernel
        if name == "mlp_mfma":
            cbound, cpeak = "mfma", BF16_MATRIX_PEAK_TFLOPS
        else:
            cbound, cpeak = "alu", FP32_VECTOR_PEAK_TFLOPS
    elif train:
        n, nbytes, flops = backward_work(x)
        name, cbound, cpeak = kernel or "bwd_mfma", "alu", FP32_VECTOR_PEAK_TFLOPS
    else:
        n, nbytes, flops = algorithmic_work(x, mask)
        name = kernel or kernel_name(x)
        if x.dual and name == "scan_mfma":
            cbound, cpeak = "mfma", BF16_MATRIX_PEAK_TFLOPS
        else:
            cbound, cpeak = "alu", FP32_VECTOR_PEAK_TFLOPS
    sec = kernel_ms / 1e3
    gbs = nbytes / sec / 1e9
    tfs = flops / sec / 1e12
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_cmp = flops / (cpeak * 1e12)
    if t_hbm >= t_cmp:
        roof = dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(gbs / HBM_PEAK_GBS, 4))
    else:
        roof = dict(bound=cbound, achieved=round(tfs, 2), peak=cpeak, unit="TFLOP/s",
                    frac=round(tfs / cpeak, 4))
    roof.update(traffic=traffic, frac_hbm=round(gbs / HBM_PEAK_GBS, 4),
                frac_compute=round(tfs / cpeak, 4), compute_peak_tflops=cpeak,
                t_hbm_us=round(t_hbm * 1e6, 1), t_compute_us=round(t_cmp * 1e6, 1),
                algorithmic_bytes=nbytes, algorithmic_flops=flops)
    if hbm_measured_gbs:
        roof.update(hbm_measured_gbs=round(hbm_measured_gbs, 1),
                    frac_hbm_measured=round(gbs / hbm_measured_gbs, 4))
    if peaks:
        # the same arithmetic's ceiling measured on this GPU (fp32 without
        # packed instructions, as the kernels are built; bf16 MFMA)
        cm = peaks["bf16_mfma"] if cpeak == BF16_MATRIX_PEAK_TFLOPS else peaks["fp32_vector"]
        roof.update(compute_measured_tflops=cm, frac_compute_measured=round(tfs / cm, 4))
    return name, roof


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle, unmodified, on a bounded sample
# ---------------------------------------------------------------------------
_CPU_SAMPLE = None


_CPU_TRAIN = False
_CPU_MASK = None
_CPU_PROJ = None   # (x, w_proj) of the layer-pass workload, float32 holding bf16 values
_CPU_SILU = False
_CPU_MLP_W1 = None   # W1 of the sampled scans (two-layer inner model)


def _oracle_worker(idx):
    from threadpoolctl import threadpool_limits

    import oracle
    x = _CPU_SAMPLE
    with threadpool_limits(limits=1):
        if _CPU_PROJ is not None:
            # the oracle's projections of the sampled scans, in the scan's input type
            from test_rnn_layer_ttt_amd.inputs import round_to_bf16
            xs, ws = _CPU_PROJ
            pairs = x.meta["subset"]
            outs = [oracle.input_projections(xs[pairs[i][0]][None], ws[pairs[i][1]][None])
                    for i in idx]
            cat = [np.concatenate([o[j] for o in outs], axis=1) for j in range(5)]
            if x.in_bf16:
                cat = [round_to_bf16(a.astype(np.float32)) for a in cat]
            args = (*cat, x.W0[:, idx], x.gamma[idx], x.beta[idx])
        else:
            args = (x.q[:, idx], x.k[:, idx], x.v[:, idx], x.eta_logit[:, idx],
                    x.gate_logit[:, idx], x.W0[:, idx], x.gamma[idx], x.beta[idx])
        m = None if _CPU_MASK is None else _CPU_MASK[:, idx]
        if _CPU_MLP_W1 is not None:
            oracle.ttt_mlp_forward(*args[:5], _CPU_MLP_W1[:, idx], *args[5:], ln=x.ln,
                                   dual=x.dual, chunk=x.chunk)
            return len(idx)
        oracle.ttt_linear_forward(*args, ln=x.ln, dual=x.dual, chunk=x.chunk, update_mask=m,
                                  silu_qk=_CPU_SILU)
        if _CPU_TRAIN:
            dout, dWf = _cotangents(x)
            oracle.ttt_linear_backward(*args, dout[:, idx], dWf[:, idx], ln=x.ln, dual=x.dual,
                                       chunk=x.chunk, silu_qk=_CPU_SILU)
    return len(idx)


def _cotangents(x):
    from test_rnn_layer_ttt_amd.inputs import make_cotangents
    B, H, T, d = x.q.shape
    return make_cotangents(B, H, T, d, seed=x.meta.get("seed", 0) + 1000)


def cpu_baseline(x, n_scans, workers, train=False, mask=None, proj=None, mlp_W1=None):
    """Time the oracle on ``n_scans`` scans of ``x`` (full length) over ``workers``
    processes; with ``train`` its forward and its backward, as one training pass;
    with ``proj`` = (x, w_proj) its input projections of each scan, then the scan;
    with ``mlp_W1`` the two-layer scan (W2 = x.W0)."""
    import multiprocessing as mp
    global _CPU_SAMPLE, _CPU_TRAIN, _CPU_MASK, _CPU_PROJ, _CPU_MLP_W1
    _CPU_TRAIN = train
    _CPU_PROJ = proj
    B, H, T, d = x.q.shape
    n_scans = min(n_scans, B * H)
    step = max(1, (B * H) // n_scans)
    pairs = [(i // H, i % H) for i in range(0, B * H, step)][:n_scans]
    _CPU_SAMPLE = x.subset(pairs)
    _CPU_MLP_W1 = None if mlp_W1 is None else np.ascontiguousarray(
        mlp_W1[[p[0] for p in pairs], [p[1] for p in pairs]][None])
    _CPU_MASK = None if mask is None else np.ascontiguousarray(
        mask[[p[0] for p in pairs], [p[1] for p in pairs]][None])
    groups = [list(range(w, n_scans, workers)) for w in range(workers)]
    groups = [g for g in groups if g]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(len(groups)) as pool:
        done = sum(pool.map(_oracle_worker, groups))
    sec = time.perf_counter() - t0
    _CPU_SAMPLE = None
    _CPU_PROJ = None
    _CPU_MLP_W1 = None
    what = (", forward and backward" if train else
            ", input projections then the scan" if proj is not None else
            ", two-layer inner model" if mlp_W1 is not None else "")
    return dict(value=round(done * T / sec, 1), unit="token-heads/s", cores=len(groups),
                kind="oracle",
                sample=f"{done} of {B * H} scans at full length T={T}"
                       f"{what} (float64 NumPy, "
                       f"{len(groups)} processes x 1 BLAS thread, {sec:.1f} s wall)")


def host_cores():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---------------------------------------------------------------------------
def load_traffic(kernel, workload):
    """HBM traffic measured by rocprofv3 counters for this kernel and source, if recorded."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{kernel}|{workload}")
    except (OSError, ValueError):
        return None
    if not rec:
        return None
    from test_rnn_layer_ttt_amd.build import source_digest
    if rec.get("source_digest") != source_digest(kernel):
        return None        # the kernel changed since the counters were taken
    return rec.get("traffic_bytes")


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="h1024_T4096_bf16", choices=sorted(WORKLOADS))
    ap.add_argument("--pass", dest="pass_", default="forward",
                    choices=("forward", "train", "project"),
                    help="forward: the scan; train: recording forward + backward; "
                         "project: the layer's input projections from x, then the scan")
    ap.add_argument("--silu-qk", action="store_true",
                    help="the :mlp variant: SiLU on q and k before the inner model")
    ap.add_argument("--mlp", action="store_true",
                    help="the scan with the two-layer inner model W2 silu(W1 x) "
                         "(ttt_mlp_forward)")
    ap.add_argument("--chunk", type=int, default=None,
                    help="run the workload in the dual form with chunks of this many tokens")
    ap.add_argument("--force-valu", action="store_true",
                    help="run the vector-ALU kernels (TTT_FORCE_VALU) where the matrix-core "
                         "ones would apply")
    ap.add_argument("--update-rate", type=float, default=None,
                    help="dual-form workloads: seeded SKIP/UPDATE decisions per chunk, each "
                         "UPDATE with this probability (ttt_linear_forward_masked)")
    ap.add_argument("--cpu-scans", type=int, default=None,
                    help="scans of the workload the CPU oracle is timed on "
                         "(default 256 for the forward, 128 for a training pass)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="launches of the dominant kernel timed with a cache flush before each")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="MiB written between cold launches (L2 and the 256 MB MALL)")
    ap.add_argument("--valu-steps", type=int, default=5,
                    help="launches of the vector-ALU kernel timed beside the matrix-core one")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed region, run one device-to-device copy of this many "
                         "MiB: a kernel of known traffic that scales the HBM byte counters")
    args = ap.parse_args()
    global _CPU_SILU
    _CPU_SILU = args.silu_qk

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: measures one GPU only; the scans of a workload shard "
              "over GPUs by (batch, head) with no communication, and no multi-GPU figure "
              "is produced.", file=sys.stderr)
        sys.exit(2)

    W1_np = None
    if args.mlp:
        if args.pass_ != "forward" or args.silu_qk or args.update_rate is not None:
            print("bench.py: --mlp times the two-layer forward alone", file=sys.stderr)
            sys.exit(2)
        from test_rnn_layer_ttt_amd.inputs import make_mlp_inputs
        x, W1_np = make_mlp_inputs(args.workload)
    else:
        x = make_inputs(args.workload)
    if args.chunk is not None:
        if args.chunk < 1 or args.mlp:
            print("bench.py: --chunk takes a chunk >= 1 and the linear inner model",
                  file=sys.stderr)
            sys.exit(2)
        x.dual, x.chunk = True, args.chunk
    B, H, T, d = x.q.shape
    train = args.pass_ == "train"
    project = args.pass_ == "project"
    if project and (d != 64 or args.update_rate is not None or args.silu_qk):
        print("bench.py: --pass project covers d = 64 and the plain scan", file=sys.stderr)
        sys.exit(2)
    if args.cpu_scans is None:
        args.cpu_scans = 128 if train else 32 if project else 256
    mask_np = None
    if args.update_rate is not None:
        if train or not x.dual:
            print("bench.py: --update-rate needs a dual-form workload and the forward pass",
                  file=sys.stderr)
            sys.exit(2)
        from test_rnn_layer_ttt_amd.inputs import make_update_mask
        mask_np = make_update_mask(B, H, T, x.chunk, args.update_rate,
                                   seed=x.meta.get("seed", 0) + 2000)

    proj_np = None
    if project:
        from test_rnn_layer_ttt_amd.inputs import make_projection_case
        xp, wp, _ = make_projection_case(B, T, H * d, H, d, seed=x.meta.get("seed", 0) + 3000)
        proj_np = (xp, wp)

    # the CPU baseline runs before any GPU use (its workers are forked)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(x, args.cpu_scans if not args.mlp else min(args.cpu_scans, 64),
                           host_cores(), train, mask_np, proj_np if project else None, W1_np)

    import torch

    import test_rnn_layer_ttt_amd as ttt
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dt = torch.bfloat16 if x.in_bf16 else torch.float32
    f = lambda a: torch.from_numpy(a).to(dev).to(dt)
    q, k, v, el, gl = f(x.q), f(x.k), f(x.v), f(x.eta_logit), f(x.gate_logit)
    W0 = torch.from_numpy(x.W0).to(dev)
    gamma = torch.from_numpy(x.gamma).to(dev)
    beta = torch.from_numpy(x.beta).to(dev)
    out = torch.empty((B, H, T, d), dtype=torch.float32, device=dev)
    Wf = torch.empty_like(W0)
    stream = torch.cuda.current_stream(dev)
    mode = ttt.mode_bits(x.ln, x.dual, x.in_bf16, args.silu_qk, args.force_valu)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), el.data_ptr(), gl.data_ptr(),
            W0.data_ptr(), gamma.data_ptr(), beta.data_ptr(), out.data_ptr(), Wf.data_ptr())
    if project:
        # the projections overwrite q, k, v, eta and gate, which the scan then reads
        xt = torch.from_numpy(proj_np[0]).to(dev).to(torch.bfloat16)
        wt = torch.from_numpy(proj_np[1]).to(dev).to(torch.bfloat16)
        proj_np = None

        def projection():
            st = ttt.ttt_linear_project(xt.data_ptr(), wt.data_ptr(), None, q.data_ptr(),
                                        k.data_ptr(), v.data_ptr(), el.data_ptr(),
                                        gl.data_ptr(), B, T, H * d, H, d, mode,
                                        stream.cuda_stream)
            if st != ttt.TTT_OK:
                raise RuntimeError(f"ttt_linear_project: {ttt.ttt_status_string(st)}")

    if args.mlp:
        W1 = torch.from_numpy(W1_np).to(dev)
        W1f = torch.empty_like(W1)
        mptrs = ptrs[:5] + (W1.data_ptr(), W0.data_ptr()) + ptrs[6:9] + (W1f.data_ptr(),
                                                                         Wf.data_ptr())

        def forward(extra_mode=0):
            st = ttt.ttt_mlp_forward(*mptrs, B, H, T, d, mode | extra_mode, x.chunk,
                                     stream.cuda_stream)
            if st != ttt.TTT_OK:
                raise RuntimeError(f"ttt_mlp_forward: {ttt.ttt_status_string(st)}")
    elif mask_np is None:
        def forward():
            st = ttt.ttt_linear_forward(*ptrs, B, H, T, d, mode, x.chunk, stream.cuda_stream)
            if st != ttt.TTT_OK:
                raise RuntimeError(f"ttt_linear_forward: {ttt.ttt_status_string(st)}")
    else:
        mask_dev = torch.from_numpy(mask_np).to(dev)
        mptrs = ptrs[:8] + (mask_dev.data_ptr(),) + ptrs[8:]

        def forward():
            st = ttt.ttt_linear_forward_masked(*mptrs, B, H, T, d, mode, x.chunk,
                                               stream.cuda_stream)
            if st != ttt.TTT_OK:
                raise RuntimeError(f"ttt_linear_forward_masked: {ttt.ttt_status_string(st)}")

    if train:
        st, rec_bytes = ttt.ttt_linear_record_bytes(B, H, T, d, mode)
        ttt.check(st)
        record = torch.empty(rec_bytes, dtype=torch.uint8, device=dev)
        st, ws_bytes = ttt.ttt_linear_backward_workspace_bytes(B, H, d, mode)
        ttt.check(st)
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        dout_np, dWf_np = _cotangents(x)
        dout = torch.from_numpy(dout_np).to(dev)
        dWf = torch.from_numpy(dWf_np).to(dev)
        grads = [torch.empty((B, H, T, d), dtype=torch.float32, device=dev) for _ in range(4)]
        deta = torch.empty((B, H, T), dtype=torch.float32, device=dev)
        dW0 = torch.empty_like(W0)
        dgamma, dbeta = torch.empty_like(gamma), torch.empty_like(beta)
        no_ln = x.ln == "none"
        bptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), el.data_ptr(), gl.data_ptr(),
                 None if no_ln else gamma.data_ptr(), None if no_ln else beta.data_ptr(),
                 record.data_ptr(), rec_bytes, workspace.data_ptr(), ws_bytes,
                 dout.data_ptr(), dWf.data_ptr(),
                 *[g.data_ptr() for g in grads[:3]], deta.data_ptr(), grads[3].data_ptr(),
                 dW0.data_ptr(), None if no_ln else dgamma.data_ptr(),
                 None if no_ln else dbeta.data_ptr())

        def forward_record():
            st = ttt.ttt_linear_forward_record(*ptrs, record.data_ptr(), rec_bytes, B, H, T, d,
                                               mode, x.chunk if x.dual else 1,
                                               stream.cuda_stream)
            if st != ttt.TTT_OK:
                raise RuntimeError(f"ttt_linear_forward_record: {ttt.ttt_status_string(st)}")

        def backward():
            st = ttt.ttt_linear_backward(*bptrs, B, H, T, d, mode, x.chunk if x.dual else 1,
                                         stream.cuda_stream)
            if st != ttt.TTT_OK:
                raise RuntimeError(f"ttt_linear_backward: {ttt.ttt_status_string(st)}")

    # the dominant kernel of a step (the one the roofline is about) and the rest
    if train:
        steps = [("record", forward_record), ("main", backward)]
    elif project:
        steps = [("main", projection), ("scan", forward)]
    else:
        steps = [("main", forward)]

    for _ in range(args.warmup):
        for _, fn in steps:
            fn()
    torch.cuda.synchronize()

    # ---- timed region: exactly K back-to-back steps between two device syncs;
    # events on the launch stream around every launch (warm caches: a step's
    # inputs may still sit in L2 / the MALL from the step before)
    ev = {tag: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.steps)] for tag, _ in steps}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        for tag, fn in steps:
            ev[tag][i][0].record(stream)
            fn()
            ev[tag][i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {tag: [a.elapsed_time(b) for a, b in ev[tag]] for tag, _ in steps}
    kernel_ms = ms["main"]
    avg_kernel_ms = float(np.mean(kernel_ms))
    ms_per_step = wall * 1e3 / args.steps

    # ---- cold: the dominant kernel again, with >= 512 MiB written between
    # launches (outside the events) so that neither L2 nor the 256 MB MALL
    # holds its inputs
    cold_ms = []
    if args.cold_steps > 0:
        flush = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device=dev)
        main_fn = dict(steps)["main"]
        for i in range(args.cold_steps):
            flush.fill_(i & 0xFF)
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            main_fn()
            b_.record(stream)
            b_.synchronize()
            cold_ms.append(a_.elapsed_time(b_))
        del flush

    # ---- the measured HBM ceiling: a 1 GiB device-to-device copy (1 GiB read,
    # 1 GiB written), median of five
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    copy_ms = []
    for _ in range(6):
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record(stream)
        dst.copy_(src)
        b_.record(stream)
        b_.synchronize()
        copy_ms.append(a_.elapsed_time(b_))
    del src, dst
    copy_gbs = 2 * (1 << 30) / (float(np.median(copy_ms[1:])) / 1e3) / 1e9
    peaks = measure_peaks(stream)

    n_tok = B * H * T
    kernel = (ttt.ttt_linear_backward_kernel(d, mode, x.chunk if x.dual else 1) if train else
              "proj_mfma" if project else
              ttt.ttt_mlp_kernel(d, mode, x.chunk) if args.mlp else
              kernel_name(x, args.force_valu))
    traffic_key = args.workload + ("/backward" if train else "/project" if project else
                                   "/mlp" if args.mlp else "")
    if args.chunk is not None:
        traffic_key += f"/chunk{args.chunk}"
    if mask_np is not None:
        traffic_key = args.workload + f"/update{args.update_rate:g}"
    if args.silu_qk:
        traffic_key += "/silu"
    kname, roof = roofline(x, avg_kernel_ms, load_traffic(kernel, traffic_key), train, mask_np,
                           project, hbm_measured_gbs=copy_gbs, kernel=kernel, mlp=args.mlp,
                           peaks=peaks)

    mode_name = ("dual-form chunk %d" % x.chunk if x.dual else "per-token") + \
        {"st": "", "exact": ", exact LN Jacobian", "none": ", no LN"}[x.ln]
    med = lambda a: round(float(np.median(a)), 4)
    line = {
        "metric": (METRIC_TRAIN if train else METRIC_PROJECT if project else
                   METRIC_MLP if args.mlp else METRIC),
        "value": round(n_tok / (ms_per_step / 1e3), 1),
        "unit": "token-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if x.in_bf16 else "f32",
        "data": "synthetic",
        "cache": "warm",
        "config": {"workload": args.workload, "B": B, "H": H, "T": T, "d": d,
                   "hidden": H * d, "mode": mode_name,
                   "inputs": "bf16" if x.in_bf16 else "fp32", "state": "fp32",
                   "precision": mlp_precision(x, kname) if args.mlp else
                   precision(x, kname) if not (train or project) else
                   ("bf16 inputs" if x.in_bf16 else "fp32 inputs") +
                   "; fp32 accumulation, fp32 gradients",
                   "kernel": kname, "kernel_ms_avg": round(avg_kernel_ms, 4),
                   "kernel_ms_median": med(kernel_ms),
                   "kernel_ms_min": round(min(kernel_ms), 4),
                   "cu_occupied": f"{min(B * H, 256)}/256" if not project else "all",
                   "peaks_measured": dict(peaks or {}, hbm_copy_gbs=round(copy_gbs, 1)),
                   "timing": "value from the wall clock of the K back-to-back steps (warm "
                             "caches); roofline from the events' average over them; cold = "
                             f"{args.flush_mib} MiB written between launches"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if cold_ms:
        line["config"]["cold"] = {"kernel_ms_median": med(cold_ms),
                                  "kernel_ms_min": round(min(cold_ms), 4),
                                  "launches": len(cold_ms), "flush_mib": args.flush_mib,
                                  "token_heads_per_s": round(n_tok / (np.median(cold_ms) / 1e3),
                                                             1)}
    if args.silu_qk:
        line["config"]["variant"] = "mlp (SiLU on q and k)"
    if args.mlp:
        line["config"]["variant"] = "two-layer inner model W2 silu(W1 x), both d x d"
    if mask_np is not None:
        line["config"]["update_rate"] = args.update_rate
        line["config"]["chunks_updated"] = float(np.mean(mask_np != 0))
    if train:
        line["config"]["pass"] = "train: recording forward + backward"
        line["config"]["forward_record_ms_avg"] = round(float(np.mean(ms["record"])), 4)
    if project:
        line["config"]["pass"] = ("layer: input projections from x [B,T,hidden] bf16, "
                                  "then the scan")
        line["config"]["scan_ms_avg"] = round(float(np.mean(ms["scan"])), 4)
        # for scale: the same product as one plain library GEMM (torch.matmul,
        # hipBLASLt) into a [B*T, H*(4d+1)] bf16 result, no bias and none of the
        # projection kernel's five scattered output layouts; both operands
        # contiguous (the weights transposed once, outside the timing)
        x2 = xt.reshape(B * T, H * d)
        w2t = wt.reshape(H * (4 * d + 1), H * d).t().contiguous()
        y2 = torch.matmul(x2, w2t)
        torch.cuda.synchronize()
        lms = []
        for _ in range(max(3, min(args.steps, 20))):
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            torch.matmul(x2, w2t, out=y2)
            b_.record(stream)
            b_.synchronize()
            lms.append(a_.elapsed_time(b_))
        line["config"]["library_gemm_ms_median"] = med(lms)
        line["config"]["projection_ms_median"] = med(ms["main"])
        del x2, w2t, y2

    # ---- the vector-ALU kernel on the same inputs, for comparison (the
    # matrix-core kernel is what a call at d = 64 runs)
    if args.mlp and args.valu_steps > 0 and kname == "mlp_mfma":
        forward(ttt.TTT_FORCE_VALU)
        torch.cuda.synchronize()
        vms = []
        for _ in range(args.valu_steps):
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            forward(ttt.TTT_FORCE_VALU)
            b_.record(stream)
            b_.synchronize()
            vms.append(a_.elapsed_time(b_))
        _, vroof = roofline(x, float(np.median(vms)), None, kernel="mlp_valu", mlp=True)
        line["config"]["valu_kernel"] = {
            "kernel": "mlp_valu", "kernel_ms_median": med(vms),
            "token_heads_per_s": round(n_tok / (np.median(vms) / 1e3), 1),
            "bound": vroof["bound"], "frac": vroof["frac"], "frac_hbm": vroof["frac_hbm"],
            "frac_compute": vroof["frac_compute"], "precision": mlp_precision(x, "mlp_valu")}
    if (not train and not project and not args.mlp and mask_np is None
            and args.valu_steps > 0 and kname == "scan_mfma"):
        vmode = mode | ttt.TTT_FORCE_VALU

        def valu():
            st = ttt.ttt_linear_forward(*ptrs, B, H, T, d, vmode, x.chunk, stream.cuda_stream)
            if st != ttt.TTT_OK:
                raise RuntimeError(f"ttt_linear_forward: {ttt.ttt_status_string(st)}")
        valu()
        torch.cuda.synchronize()
        vms = []
        for _ in range(args.valu_steps):
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            valu()
            b_.record(stream)
            b_.synchronize()
            vms.append(a_.elapsed_time(b_))
        _, vroof = roofline(x, float(np.median(vms)), None, kernel="scan_valu")
        line["config"]["valu_kernel"] = {
            "kernel": "scan_valu", "kernel_ms_median": med(vms),
            "token_heads_per_s": round(n_tok / (np.median(vms) / 1e3), 1),
            "bound": vroof["bound"], "frac": vroof["frac"], "frac_hbm": vroof["frac_hbm"],
            "frac_compute": vroof["frac_compute"], "precision": precision(x, "scan_valu")}
    print(json.dumps(line), flush=True)

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 18          # float32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": 4 * n, "copy_probe_bytes_written": 4 * n}),
              flush=True)


if __name__ == "__main__":
    main()
