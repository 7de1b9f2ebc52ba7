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
projection kernel's (bf16 MFMA).  W warm-up steps run untimed; then exactly K steps are
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


def backward_work(x):
    """Compulsory HBM bytes and flops of one backward launch (per token-head).

    Bytes: q, k, v, gate, eta in their input type; dL/dout and the recorded
    delta_t in fp32; the recorded W at every 16-token tile start (4 d^2 bytes
    per tile, d^2/4 per token); dq, dk, dv, dgate (fp32) and deta out; per
    scan dL/dW_final in and dW0 out; per head gamma, beta in and their
    gradients out.  Flops: the 12 d^2 of the per-token gradient algebra
    (G_t k_t, G_t^T delta_t, W_{t-1}^T dz_t, W_t^T dy_t and the two rank-one
    updates of G).
    """
    B, H, T, d = x.q.shape
    n = B * H * T
    s_in = 2 if x.in_bf16 else 4
    per_tok_bytes = (4 * d + 1) * s_in + 4 * d + 4 * d + (d * d) // 4 + 16 * d + 4
    nbytes = n * per_tok_bytes + B * H * 8 * d * d + H * 16 * d
    return n, nbytes, n * 12 * d * d


def ttt_record_chunk():
    """Tokens per tile of the training record (the dual form's chunk must match)."""
    from test_rnn_layer_ttt_amd.binding import RECORD_CHUNK
    return RECORD_CHUNK


def kernel_info(x):
    """Which kernel family runs this workload and which roof bounds it."""
    import test_rnn_layer_ttt_amd as ttt
    d = x.q.shape[-1]
    name = ttt.ttt_linear_kernel(d, ttt.mode_bits(x.ln, x.dual, x.in_bf16), x.chunk)
    if name == "scan_mfma":
        # the d^2 work runs on the matrix cores: the HBM stream is the binding roof
        return name, "hbm"
    # vector-ALU scan: bf16 inputs put it above the FP32-vector ridge, fp32 inputs below
    return name, ("alu" if x.in_bf16 else "hbm")


def projection_work(x):
    """Flops and compulsory HBM bytes of one projection launch: x [B,T,hidden]
    and the weights [H,4d+1,hidden] in bf16, the five results out in the
    scan's input type; 2 flops per product of hidden = H d terms."""
    B, H, T, d = x.q.shape
    hidden, rows = H * d, H * (4 * d + 1)
    out_size = 2 if x.in_bf16 else 4
    nbytes = B * T * hidden * 2 + rows * hidden * 2 + B * T * rows * out_size
    return B * H * T, nbytes, 2 * B * T * hidden * rows


def roofline(x, kernel_ms, traffic, train=False, mask=None, project=False):
    if project:
        n, nbytes, flops = projection_work(x)
        achieved = flops / (kernel_ms / 1e3) / 1e12
        return "proj_mfma", dict(bound="mfma", achieved=round(achieved, 1),
                                 peak=BF16_MATRIX_PEAK_TFLOPS, unit="TFLOP/s",
                                 frac=round(achieved / BF16_MATRIX_PEAK_TFLOPS, 4),
                                 traffic=traffic)
    if train:
        n, nbytes, flops = backward_work(x)
        name, bound = "bwd_mfma", "hbm"
    else:
        n, nbytes, flops = algorithmic_work(x, mask)
        name, bound = kernel_info(x)
    sec = kernel_ms / 1e3
    if bound == "hbm":
        achieved = nbytes / sec / 1e9
        return name, dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS,
                          unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic)
    achieved = flops / sec / 1e12
    return name, dict(bound="alu", achieved=round(achieved, 2), peak=FP32_VECTOR_PEAK_TFLOPS,
                      unit="TFLOP/s", frac=round(achieved / FP32_VECTOR_PEAK_TFLOPS, 4),
                      traffic=traffic)


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle, unmodified, on a bounded sample
# ---------------------------------------------------------------------------
_CPU_SAMPLE = None


_CPU_TRAIN = False
_CPU_MASK = None
_CPU_PROJ = None   # (x, w_proj) of the layer-pass workload, float32 holding bf16 values
_CPU_SILU = False


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


def cpu_baseline(x, n_scans, workers, train=False, mask=None, proj=None):
    """Time the oracle on ``n_scans`` scans of ``x`` (full length) over ``workers``
    processes; with ``train`` its forward and its backward, as one training pass;
    with ``proj`` = (x, w_proj) its input projections of each scan, then the scan."""
    import multiprocessing as mp
    global _CPU_SAMPLE, _CPU_TRAIN, _CPU_MASK, _CPU_PROJ
    _CPU_TRAIN = train
    _CPU_PROJ = proj
    B, H, T, d = x.q.shape
    n_scans = min(n_scans, B * H)
    step = max(1, (B * H) // n_scans)
    pairs = [(i // H, i % H) for i in range(0, B * H, step)][:n_scans]
    _CPU_SAMPLE = x.subset(pairs)
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
    what = (", forward and backward" if train else
            ", input projections then the scan" if proj is not None else "")
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
    ap.add_argument("--update-rate", type=float, default=None,
                    help="dual-form workloads: seeded SKIP/UPDATE decisions per chunk, each "
                         "UPDATE with this probability (ttt_linear_forward_masked)")
    ap.add_argument("--cpu-scans", type=int, default=None,
                    help="scans of the workload the CPU oracle is timed on "
                         "(default 256 for the forward, 128 for a training pass)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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

    x = make_inputs(args.workload)
    B, H, T, d = x.q.shape
    train = args.pass_ == "train"
    project = args.pass_ == "project"
    if project and (d != 64 or args.update_rate is not None or args.silu_qk):
        print("bench.py: --pass project covers d = 64 and the plain scan", file=sys.stderr)
        sys.exit(2)
    if train and ((x.dual and x.chunk != ttt_record_chunk()) or d != 64):
        print(f"bench.py: the backward covers d = 64, per-token or dual form with chunks of "
              f"{ttt_record_chunk()}; workload {args.workload} is not one", file=sys.stderr)
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
        cpu = cpu_baseline(x, args.cpu_scans, host_cores(), train, mask_np,
                           proj_np if project else None)

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
    mode = ttt.mode_bits(x.ln, x.dual, x.in_bf16, args.silu_qk)
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

    if mask_np is None:
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
                 record.data_ptr(), rec_bytes, dout.data_ptr(), dWf.data_ptr(),
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

    for _ in range(args.warmup):
        if train:
            forward_record()
            backward()
        elif project:
            projection()
            forward()
        else:
            forward()
    torch.cuda.synchronize()

    # events on the launch stream around the dominant kernel of each step (the
    # backward in a training pass), and around the whole step
    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    starts, ends, fstarts, fends = mk(), mk(), mk(), mk()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if train:
            fstarts[i].record(stream)
            forward_record()
            fends[i].record(stream)
            starts[i].record(stream)
            backward()
            ends[i].record(stream)
        elif project:
            starts[i].record(stream)
            projection()
            ends[i].record(stream)
            fstarts[i].record(stream)
            forward()
            fends[i].record(stream)
        else:
            starts[i].record(stream)
            forward()
            ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg_kernel_ms = float(np.mean(kernel_ms))
    ms_per_step = wall * 1e3 / args.steps
    n_tok = B * H * T
    kernel = "bwd_mfma" if train else "proj_mfma" if project else kernel_info(x)[0]
    traffic_key = args.workload + ("/backward" if train else "/project" if project else "")
    if mask_np is not None:
        traffic_key = args.workload + f"/update{args.update_rate:g}"
    if args.silu_qk:
        traffic_key += "/silu"
    kname, roof = roofline(x, avg_kernel_ms, load_traffic(kernel, traffic_key), train, mask_np,
                           project)

    mode_name = ("dual-form chunk %d" % x.chunk if x.dual else "per-token") + \
        {"st": "", "exact": ", exact LN Jacobian", "none": ", no LN"}[x.ln]
    line = {
        "metric": METRIC_TRAIN if train else METRIC_PROJECT if project else METRIC,
        "value": round(n_tok / (ms_per_step / 1e3), 1),
        "unit": "token-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "H": H, "T": T, "d": d,
                   "hidden": H * d, "mode": mode_name,
                   "inputs": "bf16" if x.in_bf16 else "fp32", "state": "fp32",
                   "kernel": kname, "kernel_ms_avg": round(avg_kernel_ms, 4),
                   "kernel_ms_min": round(min(kernel_ms), 4)},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if args.silu_qk:
        line["config"]["variant"] = "mlp (SiLU on q and k)"
    if mask_np is not None:
        line["config"]["update_rate"] = args.update_rate
        line["config"]["chunks_updated"] = float(np.mean(mask_np != 0))
    if train:
        line["config"]["pass"] = "train: recording forward + backward"
        fwd_ms = [s_.elapsed_time(e_) for s_, e_ in zip(fstarts, fends)]
        line["config"]["forward_record_ms_avg"] = round(float(np.mean(fwd_ms)), 4)
    if project:
        line["config"]["pass"] = ("layer: input projections from x [B,T,hidden] bf16, "
                                  "then the scan")
        scan_ms = [s_.elapsed_time(e_) for s_, e_ in zip(fstarts, fends)]
        line["config"]["scan_ms_avg"] = round(float(np.mean(scan_ms)), 4)
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
