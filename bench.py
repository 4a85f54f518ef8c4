"""Benchmark: fwd+bwd tokens/s of the fused classifier head + cross-entropy at
the Gemma-2-2B head shape (N = 8192 tokens, D = 2304, V = 256 000, bf16,
peaked softmax, Zipf labels, gradient filter at 2^-12) on one MI355X, and the
fraction of the bf16 dense MFMA peak its dominant kernel reaches.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]

One step = cce_forward + cce_backward (dloss = 1 / N_valid) on inputs that
are already resident in device memory; warm-up steps are not timed.  The
dominant kernel is the forward logit/log-sum-exp kernel; its duration is
taken with HIP events around cce_forward on the stream the work is enqueued
on (the bracket also holds the valid-row compaction and the ordered merge,
two single-pass kernels of a few microseconds).  The CPU baseline times the
fp64 oracle on a bounded sample of rows of the same workload.
Prints one JSON line.
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

TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "k_fwd4_gemma2_2b_head_traffic.md")
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 (published)
METRIC = "fwd+bwd tokens/sec of fused linear-CE at Gemma-2-2B shape; % MFMA peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2, help="1..7 (2 = Gemma-2-2B head)")
    ap.add_argument("--eps", type=float, default=None, help="filter threshold (default: the workload's)")
    ap.add_argument("--sort", action="store_true", help="vocabulary sort, used by the forward and the backward")
    ap.add_argument("--no-bound", action="store_true", help="backward without the forward's block-max table")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="after the timed steps, copy this many bytes device-to-device (counter calibration)")
    ap.add_argument("--cpu-rows", type=int, default=0, help="oracle sample rows (0 = about 20 s of work)")
    ap.add_argument("--no-kahan", action="store_true", help="backward with a plain fp32 dE sum (no compensation)")
    ap.add_argument("--full-de", action="store_true", help="unfiltered dE; the filter applies to dH only")
    ap.add_argument("--fine", action="store_true", help="filter per 32 x 32 sub-tile instead of per 128 x 128 block")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph and replayed (detail.graph_ms_per_step)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="also time the forward's contraction H E^T alone through the vendor BLAS (bf16 logits out)")
    ap.add_argument("--torch-context", action="store_true",
                    help="also time PyTorch cross-entropy on materialised logits (whole and in 4096-row chunks)")
    return ap.parse_args()


def cpu_baseline(x, n_rows_hint):
    """The fp64 oracle, as it stands, on a sample of rows: their lse, loss,
    dH rows, and their contributions to every dE row (the whole backward of
    those rows).  Scaled to tokens/s."""
    import numpy as np

    import oracle
    H64 = oracle.as_f64(x.H, x.dtype)
    E64 = oracle.as_f64(x.E, x.dtype)
    threads = oracle.threads()
    per_row_flops = 8.0 * x.D * x.V  # logits twice, dH row, dE contributions
    rows_n = n_rows_hint or max(threads, int(round(20.0 * threads * 4.5e9 / per_row_flops)))  # ~4.5 GFLOP/s a thread
    rows_n = max(1, min(rows_n, x.N))
    rng = np.random.default_rng(0)
    valid = np.nonzero(x.labels != x.ignore_index)[0]
    rows = np.sort(rng.choice(valid, size=min(rows_n, valid.size), replace=False))
    dl = np.full(x.N, 1.0 / max(x.n_valid, 1))
    t0 = time.perf_counter()
    lse, loss, dH = oracle.rows(H64, E64, x.labels, dl, rows, x.ignore_index)
    sub_lse = np.zeros(x.N)
    sub_lse[rows] = lse
    sub_labels = np.full(x.N, x.ignore_index, dtype=np.int64)
    sub_labels[rows] = x.labels[rows]
    # dE contributions of the sampled rows only: rows outside the sample are ignored
    Hs = H64[rows]
    dE = oracle.dE_rows(Hs, E64, sub_labels[rows], sub_lse[rows], dl[rows], np.arange(x.V), x.ignore_index)
    t = time.perf_counter() - t0
    del dE, dH
    return {"value": len(rows) / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(rows)} of {x.N} rows (full D={x.D}, V={x.V}): lse, loss, dH rows and their dE "
                      f"contributions over all V, fp64, {t:.1f} s"}


def library_gemm(H, E, fwd_ms, reps=5):
    """The forward's contraction alone, H E^T over the rows given (the valid
    ones, as the fused forward computes), through torch's matmul (the vendor
    BLAS, hipBLASLt on ROCm) into a bf16 logit tensor: the rate a library GEMM
    sustains on this shape, for context.  It computes no softmax and writes
    the logits the fused forward never stores."""
    import numpy as np
    import torch

    out = torch.empty(H.shape[0], E.shape[0], dtype=H.dtype, device=H.device)
    Et = E.t()
    for _ in range(2):
        torch.matmul(H, Et, out=out)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for e in ev:
        e[0].record()
        torch.matmul(H, Et, out=out)
        e[1].record()
    torch.cuda.synchronize()
    ms = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
    del out
    flops = 2.0 * H.shape[0] * H.shape[1] * E.shape[0]
    return {"ms": ms, "TFLOP_per_s": flops / (ms * 1e-3) / 1e12,
            "logits_GB": H.shape[0] * E.shape[0] * H.element_size() / 1e9, "fused_forward_over_library": fwd_ms / ms}


def torch_context(H, E, y, ignore_index, reps=3, chunk=4096):
    """PyTorch's own cross-entropy on the same tensors, for context: logits
    H E^T materialised in the input dtype and upcast to fp32 inside the loss,
    mean over valid rows, forward + backward; once over all rows and once in
    row chunks (each chunk's logits freed before the next).  Median ms, the
    peak device memory the step adds, and the mean loss of the last run (the
    test suite checks it against the oracle)."""
    import numpy as np
    import torch
    import torch.nn.functional as F

    n_valid = int((y != ignore_index).sum().item())
    last = {}

    def whole(Hr, Er):
        loss = F.cross_entropy(F.linear(Hr, Er).float(), y, ignore_index=ignore_index)
        loss.backward()
        last["loss"] = loss.detach()

    def chunked(Hr, Er):
        total = None
        for r0 in range(0, H.shape[0], chunk):
            r1 = min(H.shape[0], r0 + chunk)
            part = F.cross_entropy(F.linear(Hr[r0:r1], Er).float(), y[r0:r1], ignore_index=ignore_index,
                                   reduction="sum") / max(n_valid, 1)
            part.backward()
            total = part.detach() if total is None else total + part.detach()
        last["loss"] = total

    out = {}
    for name, fn in (("materialised", whole), (f"chunked_{chunk}_rows", chunked)):
        times, peak = [], 0.0
        for r in range(reps + 1):
            Hr = H.detach().clone().requires_grad_()
            Er = E.detach().clone().requires_grad_()
            torch.cuda.synchronize()
            torch.cuda.reset_peak_memory_stats()
            base = torch.cuda.memory_allocated()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record()
            fn(Hr, Er)
            ev[1].record()
            torch.cuda.synchronize()
            if r:  # the first run warms up
                times.append(ev[0].elapsed_time(ev[1]))
                peak = max(peak, (torch.cuda.max_memory_allocated() - base) / 1e9)
            del Hr, Er
        out[name] = {"ms_per_step": float(np.median(times)), "tokens_per_s": H.shape[0] / (np.median(times) * 1e-3),
                     "extra_memory_GB": peak, "mean_loss": float(last["loss"])}
    return out


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus must be 1 "
                                   "(token or vocabulary sharding across GPUs is not implemented)"}))
        sys.exit(2)
    import numpy as np
    import torch

    from linear_cross_entropy_cce_amd import binding as B
    from linear_cross_entropy_cce_amd import inputs

    dev = "cuda:0"
    torch.cuda.set_device(0)
    print(f"[bench] generating workload {a.workload}", file=sys.stderr, flush=True)
    x = inputs.make_workload(a.workload)
    eps = x.eps if a.eps is None else a.eps
    to = (lambda arr: torch.from_numpy(arr).view(torch.bfloat16).to(dev)) if x.dtype == "bf16" else \
        (lambda arr: torch.from_numpy(arr).to(dev))
    H, E = to(x.H), to(x.E)
    y = torch.from_numpy(x.labels).to(dev)
    N, D, V = x.N, x.D, x.V
    nv = x.n_valid
    dt = B.CCE_BF16 if x.dtype == "bf16" else B.CCE_F32
    loss = torch.empty(N, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    dl = torch.from_numpy(np.where(x.labels != x.ignore_index, 1.0 / max(nv, 1), 0.0).astype(np.float32)).to(dev)
    dH = torch.empty_like(H)
    dE = torch.empty_like(E)
    stats = torch.zeros(7, dtype=torch.int64, device=dev)
    # block-max table (one float per 128 x 128 logit block), as the autograd wrapper uses it
    tb = None if a.no_bound else torch.empty(B.block_max_elems(N, V), dtype=torch.float32, device=dev)
    ws_f = torch.empty(B.forward_workspace_bytes(N, D, V, dt), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(B.backward_workspace_bytes(N, D, V, dt), dtype=torch.uint8, device=dev)
    ws_s = torch.empty(B.vocab_order_workspace_bytes(N, D, V, dt), dtype=torch.uint8, device=dev) if a.sort else None
    perm = torch.empty(V, dtype=torch.int32, device=dev) if a.sort else None
    bwd_flags = (B.CCE_BWD_NO_KAHAN if a.no_kahan else 0) | (B.CCE_BWD_FULL_DE if a.full_de else 0) | \
        (B.CCE_BWD_FINE_FILTER if a.fine else 0)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    mem0 = torch.cuda.memory_allocated()

    def step(ev=None, count=False):
        if ev is not None:
            ev[3].record(stream)
        if a.sort:
            B.cce_vocab_order(H, E, y, x.ignore_index, perm=perm, ws=ws_s)
        if ev is not None:
            ev[0].record(stream)
        B.cce_forward(H, E, y, x.ignore_index, loss=loss, lse=lse, block_max=tb, ws=ws_f, perm=perm)
        if ev is not None:
            ev[1].record(stream)
        B.cce_backward(H, E, y, lse, dl, eps, x.ignore_index, perm, bwd_flags, dH=dH, dE=dE,
                       stats=stats if count else None, ws=ws_b,
                       block_max=tb)
        if ev is not None:
            ev[2].record(stream)

    print(f"[bench] warmup {a.warmup}", file=sys.stderr, flush=True)
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(a.steps)]
    print(f"[bench] timing {a.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(a.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    graph_ms = None
    if a.graph:
        # The library only enqueues kernels, so the whole step can be captured
        # and replayed; the same work with less launch overhead.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            step()
        for _ in range(a.warmup):
            graph.replay()
        torch.cuda.synchronize()
        tg = time.perf_counter()
        for _ in range(a.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - tg) * 1e3 / a.steps
        print(f"[bench] graph replay {graph_ms:.3f} ms/step", file=sys.stderr, flush=True)
    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in evs]
    sort_ms = [e[3].elapsed_time(e[0]) for e in evs]
    step_ms = wall * 1e3 / a.steps
    # The block counts for the work accounting come from one more step with
    # the (optional) counters on, outside the timed region.
    step(count=True)
    torch.cuda.synchronize()
    st = stats.cpu().numpy()
    n_live, n_label, n_total, n_recomp, n_sub = int(st[0]), int(st[1]), int(st[2]), int(st[4]), int(st[6])
    br, bv = B.filter_block()
    # Algorithmic work: the forward logits, the recomputed blocks' logits, and
    # the dH and dE products of the 32 x 32 sub-tiles that keep their softmax
    # part (4 D flops per entry; every sub-tile of a kept block without the
    # fine filter).  A label-only block keeps only its label entries, one per
    # row at most: 4 D flops per label entry (at most N_valid of them).
    f_logits = 2.0 * nv * D * V
    f_grad = 4.0 * D * n_sub * 32 * 32 + 4.0 * D * (nv if n_label else 0)
    f_exec = f_logits + 2.0 * D * n_recomp * br * bv + f_grad
    peak = PEAK_BF16_TFLOPS if x.dtype == "bf16" else PEAK_FP32_TFLOPS
    fwd_avg = float(np.mean(fwd_ms))
    achieved = f_logits / (fwd_avg * 1e-3) / 1e12
    # HBM bytes per k_fwd4 launch from the committed counter passes, while the
    # kernel's sources are the ones they were taken on (this workload only)
    from linear_cross_entropy_cce_amd import profiling as TR
    rec = TR.load(TRAFFIC_PROFILE) if a.workload == 2 else None
    traffic = rec[0] if rec and rec[1] == TR.sources_hash() else None
    out = {
        "metric": METRIC,
        "value": N / (step_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": x.dtype,
        "data": "synthetic (seeded; head shape of the named model, random values)",
        "config": {"workload": f"{x.name} (N={N}, D={D}, V={V}, {x.dtype}, eps={eps:g}, sort={a.sort})",
                   "N": N, "D": D, "V": V, "n_valid": nv, "filter_eps": eps, "sort_vocab": a.sort,
                   "filter_block": [br, bv], "kahan_de": not a.no_kahan, "full_de": a.full_de,
                   "fine_filter": a.fine},
        "roofline": {"kernel": "k_fwd4 (cce_forward bracket)", "bound": "mfma", "achieved": achieved,
                     "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak, "traffic": traffic},
        "detail": {
            "fwd_ms_mean": fwd_avg, "bwd_ms_mean": float(np.mean(bwd_ms)),
            "sort_ms_mean": float(np.mean(sort_ms)),
            "graph_ms_per_step": graph_ms,
            "fwd_ms_min": float(np.min(fwd_ms)), "bwd_ms_min": float(np.min(bwd_ms)),
            "blocks_softmax_kept": n_live, "blocks_label_only": n_label, "blocks_total": n_total,
            "kept_frac": (n_live + n_label) / max(n_total, 1),
            "subtiles_softmax_kept": n_sub, "subtile_kept_frac": n_sub / max(16 * n_total, 1),
            "blocks_recomputed": n_recomp, "recomputed_frac": n_recomp / max(n_total, 1),
            "block_max": tb is not None,
            "F_exec_TF": f_exec / 1e12, "F_exec_frac_peak": f_exec / (step_ms * 1e-3) / (peak * 1e12),
            "F6_TF": (f_logits + f_grad) / 1e12,
            "workspace_MB": (ws_f.numel() + ws_b.numel()) / 1e6,
            "block_max_MB": 0.0 if tb is None else tb.numel() * 4 / 1e6,
            "extra_alloc_MB": (torch.cuda.max_memory_allocated() - mem0) / 1e6,
            "valid_tokens_per_s": nv / (step_ms * 1e-3),
        },
    }
    if a.library_gemm:
        print("[bench] library gemm", file=sys.stderr, flush=True)
        out["library_gemm"] = library_gemm(H[y != x.ignore_index].contiguous(), E, fwd_avg)
    if a.torch_context:
        print("[bench] torch context", file=sys.stderr, flush=True)
        out["torch_context"] = torch_context(H, E, y, x.ignore_index)
    if a.copy_probe:
        src = torch.empty(a.copy_probe // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not a.no_cpu_baseline:
        print("[bench] cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(x, a.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
