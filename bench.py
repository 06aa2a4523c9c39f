"""Benchmark of the vocab-side verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5] [--mode greedy|sample]
    python bench.py --all [--jsonl FILE]       (one JSON line per workload and mode)
    python bench.py --op fuse --workload 3     (MTP input fusion at that width and batch)
    python bench.py --op loss                  (top-k soft cross-entropy draft loss + gradient)
    python bench.py --sweep                    (greedy verify time against M_eff, one line per M)

One step = one verify call (the whole hot path: LM-head stream + fused softmax/argmax
epilogue, cross-block combine, acceptance decisions and prefix scan, and in sample
mode the fp64 correction/bonus draws) over one batch of synthetic inputs already
resident in HBM. The default workload is the largest one that fits one GPU, the
large-batch rollout: H=7168, V=129280, bf16 head, B=256 requests, k=3 drafts,
stochastic verification at T=1 (1792 head rows per call). Inputs cycle through a pool
of distinct seeded steps; drafts are drawn beforehand by the library's own drafter
call (Philox word 2) from the drafter hidden states.

Prints one JSON line: verified positions/s (value), accepted and emitted tokens/s, the
per-depth acceptance P(a >= d) and the accepted-length histogram, the whole call's time
(median, p10, p90 from events on the call's stream, in a second pass over the same
inputs after the timed loop), the LM-head kernel against its roofline (HBM bandwidth
against 8 TB/s when the algorithmic bytes take longer at that rate than the
algorithmic flops at 2.5 PFLOP/s, else bf16 MFMA throughput against 2.5 PFLOP/s;
kernel time from HIP events recorded by the library on the call's stream around a
sample of the timed loop's launches), the hardware-counter traffic recorded under
profiles/ when it was taken on the current kernel source, and the CPU oracle timed on a
bounded sample of the same workload, which also checks the GPU's outcomes of the steps it
shares with the timed loop (parity_vs_oracle).
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
CSRC = os.path.join(ROOT, "mtp_draft_verification_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Paths relative to the kernel sources; the build script sets the compiler flags.
LMHEAD_SOURCES = ("lmhead.hip", "skinny.hip", "wide.hip", "headtile.hip", "mtpv_internal.h", "plan.hip",
                  "../build.py")
LOSS_SOURCES = ("loss.hip", "mtpv_internal.h", "../build.py")


def _source_hash(files):
    h = hashlib.sha256()
    for f in files:
        h.update(f.encode())
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def lmhead_source_hash():
    """Hash of the sources that define the LM-head kernels and their launch plan."""
    return _source_hash(LMHEAD_SOURCES)


def loss_source_hash():
    """Hash of the sources that define the draft-loss kernels."""
    return _source_hash(LOSS_SOURCES)


def _recorded_bytes(name, source_hash):
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_hash and m_bytes) or m_hash.group(1) != source_hash:
        return None
    return float(m_bytes.group(1))


def recorded_traffic(wl, mode):
    """HBM bytes per LM-head launch from the committed counter summary, if it was
    measured on the current kernel source; else None."""
    return _recorded_bytes(f"lmhead_{wl.name}_{mode}_traffic.md", lmhead_source_hash())


def recorded_loss_traffic(workload):
    """HBM bytes per draft-loss selection launch from the committed counter summary,
    if it was measured on the current kernel source; else None."""
    return _recorded_bytes(f"loss_{workload}_traffic.md", loss_source_hash())


def calibration_copy(mib):
    """The library's plain copy kernel on `mib` MiB, 5 launches (counter calibration)."""
    import torch
    import mtp_draft_verification_amd as mv
    nbytes = mib << 20
    src = torch.empty(nbytes, dtype=torch.uint8, device=torch.device("cuda:0"))
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(5):
        mv.copy_bytes(dst, src, nbytes)
    torch.cuda.synchronize()
    log(f"calibration copy: {nbytes} bytes read and written per launch, 5 launches")


def algorithmic(wl, mode):
    """Bytes and flops one LM-head launch must move / do: every W element once, every
    hidden row once, and 2*M*H*V flops. Positions M = B(k+1) (+ B k drafter rows)."""
    es = 2 if wl.dtype == "bf16" else 4
    M = wl.M_eff(mode)
    bytes_ = wl.V * wl.H * es + M * wl.H * es
    flops = 2.0 * M * wl.H * wl.V
    return bytes_, flops


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_vendor():
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return f"{i.get('internal_api')} {i.get('version')} ({i.get('architecture')})"
    except Exception:
        pass
    return "unknown"


def _blas_cores():
    try:
        from threadpoolctl import threadpool_info
        return max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(wl, mode, W_store, budget_s, gpu=None):
    """The oracle as it stands, on this host's cores, over a bounded number of steps.
    gpu: the benchmark's own pooled steps (drafts and outcomes per step); for those
    steps the oracle verifies the GPU's drafts and its outcomes are compared with the
    GPU's under the parity tests' rule (bit-exact except decisions the oracle puts
    within 1e-5 of a threshold, which are counted as excused)."""
    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_util import compare_outcomes
    cores = _blas_cores()
    decode = oracle.decode_bf16 if wl.dtype == "bf16" else (lambda a: np.asarray(a, dtype=np.float64))
    W64 = decode(W_store)
    n = 0
    t_total = 0.0
    accepted = 0
    cmp_pos = cmp_exc = cmp_fail = cmp_steps = 0
    while n < 3 or (t_total < budget_s and n < wl.steps):
        xt, xd = synth.hidden(wl, n)
        Xt, Xd = decode(xt), decode(xd)
        mine = gpu is not None and n < len(gpu["drafts"])
        if mine:
            drafts = gpu["drafts"][n]
        else:
            drafts, _ = oracle.draft_from_hidden(Xd, W64, wl.T, wl.seed, n)   # input preparation, untimed
        t0 = time.perf_counter()
        if mode == "greedy":
            r = oracle.verify_greedy_from_hidden(Xt, W64, drafts)
        else:
            r = oracle.verify_sample_from_hidden(Xt, Xd, W64, drafts, wl.T, wl.seed, n)
        t_total += time.perf_counter() - t0
        accepted += int(r["a"].sum())
        if mine:
            npos, nexc, fails = compare_outcomes(mode, {"a": gpu["a"][n], "out": gpu["out"][n]}, r, wl.k)
            cmp_pos += npos
            cmp_exc += nexc
            cmp_fail += len(fails)
            cmp_steps += 1
        n += 1
    pos = wl.B * (wl.k + 1) * n
    out = {"value": pos / t_total, "unit": "positions/s", "cores": cores, "kind": "oracle",
           "sample": f"{n} steps of the same workload ({pos} verified positions), fp64 numpy, "
                     f"{t_total:.1f} s of oracle time; accepted tokens/s {accepted / t_total:.3g}",
           "cpu_model": _cpu_model(), "blas": _blas_vendor()}
    parity = None
    if gpu is not None:
        parity = {"steps": cmp_steps, "positions": cmp_pos, "excused": cmp_exc, "mismatched_requests": cmp_fail}
    return out, parity


def roofline_of(alg_bytes, alg_flops, kern_s, traffic_bytes=None):
    """The roofline the LM-head kernel sits on, and where it is against it. The bound is
    HBM when moving the algorithmic bytes at 8 TB/s takes longer than the algorithmic
    flops at 2.5 PFLOP/s, else bf16 MFMA. Both fractions are given either way."""
    hbm = alg_bytes / kern_s / 1e9
    tflops = alg_flops / kern_s / 1e12
    mfma_bound = alg_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > alg_bytes / (HBM_PEAK_GBS * 1e9)
    r = ({"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
          "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)} if mfma_bound else
         {"bound": "hbm", "achieved": round(hbm, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
          "frac": round(hbm / HBM_PEAK_GBS, 4)})
    r["traffic"] = None if traffic_bytes is None else round(traffic_bytes / kern_s / 1e9, 1)
    r["traffic_unit"] = "GB/s"
    r.update({"kernel_us": round(kern_s * 1e6, 2), "algorithmic_bytes_per_launch": alg_bytes,
              "algorithmic_flops_per_launch": alg_flops, "hbm_gbs": round(hbm, 1),
              "hbm_frac": round(hbm / HBM_PEAK_GBS, 4), "mfma_tflops": round(tflops, 2),
              "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)})
    return r


def achievable(W):
    """What plain kernels reach on this machine beside the published peaks (measured after
    the timed loop, outside it): one non-temporal read sweep of W's bytes (the head, or
    the teacher logits of the draft loss),
    and back-to-back bf16 MFMAs (16x16x32) on every SIMD; median of 5 launches each,
    timed with events on the stream the library launches on."""
    import torch
    import mtp_draft_verification_amd as mv
    sink = torch.zeros(4, dtype=torch.int32, device=W.device)
    nbytes = W.numel() * W.element_size() // 16 * 16

    def median_s(fn, reps=5):
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        return float(np.median(ts))

    mv.read_bytes(W, nbytes, sink)
    t_read = median_s(lambda: mv.read_bytes(W, nbytes, sink))
    iters = 1024
    flops = mv.mfma_rate(iters, sink)
    t_mfma = median_s(lambda: mv.mfma_rate(iters, sink))
    return {"hbm_read_gbs": round(nbytes / t_read / 1e9, 1), "read_bytes": int(nbytes),
            "mfma_bf16_tflops": round(flops / t_mfma / 1e12, 1), "mfma_flops": int(flops),
            "how": "mtpv_read_bytes over the head W (non-temporal 16-byte loads, 8 KB blocks per workgroup spaced by the grid); "
                   "mtpv_mfma_rate (4 waves per CU, 16 independent 16x16x32 bf16 MFMAs per round, varied "
                   "operand bits); median of 5 launches"}


def timing_every(steps):
    """Time one launch in this many during a rate loop of `steps` calls (at least
    about 32 timed launches; every launch for short loops)."""
    return max(1, min(16, steps // 32))


def _events_time(fn, steps, warmup):
    """Wall time per call (host clock around synchronised loops) and the library's
    LM-head kernel time per call (HIP events on the call's stream)."""
    import torch
    import mtp_draft_verification_amd as mv
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    mv.timing_enable(True)
    mv.timing_read(reset=True)
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    kern_ms, n = mv.timing_read(reset=True)
    mv.timing_enable(False)
    return wall, kern_ms / 1e3 / max(n, 1)


def sweep(args):
    """Greedy verify against the number of head rows, H = 5120, V = 151936 (the
    batched / depth-5 head): flat while HBM-bound, rising past the ridge. From 16 rows
    on each line also times the bare head product through the library GEMM
    (torch.mm, hipBLASLt: bf16 logits, no epilogue) on the same inputs."""
    import torch
    import mtp_draft_verification_amd as mv
    dev = torch.device("cuda:0")
    H, V = 5120, 151936
    wl0 = synth.custom(H=H, V=V, B=1, k=3, cid=3, name="sweep_head")
    log(f"sweep: generating W [{V}, {H}] bf16")
    W = torch.from_numpy(synth.weights(wl0).view(np.int16)).view(torch.bfloat16).to(dev)
    for M in (1, 4, 16, 64, 128, 224, 384, 704, 1024, 1792):
        k = 0 if M == 1 else 3
        B = M // (k + 1)
        wl = synth.custom(H=H, V=V, B=B, k=k, cid=400 + M)
        xt, _ = synth.hidden(wl, 0)
        xt_d = torch.from_numpy(np.ascontiguousarray(xt).view(np.int16)).view(torch.bfloat16).to(dev)
        drafts = torch.zeros((B, k), dtype=torch.int32, device=dev)
        alen = torch.zeros(B, dtype=torch.int32, device=dev)
        out = torch.zeros((B, k + 1), dtype=torch.int32, device=dev)
        ws = mv.alloc_workspace(mv.MODE_GREEDY, B, k, H, V, mv.DTYPE_BF16, dev)
        wall, kern = _events_time(lambda: mv.spec_verify_greedy(xt_d, W, drafts, alen, out, ws), args.steps, args.warmup)
        alg_bytes = V * H * 2 + M * H * 2
        line = {"sweep": "greedy_verify_H5120_V151936", "M_eff": M, "B": B, "k": k,
                "ms_per_call": round(wall * 1e3, 4), "kernel_us": round(kern * 1e6, 2),
                "hbm_frac": round(alg_bytes / kern / 8e12, 4),
                "mfma_frac": round(2.0 * M * H * V / kern / 2.5e15, 4)}
        if M >= 16:
            # the same head product through the library GEMM (torch.mm -> hipBLASLt), bf16
            # in and out, no epilogue: logits only, no softmax statistics or decisions
            X = xt_d.reshape(M, H)
            L = torch.empty((M, V), dtype=torch.bfloat16, device=dev)
            for _ in range(args.warmup):
                torch.mm(X, W.t(), out=L)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                torch.mm(X, W.t(), out=L)
            e1.record()
            torch.cuda.synchronize()
            g = e0.elapsed_time(e1) / 1e3 / args.steps
            line["library_gemm_us"] = round(g * 1e6, 2)
            line["library_gemm_over_kernel"] = round(g / kern, 4)
            del L
        print(json.dumps(line), flush=True)


def bench_fuse(args, wl):
    """MTP input fusion at the workload's width and batch: tokens gathered from the head
    W (standing in for the shared embedding table, same shape), fc [H, 2H]."""
    import torch
    import mtp_draft_verification_amd as mv
    dev = torch.device("cuda:0")
    H, V, B = wl.H, wl.V, wl.B

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    log(f"fuse: H={H} V={V} B={B}; generating the table [{V}, {H}] and fc [{H}, {2 * H}]")
    E = bf(synth.weights(wl))
    pool = []
    for s in range(max(1, min(args.pool, 8))):
        tokens, _, h, ge, gh, Wfc = synth.fuse_inputs(H, V, B, step=s, embed=False)
        pool.append((torch.from_numpy(tokens).to(dev), bf(h)))
    ge_d, gh_d, Wfc_d = bf(ge), bf(gh), bf(Wfc)
    out = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = mv.alloc_fuse_workspace(B, H, dev)
    it = [0]

    def call():
        tok, h = pool[it[0] % len(pool)]
        it[0] += 1
        mv.mtp_input_fuse(tok, E, h, ge_d, gh_d, Wfc_d, 1e-6, out, ws)

    wall, kern = _events_time(call, args.steps, args.warmup)
    alg = H * 2 * H * 2 + B * 2 * H * 2          # fc weights once + the fused rows
    line = {"metric": "MTP input fusion rows/s (RMS-normalized embedding | hidden, fc 2H -> H)",
            "value": round(B / wall, 1), "unit": "rows/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(wall * 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"mtp_input_fuse_H{H}_B{B}", "H": H, "B": B, "V": V},
            "roofline": {"bound": "hbm", "achieved": round(alg / kern / 1e9, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(alg / kern / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                         "kernel_us": round(kern * 1e6, 2), "algorithmic_bytes_per_launch": alg}}
    print(json.dumps(line), flush=True)


def bench_loss(args):
    """Top-k soft cross-entropy draft loss with its gradient: teacher and student fp32
    logits [N, V] resident in HBM, one call = selection pass (loss, kept ids) +
    gradient pass. The dominant kernel is the selection pass (both rows streamed
    once); the call as a whole reads the student row a second time for the gradient."""
    import torch
    import mtp_draft_verification_amd as mv
    import oracle
    dev = torch.device("cuda:0")
    N, V, k = args.loss_rows, 151936, args.topk
    log(f"loss: generating teacher/student logits [{N}, {V}] fp32")
    T, S = synth.loss_inputs(N, V, cid=420)
    Td = torch.from_numpy(T).to(dev)
    Sd = torch.from_numpy(S).to(dev)
    loss = torch.empty(N, dtype=torch.float32, device=dev)
    idx = torch.empty((N, k), dtype=torch.int32, device=dev)
    grad = torch.empty((N, V), dtype=torch.float32, device=dev)
    ws = mv.alloc_loss_workspace(N, k, dev)
    scale = 1.0 / N

    def call():
        mv.mtp_draft_loss_topk(Td, Sd, k, loss, ws, scale, idx, grad)

    wall, kern = _events_time(call, args.steps, args.warmup)
    if args.calibrate_copy_mib > 0:
        calibration_copy(args.calibrate_copy_mib)
    workload = f"draft_loss_N{N}_V{V}_topk{k}"
    traffic = recorded_loss_traffic(workload)
    sel_bytes = N * V * 8 + N * 4 + N * k * 4            # teacher + student once, loss + kept ids
    call_bytes = N * V * 12 + N * 4 + N * k * 4          # ... + the gradient written once
    line = {"metric": "draft-loss rows/s (top-k soft cross-entropy, loss + gradient)",
            "value": round(N / wall, 1), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(wall * 1e3, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded N(0,1)*3 teacher, "
            "student = teacher + N(0,1))",
            "config": {"workload": workload, "N": N, "V": V, "topk": k, "grad": True},
            "roofline": {"bound": "hbm", "achieved": round(sel_bytes / kern / 1e9, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(sel_bytes / kern / 1e9 / HBM_PEAK_GBS, 4),
                         "traffic": None if traffic is None else round(traffic / kern / 1e9, 1),
                         "kernel_us": round(kern * 1e6, 2),
                         "algorithmic_bytes_per_launch": sel_bytes,
                         "call_frac": round(call_bytes / wall / 1e9 / HBM_PEAK_GBS, 4)}}
    ach = achievable(Td)
    line["roofline"]["achievable"] = ach
    line["roofline"]["frac_of_achievable"] = round(line["roofline"]["achieved"] / ach["hbm_read_gbs"], 4)
    if not args.no_cpu_baseline:
        # the GPU's outputs of the timed call, compared row by row with the oracle's
        loss_h, idx_h = loss.cpu().numpy(), idx.cpu().numpy()
        rows, el = 0, 0.0
        idx_bad = loss_bad = grad_bad = 0
        while el < args.cpu_budget and rows < N:
            t0 = time.perf_counter()
            lo, K_o = oracle.draft_loss(T[rows:rows + 1], S[rows:rows + 1], k)
            G = oracle.draft_loss_grad(T[rows:rows + 1], S[rows:rows + 1], k, scale)
            el += time.perf_counter() - t0
            idx_bad += int(not np.array_equal(idx_h[rows], K_o[0]))
            loss_bad += int(abs(loss_h[rows] - lo[0]) > 2e-6 + 1e-6 * abs(lo[0]))
            if rows < 8:  # whole gradient rows, under the parity tests' bound
                _, _, _, lse = oracle.draft_loss_row(T[rows], S[rows], k)
                q = np.exp(S[rows].astype(np.float64) - lse)
                tol = scale * 4e-6 * q + 1.2e-7 * np.abs(G[0]) + 1e-30
                grad_bad += int((np.abs(grad[rows].cpu().numpy() - G[0]) > tol).any())
            rows += 1
        line["cpu_baseline"] = {"value": round(rows / el, 2), "unit": "rows/s", "cores": _blas_cores(),
                                "kind": "oracle", "sample": f"{rows} rows of the same call (loss + gradient)",
                                "cpu_model": _cpu_model(), "blas": _blas_vendor()}
        line["parity_vs_oracle"] = {"rows": rows, "kept_id_mismatches": idx_bad, "loss_out_of_bound": loss_bad,
                                    "gradient_rows_checked": min(rows, 8), "gradient_rows_out_of_bound": grad_bad}
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", type=int, default=5,
                    help="1 tiny fp32, 2 decode, 3 batched sampling, 4 depth-5 chain, 5 rollout")
    ap.add_argument("--mode", choices=["greedy", "sample"], default=None)
    ap.add_argument("--pool", type=int, default=32, help="distinct seeded input steps cycled through")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run the library's plain copy kernel on this many MiB (counter calibration)")
    ap.add_argument("--op", choices=["verify", "fuse", "loss"], default="verify",
                    help="verify (default), the MTP input fusion at the workload's H and B, or the top-k "
                         "soft cross-entropy draft loss")
    ap.add_argument("--loss-rows", type=int, default=4096, help="rows (token positions) of the draft loss")
    ap.add_argument("--topk", type=int, default=256, help="teacher tokens kept by the draft loss")
    ap.add_argument("--all", action="store_true",
                    help="every workload and mode in turn, one JSON line each (per-config records)")
    ap.add_argument("--jsonl", default=None, help="also append each JSON line to this file")
    ap.add_argument("--sweep", action="store_true",
                    help="greedy verify time against M_eff at H=5120, V=151936 (one JSON line per M)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the verify step is data parallel "
              "across requests, so N GPUs each run this same single-GPU workload on their own requests.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import mtp_draft_verification_amd as mv

    if args.sweep:
        return sweep(args)
    if args.op == "loss":
        return bench_loss(args)
    wl = synth.WORKLOADS[args.workload]
    if args.op == "fuse":
        return bench_fuse(args, wl)
    if args.all:
        cases = [(c, m) for c, w in synth.WORKLOADS.items() for m in w.modes]
    else:
        cases = [(args.workload, args.mode or wl.modes[0])]
    for cid, mode in cases:
        line = bench_verify(args, synth.WORKLOADS[cid], mode)
        print(json.dumps(line), flush=True)
        if args.jsonl:
            with open(args.jsonl, "a") as fh:
                fh.write(json.dumps(line) + "\n")


def bench_verify(args, wl, mode):
    """One verify workload and mode: the timed loop, the JSON line as a dict."""
    import torch
    import mtp_draft_verification_amd as mv
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    code = mv.DTYPE_BF16 if wl.dtype == "bf16" else mv.DTYPE_F32
    B, k, H, V = wl.B, wl.k, wl.H, wl.V

    def to_dev(a):
        if wl.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    log(f"workload {wl.name} mode {mode}: generating W [{V}, {H}] {wl.dtype}")
    t0 = time.time()
    W_store = synth.weights(wl)
    Wd = to_dev(W_store)
    log(f"  W ready in {time.time() - t0:.1f} s")
    P = max(1, min(args.pool, args.steps + args.warmup))
    xt_pool, xd_pool, d_pool = [], [], []
    ws_draft = mv.alloc_workspace(mv.MODE_DRAFT, B, k, H, V, code, dev) if k > 0 else None
    for s in range(P):
        xt, xd = synth.hidden(wl, s)
        xt_pool.append(to_dev(xt))
        xd_pool.append(to_dev(xd))
        d = torch.zeros((B, k), dtype=torch.int32, device=dev)
        if k > 0:
            mv.spec_draft_sample(xd_pool[-1], Wd, wl.T, wl.seed, s, 0, d, ws_draft)
        d_pool.append(d)
    torch.cuda.synchronize()
    del ws_draft

    ws = mv.alloc_workspace(mv.MODE_GREEDY if mode == "greedy" else mv.MODE_SAMPLE, B, k, H, V, code, dev)
    K = args.steps
    alen = torch.zeros((K + args.warmup, B), dtype=torch.int32, device=dev)
    outt = torch.zeros((K + args.warmup, B, k + 1), dtype=torch.int32, device=dev)

    def step(i, slot):
        s = i % P
        if mode == "greedy":
            mv.spec_verify_greedy(xt_pool[s], Wd, d_pool[s], alen[slot], outt[slot], ws)
        else:
            mv.spec_verify_sample(xt_pool[s], xd_pool[s], Wd, d_pool[s], wl.T, wl.seed, s, alen[slot],
                                  outt[slot], ws)

    for i in range(args.warmup):
        step(i, K + i)
    torch.cuda.synchronize()
    # Events around the LM-head kernel of one call in `every`: each event pair adds a
    # few microseconds to its call, so the rate loop times a spread sample of calls.
    every = timing_every(K)
    mv.timing_enable(True, every)
    mv.timing_read(reset=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        step(i, i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    kern_ms, nlaunch = mv.timing_read(reset=True)
    mv.timing_enable(False)
    assert nlaunch == (K + every - 1) // every, (nlaunch, K, every)
    if mv.get_device_error(ws) != 0:
        raise RuntimeError("device error word set during the benchmark")

    # per-call time of the whole call (every kernel of it), from events on the stream the
    # library launches on (torch's current stream), in a second pass over the same inputs
    # so that the event records stay out of the timed loop above
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        ev[i][0].record()
        step(i, i)
        ev[i][1].record()
    torch.cuda.synchronize()
    t_call = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])

    if args.calibrate_copy_mib > 0:
        calibration_copy(args.calibrate_copy_mib)

    a_host = alen[:K].cpu().numpy()
    accepted = int(a_host.sum())
    a_hist = np.bincount(a_host.ravel(), minlength=k + 1)[:k + 1]
    pos_d = [float((a_host >= d).mean()) for d in range(1, k + 1)]
    positions = B * (k + 1) * K
    value = positions / elapsed
    alg_bytes, alg_flops = algorithmic(wl, mode)
    kern_s = kern_ms / 1e3 / nlaunch
    traffic = recorded_traffic(wl, mode)
    roofline = roofline_of(alg_bytes, alg_flops, kern_s, traffic)
    roofline["timed_launches"] = nlaunch
    ach = achievable(Wd)
    roofline["achievable"] = ach
    roofline["frac_of_achievable"] = round(
        roofline["mfma_tflops"] / ach["mfma_bf16_tflops"] if roofline["bound"] == "mfma"
        else roofline["hbm_gbs"] / ach["hbm_read_gbs"], 4)
    line = {
        "metric": "verified positions/s (accepted tokens/s alongside) at 1 GPU; % of HBM roofline",
        "value": round(value, 1),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0, 0.02) bf16 head, N(0,1) hidden, drafts drawn from the drafter rows)",
        "config": {"workload": f"{wl.name}_{mode}", "H": H, "V": V, "B": B, "k": k, "mode": mode, "T": wl.T,
                   "positions_per_step": B * (k + 1), "head_rows_per_step": wl.M_eff(mode)},
        "accepted_tokens_per_s": round(accepted / elapsed, 2),
        "emitted_tokens_per_s": round((accepted + B * K) / elapsed, 1),
        "mean_acceptance_length": round(1 + accepted / (B * K), 4),
        "acceptance": {"pos_d": [round(x, 5) for x in pos_d],
                       "rate": round(float(np.mean(pos_d)), 5) if k > 0 else None,
                       "a_hist": a_hist.tolist()},
        "t_call_us": {"median": round(float(np.median(t_call)), 2),
                      "p10": round(float(np.percentile(t_call, 10)), 2),
                      "p90": round(float(np.percentile(t_call, 90)), 2)},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        nc = min(P, K)  # timed step i used pooled input i for i < P
        gpu = {"drafts": [d.cpu().numpy() for d in d_pool[:nc]],
               "a": alen[:nc].cpu().numpy(), "out": outt[:nc].cpu().numpy()}
        line["cpu_baseline"], line["parity_vs_oracle"] = cpu_baseline(wl, mode, W_store, args.cpu_budget, gpu)
    return line


if __name__ == "__main__":
    main()
