"""Benchmark of the retained-mass block-sparse attention hot path on one MI355X.

One step = one pass of the whole path over one synthetic layer:
  losa_block_mass (exact masses) -> losa_select (top-p lists + budget order)
  -> losa_sparse_attn (frozen-pattern attention).
Inputs are resident in HBM before the timed region; every buffer and
workspace is allocated before it.  Default workload: the largest layer, the
HunyuanVideo 720p shape (24 heads x 128, 33x45x80 = 118800 tokens,
128-token blocks, p = 0.99, bf16); ``--workload 1`` is the Wan2.1-1.3B 480p
shape (12 heads x 128, 32760 tokens, 64-token blocks), ``--workload 2`` the
Wan2.1-14B 720p shape.  ``--workload 4`` runs the 50-step frozen-reuse
trajectory (construction at step 2, per-head p, Q/K drift).

Prints ONE JSON line.  value = kept-block TFLOP/s of the sparse attention
(4 * d * R * C * kept blocks / time of one losa_sparse_attn call, measured
with HIP events on the stream the kernels run on); ms_per_step is the whole
step (wall clock between device synchronisations).  The roofline object
describes the dominant call.  Its traffic field comes from a committed
rocprofv3 PMC summary and is reported only while the kernel sources still
hash to the version that was measured (null otherwise).

Other modes (used to produce the committed profile summaries):
  --copy-calibration    run a plain 1 GiB device copy three times (for
                        scaling rocprofv3 FETCH_SIZE/WRITE_SIZE);
  --summarize-pmc WL F W CF CW
                        write the traffic summary of workload WL from the
                        counter CSVs of a FETCH_SIZE run F and a WRITE_SIZE
                        run W of this benchmark, and of the copy calibration
                        under the same two counters (CF, CW);
  --summarize-trace DIR NAME "CMD"
                        write profiles/NAME.md from the kernel statistics of a
                        rocprofv3 --kernel-trace --stats run (DIR) of the
                        command CMD;
  --summarize-mfma PMC NAME "CMD"
                        write profiles/NAME.md: rocprofv3's MfmaUtil (matrix
                        cores busy, share of SIMD cycles) and MfmaFlopsBF16
                        (bf16 MFMA flops executed) per dispatch;
  --summarize-clock PMC TRACE NAME "CMDS"
                        write profiles/NAME.md: busy cycles per dispatch
                        (rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_BUSY_CYCLES run
                        PMC) against the kernel-trace durations (run TRACE),
                        i.e. the clock the matrix-core kernels sustain.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-sparse attn ms & effective TFLOP/s at p=0.99 (1 GPU); mass+select ms"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
def traffic_file(workload_name: str) -> str:
    return os.path.join(ROOT, "profiles", f"hbm_traffic_{workload_name}.json")
_CSRC = "free_block_sparse_exact_amd/csrc/"
# sources each call's kernels are built from (a traffic figure is reported only while they are unchanged)
CALL_SOURCES = {
    "losa_sparse_attn": [_CSRC + "losa_attn.hip", _CSRC + "losa_pack.hpp", _CSRC + "losa_device.hpp",
                         "free_block_sparse_exact_amd/_build.py"],
    "losa_block_mass": [_CSRC + "losa_mass.hip", _CSRC + "losa_pack.hpp", _CSRC + "losa_device.hpp",
                        _CSRC + "losa_blocksum.hpp", "free_block_sparse_exact_amd/_build.py"],
}
CALL_SOURCES["losa_select"] = [_CSRC + "losa_select.hip", _CSRC + "losa_device.hpp", _CSRC + "losa_internal.hpp",
                               "free_block_sparse_exact_amd/_build.py"]
# kernel name fragment -> (part, call) for the traffic summary
# Kernel names as rocprofv3 reports them (mangled or demangled): regular
# expressions, first match wins, so a template instance that belongs to
# another call comes before its plain name.
_ATTN_INPASS = r"attn_bf16_kernel(<\d+, true>|ILi\d+ELb1)"
_ATTN = r"attn_bf16_kernel(<\d+, false>|ILi\d+ELb0)"
_DENSE_LISTS = r"dense_bf16_kernel(<\d+, true>|ILi\d+ELb1)"
_DENSE = r"dense_bf16_kernel(<\d+, false>|ILi\d+ELb0)"
_PACK_KV = r"pack_kv_kernel(<\d+, true>|ILi\d+ELb1)"
_PACK_K = r"pack_kv_kernel(<\d+, false>|ILi\d+ELb0)"
# kernel name pattern -> (part, call) for the traffic summary
PMC_KERNELS = [(_ATTN, "attn", "losa_sparse_attn"),
               (_PACK_KV, "pack_kv", "losa_sparse_attn"),
               (r"mass_bf16_kernel", "mass", "losa_block_mass"),
               (_PACK_K, "pack_k", "losa_block_mass"),
               (r"cut_wave_kernel", "cut", "losa_select"),
               (r"cut_group_kernel", "cut_group", "losa_select"),
               (r"order_kernel", "order", "losa_select"),
               (r"compact_kernel", "compact", "losa_select")]


def kernel_label(name, table):
    """The first entry of table whose pattern occurs in the kernel name."""
    return next((e[1:] for e in table if re.search(e[0], name)), None)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _strip_c_comments(text: str) -> str:
    """C/C++/HIP source without its comments, each run of whitespace one
    space: what the compiler sees (string and character literals are kept
    as written)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def sources_hash(paths) -> str:
    """Hash of the sources a call's kernels are built from; comments and
    layout of the C++/HIP files do not count (they change no kernel)."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            data = f.read()
        if p.endswith((".hip", ".hpp", ".h", ".cpp")):
            data = _strip_c_comments(data.decode("utf-8")).encode("utf-8")
        h.update(data)
    return h.hexdigest()[:16]


def cpu_baseline(layer, wl, rows_wanted, p, budget_s=20.0):
    """Time the fp64 oracle (as it stands) on a bounded sample of query blocks
    of the same layer and scale to the full step and to kept-block TFLOP/s."""
    import oracle as O
    import synthetic as S
    R, C = wl.block, wl.key_block
    N, H, d = wl.tokens, layer.q.shape[1], wl.head_dim
    nq = wl.n_blocks
    rng = np.random.default_rng(7)
    t_mass = t_sel = t_attn = 0.0
    flops = 0.0
    done = 0
    t_start = time.time()
    cache = {}
    for _ in range(rows_wanted):
        h, i = int(rng.integers(H)), int(rng.integers(nq))
        if h not in cache:
            cache = {h: tuple(S.to_f64(getattr(layer, n)[:, h:h + 1], wl.dtype) for n in ("q", "k", "v"))}
        qh, kh, vh = cache[h]
        t0 = time.time()
        Mr = O.block_mass_rows(qh, kh, N, R, C, [(0, 0, i)])
        t1 = time.time()
        kept, s = O.select_contract_row(Mr[0].astype(np.float32), p)
        t2 = time.time()
        rp = np.array([0] * (i + 1) + [s], np.int64)
        O.sparse_attention_rows(qh, kh, vh, N, R, C, rp, kept.astype(np.int32), [(0, 0, i)])
        t3 = time.time()
        t_mass += t1 - t0
        t_sel += t2 - t1
        t_attn += t3 - t2
        flops += 4.0 * d * R * C * s
        done += 1
        if time.time() - t_start > budget_s:
            break
    rows_total = H * nq
    try:
        from threadpoolctl import threadpool_info
        cores = max([x.get("num_threads", 1) for x in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    return {
        "value": flops / t_attn / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{done} random query blocks of the same layer (fp64 numpy oracle: block masses, selection, "
                  f"sparse attention); value = the oracle's kept-block TFLOP/s on them; step time extrapolated "
                  f"linearly to all {rows_total} blocks",
        "ms_per_step_extrapolated": (t_mass + t_sel + t_attn) / done * rows_total * 1e3,
        "mass_ms_extrapolated": t_mass / done * rows_total * 1e3,
        "sparse_attn_ms_extrapolated": t_attn / done * rows_total * 1e3,
        "cpu": cpu_model(),
    }


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), with the logical CPU count."""
    name = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{name} ({os.cpu_count()} logical CPUs visible)"


def xcd_loads(order, counts, qhalves, n_xcd=8, block=32):
    """Kept blocks per XCD under the sparse attention's dispatch: workgroup
    bid runs on XCD bid % n_xcd and takes task xcd_block_task(bid) (blocks of
    32 consecutive tasks dealt to the XCDs round-robin; the tail past the last
    whole round keeps the identity); task t is query tile t % qhalves of row
    order[t // qhalves]."""
    n = len(order) * qhalves
    bid = np.arange(n)
    group = n_xcd * block
    full = n // group * group
    xcd, local = bid % n_xcd, bid // n_xcd
    task = np.where(bid >= full, bid, (local // block) * group + xcd * block + (local % block))
    work = np.asarray(counts)[np.asarray(order)[task // qhalves]]
    return np.bincount(xcd, weights=work, minlength=n_xcd)


def load_traffic(call: str, workload_name: str):
    """HBM bytes per launch of one library call from the committed PMC summary
    of this workload, if the call's kernel sources are unchanged since the
    counters were taken."""
    path = traffic_file(workload_name)
    if not os.path.exists(path):
        return None, "no PMC summary for this workload"
    with open(path) as f:
        t = json.load(f)
    c = t.get("calls", {}).get(call)
    if c is None:
        return None, "call not in the PMC summary"
    if c.get("sources_sha256_16") != sources_hash(CALL_SOURCES[call]):
        return None, "kernel sources changed since the counters were taken"
    return c.get("bytes"), t.get("command")


class Buffers:
    """Every device buffer of one step, allocated once."""

    def __init__(self, F, torch, q, k, v, geom, dev):
        H, nq, nk = geom.heads, geom.n_q, geom.n_k
        rows = geom.rows
        self.M = torch.empty((geom.batch, H, nq, nk), dtype=torch.float32, device=dev)
        self.ws_mass = torch.empty(F.losa_block_mass_workspace(geom), dtype=torch.uint8, device=dev)
        self.ws_sel = torch.empty(F.losa_select_workspace(geom), dtype=torch.uint8, device=dev)
        self.ws_attn = torch.empty(max(F.losa_sparse_attn_workspace(geom), 1), dtype=torch.uint8, device=dev)
        self.row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
        self.col_idx = torch.empty(rows * nk, dtype=torch.int32, device=dev)
        self.order = torch.empty(rows, dtype=torch.int32, device=dev)
        self.out = torch.empty_like(q)
        self.kept = torch.empty((rows, 2), dtype=torch.float32, device=dev)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="3")
    ap.add_argument("--heads", type=int, default=0,
                    help="run only the first HEADS heads of the workload (one GPU's share under head sharding)")
    ap.add_argument("--cpu-rows", type=int, default=16, help="query blocks in the oracle CPU baseline (0: skip)")
    ap.add_argument("--legs", choices=("all", "step"), default="all",
                    help="step: time the step only (no construction, reduced-search, refresh, selector-cache, graph and routing "
                         "legs), e.g. under a profiler")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--refresh-tau", type=float, default=0.75,
                    help="drift threshold of the drift-triggered refresh leg of the reuse workload")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=5,
                    metavar=("WORKLOAD", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"))
    ap.add_argument("--summarize-trace", nargs=3, metavar=("TRACE_DIR", "NAME", "COMMAND"))
    ap.add_argument("--summarize-clock", nargs=4, metavar=("PMC_DIR", "TRACE_DIR", "NAME", "COMMANDS"))
    ap.add_argument("--summarize-mfma", nargs=3, metavar=("PMC_DIR", "NAME", "COMMAND"))
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_clock:
        summarize_clock(*args.summarize_clock)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs the path on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch
    import free_block_sparse_exact_amd as F
    import synthetic as S

    wl = S.get_workload(args.workload)
    if wl.steps > 1:
        return run_reuse(args, wl)
    R, C = wl.block, wl.key_block
    N, Na, H, d = wl.tokens, wl.tokens_alloc, wl.heads, wl.head_dim
    share = 0 < args.heads < wl.heads
    if share:
        H = args.heads
    log(f"workload {wl.wid} {wl.name}: H={H}{f' of {wl.heads}' if share else ''} d={d} N={N} block={R} p={wl.p}")
    t0 = time.time()
    layer = S.make_layer(wl, heads=list(range(H)) if share else None)
    log(f"generated in {time.time() - t0:.1f}s")
    dev = torch.device("cuda:0")

    def to_dev(a):
        if wl.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    q, k, v = to_dev(layer.q), to_dev(layer.k), to_dev(layer.v)
    geom = F.Geometry.of(q, N, R, C)
    nq, nk, rows = geom.n_q, geom.n_k, geom.rows
    bufs = Buffers(F, torch, q, k, v, geom, dev)
    stream = torch.cuda.current_stream()
    p = wl.p

    def step(ev=None, st=stream):
        if ev:
            ev[0].record(st)
        F.losa_block_mass(q, k, N, R, C, out=bufs.M, ws=bufs.ws_mass, stream=st)
        if ev:
            ev[1].record(st)
        F.losa_select(bufs.M, p, N, R, C, tokens_alloc=Na, row_ptr=bufs.row_ptr, col_idx=bufs.col_idx,
                      order=bufs.order, ws=bufs.ws_sel, stream=st)
        if ev:
            ev[2].record(st)
        F.losa_sparse_attn(q, k, v, bufs.row_ptr, bufs.col_idx, bufs.order, N, R, C, out=bufs.out,
                           ws=bufs.ws_attn, stream=st)
        if ev:
            ev[3].record(st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    nnz = int(bufs.row_ptr[-1].item())
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    log(f"timed {args.steps} steps")
    ms_step = (t1 - t0) * 1e3 / args.steps
    all_legs = args.legs == "all"
    graph_ms = graph_step_ms(torch, step, stream, args.steps) if all_legs else None
    mass_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    sel_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    attn_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))

    kept_flop = 4.0 * d * R * C * nnz
    dense_flop = 4.0 * d * float(Na) * float(Na) * H
    mass_flop = 2.0 * d * float(N) * float(N) * H  # one Q K^T product over all valid scores
    attn_tflops = kept_flop / (attn_ms * 1e-3) / 1e12
    mass_tflops = mass_flop / (mass_ms * 1e-3) / 1e12
    sel_bytes = 4.0 * rows * nk + 4.0 * nnz + 8.0 * rows
    kernels = {
        "sparse_attn": {"ms": attn_ms, "tflops": attn_tflops, "frac_bf16_peak": attn_tflops / PEAK_BF16_TFLOPS,
                        "launches": "pack_kv + attn"},
        "block_mass": {"ms": mass_ms, "tflops": mass_tflops, "frac_bf16_peak": mass_tflops / PEAK_BF16_TFLOPS,
                       "launches": "pack_k + mass"},
        "select": {"ms": sel_ms, "algorithmic_bytes": sel_bytes,
                   "GBps": sel_bytes / (sel_ms * 1e-3) / 1e9,
                   "frac_hbm_peak": sel_bytes / (sel_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
    }
    def traffic_of(call):
        return load_traffic(call, wl.name) if not share else (None, "measured for whole layers only")

    # The dominant kernel is attn_bf16_kernel (the mass call splits its time over two kernels).
    traffic, traffic_src = traffic_of("losa_sparse_attn")
    roofline = {"kernel": "losa_sparse_attn (pack_kv_kernel + attn_bf16_kernel)", "bound": "mfma",
                "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": attn_tflops / PEAK_BF16_TFLOPS, "traffic": traffic, "traffic_source": traffic_src}
    traffic, traffic_src = traffic_of("losa_block_mass")
    roofline_mass = {"kernel": "losa_block_mass (pack_kv_kernel + mass_bf16_kernel)",
                     "bound": "mfma", "achieved": mass_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": mass_tflops / PEAK_BF16_TFLOPS, "traffic": traffic, "traffic_source": traffic_src}
    counts = np.diff(bufs.row_ptr.cpu().numpy().astype(np.int64))
    per_xcd = xcd_loads(bufs.order.cpu().numpy(), counts, R // 64)
    routing = None
    inpass = None
    if all_legs:
        other_legs(F, torch, q, k, v, bufs, geom, wl, stream, dev, kernels, kept_flop)
        routing = pooled_routing(F, torch, q, k, bufs, geom, wl, stream, dev)
        inpass = inpass_routing(F, torch, q, k, v, bufs, geom, wl, stream, dev)
    cpu = None
    if args.cpu_rows > 0:
        log("timing the CPU oracle baseline ...")
        cpu = cpu_baseline(layer, wl, args.cpu_rows, wl.p, args.cpu_budget)
    sel_traffic, sel_src = traffic_of("losa_select")
    roofline_select = {"kernel": "losa_select (all its kernels)", "bound": "hbm", "achieved": sel_bytes / (sel_ms * 1e-3) / 1e9,
                       "peak": PEAK_HBM_GBS, "unit": "GB/s",
                       "frac": sel_bytes / (sel_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "traffic": sel_traffic,
                       "traffic_source": sel_src,
                       "algorithmic_bytes": "4 per mass read + 4 per kept index + 8 per row (row_ptr, order)"}
    res = {
        "metric": METRIC,
        "value": attn_tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "graph_ms_per_step": graph_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded random-Fourier-feature Q/K + N(0,1) noise and sinks, N(0,1) V; no trained weights)",
        "config": {"workload": wl.name + (f" (heads 0-{H - 1} of {wl.heads})" if share else ""), "batch": 1,
                   "heads": H, "head_dim": d, "tokens": N, "tokens_alloc": Na,
                   "block": R, "k_block": C, "p": wl.p, "parallelism": "single GPU"},
        "sparse_attn_ms": attn_ms,
        "mass_select_ms": mass_ms + sel_ms,
        "mass_ms": mass_ms,
        "select_ms": sel_ms,
        "dense_equiv_tflops": dense_flop / (attn_ms * 1e-3) / 1e12,
        "nnz_blocks": nnz,
        "coverage": nnz / float(rows * nk),
        "imbalance_per_xcd_max_over_mean": float(per_xcd.max() / per_xcd.mean()),
        "kernels": kernels,
        "roofline": roofline,
        "roofline_mass": roofline_mass,
        "roofline_select": roofline_select,
        "pooled_routing": routing,
        "inpass_threshold": inpass,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res))


INPASS_THETA = (0.1, 0.01, 0.001)


def inpass_routing(F, torch, q, k, v, bufs, geom, wl, stream, dev):
    """On-the-fly block thresholding inside the attention call
    (losa_sparse_attn_threshold: pooled proxy, decisions in the kernel, no
    proxy matrix) against the same rule as three calls (losa_pooled_mass ->
    losa_select_threshold -> losa_sparse_attn): time, kept-block TFLOP/s,
    coverage and recall under the exact masses (bufs.M holds them)."""
    N, R, C, d = geom.tokens, geom.q_block, geom.k_block, geom.head_dim
    rows, nk = geom.rows, geom.n_k
    w = torch.tensor(np.tile(np.array([min(R, N - i * R) for i in range(geom.n_q)], np.float64), rows // geom.n_q),
                     device=dev)
    M = bufs.M.view(rows, nk).double()
    total = (M.sum(dim=1) * w).sum()
    ws_t = torch.empty(F.losa_sparse_attn_threshold_workspace(geom), dtype=torch.uint8, device=dev)
    cnt = torch.empty(rows, dtype=torch.int32, device=dev)
    mask = torch.empty((rows, (nk + 31) // 32), dtype=torch.int32, device=dev)
    P = torch.empty_like(bufs.M)
    ws_p = torch.empty(F.losa_pooled_mass_workspace(geom), dtype=torch.uint8, device=dev)
    shifts = torch.arange(32, device=dev, dtype=torch.int32)
    out = {"theta": list(INPASS_THETA), "inpass_ms": [], "inpass_tflops": [], "three_calls_ms": [],
           "coverage": [], "recall": [], "same_blocks_as_three_calls": []}
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(4)]
    for theta in INPASS_THETA:
        for e0, e1 in evs:
            e0.record(stream)
            F.losa_sparse_attn_threshold(q, k, v, theta, N, R, C, out=bufs.out, kept_count=cnt, kept_mask=mask,
                                         ws=ws_t, stream=stream)
            e1.record(stream)
        torch.cuda.synchronize()
        t_in = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs[1:]]))
        bits = ((mask.unsqueeze(-1) >> shifts) & 1).view(rows, -1)[:, :nk].bool()
        nnz = int(cnt.sum().item())
        kept = ((M * bits).sum(dim=1) * w).sum()
        for e0, e1 in evs:
            e0.record(stream)
            F.losa_pooled_mass(q, k, N, R, C, out=P, ws=ws_p, stream=stream)
            F.losa_select_threshold(P, theta, N, R, C, tokens_alloc=geom.tokens_alloc, row_ptr=bufs.row_ptr,
                                    col_idx=bufs.col_idx, order=bufs.order, ws=bufs.ws_sel, stream=stream)
            F.losa_sparse_attn(q, k, v, bufs.row_ptr, bufs.col_idx, bufs.order, N, R, C, out=bufs.out,
                               ws=bufs.ws_attn, stream=stream)
            e1.record(stream)
        torch.cuda.synchronize()
        t_3 = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs[1:]]))
        out["inpass_ms"].append(t_in)
        out["inpass_tflops"].append(4.0 * d * R * C * nnz / (t_in * 1e-3) / 1e12)
        out["three_calls_ms"].append(t_3)
        out["coverage"].append(nnz / float(rows * nk))
        out["recall"].append(float(kept / total))
        out["same_blocks_as_three_calls"].append(int(bufs.row_ptr[-1].item()) == nnz)
        log(f"in-pass thresholding theta {theta}: {t_in:.3f} ms (three calls {t_3:.3f} ms), coverage "
            f"{out['coverage'][-1]:.4f}, recall {out['recall'][-1]:.5f}")
    out["note"] = ("recall under the exact masses of the layer; same_blocks_as_three_calls compares kept-block totals "
                   "(the three-call path decides on fp32 proxy masses, the in-pass call on fp64 pooled scores)")
    return out


def other_legs(F, torch, q, k, v, bufs, geom, wl, stream, dev, kernels, kept_flop):
    """Calls timed after the steps, not part of ms_per_step: the construction
    call, the sparse attention with the masses within its lists, and the
    drift-triggered refresh's two calls."""
    N, R, C = wl.tokens, wl.block, wl.key_block
    H, d = geom.heads, geom.head_dim
    # The construction call (dense attention + exact masses in one pass), timed
    # on its own after the steps; not part of ms_per_step.
    ws_dense = torch.empty(F.losa_dense_attn_mass_workspace(geom), dtype=torch.uint8, device=dev)
    M_dense = torch.empty_like(bufs.M)
    F.losa_dense_attn_mass(q, k, v, N, R, C, out=bufs.out, M=M_dense, ws=ws_dense, stream=stream)
    dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
    for e0, e1 in dev_ev:
        e0.record(stream)
        F.losa_dense_attn_mass(q, k, v, N, R, C, out=bufs.out, M=M_dense, ws=ws_dense, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    dense_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in dev_ev]))
    del ws_dense, M_dense
    construct_flop = 4.0 * d * float(N) * float(N) * H  # Q K^T and P V over all valid scores
    kernels["dense_attn_mass"] = {"ms": dense_ms, "tflops": construct_flop / (dense_ms * 1e-3) / 1e12,
                                  "frac_bf16_peak": construct_flop / (dense_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                  "launches": "pack_kv + dense (+ add_halves at R = 128)",
                                  "note": "construction step: dense O and exact M in one pass; not in ms_per_step"}
    # Sparse attention that also returns the masses within the lists (the
    # reduced search's evaluation), on the step's lists; not part of ms_per_step.
    ws_sm = torch.empty(F.losa_sparse_attn_mass_workspace(geom), dtype=torch.uint8, device=dev)
    M_list = torch.empty_like(bufs.M)
    sm_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(6)]
    for t, (e0, e1) in enumerate(sm_ev):
        e0.record(stream)
        F.losa_sparse_attn_mass(q, k, v, bufs.row_ptr, bufs.col_idx, bufs.order, N, R, C, out=bufs.out,
                                M=M_list, ws=ws_sm, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    sm_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in sm_ev[1:]]))
    del ws_sm, M_list
    kernels["sparse_attn_mass"] = {"ms": sm_ms, "tflops": kept_flop / (sm_ms * 1e-3) / 1e12,
                                   "frac_bf16_peak": kept_flop / (sm_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                   "launches": "pack_kv + dense over the lists (+ add_halves at R = 128)",
                                   "note": "sparse attention plus the exact masses within the lists (reduced "
                                           "search); kept-block flops; not in ms_per_step"}
    kernels.update(refresh_calls(F, torch, q, k, bufs, geom, wl, stream, dev))
    kernels["select_cache"] = select_cache_leg(F, torch, bufs, geom, wl, stream, dev)


def select_cache_leg(F, torch, bufs, geom, wl, stream, dev, reps=10):
    """The selector alone, cold and warm.  Cold: a 512 MB buffer (twice the
    256 MB Infinity Cache) is overwritten before each call, so the masses come
    from HBM.  Warm: the call repeated back to back (in the step, the masses
    were written by the mass kernel just before)."""
    N, R, C, Na = wl.tokens, wl.block, wl.key_block, wl.tokens_alloc
    nnz = int(bufs.row_ptr[-1].item())
    sel_bytes = 4.0 * geom.rows * geom.n_k + 4.0 * nnz + 8.0 * geom.rows

    def sel():
        F.losa_select(bufs.M, wl.p, N, R, C, tokens_alloc=Na, row_ptr=bufs.row_ptr, col_idx=bufs.col_idx,
                      order=bufs.order, ws=bufs.ws_sel, stream=stream)

    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    out = {}
    for kind in ("cold", "warm"):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        sel()
        for e0, e1 in evs:
            if kind == "cold":
                flush.fill_(1)  # a fill kernel on the same stream
            e0.record(stream)
            sel()
            e1.record(stream)
        torch.cuda.synchronize()
        ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))
        gbs = sel_bytes / (ms * 1e-3) / 1e9
        out[f"{kind}_ms"] = ms
        out[f"{kind}_GBps"] = gbs
        out[f"{kind}_frac_hbm_peak"] = gbs / PEAK_HBM_GBS
    del flush
    out["algorithmic_bytes"] = sel_bytes
    out["note"] = ("median of %d calls; cold: a 512 MB buffer overwritten before each call; not in ms_per_step"
                   % reps)
    return out


ROUTING_P = (0.9, 0.95, 0.99, 0.995, 0.999)
ROUTING_THETA = (0.1, 0.03, 0.01, 0.003, 0.001)


def pooled_routing(F, torch, q, k, bufs, geom, wl, stream, dev):
    """Exact masses vs pooled proxy masses as the selector's input (LoSA page,
    Motivation Summary: coarse estimates are miscalibrated near 99% recall):
    for each p, the true recall (under the exact M) and the coverage of the
    lists built from each.  M in bufs holds the exact masses of this layer."""
    N, R, C = geom.tokens, geom.q_block, geom.k_block
    nq, nk, rows = geom.n_q, geom.n_k, geom.rows
    P = torch.empty_like(bufs.M)
    ws_p = torch.empty(F.losa_pooled_mass_workspace(geom), dtype=torch.uint8, device=dev)
    F.losa_pooled_mass(q, k, N, R, C, out=P, ws=ws_p, stream=stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
    for e0, e1 in evs:
        e0.record(stream)
        F.losa_pooled_mass(q, k, N, R, C, out=P, ws=ws_p, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    pooled_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    w = np.tile(np.array([min(R, N - i * R) for i in range(nq)], np.float64), rows // nq)
    out = {"pooled_ms": pooled_ms, "p": list(ROUTING_P), "exact": {"recall": [], "coverage": []},
           "pooled": {"recall": [], "coverage": []}}
    for p in ROUTING_P:
        for name, src in (("exact", bufs.M), ("pooled", P)):
            F.losa_select(src, p, N, R, C, tokens_alloc=geom.tokens_alloc, row_ptr=bufs.row_ptr,
                          col_idx=bufs.col_idx, order=bufs.order, ws=bufs.ws_sel, stream=stream)
            F.losa_retained_mass(bufs.M, bufs.row_ptr, bufs.col_idx, N, R, C, out=bufs.kept, stream=stream)
            kept = bufs.kept.cpu().numpy().astype(np.float64)
            nnz = int(bufs.row_ptr[-1].item())
            out[name]["recall"].append(float((kept[:, 0] * w).sum() / (kept[:, 1] * w).sum()))
            out[name]["coverage"].append(nnz / float(rows * nk))
    # Online block thresholding (the Sol-Attn page's block thresholding during
    # the online pass): the same two inputs, kept when at least theta times the
    # running maximum.
    thr = {"theta": list(ROUTING_THETA), "exact": {"recall": [], "coverage": []},
           "pooled": {"recall": [], "coverage": []}}
    for theta in ROUTING_THETA:
        for name, src in (("exact", bufs.M), ("pooled", P)):
            F.losa_select_threshold(src, theta, N, R, C, tokens_alloc=geom.tokens_alloc, row_ptr=bufs.row_ptr,
                                    col_idx=bufs.col_idx, order=bufs.order, ws=bufs.ws_sel, stream=stream)
            F.losa_retained_mass(bufs.M, bufs.row_ptr, bufs.col_idx, N, R, C, out=bufs.kept, stream=stream)
            kept = bufs.kept.cpu().numpy().astype(np.float64)
            nnz = int(bufs.row_ptr[-1].item())
            thr[name]["recall"].append(float((kept[:, 0] * w).sum() / (kept[:, 1] * w).sum()))
            thr[name]["coverage"].append(nnz / float(rows * nk))
    for e0, e1 in evs:
        e0.record(stream)
        F.losa_select_threshold(P, ROUTING_THETA[2], N, R, C, tokens_alloc=geom.tokens_alloc, row_ptr=bufs.row_ptr,
                                col_idx=bufs.col_idx, order=bufs.order, ws=bufs.ws_sel, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    thr["select_threshold_ms"] = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs[1:]]))
    out["threshold"] = thr
    out["note"] = ("lists from exact masses vs from pooled proxy masses (block-mean Q/K, block-weighted softmax), "
                   "by top-p and by online thresholding; recall measured under the exact masses")
    return out


_REUSE_LAYER = None


def _drift_step(s):
    """One step's drifted Q/K (bf16 bit patterns) from the layer set before the fork."""
    import synthetic as S
    return S.drift_qk(_REUSE_LAYER, s)


def graph_step_ms(torch, step, stream, steps):
    """The same step captured once in a HIP graph and replayed: every call is
    capture-safe (no allocation, no memset, state only in the caller's
    buffers), so the replay drops the host's per-call work and launch gaps."""
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step(st=side)              # one eager run on the capture stream first
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(st=torch.cuda.current_stream())
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def refresh_calls(F, torch, q, k, bufs, geom, wl, stream, dev):
    """The drift-triggered refresh's two calls on this layer, timed on their own
    (not part of ms_per_step): the query-key drift against a reference copy of
    Q and K (HBM-bound: the four tensors' valid tokens read once), and the
    per-head merge of two list sets (here the step's lists with themselves,
    every other head taken from the second set)."""
    N, R, C = wl.tokens, wl.block, wl.key_block
    q_ref, k_ref = q.clone(), k.clone()
    ws = torch.empty(F.losa_qk_drift_workspace(geom), dtype=torch.uint8, device=dev)
    drift = torch.empty((geom.batch, geom.heads, 2), dtype=torch.float64, device=dev)
    flags = torch.empty((geom.batch, geom.heads), dtype=torch.int32, device=dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(8)]
    for e0, e1 in evs:
        e0.record(stream)
        F.losa_qk_drift(q, k, q_ref, k_ref, N, 0.5, R, C, drift=drift, refresh=flags, ws=ws, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    drift_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs[1:]]))
    drift_bytes = 4.0 * geom.batch * geom.heads * N * geom.head_dim * q.element_size()
    del q_ref, k_ref, ws
    take = (torch.arange(geom.batch * geom.heads, device=dev, dtype=torch.int32) % 2).view(geom.batch, geom.heads)
    rows, nk = geom.rows, geom.n_k
    rp = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    ci = torch.empty(rows * nk, dtype=torch.int32, device=dev)
    order = torch.empty(rows, dtype=torch.int32, device=dev)
    ws = torch.empty(F.losa_merge_lists_workspace(geom), dtype=torch.uint8, device=dev)
    for e0, e1 in evs:
        e0.record(stream)
        F.losa_merge_lists(take, bufs.row_ptr, bufs.col_idx, bufs.row_ptr, bufs.col_idx, N, R, C,
                           tokens_alloc=geom.tokens_alloc, row_ptr=rp, col_idx=ci, order=order, ws=ws, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    merge_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs[1:]]))
    nnz = int(bufs.row_ptr[-1].item())
    merge_bytes = 8.0 * nnz + 4.0 * 5 * rows  # indices read and written; row offsets of both sets, counts, order
    del rp, ci, order, ws
    return {
        "qk_drift": {"ms": drift_ms, "gbs": drift_bytes / (drift_ms * 1e-3) / 1e9,
                     "frac_hbm_peak": drift_bytes / (drift_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "bytes": drift_bytes, "launches": "drift_partial + drift_final",
                     "note": "Q, K and their references read once; not in ms_per_step"},
        "merge_lists": {"ms": merge_ms, "gbs": merge_bytes / (merge_ms * 1e-3) / 1e9, "bytes": merge_bytes,
                        "launches": "pick_counts + order + copy_lists",
                        "note": "launch-latency bound at this size; not in ms_per_step"},
    }


def refresh_trajectory(F, torch, wl, tau, steps_qk, q, k, v, bufs, geom, p_heads, w, stream, dev, frozen_recalls):
    """The reuse trajectory with a drift-triggered refresh (HASTE page, temporal
    mask reuse): at every sparse step, each head's Q and K drift against the
    step its lists were built at; when either exceeds tau the head's lists are
    rebuilt from that step's exact masses with its p (the masses of every head
    are computed, the merge keeps the other heads' lists) and the step's Q and
    K become its reference.  Drift, rebuild and sparse attention are timed."""
    N, R, C, Na = wl.tokens, wl.block, wl.key_block, wl.tokens_alloc
    H, rows, nk = geom.heads, geom.rows, geom.n_k
    q.copy_(steps_qk[wl.construct_step][0])
    k.copy_(steps_qk[wl.construct_step][1])
    q_ref, k_ref = q.clone(), k.clone()
    cur = [bufs.row_ptr.clone(), bufs.col_idx.clone(), bufs.order.clone()]
    new = [torch.empty_like(cur[0]), torch.empty_like(cur[1]), None]
    nxt = [torch.empty_like(t) for t in cur]
    M_new = torch.empty_like(bufs.M)
    ws_d = torch.empty(F.losa_qk_drift_workspace(geom), dtype=torch.uint8, device=dev)
    drift = torch.empty((1, H, 2), dtype=torch.float64, device=dev)
    flags = torch.empty((1, H), dtype=torch.int32, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    drift_ms, rebuild_ms, sparse_ms, recalls, refreshed, drift_max = [], [], [], [], [], []
    for s in range(wl.steps):
        if s == wl.construct_step:
            recalls.append(frozen_recalls[s])
            refreshed.append(0)
            drift_max.append(0.0)
            continue
        q.copy_(steps_qk[s][0])
        k.copy_(steps_qk[s][1])
        ev[0].record(stream)
        F.losa_qk_drift(q, k, q_ref, k_ref, N, tau, R, C, drift=drift, refresh=flags, ws=ws_d, stream=stream)
        ev[1].record(stream)
        f = flags.cpu().numpy()[0]          # the host decides which heads to rebuild
        drift_ms.append(ev[0].elapsed_time(ev[1]))
        drift_max.append(float(drift.cpu().numpy().max()))
        refreshed.append(int(f.sum()))
        if f.any():
            ev[2].record(stream)
            F.losa_block_mass(q, k, N, R, C, out=M_new, ws=bufs.ws_mass, stream=stream)
            F.losa_select(M_new, p_heads, N, R, C, tokens_alloc=Na, want_order=False, row_ptr=new[0],
                          col_idx=new[1], ws=bufs.ws_sel, stream=stream)
            F.losa_merge_lists(flags, cur[0], cur[1], new[0], new[1], N, R, C, tokens_alloc=Na, row_ptr=nxt[0],
                               col_idx=nxt[1], order=nxt[2], ws=bufs.ws_sel, stream=stream)
            ev[3].record(stream)
            cur, nxt = nxt, cur
            for h in np.flatnonzero(f):
                q_ref[:, h].copy_(q[:, h])
                k_ref[:, h].copy_(k[:, h])
            torch.cuda.synchronize()
            rebuild_ms.append(ev[2].elapsed_time(ev[3]))
        ev[4].record(stream)
        F.losa_sparse_attn(q, k, v, cur[0], cur[1], cur[2], N, R, C, out=bufs.out, ws=bufs.ws_attn, stream=stream)
        ev[5].record(stream)
        torch.cuda.synchronize()
        sparse_ms.append(ev[4].elapsed_time(ev[5]))
        # recall of the lists in use under this step's exact masses, not timed
        F.losa_block_mass(q, k, N, R, C, out=bufs.M, ws=bufs.ws_mass, stream=stream)
        F.losa_retained_mass(bufs.M, cur[0], cur[1], N, R, C, out=bufs.kept, stream=stream)
        kept = bufs.kept.cpu().numpy().astype(np.float64)
        recalls.append(float((kept[:, 0] * w).sum() / (kept[:, 1] * w).sum()))
        log(f"refresh leg step {s}: max drift {drift_max[-1]:.3f}, {refreshed[-1]} heads rebuilt, "
            f"recall {recalls[-1]:.6f}")
    total = float(np.sum(drift_ms) + np.sum(rebuild_ms) + np.sum(sparse_ms))
    return {"tau": tau, "measure": "per head, ||X - X_ref||_F / ||X_ref||_F for X = Q and K over the valid tokens",
            "heads_rebuilt_per_step": refreshed, "drift_max_per_step": drift_max,
            "rebuild_steps": int(sum(1 for x in refreshed if x)), "recall_per_step": recalls,
            "mean_recall": float(np.mean(recalls)), "mean_recall_frozen": float(np.mean(frozen_recalls)),
            "min_recall": float(np.min(recalls)), "min_recall_frozen": float(np.min(frozen_recalls)),
            "drift_ms_mean": float(np.mean(drift_ms)),
            "rebuild_ms_mean": float(np.mean(rebuild_ms)) if rebuild_ms else None,
            "sparse_attn_ms_mean": float(np.mean(sparse_ms)),
            "steps_ms_excluding_construction": total}


def run_reuse(args, wl):
    """Frozen-index reuse over the denoising trajectory (construction at one step,
    sparse attention with the frozen lists at every other step)."""
    import torch
    import free_block_sparse_exact_amd as F
    import synthetic as S
    R, C = wl.block, wl.key_block
    N, Na, H, d = wl.tokens, wl.tokens_alloc, wl.heads, wl.head_dim
    dev = torch.device("cuda:0")
    log(f"workload {wl.wid} {wl.name}: {wl.steps} steps, construction at step {wl.construct_step}")
    layer = S.make_layer(wl, keep_f64=True)
    p_heads = [float(x) for x in layer.p_heads]

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    # Every step's Q/K is generated (in parallel, on the host) and resident in
    # HBM before the trajectory runs, so the timed steps follow one another as
    # in a sampler instead of waiting on the generator.
    global _REUSE_LAYER
    _REUSE_LAYER = layer
    import multiprocessing as mp
    t0 = time.time()
    with mp.get_context("fork").Pool(min(8, os.cpu_count() or 1)) as pool:
        steps_qk = []
        for qs_, ks_ in pool.imap(_drift_step, range(wl.steps)):
            steps_qk.append((to_dev(qs_), to_dev(ks_)))
    log(f"generated {wl.steps} steps of Q/K in {time.time() - t0:.1f}s")
    v = to_dev(layer.v)
    geom = F.Geometry(1, H, N, Na, d, R, C, F.LOSA_BF16)
    nq, nk, rows = geom.n_q, geom.n_k, geom.rows
    q = torch.empty_like(v)
    k = torch.empty_like(v)
    bufs = Buffers(F, torch, q, k, v, geom, dev)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    w = np.tile(np.array([min(R, N - i * R) for i in range(nq)], np.float64), H)

    def load_step(s):
        q.copy_(steps_qk[s][0])
        k.copy_(steps_qk[s][1])

    # construction step: dense attention with the exact masses in one pass, then
    # the selection, from the construction step's Q/K (the step's output is the
    # dense O)
    ws_dense = torch.empty(F.losa_dense_attn_mass_workspace(geom), dtype=torch.uint8, device=dev)
    load_step(wl.construct_step)
    for warm in (True, False):
        ev[0].record(stream)
        F.losa_dense_attn_mass(q, k, v, N, R, C, out=bufs.out, M=bufs.M, ws=ws_dense, stream=stream)
        F.losa_select(bufs.M, p_heads, N, R, C, tokens_alloc=Na, row_ptr=bufs.row_ptr, col_idx=bufs.col_idx,
                      order=bufs.order, ws=bufs.ws_sel, stream=stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
    construct_ms = ev[0].elapsed_time(ev[1])
    del ws_dense
    # every other step: sparse attention on the frozen lists with that step's Q/K
    sparse_ms, recalls = [], []
    # rows whose recall the CPU baseline leg recomputes with the oracle (GPU side kept here)
    sample_rows = [(h, i) for h in (0, H // 2, H - 1) for i in (0, nq // 2, nq - 1)]
    sample_r = [h * nq + i for h, i in sample_rows]
    sample_kept = []
    for s in range(wl.steps):
        load_step(s)
        if s != wl.construct_step:
            ev[2].record(stream)
            F.losa_sparse_attn(q, k, v, bufs.row_ptr, bufs.col_idx, bufs.order, N, R, C, out=bufs.out,
                               ws=bufs.ws_attn, stream=stream)
            ev[3].record(stream)
            torch.cuda.synchronize()
            sparse_ms.append(ev[2].elapsed_time(ev[3]))
        # recall of the frozen lists under this step's exact (GPU) masses, not timed
        F.losa_block_mass(q, k, N, R, C, out=bufs.M, ws=bufs.ws_mass, stream=stream)
        F.losa_retained_mass(bufs.M, bufs.row_ptr, bufs.col_idx, N, R, C, out=bufs.kept, stream=stream)
        kept = bufs.kept.cpu().numpy().astype(np.float64)
        recalls.append(float((kept[:, 0] * w).sum() / (kept[:, 1] * w).sum()))
        sample_kept.append(kept[sample_r])
        log(f"step {s}: recall {recalls[-1]:.6f}" + (f", sparse {sparse_ms[-1]:.3f} ms" if s != wl.construct_step else ""))
    # Reduced search at the last step (GSRS card: a later top-p search within the
    # earlier candidate set, on exact weights computed inside the attention
    # pass): the masses within the frozen lists from this step's Q/K, then the
    # same per-head p within them.  bufs.M still holds this step's exact masses.
    ws_sm = torch.empty(F.losa_sparse_attn_mass_workspace(geom), dtype=torch.uint8, device=dev)
    M_list = torch.empty_like(bufs.M)
    out2 = torch.empty_like(bufs.out)
    for warm in (True, False):
        ev[2].record(stream)
        F.losa_sparse_attn_mass(q, k, v, bufs.row_ptr, bufs.col_idx, bufs.order, N, R, C, out=out2, M=M_list,
                                ws=ws_sm, stream=stream)
        ev[3].record(stream)
        torch.cuda.synchronize()
    reduced_ms = ev[2].elapsed_time(ev[3])
    rp2, ci2, _ = F.losa_select(M_list, p_heads, N, R, C, tokens_alloc=Na)
    F.losa_retained_mass(bufs.M, rp2, ci2, N, R, C, out=bufs.kept, stream=stream)
    kept2 = bufs.kept.cpu().numpy().astype(np.float64)
    reduced = {"step": wl.steps - 1, "sparse_attn_mass_ms": reduced_ms,
               "candidate_blocks": int(bufs.row_ptr[-1].item()), "kept_blocks": int(rp2[-1].item()),
               "recall_frozen_lists": recalls[-1],
               "recall_reduced_lists": float((kept2[:, 0] * w).sum() / (kept2[:, 1] * w).sum()),
               "p": "the per-head p, applied within the candidates"}
    del ws_sm, M_list, out2
    log(f"reduced search at step {wl.steps - 1}: {reduced['kept_blocks']} of {reduced['candidate_blocks']} blocks, "
        f"recall {reduced['recall_reduced_lists']:.4f} (frozen {recalls[-1]:.4f}), {reduced_ms:.3f} ms")
    refresh = refresh_trajectory(F, torch, wl, args.refresh_tau, steps_qk, q, k, v, bufs, geom, p_heads, w, stream,
                                 dev, recalls)
    rp = bufs.row_ptr.cpu().numpy().astype(np.int64)
    counts = np.diff(rp)
    nnz = int(rp[-1])
    per_head = counts.reshape(H, nq).sum(axis=1).astype(np.float64)
    order = bufs.order.cpu().numpy()
    per_xcd = xcd_loads(order, counts, R // 64)
    mean_sparse = float(np.mean(sparse_ms))
    kept_flop = 4.0 * d * R * C * nnz
    res = {
        "metric": METRIC,
        "value": kept_flop / (mean_sparse * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": wl.steps,
        "warmup": 0,
        "ms_per_step": (construct_ms + float(np.sum(sparse_ms))) / wl.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; Q/K drift q_s = q_0 + 0.02 s N(0,1) per step; no trained weights)",
        "config": {"workload": wl.name, "heads": H, "head_dim": d, "tokens": N, "block": R, "k_block": C,
                   "p_per_head": p_heads, "construct_step": wl.construct_step, "parallelism": "single GPU"},
        "construct_dense_mass_select_ms": construct_ms,
        "sparse_attn_ms_mean": mean_sparse,
        "trajectory_ms": construct_ms + float(np.sum(sparse_ms)),
        "recall_per_step": recalls,
        "coverage_per_head": (per_head / (nq * nk)).tolist(),
        "imbalance_per_head_max_over_mean": float(per_head.max() / per_head.mean()),
        "imbalance_per_xcd_max_over_mean": float(per_xcd.max() / per_xcd.mean()),
        "imbalance_per_xcd_note": "kept blocks dealt to each XCD by the sparse attention's workgroup mapping "
                                  "(a static count, not measured busy time)",
        "reduced_search": reduced,
        "drift_refresh": refresh,
        "cpu_baseline": None,
    }
    if args.cpu_rows > 0:
        log("timing the CPU oracle baseline (recall and sparse attention of sampled rows at every step) ...")
        res["cpu_baseline"] = reuse_cpu_baseline(wl, steps_qk, v, bufs, sample_rows, sample_kept, args.cpu_budget)
    print(json.dumps(res))


def reuse_cpu_baseline(wl, steps_qk, v, bufs, sample_rows, sample_kept, budget_s):
    """The oracle on sampled rows of every step of the reuse trajectory: the
    exact masses of each row under that step's Q/K (the recall of the frozen
    lists, set beside the GPU's recall of the same rows) and the sparse
    attention over the frozen list (timed, kept-block TFLOP/s).  Sample: three
    rows (first, middle and last query block) of three heads per step; steps
    past the time budget are skipped and reported as null."""
    import oracle as O
    import synthetic as S
    N, R, C, d = wl.tokens, wl.block, wl.key_block, wl.head_dim
    nq = wl.n_blocks
    rp = bufs.row_ptr.cpu().numpy().astype(np.int64)
    ci = bufs.col_idx[:int(rp[-1])].cpu().numpy()
    vh = {h: S.to_f64(v[:, h:h + 1].cpu().view(torch_int16()).numpy(), wl.dtype) for h, _ in sample_rows}
    t_start = time.time()
    t_attn, flops = 0.0, 0.0
    oracle_rec, gpu_rec = [], []
    for s in range(wl.steps):
        if time.time() - t_start > budget_s:
            oracle_rec.append(None)
            gpu_rec.append(None)
            continue
        num_o = den_o = num_g = den_g = 0.0
        for t, (h, i) in enumerate(sample_rows):
            qh = S.to_f64(steps_qk[s][0][:, h:h + 1].cpu().view(torch_int16()).numpy(), wl.dtype)
            kh = S.to_f64(steps_qk[s][1][:, h:h + 1].cpu().view(torch_int16()).numpy(), wl.dtype)
            m = O.block_mass_rows(qh, kh, N, R, C, [(0, 0, i)])[0]
            r = h * nq + i
            lst = ci[rp[r]:rp[r + 1]]
            wi = min(R, N - i * R)
            num_o += wi * m[lst].sum()
            den_o += wi * m.sum()
            num_g += wi * sample_kept[s][t, 0]
            den_g += wi * sample_kept[s][t, 1]
            rp1 = np.array([0] * (i + 1) + [len(lst)], np.int64)
            t0 = time.time()
            O.sparse_attention_rows(qh, kh, vh[h], N, R, C, rp1, lst.astype(np.int32), [(0, 0, i)])
            t_attn += time.time() - t0
            flops += 4.0 * d * R * C * len(lst)
        oracle_rec.append(float(num_o / den_o))
        gpu_rec.append(float(num_g / den_g))
    try:
        from threadpoolctl import threadpool_info
        cores = max([x.get("num_threads", 1) for x in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    diffs = [abs(a - b) for a, b in zip(oracle_rec, gpu_rec) if a is not None]
    return {"value": flops / t_attn / 1e12 if t_attn > 0 else None, "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{len(sample_rows)} query blocks (first, middle, last of three heads) at each of "
                      f"{sum(x is not None for x in oracle_rec)} steps: exact masses (recall of the frozen lists) and "
                      f"sparse attention over the frozen list; value = the oracle's kept-block TFLOP/s on them",
            "recall_sampled_oracle_per_step": oracle_rec, "recall_sampled_gpu_per_step": gpu_rec,
            "recall_sampled_max_abs_diff": max(diffs) if diffs else None, "cpu": cpu_model()}


def torch_int16():
    import torch
    return torch.int16


def copy_calibration():
    """A plain device copy of known size, for scaling the PMC byte counters."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "repeats": 3}))


def summarize_pmc(workload, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """Per-launch HBM traffic of the mass, selection and sparse-attention
    calls of one workload from rocprofv3 CSVs, scaled by a plain copy of
    1 GiB (FETCH_SIZE/WRITE_SIZE are in KiB).  Kernels launched by more than
    one call (the selector's scan kernels also serve other list builders) are
    counted over every launch of the run, so the run should time the plain
    step only (--steps 1 --warmup 1 --legs step)."""
    import synthetic as S
    wl = S.get_workload(workload)
    import csv

    def read(d, counter):
        path = os.path.join(d, "run_counter_collection.csv")
        out = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return out

    def copy_factor(d, counter):
        # the 1 GiB copy is the largest dispatch under the counter
        vals = [v for k, vs in read(d, counter).items() if "opy" in k for v in vs]
        return (1 << 30) / float(np.median(vals)) if vals else None

    fetch, write = read(fetch_dir, "FETCH_SIZE"), read(write_dir, "WRITE_SIZE")
    ff, wf = copy_factor(copy_fetch_dir, "FETCH_SIZE"), copy_factor(copy_write_dir, "WRITE_SIZE")

    def per_launch(tab, key):
        vals = [v for k, vs in tab.items() if re.search(key, k) for v in vs]
        return float(np.mean(vals)) if vals else 0.0

    calls = {}
    for key, part, call in PMC_KERNELS:
        f_raw, w_raw = per_launch(fetch, key), per_launch(write, key)
        if f_raw == 0.0 and w_raw == 0.0:
            continue  # not launched for this shape
        c = calls.setdefault(call, {"sources_sha256_16": sources_hash(CALL_SOURCES[call]), "kernels": {}, "bytes": 0.0})
        b = f_raw * (ff or 1.0) + w_raw * (wf or 1.0)
        c["kernels"][part] = {"fetch_kib_raw": f_raw / 1024.0, "write_kib_raw": w_raw / 1024.0, "bytes": b}
        c["bytes"] += b
    out = {
        "workload": f"{wl.name}: {wl.heads} heads x {wl.head_dim}, {wl.tokens} tokens, {wl.block}-token query "
                    f"blocks, {wl.key_block}-token key blocks, p = {wl.p}",
        "copy_scale": {"FETCH_SIZE": ff, "WRITE_SIZE": wf},
        "calls": calls,
        "command": f"rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -d DIR -o run -- python -u "
                   f"bench.py --workload {workload} --steps 1 --warmup 1 --cpu-rows 0 --legs step; copy scale from "
                   f"rocprofv3 --pmc <same counter> -- python -u bench.py --copy-calibration; summary by python "
                   f"bench.py --summarize-pmc {workload} DIRS",
    }
    path = traffic_file(wl.name)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


# kernel name pattern -> (short name, call it belongs to)
TRACE_KERNELS = [
    (_ATTN_INPASS, "attn_bf16_kernel (in-pass thresholding)", "losa_sparse_attn_threshold"),
    (_ATTN, "attn_bf16_kernel", "losa_sparse_attn"),
    (_PACK_KV, "pack_kv_kernel (K and V)",
     "losa_sparse_attn, losa_dense_attn_mass, losa_sparse_attn_mass, losa_sparse_attn_threshold"),
    (_PACK_K, "pack_kv_kernel (K only)", "losa_block_mass"),
    (r"mass_bf16_kernel", "mass_bf16_kernel", "losa_block_mass"),
    (_DENSE_LISTS, "dense_bf16_kernel (lists)", "losa_sparse_attn_mass"),
    (_DENSE, "dense_bf16_kernel", "losa_dense_attn_mass"),
    (r"pool_kernel(<__bf16, \d+, double>|IDF16bLi\d+EdE)", "pool_kernel (fp64 block means)",
     "losa_sparse_attn_threshold"),
    (r"pool_kernel", "pool_kernel", "losa_pooled_mass"),
    (r"proxy_kernel", "proxy_kernel", "losa_pooled_mass"),
    (r"cut_wave_kernel", "cut_wave_kernel", "losa_select"),
    (r"cut_group_kernel", "cut_group_kernel", "losa_select"),
    (r"order_kernel", "order_kernel", "losa_select, losa_select_threshold, losa_merge_lists"),
    (r"compact_kernel", "compact_kernel", "losa_select"),
    (r"retained_kernel", "retained_kernel", "losa_retained_mass"),
    (r"drift_partial_kernel", "drift_partial_kernel", "losa_qk_drift"),
    (r"drift_final_kernel", "drift_final_kernel", "losa_qk_drift"),
    (r"threshold_kernel(<false>|ILb0)", "threshold_kernel (counts)", "losa_select_threshold"),
    (r"threshold_kernel(<true>|ILb1)", "threshold_kernel (indices)", "losa_select_threshold"),
    (r"pick_counts_kernel", "pick_counts_kernel", "losa_merge_lists"),
    (r"copy_lists_kernel", "copy_lists_kernel", "losa_merge_lists"),
]


def summarize_trace(trace_dir, name, command):
    """Short text summary of a rocprofv3 --kernel-trace --stats run: average
    duration per kernel and per library call (the sums that the HIP events in
    this benchmark bracket)."""
    import csv
    path = os.path.join(trace_dir, "run_kernel_stats.csv")
    rows = list(csv.DictReader(open(path)))
    lines = [f"# rocprofv3 kernel statistics: {name}", "",
             "Command (run from the repository root, after building the library):", "",
             "    " + command, "",
             "| kernel | call | launches | average us | min us | max us | share of GPU time |",
             "|---|---|---|---|---|---|---|"]
    per_call, own, shared = {}, {}, {}
    for r in rows:
        label = kernel_label(r["Name"], TRACE_KERNELS)
        if label is None:
            continue
        short, call = label
        avg = float(r["AverageNs"]) / 1e3
        lines.append(f"| {short} | {call} | {r['Calls']} | {avg:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f}% |")
        calls = call.split(", ")
        if len(calls) == 1:
            own.setdefault(calls[0], []).append((avg, int(r["Calls"])))
        else:
            for c in calls:
                shared[c] = shared.get(c, 0.0) + avg
    # A kernel shared by several calls (the packing, the work order) runs once
    # per call and does not show which of them ran: a call is listed when a
    # kernel of its own did.  A call's own kernels launch n or a multiple of n
    # times (n = its fewest), e.g. the block means once for Q and once for K.
    for c, ks in own.items():
        n = min(k for _, k in ks)
        per_call[c] = shared.get(c, 0.0) + sum(a * round(k / n) for a, k in ks)
    lines += ["", "Average per library call (its kernels' average durations times their launches per call):", ""]
    lines += [f"* {call}: {us / 1e3:.3f} ms" for call, us in per_call.items()]
    lines.append("")
    out = os.path.join(ROOT, "profiles", name + ".md")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


CLOCK_KERNELS = [(_ATTN, "attn_bf16_kernel", "sparse_attn"),
                 (r"mass_bf16_kernel", "mass_bf16_kernel", "block_mass"),
                 (_DENSE, "dense_bf16_kernel", "dense_attn_mass")]
N_XCD, N_SE = 8, 32          # MI355X: 8 XCDs, 4 shader engines each
PEAK_CLOCK_GHZ = 2.4         # the clock the published 2.5 PFLOP/s bf16 peak assumes


def summarize_clock(pmc_dir, trace_dir, name, commands):
    """Clock the matrix-core kernels actually run at: GRBM_GUI_ACTIVE counts
    busy GPU-clock cycles (rocprofv3 sums it over the 8 XCDs), SQ_BUSY_CYCLES
    the same per shader engine (summed over 32); busy cycles per XCD over the
    kernel's unprofiled median duration give the sustained clock."""
    import csv
    pmc = {}
    for r in csv.DictReader(open(os.path.join(pmc_dir, "run_counter_collection.csv"))):
        lab = (kernel_label(r["Kernel_Name"], CLOCK_KERNELS) or (None,))[0]
        if lab is None:
            continue
        d = pmc.setdefault(lab, {}).setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    durs = {}
    for r in csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv"))):
        lab = (kernel_label(r["Kernel_Name"], CLOCK_KERNELS) or (None,))[0]
        if lab is not None:
            durs.setdefault(lab, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    trace = {lab: float(np.median(v)) for lab, v in durs.items()}
    lines = [f"# Sustained clock of the matrix-core kernels: {name}", "",
             "Commands (run from the repository root, after building the library):", ""]
    lines += ["    " + c for c in commands.split(" ;; ")]
    lines += ["", "GRBM_GUI_ACTIVE is summed over the 8 XCDs and SQ_BUSY_CYCLES over the 32 shader "
              "engines; both give the busy cycles of one XCD.  Clock = those cycles / the kernel's "
              f"median duration in the kernel trace (no counters attached).  The published bf16 peak "
              f"(2.5 PFLOP/s) assumes {PEAK_CLOCK_GHZ} GHz.", "",
              "| kernel | dispatches | GRBM cycles per XCD (M) | SQ busy cycles per SE (M) | trace median us | "
              "sustained clock GHz | share of the 2.4 GHz rate |",
              "|---|---|---|---|---|---|---|"]
    for lab in dict.fromkeys(k for _, k, _ in CLOCK_KERNELS):
        if lab not in pmc or lab not in trace:
            continue
        ds = list(pmc[lab].values())
        grbm = sum(d.get("GRBM_GUI_ACTIVE", 0.0) for d in ds) / len(ds) / N_XCD
        sq = sum(d.get("SQ_BUSY_CYCLES", 0.0) for d in ds) / len(ds) / N_SE
        ghz = grbm / trace[lab]
        lines.append(f"| {lab} | {len(ds)} | {grbm / 1e6:.2f} | {sq / 1e6:.2f} | {trace[lab] / 1e3:.1f} | "
                     f"{ghz:.2f} | {ghz / PEAK_CLOCK_GHZ:.2f} |")
    lines.append("")
    out = os.path.join(ROOT, "profiles", name + ".md")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def summarize_mfma(pmc_dir, name, command):
    """Matrix-core utilisation from rocprofv3's derived counters: MfmaUtil =
    MFMA-busy SIMD cycles / (busy GPU cycles x SIMDs), clock-independent;
    MfmaFlopsBF16 = bf16 MFMA flops the hardware executed (padding and
    recomputed chunks included), to set beside the algorithmic count."""
    import csv
    per = {}
    for r in csv.DictReader(open(os.path.join(pmc_dir, "run_counter_collection.csv"))):
        lab = (kernel_label(r["Kernel_Name"], CLOCK_KERNELS) or (None,))[0]
        if lab is None:
            continue
        d = per.setdefault(lab, {}).setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    lines = [f"# Matrix-core utilisation: {name}", "", "Command (run from the repository root, after building the library):",
             "", "    " + command, "",
             "MfmaUtil = MFMA-busy SIMD cycles / (busy GPU cycles x SIMDs), in percent: the matrix cores' share "
             "of the cycles the kernel ran, independent of the clock.  MfmaFlopsBF16 = bf16 MFMA flops executed.",
             "", "| kernel | dispatches | MfmaUtil % | bf16 MFMA TFLOP executed per dispatch |", "|---|---|---|---|"]
    for lab in dict.fromkeys(k for _, k, _ in CLOCK_KERNELS):
        if lab not in per:
            continue
        ds = list(per[lab].values())
        util = sum(d.get("MfmaUtil", 0.0) for d in ds) / len(ds)
        fl = sum(d.get("MfmaFlopsBF16", 0.0) for d in ds) / len(ds)
        lines.append(f"| {lab} | {len(ds)} | {util:.1f} | {fl / 1e12:.3f} |")
    lines.append("")
    out = os.path.join(ROOT, "profiles", name + ".md")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


if __name__ == "__main__":
    main()
