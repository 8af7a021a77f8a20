"""Benchmark of the fused linear log-prob operator on one MI355X.

One step = one pass of the whole hot path over one batch of 4096 synthetic tokens shaped
like a Qwen3-8B LM head (H=4096, real vocabulary 151669 padded to 151936, tau=0.7, no bias,
targets sampled from the fp64 softmax, stored under tests/golden):
  1. llp_forward   -- layout/mask indexing, fused bf16 MFMA GEMM + online max/sum-exp/
                      target/entropy epilogue, fixed-order cross-tile combine;
  2. llp_merge     -- rank-ordered merge of the shard partials (here one shard);
  3. llp_backward  -- gradient recompute G (bf16), dhidden = G W, dweight = G^T h
                      (LLP_FLAG_OVERWRITE_GRADS: the step's one batch is its whole
                      gradient; the accumulate form, dweight += G^T h, is timed apart);
  4. llp_top_p_replay x 4 shards + llp_merge -- compact top-p replay scoring of 4096 rows of
                      fp32 logits [4096, 151936] with <= 64 candidate ids per row.
Inputs are resident in HBM before the timed region. The value is scored tokens/s of the
step. Per-phase times come from HIP events recorded on the stream the kernels run on.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
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

METRIC = "scored tokens/s + MFMA util, fused linear-logp fwd(+bwd) at H=4096, V=151936"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
T, H, VR, VP, TAU = 4096, 4096, 151669, 151936, 0.7
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_kernel.json")
KERNEL_SOURCES = [os.path.join(ROOT, "lm_head_linear_logp_amd", "csrc", f)
                  for f in ("llp_kernels.hip", "llp_tile.hpp")]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code: comments and whitespace are left out, so that only a
    change to the code itself marks the committed counters as stale."""
    import re
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per forward-kernel launch from the committed counter summary, or None when
    the kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("bytes_per_launch")


def ingest_pmc(fetch_csv: str, write_csv: str) -> None:
    """Write profiles/traffic_fwd_kernel.json from two rocprofv3 --pmc counter CSVs (one pass
    with FETCH_SIZE, one with WRITE_SIZE, both of `bench.py --copy-calibration`). Each counter
    (KiB per dispatch) is scaled by the ratio of the known bytes of the 1 GiB device copy to
    what the same counter reads for that copy."""
    import csv

    def per_dispatch(path, counter):
        return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in csv.DictReader(open(path))
                if r["Counter_Name"] == counter]

    fd, wd = per_dispatch(fetch_csv, "FETCH_SIZE"), per_dispatch(write_csv, "WRITE_SIZE")
    fwd = next(k for k, _ in fd if "k_fwd" in k)

    def mean(ds, name):
        v = [x for k, x in ds if k == name]
        return sum(v) / len(v)

    # The calibration copy is the largest copy dispatch (other copies move a few KiB).
    copy = "__amd_rocclr_copyBuffer"
    f = {fwd: mean(fd, fwd), copy: max(x for k, x in fd if k == copy)}
    w = {fwd: mean(wd, fwd), copy: max(x for k, x in wd if k == copy)}
    gib_kib = (1 << 30) / 1024.0
    fs, ws = gib_kib / f[copy], gib_kib / w[copy]
    out = {"kernel": fwd, "kernel_source_hash": kernel_source_hash(),
           "fetch_kib_per_dispatch": f[fwd], "write_kib_per_dispatch": w[fwd],
           "copy_kernel": copy, "copy_fetch_kib": f[copy], "copy_write_kib": w[copy],
           "fetch_scale": fs, "write_scale": ws,
           "bytes_per_launch": (f[fwd] * fs + w[fwd] * ws) * 1024.0,
           "algorithmic_bytes_per_launch": float(2 * (VR * H + T * H) + T * 64),
           "command": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -- "
                      "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --skip-config4 --copy-calibration"}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def host_cpu() -> dict:
    """The host the CPU baseline runs on: CPU model, logical CPUs, CPUs this process may use,
    and the BLAS thread count the oracle's matrix products get."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        blas = os.cpu_count()
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable,
            "blas_threads": int(blas), "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def cpu_baseline(rows: int = 2560, topp: dict = None) -> dict:
    """The fp64 oracle (as it stands) timed on this host's cores, excluding input generation
    and conversion:
      * the bench workload: forward + backward of `rows` of the 4096 config-2 rows (the
        reported value, scaled to scored tokens/s);
      * config 1 (T=64, H=256, V=1000/1024): forward, 1 warm-up + 5 reps, in ms;
      * config 5 (top-p replay of 4096 rows over 4 shards and the merge): 1 rep, in s;
      * config 4 (16 packed sequences, 40874 scored rows, forward + backward): stated from the
        measured per-row forward+backward rate, which it shares (the same products per row;
        the per-chunk dweight product is part of that rate), not run (it would take minutes)."""
    import oracle
    import synth
    hc = host_cpu()
    base = synth.config2_base()
    tg = np.loadtxt(os.path.join(ROOT, "tests", "golden", "config2_targets.txt"), dtype=np.int64,
                    comments="#")
    w64 = oracle.bf16_to_f64(synth.full_weight()[:VR])   # input conversion, not timed
    h = base["hidden"][:rows]
    dlogp = synth.rng(2, 70).standard_normal(rows)
    log(f"cpu baseline: oracle forward+backward of {rows} rows")
    t0 = time.perf_counter()
    f = oracle.forward(h, w64, None, TAU, tg[:rows], None, VR)
    oracle.backward(h, w64, None, TAU, tg[:rows], None, 0, VP, VR, f["lse"], dlogp)
    dt = time.perf_counter() - t0
    del w64
    c1 = synth.config1()
    c1w = oracle.bf16_to_f64(c1["weight"])
    reps = []
    for i in range(6):
        t1 = time.perf_counter()
        oracle.forward(c1["hidden"], c1w, c1["bias"], c1["temperature"], c1["targets"],
                       c1["mask"], c1["real_vocab"])
        if i:
            reps.append((time.perf_counter() - t1) * 1e3)
    log("cpu baseline: oracle top-p replay of config 5")
    tp = topp if topp is not None else synth.topp_case()
    t1 = time.perf_counter()
    parts = []
    for off, n in synth.shard_ranges():
        p = oracle.top_p_replay(tp["logits"][:, off:off + n], tp["replay_ids"], tp["targets"],
                                TAU, off, n, VR)
        p["entropy"] = None
        parts.append(p)
    oracle.merge(parts)
    c5 = time.perf_counter() - t1
    c4_scored = int(synth.config4_layout()["mask"].sum())
    rate = rows / dt
    return {"value": rate, "unit": "scored tokens/s", "cores": hc["blas_threads"],
            "kind": "oracle", "host": hc,
            "sample": f"fp64 oracle forward+backward of {rows} of the 4096 rows "
                      f"(H=4096, V=151669/151936), {dt:.1f} s on {hc['blas_threads']} BLAS "
                      f"threads",
            "config1_forward_ms": {"median": float(np.median(reps)), "min": float(min(reps)),
                                   "reps": len(reps)},
            "config5_topp_4shards_merge_s": c5,
            "config4_forward_backward_s_stated": {
                "value": c4_scored / rate, "scored_rows": c4_scored,
                "how": "scored rows / the measured forward+backward rate (not run)"}}


def gpu_clock_sampler(device_index: int = 0):
    """Samples the GPU's graphics clock (amdsmi) in a background thread while the timed steps
    run. Returns (start, stop) callables; stop() gives a summary dict, or None with a reason
    when no sample could be taken."""
    import threading
    state = {"samples": [], "error": None}
    stop_ev = threading.Event()

    def pick_handle(amdsmi):
        import torch
        handles = amdsmi.amdsmi_get_processor_handles()
        if len(handles) == 1:
            return handles[0]
        pr = torch.cuda.get_device_properties(device_index)
        bus = getattr(pr, "pci_bus_id", None)
        for h in handles:
            bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)     # "dddd:bb:dd.f"
            if bus is not None and int(bdf.split(":")[1], 16) == int(bus):
                return h
        return handles[0]

    def run():
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            try:
                h = pick_handle(amdsmi)
                while not stop_ev.is_set():
                    m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                    cur = m.get("current_gfxclks")
                    vals = [v for v in (cur if isinstance(cur, (list, tuple)) else [cur])
                            if isinstance(v, (int, float)) and 0 < v < 10000]
                    if not vals:
                        v = m.get("average_gfxclk_frequency")
                        vals = [v] if isinstance(v, (int, float)) and 0 < v < 10000 else []
                    if vals:
                        state["samples"].append(tuple(float(v) for v in vals))
                    stop_ev.wait(0.01)
            finally:
                amdsmi.amdsmi_shut_down()
        except Exception as e:  # no amdsmi, no permission, unknown metrics layout
            state["error"] = f"{type(e).__name__}: {e}"

    th = threading.Thread(target=run, daemon=True)

    def stop():
        stop_ev.set()
        th.join(timeout=5)
        xs = state["samples"]
        if not xs:
            return {"mhz_median": None, "reason": state["error"] or "no samples"}
        mean = np.array([np.mean(x) for x in xs])
        per = [np.median([x[i] for x in xs if len(x) > i]) for i in range(max(len(x) for x in xs))]
        return {"mhz_median": float(np.median(mean)), "mhz_min": float(mean.min()),
                "mhz_max": float(mean.max()), "samples": len(xs),
                "distinct_samples": len(set(xs)),
                "per_xcd_mhz_median": [float(v) for v in per],
                "source": "amdsmi gpu_metrics current_gfxclks (mean over XCDs), sampled every "
                          "10 ms from the warm-up to the end of the timed steps; the firmware "
                          "refreshes these values less often than that (distinct_samples)"}
    return th.start, stop


def measure_vendor_gemm(h, W, stream, fwd, reps=20):
    """Context for the forward's roofline fraction: the vendor library's plain GEMM of the same
    operands (torch.matmul -> hipBLASLt), h [4096, 4096] x W^T over the padded vocabulary, bf16
    logits out and no epilogue. It is not part of the path; it shows the MFMA rate a tuned
    library reaches on this shape under the chip's power limit. The clock takes tens of
    milliseconds to settle after a change of load, so both kernels first run 15 times, then
    `reps` pairs (vendor GEMM, fused forward) alternate, each call timed with HIP events on the
    stream; medians are reported, so the two figures are taken under the same conditions."""
    import torch
    out = torch.empty((h.shape[0], W.shape[0]), dtype=torch.bfloat16, device=h.device)
    wt = W.t()
    gemm = lambda: torch.matmul(h, wt, out=out)
    for _ in range(15):
        gemm()
        fwd()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps + 1)]
    ev[0].record(stream)
    for i in range(reps):
        gemm()
        ev[2 * i + 1].record(stream)
        fwd()
        ev[2 * i + 2].record(stream)
    torch.cuda.synchronize()
    d = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(2 * reps)])
    g_ms, f_ms = float(np.median(d[0::2])), float(np.median(d[1::2]))
    del out
    flop = 2.0 * h.shape[0] * h.shape[1] * W.shape[0]
    tf = flop / (g_ms * 1e-3) / 1e12
    return {"vendor_gemm": {"what": "torch.matmul (hipBLASLt) of h [4096, 4096] by W^T "
                                    "[4096, 151936], bf16 out, no epilogue; median of 20 calls "
                                    "alternating with the fused forward after 15 warm-up pairs",
                            "us": g_ms * 1e3, "tflops": tf, "frac": tf / PEAK_BF16_TFLOPS,
                            "fused_forward_alternating_us": f_ms * 1e3,
                            "fused_forward_alternating_frac":
                                2.0 * T * H * VR / (f_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}}


def measure_next_rows(llp, logits, rids, rtg, shards, stream, busy, reps=10):
    """The rows beyond the step, on the same config-5 logits [4096, 151936] fp32, timed with
    HIP events on the launch stream (mean over `reps` calls after a warm-up call):
    the logits-input forward over the full real vocabulary (HBM bound: it reads every real
    logit once), and the dense keep-mask replay of the same nuclei over the 4 shards next to
    the compact replay (the dense pass reads the whole T x V_loc mask). `busy` queues a
    few milliseconds of GPU work ahead of each timed group, so that the host has enqueued the
    group's calls before the GPU reaches them and the events see kernel time, not the gaps of
    per-call host overhead."""
    import torch

    def timed(fn):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        busy()
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps  # ms

    log("logits-input forward and dense keep mask (config-5 logits)")
    lf_ms = timed(lambda: llp.forward_logits(logits, rtg, temperature=TAU, real_vocab=VR,
                                             padded_vocab=VP))
    lf_bytes = T * VR * 4 + T * (8 + 17)      # every real logit once; target in, partials out
    keep = torch.zeros((T, VP), dtype=torch.uint8, device="cuda")
    valid = rids >= 0
    keep[torch.arange(T, device="cuda")[:, None].expand_as(rids)[valid], rids[valid]] = 1

    # The replay calls take microseconds at T=4096, less than a call's host overhead, so the
    # dense/compact comparison runs on config 5 tiled 16x (T=65536, the size the cost ratio
    # is quoted at): the same rows repeated.
    rep = 16
    logits_b, keep_b = logits.repeat(rep, 1), keep.repeat(rep, 1)
    rids_b, rtg_b = rids.repeat(rep, 1), rtg.repeat(rep)
    del keep
    Tb = T * rep

    def dense():
        for r, (off, n) in enumerate(shards):
            llp.keep_mask_replay(logits_b[:, off:off + n], keep_b[:, off:off + n], rtg_b,
                                 temperature=TAU, offset=off, real_vocab=VR, padded_vocab=VP,
                                 rank=r, world=4, local_size=n)

    def compact():
        for r, (off, n) in enumerate(shards):
            llp.top_p_replay(logits_b[:, off:off + n], rids_b, rtg_b, temperature=TAU,
                             offset=off, real_vocab=VR, padded_vocab=VP, rank=r, world=4,
                             local_size=n)

    dense_ms, compact_ms = timed(dense), timed(compact)
    dense_bytes = Tb * VR * 1 + rep * int(valid.sum().item()) * 4 + Tb * 4 * (8 + 13)
    # Compact replay, per row and shard: 64 ids (512 B), the target (8 B), 13 B of partials;
    # each distinct candidate's logit (4 B) once over the shards.
    srt = rids.sort(dim=1).values
    uniq = int(((srt[:, 1:] != srt[:, :-1]) & (srt[:, 1:] >= 0)).sum().item()
               + (srt[:, 0] >= 0).sum().item())
    compact_bytes = Tb * 4 * (64 * 8 + 8 + 13) + rep * uniq * 4
    del logits_b, keep_b, rids_b, rtg_b
    return {
        "logits_forward": {"us": lf_ms * 1e3, "algorithmic_bytes": lf_bytes,
                           "GBps": lf_bytes / (lf_ms * 1e-3) / 1e9, "peak_GBps": PEAK_HBM_GBS,
                           "frac": lf_bytes / (lf_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                           "workload": "fp32 logits [4096, 151936], 151669 real columns, "
                                       "entropy on"},
        "keep_mask_replay": {"dense_us": dense_ms * 1e3, "compact_us": compact_ms * 1e3,
                             "dense_over_compact": dense_ms / compact_ms,
                             "dense_algorithmic_bytes": dense_bytes,
                             "dense_GBps": dense_bytes / (dense_ms * 1e-3) / 1e9,
                             "compact_algorithmic_bytes": compact_bytes,
                             "compact_GBps": compact_bytes / (compact_ms * 1e-3) / 1e9,
                             "workload": "config-5 nuclei tiled 16x (T=65536) over 4 shards "
                                         "of 37984 columns"},
    }


def measure_config4(llp, W, stream, busy, reps=2):
    """Config 4 after the timed steps: 16 packed sequences (lengths U{256..7168}, the first
    20-40% of each loss-masked), chunked at 4096 rows in order; per chunk the forward (logp),
    then the backward with that chunk's lse, dhidden per chunk, dweight overwritten by the
    first chunk and accumulated by the rest (one training step's gradient). Mean of `reps`
    timed passes after one warm-up pass, each queued behind `busy`."""
    import torch
    import synth

    log("config 4: packed variable-length forward + backward, chunks of 4096")
    case = synth.config4_case()
    Tp = case["T"]
    h = torch.from_numpy(np.ascontiguousarray(case["hidden"]).view(np.int16)).view(torch.bfloat16).cuda()
    tg = torch.from_numpy(case["targets"]).cuda()
    mk = torch.from_numpy(case["mask"]).cuda()
    dl = torch.from_numpy(case["dlogp"]).cuda()
    scored = int(case["mask"].sum())
    del case
    dH = torch.empty((Tp, H), dtype=torch.bfloat16, device="cuda")
    dW = torch.empty((VP, H), dtype=torch.float32, device="cuda")
    chunks = [(c0, min(Tp, c0 + T)) for c0 in range(0, Tp, T)]

    def one_pass():
        for i, (c0, c1) in enumerate(chunks):
            o = llp.forward(h[c0:c1], W, tg[c0:c1], temperature=TAU, loss_mask=mk[c0:c1],
                            real_vocab=VR, padded_vocab=VP, want_entropy=False)
            llp.backward(h[c0:c1], W, tg[c0:c1], o["lse"], dl[c0:c1], temperature=TAU,
                         loss_mask=mk[c0:c1], real_vocab=VR, padded_vocab=VP, dweight=dW,
                         dhidden=dH[c0:c1], overwrite=(i == 0))

    lse = torch.empty(Tp, dtype=torch.float32, device="cuda")
    ws = {}

    def one_pass_whole(slabs=False):
        # The forward in chunks of 4096 rows as above; then ONE backward over the whole pack
        # with the chunks' lse: dweight is written once (no read-modify-write per chunk).
        for c0, c1 in chunks:
            o = llp.forward(h[c0:c1], W, tg[c0:c1], temperature=TAU, loss_mask=mk[c0:c1],
                            real_vocab=VR, padded_vocab=VP, want_entropy=False)
            lse[c0:c1] = o["lse"]
        llp.backward(h, W, tg, lse, dl, temperature=TAU, loss_mask=mk, real_vocab=VR,
                     padded_vocab=VP, dweight=dW, dhidden=dH, overwrite=True,
                     workspace=ws.get("bwd_slabs" if slabs else "bwd"), g_slabs=slabs)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        busy()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    ms = timed(one_pass)
    # The whole-pack backward's workspace (G for every scored row: ~17 GB here), allocated
    # once outside the timed passes, as a training loop would keep it.
    import lm_head_linear_logp_amd._capi as capi
    req = llp._request(h, W, tg, TAU, None, mk, None, 0, VR, VP, 0, 1, False, None)
    ws["bwd"] = torch.empty(llp.workspace_bytes(req, capi.LLP_OP_BACKWARD), dtype=torch.uint8,
                            device="cuda")
    ms_whole = timed(one_pass_whole)
    ws_gb = ws["bwd"].numel() / 1e9
    del ws["bwd"]
    # The same whole-pack backward with G held one vocabulary slab at a time.
    req.flags |= capi.LLP_FLAG_G_SLABS
    ws["bwd_slabs"] = torch.empty(llp.workspace_bytes(req, capi.LLP_OP_BACKWARD),
                                  dtype=torch.uint8, device="cuda")
    ms_slabs = timed(lambda: one_pass_whole(True))
    ws_slab_gb = ws["bwd_slabs"].numel() / 1e9
    flop = 4.0 * 2.0 * H * VR * scored   # forward + the backward's three products
    del h, tg, mk, dl, dH, dW, lse, ws
    torch.cuda.empty_cache()
    return {"config4_forward_backward": {
        "packed_tokens": Tp, "scored_tokens": scored, "chunks": len(chunks), "ms": ms,
        "scored_tokens_per_s": scored / (ms * 1e-3), "tflops": flop / (ms * 1e-3) / 1e12,
        "workload": "16 packed sequences, lengths U{256..7168}, first 20-40% of each masked, "
                    "chunks of 4096 rows in order; forward then backward per chunk, dweight "
                    "overwritten by the first chunk and accumulated by the rest"},
        "config4_forward_chunked_backward_whole": {
            "ms": ms_whole, "scored_tokens_per_s": scored / (ms_whole * 1e-3),
            "tflops": flop / (ms_whole * 1e-3) / 1e12, "backward_workspace_GB": ws_gb,
            "workload": "the same pass: forward per 4096-row chunk, then one backward over "
                        "all 56583 rows (dweight written once; logp and dhidden rows bitwise "
                        "those of the chunked pass, dweight equal to rounding)"},
        "config4_forward_chunked_backward_whole_g_slabs": {
            "ms": ms_slabs, "scored_tokens_per_s": scored / (ms_slabs * 1e-3),
            "tflops": flop / (ms_slabs * 1e-3) / 1e12, "backward_workspace_GB": ws_slab_gb,
            "workload": "the whole-pack pass above with LLP_FLAG_G_SLABS: G held one slab of "
                        "32768 vocabulary columns at a time"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=2560)
    ap.add_argument("--skip-config4", action="store_true",
                    help="leave out the config-4 and slab-mode backward measurements (profiling "
                         "runs: their launches would mix other shapes into the per-kernel "
                         "averages)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB device copy before the warm-up (counter calibration)")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the forward kernel's measured HBM traffic and exit")
    args = ap.parse_args()
    if args.ingest_pmc:
        ingest_pmc(*args.ingest_pmc)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the hot path on one GPU only: the library has no multi-GPU "
              "path (vocabulary shards run one after another on one GPU and are merged in "
              "rank order by llp_merge).", file=sys.stderr)
        sys.exit(2)

    import torch
    import lm_head_linear_logp_amd as llp
    import synth

    info = llp.open(0)
    log(f"library {info['version']} route {info['route']} on {info['arch']} ({info['num_cus']} CUs)")

    def d16(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()

    log("generating inputs (W 151936x4096 bf16, h 4096x4096 bf16, top-p logits 4096x151936 fp32)")
    base = synth.config2_base()
    tg_np = np.loadtxt(os.path.join(ROOT, "tests", "golden", "config2_targets.txt"),
                       dtype=np.int64, comments="#")
    W = d16(synth.full_weight())
    h = d16(base["hidden"])
    tg = torch.from_numpy(tg_np).cuda()
    dlogp = torch.from_numpy(synth.rng(2, 70).standard_normal(T).astype(np.float32)).cuda()
    tp = synth.topp_case()
    # Algorithmic bytes of the top-p phase: per row and shard the 64 ids (512 B), the target
    # (8 B) and 13 B of partials; each distinct candidate's logit (4 B) once; the merge reads
    # 4 x 9 B of partials and writes logp and lse (8 B) per row.
    uniq = sum(np.unique(r[r >= 0]).size for r in tp["replay_ids"])
    topp_bytes = T * 4 * (64 * 8 + 8 + 13) + 4 * uniq + T * (4 * 9 + 8)
    logits = torch.from_numpy(tp["logits"]).cuda()
    rids = torch.from_numpy(tp["replay_ids"]).cuda()
    rtg = torch.from_numpy(tp["targets"]).cuda()
    if args.no_cpu_baseline:
        del tp
        tp = None
    shards = synth.shard_ranges()
    dW = torch.empty((VP, H), dtype=torch.float32, device="cuda")
    dH = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()


    def step(record):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(5)] if record else None
        if e: e[0].record(stream)
        out = llp.forward(h, W, tg, temperature=TAU, real_vocab=VR, padded_vocab=VP)
        if e: e[1].record(stream)
        mg = llp.merge([out])
        if e: e[2].record(stream)
        llp.backward(h, W, tg, mg["lse"], dlogp, temperature=TAU, real_vocab=VR, padded_vocab=VP,
                     dweight=dW, dhidden=dH, overwrite=True)
        if e: e[3].record(stream)
        parts = [llp.top_p_replay(logits[:, off:off + n], rids, rtg, temperature=TAU, offset=off,
                                  real_vocab=VR, padded_vocab=VP, rank=r, world=4)
                 for r, (off, n) in enumerate(shards)]
        llp.merge(parts, want_entropy=False)
        if e: e[4].record(stream)
        return e

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    clk_start, clk_stop = gpu_clock_sampler(0)
    clk_start()
    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    events = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        events.append(step(True))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clock = clk_stop()
    ph = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in events])  # ms
    per_step = np.array([e[0].elapsed_time(e[4]) for e in events])                    # ms
    total_ms = float(events[0][0].elapsed_time(events[-1][4]))
    ms_per_step = total_ms / args.steps
    fwd_ms, merge_ms, bwd_ms, topp_ms = (float(x) for x in ph.mean(axis=0))
    # The accumulate form of the backward (dweight += G^T h, what the later chunks of a step
    # run), after the timed steps, on the same inputs.
    mg = llp.merge([llp.forward(h, W, tg, temperature=TAU, real_vocab=VR, padded_vocab=VP)])
    ea = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    llp.backward(h, W, tg, mg["lse"], dlogp, temperature=TAU, real_vocab=VR, padded_vocab=VP,
                 dweight=dW, dhidden=dH)
    ea[0].record(stream)
    for _ in range(5):
        llp.backward(h, W, tg, mg["lse"], dlogp, temperature=TAU, real_vocab=VR,
                     padded_vocab=VP, dweight=dW, dhidden=dH)
    ea[1].record(stream)
    torch.cuda.synchronize()
    bwd_acc_ms = float(ea[0].elapsed_time(ea[1])) / 5
    # The backward of a biased head (fp32 bias ~ N(0, 0.02^2) over the padded vocabulary):
    # adds the bias gradient, each gradient tile's column sums then their sum over the token
    # blocks. 1 + 5 calls, dweight and dbias overwritten.
    bias = torch.from_numpy(
        (synth.rng(2, 71).standard_normal(VP) * 0.02).astype(np.float32)).cuda()
    dbias = torch.empty(VP, dtype=torch.float32, device="cuda")
    mgb = llp.merge([llp.forward(h, W, tg, temperature=TAU, real_vocab=VR, padded_vocab=VP,
                                 bias=bias)])

    def bwd_bias():
        llp.backward(h, W, tg, mgb["lse"], dlogp, temperature=TAU, real_vocab=VR,
                     padded_vocab=VP, bias=bias, dweight=dW, dhidden=dH, dbias=dbias,
                     overwrite=True)
    bwd_bias()
    ea[0].record(stream)
    for _ in range(5):
        bwd_bias()
    ea[1].record(stream)
    torch.cuda.synchronize()
    bwd_bias_ms = float(ea[0].elapsed_time(ea[1])) / 5
    # The backward with G held one vocabulary slab at a time (LLP_FLAG_G_SLABS): the same rows,
    # dweight overwritten, 1 + 5 calls; its workspace beside the default mode's.
    import lm_head_linear_logp_amd._capi as capi

    def bwd_ws(slabs):
        r = llp._request(h, W, tg, TAU, None, None, None, 0, VR, VP, 0, 1, False, None)
        r.flags |= capi.LLP_FLAG_OVERWRITE_GRADS | (capi.LLP_FLAG_G_SLABS if slabs else 0)
        return llp.workspace_bytes(r, capi.LLP_OP_BACKWARD)
    bwd_slab_ms = ws_slab_gb = None
    ws_default_gb = bwd_ws(False) / 1e9
    if not args.skip_config4:
        ws_slab = torch.empty(bwd_ws(True), dtype=torch.uint8, device="cuda")

        def bwd_slabs():
            llp.backward(h, W, tg, mg["lse"], dlogp, temperature=TAU, real_vocab=VR,
                         padded_vocab=VP, dweight=dW, dhidden=dH, overwrite=True, g_slabs=True,
                         workspace=ws_slab)
        bwd_slabs()
        ea[0].record(stream)
        for _ in range(5):
            bwd_slabs()
        ea[1].record(stream)
        torch.cuda.synchronize()
        bwd_slab_ms = float(ea[0].elapsed_time(ea[1])) / 5
        ws_slab_gb = ws_slab.numel() / 1e9
        del ws_slab
    del mg, mgb, bias, dbias
    log(f"phases (ms): forward {fwd_ms:.3f} merge {merge_ms:.3f} backward {bwd_ms:.3f} "
        f"top-p {topp_ms:.3f}; step {ms_per_step:.3f} (host wall {1e3 * wall / args.steps:.3f}); "
        f"backward with dweight accumulated {bwd_acc_ms:.3f}, with a bias {bwd_bias_ms:.3f}, "
        f"G in slabs {bwd_slab_ms}")

    flop_fwd = 2.0 * T * H * VR
    ach_fwd = flop_fwd / (fwd_ms * 1e-3) / 1e12
    flop_bwd = 3.0 * flop_fwd
    ach_bwd = flop_bwd / (bwd_ms * 1e-3) / 1e12
    res = {
        "metric": METRIC,
        "value": T / (ms_per_step * 1e-3),
        "unit": "scored tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Qwen3-8B-shaped LM head, one shard: T=4096 scored tokens, "
                               "H=4096, V=151669 real / 151936 padded, tau=0.7, no bias; "
                               "forward+merge+backward, plus top-p replay of 4096 rows x 4 "
                               "shards (K=64)",
                   "T": T, "H": H, "real_vocab": VR, "padded_vocab": VP, "temperature": TAU},
        "roofline": {"kernel": "k_fwd (fused GEMM + online LSE epilogue; timed with its "
                               "layout and combine launches)",
                     "bound": "mfma", "achieved": ach_fwd, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": ach_fwd / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic()},
        "ms_per_step_median": float(np.median(per_step)),
        "ms_per_step_min": float(per_step.min()),
        "gpu_clock": clock,
        "phases_ms": {"forward": fwd_ms, "merge": merge_ms, "backward": bwd_ms,
                      "top_p_4shards_plus_merge": topp_ms},
        "phases_ms_median": {k: float(v) for k, v in zip(
            ("forward", "merge", "backward", "top_p_4shards_plus_merge"), np.median(ph, axis=0))},
        "phases_ms_min": {k: float(v) for k, v in zip(
            ("forward", "merge", "backward", "top_p_4shards_plus_merge"), ph.min(axis=0))},
        "forward_tokens_per_s": T / (fwd_ms * 1e-3),
        "backward_tflops": ach_bwd,
        "backward_accumulate": {"ms": bwd_acc_ms, "tflops": flop_bwd / (bwd_acc_ms * 1e-3) / 1e12,
                                "what": "llp_backward with dweight += G^T h (later chunks of a "
                                        "step), 5 calls after the timed steps"},
        "backward_with_bias": {"ms": bwd_bias_ms,
                               "what": "llp_backward of the same rows with an fp32 bias "
                                       "[151936] and its gradient, dweight and dbias "
                                       "overwritten, 5 calls after the timed steps"},
        "backward_g_slabs": {"ms": bwd_slab_ms,
                             "tflops": flop_bwd / (bwd_slab_ms * 1e-3) / 1e12 if bwd_slab_ms else None,
                             "workspace_GB": ws_slab_gb, "default_workspace_GB": ws_default_gb,
                             "what": "llp_backward with LLP_FLAG_G_SLABS (G held one slab of "
                                     "32768 vocabulary columns at a time, 5 slabs), dweight "
                                     "overwritten, 5 calls after the timed steps"},
        "forward_backward_tflops": (flop_fwd + flop_bwd) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12,
        "top_p": {"us": topp_ms * 1e3, "algorithmic_bytes": topp_bytes,
                  "GBps": topp_bytes / (topp_ms * 1e-3) / 1e9, "peak_GBps": PEAK_HBM_GBS},
    }
    res.update(measure_next_rows(
        llp, logits, rids, rtg, shards, stream,
        busy=lambda: llp.forward(h, W, tg, temperature=TAU, real_vocab=VR, padded_vocab=VP)))
    if not args.skip_config4:
        res.update(measure_config4(
            llp, W, stream,
            busy=lambda: llp.forward(h, W, tg, temperature=TAU, real_vocab=VR, padded_vocab=VP)))
    res.update(measure_vendor_gemm(
        h, W, stream,
        lambda: llp.forward(h, W, tg, temperature=TAU, real_vocab=VR, padded_vocab=VP)))
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_rows} rows")
        del W, h, logits, dW, dH
        torch.cuda.empty_cache()
        res["cpu_baseline"] = cpu_baseline(args.cpu_rows, tp)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
