"""Benchmark of the CSA2 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch of synthetic input:
for the 128K decode workload (batch 8, 131,072 visible entries per query) the
Full layer scores every visible index key, builds the block-max candidate
pool, selects the top-512 and runs sparse attention; a Reindex layer on the
same cache then scores only the pool, selects its own top-512 and runs its
attention.  Inputs are resident in HBM before timing starts.  Steps rotate
over several independent copies of the inputs so that the 256 MB
Infinity Cache cannot serve a step from the previous step's reads.

One JSON line is printed: whole-step throughput in index keys scored per
second (plus sparse-attention queries per second), the roofline of the
dominant kernel measured with HIP events on the launch stream, and the CPU
oracle timed on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "index keys scored/s + sparse-attn queries/s at 128K ctx; % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
ATTN_BYTES_PER_QUERY = 512 * 320 + 128 * 528 + 65536 + 65536 + 2048   # 364,544
ATTN_BYTES_PER_QUERY_S16 = 512 * 288 + 128 * 528 + 65536 + 65536 + 2048   # the 288-B record
INDEX_BYTES_PER_KEY = 128 + 4 + 4                                       # key + scale + score
INDEX_BYTES_PER_KEY_FP4 = 64 + 8 + 4                                    # E2M1 key + 8 E4M3 scales + score


def _index_bytes(wl):
    return INDEX_BYTES_PER_KEY_FP4 if getattr(wl, "k_fmt", "fp8") == "fp4s16" else INDEX_BYTES_PER_KEY
SCORE_BYTES = 4


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_128k")
    ap.add_argument("--copies", type=int, default=3,
                    help="independent input copies the steps rotate over")
    ap.add_argument("--cpu-sample", type=int, default=None,
                    help="queries of the CPU-oracle sample (default: all queries, max 8)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-serving", action="store_true",
                    help="skip the serving-shaped step (paged caches, slots, inverse RoPE)")
    ap.add_argument("--no-cache-write", action="store_true",
                    help="skip the Full-layer cache-write measurement")
    ap.add_argument("--no-targets", action="store_true",
                    help="skip the two target workloads (prefill chunk scoring, decoder-group attention)")
    ap.add_argument("--samples", type=int, default=50,
                    help="timed samples per stage and protocol (median, p10, p90 reported)")
    ap.add_argument("--stage-reps", type=int, default=8,
                    help="rounds over the input copies in one rotated stage sample")
    ap.add_argument("--summarize-profiles", nargs=4, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "OUT_DIR"),
                    help="no GPU: turn rocprofv3 CSV output of this benchmark (a --kernel-trace "
                         "--stats run, a --pmc FETCH_SIZE run and a --pmc WRITE_SIZE run) into the "
                         "text summaries and per-stage traffic records kept under profiles/")
    ap.add_argument("--summarize-mfma", nargs=3, metavar=("MFMA_DIR", "TRACE_DIR", "OUT_DIR"),
                    help="no GPU: summarize a rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE "
                         "SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU run of this benchmark")
    ap.add_argument("--stage-only", default=None, metavar="STAGE",
                    help="run one full step, then only the calls of STAGE (e.g. sparse_attn) "
                         "--repeat times, and exit: a short target for counter runs")
    ap.add_argument("--repeat", type=int, default=10)
    ap.add_argument("--summarize-sq", nargs="+", metavar="PATH",
                    help="no GPU: OUT_FILE then rocprofv3 --pmc output dirs of SQ counters")
    ap.add_argument("--profile-command", default="",
                    help="the benchmark command the profiles were taken on (recorded in the summaries)")
    return ap.parse_args()


STAGE_TIMED_REPLAYS = 5


def _source_hash():
    h = hashlib.sha1()
    csrc = os.path.join(ROOT, "top_sparse_long_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


PREFILL_MIN_Q = 256                      # batches this large share every staged key / row
INDEX_FLOPS_PER_PAIR = 2 * 32 * 128      # 32 heads x 128 dims, multiply + add
ATTN_KEYS = 128 + 512                    # SWA window + top-k per query
ATTN_FLOPS_PER_QUERY = 2 * 64 * ATTN_KEYS * 512 * 2   # S = q K^T and O = P V: 83.9 MFLOP


def _stage_work(run, stage):
    """(algorithmic bytes, FLOPs, units, bound) of one launch of a stage.

    bound is the roofline that limits the stage at full efficiency: "mfma"
    for index scoring and attention when the batch shares every staged key
    (query-tiled prefill: 8,192 FLOP per (query, key) pair, 83.9 MFLOP per
    attention query), else "hbm" (the bytes the method must move)."""
    wl = run.wl
    nvis = wl.n_vis().clamp(max=run.n_cols)
    shared = wl.Q >= PREFILL_MIN_Q
    if stage == "index_scores_dense":
        # plus the fused block maxima (4 B per block) when the step emits them;
        # without the 4-B score when the Full layer re-scores its best blocks
        fused = any(run.fuses_block_max(li) for li, l in enumerate(wl.layers) if l.mode == "full")
        extra = 4.0 / wl.block_size if fused else 0.0
        if any(run.rescored(li, overlap_route=True) for li in range(len(wl.layers))):
            extra -= SCORE_BYTES
        pairs = int(nvis.sum().item())
        return (float(pairs) * (_index_bytes(wl) + extra), float(pairs) * INDEX_FLOPS_PER_PAIR, pairs,
                "mfma" if shared else "hbm")
    if stage == "index_scores_top":
        pairs = wl.Q * run.top_cols
        return float(pairs) * _index_bytes(wl), float(pairs) * INDEX_FLOPS_PER_PAIR, pairs, "hbm"
    if stage == "topk_top":
        return float(wl.Q * run.top_cols) * SCORE_BYTES, 0.0, wl.Q * run.top_cols, "hbm"
    if stage == "index_scores_pool":
        pairs = wl.Q * run.pool_cols
        return float(pairs) * _index_bytes(wl), float(pairs) * INDEX_FLOPS_PER_PAIR, pairs, "hbm"
    if stage == "block_candidates" and run.fuse_block_max:
        nblk = (nvis + wl.block_size - 1) // wl.block_size
        return float(nblk.sum().item()) * SCORE_BYTES, 0.0, int(nvis.sum().item()), "hbm"
    nblk = (nvis + wl.block_size - 1) // wl.block_size
    if stage == "top_blocks_and_blocks":
        # one read of the block maxima (both rankings read the same)
        return float(nblk.sum().item()) * SCORE_BYTES, 0.0, int(nvis.sum().item()), "hbm"
    # the top-k through block maxima reads the maxima, then the scores of the
    # k best blocks (the library takes this route when k * block_size <= 32,768)
    via = (run.via_blocks and run.fuse_block_max and wl.topk * wl.block_size <= 32768)
    topk_read = nblk + nvis.clamp(max=wl.topk * wl.block_size) if via else nvis
    if stage == "topk_and_blocks":
        # the pool reads the block maxima when the scoring pass wrote them,
        # else the scores again
        pool = nblk if run.fuse_block_max else nvis
        return (float((topk_read + pool).sum().item()) * SCORE_BYTES, 0.0, int(nvis.sum().item()),
                "hbm")
    if stage == "topk_blocks":
        return float(topk_read.sum().item()) * SCORE_BYTES, 0.0, int(nvis.sum().item()), "hbm"
    if stage in ("topk_dense", "block_candidates"):
        return float(nvis.sum().item()) * SCORE_BYTES, 0.0, int(nvis.sum().item()), "hbm"
    if stage == "topk_pool":
        return float(wl.Q * run.pool_cols) * SCORE_BYTES, 0.0, wl.Q * run.pool_cols, "hbm"
    if stage == "sparse_attn":
        per_q = (ATTN_BYTES_PER_QUERY_S16 if getattr(wl, "main_fmt", "fp4") == "fp4s16"
                 else ATTN_BYTES_PER_QUERY)
        return (float(wl.Q) * per_q, float(wl.Q) * ATTN_FLOPS_PER_QUERY, wl.Q,
                "mfma" if shared else "hbm")
    raise KeyError(stage)


def _traffic(stage, workload, launches_bytes):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{stage}_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except Exception:
        return None
    if rec.get("source_sha1") != _source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


# kernels of each stage, as they appear in the profiler's kernel names
STAGE_KERNELS = {
    "index_scores_dense": ("index_scores_fp8_kernel<false", "index_scores_prefill_kernel",
                           "index_scores_f32_kernel"),
    "index_scores_pool": ("index_scores_fp8_kernel<true",),
    "block_candidates": ("select_kernel<2,",),
    "topk_dense": ("select_kernel<0,", "select_kernel<3,"),
    "topk_pool": ("select_kernel<1,",),
    # the re-scoring route of a Full layer (its kernels are the pool stages')
    "top_blocks_and_blocks": ("select_pair_kernel", "select_kernel<5,", "select_kernel<2,", "select_kernel<3,"),
    "index_scores_top": ("index_scores_fp8_kernel<true",),
    "topk_top": ("select_kernel<1,",),
    "topk_blocks": ("select_kernel<5,", "select_kernel<4,"),
    "topk_and_blocks": ("select_pair_kernel", "select_kernel<0,", "select_kernel<2,", "select_kernel<3,",
                        "select_kernel<4,", "select_kernel<5,"),
    "sparse_attn": ("sparse_attn_pipe_kernel", "sparse_attn_wide_kernel", "sparse_attn_combine_kernel",
                    "sparse_attn_f32_kernel"),
    # the 65,536-token m = 2 chunk (the decode-batch calls use the prefetching
    # variant, cache_write_kernel<m, true>, and are not part of this record)
    "cache_write": ("cache_write_kernel<2, false>", "cache_pend_kernel"),
}
# counter calibration: the benchmark's streaming read and write of 2 GiB each
# (csa2_diag_stream_read / _write, run by read_ceiling) move known bytes
CALIB_READ_KERNEL = "stream_read_kernel"
CALIB_WRITE_KERNEL = "stream_write_kernel"
CALIB_KIB = 2 * 1024 * 1024


def _find_csv(d, suffix):
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def _counter_per_kernel(path):
    import csv
    per = {}
    for row in csv.DictReader(open(path)):
        per.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return per


def summarize_profiles(trace_dir, fetch_dir, write_dir, out_dir, workload, command):
    """Write kernels_<workload>.txt, counters_<workload>.txt and one
    traffic_<stage>_<workload>.json per stage from rocprofv3 CSV output."""
    import csv
    os.makedirs(out_dir, exist_ok=True)
    stats = list(csv.DictReader(open(_find_csv(trace_dir, "kernel_stats.csv"))))
    lines = [f"# rocprofv3 kernel-trace summary, workload {workload}",
             f"# command: rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -- {command}",
             f"# columns: calls, average us, min us, max us, kernel", ""]
    avg_us = {}
    for row in stats:
        name = row["Name"]
        if "csa2::" not in name:
            continue
        avg = float(row["AverageNs"]) / 1e3
        avg_us[name] = avg
        lines.append(f"{int(row['Calls']):6d} {avg:10.2f} {float(row['MinNs']) / 1e3:10.2f} "
                     f"{float(row['MaxNs']) / 1e3:10.2f}  {name}")
    with open(os.path.join(out_dir, f"kernels_{workload}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")

    fetch = _counter_per_kernel(_find_csv(fetch_dir, "counter_collection.csv"))
    write = _counter_per_kernel(_find_csv(write_dir, "counter_collection.csv"))
    def _calib(per, pat):
        vals = sorted(v for n, vs in per.items() if pat in n for v in vs)
        return vals[len(vals) // 2] if vals else None
    fraw = _calib(fetch, CALIB_READ_KERNEL)
    wraw = _calib(write, CALIB_WRITE_KERNEL)
    fscale = CALIB_KIB / fraw if fraw else 1.0
    wscale = CALIB_KIB / wraw if wraw else 1.0
    lines = [f"# rocprofv3 counter summary (KiB per dispatch, averaged), workload {workload}",
             f"# commands: rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -- {command}",
             f"#           rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -- {command}",
             f"# calibration: the {CALIB_KIB} KiB streaming read reads FETCH_SIZE "
             f"{fraw or 0:.1f} KiB -> scale {fscale:.4f}; the {CALIB_KIB} KiB streaming write "
             f"writes WRITE_SIZE {wraw or 0:.1f} KiB -> scale {wscale:.4f} (median dispatch)",
             "# columns: dispatches, FETCH_SIZE raw, WRITE_SIZE raw, scaled HBM MB (read + write), kernel", ""]
    per_kernel_bytes = {}
    for name in sorted(set(fetch) | set(write)):
        if "csa2::" not in name:
            continue
        fr = sum(fetch.get(name, [0])) / max(1, len(fetch.get(name, [])))
        wr = sum(write.get(name, [0])) / max(1, len(write.get(name, [])))
        b = (fr * fscale + wr * wscale) * 1024
        per_kernel_bytes[name] = b
        lines.append(f"{len(fetch.get(name, [])):6d} {fr:12.1f} {wr:12.1f} {b / 1e6:12.3f}  {name}")
    with open(os.path.join(out_dir, f"counters_{workload}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")

    src = _source_hash()
    # A Full layer on the re-score route runs the dense scorer without score
    # stores (its last template argument false); its stages then share
    # kernels with the pool stages, and the paired selection launch belongs
    # to top_blocks_and_blocks instead of topk_and_blocks.
    rescore = any("index_scores_fp8_kernel<false" in n and ", false>(csa2::IndexScoreArgs)" in n
                  for n in per_kernel_bytes)
    skip = ({"topk_and_blocks", "index_scores_pool", "topk_pool", "index_scores_top", "topk_top"} if rescore
            else {"top_blocks_and_blocks", "index_scores_top", "topk_top"})
    for stage, pats in STAGE_KERNELS.items():
        # a stage is present when one of its own kernels is (the selection
        # list-stage kernels are shared between stages and do not count)
        own = [p for p in pats if p != "select_kernel<3,"]
        if stage in ("topk_and_blocks", "top_blocks_and_blocks"):
            own = ["select_pair_kernel"]
        if not any(p in n for p in own for n in per_kernel_bytes):
            continue
        # stages whose dispatches cannot be told apart by kernel name
        if stage in skip:
            continue
        # with the shared-launch call the separate-call stages do not occur
        if stage in ("topk_dense", "block_candidates", "topk_blocks") and any(
                "select_pair_kernel" in n for n in per_kernel_bytes):
            continue
        names = [n for n in per_kernel_bytes if any(p in n for p in pats)]
        rec = {"stage": stage, "workload": workload, "kernels": names,
               "hbm_bytes_per_launch": sum(per_kernel_bytes[n] for n in names),
               "rocprof_avg_us": {n: avg_us.get(n) for n in names},
               "fetch_scale": fscale, "write_scale": wscale, "source_sha1": src,
               "command": command}
        with open(os.path.join(out_dir, f"traffic_{stage}_{workload}.json"), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")


F16_PEAK_TFLOPS = 2500.0
N_SIMD = 256 * 4


def summarize_mfma(mfma_dir, trace_dir, out_dir, workload, command):
    """Write mfma_<workload>.txt: per csa2 kernel, MFMA busy share of the
    SIMD cycles while it ran and the f16 MFMA FLOP rate it reached."""
    import csv
    os.makedirs(out_dir, exist_ok=True)
    per = {}
    for row in csv.DictReader(open(_find_csv(mfma_dir, "counter_collection.csv"))):
        if "csa2::" not in row["Kernel_Name"]:
            continue
        d = per.setdefault(row["Kernel_Name"], {})
        d.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
    avg_us = {}
    for row in csv.DictReader(open(_find_csv(trace_dir, "kernel_stats.csv"))):
        avg_us[row["Name"]] = float(row["AverageNs"]) / 1e3
    lines = [f"# rocprofv3 MFMA counters, workload {workload}",
             f"# command: rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_F16 "
             f"SQ_INSTS_VALU --output-format csv -d <dir> -- {command}",
             "# busy% = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs * 1024 SIMDs);",
             "# TFLOP/s = 512 * SQ_INSTS_VALU_MFMA_MOPS_F16 / average duration from the kernel trace;",
             f"# frac = TFLOP/s / {F16_PEAK_TFLOPS:.0f} (dense f16 MFMA peak)",
             "# columns: dispatches, busy%, f16 TFLOP/s, frac of f16 peak, VALU insts per dispatch, kernel", ""]
    for name, d in sorted(per.items()):
        mean = {k: sum(v) / len(v) for k, v in d.items()}
        gui = mean.get("GRBM_GUI_ACTIVE", 0.0)
        busy = mean.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        util = 100.0 * busy / (gui / 8.0 * N_SIMD) if gui else 0.0
        flops = 512.0 * mean.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0)
        us = avg_us.get(name)
        tf = flops / (us * 1e-6) / 1e12 if us else 0.0
        lines.append(f"{len(d.get('GRBM_GUI_ACTIVE', [])):6d} {util:7.1f} {tf:9.1f} {tf / F16_PEAK_TFLOPS:7.3f} "
                     f"{mean.get('SQ_INSTS_VALU', 0.0):14.0f}  {name}")
    with open(os.path.join(out_dir, f"mfma_{workload}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_sq(dirs, out_path, workload, stage, commands):
    """Write a per-kernel table of SQ counters (averaged per dispatch) from
    one or more rocprofv3 --pmc runs, with derived shares of the SIMD time."""
    import csv
    per = {}
    for d in dirs:
        for row in csv.DictReader(open(_find_csv(d, "counter_collection.csv"))):
            if "csa2::" not in row["Kernel_Name"]:
                continue
            per.setdefault(row["Kernel_Name"], {}).setdefault(row["Counter_Name"], []).append(
                float(row["Counter_Value"]))
    lines = [f"# rocprofv3 SQ counters, workload {workload}, stage {stage} (values per dispatch)"]
    lines += [f"# command: {c}" for c in commands]
    lines += ["# derived: SIMD-cycles = GRBM_GUI_ACTIVE / 8 XCDs * 1024 SIMDs;",
              "#   mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / SIMD-cycles;",
              "#   valu_issue = 4 * SQ_ACTIVE_INST_VALU / SIMD-cycles (quad-cycles);",
              "#   wave_wait = SQ_WAIT_ANY / SQ_WAVE_CYCLES", ""]
    for name, d in sorted(per.items()):
        mean = {k: sum(v) / len(v) for k, v in d.items()}
        lines.append(name)
        for k in sorted(mean):
            lines.append(f"    {k:28s} {mean[k]:.4g}")
        gui = mean.get("GRBM_GUI_ACTIVE")
        if gui:
            simd = gui / 8.0 * N_SIMD
            if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
                lines.append(f"    mfma_busy                    {mean['SQ_VALU_MFMA_BUSY_CYCLES'] / simd:.3f}")
            if "SQ_ACTIVE_INST_VALU" in mean:
                lines.append(f"    valu_issue                   {4 * mean['SQ_ACTIVE_INST_VALU'] / simd:.3f}")
        if mean.get("SQ_WAVE_CYCLES") and "SQ_WAIT_ANY" in mean:
            lines.append(f"    wave_wait                    {mean['SQ_WAIT_ANY'] / mean['SQ_WAVE_CYCLES']:.3f}")
        lines.append("")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


def _host_inputs(wl, sample):
    """Host copies of what the oracle needs for the sampled queries (not timed)."""
    import numpy as np
    import torch
    q_seq = wl.q_seq.cpu().numpy()
    seqs = sorted(set(int(q_seq[t]) for t in sample))
    inputs = {}
    for b in seqs:
        base, n = int(wl.seq_base[b]), int(wl.n_entries[b])
        rows = torch.arange(base, base + n, device=wl.k_idx.device)
        ks = wl.k_scale[rows].cpu().numpy() if wl.k_scale is not None else None
        inputs[b] = (wl.k_idx[rows].cpu().numpy(), ks, wl.main_kv[rows].cpu().numpy())
    layers = []
    for lay in wl.layers:
        d = {"mode": lay.mode, "q": lay.q[sample].cpu().numpy(), "swa": lay.swa.cpu().numpy(),
             "sink": lay.sink.cpu().numpy().astype(np.float64)}
        if lay.q_idx is not None:
            d["q_idx"] = lay.q_idx[sample].cpu().numpy()
            d["q_scale"] = lay.q_scale[sample].cpu().numpy() if lay.q_scale is not None else None
            d["w"] = lay.w[sample].cpu().numpy()
        layers.append(d)
    return inputs, layers


def _oracle_pass(wl, sample, inputs, layers):
    """The oracle over every layer of the step for the sampled queries; returns
    (index keys scored, seconds).  Decoding each query's rows is timed too."""
    import numpy as np
    import oracle
    q_seq = wl.q_seq.cpu().numpy()
    q_pos = wl.q_pos.cpu().numpy()
    swa_base = wl.swa_base.cpu().numpy()
    swa_pos0 = wl.swa_pos0.cpu().numpy()
    quant = wl.quantized
    keys_scored = 0
    t0 = time.perf_counter()
    for j, t in enumerate(sample):
        b = int(q_seq[t])
        kc, ks, mk = inputs[b]
        if not quant:
            k_rows, main_rows = kc.astype(np.float64), mk.astype(np.float64)
        else:
            k_rows = (oracle.decode_fp4s16_rows(kc, ks) if getattr(wl, "k_fmt", "fp8") == "fp4s16"
                      else oracle.decode_e4m3_rows(kc, ks))
            main_rows = (oracle.decode_fp4s16_records(mk) if getattr(wl, "main_fmt", "fp4") == "fp4s16"
                         else oracle.decode_fp4_records(mk))
        pos1, seq0, base0 = np.array([q_pos[t]]), np.array([0]), np.array([0])
        n = int(oracle.visible_count(pos1, wl.ratio)[0])
        cand = idx = None
        for li, lay in enumerate(layers):
            if lay["mode"] in ("full", "reindex"):
                if quant:
                    qv = oracle.decode_e4m3_rows(lay["q_idx"][j:j + 1], lay["q_scale"][j:j + 1])
                    wv = oracle.decode_bf16(lay["w"][j:j + 1])
                else:
                    qv = lay["q_idx"][j:j + 1].astype(np.float64)
                    wv = lay["w"][j:j + 1].astype(np.float64)
            if lay["mode"] == "full":
                sc = oracle.index_scores_dense(qv, wv, k_rows, base0, seq0, pos1, wl.ratio, n)
                keys_scored += n
                if any(l["mode"] == "reindex" for l in layers[li + 1:]):
                    cand = oracle.block_candidates(sc, pos1, wl.ratio, wl.block_size, wl.n_blocks)
                idx = oracle.topk_rows_dense(sc, pos1, wl.ratio, wl.topk)
            elif lay["mode"] == "reindex":
                sc = oracle.index_scores_pool(qv, wv, k_rows, base0, seq0, pos1, wl.ratio, cand,
                                              wl.block_size)
                keys_scored += sc.shape[1]
                idx = oracle.topk_rows_pool(sc, cand, wl.block_size, wl.topk)
            swa = oracle.decode_swa_records(lay["swa"]) if quant else lay["swa"].astype(np.float64)
            qa = oracle.decode_bf16(lay["q"][j:j + 1]) if quant else lay["q"][j:j + 1].astype(np.float64)
            oracle.sparse_attn(qa, main_rows, base0, idx, swa, swa_base[b:b + 1], swa_pos0[b:b + 1],
                               None, wl.window, seq0, pos1, lay["sink"], wl.softmax_scale, wl.ratio)
    return keys_scored, time.perf_counter() - t0


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, n_sample):
    """Time the oracle on the first n_sample queries of the workload's whole
    path (both layers), on the host cores with the BLAS threads it gets."""
    from threadpoolctl import threadpool_info
    sample = list(range(min(n_sample, wl.Q)))
    inputs, layers = _host_inputs(wl, sample)
    keys, dt = _oracle_pass(wl, sample, inputs, layers)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": keys / dt, "unit": "index keys scored/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": _cpu_model(),
            "host_cpus": {"os_cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))},
            "sample": f"{len(sample)} of {wl.Q} queries through every layer of the step "
                      f"(float64 NumPy oracle, {dt:.1f} s wall)"}


def cpu_single_core(synth):
    """The oracle on one thread: all 16 queries of the tiny fp32 Full layer
    (2,048 entries) and two queries of the 128K decode step (both layers)."""
    from threadpoolctl import threadpool_limits
    out = {}
    with threadpool_limits(limits=1):
        for name, n in (("tiny_full_fp32", 16), ("decode_128k", 2)):
            wl = synth.make_workload(name, device="cuda")
            sample = list(range(min(n, wl.Q)))
            inputs, layers = _host_inputs(wl, sample)
            keys, dt = _oracle_pass(wl, sample, inputs, layers)
            out[name] = {"value": keys / dt, "unit": "index keys scored/s", "cores": 1,
                         "queries_per_s": len(sample) / dt,
                         "sample": f"{len(sample)} of {wl.Q} queries, {dt:.2f} s wall"}
            del wl, inputs, layers
    return {"single_core": out}


# Full-layer cache write of the encoder prefill chunk: per entry, two tokens'
# bf16 c and z rows in, the RoPE table row, the 320-byte main record and the
# 132 bytes of FP8 index key out, and the two tokens' ids and positions
CW_TOKENS = 65536
CW_BYTES_PER_ENTRY = 2 * (1024 + 1024) + 256 + 320 + 128 + 4 + 2 * 8
CW_BYTES_PER_CALL = 128 * 512 * 2 + 512 * 4 + 128 * 4      # W_IK and the two norm weights


def cache_write_stage(torch, synth, tsl, wl, reps, n_copies, workload):
    """Time csa2_cache_write on (a) the 65,536-token m = 2 encoder prefill
    chunk (32,768 entries; roofline) and (b) the decode batch of the bench
    workload (one token per query at its ratio and cache formats)."""
    dev = "cuda"

    def outputs(n, main_fmt, k_fmt):
        if main_fmt == "fp4s16":
            main = torch.empty((n, 288), dtype=torch.uint8, device=dev)
            mrows = tsl.rows_fp4s16_records(main)
        else:
            main = torch.empty((n, 320), dtype=torch.uint8, device=dev)
            mrows = tsl.rows_fp4_records(main)
        if k_fmt == "fp4s16":
            kc = torch.empty((n, 64), dtype=torch.uint8, device=dev)
            ks = torch.empty((n, 8), dtype=torch.uint8, device=dev)
            krows = tsl.rows_fp4s16(kc, ks)
        else:
            kc = torch.empty((n, 128), dtype=torch.uint8, device=dev)
            ks = torch.empty((n,), dtype=torch.float32, device=dev)
            krows = tsl.rows_fp8(kc, ks)
        return (main, kc, ks), mrows, krows

    def timed(fns):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for f in fns:
                f()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for f in fns:
                f()
        g.replay()
        torch.cuda.synchronize()
        times = []
        for _ in range(STAGE_TIMED_REPLAYS):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(torch.cuda.current_stream())
            g.replay()
            e1.record(torch.cuda.current_stream())
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return sorted(times)[len(times) // 2] * 1e3 / len(fns)

    def call(inp, bufs, base, n):
        _, mrows, krows = bufs
        return lambda: tsl.csa2_cache_write(inp.c, inp.z if inp.ratio == 2 else None, inp.tok_seq,
                                            inp.tok_pos, inp.ratio, inp.pend, inp.n_seq,
                                            inp.kv_norm_w, inp.w_ik, inp.k_norm_w, inp.eps,
                                            inp.rope_cs, mrows, base, n, krows, base, n)

    # (a) the prefill chunk, rotated over input copies
    n_ent = CW_TOKENS // 2
    inps = [synth.cache_write_inputs(7000 + c, [(0, 0, CW_TOKENS)], 2, dev) for c in range(n_copies)]
    bufs = outputs(n_ent, "fp4", "fp8")
    zero = torch.zeros(1, dtype=torch.int64, device=dev)
    fns = [call(i, bufs, zero, n_ent) for _ in range(reps) for i in inps]
    us = timed(fns)
    nbytes = n_ent * CW_BYTES_PER_ENTRY + CW_BYTES_PER_CALL
    achieved = nbytes / (us * 1e-6) / 1e9
    prefill = {"workload": "encoder prefill chunk: 65,536 tokens at m = 2 -> 32,768 entries, "
                           "320-B main records + FP8 index keys",
               "avg_us": us, "entries_per_s": n_ent / (us * 1e-6),
               "roofline": {"bound": "hbm", "kernel": "cache_write", "achieved": achieved,
                            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                            "traffic": _traffic("cache_write", workload, nbytes),
                            "algorithmic_bytes": nbytes}}
    del inps, bufs, fns
    # (b) the decode batch: each query's sequence gets its newest token
    pos = wl.q_pos.cpu().tolist()
    seqs = wl.q_seq.cpu().tolist()
    runs = [(s, p, 1) for s, p in zip(seqs, pos)]
    inp = synth.cache_write_inputs(7100, runs, wl.ratio, dev, n_seq=max(seqs) + 1)
    if len(set(seqs)) == len(seqs):
        # one token per sequence: sequence s's entry lands in row s
        base_l = [0] * inp.n_seq
        for s_, p_ in zip(seqs, pos):
            base_l[s_] = s_ - p_ // wl.ratio
        n_rows = inp.n_seq
    else:
        span = max(p // wl.ratio for p in pos) + 1
        base_l = [s_ * span for s_ in range(inp.n_seq)]
        n_rows = inp.n_seq * span
    base = torch.tensor(base_l, dtype=torch.int64, device=dev)
    bufs = outputs(n_rows, getattr(wl, "main_fmt", "fp4"), getattr(wl, "k_fmt", "fp8"))
    us_dec = timed([call(inp, bufs, base, n_rows) for _ in range(reps * n_copies)])
    decode = {"workload": f"one new token for each of the {len(runs)} queries at m = {wl.ratio}",
              "avg_us": us_dec}
    return {"prefill_chunk": prefill, "decode_batch": decode}


def _pct(xs, q):
    xs = sorted(xs)
    i = min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))
    return xs[i]


def _stats(us):
    return {"median_us": _pct(us, 0.5), "p10_us": _pct(us, 0.1), "p90_us": _pct(us, 0.9),
            "samples": len(us)}


class Timer:
    """HIP-graph capture and event timing on torch's current stream (the
    stream the library's kernels are launched on)."""

    def __init__(self, torch, cold_bytes):
        self.torch = torch
        self.stream = torch.cuda.current_stream()
        # read before every cold sample, outside the timed region, so the
        # sample's reads find neither the L2 nor the 256 MB Infinity Cache
        # warm (a read leaves no dirty lines to write back during the sample)
        self.flush_buf = torch.ones((cold_bytes // 4,), dtype=torch.float32, device="cuda")
        # a GPU-side spin before each timed region lets the host enqueue the
        # region's graph before the GPU reaches its start event
        self.spin_cycles = 1 << 20
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        torch.cuda._sleep(self.spin_cycles)
        e1.record(self.stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3
        self.spin_cycles = max(1, int(self.spin_cycles * 60.0 / max(us, 1e-3)))   # about 60 us

    def flush(self):
        self.flush_sink = self.flush_buf.amax()

    def spin(self):
        self.torch.cuda._sleep(self.spin_cycles)

    def capture(self, fns):
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for f in fns:
                f()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for f in fns:
                f()
        return g

    def sample(self, n, body):
        """n timed samples; body(i) enqueues sample i's untimed prefix and
        returns what to time: a graph (replayed) or a list of calls (launched
        directly, which adds no graph dispatch to a region of one or a few
        launches).  Everything is enqueued back to back and read after one
        synchronisation.  Returns milliseconds per sample."""
        torch = self.torch
        evs = []
        for i in range(n):
            work = body(i)
            self.spin()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            if isinstance(work, list):
                for f in work:
                    f()
            else:
                work.replay()
            e1.record(self.stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]


def stage_stats(timer, rs, n_samples, reps, protocols=("rotated", "cold", "warm")):
    """Per stage of one step, launch durations in microseconds:

    rotated  graph replays of every input copy's calls of the stage, `reps`
             times over (so no launch reads what the launch before it read);
             each sample is one replay, divided by its launches;
    cold     one copy's calls after a 1 GiB read that evicts the L2 and the
             Infinity Cache;
    warm     one copy's calls right after the same calls ran.
    The medians of `rotated` are the stage times the roofline uses."""
    names = []
    for name, _ in rs[0].steps(overlap_route=True):
        if name != "reset" and name not in names:
            names.append(name)
    out = {}
    for name in names:
        per_copy = [[f for n, f in r.steps(overlap_route=True) if n == name] for r in rs]
        calls = len(per_copy[0])
        rot = timer.capture([f for _ in range(reps) for r in rs for n, f in r.steps(overlap_route=True)
                             if n == name])
        rot.replay()
        for fns in per_copy:
            for f in fns:
                f()
        timer.torch.cuda.synchronize()
        nbytes, flops, units, bound = _stage_work(rs[0], name)
        rec = {"calls_per_step": calls, "algorithmic_bytes": nbytes, "flops": flops,
               "units": units, "bound": bound}
        if "rotated" in protocols:
            ms = timer.sample(n_samples, lambda i: rot)
            rec["rotated"] = _stats([m * 1e3 / (reps * len(rs) * calls) for m in ms])
        if "cold" in protocols:
            def cold(i):
                timer.flush()
                return per_copy[i % len(rs)]
            rec["cold"] = _stats([m * 1e3 / calls for m in timer.sample(n_samples, cold)])
        if "warm" in protocols:
            def warm(i):
                fns = per_copy[i % len(rs)]
                for f in fns:
                    f()
                return fns
            rec["warm"] = _stats([m * 1e3 / calls for m in timer.sample(n_samples, warm)])
        t = rec["rotated"]["median_us"] * 1e-6
        rec["avg_us"] = rec["rotated"]["median_us"]
        rec["hbm_frac"] = nbytes / t / (HBM_PEAK_GBS * 1e9)
        if READ_CEILING:
            rec["hbm_frac_of_read_ceiling"] = nbytes / t / (READ_CEILING["GB/s"] * 1e9)
        if flops:
            rec["mfma_frac_f16"] = flops / t / (F16_PEAK_TFLOPS * 1e12)
            if name.startswith("index_scores"):
                rec["mfma_frac_fp8"] = flops / t / (FP8_PEAK_TFLOPS * 1e12)
        for proto in ("cold", "warm"):
            if proto in rec:
                rec[proto]["hbm_frac"] = nbytes / (rec[proto]["median_us"] * 1e-6) / (HBM_PEAK_GBS * 1e9)
        out[name] = rec
        del per_copy, rot
    return out


def measure_workload(torch, synth, LayerRunner, timer, name, args, copies, steps, warmup):
    """Whole-step time and per-stage times of one workload."""
    runs = [LayerRunner(synth.make_workload(name, device="cuda", seed_offset=1000 * c))
            for c in range(max(1, copies))]
    torch.cuda.synchronize()
    # the pass as it runs: each layer's attention on a second stream,
    # overlapping the next layers' scoring and selection
    step_graphs = [timer.capture([f for _, f in r.steps(concurrent=True)]) for r in runs]
    for i in range(warmup):
        step_graphs[i % len(step_graphs)].replay()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(timer.stream)
    for i in range(steps):
        step_graphs[i % len(step_graphs)].replay()
    ev1.record(timer.stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    del step_graphs
    # the same pass with every call on one stream, for reference
    serial_graphs = [timer.capture([f for _, f in r.steps(overlap_route=True)]) for r in runs]
    for i in range(warmup):
        serial_graphs[i % len(serial_graphs)].replay()
    torch.cuda.synchronize()
    ev2 = torch.cuda.Event(enable_timing=True)
    ev3 = torch.cuda.Event(enable_timing=True)
    ev2.record(timer.stream)
    for i in range(steps):
        serial_graphs[i % len(serial_graphs)].replay()
    ev3.record(timer.stream)
    torch.cuda.synchronize()
    del serial_graphs
    stages = stage_stats(timer, runs, args.samples, args.stage_reps)
    run0 = runs[0]
    wl = run0.wl
    keys = 0
    n_attn = 0
    for lay in wl.layers:
        if lay.mode == "full":
            keys += int(wl.n_vis().clamp(max=run0.n_cols).sum().item())
        elif lay.mode == "reindex":
            keys += wl.Q * run0.pool_cols
        n_attn += wl.Q
    return {"runs": runs, "ms_per_step": (t1 - t0) * 1e3 / steps,
            "gpu_ms_per_step": ev0.elapsed_time(ev1) / steps,
            "serial_gpu_ms_per_step": ev2.elapsed_time(ev3) / steps, "stages": stages,
            "index_keys_per_step": keys, "attn_queries_per_step": n_attn}


READ_CEILING = {}   # the measured streaming-read rate, filled by read_ceiling()


def read_ceiling(torch, tsl, gib=2, reps=10):
    """The chip's practical HBM read rate: csa2_diag_stream_read over a
    2 GiB buffer (16-byte non-temporal loads, nothing computed), median of
    reps timed launches on the launch stream."""
    src = torch.ones((gib << 30) // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(4096, dtype=torch.float32, device="cuda")
    for _ in range(2):
        tsl.csa2_diag_stream_read(src, sink)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        tsl.csa2_diag_stream_read(src, sink)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    ts.sort()
    t = ts[len(ts) // 2]
    gbs = src.numel() * 4 / t / 1e9
    # the write counterpart over the same buffer
    for _ in range(2):
        tsl.csa2_diag_stream_write(src, 0.5)
    torch.cuda.synchronize()
    tw = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        tsl.csa2_diag_stream_write(src, 0.5)
        e1.record()
        torch.cuda.synchronize()
        tw.append(e0.elapsed_time(e1) * 1e-3)
    tw.sort()
    wgbs = src.numel() * 4 / tw[len(tw) // 2] / 1e9
    del src, sink
    torch.cuda.empty_cache()
    READ_CEILING["GB/s"] = gbs
    return {"kernel": "csa2_diag_stream_read", "bytes": gib << 30, "median_us": t * 1e6,
            "achieved": gbs, "unit": "GB/s", "frac_of_peak": gbs / HBM_PEAK_GBS,
            "write_achieved": wgbs, "write_kernel": "csa2_diag_stream_write",
            "what": "16-byte non-temporal loads (stores) in a grid-stride loop over 2 GiB, nothing "
                    "computed: the practical read ceiling for the HBM-bound stages"}


def _roofline(stage, rec, workload):
    """The roofline record of one stage from its rotated median."""
    t = rec["avg_us"] * 1e-6
    if rec["bound"] == "mfma":
        achieved = rec["flops"] / t / 1e12
        peak = FP8_PEAK_TFLOPS if stage.startswith("index_scores") else F16_PEAK_TFLOPS
        r = {"bound": "mfma", "kernel": stage, "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
             "frac": achieved / peak}
        if stage.startswith("index_scores"):
            r["frac_of_f16_peak"] = achieved / F16_PEAK_TFLOPS
        r["traffic"] = _traffic(stage, workload, rec["algorithmic_bytes"])
        return r
    achieved = rec["algorithmic_bytes"] / t / 1e9
    r = {"bound": "hbm", "kernel": stage, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": achieved / HBM_PEAK_GBS,
         "traffic": _traffic(stage, workload, rec["algorithmic_bytes"])}
    if READ_CEILING:
        r["frac_of_read_ceiling"] = achieved / READ_CEILING["GB/s"]
    return r


def mfma_valu_overlap(torch, tsl, iters=2048, reps=5):
    """Whether matrix-core products and vector ALU work overlap on a SIMD
    (csa2_diag_mfma_valu): the loop of eight independent 32x32x16 f16
    products, of 64 independent fp32 FMAs, and of both, two waves per SIMD
    on every CU; median of reps timed launches each.  overlap = the share
    of the shorter loop's time hidden when both run: 1 if they overlap
    fully, 0 if they serialize."""
    sink = torch.empty(256 * 512, dtype=torch.float32, device="cuda")
    res = {}
    for mode, key in ((1, "mfma_us"), (2, "valu_us"), (3, "both_us")):
        tsl.csa2_diag_mfma_valu(mode, iters, sink)
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            tsl.csa2_diag_mfma_valu(mode, iters, sink)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        res[key] = sorted(ts)[len(ts) // 2]
    hidden = res["mfma_us"] + res["valu_us"] - res["both_us"]
    res["overlap"] = hidden / min(res["mfma_us"], res["valu_us"])
    res["what"] = ("per iteration and wave: 8 independent v_mfma_f32_32x32x16_f16, 64 independent fp32 FMAs, "
                   "or both; 256 workgroups of 8 waves, %d iterations" % iters)
    return res


def targets(torch, synth, LayerRunner, timer, args):
    """The two stated targets, each on its own workload: prefill index
    scoring at >= 0.5 of the FP8 MFMA peak (the 4,096-query m = 2 chunk) and
    decode sparse attention at >= 0.6 of HBM (the batch-64, 262,144-entry
    decoder group, per layer)."""
    out = {}
    for name in ("prefill_m2_chunk", "decoder_group_256k"):
        m = measure_workload(torch, synth, LayerRunner, timer, name, args, args.copies,
                             max(3, args.steps // 4), max(1, args.warmup // 2))
        st = m["stages"]
        rec = {"ms_per_step": m["gpu_ms_per_step"], "serial_ms_per_step": m["serial_gpu_ms_per_step"],
               "stages": {k: {kk: vv for kk, vv in v.items()} for k, v in st.items()}}
        if name == "prefill_m2_chunk":
            sc = st["index_scores_dense"]
            rec["target"] = {"stage": "index_scores_dense", "what": "MFMA FLOP rate against the FP8 peak",
                             "frac": sc["mfma_frac_fp8"], "frac_of_f16_peak": sc["mfma_frac_f16"],
                             "goal": 0.5, "met": sc["mfma_frac_fp8"] >= 0.5,
                             "pairs_per_s": sc["units"] / (sc["avg_us"] * 1e-6)}
            rec["roofline_scores"] = _roofline("index_scores_dense", sc, name)
            rec["roofline_attention"] = _roofline("sparse_attn", st["sparse_attn"], name)
        else:
            at = st["sparse_attn"]
            rec["target"] = {"stage": "sparse_attn", "what": "algorithmic bytes per layer call against HBM",
                             "frac": at["hbm_frac"], "frac_cold": at["cold"]["hbm_frac"],
                             "frac_warm": at["warm"]["hbm_frac"], "goal": 0.6,
                             "met": at["hbm_frac"] >= 0.6,
                             "us_per_layer": at["avg_us"],
                             "queries_per_s": at["units"] / (at["avg_us"] * 1e-6)}
            rec["roofline_attention"] = _roofline("sparse_attn", at, name)
            rec["roofline_scores"] = _roofline("index_scores_dense", st["index_scores_dense"], name)
        out[name] = rec
        del m
        torch.cuda.empty_cache()
    return out


def main():
    args = _parse()
    if args.summarize_profiles:
        summarize_profiles(*args.summarize_profiles, args.workload, args.profile_command)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma, args.workload, args.profile_command)
        return
    if args.summarize_sq:
        out_path, *dirs = args.summarize_sq
        summarize_sq(dirs, out_path, args.workload, args.stage_only or "-",
                     args.profile_command.split(" ;; "))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); sharding the path "
              "over several GPUs is designed, not built or measured.", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import top_sparse_long_amd as tsl
    from top_sparse_long_amd.driver import LayerRunner

    tsl.load()
    dev = "cuda"
    if args.stage_only:
        run = LayerRunner(synth.make_workload(args.workload, device=dev))
        steps = run.steps(overlap_route=True)
        for _, fn in steps:
            fn()
        calls = [fn for name, fn in steps if name == args.stage_only]
        if not calls:
            print(f"no stage {args.stage_only!r} in {args.workload}: "
                  f"{sorted(set(n for n, _ in steps))}", file=sys.stderr)
            sys.exit(2)
        for _ in range(args.repeat):
            for fn in calls:
                fn()
        torch.cuda.synchronize()
        print(json.dumps({"workload": args.workload, "stage": args.stage_only,
                          "calls": args.repeat * len(calls)}), flush=True)
        return
    ceiling = read_ceiling(torch, tsl)
    overlap = mfma_valu_overlap(torch, tsl)
    timer = Timer(torch, 1 << 30)

    m = measure_workload(torch, synth, LayerRunner, timer, args.workload, args, args.copies,
                         args.steps, args.warmup)
    runs = m["runs"]
    stages = m["stages"]
    ms_per_step = m["ms_per_step"]
    gpu_ms_per_step = m["gpu_ms_per_step"]
    serial_gpu_ms_per_step = m["serial_gpu_ms_per_step"]
    dom = max(stages, key=lambda s: stages[s]["avg_us"] * stages[s]["calls_per_step"])
    roofline = _roofline(dom, stages[dom], args.workload)
    roofline["achieved_from"] = ("median of per-launch times over graph replays rotated across "
                                 "the input copies, HIP events on the launch stream")
    wl = runs[0].wl
    value = m["index_keys_per_step"] / (ms_per_step * 1e-3)
    attn = stages.get("sparse_attn")
    attn_qps = attn["units"] / (attn["avg_us"] * 1e-6) if attn else None

    # the same step with serving-shaped I/O: index keys and main-KV records in
    # 64-slot pages of a random page order (index-key pages of 64 keys, then
    # their 64 scales), the top-k writing physical slots, attention gathering
    # by slot and turning its output back by RoPE
    serving = None
    if not args.no_serving and wl.quantized:
        pruns = [LayerRunner(r.wl, paged=synth.paged_layout(r.wl, 900 + c))
                 for c, r in enumerate(runs)]
        pgraphs = [timer.capture([f for _, f in r.steps(concurrent=True)]) for r in pruns]
        for i in range(args.warmup):
            pgraphs[i % len(pgraphs)].replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(timer.stream)
        for i in range(args.steps):
            pgraphs[i % len(pgraphs)].replay()
        e1.record(timer.stream)
        torch.cuda.synchronize()
        sms = e0.elapsed_time(e1) / args.steps
        del pgraphs
        pst = stage_stats(timer, pruns, args.samples, args.stage_reps, protocols=("rotated",))
        serving = {"io": "64-slot pages in random order; index-key pages of 64 keys then 64 "
                         "scales; top-k written as slots; attention by slot with inverse RoPE",
                   "gpu_ms_per_step": sms, "value": m["index_keys_per_step"] / (sms * 1e-3),
                   "unit": "index keys scored/s",
                   "stages_us": {k: v["avg_us"] for k, v in pst.items()}}
        del pruns

    cache_write = None
    if not args.no_cache_write:
        cache_write = cache_write_stage(torch, synth, tsl, wl, args.stage_reps, len(runs), args.workload)

    del runs, m
    torch.cuda.empty_cache()
    tgt = None
    if not args.no_targets:
        tgt = targets(torch, synth, LayerRunner, timer, args)

    cpu = None
    if not args.no_cpu_baseline:
        n_sample = args.cpu_sample if args.cpu_sample is not None else min(8, wl.Q)
        cpu = cpu_baseline(wl, n_sample)
        cpu.update(cpu_single_core(synth))

    out = {
        "metric": METRIC, "value": value, "unit": "index keys scored/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "gpu_ms_per_step": gpu_ms_per_step,
        "serial_gpu_ms_per_step": serial_gpu_ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": args.workload, "batch": wl.Q, "ctx_entries": wl.max_cols(),
                   "ratio": wl.ratio, "layers": [l.mode for l in wl.layers],
                   "topk": wl.topk, "pool_blocks": wl.n_blocks, "block_size": wl.block_size,
                   "index_k_format": ("e2m1+e4m3/16" if getattr(wl, "k_fmt", "fp8") == "fp4s16"
                                      else "e4m3+f32/row"),
                   "main_kv_record": ("288 B e2m1+e4m3/16" if getattr(wl, "main_fmt", "fp4") == "fp4s16"
                                      else "320 B e2m1+f32/32"),
                   "input_copies": args.copies,
                   "full_layer_selections": "shared launch; the top-k ranks blocks by their fused maxima first",
                   "schedule": ("each layer's attention on a second stream, overlapping the next layers' "
                                "scoring and selection (serial_gpu_ms_per_step: one stream)")},
        "sparse_attn_queries_per_s": attn_qps,
        "roofline": roofline,
        "hbm_read_ceiling": ceiling,
        "mfma_valu_overlap": overlap,
        "cpu_baseline": cpu,
        "stages": stages,
        "targets": tgt,
        "serving_io": serving,
        "cache_write": cache_write,
        "source_sha1": _source_hash(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
