#!/usr/bin/env python3
"""Benchmark of the compressed-attention block-selection chain on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload sweep]

A step is one call of the whole chain (admission + compaction, head-weight
fold, candidate floors, the shared key stream that scores every admitted block
for every row, the bounded radix select with the ordered output) over one
batch of synthetic input already resident in HBM.  The default workload is the
43-layer sweep at 300k context (43 layers x 6 verify rows x 75,000 compressed
blocks, d = 128, H = 64, k = 512).

Cold discipline: enough distinct copies of the inputs are rotated that at
least 512 MB (twice the 256 MB Infinity Cache) of algorithmic bytes are
touched between two uses of one copy, so no step can be served from the cache.

Prints one JSON line on stdout.  Besides the contract's keys it carries:
  roofline       the chain's algorithmic bytes per step over its device time
                 per step (HIP events around back-to-back steps), against the
                 8 TB/s HBM peak; `traffic` from the committed rocprofv3
                 counters when they were taken on the current kernel sources;
  ceiling        calibration launches on the same inputs: an empty kernel, a
                 plain read of every key row, a gather of exactly the admitted
                 rows with the key stream's addressing;
  single_calls   the 300k and 6-row verify configs as single calls, and the
                 300k config batched 43 layers to a call: median, p10 and p90 of
                 the per-call device time over event-bracketed calls, per-kernel
                 medians, the chain's fraction of the HBM peak, parity;
  cpu_baseline   the oracle timed on one host core on whole selections of the
                 workload (outputs compared with the GPU's), with the host's CPU
                 model and core count;
  attend         attention over the last step's selection (not part of value);
  q8             the same workload with the keys as the 8-bit stream (int8
                 codes, one fp16 scale per 32): throughput and its own
                 roofline on that stream's algorithmic bytes (not part of value);
  relu           the same workload under the per-head ReLU score: the score
                 kernel's flops against the bf16 MFMA peak (not part of value);
  decode         the 300k x43 and sweep configs decoded serially (each layer's
                 query depends on the previous layer's selection): per-layer
                 latency of eager launches and of one captured graph replay;
  pipelined      independent calls of the sweep, 300k x43, 300k and verify
                 configs in flight on 2 and 3 streams (one handle each): per
                 call time and the chain's fraction of the HBM peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak
MALL_BYTES = 256 << 20
COLD_BYTES = 2 * MALL_BYTES
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "sparse_attention_block_ds_amd", "csrc")
METRIC = "candidate blocks selected/sec per layer-row; achieved HBM GB/s vs peak"
WORKLOADS = {
    "sweep": "43-layer sweep at 300k context: 43 layers x 6 verify rows x 75,000 blocks",
    "300k": "300k-context decode: 1 row x 75,000 blocks, mask p=0.6",
    "300k_x43": "300k-context decode batched: 43 layers x 1 row x 75,000 blocks, mask p=0.6",
    "verify": "6-row verify: 6 rows x 32,768 blocks",
    "verify_int": "6-row verify, integer values: 6 rows x 32,768 blocks",
    "8k": "8k-context decode: 1 row x 2,048 blocks",
    "tiny": "tiny: 1 row x 4,096 blocks, H=4, d=64",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="sweep", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget for the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--engine", default="mfma", choices=["mfma", "valu"],
                    help="key-stream engine: bf16 matrix cores (default) or fp32 vector FMAs")
    ap.add_argument("--no-attend", action="store_true", help="skip the attention leg")
    ap.add_argument("--no-singles", action="store_true", help="skip the single-call legs")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the calibration launches")
    ap.add_argument("--no-q8", action="store_true", help="skip the 8-bit key stream leg")
    ap.add_argument("--no-relu", action="store_true", help="skip the per-head ReLU score leg")
    ap.add_argument("--no-decode", action="store_true", help="skip the serial decode legs")
    ap.add_argument("--no-pipelined", action="store_true",
                    help="skip the legs with independent calls in flight on several streams")
    ap.add_argument("--calls", type=int, default=200,
                    help="event-bracketed calls per single-call leg")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB read + 1 GiB write elementwise kernel, to scale "
                         "the FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def copy_calibration():
    """A plain elementwise kernel of known traffic: reads 1 GiB, writes 1 GiB."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_kernel": "bitwise_not int32", "bytes_read": n * 4, "bytes_written": n * 4,
                      "launches": 3}), flush=True)


def host_cpu():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count()


def sources_sha256():
    """One digest over every library source, so counters taken on other sources are not used."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def admitted_counts(p):
    """Admitted blocks per (layer, row) and the union-admitted bits per layer (host numpy)."""
    import numpy as np
    L, R, N = p.layers, p.rows, p.blocks
    lim = np.full((L, R), N, np.int64) if p.limit is None else np.clip(p.limit.astype(np.int64), 0, N)
    below = np.arange(N)[None, :]
    if p.mask is None:
        ubits = below < lim.max(axis=1)[:, None]
        return lim, ubits
    bits = np.unpackbits(p.mask.view(np.uint8), axis=-1, bitorder="little")[..., :N].astype(bool)
    per_row = np.zeros((L, R), np.int64)
    ubits = np.zeros((L, N), bool)
    for l in range(L):
        for r in range(R):
            adm = bits[l, 0 if bits.shape[1] == 1 else r] & (below[0] < lim[l, r])
            per_row[l, r] = adm.sum()
            ubits[l] |= adm
    return per_row, ubits


def algorithmic_bytes(p, union_count, fmt="bf16"):
    """Bytes the method itself must move per call (intermediates excluded): the
    union-admitted key rows (read once for all rows: 2d bytes each in bf16,
    d codes + d/32 fp16 scales on the 8-bit stream), the mask, q and w, the
    limits and the outputs."""
    import numpy as np
    row = 2 * p.dim if fmt == "bf16" else p.dim + 2 * (p.dim // 32)
    keys = int(union_count) * row
    mask = 0 if p.mask is None else int(np.prod(p.mask.shape)) * 4
    qw = p.layers * p.rows * p.heads * (p.dim + 1) * 2
    lim = 0 if p.limit is None else p.layers * p.rows * 4
    out = p.layers * p.rows * (p.k * 8 + 4)
    return {"keys": keys, "total": keys + mask + qw + lim + out}


def load_traffic(workload):
    """Counter-measured HBM bytes per launch, if taken on the current library sources."""
    path = os.path.join(PROFILES, f"chain_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("sources_sha256") != sources_sha256():
        return None
    return rec.get("traffic_bytes_per_launch")


def pct(xs):
    import numpy as np
    a = np.asarray(xs, np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90))}


class Runner:
    """One workload on the device: rotated input copies, outputs, a handle."""

    def __init__(self, p, engine, stream, sets=None, fmt="bf16", score="linear"):
        import numpy as np
        import torch
        from sparse_attention_block_ds_amd import selector as sel
        self.p = p
        self.stream = stream
        self.fmt = fmt
        self.per_row, self.ubits = admitted_counts(p)
        self.alg = algorithmic_bytes(p, self.ubits.sum(), fmt)
        n = max(2, math.ceil(COLD_BYTES / self.alg["total"])) if sets is None else sets
        first = sel.upload(p, "cuda:0")
        if fmt == "q8":  # the keys become the 8-bit stream, made by the quantise kernel
            q, w, keys, mask, limit = first
            first = (q, w, sel.quantize_q8(keys, stream=stream), mask, limit)
            del keys
            torch.cuda.synchronize()
        clone = lambda t: None if t is None else (tuple(x.clone() for x in t) if isinstance(t, tuple)
                                                  else t.clone())
        self.sets = [first] + [tuple(clone(t) for t in first) for _ in range(n - 1)]
        self.n_sets = n
        self.selector = sel.Selector(max_layers=p.layers, max_rows=p.rows, max_heads=p.heads,
                                     max_dim=p.dim, max_blocks=p.blocks, max_k=p.k, device=0,
                                     engine=engine, score=score)
        L, R, k = p.layers, p.rows, p.k
        self.outs = [(torch.empty((L, R, k), dtype=torch.int32, device="cuda:0"),
                      torch.empty((L, R, k), dtype=torch.float32, device="cuda:0"),
                      torch.empty((L, R), dtype=torch.int32, device="cuda:0"))
                     for _ in range(n)]
        self.candidates = int(np.asarray(self.per_row).sum())
        torch.cuda.synchronize()

    def step(self, i, events=None):
        q, w, keys, mask, limit = self.sets[i % self.n_sets]
        if self.fmt == "q8":
            self.selector.score_select_q8(q, w, keys[0], keys[1], self.p.k, mask, limit,
                                          out=self.outs[i % self.n_sets], stream=self.stream,
                                          events=events)
        else:
            self.selector.score_select(q, w, keys, self.p.k, mask, limit,
                                       out=self.outs[i % self.n_sets], stream=self.stream,
                                       events=events)

    def output(self, i):
        return tuple(t.cpu().numpy() for t in self.outs[i % self.n_sets])

    def close(self):
        self.selector.close()


def time_back_to_back(run, steps, warmup):
    """Wall and device milliseconds per step over `steps` back-to-back steps."""
    import torch
    for i in range(warmup):
        run.step(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(run.stream)
    for i in range(steps):
        run.step(i)
    b.record(run.stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1000.0 / steps
    return wall, a.elapsed_time(b) / steps


def per_call(run, calls):
    """Per-call device time (events right before and after each call, calls
    back to back) and per-kernel device times from the profiled entry point."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(calls)]
    for i, (a, b) in enumerate(evs):
        a.record(run.stream)
        run.step(i)
        b.record(run.stream)
    torch.cuda.synchronize()
    call_us = [a.elapsed_time(b) * 1000.0 for a, b in evs]
    kev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(calls)]
    for i in range(calls):
        run.step(i, kev[i])
    torch.cuda.synchronize()
    names = ("prep", "score", "select")
    kernels = {n: pct([e[j].elapsed_time(e[j + 1]) * 1000.0 for e in kev])["median"]
               for j, n in enumerate(names)}
    return pct(call_us), kernels


def _sub_problem(p, l, r):
    from sparse_attention_block_ds_amd import workloads as wl
    mrow = 0 if p.mask is None or p.mask.shape[1] == 1 else r
    return wl.Problem("s", p.k, p.q[l:l + 1, r:r + 1], p.w[l:l + 1, r:r + 1], p.keys[l:l + 1],
                      None if p.mask is None else p.mask[l:l + 1, mrow:mrow + 1],
                      None if p.limit is None else p.limit[l:l + 1, r:r + 1])


def _accept(p, sub, out, l, r, ora, lib, scorer=None):
    """The acceptance rule for one (layer, row): bit-exact on integer inputs
    (bf16 keys); otherwise count exact, every returned score within 1e-6 +
    1e-5 |oracle score of that block|, and every selected block's oracle score
    >= oracle m-th score - 1e-4 max |score|.  `scorer(blocks)` gives the
    oracle's per-block scores when the keys are not sub.keys (the 8-bit
    stream, always under the general rule)."""
    import numpy as np
    import oracle
    g_idx, g_score, g_count = out
    o_idx, o_score, o_count = ora
    if p.integer_valued and scorer is None:
        return (np.array_equal(o_idx[0, 0], g_idx[l, r]) and
                np.array_equal(o_score[0, 0], g_score[l, r]) and o_count[0, 0] == g_count[l, r])
    m = int(o_count[0, 0])
    if g_count[l, r] != m or not np.all(g_idx[l, r, m:] == -1):
        return False
    if m == 0:
        return True
    if scorer is None:
        s_or = oracle.score_blocks(sub.q, sub.w, sub.keys, 0, 0, g_idx[l, r, :m], lib=lib)
    else:
        s_or = scorer(g_idx[l, r, :m])
    kth = float(o_score[0, 0, m - 1])
    maxabs = max(abs(float(o_score[0, 0, 0])), abs(kth))
    return (bool(np.all(np.abs(g_score[l, r, :m] - s_or) <= 1e-6 + 1e-5 * np.abs(s_or))) and
            bool(np.all(s_or >= kth - 1e-4 * maxabs)))


def check_parity(p, out, pairs):
    """Number of (layer, row) pairs that fail the acceptance rule against the oracle."""
    import oracle
    lib = oracle.load()
    bad = 0
    for l, r in pairs:
        sub = _sub_problem(p, l, r)
        ora = oracle.select(sub.q, sub.w, sub.keys, sub.k, sub.mask, sub.limit, lib=lib)
        bad += 0 if _accept(p, sub, out, l, r, ora, lib) else 1
    return bad


def cpu_baseline(p, gpu_out, budget_s, per_row):
    """The oracle (one thread, as written, pinned to one core) on whole
    (layer, row) selections of this workload until about budget_s seconds have
    been spent; the GPU's outputs for those selections are checked against it."""
    import oracle
    lib = oracle.load()
    step = max(1, p.layers // 4)
    layers = list(range(0, p.layers, step)) + [l for l in range(p.layers) if l % step]
    order = [(l, r) for l in layers for r in range(p.rows)]
    prev = os.sched_getaffinity(0)
    os.sched_setaffinity(0, {min(prev)})
    done, cand, spent, bad = 0, 0, 0.0, 0
    try:
        for l, r in order:
            sub = _sub_problem(p, l, r)
            t0 = time.perf_counter()
            ora = oracle.select(sub.q, sub.w, sub.keys, sub.k, sub.mask, sub.limit, lib=lib)
            spent += time.perf_counter() - t0
            cand += int(per_row[l, r])
            done += 1
            bad += 0 if _accept(p, sub, gpu_out, l, r, ora, lib) else 1
            if spent >= budget_s:
                break
    finally:
        os.sched_setaffinity(0, prev)
    model, ncpu = host_cpu()
    return {"value": cand / spent, "unit": "candidate blocks/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} whole (layer,row) selections of this workload "
                      f"({cand} candidate blocks, {spent:.1f} s on one pinned core)",
            "host_cpu": model, "host_cores": ncpu, "_bad": bad, "_checked": done}


def balanced_ranges(ubits, groups):
    """Flattened (layer * N + block) range starts that give every workgroup the
    same number of union-admitted rows, with in-layer starts aligned to 32."""
    import numpy as np
    L, N = ubits.shape
    cum = np.cumsum(ubits.reshape(-1))
    total = int(cum[-1]) if cum.size else 0
    targets = (np.arange(groups + 1, dtype=np.int64) * total) // groups
    pos = np.searchsorted(cum, targets, side="left").astype(np.int64)
    pos = pos - (pos % N) % 32
    pos[0], pos[-1] = 0, L * N
    return np.maximum.accumulate(pos)


def ceiling(run, cus):
    """Calibration launches on the first input copy: an empty kernel (256 and
    4 x CU workgroups), a plain read of every key row, and the gather of the
    union-admitted rows only (ranges balanced by admitted count)."""
    import numpy as np
    import torch
    from sparse_attention_block_ds_amd import selector as sel
    p = run.p
    q, w, keys, mask, limit = run.sets[0]
    G = 4 * cus
    sink = torch.zeros(G, dtype=torch.int32, device="cuda:0")

    def med_us(fn, reps):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for a, b in evs:
            a.record(run.stream)
            fn()
            b.record(run.stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) * 1000.0 for a, b in evs]))

    res = {}
    for wg in (256, G):
        res[f"empty_kernel_us_{wg}_wgs"] = med_us(
            lambda: sel.calibrate(sel.DS_SEL_CALIB_EMPTY, wg, sink, stream=run.stream), 100)
    packed = keys.shape[2] == p.dim
    if packed:
        nbytes = p.layers * p.blocks * p.dim * 2
        us = med_us(lambda: sel.calibrate(sel.DS_SEL_CALIB_READ, G, sink, keys=keys,
                                          stream=run.stream), 20)
        res["read_all_rows"] = {"bytes": nbytes, "us": us, "gbs": nbytes / us / 1e3}
    ranges = torch.from_numpy(balanced_ranges(run.ubits, G)).to("cuda:0")
    gmask = None
    if mask is not None and mask.shape[1] == 1:
        gmask = mask
    if mask is None or gmask is not None:
        nbytes = int(run.ubits.sum()) * 2 * p.dim
        us = med_us(lambda: sel.calibrate(sel.DS_SEL_CALIB_GATHER, G, sink, keys=keys, mask=gmask,
                                          ranges=ranges, stream=run.stream), 20)
        res["gather_admitted_rows"] = {"bytes": nbytes, "us": us, "gbs": nbytes / us / 1e3}
    res["note"] = (f"median of event-timed launches of {G} workgroups x 256 threads "
                   "(empty: also 256); the read and gather touch the same bytes as one step")
    return res


def single_leg(name, engine, stream, calls):
    """One single-call config: per-call device-time percentiles, per-kernel
    medians, back-to-back throughput, parity of sampled (layer, row) pairs."""
    import numpy as np
    from sparse_attention_block_ds_amd import workloads as wl
    t0 = time.perf_counter()
    p = wl.make(name)
    run = Runner(p, engine, stream)
    log(f"[bench] single-call leg {name}: {run.n_sets} input copies, generated+uploaded in "
        f"{time.perf_counter() - t0:.1f}s")
    wall_ms, dev_ms = time_back_to_back(run, calls, 10)
    call_us, kernels = per_call(run, calls)
    out = run.output(calls - 1)
    pairs = [(l, r) for l in sorted({0, p.layers // 2, p.layers - 1}) for r in range(p.rows)]
    # the last call used copy (calls - 1) % n_sets, whose values equal the host problem
    bad = check_parity(p, out, pairs)
    run.close()
    if bad:
        log(f"[bench] PARITY FAILURE in the {name} leg: {bad} of {len(pairs)} pairs")
        sys.exit(3)
    alg = run.alg["total"]
    return {
        "workload": WORKLOADS[name], "input_copies": run.n_sets,
        "device_us_per_call": call_us,
        "kernels_us_median": kernels,
        "back_to_back_us_per_call": dev_ms * 1000.0,
        "algorithmic_bytes": alg,
        "chain_frac_hbm": alg / (call_us["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "chain_frac_hbm_back_to_back": alg / (dev_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "candidate_blocks_per_s": run.candidates / (call_us["median"] * 1e-6),
        "parity": f"{len(pairs)} (layer,row) pairs match the oracle "
                  + ("bit-exact" if p.integer_valued else "(tolerance + set rule)"),
    }


def q8_leg(p, stream, steps, warmup):
    """The same workload on the 8-bit key stream (ds_sel_score_select_q8 over
    codes and scales made by the quantise kernel): back-to-back throughput,
    per-call and per-kernel device times, the chain's and the score kernel's
    fraction of the HBM peak on the stream's algorithmic bytes; the stream of
    sampled layers is checked bit for bit against the oracle's quantiser and
    sampled (layer, row) selections against the oracle's 8-bit selection
    (tolerance + set rule: 8-bit scores are not exact)."""
    import numpy as np
    import oracle
    t0 = time.perf_counter()
    run = Runner(p, "mfma", stream, fmt="q8")
    log(f"[bench] q8 leg: {run.n_sets} input copies, quantised in {time.perf_counter() - t0:.1f}s")
    wall_ms, dev_ms = time_back_to_back(run, steps, warmup)
    call_us, kernels = per_call(run, steps)
    out = run.output(steps - 1)
    codes_d, scales_d = run.sets[(steps - 1) % run.n_sets][2]
    lib = oracle.load()
    layers = sorted({0, p.layers // 2, p.layers - 1})
    pairs = [(l, r) for l in layers for r in sorted({0, p.rows - 1})]
    bad = 0
    for l in layers:
        c_o, s_o = oracle.quantize_q8(p.keys[l:l + 1], lib=lib)
        c_g = codes_d[l:l + 1].cpu().numpy()
        s_g = scales_d[l:l + 1].cpu().numpy().view(np.uint16)
        if not (np.array_equal(c_o, c_g) and np.array_equal(s_o, s_g)):
            log(f"[bench] PARITY FAILURE in the q8 leg: layer {l}'s 8-bit stream differs")
            sys.exit(3)
        for r in sorted({0, p.rows - 1}):
            sub = _sub_problem(p, l, r)
            ora = oracle.select_q8(sub.q, sub.w, c_o, s_o, sub.k, sub.mask, sub.limit, lib=lib)
            scorer = lambda blocks: oracle.score_blocks_q8(sub.q, sub.w, c_o, s_o, 0, 0, blocks, lib=lib)
            bad += 0 if _accept(p, sub, out, l, r, ora, lib, scorer=scorer) else 1
    candidates, alg, n_sets = run.candidates, run.alg, run.n_sets
    run.close()
    if bad:
        log(f"[bench] PARITY FAILURE in the q8 leg: {bad} of {len(pairs)} pairs")
        sys.exit(3)
    achieved = alg["total"] / (dev_ms * 1e-3) / 1e9
    score_gbs = alg["keys"] / (kernels["score"] * 1e-6) / 1e9
    return {
        "workload": WORKLOADS[p.name] + ", keys as the 8-bit stream (int8 codes, fp16 scale per 32)",
        "input_copies": n_sets, "ms_per_step": wall_ms, "device_ms_per_step": dev_ms,
        "candidate_blocks_per_s": candidates / (wall_ms * 1e-3),
        "device_us_per_call": call_us, "kernels_us_median": kernels,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "algorithmic_bytes": alg["total"],
                     "bytes_per_key_row": p.dim + 2 * (p.dim // 32),
                     "score_kernel": {"algorithmic_key_bytes": alg["keys"],
                                      "us_median": kernels["score"], "gbs": score_gbs,
                                      "frac": score_gbs / HBM_PEAK_GBS}},
        "parity": f"8-bit stream of layers {layers} bit-exact vs the oracle's quantiser; "
                  f"{len(pairs)} (layer,row) pairs vs the oracle's 8-bit selection "
                  "(tolerance + set rule)",
    }


def relu_leg(p, stream, steps, warmup):
    """The same workload under the per-head ReLU score (a handle created with
    DS_SEL_FLAG_HEAD_RELU): every (row, head) pair meets every admitted key, so
    the score kernel is a matrix-core contraction.  Its algorithmic work is
    2 H d flops per admitted (row, block) pair; it is reported against the
    dense bf16 MFMA peak, with the key bytes against the HBM peak beside it.
    Sampled (layer, row) selections are checked against the oracle's ReLU
    selection (bit-exact on integer inputs, else the tolerance + set rule)."""
    import oracle
    t0 = time.perf_counter()
    run = Runner(p, "mfma", stream, score="relu")
    log(f"[bench] relu leg: {run.n_sets} input copies, ready in {time.perf_counter() - t0:.1f}s")
    wall_ms, dev_ms = time_back_to_back(run, steps, warmup)
    call_us, kernels = per_call(run, steps)
    out = run.output(steps - 1)
    lib = oracle.load()
    pairs = [(l, r) for l in sorted({0, p.layers // 2, p.layers - 1}) for r in sorted({0, p.rows - 1})]
    bad = 0
    for l, r in pairs:
        sub = _sub_problem(p, l, r)
        ora = oracle.select(sub.q, sub.w, sub.keys, sub.k, sub.mask, sub.limit, lib=lib, score="relu")
        scorer = lambda blocks: oracle.score_blocks(sub.q, sub.w, sub.keys, 0, 0, blocks, lib=lib,
                                                    score="relu")
        if p.integer_valued:
            scorer = None
        bad += 0 if _accept(p, sub, out, l, r, ora, lib, scorer=scorer) else 1
    candidates, alg, n_sets = run.candidates, run.alg, run.n_sets
    run.close()
    if bad:
        log(f"[bench] PARITY FAILURE in the relu leg: {bad} of {len(pairs)} pairs")
        sys.exit(3)
    flops = 2.0 * p.heads * p.dim * candidates
    tflops = flops / (kernels["score"] * 1e-6) / 1e12
    score_gbs = alg["keys"] / (kernels["score"] * 1e-6) / 1e9
    return {
        "workload": WORKLOADS[p.name] + ", score sum_h w_h max(q_h . K, 0)",
        "input_copies": n_sets, "ms_per_step": wall_ms, "device_ms_per_step": dev_ms,
        "candidate_blocks_per_s": candidates / (wall_ms * 1e-3),
        "device_us_per_call": call_us, "kernels_us_median": kernels,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                     "kernel": "score (per-head ReLU, bf16 MFMA)",
                     "flops_per_step": flops, "flops_per_candidate": 2 * p.heads * p.dim,
                     "key_bytes_gbs": score_gbs, "key_bytes_frac_hbm": score_gbs / HBM_PEAK_GBS},
        "parity": f"{len(pairs)} (layer,row) pairs vs the oracle's ReLU selection "
                  + ("bit-exact" if p.integer_valued else "(tolerance + set rule)"),
    }


def pipelined_leg(name, engine, calls, streams=(2, 3)):
    """Independent calls in flight together: S handles on S created streams
    (default priority), consecutive calls alternating between them, so that one
    call's latency-bound prep and select overlap another's key stream.  Per
    call: wall time over `calls` calls between two synchronisations, and the
    chain's algorithmic bytes over it; parity of the last call's outputs on
    sampled (layer, row) pairs."""
    import torch
    from sparse_attention_block_ds_amd import selector as sel
    from sparse_attention_block_ds_amd import workloads as wl
    p = wl.make(name)
    per_row, ubits = admitted_counts(p)
    alg = algorithmic_bytes(p, ubits.sum())["total"]
    n_sets = max(4, math.ceil(COLD_BYTES / alg))
    sets = [sel.upload(p, "cuda:0") for _ in range(n_sets)]
    outs = [(torch.empty((p.layers, p.rows, p.k), dtype=torch.int32, device="cuda:0"),
             torch.empty((p.layers, p.rows, p.k), dtype=torch.float32, device="cuda:0"),
             torch.empty((p.layers, p.rows), dtype=torch.int32, device="cuda:0")) for _ in range(n_sets)]
    res = {"workload": WORKLOADS[name], "input_copies": n_sets, "algorithmic_bytes": alg}
    last = None
    for S in streams:
        hs = [sel.Selector(p.layers, p.rows, p.heads, p.dim, p.blocks, p.k, device=0, engine=engine)
              for _ in range(S)]
        st = [torch.cuda.Stream() for _ in range(S)]

        def call(i):
            q, w, keys, mask, limit = sets[i % n_sets]
            hs[i % S].score_select(q, w, keys, p.k, mask, limit, out=outs[i % n_sets], stream=st[i % S])
        for i in range(2 * S + 4):
            call(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(calls):
            call(i)
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) * 1e6 / calls
        last = (calls - 1) % n_sets
        for h in hs:
            h.close()
        res[f"streams_{S}"] = {"us_per_call": us, "chain_frac_hbm": alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                               "candidate_blocks_per_s": float(per_row.sum()) / (us * 1e-6)}
    out = tuple(t.cpu().numpy() for t in outs[last])
    pairs = [(l, r) for l in sorted({0, p.layers - 1}) for r in sorted({0, p.rows - 1})]
    bad = check_parity(p, out, pairs)
    if bad:
        log(f"[bench] PARITY FAILURE in the pipelined {name} leg: {bad} pairs")
        sys.exit(3)
    res["parity"] = f"{len(pairs)} (layer,row) pairs of the last call vs the oracle"
    return res


def decode_leg(name, stream, reps):
    """Serial decode over the workload's layers (each layer's query depends on
    the previous layer's selection): per-layer device time of eager launches
    (4 L - 1 kernels enqueued one by one) and of the captured graph replay,
    median / p10 / p90 over `reps` decodes, HIP events on the launch stream.
    Two input copies alternate.  Sampled layers are checked against the oracle
    given the GPU's own previous layer (bit-exact on integer inputs)."""
    import numpy as np
    import torch
    import oracle
    from sparse_attention_block_ds_amd import selector as sel
    from sparse_attention_block_ds_amd import workloads as wl
    p = wl.make(name)
    L, R, H = p.layers, p.rows, p.heads
    s = sel.Selector(max_layers=L, max_rows=R, max_heads=H, max_dim=p.dim, max_blocks=p.blocks,
                     max_k=p.k, device=0)
    cap = torch.cuda.Stream()
    sets = []
    for _ in range(2):
        q, w, keys, mask, limit = sel.upload(p, "cuda:0")
        qw = torch.empty_like(q)
        out = (torch.empty((L, R, p.k), dtype=torch.int32, device="cuda:0"),
               torch.empty((L, R, p.k), dtype=torch.float32, device="cuda:0"),
               torch.empty((L, R), dtype=torch.int32, device="cuda:0"))
        sets.append((q, w, keys, mask, limit, qw, out))
    plans = [s.decode_plan(q, w, keys, p.k, mask, limit, q_work=qw, out=out, stream=cap)
             for q, w, keys, mask, limit, qw, out in sets]

    def timed(fn):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        with torch.cuda.stream(cap):
            for i in range(3):
                fn(i)
            for i, (a, b) in enumerate(evs):
                a.record(cap)
                fn(i)
                b.record(cap)
        torch.cuda.synchronize()
        return pct([a.elapsed_time(b) * 1000.0 / L for a, b in evs])

    def eager(i):
        q, w, keys, mask, limit, qw, out = sets[i % 2]
        s.decode(q, w, keys, p.k, mask, limit, q_work=qw, out=out, stream=cap)

    eager_us = timed(eager)
    graph_us = timed(lambda i: plans[i % 2].launch(cap))
    # the last replay used set (reps - 1) % 2
    idx, score, count = (t.cpu().numpy() for t in sets[(reps - 1) % 2][6])
    bad = 0
    checked = sorted({1, L // 2, L - 1} if L > 1 else {0})
    lib = oracle.load()
    for l in checked:
        ql = p.q[l:l + 1].copy()
        if l > 0:
            for r in range(R):
                sh = int(idx[l - 1, r, 0]) % H if count[l - 1, r] > 0 else 0
                ql[0, r] = np.roll(p.q[l, r], -sh, axis=0)
        for r in range(R):
            sub = _sub_problem(wl.Problem("layer", p.k, np.concatenate([p.q[:l], ql, p.q[l + 1:]]), p.w,
                                          p.keys, p.mask, p.limit, p.integer_valued), l, r)
            ora = oracle.select(sub.q, sub.w, sub.keys, sub.k, sub.mask, sub.limit, lib=lib)
            bad += 0 if _accept(p, sub, (idx, score, count), l, r, ora, lib) else 1
    for pl in plans:
        pl.close()
    s.close()
    if bad:
        log(f"[bench] PARITY FAILURE in the {name} decode leg: {bad} selections")
        sys.exit(3)
    return {"workload": WORKLOADS[name] + ", layers serially dependent", "layers": L,
            "eager_us_per_layer": eager_us, "graph_us_per_layer": graph_us,
            "launches_per_decode": 4 * L - 1,
            "parity": f"layers {checked} x {R} rows vs the oracle given the GPU's previous layer "
                      + ("bit-exact" if p.integer_valued else "(tolerance + set rule)")}


def attend_leg(run, steps):
    """Attention over the last step's selection (64 query heads per row, bf16 q
    and values drawn on the device from a fixed seed), timed with HIP events on
    the launch stream; two (layer, row) pairs are checked against the fp64
    oracle.  Algorithmic bytes per (layer, row): count x 2 x 2d (the selected K
    and V rows) + H d 2 (q) + H d 4 (the fp32 output); flops 4 H d per block."""
    import numpy as np
    import torch
    import oracle
    p, stream = run.p, run.stream
    i_last = steps - 1
    keys = run.sets[i_last % run.n_sets][2]
    idx, _, count = run.outs[i_last % run.n_sets]
    L, R, H, d, N = p.layers, p.rows, p.heads, p.dim, p.blocks
    g = torch.Generator(device="cuda:0")
    g.manual_seed(1234)
    qa = torch.randn((L, R, H, d), generator=g, device="cuda:0").to(torch.bfloat16)
    values = torch.randn((L, N, d), generator=g, device="cuda:0").to(torch.bfloat16)
    out = torch.empty((L, R, H, d), dtype=torch.float32, device="cuda:0")
    scale = 1.0 / math.sqrt(d)
    for _ in range(3):
        run.selector.attend(qa, keys, values, idx, count, scale, out=out, stream=stream)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(20)]
    for a, b in evs:
        a.record(stream)
        run.selector.attend(qa, keys, values, idx, count, scale, out=out, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
    cnt = count.cpu().numpy().astype(np.int64)
    sel_blocks = int(np.clip(cnt, 0, p.k).sum())
    nbytes = sel_blocks * 2 * 2 * d + L * R * H * d * (2 + 4)
    flops = 4.0 * H * d * sel_blocks
    bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    worst = 0.0
    for l, r in ((0, 0), (L - 1, R - 1)):
        ref = oracle.attend(bits(qa[l:l + 1, r:r + 1]), bits(keys[l:l + 1]), bits(values[l:l + 1]),
                            idx[l:l + 1, r:r + 1].cpu().numpy(), count[l:l + 1, r:r + 1].cpu().numpy(),
                            scale)
        err = np.abs(out[l:l + 1, r:r + 1].cpu().numpy() - ref).max() / max(np.abs(ref).max(), 1e-30)
        worst = max(worst, float(err))
    if not worst <= 1e-4:
        log(f"[bench] ATTENTION PARITY FAILURE: relative max error {worst:.3e}")
        sys.exit(3)
    return {"kernel": "attend (softmax(q K^T) V over the selected blocks)", "us_median": ms * 1000.0,
            "selected_blocks": sel_blocks, "algorithmic_bytes": nbytes,
            "achieved_gbs": nbytes / (ms / 1000.0) / 1e9,
            "frac_hbm": nbytes / (ms / 1000.0) / 1e9 / HBM_PEAK_GBS,
            "tflops": flops / (ms / 1000.0) / 1e12,
            "parity": f"2 (layer,row) pairs vs the fp64 oracle, max relative error {worst:.1e}"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the selection chain runs on a single MI355X here; "
              "multi-GPU runs are not part of this build (see the sharding note in DESIGN.md).",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch
    from sparse_attention_block_ds_amd import workloads as wl

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    torch.cuda.set_device(0)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    t_gen = time.perf_counter()
    p = wl.make(args.workload)
    run = Runner(p, args.engine, stream)
    log(f"[bench] workload {p.name}: L={p.layers} R={p.rows} H={p.heads} d={p.dim} N={p.blocks} "
        f"k={p.k}; candidates {run.candidates}; {run.n_sets} input copies; "
        f"ready in {time.perf_counter() - t_gen:.1f}s")

    # timed region: exactly K back-to-back steps
    ms_per_step, dev_ms = time_back_to_back(run, args.steps, args.warmup)
    log(f"[bench] {args.steps} steps: {ms_per_step:.4f} ms wall, {dev_ms:.4f} ms device per step")
    call_us, kernels = per_call(run, args.steps)
    gpu_out = run.output(args.steps - 1)

    value = run.candidates / (ms_per_step / 1000.0)
    achieved = run.alg["total"] / (dev_ms / 1000.0) / 1e9
    score_gbs = run.alg["keys"] / (kernels["score"] * 1e-6) / 1e9

    cpu, parity = None, "not checked (--no-cpu-baseline)"
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(p, gpu_out, args.cpu_seconds, run.per_row)
        if cpu["_bad"]:
            log(f"[bench] PARITY FAILURE on {cpu['_bad']} of {cpu['_checked']} sampled selections")
            sys.exit(3)
        parity = f"{cpu['_checked']} whole selections match the oracle " + \
                 ("bit-exact" if p.integer_valued else "(tolerance + set rule)")
        cpu = {k: v for k, v in cpu.items() if not k.startswith("_")}
        log(f"[bench] cpu baseline done: {parity}")

    ceil = None if args.no_ceiling else ceiling(run, cus)
    if ceil:
        log(f"[bench] ceiling: {json.dumps(ceil)}")
    attend = None
    if not args.no_attend and p.heads >= 16:
        attend = attend_leg(run, args.steps)
        log("[bench] attention leg done")
    candidates, n_sets, alg = run.candidates, run.n_sets, run.alg
    run.close()
    del run
    torch.cuda.empty_cache()

    singles = None
    if not args.no_singles and args.workload == "sweep":
        singles = {}
        for name in ("300k", "verify", "300k_x43"):
            singles[name] = single_leg(name, args.engine, stream, args.calls)
            log(f"[bench] {name}: {json.dumps(singles[name]['device_us_per_call'])} us per call")
            torch.cuda.empty_cache()

    relu = None
    if not args.no_relu:
        from sparse_attention_block_ds_amd import selector as sel_mod
        try:
            relu = relu_leg(p, stream, args.steps, args.warmup)
            log(f"[bench] relu leg: {relu['ms_per_step']:.4f} ms per step, score kernel "
                f"{relu['roofline']['frac']:.3f} of the bf16 MFMA peak")
        except sel_mod.DsSelError as e:  # heads too many for the LDS stage at this shape
            if e.status != sel_mod.DS_SEL_E_UNSUPPORTED:
                raise
            relu = {"skipped": str(e)}
        torch.cuda.empty_cache()

    pipelined = None
    if not args.no_pipelined and args.workload == "sweep":
        pipelined = {}
        for name, calls in (("sweep", 60), ("300k_x43", 60), ("300k", 400), ("verify", 400)):
            pipelined[name] = pipelined_leg(name, args.engine, calls)
            log(f"[bench] pipelined {name}: " + ", ".join(
                f"{k} {v['us_per_call']:.1f} us/call ({v['chain_frac_hbm']:.3f})"
                for k, v in pipelined[name].items() if k.startswith("streams_")))
            torch.cuda.empty_cache()

    decode = None
    if not args.no_decode and args.workload == "sweep":
        decode = {}
        for name in ("300k_x43", "sweep"):
            decode[name] = decode_leg(name, stream, 20)
            log(f"[bench] decode {name}: eager {decode[name]['eager_us_per_layer']['median']:.1f} us, "
                f"graph {decode[name]['graph_us_per_layer']['median']:.1f} us per layer")
            torch.cuda.empty_cache()

    q8 = None
    if not args.no_q8 and p.dim % 32 == 0:
        q8 = q8_leg(p, stream, args.steps, args.warmup)
        log(f"[bench] q8 leg: {q8['ms_per_step']:.4f} ms per step, chain "
            f"{q8['roofline']['frac']:.3f} of the HBM peak")
        torch.cuda.empty_cache()

    traffic = load_traffic(p.name)
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "candidate blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": WORKLOADS[p.name],
            "layers": p.layers, "rows": p.rows, "heads": p.heads, "dim": p.dim,
            "blocks": p.blocks, "k": p.k, "candidates_per_step": candidates,
            "input_copies_rotated": n_sets, "engine": args.engine,
        },
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
            "kernel": "chain (prep + score + select): algorithmic bytes per step / device time per step",
            "algorithmic_bytes": alg["total"],
            "score_kernel": {"algorithmic_key_bytes": alg["keys"],
                             "us_median": kernels["score"], "gbs": score_gbs,
                             "frac": score_gbs / HBM_PEAK_GBS},
        },
        "ceiling": ceil,
        "cpu_baseline": cpu,
        "kernels_us_median": kernels,
        "device_us_per_call": call_us,
        "device_ms_per_step": dev_ms,
        "layer_row_selections_per_s": p.layers * p.rows / (ms_per_step / 1000.0),
        "parity": parity,
        "single_calls": singles,
        "attend": attend,
        "q8": q8,
        "relu": relu,
        "decode": decode,
        "pipelined": pipelined,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
