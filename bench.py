"""Benchmark: block top-k sparse decode attention on one MI355X.

A step is one decode step of the method over the whole batch, all on one HIP
stream: S1 centroid update of the page holding each sequence's newest token,
S2+S3 group scoring and top-k selection, S4 attention over the selected blocks.
The timed step is the library's single-launch form through the block sketches
(btk_decode_step_sketch: every block's 8-bit sketch row bounds its score, only
the blocks that could be selected are scored from their fp32 centroid rows;
indices, outputs and centroids identical to btk_decode_step, checked on every
replica).  Beside it: the single launch that scans every fp32 centroid row
(btk_decode_step), and the same step as three calls (btk_centroid_update,
btk_select, btk_sparse_attend) with a per-kernel breakdown.  The KV append itself is the
caller's op and is not timed; lengths stay fixed so every step is the same
work.  The workload is the Qwen3-8B-shaped decode layer (B=32, Hq=32, Hkv=8,
D=128, bf16, ragged contexts U[4096, 32768], shuffled 16-token pages, top-k =
32 blocks), drawn by ``synth`` with seed 3000.

Inputs are resident in HBM before timing starts.  The step rotates over
``--replicas`` independent copies of the KV cache, centroids and tables so that
consecutive steps touch different memory: a sparse step's working set (about
220 MB) would otherwise stay in the 256 MB last-level cache between steps,
which a real model, with its other layers in between, never sees.

Prints one JSON line.  ``value`` is query-tokens/s = B / step time.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X published HBM3E bandwidth
METRIC = "sparse decode attention query-tokens/s + achieved HBM GB/s (% of peak), vs dense"
WORKLOAD = ("qwen3-8b-shaped decode layer: B=32, Hq=32, Hkv=8 (group 4), D=128, bf16, "
            "contexts U[4096,32768], 16-token pages, shuffled block table, top_k=32 blocks")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_step_unit_kernel_qwen3-8b_traffic.json")
PLAIN_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_step_kernel_qwen3-8b_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "block_top_sparse_btk_amd", "csrc", f)
                  for f in ("step.hip", "select_dev.h", "attend_dev.h", "centroid_dev.h",
                            "sketch_dev.h", "btk_internal.h")]


# ---------------------------------------------------------------- byte model

def dense_kv_bytes_per_token(num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K and V bytes one cached token costs one layer's dense decode attention."""
    return 2 * num_kv_heads * head_dim * elem_bytes


def selected_tokens(indices, seq_lens, page=16):
    """Valid tokens of the selected blocks, per (sequence, KV head) unit."""
    out = []
    for b, L in enumerate([int(x) for x in seq_lens]):
        row = []
        for g in range(indices.shape[1]):
            js = [j for j in indices[b, g].tolist() if j >= 0]
            row.append(sum(min(page, L - j * page) for j in js))
        out.append(row)
    return out


def algorithmic_bytes(seq_lens, num_q_heads, num_kv_heads, head_dim, top_k, elem_bytes,
                      page=16, sel_tokens=None):
    """Bytes each kernel of a step must move (reads + writes), by the method's definition.

    Per unit (sequence b, KV head g), r = Hq/Hkv, e = element bytes, n_b blocks:
      S1 centroid:  the newest token's page keys (v_last*D*e) + one centroid (4*D)
      S2+S3 select: group queries (r*D*e) + n_b centroids (4*D*n_b) + k indices (4*k),
                    and the sequence's block table (4*n_b) once per sequence
      S4 attend:    k indices + their block-table entries (8*k), queries (r*D*e),
                    K and V of the selected blocks' valid tokens (2*v_j*D*e), out (r*D*e)
      dense:        table (4*n_b per sequence) + q and out (2*r*D*e) + all K,V (2*L*D*e)
      local:        the same over the most recent min(k, n_b) blocks: their table
                    entries (4*k_b per sequence), q and out, K,V of their valid tokens
      token:        the token-level baseline with a budget of 16*k tokens: table (4*n_b
                    per sequence), q and out, every valid key (L*D*e) and the K,V
                    of the kept tokens (2*min(16k, L)*D*e)
    """
    r, D, e, P = num_q_heads // num_kv_heads, head_dim, elem_bytes, page
    cen = sel = att = dense = local = token = 0
    for b, L in enumerate([int(x) for x in seq_lens]):
        nb = (L + P - 1) // P
        kb = min(top_k, nb)
        v_last = L - (nb - 1) * P
        sel += 4 * nb
        dense += 4 * nb
        local += 4 * kb
        local_toks = L - P * (nb - kb)
        token += 4 * nb
        for g in range(num_kv_heads):
            # valid tokens of the selected blocks: exact when the selection is
            # given, else every selected block full (or all of L when k >= n_b)
            toks = sel_tokens[b][g] if sel_tokens is not None else (L if kb == nb else kb * P)
            cen += v_last * D * e + 4 * D
            sel += r * D * e + 4 * D * nb + 4 * top_k
            att += 8 * top_k + 2 * r * D * e + 2 * toks * D * e
            dense += 2 * r * D * e + 2 * L * D * e
            local += 2 * r * D * e + 2 * local_toks * D * e
            token += 2 * r * D * e + L * D * e + 2 * min(P * top_k, L) * D * e
    return {"centroid": cen, "select": sel, "attend": att, "step": cen + sel + att,
            "dense": dense, "local": local, "token": token}


def sketch_step_bytes(seq_lens, num_q_heads, num_kv_heads, head_dim, top_k, elem_bytes,
                      cand_counts, sel_tokens, page=16, fp32_scan=False):
    """Bytes the step through the block sketch must move (btk_decode_step_sketch).

    Per unit, as the full step (algorithmic_bytes) except the centroid scan:
      S1:     the newest token's page keys (v_last*D*e), its centroid (4*D) and its
              rebuilt sketch row (D + 8)
      S2+S3:  group queries (r*D*e), every block's sketch row (n_b*(D + 8): codes and
              header), the fp32 centroid rows of the unit's m candidates (4*D*m),
              k indices (4*k); the sequence's block table (4*n_b) once per sequence
      S4:     as in the full step
    cand_counts[b][g] = m (0 when every block is kept), sel_tokens as for
    algorithmic_bytes. fp32_scan: the launch took the persistent fp32-scan kernel (too
    few units to fill the device), which reads every block's fp32 row (4*D*n_b) and no
    sketch row, and writes the refreshed block's sketch row as above.
    """
    r, D, e, P = num_q_heads // num_kv_heads, head_dim, elem_bytes, page
    total = 0
    for b, L in enumerate([int(x) for x in seq_lens]):
        nb = (L + P - 1) // P
        v_last = L - (nb - 1) * P
        total += 4 * nb
        for g in range(num_kv_heads):
            m = int(cand_counts[b][g])
            total += v_last * D * e + 4 * D + D + 8
            if fp32_scan:
                total += r * D * e + 4 * D * nb + 4 * top_k
            else:
                total += r * D * e + nb * (D + 8) + 4 * D * m + 4 * top_k
            total += 8 * top_k + 2 * r * D * e + 2 * sel_tokens[b][g] * D * e
    return total


# ---------------------------------------------------------------- helpers

def _sketch_takes_unit_kernel(B, hkv, max_blocks, dev) -> bool:
    """Which kernel btk_decode_step_sketch launches for these workloads: one workgroup per
    (sequence, KV head) unit when the units fill the device (at least one per compute unit)
    and the table fits its block limit (3072), else the persistent fp32-scan kernel. Its other
    limits (top-k <= 256, group <= 8, one attention split) hold for every workload here."""
    import torch
    return (B * hkv >= torch.cuda.get_device_properties(dev).multi_processor_count
            and max_blocks <= 3072)


def _sources_digest() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _measured_traffic(path=TRAFFIC_FILE):
    """HBM bytes per decode-step launch from the committed rocprofv3 counter
    runs, or None if the kernel source changed since they were taken."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != _sources_digest():
        return None
    return t.get("traffic_bytes_per_launch")


def _cpu_baseline(bt, seconds: float):
    """The oracle's sparse step on the host cores, time-bounded."""
    import torch
    import oracle

    first = (bt.seq_lens - 1).to(torch.int32)
    cents = oracle.centroids(bt.k_cache, bt.block_table, bt.seq_lens)
    steps, t0 = 0, time.perf_counter()
    while True:
        oracle.sparse_step(bt.q, bt.k_cache, bt.v_cache, bt.block_table, bt.seq_lens, bt.top_k,
                           cents=cents, first_pos=first)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds and steps >= 2:
            break
    per_step = el / steps
    return {"value": bt.batch / per_step, "unit": "query-tokens/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"{steps} full sparse decode steps of the same batch (S1 newest-token pages, "
                      f"scores, top-k, attention), {el:.1f} s of CPU time on "
                      f"{oracle.max_threads()} threads"}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rates(bt, seconds: float):
    """The oracle's sparse step on the host: all threads on the whole batch for
    about `seconds`, and one thread on one sequence (all its KV heads), both as
    query-tokens/s of the whole batch's step."""
    import torch
    import oracle

    first = (bt.seq_lens - 1).to(torch.int32)
    cents = oracle.centroids(bt.k_cache, bt.block_table, bt.seq_lens)
    threads = oracle.max_threads()
    steps, t0 = 0, time.perf_counter()
    while True:
        oracle.sparse_step(bt.q, bt.k_cache, bt.v_cache, bt.block_table, bt.seq_lens, bt.top_k,
                           cents=cents, first_pos=first)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    all_rate = bt.batch * steps / el
    oracle.set_threads(1)
    try:
        n1, t0 = 0, time.perf_counter()
        while True:
            b = n1 % bt.batch
            oracle.sparse_step(bt.q[b:b + 1], bt.k_cache, bt.v_cache, bt.block_table[b:b + 1],
                               bt.seq_lens[b:b + 1], bt.top_k, cents=cents,
                               first_pos=first[b:b + 1])
            n1 += 1
            el1 = time.perf_counter() - t0
            if el1 >= seconds / 2 and n1 >= 1:
                break
    finally:
        oracle.set_threads(threads)
    return {"value": round(all_rate, 1), "unit": "query-tokens/s", "cores": threads,
            "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": f"{steps} full steps of the batch in {el:.1f} s on {threads} threads",
            "one_thread": {"value": round(n1 / el1, 2), "unit": "query-tokens/s", "cores": 1,
                           "sample": f"{n1} one-sequence steps (all KV heads) in {el1:.1f} s"}}


def _pcts(xs):
    xs = sorted(xs)
    pick = lambda q: xs[min(len(xs) - 1, int(round(q * (len(xs) - 1))))]  # noqa: E731
    return {"p10": round(pick(0.1), 3), "p50": round(pick(0.5), 3), "p90": round(pick(0.9), 3)}


def measure_workload(name, bt, dev, steps, cpu_seconds, replicas=None, cpu_sample=None):
    """One workload's line: the single-launch step and the dense kernel on the same
    inputs (rotating replicas, HIP events on the library's stream), algorithmic
    bytes, roofline fraction, bytes per token, p10/p50/p90 of batch averages, the
    oracle on the host."""
    import torch

    import block_top_sparse_btk_amd as btk

    B, hq, hkv, D, k = bt.batch, bt.num_q_heads, bt.num_kv_heads, bt.head_dim, bt.top_k
    e = 2 if bt.dtype == torch.bfloat16 else 4
    nb0 = algorithmic_bytes(bt.seq_lens.tolist(), hq, hkv, D, k, e)
    if replicas is None:  # enough copies that consecutive steps miss the last-level cache
        replicas = max(2, min(16, -(-600_000_000 // max(1, nb0["step"]))))
    if bt.k_cache.is_cuda:  # drawn on the device: far larger than the cache already
        replicas = 1
    lib = btk._lib()
    stream = torch.cuda.current_stream(dev)
    hs = stream.cuda_stream
    base = bt.to(dev)
    prob = btk.make_problem(base.q, base.k_cache, base.block_table)
    first = (base.seq_lens - 1).to(torch.int32)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    reps = []
    for i in range(replicas):
        d = base if i == 0 else bt.to(dev)
        cent = torch.zeros((bt.num_pages, hkv, D), dtype=torch.float32, device=dev)
        btk.btk_centroid_update(d.k_cache, d.block_table, d.seq_lens, cent, problem=prob)
        ws = btk.new_workspace(prob, k, dev)
        idx = torch.empty((B, hkv, k), dtype=torch.int32, device=dev)
        out, dout = torch.empty_like(d.q), torch.empty_like(d.q)
        sk = btk.new_sketch(prob, dev)
        btk.btk_sketch_update(cent, d.block_table, d.seq_lens, sk, ws, problem=prob)
        sidx, sout = torch.empty_like(idx), torch.empty_like(out)
        cc = torch.zeros((B, hkv), dtype=torch.int32, device=dev)
        reps.append(dict(d=d, ws=ws, idx=idx, out=out, sidx=sidx, sout=sout, cc=cc,
                         keep=(cent, dout, sk),
                         step=(ctypes.byref(prob), p(d.q), p(d.k_cache), p(d.v_cache),
                               p(d.block_table), p(d.seq_lens), p(first), p(cent), k, p(idx),
                               p(out), None, p(ws), ws.numel(), hs),
                         sk=(ctypes.byref(prob), p(d.q), p(d.k_cache), p(d.v_cache),
                             p(d.block_table), p(d.seq_lens), p(first), p(cent), p(sk),
                             sk.numel(), k, p(sidx), p(sout), None, p(cc), p(ws), ws.numel(),
                             hs),
                         den=(ctypes.byref(prob), p(d.q), p(d.k_cache), p(d.v_cache),
                              p(d.block_table), p(d.seq_lens), p(dout), None, p(ws), ws.numel(),
                              hs)))
    torch.cuda.synchronize()

    def check(st):
        if st:
            raise RuntimeError(f"{name}: library call failed: {lib.btk_status_string(st).decode()}")

    def timed(fn_name, key, n, batch):
        f = getattr(lib, fn_name)
        for i in range(10):
            check(f(*reps[i % replicas][key]))
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(max(1, n // batch))]
        i = 0
        for e0, e1 in evs:
            e0.record(stream)
            for _ in range(batch):
                check(f(*reps[i % replicas][key]))
                i += 1
            e1.record(stream)
        torch.cuda.synchronize()
        per = [1e3 * e0.elapsed_time(e1) / batch for e0, e1 in evs]
        return sum(per) / len(per), per

    step_us, step_per = timed("btk_decode_step", "step", steps, 10)
    sk_us, sk_per = timed("btk_decode_step_sketch", "sk", steps, 10)
    dense_us, dense_per = timed("btk_dense_attend", "den", max(10, steps // 5), 5)
    for r in reps:
        if btk.workspace_error_bits(r["ws"]):
            raise RuntimeError(f"{name}: device-side input guard fired")
        if not (torch.equal(r["sidx"], r["idx"]) and torch.equal(r["sout"], r["out"])):
            raise RuntimeError(f"{name}: the sketched step disagrees with the step")
    sel_toks = selected_tokens(reps[0]["idx"].cpu(), bt.seq_lens.cpu())
    nb = algorithmic_bytes(bt.seq_lens.tolist(), hq, hkv, D, k, e, sel_tokens=sel_toks)
    cc = reps[0]["cc"].cpu()
    unit = _sketch_takes_unit_kernel(B, hkv, bt.block_table.shape[1], dev)
    sk_bytes = sketch_step_bytes(bt.seq_lens.tolist(), hq, hkv, D, k, e, cc.tolist(), sel_toks,
                                 fp32_scan=not unit)
    sk_gbps = sk_bytes / (sk_us * 1e-6) / 1e9
    gbps = nb["step"] / (step_us * 1e-6) / 1e9
    dgbps = nb["dense"] / (dense_us * 1e-6) / 1e9
    res = {"workload": name, "batch": B, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": D,
           "top_k": k, "seed": bt.seed,
           "contexts": {"min": int(bt.seq_lens.min()), "mean": round(float(bt.seq_lens.float().mean()), 1),
                        "max": int(bt.seq_lens.max())},
           "replicas": replicas,
           "step": {"kernel": "decode_step_kernel", "us": round(step_us, 3),
                    "us_batches": _pcts(step_per), "value": round(B / (step_us * 1e-6), 1),
                    "unit": "query-tokens/s", "gbps": round(gbps, 1),
                    "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4), "bytes": nb["step"],
                    "bytes_per_token": round(nb["step"] / B, 1)},
           "dense": {"kernel": "attend_kernel (every block)", "us": round(dense_us, 3),
                     "us_batches": _pcts(dense_per), "value": round(B / (dense_us * 1e-6), 1),
                     "unit": "query-tokens/s", "gbps": round(dgbps, 1),
                     "frac_of_peak": round(dgbps / HBM_PEAK_GBPS, 4), "bytes": nb["dense"],
                     "bytes_per_token": round(nb["dense"] / B, 1)},
           "sketch_step": {"kernel": ("decode_step_unit_kernel" if unit
                                      else "decode_step_kernel (fp32 scan, sketch rows kept "
                                           "current)"),
                           "us": round(sk_us, 3), "us_batches": _pcts(sk_per),
                           "value": round(B / (sk_us * 1e-6), 1), "unit": "query-tokens/s",
                           "gbps": round(sk_gbps, 1),
                           "frac_of_peak": round(sk_gbps / HBM_PEAK_GBPS, 4), "bytes": sk_bytes,
                           "bytes_per_token": round(sk_bytes / B, 1),
                           "candidates_per_unit": round(float(cc.float().mean()), 1),
                           "speedup_vs_dense": round(dense_us / sk_us, 2)},
           "speedup_vs_dense": round(dense_us / step_us, 2),
           "best_step_us": round(min(step_us, sk_us), 3),
           "best_speedup_vs_dense": round(dense_us / min(step_us, sk_us), 2),
           "bytes_ratio": round(nb["dense"] / nb["step"], 2),
           "note": "times are HIP-event averages over back-to-back launches; us_batches: "
                   "percentiles of the averages of batches of 10 (step) / 5 (dense) launches"}
    del reps, base
    torch.cuda.empty_cache()
    if cpu_seconds > 0:
        res["cpu_baseline"] = _oracle_rates(cpu_sample if cpu_sample is not None else bt,
                                            cpu_seconds)
        if cpu_sample is not None:
            res["cpu_baseline"]["sample"] += (f" (a sample of {cpu_sample.batch} of the "
                                              f"{B} sequences, copied to the host)")
    return res


# One GPU's share of the Qwen3-8B serving batch of the Kinetics README's block
# top-k benchmark ("Benchmark Block TopK Attention throughput": batch 4096,
# 32768-token contexts, 64 pages kept, eight-way tensor parallel so one KV head
# and its four query heads per GPU).  Its 69 GB of caches are drawn on the
# device; the oracle's rate is taken on a few of its sequences copied out.
SHARE = dict(batch=4096, num_q_heads=4, num_kv_heads=1, head_dim=128, context=32768, top_k=64,
             seed=8004)


def workload_batch(cfg, ctx, dev):
    """(batch, host sample for the oracle's rate or None) of one workload."""
    import synth
    if cfg == "share":
        bt = synth.make_device_batch(device=dev, name="qwen3-8b-share", **SHARE)
        sample, _ = synth.extract(bt, [0, 1365, 2730, 4095])
        return bt, sample
    return synth.make_config(cfg, context=ctx), None


WORKLOADS = [("qwen3-0.6b-shaped B=64 L=8192 k=16", 2, None),
             ("qwen3-30b-a3b-shaped Best-of-N B=16 (2048 shared + 30720) k=64", 4, None),
             ("qwen3-32b-shaped B=8 L=8192 k=64", 5, 8192),
             ("qwen3-32b-shaped B=8 L=16384 k=64", 5, 16384),
             ("qwen3-32b-shaped B=8 L=32768 k=64", 5, 32768),
             ("qwen3-32b-shaped B=8 L=65536 k=64", 5, 65536),
             ("qwen3-8b one-GPU share B=4096 Hq=4 Hkv=1 L=32768 k=64", "share", None)]


# ---------------------------------------------------------------- main

def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=6)
    ap.add_argument("--dense-steps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="skip the HIP-graph replay measurement")
    ap.add_argument("--no-append", dest="append", action="store_false",
                    help="skip the step with the fused KV append")
    ap.add_argument("--no-best-of-n", dest="best_of_n", action="store_false",
                    help="skip the shared-prefix (Best-of-N) selection comparison")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, run plain 1 GiB device copies (counter calibration)")
    ap.add_argument("--no-workloads", dest="workloads", action="store_false",
                    help="skip the other workloads (0.6B, 30B-A3B, 32B sweep)")
    ap.add_argument("--workload-cpu-seconds", type=float, default=3.0,
                    help="host seconds per workload for the oracle (0: skip)")
    ap.add_argument("--only-workload", type=int, default=None,
                    help="time only the other workload with this index (for profiling runs)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import torch

    import block_top_sparse_btk_amd as btk
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only_workload is not None:
        name, cfg, ctx = WORKLOADS[args.only_workload]
        res = measure_workload(name, workload_batch(cfg, ctx, dev)[0], dev, args.steps, 0.0)
        print(json.dumps(res), flush=True)
        return
    bt = synth.make_config(3)
    B, hq, hkv, D, k = bt.batch, bt.num_q_heads, bt.num_kv_heads, bt.head_dim, bt.top_k
    e = 2
    nbytes = algorithmic_bytes(bt.seq_lens.tolist(), hq, hkv, D, k, e)

    # replicas: independent device copies of everything a step reads or writes
    reps = []
    base = bt.to(dev)
    prob = btk.make_problem(base.q, base.k_cache, base.block_table)
    first = (base.seq_lens - 1).to(torch.int32)
    for i in range(args.replicas):
        d = base if i == 0 else bt.to(dev)
        cent = torch.zeros((bt.num_pages, hkv, D), dtype=torch.float32, device=dev)
        btk.btk_centroid_update(d.k_cache, d.block_table, d.seq_lens, cent, problem=prob)
        ws = btk.new_workspace(prob, k, dev)
        sk = btk.new_sketch(prob, dev)
        btk.btk_sketch_update(cent, d.block_table, d.seq_lens, sk, ws, problem=prob)
        reps.append(dict(d=d, cent=cent, ws=ws, sk=sk,
                         idx=torch.empty((B, hkv, k), dtype=torch.int32, device=dev),
                         out=torch.empty_like(d.q), first=first.clone(),
                         kidx=torch.empty((B, hkv, k), dtype=torch.int32, device=dev),
                         kout=torch.empty_like(d.q),
                         cc=torch.zeros((B, hkv), dtype=torch.int32, device=dev)))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    lib = btk._lib()
    hs = stream.cuda_stream

    # Lean dispatch: the C entry points with prebuilt argument tuples, so host
    # overhead stays far below the GPU time of a step (the binding's per-call
    # shape checks were done when the replicas were built).
    def calls(rep):
        d = rep["d"]
        P = ctypes.byref(prob)
        p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        ws, wsn = p(rep["ws"]), rep["ws"].numel()
        return {"step": (P, p(d.q), p(d.k_cache), p(d.v_cache), p(d.block_table),
                         p(d.seq_lens), p(rep["first"]), p(rep["cent"]), k, p(rep["idx"]),
                         p(rep["out"]), None, ws, wsn, hs),
                "sk": (P, p(d.q), p(d.k_cache), p(d.v_cache), p(d.block_table),
                       p(d.seq_lens), p(rep["first"]), p(rep["cent"]), p(rep["sk"]),
                       rep["sk"].numel(), k, p(rep["kidx"]), p(rep["kout"]), None, p(rep["cc"]),
                       ws, wsn, hs),
                "cen": (P, p(d.k_cache), p(d.block_table), p(d.seq_lens), p(rep["first"]),
                        p(rep["cent"]), hs),
                "sel": (P, p(d.q), p(rep["cent"]), p(d.block_table), p(d.seq_lens), k,
                        p(rep["idx"]), None, ws, wsn, hs),
                "att": (P, p(d.q), p(d.k_cache), p(d.v_cache), p(d.block_table), p(d.seq_lens),
                        p(rep["idx"]), k, p(rep["sout"]), None, ws, wsn, hs),
                "den": (P, p(d.q), p(d.k_cache), p(d.v_cache), p(d.block_table), p(d.seq_lens),
                        p(rep["dout"]), None, ws, wsn, hs),
                "loc": (P, p(d.q), p(d.k_cache), p(d.v_cache), p(d.block_table), p(d.seq_lens),
                        k, p(rep["dout"]), None, ws, wsn, hs)}

    for rep in reps:
        rep["dout"] = torch.empty_like(rep["d"].q)
        rep["sout"] = torch.empty_like(rep["d"].q)
        rep["calls"] = calls(rep)
    f_step, f_cen, f_sel, f_att, f_den, f_loc = (lib.btk_decode_step, lib.btk_centroid_update,
                                                 lib.btk_select, lib.btk_sparse_attend,
                                                 lib.btk_dense_attend, lib.btk_local_attend)

    def check(st):
        if st:
            raise RuntimeError(f"library call failed: {lib.btk_status_string(st).decode()}")

    def sep_step(rep):
        c = rep["calls"]
        check(f_cen(*c["cen"]) | f_sel(*c["sel"]) | f_att(*c["att"]))

    # the step through the block sketches first warmed up; results must equal
    # the fp32-scan step's bit for bit (checked on every replica below)
    f_sk = lib.btk_decode_step_sketch
    for i in range(args.warmup):
        check(f_sk(*reps[i % len(reps)]["calls"]["sk"]))
    torch.cuda.synchronize()

    # timed region: exactly K steps (one kernel each), bracketed by synchronize
    # and by one HIP event pair on the library's stream; the launch average is
    # the event time over K, so it counts the gaps between launches too (an
    # event pair around every launch would add its own ~8 us to each step)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        check(f_sk(*reps[i % len(reps)]["calls"]["sk"]))
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / args.steps
    sk_us = 1e3 * ev0.elapsed_time(ev1) / args.steps
    # spread: the same launches in batches of 10, one event pair per batch
    bev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(max(1, args.steps // 10))]
    i = 0
    for e0, e1 in bev:
        e0.record(stream)
        for _ in range(10):
            check(f_sk(*reps[i % len(reps)]["calls"]["sk"]))
            i += 1
        e1.record(stream)
    torch.cuda.synchronize()
    sk_batches = _pcts([1e3 * e0.elapsed_time(e1) / 10 for e0, e1 in bev])

    # the single launch that scans every fp32 centroid row (btk_decode_step):
    # same launches, same event brackets
    for i in range(args.warmup):
        check(f_step(*reps[i % len(reps)]["calls"]["step"]))
        sep_step(reps[i % len(reps)])
    torch.cuda.synchronize()
    sev0, sev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    sev0.record(stream)
    for i in range(args.steps):
        check(f_step(*reps[i % len(reps)]["calls"]["step"]))
    sev1.record(stream)
    torch.cuda.synchronize()
    plain_ms = 1e3 * (time.perf_counter() - t0) / args.steps
    step_us = 1e3 * sev0.elapsed_time(sev1) / args.steps
    i = 0
    for e0, e1 in bev:
        e0.record(stream)
        for _ in range(10):
            check(f_step(*reps[i % len(reps)]["calls"]["step"]))
            i += 1
        e1.record(stream)
    torch.cuda.synchronize()
    step_batches = _pcts([1e3 * e0.elapsed_time(e1) / 10 for e0, e1 in bev])

    # the same step as three calls: whole-step time, then a per-kernel pass
    t0 = time.perf_counter()
    for i in range(args.steps):
        sep_step(reps[i % len(reps)])
    torch.cuda.synchronize()
    sep_ms = 1e3 * (time.perf_counter() - t0) / args.steps
    kev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        c, ev = reps[i % len(reps)]["calls"], kev[i]
        ev[0].record(stream)
        f_cen(*c["cen"])
        ev[1].record(stream)
        f_sel(*c["sel"])
        ev[2].record(stream)
        f_att(*c["att"])
        ev[3].record(stream)
    torch.cuda.synchronize()
    kern = {name: 1e3 * sum(ev[j].elapsed_time(ev[j + 1]) for ev in kev) / args.steps
            for j, name in enumerate(("centroid", "select", "attend"))}

    # the step replayed from HIP graphs (one captured launch per replica)
    graph_ms = None
    if args.graph:
        graphs = []
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for rep in reps:  # capture on a side stream; the call names it explicitly
                c = tuple(x if x is not hs else side.cuda_stream for x in rep["calls"]["sk"])
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    check(f_sk(*c))
                graphs.append(g)
        stream.wait_stream(side)
        for i in range(args.warmup):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        graph_ms = 1e3 * (time.perf_counter() - t0) / args.steps

    # dense comparison on the same inputs
    for i in range(3):
        check(f_den(*reps[i % len(reps)]["calls"]["den"]))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.dense_steps):
        check(f_den(*reps[i % len(reps)]["calls"]["den"]))
    torch.cuda.synchronize()
    dense_ms = 1e3 * (time.perf_counter() - t0) / args.dense_steps

    # local-window baseline (the most recent top_k blocks), same inputs
    for i in range(args.warmup):
        check(f_loc(*reps[i % len(reps)]["calls"]["loc"]))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        check(f_loc(*reps[i % len(reps)]["calls"]["loc"]))
    torch.cuda.synchronize()
    local_ms = 1e3 * (time.perf_counter() - t0) / args.steps

    # token-level baseline (budget 16 * top_k tokens), same inputs, one workspace
    tws = btk.new_token_workspace(prob, 16 * k, dev)
    P_ = ctypes.byref(prob)
    pp = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    tok_calls = [(P_, pp(r["d"].q), pp(r["d"].k_cache), pp(r["d"].v_cache), pp(r["d"].block_table),
                  pp(r["d"].seq_lens), 16 * k, None, pp(r["dout"]), None, pp(tws), tws.numel(), hs)
                 for r in reps]
    f_tok = lib.btk_token_topk_attend
    for i in range(3):
        check(f_tok(*tok_calls[i % len(reps)]))
    torch.cuda.synchronize()
    tok_steps = max(1, args.steps // 4)
    t0 = time.perf_counter()
    for i in range(tok_steps):
        check(f_tok(*tok_calls[i % len(reps)]))
    torch.cuda.synchronize()
    token_ms = 1e3 * (time.perf_counter() - t0) / tok_steps
    if btk.workspace_error_bits(tws):
        raise RuntimeError("device-side input guard fired during the token-level baseline")
    for r in reps:
        if btk.workspace_error_bits(r["ws"]):
            raise RuntimeError("device-side input guard fired during the benchmark")
    for r in reps:  # the three forms of the step agree
        if not torch.equal(r["out"], r["sout"]):
            raise RuntimeError("single-launch and three-call steps disagree")
        if not (torch.equal(r["out"], r["kout"]) and torch.equal(r["idx"], r["kidx"])):
            raise RuntimeError("the step and the sketched step disagree")

    # Best-of-N: the Qwen3-30B-A3B-shaped batch (16 samples sharing a 2048-token
    # prompt), select vs the shared-prefix select that reads the prompt's centroid
    # rows once per KV head (identical results)
    bon = None
    if args.best_of_n:
        b4 = synth.make_config(4)
        prefix = b4.notes.get("shared_prefix", 2048) // 16
        k4 = b4.top_k
        # six replicas (about 400 MB of centroid rows) so that cycling through
        # them misses the 256 MB last-level cache: "cold"; replica 0 alone: "warm"
        r4 = []
        for i in range(6):
            d4 = b4.to(dev)
            p4 = btk.make_problem(d4.q, d4.k_cache, d4.block_table)
            c4 = torch.zeros((b4.num_pages, b4.num_kv_heads, b4.head_dim), device=dev)
            btk.btk_centroid_update(d4.k_cache, d4.block_table, d4.seq_lens, c4, problem=p4)
            w4 = btk.new_workspace(p4, k4, dev)
            i4 = torch.empty((b4.batch, b4.num_kv_heads, k4), dtype=torch.int32, device=dev)
            j4 = torch.empty_like(i4)
            r4.append((d4, p4, c4, w4, i4, j4))

        def run_sel(r):
            d4, p4, c4, w4, i4, _ = r
            btk.btk_select(d4.q, c4, d4.block_table, d4.seq_lens, k4, w4, indices=i4, problem=p4)

        def run_shr(r):
            d4, p4, c4, w4, _, j4 = r
            btk.btk_select_shared(d4.q, c4, d4.block_table, d4.seq_lens, [0, b4.batch], [prefix],
                                  k4, w4, indices=j4, problem=p4)

        # each kernel is about as short as the host's time to issue it, so a host
        # stall would land in a plain loop's time: the calls are captured in a
        # HIP graph (24 back to back) and the median of 10 timed replays is kept
        def graph_us(fn, rs):
            for r in rs:
                fn(r)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(24):
                    fn(rs[i % len(rs)])
            g.replay()
            torch.cuda.synchronize()
            reps_us = []
            for _ in range(10):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                reps_us.append(1e3 * e0.elapsed_time(e1) / 24)
            return sorted(reps_us)[len(reps_us) // 2]

        times = {"select_cold": graph_us(run_sel, r4), "select_shared_cold": graph_us(run_shr, r4),
                 "select_warm": graph_us(run_sel, r4[:1]),
                 "select_shared_warm": graph_us(run_shr, r4[:1])}
        for _, _, _, w4, i4, j4 in r4:
            if not torch.equal(i4, j4) or btk.workspace_error_bits(w4):
                raise RuntimeError("shared-prefix selection disagrees with select")
        sel4 = algorithmic_bytes(b4.seq_lens.tolist(), b4.num_q_heads, b4.num_kv_heads,
                                 b4.head_dim, b4.top_k, 2)["select"]
        saved = (b4.batch - 1) * b4.num_kv_heads * prefix * 4 * b4.head_dim
        bon = {"workload": "qwen3-30b-a3b-shaped Best-of-N: B=16 samples sharing a 2048-token "
                           "prompt + 30720 private tokens, Hq=32, Hkv=4, D=128, bf16, top_k=64",
               "select_us": round(times["select_cold"], 2),
               "select_shared_us": round(times["select_shared_cold"], 2),
               "select_warm_us": round(times["select_warm"], 2),
               "select_shared_warm_us": round(times["select_shared_warm"], 2),
               "select_bytes": sel4, "select_shared_bytes": sel4 - saved,
               "note": "cold: six replicas in turn (about 400 MB of centroid rows, more than the "
                       "256 MB last-level cache); warm: one replica; identical indices; median "
                       "of 10 replays of a HIP graph of 24 calls"}
        del r4

    # the step with the KV append fused in (btk_decode_step_append): the appended
    # key and value are each sequence's newest token as drawn, so every replica's
    # caches stay as they are and the results must equal the step's bit for bit
    app = None
    if args.append:
        Ll = bt.seq_lens.long()
        pg = bt.block_table[torch.arange(B), (Ll - 1) // 16].long()[:, None]
        sl = ((Ll - 1) % 16)[:, None]
        hh = torch.arange(hkv)[None, :]
        k_new = bt.k_cache[pg, hh, sl, :].contiguous().to(dev)
        v_new = bt.v_cache[pg, hh, :, sl].contiguous().to(dev)
        f_app = lib.btk_decode_step_append
        p_ = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        for rep in reps:
            rep["aidx"] = torch.empty_like(rep["idx"])
            rep["aout"] = torch.empty_like(rep["out"])
            d = rep["d"]
            rep["app"] = (ctypes.byref(prob), p_(d.q), p_(k_new), p_(v_new), p_(d.k_cache),
                          p_(d.v_cache), p_(d.block_table), p_(d.seq_lens), p_(rep["cent"]), k,
                          p_(rep["aidx"]), p_(rep["aout"]), None, p_(rep["ws"]),
                          rep["ws"].numel(), hs)
        for i in range(args.warmup):
            check(f_app(*reps[i % len(reps)]["app"]))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            check(f_app(*reps[i % len(reps)]["app"]))
        torch.cuda.synchronize()
        app_ms = 1e3 * (time.perf_counter() - t0) / args.steps
        for rep in reps:
            if not (torch.equal(rep["aidx"], rep["idx"]) and torch.equal(rep["aout"], rep["out"])):
                raise RuntimeError("the step with the fused append disagrees with the step")
        # the same append as two PyTorch index writes, then the single-launch step
        pgd, sld, hhd = pg.to(dev), sl.to(dev), hh.to(dev)
        def torch_append_step(rep):
            rep["d"].k_cache[pgd, hhd, sld, :] = k_new
            rep["d"].v_cache[pgd, hhd, :, sld] = v_new
            check(f_step(*rep["calls"]["step"]))
        for i in range(args.warmup):
            torch_append_step(reps[i % len(reps)])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            torch_append_step(reps[i % len(reps)])
        torch.cuda.synchronize()
        sep_app_ms = 1e3 * (time.perf_counter() - t0) / args.steps
        app = (app_ms, sep_app_ms)

    if args.copy_probe:
        # counter calibration: a 1 GiB device copy (3 dispatches), then the
        # library's row-read probe with the centroid scan's request shape, over
        # 1 GiB in order (3 dispatches) and over 2^21 distinct random rows of a
        # 4 GiB buffer (3 dispatches, a new permutation each)
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del dst
        for _ in range(3):
            btk.btk_probe_row_read(src)
        torch.cuda.synchronize()
        del src
        big = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(7)
        for _ in range(3):
            ids = torch.randperm(big.numel() // 512, device=dev, generator=gen)[:1 << 21]
            ids = ids.to(torch.int32)
            torch.cuda.synchronize()
            btk.btk_probe_row_read(big, row_ids=ids)
            torch.cuda.synchronize()
        del big

    # exact S4 bytes from the blocks actually selected (every replica selects the same)
    nbytes = algorithmic_bytes(bt.seq_lens.tolist(), hq, hkv, D, k, e,
                               sel_tokens=selected_tokens(reps[0]["idx"].cpu(), bt.seq_lens))
    value = B / (ms_per_step * 1e-3)
    dense_gbps = nbytes["dense"] / (dense_ms * 1e-3) / 1e9
    sel_toks = selected_tokens(reps[0]["idx"].cpu(), bt.seq_lens)
    cc = reps[0]["cc"].cpu()
    # the headline kernel's own algorithmic bytes: sketch rows, the candidates'
    # fp32 centroid rows, the rest as the fp32-scan step
    if not _sketch_takes_unit_kernel(B, hkv, bt.block_table.shape[1], dev):
        raise RuntimeError("the headline layer's units do not fill this device: the roofline "
                           "below is for decode_step_unit_kernel")
    sk_bytes = sketch_step_bytes(bt.seq_lens.tolist(), hq, hkv, D, k, e, cc.tolist(), sel_toks)
    sk_step_gbps = sk_bytes / (ms_per_step * 1e-3) / 1e9
    sk_gbps = sk_bytes / (sk_us * 1e-6) / 1e9
    plain_gbps = nbytes["step"] / (step_us * 1e-6) / 1e9
    fp32_scan = {"kernel": "decode_step_kernel (persistent, every fp32 centroid row scanned): "
                           "btk_decode_step",
                 "ms_per_step": round(plain_ms, 5), "value": round(B / (plain_ms * 1e-3), 1),
                 "unit": "query-tokens/s", "avg_launch_us": round(step_us, 3),
                 "launch_us_batches": step_batches,
                 "algorithmic_bytes_per_launch": nbytes["step"],
                 "achieved": round(plain_gbps, 1), "frac": round(plain_gbps / HBM_PEAK_GBPS, 4),
                 "traffic": _measured_traffic(PLAIN_TRAFFIC_FILE),
                 "bytes_per_token": round(nbytes["step"] / B, 1),
                 "speedup_vs_dense": round(1e3 * dense_ms / step_us, 2),
                 "method_bytes_rate_of_headline": {
                     "gbps": round(nbytes["step"] / (sk_us * 1e-6) / 1e9, 1),
                     "note": "the bytes this fp32-scan step must move, over the headline "
                             "kernel's launch time: the rate at which the sketched kernel does "
                             "the fp32-scan step's work (it reads fewer bytes, so this is not a "
                             "bandwidth it sustains)"}}
    if app is not None:
        app_bytes = nbytes["step"] + 4 * B * hkv * D * e  # new K,V read and written
        app = {"ms_per_step": round(app[0], 5), "value": round(B / (app[0] * 1e-3), 1),
               "bytes_per_step": app_bytes, "gbps": round(app_bytes / (app[0] * 1e-3) / 1e9, 1),
               "torch_append_then_step_ms": round(app[1], 5),
               "note": "btk_decode_step_append: the newest token's key and value written into "
                       "the caches inside the same launch; results identical to the step; "
                       "torch_append_then_step_ms: the same append as two PyTorch index "
                       "writes followed by btk_decode_step"}
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded Qwen3-8B-shaped decode batch (no dataset or weights)",
        "config": {"workload": WORKLOAD, "batch": B, "num_q_heads": hq, "num_kv_heads": hkv,
                   "head_dim": D, "page_size": 16, "top_k": k, "seed": bt.seed,
                   "mean_context": round(float(bt.seq_lens.float().mean()), 1),
                   "replicas": args.replicas},
        "step_gbps": round(sk_step_gbps, 1),
        "step_frac_of_peak": round(sk_step_gbps / HBM_PEAK_GBPS, 4),
        "bytes_per_step": sk_bytes,
        "bytes_per_token": round(sk_bytes / B, 1),
        "roofline": {"bound": "hbm",
                     "kernel": "decode_step_unit_kernel (S1 + S2 + S3 + S4 in one launch, "
                               "through the block sketches, one workgroup per unit)",
                     "achieved": round(sk_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(sk_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": _measured_traffic(),
                     "algorithmic_bytes_per_launch": sk_bytes,
                     "avg_launch_us": round(sk_us, 3),
                     "launch_us_batches": sk_batches,
                     "candidates_per_unit": {"mean": round(float(cc.float().mean()), 1),
                                             "max": int(cc.max())}},
        "fp32_scan_step": fp32_scan,
        "three_calls": {"ms_per_step": round(sep_ms, 5),
                        "value": round(B / (sep_ms * 1e-3), 1),
                        "kernels_us": {kk: round(v, 2) for kk, v in kern.items()},
                        "algorithmic_bytes": {kk: nbytes[kk]
                                              for kk in ("centroid", "select", "attend")}},
        "dense": {"value": round(B / (dense_ms * 1e-3), 1), "unit": "query-tokens/s",
                  "ms_per_step": round(dense_ms, 4), "gbps": round(dense_gbps, 1),
                  "frac_of_peak": round(dense_gbps / HBM_PEAK_GBPS, 4),
                  "bytes_per_step": nbytes["dense"],
                  "bytes_per_token": round(nbytes["dense"] / B, 1)},
        "speedup_vs_dense": round(dense_ms / ms_per_step, 2),
        "local_window": {"window_blocks": k, "value": round(B / (local_ms * 1e-3), 1),
                         "unit": "query-tokens/s", "ms_per_step": round(local_ms, 5),
                         "gbps": round(nbytes["local"] / (local_ms * 1e-3) / 1e9, 1),
                         "frac_of_peak": round(nbytes["local"] / (local_ms * 1e-3) / 1e9
                                               / HBM_PEAK_GBPS, 4),
                         "bytes_per_step": nbytes["local"]},
        "token_topk": {"top_tokens": 16 * k, "value": round(B / (token_ms * 1e-3), 1),
                       "unit": "query-tokens/s", "ms_per_step": round(token_ms, 5),
                       "gbps": round(nbytes["token"] / (token_ms * 1e-3) / 1e9, 1),
                       "frac_of_peak": round(nbytes["token"] / (token_ms * 1e-3) / 1e9
                                             / HBM_PEAK_GBPS, 4),
                       "bytes_per_step": nbytes["token"]},
        "best_of_n": bon,
        "fused_append": app,
        "graph_replay": None if graph_ms is None else {
            "ms_per_step": round(graph_ms, 5), "value": round(B / (graph_ms * 1e-3), 1),
            "step_gbps": round(sk_bytes / (graph_ms * 1e-3) / 1e9, 1)},
    }
    if args.workloads:
        # the other workloads (each a full line of its own numbers)
        del reps
        torch.cuda.empty_cache()
        result["workloads"] = []
        for name, cfg, ctx in WORKLOADS:
            wb, sample = workload_batch(cfg, ctx, dev)
            result["workloads"].append(
                measure_workload(name, wb, dev, max(50, args.steps // 2),
                                 0.0 if args.no_cpu_baseline else args.workload_cpu_seconds,
                                 cpu_sample=sample))
            del wb, sample
            torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = _cpu_baseline(bt, args.cpu_seconds)
        result["cpu_baseline"]["cpu_model"] = _cpu_model()
        one = _oracle_rates(bt, 2.0)["one_thread"]  # one sequence at a time on one thread
        result["cpu_baseline"]["one_thread"] = one
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
