"""Benchmark of the paged-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config chunked_prefill_mix]
                    [--iters 50] [--warm-calls 10] [--no-configs] [--no-extra] [--no-cpu]

A step is one pass of the whole path over one synthetic batch: metadata
build, cache write of the step's new K/V, decode attention of the 1-token
requests, varlen prefill attention of the rest (whichever the batch has).
The headline workload is the 8192-token chunked-prefill mix (6 prefill chunks
of 512..2048 new tokens after 0..4096 cached ones, 862 one-token decodes with
256..8192 cached; 32 query / 8 K/V heads, head_dim 128, bf16, 16-token
blocks): the largest of the five measured workloads and the only one that
carries both halves of the metric.  ``value`` is its decode KV GB/s over the
whole step: every K/V byte each decode request must read (seq_len * Hkv * D *
2 * bytes, counted once per request) divided by the step's wall time, inputs
resident in HBM.

Also on the same JSON line:
* ``roofline``: the dominant kernel of the step (the decode call: split
  kernel and its reduce) against the HBM peak, timed live with HIP events on
  the launch stream over the timed steps; ``roofline_prefill``: the prefill
  kernel against the bf16 MFMA peak, timed the same way;
* ``cpu_baseline``: the oracle (plain NumPy float64) on the host cores over
  a bounded sample of the same batch's decodes, in the same unit;
* ``configs``: each of the five workloads (the tour's 3-request step, the
  MHA, GQA and long-context fp8 MQA decode batches, the mixed batch): every
  call of its step timed alone (median, p10, p90 of ``--iters`` runs after
  ``--warm-calls`` warm-ups, each run after a 1 GiB read that evicts L2 and
  the 256 MB last-level cache), a roofline object per attention call, and the
  oracle's time on a bounded sample of that workload;
* ``extra``: the GQA, mixed and long MQA shapes over an int8 cache, the fused
  RoPE + cache write, 1024-key sliding window + ALiBi attention, block copy /
  swap on the GQA pool, and a plain device-to-device copy as the context
  figure for HBM bandwidth.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from paged_kv_cache_hkv_amd import binding as B  # noqa: E402
from paged_kv_cache_hkv_amd import synth as S  # noqa: E402
from paged_kv_cache_hkv_amd.step import PagedAttentionStep  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA
CSRC = os.path.join(ROOT, "paged_kv_cache_hkv_amd", "csrc")
KERNEL_SRC = {"decode": os.path.join(CSRC, "pa_decode.hip"),
              "prefill": os.path.join(CSRC, "pa_prefill.hip")}
METRIC = "paged decode attn achieved KV GB/s (% HBM peak) + prefill query tok/s (% MFMA)"


# ------------------------------------------------------------ work counts --

def kv_bytes(wl, reqs):
    """Algorithmic KV bytes of decode requests: every K/V element once per request."""
    e = wl.cache_elem_bytes
    s = wl.seq_lens_host[list(reqs)].astype(np.int64)
    return int(s.sum()) * wl.num_kv_heads * wl.head_dim * 2 * e


def prefill_flops(wl, reqs):
    """Algorithmic prefill flops: QK and PV over the causal pairs only."""
    tot = 0
    for r in reqs:
        n = int(wl.query_lens[r])
        c = int(wl.num_computed[r])
        tot += 4 * wl.num_q_heads * wl.head_dim * (n * c + n * (n + 1) // 2)
    return tot


def window_kv_bytes(wl, reqs, window):
    """KV bytes a decode must read under a sliding window: the last min(s, W) keys."""
    e = wl.cache_elem_bytes
    s = np.minimum(wl.seq_lens_host[list(reqs)].astype(np.int64), window)
    return int(s.sum()) * wl.num_kv_heads * wl.head_dim * 2 * e


def window_prefill_flops(wl, reqs, window):
    """Prefill flops over the pairs a sliding window leaves: query at position p
    sees min(p + 1, W) keys."""
    tot = 0
    for r in reqs:
        n, c = int(wl.query_lens[r]), int(wl.num_computed[r])
        seen = np.minimum(np.arange(c, c + n, dtype=np.int64) + 1, window)
        tot += 4 * wl.num_q_heads * wl.head_dim * int(seen.sum())
    return tot


def write_bytes(wl):
    """Algorithmic bytes of the cache write: new K/V rows read, cache rows written."""
    T = wl.num_tokens
    row = wl.num_kv_heads * wl.head_dim
    return 2 * T * row * 2 + 2 * T * row * wl.cache_elem_bytes


def rope_table(max_position, rotary_dim, base, device):
    """float32 [max_position, rotary_dim]: cos(p*f_j) then sin(p*f_j), f_j = base^(-2j/R),
    angles in float64 (the caller-built table the fused call takes)."""
    j = np.arange(rotary_dim // 2, dtype=np.float64)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * base ** (-2.0 * j / rotary_dim)
    tab = np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)
    return torch.from_numpy(tab).to(device)


def rope_bytes(wl, rotary_dim):
    """Algorithmic bytes of one fused RoPE + cache write over the batch's real tokens:
    q rotated part read and written, k and v read, k and v cache rows written, the
    token's cos/sin row, its position and slot."""
    T, hq, hkv, d = wl.num_tokens, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    e = wl.cache_elem_bytes
    per = 2 * hq * rotary_dim * 2 + 2 * hkv * d * 2 + 2 * hkv * d * e + rotary_dim * 4 + 16
    return T * per


# ---------------------------------------------------------------- rooflines --

def src_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(workload, kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, if still current."""
    path = os.path.join(ROOT, "profiles", f"{workload}_{kernel}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_src_sha") != src_sha(KERNEL_SRC[kernel]):
        return None
    return rec.get("hbm_bytes_per_launch")


def roofline_hbm(nbytes, ms, workload, kernel_name):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": read_traffic(workload, "decode"),
            "kernel": kernel_name, "kernel_ms": round(ms, 4), "algorithmic_bytes": nbytes}


def roofline_mfma(flops, ms, workload, kernel_name):
    tf = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "traffic": read_traffic(workload, "prefill"), "kernel": kernel_name,
            "kernel_ms": round(ms, 4), "algorithmic_flops": flops}


DECODE_KERNEL = "pa_decode (decode_kernel + decode_reduce_kernel)"
PREFILL_KERNEL = "pa_prefill_varlen (prefill_pp_kernel)"


# ------------------------------------------------------------------ timing --

def time_calls(fn_list, iters, warm, flush):
    """Median / p10 / p90 milliseconds of each callable, HIP events on the current
    stream, each run after a cache-evicting read (reads only, so no dirty lines
    are left to write back inside the timed call)."""
    stream = torch.cuda.current_stream()
    for _ in range(warm):
        for fn in fn_list:
            fn()
    res = [[] for _ in fn_list]
    for _ in range(iters):
        for i, fn in enumerate(fn_list):
            flush.sum()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            res[i].append((a, b))
    torch.cuda.synchronize()
    out = []
    for pairs in res:
        ms = np.array([a.elapsed_time(b) for a, b in pairs])
        out.append((float(np.median(ms)), float(np.percentile(ms, 10)),
                    float(np.percentile(ms, 90))))
    return out


def put_times(rec, names, times):
    for nm, (med, p10, p90) in zip(names, times):
        rec[f"{nm}_ms"] = round(med, 4)
        rec[f"{nm}_ms_p10_p90"] = [round(p10, 4), round(p90, 4)]


# ---------------------------------------------------------- oracle timing --

def host_threads():
    return len(os.sched_getaffinity(0))


def take_snapshot(wl, t, requests):
    """Host copy of the requests' blocks as drawn, before any kernel writes the pool."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from harness import Snapshot   # test infrastructure
    return Snapshot(wl, t, requests)


def decode_sample(wl, budget_units=400000):
    """Decode requests from the start of the batch up to a bounded number of
    (block, K/V head) units (the host snapshot they need stays a few GB)."""
    out, tot = [], 0
    for r in range(wl.num_decodes):
        nb = -(-int(wl.seq_lens_host[r]) // wl.block_size) * wl.num_kv_heads
        if out and tot + nb > budget_units:
            break
        out.append(r)
        tot += nb
    return out


def cpu_baseline(wl, t, snap, decodes, prefills, budget_s=12.0):
    """The oracle as it stands, on the host cores (BLAS threads = the cores this
    process may run on), over the sampled requests in order until the budget is
    spent: decode KV GB/s and prefill query tok/s.  The snapshot (D2H copy) is
    taken beforehand and not timed."""
    from harness import OraclePrep   # test infrastructure: the oracle
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=host_threads())
    except ImportError:   # BLAS then runs with its own default thread count
        limiter = None
    try:
        t0 = time.perf_counter()
        prep = OraclePrep(wl, t, snap)
        setup = time.perf_counter() - t0
        res = {}
        done, spent = [], 0.0
        for r in decodes:
            if spent >= budget_s:
                break
            t0 = time.perf_counter()
            prep.rows([r])
            spent += time.perf_counter() - t0
            done.append(r)
        if done:
            kb = kv_bytes(wl, done)
            res["decode"] = {"value": round(kb / spent / 1e9, 4), "unit": "GB/s",
                             "cores": host_threads(), "kind": "oracle",
                             "sample": f"first {len(done)} of {wl.num_decodes} decode requests of "
                                       f"{wl.name} ({kb} KV bytes, {spent:.1f} s, NumPy float64, "
                                       f"oracle scatter and setup {setup:.1f} s not counted)"}
        done_p, spent_p = [], 0.0
        for r in prefills:
            if spent_p >= budget_s:
                break
            t0 = time.perf_counter()
            prep.rows([r])
            spent_p += time.perf_counter() - t0
            done_p.append(r)
        if done_p:
            toks = int(sum(int(wl.query_lens[r]) for r in done_p))
            fl = prefill_flops(wl, done_p)
            res["prefill"] = {"value": round(toks / spent_p, 1), "unit": "query tok/s",
                              "cores": host_threads(), "kind": "oracle",
                              "gflops": round(fl / spent_p / 1e9, 2),
                              "sample": f"{len(done_p)} of {wl.num_reqs - wl.num_decodes} prefill "
                                        f"chunks of {wl.name}, fewest causal pairs first ({toks} "
                                        f"query tokens, {spent_p:.1f} s, NumPy float64)"}
        return res
    finally:
        if limiter is not None:
            limiter.unregister()


# --------------------------------------------------------------- workloads --

def attention_calls(wl, st):
    fns, names = [], []
    if wl.num_decodes:
        fns.append(st.decode)
        names.append("decode")
    if wl.num_reqs > wl.num_decodes:
        fns.append(st.prefill)
        names.append("prefill")
    return fns, names


def add_rooflines(rec, wl, prefix=""):
    if wl.num_decodes:
        kb = kv_bytes(wl, range(wl.num_decodes))
        rec[prefix + "roofline_decode"] = roofline_hbm(kb, rec[prefix + "decode_ms"], wl.name,
                                                       DECODE_KERNEL)
    if wl.num_reqs > wl.num_decodes:
        pre = range(wl.num_decodes, wl.num_reqs)
        fl = prefill_flops(wl, pre)
        toks = int(wl.query_lens[wl.num_decodes:].sum())
        rec[prefix + "roofline_prefill"] = roofline_mfma(fl, rec[prefix + "prefill_ms"], wl.name,
                                                         PREFILL_KERNEL)
        rec[prefix + "prefill_tok_per_s"] = round(toks / (rec[prefix + "prefill_ms"] * 1e-3), 1)


def bench_config(wl, t, args, flush, snap=None, cpu_req=None, cpu_budget=6.0):
    """Every call of the workload's step timed alone, with rooflines and the
    oracle's time on a bounded sample."""
    st = PagedAttentionStep(wl, t)
    st.run()
    torch.cuda.synchronize()
    rec = {"workload": wl.name, "cache": wl.cache_kind, "requests": wl.num_reqs,
           "decodes": wl.num_decodes, "tokens": wl.num_tokens,
           "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
           "head_dim": wl.head_dim}
    fns, names = attention_calls(wl, st)
    fns += [st.metadata, st.cache_write]
    names += ["metadata", "cache_write"]
    put_times(rec, names, time_calls(fns, args.iters, args.warm_calls, flush))
    add_rooflines(rec, wl)
    wb = write_bytes(wl)
    rec["cache_write_bytes"] = wb
    rec["cache_write_GBps"] = round(wb / (rec["cache_write_ms"] * 1e-3) / 1e9, 1)
    if wl.num_decodes:
        rec["decode_kv_bytes"] = kv_bytes(wl, range(wl.num_decodes))
    if snap is not None:
        rec["cpu_baseline"] = cpu_baseline(wl, t, snap, *cpu_req, budget_s=cpu_budget)
    del st
    return rec


def cpu_sample(wl, budget_units=400000):
    """Requests the oracle is timed on: decodes from the start of the batch and,
    for mixed batches, every prefill chunk, fewest causal pairs first (the
    timing loop stops when its budget is spent)."""
    dec = decode_sample(wl, budget_units)
    pre = sorted(range(wl.num_decodes, wl.num_reqs), key=lambda r: prefill_flops(wl, [r]))
    return dec, pre


def bench_masks(wl, t, args, flush, window=1024):
    """Decode / prefill with a sliding window and ALiBi slopes on the same batch."""
    h = wl.num_q_heads
    sl = torch.tensor([2.0 ** (-8.0 * (i + 1) / h) for i in range(h)], dtype=torch.float32,
                      device="cuda")
    st = PagedAttentionStep(wl, t, sliding_window=window, alibi_slopes=sl)
    st.metadata()
    fns, names = attention_calls(wl, st)
    rec = {"workload": wl.name, "sliding_window": window, "alibi": True}
    put_times(rec, names, time_calls(fns, args.iters, args.warm_calls, flush))
    if wl.num_decodes:
        kb = window_kv_bytes(wl, range(wl.num_decodes), window)
        rec["roofline_decode"] = roofline_hbm(kb, rec["decode_ms"], wl.name + "_window",
                                              DECODE_KERNEL + ", window + ALiBi")
        rec["roofline_decode"]["traffic"] = None
    if wl.num_reqs > wl.num_decodes:
        fl = window_prefill_flops(wl, range(wl.num_decodes, wl.num_reqs), window)
        rec["roofline_prefill"] = roofline_mfma(fl, rec["prefill_ms"], wl.name + "_window",
                                                PREFILL_KERNEL + ", window + ALiBi")
        rec["roofline_prefill"]["traffic"] = None
    del st
    return rec


def bench_rope(wl, t, args, flush):
    st = PagedAttentionStep(wl, t)
    st.metadata()
    table = rope_table(wl.max_seq_len, wl.head_dim, 10000.0, "cuda")
    rec = {"workload": wl.name, "rotary_dim": wl.head_dim}
    put_times(rec, ["rope_cache_write"],
              time_calls([lambda: st.rope_cache_write(table, wl.head_dim, True)], args.iters,
                         args.warm_calls, flush))
    rb = rope_bytes(wl, wl.head_dim)
    rec["rope_cache_write_bytes"] = rb
    gbs = rb / (rec["rope_cache_write_ms"] * 1e-3) / 1e9
    rec["rope_cache_write_GBps"] = round(gbs, 1)
    rec["rope_cache_write_hbm_frac"] = round(gbs / HBM_PEAK_GBS, 4)
    del st
    return rec


def bench_blocks(wl, t, desc, args, flush, n_pairs=4096):
    """pa_copy_blocks on the workload's pool: n_pairs blocks copied inside the
    device pool, swapped out to a pinned host pool and swapped back in; beside
    them, torch's contiguous copy of the same bytes between pinned host memory
    and the device (the host link's rate for one large transfer)."""
    nb = t.key_cache.shape[0]
    rng = np.random.default_rng(11)
    perm = rng.permutation(nb)
    blk = t.key_cache[0].numel() * t.key_cache.element_size()
    shape = (n_pairs,) + tuple(t.key_cache.shape[1:])
    host_k = torch.empty(shape, dtype=t.key_cache.dtype, pin_memory=True)
    host_v = torch.empty(shape, dtype=t.value_cache.dtype, pin_memory=True)
    dev_buf = torch.empty(shape, dtype=t.key_cache.dtype, device="cuda")
    host_ids = np.arange(n_pairs)
    copy_pairs = torch.from_numpy(np.stack([perm[:n_pairs], perm[n_pairs:2 * n_pairs]], 1)).cuda()
    out_pairs = torch.from_numpy(np.stack([perm[:n_pairs], host_ids], 1)).cuda()
    in_pairs = torch.from_numpy(np.stack([host_ids, perm[2 * n_pairs:3 * n_pairs]], 1)).cuda()
    kc, vc = t.key_cache, t.value_cache
    fns = [
        lambda: B.pa_copy_blocks(desc, kc, vc, kc, vc, copy_pairs),
        lambda: B.pa_copy_blocks(desc, kc, vc, host_k, host_v, out_pairs),
        lambda: B.pa_copy_blocks(desc, host_k, host_v, kc, vc, in_pairs),
        lambda: host_k.copy_(dev_buf, non_blocking=True),
        lambda: dev_buf.copy_(host_k, non_blocking=True),
    ]
    times = time_calls(fns, max(10, args.iters // 5), 3, flush)
    moved = 2 * n_pairs * blk                       # K and V blocks
    rec = {"workload": wl.name, "pairs": n_pairs, "block_bytes": blk, "bytes_per_call": moved}
    for nm, (med, p10, p90), nbytes in zip(
            ["copy", "swap_out", "swap_in", "torch_d2h_contiguous", "torch_h2d_contiguous"], times,
            [moved, moved, moved, n_pairs * blk, n_pairs * blk]):
        rec[f"{nm}_ms"] = round(med, 4)
        rec[f"{nm}_ms_p10_p90"] = [round(p10, 4), round(p90, 4)]
        rec[f"{nm}_GBps"] = round(nbytes / (med * 1e-3) / 1e9, 1)
    # the device copy reads and writes every byte in HBM
    rec["copy_hbm_frac"] = round(2 * moved / (rec["copy_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    del host_k, host_v, dev_buf
    return rec


def bench_d2d_copy(args, flush, nbytes=1 << 30):
    """torch's device-to-device copy of 1 GiB: HBM bytes read + written per second."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    rec = {"bytes": nbytes}
    put_times(rec, ["copy"], time_calls([lambda: dst.copy_(src)], args.iters, args.warm_calls,
                                        flush))
    gbs = 2 * nbytes / (rec["copy_ms"] * 1e-3) / 1e9
    rec["read_plus_write_GBps"] = round(gbs, 1)
    rec["hbm_frac"] = round(gbs / HBM_PEAK_GBS, 4)
    del src, dst
    return rec


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# -------------------------------------------------------------------- main --

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="chunked_prefill_mix")
    ap.add_argument("--cache", choices=["act", "fp8_e4m3", "int8"], default=None,
                    help="run the headline workload over this cache format instead of its own")
    ap.add_argument("--iters", type=int, default=50, help="timed runs per call in configs/extra")
    ap.add_argument("--warm-calls", type=int, default=10, help="untimed runs per call first")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the headline cpu_baseline")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--fused-rope", action="store_true",
                    help="each step rotates q and k by position in the cache-write launch "
                         "(pa_rope_cache_write, rotary_dim = head_dim) instead of pa_cache_write")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="first run a plain device-to-device copy of this many bytes three times "
                         "(the known-size kernel that calibrates rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(each GPU would run the same kernels on its own share of requests or heads)",
              file=sys.stderr)
        sys.exit(2)
    B.load()
    torch.cuda.init()
    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes // 16, 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- headline: the whole step, K timed steps ----
    wl = S.CONFIGS[args.config]()
    if args.cache is not None:
        wl = S.with_cache(wl, args.cache)
    t = S.make_tensors(wl, "cuda", poison=False)
    cpu_req = cpu_sample(wl, budget_units=1000000)
    snap = None if args.no_cpu else take_snapshot(wl, t, cpu_req[0] + cpu_req[1])
    st = PagedAttentionStep(wl, t)
    stream = torch.cuda.current_stream()
    if args.fused_rope:
        table = rope_table(wl.max_seq_len, wl.head_dim, 10000.0, "cuda")
        write = lambda: st.rope_cache_write(table, wl.head_dim, True)
    else:
        write = st.cache_write
    for _ in range(args.warmup):
        st.metadata()
        write()
        st.attention()
    torch.cuda.synchronize()

    ev_d, ev_p = [], []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        st.metadata()
        write()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        c = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        st.decode()
        b.record(stream)
        st.prefill()
        c.record(stream)
        ev_d.append((a, b))
        ev_p.append((b, c))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    nd = wl.num_decodes
    kb = kv_bytes(wl, range(nd))
    value = kb / (ms_step * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if wl.act_dtype == torch.float16 else "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "requests": wl.num_reqs, "decodes": nd,
                   "prefill_chunks": wl.num_reqs - nd, "tokens": wl.num_tokens,
                   "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "block_size": wl.block_size,
                   "pool_blocks": wl.pool_blocks, "kv_bytes_per_step": kb,
                   "step": ("metadata + rope_cache_write" if args.fused_rope else
                            "metadata + cache_write") + " + decode + prefill",
                   "parallelism": "single GPU"},
    }
    if nd:
        dec_ms = float(np.mean([x.elapsed_time(y) for x, y in ev_d]))
        line["roofline"] = roofline_hbm(kb, dec_ms, wl.name, DECODE_KERNEL)
    if wl.num_reqs > nd:
        pre_ms = float(np.mean([x.elapsed_time(y) for x, y in ev_p]))
        pre = range(nd, wl.num_reqs)
        line["roofline_prefill"] = roofline_mfma(prefill_flops(wl, pre), pre_ms, wl.name,
                                                 PREFILL_KERNEL)
        toks = int(wl.query_lens[nd:].sum())
        line["prefill_tok_per_s"] = round(toks / (pre_ms * 1e-3), 1)
        line["prefill_tokens_per_step"] = toks
    if "roofline" not in line:
        line["roofline"] = line.pop("roofline_prefill")
    print(f"# headline {json.dumps(line)}", file=sys.stderr, flush=True)

    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    # the headline workload's own record (its tensors are reused)
    base_cpu = None
    if not args.no_configs:
        del st
        rec = bench_config(wl, t, args, flush, snap, cpu_req, cpu_budget=args.cpu_budget)
        base_cpu = rec.get("cpu_baseline")
        configs = {wl.name: rec}
        print(f"# config {json.dumps(rec)}", file=sys.stderr, flush=True)
    elif snap is not None:
        base_cpu = cpu_baseline(wl, t, snap, *cpu_req, budget_s=args.cpu_budget)
    if not args.no_extra:
        extra = [bench_rope(wl, t, args, flush), bench_masks(wl, t, args, flush)]
    del t, snap
    free()

    if not args.no_configs:
        for name in S.CONFIGS:
            if name == wl.name:
                continue
            w = S.CONFIGS[name]()
            tt = S.make_tensors(w, "cuda", poison=False)
            req = cpu_sample(w)
            sn = None if args.no_cpu else take_snapshot(w, tt, req[0] + req[1])
            configs[name] = bench_config(w, tt, args, flush, sn, req)
            print(f"# config {json.dumps(configs[name])}", file=sys.stderr, flush=True)
            if not args.no_extra and name == "decode_gqa":
                extra.append(bench_masks(w, tt, args, flush))
                extra.append(bench_blocks(w, tt, PagedAttentionStep(w, tt).desc, args, flush))
            if not args.no_extra and name in ("decode_gqa", "mqa_fp8_long"):
                extra.append(bench_rope(w, tt, args, flush))
            del tt, sn
            free()
        line["configs"] = [configs[n] for n in S.CONFIGS if n in configs]

    if not args.no_extra:
        for name in ("decode_gqa", "chunked_prefill_mix", "mqa_fp8_long"):
            w = S.with_cache(S.CONFIGS[name](), "int8")
            tt = S.make_tensors(w, "cuda", poison=False)
            rec = bench_config(w, tt, args, flush)
            extra.append(rec)
            print(f"# extra {json.dumps(rec)}", file=sys.stderr, flush=True)
            del tt
            free()
        extra.append({"workload": "device_to_device_copy", **bench_d2d_copy(args, flush)})
        line["extra"] = extra
    del flush
    free()

    if base_cpu is not None and "decode" in base_cpu:
        line["cpu_baseline"] = base_cpu["decode"]
        if "prefill" in base_cpu:
            line["cpu_baseline_prefill"] = base_cpu["prefill"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
