"""Benchmark of the paged-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config decode_mha]
                    [--no-extra] [--no-cpu]

A step is one pass of the whole path over one synthetic batch: metadata
build, cache write of the step's new K/V, decode attention, varlen prefill
attention (whichever the batch has).  The headline workload is the 64-request
MHA decode batch (contexts uniform in 512..4096, 32/32 heads, head_dim 128,
fp16, 65536-block pool).  ``value`` is its KV GB/s: every K/V byte each
decode request must read (seq_len * Hkv * D * 2 * bytes, counted once per
request) divided by the step time, inputs resident in HBM.

Also reported on the same JSON line:
* ``roofline`` of the dominant kernel (the decode call: split kernel plus its
  reduce), timed live with HIP events on the launch stream;
* ``cpu_baseline``: the oracle on the host cores over a bounded sample of the
  same batch;
* ``extra``: the other measured workloads (GQA decode, chunked-prefill mix,
  long-context fp8 MQA decode, and the GQA decode, mixed batch and long MQA
  decode again over an int8 cache), each call timed with events after a 1 GiB
  cache-evicting read; besides attention and the cache write this times the
  fused RoPE + cache write (rotary_dim = head_dim, half-split pairs), on the
  GQA pool the block copy / swap out / swap in of 4096 blocks, and on the GQA
  and mixed batches attention with a 1024-key sliding window and ALiBi.
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
DECODE_SRC = os.path.join(ROOT, "paged_kv_cache_hkv_amd", "csrc", "pa_decode.hip")
PREFILL_SRC = os.path.join(ROOT, "paged_kv_cache_hkv_amd", "csrc", "pa_prefill.hip")


def kv_bytes(wl, reqs):
    e = wl.cache_elem_bytes
    s = wl.seq_lens_host[list(reqs)].astype(np.int64)
    return int(s.sum()) * wl.num_kv_heads * wl.head_dim * 2 * e


def prefill_flops(wl, reqs):
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


def bench_masks(wl, t, iters, flush, window=1024):
    """Decode / prefill with a sliding window and ALiBi slopes on the same batch."""
    h = wl.num_q_heads
    sl = torch.tensor([2.0 ** (-8.0 * (i + 1) / h) for i in range(h)], dtype=torch.float32,
                      device="cuda")
    st = PagedAttentionStep(wl, t, sliding_window=window, alibi_slopes=sl)
    st.metadata()
    fns, names = [], []
    if wl.num_decodes:
        fns.append(st.decode)
        names.append("decode")
    if wl.num_reqs > wl.num_decodes:
        fns.append(st.prefill)
        names.append("prefill")
    for f in fns:
        f()
    rec = {"sliding_window": window, "alibi": True}
    for nm, (med, p10, p90) in zip(names, time_calls(fns, iters, flush)):
        rec[f"{nm}_ms"] = round(med, 4)
    if wl.num_decodes:
        kb = window_kv_bytes(wl, range(wl.num_decodes), window)
        rec["decode_kv_bytes"] = kb
        rec["decode_kv_GBps"] = round(kb / (rec["decode_ms"] * 1e-3) / 1e9, 1)
        rec["decode_hbm_frac"] = round(kb / (rec["decode_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    if wl.num_reqs > wl.num_decodes:
        fl = window_prefill_flops(wl, range(wl.num_decodes, wl.num_reqs), window)
        rec["prefill_flops"] = fl
        rec["prefill_TFLOPs"] = round(fl / (rec["prefill_ms"] * 1e-3) / 1e12, 1)
        rec["prefill_mfma_frac"] = round(fl / (rec["prefill_ms"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
    del st
    return rec


def src_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(name, kernel_src):
    """HBM bytes per launch from committed rocprofv3 counter runs, if still current."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_src_sha") != src_sha(kernel_src):
        return None
    return rec.get("hbm_bytes_per_launch")


def time_calls(fn_list, iters, flush):
    """Median / p10 / p90 milliseconds of each callable, events on the current stream."""
    stream = torch.cuda.current_stream()
    res = [[] for _ in fn_list]
    for _ in range(iters):
        flush.sum()                     # evict L2 and the 256 MB last-level cache (reads only,
                                        # so no dirty lines are left to write back in the call)
        for i, fn in enumerate(fn_list):
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


def bench_extra(name, iters, flush, kind=None):
    wl = S.CONFIGS[name]()
    if kind is not None:
        wl = S.with_cache(wl, kind)
    t = S.make_tensors(wl, "cuda", poison=False)
    st = PagedAttentionStep(wl, t)
    st.run()
    torch.cuda.synchronize()
    rec = {"workload": wl.name, "cache": wl.cache_kind, "requests": wl.num_reqs,
           "decodes": wl.num_decodes, "tokens": wl.num_tokens}
    fns, names = [], []
    if wl.num_decodes:
        fns.append(st.decode)
        names.append("decode")
    if wl.num_reqs > wl.num_decodes:
        fns.append(st.prefill)
        names.append("prefill")
    fns.append(st.cache_write)
    names.append("cache_write")
    table = rope_table(wl.max_seq_len, wl.head_dim, 10000.0, "cuda")
    fns.append(lambda: st.rope_cache_write(table, wl.head_dim, True))
    names.append("rope_cache_write")
    for _ in range(3):
        for f in fns:
            f()
    times = time_calls(fns, iters, flush)
    for nm, (med, p10, p90) in zip(names, times):
        rec[f"{nm}_ms"] = round(med, 4)
        rec[f"{nm}_ms_p10_p90"] = [round(p10, 4), round(p90, 4)]
    rb = rope_bytes(wl, wl.head_dim)
    rec["rope_cache_write_bytes"] = rb
    rec["rope_cache_write_GBps"] = round(rb / (rec["rope_cache_write_ms"] * 1e-3) / 1e9, 1)
    if wl.num_decodes:
        kb = kv_bytes(wl, range(wl.num_decodes))
        gbs = kb / (rec["decode_ms"] * 1e-3) / 1e9
        rec["decode_kv_bytes"] = kb
        rec["decode_kv_GBps"] = round(gbs, 1)
        rec["decode_hbm_frac"] = round(gbs / HBM_PEAK_GBS, 4)
    if wl.num_reqs > wl.num_decodes:
        pre = range(wl.num_decodes, wl.num_reqs)
        fl = prefill_flops(wl, pre)
        toks = int(wl.query_lens[wl.num_decodes:].sum())
        sec = rec["prefill_ms"] * 1e-3
        rec["prefill_flops"] = fl
        rec["prefill_tok_per_s"] = round(toks / sec, 1)
        rec["prefill_TFLOPs"] = round(fl / sec / 1e12, 1)
        rec["prefill_mfma_frac"] = round(fl / sec / 1e12 / BF16_PEAK_TFLOPS, 4)
    if wl.name == "decode_gqa":
        rec["copy_blocks"] = bench_blocks(wl, t, st.desc, iters, flush)
    if wl.name in ("decode_gqa", "chunked_prefill_mix"):
        rec["window_alibi"] = bench_masks(wl, t, iters, flush)
    del st, t
    torch.cuda.empty_cache()
    return rec


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


def bench_blocks(wl, t, desc, iters, flush, n_pairs=4096):
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
    for f in fns:
        f()
    times = time_calls(fns, iters, flush)
    moved = 2 * n_pairs * blk                       # K and V blocks
    rec = {"pairs": n_pairs, "block_bytes": blk, "bytes_per_call": moved}
    for nm, (med, p10, p90), nbytes in zip(
            ["copy", "swap_out", "swap_in", "torch_d2h_contiguous", "torch_h2d_contiguous"], times,
            [moved, moved, moved, n_pairs * blk, n_pairs * blk]):
        rec[f"{nm}_ms"] = round(med, 4)
        rec[f"{nm}_GBps"] = round(nbytes / (med * 1e-3) / 1e9, 1)
    # the device copy reads and writes every byte in HBM
    rec["copy_hbm_frac"] = round(2 * moved / (rec["copy_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    del host_k, host_v, dev_buf
    return rec


def take_snapshot(wl, t):
    """Host copy of the decode requests' blocks as drawn, before any kernel runs."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from harness import Snapshot   # test infrastructure
    return Snapshot(wl, t, list(range(wl.num_decodes)))


def cpu_baseline(wl, t, snap, budget_s=12.0):
    """The oracle (as it stands) on the host, over the batch's requests in order."""
    from harness import oracle_outputs   # test infrastructure: the oracle
    reqs_all = list(range(wl.num_decodes))
    done, spent, kb = 0, 0.0, 0
    chunk = 4
    while done < len(reqs_all) and spent < budget_s:
        req = reqs_all[done:done + chunk]
        t0 = time.perf_counter()
        oracle_outputs(wl, t, snap, req)
        spent += time.perf_counter() - t0
        kb += kv_bytes(wl, req)
        done += len(req)
    return {"value": round(kb / spent / 1e9, 4), "unit": "GB/s", "cores": torch.get_num_threads(),
            "kind": "oracle",
            "sample": f"first {done} of {len(reqs_all)} decode requests of {wl.name} "
                      f"({kb} KV bytes, {spent:.1f} s, NumPy float64)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="decode_mha")
    ap.add_argument("--extra-iters", type=int, default=20)
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
    wl = S.CONFIGS[args.config]()
    t = S.make_tensors(wl, "cuda", poison=False)
    snap = None if args.no_cpu else take_snapshot(wl, t)
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

    ev = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        st.metadata()
        write()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        st.decode()
        b.record(stream)
        st.prefill()
        ev.append((a, b))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    dec_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))

    kb = kv_bytes(wl, range(wl.num_decodes))
    value = kb / (ms_step * 1e-3) / 1e9
    achieved = kb / (dec_ms * 1e-3) / 1e9
    line = {
        "metric": "paged decode attn achieved KV GB/s (% HBM peak) + prefill query tok/s (% MFMA)",
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
        "config": {"workload": wl.name, "requests": wl.num_reqs, "decodes": wl.num_decodes,
                   "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "block_size": wl.block_size,
                   "pool_blocks": wl.pool_blocks, "kv_bytes_per_step": kb,
                   "step": ("metadata + rope_cache_write" if args.fused_rope else
                            "metadata + cache_write") + " + decode (+ prefill when present)",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": read_traffic(wl.name + "_decode", DECODE_SRC),
                     "kernel": "pa_decode (decode_kernel + decode_reduce_kernel)",
                     "kernel_ms": round(dec_ms, 4)},
    }
    if not args.no_extra:
        del st
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        extra = []
        for name, kind in (("decode_gqa", None), ("chunked_prefill_mix", None),
                           ("mqa_fp8_long", None), ("decode_gqa", "int8"),
                           ("chunked_prefill_mix", "int8"), ("mqa_fp8_long", "int8")):
            extra.append(bench_extra(name, args.extra_iters, flush, kind))
            print(f"# {json.dumps(extra[-1])}", file=sys.stderr, flush=True)
        line["extra"] = extra
        del flush
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(wl, t, snap)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
