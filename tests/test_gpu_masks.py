"""GPU parity of the mask variants (sliding window, ALiBi) of pa_decode and
pa_prefill_varlen against the oracle (oracle/attention.py), through the C ABI.

Same bars as the plain path: max-abs within 5e-3 (fp16), 2e-2 (bf16), 6e-2
(fp8 K/V), the activation dtype's for int8 K/V.  Windows from 1 key (the row's own value) through windows shorter
than a block, spanning block and 64-key tile edges, to longer than every
sequence; ALiBi alone and with a window; MHA, GQA, MQA with 32 query heads
per K/V head; 16-bit, fp8 and int8 caches; chunked prefills with cached prefixes
and decodes in one batch.
"""

import numpy as np
import pytest
import torch

from paged_kv_cache_hkv_amd import binding as B
from paged_kv_cache_hkv_amd import synth as S
from paged_kv_cache_hkv_amd.step import PagedAttentionStep

from harness import Snapshot, compare, oracle_metadata, oracle_outputs, tol_of

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def slopes(h):
    """Geometric ALiBi slopes 2^(-8 i / h), i = 1..h, as float32."""
    return np.array([2.0 ** (-8.0 * (i + 1) / h) for i in range(h)], np.float32)


def _check(wl, window, alibi, workers=0, requests=None):
    _need_gpu()
    t = S.make_tensors(wl, DEV, poison=True)
    sl = slopes(wl.num_q_heads) if alibi else None
    sl_dev = torch.from_numpy(sl).to(DEV) if alibi else None
    if requests is None:
        requests = list(range(wl.num_reqs))
    snap = Snapshot(wl, t, requests)
    step = PagedAttentionStep(wl, t, decode_workers=workers, sliding_window=window,
                              alibi_slopes=sl_dev)
    print(f"[masks] {wl.name} window={window} alibi={alibi} workers={workers}", flush=True)
    step.run()
    torch.cuda.synchronize()
    qsl, _, _, _ = oracle_metadata(wl)
    expect = oracle_outputs(wl, t, snap, requests, sliding_window=window,
                            alibi_slopes=None if sl is None else sl.astype(np.float64))
    err, rms = compare(wl, step.out, expect, qsl)
    tol = tol_of(wl)
    print(f"[masks] max_abs={err:.3e} rms={rms:.3e} tol={tol}", flush=True)
    assert err <= tol, (wl.name, window, alibi, err, tol)


def _mixed(seed, hq, hkv, act, fp8, int8=False):
    # decodes (cached lengths incl. block edges) then chunked prefills (cached, new)
    return S.random_batch(seed, [0, 15, 16, 63, 64, 200, 700], [(0, 1), (0, 70), (40, 129), (300, 33)],
                          hq=hq, hkv=hkv, d=128, act=act, fp8=fp8, int8=int8, pad=3)


@pytest.mark.parametrize("window", [1, 7, 16, 64, 100, 5000])
@pytest.mark.parametrize("alibi", [False, True])
def test_mixed_gqa_bf16(window, alibi):
    _check(_mixed(51, 8, 2, torch.bfloat16, False), window, alibi)


@pytest.mark.parametrize("window,alibi", [(0, True), (33, False), (33, True)])
@pytest.mark.parametrize("hq,hkv,act,fp8", [
    (4, 4, torch.float16, False),     # MHA
    (8, 2, torch.bfloat16, True),     # GQA, fp8 cache (register prefill path)
    (32, 1, torch.bfloat16, True),    # MQA, two MFMA column tiles in decode
    (32, 1, torch.float16, False),
])
def test_head_layouts(window, alibi, hq, hkv, act, fp8):
    _check(_mixed(52 + hq, hq, hkv, act, fp8), window, alibi)


@pytest.mark.parametrize("workers", [1, 7, 64])
def test_window_with_forced_splits(workers):
    """Few workers: segments cut at many places, partials merged by the reduce."""
    wl = S.random_batch(53, [500, 1000, 37, 2000], [], hq=8, hkv=2, d=128, act=torch.bfloat16)
    _check(wl, 300, True, workers=workers)


def test_head_dim_64_walkthrough():
    """The tour's batch (f16, 8/8 heads, D 64) with a 100-token window and ALiBi."""
    _check(S.CONFIGS["walkthrough"](), 100, True)


def test_decode_gqa_full_size_sampled():
    """The 256-request GQA decode batch at full size with a 1024-token window and
    ALiBi: sampled requests against the oracle."""
    wl = S.CONFIGS["decode_gqa"]()
    _check(wl, 1024, True, requests=[0, 37, 128, 255])


@pytest.mark.parametrize("window,alibi", [(0, True), (33, True), (100, False)])
@pytest.mark.parametrize("hq,hkv,act", [(8, 2, torch.bfloat16), (32, 1, torch.float16)])
def test_int8_cache(window, alibi, hq, hkv, act):
    _check(_mixed(60 + hq, hq, hkv, act, False, int8=True), window, alibi)


@pytest.mark.parametrize("alibi", [False, True])
def test_unbounded_window_walkthrough(alibi):
    """A window of 2^31 - 1 keys (a caller's way to say "unbounded") on the tour's
    batch: R3's first query tile holds rows before the sequence start, whose
    window edge would fall below -2^31 in 32 bits; every key stays visible."""
    _check(S.CONFIGS["walkthrough"](), 2 ** 31 - 1, alibi)
