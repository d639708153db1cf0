"""GPU parity of the HIP path against the oracle, through the C ABI.

Bars: metadata and cache bytes bit-exact; attention max-abs within 5e-3
(fp16), 2e-2 (bf16), 6e-2 (fp8 K/V, the oracle dequantising the identical
codes); int8 K/V keep the activation dtype's bar (every code is exact in
bf16 and fp16, so the cache format adds no rounding of its own).  Small shapes
compare every output row; the five measured workloads at full size are in
test_gpu_full.py.
"""

import numpy as np
import pytest
import torch

from paged_kv_cache_hkv_amd import binding as B
from paged_kv_cache_hkv_amd import synth as S
from paged_kv_cache_hkv_amd.step import PagedAttentionStep
from oracle import cache as OC
from oracle import codecs as OD

from harness import (Snapshot, act_name, bits16, cache_bits, compare, oracle_cache_dtype,
                     oracle_metadata, oracle_outputs, tol_of)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def _run_and_check(wl, requests=None, workers=0, poison=True, qsl_len=None, tensors=None):
    _need_gpu()
    t = tensors if tensors is not None else S.make_tensors(wl, DEV, poison=poison)
    if requests is None:
        requests = list(range(wl.num_reqs))
    snap = Snapshot(wl, t, requests)
    step = PagedAttentionStep(wl, t, decode_workers=workers, qsl_len=qsl_len)
    step.run()
    torch.cuda.synchronize()
    qsl, _, _, _ = oracle_metadata(wl, qsl_len)
    expect = oracle_outputs(wl, t, snap, requests, qsl_len)
    err, rms = compare(wl, step.out, expect, qsl)
    tol = tol_of(wl)
    print(f"[{wl.name}] requests={len(requests)} max_abs={err:.3e} rms={rms:.3e} tol={tol}",
          flush=True)
    assert err <= tol, (wl.name, err, tol)
    return step, t


# ---------------------------------------------------------------- metadata --

@pytest.mark.parametrize("wl_fn", [
    lambda: S.walkthrough(),
    lambda: S.random_batch(11, [0, 15, 16, 17, 31], [(0, 1), (5, 0), (3, 40), (0, 0), (100, 33)],
                           pad=7),
    lambda: S.chunked_prefill_mix(),
])
def test_metadata_bit_exact(wl_fn):
    _need_gpu()
    wl = wl_fn()
    t = S.make_tensors(wl, DEV, poison=False)
    qsl_len = wl.num_reqs + 1 + 9
    step = PagedAttentionStep(wl, t, qsl_len=qsl_len)
    step.positions.fill_(-7)
    step.metadata()
    torch.cuda.synchronize()
    qsl, seq_lens, pos, slots = oracle_metadata(wl, qsl_len)
    assert step.qsl.cpu().tolist() == qsl
    assert step.seq_lens.cpu().tolist() == seq_lens
    assert step.slot_mapping.cpu().tolist() == slots
    got_pos = step.positions.cpu().tolist()
    for i, p in enumerate(pos):
        assert got_pos[i] == (-7 if p is None else p), i   # padding rows untouched


# ------------------------------------------------------------- cache write --

@pytest.mark.parametrize("act,kind", [(torch.float16, "act"), (torch.bfloat16, "act"),
                                      (torch.bfloat16, "fp8"), (torch.float16, "fp8"),
                                      (torch.bfloat16, "int8"), (torch.float16, "int8")])
@pytest.mark.parametrize("d", [64, 128])
def test_cache_write_bit_exact(act, kind, d):
    _need_gpu()
    wl = S.random_batch(21 + d, [3, 16, 200], [(0, 37), (16, 16)], hq=8, hkv=4, d=d, act=act,
                        fp8=kind == "fp8", int8=kind == "int8", pad=5)
    t = S.make_tensors(wl, DEV, poison=True)
    one = wl.cache_8bit
    before_k = cache_bits(t.key_cache, one)
    before_v = cache_bits(t.value_cache, one)
    step = PagedAttentionStep(wl, t)
    step.metadata()
    step.cache_write()
    torch.cuda.synchronize()
    _, _, _, slots = oracle_metadata(wl)
    T = step.T_pad
    act_n = act_name(act)
    want_k, want_v = OC.scatter(before_k, before_v, bits16(t.k_new[:T]), bits16(t.v_new[:T]),
                                slots, wl.block_size, act_dtype=act_n,
                                cache_dtype=oracle_cache_dtype(wl),
                                k_inv_scale=np.float32(1) / np.float32(t.k_scale),
                                v_inv_scale=np.float32(1) / np.float32(t.v_scale), num_tokens=T)
    # every byte of the pool: written slots equal the oracle, all others unchanged
    assert np.array_equal(cache_bits(t.key_cache, one), want_k)
    assert np.array_equal(cache_bits(t.value_cache, one), want_v)


def test_fp8_encode_exhaustive_on_gpu():
    """All 65536 bf16 and fp16 inputs through pa_cache_write's encoder vs the oracle's."""
    _need_gpu()
    for act in (torch.bfloat16, torch.float16):
        for scale in (0.125, 0.0137):
            bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
            x = bits.view(act).reshape(512, 1, 128).to(DEV)
            kc = torch.zeros((32, 16, 1, 128), dtype=torch.uint8, device=DEV)
            vc = torch.zeros_like(kc)
            slots = torch.arange(512, dtype=torch.int64, device=DEV)
            desc = B.make_desc(8, 1, 128, 16, B.PA_BF16 if act == torch.bfloat16 else B.PA_F16,
                               B.PA_FP8_E4M3, k_scale=scale, v_scale=scale)
            B.pa_cache_write(desc, x, x, slots, kc, vc)
            torch.cuda.synchronize()
            got = kc.reshape(-1).cpu().numpy()
            with np.errstate(invalid="ignore"):
                xf = OD.decode(bits.numpy().view(np.uint16), act_name(act)).astype(np.float32)
            want = OD.e4m3fn_encode(xf, np.float32(1) / np.float32(scale))
            assert np.array_equal(got, want), (act, scale, np.nonzero(got != want)[0][:10])


def test_int8_encode_exhaustive_on_gpu():
    """All 65536 bf16 and fp16 inputs (NaN, infinities, ties included) through
    pa_cache_write's int8 encoder vs the oracle's."""
    _need_gpu()
    for act in (torch.bfloat16, torch.float16):
        for scale in (0.125, 0.0137, 3.0e-5):
            bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
            x = bits.view(act).reshape(512, 1, 128).to(DEV)
            kc = torch.full((32, 16, 1, 128), -128, dtype=torch.int8, device=DEV)
            vc = torch.full_like(kc, -128)
            slots = torch.arange(512, dtype=torch.int64, device=DEV)
            desc = B.make_desc(8, 1, 128, 16, B.PA_BF16 if act == torch.bfloat16 else B.PA_F16,
                               B.PA_INT8, k_scale=scale, v_scale=scale)
            B.pa_cache_write(desc, x, x, slots, kc, vc)
            torch.cuda.synchronize()
            got = kc.reshape(-1).cpu().numpy()
            with np.errstate(invalid="ignore"):
                xf = OD.decode(bits.numpy().view(np.uint16), act_name(act)).astype(np.float32)
            want = OD.int8_encode(xf, np.float32(1) / np.float32(scale))
            assert np.array_equal(got, want), (act, scale, np.nonzero(got != want)[0][:10])
            assert np.array_equal(vc.reshape(-1).cpu().numpy(), want)


# -------------------------------------------------------- attention parity --

def test_walkthrough_parity():
    """The pages' 3-request step: R1, R2 decode; R3 prefills 298 tokens."""
    wl = S.walkthrough()
    step, t = _run_and_check(wl, qsl_len=1025)
    # padding rows 300..303 are never written
    assert torch.all(step.out[300:] == 0)


SHAPES = [(8, 8, 64), (32, 8, 128), (32, 1, 128), (32, 32, 128), (16, 2, 64), (12, 4, 128),
          (24, 1, 64)]
DTYPES = [(torch.float16, "act"), (torch.bfloat16, "act"), (torch.bfloat16, "fp8"),
          (torch.float16, "fp8"), (torch.bfloat16, "int8"), (torch.float16, "int8")]


@pytest.mark.parametrize("hq,hkv,d", SHAPES)
@pytest.mark.parametrize("act,kind", DTYPES)
def test_small_mixed_parity(hq, hkv, d, act, kind):
    seed = (hq * 100 + hkv * 10 + d + {"act": 0, "fp8": 7, "int8": 11}[kind]
            + (3 if act == torch.float16 else 0))
    decodes = [0, 14, 15, 16, 31, 32, 33, 298, 540, 1000]
    prefills = [(0, 1), (0, 17), (7, 40), (16, 100), (100, 129), (0, 298), (33, 64)]
    wl = S.random_batch(seed, decodes, prefills, hq=hq, hkv=hkv, d=d, act=act,
                        fp8=kind == "fp8", int8=kind == "int8", pad=3)
    _run_and_check(wl)


@pytest.mark.parametrize("case", ["equal_lengths", "many_requests"])
def test_prefill_dispatch_order_parity(case):
    """The prefill's work lists rank requests longest first within each run of
    64 (ties by index): a group of six requests of one sequence length with 1 to
    300 new tokens (so their tile counts differ) and a pair of another length;
    70 small prefills take two runs of the per-wave request cursor."""
    if case == "equal_lengths":
        prefills = [(0, 300), (100, 200), (50, 120), (200, 100), (0, 300), (250, 50), (50, 120),
                    (299, 1)]
        wl = S.random_batch(91, [40, 7], prefills, hq=16, hkv=4, d=128, act=torch.bfloat16)
    else:
        rng = np.random.default_rng(92)
        prefills = [(int(c), int(n)) for c, n in zip(rng.integers(0, 80, 70), rng.integers(1, 90, 70))]
        wl = S.random_batch(92, [33], prefills, hq=8, hkv=2, d=64, act=torch.float16)
    _run_and_check(wl)


def test_prefill_unpinned_schedule_parity():
    """More head groups than compute units (320 query heads, one per K/V head):
    the grid is no multiple of the head-group count, so every workgroup takes
    items of every head group from one shared list instead of keeping one group."""
    wl = S.random_batch(93, [20], [(0, 150), (40, 90), (300, 33), (0, 1)], hq=320, hkv=320, d=64,
                        act=torch.float16)
    _run_and_check(wl)


@pytest.mark.parametrize("workers", [1, 7, 64, 1000, 5000])
def test_long_decode_split_parity(workers):
    """Long contexts cut between decode workers in every way: one worker (no
    cuts), a few long shares, many short ones, and more workers than units
    (empty shares)."""
    wl = S.random_batch(77, [2047, 2048, 2049, 4000, 5000], [(3000, 5)], hq=32, hkv=4, d=128,
                        act=torch.bfloat16)
    _run_and_check(wl, workers=workers)
