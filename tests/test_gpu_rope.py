"""GPU parity of pa_rope_cache_write against the oracle (oracle/rope.py).

Integer-exact: the kernel's float32 steps are the oracle's, so the rotated
query rows and every written cache byte must match bit for bit; cache slots
that no token addresses must be unchanged.  Positions and slots come from the
oracle's metadata, the cos/sin table from the oracle's table builder; nothing
the oracle consumes comes from the library.
"""

import numpy as np
import pytest
import torch

from oracle import cache as OC
from oracle import rope as OR
from paged_kv_cache_hkv_amd import binding as B
from paged_kv_cache_hkv_amd import synth as S

from harness import act_name, bits16, cache_bits, oracle_cache_dtype, oracle_metadata

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def _check(wl, rotary_dim, neox, base=10000.0, max_position=None, bad_positions=(), whole_pool=True):
    _need_gpu()
    t = S.make_tensors(wl, DEV, poison=True)
    _, _, positions, slots = oracle_metadata(wl)
    Tp = t.q.shape[0]
    pos = np.array([0 if p is None else p for p in positions[:Tp]], np.int64)
    slots = np.array(slots[:Tp], np.int64)
    if max_position is None:
        max_position = int(pos.max()) + 1
    for i, v in bad_positions:
        pos[i] = v
    table = OR.cos_sin_table(max_position, rotary_dim, base)
    act = act_name(wl.act_dtype)
    fp8 = wl.cache_8bit          # one-byte cache elements
    cache_dt = oracle_cache_dtype(wl)
    cache_code = {"act": B.PA_F16 if act == "f16" else B.PA_BF16, "fp8_e4m3": B.PA_FP8_E4M3,
                  "int8": B.PA_INT8}[wl.cache_kind]
    q0, k0, v0 = bits16(t.q), bits16(t.k_new), bits16(t.v_new)
    if whole_pool:
        kc0, vc0 = cache_bits(t.key_cache, fp8), cache_bits(t.value_cache, fp8)
    desc = B.make_desc(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size,
                       B.PA_F16 if act == "f16" else B.PA_BF16,
                       cache_code, k_scale=t.k_scale, v_scale=t.v_scale)
    print(f"[rope] {wl.name} rotary_dim={rotary_dim} neox={neox} tokens={Tp}", flush=True)
    B.pa_rope_cache_write(desc, torch.from_numpy(pos).to(DEV), torch.from_numpy(table).to(DEV),
                          rotary_dim, neox, t.q, t.k_new, t.v_new,
                          torch.from_numpy(slots).to(DEV), t.key_cache, t.value_cache,
                          num_tokens=Tp)
    torch.cuda.synchronize()
    k_inv = np.float32(1) / np.float32(t.k_scale)
    v_inv = np.float32(1) / np.float32(t.v_scale)
    # query rows: rotated in place where the position is in the table
    assert np.array_equal(bits16(t.q), OR.apply_rope(q0, act, pos, table, rotary_dim, neox))
    # K/V inputs are not modified
    assert np.array_equal(bits16(t.k_new), k0) and np.array_equal(bits16(t.v_new), v0)
    if whole_pool:
        _, want_k, want_v = OR.rope_cache_write(q0, k0, v0, pos, table, rotary_dim, neox, slots,
                                                kc0, vc0, wl.block_size, act, cache_dt,
                                                k_inv, v_inv, Tp)
        assert np.array_equal(cache_bits(t.key_cache, fp8), want_k)
        assert np.array_equal(cache_bits(t.value_cache, fp8), want_v)
    else:
        # large pools: the written rows, built with the oracle's scatter on a
        # zero pool holding just those slots
        ok = (pos >= 0) & (pos < max_position) & (slots >= 0)
        idx = np.nonzero(ok)[0]
        H, D = wl.num_kv_heads, wl.head_dim
        dt = np.uint8 if fp8 else np.uint16
        zero = np.zeros((len(idx), 1, H, D), dt)
        k_rot = OR.apply_rope(k0[idx], act, pos[idx], table, rotary_dim, neox)
        want_k, want_v = OC.scatter(zero, zero, k_rot, v0[idx], np.arange(len(idx)), 1, act,
                                    cache_dt, k_inv, v_inv)
        sl = torch.from_numpy(slots[idx]).to(DEV)
        got_k = cache_bits(t.key_cache.view(-1, H, D).index_select(0, sl), fp8)
        got_v = cache_bits(t.value_cache.view(-1, H, D).index_select(0, sl), fp8)
        assert np.array_equal(got_k, want_k[:, 0]) and np.array_equal(got_v, want_v[:, 0])


@pytest.mark.parametrize("rotary_dim,neox", [(64, True), (64, False), (32, True), (16, False)])
def test_walkthrough(rotary_dim, neox):
    """The tour's three requests (f16, 8/8 heads, D 64), padding rows included."""
    _check(S.CONFIGS["walkthrough"](), rotary_dim, neox)


@pytest.mark.parametrize("act", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("kind", ["act", "fp8", "int8"])
@pytest.mark.parametrize("neox", [True, False])
def test_gqa_batches(act, kind, neox):
    wl = S.random_batch(31, [3, 16, 200], [(0, 37), (16, 16), (5, 100)], hq=8, hkv=2, d=128,
                        act=act, fp8=kind == "fp8", int8=kind == "int8", pad=5)
    _check(wl, 128, neox, base=500000.0)


def test_positions_outside_the_table_are_left_alone():
    wl = S.random_batch(32, [40, 7], [(0, 30)], hq=4, hkv=4, d=128, act=torch.bfloat16, pad=3)
    # token 0: negative position; token 3: position == max_position; token 5 stays valid
    _check(wl, 96, True, max_position=64, bad_positions=[(0, -5), (3, 64), (4, 10 ** 9)])


def test_chunked_prefill_mix_full_size():
    """The 8192-token mixed batch (bf16, 32/8 heads, D 128): written rows bit-exact."""
    _check(S.CONFIGS["chunked_prefill_mix"](), 128, True, base=500000.0, whole_pool=False)
