"""GPU test of pa_decode_noalloc (the decode entry point that allocates nothing
and runs on the library's per-GPU scratch array) against pa_decode with a
caller's workspace, through the C ABI.

Two calls in a row on one GPU, the second with a smaller batch (the array
keeps the first call's contents): each must give output bit-identical to
pa_decode's on the same input, and both must match the oracle at the dtype's
bar.  A call needing more than the array is refused with
PA_ERR_WORKSPACE_TOO_SMALL.
"""

import pytest
import torch

from paged_kv_cache_hkv_amd import binding as B
from paged_kv_cache_hkv_amd import synth as S
from paged_kv_cache_hkv_amd.step import PagedAttentionStep

from harness import Snapshot, compare, oracle_metadata, oracle_outputs, tol_of

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _decode_both(wl):
    """pa_decode (caller's workspace) and pa_decode_noalloc on the same step."""
    t = S.make_tensors(wl, DEV, poison=True)
    requests = list(range(wl.num_reqs))
    snap = Snapshot(wl, t, requests)
    st = PagedAttentionStep(wl, t)
    st.metadata()
    st.cache_write()
    st.decode()
    torch.cuda.synchronize()
    ref = st.out.clone()
    st.out.fill_(7.0)                      # rows the call must rewrite
    print(f"[noalloc] {wl.name}: {wl.num_reqs} decodes, max_seq_len {wl.max_seq_len}, "
          f"cache {wl.cache_kind}", flush=True)
    B.pa_decode_noalloc(st.desc, 0, wl.num_decodes, t.q, st.qsl, st.seq_lens, t.block_tables,
                        t.key_cache, t.value_cache, st.max_seq_len, st.out)
    torch.cuda.synchronize()
    T = wl.num_tokens
    assert torch.equal(ref[:T].view(torch.int16), st.out[:T].view(torch.int16))
    qsl, _, _, _ = oracle_metadata(wl)
    expect = oracle_outputs(wl, t, snap, requests)
    err, rms = compare(wl, st.out, expect, qsl)
    print(f"[noalloc] max_abs={err:.3e} rms={rms:.3e} tol={tol_of(wl)}", flush=True)
    assert err <= tol_of(wl), err


@pytest.mark.parametrize("kind", ["act", "fp8", "mqa_fp8"])
def test_noalloc_two_calls(kind):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()
    fp8 = kind != "act"
    hkv = 1 if kind == "mqa_fp8" else 8     # 32 query heads per K/V head: the largest partials
    big = S.random_batch(41, [6000, 17, 3000, 9000, 1, 2048, 700, 4095] * 4, [], hq=32, hkv=hkv,
                         d=128, act=torch.bfloat16, fp8=fp8)
    small = S.random_batch(42, [100, 2500, 33], [], hq=32, hkv=hkv, d=128, act=torch.bfloat16,
                           fp8=fp8)
    _decode_both(big)
    _decode_both(small)


def test_noalloc_refuses_oversized_call():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()
    wl = S.random_batch(43, [100, 200], [], hq=32, hkv=8, d=128, act=torch.bfloat16)
    t = S.make_tensors(wl, DEV)
    st = PagedAttentionStep(wl, t)
    st.metadata()
    # 2^20 workers' partial slots: far beyond the array
    desc = B.make_desc(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size, B.PA_BF16,
                       decode_workers=1 << 20)
    with pytest.raises(B.PaError) as e:
        B.pa_decode_noalloc(desc, 0, wl.num_decodes, t.q, st.qsl, st.seq_lens, t.block_tables,
                            t.key_cache, t.value_cache, st.max_seq_len, st.out)
    assert e.value.status == B.PA_ERR_WORKSPACE_TOO_SMALL
