"""Full-size GPU parity: the five measured workloads against the oracle.

Each workload runs once at full size through the C ABI in the launch
configuration the benchmark times (library-chosen decode workers, the pool
poisoned outside every listed block and past every sequence), and the oracle
recomputes its rows from the generator's pool as drawn (a host snapshot taken
before the library writes to it) and its own metadata and scatter.  Compared
element by element at the dtype's bar:

* the tour's 3-request step, the 64-request MHA decode batch, the 256-request
  GQA decode batch, the 8192-token chunked-prefill mix (six prefill chunks and
  862 decodes) and the 32-request long-context fp8 MQA decode batch;
* the same GQA, mixed and long MQA shapes over an int8 cache;

every row of every request.

Every cache block the compared requests list is also checked bit for bit
after the step's write against the oracle's scatter.  The oracle computes one
request at a time, so each workload is split into parts of a few tens of
seconds of host work.
"""

import gc

import numpy as np
import pytest
import torch

from paged_kv_cache_hkv_amd import binding as B
from paged_kv_cache_hkv_amd import synth as S
from paged_kv_cache_hkv_amd.step import PagedAttentionStep

from harness import OraclePrep, Snapshot, cache_bits, compare, oracle_metadata, tol_of

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _workload(name, kind):
    wl = S.CONFIGS[name]()
    return wl if kind is None else S.with_cache(wl, kind)


def _split(reqs, n):
    reqs = list(reqs)
    k = -(-len(reqs) // n)
    return [reqs[i:i + k] for i in range(0, len(reqs), k)]


def _parts(name, kind):
    """Lists of requests, one per test part: every request of the workload."""
    wl = _workload(name, kind)
    nd, R = wl.num_decodes, wl.num_reqs
    if name == "chunked_prefill_mix":
        # each prefill chunk on its own, then the decodes in parts
        return [[r] for r in range(nd, R)] + _split(range(nd), 4)
    parts = {"walkthrough": 1, "decode_mha": 2, "decode_gqa": 4, "mqa_fp8_long": 2}[name]
    return _split(range(R), parts)


WORKLOADS = [("walkthrough", None), ("decode_mha", None), ("decode_gqa", None),
             ("mqa_fp8_long", None), ("chunked_prefill_mix", None), ("decode_gqa", "int8"),
             ("mqa_fp8_long", "int8"), ("chunked_prefill_mix", "int8")]
PLAN = {key: _parts(*key) for key in WORKLOADS}
CASES = [(key, i) for key in WORKLOADS for i in range(len(PLAN[key]))]

_CUR = {}


def _run(key):
    """Run the workload once on the GPU; keep its output rows, the cache blocks
    of the compared requests after the write, and the oracle's inputs."""
    if _CUR.get("key") == key:
        return _CUR
    _CUR.clear()
    gc.collect()
    torch.cuda.empty_cache()
    wl = _workload(*key)
    print(f"[full] {wl.name}: {wl.num_reqs} requests, {wl.num_tokens} tokens, pool "
          f"{wl.pool_blocks} blocks", flush=True)
    t = S.make_tensors(wl, DEV, poison=True)
    reqs = sorted(set().union(*map(set, PLAN[key])))
    snap = Snapshot(wl, t, reqs)           # the pool as drawn, before the write
    step = PagedAttentionStep(wl, t)
    step.run()
    torch.cuda.synchronize()
    out = step.out.cpu()
    idx = torch.from_numpy(snap.ids).to(DEV)
    kafter = cache_bits(t.key_cache.index_select(0, idx), wl.cache_8bit)
    vafter = cache_bits(t.value_cache.index_select(0, idx), wl.cache_8bit)
    prep = OraclePrep(wl, t, snap)
    del step, t, idx
    gc.collect()
    torch.cuda.empty_cache()
    _CUR.update(key=key, wl=wl, out=out, prep=prep, kafter=kafter, vafter=vafter,
                cache_checked=False)
    return _CUR


@pytest.mark.parametrize("key,part", CASES, ids=[f"{k[0]}{'_' + k[1] if k[1] else ''}-{i}"
                                                 for k, i in CASES])
def test_full_size_parity(key, part):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()
    st = _run(key)
    wl, prep = st["wl"], st["prep"]
    if not st["cache_checked"]:
        # every slot of the compared requests' blocks, bit for bit
        assert np.array_equal(st["kafter"], prep.kc), "key cache differs from the oracle scatter"
        assert np.array_equal(st["vafter"], prep.vc), "value cache differs from the oracle scatter"
        st["cache_checked"] = True
    reqs = PLAN[key][part]
    expect = prep.rows(reqs)
    qsl, _, _, _ = oracle_metadata(wl)
    err, rms = compare(wl, st["out"], expect, qsl)
    tol = tol_of(wl)
    rows = sum(e.shape[0] for e in expect.values())
    print(f"[full] {wl.name} part {part}: {len(reqs)} requests, {rows} rows, max_abs={err:.3e} "
          f"rms={rms:.3e} tol={tol}", flush=True)
    assert err <= tol, (wl.name, part, err, tol)
