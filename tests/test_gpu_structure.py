"""Structural GPU tests: properties that hold at any size.

At long contexts a max-abs tolerance cannot see one missing 16-token block
(its weight in the softmax is too small), so these tests probe positions and
invariants directly:

* spike: one key per request aligned with its query and a marker value: the
  output must equal the marker, wherever the key sits (block boundaries,
  the cuts between decode workers, the token written this step);
* block permutation: the same logical K/V under other physical block ids give
  bit-identical outputs;
* determinism: two runs give bit-identical outputs;
* split invariance: different decode worker counts agree to rounding (1e-3
  of the largest output in fp16);
* request order: shuffling the batch leaves prefill rows bit-identical and
  decode rows within the split-invariance bar;
* aliasing: requests that share prefix blocks read them correctly;
* absent blocks: table entries outside the pool hold no keys (rows with no
  visible key are zero);
* rising scores: prefill rows whose maxima grow after their first key tile,
  a little, a lot, and past exp2's range against the old reference.
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


def _slot(wl, r, j):
    return int(wl.block_tables[r, j // wl.block_size]) * wl.block_size + j % wl.block_size


def _enc(wl, x, scale):
    """x (float) as stored in the cache format."""
    if wl.cache_fp8:
        return torch.clamp(x / scale, -448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    if wl.cache_int8:
        return torch.clamp(torch.round(x / scale), -127, 127).to(torch.int8)
    return x.to(wl.act_dtype)


@pytest.mark.parametrize("case", ["gqa_bf16", "mqa_fp8", "mha_f16", "gqa_int8"])
def test_spike_positions(case):
    _need_gpu()
    if case == "gqa_bf16":
        cached = [8191, 8192, 8193, 20000]
        wl = S.random_batch(5, cached, [], hq=32, hkv=8, d=128, act=torch.bfloat16)
    elif case == "mqa_fp8":
        cached = [32768, 32768, 4095, 1]
        wl = S.random_batch(6, cached, [], hq=32, hkv=1, d=128, act=torch.bfloat16, fp8=True)
    elif case == "gqa_int8":
        cached = [8191, 30000, 100, 0]
        wl = S.random_batch(9, cached, [], hq=32, hkv=4, d=128, act=torch.float16, int8=True)
    else:
        cached = [2047, 3000, 64, 17]
        wl = S.random_batch(7, cached, [], hq=16, hkv=16, d=64, act=torch.float16)
    t = S.make_tensors(wl, DEV, poison=True)
    step = PagedAttentionStep(wl, t)
    d, hkv, G = wl.head_dim, wl.num_kv_heads, wl.group
    rng = np.random.default_rng(99)
    # query rows: one sign pattern per K/V head, shared by its G query heads
    sign = torch.from_numpy(rng.choice([-1.0, 1.0], size=(wl.num_reqs, hkv, d))).float()
    q = sign.repeat_interleave(G, dim=1).to(wl.act_dtype).to(DEV)
    t.q[:wl.num_reqs] = q
    # spike magnitude: large but representable in the cache format
    amp = 5.0
    marker = torch.from_numpy(rng.choice([-3.0, 3.0], size=(wl.num_reqs, hkv, d))).float()

    def enc(x, scale):
        return _enc(wl, x, scale)

    positions = {}
    for r in range(wl.num_reqs):
        s = int(wl.seq_lens_host[r])
        cands = [0, 15, 16, s - 1, s // 2, max(0, s - 17)]
        positions[r] = cands[(r * 7) % len(cands)]
    # put the spike either into the cache or into this step's new row (position s-1)
    qsl, _, _, _ = oracle_metadata(wl)
    kspike = {r: amp * sign[r] for r in range(wl.num_reqs)}
    for r, j in positions.items():
        s = int(wl.seq_lens_host[r])
        if j == s - 1:
            t.k_new[qsl[r]] = kspike[r].to(wl.act_dtype).to(DEV)
            t.v_new[qsl[r]] = marker[r].to(wl.act_dtype).to(DEV)
        else:
            slot = _slot(wl, r, j)
            b, o = slot // wl.block_size, slot % wl.block_size
            t.key_cache[b, o] = enc(kspike[r], t.k_scale).to(DEV)
            t.value_cache[b, o] = enc(marker[r], t.v_scale).to(DEV)
    step.run()
    torch.cuda.synchronize()
    out = step.out.float().cpu()
    for r, j in positions.items():
        mk = marker[r]
        if wl.cache_fp8:   # the marker as stored: its e4m3 code times the scale
            mk = enc(mk, t.v_scale).view(torch.float8_e4m3fn).float() * t.v_scale
        elif wl.cache_int8:
            mk = enc(mk, t.v_scale).float() * t.v_scale
        want = mk.repeat_interleave(G, dim=0)                 # [Hq, D]
        got = out[qsl[r]]
        err = float((got - want).abs().max())
        print(f"[spike {case}] r={r} s={int(wl.seq_lens_host[r])} pos={j} err={err:.3e}",
              flush=True)
        assert err < 0.05, (r, j, err)


def _permuted(wl, t, seed):
    """The same logical cache under a new random physical numbering."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(wl.pool_blocks)
    perm_t = torch.from_numpy(perm).to(DEV)
    kc = torch.empty_like(t.key_cache)
    vc = torch.empty_like(t.value_cache)
    kc[perm_t] = t.key_cache
    vc[perm_t] = t.value_cache
    bt = wl.block_tables.copy()
    valid = bt >= 0
    bt[valid] = perm[bt[valid]]
    wl2 = S.Workload(**{**wl.__dict__, "block_tables": bt.astype(np.int32)})
    t2 = S.Tensors(q=t.q, k_new=t.k_new, v_new=t.v_new, key_cache=kc, value_cache=vc,
                   num_computed=t.num_computed, query_lens=t.query_lens,
                   block_tables=torch.from_numpy(bt.astype(np.int32)).to(DEV),
                   k_scale=t.k_scale, v_scale=t.v_scale)
    return wl2, t2


@pytest.mark.parametrize("kind", ["act", "fp8", "int8"])
def test_block_permutation_bit_identical(kind):
    _need_gpu()
    wl = S.random_batch(8, [100, 3000, 5000, 17], [(0, 200), (300, 130)], hq=32, hkv=8, d=128,
                        act=torch.bfloat16, fp8=kind == "fp8", int8=kind == "int8")
    t = S.make_tensors(wl, DEV)
    wl2, t2 = _permuted(wl, t, 3)
    a = PagedAttentionStep(wl, t)
    a.run()
    b = PagedAttentionStep(wl2, t2)
    b.run()
    torch.cuda.synchronize()
    T = wl.num_tokens
    assert torch.equal(a.out[:T].view(torch.int16), b.out[:T].view(torch.int16))


def test_determinism_two_runs():
    _need_gpu()
    wl = S.random_batch(9, [4000, 8000, 12], [(1000, 300)], hq=32, hkv=8, d=128,
                        act=torch.bfloat16)
    t = S.make_tensors(wl, DEV)
    st = PagedAttentionStep(wl, t, decode_workers=256)
    st.run()
    torch.cuda.synchronize()
    first = st.out.clone()
    st.out.zero_()
    st.attention()
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), st.out.view(torch.int16))


# Split invariance bars, relative to the largest output magnitude.  The PV
# product takes probabilities rounded to the activation type relative to each
# worker's own reference maximum, so two cuttings of one head round different
# mantissas: a relative spread of ~2^-12 (fp16) or ~2^-9 (bf16) per weight,
# which averages down over the keys.  1e-3 holds for fp16; bf16 keeps two
# rounding steps of its 8-bit mantissa.
SPLIT_REL = {torch.float16: 1e-3, torch.bfloat16: 8e-3}


@pytest.mark.parametrize("act", [torch.float16, torch.bfloat16])
def test_split_invariance(act):
    """Different decode worker counts cut the key stream at different places;
    the merged results differ only by rounding: within 1e-3 of the output's
    largest magnitude in fp16 (8e-3 in bf16, see SPLIT_REL)."""
    _need_gpu()
    wl = S.random_batch(10, [6000, 9000, 300, 20000], [], hq=32, hkv=4, d=128, act=act)
    t = S.make_tensors(wl, DEV)
    outs = []
    for workers in (3, 77, 0, 1):
        st = PagedAttentionStep(wl, t, decode_workers=workers)
        if not outs:
            st.run()                 # write this step's tokens once
        else:
            st.metadata()
            st.attention()
        torch.cuda.synchronize()
        outs.append(st.out[:wl.num_tokens].float())
    ref = outs[-1]
    for o in outs[:-1]:
        rel = float((o - ref).abs().max() / ref.abs().max())
        print(f"[split] {act} rel={rel:.2e}", flush=True)
        assert rel < SPLIT_REL[act], rel


@pytest.mark.parametrize("kind", ["act", "fp8"])
def test_request_order_invariance(kind):
    """The same requests in another batch order (decodes shuffled among
    themselves, prefills among themselves): prefill rows are bit-identical
    (each query tile is computed the same way wherever it is dispatched);
    decode rows, whose heads the workers now cut at other places, agree
    within the split-invariance bar; both match the oracle."""
    _need_gpu()
    wl = S.random_batch(14, [4000, 17, 900, 2500, 64, 7000], [(0, 300), (500, 129), (64, 64)],
                        hq=32, hkv=8, d=128, act=torch.bfloat16, fp8=kind == "fp8")
    t = S.make_tensors(wl, DEV)
    requests = list(range(wl.num_reqs))
    snap = Snapshot(wl, t, requests)
    a = PagedAttentionStep(wl, t)
    a.run()
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    nd = wl.num_decodes
    order = np.concatenate([rng.permutation(nd), nd + rng.permutation(wl.num_reqs - nd)])
    qsl, _, _, _ = oracle_metadata(wl)
    rows = np.concatenate([np.arange(qsl[r], qsl[r + 1]) for r in order])
    wl2 = S.Workload(**{**wl.__dict__, "num_computed": wl.num_computed[order].copy(),
                        "query_lens": wl.query_lens[order].copy(),
                        "block_tables": wl.block_tables[order].copy()})
    ridx = torch.from_numpy(rows).to(DEV)
    T = wl.num_tokens

    def reorder(x):
        y = x.clone()
        y[:T] = x[ridx]
        return y

    # the pool already holds this step's tokens; the second write stores the same bytes
    t2 = S.Tensors(q=reorder(t.q), k_new=reorder(t.k_new), v_new=reorder(t.v_new),
                   key_cache=t.key_cache, value_cache=t.value_cache,
                   num_computed=torch.from_numpy(wl2.num_computed).to(DEV),
                   query_lens=torch.from_numpy(wl2.query_lens).to(DEV),
                   block_tables=torch.from_numpy(wl2.block_tables).to(DEV),
                   k_scale=t.k_scale, v_scale=t.v_scale)
    b = PagedAttentionStep(wl2, t2)
    b.run()
    torch.cuda.synchronize()
    qsl2, _, _, _ = oracle_metadata(wl2)
    for i, r in enumerate(order.tolist()):
        ya = a.out[qsl[r]:qsl[r + 1]]
        yb = b.out[qsl2[i]:qsl2[i + 1]]
        if r >= nd:
            assert torch.equal(ya.view(torch.int16), yb.view(torch.int16)), r
        else:
            fa, fb = ya.float(), yb.float()
            rel = float((fa - fb).abs().max() / fa.abs().max())
            assert rel < SPLIT_REL[wl.act_dtype], (r, rel)
    expect = oracle_outputs(wl, t, snap, requests)
    err, _ = compare(wl, a.out, expect, qsl)
    assert err <= tol_of(wl), err


def test_aliased_prefix_blocks():
    """Two requests list the same physical blocks for a shared cached prefix."""
    _need_gpu()
    wl = S.random_batch(12, [64, 200], [(64, 30)], hq=8, hkv=2, d=128, act=torch.bfloat16)
    bt = wl.block_tables.copy()
    # requests 1 and 2 reuse request 0's first 4 blocks (64 cached tokens)
    bt[1, :4] = bt[0, :4]
    bt[2, :4] = bt[0, :4]
    wl = S.Workload(**{**wl.__dict__, "block_tables": bt})
    t = S.make_tensors(wl, DEV)
    snap = Snapshot(wl, t, list(range(wl.num_reqs)))
    st = PagedAttentionStep(wl, t)
    st.run()
    torch.cuda.synchronize()
    qsl, _, _, _ = oracle_metadata(wl)
    expect = oracle_outputs(wl, t, snap, list(range(wl.num_reqs)))
    err, _ = compare(wl, st.out, expect, qsl)
    assert err <= tol_of(wl), err


@pytest.mark.parametrize("kind", ["act", "fp8", "int8"])
@pytest.mark.parametrize("hq,hkv,d,act", [(8, 2, 128, torch.bfloat16), (32, 1, 128, torch.bfloat16),
                                          (8, 8, 64, torch.float16)])
def test_absent_blocks(kind, hq, hkv, d, act):
    """Table entries outside the pool (negative or past it) hold no keys: decode
    and prefill leave those keys out, a row with no visible key is zero, and
    the cache write skips tokens whose block is absent."""
    _need_gpu()
    wl = S.random_batch(13 + d + hq, [40, 100, 31, 500], [(0, 70), (33, 64), (200, 90), (0, 20)],
                        hq=hq, hkv=hkv, d=d, act=act, fp8=kind == "fp8", int8=kind == "int8", pad=3)
    t = S.make_tensors(wl, DEV, poison=True)
    bt = wl.block_tables.copy()
    pool = wl.pool_blocks
    bt[0, 1] = -1                 # decode: a middle block
    bt[1, 6] = -1                 # decode: the block of this step's token
    bt[2, :2] = -1                # decode: every block -> zero output
    bt[3, 0] = pool + 5           # decode: past the pool
    bt[3, 17] = 2 ** 30
    bt[4, 2] = -1                 # prefill: a block of its new tokens
    bt[5, 0] = -1                 # prefill: a block of its cached prefix
    bt[6, 12] = pool + 1
    bt[6, 13] = -3
    bt[7, 0] = -1                 # prefill: its first 16 queries see no key
    wl = S.Workload(**{**wl.__dict__, "block_tables": bt})
    t = S.Tensors(q=t.q, k_new=t.k_new, v_new=t.v_new, key_cache=t.key_cache,
                  value_cache=t.value_cache, num_computed=t.num_computed, query_lens=t.query_lens,
                  block_tables=torch.from_numpy(bt).to(DEV), k_scale=t.k_scale, v_scale=t.v_scale)
    requests = list(range(wl.num_reqs))
    snap = Snapshot(wl, t, requests)
    st = PagedAttentionStep(wl, t)
    print(f"[absent] kind={kind} hq={hq} hkv={hkv} d={d}", flush=True)
    st.run()
    torch.cuda.synchronize()
    qsl, _, _, _ = oracle_metadata(wl)
    expect = oracle_outputs(wl, t, snap, requests)
    assert not np.any(expect[2])                       # the oracle's own zero row
    err, _ = compare(wl, st.out, expect, qsl)
    assert err <= tol_of(wl), err
    assert torch.all(st.out[qsl[2]:qsl[3]] == 0)       # every block absent
    assert torch.all(st.out[qsl[7]:qsl[7] + 16] == 0)  # queries with no visible key


@pytest.mark.parametrize("kind", ["act", "fp8", "int8"])
@pytest.mark.parametrize("hq,hkv,d,act", [(8, 2, 128, torch.bfloat16), (8, 8, 64, torch.float16)])
def test_prefill_rising_scores(kind, hq, hkv, d, act):
    """Prefill rows whose score maxima rise after their first 64-key tile (the
    tile that sets each row's reference max): by about 10 in log2 units (just
    past the lazy-rescale threshold of 8), by about 40, and by more than 128
    (exp2 against the old reference would overflow).  Every query of a request
    shares one sign pattern per K/V head (amplitude qa); spike keys are that
    pattern times an amplitude, in the cached prefix and among the new tokens."""
    _need_gpu()
    wl = S.random_batch(31 + d, [30], [(0, 300), (100, 200), (150, 100)], hq=hq, hkv=hkv, d=d,
                        act=act, fp8=kind == "fp8", int8=kind == "int8")
    t = S.make_tensors(wl, DEV)
    G = wl.group
    qsl, _, _, _ = oracle_metadata(wl)
    rng = np.random.default_rng(17)
    # random keys score ~N(0, qa^2) (natural units); a spike of amplitude a
    # scores a * qa * sqrt(d); 8-bit formats saturate near 4.4 (the scale's amax)
    qa = 2.5 if d == 128 else 3.0
    a1 = 0.45 if d == 128 else 0.6
    spikes = {1: [(70, a1), (150, 1.5)],        # new tokens: a small, then a large rise
              2: [(230, 4.5)],                  # new token: exp2 overflow
              3: [(100, 1.5), (210, 4.5)]}      # cached prefix, then a new token
    for r, keys in spikes.items():
        n = int(qsl[r + 1] - qsl[r])
        c = int(wl.seq_lens_host[r]) - n
        sign = torch.from_numpy(rng.choice([-1.0, 1.0], size=(hkv, d))).float()
        t.q[qsl[r]:qsl[r + 1]] = (qa * sign).repeat_interleave(G, dim=0).to(act).to(DEV)
        for pos, amp in keys:
            k = amp * sign
            if pos >= c:
                t.k_new[qsl[r] + pos - c] = k.to(act).to(DEV)
            else:
                slot = _slot(wl, r, pos)
                t.key_cache[slot // wl.block_size, slot % wl.block_size] = _enc(wl, k, t.k_scale).to(DEV)
    requests = list(range(wl.num_reqs))
    snap = Snapshot(wl, t, requests)
    st = PagedAttentionStep(wl, t)
    print(f"[rising] kind={kind} hq={hq} hkv={hkv} d={d}", flush=True)
    st.run()
    torch.cuda.synchronize()
    expect = oracle_outputs(wl, t, snap, requests)
    err, _ = compare(wl, st.out, expect, qsl)
    assert err <= tol_of(wl), err
