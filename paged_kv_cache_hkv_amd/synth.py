"""Seeded synthetic inputs for the paged-attention path.

This module only draws inputs: request lengths, block tables and tensor
values.  It holds none of the attention arithmetic (no slot mapping, no
scatter, no softmax, no 8-bit encoder of the method); tests and the benchmark
feed what it draws both to the HIP library and to the oracle.

Workloads (shapes follow the walkthrough pages and the five measured
configurations):

* ``walkthrough``  -- the 3-request step of "Tour: One forward pass": R1
  decodes after 540 cached tokens, R2 after 129, R3 prefills 298 tokens;
  Hq = Hkv = 8, head_dim 64, fp16, a 2048-block pool.
* ``decode_mha``   -- 64 decodes, cached length uniform in [512, 4096];
  Hq = Hkv = 32, head_dim 128, fp16, 65536-block pool.
* ``decode_gqa``   -- 256 decodes, cached length log-uniform in [1024, 8192];
  Hq = 32, Hkv = 8, head_dim 128, bf16, pool twice the blocks needed.
* ``chunked_prefill_mix`` -- 6 prefill chunks of 512..2048 new tokens after
  0..4096 cached ones (redrawn as a set until they total at most 8191), then
  enough 1-token decodes (cached 256..8192) to reach 8192 scheduled tokens;
  decodes first; Hq = 32, Hkv = 8, head_dim 128, bf16.
* ``mqa_fp8_long`` -- 32 decodes after 32768 cached tokens; Hq = 32, Hkv = 1,
  head_dim 128, bf16 queries, fp8 e4m3 K/V with per-tensor scales, a
  131072-block pool.

Block tables: one seeded permutation of the pool; request r takes the next
blocks it needs (its length divided by the block size, rounded up), in batch
order; unused table entries are -1.  Tensor values are N(0, 1) draws in
float32 from a seeded torch generator on the target device, rounded to the
activation dtype.  Every block a table lists is filled with such draws; all
other pool blocks are filled with NaN (0x7F for fp8), so a kernel that reads
outside the table shows up.  With ``poison`` the slots of each request's last
listed block that lie at or past its sequence length are poisoned the same
way (NaN / 0x7F / -128), so a read of a key past the sequence shows up too
(for int8, -128 is finite: such a read only shows up through the error it
adds).  For fp8 caches the per-tensor scale is float32(amax / 448) of the
drawn values and the stored codes come from torch's own float8_e4m3fn cast.  For int8 caches the scale is
float32(amax / 127) and the stored codes are the drawn values divided by the
scale, rounded by torch.round and clamped to -127..127: the generator's own
quantisation (the codes and the scale are simply inputs); unused blocks hold
-128, a code the write path never produces.
"""

from dataclasses import dataclass, field, replace

import numpy as np
import torch


@dataclass
class Workload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    act_dtype: torch.dtype
    cache_kind: str               # "act" (the activation dtype), "fp8_e4m3" or "int8"
    pool_blocks: int
    num_computed: np.ndarray      # int32 [R]
    query_lens: np.ndarray        # int32 [R]
    num_decodes: int              # requests [0, num_decodes) have query_len 1
    block_tables: np.ndarray      # int32 [R, W]
    seed: int
    num_tokens_padded: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def cache_fp8(self):
        return self.cache_kind == "fp8_e4m3"

    @property
    def cache_int8(self):
        return self.cache_kind == "int8"

    @property
    def cache_8bit(self):
        return self.cache_kind in ("fp8_e4m3", "int8")

    @property
    def cache_elem_bytes(self):
        return 1 if self.cache_8bit else 2

    @property
    def num_reqs(self):
        return int(self.query_lens.shape[0])

    @property
    def seq_lens_host(self):
        return (self.num_computed.astype(np.int64) + self.query_lens).astype(np.int64)

    @property
    def num_tokens(self):
        return int(self.query_lens.sum())

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_query_len(self):
        return int(self.query_lens.max()) if self.num_reqs else 0

    @property
    def max_seq_len(self):
        return int(self.seq_lens_host.max()) if self.num_reqs else 0


def _blocks_needed(length, block_size):
    return (int(length) + block_size - 1) // block_size


def block_tables_from_lengths(rng, lengths, block_size, pool_blocks, width=None):
    """Rows of physical block ids: one permutation of the pool, handed out in order."""
    need = [_blocks_needed(s, block_size) for s in lengths]
    total = int(sum(need))
    if total > pool_blocks:
        raise ValueError(f"pool of {pool_blocks} blocks cannot hold {total}")
    if width is None:
        width = max(need) if need else 1
    width = max(width, 1)
    perm = rng.permutation(pool_blocks).astype(np.int32)
    table = np.full((len(lengths), width), -1, dtype=np.int32)
    k = 0
    for r, nb in enumerate(need):
        table[r, :nb] = perm[k:k + nb]
        k += nb
    return table


def _kind(fp8=False, int8=False):
    if fp8 and int8:
        raise ValueError("one cache format at a time")
    return "fp8_e4m3" if fp8 else ("int8" if int8 else "act")


def _finish(name, rng, hq, hkv, d, bs, act, kind, pool, comp, ql, num_decodes, seed, pad_to=None,
            width=None, meta=None):
    comp = np.asarray(comp, dtype=np.int32)
    ql = np.asarray(ql, dtype=np.int32)
    lengths = comp.astype(np.int64) + ql
    bt = block_tables_from_lengths(rng, lengths, bs, pool, width)
    T = int(ql.sum())
    return Workload(name, hq, hkv, d, bs, act, kind, pool, comp, ql, num_decodes, bt, seed,
                    num_tokens_padded=pad_to if pad_to is not None else T, meta=meta or {})


def walkthrough(seed=1):
    rng = np.random.default_rng(seed)
    return _finish("walkthrough", rng, 8, 8, 64, 16, torch.float16, "act", 2048,
                   [540, 129, 0], [1, 1, 298], 2, seed, pad_to=304)


def decode_mha(seed=2):
    rng = np.random.default_rng(seed)
    comp = rng.integers(512, 4096, size=64, endpoint=True)
    return _finish("decode_mha", rng, 32, 32, 128, 16, torch.float16, "act", 65536,
                   comp, np.ones(64, np.int32), 64, seed)


def _pool_twice(lengths, bs):
    need = sum(_blocks_needed(s, bs) for s in lengths)
    return int(-(-2 * need // 1024) * 1024)


def decode_gqa(seed=3):
    rng = np.random.default_rng(seed)
    comp = np.rint(np.exp(rng.uniform(np.log(1024), np.log(8192), size=256))).astype(np.int32)
    pool = _pool_twice(comp + 1, 16)
    return _finish("decode_gqa", rng, 32, 8, 128, 16, torch.bfloat16, "act", pool,
                   comp, np.ones(256, np.int32), 256, seed)


def chunked_prefill_mix(seed=4, budget=8192, num_chunks=6):
    rng = np.random.default_rng(seed)
    while True:
        n = rng.integers(512, 2048, size=num_chunks, endpoint=True)
        if n.sum() <= budget - 1:
            break
    c_pre = rng.integers(0, 4096, size=num_chunks, endpoint=True)
    num_dec = int(budget - n.sum())
    c_dec = rng.integers(256, 8192, size=num_dec, endpoint=True)
    comp = np.concatenate([c_dec, c_pre]).astype(np.int32)
    ql = np.concatenate([np.ones(num_dec, np.int64), n]).astype(np.int32)
    pool = _pool_twice(comp.astype(np.int64) + ql, 16)
    return _finish("chunked_prefill_mix", rng, 32, 8, 128, 16, torch.bfloat16, "act", pool,
                   comp, ql, num_dec, seed)


def mqa_fp8_long(seed=5):
    rng = np.random.default_rng(seed)
    return _finish("mqa_fp8_long", rng, 32, 1, 128, 16, torch.bfloat16, "fp8_e4m3", 131072,
                   np.full(32, 32768, np.int32), np.ones(32, np.int32), 32, seed)


def with_cache(wl, kind):
    """The same workload over another cache format ("act", "fp8_e4m3", "int8")."""
    _kind(kind == "fp8_e4m3", kind == "int8")
    if kind not in ("act", "fp8_e4m3", "int8"):
        raise ValueError(kind)
    base = wl.name.replace("_fp8", "")
    suffix = "" if kind == "act" else "_" + kind.split("_")[0]
    return replace(wl, cache_kind=kind, name=base + suffix)


CONFIGS = {
    "walkthrough": walkthrough,
    "decode_mha": decode_mha,
    "decode_gqa": decode_gqa,
    "chunked_prefill_mix": chunked_prefill_mix,
    "mqa_fp8_long": mqa_fp8_long,
}


def random_batch(seed, decode_cached=(), prefills=(), hq=8, hkv=2, d=128, act=torch.bfloat16,
                 fp8=False, pool=None, pad=0, width=None, block_size=16, int8=False):
    """A small mixed batch: decodes (cached lengths) first, then (cached, new) prefills."""
    rng = np.random.default_rng(seed)
    comp = list(decode_cached) + [c for c, _ in prefills]
    ql = [1] * len(decode_cached) + [n for _, n in prefills]
    lengths = np.asarray(comp, np.int64) + np.asarray(ql, np.int64)
    need = sum(_blocks_needed(s, block_size) for s in lengths)
    if pool is None:
        pool = max(64, 2 * need + 16)
    T = int(sum(ql))
    return _finish(f"random{seed}", rng, hq, hkv, d, block_size, act, _kind(fp8, int8), pool,
                   comp, ql,
                   len(decode_cached), seed, pad_to=T + pad, width=width)


@dataclass
class Tensors:
    q: torch.Tensor              # [T_pad, Hq, D] act dtype
    k_new: torch.Tensor          # [T_pad, Hkv, D] act dtype
    v_new: torch.Tensor
    key_cache: torch.Tensor      # [NB, bs, Hkv, D] act dtype, uint8 (fp8 codes) or int8
    value_cache: torch.Tensor
    num_computed: torch.Tensor   # int32 [R]
    query_lens: torch.Tensor     # int32 [R]
    block_tables: torch.Tensor   # int32 [R, W]
    k_scale: float = 1.0
    v_scale: float = 1.0
    # per K/V head scales of a quantized cache (float32 device tensors [Hkv]),
    # used in place of k_scale / v_scale when set
    k_scales: object = None
    v_scales: object = None


def with_head_scales(t, seed, k=True, v=True):
    """The same tensors read with per-K/V-head scales: head h's scale is the
    tensor scale times a factor in [2^-1.5, 2^1.5] (drawn per seed), so the
    pool's codes stand for other values and new rows are written with other
    inverse scales (some saturating)."""
    hkv = t.key_cache.shape[2]
    rng = np.random.default_rng(seed)
    dev = t.key_cache.device
    def draw(base):
        f = np.exp2(rng.uniform(-1.5, 1.5, size=hkv))
        return torch.from_numpy((np.float32(base) * f).astype(np.float32)).to(dev)
    return replace(t, k_scales=draw(t.k_scale) if k else None, v_scales=draw(t.v_scale) if v else None)


def _randn(gen, shape, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _poison_value(cache):
    if cache.dtype == torch.uint8:
        return 0x7F           # fp8 e4m3fn NaN
    if cache.dtype == torch.int8:
        return -128           # a code the write path never produces
    return float("nan")


def tail_slots(wl):
    """(block, slot) pairs past each request's sequence in its last listed block."""
    bs = wl.block_size
    blocks, slots = [], []
    for r, s in enumerate(wl.seq_lens_host.tolist()):
        if s <= 0 or s % bs == 0:
            continue
        b = int(wl.block_tables[r, (s - 1) // bs])
        if 0 <= b < wl.pool_blocks:
            for o in range(s % bs, bs):
                blocks.append(b)
                slots.append(o)
    return np.asarray(blocks, np.int64), np.asarray(slots, np.int64)


def _poison_tails(wl, kc, vc, device):
    blocks, slots = tail_slots(wl)
    if blocks.size == 0:
        return
    bi = torch.from_numpy(blocks).to(device)
    si = torch.from_numpy(slots).to(device)
    for cache in (kc, vc):
        cache[bi, si] = _poison_value(cache)


def make_tensors(wl, device, poison=True, chunk_blocks=8192):
    """Draw every tensor of the workload on ``device`` (deterministic per seed)."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(wl.seed) * 1000003 + 17)
    T_pad = max(wl.num_tokens_padded, wl.num_tokens)
    hq, hkv, d, bs = wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size
    act = wl.act_dtype
    q = _randn(gen, (T_pad, hq, d), device).to(act)
    k_new32 = _randn(gen, (T_pad, hkv, d), device)
    v_new32 = _randn(gen, (T_pad, hkv, d), device)
    k_new, v_new = k_new32.to(act), v_new32.to(act)

    used = np.unique(wl.block_tables[wl.block_tables >= 0]).astype(np.int64)
    used_t = torch.from_numpy(used).to(device)
    pool_shape = (wl.pool_blocks, bs, hkv, d)
    if wl.cache_8bit:
        fp8 = wl.cache_fp8
        code_max = 448.0 if fp8 else 127.0
        cdt = torch.uint8 if fp8 else torch.int8
        kc = torch.empty(pool_shape, dtype=cdt, device=device)
        vc = torch.empty(pool_shape, dtype=cdt, device=device)
        kc.fill_((0x7F if fp8 else -128) if poison else 0)
        vc.fill_((0x7F if fp8 else -128) if poison else 0)
        # amax over every drawn value of the tensor (pool blocks and new tokens)
        scales = []
        for cache, new32 in ((kc, k_new32), (vc, v_new32)):
            state = gen.get_state()
            amax = new32.to(act).float().abs().max()
            for lo in range(0, used.size, chunk_blocks):
                ids = used_t[lo:lo + chunk_blocks]
                vals = _randn(gen, (ids.numel(), bs, hkv, d), device).to(act).float()
                amax = torch.maximum(amax, vals.abs().max())
            scale = float(np.float32(amax.item()) / np.float32(code_max))
            gen.set_state(state)
            inv = np.float32(1.0) / np.float32(scale)
            for lo in range(0, used.size, chunk_blocks):
                ids = used_t[lo:lo + chunk_blocks]
                vals = _randn(gen, (ids.numel(), bs, hkv, d), device).to(act).float()
                if fp8:
                    y = torch.clamp(vals * float(inv), -448.0, 448.0)
                    cache[ids] = y.to(torch.float8_e4m3fn).view(torch.uint8)
                else:
                    cache[ids] = torch.clamp(torch.round(vals / scale), -127, 127).to(torch.int8)
            scales.append(scale)
        k_scale, v_scale = scales
    else:
        kc = torch.empty(pool_shape, dtype=act, device=device)
        vc = torch.empty(pool_shape, dtype=act, device=device)
        if poison:
            kc.fill_(float("nan"))
            vc.fill_(float("nan"))
        else:
            kc.zero_()
            vc.zero_()
        for cache in (kc, vc):
            for lo in range(0, used.size, chunk_blocks):
                ids = used_t[lo:lo + chunk_blocks]
                cache[ids] = _randn(gen, (ids.numel(), bs, hkv, d), device).to(act)
        k_scale = v_scale = 1.0
    if poison:
        _poison_tails(wl, kc, vc, device)
    return Tensors(
        q=q, k_new=k_new, v_new=v_new, key_cache=kc, value_cache=vc,
        num_computed=torch.from_numpy(wl.num_computed.astype(np.int32)).to(device),
        query_lens=torch.from_numpy(wl.query_lens.astype(np.int32)).to(device),
        block_tables=torch.from_numpy(wl.block_tables.astype(np.int32)).to(device),
        k_scale=k_scale, v_scale=v_scale)
