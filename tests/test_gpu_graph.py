"""The calls of one step captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed: every call only enqueues kernels on the given stream and allocates
nothing, so a captured step must reproduce the eager step bit for bit on every
replay.  The replays are interleaved with eager work and synchronisations,
and each one is checked (output rows and every cache byte)."""

import pytest
import torch

from paged_kv_cache_hkv_amd import binding as B
from paged_kv_cache_hkv_amd import synth as S
from paged_kv_cache_hkv_amd.step import PagedAttentionStep

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def _bits(t):
    return t.detach().contiguous().view(torch.uint8).clone()


@pytest.mark.parametrize("kind", ["act", "fp8", "int8"])
def test_captured_step_replays_bit_identical(kind):
    _need_gpu()
    wl = S.random_batch(71, [5, 40, 300, 1000], [(0, 70), (64, 100)], hq=16, hkv=4, d=128,
                        act=torch.bfloat16, fp8=kind == "fp8", int8=kind == "int8", pad=3)
    t = S.make_tensors(wl, DEV, poison=False)
    st = PagedAttentionStep(wl, t)
    st.run()                       # eager reference (also loads the library)
    torch.cuda.synchronize()
    want_out, want_k, want_v = _bits(st.out), _bits(t.key_cache), _bits(t.value_cache)

    g = torch.cuda.CUDAGraph()
    st.out.fill_(0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        st.run()
    torch.cuda.synchronize()
    scratch = torch.empty(1 << 20, device=DEV)
    for rep in range(3):
        st.out.fill_(0)            # eager work between replays
        scratch.normal_()
        torch.cuda.synchronize()
        print(f"[graph] kind={kind} replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(st.out), want_out), rep
        assert torch.equal(_bits(t.key_cache), want_k), rep
        assert torch.equal(_bits(t.value_cache), want_v), rep
