"""kv_decode_attn_noalloc (the decode that takes its workspace from the library's per-GPU scratch array)
against kv_decode_attn on the same cache and queries: two calls in a row, the second with a smaller input,
so the second runs over scratch the first left full of its partials.  Both entry points launch the same
kernels over the same grid, so the outputs agree bit for bit; sampled heads are also held to the oracle's
bar, and a decode whose workspace exceeds the scratch is refused before anything is enqueued.
"""
import ctypes

import numpy as np
import pytest

import synth
from kvq_cases import TOL, _say, build_cache, check_out, source_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_15_amd as K
    return K


def _both(K, bc, q_np):
    import torch
    q = source_torch(q_np, "cuda")
    maxT = int(bc.lens.max())
    ref = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    ws = K.workspace_for(bc.cfg, len(bc.lens), maxT, "cuda")
    K.kv_decode_attn(bc.cache, q, ref, maxT, ws)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    K.kv_decode_attn_noalloc(bc.cache, q, out, maxT)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), out.cpu().numpy()


@pytest.mark.parametrize("name,lens1,lens2,split", [
    ("gqa_b1_32k", [9000, 131, 4100, 0, 2600], [700, 300], 0),
    ("gqa_b1_32k", [6000, 5000, 260], [1000], 512),
    ("saw_int4_b16_16k", [5000, 77, 2000, 3000], [1500, 640], 0),
])
def test_noalloc_matches_workspace_decode(K, name, lens1, lens2, split):
    wl = synth.WORKLOADS[name]
    for step, lens in enumerate((lens1, lens2)):
        _say(f"no-alloc: {name} call {step + 1} lens={lens} split={split}")
        bc = build_cache(K, wl, lens, split_tokens=split)
        q = synth.queries(synth.scaled(wl, batch=len(lens)))
        ref, out = _both(K, bc, q)
        assert np.isfinite(out).all()
        assert np.array_equal(out, ref), f"max |noalloc - decode| = {np.abs(out - ref).max():.3e}"
        heads = [(b, h) for b in range(len(lens)) for h in (0, wl.n_kv_heads - 1)]
        worst = check_out(bc, out, q, heads)
        _say(f"   identical to kv_decode_attn; worst |noalloc - oracle| = {worst:.2e} (bar {TOL})")


def test_noalloc_refuses_beyond_the_page_table(K):
    import torch
    wl = synth.WORKLOADS["gqa_b1_32k"]
    bc = build_cache(K, wl, [300, 200], split_tokens=512)
    q = source_torch(synth.queries(synth.scaled(wl, batch=2)), "cuda")
    out = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    # a host-side maximum length beyond the page table: refused before any launch, the output untouched
    T = int(bc.lens.max())
    while K.pages_for_len(bc.cfg, T) <= bc.max_pages:
        T += 64
    with pytest.raises(K.KvqError) as ei:
        K.kv_decode_attn_noalloc(bc.cache, q, out, T)
    assert ei.value.status == K.KVQ_ERANGE
    torch.cuda.synchronize()
    assert float(out.abs().max()) == 0.0
