"""The read-bandwidth probe (kvq_read_probe) reads exactly the quantized head blocks the split-K decode reads.

Each walk's XOR of 32-bit words is recomputed on the CPU from a host copy of the pages, the page table and
the decode's chunking (kvq_decode_shape_of): walk w of a sequence's n_chunks chunks takes chunks
w n / walks .. (w + 1) n / walks - 1, i.e. its groups up to the sequence's quantized group count, each group
the two pages 2 g, 2 g + 1 of the page-table row.  Integer work: compared bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle as O
import synth
from kvq_cases import build_cache, head_bytes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import decode_attention_15_amd as K
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return K


def _say(msg):
    print(msg, flush=True)


def balanced_gpc(ngs, quads, nwg, floor=4):
    """The decode's balanced chunk size, restated from the header's rule: the smallest G >= 4 whose chunks,
    ceil(groups / G) per (sequence, head quad), fit the nwg chunk work-groups."""
    chunks = lambda G: sum(-(-n // G) for n in ngs) * quads
    G = max(floor, -(-sum(ngs) * quads // nwg))
    while chunks(G) > nwg:
        G += 1
    return G


def _xor(pages, pt, b, h, groups, hb, pb):
    acc = np.uint32(0)
    for g in groups:
        for p in (pt[b, 2 * g], pt[b, 2 * g + 1]):
            blk = pages[int(p) * pb + h * hb:int(p) * pb + (h + 1) * hb]
            acc ^= np.bitwise_xor.reduce(blk.view(np.uint32))
    return acc


def _expected(bc, shape, max_len):
    """Expected slots; under balanced chunking the slots past a sequence's chunk count keep -1."""
    pages = bc.cache.pages.cpu().numpy()
    pt = bc.cache.page_table.cpu().numpy().reshape(len(bc.lens), -1)
    wl = bc.wl
    hb = head_bytes(wl.scheme)
    pb = hb * wl.n_kv_heads
    if shape["balanced"]:
        slots = shape["max_chunks"]
        want = np.full((len(bc.lens), wl.n_kv_heads, slots), 0xFFFFFFFF, dtype=np.uint32)
        cap = min(slots * 4, pt.shape[1] // 2)  # the launch bound at the 4-group floor, the page-table row
        ngs = [min(O.n_groups(int(T), wl.n_sink, wl.n_recent), cap) for T in bc.lens]
        nwg = shape["splitk_workgroups"] - len(bc.lens) * wl.n_kv_heads
        G = balanced_gpc(ngs, wl.n_kv_heads // 4, nwg)
        for b, ng in enumerate(ngs):
            for c in range(-(-ng // G)):
                for h in range(wl.n_kv_heads):
                    want[b, h, c] = _xor(pages, pt, b, h, range(c * G, min((c + 1) * G, ng)), hb, pb)
        return want
    nc, walks, gpc = shape["n_chunks"], shape["walks"], shape["chunk_units"]
    want = np.zeros((len(bc.lens), wl.n_kv_heads, walks), dtype=np.uint32)
    for b, T in enumerate(bc.lens):
        ng = min(O.n_groups(int(T), wl.n_sink, wl.n_recent), pt.shape[1] // 2)
        for w in range(walks):
            g0 = (w * nc // walks) * gpc
            g1 = min(((w + 1) * nc // walks) * gpc, ng)
            for h in range(wl.n_kv_heads):
                want[b, h, w] = _xor(pages, pt, b, h, range(g0, g1), hb, pb)
    return want


def _slots(shape):
    return shape["max_chunks"] if shape["balanced"] else shape["walks"]


@pytest.mark.parametrize("name,kw,lens,split", [
    ("gqa_b1_32k", {}, [5000, 100, 9000], 0),                               # head quads, one empty sequence
    ("tiny_1h_4k", {}, [4096], 0),                                          # one kv head: walks per wave
    ("gqa_b1_32k", dict(scheme="int4_channel"), [3000, 6100], 0),           # 4-bit codes: 8704-byte head blocks
    ("batch32_32k", dict(n_q_heads=8, n_kv_heads=2), [2000, 3900, 0, 2600] * 4, 256),  # two kv heads, split
    ("batch32_32k", {}, [9000, 700, 0, 6100, 2600, 4000, 300, 8200] * 4, 0),  # balanced: ragged, several G
])
def test_probe_reads_the_decode_bytes(K, name, kw, lens, split):
    import torch
    wl = synth.scaled(synth.WORKLOADS[name], batch=len(lens), **kw)
    lens = np.asarray(lens, dtype=np.int64)
    bc = build_cache(K, wl, lens, split_tokens=split)
    max_len = int(lens.max())
    shape = K.decode_shape(bc.cfg, len(lens), max_len)
    _say(f"probe: {name} {kw} lens {lens.tolist()} split {split}: {shape}")
    out = torch.full((len(lens), wl.n_kv_heads, _slots(shape)), -1, dtype=torch.int32, device="cuda")
    K.read_probe(bc.cache, out, max_len)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    want = _expected(bc, shape, max_len)
    assert np.array_equal(got, want), f"{np.argwhere(got != want)[:5].tolist()}"


def test_probe_walks_several_chunks(K):
    """An explicit 512-token split with more chunks than one round of work-groups holds: walks of several
    chunks (span >= 2), ragged lengths with two empty sequences."""
    import torch
    batch = 32
    wl = synth.scaled(synth.WORKLOADS["batch32_32k"], batch=batch)
    rng = np.random.default_rng(batch * 7919 + 3000)
    lens = rng.integers(3000, 7001, size=batch)
    lens[3] = 0
    lens[batch - 2] = 0
    bc = build_cache(K, wl, lens, split_tokens=512, decode_impl=K.DECODE_MFMA, seqs_per_call=8)
    max_len = int(lens.max())
    shape = K.decode_shape(bc.cfg, batch, max_len)
    _say(f"probe: batch {batch}, lens {lens.min()}..{lens.max()}, split 512: {shape}")
    assert shape["span"] >= 2
    out = torch.full((batch, wl.n_kv_heads, _slots(shape)), -1, dtype=torch.int32, device="cuda")
    K.read_probe(bc.cache, out, max_len)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, _expected(bc, shape, max_len))
