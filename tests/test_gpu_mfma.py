"""GPU parity of the matrix-core decode (DECODE_MFMA), every scheme: the split-K kernel's per-group sums over
channels and tokens on v_mfma_i32_16x16x64_i8 with three-limb (22-bit or 20-bit) operands, against the fp64
oracle on the same seeded caches (bar 2e-3), and against the fp32 decode of the same cache where it exists.

Cases span every GQA ratio the kernel lays out differently (1, 2 and 4: four matrix rows per head; 8: two
rows per head plus a tile of top limbs), automatic and explicit splits (every wave walks a chunk of its
own; with more chunks than one round of work-groups holds, several in a row), ragged and empty sequences,
and appends that demote groups.  The full-size shapes are in test_gpu_wide_parity.py.
"""
import numpy as np
import pytest

import synth
from kvq_cases import TOL, _host, _say, build_cache, check_int2, check_out, run_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_15_amd as K
    return K


def _case(K, wl, lens, heads, append_steps=0, chunk=None, split=0, check_codes=True):
    bc = build_cache(K, wl, lens, append_steps=append_steps, chunk=chunk, split_tokens=split,
                     decode_impl=K.DECODE_MFMA)
    if check_codes:
        pages, band = _host(bc)
        for b in range(len(lens)):
            if lens[b]:
                for h in heads:
                    check_int2(bc, b, h, pages=pages, band=band)
    q = synth.queries(synth.scaled(wl, batch=len(lens)))
    out = run_decode(K, bc, q)
    worst = check_out(bc, out, q, [(b, h) for b in range(len(lens)) for h in range(wl.n_kv_heads)])
    _say(f"   worst |mfma - oracle| = {worst:.2e}")
    return bc, q, out


def test_mfma_single_head_fp32_source(K):
    wl = synth.WORKLOADS["tiny_1h_4k"]
    _say("mfma: tiny 1 head (GQA 1), T=4096, fp32 source with x10 outlier channels, 96 appends")
    _case(K, wl, [4096], [0], append_steps=96)


def test_mfma_gqa4_ragged_with_appends(K):
    wl = synth.WORKLOADS["gqa_b1_32k"]
    lens = [3000, 131, 700, 0, 260, 2051]
    _say(f"mfma: GQA 4 ragged lens={lens}, 5 appends")
    _case(K, wl, lens, [0, 3, 7], append_steps=5)


def test_mfma_gqa2_ragged(K):
    wl = synth.scaled(synth.WORKLOADS["gqa_b1_32k"], n_q_heads=16, n_kv_heads=8)
    lens = [2900, 1000, 133, 0]
    _say(f"mfma: GQA 2 lens={lens}, 3 appends")
    _case(K, wl, lens, [0, 5], append_steps=3)


@pytest.mark.parametrize("split", [0, 512])
def test_mfma_gqa8_decaying_spectrum(K, split):
    wl = synth.scaled(synth.WORKLOADS["long_b4_131k"], batch=2)
    lens = [5000, 2222]
    _say(f"mfma: GQA 8, sigma_c = (c+1)^-0.5, lens={lens}, split {split}")
    _case(K, wl, lens, [0, 5], append_steps=3, split=split)


@pytest.mark.parametrize("split", [128, 256, 1024])
def test_mfma_gqa4_explicit_splits(K, split):
    """Explicit splits: each wave walks a chunk of its own (one or more groups) and stores its partial."""
    wl = synth.WORKLOADS["batch32_32k"]
    lens = [4100, 2000, 260, 1029, 3000, 388, 9000]
    _say(f"mfma: GQA 4 lens={lens}, split {split}, 800-token prefill chunks")
    _case(K, wl, lens, [2], chunk=800, split=split, check_codes=False)


@pytest.mark.parametrize("name,kw,batch,lo,hi", [
    ("batch32_32k", {}, 32, 3000, 7000),                          # GQA 4, head quads
    ("long_b4_131k", {}, 16, 11000, 14000),                       # GQA 8, head quads
    ("saw_int4_b16_16k", {}, 32, 4000, 7000),                     # INT4 per token: page pairs
    ("batch32_32k", dict(n_q_heads=8, n_kv_heads=2), 64, 9000, 12000),  # two kv heads: four walks per work-group
])
def test_mfma_walks_several_chunks(K, name, kw, batch, lo, hi):
    """An explicit 512-token split with more chunks than one round of work-groups holds: each wave walks
    several consecutive chunks, storing a partial at every chunk boundary.  Ragged lengths (two of them empty)
    put the boundaries and the ends of the walks everywhere; the whole output is compared with the fp32
    decode of the same cache (one chunk per work-group) and sampled heads with the oracle."""
    wl = synth.scaled(synth.WORKLOADS[name], batch=batch, **kw)
    rng = np.random.default_rng(batch * 7919 + lo)
    lens = rng.integers(lo, hi + 1, size=batch)
    lens[3] = 0
    lens[batch - 2] = 0
    bc = build_cache(K, wl, lens, split_tokens=512, decode_impl=K.DECODE_MFMA, seqs_per_call=8)
    shape = K.decode_shape(bc.cfg, batch, int(lens.max()))
    _say(f"mfma: {name} {kw} batch {batch}, lens {lens.min()}..{lens.max()}, split 512: {shape}")
    assert shape["matrix_cores"] == 1 and shape["span"] >= 2
    q = synth.queries(wl)
    out = run_decode(K, bc, q)
    assert np.isfinite(out).all()
    bc.cfg.decode_impl = K.DECODE_F32
    ref = run_decode(K, bc, q)
    bc.cfg.decode_impl = K.DECODE_MFMA
    d32 = np.abs(out - ref).max()
    _say(f"   max |mfma - f32| over all heads = {d32:.2e}")
    assert d32 <= TOL
    pairs = [(b, h) for b in (0, 3, 5, batch // 2, batch - 1) for h in (0, wl.n_kv_heads - 1)]
    worst = check_out(bc, out, q, pairs)
    _say(f"   worst |mfma - oracle| = {worst:.2e}")


@pytest.mark.parametrize("name,kw,batch,lo,hi", [
    ("batch32_32k", {}, 32, 300, 9000),                            # GQA 4
    ("long_b4_131k", dict(split_tokens=0), 16, 1000, 12000),        # GQA 8
    ("batch32_32k", dict(scheme="int4_channel"), 16, 300, 6000),   # 4-bit codes
    ("batch32_32k", {}, 256, 300, 2500),                           # GQA 4, more work-groups than one round
    ("long_b4_131k", dict(split_tokens=0), 192, 300, 2000),         # GQA 8, likewise
])
def test_balanced_chunking_ragged(K, name, kw, batch, lo, hi):
    """Automatic chunks chosen on the device from the batch's lengths (balanced chunking): ragged lengths, two of
    them without a quantized group, put the chunk size between the 4-group floor and the longest sequence; the
    whole output is compared with the fp32 decode of the same cache and sampled heads with the oracle.  The large
    batches have more (sequence, head quad) rows than chunk slots and more work-groups than one round holds: the
    band work-groups go first."""
    wl = synth.scaled(synth.WORKLOADS[name], batch=batch, **kw)
    rng = np.random.default_rng(batch * 131 + lo)
    lens = rng.integers(lo, hi + 1, size=batch)
    lens[1] = 0
    lens[batch - 3] = 200
    bc = build_cache(K, wl, lens, decode_impl=K.DECODE_MFMA, seqs_per_call=8)
    shape = K.decode_shape(bc.cfg, batch, int(lens.max()))
    _say(f"balanced: {name} {kw} batch {batch}, lens {lens.min()}..{lens.max()}: {shape}")
    assert shape["balanced"] == 1
    assert shape["band_first"] == (1 if batch >= 128 else 0)
    q = synth.queries(wl)
    out = run_decode(K, bc, q)
    assert np.isfinite(out).all()
    if wl.scheme == "int2_channel":  # the fp32 decode covers INT2 per channel and INT4 per token
        bc.cfg.decode_impl = K.DECODE_F32
        ref = run_decode(K, bc, q)
        bc.cfg.decode_impl = K.DECODE_MFMA
        d32 = np.abs(out - ref).max()
        _say(f"   max |mfma - f32| over all heads = {d32:.2e}")
        assert d32 <= TOL
    pairs = [(b, h) for b in (0, 1, 2, batch // 2, batch - 3, batch - 1) for h in (0, wl.n_kv_heads - 1)]
    worst = check_out(bc, out, q, pairs)
    _say(f"   worst |mfma - oracle| = {worst:.2e}")


def test_mfma_agrees_with_f32(K):
    """Same cache, two decodes: the matrix-core one (three-limb operands) close to the exact fp32 one."""
    for name, lens in (("tiny_1h_4k", [4096]), ("gqa_b1_32k", [2900, 1000]), ("long_b4_131k", [3000, 700])):
        wl = synth.WORKLOADS[name]
        bc = build_cache(K, wl, lens)
        q = synth.queries(synth.scaled(wl, batch=len(lens)))
        outs = {}
        for nm, c in (("f32", K.DECODE_F32), ("mfma", K.DECODE_MFMA)):
            bc.cfg.decode_impl = c
            outs[nm] = run_decode(K, bc, q)
        d32 = np.abs(outs["mfma"] - outs["f32"]).max()
        _say(f"mfma vs f32 on {name} lens={lens}: {d32:.2e}")
        assert d32 <= 2e-4


def test_mfma_is_deterministic(K):
    wl = synth.WORKLOADS["gqa_b1_32k"]
    bc = build_cache(K, wl, [2500, 900], decode_impl=K.DECODE_MFMA)
    q = synth.queries(synth.scaled(wl, batch=2))
    assert np.array_equal(run_decode(K, bc, q), run_decode(K, bc, q))


# ------------------------------------------------------------------ per-token INT2 on the matrix cores


def _tok(wl, **kw):
    return synth.scaled(wl, scheme="int2_token", **kw)


def test_mfma_int2_token_single_head_fp32_source(K):
    wl = _tok(synth.WORKLOADS["tiny_1h_4k"])
    _say("mfma per-token INT2: tiny 1 head (GQA 1), T=4096, fp32 source with x10 outlier channels, 40 appends")
    _case(K, wl, [4096], [0], append_steps=40)


def test_mfma_int2_token_gqa4_ragged_with_appends(K):
    wl = _tok(synth.WORKLOADS["gqa_b1_32k"])
    lens = [3000, 131, 700, 0, 260, 2051]
    _say(f"mfma per-token INT2: GQA 4 ragged lens={lens}, 5 appends")
    _case(K, wl, lens, [0, 3, 7], append_steps=5)


def test_mfma_int2_token_gqa2(K):
    wl = _tok(synth.WORKLOADS["gqa_b1_32k"], n_q_heads=16, n_kv_heads=8)
    lens = [2900, 1000, 133]
    _say(f"mfma per-token INT2: GQA 2 lens={lens}")
    _case(K, wl, lens, [0, 5])


@pytest.mark.parametrize("split", [0, 512])
def test_mfma_int2_token_gqa8_decaying_spectrum(K, split):
    wl = _tok(synth.WORKLOADS["long_b4_131k"], batch=2)
    lens = [5000, 2222]
    _say(f"mfma per-token INT2: GQA 8, sigma_c = (c+1)^-0.5, lens={lens}, split {split}")
    _case(K, wl, lens, [0, 5], append_steps=3, split=split)


def test_mfma_int2_token_workloads(K):
    for name, lens in (("tiny_1h_4k", [4096]), ("gqa_b1_32k", [2900, 1000]), ("long_b4_131k", [3000, 700])):
        wl = _tok(synth.WORKLOADS[name])
        bc = build_cache(K, wl, lens)
        q = synth.queries(synth.scaled(wl, batch=len(lens)))
        out = run_decode(K, bc, q)
        worst = check_out(bc, out, q, [(b, h) for b in range(len(lens)) for h in range(wl.n_kv_heads)])
        _say(f"per-token mfma on {name} lens={lens}: worst |mfma - oracle| = {worst:.2e}")


def test_mfma_int2_token_batch32_full_sampled(K):
    wl = _tok(synth.WORKLOADS["batch32_32k"])
    lens = synth.seq_lens(wl)
    _say("mfma per-token INT2: batch32_32k full")
    bc = build_cache(K, wl, lens, seqs_per_call=4, decode_impl=K.DECODE_MFMA)
    q = synth.queries(wl)
    out = run_decode(K, bc, q)
    assert np.isfinite(out).all()
    worst = check_out(bc, out, q, [(0, 0), (31, 7)])
    _say(f"   worst |mfma - oracle| = {worst:.2e}")


# ------------------------------------------------------------------ INT4 per token on the matrix cores


@pytest.mark.parametrize("split", [0, 128, 256])
def test_mfma_int4_token_small(K, split):
    """Lengths end inside a pair's second page, inside its first page (second page missing) and on a page
    boundary; automatic and explicit splits."""
    from kvq_cases import check_int4
    wl = synth.WORKLOADS["saw_int4_b16_16k"]
    lens = [1000, 333, 66, 40, 128, 1]
    _say(f"mfma int4 per token lens={lens} split={split}")
    bc = build_cache(K, wl, lens, append_steps=7, chunk=256, decode_impl=K.DECODE_MFMA, split_tokens=split)
    pages = bc.cache.pages.cpu().numpy()
    for b in (0, 2):
        check_int4(bc, b, 6, pages)
    q = synth.queries(synth.scaled(wl, batch=len(lens)))
    out = run_decode(K, bc, q)
    worst = check_out(bc, out, q, [(b, h) for b in range(len(lens)) for h in range(8)])
    _say(f"   worst |mfma - oracle| = {worst:.2e}")


@pytest.mark.parametrize("gq,block", [(1, 128), (2, 16), (8, 64)])
def test_mfma_int4_token_gqa_and_blocks(K, gq, block):
    wl = synth.scaled(synth.WORKLOADS["saw_int4_b16_16k"], n_q_heads=8 * gq, n_kv_heads=8, hadamard_block=block)
    lens = [700, 2049]
    _say(f"mfma int4 per token: GQA {gq}, Hadamard block {block}, lens={lens}")
    _case(K, wl, lens, [], chunk=512, check_codes=False)


def test_mfma_int4_token_agrees_with_f32(K):
    wl = synth.WORKLOADS["saw_int4_b16_16k"]
    lens = [1500, 300]
    bc = build_cache(K, wl, lens)
    q = synth.queries(synth.scaled(wl, batch=len(lens)))
    outs = {}
    for nm, c in (("f32", K.DECODE_F32), ("mfma", K.DECODE_MFMA)):
        bc.cfg.decode_impl = c
        outs[nm] = run_decode(K, bc, q)
    d32 = np.abs(outs["mfma"] - outs["f32"]).max()
    _say(f"int4 per token mfma vs f32: {d32:.2e}")
    assert d32 <= 2e-4


def test_mfma_int4_token_full_sampled(K):
    wl = synth.WORKLOADS["saw_int4_b16_16k"]
    _say("mfma int4 per token: B=16, T=16384, 8192-token prefill chunks")
    bc = build_cache(K, wl, [16384] * 16, chunk=8192, seqs_per_call=4, decode_impl=K.DECODE_MFMA)
    q = synth.queries(wl)
    out = run_decode(K, bc, q)
    assert np.isfinite(out).all()
    worst = check_out(bc, out, q, [(0, 0), (15, 7)])
    _say(f"   worst |mfma - oracle| = {worst:.2e}")


# ------------------------------------------------------------------ per-channel INT4 on the matrix cores


def _c4(wl, **kw):
    return synth.scaled(wl, scheme="int4_channel", **kw)


def test_mfma_int4_channel_single_head_fp32_source(K):
    _say("mfma per-channel INT4: tiny 1 head, T=4096, fp32 source with x10 outlier channels, 20 appends")
    _case(K, _c4(synth.WORKLOADS["tiny_1h_4k"]), [4096], [0], append_steps=20)


def test_mfma_int4_channel_gqa2_ragged_with_appends(K):
    wl = _c4(synth.WORKLOADS["gqa_b1_32k"], n_q_heads=16, n_kv_heads=8)
    lens = [2900, 1000, 133, 0]
    _say(f"mfma per-channel INT4: GQA 2, lens={lens}, 5 appends")
    _case(K, wl, lens, [0, 3, 7], append_steps=5)


@pytest.mark.parametrize("split", [0, 256])
def test_mfma_int4_channel_gqa4_batch(K, split):
    wl = _c4(synth.WORKLOADS["batch32_32k"])
    lens = [4100, 2000, 260, 1029, 3000, 388]
    _say(f"mfma per-channel INT4: GQA 4, lens={lens}, split {split}, 800-token prefill chunks, 2 appends")
    _case(K, wl, lens, [0, 5], append_steps=2, chunk=800, split=split)


def test_mfma_int4_channel_gqa8_decaying_spectrum(K):
    wl = _c4(synth.WORKLOADS["long_b4_131k"], batch=2)
    _say("mfma per-channel INT4: GQA 8, sigma_c = (c+1)^-0.5, lens [3000, 700], split 512")
    _case(K, wl, [3000, 700], [0, 5], chunk=1000, split=512)


def test_mfma_int4_channel_workloads(K):
    for name, lens in (("gqa_b1_32k", [2900, 1000]), ("long_b4_131k", [3000, 700])):
        wl = _c4(synth.WORKLOADS[name])
        bc = build_cache(K, wl, lens)
        q = synth.queries(synth.scaled(wl, batch=len(lens)))
        out = run_decode(K, bc, q)
        worst = check_out(bc, out, q, [(b, h) for b in range(len(lens)) for h in range(wl.n_kv_heads)])
        _say(f"per-channel INT4 mfma on {name}: worst |mfma - oracle| = {worst:.2e}")


def test_mfma_int4_channel_batch32_full_sampled(K):
    wl = _c4(synth.WORKLOADS["batch32_32k"])
    lens = synth.seq_lens(wl)
    _say("mfma per-channel INT4: batch32_32k full")
    bc = build_cache(K, wl, lens, seqs_per_call=4, decode_impl=K.DECODE_MFMA)
    q = synth.queries(wl)
    out = run_decode(K, bc, q)
    assert np.isfinite(out).all()
    worst = check_out(bc, out, q, [(0, 1), (31, 6)])
    _say(f"   worst |mfma - oracle| = {worst:.2e}")
