"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Bar: codes, bf16 scales/zeros and band bytes bit-exact; attention outputs within 2e-3 absolute.  The fp32
decode (DECODE_F32) differs from the fp64 oracle by fp32 rounding only; the default matrix-core decode also
rounds the key-side operand and the softmax weights to 22-bit (2-bit codes) or 20-bit (4-bit codes) integers,
far inside the bar.
"""
import sys

import numpy as np
import pytest

import oracle as O
import synth
from kvq_cases import (TOL, _host, _say, build_cache, check_int2, check_int4, check_out, oracle_out, read_band,
                       read_int2_group, read_int4_tokens, run_decode, source_of)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_15_amd as K
    return K


# ------------------------------------------------------------------------- stage-wise: rotation


@pytest.mark.parametrize("rotation", ["oscar", "saw", "saw16", "saw32", "saw64"])
@pytest.mark.parametrize("rho", [1.0, 0.96, 0.92, 0.89, 0.88, 0.5])
def test_debug_rotate_bit_exact(K, rotation, rho):
    """Rotation and per-token clip bit-exact against the oracle.  The clip's order statistics take two
    routes (the largest values visited one by one for rho >= 0.89, a bitwise search below), so the clip
    ratios cover both and their boundary; tokens 300..363 are built so that their rotated magnitudes repeat
    (one-hot and two-hot vectors, constant vectors, zeros), which the first route must count correctly."""
    import torch
    from kvq_cases import config_for, rotations, source_torch
    wl = synth.WORKLOADS["gqa_b1_32k" if rotation == "oscar" else "saw_int4_b16_16k"]
    block = int(rotation[3:]) if rotation.startswith("saw") and len(rotation) > 3 else 128
    wl = synth.scaled(wl, hadamard_block=block)
    _say(f"debug_rotate {rotation} rho={rho}")
    rk, rv = rotations(wl)
    cfg = config_for(K, wl)
    x = synth.kv_tokens(wl, 0, 0, 300, "k")[:, 0].copy()
    rep = np.zeros((64, 128), np.float32)
    for i in range(16):
        rep[i, (7 * i) % 128] = 1.0 + i                # one-hot
        rep[16 + i, i] = rep[16 + i, 127 - i] = -2.0    # two-hot
        rep[32 + i, :] = 0.25 * (i + 1)                 # constant
    x = np.concatenate([x, rep if x.dtype == np.float32 else synth.to_bf16_bits(rep)])
    pt = torch.zeros((1, 1), dtype=torch.int32)
    cache = K.allocate_cache(cfg, 1, pt, torch.from_numpy(rk), torch.from_numpy(rv), n_pages=1)
    out = torch.empty((x.shape[0], 128), dtype=torch.float32, device="cuda")
    K.kvq_debug_rotate(cache, 0, source_torch(x, "cuda"), rho, out)
    got = out.cpu().numpy()
    xv = O.bf16_value(x)
    want = O.rotate_dense(xv, rk) if rotation == "oscar" else O.rotate_hadamard(xv, rk.astype(np.int8), block)
    if rho < 1.0:
        want = O.clip_tokens(want, rho)
    bad = np.argwhere(got.view(np.uint32) != want.view(np.uint32))
    if len(bad):
        t, c = bad[0]
        _say(f"   got {got[t, c]!r} ({got.view(np.uint32)[t, c]:#x}) want {want[t, c]!r} ({want.view(np.uint32)[t, c]:#x})")
    assert len(bad) == 0, f"{len(bad)} mismatches in tokens {np.unique(bad[:, 0])[:10].tolist()}, first {bad[:3].tolist()}"


# ------------------------------------------------------------------------- small, element by element


def test_tiny_single_head_full(K):
    wl = synth.WORKLOADS["tiny_1h_4k"]
    _say("tiny_1h_4k: prefill 4000 + 96 appends, T=4096")
    bc = build_cache(K, wl, [4096], append_steps=96)
    check_int2(bc, 0, 0)
    q = synth.queries(synth.scaled(wl, batch=1))
    out = run_decode(K, bc, q)
    worst = check_out(bc, out, q, [(0, 0)])
    _say(f"  worst |diff| {worst:.2e}")


@pytest.mark.parametrize("impl", ["auto", "f32"])
def test_gqa_ragged_batch(K, impl):
    wl = synth.WORKLOADS["gqa_b1_32k"]
    lens = [3000, 131, 700, 0, 260]
    _say(f"gqa ragged lens={lens} impl={impl}")
    bc = build_cache(K, wl, lens, append_steps=5, decode_impl={"f32": K.DECODE_F32}.get(impl, K.DECODE_AUTO))
    pages, band = _host(bc)
    for b in range(len(lens)):
        for h in (0, 3, 7):
            if lens[b]:
                check_int2(bc, b, h, pages=pages, band=band)
    q = synth.queries(synth.scaled(wl, batch=len(lens)))
    out = run_decode(K, bc, q)
    check_out(bc, out, q, [(b, h) for b in range(len(lens)) for h in range(8)])


def test_prefill_and_appends_give_identical_bytes(K):
    wl = synth.WORKLOADS["gqa_b1_32k"]
    lens = [1500, 777]
    _say("prefill-vs-append invariance")
    a = build_cache(K, wl, lens)
    b = build_cache(K, wl, lens, append_steps=300, chunk=200)
    pa, ba = _host(a)
    pb, bb = _host(b)
    assert np.array_equal(a.cache.seq_lens.cpu().numpy(), np.array(lens, np.int32))
    assert np.array_equal(b.cache.seq_lens.cpu().numpy(), np.array(lens, np.int32))
    for s in range(2):
        for h in range(8):
            ng = O.n_groups(lens[s], 4, 128)
            for g in range(ng):
                ga, gb = read_int2_group(a, pa, s, h, g), read_int2_group(b, pb, s, h, g)
                for key in ga:
                    assert np.array_equal(ga[key], gb[key]), (s, h, g, key)
            pos = O.band_positions(lens[s], 4, 128)
            ka, va = read_band(a, ba, s, h, pos)
            kb, vb = read_band(b, bb, s, h, pos)
            assert np.array_equal(ka, kb) and np.array_equal(va, vb)


@pytest.mark.parametrize("impl", ["auto", "f32"])
def test_long_context_gq8_small(K, impl):
    wl = synth.scaled(synth.WORKLOADS["long_b4_131k"], batch=2)
    lens = [5000, 2222]
    _say(f"long gq8 small lens={lens}, split 512, impl={impl}")
    bc = build_cache(K, wl, lens, append_steps=3, split_tokens=512,
                     decode_impl={"f32": K.DECODE_F32}.get(impl, K.DECODE_AUTO))
    pages, band = _host(bc)
    for b in range(2):
        for h in (0, 5):
            check_int2(bc, b, h, pages=pages, band=band)
    q = synth.queries(synth.scaled(wl, batch=2))
    out = run_decode(K, bc, q)
    check_out(bc, out, q, [(b, h) for b in range(2) for h in range(8)])


@pytest.mark.parametrize("scheme", ["int2_channel", "int4_channel"])
def test_split_size_does_not_change_the_result(K, scheme):
    """The automatic split (one work-group per chunk) and explicit splits (one wave per chunk, four chunks
    per work-group, the last work-group partly empty) give the same output up to the order of the merge."""
    wl = synth.scaled(synth.WORKLOADS["gqa_b1_32k"], scheme=scheme)
    lens = [4000, 1234]
    _say(f"split invariance ({scheme})")
    outs = []
    q = synth.queries(synth.scaled(wl, batch=2))
    for split in (0, 128, 256, 512, 2048):
        bc = build_cache(K, wl, lens, split_tokens=split)
        outs.append(run_decode(K, bc, q))
    for o in outs[1:]:
        assert np.abs(outs[0] - o).max() < 1e-5
    check_out(bc, outs[-1], q, [(b, h) for b in range(2) for h in range(8)])


@pytest.mark.parametrize("impl,split", [("auto", 0), ("f32", 0), ("auto", 64), ("mfma", 128), ("mfma", 256)])
def test_saw_int4_small(K, impl, split):
    """INT4 per token on every decode path: the automatic choice (matrix cores over page pairs; the fp32
    path for a 64-token split, whose chunks hold half pairs), each implementation explicitly, and explicit
    splits (one pair chunk per wave).  Lengths end inside a pair's second page, inside its first page
    (the pair's second page missing), and on a page boundary."""
    wl = synth.WORKLOADS["saw_int4_b16_16k"]
    lens = [1000, 333, 66, 40, 128]
    _say(f"saw int4 small lens={lens} impl={impl} split={split}")
    code = {"f32": K.DECODE_F32, "mfma": K.DECODE_MFMA}.get(impl, K.DECODE_AUTO)
    bc = build_cache(K, wl, lens, append_steps=7, chunk=256, decode_impl=code, split_tokens=split)
    pages = bc.cache.pages.cpu().numpy()
    for b in range(len(lens)):
        for h in (0, 6):
            check_int4(bc, b, h, pages)
    q = synth.queries(synth.scaled(wl, batch=len(lens)))
    out = run_decode(K, bc, q)
    check_out(bc, out, q, [(b, h) for b in range(len(lens)) for h in range(8)])


def test_matrix_core_decode_agrees_with_f32(K):
    """The matrix-core decode against the fp32 decode on the same cache: one head with an fp32 source and x10
    outlier channels (4096 tokens), GQA 4 and GQA 8 INT2 caches and the INT4 per-token cache; both within the
    oracle bar."""
    for name, lens in (("tiny_1h_4k", [4096]), ("gqa_b1_32k", [2900, 1000]), ("long_b4_131k", [3000, 700]),
                       ("saw_int4_b16_16k", [1500, 300])):
        wl = synth.WORKLOADS[name]
        _say(f"mfma vs f32: {name} lens={lens}")
        bc = build_cache(K, wl, lens)
        q = synth.queries(synth.scaled(wl, batch=len(lens)))
        outs = []
        for c in (K.DECODE_F32, K.DECODE_MFMA):
            bc.cfg.decode_impl = c
            outs.append(run_decode(K, bc, q))
        diff = np.abs(outs[0] - outs[1]).max()
        _say(f"   max |mfma - f32| = {diff:.2e}")
        assert diff <= TOL
        check_out(bc, outs[1], q, [(b, h) for b in range(len(lens)) for h in range(wl.n_kv_heads)])


def test_decode_is_deterministic(K):
    wl = synth.WORKLOADS["gqa_b1_32k"]
    bc = build_cache(K, wl, [2500])
    q = synth.queries(synth.scaled(wl, batch=1))
    o1 = run_decode(K, bc, q)
    o2 = run_decode(K, bc, q)
    assert np.array_equal(o1, o2)


@pytest.mark.parametrize("name,impl", [("gqa_b1_32k", "auto"), ("gqa_b1_32k", "f32"), ("long_b4_131k", "auto"),
                                       ("saw_int4_b16_16k", "auto")])
def test_timed_decode_equals_the_decode(K, name, impl):
    """kv_decode_attn_timed (events recorded by the split-K dispatch) gives the bytes kv_decode_attn gives,
    and its events bracket a positive interval."""
    import torch
    wl = synth.scaled(synth.WORKLOADS[name], batch=2)
    decode_impl = {"auto": K.DECODE_AUTO, "f32": K.DECODE_F32}[impl]
    bc = build_cache(K, wl, [2500, 700], decode_impl=decode_impl)
    from kvq_cases import source_torch
    q = source_torch(synth.queries(wl), "cuda")
    ws = K.workspace_for(bc.cfg, 2, 2500)
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    ref = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    K.kv_decode_attn(bc.cache, q, ref, 2500, ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    K.kv_decode_attn_timed(bc.cache, q, out, 2500, ws, e0, e1)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    ms = e0.elapsed_time(e1)
    _say(f"timed decode {name} {impl}: split-K {ms * 1e3:.1f} us")
    assert 0.0 < ms < 100.0


def test_error_codes_from_the_device_calls(K):
    import torch
    wl = synth.WORKLOADS["gqa_b1_32k"]
    bc = build_cache(K, wl, [600])
    q = torch.zeros((1, 32, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((1, 32, 128), dtype=torch.float32, device="cuda")
    ws = K.workspace_for(bc.cfg, 1, 600)
    with pytest.raises(K.KvqError) as e:
        K.kv_decode_attn(bc.cache, q, out, 600, ws[:10])
    assert e.value.status == K.KVQ_ENOSPACE
    with pytest.raises(K.KvqError) as e:
        K.kv_decode_attn(bc.cache, q, out, 10 ** 6, K.workspace_for(bc.cfg, 1, 10 ** 6))
    assert e.value.status == K.KVQ_ERANGE


# ------------------------------------------------------------------------- full sizes, sampled


def test_gqa_b1_32k_full_sampled(K):
    wl = synth.WORKLOADS["gqa_b1_32k"]
    _say("gqa_b1_32k full: T=32768")
    bc = build_cache(K, wl, [32768], append_steps=2)
    pages, band = _host(bc)
    for h in (0, 7):
        check_int2(bc, 0, h, groups=[0, 127, O.n_groups(32768, 4, 128) - 1], pages=pages, band=band)
    q = synth.queries(wl)
    out = run_decode(K, bc, q)
    check_out(bc, out, q, [(0, 2), (0, 7)])