"""GPU parity of the scheme variants: per-token INT2 (KVQ_INT2_TOKEN, min/max over a token's 128 channels
as the English OSCAR summary page states §3.4.4 step 3), per-channel INT4 (KVQ_INT4_CHANNEL, the
per-channel groups with 15 levels) and key-only rotation (V quantized in its own frame, [SAW] App. C's
default) for every scheme.  Same bar as the main parity tests: codes, bf16
scales/zeros and band bytes bit-exact against the oracle, outputs within 2e-3.
"""
import numpy as np
import pytest

import oracle as O
import synth
from kvq_cases import _host, _say, build_cache, check_int2, check_int4, check_out, run_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_15_amd as K
    return K


def _int2_case(K, wl, lens, heads, append_steps=0, chunk=None, split=0):
    bc = build_cache(K, wl, lens, append_steps=append_steps, chunk=chunk, split_tokens=split)
    pages, band = _host(bc)
    for b in range(len(lens)):
        for h in heads:
            check_int2(bc, b, h, pages=pages, band=band)
    q = synth.queries(synth.scaled(wl, batch=len(lens)))
    out = run_decode(K, bc, q)
    worst = check_out(bc, out, q, [(b, h) for b in range(len(lens)) for h in range(wl.n_kv_heads)])
    _say(f"   max |out - oracle| = {worst:.2e}")


def test_int2_token_single_head_fp32_source(K):
    wl = synth.scaled(synth.WORKLOADS["tiny_1h_4k"], scheme="int2_token")
    _say("int2 per token: tiny 1 head, T=4096, fp32 source with x10 outlier channels")
    _int2_case(K, wl, [4096], [0])


def test_int2_token_gqa_ragged_with_appends(K):
    wl = synth.scaled(synth.WORKLOADS["gqa_b1_32k"], scheme="int2_token")
    _say("int2 per token: GQA 4, lens [2900, 1000, 133], 5 appends (demotions on the way)")
    _int2_case(K, wl, [2900, 1000, 133], [0, 3, 7], append_steps=5)


def test_int2_token_gq8_decaying_spectrum_chunked(K):
    wl = synth.scaled(synth.WORKLOADS["long_b4_131k"], scheme="int2_token")
    _say("int2 per token: GQA 8, sigma_c = (c+1)^-0.5, lens [3000, 700], 1000-token prefill chunks, split 512")
    _int2_case(K, wl, [3000, 700], [0, 5], chunk=1000, split=512)


def test_int2_token_gqa_full_sampled(K):
    wl = synth.scaled(synth.WORKLOADS["gqa_b1_32k"], scheme="int2_token")
    _say("int2 per token: gqa_b1_32k full, T=32768")
    bc = build_cache(K, wl, [32768], append_steps=2)
    pages, band = _host(bc)
    for h in (1, 6):
        check_int2(bc, 0, h, groups=[0, 100, O.n_groups(32768, 4, 128) - 1], pages=pages, band=band)
    q = synth.queries(wl)
    out = run_decode(K, bc, q)
    check_out(bc, out, q, [(0, 1), (0, 6)])


def test_int4_channel_single_head_fp32_source(K):
    wl = synth.scaled(synth.WORKLOADS["tiny_1h_4k"], scheme="int4_channel")
    _say("int4 per channel: tiny 1 head, T=4096, fp32 source with x10 outlier channels")
    _int2_case(K, wl, [4096], [0])


def test_int4_channel_gq2_ragged_with_appends(K):
    wl = synth.scaled(synth.WORKLOADS["gqa_b1_32k"], scheme="int4_channel", n_q_heads=16, n_kv_heads=8)
    _say("int4 per channel: GQA 2, lens [2900, 1000, 133, 0], 5 appends (demotions on the way)")
    _int2_case(K, wl, [2900, 1000, 133, 0], [0, 3, 7], append_steps=5)


def test_int4_channel_gq4_batch_split(K):
    wl = synth.scaled(synth.WORKLOADS["batch32_32k"], scheme="int4_channel")
    lens = [4100, 2000, 260, 1029, 3000, 388]
    _say(f"int4 per channel: GQA 4, lens {lens}, 800-token prefill chunks, 2 appends")
    _int2_case(K, wl, lens, [0, 5], append_steps=2, chunk=800)


def test_int4_channel_gq8_decaying_spectrum_chunked(K):
    wl = synth.scaled(synth.WORKLOADS["long_b4_131k"], scheme="int4_channel")
    _say("int4 per channel: GQA 8, sigma_c = (c+1)^-0.5, lens [3000, 700], 1000-token prefill chunks, split 512")
    _int2_case(K, wl, [3000, 700], [0, 5], chunk=1000, split=512)


def test_int4_channel_batch32_full_sampled(K):
    """The batch32_32k shape at its full size (32 x 32768 tokens, 8 kv heads, 32 q heads) with per-channel
    INT4: groups and outputs sampled over sequences and heads."""
    wl = synth.scaled(synth.WORKLOADS["batch32_32k"], scheme="int4_channel")
    lens = [32768] * 32
    _say("int4 per channel: batch32_32k full size, sampled")
    bc = build_cache(K, wl, lens, append_steps=1, seqs_per_call=4)
    pages, band = _host(bc)
    ng = O.n_groups(32768, wl.n_sink, wl.n_recent)
    for b, h in ((0, 0), (17, 5), (31, 7)):
        check_int2(bc, b, h, groups=[0, ng // 2, ng - 1], pages=pages, band=band)
    q = synth.queries(wl)
    out = run_decode(K, bc, q)
    worst = check_out(bc, out, q, [(0, 0), (9, 2), (17, 5), (31, 7)])
    _say(f"   max |out - oracle| = {worst:.2e}")


@pytest.mark.parametrize("scheme", ["int2_channel", "int2_token", "int4_channel"])
def test_key_only_rotation_int2(K, scheme):
    wl = synth.scaled(synth.WORKLOADS["gqa_b1_32k"], scheme=scheme, key_only=True)
    _say(f"key-only rotation, {scheme}: lens [2500, 400], 3 appends")
    _int2_case(K, wl, [2500, 400], [0, 4], append_steps=3)


def test_key_only_rotation_int4(K):
    wl = synth.scaled(synth.WORKLOADS["saw_int4_b16_16k"], key_only=True)
    lens = [1500, 37, 64]
    _say(f"key-only rotation, int4 per token: lens {lens}, 2 appends")
    bc = build_cache(K, wl, lens, append_steps=2, chunk=500)
    pages = bc.cache.pages.cpu().numpy()
    for b in range(len(lens)):
        for h in (0, 6):
            check_int4(bc, b, h, pages)
    q = synth.queries(synth.scaled(wl, batch=len(lens)))
    out = run_decode(K, bc, q)
    check_out(bc, out, q, [(b, h) for b in range(len(lens)) for h in range(8)])


def test_key_only_equals_an_identity_value_rotation(K):
    """Key-only rotation stores exactly what the full path stores with R_V = I (a rotation by the identity
    is exact), and decodes to the same output (the identity un-rotation adds only zeros)."""
    import torch
    import kvq_cases as C
    wl = synth.scaled(synth.WORKLOADS["gqa_b1_32k"], n_q_heads=8, n_kv_heads=2, batch=1)
    T = 1200
    _say(f"key-only vs R_V = I: T={T}")
    ko = build_cache(K, synth.scaled(wl, key_only=True), [T])
    # the same cache recipe through the public allocation path, V rotated by the identity
    rk, _ = C.rotations(wl)
    cfg = C.config_for(K, wl)
    mp = max(1, K.pages_for_len(cfg, T))
    n_pool = mp + 3
    pt = K.build_page_table(1, mp, n_pool, seed=0 if wl.identity_pages else wl.seed)
    eye = torch.eye(128, dtype=torch.float32)
    cache = K.allocate_cache(cfg, 1, torch.from_numpy(pt), torch.from_numpy(rk), eye, n_pages=n_pool)
    k, v = C.source_of(wl, 0, T)
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    K.kv_rotate_quant_write(cache, C.source_torch(k, "cuda"), C.source_torch(v, "cuda"), cu, T)
    q = synth.queries(wl)
    out = torch.empty((1, 8, 128), dtype=torch.float32, device="cuda")
    K.kv_decode_attn(cache, C.source_torch(q, "cuda"), out, T, K.workspace_for(cfg, 1, T))
    torch.cuda.synchronize()
    assert np.array_equal(ko.cache.page_table.cpu().numpy(), pt)
    pb = K.page_bytes(cfg)
    pa, pi = ko.cache.pages.cpu().numpy(), cache.pages.cpu().numpy()
    for phys in pt[0, :2 * O.n_groups(T, wl.n_sink, wl.n_recent)]:
        assert np.array_equal(pa[phys * pb:(phys + 1) * pb], pi[phys * pb:(phys + 1) * pb])
    assert np.abs(out.cpu().numpy() - run_decode(K, ko, q)).max() < 1e-6


@pytest.mark.parametrize("block", [16, 32, 64])
def test_int4_block_hadamard_orders(K, block):
    """[SAW] eq. (1) block orders h = 16, 32, 64: codes bit-exact, outputs within the bar, through the
    write (prefill chunks + appends), the query rotation and the merge's inverse rotation."""
    wl = synth.scaled(synth.WORKLOADS["saw_int4_b16_16k"], hadamard_block=block)
    lens = [1300, 511]
    _say(f"int4 with Hadamard block {block}: lens {lens}, 3 appends")
    bc = build_cache(K, wl, lens, append_steps=3, chunk=600)
    pages = bc.cache.pages.cpu().numpy()
    for b in range(len(lens)):
        for h in (1, 7):
            check_int4(bc, b, h, pages)
    q = synth.queries(synth.scaled(wl, batch=len(lens)))
    out = run_decode(K, bc, q)
    worst = check_out(bc, out, q, [(b, h) for b in range(len(lens)) for h in range(8)])
    _say(f"   max |out - oracle| = {worst:.2e}")
