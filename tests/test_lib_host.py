"""Host-side checks of libkvq (no GPU): exported symbols, sizes, bit accounting, validation, builders."""
import json
import os
import re

import numpy as np
import pytest

import decode_attention_15_amd as K
import oracle as O
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "kvq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq?_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert "kv_decode_attn" in names and "kv_rotate_quant_write" in names
    for n in names:
        assert hasattr(K._lib, n), n
    assert sorted(K.EXPORTED) == names


def test_version_and_strerror():
    assert "gfx950" in K.version()
    for st in (0, -1, -2, -3, -4, -5):
        assert K.strerror(st) and K.strerror(st) != "unknown status"


def test_page_and_band_sizes():
    cfg = K.make_config(8, 32)
    assert K.page_bytes(cfg) == 8 * 4608
    assert K.band_slots(cfg) == 4 + 128 + 128
    assert K.band_bytes(cfg, 32) == 32 * 8 * 260 * 512
    cfg4 = K.make_config(8, 32, scheme=K.INT4_TOKEN, rotation=K.ROT_HADAMARD, n_sink=0, n_recent=0,
                         clip_k=1.0, clip_v=1.0)
    assert K.page_bytes(cfg4) == 8 * 8704
    assert K.band_slots(cfg4) == 0
    # 72 bytes per INT2 token and kv head; 136 for INT4 (codes + bf16 scale/zero)
    assert K.page_bytes(cfg) / (64 * 8) == 72
    assert K.page_bytes(cfg4) / (64 * 8) == 136


def test_pages_for_len_follows_the_group_layout():
    cfg = K.make_config(8, 32)
    for T in (0, 4, 259, 260, 4096, 32768):
        assert K.pages_for_len(cfg, T) == 2 * O.n_groups(T, 4, 128)
    cfg4 = K.make_config(8, 32, scheme=K.INT4_TOKEN, rotation=K.ROT_HADAMARD, n_sink=0, n_recent=0)
    assert K.pages_for_len(cfg4, 16384) == 256 and K.pages_for_len(cfg4, 65) == 2


def test_bits_per_element_match_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "bits_per_element.json")))
    S0, W = g["band"]
    cfg = K.make_config(8, 32, n_sink=S0, n_recent=W)
    # all-quantized region
    T_big = S0 + W + 128 * 100000
    region = K.bits_per_element(cfg, T_big)
    assert abs(region - g["int2_region_bpe"]) < 0.01
    # at ~128K with the tail exactly W long, the band adds ~0.034 and the total is ~2.28
    T = S0 + W + 128 * ((g["context"] - S0 - W) // 128)
    bpe = K.bits_per_element(cfg, T)
    assert abs(bpe - g["int2_total_bpe_64_256_at_128k"]) < 0.006
    assert abs((bpe - 2.25) - g["int2_band_extra_bpe_64_256_at_128k"]) < 0.002
    cfg4 = K.make_config(8, 32, scheme=K.INT4_TOKEN, rotation=K.ROT_HADAMARD, n_sink=0, n_recent=0)
    assert K.bits_per_element(cfg4, 16384) == pytest.approx(g["int4_bpe"])


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, K.KVQ_EUNSUPPORTED), ("page_tokens", 32, K.KVQ_EUNSUPPORTED),
    ("scheme", 7, K.KVQ_EUNSUPPORTED), ("rotation", 5, K.KVQ_EUNSUPPORTED),
    ("n_q_heads", 30, K.KVQ_EINVAL), ("n_kv_heads", 0, K.KVQ_EINVAL), ("clip_k", 0.0, K.KVQ_EINVAL),
    ("clip_v", 1.5, K.KVQ_EINVAL), ("split_tokens", 100, K.KVQ_EINVAL), ("n_sink", -1, K.KVQ_EINVAL),
    ("decode_impl", 9, K.KVQ_EINVAL), ("decode_impl", -1, K.KVQ_EINVAL),
    ("key_only_rotation", 2, K.KVQ_EINVAL), ("key_only_rotation", -1, K.KVQ_EINVAL), ("scheme", 4, K.KVQ_EUNSUPPORTED),
])
def test_config_validation(field, value, status):
    cfg = K.make_config(8, 32)
    assert K.check_config(cfg) == K.KVQ_OK
    setattr(cfg, field, value)
    assert K.check_config(cfg) == status
    assert K.page_bytes(cfg) == 0


def test_gqa_ratio_16_is_unsupported_and_int4_rejects_a_band():
    assert K.check_config(K.make_config(1, 16)) == K.KVQ_EUNSUPPORTED
    assert K.check_config(K.make_config(8, 32, scheme=K.INT4_TOKEN, n_sink=4)) == K.KVQ_EINVAL


def test_calls_reject_null_pointers_before_touching_the_device():
    import ctypes
    cfg = K.make_config(8, 32)
    cache = K.Cache()
    st = K._lib_write(ctypes.byref(cfg), ctypes.byref(cache), None, None, 0, None, 1, 1, None)
    assert st == K.KVQ_EINVAL
    st = K._lib_decode(ctypes.byref(cfg), ctypes.byref(cache), None, 0, None, 10, None, 0, None)
    assert st == K.KVQ_EINVAL


def test_workspace_grows_with_context_and_batch():
    cfg = K.make_config(8, 32)
    a = K.decode_workspace_bytes(cfg, 1, 4096)
    b = K.decode_workspace_bytes(cfg, 1, 32768)
    c = K.decode_workspace_bytes(cfg, 32, 32768)
    assert 0 < a < b < c
    assert K.decode_workspace_bytes(cfg, 0, 10) == 0


def test_oscar_builder_matches_the_oracle_construction():
    wl = synth.WORKLOADS["tiny_1h_4k"]
    G = synth.rotation_gaussian(wl, "k")
    R_lib = K.build_oscar_rotation(G)
    R_or = O.oscar_rotation(G)
    assert np.abs(R_lib - R_or).max() < 1e-12
    assert np.abs(R_lib.T @ R_lib - np.eye(128)).max() < 1e-13


def test_compose_and_hadamard_builders():
    U = O.orthonormal_from_gaussian(synth.rotation_gaussian(synth.WORKLOADS["tiny_1h_4k"], "v"))
    assert np.abs(K.compose_oscar_rotation(U) - U @ O.hadamard() @ O.bit_reversal_matrix()).max() < 1e-13
    s = synth.sign_vector(synth.WORKLOADS["saw_int4_b16_16k"], "k")
    assert np.abs(K.build_hadamard_rotation(s.astype(np.float32)) - O.saw_rotation_matrix(s)).max() < 1e-15
    with pytest.raises(K.KvqError):
        K.build_hadamard_rotation(np.full(128, 0.5, np.float32))


def test_one_hip_runtime_in_the_process():
    """The binding loads torch's HIP runtime first, so libkvq binds to it instead of a second copy."""
    import subprocess
    import sys
    code = ("import os, decode_attention_15_amd\n"
            "m = open(f'/proc/{os.getpid()}/maps').read()\n"
            "print(len({l.split()[-1] for l in m.splitlines() if 'libamdhip64' in l}))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().splitlines()[-1] == "1"


def test_decode_implementations_accepted_for_both_schemes():
    for scheme, rot, s0, w, ck, cv in ((K.INT2_CHANNEL, K.ROT_DENSE, 4, 128, 0.96, 0.92),
                                       (K.INT4_TOKEN, K.ROT_HADAMARD, 0, 0, 1.0, 1.0)):
        for impl in (K.DECODE_AUTO, K.DECODE_F32, K.DECODE_MFMA):
            cfg = K.make_config(8, 32, scheme=scheme, rotation=rot, n_sink=s0, n_recent=w, clip_k=ck, clip_v=cv,
                                decode_impl=impl)
            assert K.check_config(cfg) == K.KVQ_OK
        # the retired integer-dot decodes (3, 4) and other values are unknown
        for impl in (3, 4, -1, 99):
            cfg = K.make_config(8, 32, scheme=scheme, rotation=rot, n_sink=s0, n_recent=w, clip_k=ck, clip_v=cv,
                                decode_impl=impl)
            assert K.check_config(cfg) == K.KVQ_EINVAL
    # INT4 per token on the matrix cores walks page pairs: an explicit split must hold whole pairs
    for split, want in ((64, K.KVQ_EUNSUPPORTED), (192, K.KVQ_EUNSUPPORTED), (128, K.KVQ_OK), (512, K.KVQ_OK)):
        cfg = K.make_config(8, 32, scheme=K.INT4_TOKEN, rotation=K.ROT_HADAMARD, n_sink=0, n_recent=0,
                            clip_k=1.0, clip_v=1.0, split_tokens=split, decode_impl=K.DECODE_MFMA)
        assert K.check_config(cfg) == want
        cfg.decode_impl = K.DECODE_AUTO  # the automatic choice takes the fp32 path there instead
        assert K.check_config(cfg) == K.KVQ_OK


def test_matrix_core_decode_schemes():
    for scheme, rot, s0, w, ck, cv, want in (
            (K.INT2_CHANNEL, K.ROT_DENSE, 4, 128, 0.96, 0.92, K.KVQ_OK),
            (K.INT2_CHANNEL, K.ROT_HADAMARD, 4, 256, 0.96, 0.92, K.KVQ_OK),
            (K.INT2_TOKEN, K.ROT_DENSE, 4, 128, 0.96, 0.92, K.KVQ_OK),
            (K.INT4_CHANNEL, K.ROT_DENSE, 4, 128, 0.96, 0.92, K.KVQ_OK),
            (K.INT4_TOKEN, K.ROT_HADAMARD, 0, 0, 1.0, 1.0, K.KVQ_OK)):
        for split in (0, 512):
            cfg = K.make_config(8, 32, scheme=scheme, rotation=rot, n_sink=s0, n_recent=w, clip_k=ck, clip_v=cv,
                                split_tokens=split, decode_impl=K.DECODE_MFMA)
            assert K.check_config(cfg) == want, (scheme, split)


def test_int2_token_scheme_config():
    """Per-token INT2: same sink/recent rules and sizes as the per-channel scheme; built on the matrix cores."""
    for impl, want in ((K.DECODE_AUTO, K.KVQ_OK), (K.DECODE_MFMA, K.KVQ_OK), (K.DECODE_F32, K.KVQ_EUNSUPPORTED)):
        cfg = K.make_config(8, 32, scheme=K.INT2_TOKEN, decode_impl=impl)
        assert K.check_config(cfg) == want
    a = K.make_config(8, 32, scheme=K.INT2_TOKEN)
    c = K.make_config(8, 32, scheme=K.INT2_CHANNEL)
    for T in (0, 100, 4096, 32768):
        assert K.pages_for_len(a, T) == K.pages_for_len(c, T)
        assert K.bits_per_element(a, max(T, 1)) == K.bits_per_element(c, max(T, 1))
    assert K.page_bytes(a) == K.page_bytes(c) and K.band_bytes(a, 4) == K.band_bytes(c, 4)
    assert K.check_config(K.make_config(8, 32, key_only_rotation=True)) == K.KVQ_OK


def test_int4_channel_scheme_config():
    """Per-channel INT4: the INT2 groups, band and page count on the INT4 page size; built on the matrix cores."""
    for impl, want in ((K.DECODE_AUTO, K.KVQ_OK), (K.DECODE_MFMA, K.KVQ_OK), (K.DECODE_F32, K.KVQ_EUNSUPPORTED)):
        assert K.check_config(K.make_config(8, 32, scheme=K.INT4_CHANNEL, decode_impl=impl)) == want
    a = K.make_config(8, 32, scheme=K.INT4_CHANNEL)
    c = K.make_config(8, 32, scheme=K.INT2_CHANNEL)
    t = K.make_config(8, 32, scheme=K.INT4_TOKEN, rotation=K.ROT_HADAMARD, n_sink=0, n_recent=0, clip_k=1.0,
                      clip_v=1.0)
    assert K.page_bytes(a) == K.page_bytes(t) == 8 * 8704
    assert K.band_slots(a) == K.band_slots(c) and K.band_bytes(a, 4) == K.band_bytes(c, 4)
    for T in (0, 100, 4096, 32768):
        assert K.pages_for_len(a, T) == K.pages_for_len(c, T)
    # one full group past the band: 128 x 128 codes at 4 bits + 2 x 128 bf16 per K and V
    T = 4 + 128 + 128
    want = (2 * (128 * 128 / 2 + 2 * 128 * 2) + (T - 128) * 512) * 8 / (2 * T * 128)
    assert abs(K.bits_per_element(a, T) - want) < 1e-9
    for hb in (16, 32, 64):
        assert K.check_config(K.make_config(8, 32, scheme=K.INT4_CHANNEL, rotation=K.ROT_HADAMARD,
                                            hadamard_block=hb)) == K.KVQ_OK


# ------------------------------------------------------------------ page tables and the write's length bound
# ([OSCAR] §3.4.5: the paged cache, logical pages mapped to physical pages of a pool)


def test_build_page_table_identity_and_seeded():
    pt = K.build_page_table(3, 5, 15, seed=0)
    assert np.array_equal(pt, np.arange(15, dtype=np.int32).reshape(3, 5))
    a = K.build_page_table(4, 6, 40, seed=1234)
    b = K.build_page_table(4, 6, 40, seed=1234)
    c = K.build_page_table(4, 6, 40, seed=1235)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert a.shape == (4, 6) and len(set(a.ravel().tolist())) == 24
    assert a.min() >= 0 and a.max() < 40
    assert K.check_page_table(a, 40) == K.KVQ_OK
    # a full pool is a permutation of it
    full = K.build_page_table(8, 16, 128, seed=7)
    assert sorted(full.ravel().tolist()) == list(range(128))


def test_build_page_table_errors():
    out = np.empty(16, dtype=np.int32)
    vp = out.ctypes.data_as(K.ctypes.c_void_p)
    assert K._lib_build_pt(4, 4, 15, 1, vp) == K.KVQ_ERANGE       # 16 pages asked of a pool of 15
    assert K._lib_build_pt(0, 4, 16, 1, vp) == K.KVQ_EINVAL
    assert K._lib_build_pt(4, -1, 16, 1, vp) == K.KVQ_EINVAL
    assert K._lib_build_pt(4, 4, 0, 1, vp) == K.KVQ_EINVAL
    assert K._lib_build_pt(4, 4, 16, 1, None) == K.KVQ_EINVAL


def test_check_page_table_finds_out_of_pool_and_shared_pages():
    pt = K.build_page_table(2, 3, 6, seed=3)
    assert K.check_page_table(pt, 6) == K.KVQ_OK
    bad = pt.copy()
    bad[1, 2] = 6
    assert K.check_page_table(bad, 6) == K.KVQ_ERANGE
    bad[1, 2] = -1
    assert K.check_page_table(bad, 6) == K.KVQ_ERANGE
    dup = pt.copy()
    dup[1, 0] = dup[0, 0]
    assert K.check_page_table(dup, 6) == K.KVQ_EINVAL


def _fake_cache(cfg, batch, max_pages, n_pages=1 << 20):
    # non-NULL stand-ins for device pointers: only calls that fail validation, before any device work, use it
    f = 0x1000
    return K.Cache(f, n_pages, f, f, max_pages, f, f, f, batch)


def test_write_length_bound_is_checked_before_any_launch():
    f = 0x1000
    for scheme, kw in ((K.INT2_CHANNEL, {}), (K.INT4_TOKEN, dict(rotation=K.ROT_HADAMARD, n_sink=0, n_recent=0,
                                                                   clip_k=1.0, clip_v=1.0))):
        cfg = K.make_config(8, 32, scheme=scheme, **kw)
        T = 4096
        mp = K.pages_for_len(cfg, T)
        cs = _fake_cache(cfg, 2, mp)
        # one token more than the page-table row holds: KVQ_ERANGE, nothing enqueued
        T_over = T + (129 if scheme == K.INT2_CHANNEL else 64)
        assert K.pages_for_len(cfg, T_over) > mp
        st = K._lib_write(K.ctypes.byref(cfg), K.ctypes.byref(cs), f, f, K.BF16, f, 1, T_over, None)
        assert st == K.KVQ_ERANGE
        # negative bounds
        assert K._lib_write(K.ctypes.byref(cfg), K.ctypes.byref(cs), f, f, K.BF16, f, 1, -1, None) == K.KVQ_EINVAL
        assert K._lib_write(K.ctypes.byref(cfg), K.ctypes.byref(cs), f, f, K.BF16, f, -1, T, None) == K.KVQ_EINVAL
        # a pool of no pages is no cache
        cs0 = _fake_cache(cfg, 2, mp, n_pages=0)
        assert K._lib_write(K.ctypes.byref(cfg), K.ctypes.byref(cs0), f, f, K.BF16, f, 1, T, None) == K.KVQ_EINVAL


def test_debug_unpack_validation():
    f = 0x1000
    cfg = K.make_config(8, 32)
    cs = _fake_cache(cfg, 2, 8)
    call = lambda seq, h, n: K._lib_debug_unpack(K.ctypes.byref(cfg), K.ctypes.byref(cs), seq, h, n, f, f, None)
    assert call(2, 0, 128) == K.KVQ_EINVAL    # sequence outside the batch
    assert call(0, 8, 128) == K.KVQ_EINVAL    # kv head outside the layer
    assert call(0, 0, 100) == K.KVQ_EINVAL    # not whole groups
    assert call(0, 0, 128 * 5) == K.KVQ_ERANGE  # 10 pages of a row of 8
    assert call(0, 0, 0) == K.KVQ_OK          # nothing to read


def test_noalloc_decode_refuses_what_the_scratch_cannot_hold():
    """kv_decode_attn_noalloc: argument errors and a workspace beyond its fixed scratch are refused on the
    host, before anything touches the device (the pointers here are never dereferenced)."""
    f = 0x1000
    cfg = K.make_config(8, 32, split_tokens=512)
    T = 32768
    mp = K.pages_for_len(cfg, T)
    # batch 32 at 32k tokens and the smallest split fits; batch 64 does not
    assert K.decode_workspace_bytes(cfg, 32, T) <= K.NOALLOC_SCRATCH_BYTES
    assert K.decode_workspace_bytes(cfg, 64, T) > K.NOALLOC_SCRATCH_BYTES
    cs = _fake_cache(cfg, 64, mp)
    st = K._lib_decode_noalloc(K.ctypes.byref(cfg), K.ctypes.byref(cs), f, K.F32, f, T, None)
    assert st == K.KVQ_ENOSPACE
    assert "scratch" in K.last_error()
    # beyond the page table, null pointers, a bad dtype
    assert K._lib_decode_noalloc(K.ctypes.byref(cfg), K.ctypes.byref(cs), f, K.F32, f, T + 129, None) == K.KVQ_ERANGE
    assert K._lib_decode_noalloc(K.ctypes.byref(cfg), K.ctypes.byref(cs), None, K.F32, f, T, None) == K.KVQ_EINVAL
    assert K._lib_decode_noalloc(K.ctypes.byref(cfg), K.ctypes.byref(cs), f, 7, f, T, None) == K.KVQ_EINVAL
    assert K._lib_decode_noalloc(K.ctypes.byref(cfg), K.ctypes.byref(cs), f, K.F32, f, -1, None) == K.KVQ_EINVAL


def test_decode_shape_chunks_and_walks():
    """The decode's chunking and grid (host only): automatic chunks give one chunk per wave and fit one round
    of work-groups; an explicit split keeps its chunks and lets a wave walk several in a row."""
    cfg = K.make_config(8, 32)
    sh = K.decode_shape(cfg, 32, 32768)
    ng = 255  # groups of a 32768-token sequence with 4 sink and 128 recent tokens
    assert sh["matrix_cores"] == 1 and sh["span"] == 1 and sh["walks"] == sh["n_chunks"]
    assert sh["n_chunks"] == -(-ng // sh["chunk_units"]) and 4 <= sh["chunk_units"] <= 32
    assert sh["splitk_workgroups"] == 32 * 2 * sh["n_chunks"] + 256 <= 256 * 3 and sh["band_first"] == 0
    # 512-token split at 4 x 131k, GQA 8: 256 chunks of 4 groups in 92 walks of 2 or 3 chunks per (sequence,
    # head quad), filling the 768 slots of one round (3 per CU) with the 32 band work-groups
    cfg8 = K.make_config(8, 64, n_recent=256, split_tokens=512)
    sh = K.decode_shape(cfg8, 4, 131072)
    assert sh["chunk_units"] == 4 and sh["n_chunks"] == 256 and sh["walks"] == 92 and sh["span"] == 3
    assert sh["splitk_workgroups"] == 4 * 2 * 92 + 32 == 768 and sh["band_first"] == 0
    # the fp32 decode walks one chunk per work-group
    cfg.decode_impl = K.DECODE_F32
    sh = K.decode_shape(cfg, 32, 32768)
    assert sh["matrix_cores"] == 0 and sh["span"] == 1 and sh["walks"] == sh["n_chunks"]
    assert sh["splitk_workgroups"] == 256 * sh["n_chunks"] + 256
    # explicit split at batch 32: 64 chunks per sequence, 8 in a row (32 groups)
    cfg = K.make_config(8, 32, split_tokens=512)
    sh = K.decode_shape(cfg, 32, 32768)
    assert sh["n_chunks"] == 64 and sh["walks"] == 8 and sh["span"] == 8 and sh["splitk_workgroups"] == 64 * 8 + 256
    # two kv heads (no head quads): four walks per work-group, the last work-group of a row partly idle
    cfg2 = K.make_config(2, 8, split_tokens=512)
    sh = K.decode_shape(cfg2, 64, 12000)
    assert sh["walks"] >= 2 and sh["splitk_workgroups"] == 128 * (-(-sh["walks"] // 4)) + 128
    with pytest.raises(K.KvqError):
        K.decode_shape(cfg, 0, 100)


def test_read_probe_refuses_on_the_host():
    """kvq_read_probe: schemes without the matrix-core grouped walk, null output, negative or too long
    lengths are refused before anything touches the device (the pointers here are never dereferenced)."""
    f = 0x1000
    T = 4096
    cfg = K.make_config(8, 32)
    cs = _fake_cache(cfg, 2, K.pages_for_len(cfg, T))
    probe = K._lib_read_probe
    assert probe(K.ctypes.byref(cfg), K.ctypes.byref(cs), None, T, None) == K.KVQ_EINVAL
    assert probe(K.ctypes.byref(cfg), K.ctypes.byref(cs), f, -1, None) == K.KVQ_EINVAL
    assert probe(K.ctypes.byref(cfg), K.ctypes.byref(cs), f, T + 129, None) == K.KVQ_ERANGE
    cfg.decode_impl = K.DECODE_F32
    assert probe(K.ctypes.byref(cfg), K.ctypes.byref(cs), f, T, None) == K.KVQ_EUNSUPPORTED
    cfg4 = K.make_config(8, 32, K.INT4_TOKEN, K.ROT_HADAMARD, 0, 0, 1.0, 1.0)
    cs4 = _fake_cache(cfg4, 2, K.pages_for_len(cfg4, T))
    assert probe(K.ctypes.byref(cfg4), K.ctypes.byref(cs4), f, T, None) == K.KVQ_EUNSUPPORTED


def test_balanced_chunking_is_reported():
    """Automatic chunks of the grouped schemes in head quads are chosen on the device from the lengths
    (balanced); the host reports the choice for uniform lengths and the bound the workspace holds."""
    cfg = K.make_config(8, 32)
    sh = K.decode_shape(cfg, 32, 32768)
    assert sh["balanced"] == 1 and sh["chunk_units"] == 32 and sh["n_chunks"] == 8
    assert sh["max_chunks"] == -(-255 // 4)  # chunks of at least 4 groups
    assert K.decode_workspace_bytes(cfg, 32, 32768) >= 4 * 32 * 32 * (1 + sh["max_chunks"]) * 130
    # batch 1: the 4-group floor
    sh1 = K.decode_shape(cfg, 1, 32768)
    assert sh1["balanced"] == 1 and sh1["chunk_units"] == 4
    # not balanced: an explicit split, the fp32 decode, kv heads not in fours, INT4 per token
    for c in (K.make_config(8, 32, split_tokens=512), K.make_config(8, 32, decode_impl=K.DECODE_F32),
              K.make_config(2, 8), K.make_config(8, 32, K.INT4_TOKEN, K.ROT_HADAMARD, 0, 0, 1.0, 1.0)):
        assert K.decode_shape(c, 32, 32768)["balanced"] == 0
