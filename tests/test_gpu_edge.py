"""GPU parity on degenerate inputs and boundary lengths (through the C ABI, against the CPU oracle).

Covers what random N(0,1) caches never produce: all-zero groups (b = a, so s = 1 and a signed zero
point), channels constant over a group, very large and very small (fp32-subnormal after rotation)
magnitudes, no clipping (rho = 1), and lengths at the sink / window / group boundaries.
"""
import sys

import numpy as np
import pytest

import oracle as O
import synth
from kvq_cases import GROUPED, config_for, read_band, read_int2_group, rotations, source_torch

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_15_amd as K
    return K


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class _BC:
    """Minimal stand-in for kvq_cases.BuiltCache: what the layout readers use (wl.scheme, wl.n_kv_heads)."""

    def __init__(self, wl, cache):
        self.wl, self.cache = wl, cache


def _write_and_check(K, wl, kb, vb, clip=(0.96, 0.92), chunks=None, decode=True, decode_impl=0):
    """Write bf16 K/V [T, n_kv, 128] for one sequence, compare every group, the band and the decode output."""
    import torch
    T = kb.shape[0]
    wl = synth.scaled(wl, batch=1, clip_k=clip[0], clip_v=clip[1])
    cfg = config_for(K, wl, 0, decode_impl)
    rk, rv = rotations(wl)
    max_pages = max(1, K.pages_for_len(cfg, T))
    n_pool = max_pages + 2
    pt = K.build_page_table(1, max_pages, n_pool, seed=0 if wl.identity_pages else wl.seed)
    cache = K.allocate_cache(cfg, 1, torch.from_numpy(pt), torch.from_numpy(rk), torch.from_numpy(rv), n_pages=n_pool)
    done = 0
    for n in (chunks or [T]):
        cu = torch.tensor([0, n], dtype=torch.int32, device="cuda")
        K.kv_rotate_quant_write(cache, source_torch(kb[done:done + n], "cuda"), source_torch(vb[done:done + n], "cuda"),
                                cu, n)
        done += n
    torch.cuda.synchronize()
    assert int(cache.seq_lens.item()) == T
    pages = cache.pages.cpu().numpy()
    band = cache.band.cpu().numpy().view(np.uint16)
    bc = _BC(wl, cache)
    worst = 0.0
    axis = GROUPED[wl.scheme]
    for h in range(wl.n_kv_heads):
        st = O.int2_state(kb[:, h], vb[:, h], T, wl.n_sink, wl.n_recent, wl.clip_k, wl.clip_v, rk, rv, axis=axis)
        for i, g in enumerate(st["groups"]):
            got = read_int2_group(bc, pages, 0, h, int(g))
            for key in ("k_codes", "v_codes", "k_s16", "k_z16", "v_s16", "v_z16"):
                assert np.array_equal(got[key], st[key][i]), f"h={h} group {g} {key}"
        bk, bv = read_band(bc, band, 0, h, st["band_pos"])
        assert np.array_equal(bk, st["band_k"]) and np.array_equal(bv, st["band_v"]), f"band h={h}"
        if decode and T > 0:
            q = synth.queries(wl)
            qh = q[0, h * wl.gq:(h + 1) * wl.gq]
            Kh, Vh = O.int2_keys_values(st, rk, rv)
            want = O.attend(O.query_values(qh), Kh, Vh)
            if h == 0:
                out = torch.empty((1, wl.n_q_heads, 128), dtype=torch.float32, device="cuda")
                K.kv_decode_attn(cache, source_torch(q, "cuda"), out, T, K.workspace_for(cfg, 1, T))
                torch.cuda.synchronize()
                got_out = out.cpu().numpy()
            err = np.abs(got_out[0, h * wl.gq:(h + 1) * wl.gq] - want).max()
            worst = max(worst, err)
            assert np.isfinite(got_out).all()
            assert err <= TOL, f"h={h}: max |diff| {err:.3e}"
    return worst


def _bf16(x):
    return synth.to_bf16_bits(np.asarray(x, dtype=np.float32))


WL = synth.scaled(synth.WORKLOADS["gqa_b1_32k"], n_q_heads=8, n_kv_heads=2)
SCHEMES = pytest.mark.parametrize("scheme", ["int2_channel", "int2_token", "int4_channel"])


@SCHEMES
def test_all_zero_groups_and_constant_channels(K, scheme):
    T = 4 + 128 + 3 * 128 + 50
    rng = np.random.default_rng(5)
    k = rng.standard_normal((T, 2, 128)).astype(np.float32)
    v = rng.standard_normal((T, 2, 128)).astype(np.float32)
    k[4:132] = 0.0                     # group 0 of both heads all zero: rotated zeros, s = 1, z = -0
    v[4:132] = 0.0
    k[132:260, 0, :] = 0.75            # group 1, head 0: every token the same constant vector
    v[132:260, 1, :] = -2.0
    _say(f"all-zero group, constant tokens ({scheme})")
    _write_and_check(K, synth.scaled(WL, scheme=scheme), _bf16(k), _bf16(v))


@SCHEMES
def test_large_and_tiny_magnitudes(K, scheme):
    T = 4 + 128 + 2 * 128 + 7
    rng = np.random.default_rng(6)
    k = rng.standard_normal((T, 2, 128)).astype(np.float32)
    v = rng.standard_normal((T, 2, 128)).astype(np.float32)
    k[4:132] *= 3.0e4                  # group 0: large values
    v[4:132] *= 1.0e-3
    k[132:260] *= 1.0e-36              # group 1: tiny values; rotated results are fp32 subnormals
    v[132:260] *= 1.0e-37
    _say(f"large and tiny magnitudes ({scheme})")
    _write_and_check(K, synth.scaled(WL, scheme=scheme), _bf16(k), _bf16(v), decode=False)


@SCHEMES
def test_no_clip(K, scheme):
    T = 4 + 128 + 2 * 128 + 1
    rng = np.random.default_rng(7)
    k = (rng.standard_normal((T, 2, 128)) * 3).astype(np.float32)
    v = rng.standard_normal((T, 2, 128)).astype(np.float32)
    _say(f"clip ratio 1 (no clip) ({scheme})")
    _write_and_check(K, synth.scaled(WL, scheme=scheme), _bf16(k), _bf16(v), clip=(1.0, 1.0))


@SCHEMES
@pytest.mark.parametrize("T", [1, 3, 4, 5, 132, 259, 260, 261, 387, 388, 389])
def test_lengths_at_the_sink_window_group_boundaries(K, T, scheme):
    rng = np.random.default_rng(100 + T)
    k = rng.standard_normal((T, 2, 128)).astype(np.float32)
    v = rng.standard_normal((T, 2, 128)).astype(np.float32)
    _say(f"boundary length T={T} ({scheme})")
    # written one token at a time below 8 tokens, else in two uneven chunks
    chunks = [1] * T if T < 8 else [T // 3, T - T // 3]
    _write_and_check(K, synth.scaled(WL, scheme=scheme), _bf16(k), _bf16(v), chunks=chunks)


# ------------------------------------------------------------------ INT4 per token ([SAW] App. A.1)

SAW = synth.scaled(synth.WORKLOADS["saw_int4_b16_16k"], n_q_heads=8, n_kv_heads=2, batch=1)


def _int4_expected(wl, k, v, rk, rv):
    """Oracle codes and metadata of every token of one kv head (source [T, 128]), either rotation."""
    if wl.rotation == "saw":
        return O.int4_state(k, v, len(k), rk.astype(np.int8), rv.astype(np.int8), block=wl.hadamard_block)
    xk = O.rotate_dense(O.bf16_value(O.source_to_bf16(k)), rk)
    xv = O.rotate_dense(O.bf16_value(O.source_to_bf16(v)), rv)
    qk, sk, zk = O.quantize_int4_token(xk)
    qv, sv, zv = O.quantize_int4_token(xv)
    return {"k_codes": qk, "k_s16": sk, "k_z16": zk, "v_codes": qv, "v_s16": sv, "v_z16": zv}


def _int4_keys_values(wl, st, rk, rv):
    if wl.rotation == "saw":
        return O.int4_keys_values(st, rk.astype(np.int8), rv.astype(np.int8), wl.hadamard_block)
    xk = O.dequantize(st["k_codes"], st["k_s16"][:, None], st["k_z16"][:, None])
    xv = O.dequantize(st["v_codes"], st["v_s16"][:, None], st["v_z16"][:, None])
    return xk @ rk.astype(np.float64).T, xv @ rv.astype(np.float64).T


def _int4_write_and_check(K, wl, k, v, chunks, misalign=False, decode=True):
    """Write K/V [T, n_kv, 128] (bf16 bits or fp32) of one sequence in `chunks`, each chunk's source placed
    4 bytes past a 16-byte boundary if `misalign`; compare every token's codes and metadata, and the decode
    output if `decode`."""
    import torch
    from kvq_cases import read_int4_tokens
    T = k.shape[0]
    cfg = config_for(K, wl)
    rk, rv = rotations(wl)
    max_pages = max(1, K.pages_for_len(cfg, T))
    n_pool = max_pages + 2
    pt = K.build_page_table(1, max_pages, n_pool, seed=0 if wl.identity_pages else wl.seed)
    cache = K.allocate_cache(cfg, 1, torch.from_numpy(pt), torch.from_numpy(rk), torch.from_numpy(rv), n_pages=n_pool)

    def dev(x):
        t = source_torch(np.ascontiguousarray(x), "cuda")
        if not misalign:
            return t
        pad = 2 if t.dtype == torch.bfloat16 else 1
        buf = torch.zeros(t.numel() + pad, dtype=t.dtype, device="cuda")
        buf[pad:] = t.reshape(-1)
        out = buf[pad:].view(t.shape)
        assert out.data_ptr() % 16 != 0
        return out

    done = 0
    for n in chunks:
        cu = torch.tensor([0, n], dtype=torch.int32, device="cuda")
        K.kv_rotate_quant_write(cache, dev(k[done:done + n]), dev(v[done:done + n]), cu, n)
        done += n
    torch.cuda.synchronize()
    assert done == T and int(cache.seq_lens.item()) == T
    pages = cache.pages.cpu().numpy()
    bc = _BC(wl, cache)
    q = synth.queries(wl)
    if decode:
        out = torch.empty((1, wl.n_q_heads, 128), dtype=torch.float32, device="cuda")
        K.kv_decode_attn(cache, source_torch(q, "cuda"), out, T, K.workspace_for(cfg, 1, T))
        torch.cuda.synchronize()
        got_out = out.cpu().numpy()
    worst = 0.0
    for h in range(wl.n_kv_heads):
        st = _int4_expected(wl, k[:, h], v[:, h], rk, rv)
        got = read_int4_tokens(bc, pages, 0, h, T)
        for key in ("k_codes", "v_codes", "k_s16", "k_z16", "v_s16", "v_z16"):
            bad = np.argwhere(got[key] != st[key])
            assert len(bad) == 0, f"h={h} {key}: {len(bad)} mismatches, first {bad[:5].tolist()}"
        if not decode:
            continue
        Kh, Vh = _int4_keys_values(wl, st, rk, rv)
        want = O.attend(O.query_values(q[0, h * wl.gq:(h + 1) * wl.gq]), Kh, Vh)
        err = np.abs(got_out[0, h * wl.gq:(h + 1) * wl.gq] - want).max()
        worst = max(worst, err)
        assert err <= TOL, f"h={h}: max |diff| {err:.3e}"
    return worst


def _int4_tokens(T, seed):
    """Random tokens with degenerate ones mixed in: all zero, all -0, constant, positive only (minimum far
    above zero, or exactly +0), one-hot."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, 2, 128)).astype(np.float32)
    x[3] = 0.0
    x[4] = -0.0
    x[70:74] = 0.75
    x[75] = np.abs(x[75]) + 4.0
    x[76] = np.abs(x[76]); x[76, :, 5] = 0.0
    x[130] = 0.0; x[130, :, 17] = 3.0
    return x


def _heavy_unattended_token(wl, k, v, t):
    """Token t of every kv head gets values 10^4 times larger than the rest and a key pointing away from
    the sum of the head's queries, so each query head gives it a logit near -50: a value scale that
    dominates its page while its softmax weight is nil."""
    q = O.query_values(synth.queries(wl)[0])
    for h in range(wl.n_kv_heads):
        u = q[h * wl.gq:(h + 1) * wl.gq].sum(axis=0)
        k[t, h] = (-50.0 * np.sqrt(128.0) / np.abs(q[h * wl.gq:(h + 1) * wl.gq] @ (u / np.linalg.norm(u))).min()
                   * u / np.linalg.norm(u)).astype(np.float32)
        v[t, h] *= 1.0e4


@pytest.mark.parametrize("block", [16, 128])
def test_int4_token_degenerate_tokens_and_page_boundaries(K, block):
    """Codes and metadata bit-exact (zero points of zero tokens stored as +0), with appends that start and
    end inside pages: single tokens, a chunk ending one short of a page, a chunk crossing two pages."""
    wl = synth.scaled(SAW, hadamard_block=block)
    T = 400
    k, v = _int4_tokens(T, 11), _int4_tokens(T, 12)
    _heavy_unattended_token(wl, k, v, 200)
    _say(f"int4 per token, degenerate tokens, block {block}")
    _int4_write_and_check(K, wl, _bf16(k), _bf16(v), [1, 62, 1, 64, 1, 150, 121])


def test_int4_token_large_and_tiny_magnitudes(K):
    """Codes and metadata bit-exact for tokens at 1e30 and 1e-30 times the rest, and at 1e-38 (fp32
    subnormal sources after bf16 rounding and rotation)."""
    T = 200
    k, v = _int4_tokens(T, 17), _int4_tokens(T, 18)
    k[10], v[11] = k[10] * 1e30, v[11] * 1e30
    k[12], v[13] = k[12] * 1e-30, v[13] * 1e-30
    k[65], v[66] = k[65] * 1e-38, v[66] * 1e-38
    _say("int4 per token, large and tiny magnitudes")
    _int4_write_and_check(K, SAW, _bf16(k), _bf16(v), [70, 130], decode=False)


def test_int4_token_fp32_and_unaligned_sources(K):
    """An fp32 source (rounded to bf16 on entry) and bf16 sources 4 bytes past a 16-byte boundary (read a
    value at a time) store the same bits as the oracle."""
    T = 300
    k, v = _int4_tokens(T, 13), _int4_tokens(T, 14)
    _say("int4 per token, fp32 source")
    _int4_write_and_check(K, SAW, k, v, [100, 1, 199])
    _say("int4 per token, unaligned bf16 source")
    _int4_write_and_check(K, SAW, _bf16(k), _bf16(v), [100, 1, 199], misalign=True)


def test_int4_token_dense_rotation(K):
    """INT4 per token under a dense OSCAR rotation (QR x Hadamard x bit reversal)."""
    T = 333
    k, v = _int4_tokens(T, 15), _int4_tokens(T, 16)
    _say("int4 per token, dense rotation")
    _int4_write_and_check(K, synth.scaled(SAW, rotation="oscar"), _bf16(k), _bf16(v), [64, 5, 264])


# ------------------------------------------------------------------ the matrix-core INT2 decode


def test_matrix_core_decode_zero_and_constant_groups(K):
    """All-zero groups (alpha = 0 for every channel: every logit of the group equal) and constant tokens
    (every code equal) on the matrix-core decode."""
    T = 4 + 128 + 3 * 128 + 50
    rng = np.random.default_rng(5)
    k = rng.standard_normal((T, 2, 128)).astype(np.float32)
    v = rng.standard_normal((T, 2, 128)).astype(np.float32)
    k[4:132] = 0.0
    v[4:132] = 0.0
    k[132:260, 0, :] = 0.75
    v[132:260, 1, :] = -2.0
    _say("matrix-core decode: all-zero group, constant tokens")
    _write_and_check(K, WL, _bf16(k), _bf16(v), decode_impl=K.DECODE_MFMA)


def test_matrix_core_decode_no_clip_wide_range(K):
    T = 4 + 128 + 2 * 128 + 1
    rng = np.random.default_rng(7)
    k = (rng.standard_normal((T, 2, 128)) * 3).astype(np.float32)
    v = rng.standard_normal((T, 2, 128)).astype(np.float32)
    _say("matrix-core decode: clip ratio 1, keys x3")
    _write_and_check(K, WL, _bf16(k), _bf16(v), clip=(1.0, 1.0), decode_impl=K.DECODE_MFMA)


@pytest.mark.parametrize("T", [1, 5, 132, 259, 260, 261, 387, 388, 389, 516, 517])
def test_matrix_core_decode_boundary_lengths(K, T):
    rng = np.random.default_rng(100 + T)
    k = rng.standard_normal((T, 2, 128)).astype(np.float32)
    v = rng.standard_normal((T, 2, 128)).astype(np.float32)
    _say(f"matrix-core decode: boundary length T={T}")
    chunks = [1] * T if T < 8 else [T // 3, T - T // 3]
    _write_and_check(K, WL, _bf16(k), _bf16(v), chunks=chunks, decode_impl=K.DECODE_MFMA)


@pytest.mark.parametrize("T", [1, 5, 259, 260, 261, 389, 517])
def test_matrix_core_decode_per_token_boundary_lengths_and_constant_tokens(K, T):
    """Per-token INT2 on the matrix cores: boundary lengths, with a constant token (s = 1 rule) and an
    all-zero token inside the first group when there is one."""
    rng = np.random.default_rng(300 + T)
    k = rng.standard_normal((T, 2, 128)).astype(np.float32)
    v = rng.standard_normal((T, 2, 128)).astype(np.float32)
    if T > 140:
        k[10, 0, :] = 0.5
        v[11, 1, :] = 0.0
        k[12] = 0.0
    _say(f"matrix-core decode, per-token INT2: T={T}")
    chunks = [1] * T if T < 8 else [T // 3, T - T // 3]
    _write_and_check(K, synth.scaled(WL, scheme="int2_token"), _bf16(k), _bf16(v), chunks=chunks,
                     decode_impl=K.DECODE_MFMA)


@pytest.mark.parametrize("T", [5, 260, 389, 517])
def test_matrix_core_decode_per_channel_int4_edges(K, T):
    """Per-channel INT4 on the matrix cores: boundary lengths, an all-zero group and constant tokens."""
    rng = np.random.default_rng(500 + T)
    k = rng.standard_normal((T, 2, 128)).astype(np.float32)
    v = rng.standard_normal((T, 2, 128)).astype(np.float32)
    if T > 260:
        k[4:132] = 0.0
        v[132:260, 1, :] = -2.0
    _say(f"matrix-core decode, per-channel INT4: T={T}")
    chunks = [1] * T if T < 8 else [T // 3, T - T // 3]
    _write_and_check(K, synth.scaled(WL, scheme="int4_channel"), _bf16(k), _bf16(v), chunks=chunks,
                     decode_impl=K.DECODE_MFMA)
