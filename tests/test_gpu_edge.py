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


def _write_and_check(K, wl, kb, vb, clip=(0.96, 0.92), chunks=None, decode=True):
    """Write bf16 K/V [T, n_kv, 128] for one sequence, compare every group, the band and the decode output."""
    import torch
    T = kb.shape[0]
    wl = synth.scaled(wl, batch=1, clip_k=clip[0], clip_v=clip[1])
    cfg = config_for(K, wl)
    rk, rv = rotations(wl)
    max_pages = max(1, K.pages_for_len(cfg, T))
    pt, n_pool = synth.page_table(wl, max_pages, max_pages + 2)
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
