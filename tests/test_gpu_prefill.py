"""GPU parity of prefill attention over the quantized history ([NOVA] §3 "Long context": chunked prefill;
[SAW] prefill stage): after a chunk is written, each of its queries attends every cached token at a position
not after its own, as the cache holds it.  Against the oracle's causal attention on the same seeded inputs,
within the 2e-3 bar, for every scheme (INT2 per channel and per token, INT4 per channel over 128-token
groups with the bf16 band; INT4 per token over page pairs, randomized Hadamard of block 128 or 16); a
one-query chunk also equals the decode step's output.
"""
import numpy as np
import pytest

import oracle as O
import synth
from kvq_cases import GROUPED, TOL, _say, build_cache, run_decode, source_of, source_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_15_amd as K
    return K


def _prefill(K, bc, chunk):
    """Queries of each sequence's last chunk[b] positions through kv_prefill_attn -> [rows], host."""
    import torch
    wl = bc.wl
    qs, cu = [], [0]
    for b, n in enumerate(chunk):
        T = int(bc.lens[b])
        qs.append(synth.prefill_queries(wl, b, T - n, n))
        cu.append(cu[-1] + n)
    q = source_torch(np.concatenate(qs), "cuda")
    cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda")
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    ws = K.prefill_workspace_for(bc.cfg, q.shape[0])
    K.kv_prefill_attn(bc.cache, q, cu_t, max(chunk), out, ws)
    torch.cuda.synchronize()
    return np.concatenate(qs), np.array(cu), out.cpu().numpy()


def _check(bc, qs, cu, out, heads, rows=None):
    wl = bc.wl
    worst = 0.0
    for b in range(len(bc.lens)):
        T = int(bc.lens[b])
        n = cu[b + 1] - cu[b]
        sel = np.arange(n) if rows is None else np.asarray([r for r in rows if r < n])
        k, v = source_of(wl, b, T)
        for h in heads:
            qh = qs[cu[b] + sel][:, h * wl.gq:(h + 1) * wl.gq]
            if wl.scheme in GROUPED:
                want = O.prefill_int2(qh, T - n + sel, k[:, h], v[:, h], T, wl.n_sink, wl.n_recent, wl.clip_k,
                                      wl.clip_v, bc.rk, bc.rv, axis=GROUPED[wl.scheme])
            else:
                want = O.prefill_int4(qh, T - n + sel, k[:, h], v[:, h], T, bc.rk.astype(np.int8),
                                      None if bc.rv is None else bc.rv.astype(np.int8), block=wl.hadamard_block)
            got = out[cu[b] + sel][:, h * wl.gq:(h + 1) * wl.gq]
            assert np.isfinite(got).all(), f"b={b} h={h}: non-finite output"
            err = np.abs(got - want).max()
            worst = max(worst, err)
            assert err <= TOL, f"b={b} h={h}: max |diff| {err:.3e}"
    _say(f"   max |out - oracle| = {worst:.2e}")


@pytest.mark.parametrize("name,lens,chunk,heads", [
    ("gqa_b1_32k", [700, 300], [64, 37], [0, 5]),           # GQ 4; both chunks complete a group
    ("gqa_b1_32k", [390, 1100], [130, 200], [2]),           # chunks spanning group boundaries
    ("tiny_1h_4k", [2000], [150], [0]),                     # GQ 1, fp32 source, x10 outliers
    ("long_b4_131k", [900, 520], [70, 129], [1, 6]),        # GQ 8, W = 256, decaying spectrum
])
def test_prefill_chunk_matches_the_oracle(K, name, lens, chunk, heads):
    wl = synth.WORKLOADS[name]
    _say(f"prefill {name} lens={lens} chunk={chunk}")
    bc = build_cache(K, wl, lens, chunk=None)
    qs, cu, out = _prefill(K, bc, chunk)
    _check(bc, qs, cu, out, heads)


def test_prefill_key_only_rotation(K):
    wl = synth.scaled(synth.WORKLOADS["gqa_b1_32k"], key_only=True)
    _say("prefill, key-only rotation")
    bc = build_cache(K, wl, [800], chunk=None)
    qs, cu, out = _prefill(K, bc, [90])
    _check(bc, qs, cu, out, [3])


def test_prefill_of_one_query_is_the_decode_step(K):
    """A one-token chunk: the prefill output equals the decode output on the same cache and query."""
    import torch
    wl = synth.WORKLOADS["gqa_b1_32k"]
    lens = [1500, 333]
    bc = build_cache(K, wl, lens)
    qs, cu, out = _prefill(K, bc, [1, 1])
    dec = run_decode(K, bc, qs)  # rows are one per sequence: the decode's [batch, n_q, 128]
    assert np.abs(out - dec).max() <= TOL
    _check(bc, qs, cu, out, range(8))


def test_prefill_gqa_32k_sampled(K):
    """The GQA workload at full length: 28672 tokens of history, then a 4096-token chunk; sampled rows."""
    wl = synth.WORKLOADS["gqa_b1_32k"]
    _say("prefill gqa_b1_32k: 28672 + 4096 chunk")
    bc = build_cache(K, wl, [32768], chunk=8192)
    qs, cu, out = _prefill(K, bc, [4096])
    assert np.isfinite(out).all()
    _check(bc, qs, cu, out, [0, 7], rows=[0, 1, 127, 128, 1000, 2047, 4095])


# ------------------------------------------------------------------------- the other schemes


def _wl(name, **kw):
    return synth.scaled(synth.WORKLOADS[name], **kw)


SCHEME_CASES = [
    # (label, workload, lens, chunk, heads)
    ("int2 per token, GQ 4", _wl("gqa_b1_32k", scheme="int2_token"), [700, 390], [64, 130], [0, 5]),
    ("int2 per token, GQ 8", _wl("long_b4_131k", scheme="int2_token", batch=2), [900, 520], [70, 129], [1, 6]),
    ("int4 per channel, GQ 4", _wl("gqa_b1_32k", scheme="int4_channel"), [700, 1100], [64, 200], [2, 7]),
    ("int4 per channel, GQ 8", _wl("long_b4_131k", scheme="int4_channel", batch=2), [900, 520], [70, 129], [3]),
    ("int4 per token, GQ 4", _wl("saw_int4_b16_16k", batch=3), [700, 333, 1025], [64, 129, 200], [0, 6]),
    ("int4 per token, GQ 4, Hadamard block 16", _wl("saw_int4_b16_16k", batch=2, hadamard_block=16), [640, 97],
     [128, 97], [4]),
    ("int4 per token, GQ 8", _wl("saw_int4_b16_16k", batch=2, n_q_heads=64), [515, 190], [131, 63], [1, 7]),
    ("int4 per token, GQ 1", _wl("saw_int4_b16_16k", batch=1, n_q_heads=8), [300], [300], [2]),
]


@pytest.mark.parametrize("label,wl,lens,chunk,heads", SCHEME_CASES, ids=[c[0] for c in SCHEME_CASES])
def test_prefill_every_scheme(K, label, wl, lens, chunk, heads):
    _say(f"prefill {label}: lens={lens} chunk={chunk}")
    bc = build_cache(K, wl, lens, chunk=None)
    qs, cu, out = _prefill(K, bc, chunk)
    _check(bc, qs, cu, out, heads)


@pytest.mark.parametrize("name,kw", [("gqa_b1_32k", dict(scheme="int2_token")),
                                     ("gqa_b1_32k", dict(scheme="int4_channel")),
                                     ("saw_int4_b16_16k", dict(batch=2))])
def test_prefill_key_only_every_scheme(K, name, kw):
    wl = _wl(name, key_only=True, **kw)
    _say(f"prefill {wl.scheme}, key-only rotation")
    bc = build_cache(K, wl, [800, 300][:wl.batch] if wl.batch > 1 else [800], chunk=None)
    qs, cu, out = _prefill(K, bc, [90, 45][:len(bc.lens)])
    _check(bc, qs, cu, out, [3])


@pytest.mark.parametrize("name,kw", [("gqa_b1_32k", dict(scheme="int2_token")),
                                     ("gqa_b1_32k", dict(scheme="int4_channel")),
                                     ("saw_int4_b16_16k", dict(batch=2))])
def test_prefill_of_one_query_is_the_decode_step_every_scheme(K, name, kw):
    wl = _wl(name, **kw)
    lens = [1500, 333]
    bc = build_cache(K, wl, lens)
    qs, cu, out = _prefill(K, bc, [1, 1])
    dec = run_decode(K, bc, qs)
    d = np.abs(out - dec).max()
    _say(f"prefill {wl.scheme}: one query vs decode {d:.2e}")
    assert d <= TOL
    _check(bc, qs, cu, out, range(8))


def test_prefill_saw_int4_full_sampled(K):
    """The INT4 workload at full length: 16384 tokens, the last 8192 a chunk; sampled rows of 2 sequences."""
    wl = _wl("saw_int4_b16_16k", batch=2)
    _say("prefill saw_int4: 8192 + 8192 chunk")
    bc = build_cache(K, wl, [16384, 16384], chunk=8192)
    qs, cu, out = _prefill(K, bc, [8192, 8192])
    assert np.isfinite(out).all()
    _check(bc, qs, cu, out, [0, 5], rows=[0, 1, 63, 64, 127, 128, 4097, 8191])
