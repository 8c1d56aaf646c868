"""GPU parity at the full sizes of the measured workloads, in the launch configuration the benchmark times
(automatic chunks for the batch workloads, the 512-token split at 4 x 131k), compared over many (sequence,
kv head) pairs spread across the batch and so across the split-K grid's chunk positions and XCDs:

- batch32_32k (32 x 32768 tokens, 32 q / 8 kv heads): every kv head of 8 sequences (64 pairs), the last 130
  tokens appended one at a time (one group demoted on the way), codes and band of sampled groups;
- long_b4_131k (4 x 131072 tokens, GQA 8, 512-token chunks): 8 pairs, codes at chunk and walk boundaries;
- batch32_8k_32k (ragged 8k..32k): 16 pairs;
- saw_int4_b16_16k (INT4 per token, 16 x 16384): 16 pairs, codes of sampled tokens.

The oracle's outputs come from CPU workers that started before the GPU was touched (oracle_pool).
"""
import numpy as np
import pytest

import oracle as O
import oracle_pool
import synth
from kvq_cases import TOL, _host, _say, build_cache, read_band, read_int2_group, read_int4_tokens, run_decode

pytestmark = pytest.mark.gpu

ORACLE_JOBS = {}


def _register(prefix, specs):
    keys = []
    for i, spec in enumerate(specs):
        key = f"{prefix}/{i}"
        ORACLE_JOBS[key] = spec
        keys.append(key)

    def deco(fn):
        fn.oracle_jobs = tuple(keys)
        return fn
    return deco, keys


# batch32_32k: all 8 kv heads of 8 sequences; codes of groups at the automatic chunks' boundaries (32 groups)
B32 = synth.WORKLOADS["batch32_32k"]
B32_LENS = synth.seq_lens(B32)
B32_SEQS = (0, 4, 9, 13, 18, 22, 27, 31)
_ng32 = O.n_groups(32768, B32.n_sink, B32.n_recent)
B32_GROUPS = [0, 31, 32, 127, 128, _ng32 - 1]
_b32, B32_KEYS = _register("b32", [oracle_pool.job("batch32_32k", B32_LENS, b, range(8),
                                                   groups={(b % 8): B32_GROUPS}) for b in B32_SEQS])

# long_b4_131k: two kv heads of every sequence; groups at 512-token chunk ends and at the ends of the walks
L4 = synth.WORKLOADS["long_b4_131k"]
L4_LENS = np.full(4, 131072, dtype=np.int64)
_ngl = O.n_groups(131072, L4.n_sink, L4.n_recent)
L4_GROUPS = [0, 3, 4, 19, 20, 500, _ngl - 1]
L4_PAIRS = [(0, 0), (0, 7), (1, 3), (1, 4), (2, 1), (2, 6), (3, 2), (3, 5)]
_l4, L4_KEYS = _register("l4", [oracle_pool.job("long_b4_131k", L4_LENS, b, [h], groups={h: L4_GROUPS})
                                for b, h in L4_PAIRS])

# batch32_8k_32k: two kv heads of 8 sequences
R32 = synth.WORKLOADS["batch32_8k_32k"]
R32_LENS = synth.seq_lens(R32)
R32_SEQS = (1, 5, 8, 14, 17, 23, 26, 30)
_r32, R32_KEYS = _register("r32", [oracle_pool.job("batch32_8k_32k", R32_LENS, b, [b % 8, (b + 3) % 8],
                                                   groups={b % 8: [0, int(O.n_groups(int(R32_LENS[b]), 4, 128)) - 1]})
                                   for b in R32_SEQS])

# saw_int4_b16_16k: four kv heads of 4 sequences, codes of tokens at page and page-pair boundaries
S16 = synth.WORKLOADS["saw_int4_b16_16k"]
S16_LENS = np.full(16, 16384, dtype=np.int64)
S16_TOKENS = [0, 63, 64, 127, 128, 8191, 8192, 16383]
_s16, S16_KEYS = _register("s16", [oracle_pool.job("saw_int4_b16_16k", S16_LENS, b, [(b + j) % 8 for j in range(0, 8, 2)],
                                                   tokens={b % 8: S16_TOKENS}) for b in (0, 5, 10, 15)])


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_15_amd as K
    return K


def _compare(bc, out, keys, pages=None, band=None):
    """Outputs of every pair of the jobs against the oracle (bar TOL), codes and band where sampled."""
    gq = bc.wl.gq
    worst, n = 0.0, 0
    for key in keys:
        spec = ORACLE_JOBS[key]
        b = spec["b"]
        res = oracle_pool.result(key, spec)
        _say(f"   oracle {key} (sequence {b}, kv heads {sorted(res)})")
        for h, r in res.items():
            got = out[b, h * gq:(h + 1) * gq]
            err = float(np.abs(got - r["out"]).max())
            assert err <= TOL, f"b={b} h={h} T={spec['lens'][b]}: max |diff| {err:.3e}"
            worst = max(worst, err)
            n += 1
            for g, want in r.get("groups", {}).items():
                have = read_int2_group(bc, pages, b, h, g)
                for name, arr in want.items():
                    assert np.array_equal(have[name], arr), f"b={b} h={h} group {g} {name}"
            if "band" in r:
                pos, bk, bv = r["band"]
                hk, hv = read_band(bc, band, b, h, pos)
                assert np.array_equal(hk, bk) and np.array_equal(hv, bv), f"band b={b} h={h}"
            if "tokens" in r and len(r["tokens"]):
                have = read_int4_tokens(bc, pages, b, h, int(spec["lens"][b]))
                for name, arr in r["state"].items():
                    assert np.array_equal(have[name][r["tokens"]], arr), f"b={b} h={h} {name}"
    return worst, n


@_b32
def test_batch32_32k_full_64_pairs(K):
    _say("full size: batch32_32k, 32 x 32768 (last 130 tokens appended), automatic chunks")
    bc = build_cache(K, B32, B32_LENS, append_steps=130, seqs_per_call=4)
    _say(f"   decode shape {K.decode_shape(bc.cfg, 32, 32768)}")
    q = synth.queries(B32)
    out = run_decode(K, bc, q)
    assert np.isfinite(out).all()
    pages, band = _host(bc)
    worst, n = _compare(bc, out, B32_KEYS, pages, band)
    _say(f"   {n} (sequence, kv head) pairs, worst |gpu - oracle| = {worst:.2e}")
    assert n == 64


@_l4
def test_long_b4_131k_full_8_pairs(K):
    _say("full size: long_b4_131k, 4 x 131072, GQA 8, 512-token chunks")
    bc = build_cache(K, L4, L4_LENS, split_tokens=512, seqs_per_call=1)
    _say(f"   decode shape {K.decode_shape(bc.cfg, 4, 131072)}")
    q = synth.queries(L4)
    out = run_decode(K, bc, q)
    assert np.isfinite(out).all()
    pages, band = _host(bc)
    worst, n = _compare(bc, out, L4_KEYS, pages, band)
    _say(f"   {n} pairs, worst |gpu - oracle| = {worst:.2e}")
    assert n == 8


@_r32
def test_batch32_ragged_full_16_pairs(K):
    _say(f"full size: batch32_8k_32k, lens {R32_LENS.min()}..{R32_LENS.max()}, automatic chunks")
    bc = build_cache(K, R32, R32_LENS, seqs_per_call=4)
    q = synth.queries(R32)
    out = run_decode(K, bc, q)
    assert np.isfinite(out).all()
    pages, band = _host(bc)
    worst, n = _compare(bc, out, R32_KEYS, pages, band)
    _say(f"   {n} pairs, worst |gpu - oracle| = {worst:.2e}")
    assert n == 16


@_s16
def test_saw_int4_full_16_pairs(K):
    _say("full size: saw_int4_b16_16k, 16 x 16384, 8192-token prefill chunks")
    bc = build_cache(K, S16, S16_LENS, chunk=8192, seqs_per_call=4)
    q = synth.queries(S16)
    out = run_decode(K, bc, q)
    assert np.isfinite(out).all()
    pages = bc.cache.pages.cpu().numpy()
    worst, n = _compare(bc, out, S16_KEYS, pages)
    _say(f"   {n} pairs, worst |gpu - oracle| = {worst:.2e}")
    assert n == 16
