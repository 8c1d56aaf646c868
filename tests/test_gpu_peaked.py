"""GPU parity of the default (matrix-core) decodes under peaked attention.

The workloads' N(0,1) queries give flat attention.  Retrieval-style attention, which the pages evaluate
([OSCAR] "Long-Context Robustness on RULER-NIAH"), puts almost all weight on a few tokens; there the
logits' absolute error matters most, since a logit error e changes a dominant token's weight by about e.
These cases scale the workload's queries by 4, 8 and 16 (exact in bf16: powers of two) and build needle
queries, q = 2 k_t for a token t of the quantized history (a different t per query head), so that one
token's logit stands far above the rest.  Every scheme's default decode is compared element by element
with the fp64 oracle ([OSCAR] §3.4.4 steps 3-4; [SAW] App. A.4 eq. 13-14) at the same 2e-3 bar, at GQA 4
and GQA 8 (the two matrix-row layouts of the decode).
"""
import numpy as np
import pytest

import oracle as O
import synth
from kvq_cases import GROUPED, TOL, _say, build_cache, run_decode, source_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_15_amd as K
    return K


def _workload(scheme: str, gq: int) -> synth.Workload:
    if scheme == "int4_token":
        return synth.scaled(synth.WORKLOADS["saw_int4_b16_16k"], n_q_heads=8 * gq, n_kv_heads=8)
    return synth.scaled(synth.WORKLOADS["gqa_b1_32k"], scheme=scheme, n_q_heads=8 * gq, n_kv_heads=8)


def _keys_values(bc, b, h, T):
    """Oracle's dequantized, inverse-rotated keys and values of one (seq, kv head), fp64, and the token
    positions of their rows."""
    wl = bc.wl
    k, v = source_of(wl, b, T)
    if wl.scheme in GROUPED:
        st = O.int2_state(k[:, h], v[:, h], T, wl.n_sink, wl.n_recent, wl.clip_k, wl.clip_v, bc.rk, bc.rv,
                          axis=GROUPED[wl.scheme])
        K_, V_ = O.int2_keys_values(st, bc.rk, bc.rv)
        pos = O.token_positions(st, T, wl.n_sink, wl.n_recent)
        first_q = wl.n_sink  # first quantized position
        last_q = wl.n_sink + 128 * st["n_groups"]
    else:
        sk = bc.rk.astype(np.int8)
        sv = None if bc.rv is None else bc.rv.astype(np.int8)
        st = O.int4_state(k[:, h], v[:, h], T, sk, sv, block=wl.hadamard_block)
        K_, V_ = O.int4_keys_values(st, sk, sv, wl.hadamard_block)
        pos = np.arange(T)
        first_q, last_q = 0, T
    return K_, V_, pos, (first_q, last_q), k


def _queries(wl, lens, variant, srcs):
    """Query bits [batch, n_q, 128] for a variant: 'xS' scales the workload's queries by S, 'needle' sets
    q head j of kv head h to 2 k_t of a quantized-region token t that differs per head."""
    base = synth.queries(wl)
    f = O.bf16_value(base).astype(np.float32)
    if variant.startswith("x"):
        return synth.to_bf16_bits(f * np.float32(int(variant[1:])))
    q = np.empty_like(f)
    rng = np.random.default_rng(np.random.SeedSequence([wl.seed, 0x6E33D1E]))
    for b, T in enumerate(lens):
        for h in range(wl.n_kv_heads):
            k_src, (lo, hi) = srcs[(b, h)]
            for j in range(wl.gq):
                t = int(rng.integers(lo, hi))
                row = O.bf16_value(O.source_to_bf16(k_src[t:t + 1, h]))[0]
                q[b, h * wl.gq + j] = 2.0 * row
    return synth.to_bf16_bits(q)


VARIANTS = ["x1", "x4", "x8", "x16", "needle"]


@pytest.mark.parametrize("gq", [4, 8])
@pytest.mark.parametrize("scheme", ["int2_channel", "int2_token", "int4_channel", "int4_token"])
def test_peaked_attention_default_decode(K, scheme, gq):
    wl = _workload(scheme, gq)
    lens = [3000, 1700]
    _say(f"peaked attention: {scheme}, GQA {gq}, lens={lens}")
    bc = build_cache(K, wl, lens, append_steps=3)
    wlb = bc.wl
    kv = {}
    srcs = {}
    for b, T in enumerate(lens):
        for h in range(wlb.n_kv_heads):
            K_, V_, pos, rng_q, k_src = _keys_values(bc, b, h, T)
            kv[(b, h)] = (K_, V_)
            srcs[(b, h)] = (k_src, rng_q)
    worst = {}
    for var in VARIANTS:
        q = _queries(wlb, lens, var, srcs)
        out = run_decode(K, bc, q)
        qv = O.query_values(q)
        err = 0.0
        for b in range(len(lens)):
            for h in range(wlb.n_kv_heads):
                K_, V_ = kv[(b, h)]
                want = O.attend(qv[b, h * wlb.gq:(h + 1) * wlb.gq], K_, V_)
                got = out[b, h * wlb.gq:(h + 1) * wlb.gq]
                err = max(err, float(np.abs(got - want).max()))
        worst[var] = err
        _say(f"   {var:>6}: max |decode - oracle| = {err:.2e}")
    bad = {k: v for k, v in worst.items() if not v <= TOL}
    assert not bad, f"{scheme} GQA {gq}: over the {TOL} bar: {bad}"
