"""GPU parity of the split decode's merge at chunk counts that reach every part of its walk, against the
fp64 oracle (bar 2e-3).

The decode runs on the matrix cores with 128-token splits (one group per chunk), so a head has as many
chunk partials as quantized groups. Two work-group layouts are covered:
- few (sequence, kv head) pairs: one work-group per q head, 32 chunk slices;
- 128 pairs or more: one work-group per kv head, 8 slices per head.
Each case has more chunks than slices, so slices fold several partials and the loop after the first
chunk runs with its remainder. Ragged lengths leave most slices with no chunk, and one sequence ends
inside its band, with no quantized chunk at all.
"""
import pytest

import synth
from kvq_cases import _say, build_cache, check_out, run_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_15_amd as K
    return K


def _lens(wl, chunks, extra):
    """Lengths with `chunks` complete 128-token groups beyond the sink and window, plus `extra` tail tokens."""
    base = wl.n_sink + wl.n_recent
    return [base + 128 * c + e for c, e in zip(chunks, extra)]


def _run(K, wl, lens, pairs, append_steps):
    bc = build_cache(K, wl, lens, append_steps=append_steps, split_tokens=128, decode_impl=K.DECODE_MFMA)
    q = synth.queries(synth.scaled(wl, batch=len(lens)))
    out = run_decode(K, bc, q)
    worst = check_out(bc, out, q, pairs)
    _say(f"   worst |decode - oracle| = {worst:.2e}")


def test_merge_one_q_head_per_workgroup(K):
    wl = synth.WORKLOADS["gqa_b1_32k"]  # 8 kv heads: 4 sequences give 32 pairs (one q head per work-group)
    lens = _lens(wl, [75, 40, 3], [37, 5, 0]) + [100]
    _say(f"merge: 32 slices per q head, 128-token chunks, lens={lens} (75, 40, 3, 0 chunks), 2 appends")
    _run(K, wl, lens, [(b, h) for b in range(len(lens)) for h in range(wl.n_kv_heads)], append_steps=2)


def test_merge_one_kv_head_per_workgroup(K):
    wl = synth.WORKLOADS["gqa_b1_32k"]  # 16 sequences x 8 kv heads = 128 pairs (all GQ heads per work-group)
    chunks = [21, 9, 0, 17, 1, 8, 12, 3, 20, 5, 16, 2, 11, 7, 19, 4]
    lens = _lens(wl, chunks, [b * 7 % 120 for b in range(16)])
    lens[2] = 90  # inside the band: no quantized chunk
    _say(f"merge: 8 slices per head, 128-token chunks, 16 sequences with 0-21 chunks, 1 append")
    pairs = [(b, h) for b in (0, 1, 2, 3, 7, 8, 15) for h in (0, 3, 7)]
    _run(K, wl, lens, pairs, append_steps=1)
