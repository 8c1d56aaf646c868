"""GPU checks of the C ABI's boundary calls ([OSCAR] §3.4.5: the paged cache behind a page table).

kvq_debug_unpack reads a (sequence, kv head)'s quantized tokens back through the library; the result must equal
both the test-side layout readers (written from include/kvq.h independently of the kernels) and the oracle's
codes and bf16 scales/zeros, for every scheme.  A write whose host length bound passes the page-table row is
refused with KVQ_ERANGE before anything is enqueued, and leaves the cache as it was.
"""
import numpy as np
import pytest

import oracle as O
import synth
from kvq_cases import GROUPED, _host, _say, build_cache, read_int2_group, read_int4_tokens, source_of, source_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_15_amd as K
    return K


@pytest.mark.parametrize("scheme", ["int2_channel", "int2_token", "int4_channel", "int4_token"])
def test_debug_unpack_equals_layout_readers_and_oracle(K, scheme):
    base = synth.WORKLOADS["saw_int4_b16_16k" if scheme == "int4_token" else "gqa_b1_32k"]
    wl = base if scheme == "int4_token" else synth.scaled(base, scheme=scheme)
    lens = [1500, 700]
    _say(f"debug_unpack {scheme} lens={lens}")
    bc = build_cache(K, wl, lens, append_steps=2, chunk=512)
    pages, _ = _host(bc)
    for b in range(len(lens)):
        T = lens[b]
        for h in (0, 5):
            if scheme in GROUPED:
                ng = O.n_groups(T, bc.wl.n_sink, bc.wl.n_recent)
                codes, sz = K.kvq_debug_unpack(bc.cache, b, h, 128 * ng)
                codes, sz = codes.cpu().numpy(), sz.cpu().numpy().view(np.uint16)
                k, v = source_of(bc.wl, b, T)
                st = O.int2_state(k[:, h], v[:, h], T, bc.wl.n_sink, bc.wl.n_recent, bc.wl.clip_k, bc.wl.clip_v,
                                  bc.rk, bc.rv, axis=GROUPED[scheme])
                for g in range(ng):
                    rd = read_int2_group(bc, pages, b, h, g)
                    kc, vc = codes[128 * g:128 * (g + 1), 0], codes[128 * g:128 * (g + 1), 1]
                    assert np.array_equal(kc, rd["k_codes"]) and np.array_equal(vc, rd["v_codes"])
                    assert np.array_equal(kc, st["k_codes"][g]) and np.array_equal(vc, st["v_codes"][g])
                    if scheme == "int2_token":
                        got = sz[128 * g:128 * (g + 1)]  # [token][K|V][scale|zero]
                        for key, (side, e) in (("k_s16", (0, 0)), ("k_z16", (0, 1)), ("v_s16", (1, 0)), ("v_z16", (1, 1))):
                            assert np.array_equal(got[:, side, e], rd[key]) and np.array_equal(got[:, side, e], st[key][g])
                    else:
                        got = sz[g]  # [K|V][scale|zero][channel]
                        for key, (side, e) in (("k_s16", (0, 0)), ("k_z16", (0, 1)), ("v_s16", (1, 0)), ("v_z16", (1, 1))):
                            assert np.array_equal(got[side, e], rd[key]) and np.array_equal(got[side, e], st[key][g])
            else:
                codes, sz = K.kvq_debug_unpack(bc.cache, b, h, T)
                codes, sz = codes.cpu().numpy(), sz.cpu().numpy().view(np.uint16)
                rd = read_int4_tokens(bc, pages, b, h, T)
                k, v = source_of(bc.wl, b, T)
                st = O.int4_state(k[:, h], v[:, h], T, bc.rk.astype(np.int8),
                                  None if bc.rv is None else bc.rv.astype(np.int8), block=bc.wl.hadamard_block)
                assert np.array_equal(codes[:, 0], rd["k_codes"]) and np.array_equal(codes[:, 1], rd["v_codes"])
                assert np.array_equal(codes[:, 0], st["k_codes"]) and np.array_equal(codes[:, 1], st["v_codes"])
                for key, (side, e) in (("k_s16", (0, 0)), ("k_z16", (0, 1)), ("v_s16", (1, 0)), ("v_z16", (1, 1))):
                    assert np.array_equal(sz[:, side, e], rd[key]) and np.array_equal(sz[:, side, e], st[key])


def test_write_past_the_page_table_is_refused(K):
    import torch
    wl = synth.WORKLOADS["gqa_b1_32k"]
    lens = [1000, 400]
    bc = build_cache(K, wl, lens)
    cap = bc.max_pages  # pages of the longest sequence: 1000 tokens
    before = bc.cache.pages.clone(), bc.cache.band.clone(), bc.cache.seq_lens.clone()
    # 300 more tokens for sequence 0 would complete groups the row has no pages for
    n = 300
    assert K.pages_for_len(bc.cfg, 1000 + n) > cap
    k = source_torch(synth.kv_tokens(bc.wl, 0, 1000, n, "k"), "cuda")
    v = source_torch(synth.kv_tokens(bc.wl, 0, 1000, n, "v"), "cuda")
    cu = torch.tensor([0, n, n], dtype=torch.int32, device="cuda")
    with pytest.raises(K.KvqError) as e:
        K.kv_rotate_quant_write(bc.cache, k, v, cu, n)  # bound from the device lengths: 1000 + 300
    assert e.value.status == K.KVQ_ERANGE
    with pytest.raises(K.KvqError) as e:
        K.kv_rotate_quant_write(bc.cache, k, v, cu, n, max_len=1300)
    assert e.value.status == K.KVQ_ERANGE
    torch.cuda.synchronize()
    assert torch.equal(bc.cache.pages, before[0]) and torch.equal(bc.cache.band, before[1])
    assert torch.equal(bc.cache.seq_lens, before[2])
