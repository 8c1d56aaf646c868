"""Test-side helpers: build a device cache from the seeded inputs and read it back by the documented layout.

The unpackers below are written from the byte layout stated in include/kvq.h, independently of the
kernels, so a packing that disagrees with the documented format fails the parity tests even when the
GPU writer and reader agree with each other.
"""
from __future__ import annotations

from dataclasses import dataclass
import sys
from typing import Dict, List, Optional

import numpy as np

import oracle as O
import synth

I2_HEAD, I4_HEAD = 4608, 8704
TOL = 2e-3  # max |output - oracle| for every workload
# schemes with 128-token groups and a bf16 band, and the oracle's quantizer axis of each
GROUPED = {"int2_channel": "channel", "int2_token": "token", "int4_channel": "channel4"}


def head_bytes(scheme: str) -> int:
    return I2_HEAD if scheme in ("int2_channel", "int2_token") else I4_HEAD


def config_for(K, wl: synth.Workload, split_tokens: int = 0, decode_impl: int = 0):
    rot = K.ROT_DENSE if wl.rotation == "oscar" else K.ROT_HADAMARD
    if wl.scheme in GROUPED:
        scheme = {"int2_channel": K.INT2_CHANNEL, "int2_token": K.INT2_TOKEN, "int4_channel": K.INT4_CHANNEL}[wl.scheme]
        return K.make_config(wl.n_kv_heads, wl.n_q_heads, scheme, rot, wl.n_sink, wl.n_recent, wl.clip_k, wl.clip_v,
                             split_tokens, decode_impl, wl.key_only, wl.hadamard_block if wl.rotation == "saw" else 0)
    return K.make_config(wl.n_kv_heads, wl.n_q_heads, K.INT4_TOKEN, rot, 0, 0, 1.0, 1.0, split_tokens, decode_impl,
                         wl.key_only, wl.hadamard_block if wl.rotation == "saw" else 0)


def rotations(wl: synth.Workload):
    """fp32 rotation inputs from the oracle's builders: dense R (OSCAR) or sign vectors (SAW); the value
    rotation is None under key-only rotation."""
    if wl.rotation == "oscar":
        rk = O.oscar_rotation(synth.rotation_gaussian(wl, "k")).astype(np.float32)
        rv = O.oscar_rotation(synth.rotation_gaussian(wl, "v")).astype(np.float32)
    else:
        rk = synth.sign_vector(wl, "k").astype(np.float32)
        rv = synth.sign_vector(wl, "v").astype(np.float32)
    return rk, (None if wl.key_only else rv)


def source_torch(arr, device):
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(arr).to(device)


@dataclass
class BuiltCache:
    wl: synth.Workload
    cfg: object
    cache: object
    lens: np.ndarray
    rk: np.ndarray
    rv: Optional[np.ndarray]
    max_pages: int


def build_cache(K, wl: synth.Workload, lens, append_steps: int = 0, chunk: Optional[int] = None,
                split_tokens: int = 0, decode_impl: int = 0, device: str = "cuda", n_pool_extra: int = 3,
                seqs_per_call: Optional[int] = None) -> BuiltCache:
    """Write sequences of the given final lengths: a prefill of len - append_steps tokens (in chunks
    of `chunk` tokens if given), then `append_steps` one-token appends for every sequence."""
    import torch
    lens = np.asarray(lens, dtype=np.int64)
    B = len(lens)
    wl = synth.scaled(wl, batch=B)
    cfg = config_for(K, wl, split_tokens, decode_impl)
    max_pages = max(1, max(K.pages_for_len(cfg, int(t)) for t in lens))
    n_pool = B * max_pages + n_pool_extra
    pt = K.build_page_table(B, max_pages, n_pool, seed=0 if wl.identity_pages else wl.seed)
    rk, rv = rotations(wl)
    cache = K.allocate_cache(cfg, B, torch.from_numpy(pt), torch.from_numpy(rk),
                             None if rv is None else torch.from_numpy(rv), n_pages=n_pool, device=device)
    # unwritten bytes are 0xFF (bf16 NaN scales/zeros), so no kernel may read them into a result
    cache.pages.fill_(255)
    cache.band.fill_(-1)
    pre = np.maximum(lens - append_steps, 0)
    seqs_per_call = B if seqs_per_call is None else seqs_per_call
    # prefill, a group of sequences per call, optionally chunked
    for s0 in range(0, B, seqs_per_call):
        sel = list(range(s0, min(B, s0 + seqs_per_call)))
        done = np.zeros(B, dtype=np.int64)
        while True:
            n_new = np.zeros(B, dtype=np.int64)
            for b in sel:
                left = pre[b] - done[b]
                n_new[b] = left if chunk is None else min(left, chunk)
            if n_new.sum() == 0:
                break
            ks, vs = [], []
            for b in sel:
                if n_new[b]:
                    ks.append(synth.kv_tokens(wl, b, int(done[b]), int(n_new[b]), "k"))
                    vs.append(synth.kv_tokens(wl, b, int(done[b]), int(n_new[b]), "v"))
            cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
            k = source_torch(np.concatenate(ks), device)
            v = source_torch(np.concatenate(vs), device)
            K.kv_rotate_quant_write(cache, k, v, torch.from_numpy(cu).to(device), int(n_new.max()), max_len=int(lens.max()))
            done += n_new
            del k, v
    # one-token appends
    for s in range(append_steps):
        # token lens[b] - append_steps + s of every sequence that has it
        n_new = (lens - append_steps + s >= 0).astype(np.int64)
        ks = [synth.kv_tokens(wl, b, int(lens[b] - append_steps + s), 1, "k") for b in range(B) if n_new[b]]
        vs = [synth.kv_tokens(wl, b, int(lens[b] - append_steps + s), 1, "v") for b in range(B) if n_new[b]]
        if not ks:
            continue
        cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
        K.kv_rotate_quant_write(cache, source_torch(np.concatenate(ks), device),
                                source_torch(np.concatenate(vs), device), torch.from_numpy(cu).to(device), 1,
                                max_len=int(lens.max()))
    torch.cuda.synchronize()
    return BuiltCache(wl, cfg, cache, lens, rk, rv, max_pages)


# ------------------------------------------------------------------------- layout readers (from kvq.h)


def _page(pages: np.ndarray, page_bytes: int, phys: int) -> np.ndarray:
    return pages[phys * page_bytes:(phys + 1) * page_bytes]


def read_int4_channel_group(bc: BuiltCache, pages: np.ndarray, b: int, h: int, g: int) -> Dict[str, np.ndarray]:
    """INT4_CHANNEL: logical codes [128 tok, 128 ch] and per-channel bf16 scale/zero bits of one group."""
    pb = bc.wl.n_kv_heads * I4_HEAD
    pt = bc.cache.page_table.cpu().numpy()
    kc = np.zeros((128, 128), np.uint8)
    vc = np.zeros((128, 128), np.uint8)
    meta = []
    for pp in range(2):
        blk = _page(pages, pb, int(pt[b, 2 * g + pp]))[h * I4_HEAD:(h + 1) * I4_HEAD]
        # K: token i's 16 words; channel 16m + 2k + e in word 2m + e, nibble k
        kw = blk[0:4096].view(np.uint32).reshape(64, 16)
        for c in range(128):
            m, k, e = c // 16, (c % 16) // 2, c % 2
            kc[pp * 64:(pp + 1) * 64, c] = (kw[:, 2 * m + e] >> (4 * k)) & 15
        # V: channel c's 8 words; token 16j + 4g + 2hh + n in word 2g + n, nibble 2j + hh
        vw = blk[4096:8192].view(np.uint32).reshape(128, 8)
        for i in range(64):
            j, gg, hh, n = i // 16, (i // 4) % 4, (i // 2) % 2, i % 2
            vc[pp * 64 + i, :] = (vw[:, 2 * gg + n] >> (4 * (2 * j + hh))) & 15
        meta.append(blk[8192:8704].view(np.uint16))
    return {"k_codes": kc, "v_codes": vc, "k_s16": meta[0][:128], "k_z16": meta[0][128:],
            "v_s16": meta[1][:128], "v_z16": meta[1][128:]}


def read_int2_group(bc: BuiltCache, pages: np.ndarray, b: int, h: int, g: int) -> Dict[str, np.ndarray]:
    """Logical codes [128 tok, 128 ch] and bf16 scale/zero bits of one group of one (seq, kv head):
    per channel [128] (INT2_CHANNEL, INT4_CHANNEL) or per token of the group [128] (INT2_TOKEN)."""
    if bc.wl.scheme == "int4_channel":
        return read_int4_channel_group(bc, pages, b, h, g)
    n_kv = bc.wl.n_kv_heads
    pb = n_kv * I2_HEAD
    pt = bc.cache.page_table.cpu().numpy()
    kc = np.zeros((128, 128), np.uint8)
    vc = np.zeros((128, 128), np.uint8)
    meta = []
    for pp in range(2):
        blk = _page(pages, pb, int(pt[b, 2 * g + pp]))[h * I2_HEAD:(h + 1) * I2_HEAD]
        kb = blk[0:2048].reshape(64, 32)
        for c in range(128):
            kc[pp * 64:(pp + 1) * 64, c] = (kb[:, c // 4] >> (2 * (c % 4))) & 3
        vb = blk[2048:4096].reshape(128, 16)
        for i in range(64):
            j, gg, r = i // 16, (i // 4) % 4, i % 4
            vc[pp * 64 + i, :] = (vb[:, 4 * gg + j] >> (2 * r)) & 3
        meta.append(blk[4096:4608].view(np.uint16))
    if bc.wl.scheme == "int2_token":
        # each page: its 64 tokens' K scales, K zeros, V scales, V zeros
        part = [np.concatenate([meta[0][64 * i:64 * i + 64], meta[1][64 * i:64 * i + 64]]) for i in range(4)]
        return {"k_codes": kc, "v_codes": vc, "k_s16": part[0], "k_z16": part[1], "v_s16": part[2], "v_z16": part[3]}
    return {"k_codes": kc, "v_codes": vc, "k_s16": meta[0][:128], "k_z16": meta[0][128:],
            "v_s16": meta[1][:128], "v_z16": meta[1][128:]}


def read_int4_tokens(bc: BuiltCache, pages: np.ndarray, b: int, h: int, T: int) -> Dict[str, np.ndarray]:
    n_kv = bc.wl.n_kv_heads
    pb = n_kv * I4_HEAD
    pt = bc.cache.page_table.cpu().numpy()
    kc = np.zeros((T, 128), np.uint8)
    vc = np.zeros((T, 128), np.uint8)
    ks = np.zeros(T, np.uint16); kz = np.zeros(T, np.uint16)
    vs = np.zeros(T, np.uint16); vz = np.zeros(T, np.uint16)
    for p in range((T + 63) // 64):
        blk = _page(pages, pb, int(pt[b, p]))[h * I4_HEAD:(h + 1) * I4_HEAD]
        n = min(64, T - 64 * p)
        kb = blk[0:4096].reshape(64, 64)
        for c in range(128):
            kc[64 * p:64 * p + n, c] = ((kb[:n, c // 2] >> (4 * (c % 2))) & 15)
        vb = blk[4096:8192].reshape(128, 32)
        for i in range(n):
            j, gg, r = i // 16, (i // 4) % 4, i % 4
            vc[64 * p + i, :] = (vb[:, 8 * gg + 2 * j + r // 2] >> (4 * (r % 2))) & 15
        km = blk[8192:8448].view(np.uint16).reshape(64, 2)
        vm = blk[8448:8704].view(np.uint16).reshape(64, 2)
        ks[64 * p:64 * p + n], kz[64 * p:64 * p + n] = km[:n, 0], km[:n, 1]
        vs[64 * p:64 * p + n], vz[64 * p:64 * p + n] = vm[:n, 0], vm[:n, 1]
    return {"k_codes": kc, "v_codes": vc, "k_s16": ks, "k_z16": kz, "v_s16": vs, "v_z16": vz}


def read_band(bc: BuiltCache, band: np.ndarray, b: int, h: int, positions: np.ndarray):
    S0, W = bc.wl.n_sink, bc.wl.n_recent
    slots = S0 + W + 128
    base = ((b * bc.wl.n_kv_heads) + h) * slots * 256
    kk = np.zeros((len(positions), 128), np.uint16)
    vv = np.zeros((len(positions), 128), np.uint16)
    for n, t in enumerate(positions):
        slot = t if t < S0 else S0 + (t - S0) % (W + 128)
        row = band[base + slot * 256: base + slot * 256 + 256]
        kk[n], vv[n] = row[:128], row[128:]
    return kk, vv


def source_of(wl: synth.Workload, b: int, T: int):
    """Full source K and V of sequence b as [T, n_kv, 128] (fp32 or bf16 bits)."""
    return synth.kv_tokens(wl, b, 0, T, "k"), synth.kv_tokens(wl, b, 0, T, "v")


def oracle_out(bc: BuiltCache, q: np.ndarray, b: int, h: int, T: int) -> np.ndarray:
    """fp64 oracle output of the GQ q heads of kv head h of sequence b."""
    k, v = source_of(bc.wl, b, T)
    gq = bc.wl.gq
    qh = q[b, h * gq:(h + 1) * gq]
    if bc.wl.scheme in GROUPED:
        o, _ = O.decode_int2(qh, k[:, h], v[:, h], T, bc.wl.n_sink, bc.wl.n_recent, bc.wl.clip_k, bc.wl.clip_v,
                             bc.rk, bc.rv, axis=GROUPED[bc.wl.scheme])
    else:
        o, _ = O.decode_int4(qh, k[:, h], v[:, h], T, bc.rk.astype(np.int8),
                             None if bc.rv is None else bc.rv.astype(np.int8), block=bc.wl.hadamard_block)
    return o


def run_decode(K, bc: BuiltCache, q_np: np.ndarray, device: str = "cuda"):
    import torch
    q = source_torch(q_np, device)
    out = torch.empty(q.shape, dtype=torch.float32, device=device)
    maxT = int(bc.lens.max())
    ws = K.workspace_for(bc.cfg, len(bc.lens), maxT, device)
    K.kv_decode_attn(bc.cache, q, out, maxT, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


# ------------------------------------------------------------------------- checks against the oracle


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _host(bc):
    return bc.cache.pages.cpu().numpy(), bc.cache.band.cpu().numpy().view(np.uint16)


def check_int2(bc, b, h, groups=None, pages=None, band=None):
    if pages is None:
        pages, band = _host(bc)
    T = int(bc.lens[b])
    k, v = source_of(bc.wl, b, T)
    st = O.int2_state(k[:, h], v[:, h], T, bc.wl.n_sink, bc.wl.n_recent, bc.wl.clip_k, bc.wl.clip_v,
                      bc.rk, bc.rv, groups=groups, axis=GROUPED[bc.wl.scheme])
    for i, g in enumerate(st["groups"]):
        got = read_int2_group(bc, pages, b, h, int(g))
        for key in ("k_codes", "v_codes", "k_s16", "k_z16", "v_s16", "v_z16"):
            want = st[key][i]
            if not np.array_equal(got[key], want):
                bad = np.argwhere(got[key] != want)
                raise AssertionError(f"b={b} h={h} group={g} {key}: {len(bad)} mismatches, first {bad[:5].tolist()}")
    bk, bv = read_band(bc, band, b, h, st["band_pos"])
    assert np.array_equal(bk, st["band_k"]), f"band K b={b} h={h}"
    assert np.array_equal(bv, st["band_v"]), f"band V b={b} h={h}"
    return st


def check_int4(bc, b, h, pages):
    T = int(bc.lens[b])
    k, v = source_of(bc.wl, b, T)
    st = O.int4_state(k[:, h], v[:, h], T, bc.rk.astype(np.int8), None if bc.rv is None else bc.rv.astype(np.int8),
                      block=bc.wl.hadamard_block)
    got = read_int4_tokens(bc, pages, b, h, T)
    for key in ("k_codes", "v_codes", "k_s16", "k_z16", "v_s16", "v_z16"):
        if not np.array_equal(got[key], st[key]):
            bad = np.argwhere(got[key] != st[key])
            raise AssertionError(f"b={b} h={h} {key}: {len(bad)} mismatches, first {bad[:5].tolist()}")


def check_out(bc, out, q, pairs):
    worst = 0.0
    for b, h in pairs:
        T = int(bc.lens[b])
        gq = bc.wl.gq
        got = out[b, h * gq:(h + 1) * gq]
        if T == 0:
            assert np.array_equal(got, np.zeros_like(got))
            continue
        want = oracle_out(bc, q, b, h, T)
        err = np.abs(got - want).max()
        worst = max(worst, err)
        assert err <= TOL, f"b={b} h={h} T={T}: max |diff| {err:.3e}"
    return worst
