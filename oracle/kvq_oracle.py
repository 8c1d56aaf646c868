"""CPU oracle: decode attention over a rotated, 2/4-bit quantized, paged KV cache.

TEST INFRASTRUCTURE ONLY.  Tests, the smoke check and the bench's CPU-baseline
leg may import this module; the GPU library and its binding never do, and it
imports nothing from them.  It is plain, slow numpy/fp64 code that follows the
pages step by step.  Its inputs come from the seeded generators in `synth`.

Sources (cited by page title and section/equation):
  [OSCAR]  "OSCAR: Offline Spectral Covariance-Aware Rotation for 2-bit KV Cache
           Quantization" (English summary page), §3.2, §3.4.2, §3.4.4, §3.4.5.
  [SAW]    "SAW-INT4: System-AWare 4-Bit KV-Cache Quantization for Real-World LLM
           Serving", §3 eq. (1), §4.1, App. A.1 eq. (3)-(4), App. A.4 eq. (12)-(14).
  [NOVA]   "Spend Bits Where Queries Look: KV Cache Vector Quantization with
           Attention-Preserving Transforms", App. B.5 and the "Bit rate" paragraph.

Readings taken where the pages leave a step open (each listed in the design doc):
  R1  Cache values are bf16: an fp32 source is rounded to bf16 (round to nearest
      even) on entry, and the quantizer consumes those bf16 values, since the
      pages demote tokens from the bf16 recent window ([OSCAR] §3.4.5).
  R2  Dense rotation: x~_j = fp32( sum_i x_i * R[i][j] ), products exact in fp64
      (bf16 x fp32 needs 32 significand bits), summed in fp64 in increasing i,
      rounded once to fp32.  Randomized Hadamard ([SAW] §3, "applied via FWHT"):
      signs, then the radix-2 butterflies (a+b, a-b) for h = 1, 2, ..., 64 in
      fp64, then a multiply by 1/sqrt(128) = sqrt(2)*2^-4 in fp64, rounded to fp32.
      Block order h < 128 ([SAW] eq. (1)): butterflies for h' < h only, within each
      block, and 1/sqrt(h) = 2^(-k/2) (k = log2 h even) or sqrt(2)*2^(-(k+1)/2) (odd).
  R3  Clip ([OSCAR] §3.4.4 step 2): tau = linear-interpolation quantile of |x~|
      over the 128 channels: y sorted ascending, h = 127*rho (double), j = floor(h),
      f = fp32(h - j), tau = y[j] + f*(y[j+1]-y[j]) in fp32 with each operation
      rounded (no fused multiply-add); tau = y[127] when j = 127.
  R4  INT2 axis: per channel over 128-token groups (the workload's statement);
      the clip stays per token, before the group min/max.  The per-token reading of
      the English page (min/max over a token's 128 channels) is the second INT2
      scheme; both demote whole 128-token groups (R7).
  R5  Scale and zero ([OSCAR] §3.4.4 step 3): s = (b-a)/3 in fp32 (s = 1 if b == a),
      stored as bf16; z = -a/s' with the stored s', stored as bf16; the encoder
      uses the stored s', z' so encode and decode agree.  Code
      q = clamp(rint(fp32(fp32(x/s') + z')), 0, 3), rint = half to even.
  R6  INT4 ([SAW] eq. (3)-(4)): per token, s = (max-min)/15 (bf16 stored), integer
      z = rint(-min/s') (bf16 stored), q = clamp(rint(x/s') + z', 0, 15).
  R18 The integer zero point of R6 has one zero, stored as +0 (a zero minimum, or
      -min/s' of magnitude below one half, would otherwise give -0 or +0 by sign).
  R7  Layout of a length-T cache: tokens [0, S0) are the bf16 sink; groups
      g = 0..n_g-1 cover [S0+128g, S0+128(g+1)) with n_g = max(0, (T-S0-W)//128);
      the rest is the bf16 tail (W..W+127 tokens once T >= S0+W).
  R8  Attention ([OSCAR] §3.4.4 step 4): the decode query attends every cached
      token; dequantized tokens are x^ = s'(q - z') in the rotated frame and
      k^ = x^ R_K^T, v^ = x^ R_V^T; bf16 band tokens are used as stored.
      logits = q.k/sqrt(128), softmax, weighted sum of values, all in fp64.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Dict, Optional

import numpy as np

D = 128
GROUP = 128

# ----------------------------------------------------------------------------
# bf16 storage ([OSCAR] §3.4.4: bf16 scale/zero; §3.4.5: bf16 sink/recent)
# ----------------------------------------------------------------------------


def bf16_rne(x) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return ((u >> 16) & 0xFFFF).astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    """bf16 bit pattern -> float32 value (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def source_to_bf16(src: np.ndarray) -> np.ndarray:
    """Reading R1: the cache holds bf16; fp32 sources are rounded, bf16 sources pass."""
    if src.dtype == np.uint16:
        return src
    return bf16_rne(src)


# ----------------------------------------------------------------------------
# Rotation builders ([OSCAR] §3.4.2; [SAW] §3 eq. (1))
# ----------------------------------------------------------------------------


def hadamard(d: int = D) -> np.ndarray:
    """Normalized Walsh-Hadamard matrix, Sylvester order: H[i][j] = (-1)^popcount(i&j)/sqrt(d).

    [OSCAR] §3.4.2 Factor 2: orthogonal, every entry +-1/sqrt(d).
    """
    i = np.arange(d)
    par = np.array([[bin(a & b).count("1") & 1 for b in i] for a in i])
    return np.where(par == 0, 1.0, -1.0) / np.sqrt(d)


def bit_reversal(d: int = D) -> np.ndarray:
    """beta(k): k with its log2(d) bits reversed ([OSCAR] §3.4.2 Factor 3)."""
    nb = d.bit_length() - 1
    return np.array([int(format(k, f"0{nb}b")[::-1], 2) for k in range(d)])


def bit_reversal_matrix(d: int = D) -> np.ndarray:
    """P_br with P[k][beta(k)] = 1: (X P_br)[:, beta(k)] = X[:, k]."""
    P = np.zeros((d, d))
    P[np.arange(d), bit_reversal(d)] = 1.0
    return P


def orthonormal_from_gaussian(G: np.ndarray) -> np.ndarray:
    """Q factor of a Householder QR of G, signs fixed so that diag(R) > 0.

    Stands in for the calibrated eigenbasis U of [OSCAR] §3.2 step 3 (the
    workload fixes U as the QR of a seeded Gaussian; no calibration data here).
    """
    Q, Rt = np.linalg.qr(G)
    s = np.sign(np.diag(Rt))
    s[s == 0] = 1.0
    return Q * s[None, :]


def oscar_rotation(G: np.ndarray) -> np.ndarray:
    """R = U . H_Had . P_br in fp64 ([OSCAR] §3.4.2, order U first, H second, P_br last)."""
    return orthonormal_from_gaussian(G) @ hadamard(G.shape[0]) @ bit_reversal_matrix(G.shape[0])


def saw_rotation_matrix(sign: np.ndarray, block: int = D) -> np.ndarray:
    """Dense fp64 form of the randomized block-diagonal Hadamard diag(sign) . diag(H_h, ..., H_h)
    ([SAW] §3 eq. (1): each block of h channels rotated by the same normalized h x h Hadamard)."""
    d = len(sign)
    Hb = np.zeros((d, d))
    for i in range(0, d, block):
        Hb[i:i + block, i:i + block] = hadamard(block)
    return np.asarray(sign, dtype=np.float64)[:, None] * Hb


# ----------------------------------------------------------------------------
# Rotation from a calibration covariance ([OSCAR] §3.2 offline steps 2-3,
# §3.4.2 Factor 1)
# ----------------------------------------------------------------------------


def query_covariance(q) -> np.ndarray:
    """C_Q = (1/N) sum_n q_n^T q_n over N query rows ([OSCAR] §3.2 step 2(a)), fp64."""
    q = np.asarray(q, dtype=np.float64).reshape(-1, D)
    return q.T @ q / q.shape[0]


def score_value_covariance(v, s) -> np.ndarray:
    """C_S = (1/N) V^T S^T S V for values V [n_keys][d] and scores S [N][n_keys] ([OSCAR] §3.2 step 2(b))."""
    X = np.asarray(s, dtype=np.float64) @ np.asarray(v, dtype=np.float64).reshape(-1, D)
    return X.T @ X / X.shape[0]


def eigenbasis(C):
    """C = U diag(lam) U^T with lam descending ([OSCAR] §3.4.2 Factor 1, lambda_1 >= ... >= lambda_d).

    numpy's symmetric eigensolver is the library step.  Each eigenvector's sign is fixed so that its
    entry of largest magnitude (first such index) is positive.  Returns (U, lam).
    """
    lam, V = np.linalg.eigh(np.asarray(C, dtype=np.float64))
    order = np.argsort(-lam, kind="stable")
    lam, V = lam[order], V[:, order]
    top = np.argmax(np.abs(V), axis=0)
    sign = np.where(V[top, np.arange(V.shape[1])] < 0, -1.0, 1.0)
    return V * sign[None, :], lam


def oscar_rotation_from_covariance(C) -> np.ndarray:
    """R = U . H_Had . P_br with U the eigenbasis of the calibration covariance ([OSCAR] §3.2 step 3)."""
    U, _ = eigenbasis(C)
    d = U.shape[0]
    return U @ hadamard(d) @ bit_reversal_matrix(d)


# ----------------------------------------------------------------------------
# Write path ([OSCAR] §3.4.4 steps 1-3, §3.4.5 prefill kernel steps 1-6)
# ----------------------------------------------------------------------------


def rotate_dense(x: np.ndarray, R32: np.ndarray) -> np.ndarray:
    """Reading R2: x~ = x . R, fp64 products summed in increasing channel index, one fp32 rounding.

    x: [N, 128] values exactly representable in bf16; R32: [128, 128] float32.
    """
    x64 = np.asarray(x, dtype=np.float64)
    R64 = np.asarray(R32, dtype=np.float32).astype(np.float64)
    acc = np.zeros((x64.shape[0], R64.shape[1]))
    for i in range(R64.shape[0]):
        acc = acc + x64[:, i:i + 1] * R64[i:i + 1, :]
    return acc.astype(np.float32)


INV_SQRT128_F64 = float(np.ldexp(np.sqrt(2.0), -4))


def fwht_fp64(y: np.ndarray, block: Optional[int] = None) -> np.ndarray:
    """Unnormalized radix-2 Walsh-Hadamard transform along the last axis, fp64, on every block of
    `block` consecutive entries (default: the whole axis).

    Stage h (h = 1, 2, ..., block/2) maps each pair (i, i+h) with i & h == 0 to (a+b, a-b).
    """
    y = np.array(y, dtype=np.float64, copy=True)
    d = y.shape[-1]
    block = d if block is None else block
    h = 1
    while h < block:
        yr = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = yr[..., 0, :].copy()
        b = yr[..., 1, :].copy()
        yr[..., 0, :] = a + b
        yr[..., 1, :] = a - b
        h *= 2
    return y


def hadamard_scale(block: int) -> float:
    """fp64 normalization 1/sqrt(h) of an order-h = 2^k Hadamard block (reading R2): 2^(-k/2) exactly for
    even k, fp64(sqrt(2)) * 2^(-(k+1)/2) for odd k (so h = 128 gives sqrt(2) * 2^-4)."""
    k = block.bit_length() - 1
    assert block == 1 << k
    return 2.0 ** (-k // 2) if k % 2 == 0 else float(np.sqrt(2.0)) * 2.0 ** (-(k + 1) // 2)


def rotate_hadamard(x: np.ndarray, sign: np.ndarray, block: int = D) -> np.ndarray:
    """Reading R2 for the randomized (block-diagonal) Hadamard of [SAW] §3 eq. (1):
    x . diag(sign) . diag(H_h, ..., H_h), computed per block via FWHT in fp64, rounded once."""
    y = np.asarray(x, dtype=np.float64) * np.asarray(sign, dtype=np.float64)[None, :]
    return (fwht_fp64(y, block) * hadamard_scale(block)).astype(np.float32)


def clip_index(rho: float):
    """(j, f) of the linear-interpolation quantile at level rho over 128 channels (reading R3)."""
    rho32 = float(np.float32(rho))
    if not (0.0 < rho32 <= 1.0):
        raise ValueError("clip ratio must lie in (0, 1]")
    h = 127.0 * rho32
    j = int(np.floor(h))
    return j, np.float32(h - j)


def clip_threshold(xt: np.ndarray, rho: float) -> np.ndarray:
    """tau_t = quantile_rho(|x~_t|) per token ([OSCAR] §3.4.4 step 2), reading R3."""
    j, f = clip_index(rho)
    y = np.sort(np.abs(np.asarray(xt, dtype=np.float32)), axis=1)
    if j >= D - 1:
        return y[:, D - 1].copy()
    diff = (y[:, j + 1] - y[:, j]).astype(np.float32)
    step = (f * diff).astype(np.float32)
    return (y[:, j] + step).astype(np.float32)


def clip_tokens(xt: np.ndarray, rho: float) -> np.ndarray:
    """clip(x~_t, -tau_t, tau_t) per token ([OSCAR] §3.4.4 step 2)."""
    tau = clip_threshold(xt, rho)[:, None]
    return np.minimum(np.maximum(xt, -tau), tau).astype(np.float32)


F32 = np.float32


def quantize_int2_channel_group(xc: np.ndarray, qmax: int = 3):
    """Asymmetric affine INT2 of one 128-token group, per channel ([OSCAR] §3.4.4 step 3; R4, R5);
    qmax = 15 gives the per-channel INT4 variant with the same arithmetic.

    xc: [128 tokens, 128 channels] float32 (clipped, rotated).
    Returns codes uint8 [tokens, channels], s16 and z16 bf16 bits [channels].
    """
    xc = np.asarray(xc, dtype=np.float32)
    a = xc.min(axis=0)
    b = xc.max(axis=0)
    s = np.where(b > a, ((b - a).astype(F32) / F32(qmax)).astype(F32), F32(1)).astype(F32)
    s16 = bf16_rne(s)
    sp = bf16_value(s16)
    z = ((-a).astype(F32) / sp).astype(F32)
    z16 = bf16_rne(z)
    zp = bf16_value(z16)
    t = (xc / sp[None, :]).astype(F32)
    t = (t + zp[None, :]).astype(F32)
    q = np.clip(np.rint(t), 0, qmax).astype(np.uint8)
    return q, s16, z16


def quantize_int2_token(x: np.ndarray):
    """Asymmetric affine INT2 per token over its 128 channels ([OSCAR] §3.4.4 step 3 as the English page
    states it: per-token min-max over a group of G = 128 channels; R5's rounding, per token).

    x: [N tokens, 128 channels] float32 (clipped, rotated).
    Returns codes uint8 [N, 128], s16 and z16 bf16 bits [N].
    """
    x = np.asarray(x, dtype=np.float32)
    a = x.min(axis=1)
    b = x.max(axis=1)
    s = np.where(b > a, ((b - a).astype(F32) / F32(3)).astype(F32), F32(1)).astype(F32)
    s16 = bf16_rne(s)
    sp = bf16_value(s16)
    z = ((-a).astype(F32) / sp).astype(F32)
    z16 = bf16_rne(z)
    zp = bf16_value(z16)
    t = (x / sp[:, None]).astype(F32)
    t = (t + zp[:, None]).astype(F32)
    q = np.clip(np.rint(t), 0, 3).astype(np.uint8)
    return q, s16, z16


def quantize_int4_token(x: np.ndarray):
    """Token-wise asymmetric INT4 ([SAW] App. A.1 eq. (3)-(4); reading R6).

    x: [N, 128] float32 (rotated).  Returns codes uint8 [N, 128], s16, z16 [N].
    """
    x = np.asarray(x, dtype=np.float32)
    a = x.min(axis=1)
    b = x.max(axis=1)
    s = np.where(b > a, ((b - a).astype(F32) / F32(15)).astype(F32), F32(1)).astype(F32)
    s16 = bf16_rne(s)
    sp = bf16_value(s16)
    # z is an integer ([SAW] eq. (3)), and an integer has one zero: stored as +0 (reading R18), so the sign
    # of a zero minimum never reaches the stored bits
    z = (np.rint(((-a).astype(F32) / sp).astype(F32)).astype(F32) + F32(0)).astype(F32)
    z16 = bf16_rne(z)
    zp = bf16_value(z16)
    r = np.rint((x / sp[:, None]).astype(F32)).astype(F32)
    q = np.clip((r + zp[:, None]).astype(F32), 0, 15).astype(np.uint8)
    return q, s16, z16


def dequantize(codes: np.ndarray, s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """x^ = s'(q - z') in fp64 ([OSCAR] §3.4.4 step 3; [SAW] eq. (4)); s16/z16 broadcast."""
    sp = bf16_value(s16).astype(np.float64)
    zp = bf16_value(z16).astype(np.float64)
    return sp * (codes.astype(np.float64) - zp)


# ----------------------------------------------------------------------------
# Cache state of one (sequence, kv head) for a context of length T (reading R7)
# ----------------------------------------------------------------------------


def n_groups(T: int, n_sink: int, n_recent: int) -> int:
    return max(0, (T - n_sink - n_recent) // GROUP)


def band_positions(T: int, n_sink: int, n_recent: int) -> np.ndarray:
    """Token positions kept in bf16: the sink and the tail."""
    ng = n_groups(T, n_sink, n_recent)
    sink = np.arange(min(T, n_sink))
    tail = np.arange(n_sink + GROUP * ng, T) if T > n_sink else np.arange(0)
    return np.concatenate([sink, tail]).astype(np.int64)


def int2_state(k_src, v_src, T: int, n_sink: int, n_recent: int, clip_k: float, clip_v: float,
               R_K32: np.ndarray, R_V32: Optional[np.ndarray], groups=None, axis: str = "channel"
               ) -> Dict[str, np.ndarray]:
    """Quantized state of one (seq, kv head) holding tokens [0, T) under an INT2 scheme.

    k_src/v_src: [>=T, 128] float32 or bf16 bits.  `groups` limits the groups computed
    (for sampled checks on large caches); default all.  axis: "channel" (R4: per channel over
    the group) or "token" (per token over its channels).  R_V32 = None: key-only rotation, the
    values are quantized in their own frame.
    """
    # axis "channel4": the per-channel INT4 variant (same groups, band and arithmetic, 15 levels)
    quant = {"channel": quantize_int2_channel_group, "token": quantize_int2_token,
             "channel4": lambda x: quantize_int2_channel_group(x, 15)}[axis]
    kb = source_to_bf16(np.asarray(k_src)[:T])
    vb = source_to_bf16(np.asarray(v_src)[:T])
    ng = n_groups(T, n_sink, n_recent)
    gl = list(range(ng)) if groups is None else list(groups)
    out = {"n_groups": ng, "groups": np.array(gl, dtype=np.int64), "axis": axis,
           "band_pos": band_positions(T, n_sink, n_recent)}
    out["band_k"] = kb[out["band_pos"]]
    out["band_v"] = vb[out["band_pos"]]
    kc, vc, ks, kz, vs, vz = [], [], [], [], [], []
    for g in gl:
        t0 = n_sink + GROUP * g
        xk = rotate_dense(bf16_value(kb[t0:t0 + GROUP]), R_K32)
        xv = bf16_value(vb[t0:t0 + GROUP]) if R_V32 is None else rotate_dense(bf16_value(vb[t0:t0 + GROUP]), R_V32)
        qk, sk, zk = quant(clip_tokens(xk, clip_k))
        qv, sv, zv = quant(clip_tokens(xv, clip_v))
        kc.append(qk); vc.append(qv); ks.append(sk); kz.append(zk); vs.append(sv); vz.append(zv)
    e8 = np.zeros((0, GROUP, D), np.uint8)
    e16 = np.zeros((0, D), np.uint16)
    out["k_codes"] = np.stack(kc) if kc else e8
    out["v_codes"] = np.stack(vc) if vc else e8
    out["k_s16"] = np.stack(ks) if ks else e16
    out["k_z16"] = np.stack(kz) if kz else e16
    out["v_s16"] = np.stack(vs) if vs else e16
    out["v_z16"] = np.stack(vz) if vz else e16
    return out


def int4_state(k_src, v_src, T: int, sign_k: np.ndarray, sign_v: Optional[np.ndarray],
               tokens=None, block: int = D) -> Dict[str, np.ndarray]:
    """Token-wise INT4 state of one (seq, kv head) after the randomized Hadamard ([SAW]); sign_v = None:
    key-only rotation ([SAW] App. C), values quantized in their own frame."""
    idx = np.arange(T) if tokens is None else np.asarray(tokens)
    kb = source_to_bf16(np.asarray(k_src)[idx])
    vb = source_to_bf16(np.asarray(v_src)[idx])
    qk, sk, zk = quantize_int4_token(rotate_hadamard(bf16_value(kb), sign_k, block))
    xv = bf16_value(vb) if sign_v is None else rotate_hadamard(bf16_value(vb), sign_v, block)
    qv, sv, zv = quantize_int4_token(xv)
    return {"tokens": idx, "k_codes": qk, "k_s16": sk, "k_z16": zk,
            "v_codes": qv, "v_s16": sv, "v_z16": zv}


# ----------------------------------------------------------------------------
# Attention (reading R8)
# ----------------------------------------------------------------------------


def attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray) -> np.ndarray:
    """softmax(q K^T / sqrt(d)) V for each query row, fp64 ([OSCAR] §3.4.5 eq. for O)."""
    q = np.asarray(q, dtype=np.float64)
    logits = q @ np.asarray(keys, dtype=np.float64).T / np.sqrt(q.shape[-1])
    m = logits.max(axis=-1, keepdims=True)
    p = np.exp(logits - m)
    p /= p.sum(axis=-1, keepdims=True)
    return p @ np.asarray(vals, dtype=np.float64)


def int2_keys_values(state, R_K32, R_V32):
    """Dequantized, inverse-rotated K^ and V^ of every group plus the bf16 band, fp64 (R_V32 = None:
    the values were not rotated)."""
    RK = np.asarray(R_K32, dtype=np.float32).astype(np.float64)
    RV = np.eye(D) if R_V32 is None else np.asarray(R_V32, dtype=np.float32).astype(np.float64)
    keys = [bf16_value(state["band_k"]).astype(np.float64)]
    vals = [bf16_value(state["band_v"]).astype(np.float64)]
    # per-channel scales broadcast over tokens (rows), per-token ones over channels (columns)
    bc = (lambda x: x[:, None]) if state.get("axis", "channel") == "token" else (lambda x: x[None, :])
    for i in range(len(state["groups"])):
        xk = dequantize(state["k_codes"][i], bc(state["k_s16"][i]), bc(state["k_z16"][i]))
        xv = dequantize(state["v_codes"][i], bc(state["v_s16"][i]), bc(state["v_z16"][i]))
        keys.append(xk @ RK.T)
        vals.append(xv @ RV.T)
    return np.concatenate(keys), np.concatenate(vals)


def int4_keys_values(state, sign_k, sign_v, block: int = D):
    RK = saw_rotation_matrix(sign_k, block)
    RV = np.eye(D) if sign_v is None else saw_rotation_matrix(sign_v, block)
    xk = dequantize(state["k_codes"], state["k_s16"][:, None], state["k_z16"][:, None])
    xv = dequantize(state["v_codes"], state["v_s16"][:, None], state["v_z16"][:, None])
    # the write multiplied by fp64(1/sqrt(128)); H here is exactly orthonormal in fp64
    return xk @ RK.T, xv @ RV.T


def query_values(q) -> np.ndarray:
    """Decode query as fp64: bf16 bit patterns or float32 values."""
    q = np.asarray(q)
    if q.dtype == np.uint16:
        return bf16_value(q).astype(np.float64)
    return q.astype(np.float64)


def decode_int2(q_heads, k_src, v_src, T, n_sink, n_recent, clip_k, clip_v, R_K32, R_V32, axis="channel"):
    """Output [g_q, 128] for the query heads sharing one kv head, INT2 schemes, fp64."""
    st = int2_state(k_src, v_src, T, n_sink, n_recent, clip_k, clip_v, R_K32, R_V32, axis=axis)
    K, V = int2_keys_values(st, R_K32, R_V32)
    return attend(query_values(q_heads), K, V), st


def token_positions(state, T: int, n_sink: int, n_recent: int) -> np.ndarray:
    """Positions of the tokens in the order int2_keys_values returns them: band, then groups."""
    pos = [np.asarray(state["band_pos"], dtype=np.int64)]
    for g in state["groups"]:
        pos.append(n_sink + GROUP * int(g) + np.arange(GROUP))
    return np.concatenate(pos)


def attend_causal(q_rows: np.ndarray, q_pos: np.ndarray, keys: np.ndarray, vals: np.ndarray,
                  key_pos: np.ndarray) -> np.ndarray:
    """Row i of q_rows [n, g_q, d] attends the keys with position <= q_pos[i] ([NOVA] §3 "Long context":
    chunked prefill over the cache as it stands after the chunk's write), fp64."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    out = np.zeros(q_rows.shape)
    for i in range(q_rows.shape[0]):
        vis = key_pos <= q_pos[i]
        out[i] = attend(q_rows[i], keys[vis], vals[vis])
    return out


def prefill_int2(q_rows, q_pos, k_src, v_src, T, n_sink, n_recent, clip_k, clip_v, R_K32, R_V32, axis="channel"):
    """Prefill attention of the chunk's queries over an INT2 cache of length T (chunk included)."""
    st = int2_state(k_src, v_src, T, n_sink, n_recent, clip_k, clip_v, R_K32, R_V32, axis=axis)
    K, V = int2_keys_values(st, R_K32, R_V32)
    return attend_causal(query_values(q_rows), np.asarray(q_pos), K, V, token_positions(st, T, n_sink, n_recent))


def prefill_int4(q_rows, q_pos, k_src, v_src, T, sign_k, sign_v, block: int = D):
    """Prefill attention of the chunk's queries over an INT4 per-token cache of length T (chunk included):
    the chunk is written (rotated and quantized per token) before its queries read the cache back ([SAW]
    prefill stage; [NOVA] §3 "Long context"), so every visible token, the chunk's own included, is read
    dequantized and inverse-rotated."""
    st = int4_state(k_src, v_src, T, sign_k, sign_v, block=block)
    K, V = int4_keys_values(st, sign_k, sign_v, block)
    return attend_causal(query_values(q_rows), np.asarray(q_pos), K, V, np.arange(T))


def decode_int4(q_heads, k_src, v_src, T, sign_k, sign_v, block: int = D):
    st = int4_state(k_src, v_src, T, sign_k, sign_v, block=block)
    K, V = int4_keys_values(st, sign_k, sign_v, block)
    return attend(query_values(q_heads), K, V), st


# ----------------------------------------------------------------------------
# Exact rational helpers (used by pins; slow)
# ----------------------------------------------------------------------------


def exact_dot(x, col) -> Fraction:
    """Exact rational value of sum_i x_i * col_i for floating-point inputs."""
    return sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x, col)), Fraction(0))


def round_fraction_to_f32(v: Fraction) -> np.float32:
    """Round an exact rational to the nearest float32 (ties to even), normal range."""
    if v == 0:
        return np.float32(0.0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # scale so that the integer part holds 24 significant bits
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    scaled = a / Fraction(2) ** (e - 23)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return np.float32(sign * float(Fraction(n) * Fraction(2) ** (e - 23)))
