// Prefill attention over an already-quantized history: the queries of a chunk that has just been
// written attend to every cached token at a position not after their own ([NOVA] §3 "Long context":
// chunked prefill, each chunk quantized on write, so later chunks read a quantized history; [SAW]
// Fig. "Prefill Stage": save the chunk, read the cache back, attention).  The cache is read as it stands
// after the chunk's write: bf16 sink/tail tokens and INT2 per-channel groups, in the rotated frame for the
// groups (query rotated once, output un-rotated once by R_V^T) as in the decode.
//
// Contractions run on the matrix cores:
//  - INT2 groups on v_mfma_i32_16x16x64_i8 in 24-bit fixed point: per (query head, group) the key-side
//    operand a = rint(alpha S / max|alpha|), alpha = q~ s, and the weights u = rint(S p), p = 2^(logit -
//    group max), S = 8355584, each as three signed byte limbs (65536 hi + 256 mid + lo) against the 2-bit
//    codes (exact int32 sums per limb).  Outputs can be an order of magnitude above 1 (outlier channels),
//    so the operands keep more bits than the decode's 16;
//  - bf16 band tokens on v_mfma_f32_16x16x32_bf16 with the query and the weights split into bf16 hi + lo
//    (about 16 significant bits) against the exact bf16 values;
//  - the un-rotation on the same bf16 instruction with both operands split (hi hi + hi lo + lo hi).
// Operand layouts (16 x 16 tiles; lane l, q = l / 16): i8: A row l % 16, k = 16 q + byte index; B the
// same k, column l % 16; bf16: k = 8 q + element index; D: column l % 16, rows 4 q + 0..3.  The k index
// of a contraction may map to channels or tokens in any order used by both operands; the mappings below
// are chosen so that a lane's own results feed the next contraction without moving data between lanes.
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

// full scale of three signed byte limbs (the largest is 127 (65536 + 256 + 1) = 8355711), kept 127 below
// it: an fp32 product near 2^23 rounds by up to 0.5, and rint(max|alpha| * S / max|alpha|) must not pass it
constexpr float kS24 = 8355584.0f;
constexpr int kCols = 64;        // (query, head) columns per work-group, 16 per wave

__device__ inline i32x4 mfma_i8(i32x4 a, i32x4 b, i32x4 c) { return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0); }
__device__ inline f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// bf16 round to nearest even as bits (finite inputs), and the split x ~ hi + lo
__device__ inline uint32_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ inline void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const uint32_t h0 = bf16_bits(x0), h1 = bf16_bits(x1);
  const uint32_t l0 = bf16_bits(x0 - __uint_as_float(h0 << 16)), l1 = bf16_bits(x1 - __uint_as_float(h1 << 16));
  hi = h0 | (h1 << 16);
  lo = l0 | (l1 << 16);
}
// eight floats -> bf16x8 hi and lo operands
__device__ inline void split8(const float (&x)[8], u32x4& hi, u32x4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) split2(x[2 * k], x[2 * k + 1], h[k], l[k]);
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{l[0], l[1], l[2], l[3]};
}

// signed byte limbs of x = 65536 hi + 256 mid + lo (lo, mid, hi in [-128, 127]): lo = x mod 256,
// mid = ((x + 128) >> 8) mod 256, hi = (((x + 128) >> 8) + 128) >> 8; four values' limbs per word
__device__ inline uint32_t pack_bytes(int a0, int a1, int a2, int a3) {
  return __builtin_amdgcn_perm(__builtin_amdgcn_perm(a3, a2, 0x0c0c0400u), __builtin_amdgcn_perm(a1, a0, 0x0c0c0400u),
                               0x05040100u);
}
__device__ inline int limb_up(int x) { return (x + 128) >> 8; }
// limbs [lo, mid, hi] of four values as the dwords of three operands
__device__ inline void pack_limbs(int a0, int a1, int a2, int a3, uint32_t (&w)[3]) {
  w[0] = pack_bytes(a0, a1, a2, a3);
  const int b0 = limb_up(a0), b1 = limb_up(a1), b2 = limb_up(a2), b3 = limb_up(a3);
  w[1] = pack_bytes(b0, b1, b2, b3);
  w[2] = pack_bytes(limb_up(b0), limb_up(b1), limb_up(b2), limb_up(b3));
}
__device__ inline float limbs_value(const i32x4& h, const i32x4& m, const i32x4& l, int i) {
  return fmaf((float)h[i], 65536.0f, (float)(m[i] * 256 + l[i]));
}
// a 32-bit word of 2-bit codes as four int8 vectors: dword k' holds field k' of every byte
__device__ inline i32x4 unpack_codes(uint32_t w) {
  return i32x4{(int)(w & 0x03030303u), (int)((w >> 2) & 0x03030303u), (int)((w >> 4) & 0x03030303u),
               (int)((w >> 6) & 0x03030303u)};
}
// reductions over the 4 lanes of a column (lanes l, l ^ 16, l ^ 32, l ^ 48)
__device__ inline float col_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  return fmaxf(x, __shfl_xor(x, 32, 64));
}
__device__ inline float col_sum(float x) {
  x += __shfl_xor(x, 16, 64);
  return x + __shfl_xor(x, 32, 64);
}
__device__ inline float exp2_or_zero(float a, float m) { return a == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(a - m); }

__device__ inline uint32_t lds_addr_p(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ inline void dma16_p(uint32_t lds, const void* gaddr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(gaddr) : "memory");
}

struct GroupBuf {
  uint32_t k[2][512];   // key codes, page p token t at [p][8 t .. 8 t + 7]
  uint32_t v[2][512];   // value codes, page p channel c at [p][4 c .. 4 c + 3]
  uint16_t meta[512];   // K scales[128], K zeros[128] (even page), V scales[128], V zeros[128] (odd page)
};

template <int GQ>
__global__ __launch_bounds__(256) void prefill_int2_kernel(DecodeArgs a) {
  __shared__ GroupBuf gb[2];
  const Geo& g = a.g;
  const int b = blockIdx.z, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q0 = a.cu_q[b], nq = a.cu_q[b + 1] - q0;
  if ((int)blockIdx.x * kCols >= nq * GQ) return;
  const int T = a.seq_lens[b];
  // this lane's column: query qi of the chunk (position T - nq + qi), head hh of kv head h
  const int gc = blockIdx.x * kCols + wave * 16 + (lane & 15);
  const int qi = gc / GQ, hh = gc % GQ;
  const bool cvalid = qi < nq;
  const int qpos = cvalid ? T - nq + qi : -1;
  const long long row = ((long long)(q0 + (cvalid ? qi : 0)) * g.n_q + h * GQ + hh) * D;
  // the work-group's last visible position (uniform)
  const int last_q = min(nq - 1, ((int)blockIdx.x * kCols + kCols - 1) / GQ);
  const int pos_max = T - nq + last_q;

  // ---- band (sink + tail, bf16, original frame): blocks of 64 tokens
  const int ng = n_groups_of(T, g.S0, g.W);
  const int n_sink = T < g.S0 ? T : g.S0;
  const int tail0 = g.S0 + GROUP * ng;
  const int n_tail = T > tail0 ? T - tail0 : 0;
  const int nb = n_sink + n_tail;
  const uint16_t* band = a.band + ((long long)b * g.n_kv + h) * g.slots * 256;
  auto bpos = [&](int k) { return k < n_sink ? k : tail0 + (k - n_sink); };
  auto bslot = [&](int k) { return band_slot_of(bpos(k), g.S0, g.W); };
  float mb = -INFINITY, lb = 0.0f;
  f32x4 ob[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) ob[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (nb > 0) {
    // query (original frame, log2e / sqrt(d) folded in) for channels 32 ks + 8 q + e, as hi/lo operands
    u32x4 qh[4], ql[4];
    {
      const float* qb = a.qband + row;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = qb[32 * ks + 8 * q + e];
        split8(x, qh[ks], ql[ks]);
      }
    }
    for (int k0 = 0; k0 < nb; k0 += 64) {
      // S^T (64 tokens x 16 columns): token 16 mt + (l % 16) is the A row; channels 32 ks + 8 q + e
      float s[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int kk = min(k0 + 16 * mt + (lane & 15), nb - 1);  // rows past the band repeat a valid one
        const uint16_t* kr = band + (long long)bslot(kk) * 256;
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const u32x4 av = *reinterpret_cast<const u32x4*>(kr + 32 * ks + 8 * q);
          acc = mfma_bf16(av, qh[ks], acc);
          acc = mfma_bf16(av, ql[ks], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k = k0 + 16 * mt + 4 * q + i;
          s[mt][i] = (k < nb && bpos(k) <= qpos) ? acc[i] : -INFINITY;
        }
      }
      float bm = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) bm = fmaxf(bm, s[mt][i]);
      bm = col_max(bm);
      const float mnew = fmaxf(mb, bm);
      const float sc = exp2_or_zero(mb, mnew);
      float p[4][4], ps = 0.0f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[mt][i] = exp2_or_zero(s[mt][i], mnew);
          ps += p[mt][i];
        }
      lb = lb * sc + col_sum(ps);
      mb = mnew;
      // O_b^T (128 channels x 16 columns) += V^T P^T: k = 8 q + e maps to token 32 ks + 4 q + e (e < 4)
      // and 32 ks + 16 + 4 q + e - 4 (e >= 4), i.e. this lane's own weights of tiles 2 ks, 2 ks + 1
      u32x4 ph[2], pl[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const float x[8] = {p[2 * ks][0], p[2 * ks][1], p[2 * ks][2], p[2 * ks][3],
                            p[2 * ks + 1][0], p[2 * ks + 1][1], p[2 * ks + 1][2], p[2 * ks + 1][3]};
        split8(x, ph[ks], pl[ks]);
      }
      int slots[2][8];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int k = k0 + 32 * ks + (e < 4 ? 4 * q + e : 16 + 4 * q + e - 4);
          slots[ks][e] = bslot(min(k, nb - 1));
        }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const int c = 16 * mt + (lane & 15);
        f32x4 acc = ob[mt] * sc;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            w[e] = (uint32_t)band[(long long)slots[ks][2 * e] * 256 + 128 + c] |
                   ((uint32_t)band[(long long)slots[ks][2 * e + 1] * 256 + 128 + c] << 16);
          const u32x4 av = {w[0], w[1], w[2], w[3]};
          acc = mfma_bf16(av, ph[ks], acc);
          acc = mfma_bf16(av, pl[ks], acc);
        }
        ob[mt] = acc;
      }
    }
  }

  // ---- INT2 per-channel groups (rotated frame), double-buffered in LDS
  // rotated query of this column for channels 16 m + 4 j + k' of words m = q and m = 4 + q, in the order
  // e = 4 j + k' (the byte order of an unpacked code word)
  float qr[2][16];
  {
    const float* qp = a.qrot + row;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 16; ++e) qr[ks][e] = qp[16 * (4 * ks + q) + e];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 16; ++e) asm volatile("" ::"v"(qr[ks][e]));  // loads complete before the walk
  }
  int g_end = ng;
  {
    // groups whose first token is after every column's position are invisible
    const int gv = pos_max < g.S0 ? 0 : (pos_max - g.S0) / GROUP + 1;
    if (gv < g_end) g_end = gv;
    if (g_end > g.max_pages / 2) g_end = g.max_pages / 2;
  }
  float m = -INFINITY, l = 0.0f;
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const int32_t* pt = a.page_table + (long long)b * g.max_pages;
  const long long hoff = (long long)h * I2_HEAD_BYTES;
  // copies of one group: wave 0 K page 0, wave 1 K page 1, wave 2 V page 0, wave 3 V page 1 + metadata
  auto issue = [&](int gi, int buf) {
    const int pp = wave & 1;
    const uint8_t* pg = a.pages + pool_page(g, pt[2 * gi + pp]) * g.page_bytes + hoff;
    uint32_t* dst = wave < 2 ? gb[buf].k[pp] : gb[buf].v[pp];
    const uint8_t* src = pg + (wave < 2 ? I2_K_OFF : I2_V_OFF);
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16_p(lds_addr_p(dst + 256 * j), src + 1024 * j + 16 * lane);
    if (wave == 3) {
      const uint8_t* pm = a.pages + pool_page(g, pt[2 * gi + (lane >> 5)]) * g.page_bytes + hoff + I2_META_OFF;
      dma16_p(lds_addr_p(gb[buf].meta), pm + 16 * (lane & 31));
    }
  };
  if (g_end > 0) issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int gi = 0; gi < g_end; ++gi) {
    const int buf = gi & 1;
    if (gi + 1 < g_end) issue(gi + 1, buf ^ 1);
    const GroupBuf& B = gb[buf];
    const int gpos = g.S0 + GROUP * gi;
    // 1. key-side operand of this column: a = rint(alpha 32639 / max |alpha|), alpha = q~ s_k
    float al[2][16];
    float amx = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int c = 16 * (4 * ks + q) + 4 * (e >> 2) + (e & 3);  // e = 4 j + k' -> channel 16 m + 4 j + k'
        al[ks][e] = qr[ks][e] * bf16_to_f32(B.meta[c]);
        amx = fmaxf(amx, fabsf(al[ks][e]));
      }
    amx = col_max(amx);
    const float inv = amx > 0.0f ? kS24 / amx : 0.0f;
    int ai[2][16];
    float zs = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int c = 16 * (4 * ks + q) + 4 * (e >> 2) + (e & 3);
        ai[ks][e] = (int)rintf(al[ks][e] * inv);
        zs = fmaf((float)ai[ks][e], bf16_to_f32(B.meta[D + c]), zs);
      }
    zs = col_sum(zs);
    const float Acol = amx * (1.0f / kS24), AZ = Acol * zs;
    // B operands (limbs lo, mid, hi): dword k' of word m holds channels 16 m + 4 j + k' in byte j (e = 4 j + k')
    i32x4 bq[2][3];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int* x = ai[ks];
      uint32_t w[4][3];
#pragma unroll
      for (int k = 0; k < 4; ++k) pack_limbs(x[k], x[4 + k], x[8 + k], x[12 + k], w[k]);
#pragma unroll
      for (int lb = 0; lb < 3; ++lb) bq[ks][lb] = i32x4{(int)w[0][lb], (int)w[1][lb], (int)w[2][lb], (int)w[3][lb]};
    }
    // 2. logits S^T (128 tokens x 16 columns): token 16 mt + (l % 16) is the A row, its code word 4 ks + q
    float lg[8][4];
    float gm = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const int t = 16 * mt + (lane & 15);
      const uint32_t* kr = B.k[t >> 6] + 8 * (t & 63);
      i32x4 cl = {0, 0, 0, 0}, cm = {0, 0, 0, 0}, ch = {0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const i32x4 av = unpack_codes(kr[4 * ks + q]);
        cl = mfma_i8(av, bq[ks][0], cl);
        cm = mfma_i8(av, bq[ks][1], cm);
        ch = mfma_i8(av, bq[ks][2], ch);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 16 * mt + 4 * q + i;
        const float x = fmaf(Acol, limbs_value(ch, cm, cl, i), -AZ);
        lg[mt][i] = (gpos + tok <= qpos) ? x : -INFINITY;
        gm = fmaxf(gm, lg[mt][i]);
      }
    }
    gm = col_max(gm);
    // 3. weights u = floor(S p + 0.5), p = 2^(logit - group max), as byte limbs; the B operand of page
    // kp: k = 16 q + 4 r + j maps to token 64 kp + 16 j + 4 q + r, this lane's logit (tile 4 kp + j, r)
    int u[8][4];
    float us = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u[mt][i] = (int)fmaf(exp2_or_zero(lg[mt][i], gm), kS24, 0.5f);
        us += (float)u[mt][i];
      }
    const float Pf = col_sum(us);
    i32x4 uq[2][3];
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      uint32_t w[4][3];  // dword r: tokens 16 j + 4 q + r of page kp in byte j
#pragma unroll
      for (int r = 0; r < 4; ++r) pack_limbs(u[4 * kp][r], u[4 * kp + 1][r], u[4 * kp + 2][r], u[4 * kp + 3][r], w[r]);
#pragma unroll
      for (int lb = 0; lb < 3; ++lb) uq[kp][lb] = i32x4{(int)w[0][lb], (int)w[1][lb], (int)w[2][lb], (int)w[3][lb]};
    }
    // 4. values U^T (128 channels x 16 columns): channel 16 mt + (l % 16) is the A row; its code word q of
    // page kp holds tokens 16 j + 4 q + r (byte j, field r) = k index 16 q + 4 r + j
    const float mnew = fmaxf(m, gm);
    const float sc = exp2_or_zero(m, mnew);
    const float wg = exp2_or_zero(gm, mnew) * (1.0f / kS24);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const int c = 16 * mt + (lane & 15);
      i32x4 cl = {0, 0, 0, 0}, cm = {0, 0, 0, 0}, ch = {0, 0, 0, 0};
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        const i32x4 av = unpack_codes(B.v[kp][4 * c + q]);
        cl = mfma_i8(av, uq[kp][0], cl);
        cm = mfma_i8(av, uq[kp][1], cm);
        ch = mfma_i8(av, uq[kp][2], ch);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int cc = 16 * mt + 4 * q + i;
        const float sv = bf16_to_f32(B.meta[2 * D + cc]), zv = bf16_to_f32(B.meta[3 * D + cc]);
        const float U = limbs_value(ch, cm, cl, i);
        o[mt][i] = fmaf(o[mt][i], sc, (wg * sv) * fmaf(-zv, Pf, U));
      }
    }
    l = fmaf(l, sc, wg * Pf);
    m = mnew;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's copies of the next group
    __syncthreads();                                    // everyone's copies landed, this group released
  }

  // ---- un-rotate (O^T <- R_V O^T) unless values were never rotated; the k index of step ks maps to
  // channel 32 ks + 4 q + e (e < 4) and 32 ks + 16 + 4 q + e - 4 (e >= 4): this lane's tiles 2 ks, 2 ks + 1
  // (uniform branch: the matrix instructions read every lane's operands; a column that saw nothing holds
  // zeros and passes through unchanged)
  f32x4 of[8];
  if (g.key_only) {
#pragma unroll
    for (int i = 0; i < 8; ++i) of[i] = o[i];
  } else {
    u32x4 oh[4], ol[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const float x[8] = {o[2 * ks][0], o[2 * ks][1], o[2 * ks][2], o[2 * ks][3],
                          o[2 * ks + 1][0], o[2 * ks + 1][1], o[2 * ks + 1][2], o[2 * ks + 1][3]};
      split8(x, oh[ks], ol[ks]);
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const float* rv = a.rot_v + (16 * mt + (lane & 15)) * D;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const float4 r0 = *reinterpret_cast<const float4*>(rv + 32 * ks + 4 * q);
        const float4 r1 = *reinterpret_cast<const float4*>(rv + 32 * ks + 16 + 4 * q);
        const float x[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
        u32x4 rh, rl;
        split8(x, rh, rl);
        acc = mfma_bf16(rh, oh[ks], acc);
        acc = mfma_bf16(rh, ol[ks], acc);
        acc = mfma_bf16(rl, oh[ks], acc);
      }
      of[mt] = acc;
    }
  }
  // ---- combine with the band and normalize; channels 16 mt + 4 q + i of this column
  if (!cvalid) return;
  const float M = fmaxf(m, mb);
  const float si = exp2_or_zero(m, M), sb = exp2_or_zero(mb, M);
  const float den = l * si + lb * sb;
  const float rden = den > 0.0f ? 1.0f / den : 0.0f;
  float* out = a.out + row;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    const f32x4 r = (of[mt] * si + ob[mt] * sb) * rden;
    *reinterpret_cast<float4*>(out + 16 * mt + 4 * q) = make_float4(r[0], r[1], r[2], r[3]);
  }
}

}  // namespace

hipError_t launch_prefill(const DecodeArgs& a, int max_q, hipStream_t s) {
  const Geo& g = a.g;
  if (max_q <= 0) return hipSuccess;
  const dim3 grid((max_q * g.gq + kCols - 1) / kCols, g.n_kv, g.batch);
  switch (g.gq) {
    case 1: hipLaunchKernelGGL(prefill_int2_kernel<1>, grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(prefill_int2_kernel<2>, grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL(prefill_int2_kernel<4>, grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL(prefill_int2_kernel<8>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
