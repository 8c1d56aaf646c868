// Prefill attention over an already-quantized history: the queries of a chunk that has just been
// written attend to every cached token at a position not after their own ([NOVA] §3 "Long context":
// chunked prefill, each chunk quantized on write, so later chunks read a quantized history; [SAW]
// Fig. "Prefill Stage": save the chunk, read the cache back, attention).  The cache is read as it stands
// after the chunk's write, for every scheme: bf16 sink/tail tokens and 128-token groups (INT2 per channel
// or per token, INT4 per channel), or INT4 per-token pages read in pairs of 128 tokens; quantized tokens in
// the rotated frame (query rotated once, output un-rotated once) as in the decode.
//
// Contractions run on the matrix cores:
//  - quantized tokens on v_mfma_i32_16x16x64_i8 in fixed point, three signed byte limbs (65536 hi + 256 mid +
//    lo, split by one FMA with a magic addend) against the 2- or 4-bit codes, full scale S = 4,000,000 (2-bit
//    codes) or 1,000,000 (4-bit codes), so that the limbs' int32 sums recombine exactly in int32.
//    Per channel: per (query head, group) the key-side operand a = rint(alpha S / max|alpha|), alpha = q~ s,
//    and the weights u = rint(S p), p = 2^(logit - group max).  Per token: the key-side operand is the
//    rotated query itself (a = rint(q~ S / max|q~|), once per query), logit_t = A s_t (D_t - z_t sum_c a_c),
//    and the weights u_t = rint(S p_t s'_t / S'), S' the unit's largest p_t s'_t, the value sum adding
//    (S' / S) (U_c - sum_t u_t z'_t).  Outputs can be an order of magnitude above 1 (outlier channels), so
//    the operands keep more bits than 16;
//  - bf16 band tokens on v_mfma_f32_16x16x32_bf16 with the query and the weights split into bf16 hi + lo
//    (about 16 significant bits) against the exact bf16 values;
//  - the dense un-rotation on the same bf16 instruction with both operands split (hi hi + hi lo + lo hi);
//    the randomized Hadamard's un-rotation is a fp32 Walsh-Hadamard transform in registers.
// Operand layouts (16 x 16 tiles; lane l, q = l / 16): i8: A row l % 16, k = 16 q + byte index; B the
// same k, column l % 16; bf16: k = 8 q + element index; D: column l % 16, rows 4 q + 0..3.  The k index
// of a contraction may map to channels or tokens in any order used by both operands; the mappings below
// are chosen so that a lane's own results feed the next contraction without moving data between lanes.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

constexpr int kCols = 64;        // (query, head) columns per work-group, 16 per wave

__device__ inline i32x4 mfma_i8(i32x4 a, i32x4 b, i32x4 c) { return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0); }

// the value lo + 256 mid + 65536 hi of element i of three limb sums (exact in int32 at the full scales used)
__device__ inline float limbs_value(const i32x4& h, const i32x4& m, const i32x4& l, int i) {
  return (float)(int)(((((uint32_t)h[i] << 8) + (uint32_t)m[i]) << 8) + (uint32_t)l[i]);
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

// What the prefill kernel reads of a scheme's pages: code bits, the words of a key row (one token, 128
// channels) and of a value row (one channel, 64 tokens of a page), the offsets in a kv head's block of a
// page, and whether the scales and zeros are per channel of a group or per token.
template <int SCHEME>
struct PrefillScheme {
  static constexpr bool GROUPED = SCHEME != KVQ_INT4_TOKEN;  // 128-token groups aligned at S0, bf16 band
  static constexpr bool TOK = SCHEME == KVQ_INT2_TOKEN || SCHEME == KVQ_INT4_TOKEN;
  static constexpr int BITS = (SCHEME == KVQ_INT2_CHANNEL || SCHEME == KVQ_INT2_TOKEN) ? 2 : 4;
  static constexpr int HEAD = BITS == 2 ? I2_HEAD_BYTES : I4_HEAD_BYTES;
  static constexpr int VOFF = BITS == 2 ? I2_V_OFF : I4_V_OFF;
  static constexpr int MOFF = BITS == 2 ? I2_META_OFF : I4_KMETA_OFF;  // 512 B per page in every layout
  static constexpr int KROW = BITS == 2 ? 8 : 16;  // words per key row
  static constexpr int VROW = BITS == 2 ? 4 : 8;   // words per value row and page
};

// Key operand of a token row for the channels of 16-channel block m (k = 16 q + 4 k' + j: dword k', byte j):
//  - 2-bit codes (channel c in byte c / 4, field c % 4): word m, dword k' = field k' -> channel 16 m + 4 j + k'
//    (codes_i8_pair unpacks the two k steps' words m = q and 4 + q together);
//  - per-channel 4-bit (word 2 m + e holds channels 16 m + 2 k + e in nibble k): low nibbles of words 2 m,
//    2 m + 1, then their high nibbles -> channel 16 m + 4 j + k';
//  - per-token 4-bit (channel c in byte c / 2, even c low): words 2 m, 2 m + 1, low then high nibbles of
//    each -> channel 16 m + 8 (k' / 2) + 2 j + k' % 2.
template <int SCHEME>
__device__ inline int key_channel(int m, int e) {  // e = 4 j + k'
  if constexpr (SCHEME == KVQ_INT4_TOKEN) return 16 * m + 8 * ((e & 3) >> 1) + 2 * (e >> 2) + (e & 1);
  return 16 * m + e;
}
__device__ inline i32x4 nib_lo_lo_hi_hi(uint32_t w0, uint32_t w1) {
  return i32x4{(int)(w0 & 0x0F0F0F0Fu), (int)(w1 & 0x0F0F0F0Fu), (int)((w0 >> 4) & 0x0F0F0F0Fu),
               (int)((w1 >> 4) & 0x0F0F0F0Fu)};
}
__device__ inline i32x4 nib_lo_hi_lo_hi(uint32_t w0, uint32_t w1) {
  return i32x4{(int)(w0 & 0x0F0F0F0Fu), (int)((w0 >> 4) & 0x0F0F0F0Fu), (int)(w1 & 0x0F0F0F0Fu),
               (int)((w1 >> 4) & 0x0F0F0F0Fu)};
}
template <int SCHEME>
__device__ inline i32x4 key_codes(const uint32_t* row, int m) {  // 4-bit codes
  static_assert(PrefillScheme<SCHEME>::BITS == 4, "2-bit words go through codes_i8_pair");
  if constexpr (SCHEME == KVQ_INT4_CHANNEL) return nib_lo_lo_hi_hi(row[2 * m], row[2 * m + 1]);
  else return nib_lo_hi_lo_hi(row[2 * m], row[2 * m + 1]);
}
// Value operand of a channel row of one page, lane q (k = 16 q + 4 d + b: dword d, byte b), tokens (of the
// page) 16 J + 4 q + R:
//  - 2-bit codes (token 16 j + 4 g + r in byte 4 g + j, field r): word q, dword d = field d -> J = b, R = d
//    (codes_i8_pair unpacks the two pages' words together);
//  - per-channel 4-bit (word 2 g + n holds tokens 16 j + 4 g + 2 h + n in nibble 2 j + h): low nibbles of
//    words 2 q, 2 q + 1, then their high nibbles -> J = b, R = d;
//  - per-token 4-bit (token 16 j + 4 g + r in byte 8 g + 2 j + r / 2, even r low): words 2 q, 2 q + 1, low
//    then high nibbles of each -> J = 2 (d / 2) + b / 2, R = 2 (b % 2) + d % 2.
template <int SCHEME>
__device__ inline i32x4 value_codes(const uint32_t* row, int q) {  // 4-bit codes
  static_assert(PrefillScheme<SCHEME>::BITS == 4, "2-bit words go through codes_i8_pair");
  if constexpr (SCHEME == KVQ_INT4_CHANNEL) return nib_lo_lo_hi_hi(row[2 * q], row[2 * q + 1]);
  else return nib_lo_hi_lo_hi(row[2 * q], row[2 * q + 1]);
}
template <int SCHEME>
__device__ inline void value_tok(int d, int b, int& J, int& R) {
  if constexpr (SCHEME == KVQ_INT4_TOKEN) {
    J = 2 * (d >> 1) + (b >> 1);
    R = 2 * (b & 1) + (d & 1);
  } else {
    J = b;
    R = d;
  }
}

// The page pair of one 128-token unit: grouped schemes' group (two pages), or two consecutive INT4 pages
template <int BITS>
struct GroupBuf {
  uint32_t k[2][64 * (BITS == 2 ? 8 : 16)];   // page p, token t at [p][KROW t ..]
  uint32_t v[2][128 * (BITS == 2 ? 4 : 8)];   // page p, channel c at [p][VROW c ..]
  uint16_t meta[512];                         // the pages' 512-byte metadata blocks, page 0 then page 1
};

// The limbs of 16 magic-rounded values ef[e] (e = 4 j + k', each fmaf(x, scale, kRound3), or kRoundU for
// non-negative values, U) as the three i8 operands lo, mid, hi: dword k' holds the limbs of ef[k'],
// ef[4 + k'], ef[8 + k'], ef[12 + k'] in bytes 0..3
template <bool U = false>
__device__ inline void limb_operands(const float (&ef)[16], i32x4 (&op)[3]) {
  uint32_t w[4][3];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if constexpr (U) limbs3u(ef[k], ef[4 + k], ef[8 + k], ef[12 + k], w[k][0], w[k][1], w[k][2]);
    else limbs3(ef[k], ef[4 + k], ef[8 + k], ef[12 + k], w[k][0], w[k][1], w[k][2]);
  }
#pragma unroll
  for (int lb = 0; lb < 3; ++lb) op[lb] = i32x4{(int)w[0][lb], (int)w[1][lb], (int)w[2][lb], (int)w[3][lb]};
}

template <int GQ, int SCHEME>
__global__ __launch_bounds__(256) void prefill_kernel(DecodeArgs a) {
  using SC = PrefillScheme<SCHEME>;
  constexpr float S = SC::BITS == 2 ? 4000000.0f : 1000000.0f;  // full scale of the fixed-point operands
  __shared__ GroupBuf<SC::BITS> gb[2];
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
  // every column of the work-group holds a query, the first at position pos_min (uniform)
  const bool all_cols_valid = ((int)blockIdx.x + 1) * kCols <= nq * GQ;
  const int pos_min = T - nq + ((int)blockIdx.x * kCols) / GQ;

  // ---- band (sink + tail, bf16, original frame): blocks of 64 tokens
  const int ng = SC::GROUPED ? n_groups_of(T, g.S0, g.W) : 0;
  float mb = -INFINITY, lb = 0.0f;
  f32x4 ob[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) ob[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (SC::GROUPED) {
    const int n_sink = T < g.S0 ? T : g.S0;
    const int tail0 = g.S0 + GROUP * ng;
    const int n_tail = T > tail0 ? T - tail0 : 0;
    const int nb = n_sink + n_tail;
    const uint16_t* band = a.band + ((long long)b * g.n_kv + h) * g.slots * 256;
    auto bpos = [&](int k) { return k < n_sink ? k : tail0 + (k - n_sink); };
    auto bslot = [&](int k) { return band_slot_of(bpos(k), g.S0, g.W); };
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
  }

  // ---- quantized 128-token units (rotated frame), double-buffered in LDS
  // rotated query of this column for the channels of blocks m = q and m = 4 + q, in the order e = 4 j + k'
  // (the byte order of an unpacked code word)
  float qr[2][16];
  {
    const float* qp = a.qrot + row;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 16; ++e) qr[ks][e] = qp[key_channel<SCHEME>(4 * ks + q, e)];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 16; ++e) asm volatile("" ::"v"(qr[ks][e]));  // loads complete before the walk
  }
  // units (groups, or INT4 page pairs) whose first token is after every column's position are invisible
  const int u0 = SC::GROUPED ? g.S0 : 0;  // position of unit 0's first token
  const int npages = (T + PAGE - 1) / PAGE;
  int g_end = SC::GROUPED ? ng : (npages + 1) / 2;
  {
    const int gv = pos_max < u0 ? 0 : (pos_max - u0) / GROUP + 1;
    if (gv < g_end) g_end = gv;
    const int row_units = SC::GROUPED ? g.max_pages / 2 : (g.max_pages + 1) / 2;  // never past the table row
    if (g_end > row_units) g_end = row_units;
  }
  // per token: the key-side operand is the rotated query, once (A = max|q~| / S, FS = sum_c a_c)
  i32x4 bq_tok[2][3];
  float A_tok = 0.0f, FS_tok = 0.0f;
  if constexpr (SC::TOK) {
    float amx = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 16; ++e) amx = fmaxf(amx, fabsf(qr[ks][e]));
    amx = col_max(amx);
    const float inv = amx > 0x1p-100f ? S / amx : 0.0f;
    float fs = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float ef[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        ef[e] = fmaf(qr[ks][e], inv, kRound3);
        fs += ef[e] - kRound3;  // the integer a exactly
      }
      limb_operands(ef, bq_tok[ks]);
    }
    FS_tok = col_sum(fs);
    A_tok = amx * (1.0f / S);
  }
  float m = -INFINITY, l = 0.0f;
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const int32_t* pt = a.page_table + (long long)b * g.max_pages;
  const long long hoff = (long long)h * SC::HEAD;
  // the two pages of unit gi (an INT4 sequence with an odd page count reads its last page twice, the
  // second copy past the length and never weighted)
  auto page_of = [&](int gi, int pp) {
    int idx = 2 * gi + pp;
    if (!SC::GROUPED && idx >= npages) idx = npages - 1;
    if (idx >= g.max_pages) idx = g.max_pages - 1;
    return a.pages + pool_page(g, pt[idx]) * g.page_bytes + hoff;
  };
  // copies of one unit: wave 0 K page 0, wave 1 K page 1, wave 2 V page 0, wave 3 V page 1 + metadata
  constexpr int NCP = SC::BITS == 2 ? 2 : 4;  // 1 KB copies per page and side
  auto issue = [&](int gi, int buf) {
    const int pp = wave & 1;
    const uint8_t* pg = page_of(gi, pp);
    uint32_t* dst = wave < 2 ? gb[buf].k[pp] : gb[buf].v[pp];
    const uint8_t* src = pg + (wave < 2 ? 0 : SC::VOFF);
#pragma unroll
    for (int j = 0; j < NCP; ++j) dma16_p(lds_addr_p(dst + 256 * j), src + 1024 * j + 16 * lane);
    if (wave == 3) dma16_p(lds_addr_p(gb[buf].meta), page_of(gi, lane >> 5) + SC::MOFF + 16 * (lane & 31));
  };
  if (g_end > 0) issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int gi = 0; gi < g_end; ++gi) {
    const int buf = gi & 1;
    if (gi + 1 < g_end) issue(gi + 1, buf ^ 1);
    const GroupBuf<SC::BITS>& B = gb[buf];
    const int gpos = u0 + GROUP * gi;
    // 1. key-side operand: per channel a = rint(alpha S / max|alpha|), alpha = q~ s_k of this group; per
    //    token the query's, built once
    i32x4 bq[2][3];
    float Acol, AZ = 0.0f;
    if constexpr (SC::TOK) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int lb3 = 0; lb3 < 3; ++lb3) bq[ks][lb3] = bq_tok[ks][lb3];
      Acol = A_tok;
    } else {
      float al[2][16];
      float amx = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int c = key_channel<SCHEME>(4 * ks + q, e);
          al[ks][e] = qr[ks][e] * bf16_to_f32(B.meta[c]);
          amx = fmaxf(amx, fabsf(al[ks][e]));
        }
      amx = col_max(amx);
      const float inv = amx > 0x1p-100f ? S / amx : 0.0f;
      float zs = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float ef[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int c = key_channel<SCHEME>(4 * ks + q, e);
          ef[e] = fmaf(al[ks][e], inv, kRound3);
          zs = fmaf(al[ks][e], bf16_to_f32(B.meta[D + c]), zs);  // A a equals alpha to 2^-23 of max|alpha|
        }
        limb_operands(ef, bq[ks]);
      }
      zs = col_sum(zs);
      Acol = amx * (1.0f / S);
      AZ = zs;
    }
    // this lane's tokens: 16 mt + 4 q + i of the unit (page mt / 4, token 16 (mt % 4) + 4 q + i of it)
    // the scales (s) and zeros (z) of tokens 16 mt + 4 q + 0..3, K (side 0) or V (side 1), by one LDS read:
    // per-token INT2 keeps a page's 64 K scales, K zeros, V scales, V zeros in runs; INT4 keeps (s, z) pairs
    auto tok_meta4 = [&](int mt, int side, float (&sv)[4], float (&zv)[4]) {
      const int pg = mt >> 2, t0 = 16 * (mt & 3) + 4 * q;
      if constexpr (SCHEME == KVQ_INT2_TOKEN) {
        const uint2 ws = *reinterpret_cast<const uint2*>(&B.meta[256 * pg + 128 * side + t0]);
        const uint2 wz = *reinterpret_cast<const uint2*>(&B.meta[256 * pg + 128 * side + 64 + t0]);
        sv[0] = __uint_as_float(ws.x << 16), sv[1] = __uint_as_float(ws.x & 0xffff0000u);
        sv[2] = __uint_as_float(ws.y << 16), sv[3] = __uint_as_float(ws.y & 0xffff0000u);
        zv[0] = __uint_as_float(wz.x << 16), zv[1] = __uint_as_float(wz.x & 0xffff0000u);
        zv[2] = __uint_as_float(wz.y << 16), zv[3] = __uint_as_float(wz.y & 0xffff0000u);
      } else {
        const uint4 w = *reinterpret_cast<const uint4*>(&B.meta[256 * pg + 128 * side + 2 * t0]);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sv[i] = __uint_as_float(ww[i] << 16);
          zv[i] = __uint_as_float(ww[i] & 0xffff0000u);
        }
      }
    };
    // 2. logits S^T (128 tokens x 16 columns): token 16 mt + (l % 16) is the A row
    // 3. weights as byte limbs.  Per channel u = floor(S p + 0.5), p = 2^(logit - group max); per token
    //    u_t = floor(S p_t s'_t / S' + 0.5), S' = max_t p_t s'_t of the column, with P = sum_t p_t and
    //    Z = sum_t u_t z'_t
    // FULL: every token of the unit is visible to every column of the work-group (a uniform condition), so
    // no logit is masked and no weight needs the masked case's checks; the results are the same either way.
    float gm = -INFINITY;
    float u[8][4];  // magic-rounded weights
    float Pf, Sg = 0.0f, Zt = 0.0f;
    auto logits_weights = [&](auto full_tag) {
      constexpr bool FULL = decltype(full_tag)::value;
      float lg[8][4];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const int t = 16 * mt + (lane & 15);
        const uint32_t* kr = B.k[t >> 6] + SC::KROW * (t & 63);
        i32x4 cl = {0, 0, 0, 0}, cm = {0, 0, 0, 0}, ch = {0, 0, 0, 0};
        i32x4 av[2];
        if constexpr (SC::BITS == 2) {
          codes_i8_pair(kr[q], kr[4 + q], av[0], av[1]);
        } else {
          av[0] = key_codes<SCHEME>(kr, q);
          av[1] = key_codes<SCHEME>(kr, 4 + q);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          cl = mfma_i8(av[ks], bq[ks][0], cl);
          cm = mfma_i8(av[ks], bq[ks][1], cm);
          ch = mfma_i8(av[ks], bq[ks][2], ch);
        }
        float ks4[4], kz4[4];
        if constexpr (SC::TOK) tok_meta4(mt, 0, ks4, kz4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = 16 * mt + 4 * q + i;
          float x;
          if constexpr (SC::TOK) x = (Acol * ks4[i]) * fmaf(-kz4[i], FS_tok, limbs_value(ch, cm, cl, i));
          else x = fmaf(Acol, limbs_value(ch, cm, cl, i), -AZ);
          lg[mt][i] = (FULL || gpos + tok <= qpos) ? x : -INFINITY;
          gm = fmaxf(gm, lg[mt][i]);
        }
      }
      gm = col_max(gm);
      auto weight = [&](float x) { return FULL ? __builtin_amdgcn_exp2f(x - gm) : exp2_or_zero(x, gm); };
      if constexpr (SC::TOK) {
        float pw[8][4], vz[8][4], wmx = 0.0f, ps = 0.0f;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
          float vs4[4];
          tok_meta4(mt, 1, vs4, vz[mt]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = weight(lg[mt][i]);
            ps += p;
            // tokens past the length (their metadata unwritten) take no weight
            pw[mt][i] = (!FULL && lg[mt][i] == -INFINITY) ? 0.0f : p * vs4[i];
            wmx = fmaxf(wmx, pw[mt][i]);
          }
        }
        Sg = col_max(wmx);
        Pf = col_sum(ps);
        // below 2^-100 the unit's value terms are beyond fp32's reach next to the others: weights 0
        const float r = Sg > 0x1p-100f ? S / Sg : 0.0f;
        float zs = 0.0f;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            u[mt][i] = fmaf(pw[mt][i], r, kRoundU);
            if (FULL || lg[mt][i] != -INFINITY) zs = fmaf(u[mt][i] - kRoundU, vz[mt][i], zs);
          }
        Zt = col_sum(zs);
      } else {
        float us = 0.0f;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            u[mt][i] = fmaf(weight(lg[mt][i]), S, kRoundU);
            us += u[mt][i] - kRoundU;
          }
        Pf = col_sum(us);
      }
    };
    if (all_cols_valid && gpos + GROUP - 1 <= pos_min) {
      logits_weights(std::true_type{});
    } else {
      logits_weights(std::false_type{});
    }
    // B operand of page kp: dword d, byte bb holds the weight of token 16 J + 4 q + R of the page, i.e. this
    // lane's logit (tile 4 kp + J, i = R)
    i32x4 uq[2][3];
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      float x[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {  // e = 4 bb + d (the order limb_operands packs)
        int J, R;
        value_tok<SCHEME>(e & 3, e >> 2, J, R);
        x[e] = u[4 * kp + J][R];
      }
      limb_operands<true>(x, uq[kp]);
    }
    // 4. values U^T (128 channels x 16 columns): channel 16 mt + (l % 16) is the A row
    const float mnew = fmaxf(m, gm);
    const float sc = exp2_or_zero(m, mnew);
    const float eg = exp2_or_zero(gm, mnew);
    const float wg = SC::TOK ? eg * Sg * (1.0f / S) : eg * (1.0f / S);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const int c = 16 * mt + (lane & 15);
      i32x4 cl = {0, 0, 0, 0}, cm = {0, 0, 0, 0}, ch = {0, 0, 0, 0};
      i32x4 av[2];
      if constexpr (SC::BITS == 2) {
        codes_i8_pair(B.v[0][SC::VROW * c + q], B.v[1][SC::VROW * c + q], av[0], av[1]);
      } else {
        av[0] = value_codes<SCHEME>(B.v[0] + SC::VROW * c, q);
        av[1] = value_codes<SCHEME>(B.v[1] + SC::VROW * c, q);
      }
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        cl = mfma_i8(av[kp], uq[kp][0], cl);
        cm = mfma_i8(av[kp], uq[kp][1], cm);
        ch = mfma_i8(av[kp], uq[kp][2], ch);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float U = limbs_value(ch, cm, cl, i);
        if constexpr (SC::TOK) {
          o[mt][i] = fmaf(o[mt][i], sc, wg * (U - Zt));
        } else {
          const int cc = 16 * mt + 4 * q + i;
          const float sv = bf16_to_f32(B.meta[2 * D + cc]), zv = bf16_to_f32(B.meta[3 * D + cc]);
          o[mt][i] = fmaf(o[mt][i], sc, (wg * sv) * fmaf(-zv, Pf, U));
        }
      }
    }
    l = SC::TOK ? fmaf(l, sc, eg * Pf) : fmaf(l, sc, wg * Pf);
    m = mnew;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's copies of the next unit
    __syncthreads();                                    // everyone's copies landed, this unit released
  }

  // ---- un-rotate unless values were never rotated (uniform branches: the matrix instructions read every
  // lane's operands; a column that saw nothing holds zeros and passes through unchanged)
  f32x4 of[8];
  if (g.key_only) {
#pragma unroll
    for (int i = 0; i < 8; ++i) of[i] = o[i];
  } else if (g.rotation == KVQ_ROT_DENSE) {
    // O^T <- R_V O^T; the k index of step ks maps to channel 32 ks + 4 q + e (e < 4) and 32 ks + 16 + 4 q +
    // e - 4 (e >= 4): this lane's tiles 2 ks, 2 ks + 1
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
  } else {
    // randomized Hadamard ([SAW] eq. 1): o H_blk, then the signs and 1/sqrt(h).  Channel 16 mt + 4 q + i:
    // butterflies over bits 0-1 within a lane's quad, bits 2-3 across lanes q (16 and 32 apart), bits 4-6
    // across its tiles
    float x[8][4];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[mt][i] = o[mt][i];
#pragma unroll
    for (int st = 0; st < 7; ++st) {  // stage hb = 2^st of the blocks' transform (uniform)
      const int hb = 1 << st;
      if (hb >= g.hblock) break;
      if (hb < 4) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
          float y[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) y[i] = (i & hb) ? x[mt][i ^ hb] - x[mt][i] : x[mt][i] + x[mt][i ^ hb];
#pragma unroll
          for (int i = 0; i < 4; ++i) x[mt][i] = y[i];
        }
      } else if (hb < 16) {
        const int lx = 16 * (hb >> 2);  // 16 or 32
        const bool upper = (q & (hb >> 2)) != 0;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float other = __shfl_xor(x[mt][i], lx, 64);
            x[mt][i] = upper ? other - x[mt][i] : x[mt][i] + other;
          }
      } else {
        const int tb = hb >> 4;  // 1, 2 or 4
        float y[8][4];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) y[mt][i] = (mt & tb) ? x[mt ^ tb][i] - x[mt][i] : x[mt][i] + x[mt ^ tb][i];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[mt][i] = y[mt][i];
      }
    }
    const float hs = (float)g.hscale;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const float4 sg = *reinterpret_cast<const float4*>(a.rot_v + 16 * mt + 4 * q);
      of[mt] = f32x4{x[mt][0] * sg.x * hs, x[mt][1] * sg.y * hs, x[mt][2] * sg.z * hs, x[mt][3] * sg.w * hs};
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

template <int SCHEME>
hipError_t launch_prefill_scheme(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  switch (a.g.gq) {
    case 1: hipLaunchKernelGGL((prefill_kernel<1, SCHEME>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<2, SCHEME>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<4, SCHEME>), grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((prefill_kernel<8, SCHEME>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const DecodeArgs& a, int max_q, hipStream_t s) {
  const Geo& g = a.g;
  if (max_q <= 0) return hipSuccess;
  const dim3 grid((max_q * g.gq + kCols - 1) / kCols, g.n_kv, g.batch);
  switch (g.scheme) {
    case KVQ_INT2_CHANNEL: return launch_prefill_scheme<KVQ_INT2_CHANNEL>(a, grid, s);
    case KVQ_INT2_TOKEN: return launch_prefill_scheme<KVQ_INT2_TOKEN>(a, grid, s);
    case KVQ_INT4_CHANNEL: return launch_prefill_scheme<KVQ_INT4_CHANNEL>(a, grid, s);
    case KVQ_INT4_TOKEN: return launch_prefill_scheme<KVQ_INT4_TOKEN>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
