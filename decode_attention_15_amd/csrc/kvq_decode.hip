// Read path: one decode attention step over the rotated, quantized, paged cache.
//
// [OSCAR] summary page §3.4.4 step 4 (dequantize in the rotated frame, inverse-rotate) and §3.4.5
// (three cache segments, split partials merged with softmax rescaling); [SAW] §4.1 and App. A.4
// eq. (13)-(14) (query rotated once, logits against dequantized rotated keys, output un-rotated);
// [NOVA] App. B.5 (query folded once per step, two-stage split-KV decode).
//
// Logits are kept in log2 units: the query is pre-scaled by log2(e)/sqrt(128) so exp2 gives e^x.
// For a per-channel INT2 group with key scales s_c and zeros z_c:
//   logit_t = sum_c q~_c s_c (code_tc - z_c) = sum_c alpha_c code_tc - beta,
//   alpha_c = q~_c s_c, beta = sum_c alpha_c z_c,
// and with value scales/zeros the group's output contribution is
//   o~_c += s_c (sum_t p_t code_tc - z_c sum_t p_t),
// so per element the kernel only converts a 2-bit code and multiplies.
#include <hip/hip_runtime.h>

#include <hip/hip_ext.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr float kInvSqrt128 = 0.08838834764831845f;
constexpr int kThreads = 256;

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// LDS written by a wave and then read back by other lanes of the same wave.
__device__ inline void wave_lds_sync() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

__device__ inline float exp2_safe_diff(float a, float b) {
  // 2^(a-b) with 2^(-inf - -inf) taken as 0
  return (a == -INFINITY) ? 0.0f : exp2f(a - b);
}

// ---------------------------------------------------------------------------------------------
// Split-K decode, vector ALU.  Work-group (unit, kv head, seq): unit 0 = bf16 band (sink + tail),
// unit u >= 1 = quantized chunk u-1.  Each of the 4 waves walks its own groups/pages with an
// online softmax; the waves are merged in LDS and one partial (m, l, o[128]) per q head written.
// ---------------------------------------------------------------------------------------------
// Per-wave LDS of the matrix-core units: the key and the value codes of a group or page pair, the metadata of
// two of them (double-buffered, 1 KB each; at GQ 8 with 2-bit codes one buffer, whose lanes take the key-side
// words to registers and the value scales and zeros to a 512-byte side buffer before the next group's copy
// lands, so that three work-groups fit a CU), and one operand plane with rows (head, limb)
// of 128 bytes in k order (stride 144: consecutive rows start in different banks) and a last row that stays
// zero for the matrix rows no head fills.  The plane holds the key-side operand while the key products read
// it and the softmax weights while the value products read them.
template <int GQ, int KU = 256>
struct MfmaWave {
  static constexpr int ROWS = 3 * GQ;
  static constexpr int RSTRIDE = 144;
  static constexpr int MB = (GQ == 8 && KU == 256) ? 1 : 2;  // metadata buffers
  uint4 kst[KU];  // key codes: 4 KB (2-bit codes of a group) or 8 KB (4-bit codes of a group or page pair)
  uint4 vst[KU];  // value codes, the same size
  uint4 mst[MB][64];
  uint8_t plane[(ROWS + 1) * RSTRIDE];
  uint4 vsz[MB == 1 ? 32 : 0];  // one metadata buffer: the group's value scales and zeros
};
template <int GQ, bool MF, int KU>
struct MfmaLds {};
template <int GQ, int KU>
struct MfmaLds<GQ, true, KU> {
  MfmaWave<GQ, KU> w[4];
};

// STG: code staging per wave and group in units of 4 KB (2 for 4-bit per-channel codes); MF: the
// matrix-core unit's buffers
template <int GQ, int STG = 1, bool MF = false>
struct DecodeLds {
  union {
    MfmaLds<GQ, MF, 256 * STG> mf;
    struct {                     // band unit, fp32 INT2 and INT4 paths
      float qband[GQ][D];
      float alpha[4][GQ][D];     // per wave: alpha (INT2) / rotated query (INT4)
      float p[4][GQ][D];         // per wave: softmax numerators of the current group/page
    } f;
    float co[4][GQ][D];          // the waves' outputs, written once every wave has finished its walk
  };
  float cm[4][GQ];
  float cl[4][GQ];
};

// The four waves' partials (m, l, o in L.co/cm/cl) combined into the work-group's partial of `unit`.
template <int GQ, typename Lds>
__device__ void combine_waves(Lds& L, const DecodeArgs& a, int b, int h, int unit) {
  __syncthreads();
  const Geo& g = a.g;
  for (int e = threadIdx.x; e < GQ * D; e += kThreads) {
    const int hh = e / D, c = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, L.cm[w][hh]);
    float acc = 0.0f, lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sc = exp2_safe_diff(L.cm[w][hh], M);
      acc += sc * L.co[w][hh][c];
      lsum += sc * L.cl[w][hh];
    }
    float* part = a.partials + (((long long)b * g.n_q + h * GQ + hh) * g.n_units + unit) * PART_STRIDE;
    part[2 + c] = acc;
    if (c == 0) {
      part[0] = M;
      part[1] = lsum;
    }
  }
}

template <int GQ, typename Lds>
__device__ void combine_and_store(Lds& L, const DecodeArgs& a, int b, int h, int unit, int wave, int lane,
                                  const float (&m)[GQ], const float (&l)[GQ], const float (&o)[GQ][2], int c0, int c1) {
  __syncthreads();  // co shares its LDS with the walks' buffers
#pragma unroll
  for (int hh = 0; hh < GQ; ++hh) {
    L.co[wave][hh][c0] = o[hh][0];
    L.co[wave][hh][c1] = o[hh][1];
    if (lane == 0) {
      L.cm[wave][hh] = m[hh];
      L.cl[wave][hh] = l[hh];
    }
  }
  combine_waves<GQ>(L, a, b, h, unit);
}

template <int GQ>
__device__ inline void softmax_update(float (&m)[GQ], float (&l)[GQ], float (&o)[GQ][2], int hh, float mx_tile,
                                      float& mnew_out) {
  const float mnew = fmaxf(m[hh], mx_tile);
  const float sc = exp2_safe_diff(m[hh], mnew);
  l[hh] *= sc;
  o[hh][0] *= sc;
  o[hh][1] *= sc;
  m[hh] = mnew;
  mnew_out = mnew;
}

// The bf16 band (sink and tail tokens, original frame) of one (sequence, kv head) walked by NW waves: wave w
// takes the 64-token blocks w, w + NW, ..; each lane one token of a block for the logits (its whole key row
// in flight at once), then channels 2 lane, 2 lane + 1 of the block's value rows, 16 tokens at a time with
// the next 16 in flight.  qb: the GQ heads' queries times log2e/sqrt(128) in LDS; pb: this wave's softmax
// numerators [GQ][64] in LDS.  Returns the wave's partial (m, l, o) of every head.
template <int GQ, int NW>
__device__ void band_walk(const DecodeArgs& a, int b, int h, int T, const float (*qb)[D], float (*pb)[64], int wave,
                          int lane, float (&m)[GQ], float (&l)[GQ], float (&o)[GQ][2]) {
  const Geo& g = a.g;
  const int ng = n_groups_of(T, g.S0, g.W);
  const int n_sink = T < g.S0 ? T : g.S0;
  const int tail0 = g.S0 + GROUP * ng;
  const int n_tail = T > tail0 ? T - tail0 : 0;
  const int nb = n_sink + n_tail;
  const uint16_t* band = a.band + ((long long)b * g.n_kv + h) * g.slots * 256;
#pragma unroll
  for (int hh = 0; hh < GQ; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.0f;
    o[hh][0] = o[hh][1] = 0.0f;
  }
  auto slot_of = [&](int k) {
    const int pos = k < n_sink ? k : tail0 + (k - n_sink);
    return band_slot_of(pos, g.S0, g.W);
  };
  for (int blk = wave; blk * 64 < nb; blk += NW) {
    const int k = blk * 64 + lane;
    const bool valid = k < nb;
    float lg[GQ];
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) lg[hh] = 0.0f;
    if (valid) {
      const uint4* kr = reinterpret_cast<const uint4*>(band + (long long)slot_of(k) * 256);
      uint4 kw[16];  // the token's whole key row in flight at once
#pragma unroll
      for (int v8 = 0; v8 < 16; ++v8) kw[v8] = kr[v8];
#pragma unroll
      for (int v8 = 0; v8 < 16; ++v8) {
        const uint4 w = kw[v8];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int p2 = 0; p2 < 4; ++p2) {
          const float k0 = __uint_as_float(ws[p2] << 16), k1 = __uint_as_float(ws[p2] & 0xffff0000u);
          const int c = v8 * 8 + p2 * 2;
#pragma unroll
          for (int hh = 0; hh < GQ; ++hh) lg[hh] += qb[hh][c] * k0 + qb[hh][c + 1] * k1;
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      const float x = valid ? lg[hh] : -INFINITY;
      float mnew;
      softmax_update<GQ>(m, l, o, hh, wave_max(x), mnew);
      const float p = valid ? exp2f(x - mnew) : 0.0f;
      pb[hh][lane] = p;
      l[hh] += wave_sum(p);
    }
    wave_lds_sync();
    const int nk = (nb - blk * 64) < 64 ? (nb - blk * 64) : 64;
    constexpr int VB = 16;
    auto load_rows = [&](int k0, uint32_t (&dst)[VB]) {
#pragma unroll
      for (int q = 0; q < VB; ++q) {
        const int kk = k0 + q < nk ? k0 + q : nk - 1;
        dst[q] = *reinterpret_cast<const uint32_t*>(band + (long long)slot_of(blk * 64 + kk) * 256 + 128 + 2 * lane);
      }
    };
    uint32_t vn[VB];
    load_rows(0, vn);
    for (int k8 = 0; k8 < nk; k8 += VB) {
      uint32_t vv[VB];
#pragma unroll
      for (int q = 0; q < VB; ++q) vv[q] = vn[q];
      if (k8 + VB < nk) load_rows(k8 + VB, vn);
#pragma unroll
      for (int q = 0; q < VB; ++q) {
        if (k8 + q >= nk) break;
        const float v0 = __uint_as_float(vv[q] << 16), v1 = __uint_as_float(vv[q] & 0xffff0000u);
#pragma unroll
        for (int hh = 0; hh < GQ; ++hh) {
          const float p = pb[hh][k8 + q];
          o[hh][0] += p * v0;
          o[hh][1] += p * v1;
        }
      }
    }
    wave_lds_sync();
  }
}

// The band unit of the split-K launch: one work-group (4 waves) per (sequence, kv head), its partial stored
// as unit 0.
template <int GQ, typename Lds>
__device__ void band_unit(Lds& L, const DecodeArgs& a, int b, int h, int T) {
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int e = tid; e < GQ * D; e += kThreads)
    L.f.qband[e / D][e % D] = a.qband[((long long)b * g.n_q + h * GQ + e / D) * D + e % D];
  __syncthreads();
  float m[GQ], l[GQ], o[GQ][2];
  band_walk<GQ, 4>(a, b, h, T, L.f.qband, reinterpret_cast<float(*)[64]>(&L.f.p[wave][0][0]), wave, lane, m, l, o);
  combine_and_store<GQ>(L, a, b, h, 0, wave, lane, m, l, o, 2 * lane, 2 * lane + 1);
}

// The band unit of the matrix-core decode at GQ 8: the bf16 sink and tail tokens of one (sequence, kv head) on
// v_mfma_f32_16x16x32_bf16, the work-group's four waves taking blocks of 64 tokens in turn and combined in
// LDS into the partial of unit 0.  Matrix columns are the kv head's GQ query heads (the other columns hold a
// zero query and are dropped); the query (original frame, log2e / sqrt(d) folded in) and the softmax weights
// are split into bf16 hi + lo against the exact bf16 keys and values, with fp32 sums.
//  - logits S^T (64 tokens x 16 columns): token 16 mt + (l % 16) is the A row, k = channels 32 ks + 8 q + e;
//  - values O^T (128 channels x 16 columns) += V^T P^T: k = 8 q + e is token 32 ks + 4 q + e (e < 4) or
//    32 ks + 16 + 4 q + e - 4 (e >= 4), the lane's own weights of tiles 2 ks and 2 ks + 1;
//  - results: column l % 16, rows 4 q + 0..3.
template <int GQ, typename Lds>
__device__ void band_unit_mfma(Lds& L, const DecodeArgs& a, int b, int h, int T) {
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, col = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ng = n_groups_of(T, g.S0, g.W);
  const int n_sink = T < g.S0 ? T : g.S0;
  const int tail0 = g.S0 + GROUP * ng;
  const int n_tail = T > tail0 ? T - tail0 : 0;
  const int nb = n_sink + n_tail;
  const uint16_t* band = a.band + ((long long)b * g.n_kv + h) * g.slots * 256;
  auto bslot = [&](int k) { return band_slot_of(k < n_sink ? k : tail0 + (k - n_sink), g.S0, g.W); };
  const bool hv = col < GQ;
  kvq_u32x4 qh[4], ql[4];
  {
    const float* qb = a.qband + ((long long)b * g.n_q + h * GQ + (hv ? col : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = hv ? qb[32 * ks + 8 * q + e] : 0.0f;
      split8(x, qh[ks], ql[ks]);
    }
  }
  float mb = -INFINITY, lb = 0.0f;
  kvq_f32x4 ob[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) ob[i] = kvq_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int k0 = 64 * wave; k0 < nb; k0 += 256) {
    float s[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int kk = min(k0 + 16 * mt + col, nb - 1);  // rows past the band repeat a valid one
      const uint16_t* kr = band + (long long)bslot(kk) * 256;
      kvq_f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const kvq_u32x4 av = *reinterpret_cast<const kvq_u32x4*>(kr + 32 * ks + 8 * q);
        acc = mfma_bf16(av, qh[ks], acc);
        acc = mfma_bf16(av, ql[ks], acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) s[mt][i] = (k0 + 16 * mt + 4 * q + i < nb) ? acc[i] : -INFINITY;
    }
    float bm = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) bm = fmaxf(bm, s[mt][i]);
    bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));  // the column's maximum over the block
    const float mnew = fmaxf(mb, bm);
    const float sc = exp2_safe_diff(mb, mnew);
    float p[4][4], ps = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[mt][i] = exp2_safe_diff(s[mt][i], mnew);
        ps += p[mt][i];
      }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    lb = lb * sc + ps;
    mb = mnew;
    kvq_u32x4 ph[2], pl[2];
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
      const int c = 16 * mt + col;
      kvq_f32x4 acc = ob[mt] * sc;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = (uint32_t)band[(long long)slots[ks][2 * e] * 256 + 128 + c] |
                 ((uint32_t)band[(long long)slots[ks][2 * e + 1] * 256 + 128 + c] << 16);
        const kvq_u32x4 av = {w[0], w[1], w[2], w[3]};
        acc = mfma_bf16(av, ph[ks], acc);
        acc = mfma_bf16(av, pl[ks], acc);
      }
      ob[mt] = acc;
    }
  }
  // the four waves' partials to LDS (column col = head, channels 16 mt + 4 q + i), then combined
  __syncthreads();
  if (hv) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) L.co[wave][col][16 * mt + 4 * q + i] = ob[mt][i];
    if (q == 0) {
      L.cm[wave][col] = mb;
      L.cl[wave][col] = lb;
    }
  }
  combine_waves<GQ>(L, a, b, h, 0);
}

template <int GQ, typename Lds>
__device__ void int2_unit(Lds& L, const DecodeArgs& a, int b, int h, int T, int chunk) {
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ng = n_groups_of(T, g.S0, g.W);
  const int g_begin = chunk * g.gpc;
  int g_end = (g_begin + g.gpc) < ng ? (g_begin + g.gpc) : ng;
  if (g_end > g.max_pages / 2) g_end = g.max_pages / 2;  // never index past the page-table row
  float qr[GQ][2];
#pragma unroll
  for (int hh = 0; hh < GQ; ++hh) {
    const float* q = a.qrot + ((long long)b * g.n_q + h * GQ + hh) * D;
    qr[hh][0] = q[lane];
    qr[hh][1] = q[lane + 64];
  }
  float m[GQ], l[GQ], o[GQ][2];
#pragma unroll
  for (int hh = 0; hh < GQ; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.0f;
    o[hh][0] = o[hh][1] = 0.0f;
  }
  const int32_t* pt = a.page_table + (long long)b * g.max_pages;
  const long long hoff = (long long)h * I2_HEAD_BYTES;
  for (int gi = g_begin + wave; gi < g_end; gi += 4) {
    const uint8_t* pg[2] = {a.pages + pool_page(g, pt[2 * gi]) * g.page_bytes + hoff,
                            a.pages + pool_page(g, pt[2 * gi + 1]) * g.page_bytes + hoff};
    const uint16_t* km = reinterpret_cast<const uint16_t*>(pg[0] + I2_META_OFF);
    const uint16_t* vm = reinterpret_cast<const uint16_t*>(pg[1] + I2_META_OFF);
    const float sk0 = bf16_to_f32(km[lane]), sk1 = bf16_to_f32(km[lane + 64]);
    const float zk0 = bf16_to_f32(km[D + lane]), zk1 = bf16_to_f32(km[D + lane + 64]);
    float beta[GQ];
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      const float a0 = qr[hh][0] * sk0, a1 = qr[hh][1] * sk1;
      L.f.alpha[wave][hh][lane] = a0;
      L.f.alpha[wave][hh][lane + 64] = a1;
      beta[hh] = wave_sum(a0 * zk0 + a1 * zk1);
    }
    wave_lds_sync();
    // logits of tokens lane (page 0) and 64 + lane (page 1)
    float lg[2][GQ];
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const uint4* kp = reinterpret_cast<const uint4*>(pg[pp] + I2_K_OFF + lane * 32);
      float acc[GQ];
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) acc[hh] = 0.0f;
#pragma unroll 1
      for (int half = 0; half < 2; ++half) {
        const uint4 kk = kp[half];
        const uint32_t w[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
#pragma unroll 1
          for (int by = 0; by < 4; ++by) {
            const uint32_t x = w[wd] >> (8 * by);
            const float f0 = (float)(x & 3u), f1 = (float)((x >> 2) & 3u), f2 = (float)((x >> 4) & 3u),
                        f3 = (float)((x >> 6) & 3u);
            const int c = half * 64 + wd * 16 + by * 4;
#pragma unroll
            for (int hh = 0; hh < GQ; ++hh) {
              const float4 al = *reinterpret_cast<const float4*>(&L.f.alpha[wave][hh][c]);
              acc[hh] += al.x * f0 + al.y * f1 + al.z * f2 + al.w * f3;
            }
          }
        }
      }
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) lg[pp][hh] = acc[hh] - beta[hh];
    }
    float P[GQ];
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      float mnew;
      softmax_update<GQ>(m, l, o, hh, wave_max(fmaxf(lg[0][hh], lg[1][hh])), mnew);
      const float p0 = exp2f(lg[0][hh] - mnew), p1 = exp2f(lg[1][hh] - mnew);
      L.f.p[wave][hh][lane] = p0;
      L.f.p[wave][hh][64 + lane] = p1;
      P[hh] = wave_sum(p0 + p1);
      l[hh] += P[hh];
    }
    wave_lds_sync();
    // V: channels lane and lane + 64
    float u[GQ][2];
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) u[hh][0] = u[hh][1] = 0.0f;
#pragma unroll 1
    for (int pp = 0; pp < 2; ++pp) {
      const uint4 r0 = *reinterpret_cast<const uint4*>(pg[pp] + I2_V_OFF + lane * 16);
      const uint4 r1 = *reinterpret_cast<const uint4*>(pg[pp] + I2_V_OFF + (lane + 64) * 16);
      const uint32_t w0[4] = {r0.x, r0.y, r0.z, r0.w}, w1[4] = {r1.x, r1.y, r1.z, r1.w};
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
#pragma unroll 1
        for (int j = 0; j < 4; ++j) {
          const uint32_t x0 = w0[gg] >> (8 * j), x1 = w1[gg] >> (8 * j);
          const int i0 = pp * 64 + 16 * j + 4 * gg;
#pragma unroll
          for (int hh = 0; hh < GQ; ++hh) {
            const float4 p4 = *reinterpret_cast<const float4*>(&L.f.p[wave][hh][i0]);
            u[hh][0] += p4.x * (float)(x0 & 3u) + p4.y * (float)((x0 >> 2) & 3u) + p4.z * (float)((x0 >> 4) & 3u) +
                        p4.w * (float)((x0 >> 6) & 3u);
            u[hh][1] += p4.x * (float)(x1 & 3u) + p4.y * (float)((x1 >> 2) & 3u) + p4.z * (float)((x1 >> 4) & 3u) +
                        p4.w * (float)((x1 >> 6) & 3u);
          }
        }
      }
    }
    const float sv0 = bf16_to_f32(vm[lane]), sv1 = bf16_to_f32(vm[lane + 64]);
    const float zv0 = bf16_to_f32(vm[D + lane]), zv1 = bf16_to_f32(vm[D + lane + 64]);
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      o[hh][0] += sv0 * (u[hh][0] - zv0 * P[hh]);
      o[hh][1] += sv1 * (u[hh][1] - zv1 * P[hh]);
    }
    wave_lds_sync();
  }
  combine_and_store<GQ>(L, a, b, h, 1 + chunk, wave, lane, m, l, o, lane, lane + 64);
}

// ---------------------------------------------------------------------------------------------
// Cross-lane reductions of the matrix-core decode.
// seg_reduce<N>: reduce within aligned segments of N lanes (N = 8..64); every lane of a segment gets the
// segment's result.  Pairings: quad xor 1, quad xor 2, half-row mirror, row mirror (DPP), then xor 16
// and xor 32 (cross-row exchanges).
// ---------------------------------------------------------------------------------------------
#define KVQ_MOVDPP(x, ctrl) __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), (ctrl), 0xF, 0xF, false))

template <int N, typename Op>
__device__ inline float seg_reduce(float x, Op op) {
  x = op(x, KVQ_MOVDPP(x, 0xB1));   // quad_perm [1,0,3,2]
  x = op(x, KVQ_MOVDPP(x, 0x4E));   // quad_perm [2,3,0,1]
  x = op(x, KVQ_MOVDPP(x, 0x141));  // row_half_mirror: i <-> 7-i
  if (N >= 16) x = op(x, KVQ_MOVDPP(x, 0x140));  // row_mirror: i <-> 15-i
  if (N >= 32) {  // rows 0|1 and 2|3
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  if (N >= 64) {  // halves
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return x;
}

// Wave-uniform read of data the kernel never writes, through the scalar cache (constant address space).
__device__ inline int2 scalar_load_int2(const int2* p) {
  const __attribute__((address_space(4))) int* q = (const __attribute__((address_space(4))) int*)(uintptr_t)p;
  return make_int2(q[0], q[1]);
}
__device__ inline int scalar_load_int(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int*)(uintptr_t)p;
}

template <int GQ>
struct HeadLog2 {
  static constexpr int v = GQ == 1 ? 0 : GQ == 2 ? 1 : GQ == 4 ? 2 : 3;
};

struct OpMax {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};

// Segment reductions whose cross-lane moves fold into the operation (v_add_f32_dpp, v_max_i32_dpp): the
// moves read valid lanes only, so the bound-control fill value never enters a result.
#define KVQ_UPDDPP(x, ctrl) __builtin_amdgcn_update_dpp(0, (x), (ctrl), 0xF, 0xF, true)
template <int N>
__device__ inline float seg_sum(float x) {
  x += __int_as_float(KVQ_UPDDPP(__float_as_int(x), 0xB1));
  x += __int_as_float(KVQ_UPDDPP(__float_as_int(x), 0x4E));
  x += __int_as_float(KVQ_UPDDPP(__float_as_int(x), 0x141));
  if (N >= 16) x += __int_as_float(KVQ_UPDDPP(__float_as_int(x), 0x140));
  if (N >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if (N >= 64) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return x;
}
template <int N>
__device__ inline int seg_max_i(int x) {
  x = max(x, KVQ_UPDDPP(x, 0xB1));
  x = max(x, KVQ_UPDDPP(x, 0x4E));
  x = max(x, KVQ_UPDDPP(x, 0x141));
  if (N >= 16) x = max(x, KVQ_UPDDPP(x, 0x140));
  if (N >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
    x = max((int)r[0], (int)r[1]);
  }
  if (N >= 64) {
    const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
    x = max((int)r[0], (int)r[1]);
  }
  return x;
}

// max of two floats without the sNaN quieting that fmaxf adds for operands of unknown origin
__device__ inline float fmax_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// ---------------------------------------------------------------------------------------------
// Global -> LDS copies of 16 bytes per lane (lane i's bytes land at the LDS address in M0 + 16 i), issued
// from inline assembly so that the compiler adds no waits of its own for them: the matrix-core units keep
// every global read of their loops in this form and wait on the vector-memory counter explicitly.  Per-lane
// 64-bit address, or a uniform base plus a per-lane 32-bit offset.  The blocks write M0, which the compiler
// does not track: no compiler-emitted instruction in these kernels may use M0 (the tests check the compiled
// assembly for exactly that).
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// NT: a non-temporal (streaming) read, for bytes that are read once per step.
template <bool NT = false>
__device__ inline void dma16(uint32_t lds, const void* gaddr) {
  if constexpr (NT) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(lds), "v"(gaddr) : "memory");
  } else {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(gaddr) : "memory");
  }
}
template <bool NT = false>
__device__ inline void dma16_base(uint32_t lds, const void* gbase, uint32_t voff) {
  if constexpr (NT) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(lds), "v"(voff), "s"(gbase)
                 : "memory");
  } else {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(gbase)
                 : "memory");
  }
}
// dma16_base for the lanes of one half of the wave (HI: lanes 32..63), inside a branch on the lane's half.  The
// two halves' blocks differ in text, so that the compiler keeps them in their branches (blocks merged after
// the branch would take a per-lane base).
template <bool HI>
__device__ inline void dma16_half(uint32_t lds, const void* gbase, uint32_t voff) {
  if constexpr (HI) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt ; upper half" ::"s"(lds), "v"(voff),
                 "s"(gbase) : "memory");
  } else {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt ; lower half" ::"s"(lds), "v"(voff),
                 "s"(gbase) : "memory");
  }
}
#define KVQ_WAIT_VM(n) asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory")
// The grouped schemes' code and metadata copies stream (measured on MI355X at batch 32 x 32k: the split-K
// kernel about 10% faster than with default-policy copies); the INT4 per-token walk keeps the default policy
// (measured slightly slower with streaming copies).
constexpr bool kStreamCopies = true;
template <int GQ, typename Lds>
__device__ void int4_unit(Lds& L, const DecodeArgs& a, int b, int h, int T, int chunk) {
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_pages = (T + PAGE - 1) / PAGE;
  const int p_begin = chunk * g.gpc;
  int p_end = (p_begin + g.gpc) < n_pages ? (p_begin + g.gpc) : n_pages;
  if (p_end > g.max_pages) p_end = g.max_pages;
  // rotated query of the GQ heads in every wave's alpha slot, and its channel sum
  float qsum[GQ];
#pragma unroll
  for (int hh = 0; hh < GQ; ++hh) {
    const float* q = a.qrot + ((long long)b * g.n_q + h * GQ + hh) * D;
    const float q0 = q[lane], q1 = q[lane + 64];
    L.f.alpha[wave][hh][lane] = q0;
    L.f.alpha[wave][hh][lane + 64] = q1;
    qsum[hh] = wave_sum(q0 + q1);
  }
  wave_lds_sync();
  float m[GQ], l[GQ], o[GQ][2];
#pragma unroll
  for (int hh = 0; hh < GQ; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.0f;
    o[hh][0] = o[hh][1] = 0.0f;
  }
  const int32_t* pt = a.page_table + (long long)b * g.max_pages;
  const long long hoff = (long long)h * I4_HEAD_BYTES;
  for (int pi = p_begin + wave; pi < p_end; pi += 4) {
    const uint8_t* pg = a.pages + pool_page(g, pt[pi]) * g.page_bytes + hoff;
    const int t = pi * PAGE + lane;
    const bool valid = t < T;
    const uint16_t* kmeta = reinterpret_cast<const uint16_t*>(pg + I4_KMETA_OFF + 4 * lane);
    const uint16_t* vmeta = reinterpret_cast<const uint16_t*>(pg + I4_VMETA_OFF + 4 * lane);
    const float sk = bf16_to_f32(kmeta[0]), zk = bf16_to_f32(kmeta[1]);
    const float sv = bf16_to_f32(vmeta[0]), zv = bf16_to_f32(vmeta[1]);
    float acc[GQ];
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) acc[hh] = 0.0f;
    const uint4* kp = reinterpret_cast<const uint4*>(pg + I4_K_OFF + lane * 64);
#pragma unroll 1
    for (int v16 = 0; v16 < 4; ++v16) {
      const uint4 w = kp[v16];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const int c = v16 * 32 + wd * 8;
        float f[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) f[k] = (float)((ws[wd] >> (4 * k)) & 15u);
#pragma unroll
        for (int hh = 0; hh < GQ; ++hh) {
          const float4 a0 = *reinterpret_cast<const float4*>(&L.f.alpha[wave][hh][c]);
          const float4 a1 = *reinterpret_cast<const float4*>(&L.f.alpha[wave][hh][c + 4]);
          acc[hh] += a0.x * f[0] + a0.y * f[1] + a0.z * f[2] + a0.w * f[3] + a1.x * f[4] + a1.y * f[5] +
                     a1.z * f[6] + a1.w * f[7];
        }
      }
    }
    float wz[GQ];
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      const float x = valid ? sk * (acc[hh] - zk * qsum[hh]) : -INFINITY;
      float mnew;
      softmax_update<GQ>(m, l, o, hh, wave_max(x), mnew);
      const float p = valid ? exp2f(x - mnew) : 0.0f;
      // slots past the end of the sequence hold unwritten scales/zeros: keep them out of every sum
      const float w = valid ? p * sv : 0.0f;
      L.f.p[wave][hh][lane] = w;
      l[hh] += wave_sum(p);
      wz[hh] = wave_sum(valid ? w * zv : 0.0f);
    }
    wave_lds_sync();
    // V: channels lane and lane + 64, rows of 32 bytes; token 16j + 4g + r in byte 8g + 2j + r/2
    const uint4* r0p = reinterpret_cast<const uint4*>(pg + I4_V_OFF + lane * 32);
    const uint4* r1p = reinterpret_cast<const uint4*>(pg + I4_V_OFF + (lane + 64) * 32);
    const uint4 a0 = r0p[0], a1 = r0p[1], b0 = r1p[0], b1 = r1p[1];
    const uint32_t w0[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const uint32_t w1[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
#pragma unroll 1
      for (int j = 0; j < 4; ++j) {
        // byte pair 8g + 2j lives in word (8g + 2j) / 4 at bit 8 * ((8g + 2j) % 4)
        const int wi = (8 * gg + 2 * j) >> 2, sh = 8 * ((8 * gg + 2 * j) & 3);
        const uint32_t x0 = w0[wi] >> sh, x1 = w1[wi] >> sh;
        const int i0 = 16 * j + 4 * gg;
#pragma unroll
        for (int hh = 0; hh < GQ; ++hh) {
          const float4 p4 = *reinterpret_cast<const float4*>(&L.f.p[wave][hh][i0]);
          o[hh][0] += p4.x * (float)(x0 & 15u) + p4.y * (float)((x0 >> 4) & 15u) + p4.z * (float)((x0 >> 8) & 15u) +
                      p4.w * (float)((x0 >> 12) & 15u);
          o[hh][1] += p4.x * (float)(x1 & 15u) + p4.y * (float)((x1 >> 4) & 15u) + p4.z * (float)((x1 >> 8) & 15u) +
                      p4.w * (float)((x1 >> 12) & 15u);
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      o[hh][0] -= wz[hh];
      o[hh][1] -= wz[hh];
    }
    wave_lds_sync();
  }
  combine_and_store<GQ>(L, a, b, h, 1 + chunk, wave, lane, m, l, o, lane, lane + 64);
}

// ---------------------------------------------------------------------------------------------
// INT2 per-channel chunk on the int8 matrix cores (v_mfma_i32_16x16x64_i8), fixed point.  Per group and head
// the key-side operand alpha = q~ s is rounded to integers a = rint(alpha S / max|alpha|) and the softmax
// weights p = 2^(logit - group max) in (0, 1] to u = rint(S p), S = 4,000,000 (2-bit codes) or 1,000,000
// (4-bit codes), each as three signed byte limbs lo + 256 mid + 65536 hi; with A = max|alpha| / S,
//   logit_t = A (sum_c a_c code_tc - sum_c a_c z_c),
//   o~_c   += (2^(group max - m) / S) s_c (sum_t u_t code_tc - z_c sum_t u_t).
// The rounding error is 2^-22 (2^-20) of the largest operand, so even attention that puts all its weight on
// one token (logits far apart, large value outliers) stays within the fp64 oracle's bar; two limbs (15 bits)
// did not.  Both sums are 16 x 16 x 64 matrix products whose rows are (head, limb) pairs, so the GQA heads
// that share the kv head also share one pass over the codes ([SAW] App. A.4 eq. 13-14; [NOVA] §2 query groups):
//   keys    D[(head, limb)][token]   = sum_channels limb(a) code, 8 token tiles x 2 channel halves;
//   values  D[(head, limb)][channel] = sum_tokens limb(u) code, 8 channel tiles x 2 pages;
// and sum_t u_t is one more product against a vector of ones.  The limb sums are exact int32 sums and the
// codes stay 2-bit in HBM: each 32-bit code word becomes four int8 vectors, (w >> 2n) & 0x03030303.
// Matrix rows: head h, limb L at row 4 h + L (GQ <= 4; rows with L = 3 are zero); at GQ = 8 the lo and mid
// limbs at rows 2 h + L of one tile and the hi limbs at rows 2 h of a second tile (odd rows zero).
// Operand layouts (lane l, q = l / 16, c = l % 16): A row c, k = 16 q + byte; B the same k, column c;
// D column c, rows 4 q + r.  So a lane's key results (head(s) of rows 4 q.., token column c) are its
// weights' producer lane, and its value results hold head q's channels c + 16 tau.
//  - key k order (k = 64 sigma + 16 q + 4 n + b): channel 16 (2 q + sigma) + 4 b + n, i.e. lane q expands
//    code words 2 q, 2 q + 1 of a token (channel 16 m + 4 b + n in byte b, bits 2 n);
//  - value k order (k = 64 kappa + 16 q + 4 n + b): token 64 kappa + 16 b + 4 q + n of page kappa, i.e. lane
//    q expands code word q of a channel (token 16 b + 4 q + n in byte b, bits 2 n);
//  - key tile i, column c: token T(i, c) = 64 (c / 8) + 2 (c % 8) + 16 (i % 4) + i / 4, the token at value
//    position 8 c + i, so each lane stores its 8 weights of a head as 8 consecutive bytes of a plane row.
// Key codes are staged with their rows permuted (token t at row t ^ ((t >> 2) & 3)) so that the 8-byte
// operand reads of a tile spread over all LDS banks.  All global reads are LDS copies, issued for a whole
// group (metadata, key and value codes: 9 KB of 2-bit codes) one group ahead: as soon as a group's codes
// are in registers, the next group's copies go out and stay in flight while this group is multiplied.
// The wait at the top of a group counts every copy.
// ---------------------------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(4))) int mf_i32x4;

__device__ __forceinline__ mf_i32x4 mfma_i8x64(mf_i32x4 a, mf_i32x4 b, mf_i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ mf_i32x4 u4_i32x4(uint4 v) { return mf_i32x4{(int)v.x, (int)v.y, (int)v.z, (int)v.w}; }
template <int BITS>
struct Limb3 {
  static constexpr float S = BITS == 2 ? 4000000.0f : 1000000.0f;
};
// A head's value lo + 256 mid + 65536 hi from the matrix-core limb sums of this lane (two's complement; the
// true value fits in int32).  Rows 4 q + r of a result tile: up to GQ 4 head q with limb r (r < 3); at GQ 8
// heads 2 q + r / 2 with limb r % 2, the top limbs in a second tile at rows 4 q + 2 e.
template <int GQ>
__device__ __forceinline__ int limbs3_sum(const mf_i32x4& t, const mf_i32x4& x, int e) {
  // plain integer arithmetic on the matrix-core results: the compiler places the wait states the matrix
  // cores need before a vector instruction reads their results (it cannot for inline assembly)
  const uint32_t hi = GQ == 8 ? (uint32_t)x[2 * e] : (uint32_t)t[2];
  const uint32_t mid = GQ == 8 ? (uint32_t)t[2 * e + 1] : (uint32_t)t[1];
  const uint32_t lo = GQ == 8 ? (uint32_t)t[2 * e] : (uint32_t)t[0];
  return (int)((((hi << 8) + mid) << 8) + lo);
}
// N 32-bit words to LDS at dst (aligned to 4 N bytes).
template <int N>
__device__ __forceinline__ void store_words(uint8_t* dst, const uint32_t (&w)[N]) {
  if constexpr (N == 4) *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  else if constexpr (N == 2) *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
  else *reinterpret_cast<uint32_t*>(dst) = w[0];
}
// The key-side operand of one head: x holds this lane's NCH positions (Q0..), the head's LPH lanes hold
// all 128.  a = rint(x S / max|x|) over the head goes to rows rows, rows + RS, rows + 2 RS (lo, mid, hi),
// bytes 0..NCH-1; zsum gets the head's sum of a zk (ZX: of x zk, which A a equals to 2^-23 of max|x|);
// returns A = max|x| / S (logit = A sum a code).
template <int LPH, int NCH, int RS, bool ZX = false>
__device__ __forceinline__ float round_operand3(const float (&x)[NCH], const float (&zk)[NCH], float S, uint8_t* rows,
                                                float& zsum) {
  int amx_i = 0;  // max |x| as its bit pattern (non-negative floats order as their bits)
#pragma unroll
  for (int i = 0; i < NCH; ++i) amx_i = max(amx_i, __float_as_int(fabsf(x[i])));
  const float amx = __int_as_float(seg_max_i<LPH>(amx_i));
  // |rint(x inv)| <= S + 1: far inside the limbs' range (4,161,407)
  const float inv = amx > 0x1p-100f ? S * __builtin_amdgcn_rcpf(amx) : 0.0f;
  float ev[NCH];
  float zs = 0.0f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    ev[i] = fmaf(x[i], inv, kRound3);
    zs = ZX ? fmaf(x[i], zk[i], zs) : fmaf(ev[i] - kRound3, zk[i], zs);  // ev - kRound3 = a exactly
  }
  zsum = seg_sum<LPH>(zs);
  if constexpr (NCH >= 4) {
    uint32_t lo[NCH / 4], mid[NCH / 4], hi[NCH / 4];
#pragma unroll
    for (int k = 0; k < NCH / 4; ++k)
      limbs3(ev[4 * k], ev[4 * k + 1], ev[4 * k + 2], ev[4 * k + 3], lo[k], mid[k], hi[k]);
    store_words<NCH / 4>(rows, lo);
    store_words<NCH / 4>(rows + RS, mid);
    store_words<NCH / 4>(rows + 2 * RS, hi);
  } else {
    uint32_t lo, mid, hi;
    limbs3(ev[0], ev[1], ev[0], ev[1], lo, mid, hi);
    *reinterpret_cast<uint16_t*>(rows) = (uint16_t)lo;
    *reinterpret_cast<uint16_t*>(rows + RS) = (uint16_t)mid;
    *reinterpret_cast<uint16_t*>(rows + 2 * RS) = (uint16_t)hi;
  }
  return amx * (1.0f / S);
}
// Eight weights of one head (value positions 8 c + i, rounded with kRoundU) to its three limb rows.
template <int RS>
__device__ __forceinline__ void store_weights3(uint8_t* dst, const float (&ew)[8]) {
  uint32_t lo0, mid0, hi0, lo1, mid1, hi1;
  limbs3u(ew[0], ew[1], ew[2], ew[3], lo0, mid0, hi0);
  limbs3u(ew[4], ew[5], ew[6], ew[7], lo1, mid1, hi1);
  *reinterpret_cast<uint2*>(dst) = make_uint2(lo0, lo1);
  *reinterpret_cast<uint2*>(dst + RS) = make_uint2(mid0, mid1);
  *reinterpret_cast<uint2*>(dst + 2 * RS) = make_uint2(hi0, hi1);
}
// key k position -> channel (see the k order above)
__host__ __device__ constexpr int mf_key_channel(int Q) {
  return 16 * (2 * ((Q & 63) >> 4) + (Q >> 6)) + 4 * (Q & 3) + ((Q & 15) >> 2);
}

// two 32-bit words of 4-bit codes as 16 int8 values: low nibbles of w0, high of w0, low of w1, high of w1
__device__ __forceinline__ mf_i32x4 nibbles_i8(uint32_t w0, uint32_t w1) {
  return mf_i32x4{(int)(w0 & 0x0F0F0F0Fu), (int)((w0 >> 4) & 0x0F0F0F0Fu), (int)(w1 & 0x0F0F0F0Fu),
                  (int)((w1 >> 4) & 0x0F0F0F0Fu)};
}
// key k position -> channel, per-channel INT4 (channel 16 m + 2 k + e in word 2 m + e, nibble k): lane q
// reads words 4 q + 2 sigma, + 1 of a token row, whose low and high nibbles give channels 16 (2 q + sigma) +
// 4 b + 2 h + e (b the byte, h = high nibble, e the word's parity); k = 64 sigma + 16 q + 4 (2 e + h) + b
__host__ __device__ constexpr int mf_key_channel_c4(int Q) {
  return 16 * (2 * ((Q & 63) >> 4) + (Q >> 6)) + 4 * (Q & 3) + 2 * (((Q & 15) >> 2) & 1) + (((Q & 15) >> 2) >> 1);
}

template <int GQ, bool TOK, int BITS, typename Lds>
__device__ void int2_unit_mfma(Lds& L, const DecodeArgs& a, int b, int h, int T, int c0, int c1, int gpc) {
  constexpr int LG = HeadLog2<GQ>::v;
  constexpr int LPH = 64 >> LG;        // lanes per head in the alpha step
  constexpr int NCH = 2 * GQ;          // key positions per lane in the alpha step
  constexpr int RPH = GQ == 8 ? 2 : 4;  // matrix rows per head (first tile)
  constexpr int HPL = GQ == 8 ? 2 : 1;  // heads per lane in the results
  constexpr int KU = 128 * BITS;  // staging of a group's key or value codes, in 16-byte units
  constexpr int NCP = KU / 64;    // copies per group and side
  constexpr int RS = MfmaWave<GQ, KU>::RSTRIDE;
  constexpr int ROWS = MfmaWave<GQ, KU>::ROWS;
  constexpr float S = Limb3<BITS>::S;
  constexpr bool M1 = MfmaWave<GQ, KU>::MB == 1;  // one metadata buffer: its words to registers first
  static_assert(!M1 || (NCH == 16 && BITS == 2), "single metadata buffer: GQ 8, 2-bit codes");
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ng = n_groups_of(T, g.S0, g.W);
  // this wave walks chunks c0 .. c1 - 1 of gpc groups (groups g_first .. g_end - 1), storing a partial per
  // chunk; groups past the launch bound are cut
  const int g_first = c0 * gpc;
  int g_end = c1 * gpc;
  if (g_end > ng) g_end = ng;
  if (g_end > (g.n_units - 1) * g.gpc) g_end = (g.n_units - 1) * g.gpc;
  if (g_end > g.max_pages / 2) g_end = g.max_pages / 2;            // never index past the page-table row
  MfmaWave<GQ, KU>& W = L.mf.w[wave];
  const int q4 = lane >> 4, c = lane & 15;

  // the rows no head fills read the zero row of the plane
  if (lane < 32) reinterpret_cast<uint32_t*>(W.plane + ROWS * RS)[lane] = 0u;
  // A-operand rows of this lane: matrix row c = (head, limb); at GQ 8 a second tile of top limbs
  const int rh = c / RPH, rl = c % RPH;
  const int prow = GQ == 8 ? 3 * rh + rl : ((rl < 3 && rh < GQ) ? 3 * rh + rl : ROWS);
  const int prow2 = rl == 0 ? 3 * rh + 2 : ROWS;
  const uint8_t* op_rd = W.plane + prow * RS + 16 * q4;
  const uint8_t* op_rd2 = W.plane + prow2 * RS + 16 * q4;
  auto load_op = [&](mf_i32x4 (&A)[2][2]) {
    A[0][0] = u4_i32x4(*reinterpret_cast<const uint4*>(op_rd));
    A[0][1] = u4_i32x4(*reinterpret_cast<const uint4*>(op_rd + 64));
    if constexpr (GQ == 8) {
      A[1][0] = u4_i32x4(*reinterpret_cast<const uint4*>(op_rd2));
      A[1][1] = u4_i32x4(*reinterpret_cast<const uint4*>(op_rd2 + 64));
    }
  };
  // key operand reads. 2-bit: tile i at staged row 64 (c / 8) + 4 ((c / 2) % 4) + 16 (i % 4) + (y0 ^ (i / 4)),
  // 8 bytes 8 q4..; 4-bit: token row T(i, c) = 64 (c / 8) + 4 ((c / 2) % 4) + (c % 2) + 16 (i % 4) + 2 (i / 4)
  // as it is, 16 bytes 16 q4..
  const int y0 = (2 * (c & 1)) ^ ((c >> 1) & 3);
  const int krow = 64 * (c >> 3) + 4 * ((c >> 1) & 3);
  const uint8_t* k_rd0 = BITS == 2 ? reinterpret_cast<const uint8_t*>(W.kst) + 32 * (krow + y0) + 8 * q4
                                   : reinterpret_cast<const uint8_t*>(W.kst) + 64 * (krow + (c & 1)) + 16 * q4;
  const uint8_t* k_rd1 = BITS == 2 ? reinterpret_cast<const uint8_t*>(W.kst) + 32 * (krow + (y0 ^ 1)) + 8 * q4
                                   : k_rd0 + 128;
  // value operand reads: channel c + 16 tau, code word q4 (2-bit) or words 2 q4, 2 q4 + 1 (4-bit), page kappa
  const uint32_t* v_rd = reinterpret_cast<const uint32_t*>(W.vst) + (BITS == 2 ? 4 * c + q4 : 8 * c + 2 * q4);
  // alpha step: head ah, key positions Q0 .. Q0 + NCH - 1
  const int ah = lane >> (6 - LG);
  const int Q0 = (lane & (LPH - 1)) * NCH;
  uint8_t* const a_rows = W.plane + (3 * ah) * RS + Q0;
  // copies: per-lane offsets of the permuted key rows (copy j: page j / 2, 16-byte slots 64 j + lane, i.e.
  // half lane % 2 of staged row 32 (j % 2) + lane / 2 of that page)
  uint32_t koff[2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int tl = 32 * jj + ((lane >> 1) ^ ((lane >> 3) & 3));
    koff[jj] = (uint32_t)(tl * 32 + 16 * (lane & 1));
  }
  const uint32_t kst_a = lds_addr(W.kst), vst_a = lds_addr(W.vst);
  const uint32_t mst_a0 = lds_addr(W.mst[0]), mst_a1 = lds_addr(W.mst[M1 ? 0 : 1]);
  const uint8_t* pages = a.pages;
  const long long pbytes = g.page_bytes, hoff = (long long)h * g.head_bytes;
  auto page_of = [&](int idx) { return pages + pool_page(g, idx) * pbytes + hoff; };
  constexpr int META = BITS == 2 ? I2_META_OFF : I4C_META_OFF;
  constexpr int KOFF = BITS == 2 ? I2_K_OFF : I4C_K_OFF, VOFF = BITS == 2 ? I2_V_OFF : I4C_V_OFF;
  auto issue_m = [&](int2 p, int buf) {
    if constexpr (M1) {
      // the two pages' halves as two copies of 32 lanes each: page bases in scalar registers (taken before the
      // branch), 32-bit lane offsets
      auto uniform = [](const uint8_t* ptr) {
        const uint64_t v = (uint64_t)(uintptr_t)ptr;
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
        return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
      };
      const uint8_t* bx = uniform(page_of(p.x) + META);
      const uint8_t* by = uniform(page_of(p.y) + META);
      const uint32_t off = (uint32_t)(lane & 31) * 16;
      if (lane < 32) dma16_half<false>(mst_a0, bx, off);
      else dma16_half<true>(mst_a0, by, off);
    } else {
      const uint8_t* src = (lane >= 32 ? page_of(p.y) : page_of(p.x)) + META + (lane & 31) * 16;
      dma16<kStreamCopies>(buf ? mst_a1 : mst_a0, src);
    }
  };
  auto issue_k = [&](int2 p) {
    if constexpr (BITS == 2) {
#pragma unroll
      for (int j = 0; j < 4; ++j) dma16_base<kStreamCopies>(kst_a + 1024 * j, page_of(j < 2 ? p.x : p.y) + KOFF, koff[j & 1]);
    } else {
#pragma unroll
      for (int j = 0; j < NCP; ++j)
        dma16_base<kStreamCopies>(kst_a + 1024 * j, page_of(j < NCP / 2 ? p.x : p.y) + KOFF + 1024 * (j % (NCP / 2)), lane * 16);
    }
  };
  auto issue_v = [&](int2 p) {
#pragma unroll
    for (int j = 0; j < NCP; ++j)
      dma16_base<kStreamCopies>(vst_a + 1024 * j, page_of(j < NCP / 2 ? p.x : p.y) + VOFF + 1024 * (j % (NCP / 2)), lane * 16);
  };

  float qa[NCH];
  {
    const float* q = a.qrot + ((long long)b * g.n_q + h * GQ + ah) * D;
#pragma unroll
    for (int i = 0; i < NCH; ++i) qa[i] = q[BITS == 2 ? mf_key_channel(Q0 + i) : mf_key_channel_c4(Q0 + i)];
#pragma unroll
    for (int i = 0; i < NCH; ++i) asm volatile("" ::"v"(qa[i]));  // the loads' wait stays before the walk
  }
  // per-head values of this lane's result heads (head q4 HPL + e is the key step's lanes (q4 HPL + e) LPH)
  auto head_value = [&](float v, int e) { return __shfl(v, ((q4 * HPL + e) & (GQ - 1)) * LPH, 64); };
  // per-token INT2: the key-side operand is the rotated query itself, once per walk
  float At[HPL], FSt[HPL];
  mf_i32x4 At_op[2][2];
  if constexpr (TOK) {
    float one[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) one[i] = 1.0f;
    float fs;
    const float Ah = round_operand3<LPH, NCH, RS>(qa, one, S, a_rows, fs);
#pragma unroll
    for (int e = 0; e < HPL; ++e) {
      At[e] = head_value(Ah, e);
      FSt[e] = head_value(fs, e);
    }
    wave_lds_sync();
    load_op(At_op);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before the first weights overwrite the plane
  }
  float m[HPL], l[HPL], o[HPL][8];
#pragma unroll
  for (int e = 0; e < HPL; ++e) {
    m[e] = -INFINITY;
    l[e] = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) o[e][t] = 0.0f;
  }
  // page pairs: the first by scalar loads; afterwards a group's copies go out together with a vector load of
  // the pair after it, which arrives with them (a scalar-cache miss on the page table, cold every step, would
  // otherwise hold up the next group's copies)
  const int32_t* ptrow = a.page_table + (long long)b * g.max_pages;
  auto pair_v = [&](int gi) { return make_int2(ptrow[2 * gi], ptrow[2 * gi + 1]); };
  int2 pv = make_int2(0, 0);
  int mb = 0;
  if (g_first < g_end) {
    const int2 p0 = scalar_load_int2(reinterpret_cast<const int2*>(ptrow) + g_first);
    issue_m(p0, 0);
    issue_k(p0);
    issue_v(p0);
    if (g_first + 1 < g_end) pv = pair_v(g_first + 1);
  }
  // the partial of chunk ci (per channel, o and l carry the weights' factor S), then a fresh softmax state;
  // every partial a merge reads is written, chunks past the length have none
  auto store_partial = [&](int ci) {
#pragma unroll
    for (int e = 0; e < HPL; ++e) {
      const int he = q4 * HPL + e;
      const float f = TOK ? 1.0f : 1.0f / S;
      if (he < GQ) {
        float* part = a.partials + (((long long)b * g.n_q + h * GQ + he) * g.n_units + 1 + ci) * PART_STRIDE;
#pragma unroll
        for (int t = 0; t < 8; ++t) part[2 + c + 16 * t] = o[e][t] * f;
        if (c == 0) {
          part[0] = m[e];
          part[1] = l[e] * f;
        }
      }
      m[e] = -INFINITY;
      l[e] = 0.0f;
#pragma unroll
      for (int t = 0; t < 8; ++t) o[e][t] = 0.0f;
    }
  };
  const mf_i32x4 zero4 = {0, 0, 0, 0};
  const mf_i32x4 ones4 = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
  int left = gpc;  // groups left in the current chunk
  for (int gi = g_first; gi < g_end; ++gi) {
    const bool has_next = gi + 1 < g_end;  // uniform
    KVQ_WAIT_VM(0);  // this group's metadata, key and value codes, and the next group's pages
    wave_lds_sync();
    // 0. the group's codes to registers (key tiles: 2-bit .x, .y; 4-bit all four words; value tiles: 2-bit
    //    .x, 4-bit both words), then the next group's copies into the buffers they leave
    uint4 kw[8];
    uint2 vw[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (BITS == 2) {
        const uint2 t2 = *reinterpret_cast<const uint2*>((i < 4 ? k_rd0 : k_rd1) + 512 * (i & 3));
        kw[i] = make_uint4(t2.x, t2.y, 0u, 0u);
      } else {
        kw[i] = *reinterpret_cast<const uint4*>((i < 4 ? k_rd0 : k_rd1) + 1024 * (i & 3));
      }
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if constexpr (BITS == 2) {
        // the two pages' words of channel tile t side by side (one 64-bit shift unpacks both)
        const uint2 pr = make_uint2(v_rd[64 * t], v_rd[512 + 64 * t]);
        vw[t][0] = make_uint2(pr.x, pr.y);
        vw[t][1] = make_uint2(pr.y, 0u);
      } else {
        vw[t][0] = *reinterpret_cast<const uint2*>(v_rd + 128 * t);
        vw[t][1] = *reinterpret_cast<const uint2*>(v_rd + 1024 + 128 * t);
      }
    }
    // one metadata buffer: before the next group's copy lands there, this lane's metadata words to registers
    // (per token: the words of step 1; per channel: the alpha step's scale/zero pairs of positions Q0 + i,
    // i % 8 < 4) and the value scales and zeros to the side buffer
    uint32_t mkw[M1 ? 16 : 1];
    if constexpr (M1) {
      const uint16_t* ms0 = reinterpret_cast<const uint16_t*>(W.mst[0]);
      if constexpr (TOK) {
        const uint32_t* mw = reinterpret_cast<const uint32_t*>(ms0 + 256 * (c >> 3) + 2 * (c & 7));
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
          for (int j = 0; j < 4; ++j) mkw[4 * k + j] = mw[8 * k + 32 * j];
      } else {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          if ((i & 4) == 0) {
            const int ch = mf_key_channel(Q0 + i), j = 4 * (i >> 3) + (i & 3);
            mkw[j] = reinterpret_cast<const uint32_t*>(ms0)[ch >> 1];
            mkw[8 + j] = reinterpret_cast<const uint32_t*>(ms0 + D)[ch >> 1];
          }
        }
        reinterpret_cast<uint2*>(W.vsz)[lane] = reinterpret_cast<const uint2*>(ms0 + 2 * D)[lane];
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (has_next) {
      const int2 pn = make_int2(__builtin_amdgcn_readfirstlane(pv.x), __builtin_amdgcn_readfirstlane(pv.y));
      issue_m(pn, mb ^ 1);
      issue_k(pn);
      issue_v(pn);
      if (gi + 2 < g_end) pv = pair_v(gi + 2);
    }
    const uint16_t* ms = reinterpret_cast<const uint16_t*>(W.mst[mb]);
    // 1. per channel: key-side operand alpha = q~ s of head ah at positions Q0 + i, three limbs;
    //    per token: the group's token scales and zeros (tokens T(i, c) of the lane's page c / 8)
    float Ae[HPL], AZe[HPL];
    float tks[8], tkz[8], tvs[8], tvz[8];
    if constexpr (TOK) {
      // tokens 2 (c % 8) + 16 k + {0, 1} of page c / 8: one word per pair; K s, K z, V s, V z at 0, 64, 128, 192
      const uint32_t* mw = reinterpret_cast<const uint32_t*>(ms + 256 * (c >> 3) + 2 * (c & 7));
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t w0 = M1 ? mkw[4 * k] : mw[8 * k], w1 = M1 ? mkw[4 * k + 1] : mw[8 * k + 32];
        const uint32_t w2 = M1 ? mkw[4 * k + 2] : mw[8 * k + 64], w3 = M1 ? mkw[4 * k + 3] : mw[8 * k + 96];
        tks[k] = __uint_as_float(w0 << 16);
        tks[k + 4] = __uint_as_float(w0 & 0xffff0000u);
        tkz[k] = __uint_as_float(w1 << 16);
        tkz[k + 4] = __uint_as_float(w1 & 0xffff0000u);
        tvs[k] = __uint_as_float(w2 << 16);
        tvs[k + 4] = __uint_as_float(w2 & 0xffff0000u);
        tvz[k] = __uint_as_float(w3 << 16);
        tvz[k + 4] = __uint_as_float(w3 & 0xffff0000u);
      }
#pragma unroll
      for (int e = 0; e < HPL; ++e) {
        Ae[e] = At[e];
        AZe[e] = FSt[e];
      }
    } else {
      float al[NCH], zk[NCH];
      if constexpr (NCH >= 8 && BITS == 2) {
        // positions i and i + 4 (i % 8 < 4) are channels ch, ch + 1 with ch even: one word per pair
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          if ((i & 4) == 0) {
            const int ch = mf_key_channel(Q0 + i), j = 4 * (i >> 3) + (i & 3);
            const uint32_t sw = M1 ? mkw[j] : reinterpret_cast<const uint32_t*>(ms)[ch >> 1];
            const uint32_t zw = M1 ? mkw[8 + j] : reinterpret_cast<const uint32_t*>(ms + D)[ch >> 1];
            al[i] = qa[i] * __uint_as_float(sw << 16);
            al[i + 4] = qa[i + 4] * __uint_as_float(sw & 0xffff0000u);
            zk[i] = __uint_as_float(zw << 16);
            zk[i + 4] = __uint_as_float(zw & 0xffff0000u);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          const int ch = BITS == 2 ? mf_key_channel(Q0 + i) : mf_key_channel_c4(Q0 + i);
          al[i] = qa[i] * bf16_to_f32(ms[ch]);
          zk[i] = bf16_to_f32(ms[D + ch]);
        }
      }
      float zs;
      const float Ah = round_operand3<LPH, NCH, RS, true>(al, zk, S, a_rows, zs);
      const float AZh = zs;
#pragma unroll
      for (int e = 0; e < HPL; ++e) {
        Ae[e] = head_value(Ah, e);
        AZe[e] = head_value(AZh, e);
      }
    }
    wave_lds_sync();

    // 2. key products: 8 token tiles x 2 channel halves (at GQ 8 also for the top-limb tile)
    mf_i32x4 A[2][2];
    if constexpr (TOK) {
#pragma unroll
      for (int x = 0; x < 2; ++x) A[x][0] = At_op[x][0], A[x][1] = At_op[x][1];
    } else {
      load_op(A);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before the weights overwrite the plane
    }
    mf_i32x4 acc[8], accx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mf_i32x4 c0, c1;
      if constexpr (BITS == 2) {
        codes_i8_pair(kw[i].x, kw[i].y, c0, c1);
      } else {
        c0 = nibbles_i8(kw[i].x, kw[i].y);
        c1 = nibbles_i8(kw[i].z, kw[i].w);
      }
      acc[i] = mfma_i8x64(A[0][0], c0, zero4);
      acc[i] = mfma_i8x64(A[0][1], c1, acc[i]);
      if constexpr (GQ == 8) {
        accx[i] = mfma_i8x64(A[1][0], c0, zero4);
        accx[i] = mfma_i8x64(A[1][1], c1, accx[i]);
      }
    }

    // 3. per channel: logit = A val - AZ, the group maximum is that of the integer sums (A >= 0), weights
    //    u = rint(S 2^(A (val - val_max))); per token: logit_t = A s_t (val_t - z_t sum_c a_c), weights
    //    u_t = rint(S p_t s'_t / S') with S' the group's largest p_t s'_t of the head, their sums
    //    P = sum_t p_t and Z = sum_t u_t z'_t; weights as limbs at positions 8 c + i of the plane
    float mg[HPL], Sg[HPL], Pt[HPL], Zt[HPL];
#pragma unroll
    for (int e = 0; e < HPL; ++e) {
      float ew[8];
      if constexpr (TOK) {
        float lg[8];
        float lmx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          lg[i] = (Ae[e] * tks[i]) * fmaf(-tkz[i], AZe[e], (float)limbs3_sum<GQ>(acc[i], accx[i], e));
          lmx = fmaxf(lmx, lg[i]);
        }
        mg[e] = seg_reduce<16>(lmx, OpMax());
        float pw[8], wmx = 0.0f, ps = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float pp = __builtin_amdgcn_exp2f(lg[i] - mg[e]);
          ps += pp;
          pw[i] = pp * tvs[i];
          wmx = fmaxf(wmx, pw[i]);
        }
        Sg[e] = seg_reduce<16>(wmx, OpMax());
        Pt[e] = seg_sum<16>(ps);
        // below 2^-100 the group's value terms are beyond fp32's reach next to the others: weights 0
        const float r = Sg[e] > 0x1p-100f ? S * __builtin_amdgcn_rcpf(Sg[e]) : 0.0f;
        float zs = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          ew[i] = fmaf(pw[i], r, kRoundU);
          zs = fmaf(ew[i] - kRoundU, tvz[i], zs);
        }
        Zt[e] = seg_sum<16>(zs);
      } else {
        int v[8];
        int vmx = (int)0x80000000u;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          v[i] = limbs3_sum<GQ>(acc[i], accx[i], e);
          vmx = max(vmx, v[i]);
        }
        vmx = seg_max_i<16>(vmx);
        const float ref = Ae[e] * (float)vmx;
        mg[e] = ref - AZe[e];
#pragma unroll
        for (int i = 0; i < 8; ++i) ew[i] = fmaf(__builtin_amdgcn_exp2f(fmaf(Ae[e], (float)v[i], -ref)), S, kRoundU);
      }
      const int he = q4 * HPL + e;
      if (he < GQ) store_weights3<RS>(W.plane + (3 * he) * RS + 8 * c, ew);
    }
    wave_lds_sync();

    // 4. value products: 8 channel tiles x 2 pages, and the weight sums
    mf_i32x4 Wt[2][2];
    load_op(Wt);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before the next group's operand overwrites it
    mf_i32x4 accp = zero4, accpx = zero4;
    if constexpr (!TOK) {
      accp = mfma_i8x64(Wt[0][0], ones4, zero4);
      accp = mfma_i8x64(Wt[0][1], ones4, accp);
      if constexpr (GQ == 8) {
        accpx = mfma_i8x64(Wt[1][0], ones4, zero4);
        accpx = mfma_i8x64(Wt[1][1], ones4, accpx);
      }
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      mf_i32x4 c0, c1;
      if constexpr (BITS == 2) {
        codes_i8_pair(vw[t][0].x, vw[t][0].y, c0, c1);
      } else {
        c0 = nibbles_i8(vw[t][0].x, vw[t][0].y);
        c1 = nibbles_i8(vw[t][1].x, vw[t][1].y);
      }
      acc[t] = mfma_i8x64(Wt[0][0], c0, zero4);
      acc[t] = mfma_i8x64(Wt[0][1], c1, acc[t]);
      if constexpr (GQ == 8) {
        accx[t] = mfma_i8x64(Wt[1][0], c0, zero4);
        accx[t] = mfma_i8x64(Wt[1][1], c1, accx[t]);
      }
    }

    // 5. online-softmax update in the rotated value frame (per channel: o and l carry the weights' factor
    //    S; per token: the group adds (S' / S) (U_c - Z) to o and P to l)
#pragma unroll
    for (int e = 0; e < HPL; ++e) {
      const float mnew = fmax_raw(m[e], mg[e]);
      const float sc = __builtin_amdgcn_exp2f(m[e] - mnew);  // 0 before the first group (m = -inf)
      const float eg = __builtin_amdgcn_exp2f(mg[e] - mnew);
      if constexpr (TOK) {
        const float wg = eg * Sg[e] * (1.0f / S);
#pragma unroll
        for (int t = 0; t < 8; ++t)
          o[e][t] = fmaf(o[e][t], sc, wg * ((float)limbs3_sum<GQ>(acc[t], accx[t], e) - Zt[e]));
        l[e] = fmaf(l[e], sc, eg * Pt[e]);
        m[e] = mnew;
        continue;
      }
      const float Pf = (float)limbs3_sum<GQ>(accp, accpx, e);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int ch = c + 16 * t;
        // the value scales and zeros: the side buffer's two runs (one metadata buffer) or the metadata's second half
        const uint16_t* vsz = M1 ? reinterpret_cast<const uint16_t*>(W.vsz) : ms + 2 * D;
        const float sv = bf16_to_f32(vsz[ch]), zv = bf16_to_f32(vsz[D + ch]);
        const float Y = fmaf(-zv, Pf, (float)limbs3_sum<GQ>(acc[t], accx[t], e));
        o[e][t] = fmaf(eg * sv, Y, o[e][t] * sc);
      }
      l[e] = fmaf(eg, Pf, l[e] * sc);
      m[e] = mnew;
    }
    if constexpr (!M1) mb ^= 1;
    if (--left == 0 || !has_next) {  // uniform: the end of a chunk
      store_partial(gi / gpc);
      left = gpc;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// INT4 per-token chunk ([SAW] App. A.1 token-wise INT4, eq. 13-14) on the int8 matrix cores: the per-token
// INT2 unit's algebra (key-side operand = the rotated query, three limbs at full scale S = 1,000,000, once
// per walk; logit_t = A s_t (D_t - z_t sum_c a_c); weights u_t = rint(S p_t s'_t / S')) over page pairs
// (128 tokens) of 4-bit
// codes, each 32-bit code word two int8 vectors ((w >> 4n) & 0x0F0F0F0F).  Tokens past the length take no
// weight; a missing second page of a pair is the first again (read, never weighted).
//  - key k order (k = 64 sigma + 16 q + 4 d + b): channel 16 (2 q + sigma) + 8 (d / 2) + 2 b + d % 2, i.e.
//    lane q reads the 16 bytes 32 q + 16 sigma.. of a token row (channel c in byte c / 2, even c low);
//  - value k order (k = 64 kappa + 16 q + 4 d + b): token 64 kappa + 16 (2 (d / 2) + b / 2) + 4 q + 2 (b % 2)
//    + d % 2, i.e. lane q reads code words 2 q, 2 q + 1 of a channel row (token 16 j + 4 g + r in byte
//    8 g + 2 j + r / 2, even r low);
//  - key tile i, column c: token T(i, c) = 64 (c / 8) + 32 (c % 2) + 16 ((i / 2) % 2) + 4 ((c / 2) % 4) +
//    2 (i % 2) + i / 4, the token at value position 8 c + i.
// Key rows are staged with adjacent tokens swapped where bit 2 of the token is set (row t ^ ((t >> 2) & 1)),
// so that a tile's 16-byte operand reads use all LDS banks.
// ---------------------------------------------------------------------------------------------
// key k position -> channel (4-bit codes)
__host__ __device__ constexpr int mf_key_channel4(int Q) {
  return 16 * (2 * ((Q & 63) >> 4) + (Q >> 6)) + 8 * (((Q & 15) >> 2) >> 1) + 2 * (Q & 3) + (((Q & 15) >> 2) & 1);
}

template <int GQ, typename Lds>
__device__ void int4tok_unit_mfma(Lds& L, const DecodeArgs& a, int b, int h, int T, int c0, int c1) {
  constexpr int LG = HeadLog2<GQ>::v;
  constexpr int LPH = 64 >> LG;
  constexpr int NCH = 2 * GQ;
  constexpr int RPH = GQ == 8 ? 2 : 4;
  constexpr int HPL = GQ == 8 ? 2 : 1;
  constexpr int ROWS = MfmaWave<GQ, 512>::ROWS;
  constexpr int RS = MfmaWave<GQ, 512>::RSTRIDE;
  constexpr float S = Limb3<4>::S;
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int npages = (T + PAGE - 1) / PAGE;
  const int npairs = (npages + 1) / 2;
  // this wave walks chunks c0 .. c1 - 1 (an even number of pages each: page pairs pb .. pe - 1), storing a
  // partial per chunk
  const int ppc = g.gpc / 2;  // page pairs per chunk
  const int pb = c0 * ppc;
  int pe = c1 * ppc;
  if (pe > npairs) pe = npairs;
  if (2 * pe > g.max_pages + 1) pe = (g.max_pages + 1) / 2;          // never index past the page-table row
  MfmaWave<GQ, 512>& W = L.mf.w[wave];
  const int q4 = lane >> 4, c = lane & 15;

  if (lane < 32) reinterpret_cast<uint32_t*>(W.plane + ROWS * RS)[lane] = 0u;
  // A-operand rows (the INT2 unit's layout): (head, limb) pairs, at GQ 8 a second tile of top limbs
  const int rh = c / RPH, rl = c % RPH;
  const int prow = GQ == 8 ? 3 * rh + rl : ((rl < 3 && rh < GQ) ? 3 * rh + rl : ROWS);
  const int prow2 = rl == 0 ? 3 * rh + 2 : ROWS;
  const uint8_t* op_rd = W.plane + prow * RS + 16 * q4;
  const uint8_t* op_rd2 = W.plane + prow2 * RS + 16 * q4;
  auto load_op = [&](mf_i32x4 (&A)[2][2]) {
    A[0][0] = u4_i32x4(*reinterpret_cast<const uint4*>(op_rd));
    A[0][1] = u4_i32x4(*reinterpret_cast<const uint4*>(op_rd + 64));
    if constexpr (GQ == 8) {
      A[1][0] = u4_i32x4(*reinterpret_cast<const uint4*>(op_rd2));
      A[1][1] = u4_i32x4(*reinterpret_cast<const uint4*>(op_rd2 + 64));
    }
  };
  // key operand reads: tile i at staged row 64 (c / 8) + 32 (c % 2) + 4 ((c / 2) % 4) + (y ^ (i / 4)) plus
  // 16 ((i / 2) % 2) + 2 (i % 2), with y = (c / 2) % 2
  const int y = (c >> 1) & 1;
  const int krow = 64 * (c >> 3) + 32 * (c & 1) + 4 * ((c >> 1) & 3);
  const uint8_t* k_rd0 = reinterpret_cast<const uint8_t*>(W.kst) + 64 * (krow + y) + 16 * q4;
  const uint8_t* k_rd1 = reinterpret_cast<const uint8_t*>(W.kst) + 64 * (krow + (y ^ 1)) + 16 * q4;
  // value operand reads: channel c + 16 tau, code words 2 q4, 2 q4 + 1, page kappa
  const uint8_t* v_rd = reinterpret_cast<const uint8_t*>(W.vst) + 32 * c + 8 * q4;
  // this lane's tokens T(i, c) (pair-local), their metadata words: K (s, z) at (2 page) 64 + t, V at + 64
  const int tok0 = 64 * (c >> 3) + 32 * (c & 1) + 4 * ((c >> 1) & 3);
  const int ah = lane >> (6 - LG);
  const int Q0 = (lane & (LPH - 1)) * NCH;
  // copies: key slots 64 j + lane hold staged row 16 j + lane / 4, quarter lane % 4
  const uint32_t koff = (uint32_t)(64 * ((lane >> 2) ^ ((lane >> 4) & 1)) + 16 * (lane & 3));
  const uint32_t kst_a = lds_addr(W.kst), vst_a = lds_addr(W.vst);
  const uint32_t mst_a0 = lds_addr(W.mst[0]), mst_a1 = lds_addr(W.mst[1]);
  const uint8_t* pages = a.pages;
  const long long pbytes = g.page_bytes, hoff = (long long)h * g.head_bytes;
  auto page_of = [&](int idx) { return pages + pool_page(g, idx) * pbytes + hoff; };
  auto issue_m = [&](int2 p, int buf) {
    const uint8_t* src = (lane >= 32 ? page_of(p.y) : page_of(p.x)) + ((lane & 16) ? I4_VMETA_OFF : I4_KMETA_OFF) +
                         (lane & 15) * 16;
    dma16(buf ? mst_a1 : mst_a0, src);
  };
  auto issue_k = [&](int2 p) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      dma16_base(kst_a + 1024 * j, page_of(j < 4 ? p.x : p.y) + I4_K_OFF + 1024 * (j & 3), koff);
  };
  auto issue_v = [&](int2 p) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      dma16_base(vst_a + 1024 * j, page_of(j < 4 ? p.x : p.y) + I4_V_OFF + 1024 * (j & 3), lane * 16);
  };
  // page pairs (a missing second page is the first again): the first by scalar loads; afterwards a pair's
  // copies go out together with a vector load of the pair after it, which arrives with them
  const int32_t* ptr = a.page_table + (long long)b * g.max_pages;
  auto pages_of = [&](int i) {
    const int x = scalar_load_int(ptr + 2 * i);
    const int yy = 2 * i + 1 < npages ? scalar_load_int(ptr + 2 * i + 1) : x;
    return make_int2(x, yy);
  };
  auto pages_v = [&](int i) {
    const int x = ptr[2 * i];
    const int yy = 2 * i + 1 < npages ? ptr[2 * i + 1] : x;
    return make_int2(x, yy);
  };

  // 0. the key-side operand, once: the rotated query of head ah at positions Q0 + i, three limbs
  float At[HPL], FSt[HPL];
  mf_i32x4 Aq[2][2];
  {
    float qa[NCH], one[NCH];
    const float* q = a.qrot + ((long long)b * g.n_q + h * GQ + ah) * D;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      qa[i] = q[mf_key_channel4(Q0 + i)];
      one[i] = 1.0f;
    }
    float fs;
    const float Ah = round_operand3<LPH, NCH, RS>(qa, one, S, W.plane + (3 * ah) * RS + Q0, fs);
#pragma unroll
    for (int e = 0; e < HPL; ++e) {
      const int src = ((q4 * HPL + e) & (GQ - 1)) * LPH;
      At[e] = __shfl(Ah, src, 64);
      FSt[e] = __shfl(fs, src, 64);
    }
    wave_lds_sync();
    load_op(Aq);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before the first weights overwrite the plane
  }
  float m[HPL], l[HPL], o[HPL][8];
#pragma unroll
  for (int e = 0; e < HPL; ++e) {
    m[e] = -INFINITY;
    l[e] = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) o[e][t] = 0.0f;
  }
  int2 pv = make_int2(0, 0);
  int mb = 0;
  if (pb < pe) {
    const int2 p0 = pages_of(pb);
    issue_m(p0, 0);
    issue_k(p0);
    issue_v(p0);
    if (pb + 1 < pe) pv = pages_v(pb + 1);
  }
  // the partial of chunk ci, then a fresh softmax state; every partial a merge reads is written, chunks past
  // the length have none
  auto store_partial = [&](int ci) {
#pragma unroll
    for (int e = 0; e < HPL; ++e) {
      const int he = q4 * HPL + e;
      if (he < GQ) {
        float* part = a.partials + (((long long)b * g.n_q + h * GQ + he) * g.n_units + 1 + ci) * PART_STRIDE;
#pragma unroll
        for (int t = 0; t < 8; ++t) part[2 + c + 16 * t] = o[e][t];
        if (c == 0) {
          part[0] = m[e];
          part[1] = l[e];
        }
      }
      m[e] = -INFINITY;
      l[e] = 0.0f;
#pragma unroll
      for (int t = 0; t < 8; ++t) o[e][t] = 0.0f;
    }
  };
  const mf_i32x4 zero4 = {0, 0, 0, 0};
  int left = ppc;  // page pairs left in the current chunk
  for (int pi = pb; pi < pe; ++pi) {
    const bool has_next = pi + 1 < pe;  // uniform
    KVQ_WAIT_VM(0);  // this pair's metadata, key and value codes, and the next pair's pages
    wave_lds_sync();
    // 0. the pair's codes and the lane's token metadata to registers, then the next pair's copies
    uint4 kw[8];
    uint2 vw[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      kw[i] = *reinterpret_cast<const uint4*>((i < 4 ? k_rd0 : k_rd1) + 1024 * ((i >> 1) & 1) + 128 * (i & 1));
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      vw[t][0] = *reinterpret_cast<const uint2*>(v_rd + 512 * t);
      vw[t][1] = *reinterpret_cast<const uint2*>(v_rd + 4096 + 512 * t);
    }
    // the lane's tokens: K and V (scale, zero) words, validity
    const uint32_t* mw = reinterpret_cast<const uint32_t*>(W.mst[mb]) + 128 * (c >> 3);  // its page's K, then V
    float tks[8], tkz[8], tvs[8], tvz[8];
    bool ok[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = tok0 + 16 * ((i >> 1) & 1) + 2 * (i & 1) + (i >> 2);  // T(i, c)
      const uint32_t wk = mw[t & 63], wv = mw[64 + (t & 63)];
      ok[i] = pi * 128 + t < T;
      tks[i] = __uint_as_float(wk << 16);
      tkz[i] = __uint_as_float(wk & 0xffff0000u);
      // tokens past the length: no value scale or zero (their metadata may be anything)
      tvs[i] = ok[i] ? __uint_as_float(wv << 16) : 0.0f;
      tvz[i] = ok[i] ? __uint_as_float(wv & 0xffff0000u) : 0.0f;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (has_next) {
      const int2 pn = make_int2(__builtin_amdgcn_readfirstlane(pv.x), __builtin_amdgcn_readfirstlane(pv.y));
      issue_m(pn, mb ^ 1);
      issue_k(pn);
      issue_v(pn);
      if (pi + 2 < pe) pv = pages_v(pi + 2);
    }

    // 1. key products: 8 token tiles x 2 channel halves (at GQ 8 also for the top-limb tile)
    mf_i32x4 acc[8], accx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const mf_i32x4 c0 = nibbles_i8(kw[i].x, kw[i].y), c1 = nibbles_i8(kw[i].z, kw[i].w);
      acc[i] = mfma_i8x64(Aq[0][0], c0, zero4);
      acc[i] = mfma_i8x64(Aq[0][1], c1, acc[i]);
      if constexpr (GQ == 8) {
        accx[i] = mfma_i8x64(Aq[1][0], c0, zero4);
        accx[i] = mfma_i8x64(Aq[1][1], c1, accx[i]);
      }
    }

    // 2. logits, the pair's maximum, weights u_t = rint(S p_t s'_t / S'), P = sum p_t, Z = sum u_t z'_t
    float mg[HPL], Sg[HPL], Pt[HPL], Zt[HPL];
#pragma unroll
    for (int e = 0; e < HPL; ++e) {
      float lg[8];
      float lmx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = (At[e] * tks[i]) * fmaf(-tkz[i], FSt[e], (float)limbs3_sum<GQ>(acc[i], accx[i], e));
        lg[i] = ok[i] ? x : -INFINITY;
        lmx = fmaxf(lmx, lg[i]);
      }
      mg[e] = seg_reduce<16>(lmx, OpMax());  // finite: every pair has a token within the length
      float pw[8], wmx = 0.0f, ps = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pp = __builtin_amdgcn_exp2f(lg[i] - mg[e]);  // 0 for a token past the length
        ps += pp;
        pw[i] = pp * tvs[i];
        wmx = fmaxf(wmx, pw[i]);
      }
      Sg[e] = seg_reduce<16>(wmx, OpMax());
      Pt[e] = seg_sum<16>(ps);
      const float r = Sg[e] > 0x1p-100f ? S * __builtin_amdgcn_rcpf(Sg[e]) : 0.0f;
      float ew[8];
      float zs = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ew[i] = fmaf(pw[i], r, kRoundU);
        zs = fmaf(ew[i] - kRoundU, tvz[i], zs);
      }
      Zt[e] = seg_sum<16>(zs);
      const int he = q4 * HPL + e;
      if (he < GQ) store_weights3<RS>(W.plane + (3 * he) * RS + 8 * c, ew);
    }
    wave_lds_sync();

    // 3. value products: 8 channel tiles x 2 pages
    mf_i32x4 Wt[2][2];
    load_op(Wt);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before the next pair's weights overwrite them
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const mf_i32x4 c0 = nibbles_i8(vw[t][0].x, vw[t][0].y), c1 = nibbles_i8(vw[t][1].x, vw[t][1].y);
      acc[t] = mfma_i8x64(Wt[0][0], c0, zero4);
      acc[t] = mfma_i8x64(Wt[0][1], c1, acc[t]);
      if constexpr (GQ == 8) {
        accx[t] = mfma_i8x64(Wt[1][0], c0, zero4);
        accx[t] = mfma_i8x64(Wt[1][1], c1, accx[t]);
      }
    }

    // 4. online-softmax update in the rotated value frame: the pair adds (S' / S) (U_c - Z) and P
#pragma unroll
    for (int e = 0; e < HPL; ++e) {
      const float mnew = fmax_raw(m[e], mg[e]);
      const float sc = __builtin_amdgcn_exp2f(m[e] - mnew);  // 0 before the first pair (m = -inf)
      const float eg = __builtin_amdgcn_exp2f(mg[e] - mnew);
      const float wg = eg * Sg[e] * (1.0f / S);
#pragma unroll
      for (int t = 0; t < 8; ++t)
        o[e][t] = fmaf(o[e][t], sc, wg * ((float)limbs3_sum<GQ>(acc[t], accx[t], e) - Zt[e]));
      l[e] = fmaf(l[e], sc, eg * Pt[e]);
      m[e] = mnew;
    }
    mb ^= 1;
    if (--left == 0 || !has_next) {  // uniform: the end of a chunk
      store_partial(pi / ppc);
      left = ppc;
    }
  }
}

// One-dimensional split-K grid: the quantized-chunk work-groups, chunk-major (every sequence's first chunk
// work-groups, then every sequence's second, ...), and one band work-group per (sequence, kv head).  The hardware
// hands consecutive work-groups to the eight XCDs in turn, so every XCD gets the same mix of chunk positions
// (sequence-major, a chunk position would stay on one XCD, and the last chunks, which short sequences lack,
// would leave theirs idle).  When the launch fits the GPU in one round of work-groups the band work-groups
// come last (measured faster at batch 32 x 32k); when it takes several rounds they come first, so that they
// overlap the chunk walks instead of trailing them.  What a chunk work-group walks: splitk_chunk_wgs.
//
// Work-group i of the split-K grid: true for a band work-group (idx = its (sequence, kv head) pair), false
// for a chunk work-group (idx = its index among the chunk work-groups).
__device__ inline bool splitk_is_band(const Geo& g, int i, int& idx) {
  const int pairs = g.batch * g.n_kv, nw = splitk_chunk_wgs(g);
  if (g.band_first) {
    idx = i < pairs ? i : i - pairs;
    return i < pairs;
  }
  idx = i < nw ? i : i - nw;
  return i >= nw;
}
// fp32 decode: the unit (0 = band, u >= 1 = chunk u - 1), kv head and sequence of this work-group
__device__ inline void splitk_unit_of(const Geo& g, int& unit, int& h, int& b) {
  const int pairs = g.batch * g.n_kv;
  int idx;
  const bool band = splitk_is_band(g, blockIdx.x, idx);
  const int pair = band ? idx : idx % pairs;
  unit = band ? 0 : 1 + idx / pairs;
  h = pair % g.n_kv;
  b = pair / g.n_kv;
}
// Matrix-core launch of the grouped schemes.  Work-groups per CU, as the LDS allows (160 KB): 2-bit codes
// three (48.5 KB each up to GQ 4, 53.6 KB at GQ 8); 4-bit codes two up to GQ 4 (81 KB), one at GQ 8.
template <int GQ, bool TOK, int BITS>
__global__ __launch_bounds__(kThreads, GQ <= 4 ? (BITS == 2 ? 3 : 2) : (BITS == 2 ? 3 : 1)) void decode_mfma_kernel(DecodeArgs a) {
  __shared__ DecodeLds<GQ, BITS / 2, true> L;
  const Geo& g = a.g;
  int i;
  if (splitk_is_band(g, blockIdx.x, i)) {
    // GQ 8 fills half the matrix columns: the band on the matrix cores (measured 2.3x faster than the
    // vector band at 4 x 380 tokens); at GQ <= 4 the vector band is faster
    if constexpr (GQ == 8) band_unit_mfma<GQ>(L, a, i / g.n_kv, i % g.n_kv, a.seq_lens[i / g.n_kv]);
    else band_unit<GQ>(L, a, i / g.n_kv, i % g.n_kv, a.seq_lens[i / g.n_kv]);
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (g.balanced) {
    // the chunk size from the batch's lengths (every wave computes it), one chunk per work-group
    const int lane = threadIdx.x & 63;
    const int G = balanced_gpc(g, a.seq_lens, lane);
    if (i == 0 && threadIdx.x == 0) a.sched[0] = G;  // for the merge
    int b, quad, c;
    if (!balanced_wg(g, a.seq_lens, i, lane, G, b, quad, c)) return;  // uniform over the work-group
    int2_unit_mfma<GQ, TOK, BITS>(L, a, b, 4 * quad + wave, a.seq_lens[b], c, c + 1, G);
    return;
  }
  int b, h, c0, c1;
  const int first = wave_chunk_of(g, i, wave, b, h, c0, c1);
  const int T = a.seq_lens[b];
  int n_chunks = (n_groups_of(T, g.S0, g.W) + g.gpc - 1) / g.gpc;
  if (n_chunks > g.n_units - 1) n_chunks = g.n_units - 1;  // lengths beyond the launch bound are cut
  if (first >= n_chunks) return;                           // uniform over the work-group
  int2_unit_mfma<GQ, TOK, BITS>(L, a, b, h, T, c0, c1, g.gpc);
}

// Matrix-core INT4 per-token launch (page pairs; no band: the band work-groups store an empty partial).
template <int GQ>
__global__ __launch_bounds__(kThreads, GQ <= 4 ? 2 : 1) void decode_mfma4_kernel(DecodeArgs a) {
  __shared__ DecodeLds<GQ, 2, true> L;
  const Geo& g = a.g;
  int i;
  if (splitk_is_band(g, blockIdx.x, i)) {
    const int b = i / g.n_kv, h = i % g.n_kv;
    for (int e = threadIdx.x; e < GQ * PART_STRIDE; e += kThreads) {
      const int hh = e / PART_STRIDE, k = e % PART_STRIDE;
      float* part = a.partials + (((long long)b * g.n_q + h * GQ + hh) * g.n_units) * PART_STRIDE;
      part[k] = (k == 0) ? -INFINITY : 0.0f;
    }
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int b, h, c0, c1;
  const int first = wave_chunk_of(g, i, wave, b, h, c0, c1);
  const int T = a.seq_lens[b];
  int n_chunks = ((T + PAGE - 1) / PAGE + g.gpc - 1) / g.gpc;
  if (n_chunks > g.n_units - 1) n_chunks = g.n_units - 1;  // lengths beyond the launch bound are cut
  if (first >= n_chunks) return;                           // uniform over the work-group
  int4tok_unit_mfma<GQ>(L, a, b, h, T, c0, c1);
}

// fp32 decode (exact arithmetic on the codes; the cross-check of the matrix-core decode): the four waves of
// a work-group share a chunk and are combined in LDS.  INT2 per channel (groups) and INT4 per token (pages).
template <int GQ, int SCHEME>
__global__ __launch_bounds__(kThreads) void decode_f32_kernel(DecodeArgs a) {
  static_assert(SCHEME == KVQ_INT2_CHANNEL || SCHEME == KVQ_INT4_TOKEN, "fp32 decode schemes");
  __shared__ DecodeLds<GQ, 1> L;
  const Geo& g = a.g;
  int unit, h, b;
  splitk_unit_of(g, unit, h, b);
  const int T = a.seq_lens[b];
  constexpr bool grouped = is_grouped(SCHEME);
  int n_chunks;
  if (grouped) {
    const int ng = n_groups_of(T, g.S0, g.W);
    n_chunks = (ng + g.gpc - 1) / g.gpc;
  } else {
    n_chunks = ((T + PAGE - 1) / PAGE + g.gpc - 1) / g.gpc;
  }
  if (n_chunks > g.n_units - 1) n_chunks = g.n_units - 1;  // lengths beyond the launch bound are cut
  if (unit > n_chunks) return;
  if (unit == 0) {
    if constexpr (grouped) {
      band_unit<GQ>(L, a, b, h, T);
    } else {
      // no band: an empty partial
      for (int e = threadIdx.x; e < GQ * PART_STRIDE; e += kThreads) {
        const int hh = e / PART_STRIDE, k = e % PART_STRIDE;
        float* part = a.partials + (((long long)b * g.n_q + h * GQ + hh) * g.n_units) * PART_STRIDE;
        part[k] = (k == 0) ? -INFINITY : 0.0f;
      }
    }
  } else if constexpr (SCHEME == KVQ_INT2_CHANNEL) {
    int2_unit<GQ>(L, a, b, h, T, unit - 1);
  } else {
    int4_unit<GQ>(L, a, b, h, T, unit - 1);
  }
}

// ---------------------------------------------------------------------------------------------
// Query preparation ([SAW] §4.1 and [NOVA] App. B.5: the query rotated once per step): one work-group of 512
// threads per (kv head, query row): q~ = (q R_K) log2e/sqrt(128) for the quantized tokens (rotated frame) and
// q log2e/sqrt(128) for the bf16 band (original frame), both to the workspace.
// ---------------------------------------------------------------------------------------------
template <int GQ>
__global__ __launch_bounds__(512) void prep_kernel(DecodeArgs a) {
  __shared__ float qs[GQ][D];
  __shared__ float part[4][GQ][D];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int j = tid & (D - 1), qtr = tid >> 7;  // column j, quarter qtr of the 128 input channels
  const long long base = ((long long)b * a.g.n_q + h * GQ) * D;
  const float scale = LOG2E * kInvSqrt128;
  const bool dense = a.g.rotation == KVQ_ROT_DENSE;
  // this thread's 32 entries of column j of R_K, read together with the queries (one round trip)
  float rk[32];
  if (dense) {
#pragma unroll
    for (int i = 0; i < 32; ++i) rk[i] = a.rot_k[(qtr * 32 + i) * D + j];
  }
  for (int e = tid; e < GQ * D; e += 512) {
    const int hh = e / D, c = e % D;
    const float qv = a.q_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(a.q)[base + e])
                              : static_cast<const float*>(a.q)[base + e];
    a.qband[base + e] = qv * scale;
    qs[hh][c] = dense ? qv : qv * a.rot_k[c];
  }
  __syncthreads();
  if (dense) {
    float r[GQ];
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) r[hh] = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i)
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) r[hh] = fmaf(qs[hh][qtr * 32 + i], rk[i], r[hh]);
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) part[qtr][hh][j] = r[hh];
    __syncthreads();
    for (int e = tid; e < GQ * D; e += 512) {
      const int hh = e / D, c = e % D;
      a.qrot[base + e] = ((part[0][hh][c] + part[1][hh][c]) + (part[2][hh][c] + part[3][hh][c])) * scale;
    }
  } else {
    // randomized (block-diagonal) Hadamard: FWHT within blocks of h channels in LDS
    for (int hb = 1; hb < a.g.hblock; hb <<= 1) {
      float x[GQ / 4 + 1];
      int n = 0;
      for (int e = tid; e < GQ * D; e += 512) {
        const int hh = e / D, c = e % D;
        const float u = qs[hh][c], v = qs[hh][c ^ hb];
        x[n++] = (c & hb) ? (v - u) : (u + v);
      }
      __syncthreads();
      n = 0;
      for (int e = tid; e < GQ * D; e += 512) qs[e / D][e % D] = x[n++];
      __syncthreads();
    }
    const float hs = (float)a.g.hscale;
    for (int e = tid; e < GQ * D; e += 512) a.qrot[base + e] = qs[e / D][e % D] * hs * scale;
  }
}

// ---------------------------------------------------------------------------------------------
// Merge ([OSCAR] §3.4.5 step 4, the second kernel of the split decode; [NOVA] App. B.5): one work-group
// per (kv head, seq) for its GQ query heads, 256 threads per head up to 4 heads (or one work-group of
// 1024 threads per q head when the pairs are few).  Per head, the chunk
// partials (rotated value frame) are combined with their softmax weights 2^(m_u - M); the results are
// un-rotated by R_V^T, which the work-group reads once for all its heads (every element by one thread),
// combined with the band partial (original frame) and normalized.  The weighted sum over chunks spreads
// (channel quad, chunk slice) over the threads; each slice keeps a running maximum of its own, so the
// partials, the band partial and the R_V rows are all loaded before the first wait.
// ---------------------------------------------------------------------------------------------
// HPW: query heads per work-group (all GQ heads of a kv head when there are enough (seq, kv head)
// pairs to fill the chip, else one, so that long contexts with few sequences still spread their
// chunk partials over many work-groups).  One head per work-group takes 32 chunk slices (1024
// threads), so that the many chunks of a long context are read with four times the loads in flight.
template <int HPW>
struct MergeShape {
  static constexpr int SUB = HPW < 4 ? HPW : 4;     // sub-blocks, one head each at a time
  static constexpr int SL = HPW == 1 ? 32 : 8;      // chunk slices of a sub-block
  static constexpr int SUBT = (D / 4) * SL;         // threads of a sub-block: channel quads x slices
  static constexpr int NT = SUBT * SUB;             // threads
  static constexpr int PARTS = NT / D;              // channel ranges of the un-rotation
};

template <int GQ, int HPW>
__global__ __launch_bounds__(MergeShape<HPW>::NT) void merge_kernel(DecodeArgs a) {
  constexpr int SUB = MergeShape<HPW>::SUB, NT = MergeShape<HPW>::NT, PARTS = MergeShape<HPW>::PARTS;
  constexpr int kMergeSlices = MergeShape<HPW>::SL, SUBT = MergeShape<HPW>::SUBT;
  static_assert(NT <= 1024 && SUBT >= D, "work-group shape");
  constexpr int CPP = D / PARTS;  // channels per part of the dense un-rotation
  static_assert(HPW * D <= NT, "every thread owns at most one output element");
  __shared__ float Ms[HPW], Ls[HPW];
  __shared__ float4 osum[SUB][kMergeSlices][D / 4];
  __shared__ float sm[SUB][kMergeSlices], sl_sum[SUB][kMergeSlices];
  __shared__ float ob[HPW][D];
  __shared__ float un[PARTS][HPW][D];
  const Geo& g = a.g;
  const int b = blockIdx.y, tid = threadIdx.x;
  const long long q0 = (long long)b * g.n_q + (long long)blockIdx.x * HPW;  // first q head of this work-group
  auto part_of = [&](int hh) { return a.partials + (q0 + hh) * g.n_units * PART_STRIDE; };  // unit 0: band
  // The loads are issued before the first wait, so that a merge of up to eight chunks takes one memory
  // round trip rather than one per phase: this thread's band-partial element, its range of an R_V row
  // and the first chunk partial of its slice are read before the sequence length has arrived.
  const bool owns = tid < HPW * D;
  const int eh = tid / D, ec = tid % D;  // the output element (head, channel) this thread writes
  float band_m = -INFINITY, band_l = 0.0f, band_o = 0.0f;
  if (owns) {
    const float* bb = part_of(eh);
    band_m = bb[0];
    band_l = bb[1];
    band_o = bb[2 + ec];
  }
  const bool dense = !g.key_only && g.rotation == KVQ_ROT_DENSE;
  const int rj = tid & (D - 1), rpart = tid / D;  // dense un-rotation: row rj, channel range rpart
  float4 rrow[CPP / 4];
  if (dense) {
    const float4* row = reinterpret_cast<const float4*>(a.rot_v + rj * D + rpart * CPP);
#pragma unroll
    for (int i = 0; i < CPP / 4; ++i) rrow[i] = row[i];
  }
  const int n_max = g.n_units - 1;
  // balanced chunking: the chunk size the split-K launch chose (read with the first partials)
  int gb = 1;
  if (g.balanced) {
    gb = a.sched[0];
    if (gb < 1) gb = 1;
  }
  int n_chunks = 0, seq_len = 0;  // set on the first pass below, once the first partials are in flight

  // 1. per head: M = max_u m_u, L = sum_u 2^(m_u - M) l_u, o[c] = sum_u 2^(m_u - M) o_u[c].  Sub-block sb
  // takes heads sb, sb + SUB, ..; its thread (channel quad cq, slice sl) folds chunks u = sl + 1 + SL k into
  // a running (max, sum, o) of its own, and the slices are combined in LDS with their own maxima.
  const int sb = tid / SUBT, lt = tid % SUBT;
  const int cq = lt & (D / 4 - 1), sl = lt / (D / 4);
#pragma unroll 1
  for (int h0 = 0; h0 < HPW; h0 += SUB) {
    const int hh = h0 + sb;
    const float* base = part_of(hh);
    float mloc = -INFINITY, lloc = 0.0f;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    auto load = [&](int u, float& mu, float& lu, float2& o01, float2& o23) {
      const float* pu = base + u * PART_STRIDE;
      mu = pu[0];
      lu = pu[1];
      const float* o = pu + 2 + 4 * cq;  // 8-byte aligned: two float2 loads
      o01 = *reinterpret_cast<const float2*>(o);
      o23 = *reinterpret_cast<const float2*>(o + 2);
    };
    auto fold = [&](float mu, float lu, float2 o01, float2 o23) {
      const float mn = fmaxf(mloc, mu);
      const float sc = exp2_safe_diff(mloc, mn), w = exp2_safe_diff(mu, mn);
      acc.x = fmaf(w, o01.x, acc.x * sc);
      acc.y = fmaf(w, o01.y, acc.y * sc);
      acc.z = fmaf(w, o23.x, acc.z * sc);
      acc.w = fmaf(w, o23.y, acc.w * sc);
      lloc = fmaf(w, lu, lloc * sc);
      mloc = mn;
    };
    // the slice's first chunk is read without a branch (an existing unit, unit 0 when the launch has
    // no chunk units; it is dropped below when past the sequence's chunk count)
    float mu, lu;
    float2 o01, o23;
    const int u1 = 1 + sl;
    load(u1 <= n_max ? u1 : n_max, mu, lu, o01, o23);
    if (h0 == 0) {
      const int T = a.seq_lens[b];
      if (g.balanced) {
        n_chunks = (balanced_groups(g, T) + gb - 1) / gb;
      } else if (is_grouped(g.scheme)) {
        n_chunks = (n_groups_of(T, g.S0, g.W) + g.gpc - 1) / g.gpc;
      } else {
        n_chunks = ((T + PAGE - 1) / PAGE + g.gpc - 1) / g.gpc;
      }
      if (n_chunks > n_max) n_chunks = n_max;
      seq_len = T;
    }
    if (u1 <= n_chunks) fold(mu, lu, o01, o23);
#pragma unroll 4
    for (int u = u1 + kMergeSlices; u <= n_chunks; u += kMergeSlices) {
      load(u, mu, lu, o01, o23);
      fold(mu, lu, o01, o23);
    }
    osum[sb][sl][cq] = acc;
    if (cq == 0) {
      sm[sb][sl] = mloc;
      sl_sum[sb][sl] = lloc;
    }
    __syncthreads();
    if (lt < D) {
      float M = -INFINITY;
#pragma unroll
      for (int s2 = 0; s2 < kMergeSlices; ++s2) M = fmaxf(M, sm[sb][s2]);
      const int k = lt & 3;
      float v = 0.0f, L = 0.0f;
#pragma unroll
      for (int s2 = 0; s2 < kMergeSlices; ++s2) {
        const float w = exp2_safe_diff(sm[sb][s2], M);
        const float4 t = osum[sb][s2][lt >> 2];
        v = fmaf(w, k == 0 ? t.x : k == 1 ? t.y : k == 2 ? t.z : t.w, v);
        L = fmaf(w, sl_sum[sb][s2], L);
      }
      ob[hh][lt] = v;
      if (lt == 0) {
        Ms[hh] = M;
        Ls[hh] = L;
      }
    }
    __syncthreads();
  }
  // 2. un-rotate every head: o_j = sum_c ob[c] R_V[j][c] (dense: thread (j, part) holds the part-th
  // range of row j of R_V, applied to all heads), the randomized Hadamard's inverse, or nothing under
  // key-only rotation
  if (g.key_only) {
    for (int e = tid; e < HPW * D; e += NT) {
      un[0][e / D][e % D] = ob[e / D][e % D];
#pragma unroll
      for (int p = 1; p < PARTS; ++p) un[p][e / D][e % D] = 0.0f;
    }
  } else if (dense) {
    float s0[HPW], s1[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) s0[hh] = s1[hh] = 0.0f;
#pragma unroll
    for (int i = 0; i < CPP / 4; ++i) {
      const float4 r = rrow[i];
      const int c = rpart * CPP + 4 * i;
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        s0[hh] = fmaf(ob[hh][c], r.x, s0[hh]);
        s1[hh] = fmaf(ob[hh][c + 1], r.y, s1[hh]);
        s0[hh] = fmaf(ob[hh][c + 2], r.z, s0[hh]);
        s1[hh] = fmaf(ob[hh][c + 3], r.w, s1[hh]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) un[rpart][hh][rj] = s0[hh] + s1[hh];
  } else {
    // (ob H_blk) * sign / sqrt(h): FWHT within blocks of h channels in LDS, all heads at once
    for (int hb = 1; hb < g.hblock; hb <<= 1) {
      float x[(HPW * D + NT - 1) / NT];
      int n = 0;
      for (int e = tid; e < HPW * D; e += NT) {
        const int hh = e / D, c = e % D;
        x[n++] = (c & hb) ? (ob[hh][c ^ hb] - ob[hh][c]) : (ob[hh][c] + ob[hh][c ^ hb]);
      }
      __syncthreads();
      n = 0;
      for (int e = tid; e < HPW * D; e += NT) ob[e / D][e % D] = x[n++];
      __syncthreads();
    }
    for (int e = tid; e < HPW * D; e += NT) {
      un[0][e / D][e % D] = ob[e / D][e % D] * a.rot_v[e % D] * (float)g.hscale;
#pragma unroll
      for (int p = 1; p < PARTS; ++p) un[p][e / D][e % D] = 0.0f;
    }
  }
  __syncthreads();
  // 3. combine with the band partial (unit 0, original frame) and normalize
  if (owns) {
    const float M = Ms[eh];
    const float mb = (seq_len > 0) ? band_m : -INFINITY;
    const float Mf = fmaxf(M, mb);
    float res = 0.0f;
    if (Mf != -INFINITY) {
      float o = 0.0f;
#pragma unroll
      for (int p = 0; p < PARTS; ++p) o += un[p][eh][ec];
      const float si = exp2_safe_diff(M, Mf), sb2 = exp2_safe_diff(mb, Mf);
      const float num = o * si + (mb == -INFINITY ? 0.0f : band_o * sb2);
      const float den = Ls[eh] * si + (mb == -INFINITY ? 0.0f : band_l * sb2);
      res = num / den;
    }
    a.out[(q0 + eh) * D + ec] = res;
  }
}

template <int GQ>
hipError_t launch_gq(const DecodeArgs& a, int stages, hipStream_t s, hipEvent_t split_begin, hipEvent_t split_end) {
  const Geo& g = a.g;
  if (stages & KVQ_STAGE_QPREP) hipLaunchKernelGGL(prep_kernel<GQ>, dim3(g.n_kv, g.batch), dim3(512), 0, s, a);
  if (stages & KVQ_STAGE_SPLITK) {
    // matrix-core decode: a wave per chunk, four chunks per work-group; fp32 decode: a chunk per work-group.
    // With events, the dispatch itself records them at the kernel's start and end (hipExtLaunchKernel).
    const dim3 grid(splitk_wgs(g)), block(kThreads);
    auto launch = [&](auto kernel) {
      if (split_begin) hipExtLaunchKernelGGL(kernel, grid, block, 0, s, split_begin, split_end, 0, a);
      else hipLaunchKernelGGL(kernel, grid, block, 0, s, a);
    };
    if (a.impl == KVQ_DECODE_MFMA) {
      if (g.scheme == KVQ_INT4_CHANNEL) launch(decode_mfma_kernel<GQ, false, 4>);
      else if (g.scheme == KVQ_INT2_TOKEN) launch(decode_mfma_kernel<GQ, true, 2>);
      else if (g.scheme == KVQ_INT2_CHANNEL) launch(decode_mfma_kernel<GQ, false, 2>);
      else launch(decode_mfma4_kernel<GQ>);
    } else {
      // the API admits the fp32 decode for these two schemes only
      if (g.scheme == KVQ_INT2_CHANNEL) launch(decode_f32_kernel<GQ, KVQ_INT2_CHANNEL>);
      else if (g.scheme == KVQ_INT4_TOKEN) launch(decode_f32_kernel<GQ, KVQ_INT4_TOKEN>);
      else return hipErrorInvalidValue;
    }
  }
  if (stages & KVQ_STAGE_MERGE) {
    if (g.batch * g.n_kv >= 128)
      hipLaunchKernelGGL((merge_kernel<GQ, GQ>), dim3(g.n_kv, g.batch), dim3(MergeShape<GQ>::NT), 0, s, a);
    else
      hipLaunchKernelGGL((merge_kernel<GQ, 1>), dim3(g.n_q, g.batch), dim3(MergeShape<1>::NT), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qprep_rows(const DecodeArgs& a, int rows, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid(a.g.n_kv, rows);
  switch (a.g.gq) {
    case 1: hipLaunchKernelGGL(prep_kernel<1>, grid, dim3(512), 0, s, a); break;
    case 2: hipLaunchKernelGGL(prep_kernel<2>, grid, dim3(512), 0, s, a); break;
    case 4: hipLaunchKernelGGL(prep_kernel<4>, grid, dim3(512), 0, s, a); break;
    case 8: hipLaunchKernelGGL(prep_kernel<8>, grid, dim3(512), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int stages, hipStream_t s, hipEvent_t split_begin, hipEvent_t split_end) {
  switch (a.g.gq) {
    case 1: return launch_gq<1>(a, stages, s, split_begin, split_end);
    case 2: return launch_gq<2>(a, stages, s, split_begin, split_end);
    case 4: return launch_gq<4>(a, stages, s, split_begin, split_end);
    case 8: return launch_gq<8>(a, stages, s, split_begin, split_end);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
