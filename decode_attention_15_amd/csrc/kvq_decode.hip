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

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr float kInvSqrt128 = 0.08838834764831845f;
// Full scale of the 16-bit key-side operand and of the value-side softmax weights in the integer-dot
// decode: both split into two signed bytes 256 hi + lo, so |x| <= 32639 (hi = (x + 128) >> 8 <= 127).
constexpr float kAScale = 32639.0f;
constexpr float kPScale = 32511.0f;
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

// ---- 64-lane reductions with DPP.  Steps: quad xor 1, quad xor 2, half-row mirror, row mirror (every
// lane then holds its 16-lane row's result), row broadcast 15 into rows 1 and 3, row broadcast 31 into
// rows 2 and 3; lane 63 ends with the whole wave's result, which is returned to every lane (uniform).
// The whole wave must be active.
#define KVQ_DPP(old, v, ctrl, rmask) __builtin_amdgcn_update_dpp((old), (v), (ctrl), (rmask), 0xF, false)

template <typename Op>
__device__ inline int wave_reduce_bits(int v, int ident, Op op) {
  v = op(v, KVQ_DPP(ident, v, 0xB1, 0xF));   // quad_perm [1,0,3,2]
  v = op(v, KVQ_DPP(ident, v, 0x4E, 0xF));   // quad_perm [2,3,0,1]
  v = op(v, KVQ_DPP(ident, v, 0x141, 0xF));  // row_half_mirror
  v = op(v, KVQ_DPP(ident, v, 0x140, 0xF));  // row_mirror
  v = op(v, KVQ_DPP(ident, v, 0x142, 0xA));  // row_bcast15 -> rows 1, 3
  v = op(v, KVQ_DPP(ident, v, 0x143, 0xC));  // row_bcast31 -> rows 2, 3
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ inline float wave_max_u(float x) {
  return __int_as_float(wave_reduce_bits(__float_as_int(x), __float_as_int(-INFINITY), [](int a, int b) {
    return __float_as_int(fmaxf(__int_as_float(a), __int_as_float(b)));
  }));
}

__device__ inline float wave_sum_u(float x) {
  return __int_as_float(wave_reduce_bits(__float_as_int(x), 0, [](int a, int b) {
    return __float_as_int(__int_as_float(a) + __int_as_float(b));
  }));
}

__device__ inline uint32_t wave_sum_u32(uint32_t x) {
  return (uint32_t)wave_reduce_bits((int)x, 0, [](int a, int b) { return (int)((uint32_t)a + (uint32_t)b); });
}

// ---------------------------------------------------------------------------------------------
// Query preparation: q~ = (q R_K) * log2e/sqrt(128) for quantized tokens (rotated frame), and
// q * log2e/sqrt(128) for the bf16 band (original frame).
// ---------------------------------------------------------------------------------------------
template <int GQ>
__global__ __launch_bounds__(512) void qprep_kernel(DecodeArgs a) {
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
// Split-K decode, vector ALU.  Work-group (unit, kv head, seq): unit 0 = bf16 band (sink + tail),
// unit u >= 1 = quantized chunk u-1.  Each of the 4 waves walks its own groups/pages with an
// online softmax; the waves are merged in LDS and one partial (m, l, o[128]) per q head written.
// ---------------------------------------------------------------------------------------------
// Per-wave LDS of the matrix-core INT2 unit: the key, then the value codes of a group (one 4 KB buffer),
// the metadata of two groups (double-buffered, 1 KB each), and the two operand planes it builds per group,
// each with rows
// (head, limb) of 128 bytes in k order (stride 144: consecutive rows start in different banks) and a last
// row that stays zero for the matrix rows no head fills.
template <int GQ, int KU = 256>
struct MfmaWave {
  static constexpr int ROWS = 2 * GQ;
  static constexpr int RSTRIDE = 144;
  uint4 kst[KU];  // 4 KB (2-bit codes of a group) or 8 KB (4-bit codes of a page pair)
  uint4 mst[2][64];
  uint8_t aplane[(ROWS + 1) * RSTRIDE];
  uint8_t wplane[(ROWS + 1) * RSTRIDE];
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
    struct {                     // band unit, fp32 INT2 path, INT4 path
      float qband[GQ][D];
      float alpha[4][GQ][D];     // per wave: alpha (INT2) / rotated query (INT4)
      float p[4][GQ][D];         // per wave: softmax numerators of the current group/page
    } f;
    struct {                     // 16-bit INT2 path
      uint8_t abytes[4][GQ * 256];  // per wave: key-side operand words [head][limb][32]
      uint8_t pbytes[4][GQ * 256];  // per wave: value-side operand words [head][limb][32]
      uint4 vstage[4][256 * STG];   // per wave: key, then value codes of the current group (both pages)
      uint4 mstage[4][64];          // per wave: key and value scales/zeros of a group (nibble-digit path)
    } d;
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

// Partial of one wave's own chunk (wave chunks): no combination with the other waves of the work-group.
template <int GQ>
__device__ void store_wave_partial(const DecodeArgs& a, int b, int h, int unit, int lane, const float (&m)[GQ],
                                   const float (&l)[GQ], const float (&o)[GQ][2], int c0, int c1) {
  const Geo& g = a.g;
#pragma unroll
  for (int hh = 0; hh < GQ; ++hh) {
    float* part = a.partials + (((long long)b * g.n_q + h * GQ + hh) * g.n_units + unit) * PART_STRIDE;
    part[2 + c0] = o[hh][0];
    part[2 + c1] = o[hh][1];
    if (lane == 0) {
      part[0] = m[hh];
      part[1] = l[hh];
    }
  }
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

template <int GQ, typename Lds>
__device__ void band_unit(Lds& L, const DecodeArgs& a, int b, int h, int T) {
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the value rows' slots are scalar
  for (int e = tid; e < GQ * D; e += kThreads)
    L.f.qband[e / D][e % D] = a.qband[((long long)b * g.n_q + h * GQ + e / D) * D + e % D];
  __syncthreads();
  const int ng = n_groups_of(T, g.S0, g.W);
  const int n_sink = T < g.S0 ? T : g.S0;
  const int tail0 = g.S0 + GROUP * ng;
  const int n_tail = T > tail0 ? T - tail0 : 0;
  const int nb = n_sink + n_tail;
  const uint16_t* band = a.band + ((long long)b * g.n_kv + h) * g.slots * 256;
  float m[GQ], l[GQ], o[GQ][2];
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
  for (int blk = wave; blk * 64 < nb; blk += 4) {
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
          for (int hh = 0; hh < GQ; ++hh) lg[hh] += L.f.qband[hh][c] * k0 + L.f.qband[hh][c + 1] * k1;
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      const float x = valid ? lg[hh] : -INFINITY;
      float mnew;
      softmax_update<GQ>(m, l, o, hh, wave_max(x), mnew);
      const float p = valid ? exp2f(x - mnew) : 0.0f;
      L.f.p[wave][hh][lane] = p;
      l[hh] += wave_sum(p);
    }
    wave_lds_sync();
    const int nk = (nb - blk * 64) < 64 ? (nb - blk * 64) : 64;
    // value rows (channels 2 lane, 2 lane + 1) 16 tokens at a time, the next 16 in flight while these are
    // summed, so that the block costs about one memory latency rather than one per batch
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
          const float p = L.f.p[wave][hh][k8 + q];
          o[hh][0] += p * v0;
          o[hh][1] += p * v1;
        }
      }
    }
    wave_lds_sync();
  }
  combine_and_store<GQ>(L, a, b, h, 0, wave, lane, m, l, o, 2 * lane, 2 * lane + 1);
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
    const uint8_t* pg[2] = {a.pages + (long long)pt[2 * gi] * g.page_bytes + hoff,
                            a.pages + (long long)pt[2 * gi + 1] * g.page_bytes + hoff};
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
// Cross-lane reductions used by the 16-bit INT2 decode.
// seg_reduce<N>: reduce within aligned segments of N lanes (N = 8..64); every lane of a segment gets the
// segment's result.  Pairings: quad xor 1, quad xor 2, half-row mirror, row mirror (DPP), then xor 16
// and xor 32 (cross-row exchanges).
// heads_allreduce<GQ>: GQ values per lane (one per head) reduced over all 64 lanes.  The first log2(GQ)
// steps exchange half of the remaining values with the lane across bit 5, 4, 3 (each lane keeps the
// heads whose index bits match its own lane bits), then the one remaining value is reduced within its
// segment; head h ends in lane h << (6 - log2 GQ) and is read from there (uniform result).
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

// Signed 4-way byte dot product with a zero accumulator (VOP3P form: no register to clear first).
__device__ inline int sdot4_z(uint32_t a, uint32_t b) {
  int r;
  asm("v_dot4_i32_i8 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

template <int GQ>
struct HeadLog2 {
  static constexpr int v = GQ == 1 ? 0 : GQ == 2 ? 1 : GQ == 4 ? 2 : 3;
};

__device__ inline float xor_exchange(float x, int bit) {
  if (bit == 3) return KVQ_MOVDPP(x, 0x128);  // row_ror:8 == lane xor 8 within a row
  return __shfl_xor(x, 1 << bit, 64);
}

template <int GQ, typename Op>
__device__ inline void heads_allreduce(const float (&v)[GQ], Op op, int lane, float (&out)[GQ]) {
  constexpr int LG = HeadLog2<GQ>::v;
  float cur[GQ];
#pragma unroll
  for (int i = 0; i < GQ; ++i) cur[i] = v[i];
#pragma unroll
  for (int s = 0; s < LG; ++s) {
    const int bit = 5 - s;
    const int half = GQ >> (s + 1);
#pragma unroll
    for (int i = 0; i < half; ++i) {
      if (bit >= 4) {
        // permlane swap of (cur[i], cur[half + i]) across lane bit `bit`: the first result holds cur[i] of
        // this lane (bit clear) or cur[half + i] of the partner (bit set), the second the other half; their
        // combination is head i over the lane pair where the bit is clear, head half + i where it is set
        const auto r = bit == 5 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(cur[i]),
                                                                   __float_as_uint(cur[half + i]), false, false)
                                : __builtin_amdgcn_permlane16_swap(__float_as_uint(cur[i]),
                                                                   __float_as_uint(cur[half + i]), false, false);
        cur[i] = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
      } else {
        const bool up = (lane >> bit) & 1;
        const float send = up ? cur[i] : cur[half + i];
        const float keep = up ? cur[half + i] : cur[i];
        cur[i] = op(keep, xor_exchange(send, bit));
      }
    }
  }
  const float x = seg_reduce<(64 >> LG)>(cur[0], op);
#pragma unroll
  for (int hh = 0; hh < GQ; ++hh)
    out[hh] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), hh << (6 - LG)));
}

struct OpMax {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct OpAdd {
  __device__ float operator()(float a, float b) const { return a + b; }
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

// heads_allreduce over integers (max) or floats (sum) with the folded segment steps.
template <int GQ, typename T, typename Op, typename Seg>
__device__ inline void heads_allreduce_fast(const T (&v)[GQ], Op op, Seg seg, int lane, T (&out)[GQ]) {
  constexpr int LG = HeadLog2<GQ>::v;
  T cur[GQ];
#pragma unroll
  for (int i = 0; i < GQ; ++i) cur[i] = v[i];
#pragma unroll
  for (int s = 0; s < LG; ++s) {
    const int bit = 5 - s;
    const int half = GQ >> (s + 1);
#pragma unroll
    for (int i = 0; i < half; ++i) {
      if (bit >= 4) {
        const auto r = bit == 5 ? __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, cur[i]),
                                                                   __builtin_bit_cast(uint32_t, cur[half + i]), false, false)
                                : __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, cur[i]),
                                                                   __builtin_bit_cast(uint32_t, cur[half + i]), false, false);
        // copy the pair's elements out before reinterpreting them: a bit_cast of the element expressions
        // themselves reads the first element twice with this compiler
        const uint32_t r0 = r[0], r1 = r[1];
        cur[i] = op(__builtin_bit_cast(T, r0), __builtin_bit_cast(T, r1));
      } else {  // bit 3: lane xor 8 within a row
        const bool up = (lane >> bit) & 1;
        const T send = up ? cur[i] : cur[half + i];
        const T keep = up ? cur[half + i] : cur[i];
        cur[i] = op(keep, __builtin_bit_cast(T, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, send), 0x128, 0xF, 0xF, false)));
      }
    }
  }
  const T x = seg(cur[0]);
#pragma unroll
  for (int hh = 0; hh < GQ; ++hh)
    out[hh] = __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), hh << (6 - LG)));
}

// max of two floats without the sNaN quieting that fmaxf adds for operands of unknown origin
__device__ inline float fmax_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// ---------------------------------------------------------------------------------------------
// INT2 chunk, 16-bit fixed point on the 4-way byte dot product (v_dot4).  Same algebra as
// int2_unit, with the two per-group operands quantized to 16 bits:
//   - alpha_{h,c} = q~_{h,c} s_c is rounded to an integer a_{h,c} = rint(alpha * 32639 / max_c |alpha|)
//     (per group and head), so that logit_t = A_h (sum_c a_{h,c} code_{t,c} - sum_c a_{h,c} z_c) with
//     A_h = max|alpha| / 32639; a = 256 hi + lo with signed bytes hi, lo, two signed dot4 per 4 channels.
//   - p_t = 2^(logit_t - max_group) in (0, 1] is rounded to u_t = rint(32511 p_t), u = 256 hi + lo with
//     signed bytes, two signed dot4 per 4 tokens of a channel; the group's output and weight are
//     2^(max_group - m) / 32511 times s_c (sum_t u_t code_{t,c} - z_c sum_t u_t) and sum_t u_t.
//     (Signed dot4 has a tied-accumulator form with no wait state between dependent issues.)
// Lane roles.  Keys: tokens lane of the group's even and odd page.  Values: channels lane, lane + 64.
// alpha: lane handles head lane >> (6 - log2 GQ) and 2 GQ consecutive channels of it, so that the per-head
// maxima and sums are segment reductions.  The integer operands of a group are exchanged through per-wave
// LDS bytes laid out so that one 16-byte read gives the words that pair with the four byte-lanes of one
// 32-bit code word:
//   K code word m of a token holds channels 16m + 4j + k in byte j, bits 2k; (w >> 2k) & 0x03030303 has
//   channel 16m + 4j + k in byte j, so alpha word (m, k) holds channel 16m + 4j + k in byte j;
//   V code word g of a channel holds token 16j + 4g + r in byte j, bits 2r, so p word (page, g, k) holds
//   token 16j + 4g + k of that page in byte j.
// ---------------------------------------------------------------------------------------------
template <int GQ, typename Lds>
__device__ void int2_unit_dot16(Lds& L, const DecodeArgs& a, int b, int h, int T, int chunk) {
  constexpr int LG = HeadLog2<GQ>::v;
  constexpr int LPH = 64 >> LG;   // lanes per head in the alpha step
  constexpr int NCH = 2 * GQ;     // channels per lane in the alpha step
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ng = n_groups_of(T, g.S0, g.W);
  const int g_begin = chunk * g.gpc;
  int g_end = (g_begin + g.gpc) < ng ? (g_begin + g.gpc) : ng;
  if (g_end > g.max_pages / 2) g_end = g.max_pages / 2;  // never index past the page-table row
  const int c0 = lane, c1 = lane + 64;
  const int ah = lane >> (6 - LG);         // head of this lane in the alpha step
  const int ac0 = (lane & (LPH - 1)) * NCH;  // its first channel
  float qa[NCH];
  {
    const float* q = a.qrot + ((long long)b * g.n_q + h * GQ + ah) * D + ac0;
#pragma unroll
    for (int i = 0; i < NCH; ++i) qa[i] = q[i];
  }
  float m[GQ], l[GQ], o[GQ][2];
#pragma unroll
  for (int hh = 0; hh < GQ; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.0f;
    o[hh][0] = o[hh][1] = 0.0f;
  }
  // per-wave operand bytes: [head][limb lo, hi][32 words]
  uint8_t* abytes = L.d.abytes[wave];
  uint8_t* pbytes = L.d.pbytes[wave];
  uint4* vst = L.d.vstage[wave];
  uint8_t* alo = abytes + ah * 256;
  uint8_t* ahi = alo + 128;
  const int pb0 = ((((lane >> 2) & 3) * 4 + (lane & 3)) << 2) + (lane >> 4);  // token lane of the even page
  const int pb1 = pb0 + 64;                                                    // token lane of the odd page
  // the page table is read-only here: scalar loads, the next group's entries one iteration ahead
  const int2* pt = reinterpret_cast<const int2*>(a.page_table + (long long)b * g.max_pages);
  const long long hoff = (long long)h * I2_HEAD_BYTES;
  int2 pnext = make_int2(0, 0);
  if (g_begin + wave < g_end) pnext = scalar_load_int2(pt + g_begin + wave);
  for (int gi = g_begin + wave; gi < g_end; gi += 4) {
    const int2 pcur = pnext;
    if (gi + 4 < g_end) pnext = scalar_load_int2(pt + gi + 4);
    const uint8_t* pg0 = a.pages + (long long)pcur.x * g.page_bytes + hoff;
    const uint8_t* pg1 = a.pages + (long long)pcur.y * g.page_bytes + hoff;
    const uint4 k00 = reinterpret_cast<const uint4*>(pg0 + I2_K_OFF + lane * 32)[0];
    const uint4 k01 = reinterpret_cast<const uint4*>(pg0 + I2_K_OFF + lane * 32)[1];
    const uint4 k10 = reinterpret_cast<const uint4*>(pg1 + I2_K_OFF + lane * 32)[0];
    const uint4 k11 = reinterpret_cast<const uint4*>(pg1 + I2_K_OFF + lane * 32)[1];
    // value codes go straight to LDS (no registers held while in flight): 1 KB per instruction,
    // lane i's 16 bytes at vst + 64 j + i; vst[64 pp' + c'] = row of channel c' (+64 for j odd) of page pp
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds(
          (__attribute__((address_space(1))) void*)((j < 2 ? pg0 : pg1) + I2_V_OFF + (j & 1) * 1024 + lane * 16),
          (__attribute__((address_space(3))) void*)(vst + 64 * j), 16, 0, 0);
    const uint32_t* kmeta = reinterpret_cast<const uint32_t*>(pg0 + I2_META_OFF);
    uint32_t skw[NCH / 2], zkw[NCH / 2];
#pragma unroll
    for (int i = 0; i < NCH / 2; ++i) {
      skw[i] = kmeta[ac0 / 2 + i];
      zkw[i] = kmeta[(D + ac0) / 2 + i];
    }
    const uint16_t* vm = reinterpret_cast<const uint16_t*>(pg1 + I2_META_OFF);
    const float sv0 = bf16_to_f32(vm[c0]), sv1 = bf16_to_f32(vm[c1]);
    const float zv0 = bf16_to_f32(vm[D + c0]), zv1 = bf16_to_f32(vm[D + c1]);

    // 1. alpha of this group for head ah, channels ac0.., 16-bit, as byte limbs in LDS
    float A[GQ], AZ[GQ];
    {
      float al[NCH];
      float amx = 0.0f;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const uint32_t w = skw[i >> 1];
        al[i] = qa[i] * __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
        amx = fmaxf(amx, fabsf(al[i]));
      }
      amx = seg_reduce<LPH>(amx, OpMax());
      const float inv = amx > 0.0f ? kAScale / amx : 0.0f;
      int ai[NCH];
      float zs = 0.0f;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        ai[i] = (int)rintf(al[i] * inv);
        const uint32_t w = zkw[i >> 1];
        zs = fmaf((float)ai[i], __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16)), zs);
      }
      zs = seg_reduce<LPH>(zs, OpAdd());
      const float Ah = amx * (1.0f / kAScale);
      const float AZh = Ah * zs;
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
        A[hh] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Ah), hh * LPH));
        AZ[hh] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(AZh), hh * LPH));
      }
      // channel c -> alpha word (c >> 4) * 4 + (c & 3), byte (c >> 2) & 3
      if constexpr (NCH == 16) {
        // channels 16r .. 16r+15: word r*4 + k holds channels 16r + 4j + k in byte j
        uint32_t wl[4], wh[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          wl[k] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(ai[12 + k], ai[8 + k], 0x0c0c0400u),
                                        __builtin_amdgcn_perm(ai[4 + k], ai[k], 0x0c0c0400u), 0x05040100u);
          const int h0 = (ai[k] + 128) >> 8, h1 = (ai[4 + k] + 128) >> 8, h2 = (ai[8 + k] + 128) >> 8,
                    h3 = (ai[12 + k] + 128) >> 8;
          wh[k] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(h3, h2, 0x0c0c0400u),
                                        __builtin_amdgcn_perm(h1, h0, 0x0c0c0400u), 0x05040100u);
        }
        *reinterpret_cast<uint4*>(alo + ac0) = make_uint4(wl[0], wl[1], wl[2], wl[3]);
        *reinterpret_cast<uint4*>(ahi + ac0) = make_uint4(wh[0], wh[1], wh[2], wh[3]);
      } else if constexpr (NCH == 8) {
        // channels 8r .. 8r+7: channels 8r + k and 8r + 4 + k share word ((r >> 1) * 4 + k), bytes j0, j0 + 1
        const int r = lane & (LPH - 1);
        const int base = ((r >> 1) * 16) + 2 * (r & 1);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t lo2 = __builtin_amdgcn_perm(ai[4 + k], ai[k], 0x0c0c0400u);
          const uint32_t hi2 = __builtin_amdgcn_perm((ai[4 + k] + 128) >> 8, (ai[k] + 128) >> 8, 0x0c0c0400u);
          *reinterpret_cast<uint16_t*>(alo + base + 4 * k) = (uint16_t)lo2;
          *reinterpret_cast<uint16_t*>(ahi + base + 4 * k) = (uint16_t)hi2;
        }
      } else {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          const int c = ac0 + i;
          const int off = (((c >> 4) * 4 + (c & 3)) << 2) + ((c >> 2) & 3);
          alo[off] = (uint8_t)ai[i];
          ahi[off] = (uint8_t)((ai[i] + 128) >> 8);
        }
      }
    }
    wave_lds_sync();

    // 2. key dots: token lane of each page against every head
    int acc[2][GQ][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) acc[t][hh][0] = acc[t][hh][1] = 0;
    const uint32_t kw[2][8] = {{k00.x, k00.y, k00.z, k00.w, k01.x, k01.y, k01.z, k01.w},
                               {k10.x, k10.y, k10.z, k10.w, k11.x, k11.y, k11.z, k11.w}};
    // operand words in order (mw, head, limb); the read of the next one is issued before the current dots
    auto aword = [&](int idx) {
      const int mw = idx / (2 * GQ), hh = (idx / 2) % GQ, lb = idx & 1;
      return *reinterpret_cast<const uint4*>(abytes + hh * 256 + lb * 128 + mw * 16);
    };
    uint4 wk = aword(0);
#pragma unroll
    for (int mw = 0; mw < 8; ++mw) {
      uint32_t e[2][4];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int k = 0; k < 4; ++k) e[t][k] = (kw[t][mw] >> (2 * k)) & 0x03030303u;
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
#pragma unroll
        for (int lb = 0; lb < 2; ++lb) {
          const int idx = (mw * GQ + hh) * 2 + lb;
          const uint4 w = wk;
          if (idx + 1 < 16 * GQ) wk = aword(idx + 1);
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            int r = mw == 0 ? sdot4_z(w.x, e[t][0]) : __builtin_amdgcn_sdot4((int)w.x, (int)e[t][0], acc[t][hh][lb], false);
            r = __builtin_amdgcn_sdot4((int)w.y, (int)e[t][1], r, false);
            r = __builtin_amdgcn_sdot4((int)w.z, (int)e[t][2], r, false);
            r = __builtin_amdgcn_sdot4((int)w.w, (int)e[t][3], r, false);
            acc[t][hh][lb] = r;
          }
        }
      }
    }

    // 3. logits, group max, 16-bit weights as byte limbs in LDS
    float lg[2][GQ], mg[GQ], Pf[GQ];
    {
      float mx[GQ];
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
        lg[0][hh] = fmaf(A[hh], (float)(acc[0][hh][1] * 256 + acc[0][hh][0]), -AZ[hh]);
        lg[1][hh] = fmaf(A[hh], (float)(acc[1][hh][1] * 256 + acc[1][hh][0]), -AZ[hh]);
        mx[hh] = fmaxf(lg[0][hh], lg[1][hh]);
      }
      heads_allreduce<GQ>(mx, OpMax(), lane, mg);
    }
    {
      float ps[GQ];
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
        // u = floor(kPScale p + 0.5): p in (0, 1], u in [0, kPScale]; u = 256 hi + lo with signed bytes
        const int u0 = (int)fmaf(__builtin_amdgcn_exp2f(lg[0][hh] - mg[hh]), kPScale, 0.5f);
        const int u1 = (int)fmaf(__builtin_amdgcn_exp2f(lg[1][hh] - mg[hh]), kPScale, 0.5f);
        ps[hh] = (float)(u0 + u1);
        uint8_t* lo = pbytes + hh * 256;
        uint8_t* hi = lo + 128;
        lo[pb0] = (uint8_t)u0;
        hi[pb0] = (uint8_t)((u0 + 128) >> 8);
        lo[pb1] = (uint8_t)u1;
        hi[pb1] = (uint8_t)((u1 + 128) >> 8);
      }
      heads_allreduce<GQ>(ps, OpAdd(), lane, Pf);  // integers below 2^24: exact in fp32
    }
    wave_lds_sync();

    // 4. value dots: channels c0, c1 against the weights of every head
    int accv[2][GQ][2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) accv[c][hh][0] = accv[c][hh][1] = 0;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the value codes have landed in LDS
    const uint4 v00 = vst[c0], v01 = vst[64 + c0], v10 = vst[128 + c0], v11 = vst[192 + c0];
    const uint32_t vw[2][2][4] = {{{v00.x, v00.y, v00.z, v00.w}, {v10.x, v10.y, v10.z, v10.w}},
                                  {{v01.x, v01.y, v01.z, v01.w}, {v11.x, v11.y, v11.z, v11.w}}};
    // operand words in order (page, word, head, limb), read one ahead
    auto pword = [&](int idx) {
      const int pg = idx / (2 * GQ), hh = (idx / 2) % GQ, lb = idx & 1;  // pg = pp * 4 + gw
      return *reinterpret_cast<const uint4*>(pbytes + hh * 256 + lb * 128 + pg * 16);
    };
    uint4 wv = pword(0);
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
#pragma unroll
      for (int gw = 0; gw < 4; ++gw) {
        uint32_t e[2][4];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int k = 0; k < 4; ++k) e[c][k] = (vw[c][pp][gw] >> (2 * k)) & 0x03030303u;
#pragma unroll
        for (int hh = 0; hh < GQ; ++hh) {
#pragma unroll
          for (int lb = 0; lb < 2; ++lb) {
            const int idx = ((pp * 4 + gw) * GQ + hh) * 2 + lb;
            const uint4 w = wv;
            if (idx + 1 < 16 * GQ) wv = pword(idx + 1);
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              const int first = pp == 0 && gw == 0;
              int r = first ? sdot4_z(w.x, e[c][0]) : __builtin_amdgcn_sdot4((int)w.x, (int)e[c][0], accv[c][hh][lb], false);
              r = __builtin_amdgcn_sdot4((int)w.y, (int)e[c][1], r, false);
              r = __builtin_amdgcn_sdot4((int)w.z, (int)e[c][2], r, false);
              r = __builtin_amdgcn_sdot4((int)w.w, (int)e[c][3], r, false);
              accv[c][hh][lb] = r;
            }
          }
        }
      }
    }

    // 5. online-softmax update in the rotated value frame
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      const float mnew = fmaxf(m[hh], mg[hh]);
      const float sc = exp2_safe_diff(m[hh], mnew);
      const float wg = __builtin_amdgcn_exp2f(mg[hh] - mnew) * (1.0f / kPScale);
      const float U0 = (float)(accv[0][hh][1] * 256 + accv[0][hh][0]);
      const float U1 = (float)(accv[1][hh][1] * 256 + accv[1][hh][0]);
      o[hh][0] = fmaf(o[hh][0], sc, (wg * sv0) * fmaf(-zv0, Pf[hh], U0));
      o[hh][1] = fmaf(o[hh][1], sc, (wg * sv1) * fmaf(-zv1, Pf[hh], U1));
      l[hh] = fmaf(l[hh], sc, wg * Pf[hh]);
      m[hh] = mnew;
    }
    wave_lds_sync();
  }
  combine_and_store<GQ>(L, a, b, h, 1 + chunk, wave, lane, m, l, o, c0, c1);
}

// ---------------------------------------------------------------------------------------------
// INT2 chunk (and per-channel INT4), 16-bit fixed point on the 8-way nibble dot product (v_dot8).  Same
// algebra as int2_unit_dot16.  The key-side operand a = rint(alpha * 30583 / max|alpha|) is written as four
// signed 4-bit digits
//   a = d0 + 16 d1 + 256 d2 + 4096 d3,  d_k in [-8, 7]  (|a| <= 0x7777 = 30583),
// read off the biased value a + 0x8888 (whose hex digits are d_k + 8) by flipping bit 3 of every nibble;
// the weights u = rint(65535 p), p in [0, 1], are non-negative and use their four hex digits as they are
// (unsigned products).  A 2-bit code fills a nibble after a single mask, so one code word unpacks in three
// operations (seven for the byte form), and one dot8 multiplies 8 codes with one digit of 8 operands.
//   K code word m (channel 16m + 4j + k in byte j, bits 2k): (w >> 2n) & 0x33333333 holds channel
//   16m + 4j + n in the low and 16m + 4j + n + 2 in the high nibble of byte j (n = 0, 1);
//   V code word g of a channel (token 16j + 4g + r in byte j, bits 2r): (w >> 2n) & 0x33333333 holds
//   tokens 16j + 4g + n and 16j + 4g + n + 2 in byte j.
// The digit words of the key-side operand (head, m) and of the weights (head, page, g) put the digits of
// the same channels / tokens in the same nibbles; per (head, m) or (head, page, g) eight words,
//   X = [n0 d0, n0 d2, n1 d0, n1 d2],  Y = [n0 d1, n0 d3, n1 d1, n1 d3].
// Lane roles.  Keys: tokens t and t + 2 of one page (page = lane bit 5, t = 16 j + 4 g + r with j, g, r
// from lane bits 3-4, 1-2, 0), so that a lane owns both tokens of a weight nibble pair and writes whole
// bytes.  Values: channels lane, lane + 64.
// ---------------------------------------------------------------------------------------------
// Global -> LDS copies of 16 bytes per lane (lane i's bytes land at the LDS address in M0 + 16 i), issued
// from inline assembly so that the compiler adds no waits of its own for them: the nibble-digit unit keeps
// every global read of its loop in this form and waits on the vector-memory counter explicitly.  Per-lane
// 64-bit address, or a uniform base plus a per-lane 32-bit offset.
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ inline void dma16(uint32_t lds, const void* gaddr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(gaddr) : "memory");
}
__device__ inline void dma16_base(uint32_t lds, const void* gbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(gbase)
               : "memory");
}
// With an immediate offset: the instruction adds it to the LDS address too, so M0 is set OFF lower and the
// bytes land at lds + 16 i as with dma16.
template <int OFF>
__device__ inline void dma16_off(uint32_t lds, const void* gaddr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:%2" ::"s"(lds - OFF), "v"(gaddr),
               "i"(OFF)
               : "memory");
}
#define KVQ_WAIT_VM(n) asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory")

constexpr float kScale8 = 30583.0f;  // 0x7777: largest magnitude of four signed digits
constexpr int kBias8 = 0x8888;
constexpr float kScaleW = 65535.0f;  // value-side weights: four unsigned digits
// Rounding by a magic addend: for |x| <= 2^21, fp32(x + 1.5 * 2^23 + c) = 1.5 * 2^23 + c + rint(x) exactly
// (ties to even), and the low 16 bits of its encoding are rint(x) + c when 0 <= rint(x) + c < 2^16.
constexpr float kRoundA = 12582912.0f + (float)kBias8;  // key side: low half = a + 0x8888
constexpr float kRoundW = 8388608.0f;                   // weights (x >= 0): 2^23 + u, low half = u
constexpr uint32_t kRoundWBits = 0x4B000000u;

// ((r3 * 16 + r2) * 16 + r1) * 16 + r0 in three shift-adds
__device__ __forceinline__ int shl4_add(int hi, int lo) {
  int r;
  asm("v_lshl_add_u32 %0, %1, 4, %2" : "=v"(r) : "v"(hi), "v"(lo));
  return r;
}

__device__ inline int sdot8_z(uint32_t a, uint32_t b) {
  int r;
  asm("v_dot8_i32_i4 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ inline int sdot8(uint32_t a, uint32_t b, int c) { return __builtin_amdgcn_sdot8((int)a, (int)b, c, false); }
__device__ inline int udot8_z(uint32_t a, uint32_t b) {
  int r;
  asm("v_dot8_u32_u4 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ inline int udot8(uint32_t a, uint32_t b, int c) {
  return (int)__builtin_amdgcn_udot8(a, b, (uint32_t)c, false);
}

// Nibble pairs of two biased values (one per 16-bit half, or one each): X has [d0(lo) | d0(hi) << 4,
// d2(lo) | d2(hi) << 4] per 16-bit half, Y the d1 and d3 pairs; both still biased.
__device__ inline uint32_t nib_x(uint32_t lo, uint32_t hi) { return (lo & 0x0F0F0F0Fu) | ((hi << 4) & 0xF0F0F0F0u); }
__device__ inline uint32_t nib_y(uint32_t lo, uint32_t hi) { return ((lo >> 4) & 0x0F0F0F0Fu) | (hi & 0xF0F0F0F0u); }

// 4 x 4 byte transpose: o[k] byte i = x[i] byte k
__device__ inline uint4 byte_transpose(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3) {
  const uint32_t a = __builtin_amdgcn_perm(x1, x0, 0x05010400u);  // x0.b0 x1.b0 x0.b1 x1.b1
  const uint32_t b = __builtin_amdgcn_perm(x1, x0, 0x07030602u);  // x0.b2 x1.b2 x0.b3 x1.b3
  const uint32_t c = __builtin_amdgcn_perm(x3, x2, 0x05010400u);
  const uint32_t e = __builtin_amdgcn_perm(x3, x2, 0x07030602u);
  return make_uint4(__builtin_amdgcn_perm(c, a, 0x05040100u), __builtin_amdgcn_perm(c, a, 0x07060302u),
                    __builtin_amdgcn_perm(e, b, 0x05040100u), __builtin_amdgcn_perm(e, b, 0x07060302u));
}

// Per-wave state of the nibble-digit units: LDS areas, lane roles and the group copy pipeline.
// Copies of one group in issue order: M (1 copy: the even page's metadata to lanes 0-31, the odd page's
// to lanes 32-63), K (2-bit codes: 4 copies, copy j lane i = half j & 1 of token kt + 2 (j >> 1) of page kp;
// 4-bit codes: 8 copies, copy j = quarter j & 3 of token kt + 2 (j >> 2)), V (2-bit: 4 copies of 1 KB,
// half j & 1 of page j >> 1; 4-bit: 8 copies, copy j lane i = half j & 1 of channel i + 64 ((j >> 1) & 1)
// of page j >> 2).  Every copy lands at stage + 1 KB j + 16 i, so that each lane reads its own 16 bytes.
// The next group's copy of each is issued as soon as the current one has been read into registers, so
// every copy has a whole group's work to land; the waits count the copies issued after the one needed.
template <int GQ, int BITS>
struct Dot8Wave {
  static constexpr int NCOPY = 2 * BITS;                            // K (and V) copies per group
  static constexpr int META = BITS == 4 ? I4C_META_OFF : I2_META_OFF;
  uint32_t* adig;       // key digit words [head][m][8]
  uint8_t* pdig;        // weight digit words [head][page * 4 + g][8]
  uint16_t* aval;       // biased 16-bit key operands [head][128] (aliases pdig while the digits are built)
  const uint4* vst;     // value codes of a group
  const uint4* kst;     // key codes of a group, lane-ordered (the same buffer: keys are read out before the
                        // group's value codes are copied in)
  const uint16_t* mst;  // metadata of a group's two pages (1 KB)
  uint32_t vst_a, kst_a, mst_a;
  const uint8_t* pages;
  long long page_bytes, hoff;
  int lane, kp, kt;

  template <typename Lds>
  __device__ Dot8Wave(Lds& L, const DecodeArgs& a, int h, int wave, int lane_) {
    adig = reinterpret_cast<uint32_t*>(L.d.abytes[wave]);
    pdig = L.d.pbytes[wave];
    aval = reinterpret_cast<uint16_t*>(L.d.pbytes[wave]);
    vst = L.d.vstage[wave];
    kst = L.d.vstage[wave];
    mst = reinterpret_cast<const uint16_t*>(L.d.mstage[wave]);
    vst_a = lds_addr(vst);
    kst_a = lds_addr(kst);
    mst_a = lds_addr(mst);
    pages = a.pages;
    page_bytes = a.g.page_bytes;
    hoff = (long long)h * a.g.head_bytes;
    lane = lane_;
    kp = lane >> 5;
    kt = 16 * ((lane >> 3) & 3) + 4 * ((lane >> 1) & 3) + (lane & 1);
  }
  __device__ const uint8_t* page_of(int idx) const { return pages + (long long)idx * page_bytes + hoff; }
  // the lane's page of the pair: both page addresses are wave-uniform, the choice per lane is a select
  __device__ const uint8_t* lane_page(int2 p, bool second) const {
    const uint8_t* px = page_of(p.x);
    const uint8_t* py = page_of(p.y);
    return second ? py : px;
  }
  __device__ void issue_m(int2 p) const { dma16(mst_a, lane_page(p, lane >= 32) + META + (lane & 31) * 16); }
  __device__ void issue_k(int2 p) const {
    if constexpr (BITS == 4) {
      const uint8_t* src = lane_page(p, kp) + I4C_K_OFF + kt * 64;
      dma16_off<0>(kst_a, src);
      dma16_off<16>(kst_a + 1024, src);
      dma16_off<32>(kst_a + 2048, src);
      dma16_off<48>(kst_a + 3072, src);
      dma16_off<128>(kst_a + 4096, src);
      dma16_off<144>(kst_a + 5120, src);
      dma16_off<160>(kst_a + 6144, src);
      dma16_off<176>(kst_a + 7168, src);
    } else {
      const uint8_t* src = lane_page(p, kp) + I2_K_OFF + kt * 32;
      dma16_off<0>(kst_a, src);
      dma16_off<16>(kst_a + 1024, src);
      dma16_off<64>(kst_a + 2048, src);
      dma16_off<80>(kst_a + 3072, src);
    }
  }
  __device__ void issue_v(int2 p) const {
    if constexpr (BITS == 4) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        dma16_base(vst_a + 1024 * j, page_of(j < 4 ? p.x : p.y) + I4C_V_OFF + ((j >> 1) & 1) * 2048 + (j & 1) * 16,
                   lane * 32);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dma16_base(vst_a + 1024 * j, page_of(j < 2 ? p.x : p.y) + I2_V_OFF + (j & 1) * 1024, lane * 16);
    }
  }
};

// Packed biased 16-bit key operands of head ah, channels ac0 .. ac0 + 2 NW - 1 (word i: channel pair 2i, 2i + 1)
// to aval.
template <int NW>
__device__ __forceinline__ void store_key_operands(uint16_t* aval, int ah, int ac0, const uint32_t (&pk)[NW]) {
  uint32_t* dst = reinterpret_cast<uint32_t*>(aval + ah * D + ac0);
  if constexpr (NW >= 2) {
#pragma unroll
    for (int i = 0; i < NW; i += 2) *reinterpret_cast<uint2*>(dst + i) = make_uint2(pk[i], pk[i + 1]);
  } else {
    dst[0] = pk[0];
  }
}

// Low halves of two magic-rounded encodings as one word: lo16(e0) | lo16(e1) << 16.
__device__ __forceinline__ uint32_t pack_lo16(float e0, float e1) {
  return __builtin_amdgcn_perm(__float_as_uint(e1), __float_as_uint(e0), 0x05040100u);
}

// Key digit words from the biased operands: lane task (head, m, X or Y) reads the 16 channels of word m.
// X takes digits 0 and 2 (low nibble of each byte), Y digits 1 and 3 (high nibble); the task's choice is a
// shift amount, so that the wave does not diverge.
template <int GQ>
__device__ __forceinline__ void build_key_digits(uint32_t* adig, const uint16_t* aval, int lane) {
#pragma unroll
  for (int u = lane; u < 16 * GQ; u += 64) {
    const int hh = u >> 4, mw = (u >> 1) & 7;
    const uint32_t sl = (u & 1) * 4, sh = 4 - sl;
    const uint4* src = reinterpret_cast<const uint4*>(aval + hh * D + 16 * mw);
    const uint4 d0 = src[0], d1 = src[1];  // channel pairs (16 mw + 2 i, + 1), i = 0..7
    const uint32_t dd[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
    uint32_t z[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      z[j] = (((dd[2 * j] >> sl) & 0x0F0F0F0Fu) | ((dd[2 * j + 1] << sh) & 0xF0F0F0F0u)) ^ 0x88888888u;
    reinterpret_cast<uint4*>(adig)[(hh * 8 + mw) * 2 + (u & 1)] = byte_transpose(z[0], z[1], z[2], z[3]);
  }
}

// One 32-bit code word (nibble vectors nb[0], nb[1]) against the digit words X, Y of one head; signed
// (key side) or unsigned (value side) 4-bit products.
template <bool SIGNED>
__device__ __forceinline__ void dot8_word(int (&r)[4], uint4 X, uint4 Y, const uint32_t (&nb)[2], bool first) {
  auto d = [](uint32_t x, uint32_t y, int c) { return SIGNED ? sdot8(x, y, c) : udot8(x, y, c); };
  auto dz = [](uint32_t x, uint32_t y) { return SIGNED ? sdot8_z(x, y) : udot8_z(x, y); };
  if (first) {
    r[0] = dz(X.x, nb[0]);
    r[2] = dz(X.y, nb[0]);
    r[1] = dz(Y.x, nb[0]);
    r[3] = dz(Y.y, nb[0]);
  } else {
    r[0] = d(X.x, nb[0], r[0]);
    r[2] = d(X.y, nb[0], r[2]);
    r[1] = d(Y.x, nb[0], r[1]);
    r[3] = d(Y.y, nb[0], r[3]);
  }
  r[0] = d(X.z, nb[1], r[0]);
  r[2] = d(X.w, nb[1], r[2]);
  r[1] = d(Y.z, nb[1], r[1]);
  r[3] = d(Y.w, nb[1], r[3]);
}

__device__ __forceinline__ int digits_value(const int (&r)[4]) { return shl4_add(shl4_add(shl4_add(r[3], r[2]), r[1]), r[0]); }

// Nibble vectors of code word pair idx: nb[0] holds the codes that pair with the X.x / X.y / Y.x / Y.y digit
// words, nb[1] those of X.z / X.w / Y.z / Y.w.  2-bit codes: word idx, even then odd code positions
// (values 0..3); 4-bit codes: words 2 idx and 2 idx + 1, as they are (values 0..15, unsigned products), or
// less 8 (values -8..7, signed products; the offset is taken out of the zero points).
template <int BITS, bool SIGNED, int N>
__device__ __forceinline__ void code_nibbles(uint32_t (&nb)[2], const uint32_t (&w)[N], int idx) {
  if constexpr (BITS == 4) {
    const uint32_t f = SIGNED ? 0x88888888u : 0u;
    nb[0] = w[2 * idx] ^ f;
    nb[1] = w[2 * idx + 1] ^ f;
  } else {
    nb[0] = w[idx] & 0x33333333u;
    nb[1] = (w[idx] >> 2) & 0x33333333u;
  }
}

// acc[t][head] = digit sums of tokens kt, kt + 2 (code words kw[t]) against the key digit words.
template <int GQ, int BITS>
__device__ __forceinline__ void key_dots(const uint32_t* adig, const uint32_t (&kw)[2][4 * BITS],
                                         int (&acc)[2][GQ][4]) {
  auto aword = [&](int idx) { return reinterpret_cast<const uint4*>(adig)[idx]; };  // idx = (hh 8 + mw) 2 + y
  uint4 wx = aword(0), wy = aword(1);
#pragma unroll
  for (int mw = 0; mw < 8; ++mw) {
    uint32_t nb[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) code_nibbles<BITS, true>(nb[t], kw[t], mw);
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      const uint4 X = wx, Y = wy;
      const int nxt = mw * GQ + hh + 1;
      if (nxt < 8 * GQ) {
        const int nm = nxt / GQ, nh = nxt % GQ;
        wx = aword((nh * 8 + nm) * 2);
        wy = aword((nh * 8 + nm) * 2 + 1);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) dot8_word<true>(acc[t][hh], X, Y, nb[t], mw == 0);
    }
  }
}

// accv[c][head] = digit sums of channels lane, lane + 64 (code words vw[c][page]) against the unsigned
// weight digits.
template <int GQ, int BITS>
__device__ __forceinline__ void value_dots(const uint8_t* pdig, const uint32_t (&vw)[2][2][2 * BITS],
                                           int (&accv)[2][GQ][4]) {
  auto pword = [&](int idx) { return reinterpret_cast<const uint4*>(pdig)[idx]; };  // ((hh 8 + pg) 2 + y)
  uint4 px = pword(0), py = pword(1);
#pragma unroll
  for (int pg = 0; pg < 8; ++pg) {  // pg = page * 4 + g
    uint32_t nb[2][2];
#pragma unroll
    for (int c = 0; c < 2; ++c) code_nibbles<BITS, false>(nb[c], vw[c][pg >> 2], pg & 3);
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      const uint4 X = px, Y = py;
      const int nxt = pg * GQ + hh + 1;
      if (nxt < 8 * GQ) {
        const int npg = nxt / GQ, nh = nxt % GQ;
        px = pword((nh * 8 + npg) * 2);
        py = pword((nh * 8 + npg) * 2 + 1);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) dot8_word<false>(accv[c][hh], X, Y, nb[c], pg == 0);
    }
  }
}

// Weight digits of the lane's tokens kt, kt + 2 (unsigned 16-bit weights in the low halves of u0, u1) for
// one head: byte kj of the words (page kp, g, n = kt & 1, digit 0..3).
// pw = pdig + head * 256 + ((kp 4 + g) 8 + n 2) 4 + kj.
__device__ __forceinline__ void store_weight_digits(uint8_t* pw, uint32_t u0, uint32_t u1) {
  const uint32_t x = nib_x(u0, u1), y = nib_y(u0, u1);
  pw[0] = (uint8_t)x;          // n d0
  pw[4] = (uint8_t)(x >> 8);   // n d2
  pw[16] = (uint8_t)y;         // n d1
  pw[20] = (uint8_t)(y >> 8);  // n d3
}

template <int GQ, int BITS, typename Lds>
__device__ void int2_unit_dot8(Lds& L, const DecodeArgs& a, int b, int h, int T, int chunk) {
  constexpr int LG = HeadLog2<GQ>::v;
  constexpr int LPH = 64 >> LG;   // lanes per head in the alpha step
  constexpr int NCH = 2 * GQ;     // channels per lane in the alpha step
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ng = n_groups_of(T, g.S0, g.W);
  // the wave's groups: its own chunk, walked in order (wave chunks), or every fourth group of the work-group's
  const bool wc = g.wave_chunks != 0;
  const int chunk_id = wc ? 4 * chunk + wave : chunk;
  const int g_begin = chunk_id * g.gpc;
  int g_end = (g_begin + g.gpc) < ng ? (g_begin + g.gpc) : ng;
  if (g_end > g.max_pages / 2) g_end = g.max_pages / 2;  // never index past the page-table row
  const int gstep = wc ? 1 : 4;
  const int g_first = wc ? g_begin : g_begin + wave;
  const int c0 = lane, c1 = lane + 64;
  const int ah = lane >> (6 - LG);           // head of this lane in the alpha step
  const int ac0 = (lane & (LPH - 1)) * NCH;  // its first channel
  Dot8Wave<GQ, BITS> W(L, a, h, wave, lane);
  constexpr float ZOFF = BITS == 4 ? 8.0f : 0.0f;  // 4-bit key codes enter the dot products less 8
  // weight digit bytes of this lane's tokens: word (page kp, g, n) byte j of each head
  uint8_t* pw = W.pdig + ((W.kp * 4 + ((lane >> 1) & 3)) * 8 + (lane & 1) * 2) * 4 + ((lane >> 3) & 3);
  float qa[NCH];
  {
    const float* q = a.qrot + ((long long)b * g.n_q + h * GQ + ah) * D + ac0;
#pragma unroll
    for (int i = 0; i < NCH; ++i) qa[i] = q[i];
    // consume the query here, so that the compiler's own wait for these loads sits before the loop and not
    // inside it (where, not knowing of the copies below, it would wait for all of them)
#pragma unroll
    for (int i = 0; i < NCH; ++i) asm volatile("" ::"v"(qa[i]));
  }
  float m[GQ], l[GQ], o[GQ][2];
#pragma unroll
  for (int hh = 0; hh < GQ; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.0f;
    o[hh][0] = o[hh][1] = 0.0f;
  }
  const int2* pt = reinterpret_cast<const int2*>(a.page_table + (long long)b * g.max_pages);
  // copies in flight, in issue order: this group's M and K; the next group's M is issued once this M is read,
  // this group's V once its K is read (into the same buffer), the next group's K once this V is read
  int2 pcur = make_int2(0, 0), pnext = make_int2(0, 0);
  if (g_first < g_end) {
    pcur = scalar_load_int2(pt + g_first);
    W.issue_m(pcur);
    W.issue_k(pcur);
  }
  for (int gi = g_first; gi < g_end; gi += gstep) {
    const bool has_next = gi + gstep < g_end;  // uniform
    if (has_next) pnext = scalar_load_int2(pt + gi + gstep);
    if constexpr (BITS == 4) KVQ_WAIT_VM(8);  // this group's M copy (its K copies may still be in flight)
    else KVQ_WAIT_VM(4);
    uint32_t skw[NCH / 2], zkw[NCH / 2];
#pragma unroll
    for (int i = 0; i < NCH / 2; ++i) {
      skw[i] = reinterpret_cast<const uint32_t*>(W.mst)[ac0 / 2 + i];
      zkw[i] = reinterpret_cast<const uint32_t*>(W.mst)[(D + ac0) / 2 + i];
    }
    const float sv0 = bf16_to_f32(W.mst[2 * D + c0]), sv1 = bf16_to_f32(W.mst[2 * D + c1]);
    const float zv0 = bf16_to_f32(W.mst[3 * D + c0]), zv1 = bf16_to_f32(W.mst[3 * D + c1]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before the next group's copy overwrites it
    if (has_next) W.issue_m(pnext);

    // 1. alpha of this group for head ah, channels ac0.., 16-bit, biased, to LDS
    float A[GQ], AZ[GQ];
    {
      float al[NCH];
      int amx_i = 0;  // max |alpha| as its bit pattern (non-negative floats order as their bits)
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const uint32_t w = skw[i >> 1];
        al[i] = qa[i] * __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
        amx_i = max(amx_i, __float_as_int(fabsf(al[i])));
      }
      const float amx = __int_as_float(seg_max_i<LPH>(amx_i));
      // a = rint(alpha * inv) in [-30583, 30583] (the reciprocal's 1-ulp error cannot carry the largest past
      // 30583.5); below 2^-100 the coefficients are taken as zero (their logit terms are below fp32's reach)
      const float inv = amx > 0x1p-100f ? kScale8 * __builtin_amdgcn_rcpf(amx) : 0.0f;
      uint32_t pk[NCH / 2];
      float zs = 0.0f;
#pragma unroll
      for (int i = 0; i < NCH; i += 2) {
        const float e0 = fmaf(al[i], inv, kRoundA), e1 = fmaf(al[i + 1], inv, kRoundA);
        const uint32_t w = zkw[i >> 1];
        zs = fmaf(e0 - kRoundA, __uint_as_float(w << 16) - ZOFF, zs);
        zs = fmaf(e1 - kRoundA, __uint_as_float(w & 0xffff0000u) - ZOFF, zs);
        pk[i >> 1] = pack_lo16(e0, e1);  // a + 0x8888 of both channels
      }
      zs = seg_sum<LPH>(zs);
      const float Ah = amx * (1.0f / kScale8);
      const float AZh = Ah * zs;
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
        A[hh] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Ah), hh * LPH));
        AZ[hh] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(AZh), hh * LPH));
      }
      store_key_operands<NCH / 2>(W.aval, ah, ac0, pk);
    }
    wave_lds_sync();
    // 2. key digit words
    build_key_digits<GQ>(W.adig, W.aval, lane);
    wave_lds_sync();

    // 3. key dots: tokens kt, kt + 2 of page kp against every head
    // this group's K copies (the next group's M may be in flight)
    if (has_next) KVQ_WAIT_VM(1);
    else KVQ_WAIT_VM(0);
    uint32_t kw[2][4 * BITS];
#pragma unroll
    for (int j = 0; j < 2 * BITS; ++j) {  // copy j: token j / BITS, words 4 (j % BITS) ..
      const uint4 kk = W.kst[64 * j + c0];
      uint32_t* dst = &kw[j / BITS][4 * (j % BITS)];
      dst[0] = kk.x, dst[1] = kk.y, dst[2] = kk.z, dst[3] = kk.w;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    W.issue_v(pcur);  // into the buffer the key codes have left
    int acc[2][GQ][4];
    key_dots<GQ, BITS>(W.adig, kw, acc);

    // 4. logits logit_t = A val_t - AZ; their group maximum is that of the integer sums val_t (A >= 0);
    //    weights p_t = 2^(A (val_t - val_max)) <= 1 as unsigned 16-bit nibble digits in LDS
    float mg[GQ], Pf[GQ];
    {
      float vf[2][GQ];
      int mx[GQ], vmax[GQ];
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
        const int v0 = digits_value(acc[0][hh]), v1 = digits_value(acc[1][hh]);
        vf[0][hh] = (float)v0;
        vf[1][hh] = (float)v1;
        mx[hh] = max(v0, v1);
      }
      heads_allreduce_fast<GQ>(mx, [](int x, int y) { return max(x, y); }, [](int x) { return seg_max_i<(64 >> LG)>(x); },
                               lane, vmax);
      float ps[GQ];
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
        const float vm = (float)vmax[hh];
        mg[hh] = fmaf(A[hh], vm, -AZ[hh]);
        const float ref = A[hh] * vm;
        // u = rint(65535 p) in [0, 65535], in the low half of the magic-rounded encoding (p exceeds 1 by at
        // most the rounding of ref, far below half a unit of u)
        const uint32_t u0 = __float_as_uint(fmaf(__builtin_amdgcn_exp2f(fmaf(A[hh], vf[0][hh], -ref)), kScaleW, kRoundW));
        const uint32_t u1 = __float_as_uint(fmaf(__builtin_amdgcn_exp2f(fmaf(A[hh], vf[1][hh], -ref)), kScaleW, kRoundW));
        ps[hh] = (float)(int)(u0 + u1 - 2 * kRoundWBits);
        store_weight_digits(pw + hh * 256, u0, u1);
      }
      // integers below 2^24: exact in fp32
      heads_allreduce_fast<GQ>(ps, [](float x, float y) { return x + y; }, [](float x) { return seg_sum<(64 >> LG)>(x); },
                               lane, Pf);
    }
    wave_lds_sync();

    // 5. value dots: channels c0, c1 against the weights of every head
    KVQ_WAIT_VM(0);  // this group's V copies, the youngest in flight
    uint32_t vw[2][2][2 * BITS];  // [channel c0 | c1][page][word]
#pragma unroll
    for (int j = 0; j < 2 * BITS; ++j) {
      const uint4 vv = W.vst[64 * j + c0];
      // 2-bit: copy j = page j >> 1, channel j & 1; 4-bit: page j >> 2, channel (j >> 1) & 1, words 4 (j & 1) ..
      uint32_t* dst = BITS == 4 ? &vw[(j >> 1) & 1][j >> 2][4 * (j & 1)] : &vw[j & 1][j >> 1][0];
      dst[0] = vv.x, dst[1] = vv.y, dst[2] = vv.z, dst[3] = vv.w;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (has_next) W.issue_k(pnext);
    int accv[2][GQ][4];
    value_dots<GQ, BITS>(W.pdig, vw, accv);

    // 6. online-softmax update in the rotated value frame; o and l carry the weights' factor 65535 (both
    //    are divided by it after the walk), and are rescaled in place so that they keep their registers
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      const float mnew = fmax_raw(m[hh], mg[hh]);          // finite: every group's logits are
      const float sc = __builtin_amdgcn_exp2f(m[hh] - mnew);  // 0 before the first group (m = -inf)
      const float eg = __builtin_amdgcn_exp2f(mg[hh] - mnew);
      const float Y0 = fmaf(-zv0, Pf[hh], (float)digits_value(accv[0][hh]));
      const float Y1 = fmaf(-zv1, Pf[hh], (float)digits_value(accv[1][hh]));
      o[hh][0] *= sc;
      o[hh][0] = fmaf(eg * sv0, Y0, o[hh][0]);
      o[hh][1] *= sc;
      o[hh][1] = fmaf(eg * sv1, Y1, o[hh][1]);
      l[hh] *= sc;
      l[hh] = fmaf(eg, Pf[hh], l[hh]);
      m[hh] = mnew;
    }
    wave_lds_sync();
    pcur = pnext;
  }
#pragma unroll
  for (int hh = 0; hh < GQ; ++hh) {
    o[hh][0] *= 1.0f / kScaleW;
    o[hh][1] *= 1.0f / kScaleW;
    l[hh] *= 1.0f / kScaleW;
  }
  if (wc) {
    // every partial a merge reads is written; chunks past the length or the launch bound have none
    if (g_begin < ng && chunk_id < g.n_units - 1) store_wave_partial<GQ>(a, b, h, 1 + chunk_id, lane, m, l, o, c0, c1);
  } else {
    combine_and_store<GQ>(L, a, b, h, 1 + chunk, wave, lane, m, l, o, c0, c1);
  }
}

// ---------------------------------------------------------------------------------------------
// Per-token INT2 chunk ([OSCAR] §3.4.4 step 3 taken per token over its 128 channels) on the nibble dot
// product.  With the key scale s_t and zero z_t of token t,
//   logit_t = s_t (sum_c q~_c code_tc - z_t sum_c q~_c),
// so the key-side operand is the rotated query itself, rounded once per work-group to 16 bits,
// a_c = rint(30583 q~_c / max|q~|), A = max|q~| / 30583: logit_t = A s_t (sum_c a_c code_tc - z_t sum_c a_c),
// and its digit words are built once before the walk.  Values: the group adds
//   sum_t p_t s'_t (code'_tc - z'_t) = (S' / 65535) (sum_t u_t code'_tc - sum_t u_t z'_t)
// to the output, with the weights p_t s'_t rounded to u_t = rint(65535 p_t s'_t / S'), S' the group's
// largest weight p_t s'_t of the head (p_t <= 1 relative to the group's largest logit), and sum_t p_t to the
// softmax sum.
// Lane roles, digit words and the copy pipeline as in int2_unit_dot8; the metadata of a page holds its
// tokens' K scales, K zeros, V scales, V zeros (64 bf16 each).
// ---------------------------------------------------------------------------------------------
template <int GQ, typename Lds>
__device__ void int2tok_unit_dot8(Lds& L, const DecodeArgs& a, int b, int h, int T, int chunk) {
  constexpr int LG = HeadLog2<GQ>::v;
  constexpr int LPH = 64 >> LG;
  constexpr int NCH = 2 * GQ;
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ng = n_groups_of(T, g.S0, g.W);
  // the wave's groups: its own chunk, walked in order (wave chunks), or every fourth group of the work-group's
  const bool wc = g.wave_chunks != 0;
  const int chunk_id = wc ? 4 * chunk + wave : chunk;
  const int g_begin = chunk_id * g.gpc;
  int g_end = (g_begin + g.gpc) < ng ? (g_begin + g.gpc) : ng;
  if (g_end > g.max_pages / 2) g_end = g.max_pages / 2;  // never index past the page-table row
  const int gstep = wc ? 1 : 4;
  const int g_first = wc ? g_begin : g_begin + wave;
  const int c0 = lane, c1 = lane + 64;
  const int ah = lane >> (6 - LG);
  const int ac0 = (lane & (LPH - 1)) * NCH;
  Dot8Wave<GQ, 2> W(L, a, h, wave, lane);
  uint8_t* pw = W.pdig + ((W.kp * 4 + ((lane >> 1) & 3)) * 8 + (lane & 1) * 2) * 4 + ((lane >> 3) & 3);
  const int mt0 = W.kp * 256 + (W.kt & 63);  // metadata index of token kt (page kp): K s; +64 K z; +128, +192 V

  // 0. the key-side operand, once: rotated query of head ah, channels ac0.., as digit words
  float A[GQ], FS[GQ];  // A_h and sum_c a_c (an integer below 2^22: exact in fp32)
  {
    float qa[NCH];
    const float* q = a.qrot + ((long long)b * g.n_q + h * GQ + ah) * D + ac0;
#pragma unroll
    for (int i = 0; i < NCH; ++i) qa[i] = q[i];
    float amx = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) amx = fmaxf(amx, fabsf(qa[i]));
    amx = seg_reduce<LPH>(amx, OpMax());
    const float inv = amx > 0x1p-100f ? kScale8 * __builtin_amdgcn_rcpf(amx) : 0.0f;
    uint32_t pk[NCH / 2];
    float fsum = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; i += 2) {
      const float e0 = fmaf(qa[i], inv, kRoundA), e1 = fmaf(qa[i + 1], inv, kRoundA);
      fsum += (e0 - kRoundA) + (e1 - kRoundA);  // integers: exact
      pk[i >> 1] = pack_lo16(e0, e1);
    }
    const float fs = seg_reduce<LPH>(fsum, OpAdd());
    const float Ah = amx * (1.0f / kScale8);
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      A[hh] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Ah), hh * LPH));
      FS[hh] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fs), hh * LPH));
    }
    store_key_operands<NCH / 2>(W.aval, ah, ac0, pk);
    wave_lds_sync();
    build_key_digits<GQ>(W.adig, W.aval, lane);
    wave_lds_sync();
  }
  float m[GQ], l[GQ], o[GQ][2];
#pragma unroll
  for (int hh = 0; hh < GQ; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.0f;
    o[hh][0] = o[hh][1] = 0.0f;
  }
  const int2* pt = reinterpret_cast<const int2*>(a.page_table + (long long)b * g.max_pages);
  // copies in flight as in int2_unit_dot8: M and K of a group, its V once its K is read, the next K after V
  int2 pcur = make_int2(0, 0), pnext = make_int2(0, 0);
  if (g_first < g_end) {
    pcur = scalar_load_int2(pt + g_first);
    W.issue_m(pcur);
    W.issue_k(pcur);
  }
  for (int gi = g_first; gi < g_end; gi += gstep) {
    const bool has_next = gi + gstep < g_end;  // uniform
    if (has_next) pnext = scalar_load_int2(pt + gi + gstep);
    KVQ_WAIT_VM(4);  // this group's M copy (its K copies may still be in flight)
    float sk[2], zk[2], svt[2], zvt[2];  // tokens kt, kt + 2
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sk[t] = bf16_to_f32(W.mst[mt0 + 2 * t]);
      zk[t] = bf16_to_f32(W.mst[mt0 + 2 * t + 64]);
      svt[t] = bf16_to_f32(W.mst[mt0 + 2 * t + 128]);
      zvt[t] = bf16_to_f32(W.mst[mt0 + 2 * t + 192]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (has_next) W.issue_m(pnext);

    // 1. key dots (this group's K copies; the next group's M may be in flight)
    if (has_next) KVQ_WAIT_VM(1);
    else KVQ_WAIT_VM(0);
    const uint4 k00 = W.kst[c0], k01 = W.kst[64 + c0], k10 = W.kst[128 + c0], k11 = W.kst[192 + c0];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    W.issue_v(pcur);  // into the buffer the key codes have left
    int acc[2][GQ][4];
    const uint32_t kw[2][8] = {{k00.x, k00.y, k00.z, k00.w, k01.x, k01.y, k01.z, k01.w},
                               {k10.x, k10.y, k10.z, k10.w, k11.x, k11.y, k11.z, k11.w}};
    key_dots<GQ, 2>(W.adig, kw, acc);

    // 2. logits, group max, weights p_t s'_t / S' as digits, sum_t p_t and sum_t u_t z'_t
    float lg[2][GQ], mg[GQ], Pl[GQ], Zs[GQ];
    {
      float mx[GQ];
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
          lg[t][hh] = (A[hh] * sk[t]) * fmaf(-zk[t], FS[hh], (float)digits_value(acc[t][hh]));
        mx[hh] = fmaxf(lg[0][hh], lg[1][hh]);
      }
      heads_allreduce<GQ>(mx, OpMax(), lane, mg);
    }
    // S'_h: the group's largest weight p_t s'_t of head h (positive: the largest logit has p = 1)
    float p[2][GQ], Sw[GQ];
    {
      float sm[GQ];
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
        p[0][hh] = __builtin_amdgcn_exp2f(lg[0][hh] - mg[hh]);
        p[1][hh] = __builtin_amdgcn_exp2f(lg[1][hh] - mg[hh]);
        sm[hh] = fmaxf(p[0][hh] * svt[0], p[1][hh] * svt[1]);
      }
      heads_allreduce<GQ>(sm, OpMax(), lane, Sw);
    }
    {
      float ps[GQ], zs[GQ];
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
        const float r = Sw[hh] > 0.0f ? kScaleW / Sw[hh] : 0.0f;
        const float e0 = fmaf(p[0][hh] * svt[0], r, kRoundW), e1 = fmaf(p[1][hh] * svt[1], r, kRoundW);
        const uint32_t u0 = __float_as_uint(e0), u1 = __float_as_uint(e1);
        ps[hh] = p[0][hh] + p[1][hh];
        zs[hh] = fmaf(e0 - kRoundW, zvt[0], (e1 - kRoundW) * zvt[1]);
        store_weight_digits(pw + hh * 256, u0, u1);
      }
      heads_allreduce<GQ>(ps, OpAdd(), lane, Pl);
      heads_allreduce<GQ>(zs, OpAdd(), lane, Zs);
    }
    wave_lds_sync();

    // 3. value dots
    KVQ_WAIT_VM(0);  // this group's V copies, the youngest in flight
    const uint4 v00 = W.vst[c0], v01 = W.vst[64 + c0], v10 = W.vst[128 + c0], v11 = W.vst[192 + c0];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (has_next) W.issue_k(pnext);
    int accv[2][GQ][4];
    const uint32_t vw[2][2][4] = {{{v00.x, v00.y, v00.z, v00.w}, {v10.x, v10.y, v10.z, v10.w}},
                                  {{v01.x, v01.y, v01.z, v01.w}, {v11.x, v11.y, v11.z, v11.w}}};
    value_dots<GQ, 2>(W.pdig, vw, accv);

    // 4. online-softmax update in the rotated value frame
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      const float mnew = fmaxf(m[hh], mg[hh]);
      const float sc = __builtin_amdgcn_exp2f(m[hh] - mnew);  // 0 before the first group (m = -inf)
      const float eg = __builtin_amdgcn_exp2f(mg[hh] - mnew);
      const float wg = eg * Sw[hh] * (1.0f / kScaleW);
      o[hh][0] = fmaf(o[hh][0], sc, wg * ((float)digits_value(accv[0][hh]) - Zs[hh]));
      o[hh][1] = fmaf(o[hh][1], sc, wg * ((float)digits_value(accv[1][hh]) - Zs[hh]));
      l[hh] = fmaf(l[hh], sc, eg * Pl[hh]);
      m[hh] = mnew;
    }
    wave_lds_sync();
    pcur = pnext;
  }
  if (wc) {
    // every partial a merge reads is written; chunks past the length or the launch bound have none
    if (g_begin < ng && chunk_id < g.n_units - 1) store_wave_partial<GQ>(a, b, h, 1 + chunk_id, lane, m, l, o, c0, c1);
  } else {
    combine_and_store<GQ>(L, a, b, h, 1 + chunk, wave, lane, m, l, o, c0, c1);
  }
}

// ---------------------------------------------------------------------------------------------
// INT4 token-wise chunk ([SAW] App. A.1 eq. (3)-(4), App. A.4 eq. (13)) on the nibble dot product, with
// the per-token INT2 unit's algebra: the key-side operand is the rotated query, rounded once per
// work-group to a_c (16-bit, four signed digits), and
//   logit_t = A s_t (sum_c a_c (code_tc - 8) + (8 - z_t) sum_c a_c)
// (4-bit key codes enter the signed products less 8); values: the weights p_t s'_t / S' as unsigned
// 16-bit digits against the codes as they are.  The page layout is the INT4 one as written: a key code
// word holds 8 consecutive channels (word m, nibble k = channel 8m + k), so the key digit words are built
// for that order (word (m, d): nibble k = digit d of a_{8m+k}); a value code word of a channel holds
// tokens 16(2jh + jl) + 4g + r at nibble 4jl + r (word 2g + jh), so a lane owns the two tokens of one byte,
// t0 = 16j + 4g + 2h and t0 + 1 (j, g, h from lane bits 3-4, 1-2, 0; page = lane bit 5).  Pages are walked
// in pairs (128 tokens, two pages as the grouped schemes' groups); tokens past the length are masked by
// selects, and a missing second page of the last pair is replaced by the first (read, never used).
// ---------------------------------------------------------------------------------------------
// Key digit words for 8-consecutive-channel code words: task (head, m) reads channels 8m .. 8m + 7.
template <int GQ>
__device__ __forceinline__ void build_key_digits_seq(uint32_t* adig, const uint16_t* aval, int lane) {
#pragma unroll
  for (int u = lane; u < 16 * GQ; u += 64) {
    const int hh = u >> 4, m = u & 15;
    const uint4 v = *reinterpret_cast<const uint4*>(aval + hh * D + 8 * m);  // channel pairs (8m + 2i, + 1)
    const uint32_t pr[4] = {v.x, v.y, v.z, v.w};
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t by[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t t = (pr[i] >> (4 * d)) & 0x000F000Fu;  // digit d of both channels of the pair
        by[i] = (t | (t >> 12)) & 0xFFu;                      // low nibble channel 8m + 2i, high 8m + 2i + 1
      }
      w[d] = (by[0] | (by[1] << 8) | (by[2] << 16) | (by[3] << 24)) ^ 0x88888888u;
    }
    reinterpret_cast<uint4*>(adig)[hh * 16 + m] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// acc[t][head][d] = digit-d sums of tokens t0, t0 + 1 (16 code words each) against the key digit words.
template <int GQ>
__device__ __forceinline__ void key_dots_seq(const uint32_t* adig, const uint32_t (&kw)[2][16], int (&acc)[2][GQ][4]) {
  auto aword = [&](int idx) { return reinterpret_cast<const uint4*>(adig)[idx]; };  // idx = hh 16 + m
  uint4 nxt = aword(0);
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const uint32_t nb[2] = {kw[0][m] ^ 0x88888888u, kw[1][m] ^ 0x88888888u};
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      const uint4 X = nxt;
      const int k = hh * 16 + m;  // the next word read: (head + 1, m), or (0, m + 1)
      const int kn = hh + 1 < GQ ? k + 16 : m + 1;
      if (hh + 1 < GQ || m + 1 < 16) nxt = aword(kn);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (m == 0) {
          acc[t][hh][0] = sdot8_z(X.x, nb[t]);
          acc[t][hh][1] = sdot8_z(X.y, nb[t]);
          acc[t][hh][2] = sdot8_z(X.z, nb[t]);
          acc[t][hh][3] = sdot8_z(X.w, nb[t]);
        } else {
          acc[t][hh][0] = sdot8(X.x, nb[t], acc[t][hh][0]);
          acc[t][hh][1] = sdot8(X.y, nb[t], acc[t][hh][1]);
          acc[t][hh][2] = sdot8(X.z, nb[t], acc[t][hh][2]);
          acc[t][hh][3] = sdot8(X.w, nb[t], acc[t][hh][3]);
        }
      }
    }
  }
}

// accv[c][head][d] = digit-d sums of channels lane, lane + 64 (8 code words per page) against the weights;
// weight digit words [head][page][word][d].
template <int GQ>
__device__ __forceinline__ void value_dots_seq(const uint8_t* pdig, const uint32_t (&vw)[2][2][8], int (&accv)[2][GQ][4]) {
  auto pword = [&](int idx) { return reinterpret_cast<const uint4*>(pdig)[idx]; };  // idx = (hh 2 + pg) 8 + W
  uint4 nxt = pword(0);
#pragma unroll
  for (int pw = 0; pw < 16; ++pw) {  // pw = page * 8 + word
    const uint32_t nb[2] = {vw[0][pw >> 3][pw & 7], vw[1][pw >> 3][pw & 7]};
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      const uint4 X = nxt;
      const int kn = hh + 1 < GQ ? (hh + 1) * 16 + pw : pw + 1;
      if (hh + 1 < GQ || pw + 1 < 16) nxt = pword(kn);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        if (pw == 0) {
          accv[c][hh][0] = udot8_z(X.x, nb[c]);
          accv[c][hh][1] = udot8_z(X.y, nb[c]);
          accv[c][hh][2] = udot8_z(X.z, nb[c]);
          accv[c][hh][3] = udot8_z(X.w, nb[c]);
        } else {
          accv[c][hh][0] = udot8(X.x, nb[c], accv[c][hh][0]);
          accv[c][hh][1] = udot8(X.y, nb[c], accv[c][hh][1]);
          accv[c][hh][2] = udot8(X.z, nb[c], accv[c][hh][2]);
          accv[c][hh][3] = udot8(X.w, nb[c], accv[c][hh][3]);
        }
      }
    }
  }
}

template <int GQ, typename Lds>
__device__ void int4tok_unit_dot8(Lds& L, const DecodeArgs& a, int b, int h, int T, int chunk) {
  constexpr int LG = HeadLog2<GQ>::v;
  constexpr int LPH = 64 >> LG;
  constexpr int NCH = 2 * GQ;
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int npages = (T + PAGE - 1) / PAGE;
  const int npairs = (npages + 1) / 2;
  // the wave's page pairs: its own chunk (wave chunks) or every fourth pair of the work-group's chunk
  const bool wc = g.wave_chunks != 0;
  const int chunk_id = wc ? 4 * chunk + wave : chunk;
  const int pb = chunk_id * g.gpc / 2;  // chunks hold an even number of pages
  int pe = pb + g.gpc / 2 < npairs ? pb + g.gpc / 2 : npairs;
  if (2 * pe > g.max_pages + 1) pe = (g.max_pages + 1) / 2;  // never index past the page-table row
  const int pstep = wc ? 1 : 4;
  const int p_first = wc ? pb : pb + wave;
  const int c0 = lane, c1 = lane + 64;
  const int ah = lane >> (6 - LG);
  const int ac0 = (lane & (LPH - 1)) * NCH;
  Dot8Wave<GQ, 4> W(L, a, h, wave, lane);
  const int kp = lane >> 5;
  const int jj = (lane >> 3) & 3, gg = (lane >> 1) & 3, hb = lane & 1;
  const int t0 = 16 * jj + 4 * gg + 2 * hb;  // this lane's tokens t0, t0 + 1 of page kp
  // weight digit bytes of this lane's token pair: word (head, page kp, 2 gg + jj / 2, d), byte 2 (jj & 1) + hb
  uint8_t* pw = W.pdig + (kp * 8 + 2 * gg + (jj >> 1)) * 16 + 2 * (jj & 1) + hb;
  const uint16_t* mk = W.mst + ((kp * 2 + 0) * 64 + t0) * 2;  // K (s, z) of token t0; + 2 for t0 + 1
  const uint16_t* mv = W.mst + ((kp * 2 + 1) * 64 + t0) * 2;

  auto issue_m = [&](int2 p) {
    dma16(W.mst_a, W.lane_page(p, lane >= 32) + ((lane & 16) ? I4_VMETA_OFF : I4_KMETA_OFF) + (lane & 15) * 16);
  };
  auto issue_k = [&](int2 p) {
    const uint8_t* src = W.lane_page(p, kp) + I4_K_OFF + t0 * 64;  // tokens t0, t0 + 1: 128 contiguous bytes
    dma16_off<0>(W.kst_a, src);
    dma16_off<16>(W.kst_a + 1024, src);
    dma16_off<32>(W.kst_a + 2048, src);
    dma16_off<48>(W.kst_a + 3072, src);
    dma16_off<64>(W.kst_a + 4096, src);
    dma16_off<80>(W.kst_a + 5120, src);
    dma16_off<96>(W.kst_a + 6144, src);
    dma16_off<112>(W.kst_a + 7168, src);
  };
  // pages of pair i; the second is the first again when the sequence ends in the first
  const int32_t* ptr = a.page_table + (long long)b * g.max_pages;
  // (scalar loads: a vector load here would enter the counter the copy pipeline's waits count)
  auto pages_of = [&](int i) {
    const int x = scalar_load_int(ptr + 2 * i);
    const int y = 2 * i + 1 < npages ? scalar_load_int(ptr + 2 * i + 1) : x;
    return make_int2(x, y);
  };

  // 0. the key-side operand, once
  float A[GQ], FS[GQ];
  {
    float qa[NCH];
    const float* q = a.qrot + ((long long)b * g.n_q + h * GQ + ah) * D + ac0;
#pragma unroll
    for (int i = 0; i < NCH; ++i) qa[i] = q[i];
    int amx_i = 0;
#pragma unroll
    for (int i = 0; i < NCH; ++i) amx_i = max(amx_i, __float_as_int(fabsf(qa[i])));
    const float amx = __int_as_float(seg_max_i<LPH>(amx_i));
    const float inv = amx > 0x1p-100f ? kScale8 * __builtin_amdgcn_rcpf(amx) : 0.0f;
    uint32_t pk[NCH / 2];
    float fsum = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; i += 2) {
      const float e0 = fmaf(qa[i], inv, kRoundA), e1 = fmaf(qa[i + 1], inv, kRoundA);
      fsum += (e0 - kRoundA) + (e1 - kRoundA);  // integers: exact
      pk[i >> 1] = pack_lo16(e0, e1);
    }
    const float fs = seg_sum<LPH>(fsum);
    const float Ah = amx * (1.0f / kScale8);
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      A[hh] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Ah), hh * LPH));
      FS[hh] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fs), hh * LPH));
    }
    store_key_operands<NCH / 2>(W.aval, ah, ac0, pk);
    wave_lds_sync();
    build_key_digits_seq<GQ>(W.adig, W.aval, lane);
    wave_lds_sync();
  }
  float m[GQ], l[GQ], o[GQ][2];
#pragma unroll
  for (int hh = 0; hh < GQ; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.0f;
    o[hh][0] = o[hh][1] = 0.0f;
  }
  // copies in flight as in int2_unit_dot8: M and K of a pair, its V once its K is read, the next K after V
  int2 pcur = make_int2(0, 0), pnext = make_int2(0, 0);
  if (p_first < pe) {
    pcur = pages_of(p_first);
    issue_m(pcur);
    issue_k(pcur);
  }
  for (int pi = p_first; pi < pe; pi += pstep) {
    const bool has_next = pi + pstep < pe;  // uniform
    if (has_next) pnext = pages_of(pi + pstep);
    KVQ_WAIT_VM(8);  // this pair's M copy (its K copies may still be in flight)
    const int tok = pi * 128 + kp * 64 + t0;
    const bool v0 = tok < T, v1 = tok + 1 < T;
    float sk[2], zk[2], svt[2], zvt[2];
    sk[0] = bf16_to_f32(mk[0]);
    zk[0] = bf16_to_f32(mk[1]);
    sk[1] = bf16_to_f32(mk[2]);
    zk[1] = bf16_to_f32(mk[3]);
    svt[0] = bf16_to_f32(mv[0]);
    zvt[0] = bf16_to_f32(mv[1]);
    svt[1] = bf16_to_f32(mv[2]);
    zvt[1] = bf16_to_f32(mv[3]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (has_next) issue_m(pnext);
    // tokens past the length: no weight, no value scale or zero (their metadata may be anything)
    svt[0] = v0 ? svt[0] : 0.0f;
    zvt[0] = v0 ? zvt[0] : 0.0f;
    svt[1] = v1 ? svt[1] : 0.0f;
    zvt[1] = v1 ? zvt[1] : 0.0f;

    // 1. key dots (this pair's K copies; the next pair's M may be in flight)
    if (has_next) KVQ_WAIT_VM(1);
    else KVQ_WAIT_VM(0);
    uint32_t kw[2][16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint4 kk = W.kst[64 * j + c0];
      uint32_t* dst = &kw[j >> 2][4 * (j & 3)];
      dst[0] = kk.x, dst[1] = kk.y, dst[2] = kk.z, dst[3] = kk.w;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    W.issue_v(pcur);  // into the buffer the key codes have left
    int acc[2][GQ][4];
    key_dots_seq<GQ>(W.adig, kw, acc);

    // 2. logits, pair max, weights p_t s'_t / S' as unsigned digits, sum_t p_t and sum_t u_t z'_t
    float lg[2][GQ], mg[GQ], Pl[GQ], Zs[GQ];
    {
      float mx[GQ];
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float x = (A[hh] * sk[t]) * fmaf(8.0f - zk[t], FS[hh], (float)digits_value(acc[t][hh]));
          lg[t][hh] = (t == 0 ? v0 : v1) ? x : -INFINITY;
        }
        mx[hh] = fmaxf(lg[0][hh], lg[1][hh]);
      }
      heads_allreduce<GQ>(mx, OpMax(), lane, mg);
    }
    // S'_h: the pair's largest weight p_t s'_t of head h (positive: the largest logit has p = 1)
    float p[2][GQ], Sw[GQ];
    {
      float sm[GQ];
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
        p[0][hh] = __builtin_amdgcn_exp2f(lg[0][hh] - mg[hh]);
        p[1][hh] = __builtin_amdgcn_exp2f(lg[1][hh] - mg[hh]);
        sm[hh] = fmaxf(p[0][hh] * svt[0], p[1][hh] * svt[1]);
      }
      heads_allreduce<GQ>(sm, OpMax(), lane, Sw);
    }
    {
      float ps[GQ], zs[GQ];
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
        const float r = Sw[hh] > 0.0f ? kScaleW / Sw[hh] : 0.0f;
        const float e0 = fmaf(p[0][hh] * svt[0], r, kRoundW), e1 = fmaf(p[1][hh] * svt[1], r, kRoundW);
        const uint32_t u0 = __float_as_uint(e0), u1 = __float_as_uint(e1);
        ps[hh] = p[0][hh] + p[1][hh];
        zs[hh] = fmaf(e0 - kRoundW, zvt[0], (e1 - kRoundW) * zvt[1]);
        const uint32_t x = nib_x(u0, u1), y = nib_y(u0, u1);
        uint8_t* q = pw + hh * 256;
        q[0] = (uint8_t)x;         // d0
        q[4] = (uint8_t)y;         // d1
        q[8] = (uint8_t)(x >> 8);  // d2
        q[12] = (uint8_t)(y >> 8); // d3
      }
      heads_allreduce<GQ>(ps, OpAdd(), lane, Pl);
      heads_allreduce<GQ>(zs, OpAdd(), lane, Zs);
    }
    wave_lds_sync();

    // 3. value dots
    KVQ_WAIT_VM(0);  // this pair's V copies, the youngest in flight
    uint32_t vw[2][2][8];  // [channel c0 | c1][page][word]
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint4 vv = W.vst[64 * j + c0];
      uint32_t* dst = &vw[(j >> 1) & 1][j >> 2][4 * (j & 1)];
      dst[0] = vv.x, dst[1] = vv.y, dst[2] = vv.z, dst[3] = vv.w;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (has_next) issue_k(pnext);
    int accv[2][GQ][4];
    value_dots_seq<GQ>(W.pdig, vw, accv);

    // 4. online-softmax update in the rotated value frame
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      const float mnew = fmax_raw(m[hh], mg[hh]);
      const float sc = __builtin_amdgcn_exp2f(m[hh] - mnew);  // 0 before the first pair (m = -inf)
      const float eg = __builtin_amdgcn_exp2f(mg[hh] - mnew);
      const float wg = eg * Sw[hh] * (1.0f / kScaleW);
      o[hh][0] = fmaf(o[hh][0], sc, wg * ((float)digits_value(accv[0][hh]) - Zs[hh]));
      o[hh][1] = fmaf(o[hh][1], sc, wg * ((float)digits_value(accv[1][hh]) - Zs[hh]));
      l[hh] = fmaf(l[hh], sc, eg * Pl[hh]);
      m[hh] = mnew;
    }
    wave_lds_sync();
    pcur = pnext;
  }
  if (wc) {
    if (pb < npairs && chunk_id < g.n_units - 1) store_wave_partial<GQ>(a, b, h, 1 + chunk_id, lane, m, l, o, c0, c1);
  } else {
    combine_and_store<GQ>(L, a, b, h, 1 + chunk, wave, lane, m, l, o, c0, c1);
  }
}

// ---------------------------------------------------------------------------------------------
// INT4 token-wise page walk, 16-bit fixed point on v_dot4 ([SAW] App. A.1 eq. (3)-(4), App. A.4 eq. (13)):
//   logit_t = s_t (sum_c q~_c code_tc - z_t sum_c q~_c): the key-side operand is the rotated query
//   itself, rounded once per work-group to a_c = rint(q~_c 32639 / max|q~|) (A = max|q~| / 32639),
//   so logit_t = A s_t (sum_c a_c code_tc - z_t sum_c a_c).
//   out_c = sum_t p_t s'_t (code'_tc - z'_t): the value-side weight w_t = p_t s'_t (p_t = 2^(logit_t -
//   max over the page) <= 1) is rounded to u_t = rint(65535 w_t / S'), S' = max over the page of w_t,
//   so out_c = (S' / 65535) (sum_t u_t code'_tc - sum_t u_t z'_t).
// Both 16-bit operands are split into two byte limbs as in int2_unit_dot16.  Lane roles: key token lane of
// the page; value channels lane, lane + 64.  Operand words in LDS:
//   key code word m (channels 8m .. 8m+7, channel c in byte (c/2) % 4, low nibble = even c):
//     (w >> 4n) & 0x0F0F0F0F holds channel 8m + 2j + n in byte j -> alpha word (2m + n), byte j;
//   value code word W of a channel (tokens 16j + 4g + r in byte 8g + 2j + r/2, nibble r % 2, W = 2g + j/2):
//     (w >> 4n) & 0x0F0F0F0F holds, in byte bw, token 16 (2 (W % 2) + bw / 2) + 4 (W / 2) + 2 (bw % 2) + n
//     -> weight word (2W + n), byte bw.
// ---------------------------------------------------------------------------------------------
template <int GQ, typename Lds>
__device__ void int4_unit_dot16(Lds& L, const DecodeArgs& a, int b, int h, int T, int chunk) {
  constexpr int LG = HeadLog2<GQ>::v;
  constexpr int LPH = 64 >> LG;
  constexpr int NCH = 2 * GQ;
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_pages = (T + PAGE - 1) / PAGE;
  const int p_begin = chunk * g.gpc;
  int p_end = (p_begin + g.gpc) < n_pages ? (p_begin + g.gpc) : n_pages;
  if (p_end > g.max_pages) p_end = g.max_pages;
  const int c0 = lane, c1 = lane + 64;
  uint8_t* abytes = L.d.abytes[wave];
  uint8_t* pbytes = L.d.pbytes[wave];

  // 1. key-side operand: the rotated query of each head, 16-bit, once for all pages of this chunk
  float A[GQ], QA[GQ];
  {
    const int ah = lane >> (6 - LG);
    const int ac0 = (lane & (LPH - 1)) * NCH;
    const float* q = a.qrot + ((long long)b * g.n_q + h * GQ + ah) * D + ac0;
    float qa[NCH];
    float amx = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      qa[i] = q[i];
      amx = fmaxf(amx, fabsf(qa[i]));
    }
    amx = seg_reduce<LPH>(amx, OpMax());
    const float inv = amx > 0.0f ? kAScale / amx : 0.0f;
    float qsum = 0.0f;
    uint8_t* lo = abytes + ah * 256;
    uint8_t* hi = lo + 128;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ai = (int)rintf(qa[i] * inv);
      qsum += (float)ai;
      const int c = ac0 + i;
      const int off = ((((c >> 3) * 2) + (c & 1)) << 2) + ((c >> 1) & 3);
      lo[off] = (uint8_t)ai;
      hi[off] = (uint8_t)((ai + 128) >> 8);
    }
    qsum = seg_reduce<LPH>(qsum, OpAdd());  // integers of magnitude < 2^22: exact
    const float Ah = amx * (1.0f / kAScale);
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      A[hh] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Ah), hh * LPH));
      QA[hh] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(qsum), hh * LPH));
    }
  }
  wave_lds_sync();

  float m[GQ], l[GQ], o[GQ][2];
#pragma unroll
  for (int hh = 0; hh < GQ; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.0f;
    o[hh][0] = o[hh][1] = 0.0f;
  }
  // token lane -> weight word (2W + n), byte bw
  const int tj = lane >> 4, tg = (lane >> 2) & 3, tr = lane & 3;
  const int pboff = ((2 * (2 * tg + (tj >> 1)) + (tr & 1)) << 2) + 2 * (tj & 1) + (tr >> 1);
  const long long hoff = (long long)h * I4_HEAD_BYTES;
  const int32_t* pt = a.page_table + (long long)b * g.max_pages;
  for (int pi = p_begin + wave; pi < p_end; pi += 4) {
    const uint8_t* pg = a.pages + (long long)pt[pi] * g.page_bytes + hoff;
    const int t = pi * PAGE + lane;
    const bool valid = t < T;
    const uint4* kr = reinterpret_cast<const uint4*>(pg + I4_K_OFF + lane * 64);
    const uint4 k0 = kr[0], k1 = kr[1], k2 = kr[2], k3 = kr[3];
    const uint4 v00 = reinterpret_cast<const uint4*>(pg + I4_V_OFF + c0 * 32)[0];
    const uint4 v01 = reinterpret_cast<const uint4*>(pg + I4_V_OFF + c0 * 32)[1];
    const uint4 v10 = reinterpret_cast<const uint4*>(pg + I4_V_OFF + c1 * 32)[0];
    const uint4 v11 = reinterpret_cast<const uint4*>(pg + I4_V_OFF + c1 * 32)[1];
    const uint32_t kmw = *reinterpret_cast<const uint32_t*>(pg + I4_KMETA_OFF + 4 * lane);
    const uint32_t vmw = *reinterpret_cast<const uint32_t*>(pg + I4_VMETA_OFF + 4 * lane);
    const float sk = __uint_as_float(kmw << 16), zk = __uint_as_float(kmw & 0xffff0000u);
    const float sv = __uint_as_float(vmw << 16), zv = __uint_as_float(vmw & 0xffff0000u);

    // 2. key dots
    int acc[GQ][2];
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) acc[hh][0] = acc[hh][1] = 0;
    const uint32_t kw[16] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w,
                             k2.x, k2.y, k2.z, k2.w, k3.x, k3.y, k3.z, k3.w};
#pragma unroll
    for (int mp = 0; mp < 8; ++mp) {  // pairs of code words (16 channels)
      const uint32_t e00 = kw[2 * mp] & 0x0F0F0F0Fu, e01 = (kw[2 * mp] >> 4) & 0x0F0F0F0Fu;
      const uint32_t e10 = kw[2 * mp + 1] & 0x0F0F0F0Fu, e11 = (kw[2 * mp + 1] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
#pragma unroll
        for (int lb = 0; lb < 2; ++lb) {
          const uint4 w = *reinterpret_cast<const uint4*>(abytes + hh * 256 + lb * 128 + mp * 16);
          int r = acc[hh][lb];
          r = __builtin_amdgcn_sdot4((int)w.x, (int)e00, r, false);
          r = __builtin_amdgcn_sdot4((int)w.y, (int)e01, r, false);
          r = __builtin_amdgcn_sdot4((int)w.z, (int)e10, r, false);
          r = __builtin_amdgcn_sdot4((int)w.w, (int)e11, r, false);
          acc[hh][lb] = r;
        }
      }
    }

    // 3. logits, page max, weights
    float lg[GQ], mg[GQ], psum[GQ], uz[GQ];
    {
      float mx[GQ];
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
        // sum_c a_c (code_tc - z_t) in integers (z_t is an integer for INT4), then one conversion
        const int lint = acc[hh][1] * 256 + acc[hh][0] - (valid ? (int)zk : 0) * (int)QA[hh];
        lg[hh] = valid ? (A[hh] * sk) * (float)lint : -INFINITY;
        mx[hh] = lg[hh];
      }
      heads_allreduce<GQ>(mx, OpMax(), lane, mg);
    }
    // S'_h: the page's largest weight p_t s'_t of head h (positive: the largest logit has p = 1); tokens
    // past the end of the sequence have weight 0, and their (unwritten) metadata is never read
    float pexp[GQ], Sw[GQ];
    {
      float sm[GQ];
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
        pexp[hh] = valid ? __builtin_amdgcn_exp2f(lg[hh] - mg[hh]) : 0.0f;
        sm[hh] = valid ? pexp[hh] * sv : 0.0f;
      }
      heads_allreduce<GQ>(sm, OpMax(), lane, Sw);
    }
    {
      float pp[GQ], zz[GQ];
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
        const float p = pexp[hh];
        const float rs = Sw[hh] > 0.0f ? 65535.0f / Sw[hh] : 0.0f;
        const uint32_t u = valid ? (uint32_t)fmaf(p * sv, rs, 0.5f) : 0u;
        pp[hh] = p;
        zz[hh] = valid ? (float)u * zv : 0.0f;
        uint8_t* lo = pbytes + hh * 256;
        lo[pboff] = (uint8_t)u;
        lo[pboff + 128] = (uint8_t)(u >> 8);
      }
      heads_allreduce<GQ>(pp, OpAdd(), lane, psum);
      heads_allreduce<GQ>(zz, OpAdd(), lane, uz);
    }
    wave_lds_sync();

    // 4. value dots: channels c0, c1; code word W of each channel against weight words (2W, 2W + 1)
    uint32_t accv[2][GQ][2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) accv[c][hh][0] = accv[c][hh][1] = 0u;
    const uint32_t vw[2][8] = {{v00.x, v00.y, v00.z, v00.w, v01.x, v01.y, v01.z, v01.w},
                               {v10.x, v10.y, v10.z, v10.w, v11.x, v11.y, v11.z, v11.w}};
#pragma unroll
    for (int wp = 0; wp < 4; ++wp) {  // pairs of code words
      uint32_t e[2][4];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        e[c][0] = vw[c][2 * wp] & 0x0F0F0F0Fu;
        e[c][1] = (vw[c][2 * wp] >> 4) & 0x0F0F0F0Fu;
        e[c][2] = vw[c][2 * wp + 1] & 0x0F0F0F0Fu;
        e[c][3] = (vw[c][2 * wp + 1] >> 4) & 0x0F0F0F0Fu;
      }
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
#pragma unroll
        for (int lb = 0; lb < 2; ++lb) {
          const uint4 w = *reinterpret_cast<const uint4*>(pbytes + hh * 256 + lb * 128 + wp * 16);
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            uint32_t r = accv[c][hh][lb];
            r = __builtin_amdgcn_udot4(w.x, e[c][0], r, false);
            r = __builtin_amdgcn_udot4(w.y, e[c][1], r, false);
            r = __builtin_amdgcn_udot4(w.z, e[c][2], r, false);
            r = __builtin_amdgcn_udot4(w.w, e[c][3], r, false);
            accv[c][hh][lb] = r;
          }
        }
      }
    }

    // 5. online-softmax update (rotated value frame)
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      const float mnew = fmaxf(m[hh], mg[hh]);
      const float sc = exp2_safe_diff(m[hh], mnew);
      const float wpg = exp2_safe_diff(mg[hh], mnew);
      const float ws = wpg * Sw[hh] * (1.0f / 65535.0f);
      const float U0 = (float)(accv[0][hh][1] * 256u + accv[0][hh][0]);
      const float U1 = (float)(accv[1][hh][1] * 256u + accv[1][hh][0]);
      o[hh][0] = fmaf(o[hh][0], sc, ws * (U0 - uz[hh]));
      o[hh][1] = fmaf(o[hh][1], sc, ws * (U1 - uz[hh]));
      l[hh] = fmaf(l[hh], sc, wpg * psum[hh]);
      m[hh] = mnew;
    }
    wave_lds_sync();
  }
  combine_and_store<GQ>(L, a, b, h, 1 + chunk, wave, lane, m, l, o, c0, c1);
}

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
    const uint8_t* pg = a.pages + (long long)pt[pi] * g.page_bytes + hoff;
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
// INT2 per-channel chunk on the int8 matrix cores (v_mfma_i32_16x16x64_i8).  The fixed-point algebra is
// that of int2_unit_dot16: per group and head the key-side operand a = rint(alpha 32639 / max|alpha|),
// alpha = q~ s, and the softmax weights u = rint(32511 p), p = 2^(logit - group max), each as two signed
// byte limbs 256 hi + lo; with A = max|alpha| / 32639,
//   logit_t = A (sum_c a_c code_tc - sum_c a_c z_c),
//   o~_c   += (2^(group max - m) / 32511) s_c (sum_t u_t code_tc - z_c sum_t u_t).
// Both sums are 16 x 16 x 64 matrix products whose rows are (head, limb) pairs, so the GQA heads that share
// the kv head also share one pass over the codes ([SAW] App. A.4 eq. 13-14; [NOVA] §2 query groups):
//   keys    D[(head, limb)][token]   = sum_channels limb(a) code, 8 token tiles x 2 channel halves;
//   values  D[(head, limb)][channel] = sum_tokens limb(u) code, 8 channel tiles x 2 pages;
// and sum_t u_t is one more product against a vector of ones.  The limbs are exact int32 sums and the
// codes stay 2-bit in HBM: each 32-bit code word becomes four int8 vectors, (w >> 2n) & 0x03030303.
// Matrix rows: head h, limb L at row 4 h + L (GQ <= 4; rows with L >= 2 are zero) or 2 h + L (GQ = 8).
// Operand layouts (lane l, q = l / 16, c = l % 16): A row c, k = 16 q + byte; B the same k, column c;
// D column c, rows 4 q + r.  So a lane's key results (head(s) of rows 4 q.., token column c) are its
// weights' producer lane, and its value results hold head q's channels c + 16 tau.
//  - key k order (k = 64 sigma + 16 q + 4 n + b): channel 16 (2 q + sigma) + 4 b + n, i.e. lane q expands
//    code words 2 q, 2 q + 1 of a token (channel 16 m + 4 b + n in byte b, bits 2 n);
//  - value k order (k = 64 kappa + 16 q + 4 n + b): token 64 kappa + 16 b + 4 q + n of page kappa, i.e. lane
//    q expands code word q of a channel (token 16 b + 4 q + n in byte b, bits 2 n);
//  - key tile i, column c: token T(i, c) = 64 (c / 8) + 2 (c % 8) + 16 (i % 4) + i / 4, the token at value
//    position 8 c + i, so each lane stores its 8 weights of a head as 8 consecutive bytes of the weight plane.
// Key codes are staged with their rows permuted (token t at row t ^ ((t >> 2) & 3)) so that the 8-byte
// operand reads of a tile spread over all LDS banks.  All global reads are LDS copies: a group's metadata
// one group ahead, its key codes while the previous group's values are multiplied, and its value codes,
// into the buffer the keys leave, while its keys are multiplied; the waits count the copies.
// ---------------------------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(4))) int mf_i32x4;

__device__ __forceinline__ mf_i32x4 mfma_i8x64(mf_i32x4 a, mf_i32x4 b, mf_i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}
// 16 2-bit codes as 16 int8 values: dword n holds field n of every byte
__device__ __forceinline__ mf_i32x4 codes_i8(uint32_t w) {
  return mf_i32x4{(int)(w & 0x03030303u), (int)((w >> 2) & 0x03030303u), (int)((w >> 4) & 0x03030303u),
                  (int)((w >> 6) & 0x03030303u)};
}
__device__ __forceinline__ mf_i32x4 u4_i32x4(uint4 v) { return mf_i32x4{(int)v.x, (int)v.y, (int)v.z, (int)v.w}; }
// lo + 256 hi of two int32 limb sums (two's complement).  Plain code, not inline assembly: its operands
// are matrix-core results, and only instructions the compiler emits itself get the wait states that
// reading those registers needs.
__device__ __forceinline__ int limbs_sum(int lo, int hi) { return (int)((uint32_t)lo + ((uint32_t)hi << 8)); }
// Magic rounding with the limb bias: fp32(x + 1.5 * 2^23 + 128) has rint(x) + 128 in the low half of its
// encoding (|x| <= 32639), whose low byte xor 0x80 is the signed limb lo = x mod 256 and whose high byte is
// hi = (x + 128) >> 8 in [-128, 127].
constexpr float kRoundL = 12582912.0f + 128.0f;
__device__ __forceinline__ void limbs4(float e0, float e1, float e2, float e3, uint32_t& lo, uint32_t& hi) {
  const uint32_t p01 = pack_lo16(e0, e1), p23 = pack_lo16(e2, e3);
  lo = __builtin_amdgcn_perm(p23, p01, 0x06040200u) ^ 0x80808080u;
  hi = __builtin_amdgcn_perm(p23, p01, 0x07050301u);
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
__device__ void int2_unit_mfma(Lds& L, const DecodeArgs& a, int b, int h, int T, int chunk) {
  constexpr int LG = HeadLog2<GQ>::v;
  constexpr int LPH = 64 >> LG;        // lanes per head in the alpha step
  constexpr int NCH = 2 * GQ;          // key positions per lane in the alpha step
  constexpr int RPH = GQ == 8 ? 2 : 4;  // matrix rows per head
  constexpr int HPL = GQ == 8 ? 2 : 1;  // heads per lane in the results
  constexpr int ROWS = 2 * GQ;
  constexpr int KU = 128 * BITS;  // staging of a group's key or value codes, in 16-byte units
  constexpr int NCP = KU / 64;    // copies per group and side
  constexpr int RS = MfmaWave<GQ, KU>::RSTRIDE;
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ng = n_groups_of(T, g.S0, g.W);
  const bool wc = g.wave_chunks != 0;
  const int chunk_id = wc ? 4 * chunk + wave : chunk;
  const int g_begin = chunk_id * g.gpc;
  int g_end = (g_begin + g.gpc) < ng ? (g_begin + g.gpc) : ng;
  if (g_end > g.max_pages / 2) g_end = g.max_pages / 2;  // never index past the page-table row
  const int gstep = wc ? 1 : 4;
  const int g_first = wc ? g_begin : g_begin + wave;
  MfmaWave<GQ, KU>& W = L.mf.w[wave];
  const int q4 = lane >> 4, c = lane & 15;

  // the rows no head fills read the zero row of each plane
  if (lane < 32) {
    reinterpret_cast<uint32_t*>(W.aplane + ROWS * RS)[lane] = 0u;
    reinterpret_cast<uint32_t*>(W.wplane + ROWS * RS)[lane] = 0u;
  }
  // A-operand row of this lane: matrix row c = (head, limb)
  const int rh = c / RPH, rl = c % RPH;
  const int prow = (rl < 2 && rh < GQ) ? 2 * rh + rl : ROWS;
  const uint8_t* a_rd = W.aplane + prow * RS + 16 * q4;
  const uint8_t* w_rd = W.wplane + prow * RS + 16 * q4;
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
  const uint32_t* v_rd = reinterpret_cast<const uint32_t*>(W.kst) + (BITS == 2 ? 4 * c + q4 : 8 * c + 2 * q4);
  // alpha step: head ah, key positions Q0 .. Q0 + NCH - 1
  const int ah = lane >> (6 - LG);
  const int Q0 = (lane & (LPH - 1)) * NCH;
  // copies: per-lane offsets of the permuted key rows (copy j: page j / 2, 16-byte slots 64 j + lane, i.e.
  // half lane % 2 of staged row 32 (j % 2) + lane / 2 of that page)
  uint32_t koff[2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int tl = 32 * jj + ((lane >> 1) ^ ((lane >> 3) & 3));
    koff[jj] = (uint32_t)(tl * 32 + 16 * (lane & 1));
  }
  const uint32_t kst_a = lds_addr(W.kst);
  const uint32_t mst_a0 = lds_addr(W.mst[0]), mst_a1 = lds_addr(W.mst[1]);
  const uint8_t* pages = a.pages;
  const long long pbytes = g.page_bytes, hoff = (long long)h * g.head_bytes;
  auto page_of = [&](int idx) { return pages + (long long)idx * pbytes + hoff; };
  constexpr int META = BITS == 2 ? I2_META_OFF : I4C_META_OFF;
  constexpr int KOFF = BITS == 2 ? I2_K_OFF : I4C_K_OFF, VOFF = BITS == 2 ? I2_V_OFF : I4C_V_OFF;
  auto issue_m = [&](int2 p, int buf) {
    const uint8_t* src = (lane >= 32 ? page_of(p.y) : page_of(p.x)) + META + (lane & 31) * 16;
    dma16(buf ? mst_a1 : mst_a0, src);
  };
  auto issue_k = [&](int2 p) {
    if constexpr (BITS == 2) {
#pragma unroll
      for (int j = 0; j < 4; ++j) dma16_base(kst_a + 1024 * j, page_of(j < 2 ? p.x : p.y) + KOFF, koff[j & 1]);
    } else {
#pragma unroll
      for (int j = 0; j < NCP; ++j)
        dma16_base(kst_a + 1024 * j, page_of(j < NCP / 2 ? p.x : p.y) + KOFF + 1024 * (j % (NCP / 2)), lane * 16);
    }
  };
  auto issue_v = [&](int2 p) {
#pragma unroll
    for (int j = 0; j < NCP; ++j)
      dma16_base(kst_a + 1024 * j, page_of(j < NCP / 2 ? p.x : p.y) + VOFF + 1024 * (j % (NCP / 2)), lane * 16);
  };

  float qa[NCH];
  {
    const float* q = a.qrot + ((long long)b * g.n_q + h * GQ + ah) * D;
#pragma unroll
    for (int i = 0; i < NCH; ++i) qa[i] = q[BITS == 2 ? mf_key_channel(Q0 + i) : mf_key_channel_c4(Q0 + i)];
#pragma unroll
    for (int i = 0; i < NCH; ++i) asm volatile("" ::"v"(qa[i]));  // the loads' wait stays before the walk
  }
  // key-side operand x (positions Q0 + i of head ah) rounded to 16 bits against its head's largest |x|, as
  // limbs in the key plane; returns the scale A = max|x| / 32639, and in zsum the sum of the rounded values
  // times zk (per channel; 1 gives their plain sum)
  auto key_operand = [&](const float (&x)[NCH], const float (&zk)[NCH], float& zsum) -> float {
    int amx_i = 0;  // max |x| as its bit pattern (non-negative floats order as their bits)
#pragma unroll
    for (int i = 0; i < NCH; ++i) amx_i = max(amx_i, __float_as_int(fabsf(x[i])));
    const float amx = __int_as_float(seg_max_i<LPH>(amx_i));
    // |rint(x inv)| <= 32639: the reciprocal's 1-ulp error cannot carry the largest past 32639.5
    const float inv = amx > 0x1p-100f ? kAScale * __builtin_amdgcn_rcpf(amx) : 0.0f;
    float ev[NCH];
    float zs = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      ev[i] = fmaf(x[i], inv, kRoundL);
      zs = fmaf(ev[i] - kRoundL, zk[i], zs);  // with the rounded values: exact products of integers up to 2^15
    }
    zsum = seg_sum<LPH>(zs);
    uint8_t* dst0 = W.aplane + (2 * ah) * RS + Q0;
    uint8_t* dst1 = dst0 + RS;
    if constexpr (NCH >= 4) {
      uint32_t lo[NCH / 4], hi[NCH / 4];
#pragma unroll
      for (int k = 0; k < NCH / 4; ++k) limbs4(ev[4 * k], ev[4 * k + 1], ev[4 * k + 2], ev[4 * k + 3], lo[k], hi[k]);
      if constexpr (NCH == 16) {
        *reinterpret_cast<uint4*>(dst0) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        *reinterpret_cast<uint4*>(dst1) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      } else if constexpr (NCH == 8) {
        *reinterpret_cast<uint2*>(dst0) = make_uint2(lo[0], lo[1]);
        *reinterpret_cast<uint2*>(dst1) = make_uint2(hi[0], hi[1]);
      } else {
        *reinterpret_cast<uint32_t*>(dst0) = lo[0];
        *reinterpret_cast<uint32_t*>(dst1) = hi[0];
      }
    } else {
      uint32_t lo, hi;
      limbs4(ev[0], ev[1], ev[0], ev[1], lo, hi);
      *reinterpret_cast<uint16_t*>(dst0) = (uint16_t)lo;
      *reinterpret_cast<uint16_t*>(dst1) = (uint16_t)hi;
    }
    return amx * (1.0f / kAScale);
  };
  // per-head values of this lane's result heads (head q4 HPL + e is the key step's lanes (q4 HPL + e) LPH)
  auto head_value = [&](float v, int e) { return __shfl(v, ((q4 * HPL + e) & (GQ - 1)) * LPH, 64); };
  // per-token INT2: the key-side operand is the rotated query itself, once per walk
  float At[HPL], FSt[HPL];
  mf_i32x4 A0t = {0, 0, 0, 0}, A1t = {0, 0, 0, 0};
  if constexpr (TOK) {
    float one[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) one[i] = 1.0f;
    float fs;
    const float Ah = key_operand(qa, one, fs);
#pragma unroll
    for (int e = 0; e < HPL; ++e) {
      At[e] = head_value(Ah, e);
      FSt[e] = head_value(fs, e);
    }
    wave_lds_sync();
    A0t = u4_i32x4(*reinterpret_cast<const uint4*>(a_rd));
    A1t = u4_i32x4(*reinterpret_cast<const uint4*>(a_rd + 64));
  }
  float m[HPL], l[HPL], o[HPL][8];
#pragma unroll
  for (int e = 0; e < HPL; ++e) {
    m[e] = -INFINITY;
    l[e] = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) o[e][t] = 0.0f;
  }
  const int2* pt = reinterpret_cast<const int2*>(a.page_table + (long long)b * g.max_pages);
  int2 pcur = make_int2(0, 0), pnext = make_int2(0, 0);
  int mb = 0;
  if (g_first < g_end) {
    pcur = scalar_load_int2(pt + g_first);
    issue_m(pcur, 0);
    issue_k(pcur);
  }
  wave_lds_sync();
  const mf_i32x4 zero4 = {0, 0, 0, 0};
  const mf_i32x4 ones4 = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
  for (int gi = g_first; gi < g_end; gi += gstep) {
    const bool has_next = gi + gstep < g_end;  // uniform
    if (has_next) pnext = scalar_load_int2(pt + gi + gstep);
    // this group's metadata (its key copies may be in flight)
    if constexpr (NCP == 4) KVQ_WAIT_VM(4);
    else KVQ_WAIT_VM(8);
    const uint16_t* ms = reinterpret_cast<const uint16_t*>(W.mst[mb]);
    // 1. per channel: key-side operand alpha = q~ s of head ah at positions Q0 + i, two limbs;
    //    per token: the group's token scales and zeros (tokens T(i, c) of the lane's page c / 8)
    float Ae[HPL], AZe[HPL];
    float tks[8], tkz[8], tvs[8], tvz[8];
    if constexpr (TOK) {
      // tokens 2 (c % 8) + 16 k + {0, 1} of page c / 8: one word per pair; K s, K z, V s, V z at 0, 64, 128, 192
      const uint32_t* mw = reinterpret_cast<const uint32_t*>(ms + 256 * (c >> 3) + 2 * (c & 7));
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t w0 = mw[8 * k], w1 = mw[8 * k + 32], w2 = mw[8 * k + 64], w3 = mw[8 * k + 96];
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
            const int ch = mf_key_channel(Q0 + i);
            const uint32_t sw = reinterpret_cast<const uint32_t*>(ms)[ch >> 1];
            const uint32_t zw = reinterpret_cast<const uint32_t*>(ms + D)[ch >> 1];
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
      const float Ah = key_operand(al, zk, zs);
      const float AZh = Ah * zs;
#pragma unroll
      for (int e = 0; e < HPL; ++e) {
        Ae[e] = head_value(Ah, e);
        AZe[e] = head_value(AZh, e);
      }
    }
    if (has_next) issue_m(pnext, mb ^ 1);
    wave_lds_sync();

    // 2. key products: 8 token tiles x 2 channel halves
    if (has_next) KVQ_WAIT_VM(1);  // this group's key copies (the next metadata follows)
    else KVQ_WAIT_VM(0);
    uint4 kw[8];  // 2-bit: .x, .y; 4-bit: all four words
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (BITS == 2) {
        const uint2 t2 = *reinterpret_cast<const uint2*>((i < 4 ? k_rd0 : k_rd1) + 512 * (i & 3));
        kw[i] = make_uint4(t2.x, t2.y, 0u, 0u);
      } else {
        kw[i] = *reinterpret_cast<const uint4*>((i < 4 ? k_rd0 : k_rd1) + 1024 * (i & 3));
      }
    }
    const mf_i32x4 A0 = TOK ? A0t : u4_i32x4(*reinterpret_cast<const uint4*>(a_rd));
    const mf_i32x4 A1 = TOK ? A1t : u4_i32x4(*reinterpret_cast<const uint4*>(a_rd + 64));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    issue_v(pcur);  // into the buffer the key codes have left
    mf_i32x4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc[i] = mfma_i8x64(A0, BITS == 2 ? codes_i8(kw[i].x) : nibbles_i8(kw[i].x, kw[i].y), zero4);
      acc[i] = mfma_i8x64(A1, BITS == 2 ? codes_i8(kw[i].y) : nibbles_i8(kw[i].z, kw[i].w), acc[i]);
    }

    // 3. per channel: logit = A val - AZ, the group maximum is that of the integer sums (A >= 0), weights
    //    u = rint(32511 2^(A (val - val_max))); per token: logit_t = A s_t (val_t - z_t sum_c a_c), weights
    //    u_t = rint(32511 p_t s'_t / S') with S' the group's largest p_t s'_t of the head, their sums
    //    P = sum_t p_t and Z = sum_t u_t z'_t; weights as limbs at positions 8 c + i of the weight plane
    float mg[HPL], Sg[HPL], Pt[HPL], Zt[HPL];
#pragma unroll
    for (int e = 0; e < HPL; ++e) {
      float ew[8];
      if constexpr (TOK) {
        float lg[8];
        float lmx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          lg[i] = (Ae[e] * tks[i]) * fmaf(-tkz[i], AZe[e], (float)limbs_sum(acc[i][2 * e], acc[i][2 * e + 1]));
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
        const float r = Sg[e] > 0x1p-100f ? kPScale * __builtin_amdgcn_rcpf(Sg[e]) : 0.0f;
        float zs = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          ew[i] = fmaf(pw[i], r, kRoundL);
          zs = fmaf(ew[i] - kRoundL, tvz[i], zs);
        }
        Zt[e] = seg_sum<16>(zs);
      } else {
      int v[8];
      int vmx = (int)0x80000000u;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[i] = limbs_sum(acc[i][2 * e], acc[i][2 * e + 1]);
        vmx = max(vmx, v[i]);
      }
      vmx = seg_max_i<16>(vmx);
      const float ref = Ae[e] * (float)vmx;
      mg[e] = ref - AZe[e];
#pragma unroll
      for (int i = 0; i < 8; ++i) ew[i] = fmaf(__builtin_amdgcn_exp2f(fmaf(Ae[e], (float)v[i], -ref)), kPScale, kRoundL);
      }
      uint32_t lo0, hi0, lo1, hi1;
      limbs4(ew[0], ew[1], ew[2], ew[3], lo0, hi0);
      limbs4(ew[4], ew[5], ew[6], ew[7], lo1, hi1);
      const int he = q4 * HPL + e;
      if (he < GQ) {
        uint8_t* dst = W.wplane + (2 * he) * RS + 8 * c;
        *reinterpret_cast<uint2*>(dst) = make_uint2(lo0, lo1);
        *reinterpret_cast<uint2*>(dst + RS) = make_uint2(hi0, hi1);
      }
    }
    wave_lds_sync();

    // 4. value products: 8 channel tiles x 2 pages, and the weight sums
    KVQ_WAIT_VM(0);  // this group's value copies, the youngest in flight
    uint2 vw[8][2];  // 2-bit: .x; 4-bit: both words
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if constexpr (BITS == 2) {
        vw[t][0] = make_uint2(v_rd[64 * t], 0u);
        vw[t][1] = make_uint2(v_rd[512 + 64 * t], 0u);
      } else {
        vw[t][0] = *reinterpret_cast<const uint2*>(v_rd + 128 * t);
        vw[t][1] = *reinterpret_cast<const uint2*>(v_rd + 1024 + 128 * t);
      }
    }
    const mf_i32x4 W0 = u4_i32x4(*reinterpret_cast<const uint4*>(w_rd));
    const mf_i32x4 W1 = u4_i32x4(*reinterpret_cast<const uint4*>(w_rd + 64));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (has_next) issue_k(pnext);
    mf_i32x4 accp = zero4;
    if constexpr (!TOK) {
      accp = mfma_i8x64(W0, ones4, zero4);
      accp = mfma_i8x64(W1, ones4, accp);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      acc[t] = mfma_i8x64(W0, BITS == 2 ? codes_i8(vw[t][0].x) : nibbles_i8(vw[t][0].x, vw[t][0].y), zero4);
      acc[t] = mfma_i8x64(W1, BITS == 2 ? codes_i8(vw[t][1].x) : nibbles_i8(vw[t][1].x, vw[t][1].y), acc[t]);
    }

    // 5. online-softmax update in the rotated value frame (per channel: o and l carry the weights' factor
    //    32511; per token: the group adds (S' / 32511) (U_c - Z) to o and P to l)
#pragma unroll
    for (int e = 0; e < HPL; ++e) {
      const float mnew = fmax_raw(m[e], mg[e]);
      const float sc = __builtin_amdgcn_exp2f(m[e] - mnew);  // 0 before the first group (m = -inf)
      const float eg = __builtin_amdgcn_exp2f(mg[e] - mnew);
      if constexpr (TOK) {
        const float wg = eg * Sg[e] * (1.0f / kPScale);
#pragma unroll
        for (int t = 0; t < 8; ++t)
          o[e][t] = fmaf(o[e][t], sc, wg * ((float)limbs_sum(acc[t][2 * e], acc[t][2 * e + 1]) - Zt[e]));
        l[e] = fmaf(l[e], sc, eg * Pt[e]);
        m[e] = mnew;
        continue;
      }
      const float Pf = (float)limbs_sum(accp[2 * e], accp[2 * e + 1]);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int ch = c + 16 * t;
        const float sv = bf16_to_f32(ms[2 * D + ch]), zv = bf16_to_f32(ms[3 * D + ch]);
        const float Y = fmaf(-zv, Pf, (float)limbs_sum(acc[t][2 * e], acc[t][2 * e + 1]));
        o[e][t] = fmaf(eg * sv, Y, o[e][t] * sc);
      }
      l[e] = fmaf(eg, Pf, l[e] * sc);
      m[e] = mnew;
    }
    mb ^= 1;
    pcur = pnext;
  }
  if constexpr (!TOK) {
#pragma unroll
    for (int e = 0; e < HPL; ++e) {
#pragma unroll
      for (int t = 0; t < 8; ++t) o[e][t] *= 1.0f / kPScale;
      l[e] *= 1.0f / kPScale;
    }
  }
  if (wc) {
    // every partial a merge reads is written; chunks past the length or the launch bound have none
    if (g_begin < ng && chunk_id < g.n_units - 1) {
#pragma unroll
      for (int e = 0; e < HPL; ++e) {
        const int he = q4 * HPL + e;
        if (he < GQ) {
          float* part = a.partials + (((long long)b * g.n_q + h * GQ + he) * g.n_units + 1 + chunk_id) * PART_STRIDE;
#pragma unroll
          for (int t = 0; t < 8; ++t) part[2 + c + 16 * t] = o[e][t];
          if (c == 0) {
            part[0] = m[e];
            part[1] = l[e];
          }
        }
      }
    }
  } else {
    __syncthreads();  // co shares its LDS with the walks' buffers
#pragma unroll
    for (int e = 0; e < HPL; ++e) {
      const int he = q4 * HPL + e;
      if (he < GQ) {
#pragma unroll
        for (int t = 0; t < 8; ++t) L.co[wave][he][c + 16 * t] = o[e][t];
        if (c == 0) {
          L.cm[wave][he] = m[e];
          L.cl[wave][he] = l[e];
        }
      }
    }
    combine_waves<GQ>(L, a, b, h, 1 + chunk);
  }
}

// ---------------------------------------------------------------------------------------------
// INT4 per-token chunk ([SAW] App. A.1 token-wise INT4, eq. 13-14) on the int8 matrix cores: the per-token
// INT2 unit's algebra (key-side operand = the rotated query, two limbs, once per walk; logit_t = A s_t
// (D_t - z_t sum_c a_c); weights u_t = rint(32511 p_t s'_t / S')) over page pairs (128 tokens) of 4-bit
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
__device__ void int4tok_unit_mfma(Lds& L, const DecodeArgs& a, int b, int h, int T, int chunk) {
  constexpr int LG = HeadLog2<GQ>::v;
  constexpr int LPH = 64 >> LG;
  constexpr int NCH = 2 * GQ;
  constexpr int RPH = GQ == 8 ? 2 : 4;
  constexpr int HPL = GQ == 8 ? 2 : 1;
  constexpr int ROWS = 2 * GQ;
  constexpr int RS = MfmaWave<GQ, 512>::RSTRIDE;
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int npages = (T + PAGE - 1) / PAGE;
  const int npairs = (npages + 1) / 2;
  const int chunk_id = 4 * chunk + wave;  // one chunk (an even number of pages) per wave
  const int pb = chunk_id * (g.gpc / 2);
  int pe = pb + g.gpc / 2 < npairs ? pb + g.gpc / 2 : npairs;
  if (2 * pe > g.max_pages + 1) pe = (g.max_pages + 1) / 2;  // never index past the page-table row
  MfmaWave<GQ, 512>& W = L.mf.w[wave];
  const int q4 = lane >> 4, c = lane & 15;

  if (lane < 32) {
    reinterpret_cast<uint32_t*>(W.aplane + ROWS * RS)[lane] = 0u;
    reinterpret_cast<uint32_t*>(W.wplane + ROWS * RS)[lane] = 0u;
  }
  const int rh = c / RPH, rl = c % RPH;
  const int prow = (rl < 2 && rh < GQ) ? 2 * rh + rl : ROWS;
  const uint8_t* a_rd = W.aplane + prow * RS + 16 * q4;
  const uint8_t* w_rd = W.wplane + prow * RS + 16 * q4;
  // key operand reads: tile i at staged row 64 (c / 8) + 32 (c % 2) + 4 ((c / 2) % 4) + (y ^ (i / 4)) plus
  // 16 ((i / 2) % 2) + 2 (i % 2), with y = (c / 2) % 2
  const int y = (c >> 1) & 1;
  const int krow = 64 * (c >> 3) + 32 * (c & 1) + 4 * ((c >> 1) & 3);
  const uint8_t* k_rd0 = reinterpret_cast<const uint8_t*>(W.kst) + 64 * (krow + y) + 16 * q4;
  const uint8_t* k_rd1 = reinterpret_cast<const uint8_t*>(W.kst) + 64 * (krow + (y ^ 1)) + 16 * q4;
  // value operand reads: channel c + 16 tau, code words 2 q4, 2 q4 + 1, page kappa
  const uint8_t* v_rd = reinterpret_cast<const uint8_t*>(W.kst) + 32 * c + 8 * q4;
  // this lane's tokens T(i, c) (pair-local), their metadata words: K (s, z) at (2 page) 64 + t, V at + 64
  const int tok0 = 64 * (c >> 3) + 32 * (c & 1) + 4 * ((c >> 1) & 3);
  const int ah = lane >> (6 - LG);
  const int Q0 = (lane & (LPH - 1)) * NCH;
  // copies: key slots 64 j + lane hold staged row 16 j + lane / 4, quarter lane % 4
  const uint32_t koff = (uint32_t)(64 * ((lane >> 2) ^ ((lane >> 4) & 1)) + 16 * (lane & 3));
  const uint32_t kst_a = lds_addr(W.kst);
  const uint32_t mst_a0 = lds_addr(W.mst[0]), mst_a1 = lds_addr(W.mst[1]);
  const uint8_t* pages = a.pages;
  const long long pbytes = g.page_bytes, hoff = (long long)h * g.head_bytes;
  auto page_of = [&](int idx) { return pages + (long long)idx * pbytes + hoff; };
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
      dma16_base(kst_a + 1024 * j, page_of(j < 4 ? p.x : p.y) + I4_V_OFF + 1024 * (j & 3), lane * 16);
  };
  const int32_t* ptr = a.page_table + (long long)b * g.max_pages;
  auto pages_of = [&](int i) {  // scalar loads: a vector load would enter the counter the waits count
    const int x = scalar_load_int(ptr + 2 * i);
    const int yy = 2 * i + 1 < npages ? scalar_load_int(ptr + 2 * i + 1) : x;
    return make_int2(x, yy);
  };

  // 0. the key-side operand, once: the rotated query of head ah at positions Q0 + i, two limbs
  float At[HPL], FSt[HPL];
  mf_i32x4 A0, A1;
  {
    float qa[NCH];
    const float* q = a.qrot + ((long long)b * g.n_q + h * GQ + ah) * D;
#pragma unroll
    for (int i = 0; i < NCH; ++i) qa[i] = q[mf_key_channel4(Q0 + i)];
    int amx_i = 0;
#pragma unroll
    for (int i = 0; i < NCH; ++i) amx_i = max(amx_i, __float_as_int(fabsf(qa[i])));
    const float amx = __int_as_float(seg_max_i<LPH>(amx_i));
    const float inv = amx > 0x1p-100f ? kAScale * __builtin_amdgcn_rcpf(amx) : 0.0f;
    float ev[NCH];
    float fs = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      ev[i] = fmaf(qa[i], inv, kRoundL);
      fs += ev[i] - kRoundL;  // integers: exact
    }
    fs = seg_sum<LPH>(fs);
    const float Ah = amx * (1.0f / kAScale);
    uint8_t* dst0 = W.aplane + (2 * ah) * RS + Q0;
    uint8_t* dst1 = dst0 + RS;
    if constexpr (NCH >= 4) {
      uint32_t lo[NCH / 4], hi[NCH / 4];
#pragma unroll
      for (int k = 0; k < NCH / 4; ++k) limbs4(ev[4 * k], ev[4 * k + 1], ev[4 * k + 2], ev[4 * k + 3], lo[k], hi[k]);
#pragma unroll
      for (int k = 0; k < NCH / 4; ++k) {
        reinterpret_cast<uint32_t*>(dst0)[k] = lo[k];
        reinterpret_cast<uint32_t*>(dst1)[k] = hi[k];
      }
    } else {
      uint32_t lo, hi;
      limbs4(ev[0], ev[1], ev[0], ev[1], lo, hi);
      *reinterpret_cast<uint16_t*>(dst0) = (uint16_t)lo;
      *reinterpret_cast<uint16_t*>(dst1) = (uint16_t)hi;
    }
#pragma unroll
    for (int e = 0; e < HPL; ++e) {
      const int src = ((q4 * HPL + e) & (GQ - 1)) * LPH;
      At[e] = __shfl(Ah, src, 64);
      FSt[e] = __shfl(fs, src, 64);
    }
    wave_lds_sync();
    A0 = u4_i32x4(*reinterpret_cast<const uint4*>(a_rd));
    A1 = u4_i32x4(*reinterpret_cast<const uint4*>(a_rd + 64));
  }
  float m[HPL], l[HPL], o[HPL][8];
#pragma unroll
  for (int e = 0; e < HPL; ++e) {
    m[e] = -INFINITY;
    l[e] = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) o[e][t] = 0.0f;
  }
  int2 pcur = make_int2(0, 0), pnext = make_int2(0, 0);
  int mb = 0;
  if (pb < pe) {
    pcur = pages_of(pb);
    issue_m(pcur, 0);
    issue_k(pcur);
  }
  wave_lds_sync();
  const mf_i32x4 zero4 = {0, 0, 0, 0};
  for (int pi = pb; pi < pe; ++pi) {
    const bool has_next = pi + 1 < pe;  // uniform
    if (has_next) pnext = pages_of(pi + 1);
    KVQ_WAIT_VM(8);  // this pair's metadata (its key copies may be in flight)
    // 1. the lane's tokens: K and V (scale, zero) words, validity
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
    if (has_next) issue_m(pnext, mb ^ 1);

    // 2. key products: 8 token tiles x 2 channel halves
    if (has_next) KVQ_WAIT_VM(1);  // this pair's key copies (the next metadata follows)
    else KVQ_WAIT_VM(0);
    uint4 kw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      kw[i] = *reinterpret_cast<const uint4*>((i < 4 ? k_rd0 : k_rd1) + 1024 * ((i >> 1) & 1) + 128 * (i & 1));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    issue_v(pcur);  // into the buffer the key codes have left
    mf_i32x4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc[i] = mfma_i8x64(A0, nibbles_i8(kw[i].x, kw[i].y), zero4);
      acc[i] = mfma_i8x64(A1, nibbles_i8(kw[i].z, kw[i].w), acc[i]);
    }

    // 3. logits, the pair's maximum, weights u_t = rint(32511 p_t s'_t / S'), P = sum p_t, Z = sum u_t z'_t
    float mg[HPL], Sg[HPL], Pt[HPL], Zt[HPL];
#pragma unroll
    for (int e = 0; e < HPL; ++e) {
      float lg[8];
      float lmx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = (At[e] * tks[i]) * fmaf(-tkz[i], FSt[e], (float)limbs_sum(acc[i][2 * e], acc[i][2 * e + 1]));
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
      const float r = Sg[e] > 0x1p-100f ? kPScale * __builtin_amdgcn_rcpf(Sg[e]) : 0.0f;
      float ew[8];
      float zs = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ew[i] = fmaf(pw[i], r, kRoundL);
        zs = fmaf(ew[i] - kRoundL, tvz[i], zs);
      }
      Zt[e] = seg_sum<16>(zs);
      uint32_t lo0, hi0, lo1, hi1;
      limbs4(ew[0], ew[1], ew[2], ew[3], lo0, hi0);
      limbs4(ew[4], ew[5], ew[6], ew[7], lo1, hi1);
      const int he = q4 * HPL + e;
      if (he < GQ) {
        uint8_t* dst = W.wplane + (2 * he) * RS + 8 * c;
        *reinterpret_cast<uint2*>(dst) = make_uint2(lo0, lo1);
        *reinterpret_cast<uint2*>(dst + RS) = make_uint2(hi0, hi1);
      }
    }
    wave_lds_sync();

    // 4. value products: 8 channel tiles x 2 pages
    KVQ_WAIT_VM(0);  // this pair's value copies, the youngest in flight
    uint2 vw[8][2];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      vw[t][0] = *reinterpret_cast<const uint2*>(v_rd + 512 * t);
      vw[t][1] = *reinterpret_cast<const uint2*>(v_rd + 4096 + 512 * t);
    }
    const mf_i32x4 W0 = u4_i32x4(*reinterpret_cast<const uint4*>(w_rd));
    const mf_i32x4 W1 = u4_i32x4(*reinterpret_cast<const uint4*>(w_rd + 64));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (has_next) issue_k(pnext);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      acc[t] = mfma_i8x64(W0, nibbles_i8(vw[t][0].x, vw[t][0].y), zero4);
      acc[t] = mfma_i8x64(W1, nibbles_i8(vw[t][1].x, vw[t][1].y), acc[t]);
    }

    // 5. online-softmax update in the rotated value frame: the pair adds (S' / 32511) (U_c - Z) and P
#pragma unroll
    for (int e = 0; e < HPL; ++e) {
      const float mnew = fmax_raw(m[e], mg[e]);
      const float sc = __builtin_amdgcn_exp2f(m[e] - mnew);  // 0 before the first pair (m = -inf)
      const float eg = __builtin_amdgcn_exp2f(mg[e] - mnew);
      const float wg = eg * Sg[e] * (1.0f / kPScale);
#pragma unroll
      for (int t = 0; t < 8; ++t)
        o[e][t] = fmaf(o[e][t], sc, wg * ((float)limbs_sum(acc[t][2 * e], acc[t][2 * e + 1]) - Zt[e]));
      l[e] = fmaf(l[e], sc, eg * Pt[e]);
      m[e] = mnew;
    }
    mb ^= 1;
    pcur = pnext;
  }
  // every partial a merge reads is written; chunks past the length or the launch bound have none
  if (pb < npairs && chunk_id < g.n_units - 1) {
#pragma unroll
    for (int e = 0; e < HPL; ++e) {
      const int he = q4 * HPL + e;
      if (he < GQ) {
        float* part = a.partials + (((long long)b * g.n_q + h * GQ + he) * g.n_units + 1 + chunk_id) * PART_STRIDE;
#pragma unroll
        for (int t = 0; t < 8; ++t) part[2 + c + 16 * t] = o[e][t];
        if (c == 0) {
          part[0] = m[e];
          part[1] = l[e];
        }
      }
    }
  }
}

// Work-groups of the split-K launch per (sequence, kv head), besides its band unit.
__host__ __device__ inline int splitk_wgs_per_pair(const Geo& g) {
  return g.wave_chunks ? (g.n_units - 1 + 3) / 4 : g.n_units - 1;
}
// One-dimensional grid: the quantized-chunk work-groups first, chunk-major (every pair's first chunk
// work-group, then every pair's second, ...), then the band work-groups.  The hardware hands consecutive
// work-groups to the eight XCDs in turn, so every XCD gets the same mix of chunk positions (pair-major,
// a chunk position would stay on one XCD, and the last chunks, which short sequences lack, would leave
// theirs idle; a band unit inside each pair's run would do the same to the band), and the short band
// work-groups fill the end of the launch.
__device__ inline void splitk_unit_of(const Geo& g, int& unit, int& h, int& b) {
  const int m = splitk_wgs_per_pair(g);
  const int pairs = g.batch * g.n_kv;
  const int i = blockIdx.x;
  int pair;
  if (i < pairs * m) {
    pair = i % pairs;
    unit = 1 + i / pairs;
  } else {
    pair = i - pairs * m;
    unit = 0;
  }
  h = pair % g.n_kv;
  b = pair / g.n_kv;
}

// Matrix-core INT2 launch: its own kernel so that the register bound allows four waves per SIMD at GQ <= 4.
template <int GQ, bool TOK, int BITS>
__global__ __launch_bounds__(kThreads, GQ <= 4 ? (BITS == 2 ? 4 : 3) : 2) void decode_mfma_kernel(DecodeArgs a) {
  __shared__ DecodeLds<GQ, BITS / 2, true> L;
  const Geo& g = a.g;
  int unit, h, b;
  splitk_unit_of(g, unit, h, b);
  const int T = a.seq_lens[b];
  int n_chunks = (n_groups_of(T, g.S0, g.W) + g.gpc - 1) / g.gpc;
  if (n_chunks > g.n_units - 1) n_chunks = g.n_units - 1;  // lengths beyond the launch bound are cut
  if (unit > (n_chunks + 3) / 4) return;
  if (unit == 0) band_unit<GQ>(L, a, b, h, T);
  else int2_unit_mfma<GQ, TOK, BITS>(L, a, b, h, T, unit - 1);
}

// Matrix-core INT4 per-token launch (page pairs; no band: unit 0 stores an empty partial).
template <int GQ>
__global__ __launch_bounds__(kThreads, GQ <= 4 ? 3 : 2) void decode_mfma4_kernel(DecodeArgs a) {
  __shared__ DecodeLds<GQ, 2, true> L;
  const Geo& g = a.g;
  int unit, h, b;
  splitk_unit_of(g, unit, h, b);
  const int T = a.seq_lens[b];
  int n_chunks = ((T + PAGE - 1) / PAGE + g.gpc - 1) / g.gpc;
  if (n_chunks > g.n_units - 1) n_chunks = g.n_units - 1;  // lengths beyond the launch bound are cut
  if (unit > (n_chunks + 3) / 4) return;
  if (unit == 0) {
    for (int e = threadIdx.x; e < GQ * PART_STRIDE; e += kThreads) {
      const int hh = e / PART_STRIDE, k = e % PART_STRIDE;
      float* part = a.partials + (((long long)b * g.n_q + h * GQ + hh) * g.n_units) * PART_STRIDE;
      part[k] = (k == 0) ? -INFINITY : 0.0f;
    }
  } else {
    int4tok_unit_mfma<GQ>(L, a, b, h, T, unit - 1);
  }
}

// MODE: 0 fp32, 1 16-bit on the byte dot product, 2 16-bit on the nibble dot product (grouped schemes)
template <int GQ, int SCHEME, int MODE>
__global__ __launch_bounds__(kThreads) void decode_valu_kernel(DecodeArgs a) {
  __shared__ DecodeLds<GQ, (SCHEME == KVQ_INT4_CHANNEL || (SCHEME == KVQ_INT4_TOKEN && MODE == 2)) ? 2 : 1> L;
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
  if (unit > (g.wave_chunks ? (n_chunks + 3) / 4 : n_chunks)) return;
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
  } else if constexpr (SCHEME == KVQ_INT4_CHANNEL) {
    int2_unit_dot8<GQ, 4>(L, a, b, h, T, unit - 1);
  } else if constexpr (SCHEME == KVQ_INT2_TOKEN) {
    int2tok_unit_dot8<GQ>(L, a, b, h, T, unit - 1);
  } else if constexpr (SCHEME == KVQ_INT2_CHANNEL) {
    if constexpr (MODE == 2) int2_unit_dot8<GQ, 2>(L, a, b, h, T, unit - 1);
    else if constexpr (MODE == 1) int2_unit_dot16<GQ>(L, a, b, h, T, unit - 1);
    else int2_unit<GQ>(L, a, b, h, T, unit - 1);
  } else {
    if constexpr (MODE == 2) int4tok_unit_dot8<GQ>(L, a, b, h, T, unit - 1);
    else if constexpr (MODE == 1) int4_unit_dot16<GQ>(L, a, b, h, T, unit - 1);
    else int4_unit<GQ>(L, a, b, h, T, unit - 1);
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
      if (is_grouped(g.scheme)) {
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
hipError_t launch_gq(const DecodeArgs& a, int stages, hipStream_t s) {
  const Geo& g = a.g;
  if (stages & KVQ_STAGE_QPREP) hipLaunchKernelGGL(qprep_kernel<GQ>, dim3(g.n_kv, g.batch), dim3(512), 0, s, a);
  if (stages & KVQ_STAGE_SPLITK) {
    // wave chunks: four chunks per work-group
    const dim3 grid((1 + splitk_wgs_per_pair(g)) * g.batch * g.n_kv), block(kThreads);
    // AUTO: 16-bit operands on the nibble dot product for INT2, the fp32 kernel for INT4 (faster there:
    // per-token scales leave the fp32 path no per-group work, and 4-bit codes convert cheaply)
    if (g.scheme == KVQ_INT4_CHANNEL) {
      if (a.impl == KVQ_DECODE_MFMA) hipLaunchKernelGGL((decode_mfma_kernel<GQ, false, 4>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((decode_valu_kernel<GQ, KVQ_INT4_CHANNEL, 2>), grid, block, 0, s, a);
    } else if (g.scheme == KVQ_INT2_TOKEN) {
      if (a.impl == KVQ_DECODE_MFMA) hipLaunchKernelGGL((decode_mfma_kernel<GQ, true, 2>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((decode_valu_kernel<GQ, KVQ_INT2_TOKEN, 2>), grid, block, 0, s, a);
    } else if (g.scheme == KVQ_INT2_CHANNEL) {
      if (a.impl == KVQ_DECODE_MFMA) hipLaunchKernelGGL((decode_mfma_kernel<GQ, false, 2>), grid, block, 0, s, a);
      else if (a.impl == KVQ_DECODE_F32) hipLaunchKernelGGL((decode_valu_kernel<GQ, KVQ_INT2_CHANNEL, 0>), grid, block, 0, s, a);
      else if (a.impl == KVQ_DECODE_DOT16) hipLaunchKernelGGL((decode_valu_kernel<GQ, KVQ_INT2_CHANNEL, 1>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((decode_valu_kernel<GQ, KVQ_INT2_CHANNEL, 2>), grid, block, 0, s, a);
    } else {
      // the API resolves AUTO for INT4 per token (nibble digits when the chunks hold whole page pairs)
      if (a.impl == KVQ_DECODE_MFMA) hipLaunchKernelGGL(decode_mfma4_kernel<GQ>, grid, block, 0, s, a);
      else if (a.impl == KVQ_DECODE_DOT8) hipLaunchKernelGGL((decode_valu_kernel<GQ, KVQ_INT4_TOKEN, 2>), grid, block, 0, s, a);
      else if (a.impl == KVQ_DECODE_DOT16) hipLaunchKernelGGL((decode_valu_kernel<GQ, KVQ_INT4_TOKEN, 1>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((decode_valu_kernel<GQ, KVQ_INT4_TOKEN, 0>), grid, block, 0, s, a);
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
    case 1: hipLaunchKernelGGL(qprep_kernel<1>, grid, dim3(512), 0, s, a); break;
    case 2: hipLaunchKernelGGL(qprep_kernel<2>, grid, dim3(512), 0, s, a); break;
    case 4: hipLaunchKernelGGL(qprep_kernel<4>, grid, dim3(512), 0, s, a); break;
    case 8: hipLaunchKernelGGL(qprep_kernel<8>, grid, dim3(512), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int stages, hipStream_t s) {
  switch (a.g.gq) {
    case 1: return launch_gq<1>(a, stages, s);
    case 2: return launch_gq<2>(a, stages, s);
    case 4: return launch_gq<4>(a, stages, s);
    case 8: return launch_gq<8>(a, stages, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
