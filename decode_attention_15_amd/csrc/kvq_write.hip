// Write path: rotate -> clip -> quantize -> pack into pages, plus the bf16 band.
//
// [OSCAR] summary page §3.4.4 (steps 1-3) and §3.4.5 (fused prefill write, window demotion);
// [SAW] §3 eq. (1), §4.1 (fused rotation-quantization write), App. A.1 eq. (3)-(4).
//
// Built with -ffp-contract=off: every rounding below is the one the cache format specifies
// (see include/kvq.h), so a CPU implementation of the same definition gets the same bits.
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr unsigned kFull = 0xffffffffu;
// LDS rows of a group's input tokens are padded by one float so that the 16 rows one matrix-core
// operand reads sit in different banks
constexpr int XS_STRIDE = D + 1;

__device__ inline float src_as_bf16_value(const void* src, int src_bf16, long long idx) {
  if (src_bf16) return bf16_to_f32(static_cast<const uint16_t*>(src)[idx]);
  return bf16_to_f32(f32_to_bf16_rne(static_cast<const float*>(src)[idx]));
}

__device__ inline uint16_t src_as_bf16_bits(const void* src, int src_bf16, long long idx) {
  if (src_bf16) return static_cast<const uint16_t*>(src)[idx];
  return f32_to_bf16_rne(static_cast<const float*>(src)[idx]);
}

__device__ inline uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, m, 64);
    v = o < v ? o : v;
  }
  return v;
}

__device__ inline float wave_min_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fminf(v, __shfl_xor(v, m, 64));
  return v;
}

__device__ inline float wave_max_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

__device__ inline int wave_count(bool p) { return __popcll(__ballot(p)); }

// Integer zero point of the token-wise INT4 scheme, rint(-min / s'); an integer has one zero, stored as +0
// (adding +0 turns -0 into +0 and leaves every other value as it is), so the sign of a zero minimum
// cannot reach the stored bits.
__device__ inline float int_zero_point(float amin, float sp) { return __fadd_rn(rintf(__fdiv_rn(-amin, sp)), 0.0f); }

// Correctly rounded x / s for a scale s stored as bf16 (8-bit significand), from rs = 1 / s in fp64.  The
// quotient never lies on a midpoint between fp32 neighbours (x = m s with m such a midpoint would need an
// odd factor above 2^24 in x's 24-bit significand), nor within 2^-33 of one relative to its size (the
// distance is a multiple of ulp/2 / s' for the significand s' < 2^8 of s); x rs is within 2^-52 of x / s,
// so rounding it to fp32 gives RN(x / s).  Exhaustively checked over every fp32 significand of x and
// every bf16 significand of s.
__device__ inline double rcp_of_bf16(float s) { return 1.0 / (double)s; }
__device__ inline float div_by_bf16(float x, double rs) { return (float)((double)x * rs); }

// fp64 / fp32 value of lane l ^ 1 (CTRL 0xB1) or l ^ 2 (CTRL 0x4E) of the lane's quad (DPP quad permute)
template <int CTRL>
__device__ __forceinline__ double quad_swap_f64(double v) {
  const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, true);
  return __hiloint2double(hi, lo);
}

template <int CTRL>
__device__ __forceinline__ float quad_swap_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// j-th smallest (0-based) of the 128 non-negative floats held two per lane, as bit patterns
// (non-negative IEEE floats order like their unsigned bit patterns).  Greedy construction of the
// largest v with #{x < v} <= j, one bit at a time.
__device__ inline uint32_t wave_select_u32(uint32_t u0, uint32_t u1, int j) {
  uint32_t prefix = 0;
  for (int bit = 30; bit >= 0; --bit) {
    const uint32_t cand = prefix | (1u << bit);
    const int cnt = wave_count(u0 < cand) + wave_count(u1 < cand);
    if (cnt <= j) prefix = cand;
  }
  return prefix;
}

// Largest of 64 lanes' non-negative values (below 2^31), every lane: DPP-folded steps within rows, then
// the row and half swaps.
#define KVQ_UPDDPP(x, ctrl) __builtin_amdgcn_update_dpp(0, (x), (ctrl), 0xF, 0xF, true)
__device__ inline int wave_max_i32(int x) {
  x = max(x, KVQ_UPDDPP(x, 0xB1));   // quad_perm [1,0,3,2]
  x = max(x, KVQ_UPDDPP(x, 0x4E));   // quad_perm [2,3,0,1]
  x = max(x, KVQ_UPDDPP(x, 0x141));  // row_half_mirror
  x = max(x, KVQ_UPDDPP(x, 0x140));  // row_mirror
  const auto r16 = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  const uint32_t a16 = r16[0], b16 = r16[1];
  x = max((int)a16, (int)b16);
  const auto r32 = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  const uint32_t a32 = r32[0], b32 = r32[1];
  return max((int)a32, (int)b32);
}

// y_j and y_{j+1} of the 128 non-negative floats (bit patterns, two per lane) for j near the top: the
// distinct values are visited from the largest down, `above` counting the values greater than the
// current one, until the current one is the (128 - j)-th largest; y_{j+1} is the same value when its
// repeats reach past it, else the previously visited value.  At most 128 - j rounds, all wave-uniform.
__device__ inline void wave_top_select_u32(uint32_t u0, uint32_t u1, int j, uint32_t& yj, uint32_t& yj1) {
  const int k = D - j;
  uint32_t cur = kFull, prev = kFull;
  int above = 0;
  for (;;) {
    const uint32_t c0 = u0 < cur ? u0 : 0u, c1 = u1 < cur ? u1 : 0u;
    const uint32_t m = (uint32_t)wave_max_i32((int)(c0 > c1 ? c0 : c1));
    const int cnt = wave_count(u0 == m) + wave_count(u1 == m);
    if (above + cnt >= k) {
      yj = m;
      yj1 = (k - 1 > above) ? m : prev;
      return;
    }
    above += cnt;
    prev = m;
    cur = m;
  }
}

// wave_max_i32 of two independent values, step by step in turn, so that each step's result is not read by the
// next instruction (a DPP read of a VGPR that the previous instruction wrote waits two cycles)
__device__ inline void wave_max2_i32(int& x, int& y) {
  x = max(x, KVQ_UPDDPP(x, 0xB1));
  y = max(y, KVQ_UPDDPP(y, 0xB1));
  x = max(x, KVQ_UPDDPP(x, 0x4E));
  y = max(y, KVQ_UPDDPP(y, 0x4E));
  x = max(x, KVQ_UPDDPP(x, 0x141));
  y = max(y, KVQ_UPDDPP(y, 0x141));
  x = max(x, KVQ_UPDDPP(x, 0x140));
  y = max(y, KVQ_UPDDPP(y, 0x140));
  const auto x16 = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  const auto y16 = __builtin_amdgcn_permlane16_swap((uint32_t)y, (uint32_t)y, false, false);
  x = max((int)x16[0], (int)x16[1]);
  y = max((int)y16[0], (int)y16[1]);
  const auto x32 = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  const auto y32 = __builtin_amdgcn_permlane32_swap((uint32_t)y, (uint32_t)y, false, false);
  x = max((int)x32[0], (int)x32[1]);
  y = max((int)y32[0], (int)y32[1]);
}

// wave_top_select_u32 for two tokens at once (a: a0, a1; b: b0, b1): the two tokens' rounds are independent, so
// their wave reductions interleave; a token that is done keeps its results while the other finishes
__device__ inline void wave_top_select2_u32(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, int j, uint32_t& ya,
                                            uint32_t& ya1, uint32_t& yb, uint32_t& yb1) {
  const int k = D - j;
  uint32_t cura = kFull, preva = kFull, curb = kFull, prevb = kFull;
  int abovea = 0, aboveb = 0;
  bool da = false, db = false;
  for (;;) {
    const uint32_t ca0 = a0 < cura ? a0 : 0u, ca1 = a1 < cura ? a1 : 0u;
    const uint32_t cb0 = b0 < curb ? b0 : 0u, cb1 = b1 < curb ? b1 : 0u;
    int ia = (int)(ca0 > ca1 ? ca0 : ca1), ib = (int)(cb0 > cb1 ? cb0 : cb1);
    wave_max2_i32(ia, ib);
    const uint32_t ma = (uint32_t)ia, mb = (uint32_t)ib;
    const int cnta = wave_count(a0 == ma) + wave_count(a1 == ma);
    const int cntb = wave_count(b0 == mb) + wave_count(b1 == mb);
    if (!da) {
      if (abovea + cnta >= k) {
        ya = ma;
        ya1 = (k - 1 > abovea) ? ma : preva;
        da = true;
      } else {
        abovea += cnta;
        preva = ma;
        cura = ma;
      }
    }
    if (!db) {
      if (aboveb + cntb >= k) {
        yb = mb;
        yb1 = (k - 1 > aboveb) ? mb : prevb;
        db = true;
      } else {
        aboveb += cntb;
        prevb = mb;
        curb = mb;
      }
    }
    if (da && db) return;
  }
}

// clip(x, -tau, tau) as two comparisons, each taking its second operand when the two compare equal, so
// that a zero of either sign clipped at tau = 0 gives +0 as the cache format's definition does
__device__ inline float clip_to(float x, float tau) {
  const float y = x > -tau ? x : -tau;
  return y < tau ? y : tau;
}

// Per-token clip threshold: linear-interpolation quantile of |x| at (j, f) ([OSCAR] §3.4.4 step 2).
__device__ inline float clip_tau(float x0, float x1, int j, float f) {
  const uint32_t u0 = __float_as_uint(x0) & 0x7fffffffu;
  const uint32_t u1 = __float_as_uint(x1) & 0x7fffffffu;
  uint32_t yj, yj1;
  if (j >= D - 1) return __uint_as_float(wave_select_u32(u0, u1, j));
  if (j >= D - 16) {
    // near the top (clip ratios from about 0.88): a few rounds over the largest values
    wave_top_select_u32(u0, u1, j, yj, yj1);
  } else {
    yj = wave_select_u32(u0, u1, j);
    if (wave_count(u0 <= yj) + wave_count(u1 <= yj) >= j + 2) {
      yj1 = yj;
    } else {
      const uint32_t m0 = u0 > yj ? u0 : kFull;
      const uint32_t m1 = u1 > yj ? u1 : kFull;
      yj1 = wave_min_u32(m0 < m1 ? m0 : m1);
    }
  }
  const float y0 = __uint_as_float(yj), y1 = __uint_as_float(yj1);
  return __fadd_rn(y0, __fmul_rn(f, __fsub_rn(y1, y0)));
}

// clip_tau for two tokens (a: xa0, xa1; b: xb0, xb1), the same thresholds: near the top the two selections run
// interleaved
__device__ inline void clip_tau2(float xa0, float xa1, float xb0, float xb1, int j, float f, float& ta, float& tb) {
  if (j >= D - 1 || j < D - 16) {
    ta = clip_tau(xa0, xa1, j, f);
    tb = clip_tau(xb0, xb1, j, f);
    return;
  }
  uint32_t ya, ya1, yb, yb1;
  wave_top_select2_u32(__float_as_uint(xa0) & 0x7fffffffu, __float_as_uint(xa1) & 0x7fffffffu,
                       __float_as_uint(xb0) & 0x7fffffffu, __float_as_uint(xb1) & 0x7fffffffu, j, ya, ya1, yb, yb1);
  const float a_lo = __uint_as_float(ya), a_hi = __uint_as_float(ya1);
  const float b_lo = __uint_as_float(yb), b_hi = __uint_as_float(yb1);
  ta = __fadd_rn(a_lo, __fmul_rn(f, __fsub_rn(a_hi, a_lo)));
  tb = __fadd_rn(b_lo, __fmul_rn(f, __fsub_rn(b_hi, b_lo)));
}

// Unnormalized radix-2 Walsh-Hadamard transform of 128 fp64 values held as (e0 = x[lane],
// e1 = x[lane + 64]), on every block of `block` consecutive values: stages h = 1, 2, ..., block/2 each
// map the pair (i, i+h), i & h == 0, to (a+b, a-b).
__device__ inline void fwht_wave(double& e0, double& e1, int lane, int block) {
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
    if (h >= block) break;
    const double p0 = __shfl_xor(e0, h, 64);
    const double p1 = __shfl_xor(e1, h, 64);
    if (lane & h) {
      e0 = p0 - e0;
      e1 = p1 - e1;
    } else {
      e0 = e0 + p0;
      e1 = e1 + p1;
    }
  }
  if (block == 128) {
    const double a = e0, b = e1;
    e0 = a + b;
    e1 = a - b;
  }
}

// Rotation of one vector whose 128 bf16 values are in LDS (xs) into (y0, y1) = (x~[lane], x~[lane+64]).
// Dense: fp64 products summed in increasing i, rounded once.  Hadamard: sign flip, block FWHT, * 1/sqrt(h).
__device__ inline void rotate_vec(const float* xs, const float* rot, int rotation, int hblock, double hscale,
                                  int lane, float& y0, float& y1) {
  if (rotation == KVQ_ROT_DENSE) {
    double a0 = 0.0, a1 = 0.0;
    for (int i = 0; i < D; ++i) {
      const double x = (double)xs[i];
      a0 = fma(x, (double)rot[i * D + lane], a0);
      a1 = fma(x, (double)rot[i * D + lane + 64], a1);
    }
    y0 = (float)a0;
    y1 = (float)a1;
  } else {
    double e0 = (double)xs[lane] * (double)rot[lane];
    double e1 = (double)xs[lane + 64] * (double)rot[lane + 64];
    fwht_wave(e0, e1, lane, hblock);
    y0 = (float)(e0 * hscale);
    y1 = (float)(e1 * hscale);
  }
}

// Dense rotation of a 128-token group, X~ = X R (X: 128 tokens x XS_STRIDE in LDS, fp32 values of bf16; R fp32
// row-major), on the fp64 matrix cores: v_mfma_f64_16x16x4f64 adds its four products to the accumulator
// one after another in k order, with one fp64 rounding per addition, so the chain over k = 0..127 gives
// the same bits as the sequential fp64 sum the cache format specifies (every product x_i R[i][j] is exact
// in fp64).  Operand layout: lane l supplies A[row l % 16][k l / 16] and B[k l / 16][col l % 16]; the
// result lands in lane l, register r at row l / 16 + 4 r, column l % 16.  Wave w computes tokens
// [32w, 32w + 32) x all 128 columns in one pass (2 x 8 tiles of 16 x 16, 32 steps of k = 4), and since a
// token's rotated row depends on its own input row only, which no other wave reads, it writes the
// results over its input rows.
__device__ inline void rotate_group_mfma(float* xs, const float* rot, int wave, int lane) {
  typedef double d4 __attribute__((ext_vector_type(4)));
  const int li = lane & 15, lk = lane >> 4;
  const int t0 = wave * 32;
  d4 acc[2][8];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) acc[rt][ct] = d4{0.0, 0.0, 0.0, 0.0};
  // R is read from L2, one load per column tile, two steps ahead in two alternating sets (no copies between
  // them): a step converts its set, reloads it for two steps later and multiplies
  float bA[8], bB[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    bA[ct] = rot[lk * D + 16 * ct + li];
    bB[ct] = rot[(4 + lk) * D + 16 * ct + li];
    // opaque starting values: otherwise the compiler merges these loads with the loop's and issues every
    // load right before its use
    asm volatile("" : "+v"(bA[ct]), "+v"(bB[ct]));
  }
  auto step = [&](int s, float (&bs)[8]) {
    const int kk = 4 * s + lk;
    double bv[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) bv[ct] = (double)bs[ct];
    // the last two steps reload row D - 1 (in bounds, never used): no branch around the loads
    const int kn = min(kk + 8, D - 1);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) bs[ct] = rot[kn * D + 16 * ct + li];
    double av[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) av[rt] = (double)xs[(t0 + 16 * rt + li) * XS_STRIDE + kk];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) acc[rt][ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[rt], bv[ct], acc[rt][ct], 0, 0, 0);
  };
#pragma unroll 1
  for (int s = 0; s < D / 4; s += 2) {
    step(s, bA);
    step(s + 1, bB);
  }
  // every read of these rows was consumed by the matrix cores above (a wave's LDS accesses stay in order)
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        xs[(t0 + 16 * rt + lk + 4 * r) * XS_STRIDE + 16 * ct + li] = (float)acc[rt][ct][r];
}

// ---------------------------------------------------------------------------------------------
// INT2 groups (and their 4-bit per-channel variant).  One work-group quantizes one (sequence, kv head,
// K|V, new group): gather 128 bf16 tokens (band or new input) -> rotate -> per-token clip -> min/max per
// channel over the group (KVQ_INT2_CHANNEL, KVQ_INT4_CHANNEL) or per token over its channels
// (KVQ_INT2_TOKEN) -> bf16 scale/zero -> codes -> K token-major rows / V channel-major rows + metadata.
// ---------------------------------------------------------------------------------------------
constexpr int kGroupLds = GROUP * XS_STRIDE * (int)sizeof(float);  // two work-groups per CU

// TOK: per-token INT2 (its own instance, so that its per-token steps leave the per-channel schemes' code as it is)
template <bool TOK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void int2_group_kernel(WriteArgs a) {
  extern __shared__ float lds[];
  float* xs = lds;  // [128 tokens][XS_STRIDE] inputs (bf16 values), rotated and clipped in place
  float* xr = xs;   // the same rows once rotated
  __shared__ float red_min[2][D], red_max[2][D];
  __shared__ float s_zp[D];   // zero point per channel, or per token of the group
  __shared__ double s_rs[D];  // 1 / s' in fp64, likewise

  const Geo& g = a.g;
  const int lg = blockIdx.x;
  const int which = blockIdx.y & 1;
  const int h = blockIdx.y >> 1;
  const int b = blockIdx.z;
  const int T0 = a.seq_lens[b];
  const int c0 = a.cu_new[b];
  const int n_new = a.cu_new[b + 1] - c0;
  const int T1 = T0 + n_new;
  const int grp = n_groups_of(T0, g.S0, g.W) + lg;
  if (grp >= n_groups_of(T1, g.S0, g.W)) return;
  if (2 * grp + 1 >= g.max_pages) return;  // beyond the page-table row: nothing is written

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const void* src = which ? a.v : a.k;
  const float* rot = which ? a.rot_v : a.rot_k;
  const int t_first = g.S0 + GROUP * grp;

  // 1. gather: four channels per thread and step (8-byte bf16, 16-byte fp32 loads) when the band and the source
  //    are aligned for them, else one value per step
  const bool vec4 = (reinterpret_cast<uintptr_t>(a.band) & 7) == 0 &&
                    (reinterpret_cast<uintptr_t>(src) & (a.src_bf16 ? 7 : 15)) == 0;
  if (vec4) {
    for (int e4 = tid; e4 < GROUP * D / 4; e4 += 256) {
      const int tl = e4 >> 5, c = 4 * (e4 & 31);
      const int t = t_first + tl;
      float v[4];
      if (t < T0) {
        const long long slot = band_slot_of(t, g.S0, g.W);
        const long long off = (((long long)b * g.n_kv + h) * g.slots + slot) * 256 + which * 128 + c;
        const uint2 w = *reinterpret_cast<const uint2*>(a.band + off);
        v[0] = __uint_as_float(w.x << 16);
        v[1] = __uint_as_float(w.x & 0xffff0000u);
        v[2] = __uint_as_float(w.y << 16);
        v[3] = __uint_as_float(w.y & 0xffff0000u);
      } else {
        const long long idx = ((long long)(c0 + (t - T0)) * g.n_kv + h) * D + c;
        if (a.src_bf16) {
          const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(src) + idx);
          v[0] = __uint_as_float(w.x << 16);
          v[1] = __uint_as_float(w.x & 0xffff0000u);
          v[2] = __uint_as_float(w.y << 16);
          v[3] = __uint_as_float(w.y & 0xffff0000u);
        } else {
          const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + idx);
          v[0] = bf16_to_f32(f32_to_bf16_rne(f.x));
          v[1] = bf16_to_f32(f32_to_bf16_rne(f.y));
          v[2] = bf16_to_f32(f32_to_bf16_rne(f.z));
          v[3] = bf16_to_f32(f32_to_bf16_rne(f.w));
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) xs[tl * XS_STRIDE + c + i] = v[i];
    }
  } else {
    for (int e = tid; e < GROUP * D; e += 256) {
      const int tl = e >> 7, c = e & (D - 1);
      const int t = t_first + tl;
      float val;
      if (t < T0) {
        const long long slot = band_slot_of(t, g.S0, g.W);
        const long long off = (((long long)b * g.n_kv + h) * g.slots + slot) * 256 + which * 128 + c;
        val = bf16_to_f32(a.band[off]);
      } else {
        const long long row = c0 + (t - T0);
        val = src_as_bf16_value(src, a.src_bf16, (row * g.n_kv + h) * D + c);
      }
      xs[tl * XS_STRIDE + c] = val;
    }
  }
  __syncthreads();

  // 2. rotation (none for V under key-only rotation: the bf16 values themselves)
  constexpr bool tokenwise = TOK;
  const bool four = g.scheme == KVQ_INT4_CHANNEL;
  const float levels = four ? 15.0f : 3.0f;
  const long long hoff = (long long)h * g.head_bytes;
  const int moff = four ? I4C_META_OFF : I2_META_OFF;
  if (which == 1 && g.key_only) {
    // the values themselves
  } else if (g.rotation == KVQ_ROT_DENSE) {
    rotate_group_mfma(xs, rot, wave, lane);
  } else {
    for (int tl = wave * 32; tl < wave * 32 + 32; ++tl) {
      float y0, y1;  // each lane reads its own two inputs of the row before writing them
      rotate_vec(xs + tl * XS_STRIDE, rot, g.rotation, g.hblock, g.hscale, lane, y0, y1);
      xr[tl * XS_STRIDE + lane] = y0;
      xr[tl * XS_STRIDE + lane + 64] = y1;
    }
  }

  // 3. per-token clip, two tokens at a time (no barrier before it: every wave rotated exactly the rows it clips,
  //    and a wave's LDS accesses stay in order)
  const int cj = which ? a.clip_j_v : a.clip_j_k;
  const float cf = which ? a.clip_f_v : a.clip_f_k;
  if (cj < D - 1) {
    for (int tl = wave * 32; tl < wave * 32 + 32; tl += 2) {
      float* ra = xr + tl * XS_STRIDE;
      float* rb = ra + XS_STRIDE;
      const float a0 = ra[lane], a1 = ra[lane + 64], b0 = rb[lane], b1 = rb[lane + 64];
      float ta, tb;
      clip_tau2(a0, a1, b0, b1, cj, cf, ta, tb);
      ra[lane] = clip_to(a0, ta);
      ra[lane + 64] = clip_to(a1, ta);
      rb[lane] = clip_to(b0, tb);
      rb[lane + 64] = clip_to(b1, tb);
    }
  }
  __syncthreads();

  // 4. min/max per channel over the group (or per token over its channels), bf16 scale and zero
  if constexpr (tokenwise) {
    // each wave takes 32 tokens, which lie in one page of the group, whose metadata block is looked up once
    uint16_t* const meta_w =
        reinterpret_cast<uint16_t*>(a.pages + pool_page(g, a.page_table[(long long)b * g.max_pages + 2 * grp + (wave >> 1)]) * g.page_bytes +
                                    hoff + moff) + which * 128;
    // lanes t and t + 32 take token wave * 32 + t, 64 channels each, read from its row: half 0 channels 0-63,
    // half 1 channels 96-127 then 64-95 (on 64 banks the two halves' reads then fall on disjoint banks); one
    // swap across the two halves completes the token's minimum and maximum
    float t_mn, t_mx;
    {
      const int hf = lane >> 5;
      const float* row = xr + (wave * 32 + (lane & 31)) * XS_STRIDE;
      const float* r0 = row + 96 * hf;
      const float* r1 = row + 32 + 32 * hf;
      float mn0 = r0[0], mx0 = r0[0], mn1 = r1[0], mx1 = r1[0];
#pragma unroll
      for (int k = 1; k < 32; ++k) {
        mn0 = fminf(mn0, r0[k]);
        mx0 = fmaxf(mx0, r0[k]);
        mn1 = fminf(mn1, r1[k]);
        mx1 = fmaxf(mx1, r1[k]);
      }
      const float mn = fminf(mn0, mn1), mx = fmaxf(mx0, mx1);
      const auto pm = __builtin_amdgcn_permlane32_swap(__float_as_uint(mn), __float_as_uint(mn), false, false);
      const auto px = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      t_mn = fminf(__uint_as_float(pm[0]), __uint_as_float(pm[1]));
      t_mx = fmaxf(__uint_as_float(px[0]), __uint_as_float(px[1]));
    }
    if (lane < 32) {
      const int tl = wave * 32 + lane;
      const float s = (t_mx > t_mn) ? __fdiv_rn(__fsub_rn(t_mx, t_mn), levels) : 1.0f;
      const uint16_t s16 = f32_to_bf16_rne(s);
      const float sp = bf16_to_f32(s16);
      const uint16_t z16 = f32_to_bf16_rne(__fdiv_rn(-t_mn, sp));
      s_rs[tl] = rcp_of_bf16(sp);
      s_zp[tl] = bf16_to_f32(z16);
      // the token's page: its K (which = 0) or V (which = 1) scales[64] then zeros[64]
      meta_w[tl & 63] = s16;
      meta_w[64 + (tl & 63)] = z16;
    }
  } else {
    const int c = tid & (D - 1), half = tid >> 7;
    float mn = INFINITY, mx = -INFINITY;
    for (int tl = half * 64; tl < half * 64 + 64; ++tl) {
      const float x = xr[tl * XS_STRIDE + c];
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    red_min[half][c] = mn;
    red_max[half][c] = mx;
  }
  __syncthreads();
  if (!tokenwise && tid < D) {
    const float amin = fminf(red_min[0][tid], red_min[1][tid]);
    const float bmax = fmaxf(red_max[0][tid], red_max[1][tid]);
    const float s = (bmax > amin) ? __fdiv_rn(__fsub_rn(bmax, amin), levels) : 1.0f;
    const uint16_t s16 = f32_to_bf16_rne(s);
    const float sp = bf16_to_f32(s16);
    const uint16_t z16 = f32_to_bf16_rne(__fdiv_rn(-amin, sp));
    s_rs[tid] = rcp_of_bf16(sp);
    s_zp[tid] = bf16_to_f32(z16);
    const long long phys = pool_page(g, a.page_table[(long long)b * g.max_pages + 2 * grp + which]);
    uint16_t* meta = reinterpret_cast<uint16_t*>(a.pages + phys * g.page_bytes + hoff + moff);
    meta[tid] = s16;
    meta[D + tid] = z16;
  }
  __syncthreads();

  // 5. codes and packing
  auto code = [&](float x, int c, int tl) -> uint32_t {
    const int i = tokenwise ? tl : c;
    float t = __fadd_rn(div_by_bf16(x, s_rs[i]), s_zp[i]);
    t = fminf(fmaxf(rintf(t), 0.0f), levels);
    return (uint32_t)t;
  };
  if (which == 0) {
    // K, token-major; thread (token tl, half): channels 64 half .. 64 half + 63
    const int tl = tid >> 1, half = tid & 1;
    const long long phys = pool_page(g, a.page_table[(long long)b * g.max_pages + 2 * grp + (tl >> 6)]);
    uint8_t* row = a.pages + phys * g.page_bytes + hoff + I2_K_OFF;
    const float* x = xr + tl * XS_STRIDE + half * 64;
    if (four) {
      // 64 bytes per token; channel block m (16m .. 16m + 15): word 2m nibble k = channel 16m + 2k,
      // word 2m + 1 nibble k = channel 16m + 2k + 1
      uint32_t w8[8];
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          uint32_t w = 0;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int cl = 16 * bi + 2 * k + e;
            w |= code(x[cl], half * 64 + cl, tl) << (4 * k);
          }
          w8[2 * bi + e] = w;
        }
      uint4* dst = reinterpret_cast<uint4*>(row + (tl & 63) * 64 + half * 32);
      dst[0] = make_uint4(w8[0], w8[1], w8[2], w8[3]);
      dst[1] = make_uint4(w8[4], w8[5], w8[6], w8[7]);
    } else {
      // 32 bytes per token, channel c in byte c/4 bits 2*(c%4)
      uint32_t w4[4];
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < 16; ++k) w |= code(x[wd * 16 + k], half * 64 + wd * 16 + k, tl) << (2 * k);
        w4[wd] = w;
      }
      *reinterpret_cast<uint4*>(row + (tl & 63) * 32 + half * 16) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
  } else {
    // V, channel-major; thread (channel c, page ph of the group); token i = 16j + 4gg + r of the page
    const int c = tid & (D - 1), ph = tid >> 7;
    const long long phys = pool_page(g, a.page_table[(long long)b * g.max_pages + 2 * grp + ph]);
    const float* x = xr + ph * 64 * XS_STRIDE + c;
    if (four) {
      // 32-byte rows: token 16j + 4gg + 2hh + n in word 2gg + n, nibble 2j + hh
      uint32_t w8[8];
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          uint32_t w = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int i = 16 * j + 4 * gg + 2 * hh + n;
              w |= code(x[i * XS_STRIDE], c, ph * 64 + i) << (4 * (2 * j + hh));
            }
          w8[2 * gg + n] = w;
        }
      uint4* dst = reinterpret_cast<uint4*>(a.pages + phys * g.page_bytes + hoff + I4C_V_OFF + c * 32);
      dst[0] = make_uint4(w8[0], w8[1], w8[2], w8[3]);
      dst[1] = make_uint4(w8[4], w8[5], w8[6], w8[7]);
    } else {
      // 16-byte rows: token 16j + 4gg + r in byte 4gg + j, bits 2r
      uint32_t w4[4];
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 16 * j + 4 * gg + r;
            w |= code(x[i * XS_STRIDE], c, ph * 64 + i) << (8 * j + 2 * r);
          }
        w4[gg] = w;
      }
      *reinterpret_cast<uint4*>(a.pages + phys * g.page_bytes + hoff + I2_V_OFF + c * 16) =
          make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
  }
}

// bf16 band writes: sink tokens and tokens that are still in the tail after the append.  ADVANCE (one
// new token at most per sequence, so one work-group per sequence reads its length): the work-group also
// advances that length once all its threads have read it.
template <bool ADVANCE>
__global__ __launch_bounds__(256) void band_write_kernel(WriteArgs a) {
  const Geo& g = a.g;
  const int r = blockIdx.x, b = blockIdx.y;
  const int T0 = a.seq_lens[b];
  const int c0 = a.cu_new[b];
  const int n_new = a.cu_new[b + 1] - c0;
  const int t = T0 + r;
  const int ng1 = n_groups_of(T0 + n_new, g.S0, g.W);
  if (r < n_new && (t < g.S0 || t >= g.S0 + GROUP * ng1)) {
    const long long slot = band_slot_of(t, g.S0, g.W);
    const uintptr_t amask = a.src_bf16 ? 7 : 15;
    if ((reinterpret_cast<uintptr_t>(a.band) & 7) == 0 && ((reinterpret_cast<uintptr_t>(a.k) | reinterpret_cast<uintptr_t>(a.v)) & amask) == 0) {
      // four channels per thread and step: 8-byte bf16 stores from 8-byte bf16 or 16-byte fp32 loads
      for (int e4 = threadIdx.x; e4 < g.n_kv * 64; e4 += 256) {
        const int h = e4 >> 6, kv = (e4 >> 5) & 1, c = 4 * (e4 & 31);
        const long long idx = ((long long)(c0 + r) * g.n_kv + h) * D + c;
        const void* src = kv ? a.v : a.k;
        uint2 w;
        if (a.src_bf16) {
          w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(src) + idx);
        } else {
          const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + idx);
          w = make_uint2((uint32_t)f32_to_bf16_rne(f.x) | ((uint32_t)f32_to_bf16_rne(f.y) << 16),
                         (uint32_t)f32_to_bf16_rne(f.z) | ((uint32_t)f32_to_bf16_rne(f.w) << 16));
        }
        *reinterpret_cast<uint2*>(a.band + (((long long)b * g.n_kv + h) * g.slots + slot) * 256 + kv * 128 + c) = w;
      }
    } else {
      for (int e = threadIdx.x; e < g.n_kv * 256; e += 256) {
        const int h = e >> 8, kv = (e >> 7) & 1, c = e & (D - 1);
        const long long idx = ((long long)(c0 + r) * g.n_kv + h) * D + c;
        a.band[(((long long)b * g.n_kv + h) * g.slots + slot) * 256 + kv * 128 + c] =
            src_as_bf16_bits(kv ? a.v : a.k, a.src_bf16, idx);
      }
    }
  }
  if constexpr (ADVANCE) {
    __syncthreads();
    if (threadIdx.x == 0) a.seq_lens[b] = T0 + n_new;
  }
}

__global__ void advance_kernel(int32_t* seq_lens, const int32_t* cu_new, int batch) {
  for (int b = threadIdx.x; b < batch; b += blockDim.x) seq_lens[b] += cu_new[b + 1] - cu_new[b];
}

// ---------------------------------------------------------------------------------------------
// INT4 token-wise ([SAW]).  One work-group owns an aligned quad of 4 tokens of one (sequence,
// kv head, K|V): each wave rotates and quantizes one new token; the V nibbles of the quad share
// bytes, so the work-group merges them with the bytes of tokens outside the append.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void int4_quad_kernel(WriteArgs a) {
  __shared__ float xs[4][D];
  __shared__ uint8_t codes[4][D];
  const Geo& g = a.g;
  const int which = blockIdx.y & 1;
  const int h = blockIdx.y >> 1;
  const int b = blockIdx.z;
  const int T0 = a.seq_lens[b];
  const int c0 = a.cu_new[b];
  const int n_new = a.cu_new[b + 1] - c0;
  const int T1 = T0 + n_new;
  if (n_new <= 0) return;
  const int quad = (T0 >> 2) + blockIdx.x;
  if (quad * 4 >= T1) return;
  if ((quad * 4) / PAGE >= g.max_pages) return;  // beyond the page-table row: nothing is written
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = quad * 4 + wave;
  const bool is_new = (t >= T0 && t < T1);
  const void* src = which ? a.v : a.k;
  const float* rot = which ? a.rot_v : a.rot_k;
  const long long phys = pool_page(g, a.page_table[(long long)b * g.max_pages + (quad * 4) / PAGE]);
  uint8_t* head = a.pages + phys * g.page_bytes + (long long)h * I4_HEAD_BYTES;
  if (is_new) {
    const long long row = c0 + (t - T0);
    xs[wave][lane] = src_as_bf16_value(src, a.src_bf16, (row * g.n_kv + h) * D + lane);
    xs[wave][lane + 64] = src_as_bf16_value(src, a.src_bf16, (row * g.n_kv + h) * D + lane + 64);
  }
  __syncthreads();
  if (is_new) {
    float y0, y1;
    if (which == 1 && g.key_only) {  // key-only rotation: V quantized in its own frame
      y0 = xs[wave][lane];
      y1 = xs[wave][lane + 64];
    } else {
      rotate_vec(xs[wave], rot, g.rotation, g.hblock, g.hscale, lane, y0, y1);
    }
    const float amin = wave_min_f32(fminf(y0, y1));
    const float bmax = wave_max_f32(fmaxf(y0, y1));
    const float s = (bmax > amin) ? __fdiv_rn(__fsub_rn(bmax, amin), 15.0f) : 1.0f;
    const uint16_t s16 = f32_to_bf16_rne(s);
    const float sp = bf16_to_f32(s16);
    const uint16_t z16 = f32_to_bf16_rne(int_zero_point(amin, sp));
    const float zp = bf16_to_f32(z16);
    const double rs = rcp_of_bf16(sp);
    auto code4 = [&](float x) -> uint32_t {
      float q = __fadd_rn(rintf(div_by_bf16(x, rs)), zp);
      q = fminf(fmaxf(q, 0.0f), 15.0f);
      return (uint32_t)q;
    };
    codes[wave][lane] = (uint8_t)code4(y0);
    codes[wave][lane + 64] = (uint8_t)code4(y1);
    if (lane == 0) {
      uint16_t* meta = reinterpret_cast<uint16_t*>(head + (which ? I4_VMETA_OFF : I4_KMETA_OFF) + 4 * (t & 63));
      meta[0] = s16;
      meta[1] = z16;
    }
  }
  __syncthreads();
  if (which == 0) {
    // K rows: token-major, 64 bytes per token; lanes 0..15 of a new token's wave each pack 8 channels
    if (is_new && lane < 16) {
      uint32_t w = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) w |= (uint32_t)codes[wave][lane * 8 + k] << (4 * k);
      *reinterpret_cast<uint32_t*>(head + I4_K_OFF + (t & 63) * 64 + lane * 4) = w;
    }
  } else if (tid < D) {
    // V rows: channel-major, 32 bytes per channel; token i = 16j + 4g + r in byte 8g + 2j + r/2
    const int c = tid;
    const int i0 = (quad * 4) & 63;
    const int j = i0 >> 4, gg = (i0 >> 2) & 3;
    uint16_t* p = reinterpret_cast<uint16_t*>(head + I4_V_OFF + c * 32 + 8 * gg + 2 * j);
    uint32_t v = *p;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tr = quad * 4 + r;
      if (tr >= T0 && tr < T1) v = (v & ~(0xFu << (4 * r))) | ((uint32_t)codes[r][c] << (4 * r));
    }
    *p = (uint16_t)v;
  }
}

// ---------------------------------------------------------------------------------------------
// INT4 token-wise under the randomized Hadamard of block order HB ([SAW] §3 eq. (1), App. A.1
// eq. (3)-(4)).  One work-group per (64-token page, kv head, K|V, sequence) that the append reaches; lane
// l of wave w holds token 16 w + l / 4 of the page and its channels 32 (l % 4) + i, i = 0..31.  The
// butterfly stages h = 1..16 pair channels of one lane, h = 32 and 64 pair lanes l ^ 1 and l ^ 2 of the
// quad, and the token's min and max are quad reductions.  K rows (token-major) and the metadata are written
// by the token's own lanes; the V rows (channel-major, two tokens per byte) are assembled from the page's
// nibble words in LDS by an 8 x 8 nibble transpose, merged with the stored nibbles of tokens outside the
// append.  Sources are read 16 bytes at a time (the launcher checks their alignment).
// ---------------------------------------------------------------------------------------------
template <int HB>
__global__ __launch_bounds__(256) void int4_page_kernel(WriteArgs a) {
  __shared__ uint32_t nib[PAGE * 16];  // [token][word m]: nibble k of word m = channel 8 m + k
  const Geo& g = a.g;
  const int which = blockIdx.y & 1;
  const int h = blockIdx.y >> 1;
  const int b = blockIdx.z;
  const int T0 = a.seq_lens[b];
  const int c0 = a.cu_new[b];
  const int n_new = a.cu_new[b + 1] - c0;
  const int T1 = T0 + n_new;
  if (n_new <= 0) return;
  const int page = T0 / PAGE + blockIdx.x;
  if (page * PAGE >= T1 || page >= g.max_pages) return;  // past the append or the page-table row
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tk = 16 * wave + (lane >> 2), qd = lane & 3;
  const int t = page * PAGE + tk;
  const bool is_new = t >= T0 && t < T1;
  const long long phys = pool_page(g, a.page_table[(long long)b * g.max_pages + page]);
  uint8_t* head = a.pages + phys * g.page_bytes + (long long)h * I4_HEAD_BYTES;

  float y[32];
  if (is_new) {
    const long long base = ((long long)(c0 + t - T0) * g.n_kv + h) * D + 32 * qd;
    const void* src = which ? a.v : a.k;
    if (a.src_bf16) {
      const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + base);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint4 w = p[k];
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          y[8 * k + 2 * m] = __uint_as_float(ww[m] << 16);
          y[8 * k + 2 * m + 1] = __uint_as_float(ww[m] & 0xffff0000u);
        }
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) + base);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float4 w = p[k];
        y[4 * k] = bf16_to_f32(f32_to_bf16_rne(w.x));
        y[4 * k + 1] = bf16_to_f32(f32_to_bf16_rne(w.y));
        y[4 * k + 2] = bf16_to_f32(f32_to_bf16_rne(w.z));
        y[4 * k + 3] = bf16_to_f32(f32_to_bf16_rne(w.w));
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) y[i] = 0.0f;
  }

  if (!(which == 1 && g.key_only)) {  // key-only rotation: V quantized in its own frame
    const float* sg = (which ? a.rot_v : a.rot_k) + 32 * qd;
    double e[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) e[i] = (double)y[i] * (double)sg[i];
#pragma unroll
    for (int hs = 1; hs < 32 && hs < HB; hs <<= 1) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if (i & hs) continue;
        const double lo = e[i], hi = e[i + hs];
        e[i] = lo + hi;
        e[i + hs] = lo - hi;
      }
    }
    // across the quad: the upper channel of a pair takes partner - own, the lower own + partner
    if constexpr (HB >= 64) {
      const double sgn = (qd & 1) ? -1.0 : 1.0;
#pragma unroll
      for (int i = 0; i < 32; ++i) e[i] = fma(sgn, e[i], quad_swap_f64<0xB1>(e[i]));
    }
    if constexpr (HB >= 128) {
      const double sgn = (qd & 2) ? -1.0 : 1.0;
#pragma unroll
      for (int i = 0; i < 32; ++i) e[i] = fma(sgn, e[i], quad_swap_f64<0x4E>(e[i]));
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) y[i] = (float)(e[i] * g.hscale);
  }

  float amin = y[0], bmax = y[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) {
    amin = fminf(amin, y[i]);
    bmax = fmaxf(bmax, y[i]);
  }
  amin = fminf(amin, quad_swap_f32<0xB1>(amin));
  bmax = fmaxf(bmax, quad_swap_f32<0xB1>(bmax));
  amin = fminf(amin, quad_swap_f32<0x4E>(amin));
  bmax = fmaxf(bmax, quad_swap_f32<0x4E>(bmax));
  const float s = (bmax > amin) ? __fdiv_rn(__fsub_rn(bmax, amin), 15.0f) : 1.0f;
  const uint16_t s16 = f32_to_bf16_rne(s);
  const float sp = bf16_to_f32(s16);
  const uint16_t z16 = f32_to_bf16_rne(int_zero_point(amin, sp));
  const float zp = bf16_to_f32(z16);
  const double rs = rcp_of_bf16(sp);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float q = __fadd_rn(rintf(div_by_bf16(y[i], rs)), zp);
    q = fminf(fmaxf(q, 0.0f), 15.0f);
    w[i >> 3] |= (uint32_t)q << (4 * (i & 7));
  }
  if (is_new && qd == 0)
    *reinterpret_cast<uint32_t*>(head + (which ? I4_VMETA_OFF : I4_KMETA_OFF) + 4 * tk) =
        (uint32_t)s16 | ((uint32_t)z16 << 16);
  if (which == 0) {
    if (is_new) *reinterpret_cast<uint4*>(head + I4_K_OFF + tk * 64 + 16 * qd) = make_uint4(w[0], w[1], w[2], w[3]);
    return;
  }
  reinterpret_cast<uint4*>(nib)[tk * 4 + qd] = make_uint4(w[0], w[1], w[2], w[3]);
  __syncthreads();
  if (tid >= 128) return;
  // V word wi of channel 8 cb + c: nibble p holds token 32 (wi & 1) + 16 (p >> 2) + 4 (wi >> 1) + (p & 3)
  const int wi = tid & 7, cb = tid >> 3;
  const int tbase = 32 * (wi & 1) + 4 * (wi >> 1);
  uint32_t A[8];
  uint32_t keep = 0;  // nibbles of tokens outside the append
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int tp = tbase + 16 * (p >> 2) + (p & 3);
    A[p] = nib[tp * 16 + cb];
    const int tt = page * PAGE + tp;
    if (tt < T0 || tt >= T1) keep |= 0xFu << (4 * p);
  }
  if (keep == 0xFFFFFFFFu) return;
  // 8 x 8 nibble transpose: afterwards nibble p of A[c] is nibble c of the word read for token slot p
#pragma unroll
  for (int p = 0; p < 8; p += 2) {
    const uint32_t x = ((A[p] >> 4) ^ A[p + 1]) & 0x0F0F0F0Fu;
    A[p + 1] ^= x;
    A[p] ^= x << 4;
  }
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    if (p & 2) continue;
    const uint32_t x = ((A[p] >> 8) ^ A[p + 2]) & 0x00FF00FFu;
    A[p + 2] ^= x;
    A[p] ^= x << 8;
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t x = ((A[p] >> 16) ^ A[p + 4]) & 0x0000FFFFu;
    A[p + 4] ^= x;
    A[p] ^= x << 16;
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint32_t* dst = reinterpret_cast<uint32_t*>(head + I4_V_OFF + (8 * cb + c) * 32 + 4 * wi);
    *dst = keep ? ((A[c] & ~keep) | (*dst & keep)) : A[c];
  }
}

__global__ __launch_bounds__(64) void debug_rotate_kernel(const float* rot, int rotation, int hblock, double hscale,
                                                          const void* x, int src_bf16, int n, int clip_j, float clip_f,
                                                          float* out) {
  __shared__ float xs[D];
  const int v = blockIdx.x, lane = threadIdx.x;
  if (v >= n) return;
  xs[lane] = src_as_bf16_value(x, src_bf16, (long long)v * D + lane);
  xs[lane + 64] = src_as_bf16_value(x, src_bf16, (long long)v * D + lane + 64);
  __syncthreads();
  float y0, y1;
  rotate_vec(xs, rot, rotation, hblock, hscale, lane, y0, y1);
  if (clip_j < D - 1) {
    const float tau = clip_tau(y0, y1, clip_j, clip_f);
    y0 = clip_to(y0, tau);
    y1 = clip_to(y1, tau);
  }
  out[(long long)v * D + lane] = y0;
  out[(long long)v * D + lane + 64] = y1;
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// Test hook: the quantized tokens of one (sequence, kv head) read back from the pages in logical order, by
// the byte layout include/kvq.h states.  One thread per (token, K or V, channel); the threads with channel
// < 2 of each (token, side) also write that token's scale and zero (per-token schemes), and those of each
// group's first tokens the group's per-channel scales and zeros.
// ---------------------------------------------------------------------------------------------
__global__ void debug_unpack_kernel(WriteArgs a, int seq, int kv_head, int n_tokens, uint8_t* codes_out,
                                    uint16_t* sz_out) {
  const Geo& g = a.g;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n_tokens * 2 * D) return;
  const int u = e / (2 * D), side = (e / D) % 2, c = e % D;  // quantized token u, K (0) or V (1), channel c
  const int i = u % PAGE;
  const uint8_t* hb = a.pages + pool_page(g, a.page_table[(long long)seq * g.max_pages + u / PAGE]) * g.page_bytes +
                      (long long)kv_head * g.head_bytes;
  const int j = i / 16, gg = (i / 4) % 4, r = i % 4;
  int code;
  if (is_int2(g.scheme)) {
    code = side == 0 ? (hb[I2_K_OFF + 32 * i + c / 4] >> (2 * (c % 4))) & 3
                     : (hb[I2_V_OFF + 16 * c + 4 * gg + j] >> (2 * r)) & 3;
  } else if (g.scheme == KVQ_INT4_CHANNEL) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(hb);
    if (side == 0) {
      const int m = c / 16, k = (c % 16) / 2, ee = c % 2;
      code = (w[(I4C_K_OFF + 64 * i) / 4 + 2 * m + ee] >> (4 * k)) & 15;
    } else {
      const int hh = (i / 2) % 2, n = i % 2;
      code = (w[(I4C_V_OFF + 32 * c) / 4 + 2 * gg + n] >> (4 * (2 * j + hh))) & 15;
    }
  } else {
    code = side == 0 ? (hb[I4_K_OFF + 64 * i + c / 2] >> (4 * (c % 2))) & 15
                     : (hb[I4_V_OFF + 32 * c + 8 * gg + 2 * j + r / 2] >> (4 * (r % 2))) & 15;
  }
  codes_out[((long long)u * 2 + side) * D + c] = (uint8_t)code;
  const uint16_t* m16 = reinterpret_cast<const uint16_t*>(hb);
  if (g.scheme == KVQ_INT2_CHANNEL || g.scheme == KVQ_INT4_CHANNEL) {
    // group u / 128: scales and zeros of channel c, side `side` (even page K, odd page V), by its first token
    if (u % GROUP == 0) {
      const int grp = u / GROUP;
      const uint8_t* mp = a.pages + pool_page(g, a.page_table[(long long)seq * g.max_pages + 2 * grp + side]) * g.page_bytes +
                          (long long)kv_head * g.head_bytes + (g.scheme == KVQ_INT2_CHANNEL ? I2_META_OFF : I4C_META_OFF);
      const uint16_t* mm = reinterpret_cast<const uint16_t*>(mp);
      uint16_t* dst = sz_out + (((long long)grp * 2 + side) * 2) * D;
      dst[c] = mm[c];
      dst[D + c] = mm[D + c];
    }
  } else if (c < 2) {
    // per token: (scale, zero) of side `side`
    uint16_t v;
    if (g.scheme == KVQ_INT2_TOKEN) v = m16[(I2_META_OFF / 2) + 128 * side + 64 * c + i];
    else v = m16[((side == 0 ? I4_KMETA_OFF : I4_VMETA_OFF) / 2) + 2 * i + c];
    sz_out[((long long)u * 2 + side) * 2 + c] = v;
  }
}

hipError_t launch_write_int2(const WriteArgs& a, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    for (const void* f : {(const void*)int2_group_kernel<false>, (const void*)int2_group_kernel<true>}) {
      const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kGroupLds);
      if (e != hipSuccess) return e;
    }
    attr_set = true;
  }
  // n new tokens complete at most n / 128 + 1 groups of a sequence
  const int max_groups = a.max_new / GROUP + 1;
  if (a.max_new == 0) return hipSuccess;  // nothing appended: the lengths stay
  const dim3 grid(max_groups, a.g.n_kv * 2, a.g.batch);
  if (a.g.scheme == KVQ_INT2_TOKEN) hipLaunchKernelGGL(int2_group_kernel<true>, grid, dim3(256), kGroupLds, s, a);
  else hipLaunchKernelGGL(int2_group_kernel<false>, grid, dim3(256), kGroupLds, s, a);
  if (a.max_new == 1) {
    // the decode step's append: the band write advances the lengths itself
    hipLaunchKernelGGL(band_write_kernel<true>, dim3(1, a.g.batch), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(band_write_kernel<false>, dim3(a.max_new, a.g.batch), dim3(256), 0, s, a);
    hipLaunchKernelGGL(advance_kernel, dim3(1), dim3(256), 0, s, a.seq_lens, a.cu_new, a.g.batch);
  }
  return hipGetLastError();
}

hipError_t launch_write_int4(const WriteArgs& a, hipStream_t s) {
  if (a.max_new > 0) {
    const bool aligned = reinterpret_cast<uintptr_t>(a.k) % 16 == 0 && reinterpret_cast<uintptr_t>(a.v) % 16 == 0;
    if (a.g.rotation == KVQ_ROT_HADAMARD && aligned) {
      // n new tokens reach at most (n + 62) / 64 + 1 pages of a sequence
      const dim3 grid((a.max_new + 62) / PAGE + 1, a.g.n_kv * 2, a.g.batch);
      switch (a.g.hblock) {
        case 16: hipLaunchKernelGGL(int4_page_kernel<16>, grid, dim3(256), 0, s, a); break;
        case 32: hipLaunchKernelGGL(int4_page_kernel<32>, grid, dim3(256), 0, s, a); break;
        case 64: hipLaunchKernelGGL(int4_page_kernel<64>, grid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL(int4_page_kernel<128>, grid, dim3(256), 0, s, a); break;
      }
    } else {
      const int quads = (a.max_new + 3) / 4 + 1;
      hipLaunchKernelGGL(int4_quad_kernel, dim3(quads, a.g.n_kv * 2, a.g.batch), dim3(256), 0, s, a);
    }
  }
  hipLaunchKernelGGL(advance_kernel, dim3(1), dim3(256), 0, s, a.seq_lens, a.cu_new, a.g.batch);
  return hipGetLastError();
}

hipError_t launch_debug_unpack(const WriteArgs& a, int seq, int kv_head, int n_tokens, uint8_t* codes_out,
                               uint16_t* sz_out, hipStream_t s) {
  const int n = n_tokens * 2 * D;
  hipLaunchKernelGGL(debug_unpack_kernel, dim3((n + 255) / 256), dim3(256), 0, s, a, seq, kv_head, n_tokens, codes_out,
                     sz_out);
  return hipGetLastError();
}

hipError_t launch_debug_rotate(const float* rot, int rotation, int hblock, double hscale, const void* x, int src_bf16,
                               int n, int clip_j, float clip_f, float* out, hipStream_t s) {
  if (n > 0)
    hipLaunchKernelGGL(debug_rotate_kernel, dim3(n), dim3(64), 0, s, rot, rotation, hblock, hscale, x, src_bf16, n,
                       clip_j, clip_f, out);
  return hipGetLastError();
}

}  // namespace kvq
