// Internal declarations shared by the libkvq translation units (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

constexpr int D = 128;            // head dim
constexpr int PAGE = 64;          // tokens per page
constexpr int GROUP = 128;        // tokens per INT2 per-channel group
constexpr int SLOT_BYTES = 512;   // one band token: bf16 K[128] then bf16 V[128]

// INT2 per-channel head block inside a page
constexpr int I2_K_OFF = 0;
constexpr int I2_V_OFF = 2048;
constexpr int I2_META_OFF = 4096;
constexpr int I2_HEAD_BYTES = 4608;
// INT4 token-wise head block inside a page
constexpr int I4_K_OFF = 0;
constexpr int I4_V_OFF = 4096;
constexpr int I4_KMETA_OFF = 8192;
constexpr int I4_VMETA_OFF = 8448;
constexpr int I4_HEAD_BYTES = 8704;
// INT4 per-channel head block: the INT4 page size with the INT2 per-channel metadata arrangement
constexpr int I4C_K_OFF = 0;
constexpr int I4C_V_OFF = 4096;
constexpr int I4C_META_OFF = 8192;

// 1/sqrt(128) as used by the randomized-Hadamard write: sqrt(2) * 2^-4 rounded once to fp64
constexpr double INV_SQRT128_F64 = 0x1.6a09e667f3bcdp-4;
constexpr float LOG2E = 1.4426950408889634f;

// Geometry handed to kernels by value.
struct Geo {
  int batch;
  int n_kv;
  int n_q;
  int gq;
  int scheme;
  int rotation;
  int key_only;     // 1: V neither rotated on write nor un-rotated on read
  int hblock;       // Hadamard block order h (16, 32, 64, 128)
  double hscale;    // its fp64 normalization 1/sqrt(h)
  int S0;
  int W;
  int slots;        // band slots per (seq, kv head)
  int max_pages;    // page-table row length
  long long n_pages;  // physical pages in the pool
  int head_bytes;
  long long page_bytes;
  int gpc;          // groups (grouped schemes) or pages (INT4 per token) per decode chunk
  int n_units;      // decode partial units per (seq, q head): 1 band unit + chunks
  int wave_chunks;  // 1: each wave of a work-group walks chunks of its own and stores their partials
  int walks;        // matrix-core decode: walks per (sequence, head quad) or per (sequence, kv head); walk w
                    // of n chunks takes chunks w n / walks .. (w + 1) n / walks - 1 (a partial per chunk)
  int band_first;   // 1: the split-K grid starts with its band work-groups (launches of more than one round)
  int balanced;     // 1: chunk size chosen on the device from the batch's lengths (gpc is its floor; see below)
  int nwg;          // balanced: chunk work-groups of the launch
};

// both INT2 schemes share the page layout; they and per-channel INT4 share the band and the group demotion
__host__ __device__ constexpr bool is_int2(int scheme) { return scheme == KVQ_INT2_CHANNEL || scheme == KVQ_INT2_TOKEN; }
__host__ __device__ constexpr bool is_grouped(int scheme) { return is_int2(scheme) || scheme == KVQ_INT4_CHANNEL; }

__host__ __device__ inline int n_groups_of(int T, int S0, int W) {
  int r = T - S0 - W;
  return r > 0 ? r / GROUP : 0;
}

// Chunk work-groups of the split-K grid (the band work-groups, one per (sequence, kv head), come on top):
//  - matrix-core decode, n_kv a multiple of 4 (head quads): one walk of four kv heads of a sequence, wave w
//    taking head 4 hq + w, so that the work-group's copies of a page read four neighbouring head blocks
//    together;
//  - matrix-core decode otherwise: four consecutive walks of one (sequence, kv head), one per wave;
//  - fp32 decode: one chunk of one (sequence, kv head), shared by the four waves.
__host__ __device__ inline bool splitk_head_quads(const Geo& g) { return g.wave_chunks && g.n_kv % 4 == 0; }
__host__ __device__ inline int splitk_chunk_wgs(const Geo& g) {
  if (g.balanced) return g.nwg;
  const int nc = g.n_units - 1;
  if (!g.wave_chunks) return g.batch * g.n_kv * nc;
  if (splitk_head_quads(g)) return g.batch * (g.n_kv / 4) * g.walks;
  return g.batch * g.n_kv * ((g.walks + 3) / 4);
}
// the chunks of walk w (of g.walks) of a sequence's n_units - 1 chunks: [*c0, *c1)
__host__ __device__ inline void walk_chunks(const Geo& g, int w, int* c0, int* c1) {
  const long long nc = g.n_units - 1;
  *c0 = (int)(w * nc / g.walks);
  *c1 = (int)((w + 1) * nc / g.walks);
}
__host__ __device__ inline int splitk_wgs(const Geo& g) { return splitk_chunk_wgs(g) + g.batch * g.n_kv; }

// ---- balanced automatic chunking (g.balanced) ----
// The chunk size G (groups) is the smallest G >= g.gpc for which the chunks of every (sequence, head quad),
// ceil(groups / G) each, fit the g.nwg chunk work-groups; chunk work-group i takes one chunk, sequences in
// order, then chunks, then head quads.  A sequence's groups are cut at the launch bound ((n_units - 1) gpc,
// so that no chunk index reaches n_units - 1) and at the page-table row.  The functions are wave-level: the
// calling wave's 64 lanes all take part and all get the results.
__device__ inline int balanced_groups(const Geo& g, int T) {
  const int n = n_groups_of(T, g.S0, g.W);
  int cap = (g.n_units - 1) * g.gpc;
  if (cap > g.max_pages / 2) cap = g.max_pages / 2;
  return n < cap ? n : cap;
}
__device__ inline int wave_sum_i(int x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}
__device__ inline int wave_max_i(int x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const int y = __shfl_xor(x, m, 64);
    x = x > y ? x : y;
  }
  return x;
}
// chunk work-groups the batch needs at chunk size G
__device__ inline int balanced_chunks(const Geo& g, const int32_t* seq_lens, int lane, int G) {
  int c = 0;
  for (int b0 = 0; b0 < g.batch; b0 += 64) {
    const int b = b0 + lane;
    if (b < g.batch) c += (balanced_groups(g, seq_lens[b]) + G - 1) / G;
  }
  return __builtin_amdgcn_readfirstlane(wave_sum_i(c)) * (g.n_kv / 4);
}
__device__ inline int balanced_gpc(const Geo& g, const int32_t* seq_lens, int lane) {
  int s = 0, mx = 0;
  for (int b0 = 0; b0 < g.batch; b0 += 64) {
    const int b = b0 + lane;
    const int n = b < g.batch ? balanced_groups(g, seq_lens[b]) : 0;
    s += n;
    mx = mx > n ? mx : n;
  }
  s = wave_sum_i(s) * (g.n_kv / 4);
  mx = wave_max_i(mx);
  // the results are wave-uniform: say so to the compiler (scalar registers)
  s = __builtin_amdgcn_readfirstlane(s);
  mx = __builtin_amdgcn_readfirstlane(mx);
  int lo = (s + g.nwg - 1) / g.nwg;
  if (lo < g.gpc) lo = g.gpc;
  if (balanced_chunks(g, seq_lens, lane, lo) <= g.nwg) return lo;
  // chunks(lo) > nwg >= chunks(mx): at G = mx every (sequence, head quad) has at most one chunk and the host
  // gives at least one work-group per (sequence, head quad); the count does not grow with G
  int hi = mx;
  while (hi - lo > 1) {
    const int mid = lo + (hi - lo) / 2;
    if (balanced_chunks(g, seq_lens, lane, mid) <= g.nwg) hi = mid;
    else lo = mid;
  }
  return hi;
}
// chunk work-group i at chunk size G: its sequence b, head quad and chunk c; false when it has none
__device__ inline bool balanced_wg(const Geo& g, const int32_t* seq_lens, int i, int lane, int G, int& b,
                                   int& quad, int& c) {
  const int quads = g.n_kv / 4;
  int base = 0;
  for (int b0 = 0; b0 < g.batch; b0 += 64) {
    const int bb = b0 + lane;
    const int cnt = bb < g.batch ? (balanced_groups(g, seq_lens[bb]) + G - 1) / G * quads : 0;
    int incl = cnt;  // inclusive prefix sum over the lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(incl, d, 64);
      if (lane >= d) incl += t;
    }
    const int total = __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
    if (i < base + total) {
      const unsigned long long hit = __ballot(incl > i - base);
      const int l = __ffsll((long long)hit) - 1;  // the first lane whose prefix passes i
      const int local = i - base - __builtin_amdgcn_readfirstlane(__shfl(incl - cnt, l, 64));
      b = __builtin_amdgcn_readfirstlane(b0 + l);
      c = local / quads;
      quad = local % quads;
      return true;
    }
    base += total;
  }
  return false;
}
// matrix-core decode, chunk work-group i: its sequence, and this wave's kv head and walk (chunks c0 .. c1 - 1,
// empty past the walks); returns the work-group's first chunk (every wave's at least that)
__device__ inline int wave_chunk_of(const Geo& g, int i, int wave, int& b, int& h, int& c0, int& c1) {
  if (splitk_head_quads(g)) {
    const int quads = g.n_kv / 4, per = g.batch * quads;
    const int r = i % per;
    b = r / quads;
    h = 4 * (r % quads) + wave;
    walk_chunks(g, i / per, &c0, &c1);
    return c0;
  }
  const int pairs = g.batch * g.n_kv, pair = i % pairs;
  b = pair / g.n_kv;
  h = pair % g.n_kv;
  const int w = 4 * (i / pairs) + wave;
  int first, unused;
  walk_chunks(g, 4 * (i / pairs), &first, &unused);
  if (w < g.walks) {
    walk_chunks(g, w, &c0, &c1);
  } else {
    c0 = c1 = g.n_units - 1;
  }
  return first;
}

__host__ __device__ inline int band_slot_of(int t, int S0, int W) {
  return t < S0 ? t : S0 + (t - S0) % (W + GROUP);
}

// A physical page index from the page table, held inside the pool: an entry outside [0, n_pages) (which
// kvq_check_page_table reports on the host) is taken as the last page, so no access leaves the pool.
__host__ __device__ inline long long pool_page(const Geo& g, int32_t p) {
  const unsigned long long u = (unsigned long long)(unsigned int)p;
  return (long long)(u < (unsigned long long)g.n_pages ? u : (unsigned long long)(g.n_pages - 1));
}

__device__ inline uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

typedef __attribute__((ext_vector_type(4))) int kvq_i32x4;
// Two words of 2-bit codes as the int8 operands of two matrix products: dword n of each holds field n of every
// byte ((w >> 2 n) & 0x03030303), both words' fields from one 64-bit shift.
__device__ __forceinline__ uint64_t shr64(uint64_t w, int n) {
  // one 64-bit shift (the compiler would split a C++ shift into two 32-bit ones); its operand is a load's
  // result, not a matrix-core one
  uint64_t r;
  asm("v_lshrrev_b64 %0, %1, %2" : "=v"(r) : "i"(n), "v"(w));
  return r;
}
__device__ __forceinline__ void codes_i8_pair(uint32_t w0, uint32_t w1, kvq_i32x4& c0, kvq_i32x4& c1) {
  const uint64_t w = ((uint64_t)w1 << 32) | w0;
  const uint64_t s2 = shr64(w, 2), s4 = shr64(w, 4), s6 = shr64(w, 6);
  constexpr uint32_t M = 0x03030303u;
  c0 = kvq_i32x4{(int)(w0 & M), (int)((uint32_t)s2 & M), (int)((uint32_t)s4 & M), (int)((uint32_t)s6 & M)};
  c1 = kvq_i32x4{(int)(w1 & M), (int)((uint32_t)(s2 >> 32) & M), (int)((uint32_t)(s4 >> 32) & M),
                (int)((uint32_t)(s6 >> 32) & M)};
}

// Three signed byte limbs.  An operand x with |x| <= S is rounded to an integer a = lo + 256 mid + 65536 hi
// (lo, mid in [-128, 127], hi in [-64, 63]) by one FMA with the magic addend 2^23 + 0x408080: the result
// lies in [2^23, 2^24), where fp32 spacing is 1, so it is the exact 2^23 + 0x408080 + rint(x) (ties to even)
// and the low 23 bits of its encoding are y = a + 0x408080 in [0, 2^23).  Bytes 0 and 1 of y less 128 are
// lo and mid (xor 0x80 as signed bytes); byte 2 (7 bits) less 64 is hi.  A full scale S of 4,000,000 against
// 2-bit codes (1,000,000 against 4-bit codes) keeps every int32 sum of 128 products with codes exact:
// 128 * 3 * 4,000,000 and 128 * 15 * 1,000,000 are below 2^31.
constexpr float kRound3 = 12615808.0f;  // 2^23 + 0x408080
__device__ __forceinline__ void limbs3(float e0, float e1, float e2, float e3, uint32_t& lo, uint32_t& mid,
                                       uint32_t& hi) {
  const uint32_t u0 = __float_as_uint(e0), u1 = __float_as_uint(e1), u2 = __float_as_uint(e2), u3 = __float_as_uint(e3);
  const uint32_t a01 = __builtin_amdgcn_perm(u1, u0, 0x05010400u);  // u0.b0 u1.b0 u0.b1 u1.b1
  const uint32_t a23 = __builtin_amdgcn_perm(u3, u2, 0x05010400u);
  const uint32_t h01 = __builtin_amdgcn_perm(u1, u0, 0x06020602u);  // u0.b2 u1.b2 (twice)
  const uint32_t h23 = __builtin_amdgcn_perm(u3, u2, 0x06020602u);
  lo = __builtin_amdgcn_perm(a23, a01, 0x05040100u) ^ 0x80808080u;
  mid = __builtin_amdgcn_perm(a23, a01, 0x07060302u) ^ 0x80808080u;
  const uint32_t y = __builtin_amdgcn_perm(h23, h01, 0x05040100u) ^ 0x40404040u;
  hi = y | ((y & 0x40404040u) << 1);  // bit 6 extended into bit 7: y2 - 64 as a signed byte
}

// Non-negative operands u <= S (softmax weights): rounded by one FMA with the magic addend 2^23 + 0x8080, whose encoding's low
// 23 bits are y = u + 0x8080; bytes 0 and 1 of y less 128 are lo and mid, byte 2 is hi (0 ..< 64, no sign)
constexpr float kRoundU = 8421504.0f;  // 2^23 + 0x8080
__device__ __forceinline__ void limbs3u(float e0, float e1, float e2, float e3, uint32_t& lo, uint32_t& mid,
                                        uint32_t& hi) {
  const uint32_t u0 = __float_as_uint(e0), u1 = __float_as_uint(e1), u2 = __float_as_uint(e2), u3 = __float_as_uint(e3);
  const uint32_t a01 = __builtin_amdgcn_perm(u1, u0, 0x05010400u);  // u0.b0 u1.b0 u0.b1 u1.b1
  const uint32_t a23 = __builtin_amdgcn_perm(u3, u2, 0x05010400u);
  const uint32_t h01 = __builtin_amdgcn_perm(u1, u0, 0x06020602u);  // u0.b2 u1.b2 (twice)
  const uint32_t h23 = __builtin_amdgcn_perm(u3, u2, 0x06020602u);
  lo = __builtin_amdgcn_perm(a23, a01, 0x05040100u) ^ 0x80808080u;
  mid = __builtin_amdgcn_perm(a23, a01, 0x07060302u) ^ 0x80808080u;
  hi = __builtin_amdgcn_perm(h23, h01, 0x05040100u);
}
// bf16 matrix-core operands: fp32 values split into bf16 hi + lo (hi the round-to-nearest-even bf16 of x, lo
// that of the remainder: about 16 significant bits together) for v_mfma_f32_16x16x32_bf16, whose products of
// bf16 values are exact and whose sums are fp32
typedef __attribute__((ext_vector_type(4))) float kvq_f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int kvq_u32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 kvq_bf16x8;
__device__ inline kvq_f32x4 mfma_bf16(kvq_u32x4 a, kvq_u32x4 b, kvq_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(kvq_bf16x8, a), __builtin_bit_cast(kvq_bf16x8, b),
                                                  c, 0, 0, 0);
}
// bf16 round to nearest even as bits (finite inputs)
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
__device__ inline void split8(const float (&x)[8], kvq_u32x4& hi, kvq_u32x4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) split2(x[2 * k], x[2 * k + 1], h[k], l[k]);
  hi = kvq_u32x4{h[0], h[1], h[2], h[3]};
  lo = kvq_u32x4{l[0], l[1], l[2], l[3]};
}

// ---- launchers implemented in kvq_write.hip / kvq_decode.hip ----
struct WriteArgs {
  Geo g;
  uint8_t* pages;
  uint16_t* band;
  const int32_t* page_table;
  int32_t* seq_lens;
  const int32_t* cu_new;
  const void* k;
  const void* v;
  int src_bf16;
  const float* rot_k;
  const float* rot_v;
  int clip_j_k, clip_j_v;
  float clip_f_k, clip_f_v;
  int max_new;
};

hipError_t launch_write_int2(const WriteArgs& a, hipStream_t s);
hipError_t launch_write_int4(const WriteArgs& a, hipStream_t s);
hipError_t launch_debug_unpack(const WriteArgs& a, int seq, int kv_head, int n_tokens, uint8_t* codes_out,
                               uint16_t* sz_out, hipStream_t s);
hipError_t launch_debug_rotate(const float* rot, int rotation, int hblock, double hscale, const void* x, int src_bf16,
                               int n, int clip_j, float clip_f, float* out, hipStream_t s);

struct DecodeArgs {
  Geo g;
  const uint8_t* pages;
  const uint16_t* band;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const void* q;
  int q_bf16;
  const float* rot_k;
  const float* rot_v;
  float* out;
  float* qrot;      // [batch][n_q][128]
  float* qband;     // [batch][n_q][128]
  float* partials;  // [batch][n_q][n_units][PART_STRIDE]
  int* sched;       // balanced chunking: [0] the chunk size G the split-K launch used (the merge reads it)
  int impl;
  const int32_t* cu_q;  // prefill: [batch + 1] prefix sums of each sequence's chunk queries
};

constexpr int PART_STRIDE = 2 + D;  // m, l, o[128]

// split_begin / split_end (null, or both set): events the split-K dispatch records at the kernel's start and end
hipError_t launch_decode(const DecodeArgs& a, int stages, hipStream_t s, hipEvent_t split_begin = nullptr,
                         hipEvent_t split_end = nullptr);
// query rotation of `rows` query rows (q, qrot, qband indexed as [row][n_q][128])
hipError_t launch_qprep_rows(const DecodeArgs& a, int rows, hipStream_t s);
hipError_t launch_prefill(const DecodeArgs& a, int max_q, hipStream_t s);
hipError_t launch_read_probe(const DecodeArgs& a, uint32_t* xor_out, hipStream_t s);

}  // namespace kvq
