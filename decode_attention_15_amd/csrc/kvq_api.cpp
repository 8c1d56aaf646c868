// Host side of the C ABI: validation, sizes, rotation builders and kernel launches.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <stdint.h>

#include <mutex>
#include <vector>

#include "kvq_internal.h"

using namespace kvq;

// Workspace of kv_decode_attn_noalloc: a file-scope device array, one per GPU the library runs on, held until
// the process ends.  Host code never passes `scratch` itself to a kernel (on the host it names a stand-in,
// not device memory): the device address comes from hipGetSymbolAddress, once per device, with that device
// current.
static __device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_SCRATCH_BYTES];

namespace {

int gq_of(const kvq_config* c) { return c->n_q_heads / c->n_kv_heads; }

int head_bytes_of(const kvq_config* c) { return is_int2(c->scheme) ? I2_HEAD_BYTES : I4_HEAD_BYTES; }  // INT4 per channel: 8704

int check_config(const kvq_config* c) {
  if (!c) return KVQ_EINVAL;
  if (c->head_dim != D || c->page_tokens != PAGE || c->group_tokens != GROUP) return KVQ_EUNSUPPORTED;
  if (!is_grouped(c->scheme) && c->scheme != KVQ_INT4_TOKEN) return KVQ_EUNSUPPORTED;
  if (c->rotation != KVQ_ROT_DENSE && c->rotation != KVQ_ROT_HADAMARD) return KVQ_EUNSUPPORTED;
  if (c->n_kv_heads < 1 || c->n_q_heads < 1 || c->n_q_heads % c->n_kv_heads != 0) return KVQ_EINVAL;
  const int gq = gq_of(c);
  if (gq != 1 && gq != 2 && gq != 4 && gq != 8) return KVQ_EUNSUPPORTED;
  if (c->n_sink < 0 || c->n_recent < 0) return KVQ_EINVAL;
  if (c->scheme == KVQ_INT4_TOKEN && (c->n_sink != 0 || c->n_recent != 0)) return KVQ_EINVAL;
  if (!(c->clip_k > 0.0f && c->clip_k <= 1.0f) || !(c->clip_v > 0.0f && c->clip_v <= 1.0f)) return KVQ_EINVAL;
  const int unit = is_grouped(c->scheme) ? GROUP : PAGE;
  if (c->split_tokens < 0 || c->split_tokens % unit != 0) return KVQ_EINVAL;
  if (c->decode_impl != KVQ_DECODE_AUTO && c->decode_impl != KVQ_DECODE_F32 && c->decode_impl != KVQ_DECODE_MFMA)
    return KVQ_EINVAL;
  // the matrix-core decode is built for every scheme; it walks INT4 per token in page pairs, so an explicit
  // split must hold whole pairs there
  if (c->decode_impl == KVQ_DECODE_MFMA && c->scheme == KVQ_INT4_TOKEN && c->split_tokens % (2 * PAGE) != 0)
    return KVQ_EUNSUPPORTED;
  // the fp32 decode (exact cross-check) is built for INT2 per channel and INT4 per token
  if (c->decode_impl == KVQ_DECODE_F32 && c->scheme != KVQ_INT2_CHANNEL && c->scheme != KVQ_INT4_TOKEN)
    return KVQ_EUNSUPPORTED;
  if (c->key_only_rotation != 0 && c->key_only_rotation != 1) return KVQ_EINVAL;
  const int hb = c->hadamard_block;
  if (c->rotation == KVQ_ROT_HADAMARD ? (hb != 0 && hb != 16 && hb != 32 && hb != 64 && hb != 128)
                                      : (hb != 0 && hb != 128))
    return KVQ_EINVAL;
  return KVQ_OK;
}

int check_cache(const kvq_config* c, const kvq_cache* k) {
  if (!k || !k->pages || !k->page_table || !k->seq_lens || !k->rot_k || (!k->rot_v && !c->key_only_rotation))
    return KVQ_EINVAL;
  if (k->batch < 1 || k->max_pages_per_seq < 0 || k->n_pages < 1) return KVQ_EINVAL;
  if (is_grouped(c->scheme) && !k->band) return KVQ_EINVAL;
  return KVQ_OK;
}

void clip_params(float rho, int* j, float* f) {
  const double h = 127.0 * (double)rho;
  const double fl = floor(h);
  *j = (int)fl;
  *f = (float)(h - fl);
}

// the matrix-core decode: asked for, or the automatic choice for every scheme (INT4 per token: when split
// into whole page pairs)
bool uses_mfma(const kvq_config* c) {
  if (c->decode_impl == KVQ_DECODE_MFMA) return true;
  if (c->decode_impl != KVQ_DECODE_AUTO) return false;
  return is_grouped(c->scheme) || c->split_tokens % (2 * PAGE) == 0;
}

// decode work split: groups (INT2) or pages (INT4) per chunk
// Split-K work-groups one CU holds at once: the kernel's LDS (160 KB per CU) decides.  Matrix-core decode,
// 2-bit codes: 3 up to GQA 4, 2 at GQA 8; 4-bit codes: 2 up to GQA 4, 1 at GQA 8.  fp32 decode: 4.
int wgs_per_cu(const kvq_config* c) {
  if (!uses_mfma(c)) return 4;
  const bool four = c->scheme == KVQ_INT4_CHANNEL || c->scheme == KVQ_INT4_TOKEN;
  return gq_of(c) <= 4 ? (four ? 2 : 3) : (four ? 1 : 3);
}

// Balanced automatic chunking: the matrix-core decode of the grouped schemes in head quads with no explicit
// split picks its chunk size on the device from the batch's actual lengths (at least 4 groups), so that a
// batch of short and long sequences spreads its groups evenly over the work-groups of one round.
bool balanced_mode(const kvq_config* c) {
  return uses_mfma(c) && is_grouped(c->scheme) && c->split_tokens <= 0 && c->n_kv_heads % 4 == 0;
}
constexpr int kBalancedFloor = 4;  // groups per chunk at least
constexpr size_t kSchedBytes = 256;  // the workspace's tail: the balanced chunk size

int chunk_units(const kvq_config* c, int batch, int max_seq_len) {
  if (c->split_tokens > 0) return c->split_tokens / (is_grouped(c->scheme) ? GROUP : PAGE);
  if (balanced_mode(c)) return kBalancedFloor;
  int units;  // quantized groups/pages per sequence
  if (is_grouped(c->scheme)) units = n_groups_of(max_seq_len, c->n_sink, c->n_recent);
  else units = (max_seq_len + PAGE - 1) / PAGE;
  const int pairs = batch * c->n_kv_heads;
  if (uses_mfma(c)) {
    // one chunk per wave, sized so that the chunk work-groups and the band work-groups (the grouped schemes'
    // band units; INT4 per token's are empty and finish at once) fill the work-group slots of the 256 CUs of
    // an MI355X in one round.  At least 4 groups (pages) per chunk, so that a wave's copies stay in flight
    // across several of them (measured: batch 1 x 32k, 4-group chunks beat 1-group ones), and at most 32.
    long long chunk_wgs = 256LL * wgs_per_cu(c) - (is_grouped(c->scheme) ? pairs : 0);
    if (chunk_wgs < 256) chunk_wgs = 256;
    const long long total = (long long)pairs * units;
    long long per = (total + 4 * chunk_wgs - 1) / (4 * chunk_wgs);
    if (per < 4) per = 4;
    if (per > 32) per = 32;
    if (c->scheme == KVQ_INT4_TOKEN) per = (per + 1) & ~1LL;  // whole page pairs
    return (int)per;
  }
  const int target_wgs = 2048;
  int chunks = (target_wgs + pairs - 1) / pairs;
  if (chunks < 1) chunks = 1;
  int per = (units + chunks - 1) / chunks;
  per = ((per + 3) / 4) * 4;  // the 4 waves of a work-group share a chunk
  const int cap = is_grouped(c->scheme) ? 16 : 32;
  if (per > cap) per = cap;
  if (per < 4) per = 4;
  return per;
}

// Walks per (sequence, head quad) — or per (sequence, kv head) when the kv heads do not come in fours — of
// the matrix-core decode; walk w of n chunks takes chunks w n / walks .. (w + 1) n / walks - 1.  Automatic
// chunks are already sized to fill the GPU in one round: one chunk per walk.  An explicit split fixes the
// chunks the merge combines, which can be many more than the waves of one round: then as many walks as fill
// the work-group slots of one round (a wave walks consecutive chunks, its copies running on across their
// boundaries), with at most 32 groups (pages) per walk.
int walks_of(const kvq_config* c, int batch, int n_chunks, int per) {
  if (c->split_tokens <= 0 || n_chunks <= 1) return n_chunks < 1 ? 1 : n_chunks;
  const long long pairs = (long long)batch * c->n_kv_heads;
  long long slots = 256LL * wgs_per_cu(c) - (is_grouped(c->scheme) ? pairs : 0);  // chunk work-groups per round
  if (slots < 256) slots = 256;
  // rows of work-groups (head quads: one row per (sequence, quad), one walk per work-group; otherwise one row per
  // (sequence, kv head), four walks per work-group)
  const bool quads = c->n_kv_heads % 4 == 0;
  const long long rows = quads ? pairs / 4 : pairs, walks_per_wg = quads ? 1 : 4;
  long long walks = slots / rows * walks_per_wg;
  const long long max_chunks = 32 / per > 1 ? 32 / per : 1;    // chunks per walk
  const long long min_walks = (n_chunks + max_chunks - 1) / max_chunks;
  if (walks < min_walks) walks = min_walks;
  if (walks > n_chunks) walks = n_chunks;
  return (int)(walks < 1 ? 1 : walks);
}

int max_chunks_of(const kvq_config* c, int max_seq_len, int per) {
  int units;
  if (is_grouped(c->scheme)) units = n_groups_of(max_seq_len, c->n_sink, c->n_recent);
  else units = (max_seq_len + PAGE - 1) / PAGE;
  return (units + per - 1) / per;
}

// The decode's chunking and split-K grid for lengths up to max_seq_len (g holds the cache's geometry).
void set_decode_shape(const kvq_config* c, int max_seq_len, Geo& g) {
  const int per = chunk_units(c, g.batch, max_seq_len);
  g.gpc = per;
  g.n_units = 1 + max_chunks_of(c, max_seq_len, per);
  // the matrix-core decode: every wave walks chunks of its own; the fp32 decode: one chunk per work-group
  const bool mfma = uses_mfma(c);
  g.wave_chunks = mfma ? 1 : 0;
  g.walks = mfma ? walks_of(c, g.batch, g.n_units - 1, per) : 1;
  g.balanced = balanced_mode(c) ? 1 : 0;
  if (g.balanced) {
    // one chunk per work-group: as many chunk work-groups as one round holds beside the band work-groups, and
    // at least one per (sequence, head quad), so that one chunk per row always fits
    const long long rows = (long long)g.batch * (c->n_kv_heads / 4);
    long long slots = 256LL * wgs_per_cu(c) - (long long)g.batch * c->n_kv_heads;
    if (slots < 256) slots = 256;
    g.nwg = (int)(rows > slots ? rows : slots);
    g.walks = g.n_units - 1;  // chunks of one (sequence, head quad) at most
  }
  // band work-groups first when the split-K launch takes more than one round of work-groups (see the grid)
  g.band_first = splitk_wgs(g) > 256LL * wgs_per_cu(c) ? 1 : 0;
}

Geo make_geo(const kvq_config* c, const kvq_cache* k) {
  Geo g;
  memset(&g, 0, sizeof(g));
  g.batch = k->batch;
  g.n_kv = c->n_kv_heads;
  g.n_q = c->n_q_heads;
  g.gq = gq_of(c);
  g.scheme = c->scheme;
  g.rotation = c->rotation;
  g.key_only = c->key_only_rotation;
  g.hblock = c->hadamard_block ? c->hadamard_block : D;
  {
    int k = 0;
    while ((1 << k) < g.hblock) ++k;
    // 1/sqrt(2^k): exact for even k, fp64(sqrt 2) scaled by a power of two for odd k
    g.hscale = (k % 2 == 0) ? ldexp(1.0, -k / 2) : ldexp(sqrt(2.0), -(k + 1) / 2);
  }
  g.S0 = c->n_sink;
  g.W = c->n_recent;
  g.slots = kvq_band_slots(c);
  g.max_pages = k->max_pages_per_seq;
  g.n_pages = k->n_pages;
  g.head_bytes = head_bytes_of(c);
  g.page_bytes = (long long)g.head_bytes * c->n_kv_heads;
  return g;
}

// ---- fp64 rotation builders ----
void sylvester_hadamard(double* H) {
  const double s = 1.0 / sqrt((double)D);
  for (int i = 0; i < D; ++i)
    for (int j = 0; j < D; ++j) H[i * D + j] = (__builtin_popcount(i & j) & 1) ? -s : s;
}

int bit_reverse7(int k) {
  int r = 0;
  for (int b = 0; b < 7; ++b) r |= ((k >> b) & 1) << (6 - b);
  return r;
}

// Householder QR of the row-major n x n matrix A (overwritten by R); Q returned row-major,
// with column signs fixed so that diag(R) > 0.
void householder_qr(std::vector<double>& A, std::vector<double>& Q, int n) {
  Q.assign((size_t)n * n, 0.0);
  for (int i = 0; i < n; ++i) Q[(size_t)i * n + i] = 1.0;
  std::vector<double> v(n);
  for (int k = 0; k < n; ++k) {
    double norm2 = 0.0;
    for (int i = k; i < n; ++i) norm2 += A[(size_t)i * n + k] * A[(size_t)i * n + k];
    const double norm = sqrt(norm2);
    if (norm == 0.0) continue;
    const double alpha = A[(size_t)k * n + k] > 0 ? -norm : norm;
    for (int i = 0; i < n; ++i) v[i] = i < k ? 0.0 : A[(size_t)i * n + k];
    v[k] -= alpha;
    double vn2 = 0.0;
    for (int i = k; i < n; ++i) vn2 += v[i] * v[i];
    if (vn2 == 0.0) continue;
    for (int j = k; j < n; ++j) {
      double s = 0.0;
      for (int i = k; i < n; ++i) s += v[i] * A[(size_t)i * n + j];
      const double f = 2.0 * s / vn2;
      for (int i = k; i < n; ++i) A[(size_t)i * n + j] -= f * v[i];
    }
    for (int i = 0; i < n; ++i) {
      double s = 0.0;
      for (int l = k; l < n; ++l) s += Q[(size_t)i * n + l] * v[l];
      const double f = 2.0 * s / vn2;
      for (int l = k; l < n; ++l) Q[(size_t)i * n + l] -= f * v[l];
    }
  }
  for (int k = 0; k < n; ++k) {
    if (A[(size_t)k * n + k] < 0) {
      for (int i = 0; i < n; ++i) Q[(size_t)i * n + k] = -Q[(size_t)i * n + k];
      for (int j = 0; j < n; ++j) A[(size_t)k * n + j] = -A[(size_t)k * n + j];
    }
  }
}

void compose_u_h_pbr(const double* U, double* R) {
  std::vector<double> H((size_t)D * D), UH((size_t)D * D, 0.0);
  sylvester_hadamard(H.data());
  for (int i = 0; i < D; ++i)
    for (int k = 0; k < D; ++k) {
      const double u = U[i * D + k];
      for (int j = 0; j < D; ++j) UH[(size_t)i * D + j] += u * H[(size_t)k * D + j];
    }
  // (X P_br)[:, beta(k)] = X[:, k]
  for (int i = 0; i < D; ++i)
    for (int k = 0; k < D; ++k) R[i * D + bit_reverse7(k)] = UH[(size_t)i * D + k];
}

thread_local char g_last_error[256] = "";


constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on the first call on that device).
hipError_t scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// Status of a launch sequence; a failure records the HIP error name for kvq_last_error().
int to_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return KVQ_OK;
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d): %s", what, hipGetErrorName(e), (int)e,
           hipGetErrorString(e));
  return KVQ_EDEVICE;
}

// Clear an error a previous, unrelated HIP call left behind, so that the status after our launches
// describes our launches only.  A sticky device error is returned again by the next launch check.
void clear_stale_error() { (void)hipGetLastError(); }

}  // namespace

extern "C" {

int kvq_check_config(const kvq_config* cfg) { return check_config(cfg); }

size_t kvq_page_bytes(const kvq_config* cfg) {
  if (check_config(cfg) != KVQ_OK) return 0;
  return (size_t)head_bytes_of(cfg) * (size_t)cfg->n_kv_heads;
}

int32_t kvq_band_slots(const kvq_config* cfg) {
  if (check_config(cfg) != KVQ_OK) return 0;
  return is_grouped(cfg->scheme) ? cfg->n_sink + cfg->n_recent + GROUP : 0;
}

size_t kvq_band_bytes(const kvq_config* cfg, int32_t batch) {
  if (check_config(cfg) != KVQ_OK || batch < 0) return 0;
  return (size_t)batch * cfg->n_kv_heads * (size_t)kvq_band_slots(cfg) * SLOT_BYTES;
}

int32_t kvq_pages_for_len(const kvq_config* cfg, int32_t seq_len) {
  if (check_config(cfg) != KVQ_OK || seq_len < 0) return -1;
  if (is_grouped(cfg->scheme)) return 2 * n_groups_of(seq_len, cfg->n_sink, cfg->n_recent);
  return (seq_len + PAGE - 1) / PAGE;
}

size_t kvq_decode_workspace_bytes(const kvq_config* cfg, int32_t batch, int32_t max_seq_len) {
  if (check_config(cfg) != KVQ_OK || batch < 1 || max_seq_len < 0) return 0;
  const int per = chunk_units(cfg, batch, max_seq_len);
  const int n_units = 1 + max_chunks_of(cfg, max_seq_len, per);
  const size_t nq = (size_t)batch * cfg->n_q_heads;
  return sizeof(float) * (2 * nq * D + nq * (size_t)n_units * PART_STRIDE) + kSchedBytes;
}

double kvq_bits_per_element(const kvq_config* cfg, int64_t seq_len) {
  if (check_config(cfg) != KVQ_OK || seq_len <= 0) return 0.0;
  double bytes;
  if (is_grouped(cfg->scheme)) {
    const int64_t ng = n_groups_of((int)seq_len, cfg->n_sink, cfg->n_recent);
    // per group and K|V: 128x128 codes at 2 (4) bits + 128 bf16 scales + 128 bf16 zeros
    const int code_bytes = cfg->scheme == KVQ_INT4_CHANNEL ? GROUP * D / 2 : GROUP * D / 4;
    bytes = (double)ng * 2.0 * (code_bytes + 2 * D * 2) + (double)(seq_len - GROUP * ng) * SLOT_BYTES;
  } else {
    bytes = (double)seq_len * 2.0 * (D / 2 + 4);
  }
  return bytes * 8.0 / ((double)seq_len * 2.0 * D);
}

int kvq_build_oscar_rotation(const double* gaussian_host, double* R_out_host) {
  if (!gaussian_host || !R_out_host) return KVQ_EINVAL;
  std::vector<double> A(gaussian_host, gaussian_host + D * D), Q;
  householder_qr(A, Q, D);
  compose_u_h_pbr(Q.data(), R_out_host);
  return KVQ_OK;
}

int kvq_compose_oscar_rotation(const double* U_host, double* R_out_host) {
  if (!U_host || !R_out_host) return KVQ_EINVAL;
  compose_u_h_pbr(U_host, R_out_host);
  return KVQ_OK;
}

int kvq_build_hadamard_rotation(const float* sign_host, double* R_out_host) {
  if (!sign_host || !R_out_host) return KVQ_EINVAL;
  std::vector<double> H((size_t)D * D);
  sylvester_hadamard(H.data());
  for (int i = 0; i < D; ++i) {
    if (sign_host[i] != 1.0f && sign_host[i] != -1.0f) return KVQ_EINVAL;
    for (int j = 0; j < D; ++j) R_out_host[i * D + j] = (double)sign_host[i] * H[(size_t)i * D + j];
  }
  return KVQ_OK;
}

int kv_rotate_quant_write(const kvq_config* cfg, kvq_cache* cache, const void* k, const void* v, int32_t dtype,
                          const int32_t* cu_new, int32_t max_new_host, int32_t max_len_host, hipStream_t stream) {
  int st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if ((st = check_cache(cfg, cache)) != KVQ_OK) return st;
  if (!k || !v || !cu_new || max_new_host < 0 || max_len_host < 0 || (dtype != KVQ_F32 && dtype != KVQ_BF16))
    return KVQ_EINVAL;
  // every sequence's length after the append must fit the page-table row
  if (kvq_pages_for_len(cfg, max_len_host) > cache->max_pages_per_seq) return KVQ_ERANGE;
  WriteArgs a;
  memset(&a, 0, sizeof(a));
  a.g = make_geo(cfg, cache);
  a.pages = static_cast<uint8_t*>(cache->pages);
  a.band = static_cast<uint16_t*>(cache->band);
  a.page_table = cache->page_table;
  a.seq_lens = cache->seq_lens;
  a.cu_new = cu_new;
  a.k = k;
  a.v = v;
  a.src_bf16 = dtype == KVQ_BF16;
  a.rot_k = cache->rot_k;
  a.rot_v = cache->rot_v;
  clip_params(cfg->clip_k, &a.clip_j_k, &a.clip_f_k);
  clip_params(cfg->clip_v, &a.clip_j_v, &a.clip_f_v);
  a.max_new = max_new_host;
  clear_stale_error();
  hipError_t e = is_grouped(cfg->scheme) ? launch_write_int2(a, stream) : launch_write_int4(a, stream);
  return to_status(e, "kv_rotate_quant_write");
}

int kv_decode_attn(const kvq_config* cfg, const kvq_cache* cache, const void* q, int32_t dtype, float* out,
                   int32_t max_seq_len_host, void* workspace, size_t ws_bytes, hipStream_t stream) {
  return kv_decode_attn_stages(cfg, cache, q, dtype, out, max_seq_len_host, workspace, ws_bytes, KVQ_STAGE_ALL,
                               stream);
}

namespace {
int decode_with(const kvq_config* cfg, const kvq_cache* cache, const void* q, int32_t dtype, float* out,
                int32_t max_seq_len_host, void* workspace, size_t ws_bytes, int32_t stages, hipEvent_t split_begin,
                hipEvent_t split_end, hipStream_t stream) {
  if (stages < 0 || stages > KVQ_STAGE_ALL) return KVQ_EINVAL;
  int st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if ((st = check_cache(cfg, cache)) != KVQ_OK) return st;
  if (!q || !out || !workspace || max_seq_len_host < 0 || (dtype != KVQ_F32 && dtype != KVQ_BF16))
    return KVQ_EINVAL;
  if (kvq_pages_for_len(cfg, max_seq_len_host) > cache->max_pages_per_seq) return KVQ_ERANGE;
  const size_t need = kvq_decode_workspace_bytes(cfg, cache->batch, max_seq_len_host);
  if (ws_bytes < need) return KVQ_ENOSPACE;
  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.g = make_geo(cfg, cache);
  set_decode_shape(cfg, max_seq_len_host, a.g);
  const bool mfma = uses_mfma(cfg);
  a.pages = static_cast<const uint8_t*>(cache->pages);
  a.band = static_cast<const uint16_t*>(cache->band);
  a.page_table = cache->page_table;
  a.seq_lens = cache->seq_lens;
  a.q = q;
  a.q_bf16 = dtype == KVQ_BF16;
  a.rot_k = cache->rot_k;
  a.rot_v = cache->rot_v;
  a.out = out;
  const size_t nq = (size_t)cache->batch * cfg->n_q_heads;
  float* ws = static_cast<float*>(workspace);
  a.qrot = ws;
  a.qband = ws + nq * D;
  a.partials = ws + 2 * nq * D;
  a.sched = reinterpret_cast<int*>(a.partials + nq * (size_t)a.g.n_units * PART_STRIDE);
  a.impl = mfma ? KVQ_DECODE_MFMA : KVQ_DECODE_F32;
  clear_stale_error();
  return to_status(launch_decode(a, stages, stream, split_begin, split_end), "kv_decode_attn");
}
}  // namespace

int kv_decode_attn_stages(const kvq_config* cfg, const kvq_cache* cache, const void* q, int32_t dtype, float* out,
                          int32_t max_seq_len_host, void* workspace, size_t ws_bytes, int32_t stages,
                          hipStream_t stream) {
  return decode_with(cfg, cache, q, dtype, out, max_seq_len_host, workspace, ws_bytes, stages, nullptr, nullptr,
                     stream);
}

int kv_decode_attn_timed(const kvq_config* cfg, const kvq_cache* cache, const void* q, int32_t dtype, float* out,
                         int32_t max_seq_len_host, void* workspace, size_t ws_bytes, hipEvent_t split_begin,
                         hipEvent_t split_end, hipStream_t stream) {
  if (!split_begin || !split_end) return KVQ_EINVAL;
  return decode_with(cfg, cache, q, dtype, out, max_seq_len_host, workspace, ws_bytes, KVQ_STAGE_ALL, split_begin,
                     split_end, stream);
}

int kvq_decode_shape_of(const kvq_config* cfg, int32_t batch, int32_t max_seq_len, kvq_decode_shape* out) {
  int st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (!out || batch < 1 || max_seq_len < 0) return KVQ_EINVAL;
  kvq_cache k;
  memset(&k, 0, sizeof(k));
  k.batch = batch;
  Geo g = make_geo(cfg, &k);
  set_decode_shape(cfg, max_seq_len, g);
  out->chunk_units = g.gpc;
  out->n_chunks = g.n_units - 1;
  out->walks = g.wave_chunks ? g.walks : out->n_chunks;
  out->span = g.wave_chunks ? (out->n_chunks + g.walks - 1) / g.walks : 1;
  out->splitk_workgroups = splitk_wgs(g);
  out->band_first = g.band_first;
  out->matrix_cores = g.wave_chunks;
  out->balanced = g.balanced;
  out->max_chunks = g.n_units - 1;
  if (g.balanced) {
    // the device's rule when every sequence has max_seq_len tokens: the smallest G >= the floor whose chunks
    // fit the chunk work-groups
    const long long rows = (long long)batch * (cfg->n_kv_heads / 4);
    const long long ng = n_groups_of(max_seq_len, cfg->n_sink, cfg->n_recent);
    long long G = (rows * ng + g.nwg - 1) / g.nwg;
    if (G < g.gpc) G = g.gpc;
    while (ng > 0 && rows * ((ng + G - 1) / G) > g.nwg) ++G;
    out->chunk_units = (int32_t)G;
    out->n_chunks = ng > 0 ? (int32_t)((ng + G - 1) / G) : 0;
    out->walks = out->n_chunks;
    out->span = 1;
  }
  return KVQ_OK;
}

int kvq_read_probe(const kvq_config* cfg, const kvq_cache* cache, uint32_t* xor_out, int32_t max_seq_len_host,
                   hipStream_t stream) {
  int st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if ((st = check_cache(cfg, cache)) != KVQ_OK) return st;
  if (!xor_out || max_seq_len_host < 0) return KVQ_EINVAL;
  if (!is_grouped(cfg->scheme) || !uses_mfma(cfg)) return KVQ_EUNSUPPORTED;
  if (kvq_pages_for_len(cfg, max_seq_len_host) > cache->max_pages_per_seq) return KVQ_ERANGE;
  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.g = make_geo(cfg, cache);
  set_decode_shape(cfg, max_seq_len_host, a.g);
  a.pages = static_cast<const uint8_t*>(cache->pages);
  a.page_table = cache->page_table;
  a.seq_lens = cache->seq_lens;
  clear_stale_error();
  return to_status(launch_read_probe(a, xor_out, stream), "kvq_read_probe");
}

int kv_decode_attn_noalloc(const kvq_config* cfg, const kvq_cache* cache, const void* q, int32_t dtype, float* out,
                           int32_t max_seq_len_host, hipStream_t stream) {
  // every check that needs no device comes first, so that a call that cannot run touches nothing
  int st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if ((st = check_cache(cfg, cache)) != KVQ_OK) return st;
  if (!q || !out || max_seq_len_host < 0 || (dtype != KVQ_F32 && dtype != KVQ_BF16)) return KVQ_EINVAL;
  if (kvq_pages_for_len(cfg, max_seq_len_host) > cache->max_pages_per_seq) return KVQ_ERANGE;
  const size_t need = kvq_decode_workspace_bytes(cfg, cache->batch, max_seq_len_host);
  if (need > (size_t)KVQ_NOALLOC_SCRATCH_BYTES) {
    snprintf(g_last_error, sizeof(g_last_error),
             "kv_decode_attn_noalloc: the decode needs %zu bytes of workspace, the scratch holds %zu",
             need, (size_t)KVQ_NOALLOC_SCRATCH_BYTES);
    return KVQ_ENOSPACE;
  }
  void* ws = nullptr;
  clear_stale_error();
  hipError_t e = scratch_of_current_device(&ws);
  if (e != hipSuccess) return to_status(e, "kv_decode_attn_noalloc (scratch address)");
  return kv_decode_attn_stages(cfg, cache, q, dtype, out, max_seq_len_host, ws, (size_t)KVQ_NOALLOC_SCRATCH_BYTES,
                               KVQ_STAGE_ALL, stream);
}

size_t kvq_prefill_workspace_bytes(const kvq_config* cfg, int32_t total_q) {
  if (check_config(cfg) != KVQ_OK || total_q < 0) return 0;
  return sizeof(float) * 2 * (size_t)total_q * cfg->n_q_heads * D;
}

int kv_prefill_attn(const kvq_config* cfg, const kvq_cache* cache, const void* q, int32_t dtype, const int32_t* cu_q,
                    int32_t total_q_host, int32_t max_q_host, float* out, void* workspace, size_t ws_bytes,
                    hipStream_t stream) {
  int st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if ((st = check_cache(cfg, cache)) != KVQ_OK) return st;
  if (!q || !cu_q || !out || total_q_host < 0 || max_q_host < 0 || (dtype != KVQ_F32 && dtype != KVQ_BF16))
    return KVQ_EINVAL;
  if (total_q_host == 0) return KVQ_OK;
  if (!workspace) return KVQ_EINVAL;
  if (ws_bytes < kvq_prefill_workspace_bytes(cfg, total_q_host)) return KVQ_ENOSPACE;
  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.g = make_geo(cfg, cache);
  a.pages = static_cast<const uint8_t*>(cache->pages);
  a.band = static_cast<const uint16_t*>(cache->band);
  a.page_table = cache->page_table;
  a.seq_lens = cache->seq_lens;
  a.q = q;
  a.q_bf16 = dtype == KVQ_BF16;
  a.rot_k = cache->rot_k;
  a.rot_v = cache->rot_v;
  a.out = out;
  float* ws = static_cast<float*>(workspace);
  a.qrot = ws;
  a.qband = ws + (size_t)total_q_host * cfg->n_q_heads * D;
  a.cu_q = cu_q;
  a.impl = cfg->decode_impl;
  clear_stale_error();
  hipError_t e = launch_qprep_rows(a, total_q_host, stream);
  if (e == hipSuccess) e = launch_prefill(a, max_q_host, stream);
  return to_status(e, "kv_prefill_attn");
}

int kvq_debug_rotate(const kvq_config* cfg, const kvq_cache* cache, int32_t which, const void* x, int32_t dtype,
                     int32_t n, float rho, float* out, hipStream_t stream) {
  int st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (!cache || !x || !out || n < 0 || (which != 0 && which != 1) || (dtype != KVQ_F32 && dtype != KVQ_BF16))
    return KVQ_EINVAL;
  if (!(rho > 0.0f && rho <= 1.0f)) return KVQ_EINVAL;
  const float* rot = which ? cache->rot_v : cache->rot_k;
  if (!rot) return KVQ_EINVAL;
  int j;
  float f;
  clip_params(rho, &j, &f);
  clear_stale_error();
  const Geo g = make_geo(cfg, cache);
  return to_status(launch_debug_rotate(rot, cfg->rotation, g.hblock, g.hscale, x, dtype == KVQ_BF16, n, j, f, out,
                                       stream),
                   "kvq_debug_rotate");
}

int kvq_build_page_table(int32_t batch, int32_t max_pages_per_seq, int64_t n_pages, uint64_t seed,
                         int32_t* table_out_host) {
  if (!table_out_host || batch < 1 || max_pages_per_seq < 0 || n_pages < 1 || n_pages > INT32_MAX)
    return KVQ_EINVAL;
  const int64_t need = (int64_t)batch * max_pages_per_seq;
  if (need > n_pages) return KVQ_ERANGE;
  if (seed == 0) {  // sequence b takes pages b * max_pages_per_seq ..
    for (int64_t i = 0; i < need; ++i) table_out_host[i] = (int32_t)i;
    return KVQ_OK;
  }
  // a seeded random permutation of the pool (Fisher-Yates driven by splitmix64), its first `need` entries
  std::vector<int32_t> perm((size_t)n_pages);
  for (int64_t i = 0; i < n_pages; ++i) perm[(size_t)i] = (int32_t)i;
  uint64_t x = seed;
  auto next = [&x]() {
    uint64_t z = (x += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  };
  for (int64_t i = n_pages - 1; i > 0; --i) {
    // unbiased draw from [0, i]: reject the top partial range
    const uint64_t range = (uint64_t)i + 1, lim = UINT64_MAX - UINT64_MAX % range;
    uint64_t r;
    do r = next(); while (r >= lim);
    const int64_t j = (int64_t)(r % range);
    const int32_t t = perm[(size_t)i];
    perm[(size_t)i] = perm[(size_t)j];
    perm[(size_t)j] = t;
  }
  for (int64_t i = 0; i < need; ++i) table_out_host[i] = perm[(size_t)i];
  return KVQ_OK;
}

int kvq_check_page_table(const int32_t* table_host, int32_t batch, int32_t max_pages_per_seq, int64_t n_pages) {
  if (!table_host || batch < 1 || max_pages_per_seq < 0 || n_pages < 1) return KVQ_EINVAL;
  std::vector<uint8_t> used((size_t)n_pages, 0);
  const int64_t n = (int64_t)batch * max_pages_per_seq;
  for (int64_t i = 0; i < n; ++i) {
    const int32_t p = table_host[i];
    if (p < 0 || p >= n_pages) return KVQ_ERANGE;
    if (used[(size_t)p]) return KVQ_EINVAL;  // two logical pages on one physical page
    used[(size_t)p] = 1;
  }
  return KVQ_OK;
}

int kvq_debug_unpack(const kvq_config* cfg, const kvq_cache* cache, int32_t seq, int32_t kv_head, int32_t n_tokens_host,
                     uint8_t* codes_out, uint16_t* sz_out, hipStream_t stream) {
  int st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if ((st = check_cache(cfg, cache)) != KVQ_OK) return st;
  if (!codes_out || !sz_out || seq < 0 || seq >= cache->batch || kv_head < 0 || kv_head >= cfg->n_kv_heads ||
      n_tokens_host < 0)
    return KVQ_EINVAL;
  if (is_grouped(cfg->scheme) && n_tokens_host % GROUP != 0) return KVQ_EINVAL;
  if ((n_tokens_host + PAGE - 1) / PAGE > cache->max_pages_per_seq) return KVQ_ERANGE;
  if (n_tokens_host == 0) return KVQ_OK;
  WriteArgs a;
  memset(&a, 0, sizeof(a));
  a.g = make_geo(cfg, cache);
  a.pages = static_cast<uint8_t*>(cache->pages);
  a.page_table = cache->page_table;
  clear_stale_error();
  return to_status(launch_debug_unpack(a, seq, kv_head, n_tokens_host, codes_out, sz_out, stream), "kvq_debug_unpack");
}

const char* kvq_strerror(int status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_EINVAL: return "invalid argument";
    case KVQ_ERANGE: return "length or page index out of range";
    case KVQ_ENOSPACE: return "workspace too small";
    case KVQ_EUNSUPPORTED: return "unsupported configuration";
    case KVQ_EDEVICE: return "HIP device error";
    default: return "unknown status";
  }
}

const char* kvq_version(void) { return "kvq 0.1 gfx950"; }

const char* kvq_last_error(void) { return g_last_error; }

}  // extern "C"
