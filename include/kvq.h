/*
 * kvq.h — C ABI for decode attention over a rotated, 2/4-bit quantized, paged KV cache on MI355X (gfx950).
 *
 * The operations follow these pages (cited by title and section):
 *   [OSCAR] "OSCAR: Offline Spectral Covariance-Aware Rotation for 2-bit KV Cache Quantization"
 *           (English summary page): §3.4.2 rotation R = U·H·P_br; §3.4.4 per-token clip, asymmetric
 *           affine INT2, dequantize then inverse-rotate; §3.4.5 fused write kernel, three-segment cache
 *           [bf16 sink | INT2 history | bf16 recent], FlashDecoding split + merge.
 *   [SAW]   "SAW-INT4: System-AWare 4-Bit KV-Cache Quantization for Real-World LLM Serving": §3 eq. (1)
 *           block-diagonal randomized Hadamard; App. A.1 eq. (3)-(4) token-wise INT4; §4.1 and
 *           App. A.4 eq. (13)-(14) attention with the query rotated once and the output un-rotated.
 *   [NOVA]  "Spend Bits Where Queries Look: ...", App. B.5: query rotated once per step and a two-stage
 *           split-KV decode (partials, then combine); "Bit rate": 2 + 32/128 bits per INT2 element.
 *
 * Conventions
 *  - head_dim is 128.  Vectors are rows; a rotation R is applied as x~ = x·R, so the inverse is R^T.
 *  - Every buffer pointer in kvq_cache and in the calls below is a DEVICE pointer allocated by the
 *    caller (for example a torch tensor's data_ptr()).  Host pointers are named *_host.  The library
 *    never allocates or frees device memory and keeps no state between calls.
 *  - Device work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and is asynchronous.
 *    Argument validation is synchronous and happens before anything is enqueued.
 *  - Every int-returning call returns KVQ_OK (0) or a negative kvq_status; kvq_strerror() names it.
 *    No C++ exception crosses the ABI.  A HIP launch error is returned as KVQ_EDEVICE.
 *  - Calls on the same cache must be ordered (same stream or explicit events); the library does not
 *    lock.  Page contents are only valid for tokens the write calls have produced.
 *
 * Cache layout (all little-endian)
 *  - Sequence b holds tokens [0, T_b), T_b = seq_lens[b].  With S0 = n_sink, W = n_recent, G = 128:
 *      INT2 schemes and INT4_CHANNEL: n_g = max(0, (T - S0 - W) / G) full 128-token groups are quantized; group g
 *      covers tokens [S0 + 128g, S0 + 128g + 128); tokens [0, min(T, S0)) (sink) and
 *      [S0 + 128 n_g, T) (tail, W..W+127 tokens once T >= S0+W) are kept as bf16 in the band.
 *      INT4 scheme: every token is quantized on write (S0 = W = 0, no band).
 *  - Quantized token u (u = t - S0 for INT2, u = t for INT4) of sequence b lives in logical page
 *    u / 64 at in-page index i = u % 64; page_table[b * max_pages_per_seq + u / 64] is its physical
 *    page.  A physical page holds 64 tokens of all n_kv_heads: head h at byte h * head_bytes.
 *  - INT2 head block (head_bytes = 4608), both INT2 schemes:
 *      [0, 2048)     K codes, token-major: token i at 32*i; channel c in byte c/4, bits 2*(c%4).
 *      [2048, 4096)  V codes, channel-major: channel c at 2048 + 16*c; token i = 16j + 4g + r
 *                    (j, g, r in 0..3) in byte 4*g + j, bits 2*r.
 *      [4096, 4608)  per channel (KVQ_INT2_CHANNEL): group metadata, on the group's even page K
 *                    scales[128] then K zeros[128], on its odd page V scales[128] then V zeros[128];
 *                    per token (KVQ_INT2_TOKEN): the page's own tokens, K scales[64], K zeros[64],
 *                    V scales[64], V zeros[64]; all bf16.
 *  - INT4 per-channel head block (head_bytes = 8704):
 *      [0, 4096)     K codes, token-major: token i at 64*i, 16 little-endian 32-bit words; channel
 *                    16m + 2k + e (k < 8, e in {0, 1}) in word 2m + e, bits 4k .. 4k+3.
 *      [4096, 8192)  V codes, channel-major: channel c at 4096 + 32*c, 8 words; token i = 16j + 4g + 2h + n
 *                    (j, g < 4; h, n in {0, 1}) in word 2g + n, bits 4(2j + h) .. 4(2j + h) + 3.
 *      [8192, 8704)  group metadata as for INT2 per channel: even page K scales[128], K zeros[128];
 *                    odd page V scales[128], V zeros[128]; bf16.
 *  - INT4 token-wise head block (head_bytes = 8704):
 *      [0, 4096)     K codes, token-major: token i at 64*i; channel c in byte c/2, low nibble = even c.
 *      [4096, 8192)  V codes, channel-major: channel c at 4096 + 32*c; token i = 16j + 4g + r in
 *                    byte 8*g + 2*j + r/2, low nibble when r is even.
 *      [8192, 8448)  K per-token (scale, zero) bf16 pairs, token i at 8192 + 4*i.
 *      [8448, 8704)  V per-token (scale, zero) bf16 pairs.
 *  - Band (INT2 schemes, INT4_CHANNEL): per (b, kv head) kvq_band_slots() slots of 512 bytes: bf16 K[128] then
 *    bf16 V[128], unrotated.  Token t < S0 sits in slot t; a tail token t in slot
 *    S0 + (t - S0) % (W + 128).  Band base of (b, h) = ((b * n_kv_heads) + h) * slots * 512.
 *
 * Numerics of the write path (identical bits on any conforming implementation)
 *  - Values enter the cache as bf16 (round to nearest even for an fp32 source); the quantizer reads
 *    those bf16 values, exactly as a token demoted from the bf16 recent window.
 *  - Dense rotation: x~_j = fp32( fp64 sum over i = 0..127 in increasing i of x_i * R[i][j] ).
 *    Randomized Hadamard ([SAW]): sign flip, radix-2 butterflies (a+b, a-b) for h = 1..64 in fp64,
 *    times 1/sqrt(128) (= sqrt(2)*2^-4 in fp64), rounded to fp32.  Block order h < 128: the butterflies
 *    for h' = 1..h/2 only (each block of h channels separately), times 1/sqrt(h) = 2^(-k/2) for even
 *    k = log2 h, fp64(sqrt(2)) * 2^(-(k+1)/2) for odd k.
 *  - Clip ([OSCAR] §3.4.4): tau = y[j] + f*(y[j+1] - y[j]) in fp32 without fusion, y = sorted |x~|,
 *    j = floor(127*rho), f = fp32(127*rho - j) (tau = y[127] when j = 127); x = min(max(x~, -tau), tau),
 *    each of max and min taking its second operand when the two compare equal (a zero clipped at tau = 0
 *    is +0).
 *  - INT2 per channel over the group: s = fp32((b-a)/3) (1 if b == a) -> bf16 s'; z = fp32(-a/s') ->
 *    bf16 z'; code = clamp(rint(fp32(fp32(x/s') + z')), 0, 3), rint ties to even.  INT2 per token:
 *    the same with a, b the min and max of the token's 128 (clipped) channels.  INT4 per channel: the same
 *    per-channel arithmetic with 15 levels: s = fp32((b-a)/15), code = clamp(rint(fp32(fp32(x/s') + z')), 0, 15).
 *  - Key-only rotation (key_only_rotation = 1): V is quantized in its own frame (no rotation, the
 *    bf16 values exactly) and the output is not un-rotated; K is rotated as above.
 *  - INT4 per token: s = fp32((b-a)/15) -> bf16 s'; z = rint(fp32(-a/s')) + 0 -> bf16 z' (an integer zero
 *    point has one zero, stored as +0);
 *    code = clamp(rint(fp32(x/s')) + z', 0, 15).
 *  - Dequantized value x^ = s'(code - z').
 */
#ifndef KVQ_H_
#define KVQ_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_EINVAL = -1,        /* bad configuration value or NULL pointer */
  KVQ_ERANGE = -2,        /* a length or page index exceeds what the cache/page table holds */
  KVQ_ENOSPACE = -3,      /* workspace smaller than kvq_decode_workspace_bytes() */
  KVQ_EUNSUPPORTED = -4,  /* head_dim != 128, unknown scheme/rotation, or a combination not built */
  KVQ_EDEVICE = -5        /* a HIP call or kernel launch failed */
} kvq_status;

/* INT2_CHANNEL: asymmetric INT2 per channel over 128-token groups (the workloads' statement);
   INT4_TOKEN:   [SAW] token-wise asymmetric INT4, integer zero point, no band;
   INT2_TOKEN:   [OSCAR] §3.4.4 step 3 as the English page states it: asymmetric INT2 per token over its
                 128 channels (one group per head), real zero point; same pages, band and demotion as
                 INT2_CHANNEL, with per-token scales/zeros in the page metadata;
   INT4_CHANNEL: the per-channel scheme with 4-bit codes (15 levels, real zero point), same band and
                 128-token groups, INT4 page size. */
typedef enum { KVQ_INT2_CHANNEL = 0, KVQ_INT4_TOKEN = 1, KVQ_INT2_TOKEN = 2, KVQ_INT4_CHANNEL = 3 } kvq_scheme;
typedef enum { KVQ_F32 = 0, KVQ_BF16 = 1 } kvq_dtype;
typedef enum { KVQ_ROT_DENSE = 0, KVQ_ROT_HADAMARD = 1 } kvq_rotation;
/* Arithmetic of the quantized-token part of the decode (the bf16 band is always fp32):
   MFMA  - every scheme: the key-side operand (per-channel schemes: alpha = q~ s per group and head; per-token
           schemes: q~ once per walk) and the softmax weights (times the value scales for the per-token
           schemes) rounded to integers scaled to their maximum, 4,000,000 for 2-bit codes and 1,000,000 for
           4-bit codes (22 and 20 bits, so that every int32 sum over 128 codes stays exact), split into three
           signed byte limbs and multiplied with the 2-bit or 4-bit codes on the int8 matrix cores, 16 x 16 x 64
           products whose rows are (query head, limb) pairs, so the query heads of a kv head share one pass over
           the codes; every wave walks a chunk of its own (split_tokens = 0: 4 to 32 groups or pages per chunk,
           chosen by size); INT4_TOKEN walks page pairs, so an explicit split_tokens must be a
           multiple of 128;
   F32   - fp32 FMA on the codes with exact per-group alpha = q~ s and softmax weights: the cross-check of the
           matrix-core decode, built for INT2_CHANNEL and INT4_TOKEN (other schemes: KVQ_EUNSUPPORTED);
   AUTO  - MFMA (INT4_TOKEN with a split of an odd number of pages: F32). */
typedef enum {
  KVQ_DECODE_AUTO = 0,
  KVQ_DECODE_F32 = 1,
  KVQ_DECODE_MFMA = 2
} kvq_decode_impl;

/* Static description of one attention layer's cache. */
typedef struct {
  int32_t head_dim;      /* must be 128 */
  int32_t n_kv_heads;    /* >= 1 */
  int32_t n_q_heads;     /* multiple of n_kv_heads; q head h reads kv head h / (n_q_heads / n_kv_heads) */
  int32_t scheme;        /* kvq_scheme */
  int32_t rotation;      /* kvq_rotation: DENSE (OSCAR R, fp32 128x128) or HADAMARD (SAW, 128 signs) */
  int32_t page_tokens;   /* must be 64 */
  int32_t group_tokens;  /* must be 128 (INT2 demotion group length) */
  int32_t n_sink;        /* S0 >= 0 (INT2 schemes; 0 for INT4) */
  int32_t n_recent;      /* W >= 0 (INT2 schemes; 0 for INT4) */
  float clip_k;          /* rho_K in (0, 1]; 1 = no clip (INT2 only) */
  float clip_v;          /* rho_V in (0, 1] */
  int32_t split_tokens;  /* quantized tokens per decode chunk, each merged from one partial: a multiple of 128
                            (grouped schemes) or 64 (INT4_TOKEN), or 0 = chosen by size (matrix-core decode: 4 to
                            32 groups or pages per chunk).  On the matrix-core
                            decode each wave of a work-group walks a chunk of its own and a work-group takes
                            four; on the fp32 decode the four waves of a work-group share one chunk. */
  int32_t decode_impl;   /* kvq_decode_impl */
  int32_t key_only_rotation;  /* 0: K and V rotated (V by R_V on write, outputs un-rotated by R_V^T);
                                 1: only K rotated ([SAW] App. C default), V kept in its own frame and
                                 kvq_cache.rot_v unused (may be NULL) */
  int32_t hadamard_block;     /* HADAMARD rotation: block order h of [SAW] eq. (1), the same normalized
                                 h x h Hadamard on each block of h channels after the sign flip:
                                 16, 32, 64 or 128 (0 = 128); DENSE: 0 or 128 */
} kvq_config;

/* Device-resident cache of a batch of sequences.  All pointers are device pointers owned by the caller. */
typedef struct {
  void* pages;                /* physical page pool, n_pages * kvq_page_bytes() bytes */
  int64_t n_pages;
  void* band;                 /* bf16 band, kvq_band_bytes(cfg, batch) bytes (may be NULL for INT4) */
  const int32_t* page_table;  /* [batch][max_pages_per_seq] logical -> physical page */
  int32_t max_pages_per_seq;
  int32_t* seq_lens;          /* [batch] tokens cached so far; advanced by kv_rotate_quant_write */
  const float* rot_k;         /* DENSE: R_K fp32 row-major [128][128]; HADAMARD: signs fp32 [128] (+1/-1) */
  const float* rot_v;         /* same for V (unused and may be NULL with key_only_rotation) */
  int32_t batch;
} kvq_cache;

/* ---- sizes (host only, no device access) ---- */

/* Bytes of one physical page (64 tokens x all kv heads), 0 on a bad config. */
size_t kvq_page_bytes(const kvq_config* cfg);
/* Band slots per (sequence, kv head): S0 + W + 128 for INT2, 0 for INT4. */
int32_t kvq_band_slots(const kvq_config* cfg);
/* Bytes of the band for `batch` sequences. */
size_t kvq_band_bytes(const kvq_config* cfg, int32_t batch);
/* Logical pages a sequence of `seq_len` tokens occupies (INT2: 2 per full group, INT4: ceil(seq_len/64)),
   -1 on a bad config.  Size max_pages_per_seq with the largest length the cache will reach. */
int32_t kvq_pages_for_len(const kvq_config* cfg, int32_t seq_len);
/* Workspace bytes kv_decode_attn needs for `batch` sequences of at most `max_seq_len` tokens. */
size_t kvq_decode_workspace_bytes(const kvq_config* cfg, int32_t batch, int32_t max_seq_len);
/* Storage bits per cached K/V element for one sequence of `seq_len` tokens ([NOVA] "Bit rate"). */
double kvq_bits_per_element(const kvq_config* cfg, int64_t seq_len);
/* Validate a configuration (KVQ_OK or the status a call would return). */
int kvq_check_config(const kvq_config* cfg);

/* ---- rotation builders (host, fp64) ---- */

/* [OSCAR] §3.4.2: R = U·H·P_br with U the Q factor of a Householder QR of `gaussian_host` (row-major
   128x128, fp64), signs fixed so that diag of the triangular factor is positive, H the normalized
   Sylvester Hadamard matrix, and P_br[k][beta(k)] = 1 for the 7-bit bit reversal beta.  U stands in for
   the calibrated eigenbasis.  Writes R row-major to `R_out_host` (128x128 fp64). */
int kvq_build_oscar_rotation(const double* gaussian_host, double* R_out_host);
/* Same construction from a given orthonormal basis U (columns = eigenvectors sorted by decreasing
   eigenvalue): R = U·H·P_br. */
int kvq_compose_oscar_rotation(const double* U_host, double* R_out_host);
/* [SAW] §3: dense form diag(sign)·H of the randomized Hadamard (for reference/inspection). */
int kvq_build_hadamard_rotation(const float* sign_host, double* R_out_host);

/* ---- page tables (host) ----
   The paged cache ([OSCAR] §3.4.5: pages indexed through a page table) maps logical page p of sequence b to
   physical page table[b * max_pages_per_seq + p] of the pool. */
/* Fill table_out_host [batch][max_pages_per_seq] with distinct physical pages of a pool of n_pages: seed 0
   gives sequence b the pages b * max_pages_per_seq + p; any other seed the first batch * max_pages_per_seq
   entries of a seeded random permutation of the pool (Fisher-Yates, splitmix64 stream from `seed`).  The
   caller uploads the table.  Errors: KVQ_EINVAL (NULL, batch < 1, max_pages_per_seq < 0, n_pages < 1 or
   above 2^31 - 1), KVQ_ERANGE (batch * max_pages_per_seq > n_pages). */
int kvq_build_page_table(int32_t batch, int32_t max_pages_per_seq, int64_t n_pages, uint64_t seed,
                         int32_t* table_out_host);
/* Validate a host copy of a page table: KVQ_ERANGE if an entry lies outside [0, n_pages), KVQ_EINVAL if two
   entries name the same physical page (or for NULL / non-positive sizes), else KVQ_OK. */
int kvq_check_page_table(const int32_t* table_host, int32_t batch, int32_t max_pages_per_seq, int64_t n_pages);

/* ---- calibration: the rotation from an attention-aware covariance (host, fp64) ----
   [OSCAR] §3.2 offline steps 2-3 and §3.4.2 Factor 1: the key rotation's U is the eigenbasis of the query
   covariance C_Q, the value rotation's U that of the score-weighted value covariance C_S, eigenvectors in
   columns by decreasing eigenvalue, and R = U·H·P_br.  All buffers are caller-owned host memory; inputs
   are read only.  Errors: KVQ_EINVAL for NULL pointers, non-positive counts, non-finite inputs or a
   non-symmetric C (|C_ij - C_ji| > 1e-12 max|C|); KVQ_ERANGE if the eigensolver does not converge. */
/* C_Q = (1/N) sum_n q_n^T q_n for N = n_rows query rows q [n_rows][128] (fp32); fp64 sums over n in
   increasing order.  Writes C [128][128] row-major. */
int kvq_query_covariance(const float* q_host, int64_t n_rows, double* C_out_host);
/* C_S = (1/N) (S V)^T (S V) for values V [n_keys][128] and attention scores S [n_rows][n_keys] (fp32,
   row-major), N = n_rows; row n of S V is summed over keys in increasing order in fp64. */
int kvq_score_value_covariance(const float* v_host, int64_t n_keys, const float* s_host, int64_t n_rows,
                               double* C_out_host);
/* Symmetric eigendecomposition C = U diag(lambda) U^T (cyclic Jacobi, fp64): lambda [128] descending,
   column k of U [128][128] (row-major) the unit eigenvector of lambda[k], its entry of largest magnitude
   (first such index) positive.  Within a repeated eigenvalue the basis is any orthonormal one. */
int kvq_eigenbasis(const double* C_host, double* U_out_host, double* lambda_out_host);
/* R = U·H·P_br with U the eigenbasis of C (kvq_eigenbasis followed by kvq_compose_oscar_rotation). */
int kvq_build_oscar_rotation_from_covariance(const double* C_host, double* R_out_host);

/* ---- the hot path ---- */

/* Append tokens to every sequence of the cache ([OSCAR] §3.4.5 prefill and window-demotion kernels;
   [SAW] §4.1 fused rotate-quantize write).
   k, v: device [total_new][n_kv_heads][128], fp32 or bf16 (`dtype`), sequence b's new tokens at rows
   cu_new[b] .. cu_new[b+1]-1 (cu_new: device int32 [batch+1], non-decreasing, cu_new[0] = 0).
   max_new_host bounds cu_new[b+1]-cu_new[b] over b (it sizes the launch grids); max_len_host bounds every
   sequence's length after the append (seq_lens[b] + new tokens), host side, as kv_decode_attn's bound.
   Token t of sequence b is t = seq_lens[b] + row offset.  INT2: sink/tail tokens go to the band; every
   128-token group completed by the append is rotated, clipped, quantized and packed (reading band
   tokens and new tokens as needed).  INT4: every new token is rotated and quantized.  Finally
   seq_lens[b] += new tokens.  Errors: KVQ_EINVAL (NULL, bad dtype, max_new_host or max_len_host < 0),
   KVQ_ERANGE (max_len_host needs more pages than max_pages_per_seq: nothing is enqueued), KVQ_EDEVICE.
   The device side trusts the bounds: a length beyond max_len_host is not written past the page-table row,
   and a page-table entry outside [0, n_pages) is taken as the pool's last page (kvq_check_page_table finds
   such entries on the host). */
int kv_rotate_quant_write(const kvq_config* cfg, kvq_cache* cache, const void* k, const void* v,
                          int32_t dtype, const int32_t* cu_new, int32_t max_new_host, int32_t max_len_host,
                          hipStream_t stream);

/* One decode attention step ([OSCAR] §3.4.4 step 4 and §3.4.5; [SAW] App. A.4 eq. (13)-(14)).
   q: device [batch][n_q_heads][128] fp32 or bf16; out: device fp32 [batch][n_q_heads][128].
   out[b][h] = softmax(q·K^T/sqrt(128))·V over all seq_lens[b] cached tokens, where quantized tokens
   are read as K^ = X^·R_K^T, V^ = X^·R_V^T: computed as (q·R_K)·X^ for the logits and (p·X^)·R_V^T
   for the output, with an online softmax over split chunks merged in a second kernel.
   max_seq_len_host bounds seq_lens (it sizes the grid); workspace: device scratch of ws_bytes >=
   kvq_decode_workspace_bytes(cfg, batch, max_seq_len_host).  A sequence with seq_len 0 yields zeros.
   Errors: KVQ_EINVAL, KVQ_ERANGE (max_seq_len_host beyond the page table), KVQ_ENOSPACE, KVQ_EDEVICE. */
int kv_decode_attn(const kvq_config* cfg, const kvq_cache* cache, const void* q, int32_t dtype, float* out,
                   int32_t max_seq_len_host, void* workspace, size_t ws_bytes, hipStream_t stream);

/* The decode step restricted to some of its three kernels, to time one of them in isolation:
   `stages` is a bitmask of KVQ_STAGE_QPREP (query rotation), KVQ_STAGE_SPLITK (split-K partials of the
   quantized chunks and the bf16 band) and
   KVQ_STAGE_MERGE (merge, un-rotate, normalize); a later stage reads what an earlier call left in the
   workspace.  kv_decode_attn() equals stages = KVQ_STAGE_ALL.  Same arguments and errors otherwise. */
enum { KVQ_STAGE_QPREP = 1, KVQ_STAGE_SPLITK = 2, KVQ_STAGE_MERGE = 4, KVQ_STAGE_ALL = 7 };
int kv_decode_attn_stages(const kvq_config* cfg, const kvq_cache* cache, const void* q, int32_t dtype, float* out,
                          int32_t max_seq_len_host, void* workspace, size_t ws_bytes, int32_t stages,
                          hipStream_t stream);

/* kv_decode_attn with two caller-created HIP events (hipEventCreate, timing enabled; the caller owns and
   destroys them) that the split-K kernel's dispatch itself records at the kernel's start and end
   (hipExtLaunchKernel), so that hipEventElapsedTime(split_begin, split_end) is the split-K kernel's time
   whatever the host does around the call (a measurement hook).  Same arguments, results and errors as
   kv_decode_attn; KVQ_EINVAL for a null event. */
int kv_decode_attn_timed(const kvq_config* cfg, const kvq_cache* cache, const void* q, int32_t dtype, float* out,
                         int32_t max_seq_len_host, void* workspace, size_t ws_bytes, hipEvent_t split_begin,
                         hipEvent_t split_end, hipStream_t stream);

/* How kv_decode_attn splits its work for a batch of sequences up to max_seq_len tokens (host only; no device
   work): the quantized history of a sequence is cut into chunks of chunk_units groups of 128 tokens (grouped
   schemes) or pages of 64 tokens (INT4 per token), each chunk giving one softmax partial (m, l, o) that the
   merge combines ([OSCAR] §3.4.5 step 4, FlashDecoding; [NOVA] App. B.5, two-stage split-KV).  An explicit
   split_tokens fixes the chunks; 0 lets the library size them to the GPU.  On the matrix cores a sequence's
   chunks are split into `walks` runs of consecutive chunks (per head quad, or per kv head when the kv heads
   do not come in fours), one wave walking each run.  Balanced chunking (balanced = 1: the grouped schemes on
   the matrix cores, kv heads in fours, split_tokens = 0): the decode picks the chunk size on the device from
   the batch's actual lengths, the smallest G >= 4 groups whose chunks (ceil(groups / G) per sequence and head
   quad) fit the launch's chunk work-groups, one chunk per work-group; chunk_units, n_chunks and walks then
   report the choice for a batch whose every sequence has max_seq_len tokens, and max_chunks the most chunks
   one sequence can have (the workspace's bound).  Errors: KVQ_EINVAL (null out, batch < 1, negative
   length), config errors. */
typedef struct kvq_decode_shape {
  int32_t chunk_units;        /* groups (grouped schemes) or pages (INT4 per token) per chunk */
  int32_t n_chunks;           /* chunks of a sequence of max_seq_len tokens */
  int32_t walks;              /* runs of chunks per sequence and head quad (or kv head); n_chunks on the fp32 decode */
  int32_t span;               /* most chunks in one run (1 on the fp32 decode) */
  int32_t splitk_workgroups;  /* work-groups of the split-K launch, band work-groups included */
  int32_t band_first;         /* 1: the launch starts with its band work-groups */
  int32_t matrix_cores;       /* 1: the matrix-core decode runs, 0: the fp32 decode */
  int32_t balanced;           /* 1: balanced chunking, the chunk size chosen on the device from the lengths */
  int32_t max_chunks;         /* chunks of one sequence at most (partials per q head the workspace holds, less 1) */
} kvq_decode_shape;
int kvq_decode_shape_of(const kvq_config* cfg, int32_t batch, int32_t max_seq_len, kvq_decode_shape* out);

/* Read-bandwidth probe of the split-K decode (a measurement hook; it computes no attention).  It reads every
   quantized head block that kv_decode_attn's split-K kernel reads for lengths up to max_seq_len_host, with the
   same chunks, walks, work-groups and page-pair order ([OSCAR] §3.4.5, the paged INT2 cache and its chunked
   decode walk), and only folds the 32-bit words each walk read with XOR: xor_out[(b * n_kv_heads + h) * walks
   + w] (device, uint32, batch * n_kv_heads * walks words, `walks` from kvq_decode_shape_of) receives walk w's
   XOR for sequence b and kv head h, 0 for a walk with no quantized group.  Under balanced chunking the slots
   are [(b * n_kv_heads + h) * max_chunks + c], chunk c of the decode's choice for the actual lengths, and
   the slots past a sequence's chunk count are left as they were.  The band is not read.  Timing it
   gives the rate at which the GPU streams the decode's read pattern with no arithmetic beside it.  Grouped
   schemes on the matrix-core decode only: KVQ_EUNSUPPORTED for INT4 per token or decode_impl = fp32.  Other
   errors as kv_decode_attn (config, cache, KVQ_EINVAL for a null xor_out or negative length, KVQ_ERANGE when
   the length needs more pages than the page-table row holds, KVQ_EDEVICE on a launch error). */
int kvq_read_probe(const kvq_config* cfg, const kvq_cache* cache, uint32_t* xor_out, int32_t max_seq_len_host,
                   hipStream_t stream);

/* kv_decode_attn without a workspace argument, for callers that cannot allocate device memory (code under
   HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): it calls no hipMalloc, hipFree or
   allocating routine.  Its workspace is a file-scope device array of KVQ_NOALLOC_SCRATCH_BYTES (64 MiB) that
   every GPU the library runs on holds until the process ends; its address on the current device is looked up
   once per device.  Every call on a GPU shares that GPU's array, so calls that overlap on one GPU (other
   streams or threads) race: the caller orders them.  Nothing in it needs clearing between calls: every
   partial the merge reads is written by the same call.  Same arguments and results as kv_decode_attn;
   KVQ_ENOSPACE (checked on the host, nothing enqueued, kvq_last_error() gives the sizes) when
   kvq_decode_workspace_bytes(cfg, batch, max_seq_len_host) exceeds KVQ_NOALLOC_SCRATCH_BYTES. */
#define KVQ_NOALLOC_SCRATCH_BYTES (64u << 20)
int kv_decode_attn_noalloc(const kvq_config* cfg, const kvq_cache* cache, const void* q, int32_t dtype, float* out,
                           int32_t max_seq_len_host, hipStream_t stream);

/* Prefill attention over the quantized history ([NOVA] §3 "Long context": chunked prefill, every chunk
   quantized on write so later chunks attend to a quantized history; [SAW] prefill stage: save, read back,
   attend).  Call after kv_rotate_quant_write has appended the chunk: sequence b's chunk is its last
   n_b = cu_q[b+1] - cu_q[b] tokens (positions T_b - n_b .. T_b - 1, T_b = seq_lens[b] after the write),
   and its query at position p attends every cached token at a position <= p, as the cache holds it
   (bf16 band tokens and dequantized groups, or dequantized INT4 per-token pages, the chunk's own tokens
   included).  Every scheme and rotation.  Arithmetic: 24-bit fixed point (three signed byte limbs) against
   the codes on the int8 matrix cores, bf16 hi/lo splits for the band and the dense un-rotation, a fp32
   Walsh-Hadamard transform for the randomized Hadamard's.
     q     [total_q][n_q_heads][128] fp32 or bf16 (dtype), device; rows ordered by sequence then query.
     cu_q  [batch + 1] int32 prefix sums of n_b, device; total_q = cu_q[batch], max_q = max n_b (host).
     out   [total_q][n_q_heads][128] fp32, device, written for every query row.
     workspace of kvq_prefill_workspace_bytes(cfg, total_q) bytes (rotated and band-frame queries).
   KVQ_ENOSPACE for a small workspace; n_b must not exceed T_b (not checked on the device: queries beyond
   the cache attend nothing and output zeros). */
size_t kvq_prefill_workspace_bytes(const kvq_config* cfg, int32_t total_q);
int kv_prefill_attn(const kvq_config* cfg, const kvq_cache* cache, const void* q, int32_t dtype, const int32_t* cu_q,
                    int32_t total_q, int32_t max_q, float* out, void* workspace, size_t ws_bytes, hipStream_t stream);

/* Test hook: the write path's rotation (and clip when rho < 1) of n vectors x [n][128] (fp32 or bf16)
   to fp32 [n][128], using the cache's K (which = 0) or V (which = 1) rotation.  Not used by the hot path. */
int kvq_debug_rotate(const kvq_config* cfg, const kvq_cache* cache, int32_t which, const void* x, int32_t dtype,
                     int32_t n, float rho, float* out, hipStream_t stream);

/* Test hook: the first n_tokens_host quantized tokens of (sequence seq, kv head kv_head) read back from the
   pages in logical order (quantized token u is position S0 + u for the grouped schemes, position u for INT4
   per token), by the layout above.  Device outputs:
     codes_out  uint8 [n_tokens][2][128]: K codes, then V codes of each token;
     sz_out     bf16 bits, per-channel schemes [n_tokens / 128][2][2][128] (per group: K scales, K zeros,
                V scales, V zeros), per-token schemes [n_tokens][2][2] (per token: K scale, K zero, V scale,
                V zero).
   n_tokens_host must be a multiple of 128 for the grouped schemes.  Errors: KVQ_EINVAL, KVQ_ERANGE (more
   pages than max_pages_per_seq), KVQ_EDEVICE.  Not used by the hot path. */
int kvq_debug_unpack(const kvq_config* cfg, const kvq_cache* cache, int32_t seq, int32_t kv_head,
                     int32_t n_tokens_host, uint8_t* codes_out, uint16_t* sz_out, hipStream_t stream);

const char* kvq_strerror(int status);
/* Library version string. */
const char* kvq_version(void);
/* Text of the last KVQ_EDEVICE failure on the calling thread (the HIP error name and string, and the
   call that saw it); "" if none.  The pointer stays valid until the thread's next failing call. */
const char* kvq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H_ */
