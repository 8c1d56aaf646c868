// Read-bandwidth probe of the split-K decode (a measurement hook, no attention arithmetic).
//
// The probe reads exactly the quantized head blocks that the matrix-core split-K decode reads for the
// grouped schemes, with the decode's grid (the same chunks, walks, work-groups of head quads or kv-head rows,
// and page-pair order) and its streaming (non-temporal) read policy, one group (the two pages' head blocks
// of one kv head) at a time.  Each lane keeps the next group's 16-byte loads in flight while it folds the
// current group into a running XOR, and each wave stores the XOR of all 32-bit words its walk read.  Timing
// a launch gives the rate at which the GPU streams this read pattern when nothing else runs; the XOR lets a
// test confirm that the probe read the bytes the decode reads ([OSCAR] §3.4.5 paged INT2 cache layout; the
// decode's chunked walk follows [OSCAR] §3.4.5 step 4 and [NOVA] App. B.5, two-stage split-KV).
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kProbeThreads = 256;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// NK 1 KB wave loads per group: the two pages' head blocks of one kv head (2 x 4608 B for 2-bit codes,
// 2 x 8704 B for 4-bit codes), lane-contiguous 16-byte pieces
template <int NK>
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(DecodeArgs a, uint32_t* xor_out) {
  const Geo& g = a.g;
  const int i = blockIdx.x, lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int b, h, c0, c1, gpc = g.gpc;
  int w;  // this wave's walk index (the output slot)
  if (g.balanced) {
    // the decode's balanced chunking: one chunk of G groups per work-group, the chunk index is the slot
    gpc = balanced_gpc(g, a.seq_lens, lane);
    int quad, c;
    if (!balanced_wg(g, a.seq_lens, i, lane, gpc, b, quad, c)) return;
    h = 4 * quad + wave;
    c0 = c;
    c1 = c + 1;
    w = c;
  } else {
    (void)wave_chunk_of(g, i, wave, b, h, c0, c1);
    // a wave past the walks of its row has none
    if (splitk_head_quads(g)) {
      w = i / (g.batch * (g.n_kv / 4));
    } else {
      w = 4 * (i / (g.batch * g.n_kv)) + wave;
      if (w >= g.walks) return;
    }
  }
  const int T = a.seq_lens[b];
  const int ng = n_groups_of(T, g.S0, g.W);
  int g_first = c0 * gpc, g_end = c1 * gpc;
  if (g_end > ng) g_end = ng;
  if (g_end > (g.n_units - 1) * g.gpc) g_end = (g.n_units - 1) * g.gpc;  // the launch bound
  if (g_end > g.max_pages / 2) g_end = g.max_pages / 2;  // never index past the page-table row
  const int32_t* ptrow = a.page_table + (long long)b * g.max_pages;
  const long long hb = g.head_bytes, hoff = (long long)h * hb;
  auto load = [&](int gi, uint4 (&v)[NK]) {
    const uint8_t* p0 = a.pages + pool_page(g, ptrow[2 * gi]) * g.page_bytes + hoff;
    const uint8_t* p1 = a.pages + pool_page(g, ptrow[2 * gi + 1]) * g.page_bytes + hoff;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const long long off = 1024LL * k + 16 * lane;  // inside the 2 hb bytes of the group (NK KB = 2 hb)
      const uint8_t* src = off < hb ? p0 + off : p1 + (off - hb);
      const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));  // streaming, as the decode
      v[k] = make_uint4(w.x, w.y, w.z, w.w);
    }
  };
  uint32_t acc = 0;
  uint4 cur[NK], nxt[NK];
  if (g_first < g_end) load(g_first, cur);
  for (int gi = g_first; gi < g_end; ++gi) {
    if (gi + 1 < g_end) load(gi + 1, nxt);
#pragma unroll
    for (int k = 0; k < NK; ++k) acc ^= cur[k].x ^ cur[k].y ^ cur[k].z ^ cur[k].w;
#pragma unroll
    for (int k = 0; k < NK; ++k) cur[k] = nxt[k];
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, s, 64);
  if (lane == 0) xor_out[((long long)b * g.n_kv + h) * g.walks + w] = acc;
}

}  // namespace

hipError_t launch_read_probe(const DecodeArgs& a, uint32_t* xor_out, hipStream_t s) {
  const Geo& g = a.g;
  const dim3 grid(splitk_chunk_wgs(g)), block(kProbeThreads);
  if (2 * g.head_bytes == 9 * 1024) {
    hipLaunchKernelGGL(read_probe_kernel<9>, grid, block, 0, s, a, xor_out);
  } else if (2 * g.head_bytes == 17 * 1024) {
    hipLaunchKernelGGL(read_probe_kernel<17>, grid, block, 0, s, a, xor_out);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
