// api.hip -- the C ABI declared in include/prefill_attn.h: argument checks,
// optional metadata checks (check mode), grid sizing and the launch.
// Every step of the computation runs in the kernels of prefill_fwd.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "launch.h"
#include "quant_rows.h"
#include "prefill_attn.h"

namespace {

std::atomic<int> g_check_mode{-1};  // -1: not yet read from the environment
thread_local int t_last_hip_error = 0;

bool check_mode() {
  int m = g_check_mode.load(std::memory_order_relaxed);
  if (m < 0) {
    const char* e = std::getenv("PA_CHECK");
    m = (e && e[0] == '1') ? 1 : 0;
    int expected = -1;
    g_check_mode.compare_exchange_strong(expected, m);
    m = g_check_mode.load(std::memory_order_relaxed);
  }
  return m == 1;
}

// The 64-row kernel serves varlen head_dim-128 calls unless PA_FWD64=0 (kept
// for A/B measurements against the 32-row kernel).
bool fwd64_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("PA_FWD64");
    return !(e && e[0] == '0');
  }();
  return on;
}

pa_status hip_fail(hipError_t e) {
  t_last_hip_error = (int)e;
  return PA_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Host-side checks shared by both entry points.
pa_status check_common(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const int32_t* cu, int32_t num_seqs, int32_t max_seqlen,
                       int32_t num_heads, int32_t head_dim, const uint16_t* kc,
                       const uint16_t* vc, const uint16_t* out, float scale) {
  if (!q || !k || !v || !cu || !kc || !vc || !out) return PA_ERR_NULL;
  if (num_seqs < 0 || max_seqlen < 0 || num_heads < 1) return PA_ERR_SHAPE;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128) return PA_ERR_HEAD_DIM;
  if (!std::isfinite(scale)) return PA_ERR_SCALE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(kc) || !aligned16(vc) ||
      !aligned16(out))
    return PA_ERR_ALIGN;
  const void* outs[3] = {kc, vc, out};
  const void* ins[4] = {q, k, v, cu};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 4; ++j)
      if (outs[i] == ins[j]) return PA_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (outs[i] == outs[j]) return PA_ERR_ALIAS;
  }
  return PA_OK;
}

// Grid limits: x = heads, y = sequences, z = query blocks.
pa_status check_grid(int32_t num_seqs, int32_t max_seqlen, int32_t num_heads, int* grid_z) {
  const int z = pa::fwd_grid_blocks(max_seqlen);
  if (num_seqs > 65535 || z > 65535 || num_heads > 65535) return PA_ERR_SHAPE;
  *grid_z = z;
  return PA_OK;
}

// Check mode: copy metadata to the host on `stream`, wait, validate.
pa_status check_metadata(const int32_t* cu, int32_t num_seqs, int32_t max_seqlen,
                         const int32_t* prefix, int32_t cap, hipStream_t stream) {
  std::vector<int32_t> hcu(num_seqs + 1), hpre(prefix ? num_seqs : 0);
  hipError_t e = hipMemcpyAsync(hcu.data(), cu, sizeof(int32_t) * (num_seqs + 1),
                                hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return hip_fail(e);
  if (prefix) {
    e = hipMemcpyAsync(hpre.data(), prefix, sizeof(int32_t) * num_seqs, hipMemcpyDeviceToHost,
                       stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e);
  if (hcu[0] != 0) return PA_ERR_SEQLENS;
  for (int b = 0; b < num_seqs; ++b) {
    const int64_t n = (int64_t)hcu[b + 1] - hcu[b];
    if (n < 0 || n > max_seqlen) return PA_ERR_SEQLENS;
    if (prefix) {
      if (hpre[b] < 0 || (int64_t)hpre[b] + n > cap) return PA_ERR_CAPACITY;
    }
  }
  return PA_OK;
}

// Check mode, paged cache: every block a sequence touches (positions below
// prefix + length) names a block of the pool.
pa_status check_block_table(const int32_t* cu, const int32_t* prefix, int32_t num_seqs,
                            const int32_t* bt, int32_t max_blocks, int32_t num_blocks,
                            hipStream_t stream) {
  std::vector<int32_t> hcu(num_seqs + 1), hpre(num_seqs), hbt((size_t)num_seqs * max_blocks);
  hipError_t e = hipMemcpyAsync(hcu.data(), cu, sizeof(int32_t) * (num_seqs + 1),
                                hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(hpre.data(), prefix, sizeof(int32_t) * num_seqs, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(hbt.data(), bt, sizeof(int32_t) * hbt.size(), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e);
  for (int b = 0; b < num_seqs; ++b) {
    const int64_t used = ((int64_t)hpre[b] + hcu[b + 1] - hcu[b] + pa::kPageRows - 1) / pa::kPageRows;
    for (int64_t i = 0; i < used; ++i) {
      const int32_t blk = hbt[(size_t)b * max_blocks + i];
      if (blk < 0 || blk >= num_blocks) return PA_ERR_CAPACITY;
    }
  }
  return PA_OK;
}

// a quantised varlen cache: one-byte codes laid out as the bf16 cache, one
// float scale per (token, K/V head) row
struct QuantCache {
  void* kq;
  void* vq;
  float* ks;
  float* vs;
  bool fp8;  // E4M3 codes; otherwise INT8
};

pa_status run(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* cu,
              int32_t num_seqs, int32_t max_seqlen, int32_t num_heads, int32_t num_kv_heads,
              int32_t head_dim, uint16_t* kc, uint16_t* vc, int32_t cap, uint16_t* out,
              float scale, hipStream_t stream, const int32_t* prefix,
              const QuantCache* qc = nullptr) {
  if (num_kv_heads < 1 || num_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
  int nqb = 0;
  pa_status st = check_grid(num_seqs, max_seqlen, num_heads, &nqb);
  if (st != PA_OK) return st;
  if (num_seqs == 0 || max_seqlen == 0) return PA_OK;
  if (check_mode()) {
    st = check_metadata(cu, num_seqs, max_seqlen, prefix, cap, stream);
    if (st != PA_OK) return st;
  }
  pa::FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.cu = cu;
  p.prefix = prefix;
  p.kc = kc;
  p.vc = vc;
  p.out = out;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.cap = cap;
  p.grid_z = nqb;
  // scale * q.k == |scale| * (sign(scale) q).k : keep the exp2-domain factor
  // non-negative so the kernel can take the row max before scaling
  // |scale| log2(e), kept >= 2^-100 so that a masked score (-inf) always gives
  // 2^(-inf * c - m) = 0 without a select; below that bound every |s| c is far
  // under fp32 resolution of 1, so the weights are exactly uniform either way.
  p.scale_log2 = (float)std::fmax(std::fabs((double)scale) * 1.4426950408889634, 0x1p-100);
  p.neg_q = scale < 0.f ? 1 : 0;
  hipError_t e;
  const bool rows64 =
      pa::fwd64_supported(head_dim, prefix != nullptr, scale, max_seqlen, num_heads, num_kv_heads) && fwd64_enabled();
  if (qc) {
    p.kq = static_cast<int8_t*>(qc->kq);
    p.vq = static_cast<int8_t*>(qc->vq);
    p.ks = qc->ks;
    p.vs = qc->vs;
    if (rows64)
      e = pa::launch_prefill_fwd64(p, num_seqs, qc->fp8 ? pa::qrow::kCacheFp8 : pa::qrow::kCacheInt8, stream);
    else
      e = qc->fp8 ? pa::launch_prefill_fwd_fp8(p, num_seqs, head_dim, stream)
                  : pa::launch_prefill_fwd_int8(p, num_seqs, head_dim, stream);
  } else if (rows64) {
    e = pa::launch_prefill_fwd64(p, num_seqs, pa::qrow::kCacheBf16, stream);
  } else {
    e = pa::launch_prefill_fwd(p, num_seqs, head_dim, prefix != nullptr, stream);
  }
  if (e != hipSuccess) return hip_fail(e);
  return PA_OK;
}

// Compute units of the current device and resident split-attention
// work-groups per unit, queried once per device and head size.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];
std::atomic<int> g_split_occ[kMaxDevices][3][2];
std::atomic<int> g_dec_occ[kMaxDevices][3][4][2];
// Share of the split-KV work-groups that starts on the attention items (the
// rest start on the decode rows' units): with streaming decode loads the
// decode units need fewer work-groups to hold HBM busy, and about 30 % on the
// items balanced the heaviest chunked step (too few, and the long items
// finish last).
constexpr int kItemsFirstPercent = 31;
constexpr int kFuseMaxHeads = 2;
static_assert(kFuseMaxHeads <= 2, "the mixed kernel has decode units of one and two query heads only");

// Whether the decode rows run inside the split attention launch.  There they
// run beside the items, but with 8 waves per compute unit instead of 16; that
// pays where a row's unit streams K/V (one query head per K/V head) and
// costs where it computes (grouped heads: 4 or 8 query heads per load).
bool fuse_decode(int heads_per_unit) { return heads_per_unit <= kFuseMaxHeads; }

// Work-groups of the split-KV attention launch (resident ones only: it is
// persistent), the share of them that starts on the attention items when the
// decode rows run in the same launch, and the merge grid.
pa_status split_grid(int head_dim, bool fused, int* fwd_grid, int* items_first, int* merge_grid) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return hip_fail(hipErrorInvalidDevice);
  int cus = g_cus[dev].load(std::memory_order_relaxed);
  if (cus <= 0) {
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e);
    g_cus[dev].store(cus, std::memory_order_relaxed);
  }
  const int di = head_dim == 32 ? 0 : head_dim == 64 ? 1 : 2;
  int occ = g_split_occ[dev][di][fused].load(std::memory_order_relaxed);
  if (occ <= 0) {
    occ = pa::fwd_split_blocks_per_cu(head_dim, fused);
    if (occ <= 0) return hip_fail(hipErrorInvalidConfiguration);
    g_split_occ[dev][di][fused].store(occ, std::memory_order_relaxed);
  }
  *fwd_grid = cus * occ;
  // a multiple of 8: every XCD the same number
  *items_first = std::min(*fwd_grid, std::max(8, *fwd_grid * kItemsFirstPercent / 100 / 8 * 8));
  *merge_grid = cus * 8;
  return PA_OK;
}

// Work-groups of the separate decode launch: all resident ones.
pa_status decode_grid(int head_dim, int heads_per_unit, bool paged, int* grid) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return hip_fail(hipErrorInvalidDevice);
  const int cus = g_cus[dev].load(std::memory_order_relaxed);  // set by split_grid
  if (cus <= 0) return hip_fail(hipErrorInvalidConfiguration);
  const int di = head_dim == 32 ? 0 : head_dim == 64 ? 1 : 2;
  const int gi = heads_per_unit == 1 ? 0 : heads_per_unit == 2 ? 1 : heads_per_unit == 4 ? 2 : 3;
  int occ = g_dec_occ[dev][di][gi][paged].load(std::memory_order_relaxed);
  if (occ <= 0) {
    occ = pa::splitkv_decode_blocks_per_cu(head_dim, heads_per_unit, paged);
    if (occ <= 0) return hip_fail(hipErrorInvalidConfiguration);
    g_dec_occ[dev][di][gi][paged].store(occ, std::memory_order_relaxed);
  }
  *grid = cus * occ;
  return PA_OK;
}

}  // namespace

extern "C" {

size_t prefill_attn_splitkv_workspace_size(int32_t num_seqs, int32_t num_tokens,
                                           int32_t num_heads, int32_t head_dim,
                                           int32_t cache_capacity) {
  if (num_seqs < 0 || num_tokens < 0 || num_heads < 1 || cache_capacity < 1) return 0;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128) return 0;
  return pa::split_layout(num_seqs, num_tokens, num_heads, head_dim, cache_capacity).bytes;
}

}  // extern "C"

namespace {

// Split-KV chunked call; block_table non-NULL selects the paged cache
// ([num_blocks, HK, 16, D], cache_capacity = 16 * max_blocks_per_seq).
pa_status splitkv_run(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                      int32_t num_tokens, int32_t num_heads, int32_t num_kv_heads,
                      int32_t head_dim, uint16_t* k_cache, uint16_t* v_cache,
                      int32_t cache_capacity, uint16_t* out, float scale, hipStream_t stream,
                      const int32_t* prefix_lens, void* workspace, size_t workspace_bytes,
                      const int32_t* block_table, int32_t max_blocks_per_seq,
                      int32_t num_blocks, bool host_checks = true) {
  pa_status st = check_common(q, k, v, cu_seqlens, num_seqs, max_seqlen, num_heads, head_dim,
                              k_cache, v_cache, out, scale);
  if (st != PA_OK) return st;
  if (!prefix_lens || !workspace) return PA_ERR_NULL;
  const void* outs[4] = {k_cache, v_cache, out, workspace};
  const void* ins[5] = {q, k, v, cu_seqlens, prefix_lens};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 5; ++j)
      if (outs[i] == ins[j]) return PA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (outs[i] == outs[j]) return PA_ERR_ALIAS;
  }
  if (!aligned16(workspace)) return PA_ERR_ALIGN;
  if (cache_capacity < 1 || num_tokens < 0) return PA_ERR_SHAPE;
  // the decode pass addresses positions of one slab row with 32-bit element offsets
  if (!block_table && (int64_t)cache_capacity * head_dim > (int64_t)UINT32_MAX) return PA_ERR_SHAPE;
  if (num_kv_heads < 1 || num_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
  int nqb = 0;
  st = check_grid(num_seqs, max_seqlen, num_heads, &nqb);
  if (st != PA_OK) return st;
  const pa::SplitLayout L =
      pa::split_layout(num_seqs, num_tokens, num_heads, head_dim, cache_capacity);
  if (workspace_bytes < L.bytes) return PA_ERR_WORKSPACE;
  if (num_seqs == 0 || max_seqlen == 0 || num_tokens == 0) return PA_OK;
  if (host_checks && check_mode()) {
    st = check_metadata(cu_seqlens, num_seqs, max_seqlen, prefix_lens, cache_capacity, stream);
    if (st != PA_OK) return st;
    if (block_table) {
      st = check_block_table(cu_seqlens, prefix_lens, num_seqs, block_table, max_blocks_per_seq,
                             num_blocks, stream);
      if (st != PA_OK) return st;
    }
    int32_t last = 0;
    hipError_t e = hipMemcpyAsync(&last, cu_seqlens + num_seqs, sizeof(int32_t),
                                  hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e);
    if (last > num_tokens) return PA_ERR_SEQLENS;
  }
  const bool paged = block_table != nullptr;
  // One sequence with several rows (a prompt chunk over its cached prefix):
  // its new K/V rows go to the cache first, then split-KV items on the
  // 64-row kernel read every key from there, and the merge combines the
  // segments.
  if (!paged && num_seqs == 1 && max_seqlen > 1 &&
      pa::fwd64_split_supported(head_dim, scale, max_seqlen, num_heads, cache_capacity)) {
    char* ws = static_cast<char*>(workspace);
    pa::FwdParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.cu = cu_seqlens;
    p.prefix = prefix_lens;
    p.kc = k_cache;
    p.vc = v_cache;
    p.out = out;
    p.num_heads = num_heads;
    p.num_kv_heads = num_kv_heads;
    p.cap = cache_capacity;
    p.scale_log2 = (float)std::fmax(std::fabs((double)scale) * 1.4426950408889634, 0x1p-100);
    p.hdr = reinterpret_cast<const int32_t*>(ws + L.off_hdr);
    p.items = reinterpret_cast<const int4*>(ws + L.off_items);
    p.part_lse = reinterpret_cast<float*>(ws + L.off_lse);
    p.part_o = reinterpret_cast<float*>(ws + L.off_o);
    p.seg_tiles = L.seg_tiles;
    p.max_segs = L.max_segs;
    int fwd_grid = 0, items_first = 0, merge_grid = 0;
    st = split_grid(head_dim, false, &fwd_grid, &items_first, &merge_grid);
    if (st != PA_OK) return st;
    // items sized so that the units (item, head) number about two per
    // compute unit (a work-group runs two); the plan launch also appends the
    // new K/V rows to the cache
    int cus = 0;
    {
      int dev = 0;
      hipError_t e0 = hipGetDevice(&dev);
      if (e0 == hipSuccess) cus = g_cus[dev].load(std::memory_order_relaxed);  // set by split_grid
    }
    const int fill = std::max(1, 2 * std::max(cus, 1) / num_heads);
    hipError_t e = pa::launch_splitkv_plan(cu_seqlens, prefix_lens, num_seqs, num_tokens, L, 1, 2, ws,
                                           stream, /*rows_as_items=*/true, &p, head_dim, fill);
    if (e == hipSuccess) e = pa::launch_prefill_fwd64_split(p, L.max_items, stream);
    if (e == hipSuccess) e = pa::launch_splitkv_merge(p, L, ws, head_dim, merge_grid, stream);
    if (e != hipSuccess) return hip_fail(e);
    return PA_OK;
  }
  const int gc = pa::splitkv_heads_per_unit(num_heads, num_kv_heads);
  // only a batch that may hold both multi-token blocks and length-1 rows
  // gains from running them together (one lone sequence, or rows of length
  // at most 1, leave one kind of work empty)
  const bool fused = fuse_decode(gc) && num_seqs > 1 && max_seqlen > 1;
  int fwd_grid = 0, items_first = 0, merge_grid = 0, dec_grid = 0;
  st = split_grid(head_dim, fused, &fwd_grid, &items_first, &merge_grid);
  if (st == PA_OK && !fused) st = decode_grid(head_dim, gc, paged, &dec_grid);
  if (st != PA_OK) return st;

  char* ws = static_cast<char*>(workspace);
  pa::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.cu = cu_seqlens;
  p.prefix = prefix_lens;
  p.kc = k_cache;
  p.vc = v_cache;
  p.out = out;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.cap = cache_capacity;
  p.grid_z = nqb;
  p.scale_log2 = (float)std::fmax(std::fabs((double)scale) * 1.4426950408889634, 0x1p-100);
  p.neg_q = scale < 0.f ? 1 : 0;
  p.hdr = reinterpret_cast<const int32_t*>(ws + L.off_hdr);
  p.items = reinterpret_cast<const int4*>(ws + L.off_items);
  p.part_lse = reinterpret_cast<float*>(ws + L.off_lse);
  p.part_o = reinterpret_cast<float*>(ws + L.off_o);
  p.seg_tiles = L.seg_tiles;
  p.max_segs = L.max_segs;
  p.split_grid = fwd_grid;
  p.dec_items = reinterpret_cast<const int4*>(ws + L.off_dec);
  p.dec_heads = gc;
  p.fuse_decode = fused ? 1 : 0;
  p.items_first = fused ? items_first : fwd_grid;
  p.counters = reinterpret_cast<unsigned long long*>(ws + L.off_ctr);
  p.dec_grid = dec_grid;
  p.block_table = block_table;
  p.bt_stride = max_blocks_per_seq;
  hipError_t e = pa::launch_splitkv_plan(cu_seqlens, prefix_lens, num_seqs, num_tokens, L,
                                         fused ? 4 : 1, fused ? 8 : 4, ws, stream);
  // with every row of length 1 the plan makes no attention items: only the
  // decode launch has work
  if (e == hipSuccess && (fused || max_seqlen > 1)) e = pa::launch_prefill_fwd_split(p, head_dim, paged, stream);
  if (e == hipSuccess && !fused) e = pa::launch_splitkv_decode(p, head_dim, paged, stream);
  if (e == hipSuccess) e = pa::launch_splitkv_merge(p, L, ws, head_dim, merge_grid, stream);
  if (e != hipSuccess) return hip_fail(e);
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status prefill_attn_chunked_splitkv(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                       const int32_t* cu_seqlens, int32_t num_seqs,
                                       int32_t max_seqlen, int32_t num_tokens, int32_t num_heads,
                                       int32_t num_kv_heads, int32_t head_dim, uint16_t* k_cache,
                                       uint16_t* v_cache, int32_t cache_capacity, uint16_t* out,
                                       float scale, hipStream_t stream,
                                       const int32_t* prefix_lens, void* workspace,
                                       size_t workspace_bytes) {
  return splitkv_run(q, k, v, cu_seqlens, num_seqs, max_seqlen, num_tokens, num_heads,
                     num_kv_heads, head_dim, k_cache, v_cache, cache_capacity, out, scale, stream,
                     prefix_lens, workspace, workspace_bytes, nullptr, 0, 0);
}

}  // extern "C"

namespace {

// Scratch of prefill_attn_chunked_splitkv_noalloc: one array per GPU, in
// place of the caller's workspace, held until the process ends.  In host
// code `scratch` only stands for the symbol: its device address on each
// device comes from hipGetSymbolAddress (noalloc_scratch) and only that
// address is passed on.
constexpr size_t kNoAllocScratchBytes = (size_t)128 << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The current device's scratch address, looked up on the first call on that
// device (with it current, as every call here launches on the current
// device).
pa_status noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return hip_fail(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!ptr) return hip_fail(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

size_t prefill_attn_splitkv_noalloc_limit(void) { return kNoAllocScratchBytes; }

pa_status prefill_attn_chunked_splitkv_noalloc(const uint16_t* q, const uint16_t* k,
                                               const uint16_t* v, const int32_t* cu_seqlens,
                                               int32_t num_seqs, int32_t max_seqlen,
                                               int32_t num_tokens, int32_t num_heads,
                                               int32_t num_kv_heads, int32_t head_dim,
                                               uint16_t* k_cache, uint16_t* v_cache,
                                               int32_t cache_capacity, uint16_t* out, float scale,
                                               hipStream_t stream, const int32_t* prefix_lens) {
  // the problem's workspace must fit the array (0: invalid sizes, which the
  // common checks below report)
  const size_t need = prefill_attn_splitkv_workspace_size(num_seqs, num_tokens, num_heads,
                                                          head_dim, cache_capacity);
  if (need > kNoAllocScratchBytes) return PA_ERR_NOALLOC_LIMIT;
  void* ws = nullptr;
  pa_status st = noalloc_scratch(&ws);
  if (st != PA_OK) return st;
  return splitkv_run(q, k, v, cu_seqlens, num_seqs, max_seqlen, num_tokens, num_heads,
                     num_kv_heads, head_dim, k_cache, v_cache, cache_capacity, out, scale, stream,
                     prefix_lens, ws, kNoAllocScratchBytes, nullptr, 0, 0, /*host_checks=*/false);
}

pa_status prefill_attn_chunked_splitkv_paged(
    const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* cu_seqlens,
    int32_t num_seqs, int32_t max_seqlen, int32_t num_tokens, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_dim, uint16_t* k_cache, uint16_t* v_cache,
    int32_t num_blocks, const int32_t* block_table, int32_t max_blocks_per_seq, uint16_t* out,
    float scale, hipStream_t stream, const int32_t* prefix_lens, void* workspace,
    size_t workspace_bytes) {
  if (!block_table) return PA_ERR_NULL;
  if (num_blocks < 1 || max_blocks_per_seq < 1 || max_blocks_per_seq > (1 << 26)) return PA_ERR_SHAPE;
  if ((const void*)block_table == (const void*)k_cache ||
      (const void*)block_table == (const void*)v_cache || (const void*)block_table == (const void*)out ||
      (const void*)block_table == workspace)
    return PA_ERR_ALIAS;
  return splitkv_run(q, k, v, cu_seqlens, num_seqs, max_seqlen, num_tokens, num_heads,
                     num_kv_heads, head_dim, k_cache, v_cache, max_blocks_per_seq * pa::kPageRows,
                     out, scale, stream, prefix_lens, workspace, workspace_bytes, block_table,
                     max_blocks_per_seq, num_blocks);
}

pa_status prefill_attn_varlen_gqa(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                                  int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                  uint16_t* k_cache, uint16_t* v_cache, uint16_t* out,
                                  float scale, hipStream_t stream) {
  pa_status st = check_common(q, k, v, cu_seqlens, num_seqs, max_seqlen, num_heads, head_dim,
                              k_cache, v_cache, out, scale);
  if (st != PA_OK) return st;
  return run(q, k, v, cu_seqlens, num_seqs, max_seqlen, num_heads, num_kv_heads, head_dim,
             k_cache, v_cache, 0, out, scale, stream, nullptr);
}

pa_status prefill_attn_chunked_gqa(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   const int32_t* cu_seqlens, int32_t num_seqs,
                                   int32_t max_seqlen, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_dim, uint16_t* k_cache, uint16_t* v_cache,
                                   int32_t cache_capacity, uint16_t* out, float scale,
                                   hipStream_t stream, const int32_t* prefix_lens) {
  pa_status st = check_common(q, k, v, cu_seqlens, num_seqs, max_seqlen, num_heads, head_dim,
                              k_cache, v_cache, out, scale);
  if (st != PA_OK) return st;
  if (!prefix_lens) return PA_ERR_NULL;
  if ((const void*)prefix_lens == (const void*)k_cache ||
      (const void*)prefix_lens == (const void*)v_cache || (const void*)prefix_lens == (const void*)out)
    return PA_ERR_ALIAS;
  if (cache_capacity < 1) return PA_ERR_SHAPE;
  return run(q, k, v, cu_seqlens, num_seqs, max_seqlen, num_heads, num_kv_heads, head_dim,
             k_cache, v_cache, cache_capacity, out, scale, stream, prefix_lens);
}

}  // extern "C"

namespace {
pa_status quant_run(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* cu_seqlens,
                    int32_t num_seqs, int32_t max_seqlen, int32_t num_heads, int32_t num_kv_heads,
                    int32_t head_dim, void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                    uint16_t* out, float scale, hipStream_t stream, bool fp8) {
  if (!k_scale || !v_scale) return PA_ERR_NULL;
  // the bf16 checks cover q, k, v, cu, out and the code buffers
  pa_status st = check_common(q, k, v, cu_seqlens, num_seqs, max_seqlen, num_heads, head_dim,
                              static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache),
                              out, scale);
  if (st != PA_OK) return st;
  if (!aligned16(k_scale) || !aligned16(v_scale)) return PA_ERR_ALIGN;
  const void* outs[5] = {k_cache, v_cache, out, k_scale, v_scale};
  const void* ins[4] = {q, k, v, cu_seqlens};
  for (int i = 0; i < 5; ++i) {
    for (int j = 0; j < 4; ++j)
      if (outs[i] == ins[j]) return PA_ERR_ALIAS;
    for (int j = i + 1; j < 5; ++j)
      if (outs[i] == outs[j]) return PA_ERR_ALIAS;
  }
  const QuantCache qc{k_cache, v_cache, k_scale, v_scale, fp8};
  return run(q, k, v, cu_seqlens, num_seqs, max_seqlen, num_heads, num_kv_heads, head_dim,
             nullptr, nullptr, 0, out, scale, stream, nullptr, &qc);
}
}  // namespace

extern "C" {

pa_status prefill_attn_varlen_int8(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   const int32_t* cu_seqlens, int32_t num_seqs,
                                   int32_t max_seqlen, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int8_t* k_cache, int8_t* v_cache,
                                   float* k_scale, float* v_scale, uint16_t* out, float scale,
                                   hipStream_t stream) {
  return quant_run(q, k, v, cu_seqlens, num_seqs, max_seqlen, num_heads, num_kv_heads, head_dim, k_cache,
                   v_cache, k_scale, v_scale, out, scale, stream, false);
}

pa_status prefill_attn_varlen_fp8(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  const int32_t* cu_seqlens, int32_t num_seqs,
                                  int32_t max_seqlen, int32_t num_heads, int32_t num_kv_heads,
                                  int32_t head_dim, uint8_t* k_cache, uint8_t* v_cache,
                                  float* k_scale, float* v_scale, uint16_t* out, float scale,
                                  hipStream_t stream) {
  return quant_run(q, k, v, cu_seqlens, num_seqs, max_seqlen, num_heads, num_kv_heads, head_dim, k_cache,
                   v_cache, k_scale, v_scale, out, scale, stream, true);
}

pa_status prefill_attn_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                              int32_t num_heads, int32_t head_dim, uint16_t* k_cache,
                              uint16_t* v_cache, uint16_t* out, float scale,
                              hipStream_t stream) {
  return prefill_attn_varlen_gqa(q, k, v, cu_seqlens, num_seqs, max_seqlen, num_heads, num_heads,
                                 head_dim, k_cache, v_cache, out, scale, stream);
}

pa_status prefill_attn_chunked(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                               int32_t num_heads, int32_t head_dim, uint16_t* k_cache,
                               uint16_t* v_cache, int32_t cache_capacity, uint16_t* out,
                               float scale, hipStream_t stream, const int32_t* prefix_lens) {
  return prefill_attn_chunked_gqa(q, k, v, cu_seqlens, num_seqs, max_seqlen, num_heads, num_heads,
                                  head_dim, k_cache, v_cache, cache_capacity, out, scale, stream,
                                  prefix_lens);
}

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK: success";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: invalid count or size (num_seqs, max_seqlen, num_heads, num_kv_heads not dividing num_heads, cache_capacity or grid limit)";
    case PA_ERR_HEAD_DIM: return "PA_ERR_HEAD_DIM: head_dim must be 32, 64 or 128";
    case PA_ERR_SCALE: return "PA_ERR_SCALE: scale must be finite";
    case PA_ERR_ALIGN: return "PA_ERR_ALIGN: tensor pointers must be 16-byte aligned";
    case PA_ERR_ALIAS: return "PA_ERR_ALIAS: an output aliases an input or another output";
    case PA_ERR_SEQLENS: return "PA_ERR_SEQLENS: cu_seqlens must start at 0, be non-decreasing and have lengths <= max_seqlen";
    case PA_ERR_CAPACITY: return "PA_ERR_CAPACITY: prefix_lens must be >= 0 with prefix + length <= cache_capacity";
    case PA_ERR_HIP: return "PA_ERR_HIP: a HIP runtime call failed (see pa_last_hip_error)";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace smaller than prefill_attn_splitkv_workspace_size()";
    case PA_ERR_NOALLOC_LIMIT: return "PA_ERR_NOALLOC_LIMIT: the problem needs more scratch than prefill_attn_splitkv_noalloc_limit() bytes";
    default: return "unknown pa_status";
  }
}

int pa_set_check_mode(int on) {
  int prev = check_mode() ? 1 : 0;
  g_check_mode.store(on ? 1 : 0, std::memory_order_relaxed);
  return prev;
}

int pa_last_hip_error(void) { return t_last_hip_error; }

}  // extern "C"
