// splitkv.hip -- split-KV chunked prefill: the plan that cuts every query
// block's keys into segments, and the log-sum-exp merge of the segments'
// partial results.  The attention over each segment, and the length-1 rows,
// run in prefill_fwd_split_kernel (prefill_fwd.hip, decode_rows.h).
//
// Why: in a chunked-prefill step a prompt chunk runs beside many decode rows
// ["大模型 Prompt Prefill 阶段的高效 Batching 与算子排布" §3], and decode
// attention reads every cached position of its row
// (untitled page www.zwxr.cn/news/300951 §3.3).  One work-group per query
// block then walks up to cap / 64 key tiles in series, and a batch with few
// long rows leaves most compute units idle.  Splitting the keys of a block
// into segments of seg_tiles tiles gives independent items; a row's softmax
// over the union of segments is recovered exactly (in real arithmetic) from
// each segment's normalised output O_s and L_s = log2 sum_j 2^(s_j c):
//     out = sum_s 2^(L_s - M) O_s / sum_s 2^(L_s - M),   M = max_s L_s.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_rows.h"
#include "launch.h"

namespace pa {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kMinSegTiles = 16;  // 1024 keys per segment at least
constexpr int kMaxSegs = 64;      // segments per block at most (bounds the workspace)
constexpr int kMergeRows = 16;    // rows per merge entry (4 waves x 4 rows)
constexpr int kPlanThreads = 256;  // one wave per SIMD: registers for the 64-bit offsets without spilling
static_assert(kSplitCounters <= kPlanThreads, "the plan zeroes one counter per thread");

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __builtin_amdgcn_ds_bpermute(4 * (lane - o), x);
    if (lane >= o) x += y;
  }
  return x;
}

__device__ __forceinline__ float wave_max(float x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1)
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (lane ^ o), __float_as_int(x))));
  return x;
}

__device__ __forceinline__ float wave_sum(float x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1)
    x += __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (lane ^ o), __float_as_int(x)));
  return x;
}

__device__ __forceinline__ float lane_value(float x, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(4 * src, __float_as_int(x)));
}

struct SeqPlan {
  int items, dec, merges;
};

// Segments of a block whose keys span ntiles tiles: decode rows (one query,
// HBM-bound) take segments of about dec_mult * seg_tiles tiles, blocks of
// several rows (MFMA-bound, 128-row partial outputs) about item_mult *
// seg_tiles.  With separate launches short decode segments measured faster
// (dec_mult 1: more units in flight) and item_mult 4 beat 2 (fewer partials
// to write and merge).  When the decode rows run beside the items in one
// launch, long segments of both kinds measured faster (dec_mult 4: its one
// work-group per compute unit pays a fixed cost per unit; item_mult 8: the
// decode units keep the compute units busy while fewer, longer items run, and
// most blocks then need no merge).  item_tiles = item_mult * seg_tiles, or
// the fill target of the plan (see splitkv_plan_kernel).  At most max_segs.
// Segment s covers
// tiles [s * ntiles / ns, (s + 1) * ntiles / ns).
__device__ __forceinline__ int block_segments(int ntiles, bool decode_row, int seg_tiles, int max_segs,
                                              int dec_mult, int item_tiles) {
  const int target = decode_row ? dec_mult * seg_tiles : item_tiles;
  return min((ntiles + target - 1) / target, max_segs);
}

// Segments of every query block of one sequence (work items; a length-1
// sequence's go to the decode list when dec_rows is set), and the merge entries of the blocks with
// more than one segment.  Segment counts are capped at max_segs, so malformed
// metadata cannot address outside the workspace.
__device__ SeqPlan count_seq(int len, int pre, int seg_tiles, int max_segs, int dec_mult, int item_tiles,
                            bool dec_rows) {
  SeqPlan r{0, 0, 0};
  const bool row = dec_rows && len == 1;
  for (int q0 = 0; q0 < len; q0 += kQueryBlock) {
    const int qend = min(q0 + kQueryBlock, len);
    const int ntiles = (pre + qend + kKeyTile - 1) / kKeyTile;
    const int ns = block_segments(ntiles, row, seg_tiles, max_segs, dec_mult, item_tiles);
    if (ns < 1) continue;
    if (row)
      r.dec += ns;
    else
      r.items += ns;
    if (ns > 1) r.merges += (qend - q0 + kMergeRows - 1) / kMergeRows;
  }
  return r;
}

// New K/V rows for the cache, copied by the plan launch's other work-groups
// when the attention pass reads every key from the cache.
struct AppendArgs {
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* kc;
  uint16_t* vc;
  int num_kv_heads, cap, head_dim;
  int64_t rows;  // tokens x K/V heads
};

// Chunk i (16 bytes, K rows then V rows) of every new token's K and V row
// into the cache slab [B, HK, cap, D] at position prefix + (token - cu[b]);
// tokens past cu[num_seqs], and positions outside the capacity, are left alone.
__device__ __forceinline__ void append_chunk(int64_t i, const AppendArgs& a, const int32_t* __restrict__ cu,
                                             const int32_t* __restrict__ prefix, int num_seqs) {
  const int cpr = a.head_dim / 8;      // 16-byte chunks per row
  const int64_t chunks = a.rows * cpr;
  if (i >= 2 * chunks) return;
  const bool is_v = i >= chunks;
  const int64_t j = is_v ? i - chunks : i;
  const int64_t row = j / cpr;         // token * HK + hk
  const int c = (int)(j - row * cpr);
  const int hk = (int)(row % a.num_kv_heads);
  const int tok = (int)(row / a.num_kv_heads);
  if (tok >= cu[num_seqs]) return;
  int lo = 0, hi = num_seqs - 1;       // sequence lo: cu[lo] <= tok < cu[lo + 1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= tok) lo = mid; else hi = mid - 1;
  }
  const int pos = prefix[lo] + tok - cu[lo];
  if (pos < 0 || pos >= a.cap) return;
  const uint4 w = *reinterpret_cast<const uint4*>((is_v ? a.v : a.k) + row * a.head_dim + 8 * c);
  uint16_t* dst = (is_v ? a.vc : a.kc) + (((int64_t)lo * a.num_kv_heads + hk) * a.cap + pos) * a.head_dim + 8 * c;
  *reinterpret_cast<uint4*>(dst) = w;
}

// Work-group 0 plans.  Sequences are taken 256 at a time; each thread counts
// its sequence's items and merge entries, a work-group scan gives the
// offsets, and the thread writes them.  hdr[0], hdr[1] receive the totals.
// Work-groups 1 onward (when a.rows > 0) append the new K/V rows.
__global__ __launch_bounds__(kPlanThreads)
void splitkv_plan_kernel(const int32_t* __restrict__ cu, const int32_t* __restrict__ prefix,
                         int num_seqs, int num_tokens, int seg_tiles, int max_segs, int dec_mult, int item_mult,
                         int dec_rows, int64_t max_items, int64_t max_dec, int64_t max_merges,
                         int32_t* __restrict__ hdr, int4* __restrict__ items,
                         int4* __restrict__ dec, int4* __restrict__ merges,
                         unsigned long long* __restrict__ counters, AppendArgs app, int fill_per_head) {
  __shared__ int wsum[3][kPlanThreads / 64];
  const int tid = __builtin_amdgcn_workitem_id_x();
  const int wg = __builtin_amdgcn_workgroup_id_x();
  if (wg > 0) {
    append_chunk((int64_t)(wg - 1) * kPlanThreads + tid, app, cu, prefix, num_seqs);
    return;
  }
  int item_tiles = item_mult * seg_tiles;
  if (fill_per_head > 0) {
    // items of about (all blocks' tiles) / fill_per_head tiles, at least 8:
    // fill_per_head units per head fill the compute units however long the
    // prefixes are
    int64_t mine = 0;
    for (int b = tid; b < num_seqs; b += kPlanThreads) {
      const int st = cu[b], en = cu[b + 1], pre = prefix[b];
      const int len = (st >= 0 && en <= num_tokens && en > st) ? en - st : 0;
      for (int q0 = 0; q0 < len; q0 += kQueryBlock) mine += (pre + min(q0 + kQueryBlock, len) + kKeyTile - 1) / kKeyTile;
    }
    const int lane = tid & 63, wave = tid >> 6;
    const int part = (int)min(mine, (int64_t)INT32_MAX / kPlanThreads);
    const int s = wave_incl_scan(part, lane);
    if (lane == 63) wsum[0][wave] = s;
    __syncthreads();
    int64_t total = 0;
    for (int w = 0; w < kPlanThreads / 64; ++w) total += wsum[0][w];
    __syncthreads();  // wsum is reused below
    item_tiles = (int)max((int64_t)8, min((total + fill_per_head - 1) / fill_per_head, (int64_t)1 << 24));
  }
  if (tid < kSplitCounters) counters[tid] = 0;  // the attention pass hands out work through these
  const int lane = tid & 63, wave = tid >> 6;
  int64_t base_i = 0, base_d = 0, base_m = 0;
  for (int b0 = 0; b0 < num_seqs; b0 += kPlanThreads) {
    const int b = b0 + tid;
    int start = 0, len = 0, pre = 0;
    SeqPlan c{0, 0, 0};
    if (b < num_seqs) {
      start = cu[b];
      const int end = cu[b + 1];
      pre = prefix[b];
      // tokens outside [0, num_tokens) would index outside the partial buffers
      len = (start >= 0 && end <= num_tokens && end > start) ? end - start : 0;
      c = count_seq(len, pre, seg_tiles, max_segs, dec_mult, item_tiles, dec_rows != 0);
    }
    const int si = wave_incl_scan(c.items, lane);
    const int sd = wave_incl_scan(c.dec, lane);
    const int sm = wave_incl_scan(c.merges, lane);
    if (lane == 63) {
      wsum[0][wave] = si;
      wsum[1][wave] = sd;
      wsum[2][wave] = sm;
    }
    __syncthreads();
    int64_t off_i = base_i + si - c.items, off_d = base_d + sd - c.dec, off_m = base_m + sm - c.merges;
    int64_t tot_i = 0, tot_d = 0, tot_m = 0;
    for (int w = 0; w < kPlanThreads / 64; ++w) {
      if (w < wave) {
        off_i += wsum[0][w];
        off_d += wsum[1][w];
        off_m += wsum[2][w];
      }
      tot_i += wsum[0][w];
      tot_d += wsum[1][w];
      tot_m += wsum[2][w];
    }
    __syncthreads();  // wsum is rewritten by the next round
    if (c.items + c.dec > 0) {
      // items segment by segment, the blocks of one segment adjacent: with
      // item i of head h run as step i * H + h of a grid that is a multiple of
      // H and of the 8 XCDs, the blocks reading one segment's K/V tiles then
      // run at the same time on one XCD and share its L2
      const bool row = dec_rows && len == 1;
      const int nqb = (len + kQueryBlock - 1) / kQueryBlock;
      const int ntiles_last = (pre + len + kKeyTile - 1) / kKeyTile;  // the last block has the most
      const int ns_max = block_segments(ntiles_last, row, seg_tiles, max_segs, dec_mult, item_tiles);
      for (int s = 0; s < ns_max; ++s)
        for (int qb = 0; qb < nqb; ++qb) {
          const int qend = min(qb * kQueryBlock + kQueryBlock, len);
          const int ntiles = (pre + qend + kKeyTile - 1) / kKeyTile;
          const int ns = block_segments(ntiles, row, seg_tiles, max_segs, dec_mult, item_tiles);
          if (s >= ns) continue;
          if (row) {
            if (off_d < max_dec) dec[off_d] = make_int4(b, s, ns, 0);
            ++off_d;
          } else {
            if (off_i < max_items) items[off_i] = make_int4(b, qb, s, ns);
            ++off_i;
          }
        }
      for (int qb = 0; qb < nqb; ++qb) {
        const int q0 = qb * kQueryBlock;
        const int qend = min(q0 + kQueryBlock, len);
        const int ntiles = (pre + qend + kKeyTile - 1) / kKeyTile;
        const int ns = block_segments(ntiles, row, seg_tiles, max_segs, dec_mult, item_tiles);
        if (ns > 1)
          for (int r = q0; r < qend; r += kMergeRows, ++off_m)
            if (off_m < max_merges) merges[off_m] = make_int4(start + r, min(kMergeRows, qend - r), ns, 0);
      }
    }
    base_i += tot_i;
    base_d += tot_d;
    base_m += tot_m;
  }
  if (tid == 0) {
    hdr[0] = (int32_t)(base_i < max_items ? base_i : max_items);
    hdr[1] = (int32_t)(base_m < max_merges ? base_m : max_merges);
    hdr[2] = (int32_t)(base_d < max_dec ? base_d : max_dec);
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t two = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(two, bf16x2_t));
}

// Persistent: work-group steps walk (merge entry, head) pairs; wave w of the
// work-group merges rows w, w + 4, ... of the entry.  Lane l owns output
// elements 2l, 2l + 1 (lanes >= D / 2 idle); lane s < nseg holds segment s's
// L_s and weight.
template <int D>
__global__ __launch_bounds__(256)
void splitkv_merge_kernel(const int32_t* __restrict__ hdr, const int4* __restrict__ merges,
                          const float* __restrict__ part_o, const float* __restrict__ part_lse,
                          uint16_t* __restrict__ out, int num_heads, int max_segs, int grid) {
  const int tid = __builtin_amdgcn_workitem_id_x();
  const int lane = lane_id(), wave = tid >> 6;
  const int64_t steps = (int64_t)hdr[1] * num_heads;
  const bool active = lane < D / 2;
  for (int64_t g = __builtin_amdgcn_workgroup_id_x(); g < steps; g += grid) {
    const int4 e = merges[g / num_heads];
    const int h = (int)(g % num_heads);
    const int nseg = e.z;
    for (int r = wave; r < e.y; r += 4) {
      const int64_t tok = e.x + r;
      const int64_t slot0 = (tok * num_heads + h) * max_segs;
      const float L = lane < nseg ? part_lse[slot0 + lane] : -__builtin_huge_valf();
      const float M = wave_max(L, lane);
      const float w = lane < nseg ? __builtin_amdgcn_exp2f(L - M) : 0.f;
      const float W = wave_sum(w, lane);
      f32x2_t acc = {0.f, 0.f};
      const float* src = part_o + slot0 * D + 2 * lane;
      for (int s = 0; s < nseg; ++s) {
        const float ws = lane_value(w, s);
        if (active) {
          const f32x2_t o = *(const f32x2_t*)(src + (int64_t)s * D);
          acc += ws * o;
        }
      }
      if (active) {
        const float inv = 1.f / W;
        *(uint32_t*)(out + (tok * num_heads + h) * D + 2 * lane) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
      }
    }
  }
}

// Length-1 rows in a launch of their own (the split-KV call's choice when
// the rows' work is not folded into the attention launch): four-wave
// work-groups, several per compute unit, walk the decode units in a fixed
// stride.
constexpr int kDecThreads = 256;

template <int D, int GC, bool kPaged>
__global__ __launch_bounds__(kDecThreads)
void splitkv_decode_kernel(FwdParams p) {
  __shared__ float red[dec::red_floats<D, GC, kDecThreads / 64>()];
  const int64_t steps = (int64_t)p.hdr[2] * (p.num_heads / GC);
  for (int64_t g = __builtin_amdgcn_workgroup_id_x(); g < steps; g += p.dec_grid)
    dec::decode_unit<D, GC, kPaged, kDecThreads / 64>(p, g, red, nullptr, nullptr);
}

}  // namespace

SplitLayout split_layout(int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                         int32_t head_dim, int32_t cap) {
  SplitLayout L{};
  const int64_t cap_tiles = ((int64_t)cap + kKeyTile - 1) / kKeyTile;
  int64_t seg = (cap_tiles + kMaxSegs - 1) / kMaxSegs;
  if (seg < kMinSegTiles) seg = kMinSegTiles;
  L.seg_tiles = (int32_t)seg;
  L.max_segs = (int32_t)((cap_tiles + seg - 1) / seg);
  if (L.max_segs < 1) L.max_segs = 1;
  L.max_blocks = (int64_t)num_tokens / kQueryBlock + num_seqs + 1;
  L.max_items = L.max_blocks * L.max_segs;
  L.max_dec_items = ((int64_t)num_seqs + 1) * L.max_segs;
  const int64_t max_merges = (int64_t)num_tokens / kMergeRows + num_seqs + 1;
  const size_t slots = (size_t)num_tokens * num_heads * L.max_segs;
  L.off_hdr = 0;
  L.off_ctr = 256;
  L.off_items = 512;
  L.off_dec = L.off_items + round256(16 * (size_t)L.max_items);
  L.off_merges = L.off_dec + round256(16 * (size_t)L.max_dec_items);
  L.off_lse = L.off_merges + round256(16 * (size_t)max_merges);
  L.off_o = L.off_lse + round256(4 * slots);
  L.bytes = L.off_o + round256(4 * slots * head_dim);
  return L;
}

hipError_t launch_splitkv_plan(const int32_t* cu, const int32_t* prefix, int32_t num_seqs,
                               int32_t num_tokens, const SplitLayout& L, int dec_seg_mult,
                               int item_seg_mult, void* ws, hipStream_t stream, bool rows_as_items,
                               const FwdParams* append, int head_dim, int fill_per_head) {
  char* base = static_cast<char*>(ws);
  const int64_t max_merges = (int64_t)(L.off_lse - L.off_merges) / 16;
  AppendArgs app{};
  int64_t blocks = 1;
  if (append) {
    app = AppendArgs{append->k, append->v, append->kc, append->vc, append->num_kv_heads, append->cap,
                     head_dim, (int64_t)num_tokens * append->num_kv_heads};
    blocks += (2 * app.rows * (app.head_dim / 8) + kPlanThreads - 1) / kPlanThreads;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  }
  hipLaunchKernelGGL(splitkv_plan_kernel, dim3((unsigned)blocks), dim3(kPlanThreads), 0, stream, cu, prefix,
                     num_seqs, num_tokens, L.seg_tiles, L.max_segs, dec_seg_mult, item_seg_mult,
                     rows_as_items ? 0 : 1, L.max_items, L.max_dec_items,
                     max_merges, reinterpret_cast<int32_t*>(base + L.off_hdr),
                     reinterpret_cast<int4*>(base + L.off_items),
                     reinterpret_cast<int4*>(base + L.off_dec),
                     reinterpret_cast<int4*>(base + L.off_merges),
                     reinterpret_cast<unsigned long long*>(base + L.off_ctr), app, fill_per_head);
  return hipGetLastError();
}

hipError_t launch_splitkv_merge(const FwdParams& p, const SplitLayout& L, const void* ws,
                                int head_dim, int grid, hipStream_t stream) {
  const char* base = static_cast<const char*>(ws);
  const int4* merges = reinterpret_cast<const int4*>(base + L.off_merges);
  switch (head_dim) {
    case 32: hipLaunchKernelGGL(splitkv_merge_kernel<32>, dim3(grid), dim3(256), 0, stream, p.hdr, merges, p.part_o, p.part_lse, p.out, p.num_heads, L.max_segs, grid); break;
    case 64: hipLaunchKernelGGL(splitkv_merge_kernel<64>, dim3(grid), dim3(256), 0, stream, p.hdr, merges, p.part_o, p.part_lse, p.out, p.num_heads, L.max_segs, grid); break;
    case 128: hipLaunchKernelGGL(splitkv_merge_kernel<128>, dim3(grid), dim3(256), 0, stream, p.hdr, merges, p.part_o, p.part_lse, p.out, p.num_heads, L.max_segs, grid); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa

namespace pa {

namespace {
template <int D, bool kPaged>
hipError_t decode_d(const FwdParams& p, hipStream_t stream) {
  const dim3 grid(p.dec_grid), block(kDecThreads);
  switch (p.dec_heads) {
    case 1: hipLaunchKernelGGL((splitkv_decode_kernel<D, 1, kPaged>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((splitkv_decode_kernel<D, 2, kPaged>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((splitkv_decode_kernel<D, 4, kPaged>), grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL((splitkv_decode_kernel<D, 8, kPaged>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
template <int D, bool kPaged>
int decode_occ(int gc) {
  int n = 0;
  hipError_t e = hipErrorInvalidValue;
  switch (gc) {
    case 1: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, splitkv_decode_kernel<D, 1, kPaged>, kDecThreads, 0); break;
    case 2: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, splitkv_decode_kernel<D, 2, kPaged>, kDecThreads, 0); break;
    case 4: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, splitkv_decode_kernel<D, 4, kPaged>, kDecThreads, 0); break;
    case 8: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, splitkv_decode_kernel<D, 8, kPaged>, kDecThreads, 0); break;
    default: break;
  }
  return e == hipSuccess ? n : 0;
}
}  // namespace

hipError_t launch_splitkv_decode(const FwdParams& p, int head_dim, bool paged, hipStream_t stream) {
  switch (head_dim) {
    case 32: return paged ? decode_d<32, true>(p, stream) : decode_d<32, false>(p, stream);
    case 64: return paged ? decode_d<64, true>(p, stream) : decode_d<64, false>(p, stream);
    case 128: return paged ? decode_d<128, true>(p, stream) : decode_d<128, false>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

int splitkv_decode_blocks_per_cu(int head_dim, int heads_per_unit, bool paged) {
  switch (head_dim) {
    case 32: return paged ? decode_occ<32, true>(heads_per_unit) : decode_occ<32, false>(heads_per_unit);
    case 64: return paged ? decode_occ<64, true>(heads_per_unit) : decode_occ<64, false>(heads_per_unit);
    case 128: return paged ? decode_occ<128, true>(heads_per_unit) : decode_occ<128, false>(heads_per_unit);
    default: return 0;
  }
}

int splitkv_heads_per_unit(int num_heads, int num_kv_heads) {
  const int g = num_heads / num_kv_heads;
  return g % 8 == 0 ? 8 : g % 4 == 0 ? 4 : g % 2 == 0 ? 2 : 1;
}

}  // namespace pa
