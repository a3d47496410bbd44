// splitkv.hip -- split-KV chunked prefill: the plan that cuts every query
// block's keys into segments, and the log-sum-exp merge of the segments'
// partial results.  The attention over each segment runs in
// prefill_fwd_split_kernel (prefill_fwd.hip).
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

#include "launch.h"

namespace pa {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kMinSegTiles = 16;  // 1024 keys per segment at least
constexpr int kMaxSegs = 64;      // segments per block at most (bounds the workspace)
constexpr int kMergeRows = 16;    // rows per merge entry (4 waves x 4 rows)
constexpr int kPlanThreads = 1024;

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
  int items, merges;
};

// Segments of every query block of one sequence (work items), and the merge
// entries of the blocks with more than one segment.  Segment counts are
// capped at max_segs, so malformed metadata cannot address outside the
// workspace.
__device__ SeqPlan count_seq(int len, int pre, int seg_tiles, int max_segs) {
  SeqPlan r{0, 0};
  for (int q0 = 0; q0 < len; q0 += kQueryBlock) {
    const int qend = min(q0 + kQueryBlock, len);
    const int ntiles = (pre + qend + kKeyTile - 1) / kKeyTile;
    const int ns = min((ntiles + seg_tiles - 1) / seg_tiles, max_segs);
    if (ns < 1) continue;
    r.items += ns;
    if (ns > 1) r.merges += (qend - q0 + kMergeRows - 1) / kMergeRows;
  }
  return r;
}

// One work-group.  Sequences are taken 1024 at a time; each thread counts its
// sequence's items and merge entries, a work-group scan gives the offsets, and
// the thread writes them.  hdr[0], hdr[1] receive the totals.
__global__ __launch_bounds__(kPlanThreads)
void splitkv_plan_kernel(const int32_t* __restrict__ cu, const int32_t* __restrict__ prefix,
                         int num_seqs, int num_tokens, int seg_tiles, int max_segs,
                         int64_t max_items, int64_t max_merges, int32_t* __restrict__ hdr,
                         int4* __restrict__ items, int4* __restrict__ merges) {
  __shared__ int wsum[2][kPlanThreads / 64];
  const int tid = __builtin_amdgcn_workitem_id_x();
  const int lane = tid & 63, wave = tid >> 6;
  int64_t base_i = 0, base_m = 0;
  for (int b0 = 0; b0 < num_seqs; b0 += kPlanThreads) {
    const int b = b0 + tid;
    int start = 0, len = 0, pre = 0;
    SeqPlan c{0, 0};
    if (b < num_seqs) {
      start = cu[b];
      const int end = cu[b + 1];
      pre = prefix[b];
      // tokens outside [0, num_tokens) would index outside the partial buffers
      len = (start >= 0 && end <= num_tokens && end > start) ? end - start : 0;
      c = count_seq(len, pre, seg_tiles, max_segs);
    }
    const int si = wave_incl_scan(c.items, lane);
    const int sm = wave_incl_scan(c.merges, lane);
    if (lane == 63) {
      wsum[0][wave] = si;
      wsum[1][wave] = sm;
    }
    __syncthreads();
    int64_t off_i = base_i + si - c.items, off_m = base_m + sm - c.merges;
    int64_t tot_i = 0, tot_m = 0;
    for (int w = 0; w < kPlanThreads / 64; ++w) {
      if (w < wave) {
        off_i += wsum[0][w];
        off_m += wsum[1][w];
      }
      tot_i += wsum[0][w];
      tot_m += wsum[1][w];
    }
    __syncthreads();  // wsum is rewritten by the next round
    if (c.items > 0) {
      for (int qb = 0; qb * kQueryBlock < len; ++qb) {
        const int q0 = qb * kQueryBlock;
        const int qend = min(q0 + kQueryBlock, len);
        const int ntiles = (pre + qend + kKeyTile - 1) / kKeyTile;
        const int ns = min((ntiles + seg_tiles - 1) / seg_tiles, max_segs);
        for (int s = 0; s < ns; ++s, ++off_i)
          if (off_i < max_items) items[off_i] = make_int4(b, qb, s, ns);
        if (ns > 1)
          for (int r = q0; r < qend; r += kMergeRows, ++off_m)
            if (off_m < max_merges) merges[off_m] = make_int4(start + r, min(kMergeRows, qend - r), ns, 0);
      }
    }
    base_i += tot_i;
    base_m += tot_m;
  }
  if (tid == 0) {
    hdr[0] = (int32_t)(base_i < max_items ? base_i : max_items);
    hdr[1] = (int32_t)(base_m < max_merges ? base_m : max_merges);
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
  const int64_t max_merges = (int64_t)num_tokens / kMergeRows + num_seqs + 1;
  const size_t slots = (size_t)num_tokens * num_heads * L.max_segs;
  L.off_hdr = 0;
  L.off_items = 256;
  L.off_merges = L.off_items + round256(16 * (size_t)L.max_items);
  L.off_lse = L.off_merges + round256(16 * (size_t)max_merges);
  L.off_o = L.off_lse + round256(4 * slots);
  L.bytes = L.off_o + round256(4 * slots * head_dim);
  return L;
}

hipError_t launch_splitkv_plan(const int32_t* cu, const int32_t* prefix, int32_t num_seqs,
                               int32_t num_tokens, const SplitLayout& L, void* ws,
                               hipStream_t stream) {
  char* base = static_cast<char*>(ws);
  const int64_t max_merges = (int64_t)(L.off_lse - L.off_merges) / 16;
  hipLaunchKernelGGL(splitkv_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, cu, prefix,
                     num_seqs, num_tokens, L.seg_tiles, L.max_segs, L.max_items, max_merges,
                     reinterpret_cast<int32_t*>(base + L.off_hdr),
                     reinterpret_cast<int4*>(base + L.off_items),
                     reinterpret_cast<int4*>(base + L.off_merges));
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
