// launch.h -- internal interface between the C-ABI layer (api.hip) and the
// gfx950 kernels (prefill_fwd.hip, splitkv.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kQueryBlock = 128;  // query rows per block
constexpr int kKeyTile = 64;      // keys per tile

struct FwdParams {
  const uint16_t* q;        // [N, H, D] bf16
  const uint16_t* k;        // [N, num_kv_heads, D]
  const uint16_t* v;
  const int32_t* cu;        // [B + 1]
  const int32_t* prefix;    // [B] (chunked) or nullptr (varlen)
  uint16_t* kc;             // varlen: packed [HK, len_b, D] blocks; chunked: [B, HK, cap, D]
  uint16_t* vc;
  uint16_t* out;            // [N, H, D] bf16
  int32_t num_heads;        // query heads
  int32_t num_kv_heads;     // K/V heads (divides num_heads)
  int32_t cap;              // chunked cache capacity (0 for varlen)
  int32_t grid_z;           // work-groups per (head, sequence): pairs of query blocks
  float scale_log2;         // |scale| * log2(e)
  int32_t neg_q;            // 1 if scale < 0: q's sign is flipped in the kernel
  // split-KV chunked mode only (see SplitLayout)
  const int32_t* hdr;       // [0] = number of work items, [1] = number of merged blocks
  const int4* items;        // work items: {sequence, query block, segment, segments of the block}
  float* part_o;            // [N, H, max_segs, D] fp32 partial outputs (normalised)
  float* part_lse;          // [N, H, max_segs] fp32 log2-sum-exp2 of each partial
  int32_t seg_tiles;        // key tiles per segment
  int32_t max_segs;         // segments per block, at most
  int32_t split_grid;       // work-groups of the persistent split-KV launch
  const int4* dec_items;    // decode-row items: {sequence, segment, segments, 0}; hdr[2] of them
  int32_t dec_heads;        // query heads per decode unit (1, 2, 4 or 8)
  int32_t fuse_decode;      // 1: the split attention launch also runs the decode units
  int32_t items_first;      // fused: work-groups [0, items_first) start on the items, the rest on decode units
  unsigned long long* counters;  // kSplitCounters work counters, zeroed by the plan
  int32_t dec_grid;         // work-groups of the separate decode launch (fuse_decode == 0)
  // INT8 cache (varlen only): codes in kq/vq laid out as kc/vc, one float
  // scale per (token, K/V head) row in ks/vs (the cache layout without D)
  int8_t* kq;
  int8_t* vq;
  float* ks;
  float* vs;
  // paged cache (split-KV chunked only): kc/vc are [num_blocks, HK, 16, D];
  // cache position j of sequence b is row j % 16 of block
  // block_table[b * bt_stride + j / 16]
  const int32_t* block_table;
  int32_t bt_stride;
  int32_t num_seqs;         // B (set by the launch of the 64-row kernel)
};

constexpr int kPageRows = 16;  // tokens per cache block
constexpr int kSplitCounters = 9;  // item queues of the 8 XCDs, then the decode units

// Query rows per block, and work-groups per (head, sequence) for a maximum length.
int fwd_block_rows();
int fwd_grid_blocks(int max_seqlen);

// Enqueue the fused attention + cache-write kernel; returns hipGetLastError().
hipError_t launch_prefill_fwd(const FwdParams& p, int num_seqs, int head_dim, bool chunked,
                              hipStream_t stream);
// Varlen, head_dim 128, scale >= 0: the 64-row-per-wave kernel (fwd64.hip),
// same contract as launch_prefill_fwd (cache_format 0) and as
// launch_prefill_fwd_int8 / _fp8 (1, 2: p.kq, p.vq, p.ks, p.vs).
bool fwd64_supported(int head_dim, bool chunked, float scale, int max_seqlen, int num_heads, int num_kv_heads);
hipError_t launch_prefill_fwd64(const FwdParams& p, int num_seqs, int cache_format, hipStream_t stream);
// Split-KV items of a chunked call on the 64-row kernel: keys (prefix and
// new) from the cache slab, which the plan launch has filled with the call's
// new rows first (launch_splitkv_plan with append); partial results to part_o / part_lse when an item's
// block has several segments, else the output.  max_items bounds the plan's
// item count (p.hdr[0]).
bool fwd64_split_supported(int head_dim, float scale, int max_seqlen, int num_heads, int cap);
hipError_t launch_prefill_fwd64_split(const FwdParams& p, int64_t max_items, hipStream_t stream);
// Varlen with an INT8 or an FP8 (E4M3) cache (kq, vq, ks, vs instead of kc, vc).
hipError_t launch_prefill_fwd_fp8(const FwdParams& p, int num_seqs, int head_dim, hipStream_t stream);
hipError_t launch_prefill_fwd_int8(const FwdParams& p, int num_seqs, int head_dim,
                                   hipStream_t stream);

// ------------------------------------------------------------ split-KV layout
// Workspace of the split-KV chunked call, carved from one caller buffer.
// Every region starts on a 256-byte boundary.
struct SplitLayout {
  int32_t seg_tiles;     // key tiles per segment
  int32_t max_segs;      // ceil(ceil(cap / 64) / seg_tiles)
  int64_t max_blocks;    // bound on the query blocks of the batch: N / 128 + B + 1
  int64_t max_items;     // max_blocks * max_segs
  int64_t max_dec_items; // num_seqs * max_segs
  size_t off_hdr, off_ctr, off_items, off_dec, off_merges, off_lse, off_o, bytes;
};
SplitLayout split_layout(int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                         int32_t head_dim, int32_t cap);

// Plan (one work-group): item list, decode list, merge list and their counts
// in the workspace, work counters zeroed.  Then the persistent pass over the
// items and the decode rows' units (both in one launch), then the merge of
// blocks with more than one segment.
// A decode row's segments hold about dec_seg_mult * seg_tiles tiles, a
// multi-row block's about item_seg_mult * seg_tiles (both longer when the
// rows run inside the attention launch).
hipError_t launch_splitkv_plan(const int32_t* cu, const int32_t* prefix, int32_t num_seqs,
                               int32_t num_tokens, const SplitLayout& L, int dec_seg_mult,
                               int item_seg_mult, void* ws, hipStream_t stream,
                               bool rows_as_items = false, const FwdParams* append = nullptr,
                               int head_dim = 0, int fill_per_head = 0);
hipError_t launch_prefill_fwd_split(const FwdParams& p, int head_dim, bool paged, hipStream_t stream);
hipError_t launch_splitkv_merge(const FwdParams& p, const SplitLayout& L, const void* ws,
                                int head_dim, int grid, hipStream_t stream);
// Query heads per decode unit of the length-1 rows: 1, 2, 4 or 8, dividing
// num_heads / num_kv_heads; they share each load of a K/V row.
int splitkv_heads_per_unit(int num_heads, int num_kv_heads);
// The length-1 rows in a launch of their own (when fuse_decode is 0), and
// its resident work-groups per compute unit.
hipError_t launch_splitkv_decode(const FwdParams& p, int head_dim, bool paged, hipStream_t stream);
int splitkv_decode_blocks_per_cu(int head_dim, int heads_per_unit, bool paged);
// Resident work-groups per compute unit of the split attention kernel, with
// (fused) or without the decode rows (0 on error; the paged variants alike).
int fwd_split_blocks_per_cu(int head_dim, bool fused);

}  // namespace pa
