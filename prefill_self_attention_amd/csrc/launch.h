// launch.h -- internal interface between the C-ABI layer (api.hip) and the
// gfx950 kernels (prefill_fwd.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

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
};

// Query rows per block, and work-groups per (head, sequence) for a maximum length.
int fwd_block_rows();
int fwd_grid_blocks(int max_seqlen);

// Enqueue the fused attention + cache-write kernel; returns hipGetLastError().
hipError_t launch_prefill_fwd(const FwdParams& p, int num_seqs, int head_dim, bool chunked,
                              hipStream_t stream);

}  // namespace pa
