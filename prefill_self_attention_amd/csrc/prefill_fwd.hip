// prefill_fwd.hip -- causal varlen / chunked prefill attention with a fused
// KV-cache write, for gfx950 (MI355X, CDNA4).
//
// What one launch computes (see include/prefill_attn.h for the contract):
// for every sequence b, head h and new token i at absolute position p_b + i,
//     out = sum_{j <= p_b + i} softmax_j(scale * q . k_j) v_j
// ["Prefill不是热身：大模型推理的真正瓶颈与优化核心" §3 and
//  "大语言模型推理核心：Prefill与Decode原理及工程优化" §2.2: attention is
//  softmax(Q K^T / sqrt(d_k)) V; untitled page www.zwxr.cn/news/300951 §1.1:
//  a position sees itself and the positions before it], restricted to the
// keys of its own request ["大模型 Prompt Prefill 阶段的高效 Batching 与算子排布"
// §2: the varlen kernel reads cu_seqlens and never mixes requests], and the
// K/V of every new token are copied into the head-major cache
// ["大模型推理优化：Prefill、Decode与KV Cache的工程实践" §1.3].  With grouped
// K/V heads (untitled page www.zwxr.cn/news/300951 §2.4: fewer K/V heads
// than query heads shrink the cache) query head h reads K/V head
// h / (num_heads / num_kv_heads).
//
// How it is computed (blockwise, never materialising the T x T scores, and
// skipping tiles above the diagonal: www.zwxr.cn/news/300951 §3.3):
//
//  * Query blocks of 128 rows, key tiles of 64 absolute key positions.  A
//    block whose last key is e needs ceil(e / 64) tiles, so block i of a causal
//    sequence costs about i+1 units.  One work-group takes the pair of blocks
//    (z, n-1-z) of one (sequence, head): the costs of a pair sum to the same
//    total for every z, so all work-groups of a sequence carry equal work.
//  * The work-group is 8 wave64s, two per SIMD, in two groups of four; a wave
//    owns 32 query rows of the block it is on.  The pair's tile list (light
//    block, then heavy block) is split in half: the upper group walks the heavy
//    block's tiles from 0, the lower group does the light block and then the
//    heavy block's remaining (highest) tiles.  The heavy block's rows so hold
//    two partial online-softmax states, merged through LDS at the end; every
//    wave does the same number of tiles (17 at T = 2048), and each SIMD runs
//    two waves, so one wave's softmax VALU work overlaps the other's MFMAs (a
//    single wave issues VALU at about half the SIMD's rate on this part).
//  * Tiles reach LDS by direct global-to-LDS loads (global_load_lds_dwordx4:
//    lane l of an instruction fills bytes [16 l, 16 l + 16) of a 1 KB block),
//    double-buffered per group, one barrier per iteration; no staging VGPRs.
//    Rows are stored unpadded with the 16-byte chunk index XORed with
//    f(row) = 2*(row%4) + (row/4)%2: the 8-row reads of the score operand and
//    the 4-row, 32-byte transpose reads of the PV operand then hit distinct
//    banks.
//  * Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16
//    (A = K from LDS, B = Q^T held in VGPRs).  In the 32x32 accumulator lane l
//    holds query column l%32 and key rows 8*(r/4) + 4*(l/32) + r%4, so a
//    query's scores live in lanes l and l^32: one v_permlane32_swap per tile
//    for the max, none for the running sum until the end, and the O rescale is
//    a per-lane multiply.
//  * Online softmax in the exp2 domain with c = |scale| log2(e) > 0 (a
//    negative scale flips q's sign instead; the host keeps c >= 2^-100): max
//    over raw scores, p = 2^(s c - m) as one FMA and one v_exp_f32, which is 0
//    for a masked score of -inf.  The running max m only moves
//    when a tile's max exceeds it by more than 8 (lazy rescale; p stays below
//    2^8; exact in real arithmetic because O and l share one m).
//  * O^T = V^T P^T on 32x32x16 MFMA: B = P^T converted to bf16 straight from
//    the score accumulator; A = V^T read from row-major V with
//    ds_read_b64_tr_b16, which hands each lane 4 keys of its own d in the
//    accumulator's key order.
//  * Causal masking only on tiles that cross a wave's diagonal or the end of
//    the keys; a wave skips tiles wholly above its rows.
//  * KV-cache write: when a group's tile holds new tokens of the block it
//    serves, the group copies exactly those rows from LDS to the cache with
//    16-byte stores; every new token is written once.  Prefix keys of chunked
//    prefill are read from the cache, new keys always from k/v, so no
//    work-group reads a cache position this launch writes.
//  * Grid (head, sequence, pair): with H a multiple of 8 all pairs of one head
//    land on one XCD (work-groups are dealt round-robin over the 8 XCDs),
//    keeping that head's K/V in one L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "decode_rows.h"
#include "launch.h"
#include "quant_rows.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kQueryBlock;    // query rows per block (4 waves x 32)
constexpr int kGroupThreads = 256;  // one group = 4 waves
constexpr int kBN = kKeyTile;       // keys per tile
constexpr float kRescale = 8.0f;    // lazy-rescale headroom, log2 units
constexpr float kNegInf = -__builtin_huge_valf();
// Initial running max: finite, so a first tile in which every key of a row is
// masked (a group can start mid-sequence) keeps alpha = 2^0 = 1 instead of
// 2^(-inf - -inf); any real score replaces it (alpha = 0 then).
constexpr float kMInit = -1.0e30f;

__device__ __forceinline__ float row_max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row_sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// LDS reads issued as inline asm.  The main loop's tiles arrive by direct
// global-to-LDS loads; for a compiler-generated LDS read the compiler cannot
// always tell that it reads a buffer other than the ones those loads are
// filling, and then waits for all of them first.  An asm read's result is
// pending until an lds_wait* call names its registers: LDS operations
// complete in order, so "at most N outstanding" covers every read issued
// before the last N.
template <int kOff>
__device__ __forceinline__ u32x4_t lds_read_b128(uint32_t addr) {
  u32x4_t r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(kOff));
  return r;
}
template <int kOff>
__device__ __forceinline__ s16x4_t lds_read_tr(uint32_t addr) {
  s16x4_t r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(kOff));
  return r;
}
template <int N>
__device__ __forceinline__ void lds_wait(u32x4_t& a, u32x4_t& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}
template <int N, int NV>
__device__ __forceinline__ void lds_wait_tr(s16x4_t (&r)[NV]) {
  if constexpr (NV == 2) {
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(r[0]), "+v"(r[1]) : "n"(N));
  } else if constexpr (NV == 4) {
    asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]) : "n"(N));
  } else {
    static_assert(NV == 8, "2, 4 or 8 registers");
    asm volatile("s_waitcnt lgkmcnt(%8)"
                 : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7])
                 : "n"(N));
  }
}
template <int K>
__device__ __forceinline__ void lds_wait_all(u32x4_t (&a)[K], u32x4_t (&b)[K]) {
  if constexpr (K == 1) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(b[0]));
  } else if constexpr (K == 2) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(b[0]), "+v"(b[1]));
  } else {
    static_assert(K == 4, "1, 2 or 4 chunks per lane");
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]));
  }
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t*)p));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t two = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(two, bf16x2_t));
}

// INT8 / FP8 rows: quant_rows.h
using namespace qrow;

template <int D>
struct Cfg {
  static constexpr int kCpr = D / 8;                    // 16-byte chunks per row
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kTileBytes = kBN * kRowBytes;    // one K or V tile
  static constexpr int kRowsPerInst = 1024 / kRowBytes; // rows per 1 KB direct load
  static constexpr int kInstPerTile = kBN / kRowsPerInst;
  static constexpr int kInstPerWave = kInstPerTile / 4; // per tile and matrix, per wave of a group
  // LDS map, in tiles: lower group K0 V0 K1 V1 (double buffer); upper group
  // K ring of 2 and V ring of 3 (its PV step runs one interval behind).
  static constexpr int kLowerOff = 0;
  static constexpr int kUpperK = 4 * kTileBytes;
  static constexpr int kUpperV = 6 * kTileBytes;
  static constexpr int kLdsBytes = 9 * kTileBytes;
  static constexpr int kKReadBases = D / 16 < 4 ? D / 16 : 4;  // lane bases of the score operand
  static constexpr int kVReadsPerStep = 2 * (D / 32);          // transpose reads per 16-key step
  // merge buffer per upper wave (per lane: m, l and D/2 accumulators)
  static constexpr int kMergeWaveFloats = (2 + D / 2) * 64;
  static_assert(4 * kMergeWaveFloats * 4 <= kLdsBytes, "merge buffers must fit the tile area");
};

// 16-byte chunk slot of chunk c in row r (XOR swizzle, stays inside the row;
// depends on r % 8 only)
template <int D>
__device__ __forceinline__ int chunk_slot(int r, int c) {
  return c ^ ((((r & 3) << 1) | ((r >> 2) & 1)) & (Cfg<D>::kCpr - 1));
}

struct Block {
  int q0;       // first local row
  int qend;     // one past the last local row (<= len)
  int key_end;  // keys needed: absolute positions [0, key_end)
  int own_lo;   // absolute positions [own_lo, key_end) are this block's new tokens
  int ntiles;
};

__device__ __forceinline__ Block make_block(int qb, int len, int pre) {
  Block k;
  k.q0 = qb * kBM;
  k.qend = min(k.q0 + kBM, len);
  k.key_end = pre + k.qend;
  k.own_lo = pre + k.q0;
  k.ntiles = (k.key_end + kBN - 1) / kBN;
  return k;
}

// Tile of a group at position `it` of its list: tile index t of block qb (the
// heavy block qb_hi or the light block z), and whether there is one.  A free
// function of plain values, branch-free, with the block index formed by
// arithmetic: selects between captured variables get folded into selects of
// their addresses, which pins them (and whole closures) in scratch memory.
struct Pick {
  int t, qb;
  bool on_hi, valid;
};

__device__ __forceinline__ Pick pick_tile(int it, bool upper, int n_up, int e_lo, int e_hi,
                                          int z, int qb_hi) {
  Pick r;
  const bool hi = upper || it >= e_lo;
  r.on_hi = hi;
  r.t = upper ? it : (hi ? n_up + (it - e_lo) : it);
  r.valid = upper ? (it < n_up) : (!hi || r.t < e_hi);
  r.qb = z + (hi ? qb_hi - z : 0);
  return r;
}

// State of a wave's 32 query rows.
template <int D>
struct Rows {
  bf16x8_t q[D / 16];
  f32x16_t o[D / 32];
  float m, l;
};

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// The work-group's LDS: K/V tile buffers, then the merge buffers; the
// split-KV kernel's decode units reuse it for their reductions.  One array
// per fwd_item instantiation (kTag tells apart two kernels that run the same
// item), so each is used by one kernel only and keeps a fixed LDS address.
template <int D, bool kChunked, bool kSplit, int kCache, bool kPaged, int kTag>
__device__ __forceinline__ auto fwd_lds() -> uint8_t (&)[Cfg<D>::kLdsBytes] {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[Cfg<D>::kLdsBytes];
  return lds;
}

// One work item of a work-group: head h of sequence b, and either the pair of
// query blocks (z, n-1-z) over all their keys or, in split mode (kSplit), the
// single block z over key tiles [seg * seg_tiles, (seg + 1) * seg_tiles) --
// one of the nseg segments of its keys.  A block with one segment is stored
// as usual; otherwise its rows get a partial result (normalised O in fp32 and
// log2 of its sum of weights), merged by a later pass.
template <int D, bool kChunked, bool kSplit, int kCache = kCacheBf16, bool kPaged = false, int kTag = 0>
__device__ __forceinline__ void fwd_item(const FwdParams& p, int h, int b, int z, int seg, int nseg) {
  using C = Cfg<D>;
  // Every LDS read in the main loop is inline asm (lds_read_* above), so the
  // compiler places no wait for the direct loads in flight; each read is made
  // valid by an explicit lgkmcnt wait tied to its registers.
  uint8_t (&lds)[C::kLdsBytes] = fwd_lds<D, kChunked, kSplit, kCache, kPaged, kTag>();
  const int64_t H = p.num_heads;

  const int seq_start = p.cu[b];
  const int len = p.cu[b + 1] - seq_start;
  const int nqb = (len + kBM - 1) / kBM;
  const int qb_hi = kSplit ? z : nqb - 1 - z;
  if (z > qb_hi) return;                 // no block pair left for this work-group
  const int pre = kChunked ? p.prefix[b] : 0;
  const bool has_lo = !kSplit && z < qb_hi;
  const Block blo = make_block(z, len, pre);
  const Block bhi = make_block(qb_hi, len, pre);
  // split mode: segment seg of nseg covers tiles [seg * n / nseg, (seg + 1) * n / nseg)
  const int tb = kSplit ? seg * bhi.ntiles / nseg : 0;  // first key tile of the item
  const int e_lo = has_lo ? blo.ntiles : 0;
  const int e_hi = kSplit ? (seg + 1) * bhi.ntiles / nseg - tb : bhi.ntiles;
  const int n_up = (e_lo + e_hi + 1) / 2;  // tiles of the upper group
  const int n_lo = e_lo + e_hi - n_up;     // tiles of the lower group (<= n_up)

  const int tid = __builtin_amdgcn_workitem_id_x();
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int ql = lane & 31;
  const int hh = lane >> 5;
  const bool upper = wave >= 4;
  const int gw = wave & 3;               // wave within its group

  // grouped K/V heads: query head h reads K/V head hk; the first query head
  // of each group writes that K/V head's cache rows
  const int64_t HK = p.num_kv_heads;
  const int group = p.num_heads / p.num_kv_heads;
  const int hk = h / group;
  const bool writes_cache = h == hk * group;
  const int64_t row_stride = HK * D;     // K/V elements between consecutive tokens
  const uint16_t* __restrict__ kin = p.k + (int64_t)hk * D;
  const uint16_t* __restrict__ vin = p.v + (int64_t)hk * D;
  const int64_t cache_base = kChunked ? ((int64_t)b * HK + hk) * p.cap * D
                                      : (int64_t)seq_start * HK * D + (int64_t)hk * len * D;
  const float c = p.scale_log2;          // |scale| * log2(e), > 0
  const uint32_t lds0 = lds_addr(lds);
  // Paged cache ["大模型推理优化：Prefill、Decode与KV Cache的工程实践" §4.2:
  // 16-token blocks located through a block table]: position kp of this
  // (sequence, K/V head) is row kp % 16 of block bt_row[kp / 16], blocks
  // [num_blocks, HK, 16, D].
  const int32_t* __restrict__ bt_row = kPaged ? p.block_table + (int64_t)b * p.bt_stride : nullptr;
  auto cache_elem = [&](int kp) __attribute__((always_inline)) -> int64_t {
    if constexpr (kPaged)
      return (((int64_t)bt_row[kp / kPageRows] * HK + hk) * kPageRows + kp % kPageRows) * D;
    else
      return cache_base + (int64_t)kp * D;
  };

  // ---------------------------------------------------------------- staging
  // Wave gw of a group issues instructions j = 4 i + gw (i < kInstPerWave) per
  // tile and matrix; lane l fills row j * kRowsPerInst + l / kCpr, chunk slot
  // l % kCpr, from source chunk chunk_slot(row, slot) (the XOR is an
  // involution).  Rows past the block's last key read the last key instead,
  // so every LDS row holds finite data (masked keys get weight 0).
  const int lrow = lane / C::kCpr;
  const int lslot = lane % C::kCpr;

  auto row_ptr = [&](const uint16_t* __restrict__ in, const uint16_t* cache, int kp) __attribute__((always_inline)) {
    if (kChunked && kp < pre) return cache + cache_elem(kp);
    return in + (int64_t)(seq_start + kp - pre) * row_stride;
  };

  // Instruction i (< kInstPerWave) of this wave's share of the loads of tile
  // t of blk (K and V): one 1 KB global-to-LDS load per matrix.  The tile's
  // position and its case are made wave-uniform (readfirstlane), so the case
  // is a scalar branch; unless the tile mixes cached and new rows, a load is a
  // scalar base (the tile's first row) plus a 32-bit per-lane byte offset.
  // Instruction i's rows are 4 i kRowsPerInst past instruction 0's, a
  // multiple of 8 rows, so they share its swizzle slots.
  const int lrow0 = gw * C::kRowsPerInst + lrow;  // row of instruction 0
  const uint32_t lane_new = 2u * (uint32_t)(lrow0 * row_stride + 8 * chunk_slot<D>(lrow0, lslot));
  const uint32_t lane_cached = 2u * (uint32_t)(lrow0 * D + 8 * chunk_slot<D>(lrow0, lslot));
  auto issue_part = [&](const Block blk, int t, int k_off, int v_off, int i) __attribute__((always_inline)) {
    const int t0 = __builtin_amdgcn_readfirstlane(t * kBN);
    const int key_end = __builtin_amdgcn_readfirstlane(blk.key_end);
    uint8_t* const k_dst = lds + k_off;
    uint8_t* const v_dst = lds + v_off;
    const bool full = t0 + kBN <= key_end;
    const bool all_new = !kChunked || t0 >= pre;
    const bool all_cached = kChunked && t0 + kBN <= pre;
    const int j = 4 * i + gw;
    const int row = j * C::kRowsPerInst + lrow;
    if (kPaged && all_cached) {
      // (all_cached implies full) the rows of one load instruction (4, 8 or
      // 16) lie in one block
      const int r0 = t0 + j * C::kRowsPerInst;
      const int bi = __builtin_amdgcn_readfirstlane(r0 / kPageRows);
      const int64_t base = (((int64_t)bt_row[bi] * HK + hk) * kPageRows + r0 % kPageRows) * D;
      const uint32_t off = (uint32_t)(lrow * D + 8 * chunk_slot<D>(row, lslot));
      __builtin_amdgcn_global_load_lds((const void*)(p.kc + base + off), (lds_void_t*)(k_dst + 1024 * j), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(p.vc + base + off), (lds_void_t*)(v_dst + 1024 * j), 16, 0, 0);
    } else if (all_new || all_cached) {
      // all_cached implies full; a tile of new rows past the block's last key
      // reads that key instead (every LDS row holds finite data)
      const uint8_t* kt = (const uint8_t*)(all_new ? kin + (int64_t)(seq_start + t0 - pre) * row_stride
                                                   : p.kc + cache_base + (int64_t)t0 * D);
      const uint8_t* vt = (const uint8_t*)(all_new ? vin + (int64_t)(seq_start + t0 - pre) * row_stride
                                                   : p.vc + cache_base + (int64_t)t0 * D);
      uint32_t off;  // bytes from the tile's first row
      if (full)
        off = (all_new ? lane_new : lane_cached) + (uint32_t)(4 * i * C::kRowsPerInst) * 2u *
                                                       (uint32_t)(all_new ? row_stride : (int64_t)D);
      else
        off = 2u * (uint32_t)(min(row, key_end - 1 - t0) * row_stride + 8 * chunk_slot<D>(row, lslot));
      __builtin_amdgcn_global_load_lds((const void*)(kt + off), (lds_void_t*)(k_dst + 1024 * j), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vt + off), (lds_void_t*)(v_dst + 1024 * j), 16, 0, 0);
    } else {
      // a tile holding both cached and new rows (once per chunked sequence)
      const int kp = min(t0 + row, key_end - 1);
      const int col = 8 * chunk_slot<D>(row, lslot);
      __builtin_amdgcn_global_load_lds((const void*)(row_ptr(kin, p.kc, kp) + col),
                                       (lds_void_t*)(k_dst + 1024 * j), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(row_ptr(vin, p.vc, kp) + col),
                                       (lds_void_t*)(v_dst + 1024 * j), 16, 0, 0);
    }
  };
  // All of this wave's loads of tile t of blk, issued together (for a paged
  // cache with the three cases decided once per tile; the two forms compile
  // to different register allocations, each the better one for its kernels).
  auto issue_tile = [&](const Block blk, int t, int k_off, int v_off) __attribute__((always_inline)) {
    if constexpr (!kPaged) {
#pragma unroll
      for (int i = 0; i < C::kInstPerWave; ++i) issue_part(blk, t, k_off, v_off, i);
      return;
    }
    const int t0 = t * kBN;
    uint8_t* const k_dst = lds + k_off;
    uint8_t* const v_dst = lds + v_off;
    const bool full = t0 + kBN <= blk.key_end;
    const bool all_new = !kChunked || t0 >= pre;
    const bool all_cached = kChunked && t0 + kBN <= pre;
    if (kPaged && full && all_cached) {
      // the rows of one load instruction (4, 8 or 16) lie in one block
#pragma unroll
      for (int i = 0; i < C::kInstPerWave; ++i) {
        const int j = 4 * i + gw;
        const int r0 = t0 + j * C::kRowsPerInst;
        const int bi = __builtin_amdgcn_readfirstlane(r0 / kPageRows);
        const int64_t base = (((int64_t)bt_row[bi] * HK + hk) * kPageRows + r0 % kPageRows) * D;
        const int row = j * C::kRowsPerInst + lrow;
        const uint32_t off = (uint32_t)(lrow * D + 8 * chunk_slot<D>(row, lslot));
        __builtin_amdgcn_global_load_lds((const void*)(p.kc + base + off), (lds_void_t*)(k_dst + 1024 * j), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(p.vc + base + off), (lds_void_t*)(v_dst + 1024 * j), 16, 0, 0);
      }
    } else if (full && (all_new || all_cached)) {
      const int64_t step = all_new ? row_stride : (int64_t)D;
      const uint16_t* kt = all_new ? kin + (int64_t)(seq_start + t0 - pre) * row_stride
                                   : p.kc + cache_base + (int64_t)t0 * D;
      const uint16_t* vt = all_new ? vin + (int64_t)(seq_start + t0 - pre) * row_stride
                                   : p.vc + cache_base + (int64_t)t0 * D;
#pragma unroll
      for (int i = 0; i < C::kInstPerWave; ++i) {
        const int j = 4 * i + gw;
        const int row = j * C::kRowsPerInst + lrow;
        const uint32_t off = (uint32_t)(row * step + 8 * chunk_slot<D>(row, lslot));
        __builtin_amdgcn_global_load_lds((const void*)(kt + off), (lds_void_t*)(k_dst + 1024 * j), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(vt + off), (lds_void_t*)(v_dst + 1024 * j), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::kInstPerWave; ++i) {
        const int j = 4 * i + gw;
        const int row = j * C::kRowsPerInst + lrow;
        const int kp = min(t0 + row, blk.key_end - 1);
        const int col = 8 * chunk_slot<D>(row, lslot);
        __builtin_amdgcn_global_load_lds((const void*)(row_ptr(kin, p.kc, kp) + col),
                                         (lds_void_t*)(k_dst + 1024 * j), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(row_ptr(vin, p.vc, kp) + col),
                                         (lds_void_t*)(v_dst + 1024 * j), 16, 0, 0);
      }
    }
  };

  // copy the tile's new-token rows of blk from LDS to the cache (group-wide)
  auto cache_copy = [&](const Block blk, int t, int k_off, int v_off) __attribute__((always_inline)) {
    constexpr int kPer = C::kCpr / 4;    // chunks per lane and matrix
    const int t0 = t * kBN;
    const int gl = 64 * gw + lane;       // 0..255 within the group
    u32x4_t kr[kPer], vr[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = gl + kGroupThreads * i;
      const int row = idx / C::kCpr, ch = idx % C::kCpr;
      const uint32_t so = row * C::kRowBytes + 16 * chunk_slot<D>(row, ch);
      kr[i] = lds_read_b128<0>(lds0 + k_off + so);
      vr[i] = lds_read_b128<0>(lds0 + v_off + so);
    }
    lds_wait_all(kr, vr);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = gl + kGroupThreads * i;
      const int row = idx / C::kCpr, ch = idx % C::kCpr;
      const int kp = t0 + row;
      const bool mine = kp >= blk.own_lo && kp < blk.key_end;
      if constexpr (kCache != kCacheBf16) {
        // the row's absolute maximum over its kCpr lanes (all lanes take part)
        const float ka = group_max<C::kCpr>(absmax8(kr[i]));
        const float va = group_max<C::kCpr>(absmax8(vr[i]));
        if (mine) {
          const int64_t dst = cache_base + (int64_t)kp * D + 8 * ch;
          if constexpr (kCache == kCacheInt8) {
            __builtin_nontemporal_store(quantize8(kr[i], ka), (u32x2_t*)(p.kq + dst));
            __builtin_nontemporal_store(quantize8(vr[i], va), (u32x2_t*)(p.vq + dst));
          } else {
            __builtin_nontemporal_store(quantize_fp8(kr[i], ka), (u32x2_t*)(p.kq + dst));
            __builtin_nontemporal_store(quantize_fp8(vr[i], va), (u32x2_t*)(p.vq + dst));
          }
          if (ch == 0) {
            p.ks[cache_base / D + kp] = kCache == kCacheInt8 ? int8_scale(ka) : fp8_scale(ka);
            p.vs[cache_base / D + kp] = kCache == kCacheInt8 ? int8_scale(va) : fp8_scale(va);
          }
        }
      } else if (mine) {
        // streaming stores: this launch never reads these rows back, so they
        // should not take L2 lines from the K/V tiles other work-groups reuse
        const int64_t dst = cache_elem(kp) + 8 * ch;
        __builtin_nontemporal_store(kr[i], (u32x4_t*)(p.kc + dst));
        __builtin_nontemporal_store(vr[i], (u32x4_t*)(p.vc + dst));
      }
    }
  };

  // ---------------------------------------------------------------- wave state
  Rows<D> st;
  int qrow0, len_rows;  // first local row of the wave (32 rows); rows < len_rows exist

  auto begin_rows = [&](const Block& blk) __attribute__((always_inline)) {
    qrow0 = blk.q0 + 32 * gw;
    len_rows = blk.qend;
    const int row = qrow0 + ql;
    const bool ok = row < len_rows;
    const uint16_t* src = p.q + ((int64_t)(seq_start + (ok ? row : 0)) * H + h) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4_t v = ok ? *(const u32x4_t*)(src + 16 * ks) : u32x4_t{0u, 0u, 0u, 0u};
      if (p.neg_q) v ^= 0x80008000u;  // negative scale: flip the sign of q instead
      st.q[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
#pragma unroll
    for (int i = 0; i < D / 32; ++i) st.o[i] = f32x16_t{};
    st.m = kMInit;
    st.l = 0.f;
  };

  auto store_rows = [&](float l_part) __attribute__((always_inline)) {
    const int row = qrow0 + ql;
    const float inv = 1.f / row_sum_halves(l_part);
    if (row >= len_rows) return;
    // Lane (row, hh) holds d = 32 mb + 8 cc + 4 hh + [0, 4).  Lanes l and l^32
    // (the same row) trade pieces so that the hh = 0 lane holds the 8
    // consecutive d of chunk 2 cp and the hh = 1 lane those of chunk 2 cp + 1:
    // 16-byte stores, 32 contiguous bytes of a row per lane pair.
    uint16_t* dst = p.out + ((int64_t)(seq_start + row) * H + h) * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int cp = 0; cp < 2; ++cp) {
        const int ca = 2 * cp, cb = 2 * cp + 1;
        const uint32_t a0 = pack_bf16x2(st.o[mb][4 * ca + 0] * inv, st.o[mb][4 * ca + 1] * inv);
        const uint32_t a1 = pack_bf16x2(st.o[mb][4 * ca + 2] * inv, st.o[mb][4 * ca + 3] * inv);
        const uint32_t b0 = pack_bf16x2(st.o[mb][4 * cb + 0] * inv, st.o[mb][4 * cb + 1] * inv);
        const uint32_t b1 = pack_bf16x2(st.o[mb][4 * cb + 2] * inv, st.o[mb][4 * cb + 3] * inv);
        // hh = 0 sends its chunk-cb piece, hh = 1 its chunk-ca piece; lanes
        // 0-31 find the partner's value in the second result, 32-63 in the first
        const uint32_t s0 = hh ? a0 : b0, s1 = hh ? a1 : b1;
        const auto r0 = __builtin_amdgcn_permlane32_swap(s0, s0, false, false);
        const auto r1 = __builtin_amdgcn_permlane32_swap(s1, s1, false, false);
        const uint32_t o0 = hh ? r0[0] : r0[1], o1 = hh ? r1[0] : r1[1];
        const u32x4_t w = hh ? u32x4_t{o0, o1, b0, b1} : u32x4_t{a0, a1, o0, o1};
        *(u32x4_t*)(dst + 32 * mb + 8 * (hh ? cb : ca)) = w;
      }
  };

  // Split mode: the rows' partial result over this item's keys, O / l in fp32
  // and log2(l) + m (the log2 of the sum of 2^(s c) over those keys; -inf
  // when a row sees none of them), at slot (token, head, segment).
  auto store_partial = [&](float l_part) __attribute__((always_inline)) {
    const int row = qrow0 + ql;
    const float l = row_sum_halves(l_part);
    if (row >= len_rows) return;
    const bool any = l > 0.f;
    const float inv = any ? 1.f / l : 0.f;
    const int64_t slot = ((int64_t)(seq_start + row) * H + h) * p.max_segs + seg;
    float* dst = p.part_o + slot * D + 4 * hh;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const f32x4_t w = {st.o[mb][4 * cc + 0] * inv, st.o[mb][4 * cc + 1] * inv,
                           st.o[mb][4 * cc + 2] * inv, st.o[mb][4 * cc + 3] * inv};
        *(f32x4_t*)(dst + 32 * mb + 8 * cc) = w;
      }
    if (hh == 0) p.part_lse[slot] = any ? st.m + __builtin_amdgcn_logf(l) : kNegInf;
  };

  // Lane parts of the LDS read addresses (byte offsets within a tile).
  //  Score operand: lane l reads key row kr = 32 kb + l%32, chunk 2 ks + l/32;
  //  the swizzle depends on kr % 8 = l % 8 only, and for ks = j + 4 m the
  //  slot is 8 m + slot(2 j + l/32), so bases j < 4 plus immediates cover all.
  //  PV operand: lane L of 16-lane group G points at 4 consecutive d of key
  //  row 16 g + 8 r + 4 (G/2) + (L%16)/4 at d = 32 mb + 16 (G%2) + 4 (L%4) and
  //  receives the 4 keys {16 g + 8 r + 4 (G/2) + j} at its own d = 32 mb + L%32;
  //  chunk 4 mb + c lands in slot 8 (mb/2) + slot(4 (mb%2) + c), so two bases
  //  (mb even / odd) plus immediates cover all.
  uint32_t kbase[C::kKReadBases];
#pragma unroll
  for (int j = 0; j < C::kKReadBases; ++j) kbase[j] = ql * C::kRowBytes + 16 * chunk_slot<D>(ql, 2 * j + hh);
  uint32_t vbase[2];
  {
    const int tg = lane >> 4, tl = lane & 15;
    const int vrow0 = 4 * (tg >> 1) + (tl >> 2);
    const int vd0 = 16 * (tg & 1) + 4 * (tl & 3);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int d = 32 * e + vd0;
      vbase[e] = vrow0 * C::kRowBytes + 16 * chunk_slot<D>(vrow0, (d >> 3) & (C::kCpr - 1)) + 2 * (d & 7);
    }
  }

  // S^T = K Q^T for one 64-key tile (two 32-key blocks), K from LDS at k_off;
  // hook(step) runs after each 16-d step's MFMAs (the next tile's loads are
  // spread there).
  auto score = [&](int k_off, f32x16_t (&s)[2], auto&& hook) __attribute__((always_inline)) {
    constexpr int NK = D / 16;
    uint32_t kb_addr[C::kKReadBases];
#pragma unroll
    for (int j = 0; j < C::kKReadBases; ++j) kb_addr[j] = lds0 + k_off + kbase[j];
    s[0] = f32x16_t{};
    s[1] = f32x16_t{};
    u32x4_t a[NK][2];
    auto rd = [&](auto ks_tag) __attribute__((always_inline)) {
      constexpr int ks = decltype(ks_tag)::value;
      constexpr int o = 128 * (ks >> 2);
      a[ks][0] = lds_read_b128<o>(kb_addr[ks & 3]);
      a[ks][1] = lds_read_b128<o + 32 * C::kRowBytes>(kb_addr[ks & 3]);
    };
    constexpr int kAhead = NK < 4 ? NK : 4;  // 16-d steps in flight
    static_for<0, kAhead>(rd);
    static_for<0, NK>([&](auto ks_tag) __attribute__((always_inline)) {
      constexpr int ks = decltype(ks_tag)::value;
      constexpr int later = (NK - 1 - ks) < (kAhead - 1) ? (NK - 1 - ks) : (kAhead - 1);
      lds_wait<2 * later>(a[ks][0], a[ks][1]);
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[ks][0]), st.q[ks], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[ks][1]), st.q[ks], s[1], 0, 0, 0);
      if constexpr (ks + kAhead < NK) rd(std::integral_constant<int, ks + kAhead>{});
      hook(ks_tag);
    });
  };

  // Online softmax over one tile's scores: updates m, l (and rescales O when m
  // moves), returns P^T as the PV B operand.
  auto softmax = [&](f32x16_t (&s)[2], const Block blk, int t, auto mask_tag, bf16x8_t (&pb)[4]) __attribute__((always_inline)) {
    constexpr bool kMask = decltype(mask_tag)::value;
    const int t0 = t * kBN;
    const int qa = pre + qrow0 + ql;  // this lane's absolute query position
    if constexpr (kMask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kp = t0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (kp > qa || kp >= blk.key_end) s[kb][r] = kNegInf;
        }
    }
    float mx4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float m8 = s[j >> 1][8 * (j & 1)];
#pragma unroll
      for (int i = 1; i < 8; ++i) m8 = fmaxf(m8, s[j >> 1][8 * (j & 1) + i]);
      mx4[j] = m8;
    }
    const float mx = row_max_halves(fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3])));
    const float mt = (mx == kNegInf) ? mx : mx * c;
    if (__any(mt > st.m + kRescale)) {  // wave-uniform; taken on the first real tile
      const float m_new = fmaxf(st.m, mt);
      const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
      st.l *= alpha;
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb) st.o[mb] *= alpha;
      st.m = m_new;
    }
    const float neg_m = -st.m;
    float ls[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float sv = s[g >> 1][8 * (g & 1) + i];
        e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, c, neg_m));  // c > 0: masked -> 0
      }
      ls[g] = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
      u32x4_t w = {pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                   pack_bf16x2(e[6], e[7])};
      pb[g] = __builtin_bit_cast(bf16x8_t, w);
    }
    st.l += (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };

  // O^T += V^T P^T for one tile, V from LDS at v_off; 16-key steps g outer,
  // the D/32 accumulators inner (no back-to-back dependent MFMAs); hook(g)
  // runs after each step's MFMAs.
  auto pv = [&](int v_off, const bf16x8_t (&pb)[4], auto&& hook) __attribute__((always_inline)) {
    constexpr int NV = C::kVReadsPerStep;
    const uint32_t va0 = lds0 + v_off + vbase[0];
    const uint32_t va1 = lds0 + v_off + vbase[1];
    s16x4_t vt[4][NV];
    auto rd = [&](auto g_tag) __attribute__((always_inline)) {
      constexpr int g = decltype(g_tag)::value;
      static_for<0, D / 32>([&](auto mb_tag) __attribute__((always_inline)) {
        constexpr int mb = decltype(mb_tag)::value;
        constexpr int o = 128 * (mb >> 1) + 16 * g * C::kRowBytes;
        const uint32_t a = (mb & 1) ? va1 : va0;
        vt[g][2 * mb] = lds_read_tr<o>(a);
        vt[g][2 * mb + 1] = lds_read_tr<o + 8 * C::kRowBytes>(a);
      });
    };
    rd(std::integral_constant<int, 0>{});
    rd(std::integral_constant<int, 1>{});
    static_for<0, 4>([&](auto g_tag) __attribute__((always_inline)) {
      constexpr int g = decltype(g_tag)::value;
      lds_wait_tr<(g < 3 ? NV : 0)>(vt[g]);
      static_for<0, D / 32>([&](auto mb_tag) __attribute__((always_inline)) {
        constexpr int mb = decltype(mb_tag)::value;
        const bf16x8_t vf = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(vt[g][2 * mb], vt[g][2 * mb + 1], 0, 1, 2, 3, 4, 5, 6, 7));
        st.o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[g], st.o[mb], 0, 0, 0);
      });
      if constexpr (g + 2 < 4) rd(std::integral_constant<int, g + 2>{});
      hook(g_tag);
    });
  };

  // does this wave have rows that see some key of tile t, and must it mask?
  auto tile_use = [&](const Block blk, int t, bool& use, bool& mask) __attribute__((always_inline)) {
    const int t0 = t * kBN;
    const int qa0 = pre + qrow0;
    use = qrow0 < len_rows && t0 <= qa0 + 31;
    mask = (t0 + kBN - 1 > qa0) || (t0 + kBN > blk.key_end);
  };

  // ---------------------------------------------------------------- main loop
  // Interval j ends with one barrier.  Lower group: tile j as S, softmax, PV.
  // Upper group: PV of its tile j-1 (P kept in registers, V in a ring of
  // three), then S and softmax of tile j.  On each SIMD one wave's softmax so
  // runs beside the other's MFMAs.  Loads of both groups' tile j+1 are issued
  // at the start of interval j into buffers whose last readers finished
  // before the previous barrier.
  bool on_hi_rows = upper || !has_lo;  // which block's rows this wave holds
  begin_rows(make_block(on_hi_rows ? +qb_hi : +z, len, pre));

  auto lower_k = [&](int j) { return C::kLowerOff + (j & 1) * 2 * C::kTileBytes; };
  {
    const Pick p0 = pick_tile(0, upper, n_up, e_lo, e_hi, z, qb_hi);
    if (p0.valid) {
      if (upper) issue_tile(make_block(p0.qb, len, pre), tb + p0.t, C::kUpperK, C::kUpperV);
      else issue_tile(make_block(p0.qb, len, pre), tb + p0.t, lower_k(0), lower_k(0) + C::kTileBytes);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  bf16x8_t p_prev[4];
  bool have_prev = false;
  int v_prev = 2, v_cur = 0, v_next = 1;  // upper V ring: tiles j-1, j, j+1
  // The next tile's loads (kInstPerWave instructions per matrix and wave) are
  // spread between a tile's MFMA steps, so the vector memory path drains
  // them while the matrix cores work instead of stalling the issuing waves.
  auto no_hook = [](auto) __attribute__((always_inline)) {};
  auto spread = [&](bool active, const Block nb, int nt, int nk, int nv, auto steps_tag) __attribute__((always_inline)) {
    return [&, active, nb, nt, nk, nv, steps_tag](auto step_tag) __attribute__((always_inline)) {
      constexpr int kSteps = decltype(steps_tag)::value;
      constexpr int st_ = decltype(step_tag)::value;
      static_for<0, C::kInstPerWave>([&](auto i_tag) __attribute__((always_inline)) {
        constexpr int i = decltype(i_tag)::value;
        if constexpr ((i + 1) * kSteps / C::kInstPerWave - 1 == st_)
          if (active) issue_part(nb, nt, nk, nv, i);
      });
    };
  };
  for (int j = 0; j <= n_up; ++j) {
    if (upper) {
      const bool load_next = j + 1 < n_up;
      const Pick nx = pick_tile(j + 1, true, n_up, e_lo, e_hi, z, qb_hi);
      const Block nb = make_block(nx.qb, len, pre);
      const int nk = C::kUpperK + ((j + 1) & 1) * C::kTileBytes, nv = C::kUpperV + v_next * C::kTileBytes;
      // paged caches keep the burst at the start of the interval: their
      // per-instruction block lookups inside the MFMA steps cost more
      // registers than the spread saves
      if (have_prev && !kPaged)
        pv(C::kUpperV + v_prev * C::kTileBytes, p_prev, spread(load_next, nb, tb + nx.t, nk, nv, std::integral_constant<int, 4>{}));
      else if (load_next)
        issue_tile(nb, tb + nx.t, nk, nv);
      if (have_prev && kPaged) pv(C::kUpperV + v_prev * C::kTileBytes, p_prev, no_hook);
      have_prev = false;
      if (j < n_up) {
        const Block blk = bhi;
        const int t = tb + j;
        if (t * kBN + kBN > blk.own_lo)  // a self-paired block's first tiles hold new tokens
          if (writes_cache) cache_copy(blk, t, C::kUpperK + (j & 1) * C::kTileBytes, C::kUpperV + v_cur * C::kTileBytes);
        bool use, mask;
        tile_use(blk, t, use, mask);
        if (use) {
          f32x16_t s[2];
          score(C::kUpperK + (j & 1) * C::kTileBytes, s, no_hook);
          if (mask)
            softmax(s, blk, t, std::true_type{}, p_prev);
          else
            softmax(s, blk, t, std::false_type{}, p_prev);
          have_prev = true;
        }
      }
      const int r = v_prev;
      v_prev = v_cur;
      v_cur = v_next;
      v_next = r;
    } else if (j < n_lo) {
      const bool load_next = j + 1 < n_lo;
      const Pick nx = pick_tile(j + 1, false, n_up, e_lo, e_hi, z, qb_hi);
      const Block nb = make_block(nx.qb, len, pre);
      const int nk = lower_k(j + 1), nv = lower_k(j + 1) + C::kTileBytes;
      if (kPaged && load_next) issue_tile(nb, tb + nx.t, nk, nv);
      const Pick pk = pick_tile(j, false, n_up, e_lo, e_hi, z, qb_hi);
      const Block blk = make_block(pk.qb, len, pre);
      const int t = tb + pk.t;
      if (writes_cache && t * kBN + kBN > blk.own_lo) cache_copy(blk, t, lower_k(j), lower_k(j) + C::kTileBytes);
      if (pk.on_hi && !on_hi_rows) {  // lower group moves from the light block to the heavy one
        store_rows(st.l);
        on_hi_rows = true;
        begin_rows(bhi);
      }
      bool use, mask;
      tile_use(blk, t, use, mask);
      if (use) {
        f32x16_t s[2];
        bf16x8_t pb[4];
        score(lower_k(j), s, spread(load_next && !kPaged, nb, tb + nx.t, nk, nv, std::integral_constant<int, D / 16>{}));
        if (mask)
          softmax(s, blk, t, std::true_type{}, pb);
        else
          softmax(s, blk, t, std::false_type{}, pb);
        pv(lower_k(j) + C::kTileBytes, pb, no_hook);
      } else if (load_next && !kPaged) {
        issue_tile(nb, tb + nx.t, nk, nv);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of the next tile have landed
    __syncthreads();
  }

  // ---------------------------------------------------------------- merge
  if (!on_hi_rows) {  // lower group never reached the heavy block: finish the light one
    store_rows(st.l);
    on_hi_rows = true;
    begin_rows(bhi);   // empty partial state for the heavy block's rows
  }
  // the loop's last barrier has freed the tile buffers
  float* mbuf = reinterpret_cast<float*>(lds) + gw * C::kMergeWaveFloats;
  if (upper) {
    mbuf[lane] = st.m;
    mbuf[64 + lane] = st.l;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mbuf[(2 + 16 * mb + r) * 64 + lane] = st.o[mb][r];
  }
  __syncthreads();
  if (!upper && qrow0 < len_rows) {
    const float m2 = mbuf[lane];
    const float l2 = mbuf[64 + lane];
    const float m = fmaxf(st.m, m2);
    const float fa = __builtin_amdgcn_exp2f(st.m - m);  // 0 if this group saw no tile
    const float fb = __builtin_amdgcn_exp2f(m2 - m);
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[mb][r] = st.o[mb][r] * fa + mbuf[(2 + 16 * mb + r) * 64 + lane] * fb;
    st.m = m;  // the partial's log2-sum-exp2 is taken against the merged max
    if (kSplit && nseg > 1)
      store_partial(st.l * fa + l2 * fb);
    else
      store_rows(st.l * fa + l2 * fb);
  }
}

template <int D, bool kChunked, int kCache = kCacheBf16>
__global__ __launch_bounds__(kThreads)
void prefill_fwd_kernel(FwdParams p) {
  // raw id builtins: the device library's id helpers are built with IEEE mode
  // on and would not inline into this IEEE-off kernel
  const int h = __builtin_amdgcn_workgroup_id_x(), b = __builtin_amdgcn_workgroup_id_y();
  int z = __builtin_amdgcn_workgroup_id_z();
  if constexpr (kChunked && kCache == kCacheBf16) {
    // Chunked: a length-1 row (a decode row) reads its whole cached context
    // for one query, a GEMV: it runs as one VALU decode unit (decode_rows.h)
    // over all its keys, written straight to out and to the cache, instead
    // of as a 128-row MFMA block holding one row ["大模型 Prompt Prefill 阶段的高效
    // Batching 与算子排布" §3; untitled page www.zwxr.cn/news/300951 §1.2].
    const int len = p.cu[b + 1] - p.cu[b];
    if (len == 1) {
      // in the last z-layer: every layer before it holds only multi-row
      // sequences' pairs, so those are all dispatched before any decode unit
      if (z == p.grid_z - 1) {
        float* const red = reinterpret_cast<float*>(fwd_lds<D, kChunked, false, kCache, false, 0>());
        static_assert(dec::red_floats<D, 1, kWaves>() * 4 <= Cfg<D>::kLdsBytes, "decode reduction exceeds LDS");
        dec::decode_unit<D, 1, false, kWaves>(p, (int64_t)h, make_int4(b, 0, 1, 0), red, nullptr, nullptr);
      }
      return;
    }
    // pairs in reverse order: the first z-layer holds only the longest
    // sequences' pairs, so the chunk's long blocks are dispatched first and
    // the decode rows (last layer) fill the compute units behind them
    z = p.grid_z - 1 - z;
  }
  fwd_item<D, kChunked, false, kCache>(p, h, b, z, 0, 1);
}

// Split-KV chunked prefill: a persistent grid walks the planned items, item i
// of head h being step i * H + h; with the grid a multiple of H (and of the 8
// XCDs) a work-group keeps one head, and all of a head's items run on one XCD.
// The decode rows then run in a launch of their own (splitkv.hip).
template <int D, bool kPaged>
__global__ __launch_bounds__(kThreads)
void prefill_fwd_split_kernel(FwdParams p) {
  const int H = p.num_heads;
  const int64_t steps = (int64_t)p.hdr[0] * H;
  const int grid = p.split_grid;
  for (int64_t g = __builtin_amdgcn_workgroup_id_x(); g < steps; g += grid) {
    const int4 it = p.items[g / H];
    fwd_item<D, true, true, kCacheBf16, kPaged>(p, (int)(g % H), it.x, it.y, it.z, it.w);
    __syncthreads();  // the next item's first loads reuse the merge buffers
  }
}

// Split-KV chunked prefill with the decode rows in the same launch, so that
// both kinds of planned work run at once.  The attention items (a query
// block over one segment of its keys) are MFMA-bound; the decode units
// (length-1 rows, decode_rows.h) are HBM-bound ["大模型 Prompt Prefill 阶段的高效
// Batching 与算子排布" §3: a chunk runs beside decode rows in one step].
// Work-groups [0, items_first) start on the items and the rest on the decode
// units, so the matrix cores and the memory stream are busy together; a
// work-group whose list runs dry joins the other.  Item step j of head h is
// queued on XCD h % 8 and a work-group (on XCD w % 8 for work-group w) drains
// its own XCD's queue first, so the query blocks of one head that read the
// same K/V tiles share an L2.  Each work-group's first item or unit is fixed
// by its number; the rest are handed out through counters the plan zeroed
// (item j of queue x is R_x + counter x, R_x the work-groups of XCD x that
// start on the items; decode unit g is U + counter 8, U the work-groups that
// start on the units).  With no decode units all work-groups start on the
// items, with no items all on the units.
template <int D, bool kPaged>
__global__ __launch_bounds__(kThreads)
void prefill_fwd_mixed_kernel(FwdParams p) {
  __shared__ unsigned long long taken;
  const int tid = __builtin_amdgcn_workitem_id_x();
  const int wg = __builtin_amdgcn_workgroup_id_x();
  const int H = p.num_heads;
  const unsigned long long items = (uint32_t)p.hdr[0];
  const unsigned long long units = (unsigned long long)(uint32_t)p.hdr[2] * (uint32_t)(H / p.dec_heads);
  const int first = units == 0 ? p.split_grid : items == 0 ? 0 : p.items_first;  // work-groups starting on items
  auto R = [&](int x) __attribute__((always_inline)) { return (unsigned long long)(uint32_t)((first - x + 7) / 8); };
  const unsigned long long U = (uint32_t)(p.split_grid - first);
  // base + the next value of counter i, the same in every wave, or `end` once
  // base + counter has reached end.  The counter is read first: once a list
  // is empty every work-group asks at about the same time, and loads do not
  // queue behind each other at the L2 as read-modify-writes of one address do.
  auto take = [&](int i, unsigned long long base, unsigned long long end) __attribute__((always_inline)) {
    if (base >= end) return end;  // all of this list is handed out by number
    if (tid == 0) {
      unsigned long long c = __hip_atomic_load(p.counters + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (base + c < end) c = atomicAdd(p.counters + i, 1ull);
      taken = base + c < end ? base + c : end;
    }
    __syncthreads();
    const unsigned long long v = taken;
    __syncthreads();  // taken is rewritten by the next call
    return v;
  };
  // the items of queue x until it is empty, starting with the work-group's
  // own if `own`
  auto drain = [&](int x, bool own) __attribute__((always_inline)) {
    const int nh = (H - x + 7) / 8;  // heads h = x (mod 8)
    const unsigned long long end = items * nh;
    for (unsigned long long j = own ? (uint32_t)wg / 8 : take(x, R(x), end); j < end; j = take(x, R(x), end)) {
      const int4 it = p.items[j / nh];
      fwd_item<D, true, true, kCacheBf16, kPaged, 1>(p, x + 8 * (int)(j % nh), it.x, it.y, it.z, it.w);
      __syncthreads();  // the next item's first loads reuse the merge buffers
    }
  };
  float* const red = reinterpret_cast<float*>(fwd_lds<D, true, true, kCacheBf16, kPaged, 1>());
  static_assert(dec::red_floats<D, 2, kWaves>() * 4 <= Cfg<D>::kLdsBytes, "decode reduction exceeds LDS");
  const bool items_first = wg < first;
  for (int phase = 0; phase < 2; ++phase) {
    if ((phase == 0) == items_first) {
      // this XCD's queue, then the others that still hold items (all eight
      // probed in one round trip once the own queue is empty)
      uint32_t open = 1u << (wg & 7);
      for (int i = 0; i < 8; ++i) {
        if (i == 1) {
          if (tid < 8) {
            const int nh = (H - tid + 7) / 8;
            const bool more = R(tid) + __hip_atomic_load(p.counters + tid, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT) < items * nh;
            const unsigned long long mask = __ballot(more);
            if (tid == 0) taken = mask;
          }
          __syncthreads();
          open = (uint32_t)taken;
          __syncthreads();
        }
        const int x = (wg + i) & 7;
        if ((open >> x) & 1u) drain(x, phase == 0 && i == 0);
      }
    } else if (units > 0) {
      // each unit takes the next unit's number while it runs; the host sends
      // decode rows here only with one or two query heads per unit (units of
      // 4 or 8 heads would also cost registers the items need)
      unsigned long long* const ctr = p.counters + 8;
      for (unsigned long long g = phase == 0 ? (uint32_t)(wg - first) : take(8, U, units); g < units; g = U + taken) {
        if (p.dec_heads == 1)
          dec::decode_unit<D, 1, kPaged, kWaves>(p, (int64_t)g, red, ctr, &taken);
        else
          dec::decode_unit<D, 2, kPaged, kWaves>(p, (int64_t)g, red, ctr, &taken);
      }
      __syncthreads();  // every wave has read taken before take() rewrites it
    }
  }
}

template <int D, bool kChunked>
hipError_t launch_d(const FwdParams& p, int num_seqs, hipStream_t stream) {
  dim3 grid(p.num_heads, num_seqs, p.grid_z);
  hipLaunchKernelGGL((prefill_fwd_kernel<D, kChunked>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

namespace {
template <int kCache>
hipError_t launch_quant(const FwdParams& p, int num_seqs, int head_dim, hipStream_t stream) {
  const dim3 grid(p.num_heads, num_seqs, p.grid_z);
  switch (head_dim) {
    case 32: hipLaunchKernelGGL((prefill_fwd_kernel<32, false, kCache>), grid, dim3(kThreads), 0, stream, p); break;
    case 64: hipLaunchKernelGGL((prefill_fwd_kernel<64, false, kCache>), grid, dim3(kThreads), 0, stream, p); break;
    case 128: hipLaunchKernelGGL((prefill_fwd_kernel<128, false, kCache>), grid, dim3(kThreads), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_prefill_fwd_int8(const FwdParams& p, int num_seqs, int head_dim, hipStream_t stream) {
  return launch_quant<kCacheInt8>(p, num_seqs, head_dim, stream);
}

hipError_t launch_prefill_fwd_fp8(const FwdParams& p, int num_seqs, int head_dim, hipStream_t stream) {
  return launch_quant<kCacheFp8>(p, num_seqs, head_dim, stream);
}

template <int D>
void split_d(const FwdParams& p, bool paged, hipStream_t stream) {
  const dim3 grid(p.split_grid), block(kThreads);
  if (p.fuse_decode) {
    if (paged)
      hipLaunchKernelGGL((prefill_fwd_mixed_kernel<D, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((prefill_fwd_mixed_kernel<D, false>), grid, block, 0, stream, p);
  } else {
    if (paged)
      hipLaunchKernelGGL((prefill_fwd_split_kernel<D, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((prefill_fwd_split_kernel<D, false>), grid, block, 0, stream, p);
  }
}

hipError_t launch_prefill_fwd_split(const FwdParams& p, int head_dim, bool paged, hipStream_t stream) {
  switch (head_dim) {
    case 32: split_d<32>(p, paged, stream); break;
    case 64: split_d<64>(p, paged, stream); break;
    case 128: split_d<128>(p, paged, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
int split_occ(bool fused) {
  int n = 0;
  const hipError_t e =
      fused ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_fwd_mixed_kernel<D, false>, kThreads, 0)
            : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_fwd_split_kernel<D, false>, kThreads, 0);
  return e == hipSuccess ? n : 0;
}

int fwd_split_blocks_per_cu(int head_dim, bool fused) {
  switch (head_dim) {
    case 32: return split_occ<32>(fused);
    case 64: return split_occ<64>(fused);
    case 128: return split_occ<128>(fused);
    default: return 0;
  }
}

int fwd_block_rows() { return kBM; }

int fwd_grid_blocks(int max_seqlen) {
  const int nqb = (max_seqlen + kBM - 1) / kBM;
  return (nqb + 1) / 2;  // one work-group per pair of query blocks
}

hipError_t launch_prefill_fwd(const FwdParams& p, int num_seqs, int head_dim, bool chunked,
                              hipStream_t stream) {
  switch (head_dim) {
    case 32: return chunked ? launch_d<32, true>(p, num_seqs, stream) : launch_d<32, false>(p, num_seqs, stream);
    case 64: return chunked ? launch_d<64, true>(p, num_seqs, stream) : launch_d<64, false>(p, num_seqs, stream);
    case 128: return chunked ? launch_d<128, true>(p, num_seqs, stream) : launch_d<128, false>(p, num_seqs, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
