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
// ["大模型推理优化：Prefill、Decode与KV Cache的工程实践" §1.3].
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
//  * Online softmax in the exp2 domain with c = |scale| log2(e) >= 0 (a
//    negative scale flips q's sign instead): max over raw scores, p =
//    2^(s c - m) as one FMA and one v_exp_f32.  The running max m only moves
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

#include "launch.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = 128;            // query rows per block (4 waves x 32)
constexpr int kGroupThreads = 256;  // one group = 4 waves
constexpr int kBN = 64;             // keys per tile
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
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t two = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(two, bf16x2_t));
}

template <int D>
struct Cfg {
  static constexpr int kCpr = D / 8;                    // 16-byte chunks per row
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kTileBytes = kBN * kRowBytes;    // one K or V tile
  static constexpr int kSlotBytes = 2 * kTileBytes;     // K tile then V tile
  static constexpr int kRowsPerInst = 1024 / kRowBytes; // rows per 1 KB direct load
  static constexpr int kInstPerTile = kBN / kRowsPerInst;
  static constexpr int kInstPerWave = kInstPerTile / 4; // per tile, per wave of a group
  // merge buffer: per upper wave, per lane: m, l and D/2 accumulators
  static constexpr int kMergeBytes = 4 * (2 + D / 2) * 64 * 4;
  static constexpr int kLdsBytes = (4 * kSlotBytes > kMergeBytes) ? 4 * kSlotBytes : kMergeBytes;
};

// 16-byte chunk slot of chunk c in row r (XOR swizzle, stays inside the row)
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

// State of a wave's 32 query rows.
template <int D>
struct Rows {
  bf16x8_t q[D / 16];
  f32x16_t o[D / 32];
  float m, l;
};

template <int D, bool kChunked>
__global__ __launch_bounds__(kThreads)
void prefill_fwd_kernel(FwdParams p) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::kLdsBytes];

  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int z = blockIdx.z;
  const int64_t H = p.num_heads;

  const int seq_start = p.cu[b];
  const int len = p.cu[b + 1] - seq_start;
  const int nqb = (len + kBM - 1) / kBM;
  const int qb_hi = nqb - 1 - z;
  if (z > qb_hi) return;                 // no block pair left for this work-group
  const int pre = kChunked ? p.prefix[b] : 0;
  const bool has_lo = z < qb_hi;
  const Block blo = make_block(z, len, pre);
  const Block bhi = make_block(qb_hi, len, pre);
  const int e_lo = has_lo ? blo.ntiles : 0;
  const int e_hi = bhi.ntiles;
  const int n_iter = (e_lo + e_hi + 1) / 2;  // tiles of the upper group

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int ql = lane & 31;
  const int hh = lane >> 5;
  const bool upper = wave >= 4;
  const int gw = wave & 3;               // wave within its group

  uint8_t* const grp_lds = lds + (upper ? 2 * C::kSlotBytes : 0);

  const int64_t row_stride = H * D;      // elements between consecutive tokens
  const uint16_t* __restrict__ kin = p.k + (int64_t)h * D;
  const uint16_t* __restrict__ vin = p.v + (int64_t)h * D;
  const int64_t cache_base = kChunked ? ((int64_t)b * H + h) * p.cap * D
                                      : (int64_t)seq_start * H * D + (int64_t)h * len * D;
  const float c = p.scale_log2;          // |scale| * log2(e) >= 0

  // ---------------------------------------------------------------- schedule
  auto my_tile = [&](int it, bool& on_hi, int& t) -> bool {
    if (upper) { on_hi = true; t = it; return it < n_iter; }
    if (it < e_lo) { on_hi = false; t = it; return true; }
    on_hi = true;
    t = n_iter + (it - e_lo);
    return t < e_hi;
  };

  // ---------------------------------------------------------------- staging
  // Wave gw of a group issues instructions j = 4 i + gw (i < kInstPerWave) per
  // tile and matrix; lane l fills row j * kRowsPerInst + l / kCpr, chunk slot
  // l % kCpr, from source chunk chunk_slot(row, slot) (the XOR is an
  // involution).  Rows past the block's last key read the last key instead,
  // so every LDS row holds finite data (masked keys get weight 0).
  const int lrow = lane / C::kCpr;
  const int lslot = lane % C::kCpr;

  auto row_ptr = [&](const uint16_t* __restrict__ in, const uint16_t* cache, int kp) {
    if (kChunked && kp < pre) return cache + cache_base + (int64_t)kp * D;
    return in + (int64_t)(seq_start + kp - pre) * row_stride;
  };

  auto issue_tile = [&](const Block& blk, int t, int slot) {
    const int t0 = t * kBN;
    uint8_t* const k_dst = grp_lds + slot * C::kSlotBytes;
    uint8_t* const v_dst = k_dst + C::kTileBytes;
    const bool full = t0 + kBN <= blk.key_end;
    const bool all_new = !kChunked || t0 >= pre;
    const bool all_cached = kChunked && t0 + kBN <= pre;
    if (full && (all_new || all_cached)) {
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
  auto cache_copy = [&](const Block& blk, int t, int slot) {
    const int t0 = t * kBN;
    const uint8_t* const k_src = grp_lds + slot * C::kSlotBytes;
    const uint8_t* const v_src = k_src + C::kTileBytes;
    const int gl = 64 * gw + lane;       // 0..255 within the group
    for (int idx = gl; idx < kBN * C::kCpr; idx += kGroupThreads) {
      const int row = idx / C::kCpr, ch = idx % C::kCpr;
      const int kp = t0 + row;
      if (kp >= blk.own_lo && kp < blk.key_end) {
        const int so = row * C::kRowBytes + 16 * chunk_slot<D>(row, ch);
        const int64_t dst = cache_base + (int64_t)kp * D + 8 * ch;
        *(u32x4_t*)(p.kc + dst) = *(const u32x4_t*)(k_src + so);
        *(u32x4_t*)(p.vc + dst) = *(const u32x4_t*)(v_src + so);
      }
    }
  };

  // ---------------------------------------------------------------- wave state
  Rows<D> st;
  int qrow0, len_rows;  // first local row of the wave (32 rows); rows < len_rows exist

  auto begin_rows = [&](const Block& blk) {
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

  auto store_rows = [&](float l_part) {
    const int row = qrow0 + ql;
    const float inv = 1.f / row_sum_halves(l_part);
    if (row >= len_rows) return;
    uint16_t* dst = p.out + ((int64_t)(seq_start + row) * H + h) * D + 4 * hh;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        u32x2_t w = {pack_bf16x2(st.o[mb][4 * cc + 0] * inv, st.o[mb][4 * cc + 1] * inv),
                     pack_bf16x2(st.o[mb][4 * cc + 2] * inv, st.o[mb][4 * cc + 3] * inv)};
        *(u32x2_t*)(dst + 32 * mb + 8 * cc) = w;
      }
  };

  // One 64-key tile: S^T = K Q^T (two 32-key blocks), online softmax over the
  // 64 keys, O^T += V^T P^T.
  auto compute_tile = [&](const Block& blk, int t, int slot, auto mask_tag) {
    constexpr bool kMask = decltype(mask_tag)::value;
    const uint8_t* const k_lds = grp_lds + slot * C::kSlotBytes;
    const uint8_t* const v_lds = k_lds + C::kTileBytes;
    const int t0 = t * kBN;
    const int qa = pre + qrow0 + ql;  // this lane's absolute query position
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16_t{};
      const int kr = 32 * kb + ql;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8_t a = __builtin_bit_cast(
            bf16x8_t, *(const u32x4_t*)(k_lds + kr * C::kRowBytes + 16 * chunk_slot<D>(kr, 2 * ks + hh)));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, st.q[ks], s[kb], 0, 0, 0);
      }
    }
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
    bf16x8_t pb[4];
    float ls[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float sv = s[g >> 1][8 * (g & 1) + i];
        float x = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, c, neg_m));
        if constexpr (kMask) x = (sv == kNegInf) ? 0.f : x;  // also right for c == 0
        e[i] = x;
      }
      ls[g] = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
      u32x4_t w = {pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                   pack_bf16x2(e[6], e[7])};
      pb[g] = __builtin_bit_cast(bf16x8_t, w);
    }
    st.l += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    // V^T operand by transpose read: lane L of 16-lane group G points at 4
    // consecutive d of key row 16g + 8r + 4*(G/2) + (L%16)/4 at
    // d = 32 mb + 16*(G%2) + 4*(L%4), and receives the 4 keys
    // {16g + 8r + 4*(G/2) + j} at its own d = 32 mb + L%32.
    const int tg = lane >> 4, tl = lane & 15;
    const int vrow0 = 4 * (tg >> 1) + (tl >> 2);
    const int vd0 = 16 * (tg & 1) + 4 * (tl & 3);
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        s16x4_t part[2];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const int row = 16 * g + 8 * rr + vrow0;
          const int d = 32 * mb + vd0;
          const uint8_t* a = v_lds + row * C::kRowBytes + 16 * chunk_slot<D>(row, d >> 3) + 2 * (d & 7);
          part[rr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)a);
        }
        const bf16x8_t vf =
            __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
        st.o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[g], st.o[mb], 0, 0, 0);
      }
  };

  // ---------------------------------------------------------------- main loop
  bool on_hi_rows = upper || !has_lo;  // which block's rows this wave holds
  begin_rows(on_hi_rows ? bhi : blo);

  // Double-buffered slots, one barrier per iteration: the loads of the next
  // tile go to the other slot (its last readers finished before the previous
  // barrier) and land while this tile is computed.
  {
    bool oh;
    int t;
    if (my_tile(0, oh, t)) issue_tile(oh ? bhi : blo, t, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < n_iter; ++it) {
    bool oh;
    int t;
    if (it + 1 < n_iter && my_tile(it + 1, oh, t)) issue_tile(oh ? bhi : blo, t, (it + 1) & 1);
    if (my_tile(it, oh, t)) {
      const Block& blk = oh ? bhi : blo;
      if (t * kBN + kBN > blk.own_lo) cache_copy(blk, t, it & 1);
      if (oh && !on_hi_rows) {  // lower group moves from the light block to the heavy one
        store_rows(st.l);
        on_hi_rows = true;
        begin_rows(bhi);
      }
      const int t0 = t * kBN;
      const int qa0 = pre + qrow0;
      if (qrow0 < len_rows && t0 <= qa0 + 31) {  // rows present and not all above the tile
        const bool need_mask = (t0 + kBN - 1 > qa0) || (t0 + kBN > blk.key_end);
        if (need_mask)
          compute_tile(blk, t, it & 1, std::true_type{});
        else
          compute_tile(blk, t, it & 1, std::false_type{});
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
  float* mbuf = reinterpret_cast<float*>(lds) + gw * (2 + D / 2) * 64;
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
    store_rows(st.l * fa + l2 * fb);
  }
}

template <int D, bool kChunked>
hipError_t launch_d(const FwdParams& p, int num_seqs, hipStream_t stream) {
  dim3 grid(p.num_heads, num_seqs, p.grid_z);
  hipLaunchKernelGGL((prefill_fwd_kernel<D, kChunked>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

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
