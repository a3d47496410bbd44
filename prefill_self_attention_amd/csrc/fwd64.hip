// fwd64.hip -- causal varlen prefill attention with a fused bf16 KV-cache
// write, head_dim 128, for gfx950 (MI355X, CDNA4): 64 query rows per wave.
//
// Computes what prefill_fwd_kernel computes for varlen batches (see
// prefill_fwd.hip and include/prefill_attn.h): for sequence b, head h and
// token i, out = sum_{j <= i} softmax_j(scale * q_i . k_j) v_j over the keys
// of sequence b ["Prefill不是热身：大模型推理的真正瓶颈与优化核心" §3 and
// "大语言模型推理核心：Prefill与Decode原理及工程优化" §2.2: softmax(Q K^T /
// sqrt(d_k)) V; untitled page www.zwxr.cn/news/300951 §1.1: a position sees
// itself and the ones before it; "大模型 Prompt Prefill 阶段的高效 Batching 与算子排布"
// §2: requests of a flattened batch never see each other], and copies every
// token's K and V into the per-sequence [HK, len, D] cache
// ["大模型推理优化：Prefill、Decode与KV Cache的工程实践" §1.3].
//
// Why a second kernel: with 32 query rows per wave every 32x32x16 MFMA needs
// its own 1 KB operand fragment from LDS, and at the matrix cores' full rate
// four SIMDs would read 128 B per clock, which is all the LDS delivers.  Here
// a wave owns 64 query rows (two halves of 32), so each K or V fragment read
// from LDS feeds two MFMAs, and one wave runs per SIMD with 512 registers:
//
//  * O^T (64 rows x 128 columns, fp32) stays in 128 AGPRs as the MFMA
//    accumulators, and Q^T (64 rows x 128, bf16) in 64 more as the MFMA B
//    operand of the scores; scores, weights and operand slots use fixed VGPRs.
//  * The loop is software-pipelined inside the wave, in two phases per key
//    tile (gen_fwd64.py writes both, fwd64_phases.h): the score MFMAs of tile
//    j+1 run while the VALU does the softmax of tile j for rows 32..63, and
//    the PV MFMAs of tile j run while the VALU does the softmax of tile j+1
//    for rows 0..31.  The two streams are interleaved instruction by
//    instruction, so the matrix cores and the vector ALU work at the same
//    time in one wave; the next tiles' global-to-LDS loads are spread between
//    the MFMAs as well.
//  * The softmax works in the exp2 domain with a lazily moved running max,
//    as prefill_fwd.hip's does, but the common path takes a tile's weights
//    against the running max without the tile's own max (any max gives the
//    same O / l when O and l share it) and checks their sum; the first tile
//    of a run starts the running max, and a sum past its bound takes the
//    exact update out of line.  Causal masking on the diagonal tiles only;
//    the running sum adds the fp32 weights.
//  * Work split as in prefill_fwd.hip: a work-group takes the block pair
//    (z, n-1-z) of one (sequence, head); two waves (the upper group) walk the
//    heavy block's first tiles, the other two the light block (stored
//    inside the loop, during the heavy block's first score phase) and then
//    the heavy block's remaining tiles, and the heavy block's two partial
//    states are merged through LDS at the end.  Each group keeps its K and V tiles
//    in LDS rings of two (64 KB per group).
//  * Tiles that hold a block's own tokens are copied from LDS to the cache
//    with 16-byte streaming stores, every token once.
//
// Runs for varlen calls with head_dim 128 and a non-negative scale; api.hip
// sends every other case to prefill_fwd_kernel.  With an INT8 or FP8 cache the
// loop copies nothing: after the output rows each wave quantises its share of
// the work-group's own rows, read again from k and v (quant_rows.h holds the
// rule, shared with prefill_fwd_kernel, so the codes and scales are the same).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "launch.h"
#include "quant_rows.h"

namespace pa {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kRowBytes = 2 * kD;
constexpr int kBM = kQueryBlock;   // 128 query rows per block
constexpr int kBN = kKeyTile;      // 64 keys per tile
constexpr int kThreads = 256;      // 4 waves, one per SIMD
constexpr int kGroupBytes = 65536; // K ring (2 x 16 KB) + V ring (2 x 16 KB)
constexpr int kLdsBytes = 2 * kGroupBytes;
constexpr float kMInit = -1.0e30f;

// The phases keep their state in registers the compiler never allocates
// (the kernel caps its own allocation at v0-v63 and a0-a63): O^T in
// a[64:191], Q^T in a[192:255], scores, weights, operand slots and
// temporaries in v[64:255] (layout in gen_fwd64.py).  Only the generated
// phases and helpers touch them.

// Operands of the main loop (see gen_fwd64.py): wave-uniform values first.
struct Fwd64Loop {
  float c;            // |scale| * log2(e) > 0
  int32_t nit;        // iterations of the work-group (the upper group's tiles)
  int32_t nmy;        // tiles of this wave's group
  int32_t elo;        // tiles of the first run (lower group: the light block)
  int32_t jump;       // tile index minus position in the second run
  int32_t blk0, blk1; // query block of the first / second run
  int32_t r0p;        // key position of the wave's first row less 128 x block
  int32_t len;        // sequence length
  int32_t gt;         // lower group's last light position (-2: none)
  int32_t wlom1b, wwidb;  // bookkeeping window of the second run (lower group after the transition)
  uint32_t tileb;     // bytes of 64 K / V rows
  uint32_t nrec;      // bytes from the sequence's first K / V row to the end of its last
  uint32_t m0b;       // LDS address of the wave's first load block in its group
  uint32_t kbl, kbh, vbl, vbh;  // first K / V row of the sequence (this K/V head)
  uint32_t copy;      // 1: the loop copies this K/V head's rows to a bf16 cache
  uint32_t kcl, kch, vcl, vch;  // bf16 cache: the sequence's cache rows of this K/V head; INT8 / FP8 cache (the
                                // loop copies nothing): the rows' cache offset (kcl, kch), whether this head
                                // writes them (vcl) and the light block or -1 (vch), for the quantisation
  const uint16_t* qb; // first Q row of the sequence (this head)
  uint32_t kb0, kb1, kb2, kb3;  // LDS read bases of the score operand
  uint32_t vb0, vb1;            // LDS read bases of the PV operand
  uint32_t fk0, fk1, fk2, fk3, fk4, fk5, fk6, fk7;  // lane offsets of the eight loads
  int32_t vd;         // lane%32 - 4*(lane/32): diagonal mask threshold
  uint32_t cl;        // LDS lane base of the cache copy
  uint32_t crow;      // first tile row of the lane in the cache copy
  uint32_t coe, coo;  // cache byte offsets of the copy's even / odd rows
  uint32_t qo0, qo1;  // Q byte offsets of the heavy block's rows (halves 0, 1)
  uint32_t olo, ohi, onrec;  // output rows of this (sequence, head): base, bytes to the end of the last
  uint32_t oo0, oo1;  // output byte offsets of the light block's rows (halves 0, 1; + 16 lane/32)
};

// Wave-uniform values for the asm statements' SGPR operands.
__device__ __forceinline__ uint32_t sgpr_u32(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float sgpr_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}
template <class T>
__device__ __forceinline__ const T* sgpr_ptr(const T* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return reinterpret_cast<const T*>(lo | hi << 32);
}

#include "fwd64_phases.h"

// Naming v255 and a255 makes the kernel's register count cover the fixed
// registers (the compiler allocates none of them itself).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void claim_registers() { asm volatile("" ::: "v255", "a255"); }
#pragma clang diagnostic pop

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ __forceinline__ int chunk_slot(int r, int c) {
  return c ^ ((((r & 3) << 1) | ((r >> 2) & 1)) & 15);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t two = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(two, bf16x2_t));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t*)p));
}

// MFMA results are read by VALU instructions after this (accumulators of
// the last PV phase).
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n s_nop 7\n s_nop 7\n s_nop 7" ::: "memory"); }

__device__ __forceinline__ void end_interval() {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of the next tiles have landed
  __builtin_amdgcn_s_barrier();
}

// Clock stamps, in the measurement build of the library only (built with
// PA_CLOCK_STAMPS beside the product library): every wave of the varlen
// kernel records (s_memrealtime, a fixed 100 MHz counter; s_memtime, shader
// clock cycles) at its start, after the prologue, after the loop and at its
// end, in g_fwd64_stamps[8 * (4 * work-group + wave) + i]:
// i = 0..3 the real times, 4..7 the cycle counts.
#ifdef PA_CLOCK_STAMPS
constexpr bool kStamps = true;
constexpr int64_t kStampWaves = 1 << 16;
__device__ uint64_t g_fwd64_stamps[8 * kStampWaves];
#else
constexpr bool kStamps = false;
#endif
struct Stamp {
  uint64_t real, cycles;
};
__device__ __forceinline__ Stamp stamp() {
  if constexpr (kStamps) return {__builtin_amdgcn_s_memrealtime(), __builtin_amdgcn_s_memtime()};
  return {0, 0};
}

// The INT8 or FP8 cache rows of query block blk that wave `wave` writes: its
// 32 rows 32 wave .. 32 wave + 31 of the block, 16 lanes per row with 8
// values each, K and V read again from k and v (the loop has just read them,
// so they come from L2 or the Infinity Cache).  Rows past the sequence read
// its last row, so that every lane takes part in the row maximum, and store
// nothing.
template <int kCache>
__device__ __forceinline__ void quantize_block_rows(const uint16_t* kin, const uint16_t* vin, int64_t row_stride,
                                                    int8_t* kq, int8_t* vq, float* ks, float* vs,
                                                    int64_t cache_base, int blk, int len, int wave, int lane) {
  const int ch = lane & 15;
  const int r0 = blk * kBM + 32 * wave + (lane >> 4);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    qrow::u32x4_t kr[4], vr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = min(r0 + 16 * half + 4 * i, len - 1);
      kr[i] = *reinterpret_cast<const qrow::u32x4_t*>(kin + row * row_stride + 8 * ch);
      vr[i] = *reinterpret_cast<const qrow::u32x4_t*>(vin + row * row_stride + 8 * ch);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = r0 + 16 * half + 4 * i;
      const float ka = qrow::group_max<16>(qrow::absmax8(kr[i]));
      const float va = qrow::group_max<16>(qrow::absmax8(vr[i]));
      if (row < len) {
        const int64_t dst = cache_base + (int64_t)row * kD + 8 * ch;
        if constexpr (kCache == qrow::kCacheInt8) {
          __builtin_nontemporal_store(qrow::quantize8(kr[i], ka), (qrow::u32x2_t*)(kq + dst));
          __builtin_nontemporal_store(qrow::quantize8(vr[i], va), (qrow::u32x2_t*)(vq + dst));
        } else {
          __builtin_nontemporal_store(qrow::quantize_fp8(kr[i], ka), (qrow::u32x2_t*)(kq + dst));
          __builtin_nontemporal_store(qrow::quantize_fp8(vr[i], va), (qrow::u32x2_t*)(vq + dst));
        }
        if (ch == 0) {
          ks[cache_base / kD + row] = kCache == qrow::kCacheInt8 ? qrow::int8_scale(ka) : qrow::fp8_scale(ka);
          vs[cache_base / kD + row] = kCache == qrow::kCacheInt8 ? qrow::int8_scale(va) : qrow::fp8_scale(va);
        }
      }
    }
  }
}

// kSplit = false: varlen (keys from k, v; block pairs).  kSplit = true:
// split-KV items of a chunked call (keys from the cache, which already holds
// the call's new rows; each group of two waves takes its own unit (item,
// head) and writes a partial result when the item's block has several
// segments).  kCache: the varlen cache format (bf16, INT8 or FP8).
template <bool kSplit, int kCache>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_fwd64_kernel(FwdParams p) {
  static_assert(!kSplit || kCache == qrow::kCacheBf16, "the split-KV items write no cache");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];
  const Stamp st0 = stamp();
  claim_registers();
  const int tid = __builtin_amdgcn_workitem_id_x();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int ql = lane & 31;
  const int hl = lane >> 5;
  const bool upper = wave < 2;
  const int wsub = wave & 1;
  const int group = upper ? 0 : 1;
  const int64_t H = p.num_heads;
  const int64_t HK = p.num_kv_heads;
  int h, b, z, seq_start, len;
  int qb_hi, e_lo, n_up, n_lo, n_my, pfx = 0, seg = 0, nseg = 1, seg_t0 = 0;
  bool has_lo, transition;
  if constexpr (kSplit) {
    // units u = item * H + head; work-group w takes units 2 w (waves 0, 1)
    // and 2 w + 1 (waves 2, 3): with H even, one item of two heads, which
    // cover the same key tiles
    const int64_t units = (int64_t)p.hdr[0] * H;
    const int64_t u0 = 2 * (int64_t)__builtin_amdgcn_workgroup_id_x();
    if (u0 >= units) return;  // every wave returns
    const int64_t um = u0 + group, uo = u0 + 1 - group;
    const bool mine_ok = um < units;
    auto seg_tiles = [&](int64_t u, int& bb, int& qb, int& s, int& ns, int& t0) {
      const int4 it = p.items[u / H];
      bb = it.x;
      qb = it.y;
      s = it.z;
      ns = it.w;
      const int st = p.cu[bb], ln = p.cu[bb + 1] - st, pre = p.prefix[bb];
      const int nt = (min(pre + min((qb + 1) * kBM, ln), p.cap) + kBN - 1) / kBN;  // within the capacity
      t0 = s * nt / ns;
      return (s + 1) * nt / ns - t0;
    };
    int bo, qbo, so, nso, t0o;
    const int n_other = uo < units ? seg_tiles(uo, bo, qbo, so, nso, t0o) : 0;
    // an idle group (no second unit) takes the first unit's addresses and no tiles
    const int64_t ua = mine_ok ? um : uo;
    int qb;
    n_my = seg_tiles(ua, b, qb, seg, nseg, seg_t0);
    if (!mine_ok) n_my = 0;
    h = (int)(ua % H);
    seq_start = p.cu[b];
    len = p.cu[b + 1] - seq_start;
    pfx = p.prefix[b];
    z = qb;
    qb_hi = qb;
    has_lo = false;
    e_lo = 0;
    n_up = max(n_my, n_other);  // iterations of the work-group
    n_lo = 0;
    transition = false;
  } else {
    // Work-group order.  Units (sequence, head) are spread over the 8 XCDs
    // (the dispatcher places work-group i of a 1-D grid on XCD i % 8), and a
    // unit's block pairs z follow one another in its XCD's dispatch stream,
    // so the pairs that read the same head's K/V run at the same time and
    // share that XCD's L2.  With H a multiple of 8, XCD x holds heads
    // [x H/8, (x+1) H/8) of every sequence (grouped K/V heads stay together).
    const int wg = __builtin_amdgcn_workgroup_id_x();
    const int xcd = wg & 7, s = wg >> 3;
    const int u = s / p.grid_z;
    z = s - u * p.grid_z;
    if (p.num_heads % 8 == 0) {
      const int hx = p.num_heads / 8;
      b = u / hx;
      h = xcd * hx + (u - b * hx);
    } else {
      const int unit = u * 8 + xcd;
      b = unit / p.num_heads;
      h = unit - b * p.num_heads;
    }
    if (b >= p.num_seqs) return;  // padding of the last units (every wave returns)
    seq_start = p.cu[b];
    len = p.cu[b + 1] - seq_start;
    const int nqb = (len + kBM - 1) / kBM;
    qb_hi = nqb - 1 - z;
    if (z > qb_hi) return;  // no block pair left for this work-group (every wave returns)
    has_lo = z < qb_hi;
    auto ntiles_of = [=](int qb) { return (min((qb + 1) * kBM, len) + kBN - 1) / kBN; };
    e_lo = has_lo ? ntiles_of(z) : 0;
    const int e_hi = ntiles_of(qb_hi);
    n_up = (e_lo + e_hi + 1) / 2;
    n_lo = e_lo + e_hi - n_up;
    // the group's tile sequence: upper: heavy block tiles 0 .. n_up-1; lower:
    // light block tiles 0 .. e_lo-1, then heavy block tiles n_up .. e_hi-1
    n_my = upper ? n_up : n_lo;
    transition = !upper && has_lo && n_lo > e_lo;
  }

  const int hk = h / (int)(H / HK);
  const bool writes_cache = !kSplit && h == hk * (int)(H / HK);
  // elements between consecutive keys: tokens of k, v (varlen) or rows of
  // the cache (split: [B, HK, cap, D])
  const int64_t row_stride = kSplit ? (int64_t)kD : HK * kD;
  const uint16_t* kin = kSplit ? p.kc + ((int64_t)b * HK + hk) * p.cap * kD
                               : p.k + (int64_t)seq_start * row_stride + (int64_t)hk * kD;
  const uint16_t* vin = kSplit ? p.vc + ((int64_t)b * HK + hk) * p.cap * kD
                               : p.v + (int64_t)seq_start * row_stride + (int64_t)hk * kD;
  const int64_t cache_base = (int64_t)seq_start * HK * kD + (int64_t)hk * len * kD;
  const uint32_t lds0 = lds_addr(lds);
  const uint32_t gbase = lds0 + group * kGroupBytes;
  const uint32_t rs = (uint32_t)(row_stride * 2);
  const uint32_t rsq = (uint32_t)(H * kD * 2);

  Fwd64Loop L;
  L.c = p.scale_log2;
  L.nit = n_up;
  L.nmy = n_my;
  L.elo = kSplit ? 0 : upper ? n_my : e_lo;
  L.jump = kSplit ? seg_t0 : upper ? 0 : n_up - e_lo;
  L.blk0 = (upper || !has_lo) ? qb_hi : z;
  L.blk1 = qb_hi;
  L.r0p = pfx + 64 * wsub;
  L.len = len;
  L.gt = transition ? e_lo - 1 : -100;  // -100: never (g >= -1 meets none of gt - 1, gt, gt + 1)
  L.tileb = (uint32_t)kBN * rs;
  // keys [0, prefix + len), within the cache row's capacity (split)
  L.nrec = (uint32_t)((kSplit ? min(pfx + len, p.cap) : len) - 1) * rs + kRowBytes;
  L.m0b = gbase + 1024u * wsub;
  L.kbl = (uint32_t)(uintptr_t)kin;
  L.kbh = (uint32_t)((uintptr_t)kin >> 32);
  L.vbl = (uint32_t)(uintptr_t)vin;
  L.vbh = (uint32_t)((uintptr_t)vin >> 32);
  L.copy = writes_cache && kCache == qrow::kCacheBf16 ? 1u : 0u;
  uint16_t* kc = kSplit ? p.kc : p.kc + cache_base;  // the copy (varlen only) writes these
  uint16_t* vc = kSplit ? p.vc : p.vc + cache_base;
  if constexpr (kCache == qrow::kCacheBf16) {
    L.kcl = (uint32_t)(uintptr_t)kc;
    L.kch = (uint32_t)((uintptr_t)kc >> 32);
    L.vcl = (uint32_t)(uintptr_t)vc;
    L.vch = (uint32_t)((uintptr_t)vc >> 32);
  } else {
    // the loop copies nothing (copy = 0), so these carry what the
    // quantisation after the loop needs: the rows' cache offset, whether
    // this head writes them, and the light block (-1: none).  As operands of
    // the loop they are held across it at no cost in registers.
    L.kcl = (uint32_t)cache_base;
    L.kch = (uint32_t)((uint64_t)cache_base >> 32);
    L.vcl = writes_cache ? 1u : 0u;
    L.vch = has_lo ? (uint32_t)z : ~0u;
  }
  L.qb = p.q + ((int64_t)seq_start * H + h) * kD;
  L.kb0 = gbase + ql * kRowBytes + 16 * chunk_slot(ql, 0 + hl);
  L.kb1 = gbase + ql * kRowBytes + 16 * chunk_slot(ql, 2 + hl);
  L.kb2 = gbase + ql * kRowBytes + 16 * chunk_slot(ql, 4 + hl);
  L.kb3 = gbase + ql * kRowBytes + 16 * chunk_slot(ql, 6 + hl);
  {
    const int tg = lane >> 4, tl = lane & 15;
    const int vrow0 = 4 * (tg >> 1) + (tl >> 2);
    const int vd0 = 16 * (tg & 1) + 4 * (tl & 3);
    L.vb0 = gbase + vrow0 * kRowBytes + 16 * chunk_slot(vrow0, (vd0 >> 3) & 15) + 2 * (vd0 & 7);
    const int d1 = 32 + vd0;
    L.vb1 = gbase + vrow0 * kRowBytes + 16 * chunk_slot(vrow0, (d1 >> 3) & 15) + 2 * (d1 & 7);
  }
  // Loads: instruction i of a tile fills LDS block 2 i + wsub, rows
  // 8 i + r0 with r0 = 4 wsub + lane/16; lane slot lane%16 takes source
  // chunk chunk_slot(r0, slot) (the swizzle depends on the row mod 8 only).
  const int r0 = 4 * wsub + (lane >> 4);
  const uint32_t lane_chunk = 16u * (uint32_t)chunk_slot(r0, lane & 15);
  uint32_t fk[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) fk[i] = (uint32_t)(8 * i + r0) * rs + lane_chunk;
  // the loop's odd loads carry an instruction offset of 2048 bytes (which
  // moves the LDS address too); 8 rows of at least 256 bytes precede them
  L.fk0 = fk[0]; L.fk1 = fk[1] - 2048u; L.fk2 = fk[2]; L.fk3 = fk[3] - 2048u;
  L.fk4 = fk[4]; L.fk5 = fk[5] - 2048u; L.fk6 = fk[6]; L.fk7 = fk[7] - 2048u;
  L.vd = ql - 4 * hl;
  // cache copy: the wave's rows 32 wsub + 4 i + lane/16 of a tile
  {
    const int crow = 32 * wsub + (lane >> 4);
    const int slot = lane & 15;
    L.cl = gbase + crow * kRowBytes + 16 * slot;
    L.crow = crow;
    L.coe = crow * kRowBytes + 16 * chunk_slot(crow, slot);
    L.coo = crow * kRowBytes + 16 * chunk_slot(crow + 4, slot);
  }
  {
    const int first = qb_hi * kBM + 64 * wsub;
    L.qo0 = (uint32_t)min(first + ql, len - 1) * rsq + 16u * hl;
    L.qo1 = (uint32_t)min(first + 32 + ql, len - 1) * rsq + 16u * hl;
  }
  {
    const uint16_t* ob = p.out + ((int64_t)seq_start * H + h) * kD;
    L.olo = (uint32_t)(uintptr_t)ob;
    L.ohi = (uint32_t)((uintptr_t)ob >> 32);
    L.onrec = (uint32_t)(len - 1) * rsq + kRowBytes;
    const int first = z * kBM + 64 * wsub;  // the light block's rows (the store runs rows past len out of range)
    L.oo0 = (uint32_t)(first + ql) * rsq + 16u * hl;
    L.oo1 = (uint32_t)(first + 32 + ql) * rsq + 16u * hl;
  }

  // ---------------------------------------------------------------- prologue
  // Q of the first block's rows (rows past the sequence read its last row);
  // K of the group's first tile into K slot 0
  {
    const int first = (upper ? qb_hi : (has_lo ? z : qb_hi)) * kBM + 64 * wsub;
    fwd64_load_q(L.qb, (uint32_t)min(first + ql, len - 1) * rsq + 16u * hl,
                 (uint32_t)min(first + 32 + ql, len - 1) * rsq + 16u * hl);
  }
  fwd64_o_zero();
  if (n_my > 0) {
    const int t0 = kSplit ? seg_t0 : upper || e_lo > 0 ? 0 : n_up;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kin + (int64_t)t0 * kBN * row_stride), (short)0, (int)(L.nrec - (uint32_t)t0 * L.tileb), 0x00020000);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc,
          (__attribute__((address_space(3))) void*)(lds + group * kGroupBytes + 1024 * (2 * i + wsub)), 16, fk[i], 0, 0, 0);
  }
  end_interval();
  const Stamp st1 = stamp();

  // ---------------------------------------------------------------- loop
  float m0 = kMInit, l0 = 0.f, m1 = kMInit, l1 = 0.f;   // halves 0 and 1
  float m0n = kMInit, l0n = 0.f, l1n = 0.f;              // the light block's state at the transition

  // store one block's finished rows (this wave's 64), column blocks
  // [D0, D1) of 32: block i of O^T from get(i), divided by the row sums
  // (per-lane halves la0, la1).  Buffer stores through a descriptor that
  // ends at the sequence's last row drop the rows past it.
  const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.out + ((int64_t)seq_start * H + h) * kD), (short)0, (int)((uint32_t)(len - 1) * rsq + kRowBytes),
      0x00020000);
  auto store_cols = [&](int qb, float la0, float la1, auto&& get, auto d0_tag, auto d1_tag) __attribute__((always_inline)) {
    constexpr int D0 = decltype(d0_tag)::value, D1 = decltype(d1_tag)::value;
    const int first = qb * kBM + 64 * wsub;
    static_for<0, 2>([&](auto qh_tag) __attribute__((always_inline)) {
      constexpr int qh = decltype(qh_tag)::value;
      const float lsum = qh == 0 ? la0 : la1;
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
      const float inv = __builtin_amdgcn_rcpf(__uint_as_float(sw[0]) + __uint_as_float(sw[1]));
      const uint32_t rowoff = (uint32_t)(first + 32 * qh + ql) * rsq;
      static_for<D0, D1>([&](auto db_tag) __attribute__((always_inline)) {
        constexpr int db = decltype(db_tag)::value;
        const f32x16_t o = get(std::integral_constant<int, 4 * qh + db>{});
#pragma unroll
        for (int cp = 0; cp < 2; ++cp) {
          // lane (row, hl) holds d = 32 db + 8 cc + 4 hl + [0, 4).  One
          // permlane32_swap per register pair moves the upper lanes' pieces
          // of column group 2 cp and the lower lanes' of 2 cp + 1 across, so
          // every lane then holds 8 consecutive d: 2 cp + hl's
          const int ca = 2 * cp, cb = 2 * cp + 1;
          const uint32_t a0 = pack_bf16x2(o[4 * ca + 0] * inv, o[4 * ca + 1] * inv);
          const uint32_t a1 = pack_bf16x2(o[4 * ca + 2] * inv, o[4 * ca + 3] * inv);
          const uint32_t b0 = pack_bf16x2(o[4 * cb + 0] * inv, o[4 * cb + 1] * inv);
          const uint32_t b1 = pack_bf16x2(o[4 * cb + 2] * inv, o[4 * cb + 3] * inv);
          const auto x0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
          const auto x1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
          const u32x4_t w = {x0[0], x1[0], x0[1], x1[1]};
          __builtin_amdgcn_raw_buffer_store_b128(w, orsrc, rowoff + 2 * (32 * db + 8 * (ca + hl)), 0, 0);
        }
      });
    });
  };
  auto store_rows = [&](int qb, float la0, float la1, auto&& get) __attribute__((always_inline)) {
    store_cols(qb, la0, la1, get, std::integral_constant<int, 0>{}, std::integral_constant<int, 4>{});
  };
  auto o_get = [](auto i_tag) __attribute__((always_inline)) { return fwd64_o_read<decltype(i_tag)::value>(); };

  // Iterations h whose bookkeeping is the common case (see book_fast in
  // gen_fwd64.py) for a run of positions [x0, x1) holding tiles x + off of
  // block blk: h - 1 in the run, h + 2 before its end, T[h + 1] wholly
  // visible to the wave (below (R0 + 1) / 64, see kind_of) and, when the
  // wave copies to the cache, before the block's own tiles.  Encoded as
  // (lo - 1, hi - lo), or an empty window.
  auto window = [&](int x0, int x1, int off, int blk, int32_t& lom1, int32_t& wid) {
    int hi = min(x1 - 3, ((kBM * blk + L.r0p + 1) >> 6) - off - 2);
    if (L.copy) hi = min(hi, 2 * blk - off - 2);
    const int lo = x0 + 1;
    lom1 = hi < lo ? INT32_MIN : lo - 1;
    wid = hi < lo ? 0 : hi - lo;
  };
  int32_t wlom1, wwid;
  if (kSplit) window(0, n_my, seg_t0, qb_hi, wlom1, wwid);
  else if (upper) window(0, n_my, 0, qb_hi, wlom1, wwid);
  else if (has_lo) window(0, e_lo, 0, z, wlom1, wwid);
  else window(0, n_my, L.jump, qb_hi, wlom1, wwid);
  L.wlom1b = wlom1;
  L.wwidb = wwid;
  if (transition) window(e_lo, n_my, L.jump, qb_hi, L.wlom1b, L.wwidb);
  // one pass over the iterations: the lower group's light block (when a
  // heavy part follows it) is stored, and O restarted, inside the loop
  wlom1 = __builtin_amdgcn_readfirstlane(wlom1);  // wave-uniform: in-out SGPR operands
  wwid = __builtin_amdgcn_readfirstlane(wwid);
  fwd64_loop(L, m0, l0, m1, l1, m0n, l0n, l1n, wlom1, wwid);
  const Stamp st2 = stamp();

  if constexpr (kSplit) {
    mfma_drain();
    if (n_my == 0) return;
    if (nseg == 1) {
      store_rows(qb_hi, l0, l1, o_get);
      return;
    }
    // the rows' partial result over this segment's keys: O / l in fp32 and
    // m + log2(l) (log2 of the sum of 2^(s c) over those keys; -inf when a
    // row sees none of them), at slot (token, head, segment)
    static_for<0, 2>([&](auto qh_tag) __attribute__((always_inline)) {
      constexpr int qh = decltype(qh_tag)::value;
      const float lp = qh == 0 ? l0 : l1;
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lp), __float_as_uint(lp), false, false);
      const float l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      const bool any = l > 0.f;
      const float inv = any ? __builtin_amdgcn_rcpf(l) : 0.f;
      const int row = qb_hi * kBM + 64 * wsub + 32 * qh + ql;
      const int64_t slot = ((int64_t)(seq_start + row) * H + h) * p.max_segs + seg;
      float* dst = p.part_o + slot * kD + 4 * hl;
      static_for<0, 4>([&](auto db_tag) __attribute__((always_inline)) {
        constexpr int db = decltype(db_tag)::value;
        const f32x16_t o = fwd64_o_read<4 * qh + db>();
        if (row < len) {
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            const f32x4_t w = {o[4 * cc] * inv, o[4 * cc + 1] * inv, o[4 * cc + 2] * inv, o[4 * cc + 3] * inv};
            *reinterpret_cast<f32x4_t*>(dst + 32 * db + 8 * cc) = w;
          }
        }
      });
      if (row < len && hl == 0)
        p.part_lse[slot] = any ? (qh == 0 ? m0 : m1) + __builtin_amdgcn_logf(l) : -__builtin_huge_valf();
    });
    return;
  }

  // ---------------------------------------------------------------- merge
  // lower group holds the heavy block's remaining tiles (n_lo > e_lo) or
  // only the light block; the upper group the heavy block's first tiles
  const bool merge = n_lo > e_lo;
  // the quantised cache rows of the work-group's blocks (the heavy block, and
  // the light one when it has its own), after the output rows
  auto quantize_own = [&]() __attribute__((always_inline)) {
    if constexpr (kCache != qrow::kCacheBf16) {
      if (sgpr_u32(L.vcl) != 0) {
        // Everything comes from the loop's own operands (held across it
        // anyway) and from the kernel arguments read again here, through a
        // pointer the compiler cannot trace back to the prologue: nothing more
        // stays in scalar registers across the loop.
        const FwdParams* kp = (const FwdParams*)(uintptr_t)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(kp));
        const auto u64 = [](uint32_t lo, uint32_t hi) { return (uint64_t)sgpr_u32(hi) << 32 | sgpr_u32(lo); };
        const uint16_t* kq_in = reinterpret_cast<const uint16_t*>(u64(L.kbl, L.kbh));
        const uint16_t* vq_in = reinterpret_cast<const uint16_t*>(u64(L.vbl, L.vbh));
        const int64_t stride = sgpr_u32(L.tileb) / (2 * kBN);  // elements between keys
        const int64_t cbase = (int64_t)u64(L.kcl, L.kch);
        const int n = (int)sgpr_u32(L.len);
        const int light = (int)sgpr_u32(L.vch);
        quantize_block_rows<kCache>(kq_in, vq_in, stride, kp->kq, kp->vq, kp->ks, kp->vs, cbase, (int)sgpr_u32(L.blk1),
                                    n, wave, lane);
        if (light >= 0)
          quantize_block_rows<kCache>(kq_in, vq_in, stride, kp->kq, kp->vq, kp->ks, kp->vs, cbase, light, n, wave,
                                      lane);
      }
    }
  };
  mfma_drain();
  if (!merge) {
    if (upper) store_rows(qb_hi, l0, l1, o_get);
    else if (n_lo > 0) store_rows(z, l0, l1, o_get);
    quantize_own();
    return;
  }
  // the two waves holding the same rows (upper and lower, same wsub) each
  // finish half of the columns: the upper wave columns 0-63, the lower
  // 64-127.  Each passes its running maxima, row sums and the O blocks of
  // the other half through LDS (region of 4 + 64 floats per lane).
  constexpr int kRegion = 17 * 64;  // float4 per lane: (m0, l0, m1, l1), then 16 of O
  f32x4_t* mine = reinterpret_cast<f32x4_t*>(lds) + (2 * wsub + (upper ? 0 : 1)) * kRegion;
  const f32x4_t* theirs = reinterpret_cast<const f32x4_t*>(lds) + (2 * wsub + (upper ? 1 : 0)) * kRegion;
  mine[lane] = f32x4_t{m0, l0, m1, l1};
  // block i = 4 qh + db of O^T travels in slot 2 qh + (db & 1)
  static_for<0, 8>([&](auto i_tag) __attribute__((always_inline)) {
    constexpr int i = decltype(i_tag)::value;
    constexpr int db = i & 3, slot = 2 * (i >> 2) + (db & 1);
    if (upper ? db >= 2 : db < 2) {
      const f32x16_t o = fwd64_o_read<i>();
#pragma unroll
      for (int r = 0; r < 4; ++r)
        mine[(1 + 4 * slot + r) * 64 + lane] = f32x4_t{o[4 * r], o[4 * r + 1], o[4 * r + 2], o[4 * r + 3]};
    }
  });
  __syncthreads();
  const f32x4_t ml = theirs[lane];
  const float pm0 = ml[0], pl0 = ml[1], pm1 = ml[2], pl1 = ml[3];
  const float mx0 = fmaxf(m0, pm0), mx1 = fmaxf(m1, pm1);
  const float fa0 = __builtin_amdgcn_exp2f(m0 - mx0), fb0 = __builtin_amdgcn_exp2f(pm0 - mx0);
  const float fa1 = __builtin_amdgcn_exp2f(m1 - mx1), fb1 = __builtin_amdgcn_exp2f(pm1 - mx1);
  auto merged = [&](auto i_tag) __attribute__((always_inline)) {
    constexpr int i = decltype(i_tag)::value;
    constexpr int db = i & 3, slot = 2 * (i >> 2) + (db & 1);
    const float fa = i < 4 ? fa0 : fa1, fb = i < 4 ? fb0 : fb1;
    f32x16_t o = fwd64_o_read<i>();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f32x4_t x = theirs[(1 + 4 * slot + r) * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[4 * r + e] = o[4 * r + e] * fa + x[e] * fb;
    }
    return o;
  };
  const float la0 = l0 * fa0 + pl0 * fb0, la1 = l1 * fa1 + pl1 * fb1;
  if (upper)
    store_cols(qb_hi, la0, la1, merged, std::integral_constant<int, 0>{}, std::integral_constant<int, 2>{});
  else
    store_cols(qb_hi, la0, la1, merged, std::integral_constant<int, 2>{}, std::integral_constant<int, 4>{});
  quantize_own();
#ifdef PA_CLOCK_STAMPS
  const Stamp st3 = stamp();
  const int64_t w = 4 * (int64_t)__builtin_amdgcn_workgroup_id_x() + wave;
  if (lane < 8 && w < kStampWaves) {
    const Stamp& x = (lane & 3) == 0 ? st0 : (lane & 3) == 1 ? st1 : (lane & 3) == 2 ? st2 : st3;
    g_fwd64_stamps[8 * w + lane] = lane < 4 ? x.real : x.cycles;
  }
#else
  (void)st0;
  (void)st1;
  (void)st2;
#endif
}

}  // namespace

#ifdef PA_CLOCK_STAMPS
// Copies the stamps of the last varlen launch (8 uint64 per wave, waves
// 4 w + i of work-group w) to host memory; n_waves <= 65536.
extern "C" int pa_fwd64_clock_stamps(uint64_t* host, int64_t n_waves) {
  if (!host || n_waves <= 0 || n_waves > kStampWaves) return (int)hipErrorInvalidValue;
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_fwd64_stamps), 8 * sizeof(uint64_t) * n_waves);
}
#endif

bool fwd64_supported(int head_dim, bool chunked, float scale, int max_seqlen, int num_heads, int num_kv_heads) {
  // lane offsets within a sequence are 32-bit: rows of q and of k / v
  const int64_t row_bytes = (int64_t)2 * kD * (num_heads > num_kv_heads ? num_heads : num_kv_heads);
  return head_dim == 128 && !chunked && scale >= 0.f && (int64_t)max_seqlen * row_bytes < ((int64_t)1 << 31);
}

hipError_t launch_prefill_fwd64(const FwdParams& p, int num_seqs, int cache_format, hipStream_t stream) {
  FwdParams q = p;
  q.num_seqs = num_seqs;
  // units per XCD (8 XCDs), each with grid_z block pairs
  const int64_t per_xcd = ((int64_t)p.num_heads * num_seqs + 7) / 8;
  const int64_t grid = 8 * per_xcd * p.grid_z;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  switch (cache_format) {
    case qrow::kCacheBf16:
      hipLaunchKernelGGL((prefill_fwd64_kernel<false, qrow::kCacheBf16>), dim3((unsigned)grid), dim3(kThreads), 0,
                         stream, q);
      break;
    case qrow::kCacheInt8:
      hipLaunchKernelGGL((prefill_fwd64_kernel<false, qrow::kCacheInt8>), dim3((unsigned)grid), dim3(kThreads), 0,
                         stream, q);
      break;
    case qrow::kCacheFp8:
      hipLaunchKernelGGL((prefill_fwd64_kernel<false, qrow::kCacheFp8>), dim3((unsigned)grid), dim3(kThreads), 0,
                         stream, q);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool fwd64_split_supported(int head_dim, float scale, int max_seqlen, int num_heads, int cap) {
  // 32-bit offsets: rows of q and out (up to 127 past the last one), rows of
  // one (sequence, K/V head) of the cache
  const int64_t q_row = (int64_t)2 * kD * num_heads;
  return head_dim == 128 && scale >= 0.f && ((int64_t)max_seqlen + kBM) * q_row < ((int64_t)1 << 31) &&
         (int64_t)cap * kRowBytes < ((int64_t)1 << 31);
}

hipError_t launch_prefill_fwd64_split(const FwdParams& p, int64_t max_items, hipStream_t stream) {
  const int64_t grid = (max_items * p.num_heads + 1) / 2;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_fwd64_kernel<true, qrow::kCacheBf16>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}


}  // namespace pa
