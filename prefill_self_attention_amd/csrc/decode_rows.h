// decode_rows.h -- the length-1 rows of the split-KV chunked call, one unit
// at a time; included by prefill_fwd.hip (the mixed launch runs these units
// beside the attention items) and splitkv.hip (the rows' own launch).
//
// A length-1 row is one query against its cached prefix plus itself
// (untitled page www.zwxr.cn/news/300951 §3.3: decode attention reads every
// cached position of its row): per key 4 D flops against 4 D bytes of K and
// V, so a unit is bound by HBM, not by the matrix cores.  It runs on the
// vector ALUs straight from 16-byte loads: lane l of a wave owns the 8
// elements d = 8 (l % LPK) + [0, 8) of key slot l / LPK (LPK = D / 8 lanes per
// key, KPI = 64 / LPK keys per step); a lane's part of a score is four bf16
// pair dot products (v_dot2_f32_bf16, q kept as bf16 pairs), the score a DPP
// butterfly over the key's LPK lanes, and every key slot keeps its own
// online-softmax state, combined across slots and then across the W waves at
// the end of the unit.  A unit is (decode item, GC query heads of one K/V
// head): each K/V row loaded serves all GC heads.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace pa {
namespace dec {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kRescale = 8.0f;  // lazy rescale headroom, log2 units
constexpr float kMInit = -1.0e30f;

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t two = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(two, bf16x2_t));
}

template <int kCtrl>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}

// Sum over aligned groups of LPK (4, 8 or 16) lanes, result in every lane.
template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_f<0xB1>(x);                            // quad_perm [1,0,3,2]
  x += dpp_f<0x4E>(x);                            // quad_perm [2,3,0,1]
  if constexpr (LPK >= 8) x += dpp_f<0x141>(x);   // row_half_mirror
  if constexpr (LPK >= 16) x += dpp_f<0x140>(x);  // row_mirror
  return x;
}

__device__ __forceinline__ void bf16x8_to_f32(const uint4 w, float (&f)[8]) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(u[i] << 16);
    f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ float lane_read(float x, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(4 * src, __float_as_int(x)));
}

// Floats of LDS a unit of W waves needs for its reduction.
template <int D, int GC, int W>
constexpr int red_floats() { return W * GC * (2 + D); }

// Unit g of the decode list (item it = {sequence, segment, segments}, query
// heads GC * (g % (H / GC)) onward), run by the first W waves of the
// work-group; red is LDS of
// red_floats<D, GC, W>() floats.  Unless `next` is null, thread 0 also
// takes the next value of counter *next (issued first, so its latency hides
// behind the unit) and leaves it in *taken (LDS) before the final
// work-group barrier, after which every wave may read it and red may be
// reused.
template <int D, int GC, bool kPaged, int W>
__device__ __forceinline__ void decode_unit(const FwdParams& p, int64_t g, int4 it, float* red,
                                            unsigned long long* next, unsigned long long* taken) {
  constexpr int LPK = D / 8, KPI = 64 / LPK;
  // key steps whose loads are issued together (two such groups in flight):
  // as many as the registers left beside GC heads' q and O allow.  Every
  // cached K/V row is read once: streaming (non-temporal) loads.
  constexpr int kUnroll = W <= 4 || GC <= 2 ? 8 : GC == 4 ? 4 : 2;
  float (*const rd)[GC][2 + D] = reinterpret_cast<float (*)[GC][2 + D]>(red);
  const int tid = __builtin_amdgcn_workitem_id_x();
  // wave-uniform in a scalar register: the key loop below is then a scalar loop
  const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kslot = lane / LPK, dch = lane % LPK;
  const int H = p.num_heads, HK = p.num_kv_heads, G = H / HK;
  const int units = H / GC;
  const float c = p.scale_log2;
  const float neg_inf = -__builtin_huge_valf();

  unsigned long long nxt = 0;
  if (next && tid == 0) nxt = atomicAdd(next, 1ull);
  const int h0 = (int)(g % units) * GC;
  const int hk = h0 / G;
  const int b = it.x, s = it.y, ns = it.z;
  const int tok = p.cu[b];
  const int pre = p.prefix[b];
  const int ntiles = (pre + 1 + kKeyTile - 1) / kKeyTile;
  const int k0 = s * ntiles / ns * kKeyTile;
  const int k1 = min((s + 1) * ntiles / ns * kKeyTile, pre + 1);  // keys [k0, k1) of this segment
  const int per = ((k1 - k0 + W - 1) / W + KPI - 1) / KPI * KPI;
  const int w0 = k0 + wave * per;
  const int w1 = min(w0 + per, k1);            // this wave's keys
  const int64_t crow = ((int64_t)b * HK + hk) * p.cap;
  const uint16_t* __restrict__ kc = p.kc + crow * D;  // this (sequence, K/V head)'s cache
  const uint16_t* __restrict__ vc = p.vc + crow * D;
  const uint16_t* kn = p.k + ((int64_t)tok * HK + hk) * D + 8 * dch;  // the row's own key
  const uint16_t* vn = p.v + ((int64_t)tok * HK + hk) * D + 8 * dch;
  const int wc = min(w1, pre);  // the wave's cached keys are [w0, wc); key pre comes from k, v
  // paged cache: block bt_row[j / 16] of [num_blocks, HK, 16, D] holds position j
  const int32_t* __restrict__ bt_row = kPaged ? p.block_table + (int64_t)b * p.bt_stride : nullptr;
  const int last_sb = wc > w0 ? (wc - 1) / KPI * KPI : w0;  // last step's first key
  bf16x2_t qp[GC][4];  // q as bf16 pairs: the dot products run on v_dot2_f32_bf16
  float o[GC][8], m[GC], l[GC];
#pragma unroll
  for (int gi = 0; gi < GC; ++gi) {
    uint4 w = *(const uint4*)(p.q + ((int64_t)tok * H + h0 + gi) * D + 8 * dch);
    if (p.neg_q) {
      w.x ^= 0x80008000u;
      w.y ^= 0x80008000u;
      w.z ^= 0x80008000u;
      w.w ^= 0x80008000u;
    }
    qp[gi][0] = __builtin_bit_cast(bf16x2_t, w.x);
    qp[gi][1] = __builtin_bit_cast(bf16x2_t, w.y);
    qp[gi][2] = __builtin_bit_cast(bf16x2_t, w.z);
    qp[gi][3] = __builtin_bit_cast(bf16x2_t, w.w);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[gi][i] = 0.f;
    m[gi] = kMInit;
    l[gi] = 0.f;
  }

  // cached keys kb + u KPI + kslot of a group of kUnroll steps; positions
  // past the wave's last cached key load that key again (and are masked)
  // paged cache: a step's KPI keys (KPI divides 16, steps start at
  // multiples of KPI) lie in one block, one scalar block id per step; the
  // ids of a group are fetched a group ahead of its loads
  auto fetch = [&](int kb, int (&ids)[kUnroll]) __attribute__((always_inline)) {
    if constexpr (kPaged) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) ids[u] = bt_row[min(kb + u * KPI, last_sb) / kPageRows];
    }
  };
  auto load = [&](int kb, uint4 (&kr)[kUnroll], uint4 (&vr)[kUnroll], const int (&ids)[kUnroll])
      __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if constexpr (kPaged) {
        const int sb = min(kb + u * KPI, last_sb);
        const int kq = min(sb + kslot, wc - 1);
        const int64_t base = (((int64_t)ids[u] * HK + hk) * kPageRows) * D;
        const uint32_t off = (uint32_t)(kq % kPageRows) * D + 8 * dch;
        kr[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4_t*)(p.kc + base + off)));
        vr[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4_t*)(p.vc + base + off)));
      } else {
        const uint32_t off = (uint32_t)min(kb + u * KPI + kslot, wc - 1) * D + 8 * dch;
        kr[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4_t*)(kc + off)));
        vr[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4_t*)(vc + off)));
      }
    }
  };
  auto consume_one = [&](bool ok, const uint4 kr, const uint4 vr) __attribute__((always_inline)) {
    float vf[8];
    bf16x8_to_f32(vr, vf);
    const bf16x2_t k0 = __builtin_bit_cast(bf16x2_t, kr.x), k1 = __builtin_bit_cast(bf16x2_t, kr.y);
    const bf16x2_t k2 = __builtin_bit_cast(bf16x2_t, kr.z), k3 = __builtin_bit_cast(bf16x2_t, kr.w);
#pragma unroll
    for (int gi = 0; gi < GC; ++gi) {
      // bf16 products are exact in fp32; two chains of two pairs each
      float d0 = __builtin_amdgcn_fdot2_f32_bf16(qp[gi][0], k0, 0.f, false);
      float d1 = __builtin_amdgcn_fdot2_f32_bf16(qp[gi][1], k1, 0.f, false);
      d0 = __builtin_amdgcn_fdot2_f32_bf16(qp[gi][2], k2, d0, false);
      d1 = __builtin_amdgcn_fdot2_f32_bf16(qp[gi][3], k3, d1, false);
      const float dot = group_sum<LPK>(d0 + d1);  // every lane, then the mask
      const float sc = ok ? dot * c : neg_inf;
      if (__any(sc > m[gi] + kRescale)) {
        const float mn = fmaxf(m[gi], sc);
        const float a = __builtin_amdgcn_exp2f(m[gi] - mn);
        l[gi] *= a;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[gi][i] *= a;
        m[gi] = mn;
      }
      const float pe = __builtin_amdgcn_exp2f(sc - m[gi]);
      l[gi] += pe;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[gi][i] = __builtin_fmaf(pe, vf[i], o[gi][i]);
    }
  };
  auto consume = [&](int kb, const uint4 (&kr)[kUnroll], const uint4 (&vr)[kUnroll]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) consume_one(kb + u * KPI + kslot < wc, kr[u], vr[u]);
  };
  // two register sets: the next group's loads are in flight while a group
  // is consumed
  if (w0 < wc) {
    constexpr int kStep = kUnroll * KPI;
    uint4 ka[kUnroll], va[kUnroll], kb2[kUnroll], vb2[kUnroll];
    int ida[kUnroll], idb[kUnroll];
    fetch(w0, ida);
    fetch(w0 + kStep, idb);
    load(w0, ka, va, ida);
    for (int kb = w0;; kb += 2 * kStep) {
      fetch(kb + 2 * kStep, ida);
      load(kb + kStep, kb2, vb2, idb);
      consume(kb, ka, va);
      if (kb + kStep >= wc) break;
      fetch(kb + 3 * kStep, idb);
      load(kb + 2 * kStep, ka, va, ida);
      consume(kb + kStep, kb2, vb2);
      if (kb + 2 * kStep >= wc) break;
    }
  }
  if (w0 <= pre && pre < w1)  // the row's own key, in key slot 0
    consume_one(kslot == 0, *(const uint4*)kn, *(const uint4*)vn);

  // combine the KPI key slots of the wave (lanes l and l ^ x, x >= LPK)
#pragma unroll
  for (int x = LPK; x < 64; x <<= 1) {
#pragma unroll
    for (int gi = 0; gi < GC; ++gi) {
      const float m2 = lane_read(m[gi], lane ^ x);
      const float l2 = lane_read(l[gi], lane ^ x);
      const float mn = fmaxf(m[gi], m2);
      const float a = __builtin_amdgcn_exp2f(m[gi] - mn), a2 = __builtin_amdgcn_exp2f(m2 - mn);
      l[gi] = l[gi] * a + l2 * a2;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[gi][i] = o[gi][i] * a + lane_read(o[gi][i], lane ^ x) * a2;
      m[gi] = mn;
    }
  }
  // then the W waves, through LDS
  if (lane < LPK) {
#pragma unroll
    for (int gi = 0; gi < GC; ++gi) {
      if (lane == 0) {
        rd[wave][gi][0] = m[gi];
        rd[wave][gi][1] = l[gi];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) rd[wave][gi][2 + 8 * dch + i] = o[gi][i];
    }
  }
  __syncthreads();
  if (wave == 0 && lane < LPK) {
#pragma unroll
    for (int gi = 0; gi < GC; ++gi) {
      float mm = rd[0][gi][0];
#pragma unroll
      for (int w = 1; w < W; ++w) mm = fmaxf(mm, rd[w][gi][0]);
      float ll = 0.f, oo[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) oo[i] = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float a = __builtin_amdgcn_exp2f(rd[w][gi][0] - mm);
        ll = __builtin_fmaf(rd[w][gi][1], a, ll);
#pragma unroll
        for (int i = 0; i < 8; ++i) oo[i] = __builtin_fmaf(rd[w][gi][2 + 8 * dch + i], a, oo[i]);
      }
      const float inv = ll > 0.f ? 1.f / ll : 0.f;
      const int64_t row = (int64_t)tok * H + h0 + gi;
      if (ns == 1) {
        uint4 w;
        w.x = pack_bf16x2(oo[0] * inv, oo[1] * inv);
        w.y = pack_bf16x2(oo[2] * inv, oo[3] * inv);
        w.z = pack_bf16x2(oo[4] * inv, oo[5] * inv);
        w.w = pack_bf16x2(oo[6] * inv, oo[7] * inv);
        *(uint4*)(p.out + row * D + 8 * dch) = w;
      } else {
        const int64_t slot = row * p.max_segs + s;
        float* dst = p.part_o + slot * D + 8 * dch;
        *(float4*)dst = make_float4(oo[0] * inv, oo[1] * inv, oo[2] * inv, oo[3] * inv);
        *(float4*)(dst + 4) = make_float4(oo[4] * inv, oo[5] * inv, oo[6] * inv, oo[7] * inv);
        if (lane == 0) p.part_lse[slot] = ll > 0.f ? mm + __builtin_amdgcn_logf(ll) : neg_inf;
      }
    }
  }
  // the segment holding the row's own position writes its K/V to the cache,
  // once per K/V head (the unit of the group's first query heads)
  if (wave == 1 && lane < LPK && s == ns - 1 && h0 == hk * G) {
    const int64_t row = kPaged ? ((int64_t)bt_row[pre / kPageRows] * HK + hk) * kPageRows + pre % kPageRows
                               : crow + pre;
    *(uint4*)(p.kc + row * D + 8 * dch) = *(const uint4*)kn;
    *(uint4*)(p.vc + row * D + 8 * dch) = *(const uint4*)vn;
  }
  // every wave read the previous *taken before the barrier above
  if (next && tid == 0) *taken = nxt;
  __syncthreads();  // red is rewritten by the next unit
}

// Unit g of the plan's decode list p.dec_items.
template <int D, int GC, bool kPaged, int W>
__device__ __forceinline__ void decode_unit(const FwdParams& p, int64_t g, float* red,
                                            unsigned long long* next, unsigned long long* taken) {
  decode_unit<D, GC, kPaged, W>(p, g, p.dec_items[g / (p.num_heads / GC)], red, next, taken);
}

}  // namespace dec
}  // namespace pa
