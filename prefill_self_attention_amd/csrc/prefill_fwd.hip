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
//  * Work-group = (sequence b, head h, block of BM = 128 query rows); four
//    wave64s, each owning 32 consecutive query rows.  The grid is laid out
//    (head, sequence, q-block) with the q-block index reversed, so the
//    hardware dispatches the longest (highest) q-blocks first; with H a
//    multiple of 8 every q-block of one head lands on the same XCD (the
//    dispatcher deals work-groups round-robin over the 8 XCDs), which keeps
//    that head's K/V in one L2.
//  * Key tiles of BN = 64 absolute key positions.  The work-group stages
//    K[64][D] row-major and V^T[D][64] (keys permuted inside each group of 16,
//    see below) in LDS; the next tile's global loads are issued before the
//    current tile's MFMAs, so HBM latency hides behind compute.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q^T held in VGPRs for the
//    whole loop).  In the 32x32 accumulator layout lane l holds query column
//    l%32 and 16 key rows 8*(r/4) + 4*(l/32) + r%4, so a query's whole score
//    row lives in two lanes (l and l^32): the online-softmax max needs one
//    cross-half exchange per tile, the running sum none until the end, and
//    the O rescale is a per-lane multiply.
//  * Online softmax in the exp2 domain: s2 = s * scale * log2(e);
//    m' = max(m, rowmax), alpha = 2^(m - m'), p = 2^(s2 - m'),
//    l = alpha l + sum p, O = alpha O.  This streams the row normaliser that
//    the definition takes over the whole row.
//  * O^T = V^T P^T, again 32x32x16 MFMA: the B operand is P^T converted to
//    bf16 straight from the score accumulator (registers 8s..8s+7 of a
//    32-key block are keys {16s + 8*(i/4) + 4*(l/32) + i%4}); V^T in LDS
//    stores keys of each 16-group in the order [0..3, 8..11, 4..7, 12..15] so
//    the matching A operand is one 16-byte LDS read.
//  * Causal masking is applied only on tiles that cross the wave's diagonal or
//    the end of the keys; tiles wholly above a wave's diagonal are skipped by
//    that wave, and never loaded by a work-group none of whose rows sees them.
//  * KV-cache write: the work-group that owns query rows [q0, q0+BM) copies
//    K/V of exactly those tokens from the registers it staged them through,
//    with full-row coalesced stores.  Prefix keys of chunked prefill are read
//    from the cache, new keys always from k/v, so no work-group reads a cache
//    position this launch writes.
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

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;  // query rows per work-group
constexpr int kBN = 64;           // keys per tile
constexpr int kKPad = 8;          // bf16 elements of padding per K row in LDS
constexpr int kVPad = 8;          // bf16 elements of padding per V^T row in LDS

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

// Key (relative to its 16-group) stored at position i (0..7) of half `hh`
// of the group: the order matches the 32x32 accumulator's row mapping.
__device__ __forceinline__ int vt_key(int hh, int i) {
  return 8 * (i >> 2) + 4 * hh + (i & 3);
}

template <int D, bool kChunked>
struct Tile {
  // K chunks of 8 bf16 (16 B) per thread, and V dword columns for 8 keys.
  static constexpr int kKChunks = kBN * D / 8;                 // 16-B chunks per K tile
  static constexpr int kKPerThread = (kKChunks + kThreads - 1) / kThreads;
  static constexpr int kVItems = (D / 2) * (kBN / 8);           // (d pair, key octet)
  static constexpr int kVPerThread = (kVItems + kThreads - 1) / kThreads;
  static constexpr int kKStride = D + kKPad;                   // LDS row stride (elements)
  static constexpr int kVStride = kBN + kVPad;
};

template <int D, bool kChunked>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_fwd_kernel(FwdParams p) {
  using T = Tile<D, kChunked>;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kBN * T::kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * T::kVStride];

  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int qb = p.nqb - 1 - (int)blockIdx.z;
  const int64_t H = p.num_heads;

  const int seq_start = p.cu[b];
  const int len = p.cu[b + 1] - seq_start;
  const int q0 = qb * kBM;
  if (q0 >= len) return;
  const int pre = kChunked ? p.prefix[b] : 0;
  const int qend = min(q0 + kBM, len);
  const int key_end = pre + qend;             // keys this work-group needs: [0, key_end)
  const int own_lo = pre + q0;                // cache rows this work-group writes
  const int ntiles = (key_end + kBN - 1) / kBN;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int ql = lane & 31;
  const int hh = lane >> 5;

  const int64_t row_stride = H * D;           // elements between consecutive tokens
  const uint16_t* __restrict__ kin = p.k + (int64_t)h * D;
  const uint16_t* __restrict__ vin = p.v + (int64_t)h * D;
  // cache base for this (b, h): element of absolute key position 0
  int64_t cache_base;
  if (kChunked) {
    cache_base = ((int64_t)b * H + h) * p.cap * D;
  } else {
    cache_base = (int64_t)seq_start * H * D + (int64_t)h * len * D;
  }

  // ---------------------------------------------------------- Q operand (B)
  const int qrow0 = q0 + 32 * wave;           // first local row of this wave
  const bool wave_active = qrow0 < len;
  const int qa0 = pre + qrow0;                // its absolute position
  const int qa = qa0 + ql;                    // this lane's query position
  bf16x8_t qop[D / 16];
  {
    const int row = qrow0 + ql;
    const bool ok = row < len;
    const uint16_t* src = p.q + ((int64_t)(seq_start + (ok ? row : 0)) * H + h) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4_t x = ok ? *(const u32x4_t*)(src + 16 * ks) : u32x4_t{0, 0, 0, 0};
      qop[ks] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  f32x16_t o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16_t{};
  float m_run = -__builtin_huge_valf();
  float l_run = 0.f;

  // ---------------------------------------------------------- staging regs
  u32x4_t kreg[T::kKPerThread];
  uint32_t vreg[T::kVPerThread][8];

  // Source row of absolute key position kp (valid keys only).
  auto key_src = [&](const uint16_t* __restrict__ in, const uint16_t* __restrict__ cache,
                     int kp) -> const uint16_t* {
    if (kChunked && kp < pre) return cache + cache_base + (int64_t)kp * D;
    return in + (int64_t)(seq_start + kp - pre) * row_stride;
  };

  auto load_tile = [&](int t) {
    const int t0 = t * kBN;
#pragma unroll
    for (int i = 0; i < T::kKPerThread; ++i) {
      const int c = tid + kThreads * i;
      kreg[i] = u32x4_t{0, 0, 0, 0};
      if (c < T::kKChunks) {
        const int kp = t0 + c / (D / 8);
        if (kp < key_end)
          kreg[i] = *(const u32x4_t*)(key_src(kin, p.kc, kp) + 8 * (c % (D / 8)));
      }
    }
#pragma unroll
    for (int i = 0; i < T::kVPerThread; ++i) {
      const int item = tid + kThreads * i;
#pragma unroll
      for (int e = 0; e < 8; ++e) vreg[i][e] = 0u;
      if (item < T::kVItems) {
        const int dp = item % (D / 2);
        const int oct = item / (D / 2);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int kp = t0 + 16 * (oct >> 1) + vt_key(oct & 1, e);
          if (kp < key_end)
            vreg[i][e] = *(const uint32_t*)(key_src(vin, p.vc, kp) + 2 * dp);
        }
      }
    }
  };

  auto store_tile = [&](int t) {
    const int t0 = t * kBN;
#pragma unroll
    for (int i = 0; i < T::kKPerThread; ++i) {
      const int c = tid + kThreads * i;
      if (c < T::kKChunks) {
        const int r = c / (D / 8), c8 = c % (D / 8);
        *(u32x4_t*)(k_lds + r * T::kKStride + 8 * c8) = kreg[i];
        const int kp = t0 + r;
        if (kp >= own_lo && kp < key_end)
          *(u32x4_t*)(p.kc + cache_base + (int64_t)kp * D + 8 * c8) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < T::kVPerThread; ++i) {
      const int item = tid + kThreads * i;
      if (item < T::kVItems) {
        const int dp = item % (D / 2);
        const int oct = item / (D / 2);
        u32x4_t lo, hi;
        lo[0] = pack_lo(vreg[i][0], vreg[i][1]);
        lo[1] = pack_lo(vreg[i][2], vreg[i][3]);
        lo[2] = pack_lo(vreg[i][4], vreg[i][5]);
        lo[3] = pack_lo(vreg[i][6], vreg[i][7]);
        hi[0] = pack_hi(vreg[i][0], vreg[i][1]);
        hi[1] = pack_hi(vreg[i][2], vreg[i][3]);
        hi[2] = pack_hi(vreg[i][4], vreg[i][5]);
        hi[3] = pack_hi(vreg[i][6], vreg[i][7]);
        *(u32x4_t*)(vt_lds + (2 * dp) * T::kVStride + 8 * oct) = lo;
        *(u32x4_t*)(vt_lds + (2 * dp + 1) * T::kVStride + 8 * oct) = hi;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int kp = t0 + 16 * (oct >> 1) + vt_key(oct & 1, e);
          if (kp >= own_lo && kp < key_end)
            *(uint32_t*)(p.vc + cache_base + (int64_t)kp * D + 2 * dp) = vreg[i][e];
        }
      }
    }
  };

  load_tile(0);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();  // all waves are done reading the previous tile
    store_tile(t);
    __syncthreads();
    if (t + 1 < ntiles) load_tile(t + 1);

    const int t0 = t * kBN;
    if (!wave_active || t0 > qa0 + 31) continue;  // tile wholly above this wave's rows

    // S^T = K Q^T for two 32-key blocks
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16_t{};
      const uint16_t* kr = k_lds + (32 * kb + ql) * T::kKStride + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        bf16x8_t a = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(kr + 16 * ks));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[ks], s[kb], 0, 0, 0);
      }
    }

    // scale, mask, row max
    const bool need_mask = (t0 + kBN - 1 > qa0) || (t0 + kBN > key_end);
    float mx = -__builtin_huge_valf();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[kb][r] * p.scale_log2;
        if (need_mask) {
          const int kp = t0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (kp > qa || kp >= key_end) x = -__builtin_huge_valf();
        }
        s[kb][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;

    // p = 2^(s2 - m), row sum (per lane), P^T -> bf16 B operands
    float ls = 0.f;
    bf16x8_t pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          e[i] = __builtin_amdgcn_exp2f(s[kb][8 * sh + i] - m_new);
          ls += e[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x2_t two = {e[2 * i], e[2 * i + 1]};
          bf16x2_t c = __builtin_convertvector(two, bf16x2_t);
          pb[2 * kb + sh][2 * i] = c[0];
          pb[2 * kb + sh][2 * i + 1] = c[1];
        }
      }
    }
    l_run = alpha * l_run + ls;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) o[mb] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
      const uint16_t* vr = vt_lds + (32 * mb + ql) * T::kVStride + 8 * hh;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x8_t a = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(vr + 16 * g));
        o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[g], o[mb], 0, 0, 0);
      }
    }
  }

  // ---------------------------------------------------------- epilogue
  if (!wave_active) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  const int row = qrow0 + ql;
  if (row >= len) return;
  uint16_t* dst = p.out + ((int64_t)(seq_start + row) * H + h) * D + 4 * hh;
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      f32x2_t a = {o[mb][4 * c + 0] * inv, o[mb][4 * c + 1] * inv};
      f32x2_t bb = {o[mb][4 * c + 2] * inv, o[mb][4 * c + 3] * inv};
      bf16x2_t ca = __builtin_convertvector(a, bf16x2_t);
      bf16x2_t cb = __builtin_convertvector(bb, bf16x2_t);
      u32x2_t w = {__builtin_bit_cast(uint32_t, ca), __builtin_bit_cast(uint32_t, cb)};
      *(u32x2_t*)(dst + 32 * mb + 8 * c) = w;
    }
  }
}

template <int D, bool kChunked>
hipError_t launch_d(const FwdParams& p, int num_seqs, hipStream_t stream) {
  dim3 grid(p.num_heads, num_seqs, p.nqb);
  hipLaunchKernelGGL((prefill_fwd_kernel<D, kChunked>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int fwd_block_rows() { return kBM; }

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
