// Prefill attention over a short int4 KV cache (kv_len <= 256, D = 64), causal
// or not: ViT-style self-attention, where a head's whole key range is a few
// KB of codes.
//
// One workgroup per query head converts the head's entire key range once into
// LDS (exact fp16 codes, "Quantized Cross-Attention: Extending
// FlashAttention-3 with In-SRAM Dequantization" §3.1: dequantization happens
// on chip, never to HBM) and then every wave runs its 32 query rows over all
// of it with no further barrier: online softmax across 32-token key blocks
// (TurboAttention arXiv 2412.08585 §2.2), K scale on score columns in fp32,
// V scale folded into P before its fp16 rounding (§3.4 in its exact reading),
// P~ as an fp16 hi/lo pair where V scales pass the precision limit.
//
// Against the tiled prefill this removes the per-tile barriers and double
// buffering (a 197-token head is four 64-token tiles there), converts each
// head once instead of once per 128-row block, and pads keys to 8 tokens
// instead of 64: the PV product runs on v_mfma_f32_32x32x8_f16, whose K
// dimension is 8 tokens.
//
//   S^T = K Q^T    v_mfma_f32_32x32x16_f16 (M = 32 tokens, N = 32 rows, K = 16 dims)
//   O^T += V^T P^T v_mfma_f32_32x32x8_f16  (M = 32 dims, N = 32 rows, K = 8 tokens)
// Lane (r, j) = (lane % 32, lane / 32) owns query row r of its wave; its 16
// scores of a key block are tokens 8 vq + 4 j + i (vq, i in 0..3), and the four
// of step vq are exactly its B operand of the PV product for tokens 8 vq ..
// 8 vq + 7 -- no data moves between lanes except the row max.
//
// LDS (72 KB, fixed strides, so that each read of a key block is one base
// address plus immediate offsets):
//   K: fp16 rows of 64 head dims in unpack8_perm order, 144 bytes apart (an
//      odd multiple of 16: the 16 lanes of a read phase, 16 consecutive
//      tokens of one 16-byte chunk, cover all 64 banks).  Key blocks read
//      rows up to the next multiple of 32; rows past kv_len hold whatever
//      the LDS held, and their scores are replaced by -inf.
//   V: fp16 transposed, [64 dims][264 tokens] (an odd multiple of 8 tokens:
//      a PV read of 16 consecutive dims hits 16 distinct 2-dword bank
//      pairs); tokens from kv_len to the next multiple of 8 hold zeros.
//   tables: fp32 K scale x softmax_scale x log2(e) per token, fp16 V scale
//      per token (zeros past kv_len).
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "qkvfa_device.hpp"
#include "qkvfa_internal.h"

namespace qkvfa {

namespace {

typedef _Float16 half4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float16v mfma32x32x8(half4v a, half4v b, float16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x8f16(a, b, c, 0, 0, 0);
}

constexpr int kSD = 64;            // head dim of this kernel
constexpr int kSRowB = kSD / 2;    // bytes per cache row
constexpr float kSTau = 8.0f;      // lazy-rescale threshold (log2 units)
constexpr int kSMaxWaves = 8;
// query rows per workgroup: all of a head's (kShortRowGroups = 0), or row
// groups of kShortRowGroupWaves waves
constexpr int kShortRowGroups = 0;
constexpr int kShortRowGroupWaves = 4;

// LDS strides (halves), fixed so that every read of a key block is one base
// address plus immediate offsets: K rows of 72 halves (144 bytes, an odd
// multiple of 16: the 16 lanes of a read phase -- 16 consecutive tokens, one
// 16-byte chunk -- cover all 64 banks), V^T rows of 264 tokens (an odd
// multiple of 8: the 16 dims of a read phase hit 16 distinct bank pairs).
constexpr int kSKStride = 72;
constexpr int kSVStride = 264;
constexpr int kSMaxKeys = 256;

template <bool CAUSAL>
__global__ __launch_bounds__(64 * kSMaxWaves) __attribute__((amdgpu_waves_per_eu(4))) void prefill_short_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kc, const uint16_t* __restrict__ ks,
    const uint8_t* __restrict__ vc, const uint16_t* __restrict__ vs, const int32_t* __restrict__ kv_heads,
    int Hkv_all, int Hq, int Hkv, int G, int Sq, int kv_len, int64_t C, float qk_log2, int n_heads, int rgs,
    float* __restrict__ out, float* __restrict__ lse_out) {
  constexpr int D = kSD;
  __shared__ __align__(16) _Float16 sK[kSMaxKeys * kSKStride];   // K rows, fp16 codes in unpack8_perm order
  __shared__ __align__(16) _Float16 sV[kSD * kSVStride];         // V^T, fp16 codes (zeros past kv_len)
  __shared__ __align__(16) float csk[kSMaxKeys];                  // K scale x softmax scale x log2 e (0 past kv_len)
  __shared__ __align__(16) _Float16 svh[kSVStride];               // V scale (0 past kv_len)
  // per wave: largest |q| (bf16 bits), |K scale| and |V scale| (fp16 bits)
  __shared__ uint32_t s_mx[3][kSMaxWaves];
  const int lk8 = (kv_len + 7) & ~7;     // tokens converted (zeros past kv_len)
  const int lk32 = (kv_len + 31) & ~31;  // tokens the key blocks read

  const int nw = __builtin_amdgcn_readfirstlane((int)(blockDim.x >> 6));
  const int nth = 64 * nw;
  const int tid = threadIdx.x;
  const int nh = Hkv * G;   // query heads of this call per batch entry
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31;
  const int j = lane >> 5;
  // Workgroup -> (head, row group): the rgs row groups of a head run on one
  // XCD (ids 8 apart, as the dispatcher deals consecutive ids to the eight
  // XCDs in turn), so the head's codes come from HBM once.
  const int id = blockIdx.x;
  const int hh = (id / (8 * rgs)) * 8 + (id & 7);
  const int rg = (id >> 3) % rgs;
  if (hh >= n_heads) return;
  const int row0 = rg * 32 * nw;   // first query row of this workgroup
  const int row = row0 + wave * 32 + r;
  const int off = kv_len - Sq;   // >= 0 whenever CAUSAL
  const int nq = lk8 / 4;        // V token quads

  // (batch, layer query head, cache row 0) of head index hh
  auto head_of = [&](int hh, int& b, int& hq, int64_t& kvrow0) {
    b = hh / nh;
    const int h = hh - b * nh;   // query head of this call: KV head h / G of the cache
    const int g = h / G;
    hq = kv_heads ? min(max(kv_heads[g], 0), Hkv_all - 1) * G + (h - g * G) : h;
    kvrow0 = ((int64_t)b * Hkv + g) * C;
  };

  // ---- raw loads of one head (zeros past kv_len and past Sq).  K: task i =
  // dword i % 8 of row i / 8 (at least 4 waves: at most 8 tasks per thread).
  // V: task i = token quad u = (i % 16) + 16 (i / 128), dword w = (i / 16) % 8,
  // i.e. dword w of tokens 4u .. 4u + 3 (at most 3 tasks per thread).
  uint4v qraw[D / 16];
  uint32_t kraw[8];
  uint32_t vraw[3][4];
  uint32_t ksc, vsc0;
  auto issue_loads = [&](int hh) {
    int b, hq;
    int64_t kvrow0;
    head_of(hh, b, hq, kvrow0);
    if (row < Sq) {
      const uint16_t* qr = q + (((int64_t)b * Hq + hq) * Sq + row) * D;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) qraw[s] = *reinterpret_cast<const uint4v*>(qr + 8 * (2 * s + j));
    } else {
#pragma unroll
      for (int s = 0; s < D / 16; ++s) qraw[s] = uint4v{0u, 0u, 0u, 0u};
    }
    const rsrc_t rk = make_rsrc(kc + kvrow0 * kSRowB, kv_len * kSRowB);
    const rsrc_t rv = make_rsrc(vc + kvrow0 * kSRowB, kv_len * kSRowB);
    const rsrc_t rks = make_rsrc(ks + kvrow0, kv_len * 2);
    const rsrc_t rvs = make_rsrc(vs + kvrow0, kv_len * 2);
#pragma unroll
    for (int it = 0; it < 8; ++it)
      kraw[it] = __builtin_amdgcn_raw_buffer_load_b32(rk, (uint32_t)((tid + it * nth) * 4), 0, 0);
#pragma unroll
    for (int it = 0; it < 3; ++it) {
      const int i = tid + it * nth;
      const int u = (i & 15) | ((i >> 7) << 4), w = (i >> 4) & 7;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        vraw[it][k] = __builtin_amdgcn_raw_buffer_load_b32(rv, (uint32_t)((4 * u + k) * kSRowB + 4 * w), 0, 0);
    }
    ksc = __builtin_amdgcn_raw_buffer_load_b16(rks, (uint32_t)(tid * 2), 0, 0);
    vsc0 = __builtin_amdgcn_raw_buffer_load_b16(rvs, (uint32_t)(tid * 2), 0, 0);
  };

  const int wrow_lo = row0 + wave * 32;
  const int wrow_hi = min(wrow_lo + 31, Sq - 1);
  // key blocks of this wave: up to its last visible key
  const int last_key = CAUSAL ? min(kv_len - 1, wrow_hi + off) : kv_len - 1;
  const int nkb = last_key / 32 + 1;
  // blocks visible to all 32 rows and inside kv_len: no mask
  int nfull = kv_len / 32;
  if (CAUSAL) nfull = min(nfull, max(0, (wrow_lo + off + 1) / 32));
  nfull = min(nfull, nkb);
  // per-lane bases: K row r at chunk j, V^T row r at token 4 j, tables at 4 j
  const _Float16* kbase = sK + r * kSKStride + 8 * j;
  const _Float16* vbase = sV + r * kSVStride + 4 * j;
  const float* cbase = csk + 4 * j;
  const _Float16* sbase = svh + 4 * j;

  issue_loads(hh);
  {
    // ---- maxima of the loaded head
    {
      uint32_t qmb = 0;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) qmb = max(qmb, bf16x8_max_abs_bits(qraw[s]));
      qmb = bitcast<uint32_t>(wave_max_nonneg(bitcast<float>(qmb)));
      // K and V scale maxima in one reduction: |K| in bits 16-30, |V| in bits 0-14
      const uint32_t kv = ((ksc & 0x7FFFu) << 16) | (vsc0 & 0x7FFFu);
      const uint32_t kvk = bitcast<uint32_t>(wave_max_nonneg(bitcast<float>(kv & 0x7FFF0000u)));
      const uint32_t kvv = bitcast<uint32_t>(wave_max_nonneg(bitcast<float>(kv & 0x7FFFu)));
      if (lane == 0) {
        s_mx[0][wave] = qmb;
        s_mx[1][wave] = kvk >> 16;
        s_mx[2][wave] = kvv;
      }
    }
    __syncthreads();
    uint32_t qm = 0, km = 0, vm = 0;
    for (int w = 0; w < nw; ++w) {
      qm = max(qm, s_mx[0][w]);
      km = max(km, s_mx[1][w]);
      vm = max(vm, s_mx[2][w]);
    }
    qm = __builtin_amdgcn_readfirstlane(qm);
    km = __builtin_amdgcn_readfirstlane(km);
    vm = __builtin_amdgcn_readfirstlane(vm);
    // Query range: an exact power-of-two shift into fp16 range, folded into
    // the score scale (0 unless some |q| >= 65536).
    const int qshift = q_range_shift(qm);
    const float qk = qk_log2 * exp2i(qshift);
    // Query operand: row `row`, k = 8 j + e <-> head dim 8 (2 s + j) + perm8(e)
    half8v qop[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      uint16_t e16[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        e16[2 * t] = (uint16_t)(qraw[s][t] & 0xFFFFu);
        e16[2 * t + 1] = (uint16_t)(qraw[s][t] >> 16);
      }
      if (qshift == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qop[s][e] = (_Float16)bf16_to_f32(e16[perm8(e)]);
      } else {
        const float qmul = exp2i(-qshift);
#pragma unroll
        for (int e = 0; e < 8; ++e) qop[s][e] = (_Float16)(bf16_to_f32(e16[perm8(e)]) * qmul);
      }
    }
    // ---- conversion into LDS
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int i = tid + it * nth;
      if (i < lk8 * 8) {
        const int t = i >> 3, w = i & 7;
        *reinterpret_cast<half8v*>(sK + t * kSKStride + 8 * w) = unpack8_perm(kraw[it]);
      }
    }
#pragma unroll
    for (int it = 0; it < 3; ++it) {
      const int i = tid + it * nth;
      const int u = (i & 15) | ((i >> 7) << 4), w = (i >> 4) & 7;
      if (u < nq) {
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const half2v a = nib_pair2(vraw[it][0], vraw[it][1], n);
          const half2v c2 = nib_pair2(vraw[it][2], vraw[it][3], n);
          const uint2v x = {bitcast<uint32_t>(a), bitcast<uint32_t>(c2)};
          *reinterpret_cast<uint2v*>(sV + (8 * w + n) * kSVStride + 4 * u) = x;
        }
      }
    }
    if (tid < lk32) csk[tid] = f16bits_to_f32((uint16_t)ksc) * qk;
    if (tid < lk8) svh[tid] = bitcast<_Float16>((uint16_t)vsc0);
    __syncthreads();

    int b, hq;
    {
      int64_t unused;
      head_of(hh, b, hq, unused);
    }
    if (wrow_lo >= Sq) return;   // no rows in this wave (after the last barrier)

    const float cmax = f16bits_to_f32((uint16_t)km) * qk;   // max |K scale x qk|
    const bool hilo = vm > pv_scale_limit_bits(pv_code_max(4, false));
    // rescale threshold of the hi/lo form: p <= 2^tau with 2^tau max s_V <= 2^15
    const float tau_hl = fminf(kSTau, fmaxf(0.0f, 15.0f - __log2f(f16bits_to_f32((uint16_t)vm))));

    float16v o_acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o_acc[db] = float16v{};
    float m_ref = -INFINITY;   // row reference (log2 units), shared by lanes r and r + 32
    float m_use = 0.0f;        // m_ref, or 0 while the row has seen no key
    float l_run = 0.0f;        // this lane's share of sum(p), relative to m_ref

    auto block = [&](int kb, auto full_c, auto hilo_c) {
      constexpr bool FULL = decltype(full_c)::value;
      constexpr bool HILO = decltype(hilo_c)::value;
      const int t0 = 32 * kb;
      // ---- S^T = K Q^T: tokens t0 + r (lane) x 32 rows
      float16v st = float16v{};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const half8v a = *reinterpret_cast<const half8v*>(kbase + t0 * kSKStride + 16 * s);
        st = mfma32x32x16(a, qop[s], st);
      }
      // ---- online softmax; lane's tokens t0 + 8 vq + 4 j + i
      auto colf = [&](int vq) { return *reinterpret_cast<const float4v*>(cbase + t0 + 8 * vq); };
      const float tau = HILO ? tau_hl : kSTau;
      float mx;
      if constexpr (FULL) {
        // upper bound of the lane's max score: max |s| x max |csk|
        mx = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, fabsf(st[v]));
        mx *= cmax;
      } else {
        const int lim = (CAUSAL ? min(kv_len - 1, row + off) : kv_len - 1) - t0 - 4 * j;
        mx = -INFINITY;
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) {
          const float4v c = colf(vq);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool ok = 8 * vq + i <= lim;
            const float x = ok ? st[4 * vq + i] * c[i] : -INFINITY;
            st[4 * vq + i] = x;
            mx = fmaxf(mx, x);
          }
        }
      }
      if (__builtin_amdgcn_ballot_w64(mx > m_ref + tau)) {
        if constexpr (FULL) {
          mx = -INFINITY;
#pragma unroll
          for (int vq = 0; vq < 4; ++vq) {
            const float4v c = colf(vq);
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[4 * vq + i] * c[i]);
          }
        }
        mx = xor_max(mx, 32);
        const bool up = mx > m_ref + tau;
        const float alpha = up ? fast_exp2(m_ref - mx) : 1.0f;
        m_ref = up ? mx : m_ref;
        m_use = (m_ref == -INFINITY) ? 0.0f : m_ref;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o_acc[db] *= alpha;
      }
      // ---- P~ and O^T += V^T P~^T, 8 tokens per step (none past kv_len)
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        if (!FULL && t0 + 8 * vq >= kv_len) break;   // uniform
        // keeps this step's LDS reads here: hoisted, the four steps' column
        // factors, V scales and V operands would be live at once
        asm volatile("" ::: "memory");
        const half4v sv = *reinterpret_cast<const half4v*>(sbase + t0 + 8 * vq);
        float p[4];
        if constexpr (FULL) {
          const float4v c = colf(vq);
#pragma unroll
          for (int i = 0; i < 4; ++i) p[i] = fast_exp2(fmaf(st[4 * vq + i], c[i], -m_use));
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) p[i] = fast_exp2(st[4 * vq + i] - m_use);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) l_run += p[i];
        half4v ph, pl;
        if constexpr (HILO) {   // high halves pinned, low halves about them
          const half2v h0 = pv_hi2(p[0], (float)sv[0], p[1], (float)sv[1]);
          const half2v h1 = pv_hi2(p[2], (float)sv[2], p[3], (float)sv[3]);
          ph = half4v{h0[0], h0[1], h1[0], h1[1]};
          pin_v(ph);
#pragma unroll
          for (int i = 0; i < 4; ++i) pl[i] = pv_lo(p[i], (float)sv[i], ph[i]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) ph[i] = (_Float16)fmaf(p[i], (float)sv[i], 0.0f);
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const half4v a = *reinterpret_cast<const half4v*>(vbase + 32 * db * kSVStride + t0 + 8 * vq);
          o_acc[db] = mfma32x32x8(a, ph, o_acc[db]);
          if constexpr (HILO) o_acc[db] = mfma32x32x8(a, pl, o_acc[db]);
        }
      }
    };
    using T_ = std::integral_constant<bool, true>;
    using F_ = std::integral_constant<bool, false>;
    if (!hilo) {
      int kb = 0;
      for (; kb < nfull; ++kb) block(kb, T_{}, F_{});
      for (; kb < nkb; ++kb) block(kb, F_{}, F_{});
    } else {
      for (int kb = 0; kb < nkb; ++kb) block(kb, F_{}, T_{});
    }

    // ---- O = O^T / l; lane owns row `row`, head dims 32 db + 8 vq + 4 j + i
    const float l = xor_sum(l_run, 32);
    if (row < Sq) {
      const float inv = 1.0f / l;
      float* orow = out + (((int64_t)b * Hq + hq) * Sq + row) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) {
          const float4v v = {o_acc[db][4 * vq + 0] * inv, o_acc[db][4 * vq + 1] * inv,
                             o_acc[db][4 * vq + 2] * inv, o_acc[db][4 * vq + 3] * inv};
          *reinterpret_cast<float4v*>(orow + 32 * db + 8 * vq + 4 * j) = v;
        }
      }
      if (j == 0 && lse_out) lse_out[((int64_t)b * Hq + hq) * Sq + row] = (m_ref + log2f(l)) * kLn2;
    }
  }
}

}  // namespace

bool prefill_short_fits(int64_t D, int64_t Sq, int64_t kv_len, int bits) {
  return D == kSD && bits == 4 && kv_len >= 1 && kv_len <= 256 && Sq >= 1 && Sq <= 32 * kSMaxWaves;
}

hipError_t launch_prefill_short(const uint16_t* q, const uint8_t* kc, const uint16_t* ks, const uint8_t* vc,
                                const uint16_t* vs, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq,
                                int64_t kv_len, int64_t C, float softmax_scale, int causal, float* out,
                                float* lse, hipStream_t stream, const int32_t* kv_heads, int64_t Hkv_all) {
  const int Hall = (int)(kv_heads ? Hkv_all : Hkv);
  const int G = (int)(Hq / Hall);
  // row groups of 32 x nw query rows per head, at least 4 waves each (the
  // conversion's task counts assume it)
  const int rgs = kShortRowGroups > 0 ? (int)((Sq + 32 * kShortRowGroupWaves - 1) / (32 * kShortRowGroupWaves)) : 1;
  const int nw = (int)std::max<int64_t>(4, (Sq + 32 * rgs - 1) / (32 * rgs));
  const int n_heads = (int)(B * Hkv * G);
  const int grid = ((n_heads + 7) / 8) * 8 * rgs;
  auto kern = causal ? prefill_short_kernel<true> : prefill_short_kernel<false>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * nw), 0, stream, q, kc, ks, vc, vs, kv_heads, Hall,
                     (int)Hq, (int)Hkv, G, (int)Sq, (int)kv_len, C, softmax_scale * kLog2e, n_heads, rgs, out, lse);
  return hipGetLastError();
}

}  // namespace qkvfa
