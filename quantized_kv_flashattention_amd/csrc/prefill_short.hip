// Prefill attention over a short int4 KV cache (kv_len <= 256, D = 64), causal
// or not: ViT-style self-attention, where a head's whole key range is a few
// KB of codes.
//
// One workgroup per query head converts the head's entire key range once into
// LDS (exact codes: bf16 for K, fp16 for V; "Quantized Cross-Attention:
// Extending FlashAttention-3 with In-SRAM Dequantization" §3.1: dequantization
// happens on chip, never to HBM); then each of its four waves runs one or two
// blocks of 32 query rows over all of it with no further barrier: online
// softmax across 32-token key blocks (TurboAttention arXiv 2412.08585 §2.2), K
// scale on score columns in fp32, V scale folded into P before its fp16
// rounding (§3.4 in its exact reading), P~ as an fp16 hi/lo pair where V scales
// pass the precision limit.
//
// The scores are products of the bf16 queries as loaded with the exact bf16
// codes (every product exact, fp32 sums): no per-row-block query conversion,
// and no range limit on the queries.  K is converted to bf16 once per head,
// which costs more per code than the fp16 form but is amortized over the
// head's seven row blocks.
//
// Against the tiled prefill this removes the per-tile barriers and double
// buffering (a 197-token head is four 64-token tiles there), converts each
// head once instead of once per 128-row block, and pads keys to 8 tokens
// instead of 64.  LDS is sized to the head's key count (52.5 KB at 197 keys), so
// that three heads' workgroups share a compute unit and a ViT-B call (768
// heads) is one round of resident workgroups.
//
//   S^T = K Q^T    v_mfma_f32_32x32x16_bf16 (M = 32 tokens, N = 32 rows, K = 16 dims)
//   O^T += V^T P^T v_mfma_f32_32x32x16_f16  (M = 32 dims, N = 32 rows, K = 16 tokens)
// Lane (r, j) = (lane % 32, lane / 32) owns query row r of its row block; its
// 16 scores of a key block are tokens 8 vq + 4 j + i (vq, i in 0..3); those of
// steps vq = 2 hs and 2 hs + 1 are exactly its B operand of the PV product for
// the 16 tokens 16 hs .. 16 hs + 15, in the order that V^T holds them -- no data
// moves between lanes except the row max.  (v_mfma_f32_32x32x8_f16 takes as long
// as the 16-token product for half the work; it runs only the first half of a
// partial last group.)
//
// LDS (dynamic; lk8 / lk32 = key count rounded up to 8 / 32):
//   K: lk8 bf16 rows of 64 head dims in dim order, 128 bytes each; 16-byte
//      chunk c of row t sits at chunk c ^ ((t >> 1) & 7), so the 16 lanes of a
//      read phase (16 consecutive tokens, one chunk) and of a conversion write
//      phase (two rows, eight chunks) cover all 64 banks.  Key blocks read rows
//      up to lk32; rows past kv_len hold whatever the LDS held (the V region,
//      the tables, or unwritten words), and their scores are replaced by -inf.
//      The allocation covers lk32 rows.
//   V: fp16 transposed, [64 dims][Sv tokens], Sv = lk8 or lk8 + 8, whichever
//      is an odd multiple of 8 (a PV read of 16 consecutive dims then hits 16
//      distinct bank groups); tokens from kv_len to lk8 hold zeros; complete
//      16-token groups in the PV operand order (group_slot).
//   tables: fp32 K scale x softmax_scale x log2(e) per token (lk32 entries,
//      zeros past kv_len), fp16 V scale per token (lk8 entries, V^T's order);
//      then the waves' K and V scale maxima.  No static LDS: the region
//      starts at address 0, so each LDS read's constant part is an
//      instruction offset.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "qkvfa_device.hpp"
#include "qkvfa_internal.h"

namespace qkvfa {

namespace {

typedef _Float16 half4v __attribute__((ext_vector_type(4)));

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float16v mfma32x32x8(half4v a, half4v b, float16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x8f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float16v mfma32x32x16_bf16(uint4v a, uint4v b, float16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8v, a), __builtin_bit_cast(bf16x8v, b), c, 0,
                                                  0, 0);
}

// Eight int4 codes (element e in bits 4e .. 4e + 3, two's complement) -> their
// exact bf16 values, element e in half e: each nibble sign-extended, converted
// to fp32 (exact), and its upper 16 bits kept (exact: at most 4 significant bits).
__device__ __forceinline__ uint4v unpack8_bf16(uint32_t x) {
  uint4v r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float lo = (float)((int32_t)(x << (28 - 8 * p)) >> 28);
    const float hi = (float)((int32_t)(x << (24 - 8 * p)) >> 28);
    r[p] = __builtin_amdgcn_perm(bitcast<uint32_t>(hi), bitcast<uint32_t>(lo), 0x07060302u);
  }
  return r;
}

constexpr int kSD = 64;            // head dim of this kernel
constexpr int kSRowB = kSD / 2;    // bytes per cache row
constexpr float kSTau = 8.0f;      // lazy-rescale threshold (log2 units)
constexpr int kSWaves = 4;         // waves per workgroup (head)
constexpr int kSBlocks = 2;        // 32-row query blocks per wave, at most
constexpr int kSMaxKeys = 256;

// V^T row stride (tokens): lk8 or lk8 + 8, whichever is an odd multiple of 8
__host__ __device__ inline int short_v_stride(int lk8) { return ((lk8 >> 3) & 1) ? lk8 : lk8 + 8; }

// Slot of token quad u (tokens 4u .. 4u + 3) in V^T and the V-scale table:
// in a complete 16-token group, quad 2 h + j (tokens 8 h + 4 j + i of the
// group) sits at slot 2 j + h, so that the 16-token product's operand of lane
// j (tokens 4 j + i and 8 + 4 j + i) is eight consecutive values; a partial
// last group (nq quads in all) keeps token order.
__device__ __forceinline__ int group_slot(int u, int nq) {
  return ((u | 3) < nq) ? ((u & ~3) | ((u & 1) << 1) | ((u >> 1) & 1)) : u;
}

// Byte offset of the per-wave scale maxima in the dynamic LDS: after K, V^T
// and the tables (no static LDS, so that the dynamic region starts at address
// 0 and every LDS read folds its constant part into the instruction's offset)
__host__ __device__ inline int short_mx_offset(int kv_len) {
  const int lk8 = (kv_len + 7) & ~7, lk32 = (kv_len + 31) & ~31;
  return (lk8 * 128 + kSD * short_v_stride(lk8) * 2 + lk32 * 4 + lk8 * 2 + 15) & ~15;
}

// Dynamic LDS bytes of a head with kv_len keys (layout in the file comment)
inline size_t short_lds_bytes(int kv_len) {
  const size_t used = (size_t)short_mx_offset(kv_len) + 2 * kSWaves * 4;
  const size_t krows = (size_t)((kv_len + 31) & ~31) * 128;   // key blocks read K rows up to lk32
  return used > krows ? used : krows;
}

template <bool CAUSAL>
__global__ __launch_bounds__(64 * kSWaves) __attribute__((amdgpu_waves_per_eu(3))) void prefill_short_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kc, const uint16_t* __restrict__ ks,
    const uint8_t* __restrict__ vc, const uint16_t* __restrict__ vs, const int32_t* __restrict__ kv_heads,
    int Hkv_all, int Hq, int Hkv, int G, int Sq, int kv_len, int64_t C, float qk_log2, int n_heads,
    float* __restrict__ out, float* __restrict__ lse_out) {
  constexpr int D = kSD;
  constexpr int nth = 64 * kSWaves;
  extern __shared__ __align__(16) _Float16 s_lds[];
  const int lk8 = (kv_len + 7) & ~7;     // tokens converted (zeros past kv_len)
  const int lk32 = (kv_len + 31) & ~31;  // tokens the key blocks read
  const int sv = short_v_stride(lk8);
  _Float16* sK = s_lds;                                             // [lk8][64], swizzled chunks
  _Float16* sV = s_lds + lk8 * D;                                   // [64][sv]
  float* csk = reinterpret_cast<float*>(sV + D * sv);               // [lk32]
  _Float16* svh = reinterpret_cast<_Float16*>(csk + lk32);          // [lk8]
  // per wave: largest |K scale| (s_mx[wave]) and |V scale| (s_mx[kSWaves + wave]), fp16 bits
  uint32_t* s_mx = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(s_lds) + short_mx_offset(kv_len));

  const int tid = threadIdx.x;
  const int nh = Hkv * G;   // query heads of this call per batch entry
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31;
  const int j = lane >> 5;
  const int hh = blockIdx.x;
  if (hh >= n_heads) return;
  const int off = kv_len - Sq;   // >= 0 whenever CAUSAL
  const int nq = lk8 / 4;        // V token quads
  const int nblk = (Sq + 31) / 32;
  // row blocks of this wave: rbw + 4 bi (bi < kSBlocks); which wave takes a
  // head's odd block rotates with the head
  const int rbw = (wave + hh) & (kSWaves - 1);

  int b, hq;
  int64_t kvrow0;
  {
    b = hh / nh;
    const int h = hh - b * nh;   // query head of this call: KV head h / G of the cache
    const int g = h / G;
    hq = kv_heads ? min(max(kv_heads[g], 0), Hkv_all - 1) * G + (h - g * G) : h;
    kvrow0 = ((int64_t)b * Hkv + g) * C;
  }
  const uint16_t* qhead = q + ((int64_t)b * Hq + hq) * Sq * D;

  // ---- raw loads (zeros past kv_len and past Sq): K task i = dword i % 8 of
  // row i / 8 (8 tasks per thread cover 256 rows); V task i = token quad
  // u = (i % 16) + 16 (i / 128), dword w = (i / 16) % 8, i.e. dword w of
  // tokens 4u .. 4u + 3 (3 tasks: 384 tokens); the queries of one row block,
  // loaded when the block starts (the first block's with the keys), so that
  // no block's raw queries stay live through another block's loop
  uint4v qraw[D / 16];
  auto load_q = [&](int rb) {
    const int row = 32 * rb + r;
    if (row < Sq) {
      const uint16_t* qr = qhead + (int64_t)row * D;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) qraw[s] = *reinterpret_cast<const uint4v*>(qr + 8 * (2 * s + j));
    } else {
#pragma unroll
      for (int s = 0; s < D / 16; ++s) qraw[s] = uint4v{0u, 0u, 0u, 0u};
    }
  };
  uint32_t kraw[8];
  uint32_t vraw[3][4];
  uint32_t ksc, vsc0;
  {
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
  }
  load_q(rbw);

  // ---- K and V scale maxima of the head: |K| in bits 16-30, |V| in bits 0-14
  {
    const uint32_t kv = ((ksc & 0x7FFFu) << 16) | (vsc0 & 0x7FFFu);
    const uint32_t kvk = bitcast<uint32_t>(wave_max_nonneg(bitcast<float>(kv & 0x7FFF0000u)));
    const uint32_t kvv = bitcast<uint32_t>(wave_max_nonneg(bitcast<float>(kv & 0x7FFFu)));
    if (lane == 0) {
      s_mx[wave] = kvk >> 16;
      s_mx[kSWaves + wave] = kvv;
    }
  }
  // ---- conversion into LDS
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int i = tid + it * nth;
    if (i < lk8 * 8) {
      const int t = i >> 3, w = i & 7;
      *reinterpret_cast<uint4v*>(sK + t * D + 8 * (w ^ ((t >> 1) & 7))) = unpack8_bf16(kraw[it]);
    }
  }
#pragma unroll
  for (int it = 0; it < 3; ++it) {
    const int i = tid + it * nth;
    const int u = (i & 15) | ((i >> 7) << 4), w = (i >> 4) & 7;
    if (u < nq) {
      const int us = group_slot(u, nq);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const half2v a = nib_pair2(vraw[it][0], vraw[it][1], n);
        const half2v c2 = nib_pair2(vraw[it][2], vraw[it][3], n);
        const uint2v x = {bitcast<uint32_t>(a), bitcast<uint32_t>(c2)};
        *reinterpret_cast<uint2v*>(sV + (8 * w + n) * sv + 4 * us) = x;
      }
    }
  }
  __syncthreads();
  uint32_t km = 0, vm = 0;
#pragma unroll
  for (int w = 0; w < kSWaves; ++w) {
    km = max(km, s_mx[w]);
    vm = max(vm, s_mx[kSWaves + w]);
  }
  km = __builtin_amdgcn_readfirstlane(km);
  vm = __builtin_amdgcn_readfirstlane(vm);
  if (tid < lk32) csk[tid] = f16bits_to_f32((uint16_t)ksc) * qk_log2;
  if (tid < lk8) svh[4 * group_slot(tid >> 2, nq) + (tid & 3)] = bitcast<_Float16>((uint16_t)vsc0);
  __syncthreads();
  if (rbw >= nblk) return;   // no rows in this wave (after the last barrier)

  const float cmax = f16bits_to_f32((uint16_t)km) * qk_log2;   // max |K scale x qk_log2|
  const bool hilo = vm > pv_scale_limit_bits(pv_code_max(4, false));
  // rescale threshold of the hi/lo form: p <= 2^tau with 2^tau max s_V <= 2^15
  const float tau_hl = fminf(kSTau, fmaxf(0.0f, 15.0f - __log2f(f16bits_to_f32((uint16_t)vm))));
  // per-lane bases: K row r (chunk (2 s + j) ^ kx); V^T rows r and 32 + r and
  // the V-scale table at 8 j (complete 16-token groups) or 4 j (a partial
  // last group); K-scale table at 4 j
  const int kx = (r >> 1) & 7;
  const _Float16* krow = sK + r * D;
  const _Float16* vbase0 = sV + r * sv + 8 * j;
  const _Float16* vbase1 = vbase0 + 32 * sv;
  const _Float16* vbase0_p = vbase0 - 4 * j;
  const _Float16* vbase1_p = vbase1 - 4 * j;
  const float* cbase = csk + 4 * j;
  const _Float16* sbase = svh + 8 * j;
  const _Float16* sbase_p = sbase - 4 * j;

#pragma unroll
  for (int bi = 0; bi < kSBlocks; ++bi) {
    const int wrow_lo = 32 * (rbw + kSWaves * bi);
    if (wrow_lo >= Sq) break;   // uniform
    if (bi > 0) load_q(rbw + kSWaves * bi);
    const int row = wrow_lo + r;
    const int wrow_hi = min(wrow_lo + 31, Sq - 1);
    // key blocks of this row block: up to its last visible key
    const int last_key = CAUSAL ? min(kv_len - 1, wrow_hi + off) : kv_len - 1;
    const int nkb = last_key / 32 + 1;
    // blocks visible to all 32 rows and inside kv_len: no mask
    int nfull = kv_len / 32;
    if (CAUSAL) nfull = min(nfull, max(0, (wrow_lo + off + 1) / 32));
    nfull = min(nfull, nkb);

    // Query operand: the raw bf16 words of row `row`, dims 8 (2 s + j) .. + 7,
    // which is the K rows' order in LDS
    float16v o_acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o_acc[db] = float16v{};
    float m_ref = -INFINITY;   // row reference (log2 units), shared by lanes r and r + 32
    float m_use = 0.0f;        // m_ref, or 0 while the row has seen no key
    float l_run = 0.0f;        // this lane's share of sum(p), relative to m_ref

    // ---- S^T = K Q^T of key block kb: tokens 32 kb + r (lane) x 32 rows
    auto scores = [&](int kb, float16v& st) {
      st = float16v{};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const uint4v a = *reinterpret_cast<const uint4v*>(krow + 32 * kb * D + 8 * ((2 * s + j) ^ kx));
        st = mfma32x32x16_bf16(a, qraw[s], st);
      }
    };
    // ---- softmax and PV of key block kb, whose scores are st
    // FIRST: the row block's first key block, which sets the row references
    // (nothing accumulated yet to rescale)
    auto block = [&](int kb, float16v& st, auto full_c, auto hilo_c, auto first_c) {
      constexpr bool FULL = decltype(full_c)::value;
      constexpr bool HILO = decltype(hilo_c)::value;
      constexpr bool FIRST = decltype(first_c)::value;
      const int t0 = 32 * kb;
      // ---- online softmax; lane's tokens t0 + 8 vq + 4 j + i
      auto colf = [&](int vq) { return *reinterpret_cast<const float4v*>(cbase + t0 + 8 * vq); };
      const float tau = HILO ? tau_hl : kSTau;
      float mx;
      if constexpr (FULL && FIRST) {
        mx = -INFINITY;
      } else if constexpr (FULL) {
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
      if constexpr (FIRST) {
        if constexpr (FULL) {
#pragma unroll
          for (int vq = 0; vq < 4; ++vq) {
            const float4v c = colf(vq);
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[4 * vq + i] * c[i]);
          }
        }
        m_ref = xor_max(mx, 32);
        m_use = (m_ref == -INFINITY) ? 0.0f : m_ref;
      } else if (__builtin_amdgcn_ballot_w64(mx > m_ref + tau)) {
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
      // ---- P~ and O^T += V^T P~^T, 16 tokens per step.  Lane j's B operand is
      // P~ of tokens tt + 4 j + i and tt + 8 + 4 j + i (i < 4), its scores of
      // 8-token steps 2 hs and 2 hs + 1; V^T and the V-scale table hold each
      // complete 16-token group in that order, so each operand is one read.  A
      // step whose second half lies past kv_len (a masked block's partial last
      // group, stored in token order) runs its first half on the 8-token product.
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        const int tt = t0 + 16 * hs;
        if (!FULL && tt >= kv_len) break;               // uniform
        const bool part = !FULL && tt + 8 >= kv_len;   // uniform
        // keeps this step's LDS reads here: hoisted, both steps' column
        // factors, V scales and V operands would be live at once
        asm volatile("" ::: "memory");
        float p[8];
        auto exps = [&](int vq, float* pv) {
          if constexpr (FULL) {
            const float4v c = colf(vq);
#pragma unroll
            for (int i = 0; i < 4; ++i) pv[i] = fast_exp2(fmaf(st[4 * vq + i], c[i], -m_use));
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) pv[i] = fast_exp2(st[4 * vq + i] - m_use);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) l_run += pv[i];
        };
        // P~ of four tokens with V scales sv4: ph (high halves), pl (low halves, HILO)
        auto ptilde = [&](const float* pv, half4v sv4, half4v& ph, half4v& pl) {
          if constexpr (HILO) {   // high halves pinned, low halves about them
            const half2v h0 = pv_hi2(pv[0], (float)sv4[0], pv[1], (float)sv4[1]);
            const half2v h1 = pv_hi2(pv[2], (float)sv4[2], pv[3], (float)sv4[3]);
            ph = half4v{h0[0], h0[1], h1[0], h1[1]};
            pin_v(ph);
#pragma unroll
            for (int i = 0; i < 4; ++i) pl[i] = pv_lo(pv[i], (float)sv4[i], ph[i]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) ph[i] = (_Float16)fmaf(pv[i], (float)sv4[i], 0.0f);
          }
        };
        if (!part) {
          const half8v sv8 = *reinterpret_cast<const half8v*>(sbase + tt);
          exps(2 * hs, p);
          exps(2 * hs + 1, p + 4);
          half4v h0, l0, h1, l1;
          ptilde(p, half4v{sv8[0], sv8[1], sv8[2], sv8[3]}, h0, l0);
          ptilde(p + 4, half4v{sv8[4], sv8[5], sv8[6], sv8[7]}, h1, l1);
          const half8v ph = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const half8v a = *reinterpret_cast<const half8v*>((db ? vbase1 : vbase0) + tt);
            o_acc[db] = mfma32x32x16(a, ph, o_acc[db]);
            if constexpr (HILO) {
              const half8v pl = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
              o_acc[db] = mfma32x32x16(a, pl, o_acc[db]);
            }
          }
        } else {
          const half4v sv4 = *reinterpret_cast<const half4v*>(sbase_p + tt);
          exps(2 * hs, p);
          half4v ph, pl;
          ptilde(p, sv4, ph, pl);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const half4v a = *reinterpret_cast<const half4v*>((db ? vbase1_p : vbase0_p) + tt);
            o_acc[db] = mfma32x32x8(a, ph, o_acc[db]);
            if constexpr (HILO) o_acc[db] = mfma32x32x8(a, pl, o_acc[db]);
          }
        }
      }
    };
    using T_ = std::integral_constant<bool, true>;
    using F_ = std::integral_constant<bool, false>;
    // key block 0 first (nkb >= 1: every row sees key 0)
    if (!hilo) {
      {
        float16v st;
        scores(0, st);
        if (nfull > 0) block(0, st, T_{}, F_{}, T_{});
        else block(0, st, F_{}, F_{}, T_{});
      }
      int kb = 1;
      for (; kb < nfull; ++kb) {
        float16v st;
        scores(kb, st);
        block(kb, st, T_{}, F_{}, F_{});
      }
      for (; kb < nkb; ++kb) {
        float16v st;
        scores(kb, st);
        block(kb, st, F_{}, F_{}, F_{});
      }
    } else {
      for (int kb = 0; kb < nkb; ++kb) {
        float16v st;
        scores(kb, st);
        if (kb == 0) block(kb, st, F_{}, T_{}, T_{});
        else block(kb, st, F_{}, T_{}, F_{});
      }
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
  return D == kSD && bits == 4 && kv_len >= 1 && kv_len <= kSMaxKeys && Sq >= 1 && Sq <= 32 * kSWaves * kSBlocks;
}

hipError_t launch_prefill_short(const uint16_t* q, const uint8_t* kc, const uint16_t* ks, const uint8_t* vc,
                                const uint16_t* vs, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq,
                                int64_t kv_len, int64_t C, float softmax_scale, int causal, float* out,
                                float* lse, hipStream_t stream, const int32_t* kv_heads, int64_t Hkv_all) {
  const int Hall = (int)(kv_heads ? Hkv_all : Hkv);
  const int G = (int)(Hq / Hall);
  const int n_heads = (int)(B * Hkv * G);
  auto kern = causal ? prefill_short_kernel<true> : prefill_short_kernel<false>;
  // 256 keys take 66.5 KB of LDS: allow both variants more than 64 KB once
  static const hipError_t attr_nc = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_short_kernel<false>),
                                                        hipFuncAttributeMaxDynamicSharedMemorySize,
                                                        (int)short_lds_bytes(kSMaxKeys));
  static const hipError_t attr_c = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_short_kernel<true>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       (int)short_lds_bytes(kSMaxKeys));
  if (attr_nc != hipSuccess) return attr_nc;
  if (attr_c != hipSuccess) return attr_c;
  hipLaunchKernelGGL(kern, dim3(n_heads), dim3(64 * kSWaves), short_lds_bytes((int)kv_len), stream, q, kc, ks, vc,
                     vs, kv_heads, Hall, (int)Hq, (int)Hkv, G, (int)Sq, (int)kv_len, C, softmax_scale * kLog2e,
                     n_heads, out, lse);
  return hipGetLastError();
}

}  // namespace qkvfa
