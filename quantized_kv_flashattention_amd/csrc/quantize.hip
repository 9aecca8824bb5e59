// Quantize-and-append: fp32 K or V rows -> packed int4 codes + one fp16 scale
// per (token, KV head), written into cache rows [pos, pos + T).
//
// Layout follows the kernel signature of "Quantized Cross-Attention:
// Extending FlashAttention-3 with In-SRAM Dequantization" §4.1 (codes
// [b, h, seq_kv, dim*bits/32 words], scales [b, h, seq_kv, dim/GROUP_SIZE])
// with bits = 4 and GROUP_SIZE = dim; tokens are quantized as they are
// produced (Open-TQ-Metal abstract) and appended to the cache (TurboAttention
// arXiv 2412.08585 §2.1).
//
// Per row: scale = fp16_rne(max|x| / 7) by IEEE fp32 division; each code is
// clamp(rint(x / float(scale)), -8, 7) by IEEE fp32 division (the default
// HIP float division is correctly rounded; this file must not be built with
// fast-math); a zero scale gives zero codes.
//
// Work split: one thread owns 8 consecutive elements (two 16-byte loads) and
// writes one dword of codes; D/8 threads share a row and reduce its absmax
// with cross-lane max.  The kernel is HBM-bound (4D bytes read, D/2 + 2
// written per row).
#include "qkvfa_device.hpp"
#include "qkvfa_internal.h"

namespace qkvfa {

// One launch may quantize two tensors (K and V of the same tokens): blocks
// [0, nblk) take the first, blocks [nblk, 2 nblk) the second.
struct QuantTarget {
  const float* src;
  uint8_t* codes;
  uint16_t* scales;
  // head map (heads != nullptr): cache head h of the h_cache heads per batch
  // entry takes the source rows of head heads[h] of h_src (ids clamped)
  const int32_t* heads;
  int h_cache, h_src;
};

// Row index of (batch x cache head) bh in the source tensor.
__device__ __forceinline__ int64_t src_bh(const QuantTarget& t, uint32_t bh) {
  if (t.heads == nullptr) return bh;
  const int64_t b = bh / (uint32_t)t.h_cache;
  const int h = (int)(bh - b * t.h_cache);
  return b * t.h_src + min(max(t.heads[h], 0), t.h_src - 1);
}

// The TPR = D/8 lanes of one row, each holding 8 consecutive elements x:
// the row's absmax (cross-lane), its fp16 scale, and this lane's dword of codes.
template <int D>
__device__ __forceinline__ void quantize_row_part(const float (&x)[8], int sub, uint8_t* codes_row,
                                                  uint16_t* scale_ptr) {
  constexpr int TPR = D / 8;
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));
#pragma unroll
  for (int o = TPR / 2; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, TPR));
  const _Float16 s16 = quant_scale(m);
  const float s = (float)s16;
  uint32_t packed = 0;
  if (s != 0.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) packed |= quant_code(x[i], s) << (4 * i);
  }
  reinterpret_cast<uint32_t*>(codes_row)[sub] = packed;
  if (sub == 0) *scale_ptr = bitcast<uint16_t>(s16);
}

template <int D>
__global__ __launch_bounds__(256) void quantize_append_kernel(QuantTarget t0, QuantTarget t1,
                                                              uint32_t nblk, int64_t T, int64_t C,
                                                              int64_t pos, uint32_t tblocks) {
  constexpr int TPR = D / 8;          // threads per row
  constexpr int RPB = 256 / TPR;      // rows per block
  const bool second = blockIdx.x >= nblk;
  const uint32_t blk = second ? blockIdx.x - nblk : blockIdx.x;
  const QuantTarget& tg = second ? t1 : t0;
  const float* __restrict__ src = tg.src;
  uint8_t* __restrict__ codes = tg.codes;
  uint16_t* __restrict__ scales = tg.scales;
  const uint32_t bh = blk / tblocks;
  const uint32_t tb = blk - bh * tblocks;
  const int sub = threadIdx.x % TPR;
  const int64_t t = (int64_t)tb * RPB + threadIdx.x / TPR;
  if (t >= T) return;  // whole TPR-lane groups leave together

  const float4* p = reinterpret_cast<const float4*>(src + (src_bh(tg, bh) * T + t) * D) + 2 * sub;
  const float4 a = p[0];
  const float4 b = p[1];
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  const int64_t row = (int64_t)bh * C + pos + t;
  quantize_row_part<D>(x, sub, codes + row * (D / 2), scales + row);
}

// 2- and 3-bit rows (the int4 rule widened: scale = fp16(max|x| / (2^(b-1) - 1)),
// codes clamp(rint(x / scale), -2^(b-1), 2^(b-1) - 1) by IEEE fp32 division).
// A lane's 8 consecutive elements become 16 low bits (element i at bit 2i) at
// byte 2 sub of the row, and for 3 bits one byte of top bits at D/4 + sub.
template <int D, int BITS>
__device__ __forceinline__ void quantize_row_part_lowbit(const float (&x)[8], int sub, uint8_t* codes_row,
                                                         uint16_t* scale_ptr) {
  constexpr int TPR = D / 8;
  constexpr float qmax = (float)((1 << (BITS - 1)) - 1);
  constexpr float qmin = -(float)(1 << (BITS - 1));
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));
#pragma unroll
  for (int o = TPR / 2; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, TPR));
  const _Float16 s16 = (_Float16)(m / qmax);
  const float s = (float)s16;
  uint32_t lo = 0, top = 0;
  if (s != 0.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c = (uint32_t)(int)fminf(fmaxf(rintf(x[i] / s), qmin), qmax);
      lo |= (c & 3u) << (2 * i);
      top |= ((c >> 2) & 1u) << i;
    }
  }
  reinterpret_cast<uint16_t*>(codes_row)[sub] = (uint16_t)lo;
  if constexpr (BITS == 3) codes_row[D / 4 + sub] = (uint8_t)top;
  if (sub == 0) *scale_ptr = bitcast<uint16_t>(s16);
}

template <int D, int BITS>
__global__ __launch_bounds__(256) void quantize_append_lowbit_kernel(QuantTarget t0, QuantTarget t1,
                                                                     uint32_t nblk, int64_t T, int64_t C,
                                                                     int64_t pos, uint32_t tblocks) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  constexpr int ROWB = D * BITS / 8;
  const bool second = blockIdx.x >= nblk;
  const uint32_t blk = second ? blockIdx.x - nblk : blockIdx.x;
  const QuantTarget& tg = second ? t1 : t0;
  const uint32_t bh = blk / tblocks;
  const uint32_t tb = blk - bh * tblocks;
  const int sub = threadIdx.x % TPR;
  const int64_t t = (int64_t)tb * RPB + threadIdx.x / TPR;
  if (t >= T) return;  // whole TPR-lane groups leave together
  const float4* p = reinterpret_cast<const float4*>(tg.src + (src_bh(tg, bh) * T + t) * D) + 2 * sub;
  const float4 a = p[0];
  const float4 b = p[1];
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  const int64_t row = (int64_t)bh * C + pos + t;
  quantize_row_part_lowbit<D, BITS>(x, sub, tg.codes + row * ROWB, tg.scales + row);
}

hipError_t launch_quantize_append_bits(const float* src, uint8_t* codes, uint16_t* scales,
                                       const float* src2, uint8_t* codes2, uint16_t* scales2,
                                       int64_t BH, int64_t T, int D, int64_t C, int64_t pos, int bits,
                                       hipStream_t stream, const int32_t* heads, int h_cache, int h_src) {
  if (bits == 4)
    return launch_quantize_append(src, codes, scales, src2, codes2, scales2, BH, T, D, C, pos, stream, heads,
                                  h_cache, h_src);
  if (T == 0) return hipSuccess;
  const int rpb = 256 / (D / 8);
  const int64_t tblocks = (T + rpb - 1) / rpb;
  const int64_t nblk = BH * tblocks;
  const int ntensors = src2 ? 2 : 1;
  if (nblk * ntensors > 0x7FFFFFFF || tblocks > 0xFFFFFFFFll) return hipErrorInvalidValue;
  const QuantTarget t0 = {src, codes, scales, heads, h_cache, h_src};
  const QuantTarget t1 = src2 ? QuantTarget{src2, codes2, scales2, heads, h_cache, h_src} : t0;
  const dim3 grid((uint32_t)(nblk * ntensors));
  const uint32_t nb = (uint32_t)nblk, tbk = (uint32_t)tblocks;
  if (D == 128 && bits == 2)
    quantize_append_lowbit_kernel<128, 2><<<grid, dim3(256), 0, stream>>>(t0, t1, nb, T, C, pos, tbk);
  else if (D == 128)
    quantize_append_lowbit_kernel<128, 3><<<grid, dim3(256), 0, stream>>>(t0, t1, nb, T, C, pos, tbk);
  else if (bits == 2)
    quantize_append_lowbit_kernel<64, 2><<<grid, dim3(256), 0, stream>>>(t0, t1, nb, T, C, pos, tbk);
  else
    quantize_append_lowbit_kernel<64, 3><<<grid, dim3(256), 0, stream>>>(t0, t1, nb, T, C, pos, tbk);
  return hipGetLastError();
}

// Asymmetric group-wise rows (TurboAttention §2.3: a scale and a zero point;
// "Quantized Cross-Attention" §4.1: one scale per group of consecutive
// elements).  Per group of g elements: lo = min(0, min x), hi = max(0, max x),
// scale = fp16((hi - lo) / 15), zero = clamp(rint(-lo / scale), 0, 15),
// code = clamp(rint(x / scale) + zero, 0, 15), all in IEEE fp32; a zero scale
// gives zero point 0 and zero codes.  The g/8 lanes of a group reduce its
// range; its first lane writes the parameter word (scale in bits 0-15, zero
// point in bits 16-19).  Codes are stored in the cache's row orders (the
// decode reads each matrix-product block from one group): a K row keeps
// chunk c = 4 k + j (elements 8c .. 8c+7) in dword (D/32) j + k; a V row keeps
// element 16 p + w in nibble p of dword w (D = 128), or in nibble
// p + 4 (w / 8) of dword w % 8 (D = 64).
struct AsymTarget {
  const float* src;
  uint8_t* codes;
  uint32_t* params;
  int v_order;   // 1: the V row order, 0: the K row order
};

template <int D>
__global__ __launch_bounds__(256) void quantize_append_asym_kernel(AsymTarget t0, AsymTarget t1, uint32_t nblk,
                                                                   int64_t T, int64_t C, int64_t pos,
                                                                   uint32_t tblocks, int lpg) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const bool second = blockIdx.x >= nblk;
  const uint32_t blk = second ? blockIdx.x - nblk : blockIdx.x;
  const AsymTarget& tg = second ? t1 : t0;
  const uint32_t bh = blk / tblocks;
  const uint32_t tb = blk - bh * tblocks;
  const int sub = threadIdx.x % TPR;
  const int64_t t = (int64_t)tb * RPB + threadIdx.x / TPR;
  if (t >= T) return;  // whole TPR-lane groups leave together
  const float4* p = reinterpret_cast<const float4*>(tg.src + ((int64_t)bh * T + t) * D) + 2 * sub;
  const float4 a = p[0];
  const float4 b = p[1];
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  float lo = 0.0f, hi = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    lo = fminf(lo, x[i]);
    hi = fmaxf(hi, x[i]);
  }
  for (int o = 1; o < lpg; o <<= 1) {   // the group's lanes are an aligned block of lpg
    lo = fminf(lo, __shfl_xor(lo, o, TPR));
    hi = fmaxf(hi, __shfl_xor(hi, o, TPR));
  }
  const _Float16 s16 = (_Float16)((hi - lo) / 15.0f);
  const float s = (float)s16;
  uint32_t packed = 0, z = 0;
  if (s != 0.0f) {
    const float zf = fminf(fmaxf(rintf(-lo / s), 0.0f), 15.0f);
    z = (uint32_t)zf;
#pragma unroll
    for (int i = 0; i < 8; ++i) packed |= (uint32_t)fminf(fmaxf(rintf(x[i] / s) + zf, 0.0f), 15.0f) << (4 * i);
  }
  const int64_t row = (int64_t)bh * C + pos + t;
  uint32_t* out = reinterpret_cast<uint32_t*>(tg.codes + row * (D / 2));
  if (tg.v_order) {
    // dword sub gathers nibble p from the lane holding element 16 p + sub
    // (D = 128) or 16 (p % 4) + 8 (p / 4) + sub (D = 64)
    uint32_t word = 0;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int src = D == 128 ? 2 * p + (sub >> 3) : 2 * (p & 3) + (p >> 2);
      const int nib = D == 128 ? (sub & 7) : sub;
      const uint32_t w = (uint32_t)__shfl((int)packed, src, TPR);
      word |= ((w >> (4 * nib)) & 15u) << (4 * p);
    }
    out[sub] = word;
  } else {
    out[(D / 32) * (sub & 3) + (sub >> 2)] = packed;   // chunk sub = 4 k + j -> dword (D/32) j + k
  }
  if ((sub & (lpg - 1)) == 0) tg.params[row * (D / (8 * lpg)) + sub / lpg] = (uint32_t)bitcast<uint16_t>(s16) | (z << 16);
}

hipError_t launch_quantize_append_asym(const float* src, uint8_t* codes, uint32_t* params,
                                       const float* src2, uint8_t* codes2, uint32_t* params2,
                                       int64_t BH, int64_t T, int D, int64_t C, int64_t pos, int group,
                                       hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int rpb = 256 / (D / 8);
  const int64_t tblocks = (T + rpb - 1) / rpb;
  const int64_t nblk = BH * tblocks;
  const int ntensors = src2 ? 2 : 1;
  if (nblk * ntensors > 0x7FFFFFFF || tblocks > 0xFFFFFFFFll) return hipErrorInvalidValue;
  const AsymTarget t0 = {src, codes, params, 0};
  const AsymTarget t1 = src2 ? AsymTarget{src2, codes2, params2, 1} : t0;
  const dim3 grid((uint32_t)(nblk * ntensors));
  if (D == 128)
    quantize_append_asym_kernel<128><<<grid, dim3(256), 0, stream>>>(t0, t1, (uint32_t)nblk, T, C, pos,
                                                                     (uint32_t)tblocks, group / 8);
  else
    quantize_append_asym_kernel<64><<<grid, dim3(256), 0, stream>>>(t0, t1, (uint32_t)nblk, T, C, pos,
                                                                    (uint32_t)tblocks, group / 8);
  return hipGetLastError();
}

// Flush of the INT8 decode buffer (TurboAttention §3.3: a full buffer is
// compressed to the low-bit cache format): buffered rows [0, T) of every
// (batch, KV head), dequantized as the fp32 product s8 * code, are quantized
// as int4 rows into cache rows [pos, pos + T).  Blocks [0, nblk) take K,
// [nblk, 2 nblk) V.
struct FlushTarget {
  const int8_t* buf;     // [BH, buf_rows, D]
  const float* s8;       // [BH]
  uint8_t* codes;        // [BH, C, D/2]
  uint16_t* scales;      // [BH, C]
};

template <int D>
__global__ __launch_bounds__(256) void buffer_flush_kernel(FlushTarget t0, FlushTarget t1, uint32_t nblk,
                                                           int64_t T, int64_t buf_rows, int64_t C, int64_t pos,
                                                           uint32_t tblocks) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const bool second = blockIdx.x >= nblk;
  const uint32_t blk = second ? blockIdx.x - nblk : blockIdx.x;
  const FlushTarget& tg = second ? t1 : t0;
  const uint32_t bh = blk / tblocks;
  const uint32_t tb = blk - bh * tblocks;
  const int sub = threadIdx.x % TPR;
  const int64_t t = (int64_t)tb * RPB + threadIdx.x / TPR;
  if (t >= T) return;  // whole TPR-lane groups leave together
  const float s8 = tg.s8[bh];
  const uint2 c = *reinterpret_cast<const uint2*>(tg.buf + ((int64_t)bh * buf_rows + t) * D + 8 * sub);
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = s8 * (float)(int8_t)(c.x >> (8 * i));
    x[4 + i] = s8 * (float)(int8_t)(c.y >> (8 * i));
  }
  const int64_t row = (int64_t)bh * C + pos + t;
  quantize_row_part<D>(x, sub, tg.codes + row * (D / 2), tg.scales + row);
}

hipError_t launch_buffer_flush(const int8_t* k_buf, const int8_t* v_buf, const float* k_s8, const float* v_s8,
                               uint8_t* k_codes, uint16_t* k_scales, uint8_t* v_codes, uint16_t* v_scales,
                               int64_t BH, int64_t T, int64_t buf_rows, int D, int64_t C, int64_t pos,
                               hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int rpb = 256 / (D / 8);
  const int64_t tblocks = (T + rpb - 1) / rpb;
  const int64_t nblk = BH * tblocks;
  if (2 * nblk > 0x7FFFFFFF) return hipErrorInvalidValue;
  const FlushTarget t0 = {k_buf, k_s8, k_codes, k_scales};
  const FlushTarget t1 = {v_buf, v_s8, v_codes, v_scales};
  const dim3 grid((uint32_t)(2 * nblk));
  if (D == 128)
    buffer_flush_kernel<128><<<grid, dim3(256), 0, stream>>>(t0, t1, (uint32_t)nblk, T, buf_rows, C, pos,
                                                             (uint32_t)tblocks);
  else
    buffer_flush_kernel<64><<<grid, dim3(256), 0, stream>>>(t0, t1, (uint32_t)nblk, T, buf_rows, C, pos,
                                                            (uint32_t)tblocks);
  return hipGetLastError();
}

// Universal INT8 scale of the decode buffer (TurboAttention §3.3 and §5: the
// previous cache's value-range maximum; newer values beyond it are clamped):
// s8 = (7 * max_t s4[t]) / 127 over cache rows [0, L) of every (batch, KV
// head), with 7 * s4 (an fp16 value times 7, exact in fp32) the row's absmax
// as its int4 scale records it.  One 256-thread workgroup per (batch, KV
// head) and tensor, four independent loads in flight per thread.
__global__ __launch_bounds__(256) void buffer_scale_kernel(const uint16_t* k_scales, const uint16_t* v_scales,
                                                           float* k_s8, float* v_s8, int64_t BH, int64_t L,
                                                           int64_t C) {
  __shared__ float s_m[4];
  const int64_t w = blockIdx.x;          // [0, BH): K, [BH, 2 BH): V
  const bool isv = w >= BH;
  const int64_t bh = isv ? w - BH : w;
  const uint16_t* sc = (isv ? v_scales : k_scales) + bh * C;
  float m = 0.0f;   // scales are non-negative
  for (int64_t t0 = threadIdx.x; t0 < L; t0 += 4 * 256) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t t = t0 + u * 256;
      v[u] = t < L ? (float)bitcast<_Float16>(sc[t]) : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) m = fmaxf(m, v[u]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) s_m[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
    (isv ? v_s8 : k_s8)[bh] = (m * 7.0f) / 127.0f;
  }
}

hipError_t launch_buffer_scale(const uint16_t* k_scales, const uint16_t* v_scales, float* k_s8, float* v_s8,
                               int64_t BH, int64_t L, int64_t C, hipStream_t stream) {
  if (2 * BH > 0x7FFFFFFF) return hipErrorInvalidValue;
  buffer_scale_kernel<<<dim3((uint32_t)(2 * BH)), dim3(256), 0, stream>>>(k_scales, v_scales, k_s8, v_s8, BH, L,
                                                                           C);
  return hipGetLastError();
}

hipError_t launch_quantize_append(const float* src, uint8_t* codes, uint16_t* scales,
                                  const float* src2, uint8_t* codes2, uint16_t* scales2,
                                  int64_t BH, int64_t T, int D, int64_t C, int64_t pos,
                                  hipStream_t stream, const int32_t* heads, int h_cache, int h_src) {
  if (T == 0) return hipSuccess;
  const int rpb = 256 / (D / 8);
  const int64_t tblocks = (T + rpb - 1) / rpb;
  const int64_t nblk = BH * tblocks;
  const int ntensors = src2 ? 2 : 1;
  if (nblk * ntensors > 0x7FFFFFFF || tblocks > 0xFFFFFFFFll) return hipErrorInvalidValue;
  const QuantTarget t0 = {src, codes, scales, heads, h_cache, h_src};
  const QuantTarget t1 = src2 ? QuantTarget{src2, codes2, scales2, heads, h_cache, h_src} : t0;
  const dim3 grid((uint32_t)(nblk * ntensors));
  if (D == 128) {
    quantize_append_kernel<128><<<grid, dim3(256), 0, stream>>>(t0, t1, (uint32_t)nblk, T, C, pos,
                                                                (uint32_t)tblocks);
  } else {
    quantize_append_kernel<64><<<grid, dim3(256), 0, stream>>>(t0, t1, (uint32_t)nblk, T, C, pos,
                                                               (uint32_t)tblocks);
  }
  return hipGetLastError();
}

}  // namespace qkvfa
