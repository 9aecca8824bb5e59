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
};

template <int D>
__global__ __launch_bounds__(256) void quantize_append_kernel(QuantTarget t0, QuantTarget t1,
                                                              uint32_t nblk, int64_t T, int64_t C,
                                                              int64_t pos, uint32_t tblocks) {
  constexpr int TPR = D / 8;          // threads per row
  constexpr int RPB = 256 / TPR;      // rows per block
  const bool second = blockIdx.x >= nblk;
  const uint32_t blk = second ? blockIdx.x - nblk : blockIdx.x;
  const float* __restrict__ src = second ? t1.src : t0.src;
  uint8_t* __restrict__ codes = second ? t1.codes : t0.codes;
  uint16_t* __restrict__ scales = second ? t1.scales : t0.scales;
  const uint32_t bh = blk / tblocks;
  const uint32_t tb = blk - bh * tblocks;
  const int sub = threadIdx.x % TPR;
  const int64_t t = (int64_t)tb * RPB + threadIdx.x / TPR;
  if (t >= T) return;  // whole TPR-lane groups leave together

  const float4* p = reinterpret_cast<const float4*>(src + ((int64_t)bh * T + t) * D) + 2 * sub;
  const float4 a = p[0];
  const float4 b = p[1];
  float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};

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
  const int64_t row = (int64_t)bh * C + pos + t;
  reinterpret_cast<uint32_t*>(codes + row * (D / 2))[sub] = packed;
  if (sub == 0) scales[row] = bitcast<uint16_t>(s16);
}

hipError_t launch_quantize_append(const float* src, uint8_t* codes, uint16_t* scales,
                                  const float* src2, uint8_t* codes2, uint16_t* scales2,
                                  int64_t BH, int64_t T, int D, int64_t C, int64_t pos,
                                  hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int rpb = 256 / (D / 8);
  const int64_t tblocks = (T + rpb - 1) / rpb;
  const int64_t nblk = BH * tblocks;
  const int ntensors = src2 ? 2 : 1;
  if (nblk * ntensors > 0x7FFFFFFF || tblocks > 0xFFFFFFFFll) return hipErrorInvalidValue;
  const QuantTarget t0 = {src, codes, scales};
  const QuantTarget t1 = src2 ? QuantTarget{src2, codes2, scales2} : t0;
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
