// Device-side building blocks shared by the int4-KV attention kernels (gfx950).
//
// Exact int4 -> fp16 conversion.  The pages dequantize low-bit KV to FP16
// ("Quantized Cross-Attention: Extending FlashAttention-3 with In-SRAM
// Dequantization", §2.1 step 2, §3.1); here the *codes* are converted exactly
// and the per-token scales are applied to score columns (K) and folded into
// the softmax probabilities (V) instead of being multiplied into every element.
//
// Conversion: a two's-complement nibble c becomes the offset-binary value
// n = c + 8 in [0, 15] by flipping its top bit.  OR-ing n into the mantissa of
// an fp16 constant whose mantissa unit is 1 gives the exact value base + n:
//   bits 0-3  of a 16-bit half, base 1024 (0x6400): value 1024 + n
//   bits 4-7  of a 16-bit half, base   64 (0x5400): value   64 + n
// and one packed fp16 subtraction (1032 resp. 72) leaves exactly c.  Every
// step is exact (integers below 2048 are exact in fp16).  gfx950 fuses the
// flip/mask/or into one v_bitop3_b32, so two codes cost two VALU ops.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qkvfa {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef uint32_t uint4v __attribute__((ext_vector_type(4)));
typedef uint32_t uint2v __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& f) {
  static_assert(sizeof(To) == sizeof(From), "size mismatch");
  return __builtin_bit_cast(To, f);
}

// Codes held in bits 0-3 (low half) and 16-19 (high half) of x -> exact fp16 pair.
__device__ __forceinline__ half2v nib_lo_pair(uint32_t x) {
  const uint32_t y = ((x ^ 0x00080008u) & 0x000F000Fu) | 0x64006400u;
  const half2v bias = {(_Float16)1032.0f, (_Float16)1032.0f};
  return bitcast<half2v>(y) - bias;
}

// Codes held in bits 4-7 (low half) and 20-23 (high half) of x -> exact fp16 pair.
__device__ __forceinline__ half2v nib_hi_pair(uint32_t x) {
  const uint32_t y = ((x ^ 0x00800080u) & 0x00F000F0u) | 0x54005400u;
  const half2v bias = {(_Float16)72.0f, (_Float16)72.0f};
  return bitcast<half2v>(y) - bias;
}

// Eight codes of one packed dword (element i in bits 4i..4i+3) -> 8 exact fp16
// values in the order [c0, c4, c1, c5, c2, c6, c3, c7].  The matching query
// operand is permuted the same way (a dot product is order-invariant).
__device__ __forceinline__ half8v unpack8_perm(uint32_t x) {
  uint4v w;
  w[0] = bitcast<uint32_t>(nib_lo_pair(x));        // c0, c4
  w[1] = bitcast<uint32_t>(nib_hi_pair(x));        // c1, c5
  w[2] = bitcast<uint32_t>(nib_lo_pair(x >> 8));   // c2, c6
  w[3] = bitcast<uint32_t>(nib_hi_pair(x >> 8));   // c3, c7
  return bitcast<half8v>(w);
}

// Position of packed element e (0..7) in the unpack8_perm order, and back.
__host__ __device__ constexpr int perm8(int e) { return (e & 1) ? 4 + (e >> 1) : (e >> 1); }

// Byte k of dword a into bits 0-7 and byte k of dword b into bits 16-23
// (other bits zero): one v_perm_b32.  Selector bytes 0-3 pick bytes of the
// second operand, 4-7 bytes of the first, 12 gives 0x00.
__device__ __forceinline__ uint32_t pair_bytes(uint32_t a, uint32_t b, int k) {
  const uint32_t sel = (uint32_t)k | (12u << 8) | ((uint32_t)(4 + k) << 16) | (12u << 24);
  return __builtin_amdgcn_perm(b, a, sel);
}

// Nibble `nib` (0..7) of dword a and of dword b -> exact fp16 pair (a's, b's).
__device__ __forceinline__ half2v nib_pair2(uint32_t a, uint32_t b, int nib) {
  const uint32_t x = pair_bytes(a, b, nib >> 1);
  return (nib & 1) ? nib_hi_pair(x) : nib_lo_pair(x);
}

// 2- and 3-bit codes.  A 2-bit row packs element i into bits 2(i % 4) of
// byte i / 4; a 3-bit row is that 2-bit row of the low bits followed by one
// bit per element (element i at bit i % 8 of byte i / 8) holding the top
// (sign) bit.  The same magic-number conversion as for nibbles works for a
// 2-bit field f (bits 2f, 2f+1) with an fp16 whose mantissa unit puts weight
// 1 on bit 2f: 1024, 256, 64, 16 for f = 0..3.
__host__ __device__ constexpr uint32_t field_magic(int f) {
  return f == 0 ? 0x6400u : f == 1 ? 0x5C00u : f == 2 ? 0x5400u : 0x4C00u;
}
__host__ __device__ constexpr float field_base(int f) {
  return f == 0 ? 1024.0f : f == 1 ? 256.0f : f == 2 ? 64.0f : 16.0f;
}

// 2-bit field f of the bytes in bits 0-7 and 16-23 of x -> exact fp16 pair
// (two's complement codes -2..1; the sign flip makes them offset binary).
__device__ __forceinline__ half2v b2_pair(uint32_t x, int f) {
  const uint32_t m = field_magic(f);
  const uint32_t y = ((x ^ (0x00020002u << (2 * f))) & (0x00030003u << (2 * f))) | (m | (m << 16));
  const _Float16 bias = (_Float16)(field_base(f) + 2.0f);
  return bitcast<half2v>(y) - half2v{bias, bias};
}

// 3-bit code from the 2-bit field f of x (bytes in bits 0-7 and 16-23) and
// the top bits in bit f and bit 16 + f of z -> exact fp16 pair (codes -4..3).
// Offset binary n = c + 4 has the inverted top bit at field bit 2f + 2.
__device__ __forceinline__ half2v b3_pair(uint32_t x, uint32_t z, int f) {
  const uint32_t m = field_magic(f);
  const uint32_t lo = (x & (0x00030003u << (2 * f))) | (m | (m << 16));
  const uint32_t y = lo | ((~z << (f + 2)) & (0x00040004u << (2 * f)));
  const _Float16 bias = (_Float16)(field_base(f) + 4.0f);
  return bitcast<half2v>(y) - half2v{bias, bias};
}

// Bytes k and k + 1 of w into bits 0-7 and 16-23 (other bits zero).
__device__ __forceinline__ uint32_t spread_bytes(uint32_t w, int k) {
  const uint32_t sel = (uint32_t)k | (12u << 8) | ((uint32_t)(k + 1) << 16) | (12u << 24);
  return __builtin_amdgcn_perm(w, w, sel);
}

// Eight 2- or 3-bit codes -> 8 exact fp16 values in the unpack8_perm order
// [c0, c4, c1, c5, c2, c6, c3, c7].  lo16: the two bytes of their low bits
// (elements 0-3, 4-7); top8 (3-bit only): their top bits, element i at bit i.
template <int BITS>
__device__ __forceinline__ half8v unpack8_lowbit(uint32_t lo16, uint32_t top8) {
  const uint32_t x = spread_bytes(lo16, 0);
  uint4v w;
  if constexpr (BITS == 2) {
#pragma unroll
    for (int f = 0; f < 4; ++f) w[f] = bitcast<uint32_t>(b2_pair(x, f));
  } else {
    const uint32_t z = top8 | (top8 << 12);   // bits of elements f and 4 + f at f and 16 + f
#pragma unroll
    for (int f = 0; f < 4; ++f) w[f] = bitcast<uint32_t>(b3_pair(x, z, f));
  }
  return bitcast<half8v>(w);
}

// Element n (0..7) of eight 2- or 3-bit codes of two tokens a and b -> exact
// fp16 pair (a's, b's).  lo_a / lo_b: the tokens' two low-bit bytes in bits
// 0-15; top_a / top_b (3 bits only): their top-bit bytes in bits 0-7.
template <int BITS>
__device__ __forceinline__ half2v lowbit_pair2(uint32_t lo_a, uint32_t lo_b, uint32_t top_a, uint32_t top_b, int n) {
  const uint32_t x = pair_bytes(lo_a, lo_b, n >> 2);
  if constexpr (BITS == 2) {
    return b2_pair(x, n & 3);
  } else {
    const uint32_t z = pair_bytes(top_a, top_b, 0) >> (4 * (n >> 2));   // elements 4 (n/4) + f at f, 16 + f
    return b3_pair(x, z, n & 3);
  }
}

// ---- Biased conversions (decode).  A code c becomes the exact fp16 value
// c + b, with a bias b fixed by the code's position in the operand; the
// kernel takes sum(q b) out of each score (through the accumulator's initial
// value) and b sum(P~) out of each output (once per wave), instead of
// subtracting b from every value: one VALU op per two codes fewer.  The
// biases stay below 80, so the fp32 sums they ride on lose nothing that
// matters.  An fp16 with the exponent of 64 (0x5400) has mantissa unit 1/16,
// so bits 4-7 of a half hold an integer of weight 1; with the exponent of 16
// (0x4C00) the unit is 1/64 and bits 6-9 do.

// Nibbles in bits 4-7 and 20-23 of x (two's complement) -> fp16 pair c + 72.
constexpr float kNibBias = 72.0f;
__device__ __forceinline__ uint32_t nib_b72(uint32_t x) {
  return ((x ^ 0x00800080u) & 0x00F000F0u) | 0x54005400u;
}

// Eight nibbles of a dword (element i in bits 4i..4i+3) -> c + 72 in the
// unpack8_perm order [c0, c4, c1, c5, c2, c6, c3, c7].
__device__ __forceinline__ half8v unpack8_perm_b(uint32_t x) {
  uint4v w;
  w[0] = nib_b72(x << 4);   // c0, c4
  w[1] = nib_b72(x);        // c1, c5
  w[2] = nib_b72(x >> 4);   // c2, c6
  w[3] = nib_b72(x >> 8);   // c3, c7
  return bitcast<half8v>(w);
}

// One v_bitop3_b32: bit 4a + 2b + c of the table T is the result bit for
// input bits a, b, c.
template <uint32_t T>
__device__ __forceinline__ uint32_t bitop3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, T);
}
constexpr uint32_t kAndXor = 0x6C;      // (a & c) ^ b
constexpr uint32_t kAndOr = 0xEA;       // (a & b) | c
constexpr uint32_t kNotAndOr = 0xAE;    // (~a & b) | c

// 2-bit field in bits 4-5 (and 20-21) -> c + 66; in bits 6-7 (22-23) -> c + 18.
// ((x ^ s) & m) | e with the sign bit s inside the mask m and the exponent e
// outside it is (x & m) ^ (s | e): one v_bitop3.
__device__ __forceinline__ uint32_t b2_at4(uint32_t x) {
  return bitop3<kAndXor>(x, 0x00200020u | 0x54005400u, 0x00300030u);
}
__device__ __forceinline__ uint32_t b2_at6(uint32_t x) {
  return bitop3<kAndXor>(x, 0x00800080u | 0x4C004C00u, 0x00C000C0u);
}
// 3-bit code: its low two bits in bits 4-5 of x and its top bit at bit 6 of
// zs (both halves alike) -> c + 68; low bits in 6-7, top bit at 8 -> c + 20.
// The top bit enters inverted (offset binary c + 4 = low + 4 (1 - top)).
__device__ __forceinline__ uint32_t b3_at4(uint32_t x, uint32_t zs) {
  return bitop3<kNotAndOr>(zs, 0x00400040u, bitop3<kAndOr>(x, 0x00300030u, 0x54005400u));
}
__device__ __forceinline__ uint32_t b3_at6(uint32_t x, uint32_t zs) {
  return bitop3<kNotAndOr>(zs, 0x01000100u, bitop3<kAndOr>(x, 0x00C000C0u, 0x4C004C00u));
}

// Bias of pair f (0..3) of a low-bit operand built by lowbit4_b.
template <int BITS>
__host__ __device__ constexpr float lowbit_bias(int f) {
  return BITS == 2 ? ((f & 1) ? 18.0f : 66.0f) : ((f & 1) ? 20.0f : 68.0f);
}

// Four pairs of 2- or 3-bit codes: the 2-bit fields f = 0..3 of the bytes in
// bits 0-7 and 16-23 of x (3 bits: their top bits at bits f and 16 + f of z)
// -> w[f] = fp16 pair c + lowbit_bias(f).
template <int BITS>
__device__ __forceinline__ uint4v lowbit4_b(uint32_t x, uint32_t z) {
  const uint32_t xs = x << 4;   // fields 0, 1 move to bits 4-5, 6-7
  uint4v w;
  if constexpr (BITS == 2) {
    w[0] = b2_at4(xs);
    w[1] = b2_at6(xs);
    w[2] = b2_at4(x);
    w[3] = b2_at6(x);
  } else {
    w[0] = b3_at4(xs, z << 6);
    w[1] = b3_at6(xs, z << 7);
    w[2] = b3_at4(x, z << 4);
    w[3] = b3_at6(x, z << 5);
  }
  return w;
}

// Eight 2- or 3-bit codes -> c + bias in the unpack8_perm order.  lo16: the
// two bytes of their low bits (elements 0-3, 4-7); top8 (3 bits only): their
// top bits, element i at bit i.
template <int BITS>
__device__ __forceinline__ half8v unpack8_lowbit_b(uint32_t lo16, uint32_t top8) {
  const uint32_t z = BITS == 3 ? (top8 | (top8 << 12)) : 0u;   // elements f, 4 + f at bits f, 16 + f
  return bitcast<half8v>(lowbit4_b<BITS>(spread_bytes(lo16, 0), z));
}

// ---- Asymmetric group-wise rows: unsigned nibbles u.  Each enters the
// matrix products as the exact fp16 value 79 - u: flipping all four bits
// gives 15 - u, OR-ed into bits 4-7 of 64 (one v_bitop3).  The kernel then
// starts each group's score accumulator at -(79 - z) Q_g and multiplies the
// result by -s; outputs subtract their sum from the group's sum(P~ (79 - z)).

// Unsigned nibbles in bits 4-7 and 20-23 of x -> fp16 pair 79 - u.
__device__ __forceinline__ uint32_t nib_n79(uint32_t x) {
  return ((x ^ 0x00F000F0u) & 0x00F000F0u) | 0x54005400u;
}

// Eight nibbles of a dword (element i in bits 4i..4i+3) -> 79 - u in the
// unpack8_perm order [u0, u4, u1, u5, u2, u6, u3, u7].
__device__ __forceinline__ half8v unpack8_n79(uint32_t x) {
  uint4v w;
  w[0] = nib_n79(x << 4);
  w[1] = nib_n79(x);
  w[2] = nib_n79(x >> 4);
  w[3] = nib_n79(x >> 8);
  return bitcast<half8v>(w);
}

// Unsigned nibbles u of asymmetric rows -> exact fp16 u - z.  Bits 0x6400 | u
// are the fp16 1024 + u and bits 0x5400 | u << 4 are 64 + u, so subtracting
// 1024 + z (bits 0x6400 | z) or 64 + z (bits 0x5400 | z << 4) leaves u - z
// exactly.  Eight nibbles of a dword with one zero point z, in the
// unpack8_perm order [u0, u4, u1, u5, u2, u6, u3, u7] (minus z).
__device__ __forceinline__ half8v unpack8_uz(uint32_t x, uint32_t z) {
  const half2v blo = bitcast<half2v>((0x6400u | z) * 0x00010001u);
  const half2v bhi = bitcast<half2v>((0x5400u | (z << 4)) * 0x00010001u);
  uint4v w;
  w[0] = bitcast<uint32_t>(bitcast<half2v>((x & 0x000F000Fu) | 0x64006400u) - blo);
  w[1] = bitcast<uint32_t>(bitcast<half2v>((x & 0x00F000F0u) | 0x54005400u) - bhi);
  w[2] = bitcast<uint32_t>(bitcast<half2v>(((x >> 8) & 0x000F000Fu) | 0x64006400u) - blo);
  w[3] = bitcast<uint32_t>(bitcast<half2v>(((x >> 8) & 0x00F000F0u) | 0x54005400u) - bhi);
  return bitcast<half8v>(w);
}

// Nibble `nib` (0..7) of dwords a and b (unsigned codes) -> fp16 pair
// (u_a - za, u_b - zb), exact.
__device__ __forceinline__ half2v uz_pair2(uint32_t a, uint32_t b, int nib, uint32_t za, uint32_t zb) {
  const uint32_t x = pair_bytes(a, b, nib >> 1);
  if (nib & 1) {
    const uint32_t bias = (0x5400u | (za << 4)) | ((0x5400u | (zb << 4)) << 16);
    return bitcast<half2v>((x & 0x00F000F0u) | 0x54005400u) - bitcast<half2v>(bias);
  }
  const uint32_t bias = (0x6400u | za) | ((0x6400u | zb) << 16);
  return bitcast<half2v>((x & 0x000F000Fu) | 0x64006400u) - bitcast<half2v>(bias);
}

// fp32 pair -> packed fp16, round to nearest even (v_cvt_pk_f16_f32 on gfx950).
__device__ __forceinline__ half2v cvt_pk_f16(float a, float b) {
  half2v r;
  r[0] = (_Float16)a;
  r[1] = (_Float16)b;
  return r;
}

// ---- Precision of the PV operand.  P~ = fp16(p s_V) is rounded once, with
// relative error at most 2^-11.  An output is sum_j P~_j c_j / l with
// l = sum_j p_j (unrounded), so its rounding error is at most
// 2^-11 sum_j p_j s_V,j |c_j| / l <= 2^-11 cmax max_j s_V,j, where cmax is the
// largest code magnitude of a row with a normal fp16 scale (7 for int4 rows,
// 3 and 1 for 3- and 2-bit rows; a row with a subnormal scale has values
// below 2^-11 and adds nothing that matters).  An asymmetric group's codes
// satisfy |u - z| <= max(z, 15 - z), so its bound is 2^-11 s max(z, 15 - z)
// (asym_needs_hilo).
// Where a tile (decode: a wave's 32-token chunk) holds a V scale above
// pv_scale_limit(cmax), so that bound would pass kPvErrBudget, the kernels
// take P~ as two fp16 terms instead, hi = fp16(p s_V) and lo = fp16(p s_V -
// hi) (the residual is exact in fp32), and run the PV products for both:
// error at most 2^-22 relative.  Rows of moderate magnitude (every N(0, 1)
// workload) never take that branch.
constexpr float kPvErrBudget = 3.5e-3f;
__host__ __device__ constexpr float pv_scale_limit(int cmax) { return kPvErrBudget * 2048.0f / (float)cmax; }
__host__ __device__ constexpr int pv_code_max(int bits, bool asym) {
  return asym ? 15 : bits == 4 ? 7 : bits == 3 ? 3 : 1;
}
// The same limit as fp16 bits: a non-negative fp16 compares as its bit pattern.
__host__ __device__ constexpr uint32_t pv_scale_limit_bits(int cmax) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)pv_scale_limit(cmax));
}
// An asymmetric parameter word (fp16 scale s in bits 0-15, zero point z in
// bits 16-19): s max(z, 15 - z), the group's largest |value| -- past
// kPvErrBudget x 2^11 (7.168) one rounding of P~_g could cost more than the
// budget.  (s between 0.478 at z = 0 or 15 and 0.896 at z = 7 or 8.)
__device__ __forceinline__ float asym_value_max(uint32_t w) {
  const uint32_t z = (w >> 16) & 15u;
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0x7FFFu)) * (float)(z > 7u ? z : 15u - z);
}
__device__ __forceinline__ bool asym_needs_hilo(uint32_t w) { return asym_value_max(w) > kPvErrBudget * 2048.0f; }

// The low half of P~ about the high half hi that the PV product uses:
// fp16(p s - hi), the residual formed exactly by the fma.  hi must be the
// register the product reads: the callers pin it (pin_v) first, because the
// compiler may otherwise form hi again with another instruction (an fp16 fma
// rounds the product once, an fp32 product converted to fp16 twice), and
// where the product lies on an fp16 rounding midpoint the two differ by an ulp.
__device__ __forceinline__ _Float16 pv_lo(float p, float s, _Float16 hi) { return (_Float16)fmaf(p, s, -(float)hi); }
template <typename T>
__device__ __forceinline__ void pin_v(T& x) { asm volatile("" : "+v"(x)); }
// The high half by one fixed sequence, for code that forms it in two places:
// the fp32 product (opaque to the compiler, so it is not fused into an fp16
// fma), then one conversion to fp16 (round to nearest even).
__device__ __forceinline__ _Float16 pv_hi(float p, float s) {
  float x = p * s;
  pin_v(x);
  return (_Float16)x;
}
// Two high halves at once (one packed conversion).
__device__ __forceinline__ half2v pv_hi2(float p0, float s0, float p1, float s1) {
  float2v x = {p0 * s0, p1 * s1};
  pin_v(x);
  return cvt_pk_f16(x[0], x[1]);
}

// ---- Query range.  Q (bf16) enters the MFMAs as fp16, exact for magnitudes
// in [2^-14, 65536) (bf16 keeps 8 significand bits, fp16 11).  Rows of a
// workgroup with a larger element are multiplied by 2^-k first (exact), k the
// smallest shift that brings the workgroup's largest |q| below 65536, and the
// score scale by 2^k, so the scores do not change.  |bf16 bits| of the
// largest element -> k (0 for every element below 65536).
__device__ __forceinline__ int q_range_shift(uint32_t max_abs_bits) {
  const int e = (int)(max_abs_bits >> 7);   // biased bf16 exponent
  return e > 142 ? e - 142 : 0;
}
// 2^n as an fp32 (|n| < 127)
__device__ __forceinline__ float exp2i(int n) { return __builtin_bit_cast(float, (uint32_t)(127 + n) << 23); }
// Largest |bf16| bit pattern of the eight elements in a 16-byte word.
__device__ __forceinline__ uint32_t bf16x8_max_abs_bits(const uint4v& w) {
  uint32_t m = 0;
#pragma unroll
  for (int t = 0; t < 4; ++t) m = max(m, max(w[t] & 0x7FFFu, (w[t] >> 16) & 0x7FFFu));
  return m;
}

// Raw buffer descriptor over [base, base + num_bytes): loads at offsets past
// num_bytes return zero instead of touching memory (gfx9-family raw buffer
// range check; the fourth descriptor word selects 32-bit data format).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, num_bytes, 0x00020000);
}

// Row quantization, one fp16 scale per row of D values x (the arithmetic of
// every kernel that writes cache rows, so all of them agree bit for bit):
//   scale = fp16_rne(max|x| / 7)    (IEEE fp32 division, then one rounding)
//   code  = clamp(rint(x / float(scale)), -8, 7) as a 4-bit two's complement
//           nibble (IEEE fp32 division, round half to even); a zero scale
//           gives zero codes.  These files are built without fast-math.
__device__ __forceinline__ _Float16 quant_scale(float amax) { return (_Float16)(amax / 7.0f); }
__device__ __forceinline__ uint32_t quant_code(float x, float scale) {
  const float c = fminf(fmaxf(rintf(x / scale), -8.0f), 7.0f);
  return (uint32_t)(int)c & 0xFu;
}

// INT8 decode-buffer code under a universal scale: clamp(rint(x / s8), -127,
// 127) by IEEE fp32 division (outliers clamp to the range end); s8 = 0 gives 0.
__device__ __forceinline__ int quant_code8(float x, float s8) {
  if (s8 == 0.0f) return 0;
  return (int)fminf(fmaxf(rintf(x / s8), -127.0f), 127.0f);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return bitcast<float>((uint32_t)b << 16);
}

__device__ __forceinline__ float f16bits_to_f32(uint16_t b) {
  return (float)bitcast<_Float16>(b);
}


__device__ __forceinline__ float4v mfma16x16x32(half8v a, half8v b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float16v mfma32x32x16(half8v a, half8v b, float16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave64 butterfly max / sum across lanes differing in bit `mask`.
// Maximum over the 64 lanes of a wave of a non-negative float (the integer
// order of the bit patterns is the float order for non-negative values),
// returned uniformly.  Prefix maxima inside each 16-lane row, then the row
// broadcasts carry them across rows; lane 63 ends with the wave maximum.
__device__ __forceinline__ float wave_max_nonneg(float x) {
  int v = bitcast<int>(x);
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false));  // row_shr:1
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false));  // row_shr:2
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false));  // row_shr:4
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false));  // row_shr:8
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return bitcast<float>(__builtin_amdgcn_readlane(v, 63));
}

// DPP move inside 16-lane rows of the wave: lanes whose 4-lane bank is in
// BANK (bit k: lanes 4k..4k+3 of each row) take src from the lane CTRL
// names, the others keep old.
template <int CTRL, int BANK>
__device__ __forceinline__ float dpp_mov(float old, float src) {
  return bitcast<float>(__builtin_amdgcn_update_dpp(bitcast<int>(old), bitcast<int>(src), CTRL, 0xF, BANK, false));
}

// Partner values v[l ^ mask] without an LDS round trip.  Across lane halves
// (mask 32) or 16-lane rows (mask 16): v_permlane32_swap / v_permlane16_swap
// (CDNA4) exchange them in one VALU instruction -- given two copies of v, the
// swap leaves one holding every lane pair's lower value and the other its
// upper value, so each lane gets the pair (v[l], v[l ^ mask]) in some order
// (max and sum are commutative, so the result equals a shuffle's).  Inside a
// row: DPP quad permutations (masks 1, 2), a rotation by 8 (mask 8), and two
// bank-masked row shifts by 4 (mask 4).
__device__ __forceinline__ void xor_pair(float v, int mask, float& lo, float& hi) {
  if (mask == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(bitcast<uint32_t>(v), bitcast<uint32_t>(v), false, false);
    lo = bitcast<float>((uint32_t)r[0]);
    hi = bitcast<float>((uint32_t)r[1]);
  } else if (mask == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(bitcast<uint32_t>(v), bitcast<uint32_t>(v), false, false);
    lo = bitcast<float>((uint32_t)r[0]);
    hi = bitcast<float>((uint32_t)r[1]);
  } else if (mask == 8) {
    lo = v;
    hi = dpp_mov<0x128, 0xF>(v, v);                        // row_ror:8
  } else if (mask == 4) {
    lo = v;
    hi = dpp_mov<0x114, 0xA>(dpp_mov<0x104, 0x5>(v, v), v);   // row_shl:4 on banks 0, 2; row_shr:4 on 1, 3
  } else if (mask == 2) {
    lo = v;
    hi = dpp_mov<0x4E, 0xF>(v, v);                         // quad_perm [2, 3, 0, 1]
  } else if (mask == 1) {
    lo = v;
    hi = dpp_mov<0xB1, 0xF>(v, v);                         // quad_perm [1, 0, 3, 2]
  } else {
    lo = v;
    hi = __shfl_xor(v, mask, 64);
  }
}
__device__ __forceinline__ float xor_max(float v, int mask) {
  float lo, hi;
  xor_pair(v, mask, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float xor_sum(float v, int mask) {
  float lo, hi;
  xor_pair(v, mask, lo, hi);
  return lo + hi;
}

}  // namespace qkvfa
