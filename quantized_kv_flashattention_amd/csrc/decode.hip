// Split-K decode attention over an int4 KV cache, with log-sum-exp merge.
//
// Each of the G*Sq query rows of a GQA group attends cache rows [0, kv_len)
// (append-then-attend decode, TurboAttention arXiv 2412.08585 §2.1).  The KV
// length is cut into ranges ("splits"); each workgroup streams the packed
// int4 K/V codes of one (split, KV head, batch) straight from HBM with
// coalesced loads, converts the codes exactly to fp16 in registers (no
// dequantized K/V is ever written anywhere: "Quantized Cross-Attention ..."
// §3.1), and runs an online softmax (FlashAttention, TurboAttention §2.2).
// The KV tile of a head is read once for all G query heads of its group.
//
// Contractions run on MFMA v_mfma_f32_16x16x32_f16.  The score tile is
// computed transposed, S^T = K Q^T (M = 16 tokens, N = 16 query rows, K = 32
// head dims), so the packed K rows load directly as the A operand; the
// output is accumulated transposed too, O^T += V^T P^T (M = 16 head dims,
// N = 16 query rows, K = 32 tokens).  The per-token K scale multiplies score
// columns; the per-token V scale is folded into P before its fp16 rounding
// ("softmax in quantized space", same page §3.4, in the reading that keeps
// the result exact).  Scores live in log2 units (softmax_scale * log2 e is
// folded into the column scale) so the exponential is a single v_exp_f32.
//
// Lane roles inside a wave (lane = 16 j + r):
//   score tile   : lane holds query row r and tokens 8j + 4kb + i (kb, i in 0..3)
//   K operand    : lane loads token 8(r/4) + 4kb + r%4, bytes [16j, 16j+16) (D=128)
//   V operand    : lane loads dword r of tokens 8j .. 8j+7 of the 32-token chunk
//   output O^T   : lane holds query row r, head dims 32j .. 32j+31 (D=128)
// so a lane's eight probabilities are exactly the eight tokens of its V dwords
// and no data moves between lanes except the row max (two butterflies).
//
// After the loop the four waves of a workgroup merge their (m, l, O) through
// LDS; a workgroup writes the normalized partial O_s and lse_s of its split,
// and a second kernel merges splits in split order (deterministic).
#include <math.h>

#include "qkvfa_device.hpp"
#include "qkvfa_internal.h"

namespace qkvfa {

namespace {

constexpr int kWaves = 4;
constexpr int kChunk = 32;  // tokens per wave iteration

template <int D, int NB>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kc,
    const uint16_t* __restrict__ ks, const uint8_t* __restrict__ vc,
    const uint16_t* __restrict__ vs, int Hq, int Hkv, int G, int Sq, int kv_len, int64_t C,
    float qk_log2, int split_len, int n_split, float* __restrict__ out,
    float* __restrict__ lse_out, float* __restrict__ part_o, float* __restrict__ part_lse) {
  constexpr int KK = D / 32;    // QK MFMAs per 16-token block
  constexpr int DW = D / 8;     // dwords per packed row
  constexpr int NPB = D / 16;   // PV MFMAs (16 head dims each)
  constexpr int ROWB = D / 2;   // bytes per packed row
  constexpr int OSTR = D + 4;   // padded LDS row stride of the merge buffer (floats)

  __shared__ __align__(16) uint16_t s_scale[kWaves][64];
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  __shared__ __align__(16) float s_o[kWaves][16 * OSTR];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int j = lane >> 4;
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int R = G * Sq;
  const int t_begin = split * split_len;
  const int t_end = min(kv_len, t_begin + split_len);

  const int64_t kvrow0 = ((int64_t)b * Hkv + g) * C;
  const uint8_t* kbase = kc + kvrow0 * ROWB;
  const uint8_t* vbase = vc + kvrow0 * ROWB;
  const uint16_t* ksb = ks + kvrow0;
  const uint16_t* vsb = vs + kvrow0;

  // Query operand (B of S^T = K Q^T): query row nb*16 + r, k = 8j + e <->
  // head dim 8*(KK*j + kk) + perm8(e), matching the K lane's dword order.
  half8v qop[NB][KK];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int row = nb * 16 + r;
    if (row < R) {
      const int hg = row / Sq;
      const int sq = row - hg * Sq;
      const uint16_t* qr = q + (((int64_t)b * Hq + g * G + hg) * Sq + sq) * D;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const uint4v w = *reinterpret_cast<const uint4v*>(qr + 8 * (KK * j + kk));
        uint16_t e16[8];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          e16[2 * t] = (uint16_t)(w[t] & 0xFFFFu);
          e16[2 * t + 1] = (uint16_t)(w[t] >> 16);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) qop[nb][kk][e] = (_Float16)bf16_to_f32(e16[perm8(e)]);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qop[nb][kk] = half8v{};
    }
  }

  float m_run[NB], l_run[NB];
  float4v o_acc[NB][NPB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_run[nb] = -INFINITY;
    l_run[nb] = 0.0f;
#pragma unroll
    for (int p = 0; p < NPB; ++p) o_acc[nb][p] = float4v{0.f, 0.f, 0.f, 0.f};
  }

  const int n_chunks = (t_end - t_begin + kChunk - 1) / kChunk;
  for (int c = wave; c < n_chunks; c += kWaves) {
    const int c0 = t_begin + c * kChunk;

    // ---- loads (token indices clamped into [0, kv_len) for memory safety;
    //      tokens >= t_end are masked below)
    uint32_t kw[2][KK];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int tok = min(c0 + 8 * (r >> 2) + 4 * kb + (r & 3), kv_len - 1);
      const uint8_t* p = kbase + (int64_t)tok * ROWB + (4 * KK) * j;
      if constexpr (KK == 4) {
        const uint4v w = *reinterpret_cast<const uint4v*>(p);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) kw[kb][kk] = w[kk];
      } else {
        const uint2v w = *reinterpret_cast<const uint2v*>(p);
        kw[kb][0] = w[0];
        kw[kb][1] = w[1];
      }
    }
    uint32_t vw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int tok = min(c0 + 8 * j + e, kv_len - 1);
      vw[e] = *reinterpret_cast<const uint32_t*>(vbase + (int64_t)tok * ROWB + 4 * (r % DW));
      if constexpr (D == 64) vw[e] = (r >= 8) ? (vw[e] >> 16) : vw[e];
    }
    {
      const int tok = min(c0 + (lane & 31), kv_len - 1);
      s_scale[wave][lane] = (lane < 32) ? ksb[tok] : vsb[tok];
    }
    // The LDS write above and the reads below are issued by the same wave and
    // execute in order; no barrier is needed.
    const uint4v ksc = *reinterpret_cast<const uint4v*>(&s_scale[wave][8 * j]);
    const uint4v vsc = *reinterpret_cast<const uint4v*>(&s_scale[wave][32 + 8 * j]);
    float csk[8], sv[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      csk[2 * t] = f16bits_to_f32((uint16_t)(ksc[t] & 0xFFFFu)) * qk_log2;
      csk[2 * t + 1] = f16bits_to_f32((uint16_t)(ksc[t] >> 16)) * qk_log2;
      sv[2 * t] = f16bits_to_f32((uint16_t)(vsc[t] & 0xFFFFu));
      sv[2 * t + 1] = f16bits_to_f32((uint16_t)(vsc[t] >> 16));
    }
    const bool full = (c0 + kChunk <= t_end);

    // ---- V operand: nibble p of the eight token dwords -> exact fp16 (token e = k index)
    half8v vop[NPB];
#pragma unroll
    for (int p = 0; p < NPB; ++p) {
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        const half2v pr = nib_pair2(vw[2 * hh], vw[2 * hh + 1], p);
        vop[p][2 * hh] = pr[0];
        vop[p][2 * hh + 1] = pr[1];
      }
    }

#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      // ---- scores S^T for 2 x 16 tokens
      float4v s_t[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) acc = mfma16x16x32(unpack8_perm(kw[kb][kk]), qop[nb][kk], acc);
        s_t[kb] = acc;
      }
      float x[8];
      float mloc = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = s_t[e >> 2][e & 3] * csk[e];
        if (!full) v = (c0 + 8 * j + e < t_end) ? v : -INFINITY;
        x[e] = v;
        mloc = fmaxf(mloc, v);
      }
      mloc = xor_max(mloc, 16);
      mloc = xor_max(mloc, 32);
      const float m_new = fmaxf(m_run[nb], mloc);   // finite: every chunk has a valid token
      const float alpha = fast_exp2(m_run[nb] - m_new);
      float lsum = 0.0f;
      half8v pop;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = fast_exp2(x[e] - m_new);
        const float p1 = fast_exp2(x[e + 1] - m_new);
        lsum += p0 + p1;
        const half2v pr = cvt_pk_f16(p0 * sv[e], p1 * sv[e + 1]);
        pop[e] = pr[0];
        pop[e + 1] = pr[1];
      }
      l_run[nb] = l_run[nb] * alpha + lsum;
      m_run[nb] = m_new;
      if (__ballot(alpha != 1.0f)) {
#pragma unroll
        for (int p = 0; p < NPB; ++p) o_acc[nb][p] *= alpha;
      }
      // ---- O^T += V^T P^T
#pragma unroll
      for (int p = 0; p < NPB; ++p) o_acc[nb][p] = mfma16x16x32(vop[p], pop, o_acc[nb][p]);
    }
  }

  // ---- merge the four waves through LDS, one 16-row block at a time
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float l = xor_sum(l_run[nb], 16);
    l = xor_sum(l, 32);
    if (j == 0) {
      s_m[wave][r] = m_run[nb];
      s_l[wave][r] = l;
    }
    float* orow = &s_o[wave][r * OSTR];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (D == 128) {
        // head dims 32j + 8i + p, p = 0..7
        float4v lo = {o_acc[nb][0][i], o_acc[nb][1][i], o_acc[nb][2][i], o_acc[nb][3][i]};
        float4v hi = {o_acc[nb][4][i], o_acc[nb][5][i], o_acc[nb][6][i], o_acc[nb][7][i]};
        *reinterpret_cast<float4v*>(orow + 32 * j + 8 * i) = lo;
        *reinterpret_cast<float4v*>(orow + 32 * j + 8 * i + 4) = hi;
      } else {
        // M-row m = 4j + i holds head dims 8(m%8) + 4(m/8) + p, p = 0..3
        const int m = 4 * j + i;
        float4v v4 = {o_acc[nb][0][i], o_acc[nb][1][i], o_acc[nb][2][i], o_acc[nb][3][i]};
        *reinterpret_cast<float4v*>(orow + 8 * (m & 7) + 4 * (m >> 3)) = v4;
      }
    }
    __syncthreads();
    const int rows_here = min(16, R - nb * 16);
    for (int idx = threadIdx.x; idx < rows_here * D; idx += 256) {
      const int rr = idx / D;
      const int d = idx - rr * D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][rr]);
      float acc = 0.0f, den = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float wt = fast_exp2(s_m[w][rr] - M);   // empty waves: exp2(-inf) = 0
        acc += wt * s_o[w][rr * OSTR + d];
        den += wt * s_l[w][rr];
      }
      const int row = nb * 16 + rr;
      const int hg = row / Sq;
      const int sq = row - hg * Sq;
      const int64_t grow = ((int64_t)b * Hq + g * G + hg) * Sq + sq;
      const float o = acc / den;
      const float lse2 = M + __log2f(den);
      if (n_split == 1) {
        out[grow * D + d] = o;
        if (d == 0 && lse_out) lse_out[grow] = lse2 * kLn2;
      } else {
        part_o[(grow * n_split + split) * D + d] = o;
        if (d == 0) part_lse[grow * n_split + split] = lse2;   // log2 units
      }
    }
    __syncthreads();
  }
}

// Merge split partials: O = sum_s w_s O_s / sum_s w_s, w_s = 2^(lse_s - max).
template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const float* __restrict__ part_o,
                                                         const float* __restrict__ part_lse,
                                                         int n_split, float* __restrict__ out,
                                                         float* __restrict__ lse_out) {
  const int64_t row = blockIdx.x;
  const int d = threadIdx.x;
  const float* pl = part_lse + row * n_split;
  float M = -INFINITY;
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, pl[s]);
  float acc = 0.0f, den = 0.0f;
  const float* po = part_o + row * n_split * D + d;
  for (int s = 0; s < n_split; ++s) {
    const float w = fast_exp2(pl[s] - M);
    acc += w * po[(int64_t)s * D];
    den += w;
  }
  out[row * D + d] = acc / den;
  if (d == 0 && lse_out) lse_out[row] = (M + __log2f(den)) * kLn2;
}

template <int D, int NB>
hipError_t launch_split(const uint16_t* q, const uint8_t* kc, const uint16_t* ks,
                        const uint8_t* vc, const uint16_t* vs, int64_t B, int64_t Hq,
                        int64_t Hkv, int64_t Sq, int64_t kv_len, int64_t C, float qk_log2,
                        const DecodePlan& plan, float* out, float* lse, float* part_o,
                        float* part_lse, hipStream_t stream) {
  dim3 grid((uint32_t)plan.n_split, (uint32_t)Hkv, (uint32_t)B);
  decode_split_kernel<D, NB><<<grid, dim3(256), 0, stream>>>(
      q, kc, ks, vc, vs, (int)Hq, (int)Hkv, (int)(Hq / Hkv), (int)Sq, (int)kv_len, C, qk_log2,
      plan.split_len, plan.n_split, out, lse, part_o, part_lse);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const uint16_t* q, const uint8_t* kc, const uint16_t* ks, const uint8_t* vc,
                    const uint16_t* vs, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq,
                    int64_t kv_len, int64_t C, float qk_log2, const DecodePlan& plan, float* out,
                    float* lse, float* part_o, float* part_lse, hipStream_t stream) {
  const int64_t R = (Hq / Hkv) * Sq;
  hipError_t err;
  if (R <= 16)
    err = launch_split<D, 1>(q, kc, ks, vc, vs, B, Hq, Hkv, Sq, kv_len, C, qk_log2, plan, out, lse,
                             part_o, part_lse, stream);
  else if (R <= 32)
    err = launch_split<D, 2>(q, kc, ks, vc, vs, B, Hq, Hkv, Sq, kv_len, C, qk_log2, plan, out, lse,
                             part_o, part_lse, stream);
  else
    err = launch_split<D, 4>(q, kc, ks, vc, vs, B, Hq, Hkv, Sq, kv_len, C, qk_log2, plan, out, lse,
                             part_o, part_lse, stream);
  if (err != hipSuccess || plan.n_split == 1) return err;
  const int64_t rows = B * Hq * Sq;
  decode_merge_kernel<D><<<dim3((uint32_t)rows), dim3(D), 0, stream>>>(part_o, part_lse,
                                                                        plan.n_split, out, lse);
  return hipGetLastError();
}

}  // namespace

DecodePlan plan_decode(int64_t B, int64_t Hkv, int64_t kv_len, int num_splits, int num_cus) {
  const int64_t chunks = (kv_len + kChunk - 1) / kChunk;
  const int64_t units = B * Hkv;
  int64_t ns;
  if (num_splits <= 0) {
    const int64_t target_wgs = 4 * (int64_t)(num_cus > 0 ? num_cus : 256);
    ns = (target_wgs + units - 1) / units;
    const int64_t max_ns = chunks / kWaves > 0 ? chunks / kWaves : 1;   // >= one chunk per wave
    if (ns > max_ns) ns = max_ns;
  } else {
    ns = num_splits;
  }
  if (ns > chunks) ns = chunks;
  if (ns > 1024) ns = 1024;
  if (ns < 1) ns = 1;
  const int64_t cps = (chunks + ns - 1) / ns;   // chunks per split
  DecodePlan p;
  p.split_len = (int)(cps * kChunk);
  p.n_split = (int)((chunks + cps - 1) / cps);   // no empty split
  return p;
}

size_t decode_workspace_bytes(int64_t rows, int D, int n_split) {
  if (n_split <= 1) return 0;
  const size_t o = (size_t)rows * n_split * D * sizeof(float);
  const size_t l = (size_t)rows * n_split * sizeof(float);
  return ((o + 255) / 256) * 256 + l;
}

hipError_t launch_decode(const uint16_t* q, const uint8_t* kc, const uint16_t* ks,
                         const uint8_t* vc, const uint16_t* vs, int64_t B, int64_t Hq,
                         int64_t Hkv, int64_t Sq, int64_t kv_len, int64_t C, int D,
                         float softmax_scale, const DecodePlan& plan, float* out, float* lse,
                         void* workspace, hipStream_t stream) {
  const float qk_log2 = softmax_scale * kLog2e;
  float* part_o = nullptr;
  float* part_lse = nullptr;
  if (plan.n_split > 1) {
    const int64_t rows = B * Hq * Sq;
    const size_t o = (size_t)rows * plan.n_split * D * sizeof(float);
    part_o = static_cast<float*>(workspace);
    part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + ((o + 255) / 256) * 256);
  }
  if (D == 128)
    return launch_d<128>(q, kc, ks, vc, vs, B, Hq, Hkv, Sq, kv_len, C, qk_log2, plan, out, lse,
                         part_o, part_lse, stream);
  return launch_d<64>(q, kc, ks, vc, vs, B, Hq, Hkv, Sq, kv_len, C, qk_log2, plan, out, lse, part_o,
                      part_lse, stream);
}

}  // namespace qkvfa
