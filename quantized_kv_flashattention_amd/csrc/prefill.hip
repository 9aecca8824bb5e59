// Tiled prefill attention over an int4 KV cache, causal or not.
//
// FlashAttention tiling with online softmax (TurboAttention arXiv 2412.08585
// §2.2): a workgroup owns 128 query rows of one head (4 waves x 32 rows) and
// walks the key axis in tiles of 64 tokens.  For each tile the workgroup
// loads the packed int4 K/V codes (8 KB at D = 128, the "quantized KV 8 KB +
// 256 B scales" tile of "Quantized Cross-Attention ..." §3.2) and converts
// them exactly to fp16 into LDS, where all four waves share them; the codes
// are never dequantized to HBM (same page §3.1).  Scales stay per token: the
// K scale multiplies score columns, the V scale is folded into P (§3.4 in
// the reading that keeps the result exact).
//
// Contractions use v_mfma_f32_32x32x16_f16 in transposed form:
//   S^T = K Q^T   (M = 32 tokens, N = 32 query rows, K = 16 head dims)
//   O^T += V^T P^T (M = 32 head dims, N = 32 query rows, K = 16 tokens)
// so every lane owns one query row: its 32 scores of a tile need a single
// cross-lane step for the row max, and its probabilities are already in the
// B-operand position of the PV product.
//
// Causal (bottom-right aligned, row i sees keys <= i + kv_len - Sq): key tiles
// beyond the last visible key of a workgroup are never loaded; only tiles
// crossing the diagonal (or the ragged end of the keys) evaluate the mask;
// waves whose rows see nothing of a tile skip its math.  Workgroups are
// dispatched longest-first (highest query block first).
#include <math.h>

#include "qkvfa_device.hpp"
#include "qkvfa_internal.h"

namespace qkvfa {

namespace {

constexpr int BM = 128;  // query rows per workgroup
constexpr int BN = 64;   // keys per tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void prefill_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kc,
    const uint16_t* __restrict__ ks, const uint8_t* __restrict__ vc,
    const uint16_t* __restrict__ vs, int Hq, int Hkv, int G, int Sq, int kv_len, int64_t C,
    float qk_log2, int nqb, float* __restrict__ out, float* __restrict__ lse_out) {
  constexpr int KS = D / 16;   // QK k-steps
  constexpr int NDB = D / 32;  // PV output blocks
  constexpr int NCH = D / 8;   // 16-byte chunks per LDS K row
  constexpr int ROWB = D / 2;  // bytes per packed row

  // K tile: [token][D] fp16, chunk c of token t stored at chunk c ^ (t % NCH).
  // V tile: transposed [D][BN] fp16, 4-token unit u of row d stored at u ^ (d % 16).
  __shared__ __align__(16) _Float16 s_k[BN * D];
  __shared__ __align__(16) _Float16 s_v[D * BN];
  __shared__ __align__(16) float s_csk[BN];
  __shared__ __align__(16) float s_sv[BN];

  const int h = blockIdx.x;
  const int qb = CAUSAL ? (nqb - 1 - (int)blockIdx.y) : (int)blockIdx.y;
  const int b = blockIdx.z;
  const int g = h / G;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 31;
  const int j = lane >> 5;
  const int q0 = qb * BM;
  const int qrow = q0 + wave * 32 + r;
  const int off = kv_len - Sq;  // >= 0 whenever CAUSAL

  int n_tiles = (kv_len + BN - 1) / BN;
  if (CAUSAL) {
    const int last_key = min(q0 + BM - 1, Sq - 1) + off;
    n_tiles = min(n_tiles, last_key / BN + 1);
  }
  const int wrow_lo = q0 + wave * 32;
  const int wrow_hi = min(wrow_lo + 31, Sq - 1);
  const bool wave_active = wrow_lo < Sq;

  // Query operand (B of S^T = K Q^T): row qrow, k = 8j + e <-> head dim
  // 8 * (2 ks + j) + perm8(e), matching the LDS K chunk 2 ks + j.
  half8v qop[KS];
  if (qrow < Sq) {
    const uint16_t* qr = q + (((int64_t)b * Hq + h) * Sq + qrow) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4v w = *reinterpret_cast<const uint4v*>(qr + 8 * (2 * s + j));
      uint16_t e16[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        e16[2 * t] = (uint16_t)(w[t] & 0xFFFFu);
        e16[2 * t + 1] = (uint16_t)(w[t] >> 16);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) qop[s][e] = (_Float16)bf16_to_f32(e16[perm8(e)]);
    }
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) qop[s] = half8v{};
  }

  float16v o_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o_acc[db] = float16v{};
  float m_run = -INFINITY;
  float l_run = 0.0f;

  const int64_t kvrow0 = ((int64_t)b * Hkv + g) * C;
  const uint8_t* kbase = kc + kvrow0 * ROWB;
  const uint8_t* vbase = vc + kvrow0 * ROWB;

  // Loader roles.  K: thread -> token tid/4, bytes [part*D/8, +D/8).
  // V (D=128): thread -> dword dp = tid%16 of tokens 4*(tid/16) .. +3.
  // V (D=64):  thread -> dword dp = tid%8  of tokens 2*(tid/8), +1.
  constexpr int VTOK = (D == 128) ? 4 : 2;
  const int k_tok = tid >> 2;
  const int k_part = tid & 3;
  const int v_dp = tid % (D / 8);
  const int v_tg = tid / (D / 8);
  uint32_t kreg[D / 32];
  uint32_t vreg[VTOK];
  uint16_t sreg = 0;

  auto load_tile = [&](int t0) {
    {
      const int tok = min(t0 + k_tok, kv_len - 1);
      const uint8_t* p = kbase + (int64_t)tok * ROWB + k_part * (D / 8);
      if constexpr (D == 128) {
        const uint4v w = *reinterpret_cast<const uint4v*>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) kreg[i] = w[i];
      } else {
        const uint2v w = *reinterpret_cast<const uint2v*>(p);
        kreg[0] = w[0];
        kreg[1] = w[1];
      }
    }
#pragma unroll
    for (int i = 0; i < VTOK; ++i) {
      const int tok = min(t0 + VTOK * v_tg + i, kv_len - 1);
      vreg[i] = *reinterpret_cast<const uint32_t*>(vbase + (int64_t)tok * ROWB + 4 * v_dp);
    }
    if (tid < 2 * BN) {
      const int tok = min(t0 + (tid & (BN - 1)), kv_len - 1);
      sreg = (tid < BN) ? ks[kvrow0 + tok] : vs[kvrow0 + tok];
    }
  };

  load_tile(0);
  for (int kt = 0; kt < n_tiles; ++kt) {
    const int t0 = kt * BN;
    __syncthreads();  // the previous tile's LDS reads are done
    // ---- codes -> exact fp16 in LDS
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      const int c = k_part * (D / 32) + i;
      const int pc = c ^ (k_tok & (NCH - 1));
      *reinterpret_cast<half8v*>(&s_k[k_tok * D + pc * 8]) = unpack8_perm(kreg[i]);
    }
#pragma unroll
    for (int nib = 0; nib < 8; ++nib) {
      const int d = 8 * v_dp + nib;
      if constexpr (D == 128) {
        const half2v a = nib_pair2(vreg[0], vreg[1], nib);
        const half2v bb = nib_pair2(vreg[2], vreg[3], nib);
        const int pu = v_tg ^ (d & 15);
        uint2v w = {bitcast<uint32_t>(a), bitcast<uint32_t>(bb)};
        *reinterpret_cast<uint2v*>(&s_v[d * BN + pu * 4]) = w;
      } else {
        const half2v a = nib_pair2(vreg[0], vreg[1], nib);
        const int pu = (v_tg >> 1) ^ (d & 15);
        *reinterpret_cast<uint32_t*>(&s_v[d * BN + pu * 4 + (v_tg & 1) * 2]) = bitcast<uint32_t>(a);
      }
    }
    if (tid < BN)
      s_csk[tid] = f16bits_to_f32(sreg) * qk_log2;
    else if (tid < 2 * BN)
      s_sv[tid - BN] = f16bits_to_f32(sreg);
    __syncthreads();
    if (kt + 1 < n_tiles) load_tile(t0 + BN);  // prefetch the next tile's codes

    const bool need = wave_active && (!CAUSAL || t0 <= wrow_hi + off);
    if (!need) continue;

    // ---- S^T = K Q^T for two 32-token blocks
    float16v st[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      float16v acc = float16v{};
      const int tok = 32 * tb + r;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int pc = (2 * s + j) ^ (tok & (NCH - 1));
        const half8v a = *reinterpret_cast<const half8v*>(&s_k[tok * D + pc * 8]);
        acc = mfma32x32x16(a, qop[s], acc);
      }
      st[tb] = acc;
    }

    // ---- online softmax; lane's tokens: 32 tb + 8 (v/4) + 4 j + v%4
    const bool full = (t0 + BN <= kv_len) && (!CAUSAL || t0 + BN - 1 <= wrow_lo + off);
    float x[2][16];
    float mloc = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        const int tok0 = 32 * tb + 8 * vq + 4 * j;
        const float4v cs = *reinterpret_cast<const float4v*>(&s_csk[tok0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = st[tb][4 * vq + i] * cs[i];
          if (!full) {
            const int key = t0 + tok0 + i;
            const bool ok = (key < kv_len) && (!CAUSAL || key <= qrow + off);
            v = ok ? v : -INFINITY;
          }
          x[tb][4 * vq + i] = v;
          mloc = fmaxf(mloc, v);
        }
      }
    }
    mloc = xor_max(mloc, 32);
    const float m_new = fmaxf(m_run, mloc);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float lsum = 0.0f;
    half8v pop[2][2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        const int tok0 = 32 * tb + 8 * vq + 4 * j;
        const float4v sv = *reinterpret_cast<const float4v*>(&s_sv[tok0]);
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = fast_exp2(x[tb][4 * vq + i] - m_use);
          lsum += p[i];
        }
        const half2v p01 = cvt_pk_f16(p[0] * sv[0], p[1] * sv[1]);
        const half2v p23 = cvt_pk_f16(p[2] * sv[2], p[3] * sv[3]);
        // v = 4 vq + i = 8 kp + e  ->  kp = vq / 2, e = 4 (vq % 2) + i
        const int kp = vq >> 1;
        const int e0 = 4 * (vq & 1);
        pop[tb][kp][e0 + 0] = p01[0];
        pop[tb][kp][e0 + 1] = p01[1];
        pop[tb][kp][e0 + 2] = p23[0];
        pop[tb][kp][e0 + 3] = p23[1];
      }
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) o_acc[db] *= alpha;
    }

    // ---- O^T += V^T P^T; k = 8j + e <-> token 32 tb + 16 kp + 8 (e/4) + 4 j + e%4
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        const int u0 = 8 * tb + 4 * kp + j;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int d = 32 * db + r;
          const uint2v lo = *reinterpret_cast<const uint2v*>(&s_v[d * BN + ((u0 ^ (d & 15)) * 4)]);
          const uint2v hi = *reinterpret_cast<const uint2v*>(&s_v[d * BN + (((u0 + 2) ^ (d & 15)) * 4)]);
          const uint4v w = {lo[0], lo[1], hi[0], hi[1]};
          o_acc[db] = mfma32x32x16(bitcast<half8v>(w), pop[tb][kp], o_acc[db]);
        }
      }
    }
  }

  // ---- epilogue: O = O^T / l; lane owns row qrow, head dims 32 db + 8 vq + 4 j + i
  const float l = xor_sum(l_run, 32);
  if (qrow < Sq) {
    const float inv = 1.0f / l;
    float* orow = out + (((int64_t)b * Hq + h) * Sq + qrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        float4v v = {o_acc[db][4 * vq + 0] * inv, o_acc[db][4 * vq + 1] * inv,
                     o_acc[db][4 * vq + 2] * inv, o_acc[db][4 * vq + 3] * inv};
        *reinterpret_cast<float4v*>(orow + 32 * db + 8 * vq + 4 * j) = v;
      }
    }
    if (j == 0 && lse_out)
      lse_out[((int64_t)b * Hq + h) * Sq + qrow] = (m_run + log2f(l)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const uint16_t* q, const uint8_t* kc, const uint16_t* ks, const uint8_t* vc,
                  const uint16_t* vs, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq,
                  int64_t kv_len, int64_t C, float qk_log2, float* out, float* lse,
                  hipStream_t stream) {
  const int nqb = (int)((Sq + BM - 1) / BM);
  dim3 grid((uint32_t)Hq, (uint32_t)nqb, (uint32_t)B);
  prefill_kernel<D, CAUSAL><<<grid, dim3(256), 0, stream>>>(
      q, kc, ks, vc, vs, (int)Hq, (int)Hkv, (int)(Hq / Hkv), (int)Sq, (int)kv_len, C, qk_log2, nqb,
      out, lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const uint16_t* q, const uint8_t* kc, const uint16_t* ks,
                          const uint8_t* vc, const uint16_t* vs, int64_t B, int64_t Hq,
                          int64_t Hkv, int64_t Sq, int64_t kv_len, int64_t C, int D,
                          float softmax_scale, int causal, float* out, float* lse,
                          hipStream_t stream) {
  const float qk_log2 = softmax_scale * kLog2e;
  if (D == 128) {
    if (causal)
      return launch<128, true>(q, kc, ks, vc, vs, B, Hq, Hkv, Sq, kv_len, C, qk_log2, out, lse,
                               stream);
    return launch<128, false>(q, kc, ks, vc, vs, B, Hq, Hkv, Sq, kv_len, C, qk_log2, out, lse,
                              stream);
  }
  if (causal)
    return launch<64, true>(q, kc, ks, vc, vs, B, Hq, Hkv, Sq, kv_len, C, qk_log2, out, lse, stream);
  return launch<64, false>(q, kc, ks, vc, vs, B, Hq, Hkv, Sq, kv_len, C, qk_log2, out, lse, stream);
}

}  // namespace qkvfa
