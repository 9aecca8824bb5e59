// Tiled prefill attention over an int4 KV cache, causal or not.
//
// FlashAttention tiling with online softmax (TurboAttention arXiv 2412.08585
// §2.2): a workgroup owns 32 NW query rows of one head (NW waves x 32 rows)
// and walks the key axis in tiles of 64 tokens.  For each tile the workgroup
// loads the packed int4 K/V codes (8 KB at D = 128, the "quantized KV 8 KB +
// 256 B scales" tile of "Quantized Cross-Attention: Extending
// FlashAttention-3 with In-SRAM Dequantization" §3.2) and converts them
// exactly to fp16 in LDS, where all NW waves share them; codes are never
// dequantized to HBM (same page §3.1).  Scales stay per token: the K scale
// times softmax_scale * log2(e) multiplies score columns in fp32, the V scale
// is folded into P before its one fp16 rounding (§3.4 in the reading that
// keeps the result exact).  Folding either scale into fp16 K/V values instead
// would add one fp16 rounding per element, which large-magnitude channels
// turn into score errors above the attention tolerance.
//
// Contractions use v_mfma_f32_32x32x16_f16 in transposed form:
//   S^T = K Q^T   (M = 32 tokens, N = 32 query rows, K = 16 head dims)
//   O^T += V^T P^T (M = 32 head dims, N = 32 query rows, K = 16 tokens)
// so every lane owns one query row: its 32 scores of a tile are already in
// the B-operand position of the PV product.  Q (bf16) converts exactly to
// fp16; scores are kept in log2 units.
//
// The matrix work hides behind the vector work here (dequantization,
// exponentials, scale products), so the kernel is organised to issue as few
// VALU instructions per tile as it can:
//  * the conversion of a tile is shared by all NW waves;
//  * online softmax keeps a per-row reference m_ref and rescales only when a
//    tile may exceed it by more than tau (base-2 exponent; kTau, lowered on
//    tiles whose largest V scale s_max would take 2^kTau s_max near the fp16
//    limit, so that P~ = p s_V stays finite).  On full tiles the test uses an
//    upper bound, max|s| x max|csk| of the tile, so the common tile needs no
//    per-score product before the exponent: p = exp2(s csk - m_ref) is one
//    fma.  The final normalisation by l = sum(p) is unaffected;
//  * P~ = fp16(p x s_V) is one v_fma_mix per value with s_V read as fp16.  A
//    tile whose largest V scale passes pv_scale_limit (channel outliers)
//    takes P~ as an fp16 hi/lo pair and runs each PV product twice, which
//    keeps the output's rounding error below the attention tolerance.
//
// Query range: a workgroup whose queries hold an element of magnitude 65536
// or more scales them by an exact power of two into fp16 range and its score
// scale by the inverse.
//
// Pipeline: LDS is double buffered.  While a wave computes on tile kt it
// converts tile kt+1 (loaded into registers one iteration earlier) into the
// other buffer and issues the loads of tile kt+2; one barrier per tile.
// Loads go through buffer descriptors whose range ends at kv_len, so the
// ragged last tile and the look-ahead past the last tile read zeros.
//
// Causal (bottom-right aligned, row i sees keys <= i + kv_len - Sq): key tiles
// beyond the last visible key of a workgroup are never used; only tiles
// crossing the diagonal (or the ragged end of the keys) evaluate the mask;
// waves whose rows see nothing of a tile skip its math.  Workgroups are
// dispatched longest-first (highest query block first).
//
// The tile loop is instantiated twice: tiles visible to every row of the
// workgroup (all but the last few of a causal block) run a body with no
// mask, no per-wave skip and no bound/mask join, which saves about a third
// of the vector instructions per tile; the remaining tiles run the general
// body.
//
// LDS layouts (one buffer):
//   K: fp16 16-byte chunk planes: chunk c (head dims 8c..8c+7 in
//      unpack8_perm order) of token t at [c][t][8].  The QK reads of 16
//      consecutive tokens and the conversion writes of 64 consecutive tokens
//      both cover whole 256-byte bank rows.
//   V: fp16 transposed, 8-token planes: plane P holds tokens 4u..4u+3 (h = 0)
//      and 4(u+2)..4(u+2)+3 (h = 1) with u = 8 tb + 4 kp + j,
//      P = 4 tb + 2 kp + j, i.e. exactly the 8 keys one lane feeds to one PV
//      MFMA; head dim d sits at row d ^ ((d >> 4) & 7) of its plane.  The
//      swizzle makes both the PV reads (16 consecutive d) and the conversion
//      writes (d = 8 i + n) hit distinct banks.
//   scales: fp32 K scale x softmax_scale x log2(e) per token; fp16 V scale
//      ordered [j][tb][vq][i] for token 32 tb + 8 vq + 4 j + i, so a lane
//      reads the 32 V scales of its tokens as four 16-byte loads.
#include <math.h>

#include <type_traits>

#include "qkvfa_device.hpp"
#include "qkvfa_internal.h"

namespace qkvfa {

namespace {

constexpr int BN = 64;        // keys per tile
constexpr float kTau = 8.0f;  // lazy-rescale threshold, log2 units

template <int D, int NW, bool CAUSAL, int BITS, int NGA>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kc,
    const uint16_t* __restrict__ ks, const uint8_t* __restrict__ vc,
    const uint16_t* __restrict__ vs, const uint32_t* __restrict__ kp, const uint32_t* __restrict__ vp,
    const int32_t* __restrict__ kv_heads, int Hkv_all, int Hq, int Hkv, int G, int Sq, int kv_len, int64_t C,
    float qk_log2, int nqb, float* __restrict__ out, float* __restrict__ lse_out) {
  // Asymmetric group-wise rows (NGA groups per row): unsigned nibbles in the
  // cache's K and V row orders and parameter words kp/vp [B, Hkv, C, NGA]
  // (fp16 scale in bits 0-15, zero point in bits 16-19).  Codes enter LDS as
  // exact fp16 u - z.  With one group the scales act as the int4 rows' do;
  // with several, each group's QK products accumulate apart and join the
  // score under the group's K scale (PRESCALED scores), and each PV output
  // block (32 head dims, inside one group) takes its group's P~ = p s_V.
  constexpr bool ASYM = NGA > 0;
  constexpr bool PRESCALED = NGA > 1;
  constexpr int NG = ASYM ? NGA : 1;  // scale (and zero point) groups per row
  constexpr int GS = D / NG;          // elements per group
  static_assert(!ASYM || (BITS == 4 && GS >= 32 && D % GS == 0), "asymmetric rows: 4 bits, groups of >= 32");
  constexpr int BM = 32 * NW;  // query rows per workgroup
  constexpr int KS = D / 16;   // QK k-steps
  constexpr int NDB = D / 32;  // PV output blocks
  constexpr int NCH = D / 8;   // K chunk planes
  constexpr int ROWB = D * BITS / 8;  // bytes per packed row (R: 4-bit nibbles; 2/3 bits: bit planes)
  constexpr int KPL = BN * 8;  // halves per K chunk plane
  constexpr int VPL = D * 8;   // halves per V 8-token plane
  constexpr int KBUF = NCH * KPL;
  constexpr int VBUF = 8 * VPL;
  constexpr int KDW = D / (8 * NW);      // K chunks of 8 codes per thread and tile (one int4 dword each)
  constexpr int VT = D / (8 * NW);       // V tokens (x one code dword) per thread
  static_assert(KDW >= 1 && KDW <= 4 && (VT == 2 || VT == 4), "unsupported D / NW");

  __shared__ __align__(16) _Float16 s_k[2 * KBUF];
  __shared__ __align__(16) _Float16 s_v[2 * VBUF];
  __shared__ __align__(16) float s_csk[2][NG][BN];     // K scale x qk_log2 (per group)
  __shared__ __align__(16) _Float16 s_svh[2][NG][BN];  // V scale (per group), [j][tb][vq][i]
  __shared__ float s_cmax[2];                      // max |csk| of the tile
  __shared__ uint32_t s_qmx[NW];                   // per wave: largest |q| (bf16 bits)
  __shared__ uint32_t s_vmx[NW];                   // per wave: largest |V scale| (fp16 bits)
  __shared__ float s_vam[NW];                      // per wave: largest s max(z, 15 - z) (asymmetric rows)
  __shared__ __align__(16) float s_ones[BN];

  const int h = blockIdx.x;   // query head of this call: KV head h / G of the cache
  const int qb = CAUSAL ? (nqb - 1 - (int)blockIdx.y) : (int)blockIdx.y;
  const int b = blockIdx.z;
  const int g = h / G;
  // head map (kv_heads != nullptr): the cache holds KV heads kv_heads[0 ..
  // Hkv) of a layer of Hkv_all (ids clamped into range); q, out and lse are
  // the layer's, and this workgroup's query head there is hq
  const int hq = kv_heads ? min(max(__builtin_amdgcn_readfirstlane(kv_heads[g]), 0), Hkv_all - 1) * G + (h - g * G)
                          : h;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
  // 8 (2 s + j) + perm8(e), matching K chunk plane 2 s + j.  The workgroup's
  // largest |q| decides the range shift (an exact power of two, 0 unless
  // some element is 65536 or more), folded into the score scale qk.
  uint4v qraw[KS];
  half8v qop[KS];
  uint32_t qmb = 0;
  uint32_t vmb = 0;   // largest |V scale| of the workgroup's keys (fp16 bits)
  float vam = 0.0f;   // asymmetric rows: largest s max(z, 15 - z) of those keys
  if (qrow < Sq) {
    const uint16_t* qr = q + (((int64_t)b * Hq + hq) * Sq + qrow) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qraw[s] = *reinterpret_cast<const uint4v*>(qr + 8 * (2 * s + j));
      qmb = max(qmb, bf16x8_max_abs_bits(qraw[s]));
    }
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) qraw[s] = uint4v{0u, 0u, 0u, 0u};
  }
  qmb = bitcast<uint32_t>(wave_max_nonneg(bitcast<float>(qmb)));
  if (lane == 0) s_qmx[wave] = qmb;
  // the shift is known after the first barrier below; tile 0's scale table is
  // written with the unshifted score scale and corrected there if needed
  float qk = qk_log2;   // score scale in log2 units (x 2^qshift)

  float16v o_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o_acc[db] = float16v{};
  float m_ref = -INFINITY;  // row reference (log2 units), shared by lanes r and r + 32
  float m_use = 0.0f;       // m_ref, or 0 while the row has seen no key
  float l_run = 0.0f;       // this lane's share of sum(p), relative to m_ref

  const int64_t kvrow0 = ((int64_t)b * Hkv + g) * C;
  const rsrc_t rk = make_rsrc(kc + kvrow0 * ROWB, kv_len * ROWB);
  const rsrc_t rv = make_rsrc(vc + kvrow0 * ROWB, kv_len * ROWB);
  const rsrc_t rsc = make_rsrc((wave == 0 ? ks : vs) + kvrow0, kv_len * 2);
  // asymmetric rows: parameter words (NG per token)
  const rsrc_t rkp = make_rsrc(ASYM ? kp + kvrow0 * NG : nullptr, ASYM ? kv_len * NG * 4 : 0);
  const rsrc_t rvp = make_rsrc(ASYM ? vp + kvrow0 * NG : nullptr, ASYM ? kv_len * NG * 4 : 0);

  // Loader roles.  K: lane = token, wave = which ROWB / NW bytes of the row
  // (chunk planes KDW wave ..).  V: VT consecutive tokens x one dword (8 head
  // dims) per thread, mapped so that every conversion write instruction of a
  // wave covers distinct banks.  Scales: wave 0 lane t loads the K scale of
  // token t, wave 1 the V scale.
  // (2/3 bits: the chunks' low-bit bytes, 2 per chunk, and top-bit bytes, 1 per chunk at D/4)
  const uint32_t k_voff = (uint32_t)(lane * ROWB + wave * (BITS == 4 ? ROWB / NW : 2 * KDW));
  const uint32_t k_toff = (uint32_t)(lane * ROWB + D / 4 + wave * KDW);
  int v_dp, v_tok0;
  if constexpr (D == 128 && NW == 4) {
    const int t = lane >> 4;
    v_dp = lane & 15;
    v_tok0 = 4 * (8 * (wave >> 1) + 4 * (wave & 1) + 2 * (t & 1) + (t >> 1));
  } else if constexpr (D == 128 && NW == 8) {
    const int t = lane >> 4;
    v_dp = lane & 15;
    v_tok0 = 4 * (8 * (wave >> 2) + 4 * ((wave >> 1) & 1) + 2 * (t & 1) + (wave & 1)) + 2 * (t >> 1);
  } else {
    static_assert(D == 64 && NW == 4, "unsupported D / NW");
    v_dp = lane & 7;
    v_tok0 = 2 * (8 * wave + (lane >> 3));
  }
  const uint32_t v_voff = (uint32_t)(v_tok0 * ROWB + (BITS == 4 ? 4 : 2) * v_dp);
  const uint32_t v_toff = (uint32_t)(v_tok0 * ROWB + D / 4 + v_dp);
  // V store position: plane P and half h of the token unit, row slot base.
  int v_st;
  {
    const int u = v_tok0 >> 2;
    const int P = 4 * (u >> 3) + 2 * ((u >> 2) & 1) + (u & 1);
    const int hh = (u >> 1) & 1;
    const int sig = (v_dp >> 1) & 7;  // (d >> 4) & 7 for d = 8 v_dp + n
    v_st = P * VPL + (8 * v_dp + sig) * 8 + hh * 4 + (v_tok0 & 3);
  }
  // V-scale table slot of token `lane`: [j][tb][vq][i]
  const int sv_slot = ((lane >> 2) & 1) * 32 + (lane >> 5) * 16 + ((lane >> 3) & 3) * 4 + (lane & 3);

  uint32_t kw[KDW];
  uint32_t vw[VT];
  uint32_t ktop = 0;        // 3 bits: the K chunks' top-bit bytes
  uint32_t vt[VT] = {};     // 3 bits: the V tokens' top-bit bytes
  uint16_t sc = 0;
  // asymmetric rows: the parameter word of each K chunk's group (token lane)
  // and the V tokens' words (all groups); for the scale tables, waves
  // [0, NG) load the K word of group `wave` of token lane and waves
  // [NW/2, NW/2 + NG) the V word of group wave - NW/2
  static_assert(!ASYM || NG <= NW / 2, "one wave per group and tensor");
  uint32_t kpw[ASYM ? KDW : 1] = {};
  uint32_t vpw[ASYM ? VT : 1][NG] = {};
  uint32_t spw = 0;
  const bool sp_k = wave < NG;
  const bool sp_v = wave >= NW / 2 && wave < NW / 2 + NG;
  const int sp_g = sp_k ? wave : wave - NW / 2;
  // K chunk (head dims 8c..8c+7) held by dword w of an asymmetric row
  auto asym_kchunk = [](int w) { return 4 * (w % (D / 32)) + w / (D / 32); };
  // head dim held by nibble n of dword w of an asymmetric V row
  auto asym_vdim = [](int w, int n) { return D == 128 ? 16 * n + w : 16 * (n & 3) + w + 8 * (n >> 2); };
  // NG consecutive parameter words at byte offset off (+ soff)
  auto load_words = [&](const rsrc_t& rs, uint32_t off, int soff, uint32_t (&o)[NG]) {
    if constexpr (NG == 4) {
      const uint4v w = __builtin_amdgcn_raw_buffer_load_b128(rs, off, soff, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = w[i];
    } else if constexpr (NG == 2) {
      const uint2v w = __builtin_amdgcn_raw_buffer_load_b64(rs, off, soff, 0);
      o[0] = w[0];
      o[1] = w[1];
    } else {
      o[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, soff, 0);
    }
  };

  auto load_tile = [&](int t0) {
    const int so = t0 * ROWB;
    if constexpr (BITS != 4) {
      // chunk i's low bits in bits 16 (i % 2) of kw[i / 2]; V tokens' in bits 0-15
      if constexpr (KDW == 4) {
        const uint2v w = __builtin_amdgcn_raw_buffer_load_b64(rk, k_voff, so, 0);
        kw[0] = w[0];
        kw[1] = w[1];
        if constexpr (BITS == 3) ktop = __builtin_amdgcn_raw_buffer_load_b32(rk, k_toff, so, 0);
      } else {
        kw[0] = __builtin_amdgcn_raw_buffer_load_b32(rk, k_voff, so, 0);
        if constexpr (BITS == 3) ktop = __builtin_amdgcn_raw_buffer_load_b16(rk, k_toff, so, 0);
      }
#pragma unroll
      for (int i = 0; i < VT; ++i) {
        vw[i] = __builtin_amdgcn_raw_buffer_load_b16(rv, v_voff + i * ROWB, so, 0);
        if constexpr (BITS == 3) vt[i] = __builtin_amdgcn_raw_buffer_load_b8(rv, v_toff + i * ROWB, so, 0);
      }
      if (wave < 2) sc = __builtin_amdgcn_raw_buffer_load_b16(rsc, (uint32_t)(lane * 2), t0 * 2, 0);
      return;
    }
    if constexpr (KDW == 4) {
      const uint4v w = __builtin_amdgcn_raw_buffer_load_b128(rk, k_voff, so, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) kw[i] = w[i];
    } else if constexpr (KDW == 2) {
      const uint2v w = __builtin_amdgcn_raw_buffer_load_b64(rk, k_voff, so, 0);
      kw[0] = w[0];
      kw[1] = w[1];
    } else {
      kw[0] = __builtin_amdgcn_raw_buffer_load_b32(rk, k_voff, so, 0);
    }
#pragma unroll
    for (int i = 0; i < VT; ++i)
      vw[i] = __builtin_amdgcn_raw_buffer_load_b32(rv, v_voff + i * ROWB, so, 0);
    if constexpr (ASYM) {
      const int po = t0 * NG * 4;
#pragma unroll
      for (int i = 0; i < KDW; ++i) {
        const int gi = 8 * asym_kchunk(KDW * wave + i) / GS;
        kpw[i] = __builtin_amdgcn_raw_buffer_load_b32(rkp, (uint32_t)((lane * NG + gi) * 4), po, 0);
      }
#pragma unroll
      for (int i = 0; i < VT; ++i) load_words(rvp, (uint32_t)((v_tok0 + i) * NG * 4), po, vpw[i]);
      if (sp_k || sp_v)
        spw = __builtin_amdgcn_raw_buffer_load_b32(sp_k ? rkp : rvp, (uint32_t)((lane * NG + sp_g) * 4), po, 0);
    } else {
      if (wave < 2) sc = __builtin_amdgcn_raw_buffer_load_b16(rsc, (uint32_t)(lane * 2), t0 * 2, 0);
    }
  };

  // Exact codes to LDS (no scale applied), scales to their tables.
  auto store_tile = [&](int buf) {
    _Float16* sk_ = s_k + buf * KBUF;
    _Float16* sv_ = s_v + buf * VBUF;
#pragma unroll
    for (int i = 0; i < KDW; ++i) {
      const int c = ASYM ? asym_kchunk(KDW * wave + i) : KDW * wave + i;
      half8v kop;
      if constexpr (ASYM)
        kop = unpack8_uz(kw[i], (kpw[i] >> 16) & 0xFu);
      else if constexpr (BITS == 4)
        kop = unpack8_perm(kw[i]);
      else
        kop = unpack8_lowbit<BITS>(kw[i >> 1] >> (16 * (i & 1)), (ktop >> (8 * i)) & 0xFFu);
      *reinterpret_cast<half8v*>(sk_ + c * KPL + lane * 8) = kop;
    }
    // V element n of tokens (0, 1) [and (2, 3)] -> exact fp16 pair
    auto vpair = [&](int t, int n) -> half2v {
      if constexpr (BITS == 4)
        return nib_pair2(vw[t], vw[t + 1], n);
      else
        return lowbit_pair2<BITS>(vw[t], vw[t + 1], vt[t], vt[t + 1], n);
    };
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      _Float16* dst;
      half2v a, c2;
      if constexpr (ASYM) {
        // nibble n of dword v_dp holds head dim d (row slot d ^ ((d >> 4) & 7))
        const int d = asym_vdim(v_dp, n);
        const int gi = d / GS;
        dst = sv_ + (v_st & ~(VPL - 1)) + (v_st & 7) + ((d ^ ((d >> 4) & 7)) * 8);
        auto zt = [&](int t) { return (vpw[t][gi] >> 16) & 0xFu; };
        a = uz_pair2(vw[0], vw[1], n, zt(0), zt(1));
        if constexpr (VT == 4) c2 = uz_pair2(vw[2], vw[3], n, zt(2), zt(3));
      } else {
        // row slot (8 v_dp + n) ^ sig = v_st's slot with n xor-ed into bits 0-2
        dst = sv_ + (v_st ^ (n * 8));
        a = vpair(0, n);
        if constexpr (VT == 4) c2 = vpair(2, n);
      }
      if constexpr (VT == 4) {
        const uint2v w = {bitcast<uint32_t>(a), bitcast<uint32_t>(c2)};
        *reinterpret_cast<uint2v*>(dst) = w;
      } else {
        *reinterpret_cast<uint32_t*>(dst) = bitcast<uint32_t>(a);
      }
    }
    if constexpr (ASYM) {
      if (sp_k) {
        const float f = f16bits_to_f32((uint16_t)(spw & 0xFFFFu)) * qk;
        s_csk[buf][sp_g][lane] = f;
        if constexpr (!PRESCALED) {
          const float m = wave_max_nonneg(fabsf(f));
          if (lane == 0) s_cmax[buf] = m;
        }
      } else if (sp_v) {
        s_svh[buf][sp_g][sv_slot] = bitcast<_Float16>((uint16_t)(spw & 0xFFFFu));
      }
    } else if (wave == 0) {
      const float f = f16bits_to_f32(sc) * qk;
      s_csk[buf][0][lane] = f;
      const float m = wave_max_nonneg(fabsf(f));
      if (lane == 0) s_cmax[buf] = m;
    } else if (wave == 1) {
      s_svh[buf][0][sv_slot] = bitcast<_Float16>(sc);
    }
  };

  // Reader bases (halves, buffer 0).  K: plane j, token r.  V: plane j,
  // row (32 db + r) ^ sigma for each output block db.
  const int k_rd = j * KPL + r * 8;
  int v_rd[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int d = 32 * db + r;
    v_rd[db] = j * VPL + (d ^ ((d >> 4) & 7)) * 8;
  }

  if (threadIdx.x < BN) s_ones[threadIdx.x] = 1.0f;
  load_tile(0);
  // Largest |V scale| (fp16 bits) over the keys the workgroup attends; its
  // loads overlap tile 0's.  The values are 16 bits wide (the scales;
  // asymmetric rows: the low halves of the parameter words), read in aligned
  // 16-byte blocks that never leave the blocks holding them, with every
  // element outside them masked.
  {
    const int nkeys = min(kv_len, n_tiles * BN);
    const uint16_t* vb = ASYM ? reinterpret_cast<const uint16_t*>(vp + kvrow0 * NG) : vs + kvrow0;
    const int n = ASYM ? 2 * nkeys * NG : nkeys;
    const int lead = (int)((reinterpret_cast<uintptr_t>(vb) >> 1) & 7);
    const rsrc_t rs = make_rsrc(vb - lead, ((lead + n + 7) & ~7) * 2);
#pragma unroll 4
    for (int i0 = 8 * (int)threadIdx.x; i0 < lead + n; i0 += 8 * 64 * NW) {
      const uint4v w = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(i0 * 2), 0, 0);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = i0 + e - lead;
        const bool ok = i >= 0 && i < n && (!ASYM || (e & 1) == 0);
        vmb = ok ? max(vmb, (w[e >> 1] >> (16 * (e & 1))) & 0x7FFFu) : vmb;
        if constexpr (ASYM)
          if ((e & 1) == 0) vam = ok ? fmaxf(vam, asym_value_max(w[e >> 1])) : vam;
      }
    }
    vmb = bitcast<uint32_t>(wave_max_nonneg(bitcast<float>(vmb)));
    if (lane == 0) s_vmx[wave] = vmb;
    if constexpr (ASYM) {
      vam = wave_max_nonneg(vam);
      if (lane == 0) s_vam[wave] = vam;
    }
  }
  store_tile(0);
  load_tile(BN);
  __syncthreads();
  float tau_hl;
  {
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      qmb = max(qmb, s_qmx[w]);
      vmb = max(vmb, s_vmx[w]);
      if constexpr (ASYM) vam = fmaxf(vam, s_vam[w]);
    }
    vmb = __builtin_amdgcn_readfirstlane(vmb);   // uniform (LDS values)
    vam = bitcast<float>(__builtin_amdgcn_readfirstlane(bitcast<int>(vam)));
    // rescale threshold of the hi/lo form: p <= 2^tau with 2^tau s_max <=
    // 2^15 keeps P~ finite in fp16 (below the precision limit s_max is far
    // too small for that to bind: tau = kTau)
    tau_hl = fminf(kTau, fmaxf(0.0f, 15.0f - __log2f(f16bits_to_f32((uint16_t)vmb))));
    const int qshift = q_range_shift(qmb);   // uniform
    if (qshift != 0) {   // rare: K scale columns of tile 0 again, scaled by 2^qshift
      qk = qk_log2 * exp2i(qshift);
      const float f = exp2i(qshift);
      if (wave < NG) s_csk[0][wave][lane] *= f;   // wave g wrote group g's column (exact: a power of two)
      if (wave == 0 && lane == 0 && !PRESCALED) s_cmax[0] *= f;
      __syncthreads();
    }
    const float qmul = exp2i(-qshift);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint16_t e16[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        e16[2 * t] = (uint16_t)(qraw[s][t] & 0xFFFFu);
        e16[2 * t + 1] = (uint16_t)(qraw[s][t] >> 16);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) qop[s][e] = (_Float16)(bf16_to_f32(e16[perm8(e)]) * qmul);
    }
  }

  // One key tile.  ALL_FULL: the tile is visible to every row of the
  // workgroup, so no wave skips it and no mask is evaluated.  HILO: P~ as an
  // fp16 hi/lo pair.
  auto step = [&](int kt, auto all_full, auto hilo_c) {
    constexpr bool ALL_FULL = decltype(all_full)::value;
    constexpr bool HILO = decltype(hilo_c)::value;
    const int t0 = kt * BN;
    const int buf = kt & 1;
    const _Float16* sk_ = s_k + buf * KBUF;
    const _Float16* sv_ = s_v + buf * VBUF;
    const float* csk_ = &s_csk[buf][0][0];
    // column factors of the softmax: the K scale column, or ones when the
    // scores already carry their (per-group) K scales
    const float* cbase = PRESCALED ? s_ones : csk_;
    const bool need = ALL_FULL || (wave_active && (!CAUSAL || t0 <= wrow_hi + off));

    // Convert the next tile into the other buffer and fetch the one after.
    // On the last tiles this converts and fetches past the end (zeros, or
    // keys this workgroup never uses): harmless, and branch-free.
    float16v st[2];
    if (need) {
      // ---- S^T = K Q^T for two 32-token blocks
      if constexpr (PRESCALED) {
        // group by group (k-steps 16 s .. 16 s + 15 lie in group 16 s / GS);
        // each group's products scaled by its K scale column
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          st[tb] = float16v{};
#pragma unroll
          for (int gi = 0; gi < NG; ++gi) {
            float16v acc = float16v{};
#pragma unroll
            for (int s = gi * (KS / NG); s < (gi + 1) * (KS / NG); ++s) {
              const half8v a = *reinterpret_cast<const half8v*>(sk_ + k_rd + 2 * s * KPL + tb * 256);
              acc = mfma32x32x16(a, qop[s], acc);
            }
#pragma unroll
            for (int vq = 0; vq < 4; ++vq) {
              const float4v c = *reinterpret_cast<const float4v*>(csk_ + gi * BN + 32 * tb + 8 * vq + 4 * j);
#pragma unroll
              for (int i = 0; i < 4; ++i) st[tb][4 * vq + i] = fmaf(acc[4 * vq + i], c[i], st[tb][4 * vq + i]);
            }
          }
        }
        // the folded scores are complete here: without this pin the compiler
        // sinks the fold below the conversion of the next tile, keeping every
        // group's products and scale columns live across it
        asm volatile("" : "+v"(st[0]), "+v"(st[1]));
      } else {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          float16v acc = float16v{};
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            const half8v a = *reinterpret_cast<const half8v*>(sk_ + k_rd + 2 * s * KPL + tb * 256);
            acc = mfma32x32x16(a, qop[s], acc);
          }
          st[tb] = acc;
        }
      }
      store_tile(buf ^ 1);
      load_tile(t0 + 2 * BN);
    } else {
      store_tile(buf ^ 1);
      load_tile(t0 + 2 * BN);
    }

    if (need) {
      // ---- online softmax; lane's tokens: 32 tb + 8 (v/4) + 4 j + v%4
      const bool full = ALL_FULL || ((t0 + BN <= kv_len) && (!CAUSAL || t0 + BN - 1 <= wrow_lo + off));
      const float tau = HILO ? tau_hl : kTau;
      auto csk4 = [&](int tb, int vq) {
        return *reinterpret_cast<const float4v*>(cbase + 32 * tb + 8 * vq + 4 * j);
      };
      // Exponent p = exp2(st * c - m_use): with c = csk and raw scores st on
      // full tiles, with c = 1 and exact masked scores st on the others.
      const float* ctab = s_ones;
      float mx;
      if (!full) {
        const int lim = (CAUSAL ? min(kv_len - 1, qrow + off) : kv_len - 1) - t0 - 4 * j;
        mx = -INFINITY;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
          for (int vq = 0; vq < 4; ++vq) {
            const float4v c = csk4(tb, vq);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              // key t0 + 32 tb + 8 vq + 4 j + i is visible iff its offset
              // 32 tb + 8 vq + i is at most lim
              const bool ok = 32 * tb + 8 * vq + i <= lim;
              const float x = ok ? st[tb][4 * vq + i] * c[i] : -INFINITY;
              st[tb][4 * vq + i] = x;
              mx = fmaxf(mx, x);
            }
          }
        }
      } else {
        // upper bound of the lane's max score: max |s| x max |csk| of the tile
        mx = 0.0f;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, fabsf(st[tb][v]));
        }
        if constexpr (!PRESCALED) mx *= s_cmax[buf];
        ctab = cbase;
      }
      if (__builtin_amdgcn_ballot_w64(mx > m_ref + tau)) {
        // some row of the wave may rise above its reference: move the
        // reference of those rows to their new maximum, rescale their state
        if (full) {
          mx = -INFINITY;
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
            for (int vq = 0; vq < 4; ++vq) {
              const float4v c = csk4(tb, vq);
#pragma unroll
              for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[tb][4 * vq + i] * c[i]);
            }
          }
        }
        mx = xor_max(mx, 32);
        const bool up = mx > m_ref + tau;
        const float alpha = up ? fast_exp2(m_ref - mx) : 1.0f;
        m_ref = up ? mx : m_ref;
        m_use = (m_ref == -INFINITY) ? 0.0f : m_ref;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) o_acc[db] *= alpha;
      }
      if constexpr (PRESCALED) {
        // per 32-token block: probabilities once, then for each group its
        // P~_g = fp16(p s_V,g) and the PV products of the group's output blocks
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          float pr[2][8];
#pragma unroll
          for (int kp = 0; kp < 2; ++kp) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float p = fast_exp2(st[tb][8 * kp + e] - m_use);
              l_run += p;
              pr[kp][e] = p;
            }
          }
#pragma unroll
          for (int gi = 0; gi < NG; ++gi) {
            const half8v* svh = reinterpret_cast<const half8v*>(&s_svh[buf][gi][32 * j]);
#pragma unroll
            for (int kp = 0; kp < 2; ++kp) {
              const half8v sv = svh[2 * tb + kp];
              half8v pg, pl;
              if constexpr (HILO) {   // low halves about the pinned high halves
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                  const half2v h = pv_hi2(pr[kp][e], (float)sv[e], pr[kp][e + 1], (float)sv[e + 1]);
                  pg[e] = h[0];
                  pg[e + 1] = h[1];
                }
                pin_v(pg);
#pragma unroll
                for (int e = 0; e < 8; ++e) pl[e] = pv_lo(pr[kp][e], (float)sv[e], pg[e]);
              } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) pg[e] = (_Float16)fmaf(pr[kp][e], (float)sv[e], 0.0f);
              }
#pragma unroll
              for (int db = gi * (NDB / NG); db < (gi + 1) * (NDB / NG); ++db) {
                const half8v a =
                    *reinterpret_cast<const half8v*>(sv_ + v_rd[db] + (4 * tb + 2 * kp) * VPL);
                o_acc[db] = mfma32x32x16(a, pg, o_acc[db]);
                if constexpr (HILO) o_acc[db] = mfma32x32x16(a, pl, o_acc[db]);
              }
            }
          }
        }
      } else {
        const half8v* svh = reinterpret_cast<const half8v*>(&s_svh[buf][0][32 * j]);
        // p of value e of block (tb, kp): v = 4 vq + i = 8 kp + e  ->  vq = 2 kp + e/4, i = e%4
        auto prob = [&](int tb, int kp, int e) {
          const float c = ctab[32 * tb + 8 * (2 * kp + (e >> 2)) + 4 * j + (e & 3)];
          return fast_exp2(fmaf(st[tb][8 * kp + e], c, -m_use));
        };
        // ---- O^T += V^T P^T; k = 8 j + e <-> token 32 tb + 16 kp + 8 (e/4) + 4 j + e%4
        if constexpr (HILO) {
          // each high half formed once (pinned) and its low half about
          // exactly that value, then the PV products of both
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
            for (int kp = 0; kp < 2; ++kp) {
              // keeps this step's LDS reads here: hoisted, the 16 V operands
              // of the tile would be live at once
              asm volatile("" ::: "memory");
              const half8v sv = svh[2 * tb + kp];
              half8v ph, pl;
#pragma unroll
              for (int e = 0; e < 8; e += 2) {
                const float p0 = prob(tb, kp, e), p1 = prob(tb, kp, e + 1);
                l_run += p0 + p1;
                const half2v h = pv_hi2(p0, (float)sv[e], p1, (float)sv[e + 1]);
                ph[e] = h[0];
                ph[e + 1] = h[1];
                pl[e] = pv_lo(p0, (float)sv[e], h[0]);
                pl[e + 1] = pv_lo(p1, (float)sv[e + 1], h[1]);
              }
#pragma unroll
              for (int db = 0; db < NDB; ++db) {
                const half8v a =
                    *reinterpret_cast<const half8v*>(sv_ + v_rd[db] + (4 * tb + 2 * kp) * VPL);
                o_acc[db] = mfma32x32x16(a, ph, o_acc[db]);
                o_acc[db] = mfma32x32x16(a, pl, o_acc[db]);
              }
            }
          }
        } else {
          half8v pop[2][2];
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
            for (int kp = 0; kp < 2; ++kp) {
              const half8v sv = svh[2 * tb + kp];  // tokens 32 tb + 8 (2 kp + e/4) + 4 j + e%4
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const float p = prob(tb, kp, e);
                l_run += p;
                // P~ = fp16(p x s_V): one rounding of the exact product
                pop[tb][kp][e] = (_Float16)fmaf(p, (float)sv[e], 0.0f);
              }
            }
          }
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
            for (int kp = 0; kp < 2; ++kp) {
#pragma unroll
              for (int db = 0; db < NDB; ++db) {
                const half8v a =
                    *reinterpret_cast<const half8v*>(sv_ + v_rd[db] + (4 * tb + 2 * kp) * VPL);
                o_acc[db] = mfma32x32x16(a, pop[tb][kp], o_acc[db]);
              }
            }
          }
        }
      }
    }
    __syncthreads();  // tile kt+1 is in LDS; nobody still reads buffer `buf`
  };
  int n_full = kv_len / BN;
  if (CAUSAL) n_full = min(n_full, (q0 + off + 1) / BN);
  n_full = min(n_full, n_tiles);
  // A workgroup whose keys hold a V scale past the precision limit (channel
  // outliers) takes P~ as an fp16 hi/lo pair on every tile; the common loops
  // never evaluate the hi/lo products.
  using T_ = std::integral_constant<bool, true>;
  using F_ = std::integral_constant<bool, false>;
  int kt = 0;
  const bool wg_hilo = ASYM ? vam > kPvErrBudget * 2048.0f : vmb > pv_scale_limit_bits(pv_code_max(BITS, false));
  if (!wg_hilo) {
    for (; kt < n_full; ++kt) step(kt, T_{}, F_{});
    for (; kt < n_tiles; ++kt) step(kt, F_{}, F_{});
  } else {
    for (; kt < n_tiles; ++kt) step(kt, F_{}, T_{});
  }

  // ---- epilogue: O = O^T / l; lane owns row qrow, head dims 32 db + 8 vq + 4 j + i
  const float l = xor_sum(l_run, 32);
  if (qrow < Sq) {
    const float inv = 1.0f / l;
    float* orow = out + (((int64_t)b * Hq + hq) * Sq + qrow) * D;
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
      lse_out[((int64_t)b * Hq + hq) * Sq + qrow] = (m_ref + log2f(l)) * kLn2;
  }
}

struct PrefillArgs {
  const uint16_t* q;
  const uint8_t* kc;
  const uint16_t* ks;
  const uint8_t* vc;
  const uint16_t* vs;
  const uint32_t* kp;   // asymmetric rows: parameter words
  const uint32_t* vp;
  const int32_t* kv_heads;   // head map (or nullptr): the cache's Hkv heads among the layer's Hkv_all
  int64_t Hkv_all;
  int64_t B, Hq, Hkv, Sq, kv_len, C;
  float qk_log2;
  float* out;
  float* lse;
};

template <int D, int NW, bool CAUSAL, int BITS, int NGA = 0>
hipError_t launch1(const PrefillArgs& a, hipStream_t stream) {
  constexpr int BM = 32 * NW;
  const int nqb = (int)((a.Sq + BM - 1) / BM);
  const int64_t G = a.Hq / a.Hkv_all;
  dim3 grid((uint32_t)(a.Hkv * G), (uint32_t)nqb, (uint32_t)a.B);
  prefill_kernel<D, NW, CAUSAL, BITS, NGA><<<grid, dim3(64 * NW), 0, stream>>>(
      a.q, a.kc, a.ks, a.vc, a.vs, a.kp, a.vp, a.kv_heads, (int)a.Hkv_all, (int)a.Hq, (int)a.Hkv, (int)G,
      (int)a.Sq, (int)a.kv_len, a.C, a.qk_log2, nqb, a.out, a.lse);
  return hipGetLastError();
}

// bits 2, 3, 4 (symmetric rows), or asymmetric rows with ng groups per row (ng > 0)
template <int D, int NW, bool CAUSAL>
hipError_t launch(const PrefillArgs& a, hipStream_t stream, int bits, int ng) {
  if (ng == 1) return launch1<D, NW, CAUSAL, 4, 1>(a, stream);
  if (ng == 2) return launch1<D, NW, CAUSAL, 4, 2>(a, stream);
  if (ng == 4) {
    if constexpr (D == 128) return launch1<D, NW, CAUSAL, 4, 4>(a, stream);
    return hipErrorInvalidValue;
  }
  if (bits == 2) return launch1<D, NW, CAUSAL, 2>(a, stream);
  if (bits == 3) return launch1<D, NW, CAUSAL, 3>(a, stream);
  return launch1<D, NW, CAUSAL, 4>(a, stream);
}

hipError_t launch_any(const PrefillArgs& a, int D, int causal, hipStream_t stream, int bits, int ng) {
  if (D == 128) {
    if (causal) return launch<128, 8, true>(a, stream, bits, ng);
    return launch<128, 8, false>(a, stream, bits, ng);
  }
  if (causal) return launch<64, 4, true>(a, stream, bits, ng);
  return launch<64, 4, false>(a, stream, bits, ng);
}

}  // namespace

hipError_t launch_prefill(const uint16_t* q, const uint8_t* kc, const uint16_t* ks,
                          const uint8_t* vc, const uint16_t* vs, int64_t B, int64_t Hq,
                          int64_t Hkv, int64_t Sq, int64_t kv_len, int64_t C, int D,
                          float softmax_scale, int causal, float* out, float* lse,
                          hipStream_t stream, int bits, const int32_t* kv_heads, int64_t Hkv_all) {
  if (prefill_short_fits(D, Sq, kv_len, bits))
    return launch_prefill_short(q, kc, ks, vc, vs, B, Hq, Hkv, Sq, kv_len, C, softmax_scale, causal, out, lse,
                                stream, kv_heads, Hkv_all);
  const PrefillArgs a = {q, kc, ks, vc, vs, nullptr, nullptr, kv_heads, kv_heads ? Hkv_all : Hkv, B, Hq, Hkv, Sq,
                         kv_len, C, softmax_scale * kLog2e, out, lse};
  return launch_any(a, D, causal, stream, bits, 0);
}

hipError_t launch_prefill_asym(const uint16_t* q, const uint8_t* kc, const uint32_t* kp,
                               const uint8_t* vc, const uint32_t* vp, int64_t B, int64_t Hq,
                               int64_t Hkv, int64_t Sq, int64_t kv_len, int64_t C, int D, int group,
                               float softmax_scale, int causal, float* out, float* lse,
                               hipStream_t stream) {
  const PrefillArgs a = {q, kc, nullptr, vc, nullptr, kp, vp, nullptr, Hkv, B, Hq, Hkv, Sq, kv_len, C,
                         softmax_scale * kLog2e, out, lse};
  return launch_any(a, D, causal, stream, 4, D / group);
}

}  // namespace qkvfa
