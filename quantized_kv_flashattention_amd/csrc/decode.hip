// Split-K decode attention over an int4 KV cache, with log-sum-exp merge.
//
// Each of the G*Sq query rows of a GQA group attends cache rows [0, kv_len)
// (append-then-attend decode, TurboAttention arXiv 2412.08585 §2.1).  The KV
// rows are dealt to "splits" chunk by chunk: with n splits, split s takes the
// 32-token chunks s, s + n, s + 2n, ..., so the workgroups of one (batch, KV
// head) stream neighbouring rows at the same time (measured: fewer separate
// streams in flight read HBM faster than one contiguous range per split).
// Each workgroup streams the packed int4 K/V codes of one (split, KV head,
// batch) straight from HBM with
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
// Per-lane load offsets are loop-invariant; only the uniform chunk base moves.
// The next chunk's codes are loaded before the current chunk is processed.
//
// A workgroup is eight waves; wave w takes chunks w, w + 8, w + 16, ... of the
// split.  After the loop the eight waves merge their (m, l, O) through LDS.  With one split the result goes straight to `out`.  Otherwise each
// workgroup writes its split's normalized partial O_s and lse_s, and the last
// workgroup of a (batch, KV head) to finish (an atomic ticket per group)
// merges all splits in split order -- deterministic, and no second launch.
// The ticket returns to zero after the merge, ready for the next call.
//
// Append mode (a decode step that first appends its new K/V rows): before
// streaming, each workgroup quantizes the new rows of its own chunks with the
// shared row quantizer, writes codes and scales to the cache (for later steps)
// and keeps a copy in LDS.  The new rows are the last rows of the attended
// range, so the chunk loop streams only chunks of older rows and the chunks
// that hold new rows (at most three) then take them from the LDS copy: the kernel
// never reads the rows it wrote and needs no memory ordering between those
// stores and its own loads.  Outputs and the written rows are bit-identical
// to a separate append followed by decode.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "qkvfa_device.hpp"
#include "qkvfa_internal.h"

namespace qkvfa {

namespace {

// Waves per workgroup: eight, except for the 64-row variant, whose registers
// (256 per lane with eight waves) do not fit; it keeps four waves and gets
// the whole register file of its SIMD slot.
__host__ __device__ constexpr int waves_for(int NB) { return NB >= 4 ? 4 : 8; }
// 16-row blocks of the kernel that runs R query rows per group: the
// one-block kernel takes at most 8, so that hi/lo P~ chunks find free columns
__host__ __device__ constexpr int row_blocks_for(int64_t R) { return R <= 8 ? 1 : R <= 32 ? 2 : 4; }
template <int N>
struct IntTag {
  static constexpr int value = N;
};

// DPP move of a float inside 16-lane rows: lanes of the banks in BANK (bit k:
// lanes 4k..4k+3 of each row) take src from the lane CTRL names, the others
// keep old.  CTRL: 0x100 + n = row_shl:n (from lane + n), 0x110 + n =
// row_shr:n (from lane - n), 0x120 + n = row_ror:n.
template <int CTRL, int BANK = 0xF>
__device__ __forceinline__ float dpp_f(float old, float src) {
  return bitcast<float>(__builtin_amdgcn_update_dpp(bitcast<int>(old), bitcast<int>(src), CTRL, 0xF, BANK, false));
}
constexpr int kChunk = 32;     // tokens per wave iteration
constexpr int kCoherent = 16;  // buffer-op cache policy: device scope (sc1)
constexpr int kRangeSplits = 8;   // cache splits from which a split reads one range of chunks
constexpr int kMaxSplitPages = 512;         // page ids of one split cached in LDS (paged cache)
constexpr int kRaggedSplitChunks = 128;     // ragged batches: at most 128 chunks per split
constexpr int kMaxTail = 64;                // rows of the INT8 decode buffer one call attends
constexpr int kMaxMergeLse = 4 * 16 * 68;  // LSE table of the merging workgroup (floats)

// Dynamic LDS of a decode launch: the wave-merge buffer (waves x min(16, R)
// rows x (D + 4) floats), reused by the split merge for its weights
// (R x n_split) and one float4 per thread of per-part sums.
inline size_t merge_lds_bytes(int D, int waves, int R, int n_split) {
  const size_t wave_merge = (size_t)waves * (size_t)(R < 16 ? R : 16) * (size_t)(D + 4);
  const size_t split_merge = (size_t)R * (size_t)n_split + 4 + (size_t)4 * 64 * waves;
  return 4 * (wave_merge > split_merge ? wave_merge : split_merge);
}

// Dynamic LDS of the buffer split: the buffered K and V rows (int8) and the
// R x kMaxTail score table.
inline size_t tail_lds_bytes(int D, int R) {
  return (size_t)2 * kMaxTail * D + (size_t)4 * R * kMaxTail;
}

template <int D, int NB>
constexpr size_t max_merge_lds_bytes() {   // largest dynamic LDS of a kernel variant
  const size_t wave_merge = (size_t)waves_for(NB) * 16 * (D + 4);
  const size_t split_merge = (size_t)kMaxMergeLse + 4 + (size_t)4 * 64 * waves_for(NB);
  const size_t merge = 4 * (wave_merge > split_merge ? wave_merge : split_merge);
  const size_t tail = (size_t)2 * kMaxTail * D + (size_t)4 * 64 * kMaxTail;
  return merge > tail ? merge : tail;
}
constexpr int kMaxNew = 64;                 // rows one append-mode call may add

struct DecodeArgs {
  const uint16_t* q;
  const uint8_t* kc;
  const uint16_t* ks;
  const uint8_t* vc;
  const uint16_t* vs;
  float* out;
  float* lse;
  float* part_o;
  float* part_lse;
  uint32_t* tickets;
  int part_bytes;   // bytes of part_o
  // append mode (k_new != nullptr): n_new rows [B, Hkv, n_new, D] go to cache
  // rows [pos, pos + n_new) through the writable cache pointers
  const float* k_new;
  const float* v_new;
  uint8_t* kc_w;
  uint16_t* ks_w;
  uint8_t* vc_w;
  uint16_t* vs_w;
  int pos, n_new;
  // ragged lengths (kv_lens != nullptr): sequence b attends its own
  // min(max(kv_lens[b], 0), len_cap) cached rows (+ n_new appended ones).
  // paged cache (block_table != nullptr, PAGED kernels): the cache arrays are
  // page pools [num_pages, Hkv, page_size, ...]; token t of sequence b sits in
  // page block_table[b * max_pages + t / page_size] (clamped into the pool),
  // row t % page_size.
  const int32_t* kv_lens;
  const int32_t* block_table;
  int len_cap, page_size, max_pages, num_pages;
  // asymmetric group-wise rows (ASYM kernels): codes are unsigned nibbles,
  // group parameters kp/vp [B, Hkv, C, ng] (fp16 scale in bits 0-15, zero
  // point in bits 16-19) for groups of 2^gshift consecutive elements
  const uint32_t* kp;
  const uint32_t* vp;
  int ng, gshift;
  // head map (kv_heads != nullptr): KV head g of this call's cache is KV head
  // kv_heads[g] of a layer with Hkv_all KV heads (Hq, G count the layer)
  const int32_t* kv_heads;
  int Hkv_all;
  // INT8 decode buffer (tail_rows > 0): the last split attends buffered rows
  // [0, tail_rows) of tk/tv [B, Hkv, buf_rows, D] after the kv_len cache
  // rows the other splits attend; rows [tail_len, tail_rows) are the call's
  // new rows tk_new/tv_new [B, Hkv, tail_rows - tail_len, D] fp32, quantized
  // into the buffer first under the universal scales tsk/tsv [B, Hkv].
  int8_t* tk;
  int8_t* tv;
  const float* tsk;
  const float* tsv;
  const float* tk_new;
  const float* tv_new;
  int tail_len, tail_rows, buf_rows;
  int64_t C;
  int Hq, Hkv, G, Sq, kv_len, n_split;
  float qk_log2;
};

// Phase timestamps (measurement build only, QKVFA_PHASE_TRACE): workgroup
// w < kTraceWgs of a launch writes s_memrealtime values (100 MHz) to
// g_trace[w][slot]: 0 entry, 1 chunk loop start, 2 + wave: that wave's last
// chunk done, 10 wave merge and partial written, 11 ticket drawn, 12 exit,
// 13 whether the workgroup merged the splits (0/1).  Each launch rewrites
// every slot it reaches (held in LDS, written out at exit); qkv_trace_read
// copies them to the host.
constexpr int kTraceWgs = 4096;
constexpr int kTraceSlots = 16;
#ifdef QKVFA_PHASE_TRACE
__device__ uint64_t g_trace[kTraceWgs * kTraceSlots];
// stamps go to an LDS copy (an immediate LDS address: no registers kept live
// across the kernel for them); thread 0 writes the copy out as it exits
#define QKVFA_TRACE_LDS __shared__ uint64_t s_trace[kTraceSlots];
#define QKVFA_STAMP(slot, cond) \
  do {                          \
    if (cond) s_trace[(slot)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#define QKVFA_TRACE_PUT(slot, cond, v) \
  do {                                 \
    if (cond) s_trace[(slot)] = (v);   \
  } while (0)
#define QKVFA_TRACE_FLUSH()                                                                   \
  do {                                                                                        \
    if (threadIdx.x == 0 && blockIdx.x < (uint32_t)kTraceWgs) {                               \
      s_trace[12] = __builtin_amdgcn_s_memrealtime();                                         \
      for (int i_ = 0; i_ < kTraceSlots; ++i_) g_trace[blockIdx.x * kTraceSlots + i_] = s_trace[i_]; \
    }                                                                                         \
  } while (0)
#else
#define QKVFA_TRACE_LDS
#define QKVFA_STAMP(slot, cond) \
  do {                          \
  } while (0)
#define QKVFA_TRACE_PUT(slot, cond, v) \
  do {                                 \
  } while (0)
#define QKVFA_TRACE_FLUSH() \
  do {                      \
  } while (0)
#endif

// One row of D fp32 values quantized by one wave: lane l < D/2 owns elements
// 2l and 2l+1 (= byte l of the packed row).  Codes and scale go to the cache
// row in global memory and to an LDS copy.
// A wave quantizes one row: lane l < D/2 holds elements 2l, 2l + 1
template <int D>
__device__ __forceinline__ float2 load_row_pair(const float* __restrict__ src, int lane) {
  float2 v = {0.0f, 0.0f};
  if (lane < D / 2) v = *reinterpret_cast<const float2*>(src + 2 * lane);
  return v;
}
template <int D>
__device__ __forceinline__ void quantize_row_wave(float2 v, int lane, uint8_t* gcodes, uint16_t* gscale,
                                                  uint8_t* lcodes, uint16_t* lscale) {
  const float x0 = v.x, x1 = v.y;
  float m = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = xor_max(m, o);
  const _Float16 s16 = quant_scale(m);
  const float s = (float)s16;
  uint32_t byte = 0;
  if (s != 0.0f) byte = quant_code(x0, s) | (quant_code(x1, s) << 4);
  if (lane < D / 2) {
    gcodes[lane] = (uint8_t)byte;
    lcodes[lane] = (uint8_t)byte;
  }
  if (lane == 0) {
    *gscale = bitcast<uint16_t>(s16);
    *lscale = bitcast<uint16_t>(s16);
  }
}

template <int D, int BITS, int NGA = 0>
struct ChunkRegs {
  // K: the lane's D/4 elements of rows kb = 0, 1 (nibbles, or for 2/3 bits
  // the low-bit bytes: two per 8 elements); V: the lane's 8 elements of 8
  // rows (a dword of nibbles, or the low 16 bits); 3 bits also keep the top
  // bits (K: one byte per 8 elements; V: one byte per row)
  static constexpr int KW = BITS == 4 ? D / 32 : D / 64;
  uint32_t kw[2][KW];
  uint32_t vw[8];
  uint32_t kh[BITS == 3 ? 2 : 1];
  uint32_t vh[BITS == 3 ? 8 : 1];
  uint16_t sk, sv;   // K and V scale of token (lane % 32) of the chunk
  // asymmetric rows (NGA groups per row): parameter words lane * NPW + u of
  // the chunk's K and V rows (word w: token w / NGA, group w % NGA)
  static constexpr int NPW = NGA == 4 ? 2 : 1;
  uint32_t kpw[NPW];
  uint32_t vpw[NPW];
};

// One wave64 holds NB*32 + ~90 VGPRs.  The planner launches about one
// workgroup (two waves per SIMD) per CU; the one-row-block kernel still fits
// 128 VGPRs so that concurrent launches can share a CU.  The 64-row variant
// skips the one-chunk prefetch to stay within 256 VGPRs.
// (3-bit rows keep a second set of top-bit registers per chunk: their one
// row-block variant asks for three waves per SIMD instead of four.)
// PKR: the one-block kernel for at most 4 (PKR = 4) or at most 8 (PKR = 8)
// query rows per group (symmetric rows), whose softmax runs on packed
// scores; 0: the unpacked softmax.  A kernel instantiation holds one
// softmax layout only.
// APP: the append-mode instantiation (a decode step that appends its new
// K/V rows first); the plain decode's kernel carries none of that code.
template <int D, int NB, bool PAGED, int BITS, int NGA, int PKR, bool APP, bool RNG>
__global__ __launch_bounds__(64 * waves_for(NB))
__attribute__((amdgpu_waves_per_eu(NB == 1 ? ((BITS == 3 || NGA > 0) ? 3 : 4) : 1, 8)))
void decode_kernel(const DecodeArgs a) {
  constexpr bool ASYM = NGA > 0;   // asymmetric group-wise rows, NGA groups per row
  constexpr int kWaves = waves_for(NB);
  constexpr bool kPrefetch = (NB <= 2);
  // The one-block kernel over contiguous 2- and 3-bit rows takes two chunks
  // per loop trip (VALU-bound there: 9% fewer VALU instructions per chunk;
  // the int4 step measured 0.8 us slower this way, so int4 keeps one).
  constexpr bool kTwoSets = kPrefetch && NB == 1 && !PAGED && NGA == 0 && BITS != 4;
  constexpr int KK = D / 32;    // QK MFMAs per 16-token block
  constexpr int DW = D / 8;     // dwords per packed row
  constexpr int NPB = D / 16;   // PV MFMAs (16 head dims each)
  constexpr int ROWB = D * BITS / 8;   // bytes per packed row
  // Cache policy of the code, scale and parameter loads: non-temporal (each
  // row is read once per call; measured 5% faster on the 8K step).  3-bit
  // rows take two loads from each row (low and top bits), which the
  // non-temporal policy turned into separate fetches (12% slower): normal.
  constexpr int kStream = BITS == 3 ? 0 : 2;
  // bias of element e (0..7) of a K operand and of the codes of PV block p
  auto kbias = [](int e) { return BITS == 4 ? kNibBias : lowbit_bias<BITS>(e >> 1); };
  auto vbias = [](int p) { return BITS == 4 ? kNibBias : lowbit_bias<BITS>(p & 3); };
  static_assert(BITS == 4 || !PAGED, "the paged cache holds 4-bit rows");
  static_assert(!ASYM || (BITS == 4 && !PAGED && (NGA == 1 || NGA == 2 || NGA == 4) && D / NGA >= 32),
                "asymmetric rows: 4 bits, contiguous cache, groups of 32, 64 or 128 elements");
  using Regs = ChunkRegs<D, BITS, NGA>;
  constexpr int NPW = Regs::NPW;
  constexpr int OSTR = D + 4;   // padded LDS row stride of the merge buffer (floats)

  __shared__ __align__(16) _Float16 s_q[NB * 16 * D];
  __shared__ __align__(16) float s_sc[kWaves][96];   // K column scale, V scale, mask bias
  // asymmetric rows, per wave and chunk, [group][token]: K -s x softmax scale
  // x log2 e and 79 - z (fp32); V s and 79 - z (fp16)
  __shared__ __align__(16) float s_ak[ASYM ? kWaves : 1][2][ASYM ? NGA : 1][32];
  __shared__ __align__(16) _Float16 s_av[ASYM ? kWaves : 1][2][ASYM ? NGA : 1][32];
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  // wave-merge buffer [kWaves][rows_o][OSTR] floats, later the split-merge
  // weights: dynamic, sized by the launch for the rows this call has
  extern __shared__ __align__(16) float s_o[];
  __shared__ int s_last;
  __shared__ int s_qwide[kWaves];   // query range check, per wave
  __shared__ float s_den[64];
  __shared__ float s_tm[64];    // buffer split: per-row score maximum
  // append mode: this split's new rows, indexed by row - pos
  __shared__ __align__(16) uint32_t s_nk[kMaxNew * DW];
  __shared__ __align__(16) uint32_t s_nv[kMaxNew * DW];
  __shared__ uint16_t s_nks[kMaxNew];
  __shared__ uint16_t s_nvs[kMaxNew];
  // paged cache: the page ids of this split's tokens (from page t_begin / P on)
  __shared__ int s_pid[PAGED ? kMaxSplitPages : 1];

  QKVFA_TRACE_LDS
  const int lane = threadIdx.x & 63;
  QKVFA_STAMP(0, threadIdx.x == 0);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;
  const int j = lane >> 4;
  // One-dimensional grid, split index slowest: consecutive workgroups (which
  // the dispatcher deals round-robin to the eight XCDs) take different
  // (batch, KV head) units of one split, so every XCD gets an even share of
  // each split -- also when the late splits of short sequences are empty.
  const int n_units = (int)(gridDim.x / (uint32_t)a.n_split);
  const int split = (int)blockIdx.x / n_units;
  const int unit = (int)blockIdx.x - split * n_units;
  const int g = unit % a.Hkv;
  const int b = unit / a.Hkv;
  const int G = a.G, Sq = a.Sq;
  // head map: this call's cache holds KV heads kv_heads[0 .. Hkv) of a layer
  // of Hkv_all KV heads (ids clamped into range); their query rows are
  // written, other rows of q / out / lse are not touched
  const int gq = a.kv_heads ? min(max(__builtin_amdgcn_readfirstlane(a.kv_heads[g]), 0), a.Hkv_all - 1) : g;
  const int R = G * Sq;
  const int rows_o = min(16, R);   // rows per wave in the merge buffer
  // At most 4 query rows in the one 16-row block: the softmax runs on packed
  // scores (2 per lane instead of 8, the other 48 lanes' rows being padding)
  constexpr bool PK = PKR == 4;    // packed, at most 4 rows: row b's low halves in column 4 + b
  constexpr bool PK8 = PKR == 8;   // packed, at most 8 rows: row b's low halves in column 8 + b
  static_assert(PKR == 0 || (NB == 1 && !ASYM), "packed softmax: one row block, symmetric rows");
  // At most 8 query rows otherwise: rows r < 8 are duplicated into columns
  // r + 8 of the block, whose lanes carry the low halves of hi/lo P~ chunks
  constexpr bool dup_rows = NB == 1 && !PK && !PK8;   // (the launch gives this kernel at most 8 rows)
  static_assert(!APP || (BITS == 4 && NGA == 0), "append mode: 4-bit symmetric rows");
  const bool append = APP;   // the launch picks APP = (a.k_new != nullptr)
  // rows this sequence attends, and where its new rows start (append mode)
  int pos_b = a.pos;
  int L_b = a.kv_len;
  if (a.kv_lens != nullptr) {
    const int lb = min(max(__builtin_amdgcn_readfirstlane(a.kv_lens[b]), 0), a.len_cap);
    pos_b = lb;
    L_b = lb + (append ? a.n_new : 0);
  }
  // Query row `row` of this group (head gq G + row / Sq, position row % Sq)
  // is row grow0 + row of q, out and lse: heads of a group are adjacent.  Its
  // split partials are row prow0 + row of the workspace, which numbers the
  // rows of this call's (batch, KV head) units only (= grow0 without a map).
  const int64_t grow0 = ((int64_t)b * a.Hq + (int64_t)gq * G) * Sq;
  const int64_t prow0 = ((int64_t)b * a.Hkv + g) * G * Sq;
  // The chunks of cache split `split` (of ns_c; with an INT8 buffer the last
  // split attends the buffered rows instead): c_first, c_first + c_step, ...,
  // c_count of them, among the sequence's gc_end 32-token chunks.
  //  * contiguous cache, up to 7 splits (RNG false): interleaved, split s takes chunks s,
  //    s + ns_c, ...  With lengths per sequence, a sequence uses only as many
  //    splits as its length needs at the plan's chunks per split (the longest
  //    uses them all), so a short sequence keeps few workgroups busy.
  //  * contiguous int4 cache with 8 or more splits (RNG), and paged cache: a range of cps
  //    consecutive chunks.  Interleaved over many splits, each workgroup would
  //    read 2 KB pieces far apart (every 32nd chunk on the 128K-token step,
  //    which streams 1.2 us faster from ranges; with 2 splits interleaving is
  //    as fast or faster); paged, each page is read by one workgroup
  //    (interleaved, both workgroups of a page would look up its address
  //    translation: measured 9% slower on a ragged batch)
  const int t_end = L_b;
  const int gc_end = (t_end + kChunk - 1) / kChunk;   // chunks of the sequence
  int ns_c = max(a.n_split - (a.tail_rows > 0 ? 1 : 0), 1);
  const int cps = ((a.kv_len + kChunk - 1) / kChunk + ns_c - 1) / ns_c;   // the plan's chunks per split
  if (!PAGED && a.kv_lens != nullptr) ns_c = max(min(ns_c, (gc_end + cps - 1) / cps), 1);
  constexpr bool ranges = PAGED || RNG;
  const int c_first = ranges ? split * cps : split;
  const int c_step = ranges ? 1 : ns_c;
  const int c_count = ranges ? min(max(gc_end - c_first, 0), cps)
                             : (split < ns_c && gc_end > split ? (gc_end - split + ns_c - 1) / ns_c : 0);
  // splits with a chunk of this sequence: a prefix 0 .. n_used - 1
  const int n_used = ranges ? min((gc_end + cps - 1) / cps, ns_c) : min(ns_c, gc_end);
  const int t_begin = c_first * kChunk;   // first row of the split's first chunk
  const int cstride = c_step * kChunk;     // rows between its chunks
  const bool nothing = c_count == 0;
  // chunk gc of the sequence is this split's chunk number *k
  auto own_chunk = [&](int gc, int* k) {
    const int d = gc - c_first;
    *k = d / c_step;
    return d >= 0 && d % c_step == 0 && *k < c_count;
  };

  // Row index (in the cache arrays' row space) of token t of this (batch, KV
  // head): contiguous cache row (b, g, t), or row t % P of its page.
  const int64_t kvrow0 = ((int64_t)b * a.Hkv + g) * a.C;
  const int P = PAGED ? a.page_size : 1;
  const int pg0 = PAGED ? t_begin / P : 0;
  // pages of this split whose ids are cached in LDS
  const int t_last = min(t_end, (c_first + c_count) * kChunk) - 1;   // the split's last row
  const int npg = (PAGED && !nothing) ? min(t_last / P - pg0 + 1, kMaxSplitPages) : 0;
  auto page_of = [&](int t) -> int64_t {   // from the table in global memory
    const int idx = min(t / P, a.max_pages - 1);
    const int pid = __builtin_amdgcn_readfirstlane(a.block_table[(int64_t)b * a.max_pages + idx]);
    return min(max(pid, 0), a.num_pages - 1);
  };
  // from_lds: the page id comes from this split's LDS copy of its table
  // entries (filled before the chunk loop); pages past the copy (beyond its
  // capacity, or a prefetch past the split end) are read from the table.
  auto row_of = [&](int t, bool from_lds) -> int64_t {
    if constexpr (PAGED) {
      const int li = t / P - pg0;
      const int64_t pid = (from_lds && li < npg) ? (int64_t)s_pid[li] : page_of(t);
      return (pid * a.Hkv + g) * P + t % P;
    } else {
      return kvrow0 + t;
    }
  };

  // Loop-invariant per-lane byte offsets inside a chunk.
  // K: the lane's D/4 elements start at byte KK j * BITS of its row (its low
  // bits; 3 bits: top bits KK bytes from D/4 + KK j); V: its 8 elements at
  // byte BITS (r % DW) (3 bits: low bits at 2 (r % DW), top bits at D/4 + r % DW)
  const uint32_t offk = (uint32_t)((8 * (r >> 2) + (r & 3)) * ROWB + (BITS == 4 ? 4 : 2) * KK * j);  // +4 rows for kb = 1
  const uint32_t offv = (uint32_t)(8 * j * ROWB + (BITS == 4 ? 4 : 2) * (r % DW));
  const uint32_t offs = (uint32_t)(2 * (lane & 31));

  // ---- append mode: rows [pos_b, t_end) are new.  The chunk loop covers
  // this split's chunks before the first that holds a new row (chunks
  // [0, gc_main) of the sequence, rows below t_main); the split's remaining
  // (tail) chunks are handled after it, each by the wave the plain decode
  // gives it, so the arithmetic is the plain decode's.
  const int gc_main = append ? pos_b / kChunk : gc_end;
  const int t_main = append ? gc_main * kChunk : t_end;

  const bool direct = (a.n_split == 1);
  // one descriptor over all partial outputs (the planner keeps them < 2 GiB)
  const rsrc_t rpart = make_rsrc(a.part_o, direct ? 0 : a.part_bytes);

  // ---- split merge by the last workgroup of this (batch, KV head) to finish
  //      (run after this split's partial is written, or at once by a split
  //      with nothing to attend)
  auto merge_splits = [&]() {
    // ---- split merge by the last workgroup of this (batch, KV head) to finish.
    // Partials were written with device-coherent stores; waiting for their
    // completion before the barrier orders them before the ticket increment.
    // The merging workgroup reads them back with device-coherent loads, so no
    // L2 writeback or invalidation (an expensive whole-cache operation) is needed.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    uint32_t* ticket = a.tickets + (int64_t)b * a.Hkv + g;
    if (threadIdx.x == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = (prev == (uint32_t)(a.n_split - 1));
    }
    __syncthreads();
    QKVFA_STAMP(11, threadIdx.x == 0);
    QKVFA_TRACE_PUT(13, threadIdx.x == 0, (uint64_t)(s_last ? 1 : 0));
    if (!s_last) {
      QKVFA_TRACE_FLUSH();
      return;
    }
    const int n_split = a.n_split;
    // splits that start before this sequence's length; the rest attended nothing
    const int n_live = a.tail_rows > 0 ? n_split : n_used;
    // item idx: four output values (query row idx / (D/4), dims 4 (idx % (D/4)) + 0..3)
    const int n_items = R * (D / 4);
    auto item_off = [&](int idx) -> uint32_t {
      return (uint32_t)(((prow0 + idx / (D / 4)) * n_split * D + 4 * (idx % (D / 4))) * 4);
    };
    // Steps (0)-(3), instantiated for 4 or 16 splits per task loaded ahead
    // (loads of splits past the live ones still pass the memory pipeline)
    auto merge_with = [&](auto pre_tag) {
      // Work unit "task" = (item, part): part p of an item sums its splits p,
      // p + tpi, p + 2 tpi, ...  With few items (few query rows) and many splits,
      // several threads share an item (tpi > 1) so that every partial load is in
      // flight at once; their sums meet in LDS and are added in part order.
      constexpr int kNthr = 64 * kWaves;
      constexpr int kPre = decltype(pre_tag)::value;   // splits of a task loaded before the weights are known
      int tpi = 1;
      while (tpi * kPre < n_live && 2 * tpi * n_items <= kNthr) tpi *= 2;
      const int n_tasks = n_items * tpi;
      // loads of splits part + tpi (u0 + u), u < n.  Branch-free: a split past
      // the live ones (a thread without a task asks for part n_live) is read at an offset
      // past the descriptor's range, which returns zeros without a memory
      // access (loads under divergent branches make the compiler wait for them
      // at the join, serializing this prefetch with the LSE loads)
      auto load_n = [&](int item, int part, int u0, auto& o) {
        const uint32_t off0 = item_off(item);
        constexpr int n = sizeof(o) / sizeof(o[0]);
#pragma unroll
        for (int u = 0; u < n; ++u) {
          const int sp = part + tpi * (u0 + u);
          const uint32_t off = sp < n_live ? off0 + (uint32_t)(sp * D * 4) : 0x80000000u;
          o[u] = __builtin_amdgcn_raw_buffer_load_b128(rpart, off, 0, kCoherent);
        }
      };
      // acc += sum_u w[part + tpi (u0 + u)] o[u], in blocks of four weights read
      // together; an index past the live splits is clamped (its o[u] is zero)
      auto accumulate = [&](const float* wr, int part, int u0, const auto& o, float4v& acc) {
        constexpr int n = sizeof(o) / sizeof(o[0]);
#pragma unroll
        for (int blk = 0; blk < n / 4; ++blk) {
          if (tpi * (u0 + 4 * blk) < n_live) {   // uniform
            float wv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) wv[i] = wr[min(part + tpi * (u0 + 4 * blk + i), n_live - 1)];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc += wv[i] * o[4 * blk + i];
          }
        }
      };
      // (0) the partial outputs of this thread's first task (its first kPre
      //     splits), issued now: their round trip overlaps the LSE loads'
      float4v pre[kPre];
      {
        const int t0 = min((int)threadIdx.x, n_tasks - 1);
        load_n(t0 % n_items, (int)threadIdx.x < n_tasks ? t0 / n_items : n_live, 0, pre);
      }
      // (1) every live split's LSE of this group -> LDS (the wave-merge buffer is free
      //     now; the planner keeps R * n_split <= kMaxMergeLse), loads in flight together
      float* s_w = s_o;
      {
        const int total = R * n_live;
        for (int base = threadIdx.x; base < total; base += 64 * kWaves * 8) {
          float v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int idx = base + u * 64 * kWaves;
            v[u] = -INFINITY;
            if (idx < total) {
              const int row = idx / n_live;
              v[u] = __hip_atomic_load(a.part_lse + (prow0 + row) * n_split + (idx - row * n_live), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
          }
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (base + u * 64 * kWaves < total) s_w[base + u * 64 * kWaves] = v[u];
        }
      }
      __syncthreads();
      // (2) per row: max, weights 2^(lse_s - max) (in place), their sum -- one wave per row
      for (int row = wave; row < R; row += kWaves) {
        float* wr = s_w + row * n_live;
        float M = -INFINITY;
        for (int s = lane; s < n_live; s += 64) M = fmaxf(M, wr[s]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) M = xor_max(M, o);
        float den = 0.0f;
        for (int s = lane; s < n_live; s += 64) {
          const float w = fast_exp2(wr[s] - M);
          wr[s] = w;
          den += w;
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) den = xor_sum(den, o);
        if (lane == 0) {
          s_den[row] = den;
          const int64_t grow = grow0 + row;
          if (a.lse) a.lse[grow] = den > 0.0f ? (M + log2f(den)) * kLn2 : -INFINITY;
        }
      }
      __syncthreads();
      // (3) O = sum_s w_s O_s / sum_s w_s: each task sums its splits (sixteen
      //     partial loads in flight per thread; the first task starts from its
      //     prefetched splits), then the parts of an item are added in order
      float4v* s_part = reinterpret_cast<float4v*>(s_w + ((R * n_live + 3) & ~3));   // tpi > 1: [tpi][n_items]
      auto finish = [&](int item, const float4v& acc) {
        const int row = item / (D / 4);
        const float den = s_den[row];
        *reinterpret_cast<float4v*>(a.out + (grow0 + row) * D + 4 * (item - row * (D / 4))) =
            acc * (den > 0.0f ? 1.0f / den : 0.0f);
      };
      auto task = [&](int t, bool first) {
        const int item = t % n_items;
        const int part = t / n_items;
        const float* wr = s_w + (item / (D / 4)) * n_live;
        float4v acc = {0.f, 0.f, 0.f, 0.f};
        int u0 = 0;
        if (first) {
          accumulate(wr, part, 0, pre, acc);
          u0 = kPre;
        }
        for (; tpi * u0 < n_live; u0 += 16) {   // uniform
          float4v o[16];
          load_n(item, part, u0, o);
          accumulate(wr, part, u0, o, acc);
        }
        if (tpi == 1) finish(item, acc);
        else s_part[t] = acc;
      };
      if ((int)threadIdx.x < n_tasks) task(threadIdx.x, true);
      for (int t = threadIdx.x + kNthr; t < n_tasks; t += kNthr) task(t, false);
      if (tpi > 1) {
        __syncthreads();
        for (int item = threadIdx.x; item < n_items; item += kNthr) {
          float4v acc = s_part[item];
          for (int p = 1; p < tpi; ++p) acc += s_part[p * n_items + item];
          finish(item, acc);
        }
      }
    };
    if (n_live <= 4) merge_with(IntTag<4>{});
    else merge_with(IntTag<16>{});
    if (threadIdx.x == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    QKVFA_TRACE_FLUSH();
  };

  // The chunk loop, the wave merge and the partial (or direct) output of a
  // split that has cache rows to attend.
  auto main_body = [&]() {
    // Codes of the chunk starting at token c0, through buffer descriptors whose
    // range ends at lim <= kv_len (the end of the split's last chunk, before
    // any new rows): the hardware returns zero for any row at or past it
    // (those tokens are masked) without touching memory.  So no load leaves
    // the valid rows, the last chunk needs no clamping, and a chunk past the
    // split can be "loaded" unconditionally (all zeros, no traffic), which
    // keeps the prefetch branch-free: a conditional prefetch makes the
    // compiler wait for every outstanding load where the paths join.
    auto load_chunk = [&](int c0, Regs& cr, int lim, bool from_lds) {
      // a chunk is 32 rows; with a paged cache it never straddles a page.  The
      // clamp is made scalar explicitly: computed in a vector register, the
      // descriptor would look divergent and each load would become a loop.
      const int rows_left = __builtin_amdgcn_readfirstlane(min(max(lim - c0, 0), kChunk));
      const int64_t row0 = row_of(c0, from_lds);
      const rsrc_t rk = make_rsrc(a.kc + row0 * ROWB, rows_left * ROWB);
      const rsrc_t rv = make_rsrc(a.vc + row0 * ROWB, rows_left * ROWB);
      const rsrc_t rks = make_rsrc(a.ks + row0, rows_left * 2);
      const rsrc_t rvs = make_rsrc(a.vs + row0, rows_left * 2);
      if constexpr (BITS == 4) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if constexpr (KK == 4) {
            const uint4v w = __builtin_amdgcn_raw_buffer_load_b128(rk, offk + kb * 4 * ROWB, 0, kStream);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) cr.kw[kb][kk] = w[kk];
          } else {
            const uint2v w = __builtin_amdgcn_raw_buffer_load_b64(rk, offk + kb * 4 * ROWB, 0, kStream);
            cr.kw[kb][0] = w[0];
            cr.kw[kb][1] = w[1];
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) cr.vw[e] = __builtin_amdgcn_raw_buffer_load_b32(rv, offv + e * ROWB, 0, kStream);
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const uint32_t o = offk + kb * 4 * ROWB;
          if constexpr (KK == 4) {
            const uint2v w = __builtin_amdgcn_raw_buffer_load_b64(rk, o, 0, kStream);
            cr.kw[kb][0] = w[0];
            cr.kw[kb][1] = w[1];
            // top bits: KK bytes at D/4 + KK j of the row (o sits at 2 KK j)
            if constexpr (BITS == 3) cr.kh[kb] = __builtin_amdgcn_raw_buffer_load_b32(rk, o + D / 4 - KK * j, 0, kStream);
          } else {
            cr.kw[kb][0] = __builtin_amdgcn_raw_buffer_load_b32(rk, o, 0, kStream);
            if constexpr (BITS == 3) cr.kh[kb] = __builtin_amdgcn_raw_buffer_load_b16(rk, o + D / 4 - KK * j, 0, kStream);
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          cr.vw[e] = __builtin_amdgcn_raw_buffer_load_b16(rv, offv + e * ROWB, 0, kStream);
          if constexpr (BITS == 3)   // top bits: byte D/4 + r % DW of the row (offv sits at 2 (r % DW))
            cr.vh[e] = __builtin_amdgcn_raw_buffer_load_b8(rv, offv + e * ROWB + D / 4 - (r % DW), 0, kStream);
        }
      }
      if constexpr (ASYM) {
        // the chunk's 32 x NGA parameter words, NPW per lane; words past the
        // range read as zero (scale 0: the token's values are 0)
        const rsrc_t rkp = make_rsrc(a.kp + row0 * NGA, rows_left * NGA * 4);
        const rsrc_t rvp = make_rsrc(a.vp + row0 * NGA, rows_left * NGA * 4);
        if constexpr (NPW == 2) {
          const uint2v wk = __builtin_amdgcn_raw_buffer_load_b64(rkp, 8 * lane, 0, kStream);
          const uint2v wv = __builtin_amdgcn_raw_buffer_load_b64(rvp, 8 * lane, 0, kStream);
          cr.kpw[0] = wk[0];
          cr.kpw[1] = wk[1];
          cr.vpw[0] = wv[0];
          cr.vpw[1] = wv[1];
        } else {
          cr.kpw[0] = __builtin_amdgcn_raw_buffer_load_b32(rkp, 4 * lane, 0, kStream);
          cr.vpw[0] = __builtin_amdgcn_raw_buffer_load_b32(rvp, 4 * lane, 0, kStream);
        }
      } else {
        cr.sk = __builtin_amdgcn_raw_buffer_load_b16(rks, offs, 0, kStream);
        cr.sv = __builtin_amdgcn_raw_buffer_load_b16(rvs, offs, 0, kStream);
      }
    };

    // this split's chunks before gc_main
    const int n_chunks = gc_main > c_first ? min((gc_main - c_first + c_step - 1) / c_step, c_count) : 0;
    Regs cur;
    // loads stop at the end of the split's last chunk as well: a paged split's
    // range is followed by another split's rows
    const int t_ld = min(t_main, (c_first + (c_count - 1) * c_step + 1) * kChunk);
    // append mode: this wave's first quantize task (below) reads its fp32
    // row before the chunk loads are issued, so that waiting for the row does
    // not wait for them
    const int ntask = (BITS == 4 && !ASYM && append) ? 2 * max(t_end - pos_b, 0) : 0;
    auto task_src = [&](int task) {
      const bool isv = (task & 1) != 0;
      return (isv ? a.v_new : a.k_new) + (((int64_t)b * a.Hkv + g) * a.n_new + (task >> 1)) * D;
    };
    float2 first_row = {0.0f, 0.0f};
    if (kWaves - 1 - wave < ntask) first_row = load_row_pair<D>(task_src(kWaves - 1 - wave), lane);
    load_chunk(t_begin + wave * cstride, cur, t_ld, false);

    // ---- append mode: quantize the new rows of this split's chunks (one wave
    //      per row and tensor, from the last wave down: with one row block the
    //      first half of the waves converts the query meanwhile), while the
    //      first chunk loads (4-bit caches only)
    if (BITS == 4 && !ASYM && append) {
      for (int task = kWaves - 1 - wave; task < ntask; task += kWaves) {
        const int t = pos_b + (task >> 1);
        int k;
        if (!own_chunk(t / kChunk, &k)) continue;   // another split's chunk
        const bool isv = (task & 1) != 0;
        const float2 src = task == kWaves - 1 - wave ? first_row : load_row_pair<D>(task_src(task), lane);
        const int64_t row = row_of(t, false);
        uint8_t* gcodes = (isv ? a.vc_w : a.kc_w) + row * ROWB;
        uint16_t* gscale = (isv ? a.vs_w : a.ks_w) + row;
        uint8_t* lcodes = reinterpret_cast<uint8_t*>(isv ? s_nv : s_nk) + (t - pos_b) * ROWB;
        uint16_t* lscale = (isv ? s_nvs : s_nks) + (t - pos_b);
        quantize_row_wave<D>(src, lane, gcodes, gscale, lcodes, lscale);
      }
    }


    if constexpr (PAGED) {
      for (int i = threadIdx.x; i < npg; i += 64 * kWaves) {
        const int idx = min(pg0 + i, a.max_pages - 1);
        s_pid[i] = min(max(a.block_table[(int64_t)b * a.max_pages + idx], 0), a.num_pages - 1);
      }
    }

    // Query operand (B of S^T = K Q^T): query row nb*16 + r, k = 8j + e <->
    // head dim 8*(KK*j + kk) + perm8(e), matching the K lane's dword order.
    // Converted once into LDS (shared by the eight waves): 16-byte chunk c of
    // row x sits at chunk c ^ (x % 16), so the 16 rows a wave reads together
    // fall in different banks.
    // An element of magnitude 65536 or more (past fp16 range) anywhere in the
    // group: the whole group's query is converted again, scaled by an exact
    // power of two 2^-qshift, and the score scale qk carries 2^qshift.
    auto convert_q = [&](float qmul) {
      uint32_t mb = 0;
      for (int idx = threadIdx.x; idx < NB * 16 * DW; idx += 64 * kWaves) {
        const int row = idx / DW;
        const int c = idx - row * DW;
        half8v h = half8v{};
        const int src = (dup_rows && row >= 8) ? row - 8 : row;
        if (src < R) {
          const uint16_t* qr = a.q + (grow0 + src) * D + 8 * c;
          const uint4v w = *reinterpret_cast<const uint4v*>(qr);
          mb = max(mb, bf16x8_max_abs_bits(w));
          uint16_t e16[8];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            e16[2 * t] = (uint16_t)(w[t] & 0xFFFFu);
            e16[2 * t + 1] = (uint16_t)(w[t] >> 16);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) h[e] = (_Float16)(bf16_to_f32(e16[perm8(e)]) * qmul);
        }
        *reinterpret_cast<half8v*>(&s_q[(row * DW + (c ^ (row & 15 & (DW - 1)))) * 8]) = h;
      }
      return mb;
    };
    const bool q_wide = __builtin_amdgcn_ballot_w64(convert_q(1.0f) >= 0x4780u) != 0;   // >= 65536
    if (lane == 0) s_qwide[wave] = q_wide ? 1 : 0;
    __syncthreads();
    int qshift = 0;
    {
      int any = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) any |= s_qwide[w];
      if (any) {   // rare: find the group's largest |q|, convert again
        __syncthreads();
        const uint32_t mb = convert_q(1.0f);   // (values rewritten unchanged)
        if (lane == 0) s_qwide[wave] = 0;
        __syncthreads();
        __hip_atomic_fetch_max(&s_qwide[0], (int)mb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __syncthreads();
        qshift = q_range_shift((uint32_t)s_qwide[0]);
        __syncthreads();
        convert_q(exp2i(-qshift));
        __syncthreads();
      }
    }
    const float qk = a.qk_log2 * exp2i(qshift);   // score scale in log2 units

    // Codes enter the MFMAs as exact fp16 values c + b (the bias b depends on
    // the code's position only).  Scores: each QK accumulator starts at
    // -sum_d q_d b_d of its query row, so it ends at the plain dot product.
    // Outputs: s_run sums the fp16 P~ values the PV MFMAs consumed (rescaled
    // like O), and the wave merge takes b x s_run out of each output.
    float m_run[NB], l_run[NB], s_run[NB], kinit[NB];
    // asymmetric rows: Q_g = sum of the row's query elements in group g, and
    // per group the sum of P~ (79 - z) the PV MFMAs consumed (rescaled like O)
    float qg[NB][ASYM ? NGA : 1], sg[NB][ASYM ? NGA : 1];
    float4v o_acc[NB][NPB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      m_run[nb] = -INFINITY;
      l_run[nb] = 0.0f;
      s_run[nb] = 0.0f;
#pragma unroll
      for (int p = 0; p < NPB; ++p) o_acc[nb][p] = float4v{0.f, 0.f, 0.f, 0.f};
      const int qrow = nb * 16 + r;
      if constexpr (ASYM) {
        // the cache's K order gives block kk the elements 32 kk .. 32 kk + 31:
        // lane j holds query chunk 4 kk + j for it
#pragma unroll
        for (int gi = 0; gi < NGA; ++gi) {
          qg[nb][gi] = 0.0f;
          sg[nb][gi] = 0.0f;
        }
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const int qc = (4 * kk + j) ^ (qrow & 15 & (DW - 1));
          const half8v qop = *reinterpret_cast<const half8v*>(&s_q[(qrow * DW + qc) * 8]);
#pragma unroll
          for (int e = 0; e < 8; ++e) qg[nb][kk / (KK / NGA)] += (float)qop[e];
        }
#pragma unroll
        for (int gi = 0; gi < NGA; ++gi) {
          qg[nb][gi] = xor_sum(qg[nb][gi], 16);
          qg[nb][gi] = xor_sum(qg[nb][gi], 32);
        }
        kinit[nb] = 0.0f;
      } else {
        float qb = 0.0f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const int qc = (KK * j + kk) ^ (qrow & 15 & (DW - 1));
          const half8v qop = *reinterpret_cast<const half8v*>(&s_q[(qrow * DW + qc) * 8]);
#pragma unroll
          for (int e = 0; e < 8; ++e) qb = fmaf((float)qop[e], kbias(e), qb);
        }
        qb = xor_sum(qb, 16);
        qb = xor_sum(qb, 32);
        kinit[nb] = -qb;
      }
    }

    // One chunk: scores, online softmax, PV.  `cr` holds its codes and scales.
    auto process_chunk = [&](int c0, Regs& cr, int lim) {
        // ---- scales: each lane converts one, the wave reads its eight back.  A
        //      token at or past the split end gets bias -inf (score masked), so
        //      the score is one FMA on every chunk, full or not.
        // lanes 0-31: K column scale x softmax scale x log2 e; lanes 32-63: V scale
        const float scv = f16bits_to_f32(lane < 32 ? cr.sk : cr.sv);
        s_sc[wave][lane] = lane < 32 ? scv * qk : scv;
        if (lane < 32) s_sc[wave][64 + lane] = (c0 + lane < lim) ? 0.0f : -INFINITY;
        const float4v ck0 = *reinterpret_cast<const float4v*>(&s_sc[wave][8 * j]);
        const float4v ck1 = *reinterpret_cast<const float4v*>(&s_sc[wave][8 * j + 4]);
        const float4v sv0 = *reinterpret_cast<const float4v*>(&s_sc[wave][32 + 8 * j]);
        const float4v sv1 = *reinterpret_cast<const float4v*>(&s_sc[wave][32 + 8 * j + 4]);
        const float4v mb0 = *reinterpret_cast<const float4v*>(&s_sc[wave][64 + 8 * j]);
        const float4v mb1 = *reinterpret_cast<const float4v*>(&s_sc[wave][64 + 8 * j + 4]);
        const float csk[8] = {ck0[0], ck0[1], ck0[2], ck0[3], ck1[0], ck1[1], ck1[2], ck1[3]};
        const float sv[8] = {sv0[0], sv0[1], sv0[2], sv0[3], sv1[0], sv1[1], sv1[2], sv1[3]};
        const float mbias[8] = {mb0[0], mb0[1], mb0[2], mb0[3], mb1[0], mb1[1], mb1[2], mb1[3]};

        if constexpr (D == 64) {
          // lanes 8..15 own elements 4..7 of their 8: move them down
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            cr.vw[e] = (r >= 8) ? (cr.vw[e] >> (BITS == 4 ? 16 : 8)) : cr.vw[e];
            if constexpr (BITS == 3) cr.vh[e] = (r >= 8) ? (cr.vh[e] >> 4) : cr.vh[e];
          }
        }

        // ---- scores S^T for 2 x 16 tokens and every 16-row block; each K operand
        //      is converted once and used for all row blocks
        float4v s_t[NB][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) s_t[nb][kb] = float4v{kinit[nb], kinit[nb], kinit[nb], kinit[nb]};
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            half8v kop;
            if constexpr (BITS == 4) {
              kop = unpack8_perm_b(cr.kw[kb][kk]);
            } else {
              // chunk kk: low bits in bytes 2 (kk % 2), +1 of dword kk / 2; top bits in byte kk
              const uint32_t lo16 = cr.kw[kb][kk >> 1] >> (16 * (kk & 1));
              const uint32_t top8 = BITS == 3 ? (cr.kh[kb] >> (8 * kk)) & 0xFFu : 0u;
              kop = unpack8_lowbit_b<BITS>(lo16, top8);
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              const int qrow = nb * 16 + r;
              const int qc = (KK * j + kk) ^ (qrow & 15 & (DW - 1));
              const half8v qop = *reinterpret_cast<const half8v*>(&s_q[(qrow * DW + qc) * 8]);
              s_t[nb][kb] = mfma16x16x32(kop, qop, s_t[nb][kb]);
            }
          }
        }

        // the V codes as new values, so that a second PV pass converts them
        // again instead of keeping the first pass's operands live
        auto fresh_v = [&]() {
#pragma unroll
          for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(cr.vw[e]));
          if constexpr (BITS == 3) {
#pragma unroll
            for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(cr.vh[e]));
          }
        };
        // ---- O^T += V^T P^T for the P operands pp of every row block
        auto pv_products = [&](const half8v (&pp)[NB]) {
          if constexpr (BITS == 4) {
            // V operand of blocks 2k, 2k+1: byte k of the eight token dwords,
            // low and high nibble -> exact fp16 (token e = k index)
#pragma unroll
            for (int k = 0; k < NPB / 2; ++k) {
              uint4v wlo, whi;
#pragma unroll
              for (int hh = 0; hh < 4; ++hh) {
                const uint32_t xb = pair_bytes(cr.vw[2 * hh], cr.vw[2 * hh + 1], k);
                wlo[hh] = nib_b72(xb << 4);
                whi[hh] = nib_b72(xb);
              }
              const half8v vlo = bitcast<half8v>(wlo);
              const half8v vhi = bitcast<half8v>(whi);
#pragma unroll
              for (int nb = 0; nb < NB; ++nb) {
                o_acc[nb][2 * k] = mfma16x16x32(vlo, pp[nb], o_acc[nb][2 * k]);
                o_acc[nb][2 * k + 1] = mfma16x16x32(vhi, pp[nb], o_acc[nb][2 * k + 1]);
              }
            }
          } else {
            // 2/3-bit rows.  V operand of block 4 k2 + f: the 2-bit field f of
            // byte k2 of the eight tokens' low bits (3 bits: with top bit
            // 4 k2 + f of their top-bit bytes)
#pragma unroll
            for (int k2 = 0; k2 < NPB / 4; ++k2) {
              uint4v pr[4];   // pr[hh][f]: field f of tokens 2 hh, 2 hh + 1 (c + lowbit_bias(f))
#pragma unroll
              for (int hh = 0; hh < 4; ++hh) {
                const uint32_t xb = pair_bytes(cr.vw[2 * hh], cr.vw[2 * hh + 1], k2);
                const uint32_t zb = BITS == 3 ? pair_bytes(cr.vh[2 * hh], cr.vh[2 * hh + 1], 0) >> (4 * k2) : 0u;
                pr[hh] = lowbit4_b<BITS>(xb, zb);
              }
#pragma unroll
              for (int f = 0; f < 4; ++f) {
                const uint4v w = {pr[0][f], pr[1][f], pr[2][f], pr[3][f]};
                const half8v vop = bitcast<half8v>(w);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                  o_acc[nb][4 * k2 + f] = mfma16x16x32(vop, pp[nb], o_acc[nb][4 * k2 + f]);
              }
            }
          }
        };

        // A V scale of this chunk past the precision limit: P~ is taken as an
        // fp16 hi/lo pair (see pv_lo).  With free columns in the 16-row
        // block (at most 8 query rows), the low halves ride in them: the
        // packed softmax puts row b's in column 4 + b, the unpacked one
        // duplicates rows r < 8 into columns r + 8, whose lanes feed the low
        // halves (zeros in other chunks); the wave merge adds those columns
        // to their rows.  Otherwise the low halves get PV products of their own.
        constexpr uint32_t kLimBits = pv_scale_limit_bits(pv_code_max(BITS, false));
        const bool hilo = __builtin_amdgcn_ballot_w64(lane >= 32 && (uint32_t)cr.sv > kLimBits) != 0;
        // ---- online softmax per row block -> P^T operand (V scale folded in)
        half8v pop[NB];
        float pe[NB][8];    // probabilities of the unpacked softmax (for the low halves of hi/lo chunks)
        half2v hw[NB][4];   // their high halves P~
        if constexpr (PK) {
          // Packed: lane (j, 4a + b) takes slots 2a, 2a + 1 (tokens 8j + 2a,
          // 8j + 2a + 1) of row b from lane (j, b) with three bank-masked
          // row shifts per value; row maxima reduce over a with row rotations;
          // P~ returns to the B-operand layout of lanes (j, b) with row shifts
          // the other way.  l and s_run stay per lane (summed over a in the
          // wave merge); m is the same on the lanes of a row.
          const int e0 = 8 * j + 2 * (r >> 2);
          const float2v c2 = *reinterpret_cast<const float2v*>(&s_sc[wave][e0]);
          const float2v v2 = *reinterpret_cast<const float2v*>(&s_sc[wave][32 + e0]);
          const float2v m2 = *reinterpret_cast<const float2v*>(&s_sc[wave][64 + e0]);
          float y0 = s_t[0][0][0], y1 = s_t[0][0][1];
          y0 = dpp_f<0x114, 0x2>(y0, s_t[0][0][2]);
          y1 = dpp_f<0x114, 0x2>(y1, s_t[0][0][3]);
          y0 = dpp_f<0x118, 0x4>(y0, s_t[0][1][0]);
          y1 = dpp_f<0x118, 0x4>(y1, s_t[0][1][1]);
          y0 = dpp_f<0x11C, 0x8>(y0, s_t[0][1][2]);
          y1 = dpp_f<0x11C, 0x8>(y1, s_t[0][1][3]);
          const float x0 = fmaf(y0, c2[0], m2[0]);
          const float x1 = fmaf(y1, c2[1], m2[1]);
          float mloc = fmaxf(x0, x1);
          mloc = fmaxf(mloc, dpp_f<0x124>(mloc, mloc));
          mloc = fmaxf(mloc, dpp_f<0x128>(mloc, mloc));
          mloc = xor_max(mloc, 16);
          mloc = xor_max(mloc, 32);
          const float m_new = fmaxf(m_run[0], mloc);   // finite: every chunk has a valid token
          const float alpha = fast_exp2(m_run[0] - m_new);
          const float p0 = fast_exp2(x0 - m_new);
          const float p1 = fast_exp2(x1 - m_new);
          half2v q2 = cvt_pk_f16(p0 * v2[0], p1 * v2[1]);
          if (hilo) pin_v(q2);   // the low halves below are taken about exactly these values
          const float qf = bitcast<float>(q2);
          float pw[4] = {dpp_f<0xE4, 0x1>(0.0f, qf), dpp_f<0x104, 0x1>(0.0f, qf), dpp_f<0x108, 0x1>(0.0f, qf),
                         dpp_f<0x10C, 0x1>(0.0f, qf)};
          float ps = __builtin_amdgcn_fdot2(q2, half2v{1, 1}, s_run[0] * alpha, false);
          if (hilo) {   // low halves P~_lo = fp16(p s_V - P~) (residuals exact in fp32)
            asm volatile("");   // a real branch: not speculated into every chunk
            const half2v lo2 = {pv_lo(p0, v2[0], q2[0]), pv_lo(p1, v2[1], q2[1])};
            const float lf = bitcast<float>(lo2);
            ps = __builtin_amdgcn_fdot2(lo2, half2v{1, 1}, ps, false);
            pw[0] = dpp_f<0x114, 0x2>(pw[0], lf);
            pw[1] = dpp_f<0xE4, 0x2>(pw[1], lf);
            pw[2] = dpp_f<0x104, 0x2>(pw[2], lf);
            pw[3] = dpp_f<0x108, 0x2>(pw[3], lf);
          }
          const uint4v pu = {bitcast<uint32_t>(pw[0]), bitcast<uint32_t>(pw[1]), bitcast<uint32_t>(pw[2]),
                             bitcast<uint32_t>(pw[3])};
          pop[0] = bitcast<half8v>(pu);
          s_run[0] = ps;
          l_run[0] = l_run[0] * alpha + (p0 + p1);
          m_run[0] = m_new;
          if (__ballot(alpha != 1.0f)) {
#pragma unroll
            for (int p = 0; p < NPB; ++p) o_acc[0][p] *= alpha;
          }
        } else if constexpr (PK8) {
          // Packed, at most 8 rows: lane (j, 8a + b) takes slots 4a .. 4a + 3
          // (tokens 8j + 4a .. 8j + 4a + 3) of row b; lanes (j, 8 + b) get
          // slots 4-7 of lane (j, b) with one row shift per value.  Row maxima
          // reduce over a with a row rotation by 8.  P~ returns to the
          // B-operand layout of lanes (j, b) with row shifts the other way;
          // lanes (j, 8 + b) then feed the low halves of hi/lo chunks
          // (column 8 + b, added to row b in the wave merge), else zeros.
          const bool upper = r >= 8;   // a = 1
          const int e0 = 8 * j + (upper ? 4 : 0);
          const float4v c4 = *reinterpret_cast<const float4v*>(&s_sc[wave][e0]);
          const float4v v4 = *reinterpret_cast<const float4v*>(&s_sc[wave][32 + e0]);
          const float4v m4 = *reinterpret_cast<const float4v*>(&s_sc[wave][64 + e0]);
          float x[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float y = dpp_f<0x118, 0xC>(s_t[0][0][i], s_t[0][1][i]);   // row_shr:8 on lanes 8-15
            x[i] = fmaf(y, c4[i], m4[i]);
          }
          float mloc = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
          mloc = fmaxf(mloc, dpp_f<0x128>(mloc, mloc));
          mloc = xor_max(mloc, 16);
          mloc = xor_max(mloc, 32);
          const float m_new = fmaxf(m_run[0], mloc);   // finite: every chunk has a valid token
          const float alpha = fast_exp2(m_run[0] - m_new);
          float p[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) p[i] = fast_exp2(x[i] - m_new);
          half2v q01 = cvt_pk_f16(p[0] * v4[0], p[1] * v4[1]);
          half2v q23 = cvt_pk_f16(p[2] * v4[2], p[3] * v4[3]);
          if (hilo) {   // the low halves below are taken about exactly these values
            pin_v(q01);
            pin_v(q23);
          }
          const float h01 = bitcast<float>(q01), h23 = bitcast<float>(q23);
          // lanes 0-7: own slots 0-3, slots 4-7 from lane + 8 (row_shl:8)
          float pw[4] = {h01, h23, dpp_f<0x108, 0x3>(h01, h01), dpp_f<0x108, 0x3>(h23, h23)};
          // s_run: the P~ values this lane computed (high halves, and low
          // halves below), whichever lane feeds them to the products; the
          // wave merge sums the two lanes of a row
          float ps = __builtin_amdgcn_fdot2(q01, half2v{1, 1}, s_run[0] * alpha, false);
          ps = __builtin_amdgcn_fdot2(q23, half2v{1, 1}, ps, false);
          if (upper) pw[0] = pw[1] = pw[2] = pw[3] = 0.0f;   // its high halves went to lanes 0-7
          if (hilo) {   // low halves P~_lo = fp16(p s_V - P~) (residuals exact in fp32)
            asm volatile("");   // a real branch: not speculated into every chunk
            const half2v lo01 = {pv_lo(p[0], v4[0], q01[0]), pv_lo(p[1], v4[1], q01[1])};
            const half2v lo23 = {pv_lo(p[2], v4[2], q23[0]), pv_lo(p[3], v4[3], q23[1])};
            ps = __builtin_amdgcn_fdot2(lo01, half2v{1, 1}, ps, false);
            ps = __builtin_amdgcn_fdot2(lo23, half2v{1, 1}, ps, false);
            const float l01 = bitcast<float>(lo01), l23 = bitcast<float>(lo23);
            // lanes 8-15: slots 0-3 from lane - 8 (row_shr:8), own slots 4-7
            const float s01 = dpp_f<0x118, 0xC>(0.0f, l01), s23 = dpp_f<0x118, 0xC>(0.0f, l23);
            if (upper) {
              pw[0] = s01;
              pw[1] = s23;
              pw[2] = l01;
              pw[3] = l23;
            }
          }
          const uint4v pu = {bitcast<uint32_t>(pw[0]), bitcast<uint32_t>(pw[1]), bitcast<uint32_t>(pw[2]),
                             bitcast<uint32_t>(pw[3])};
          pop[0] = bitcast<half8v>(pu);
          s_run[0] = ps;
          l_run[0] = l_run[0] * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
          m_run[0] = m_new;
          if (__ballot(alpha != 1.0f)) {
#pragma unroll
            for (int q = 0; q < NPB; ++q) o_acc[0][q] *= alpha;
          }
        } else {
          // lanes of duplicated rows (columns r + 8 of a block of at most 8
          // rows): the low halves of P~ in hi/lo chunks, 0 in the others
          const bool dup_lane = dup_rows && r >= 8;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            float x[8];
            float mloc = -INFINITY;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              x[e] = fmaf(s_t[nb][e >> 2][e & 3], csk[e], mbias[e]);
              mloc = fmaxf(mloc, x[e]);
            }
            mloc = xor_max(mloc, 16);
            mloc = xor_max(mloc, 32);
            const float m_new = fmaxf(m_run[nb], mloc);   // finite: every chunk has a valid token
            const float alpha = fast_exp2(m_run[nb] - m_new);
            float lsum = 0.0f;
            uint4v pw;
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
              const float p0 = fast_exp2(x[e] - m_new);
              const float p1 = fast_exp2(x[e + 1] - m_new);
              lsum += p0 + p1;
              pe[nb][e] = p0;
              pe[nb][e + 1] = p1;
              hw[nb][e / 2] = cvt_pk_f16(p0 * sv[e], p1 * sv[e + 1]);
              pw[e / 2] = dup_lane ? 0u : bitcast<uint32_t>(hw[nb][e / 2]);
            }
            if (NB == 1 && hilo && dup_rows) {   // duplicated rows' lanes: the low halves
              asm volatile("");   // a real branch: not speculated into every chunk
#pragma unroll
              for (int h = 0; h < 4; ++h) {
                // about the high halves the row's own lane feeds (same
                // instruction on identical inputs: the same values)
                pin_v(hw[nb][h]);
                const half2v lo = {pv_lo(pe[nb][2 * h], sv[2 * h], hw[nb][h][0]),
                                   pv_lo(pe[nb][2 * h + 1], sv[2 * h + 1], hw[nb][h][1])};
                pw[h] = dup_lane ? bitcast<uint32_t>(lo) : pw[h];
              }
            }
            pop[nb] = bitcast<half8v>(pw);
            float ps = s_run[nb] * alpha;
#pragma unroll
            for (int h = 0; h < 4; ++h) ps = __builtin_amdgcn_fdot2(bitcast<half2v>(pw[h]), half2v{1, 1}, ps, false);
            s_run[nb] = ps;
            l_run[nb] = l_run[nb] * alpha + lsum;
            m_run[nb] = m_new;
            if (__ballot(alpha != 1.0f)) {
#pragma unroll
              for (int p = 0; p < NPB; ++p) o_acc[nb][p] *= alpha;
            }
          }
        }

        pv_products(pop);
        if (NB > 1 && hilo) {   // no free columns: PV products of the low halves
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            uint4v lw;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              pin_v(hw[nb][h]);
              lw[h] = bitcast<uint32_t>(half2v{pv_lo(pe[nb][2 * h], sv[2 * h], hw[nb][h][0]),
                                               pv_lo(pe[nb][2 * h + 1], sv[2 * h + 1], hw[nb][h][1])});
            }
            float pl = s_run[nb];
#pragma unroll
            for (int h = 0; h < 4; ++h) pl = __builtin_amdgcn_fdot2(bitcast<half2v>(lw[h]), half2v{1, 1}, pl, false);
            s_run[nb] = pl;
            pop[nb] = bitcast<half8v>(lw);
          }
          fresh_v();
          pv_products(pop);
        }
    };

    // One chunk of asymmetric group-wise rows.  Codes enter the MFMAs as the
    // exact fp16 value 79 - u (one v_bitop3 per pair).  Scores: the cache's K
    // order makes block kk the elements 32 kk .. 32 kk + 31, so a group's
    // blocks accumulate on their own, from -(79 - z) Q_g: the result is
    // -sum q (u - z) over the group, exact up to fp32 sums, and -s x softmax
    // scale x log2 e (fp32) adds the group's share of the score.  Outputs: the
    // cache's V order makes PV block p the elements 16 p .. 16 p + 15, so a
    // group's blocks take P~_g = fp16(p s) of the group, and sg collects
    // sum P~_g (79 - z); the wave merge forms sg - O.
    auto process_chunk_asym = [&](int c0, Regs& cr, int lim) {
      if constexpr (ASYM) {
        // a V group scale of this chunk past the precision limit: P~_g also
        // gets its low fp16 half (see pv_lo)
        bool big = false;
#pragma unroll
        for (int u = 0; u < NPW; ++u) big = big || (lane * NPW + u < 32 * NGA && asym_needs_hilo(cr.vpw[u]));
        const bool hilo = __builtin_amdgcn_ballot_w64(big) != 0;
#pragma unroll
        for (int u = 0; u < NPW; ++u) {
          const int w = lane * NPW + u;   // token w / NGA, group w % NGA
          if (w < 32 * NGA) {
            const int t = w / NGA, gi = w % NGA;
            const uint32_t pk = cr.kpw[u], pv = cr.vpw[u];
            s_ak[wave][0][gi][t] = -f16bits_to_f32((uint16_t)pk) * qk;
            s_ak[wave][1][gi][t] = 79.0f - (float)((pk >> 16) & 15u);
            s_av[wave][0][gi][t] = bitcast<_Float16>((uint16_t)pv);
            s_av[wave][1][gi][t] = bitcast<_Float16>((uint16_t)(0x5400u | ((15u - ((pv >> 16) & 15u)) << 4)));
          }
        }
        if (lane < 32) s_sc[wave][64 + lane] = (c0 + lane < lim) ? 0.0f : -INFINITY;
        const float4v mb0 = *reinterpret_cast<const float4v*>(&s_sc[wave][64 + 8 * j]);
        const float4v mb1 = *reinterpret_cast<const float4v*>(&s_sc[wave][64 + 8 * j + 4]);

        if constexpr (D == 64) {
          // lanes 8..15 own nibbles 4..7 of their dword: move them down
#pragma unroll
          for (int e = 0; e < 8; ++e) cr.vw[e] = (r >= 8) ? (cr.vw[e] >> 16) : cr.vw[e];
        }

        // ---- scores S^T (tokens 8 j + 4 kb + i of this lane), group by group
        float4v xs[NB][2];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          xs[nb][0] = mb0;
          xs[nb][1] = mb1;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int gi = 0; gi < NGA; ++gi) {
            const float4v nc = *reinterpret_cast<const float4v*>(&s_ak[wave][0][gi][8 * j + 4 * kb]);
            const float4v bz = *reinterpret_cast<const float4v*>(&s_ak[wave][1][gi][8 * j + 4 * kb]);
            float4v acc[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[nb] = bz * -qg[nb][gi];
#pragma unroll
            for (int kq = 0; kq < KK / NGA; ++kq) {
              const int kk = gi * (KK / NGA) + kq;
              const half8v kop = unpack8_n79(cr.kw[kb][kk]);
#pragma unroll
              for (int nb = 0; nb < NB; ++nb) {
                const int qrow = nb * 16 + r;
                const int qc = (4 * kk + j) ^ (qrow & 15 & (DW - 1));
                const half8v qop = *reinterpret_cast<const half8v*>(&s_q[(qrow * DW + qc) * 8]);
                acc[nb] = mfma16x16x32(kop, qop, acc[nb]);
              }
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) xs[nb][kb] += nc * acc[nb];
          }
        }

        // ---- online softmax per row block
        float pr[NB][8];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          float mloc = -INFINITY;
#pragma unroll
          for (int e = 0; e < 8; ++e) mloc = fmaxf(mloc, xs[nb][e >> 2][e & 3]);
          mloc = xor_max(mloc, 16);
          mloc = xor_max(mloc, 32);
          const float m_new = fmaxf(m_run[nb], mloc);   // finite: every chunk has a valid token
          const float alpha = fast_exp2(m_run[nb] - m_new);
          float lsum = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pr[nb][e] = fast_exp2(xs[nb][e >> 2][e & 3] - m_new);
            lsum += pr[nb][e];
          }
          l_run[nb] = l_run[nb] * alpha + lsum;
          m_run[nb] = m_new;
#pragma unroll
          for (int gi = 0; gi < NGA; ++gi) sg[nb][gi] *= alpha;
          if (__ballot(alpha != 1.0f)) {
#pragma unroll
            for (int p = 0; p < NPB; ++p) o_acc[nb][p] *= alpha;
          }
        }

        // ---- O^T += V^T P~_g^T, group by group (PV blocks 2k, 2k + 1 from byte k)
#pragma unroll
        for (int gi = 0; gi < NGA; ++gi) {
          const half8v sv = *reinterpret_cast<const half8v*>(&s_av[wave][0][gi][8 * j]);
          const uint4v bzv = *reinterpret_cast<const uint4v*>(&s_av[wave][1][gi][8 * j]);
          // the group's PV blocks for P operands pp
          auto pv_group = [&](const half8v (&pp)[NB]) {
#pragma unroll
            for (int kq = 0; kq < NPB / 2 / NGA; ++kq) {
              const int k = gi * (NPB / 2 / NGA) + kq;
              uint4v wlo, whi;
#pragma unroll
              for (int hh = 0; hh < 4; ++hh) {
                const uint32_t xb = pair_bytes(cr.vw[2 * hh], cr.vw[2 * hh + 1], k);
                wlo[hh] = nib_n79(xb << 4);
                whi[hh] = nib_n79(xb);
              }
#pragma unroll
              for (int nb = 0; nb < NB; ++nb) {
                o_acc[nb][2 * k] = mfma16x16x32(bitcast<half8v>(wlo), pp[nb], o_acc[nb][2 * k]);
                o_acc[nb][2 * k + 1] = mfma16x16x32(bitcast<half8v>(whi), pp[nb], o_acc[nb][2 * k + 1]);
              }
            }
          };
          // lanes of duplicated rows (at most 8 query rows): the low halves
          // of P~_g in hi/lo chunks, 0 in the others
          const bool dup_lane = dup_rows && r >= 8;
          half8v pop[NB];
          half2v ahw[NB][4];   // high halves P~_g
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            uint4v pw;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              ahw[nb][h] = cvt_pk_f16(pr[nb][2 * h] * (float)sv[2 * h], pr[nb][2 * h + 1] * (float)sv[2 * h + 1]);
              pw[h] = dup_lane ? 0u : bitcast<uint32_t>(ahw[nb][h]);
            }
            if (NB == 1 && hilo && dup_rows) {   // duplicated rows' lanes: the low halves
              asm volatile("");
#pragma unroll
              for (int h = 0; h < 4; ++h) {
                pin_v(ahw[nb][h]);
                const half2v lo = {pv_lo(pr[nb][2 * h], (float)sv[2 * h], ahw[nb][h][0]),
                                   pv_lo(pr[nb][2 * h + 1], (float)sv[2 * h + 1], ahw[nb][h][1])};
                pw[h] = dup_lane ? bitcast<uint32_t>(lo) : pw[h];
              }
            }
            float ps = sg[nb][gi];
#pragma unroll
            for (int h = 0; h < 4; ++h)
              ps = __builtin_amdgcn_fdot2(bitcast<half2v>(pw[h]), bitcast<half2v>(bzv[h]), ps, false);
            sg[nb][gi] = ps;
            pop[nb] = bitcast<half8v>(pw);
          }
          pv_group(pop);
          if (NB > 1 && hilo) {   // no free columns: PV products of the low halves
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              uint4v pw;
#pragma unroll
              for (int h = 0; h < 4; ++h) {
                pin_v(ahw[nb][h]);
                pw[h] = bitcast<uint32_t>(half2v{pv_lo(pr[nb][2 * h], (float)sv[2 * h], ahw[nb][h][0]),
                                                 pv_lo(pr[nb][2 * h + 1], (float)sv[2 * h + 1], ahw[nb][h][1])});
              }
              float ps = sg[nb][gi];
#pragma unroll
              for (int h = 0; h < 4; ++h)
                ps = __builtin_amdgcn_fdot2(bitcast<half2v>(pw[h]), bitcast<half2v>(bzv[h]), ps, false);
              sg[nb][gi] = ps;
              pop[nb] = bitcast<half8v>(pw);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(cr.vw[e]));
            pv_group(pop);
          }
        }
      }
    };
    auto process = [&](int c0, Regs& cr, int lim) {
      if constexpr (ASYM)
        process_chunk_asym(c0, cr, lim);
      else
        process_chunk(c0, cr, lim);
    };

    QKVFA_STAMP(1, threadIdx.x == 0);
    if constexpr (kTwoSets) {
      // Two register sets in fixed roles, two chunks per trip: no copy of the
      // prefetched set at the back edge (a copy is one VALU move per register
      // and waits for the loads it copies).
      for (int c = wave; c < n_chunks; c += 2 * kWaves) {
        const int c0 = t_begin + c * cstride;
        // Compiler-only barrier: keeps the query-operand LDS reads inside the loop
        // instead of hoisted into (NB * D / 8) live registers per lane.
        asm volatile("" ::: "memory");
        Regs nxt;
        load_chunk(c0 + kWaves * cstride, nxt, t_ld, true);
        process(c0, cur, t_main);
        asm volatile("" ::: "memory");
        load_chunk(c0 + 2 * kWaves * cstride, cur, t_ld, true);
        if (c + kWaves < n_chunks) process(c0 + kWaves * cstride, nxt, t_main);
      }
    } else {
      for (int c = wave; c < n_chunks; c += kWaves) {
        const int c0 = t_begin + c * cstride;
        asm volatile("" ::: "memory");
        if constexpr (kPrefetch) {
          Regs nxt;
          load_chunk(c0 + kWaves * cstride, nxt, t_ld, true);
          process(c0, cur, t_main);
          cur = nxt;
        } else {
          process(c0, cur, t_main);
          load_chunk(c0 + kWaves * cstride, cur, t_ld, true);
        }
      }
    }

    // ---- append mode: this split's tail chunks (chunks gc_main .. gc_end - 1
    //      of the sequence that are its own).  Rows before pos come from the
    //      cache (the load range ends at pos, so no row at or past it is
    //      read), rows from pos on from the LDS copy of the new rows.
    if constexpr (BITS == 4 && !ASYM) if (append) {
      for (int gc = gc_main; gc < gc_end; ++gc) {
        int k;
        if (!own_chunk(gc, &k) || wave != k % kWaves) continue;
        const int c0 = gc * kChunk;
        Regs cr;
        load_chunk(c0, cr, max(pos_b, c0), true);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int tk = c0 + 8 * (r >> 2) + 4 * kb + (r & 3);
          if (tk >= pos_b && tk < t_end) {
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) cr.kw[kb][kk] = s_nk[(tk - pos_b) * DW + KK * j + kk];
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int tv = c0 + 8 * j + e;
          if (tv >= pos_b && tv < t_end) cr.vw[e] = s_nv[(tv - pos_b) * DW + (r % DW)];
        }
        const int ts = c0 + (lane & 31);
        if (ts >= pos_b && ts < t_end) {
          cr.sk = s_nks[ts - pos_b];
          cr.sv = s_nvs[ts - pos_b];
        }
        process_chunk(c0, cr, t_end);
      }
    }

    QKVFA_STAMP(2 + wave, lane == 0);
    // ---- merge the eight waves through LDS, one 16-row block at a time
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if constexpr (PK) {   // per-lane sums of the packed softmax: add the four lanes of a row
        l_run[0] += dpp_f<0x124>(l_run[0], l_run[0]);
        l_run[0] += dpp_f<0x128>(l_run[0], l_run[0]);
        s_run[0] += dpp_f<0x124>(s_run[0], s_run[0]);
        s_run[0] += dpp_f<0x128>(s_run[0], s_run[0]);
      }
      if constexpr (PK8) {   // the two lanes (j, b), (j, 8 + b) of a row
        l_run[0] += dpp_f<0x128>(l_run[0], l_run[0]);
        s_run[0] += dpp_f<0x128>(s_run[0], s_run[0]);
      }
      float l = xor_sum(l_run[nb], 16);
      l = xor_sum(l, 32);
      if constexpr (ASYM) {
#pragma unroll
        for (int gi = 0; gi < NGA; ++gi) {
          float sp = xor_sum(sg[nb][gi], 16);
          sp = xor_sum(sp, 32);
#pragma unroll
          for (int p = gi * (NPB / NGA); p < (gi + 1) * (NPB / NGA); ++p) o_acc[nb][p] = sp - o_acc[nb][p];
        }
      } else {
        if constexpr (PK) {   // low-half columns 4 + b (zero unless a chunk was hi/lo) into row b
#pragma unroll
          for (int p = 0; p < NPB; ++p)
#pragma unroll
            for (int i = 0; i < 4; ++i) o_acc[0][p][i] += dpp_f<0x104>(0.0f, o_acc[0][p][i]);
        }
        if constexpr (PK8) {   // low-half columns 8 + b (zero unless a chunk was hi/lo) into row b
#pragma unroll
          for (int p = 0; p < NPB; ++p)
#pragma unroll
            for (int i = 0; i < 4; ++i) o_acc[0][p][i] += dpp_f<0x108>(0.0f, o_acc[0][p][i]);
        }
        float sp = xor_sum(s_run[nb], 16);
        sp = xor_sum(sp, 32);
#pragma unroll
        for (int p = 0; p < NPB; ++p) o_acc[nb][p] -= vbias(p) * sp;
      }
      if constexpr (dup_rows) {   // duplicated rows' columns r + 8 (the low halves) into row r
#pragma unroll
        for (int p = 0; p < NPB; ++p)
#pragma unroll
          for (int i = 0; i < 4; ++i) o_acc[0][p][i] += dpp_f<0x108>(0.0f, o_acc[0][p][i]);
      }
      if (j == 0) {
        s_m[wave][r] = m_run[nb];
        s_l[wave][r] = l;
      }
      float* orow = s_o + (wave * rows_o + r) * OSTR;
      if (ASYM && r < rows_o) {
        // the cache's V order: block p row m is head dim 16 p + m
#pragma unroll
        for (int p = 0; p < NPB; ++p) *reinterpret_cast<float4v*>(orow + 16 * p + 4 * j) = o_acc[nb][p];
      } else if (r < rows_o) {   // rows past R are padding of the 16-row block
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
      }
      __syncthreads();
      const int rows_here = min(16, R - nb * 16);
      for (int idx = threadIdx.x; idx < rows_here * (D / 4); idx += 64 * kWaves) {
        const int rr = idx / (D / 4);
        const int d = 4 * (idx - rr * (D / 4));
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][rr]);
        // every wave empty: weights 0 (not reached by a split with rows)
        const float Mz = (M == -INFINITY) ? 0.0f : M;
        float4v acc = {0.f, 0.f, 0.f, 0.f};
        float den = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float wt = fast_exp2(s_m[w][rr] - Mz);   // empty waves: exp2(-inf) = 0
          acc += wt * *reinterpret_cast<const float4v*>(s_o + (w * rows_o + rr) * OSTR + d);
          den += wt * s_l[w][rr];
        }
        const int64_t grow = grow0 + nb * 16 + rr;
        // nothing attended: output 0, LSE -inf
        const float inv = den > 0.0f ? 1.0f / den : 0.0f;
        const float lse2 = den > 0.0f ? M + log2f(den) : -INFINITY;
        if (direct) {
          *reinterpret_cast<float4v*>(a.out + grow * D + d) = acc * inv;
          if (d == 0 && a.lse) a.lse[grow] = lse2 * kLn2;
        } else {
          // device-coherent stores (sc1): visible to every XCD without an L2 writeback
          __builtin_amdgcn_raw_buffer_store_b128(
              acc * inv, rpart, (uint32_t)((((prow0 + nb * 16 + rr) * a.n_split + split) * D + d) * 4), 0,
              kCoherent);
          if (d == 0)   // log2 units
            __hip_atomic_store(a.part_lse + (prow0 + nb * 16 + rr) * a.n_split + split, lse2, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      __syncthreads();
    }
  };

  // ---- the INT8 decode buffer (TurboAttention §3.3): the last split attends
  //      the buffered rows with plain VALU arithmetic (at most 64 rows), and
  //      first quantizes the call's new rows into the buffer
  if (a.tail_rows > 0 && split == a.n_split - 1) {
    constexpr int nthr = 64 * kWaves;
    const int T = a.tail_rows;
    const int n_tnew = T - a.tail_len;
    const int64_t unit64 = (int64_t)b * a.Hkv + g;
    int8_t* gk = a.tk + unit64 * a.buf_rows * D;
    int8_t* gv = a.tv + unit64 * a.buf_rows * D;
    const float s8k = a.tsk[unit64];
    const float s8v = a.tsv[unit64];
    int8_t* lk = reinterpret_cast<int8_t*>(s_o);        // [kMaxTail][D]
    int8_t* lv = lk + kMaxTail * D;                     // [kMaxTail][D]
    float* lp = reinterpret_cast<float*>(lv + kMaxTail * D);   // [R][kMaxTail]
    // (1) buffered rows -> LDS; new rows quantized into the buffer and LDS
    for (int i = threadIdx.x; i < a.tail_len * (D / 16); i += nthr) {
      reinterpret_cast<uint4v*>(lk)[i] = reinterpret_cast<const uint4v*>(gk)[i];
      reinterpret_cast<uint4v*>(lv)[i] = reinterpret_cast<const uint4v*>(gv)[i];
    }
    for (int i = threadIdx.x; i < 2 * n_tnew * (D / 4); i += nthr) {
      const bool isv = i >= n_tnew * (D / 4);
      const int j4 = isv ? i - n_tnew * (D / 4) : i;
      const int row = j4 / (D / 4);
      const int c4 = j4 - row * (D / 4);
      const float* src = (isv ? a.tv_new : a.tk_new) + (unit64 * n_tnew + row) * D + 4 * c4;
      const float4v x = *reinterpret_cast<const float4v*>(src);
      const float s8 = isv ? s8v : s8k;
      uint32_t packed = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) packed |= ((uint32_t)quant_code8(x[e], s8) & 0xFFu) << (8 * e);
      const int off = (a.tail_len + row) * D + 4 * c4;
      *reinterpret_cast<uint32_t*>((isv ? gv : gk) + off) = packed;
      *reinterpret_cast<uint32_t*>((isv ? lv : lk) + off) = packed;
    }
    __syncthreads();
    // (2) scores in log2 units, one (query row, buffered row) pair per thread
    const float kscale = s8k * a.qk_log2;
    for (int i = threadIdx.x; i < R * T; i += nthr) {
      const int r = i / T;
      const int t = i - r * T;
      const uint16_t* qr = a.q + (grow0 + r) * D;
      const int8_t* kr = lk + t * D;
      float acc = 0.0f;
#pragma unroll 4
      for (int d = 0; d < D; d += 8) {
        const uint4v qw = *reinterpret_cast<const uint4v*>(qr + d);
        const uint2v kw = *reinterpret_cast<const uint2v*>(kr + d);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint16_t qb = (uint16_t)(qw[e >> 1] >> (16 * (e & 1)));
          const float kv = (float)(int8_t)(kw[e >> 2] >> (8 * (e & 3)));
          acc = fmaf(bf16_to_f32(qb), kv, acc);
        }
      }
      lp[r * kMaxTail + t] = acc * kscale;
    }
    __syncthreads();
    // (3) per query row: maximum, p = 2^(s - max) in place, sum -- one wave per row
    for (int r = wave; r < R; r += kWaves) {
      float m = -INFINITY;
      for (int t = lane; t < T; t += 64) m = fmaxf(m, lp[r * kMaxTail + t]);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = xor_max(m, o);
      float l = 0.0f;
      for (int t = lane; t < T; t += 64) {
        const float p = fast_exp2(lp[r * kMaxTail + t] - m);
        lp[r * kMaxTail + t] = p;
        l += p;
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) l = xor_sum(l, o);
      if (lane == 0) {
        s_tm[r] = m;
        s_den[r] = l;
      }
    }
    __syncthreads();
    // (4) O = s8v * sum_t p_t c_t / l, four head dims per thread; the
    //     normalized partial and its LSE go where a split's go
    for (int i = threadIdx.x; i < R * (D / 4); i += nthr) {
      const int r = i / (D / 4);
      const int d = 4 * (i - r * (D / 4));
      float4v acc = {0.f, 0.f, 0.f, 0.f};
      for (int t = 0; t < T; ++t) {
        const float p = lp[r * kMaxTail + t];
        const uint32_t cw = *reinterpret_cast<const uint32_t*>(lv + t * D + d);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(p, (float)(int8_t)(cw >> (8 * e)), acc[e]);
      }
      const float l = s_den[r];
      const float lse2 = s_tm[r] + log2f(l);
      const int64_t grow = grow0 + r;
      const float4v o = acc * (s8v / l);
      if (direct) {
        *reinterpret_cast<float4v*>(a.out + grow * D + d) = o;
        if (d == 0 && a.lse) a.lse[grow] = lse2 * kLn2;
      } else {
        const int64_t prow = prow0 + r;
        __builtin_amdgcn_raw_buffer_store_b128(o, rpart, (uint32_t)(((prow * a.n_split + split) * D + d) * 4), 0,
                                               kCoherent);
        if (d == 0)
          __hip_atomic_store(a.part_lse + prow * a.n_split + split, lse2, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  // ---- a split with no chunk of this sequence: nothing to attend.  It writes
  //      no partial (the merge skips it), only takes its ticket; alone, it
  //      writes the empty result (output 0, LSE -inf).
  } else if (nothing) {
    if (direct) {
      for (int idx = threadIdx.x; idx < R * (D / 4); idx += 64 * kWaves) {
        const int row = idx / (D / 4);
        const int d = 4 * (idx - row * (D / 4));
        const int64_t grow = grow0 + row;
        *reinterpret_cast<float4v*>(a.out + grow * D + d) = float4v{0.f, 0.f, 0.f, 0.f};
        if (d == 0 && a.lse) a.lse[grow] = -INFINITY;
      }
    }
  } else {
    main_body();
  }
  QKVFA_STAMP(10, threadIdx.x == 0);
  if (direct) {
    QKVFA_TRACE_FLUSH();
    return;
  }
  merge_splits();
}

template <int D, int NB, bool PAGED, int BITS, int NGA = 0, int PKR = 0, bool APP = false, bool RNG = false>
hipError_t launch_kernel2(const DecodeArgs& args, dim3 grid, size_t lds, hipStream_t stream) {
  // the merge buffer can pass 64 KiB (eight waves, 16 rows, D = 128): allow
  // this kernel the larger dynamic LDS once
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&decode_kernel<D, NB, PAGED, BITS, NGA, PKR, APP, RNG>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)(max_merge_lds_bytes<D, NB>()));
  if (attr != hipSuccess) return attr;
  decode_kernel<D, NB, PAGED, BITS, NGA, PKR, APP, RNG><<<grid, dim3(64 * waves_for(NB)), lds, stream>>>(args);
  return hipGetLastError();
}

template <int D, int NB, bool PAGED, int BITS, int NGA = 0, int PKR = 0, bool RNG = false>
hipError_t launch_kernel1(const DecodeArgs& args, dim3 grid, size_t lds, hipStream_t stream) {
  if constexpr (BITS == 4 && NGA == 0) {
    if (args.k_new != nullptr) return launch_kernel2<D, NB, PAGED, BITS, NGA, PKR, true, RNG>(args, grid, lds, stream);
  } else {
    if (args.k_new != nullptr) return hipErrorInvalidValue;   // the API allows append on 4-bit rows only
  }
  return launch_kernel2<D, NB, PAGED, BITS, NGA, PKR, false, RNG>(args, grid, lds, stream);
}

// symmetric rows with at most 4 or at most 8 query rows per group: the
// packed-softmax kernels
template <int D, int NB, bool PAGED, int BITS, int NGA = 0, bool RNG = false>
hipError_t launch_kernel(const DecodeArgs& args, dim3 grid, size_t lds, hipStream_t stream) {
  if constexpr (NB == 1 && NGA == 0) {
    if (args.G * args.Sq <= 4) return launch_kernel1<D, NB, PAGED, BITS, NGA, 4, RNG>(args, grid, lds, stream);
    return launch_kernel1<D, NB, PAGED, BITS, NGA, 8, RNG>(args, grid, lds, stream);
  } else {
    return launch_kernel1<D, NB, PAGED, BITS, NGA, 0, RNG>(args, grid, lds, stream);
  }
}

template <int D, int NB>
hipError_t launch_nb(const DecodeArgs& args, int B, int Hkv, int n_split, int bits, hipStream_t stream) {
  dim3 grid((uint32_t)n_split * (uint32_t)Hkv * (uint32_t)B);
  const int R = args.G * args.Sq;
  size_t lds = merge_lds_bytes(D, waves_for(NB), R, n_split);
  if (args.tail_rows > 0 && lds < tail_lds_bytes(D, R)) lds = tail_lds_bytes(D, R);
  if (args.kp != nullptr) {
    if (args.ng == 1) return launch_kernel<D, NB, false, 4, 1>(args, grid, lds, stream);
    if (args.ng == 2) return launch_kernel<D, NB, false, 4, 2>(args, grid, lds, stream);
    if constexpr (D == 128) return launch_kernel<D, NB, false, 4, 4>(args, grid, lds, stream);
    return hipErrorInvalidValue;
  }
  if (bits == 2) return launch_kernel<D, NB, false, 2>(args, grid, lds, stream);
  if (bits == 3) return launch_kernel<D, NB, false, 3>(args, grid, lds, stream);
  if (args.block_table != nullptr) return launch_kernel<D, NB, true, 4>(args, grid, lds, stream);
  if (n_split - (args.tail_rows > 0 ? 1 : 0) >= kRangeSplits)
    return launch_kernel<D, NB, false, 4, 0, true>(args, grid, lds, stream);
  return launch_kernel<D, NB, false, 4>(args, grid, lds, stream);
}

template <int D>
hipError_t launch_d(const DecodeArgs& args, int B, int Hkv, int n_split, int bits, hipStream_t stream) {
  const int R = args.G * args.Sq;
  if (row_blocks_for(R) == 1) return launch_nb<D, 1>(args, B, Hkv, n_split, bits, stream);
  if (row_blocks_for(R) == 2) return launch_nb<D, 2>(args, B, Hkv, n_split, bits, stream);
  return launch_nb<D, 4>(args, B, Hkv, n_split, bits, stream);
}

}  // namespace

DecodePlan plan_decode(int64_t B, int64_t Hkv, int64_t rows, int64_t kv_len, int D, int num_splits,
                       int num_cus, bool ragged) {
  const int64_t chunks = (kv_len + kChunk - 1) / kChunk;
  const int64_t units = B * Hkv;
  const int64_t rows_per_group = rows / units;
  const int waves = waves_for(row_blocks_for(rows_per_group));
  int64_t ns;
  if (num_splits <= 0) {
    // eight waves per CU (one 8-wave or two 4-wave workgroups): measured best
    // on MI355X for both a 128-group 8K-token and an 8-group 128K-token
    // decode.  Every workgroup starts at once and streams its chunks at the
    // shared HBM rate; more splits add per-split epilogue and merge latency
    // without adding bandwidth
    const int64_t target_wgs = (int64_t)(num_cus > 0 ? num_cus : 256) * 8 / waves;
    ns = (target_wgs + units - 1) / units;
    const int64_t max_ns = chunks / waves > 0 ? chunks / waves : 1;   // >= one chunk per wave
    if (ns > max_ns) ns = max_ns;
    // Lengths that differ per sequence (known only on the device): the plan
    // covers the longest, and a shorter sequence has shorter (or empty late)
    // splits.  Splits of at most kRaggedSplitChunks chunks keep the longest
    // sequences from finishing alone (measured on a 64-sequence batch of
    // 512..16384 tokens: 128-chunk splits 138 us, one split each 158 us)
    if (ragged) {
      const int64_t ns_r = (chunks + kRaggedSplitChunks - 1) / kRaggedSplitChunks;
      if (ns < ns_r) ns = ns_r;
    }
  } else {
    ns = num_splits;
  }
  if (ns > chunks) ns = chunks;
  if (ns > 1024) ns = 1024;
  // the merging workgroup keeps (rows per group) * ns weights in LDS
  const int64_t rpg = rows / units;
  if (ns > kMaxMergeLse / rpg) ns = kMaxMergeLse / rpg;
  // partial outputs (rows * ns * D fp32) are addressed with 32-bit offsets
  const int64_t max_ns_bytes = ((int64_t)1 << 31) / ((int64_t)rows * D * 4 + 1);
  if (ns > max_ns_bytes) ns = max_ns_bytes;
  if (ns < 1) ns = 1;
  DecodePlan p;
  p.n_split = (int)ns;   // <= chunks: every split has a chunk
  return p;
}

// Workspace: one uint32 ticket per (batch, KV head) at offset 0 (a fixed place
// for a given B*Hkv, whatever the other sizes), then partial outputs
// [rows][n_split][D] fp32, then partial LSE [rows][n_split] fp32 (log2 units).
static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t decode_workspace_bytes(int64_t rows, int64_t units, int D, int n_split) {
  if (n_split <= 1) return 0;
  return align256((size_t)units * sizeof(uint32_t)) +
         align256((size_t)rows * n_split * D * sizeof(float)) + (size_t)rows * n_split * sizeof(float);
}

hipError_t launch_decode(const uint16_t* q, const uint8_t* kc, const uint16_t* ks,
                         const uint8_t* vc, const uint16_t* vs, int64_t B, int64_t Hq,
                         int64_t Hkv, int64_t Sq, int64_t kv_len, int64_t C, int D,
                         float softmax_scale, const DecodePlan& plan, float* out, float* lse,
                         void* workspace, const DecodeAppend* append, const DecodeVarlen* varlen,
                         const DecodeTail* tail, int bits, hipStream_t stream, const DecodeAsym* asym,
                         const int32_t* kv_heads, int64_t Hkv_all, int64_t ticket_slots) {
  DecodeArgs a;
  a.kv_heads = kv_heads;
  a.Hkv_all = (int)(kv_heads ? Hkv_all : Hkv);
  a.q = q; a.kc = kc; a.ks = ks; a.vc = vc; a.vs = vs;
  a.kp = nullptr; a.vp = nullptr; a.ng = 1; a.gshift = 0;
  if (asym) {
    a.kp = asym->k_params;
    a.vp = asym->v_params;
    a.ng = D / asym->group;
    a.gshift = 31 - __builtin_clz((unsigned)asym->group);
  }
  a.out = out; a.lse = lse;
  a.k_new = nullptr; a.v_new = nullptr;
  a.kc_w = nullptr; a.ks_w = nullptr; a.vc_w = nullptr; a.vs_w = nullptr;
  a.pos = 0; a.n_new = 0;
  if (append) {
    a.k_new = append->k_new;
    a.v_new = append->v_new;
    a.kc_w = const_cast<uint8_t*>(kc);
    a.ks_w = const_cast<uint16_t*>(ks);
    a.vc_w = const_cast<uint8_t*>(vc);
    a.vs_w = const_cast<uint16_t*>(vs);
    a.n_new = (int)append->n_new;
    a.pos = (int)(kv_len - append->n_new);
  }
  a.kv_lens = nullptr; a.block_table = nullptr;
  a.len_cap = 0; a.page_size = 0; a.max_pages = 0; a.num_pages = 0;
  if (varlen) {
    a.kv_lens = varlen->kv_lens;
    a.block_table = varlen->block_table;
    a.len_cap = (int)(kv_len - a.n_new);
    a.page_size = (int)varlen->page_size;
    a.max_pages = (int)varlen->max_pages;
    a.num_pages = (int)varlen->num_pages;
  }
  a.tk = nullptr; a.tv = nullptr; a.tsk = nullptr; a.tsv = nullptr; a.tk_new = nullptr; a.tv_new = nullptr;
  a.tail_len = 0; a.tail_rows = 0; a.buf_rows = 0;
  if (tail && tail->buf_len + tail->n_new > 0) {
    a.tk = tail->k_buf; a.tv = tail->v_buf;
    a.tsk = tail->k_s8; a.tsv = tail->v_s8;
    a.tk_new = tail->k_new; a.tv_new = tail->v_new;
    a.tail_len = (int)tail->buf_len;
    a.tail_rows = (int)(tail->buf_len + tail->n_new);
    a.buf_rows = (int)tail->buf_rows;
  }
  a.part_o = nullptr; a.part_lse = nullptr; a.tickets = nullptr; a.part_bytes = 0;
  if (plan.n_split > 1) {
    const int64_t rows = B * Hkv * (Hq / a.Hkv_all) * Sq;   // this call's query rows
    char* w = static_cast<char*>(workspace);
    const size_t t = align256((size_t)std::max<int64_t>(B * Hkv, ticket_slots) * sizeof(uint32_t));
    const size_t o = align256((size_t)rows * plan.n_split * D * sizeof(float));
    a.tickets = reinterpret_cast<uint32_t*>(w);
    a.part_o = reinterpret_cast<float*>(w + t);
    a.part_lse = reinterpret_cast<float*>(w + t + o);
    a.part_bytes = (int)((size_t)rows * plan.n_split * D * sizeof(float));
  }
  a.C = C;
  a.Hq = (int)Hq; a.Hkv = (int)Hkv; a.G = (int)(Hq / a.Hkv_all); a.Sq = (int)Sq; a.kv_len = (int)kv_len;
  a.n_split = plan.n_split;
  a.qk_log2 = softmax_scale * kLog2e;
  if (D == 128) return launch_d<128>(a, (int)B, (int)Hkv, plan.n_split, bits, stream);
  return launch_d<64>(a, (int)B, (int)Hkv, plan.n_split, bits, stream);
}

// ---- allocation-free decode: one static scratch per device ----------------
// A file-scope device array: each device holds its own copy at its own
// address from module load until the process ends.  In host code its name
// stands for a host-side shadow, never a device address, so host code uses
// only the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

__global__ void zero_words(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

hipError_t decode_scratch(void** ptr, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    // the tickets must start at zero; a kernel rather than a memset, so a
    // first call under stream capture records no memset node
    hipLaunchKernelGGL(zero_words, dim3(16), dim3(256), 0, stream, static_cast<uint32_t*>(p), (int)kScratchTickets);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

#ifdef QKVFA_PHASE_TRACE
hipError_t trace_read(uint64_t* dst, int64_t n_wgs) {
  if (n_wgs < 0 || n_wgs > kTraceWgs) return hipErrorInvalidValue;
  return hipMemcpyFromSymbol(dst, HIP_SYMBOL(g_trace), (size_t)n_wgs * kTraceSlots * sizeof(uint64_t), 0,
                             hipMemcpyDeviceToHost);
}
#endif

}  // namespace qkvfa
