/*
 * qkvfa.h -- int4-KV FlashAttention for AMD MI355X (gfx950): the C ABI.
 *
 * The library computes attention directly over an int4-quantized KV cache
 * and dequantizes inside its kernels, so no dequantized K/V ever reaches HBM
 * ("Quantized Cross-Attention: Extending FlashAttention-3 with In-SRAM
 * Dequantization", §3.1 and §3.2; the Open-TQ-Metal abstract on the
 * "Attention Quantization" listing: int4 KV quantized on the fly and attended
 * in compressed form).  Three operations follow the prefill / append / decode
 * statement of TurboAttention (arXiv 2412.08585) §2.1: quantize-and-append,
 * decode attention of a few query rows, prefill attention (causal or not).
 *
 * Conventions shared by every call
 * --------------------------------
 * All tensors are dense, row-major, in device memory owned by the caller.
 * The library never allocates or frees memory and keeps no pointer after a
 * call returns.  Work is enqueued on `stream` (a hipStream_t; NULL = the
 * default stream) and runs asynchronously: the caller keeps every buffer
 * alive until the stream has finished it.
 *
 *   B    batch                     Hq   query heads     Hkv  KV heads
 *   G    Hq / Hkv (GQA group)      D    head dim (64 or 128)
 *   Sq   query rows per head       C    cache capacity in tokens
 *   kv_len  number of valid cache rows the query attends
 *
 *   KV cache   codes  uint8  [B, Hkv, C, D/2]   packed int4, two's complement,
 *                                               element 2i in bits 0-3 of byte i,
 *                                               element 2i+1 in bits 4-7
 *              scales uint16 [B, Hkv, C]        fp16 bit patterns, one per
 *                                               (token, KV head)
 *   value of element d of row t:  fp16(scales[t]) * code[t][d]
 *   Q          uint16 [B, Hq, Sq, D]            bfloat16 bit patterns
 *   out        float  [B, Hq, Sq, D]
 *   lse        float  [B, Hq, Sq]               natural-log log-sum-exp of the
 *                                               scaled scores, or NULL
 *   query head h reads KV head h / G.
 *
 * Errors: every argument is checked before anything is enqueued; a failing
 * call enqueues nothing, returns a nonzero qkv_status and leaves a message
 * for qkv_last_error() (thread-local).  A HIP launch error returns
 * QKV_ERR_HIP.  No C++ exception crosses this interface.
 * Preconditions that are not checked (their violation gives unspecified
 * output, never an out-of-bounds access): finite inputs; row absmax of
 * quantized data <= 7 * 65504 (fp16 scales); scores q.k * softmax_scale
 * finite in fp32.  Queries may hold any finite bfloat16: where a query
 * group's largest |q| reaches 65536 the kernels scale it by an exact power of
 * two into fp16 range and fold the inverse into the score scale.
 * Precision: the softmax probabilities enter the PV product as fp16
 * P~ = p * s_V (the V scale folded into P: "Quantized Cross-Attention", §3.4,
 * softmax in quantized space, in its exact reading); where a V scale
 * passes the limit at which one fp16 rounding of P~ could cost more than
 * 3.5e-3 of an output (int4 1.02, 3-bit 2.39, 2-bit 7.17; asymmetric rows:
 * s max(z, 15 - z) above 7.17; channel outliers, TurboAttention §3.1), P~ is
 * taken as an fp16 high/low pair, so outputs stay within 4e-3 of fp64
 * attention over the dequantized cache.
 */
#ifndef QKVFA_H
#define QKVFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QKV_OK = 0,
  QKV_ERR_INVALID_ARG = 1, /* a size, pointer or range is invalid          */
  QKV_ERR_UNSUPPORTED = 2, /* valid, but outside what the kernels implement */
  QKV_ERR_WORKSPACE = 3,   /* workspace missing or too small               */
  QKV_ERR_HIP = 4          /* the HIP runtime reported an error            */
} qkv_status;

/* Static text naming a status. */
const char* qkv_status_string(qkv_status s);
/* Message of the last failing call on this thread ("" if none). */
const char* qkv_last_error(void);
/* Library version, major*10000 + minor*100 + patch. */
int qkv_version(void);

/*
 * (a) Quantize-and-append.  Quantizes T new rows of one tensor (call once for
 * K and once for V) into cache rows [pos, pos + T); rows outside that range
 * are not touched.  Per row of D fp32 values x:
 *     scale = fp16_rne( max|x| / 7 )        (IEEE fp32 division)
 *     code  = clamp( rint( x / float(scale) ), -8, 7 )   (IEEE fp32 division,
 *             round half to even); scale == 0 gives all-zero codes.
 * Follows: the per-(token, head) scale layout of the kernel signature in
 * "Quantized Cross-Attention ..." §4.1 (GROUP_SIZE = D); int4 on the fly
 * (Open-TQ-Metal abstract); append k_t, v_t to the cache (TurboAttention
 * §2.1).
 *   src     float [B, Hkv, T, D], device, 16-byte aligned
 *   codes   uint8 [B, Hkv, C, D/2], device, 16-byte aligned (written)
 *   scales  uint16 [B, Hkv, C], device, 2-byte aligned (written)
 * Requires B, Hkv >= 1, T >= 0 (T == 0 enqueues nothing), D in {64, 128},
 * 0 <= pos, pos + T <= C.
 */
qkv_status qkv_quantize_append(const float* src, uint8_t* codes, uint16_t* scales,
                               int64_t B, int64_t Hkv, int64_t T, int64_t D,
                               int64_t C, int64_t pos, void* stream);

/*
 * (a') The same quantize-and-append for K and V of the same T tokens in one
 * launch (a decode step appends k_t and v_t together, TurboAttention §2.1).
 * Results are identical to two qkv_quantize_append calls.
 *   k_src, v_src      float [B, Hkv, T, D], device, 16-byte aligned
 *   k_codes, v_codes  uint8 [B, Hkv, C, D/2], device, 16-byte aligned (written)
 *   k_scales, v_scales uint16 [B, Hkv, C], device, 2-byte aligned (written)
 * Same requirements as qkv_quantize_append.
 */
qkv_status qkv_quantize_append_kv(const float* k_src, const float* v_src,
                                  uint8_t* k_codes, uint16_t* k_scales,
                                  uint8_t* v_codes, uint16_t* v_scales,
                                  int64_t B, int64_t Hkv, int64_t T, int64_t D,
                                  int64_t C, int64_t pos, void* stream);

/*
 * (b) Decode attention: each of the Sq query rows of every (batch, head)
 * attends cache rows [0, kv_len) with no mask (append-then-attend,
 * TurboAttention §2.1).  The KV length is split into `num_splits` ranges
 * processed in parallel; each range yields a partial output normalized over
 * its own keys plus its log-sum-exp, and the partials are merged with the
 * log-sum-exp rule (the final normalization with running max and sum of
 * FlashAttention, TurboAttention §2.2).  The K/V tile of a KV head is read
 * once for all G query heads of its group.
 *   q        uint16 [B, Hq, Sq, D] bf16 bits, device, 16-byte aligned
 *   k_codes, v_codes   uint8 [B, Hkv, C, D/2], device, 16-byte aligned
 *   k_scales, v_scales uint16 [B, Hkv, C], device, 2-byte aligned
 *   softmax_scale      multiplies Q.K before the softmax
 *   num_splits         0 = chosen by the library; else 1..1024 (clamped to
 *                      the number of 32-token chunks of kv_len)
 *   out      float [B, Hq, Sq, D], device, 16-byte aligned (written)
 *   lse      float [B, Hq, Sq] or NULL (written)
 *   workspace, workspace_bytes: device scratch of at least
 *            qkv_decode_workspace_bytes(...) bytes (may be NULL when that
 *            is 0), 16-byte aligned.  Its first 4 * B * Hkv bytes (rounded
 *            up to 256) hold one ticket counter per (batch, KV head); the
 *            rest holds split partials.  The tickets must be zero when a
 *            call starts and every completed call leaves them zero, so a
 *            workspace zeroed once serves any sequence of calls with the
 *            same B * Hkv (other sizes may change between calls).  Zero it
 *            again before using it with a different B * Hkv.  Calls that
 *            share a workspace must not run concurrently.
 * Requires D in {64, 128}, Hq % Hkv == 0, 1 <= kv_len <= C,
 * 1 <= G * Sq <= 64 (more rows belong to qkv_prefill).
 */
/* Workspace bytes for a decode of these sizes: enough for qkv_decode,
 * qkv_decode_append and qkv_decode_paged (kv_len = max_kv_len), whose split
 * plans may differ; 0 when the plan has a single split. */
size_t qkv_decode_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq,
                                  int64_t kv_len, int64_t D, int num_splits);
/* The split count the library would use for num_splits = 0 with every
 * sequence of length kv_len (the current device's CU count is queried once
 * and cached per device).  With per-sequence lengths (qkv_decode_paged with
 * kv_lens) splits are also capped at 4096 tokens each, so the count can be
 * larger. */
int qkv_decode_auto_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq,
                           int64_t kv_len, int64_t D);
qkv_status qkv_decode(const uint16_t* q,
                      const uint8_t* k_codes, const uint16_t* k_scales,
                      const uint8_t* v_codes, const uint16_t* v_scales,
                      int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t kv_len,
                      int64_t C, int64_t D, float softmax_scale, int num_splits,
                      float* out, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * qkv_decode without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments and results as qkv_decode (the same
 * kernels and split plan: outputs are bit-identical); it calls no hipMalloc,
 * hipFree or allocating routine.  The tickets and split partials live in a
 * static device array of the library, 16 MiB per device, held from module
 * load until the process ends: 16 KiB of ticket counters (B * Hkv <= 4096)
 * and up to 16 MiB - 16 KiB of partials (Sq * Hq * B * n_split * (D + 1) * 4
 * bytes, rounded up).  Larger calls fail with QKV_ERR_WORKSPACE before any
 * launch.  The first call on a device resolves that device's copy and zeroes
 * its tickets with a small kernel on `stream`; every completed call leaves
 * them zero.  All calls on one device share the array, so calls that overlap
 * on one device (other streams, other threads) race: the caller serializes
 * them.
 */
qkv_status qkv_decode_noalloc(const uint16_t* q,
                              const uint8_t* k_codes, const uint16_t* k_scales,
                              const uint8_t* v_codes, const uint16_t* v_scales,
                              int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t kv_len,
                              int64_t C, int64_t D, float softmax_scale, int num_splits,
                              float* out, float* lse, void* stream);

/*
 * 2- and 3-bit rows (the bit-width parameter of "Quantized Cross-Attention"
 * §4.1; 2-bit heads in TurboAttention §3.2).  A b-bit row of D codes takes
 * D*b/8 bytes: scale = fp16(absmax / (2^(b-1) - 1)) by IEEE fp32 division,
 * code = clamp(rint(x / scale), -2^(b-1), 2^(b-1) - 1).  2 bits: element i
 * in bits 2(i % 4) of byte i / 4.  3 bits: those 2-bit fields of the low two
 * bits (D/4 bytes), then the top bit of every code, element i at bit i % 8 of
 * byte D/4 + i / 8.  bits = 4 is the int4 format of the other calls.
 *   qkv_quantize_append_kv_bits: qkv_quantize_append_kv for b-bit rows;
 *     k_codes, v_codes uint8 [B, Hkv, C, D*bits/8].
 *   qkv_decode_bits: qkv_decode over b-bit rows (same workspace as
 *     qkv_decode: qkv_decode_workspace_bytes).
 * Requires bits in {2, 3, 4} (QKV_ERR_UNSUPPORTED otherwise) and the
 * requirements of the int4 calls.
 */
qkv_status qkv_quantize_append_kv_bits(const float* k_src, const float* v_src,
                                       uint8_t* k_codes, uint16_t* k_scales,
                                       uint8_t* v_codes, uint16_t* v_scales,
                                       int64_t B, int64_t Hkv, int64_t T, int64_t D,
                                       int64_t C, int64_t pos, int bits, void* stream);
qkv_status qkv_decode_bits(const uint16_t* q,
                           const uint8_t* k_codes, const uint16_t* k_scales,
                           const uint8_t* v_codes, const uint16_t* v_scales,
                           int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t kv_len,
                           int64_t C, int64_t D, int bits, float softmax_scale, int num_splits,
                           float* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Per-head bit widths (TurboAttention, arXiv 2412.08585, §3.2: a layer keeps
 * some KV heads at 2 bits and the rest at 4).  A layer's cache is split by
 * width: one cache per width, each holding a subset of the layer's Hkv KV
 * heads, listed by kv_heads (int32 [Hkv_sub], device, 4-byte aligned; ids
 * are clamped into [0, Hkv); each KV head of the layer belongs to one cache).
 *   qkv_quantize_append_kv_heads: quantizes rows [pos, pos + T) of the
 *     listed heads of k_src, v_src (float [B, Hkv, T, D], device) into a
 *     b-bit cache of Hkv_sub heads (k_codes, v_codes uint8
 *     [B, Hkv_sub, C, D*bits/8]; k_scales, v_scales fp16 [B, Hkv_sub, C]);
 *     cache head i takes source head kv_heads[i].
 *   qkv_decode_heads: qkv_decode for the query heads of the listed KV heads
 *     (query head h uses KV head h / (Hq/Hkv) of the layer): q, out, lse are
 *     the layer's [B, Hq, Sq, D] / [B, Hq, Sq]; only the rows of the listed
 *     heads' query heads are written.  One call per width covers the layer.
 *     Workspace: qkv_decode_workspace_bytes(B, (Hq/Hkv)*Hkv_sub, Hkv_sub, Sq,
 *     kv_len, D, num_splits), same ticket contract as qkv_decode.
 * Requires bits in {2, 3, 4}, 1 <= Hkv_sub <= Hkv (QKV_ERR_INVALID_ARG
 * otherwise), and the requirements of the int4 calls.
 */
qkv_status qkv_quantize_append_kv_heads(const float* k_src, const float* v_src,
                                        const int32_t* kv_heads, int64_t Hkv_sub,
                                        uint8_t* k_codes, uint16_t* k_scales,
                                        uint8_t* v_codes, uint16_t* v_scales,
                                        int64_t B, int64_t Hkv, int64_t T, int64_t D,
                                        int64_t C, int64_t pos, int bits, void* stream);
qkv_status qkv_decode_heads(const uint16_t* q,
                            const uint8_t* k_codes, const uint16_t* k_scales,
                            const uint8_t* v_codes, const uint16_t* v_scales,
                            const int32_t* kv_heads, int64_t Hkv_sub,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t kv_len,
                            int64_t C, int64_t D, int bits, float softmax_scale, int num_splits,
                            float* out, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Asymmetric group-wise 4-bit rows (TurboAttention, arXiv 2412.08585, §2.3:
 * a scale s and a zero point z per quantization group, value s (code - z);
 * §3.1 keeps asymmetric INT4 groups for K and V; "Quantized Cross-Attention"
 * §4.1: scales [b, h, seq_kv, dim/GROUP_SIZE]).  Each row (one token of one
 * KV head) is split into groups of `group` consecutive elements (32, 64 or
 * 128, at most D); per group, in IEEE fp32:
 *   lo = min(0, min x), hi = max(0, max x)
 *   s  = fp16_rne((hi - lo) / 15)
 *   z  = clamp(rint(-lo / s), 0, 15)
 *   u  = clamp(rint(x / s) + z, 0, 15)       (rint: half to even)
 * and a zero s gives z = 0 and all codes 0.  Layout:
 *   codes   uint8 [B, Hkv, C, D/2], unsigned u, nibble n of a row at bits
 *           4 (n % 2) of byte n / 2, in a fixed order per tensor (so that
 *           each matrix-product block of the decode reads one group):
 *             K rows: chunk c = 4 k + j (elements 8c .. 8c+7, k < D/32,
 *               j < 4) in dword (D/32) j + k, element 8c + i in nibble i;
 *             V rows: element 16 p + w (p < D/16, w < 16) in nibble p of
 *               dword w (D = 128), or in nibble p + 4 (w / 8) of dword
 *               w % 8 (D = 64)
 *   params  uint32 [B, Hkv, C, D/group]: s's fp16 bits in bits 0-15, z in
 *           bits 16-19, other bits zero; 4-byte aligned
 *   qkv_quantize_append_kv_asym: quantizes T new rows of K and V into cache
 *     rows [pos, pos + T) (arguments as qkv_quantize_append_kv).
 *   qkv_decode_asym: qkv_decode over such a cache (same workspace contract:
 *     qkv_decode_workspace_bytes).  Codes enter the matrix products exactly;
 *     scales and zero points are applied per group in fp32.
 * Requires group in {32, 64, 128} and group <= D (QKV_ERR_UNSUPPORTED
 * otherwise) and the requirements of the int4 calls.
 */
qkv_status qkv_quantize_append_kv_asym(const float* k_src, const float* v_src,
                                       uint8_t* k_codes, uint32_t* k_params,
                                       uint8_t* v_codes, uint32_t* v_params,
                                       int64_t B, int64_t Hkv, int64_t T, int64_t D,
                                       int64_t C, int64_t pos, int group, void* stream);
qkv_status qkv_decode_asym(const uint16_t* q,
                           const uint8_t* k_codes, const uint32_t* k_params,
                           const uint8_t* v_codes, const uint32_t* v_params,
                           int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t kv_len,
                           int64_t C, int64_t D, int group, float softmax_scale, int num_splits,
                           float* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * (a)+(b) One decode step in one launch: append, then attend.  Quantizes
 * n_new new K and V rows into cache rows [pos, pos + n_new), exactly as
 * qkv_quantize_append_kv does, then computes qkv_decode over cache rows
 * [0, pos + n_new) (TurboAttention §2.1: a decode step appends k_t and v_t
 * to the cache and its query attends the updated cache).  The rows written,
 * out and lse are bit-identical to qkv_quantize_append_kv followed by
 * qkv_decode with kv_len = pos + n_new and the same num_splits; the single
 * launch saves the second kernel's start and drain.
 *   k_new, v_new   float [B, Hkv, n_new, D], device, 16-byte aligned
 *   k_codes, v_codes, k_scales, v_scales: the cache as for qkv_decode; rows
 *                  [pos, pos + n_new) are written, no other row is touched
 *   workspace      as for qkv_decode with kv_len = pos + n_new (same tickets
 *                  contract; qkv_decode_workspace_bytes gives the size)
 *   other arguments as for qkv_decode.
 * Requires 0 <= pos, 1 <= n_new <= 64, pos + n_new <= C, and the
 * qkv_decode requirements.  The new rows must not alias the cache.
 */
qkv_status qkv_decode_append(const uint16_t* q, const float* k_new, const float* v_new,
                             uint8_t* k_codes, uint16_t* k_scales,
                             uint8_t* v_codes, uint16_t* v_scales,
                             int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq,
                             int64_t pos, int64_t n_new, int64_t C, int64_t D,
                             float softmax_scale, int num_splits, float* out, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * (a)+(b) over a ragged and optionally paged cache: the serving form of the
 * decode step (TurboAttention §2.1: during decoding every sequence of the
 * batch appends its new token's K and V to its own cache and attends it;
 * sequences differ in length).  Sequence b attends its own rows
 * [0, L_b), L_b = kv_lens[b] + n_new, after first quantizing its n_new new
 * rows into rows [kv_lens[b], L_b) exactly as qkv_quantize_append_kv does.
 * Per sequence, out, lse and the rows written are the same as qkv_decode_append
 * (n_new > 0) or qkv_decode (n_new = 0) on that sequence's rows alone.
 *   k_codes, v_codes   uint8 [num_pages, Hkv, page_size, D/2] page pool,
 *                      device, 16-byte aligned
 *   k_scales, v_scales uint16 [num_pages, Hkv, page_size], device
 *   block_table  int32 [B, max_pages], device, or NULL.  Token t of sequence
 *                b is row t % page_size of page block_table[b, t / page_size]
 *                (ids outside [0, num_pages) are clamped into it, so no access
 *                leaves the pool).  Needs page_size % 32 == 0.
 *                NULL: sequence b owns page b (a contiguous cache
 *                [B, Hkv, C, D/2] is the pool with page_size = C); needs
 *                max_pages == 1 and num_pages >= B, any page_size.
 *   kv_lens      int32 [B], device: rows already cached per sequence (before
 *                this call's new rows), or NULL: every sequence holds
 *                max_kv_len - n_new.  Values are clamped to
 *                [0, max_kv_len - n_new].  A sequence with L_b = 0 gets
 *                out = 0 and lse = -inf.
 *   k_new, v_new float [B, Hkv, n_new, D], device, 16-byte aligned, read
 *                only when n_new > 0 (NULL allowed otherwise); must not alias
 *                the cache.  The pages they land in must belong to one
 *                sequence each.
 *   n_new        0..64 rows appended per sequence (0: attend only)
 *   max_kv_len   upper bound of every L_b, 1 <= max_kv_len <= max_pages *
 *                page_size, >= n_new.  The split plan and the workspace size
 *                follow it (qkv_decode_workspace_bytes with kv_len =
 *                max_kv_len); splits past a sequence's length do no work.
 *   other arguments as for qkv_decode (same workspace and tickets contract).
 * Requires the qkv_decode requirements with kv_len = max_kv_len and
 * C = max_pages * page_size.
 */
qkv_status qkv_decode_paged(const uint16_t* q, const float* k_new, const float* v_new,
                            uint8_t* k_codes, uint16_t* k_scales,
                            uint8_t* v_codes, uint16_t* v_scales,
                            const int32_t* block_table, const int32_t* kv_lens,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t n_new,
                            int64_t max_kv_len, int64_t page_size, int64_t max_pages,
                            int64_t num_pages, int64_t D, float softmax_scale, int num_splits,
                            float* out, float* lse, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * INT8 decode buffer (TurboAttention §3.3 decoding buffer, and the
 * implementation paragraph of its §5): the newest tokens of every
 * (batch, KV head) -- at most 64 -- are kept as INT8 codes under one
 * universal scale, so a decode step quantizes only its own token; outliers
 * beyond the scale's range are clamped, so buffered rows are never
 * re-quantized.  A full buffer is flushed into the int4 cache.
 * Buffer layout: k_buf, v_buf int8 [B, Hkv, buf_rows, D] (1 <= buf_rows <=
 * 64), device, 16-byte aligned; k_s8, v_s8 float [B, Hkv] universal scales.
 * A buffered value is s8 * code, code = clamp(rint(x / s8), -127, 127) with
 * IEEE fp32 division (s8 = 0 gives code 0).
 */

/* Universal scales from the cache's value range: s8 = (7 * max_t s[t]) / 127
 * over rows [0, L) of every (batch, KV head), for K (k_scales -> k_s8) and V;
 * 0 when L = 0.  k_scales, v_scales uint16 fp16 bits [B, Hkv, C], device.
 * Requires 0 <= L <= C. */
qkv_status qkv_buffer_scale(const uint16_t* k_scales, const uint16_t* v_scales,
                            int64_t B, int64_t Hkv, int64_t L, int64_t C,
                            float* k_s8, float* v_s8, void* stream);

/* Flush: buffered rows [0, T) of every (batch, KV head), each value taken as
 * the fp32 product s8 * code, quantized as int4 rows (as
 * qkv_quantize_append_kv does) into cache rows [pos, pos + T).  The buffer is
 * only read.  Requires 0 <= T <= buf_rows <= 64, 0 <= pos, pos + T <= C. */
qkv_status qkv_buffer_flush(const int8_t* k_buf, const int8_t* v_buf,
                            const float* k_s8, const float* v_s8,
                            int64_t buf_rows, int64_t T,
                            uint8_t* k_codes, uint16_t* k_scales,
                            uint8_t* v_codes, uint16_t* v_scales,
                            int64_t B, int64_t Hkv, int64_t D, int64_t C, int64_t pos,
                            void* stream);

/* Decode over int4 cache rows [0, kv_len) followed by buffered rows
 * [0, buf_len + n_new), in one launch.  The n_new new rows k_new, v_new
 * (float [B, Hkv, n_new, D], device, 16-byte aligned; may be NULL when n_new
 * is 0) are first quantized into buffer rows [buf_len, buf_len + n_new).  The
 * cache rows are split as by qkv_decode (num_splits applies to them); one
 * more split per (batch, KV head) attends the buffered rows, and the LSE merge
 * combines them.  Other arguments as for qkv_decode; the workspace size is
 * qkv_decode_buffered_workspace_bytes (0 when there is a single split).
 * Requires 0 <= kv_len <= C, 0 <= buf_len, 0 <= n_new,
 * buf_len + n_new <= buf_rows <= 64, kv_len + buf_len + n_new >= 1, and the
 * qkv_decode requirements on the other arguments. */
size_t qkv_decode_buffered_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq,
                                           int64_t kv_len, int64_t D, int num_splits);
qkv_status qkv_decode_buffered(const uint16_t* q, const float* k_new, const float* v_new,
                               const uint8_t* k_codes, const uint16_t* k_scales,
                               const uint8_t* v_codes, const uint16_t* v_scales,
                               int8_t* k_buf, int8_t* v_buf,
                               const float* k_s8, const float* v_s8,
                               int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq,
                               int64_t kv_len, int64_t C,
                               int64_t buf_rows, int64_t buf_len, int64_t n_new, int64_t D,
                               float softmax_scale, int num_splits, float* out, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * (c) Prefill attention, tiled with online softmax (FlashAttention tiling,
 * TurboAttention §2.2).  causal = 0: every row sees [0, kv_len).
 * causal = 1: query row i (0 <= i < Sq) is token kv_len - Sq + i and sees
 * keys j <= i + kv_len - Sq (bottom-right aligned); key tiles entirely above
 * the diagonal are never loaded.
 *   arguments as for qkv_decode (no workspace).
 * Requires D in {64, 128}, Hq % Hkv == 0, 1 <= kv_len <= C, Sq >= 1,
 * causal in {0, 1}, causal ==> Sq <= kv_len.
 */
qkv_status qkv_prefill(const uint16_t* q,
                       const uint8_t* k_codes, const uint16_t* k_scales,
                       const uint8_t* v_codes, const uint16_t* v_scales,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t kv_len,
                       int64_t C, int64_t D, float softmax_scale, int causal,
                       float* out, float* lse, void* stream);

/* qkv_prefill over b-bit rows (the 2/3-bit layout of qkv_decode_bits; bits =
 * 4 is qkv_prefill).  Codes are converted exactly once per key tile and
 * workgroup, as for int4.  Requires bits in {2, 3, 4} (QKV_ERR_UNSUPPORTED
 * otherwise) and the qkv_prefill requirements. */
qkv_status qkv_prefill_bits(const uint16_t* q,
                            const uint8_t* k_codes, const uint16_t* k_scales,
                            const uint8_t* v_codes, const uint16_t* v_scales,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t kv_len,
                            int64_t C, int64_t D, int bits, float softmax_scale, int causal,
                            float* out, float* lse, void* stream);

/* qkv_prefill for the query heads of the listed KV heads (the per-head widths
 * of qkv_decode_heads: a cache of Hkv_sub heads at `bits` bits, cache head i
 * being KV head kv_heads[i] of a layer of Hkv KV heads; ids outside [0, Hkv)
 * are clamped).  q, out, lse are the layer's [B, Hq, Sq, D] / [B, Hq, Sq];
 * only the rows of the listed heads' query heads are written, so one call
 * per width covers the layer.  Requires bits in {2, 3, 4}
 * (QKV_ERR_UNSUPPORTED otherwise), 1 <= Hkv_sub <= Hkv, kv_heads non-null and
 * 4-byte aligned (QKV_ERR_INVALID_ARG), and the qkv_prefill requirements. */
qkv_status qkv_prefill_heads(const uint16_t* q,
                             const uint8_t* k_codes, const uint16_t* k_scales,
                             const uint8_t* v_codes, const uint16_t* v_scales,
                             const int32_t* kv_heads, int64_t Hkv_sub,
                             int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t kv_len,
                             int64_t C, int64_t D, int bits, float softmax_scale, int causal,
                             float* out, float* lse, void* stream);

/* qkv_prefill over asymmetric group-wise 4-bit rows (the layout and parameter
 * words of qkv_decode_asym; TurboAttention §2.3 and §3.1).  Codes enter LDS
 * as exact fp16 code - z; with one group per row the K scale multiplies
 * score columns and the V scale is folded into P as for int4 rows; with
 * several, each group's QK products are accumulated apart and scaled by the
 * group's K scale in fp32, and each 32-head-dim output block takes its
 * group's P~ = fp16(p s_V).  Requires group in {32, 64, 128}, group <= D
 * (QKV_ERR_UNSUPPORTED otherwise), k_params / v_params aligned to
 * 4 * (D / group) bytes, kv_len * (D / group) * 4 < 2^31, and the
 * qkv_prefill requirements. */
qkv_status qkv_prefill_asym(const uint16_t* q,
                            const uint8_t* k_codes, const uint32_t* k_params,
                            const uint8_t* v_codes, const uint32_t* v_params,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t kv_len,
                            int64_t C, int64_t D, int group, float softmax_scale, int causal,
                            float* out, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QKVFA_H */
