// Host-side launchers of the HIP kernels (internal to libqkvfa).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qkvfa {

// Quantize one tensor (src2 == nullptr) or two tensors of the same shape in one launch.
// Head map (heads != nullptr): the cache holds h_cache heads per batch entry,
// and cache head h takes the source rows of head heads[h] of the h_src heads
// per batch entry of src (BH = B * h_cache).
hipError_t launch_quantize_append(const float* src, uint8_t* codes, uint16_t* scales,
                                  const float* src2, uint8_t* codes2, uint16_t* scales2,
                                  int64_t BH, int64_t T, int D, int64_t C, int64_t pos,
                                  hipStream_t stream, const int32_t* heads = nullptr, int h_cache = 0,
                                  int h_src = 0);

struct DecodePlan {
  int n_split;     // number of splits; split s takes 32-token chunks s, s + n_split, ...
};

// Split plan for rows = B*Hq*Sq query rows; num_splits = 0 picks the count.
// ragged: per-sequence lengths up to kv_len (the count then also bounds the
// chunks per split).
DecodePlan plan_decode(int64_t B, int64_t Hkv, int64_t rows, int64_t kv_len, int D, int num_splits,
                       int num_cus, bool ragged);

// Bytes of decode workspace: split partials plus one ticket per (batch, KV head).
size_t decode_workspace_bytes(int64_t rows, int64_t units, int D, int n_split);

// Ragged / paged cache (decode): per-sequence lengths and an optional page
// table; see the kernel's argument block for the meaning.  kv_len is then the
// upper bound of every sequence's attended length (cached + new rows).
struct DecodeVarlen {
  const int32_t* kv_lens;       // [B] rows cached per sequence, or null (all kv_len - n_new)
  const int32_t* block_table;   // [B, max_pages] page ids, or null (contiguous cache)
  int64_t page_size, max_pages, num_pages;
};

// Append mode of a decode launch: n_new fp32 rows [B, Hkv, n_new, D] of K and
// V are quantized into cache rows [kv_len - n_new, kv_len) first (per
// sequence: from its own length on); the cache pointers passed to
// launch_decode must then be writable.
// INT8 decode buffer of a decode launch: one more split attends buffered rows
// [0, buf_len + n_new) of k_buf/v_buf [B, Hkv, buf_rows, D] after the cache
// rows, first quantizing the n_new fp32 rows k_new/v_new [B, Hkv, n_new, D]
// into buffer rows [buf_len, buf_len + n_new) under the universal scales
// k_s8/v_s8 [B, Hkv].  The plan passed to launch_decode counts that split.
struct DecodeTail {
  int8_t* k_buf;
  int8_t* v_buf;
  const float* k_s8;
  const float* v_s8;
  const float* k_new;
  const float* v_new;
  int64_t buf_rows, buf_len, n_new;
};

struct DecodeAppend {
  const float* k_new;
  const float* v_new;
  int64_t n_new;
};

// Asymmetric group-wise 4-bit rows: unsigned nibble codes in kc/vc (in the
// cache's K and V row orders) and one parameter word per group of `group`
// consecutive elements, k_params/v_params [B, Hkv, C, D/group] (fp16 scale in
// bits 0-15, zero point in bits 16-19); value = scale * (code - zero).  ks/vs
// are unused.
struct DecodeAsym {
  const uint32_t* k_params;
  const uint32_t* v_params;
  int group;   // 32, 64 or 128, dividing D
};

hipError_t launch_decode(const uint16_t* q, const uint8_t* kc, const uint16_t* ks,
                         const uint8_t* vc, const uint16_t* vs, int64_t B, int64_t Hq,
                         int64_t Hkv, int64_t Sq, int64_t kv_len, int64_t C, int D,
                         float softmax_scale, const DecodePlan& plan, float* out, float* lse,
                         void* workspace, const DecodeAppend* append, const DecodeVarlen* varlen,
                         const DecodeTail* tail, int bits, hipStream_t stream,
                         const DecodeAsym* asym = nullptr, const int32_t* kv_heads = nullptr,
                         int64_t Hkv_all = 0, int64_t ticket_slots = 0);

// Short-sequence prefill (kv_len <= 256, D = 64, int4 rows, Sq <= 256): one
// workgroup per query head holds the head's whole converted key range in LDS.
bool prefill_short_fits(int64_t D, int64_t Sq, int64_t kv_len, int bits);
hipError_t launch_prefill_short(const uint16_t* q, const uint8_t* kc, const uint16_t* ks, const uint8_t* vc,
                                const uint16_t* vs, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq,
                                int64_t kv_len, int64_t C, float softmax_scale, int causal, float* out,
                                float* lse, hipStream_t stream, const int32_t* kv_heads, int64_t Hkv_all);

// Static scratch of the allocation-free decode: kScratchTickets ticket
// counters at offset 0 (zero between calls), split partials from
// kScratchTicketBytes on; kScratchBytes in all.  decode_scratch returns the
// current device's copy, resolving its address (and zeroing its tickets with
// a fill kernel on `stream`) on the first call on that device.
constexpr int64_t kScratchTickets = 4096;
constexpr size_t kScratchTicketBytes = (size_t)kScratchTickets * 4;
constexpr size_t kScratchBytes = (size_t)16 << 20;
hipError_t decode_scratch(void** ptr, hipStream_t stream);

#ifdef QKVFA_PHASE_TRACE
// Measurement build: copy the decode phase timestamps of workgroups
// [0, n_wgs) of the last launch (16 uint64 each) to host memory.
hipError_t trace_read(uint64_t* dst, int64_t n_wgs);
#endif

// Quantize-append of asymmetric group-wise 4-bit K and V rows (codes and
// parameter words as in DecodeAsym) into cache rows [pos, pos + T).
hipError_t launch_quantize_append_asym(const float* src, uint8_t* codes, uint32_t* params,
                                       const float* src2, uint8_t* codes2, uint32_t* params2,
                                       int64_t BH, int64_t T, int D, int64_t C, int64_t pos, int group,
                                       hipStream_t stream);

// Quantize-append of K and V rows at 2, 3 or 4 bits (4: launch_quantize_append's
// arithmetic and layout).
hipError_t launch_quantize_append_bits(const float* src, uint8_t* codes, uint16_t* scales,
                                       const float* src2, uint8_t* codes2, uint16_t* scales2,
                                       int64_t BH, int64_t T, int D, int64_t C, int64_t pos, int bits,
                                       hipStream_t stream, const int32_t* heads = nullptr, int h_cache = 0,
                                       int h_src = 0);

hipError_t launch_buffer_scale(const uint16_t* k_scales, const uint16_t* v_scales, float* k_s8, float* v_s8,
                               int64_t BH, int64_t L, int64_t C, hipStream_t stream);

hipError_t launch_buffer_flush(const int8_t* k_buf, const int8_t* v_buf, const float* k_s8, const float* v_s8,
                               uint8_t* k_codes, uint16_t* k_scales, uint8_t* v_codes, uint16_t* v_scales,
                               int64_t BH, int64_t T, int64_t buf_rows, int D, int64_t C, int64_t pos,
                               hipStream_t stream);

hipError_t launch_prefill(const uint16_t* q, const uint8_t* kc, const uint16_t* ks,
                          const uint8_t* vc, const uint16_t* vs, int64_t B, int64_t Hq,
                          int64_t Hkv, int64_t Sq, int64_t kv_len, int64_t C, int D,
                          float softmax_scale, int causal, float* out, float* lse,
                          hipStream_t stream, int bits = 4, const int32_t* kv_heads = nullptr,
                          int64_t Hkv_all = 0);

// Prefill over asymmetric group-wise 4-bit rows (codes and parameter words as
// in DecodeAsym, groups of 32, 64 or 128 elements dividing D).
hipError_t launch_prefill_asym(const uint16_t* q, const uint8_t* kc, const uint32_t* kp,
                               const uint8_t* vc, const uint32_t* vp, int64_t B, int64_t Hq,
                               int64_t Hkv, int64_t Sq, int64_t kv_len, int64_t C, int D, int group,
                               float softmax_scale, int causal, float* out, float* lse,
                               hipStream_t stream);

}  // namespace qkvfa
