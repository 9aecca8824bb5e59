// C ABI of libqkvfa: argument validation, split planning and kernel launch.
// Every check happens before anything is enqueued; no exception leaves here.
#include "qkvfa.h"
#ifdef QKVFA_PHASE_TRACE
#include "qkvfa_trace.h"
#endif

#include <hip/hip_runtime.h>

#include <mutex>
#include <string>
#include <vector>

#include "qkvfa_internal.h"

namespace {

thread_local std::string g_last_error;

qkv_status fail(qkv_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Compute units of the current device, queried once per device.
int current_cus() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

qkv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return QKV_OK;
  return fail(QKV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Checks shared by decode and prefill.
qkv_status check_attention(const uint16_t* q, const uint8_t* kc, const uint16_t* ks,
                           const uint8_t* vc, const uint16_t* vs, int64_t B, int64_t Hq,
                           int64_t Hkv, int64_t Sq, int64_t kv_len, int64_t C, int64_t D,
                           const float* out, const float* lse, const char* fn) {
  const std::string f(fn);
  if (!q || !kc || !ks || !vc || !vs || !out)
    return fail(QKV_ERR_INVALID_ARG, f + ": null tensor pointer");
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1)
    return fail(QKV_ERR_INVALID_ARG, f + ": B, Hq, Hkv and Sq must be >= 1");
  if (D != 64 && D != 128) return fail(QKV_ERR_UNSUPPORTED, f + ": head dim must be 64 or 128");
  if (Hq % Hkv != 0) return fail(QKV_ERR_INVALID_ARG, f + ": Hq must be a multiple of Hkv");
  if (kv_len < 1 || kv_len > C) return fail(QKV_ERR_INVALID_ARG, f + ": need 1 <= kv_len <= C");
  if (C > 0x7FFFFFFFll || Sq > 0x7FFFFFFFll || Hq > 0xFFFF || Hkv > 0xFFFF || B > 0xFFFF)
    return fail(QKV_ERR_UNSUPPORTED, f + ": size beyond the supported range");
  if (!aligned(q, 16) || !aligned(kc, 16) || !aligned(vc, 16) || !aligned(out, 16))
    return fail(QKV_ERR_INVALID_ARG, f + ": q, codes and out must be 16-byte aligned");
  if (!aligned(ks, 2) || !aligned(vs, 2) || (lse && !aligned(lse, 4)))
    return fail(QKV_ERR_INVALID_ARG, f + ": misaligned scales or lse");
  return QKV_OK;
}

}  // namespace

extern "C" {

const char* qkv_status_string(qkv_status s) {
  switch (s) {
    case QKV_OK: return "ok";
    case QKV_ERR_INVALID_ARG: return "invalid argument";
    case QKV_ERR_UNSUPPORTED: return "unsupported";
    case QKV_ERR_WORKSPACE: return "workspace too small";
    case QKV_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* qkv_last_error(void) { return g_last_error.c_str(); }

int qkv_version(void) { return 100; }

qkv_status qkv_quantize_append(const float* src, uint8_t* codes, uint16_t* scales, int64_t B,
                               int64_t Hkv, int64_t T, int64_t D, int64_t C, int64_t pos,
                               void* stream) {
  if (B < 1 || Hkv < 1 || T < 0 || C < 1)
    return fail(QKV_ERR_INVALID_ARG, "qkv_quantize_append: need B, Hkv, C >= 1 and T >= 0");
  if (D != 64 && D != 128)
    return fail(QKV_ERR_UNSUPPORTED, "qkv_quantize_append: head dim must be 64 or 128");
  if (pos < 0 || pos + T > C)
    return fail(QKV_ERR_INVALID_ARG, "qkv_quantize_append: need 0 <= pos and pos + T <= C");
  if (T == 0) return QKV_OK;
  if (!src || !codes || !scales)
    return fail(QKV_ERR_INVALID_ARG, "qkv_quantize_append: null tensor pointer");
  if (!aligned(src, 16) || !aligned(codes, 16) || !aligned(scales, 2))
    return fail(QKV_ERR_INVALID_ARG, "qkv_quantize_append: misaligned pointer");
  if (B * Hkv > 0x7FFFFFFFll)
    return fail(QKV_ERR_UNSUPPORTED, "qkv_quantize_append: B * Hkv too large");
  return hip_status(qkvfa::launch_quantize_append(src, codes, scales, nullptr, nullptr, nullptr,
                                                  B * Hkv, T, (int)D, C, pos,
                                                  static_cast<hipStream_t>(stream)),
                    "qkv_quantize_append");
}

qkv_status qkv_quantize_append_kv(const float* k_src, const float* v_src, uint8_t* k_codes,
                                  uint16_t* k_scales, uint8_t* v_codes, uint16_t* v_scales,
                                  int64_t B, int64_t Hkv, int64_t T, int64_t D, int64_t C,
                                  int64_t pos, void* stream) {
  if (B < 1 || Hkv < 1 || T < 0 || C < 1)
    return fail(QKV_ERR_INVALID_ARG, "qkv_quantize_append_kv: need B, Hkv, C >= 1 and T >= 0");
  if (D != 64 && D != 128)
    return fail(QKV_ERR_UNSUPPORTED, "qkv_quantize_append_kv: head dim must be 64 or 128");
  if (pos < 0 || pos + T > C)
    return fail(QKV_ERR_INVALID_ARG, "qkv_quantize_append_kv: need 0 <= pos and pos + T <= C");
  if (T == 0) return QKV_OK;
  if (!k_src || !v_src || !k_codes || !k_scales || !v_codes || !v_scales)
    return fail(QKV_ERR_INVALID_ARG, "qkv_quantize_append_kv: null tensor pointer");
  if (!aligned(k_src, 16) || !aligned(v_src, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) ||
      !aligned(k_scales, 2) || !aligned(v_scales, 2))
    return fail(QKV_ERR_INVALID_ARG, "qkv_quantize_append_kv: misaligned pointer");
  if (B * Hkv > 0x3FFFFFFFll)
    return fail(QKV_ERR_UNSUPPORTED, "qkv_quantize_append_kv: B * Hkv too large");
  return hip_status(qkvfa::launch_quantize_append(k_src, k_codes, k_scales, v_src, v_codes, v_scales,
                                                  B * Hkv, T, (int)D, C, pos,
                                                  static_cast<hipStream_t>(stream)),
                    "qkv_quantize_append_kv");
}

int qkv_decode_auto_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t kv_len,
                           int64_t D) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || kv_len < 1 || (D != 64 && D != 128)) return 1;
  return qkvfa::plan_decode(B, Hkv, B * Hq * Sq, kv_len, (int)D, 0, current_cus(), false).n_split;
}

size_t qkv_decode_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t kv_len,
                                  int64_t D, int num_splits) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || kv_len < 1 || (D != 64 && D != 128)) return 0;
  // the larger of the uniform and the ragged plan: one size serves every decode entry point
  const int cus = current_cus();
  const qkvfa::DecodePlan p = qkvfa::plan_decode(B, Hkv, B * Hq * Sq, kv_len, (int)D, num_splits, cus, false);
  const qkvfa::DecodePlan pr = qkvfa::plan_decode(B, Hkv, B * Hq * Sq, kv_len, (int)D, num_splits, cus, true);
  return qkvfa::decode_workspace_bytes(B * Hq * Sq, B * Hkv, (int)D, p.n_split > pr.n_split ? p.n_split : pr.n_split);
}

}  // extern "C"

namespace {

// The decode entry points after their own argument checks.  C is the row
// capacity of one sequence (kv_len <= C); with a ragged / paged cache the
// launch's per-(batch, KV head) row stride is the page size instead.
qkv_status decode_common(const uint16_t* q, const uint8_t* k_codes, const uint16_t* k_scales,
                         const uint8_t* v_codes, const uint16_t* v_scales, int64_t B, int64_t Hq,
                         int64_t Hkv, int64_t Sq, int64_t kv_len, int64_t C, int64_t D,
                         float softmax_scale, int num_splits, float* out, float* lse,
                         void* workspace, size_t workspace_bytes,
                         const qkvfa::DecodeAppend* append, const qkvfa::DecodeVarlen* varlen,
                         void* stream, const char* fn, int bits = 4,
                         const qkvfa::DecodeAsym* asym = nullptr, const int32_t* kv_heads = nullptr,
                         int64_t Hkv_sub = 0, bool static_scratch = false) {
  const std::string f(fn);
  qkv_status st = check_attention(q, k_codes, k_scales, v_codes, v_scales, B, Hq, Hkv, Sq, kv_len,
                                  C, D, out, lse, fn);
  if (st != QKV_OK) return st;
  if ((Hq / Hkv) * Sq > 64)
    return fail(QKV_ERR_UNSUPPORTED, f + ": (Hq/Hkv) * Sq must be <= 64; use qkv_prefill");
  if (num_splits < 0 || num_splits > 1024)
    return fail(QKV_ERR_INVALID_ARG, f + ": num_splits must be in [0, 1024]");
  // the KV heads this call's cache holds (all of them without a head map)
  const int64_t Hc = kv_heads ? Hkv_sub : Hkv;
  const int64_t rows = B * Hc * (Hq / Hkv) * Sq;
  const qkvfa::DecodePlan plan = qkvfa::plan_decode(B, Hc, rows, kv_len, (int)D, num_splits, current_cus(),
                                                     varlen != nullptr && varlen->kv_lens != nullptr);
  // one-dimensional grid: (splits x B x heads) workgroups of up to 512 threads,
  // whose thread count must fit 32 bits
  if ((int64_t)plan.n_split * B * Hc > ((int64_t)1 << 32) / 512)
    return fail(QKV_ERR_UNSUPPORTED, f + ": too many workgroups (num_splits * B * Hkv)");
  int64_t ticket_slots = 0;
  if (static_scratch) {
    // the library's static scratch stands in for the workspace: a fixed
    // ticket region, then this call's partials
    if (plan.n_split > 1) {
      if (B * Hc > qkvfa::kScratchTickets)
        return fail(QKV_ERR_WORKSPACE, f + ": B * Hkv exceeds the static scratch's " +
                                           std::to_string(qkvfa::kScratchTickets) + " tickets; use qkv_decode");
      const size_t part = qkvfa::decode_workspace_bytes(rows, 1, (int)D, plan.n_split) - 256;
      if (qkvfa::kScratchTicketBytes + part > qkvfa::kScratchBytes)
        return fail(QKV_ERR_WORKSPACE, f + ": split partials need " + std::to_string(part) +
                                           " bytes, more than the static scratch holds (" +
                                           std::to_string(qkvfa::kScratchBytes - qkvfa::kScratchTicketBytes) +
                                           "); use fewer splits or qkv_decode");
      const hipError_t e = qkvfa::decode_scratch(&workspace, static_cast<hipStream_t>(stream));
      if (e != hipSuccess) return hip_status(e, fn);
      ticket_slots = qkvfa::kScratchTickets;
    }
  } else if (const size_t need = qkvfa::decode_workspace_bytes(rows, B * Hc, (int)D, plan.n_split); need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(QKV_ERR_WORKSPACE, f + ": workspace smaller than qkv_decode_workspace_bytes()");
    if (!aligned(workspace, 16))
      return fail(QKV_ERR_INVALID_ARG, f + ": workspace must be 16-byte aligned");
  }
  return hip_status(qkvfa::launch_decode(q, k_codes, k_scales, v_codes, v_scales, B, Hq, Hc, Sq,
                                         kv_len, varlen ? varlen->page_size : C, (int)D,
                                         softmax_scale, plan, out, lse, workspace, append, varlen,
                                         nullptr, bits, static_cast<hipStream_t>(stream), asym, kv_heads, Hkv,
                                         ticket_slots),
                    fn);
}

}  // namespace

extern "C" {

qkv_status qkv_decode(const uint16_t* q, const uint8_t* k_codes, const uint16_t* k_scales,
                      const uint8_t* v_codes, const uint16_t* v_scales, int64_t B, int64_t Hq,
                      int64_t Hkv, int64_t Sq, int64_t kv_len, int64_t C, int64_t D,
                      float softmax_scale, int num_splits, float* out, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(q, k_codes, k_scales, v_codes, v_scales, B, Hq, Hkv, Sq, kv_len, C, D,
                       softmax_scale, num_splits, out, lse, workspace, workspace_bytes, nullptr,
                       nullptr, stream, "qkv_decode");
}

qkv_status qkv_decode_noalloc(const uint16_t* q, const uint8_t* k_codes, const uint16_t* k_scales,
                              const uint8_t* v_codes, const uint16_t* v_scales, int64_t B, int64_t Hq,
                              int64_t Hkv, int64_t Sq, int64_t kv_len, int64_t C, int64_t D,
                              float softmax_scale, int num_splits, float* out, float* lse, void* stream) {
  return decode_common(q, k_codes, k_scales, v_codes, v_scales, B, Hq, Hkv, Sq, kv_len, C, D,
                       softmax_scale, num_splits, out, lse, nullptr, 0, nullptr, nullptr, stream,
                       "qkv_decode_noalloc", 4, nullptr, nullptr, 0, true);
}

qkv_status qkv_decode_bits(const uint16_t* q, const uint8_t* k_codes, const uint16_t* k_scales,
                           const uint8_t* v_codes, const uint16_t* v_scales, int64_t B, int64_t Hq,
                           int64_t Hkv, int64_t Sq, int64_t kv_len, int64_t C, int64_t D, int bits,
                           float softmax_scale, int num_splits, float* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (bits != 2 && bits != 3 && bits != 4)
    return fail(QKV_ERR_UNSUPPORTED, "qkv_decode_bits: bits must be 2, 3 or 4");
  return decode_common(q, k_codes, k_scales, v_codes, v_scales, B, Hq, Hkv, Sq, kv_len, C, D,
                       softmax_scale, num_splits, out, lse, workspace, workspace_bytes, nullptr,
                       nullptr, stream, "qkv_decode_bits", bits);
}

qkv_status qkv_quantize_append_kv_bits(const float* k_src, const float* v_src, uint8_t* k_codes,
                                       uint16_t* k_scales, uint8_t* v_codes, uint16_t* v_scales,
                                       int64_t B, int64_t Hkv, int64_t T, int64_t D, int64_t C,
                                       int64_t pos, int bits, void* stream) {
  if (bits != 2 && bits != 3 && bits != 4)
    return fail(QKV_ERR_UNSUPPORTED, "qkv_quantize_append_kv_bits: bits must be 2, 3 or 4");
  if (B < 1 || Hkv < 1 || T < 0 || C < 1)
    return fail(QKV_ERR_INVALID_ARG, "qkv_quantize_append_kv_bits: need B, Hkv, C >= 1 and T >= 0");
  if (D != 64 && D != 128)
    return fail(QKV_ERR_UNSUPPORTED, "qkv_quantize_append_kv_bits: head dim must be 64 or 128");
  if (pos < 0 || pos + T > C)
    return fail(QKV_ERR_INVALID_ARG, "qkv_quantize_append_kv_bits: need 0 <= pos and pos + T <= C");
  if (T == 0) return QKV_OK;
  if (!k_src || !v_src || !k_codes || !k_scales || !v_codes || !v_scales)
    return fail(QKV_ERR_INVALID_ARG, "qkv_quantize_append_kv_bits: null tensor pointer");
  if (!aligned(k_src, 16) || !aligned(v_src, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) ||
      !aligned(k_scales, 2) || !aligned(v_scales, 2))
    return fail(QKV_ERR_INVALID_ARG, "qkv_quantize_append_kv_bits: misaligned pointer");
  if (B * Hkv > 0x3FFFFFFFll)
    return fail(QKV_ERR_UNSUPPORTED, "qkv_quantize_append_kv_bits: B * Hkv too large");
  return hip_status(qkvfa::launch_quantize_append_bits(k_src, k_codes, k_scales, v_src, v_codes, v_scales,
                                                       B * Hkv, T, (int)D, C, pos, bits,
                                                       static_cast<hipStream_t>(stream)),
                    "qkv_quantize_append_kv_bits");
}

static bool valid_group(int64_t D, int group) {
  return (group == 32 || group == 64 || group == 128) && group <= D;
}

qkv_status qkv_quantize_append_kv_asym(const float* k_src, const float* v_src, uint8_t* k_codes,
                                       uint32_t* k_params, uint8_t* v_codes, uint32_t* v_params,
                                       int64_t B, int64_t Hkv, int64_t T, int64_t D, int64_t C,
                                       int64_t pos, int group, void* stream) {
  const char* fn = "qkv_quantize_append_kv_asym";
  if (B < 1 || Hkv < 1 || T < 0 || C < 1)
    return fail(QKV_ERR_INVALID_ARG, std::string(fn) + ": need B, Hkv, C >= 1 and T >= 0");
  if (D != 64 && D != 128) return fail(QKV_ERR_UNSUPPORTED, std::string(fn) + ": head dim must be 64 or 128");
  if (!valid_group(D, group))
    return fail(QKV_ERR_UNSUPPORTED, std::string(fn) + ": group must be 32, 64 or 128 and at most the head dim");
  if (pos < 0 || pos + T > C)
    return fail(QKV_ERR_INVALID_ARG, std::string(fn) + ": need 0 <= pos and pos + T <= C");
  if (T == 0) return QKV_OK;
  if (!k_src || !v_src || !k_codes || !k_params || !v_codes || !v_params)
    return fail(QKV_ERR_INVALID_ARG, std::string(fn) + ": null tensor pointer");
  if (!aligned(k_src, 16) || !aligned(v_src, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) ||
      !aligned(k_params, 4) || !aligned(v_params, 4))
    return fail(QKV_ERR_INVALID_ARG, std::string(fn) + ": misaligned pointer");
  if (B * Hkv > 0x3FFFFFFFll) return fail(QKV_ERR_UNSUPPORTED, std::string(fn) + ": B * Hkv too large");
  return hip_status(qkvfa::launch_quantize_append_asym(k_src, k_codes, k_params, v_src, v_codes, v_params,
                                                       B * Hkv, T, (int)D, C, pos, group,
                                                       static_cast<hipStream_t>(stream)),
                    fn);
}

qkv_status qkv_decode_asym(const uint16_t* q, const uint8_t* k_codes, const uint32_t* k_params,
                           const uint8_t* v_codes, const uint32_t* v_params, int64_t B, int64_t Hq,
                           int64_t Hkv, int64_t Sq, int64_t kv_len, int64_t C, int64_t D, int group,
                           float softmax_scale, int num_splits, float* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_group(D, group))
    return fail(QKV_ERR_UNSUPPORTED, "qkv_decode_asym: group must be 32, 64 or 128 and at most the head dim");
  if ((k_params && !aligned(k_params, 4)) || (v_params && !aligned(v_params, 4)))
    return fail(QKV_ERR_INVALID_ARG, "qkv_decode_asym: misaligned group parameters");
  const qkvfa::DecodeAsym asym = {k_params, v_params, group};
  return decode_common(q, k_codes, reinterpret_cast<const uint16_t*>(k_params), v_codes,
                       reinterpret_cast<const uint16_t*>(v_params), B, Hq, Hkv, Sq, kv_len, C, D,
                       softmax_scale, num_splits, out, lse, workspace, workspace_bytes, nullptr, nullptr,
                       stream, "qkv_decode_asym", 4, &asym);
}

qkv_status qkv_quantize_append_kv_heads(const float* k_src, const float* v_src, const int32_t* kv_heads,
                                        int64_t Hkv_sub, uint8_t* k_codes, uint16_t* k_scales,
                                        uint8_t* v_codes, uint16_t* v_scales, int64_t B, int64_t Hkv,
                                        int64_t T, int64_t D, int64_t C, int64_t pos, int bits, void* stream) {
  const char* fn = "qkv_quantize_append_kv_heads";
  const std::string f(fn);
  if (bits != 2 && bits != 3 && bits != 4) return fail(QKV_ERR_UNSUPPORTED, f + ": bits must be 2, 3 or 4");
  if (B < 1 || Hkv < 1 || T < 0 || C < 1)
    return fail(QKV_ERR_INVALID_ARG, f + ": need B, Hkv, C >= 1 and T >= 0");
  if (Hkv_sub < 1 || Hkv_sub > Hkv) return fail(QKV_ERR_INVALID_ARG, f + ": need 1 <= Hkv_sub <= Hkv");
  if (D != 64 && D != 128) return fail(QKV_ERR_UNSUPPORTED, f + ": head dim must be 64 or 128");
  if (pos < 0 || pos + T > C) return fail(QKV_ERR_INVALID_ARG, f + ": need 0 <= pos and pos + T <= C");
  if (T == 0) return QKV_OK;
  if (!k_src || !v_src || !kv_heads || !k_codes || !k_scales || !v_codes || !v_scales)
    return fail(QKV_ERR_INVALID_ARG, f + ": null pointer");
  if (!aligned(k_src, 16) || !aligned(v_src, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) ||
      !aligned(k_scales, 2) || !aligned(v_scales, 2) || !aligned(kv_heads, 4))
    return fail(QKV_ERR_INVALID_ARG, f + ": misaligned pointer");
  if (B * Hkv > 0x3FFFFFFFll) return fail(QKV_ERR_UNSUPPORTED, f + ": B * Hkv too large");
  return hip_status(qkvfa::launch_quantize_append_bits(k_src, k_codes, k_scales, v_src, v_codes, v_scales,
                                                       B * Hkv_sub, T, (int)D, C, pos, bits,
                                                       static_cast<hipStream_t>(stream), kv_heads, (int)Hkv_sub,
                                                       (int)Hkv),
                    fn);
}

qkv_status qkv_decode_heads(const uint16_t* q, const uint8_t* k_codes, const uint16_t* k_scales,
                            const uint8_t* v_codes, const uint16_t* v_scales, const int32_t* kv_heads,
                            int64_t Hkv_sub, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t kv_len,
                            int64_t C, int64_t D, int bits, float softmax_scale, int num_splits, float* out,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (bits != 2 && bits != 3 && bits != 4)
    return fail(QKV_ERR_UNSUPPORTED, "qkv_decode_heads: bits must be 2, 3 or 4");
  if (Hkv_sub < 1 || Hkv_sub > Hkv) return fail(QKV_ERR_INVALID_ARG, "qkv_decode_heads: need 1 <= Hkv_sub <= Hkv");
  if (!kv_heads || !aligned(kv_heads, 4))
    return fail(QKV_ERR_INVALID_ARG, "qkv_decode_heads: null or misaligned kv_heads");
  return decode_common(q, k_codes, k_scales, v_codes, v_scales, B, Hq, Hkv, Sq, kv_len, C, D, softmax_scale,
                       num_splits, out, lse, workspace, workspace_bytes, nullptr, nullptr, stream,
                       "qkv_decode_heads", bits, nullptr, kv_heads, Hkv_sub);
}

qkv_status qkv_decode_append(const uint16_t* q, const float* k_new, const float* v_new,
                             uint8_t* k_codes, uint16_t* k_scales, uint8_t* v_codes,
                             uint16_t* v_scales, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq,
                             int64_t pos, int64_t n_new, int64_t C, int64_t D,
                             float softmax_scale, int num_splits, float* out, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (!k_new || !v_new)
    return fail(QKV_ERR_INVALID_ARG, "qkv_decode_append: null new-row pointer");
  if (n_new < 1 || n_new > 64)
    return fail(QKV_ERR_UNSUPPORTED, "qkv_decode_append: n_new must be in [1, 64]");
  if (pos < 0 || pos + n_new > C)
    return fail(QKV_ERR_INVALID_ARG, "qkv_decode_append: need 0 <= pos and pos + n_new <= C");
  if (!aligned(k_new, 16) || !aligned(v_new, 16))
    return fail(QKV_ERR_INVALID_ARG, "qkv_decode_append: k_new and v_new must be 16-byte aligned");
  const qkvfa::DecodeAppend app = {k_new, v_new, n_new};
  return decode_common(q, k_codes, k_scales, v_codes, v_scales, B, Hq, Hkv, Sq, pos + n_new, C, D,
                       softmax_scale, num_splits, out, lse, workspace, workspace_bytes, &app,
                       nullptr, stream, "qkv_decode_append");
}

qkv_status qkv_decode_paged(const uint16_t* q, const float* k_new, const float* v_new,
                            uint8_t* k_codes, uint16_t* k_scales, uint8_t* v_codes,
                            uint16_t* v_scales, const int32_t* block_table, const int32_t* kv_lens,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t n_new,
                            int64_t max_kv_len, int64_t page_size, int64_t max_pages,
                            int64_t num_pages, int64_t D, float softmax_scale, int num_splits,
                            float* out, float* lse, void* workspace, size_t workspace_bytes,
                            void* stream) {
  const char* fn = "qkv_decode_paged";
  if (page_size < 1 || max_pages < 1 || num_pages < 1)
    return fail(QKV_ERR_INVALID_ARG, "qkv_decode_paged: page_size, max_pages and num_pages must be >= 1");
  if (page_size > 0x7FFFFFFFll / max_pages || num_pages > 0x7FFFFFFFll)
    return fail(QKV_ERR_UNSUPPORTED, "qkv_decode_paged: max_pages * page_size and num_pages must stay below 2^31");
  if (block_table) {
    if (page_size % 32 != 0)
      return fail(QKV_ERR_UNSUPPORTED, "qkv_decode_paged: page_size must be a multiple of 32");
    if (!aligned(block_table, 4))
      return fail(QKV_ERR_INVALID_ARG, "qkv_decode_paged: misaligned block_table");
  } else if (max_pages != 1 || num_pages < B) {
    return fail(QKV_ERR_INVALID_ARG,
                "qkv_decode_paged: without a block table sequence b owns page b: need max_pages == 1 "
                "and num_pages >= B");
  }
  if (kv_lens && !aligned(kv_lens, 4))
    return fail(QKV_ERR_INVALID_ARG, "qkv_decode_paged: misaligned kv_lens");
  if (n_new < 0 || n_new > 64)
    return fail(QKV_ERR_UNSUPPORTED, "qkv_decode_paged: n_new must be in [0, 64]");
  if (max_kv_len < n_new)
    return fail(QKV_ERR_INVALID_ARG, "qkv_decode_paged: need max_kv_len >= n_new");
  qkvfa::DecodeAppend app = {k_new, v_new, n_new};
  if (n_new > 0) {
    if (!k_new || !v_new)
      return fail(QKV_ERR_INVALID_ARG, "qkv_decode_paged: null new-row pointer");
    if (!aligned(k_new, 16) || !aligned(v_new, 16))
      return fail(QKV_ERR_INVALID_ARG, "qkv_decode_paged: k_new and v_new must be 16-byte aligned");
  }
  const qkvfa::DecodeVarlen vl = {kv_lens, block_table, page_size, max_pages, num_pages};
  return decode_common(q, k_codes, k_scales, v_codes, v_scales, B, Hq, Hkv, Sq, max_kv_len,
                       max_pages * page_size, D, softmax_scale, num_splits, out, lse, workspace,
                       workspace_bytes, n_new > 0 ? &app : nullptr, &vl, stream, fn);
}

qkv_status qkv_buffer_scale(const uint16_t* k_scales, const uint16_t* v_scales, int64_t B, int64_t Hkv,
                            int64_t L, int64_t C, float* k_s8, float* v_s8, void* stream) {
  if (!k_scales || !v_scales || !k_s8 || !v_s8)
    return fail(QKV_ERR_INVALID_ARG, "qkv_buffer_scale: null pointer");
  if (B < 1 || Hkv < 1 || C < 1 || L < 0 || L > C)
    return fail(QKV_ERR_INVALID_ARG, "qkv_buffer_scale: need B, Hkv, C >= 1 and 0 <= L <= C");
  if (!aligned(k_scales, 2) || !aligned(v_scales, 2) || !aligned(k_s8, 4) || !aligned(v_s8, 4))
    return fail(QKV_ERR_INVALID_ARG, "qkv_buffer_scale: misaligned pointer");
  if (B * Hkv > 0x3FFFFFFFll)
    return fail(QKV_ERR_UNSUPPORTED, "qkv_buffer_scale: B * Hkv too large");
  return hip_status(qkvfa::launch_buffer_scale(k_scales, v_scales, k_s8, v_s8, B * Hkv, L, C,
                                               static_cast<hipStream_t>(stream)),
                    "qkv_buffer_scale");
}

qkv_status qkv_buffer_flush(const int8_t* k_buf, const int8_t* v_buf, const float* k_s8, const float* v_s8,
                            int64_t buf_rows, int64_t T, uint8_t* k_codes, uint16_t* k_scales,
                            uint8_t* v_codes, uint16_t* v_scales, int64_t B, int64_t Hkv, int64_t D, int64_t C,
                            int64_t pos, void* stream) {
  if (B < 1 || Hkv < 1 || C < 1 || T < 0 || buf_rows < 1 || buf_rows > 64 || T > buf_rows)
    return fail(QKV_ERR_INVALID_ARG, "qkv_buffer_flush: need B, Hkv, C >= 1, 1 <= buf_rows <= 64, 0 <= T <= buf_rows");
  if (D != 64 && D != 128) return fail(QKV_ERR_UNSUPPORTED, "qkv_buffer_flush: head dim must be 64 or 128");
  if (pos < 0 || pos + T > C)
    return fail(QKV_ERR_INVALID_ARG, "qkv_buffer_flush: need 0 <= pos and pos + T <= C");
  if (T == 0) return QKV_OK;
  if (!k_buf || !v_buf || !k_s8 || !v_s8 || !k_codes || !k_scales || !v_codes || !v_scales)
    return fail(QKV_ERR_INVALID_ARG, "qkv_buffer_flush: null pointer");
  if (!aligned(k_buf, 16) || !aligned(v_buf, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) ||
      !aligned(k_scales, 2) || !aligned(v_scales, 2) || !aligned(k_s8, 4) || !aligned(v_s8, 4))
    return fail(QKV_ERR_INVALID_ARG, "qkv_buffer_flush: misaligned pointer");
  if (B * Hkv > 0x3FFFFFFFll)
    return fail(QKV_ERR_UNSUPPORTED, "qkv_buffer_flush: B * Hkv too large");
  return hip_status(qkvfa::launch_buffer_flush(k_buf, v_buf, k_s8, v_s8, k_codes, k_scales, v_codes, v_scales,
                                               B * Hkv, T, buf_rows, (int)D, C, pos,
                                               static_cast<hipStream_t>(stream)),
                    "qkv_buffer_flush");
}

}  // extern "C"

namespace {

// Split plan of a buffered decode: the int4 rows' plan (none when kv_len = 0)
// plus one split for the buffered rows when there are any.
qkvfa::DecodePlan buffered_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t kv_len, int64_t D,
                                int num_splits, int64_t tail_rows) {
  qkvfa::DecodePlan p;
  if (kv_len >= 1) {
    p = qkvfa::plan_decode(B, Hkv, B * Hq * Sq, kv_len, (int)D, num_splits, current_cus(), false);
  } else {
    p.n_split = 0;
  }
  if (tail_rows > 0) p.n_split += 1;
  return p;
}

}  // namespace

extern "C" {

size_t qkv_decode_buffered_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t kv_len,
                                           int64_t D, int num_splits) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || kv_len < 0 || (D != 64 && D != 128)) return 0;
  const qkvfa::DecodePlan p = buffered_plan(B, Hq, Hkv, Sq, kv_len, D, num_splits, 1);
  return qkvfa::decode_workspace_bytes(B * Hq * Sq, B * Hkv, (int)D, p.n_split);
}

qkv_status qkv_decode_buffered(const uint16_t* q, const float* k_new, const float* v_new,
                               const uint8_t* k_codes, const uint16_t* k_scales, const uint8_t* v_codes,
                               const uint16_t* v_scales, int8_t* k_buf, int8_t* v_buf, const float* k_s8,
                               const float* v_s8, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq,
                               int64_t kv_len, int64_t C, int64_t buf_rows, int64_t buf_len, int64_t n_new,
                               int64_t D, float softmax_scale, int num_splits, float* out, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream) {
  const std::string f("qkv_decode_buffered");
  if (buf_rows < 1 || buf_rows > 64)
    return fail(QKV_ERR_UNSUPPORTED, f + ": buf_rows must be in [1, 64]");
  if (buf_len < 0 || n_new < 0 || buf_len + n_new > buf_rows)
    return fail(QKV_ERR_INVALID_ARG, f + ": need 0 <= buf_len, 0 <= n_new, buf_len + n_new <= buf_rows");
  if (kv_len < 0 || kv_len > C || kv_len + buf_len + n_new < 1)
    return fail(QKV_ERR_INVALID_ARG, f + ": need 0 <= kv_len <= C and at least one row to attend");
  qkv_status st = check_attention(q, k_codes, k_scales, v_codes, v_scales, B, Hq, Hkv, Sq,
                                  kv_len > 0 ? kv_len : 1, C, D, out, lse, "qkv_decode_buffered");
  if (st != QKV_OK) return st;
  if ((Hq / Hkv) * Sq > 64)
    return fail(QKV_ERR_UNSUPPORTED, f + ": (Hq/Hkv) * Sq must be <= 64");
  if (num_splits < 0 || num_splits > 1024)
    return fail(QKV_ERR_INVALID_ARG, f + ": num_splits must be in [0, 1024]");
  const int64_t tail_rows = buf_len + n_new;
  if (tail_rows > 0) {
    if (!k_buf || !v_buf || !k_s8 || !v_s8)
      return fail(QKV_ERR_INVALID_ARG, f + ": null buffer pointer");
    if (!aligned(k_buf, 16) || !aligned(v_buf, 16) || !aligned(k_s8, 4) || !aligned(v_s8, 4))
      return fail(QKV_ERR_INVALID_ARG, f + ": misaligned buffer pointer");
  }
  if (n_new > 0) {
    if (!k_new || !v_new) return fail(QKV_ERR_INVALID_ARG, f + ": null new-row pointer");
    if (!aligned(k_new, 16) || !aligned(v_new, 16))
      return fail(QKV_ERR_INVALID_ARG, f + ": k_new and v_new must be 16-byte aligned");
  }
  const qkvfa::DecodePlan plan = buffered_plan(B, Hq, Hkv, Sq, kv_len, D, num_splits, tail_rows);
  if ((int64_t)plan.n_split * B * Hkv > ((int64_t)1 << 32) / 512)
    return fail(QKV_ERR_UNSUPPORTED, f + ": too many workgroups (num_splits * B * Hkv)");
  const size_t need = qkvfa::decode_workspace_bytes(B * Hq * Sq, B * Hkv, (int)D, plan.n_split);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(QKV_ERR_WORKSPACE, f + ": workspace smaller than qkv_decode_buffered_workspace_bytes()");
    if (!aligned(workspace, 16))
      return fail(QKV_ERR_INVALID_ARG, f + ": workspace must be 16-byte aligned");
  }
  const qkvfa::DecodeTail tail = {k_buf, v_buf, k_s8, v_s8, k_new, v_new, buf_rows, buf_len, n_new};
  return hip_status(qkvfa::launch_decode(q, k_codes, k_scales, v_codes, v_scales, B, Hq, Hkv, Sq, kv_len, C,
                                         (int)D, softmax_scale, plan, out, lse, workspace, nullptr, nullptr,
                                         &tail, 4, static_cast<hipStream_t>(stream)),
                    "qkv_decode_buffered");
}

// group > 0: asymmetric rows, k_scales / v_scales are their parameter words
static qkv_status prefill_common(const uint16_t* q, const uint8_t* k_codes, const uint16_t* k_scales,
                                 const uint8_t* v_codes, const uint16_t* v_scales, int64_t B, int64_t Hq,
                                 int64_t Hkv, int64_t Sq, int64_t kv_len, int64_t C, int64_t D,
                                 float softmax_scale, int causal, float* out, float* lse, void* stream, int bits,
                                 const char* fn, int group = 0, const int32_t* kv_heads = nullptr,
                                 int64_t Hkv_sub = 0) {
  const std::string f(fn);
  qkv_status st = check_attention(q, k_codes, k_scales, v_codes, v_scales, B, Hq, Hkv, Sq, kv_len,
                                  C, D, out, lse, fn);
  if (st != QKV_OK) return st;
  if (causal != 0 && causal != 1) return fail(QKV_ERR_INVALID_ARG, f + ": causal must be 0 or 1");
  if (causal && Sq > kv_len)
    return fail(QKV_ERR_INVALID_ARG, f + ": causal attention needs Sq <= kv_len");
  if ((Sq + 127) / 128 > 0xFFFF)
    return fail(QKV_ERR_UNSUPPORTED, f + ": too many query blocks");
  if (kv_len * (D * bits / 8) > 0x7FFFFFFFll)
    return fail(QKV_ERR_UNSUPPORTED, f + ": kv_len * D * bits / 8 must stay below 2^31 bytes");
  if (group > 0) {
    if (kv_len * (D / group) * 4 > 0x7FFFFFFFll)
      return fail(QKV_ERR_UNSUPPORTED, f + ": kv_len * (D / group) * 4 must stay below 2^31 bytes");
    return hip_status(qkvfa::launch_prefill_asym(q, k_codes, reinterpret_cast<const uint32_t*>(k_scales), v_codes,
                                                 reinterpret_cast<const uint32_t*>(v_scales), B, Hq, Hkv, Sq,
                                                 kv_len, C, (int)D, group, softmax_scale, causal, out, lse,
                                                 static_cast<hipStream_t>(stream)),
                      fn);
  }
  return hip_status(qkvfa::launch_prefill(q, k_codes, k_scales, v_codes, v_scales, B, Hq,
                                          kv_heads ? Hkv_sub : Hkv, Sq, kv_len, C, (int)D, softmax_scale, causal,
                                          out, lse, static_cast<hipStream_t>(stream), bits, kv_heads, Hkv),
                    fn);
}

qkv_status qkv_prefill(const uint16_t* q, const uint8_t* k_codes, const uint16_t* k_scales,
                       const uint8_t* v_codes, const uint16_t* v_scales, int64_t B, int64_t Hq,
                       int64_t Hkv, int64_t Sq, int64_t kv_len, int64_t C, int64_t D,
                       float softmax_scale, int causal, float* out, float* lse, void* stream) {
  return prefill_common(q, k_codes, k_scales, v_codes, v_scales, B, Hq, Hkv, Sq, kv_len, C, D, softmax_scale,
                        causal, out, lse, stream, 4, "qkv_prefill");
}

qkv_status qkv_prefill_bits(const uint16_t* q, const uint8_t* k_codes, const uint16_t* k_scales,
                            const uint8_t* v_codes, const uint16_t* v_scales, int64_t B, int64_t Hq,
                            int64_t Hkv, int64_t Sq, int64_t kv_len, int64_t C, int64_t D, int bits,
                            float softmax_scale, int causal, float* out, float* lse, void* stream) {
  if (bits != 2 && bits != 3 && bits != 4)
    return fail(QKV_ERR_UNSUPPORTED, "qkv_prefill_bits: bits must be 2, 3 or 4");
  return prefill_common(q, k_codes, k_scales, v_codes, v_scales, B, Hq, Hkv, Sq, kv_len, C, D, softmax_scale,
                        causal, out, lse, stream, bits, "qkv_prefill_bits");
}

qkv_status qkv_prefill_heads(const uint16_t* q, const uint8_t* k_codes, const uint16_t* k_scales,
                             const uint8_t* v_codes, const uint16_t* v_scales, const int32_t* kv_heads,
                             int64_t Hkv_sub, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t kv_len,
                             int64_t C, int64_t D, int bits, float softmax_scale, int causal, float* out,
                             float* lse, void* stream) {
  if (bits != 2 && bits != 3 && bits != 4)
    return fail(QKV_ERR_UNSUPPORTED, "qkv_prefill_heads: bits must be 2, 3 or 4");
  if (Hkv_sub < 1 || Hkv_sub > Hkv) return fail(QKV_ERR_INVALID_ARG, "qkv_prefill_heads: need 1 <= Hkv_sub <= Hkv");
  if (!kv_heads || !aligned(kv_heads, 4))
    return fail(QKV_ERR_INVALID_ARG, "qkv_prefill_heads: null or misaligned kv_heads");
  return prefill_common(q, k_codes, k_scales, v_codes, v_scales, B, Hq, Hkv, Sq, kv_len, C, D, softmax_scale,
                        causal, out, lse, stream, bits, "qkv_prefill_heads", 0, kv_heads, Hkv_sub);
}

qkv_status qkv_prefill_asym(const uint16_t* q, const uint8_t* k_codes, const uint32_t* k_params,
                            const uint8_t* v_codes, const uint32_t* v_params, int64_t B, int64_t Hq,
                            int64_t Hkv, int64_t Sq, int64_t kv_len, int64_t C, int64_t D, int group,
                            float softmax_scale, int causal, float* out, float* lse, void* stream) {
  if (D != 64 && D != 128) return fail(QKV_ERR_UNSUPPORTED, "qkv_prefill_asym: head dim must be 64 or 128");
  if (!valid_group(D, group))
    return fail(QKV_ERR_UNSUPPORTED, "qkv_prefill_asym: group must be 32, 64 or 128 and at most the head dim");
  const int64_t wbytes = 4 * (D / group);   // parameter words of one row
  if ((k_params && !aligned(k_params, wbytes)) || (v_params && !aligned(v_params, wbytes)))
    return fail(QKV_ERR_INVALID_ARG, "qkv_prefill_asym: parameter words must be 4 * (D / group)-byte aligned");
  return prefill_common(q, k_codes, reinterpret_cast<const uint16_t*>(k_params), v_codes,
                        reinterpret_cast<const uint16_t*>(v_params), B, Hq, Hkv, Sq, kv_len, C, D, softmax_scale,
                        causal, out, lse, stream, 4, "qkv_prefill_asym", group);
}

#ifdef QKVFA_PHASE_TRACE
qkv_status qkv_trace_read(uint64_t* dst, int64_t n_wgs) {
  if (!dst || n_wgs < 0) return fail(QKV_ERR_INVALID_ARG, "qkv_trace_read: null destination or negative count");
  const hipError_t e = qkvfa::trace_read(dst, n_wgs);
  if (e != hipSuccess) return fail(QKV_ERR_HIP, std::string("qkv_trace_read: ") + hipGetErrorString(e));
  return QKV_OK;
}
#endif

}  // extern "C"
