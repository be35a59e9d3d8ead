// C ABI of libsharq (declared in include/sharq.h): host-side argument
// validation, buffer-size queries and kernel dispatch.  Every check runs
// before anything is enqueued, so a call that returns an error leaves the
// stream untouched.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/sharq.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

sharq_status fail(sharq_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
sharq_status fail(sharq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

sharq_status ok() {
  g_last_error.clear();
  return SHARQ_OK;
}

sharq_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SHARQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_fmt(int32_t f) { return f == SHARQ_MXFP4 || f == SHARQ_NVFP4_EMU; }   // weights
bool valid_act_fmt(int32_t f) { return valid_fmt(f) || f == SHARQ_MXFP4_24; }
// the weight format an activation format multiplies with (2:4 backbones use MXFP4 weights)
int32_t weight_fmt_of(int32_t act_fmt) { return act_fmt == SHARQ_MXFP4_24 ? SHARQ_MXFP4 : act_fmt; }
bool valid_dtype(int32_t d) { return d == SHARQ_F32 || d == SHARQ_BF16; }
size_t dtype_size(int32_t d) { return d == SHARQ_F32 ? 4 : 2; }

constexpr int64_t kMaxElems = (int64_t)1 << 40;
// buffers the GEMM kernels address through buffer descriptors stay below
// 2 GiB: the kernels mark absent loads with offset bit 31, which must then lie
// past every such buffer (a load past a descriptor's size returns zeros)
constexpr int64_t kMaxDescBytes = ((int64_t)1 << 31) - 256;

sharq_status check_k(int32_t K, int mult) {
  if (K <= 0 || K % mult != 0)
    return fail(SHARQ_ERR_UNSUPPORTED_SHAPE, "K = %d must be a positive multiple of %d", K, mult);
  return SHARQ_OK;
}

// argument checks shared by the entry points (nothing is enqueued)
sharq_status prepare_checks(const void* X, int32_t dtype, int32_t T, int32_t K, int64_t ldx, const float* gamma,
                            float eps, const sharq_act* out, void* workspace, size_t workspace_bytes) {
  if (!X || !out) return fail(SHARQ_ERR_INVALID_ARGUMENT, "X and out must not be NULL");
  if (!valid_dtype(dtype)) return fail(SHARQ_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  size_t sz[7];
  if (sharq_status s = sharq_act_sizes(out->fmt, T, K, sz)) return s;
  if (K > sharq::prepare_max_k())
    return fail(SHARQ_ERR_UNSUPPORTED_SHAPE, "K = %d exceeds the supported maximum %d", K, sharq::prepare_max_k());
  if (out->T != T || out->K != K)
    return fail(SHARQ_ERR_INVALID_ARGUMENT, "out describes T=%d K=%d, call has T=%d K=%d", out->T, out->K, T, K);
  if (ldx < K) return fail(SHARQ_ERR_INVALID_ARGUMENT, "ldx = %lld < K = %d", (long long)ldx, K);
  if (!aligned16(X) || ((size_t)ldx * dtype_size(dtype)) % 16 != 0)
    return fail(SHARQ_ERR_INVALID_ARGUMENT, "X rows must start 16-byte aligned");
  if (gamma && !aligned16(gamma)) return fail(SHARQ_ERR_INVALID_ARGUMENT, "gamma must be 16-byte aligned");
  if (!(eps >= 0.0f)) return fail(SHARQ_ERR_INVALID_ARGUMENT, "eps must be >= 0");
  const uint8_t* bufs[5] = {out->bb_codes, out->bb_meta, out->bb_scale, out->res_codes, out->res_scale};
  for (const uint8_t* p : bufs) {
    if (!p) return fail(SHARQ_ERR_INVALID_ARGUMENT, "output buffers must not be NULL");
    if (!aligned16(p)) return fail(SHARQ_ERR_INVALID_ARGUMENT, "output buffers must be 16-byte aligned");
  }
  if (out->fmt == SHARQ_NVFP4_EMU) {
    if (!out->tensor_scales) return fail(SHARQ_ERR_INVALID_ARGUMENT, "NVFP4 activations need tensor_scales");
    if (!workspace || workspace_bytes < sz[6])
      return fail(SHARQ_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", sz[6], workspace_bytes);
    if (!aligned16(workspace)) return fail(SHARQ_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  }
  return SHARQ_OK;
}

sharq_status linear_checks(const sharq_act* a, const sharq_weight* w, const int32_t* group_offsets,
                           const int32_t* row_index, int32_t total_rows, float* Y, int64_t ldy) {
  if (!a || !w || !Y) return fail(SHARQ_ERR_INVALID_ARGUMENT, "a, w and Y must not be NULL");
  if (!valid_act_fmt(a->fmt) || !valid_fmt(w->fmt)) return fail(SHARQ_ERR_INVALID_ARGUMENT, "unknown format");
  if (weight_fmt_of(a->fmt) != w->fmt)
    return fail(SHARQ_ERR_FORMAT_MISMATCH, "activation format %d does not multiply weight format %d", a->fmt, w->fmt);
  if (a->K != w->K) return fail(SHARQ_ERR_FORMAT_MISMATCH, "activation K = %d != weight K = %d", a->K, w->K);
  if (sharq_status s = check_k(a->K, 128)) return s;
  if (a->T < 1 || w->D < 1 || w->n_groups < 1)
    return fail(SHARQ_ERR_UNSUPPORTED_SHAPE, "T, D and n_groups must be >= 1");
  if (total_rows < 0) return fail(SHARQ_ERR_INVALID_ARGUMENT, "total_rows < 0");
  if (ldy < w->D) return fail(SHARQ_ERR_INVALID_ARGUMENT, "ldy = %lld < D = %d", (long long)ldy, w->D);
  if (!aligned16(Y)) return fail(SHARQ_ERR_INVALID_ARGUMENT, "Y must be 16-byte aligned");
  if (w->n_groups == 1) {
    if (group_offsets) return fail(SHARQ_ERR_INVALID_ARGUMENT, "group_offsets must be NULL for one group");
    if (!row_index && total_rows > a->T)
      return fail(SHARQ_ERR_INVALID_ARGUMENT, "total_rows = %d > T = %d without row_index", total_rows, a->T);
  } else {
    if (!group_offsets) return fail(SHARQ_ERR_INVALID_ARGUMENT, "grouped linear needs group_offsets");
    if (!row_index && total_rows > a->T)
      return fail(SHARQ_ERR_INVALID_ARGUMENT, "total_rows = %d > T = %d without row_index", total_rows, a->T);
    if (w->fmt != SHARQ_MXFP4) return fail(SHARQ_ERR_UNSUPPORTED_SHAPE, "grouped linear supports MXFP4 only");
  }
  const uint8_t* bufs[7] = {a->bb_codes, a->bb_meta, a->bb_scale, a->res_codes, a->res_scale, w->payload,
                            w->scale_sp};
  for (const uint8_t* p : bufs) {
    if (!p) return fail(SHARQ_ERR_INVALID_ARGUMENT, "activation / weight buffers must not be NULL");
    if (!aligned16(p)) return fail(SHARQ_ERR_INVALID_ARGUMENT, "activation / weight buffers must be 16-byte aligned");
  }
  if ((int64_t)total_rows * w->D > kMaxElems) return fail(SHARQ_ERR_UNSUPPORTED_SHAPE, "output too large");
  // the GEMM kernels address activation and weight buffers through buffer
  // descriptors with 32-bit byte offsets
  if ((int64_t)a->T * (a->K / 2) > kMaxDescBytes || (int64_t)w->D * (w->K / 2) > kMaxDescBytes)
    return fail(SHARQ_ERR_UNSUPPORTED_SHAPE, "activation residual (T*K/2) or per-group weight payload (D*K/2) over %lld bytes",
                (long long)kMaxDescBytes);
  if (a->fmt == SHARQ_NVFP4_EMU && (!a->tensor_scales || !w->tensor_scale))
    return fail(SHARQ_ERR_INVALID_ARGUMENT, "NVFP4 needs activation and weight tensor scales");
  return SHARQ_OK;
}

}  // namespace

extern "C" {

const char* sharq_status_string(sharq_status s) {
  switch (s) {
    case SHARQ_OK: return "SHARQ_OK";
    case SHARQ_ERR_INVALID_ARGUMENT: return "SHARQ_ERR_INVALID_ARGUMENT";
    case SHARQ_ERR_UNSUPPORTED_SHAPE: return "SHARQ_ERR_UNSUPPORTED_SHAPE";
    case SHARQ_ERR_FORMAT_MISMATCH: return "SHARQ_ERR_FORMAT_MISMATCH";
    case SHARQ_ERR_WORKSPACE_TOO_SMALL: return "SHARQ_ERR_WORKSPACE_TOO_SMALL";
    case SHARQ_ERR_HIP: return "SHARQ_ERR_HIP";
  }
  return "SHARQ_ERR_UNKNOWN";
}

const char* sharq_last_error(void) { return g_last_error.c_str(); }

sharq_status sharq_timeline_records(size_t* records) {
  if (!records) return fail(SHARQ_ERR_INVALID_ARGUMENT, "records is NULL");
  *records = sharq::timeline_built() ? sharq::timeline_records() : 0;
  return ok();
}

sharq_status sharq_timeline_clear(void) {
  if (!sharq::timeline_built())
    return fail(SHARQ_ERR_INVALID_ARGUMENT, "this library is not the tile-timeline build (SHARQ_TIMELINE)");
  return from_hip(sharq::timeline_clear(), "sharq_timeline_clear");
}

sharq_status sharq_timeline_read(uint64_t* host, size_t words) {
  if (!sharq::timeline_built())
    return fail(SHARQ_ERR_INVALID_ARGUMENT, "this library is not the tile-timeline build (SHARQ_TIMELINE)");
  if (!host) return fail(SHARQ_ERR_INVALID_ARGUMENT, "host is NULL");
  if (words > sharq::timeline_records() * 8)
    return fail(SHARQ_ERR_INVALID_ARGUMENT, "words = %zu exceeds the %zu recorded", words, sharq::timeline_records() * 8);
  return from_hip(sharq::timeline_read(host, words), "sharq_timeline_read");
}

sharq_status sharq_weight_sizes(int32_t fmt, int32_t K, int32_t D, int32_t n_groups, size_t bytes_out[5]) {
  if (!bytes_out) return fail(SHARQ_ERR_INVALID_ARGUMENT, "bytes_out is NULL");
  if (!valid_fmt(fmt)) return fail(SHARQ_ERR_INVALID_ARGUMENT, "unknown format %d", fmt);
  if (sharq_status s = check_k(K, 32)) return s;
  if (D < 1 || n_groups < 1) return fail(SHARQ_ERR_UNSUPPORTED_SHAPE, "D = %d, n_groups = %d must be >= 1", D, n_groups);
  const int64_t n = (int64_t)n_groups * D;
  if (n * K > kMaxElems) return fail(SHARQ_ERR_UNSUPPORTED_SHAPE, "weight too large");
  bytes_out[0] = (size_t)(n * (K / 2));
  bytes_out[1] = (size_t)(n * (K / 32));
  bytes_out[2] = (size_t)(n * (fmt == SHARQ_MXFP4 ? K / 32 : K / 16));
  bytes_out[3] = fmt == SHARQ_MXFP4 ? 0 : (size_t)n_groups * sizeof(float);
  bytes_out[4] = fmt == SHARQ_MXFP4 ? 0 : sharq::pack_nv_workspace(K, D, n_groups);
  return ok();
}

sharq_status sharq_act_sizes(int32_t fmt, int32_t T, int32_t K, size_t bytes_out[7]) {
  if (!bytes_out) return fail(SHARQ_ERR_INVALID_ARGUMENT, "bytes_out is NULL");
  if (!valid_act_fmt(fmt)) return fail(SHARQ_ERR_INVALID_ARGUMENT, "unknown format %d", fmt);
  if (sharq_status s = check_k(K, 32)) return s;
  if (T < 1) return fail(SHARQ_ERR_UNSUPPORTED_SHAPE, "T = %d must be >= 1", T);
  if ((int64_t)T * K > kMaxElems) return fail(SHARQ_ERR_UNSUPPORTED_SHAPE, "activation too large");
  const int64_t t = T;
  bytes_out[0] = (size_t)(t * (K / 4));
  const bool nv = fmt == SHARQ_NVFP4_EMU;
  bytes_out[1] = (size_t)(t * (fmt == SHARQ_MXFP4_24 ? K / 8 : K / 16));
  bytes_out[2] = (size_t)(t * (K / 32));
  bytes_out[3] = (size_t)(t * (K / 2));
  bytes_out[4] = (size_t)(t * (nv ? K / 16 : K / 32));
  bytes_out[5] = nv ? 2 * sizeof(float) : 0;
  bytes_out[6] = nv ? sharq::prepare_nv_workspace(T, K) : 0;
  return ok();
}

sharq_status sharq_pack_weight(const void* W, int32_t dtype, int32_t K, int32_t D, int32_t n_groups, int64_t ldw,
                               int64_t group_stride, const sharq_weight* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!W || !out) return fail(SHARQ_ERR_INVALID_ARGUMENT, "W and out must not be NULL");
  if (!valid_dtype(dtype)) return fail(SHARQ_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  size_t sz[5];
  if (sharq_status s = sharq_weight_sizes(out->fmt, K, D, n_groups, sz)) return s;
  if (out->K != K || out->D != D || out->n_groups != n_groups)
    return fail(SHARQ_ERR_INVALID_ARGUMENT, "out describes K=%d D=%d n_groups=%d, call has K=%d D=%d n_groups=%d",
                out->K, out->D, out->n_groups, K, D, n_groups);
  if (ldw < D) return fail(SHARQ_ERR_INVALID_ARGUMENT, "ldw = %lld < D = %d", (long long)ldw, D);
  if (n_groups > 1 && group_stride < (int64_t)K * ldw)
    return fail(SHARQ_ERR_INVALID_ARGUMENT, "group_stride = %lld < K * ldw", (long long)group_stride);
  if (!out->payload || !out->scale_sp || !out->scale_dn)
    return fail(SHARQ_ERR_INVALID_ARGUMENT, "payload / scale buffers must not be NULL");
  if (!aligned16(out->payload) || !aligned16(out->scale_sp) || !aligned16(out->scale_dn))
    return fail(SHARQ_ERR_INVALID_ARGUMENT, "payload / scale buffers must be 16-byte aligned");
  const bool nv = out->fmt == SHARQ_NVFP4_EMU;
  if (nv) {
    if (!out->tensor_scale) return fail(SHARQ_ERR_INVALID_ARGUMENT, "NVFP4 weight needs tensor_scale");
    if (workspace_bytes < sz[4] || (sz[4] && !workspace))
      return fail(SHARQ_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", sz[4], workspace_bytes);
    if (out->scale_dn == out->scale_sp)
      return fail(SHARQ_ERR_INVALID_ARGUMENT, "NVFP4 dense view must be its own buffer (K/16 per column)");
  }
  return from_hip(sharq::launch_pack(W, dtype == SHARQ_BF16, nv, K, D, n_groups, ldw, group_stride, out->payload,
                                     out->scale_sp, out->scale_dn, out->tensor_scale, workspace,
                                     static_cast<hipStream_t>(stream)),
                  "sharq_pack_weight launch");
}

sharq_status sharq_prepare(const void* X, int32_t dtype, int32_t T, int32_t K, int64_t ldx, const float* gamma,
                           float eps, const sharq_act* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (sharq_status st = prepare_checks(X, dtype, T, K, ldx, gamma, eps, out, workspace, workspace_bytes)) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (out->fmt != SHARQ_NVFP4_EMU) {
    return from_hip(sharq::launch_prepare_mx(X, dtype == SHARQ_BF16, T, K, ldx, gamma, eps, out->bb_codes,
                                             out->bb_meta, out->bb_scale, out->res_codes, out->res_scale, s,
                                             out->fmt == SHARQ_MXFP4_24),
                    "sharq_prepare launch");
  }
  return from_hip(sharq::launch_prepare_nv(X, dtype == SHARQ_BF16, T, K, ldx, gamma, eps, out->bb_codes,
                                           out->bb_meta, out->bb_scale, out->res_codes, out->res_scale,
                                           out->tensor_scales, workspace, s),
                  "sharq_prepare launch");
}

sharq_status sharq_prepare_no_alloc(const void* X, int32_t dtype, int32_t T, int32_t K, int64_t ldx,
                                    const float* gamma, float eps, const sharq_act* out, void* stream) {
  if (!out) return fail(SHARQ_ERR_INVALID_ARGUMENT, "X and out must not be NULL");
  size_t sz[7];
  if (sharq_status st = sharq_act_sizes(out->fmt, T, K, sz)) return st;
  void* scratch = nullptr;
  if (sz[6] > 0) {
    if (sz[6] > sharq::scratch_max_bytes())
      return fail(SHARQ_ERR_UNSUPPORTED_SHAPE,
                  "T = %d needs %zu bytes of scratch; the allocation-free prepare holds %zu (use sharq_prepare "
                  "with a workspace)",
                  T, sz[6], sharq::scratch_max_bytes());
    if (sharq_status st = from_hip(sharq::scratch_device_ptr(&scratch), "sharq_prepare_no_alloc scratch lookup"))
      return st;
  }
  return sharq_prepare(X, dtype, T, K, ldx, gamma, eps, out, scratch, sz[6], stream);
}

sharq_status sharq_linear(const sharq_act* a, const sharq_weight* w, const int32_t* group_offsets,
                          const int32_t* row_index, int32_t total_rows, float* Y, int64_t ldy, void* stream) {
  if (sharq_status st = linear_checks(a, w, group_offsets, row_index, total_rows, Y, ldy)) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a->fmt != SHARQ_NVFP4_EMU) {
    return from_hip(sharq::launch_linear_mx(a->bb_codes, a->bb_meta, a->bb_scale, a->res_codes, a->res_scale,
                                            row_index, total_rows, a->T, a->K, w->payload, w->scale_sp, w->D, w->n_groups,
                                            group_offsets, Y, ldy, s, a->fmt == SHARQ_MXFP4_24),
                    "sharq_linear launch");
  }
  return from_hip(sharq::launch_linear_nv(a->bb_codes, a->bb_meta, a->bb_scale, a->res_codes, a->res_scale,
                                          a->tensor_scales, row_index, total_rows, a->T, a->K, w->payload, w->scale_sp,
                                          w->tensor_scale, w->D, Y, ldy, s),
                  "sharq_linear launch");
}

sharq_status sharq_prepare_linear(const void* X, int32_t dtype, int32_t T, int32_t K, int64_t ldx, const float* gamma,
                                  float eps, const sharq_act* act, const sharq_weight* w, float* Y, int64_t ldy,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (!act || !w) return fail(SHARQ_ERR_INVALID_ARGUMENT, "act and w must not be NULL");
  if (act->fmt != SHARQ_MXFP4)
    return fail(SHARQ_ERR_INVALID_ARGUMENT, "sharq_prepare_linear supports MXFP4 only (NVFP4: sharq_prepare + sharq_linear)");
  if (w->n_groups != 1) return fail(SHARQ_ERR_INVALID_ARGUMENT, "sharq_prepare_linear is a plain linear (n_groups = 1)");
  if (sharq_status st = prepare_checks(X, dtype, T, K, ldx, gamma, eps, act, nullptr, 0)) return st;
  if (sharq_status st = linear_checks(act, w, nullptr, nullptr, T, Y, ldy)) return st;
  if (!workspace || workspace_bytes < 16)
    return fail(SHARQ_ERR_WORKSPACE_TOO_SMALL, "workspace needs 16 bytes, got %zu", workspace ? workspace_bytes : 0);
  if (!aligned16(workspace)) return fail(SHARQ_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = dtype == SHARQ_BF16;
  if (T <= 16 && K <= sharq::decode_max_k(T))
    return from_hip(sharq::launch_prepare_linear_mx(X, bf16, T, K, ldx, gamma, eps, act->bb_codes, act->bb_meta,
                                                    act->bb_scale, act->res_codes, act->res_scale, w->payload,
                                                    w->scale_sp, w->D, Y, ldy, static_cast<uint32_t*>(workspace), s),
                    "sharq_prepare_linear launch");
  if (sharq_status st = from_hip(sharq::launch_prepare_mx(X, bf16, T, K, ldx, gamma, eps, act->bb_codes, act->bb_meta,
                                                          act->bb_scale, act->res_codes, act->res_scale, s),
                                 "sharq_prepare_linear launch"))
    return st;
  return from_hip(sharq::launch_linear_mx(act->bb_codes, act->bb_meta, act->bb_scale, act->res_codes, act->res_scale,
                                          nullptr, T, T, K, w->payload, w->scale_sp, w->D, 1, nullptr, Y, ldy, s),
                  "sharq_prepare_linear launch");
}

sharq_status sharq_prepare_linear_status(const void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || workspace_bytes < 16)
    return fail(SHARQ_ERR_WORKSPACE_TOO_SMALL, "workspace needs 16 bytes, got %zu", workspace ? workspace_bytes : 0);
  if (!aligned16(workspace)) return fail(SHARQ_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  uint32_t words[4] = {0, 0, 0, 0};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (sharq_status st = from_hip(hipMemcpyAsync(words, workspace, sizeof(words), hipMemcpyDeviceToHost, s),
                                 "sharq_prepare_linear_status copy"))
    return st;
  if (sharq_status st = from_hip(hipStreamSynchronize(s), "sharq_prepare_linear_status synchronize")) return st;
  if (words[3] != 0)
    return fail(SHARQ_ERR_HIP,
                "a single-launch decode on this workspace gave up waiting for its prepared rows; its Y was "
                "written as NaN (clear the workspace to zero before reusing it)");
  return ok();
}

sharq_status sharq_rmsnorm(const void* X, int32_t dtype, int32_t T, int32_t K, int64_t ldx, const float* gamma,
                           float eps, float* Y, int64_t ldy, void* stream) {
  if (!X || !Y) return fail(SHARQ_ERR_INVALID_ARGUMENT, "X and Y must not be NULL");
  if (!valid_dtype(dtype)) return fail(SHARQ_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (sharq_status st = check_k(K, 32)) return st;
  if (T < 1) return fail(SHARQ_ERR_UNSUPPORTED_SHAPE, "T must be >= 1");
  if (K > sharq::prepare_max_k())
    return fail(SHARQ_ERR_UNSUPPORTED_SHAPE, "K = %d exceeds the supported maximum %d", K, sharq::prepare_max_k());
  if (ldx < K || ldy < K) return fail(SHARQ_ERR_INVALID_ARGUMENT, "ldx and ldy must be >= K = %d", K);
  if (!aligned16(X) || ((size_t)ldx * dtype_size(dtype)) % 16 != 0)
    return fail(SHARQ_ERR_INVALID_ARGUMENT, "X rows must start 16-byte aligned");
  if (!aligned16(Y) || ldy % 4 != 0) return fail(SHARQ_ERR_INVALID_ARGUMENT, "Y rows must start 16-byte aligned");
  if (gamma && !aligned16(gamma)) return fail(SHARQ_ERR_INVALID_ARGUMENT, "gamma must be 16-byte aligned");
  if (!(eps >= 0.0f)) return fail(SHARQ_ERR_INVALID_ARGUMENT, "eps must be >= 0");
  return from_hip(sharq::launch_rmsnorm(X, dtype == SHARQ_BF16, T, K, ldx, gamma, eps, Y, ldy,
                                        static_cast<hipStream_t>(stream)),
                  "sharq_rmsnorm launch");
}

sharq_status sharq_quantize_mx(const float* Y, int32_t T, int32_t K, int64_t ldy, uint8_t* codes, uint8_t* scales,
                               void* stream) {
  if (!Y || !codes || !scales) return fail(SHARQ_ERR_INVALID_ARGUMENT, "Y, codes and scales must not be NULL");
  if (sharq_status st = check_k(K, 32)) return st;
  if (T < 1) return fail(SHARQ_ERR_UNSUPPORTED_SHAPE, "T must be >= 1");
  if (ldy < K) return fail(SHARQ_ERR_INVALID_ARGUMENT, "ldy = %lld < K = %d", (long long)ldy, K);
  if (!aligned16(Y) || ldy % 4 != 0) return fail(SHARQ_ERR_INVALID_ARGUMENT, "Y rows must start 16-byte aligned");
  if (!aligned16(codes) || !aligned16(scales))
    return fail(SHARQ_ERR_INVALID_ARGUMENT, "codes and scales must be 16-byte aligned");
  return from_hip(sharq::launch_quantize_mx(Y, T, K, ldy, codes, scales, static_cast<hipStream_t>(stream)),
                  "sharq_quantize_mx launch");
}

sharq_status sharq_linear_dense(const uint8_t* codes, const uint8_t* scales, int32_t T, const sharq_weight* w,
                                float* Y, int64_t ldy, void* stream) {
  if (!codes || !scales || !w || !Y) return fail(SHARQ_ERR_INVALID_ARGUMENT, "codes, scales, w and Y must not be NULL");
  if (w->fmt != SHARQ_MXFP4) return fail(SHARQ_ERR_FORMAT_MISMATCH, "sharq_linear_dense takes an MXFP4 weight");
  if (w->n_groups != 1) return fail(SHARQ_ERR_INVALID_ARGUMENT, "sharq_linear_dense is a plain linear (n_groups = 1)");
  if (sharq_status st = check_k(w->K, 512)) return st;
  if (T < 1 || w->D < 1) return fail(SHARQ_ERR_UNSUPPORTED_SHAPE, "T and D must be >= 1");
  if (ldy < w->D) return fail(SHARQ_ERR_INVALID_ARGUMENT, "ldy = %lld < D = %d", (long long)ldy, w->D);
  if (!aligned16(Y)) return fail(SHARQ_ERR_INVALID_ARGUMENT, "Y must be 16-byte aligned");
  const uint8_t* bufs[4] = {codes, scales, w->payload, w->scale_dn};
  for (const uint8_t* p : bufs) {
    if (!p) return fail(SHARQ_ERR_INVALID_ARGUMENT, "activation / weight buffers must not be NULL");
    if (!aligned16(p)) return fail(SHARQ_ERR_INVALID_ARGUMENT, "activation / weight buffers must be 16-byte aligned");
  }
  if ((int64_t)T * w->D > kMaxElems) return fail(SHARQ_ERR_UNSUPPORTED_SHAPE, "output too large");
  if ((int64_t)T * (w->K / 2) > kMaxDescBytes || (int64_t)w->D * (w->K / 2) > kMaxDescBytes)
    return fail(SHARQ_ERR_UNSUPPORTED_SHAPE, "activation codes (T*K/2) or weight payload (D*K/2) over %lld bytes",
                (long long)kMaxDescBytes);
  return from_hip(sharq::launch_linear_dense_mx(codes, scales, T, w->K, w->payload, w->scale_dn, w->D, Y, ldy,
                                                static_cast<hipStream_t>(stream)),
                  "sharq_linear_dense launch");
}

}  // extern "C"
