// Host-side launchers of the SharQ kernels (internal to libsharq).  Each
// launcher enqueues its kernels on `s` and returns the launch status; argument
// validation happens before, in api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sharq {

// Row gathers read row_index[r] from device memory; kernels clamp each index
// into [0, act_rows) and grouped kernels clamp group offsets into [0, rows],
// so malformed device tables cannot make a kernel access memory out of bounds.

// largest K the register-resident prepare kernels handle
int prepare_max_k();
size_t prepare_nv_workspace(int T, int K);
// the file-scope scratch of the allocation-free prepare: its size, and the
// current device's address of it (looked up once per device)
size_t scratch_max_bytes();
hipError_t scratch_device_ptr(void** out);
size_t pack_nv_workspace(int K, int D, int n_groups);
// tile timeline of the tracing build (SHARQ_TIMELINE): whether this build
// records it, its record count (8 words each), and synchronous clear / read
bool timeline_built();
size_t timeline_records();
hipError_t timeline_clear();
hipError_t timeline_read(uint64_t* host, size_t words);

// m24: the 2:4 element-wise backbone (metadata K/8 bytes per row) instead of 4:8 in pairs
hipError_t launch_prepare_mx(const void* X, bool bf16, int T, int K, int64_t ldx, const float* gamma, float eps,
                             uint8_t* bb_codes, uint8_t* bb_meta, uint8_t* bb_scale, uint8_t* res_codes,
                             uint8_t* res_scale, hipStream_t s, bool m24 = false);

hipError_t launch_prepare_nv(const void* X, bool bf16, int T, int K, int64_t ldx, const float* gamma, float eps,
                             uint8_t* bb_codes, uint8_t* bb_meta, uint8_t* bb_scale, uint8_t* res_codes,
                             uint8_t* res_scale, float* tensor_scales, void* workspace, hipStream_t s);

// plain baseline: RMSNorm to fp32 rows (the fused preparation's pinned
// order), MXFP4 quantization of fp32 rows, dense MXFP4 GEMM (K % 512 == 0)
hipError_t launch_rmsnorm(const void* X, bool bf16, int T, int K, int64_t ldx, const float* gamma, float eps, float* Y,
                          int64_t ldy, hipStream_t s);
hipError_t launch_quantize_mx(const float* Y, int T, int K, int64_t ldy, uint8_t* codes, uint8_t* scales,
                              hipStream_t s);
hipError_t launch_linear_dense_mx(const uint8_t* codes, const uint8_t* scales, int rows, int K, const uint8_t* payload,
                                  const uint8_t* wscale, int D, float* Y, int64_t ldy, hipStream_t s);

hipError_t launch_pack(const void* W, bool bf16, bool nv, int K, int D, int n_groups, int64_t ldw, int64_t gstride,
                       uint8_t* payload, uint8_t* scale_sp, uint8_t* scale_dn, float* tscale, void* workspace,
                       hipStream_t s);

// m24: activations with the 2:4 element-wise backbone (metadata K/8 bytes per row)
hipError_t launch_linear_mx(const uint8_t* bb_codes, const uint8_t* bb_meta, const uint8_t* bb_scale,
                            const uint8_t* res_codes, const uint8_t* res_scale, const int32_t* row_index, int rows,
                            int act_rows, int K, const uint8_t* payload, const uint8_t* wscale, int D, int n_groups,
                            const int32_t* group_offsets, float* Y, int64_t ldy, hipStream_t s, bool m24 = false);

// single-launch decode (T <= 16, K <= decode_max_k(T)): MXFP4 prepare of the
// T rows and the plain dual-path linear on them in one kernel; sync: the
// four workspace words of the counter protocol (zero before first use)
int decode_max_k(int rows);
hipError_t launch_prepare_linear_mx(const void* X, bool bf16, int T, int K, int64_t ldx, const float* gamma, float eps,
                                    uint8_t* bb_codes, uint8_t* bb_meta, uint8_t* bb_scale, uint8_t* res_codes,
                                    uint8_t* res_scale, const uint8_t* payload, const uint8_t* wscale, int D, float* Y,
                                    int64_t ldy, uint32_t* sync, hipStream_t s);

hipError_t launch_linear_nv(const uint8_t* bb_codes, const uint8_t* bb_meta, const uint8_t* bb_scale,
                            const uint8_t* res_codes, const uint8_t* res_scale, const float* a_ts,
                            const int32_t* row_index, int rows, int act_rows, int K, const uint8_t* payload,
                            const uint8_t* wscale, const float* w_ts, int D, float* Y, int64_t ldy, hipStream_t s);

}  // namespace sharq
