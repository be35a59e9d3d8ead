// Offline weight packer (xllm-io paper review §3.5): one shared FP4 payload
// for both GEMM paths plus two scale views.  Weights are scaled once per 32
// K-values of a column so both paths read the same codes; the sparse view holds
// one scale per 32, the dense view one per 16 (each per-32 scale twice).
//
// Layout: row d of a group's payload holds column d of W (K contiguous, the
// even K index in the low nibble), the layout the GEMM's B operand reads.
// Thread per (column, 128 K-values): reads are coalesced along D (the input is
// K x D row-major), each thread writes 64 contiguous payload bytes.
#include "common.h"
#include "kernels.h"

namespace sharq {

namespace {

template <bool BF16>
SHARQ_DEV float load_w(const void* W, int64_t off) {
  if (BF16) return __uint_as_float((uint32_t)(static_cast<const uint16_t*>(W)[off]) << 16);
  return static_cast<const float*>(W)[off];
}

SHARQ_DEV float nv_tensor_scale_w(float amax) { return amax == 0.0f ? 1.0f : __fdiv_rn(amax, 2688.0f); }

SHARQ_DEV float nv_scaled_w(float v, float d) {
  if (!(d > 0.0f)) return v * 0.0f;
  const float t = __fdiv_rn(v, d);
  return fminf(fmaxf(t, -6.0f), 6.0f);
}

}  // namespace

// grid: (ceil(D/256), ceil(K/128), n_groups); NV: tensor_scale[g] read per group
template <bool BF16, bool NV>
__global__ __launch_bounds__(256) void pack_kernel(const void* __restrict__ W, int K, int D, int64_t ldw,
                                                   int64_t gstride, uint8_t* __restrict__ payload,
                                                   uint8_t* __restrict__ scale_sp, uint8_t* __restrict__ scale_dn,
                                                   const float* __restrict__ tscale) {
  const int d = blockIdx.x * 256 + threadIdx.x;
  if (d >= D) return;
  const int grp = blockIdx.z;
  const int kb0 = blockIdx.y * 4;                      // first 32-block
  const int nb = min(4, K / 32 - kb0);
  const int64_t wbase = grp * gstride + d;
  const int64_t prow = ((int64_t)grp * D + d);
  uint8_t* prow_ptr = payload + prow * (K / 2);
  const float s_T = NV ? tscale[grp] : 1.0f;
  uint32_t scales = 0;
  for (int b = 0; b < nb; ++b) {
    const int k0 = (kb0 + b) * 32;
    float v[32];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      v[i] = load_w<BF16>(W, wbase + (int64_t)(k0 + i) * ldw);
      amax = fmaxf(amax, fabsf(v[i]));
    }
    uint32_t words[4];
    uint32_t sc;
    if (!NV) {
      const int e = e8m0_exponent(amax);
      const float s = exp2i(e);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t x = 0;
        x = cvt_fp4x2<0>(x, v[8 * w + 0], v[8 * w + 1], s);
        x = cvt_fp4x2<1>(x, v[8 * w + 2], v[8 * w + 3], s);
        x = cvt_fp4x2<2>(x, v[8 * w + 4], v[8 * w + 5], s);
        x = cvt_fp4x2<3>(x, v[8 * w + 6], v[8 * w + 7], s);
        words[w] = x;
      }
      sc = (uint32_t)(e + 127);
    } else {
      sc = e4m3_encode(__fdiv_rn(__fdiv_rn(amax, 6.0f), s_T));
      const float dd = __fmul_rn(e4m3_decode(sc), s_T);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t x = 0;
        x = cvt_fp4x2<0>(x, nv_scaled_w(v[8 * w + 0], dd), nv_scaled_w(v[8 * w + 1], dd), 1.0f);
        x = cvt_fp4x2<1>(x, nv_scaled_w(v[8 * w + 2], dd), nv_scaled_w(v[8 * w + 3], dd), 1.0f);
        x = cvt_fp4x2<2>(x, nv_scaled_w(v[8 * w + 4], dd), nv_scaled_w(v[8 * w + 5], dd), 1.0f);
        x = cvt_fp4x2<3>(x, nv_scaled_w(v[8 * w + 6], dd), nv_scaled_w(v[8 * w + 7], dd), 1.0f);
        words[w] = x;
      }
    }
    *reinterpret_cast<uint4*>(prow_ptr + k0 / 2) = make_uint4(words[0], words[1], words[2], words[3]);
    scales |= sc << (8 * b);
  }
  uint8_t* sp = scale_sp + prow * (K / 32) + kb0;
  if (nb == 4 && (reinterpret_cast<uintptr_t>(sp) & 3) == 0) {
    *reinterpret_cast<uint32_t*>(sp) = scales;
  } else {
    for (int b = 0; b < nb; ++b) sp[b] = (uint8_t)(scales >> (8 * b));
  }
  if (!NV) {
    if (scale_dn != scale_sp) {
      uint8_t* dn = scale_dn + prow * (K / 32) + kb0;
      for (int b = 0; b < nb; ++b) dn[b] = (uint8_t)(scales >> (8 * b));
    }
  } else {
    uint8_t* dn = scale_dn + prow * (K / 16) + 2 * kb0;
    for (int b = 0; b < nb; ++b) {
      const uint8_t s8 = (uint8_t)(scales >> (8 * b));
      dn[2 * b] = s8;
      dn[2 * b + 1] = s8;
    }
  }
}

// per-group |W| max: grid (ceil(D/256), ceil(K/ROWS), n_groups) -> partial[g][blocks]
template <bool BF16>
__global__ __launch_bounds__(256) void wamax_kernel(const void* __restrict__ W, int K, int D, int64_t ldw,
                                                    int64_t gstride, float* __restrict__ partial) {
  constexpr int ROWS = 64;
  __shared__ float lds[4];
  const int d = blockIdx.x * 256 + threadIdx.x;
  const int grp = blockIdx.z;
  float m = 0.0f;
  if (d < D) {
    const int k1 = min(K, (int)(blockIdx.y + 1) * ROWS);
    for (int k = blockIdx.y * ROWS; k < k1; ++k) m = fmaxf(m, fabsf(load_w<BF16>(W, grp * gstride + (int64_t)k * ldw + d)));
  }
#pragma unroll
  for (int s = 1; s < kWave; s <<= 1) m = fmaxf(m, __shfl_xor(m, s, kWave));
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int nblk = gridDim.x * gridDim.y;
    partial[(int64_t)grp * nblk + blockIdx.y * gridDim.x + blockIdx.x] =
        fmaxf(fmaxf(lds[0], lds[1]), fmaxf(lds[2], lds[3]));
  }
}

// one workgroup per group: tensor scale amax / 2688
__global__ __launch_bounds__(256) void wamax_finalize(const float* __restrict__ partial, int n,
                                                      float* __restrict__ tscale) {
  __shared__ float lds[4];
  const float* p = partial + (int64_t)blockIdx.x * n;
  float m = 0.0f;
  for (int i = threadIdx.x; i < n; i += 256) m = fmaxf(m, p[i]);
#pragma unroll
  for (int s = 1; s < kWave; s <<= 1) m = fmaxf(m, __shfl_xor(m, s, kWave));
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) tscale[blockIdx.x] = nv_tensor_scale_w(fmaxf(fmaxf(lds[0], lds[1]), fmaxf(lds[2], lds[3])));
}

size_t pack_nv_workspace(int K, int D, int n_groups) {
  const size_t nblk = (size_t)((D + 255) / 256) * ((K + 63) / 64);
  return nblk * n_groups * 4;
}

hipError_t launch_pack(const void* W, bool bf16, bool nv, int K, int D, int n_groups, int64_t ldw, int64_t gstride,
                       uint8_t* payload, uint8_t* scale_sp, uint8_t* scale_dn, float* tscale, void* workspace,
                       hipStream_t s) {
  if (nv) {
    dim3 ga((D + 255) / 256, (K + 63) / 64, n_groups);
    float* part = static_cast<float*>(workspace);
    if (bf16)
      hipLaunchKernelGGL(wamax_kernel<true>, ga, dim3(256), 0, s, W, K, D, ldw, gstride, part);
    else
      hipLaunchKernelGGL(wamax_kernel<false>, ga, dim3(256), 0, s, W, K, D, ldw, gstride, part);
    hipLaunchKernelGGL(wamax_finalize, dim3(n_groups), dim3(256), 0, s, part, (int)(ga.x * ga.y), tscale);
  }
  dim3 grid((D + 255) / 256, (K / 32 + 3) / 4, n_groups);
  if (bf16) {
    if (nv)
      hipLaunchKernelGGL((pack_kernel<true, true>), grid, dim3(256), 0, s, W, K, D, ldw, gstride, payload, scale_sp,
                         scale_dn, tscale);
    else
      hipLaunchKernelGGL((pack_kernel<true, false>), grid, dim3(256), 0, s, W, K, D, ldw, gstride, payload, scale_sp,
                         scale_dn, tscale);
  } else {
    if (nv)
      hipLaunchKernelGGL((pack_kernel<false, true>), grid, dim3(256), 0, s, W, K, D, ldw, gstride, payload,
                         scale_sp, scale_dn, tscale);
    else
      hipLaunchKernelGGL((pack_kernel<false, false>), grid, dim3(256), 0, s, W, K, D, ldw, gstride, payload,
                         scale_sp, scale_dn, tscale);
  }
  return hipGetLastError();
}

}  // namespace sharq
