// Dual-path GEMM for emulated NVFP4 (xllm-io paper review §3.1 two-level
// NVFP4 scaling, §3.4-§3.5 dual path with one shared weight payload).
//
// gfx950's scaled MFMA takes only power-of-two (E8M0) block scales, so an
// E4M3 block scale cannot ride along.  The product of an E2M1 value (2
// significant bits) and an E4M3 scale (4 significant bits) has at most 6
// significant bits and is exact in bf16, so each operand element is
// dequantized to q * dec(scale) in bf16 while staging and multiplied on the
// bf16 MFMA (v_mfma_f32_16x16x32_bf16, exact products, fp32 accumulation).
// The fp32 tensor scales differ between the paths, so the backbone and the
// residual keep one accumulator each inside the same tile and the epilogue
// forms Y = s_w * (s_sp * acc_sp + s_dn * acc_dn).
#include "common.h"
#include "kernels.h"

namespace sharq {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kNB = 128;                  // tile rows and columns
constexpr int kKS = 64;                   // K per staged step
constexpr int kRowB = kKS * 2;            // bytes of one staged bf16 row

SHARQ_DEV v4f mfma_bf16(uint4 a, uint4 b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

// 8 E2M1 codes (one 32-bit word) times dec -> 8 bf16 (exact: q * dec has <= 6 significant bits)
SHARQ_DEV uint4 dequant8_bf16(uint32_t word, float dec) {
  const v2f p0 = dq_fp4x2<0>(word, 1.0f), p1 = dq_fp4x2<1>(word, 1.0f);
  const v2f p2 = dq_fp4x2<2>(word, 1.0f), p3 = dq_fp4x2<3>(word, 1.0f);
  const float v[8] = {p0.x * dec, p0.y * dec, p1.x * dec, p1.y * dec, p2.x * dec, p2.y * dec, p3.x * dec, p3.y * dec};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)   // exact values: the bf16 pattern is the upper half of the fp32 pattern
    o[i] = __builtin_amdgcn_perm(__float_as_uint(v[2 * i + 1]), __float_as_uint(v[2 * i]), 0x07060302u);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// 16-byte slot of (row, chunk 0..7) in a staged bf16 tile (row = 128 bytes)
SHARQ_DEV int nslot(int row, int q) { return row * 8 + (q ^ (row & 7)); }

struct NvStage {
  uint4 a_sp[kNB * 8];
  uint4 a_dn[kNB * 8];
  uint4 b[kNB * 8];
};

}  // namespace

__global__ __launch_bounds__(256, 1) void linear_nv_tile(
    const uint8_t* __restrict__ bb_codes, const uint8_t* __restrict__ bb_meta, const uint8_t* __restrict__ bb_scale,
    const uint8_t* __restrict__ res_codes, const uint8_t* __restrict__ res_scale, const float* __restrict__ a_ts,
    const int32_t* __restrict__ row_index, int rows, int act_rows, int K, const uint8_t* __restrict__ payload,
    const uint8_t* __restrict__ wscale, const float* __restrict__ w_ts, int D, float* __restrict__ Y, int64_t ldy) {
  __shared__ NvStage st[2];
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int tiles_m = (rows + kNB - 1) / kNB;
  const int tiles_n = (D + kNB - 1) / kNB;
  const int nt = tiles_m * tiles_n;
  int b = blockIdx.x;
  if ((nt & 7) == 0) b = (b & 7) * (nt >> 3) + (b >> 3);
  const int m0 = (b % tiles_m) * kNB, n0 = (b / tiles_m) * kNB;
  const int64_t kA = K >> 2, kM = K >> 4, kS32 = K >> 5, kS16 = K >> 4, kR = K >> 1;
  const int KS = K / kKS;

  // staging units: u = tid + 256 i (i < 4): row/col = u >> 3, group g = u & 7 (8 K-values)
  const int g = tid & 7;
  int64_t arow[4], brow[4];
  bool aok[4], bok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = m0 + ((tid + 256 * i) >> 3);
    aok[i] = r < rows;
    arow[i] = aok[i] ? gather_row(row_index, r, act_rows) : 0;
    const int c = n0 + ((tid + 256 * i) >> 3);
    bok[i] = c < D;
    brow[i] = bok[i] ? c : 0;
  }
  uint32_t pc[4], pm[4], psb[4], pd[4], psd[4], pb[4], psw[4];
  // branch-free staging loads (rows / columns outside the tile read row 0,
  // whose products only reach outputs that are never stored)
  auto load_step = [&](int s) {
    const int gk = s * 8 + g;                   // global group index along K
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pc[i] = *reinterpret_cast<const uint16_t*>(bb_codes + arow[i] * kA + 2 * (int64_t)gk);
      pm[i] = bb_meta[arow[i] * kM + (gk >> 1)];
      psb[i] = bb_scale[arow[i] * kS32 + (gk >> 2)];
      pd[i] = *reinterpret_cast<const uint32_t*>(res_codes + arow[i] * kR + 4 * (int64_t)gk);
      psd[i] = res_scale[arow[i] * kS16 + (gk >> 1)];
      pb[i] = *reinterpret_cast<const uint32_t*>(payload + brow[i] * kR + 4 * (int64_t)gk);
      psw[i] = wscale[brow[i] * kS32 + (gk >> 2)];
    }
  };
  auto store_step = [&](NvStage& S) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rc = (tid + 256 * i) >> 3;
      const uint32_t nib = (g & 1) ? (pm[i] >> 4) : (pm[i] & 15u);
      S.a_sp[nslot(rc, g)] = dequant8_bf16(expand_group(pc[i], nib), e4m3_decode(psb[i]));
      S.a_dn[nslot(rc, g)] = dequant8_bf16(pd[i], e4m3_decode(psd[i]));
      S.b[nslot(rc, g)] = dequant8_bf16(pb[i], e4m3_decode(psw[i]));
    }
  };

  const int wm0 = (w >> 1) * 64, wn0 = (w & 1) * 64;
  const int kq = l >> 4, lr = l & 15;
  v4f acc_sp[4][4], acc_dn[4][4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      acc_sp[f][n] = (v4f){0.f, 0.f, 0.f, 0.f};
      acc_dn[f][n] = (v4f){0.f, 0.f, 0.f, 0.f};
    }

  load_step(0);
  store_step(st[0]);
  __syncthreads();
  for (int s = 0; s < KS; ++s) {
    load_step(min(s + 1, KS - 1));              // the last step reloads itself (unused)
    __builtin_amdgcn_sched_barrier(0);          // issue the prefetch before this step's MFMAs
    const NvStage& S = st[s & 1];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {             // two MFMA K-steps of 32
      const int q = 4 * ks + kq;                 // 16-byte chunk: K = 8 q .. 8 q + 7
      uint4 bf[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) bf[n] = S.b[nslot(wn0 + 16 * n + lr, q)];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int r = wm0 + 16 * f + lr;
        const uint4 asp = S.a_sp[nslot(r, q)];
        const uint4 adn = S.a_dn[nslot(r, q)];
#pragma unroll
        for (int n = 0; n < 4; ++n) acc_sp[f][n] = mfma_bf16(asp, bf[n], acc_sp[f][n]);
#pragma unroll
        for (int n = 0; n < 4; ++n) acc_dn[f][n] = mfma_bf16(adn, bf[n], acc_dn[f][n]);
      }
    }
    // keep the staging writes (which wait for the prefetched global loads)
    // behind this step's MFMAs, so the load latency hides under them
    __builtin_amdgcn_sched_barrier(0);
    store_step(st[(s + 1) & 1]);
    __syncthreads();
  }
  const float s_sp = a_ts[0], s_dn = a_ts[1], s_w = w_ts[0];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int c = n0 + wn0 + 16 * n + lr;
      if (c >= D) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = m0 + wm0 + 16 * f + 4 * kq + i;
        if (r < rows) Y[(int64_t)r * ldy + c] = s_w * (s_sp * acc_sp[f][n][i] + s_dn * acc_dn[f][n][i]);
      }
    }
  }
}

hipError_t launch_linear_nv(const uint8_t* bb_codes, const uint8_t* bb_meta, const uint8_t* bb_scale,
                            const uint8_t* res_codes, const uint8_t* res_scale, const float* a_ts,
                            const int32_t* row_index, int rows, int act_rows, int K, const uint8_t* payload,
                            const uint8_t* wscale, const float* w_ts, int D, float* Y, int64_t ldy, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int nt = ((rows + kNB - 1) / kNB) * ((D + kNB - 1) / kNB);
  hipLaunchKernelGGL(linear_nv_tile, dim3(nt), dim3(256), 0, s, bb_codes, bb_meta, bb_scale, res_codes, res_scale,
                     a_ts, row_index, rows, act_rows, K, payload, wscale, w_ts, D, Y, ldy);
  return hipGetLastError();
}

}  // namespace sharq
