// Device-side pieces of the MXFP4 activation preparation (xllm-io paper
// review §3.2-§3.5; kasblo explainer, method steps 1-4) shared by the
// standalone prepare kernel and the single-launch decode kernel.
#pragma once

#include "common.h"

namespace sharq {
namespace {

template <bool BF16>
SHARQ_DEV void unpack_group(const uint4& a, const uint4& b, float x[8]) {
  if (BF16) {
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y);
    x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
    x[4] = __uint_as_float(b.x); x[5] = __uint_as_float(b.y);
    x[6] = __uint_as_float(b.z); x[7] = __uint_as_float(b.w);
  }
}

// pairwise tree of the 8 squares of one group (no contraction)
SHARQ_DEV float tree8_sq(const float x[8]) {
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = __fmul_rn(x[i], x[i]);
  return __fadd_rn(__fadd_rn(__fadd_rn(q[0], q[1]), __fadd_rn(q[2], q[3])),
                   __fadd_rn(__fadd_rn(q[4], q[5]), __fadd_rn(q[6], q[7])));
}

// MXFP4 quantization of group g (8 normalized values y, one lane) and its
// stores.  Per group: pair scores, kept pairs, then per 32-value block (the 4
// lanes of a quad) the backbone scale, the codes of all four pairs (the kept
// two are compacted with one byte permute), the exact residual (y minus the
// dequantized kept pairs, y itself on dropped pairs) and its codes.  Metadata
// nibbles and scales of a block are gathered into the quad's first lane and
// stored from there.  All 64 lanes of the wave must take part (wave ballots,
// quad DPP); the output descriptors span one row, so stores of groups past
// the row (and of absent rows: zero-size descriptors) are dropped.  AUX: the
// stores' cache-policy bits.
// M24: the 2:4 element-wise backbone instead (review §3.2 general N:M mask;
// the pattern the pages pair with MXFP4): each half of the group (4 values)
// keeps its 2 largest |y|, ties to the lower index; the backbone byte of a
// half holds the kept codes (lower index in the low nibble), its metadata
// nibble their indices i0 | i1 << 2, one metadata byte per group of 8.
template <int AUX = 0, bool M24 = false>
SHARQ_DEV void mx_quantize_store(const float y[8], uint32_t g, __amdgpu_buffer_rsrc_t o_bc,
                                 __amdgpu_buffer_rsrc_t o_rc, __amdgpu_buffer_rsrc_t o_mt,
                                 __amdgpu_buffer_rsrc_t o_sb, __amdgpu_buffer_rsrc_t o_sr) {
  constexpr uint32_t kOut = 0x80000000u;
  // ---- scores, kept units (pairs, or values of each half), backbone scale
  // (the kept units hold the group's max, so the block amax is that of y)
  float sc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sc[i] = fabsf(y[i]);
  const float s0 = fmaxf(sc[0], sc[1]);
  const float s1 = fmaxf(sc[2], sc[3]);
  const float s2 = fmaxf(sc[4], sc[5]);
  const float s3 = fmaxf(sc[6], sc[7]);
  uint64_t kp[4], kq[4];
  uint32_t i0, i1, j0 = 0, j1 = 0;
  if constexpr (M24) {
    top2_lanes(sc[0], sc[1], sc[2], sc[3], kp, i0, i1);
    top2_lanes(sc[4], sc[5], sc[6], sc[7], kq, j0, j1);
  } else {
    top2_lanes(s0, s1, s2, s3, kp, i0, i1);
  }
  const uint32_t eb = e8m0_code(quad_max(fmaxf(fmaxf(s0, s1), fmaxf(s2, s3))));
  const float s_bb = exp2i((int)eb - 127);
  uint32_t bw = 0;
  bw = cvt_fp4x2<0>(bw, y[0], y[1], s_bb);
  bw = cvt_fp4x2<1>(bw, y[2], y[3], s_bb);
  bw = cvt_fp4x2<2>(bw, y[4], y[5], s_bb);
  bw = cvt_fp4x2<3>(bw, y[6], y[7], s_bb);
  // ---- residual R = y - X~_sp (exact), X~_sp = 0 on dropped pairs
  float R[8];
  {
    const v2f d[4] = {dq_fp4x2<0>(bw, s_bb), dq_fp4x2<1>(bw, s_bb), dq_fp4x2<2>(bw, s_bb), dq_fp4x2<3>(bw, s_bb)};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if constexpr (M24) {
        const uint64_t* k = p < 2 ? kp : kq;
        R[2 * p] = __fsub_rn(y[2 * p], lane_in(k[(2 * p) & 3]) ? d[p].x : 0.0f);
        R[2 * p + 1] = __fsub_rn(y[2 * p + 1], lane_in(k[(2 * p + 1) & 3]) ? d[p].y : 0.0f);
      } else {
        const bool kept = lane_in(kp[p]);
        R[2 * p] = __fsub_rn(y[2 * p], kept ? d[p].x : 0.0f);
        R[2 * p + 1] = __fsub_rn(y[2 * p + 1], kept ? d[p].y : 0.0f);
      }
    }
  }
  const float rmax = fmaxf(fmaxf(fmaxf(fabsf(R[0]), fabsf(R[1])), fmaxf(fabsf(R[2]), fabsf(R[3]))),
                           fmaxf(fmaxf(fabsf(R[4]), fabsf(R[5])), fmaxf(fabsf(R[6]), fabsf(R[7]))));
  const uint32_t er = e8m0_code(quad_max(rmax));
  const float s_r = exp2i((int)er - 127);
  uint32_t rw = 0;
  rw = cvt_fp4x2<0>(rw, R[0], R[1], s_r);
  rw = cvt_fp4x2<1>(rw, R[2], R[3], s_r);
  rw = cvt_fp4x2<2>(rw, R[4], R[5], s_r);
  rw = cvt_fp4x2<3>(rw, R[6], R[7], s_r);
  // (block values only from the quad's first lane)
  const uint32_t qo = (g & 3) == 0 ? 0u : kOut;
  if constexpr (M24) {
    // kept codes of each half: nibbles i0, i1 of bits 0-15 and j0, j1 of
    // bits 16-31; metadata of the quad's 4 groups as 32 bits in its first lane
    const uint32_t ba = __builtin_amdgcn_ubfe(bw, 4 * i0, 4) | (__builtin_amdgcn_ubfe(bw, 4 * i1, 4) << 4);
    const uint32_t bb = __builtin_amdgcn_ubfe(bw, 16 + 4 * j0, 4) | (__builtin_amdgcn_ubfe(bw, 16 + 4 * j1, 4) << 4);
    const uint32_t mb = i0 | (i1 << 2) | (j0 << 4) | (j1 << 6);
    const uint32_t m16 = mb | (dpp_u<kDppQuadXor1>(mb) << 8);
    const uint32_t m32 = (m16 & 0xFFFFu) | (dpp_u<kDppQuadXor2>(m16) << 16);
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(ba | (bb << 8)), o_bc, 2 * g, 0, AUX);
    __builtin_amdgcn_raw_buffer_store_b32(rw, o_rc, 4 * g, 0, AUX);
    __builtin_amdgcn_raw_buffer_store_b32(m32, o_mt, g | qo, 0, AUX);
  } else {
    // ---- compacted kept pair bytes (byte permute; selector 0x0C reads zero)
    const uint32_t kept2 = __builtin_amdgcn_perm(0u, bw, i0 | (i1 << 8) | 0x0C0C0000u);
    // metadata of the quad's 4 groups as 16 bits in its first lane
    const uint32_t nib = i0 | (i1 << 2);
    const uint32_t b8 = nib | (dpp_u<kDppQuadXor1>(nib) << 4);
    const uint32_t m16 = (b8 & 0xFFu) | (dpp_u<kDppQuadXor2>(b8) << 8);
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)kept2, o_bc, 2 * g, 0, AUX);
    __builtin_amdgcn_raw_buffer_store_b32(rw, o_rc, 4 * g, 0, AUX);
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)m16, o_mt, (g >> 1) | qo, 0, AUX);
  }
  __builtin_amdgcn_raw_buffer_store_b8((uint8_t)eb, o_sb, (g >> 2) | qo, 0, AUX);
  __builtin_amdgcn_raw_buffer_store_b8((uint8_t)er, o_sr, (g >> 2) | qo, 0, AUX);
}

// raw buffer descriptor of `bytes` bytes at base + byte offset off (fields
// made wave-uniform so that no waterfall loop is generated)
SHARQ_DEV __amdgpu_buffer_rsrc_t row_rsrc(const void* base, uint64_t off, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base) + off;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// One activation row prepared by the NT threads of a workgroup, held in
// registers (at most MAXC groups of 8 per thread): the MXFP4 outputs of the
// standalone prepare kernel, bit for bit.  Chunk c holds groups
// c NT .. c NT + NT - 1, so the sum of squares follows the same pinned
// pairwise tree: group tree, wave butterfly (aligned 512-value blocks), the
// chunk's waves in order, then the chunks as a tree (zero padding to a power
// of two).  load() only issues the row's and gamma's loads, so the caller can
// put other loads behind them; finish() computes and stores (cache policy
// AUX).
template <int NT, int MAXC, int AUX = 0>
struct RowPrep {
  static constexpr int WPR = NT / kWave;
  uint4 xa[MAXC], xb[MAXC];    // the thread's groups (bf16: xa; fp32: xa, xb)
  float4 ga[MAXC], gb[MAXC];   // their gamma

  // row_elem_off: element offset of the row in X; K / (8 NT) <= MAXC
  SHARQ_DEV void load(const void* X, bool bf16, int K, int64_t row_elem_off, const float* gamma) {
    const int t = threadIdx.x, G = K >> 3;
    const uint32_t es = bf16 ? 2u : 4u;
    const __amdgpu_buffer_rsrc_t rx = row_rsrc(X, (uint64_t)row_elem_off * es, (uint32_t)K * es);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const uint32_t g = (uint32_t)(c * NT + t);     // groups past K read zeros
      if (bf16) {
        const auto a = __builtin_amdgcn_raw_buffer_load_b128(rx, 16u * g, 0, 0);
        xa[c] = make_uint4(a[0], a[1], a[2], a[3]);
        xb[c] = make_uint4(0, 0, 0, 0);
      } else {
        const auto a = __builtin_amdgcn_raw_buffer_load_b128(rx, 32u * g, 0, 0);
        const auto b = __builtin_amdgcn_raw_buffer_load_b128(rx, 32u * g + 16u, 0, 0);
        xa[c] = make_uint4(a[0], a[1], a[2], a[3]);
        xb[c] = make_uint4(b[0], b[1], b[2], b[3]);
      }
      if (gamma) {
        const uint32_t k0 = g < (uint32_t)G ? 8u * g : 0u;   // lanes past K hold zeros
        ga[c] = *reinterpret_cast<const float4*>(gamma + k0);
        gb[c] = *reinterpret_cast<const float4*>(gamma + k0 + 4);
      }
    }
  }

  SHARQ_DEV void get(bool bf16, int c, float x[8]) const {
    if (bf16) unpack_group<true>(xa[c], xb[c], x);
    else unpack_group<false>(xa[c], xb[c], x);
  }

  // red: LDS scratch of at least MAXC * NT / 64 + 1 floats.  Ends with a
  // workgroup barrier; stores are issued, not awaited.
  SHARQ_DEV void finish(bool bf16, int K, const float* gamma, float eps, int row, uint8_t* bb_codes,
                        uint8_t* bb_meta, uint8_t* bb_scale, uint8_t* res_codes, uint8_t* res_scale,
                        float* red) const {
    const int t = threadIdx.x, l = t & (kWave - 1), w = t / kWave;
    float inv = 1.0f;
    if (gamma) {
      float part[MAXC];
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        float x[8];
        get(bf16, c, x);
        part[c] = wave_tree_sum(tree8_sq(x));      // chunks past K contribute +0
      }
      if (l == 0) {
#pragma unroll
        for (int c = 0; c < MAXC; ++c) red[c * WPR + w] = part[c];
      }
      __syncthreads();
      if (t == 0) {
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
          float v[WPR];
#pragma unroll
          for (int i = 0; i < WPR; ++i) v[i] = red[c * WPR + i];
#pragma unroll
          for (int n = WPR / 2; n >= 1; n >>= 1) {
#pragma unroll
            for (int i = 0; i < n; ++i) v[i] = __fadd_rn(v[2 * i], v[2 * i + 1]);
          }
          part[c] = v[0];
        }
#pragma unroll
        for (int n = MAXC / 2; n >= 1; n >>= 1) {
#pragma unroll
          for (int i = 0; i < n; ++i) part[i] = __fadd_rn(part[2 * i], part[2 * i + 1]);
        }
        const float ms = __fdiv_rn(part[0], (float)K);
        red[MAXC * WPR] = __fdiv_rn(1.0f, sqrt_rn(__fadd_rn(ms, eps)));
      }
      __syncthreads();
      inv = red[MAXC * WPR];
    }
    const __amdgpu_buffer_rsrc_t o_bc = row_rsrc(bb_codes, (uint64_t)row * (K >> 2), K >> 2);
    const __amdgpu_buffer_rsrc_t o_rc = row_rsrc(res_codes, (uint64_t)row * (K >> 1), K >> 1);
    const __amdgpu_buffer_rsrc_t o_mt = row_rsrc(bb_meta, (uint64_t)row * (K >> 4), K >> 4);
    const __amdgpu_buffer_rsrc_t o_sb = row_rsrc(bb_scale, (uint64_t)row * (K >> 5), K >> 5);
    const __amdgpu_buffer_rsrc_t o_sr = row_rsrc(res_scale, (uint64_t)row * (K >> 5), K >> 5);
    const int nch = ((K >> 3) + NT - 1) / NT;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      if (c >= nch) break;                           // whole chunk past K (uniform)
      const uint32_t g = (uint32_t)(c * NT + t);
      float y[8];
      get(bf16, c, y);
      if (gamma) {
        const float gm[8] = {ga[c].x, ga[c].y, ga[c].z, ga[c].w, gb[c].x, gb[c].y, gb[c].z, gb[c].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = __fmul_rn(__fmul_rn(y[i], inv), gm[i]);
      }
      mx_quantize_store<AUX>(y, g, o_bc, o_rc, o_mt, o_sb, o_sr);
    }
    __syncthreads();
  }
};

}  // namespace
}  // namespace sharq
