// Fused activation preparation of SharQ (xllm-io paper review §3.2-§3.5;
// kasblo explainer, method steps 1-4): RMSNorm, 4:8 in-pairs mask, backbone
// quantization + compaction, residual R = y - X~_sp and its quantization, in
// one pass over each activation row (MXFP4) or in three phases separated by
// the two tensor-wide amax reductions the emulated NVFP4 scales need.
//
// Work layout: TPR threads own one row; each thread owns whole groups of 8
// K-values (one 16-byte bf16 load or two fp32 loads), chunk c of a row being
// the 8*TPR values starting at c*8*TPR.  The row stays in registers between
// the sum of squares and the quantization, so X is read from HBM once.
//
// RMSNorm sum of squares, pinned for bit-exact codes: a pairwise tree in K
// order (zero padding to a power of two).  A thread sums its group of 8 as a
// tree, a butterfly over the wave combines aligned 512-value blocks, waves of
// the row combine in order through LDS, and the chunks are combined as a tree.
// Every fp32 operation rounds to nearest even, without contraction.
#include "common.h"
#include "kernels.h"

namespace sharq {

namespace {

template <bool BF16>
SHARQ_DEV void load_group(const void* X, int64_t off, bool ok, uint4& a, uint4& b) {
  if (!ok) { a = make_uint4(0, 0, 0, 0); b = a; return; }
  if (BF16) {
    a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(X) + off);
    b = make_uint4(0, 0, 0, 0);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(X) + off);
    a = p[0];
    b = p[1];
  }
}

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

SHARQ_DEV float tree8_sq(const float x[8]) {
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = __fmul_rn(x[i], x[i]);
  return __fadd_rn(__fadd_rn(__fadd_rn(q[0], q[1]), __fadd_rn(q[2], q[3])),
                   __fadd_rn(__fadd_rn(q[4], q[5]), __fadd_rn(q[6], q[7])));
}

// Row-resident state of one thread: its raw groups and the row's 1/rms.
template <int TPR, int MAXC, bool BF16>
struct RowRegs {
  uint4 ra[MAXC];
  uint4 rb[BF16 ? 1 : MAXC];

  SHARQ_DEV void load(const void* X, int64_t row_off, int G, int t, bool row_ok) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int g = c * TPR + t;
      uint4 b;
      load_group<BF16>(X, row_off + 8 * (int64_t)g, row_ok && g < G, ra[c], b);
      if (!BF16) rb[BF16 ? 0 : c] = b;
    }
  }
  SHARQ_DEV void get(int c, float x[8]) const {
    unpack_group<BF16>(ra[c], rb[BF16 ? 0 : c], x);
  }
};

// 1 / sqrt(mean(x^2) + eps) of the row held by the TPR threads (pinned order).
// red: LDS scratch [rows per WG][MAXC][TPR / 64].
template <int TPR, int MAXC, bool BF16>
SHARQ_DEV float row_inv_rms(const RowRegs<TPR, MAXC, BF16>& rr, int K, float eps, int t, int rsub,
                            float* red) {
  constexpr int WPR = TPR / kWave;
  float part[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    float x[8];
    rr.get(c, x);
    part[c] = tree8_sq(x);             // zeros beyond K contribute +0
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) part[c] = __fadd_rn(part[c], shfl_xor_f(part[c], m));
  }
  if (WPR > 1) {
    const int w = t / kWave;
    if ((t & (kWave - 1)) == 0) {
#pragma unroll
      for (int c = 0; c < MAXC; ++c) red[(rsub * MAXC + c) * WPR + w] = part[c];
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const float* r = red + (rsub * MAXC + c) * WPR;
      part[c] = WPR == 2 ? __fadd_rn(r[0], r[1])
                         : __fadd_rn(__fadd_rn(r[0], r[1]), __fadd_rn(r[2], r[3]));
    }
  }
#pragma unroll
  for (int w = MAXC / 2; w >= 1; w >>= 1) {
#pragma unroll
    for (int i = 0; i < w; ++i) part[i] = __fadd_rn(part[2 * i], part[2 * i + 1]);
  }
  const float ms = __fdiv_rn(part[0], (float)K);
  const float r = sqrt_rn(__fadd_rn(ms, eps));
  return __fdiv_rn(1.0f, r);
}

SHARQ_DEV void normalize(float x[8], float inv, const float* gamma, int64_t k0) {
  if (gamma == nullptr) return;
  const float4 g0 = *reinterpret_cast<const float4*>(gamma + k0);
  const float4 g1 = *reinterpret_cast<const float4*>(gamma + k0 + 4);
  const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = __fmul_rn(__fmul_rn(x[i], inv), g[i]);
}

// kept-pair bit mask of one group of 8 normalized values
SHARQ_DEV uint32_t group_mask(const float y[8], float& gmax) {
  const float s0 = fmaxf(fabsf(y[0]), fabsf(y[1]));
  const float s1 = fmaxf(fabsf(y[2]), fabsf(y[3]));
  const float s2 = fmaxf(fabsf(y[4]), fabsf(y[5]));
  const float s3 = fmaxf(fabsf(y[6]), fabsf(y[7]));
  gmax = fmaxf(fmaxf(s0, s1), fmaxf(s2, s3));
  return top2_pairs(s0, s1, s2, s3);
}

// the two kept bytes (ascending pair) of the 4-byte pair word
SHARQ_DEV uint32_t select_kept(uint32_t word, uint32_t nib) {
  const uint32_t i0 = nib & 3u, i1 = nib >> 2;
  return ((word >> (8u * i0)) & 0xFFu) | (((word >> (8u * i1)) & 0xFFu) << 8);
}

SHARQ_DEV float quad_max(float v) {
  v = fmaxf(v, shfl_xor_f(v, 1));
  return fmaxf(v, shfl_xor_f(v, 2));
}

SHARQ_DEV void store_meta_scales(uint8_t* meta_row, uint8_t* sb_row, uint8_t* sr_row, int g, uint32_t nib,
                                 uint32_t sb, uint32_t sr, bool ok, int res_per_group) {
  const uint32_t other = shfl_xor_u(nib, 1);
  if (!ok) return;
  if ((g & 1) == 0) meta_row[g >> 1] = (uint8_t)(nib | (other << 4));
  if ((g & 3) == 0) sb_row[g >> 2] = (uint8_t)sb;
  if (res_per_group == 1) {               // MXFP4: one residual scale per 32
    if ((g & 3) == 0) sr_row[g >> 2] = (uint8_t)sr;
  } else {                                 // NVFP4: one residual scale per 16
    if ((g & 1) == 0) sr_row[g >> 1] = (uint8_t)sr;
  }
}

}  // namespace

// ============================================================================
// MXFP4: one pass
// ============================================================================
template <int TPR, int MAXC, bool BF16>
__global__ __launch_bounds__(256) void prepare_mx_kernel(const void* __restrict__ X, int T, int K, int64_t ldx,
                                                         const float* __restrict__ gamma, float eps,
                                                         uint8_t* __restrict__ bb_codes, uint8_t* __restrict__ bb_meta,
                                                         uint8_t* __restrict__ bb_scale,
                                                         uint8_t* __restrict__ res_codes,
                                                         uint8_t* __restrict__ res_scale) {
  constexpr int RPW = 256 / TPR;
  __shared__ float red[RPW * MAXC * (TPR / kWave)];
  const int tid = threadIdx.x;
  const int rsub = tid / TPR, t = tid % TPR;
  const int row = blockIdx.x * RPW + rsub;
  const bool row_ok = row < T;
  const int G = K >> 3;

  RowRegs<TPR, MAXC, BF16> rr;
  rr.load(X, (int64_t)(row_ok ? row : 0) * ldx, G, t, row_ok);
  const float inv = gamma ? row_inv_rms<TPR, MAXC, BF16>(rr, K, eps, t, rsub, red) : 1.0f;

  const int64_t r = row_ok ? row : 0;
  uint8_t* meta_row = bb_meta + r * (K >> 4);
  uint8_t* sb_row = bb_scale + r * (K >> 5);
  uint8_t* sr_row = res_scale + r * (K >> 5);
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int g = c * TPR + t;
    if (c * TPR >= G) break;                       // whole chunk beyond the row (uniform)
    const bool ok = row_ok && g < G;
    float y[8];
    rr.get(c, y);
    if (ok) normalize(y, inv, gamma, 8 * (int64_t)g);
    // ---- 4:8 in-pairs mask and backbone scale (block = 4 groups = 4 lanes)
    float gmax;
    const uint32_t km = group_mask(y, gmax);
    const uint32_t nib = mask_to_nibble(km);
    const int e_bb = e8m0_exponent(quad_max(gmax));
    const float s_bb = exp2i(e_bb);
    // ---- backbone codes of all four pairs (only kept ones are stored)
    uint32_t bw = 0;
    bw = cvt_fp4x2<0>(bw, y[0], y[1], s_bb);
    bw = cvt_fp4x2<1>(bw, y[2], y[3], s_bb);
    bw = cvt_fp4x2<2>(bw, y[4], y[5], s_bb);
    bw = cvt_fp4x2<3>(bw, y[6], y[7], s_bb);
    // ---- residual R = y - X~_sp (exact), X~_sp = 0 on dropped pairs
    float R[8];
    {
      const v2f d0 = dq_fp4x2<0>(bw, s_bb), d1 = dq_fp4x2<1>(bw, s_bb);
      const v2f d2 = dq_fp4x2<2>(bw, s_bb), d3 = dq_fp4x2<3>(bw, s_bb);
      const float xt[8] = {d0.x, d0.y, d1.x, d1.y, d2.x, d2.y, d3.x, d3.y};
#pragma unroll
      for (int i = 0; i < 8; ++i) R[i] = ((km >> (i >> 1)) & 1u) ? __fsub_rn(y[i], xt[i]) : y[i];
    }
    float rmax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) rmax = fmaxf(rmax, fabsf(R[i]));
    const int e_r = e8m0_exponent(quad_max(rmax));
    const float s_r = exp2i(e_r);
    uint32_t rw = 0;
    rw = cvt_fp4x2<0>(rw, R[0], R[1], s_r);
    rw = cvt_fp4x2<1>(rw, R[2], R[3], s_r);
    rw = cvt_fp4x2<2>(rw, R[4], R[5], s_r);
    rw = cvt_fp4x2<3>(rw, R[6], R[7], s_r);
    // ---- stores
    if (ok) {
      *reinterpret_cast<uint16_t*>(bb_codes + r * (K >> 2) + 2 * (int64_t)g) = (uint16_t)select_kept(bw, nib);
      *reinterpret_cast<uint32_t*>(res_codes + r * (K >> 1) + 4 * (int64_t)g) = rw;
    }
    store_meta_scales(meta_row, sb_row, sr_row, g, nib, (uint32_t)(e_bb + 127), (uint32_t)(e_r + 127), ok, 1);
  }
}

// ============================================================================
// NVFP4 (emulated): phase 1 = RMSNorm + amax(y); phase 2 = mask, backbone
// (E4M3 per 32 logical positions under s_sp), amax(R); phase 3 = residual
// (E4M3 per 16 under s_dn).  Phases 2 and 3 recompute y from X with the
// 1/rms saved by phase 1.
// ============================================================================
namespace {

SHARQ_DEV float nv_tensor_scale(float amax) { return amax == 0.0f ? 1.0f : __fdiv_rn(amax, 2688.0f); }

// E2M1 code of fl(v / d) (d > 0) or the signed zero of v (d == 0)
SHARQ_DEV float nv_scaled(float v, float d) {
  if (!(d > 0.0f)) return v * 0.0f;
  const float t = __fdiv_rn(v, d);
  return fminf(fmaxf(t, -6.0f), 6.0f);          // saturation (|t| <= 6 is left exact)
}

// max over the WG of per-thread values (non-negative), written to out[blockIdx.x]
SHARQ_DEV void block_max_store(float v, float* out, float* lds) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v = fmaxf(v, shfl_xor_f(v, m));
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) lds[w] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = lds[0];
    for (int i = 1; i < (int)(blockDim.x / kWave); ++i) m = fmaxf(m, lds[i]);
    out[blockIdx.x] = m;
  }
}

}  // namespace

template <int TPR, int MAXC, bool BF16>
__global__ __launch_bounds__(256) void prepare_nv_phase1(const void* __restrict__ X, int T, int K, int64_t ldx,
                                                         const float* __restrict__ gamma, float eps,
                                                         float* __restrict__ inv_out, float* __restrict__ partial) {
  constexpr int RPW = 256 / TPR;
  __shared__ float red[RPW * MAXC * (TPR / kWave) + 8];
  const int tid = threadIdx.x;
  const int rsub = tid / TPR, t = tid % TPR;
  const int row = blockIdx.x * RPW + rsub;
  const bool row_ok = row < T;
  const int G = K >> 3;
  RowRegs<TPR, MAXC, BF16> rr;
  rr.load(X, (int64_t)(row_ok ? row : 0) * ldx, G, t, row_ok);
  const float inv = gamma ? row_inv_rms<TPR, MAXC, BF16>(rr, K, eps, t, rsub, red) : 1.0f;
  if (row_ok && t == 0) inv_out[row] = inv;
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int g = c * TPR + t;
    if (!(row_ok && g < G)) continue;
    float y[8];
    rr.get(c, y);
    normalize(y, inv, gamma, 8 * (int64_t)g);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(y[i]));
  }
  block_max_store(amax, partial, red + RPW * MAXC * (TPR / kWave));
}

// one workgroup: tensor scale from the partial maxima
__global__ __launch_bounds__(256) void nv_finalize_scale(const float* __restrict__ partial, int n,
                                                         float* __restrict__ scale_out) {
  __shared__ float lds[8];
  float m = 0.0f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) m = fmaxf(m, partial[i]);
#pragma unroll
  for (int s = 1; s < kWave; s <<= 1) m = fmaxf(m, shfl_xor_f(m, s));
  if ((threadIdx.x & (kWave - 1)) == 0) lds[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = lds[0];
    for (int i = 1; i < (int)(blockDim.x / kWave); ++i) a = fmaxf(a, lds[i]);
    *scale_out = nv_tensor_scale(a);
  }
}

template <int TPR, int MAXC, bool BF16, int PHASE>
__global__ __launch_bounds__(256) void prepare_nv_phase23(const void* __restrict__ X, int T, int K, int64_t ldx,
                                                          const float* __restrict__ gamma,
                                                          const float* __restrict__ inv_in,
                                                          const float* __restrict__ tensor_scales,
                                                          uint8_t* __restrict__ bb_codes, uint8_t* __restrict__ bb_meta,
                                                          uint8_t* __restrict__ bb_scale,
                                                          uint8_t* __restrict__ res_codes, uint8_t* __restrict__ res_scale,
                                                          float* __restrict__ partial) {
  constexpr int RPW = 256 / TPR;
  __shared__ float lds[8];
  const int tid = threadIdx.x;
  const int rsub = tid / TPR, t = tid % TPR;
  const int row = blockIdx.x * RPW + rsub;
  const bool row_ok = row < T;
  const int G = K >> 3;
  const int64_t r = row_ok ? row : 0;
  RowRegs<TPR, MAXC, BF16> rr;
  rr.load(X, r * ldx, G, t, row_ok);
  const float inv = row_ok ? inv_in[r] : 1.0f;
  const float s_sp = tensor_scales[0];
  const float s_dn = PHASE == 3 ? tensor_scales[1] : 1.0f;
  float rmax_all = 0.0f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int g = c * TPR + t;
    if (c * TPR >= G) break;
    const bool ok = row_ok && g < G;
    float y[8];
    rr.get(c, y);
    if (ok) normalize(y, inv, gamma, 8 * (int64_t)g);
    float gmax;
    const uint32_t km = group_mask(y, gmax);
    const uint32_t nib = mask_to_nibble(km);
    // backbone block (32 logical positions) E4M3 scale under s_sp
    const float bamax = quad_max(gmax);
    const uint32_t sc_b = e4m3_encode(__fdiv_rn(__fdiv_rn(bamax, 6.0f), s_sp));
    const float dec_b = e4m3_decode(sc_b);
    const float d_b = __fmul_rn(dec_b, s_sp);
    uint32_t bw = 0;
    bw = cvt_fp4x2<0>(bw, nv_scaled(y[0], d_b), nv_scaled(y[1], d_b), 1.0f);
    bw = cvt_fp4x2<1>(bw, nv_scaled(y[2], d_b), nv_scaled(y[3], d_b), 1.0f);
    bw = cvt_fp4x2<2>(bw, nv_scaled(y[4], d_b), nv_scaled(y[5], d_b), 1.0f);
    bw = cvt_fp4x2<3>(bw, nv_scaled(y[6], d_b), nv_scaled(y[7], d_b), 1.0f);
    float R[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q = e2m1_value((bw >> (4 * i)) & 15u);
      const float xt = __fmul_rn(__fmul_rn(q, dec_b), s_sp);
      R[i] = ((km >> (i >> 1)) & 1u) ? __fsub_rn(y[i], xt) : y[i];
    }
    if (PHASE == 2) {
      if (ok) {
        *reinterpret_cast<uint16_t*>(bb_codes + r * (K >> 2) + 2 * (int64_t)g) = (uint16_t)select_kept(bw, nib);
#pragma unroll
        for (int i = 0; i < 8; ++i) rmax_all = fmaxf(rmax_all, fabsf(R[i]));
      }
      const uint32_t other = shfl_xor_u(nib, 1);
      if (ok && (g & 1) == 0) bb_meta[r * (K >> 4) + (g >> 1)] = (uint8_t)(nib | (other << 4));
      if (ok && (g & 3) == 0) bb_scale[r * (K >> 5) + (g >> 2)] = (uint8_t)sc_b;
    } else {
      // residual block = 16 positions = 2 groups (lanes g, g^1)
      float rmax = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) rmax = fmaxf(rmax, fabsf(R[i]));
      rmax = fmaxf(rmax, shfl_xor_f(rmax, 1));
      const uint32_t sc_r = e4m3_encode(__fdiv_rn(__fdiv_rn(rmax, 6.0f), s_dn));
      const float d_r = __fmul_rn(e4m3_decode(sc_r), s_dn);
      uint32_t rw = 0;
      rw = cvt_fp4x2<0>(rw, nv_scaled(R[0], d_r), nv_scaled(R[1], d_r), 1.0f);
      rw = cvt_fp4x2<1>(rw, nv_scaled(R[2], d_r), nv_scaled(R[3], d_r), 1.0f);
      rw = cvt_fp4x2<2>(rw, nv_scaled(R[4], d_r), nv_scaled(R[5], d_r), 1.0f);
      rw = cvt_fp4x2<3>(rw, nv_scaled(R[6], d_r), nv_scaled(R[7], d_r), 1.0f);
      if (ok) {
        *reinterpret_cast<uint32_t*>(res_codes + r * (K >> 1) + 4 * (int64_t)g) = rw;
        if ((g & 1) == 0) res_scale[r * (K >> 4) + (g >> 1)] = (uint8_t)sc_r;
      }
    }
  }
  if (PHASE == 2) block_max_store(rmax_all, partial, lds);
}

// ============================================================================
// host launchers
// ============================================================================
namespace {

struct PrepGeom {
  int tpr, maxc, rpw, blocks;
};

PrepGeom prep_geometry(int T, int K) {
  const int G = K / 8;
  int tpr = 64;
  while (tpr < 256 && tpr < G) tpr *= 2;
  const int nc = (G + tpr - 1) / tpr;
  int maxc = 1;
  while (maxc < nc) maxc *= 2;
  PrepGeom g;
  g.tpr = tpr;
  g.maxc = maxc;
  g.rpw = 256 / tpr;
  g.blocks = (T + g.rpw - 1) / g.rpw;
  return g;
}

#define SHARQ_PREP_DISPATCH(MACRO)                                        \
  switch (g.tpr * 100 + g.maxc) {                                         \
    case 6401: MACRO(64, 1); break;                                       \
    case 6402: MACRO(64, 2); break;                                       \
    case 12801: MACRO(128, 1); break;                                     \
    case 12802: MACRO(128, 2); break;                                     \
    case 25601: MACRO(256, 1); break;                                     \
    case 25602: MACRO(256, 2); break;                                     \
    case 25604: MACRO(256, 4); break;                                     \
    case 25608: MACRO(256, 8); break;                                     \
    case 25616: MACRO(256, 16); break;                                    \
    default: return hipErrorInvalidValue;                                 \
  }

}  // namespace

int prepare_max_k() { return 256 * 8 * 16; }

size_t prepare_nv_workspace(int T, int K) {
  const PrepGeom g = prep_geometry(T, K);
  return (size_t)T * 4 + (size_t)g.blocks * 4 * 2 + 256;
}

hipError_t launch_prepare_mx(const void* X, bool bf16, int T, int K, int64_t ldx, const float* gamma, float eps,
                             uint8_t* bb_codes, uint8_t* bb_meta, uint8_t* bb_scale, uint8_t* res_codes,
                             uint8_t* res_scale, hipStream_t s) {
  const PrepGeom g = prep_geometry(T, K);
#define L(TPR, MAXC)                                                                                   \
  if (bf16)                                                                                            \
    hipLaunchKernelGGL((prepare_mx_kernel<TPR, MAXC, true>), dim3(g.blocks), dim3(256), 0, s, X, T, K, ldx, \
                       gamma, eps, bb_codes, bb_meta, bb_scale, res_codes, res_scale);                 \
  else                                                                                                 \
    hipLaunchKernelGGL((prepare_mx_kernel<TPR, MAXC, false>), dim3(g.blocks), dim3(256), 0, s, X, T, K, ldx, \
                       gamma, eps, bb_codes, bb_meta, bb_scale, res_codes, res_scale);
  SHARQ_PREP_DISPATCH(L)
#undef L
  return hipGetLastError();
}

hipError_t launch_prepare_nv(const void* X, bool bf16, int T, int K, int64_t ldx, const float* gamma, float eps,
                             uint8_t* bb_codes, uint8_t* bb_meta, uint8_t* bb_scale, uint8_t* res_codes,
                             uint8_t* res_scale, float* tensor_scales, void* workspace, hipStream_t s) {
  const PrepGeom g = prep_geometry(T, K);
  float* inv = static_cast<float*>(workspace);
  float* part_y = inv + T;
  float* part_r = part_y + g.blocks;
#define L(TPR, MAXC)                                                                                         \
  if (bf16) {                                                                                                \
    hipLaunchKernelGGL((prepare_nv_phase1<TPR, MAXC, true>), dim3(g.blocks), dim3(256), 0, s, X, T, K, ldx,   \
                       gamma, eps, inv, part_y);                                                             \
    hipLaunchKernelGGL(nv_finalize_scale, dim3(1), dim3(256), 0, s, part_y, g.blocks, tensor_scales);       \
    hipLaunchKernelGGL((prepare_nv_phase23<TPR, MAXC, true, 2>), dim3(g.blocks), dim3(256), 0, s, X, T, K,  \
                       ldx, gamma, inv, tensor_scales, bb_codes, bb_meta, bb_scale, res_codes, res_scale,    \
                       part_r);                                                                              \
    hipLaunchKernelGGL(nv_finalize_scale, dim3(1), dim3(256), 0, s, part_r, g.blocks, tensor_scales + 1);   \
    hipLaunchKernelGGL((prepare_nv_phase23<TPR, MAXC, true, 3>), dim3(g.blocks), dim3(256), 0, s, X, T, K,  \
                       ldx, gamma, inv, tensor_scales, bb_codes, bb_meta, bb_scale, res_codes, res_scale,    \
                       part_r);                                                                              \
  } else {                                                                                                   \
    hipLaunchKernelGGL((prepare_nv_phase1<TPR, MAXC, false>), dim3(g.blocks), dim3(256), 0, s, X, T, K, ldx,  \
                       gamma, eps, inv, part_y);                                                             \
    hipLaunchKernelGGL(nv_finalize_scale, dim3(1), dim3(256), 0, s, part_y, g.blocks, tensor_scales);       \
    hipLaunchKernelGGL((prepare_nv_phase23<TPR, MAXC, false, 2>), dim3(g.blocks), dim3(256), 0, s, X, T, K, \
                       ldx, gamma, inv, tensor_scales, bb_codes, bb_meta, bb_scale, res_codes, res_scale,    \
                       part_r);                                                                              \
    hipLaunchKernelGGL(nv_finalize_scale, dim3(1), dim3(256), 0, s, part_r, g.blocks, tensor_scales + 1);   \
    hipLaunchKernelGGL((prepare_nv_phase23<TPR, MAXC, false, 3>), dim3(g.blocks), dim3(256), 0, s, X, T, K, \
                       ldx, gamma, inv, tensor_scales, bb_codes, bb_meta, bb_scale, res_codes, res_scale,    \
                       part_r);                                                                              \
  }
  SHARQ_PREP_DISPATCH(L)
#undef L
  return hipGetLastError();
}

}  // namespace sharq
