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
#include <mutex>
#include <unordered_map>

#include "common.h"
#include "kernels.h"
#include "prep_device.h"

namespace sharq {

namespace {

// Row-resident state of one thread: its raw groups.  Loads go through a raw
// buffer descriptor spanning the row (no bytes for an absent row), so groups
// past K and absent rows read zeros without branches.
template <int TPR, int MAXC, bool BF16>
struct RowRegs {
  uint4 ra[MAXC];
  uint4 rb[BF16 ? 1 : MAXC];

  SHARQ_DEV void load(const void* X, int64_t row_off, int G, int t, bool row_ok) {
    constexpr int ES = BF16 ? 2 : 4;                   // bytes per element
    const uint64_t base = reinterpret_cast<uint64_t>(X) + (uint64_t)row_off * ES;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
    const int bytes = __builtin_amdgcn_readfirstlane(row_ok ? G * 8 * ES : 0);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, bytes, 0x00020000);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const uint32_t g = (uint32_t)(c * TPR + t);
      const auto a = __builtin_amdgcn_raw_buffer_load_b128(rs, g * (8u * ES), 0, 0);
      ra[c] = make_uint4(a[0], a[1], a[2], a[3]);
      if (!BF16) {
        const auto b = __builtin_amdgcn_raw_buffer_load_b128(rs, g * (8u * ES) + 16u, 0, 0);
        rb[BF16 ? 0 : c] = make_uint4(b[0], b[1], b[2], b[3]);
      }
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
    part[c] = wave_tree_sum(tree8_sq(x));   // zeros beyond K contribute +0
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
      // pairwise tree over the row's waves (aligned wave blocks, in order)
      const float* r = red + (rsub * MAXC + c) * WPR;
      float v[WPR];
#pragma unroll
      for (int i = 0; i < WPR; ++i) v[i] = r[i];
#pragma unroll
      for (int n = WPR / 2; n >= 1; n >>= 1) {
#pragma unroll
        for (int i = 0; i < n; ++i) v[i] = __fadd_rn(v[2 * i], v[2 * i + 1]);
      }
      part[c] = v[0];
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

}  // namespace

// ============================================================================
// MXFP4: one pass
// ============================================================================
// Per group of 8 (one lane): normalize, then mx_quantize_store (pair scores,
// kept pairs, backbone and residual codes and scales of the quad's 32-value
// block, metadata).
//
// Workgroups loop over blocks of RPW rows (block b, b + grid, ...).  gamma of
// the thread's groups is read once, and the next block's rows are loaded while
// the current block is quantized, so HBM reads, the arithmetic and the stores
// of different rows overlap inside every wave.
template <int TPR, int MAXC, bool BF16, bool NORM, bool M24 = false>
struct MxRowPass {
  static constexpr int WGT = TPR > 256 ? TPR : 256;  // threads per workgroup
  static constexpr int RPW = WGT / TPR, WPR = TPR / kWave;
  static constexpr int RED = RPW * MAXC * WPR;      // LDS floats per parity
  // gamma staged in LDS once per workgroup when the padded row fits in 32 KB,
  // else read from global memory per chunk
  static constexpr bool GLDS = NORM && TPR * MAXC * 8 * 4 <= 32768;
  static constexpr int GSM = GLDS ? TPR * MAXC * 2 : 1;   // float4s
  // the next rows are prefetched into registers when two row copies fit
  static constexpr bool CACHE = 2 * MAXC * (BF16 ? 4 : 8) <= 64;

  const float* gp;
  const float4* gs;

  // every thread of the workgroup calls this (it ends with a barrier)
  SHARQ_DEV void load_gamma(const float* gamma, int K, float4* gsm) {
    gp = gamma;
    gs = gsm;
    if (!GLDS) return;
    for (int i = threadIdx.x; i < GSM; i += WGT)
      gsm[i] = 4 * i < K ? *reinterpret_cast<const float4*>(gamma + 4 * i) : make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();
  }

  SHARQ_DEV void run(const RowRegs<TPR, MAXC, BF16>& rr, int row, bool row_ok, int K, float eps, int t, int rsub,
                     float* red, uint8_t* bb_codes, uint8_t* bb_meta, uint8_t* bb_scale, uint8_t* res_codes,
                     uint8_t* res_scale) const {
    const int G = K >> 3;
    const float inv = NORM ? row_inv_rms<TPR, MAXC, BF16>(rr, K, eps, t, rsub, red) : 1.0f;
    // output rows through raw buffer descriptors (uniform per wave): stores
    // at an offset past the row (lanes past K, absent rows) are dropped
    const int64_t r = __builtin_amdgcn_readfirstlane(row_ok ? row : 0);
    auto orow = [&](uint8_t* base, int row_bytes) {
      const uint64_t a = reinterpret_cast<uint64_t>(base) + (uint64_t)r * row_bytes;
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
      return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0,
                                               __builtin_amdgcn_readfirstlane(row_ok ? row_bytes : 0), 0x00020000);
    };
    const __amdgpu_buffer_rsrc_t o_bc = orow(bb_codes, K >> 2), o_rc = orow(res_codes, K >> 1);
    const __amdgpu_buffer_rsrc_t o_mt = orow(bb_meta, M24 ? K >> 3 : K >> 4), o_sb = orow(bb_scale, K >> 5);
    const __amdgpu_buffer_rsrc_t o_sr = orow(res_scale, K >> 5);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const uint32_t g = (uint32_t)(c * TPR + t);
      if (c * TPR >= G) break;                       // whole chunk beyond the row (uniform)
      const bool ok = row_ok && g < (uint32_t)G;
      float y[8];
      rr.get(c, y);
      if (NORM) {
        float4 ga, gb;
        if (GLDS) {
          ga = gs[2 * g];
          gb = gs[2 * g + 1];
        } else {
          const uint32_t k0 = ok ? 8u * g : 0u;      // lanes past K hold zeros
          ga = *reinterpret_cast<const float4*>(gp + k0);
          gb = *reinterpret_cast<const float4*>(gp + k0 + 4);
        }
        const float gm[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = __fmul_rn(__fmul_rn(y[i], inv), gm[i]);
      }
      mx_quantize_store<0, M24>(y, g, o_bc, o_rc, o_mt, o_sb, o_sr);
    }
  }
};

template <int TPR, int MAXC, bool BF16, bool NORM, bool M24>
__global__ __launch_bounds__(TPR > 256 ? TPR : 256) void prepare_mx_kernel(const void* __restrict__ X, int T, int K, int64_t ldx,
                                                         const float* __restrict__ gamma, float eps,
                                                         uint8_t* __restrict__ bb_codes, uint8_t* __restrict__ bb_meta,
                                                         uint8_t* __restrict__ bb_scale,
                                                         uint8_t* __restrict__ res_codes,
                                                         uint8_t* __restrict__ res_scale) {
  using Pass = MxRowPass<TPR, MAXC, BF16, NORM, M24>;
  constexpr int RPW = Pass::RPW;
  // two parities: a block's cross-wave partial sums are read before the
  // barrier of the next block, so the block after next may overwrite them
  __shared__ float red[2 * Pass::RED];
  __shared__ float4 gsm[Pass::GSM];
  const int tid = threadIdx.x;
  const int rsub = __builtin_amdgcn_readfirstlane(tid / TPR);   // TPR is a multiple of the wave
  const int t = tid % TPR;
  const int G = K >> 3;
  const int nblk = (T + RPW - 1) / RPW;

  Pass pass;
  RowRegs<TPR, MAXC, BF16> ra, rb;
  auto load = [&](RowRegs<TPR, MAXC, BF16>& rr, int blk) {
    const int row = blk * RPW + rsub;
    const bool ok = blk < nblk && row < T;
    rr.load(X, (int64_t)(ok ? row : 0) * ldx, G, t, ok);
  };
  auto step = [&](const RowRegs<TPR, MAXC, BF16>& cur, RowRegs<TPR, MAXC, BF16>& nxt, int blk, int par) {
    load(nxt, blk + (int)gridDim.x);
    const int row = blk * RPW + rsub;
    pass.run(cur, row, row < T, K, eps, t, rsub, red + par * Pass::RED, bb_codes, bb_meta, bb_scale, res_codes,
             res_scale);
  };
  int blk = blockIdx.x;
  load(ra, blk);                                       // first rows in flight while gamma is staged
  pass.load_gamma(gamma, K, gsm);
  if (Pass::CACHE) {
    while (blk < nblk) {
      step(ra, rb, blk, 0);
      blk += gridDim.x;
      if (blk >= nblk) break;
      step(rb, ra, blk, 1);
      blk += gridDim.x;
    }
  } else {
    for (int par = 0; blk < nblk; blk += gridDim.x, par ^= 1) {
      if (blk != (int)blockIdx.x) load(ra, blk);
      const int row = blk * RPW + rsub;
      pass.run(ra, row, row < T, K, eps, t, rsub, red + par * Pass::RED, bb_codes, bb_meta, bb_scale, res_codes,
               res_scale);
    }
  }
}

// ============================================================================
// Plain baseline: RMSNorm and MXFP4 quantization as two separate kernels,
// the unfused pipeline that the fused preparation replaces (xllm-io paper
// review, kernel latency breakdown of §5).  y goes through HBM in fp32, the
// precision the fused path keeps it in.
// ============================================================================
template <int TPR, int MAXC, bool BF16, bool NORM>
__global__ __launch_bounds__(TPR > 256 ? TPR : 256) void rmsnorm_kernel(const void* __restrict__ X, int T, int K,
                                                                        int64_t ldx, const float* __restrict__ gamma,
                                                                        float eps, float* __restrict__ Y, int64_t ldy) {
  constexpr int WGT = TPR > 256 ? TPR : 256, RPW = WGT / TPR, WPR = TPR / kWave;
  __shared__ float red[RPW * MAXC * WPR];
  const int tid = threadIdx.x;
  const int rsub = __builtin_amdgcn_readfirstlane(tid / TPR);
  const int t = tid % TPR, G = K >> 3;
  const int nblk = (T + RPW - 1) / RPW;
  for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const int row = blk * RPW + rsub;
    const bool ok = row < T;
    RowRegs<TPR, MAXC, BF16> rr;
    rr.load(X, (int64_t)(ok ? row : 0) * ldx, G, t, ok);
    // the same pinned 1/rms and y = (x * inv) * gamma as the fused preparation
    const float inv = NORM ? row_inv_rms<TPR, MAXC, BF16>(rr, K, eps, t, rsub, red) : 1.0f;
    float* yr = Y + (int64_t)(ok ? row : 0) * ldy;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      if (c * TPR >= G) break;                        // whole chunk beyond the row (uniform)
      const int g = c * TPR + t;
      float y[8];
      rr.get(c, y);
      if (NORM) normalize(y, inv, gamma, 8 * (int64_t)(g < G ? g : 0));
      if (ok && g < G) {
        float4* o = reinterpret_cast<float4*>(yr + 8 * (int64_t)g);
        o[0] = make_float4(y[0], y[1], y[2], y[3]);
        o[1] = make_float4(y[4], y[5], y[6], y[7]);
      }
    }
    __syncthreads();                                  // red is reused by the next block's rows
  }
}

// Plain MXFP4 of fp32 rows (review §3.1 block scale, rounded up to a power of
// two): one group of 8 per thread, the 4 groups of a 32-block in one quad;
// the block scale comes from the quad's max and is stored by its first lane.
__global__ __launch_bounds__(256) void quantize_mx_kernel(const float* __restrict__ Y, int T, int K, int64_t ldy,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const int G = K >> 3;
  const int g = blockIdx.x * 256 + threadIdx.x;
  const bool ok = g < G;                              // uniform per quad: G % 4 == 0
  for (int row = blockIdx.y; row < T; row += gridDim.y) {
    float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (ok) {
      const float4* src = reinterpret_cast<const float4*>(Y + (int64_t)row * ldy + 8 * (int64_t)g);
      const float4 a = src[0], b = src[1];
      y[0] = a.x; y[1] = a.y; y[2] = a.z; y[3] = a.w;
      y[4] = b.x; y[5] = b.y; y[6] = b.z; y[7] = b.w;
    }
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(y[i]));
    const uint32_t e = e8m0_code(quad_max(am));
    const float sc = exp2i((int)e - 127);
    uint32_t w = 0;
    w = cvt_fp4x2<0>(w, y[0], y[1], sc);
    w = cvt_fp4x2<1>(w, y[2], y[3], sc);
    w = cvt_fp4x2<2>(w, y[4], y[5], sc);
    w = cvt_fp4x2<3>(w, y[6], y[7], sc);
    if (ok) {
      reinterpret_cast<uint32_t*>(codes + (int64_t)row * (K >> 1))[g] = w;
      if ((g & 3) == 0) scales[(int64_t)row * (K >> 5) + (g >> 2)] = (uint8_t)e;
    }
  }
}

// ============================================================================
// NVFP4 (emulated): phase 1 = RMSNorm + amax(y); phase 2 = mask, backbone
// (E4M3 per 32 logical positions under s_sp), amax(R); phase 3 = residual
// (E4M3 per 16 under s_dn).  Phases 2 and 3 recompute y from X with the
// 1/rms saved by phase 1; phase 3 reads back the backbone phase 2 stored
// (kept pairs, block scale, kept codes) to form R.
// ============================================================================
namespace {

SHARQ_DEV float nv_tensor_scale(float amax) { return amax == 0.0f ? 1.0f : __fdiv_rn(amax, 2688.0f); }

// E2M1 code of fl(v / d) (d > 0) or the signed zero of v (d == 0)
SHARQ_DEV float nv_scaled(float v, float d) {
  if (!(d > 0.0f)) return v * 0.0f;
  const float t = __fdiv_rn(v, d);
  return fminf(fmaxf(t, -6.0f), 6.0f);          // saturation (|t| <= 6 is left exact)
}

// E2M1 codes (one 32-bit word, value i in nibble i) of fl(v[i] / d) under
// nv_scaled.  Fast path: with r = rcp(d) (within 1 ulp of 1/d), the products
// v * fl(r (1 - 2^-20)) and v * fl(r (1 + 2^-20)) bracket fl(v / d) strictly
// (three roundings and the reciprocal's error stay below 2^-21 relative), and
// clamping and E2M1 rounding are monotonic, so when both brackets give the
// same codes those are the codes of fl(v / d).  They differ only within about
// 2^-20 of an E2M1 rounding midpoint (or for non-normal d); then the group
// takes the correctly rounded division.
SHARQ_DEV uint32_t nv_codes8(const float v[8], float d) {
  if (d >= 0x1p-125f && d <= 0x1p125f) {
    const float r = __builtin_amdgcn_rcpf(d);
    const float rl = __fmul_rn(r, 1.0f - 0x1p-20f), rh = __fmul_rn(r, 1.0f + 0x1p-20f);
    auto cl = [](float t) { return fminf(fmaxf(t, -6.0f), 6.0f); };
    uint32_t lo = 0, hi = 0;
    lo = cvt_fp4x2<0>(lo, cl(__fmul_rn(v[0], rl)), cl(__fmul_rn(v[1], rl)), 1.0f);
    lo = cvt_fp4x2<1>(lo, cl(__fmul_rn(v[2], rl)), cl(__fmul_rn(v[3], rl)), 1.0f);
    lo = cvt_fp4x2<2>(lo, cl(__fmul_rn(v[4], rl)), cl(__fmul_rn(v[5], rl)), 1.0f);
    lo = cvt_fp4x2<3>(lo, cl(__fmul_rn(v[6], rl)), cl(__fmul_rn(v[7], rl)), 1.0f);
    hi = cvt_fp4x2<0>(hi, cl(__fmul_rn(v[0], rh)), cl(__fmul_rn(v[1], rh)), 1.0f);
    hi = cvt_fp4x2<1>(hi, cl(__fmul_rn(v[2], rh)), cl(__fmul_rn(v[3], rh)), 1.0f);
    hi = cvt_fp4x2<2>(hi, cl(__fmul_rn(v[4], rh)), cl(__fmul_rn(v[5], rh)), 1.0f);
    hi = cvt_fp4x2<3>(hi, cl(__fmul_rn(v[6], rh)), cl(__fmul_rn(v[7], rh)), 1.0f);
    if (lo == hi) return lo;
  }
  uint32_t w = 0;
  w = cvt_fp4x2<0>(w, nv_scaled(v[0], d), nv_scaled(v[1], d), 1.0f);
  w = cvt_fp4x2<1>(w, nv_scaled(v[2], d), nv_scaled(v[3], d), 1.0f);
  w = cvt_fp4x2<2>(w, nv_scaled(v[4], d), nv_scaled(v[5], d), 1.0f);
  w = cvt_fp4x2<3>(w, nv_scaled(v[6], d), nv_scaled(v[7], d), 1.0f);
  return w;
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
    uint32_t km, nib, sc_b, bw;                         // kept pairs, metadata, block scale, pair codes
    if constexpr (PHASE == 3) {
      // the backbone phase 2 stored: metadata nibble, block scale and the two
      // kept pair bytes (dropped pairs' codes stay zero; R does not use them)
      uint32_t kb = 0u;
      nib = 4u;
      sc_b = 0u;
      if (ok) {
        const uint32_t mb = bb_meta[r * (K >> 4) + (g >> 1)];
        nib = (g & 1) ? mb >> 4 : mb & 15u;
        sc_b = bb_scale[r * (K >> 5) + (g >> 2)];
        kb = *reinterpret_cast<const uint16_t*>(bb_codes + r * (K >> 2) + 2 * (int64_t)g);
      }
      const uint32_t i0 = nib & 3u, i1 = nib >> 2;
      km = (1u << i0) | (1u << i1);
      bw = ((kb & 0xFFu) << (8u * i0)) | ((kb >> 8) << (8u * i1));
    } else {
      float gmax;
      km = group_mask(y, gmax);
      nib = mask_to_nibble(km);
      // backbone block (32 logical positions) E4M3 scale under s_sp
      const float bamax = quad_max(gmax);
      sc_b = e4m3_encode(__fdiv_rn(__fdiv_rn(bamax, 6.0f), s_sp));
      bw = nv_codes8(y, __fmul_rn(e4m3_decode(sc_b), s_sp));
    }
    const float dec_b = e4m3_decode(sc_b);
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
      const uint32_t rw = nv_codes8(R, d_r);
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
  int threads = 256;
};

// compute units of the current device (queried once per device)
int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

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

// MXFP4 kernel: up to 4 groups per thread before the row is spread over more
// threads, so per-row work (1/rms) is shared by several groups
PrepGeom prep_geometry_mx(int T, int K) {
  const int G = K / 8;
  // Few rows (decode): a row spreads over up to 16 waves (one workgroup), one
  // group of 8 per thread where possible, to shorten its dependent chain.
  // Many rows: one wave per row and up to 8 groups per thread, so the
  // per-row work (1/rms) is shared by more groups and no cross-wave
  // reduction is needed.
  const bool wide = (int64_t)T * G < (int64_t)1024 * 64 * 8;
  int tpr = 64;
  if (wide) {
    while (tpr < 1024 && tpr < G) tpr *= 2;
  } else {
    while (tpr < 256 && tpr * 8 < G) tpr *= 2;
  }
  const int nc = (G + tpr - 1) / tpr;
  int maxc = 1;
  while (maxc < nc) maxc *= 2;
  PrepGeom g;
  g.tpr = tpr;
  g.maxc = maxc;
  g.threads = tpr > 256 ? tpr : 256;
  g.rpw = g.threads / tpr;
  const int nblk = (T + g.rpw - 1) / g.rpw;
  // short rows (at most 2 groups per thread, few registers): one workgroup
  // per row block, so that many waves per SIMD hide the latencies; long rows:
  // two workgroups of four waves per CU (two waves per SIMD), each looping
  // over row blocks with the next rows prefetched (measured: 32768 x 768
  // 23.6 vs 29.8 us; 4096 x 4096 16.6 vs 18.6 us the other way round)
  g.blocks = (maxc <= 2 || nblk < 2 * num_cus()) ? nblk : 2 * num_cus();
  return g;
}

#define SHARQ_PREP_MX_DISPATCH(MACRO)                                     \
  switch (g.tpr * 100 + g.maxc) {                                         \
    case 6401: MACRO(64, 1); break;                                       \
    case 6402: MACRO(64, 2); break;                                       \
    case 6404: MACRO(64, 4); break;                                       \
    case 6408: MACRO(64, 8); break;                                       \
    case 12801: MACRO(128, 1); break;                                     \
    case 12808: MACRO(128, 8); break;                                     \
    case 25601: MACRO(256, 1); break;                                     \
    case 25608: MACRO(256, 8); break;                                     \
    case 25616: MACRO(256, 16); break;                                    \
    case 51201: MACRO(512, 1); break;                                     \
    case 102401: MACRO(1024, 1); break;                                   \
    case 102402: MACRO(1024, 2); break;                                   \
    case 102404: MACRO(1024, 4); break;                                   \
    default: return hipErrorInvalidValue;                                 \
  }

}  // namespace

int prepare_max_k() { return 256 * 8 * 16; }

// ---- static scratch of the allocation-free prepare (sharq_prepare_no_alloc)
// The NVFP4 preparation needs prepare_nv_workspace(T, K) bytes of scratch
// (per-row 1/rms and per-workgroup partial maxima).  Callers that cannot
// allocate get it from this file-scope array instead: each GPU the library
// runs on holds its own copy until the process ends.  Every block writes its
// own entries before they are read, so nothing needs clearing between calls;
// calls that overlap on one GPU share the array and race.
constexpr size_t kScratchBytes = (size_t)1 << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
std::unordered_map<int, void*> g_scratch_ptr;   // device -> address of its copy of `scratch`
}  // namespace

size_t scratch_max_bytes() { return kScratchBytes; }

// Device address of the current device's `scratch` (looked up once per
// device; in host code the array's name is only a host-side stand-in).
hipError_t scratch_device_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    it = g_scratch_ptr.emplace(dev, p).first;
  }
  *out = it->second;
  return hipSuccess;
}

size_t prepare_nv_workspace(int T, int K) {
  const PrepGeom g = prep_geometry(T, K);
  return (size_t)T * 4 + (size_t)g.blocks * 4 * 2 + 256;
}

hipError_t launch_prepare_mx(const void* X, bool bf16, int T, int K, int64_t ldx, const float* gamma, float eps,
                             uint8_t* bb_codes, uint8_t* bb_meta, uint8_t* bb_scale, uint8_t* res_codes,
                             uint8_t* res_scale, hipStream_t s, bool m24) {
  const PrepGeom g = prep_geometry_mx(T, K);
#define L3(TPR, MAXC, B, N, M)                                                                                      \
  hipLaunchKernelGGL((prepare_mx_kernel<TPR, MAXC, B, N, M>), dim3(g.blocks), dim3(g.threads), 0, s, X, T, K, ldx, \
                     gamma, eps, bb_codes, bb_meta, bb_scale, res_codes, res_scale)
#define L2(TPR, MAXC, B, N)                  \
  if (m24) L3(TPR, MAXC, B, N, true);        \
  else L3(TPR, MAXC, B, N, false)
#define L(TPR, MAXC)                                   \
  if (bf16) {                                          \
    if (gamma) L2(TPR, MAXC, true, true);              \
    else L2(TPR, MAXC, true, false);                   \
  } else {                                             \
    if (gamma) L2(TPR, MAXC, false, true);             \
    else L2(TPR, MAXC, false, false);                  \
  }
  SHARQ_PREP_MX_DISPATCH(L)
#undef L
#undef L2
#undef L3
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const void* X, bool bf16, int T, int K, int64_t ldx, const float* gamma, float eps, float* Y,
                          int64_t ldy, hipStream_t s) {
  const PrepGeom g = prep_geometry_mx(T, K);
#define L2(TPR, MAXC, B, N)                                                                                 \
  hipLaunchKernelGGL((rmsnorm_kernel<TPR, MAXC, B, N>), dim3(g.blocks), dim3(g.threads), 0, s, X, T, K, ldx, \
                     gamma, eps, Y, ldy)
#define L(TPR, MAXC)                                   \
  if (bf16) {                                          \
    if (gamma) L2(TPR, MAXC, true, true);              \
    else L2(TPR, MAXC, true, false);                   \
  } else {                                             \
    if (gamma) L2(TPR, MAXC, false, true);             \
    else L2(TPR, MAXC, false, false);                  \
  }
  SHARQ_PREP_MX_DISPATCH(L)
#undef L
#undef L2
  return hipGetLastError();
}

hipError_t launch_quantize_mx(const float* Y, int T, int K, int64_t ldy, uint8_t* codes, uint8_t* scales,
                              hipStream_t s) {
  const int G = K / 8;
  dim3 grid((G + 255) / 256, T < 65535 ? T : 65535);
  hipLaunchKernelGGL(quantize_mx_kernel, grid, dim3(256), 0, s, Y, T, K, ldy, codes, scales);
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
