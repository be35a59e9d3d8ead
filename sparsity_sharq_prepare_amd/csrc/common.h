// Device-side helpers shared by the SharQ kernels (gfx950 / CDNA4).
//
// Number formats follow the SharQ pages (xllm-io paper review §3.1 block
// scales, §5.3 MXFP4 power-of-two scale; kasblo explainer: NVFP4 = 16 E2M1
// values + one E4M3 scale), with these exact rules:
//  - E2M1 rounding is to nearest, ties to the even code, saturating at 6, the
//    sign copied from the input.  gfx950's v_cvt_scalef32_pk_fp4_f32 computes
//    exactly this for x / 2^e (checked exhaustively against an integer
//    reference over all fp32 inputs |x| <= 6 * 2^e on MI355X).
//  - MXFP4 scale exponent: the smallest e with amax <= 6 * 2^e, in [-127, 127].
//  - E4M3: OCP FP8 (bias 7, max 448), nearest, ties to even, saturating.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define SHARQ_DEV __device__ __forceinline__

namespace sharq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef short v8s __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- E8M0 (MXFP4)
// amax = 1.m * 2^(E-127) (biased E): amax <= 6 * 2^e  <=>  e >= E-129 (m <= 0.5)
// or e >= E-128 (m > 0.5).  Zero and subnormal amax give e <= -128 -> -127.
SHARQ_DEV int e8m0_exponent(float amax) {
  uint32_t b = __float_as_uint(amax);
  int e = (int)(b >> 23) - 129 + ((b & 0x7FFFFFu) > 0x400000u ? 1 : 0);
  return e < -127 ? -127 : e;
}

// 2^e as fp32 (e in [-127, 127]; 2^-127 is a subnormal, handled by v_ldexp).
SHARQ_DEV float exp2i(int e) { return __builtin_amdgcn_ldexpf(1.0f, e); }

// Two E2M1 codes of a / 2^e and b / 2^e (|.| <= 6 * 2^e) into byte `sel` of `old`:
// a -> low nibble, b -> high nibble.
template <int SEL>
SHARQ_DEV uint32_t cvt_fp4x2(uint32_t old, float a, float b, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, SEL);
}

// Values of the two E2M1 codes in byte `SEL` of `word`, times scale (exact).
template <int SEL>
SHARQ_DEV v2f dq_fp4x2(uint32_t word, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, scale, SEL);
}

// ---------------------------------------------------------------- E4M3 (OCP)
// Code of non-negative u: nearest finite value, ties to even, saturating at 448.
SHARQ_DEV uint32_t e4m3_encode(float u) {
  if (!(u < 448.0f)) return 0x7Eu;
  if (u < 0.015625f) {                       // below 2^-6: subnormal grid m * 2^-9
    float m = __builtin_rintf(u * 512.0f);   // exact scaling, ties to even
    return (uint32_t)m;                      // 0..8 (8 == 0x08 == 2^-6)
  }
  uint32_t b = __float_as_uint(u);
  b = b + 0x7FFFFu + ((b >> 20) & 1u);       // round mantissa to 3 bits, ties to even
  uint32_t code = (b >> 20) - (120u << 3);   // rebias 127 -> 7
  return code > 0x7Eu ? 0x7Eu : code;
}

SHARQ_DEV float e4m3_decode(uint32_t code) {
  const uint32_t E = (code >> 3) & 15u, M = code & 7u;
  // subnormal (E = 0): M * 2^-9; normal: (8 + M) * 2^(E - 10); selects, not
  // a branch, so that callers' loops stay one basic block
  const uint32_t m = E == 0 ? M : 8u + M;
  const int e = E == 0 ? -9 : (int)E - 10;
  return __builtin_amdgcn_ldexpf((float)m, e);
}

// ---------------------------------------------------------------- E2M1 value
SHARQ_DEV float e2m1_value(uint32_t code) {
  // twice the magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 as nibbles of one word
  const float v = 0.5f * (float)((0xC8643210u >> (4u * (code & 7u))) & 15u);
  return (code & 8u) ? -v : v;
}

// ---------------------------------------------------------------- sqrt
// Correctly rounded fp32 square root of v >= 0.  v_sqrt_f32 (what __fsqrt_rn
// lowers to on gfx950) can be one ulp off; here the double-precision root is
// rounded to fp32 and then checked against the exact squares of the two
// neighbouring midpoints (a midpoint of adjacent floats has at most 26
// significant bits, so its square is exact in fp64).
SHARQ_DEV float sqrt_rn(float v) {
  if (!(v > 0.0f) || v == __builtin_inff()) return __builtin_sqrtf(v);
  const float s = (float)__builtin_sqrt((double)v);
  const uint32_t b = __float_as_uint(s);
  const float up = __uint_as_float(b + 1u), dn = __uint_as_float(b - 1u);
  const double hi = 0.5 * ((double)s + (double)up), lo = 0.5 * ((double)s + (double)dn);
  const double dv = (double)v;
  if (hi * hi < dv) return up;
  if (lo * lo > dv) return dn;
  return s;
}

// ---------------------------------------------------------------- cross-lane
SHARQ_DEV float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }
SHARQ_DEV uint32_t shfl_xor_u(uint32_t v, int m) { return (uint32_t)__shfl_xor((int)v, m, kWave); }

// DPP lane moves inside a row of 16 lanes (every lane reads a valid lane)
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i of 8 <- lane 7 - i
constexpr int kDppRowMirror = 0x140;    // lane i of 16 <- lane 15 - i
template <int CTRL>
SHARQ_DEV uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
SHARQ_DEV float dpp_f(float v) { return __uint_as_float(dpp_u<CTRL>(__float_as_uint(v))); }

// this lane's bit of a wave lane mask
SHARQ_DEV bool lane_in(uint64_t mask) { return __builtin_amdgcn_inverse_ballot_w64(mask); }

// max over the 4 lanes of a quad, in every lane
SHARQ_DEV float quad_max(float v) {
  v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
  return fmaxf(v, dpp_f<kDppQuadXor2>(v));
}

// Sum over the 64 lanes as a pairwise tree of aligned lane blocks (1+1, 2+2,
// ... 32+32), the same value in every lane.  Each level adds the partner
// block's sum; within a level every lane of a block holds the same value, so
// the mirror moves pair whole blocks like an xor would.
SHARQ_DEV float wave_tree_sum(float v) {
  v = __fadd_rn(v, dpp_f<kDppQuadXor1>(v));
  v = __fadd_rn(v, dpp_f<kDppQuadXor2>(v));
  v = __fadd_rn(v, dpp_f<kDppHalfMirror>(v));
  v = __fadd_rn(v, dpp_f<kDppRowMirror>(v));
  // rows 0+1 and 2+3: permlane16_swap of v with itself yields (r0 r0 r2 r2)
  // and (r1 r1 r3 r3)
  const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __fadd_rn(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
  // halves: (lo lo) and (hi hi)
  const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __fadd_rn(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
}

// E8M0 code (e + 127) of the smallest e in [-127, 127] with amax <= 6 * 2^e:
// with amax = 1.m * 2^(E-127), the carry of m + (0.5 - ulp) adds one exactly
// when m > 0.5, so (bits + 0x3FFFFF) >> 23 = E + [m > 0.5] = e + 129.
SHARQ_DEV uint32_t e8m0_code(float amax) {
  const uint32_t t = (__float_as_uint(amax) + 0x3FFFFFu) >> 23;
  return (t > 2u ? t : 2u) - 2u;
}

// 4:8 in-pairs top-2 of four pair scores, ties to the lower pair: returns the
// kept-pair bit mask (exactly two bits).  Pair p beats pair q (p < q) when
// s_p >= s_q; a pair is kept when fewer than two pairs beat it.
SHARQ_DEV uint32_t top2_pairs(float s0, float s1, float s2, float s3) {
  const uint32_t c01 = s0 >= s1, c02 = s0 >= s2, c03 = s0 >= s3;
  const uint32_t c12 = s1 >= s2, c13 = s1 >= s3, c23 = s2 >= s3;
  const uint32_t r0 = 3u - c01 - c02 - c03;           // pairs beating pair 0
  const uint32_t r1 = c01 + 2u - c12 - c13;
  const uint32_t r2 = c02 + c12 + 1u - c23;
  const uint32_t r3 = c03 + c13 + c23;
  return (r0 < 2u) | ((r1 < 2u) << 1) | ((r2 < 2u) << 2) | ((r3 < 2u) << 3);
}

// kept mask (bits) -> metadata nibble i0 | i1 << 2 (i0 < i1)
SHARQ_DEV uint32_t mask_to_nibble(uint32_t km) {
  // km: 3->(0,1)=4, 5->(0,2)=8, 6->(1,2)=9, 9->(0,3)=12, 10->(1,3)=13, 12->(2,3)=14
  const uint64_t lut = (4ull << 12) | (8ull << 20) | (9ull << 24) | (12ull << 36) | (13ull << 40) |
                       (14ull << 48);
  return (uint32_t)(lut >> (4u * km)) & 15u;
}

// Kept pairs of every lane's group from its four pair scores (pair p beats
// pair q > p when s_p >= s_q; a pair is kept when at most one pair beats it,
// i.e. when it beats at least two of the other three).  The comparisons are
// taken as wave lane masks so that the majority logic runs on the scalar
// unit; k[p] is the lane mask of "pair p kept", i0 < i1 the kept indices.
SHARQ_DEV void top2_lanes(float s0, float s1, float s2, float s3, uint64_t k[4], uint32_t& i0, uint32_t& i1) {
  const uint64_t c01 = __builtin_amdgcn_ballot_w64(s0 >= s1), c02 = __builtin_amdgcn_ballot_w64(s0 >= s2);
  const uint64_t c03 = __builtin_amdgcn_ballot_w64(s0 >= s3), c12 = __builtin_amdgcn_ballot_w64(s1 >= s2);
  const uint64_t c13 = __builtin_amdgcn_ballot_w64(s1 >= s3), c23 = __builtin_amdgcn_ballot_w64(s2 >= s3);
  // majority of three: (a & b) | (c & (a | b))
  k[0] = (c01 & c02) | (c03 & (c01 | c02));
  k[1] = (~c01 & c12) | (c13 & (~c01 | c12));
  k[2] = (~c02 & ~c12) | (c23 & (~c02 | ~c12));
  k[3] = (~c03 & ~c13) | (~c23 & (~c03 | ~c13));
  i0 = lane_in(k[0]) ? 0u : (lane_in(k[1]) ? 1u : 2u);
  i1 = lane_in(k[3]) ? 3u : (lane_in(k[2]) ? 2u : 1u);
}

// Expand the two kept pair-bytes of one group (byte0, byte1 of `two`) into the
// four pair slots given by the metadata nibble (zeros in dropped pairs).
SHARQ_DEV uint32_t expand_group(uint32_t two, uint32_t nib) {
  const uint32_t i0 = nib & 3u, i1 = nib >> 2;
  return ((two & 0xFFu) << (8u * i0)) | (((two >> 8) & 0xFFu) << (8u * i1));
}

// activation row of output row r: row_index[r] clamped into [0, act_rows), or r
// Tile of workgroup b among n (b < n).  Workgroups reach the 8 XCDs round
// robin, so XCD x = b % 8 gets the contiguous stretch x q + min(x, r) ..
// of the tile order (q, r = n / 8, n % 8), in dispatch order: the tiles that
// run together on one XCD share operands through its L2.  A bijection on
// [0, n) for every n.
SHARQ_DEV int xcd_tile(int b, int n) {
  const int q = n >> 3, r = n & 7, x = b & 7;
  return x * q + min(x, r) + (b >> 3);
}

SHARQ_DEV int64_t gather_row(const int32_t* row_index, int r, int act_rows) {
  if (!row_index) return r;
  const int v = row_index[r];
  return v < 0 ? 0 : (v >= act_rows ? act_rows - 1 : v);
}

}  // namespace sharq
