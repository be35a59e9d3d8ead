// Dual-path GEMM for emulated NVFP4 (xllm-io paper review §3.1 two-level
// NVFP4 scaling, §3.4-§3.5 dual path with one shared weight payload).
//
// gfx950's scaled MFMA takes only power-of-two (E8M0) block scales, so an
// E4M3 block scale cannot ride along.  An E2M1 value (2 significant bits)
// times an E4M3 scale (4 significant bits) has at most 6 significant bits and
// lies in [2^-10, 2688] when nonzero, so it is exact in fp16.  Each operand
// element is therefore dequantized to q * dec(scale) in fp16 while staging
// (one packed fp16 multiply per two values) and multiplied on the fp16 MFMA
// (v_mfma_f32_32x32x16_f16: exact products, fp32 accumulation).
// (v_cvt_scalef32_pk_bf16_fp4 cannot apply the whole scale: it uses only its
// scale's power-of-two part, measured on MI355X; the conversions here take
// scale 1.)
// The fp32 tensor scales differ between the paths, so the backbone and the
// residual keep one accumulator each inside the same tile and the epilogue
// forms Y = s_w * (s_sp * acc_sp + s_dn * acc_dn).
#include "common.h"
#include "kernels.h"
#include <type_traits>

namespace sharq {

namespace {

typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kNM = 128;                  // tile rows
constexpr int kNN = 256;                  // staged weight columns (the tile computes 256 or 224)
constexpr int kKS = 64;                   // K per step: two halves of 32 (one backbone block, two residual blocks each)

// 32x32x16 f16: lane l holds row / column (l & 31), K-values 8 (l >> 5) .. +7
// of the 16; result register i of lane l is row 8 (i / 4) + 4 (l >> 5) + i % 4,
// column l & 31
SHARQ_DEV v16f mfma_f16(uint4 a, uint4 b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
}

// dec(E4M3 code) as a pair of fp16 (exact: every E4M3 value is an fp16 normal)
SHARQ_DEV v2h dec_h2(uint32_t code) {
  const _Float16 d = (_Float16)e4m3_decode(code);
  return (v2h){d, d};
}

// 8 E2M1 codes (one 32-bit word) times dec -> 8 fp16 (exact, see above)
SHARQ_DEV uint4 dequant8_f16(uint32_t word, v2h dec) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0) * dec;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1) * dec;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2) * dec;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3) * dec;
  return make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                    __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
}

// 16-byte chunk q (0..7, 8 fp16) of a staged 128-byte row.  A 16-byte LDS
// access is served 16 lanes at a time over 256 bytes of banks.  Sixteen
// consecutive rows (from a multiple of 16) at one chunk land on 2 (row & 1) x
// 8 (q ^ ((row >> 1) & 7)) distinct 16-byte bank groups, and so do the
// staging writes (8 rows x the two halves' chunks 4 h + i), so reads and
// writes are conflict-free
SHARQ_DEV int nslot(int row, int q) { return row * 8 + (q ^ ((row >> 1) & 7)); }

struct NvStage {
  uint4 a_sp[kNM * 8];        // backbone, fp16, 128 B per row
  uint4 a_dn[kNM * 8];        // residual
  uint4 b[kNN * 8];           // weight columns
};                            // 64 KB; two stages

// expand 4 groups (8 compacted bytes + 4 metadata nibbles) into 16 code bytes
SHARQ_DEV uint4 expand4(uint32_t c_lo, uint32_t c_hi, uint32_t meta16) {
  const uint32_t m0 = (meta16 & 0x3333u) << 3, m1 = (meta16 & 0xCCCCu) << 1;
  uint4 r;
  r.x = ((c_lo & 0xFFu) << (m0 & 0x18u)) | (((c_lo >> 8) & 0xFFu) << (m1 & 0x18u));
  r.y = (((c_lo >> 16) & 0xFFu) << ((m0 >> 4) & 0x18u)) | ((c_lo >> 24) << ((m1 >> 4) & 0x18u));
  r.z = ((c_hi & 0xFFu) << ((m0 >> 8) & 0x18u)) | (((c_hi >> 8) & 0xFFu) << ((m1 >> 8) & 0x18u));
  r.w = (((c_hi >> 16) & 0xFFu) << ((m0 >> 12) & 0x18u)) | ((c_hi >> 24) << ((m1 >> 12) & 0x18u));
  return r;
}

}  // namespace

// Tile 128 x 256 (or 224 columns), eight waves (two per SIMD): wave w covers
// rows 32 (w & 3) .. and columns 128 (w >> 2) .., with one accumulator per
// path (the two paths have different tensor scales), 128 accumulator
// registers.  K advances 64 per step.  (The activation side costs most of the
// staging work and is staged once per column tile, so the wider tile stages
// it half as often as 256 x 128 did.)  BNE = 224: waves 4-7 compute three
// 32-column accumulators per path instead of four and wave 7 stages no
// weight columns (its 32 are past the tile), so a shape whose 256-wide tiles
// fall short of a whole round over the CUs fills it instead (18944 x 3584 at
// T = 2048: 224 tiles of 256 columns, 256 of 224).
//
// Staging (no DMA: operands are dequantized on the way).  A step's row of 64
// values is split in two halves of 32 (one backbone scale block, two
// residual ones); thread t stages half t & 1 of weight column t >> 1, and
// threads 256 and up also of tile row (t >> 1) - 128 (waves 4-7, one on each SIMD),
// so the two lanes of a row read adjacent bytes and one load instruction
// covers 32 rows.  Per step a thread
// loads its halves (raw buffer loads; rows and columns outside the tile read
// row 0, whose products reach only outputs that are never stored),
// dequantizes them to fp16 and writes 16-byte chunks to LDS.  Loads run two
// steps ahead.  The two waves of a SIMD overlap one's staging with the
// other's MFMAs (measured faster than interleaving them by schedule hints).
template <int BNE>
__global__ __launch_bounds__(512, 1) void linear_nv_tile(
    const uint8_t* __restrict__ bb_codes, const uint8_t* __restrict__ bb_meta, const uint8_t* __restrict__ bb_scale,
    const uint8_t* __restrict__ res_codes, const uint8_t* __restrict__ res_scale, const float* __restrict__ a_ts,
    const int32_t* __restrict__ row_index, int rows, int act_rows, int K, const uint8_t* __restrict__ payload,
    const uint8_t* __restrict__ wscale, const float* __restrict__ w_ts, int D, float* __restrict__ Y, int64_t ldy) {
  __shared__ NvStage st[2];
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  static_assert(BNE == 256 || BNE == 224, "tile columns");
  const int tiles_m = (rows + kNM - 1) / kNM, tiles_n = (D + BNE - 1) / BNE;
  const int nt = tiles_m * tiles_n;
  const int bi = xcd_tile(blockIdx.x, nt);                    // consecutive tiles on one XCD
  const int m0 = (bi % tiles_m) * kNM, n0 = (bi / tiles_m) * BNE;
  const int KS = K / kKS;
  const uint32_t kA = K >> 2, kM = K >> 4, kS32 = K >> 5, kS16 = K >> 4, kR = K >> 1;

  auto rsrc = [](const uint8_t* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0,
                                             __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
  };
  const int an = __builtin_amdgcn_readfirstlane(act_rows);
  const __amdgpu_buffer_rsrc_t r_bc = rsrc(bb_codes, (int64_t)an * kA), r_bm = rsrc(bb_meta, (int64_t)an * kM);
  const __amdgpu_buffer_rsrc_t r_bs = rsrc(bb_scale, (int64_t)an * kS32), r_rc = rsrc(res_codes, (int64_t)an * kR);
  const __amdgpu_buffer_rsrc_t r_rs = rsrc(res_scale, (int64_t)an * kS16);
  const __amdgpu_buffer_rsrc_t r_w = rsrc(payload, (int64_t)D * kR), r_ws = rsrc(wscale, (int64_t)D * kS32);

  // ---- staging roles: half h of column scol and (waves 4-7) of row srow
  const uint32_t h = tid & 1;
  // activations: waves 4-7 (one on each SIMD), which at BNE = 224 also
  // multiply the narrower half of the columns, so the waves that stage the
  // most do the fewest MFMAs
  const bool a_role = w >= 4;                          // uniform per wave
  // weight columns past the tile's BNE (wave 7 at BNE = 224) are never read
  const bool b_role = BNE == 256 || 64 * w < 2 * BNE;  // uniform per wave
  const int srow = (tid >> 1) & 127, scol = tid >> 1;
  const int gr = m0 + srow, gc = n0 + scol;
  const uint32_t ar = gr < rows ? (uint32_t)gather_row(row_index, gr, act_rows) : 0u;
  const uint32_t wc = gc < D ? (uint32_t)gc : 0u;

  struct Ld {
    uint2 bc;            // backbone: compacted codes of the half's 4 groups
    uint32_t bm, bsc;    // backbone metadata (16 bits), scale byte
    uint4 rc;            // residual codes (16 B)
    uint32_t rsc;        // residual: two scale bytes
    uint4 wcd;           // weight codes (16 B)
    uint32_t wsc;        // weight scale byte
  };
  auto load = [&](int s, Ld& L) {
    const uint32_t ss = (uint32_t)min(s, KS - 1);      // past the end: reload the last step (unused)
    if (a_role) {
      const auto c = __builtin_amdgcn_raw_buffer_load_b64(r_bc, ar * kA + 16u * ss + 8u * h, 0, 0);
      L.bc = make_uint2(c[0], c[1]);
      L.bm = __builtin_amdgcn_raw_buffer_load_b16(r_bm, ar * kM + 4u * ss + 2u * h, 0, 0);
      L.bsc = __builtin_amdgcn_raw_buffer_load_b8(r_bs, ar * kS32 + 2u * ss + h, 0, 0);
      const auto r = __builtin_amdgcn_raw_buffer_load_b128(r_rc, ar * kR + 32u * ss + 16u * h, 0, 0);
      L.rc = make_uint4(r[0], r[1], r[2], r[3]);
      L.rsc = __builtin_amdgcn_raw_buffer_load_b16(r_rs, ar * kS16 + 4u * ss + 2u * h, 0, 0);
    }
    if (b_role) {
      const auto b = __builtin_amdgcn_raw_buffer_load_b128(r_w, wc * kR + 32u * ss + 16u * h, 0, 0);
      L.wcd = make_uint4(b[0], b[1], b[2], b[3]);
      L.wsc = __builtin_amdgcn_raw_buffer_load_b8(r_ws, wc * kS32 + 2u * ss + h, 0, 0);
    }
  };
  auto store = [&](const Ld& L, NvStage& S) {
    const int q0 = 4 * (int)h;                         // the half's first 16-byte chunk
    if (a_role) {
      const uint4 e = expand4(L.bc.x, L.bc.y, L.bm);
      const v2h dec = dec_h2(L.bsc & 0xFFu);
      S.a_sp[nslot(srow, q0 + 0)] = dequant8_f16(e.x, dec);
      S.a_sp[nslot(srow, q0 + 1)] = dequant8_f16(e.y, dec);
      S.a_sp[nslot(srow, q0 + 2)] = dequant8_f16(e.z, dec);
      S.a_sp[nslot(srow, q0 + 3)] = dequant8_f16(e.w, dec);
      const v2h d0 = dec_h2(L.rsc & 0xFFu), d1 = dec_h2((L.rsc >> 8) & 0xFFu);
      S.a_dn[nslot(srow, q0 + 0)] = dequant8_f16(L.rc.x, d0);
      S.a_dn[nslot(srow, q0 + 1)] = dequant8_f16(L.rc.y, d0);
      S.a_dn[nslot(srow, q0 + 2)] = dequant8_f16(L.rc.z, d1);
      S.a_dn[nslot(srow, q0 + 3)] = dequant8_f16(L.rc.w, d1);
    }
    if (b_role) {
      const v2h db = dec_h2(L.wsc & 0xFFu);
      S.b[nslot(scol, q0 + 0)] = dequant8_f16(L.wcd.x, db);
      S.b[nslot(scol, q0 + 1)] = dequant8_f16(L.wcd.y, db);
      S.b[nslot(scol, q0 + 2)] = dequant8_f16(L.wcd.z, db);
      S.b[nslot(scol, q0 + 3)] = dequant8_f16(L.wcd.w, db);
    }
  };

  // ---- MFMA fragments and accumulators: rows wm0 + lr, columns wn0 + 32 n +
  // lr for n < FN (FN = 4, or 3 for waves 4-7 of a 224-column tile); the two
  // forms run the same loop, so every wave takes the same barriers
  const int wm0 = (w & 3) * 32, wn0 = (w >> 2) * 128;
  const int kh = l >> 5, lr = l & 31;
  auto run = [&](auto fnc) {
    constexpr int FN = decltype(fnc)::value;
    v16f acc_sp[FN], acc_dn[FN];
#pragma unroll
    for (int n = 0; n < FN; ++n) {
      acc_sp[n] = (v16f){};
      acc_dn[n] = (v16f){};
    }
    struct Frag {
      uint4 sp, dn, b[FN];   // one 16-wide K slice
    };
    auto read = [&](const NvStage& S, int ks, Frag& F) {
      const int q = 2 * ks + kh;                       // chunk: K-values 8 q .. 8 q + 7
      F.sp = S.a_sp[nslot(wm0 + lr, q)];
      F.dn = S.a_dn[nslot(wm0 + lr, q)];
#pragma unroll
      for (int n = 0; n < FN; ++n) F.b[n] = S.b[nslot(wn0 + 32 * n + lr, q)];
    };
    auto mfma = [&](const Frag& F) {
#pragma unroll
      for (int n = 0; n < FN; ++n) {
        acc_sp[n] = mfma_f16(F.sp, F.b[n], acc_sp[n]);
        acc_dn[n] = mfma_f16(F.dn, F.b[n], acc_dn[n]);
      }
    };
    auto step = [&](const NvStage& S, const Ld& Lnext, NvStage& N) {
      Frag fr[2];
      read(S, 0, fr[0]);
      store(Lnext, N);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (ks + 1 < 4) read(S, ks + 1, fr[(ks + 1) & 1]);
        mfma(fr[ks & 1]);
      }
    };

    Ld l0, l1;
    load(0, l0);
    load(1, l1);
    store(l0, st[0]);
    __syncthreads();
    // K % 128 == 0 (checked by the caller), so the number of steps is even
    for (int s = 0; s < KS; s += 2) {
      // step s: st[0] holds step s, st[1] receives step s+1
      load(s + 2, l0);
      step(st[0], l1, st[1]);
      __syncthreads();
      // step s+1
      load(s + 3, l1);
      step(st[1], l0, st[0]);
      __syncthreads();
    }

    // ---- epilogue: Y = s_w * (s_sp * acc_sp + s_dn * acc_dn)
    const float s_sp = a_ts[0], s_dn = a_ts[1], s_w = w_ts[0];
#pragma unroll
    for (int n = 0; n < FN; ++n) {
      const int c = n0 + wn0 + 32 * n + lr;
      if (c >= D) continue;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = m0 + wm0 + 8 * (i >> 2) + 4 * kh + (i & 3);
        if (r < rows) Y[(int64_t)r * ldy + c] = s_w * (s_sp * acc_sp[n][i] + s_dn * acc_dn[n][i]);
      }
    }
  };
  if (BNE == 256 || w < 4) run(std::integral_constant<int, 4>{});
  else run(std::integral_constant<int, (BNE - 128) / 32>{});
}

hipError_t launch_linear_nv(const uint8_t* bb_codes, const uint8_t* bb_meta, const uint8_t* bb_scale,
                            const uint8_t* res_codes, const uint8_t* res_scale, const float* a_ts,
                            const int32_t* row_index, int rows, int act_rows, int K, const uint8_t* payload,
                            const uint8_t* wscale, const float* w_ts, int D, float* Y, int64_t ldy, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  // tile width 256 or 224: the one with fewer rounds x width over the CUs
  // (one workgroup per CU: 128 KB of LDS)
  int ncu = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess || ncu <= 0)
    ncu = 256;
  const int tiles_m = (rows + kNM - 1) / kNM;
  const int t256 = tiles_m * ((D + 255) / 256), t224 = tiles_m * ((D + 223) / 224);
  const bool narrow = (int64_t)((t224 + ncu - 1) / ncu) * 224 < (int64_t)((t256 + ncu - 1) / ncu) * 256;
  if (narrow)
    hipLaunchKernelGGL(linear_nv_tile<224>, dim3(t224), dim3(512), 0, s, bb_codes, bb_meta, bb_scale, res_codes,
                       res_scale, a_ts, row_index, rows, act_rows, K, payload, wscale, w_ts, D, Y, ldy);
  else
    hipLaunchKernelGGL(linear_nv_tile<256>, dim3(t256), dim3(512), 0, s, bb_codes, bb_meta, bb_scale, res_codes,
                       res_scale, a_ts, row_index, rows, act_rows, K, payload, wscale, w_ts, D, Y, ldy);
  return hipGetLastError();
}

}  // namespace sharq
