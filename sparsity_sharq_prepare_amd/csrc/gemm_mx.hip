// Dual-path MXFP4 GEMM of SharQ (xllm-io paper review §3.4-§3.5):
//   Y^ = GEMM_sp(Q_sp(X_sp), Q_w,sp(W)) + GEMM_dn(Q_dn(R), Q_w,dn(W))
// Both paths read the same FP4 weight payload and scale view and accumulate
// into ONE fp32 accumulator per output tile, so no second output is ever
// materialized.  gfx950 offers no sparse MFMA that accepts FP4 operands, so
// the 4:8 in-pairs backbone is expanded (zeros in the dropped pairs) and runs
// through the same dense scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4,
// FP4 x FP4, one E8M0 scale per 32 K-values per row and per column).
//
// MFMA operand layout (16x16x128, FP4): lane l holds row (l & 15) of A and
// column (l & 15) of B for K-values 32 * (l >> 4) .. +31 (16 bytes, even K in
// the low nibble), with that 32-block's scale byte; the result lane l holds
// column (l & 15), rows 4 * (l >> 4) .. +3.
//
// Two kernels:
//  - skinny (decode, T <= 64): weight streaming.  A 16-row MFMA tile holds the
//    backbone of 8 tokens in rows 0-7 and their residual in rows 8-15, so one
//    MFMA applies a weight fragment to both paths; the epilogue adds row r and
//    row r + 8 of the tile.  K is split over the waves of a workgroup and the
//    partial tiles are summed in a fixed order through LDS.
//  - tile (prefill and grouped MoE): 256-column tiles, 256 (or 128) rows, K
//    steps of 128 staged through double-buffered LDS; the backbone is expanded
//    from its compacted bytes while staging.
#include "common.h"
#include "kernels.h"
#include "prep_device.h"
#include <algorithm>
#include <type_traits>

namespace sharq {

namespace {

SHARQ_DEV v8i as_v8i(uint4 v) {
  v8i r = {(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  return r;
}

SHARQ_DEV v4f mfma_fp4(uint4 a, uint4 b, v4f c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(as_v8i(a), as_v8i(b), c, 4, 4, 0, (int)sa, 0, (int)sb);
}

typedef float v16f __attribute__((ext_vector_type(16)));

// 32x32x64 FP4 x FP4 (on gfx950 about 2.5x the throughput of the 16x16x128
// form): lane l holds row / column (l & 31), K-values 32 * (l >> 5) .. +31;
// result register i of lane l is row 8 (i / 4) + 4 (l >> 5) + i % 4, column l & 31.
SHARQ_DEV v16f mfma32_fp4(uint4 a, uint4 b, v16f c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(as_v8i(a), as_v8i(b), c, 4, 4, 0, (int)sa, 0, (int)sb);
}

// expand 4 groups (8 compacted bytes + 4 metadata nibbles) into 16 bytes
SHARQ_DEV uint4 expand4(uint32_t c_lo, uint32_t c_hi, uint32_t meta16) {
  uint4 r;
  r.x = expand_group(c_lo & 0xFFFFu, meta16 & 15u);
  r.y = expand_group(c_lo >> 16, (meta16 >> 4) & 15u);
  r.z = expand_group(c_hi & 0xFFFFu, (meta16 >> 8) & 15u);
  r.w = expand_group(c_hi >> 16, (meta16 >> 12) & 15u);
  return r;
}

// 4 groups (8 compacted bytes c_lo, c_hi + 4 nibbles of meta16) -> 16 bytes.
// Moving i0 / i1 of every nibble to bits 3-4 of its nibble makes
// (m >> 4g) & 0x18 the byte shift 8 * i of group g.
SHARQ_DEV uint4 expand4_fast(uint32_t c_lo, uint32_t c_hi, uint32_t meta16) {
  const uint32_t m0 = (meta16 & 0x3333u) << 3;        // 8 * i0 at bits 4g + 3 .. 4g + 4
  const uint32_t m1 = (meta16 & 0xCCCCu) << 1;        // 8 * i1
  uint4 r;
  r.x = ((c_lo & 0xFFu) << (m0 & 0x18u)) | (((c_lo >> 8) & 0xFFu) << (m1 & 0x18u));
  r.y = (((c_lo >> 16) & 0xFFu) << ((m0 >> 4) & 0x18u)) | ((c_lo >> 24) << ((m1 >> 4) & 0x18u));
  r.z = ((c_hi & 0xFFu) << ((m0 >> 8) & 0x18u)) | (((c_hi >> 8) & 0xFFu) << ((m1 >> 8) & 0x18u));
  r.w = (((c_hi >> 16) & 0xFFu) << ((m0 >> 12) & 0x18u)) | ((c_hi >> 24) << ((m1 >> 12) & 0x18u));
  return r;
}

// 2:4 backbone: one 32-value block (8 groups of 4) from its 8 compacted bytes
// (c_lo, c_hi: the kept codes of group g in byte g, lower index in the low
// nibble) and its 8 metadata nibbles m32 (i0 | i1 << 2) -> 16 bytes, the kept
// codes at nibbles 4 g + i0 and 4 g + i1, zeros elsewhere
SHARQ_DEV uint32_t expand_24_pair(uint32_t b2, uint32_t m8) {
  // two groups: kept bytes b2 (bits 0-15), nibbles m8 (bits 0-7) -> 32 bits
  const uint32_t lo = ((b2 & 15u) << (4u * (m8 & 3u))) | (((b2 >> 4) & 15u) << (4u * ((m8 >> 2) & 3u)));
  const uint32_t hi = (((b2 >> 8) & 15u) << (4u * ((m8 >> 4) & 3u))) | (((b2 >> 12) & 15u) << (4u * ((m8 >> 6) & 3u)));
  return lo | (hi << 16);
}
SHARQ_DEV uint4 expand_24(uint32_t c_lo, uint32_t c_hi, uint32_t m32) {
  uint4 r;
  r.x = expand_24_pair(c_lo & 0xFFFFu, m32 & 0xFFu);
  r.y = expand_24_pair(c_lo >> 16, (m32 >> 8) & 0xFFu);
  r.z = expand_24_pair(c_hi & 0xFFFFu, (m32 >> 16) & 0xFFu);
  r.w = expand_24_pair(c_hi >> 16, m32 >> 24);
  return r;
}

}  // namespace

// ============================================================================
// skinny (decode) kernel
// ============================================================================
// grid.x = ceil(D / 16); blockDim = 64 * NW.  Wave w takes K-steps
// w, w + NW, ... in batches of J whose loads are all issued before the MFMAs.
template <int MT, int J, bool M24 = false>
__global__ __launch_bounds__(MT >= 8 ? 512 : 1024) void linear_mx_skinny(
    const uint8_t* __restrict__ bb_codes, const uint8_t* __restrict__ bb_meta, const uint8_t* __restrict__ bb_scale,
    const uint8_t* __restrict__ res_codes, const uint8_t* __restrict__ res_scale, const int32_t* __restrict__ row_index,
    int rows, int act_rows, int K, const uint8_t* __restrict__ payload, const uint8_t* __restrict__ wscale, int D,
    float* __restrict__ Y, int64_t ldy) {
  extern __shared__ float red[];                       // [NW][MT][64][4]
  const int NW = blockDim.x >> 6;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int KS = K >> 7;
  const int col = blockIdx.x * 16 + (l & 15);
  const bool col_ok = col < D;
  const int kq = l >> 4;
  const bool dn = (l & 8) != 0;                        // rows 8-15 of the MFMA tile: residual path
  int64_t arow[MT];
  bool aok[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int tok = 8 * m + (l & 7);
    aok[m] = tok < rows;
    arow[m] = aok[m] ? gather_row(row_index, tok, act_rows) : 0;
  }
  const int64_t wrow = (int64_t)(col_ok ? col : 0);
  v4f acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = (v4f){0.f, 0.f, 0.f, 0.f};

  for (int s0 = w; s0 < KS; s0 += NW * J) {
    uint4 wv[J];
    uint32_t ws[J];
    uint4 av[MT][J];
    uint32_t as[MT][J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int s = s0 + NW * j;
      const bool sv = s < KS;
      const int kb = 4 * s + kq;                       // 32-block index of this lane
      wv[j] = make_uint4(0, 0, 0, 0);
      ws[j] = 127;
      if (sv && col_ok) {
        wv[j] = *reinterpret_cast<const uint4*>(payload + wrow * (K >> 1) + 16 * (int64_t)kb);
        ws[j] = wscale[wrow * (K >> 5) + kb];
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        av[m][j] = make_uint4(0, 0, 0, 0);
        as[m][j] = 127;
        if (sv && aok[m]) {
          if (dn) {
            av[m][j] = *reinterpret_cast<const uint4*>(res_codes + arow[m] * (K >> 1) + 16 * (int64_t)kb);
            as[m][j] = res_scale[arow[m] * (K >> 5) + kb];
          } else {
            const uint2 c = *reinterpret_cast<const uint2*>(bb_codes + arow[m] * (K >> 2) + 8 * (int64_t)kb);
            av[m][j].x = c.x;
            av[m][j].y = c.y;
            if (M24) av[m][j].z = *reinterpret_cast<const uint32_t*>(bb_meta + arow[m] * (K >> 3) + 4 * (int64_t)kb);
            else av[m][j].z = *reinterpret_cast<const uint16_t*>(bb_meta + arow[m] * (K >> 4) + 2 * (int64_t)kb);
            as[m][j] = bb_scale[arow[m] * (K >> 5) + kb];
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        uint4 a = av[m][j];
        if (!dn) a = M24 ? expand_24(a.x, a.y, a.z) : expand4(a.x, a.y, a.z);
        acc[m] = mfma_fp4(a, wv[j], acc[m], as[m][j], ws[j]);
      }
    }
  }
  // fixed-order reduction over the waves, then backbone row + residual row
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    float* p = red + ((w * MT + m) * 64 + l) * 4;
    p[0] = acc[m][0]; p[1] = acc[m][1]; p[2] = acc[m][2]; p[3] = acc[m][3];
  }
  __syncthreads();
  if (w == 0 && l < 32) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float sp = 0.0f, dv = 0.0f;
        for (int ww = 0; ww < NW; ++ww) {
          sp += red[((ww * MT + m) * 64 + l) * 4 + i];
          dv += red[((ww * MT + m) * 64 + l + 32) * 4 + i];
        }
        const int tok = 8 * m + 4 * (l >> 4) + i;
        if (tok < rows && col_ok) Y[(int64_t)tok * ldy + col] = sp + dv;
      }
    }
  }
}

// ============================================================================
// decode kernel (at most 8 activation rows)
// ============================================================================
// One 16x16x128 MFMA per 128-wide K-step: MFMA rows 0-7 are the backbone of
// tokens 0-7, rows 8-15 their residual, so one accumulator holds both paths
// and the epilogue adds row t and row t + 8.
//
// The workgroup stages the activation side in LDS: for 32-block kb and MFMA
// row r the 16 code bytes (backbone expanded from its compacted pairs) sit in
// slot 16 kb + r, the scale in byte 16 kb + r.  Its loads (L2 hits) are
// issued first, then wave w issues the loads of the weight bytes of its J
// consecutive K-steps from J w (lane l: column 16 blockIdx.x + (l & 15),
// 32-block 4 s + (l >> 4)) and of their scales (one 16-byte load per four
// steps); the LDS writes wait only for the earlier activation loads, so the
// weight stream is in flight meanwhile.  All global loads are raw buffer
// loads; absent tokens, columns and steps get an offset past the buffer and
// read zero.
//
// grid.x = ceil(D / 16 CG) (+ rows producer workgroups first when fused),
// 64 NW threads, NW J >= K / 128.
//
// Fused (single-launch decode, rows <= 8): GEMM workgroups 0, 8, .., 8 (rows-1)
// also prepare one activation row each (RowPrep: the standalone prepare's
// outputs, bit for bit): they load the row and gamma, then their weights,
// quantize and store the row with write-through stores, wait until all of it
// is done, and increment sync[0] at memory.  (A release that writes the L2
// back costs microseconds; write-through stores need none.)  Workgroups go to
// the 8 XCDs round robin, so all producers share XCD 0 and its L2.  Every GEMM workgroup issues its weight loads,
// then waits (one lane, bounded polling) until sync[0] reaches rows, and only
// then loads the prepared activations with ordinary loads: on XCD 0 they hit
// the producers' L2, elsewhere the L2 holds no line of these buffers (caches
// are invalidated at kernel start and nothing reads them before the wait), so
// the first read fetches the written-back bytes and later ones hit.  The
// weight stream overlaps the preparation.  Workgroups are dispatched in index
// order on every XCD and the producers come first on XCD 0, so they are
// resident before any waiting workgroup can hold their place.  The last GEMM
// workgroup past the wait resets sync[0] and sync[1] to zero for the next
// call.
constexpr int kDecodeMaxK = 16384;                   // staged operand + reduction fit in LDS
constexpr uint32_t kFusedSpinMax = 1u << 20;         // polls before giving up (the kernel always ends)
constexpr int kAuxWriteThrough = 16;                 // store cache policy sc1: written through to memory

struct FusedPrep {
  const void* X;               // activation rows (bf16 or fp32), row r at X + r * ldx elements
  int bf16;
  int64_t ldx;
  const float* gamma;          // RMSNorm weights or null (no normalization)
  float eps;
  uint32_t* sync;              // [2] counters, zero between calls
};

template <int NK, int CG, int J, bool FUSED, bool M24 = false>
__global__ __launch_bounds__(NK * CG * 64) void linear_mx_decode(
    const uint8_t* bb_codes, const uint8_t* bb_meta, const uint8_t* bb_scale, const uint8_t* res_codes,
    const uint8_t* res_scale, const int32_t* __restrict__ row_index, int rows, int act_rows, int K,
    const uint8_t* __restrict__ payload, const uint8_t* __restrict__ wscale, int D, float* __restrict__ Y, int64_t ldy,
    FusedPrep fp) {
  static_assert(J % 4 == 0, "weight scales load four steps at a time");
  constexpr int NW = NK * CG;                          // K-splits x column groups
  extern __shared__ uint4 dsm[];
  constexpr uint32_t kOut = 0x80000000u;             // offset past every buffer here: reads zero
  constexpr int NT = NW * 64;
  const int KB = K >> 5, KS = K >> 7;
  // scale rows: MFMA row r (0-7 backbone, 8-15 residual of token r & 7) at
  // s_sm + r * KBP; KBP / 4 odd, so the 16 rows of one step's reads fall on
  // distinct banks; a spare 16-byte slot follows them
  const int KBP = ((KB + 15) & ~15) + 4;
  uint4* const a_sm = dsm;                                            // [KB + 1][16]
  uint8_t* const s_sm = reinterpret_cast<uint8_t*>(dsm + (KB + 1) * 16);   // [16][KBP] + 16
  float* const red = reinterpret_cast<float*>(dsm + (KB + 1) * 16 + (16 * KBP + 16) / 16);   // [NW][64][4]
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  auto rsrc = [](const uint8_t* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0,
                                             __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
  };

  const int n_gemm = (D + 16 * CG - 1) / (16 * CG);
  const int bx = blockIdx.x;
  // fused: workgroup bx (bx % 8 == 0) also prepares row bx / 8; its row and
  // gamma loads go out first, ahead of the weight loads (K / (8 NT) <= J / 4
  // groups per thread for every decode geometry)
  constexpr int PMAXC = J / 4 > 0 ? J / 4 : 1;
  RowPrep<NT, PMAXC, kAuxWriteThrough> rp;
  bool producer = false;
  if constexpr (FUSED) {
    producer = (bx & 7) == 0 && (bx >> 3) < rows;   // uniform
    if (producer) rp.load(fp.X, fp.bf16 != 0, K, (int64_t)(bx >> 3) * fp.ldx, fp.gamma);
    else if (bx >= n_gemm) return;                   // padding (the grid covers producer 8 (rows-1))
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- activation loads (L2 hits), as coalesced 16-byte pieces of the
  // token rows: residual piece i = block i % KB of token i / KB; backbone
  // piece i = blocks 2 (i % (KB / 2)) and + 1 of token i / (KB / 2), with
  // its 4 metadata bytes; scale piece i = 16 scale bytes of one row (backbone
  // rows first).  Wide loads keep the address unit's work per byte low (one
  // load per 16 bytes instead of five loads per 32-value block).  Pieces past
  // the end (and of absent tokens) read zeros and land in spare LDS slots.
  // Issued before the weight loads (the LDS writes then wait only for them),
  // except when fused: there the activations exist only once the producers
  // are done.  NK J >= K / 128 gives 8 KB <= NT IPT.
  constexpr int IPT = (J / (2 * CG)) > 0 ? J / (2 * CG) : 1;
  constexpr int BPT = (IPT + 1) / 2;                  // backbone pieces per thread
  const int KBh = KB >> 1, KB16 = (KB + 15) >> 4;
  const int n_res = 8 * KB, n_bb = 8 * KBh, n_sc = 16 * KB16;
  // piece index -> row by a float reciprocal instead of an integer division:
  // (i + 1/2) / n is at least 1 / (2 n) >= 2^-11 away from an integer, far
  // beyond the rounding of these small operands
  const float rKB = 1.0f / (float)KB, rKBh = 1.0f / (float)KBh, rKB16 = 1.0f / (float)KB16;
  auto qdiv = [](int i, float r) { return (int)(((float)i + 0.5f) * r); };
  auto act_row = [&](int t) -> uint32_t {
    return t < rows ? (uint32_t)gather_row(row_index, t, act_rows) : 0u;
  };
  uint4 rv[IPT], bv[BPT], sv[2];
  uint2 mv[BPT];                                      // metadata of the pair of blocks (2:4: 8 bytes)
  auto load_act = [&]() {
    const int an = __builtin_amdgcn_readfirstlane(act_rows);
    const __amdgpu_buffer_rsrc_t r_rc = rsrc(res_codes, (int64_t)an * (K >> 1));
    const __amdgpu_buffer_rsrc_t r_rs = rsrc(res_scale, (int64_t)an * (K >> 5));
    const __amdgpu_buffer_rsrc_t r_bc = rsrc(bb_codes, (int64_t)an * (K >> 2));
    const __amdgpu_buffer_rsrc_t r_bm = rsrc(bb_meta, (int64_t)an * (K >> (M24 ? 3 : 4)));
    const __amdgpu_buffer_rsrc_t r_bs = rsrc(bb_scale, (int64_t)an * (K >> 5));
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int i = tid + NT * j, t = qdiv(i, rKB), kb = i - t * KB;
      const uint32_t off = i < n_res && t < rows ? act_row(t) * (uint32_t)(K >> 1) + 16u * kb : kOut;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(r_rc, off, 0, 0);
      rv[j] = make_uint4(v[0], v[1], v[2], v[3]);
    }
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int i = tid + NT * j, t = qdiv(i, rKBh), kp = i - t * KBh;
      const bool ok = i < n_bb && t < rows;
      const uint32_t ar = ok ? act_row(t) : 0u;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(r_bc, ok ? ar * (uint32_t)(K >> 2) + 16u * kp : kOut, 0, 0);
      bv[j] = make_uint4(v[0], v[1], v[2], v[3]);
      if constexpr (M24) {
        const auto m = __builtin_amdgcn_raw_buffer_load_b64(r_bm, ok ? ar * (uint32_t)(K >> 3) + 8u * kp : kOut, 0, 0);
        mv[j] = make_uint2(m[0], m[1]);
      } else {
        mv[j] = make_uint2(__builtin_amdgcn_raw_buffer_load_b32(r_bm, ok ? ar * (uint32_t)(K >> 4) + 4u * kp : kOut, 0, 0), 0u);
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = tid + NT * j, r = qdiv(i, rKB16), p = i - r * KB16, t = r & 7;
      const bool ok = i < n_sc && t < rows;
      // bytes past a row's K / 32 belong to the next row (or read zero past
      // the buffer); they land in the row's padding
      const uint32_t off = ok ? act_row(t) * (uint32_t)(K >> 5) + 16u * p : kOut;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(r < 8 ? r_bs : r_rs, off, 0, 0);
      sv[j] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  };
  if (!FUSED) load_act();
  __builtin_amdgcn_sched_barrier(0);

  // ---- weight loads of this wave's steps (column group cg, K-split kw)
  const int cg = w % CG, kw = w / CG;
  const int col = (bx * CG + cg) * 16 + (l & 15);
  const int kq = l >> 4;
  const int s0 = kw * J;
  const __amdgpu_buffer_rsrc_t r_w = rsrc(payload, (int64_t)D * (K >> 1));
  const __amdgpu_buffer_rsrc_t r_ws = rsrc(wscale, (int64_t)D * (K >> 5));
  const uint32_t o_w = col < D ? (uint32_t)col * (uint32_t)(K >> 1) + 16u * kq : kOut;
  const uint32_t o_ws = col < D ? (uint32_t)col * (uint32_t)(K >> 5) : kOut;
  uint4 wv[J];
  uint32_t wsd[J];                                    // dword j: scales of step s0 + j (byte kq)
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t out = s0 + j < KS ? 0u : kOut;
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r_w, (o_w + 64u * (uint32_t)(s0 + j)) | out, 0, 0);
    wv[j] = make_uint4(v[0], v[1], v[2], v[3]);
  }
#pragma unroll
  for (int j = 0; j < J; j += 4) {
    // 16 bytes = blocks 4 (s0 + j) .. 4 (s0 + j + 4) - 1; past the row's end
    // only scales of zero-weight steps are affected
    const uint32_t out = s0 + j < KS ? 0u : kOut;
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r_ws, (o_ws + 4u * (uint32_t)(s0 + j)) | out, 0, 0);
    wsd[j] = v[0]; wsd[j + 1] = v[1]; wsd[j + 2] = v[2]; wsd[j + 3] = v[3];
  }
  __builtin_amdgcn_sched_barrier(0);

  if constexpr (FUSED) {
    if (producer) {
      rp.finish(fp.bf16 != 0, K, fp.gamma, fp.eps, bx >> 3, const_cast<uint8_t*>(bb_codes),
                const_cast<uint8_t*>(bb_meta), const_cast<uint8_t*>(bb_scale), const_cast<uint8_t*>(res_codes),
                const_cast<uint8_t*>(res_scale), reinterpret_cast<float*>(dsm));
      // every wave's loads and write-through stores are done (the row is in
      // memory), then the increment, performed at memory (system scope: no
      // L2 write-back is needed, and none is made)
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) __hip_atomic_fetch_add(&fp.sync[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      if (bx >= n_gemm) return;                      // producer only (tiny D)
    }
    if (tid == 0) {
      for (uint32_t it = 0; it < kFusedSpinMax; ++it) {
        if (__hip_atomic_load(&fp.sync[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= (uint32_t)rows) break;
        __builtin_amdgcn_s_sleep(2);
      }
      const uint32_t n = __hip_atomic_fetch_add(&fp.sync[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (n + 1 == (uint32_t)n_gemm) {               // every GEMM workgroup is past the wait
        __hip_atomic_store(&fp.sync[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&fp.sync[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
    load_act();
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- activation operand into LDS (waits only for the activation loads,
  // which were issued first): residual blocks as they are, backbone blocks
  // expanded to operand form, scale rows as they are.  Pieces past the end
  // write the spare block row KB or the spare scale slot, so no load is sunk
  // behind the weight loads into a conditional block.
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const int i = tid + NT * j, t = qdiv(i, rKB), kb = i - t * KB;
    a_sm[i < n_res ? 16 * kb + 8 + t : 16 * KB] = rv[j];
  }
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int i = tid + NT * j, t = qdiv(i, rKBh), kp = i - t * KBh;
    const bool ok = i < n_bb;
    if constexpr (M24) {
      a_sm[ok ? 16 * (2 * kp) + t : 16 * KB + 1] = expand_24(bv[j].x, bv[j].y, mv[j].x);
      a_sm[ok ? 16 * (2 * kp + 1) + t : 16 * KB + 2] = expand_24(bv[j].z, bv[j].w, mv[j].y);
    } else {
      a_sm[ok ? 16 * (2 * kp) + t : 16 * KB + 1] = expand4_fast(bv[j].x, bv[j].y, mv[j].x & 0xFFFFu);
      a_sm[ok ? 16 * (2 * kp + 1) + t : 16 * KB + 2] = expand4_fast(bv[j].z, bv[j].w, mv[j].x >> 16);
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = tid + NT * j, r = qdiv(i, rKB16), p = i - r * KB16;
    // row r of the scale table: backbone token r (r < 8) is MFMA row r,
    // residual token r - 8 is MFMA row r as well
    // (4-byte stores: KBP is a multiple of 4, not of 16)
    uint32_t* dst = reinterpret_cast<uint32_t*>(s_sm + (i < n_sc ? r * KBP + 16 * p : 16 * KBP));
    dst[0] = sv[j].x; dst[1] = sv[j].y; dst[2] = sv[j].z; dst[3] = sv[j].w;
  }
  __syncthreads();

  // ---- MFMAs (steps past K carry zero weights; their LDS slot is clamped)
  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int s = s0 + j < KS ? s0 + j : KS - 1;
    const int e = 64 * s + l;                        // = 16 (4 s + kq) + (l & 15)
    acc = mfma_fp4(a_sm[e], wv[j], acc, s_sm[(l & 15) * KBP + 4 * s + kq], (wsd[j] >> (8 * kq)) & 0xFFu);
  }

  // ---- fixed-order reduction over the waves; backbone row + residual row
  {
    float* p = red + (w * 64 + l) * 4;
    p[0] = acc[0]; p[1] = acc[1]; p[2] = acc[2]; p[3] = acc[3];
  }
  __syncthreads();
  if (kw == 0 && l < 32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float bsum = 0.0f, rsum = 0.0f;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const int ww = kk * CG + cg;
        bsum += red[(ww * 64 + l) * 4 + i];
        rsum += red[(ww * 64 + l + 32) * 4 + i];
      }
      // lane l < 32 holds MFMA rows 4 (l >> 4) + i (backbone of tokens 0-7);
      // lane l + 32 holds rows 8 + 4 (l >> 4) + i (their residual)
      const int t = 4 * (l >> 4) + i;
      if (t < rows && col < D) Y[(int64_t)t * ldy + col] = bsum + rsum;
    }
  }
}

// ============================================================================
// shared pieces of the tile kernel
// ============================================================================
// Staging is buffer->LDS DMA (buffer_load_dwordx4 ... lds) into LDS rings,
// no staging registers; the per-step offset is a scalar and reads past a
// buffer return zeros.  The DMAs are issued from inline assembly: they write
// no registers, and keeping them out of the compiler's sight stops it from
// waiting for every in-flight DMA before each LDS read (it cannot tell the
// ring buffers apart); completion is tracked by explicit vmcnt waits.
//
// K order inside a 128-step: lane half kh handles the 32-value blocks 2 kh
// and 2 kh + 1 (sub-steps j = 0, 1), so its two scale bytes are one 16-bit
// LDS read and the MFMA's op_sel picks byte j.  A, B and both paths use the
// same order, so the sum is unchanged.
namespace {

constexpr int kBN = 256;
constexpr int kNS = 3;                   // LDS ring depth

// 16-byte slot of (row, chunk q) in a 64-byte-per-row staged tile.  gfx950
// serves a 16-byte LDS read 16 lanes at a time over 256 bytes of banks; 16
// consecutive rows at one chunk q fall on 4 (row & 3) x 4 (q ^ swz) distinct
// 16-byte bank groups, so the read is conflict-free (measured: 4 cycles per
// wave, 8 with an XOR of bits 1 and 3, 16 with none)
SHARQ_DEV int swz(int row) { return (row >> 2) & 3; }
SHARQ_DEV int slot(int row, int q) { return row * 4 + (q ^ swz(row)); }
// 16-byte half h of a 32-byte compacted-backbone row
SHARQ_DEV int slot_sp(int row, int h) { return row * 2 + (h ^ ((row >> 3) & 1)); }

typedef int int4v __attribute__((ext_vector_type(4)));

// raw buffer resource (gfx9 layout): base, num_records = bytes, no stride
SHARQ_DEV int4v make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return (int4v){(int)(uint32_t)p, (int)((uint32_t)(p >> 32) & 0xFFFFu), (int)bytes, 0x00020000};
}
SHARQ_DEV uint32_t lds_addr(const void* p) { return (uint32_t)reinterpret_cast<uintptr_t>(p); }
// lane l of the wave writes its 16 bytes at LDS address lds + 16 l
SHARQ_DEV void dma16(int4v rs, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rs), "s"(soff), "{m0}"(lds)
               : "memory");
}

// s_waitcnt vmcnt <= N, lgkmcnt 0 (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt[5:4] at [15:14])
template <int N>
SHARQ_DEV void wait_vm_lgkm0() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}


template <int J>
SHARQ_DEV v16f mfma32_fp4_sel(uint4 a, uint4 b, v16f c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(as_v8i(a), as_v8i(b), c, 4, 4, J, (int)sa, J, (int)sb);
}

}  // namespace

// Grouped tiles: the tiles are the concatenation, over experts in order, of
// each expert's ceil(rows_e / BM) x tiles_n tiles; workgroup bid takes tile
// xcd_tile(bid, total), so each XCD works through one contiguous stretch of
// the tile order and its L2 holds the few experts of that stretch.  Every thread below 256 loads one expert's offsets
// (coalesced), tile counts are prefix-summed across the workgroup in `scan`
// (256 ints of LDS), and the thread whose range holds the tile publishes it
// through `hit` (4 ints of LDS).  Needs at least 256 threads and n_groups >=
// 1; all threads must call it.  Returns false for a surplus workgroup
// (uniform).
SHARQ_DEV bool find_group_tile(int bid, int n_groups, const int32_t* __restrict__ group_offsets, int rows, int BM,
                               int tiles_n, int* scan, int* hit, int& expert, int& start, int& count, int& tile) {
  const int tid = threadIdx.x;
  if (tid == 0) hit[0] = -1;
  // tile counts of experts e0 .. e0 + 255, inclusive prefix sums in scan[]
  auto chunk = [&](int e0, int& st, int& cnt, int& te) {
    const int e = e0 + tid;
    st = 0, cnt = 0, te = 0;
    if (tid < 256 && e < n_groups) {
      st = min(max(group_offsets[e], 0), rows);
      cnt = min(max(group_offsets[e + 1], st), rows) - st;
      te = ((cnt + BM - 1) / BM) * tiles_n;
    }
    if (tid < 256) scan[tid] = te;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {         // inclusive Hillis-Steele scan
      const int v = (tid < 256 && tid >= off) ? scan[tid - off] : 0;
      __syncthreads();
      if (tid < 256) scan[tid] += v;
      __syncthreads();
    }
  };
  // the total tile count first (with one chunk, the locating pass has it)
  int total = 0;
  if (n_groups > 256) {
    for (int e0 = 0; e0 < n_groups; e0 += 256) {      // uniform
      int st, cnt, te;
      chunk(e0, st, cnt, te);
      total += scan[255];
      __syncthreads();
    }
  }
  int t = -1, carry = 0;
  for (int e0 = 0; e0 < n_groups; e0 += 256) {        // uniform
    int st, cnt, te;
    chunk(e0, st, cnt, te);
    if (e0 == 0) {
      if (n_groups <= 256) total = scan[255];
      if (bid < total) t = xcd_tile(bid, total);
    }
    if (tid < 256 && e0 + tid < n_groups) {
      const int incl = carry + scan[tid], excl = incl - te;
      if (t >= excl && t < incl) {
        hit[0] = e0 + tid; hit[1] = st; hit[2] = cnt; hit[3] = t - excl;
      }
    }
    carry += scan[255];
    __syncthreads();
  }
  expert = hit[0];
  start = hit[1];
  count = hit[2];
  tile = hit[3];
  return expert >= 0;
}

// ============================================================================
// tile kernel (more than 64 rows; plain and grouped; K % 128 == 0)
// ============================================================================
// Tile 256 x 256 (or 224 columns), eight waves, two per SIMD covering each
// other's LDS and barrier latency; each wave holds a 128-register
// accumulator.  The layout used is 8 x 1 (wave w: rows 32 w .., all
// columns), so every backbone fragment is expanded by one wave only
// (measured about 5% faster than 4 x 2 with 64 x 128 per wave, despite the
// larger weight-fragment reads).
//
// Operand bytes per row and 128-step (codes: 64 B residual, 32 B backbone,
// 64 B weight) go through a 3-deep LDS ring.  The small per-row data (4 B of
// scales per row and step, 8 B of 4:8 metadata) would cost one cache line per
// 4-8 bytes if fetched per step, so it comes in groups of four steps (16 B of
// scales, 32 B of metadata per row) into a double-buffered side ring,
// fetched two steps before the group starts.  Every wave issues the same
// loads (5 per step, 3 more on the third step of a group), so the explicit
// wait counts are per step of a group: 5, 5, 5, 8.  The 2:4 backbone's
// metadata (16 B per row and step) is staged with each step instead: 6 per
// step, 2 more on the third step of a group.
namespace {

struct Tile8Main {
  uint4 a_dn[256 * 4];         // residual codes, 64 B per row (swizzled 16 B slots)
  uint4 b[256 * 4];            // weight payload, 64 B per column
  uint4 a_sp[256 * 2];         // compacted backbone, 32 B per row
};
struct Tile8Side {             // four steps
  uint4 meta[256 * 2];         // 32 B per row: step p at bytes 8 p .. 8 p + 7
  uint4 s_sp[256];             // 16 B per row: step p at bytes 4 p .. 4 p + 3
  uint4 s_dn[256];
  uint4 s_b[256];
};
// 2:4 backbone: its metadata (16 B per row and step) goes with the step's
// codes, and the side ring keeps the scales only (3 x 44 KB + 2 x 12 KB)
struct Tile8Main24 : Tile8Main {
  uint4 meta[256];             // 16 B per row: the step's four 32-value blocks
};
struct Tile8Side24 {
  uint4 s_sp[256];
  uint4 s_dn[256];
  uint4 s_b[256];
};

}  // namespace

template <int WROWS, int BNE, bool DENSE = false, bool GROUPED = false, bool M24 = false, bool PARTIAL = false>
__global__ __launch_bounds__(512, 1) void linear_mx_tile8(
    const uint8_t* __restrict__ bb_codes, const uint8_t* __restrict__ bb_meta, const uint8_t* __restrict__ bb_scale,
    const uint8_t* __restrict__ res_codes, const uint8_t* __restrict__ res_scale, const int32_t* __restrict__ row_index,
    int rows, int act_rows, int K, const uint8_t* __restrict__ payload, const uint8_t* __restrict__ wscale, int D,
    int n_groups, const int32_t* __restrict__ group_offsets, float* __restrict__ Y, int64_t ldy) {
  // WROWS = 4: waves 4 (rows) x 2 (columns), 64 x 128 each; WROWS = 8: 8 x 1,
  // 32 x 256 each (every backbone fragment expanded by one wave only)
  // BNE: columns the tile computes (256, or 224 so that more shapes give a
  // whole number of rounds over the CUs); staging stays 256 columns wide.
  // DENSE: the plain MXFP4 GEMM of the comparison baseline, one operand
  // (res_codes / res_scale hold plain codes and scales; no backbone)
  // GROUPED: per-expert weights (n_groups of them, group_offsets delimiting
  // each expert's rows), tiles numbered expert by expert
  // M24: the 2:4 element-wise backbone (metadata K/8 bytes per row)
  // PARTIAL: K % 512 != 0, the last side group of four steps is partial
  // (a separate instance keeps the K % 512 == 0 loop free of the check)
  static_assert(BNE == kBN || WROWS == 8, "narrow tiles only with the 8 x 1 layout");
  static_assert(!(GROUPED && DENSE) && !(M24 && DENSE), "the plain baseline has no backbone");
  // DMA instructions per wave: per step (residual, weight, backbone codes;
  // 2:4: and metadata) and per side group (4:8: metadata; activation scales,
  // weight scales)
  constexpr int NMAIN = DENSE ? 4 : (M24 ? 6 : 5), NSIDE = DENSE || M24 ? 2 : 3;
  constexpr int BM = 256, WM = BM / WROWS, WNC = BNE * WROWS / 8, FM = WM / 32, FN = WNC / 32;
  using MainT = std::conditional_t<M24, Tile8Main24, Tile8Main>;
  using SideT = std::conditional_t<M24, Tile8Side24, Tile8Side>;
  __shared__ MainT lds[kNS];
  __shared__ SideT side[2];
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int wq = w & 3;

  // ---- tile -> (first row, first column). Tiles are ordered in bands of
  // kBand row tiles that sweep all column tiles (row fastest inside a band),
  // and each XCD takes one contiguous stretch of that order: the workgroups
  // that run together on one XCD then share a few activation and weight
  // tiles through its L2 instead of all 16 row tiles of the activations
  // (measured at 4096 x 4096 x 14336: 269 -> 243 us)
  const int tiles_n = (D + BNE - 1) / BNE;
  int grp = 0, m0, n0, row_end = rows;
  if constexpr (!GROUPED) {
    const int tiles_m = (rows + BM - 1) / BM;
    const int nt = tiles_m * tiles_n;
    const int bi = xcd_tile(blockIdx.x, nt);
    constexpr int kBand = 4;
    const int band = bi / (kBand * tiles_n), band_m = min(kBand, tiles_m - band * kBand);
    const int in_band = bi - band * kBand * tiles_n;
    m0 = (band * kBand + in_band % band_m) * BM;
    n0 = (in_band / band_m) * BNE;
  } else {
    // the lookup's LDS lives in the third ring stage, which the first DMA
    // reaches only after the main loop's first barrier, when every thread has
    // read the result
    int* scan = reinterpret_cast<int*>(&lds[2].a_dn[0]);
    int e, start, cnt, b;
    if (!find_group_tile(blockIdx.x, n_groups, group_offsets, rows, BM, tiles_n, scan, scan + 256, e, start, cnt, b))
      return;                                           // surplus workgroup (uniform)
    grp = e;
    m0 = start + (b / tiles_n) * BM;
    n0 = (b % tiles_n) * BNE;
    row_end = start + cnt;
  }

  // K % 128 == 0: KS steps of 128, side groups of 4 steps (the last one may
  // be partial; its rows' side bytes past the step count are loaded but not
  // read)
  const int KS = K >> 7, G = PARTIAL ? (KS + 3) >> 2 : KS >> 2;
  const uint32_t kA = K >> 2, kM = K >> (M24 ? 3 : 4), kS = K >> 5, kR = K >> 1;
  const int4v r_dn = make_rsrc(res_codes, (uint32_t)act_rows * kR);
  const int4v r_sp = make_rsrc(bb_codes, (uint32_t)act_rows * kA);
  const int4v r_mt = make_rsrc(bb_meta, (uint32_t)act_rows * kM);
  const int4v r_ssp = make_rsrc(bb_scale, (uint32_t)act_rows * kS);
  const int4v r_sdn = make_rsrc(res_scale, (uint32_t)act_rows * kS);
  const int4v r_b = make_rsrc(payload + (int64_t)grp * D * kR, (uint32_t)D * kR);
  const int4v r_sb = make_rsrc(wscale + (int64_t)grp * D * kS, (uint32_t)D * kS);

  // activation row of tile row r (rows past the tile's end read row 0: their
  // products reach only outputs that are never stored)
  auto act_row = [&](int r) -> uint32_t {
    const int gr = m0 + r;
    return gr < row_end ? (uint32_t)gather_row(row_index, gr, act_rows) : 0u;
  };
  auto w_row = [&](int c) -> uint32_t { return n0 + c < D ? (uint32_t)(n0 + c) : 0u; };

  // ---- per-lane DMA byte offsets at step / group 0
  uint32_t o_dn[2], o_b[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int sl = 64 * (w + 8 * j) + l, row = sl >> 2, q = (sl & 3) ^ swz(row);
    o_dn[j] = act_row(row) * kR + 16 * q;
    // staged columns past the tile's BNE are never read: an offset past the
    // buffer loads zeros without a memory request
    o_b[j] = row < BNE ? w_row(row) * kR + 16 * q : 0x80000000u;
  }
  uint32_t o_sp;
  {
    const int sl = 64 * w + l, row = sl >> 1, h = (sl & 1) ^ ((row >> 3) & 1);
    o_sp = act_row(row) * kA + 16 * h;
  }
  // 4:8: 2 lanes x 16 B per row and side group; 2:4: 16 B per row and step,
  // waves w and w + 4 loading the same rows (same bytes to the same place)
  const uint32_t o_mt = M24 ? act_row(64 * wq + l) * kM : act_row((64 * w + l) >> 1) * kM + 16 * (l & 1);
  // waves 0-3: backbone scale rows and weight scale columns 64 wq + l;
  // waves 4-7: residual scale rows and the same weight columns again
  const uint32_t o_sa = act_row(64 * wq + l) * kS;
  const uint32_t o_sw = 64 * wq + l < BNE ? w_row(64 * wq + l) * kS : 0x80000000u;
  const int4v r_sa = w < 4 ? r_ssp : r_sdn;

  auto issue_main = [&](int s, MainT& st) {
    const uint32_t s64 = 64u * s, s32 = 32u * s;
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(r_dn, o_dn[j], s64, lds_addr(&st.a_dn[64 * (w + 8 * j)]));
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(r_b, o_b[j], s64, lds_addr(&st.b[64 * (w + 8 * j)]));
    if constexpr (!DENSE) dma16(r_sp, o_sp, s32, lds_addr(&st.a_sp[64 * w]));
    if constexpr (M24) dma16(r_mt, o_mt, 16u * s, lds_addr(&st.meta[64 * wq]));
  };
  auto issue_side = [&](int g, SideT& sd) {
    if constexpr (DENSE) {
      dma16(r_sdn, o_sa, 16u * g, lds_addr(&sd.s_dn[64 * wq]));   // waves w and w + 4: same bytes
    } else if constexpr (M24) {
      dma16(r_sa, o_sa, 16u * g, lds_addr(w < 4 ? &sd.s_sp[64 * wq] : &sd.s_dn[64 * wq]));
    } else {
      dma16(r_mt, o_mt, 32u * g, lds_addr(&sd.meta[64 * w]));
      dma16(r_sa, o_sa, 16u * g, lds_addr(w < 4 ? &sd.s_sp[64 * wq] : &sd.s_dn[64 * wq]));
    }
    dma16(r_sb, o_sw, 16u * g, lds_addr(&sd.s_b[64 * wq]));   // waves w and w + 4: same bytes
  };

  const int wm0 = (w % WROWS) * WM, wn0 = (w / WROWS) * WNC;
  const int kh = l >> 5, lr = l & 31;
  // per step: scales (both halves: op_sel picks the byte), metadata (low /
  // high 16 bits) and the compacted backbone (low / high 8 bytes) are read
  // once; per half-step only the weight and residual code fragments
  struct StepFrag {
    uint32_t bs[FN], ssp[FM], sdn[FM], mt[FM], mt2[FM];   // mt2: 2:4 only
    uint4 sp[FM];
  };
  struct HalfFrag {
    uint4 b[FN], dn[FM];
  };
  auto read_step = [&](const MainT& st, const SideT& sd, int p, StepFrag& S) {
    const uint16_t* s_b = reinterpret_cast<const uint16_t*>(sd.s_b);
    const uint16_t* s_sp = reinterpret_cast<const uint16_t*>(sd.s_sp);
    const uint16_t* s_dn = reinterpret_cast<const uint16_t*>(sd.s_dn);
#pragma unroll
    for (int n = 0; n < FN; ++n) S.bs[n] = s_b[8 * (wn0 + 32 * n + lr) + 2 * p + kh];
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      const int r = wm0 + 32 * f + lr;
      if constexpr (!DENSE) {
        S.sp[f] = st.a_sp[slot_sp(r, kh)];
        if constexpr (M24) {
          // the lane's two 32-value blocks: dwords 2 kh and 2 kh + 1 of the row
          const uint2 m = reinterpret_cast<const uint2*>(st.meta)[2 * r + kh];
          S.mt[f] = m.x;
          S.mt2[f] = m.y;
        } else {
          S.mt[f] = reinterpret_cast<const uint32_t*>(sd.meta)[8 * r + 2 * p + kh];
        }
        S.ssp[f] = s_sp[8 * r + 2 * p + kh];
      }
      S.sdn[f] = s_dn[8 * r + 2 * p + kh];
    }
  };
  auto read_half = [&](const MainT& st, HalfFrag& H, auto jc) {
    constexpr int J = decltype(jc)::value;
#pragma unroll
    for (int n = 0; n < FN; ++n) H.b[n] = st.b[slot(wn0 + 32 * n + lr, 2 * kh + J)];
#pragma unroll
    for (int f = 0; f < FM; ++f) H.dn[f] = st.a_dn[slot(wm0 + 32 * f + lr, 2 * kh + J)];
  };

  v16f acc[FM][FN];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int n = 0; n < FN; ++n) acc[f][n] = (v16f){};

  auto mfma_half = [&](const StepFrag& S, const HalfFrag& H, auto jc) {
    constexpr int J = decltype(jc)::value;
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      if constexpr (!DENSE) {
        uint4 asp;
        if constexpr (M24)
          asp = J == 0 ? expand_24(S.sp[f].x, S.sp[f].y, S.mt[f]) : expand_24(S.sp[f].z, S.sp[f].w, S.mt2[f]);
        else
          asp = J == 0 ? expand4_fast(S.sp[f].x, S.sp[f].y, S.mt[f] & 0xFFFFu)
                       : expand4_fast(S.sp[f].z, S.sp[f].w, S.mt[f] >> 16);
#pragma unroll
        for (int n = 0; n < FN; ++n) acc[f][n] = mfma32_fp4_sel<J>(asp, H.b[n], acc[f][n], S.ssp[f], S.bs[n]);
      }
#pragma unroll
      for (int n = 0; n < FN; ++n) acc[f][n] = mfma32_fp4_sel<J>(H.dn[f], H.b[n], acc[f][n], S.sdn[f], S.bs[n]);
    }
  };
  const std::integral_constant<int, 0> j0{};
  const std::integral_constant<int, 1> j1{};

  StepFrag sf;
  HalfFrag hf;
  issue_main(0, lds[0]);
  issue_side(0, side[0]);
  issue_main(min(1, KS - 1), lds[1]);
  for (int g = 0; g < G; ++g) {
    const SideT& sd = side[g & 1];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int s = 4 * g + p;
      if constexpr (PARTIAL)
        if (s >= KS) break;                               // partial last side group (uniform)
      // stage s (and at p = 0 side group g) landed; stage s+1 (and after
      // p = 2 side group g+1) may still be in flight.  After the barrier every
      // wave is past its reads of step s-1, whose buffer stage s+2 reuses.
      if (p == 3) wait_vm_lgkm0<NMAIN + NSIDE>();
      else wait_vm_lgkm0<NMAIN>();
      __builtin_amdgcn_s_barrier();
      issue_main(min(s + 2, KS - 1), lds[(s + 2) % kNS]);
      // side group g+1 replaces group g-1, last read at step 4 g - 1
      if (p == 2) issue_side(min(g + 1, G - 1), side[(g + 1) & 1]);
      const MainT& cur = lds[s % kNS];
      read_step(cur, sd, p, sf);
      read_half(cur, hf, j0);
      mfma_half(sf, hf, j0);
      read_half(cur, hf, j1);
      mfma_half(sf, hf, j1);
    }
  }
  wait_vm_lgkm0<0>();                                  // no DMA may land after the tile ends

  // ---- epilogue: fp32 store of the accumulator tile
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int n = 0; n < FN; ++n) {
      const int c = n0 + wn0 + 32 * n + lr;
      if (c >= D) continue;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = m0 + wm0 + 32 * fm + 8 * (i >> 2) + 4 * kh + (i & 3);
        if (r < row_end) Y[(int64_t)r * ldy + c] = acc[fm][n][i];
      }
    }
  }
}

// ============================================================================
// host launchers
// ============================================================================
namespace {
// compute units of the current device (queried once per device)
int num_cus_gemm() {
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

// decode geometry: J = 4 K-steps per wave up to K = 2048, 8 beyond (at most
// 16 K-splits); column groups of 16 per workgroup while at least 200
// workgroups remain and the workgroup stays within 16 waves.  Every
// workgroup stages the whole activation, so fewer, wider workgroups read
// less of it (measured: 4096 x 14336 with 224 workgroups of 4 column groups
// 9.6 us, with 448 of 2 10.6 us; 16 steps per wave at K = 14336 is slower).
template <bool FUSED, bool M24 = false>
hipError_t launch_decode(const uint8_t* bb_codes, const uint8_t* bb_meta, const uint8_t* bb_scale,
                         const uint8_t* res_codes, const uint8_t* res_scale, const int32_t* row_index, int rows,
                         int act_rows, int K, const uint8_t* payload, const uint8_t* wscale, int D, float* Y, int64_t ldy,
                         FusedPrep fp, hipStream_t s) {
  const int KS = K / 128;
  // 4 steps per wave up to K = 2048; up to K = 4096 too when D is too narrow
  // for column groups (more waves per workgroup keep more loads in flight:
  // 4096 x 4096 4.85 -> 4.56 us; with column groups 8 steps per wave is
  // faster: 4096 x 14336 9.4 vs 10.1 us)
  const int J = (KS <= 16 || (KS <= 32 && (D + 31) / 32 < 200)) ? 4 : 8;
  int NK = 1;
  while (NK * J < KS) NK *= 2;
  int CG = 1;
  while (NK * CG * 2 <= 16 && (D + 16 * CG * 2 - 1) / (16 * CG * 2) >= 200) CG *= 2;
  const int KBP = ((K / 32 + 15) & ~15) + 4;           // as in the kernel
  const size_t lds = (size_t)(K / 32 + 1) * 16 * 16 + (size_t)(16 * KBP + 16) / 16 * 16 +
                     (size_t)NK * CG * 64 * 4 * sizeof(float);
  const int n_gemm = (D + 16 * CG - 1) / (16 * CG);
  // fused: the producers are workgroups 0, 8, .., 8 (rows - 1)
  dim3 grid(FUSED ? std::max(n_gemm, 8 * (rows - 1) + 1) : n_gemm), block(64 * NK * CG);
#define L(NK_, CG_, J_)                                                                                                 \
  hipLaunchKernelGGL((linear_mx_decode<NK_, CG_, J_, FUSED, M24>), grid, block, lds, s, bb_codes, bb_meta, bb_scale,    \
                     res_codes, res_scale, row_index, rows, act_rows, K, payload, wscale, D, Y, ldy, fp)
  switch (J * 10000 + NK * 100 + CG) {
    case 40101: L(1, 1, 4); break;
    case 40102: L(1, 2, 4); break;
    case 40104: L(1, 4, 4); break;
    case 40108: L(1, 8, 4); break;
    case 40116: L(1, 16, 4); break;
    case 40201: L(2, 1, 4); break;
    case 40202: L(2, 2, 4); break;
    case 40204: L(2, 4, 4); break;
    case 40208: L(2, 8, 4); break;
    case 40401: L(4, 1, 4); break;
    case 40402: L(4, 2, 4); break;
    case 40404: L(4, 4, 4); break;
    case 80401: L(4, 1, 8); break;
    case 80402: L(4, 2, 8); break;
    case 80404: L(4, 4, 8); break;
    case 80801: L(8, 1, 8); break;
    case 80802: L(8, 2, 8); break;
    case 81601: L(16, 1, 8); break;
    case 40801: L(8, 1, 4); break;
    default: return hipErrorInvalidValue;
  }
#undef L
  return hipGetLastError();
}
}  // namespace

int decode_max_k() { return kDecodeMaxK; }

hipError_t launch_prepare_linear_mx(const void* X, bool bf16, int T, int K, int64_t ldx, const float* gamma, float eps,
                                    uint8_t* bb_codes, uint8_t* bb_meta, uint8_t* bb_scale, uint8_t* res_codes,
                                    uint8_t* res_scale, const uint8_t* payload, const uint8_t* wscale, int D, float* Y,
                                    int64_t ldy, uint32_t* sync, hipStream_t s) {
  if (T < 1 || T > 8 || K > kDecodeMaxK) return hipErrorInvalidValue;
  const FusedPrep fp{X, bf16 ? 1 : 0, ldx, gamma, eps, sync};
  return launch_decode<true>(bb_codes, bb_meta, bb_scale, res_codes, res_scale, nullptr, T, T, K, payload, wscale, D, Y,
                             ldy, fp, s);
}

namespace {
template <bool M24>
hipError_t launch_linear_mx_impl(const uint8_t* bb_codes, const uint8_t* bb_meta, const uint8_t* bb_scale,
                                 const uint8_t* res_codes, const uint8_t* res_scale, const int32_t* row_index, int rows,
                                 int act_rows, int K, const uint8_t* payload, const uint8_t* wscale, int D, int n_groups,
                                 const int32_t* group_offsets, float* Y, int64_t ldy, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (n_groups == 1 && rows <= 8 && K <= kDecodeMaxK)
    return launch_decode<false, M24>(bb_codes, bb_meta, bb_scale, res_codes, res_scale, row_index, rows, act_rows, K, payload,
                                wscale, D, Y, ldy, FusedPrep{}, s);
  if (n_groups == 1 && rows <= 64) {
    const int KS = K / 128;
    const int mt = (rows + 7) / 8;
    int MT = 1;
    while (MT < mt) MT *= 2;
    const int J = MT >= 8 ? 1 : 8 / MT;
    const int max_nw = MT >= 8 ? 8 : 16;
    int NW = 4;
    while (NW < max_nw && (KS + NW - 1) / NW > J) NW *= 2;
    const size_t lds = (size_t)NW * MT * 64 * 4 * sizeof(float);
    dim3 grid((D + 15) / 16), block(64 * NW);
#define L(MT_, J_)                                                                                             \
  hipLaunchKernelGGL((linear_mx_skinny<MT_, J_, M24>), grid, block, lds, s, bb_codes, bb_meta, bb_scale, res_codes, \
                     res_scale, row_index, rows, act_rows, K, payload, wscale, D, Y, ldy)
    switch (MT) {
      case 1: L(1, 8); break;
      case 2: L(2, 4); break;
      case 4: L(4, 2); break;
      default: L(8, 1); break;
    }
#undef L
    return hipGetLastError();
  }
  // the eight-wave tile (256 rows, 256 or 224 columns); K % 128 == 0 is
  // checked by the caller, and K % 512 != 0 takes the instance whose last
  // group of four steps is partial
  if (K % 128 != 0) return hipErrorInvalidValue;
  const bool partial = K % 512 != 0;
  if (n_groups == 1) {
    // tile width 256 or 224: the one with fewer rounds x width over the CUs
    const int tiles_m = (rows + 255) / 256;
    const int ncu = num_cus_gemm();
    const int t256 = tiles_m * ((D + 255) / 256), t224 = tiles_m * ((D + 223) / 224);
    const bool narrow = (int64_t)((t224 + ncu - 1) / ncu) * 224 < (int64_t)((t256 + ncu - 1) / ncu) * 256;
#define T8(BNE_, PARTIAL_)                                                                                            \
  hipLaunchKernelGGL((linear_mx_tile8<8, BNE_, false, false, M24, PARTIAL_>), dim3(narrow ? t224 : t256), dim3(512), 0, \
                     s, bb_codes, bb_meta, bb_scale, res_codes, res_scale, row_index, rows, act_rows, K, payload,       \
                     wscale, D, 1, nullptr, Y, ldy)
    if (narrow) {
      if (partial) T8(224, true);
      else T8(224, false);
    } else {
      if (partial) T8(256, true);
      else T8(256, false);
    }
#undef T8
  } else {
    // grouped: 256-wide tiles (measured on the MoE shapes, the general
    // eight-wave tile of 256 x 256 was faster than 128 x 256 with four waves
    // despite the emptier last row tile of each expert).  A bound on the
    // tile count; surplus workgroups return at once.
    const int bound = ((rows + 255) / 256 + n_groups) * ((D + 255) / 256);
#define T8G(PARTIAL_)                                                                                                 \
  hipLaunchKernelGGL((linear_mx_tile8<8, 256, false, true, M24, PARTIAL_>), dim3(bound), dim3(512), 0, s, bb_codes,    \
                     bb_meta, bb_scale, res_codes, res_scale, row_index, rows, act_rows, K, payload, wscale, D, n_groups, \
                     group_offsets, Y, ldy)
    if (partial) T8G(true);
    else T8G(false);
#undef T8G
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_linear_mx(const uint8_t* bb_codes, const uint8_t* bb_meta, const uint8_t* bb_scale,
                            const uint8_t* res_codes, const uint8_t* res_scale, const int32_t* row_index, int rows,
                            int act_rows, int K, const uint8_t* payload, const uint8_t* wscale, int D, int n_groups,
                            const int32_t* group_offsets, float* Y, int64_t ldy, hipStream_t s, bool m24) {
  return m24 ? launch_linear_mx_impl<true>(bb_codes, bb_meta, bb_scale, res_codes, res_scale, row_index, rows, act_rows,
                                           K, payload, wscale, D, n_groups, group_offsets, Y, ldy, s)
             : launch_linear_mx_impl<false>(bb_codes, bb_meta, bb_scale, res_codes, res_scale, row_index, rows,
                                            act_rows, K, payload, wscale, D, n_groups, group_offsets, Y, ldy, s);
}

// plain dense MXFP4 GEMM of the comparison baseline: Y = X~ W~ with one
// operand (codes T x K/2, E8M0 scales T x K/32), on the prefill tile
hipError_t launch_linear_dense_mx(const uint8_t* codes, const uint8_t* scales, int rows, int K, const uint8_t* payload,
                                  const uint8_t* wscale, int D, float* Y, int64_t ldy, hipStream_t s) {
  if (rows <= 0 || D <= 0) return hipSuccess;
  if (K % 512 != 0) return hipErrorInvalidValue;
  const int tiles_m = (rows + 255) / 256;
  const int ncu = num_cus_gemm();
  const int t256 = tiles_m * ((D + 255) / 256), t224 = tiles_m * ((D + 223) / 224);
  const bool narrow = (int64_t)((t224 + ncu - 1) / ncu) * 224 < (int64_t)((t256 + ncu - 1) / ncu) * 256;
  if (narrow)
    hipLaunchKernelGGL((linear_mx_tile8<8, 224, true>), dim3(t224), dim3(512), 0, s, nullptr, nullptr, nullptr, codes,
                       scales, nullptr, rows, rows, K, payload, wscale, D, 1, nullptr, Y, ldy);
  else
    hipLaunchKernelGGL((linear_mx_tile8<8, 256, true>), dim3(t256), dim3(512), 0, s, nullptr, nullptr, nullptr, codes,
                       scales, nullptr, rows, rows, K, payload, wscale, D, 1, nullptr, Y, ldy);
  return hipGetLastError();
}

}  // namespace sharq
