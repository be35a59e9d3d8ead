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
// Four kernels:
//  - skinny (2:4 backbone, T <= 64 at K > 16384): weight streaming.  A
//    16-row MFMA tile holds the backbone of 8 tokens in rows 0-7 and their
//    residual in rows 8-15, so one MFMA applies a weight fragment to both
//    paths; the epilogue adds row r and row r + 8 of the tile.  K is split
//    over the waves of a workgroup and the partial tiles are summed in a
//    fixed order through LDS.
//  - decode (T <= 8 at K <= 16384, 9-16 rows at K <= 7168): the skinny
//    scheme with the activation side staged once per workgroup in LDS in
//    operand form, one or two 16-row MFMA tiles (8 or 16 tokens) per launch
//    (2:4 backbones at 9-64 rows in chunks of launches); optionally fused
//    with the preparation of the rows (single-launch decode).
//  - batch (4:8 backbone, 17-64 rows, and 9-16 rows at K > 7168): the
//    decode scheme with the activation operand staged in double-buffered
//    chunks of K by staging waves beside the waves that load weights and
//    multiply, so the weight is read once for all rows at any K.
//  - tile8 (prefill and grouped MoE, more than 64 rows): 256 rows x 256 (or
//    224) columns, eight waves, K steps of 128 staged by buffer->LDS DMA
//    through a 3-deep ring (scales and metadata in a side ring of four-step
//    groups); the compacted backbone is staged as is and expanded in
//    registers right before its MFMAs.  Grouped: 128-row tiles, four waves,
//    a 2-deep ring, a persistent grid of two workgroups per CU.
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
// decode kernel (at most 16 activation rows)
// ============================================================================
// One 16x16x128 MFMA per 128-wide K-step: MFMA rows 0-7 are the backbone of
// tokens 0-7, rows 8-15 their residual, so one accumulator holds both paths
// and the epilogue adds row t and row t + 8.
//
// The workgroup stages the activation side in LDS: for 32-block kb and MFMA
// row r of tile m the 16 code bytes (backbone expanded from its compacted
// pairs) sit in slot 16 MT kb + 16 m + r, the scale in row 16 m + r of the
// scale table.  Its loads (L2 hits) are
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
// With 9-16 rows (MT = 2) every K-step takes two MFMAs, one per group of 8
// tokens, with twice the staged operand (so K <= 7168 fits LDS).
//
// Fused (single-launch decode, rows <= 16): GEMM workgroups 0, 8, .., 8 (rows-1)
// also prepare one activation row each (RowPrep: the standalone prepare's
// outputs, bit for bit): they load the row and gamma, then their weights,
// quantize and store the row with write-through stores, wait until all of it
// is done, and increment the done counter at memory.  (A release that writes
// the L2 back costs microseconds; write-through stores need none.)
// Workgroups go to the 8 XCDs round robin, so all producers share XCD 0 and
// its L2.  Every GEMM workgroup issues its weight loads, then waits (one lane,
// bounded polling) until the done counter reaches this call's target, and
// only then loads the prepared activations with ordinary loads: on XCD 0 they
// hit the producers' L2, elsewhere the L2 holds no line of these buffers
// (caches are invalidated at kernel start and nothing reads them before the
// wait), so the first read fetches the written-back bytes and later ones hit.
// The weight stream overlaps the preparation.  Workgroups are dispatched in
// index order on every XCD and the producers come first on XCD 0, so they
// are resident before any waiting workgroup can hold their place.
//
// Workspace words (uint32): sync[0] counts finished producer rows over all
// calls (it is never reset, so an increment can only count for its own call
// or an earlier one); sync[2] is this call's base, the value sync[0] holds
// once every earlier call's producers are done, so the wait is for
// sync[0] - sync[2] >= rows (modulo 2^32); sync[1] counts the GEMM
// workgroups past the wait, and the last one sets sync[2] += rows and
// sync[1] = 0 for the next call.  sync[3] is a sticky error word: a GEMM
// workgroup whose wait gives up (kFusedSpinMax polls, about a second; a
// correct call waits microseconds) sets it, and every GEMM workgroup that
// finds it set writes NaN to its Y columns instead of computing them, so a
// failed wait is never a silently wrong Y.  The caller clears a workspace
// (all zero) before first use and after an error; sharq_prepare_linear_status
// reads the word.
constexpr int kDecodeMaxK = 16384;                   // staged operand + reduction fit in LDS (<= 8 rows)
constexpr int kDecodeMaxK16 = 7168;                  // the same for 9-16 rows (two MFMA tiles)
constexpr uint32_t kFusedSpinMax = 1u << 20;         // polls before giving up (the kernel always ends)
constexpr int kAuxWriteThrough = 16;                 // store cache policy sc1: written through to memory

struct FusedPrep {
  const void* X;               // activation rows (bf16 or fp32), row r at X + r * ldx elements
  int bf16;
  int64_t ldx;
  const float* gamma;          // RMSNorm weights or null (no normalization)
  float eps;
  uint32_t* sync;              // [4]: done rows, GEMM workgroups past the wait, base, sticky error
};

template <int NK, int CG, int J, bool FUSED, bool M24 = false, int MT = 1>
__global__ __launch_bounds__(NK * CG * 64) void linear_mx_decode(
    const uint8_t* bb_codes, const uint8_t* bb_meta, const uint8_t* bb_scale, const uint8_t* res_codes,
    const uint8_t* res_scale, const int32_t* __restrict__ row_index, int rows, int act_rows, int K,
    const uint8_t* __restrict__ payload, const uint8_t* __restrict__ wscale, int D, float* __restrict__ Y, int64_t ldy,
    FusedPrep fp) {
  static_assert(J % 4 == 0, "weight scales load four steps at a time");
  constexpr int NW = NK * CG;                          // K-splits x column groups
  // MT MFMA tiles of 16 rows per K-step: tile m holds the backbone of tokens
  // 8 m .. 8 m + 7 in rows 0-7 and their residual in rows 8-15
  constexpr int NR = 16 * MT;
  extern __shared__ uint4 dsm[];
  constexpr uint32_t kOut = 0x80000000u;             // offset past every buffer here: reads zero
  constexpr int NT = NW * 64;
  const int KB = K >> 5, KS = K >> 7;
  // scale rows: row 16 m + r of tile m (r 0-7: backbone, 8-15: residual of
  // token 8 m + (r & 7)) at s_sm + (16 m + r) * KBP; KBP / 4 odd, so the 16
  // rows of one tile's reads fall on distinct banks; a spare 16-byte slot
  // follows them
  const int KBP = ((KB + 15) & ~15) + 4;
  uint4* const a_sm = dsm;                                            // [KB + 1][NR]
  uint8_t* const s_sm = reinterpret_cast<uint8_t*>(dsm + (KB + 1) * NR);   // [NR][KBP] + 16
  float* const red = reinterpret_cast<float*>(dsm + (KB + 1) * NR + (NR * KBP + 16) / 16);   // [NW][MT][64][4]
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
  // are done.  NK J >= K / 128 gives 8 MT KB <= NT IPT, and 2 scale pieces per
  // thread cover the NR KB16 scale pieces.
  constexpr int IPT = (MT * J / (2 * CG)) > 0 ? MT * J / (2 * CG) : 1;
  constexpr int BPT = (IPT + 1) / 2;                  // backbone pieces per thread
  const int KBh = KB >> 1, KB16 = (KB + 15) >> 4;
  const int n_res = 8 * MT * KB, n_bb = 8 * MT * KBh, n_sc = NR * KB16;
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
      const int i = tid + NT * j, r = qdiv(i, rKB16), p = i - r * KB16, t = 8 * (r >> 4) + (r & 7);
      const bool ok = i < n_sc && t < rows;
      // bytes past a row's K / 32 belong to the next row (or read zero past
      // the buffer); they land in the row's padding
      const uint32_t off = ok ? act_row(t) * (uint32_t)(K >> 5) + 16u * p : kOut;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128((r & 8) == 0 ? r_bs : r_rs, off, 0, 0);
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
  // steps [lo, hi) of this wave (lo, hi multiples of 4: one scale load per
  // four steps)
  auto load_weights = [&](auto lo_c, auto hi_c) {
    constexpr int lo = decltype(lo_c)::value, hi = decltype(hi_c)::value;
#pragma unroll
    for (int j = lo; j < hi; ++j) {
      const uint32_t out = s0 + j < KS ? 0u : kOut;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(r_w, (o_w + 64u * (uint32_t)(s0 + j)) | out, 0, 0);
      wv[j] = make_uint4(v[0], v[1], v[2], v[3]);
    }
#pragma unroll
    for (int j = lo; j < hi; j += 4) {
      // 16 bytes = blocks 4 (s0 + j) .. 4 (s0 + j + 4) - 1; past the row's
      // end only scales of zero-weight steps are affected
      const uint32_t out = s0 + j < KS ? 0u : kOut;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(r_ws, (o_ws + 4u * (uint32_t)(s0 + j)) | out, 0, 0);
      wsd[j] = v[0]; wsd[j + 1] = v[1]; wsd[j + 2] = v[2]; wsd[j + 3] = v[3];
    }
  };
  // fused: a wave's loads complete in order, so anything behind its weight
  // loads also waits for them.  Producers load their weights only after
  // their signal (its wait then covers their row stores alone) and wave 0,
  // whose lane 0 polls the counter, after the poll and its activation
  // loads; the other waves stream their weights from the start.  (Also
  // holding back the second half of the other waves' weights until after
  // their activation loads measured no better.)
  const std::integral_constant<int, 0> c0{};
  const std::integral_constant<int, J> cj{};
  bool early_w = true;
  if constexpr (FUSED) early_w = !producer && w != 0;   // uniform
  if (early_w) load_weights(c0, cj);
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
    __shared__ uint32_t failed;
    if (tid == 0) {
      const uint32_t base = __hip_atomic_load(&fp.sync[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      uint32_t bad = __hip_atomic_load(&fp.sync[3], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (!bad) {
        uint32_t it = 0;
        for (; it < kFusedSpinMax; ++it) {
          const uint32_t done = __hip_atomic_load(&fp.sync[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((int32_t)(done - base - (uint32_t)rows) >= 0) break;
          __builtin_amdgcn_s_sleep(2);
        }
        if (it == kFusedSpinMax) {                   // gave up: never compute from unready activations
          bad = 1u;
          __hip_atomic_fetch_or(&fp.sync[3], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      failed = bad;
      const uint32_t n = __hip_atomic_fetch_add(&fp.sync[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (n + 1 == (uint32_t)n_gemm) {               // every GEMM workgroup is past the wait
        __hip_atomic_store(&fp.sync[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&fp.sync[2], base + (uint32_t)rows, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
    if (failed) {                                    // uniform: NaN in this workgroup's outputs
      for (int i = tid; i < 8 * MT * 16 * CG; i += NT) {
        const int t = i / (16 * CG), c = bx * 16 * CG + i % (16 * CG);
        if (t < rows && c < D) Y[(int64_t)t * ldy + c] = __builtin_nanf("");
      }
      return;
    }
    load_act();
    if (!early_w) load_weights(c0, cj);
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
    a_sm[i < n_res ? NR * kb + 16 * (t >> 3) + 8 + (t & 7) : NR * KB] = rv[j];
  }
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int i = tid + NT * j, t = qdiv(i, rKBh), kp = i - t * KBh;
    const bool ok = i < n_bb;
    const int tr = 16 * (t >> 3) + (t & 7);          // MFMA row of token t's backbone
    if constexpr (M24) {
      a_sm[ok ? NR * (2 * kp) + tr : NR * KB + 1] = expand_24(bv[j].x, bv[j].y, mv[j].x);
      a_sm[ok ? NR * (2 * kp + 1) + tr : NR * KB + 2] = expand_24(bv[j].z, bv[j].w, mv[j].y);
    } else {
      a_sm[ok ? NR * (2 * kp) + tr : NR * KB + 1] = expand4_fast(bv[j].x, bv[j].y, mv[j].x & 0xFFFFu);
      a_sm[ok ? NR * (2 * kp + 1) + tr : NR * KB + 2] = expand4_fast(bv[j].z, bv[j].w, mv[j].x >> 16);
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = tid + NT * j, r = qdiv(i, rKB16), p = i - r * KB16;
    // row r of the scale table is MFMA row r & 15 of tile r >> 4
    // (4-byte stores: KBP is a multiple of 4, not of 16)
    uint32_t* dst = reinterpret_cast<uint32_t*>(s_sm + (i < n_sc ? r * KBP + 16 * p : NR * KBP));
    dst[0] = sv[j].x; dst[1] = sv[j].y; dst[2] = sv[j].z; dst[3] = sv[j].w;
  }
  __syncthreads();

  // ---- MFMAs (steps past K carry zero weights; their LDS slot is clamped)
  v4f acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int s = s0 + j < KS ? s0 + j : KS - 1;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int e = NR * (4 * s + kq) + 16 * m + (l & 15);
      acc[m] = mfma_fp4(a_sm[e], wv[j], acc[m], s_sm[(16 * m + (l & 15)) * KBP + 4 * s + kq],
                        (wsd[j] >> (8 * kq)) & 0xFFu);
    }
  }

  // ---- fixed-order reduction over the waves; backbone row + residual row
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    float* p = red + ((w * MT + m) * 64 + l) * 4;
    p[0] = acc[m][0]; p[1] = acc[m][1]; p[2] = acc[m][2]; p[3] = acc[m][3];
  }
  __syncthreads();
  if (kw == 0 && l < 32) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float bsum = 0.0f, rsum = 0.0f;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          const int ww = kk * CG + cg;
          bsum += red[((ww * MT + m) * 64 + l) * 4 + i];
          rsum += red[((ww * MT + m) * 64 + l + 32) * 4 + i];
        }
        // lane l < 32 holds MFMA rows 4 (l >> 4) + i of tile m (backbone of
        // tokens 8 m ..); lane l + 32 holds rows 8 + 4 (l >> 4) + i (their residual)
        const int t = 8 * m + 4 * (l >> 4) + i;
        if (t < rows && col < D) Y[(int64_t)t * ldy + col] = bsum + rsum;
      }
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
// tile timeline (tracing build only, SHARQ_TIMELINE): wave 0 of each tile
// records s_memrealtime stamps (100 MHz) at the tile's start, after its first
// step's wait and barrier, after its last step and after its epilogue stores
// are issued, plus the issuing XCC and hardware ids and the workgroup.  The
// persistent 128-row tile writes record t for tile t; the 256-row tile (one
// tile per workgroup) writes record b for workgroup b.  The batch kernel
// writes record b for workgroup b, its staging phases from the first thread
// of its first staging wave.
// ============================================================================
constexpr int kTimelineRecords = 16384;
#ifdef SHARQ_TIMELINE
__device__ uint64_t g_timeline[kTimelineRecords * 8];
#define SHARQ_TL_BY(th, t, i, v)                                                        \
  do {                                                                                  \
    if (threadIdx.x == (th) && (t) < kTimelineRecords) g_timeline[(t) * 8 + (i)] = (v); \
  } while (0)
#define SHARQ_TL(t, i, v) SHARQ_TL_BY(0, t, i, v)
#define SHARQ_TL_ID(t)                                                                                        \
  do {                                                                                                        \
    SHARQ_TL(t, 4, ((uint64_t)__builtin_amdgcn_s_getreg(kHwRegXccId) << 32) |                                \
                       (uint32_t)__builtin_amdgcn_s_getreg(kHwRegHwId));                                      \
    SHARQ_TL(t, 5, blockIdx.x);                                                                               \
  } while (0)
// s_getreg_b32 operands: all 32 bits of HW_REG_HW_ID (4) and HW_REG_XCC_ID (20)
constexpr int kHwRegHwId = (31 << 11) | 4, kHwRegXccId = (31 << 11) | 20;
#else
#define SHARQ_TL_BY(th, t, i, v) \
  do {                           \
  } while (0)
#define SHARQ_TL(t, i, v) \
  do {                    \
  } while (0)
#define SHARQ_TL_ID(t) \
  do {                 \
  } while (0)
#endif
#define SHARQ_TL_NOW() __builtin_amdgcn_s_memrealtime()

// ============================================================================
// batch kernel (4:8 backbone; 17-64 rows, and 9-16 rows at K > 7168): the
// decode scheme with the activation operand staged in chunks of K, so the
// weight is read once for all rows at any K
// ============================================================================
// grid.x = ceil(D / (16 CG)); CG NK = 4 compute waves and 4 staging waves.  K is
// processed in chunks of KC = NK JC steps of 128, through two LDS stages
// holding the chunk's activation operand (backbone expanded) and scales.
//  - Staging waves load a chunk's pieces (coalesced 16-byte pieces of the
//    token rows, as in the decode kernel) three chunks ahead into registers
//    and write them to a stage in operand form.
//  - Compute wave (cg, kw) multiplies steps kw JC .. kw JC + JC - 1 of every
//    chunk for the 16 columns of column group cg, with its weights loaded
//    two chunks ahead.
// A wave's loads complete in order, so splitting the two streams over
// different waves lets each run ahead without waiting for the other.  MT
// MFMA tiles of 16 rows (tile m: the backbone of tokens 8 m .. 8 m + 7 in
// rows 0-7, their residual in rows 8-15) share each weight fragment; the NK
// partial tiles of a column group are summed in a fixed order through LDS at
// the end.  Every slot of a stage is written each chunk (absent tokens and
// blocks past K as zeros), so a product never meets a stale byte.
constexpr int kBatchStagingWaves = 4;
template <int MT, int CG, int NK, int JC>
__global__ __launch_bounds__((CG * NK + kBatchStagingWaves) * 64) void linear_mx_batch(
    const uint8_t* bb_codes, const uint8_t* bb_meta, const uint8_t* bb_scale, const uint8_t* res_codes,
    const uint8_t* res_scale, const int32_t* __restrict__ row_index, int rows, int act_rows, int K,
    const uint8_t* __restrict__ payload, const uint8_t* __restrict__ wscale, int D, float* __restrict__ Y, int64_t ldy) {
  constexpr int NCW = CG * NK;                          // compute waves
  static_assert(NCW == 4, "four compute waves");
  constexpr int NST = kBatchStagingWaves * 64;          // staging threads
  constexpr int NR = 16 * MT;                          // MFMA rows per step
  constexpr int KC = NK * JC;                          // steps per chunk
  constexpr int BC = 4 * KC;                           // 32-value blocks per chunk
  constexpr int SP = BC + 4;                           // scale row pitch: SP / 4 odd, 16 rows on distinct banks
  // operand row pitch: BC + 1 slots, so the 16 rows one MFMA read touches
  // start 4 banks apart (16 lanes x 16 bytes on distinct banks) and a
  // piece's store, consecutive blocks of one row, is contiguous
  constexpr int BCP = BC + 1;
  static_assert((SP / 4) % 2 == 1, "scale pitch");
  constexpr int WD = 2;                                // weight chunks in flight per compute wave
  constexpr uint32_t kOut = 0x80000000u;             // offset past every buffer here: reads zero
  extern __shared__ uint4 dsm[];
  uint4* const a_st = dsm;                                                       // [2][NR][BCP]
  uint8_t* const s_st = reinterpret_cast<uint8_t*>(dsm + 2 * NR * BCP);          // [2][NR][SP]
  float* const red = reinterpret_cast<float*>(dsm);                              // after the last chunk: [NCW][MT][64][4]
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int KB = K >> 5, KS = K >> 7, NC = (KS + KC - 1) / KC;
  auto rsrc = [](const uint8_t* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0,
                                             __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
  };
  const int cg = w % CG, kw = w / CG;                  // compute waves
  const int col = (blockIdx.x * CG + cg) * 16 + (l & 15);
  const int kq = l >> 4;
  v4f acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = (v4f){0.f, 0.f, 0.f, 0.f};
  SHARQ_TL(blockIdx.x, 0, SHARQ_TL_NOW());
  SHARQ_TL_ID(blockIdx.x);

  if (w >= NCW) {
    // ---- staging waves.  Residual pieces: 8 MT token slots x BC blocks;
    // backbone pieces: 8 MT x BC / 2 block pairs; scale pieces: NR rows x
    // BC / 16.  Two register sets: chunk k's pieces in set k & 1.
    constexpr int NRES = 8 * MT * BC, NBB = 8 * MT * BC / 2, NSC = NR * (BC / 16);
    constexpr int RPT = (NRES + NST - 1) / NST, BPT = (NBB + NST - 1) / NST, SPT = (NSC + NST - 1) / NST;
    const int ts = tid - NCW * 64;
    const int an = __builtin_amdgcn_readfirstlane(act_rows);
    const __amdgpu_buffer_rsrc_t r_rc = rsrc(res_codes, (int64_t)an * (K >> 1));
    const __amdgpu_buffer_rsrc_t r_rs = rsrc(res_scale, (int64_t)an * (K >> 5));
    const __amdgpu_buffer_rsrc_t r_bc = rsrc(bb_codes, (int64_t)an * (K >> 2));
    const __amdgpu_buffer_rsrc_t r_bm = rsrc(bb_meta, (int64_t)an * (K >> 4));
    const __amdgpu_buffer_rsrc_t r_bs = rsrc(bb_scale, (int64_t)an * (K >> 5));
    // the activation row of each of this thread's pieces (or none)
    auto act_row = [&](int t) -> uint32_t {
      return t < rows ? (uint32_t)gather_row(row_index, t, act_rows) : kOut;
    };
    uint32_t res_row[RPT], bb_row[BPT], sc_row[SPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int i = ts + NST * j;
      res_row[j] = i < NRES ? act_row(i / BC) : kOut;
    }
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int i = ts + NST * j;
      bb_row[j] = i < NBB ? act_row(i / (BC / 2)) : kOut;
    }
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int i = ts + NST * j, r = i / (BC / 16);
      sc_row[j] = i < NSC ? act_row(8 * (r >> 4) + (r & 7)) : kOut;
    }
    uint4 rv[3][RPT], bv[3][BPT], sv[3][SPT];
    uint32_t mv[3][BPT];
    // chunk c's pieces into register set q = c % 3 (blocks past K read
    // zero); the set index is a compile-time constant (the loop below is
    // unrolled by three), so the sets stay in registers
    auto load_chunk = [&](int c, auto qc) {
      constexpr int q = decltype(qc)::value;
      const int b0 = c * BC;                           // first block of the chunk
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        const int i = ts + NST * j, kb = b0 + i % BC;
        const uint32_t off = res_row[j] != kOut && kb < KB ? res_row[j] * (uint32_t)(K >> 1) + 16u * kb : kOut;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r_rc, off, 0, 0);
        rv[q][j] = make_uint4(v[0], v[1], v[2], v[3]);
      }
#pragma unroll
      for (int j = 0; j < BPT; ++j) {
        const int i = ts + NST * j, kp = (b0 >> 1) + i % (BC / 2);
        const bool ok = bb_row[j] != kOut && 2 * kp < KB;
        const auto v =
            __builtin_amdgcn_raw_buffer_load_b128(r_bc, ok ? bb_row[j] * (uint32_t)(K >> 2) + 16u * kp : kOut, 0, 0);
        bv[q][j] = make_uint4(v[0], v[1], v[2], v[3]);
        mv[q][j] = __builtin_amdgcn_raw_buffer_load_b32(r_bm, ok ? bb_row[j] * (uint32_t)(K >> 4) + 4u * kp : kOut, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < SPT; ++j) {
        const int i = ts + NST * j, r = i / (BC / 16), p = i % (BC / 16), kb = b0 + 16 * p;
        // bytes past the row's K / 32 are the next row's scales (or zero
        // past the buffer): finite, and met only by zero weights
        const uint32_t off = sc_row[j] != kOut && kb < KB ? sc_row[j] * (uint32_t)(K >> 5) + kb : kOut;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128((r & 8) == 0 ? r_bs : r_rs, off, 0, 0);
        sv[q][j] = make_uint4(v[0], v[1], v[2], v[3]);
      }
    };
    // register set q into LDS stage st (chunk c: set c % 3, stage c & 1)
    auto store_chunk = [&](auto qc, int st) {
      constexpr int q = decltype(qc)::value;
      uint4* const a = a_st + st * NR * BCP;
      uint8_t* const sc = s_st + st * NR * SP;
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        const int i = ts + NST * j, t = i / BC, kb = i % BC;
        if (i < NRES) a[(16 * (t >> 3) + 8 + (t & 7)) * BCP + kb] = rv[q][j];
      }
#pragma unroll
      for (int j = 0; j < BPT; ++j) {
        const int i = ts + NST * j, t = i / (BC / 2), kp = i % (BC / 2), tr = 16 * (t >> 3) + (t & 7);
        if (i < NBB) {
          a[tr * BCP + 2 * kp] = expand4_fast(bv[q][j].x, bv[q][j].y, mv[q][j] & 0xFFFFu);
          a[tr * BCP + 2 * kp + 1] = expand4_fast(bv[q][j].z, bv[q][j].w, mv[q][j] >> 16);
        }
      }
#pragma unroll
      for (int j = 0; j < SPT; ++j) {
        const int i = ts + NST * j, r = i / (BC / 16), p = i % (BC / 16);
        if (i < NSC) {
          // 4-byte stores: SP is a multiple of 4, not of 16
          uint32_t* dst = reinterpret_cast<uint32_t*>(sc + r * SP + 16 * p);
          dst[0] = sv[q][j].x; dst[1] = sv[q][j].y; dst[2] = sv[q][j].z; dst[3] = sv[q][j].w;
        }
      }
    };
    const std::integral_constant<int, 0> q0{};
    const std::integral_constant<int, 1> q1{};
    const std::integral_constant<int, 2> q2{};
    load_chunk(0, q0);
    if (NC > 1) load_chunk(1, q1);
    if (NC > 2) load_chunk(2, q2);
    store_chunk(q0, 0);
    SHARQ_TL_BY(NCW * 64, blockIdx.x, 1, SHARQ_TL_NOW());
    if (NC > 3) load_chunk(3, q0);                     // set 0 is free again
    // the barrier of chunk c: every compute wave is past chunk c - 1, which
    // read the stage chunk c + 1 goes to; chunk c + 1 is in set qn =
    // (c + 1) % 3, which then takes chunk c + 4 (three chunks of loads in
    // flight)
    auto step = [&](int c, auto qn) {
      __syncthreads();
      if (c + 1 < NC) {
        store_chunk(qn, (c + 1) & 1);
        if (c == 0) SHARQ_TL_BY(NCW * 64, blockIdx.x, 7, SHARQ_TL_NOW());
        if (c + 4 < NC) load_chunk(c + 4, qn);
      }
    };
    for (int c0 = 0; c0 < NC; c0 += 3) {
      step(c0, q1);
      if (c0 + 1 >= NC) break;
      step(c0 + 1, q2);
      if (c0 + 2 >= NC) break;
      step(c0 + 2, q0);
    }
  } else {
    // ---- compute waves: weights of this wave's steps, WD chunks ahead
    const __amdgpu_buffer_rsrc_t r_w = rsrc(payload, (int64_t)D * (K >> 1));
    const __amdgpu_buffer_rsrc_t r_ws = rsrc(wscale, (int64_t)D * (K >> 5));
    const uint32_t o_w = col < D ? (uint32_t)col * (uint32_t)(K >> 1) + 16u * kq : kOut;
    const uint32_t o_ws = col < D ? (uint32_t)col * (uint32_t)(K >> 5) : kOut;
    uint4 wv[WD][JC];
    uint32_t wsd[WD][JC];                              // dword: the 4 block scales of the step (byte kq)
    auto load_w = [&](int c, auto bc) {                // slot b: a compile-time constant
      constexpr int b = decltype(bc)::value;
#pragma unroll
      for (int j = 0; j < JC; ++j) {
        const int s = c * KC + kw * JC + j;
        const uint32_t out = s < KS ? 0u : kOut;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r_w, (o_w + 64u * (uint32_t)s) | out, 0, 0);
        wv[b][j] = make_uint4(v[0], v[1], v[2], v[3]);
        wsd[b][j] = __builtin_amdgcn_raw_buffer_load_b32(r_ws, (o_ws + 4u * (uint32_t)s) | out, 0, 0);
      }
    };
    // chunk c = c0 + b uses weight slot b and stage c & 1 (WD even), both
    // compile-time constants in the unrolled body
    auto chunk = [&](int c, auto bc) {
      constexpr int b = decltype(bc)::value;
      // stage c & 1 is written
      __syncthreads();
      const uint4* const a = a_st + (b & 1) * NR * BCP;
      const uint8_t* const sc = s_st + (b & 1) * NR * SP;
#pragma unroll
      for (int j = 0; j < JC; ++j) {
        const int sl = kw * JC + j;                    // step within the chunk
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const int r = 16 * m + (l & 15);
          acc[m] = mfma_fp4(a[r * BCP + 4 * sl + kq], wv[b][j], acc[m], sc[r * SP + 4 * sl + kq],
                            (wsd[b][j] >> (8 * kq)) & 0xFFu);
        }
        // one step's operand reads at a time: hoisting a whole chunk's reads
        // ahead of its MFMAs would not fit the registers
        __builtin_amdgcn_sched_barrier(0);
      }
      if (c == 0) SHARQ_TL(blockIdx.x, 6, SHARQ_TL_NOW());
      // unconditional (steps past K read zero): a branch here lets the
      // compiler sink the chunk's MFMAs below the new loads, which then
      // need a second copy of the slot's registers and spill
      load_w(c + WD, bc);
    };
    const std::integral_constant<int, 0> b0{};
    const std::integral_constant<int, 1> b1{};
    load_w(0, b0);
    if (NC > 1) load_w(1, b1);
    for (int c0 = 0; c0 < NC; c0 += WD) {
      chunk(c0, b0);
      if (c0 + 1 >= NC) break;
      chunk(c0 + 1, b1);
    }
  }
  SHARQ_TL(blockIdx.x, 2, SHARQ_TL_NOW());
  __syncthreads();                                     // every wave is past its last use of the stages

  // ---- fixed-order reduction over the K-splits; backbone row + residual row
  if (w < NCW) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float* p = red + ((w * MT + m) * 64 + l) * 4;
      p[0] = acc[m][0]; p[1] = acc[m][1]; p[2] = acc[m][2]; p[3] = acc[m][3];
    }
  }
  __syncthreads();
  if (w < NCW && kw == 0 && l < 32) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float bsum = 0.0f, rsum = 0.0f;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          const int ww = kk * CG + cg;
          bsum += red[((ww * MT + m) * 64 + l) * 4 + i];
          rsum += red[((ww * MT + m) * 64 + l + 32) * 4 + i];
        }
        // lane l < 32 holds MFMA rows 4 (l >> 4) + i of tile m (backbone of
        // tokens 8 m ..); lane l + 32 holds rows 8 + 4 (l >> 4) + i (their residual)
        const int t = 8 * m + 4 * (l >> 4) + i;
        if (t < rows && col < D) Y[(int64_t)t * ldy + col] = bsum + rsum;
      }
    }
  }
  SHARQ_TL(blockIdx.x, 3, SHARQ_TL_NOW());
}


// ============================================================================
// tile kernel (more than 64 rows; plain and grouped; K % 128 == 0)
// ============================================================================
// Tile 256 x 256 (or 224 columns), eight waves, two per SIMD covering each
// other's LDS and barrier latency; each wave holds a 128-register
// accumulator.  The grouped (MoE) form uses 128-row tiles with four waves
// and a two-stage ring (80 KB), two workgroups per CU.  The layout used is 8 x 1 (wave w: rows 32 w .., all
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

// BM: tile rows (256: eight waves, one workgroup per CU; 128: four waves, two
// workgroups per CU)
template <int BM>
struct Tile8Main {
  uint4 a_dn[BM * 4];          // residual codes, 64 B per row (swizzled 16 B slots)
  uint4 b[256 * 4];            // weight payload, 64 B per column
  uint4 a_sp[BM * 2];          // compacted backbone, 32 B per row
};
template <int BM>
struct Tile8Side {             // four steps
  uint4 meta[BM * 2];          // 32 B per row: step p at bytes 8 p .. 8 p + 7
  uint4 s_sp[BM];              // 16 B per row: step p at bytes 4 p .. 4 p + 3
  uint4 s_dn[BM];
  uint4 s_b[256];
};
// 2:4 backbone: its metadata (16 B per row and step) goes with the step's
// codes, and the side ring keeps the scales only (3 x 44 KB + 2 x 12 KB)
template <int BM>
struct Tile8Main24 : Tile8Main<BM> {
  uint4 meta[BM];              // 16 B per row: the step's four 32-value blocks
};
template <int BM>
struct Tile8Side24 {
  uint4 s_sp[BM];
  uint4 s_dn[BM];
  uint4 s_b[256];
};

}  // namespace

template <int BM, int BNE, bool DENSE = false, bool GROUPED = false, bool M24 = false, bool PARTIAL = false>
__global__ __launch_bounds__(2 * BM, BM == 256 ? 1 : 2) void linear_mx_tile8(
    const uint8_t* __restrict__ bb_codes, const uint8_t* __restrict__ bb_meta, const uint8_t* __restrict__ bb_scale,
    const uint8_t* __restrict__ res_codes, const uint8_t* __restrict__ res_scale, const int32_t* __restrict__ row_index,
    int rows, int act_rows, int K, const uint8_t* __restrict__ payload, const uint8_t* __restrict__ wscale, int D,
    int n_groups, const int32_t* __restrict__ group_offsets, float* __restrict__ Y, int64_t ldy) {
  // BM: tile rows; BM / 32 waves, wave w covering rows 32 w .. and all
  // columns (every backbone fragment expanded by one wave only).  BM = 256:
  // a 3-deep ring (160 KB, one workgroup per CU); BM = 128: a 2-deep ring
  // (80 KB), so two workgroups share a CU and one's epilogue overlaps the
  // other's MFMAs
  // BNE: columns the tile computes (256, or 224 so that more shapes give a
  // whole number of rounds over the CUs); staging stays 256 columns wide.
  // DENSE: the plain MXFP4 GEMM of the comparison baseline, one operand
  // (res_codes / res_scale hold plain codes and scales; no backbone)
  // GROUPED: per-expert weights (n_groups of them, group_offsets delimiting
  // each expert's rows), tiles numbered expert by expert
  // M24: the 2:4 element-wise backbone (metadata K/8 bytes per row)
  // PARTIAL: K % 512 != 0, the last side group of four steps is partial
  // (a separate instance keeps the K % 512 == 0 loop free of the check)
  static_assert(BM == 256 || BM == 128, "tile rows");
  static_assert(!(GROUPED && DENSE) && !(M24 && DENSE), "the plain baseline has no backbone");
  constexpr int NW = BM / 32;                   // waves
  constexpr int NS = BM == 256 ? kNS : 2;       // LDS ring depth
  constexpr int WB = 16 / NW;                   // weight-code DMAs per wave and step
  // DMA instructions per wave: per step (residual, weight, backbone codes;
  // 2:4: and metadata) and per side group (4:8: metadata; activation scales,
  // weight scales)
  constexpr int NMAIN = 2 + WB + (DENSE ? 0 : 1) + (M24 ? 1 : 0), NSIDE = DENSE || M24 ? 2 : 3;
  constexpr int WM = 32, WNC = BNE, FM = 1, FN = WNC / 32;
  using MainT = std::conditional_t<M24, Tile8Main24<BM>, Tile8Main<BM>>;
  using SideT = std::conditional_t<M24, Tile8Side24<BM>, Tile8Side<BM>>;
  __shared__ MainT lds[NS];
  __shared__ SideT side[2];
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  // activation scale rows 64 wq .. (half the waves each for the backbone and
  // the residual scales; 2:4 metadata and the plain baseline's scales are
  // loaded twice, by waves w and w + NW / 2) and weight scale columns
  // 64 wb .. (waves w and w + 4 load the same bytes when NW = 8)
  const int wq = w % (NW / 2), wb = w & 3;

  // ---- tile order. Tiles are ordered in bands of kBand row tiles that
  // sweep all column tiles (row fastest inside a band), and each XCD takes
  // one contiguous stretch of that order: the workgroups that run together on
  // one XCD then share a few activation and weight tiles through its L2
  // instead of all 16 row tiles of the activations (measured at 4096 x 4096
  // x 14336: 269 -> 243 us).  Grouped tiles are numbered expert by expert
  // (each expert's ceil(rows_e / BM) x tiles_n tiles, row tiles outer), so an
  // XCD's stretch covers a few experts.
  const int tiles_n = (D + BNE - 1) / BNE;
  constexpr int kBand = 4;
  auto band_tile = [&](int t, int& m0, int& n0) {
    const int tiles_m = (rows + BM - 1) / BM;
    const int band = t / (kBand * tiles_n), band_m = min(kBand, tiles_m - band * kBand);
    const int in_band = t - band * kBand * tiles_n;
    m0 = (band * kBand + in_band % band_m) * BM;
    n0 = (in_band / band_m) * BNE;
  };

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
  const bool first_half = w < NW / 2;                  // uniform
  const int4v r_sa = first_half ? r_ssp : r_sdn;

  // ---- one tile: rows m0 .. row_end - 1 (at most BM of them), columns
  // n0 .., the weight descriptors of its expert, and every lane's DMA byte
  // offsets at step / group 0.  Rows past the tile's end (the last row tile
  // of the matrix or of an expert) get an offset past every buffer, so their
  // DMAs load zeros without a memory request (their products reach only
  // outputs that are never stored).
  constexpr uint32_t kAbsent = 0x80000000u;
  struct TileRows {            // activation rows the lane's DMAs read (or kAbsent)
    uint32_t dn[2], sp, sa;    // residual rows; backbone (and 4:8 metadata) row; scale (and 2:4 metadata) row
  };
  struct TileOff {
    int m0, n0, row_end;
    int4v r_b, r_sb;
    uint32_t dn[2], b[WB], sp, mt, sa, sw;
  };
  // gathered rows: row_index loads when rows are gathered
  auto tile_rows = [&](int m0, int row_end, TileRows& tr) {
    auto g = [&](int r) -> uint32_t {
      const int gr = m0 + r;
      return gr < row_end ? (uint32_t)gather_row(row_index, gr, act_rows) : kAbsent;
    };
#pragma unroll
    for (int j = 0; j < 2; ++j) tr.dn[j] = g((64 * (w + NW * j) + l) >> 2);
    tr.sp = g((64 * w + l) >> 1);
    tr.sa = g(64 * wq + l);
  };
  auto tile_off = [&](int grp, int m0, int n0, int row_end, const TileRows& tr, TileOff& o) {
    auto off = [&](uint32_t row, uint32_t bytes) -> uint32_t { return row == kAbsent ? kAbsent : row * bytes; };
    auto w_row = [&](int c) -> uint32_t { return n0 + c < D ? (uint32_t)(n0 + c) : 0u; };
    o.m0 = m0;
    o.n0 = n0;
    o.row_end = row_end;
    o.r_b = make_rsrc(payload + (int64_t)grp * D * kR, (uint32_t)D * kR);
    o.r_sb = make_rsrc(wscale + (int64_t)grp * D * kS, (uint32_t)D * kS);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int sl = 64 * (w + NW * j) + l, row = sl >> 2, q = (sl & 3) ^ swz(row);
      o.dn[j] = off(tr.dn[j], kR) + 16 * q;
    }
#pragma unroll
    for (int j = 0; j < WB; ++j) {
      const int sl = 64 * (w + NW * j) + l, col = sl >> 2, q = (sl & 3) ^ swz(col);
      // staged columns past the tile's BNE are never read: an offset past
      // the buffer loads zeros without a memory request
      o.b[j] = col < BNE ? w_row(col) * kR + 16 * q : kAbsent;
    }
    {
      const int sl = 64 * w + l, row = sl >> 1, h = (sl & 1) ^ ((row >> 3) & 1);
      o.sp = off(tr.sp, kA) + 16 * h;
    }
    // 4:8: 2 lanes x 16 B per row and side group; 2:4: 16 B per row and
    // step, waves w and w + NW / 2 loading the same rows (same bytes to the
    // same place)
    o.mt = M24 ? off(tr.sa, kM) : off(tr.sp, kM) + 16 * (l & 1);
    // the first half of the waves: backbone scale rows 64 wq + l; the
    // second half: residual scale rows (the plain baseline: its scales,
    // twice)
    o.sa = off(tr.sa, kS);
    o.sw = 64 * wb + l < BNE ? w_row(64 * wb + l) * kS : kAbsent;
  };

  auto issue_main = [&](int s, MainT& st, const TileOff& o) {
    const uint32_t s64 = 64u * s, s32 = 32u * s;
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(r_dn, o.dn[j], s64, lds_addr(&st.a_dn[64 * (w + NW * j)]));
#pragma unroll
    for (int j = 0; j < WB; ++j) dma16(o.r_b, o.b[j], s64, lds_addr(&st.b[64 * (w + NW * j)]));
    if constexpr (!DENSE) dma16(r_sp, o.sp, s32, lds_addr(&st.a_sp[64 * w]));
    if constexpr (M24) dma16(r_mt, o.mt, 16u * s, lds_addr(&st.meta[64 * wq]));
  };
  auto issue_side = [&](int g, SideT& sd, const TileOff& o) {
    if constexpr (DENSE) {
      dma16(r_sdn, o.sa, 16u * g, lds_addr(&sd.s_dn[64 * wq]));   // waves w and w + NW / 2: same bytes
    } else if constexpr (M24) {
      dma16(r_sa, o.sa, 16u * g, lds_addr(first_half ? &sd.s_sp[64 * wq] : &sd.s_dn[64 * wq]));
    } else {
      dma16(r_mt, o.mt, 32u * g, lds_addr(&sd.meta[64 * w]));
      dma16(r_sa, o.sa, 16u * g, lds_addr(first_half ? &sd.s_sp[64 * wq] : &sd.s_dn[64 * wq]));
    }
    dma16(o.r_sb, o.sw, 16u * g, lds_addr(&sd.s_b[64 * wb]));   // NW = 8: waves w and w + 4 load the same bytes
  };

  const int wm0 = 32 * w, wn0 = 0;
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
  auto zero_acc = [&]() {
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int n = 0; n < FN; ++n) acc[f][n] = (v16f){};
  };

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
  auto compute_step = [&](const MainT& cur, const SideT& sd, int p) {
    read_step(cur, sd, p, sf);
    read_half(cur, hf, j0);
    mfma_half(sf, hf, j0);
    read_half(cur, hf, j1);
    mfma_half(sf, hf, j1);
  };
  // 256-row tiles, 4:8 at 224 columns and plain: a side group's scale and
  // metadata bytes are read once per group of four steps, each 16-byte
  // record (a column's or row's four steps) with one conflict-free 16-byte
  // read, instead of a 2- or 4-byte read per step (2- and 4-way bank
  // conflicts).  Of a record's dword p (step p) the lane needs bytes 2 kh
  // and 2 kh + 1; steps 2 q and 2 q + 1 are packed into one dword (low and
  // high half), so a step's two scale bytes sit in bytes 0 and 1 after a
  // shift, where the MFMA's op_sel picks them as before.  4:8 metadata: the
  // lane's dword of each step, from the row's two 16-byte halves.  2:4
  // tiles and 256-wide 4:8 tiles keep the per-step reads (the held bytes
  // would not fit their registers).
  constexpr bool kGroupSide = !M24 && (DENSE || FN <= 7);
  struct GroupFrag {
    uint32_t bs[FN][2], ssp[FM][2], sdn[FM][2], mt[FM][4];
  };
  auto read_group = [&](const SideT& sd, GroupFrag& Gf) {
    const uint32_t sel = kh ? 0x07060302u : 0x05040100u;   // bytes 2 kh, 2 kh + 1 of two dwords
#pragma unroll
    for (int n = 0; n < FN; ++n) {
      const uint4 v = sd.s_b[wn0 + 32 * n + lr];
      Gf.bs[n][0] = __builtin_amdgcn_perm(v.y, v.x, sel);
      Gf.bs[n][1] = __builtin_amdgcn_perm(v.w, v.z, sel);
    }
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      const int r = wm0 + 32 * f + lr;
      if constexpr (!DENSE && !M24) {
        const uint4 v = sd.s_sp[r];
        Gf.ssp[f][0] = __builtin_amdgcn_perm(v.y, v.x, sel);
        Gf.ssp[f][1] = __builtin_amdgcn_perm(v.w, v.z, sel);
        const uint4 m0 = sd.meta[2 * r], m1 = sd.meta[2 * r + 1];
        Gf.mt[f][0] = kh ? m0.y : m0.x;
        Gf.mt[f][1] = kh ? m0.w : m0.z;
        Gf.mt[f][2] = kh ? m1.y : m1.x;
        Gf.mt[f][3] = kh ? m1.w : m1.z;
      }
      const uint4 v = sd.s_dn[r];
      Gf.sdn[f][0] = __builtin_amdgcn_perm(v.y, v.x, sel);
      Gf.sdn[f][1] = __builtin_amdgcn_perm(v.w, v.z, sel);
    }
  };
  auto compute_step_g = [&](const MainT& cur, const GroupFrag& Gf, int p) {
    const int q = p >> 1, sh = 16 * (p & 1);
#pragma unroll
    for (int n = 0; n < FN; ++n) sf.bs[n] = Gf.bs[n][q] >> sh;
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      if constexpr (!DENSE) {
        sf.sp[f] = cur.a_sp[slot_sp(wm0 + 32 * f + lr, kh)];
        sf.mt[f] = Gf.mt[f][p];
        sf.ssp[f] = Gf.ssp[f][q] >> sh;
      }
      sf.sdn[f] = Gf.sdn[f][q] >> sh;
    }
    read_half(cur, hf, j0);
    mfma_half(sf, hf, j0);
    read_half(cur, hf, j1);
    mfma_half(sf, hf, j1);
  };

  // ---- epilogue: fp32 store of the accumulator tile
  auto epilogue = [&](const TileOff& o) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
      for (int n = 0; n < FN; ++n) {
        const int c = o.n0 + wn0 + 32 * n + lr;
        if (c >= D) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = o.m0 + wm0 + 32 * fm + 8 * (i >> 2) + 4 * kh + (i & 3);
          if (r < o.row_end) Y[(int64_t)r * ldy + c] = acc[fm][n][i];
        }
      }
    }
  };

  if constexpr (NS == 3) {
    // ---- 256-row tiles: one tile per workgroup
    int grp = 0, m0, n0, row_end = rows;
    if constexpr (!GROUPED) {
      band_tile(xcd_tile(blockIdx.x, ((rows + BM - 1) / BM) * tiles_n), m0, n0);
    } else {
      // the lookup's LDS lives in the last ring stage, which the first DMA
      // reaches only after the main loop's first barrier, when every thread
      // has read the result
      int* scan = reinterpret_cast<int*>(&lds[NS - 1].a_dn[0]);
      int e, start, cnt, b;
      if (!find_group_tile(blockIdx.x, n_groups, group_offsets, rows, BM, tiles_n, scan, scan + 256, e, start, cnt, b))
        return;                                         // surplus workgroup (uniform)
      grp = __builtin_amdgcn_readfirstlane(e);
      start = __builtin_amdgcn_readfirstlane(start);
      cnt = __builtin_amdgcn_readfirstlane(cnt);
      b = __builtin_amdgcn_readfirstlane(b);
      m0 = start + (b / tiles_n) * BM;
      n0 = (b % tiles_n) * BNE;
      row_end = start + cnt;
    }
    TileRows tr;
    tile_rows(m0, row_end, tr);
    TileOff o;
    tile_off(grp, m0, n0, row_end, tr, o);
    // a wave whose rows all lie past the tile's end (an expert's or the
    // matrix's last row tile) issues its share of the DMAs and takes every
    // barrier, but reads no fragments and issues no MFMAs, leaving its
    // SIMD's matrix core to the other wave there (uniform per wave)
    const bool live = m0 + wm0 < row_end;
    SHARQ_TL(blockIdx.x, 0, SHARQ_TL_NOW());
    SHARQ_TL_ID(blockIdx.x);
    zero_acc();
    issue_main(0, lds[0], o);
    issue_side(0, side[0], o);
    issue_main(min(1, KS - 1), lds[1], o);
    for (int g = 0; g < G; ++g) {
      const SideT& sd = side[g & 1];
      [[maybe_unused]] GroupFrag gf;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int s = 4 * g + p;
        if constexpr (PARTIAL)
          if (s >= KS) break;                             // partial last side group (uniform)
        // stage s (and at p = 0 side group g) landed; stage s+1 (and after
        // p = 2 side group g+1) may still be in flight.  After the barrier
        // every wave is past its reads of step s-1, whose buffer stage s+2
        // reuses.
        if (p == 3) wait_vm_lgkm0<NMAIN + NSIDE>();
        else wait_vm_lgkm0<NMAIN>();
        __builtin_amdgcn_s_barrier();
        if (s == 0) SHARQ_TL(blockIdx.x, 1, SHARQ_TL_NOW());
        issue_main(min(s + 2, KS - 1), lds[(s + 2) % NS], o);
        // side group g+1 replaces group g-1, last read at step 4 g - 1
        if (p == 2) issue_side(min(g + 1, G - 1), side[(g + 1) & 1], o);
        if constexpr (!kGroupSide) {
          if (live) compute_step(lds[s % NS], sd, p);
        } else if (live) {
          if (p == 0) read_group(sd, gf);
          compute_step_g(lds[s % NS], gf, p);
        }
      }
    }
    SHARQ_TL(blockIdx.x, 2, SHARQ_TL_NOW());
    wait_vm_lgkm0<0>();                                // no DMA may land after the tile ends
    if (live) epilogue(o);
    SHARQ_TL(blockIdx.x, 3, SHARQ_TL_NOW());
  } else {
    // ---- 128-row tiles, persistent: two workgroups per CU, each taking
    // every J-th tile of its XCD's stretch.  During a tile's last step the
    // next tile's first stage and side group are already in flight (into the
    // ring slots that step no longer reads), and its gathered rows were
    // loaded at the first step, so the lookup, the ring fill and the fp32
    // epilogue of consecutive tiles overlap instead of following one another
    // (the grid's workgroups stay resident, no relaunch per tile).
    int total;
    // grouped: inclusive tile prefix sums of experts 64 c + l in lane l (c <
    // 4, at most 256 experts), built once through the LDS of ring stage 1,
    // which the first DMA reaches only after the loop's first barrier
    int tb_incl[4];
    auto expert_rows = [&](int e, int& st, int& cnt) {
      st = min(max(group_offsets[e], 0), rows);
      cnt = min(max(group_offsets[e + 1], st), rows) - st;
    };
    if constexpr (GROUPED) {
      int* scan = reinterpret_cast<int*>(&lds[1].a_dn[0]);
      int te = 0;                                       // 256 threads: expert tid
      if (tid < n_groups) {
        int st, cnt;
        expert_rows(tid, st, cnt);
        te = ((cnt + BM - 1) / BM) * tiles_n;
      }
      scan[tid] = te;
      __syncthreads();
      for (int d = 1; d < 256; d <<= 1) {               // inclusive Hillis-Steele scan
        const int v = tid >= d ? scan[tid - d] : 0;
        __syncthreads();
        scan[tid] += v;
        __syncthreads();
      }
      total = __builtin_amdgcn_readfirstlane(scan[255]);
#pragma unroll
      for (int c = 0; c < 4; ++c) tb_incl[c] = scan[64 * c + l];
    } else {
      total = ((rows + BM - 1) / BM) * tiles_n;
    }
    // tile t -> expert, rows and columns (uniform)
    auto tile_of = [&](int t, int& grp, int& m0, int& n0, int& row_end) {
      if constexpr (GROUPED) {
        // the first expert whose inclusive tile prefix exceeds t (experts
        // with no tiles share their predecessor's prefix and are skipped)
        int cc = 3, lane = 0;
#pragma unroll
        for (int c = 3; c >= 0; --c) {
          const uint64_t m = __builtin_amdgcn_ballot_w64(t < tb_incl[c]);
          if (m) {
            cc = c;
            lane = __builtin_ctzll(m);
          }
        }
        int prev = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (c == cc && lane > 0) prev = __builtin_amdgcn_readlane(tb_incl[c], lane - 1);
          if (c + 1 == cc && lane == 0) prev = __builtin_amdgcn_readlane(tb_incl[c], 63);
        }
        grp = 64 * cc + lane;
        int st, cnt;
        expert_rows(grp, st, cnt);                      // uniform address: scalar loads
        const int b = t - prev;
        m0 = st + (b / tiles_n) * BM;
        n0 = (b % tiles_n) * BNE;
        row_end = st + cnt;
      } else {
        band_tile(t, m0, n0);
        grp = 0;
        row_end = rows;
      }
    };
    // this workgroup's tiles: lo + k for k = j, j + J, .. below len, where
    // the tile order is cut into NX stretches, one per XCD (workgroup b runs
    // on XCD b mod 8), and the J workgroups of stretch x interleave in it,
    // so together they sweep it front to back
    const int P = gridDim.x, NX = P < 8 ? P : 8, x = blockIdx.x % NX;
    const int J = (P - x + NX - 1) / NX;                // workgroups of stretch x
    const int q = total / NX, rr = total % NX;
    const int lo = x * q + min(x, rr), len = q + (x < rr ? 1 : 0);
    int k = blockIdx.x / NX;
    if (k >= len) return;                               // surplus workgroup (uniform)

    // the current tile (uniform) and its gathered rows; the per-lane DMA
    // offsets are recomputed where needed rather than kept for two tiles
    int cg, cm0, cn0, cre;
    tile_of(lo + k, cg, cm0, cn0, cre);
    TileRows ctr;
    tile_rows(cm0, cre, ctr);
    {
      TileOff o0;
      tile_off(cg, cm0, cn0, cre, ctr, o0);
      issue_main(0, lds[0], o0);
      issue_side(0, side[0], o0);
    }
    int sbase = 0, gbase = 0;                           // ring positions of the tile's step 0 / group 0
    while (true) {
      TileOff oc;
      tile_off(cg, cm0, cn0, cre, ctr, oc);
      k += J;
      const bool has_next = k < len;                    // uniform
      int ng = 0, nm0 = 0, nn0 = 0, nre = 0;
      if (has_next) tile_of(lo + k, ng, nm0, nn0, nre);
      TileRows ntr;
      // as in the 256-row tile: a wave past the tile's end issues its DMAs
      // and takes the barriers, but no fragment reads or MFMAs
      const bool live = cm0 + wm0 < cre;
      const int cur_t = lo + k - J;                     // this tile's index
      SHARQ_TL(cur_t, 0, SHARQ_TL_NOW());
      SHARQ_TL_ID(cur_t);
      zero_acc();
      for (int g = 0; g < G; ++g) {
        const SideT& sd = side[(gbase + g) & 1];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int s = 4 * g + p;
          if constexpr (PARTIAL)
            if (s >= KS) break;                           // partial last side group (uniform)
          const bool last = s == KS - 1;
          // two stages: stage s (and at p = 0 side group g) landed.  Only
          // side group g+1, issued at p = 0 after stage s, may still be in
          // flight at p = 1; the last group issues none (the next tile's
          // group 0 goes out with its stage 0 at the tile's last step).
          // After the barrier every wave is past step s-1, whose ring slot
          // stage s+1 reuses, and at p = 0 past step 4 g - 1, the last
          // reader of the side slot group g+1 reuses.
          if (p == 1 && g + 1 < G) wait_vm_lgkm0<NSIDE>();
          else wait_vm_lgkm0<0>();
          __builtin_amdgcn_s_barrier();
          // the next tile's gathered rows: loaded here, first read at this
          // tile's last step, after its wait for every load
          if (s == 0) SHARQ_TL(cur_t, 1, SHARQ_TL_NOW());
          if (s == 0 && has_next) tile_rows(nm0, nre, ntr);
          if (!last) {
            issue_main(s + 1, lds[(sbase + s + 1) & 1], oc);
          } else if (has_next) {
            // the next tile's stage 0 into the slot step s-1 used, and its
            // group 0 into the slot of this tile's group G-2 (or, with one
            // group per tile, the previous tile's last group)
            TileOff on;
            tile_off(ng, nm0, nn0, nre, ntr, on);
            issue_main(0, lds[(sbase + s + 1) & 1], on);
            issue_side(0, side[(gbase + G) & 1], on);
          }
          if (p == 0 && g + 1 < G) issue_side(g + 1, side[(gbase + g + 1) & 1], oc);
          if (live) compute_step(lds[(sbase + s) & 1], sd, p);
        }
      }
      SHARQ_TL(cur_t, 2, SHARQ_TL_NOW());
      if (!has_next) wait_vm_lgkm0<0>();               // no DMA may land after the workgroup ends
      if (live) epilogue(oc);
      SHARQ_TL(cur_t, 3, SHARQ_TL_NOW());
      if (!has_next) break;
      sbase += KS;
      gbase += G;
      cg = ng;
      cm0 = nm0;
      cn0 = nn0;
      cre = nre;
      ctr = ntr;
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
template <bool FUSED, bool M24 = false, int MT = 1>
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
  constexpr int NR = 16 * MT;
  const size_t lds = (size_t)(K / 32 + 1) * NR * 16 + (size_t)(NR * KBP + 16) / 16 * 16 +
                     (size_t)NK * CG * MT * 64 * 4 * sizeof(float);
  if (lds > 160 * 1024) return hipErrorInvalidValue;   // callers keep K within decode_max_k(rows)
  const int n_gemm = (D + 16 * CG - 1) / (16 * CG);
  // fused: the producers are workgroups 0, 8, .., 8 (rows - 1)
  dim3 grid(FUSED ? std::max(n_gemm, 8 * (rows - 1) + 1) : n_gemm), block(64 * NK * CG);
#define L(NK_, CG_, J_)                                                                                                 \
  hipLaunchKernelGGL((linear_mx_decode<NK_, CG_, J_, FUSED, M24, MT>), grid, block, lds, s, bb_codes, bb_meta, bb_scale, \
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
    case 81601:                                      // K > 8192: one tile of 8 rows only
      if constexpr (MT == 1) L(16, 1, 8);
      else return hipErrorInvalidValue;
      break;
    case 40801: L(8, 1, 4); break;
    default: return hipErrorInvalidValue;
  }
#undef L
  return hipGetLastError();
}
}  // namespace

// the batch kernel (4:8 backbone) with MT = 2 (16 rows), 4 (32) or 8 (64)
// MFMA tiles; column groups as in the decode kernel (the widest with at least
// 200 workgroups), K chunks split over the compute waves of a column group
template <int MT>
hipError_t launch_batch(const uint8_t* bb_codes, const uint8_t* bb_meta, const uint8_t* bb_scale,
                        const uint8_t* res_codes, const uint8_t* res_scale, const int32_t* row_index, int rows,
                        int act_rows, int K, const uint8_t* payload, const uint8_t* wscale, int D, float* Y, int64_t ldy,
                        hipStream_t s) {
  // column groups as in the decode kernel; four compute waves (NK = 4 / CG
  // K-splits) and four staging waves.  Steps per compute wave and chunk JC
  // from a sweep over the Llama-3.1-8B decode shapes at 17-64 rows (JC = 8,
  // and weights four chunks ahead instead of two, measured slower): 4, or 2
  // for MT = 8 below four column groups
  int CG = 1;
  while (CG < 4 && (D + 32 * CG - 1) / (32 * CG) >= 200) CG *= 2;
  const int NK = 4 / CG, JC = (MT == 8 && CG < 4) ? 2 : 4;
  const int KC = NK * JC, BC = 4 * KC, SP = BC + 4, NR = 16 * MT;
  const size_t stage = (size_t)2 * NR * (BC + 1) * 16 + (size_t)2 * NR * SP, red = (size_t)4 * MT * 64 * 4 * sizeof(float);
  const size_t lds = std::max(stage, red);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  dim3 grid((D + 16 * CG - 1) / (16 * CG)), block(64 * (4 + kBatchStagingWaves));
#define L(CG_, NK_, JC_)                                                                                                 \
  hipLaunchKernelGGL((linear_mx_batch<MT, CG_, NK_, JC_>), grid, block, lds, s, bb_codes, bb_meta, bb_scale, res_codes, \
                     res_scale, row_index, rows, act_rows, K, payload, wscale, D, Y, ldy)
  switch (CG) {
    case 4: L(4, 1, 4); break;
    case 2: L(2, 2, MT == 8 ? 2 : 4); break;
    default: L(1, 4, MT == 8 ? 2 : 4); break;
  }
#undef L
  return hipGetLastError();
}

// largest K the decode kernel stages for `rows` rows (8 rows: one MFMA tile;
// 9-16 rows: two, twice the staged operand)
int decode_max_k(int rows) { return rows <= 8 ? kDecodeMaxK : (rows <= 16 ? kDecodeMaxK16 : 0); }

hipError_t launch_prepare_linear_mx(const void* X, bool bf16, int T, int K, int64_t ldx, const float* gamma, float eps,
                                    uint8_t* bb_codes, uint8_t* bb_meta, uint8_t* bb_scale, uint8_t* res_codes,
                                    uint8_t* res_scale, const uint8_t* payload, const uint8_t* wscale, int D, float* Y,
                                    int64_t ldy, uint32_t* sync, hipStream_t s) {
  if (T < 1 || K > decode_max_k(T)) return hipErrorInvalidValue;
  const FusedPrep fp{X, bf16 ? 1 : 0, ldx, gamma, eps, sync};
  if (T > 8)
    return launch_decode<true, false, 2>(bb_codes, bb_meta, bb_scale, res_codes, res_scale, nullptr, T, T, K, payload,
                                         wscale, D, Y, ldy, fp, s);
  return launch_decode<true>(bb_codes, bb_meta, bb_scale, res_codes, res_scale, nullptr, T, T, K, payload, wscale, D, Y,
                             ldy, fp, s);
}

namespace {
// rows of the plain (single-expert) tile: 256 (one workgroup per tile) or
// 128 (a persistent grid, two workgroups per CU)
constexpr int kPlainTileRows = 256;

template <bool M24>
hipError_t launch_linear_mx_impl(const uint8_t* bb_codes, const uint8_t* bb_meta, const uint8_t* bb_scale,
                                 const uint8_t* res_codes, const uint8_t* res_scale, const int32_t* row_index, int rows,
                                 int act_rows, int K, const uint8_t* payload, const uint8_t* wscale, int D, int n_groups,
                                 const int32_t* group_offsets, float* Y, int64_t ldy, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (n_groups == 1 && rows <= 8 && K <= kDecodeMaxK)
    return launch_decode<false, M24>(bb_codes, bb_meta, bb_scale, res_codes, res_scale, row_index, rows, act_rows, K, payload,
                                wscale, D, Y, ldy, FusedPrep{}, s);
  // 17-64 rows: the batch kernel, the weight read once for all rows (the
  // chunks of decode launches below read it once per chunk).  Llama-3.1-8B
  // decode shapes 4096 x 4096 / 4096 x 14336 / 14336 x 4096: batch kernel
  // 9.2 / 16.2 / 19.9 us at 32 rows and 13.2 / 21.4 / 30.5 us at 64; decode
  // launches 12.4 / 20.1 / 34.1 and 24.1 / 39.0 / 67.2 us
  if (n_groups == 1 && rows > 8 && rows <= 16 && K > kDecodeMaxK16 && !M24)
    return launch_batch<2>(bb_codes, bb_meta, bb_scale, res_codes, res_scale, row_index, rows, act_rows, K, payload,
                           wscale, D, Y, ldy, s);
  if (n_groups == 1 && rows > 16 && rows <= 64 && !M24) {
    return rows <= 32 ? launch_batch<4>(bb_codes, bb_meta, bb_scale, res_codes, res_scale, row_index, rows, act_rows, K,
                                        payload, wscale, D, Y, ldy, s)
                      : launch_batch<8>(bb_codes, bb_meta, bb_scale, res_codes, res_scale, row_index, rows, act_rows, K,
                                        payload, wscale, D, Y, ldy, s);
  }
  if (n_groups == 1 && rows <= 64 && K <= kDecodeMaxK) {
    // 9-64 rows: the decode kernel on chunks of 16 rows (two MFMA tiles,
    // K <= 7168) or 8 rows (one tile, K <= 16384), one launch per chunk,
    // each streaming the weight once.  Measured against the skinny kernel
    // (Llama-3.1-8B decode shapes, 4096 x 4096 / 4096 x 14336 / 14336 x 4096):
    // 16 rows 6.6 / 11.0 / 18.0 (two 8-row launches) against - / - / 30.0 us;
    // the skinny kernel took 19.9 / 73.6 / 50.6 us at 32 rows and 32.4 /
    // 108.5 / 93.5 us at 64.
    const int chunk = K <= kDecodeMaxK16 ? 16 : 8;
    for (int r0 = 0; r0 < rows; r0 += chunk) {
      const int n = std::min(chunk, rows - r0);
      const int64_t o = row_index ? 0 : r0;             // gathered rows: row_index[r0 ..] instead
      const int32_t* ri = row_index ? row_index + r0 : nullptr;
      const uint8_t *bc = bb_codes + o * (K >> 2), *bm = bb_meta + o * (K >> (M24 ? 3 : 4)),
                    *bs = bb_scale + o * (K >> 5), *rc = res_codes + o * (K >> 1), *rs = res_scale + o * (K >> 5);
      const int ar = act_rows - (int)o;
      float* y = Y + (int64_t)r0 * ldy;
      const hipError_t e =
          n > 8 ? launch_decode<false, M24, 2>(bc, bm, bs, rc, rs, ri, n, ar, K, payload, wscale, D, y, ldy, FusedPrep{}, s)
                : launch_decode<false, M24>(bc, bm, bs, rc, rs, ri, n, ar, K, payload, wscale, D, y, ldy, FusedPrep{}, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
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
  const int ncu = num_cus_gemm();
  if (n_groups == 1) {
    // tile width 256 or 224: the one with fewer rounds x width over the CUs
    // (256 rows: at 4096 x 4096 x 14336 the 128-row tile, two workgroups
    // per CU, measured the same, 278.9 against 277.5-280.2 us, and stages
    // each weight column twice as often)
    constexpr int PBM = kPlainTileRows;
    constexpr int slots = PBM == 256 ? 1 : 2;          // workgroups per CU
    const int tiles_m = (rows + PBM - 1) / PBM;
    const int t256 = tiles_m * ((D + 255) / 256), t224 = tiles_m * ((D + 223) / 224);
    const int ns = slots * ncu;
    const bool narrow = (int64_t)((t224 + ns - 1) / ns) * 224 < (int64_t)((t256 + ns - 1) / ns) * 256;
    const int tiles = narrow ? t224 : t256;
    // 256 rows: one workgroup per tile; 128 rows: a persistent grid
    const int grid = PBM == 256 ? tiles : std::min(tiles, ns);
#define T8(BNE_, PARTIAL_)                                                                                            \
  hipLaunchKernelGGL((linear_mx_tile8<PBM, BNE_, false, false, M24, PARTIAL_>), dim3(grid), dim3(2 * PBM), 0, s,      \
                     bb_codes, bb_meta, bb_scale, res_codes, res_scale, row_index, rows, act_rows, K, payload, wscale,  \
                     D, 1, nullptr, Y, ldy)
    if (narrow) {
      if (partial) T8(224, true);
      else T8(224, false);
    } else {
      if (partial) T8(256, true);
      else T8(256, false);
    }
#undef T8
  } else if (n_groups <= 256) {
    // grouped: 128 x 256 tiles, two workgroups per CU: one workgroup's fp32
    // epilogue overlaps the other's MFMAs, and an expert's last row tile
    // wastes at most 127 rows.  Measured at the Qwen3-30B-A3B MoE shapes
    // (128 experts, top-8 of 4096 tokens): up 111.5 -> 90.3 us, down
    // 142.8 -> 130.0 us against the 256-row tile.  A persistent grid of two
    // workgroups per CU (at most the bound on the tile count); the expert
    // table of up to 256 experts sits in registers.
    constexpr int GBM = 128;
    const int bound = ((rows + GBM - 1) / GBM + n_groups) * ((D + 255) / 256);
    const int grid = std::min(bound, 2 * ncu);
#define T8G(PARTIAL_)                                                                                                 \
  hipLaunchKernelGGL((linear_mx_tile8<GBM, 256, false, true, M24, PARTIAL_>), dim3(grid), dim3(2 * GBM), 0, s, bb_codes, \
                     bb_meta, bb_scale, res_codes, res_scale, row_index, rows, act_rows, K, payload, wscale, D, n_groups, \
                     group_offsets, Y, ldy)
    if (partial) T8G(true);
    else T8G(false);
#undef T8G
  } else {
    // more than 256 experts: 256 x 256 tiles, one workgroup per tile (a
    // bound on the tile count; surplus workgroups return at once), each
    // locating its expert by a workgroup prefix sum
    constexpr int GBM = 256;
    const int bound = ((rows + GBM - 1) / GBM + n_groups) * ((D + 255) / 256);
#define T8G(PARTIAL_)                                                                                                 \
  hipLaunchKernelGGL((linear_mx_tile8<GBM, 256, false, true, M24, PARTIAL_>), dim3(bound), dim3(2 * GBM), 0, s, bb_codes, \
                     bb_meta, bb_scale, res_codes, res_scale, row_index, rows, act_rows, K, payload, wscale, D, n_groups, \
                     group_offsets, Y, ldy)
    if (partial) T8G(true);
    else T8G(false);
#undef T8G
  }
  return hipGetLastError();
}
}  // namespace

// ---- tile timeline accessors (tracing build; elsewhere they report absence)
bool timeline_built() {
#ifdef SHARQ_TIMELINE
  return true;
#else
  return false;
#endif
}
size_t timeline_records() { return kTimelineRecords; }
hipError_t timeline_clear() {
#ifdef SHARQ_TIMELINE
  static uint64_t zeros[kTimelineRecords * 8];
  return hipMemcpyToSymbol(HIP_SYMBOL(g_timeline), zeros, sizeof(zeros), 0, hipMemcpyHostToDevice);
#else
  return hipErrorNotSupported;
#endif
}
hipError_t timeline_read(uint64_t* host, size_t words) {
#ifdef SHARQ_TIMELINE
  if (words > (size_t)kTimelineRecords * 8) words = (size_t)kTimelineRecords * 8;
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_timeline), words * sizeof(uint64_t), 0, hipMemcpyDeviceToHost);
#else
  (void)host;
  (void)words;
  return hipErrorNotSupported;
#endif
}

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
    hipLaunchKernelGGL((linear_mx_tile8<256, 224, true>), dim3(t224), dim3(512), 0, s, nullptr, nullptr, nullptr, codes,
                       scales, nullptr, rows, rows, K, payload, wscale, D, 1, nullptr, Y, ldy);
  else
    hipLaunchKernelGGL((linear_mx_tile8<256, 256, true>), dim3(t256), dim3(512), 0, s, nullptr, nullptr, nullptr, codes,
                       scales, nullptr, rows, rows, K, payload, wscale, D, 1, nullptr, Y, ldy);
  return hipGetLastError();
}

}  // namespace sharq
