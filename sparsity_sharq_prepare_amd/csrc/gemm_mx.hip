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

namespace sharq {

namespace {

SHARQ_DEV v8i as_v8i(uint4 v) {
  v8i r = {(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  return r;
}

SHARQ_DEV v4f mfma_fp4(uint4 a, uint4 b, v4f c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(as_v8i(a), as_v8i(b), c, 4, 4, 0, (int)sa, 0, (int)sb);
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

}  // namespace

// ============================================================================
// skinny (decode) kernel
// ============================================================================
// grid.x = ceil(D / 16); blockDim = 64 * NW.  Wave w takes K-steps
// w, w + NW, ... in batches of J whose loads are all issued before the MFMAs.
template <int MT, int J>
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
            av[m][j].z = *reinterpret_cast<const uint16_t*>(bb_meta + arow[m] * (K >> 4) + 2 * (int64_t)kb);
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
        if (!dn) a = expand4(a.x, a.y, a.z);
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
// tile kernel (prefill / grouped)
// ============================================================================
namespace {

constexpr int kBN = 256;
constexpr int kRowBytes = 64;            // 128 FP4 values per staged row

// 16-byte slot of (row, chunk) in a staged tile: XOR swizzle so that the 16
// rows an MFMA fragment read touches fall in distinct banks
SHARQ_DEV int slot(int row, int q) { return row * 4 + (q ^ (((row >> 1) ^ (row >> 3)) & 3)); }

template <int BM>
struct Stage {
  uint4 a_sp[BM * 4];
  uint4 a_dn[BM * 4];
  uint4 b[kBN * 4];
  uint32_t s_sp[BM];
  uint32_t s_dn[BM];
  uint32_t s_b[kBN];
};

}  // namespace

template <int BM, bool GROUPED>
__global__ __launch_bounds__(256, 1) void linear_mx_tile(
    const uint8_t* __restrict__ bb_codes, const uint8_t* __restrict__ bb_meta, const uint8_t* __restrict__ bb_scale,
    const uint8_t* __restrict__ res_codes, const uint8_t* __restrict__ res_scale, const int32_t* __restrict__ row_index,
    int rows, int act_rows, int K, const uint8_t* __restrict__ payload, const uint8_t* __restrict__ wscale, int D,
    int n_groups, const int32_t* __restrict__ group_offsets, float* __restrict__ Y, int64_t ldy) {
  constexpr int WM = BM / 2, FM = WM / 16, FN = 8, UA = BM / 64;
  __shared__ Stage<BM> st[2];
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int tiles_n = (D + kBN - 1) / kBN;

  // ---- tile -> (group, first row, row end, first column)
  int grp = 0, m0, row_end, n0;
  if (!GROUPED) {
    const int tiles_m = (rows + BM - 1) / BM;
    const int nt = tiles_m * tiles_n;
    int b = blockIdx.x;
    if ((nt & 7) == 0) b = (b & 7) * (nt >> 3) + (b >> 3);   // consecutive tiles on one XCD
    const int tm = b % tiles_m, tn = b / tiles_m;
    m0 = tm * BM;
    row_end = rows;
    n0 = tn * kBN;
  } else {
    int b = blockIdx.x;
    int e = 0, start = 0, cnt = 0;
    for (; e < n_groups; ++e) {
      start = min(max(group_offsets[e], 0), rows);
      cnt = min(max(group_offsets[e + 1], start), rows) - start;
      const int te = ((cnt + BM - 1) / BM) * tiles_n;
      if (b < te) break;
      b -= te;
    }
    if (e >= n_groups) return;                          // surplus workgroup (uniform)
    grp = e;
    const int tm = b / tiles_n, tn = b % tiles_n;
    m0 = start + tm * BM;
    row_end = start + cnt;
    n0 = tn * kBN;
  }

  const int KS = K >> 7;
  const int64_t kA = K >> 2, kM = K >> 4, kS = K >> 5, kR = K >> 1;
  const uint8_t* pay = payload + (int64_t)grp * D * kR;
  const uint8_t* wsc = wscale + (int64_t)grp * D * kS;

  // ---- per-thread staging rows (A: rows u >> 2 of units u = tid + 256 i)
  int64_t arow[UA];
  bool aok[UA];
#pragma unroll
  for (int i = 0; i < UA; ++i) {
    const int r = m0 + ((tid + 256 * i) >> 2);
    aok[i] = r < row_end;
    arow[i] = aok[i] ? gather_row(row_index, r, act_rows) : 0;
  }
  const int q = tid & 3;
  int64_t brow[4];
  bool bok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = n0 + ((tid + 256 * i) >> 2);
    bok[i] = c < D;
    brow[i] = bok[i] ? c : 0;
  }
  const bool srow_a = tid < BM;
  const int sr = m0 + tid;
  const bool sa_ok = srow_a && sr < row_end;
  const int64_t sarow = sa_ok ? gather_row(row_index, sr, act_rows) : 0;
  const bool sb_ok = n0 + tid < D;
  const int64_t sbrow = sb_ok ? n0 + tid : 0;

  // ---- prefetch registers
  uint2 pc[UA];
  uint32_t pm[UA];
  uint4 pd[UA];
  uint4 pb[4];
  uint32_t ps_sp = 0, ps_dn = 0, ps_b = 0;

  auto load_step = [&](int s) {
#pragma unroll
    for (int i = 0; i < UA; ++i) {
      pc[i] = make_uint2(0, 0);
      pm[i] = 0;
      pd[i] = make_uint4(0, 0, 0, 0);
      if (aok[i]) {
        pc[i] = *reinterpret_cast<const uint2*>(bb_codes + arow[i] * kA + 32 * (int64_t)s + 8 * q);
        pm[i] = *reinterpret_cast<const uint16_t*>(bb_meta + arow[i] * kM + 8 * (int64_t)s + 2 * q);
        pd[i] = *reinterpret_cast<const uint4*>(res_codes + arow[i] * kR + 64 * (int64_t)s + 16 * q);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pb[i] = make_uint4(0, 0, 0, 0);
      if (bok[i]) pb[i] = *reinterpret_cast<const uint4*>(pay + brow[i] * kR + 64 * (int64_t)s + 16 * q);
    }
    ps_sp = 0x7F7F7F7Fu;
    ps_dn = 0x7F7F7F7Fu;
    ps_b = 0x7F7F7F7Fu;
    if (sa_ok) {
      ps_sp = *reinterpret_cast<const uint32_t*>(bb_scale + sarow * kS + 4 * (int64_t)s);
      ps_dn = *reinterpret_cast<const uint32_t*>(res_scale + sarow * kS + 4 * (int64_t)s);
    }
    if (sb_ok) ps_b = *reinterpret_cast<const uint32_t*>(wsc + sbrow * kS + 4 * (int64_t)s);
  };
  auto store_step = [&](Stage<BM>& S) {
#pragma unroll
    for (int i = 0; i < UA; ++i) {
      const int row = (tid + 256 * i) >> 2;
      S.a_sp[slot(row, q)] = expand4(pc[i].x, pc[i].y, pm[i]);
      S.a_dn[slot(row, q)] = pd[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) S.b[slot((tid + 256 * i) >> 2, q)] = pb[i];
    if (srow_a) {
      S.s_sp[tid] = ps_sp;
      S.s_dn[tid] = ps_dn;
    }
    S.s_b[tid] = ps_b;
  };

  const int wm0 = (w >> 1) * WM, wn0 = (w & 1) * 128;
  const int kq = l >> 4, lr = l & 15;
  v4f acc[FM][FN];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int n = 0; n < FN; ++n) acc[f][n] = (v4f){0.f, 0.f, 0.f, 0.f};

  load_step(0);
  store_step(st[0]);
  __syncthreads();
  for (int s = 0; s < KS; ++s) {
    const bool more = s + 1 < KS;
    if (more) load_step(s + 1);
    const Stage<BM>& S = st[s & 1];
    uint4 bf[FN];
    uint32_t bs[FN];
#pragma unroll
    for (int n = 0; n < FN; ++n) {
      const int c = wn0 + 16 * n + lr;
      bf[n] = S.b[slot(c, kq)];
      bs[n] = (S.s_b[c] >> (8 * kq)) & 0xFFu;
    }
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      const int r = wm0 + 16 * f + lr;
      const uint4 asp = S.a_sp[slot(r, kq)];
      const uint4 adn = S.a_dn[slot(r, kq)];
      const uint32_t ssp = (S.s_sp[r] >> (8 * kq)) & 0xFFu;
      const uint32_t sdn = (S.s_dn[r] >> (8 * kq)) & 0xFFu;
#pragma unroll
      for (int n = 0; n < FN; ++n) acc[f][n] = mfma_fp4(asp, bf[n], acc[f][n], ssp, bs[n]);
#pragma unroll
      for (int n = 0; n < FN; ++n) acc[f][n] = mfma_fp4(adn, bf[n], acc[f][n], sdn, bs[n]);
    }
    if (more) store_step(st[(s + 1) & 1]);
    __syncthreads();
  }

  // ---- epilogue: fp32 store of the single accumulator tile
#pragma unroll
  for (int f = 0; f < FM; ++f) {
#pragma unroll
    for (int n = 0; n < FN; ++n) {
      const int c = n0 + wn0 + 16 * n + lr;
      if (c >= D) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = m0 + wm0 + 16 * f + 4 * kq + i;
        if (r < row_end) Y[(int64_t)r * ldy + c] = acc[f][n][i];
      }
    }
  }
}

// ============================================================================
// host launchers
// ============================================================================
hipError_t launch_linear_mx(const uint8_t* bb_codes, const uint8_t* bb_meta, const uint8_t* bb_scale,
                            const uint8_t* res_codes, const uint8_t* res_scale, const int32_t* row_index, int rows,
                            int act_rows, int K, const uint8_t* payload, const uint8_t* wscale, int D, int n_groups,
                            const int32_t* group_offsets, float* Y, int64_t ldy, hipStream_t s) {
  if (rows == 0) return hipSuccess;
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
  hipLaunchKernelGGL((linear_mx_skinny<MT_, J_>), grid, block, lds, s, bb_codes, bb_meta, bb_scale, res_codes, \
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
  const int tiles_n = (D + kBN - 1) / kBN;
  if (n_groups == 1) {
    const int tiles_m = (rows + 255) / 256;
    hipLaunchKernelGGL((linear_mx_tile<256, false>), dim3(tiles_m * tiles_n), dim3(256), 0, s, bb_codes, bb_meta,
                       bb_scale, res_codes, res_scale, row_index, rows, act_rows, K, payload, wscale, D, 1, group_offsets, Y,
                       ldy);
  } else {
    const int bound = ((rows + 127) / 128 + n_groups) * tiles_n;
    hipLaunchKernelGGL((linear_mx_tile<128, true>), dim3(bound), dim3(256), 0, s, bb_codes, bb_meta, bb_scale,
                       res_codes, res_scale, row_index, rows, act_rows, K, payload, wscale, D, n_groups, group_offsets, Y,
                       ldy);
  }
  return hipGetLastError();
}

}  // namespace sharq
