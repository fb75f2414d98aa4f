// Matrix-core GEMMs of the block: out = epilogue(A . B^T) with A = activations [M, K]
// (tokens) and B = weights [N, K], both K-contiguous.
//
//  - W8A8: v_mfma_i32_16x16x64_i8, exact int32 accumulation, dequantised in the epilogue
//    with the per-token activation scale and the per-output-channel weight scale
//    ("h3-metal: Apple Silicon을 위한 네이티브 MiniMax-H3 추론", section "Int8 양자화";
//    "맥북에서 AI 영상 생성 모델 돌리기 …", section "int8 이 뭔가요").
//  - BF16 baseline: v_mfma_f32_16x16x32_bf16 on the dense bf16 weights.
//
// Both instructions take 16 bytes of K per lane per operand, so one byte-addressed tile
// pipeline serves both: a K step is 64 bytes (64 int8 or 32 bf16 elements).
//
// Two kernels share the epilogues. gemm_w4_kernel (int8 weights in the tiled layout of
// h3k_tile_weights, the block's path): one wave per SIMD, accumulators in AGPRs, weights
// straight to registers, tokens through LDS. gemm_pp_kernel (row-major weights, bf16
// operands, the raw int8 GEMM entry point): eight waves in two ping-pong groups, both
// operands through LDS. Their results are bit-identical.
//
// The matrix-core output is computed transposed (weights are the MFMA "A" operand): a
// lane then holds four consecutive output channels of one token, which is what the
// fused epilogues want -- RoPE rotates channel pairs (2i, 2i+1) inside one lane, and the
// head-major Q/K scatter stores 4 consecutive head dims per lane. Epilogues:
//   RAW_I32  int32 accumulators (exactness check of the main loop)
//   QKV      dequant, 3D RoPE on Q and K, scatter to head-major Q, K [H, L, Dh] and
//            transposed V [H, Dh, L] (the layout attention consumes), in fp16 (the
//            attention's operand type; bf16 when attention runs on bf16 operands)
//   GELU     dequant + exact erf GELU (MLP up)
//   RESID    dequant + gated residual out = res + gate[n] * y (out-proj, MLP down)
#include "h3k_internal.h"

#include <type_traits>

namespace h3k {

template <bool OUTF32>
__device__ __forceinline__ void store4(void *base, int64_t idx, float y0, float y1, float y2,
                                       float y3) {
  if constexpr (OUTF32) {
    *(float4 *)((float *)base + idx) = make_float4(y0, y1, y2, y3);
  } else {
    *(uint2 *)((uint16_t *)base + idx) = make_uint2(pack_bf2(y0, y1), pack_bf2(y2, y3));
  }
}
template <bool OUTF32>
__device__ __forceinline__ void load4(const void *base, int64_t idx, float v[4]) {
  if constexpr (OUTF32) {
    float4 t = *(const float4 *)((const float *)base + idx);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  } else {
    uint2 t = *(const uint2 *)((const uint16_t *)base + idx);
    v[0] = __uint_as_float(t.x << 16);
    v[1] = __uint_as_float(t.x & 0xffff0000u);
    v[2] = __uint_as_float(t.y << 16);
    v[3] = __uint_as_float(t.y & 0xffff0000u);
  }
}
template <bool OUTF32>
__device__ __forceinline__ void store1(void *base, int64_t idx, float y) {
  if constexpr (OUTF32)
    ((float *)base)[idx] = y;
  else
    ((uint16_t *)base)[idx] = f2bf(y);
}

// Exact (erf) GELU, z Phi(z), written as max(z, 0) - |z| erfc(|z| / sqrt 2) / 2 (the same
// value for either sign of z, with no 1 + erf cancellation for negative z). erfc without
// branches: Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26,
// erfc(a) = (a1 t + ... + a5 t^5) e^(-a^2), t = 1 / (1 + p a), a >= 0, absolute error
// <= 1.5e-7; here a = |z| / sqrt 2, with 1/2 folded into the coefficients and 1 / sqrt 2
// into p. The hardware reciprocal and exp2 add about an ulp each; in fp32 the GELU error
// stays below 1e-7 (1 + |z|).
__device__ __forceinline__ float gelu_erf(float z) {
  constexpr float kP = 0.3275911f * 0.70710678118654752f;
  constexpr float kE = -0.5f * 1.4426950408889634f;  // e^(-z^2 / 2) = 2^(kE z^2)
  const float az = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(fmaf(kP, az, 1.0f));
  float poly = fmaf(0.5f * 1.061405429f, t, 0.5f * -1.453152027f);
  poly = fmaf(poly, t, 0.5f * 1.421413741f);
  poly = fmaf(poly, t, 0.5f * -0.284496736f);
  poly = fmaf(poly, t, 0.5f * 0.254829592f);
  poly *= t;
  const float e = __builtin_amdgcn_exp2f((z * z) * kE);
  return fmaf(-az, poly * e, fmaxf(z, 0.f));
}
// fp64 GELU of the fp32 debug path: z Phi(z) = z erfc(-z / sqrt 2) / 2 with the math
// library's double erfc (no cancellation for negative z either)
__device__ __forceinline__ double gelu_erf(double z) {
  return 0.5 * z * erfc(z * -0.70710678118654752440);
}

// Table offsets of token l's three axes: pair i of head_dim turns by tbl[ofs.x + i] (i < Pt),
// tbl[ofs.y + i] (Pt <= i < Pt + Ph) or tbl[ofs.z + i] (the rest); the pair-index bases are
// folded into the offsets.
__device__ __forceinline__ int3 rope_offsets(const RopeGeom &g, int64_t l) {
  const int hw = g.Hg * g.Wg;
  const int t = (int)(l / hw);
  const int rem = (int)(l - (int64_t)t * hw);
  const int h = rem / g.Wg;
  const int w = rem - h * g.Wg;
  return make_int3(t * g.Pt, g.base_h + h * g.Ph - g.Pt, g.base_w + w * g.Pw - g.Pt - g.Ph);
}
template <typename CS>
__device__ __forceinline__ CS rope_cs(const void *tbl, const RopeGeom &g, int i, int3 ofs) {
  const int e = i < g.Pt ? ofs.x + i : (i < g.Pt + g.Ph ? ofs.y + i : ofs.z + i);
  return ((const CS *)tbl)[e];
}

template <bool BF16>
__device__ __forceinline__ auto mma(v4i b, v4i a, typename std::conditional<BF16, v4f, v4i>::type c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, b),
                                                   __builtin_bit_cast(v8bf, a), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(b, a, c, 0, 0, 0);
}

// Origin of tile t. The hardware places work-group b on XCD b % 8, and a persistent
// work-group b takes tiles b, b + G, b + 2G, ... (G, the grid, a multiple of 8 or the tile
// count), so t % 8 is the XCD. Each XCD gets a contiguous range of logical tiles, walked in
// groups of 8 M-tiles so that concurrent work-groups of an XCD share weight and activation
// tiles in that XCD's L2.
template <int BN, int BM>
__device__ __forceinline__ void tile_origin(const GemmArgs &a, int64_t t, int64_t &m0, int &n0) {
  const int n_tiles = a.N / BN;
  const int64_t m_tiles = (a.M + BM - 1) / BM;
  const int64_t nwg = (int64_t)n_tiles * m_tiles;
  if ((nwg & 7) == 0) t = (t & 7) * (nwg >> 3) + (t >> 3);
  constexpr int GM = 8;
  const int64_t group = t / ((int64_t)GM * n_tiles);
  const int64_t first_m = group * GM;
  const int64_t gsize = (m_tiles - first_m) < GM ? (m_tiles - first_m) : GM;
  const int64_t in_group = t - group * GM * n_tiles;
  m0 = (first_m + in_group % gsize) * BM;
  n0 = (int)(in_group / gsize) * BN;
}

// Per-column-block operands of the epilogue (one 16-channel block i of a wave's tile),
// loaded ahead of use so that the global-memory latency of one block overlaps the
// arithmetic and stores of the blocks before it. Fields an epilogue does not use are never
// touched and take no registers. F64: the fp32-output (debug) instantiations, whose
// epilogue arithmetic is fp64 and whose RoPE table holds fp64 (cos, sin).
template <int TM, bool RESF32, bool F64>
struct EpiChunk {
  float sw[4];                  // weight scales of the lane's 4 channels
  float g[4];                   // gate (RESID)
  uint32_t r[TM][RESF32 ? 4 : 2];  // residual bits, fp32 or packed bf16 (RESID)
  typename std::conditional<F64, double2, float2>::type cs[TM][2];  // RoPE (cos, sin) of the
                                                                     // lane's two pairs (QKV)
};

// LDS staging of 16-bit epilogue outputs: 64 rows of 128 bytes per wave, at a padded
// 144-byte pitch or (swizzled) at 128 bytes
constexpr int kStagePitch = 144;
constexpr int kStageBytes = 64 * kStagePitch;
constexpr int kStageSwz = 64 * 128;
// The swizzled layout makes the row-order stores cheaper (out-projection, MLP up and down
// 2.5-4% faster, bank conflicts per LDS instruction 0.13-0.19 -> 0.08-0.13); the QKV
// epilogue's transposed 2-byte V^T writes pay its address arithmetic (13% slower), so QKV
// keeps the padded pitch.
template <int EPI>
constexpr bool kSwzStage = EPI != EPI_QKV;

__device__ __forceinline__ float fma_e(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double fma_e(double a, double b, double c) { return __builtin_fma(a, b, c); }

// Epilogue of one wave's TN x TM block of 16x16 accumulator tiles. acc[i][j][r] = C[m][n]
// with m = token m_base + 16 j + (lane & 15) and n = channel n_base + 16 i + 4 (lane >> 4) + r.
// Loads use token rows clamped to M - 1; only the stores test m < M.
//
// 16-bit outputs go through `stage`, 8 KB of LDS private to the wave, 64 channels (four
// column blocks) at a time: the values are written there in the output's row order and read
// back 16 bytes per lane, so that every store instruction writes whole 128-byte lines (a
// token's 64 channels of Q, K or a row-major output; 64 tokens of one V^T row). Written
// directly, a 16-channel block gives a lane 8 bytes of a row (32 bytes per row per
// instruction), and V^T 2 bytes. The staged V^T path needs M % 8 == 0 (the block's token
// counts are). A staged 64-channel slice is stored after all its residual loads have
// completed and only the wave touches it, so an output aliasing the residual stays correct.
// SWZ: stage rows at a 128-byte pitch with the 16-byte chunk c of row r at position
// c ^ ((r >> 1) & 7) (8 KB per wave) instead of the padded 144-byte pitch. Either layout keeps
// the row-order writes (16 rows x 16 bytes per 32 lanes), the transposed V^T writes (4 rows
// 4 apart x 32 bytes) and the whole-line reads free of bank conflicts; the swizzled one
// needs no padding.
template <int TN, int TM, bool BF16, int EPI, bool OUTF32, bool RESF32, bool OH, bool SWZ = false,
          typename AccT>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs &a, AccT (&acc)[TN][TM],
                                              int n_base, int64_t m_base, int lane,
                                              uint8_t *stage) {
  constexpr bool STAGED = !OUTF32 && EPI != EPI_RAW_I32;
  // fp32 outputs (the debug path): dequant, RoPE, GELU and the gated residual in fp64,
  // rounded once to fp32 at the store
  using E = typename std::conditional<OUTF32, double, float>::type;
  using CS = typename std::conditional<OUTF32, double2, float2>::type;
  // A bf16 residual is read in whole lines too: each 64-channel slice of it is loaded 16
  // bytes per lane in the row order of the stage, written into the stage, and each chunk
  // reads its residual from the stage position its output then overwrites (same lane).
  // The next slice's lines are loaded during the second half of the current slice.
  constexpr bool LRES = STAGED && EPI == EPI_RESID && !RESF32;
  // column blocks whose per-channel operands are loaded ahead
  constexpr int PF = (EPI == EPI_QKV || RESF32 || LRES) ? 1 : 2;
  // QKV: the wave's 128 channels lie in one section (d % 128 == 0); V^T is stored transposed
  const int sec = EPI == EPI_QKV ? n_base / a.d : 0;
  const bool vsec = EPI == EPI_QKV && sec == 2;
  // stage layout: 64 rows of 128 bytes at a 144-byte pitch (the padding spreads a column
  // of the row-major writes over the banks); rows are tokens (row-major outputs) or
  // channels (V^T). Every address is a per-lane base plus a constant.
  auto at = [&](int row, int col) -> uint8_t * {  // byte `col` of stage row `row`
    if constexpr (SWZ)
      return stage + row * 128 + ((((col >> 4) ^ (row >> 1)) & 7) << 4) + (col & 15);
    else
      return stage + row * kStagePitch + col;
  };
  auto stage_put8 = [&](int row, int col2, uint2 v) {  // 8 bytes at byte column col2
    *(uint2 *)at(row, col2) = v;
  };
  auto stage_put2 = [&](int row, int col2, uint16_t v) { *(uint16_t *)at(row, col2) = v; };
  // write back the staged 64 channels starting at channel n_pass
  auto stage_flush = [&](int n_pass) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int row = k * 8 + (lane >> 3), u = lane & 7;
      const uint4 v = *(const uint4 *)at(row, u * 16);
      if constexpr (EPI == EPI_QKV) {
        const int c = n_pass - sec * a.d;  // channel within the section, 64-aligned
        const int head = c / a.Dh, dh0 = c - head * a.Dh;
        if (vsec) {
          const int64_t m = m_base + u * 8;
          if (m < a.M)
            *(uint4 *)((uint16_t *)a.vt + ((int64_t)head * a.Dh + dh0 + row) * a.M + m) = v;
        } else {
          const int64_t m = m_base + row;
          if (m < a.M)
            *(uint4 *)((uint16_t *)(sec == 0 ? a.q : a.k) + ((int64_t)head * a.M + m) * a.Dh +
                       dh0 + u * 8) = v;
        }
      } else {
        const int64_t m = m_base + row;
        if (m < a.M) *(uint4 *)((uint16_t *)a.out + m * a.N + n_pass + u * 8) = v;
      }
    }
  };
  v4i rl[LRES ? 8 : 1];  // residual lines of one slice: rows 8 k + lane / 8, bytes 16 (lane % 8)
  auto load_res_slice = [&](int sl) {
    static_for<LRES ? 8 : 0>([&](auto K) {
      constexpr int k = K;
      const int64_t m = m_base + k * 8 + (lane >> 3);
      rl[k] = *(const v4i *)((const uint16_t *)a.res + (m < a.M ? m : a.M - 1) * a.N + n_base +
                             sl * 64 + (lane & 7) * 8);
    });
  };
  auto put_res_slice = [&]() {
    static_for<LRES ? 8 : 0>([&](auto K) {
      constexpr int k = K;
      *(v4i *)at(k * 8 + (lane >> 3), (lane & 7) * 16) = rl[k];
    });
  };
  // 16-bit values (bf16, or fp16 when OH) of column block i, token tile j (channels
  // 4 (lane >> 4) .. + 3 of the block)
  auto stage_vals = [&](int i, int j, const float (&v)[4]) {
    const int t = j * 16 + (lane & 15);           // token within the wave's 64
    const int cb = (i & 3) * 16 + (lane >> 4) * 4;  // channel within the 64 being staged
    if (vsec) {
#pragma unroll
      for (int r = 0; r < 4; ++r) stage_put2(cb + r, t * 2, OH ? f2h(v[r]) : f2bf(v[r]));
    } else {
      stage_put8(t, cb * 2, make_uint2(pack16<OH>(v[0], v[1]), pack16<OH>(v[2], v[3])));
    }
  };
  int64_t mrow[TM];
  bool mval[TM];
  float sa[TM];
  int3 rofs[TM];  // RoPE table offsets of the lane's token in each 16-row tile (QKV only)
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int64_t m = m_base + j * 16 + (lane & 15);
    mval[j] = m < a.M;
    mrow[j] = mval[j] ? m : a.M - 1;
    sa[j] = 1.f;
    if constexpr (!BF16 && EPI != EPI_RAW_I32) sa[j] = a.sa[mrow[j]];
    if constexpr (EPI == EPI_QKV) rofs[j] = rope_offsets(a.rg, mrow[j]);
  }

  auto load_chunk = [&](EpiChunk<TM, RESF32, OUTF32> &c, int i) {
    const int n = n_base + i * 16 + (lane >> 4) * 4;
    if constexpr (!BF16 && EPI != EPI_RAW_I32) {
      const float4 t4 = *(const float4 *)(a.sw + n);
      c.sw[0] = t4.x; c.sw[1] = t4.y; c.sw[2] = t4.z; c.sw[3] = t4.w;
    }
    if constexpr (EPI == EPI_RESID) {
      const float4 g4 = *(const float4 *)(a.gate + n);
      c.g[0] = g4.x; c.g[1] = g4.y; c.g[2] = g4.z; c.g[3] = g4.w;
#pragma unroll
      for (int j = 0; j < (LRES ? 0 : TM); ++j) {
        if constexpr (RESF32) {
          const uint4 u = *(const uint4 *)((const float *)a.res + mrow[j] * a.N + n);
          c.r[j][0] = u.x; c.r[j][1] = u.y; c.r[j][2] = u.z; c.r[j][3] = u.w;
        } else {
          const uint2 u = *(const uint2 *)((const uint16_t *)a.res + mrow[j] * a.N + n);
          c.r[j][0] = u.x; c.r[j][1] = u.y;
        }
      }
    }
    if constexpr (EPI == EPI_QKV) {
      const int sec = n / a.d;
      const int dh = (n - sec * a.d) % a.Dh;
      if (sec < 2) {
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
          for (int p = 0; p < 2; ++p) c.cs[j][p] = rope_cs<CS>(a.rope, a.rg, dh / 2 + p, rofs[j]);
      }
    }
  };

  // fp32 outputs: column blocks are stored in pairs (i - 1, i), each store instruction
  // writing 8 rows x 128 contiguous bytes (full lines) after a row_ror:8 exchange
  float hold[TM][4];
  auto emit = [&](int i, int j, float (&v)[4]) {
    if constexpr (OUTF32 && (EPI == EPI_GELU || EPI == EPI_RESID)) {
      if ((i & 1) == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) hold[j][r] = v[r];
        return;
      }
      const bool lo = (lane & 15) < 8;
      float X[4], Y[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = dpp_mov<0x128>(hold[j][r]);
        const float br = dpp_mov<0x128>(v[r]);
        X[r] = lo ? hold[j][r] : br;
        Y[r] = lo ? ar : v[r];
      }
      const int nn = n_base + (i - 1) * 16 + (lane >> 4) * 4 + (lo ? 0 : 16);
      const int64_t rx = m_base + j * 16 + (lane & 7);
      if (rx < a.M) store4<true>(a.out, rx * a.N + nn, X[0], X[1], X[2], X[3]);
      if (rx + 8 < a.M) store4<true>(a.out, (rx + 8) * a.N + nn, Y[0], Y[1], Y[2], Y[3]);
    } else {
      stage_vals(i, j, v);
    }
  };

  auto store_chunk = [&](const EpiChunk<TM, RESF32, OUTF32> &c, int i) {
    const int n = n_base + i * 16 + (lane >> 4) * 4;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int64_t m = mrow[j];
      if constexpr (EPI == EPI_RAW_I32) {
        if constexpr (!BF16) {
          const v4i v = acc[i][j];
          if (mval[j]) *(int4 *)(a.c32 + m * a.N + n) = make_int4(v[0], v[1], v[2], v[3]);
        }
      } else {
        E y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (BF16)
            y[r] = acc[i][j][r];
          else
            y[r] = ((E)acc[i][j][r] * (E)sa[j]) * (E)c.sw[r];
        }
        if constexpr (EPI == EPI_QKV) {
          const int cc = n - sec * a.d;
          const int head = cc / a.Dh;
          const int dh = cc - head * a.Dh;
          if (sec < 2) {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              const CS cs = c.cs[j][p];
              const E u0 = y[2 * p], u1 = y[2 * p + 1];
              // one fused multiply-add each, in a fixed order: left to the compiler, the two
              // products of a difference can be fused either way, and the choice differed
              // between kernels instantiating this epilogue (one ulp where they cancel)
              y[2 * p] = fma_e(u0, (E)cs.x, -(u1 * (E)cs.y));
              y[2 * p + 1] = fma_e(u0, (E)cs.y, u1 * (E)cs.x);
            }
            if (sec == 0) {
#pragma unroll
              for (int r = 0; r < 4; ++r) y[r] *= a.q_scale;
            }
            if constexpr (STAGED)
              stage_vals(i, j, y);
            else if (mval[j])
              store4<OUTF32>(sec == 0 ? a.q : a.k, ((int64_t)head * a.M + m) * a.Dh + dh,
                             (float)y[0], (float)y[1], (float)y[2], (float)y[3]);
          } else if constexpr (STAGED) {
            stage_vals(i, j, y);
          } else if (mval[j]) {
            const int64_t base = ((int64_t)head * a.Dh + dh) * a.M + m;
#pragma unroll
            for (int r = 0; r < 4; ++r) store1<OUTF32>(a.vt, base + (int64_t)r * a.M, (float)y[r]);
          }
        } else if constexpr (EPI == EPI_GELU) {
          float v[4] = {(float)gelu_erf(y[0]), (float)gelu_erf(y[1]), (float)gelu_erf(y[2]),
                        (float)gelu_erf(y[3])};
          emit(i, j, v);
        } else if constexpr (EPI == EPI_RESID) {
          E r4[4];
          if constexpr (LRES) {
            const int t = j * 16 + (lane & 15), cb = (i & 3) * 16 + (lane >> 4) * 4;
            const uint2 u = *(const uint2 *)at(t, cb * 2);
            r4[0] = __uint_as_float(u.x << 16);
            r4[1] = __uint_as_float(u.x & 0xffff0000u);
            r4[2] = __uint_as_float(u.y << 16);
            r4[3] = __uint_as_float(u.y & 0xffff0000u);
          } else if constexpr (RESF32) {
#pragma unroll
            for (int r = 0; r < 4; ++r) r4[r] = __uint_as_float(c.r[j][r]);
          } else {
            r4[0] = __uint_as_float(c.r[j][0] << 16);
            r4[1] = __uint_as_float(c.r[j][0] & 0xffff0000u);
            r4[2] = __uint_as_float(c.r[j][1] << 16);
            r4[3] = __uint_as_float(c.r[j][1] & 0xffff0000u);
          }
          float v[4] = {(float)(r4[0] + (E)c.g[0] * y[0]), (float)(r4[1] + (E)c.g[1] * y[1]),
                        (float)(r4[2] + (E)c.g[2] * y[2]), (float)(r4[3] + (E)c.g[3] * y[3])};
          emit(i, j, v);
        }
      }
    }
  };

  EpiChunk<TM, RESF32, OUTF32> buf[PF + 1];
  if constexpr (LRES) load_res_slice(0);
  static_for<PF>([&](auto I) { load_chunk(buf[I], I); });
  static_for<TN>([&](auto I) {
    constexpr int i = I;
    // this slice's residual into the stage; the next slice's loads once two column blocks
    // have freed their accumulator registers
    if constexpr (LRES && (i & 3) == 0) put_res_slice();
    if constexpr (LRES && (i & 3) == 2 && i + 2 < TN) load_res_slice(i / 4 + 1);
    if constexpr (i + PF < TN) load_chunk(buf[(i + PF) % (PF + 1)], i + PF);
    store_chunk(buf[i % (PF + 1)], i);
    if constexpr (STAGED && (i & 3) == 3) stage_flush(n_base + (i - 3) * 16);
  });
}

// ------------------------------------------------------------------ ping-pong kernel
// 256 x 256 work-group tile, 8 waves in two groups of four. Waves w and w + 4 run on the
// same SIMD, so group g = w / 4 puts one wave of each group on every SIMD. The groups are
// offset by one barrier: while the waves of one group issue the matrix-core work of a K
// step from registers, the waves of the other group load the next step's fragments from
// LDS and issue global -> LDS copies, so each SIMD always has one wave feeding its matrix
// core. Group g owns weight rows [128 g, 128 g + 128) of the tile, wave w % 4 owns tokens
// [64 (w % 4), 64 (w % 4) + 64): 8 x 4 accumulator tiles of 16 x 16 per wave.
//
// A K step is 64 bytes (one MFMA K step); LDS holds two stages of two steps each. A stage
// is 128 bytes of K for the 256 weight rows then the 256 token rows, stored row-major with
// 128-byte rows; the 16-byte chunk c of row r sits at position c ^ (r % 8). A global -> LDS
// copy instruction fills 8 rows (1 KB, lane l writes offset 16 l): lane l fetches row l / 8,
// chunk (l % 8) ^ (l / 8 % 8), so eight consecutive lanes read one full 128-byte line. The
// MFMA fragment of lane l (row l % 16, chunk 4 h + l / 16 for the stage's step h) is read
// from position (4 h + l / 16) ^ (l % 8); the XOR spreads a fragment read over the banks.
constexpr int PP_SB = 128;                    // bytes of K per stage (two MFMA K steps)
constexpr int PP_STAGE = (256 + 256) * PP_SB;  // LDS bytes of one stage

// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0] + [15:14], expcnt [6:4], lgkmcnt [11:8])
constexpr int waitcnt_vm_lgkm0(int vm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (0 << 8);
}

// Work-group barrier without a memory fence. A fenced barrier (__syncthreads) waits for
// every outstanding global -> LDS copy (vmcnt(0)), which would drain the copy pipeline at
// each barrier; ordering is instead made explicit with s_waitcnt before the barrier. The
// asm memory clobber keeps the compiler from moving memory accesses across it and the
// scheduling barriers keep the matrix-core work inside its phase.
#define H3K_PP_SYNC()                                   \
  {                                                     \
    __builtin_amdgcn_sched_barrier(0);                  \
    asm volatile("s_barrier" ::: "memory");             \
    __builtin_amdgcn_sched_barrier(0);                  \
  }

// OH: 16-bit outputs stored as fp16 instead of bf16 (the QKV epilogue's attention inputs)
template <bool BF16, int EPI, bool OUTF32, bool RESF32, bool OH>
__global__ __launch_bounds__(512) void gemm_pp_kernel(const GemmArgs a) {
  constexpr int TN = 8, TM = 4;
  using AccT = typename std::conditional<BF16, v4f, v4i>::type;

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // wave index made visibly uniform so that branches on the group are scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wq = wave & 3;

  const int64_t ntiles = (int64_t)(a.N / 256) * ((a.M + 255) / 256);
  int64_t t = blockIdx.x;
  int64_t m0;
  int n0;
  tile_origin<256, 256>(a, t, m0, n0);
  const int64_t Kb = (int64_t)a.K * (BF16 ? 2 : 1);
  const int ns = (int)(Kb / PP_SB);  // stages

  // global -> LDS copies: wave w copies the 8-row groups w, w + 8, w + 16, w + 24 of the
  // weight tile and of the token tile in every stage. Token rows past M read row M - 1:
  // they only feed accumulator rows that are never stored. The copies are buffer loads
  // (MUBUF) from resources based at the tile's first row, so 32-bit offsets suffice and
  // they count only in vmcnt.
  const int cr = lane >> 3, cc = (lane & 7) ^ cr;
  const uint32_t oB = (uint32_t)((wave * 8 + cr) * Kb + cc * 16);
  const uint32_t oB_q = (uint32_t)(64 * Kb);  // 8 row groups further down the weight tile
  __amdgpu_buffer_rsrc_t brs, ars;
  uint32_t oA[4];
  auto tile_copy_setup = [&](int64_t tm0, int tn0, __amdgpu_buffer_rsrc_t &b_rs,
                             __amdgpu_buffer_rsrc_t &a_rs, uint32_t (&o_a)[4]) {
    b_rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const uint8_t *)a.B + (int64_t)tn0 * Kb), (short)0, (int)0xffffffffu, 0x00020000);
    a_rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const uint8_t *)a.A + tm0 * Kb), (short)0, (int)0xffffffffu, 0x00020000);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t m = tm0 + (wave + 8 * q) * 8 + cr;
      o_a[q] = (uint32_t)(((m < a.M ? m : a.M - 1) - tm0) * Kb + cc * 16);
    }
  };
  tile_copy_setup(m0, n0, brs, ars, oA);
#define H3K_PP_COPY_WITH(s_, b_rs, a_rs, o_a)                                               \
  {                                                                                         \
    const uint32_t ko = (uint32_t)(s_) * PP_SB;                                             \
    uint8_t *dst = smem + ((s_) & 1) * PP_STAGE + wave * 1024;                              \
    _Pragma("unroll") for (int q = 0; q < 4; ++q)                                           \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rs,                                        \
          (__attribute__((address_space(3))) void *)(dst + q * 8192), 16,                   \
          oB + q * oB_q + ko, 0, 0, 0);                                                     \
    _Pragma("unroll") for (int q = 0; q < 4; ++q)                                           \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rs,                                        \
          (__attribute__((address_space(3))) void *)(dst + 32768 + q * 8192), 16,           \
          o_a[q] + ko, 0, 0, 0);                                                            \
  }
#define H3K_PP_COPY(s_) H3K_PP_COPY_WITH(s_, brs, ars, oA)

  AccT acc[TN][TM];
  // fragments of one step: weight rows 128 grp + 16 i, token rows 64 wq + 16 j
  v4i fb[TN], fa[TM];
  const int frag_off = (lane & 15) * PP_SB + (((lane >> 4) ^ (lane & 7)) * 16);
#define H3K_PP_READ(s_, h_)                                                                 \
  {                                                                                         \
    const uint8_t *src = smem + ((s_) & 1) * PP_STAGE + (frag_off ^ ((h_) * 64));           \
    _Pragma("unroll") for (int i = 0; i < TN; ++i) fb[i] =                                  \
        *(const v4i *)(src + (grp * TN + i) * 16 * PP_SB);                                  \
    _Pragma("unroll") for (int j = 0; j < TM; ++j) fa[j] =                                  \
        *(const v4i *)(src + 32768 + (wq * TM + j) * 16 * PP_SB);                           \
  }
#define H3K_PP_MFMA()                                                                       \
  {                                                                                         \
    _Pragma("unroll") for (int i = 0; i < TN; ++i)                                          \
    _Pragma("unroll") for (int j = 0; j < TM; ++j) acc[i][j] = mma<BF16>(fb[i], fa[j], acc[i][j]); \
  }

  // Step k = 2 s + h reads stage s (buffer s % 2). Barrier instances are counted from the
  // tile's first one: instance 2k + 1 ends group 0's memory phase of step k and group 1's
  // compute phase of step k - 1; instance 2k + 2 ends group 0's compute phase of step k and
  // group 1's memory phase of step k.
  //  - The copies of stage s + 1 are issued in the memory phase of step 2 s: buffer (s + 1) % 2
  //    last held stage s - 1, whose last reader (group 1, step 2 s - 1) passed instance 4 s.
  //  - Each wave waits for its own copies at the end of its memory phase of step 2 s + 1, at
  //    the latest instance 4 s + 4, before which nobody reads stage s + 1.
  //  - After instance 4 ns every read of the tile's stages is complete, so both groups copy
  //    stage 0 of their next tile into buffer 0 before their epilogue; the epilogue's
  //    global-memory latency then covers that copy's.
  H3K_PP_COPY(0);
  for (;;) {
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) acc[i][j] = AccT{0, 0, 0, 0};
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    H3K_PP_SYNC();
    if (grp) H3K_PP_SYNC();

    for (int st = 0; st < ns; ++st) {
      if (st + 1 < ns) H3K_PP_COPY(st + 1);
      H3K_PP_READ(st, 0);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
      H3K_PP_SYNC();
      H3K_PP_MFMA();
      H3K_PP_SYNC();
      H3K_PP_READ(st, 1);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
      H3K_PP_SYNC();
      H3K_PP_MFMA();
      // Group 1's last compute phase needs no closing barrier (no LDS access follows), which
      // leaves both groups with the same barrier count; group 0 closes its last compute
      // phase at the instance that ends group 1's last memory phase, then runs its epilogue
      // while group 1 computes.
      if (st + 1 < ns || grp == 0) H3K_PP_SYNC();
    }

    const int64_t tn = t + gridDim.x;
    const bool more = tn < ntiles;
    int64_t m0n = 0;
    int n0n = 0;
    if (more) {
      tile_origin<256, 256>(a, tn, m0n, n0n);
      tile_copy_setup(m0n, n0n, brs, ars, oA);
      H3K_PP_COPY(0);
    }
    // LDS from buffer 1 on is free until the next tile's first loop iteration (its stage 0
    // goes to buffer 0): each wave stages there
    gemm_epilogue<TN, TM, BF16, EPI, OUTF32, RESF32, OH, kSwzStage<EPI>>(
        a, acc, n0 + grp * TN * 16, m0 + wq * TM * 16, lane,
        smem + PP_STAGE + wave * (kSwzStage<EPI> ? kStageSwz : kStageBytes));
    if (!more) break;
    t = tn;
    m0 = m0n;
    n0 = n0n;
  }
}
#undef H3K_PP_COPY
#undef H3K_PP_COPY_WITH
#undef H3K_PP_READ
#undef H3K_PP_MFMA

// ------------------------------------------------------------------ one-wave-per-SIMD kernel
// int8 operands (int32 accumulators) or bf16 ones (fp32 accumulators; the same 16 bytes of K
// per lane and fragment, so the same byte pipeline). The same 256 x 256 work-group tile and
// tile order as the ping-pong kernel, with four waves, one per SIMD. Wave w
// owns weight rows [64 w, 64 w + 64) of the tile and all 256 tokens: 4 x 16 accumulator
// tiles, 256 registers, held in the accumulation registers (AGPRs) by issuing the MFMAs as
// inline assembly whose accumulator operand is constrained to them (left to the compiler,
// that layout turned into register moves around every MFMA).
//
// Operands. The weights come in the tiled layout of h3k_tile_weights: each MFMA fragment
// (16 rows x 64 bytes of K) is one contiguous kilobyte in which lane l's 16 bytes sit at
// offset 16 l, so a fragment is one whole-line 16-byte-per-lane load straight into
// registers; every weight row belongs to one wave, so nothing is loaded twice. Only the
// tokens go through LDS, in a ring of W4_NS stages of 128 bytes of K (the copies and the
// fragment layout of the ping-pong kernel): that halves the LDS writes per multiply, which
// run at a quarter of the read rate, and cuts the fragment reads per multiply by a third.
//
// Schedule of stage s (K steps 2 s and 2 s + 1), inside each wave:
//   step 2 s:   64 MFMAs; after the four that use token fragment j, fragment j of step
//               2 s + 1 is read into the same registers; the eight weight fragments of
//               stage s + 1 are loaded (A ring of two stages, by parity);
//   barrier:    each wave first waits for its copies of stage s + 1 (issued two stages
//               earlier), so after it stage s + 1 is complete and stage s - 1 is free;
//   step 2 s+1: 64 MFMAs; fragment j of step 2 s + 2 (stage s + 1) read likewise; the copies
//               of stage s + W4_NS - 1 go into the buffer stage s - 1 left.
// Every stage issues the same loads: past the last stage they re-read the last stage into
// registers and a buffer that nothing reads as data, so the body has no branches (a branch
// there made the compiler spill). After the last stage the next tile's first stages are
// copied and its first weight fragments loaded before the epilogue, so their latency
// overlaps the epilogue's. The epilogue runs as four 64-token slices through the generic
// one, staging in the buffer the next tile fills last.
constexpr int W4_NS = 4;               // LDS stages of the token operand
constexpr int W4_STG = 256 * PP_SB;    // 32 KB: 256 token rows x 128 bytes of K

template <int EPI>
constexpr int w4_stage_bytes() { return kSwzStage<EPI> ? kStageSwz : kStageBytes; }
template <int EPI>
constexpr int w4_lds_bytes() {
  return W4_NS * W4_STG > (W4_NS - 1) * W4_STG + 4 * w4_stage_bytes<EPI>()
             ? W4_NS * W4_STG
             : (W4_NS - 1) * W4_STG + 4 * w4_stage_bytes<EPI>();
}

// acc += w x^T on the matrix cores, accumulator in AGPRs (int8 -> int32, or bf16 -> fp32
// with the same 16 bytes of K per lane); the zero form starts a tile
__device__ __forceinline__ void mma_agpr(v4i &acc, const v4i &w, const v4i &x) {
  asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc) : "v"(w), "v"(x));
}
__device__ __forceinline__ void mma_agpr_zero(v4i &acc, const v4i &w, const v4i &x) {
  asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, 0" : "=a"(acc) : "v"(w), "v"(x));
}
__device__ __forceinline__ void mma_agpr(v4f &acc, const v4i &w, const v4i &x) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(w), "v"(x));
}
__device__ __forceinline__ void mma_agpr_zero(v4f &acc, const v4i &w, const v4i &x) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(w), "v"(x));
}

template <bool BF16, int EPI, bool OUTF32, bool RESF32, bool OH>
__global__ __launch_bounds__(256, 1) void gemm_w4_kernel(const GemmArgs a) {
  using AccT = typename std::conditional<BF16, v4f, v4i>::type;
  constexpr int NS = W4_NS;
  constexpr bool SWZ = kSwzStage<EPI>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t ntiles = (int64_t)(a.N / 256) * ((a.M + 255) / 256);
  const int K = a.K * (BF16 ? 2 : 1), ksteps = K / 64, ns = K / PP_SB;  // K in bytes
  // copy lane: row cr of an 8-row group, global chunk cc (stored at chunk position lane % 8)
  const int cr = lane >> 3, cc = (lane & 7) ^ cr;
  const int frag_off = (lane & 15) * PP_SB + (((lane >> 4) ^ (lane & 7)) * 16);
  uint8_t *stage_ep = smem + (NS - 1) * W4_STG + wave * w4_stage_bytes<EPI>();

  int64_t t = blockIdx.x, m0;
  int n0;
  tile_origin<256, 256>(a, t, m0, n0);
  // Buffer resources based at the tile's first token row and at the wave's first weight
  // fragment row, so 32-bit offsets suffice: token rows past M read row M - 1 (they only
  // feed accumulator rows that are never stored).
  __amdgpu_buffer_rsrc_t xrs, wrs;
  uint32_t xo[8];
  auto setup = [&](int64_t tm0, int tn0) {
    xrs = __builtin_amdgcn_make_buffer_rsrc((void *)((const int8_t *)a.A + tm0 * K), (short)0,
                                            (int)0xffffffffu, 0x00020000);
    wrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.Bt + (int64_t)(tn0 / 16 + 4 * wave) * ksteps * 1024), (short)0,
        (int)0xffffffffu, 0x00020000);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int64_t m = tm0 + (wave + 4 * q) * 8 + cr;
      xo[q] = (uint32_t)(((m < a.M ? m : a.M - 1) - tm0) * K + cc * 16);
    }
  };
  v4i A[2][2][4];  // weight fragments [stage parity][step in stage][16-row block]
  auto load_a = [&](int p, int h, int i, int st) {
    const v4i v = __builtin_amdgcn_raw_buffer_load_b128(
        wrs, (uint32_t)(lane * 16), (uint32_t)((i * ksteps + 2 * st + h) * 1024), 0);
    if (p == 0) A[0][h][i] = v; else A[1][h][i] = v;
  };
  auto copy = [&](int q, int st) {  // 8 token rows of stage st (one kilobyte of LDS)
    uint8_t *dst = smem + (st % NS) * W4_STG + (wave + 4 * q) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (__attribute__((address_space(3))) void *)dst,
                                             16, xo[q] + (uint32_t)st * PP_SB, 0, 0, 0);
  };
  // the first stages of a tile: copies of stages 0 .. NS-2, weight fragments of stage 0
  auto prologue = [&]() {
#pragma unroll
    for (int st = 0; st < NS - 1; ++st) {
      const int sc = st < ns ? st : ns - 1;
#pragma unroll
      for (int q = 0; q < 8; ++q) copy(q, sc);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) load_a(0, h, i, 0);
  };
  AccT acc[4][4][4];  // [64-token slice g][16-row weight block i][token block j within g]
  v4i B[16];

  auto stage = [&](int s, auto P, auto FIRST) {
    constexpr int p = decltype(P)::value;
    constexpr bool first = decltype(FIRST)::value;
    const uint8_t *cur = smem + (s % NS) * W4_STG;
    const uint8_t *nxt = smem + ((s + 1) % NS) * W4_STG;
    const int sa = s + 1 < ns ? s + 1 : ns - 1;            // weight fragments of stage s+1
    const int sc = s + NS - 1 < ns ? s + NS - 1 : ns - 1;  // token copies of stage s+NS-1
#pragma unroll
    for (int j = 0; j < 16; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (first) mma_agpr_zero(acc[j >> 2][i][j & 3], A[p][0][i], B[j]);
        else mma_agpr(acc[j >> 2][i][j & 3], A[p][0][i], B[j]);
      }
      B[j] = *(const v4i *)(cur + (frag_off ^ 64) + j * 16 * PP_SB);
      if (j < 8) load_a(p ^ 1, j >> 2, j & 3, sa);
    }
    // this wave's copies of stage s+1 are complete: after them it issued the weight
    // fragments of stage s+1 (8) and, for each stage in between, copies and fragments (16)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(8 + 16 * (NS - 3)));
    H3K_PP_SYNC();
#pragma unroll
    for (int j = 0; j < 16; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) mma_agpr(acc[j >> 2][i][j & 3], A[p][1][i], B[j]);
      B[j] = *(const v4i *)(nxt + frag_off + j * 16 * PP_SB);
      if (j & 1) copy(j >> 1, sc);
    }
  };

  setup(m0, n0);
  prologue();
  for (;;) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    H3K_PP_SYNC();
#pragma unroll
    for (int j = 0; j < 16; ++j) B[j] = *(const v4i *)(smem + frag_off + j * 16 * PP_SB);
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using F0 = std::integral_constant<bool, false>;
    stage(0, P0{}, std::integral_constant<bool, true>{});
    int s = 1;
    if (ns > 1) {
      stage(1, P1{}, F0{});
      s = 2;
    }
    for (; s + 1 < ns; s += 2) {
      stage(s, P0{}, F0{});
      stage(s + 1, P1{}, F0{});
    }
    if (s < ns) stage(s, P0{}, F0{});
    // the last MFMAs' results are read by the epilogue: wait states for the matrix pipe
    asm volatile("s_nop 15\n s_nop 15\n s_nop 15\n s_nop 15" ::: "memory");
    // every wave is done with this tile's stages before the next tile's copies land
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    H3K_PP_SYNC();
    const int64_t tn = t + gridDim.x;
    const bool more = tn < ntiles;
    int64_t m0n = 0;
    int n0n = 0;
    if (more) {
      tile_origin<256, 256>(a, tn, m0n, n0n);
      setup(m0n, n0n);
      prologue();
    }
    static_for<4>([&](auto G) {
      constexpr int g = G;
      // an ordering point per slice: its accumulators are read after the wait states above
      // and after the previous slice's stores, not all at once (which would spill)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(acc[g][i][j]));
      gemm_epilogue<4, 4, BF16, EPI, OUTF32, RESF32, OH, SWZ>(a, acc[g], n0 + 64 * wave,
                                                               m0 + 64 * g, lane, stage_ep);
    });
    if (!more) break;
    t = tn;
    m0 = m0n;
    n0 = n0n;
  }
}

// int8 weights [N, K] -> tiled: 16-byte chunk c of the output holds row
// 16 (c / 64 / (K / 64)) + (c % 64) % 16, bytes 64 ((c / 64) % (K / 64)) + 16 ((c % 64) / 16) ..+15
__global__ __launch_bounds__(256) void tile_weights_kernel(const int8_t *__restrict__ q, int64_t N,
                                                           int64_t K, int8_t *__restrict__ qt) {
  const int64_t KB = K / 64, chunks = N * K / 16;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t l = c & 63, tile = c >> 6;
    const int64_t nb = tile / KB, kb = tile - nb * KB;
    const int64_t row = nb * 16 + (l & 15), col = kb * 64 + (l >> 4) * 16;
    *(uint4 *)(qt + c * 16) = *(const uint4 *)(q + row * K + col);
  }
}

hipError_t launch_tile_weights(const int8_t *q, int64_t N, int64_t K, int8_t *qt, hipStream_t s) {
  if (N <= 0 || K <= 0 || N % 16 || K % 64) return hipErrorInvalidValue;
  const int64_t chunks = N * K / 16;
  const int64_t blocks = (chunks + 255) / 256 < 8192 ? (chunks + 255) / 256 : 8192;
  tile_weights_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(q, N, K, qt);
  return hipGetLastError();
}

// compute units of the current device, queried once per device
static hipError_t compute_units(int *n) {
  static std::atomic<int> cached[64];  // zero-initialised (static storage)
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (v <= 0) return hipErrorInvalidValue;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  *n = v;
  return hipSuccess;
}

template <bool BF16, int EPI, bool OUTF32, bool RESF32, bool OH>
static hipError_t run_gemm_pp(const GemmArgs &a, hipStream_t s) {
  auto kern = gemm_pp_kernel<BF16, EPI, OUTF32, RESF32, OH>;
  constexpr size_t lds = (size_t)PP_STAGE + 8 * (kSwzStage<EPI> ? kStageSwz : kStageBytes);
  static_assert(lds >= (size_t)2 * PP_STAGE && lds <= 160 * 1024, "LDS budget");
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = ensure_dynamic_lds((const void *)kern, (int)lds, lds_set);
      e != hipSuccess)
    return e;
  // persistent: one work-group per compute unit (the LDS footprint allows one), each
  // walking tiles b, b + grid, ...
  const int64_t nwg = ((a.M + 255) / 256) * (a.N / 256);
  int n_cu = 0;
  if (hipError_t e = compute_units(&n_cu); e != hipSuccess) return e;
  const int64_t full = n_cu >= 8 ? (n_cu & ~7) : n_cu;  // keeps tile % 8 == XCD
  const int64_t grid = nwg < full ? nwg : full;
  kern<<<dim3((unsigned)grid), dim3(512), lds, s>>>(a);
  return hipGetLastError();
}

template <bool BF16, int EPI, bool OUTF32, bool RESF32, bool OH>
static hipError_t run_gemm_w4(const GemmArgs &a, hipStream_t s) {
  auto kern = gemm_w4_kernel<BF16, EPI, OUTF32, RESF32, OH>;
  constexpr size_t lds = (size_t)w4_lds_bytes<EPI>();
  static_assert(lds <= 160 * 1024, "LDS budget");
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = ensure_dynamic_lds((const void *)kern, (int)lds, lds_set); e != hipSuccess)
    return e;
  const int64_t nwg = ((a.M + 255) / 256) * (a.N / 256);
  int n_cu = 0;
  if (hipError_t e = compute_units(&n_cu); e != hipSuccess) return e;
  const int64_t full = n_cu >= 8 ? (n_cu & ~7) : n_cu;  // keeps tile % 8 == XCD
  const int64_t grid = nwg < full ? nwg : full;
  kern<<<dim3((unsigned)grid), dim3(256), lds, s>>>(a);
  return hipGetLastError();
}

template <bool BF16, int EPI, bool OUTF32, bool RESF32, bool OH = false>
static hipError_t gemm_tiles(const GemmArgs &a, hipStream_t s) {
  if (a.Bt) return run_gemm_w4<BF16, EPI, OUTF32, RESF32, OH>(a, s);
  return run_gemm_pp<BF16, EPI, OUTF32, RESF32, OH>(a, s);
}
// instantiated type combinations (operands -> outputs):
//   QKV    int8 -> fp16 | int8 -> bf16 | int8 -> fp32 | bf16 -> fp16 | bf16 -> bf16
//   GELU   int8 -> bf16 | int8 -> fp32 | bf16 -> bf16
//   RESID  residual and output bf16 (int8 or bf16 operands) | fp32 (int8 operands)
static hipError_t gemm_dispatch(EpiKind kind, const GemmArgs &a, hipStream_t s) {
  const bool B = a.bf16_ops, OF = a.out_f32, RF = a.res_f32;
  if (kind == EPI_QKV && !OF && a.M % 8) return hipErrorInvalidValue;  // staged V^T rows
  switch (kind) {
    case EPI_QKV:
      if (OF && a.qkv_f16) return hipErrorInvalidValue;
      if (B) {
        if (OF) return hipErrorInvalidValue;
        return a.qkv_f16 ? gemm_tiles<true, EPI_QKV, false, false, true>(a, s)
                         : gemm_tiles<true, EPI_QKV, false, false, false>(a, s);
      }
      if (OF) return gemm_tiles<false, EPI_QKV, true, false>(a, s);
      return a.qkv_f16 ? gemm_tiles<false, EPI_QKV, false, false, true>(a, s)
                       : gemm_tiles<false, EPI_QKV, false, false, false>(a, s);
    case EPI_GELU:
      if (B) return OF ? hipErrorInvalidValue : gemm_tiles<true, EPI_GELU, false, false>(a, s);
      return OF ? gemm_tiles<false, EPI_GELU, true, false>(a, s)
                : gemm_tiles<false, EPI_GELU, false, false>(a, s);
    case EPI_RESID:
      // residual and output share the activation type: bf16, or fp32 on the debug path
      if (RF != OF) return hipErrorInvalidValue;
      if (OF) return B ? hipErrorInvalidValue : gemm_tiles<false, EPI_RESID, true, true>(a, s);
      return B ? gemm_tiles<true, EPI_RESID, false, false>(a, s)
               : gemm_tiles<false, EPI_RESID, false, false>(a, s);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(EpiKind kind, const GemmArgs &a, hipStream_t s) {
  if (kind == EPI_RAW_I32) {
    if (a.bf16_ops || a.out_f32) return hipErrorInvalidValue;
    return gemm_tiles<false, EPI_RAW_I32, false, false>(a, s);
  }
  return gemm_dispatch(kind, a, s);
}

}  // namespace h3k
