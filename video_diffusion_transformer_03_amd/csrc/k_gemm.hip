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
// The matrix-core output is computed transposed (weights are the MFMA "A" operand): a
// lane then holds four consecutive output channels of one token, which is what the
// fused epilogues want -- RoPE rotates channel pairs (2i, 2i+1) inside one lane, and the
// head-major Q/K scatter stores 4 consecutive head dims per lane. Epilogues:
//   RAW_I32  int32 accumulators (exactness check of the main loop)
//   QKV      dequant, 3D RoPE on Q and K, scatter to head-major Q, K [H, L, Dh] and
//            transposed V [H, Dh, L] (the layout attention consumes)
//   GELU     dequant + exact erf GELU (MLP up)
//   RESID    dequant + gated residual out = res + gate[n] * y (out-proj, MLP down)
#include "h3k_internal.h"

#include <type_traits>

namespace h3k {

// work-group tile (BN weights rows x BM tokens) and wave grid (WN x WM waves)
#ifndef H3K_GEMM_BN
#define H3K_GEMM_BN 256
#define H3K_GEMM_BM 256
#define H3K_GEMM_WN 2
#define H3K_GEMM_WM 4
#endif

#ifndef H3K_GEMM_PAD
#define H3K_GEMM_PAD 32  // 160-byte pitch: conflict-free 16-byte fragment reads on gfx950
#endif

constexpr int KB = 128;                 // bytes of K staged per pipeline step
constexpr int KBP = KB + H3K_GEMM_PAD;  // LDS row pitch (bytes): the pad spreads rows over banks

template <int BN, int BM>
constexpr size_t gemm_lds_bytes() {
  return (size_t)2 * (BN + BM) * KBP;
}

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

__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

// rotation (cos, sin) of pair i of head_dim for token l
__device__ __forceinline__ float2 rope_cs(const float2 *tbl, const RopeGeom &g, int i,
                                          int64_t l) {
  const int hw = g.Hg * g.Wg;
  const int t = (int)(l / hw);
  const int rem = (int)(l - (int64_t)t * hw);
  const int h = rem / g.Wg;
  const int w = rem - h * g.Wg;
  int e;
  if (i < g.Pt)
    e = t * g.Pt + i;
  else if (i < g.Pt + g.Ph)
    e = g.base_h + h * g.Ph + (i - g.Pt);
  else
    e = g.base_w + w * g.Pw + (i - g.Pt - g.Ph);
  return tbl[e];
}

template <int I, typename T>
__device__ __forceinline__ T &pick(T &a, T &b, T &c, T &d) {
  if constexpr (I == 0) return a;
  else if constexpr (I == 1) return b;
  else if constexpr (I == 2) return c;
  else return d;
}

template <bool BF16>
__device__ __forceinline__ auto mma(v4i b, v4i a, typename std::conditional<BF16, v4f, v4i>::type c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, b),
                                                   __builtin_bit_cast(v8bf, a), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(b, a, c, 0, 0, 0);
}

template <int BN, int BM, int WN, int WM, bool BF16, int EPI, bool OUTF32, bool RESF32>
__global__ __launch_bounds__(WN *WM * 64) void gemm_kernel(const GemmArgs a) {
  constexpr int NT = WN * WM * 64;
  constexpr int TN = BN / WN / 16;  // 16-row MFMA tiles per wave along N
  constexpr int TM = BM / WM / 16;  // 16-col MFMA tiles per wave along M
  constexpr int CPR = KB / 16;      // 16-byte chunks per staged row
  constexpr int CH_B = BN * CPR / NT;
  constexpr int CH_A = BM * CPR / NT;
  static_assert(BN * CPR % NT == 0 && BM * CPR % NT == 0, "tile/threads mismatch");
  using AccT = typename std::conditional<BF16, v4f, v4i>::type;

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t *sB = smem;                  // [2][BN][KBP] weights
  uint8_t *sA = smem + 2 * BN * KBP;   // [2][BM][KBP] activations

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave / WM, wm = wave % WM;

  // ---- tile schedule: the work-groups the hardware places on one XCD (bid % 8) get a
  // contiguous range of logical tiles, walked in groups of 8 M-tiles so that concurrent
  // work-groups of an XCD share weight and activation tiles in that XCD's L2.
  const int n_tiles = a.N / BN;
  const int64_t m_tiles = (a.M + BM - 1) / BM;
  const int64_t nwg = (int64_t)n_tiles * m_tiles;
  int64_t t = blockIdx.x;
  if ((nwg & 7) == 0) t = (t & 7) * (nwg >> 3) + (t >> 3);
  constexpr int GM = 8;
  const int64_t group = t / ((int64_t)GM * n_tiles);
  const int64_t first_m = group * GM;
  const int64_t gsize = (m_tiles - first_m) < GM ? (m_tiles - first_m) : GM;
  const int64_t in_group = t - group * GM * n_tiles;
  const int64_t tm_idx = first_m + in_group % gsize;
  const int tn_idx = (int)(in_group / gsize);
  const int64_t m0 = tm_idx * BM;
  const int n0 = tn_idx * BN;

  const int64_t Kb = (int64_t)a.K * (BF16 ? 2 : 1);
  const uint8_t *gA = (const uint8_t *)a.A;
  const uint8_t *gB = (const uint8_t *)a.B;
  const int nk = (int)(Kb / KB);

  // staging registers (named scalars, not arrays: they stay in VGPRs across iterations)
  static_assert(CH_B <= 4 && CH_A <= 4, "at most 4 staged chunks per thread and operand");
  uint4 rb0, rb1, rb2, rb3, ra0, ra1, ra2, ra3;
#define H3K_GLOAD(kt_)                                                                       \
  {                                                                                          \
    const int64_t kof = (int64_t)(kt_) * KB;                                                 \
    static_for<CH_B>([&](auto I) {                                                           \
      const int c = tid + I * NT, row = c / CPR, col = c % CPR;                              \
      pick<I>(rb0, rb1, rb2, rb3) = *(const uint4 *)(gB + (int64_t)(n0 + row) * Kb + kof + col * 16);              \
    });                                                                                      \
    static_for<CH_A>([&](auto I) {                                                           \
      const int c = tid + I * NT, row = c / CPR, col = c % CPR;                              \
      /* rows past M read row M-1: they only feed output rows that are never stored */       \
      const int64_t m = (m0 + row) < a.M ? (m0 + row) : (a.M - 1);                           \
      pick<I>(ra0, ra1, ra2, ra3) = *(const uint4 *)(gA + m * Kb + kof + col * 16);                                \
    });                                                                                      \
  }
#define H3K_LSTORE(buf_)                                                                     \
  {                                                                                          \
    static_for<CH_B>([&](auto I) {                                                           \
      const int c = tid + I * NT, row = c / CPR, col = c % CPR;                              \
      *(uint4 *)(sB + ((buf_) * BN + row) * KBP + col * 16) = pick<I>(rb0, rb1, rb2, rb3);                         \
    });                                                                                      \
    static_for<CH_A>([&](auto I) {                                                           \
      const int c = tid + I * NT, row = c / CPR, col = c % CPR;                              \
      *(uint4 *)(sA + ((buf_) * BM + row) * KBP + col * 16) = pick<I>(ra0, ra1, ra2, ra3);                         \
    });                                                                                      \
  }

  AccT acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = AccT{0, 0, 0, 0};

  const int frow = lane & 15, fk = (lane >> 4) * 16;
  // one pipeline step: MFMAs over the KB bytes of K staged in LDS buffer cur_
#define H3K_COMPUTE(cur_)                                                                     \
  {                                                                                          \
    const uint8_t *bB = sB + ((cur_) * BN + wn * TN * 16 + frow) * KBP + fk;                 \
    const uint8_t *bA = sA + ((cur_) * BM + wm * TM * 16 + frow) * KBP + fk;                 \
    _Pragma("unroll") for (int ks = 0; ks < KB / 64; ++ks) {                                 \
      v4i fb[TN], fa[TM];                                                                    \
      _Pragma("unroll") for (int i = 0; i < TN; ++i) fb[i] =                                 \
          *(const v4i *)(bB + i * 16 * KBP + ks * 64);                                       \
      _Pragma("unroll") for (int j = 0; j < TM; ++j) fa[j] =                                 \
          *(const v4i *)(bA + j * 16 * KBP + ks * 64);                                       \
      _Pragma("unroll") for (int i = 0; i < TN; ++i)                                         \
      _Pragma("unroll") for (int j = 0; j < TM; ++j) acc[i][j] = mma<BF16>(fb[i], fa[j], acc[i][j]); \
    }                                                                                        \
  }
  // Software pipeline, prefetch distance 2. Iteration kt: store the registers holding
  // tile kt+1 (loaded one iteration earlier) into LDS buffer (kt+1)&1, issue the global
  // loads of tile kt+2, then run the MFMAs of tile kt from buffer kt&1. The barrier that
  // ends iteration kt-1 separates both the reads of buffer (kt+1)&1 in iteration kt-1
  // from its rewrite here, and the rewrite of buffer kt&1 from the reads below.
  H3K_GLOAD(0);
  H3K_LSTORE(0);
  H3K_GLOAD(nk > 1 ? 1 : 0);  // (re-reads tile 0 when there is no tile 1; unused then)
  __syncthreads();
  int kt = 0;
  for (; kt + 2 < nk; ++kt) {
    H3K_LSTORE((kt + 1) & 1);
    H3K_GLOAD(kt + 2);
    H3K_COMPUTE(kt & 1);
#ifdef H3K_GEMM_SGB2
    // issue order for the scheduler: LDS stores, global loads, then the second K step's
    // fragment reads spread over the first K step's MFMAs
    static_assert(KB == 128, "schedule written for two 64-byte K steps");
    __builtin_amdgcn_sched_group_barrier(0x200, CH_A + CH_B, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, CH_A + CH_B, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, TN + TM, 0);
    static_for<TN + TM>([&](auto) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    });
    __builtin_amdgcn_sched_group_barrier(0x008, TN * TM * 2 - 2 * (TN + TM), 0);
#endif
    __syncthreads();
  }
  if (kt + 1 < nk) {
    H3K_LSTORE((kt + 1) & 1);
    H3K_COMPUTE(kt & 1);
    __syncthreads();
    ++kt;
  }
  H3K_COMPUTE(kt & 1);

  // ---- epilogue. acc[i][j][r] = C[m][n] with m = token (lane & 15 within tile j),
  // n = channel (4 * (lane >> 4) + r within tile i).
#pragma unroll
  for (int i = 0; i < TN; ++i) {
    const int n = n0 + wn * TN * 16 + i * 16 + (lane >> 4) * 4;
    float sw[4] = {1.f, 1.f, 1.f, 1.f};
    if constexpr (!BF16 && EPI != EPI_RAW_I32) {
      float4 t4 = *(const float4 *)(a.sw + n);
      sw[0] = t4.x; sw[1] = t4.y; sw[2] = t4.z; sw[3] = t4.w;
    }
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int64_t m = m0 + wm * TM * 16 + j * 16 + (lane & 15);
      if (m >= a.M) continue;
      if constexpr (EPI == EPI_RAW_I32) {
        if constexpr (!BF16) {
          v4i v = acc[i][j];
          *(int4 *)(a.c32 + m * a.N + n) = make_int4(v[0], v[1], v[2], v[3]);
        }
      } else {
        float y[4];
        if constexpr (BF16) {
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = acc[i][j][r];
        } else {
          const float sa = a.sa[m];
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = ((float)acc[i][j][r] * sa) * sw[r];
        }
        if constexpr (EPI == EPI_QKV) {
          const int sec = n / a.d;
          const int c = n - sec * a.d;
          const int head = c / a.Dh;
          const int dh = c - head * a.Dh;
          if (sec < 2) {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              const float2 cs = rope_cs(a.rope, a.rg, dh / 2 + p, m);
              const float u0 = y[2 * p], u1 = y[2 * p + 1];
              y[2 * p] = u0 * cs.x - u1 * cs.y;
              y[2 * p + 1] = u0 * cs.y + u1 * cs.x;
            }
            store4<OUTF32>(sec == 0 ? a.q : a.k, ((int64_t)head * a.M + m) * a.Dh + dh, y[0],
                           y[1], y[2], y[3]);
          } else {
            const int64_t base = ((int64_t)head * a.Dh + dh) * a.M + m;
#pragma unroll
            for (int r = 0; r < 4; ++r) store1<OUTF32>(a.vt, base + (int64_t)r * a.M, y[r]);
          }
        } else if constexpr (EPI == EPI_GELU) {
          store4<OUTF32>(a.out, m * a.N + n, gelu_erf(y[0]), gelu_erf(y[1]), gelu_erf(y[2]),
                         gelu_erf(y[3]));
        } else if constexpr (EPI == EPI_RESID) {
          float r4[4];
          load4<RESF32>(a.res, m * a.N + n, r4);
          const float4 g4 = *(const float4 *)(a.gate + n);
          store4<OUTF32>(a.out, m * a.N + n, r4[0] + g4.x * y[0], r4[1] + g4.y * y[1],
                         r4[2] + g4.z * y[2], r4[3] + g4.w * y[3]);
        }
      }
    }
  }
}

#undef H3K_GLOAD
#undef H3K_LSTORE
#undef H3K_COMPUTE

template <int BN, int BM, int WN, int WM, bool BF16, int EPI, bool OUTF32, bool RESF32>
static hipError_t run_gemm(const GemmArgs &a, hipStream_t s) {
  auto kern = gemm_kernel<BN, BM, WN, WM, BF16, EPI, OUTF32, RESF32>;
  constexpr size_t lds = gemm_lds_bytes<BN, BM>();
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t m_tiles = (a.M + BM - 1) / BM;
  const int64_t nwg = m_tiles * (a.N / BN);
  kern<<<dim3((unsigned)nwg), dim3(WN * WM * 64), lds, s>>>(a);
  return hipGetLastError();
}

template <bool BF16, int EPI, bool OUTF32, bool RESF32>
static hipError_t gemm_tiles(const GemmArgs &a, hipStream_t s) {
  return run_gemm<H3K_GEMM_BN, H3K_GEMM_BM, H3K_GEMM_WN, H3K_GEMM_WM, BF16, EPI, OUTF32, RESF32>(a, s);
}

// instantiated type combinations:
//   QKV    int8 -> bf16 | int8 -> fp32 | bf16 -> bf16
//   GELU   int8 -> fp32 | bf16 -> bf16
//   RESID  residual/out: bf16/fp32, fp32/fp32, fp32/bf16 (int8 and bf16 operands)
static hipError_t gemm_dispatch(EpiKind kind, const GemmArgs &a, hipStream_t s) {
  const bool B = a.bf16_ops, OF = a.out_f32, RF = a.res_f32;
  switch (kind) {
    case EPI_QKV:
      if (B) return OF ? hipErrorInvalidValue : gemm_tiles<true, EPI_QKV, false, false>(a, s);
      return OF ? gemm_tiles<false, EPI_QKV, true, false>(a, s)
                : gemm_tiles<false, EPI_QKV, false, false>(a, s);
    case EPI_GELU:
      if (B) return OF ? hipErrorInvalidValue : gemm_tiles<true, EPI_GELU, false, false>(a, s);
      return OF ? gemm_tiles<false, EPI_GELU, true, false>(a, s) : hipErrorInvalidValue;
    case EPI_RESID:
      if (!RF && OF)
        return B ? gemm_tiles<true, EPI_RESID, true, false>(a, s)
                 : gemm_tiles<false, EPI_RESID, true, false>(a, s);
      if (RF && OF)
        return B ? hipErrorInvalidValue : gemm_tiles<false, EPI_RESID, true, true>(a, s);
      if (RF && !OF)
        return B ? gemm_tiles<true, EPI_RESID, false, true>(a, s)
                 : gemm_tiles<false, EPI_RESID, false, true>(a, s);
      return hipErrorInvalidValue;
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(EpiKind kind, const GemmArgs &a, hipStream_t s) {
  if (kind == EPI_RAW_I32) {
    if (a.bf16_ops || a.out_f32) return hipErrorInvalidValue;
    return run_gemm<H3K_GEMM_BN, H3K_GEMM_BM, H3K_GEMM_WN, H3K_GEMM_WM, false, EPI_RAW_I32, false,
                    false>(a, s);
  }
  return gemm_dispatch(kind, a, s);
}

}  // namespace h3k
