// Multi-head softmax attention over the video tokens (no mask), flash-style: key/value
// tiles stream through LDS and an online softmax keeps the running row maximum and row
// sum, so memory stays O(L * d) at any sequence length.
//
// Inputs come head-major from the QKV projection ("h3-metal: Apple Silicon을 위한
// 네이티브 MiniMax-H3 추론", section "Metal 4 및 TensorOps": Q/K/V routed straight into
// head-major attention inputs). Layouts: Q, K [H, L, Dh]; V transposed [H, Dh, L];
// O [L, H*Dh] (token-major, head e in columns e*Dh .. e*Dh + Dh - 1).
//
// bf16 kernel: both products run on v_mfma_f32_16x16x32_bf16 in transposed form so that a
// lane always owns one query column:
//   S^T = K Q^T   (A = K rows from LDS, B = Q held in registers)
//   O^T = V^T P^T (A = V^T rows from LDS, B = P^T taken straight from the S^T registers)
// The 8 key slots of the P^T operand are the lane's own S^T values, and V^T is read
// with the same key order, so no cross-lane data movement is needed between the two
// products; the softmax statistics live in the same lane as the output columns they
// scale. P is rounded to bf16 for the second product; max, exp and sums are fp32.
#include "h3k_internal.h"

namespace h3k {

__device__ __forceinline__ uint4 ld16(const uint16_t *p) { return *(const uint4 *)p; }

#ifndef H3K_ATTN_OCC
#define H3K_ATTN_OCC 2  // waves per SIMD the register budget is sized for
#endif
#ifndef H3K_ATTN_KPAD
#define H3K_ATTN_KPAD 16  // elements of padding per K-tile row in LDS
#endif
#ifndef H3K_ATTN_VPAD
#define H3K_ATTN_VPAD 16  // elements of padding per V^T-tile row in LDS
#endif

template <int DH>
struct AttnCfg {
  static constexpr int BQ = 128;                  // queries per work-group (4 waves x 32)
  static constexpr int BK = 64;                   // keys per tile
  static constexpr int KP = DH + H3K_ATTN_KPAD;   // K tile row pitch (elements)
  static constexpr int VP = BK + H3K_ATTN_VPAD;   // V^T tile row pitch (elements)
  static constexpr int K_ELEMS = BK * KP;
  static constexpr int V_ELEMS = DH * VP;
  static constexpr size_t LDS = (size_t)2 * (K_ELEMS + V_ELEMS) * 2;
  static constexpr int KCH = BK * DH / 8 / 256;  // 16-byte chunks per thread, K tile
  static constexpr int VCH = DH * BK / 8 / 256;  // 16-byte chunks per thread, V^T tile
};

// Lazy rescaling: the running maximum used for exp2 is only moved when a row's true
// maximum exceeds it by more than 2^8 -- P stays <= 256 and the O/l rescale (one multiply
// per accumulator) is skipped in most tiles. Softmax is invariant to the subtracted
// constant, so the result is unchanged.
constexpr float kRescaleLog2 = 8.0f;

// Key order inside a 32-key block: S^T tile t (16 rows) takes key 8*(i/4) + 4*t + i%4 in
// its row i, so the 8 P^T slots a lane group g holds (rows 4g..4g+3 of tiles 0 and 1) are
// the 8 consecutive keys 8g..8g+7 -- one 16-byte V^T read per operand. The permutation is
// applied when the K tile is written to LDS (key k of a block goes to row krow_of(k)), so
// the fragment reads walk LDS rows in natural order (bank-conflict free at this pitch).
__device__ __forceinline__ int kperm(int t, int i) { return 8 * (i >> 2) + 4 * t + (i & 3); }
__device__ __forceinline__ int krow_of(int key) {  // inverse of kperm within 32-key blocks
  const int k = key & 31;
  return (key & ~31) + ((k >> 2) & 1) * 16 + (k >> 3) * 4 + (k & 3);
}

struct AttnState {
  v4f o[8][2];   // O^T accumulators (dh tile, query tile); up to DH = 128
  float m[2];    // running max (log2 domain, scaled) per query tile
  float l[2];    // per-lane partial row sums
};

// one K/V tile: S^T = K Q^T, online softmax, O^T += V^T P^T
template <int DH, bool MASK>
__device__ __forceinline__ void attn_tile(AttnState &st, const v8bf (&qf)[2][DH / 32],
                                          const uint16_t *cK, const uint16_t *cV, int lane,
                                          int64_t k0, int64_t L, float sl2) {
  using C = AttnCfg<DH>;
  constexpr int KP = C::KP, VP = C::VP, NKK = DH / 32, NDT = DH / 16;
  const int g = lane >> 4, c16 = lane & 15;
  v4f s[4][2];
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4) s[t4][0] = s[t4][1] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      v8bf kf = __builtin_bit_cast(v8bf, ld16(cK + (t4 * 16 + c16) * KP + kk * 32 + g * 8));
      s[t4][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[0][kk], s[t4][0], 0, 0, 0);
      s[t4][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[1][kk], s[t4][1], 0, 0, 0);
    }
  }
  // lane holds S^T for query c16 and keys k0 + (t4/2)*32 + kperm(t4&1, 4g + r)
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    if constexpr (MASK) {
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (k0 + (t4 >> 1) * 32 + kperm(t4 & 1, 4 * g + r) >= L) s[t4][qt][r] = -INFINITY;
    }
    // running max of the lane's 16 scores as a chain of three-input maxima (v_max3_f32;
    // this file is compiled without NaN quieting, see build.py)
    float mx = fmaxf(fmaxf(s[0][qt][0], s[0][qt][1]), s[0][qt][2]);
    mx = fmaxf(fmaxf(mx, s[0][qt][3]), s[1][qt][0]);
    mx = fmaxf(fmaxf(mx, s[1][qt][1]), s[1][qt][2]);
    mx = fmaxf(fmaxf(mx, s[1][qt][3]), s[2][qt][0]);
    mx = fmaxf(fmaxf(mx, s[2][qt][1]), s[2][qt][2]);
    mx = fmaxf(fmaxf(mx, s[2][qt][3]), s[3][qt][0]);
    mx = fmaxf(fmaxf(mx, s[3][qt][1]), s[3][qt][2]);
    mx = fmaxf(mx, s[3][qt][3]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = mx * sl2;
    const bool grow = mnew > st.m[qt] + kRescaleLog2;
    if (__builtin_amdgcn_read_exec() & __ballot(grow)) {
      const float mref = grow ? mnew : st.m[qt];
      const float alpha = __builtin_amdgcn_exp2f(st.m[qt] - mref);
      st.m[qt] = mref;
      st.l[qt] *= alpha;
#pragma unroll
      for (int i = 0; i < NDT; ++i) st.o[i][qt] *= alpha;
    }
    const float mneg = -st.m[qt];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        s[t4][qt][r] = __builtin_amdgcn_exp2f(fmaf(s[t4][qt][r], sl2, mneg));
  }
  // O^T += V^T P^T over two 32-key steps; slots of lane group g = keys 8g .. 8g+7. The
  // row sum l accumulates the same bf16-rounded P the matrix cores consume (one dot2 per
  // packed pair against (1, 1)), so O = sum(p v) / sum(p) is normalised consistently.
  const v2bf ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    v8bf pb[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      uint4 u;
      u.x = pack_bf2(s[2 * ks][qt][0], s[2 * ks][qt][1]);
      u.y = pack_bf2(s[2 * ks][qt][2], s[2 * ks][qt][3]);
      u.z = pack_bf2(s[2 * ks + 1][qt][0], s[2 * ks + 1][qt][1]);
      u.w = pack_bf2(s[2 * ks + 1][qt][2], s[2 * ks + 1][qt][3]);
      float l = st.l[qt];
      l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, u.x), ones, l, false);
      l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, u.y), ones, l, false);
      l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, u.z), ones, l, false);
      l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, u.w), ones, l, false);
      st.l[qt] = l;
      pb[qt] = __builtin_bit_cast(v8bf, u);
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      v8bf vf = __builtin_bit_cast(v8bf, ld16(cV + (dt * 16 + c16) * VP + ks * 32 + g * 8));
      st.o[dt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[0], st.o[dt][0], 0, 0, 0);
      st.o[dt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[1], st.o[dt][1], 0, 0, 0);
    }
  }
}

template <int DH, bool OF32>
__global__ __launch_bounds__(256, H3K_ATTN_OCC) void attn_bf16_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ Vt, void *__restrict__ Ov, int H, int64_t L, float sl2) {
  using C = AttnCfg<DH>;
  constexpr int BK = C::BK, KP = C::KP, VP = C::VP;
  constexpr int NKK = DH / 32;
  constexpr int NDT = DH / 16;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  uint16_t *sK = lds;                   // [2][BK][KP]
  uint16_t *sV = lds + 2 * C::K_ELEMS;  // [2][DH][VP]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int head = blockIdx.y;
  const int64_t q0 = (int64_t)blockIdx.x * C::BQ + wave * 32;
  const uint16_t *Qh = Q + (int64_t)head * L * DH;
  const uint16_t *Kh = K + (int64_t)head * L * DH;
  const uint16_t *Vh = Vt + (int64_t)head * DH * L;
  const int g = lane >> 4, c16 = lane & 15;
  const uint32_t Lu = (uint32_t)L;

  // Q^T operand: lane supplies query (q0 + qt*16 + c16), head dims kk*32 + g*8 .. +8;
  // query rows past L read row L-1 and are not stored
  v8bf qf[2][NKK];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int64_t qi = (q0 + qt * 16 + c16) < L ? (q0 + qt * 16 + c16) : (L - 1);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[qt][kk] = __builtin_bit_cast(v8bf, ld16(Qh + qi * DH + kk * 32 + g * 8));
  }

  AttnState st;
#pragma unroll
  for (int i = 0; i < 8; ++i) st.o[i][0] = st.o[i][1] = v4f{0.f, 0.f, 0.f, 0.f};
  st.m[0] = st.m[1] = -INFINITY;
  st.l[0] = st.l[1] = 0.f;

  // staged-tile coordinates: thread tid moves 16-byte chunk tid + 256*i of each tile.
  // K tile [BK][DH]: row kr0 + i*KRI, column kc; V^T tile [DH][BK]: row vr0 + i*VRI,
  // column vc. Element offsets are 32-bit (L*DH < 2^31).
  constexpr int KCPR = DH / 8, VCPR = BK / 8;   // chunks per row
  constexpr int KRI = 256 / KCPR, VRI = 256 / VCPR;
  const int kr0 = tid / KCPR, kc = (tid % KCPR) * 8;
  const int vr0 = tid / VCPR, vc = (tid % VCPR) * 8;
  uint4 rk[C::KCH], rv[C::VCH];
  // keys past L read key L-1 (K) or the last valid 8-key chunk (V^T; L % 8 == 0): their
  // scores are masked to -inf, so their p = 0 meets finite values
#define H3K_ATTN_GLOAD(kt_)                                                                    \
  {                                                                                            \
    const uint32_t k0_ = (uint32_t)(kt_) * BK;                                                 \
    _Pragma("unroll") for (int i = 0; i < C::KCH; ++i) {                                       \
      const uint32_t key = min(k0_ + (uint32_t)(kr0 + i * KRI), Lu - 1u);                      \
      rk[i] = ld16(Kh + key * DH + kc);                                                        \
    }                                                                                          \
    const uint32_t vkey = min(k0_ + (uint32_t)vc, Lu - 8u);                                    \
    _Pragma("unroll") for (int i = 0; i < C::VCH; ++i)                                         \
        rv[i] = ld16(Vh + (uint32_t)(vr0 + i * VRI) * Lu + vkey);                              \
  }
#define H3K_ATTN_LSTORE(buf_)                                                                  \
  {                                                                                            \
    _Pragma("unroll") for (int i = 0; i < C::KCH; ++i)                                         \
        *(uint4 *)(sK + (buf_) * C::K_ELEMS + krow_of(kr0 + i * KRI) * KP + kc) = rk[i];     \
    _Pragma("unroll") for (int i = 0; i < C::VCH; ++i)                                         \
        *(uint4 *)(sV + (buf_) * C::V_ELEMS + (vr0 + i * VRI) * VP + vc) = rv[i];              \
  }

  const int nkt = (int)((L + BK - 1) / BK);
  const bool tail = (L % BK) != 0;
  H3K_ATTN_GLOAD(0);
  H3K_ATTN_LSTORE(0);
  __syncthreads();
  for (int kt = 0; kt + 1 < nkt; ++kt) {
    const int cur = kt & 1;
    H3K_ATTN_GLOAD(kt + 1);
    attn_tile<DH, false>(st, qf, sK + cur * C::K_ELEMS, sV + cur * C::V_ELEMS, lane,
                         (int64_t)kt * BK, L, sl2);
    H3K_ATTN_LSTORE(cur ^ 1);
    __syncthreads();
  }
  {
    const int cur = (nkt - 1) & 1;
    if (tail)
      attn_tile<DH, true>(st, qf, sK + cur * C::K_ELEMS, sV + cur * C::V_ELEMS, lane,
                          (int64_t)(nkt - 1) * BK, L, sl2);
    else
      attn_tile<DH, false>(st, qf, sK + cur * C::K_ELEMS, sV + cur * C::V_ELEMS, lane,
                           (int64_t)(nkt - 1) * BK, L, sl2);
  }
#undef H3K_ATTN_GLOAD
#undef H3K_ATTN_LSTORE

  const int64_t ldo = (int64_t)H * DH;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float l = st.l[qt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = 1.0f / l;
    const int64_t qi = q0 + qt * 16 + c16;
    if (qi < L) {
      const int64_t obase = qi * ldo + (int64_t)head * DH + g * 4;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        v4f v = st.o[dt][qt];
        if constexpr (OF32) {
          *(float4 *)((float *)Ov + obase + dt * 16) =
              make_float4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
        } else {
          *(uint2 *)((uint16_t *)Ov + obase + dt * 16) =
              make_uint2(pack_bf2(v[0] * inv, v[1] * inv), pack_bf2(v[2] * inv, v[3] * inv));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------- fp32
// Debug path: fp32 everywhere, plain FMA arithmetic. 64 queries per work-group, four
// threads per query, each owning DH/4 head dims; 32-key tiles of K and V^T in LDS.
template <int DH>
__global__ __launch_bounds__(256) void attn_f32_kernel(const float *__restrict__ Q,
                                                       const float *__restrict__ K,
                                                       const float *__restrict__ Vt,
                                                       float *__restrict__ O, int H, int64_t L,
                                                       float sl2) {
  constexpr int TK = 32, DP = DH / 4;
  __shared__ float sK[TK][DH + 1];
  __shared__ float sV[DH][TK + 1];
  const int tid = threadIdx.x, head = blockIdx.y;
  const int part = tid & 3;
  const int64_t qi = (int64_t)blockIdx.x * 64 + (tid >> 2);
  const float *Qh = Q + (int64_t)head * L * DH;
  const float *Kh = K + (int64_t)head * L * DH;
  const float *Vh = Vt + (int64_t)head * DH * L;
  float q[DP], o[DP];
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    q[e] = qi < L ? Qh[qi * DH + part * DP + e] : 0.f;
    o[e] = 0.f;
  }
  float mrow = -INFINITY, lsum = 0.f;
  for (int64_t k0 = 0; k0 < L; k0 += TK) {
    __syncthreads();
    for (int i = tid; i < TK * DH; i += 256) {
      const int r = i / DH, c = i % DH;
      sK[r][c] = (k0 + r < L) ? Kh[(k0 + r) * DH + c] : 0.f;
    }
    for (int i = tid; i < TK * DH; i += 256) {
      const int r = i / TK, c = i % TK;
      sV[r][c] = (k0 + c < L) ? Vh[(int64_t)r * L + k0 + c] : 0.f;
    }
    __syncthreads();
    float s[TK];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < DP; ++e) a = fmaf(q[e], sK[j][part * DP + e], a);
      a += __shfl_xor(a, 1, 64);
      a += __shfl_xor(a, 2, 64);
      s[j] = (k0 + j < L) ? a * sl2 : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float mnew = fmaxf(mrow, mx);
    const float alpha = exp2f(mrow - mnew);
    mrow = mnew;
    lsum *= alpha;
#pragma unroll
    for (int e = 0; e < DP; ++e) o[e] *= alpha;
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      const float p = exp2f(s[j] - mnew);
      lsum += p;
#pragma unroll
      for (int e = 0; e < DP; ++e) o[e] = fmaf(p, sV[part * DP + e][j], o[e]);
    }
  }
  if (qi < L) {
    const float inv = 1.0f / lsum;
    float *orow = O + qi * (int64_t)H * DH + (int64_t)head * DH + part * DP;
#pragma unroll
    for (int e = 0; e < DP; ++e) orow[e] = o[e] * inv;
  }
}

template <int DH, bool OF32>
static hipError_t attn_mfma(const void *q, const void *k, const void *vt, void *o, int H,
                            int64_t L, float sl2, hipStream_t s) {
  using C = AttnCfg<DH>;
  auto kern = attn_bf16_kernel<DH, OF32>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid((unsigned)((L + C::BQ - 1) / C::BQ), (unsigned)H);
  kern<<<grid, 256, C::LDS, s>>>((const uint16_t *)q, (const uint16_t *)k,
                                 (const uint16_t *)vt, o, H, L, sl2);
  return hipGetLastError();
}

template <int DH>
static hipError_t attn_dispatch(const void *q, const void *k, const void *vt, void *o, int H,
                                int64_t L, float sl2, bool in_f32, bool out_f32, hipStream_t s) {
  if (in_f32) {
    dim3 grid((unsigned)((L + 63) / 64), (unsigned)H);
    attn_f32_kernel<DH><<<grid, 256, 0, s>>>((const float *)q, (const float *)k,
                                             (const float *)vt, (float *)o, H, L, sl2);
    return hipGetLastError();
  }
  return out_f32 ? attn_mfma<DH, true>(q, k, vt, o, H, L, sl2, s)
                 : attn_mfma<DH, false>(q, k, vt, o, H, L, sl2, s);
}

hipError_t launch_attention(const void *q, const void *k, const void *vt, void *o, int H,
                            int64_t L, int Dh, float scale, bool in_f32, bool out_f32,
                            hipStream_t s) {
  const float sl2 = scale * 1.4426950408889634f;  // exp(x) = exp2(x * log2(e))
  if (Dh == 128) return attn_dispatch<128>(q, k, vt, o, H, L, sl2, in_f32, out_f32, s);
  if (Dh == 64) return attn_dispatch<64>(q, k, vt, o, H, L, sl2, in_f32, out_f32, s);
  return hipErrorInvalidValue;
}

}  // namespace h3k
