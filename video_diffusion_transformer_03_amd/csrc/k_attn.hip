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

template <int DH>
struct AttnCfg {
  static constexpr int BQ = 128;        // queries per work-group (4 waves x 32)
  static constexpr int BK = 64;         // keys per tile
  static constexpr int KP = DH + 8;     // K tile row pitch (elements)
  static constexpr int VP = BK + 8;     // V^T tile row pitch (elements)
  static constexpr int K_ELEMS = BK * KP;
  static constexpr int V_ELEMS = DH * VP;
  static constexpr size_t LDS = (size_t)2 * (K_ELEMS + V_ELEMS) * 2;
  static constexpr int KCH = BK * DH / 8 / 256;  // 16-byte chunks per thread, K tile
  static constexpr int VCH = DH * BK / 8 / 256;  // 16-byte chunks per thread, V^T tile
};

#ifndef H3K_ATTN_OCC
#define H3K_ATTN_OCC 2  // waves per SIMD the register budget is sized for
#endif

template <int DH, bool OF32>
__global__ __launch_bounds__(256, H3K_ATTN_OCC) void attn_bf16_kernel(const uint16_t *__restrict__ Q,
                                                        const uint16_t *__restrict__ K,
                                                        const uint16_t *__restrict__ Vt,
                                                        void *__restrict__ Ov, int H,
                                                        int64_t L, float sl2) {
  using C = AttnCfg<DH>;
  constexpr int BK = C::BK, KP = C::KP, VP = C::VP;
  constexpr int NKK = DH / 32;  // K-steps of the QK^T product (32 head dims each)
  constexpr int NDT = DH / 16;  // 16-row output tiles along the head dim
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

  // Q^T operand: lane supplies query (q0 + qt*16 + c16), head dims kk*32 + g*8 .. +8
  v8bf qf[2][NKK];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    // query rows past L read row L-1; their outputs are not stored
    const int64_t qi = (q0 + qt * 16 + c16) < L ? (q0 + qt * 16 + c16) : (L - 1);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      uint4 u = ld16(Qh + qi * DH + kk * 32 + g * 8);
      qf[qt][kk] = __builtin_bit_cast(v8bf, u);
    }
  }

  v4f o[NDT][2];
#pragma unroll
  for (int i = 0; i < NDT; ++i) o[i][0] = o[i][1] = v4f{0.f, 0.f, 0.f, 0.f};
  float mrow[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};

  uint4 rk[C::KCH], rv[C::VCH];
  auto gload = [&](int kt) {
    const int64_t k0 = (int64_t)kt * BK;
#pragma unroll
    for (int i = 0; i < C::KCH; ++i) {
      const int c = tid + i * 256, row = c / (DH / 8), col = c % (DH / 8);
      // keys past L read key L-1: their scores are masked to -inf, so p = 0
      const int64_t key = (k0 + row) < L ? (k0 + row) : (L - 1);
      rk[i] = ld16(Kh + key * DH + col * 8);
    }
#pragma unroll
    for (int i = 0; i < C::VCH; ++i) {
      const int c = tid + i * 256, row = c / (BK / 8), col = c % (BK / 8);
      // L % 8 == 0: a chunk is all valid or all past L; chunks past L read the last valid
      // chunk, whose finite values meet p = 0
      const int64_t key = (k0 + col * 8) < L ? (k0 + col * 8) : (L - 8);
      rv[i] = ld16(Vh + (int64_t)row * L + key);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::KCH; ++i) {
      const int c = tid + i * 256, row = c / (DH / 8), col = c % (DH / 8);
      *(uint4 *)(sK + buf * C::K_ELEMS + row * KP + col * 8) = rk[i];
    }
#pragma unroll
    for (int i = 0; i < C::VCH; ++i) {
      const int c = tid + i * 256, row = c / (BK / 8), col = c % (BK / 8);
      *(uint4 *)(sV + buf * C::V_ELEMS + row * VP + col * 8) = rv[i];
    }
  };

  const int nkt = (int)((L + BK - 1) / BK);
  gload(0);
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nkt) gload(kt + 1);
    const uint16_t *cK = sK + cur * C::K_ELEMS;
    const uint16_t *cV = sV + cur * C::V_ELEMS;

    // S^T[key][query] for 4 key tiles x 2 query tiles
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

    // online softmax; lane holds keys kt*BK + t4*16 + g*4 + r of query c16
    const int64_t kbase = (int64_t)kt * BK + g * 4;
    const bool tail = (int64_t)(kt + 1) * BK > L;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float mx = -INFINITY;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = s[t4][qt][r] * sl2;
          if (tail && kbase + t4 * 16 + r >= L) v = -INFINITY;
          s[t4][qt][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(mrow[qt], mx);
      const float alpha = exp2f(mrow[qt] - mnew);
      mrow[qt] = mnew;
      float ps = 0.f;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = exp2f(s[t4][qt][r] - mnew);
          s[t4][qt][r] = p;
          ps += p;
        }
      lsum[qt] = lsum[qt] * alpha + ps;
#pragma unroll
      for (int i = 0; i < NDT; ++i) o[i][qt] *= alpha;
    }

    // O^T += V^T P^T over two 32-key steps
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
        pb[qt] = __builtin_bit_cast(v8bf, u);
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const uint16_t *vr = cV + (dt * 16 + c16) * VP + g * 4;
        uint2 v0 = *(const uint2 *)(vr + (2 * ks) * 16);
        uint2 v1 = *(const uint2 *)(vr + (2 * ks + 1) * 16);
        v8bf vf = __builtin_bit_cast(v8bf, make_uint4(v0.x, v0.y, v1.x, v1.y));
        o[dt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[0], o[dt][0], 0, 0, 0);
        o[dt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[1], o[dt][1], 0, 0, 0);
      }
    }

    if (kt + 1 < nkt) lstore(cur ^ 1);
    __syncthreads();
  }

  const int64_t ldo = (int64_t)H * DH;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float l = lsum[qt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = 1.0f / l;
    const int64_t qi = q0 + qt * 16 + c16;
    if (qi < L) {
      const int64_t obase = qi * ldo + (int64_t)head * DH + g * 4;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        v4f v = o[dt][qt];
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
