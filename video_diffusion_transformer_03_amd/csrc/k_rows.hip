// Bandwidth-bound kernels of the block: AdaLN modulation GEMV, the fused
// LayerNorm + modulate + per-token int8 quantiser, the plain per-row quantiser, the RoPE
// rotation table, and horizontal token pairing / unpairing.
//
// Pages: "h3-metal: Apple Silicon을 위한 네이티브 MiniMax-H3 추론", section "Int8 양자화"
// (the QKV and MLP activation quantisers folded into the gated AdaLN kernel, dynamic
// per-row activation scales) and the "속도 및 품질 트레이드오프" table (token reduction
// pairs horizontal video tokens in the middle blocks).
#include "h3k_internal.h"

#include <math.h>

namespace h3k {

// ============================================================== RoPE table
RopeGeom rope_geom(int head_dim, int T, int Hg, int Wg, float w_scale, float w_offset) {
  RopeGeom g;
  int P = head_dim / 2, p3 = P / 3;
  g.Pt = P - 2 * p3;
  g.Ph = p3;
  g.Pw = p3;
  g.T = T;
  g.Hg = Hg;
  g.Wg = Wg;
  g.base_h = T * g.Pt;
  g.base_w = g.base_h + Hg * g.Ph;
  g.w_scale = w_scale;
  g.w_offset = w_offset;
  return g;
}
size_t rope_table_entries(const RopeGeom &g) {
  return (size_t)g.T * g.Pt + (size_t)g.Hg * g.Ph + (size_t)g.Wg * g.Pw;
}

// entry (axis a, position p, pair j) -> (cos, sin) of p * theta^(-j / P_a), in fp64, stored
// as float2, or as double2 for the fp32 debug path's fp64 QKV epilogue
template <typename CS>
__global__ void rope_table_kernel(CS *tbl, RopeGeom g, double theta) {
  int e = blockIdx.x * blockDim.x + threadIdx.x;
  int n = g.T * g.Pt + g.Hg * g.Ph + g.Wg * g.Pw;
  if (e >= n) return;
  double pos;
  int j, P;
  if (e < g.base_h) {
    P = g.Pt; pos = e / P; j = e % P;
  } else if (e < g.base_w) {
    int r = e - g.base_h;
    P = g.Ph; pos = r / P; j = r % P;
  } else {
    int r = e - g.base_w;
    P = g.Pw; j = r % P;
    pos = (double)(r / P) * (double)g.w_scale + (double)g.w_offset;
  }
  double ang = pos * pow(theta, -(double)j / (double)P);
  tbl[e].x = cos(ang);
  tbl[e].y = sin(ang);
}

hipError_t launch_rope_table(void *tbl, const RopeGeom &g, float theta, bool f64, hipStream_t s) {
  int n = (int)rope_table_entries(g);
  if (f64)
    rope_table_kernel<<<(n + 255) / 256, 256, 0, s>>>((double2 *)tbl, g, (double)theta);
  else
    rope_table_kernel<<<(n + 255) / 256, 256, 0, s>>>((float2 *)tbl, g, (double)theta);
  return hipGetLastError();
}

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// ============================================================== AdaLN GEMV
// sum over the 64 lanes of a wave in fp64 (lane shuffles; fp64 paths only)
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// m[i] = sum_j W[i, j] c[j]. One wave per output row; each lane keeps the slice of c
// it multiplies in registers (MAXC 16-byte chunks of W per lane). W is read once, with
// nontemporal loads (12% faster than cached loads at 6d x d_c = 30720 x 5120).
// F64: products and sums in fp64 (a bf16 x fp32 product is exact there), one rounding to
// fp32 at the end, so m is the fp32 value nearest the exact sum (fp32 debug path).
template <int MAXC, bool F64>
__global__ __launch_bounds__(256) void adaln_kernel(const uint16_t *__restrict__ W,
                                                    const float *__restrict__ c,
                                                    float *__restrict__ m, int64_t n_out,
                                                    int dc, int rows_per_wave) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nch = dc / 8;
  float cv[MAXC][8];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    int ch = lane + 64 * i;
    if (ch < nch) {
      float4 a = *(const float4 *)(c + ch * 8);
      float4 b = *(const float4 *)(c + ch * 8 + 4);
      cv[i][0] = a.x; cv[i][1] = a.y; cv[i][2] = a.z; cv[i][3] = a.w;
      cv[i][4] = b.x; cv[i][5] = b.y; cv[i][6] = b.z; cv[i][7] = b.w;
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) cv[i][t] = 0.f;
    }
  }
  for (int r = 0; r < rows_per_wave; ++r) {
    int64_t row = wave * rows_per_wave + r;
    if (row >= n_out) break;
    const uint16_t *wr = W + row * dc;
    float acc = 0.f;
    double acc64 = 0.0;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      int ch = lane + 64 * i;
      if (ch < nch) {
        const v4u u = __builtin_nontemporal_load((const v4u *)(wr + ch * 8));
        const uint32_t w4[4] = {u[0], u[1], u[2], u[3]};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if constexpr (F64) {
            acc64 = fma((double)__uint_as_float(w4[t] << 16), (double)cv[i][2 * t], acc64);
            acc64 = fma((double)__uint_as_float(w4[t] & 0xffff0000u), (double)cv[i][2 * t + 1], acc64);
          } else {
            acc = fmaf(__uint_as_float(w4[t] << 16), cv[i][2 * t], acc);
            acc = fmaf(__uint_as_float(w4[t] & 0xffff0000u), cv[i][2 * t + 1], acc);
          }
        }
      }
    }
    if constexpr (F64) acc = (float)wave_sum_f64(acc64);
    else acc = wave_sum(acc);
    if (lane == 0) m[row] = acc;
  }
}

hipError_t launch_adaln(const uint16_t *w, const float *c, float *m, int64_t n_out, int dc,
                        bool f64, hipStream_t s) {
  const int rpw = 4;
  int64_t waves = (n_out + rpw - 1) / rpw;
  dim3 grid((unsigned)((waves + 3) / 4));
  int maxc = (dc / 8 + 63) / 64;
  if (maxc <= 4)
    (f64 ? adaln_kernel<4, true> : adaln_kernel<4, false>)<<<grid, 256, 0, s>>>(w, c, m, n_out, dc, rpw);
  else if (maxc <= 10)
    (f64 ? adaln_kernel<10, true> : adaln_kernel<10, false>)<<<grid, 256, 0, s>>>(w, c, m, n_out, dc, rpw);
  else
    (f64 ? adaln_kernel<16, true> : adaln_kernel<16, false>)<<<grid, 256, 0, s>>>(w, c, m, n_out, dc, rpw);
  return hipGetLastError();
}

// ============================================================== per-row kernels
// One row per WPR waves; 256 threads = 4 waves per block, so 4 / WPR rows per block.
// Each thread holds up to MAXV vectors of 8 elements of its row in registers; the row is
// read from HBM once and written once.
__device__ __forceinline__ void load8(const uint16_t *p, float v[8]) {
  uint4 u = *(const uint4 *)p;
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    v[2 * t] = __uint_as_float(w[t] << 16);
    v[2 * t + 1] = __uint_as_float(w[t] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float *p, float v[8]) {
  float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// streaming variant for fp32 inputs read exactly once (nontemporal: no cache allocation);
// bf16 rows of the quantisers stay packed and load their own way
__device__ __forceinline__ void load8_nt(const float *p, float v[8]) {
  const v4f a = __builtin_nontemporal_load((const v4f *)p);
  const v4f b = __builtin_nontemporal_load((const v4f *)(p + 4));
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    v[t] = a[t];
    v[4 + t] = b[t];
  }
}

template <int WPR>
__device__ __forceinline__ float group_reduce(float v, bool is_max, float *red) {
  v = is_max ? wave_max(v) : wave_sum(v);
  if constexpr (WPR == 1) {
    return v;
  } else {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();  // earlier readers of red are done
    if (lane == 0) red[wave] = v;
    __syncthreads();
    const int g0 = (wave / WPR) * WPR;
    float r = red[g0];
#pragma unroll
    for (int j = 1; j < WPR; ++j) r = is_max ? fmaxf(r, red[g0 + j]) : r + red[g0 + j];
    return r;
  }
}

// sum over the WPR waves of a row in fp64 (shuffles within a wave, then LDS)
template <int WPR>
__device__ __forceinline__ double group_sum_f64(double v, double *red) {
  v = wave_sum_f64(v);
  if constexpr (WPR == 1) {
    return v;
  } else {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();  // earlier readers of red are done
    if (lane == 0) red[wave] = v;
    __syncthreads();
    const int g0 = (wave / WPR) * WPR;
    double r = red[g0];
#pragma unroll
    for (int j = 1; j < WPR; ++j) r += red[g0 + j];
    return r;
  }
}

enum { RM_LNQ = 0, RM_LN_BF16 = 1, RM_Q = 2 };

template <int MODE, typename Tin, int WPR, int MAXV>
__global__ __launch_bounds__(256) void row_kernel(const Tin *__restrict__ x,
                                                  const float *__restrict__ shift,
                                                  const float *__restrict__ scale,
                                                  int64_t rows, int cols, float eps,
                                                  int8_t *__restrict__ q,
                                                  float *__restrict__ sc,
                                                  uint16_t *__restrict__ hout) {
  __shared__ float red[4];
  // fp32 rows of the LayerNorm quantiser (fp32 debug path): mean, variance and modulation in
  // fp64, one rounding of h to fp32 before the quantiser, so that h is the fp32 value
  // nearest the exact one and the codes do not depend on the summation order
  constexpr bool F64 = std::is_same<Tin, float>::value && MODE == RM_LNQ;
  __shared__ double red64[F64 ? 4 : 1];
  // one-wave rows (d <= 5120): the block's four rows share shift and scale through LDS, so
  // each row reads them from L2 a quarter as often and their loads overlap the row's
  constexpr bool LDSP = (MODE == RM_LNQ || MODE == RM_LN_BF16) && WPR == 1 && MAXV <= 10;
  // four planes of MAXV * 64 float4: shift[8c .. 8c+3], shift[8c+4 ..], scale likewise, so
  // that lane c's 16-byte reads of a plane are consecutive (no bank conflicts)
  constexpr int LP = LDSP ? MAXV * 64 : 1;
  __shared__ float4 lss[4 * LP];
  // 16-bit rows stay packed in registers (half the registers of an fp32 copy): a bf16
  // LayerNorm row through its mean and variance passes (the modulated fp32 values then
  // replace it), a bf16 or fp16 quantiser row throughout (absmax on the bit patterns,
  // unpacked again for the codes). Tin = _Float16 (fp16 rows) occurs only in RM_Q.
  constexpr bool HALF = std::is_same<Tin, _Float16>::value;
  static_assert(!HALF || MODE == RM_Q, "fp16 rows are quantised only");
  constexpr bool PACKED = std::is_same<Tin, uint16_t>::value || HALF;
  constexpr int NT = WPR * 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * (4 / WPR) + wave / WPR;
  const int tid = (wave % WPR) * 64 + lane;
  const bool active = row < rows;
  const int nvec = cols / 8;
  const Tin *xr = x + (active ? row : 0) * (int64_t)cols;

  float v[MAXV][8];
  uint4 raw[PACKED ? MAXV : 1];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    int c = tid + i * NT;
    if constexpr (PACKED && MODE == RM_Q) {  // O and g are read once
      raw[i] = make_uint4(0, 0, 0, 0);
      if (active && c < nvec) {
        const v4u u = __builtin_nontemporal_load((const v4u *)(xr + (int64_t)c * 8));
        raw[i] = make_uint4(u[0], u[1], u[2], u[3]);
      }
    } else if constexpr (PACKED) {
      raw[i] = (active && c < nvec) ? *(const uint4 *)(xr + (int64_t)c * 8) : make_uint4(0, 0, 0, 0);
    } else if (active && c < nvec) {
      if constexpr (MODE == RM_Q)  // O and g are read once
        load8_nt(xr + (int64_t)c * 8, v[i]);
      else
        load8(xr + (int64_t)c * 8, v[i]);
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) v[i][t] = 0.f;
    }
  }

  if constexpr (LDSP) {
    const int nv = cols / 8;  // <= MAXV * 64
    for (int c = threadIdx.x; c < nv; c += 256) {
      lss[c] = *(const float4 *)(shift + c * 8);
      lss[LP + c] = *(const float4 *)(shift + c * 8 + 4);
      lss[2 * LP + c] = *(const float4 *)(scale + c * 8);
      lss[3 * LP + c] = *(const float4 *)(scale + c * 8 + 4);
    }
    __syncthreads();
  }

  if constexpr (F64) {
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < MAXV; ++i)
#pragma unroll
      for (int t = 0; t < 8; ++t) s += (double)v[i][t];
    const double mean = group_sum_f64<WPR>(s, red64) / (double)cols;
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      int c = tid + i * NT;
      if (c < nvec) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const double dlt = (double)v[i][t] - mean;
          ss = fma(dlt, dlt, ss);
        }
      }
    }
    const double var = group_sum_f64<WPR>(ss, red64) / (double)cols;
    const double rstd = 1.0 / sqrt(var + (double)eps);
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      int c = tid + i * NT;
      if (c < nvec) {
        float sh[8], sca[8];
        if constexpr (LDSP) {
          const float4 a0 = lss[c], a1 = lss[LP + c];
          const float4 b0 = lss[2 * LP + c], b1 = lss[3 * LP + c];
          sh[0] = a0.x; sh[1] = a0.y; sh[2] = a0.z; sh[3] = a0.w;
          sh[4] = a1.x; sh[5] = a1.y; sh[6] = a1.z; sh[7] = a1.w;
          sca[0] = b0.x; sca[1] = b0.y; sca[2] = b0.z; sca[3] = b0.w;
          sca[4] = b1.x; sca[5] = b1.y; sca[6] = b1.z; sca[7] = b1.w;
        } else {
          load8(shift + c * 8, sh);
          load8(scale + c * 8, sca);
        }
#pragma unroll
        for (int t = 0; t < 8; ++t)
          v[i][t] = (float)(((double)v[i][t] - mean) * rstd * (1.0 + (double)sca[t]) + (double)sh[t]);
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) v[i][t] = 0.f;
      }
    }
  } else if constexpr (MODE == RM_LNQ || MODE == RM_LN_BF16) {
    float s = 0.f;
    if constexpr (PACKED) {
      // pairs of bf16 summed exactly by a dot product with (1, 1)
      const v2bf ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int i = 0; i < MAXV; ++i) {
        const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
        for (int t = 0; t < 4; ++t)
          s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, w[t]), ones, s, false);
      }
#pragma unroll
      for (int i = 0; i < MAXV; ++i) {
        const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v[i][2 * t] = __uint_as_float(w[t] << 16);
          v[i][2 * t + 1] = __uint_as_float(w[t] & 0xffff0000u);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < MAXV; ++i)
#pragma unroll
        for (int t = 0; t < 8; ++t) s += v[i][t];
    }
    const float mean = group_reduce<WPR>(s, false, red) / (float)cols;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      int c = tid + i * NT;
      if (c < nvec) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          float dlt = v[i][t] - mean;
          ss = fmaf(dlt, dlt, ss);
        }
      }
    }
    const float var = group_reduce<WPR>(ss, false, red) / (float)cols;
    const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      int c = tid + i * NT;
      if (c < nvec) {
        float sh[8], sca[8];
        if constexpr (LDSP) {
          const float4 a0 = lss[c], a1 = lss[LP + c];
          const float4 b0 = lss[2 * LP + c], b1 = lss[3 * LP + c];
          sh[0] = a0.x; sh[1] = a0.y; sh[2] = a0.z; sh[3] = a0.w;
          sh[4] = a1.x; sh[5] = a1.y; sh[6] = a1.z; sh[7] = a1.w;
          sca[0] = b0.x; sca[1] = b0.y; sca[2] = b0.z; sca[3] = b0.w;
          sca[4] = b1.x; sca[5] = b1.y; sca[6] = b1.z; sca[7] = b1.w;
        } else {
          load8(shift + c * 8, sh);
          load8(scale + c * 8, sca);
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) v[i][t] = (v[i][t] - mean) * rstd * (1.0f + sca[t]) + sh[t];
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) v[i][t] = 0.f;
      }
    }
  }

  if constexpr (MODE == RM_LN_BF16) {
    if (active) {
#pragma unroll
      for (int i = 0; i < MAXV; ++i) {
        int c = tid + i * NT;
        if (c < nvec) {
          uint4 o;
          o.x = pack_bf2(v[i][0], v[i][1]);
          o.y = pack_bf2(v[i][2], v[i][3]);
          o.z = pack_bf2(v[i][4], v[i][5]);
          o.w = pack_bf2(v[i][6], v[i][7]);
          *(uint4 *)(hout + row * (int64_t)cols + (int64_t)c * 8) = o;
        }
      }
    }
  } else {
    constexpr bool RAWQ = PACKED && MODE == RM_Q;
    float a = 0.f;
    if constexpr (RAWQ) {
      // |bf16| and |fp16| order like their 15 magnitude bits read as an integer: the row's
      // largest magnitude is an integer maximum over the halves, then widened to fp32 once
      uint32_t mi = 0;
#pragma unroll
      for (int i = 0; i < MAXV; ++i) {
        const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) mi = max(mi, max(w[t] & 0x7fffu, (w[t] >> 16) & 0x7fffu));
      }
      a = HALF ? h2f_lo(mi) : __uint_as_float(mi << 16);
    } else {
#pragma unroll
      for (int i = 0; i < MAXV; ++i)
#pragma unroll
        for (int t = 0; t < 8; ++t) a = fmaxf(a, fabsf(v[i][t]));
    }
    a = group_reduce<WPR>(a, true, red);
    const float inv = a > 0.f ? 127.0f / a : 0.f;
    if (active) {
      if (tid == 0) sc[row] = a / 127.0f;
#pragma unroll
      for (int i = 0; i < MAXV; ++i) {
        int c = tid + i * NT;
        if (c < nvec) {
          float e[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) e[t] = v[i][t];
          if constexpr (RAWQ) {
            const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              e[2 * t] = HALF ? h2f_lo(w[t]) : __uint_as_float(w[t] << 16);
              e[2 * t + 1] = HALF ? h2f_hi(w[t]) : __uint_as_float(w[t] & 0xffff0000u);
            }
          }
          uint32_t lo = 0, hi = 0;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            lo |= ((uint32_t)quant_code(e[t], inv) & 0xffu) << (8 * t);
            hi |= ((uint32_t)quant_code(e[t + 4], inv) & 0xffu) << (8 * t);
          }
          *(uint2 *)(q + row * (int64_t)cols + (int64_t)c * 8) = make_uint2(lo, hi);
        }
      }
    }
  }
}

template <int MODE, typename Tin, int WPR>
static hipError_t rows_dispatch(const Tin *x, const float *shift, const float *scale,
                                int64_t rows, int cols, float eps, int8_t *q, float *sc,
                                uint16_t *hout, hipStream_t s) {
  const int nvec = cols / 8;
  const int need = (nvec + WPR * 64 - 1) / (WPR * 64);
  dim3 grid((unsigned)((rows + (4 / WPR) - 1) / (4 / WPR)));
#define H3K_ROWS(MV)                                                                    \
  row_kernel<MODE, Tin, WPR, MV><<<grid, 256, 0, s>>>(x, shift, scale, rows, cols, eps, q, \
                                                      sc, hout)
  if (need <= 1) H3K_ROWS(1);
  else if (need <= 2) H3K_ROWS(2);
  else if (need <= 4) H3K_ROWS(4);
  else if (need <= 8) H3K_ROWS(8);
  else if (need <= 10) H3K_ROWS(10);
  else H3K_ROWS(16);
#undef H3K_ROWS
  return hipGetLastError();
}

template <int MODE, typename Tin>
static hipError_t rows_wpr(const Tin *x, const float *shift, const float *scale,
                           int64_t rows, int cols, float eps, int8_t *q, float *sc,
                           uint16_t *hout, hipStream_t s) {
  // one wave per row while a lane needs at most 10 vectors, else four waves per row
  if (cols / 8 <= 640)
    return rows_dispatch<MODE, Tin, 1>(x, shift, scale, rows, cols, eps, q, sc, hout, s);
  return rows_dispatch<MODE, Tin, 4>(x, shift, scale, rows, cols, eps, q, sc, hout, s);
}

hipError_t launch_rows(int mode, const void *x, int x_type, const float *shift,
                       const float *scale, int64_t rows, int cols, float eps, int8_t *q,
                       float *sc, uint16_t *hout, hipStream_t s) {
  if (x_type == ROW_F16) {
    if (mode != RM_Q) return hipErrorInvalidValue;
    return rows_wpr<RM_Q, _Float16>((const _Float16 *)x, shift, scale, rows, cols, eps, q, sc,
                                    hout, s);
  }
  if (x_type == ROW_F32) {
    const float *xf = (const float *)x;
    if (mode == RM_LNQ) return rows_wpr<RM_LNQ, float>(xf, shift, scale, rows, cols, eps, q, sc, hout, s);
    if (mode == RM_Q) return rows_wpr<RM_Q, float>(xf, shift, scale, rows, cols, eps, q, sc, hout, s);
    return rows_wpr<RM_LN_BF16, float>(xf, shift, scale, rows, cols, eps, q, sc, hout, s);
  }
  const uint16_t *xb = (const uint16_t *)x;
  if (mode == RM_LNQ) return rows_wpr<RM_LNQ, uint16_t>(xb, shift, scale, rows, cols, eps, q, sc, hout, s);
  if (mode == RM_LN_BF16) return rows_wpr<RM_LN_BF16, uint16_t>(xb, shift, scale, rows, cols, eps, q, sc, hout, s);
  return rows_wpr<RM_Q, uint16_t>(xb, shift, scale, rows, cols, eps, q, sc, hout, s);
}

// ============================================================== token pairing
// One thread per 8 channels of one output (paired) token.
template <typename T>
__global__ __launch_bounds__(256) void token_pair_kernel(const T *__restrict__ x,
                                                         T *__restrict__ xr,
                                                         T *__restrict__ xr2, int64_t n_out,
                                                         int d) {
  const int nv = d / 8;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_out * nv) return;
  int64_t tok = i / nv;  // paired token index: ((t*Hg + h) * Wg/2 + j)
  int c = (int)(i % nv) * 8;
  // source tokens 2*tok and 2*tok + 1 (same (t, h), w = 2j and 2j + 1)
  float a[8], b[8], r[8];
  load8(x + (2 * tok) * (int64_t)d + c, a);
  load8(x + (2 * tok + 1) * (int64_t)d + c, b);
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = (a[t] + b[t]) * 0.5f;
  T *o1 = xr + tok * (int64_t)d + c;
  T *o2 = xr2 + tok * (int64_t)d + c;
  if constexpr (sizeof(T) == 2) {
    uint4 o = make_uint4(pack_bf2(r[0], r[1]), pack_bf2(r[2], r[3]), pack_bf2(r[4], r[5]),
                         pack_bf2(r[6], r[7]));
    *(uint4 *)o1 = o;
    *(uint4 *)o2 = o;
  } else {
    float4 p = make_float4(r[0], r[1], r[2], r[3]), q = make_float4(r[4], r[5], r[6], r[7]);
    ((float4 *)o1)[0] = p; ((float4 *)o1)[1] = q;
    ((float4 *)o2)[0] = p; ((float4 *)o2)[1] = q;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void token_unpair_kernel(T *__restrict__ x,
                                                           const T *__restrict__ xo,
                                                           const T *__restrict__ xi,
                                                           int64_t n_out, int d) {
  const int nv = d / 8;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_out * nv) return;
  int64_t tok = i / nv;
  int c = (int)(i % nv) * 8;
  float o[8], in[8], delta[8];
  load8(xo + tok * (int64_t)d + c, o);
  load8(xi + tok * (int64_t)d + c, in);
#pragma unroll
  for (int t = 0; t < 8; ++t) delta[t] = o[t] - in[t];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    T *p = x + (2 * tok + s2) * (int64_t)d + c;
    float v[8];
    load8(p, v);
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] += delta[t];
    if constexpr (sizeof(T) == 2) {
      *(uint4 *)p = make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]),
                               pack_bf2(v[6], v[7]));
    } else {
      ((float4 *)p)[0] = make_float4(v[0], v[1], v[2], v[3]);
      ((float4 *)p)[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

hipError_t launch_token_pair(const void *x, void *xr, void *xr2, bool f32, int T, int Hg,
                             int Wg, int d, hipStream_t s) {
  int64_t n_out = (int64_t)T * Hg * (Wg / 2);
  int64_t n = n_out * (d / 8);
  dim3 grid((unsigned)((n + 255) / 256));
  if (f32)
    token_pair_kernel<float><<<grid, 256, 0, s>>>((const float *)x, (float *)xr, (float *)xr2, n_out, d);
  else
    token_pair_kernel<uint16_t><<<grid, 256, 0, s>>>((const uint16_t *)x, (uint16_t *)xr,
                                                     (uint16_t *)xr2, n_out, d);
  return hipGetLastError();
}

hipError_t launch_token_unpair(void *x, const void *xo, const void *xi, bool f32, int T,
                               int Hg, int Wg, int d, hipStream_t s) {
  int64_t n_out = (int64_t)T * Hg * (Wg / 2);
  int64_t n = n_out * (d / 8);
  dim3 grid((unsigned)((n + 255) / 256));
  if (f32)
    token_unpair_kernel<float><<<grid, 256, 0, s>>>((float *)x, (const float *)xo, (const float *)xi, n_out, d);
  else
    token_unpair_kernel<uint16_t><<<grid, 256, 0, s>>>((uint16_t *)x, (const uint16_t *)xo,
                                                       (const uint16_t *)xi, n_out, d);
  return hipGetLastError();
}

// device-to-device copy of n16 16-byte chunks (a kernel, so that a captured stack graph
// holds kernel nodes only)
__global__ __launch_bounds__(256) void copy16_kernel(uint4 *__restrict__ dst,
                                                     const uint4 *__restrict__ src, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    dst[i] = src[i];
}

hipError_t launch_copy16(void *dst, const void *src, int64_t n16, hipStream_t s) {
  const int64_t blocks = (n16 + 255) / 256;
  dim3 grid((unsigned)(blocks < 8192 ? blocks : 8192));
  copy16_kernel<<<grid, 256, 0, s>>>((uint4 *)dst, (const uint4 *)src, n16);
  return hipGetLastError();
}

// Denoising-loop element steps, one thread per 8 elements of [L, d]; x and y (the stack
// output) in the activation type T, v (velocity) and r (cached core residual) fp32:
//   SAMPLER_FRESH    r = y - x, v = y
//   SAMPLER_REUSED   v = x + r
//   SAMPLER_EULER    x = x + dt * v (rounded to T)
template <typename T>
__global__ __launch_bounds__(256) void sampler_kernel(int mode, T *__restrict__ x,
                                                      const T *__restrict__ y, float *__restrict__ v,
                                                      float *__restrict__ r, double dt, int64_t n8) {
  // fp32 activations (the debug path): fp64 arithmetic and the exact step, each stored value
  // rounded once to fp32; bf16 activations: fp32 arithmetic
  using A = typename std::conditional<sizeof(T) == 4, double, float>::type;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const int64_t o = i * 8;
  float xs[8];
  load8(x + o, xs);
  if (mode == SAMPLER_FRESH) {
    float ys[8];
    load8(y + o, ys);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      r[o + t] = (float)((A)ys[t] - (A)xs[t]);
      v[o + t] = ys[t];
    }
  } else if (mode == SAMPLER_REUSED) {
#pragma unroll
    for (int t = 0; t < 8; ++t) v[o + t] = (float)((A)xs[t] + (A)r[o + t]);
  } else {
    float out[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) out[t] = (float)((A)xs[t] + (A)dt * (A)v[o + t]);
    if constexpr (sizeof(T) == 2) {
      *(uint4 *)(x + o) = make_uint4(pack_bf2(out[0], out[1]), pack_bf2(out[2], out[3]),
                                     pack_bf2(out[4], out[5]), pack_bf2(out[6], out[7]));
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) x[o + t] = out[t];
    }
  }
}

hipError_t launch_sampler(int mode, void *x, const void *y, float *v, float *r, double dt,
                          int64_t n, bool f32, hipStream_t s) {
  const int64_t n8 = n / 8;
  dim3 grid((unsigned)((n8 + 255) / 256));
  if (f32)
    sampler_kernel<float><<<grid, 256, 0, s>>>(mode, (float *)x, (const float *)y, v, r, dt, n8);
  else
    sampler_kernel<uint16_t><<<grid, 256, 0, s>>>(mode, (uint16_t *)x, (const uint16_t *)y, v, r,
                                                  dt, n8);
  return hipGetLastError();
}

}  // namespace h3k
