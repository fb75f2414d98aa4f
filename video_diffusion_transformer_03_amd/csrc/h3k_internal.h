// Internal declarations shared by the HIP translation units of libh3k.so.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>
#include <utility>

namespace h3k {

// ---------------------------------------------------------------- device helpers
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Compile-time loop: f(std::integral_constant<int, I>{}) for I = 0 .. N-1, every index a
// constant at inlining time (keeps small register arrays out of scratch memory).
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950)
__device__ __forceinline__ uint16_t f2bf(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
// two fp32 -> packed bf16 pair (a in the low half), round to nearest even
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  v2bf h = __builtin_convertvector((v2f){a, b}, v2bf);
  return __builtin_bit_cast(uint32_t, h);
}

// fp16 (IEEE binary16) counterparts: two fp32 -> packed fp16 pair (v_cvt_pk_f16_f32) and
// one fp32 -> fp16, round to nearest even; magnitudes above 65504 become infinite
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  v2h h = __builtin_convertvector((v2f){a, b}, v2h);
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ uint16_t f2h(float f) {
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}
// the low / high half of a packed pair widened to fp32 (exact)
__device__ __forceinline__ float h2f_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float h2f_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
// 16-bit matrix-core operands: bf16, or fp16 when F16. Both element types use the same
// 8-element (16-byte) fragments, so kernels carry them as v8bf bit patterns.
template <bool F16>
__device__ __forceinline__ uint32_t pack16(float a, float b) {
  if constexpr (F16)
    return pack_h2(a, b);
  else
    return pack_bf2(a, b);
}
template <bool F16>
__device__ __forceinline__ v4f mma16(v8bf a, v8bf b, v4f c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a),
                                                  __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// a fragment of eight 1.0 values in the operand type
template <bool F16>
__device__ __forceinline__ v8bf ones16() {
  if constexpr (F16) {
    const _Float16 one = (_Float16)1.0f;
    return __builtin_bit_cast(v8bf, v8h{one, one, one, one, one, one, one, one});
  } else {
    const __bf16 one = (__bf16)1.0f;
    return v8bf{one, one, one, one, one, one, one, one};
  }
}
// acc + the two halves of a packed pair (v_dot2 against (1, 1): exact products, fp32 sum)
template <bool F16>
__device__ __forceinline__ float add_pair16(uint32_t u, float acc) {
  if constexpr (F16) {
    const v2h ones = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(v2h, u), ones, acc, false);
  } else {
    const v2bf ones = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, u), ones, acc, false);
  }
}

// max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the 16-lane rows of the wave) with
// gfx950 row swaps in registers; a shuffle (__shfl_xor) would go through LDS
// (ds_bpermute) and wait for every outstanding LDS read.
__device__ __forceinline__ float rows_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// lane l receives x of the lane that the DPP control CTRL names (all sources valid)
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
// sum / max over the 64 lanes of a wave, the same value in every lane: within each 16-lane
// row by DPP (quad permutes [1,0,3,2] and [2,3,0,1], then half-row and row mirrors), then
// across rows with the row swaps. No LDS traffic.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  return rows_sum(v);
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));
  v = fmaxf(v, dpp_mov<0x4E>(v));
  v = fmaxf(v, dpp_mov<0x141>(v));
  v = fmaxf(v, dpp_mov<0x140>(v));
  return rows_max(v);
}

// symmetric int8 code of v given the fp32 reciprocal inv = 127 / absmax
__device__ __forceinline__ int quant_code(float v, float inv) {
  float r = __builtin_rintf(v * inv);
  r = fminf(fmaxf(r, -127.f), 127.f);
  return (int)r;
}

// ---------------------------------------------------------------- rope table
struct RopeGeom {
  int Pt, Ph, Pw;          // pairs per axis
  int T, Hg, Wg;           // grid
  int base_h, base_w;      // table offsets (entries) of the h and w axes; t starts at 0
  float w_scale, w_offset; // w position = w * w_scale + w_offset
};
RopeGeom rope_geom(int head_dim, int T, int Hg, int Wg, float w_scale, float w_offset);
size_t rope_table_entries(const RopeGeom &g);

// ---------------------------------------------------------------- launchers
// all return hipError_t of the launch (hipGetLastError)
hipError_t launch_rope_table(void *tbl, const RopeGeom &g, float theta, bool f64, hipStream_t s);
hipError_t launch_adaln(const uint16_t *w, const float *c, float *m, int64_t n_out, int dc,
                        bool f64, hipStream_t s);
// mode: 0 = LN + modulate + int8 quant, 1 = LN + modulate -> bf16, 2 = int8 quant only.
// x_type: ROW_BF16, ROW_F32, or ROW_F16 (mode 2 only)
enum RowType { ROW_BF16 = 0, ROW_F32 = 1, ROW_F16 = 2 };
hipError_t launch_rows(int mode, const void *x, int x_type, const float *shift,
                       const float *scale, int64_t rows, int cols, float eps, int8_t *q,
                       float *sc, uint16_t *hout, hipStream_t s);
hipError_t launch_token_pair(const void *x, void *xr, void *xr2, bool f32, int T, int Hg,
                             int Wg, int d, hipStream_t s);
hipError_t launch_token_unpair(void *x, const void *xo, const void *xi, bool f32, int T,
                               int Hg, int Wg, int d, hipStream_t s);
// denoising-loop element steps (see k_rows.hip); n % 8 == 0
enum SamplerMode { SAMPLER_FRESH = 0, SAMPLER_REUSED = 1, SAMPLER_EULER = 2 };
hipError_t launch_sampler(int mode, void *x, const void *y, float *v, float *r, double dt,
                          int64_t n, bool f32, hipStream_t s);
// dst = src, n16 16-byte chunks (both 16-byte aligned)
hipError_t launch_copy16(void *dst, const void *src, int64_t n16, hipStream_t s);

// GEMM: out = epilogue(A[M,K] . B[N,K]^T). A = activations (tokens), B = weights.
enum EpiKind { EPI_RAW_I32 = 0, EPI_QKV = 1, EPI_GELU = 2, EPI_RESID = 3 };
struct GemmArgs {
  const void *A;       // int8 or bf16 [M, K]
  const void *B;       // int8 or bf16 [N, K]
  // weights in the tiled layout of h3k_tile_weights (int8 codes, or the bytes of bf16
  // weights); when set, the one-wave-per-SIMD kernel reads them and B is not used
  const int8_t *Bt = nullptr;
  int64_t M;
  int N, K;            // K in elements
  bool bf16_ops;       // bf16 operands (fp32 accumulation, no dequant scales)
  bool out_f32;        // fp32 outputs instead of bf16
  bool res_f32;        // EPI_RESID: fp32 residual input instead of bf16
  const float *sa;     // per-row (token) scales [M]     (int8 only)
  const float *sw;     // per-column (channel) scales [N] (int8 only)
  // EPI_RAW_I32
  int32_t *c32;
  // EPI_QKV: q, k [H, M, Dh], vt [H, Dh, M]
  void *q, *k, *vt;
  int d, H, Dh;
  const void *rope;    // (cos, sin) table: float2, or double2 with fp32 outputs
  RopeGeom rg;
  float q_scale = 1.0f;  // EPI_QKV: factor applied to Q after RoPE, before it is rounded
  bool qkv_f16 = false;  // EPI_QKV, 16-bit outputs: Q, K, V^T stored as fp16 (else bf16)
  // EPI_GELU: out [M, N]; EPI_RESID: out[m,n] = res[m,n] + gate[n] * y
  void *out;
  const void *res;
  const float *gate;
};
hipError_t launch_gemm(EpiKind kind, const GemmArgs &a, hipStream_t s);
// int8 weights [N, K] row-major -> the tiled layout (N % 16 == 0, K % 64 == 0)
hipError_t launch_tile_weights(const int8_t *q, int64_t N, int64_t K, int8_t *qt, hipStream_t s);

// Raises a kernel's dynamic-LDS limit to `bytes` on the current device, once per device
// (the attribute is per device); `done` holds one bit per device id (< 64).
inline hipError_t ensure_dynamic_lds(const void *kern, int bytes, std::atomic<uint64_t> &done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  const uint64_t bit = (uint64_t)1 << dev;
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  done.fetch_or(bit, std::memory_order_acq_rel);
  return hipSuccess;
}

// element types of the attention tensors
enum AttnType { AT_BF16 = 0, AT_F16 = 1, AT_F32 = 2 };
// attention: q, k [H, L, Dh], vt [H, Dh, L] of type `in`, o [L, H*Dh] of type `out`.
// AT_F32 (in and out): fp64 arithmetic in a plain FMA kernel. AT_BF16 / AT_F16: 16-bit
// operands on the matrix cores (fp32 accumulation and softmax), o in bf16 or fp16.
// q_prescaled (16-bit only): q already carries scale * log2(e), the factor of the base-2
// softmax.
hipError_t launch_attention(const void *q, const void *k, const void *vt, void *o, int H,
                            int64_t L, int Dh, double scale, AttnType in, AttnType out,
                            bool q_prescaled, hipStream_t s);

}  // namespace h3k
