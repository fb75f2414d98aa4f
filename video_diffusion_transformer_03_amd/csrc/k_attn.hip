// Multi-head softmax attention over the video tokens (no mask), flash-style: key/value
// tiles stream through LDS and an online softmax keeps the running row maximum and row
// sum, so memory stays O(L * d) at any sequence length.
//
// Inputs come head-major from the QKV projection ("h3-metal: Apple Silicon을 위한
// 네이티브 MiniMax-H3 추론", section "Metal 4 및 TensorOps": Q/K/V routed straight into
// head-major attention inputs). Layouts: Q, K [H, L, Dh]; V transposed [H, Dh, L];
// O [L, H*Dh] (token-major, head e in columns e*Dh .. e*Dh + Dh - 1).
//
// 16-bit kernels: Q, K, V and P are fp16 (v_mfma_f32_16x16x32_f16) or bf16
// (v_mfma_f32_16x16x32_bf16); the two instructions have the same shape and rate. The
// block's default is fp16: 11 significant bits instead of 8 for the same bytes. Its
// scores are large (a standard deviation near 10 on the synthetic workloads), so the
// softmax is close to an argmax, and bf16 rounding of Q, K and V moves O by about 6e-3;
// the quantiser of O and those after it turn that into code flips. Both products run in
// transposed form so that a lane always owns one query column:
//   S^T = K Q^T   (A = K rows from LDS, B = Q held in registers)
//   O^T = V^T P^T (A = V^T rows from LDS, B = P^T taken straight from the S^T registers)
// The 8 key slots of the P^T operand are the lane's own S^T values, and V^T is read
// with the same key order, so no cross-lane data movement is needed between the two
// products; the softmax statistics live in the same lane as the output columns they
// scale. P is rounded to the operand type for the second product (below 2^15 with the
// lazy maximum below, inside the fp16 range); max, exp and sums are fp32.
#include "h3k_internal.h"

namespace h3k {

// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0] + [15:14], expcnt [6:4], lgkmcnt [11:8])
constexpr int waitcnt_vm_lgkm0(int vm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (0 << 8);
}
// Work-group barrier without a memory fence, so global -> LDS copies stay in flight across
// it (a fenced barrier waits for all of them); callers order memory with s_waitcnt first.
#define H3K_PP_SYNC()                                   \
  {                                                     \
    __builtin_amdgcn_sched_barrier(0);                  \
    asm volatile("s_barrier" ::: "memory");             \
    __builtin_amdgcn_sched_barrier(0);                  \
  }

__device__ __forceinline__ uint4 ld16(const uint16_t *p) { return *(const uint4 *)p; }


constexpr int kAttnOcc = 2;   // waves per SIMD the register budget is sized for
constexpr int kAttnKPad = 16;  // elements of padding per K-tile row in LDS
constexpr int kAttnVPad = 16;  // elements of padding per V^T-tile row in LDS

template <int DH>
struct AttnCfg {
  static constexpr int BQ = 128;                  // queries per work-group (4 waves x 32)
  static constexpr int BK = 64;                   // keys per tile
  static constexpr int KP = DH + kAttnKPad;   // K tile row pitch (elements)
  static constexpr int VP = BK + kAttnVPad;   // V^T tile row pitch (elements)
  static constexpr int K_ELEMS = BK * KP;
  static constexpr int V_ELEMS = DH * VP;
  static constexpr size_t LDS = (size_t)2 * (K_ELEMS + V_ELEMS) * 2;
  static constexpr int KCH = BK * DH / 8 / 256;  // 16-byte chunks per thread, K tile
  static constexpr int VCH = DH * BK / 8 / 256;  // 16-byte chunks per thread, V^T tile
};

// Lazy rescaling: the running maximum used for exp2 is only moved when a row's true
// maximum exceeds it by more than 15 (base-2 exponent) -- P stays <= 2^15, inside the fp16
// range (65504), and the O/l rescale (one multiply per accumulator) is skipped in most
// tiles. Softmax is invariant to the subtracted constant, so the result is unchanged; a
// larger bound only widens the range of P below the row maximum that fp16 keeps normal.
// At the block's score spread (a deviation near 10, natural-log units) the running maximum
// of a row still moves about once over 16384 keys, against 1.8 times with a bound of 8, and
// a wave rescales in a third fewer iterations.
constexpr float kRescaleLog2 = 15.0f;

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
template <bool F16, int DH, bool MASK>
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
      s[t4][0] = mma16<F16>(kf, qf[0][kk], s[t4][0]);
      s[t4][1] = mma16<F16>(kf, qf[1][kk], s[t4][1]);
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
    mx = rows_max(mx);
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
  // row sum l accumulates the same rounded P the matrix cores consume (one dot2 per packed
  // pair against (1, 1)), so O = sum(p v) / sum(p) is normalised consistently.
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    v8bf pb[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      uint4 u;
      u.x = pack16<F16>(s[2 * ks][qt][0], s[2 * ks][qt][1]);
      u.y = pack16<F16>(s[2 * ks][qt][2], s[2 * ks][qt][3]);
      u.z = pack16<F16>(s[2 * ks + 1][qt][0], s[2 * ks + 1][qt][1]);
      u.w = pack16<F16>(s[2 * ks + 1][qt][2], s[2 * ks + 1][qt][3]);
      float l = st.l[qt];
      l = add_pair16<F16>(u.x, l);
      l = add_pair16<F16>(u.y, l);
      l = add_pair16<F16>(u.z, l);
      l = add_pair16<F16>(u.w, l);
      st.l[qt] = l;
      pb[qt] = __builtin_bit_cast(v8bf, u);
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      v8bf vf = __builtin_bit_cast(v8bf, ld16(cV + (dt * 16 + c16) * VP + ks * 32 + g * 8));
      st.o[dt][0] = mma16<F16>(vf, pb[0], st.o[dt][0]);
      st.o[dt][1] = mma16<F16>(vf, pb[1], st.o[dt][1]);
    }
  }
}

// F16: fp16 operands (else bf16); OF16: O stored as fp16 (else bf16)
template <bool F16, bool OF16, int DH>
__global__ __launch_bounds__(256, kAttnOcc) void attn_h_kernel(
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
    attn_tile<F16, DH, false>(st, qf, sK + cur * C::K_ELEMS, sV + cur * C::V_ELEMS, lane,
                              (int64_t)kt * BK, L, sl2);
    H3K_ATTN_LSTORE(cur ^ 1);
    __syncthreads();
  }
  {
    const int cur = (nkt - 1) & 1;
    if (tail)
      attn_tile<F16, DH, true>(st, qf, sK + cur * C::K_ELEMS, sV + cur * C::V_ELEMS, lane,
                               (int64_t)(nkt - 1) * BK, L, sl2);
    else
      attn_tile<F16, DH, false>(st, qf, sK + cur * C::K_ELEMS, sV + cur * C::V_ELEMS, lane,
                                (int64_t)(nkt - 1) * BK, L, sl2);
  }
#undef H3K_ATTN_GLOAD
#undef H3K_ATTN_LSTORE

  const int64_t ldo = (int64_t)H * DH;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float l = st.l[qt];
    l = rows_sum(l);
    const float inv = 1.0f / l;
    const int64_t qi = q0 + qt * 16 + c16;
    if (qi < L) {
      const int64_t obase = qi * ldo + (int64_t)head * DH + g * 4;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        v4f v = st.o[dt][qt];
        *(uint2 *)((uint16_t *)Ov + obase + dt * 16) =
            make_uint2(pack16<OF16>(v[0] * inv, v[1] * inv), pack16<OF16>(v[2] * inv, v[3] * inv));
      }
    }
  }
}

// ---------------------------------------------------------------------------- bf16, Dh = 128
// Software-pipelined kernel: 8 waves x 32 queries per work-group. Iteration j overlaps,
// inside each wave, the matrix-core products of one tile with the softmax arithmetic of
// another (a wave's own VALU work issues between its MFMAs; work of a second wave on the
// same SIMD overlaps far less):
//   phase 1: S(j+1) = K(j+1) Q^T        with  P(j) = exp2(S(j) - m) of its first 32 keys
//   phase 2: O += V(j) P(j)^T           with  P(j) of its last 32 keys, row maximum of
//                                             S(j+1), rescale decision
// The row sums l come out of phase 2's matrix-core work (an extra accumulator block with
// an all-ones V^T operand). The O / l rescale a new maximum calls for is applied at the
// start of the next iteration, after phase 2 has added the tile scaled by the old maximum.
//
// K and V^T tiles reach LDS through direct global -> LDS copies into four resident
// stages; stage u holds K tile u and V^T tile u - 1 (what iteration u - 1 reads), and
// iteration j issues the copies of stage j + 4. LDS layouts (16-byte chunks, XOR swizzles
// keep fragment reads free of bank conflicts; every copy instruction fills 1 KB and reads
// whole 128-byte lines):
//   K   64 rows x 256 B: row R holds key kof(R) of the tile (the kperm order above), chunk
//       c at position c ^ (R % 16)
//   V^T 128 rows (head dims) x 128 B (64 keys): chunk c at position c ^ (R % 8)
namespace v2 {
constexpr int NW = 8, BQ = NW * 32, BK = 64, DH = 128;
constexpr int NB = 4, DIST = 4;            // resident stages; iteration j copies stage j + DIST
constexpr int K_BYTES = BK * DH * 2;       // 16 KB
constexpr int STAGE = 2 * K_BYTES;         // K then V^T
constexpr size_t LDS = (size_t)NB * STAGE;
constexpr int COPIES = 4;                  // copy instructions per wave and stage

__device__ __forceinline__ int kof(int R) {  // key (within the tile) held by K row R
  const int i = R & 15;
  return (R & ~31) + 8 * (i >> 2) + 4 * ((R >> 4) & 1) + (i & 3);
}

// S^T = K Q^T for one K tile: lane holds keys (t4/2)*32 + 8g + 4(t4%2) + r, query c16
template <bool F16>
__device__ __forceinline__ void s_tile(v4f (&s)[4][2], const v8bf (&qf)[2][4],
                                       const uint8_t *kb, int koff) {
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4) s[t4][0] = s[t4][1] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      const v8bf kf = *(const v8bf *)(kb + t4 * 4096 + (koff ^ (kk * 64)));
      s[t4][0] = mma16<F16>(kf, qf[0][kk], s[t4][0]);
      s[t4][1] = mma16<F16>(kf, qf[1][kk], s[t4][1]);
    }
  }
}

// P = exp2(S sl2 - m) rounded to the operand type (the P^T operand, keys 8g .. 8g+7 of
// each 32-key step). QPRE: S already holds the exponent (scaled scores minus m), P = exp2(S).
template <bool F16, bool QPRE>
__device__ __forceinline__ void exp_tile(const v4f (&s)[4][2], v8bf (&pb)[2][2],
                                         const float (&m)[2], float sl2) {
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float mneg = -m[qt];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float p[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (QPRE) {
          p[r] = __builtin_amdgcn_exp2f(s[2 * ks][qt][r]);
          p[4 + r] = __builtin_amdgcn_exp2f(s[2 * ks + 1][qt][r]);
        } else {
          p[r] = __builtin_amdgcn_exp2f(fmaf(s[2 * ks][qt][r], sl2, mneg));
          p[4 + r] = __builtin_amdgcn_exp2f(fmaf(s[2 * ks + 1][qt][r], sl2, mneg));
        }
      }
      uint4 u;
      u.x = pack16<F16>(p[0], p[1]);
      u.y = pack16<F16>(p[2], p[3]);
      u.z = pack16<F16>(p[4], p[5]);
      u.w = pack16<F16>(p[6], p[7]);
      pb[ks][qt] = __builtin_bit_cast(v8bf, u);
    }
  }
}

// Accumulator block NO = 8 of O^T holds the row sum: its V^T operand is all ones, so every
// row of the block is the sum over keys of the rounded P the other blocks consume
constexpr int NO = 9;

// O^T += V^T P^T for one V^T tile (and the row-sum block)
template <bool F16>
__device__ __forceinline__ void pv_tile(v4f (&o)[NO][2], const v8bf (&pb)[2][2],
                                        const uint8_t *vb, int voff) {
  const v8bf ones = ones16<F16>();
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    o[8][0] = mma16<F16>(ones, pb[ks][0], o[8][0]);
    o[8][1] = mma16<F16>(ones, pb[ks][1], o[8][1]);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const v8bf vf = *(const v8bf *)(vb + dt * 2048 + (voff ^ (ks * 64)));
      o[dt][0] = mma16<F16>(vf, pb[ks][0], o[dt][0]);
      o[dt][1] = mma16<F16>(vf, pb[ks][1], o[dt][1]);
    }
  }
}

// Row maxima of a score tile in the exp2 domain (with MASK, keys >= kmax of the tile are
// set to -inf first); grow = some row exceeds the running maximum m by more than
// kRescaleLog2.
// QPRE: the tile already holds exponents relative to m, and mnew is that relative maximum.
template <bool MASK, bool QPRE>
__device__ __forceinline__ bool max_vals(v4f (&s)[4][2], const float (&m)[2], float (&mnew)[2],
                                         float sl2, int g, int kmax) {
  if (MASK && kmax < BK) {
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = (t4 >> 1) * 32 + 8 * g + 4 * (t4 & 1) + r;
        if (key >= kmax) s[t4][0][r] = s[t4][1][r] = -INFINITY;
      }
  }
  bool grow = false;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float mx = fmaxf(fmaxf(s[0][qt][0], s[0][qt][1]), s[0][qt][2]);
    mx = fmaxf(fmaxf(mx, s[0][qt][3]), s[1][qt][0]);
    mx = fmaxf(fmaxf(mx, s[1][qt][1]), s[1][qt][2]);
    mx = fmaxf(fmaxf(mx, s[1][qt][3]), s[2][qt][0]);
    mx = fmaxf(fmaxf(mx, s[2][qt][1]), s[2][qt][2]);
    mx = fmaxf(fmaxf(mx, s[2][qt][3]), s[3][qt][0]);
    mx = fmaxf(fmaxf(mx, s[3][qt][1]), s[3][qt][2]);
    mx = fmaxf(mx, s[3][qt][3]);
    mx = rows_max(mx);
    if constexpr (QPRE) {
      mnew[qt] = mx;
      grow |= mx > kRescaleLog2;
    } else {
      mnew[qt] = mx * sl2;
      grow |= mnew[qt] > m[qt] + kRescaleLog2;
    }
  }
  return grow;
}

// Lazy rescale decision: the running maximum m moves only when a row's maximum exceeds it
// by more than kRescaleLog2 (P then stays <= 2^15). Returns whether any row of the wave moved
// (alpha then holds the factors for O and l; QPRE: shift holds how far m moved, to be
// taken off the pending score tile, which was formed relative to the old m).
// PART: mnew holds each lane's partial maximum over its own keys and grow that lane's
// test; a row's maximum exceeds the bound exactly when one of its lanes' partials does,
// so the cross-lane reduction runs only when some lane of the wave saw growth.
template <bool QPRE, bool PART = false>
__device__ __forceinline__ bool rescale_decision(bool grow, float (&mnew)[2],
                                                 float (&m)[2], float (&alpha)[2],
                                                 float (&shift)[2], float sl2 = 1.f) {
  if (!(__builtin_amdgcn_read_exec() & __ballot(grow))) return false;
  if constexpr (PART) {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      mnew[qt] = rows_max(mnew[qt]);
      if constexpr (!QPRE) mnew[qt] *= sl2;
    }
  }
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    if constexpr (QPRE) {
      shift[qt] = mnew[qt] > kRescaleLog2 ? mnew[qt] : 0.f;
      alpha[qt] = __builtin_amdgcn_exp2f(-shift[qt]);
      m[qt] += shift[qt];
    } else {
      const float mref = mnew[qt] > m[qt] + kRescaleLog2 ? mnew[qt] : m[qt];
      alpha[qt] = __builtin_amdgcn_exp2f(m[qt] - mref);
      m[qt] = mref;
    }
  }
  return true;
}

// QPRE: a score tile formed relative to an older m, brought to the current one
__device__ __forceinline__ void shift_tile(v4f (&s)[4][2], const float (&shift)[2]) {
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int r = 0; r < 4; ++r) s[t4][qt][r] -= shift[qt];
}

constexpr int PD = 3;  // LDS fragment reads issued this many MFMA pairs ahead

// One slice of the softmax of a score tile: the pair of scores PART of query tile QT in
// 32-key step KS -> two exp2 and one 16-bit pair packed into u[PART] (pb[KS][QT] once the
// four parts are done). The row sum comes from the matrix cores (accumulator block 8).
template <bool F16, bool QPRE, int QT, int KS, int PART>
__device__ __forceinline__ void softmax_slice(const v4f (&cur)[4][2], uint32_t (&u)[4],
                                              v8bf (&pb)[2][2], const float (&mneg)[2],
                                              float sl2) {
  constexpr int tt = 2 * KS + (PART >> 1), r0 = (PART & 1) * 2;
  const float p0 = QPRE ? __builtin_amdgcn_exp2f(cur[tt][QT][r0])
                        : __builtin_amdgcn_exp2f(fmaf(cur[tt][QT][r0], sl2, mneg[QT]));
  const float p1 = QPRE ? __builtin_amdgcn_exp2f(cur[tt][QT][r0 + 1])
                        : __builtin_amdgcn_exp2f(fmaf(cur[tt][QT][r0 + 1], sl2, mneg[QT]));
  u[PART] = pack16<F16>(p0, p1);
  if constexpr (PART == 3) pb[KS][QT] = __builtin_bit_cast(v8bf, make_uint4(u[0], u[1], u[2], u[3]));
}

// An iteration runs two phases of 16 hand-ordered steps (a scheduling barrier ends each
// step). The softmax of the current tile is split between them by 32-key step, so that each
// phase's VALU work fits beside its 32 MFMAs: with all of it in phase 1, that phase's VALU
// issue exceeded its matrix-core time while phase 2 carried only the row maximum.
//
// Phase 1: step i reads K fragment i + PD, issues the two MFMAs of fragment i (S^T tile t4 =
// i % 4, head-dim step kk = i / 4, both query tiles) into nxt; every odd step does one slice
// of the softmax of cur's first 32 keys (pb[0]). Steps 0, 4, 8 and 12 also issue the wave's
// four global -> LDS copies of a later stage (copy_piece(0..3)); issued together at the
// start of the iteration by all eight waves, the copies queued behind each other and stalled
// the waves' issue.
// QPRE: Q carries the base-2 softmax scale, each S tile starts from cq = -m (the MFMA's C
// operand), so it comes out as the exponents themselves and exp2 reads it directly.
template <bool F16, bool QPRE, typename CopyF>
__device__ __forceinline__ void phase_s_exp(v4f (&nxt)[4][2], const v4f (&cur)[4][2],
                                            v8bf (&pb)[2][2], const v8bf (&qf)[2][4],
                                            const uint8_t *kb, int koff, const float (&m)[2],
                                            const v4f (&cq)[2], float sl2, CopyF &&copy_piece) {
  v8bf kf[PD + 1];
  static_for<PD>([&](auto I) {
    kf[I] = *(const v8bf *)(kb + (I % 4) * 4096 + (koff ^ ((I / 4) * 64)));
  });
  const float mneg[2] = {-m[0], -m[1]};
  uint32_t u[4];
  static_for<16>([&](auto I) {
    constexpr int i = I;
    if constexpr (i % 4 == 0) copy_piece(i / 4);  // one copy instruction every fourth step
    if constexpr (i + PD < 16)
      kf[(i + PD) % (PD + 1)] =
          *(const v8bf *)(kb + ((i + PD) % 4) * 4096 + (koff ^ (((i + PD) / 4) * 64)));
    constexpr int t4 = i % 4, kk = i / 4;
    const v8bf k = kf[i % (PD + 1)];
    const v4f z = {0.f, 0.f, 0.f, 0.f};
    nxt[t4][0] = mma16<F16>(k, qf[0][kk],
                                                         kk ? nxt[t4][0] : (QPRE ? cq[0] : z));
    nxt[t4][1] = mma16<F16>(k, qf[1][kk],
                                                         kk ? nxt[t4][1] : (QPRE ? cq[1] : z));
    if constexpr (i % 2 == 1) {
      constexpr int sl = i / 2;
      softmax_slice<F16, QPRE, sl / 4, 0, sl % 4>(cur, u, pb, mneg, sl2);
    }
    __builtin_amdgcn_sched_barrier(0);
  });
}

// Phase 2, same shape: step i reads V^T fragment i + PD, issues the two MFMAs of fragment i
// (head-dim tile dt = i % 8, key step ks = i / 8) into o, and advances the lane's partial
// row maximum of nxt (query tile i / 8, two scores per step). Steps
// 0 .. 7 also do the softmax slices of cur's last 32 keys (pb[1]), which the MFMAs of steps
// 8 .. 15 consume.
template <bool F16, bool QPRE>
__device__ __forceinline__ bool phase_pv_max(v4f (&o)[NO][2], v8bf (&pb)[2][2],
                                             const v4f (&nxt)[4][2], const v4f (&cur)[4][2],
                                             const uint8_t *vb, int voff, const float (&m)[2],
                                             float (&mnew)[2], float sl2) {
  const v8bf ones = ones16<F16>();
  v8bf vf[PD + 1];
  static_for<PD>([&](auto I) {
    vf[I] = *(const v8bf *)(vb + (I % 8) * 2048 + (voff ^ ((I / 8) * 64)));
  });
  const float mneg[2] = {-m[0], -m[1]};
  uint32_t u[4];
  float mx = 0.f;
  bool grow = false;
  static_for<16>([&](auto I) {
    constexpr int i = I;
    if constexpr (i + PD < 16)
      vf[(i + PD) % (PD + 1)] =
          *(const v8bf *)(vb + ((i + PD) % 8) * 2048 + (voff ^ (((i + PD) / 8) * 64)));
    constexpr int dt = i % 8, ks = i / 8;
    const v8bf v = vf[i % (PD + 1)];
    o[dt][0] = mma16<F16>(v, pb[ks][0], o[dt][0]);
    o[dt][1] = mma16<F16>(v, pb[ks][1], o[dt][1]);
    if constexpr (i < 8) softmax_slice<F16, QPRE, i / 4, 1, i % 4>(cur, u, pb, mneg, sl2);
    if constexpr (dt == 7) {  // row sums of this key step's P
      o[8][0] = mma16<F16>(ones, pb[ks][0], o[8][0]);
      o[8][1] = mma16<F16>(ones, pb[ks][1], o[8][1]);
    }
    constexpr int qt = i / 8, st = i % 8;  // scores 2 st, 2 st + 1 of query tile qt
    const float a0 = nxt[st >> 1][qt][(st & 1) * 2], a1 = nxt[st >> 1][qt][(st & 1) * 2 + 1];
    if constexpr (st == 0)
      mx = fmaxf(a0, a1);
    else
      mx = fmaxf(fmaxf(mx, a0), a1);
    if constexpr (st == 7) {  // the lane's partial maximum and its own test (see rescale_decision)
      mnew[qt] = mx;
      if constexpr (QPRE)
        grow |= mx > kRescaleLog2;
      else
        grow |= mx * sl2 > m[qt] + kRescaleLog2;
    }
    __builtin_amdgcn_sched_barrier(0);
  });
  return grow;
}

// keys >= kmax of a score tile -> -inf (last key tile)
__device__ __forceinline__ void mask_tile(v4f (&s)[4][2], int g, int kmax) {
  if (kmax < BK) {
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = (t4 >> 1) * 32 + 8 * g + 4 * (t4 & 1) + r;
        if (key >= kmax) s[t4][0][r] = s[t4][1][r] = -INFINITY;
      }
  }
}

__device__ __forceinline__ void rescale(v4f (&o)[NO][2], const float (&alpha)[2]) {
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int dt = 0; dt < NO; ++dt) o[dt][qt] *= alpha[qt];
}
}  // namespace v2

// F16: fp16 operands (else bf16); OF16: O stored as fp16 (else bf16); QPRE: Q arrives
// multiplied by log2(e) / sqrt(Dh) (sl2 is then unused)
template <bool F16, bool OF16, bool QPRE>
__global__ __launch_bounds__(512) void attn_v2_kernel(const uint16_t *__restrict__ Q,
                                                      const uint16_t *__restrict__ K,
                                                      const uint16_t *__restrict__ Vt,
                                                      void *__restrict__ Ov, int H, int64_t L,
                                                      float sl2) {
  using namespace v2;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // wave index made visibly uniform: the copies' LDS destinations are then scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  // work-group b runs on XCD b % 8; each XCD takes a contiguous range of (query block,
  // head) pairs, query block fastest, so its concurrent work-groups share one head's K/V in L2
  const int64_t nqb = (L + BQ - 1) / BQ, total = nqb * H;
  int64_t t = blockIdx.x;
  if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
  const int head = (int)(t / nqb);
  const int64_t q0 = (t - (int64_t)head * nqb) * BQ + wave * 32;
  const uint16_t *Qh = Q + (int64_t)head * L * DH;
  const uint16_t *Kh = K + (int64_t)head * L * DH;
  const uint16_t *Vh = Vt + (int64_t)head * DH * L;
  const uint32_t Lu = (uint32_t)L;
  const int nkt = (int)((L + BK - 1) / BK);

  // Q^T operand: query q0 + qt*16 + c16 (rows past L read row L-1, never stored)
  v8bf qf[2][4];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int64_t qi = (q0 + qt * 16 + c16) < L ? (q0 + qt * 16 + c16) : (L - 1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qf[qt][kk] = __builtin_bit_cast(v8bf, ld16(Qh + qi * DH + kk * 32 + g * 8));
  }

  // copy lanes: K instructions wave and wave + 8 (rows 4i .. 4i+3), V^T instructions wave
  // and wave + 8 (rows 8i .. 8i+7). Keys past L (the partial last tile) read the next
  // head's K rows, the next V^T row's first columns (L % 8 == 0: a 16-byte chunk never
  // straddles rows) or, past the end of the tensor, zeros (below); their scores are
  // masked, so p = 0 meets finite values.
  int kkey[2], kcol[2], vrow[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int Rk = 4 * (wave + 8 * q) + (lane >> 4);
    kkey[q] = kof(Rk);
    kcol[q] = ((lane & 15) ^ (Rk & 15)) * 8;
    vrow[q] = 8 * (wave + 8 * q) + (lane >> 3);
  }
  const int vcol = ((lane & 7) ^ ((lane >> 3) & 7)) * 8;
// Buffer (MUBUF) copies rather than global_load_lds: for the latter the compiler assumes a
// pending copy may also count against lgkmcnt and waits for every outstanding LDS read at
// each fragment use, which would undo the read-ahead of the phases below. Each resource
// ends where its tensor ends, or 2^32 - 1 bytes on, whichever is nearer: the hardware
// returns zeros for bytes past it, so the partial last tile's copies need no clamping and
// none reads past the allocation. The entry points take L < 2^24, so a key or V^T column
// below L lies below byte 256 L <= 2^32 - 2048 of its head (inside either bound), and the
// last tile's copies, which reach at most byte 2^32 - 1, do not wrap the 32-bit offset.
  const uint64_t kv_end = (uint64_t)(H - head) * (uint64_t)L * (DH * 2);
  const int kv_rec = (int)(uint32_t)(kv_end < 0xffffffffull ? kv_end : 0xffffffffull);
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void *)Kh, (short)0, kv_rec, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void *)Vh, (short)0, kv_rec, 0x00020000);
  // Per-lane byte offsets of tile 0's copies; tile u adds its start as the instructions'
  // scalar offset, so the copies cost no vector instructions and take no branch.
  uint32_t kvo[2], vvo[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    kvo[q] = ((uint32_t)kkey[q] * DH + (uint32_t)kcol[q]) * 2;
    vvo[q] = ((uint32_t)vrow[q] * Lu + (uint32_t)vcol) * 2;
  }
  // piece 0, 1: K rows of copy instruction wave + 8 piece; piece 2, 3: V^T rows likewise.
  // Stage u holds K tile u and V^T tile u - 1 (stage 0: tile 0); stages past the last tile
  // repeat it into buffers no later stage's reads use.
  auto copy_piece = [&](int u, int piece) {
    uint8_t *dst = smem + (u % NB) * STAGE;
    if (piece < 2) {
      const uint32_t kt = (uint32_t)(u < nkt ? u : nkt - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs,
          (__attribute__((address_space(3))) void *)(dst + (wave + 8 * piece) * 1024), 16,
          kvo[piece], kt * (BK * DH * 2), 0, 0);
    } else {
      const uint32_t vt = (uint32_t)(u < 1 ? 0 : (u - 1 < nkt ? u - 1 : nkt - 1));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs,
          (__attribute__((address_space(3))) void *)(dst + K_BYTES + (wave + 8 * (piece - 2)) * 1024),
          16, vvo[piece - 2], vt * (BK * 2), 0, 0);
    }
  };
#define H3K_V2_COPY(u_)                                                                        \
  {                                                                                            \
    _Pragma("unroll") for (int pc = 0; pc < 4; ++pc) copy_piece((u_), pc);                     \
  }
  // fragment offsets inside a stage: K row t4*16 + c16, chunk 4kk + g; V^T row dt*16 + c16,
  // chunk 4ks + g (the kk / ks part is applied as an XOR of kk*64 / ks*64)
  const int koff = c16 * 256 + ((g ^ c16) * 16);
  const int voff = K_BYTES + c16 * 128 + ((g ^ (c16 & 7)) * 16);

  v4f o[NO][2];  // O^T blocks 0..7, row sums in block 8
#pragma unroll
  for (int i = 0; i < NO; ++i) o[i][0] = o[i][1] = v4f{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY}, alpha[2] = {1.f, 1.f};
  float shift[2] = {0.f, 0.f};
  v4f cq[2];  // QPRE: the C operand {-m, -m, -m, -m} each new S tile starts from
  v4f sa[4][2], sb[4][2];
  v8bf pb[2][2];

  // prologue: stages 0 .. DIST-1 in flight (past nkt they repeat valid tiles into buffers
  // no later copy targets); S(0) from stage 0, its maximum; then stage 1 for iteration 0
  static_for<DIST>([&](auto J) { H3K_V2_COPY(J); });
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(COPIES * (DIST - 1)));
  H3K_PP_SYNC();
  s_tile<F16>(sa, qf, smem, koff);
  float mnew[2];
  bool pend = max_vals<true, QPRE>(sa, m, mnew, sl2, g, (int)min((int64_t)BK, L));
  if constexpr (QPRE) {
    // the first tile sets m to its row maxima (every row has a valid key) and is shifted by
    // them; O and l are still zero, so nothing is pending
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      m[qt] = shift[qt] = mnew[qt];
      cq[qt] = v4f{-m[qt], -m[qt], -m[qt], -m[qt]};
    }
    shift_tile(sa, shift);
    pend = false;
  } else {
    pend = rescale_decision<false>(pend, mnew, m, alpha, shift);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(COPIES * (DIST - 2)));
  H3K_PP_SYNC();

  // iteration j reads stage j + 1. Its copies of stage j + DIST go to the buffer of stage
  // j + DIST - NB <= j, last read in iteration j - 1 (or the prologue); the wave's copy of
  // stage j + 2 is complete at the barrier ending iteration j (DIST - 2 younger stages may
  // still be in flight). Every iteration copies, also past the last stage read (nkt), so
  // the count holds throughout.
#define H3K_V2_ITER(CUR, NXT, j_, MASK)                                                        \
  {                                                                                            \
    const int jj = (j_);                                                                       \
    const uint8_t *sb_ = smem + ((jj + 1) % NB) * STAGE;                                       \
    if (pend) {                                                                                \
      rescale(o, alpha);                                                                       \
      if constexpr (QPRE) {                                                                    \
        shift_tile(CUR, shift);                                                                \
        _Pragma("unroll") for (int qt = 0; qt < 2; ++qt)                                       \
          cq[qt] = v4f{-m[qt], -m[qt], -m[qt], -m[qt]};                                        \
      }                                                                                        \
    }                                                                                          \
    phase_s_exp<F16, QPRE>(NXT, CUR, pb, qf, sb_, koff, m, cq, sl2,                            \
                           [&](int pc) { copy_piece(jj + DIST, pc); });                        \
    if (MASK) mask_tile(NXT, g, (int)min((int64_t)BK, L - (int64_t)(jj + 1) * BK));            \
    const bool grow_ = phase_pv_max<F16, QPRE>(o, pb, NXT, CUR, sb_, voff, m, mnew, sl2);           \
    pend = rescale_decision<QPRE, true>(grow_, mnew, m, alpha, shift, sl2);                    \
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(COPIES * (DIST - 2)));                         \
    H3K_PP_SYNC();                                                                             \
  }
#define H3K_V2_LAST(CUR)                                                                       \
  {                                                                                            \
    const uint8_t *sb_ = smem + (nkt % NB) * STAGE;                                            \
    if (pend) {                                                                                \
      rescale(o, alpha);                                                                       \
      if constexpr (QPRE) shift_tile(CUR, shift);                                              \
    }                                                                                          \
    exp_tile<F16, QPRE>(CUR, pb, m, sl2);                                                      \
    pv_tile<F16>(o, pb, sb_, voff);                                                                 \
  }
  // nkt - 1 iterations in pairs (the score tiles swap roles); only the last iteration, whose
  // S tile is the last key tile, can need the key mask. An odd count runs one iteration
  // first (masked variant; the mask is a no-op unless it is also the last) and moves its S
  // tile back into sa, so every path ends with the current tile in sa.
  const int nit = nkt - 1;
  int j = 0;
  if (nit & 1) {
    H3K_V2_ITER(sa, sb, 0, true);
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) sa[t4][0] = sb[t4][0], sa[t4][1] = sb[t4][1];
    j = 1;
  }
  for (; j + 2 < nit; j += 2) {
    H3K_V2_ITER(sa, sb, j, false);
    H3K_V2_ITER(sb, sa, j + 1, false);
  }
  if (j < nit) {
    H3K_V2_ITER(sa, sb, j, false);
    H3K_V2_ITER(sb, sa, j + 1, true);
  }
  H3K_V2_LAST(sa);
  // the copies of the stages past nkt land before the work-group ends
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
#undef H3K_V2_ITER
#undef H3K_V2_LAST
#undef H3K_V2_COPY

  const int64_t ldo = (int64_t)H * DH;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float inv = 1.0f / o[8][qt][0];  // every lane's block-8 values are its query's row sum
    const int64_t qi = q0 + qt * 16 + c16;
    if (qi < L) {
      const int64_t obase = qi * ldo + (int64_t)head * DH + g * 4;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const v4f v = o[dt][qt];
        *(uint2 *)((uint16_t *)Ov + obase + dt * 16) =
            make_uint2(pack16<OF16>(v[0] * inv, v[1] * inv), pack16<OF16>(v[2] * inv, v[3] * inv));
      }
    }
  }
}

// ---------------------------------------------------------------------------- fp32
// Debug path: fp32 tensors, fp64 arithmetic (scores, softmax, P V), O rounded once to fp32.
// Plain FMA code: 64 queries per work-group, four threads per query, each owning DH/4 head
// dims; 32-key tiles of K and V^T in LDS, kept as fp32 (exact values of the inputs).
template <int DH>
__global__ __launch_bounds__(256) void attn_f32_kernel(const float *__restrict__ Q,
                                                       const float *__restrict__ K,
                                                       const float *__restrict__ Vt,
                                                       float *__restrict__ O, int H, int64_t L,
                                                       double sl2) {
  constexpr int TK = 32, DP = DH / 4;
  __shared__ float sK[TK][DH + 1];
  __shared__ float sV[DH][TK + 1];
  const int tid = threadIdx.x, head = blockIdx.y;
  const int part = tid & 3;
  const int64_t qi = (int64_t)blockIdx.x * 64 + (tid >> 2);
  const float *Qh = Q + (int64_t)head * L * DH;
  const float *Kh = K + (int64_t)head * L * DH;
  const float *Vh = Vt + (int64_t)head * DH * L;
  float q[DP];
  double o[DP];
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    q[e] = qi < L ? Qh[qi * DH + part * DP + e] : 0.f;
    o[e] = 0.0;
  }
  double mrow = -INFINITY, lsum = 0.0;
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
    double s[TK];
    double mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      double a = 0.0;
#pragma unroll
      for (int e = 0; e < DP; ++e) a = fma((double)q[e], (double)sK[j][part * DP + e], a);
      a += __shfl_xor(a, 1, 64);
      a += __shfl_xor(a, 2, 64);
      s[j] = (k0 + j < L) ? a * sl2 : -INFINITY;
      mx = fmax(mx, s[j]);
    }
    const double mnew = fmax(mrow, mx);
    const double alpha = exp2(mrow - mnew);
    mrow = mnew;
    lsum *= alpha;
#pragma unroll
    for (int e = 0; e < DP; ++e) o[e] *= alpha;
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      const double p = exp2(s[j] - mnew);
      lsum += p;
#pragma unroll
      for (int e = 0; e < DP; ++e) o[e] = fma(p, (double)sV[part * DP + e][j], o[e]);
    }
  }
  if (qi < L) {
    float *orow = O + qi * (int64_t)H * DH + (int64_t)head * DH + part * DP;
#pragma unroll
    for (int e = 0; e < DP; ++e) orow[e] = (float)(o[e] / lsum);
  }
}

template <bool F16, bool OF16, bool QPRE>
static hipError_t attn_v2(const void *q, const void *k, const void *vt, void *o, int H,
                          int64_t L, float sl2, hipStream_t s) {
  auto kern = attn_v2_kernel<F16, OF16, QPRE>;
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = ensure_dynamic_lds((const void *)kern, (int)v2::LDS, lds_set);
      e != hipSuccess)
    return e;
  const int64_t nwg = ((L + v2::BQ - 1) / v2::BQ) * H;
  if (nwg > 0x7fffffff) return hipErrorInvalidValue;  // one-dimensional grid
  dim3 grid((unsigned)nwg);
  kern<<<grid, 512, v2::LDS, s>>>((const uint16_t *)q, (const uint16_t *)k,
                                  (const uint16_t *)vt, o, H, L, sl2);
  return hipGetLastError();
}

template <bool F16, bool OF16, int DH>
static hipError_t attn_h(const void *q, const void *k, const void *vt, void *o, int H,
                         int64_t L, float sl2, hipStream_t s) {
  using C = AttnCfg<DH>;
  auto kern = attn_h_kernel<F16, OF16, DH>;
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = ensure_dynamic_lds((const void *)kern, (int)C::LDS, lds_set);
      e != hipSuccess)
    return e;
  dim3 grid((unsigned)((L + C::BQ - 1) / C::BQ), (unsigned)H);
  kern<<<grid, 256, C::LDS, s>>>((const uint16_t *)q, (const uint16_t *)k,
                                 (const uint16_t *)vt, o, H, L, sl2);
  return hipGetLastError();
}

template <int DH>
static hipError_t attn_f32(const void *q, const void *k, const void *vt, void *o, int H,
                           int64_t L, double sl2, hipStream_t s) {
  dim3 grid((unsigned)((L + 63) / 64), (unsigned)H);
  attn_f32_kernel<DH><<<grid, 256, 0, s>>>((const float *)q, (const float *)k,
                                           (const float *)vt, (float *)o, H, L, sl2);
  return hipGetLastError();
}

hipError_t launch_attention(const void *q, const void *k, const void *vt, void *o, int H,
                            int64_t L, int Dh, double scale, AttnType in, AttnType out,
                            bool q_prescaled, hipStream_t s) {
  const double sl2d = scale * 1.44269504088896340736;  // exp(x) = exp2(x * log2(e))
  const float sl2 = (float)sl2d;
  if (Dh != 64 && Dh != 128) return hipErrorInvalidValue;
  if (in == AT_F32 || out == AT_F32) {
    if (in != out || q_prescaled) return hipErrorInvalidValue;
    return Dh == 128 ? attn_f32<128>(q, k, vt, o, H, L, sl2d, s)
                     : attn_f32<64>(q, k, vt, o, H, L, sl2d, s);
  }
  // operand / output type pairs: fp16 -> fp16, fp16 -> bf16 (O feeding a bf16 projection),
  // bf16 -> bf16
  const bool f16 = in == AT_F16, of16 = out == AT_F16;
  if (!f16 && of16) return hipErrorInvalidValue;
  if (Dh == 64) {
    const float sl = q_prescaled ? 1.0f : sl2;
    if (f16) return of16 ? attn_h<true, true, 64>(q, k, vt, o, H, L, sl, s)
                         : attn_h<true, false, 64>(q, k, vt, o, H, L, sl, s);
    return attn_h<false, false, 64>(q, k, vt, o, H, L, sl, s);
  }
  if (q_prescaled) {
    if (f16) return of16 ? attn_v2<true, true, true>(q, k, vt, o, H, L, sl2, s)
                         : attn_v2<true, false, true>(q, k, vt, o, H, L, sl2, s);
    return attn_v2<false, false, true>(q, k, vt, o, H, L, sl2, s);
  }
  if (f16 != of16) return hipErrorInvalidValue;
  return f16 ? attn_v2<true, true, false>(q, k, vt, o, H, L, sl2, s)
             : attn_v2<false, false, false>(q, k, vt, o, H, L, sl2, s);
}

}  // namespace h3k
