// Host side of libh3k.so: argument validation, workspace planning, the block and stack
// sequences, and per-kernel event profiling. Every entry point validates all arguments
// before the first launch and reports failures through h3k_last_error().
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/h3k.h"
#include "h3k_internal.h"

using namespace h3k;

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

#define H3K_CHECK_PTR(p)                                                  \
  do {                                                                    \
    if (!(p)) return fail(H3K_EINVAL, "%s: %s is NULL", fn, #p);          \
    if (!aligned16(p)) return fail(H3K_EINVAL, "%s: %s is not 16-byte aligned", fn, #p); \
  } while (0)

// ------------------------------------------------------------------ profiling
struct ProfRec {
  int kind;
  hipEvent_t a, b;
};
bool g_prof_on = false;
std::vector<ProfRec> g_prof;     // records of the current profiling window
std::vector<hipEvent_t> g_pool;  // spare events

hipEvent_t pool_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

struct Launch {
  // brackets one kernel launch with profiling events and optional sync
  int kind;
  hipStream_t s;
  uint32_t flags;
  hipEvent_t a = nullptr, b = nullptr;
  Launch(int k, hipStream_t st, uint32_t f) : kind(k), s(st), flags(f) {
    if (g_prof_on) {
      a = pool_event();
      b = pool_event();
      if (a && b) hipEventRecord(a, s);
    }
  }
  int done(hipError_t e, const char *fn, const char *what) {
    if (e != hipSuccess) return fail(H3K_EHIP, "%s: %s launch failed: %s", fn, what, hipGetErrorString(e));
    if (a && b) {
      hipEventRecord(b, s);
      g_prof.push_back({kind, a, b});
    }
    if (flags & H3K_F_SYNC) {
      hipError_t e2 = hipStreamSynchronize(s);
      if (e2 == hipSuccess) e2 = hipGetLastError();
      if (e2 != hipSuccess) return fail(H3K_EHIP, "%s: %s failed: %s", fn, what, hipGetErrorString(e2));
    }
    return H3K_OK;
  }
};

// ------------------------------------------------------------------ dims / workspace
int check_dims(const char *fn, const h3k_dims *dm, int64_t L) {
  if (!dm) return fail(H3K_EINVAL, "%s: dims is NULL", fn);
  if (dm->d <= 0 || dm->n_heads <= 0 || dm->head_dim <= 0 || dm->d_ff <= 0 || dm->d_cond <= 0)
    return fail(H3K_EINVAL, "%s: dims must be positive", fn);
  if (dm->d != dm->n_heads * dm->head_dim)
    return fail(H3K_EINVAL, "%s: d (%d) != n_heads (%d) * head_dim (%d)", fn, dm->d, dm->n_heads, dm->head_dim);
  if (dm->grid_t <= 0 || dm->grid_h <= 0 || dm->grid_w <= 0)
    return fail(H3K_EINVAL, "%s: grid sizes must be positive", fn);
  if (L <= 0) return fail(H3K_EINVAL, "%s: L must be positive", fn);
  if ((int64_t)dm->grid_t * dm->grid_h * dm->grid_w != L)
    return fail(H3K_EINVAL, "%s: L (%lld) != grid_t*grid_h*grid_w", fn, (long long)L);
  if (!(dm->ln_eps > 0.f) || !(dm->rope_theta > 0.f))
    return fail(H3K_EINVAL, "%s: ln_eps and rope_theta must be positive", fn);
  if (dm->head_dim != 64 && dm->head_dim != 128)
    return fail(H3K_EUNSUPPORTED, "%s: head_dim %d unsupported (64 or 128)", fn, dm->head_dim);
  if (dm->d % 256 || dm->d_ff % 256)
    return fail(H3K_EUNSUPPORTED, "%s: d and d_ff must be multiples of 256", fn);
  if (dm->d > 8192) return fail(H3K_EUNSUPPORTED, "%s: d > 8192 unsupported", fn);
  if (dm->d_ff > 32768) return fail(H3K_EUNSUPPORTED, "%s: d_ff > 32768 unsupported", fn);
  if (dm->d_cond % 8 || dm->d_cond > 8192)
    return fail(H3K_EUNSUPPORTED, "%s: d_cond must be a multiple of 8 and <= 8192", fn);
  if (L % 8) return fail(H3K_EUNSUPPORTED, "%s: L must be a multiple of 8", fn);
  if (L >= (int64_t)1 << 24) return fail(H3K_EUNSUPPORTED, "%s: L >= 2^24 unsupported", fn);
  return H3K_OK;
}

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// which projections run as bf16 GEMMs
struct Prec {
  bool qkv, out, mlp;
  explicit Prec(uint32_t f)
      : qkv(f & (H3K_F_BF16_GEMM | H3K_F_BF16_QKV)),
        out(f & (H3K_F_BF16_GEMM | H3K_F_BF16_OUT)),
        mlp(f & (H3K_F_BF16_GEMM | H3K_F_BF16_MLP)) {}
  bool any() const { return qkv || out || mlp; }
};

void plan(const h3k_dims *dm, int64_t L, uint32_t flags, h3k_ws_layout *w) {
  const size_t d = dm->d, F = dm->d_ff, H = dm->n_heads, Dh = dm->head_dim;
  const size_t T = (flags & H3K_F_FP32_DEBUG) ? 4 : 2;
  const Prec p(flags);
  const size_t Lz = (size_t)L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += up256(bytes);
    return o;
  };
  w->m = take(6 * d * 4);
  // (cos, sin) per entry, fp32 or (the debug path's fp64 QKV epilogue) fp64
  w->rope = take((size_t)(dm->grid_t + dm->grid_h + dm->grid_w) * (Dh / 2) *
                 ((flags & H3K_F_FP32_DEBUG) ? 16 : 8));
  w->s_a = take(Lz * 4);
  w->s_o = take(Lz * 4);
  w->s_a2 = take(Lz * 4);
  w->s_g = take(Lz * 4);
  w->qa = p.qkv ? 0 : take(Lz * d);
  w->qo = p.out ? 0 : take(Lz * d);
  w->qa2 = p.mlp ? 0 : take(Lz * d);
  w->qg = p.mlp ? 0 : take(Lz * F);
  w->q = take(H * Lz * Dh * T);
  w->k = take(H * Lz * Dh * T);
  w->vt = take(H * Lz * Dh * T);
  // O (the attention's output type: fp16 or bf16), x1 and g (bf16): two bytes each, four on
  // the debug path
  w->o = take(Lz * d * T);
  w->x1 = take(Lz * d * T);
  w->g = take(Lz * F * T);
  w->h = p.qkv ? take(Lz * d * 2) : 0;
  w->h2 = p.mlp ? take(Lz * d * 2) : 0;
  w->total = off;
}

template <typename P>
P *at(void *ws, size_t off) {
  return (P *)((uint8_t *)ws + off);
}

int check_weights(const char *fn, const h3k_block_weights *w, uint32_t flags) {
  if (!w) return fail(H3K_EINVAL, "%s: weights is NULL", fn);
  H3K_CHECK_PTR(w->w_ada);
  const Prec p(flags);
  if (p.qkv) {
    if (!w->wb_qkv && !w->wbt_qkv) return fail(H3K_EINVAL, "%s: wb_qkv and wbt_qkv are both NULL", fn);
  } else {
    if (!w->w_qkv && !w->wt_qkv) return fail(H3K_EINVAL, "%s: w_qkv and wt_qkv are both NULL", fn);
    H3K_CHECK_PTR(w->s_qkv);
  }
  if (p.out) {
    if (!w->wb_o && !w->wbt_o) return fail(H3K_EINVAL, "%s: wb_o and wbt_o are both NULL", fn);
  } else {
    if (!w->w_o && !w->wt_o) return fail(H3K_EINVAL, "%s: w_o and wt_o are both NULL", fn);
    H3K_CHECK_PTR(w->s_o);
  }
  if (p.mlp) {
    if (!w->wb_up && !w->wbt_up) return fail(H3K_EINVAL, "%s: wb_up and wbt_up are both NULL", fn);
    if (!w->wb_down && !w->wbt_down) return fail(H3K_EINVAL, "%s: wb_down and wbt_down are both NULL", fn);
  } else {
    if (!w->w_up && !w->wt_up) return fail(H3K_EINVAL, "%s: w_up and wt_up are both NULL", fn);
    H3K_CHECK_PTR(w->s_up);
    if (!w->w_down && !w->wt_down) return fail(H3K_EINVAL, "%s: w_down and wt_down are both NULL", fn);
    H3K_CHECK_PTR(w->s_down);
  }
  return H3K_OK;
}

int check_flags(const char *fn, uint32_t flags) {
  if (flags & ~(uint32_t)(H3K_F_BF16_GEMM | H3K_F_FP32_DEBUG | H3K_F_SYNC | H3K_F_BF16_QKV |
                          H3K_F_BF16_OUT | H3K_F_BF16_MLP | H3K_F_ATTN_BF16))
    return fail(H3K_EINVAL, "%s: unknown flag bits 0x%x", fn, flags);
  if (Prec(flags).any() && (flags & H3K_F_FP32_DEBUG))
    return fail(H3K_EUNSUPPORTED, "%s: bf16 projections with H3K_F_FP32_DEBUG are unsupported", fn);
  if ((flags & H3K_F_ATTN_BF16) && (flags & H3K_F_FP32_DEBUG))
    return fail(H3K_EUNSUPPORTED, "%s: H3K_F_ATTN_BF16 with H3K_F_FP32_DEBUG is unsupported", fn);
  return H3K_OK;
}

// Element types of the attention tensors in a block: fp32 on the debug path; otherwise
// Q, K, V^T (and P) fp16, or bf16 under H3K_F_ATTN_BF16, and O fp16 when the int8
// out-projection's quantiser reads it, bf16 when a bf16 projection consumes it or the
// attention runs on bf16.
struct AttnTypes {
  AttnType in, out;
  explicit AttnTypes(uint32_t f) {
    if (f & H3K_F_FP32_DEBUG) {
      in = out = AT_F32;
    } else if (f & H3K_F_ATTN_BF16) {
      in = out = AT_BF16;
    } else {
      in = AT_F16;
      out = Prec(f).out ? AT_BF16 : AT_F16;
    }
  }
  int o_row_type() const { return out == AT_F32 ? ROW_F32 : (out == AT_F16 ? ROW_F16 : ROW_BF16); }
};

// One block on grid (T, Hg, Wg) with w positions w * w_scale + w_offset. Arguments are
// already validated.
int block_impl(const char *fn, const void *x_in, void *x_out, const float *cond,
               const h3k_block_weights *w, const h3k_dims *dm, int T, int Hg, int Wg,
               float w_scale, float w_offset, uint32_t flags, void *ws, hipStream_t s) {
  const int64_t L = (int64_t)T * Hg * Wg;
  const int d = dm->d, F = dm->d_ff, H = dm->n_heads, Dh = dm->head_dim;
  const bool f32 = (flags & H3K_F_FP32_DEBUG) != 0;
  const int act = f32 ? ROW_F32 : ROW_BF16;  // x, x1 (and g) element type
  const Prec p(flags);
  const AttnTypes at_(flags);
  h3k_ws_layout lay;
  plan(dm, L, flags, &lay);
  float *m = at<float>(ws, lay.m);
  void *rope = at<void>(ws, lay.rope);
  int rc;

  {
    Launch l(H3K_K_ADALN, s, flags);
    if ((rc = l.done(launch_adaln(w->w_ada, cond, m, 6 * (int64_t)d, dm->d_cond, f32, s), fn, "adaln"))) return rc;
  }
  RopeGeom rg = rope_geom(Dh, T, Hg, Wg, w_scale, w_offset);
  {
    Launch l(H3K_K_ROPE_TABLE, s, flags);
    if ((rc = l.done(launch_rope_table(rope, rg, dm->rope_theta, f32, s), fn, "rope_table"))) return rc;
  }
  const float *shift1 = m, *scale1 = m + d, *gate1 = m + 2 * d;
  const float *shift2 = m + 3 * d, *scale2 = m + 4 * d, *gate2 = m + 5 * d;

  // LN + modulate (+ quant)
  {
    Launch l(H3K_K_LN_QUANT, s, flags);
    hipError_t e = p.qkv ? launch_rows(1, x_in, ROW_BF16, shift1, scale1, L, d, dm->ln_eps, nullptr,
                                       nullptr, at<uint16_t>(ws, lay.h), s)
                      : launch_rows(0, x_in, act, shift1, scale1, L, d, dm->ln_eps,
                                    at<int8_t>(ws, lay.qa), at<float>(ws, lay.s_a), nullptr, s);
    if ((rc = l.done(e, fn, "ln_modulate_quant"))) return rc;
  }
  // QKV + RoPE + head-major scatter
  GemmArgs ga{};
  ga.M = L;
  ga.out_f32 = f32;
  {
    GemmArgs a = ga;
    a.bf16_ops = p.qkv;
    a.A = p.qkv ? (const void *)at<uint16_t>(ws, lay.h) : (const void *)at<int8_t>(ws, lay.qa);
    a.B = p.qkv ? (const void *)w->wb_qkv : (const void *)w->w_qkv;
    a.Bt = p.qkv ? (const int8_t *)w->wbt_qkv : w->wt_qkv;
    a.N = 3 * d;
    a.K = d;
    a.sa = at<float>(ws, lay.s_a);
    a.sw = w->s_qkv;
    a.q = at<void>(ws, lay.q);
    a.k = at<void>(ws, lay.k);
    a.vt = at<void>(ws, lay.vt);
    a.d = d;
    a.H = H;
    a.Dh = Dh;
    a.rope = rope;
    a.rg = rg;
    // 16-bit path: Q leaves the epilogue multiplied by log2(e) / sqrt(Dh), so that attention
    // exponentiates its scores without a scaling step (one rounding of Q either way); Q, K
    // and V^T are stored in the attention's operand type
    if (!f32) a.q_scale = (1.0f / sqrtf((float)Dh)) * 1.4426950408889634f;
    a.qkv_f16 = at_.in == AT_F16;
    Launch l(H3K_K_GEMM_QKV, s, flags);
    if ((rc = l.done(launch_gemm(EPI_QKV, a, s), fn, "gemm_qkv"))) return rc;
  }
  // attention
  {
    Launch l(H3K_K_ATTENTION, s, flags);
    hipError_t e = launch_attention(at<void>(ws, lay.q), at<void>(ws, lay.k), at<void>(ws, lay.vt),
                                    at<void>(ws, lay.o), H, L, Dh, 1.0 / sqrt((double)Dh), at_.in,
                                    at_.out, !f32, s);
    if ((rc = l.done(e, fn, "attention"))) return rc;
  }
  // quantise O
  if (!p.out) {
    Launch l(H3K_K_ROWQUANT_O, s, flags);
    if ((rc = l.done(launch_rows(2, at<void>(ws, lay.o), at_.o_row_type(), nullptr, nullptr, L, d, 0.f,
                                 at<int8_t>(ws, lay.qo), at<float>(ws, lay.s_o), nullptr, s),
                     fn, "rowquant_o")))
      return rc;
  }
  // out-proj + gated residual -> x1 (workspace, activation type)
  void *x1 = at<void>(ws, lay.x1);
  {
    GemmArgs a = ga;
    a.bf16_ops = p.out;
    a.A = p.out ? (const void *)at<uint16_t>(ws, lay.o) : (const void *)at<int8_t>(ws, lay.qo);
    a.B = p.out ? (const void *)w->wb_o : (const void *)w->w_o;
    a.Bt = p.out ? (const int8_t *)w->wbt_o : w->wt_o;
    a.N = d;
    a.K = d;
    a.sa = at<float>(ws, lay.s_o);
    a.sw = w->s_o;
    a.out = x1;
    a.out_f32 = f32;
    a.res = x_in;
    a.res_f32 = f32;
    a.gate = gate1;
    Launch l(H3K_K_GEMM_O, s, flags);
    if ((rc = l.done(launch_gemm(EPI_RESID, a, s), fn, "gemm_o"))) return rc;
  }
  // LN + modulate (+ quant) of x1
  {
    Launch l(H3K_K_LN_QUANT, s, flags);
    hipError_t e = p.mlp ? launch_rows(1, x1, act, shift2, scale2, L, d, dm->ln_eps, nullptr, nullptr,
                                       at<uint16_t>(ws, lay.h2), s)
                      : launch_rows(0, x1, act, shift2, scale2, L, d, dm->ln_eps,
                                    at<int8_t>(ws, lay.qa2), at<float>(ws, lay.s_a2), nullptr, s);
    if ((rc = l.done(e, fn, "ln_modulate_quant_2"))) return rc;
  }
  // MLP up + GELU
  {
    GemmArgs a = ga;
    a.bf16_ops = p.mlp;
    a.A = p.mlp ? (const void *)at<uint16_t>(ws, lay.h2) : (const void *)at<int8_t>(ws, lay.qa2);
    a.B = p.mlp ? (const void *)w->wb_up : (const void *)w->w_up;
    a.Bt = p.mlp ? (const int8_t *)w->wbt_up : w->wt_up;
    a.N = F;
    a.K = d;
    a.sa = at<float>(ws, lay.s_a2);
    a.sw = w->s_up;
    a.out = at<void>(ws, lay.g);
    a.out_f32 = f32;
    Launch l(H3K_K_GEMM_UP, s, flags);
    if ((rc = l.done(launch_gemm(EPI_GELU, a, s), fn, "gemm_up"))) return rc;
  }
  // quantise g
  if (!p.mlp) {
    Launch l(H3K_K_ROWQUANT_G, s, flags);
    if ((rc = l.done(launch_rows(2, at<void>(ws, lay.g), act, nullptr, nullptr, L, F, 0.f,
                                 at<int8_t>(ws, lay.qg), at<float>(ws, lay.s_g), nullptr, s),
                     fn, "rowquant_g")))
      return rc;
  }
  // MLP down + gated residual: x_out = x1 + gate2 * y
  {
    GemmArgs a = ga;
    a.bf16_ops = p.mlp;
    a.A = p.mlp ? (const void *)at<uint16_t>(ws, lay.g) : (const void *)at<int8_t>(ws, lay.qg);
    a.B = p.mlp ? (const void *)w->wb_down : (const void *)w->w_down;
    a.Bt = p.mlp ? (const int8_t *)w->wbt_down : w->wt_down;
    a.N = d;
    a.K = F;
    a.sa = at<float>(ws, lay.s_g);
    a.sw = w->s_down;
    a.out = x_out;
    a.out_f32 = f32;
    a.res = x1;
    a.res_f32 = f32;
    a.gate = gate2;
    Launch l(H3K_K_GEMM_DOWN, s, flags);
    if ((rc = l.done(launch_gemm(EPI_RESID, a, s), fn, "gemm_down"))) return rc;
  }
  return H3K_OK;
}

// ------------------------------------------------------------------ allocation-free block
// Workspace of h3k_block_forward_noalloc: one array per GPU, held from the library's load
// until the process ends. The name `scratch` is a host-side handle only; host code uses the
// device address hipGetSymbolAddress returns for the current device (scratch_ptr below).
static __device__ __align__(256) uint8_t scratch[H3K_NOALLOC_MAX_BYTES];

std::mutex g_scratch_mu;
void *g_scratch_ptr[64] = {};  // per device id, filled on the first call on that device

int scratch_ptr(const char *fn, void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(H3K_EHIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(H3K_EUNSUPPORTED, "%s: device id %d >= 64", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(H3K_EHIP, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return H3K_OK;
}

}  // namespace

extern "C" {

const char *h3k_last_error(void) { return g_err.c_str(); }

int h3k_block_forward_noalloc(const void *x_in, void *x_out, const float *cond,
                              const h3k_block_weights *w, const h3k_dims *dm, int64_t L,
                              uint32_t flags, void *stream) {
  const char *fn = "h3k_block_forward_noalloc";
  int rc;
  if ((rc = check_flags(fn, flags))) return rc;
  if ((rc = check_dims(fn, dm, L))) return rc;
  H3K_CHECK_PTR(x_in);
  H3K_CHECK_PTR(x_out);
  H3K_CHECK_PTR(cond);
  if ((rc = check_weights(fn, w, flags))) return rc;
  h3k_ws_layout lay;
  plan(dm, L, flags, &lay);
  if (lay.total > (size_t)H3K_NOALLOC_MAX_BYTES)
    return fail(H3K_ENOSPC, "%s: this call needs %zu bytes of workspace, more than the %zu of the "
                "allocation-free scratch; use h3k_block_forward with a caller workspace",
                fn, lay.total, (size_t)H3K_NOALLOC_MAX_BYTES);
  void *ws = nullptr;
  if ((rc = scratch_ptr(fn, &ws))) return rc;
  // no profiling events either (creating one allocates)
  const bool prof = g_prof_on;
  g_prof_on = false;
  rc = block_impl(fn, x_in, x_out, cond, w, dm, dm->grid_t, dm->grid_h, dm->grid_w, 1.f, 0.f, flags,
                  ws, (hipStream_t)stream);
  g_prof_on = prof;
  return rc;
}

int h3k_quantize_weights(const void *w, int w_dtype, int64_t n_out, int64_t k_in,
                         int8_t *q_out, float *scale_out, void *stream) {
  const char *fn = "h3k_quantize_weights";
  H3K_CHECK_PTR(w);
  H3K_CHECK_PTR(q_out);
  H3K_CHECK_PTR(scale_out);
  if (w_dtype != H3K_DT_F32 && w_dtype != H3K_DT_BF16) return fail(H3K_EINVAL, "%s: bad w_dtype %d", fn, w_dtype);
  if (n_out <= 0 || k_in <= 0) return fail(H3K_EINVAL, "%s: sizes must be positive", fn);
  if (k_in % 8) return fail(H3K_EUNSUPPORTED, "%s: k_in must be a multiple of 8", fn);
  if (k_in > 32768) return fail(H3K_EUNSUPPORTED, "%s: k_in > 32768 unsupported", fn);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_rows(2, w, w_dtype == H3K_DT_F32 ? ROW_F32 : ROW_BF16, nullptr, nullptr,
                             n_out, (int)k_in, 0.f,
                             q_out, scale_out, nullptr, s);
  if (e != hipSuccess) return fail(H3K_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return H3K_OK;
}

size_t h3k_workspace_bytes(const h3k_dims *dm, int64_t L, uint32_t flags) {
  std::string keep = g_err;
  if (check_dims("h3k_workspace_bytes", dm, L) != H3K_OK) return 0;
  h3k_ws_layout w;
  plan(dm, L, flags, &w);
  g_err = keep;
  return w.total;
}

int h3k_workspace_layout(const h3k_dims *dm, int64_t L, uint32_t flags, h3k_ws_layout *out) {
  const char *fn = "h3k_workspace_layout";
  if (!out) return fail(H3K_EINVAL, "%s: out is NULL", fn);
  int rc = check_dims(fn, dm, L);
  if (rc) return rc;
  if ((rc = check_flags(fn, flags))) return rc;
  plan(dm, L, flags, out);
  return H3K_OK;
}

int h3k_block_forward(const void *x_in, void *x_out, const float *cond,
                      const h3k_block_weights *w, const h3k_dims *dm, int64_t L,
                      uint32_t flags, void *ws, size_t ws_bytes, void *stream) {
  const char *fn = "h3k_block_forward";
  int rc;
  if ((rc = check_flags(fn, flags))) return rc;
  if ((rc = check_dims(fn, dm, L))) return rc;
  H3K_CHECK_PTR(x_in);
  H3K_CHECK_PTR(x_out);
  H3K_CHECK_PTR(cond);
  H3K_CHECK_PTR(ws);
  if ((rc = check_weights(fn, w, flags))) return rc;
  h3k_ws_layout lay;
  plan(dm, L, flags, &lay);
  if (ws_bytes < lay.total)
    return fail(H3K_ENOSPC, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, lay.total);
  return block_impl(fn, x_in, x_out, cond, w, dm, dm->grid_t, dm->grid_h, dm->grid_w, 1.f, 0.f,
                    flags, ws, (hipStream_t)stream);
}

int h3k_block_forward_grid(const void *x_in, void *x_out, const float *cond,
                           const h3k_block_weights *w, const h3k_dims *dm, int32_t T,
                           int32_t Hg, int32_t Wg, float w_pos_scale, float w_pos_offset,
                           uint32_t flags, void *ws, size_t ws_bytes, void *stream) {
  const char *fn = "h3k_block_forward_grid";
  int rc;
  if ((rc = check_flags(fn, flags))) return rc;
  if (!dm) return fail(H3K_EINVAL, "%s: dims is NULL", fn);
  h3k_dims g = *dm;
  g.grid_t = T;
  g.grid_h = Hg;
  g.grid_w = Wg;
  const int64_t L = (int64_t)T * Hg * Wg;
  if ((rc = check_dims(fn, &g, L))) return rc;
  if (!(w_pos_scale == w_pos_scale) || !(w_pos_offset == w_pos_offset))
    return fail(H3K_EINVAL, "%s: w position mapping is NaN", fn);
  H3K_CHECK_PTR(x_in);
  H3K_CHECK_PTR(x_out);
  H3K_CHECK_PTR(cond);
  H3K_CHECK_PTR(ws);
  if ((rc = check_weights(fn, w, flags))) return rc;
  h3k_ws_layout lay;
  plan(&g, L, flags, &lay);
  if (ws_bytes < lay.total)
    return fail(H3K_ENOSPC, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, lay.total);
  return block_impl(fn, x_in, x_out, cond, w, &g, T, Hg, Wg, w_pos_scale, w_pos_offset, flags, ws,
                    (hipStream_t)stream);
}

int h3k_attention(const void *q, const void *k, const void *v, void *o, int32_t n_heads,
                  int64_t L, int32_t head_dim, double softmax_scale, int dtype, uint32_t flags,
                  void *stream) {
  const char *fn = "h3k_attention";
  H3K_CHECK_PTR(q);
  H3K_CHECK_PTR(k);
  H3K_CHECK_PTR(v);
  H3K_CHECK_PTR(o);
  if (flags & ~(uint32_t)(H3K_F_SYNC | H3K_F_Q_BASE2)) return fail(H3K_EINVAL, "%s: bad flags", fn);
  if (dtype != H3K_DT_F32 && dtype != H3K_DT_BF16 && dtype != H3K_DT_F16)
    return fail(H3K_EINVAL, "%s: bad dtype %d", fn, dtype);
  const bool base2 = (flags & H3K_F_Q_BASE2) != 0;
  if (base2 && dtype == H3K_DT_F32)
    return fail(H3K_EINVAL, "%s: H3K_F_Q_BASE2 needs a 16-bit dtype", fn);
  if (n_heads <= 0 || L <= 0) return fail(H3K_EINVAL, "%s: n_heads and L must be positive", fn);
  if (head_dim != 64 && head_dim != 128) return fail(H3K_EUNSUPPORTED, "%s: head_dim must be 64 or 128", fn);
  if (L % 8) return fail(H3K_EUNSUPPORTED, "%s: L must be a multiple of 8", fn);
  if (L >= (int64_t)1 << 24 || n_heads > 65535) return fail(H3K_EUNSUPPORTED, "%s: sizes too large", fn);
  if (!(softmax_scale > 0.0)) return fail(H3K_EINVAL, "%s: softmax_scale must be positive", fn);
  hipStream_t s = (hipStream_t)stream;
  Launch l(H3K_K_ATTENTION, s, flags);
  const AttnType t = dtype == H3K_DT_F32 ? AT_F32 : (dtype == H3K_DT_F16 ? AT_F16 : AT_BF16);
  return l.done(launch_attention(q, k, v, o, n_heads, L, head_dim, softmax_scale, t, t, base2, s),
                fn, "attention");
}

size_t h3k_stack_workspace_bytes(const h3k_dims *dm, int64_t L, int32_t tr_begin,
                                 int32_t tr_end, uint32_t flags) {
  size_t b = h3k_workspace_bytes(dm, L, flags);
  if (!b) return 0;
  if (tr_end > tr_begin) {
    const size_t T = (flags & H3K_F_FP32_DEBUG) ? 4 : 2;
    b += 2 * up256((size_t)(L / 2) * dm->d * T);
  }
  return b;
}

int h3k_stack_forward(const void *x_in, void *x_out, const float *cond,
                      const h3k_block_weights *blocks, int32_t n_blocks,
                      const h3k_dims *dm, int64_t L, int32_t tr_begin, int32_t tr_end,
                      uint32_t flags, void *ws, size_t ws_bytes, void *stream) {
  const char *fn = "h3k_stack_forward";
  int rc;
  if ((rc = check_flags(fn, flags))) return rc;
  if ((rc = check_dims(fn, dm, L))) return rc;
  H3K_CHECK_PTR(x_in);
  H3K_CHECK_PTR(x_out);
  H3K_CHECK_PTR(cond);
  H3K_CHECK_PTR(ws);
  if (!blocks) return fail(H3K_EINVAL, "%s: blocks is NULL", fn);
  if (n_blocks <= 0) return fail(H3K_EINVAL, "%s: n_blocks must be positive", fn);
  if (tr_begin < 0 || tr_end < tr_begin || tr_end > n_blocks)
    return fail(H3K_EINVAL, "%s: need 0 <= tr_begin <= tr_end <= n_blocks", fn);
  const bool tr = tr_end > tr_begin;
  if (tr && (dm->grid_w % 2))
    return fail(H3K_EINVAL, "%s: token pairing needs an even grid_w", fn);
  if (tr && ((L / 2) % 8))
    return fail(H3K_EUNSUPPORTED, "%s: paired token count L/2 must be a multiple of 8", fn);
  for (int b = 0; b < n_blocks; ++b)
    if ((rc = check_weights(fn, &blocks[b], flags))) return rc;
  const size_t need = h3k_stack_workspace_bytes(dm, L, tr_begin, tr_end, flags);
  if (ws_bytes < need) return fail(H3K_ENOSPC, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);

  hipStream_t s = (hipStream_t)stream;
  const bool f32 = (flags & H3K_F_FP32_DEBUG) != 0;
  const size_t esz = f32 ? 4 : 2;
  h3k_ws_layout lay;
  plan(dm, L, flags, &lay);
  uint8_t *xr = (uint8_t *)ws + lay.total;
  uint8_t *xr_in = xr + up256((size_t)(L / 2) * dm->d * esz);
  const int T = dm->grid_t, Hg = dm->grid_h, Wg = dm->grid_w;

  const void *src = x_in;
  for (int b = 0; b < n_blocks; ++b) {
    if (tr && b == tr_begin) {
      // x_out holds the full-resolution state x_pre until the unpair
      if (src != x_out) {
        hipError_t e = launch_copy16(x_out, src, (int64_t)L * dm->d * (int64_t)esz / 16, s);
        if (e != hipSuccess) return fail(H3K_EHIP, "%s: copy failed: %s", fn, hipGetErrorString(e));
        src = x_out;
      }
      Launch l(H3K_K_TOKEN_PAIR, s, flags);
      if ((rc = l.done(launch_token_pair(x_out, xr, xr_in, f32, T, Hg, Wg, dm->d, s), fn, "token_pair")))
        return rc;
    }
    if (tr && b >= tr_begin && b < tr_end) {
      rc = block_impl(fn, xr, xr, cond, &blocks[b], dm, T, Hg, Wg / 2, 2.f, 0.5f, flags, ws, s);
    } else {
      rc = block_impl(fn, src, x_out, cond, &blocks[b], dm, T, Hg, Wg, 1.f, 0.f, flags, ws, s);
      src = x_out;
    }
    if (rc) return rc;
    if (tr && b == tr_end - 1) {
      Launch l(H3K_K_TOKEN_UNPAIR, s, flags);
      if ((rc = l.done(launch_token_unpair(x_out, xr, xr_in, f32, T, Hg, Wg, dm->d, s), fn, "token_unpair")))
        return rc;
    }
  }
  return H3K_OK;
}

size_t h3k_denoise_workspace_bytes(const h3k_dims *dm, int64_t L, int32_t tr_begin,
                                   int32_t tr_end, uint32_t flags) {
  const size_t b = h3k_stack_workspace_bytes(dm, L, tr_begin, tr_end, flags);
  if (!b) return 0;
  const size_t T = (flags & H3K_F_FP32_DEBUG) ? 4 : 2;
  const size_t n = (size_t)L * dm->d;
  return b + up256(n * T) + 2 * up256(n * 4);
}

int h3k_denoise(void *x, const float *cond, const h3k_block_weights *blocks, int32_t n_blocks,
                const h3k_dims *dm, int64_t L, int32_t steps, int32_t reuse, int32_t core_reuse,
                int32_t layers, int32_t tr_begin, int32_t tr_end, uint32_t flags, void *ws,
                size_t ws_bytes, void *stream) {
  const char *fn = "h3k_denoise";
  int rc;
  if ((rc = check_flags(fn, flags))) return rc;
  if ((rc = check_dims(fn, dm, L))) return rc;
  H3K_CHECK_PTR(x);
  H3K_CHECK_PTR(ws);
  if (steps < 1 || reuse < 1 || core_reuse < 1)
    return fail(H3K_EINVAL, "%s: steps, reuse and core_reuse must be >= 1", fn);
  if (layers < 1 || layers > n_blocks)
    return fail(H3K_EINVAL, "%s: need 1 <= layers <= n_blocks", fn);
  if (tr_begin < 0 || tr_end < tr_begin || tr_end > layers)
    return fail(H3K_EINVAL, "%s: need 0 <= tr_begin <= tr_end <= layers", fn);
  const size_t need = h3k_denoise_workspace_bytes(dm, L, tr_begin, tr_end, flags);
  if (ws_bytes < need) return fail(H3K_ENOSPC, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  const bool f32 = (flags & H3K_F_FP32_DEBUG) != 0;
  const size_t sw = h3k_stack_workspace_bytes(dm, L, tr_begin, tr_end, flags);
  const int64_t n = L * dm->d;
  uint8_t *y = (uint8_t *)ws + sw;
  float *v = (float *)(y + up256((size_t)n * (f32 ? 4 : 2)));
  float *r = (float *)((uint8_t *)v + up256((size_t)n * 4));
  // the step: exact in fp64 on the fp32 debug path; the bf16 path uses it rounded to fp32
  const double dt = f32 ? -1.0 / (double)steps : (double)(-1.0f / (float)steps);
  int fresh = 0;
  for (int k = 0; k < steps; ++k) {
    const bool last = k == steps - 1;
    if (k % reuse == 0 || last) {
      hipError_t e;
      if (fresh % core_reuse == 0 || last) {
        if ((rc = h3k_stack_forward(x, y, cond, blocks, layers, dm, L, tr_begin, tr_end, flags, ws,
                                    sw, stream)))
          return rc;
        e = launch_sampler(SAMPLER_FRESH, x, y, v, r, dt, n, f32, s);
      } else {
        e = launch_sampler(SAMPLER_REUSED, x, nullptr, v, r, dt, n, f32, s);
      }
      if (e != hipSuccess) return fail(H3K_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
      ++fresh;
    }
    hipError_t e = launch_sampler(SAMPLER_EULER, x, nullptr, v, r, dt, n, f32, s);
    if (e != hipSuccess) return fail(H3K_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  }
  return H3K_OK;
}

struct h3k_graph_s {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

int h3k_stack_graph_create(const void *x_in, void *x_out, const float *cond,
                           const h3k_block_weights *blocks, int32_t n_blocks, const h3k_dims *dm,
                           int64_t L, int32_t tr_begin, int32_t tr_end, uint32_t flags, void *ws,
                           size_t ws_bytes, void *stream, h3k_graph **graph_out) {
  const char *fn = "h3k_stack_graph_create";
  if (!graph_out) return fail(H3K_EINVAL, "%s: graph_out is NULL", fn);
  *graph_out = nullptr;
  if (!stream) return fail(H3K_EINVAL, "%s: capture needs a created stream, not the null stream", fn);
  if (flags & H3K_F_SYNC) return fail(H3K_EINVAL, "%s: H3K_F_SYNC synchronises the stream; not capturable", fn);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeRelaxed);
  if (e != hipSuccess) return fail(H3K_EHIP, "%s: begin capture: %s", fn, hipGetErrorString(e));
  const bool prof = g_prof_on;
  g_prof_on = false;  // no event nodes in the graph
  int rc = h3k_stack_forward(x_in, x_out, cond, blocks, n_blocks, dm, L, tr_begin, tr_end, flags,
                             ws, ws_bytes, stream);
  g_prof_on = prof;
  std::string err = rc ? g_err : std::string();
  hipGraph_t graph = nullptr;
  e = hipStreamEndCapture(s, &graph);
  if (rc) {
    if (graph) hipGraphDestroy(graph);
    g_err = std::string(fn) + ": " + err;
    return rc;
  }
  if (e != hipSuccess) return fail(H3K_EHIP, "%s: end capture: %s", fn, hipGetErrorString(e));
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    hipGraphDestroy(graph);
    return fail(H3K_EHIP, "%s: instantiate: %s", fn, hipGetErrorString(e));
  }
  h3k_graph *g = new h3k_graph;
  g->graph = graph;
  g->exec = exec;
  *graph_out = g;
  return H3K_OK;
}

int h3k_graph_launch(h3k_graph *graph, void *stream) {
  const char *fn = "h3k_graph_launch";
  if (!graph) return fail(H3K_EINVAL, "%s: graph is NULL", fn);
  hipError_t e = hipGraphLaunch(graph->exec, (hipStream_t)stream);
  if (e != hipSuccess) return fail(H3K_EHIP, "%s: %s", fn, hipGetErrorString(e));
  return H3K_OK;
}

void h3k_graph_destroy(h3k_graph *graph) {
  if (!graph) return;
  if (graph->exec) hipGraphExecDestroy(graph->exec);
  if (graph->graph) hipGraphDestroy(graph->graph);
  delete graph;
}

int h3k_adaln_modulation(const uint16_t *w_ada, const float *cond, float *m, int64_t n_out,
                         int32_t d_cond, void *stream) {
  const char *fn = "h3k_adaln_modulation";
  H3K_CHECK_PTR(w_ada);
  H3K_CHECK_PTR(cond);
  H3K_CHECK_PTR(m);
  if (n_out <= 0 || d_cond <= 0) return fail(H3K_EINVAL, "%s: sizes must be positive", fn);
  if (d_cond % 8 || d_cond > 8192) return fail(H3K_EUNSUPPORTED, "%s: d_cond must be a multiple of 8, <= 8192", fn);
  hipError_t e = launch_adaln(w_ada, cond, m, n_out, d_cond, false, (hipStream_t)stream);
  if (e != hipSuccess) return fail(H3K_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return H3K_OK;
}

int h3k_ln_modulate_quant(const void *x, int x_dtype, const float *shift, const float *scale,
                          int64_t rows, int32_t cols, float eps, int8_t *q_out, float *s_out,
                          void *stream) {
  const char *fn = "h3k_ln_modulate_quant";
  H3K_CHECK_PTR(x);
  H3K_CHECK_PTR(shift);
  H3K_CHECK_PTR(scale);
  H3K_CHECK_PTR(q_out);
  H3K_CHECK_PTR(s_out);
  if (x_dtype != H3K_DT_F32 && x_dtype != H3K_DT_BF16) return fail(H3K_EINVAL, "%s: bad x_dtype", fn);
  if (rows <= 0 || cols <= 0) return fail(H3K_EINVAL, "%s: sizes must be positive", fn);
  if (cols % 256 || cols > 8192) return fail(H3K_EUNSUPPORTED, "%s: cols must be a multiple of 256, <= 8192", fn);
  if (!(eps > 0.f)) return fail(H3K_EINVAL, "%s: eps must be positive", fn);
  hipError_t e = launch_rows(0, x, x_dtype == H3K_DT_F32 ? ROW_F32 : ROW_BF16, shift, scale, rows,
                             cols, eps, q_out, s_out,
                             nullptr, (hipStream_t)stream);
  if (e != hipSuccess) return fail(H3K_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return H3K_OK;
}

int h3k_row_quantize(const void *x, int x_dtype, int64_t rows, int32_t cols, int8_t *q_out,
                     float *s_out, void *stream) {
  const char *fn = "h3k_row_quantize";
  H3K_CHECK_PTR(x);
  H3K_CHECK_PTR(q_out);
  H3K_CHECK_PTR(s_out);
  if (x_dtype != H3K_DT_F32 && x_dtype != H3K_DT_BF16 && x_dtype != H3K_DT_F16)
    return fail(H3K_EINVAL, "%s: bad x_dtype", fn);
  if (rows <= 0 || cols <= 0) return fail(H3K_EINVAL, "%s: sizes must be positive", fn);
  if (cols % 8 || cols > 32768) return fail(H3K_EUNSUPPORTED, "%s: cols must be a multiple of 8, <= 32768", fn);
  const int rt = x_dtype == H3K_DT_F32 ? ROW_F32 : (x_dtype == H3K_DT_F16 ? ROW_F16 : ROW_BF16);
  hipError_t e = launch_rows(2, x, rt, nullptr, nullptr, rows, cols, 0.f, q_out, s_out,
                             nullptr, (hipStream_t)stream);
  if (e != hipSuccess) return fail(H3K_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return H3K_OK;
}

int h3k_gemm_i8_i32(const int8_t *a, const int8_t *b, int32_t *c, int64_t M, int64_t N,
                    int64_t K, void *stream) {
  const char *fn = "h3k_gemm_i8_i32";
  H3K_CHECK_PTR(a);
  H3K_CHECK_PTR(b);
  H3K_CHECK_PTR(c);
  if (M <= 0 || N <= 0 || K <= 0) return fail(H3K_EINVAL, "%s: sizes must be positive", fn);
  if (N % 256 || K % 128) return fail(H3K_EUNSUPPORTED, "%s: need N %% 256 == 0 and K %% 128 == 0", fn);
  if (N > (1 << 20) || K > (1 << 20) || M > ((int64_t)1 << 26)) return fail(H3K_EUNSUPPORTED, "%s: sizes too large", fn);
  GemmArgs g{};
  g.A = a;
  g.B = b;
  g.M = M;
  g.N = (int)N;
  g.K = (int)K;
  g.c32 = c;
  hipError_t e = launch_gemm(EPI_RAW_I32, g, (hipStream_t)stream);
  if (e != hipSuccess) return fail(H3K_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return H3K_OK;
}

int h3k_tile_weights(const int8_t *q, int64_t n_out, int64_t k_in, int8_t *q_tiled, void *stream) {
  const char *fn = "h3k_tile_weights";
  H3K_CHECK_PTR(q);
  H3K_CHECK_PTR(q_tiled);
  if (n_out <= 0 || k_in <= 0) return fail(H3K_EINVAL, "%s: sizes must be positive", fn);
  if (n_out % 16 || k_in % 64)
    return fail(H3K_EINVAL, "%s: need n_out %% 16 == 0 and k_in %% 64 == 0", fn);
  if (n_out > (1 << 20) || k_in > (1 << 20)) return fail(H3K_EUNSUPPORTED, "%s: sizes too large", fn);
  const uintptr_t a0 = (uintptr_t)q, a1 = a0 + (uintptr_t)(n_out * k_in);
  const uintptr_t b0 = (uintptr_t)q_tiled, b1 = b0 + (uintptr_t)(n_out * k_in);
  if (a0 < b1 && b0 < a1) return fail(H3K_EINVAL, "%s: q and q_tiled overlap", fn);
  if ((a0 | b0) & 15) return fail(H3K_EINVAL, "%s: q and q_tiled must be 16-byte aligned", fn);
  hipError_t e = launch_tile_weights(q, n_out, k_in, q_tiled, (hipStream_t)stream);
  if (e != hipSuccess) return fail(H3K_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return H3K_OK;
}

int h3k_gemm_i8_i32_tiled(const int8_t *a, const int8_t *b_tiled, int32_t *c, int64_t M,
                          int64_t N, int64_t K, void *stream) {
  const char *fn = "h3k_gemm_i8_i32_tiled";
  H3K_CHECK_PTR(a);
  H3K_CHECK_PTR(b_tiled);
  H3K_CHECK_PTR(c);
  if (M <= 0 || N <= 0 || K <= 0) return fail(H3K_EINVAL, "%s: sizes must be positive", fn);
  if (N % 256 || K % 128) return fail(H3K_EUNSUPPORTED, "%s: need N %% 256 == 0 and K %% 128 == 0", fn);
  if (N > (1 << 20) || K > (1 << 20) || M > ((int64_t)1 << 26)) return fail(H3K_EUNSUPPORTED, "%s: sizes too large", fn);
  GemmArgs g{};
  g.A = a;
  g.Bt = b_tiled;
  g.M = M;
  g.N = (int)N;
  g.K = (int)K;
  g.c32 = c;
  hipError_t e = launch_gemm(EPI_RAW_I32, g, (hipStream_t)stream);
  if (e != hipSuccess) return fail(H3K_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return H3K_OK;
}

int h3k_token_pair(const void *x, void *xr, void *xr_copy, int x_dtype, int32_t T, int32_t Hg,
                   int32_t Wg, int32_t d, void *stream) {
  const char *fn = "h3k_token_pair";
  H3K_CHECK_PTR(x);
  H3K_CHECK_PTR(xr);
  H3K_CHECK_PTR(xr_copy);
  if (x_dtype != H3K_DT_F32 && x_dtype != H3K_DT_BF16) return fail(H3K_EINVAL, "%s: bad x_dtype", fn);
  if (T <= 0 || Hg <= 0 || Wg <= 0 || d <= 0) return fail(H3K_EINVAL, "%s: sizes must be positive", fn);
  if (Wg % 2) return fail(H3K_EINVAL, "%s: Wg must be even", fn);
  if (d % 8) return fail(H3K_EUNSUPPORTED, "%s: d must be a multiple of 8", fn);
  hipError_t e = launch_token_pair(x, xr, xr_copy, x_dtype == H3K_DT_F32, T, Hg, Wg, d, (hipStream_t)stream);
  if (e != hipSuccess) return fail(H3K_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return H3K_OK;
}

int h3k_token_unpair(void *x_pre, const void *xr_out, const void *xr_in, int x_dtype, int32_t T,
                     int32_t Hg, int32_t Wg, int32_t d, void *stream) {
  const char *fn = "h3k_token_unpair";
  H3K_CHECK_PTR(x_pre);
  H3K_CHECK_PTR(xr_out);
  H3K_CHECK_PTR(xr_in);
  if (x_dtype != H3K_DT_F32 && x_dtype != H3K_DT_BF16) return fail(H3K_EINVAL, "%s: bad x_dtype", fn);
  if (T <= 0 || Hg <= 0 || Wg <= 0 || d <= 0) return fail(H3K_EINVAL, "%s: sizes must be positive", fn);
  if (Wg % 2) return fail(H3K_EINVAL, "%s: Wg must be even", fn);
  if (d % 8) return fail(H3K_EUNSUPPORTED, "%s: d must be a multiple of 8", fn);
  hipError_t e = launch_token_unpair(x_pre, xr_out, xr_in, x_dtype == H3K_DT_F32, T, Hg, Wg, d,
                                     (hipStream_t)stream);
  if (e != hipSuccess) return fail(H3K_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return H3K_OK;
}

int h3k_profile_enable(int on) {
  for (auto &r : g_prof) {
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_prof.clear();
  g_prof_on = on != 0;
  return H3K_OK;
}

int h3k_profile_read(int kind, int64_t *count, double *total_ms) {
  const char *fn = "h3k_profile_read";
  if (kind < 0 || kind >= H3K_K_COUNT) return fail(H3K_EINVAL, "%s: bad kind %d", fn, kind);
  if (!count || !total_ms) return fail(H3K_EINVAL, "%s: NULL output", fn);
  int64_t n = 0;
  double t = 0.0;
  for (auto &r : g_prof) {
    if (r.kind != kind) continue;
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return fail(H3K_EHIP, "%s: %s", fn, hipGetErrorString(e));
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return fail(H3K_EHIP, "%s: %s", fn, hipGetErrorString(e));
    ++n;
    t += ms;
  }
  *count = n;
  *total_ms = t;
  return H3K_OK;
}

}  // extern "C"
