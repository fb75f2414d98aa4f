"""Python binding of libh3k.so (ctypes): argument marshalling only.

Every step of the block runs in the library's HIP kernels; torch provides device memory
and the current stream. There is no fallback: if the library is missing, or a tensor is
not on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libh3k.so")

OK, EINVAL, EUNSUPPORTED, ENOSPC, EHIP = 0, -1, -2, -3, -4
F_BF16_GEMM, F_FP32_DEBUG, F_SYNC = 1, 2, 4
# per-projection bf16 GEMMs (the precision series); F_BF16_GEMM is all three
F_BF16_QKV, F_BF16_OUT, F_BF16_MLP = 8, 16, 32
DT_F32, DT_BF16 = 0, 1
KERNELS = ["adaln", "rope_table", "ln_quant", "gemm_qkv", "attention", "rowquant_o",
           "gemm_o", "gemm_up", "rowquant_g", "gemm_down", "token_pair", "token_unpair"]


class H3kError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"h3k error {code}: {msg}")
        self.code = code


class Dims(C.Structure):
    _fields_ = [("d", C.c_int32), ("n_heads", C.c_int32), ("head_dim", C.c_int32),
                ("d_ff", C.c_int32), ("d_cond", C.c_int32), ("grid_t", C.c_int32),
                ("grid_h", C.c_int32), ("grid_w", C.c_int32), ("rope_theta", C.c_float),
                ("ln_eps", C.c_float)]


class BlockWeightsC(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "w_ada", "w_qkv", "s_qkv", "w_o", "s_o", "w_up", "s_up", "w_down", "s_down",
        "wb_qkv", "wb_o", "wb_up", "wb_down")]


class WsLayout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in (
        "m", "rope", "s_a", "s_o", "s_a2", "s_g", "qa", "qo", "qa2", "qg", "q", "k", "vt",
        "o", "x1", "g", "h", "h2", "total")]


_lib = None


def lib() -> C.CDLL:
    """Load libh3k.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m video_diffusion_transformer_03_amd.build`")
        L = C.CDLL(LIB_PATH)
        vp, i64, i32, u32, f32, sz = C.c_void_p, C.c_int64, C.c_int32, C.c_uint32, C.c_float, C.c_size_t
        sigs = {
            "h3k_quantize_weights": (C.c_int, [vp, C.c_int, i64, i64, vp, vp, vp]),
            "h3k_workspace_bytes": (sz, [C.POINTER(Dims), i64, u32]),
            "h3k_workspace_layout": (C.c_int, [C.POINTER(Dims), i64, u32, C.POINTER(WsLayout)]),
            "h3k_block_forward": (C.c_int, [vp, vp, vp, C.POINTER(BlockWeightsC), C.POINTER(Dims),
                                            i64, u32, vp, sz, vp]),
            "h3k_block_forward_grid": (C.c_int, [vp, vp, vp, C.POINTER(BlockWeightsC), C.POINTER(Dims),
                                                 i32, i32, i32, f32, f32, u32, vp, sz, vp]),
            "h3k_attention": (C.c_int, [vp, vp, vp, vp, i32, i64, i32, C.c_double, u32, vp]),
            "h3k_stack_workspace_bytes": (sz, [C.POINTER(Dims), i64, i32, i32, u32]),
            "h3k_stack_forward": (C.c_int, [vp, vp, vp, C.POINTER(BlockWeightsC), i32,
                                            C.POINTER(Dims), i64, i32, i32, u32, vp, sz, vp]),
            "h3k_adaln_modulation": (C.c_int, [vp, vp, vp, i64, i32, vp]),
            "h3k_ln_modulate_quant": (C.c_int, [vp, C.c_int, vp, vp, i64, i32, f32, vp, vp, vp]),
            "h3k_row_quantize": (C.c_int, [vp, C.c_int, i64, i32, vp, vp, vp]),
            "h3k_gemm_i8_i32": (C.c_int, [vp, vp, vp, i64, i64, i64, vp]),
            "h3k_token_pair": (C.c_int, [vp, vp, vp, C.c_int, i32, i32, i32, i32, vp]),
            "h3k_token_unpair": (C.c_int, [vp, vp, vp, C.c_int, i32, i32, i32, i32, vp]),
            "h3k_last_error": (C.c_char_p, []),
            "h3k_denoise_workspace_bytes": (sz, [C.POINTER(Dims), i64, i32, i32, u32]),
            "h3k_denoise": (C.c_int, [vp, vp, C.POINTER(BlockWeightsC), i32, C.POINTER(Dims), i64,
                                      i32, i32, i32, i32, i32, i32, u32, vp, sz, vp]),
            "h3k_stack_graph_create": (C.c_int, [vp, vp, vp, C.POINTER(BlockWeightsC), i32,
                                                 C.POINTER(Dims), i64, i32, i32, u32, vp, sz, vp,
                                                 C.POINTER(vp)]),
            "h3k_graph_launch": (C.c_int, [vp, vp]),
            "h3k_graph_destroy": (None, [vp]),
            "h3k_profile_enable": (C.c_int, [C.c_int]),
            "h3k_profile_read": (C.c_int, [C.c_int, C.POINTER(i64), C.POINTER(C.c_double)]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().h3k_last_error().decode()


def _check(rc: int):
    if rc != OK:
        raise H3kError(rc, last_error())


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dev(t: Optional[torch.Tensor], name: str) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DT_BF16
    if t.dtype == torch.float32:
        return DT_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def make_dims(d, n_heads, head_dim, d_ff, d_cond, grid, rope_theta=10000.0, ln_eps=1e-6) -> Dims:
    return Dims(d, n_heads, head_dim, d_ff, d_cond, grid[0], grid[1], grid[2], rope_theta, ln_eps)


def dims_of(wl) -> Dims:
    """Dims of a synthetic workload description (d, n_heads, head_dim, d_ff, d_cond, grid)."""
    return make_dims(wl.d, wl.n_heads, wl.head_dim, wl.d_ff, wl.d_cond, wl.grid)


@dataclass
class BlockWeights:
    """Device tensors of one block (int8 codes + fp32 scales; optional dense bf16)."""
    w_ada: torch.Tensor
    w_qkv: Optional[torch.Tensor] = None
    s_qkv: Optional[torch.Tensor] = None
    w_o: Optional[torch.Tensor] = None
    s_o: Optional[torch.Tensor] = None
    w_up: Optional[torch.Tensor] = None
    s_up: Optional[torch.Tensor] = None
    w_down: Optional[torch.Tensor] = None
    s_down: Optional[torch.Tensor] = None
    wb_qkv: Optional[torch.Tensor] = None
    wb_o: Optional[torch.Tensor] = None
    wb_up: Optional[torch.Tensor] = None
    wb_down: Optional[torch.Tensor] = None

    def c_struct(self) -> BlockWeightsC:
        return BlockWeightsC(*[_dev(getattr(self, f), f) for f, _ in BlockWeightsC._fields_])


# ------------------------------------------------------------------------ entry points
def quantize_weights(w: torch.Tensor, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-output-channel int8 quantisation of w [N, K] (bf16 or fp32, on the GPU)."""
    n, k = w.shape
    q = torch.empty((n, k), dtype=torch.int8, device=w.device)
    s = torch.empty((n,), dtype=torch.float32, device=w.device)
    _check(lib().h3k_quantize_weights(_dev(w, "w"), _dt(w), n, k, q.data_ptr(), s.data_ptr(),
                                      _stream(stream)))
    return q, s


def quantize_block(wb: Dict[str, torch.Tensor], keep_bf16: bool = False, stream=None) -> BlockWeights:
    """BlockWeights from dense bf16 device weights {w_ada, w_qkv, w_o, w_up, w_down}."""
    out = BlockWeights(w_ada=wb["w_ada"])
    for k in ("w_qkv", "w_o", "w_up", "w_down"):
        q, s = quantize_weights(wb[k], stream)
        setattr(out, k, q)
        setattr(out, "s" + k[1:], s)
        if keep_bf16:
            setattr(out, "wb" + k[1:], wb[k])
    return out


def workspace_bytes(dims: Dims, L: int, flags: int = 0) -> int:
    n = lib().h3k_workspace_bytes(C.byref(dims), L, flags)
    if n == 0:
        raise H3kError(EINVAL, "invalid dims for workspace_bytes")
    return n


def workspace_layout(dims: Dims, L: int, flags: int = 0) -> Dict[str, int]:
    lay = WsLayout()
    _check(lib().h3k_workspace_layout(C.byref(dims), L, flags, C.byref(lay)))
    return {f: getattr(lay, f) for f, _ in WsLayout._fields_}


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty((nbytes,), dtype=torch.uint8, device=device)


def block_forward(x: torch.Tensor, cond: torch.Tensor, w: BlockWeights, dims: Dims,
                  flags: int = 0, ws: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    L = x.shape[0]
    if ws is None:
        ws = alloc_workspace(workspace_bytes(dims, L, flags), x.device)
    if out is None:
        out = torch.empty_like(x)
    wc = w.c_struct()
    _check(lib().h3k_block_forward(_dev(x, "x"), _dev(out, "out"), _dev(cond, "cond"), C.byref(wc),
                                   C.byref(dims), L, flags, _dev(ws, "ws"), ws.numel(),
                                   _stream(stream)))
    return out


def block_forward_grid(x: torch.Tensor, cond: torch.Tensor, w: BlockWeights, dims: Dims, grid,
                       w_pos_scale: float = 1.0, w_pos_offset: float = 0.0, flags: int = 0,
                       ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """One block on the token grid `grid` with w positions w * scale + offset."""
    T, Hg, Wg = grid
    L = x.shape[0]
    if ws is None:
        g = Dims.from_buffer_copy(dims)
        g.grid_t, g.grid_h, g.grid_w = T, Hg, Wg
        ws = alloc_workspace(workspace_bytes(g, L, flags), x.device)
    if out is None:
        out = torch.empty_like(x)
    wc = w.c_struct()
    _check(lib().h3k_block_forward_grid(_dev(x, "x"), _dev(out, "out"), _dev(cond, "cond"), C.byref(wc),
                                        C.byref(dims), T, Hg, Wg, float(w_pos_scale), float(w_pos_offset),
                                        flags, _dev(ws, "ws"), ws.numel(), _stream(stream)))
    return out


def ws_view(ws: torch.Tensor, layout: Dict[str, int], name: str, dtype, shape) -> torch.Tensor:
    """A view of one intermediate inside a block workspace."""
    n = 1
    for s in shape:
        n *= s
    nbytes = n * torch.empty((), dtype=dtype).element_size()
    off = layout[name]
    return ws[off:off + nbytes].view(dtype).view(*shape)


def attention(q: torch.Tensor, k: torch.Tensor, vt: torch.Tensor, softmax_scale: Optional[float] = None,
              flags: int = 0, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """q, k [H, L, Dh]; vt [H, Dh, L] -> o [L, H*Dh]."""
    H, L, Dh = q.shape
    if softmax_scale is None:
        softmax_scale = Dh ** -0.5
    if out is None:
        out = torch.empty((L, H * Dh), dtype=q.dtype, device=q.device)
    _check(lib().h3k_attention(_dev(q, "q"), _dev(k, "k"), _dev(vt, "vt"), _dev(out, "out"), H, L, Dh,
                               float(softmax_scale), flags, _stream(stream)))
    return out


def stack_workspace_bytes(dims: Dims, L: int, tr_begin: int, tr_end: int, flags: int = 0) -> int:
    n = lib().h3k_stack_workspace_bytes(C.byref(dims), L, tr_begin, tr_end, flags)
    if n == 0:
        raise H3kError(EINVAL, "invalid dims for stack_workspace_bytes")
    return n


def stack_forward(x: torch.Tensor, cond: torch.Tensor, blocks: Sequence[BlockWeights], dims: Dims,
                  tr_begin: int = 0, tr_end: int = 0, flags: int = 0,
                  ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    L = x.shape[0]
    if ws is None:
        ws = alloc_workspace(stack_workspace_bytes(dims, L, tr_begin, tr_end, flags), x.device)
    if out is None:
        out = torch.empty_like(x)
    arr = (BlockWeightsC * len(blocks))(*[b.c_struct() for b in blocks])
    _check(lib().h3k_stack_forward(_dev(x, "x"), _dev(out, "out"), _dev(cond, "cond"), arr, len(blocks),
                                   C.byref(dims), L, tr_begin, tr_end, flags, _dev(ws, "ws"),
                                   ws.numel(), _stream(stream)))
    return out


def denoise_workspace_bytes(dims: Dims, L: int, tr_begin: int = 0, tr_end: int = 0, flags: int = 0) -> int:
    return lib().h3k_denoise_workspace_bytes(C.byref(dims), L, tr_begin, tr_end, flags)


def denoise(x: torch.Tensor, cond: torch.Tensor, blocks: Sequence[BlockWeights], dims: Dims,
            steps: int, reuse: int = 1, core_reuse: int = 1, layers: Optional[int] = None,
            tr_begin: int = 0, tr_end: int = 0, flags: int = 0,
            ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """h3k_denoise: `steps` Euler steps on x in place (x: [L, d] noise in, result out)."""
    L = x.shape[0]
    layers = len(blocks) if layers is None else layers
    if ws is None:
        ws = alloc_workspace(denoise_workspace_bytes(dims, L, tr_begin, tr_end, flags), x.device)
    arr = (BlockWeightsC * len(blocks))(*[b.c_struct() for b in blocks])
    _check(lib().h3k_denoise(_dev(x, "x"), _dev(cond, "cond"), arr, len(blocks), C.byref(dims), L,
                             steps, reuse, core_reuse, layers, tr_begin, tr_end, flags,
                             _dev(ws, "ws"), ws.numel(), _stream(stream)))
    return x


class StackGraph:
    """A recorded h3k_stack_forward call (h3k_stack_graph_create). launch() replays it on
    a stream; it reads x and cond as they are at launch time and writes out. Holds the
    tensors it was recorded with, so they stay alive while the graph exists."""

    def __init__(self, x, cond, blocks, dims, tr_begin, tr_end, flags, ws, out, capture_stream):
        self._keep = (x, cond, list(blocks), ws, out)
        self.out = out
        arr = (BlockWeightsC * len(blocks))(*[b.c_struct() for b in blocks])
        h = C.c_void_p()
        _check(lib().h3k_stack_graph_create(_dev(x, "x"), _dev(out, "out"), _dev(cond, "cond"), arr,
                                            len(blocks), C.byref(dims), x.shape[0], tr_begin, tr_end,
                                            flags, _dev(ws, "ws"), ws.numel(),
                                            C.c_void_p(capture_stream.cuda_stream), C.byref(h)))
        self._h = h

    def launch(self, stream=None) -> torch.Tensor:
        _check(lib().h3k_graph_launch(self._h, _stream(stream)))
        return self.out

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            lib().h3k_graph_destroy(h)
            self._h = None


def stack_graph(x: torch.Tensor, cond: torch.Tensor, blocks: Sequence[BlockWeights], dims: Dims,
                tr_begin: int = 0, tr_end: int = 0, flags: int = 0,
                ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> StackGraph:
    """Record a stack step (captured on a side stream created here; nothing runs)."""
    L = x.shape[0]
    if ws is None:
        ws = alloc_workspace(stack_workspace_bytes(dims, L, tr_begin, tr_end, flags), x.device)
    if out is None:
        out = torch.empty_like(x)
    side = torch.cuda.Stream(device=x.device)
    torch.cuda.current_stream(x.device).synchronize()
    return StackGraph(x, cond, blocks, dims, tr_begin, tr_end, flags, ws, out, side)


def adaln_modulation(w_ada: torch.Tensor, cond: torch.Tensor, stream=None) -> torch.Tensor:
    n, dc = w_ada.shape
    m = torch.empty((n,), dtype=torch.float32, device=w_ada.device)
    _check(lib().h3k_adaln_modulation(_dev(w_ada, "w_ada"), _dev(cond, "cond"), m.data_ptr(), n, dc,
                                      _stream(stream)))
    return m


def ln_modulate_quant(x: torch.Tensor, shift: torch.Tensor, scale: torch.Tensor, eps: float = 1e-6,
                      stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    s = torch.empty((rows,), dtype=torch.float32, device=x.device)
    _check(lib().h3k_ln_modulate_quant(_dev(x, "x"), _dt(x), _dev(shift, "shift"), _dev(scale, "scale"),
                                       rows, cols, eps, q.data_ptr(), s.data_ptr(), _stream(stream)))
    return q, s


def row_quantize(x: torch.Tensor, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    s = torch.empty((rows,), dtype=torch.float32, device=x.device)
    _check(lib().h3k_row_quantize(_dev(x, "x"), _dt(x), rows, cols, q.data_ptr(), s.data_ptr(),
                                  _stream(stream)))
    return q, s


def gemm_i8_i32(a: torch.Tensor, b: torch.Tensor, stream=None) -> torch.Tensor:
    M, K = a.shape
    N = b.shape[0]
    c = torch.empty((M, N), dtype=torch.int32, device=a.device)
    _check(lib().h3k_gemm_i8_i32(_dev(a, "a"), _dev(b, "b"), c.data_ptr(), M, N, K, _stream(stream)))
    return c


def token_pair(x: torch.Tensor, grid, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    T, Hg, Wg = grid
    d = x.shape[1]
    xr = torch.empty((T * Hg * (Wg // 2), d), dtype=x.dtype, device=x.device)
    xr2 = torch.empty_like(xr)
    _check(lib().h3k_token_pair(_dev(x, "x"), xr.data_ptr(), xr2.data_ptr(), _dt(x), T, Hg, Wg, d,
                                _stream(stream)))
    return xr, xr2


def token_unpair(x_pre: torch.Tensor, xr_out: torch.Tensor, xr_in: torch.Tensor, grid,
                 stream=None) -> torch.Tensor:
    """In place on x_pre; returns it."""
    T, Hg, Wg = grid
    _check(lib().h3k_token_unpair(_dev(x_pre, "x_pre"), _dev(xr_out, "xr_out"), _dev(xr_in, "xr_in"),
                                  _dt(x_pre), T, Hg, Wg, x_pre.shape[1], _stream(stream)))
    return x_pre


def profile_enable(on: bool = True):
    _check(lib().h3k_profile_enable(1 if on else 0))


def profile_read() -> Dict[str, Tuple[int, float]]:
    """{kernel: (launches, total ms)} for the records since profile_enable."""
    out = {}
    for i, name in enumerate(KERNELS):
        n = C.c_int64()
        t = C.c_double()
        _check(lib().h3k_profile_read(i, C.byref(n), C.byref(t)))
        out[name] = (n.value, t.value)
    return out
