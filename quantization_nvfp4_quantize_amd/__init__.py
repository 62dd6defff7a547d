"""Python binding of libnvfp4moe.so, the MI355X (gfx950) NVFP4 MoE hot path.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/nvfp4moe.h``.  torch supplies
device memory (``data_ptr()``) and the current stream; nothing here computes
on the host.  If the shared library has not been built this module raises on
import -- there is no fallback path.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4moe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
        "or `python quantization_nvfp4_quantize_amd/build.py` (needs hipcc for gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t


class MoeArgs(ctypes.Structure):
    """Mirror of nvfp4_moe_args (include/nvfp4moe.h)."""
    _fields_ = [
        ("T", _i64), ("H", _i64), ("I", _i64), ("E", _i64), ("topk", _i64),
        ("x", _vp), ("x_gs_in", _vp), ("topk_ids", _vp), ("topk_w", _vp),
        ("w1_q", _vp), ("w1_sf", _vp), ("w1_gs", _vp),
        ("w2_q", _vp), ("w2_sf", _vp), ("w2_gs", _vp),
        ("a2_gs", _vp), ("out", _vp), ("out_dtype", ctypes.c_int),
        ("xq", _vp), ("xsf", _vp), ("x_gs_out", _vp),
        ("l1_c_bf16", _vp), ("l1_q", _vp), ("l1_sf", _vp), ("err_count", _vp),
        ("stage_events", ctypes.POINTER(_vp)),
        ("tile_rows", ctypes.c_int32),
        ("a2_gs_out", _vp),
        ("l1_unfused", ctypes.c_int32),
        ("aux_stream", _vp),
        ("aux_events", ctypes.POINTER(_vp)),
        ("w1_sf_paired", _vp), ("w2_sf_paired", _vp),
    ]


_SIG = {
    "nvfp4_version": (ctypes.c_int, []),
    "nvfp4_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "nvfp4_last_error": (ctypes.c_char_p, []),
    "nvfp4_quantize_workspace_size": (_sz, [_i64, _i64]),
    "nvfp4_quantize": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "nvfp4_dequantize": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, ctypes.c_int, _vp, _vp]),
    "nvfp4_pair_scales": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp]),
    "nvfp4_gemm_swiglu_quant_workspace_size": (_sz, [_i64, _i64, _i64]),
    "nvfp4_gemm_swiglu_quant": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _i64,
                                               _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "nvfp4_linear_workspace_size": (_sz, [_i64, _i64, _i64]),
    "nvfp4_linear": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _vp, _vp, _i64, ctypes.c_int, _vp, _vp,
                                    _vp, _sz, _vp]),
    "mxfp4_quantize": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "mxfp4_dequantize": (ctypes.c_int, [_vp, _vp, _i64, _i64, ctypes.c_int, _vp, _vp]),
    "mxfp4_linear_workspace_size": (_sz, [_i64, _i64, _i64]),
    "mxfp4_linear": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _i64, ctypes.c_int, _vp, _vp, _sz, _vp]),
    "moe_expert_ffn_nvfp4_workspace_size": (_sz, [ctypes.POINTER(MoeArgs)]),
    "moe_expert_ffn_nvfp4": (ctypes.c_int, [ctypes.POINTER(MoeArgs), _vp, _sz, _vp]),
    "moe_expert_ffn_nvfp4_noalloc": (ctypes.c_int, [ctypes.POINTER(MoeArgs), _vp]),
}
for _name, (_res, _args) in _SIG.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTS = tuple(_SIG)


class Nvfp4Error(RuntimeError):
    def __init__(self, status, where):
        msg = _lib.nvfp4_last_error().decode() or _lib.nvfp4_status_string(status).decode()
        super().__init__(f"{where}: status {status}: {msg}")
        self.status = status


def _check(status, where):
    if status != 0:
        raise Nvfp4Error(status, where)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require(t, dtype, name):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(nbytes, device):
    """A fresh device workspace of at least nbytes for one call.

    It comes from torch's caching allocator on the current stream, so a block
    is handed out again only after the work queued on that stream has used
    it: calls on different streams never share one, and a graph captured
    around a call keeps its block in the graph's private pool for as long as
    the graph lives.  (The allocator caches freed blocks, so a call of the
    same size costs no device allocation.)"""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ API
def quantize(x, gs=None, out=None):
    """bf16 [M][K] -> (q uint8 [M][K/2], sf uint8 [M][K/16], gs float32 [1]).

    gs: optional float32 [1] device tensor (supplied global scale); by default
    the global scale is max|x| / 2688 computed on the device."""
    _require(x, torch.bfloat16, "x")
    _require(gs, torch.float32, "gs")
    M, K = x.shape
    dev = x.device
    if out is None:
        q = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        sf = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
        gs_out = torch.empty(1, dtype=torch.float32, device=dev) if gs is None else None
    else:
        q, sf, gs_out = out
        if gs is not None:
            gs_out = None  # the supplied scale is returned as is; nothing to copy
    wsz = _lib.nvfp4_quantize_workspace_size(M, K)
    ws = _workspace(wsz, dev)
    _check(_lib.nvfp4_quantize(_p(x), M, K, _p(gs), _p(q), _p(sf), _p(gs_out), _p(ws), ws.numel(),
                               _stream(dev)), "nvfp4_quantize")
    return q, sf, (gs if gs is not None else gs_out)


def dequantize(q, sf, gs, out_dtype=torch.bfloat16, out=None):
    """NVFP4 -> bf16 or float32 [M][K]."""
    _require(q, torch.uint8, "q")
    _require(sf, torch.uint8, "sf")
    _require(gs, torch.float32, "gs")
    M, K2 = q.shape
    K = 2 * K2
    if out is None:
        out = torch.empty((M, K), dtype=out_dtype, device=q.device)
    code = {torch.bfloat16: 0, torch.float32: 1}[out.dtype]
    _check(_lib.nvfp4_dequantize(_p(q), _p(sf), _p(gs), M, K, code, _p(out), _stream(q.device)),
           "nvfp4_dequantize")
    return out


def gemm_swiglu_quant(a_q, a_sf, a_gs, w_q, w_sf, w_gs, out_gs, want_bf16=True, out=None, expand_a=True):
    """One expert's L1 stage: returns (c bf16 [M][I] or None, c_q [M][I/2],
    c_sf [M][I/16]).  Weight rows are gate/up interleaved by 8.
    expand_a: pass a workspace (the activations are expanded to f16 once),
    else none (the GEMM dequantizes the NVFP4 activations into LDS)."""
    for t, n, d in ((a_q, "a_q", torch.uint8), (a_sf, "a_sf", torch.uint8), (a_gs, "a_gs", torch.float32),
                    (w_q, "w_q", torch.uint8), (w_sf, "w_sf", torch.uint8), (w_gs, "w_gs", torch.float32),
                    (out_gs, "out_gs", torch.float32)):
        _require(t, d, n)
    M, K = a_q.shape[0], a_q.shape[1] * 2
    N2 = w_q.shape[0]
    I = N2 // 2
    dev = a_q.device
    if out is None:
        c = torch.empty((M, I), dtype=torch.bfloat16, device=dev) if want_bf16 else None
        cq = torch.empty((M, I // 2), dtype=torch.uint8, device=dev)
        csf = torch.empty((M, I // 16), dtype=torch.uint8, device=dev)
    else:
        c, cq, csf = out
    ws = _workspace(_lib.nvfp4_gemm_swiglu_quant_workspace_size(M, K, N2), dev) if expand_a else None
    _check(_lib.nvfp4_gemm_swiglu_quant(_p(a_q), _p(a_sf), _p(a_gs), M, K, _p(w_q), _p(w_sf), _p(w_gs),
                                        N2, _p(out_gs), _p(c), _p(cq), _p(csf), _p(ws),
                                        0 if ws is None else ws.numel(), _stream(dev)), "nvfp4_gemm_swiglu_quant")
    return c, cq, csf


def linear(x, w_q, w_sf, w_gs, out_dtype=torch.bfloat16, x_gs=None, x_gs_out=None, out=None, ws=None):
    """Dense NVFP4 linear: y [M][N] = alpha * NVFP4(x) @ W^T (out_dtype bf16 or
    float32).  x bf16 [M][K]; w_q [N][K/2], w_sf [N][K/16], w_gs float32 [1];
    x_gs: supplied activation global scale (float32 [1]) or None (dynamic);
    x_gs_out: float32 [1] that receives the scale used."""
    _require(x, torch.bfloat16, "x")
    for t, n, d in ((w_q, "w_q", torch.uint8), (w_sf, "w_sf", torch.uint8), (w_gs, "w_gs", torch.float32),
                    (x_gs, "x_gs", torch.float32), (x_gs_out, "x_gs_out", torch.float32)):
        _require(t, d, n)
    M, K = x.shape
    N = w_q.shape[0]
    dev = x.device
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    code = {torch.bfloat16: 0, torch.float32: 1}[out.dtype]
    if ws is None:
        ws = _workspace(_lib.nvfp4_linear_workspace_size(M, K, N), dev)
    _check(_lib.nvfp4_linear(_p(x), M, K, _p(x_gs), _p(w_q), _p(w_sf), _p(w_gs), N, code, _p(out),
                             _p(x_gs_out), _p(ws), ws.numel(), _stream(dev)), "nvfp4_linear")
    return out


def linear_workspace(M, K, N, device):
    """A dedicated workspace for nvfp4_linear (e.g. for graph capture)."""
    return torch.empty(max(int(_lib.nvfp4_linear_workspace_size(M, K, N)), 256), dtype=torch.uint8,
                       device=device)


# ------------------------------------------------------------------ MXFP4
# The separately labelled OCP MX v1.0 format (E8M0 scale per 32 elements) on
# the scaled FP4 MFMA; not the NVFP4 of the functions above.
def mx_quantize(x, out=None):
    """bf16 [M][K] (K % 32 == 0) -> (q uint8 [M][K/2], scale codes uint8 [M][K/32])."""
    _require(x, torch.bfloat16, "x")
    M, K = x.shape
    if out is None:
        out = (torch.empty((M, K // 2), dtype=torch.uint8, device=x.device),
               torch.empty((M, K // 32), dtype=torch.uint8, device=x.device))
    q, sc = out
    _check(_lib.mxfp4_quantize(_p(x), M, K, _p(q), _p(sc), _stream(x.device)), "mxfp4_quantize")
    return q, sc


def mx_dequantize(q, sc, out_dtype=torch.bfloat16, out=None):
    """MXFP4 -> bf16 or float32 [M][K]."""
    _require(q, torch.uint8, "q")
    _require(sc, torch.uint8, "scale")
    M, K = q.shape[0], 2 * q.shape[1]
    if out is None:
        out = torch.empty((M, K), dtype=out_dtype, device=q.device)
    code = {torch.bfloat16: 0, torch.float32: 1}[out.dtype]
    _check(_lib.mxfp4_dequantize(_p(q), _p(sc), M, K, code, _p(out), _stream(q.device)), "mxfp4_dequantize")
    return out


def mx_linear(x, w_q, w_sc, out_dtype=torch.bfloat16, out=None, ws=None):
    """Dense MXFP4 linear: y [M][N] = MXFP4(x) @ W^T with W MXFP4 [N][K]."""
    _require(x, torch.bfloat16, "x")
    _require(w_q, torch.uint8, "w_q")
    _require(w_sc, torch.uint8, "w_scale")
    M, K = x.shape
    N = w_q.shape[0]
    dev = x.device
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    code = {torch.bfloat16: 0, torch.float32: 1}[out.dtype]
    if ws is None:
        ws = _workspace(_lib.mxfp4_linear_workspace_size(M, K, N), dev)
    _check(_lib.mxfp4_linear(_p(x), M, K, _p(w_q), _p(w_sc), N, code, _p(out), _p(ws), ws.numel(),
                             _stream(dev)), "mxfp4_linear")
    return out


def mx_linear_workspace(M, K, N, device):
    """A dedicated workspace for mxfp4_linear (e.g. for graph capture)."""
    return torch.empty(max(int(_lib.mxfp4_linear_workspace_size(M, K, N)), 256), dtype=torch.uint8,
                       device=device)


def pair_scales(sf, out=None):
    """A weight block-scale tensor [..., R, C] (uint8, C = K/16 bytes per row)
    in the row-paired layout of nvfp4_pair_scales (each 128-byte line holds
    64 bytes of rows 2j and 2j + 1), for the 32-row MoE tiles.  The leading
    dimensions are taken as more rows (the experts' rows are consecutive);
    needs an even row count per matrix and C % 64 == 0.  Returns a new
    tensor of the same shape (or fills out)."""
    _require(sf, torch.uint8, "sf")
    C = sf.shape[-1]
    R = sf.numel() // C if C else 0
    if out is None:
        out = torch.empty_like(sf)
    _require(out, torch.uint8, "out")
    _check(_lib.nvfp4_pair_scales(_p(sf), R, C, _p(out), _stream(sf.device)), "nvfp4_pair_scales")
    return out


def moe_args(x, topk_ids, topk_w, w1_q, w1_sf, w1_gs, w2_q, w2_sf, w2_gs, a2_gs, out,
             x_gs=None, xq=None, xsf=None, x_gs_out=None, l1_c=None, l1_q=None, l1_sf=None,
             err_count=None, tile_rows=0, a2_gs_out=None, l1_unfused=False, aux=None,
             w1_sf_paired=None, w2_sf_paired=None):
    """Build the nvfp4_moe_args struct from tensors.  The struct holds
    references to every tensor it points at, so they stay allocated for as
    long as the struct lives (a temporary passed here cannot be freed and its
    memory reused while a launch still reads it).
    tile_rows: 0 lets the library choose the GEMM tiles; 32 or 256 forces
    one tile height, 288 the mixed tiling (256-row tiles, each expert's last
    block of at most 64 rows on one or two 32-row tiles).
    a2_gs None: dynamic L1-output global scale (unfused flow); l1_unfused:
    True / 1 the unfused flow with the supplied a2_gs, "interleaved" / 2 the
    interleaved-output flow; a2_gs_out receives the scale.  aux: None, or
    (torch.cuda.Stream, (torch.cuda.Event, torch.cuda.Event)) on which the
    short tiles of the mixed tiling run concurrently (the events must have
    been recorded once, so that they exist); the struct then holds the event
    handle array, which the caller keeps alive with the struct.
    w1_sf_paired, w2_sf_paired: pair_scales(w1_sf), pair_scales(w2_sf), read
    by the 32-row tiles when H (resp. I) is a multiple of 1024."""
    _require(x, torch.bfloat16, "x")
    _require(topk_ids, torch.int32, "topk_ids")
    _require(topk_w, torch.float32, "topk_w")
    T, H = x.shape
    E, N2 = w1_q.shape[0], w1_q.shape[1]
    k = topk_ids.shape[1]
    code = {torch.bfloat16: 0, torch.float32: 1}[out.dtype]
    a = MoeArgs(T, H, N2 // 2, E, k, _p(x), _p(x_gs), _p(topk_ids), _p(topk_w),
                _p(w1_q), _p(w1_sf), _p(w1_gs), _p(w2_q), _p(w2_sf), _p(w2_gs), _p(a2_gs),
                _p(out), code, _p(xq), _p(xsf), _p(x_gs_out), _p(l1_c), _p(l1_q), _p(l1_sf),
                _p(err_count))
    _require(w1_sf_paired, torch.uint8, "w1_sf_paired")
    _require(w2_sf_paired, torch.uint8, "w2_sf_paired")
    a._refs = (x, topk_ids, topk_w, w1_q, w1_sf, w1_gs, w2_q, w2_sf, w2_gs, a2_gs, out, x_gs, xq, xsf, x_gs_out,
               l1_c, l1_q, l1_sf, err_count, a2_gs_out, w1_sf_paired, w2_sf_paired)
    a.w1_sf_paired = _p(w1_sf_paired)
    a.w2_sf_paired = _p(w2_sf_paired)
    a.tile_rows = int(tile_rows)
    a.a2_gs_out = _p(a2_gs_out)
    a.l1_unfused = {False: 0, True: 1, 0: 0, 1: 1, 2: 2, "interleaved": 2}[l1_unfused]
    if aux is not None:
        stream, (ev0, ev1) = aux
        a._aux_events = (ctypes.c_void_p * 2)(ev0.cuda_event, ev1.cuda_event)
        a.aux_stream = stream.cuda_stream
        a.aux_events = ctypes.cast(a._aux_events, ctypes.POINTER(ctypes.c_void_p))
    return a


def moe_workspace_size(args):
    return int(_lib.moe_expert_ffn_nvfp4_workspace_size(ctypes.byref(args)))


def moe_expert_ffn_raw(args, device, ws=None):
    """Launch with a prepared MoeArgs (the bench's hot loop uses this)."""
    need = moe_workspace_size(args)
    if ws is None:
        ws = _workspace(need, device)
    _check(_lib.moe_expert_ffn_nvfp4(ctypes.byref(args), _p(ws), ws.numel(), _stream(device)),
           "moe_expert_ffn_nvfp4")


def moe_expert_ffn_noalloc(args, device):
    """Launch with a prepared MoeArgs on the library's static per-GPU scratch
    buffer (moe_expert_ffn_nvfp4_noalloc): no workspace is allocated here
    or in the library.  Calls that overlap on one GPU race on that buffer."""
    _check(_lib.moe_expert_ffn_nvfp4_noalloc(ctypes.byref(args), _stream(device)), "moe_expert_ffn_nvfp4_noalloc")


def moe_expert_ffn(x, topk_ids, topk_w, w1_q, w1_sf, w1_gs, w2_q, w2_sf, w2_gs, a2_gs,
                   out_dtype=torch.bfloat16, x_gs=None, debug=False, tile_rows=0, l1_unfused=False,
                   aux=None, w1_sf_paired=None, w2_sf_paired=None):
    """NVFP4 MoE expert FFN.  Returns y [T][H] (out_dtype), plus with
    debug=True a dict of the intermediate outputs (xq, xsf, x_gs, l1_c,
    l1_q, l1_sf, err_count, a2_gs_out).  a2_gs None: dynamic L1-output
    global scale.  tile_rows, l1_unfused, aux, w1_sf_paired, w2_sf_paired:
    see moe_args."""
    T, H = x.shape
    I = w1_q.shape[1] // 2
    k = topk_ids.shape[1]
    P = T * k
    dev = x.device
    out = torch.empty((T, H), dtype=out_dtype, device=dev)
    dbg = {}
    if debug:
        dbg = dict(xq=torch.empty((T, H // 2), dtype=torch.uint8, device=dev),
                   xsf=torch.empty((T, H // 16), dtype=torch.uint8, device=dev),
                   x_gs_out=torch.empty(1, dtype=torch.float32, device=dev),
                   l1_c=torch.zeros((P, I), dtype=torch.bfloat16, device=dev),
                   l1_q=torch.zeros((P, I // 2), dtype=torch.uint8, device=dev),
                   l1_sf=torch.zeros((P, I // 16), dtype=torch.uint8, device=dev),
                   err_count=torch.zeros(1, dtype=torch.int32, device=dev),
                   a2_gs_out=torch.empty(1, dtype=torch.float32, device=dev))
    args = moe_args(x, topk_ids, topk_w, w1_q, w1_sf, w1_gs, w2_q, w2_sf, w2_gs, a2_gs, out,
                    x_gs=x_gs, tile_rows=tile_rows, l1_unfused=l1_unfused, aux=aux,
                    w1_sf_paired=w1_sf_paired, w2_sf_paired=w2_sf_paired, **dbg)
    moe_expert_ffn_raw(args, dev)
    if debug:
        return out, dbg
    return out


def quantize_experts(w, gs_out=None):
    """Quantize a stack of expert weight matrices [E][R][K] (bf16), each with
    its own dynamic global scale.  Returns (q [E][R][K/2], sf [E][R][K/16],
    gs float32 [E]).  Model preparation, not part of the hot path."""
    E, R, K = w.shape
    dev = w.device
    q = torch.empty((E, R, K // 2), dtype=torch.uint8, device=dev)
    sf = torch.empty((E, R, K // 16), dtype=torch.uint8, device=dev)
    gs = torch.empty(E, dtype=torch.float32, device=dev) if gs_out is None else gs_out
    for e in range(E):
        quantize(w[e], out=(q[e], sf[e], gs[e:e + 1]))
    return q, sf, gs
