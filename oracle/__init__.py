"""NVFP4 CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it, and the two share no code.

Thin numpy/ctypes wrapper around ``nvfp4_oracle.c`` and ``mxfp4_oracle.c``:
argument marshalling, and the composition of C calls in the pages' order
(``moe_tokens_dynamic`` runs the C MoE once for the L1 outputs, takes their
global scale with the C rule, then runs the C MoE with it); every arithmetic
step lives in the C files.  ``nvfp4_oracle.c`` cites the pages ("nvfp4-megamoe-kernel":
NVFP4-1.1_APPROACH_PART_2.md, NVFP4-1.1_APPROACH.md, DEBUG_LOG.md "NVFP4 MoE
Pipeline") it follows; ``mxfp4_oracle.c`` follows the OCP Microscaling
Formats (MX) Specification v1.0, which defines the MXFP4 format of the
separately labelled scaled-MFMA variant (the pages do not define it).

``Oracle(path)`` wraps one build of the library (tests also load deliberately
mutated builds to show that the pins catch plausible mistakes); the module
level functions use the default build next to this file.
"""
import ctypes
import importlib
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB = os.path.join(_HERE, "liborc.so")

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)


class MoeProblem(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64), ("H", ctypes.c_int64), ("I", ctypes.c_int64),
        ("E", ctypes.c_int64), ("topk", ctypes.c_int64),
        ("x", _u16p), ("x_gs_in", _f32p),
        ("topk_ids", _i32p), ("topk_w", _f32p),
        ("w1_q", _u8p), ("w1_sf", _u8p), ("w1_gs", _f32p),
        ("w2_q", _u8p), ("w2_sf", _u8p), ("w2_gs", _f32p),
        ("a2_gs", ctypes.c_float),
    ]


_SIGNATURES = {
    "orc_bf16_to_float": (ctypes.c_float, [ctypes.c_uint16]),
    "orc_double_to_bf16": (ctypes.c_uint16, [ctypes.c_double]),
    "orc_e4m3_value": (ctypes.c_double, [ctypes.c_uint32]),
    "orc_e4m3_encode": (ctypes.c_uint32, [ctypes.c_float]),
    "orc_e4m3_encode_array": (None, [_f32p, ctypes.c_int64, _u8p]),
    "orc_step_to_idx": (ctypes.c_int, [ctypes.c_int]),
    "orc_e2m1_value": (ctypes.c_double, [ctypes.c_uint32]),
    "orc_e2m1_nibble": (ctypes.c_uint32, [ctypes.c_float, ctypes.c_int]),
    "orc_global_scale": (ctypes.c_float, [_u16p, ctypes.c_int64]),
    "orc_quantize_block": (ctypes.c_uint32, [_f32p, ctypes.c_float, _u8p]),
    "orc_quantize": (None, [_u16p, ctypes.c_int64, ctypes.c_int64, ctypes.c_float, _u8p, _u8p,
                            ctypes.c_int]),
    "orc_dequantize": (None, [_u8p, _u8p, ctypes.c_float, ctypes.c_int64, ctypes.c_int64,
                              _f32p]),
    "orc_dequantize_bf16": (None, [_u8p, _u8p, ctypes.c_float, ctypes.c_int64, ctypes.c_int64,
                                   _u16p]),
    "orc_l1_swiglu_rows": (None, [_u8p, _u8p, ctypes.c_float, ctypes.c_int64, _u8p, _u8p,
                                  ctypes.c_float, ctypes.c_int64, _i64p, ctypes.c_int64, _f64p,
                                  _u16p, ctypes.c_int]),
    "orc_mx_scale_value": (ctypes.c_double, [ctypes.c_uint32]),
    "orc_mx_scale_code": (ctypes.c_uint32, [ctypes.c_double]),
    "orc_mx_e2m1_value": (ctypes.c_double, [ctypes.c_uint32]),
    "orc_mx_e2m1_nibble": (ctypes.c_uint32, [ctypes.c_double]),
    "orc_mx_quantize_block": (ctypes.c_uint32, [_u16p, _u8p]),
    "orc_mx_quantize": (None, [_u16p, ctypes.c_int64, ctypes.c_int64, _u8p, _u8p]),
    "orc_mx_dequantize": (None, [_u8p, _u8p, ctypes.c_int64, ctypes.c_int64, _f64p]),
    "orc_mx_linear": (None, [_u8p, _u8p, ctypes.c_int64, ctypes.c_int64, _u8p, _u8p, ctypes.c_int64,
                             _f64p, ctypes.c_int]),
    "orc_linear_rows": (None, [_u8p, _u8p, ctypes.c_float, ctypes.c_int64, _u8p, _u8p, ctypes.c_float, _i64p,
                                ctypes.c_int64, _i64p, ctypes.c_int64, _f32p, ctypes.c_int]),
    "orc_moe_tokens": (ctypes.c_float, [ctypes.POINTER(MoeProblem), _i64p, ctypes.c_int64,
                                        _f32p, _u16p, _u8p, _u8p, ctypes.c_int]),
}


def _ptr(a, typ):
    if a is None:
        return ctypes.cast(None, typ)
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(typ)


def default_threads():
    return max(1, min(16, os.cpu_count() or 1))


class Oracle:
    """One loaded build of the oracle library."""

    def __init__(self, path=DEFAULT_LIB):
        if path == DEFAULT_LIB and not os.path.exists(path):
            # import the submodule explicitly: a from-import would first look the
            # name up through this module's __getattr__ and recurse into here
            _b = importlib.import_module(__name__ + ".build")
            _b.build()
        self.path = path
        L = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        self.L = L

    # ------------------------------------------------------------ scalars
    def e4m3_value(self, code):
        return self.L.orc_e4m3_value(int(code))

    def e4m3_encode(self, v):
        return int(self.L.orc_e4m3_encode(float(v)))

    def e4m3_encode_array(self, v):
        v = np.ascontiguousarray(v, np.float32)
        out = np.zeros(v.shape, np.uint8)
        self.L.orc_e4m3_encode_array(_ptr(v, _f32p), v.size, _ptr(out, _u8p))
        return out

    def step_to_idx(self, hs):
        return int(self.L.orc_step_to_idx(int(hs)))

    def e2m1_value(self, nibble):
        return self.L.orc_e2m1_value(int(nibble))

    def e2m1_nibble(self, s, negative):
        return int(self.L.orc_e2m1_nibble(float(s), 1 if negative else 0))

    def double_to_bf16(self, v):
        return int(self.L.orc_double_to_bf16(float(v)))

    # ------------------------------------------------------------ tensors
    def global_scale(self, x_bf16):
        """x_bf16: uint16 array of bf16 bit patterns."""
        x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
        return np.float32(self.L.orc_global_scale(_ptr(x, _u16p), x.size))

    def quantize_block(self, xb, g):
        xb = np.ascontiguousarray(xb, dtype=np.float32)
        assert xb.size == 16
        q = np.zeros(8, np.uint8)
        sf = self.L.orc_quantize_block(_ptr(xb, _f32p), float(np.float32(g)), _ptr(q, _u8p))
        return q, int(sf)

    def quantize(self, x_bf16, g, threads=None):
        """x_bf16: uint16 [M][K] bf16 bit patterns, K % 16 == 0.
        Returns (q uint8 [M][K/2], sf uint8 [M][K/16])."""
        x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
        M, K = x.shape
        assert K % 16 == 0
        q = np.zeros((M, K // 2), np.uint8)
        sf = np.zeros((M, K // 16), np.uint8)
        if M:
            self.L.orc_quantize(_ptr(x, _u16p), M, K, float(np.float32(g)), _ptr(q, _u8p),
                                _ptr(sf, _u8p), threads or default_threads())
        return q, sf

    def dequantize(self, q, sf, g, out_dtype="f32"):
        """Returns fp32 values, or bf16 bit patterns (uint16) for "bf16"."""
        q = np.ascontiguousarray(q, dtype=np.uint8)
        sf = np.ascontiguousarray(sf, dtype=np.uint8)
        M, K2 = q.shape
        K = 2 * K2
        assert sf.shape == (M, K // 16)
        if out_dtype == "f32":
            out = np.zeros((M, K), np.float32)
            self.L.orc_dequantize(_ptr(q, _u8p), _ptr(sf, _u8p), float(np.float32(g)), M, K,
                                  _ptr(out, _f32p))
        else:
            out = np.zeros((M, K), np.uint16)
            self.L.orc_dequantize_bf16(_ptr(q, _u8p), _ptr(sf, _u8p), float(np.float32(g)), M,
                                       K, _ptr(out, _u16p))
        return out

    def l1_swiglu_rows(self, aq, asf, a_gs, wq, wsf, w_gs, rows, want_h=False, threads=None):
        """Single-expert L1 GEMM + SwiGLU for a list of activation rows.
        aq [M][K/2], asf [M][K/16]; wq [N2][K/2], wsf [N2][K/16] (rows
        interleaved by 8: gate, up).  Returns (c bf16 bits [n][N2/2],
        h fp64 [n][N2] or None)."""
        aq = np.ascontiguousarray(aq, np.uint8)
        asf = np.ascontiguousarray(asf, np.uint8)
        wq = np.ascontiguousarray(wq, np.uint8)
        wsf = np.ascontiguousarray(wsf, np.uint8)
        rows = np.ascontiguousarray(rows, np.int64)
        K = aq.shape[1] * 2
        N2 = wq.shape[0]
        n = rows.size
        c = np.zeros((n, N2 // 2), np.uint16)
        h = np.zeros((n, N2), np.float64) if want_h else None
        if n:
            self.L.orc_l1_swiglu_rows(_ptr(aq, _u8p), _ptr(asf, _u8p), float(np.float32(a_gs)),
                                      K, _ptr(wq, _u8p), _ptr(wsf, _u8p),
                                      float(np.float32(w_gs)), N2, _ptr(rows, _i64p), n,
                                      _ptr(h, _f64p), _ptr(c, _u16p),
                                      threads or default_threads())
        return c, h

    def moe_tokens(self, x, topk_ids, topk_w, w1_q, w1_sf, w1_gs, w2_q, w2_sf, w2_gs, a2_gs,
                   tokens=None, x_gs=None, want_pairs=False, threads=None):
        """MoE expert FFN for the listed tokens (all tokens by default).
        Returns dict: y fp32 [n][H], x_gs; with want_pairs also c [n][k][I]
        bf16 bits, a2_q [n][k][I/2], a2_sf [n][k][I/16]."""
        x = np.ascontiguousarray(x, np.uint16)
        T, H = x.shape
        topk_ids = np.ascontiguousarray(topk_ids, np.int32)
        topk_w = np.ascontiguousarray(topk_w, np.float32)
        k = topk_ids.shape[1]
        w1_q = np.ascontiguousarray(w1_q, np.uint8)
        w1_sf = np.ascontiguousarray(w1_sf, np.uint8)
        w2_q = np.ascontiguousarray(w2_q, np.uint8)
        w2_sf = np.ascontiguousarray(w2_sf, np.uint8)
        w1_gs = np.ascontiguousarray(w1_gs, np.float32)
        w2_gs = np.ascontiguousarray(w2_gs, np.float32)
        E, N2 = w1_q.shape[0], w1_q.shape[1]
        I = N2 // 2
        assert w1_q.shape == (E, 2 * I, H // 2) and w1_sf.shape == (E, 2 * I, H // 16)
        assert w2_q.shape == (E, H, I // 2) and w2_sf.shape == (E, H, I // 16)
        if tokens is None:
            tokens = np.arange(T, dtype=np.int64)
        tokens = np.ascontiguousarray(tokens, np.int64)
        n = tokens.size
        xg = None if x_gs is None else np.array([x_gs], np.float32)
        pb = MoeProblem(T, H, I, E, k, _ptr(x, _u16p), _ptr(xg, _f32p), _ptr(topk_ids, _i32p),
                        _ptr(topk_w, _f32p), _ptr(w1_q, _u8p), _ptr(w1_sf, _u8p),
                        _ptr(w1_gs, _f32p), _ptr(w2_q, _u8p), _ptr(w2_sf, _u8p),
                        _ptr(w2_gs, _f32p), float(np.float32(a2_gs)))
        y = np.zeros((n, H), np.float32)
        c = a2q = a2sf = None
        if want_pairs:
            c = np.zeros((n, k, I), np.uint16)
            a2q = np.zeros((n, k, I // 2), np.uint8)
            a2sf = np.zeros((n, k, I // 16), np.uint8)
        used = self.L.orc_moe_tokens(ctypes.byref(pb), _ptr(tokens, _i64p), n, _ptr(y, _f32p),
                                     _ptr(c, _u16p), _ptr(a2q, _u8p), _ptr(a2sf, _u8p),
                                     threads or default_threads())
        out = {"y": y, "x_gs": np.float32(used)}
        if want_pairs:
            out.update(c=c, a2_q=a2q, a2_sf=a2sf)
        return out

    def linear(self, x_bf16, w_q, w_sf, w_gs, x_gs=None, rows=None, cols=None, threads=None):
        """Dense NVFP4 linear (the MoE's activation quantization and GEMM
        without routing, DEBUG_LOG.md "NVFP4 MoE Pipeline"): x is quantized
        with g = x_gs or the global scale of the whole x, both operands are
        dequantized exactly (e2m1 * block scale, no global scale) and
        y = f32(g * w_gs) * (A @ W^T) in fp64 (orc_linear_rows), returned as
        fp32 for the listed rows and output columns (all by default), with g."""
        x = np.ascontiguousarray(x_bf16, np.uint16)
        g = self.global_scale(x) if x_gs is None else np.float32(x_gs)
        rows = np.arange(x.shape[0]) if rows is None else np.asarray(rows, np.int64)
        cols = np.arange(w_q.shape[0]) if cols is None else np.asarray(cols, np.int64)
        xq, xsf = self.quantize(x[rows], g)  # rows are independent given g
        w_q = np.ascontiguousarray(w_q, np.uint8)
        w_sf = np.ascontiguousarray(w_sf, np.uint8)
        K = x.shape[1]
        assert w_q.shape[1] * 2 == K and w_sf.shape[1] * 16 == K
        loc = np.ascontiguousarray(np.arange(rows.size), np.int64)
        cols = np.ascontiguousarray(cols, np.int64)
        y = np.zeros((rows.size, cols.size), np.float32)
        if rows.size and cols.size:
            self.L.orc_linear_rows(_ptr(xq, _u8p), _ptr(xsf, _u8p), float(g), K, _ptr(w_q, _u8p),
                                   _ptr(w_sf, _u8p), float(np.float32(w_gs)), _ptr(loc, _i64p), loc.size,
                                   _ptr(cols, _i64p), cols.size, _ptr(y, _f32p),
                                   threads or default_threads())
        return y, np.float32(g)

    def moe_tokens_dynamic(self, x, topk_ids, topk_w, w1_q, w1_sf, w1_gs, w2_q, w2_sf, w2_gs,
                           tokens=None, x_gs=None, want_pairs=False, threads=None):
        """MoE expert FFN with a dynamic global scale for the L1 output, as
        in DEBUG_LOG.md "NVFP4 MoE Pipeline" (stage_activation of the
        activated rows): the SwiGLU output c of every valid pair of every
        token is formed first, its global scale is g2 = amax / 2688 by the
        same rule as for the activations, and then the listed tokens are run
        with g2 as the L1-output scale.  Returns moe_tokens' dict plus a2_gs."""
        T = np.asarray(x).shape[0]
        # c does not depend on the L1-output scale: any placeholder works here
        allc = self.moe_tokens(x, topk_ids, topk_w, w1_q, w1_sf, w1_gs, w2_q, w2_sf, w2_gs, 1.0,
                               tokens=np.arange(T), x_gs=x_gs, want_pairs=True,
                               threads=threads)["c"]
        # pairs of skipped experts stay zero in c and do not change the amax
        g2 = self.global_scale(allc.reshape(-1, allc.shape[-1]))
        out = self.moe_tokens(x, topk_ids, topk_w, w1_q, w1_sf, w1_gs, w2_q, w2_sf, w2_gs, g2,
                              tokens=tokens, x_gs=x_gs, want_pairs=want_pairs, threads=threads)
        out["a2_gs"] = np.float32(g2)
        return out


    # ------------------------------------------------------------ MXFP4
    # The OCP MX v1.0 format (E8M0 scale per 32 elements), mxfp4_oracle.c.
    def mx_scale_value(self, code):
        return self.L.orc_mx_scale_value(int(code))

    def mx_scale_code(self, amax):
        return int(self.L.orc_mx_scale_code(float(amax)))

    def mx_e2m1_value(self, nibble):
        return self.L.orc_mx_e2m1_value(int(nibble))

    def mx_e2m1_nibble(self, v):
        return int(self.L.orc_mx_e2m1_nibble(float(v)))

    def mx_quantize_block(self, xb_bf16):
        xb = np.ascontiguousarray(xb_bf16, dtype=np.uint16)
        assert xb.size == 32
        q = np.zeros(16, np.uint8)
        code = self.L.orc_mx_quantize_block(_ptr(xb, _u16p), _ptr(q, _u8p))
        return q, int(code)

    def mx_quantize(self, x_bf16):
        """x_bf16: uint16 [M][K] bf16 bit patterns, K % 32 == 0.
        Returns (q uint8 [M][K/2], scale codes uint8 [M][K/32])."""
        x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
        M, K = x.shape
        assert K % 32 == 0
        q = np.zeros((M, K // 2), np.uint8)
        sc = np.zeros((M, K // 32), np.uint8)
        if M:
            self.L.orc_mx_quantize(_ptr(x, _u16p), M, K, _ptr(q, _u8p), _ptr(sc, _u8p))
        return q, sc

    def mx_dequantize(self, q, sc):
        """Exact values (float64) of an MXFP4 matrix."""
        q = np.ascontiguousarray(q, dtype=np.uint8)
        sc = np.ascontiguousarray(sc, dtype=np.uint8)
        M, K2 = q.shape
        K = 2 * K2
        assert sc.shape == (M, K // 32)
        out = np.zeros((M, K), np.float64)
        if M:
            self.L.orc_mx_dequantize(_ptr(q, _u8p), _ptr(sc, _u8p), M, K, _ptr(out, _f64p))
        return out

    def mx_linear(self, aq, asc, wq, wsc, threads=None):
        """y [M][N] = A @ W^T in float64 for MXFP4 A [M][K], W [N][K]."""
        aq, asc = np.ascontiguousarray(aq, np.uint8), np.ascontiguousarray(asc, np.uint8)
        wq, wsc = np.ascontiguousarray(wq, np.uint8), np.ascontiguousarray(wsc, np.uint8)
        M, K = aq.shape[0], aq.shape[1] * 2
        N = wq.shape[0]
        assert wq.shape[1] * 2 == K and asc.shape == (M, K // 32) and wsc.shape == (N, K // 32)
        y = np.zeros((M, N), np.float64)
        if M and N:
            self.L.orc_mx_linear(_ptr(aq, _u8p), _ptr(asc, _u8p), M, K, _ptr(wq, _u8p), _ptr(wsc, _u8p), N,
                                 _ptr(y, _f64p), threads or default_threads())
        return y


_default = None


def default():
    global _default
    if _default is None:
        _default = Oracle()
    return _default


_SUBMODULES = ("build",)


def __getattr__(name):
    # module-level access to the default build's methods: oracle.quantize(...)
    if name.startswith("_"):
        raise AttributeError(name)
    if name in _SUBMODULES:
        return importlib.import_module(__name__ + "." + name)
    return getattr(default(), name)
