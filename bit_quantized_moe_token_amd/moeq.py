"""Python binding of libmoeq over torch device tensors.

torch provides device memory and the current HIP stream; each function below
validates shapes, passes raw pointers to the C ABI and returns the tensors
the library filled.  No arithmetic of the method happens here.
"""

import ctypes
from ctypes import c_void_p

import numpy as np
import torch

from . import _lib
from ._lib import MoeqError, check, lib  # noqa: F401

GATE, UP, DOWN = 0, 1, 2


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, dtype, shape, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ------------------------------------------------------------- encoding

def quantize_rtn(w, bits, G):
    """Asymmetric RTN of an fp16 block [N, K]: (codes u8 [N,K], scales fp16
    [N,K/G], zeros u8 [N,K/G])."""
    N, K = w.shape
    _need(w, torch.float16, (N, K), "w")
    codes = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    scales = torch.empty((N, K // G), dtype=torch.float16, device=w.device)
    zeros = torch.empty((N, K // G), dtype=torch.uint8, device=w.device)
    check(lib().moeq_quantize_rtn(_ptr(w), N, K, G, bits, _ptr(codes), _ptr(scales), _ptr(zeros),
                                  _stream()), "moeq_quantize_rtn")
    return codes, scales, zeros


def build_lut(w, codes4, scales, zeros, q, G):
    """16-slot fp16 LUT [N, K/G, 16] of a block committed to q bit-planes."""
    N, K = w.shape
    _need(w, torch.float16, (N, K), "w")
    _need(codes4, torch.uint8, (N, K), "codes4")
    _need(scales, torch.float16, (N, K // G), "scales")
    _need(zeros, torch.uint8, (N, K // G), "zeros")
    lut = torch.empty((N, K // G, 16), dtype=torch.float16, device=w.device)
    check(lib().moeq_build_lut(_ptr(w), _ptr(codes4), _ptr(scales), _ptr(zeros), N, K, G, q,
                               _ptr(lut), _stream()), "moeq_build_lut")
    return lut


def fit_lowrank(w, codes, scales, zeros, G, omega, r, power_iters=2):
    """Rank-r compensator factors (U fp16 [N, r], V fp16 [r, K]) of the mean
    RTN residual of the blocks w [n, N, K] (or one block [N, K]); omega
    fp32 [K, l] is the Gaussian test matrix (see moeq_fit_lowrank)."""
    if w.dim() == 2:
        w, codes, scales, zeros = (t.unsqueeze(0) for t in (w, codes, scales, zeros))
    n_mat, N, K = w.shape
    l = omega.shape[1]
    _need(w, torch.float16, (n_mat, N, K), "w")
    _need(codes, torch.uint8, (n_mat, N, K), "codes")
    _need(scales, torch.float16, (n_mat, N, K // G), "scales")
    _need(zeros, torch.uint8, (n_mat, N, K // G), "zeros")
    _need(omega, torch.float32, (K, l), "omega")
    n = ctypes.c_size_t(0)
    check(lib().moeq_fit_lowrank_workspace_size(N, K, r, l, ctypes.byref(n)), "moeq_fit_lowrank_workspace_size")
    ws = torch.empty((max(1, n.value),), dtype=torch.uint8, device=w.device)
    U = torch.empty((N, r), dtype=torch.float16, device=w.device)
    V = torch.empty((r, K), dtype=torch.float16, device=w.device)
    check(lib().moeq_fit_lowrank(_ptr(w), _ptr(codes), _ptr(scales), _ptr(zeros), n_mat, N, K, G, _ptr(omega), l, r,
                                 power_iters, _ptr(U), _ptr(V), _ptr(ws), n.value, _stream()), "moeq_fit_lowrank")
    return U, V


# ---------------------------------------------------------------- layer

def _ptr_array(tensors):
    arr = (ctypes.c_void_p * len(tensors))()
    for i, t in enumerate(tensors):
        arr[i] = t.data_ptr() if t is not None else 0
    return arr


class PackedLayer:
    """A packed quantized layer: one device buffer plus the library handle.

    blocks: list over b = e*3 + blk of dicts with
      INT:      codes u8 [N,K], scales fp16 [N,K/G], zeros u8 [N,K/G]
      bitplane: codes (4-bit parent codes) u8 [N,K], lut fp16 [N,K/G,16]
    factors: list over b of (U [N,r], V [r,K]) fp16 or None (r = 0)
    shared: list over group*3+blk of (Us, Vs) or None (rs = 0)
    """

    def __init__(self, E, H, I, G, fmt, bits, blocks, factors=None, shared=None, share=0,
                 device=None):
        device = device or torch.device("cuda", torch.cuda.current_device())
        self.E, self.H, self.I, self.G = E, H, I, G
        self.fmt = fmt
        self.bits = np.asarray(bits, dtype=np.uint8).reshape(E * 3).copy()
        nb = 3 * E
        assert len(blocks) == nb
        fmt_id = _lib.FMT_INT if fmt == "int" else _lib.FMT_BITPLANE
        self._keep = []
        codes = _ptr_array([b["codes"] for b in blocks])
        if fmt == "int":
            scales = _ptr_array([b["scales"] for b in blocks])
            zeros = _ptr_array([b["zeros"] for b in blocks])
            luts = None
        else:
            scales = zeros = None
            luts = _ptr_array([b["lut"] for b in blocks])
        r = 0
        U = V = None
        if factors is not None and factors[0] is not None:
            r = factors[0][0].shape[1]
            U = _ptr_array([f[0] for f in factors])
            V = _ptr_array([f[1] for f in factors])
        rs = 0
        Us = Vs = None
        if shared is not None and shared[0] is not None:
            rs = shared[0][0].shape[1]
            Us = _ptr_array([f[0] for f in shared])
            Vs = _ptr_array([f[1] for f in shared])
        self.r, self.rs, self.share = r, rs, share
        bits_arr = (ctypes.c_uint8 * nb)(*[int(b) for b in self.bits])
        cast = lambda a: ctypes.cast(a, _lib.c_vpp) if a is not None else None
        d = _lib.LayerDesc(E, H, I, G, fmt_id, ctypes.cast(bits_arr, _lib.c_u8p), cast(codes),
                           cast(scales), cast(zeros), cast(luts), r, cast(U), cast(V), rs, share,
                           cast(Us), cast(Vs))
        self._desc_keep = (bits_arr, codes, scales, zeros, luts, U, V, Us, Vs)
        nbytes = ctypes.c_size_t(0)
        check(lib().moeq_pack_size(ctypes.byref(d), ctypes.byref(nbytes)), "moeq_pack_size")
        self.buf = torch.empty(nbytes.value, dtype=torch.uint8, device=device)
        handle = ctypes.c_void_p(0)
        check(lib().moeq_pack(ctypes.byref(d), _ptr(self.buf), nbytes.value, _stream(),
                              ctypes.byref(handle)), "moeq_pack")
        self.handle = handle
        self.nbytes = nbytes.value

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value and _lib._lib is not None:
            _lib._lib.moeq_layer_destroy(h)
            self.handle = None

    def block_bytes(self, e, blk):
        out = ctypes.c_size_t(0)
        check(lib().moeq_layer_block_bytes(self.handle, e, blk, ctypes.byref(out)), "block_bytes")
        return out.value

    def shared_bytes(self, g, blk):
        out = ctypes.c_size_t(0)
        check(lib().moeq_layer_shared_bytes(self.handle, g, blk, ctypes.byref(out)), "shared_bytes")
        return out.value

    def block_shape(self, blk):
        return (self.I, self.H) if blk in (GATE, UP) else (self.H, self.I)

    def debug_unpack(self, e, blk):
        N, K = self.block_shape(blk)
        out = torch.empty((N, K), dtype=torch.uint8, device=self.buf.device)
        check(lib().moeq_debug_unpack(self.handle, e, blk, _ptr(out), _stream()), "moeq_debug_unpack")
        return out

    def commit_bits(self, e, blk, q, lut):
        """Commit bit-plane count q of block (e, blk) with its LUT [N, K/G, 16]
        (see moeq_commit_bits); stream-ordered on the current stream."""
        N, K = self.block_shape(blk)
        _need(lut, torch.float16, (N, K // self.G, 16), "lut")
        check(lib().moeq_commit_bits(self.handle, e, blk, q, _ptr(lut), _stream()), "moeq_commit_bits")

    def committed_bits(self, e, blk):
        q = ctypes.c_int32(0)
        check(lib().moeq_committed_bits(self.handle, e, blk, ctypes.byref(q)), "moeq_committed_bits")
        return q.value

    def plane_release(self, e, blk, host, stream=None):
        """Copy the planes above the committed q to the pinned host tensor
        `host` (uint8, plane p at offset p * plane_bytes) on `stream`
        (default: the current stream) and mark them released."""
        s = ctypes.c_void_p((stream or torch.cuda.current_stream()).cuda_stream)
        check(lib().moeq_plane_release(self.handle, e, blk, _ptr(host), host.numel(), s), "moeq_plane_release")

    def plane_reload(self, e, blk, q, host, stream=None):
        """Copy planes back from `host` until q planes are resident (see
        moeq_plane_reload)."""
        s = ctypes.c_void_p((stream or torch.cuda.current_stream()).cuda_stream)
        check(lib().moeq_plane_reload(self.handle, e, blk, q, _ptr(host), host.numel(), s), "moeq_plane_reload")

    def plane_event(self, e, blk):
        """The hipEvent_t (as an integer) of the block's last release or reload copy."""
        ev = c_void_p(0)
        check(lib().moeq_plane_event(self.handle, e, blk, ctypes.byref(ev)), "moeq_plane_event")
        return ev.value

    def resident_planes(self, e, blk):
        n = ctypes.c_int32(0)
        check(lib().moeq_resident_planes(self.handle, e, blk, ctypes.byref(n)), "moeq_resident_planes")
        return n.value

    def set_desired_bits(self, e, blk, d):
        check(lib().moeq_set_desired_bits(self.handle, e, blk, d), "moeq_set_desired_bits")

    def desired_bits(self, e, blk):
        d = ctypes.c_int32(0)
        check(lib().moeq_desired_bits(self.handle, e, blk, ctypes.byref(d)), "moeq_desired_bits")
        return d.value

    def plane_region(self, e, blk, plane):
        """(device address, bytes) of bit-plane `plane` (0 = most significant)."""
        ptr, n = c_void_p(0), ctypes.c_size_t(0)
        check(lib().moeq_plane_region(self.handle, e, blk, plane, ctypes.byref(ptr), ctypes.byref(n)),
              "moeq_plane_region")
        return ptr.value, n.value


def quantize_block(w, fmt, bits, G):
    """Quantize one fp16 block with the library's kernels into the pack input
    dict (INT: codes/scales/zeros; bit-plane: 4-bit parent codes + LUT)."""
    if fmt == "int":
        c, s, z = quantize_rtn(w, bits, G)
        return dict(codes=c, scales=s, zeros=z)
    c, s, z = quantize_rtn(w, 4, G)
    return dict(codes=c, lut=build_lut(w, c, s, z, bits, G))


# -------------------------------------------------------------- routing

class RoutingOut:
    def __init__(self, T, E, k, device):
        self.T, self.E, self.k = T, E, k
        P = T * k
        self.ids = torch.empty((T, k), dtype=torch.int32, device=device)
        self.gates = torch.empty((T, k), dtype=torch.float32, device=device)
        self.offsets = torch.empty((E + 1,), dtype=torch.int32, device=device)
        self.sorted_pairs = torch.empty((P,), dtype=torch.int32, device=device)
        self.pair_pos = torch.empty((P,), dtype=torch.int32, device=device)
        self.c = _lib.Routing(self.ids.data_ptr(), self.gates.data_ptr(), self.offsets.data_ptr(),
                              self.sorted_pairs.data_ptr(), self.pair_pos.data_ptr())
        n = ctypes.c_size_t(0)
        check(lib().moeq_route_workspace_size(T, E, k, ctypes.byref(n)), "moeq_route_workspace_size")
        self.ws = torch.empty((max(1, n.value),), dtype=torch.uint8, device=device)
        self.ws_bytes = n.value


def route(logits, k, out=None):
    """Top-k routing and counting sort of fp32 logits [T, E] (see moeq_route)."""
    T, E = logits.shape
    _need(logits, torch.float32, (T, E), "logits")
    if out is None:
        out = RoutingOut(T, E, k, logits.device)
    check(lib().moeq_route(_ptr(logits), T, E, k, ctypes.byref(out.c), _ptr(out.ws), out.ws_bytes, _stream()),
          "moeq_route")
    return out


def route_mass(routing, edges=()):
    """Per-expert routing mass and (with edges) bucket index (see moeq_route_mass)."""
    E = routing.E
    mass = torch.empty((E,), dtype=torch.float32, device=routing.ids.device)
    bucket = torch.empty((E,), dtype=torch.int32, device=routing.ids.device) if len(edges) else None
    ed = (ctypes.c_float * max(1, len(edges)))(*[float(v) for v in edges])
    check(lib().moeq_route_mass(ctypes.byref(routing.c), routing.T, E, routing.k,
                                ctypes.cast(ed, c_void_p) if len(edges) else None, len(edges),
                                _ptr(mass), _ptr(bucket), _stream()), "moeq_route_mass")
    return mass, bucket


def plan_reductions(q, bytes_tbl, g, mu, eta, eps, target):
    """Greedy bit-plane release plan (see moeq_plan_reductions); host arrays.
    Returns (planned q, block of each action in order, released bytes, damage)."""
    q = np.ascontiguousarray(q, dtype=np.int32).copy()
    n = q.shape[0]
    bt = np.ascontiguousarray(bytes_tbl, dtype=np.float64).reshape(n, 3)
    gg = np.ascontiguousarray(g, dtype=np.float64).reshape(n, 3)
    mu = np.ascontiguousarray(mu, dtype=np.float64).reshape(n)
    eta = np.ascontiguousarray(eta, dtype=np.float64).reshape(n)
    cap = int(2 * n) + 1
    order = np.zeros(cap, dtype=np.int32)
    rel, dmg, na = ctypes.c_double(0), ctypes.c_double(0), ctypes.c_int32(0)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    check(lib().moeq_plan_reductions(n, q.ctypes.data_as(ip), bt.ctypes.data_as(dp), gg.ctypes.data_as(dp),
                                     mu.ctypes.data_as(dp), eta.ctypes.data_as(dp), float(eps), float(target),
                                     order.ctypes.data_as(ip), cap, ctypes.byref(rel), ctypes.byref(dmg),
                                     ctypes.byref(na)), "moeq_plan_reductions")
    return q, order[:na.value].tolist(), rel.value, dmg.value


# ------------------------------------------------------------ expert FFN

class FfnWorkspace:
    """Workspace of moeq_expert_ffn, or (forward=True) of moeq_moe_forward."""

    def __init__(self, layer, T, k, path=0, split_k=0, forward=False):
        self.opts = _lib.FfnOptions(path, split_k)
        n = ctypes.c_size_t(0)
        size_fn = lib().moeq_forward_workspace_size if forward else lib().moeq_ffn_workspace_size
        check(size_fn(layer.handle, T, k, ctypes.byref(self.opts), ctypes.byref(n)), "workspace_size")
        self.nbytes = n.value
        self.buf = torch.empty(max(256, n.value), dtype=torch.uint8, device=layer.buf.device)


def expert_ffn(layer, x, routing, n_comp, out=None, out_dtype=torch.float16, ws=None, path=0,
               split_k=0):
    """Routed expert FFN y [T, H] (see moeq_expert_ffn)."""
    T = routing.T
    k = routing.k
    _need(x, torch.float16, (T, layer.H), "x")
    if out is None:
        out = torch.empty((T, layer.H), dtype=out_dtype, device=x.device)
    ydt = _lib.F32 if out.dtype == torch.float32 else _lib.F16
    _need(out, out.dtype, (T, layer.H), "out")
    if ws is None:
        ws = FfnWorkspace(layer, T, k, path, split_k)
    check(lib().moeq_expert_ffn(layer.handle, _ptr(x), T, k, ctypes.byref(routing.c), n_comp,
                                _ptr(out), ydt, _ptr(ws.buf), ws.buf.numel(), ctypes.byref(ws.opts),
                                _stream()), "moeq_expert_ffn")
    return out


def moe_forward(layer, logits, x, k, n_comp, routing=None, out=None, out_dtype=torch.float16, ws=None,
                path=0, split_k=0):
    """Routing and the expert FFN in one call (see moeq_moe_forward).
    Returns (y [T, H], routing)."""
    T, E = logits.shape
    _need(logits, torch.float32, (T, E), "logits")
    _need(x, torch.float16, (T, layer.H), "x")
    if routing is None:
        routing = RoutingOut(T, E, k, x.device)
    if out is None:
        out = torch.empty((T, layer.H), dtype=out_dtype, device=x.device)
    ydt = _lib.F32 if out.dtype == torch.float32 else _lib.F16
    _need(out, out.dtype, (T, layer.H), "out")
    if ws is None:
        ws = FfnWorkspace(layer, T, k, path, split_k, forward=True)
    check(lib().moeq_moe_forward(layer.handle, _ptr(logits), _ptr(x), T, k, n_comp, ctypes.byref(routing.c),
                                 _ptr(out), ydt, _ptr(ws.buf), ws.buf.numel(), ctypes.byref(ws.opts), _stream()),
          "moeq_moe_forward")
    return out, routing


# ------------------------------------------------------------ profiling

def profile_enable(on=True):
    check(lib().moeq_profile_enable(1 if on else 0), "moeq_profile_enable")


def profile_read(max_kernels=64):
    names = (ctypes.c_char_p * max_kernels)()
    launches = (ctypes.c_int32 * max_kernels)()
    ms = (ctypes.c_double * max_kernels)()
    n = ctypes.c_int32(0)
    check(lib().moeq_profile_read(max_kernels, names, launches, ms, ctypes.byref(n)), "moeq_profile_read")
    return {names[i].decode(): (int(launches[i]), float(ms[i])) for i in range(min(n.value, max_kernels))}
