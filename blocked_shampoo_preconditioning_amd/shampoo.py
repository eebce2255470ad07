"""ctypes binding of libshampoo_mi355x.so (the C ABI in include/shampoo.h).

The functions keep the C names and only marshal arguments: every step of the
method runs in the HIP library. PyTorch provides device memory (the
workspace, parameters and gradients) and the stream. A missing library is an
error; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libshampoo_mi355x.so")
HEADER_PATH = os.path.join(os.path.dirname(HERE), "include", "shampoo.h")

SHAMPOO_OK = 0
SHAMPOO_ERR_INVALID_ARG = 1
SHAMPOO_ERR_UNSUPPORTED = 2
SHAMPOO_ERR_WORKSPACE_TOO_SMALL = 3
SHAMPOO_ERR_MISALIGNED = 4
SHAMPOO_ERR_NO_ROOTS = 5
SHAMPOO_ERR_HIP = 6
SHAMPOO_F32 = 0
SHAMPOO_BF16 = 1
SHAMPOO_FORCE_REFRESH = 1
SHAMPOO_NO_AUTO_REFRESH = 2
TIMING_CLASSES = ("pack", "stats", "norms", "newton_gemm", "newton_aux", "apply", "stats_aux",
                  "apply_aux")
ROOT_METHODS = {"newton": 0, "newton_db": 1, "chebyshev": 2}
# shampoo_fp32_gemm_t: fp32 MFMA, fp32 operands split into three bf16 terms,
# or scaled and split into two fp16 terms
GEMM_MODES = {"f32": 0, "split": 1, "split16": 2}


class MatrixDesc(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("ld", ctypes.c_int64)]


class Config(ctypes.Structure):
    _fields_ = [("block_rows", ctypes.c_int32), ("block_cols", ctypes.c_int32),
                ("beta2", ctypes.c_double), ("stat_scale", ctypes.c_double),
                ("eps", ctypes.c_double), ("lr", ctypes.c_double),
                ("root_every", ctypes.c_int32), ("newton_max_iters", ctypes.c_int32),
                ("newton_tol", ctypes.c_double), ("newton_scale_mode", ctypes.c_int32),
                ("param_dtype", ctypes.c_int32), ("grad_dtype", ctypes.c_int32),
                ("momentum", ctypes.c_double), ("root_method", ctypes.c_int32),
                ("cheb_degree", ctypes.c_int32), ("fp32_gemm", ctypes.c_int32)]


class Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("n_blocks", "grad_packed", "stats", "roots",
                                              "newton_status", "newton_iters", "newton_scale",
                                              "newton_residual", "momentum", "workspace_bytes",
                                              "root_maxima")]


class Timing(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double * 8), ("flops", ctypes.c_double * 8),
                ("bytes", ctypes.c_double * 8), ("launches", ctypes.c_int64 * 8)]


MAX_ORDER = 4


class TensorDesc(ctypes.Structure):
    _fields_ = [("order", ctypes.c_int32), ("dims", ctypes.c_int64 * MAX_ORDER),
                ("strides", ctypes.c_int64 * MAX_ORDER)]


class TensorInfo(ctypes.Structure):
    _fields_ = [("order", ctypes.c_int32), ("block_dims", ctypes.c_int32 * MAX_ORDER),
                ("n_blocks", ctypes.c_int64), ("block_elems", ctypes.c_int64),
                ("stats", ctypes.c_int64 * MAX_ORDER), ("roots", ctypes.c_int64 * MAX_ORDER),
                ("factor_group", ctypes.c_int32 * MAX_ORDER)]


class ShampooError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"shampoo error {code}: {message}")
        self.code = code


_lib = None

_P = ctypes.c_void_p
_PP = ctypes.POINTER(ctypes.c_void_p)
_SIGNATURES = {
    "shampoo_config_default": [ctypes.POINTER(Config)],
    "shampoo_workspace_size": [ctypes.POINTER(Config), ctypes.POINTER(MatrixDesc), ctypes.c_int32,
                               ctypes.POINTER(ctypes.c_size_t)],
    "shampoo_init": [ctypes.POINTER(Config), ctypes.POINTER(MatrixDesc), ctypes.c_int32, _P,
                     ctypes.c_size_t, _P, ctypes.POINTER(_P)],
    "shampoo_step": [_P, _PP, _PP, ctypes.c_uint32, _P],
    "shampoo_refresh_roots": [_P, _P],
    "shampoo_destroy": [_P],
    "shampoo_state_layout": [_P, ctypes.POINTER(Layout)],
    "shampoo_get_step": [_P, ctypes.POINTER(ctypes.c_int64)],
    "shampoo_set_step": [_P, ctypes.c_int64],
    "shampoo_restore": [_P, ctypes.c_int64, ctypes.c_void_p],
    "shampoo_pack": [_P, _PP, _P],
    "shampoo_unpack": [_P, _PP, _P],
    "shampoo_precondition": [_P, _P, _P],
    "shampoo_precondition_noalloc": [_P, _P, _P],
    "shampoo_get_status": [_P, _P, ctypes.POINTER(ctypes.c_int32)],
    "shampoo_set_timing": [_P, ctypes.c_int32, _P],
    "shampoo_get_timing": [_P, ctypes.POINTER(Timing)],
    "shampoo_status_string": [ctypes.c_int],
    "shampoo_last_error": [],
    "shampoo_tensor_workspace_size": [ctypes.POINTER(Config), ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(TensorDesc),
                                      ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)],
    "shampoo_tensor_init": [ctypes.POINTER(Config), ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                            ctypes.POINTER(TensorDesc), ctypes.c_int32, _P, ctypes.c_size_t, _P,
                            ctypes.POINTER(_P)],
    "shampoo_tensor_info": [_P, ctypes.POINTER(TensorInfo)],
}


def load_library(path=None):
    """Load the HIP library (once). Raises if it has not been built.

    torch is imported first when it is installed: PyTorch-ROCm brings its own
    HIP runtime, and the library must bind to that one; a second runtime
    loaded next to it does not see the device.
    """
    global _lib
    if _lib is not None:
        return _lib
    path = LIB_PATH if path is None else path
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          f"`python -m blocked_shampoo_preconditioning_amd.build`")
    lib = ctypes.CDLL(path)
    for name, argtypes in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_char_p if name in ("shampoo_status_string", "shampoo_last_error") \
            else ctypes.c_int
    _lib = lib
    return lib


def header_functions(path=HEADER_PATH):
    """Names of the functions include/shampoo.h declares."""
    text = open(path).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(shampoo_\w+)\s*\(", text, re.M)))


def _check(code):
    if code != SHAMPOO_OK:
        lib = load_library()
        raise ShampooError(code, lib.shampoo_last_error().decode())


def _ptr_array(ptrs):
    arr = (ctypes.c_void_p * max(1, len(ptrs)))(*[ctypes.c_void_p(p) for p in ptrs])
    return ctypes.cast(arr, _PP), arr


# ---------------------------------------------------------------------------
# Functions with the C names (argument marshalling only)
# ---------------------------------------------------------------------------
def shampoo_config_default():
    cfg = Config()
    _check(load_library().shampoo_config_default(ctypes.byref(cfg)))
    return cfg


def make_descs(shapes, lds=None):
    descs = (MatrixDesc * max(1, len(shapes)))()
    for i, (r, c) in enumerate(shapes):
        descs[i] = MatrixDesc(r, c, c if lds is None else lds[i])
    return descs


def shampoo_workspace_size(cfg, descs, n_mats):
    out = ctypes.c_size_t(0)
    _check(load_library().shampoo_workspace_size(ctypes.byref(cfg), descs, n_mats, ctypes.byref(out)))
    return out.value


def shampoo_init(cfg, descs, n_mats, workspace_ptr, workspace_bytes, stream):
    h = ctypes.c_void_p()
    _check(load_library().shampoo_init(ctypes.byref(cfg), descs, n_mats, ctypes.c_void_p(workspace_ptr),
                                       workspace_bytes, ctypes.c_void_p(stream), ctypes.byref(h)))
    return h


def shampoo_step(h, param_ptrs, grad_ptrs, flags, stream):
    p, _pk = _ptr_array(param_ptrs)
    g, _gk = _ptr_array(grad_ptrs)
    _check(load_library().shampoo_step(h, p, g, flags, ctypes.c_void_p(stream)))


def shampoo_refresh_roots(h, stream):
    _check(load_library().shampoo_refresh_roots(h, ctypes.c_void_p(stream)))


def shampoo_destroy(h):
    _check(load_library().shampoo_destroy(h))


def shampoo_state_layout(h):
    out = Layout()
    _check(load_library().shampoo_state_layout(h, ctypes.byref(out)))
    return out


def shampoo_get_step(h):
    t = ctypes.c_int64()
    _check(load_library().shampoo_get_step(h, ctypes.byref(t)))
    return t.value


def shampoo_set_step(h, t):
    _check(load_library().shampoo_set_step(h, t))


def shampoo_restore(h, t, stream=None):
    _check(load_library().shampoo_restore(h, t, stream))


def shampoo_pack(h, grad_ptrs, stream):
    g, _gk = _ptr_array(grad_ptrs)
    _check(load_library().shampoo_pack(h, g, ctypes.c_void_p(stream)))


def shampoo_unpack(h, dst_ptrs, stream):
    d, _dk = _ptr_array(dst_ptrs)
    _check(load_library().shampoo_unpack(h, d, ctypes.c_void_p(stream)))


def shampoo_precondition(h, out_ptr, stream):
    _check(load_library().shampoo_precondition(h, ctypes.c_void_p(out_ptr), ctypes.c_void_p(stream)))


def shampoo_precondition_noalloc(h, out_ptr, stream):
    _check(load_library().shampoo_precondition_noalloc(h, ctypes.c_void_p(out_ptr),
                                                       ctypes.c_void_p(stream)))


def shampoo_get_status(h, stream):
    n = ctypes.c_int32()
    _check(load_library().shampoo_get_status(h, ctypes.c_void_p(stream), ctypes.byref(n)))
    return n.value


def shampoo_set_timing(h, enable, stream):
    _check(load_library().shampoo_set_timing(h, int(enable), ctypes.c_void_p(stream)))


def shampoo_get_timing(h):
    t = Timing()
    _check(load_library().shampoo_get_timing(h, ctypes.byref(t)))
    return {name: {"ms": t.ms[i], "flops": t.flops[i], "bytes": t.bytes[i],
                   "launches": t.launches[i]} for i, name in enumerate(TIMING_CLASSES)}


def make_tensor_descs(shapes, strides=None):
    """Descriptors of tensors (row-major contiguous unless strides are given)."""
    descs = (TensorDesc * max(1, len(shapes)))()
    for i, shape in enumerate(shapes):
        k = len(shape)
        if strides is None:
            st, acc = [0] * k, 1
            for d in range(k - 1, -1, -1):
                st[d] = acc
                acc *= max(1, shape[d])
        else:
            st = strides[i]
        descs[i].order = k
        for d in range(k):
            descs[i].dims[d] = shape[d]
            descs[i].strides[d] = st[d]
    return descs


def _block_dims(block_dims):
    arr = (ctypes.c_int32 * MAX_ORDER)(*[int(b) for b in block_dims])
    return arr


def shampoo_tensor_workspace_size(cfg, block_dims, descs, n_tensors):
    out = ctypes.c_size_t(0)
    _check(load_library().shampoo_tensor_workspace_size(
        ctypes.byref(cfg), len(block_dims), _block_dims(block_dims), descs, n_tensors,
        ctypes.byref(out)))
    return out.value


def shampoo_tensor_init(cfg, block_dims, descs, n_tensors, workspace_ptr, workspace_bytes, stream):
    h = ctypes.c_void_p()
    _check(load_library().shampoo_tensor_init(
        ctypes.byref(cfg), len(block_dims), _block_dims(block_dims), descs, n_tensors,
        ctypes.c_void_p(workspace_ptr), workspace_bytes, ctypes.c_void_p(stream), ctypes.byref(h)))
    return h


def shampoo_tensor_info(h):
    out = TensorInfo()
    _check(load_library().shampoo_tensor_info(h, ctypes.byref(out)))
    return out


# ---------------------------------------------------------------------------
# Convenience wrapper over torch tensors
# ---------------------------------------------------------------------------
class Shampoo:
    """Blocked Shampoo over a list of 2-D CUDA tensors (parameters).

    The workspace is one uint8 tensor allocated here with torch; the library
    keeps all state in it. Every call runs on torch's current stream.
    """

    def __init__(self, shapes, block_rows=1024, block_cols=1024, beta2=0.999, eps=1e-6, lr=1e-3,
                 root_every=10, stat_scale=None, newton_max_iters=25, newton_tol=1e-6,
                 newton_scale_mode=3, dtype="f32", device="cuda", lds=None, momentum=0.0,
                 root_method="newton", cheb_degree=128, fp32_gemm="split16"):
        import torch
        self.torch = torch
        self.shapes = [tuple(int(v) for v in s) for s in shapes]
        self.lds = [c for (_, c) in self.shapes] if lds is None else list(lds)
        cfg = shampoo_config_default()
        cfg.block_rows, cfg.block_cols = block_rows, block_cols
        cfg.beta2, cfg.eps, cfg.lr = beta2, eps, lr
        cfg.stat_scale = -1.0 if stat_scale is None else stat_scale
        cfg.root_every = root_every
        cfg.newton_max_iters, cfg.newton_tol = newton_max_iters, newton_tol
        cfg.newton_scale_mode = newton_scale_mode
        cfg.momentum = momentum
        cfg.root_method = ROOT_METHODS[root_method]
        cfg.cheb_degree = cheb_degree
        cfg.fp32_gemm = GEMM_MODES[fp32_gemm]
        dt = {"f32": SHAMPOO_F32, "bf16": SHAMPOO_BF16}[dtype]
        cfg.param_dtype = cfg.grad_dtype = dt
        self.cfg = cfg
        self.descs = make_descs(self.shapes, self.lds)
        self.n = len(self.shapes)
        nbytes = shampoo_workspace_size(cfg, self.descs, self.n)
        self.workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        base = self.workspace.data_ptr()
        self._ws_ptr = (base + 255) // 256 * 256
        self._ws_off = self._ws_ptr - base
        self.handle = shampoo_init(cfg, self.descs, self.n, self._ws_ptr, nbytes, self._stream())
        self.layout = shampoo_state_layout(self.handle)

    def _stream(self):
        return self.torch.cuda.current_stream().cuda_stream

    def close(self):
        if self.handle is not None:
            self.torch.cuda.current_stream().synchronize()
            shampoo_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def step(self, params, grads, flags=0):
        shampoo_step(self.handle, [p.data_ptr() for p in params], [g.data_ptr() for g in grads],
                     flags, self._stream())

    def refresh_roots(self):
        shampoo_refresh_roots(self.handle, self._stream())

    def pack(self, grads):
        shampoo_pack(self.handle, [g.data_ptr() for g in grads], self._stream())

    def unpack(self, dsts):
        shampoo_unpack(self.handle, [d.data_ptr() for d in dsts], self._stream())

    def precondition(self, out):
        shampoo_precondition(self.handle, out.data_ptr(), self._stream())

    def precondition_noalloc(self, out):
        shampoo_precondition_noalloc(self.handle, out.data_ptr(), self._stream())

    def n_diverged(self):
        return shampoo_get_status(self.handle, self._stream())

    def set_timing(self, enable):
        shampoo_set_timing(self.handle, enable, self._stream())

    def timing(self):
        return shampoo_get_timing(self.handle)

    @property
    def t(self):
        return shampoo_get_step(self.handle)

    # --- views of the state inside the workspace (no copies) ---
    def _view(self, off, count, dtype):
        torch = self.torch
        esz = torch.tensor([], dtype=dtype).element_size()
        start = self._ws_off + off
        return self.workspace[start:start + count * esz].view(dtype)

    @property
    def n_blocks(self):
        return int(self.layout.n_blocks)

    def grad_packed(self):
        B, br, bc = self.n_blocks, self.cfg.block_rows, self.cfg.block_cols
        return self._view(self.layout.grad_packed, B * br * bc, self.torch.float32).view(B, br, bc)

    def _factors(self, off):
        B, br, bc = self.n_blocks, self.cfg.block_rows, self.cfg.block_cols
        flat = self._view(off, B * (br * br + bc * bc), self.torch.float32)
        return flat[:B * br * br].view(B, br, br), flat[B * br * br:].view(B, bc, bc)

    def stats(self):
        return self._factors(self.layout.stats)

    def momentum_buffer(self):
        if self.layout.momentum < 0:
            return None
        B, br, bc = self.n_blocks, self.cfg.block_rows, self.cfg.block_cols
        return self._view(self.layout.momentum, B * br * bc, self.torch.float32).view(B, br, bc)

    def roots(self):
        return self._factors(self.layout.roots)

    def root_maxima(self):
        """Versioned exponent words of the roots (fp16 split products only)."""
        if self.layout.root_maxima < 0:
            return None
        return self._view(self.layout.root_maxima, 2 * self.n_blocks, self.torch.int64)

    def newton_info(self):
        B = self.n_blocks
        st = self._view(self.layout.newton_status, 2 * B, self.torch.int32)
        it = self._view(self.layout.newton_iters, 2 * B, self.torch.int32)
        sc = self._view(self.layout.newton_scale, 2 * B, self.torch.float32)
        return st, it, sc

    def newton_residual(self):
        return self._view(self.layout.newton_residual, 2 * self.n_blocks, self.torch.float32)


class TensorShampoo(Shampoo):
    """Order-k tensor Shampoo over a list of CUDA tensors of one order k
    (contiguous unless strides are given): one statistic per dimension, cut
    into blocks of block_dims. Same calls as Shampoo; state views per
    dimension."""

    def __init__(self, shapes, block_dims, beta2=0.999, eps=1e-6, lr=1e-3, root_every=10,
                 stat_scale=None, newton_max_iters=25, newton_tol=1e-6, newton_scale_mode=3,
                 dtype="f32", device="cuda", strides=None, momentum=0.0, root_method="newton",
                 cheb_degree=128, fp32_gemm="split16"):
        import torch
        self.torch = torch
        self.shapes = [tuple(int(v) for v in s) for s in shapes]
        self.block_dims = tuple(int(b) for b in block_dims)
        cfg = shampoo_config_default()
        cfg.beta2, cfg.eps, cfg.lr = beta2, eps, lr
        cfg.stat_scale = -1.0 if stat_scale is None else stat_scale
        cfg.root_every = root_every
        cfg.newton_max_iters, cfg.newton_tol = newton_max_iters, newton_tol
        cfg.newton_scale_mode = newton_scale_mode
        cfg.momentum = momentum
        cfg.root_method = ROOT_METHODS[root_method]
        cfg.cheb_degree = cheb_degree
        cfg.fp32_gemm = GEMM_MODES[fp32_gemm]
        dt = {"f32": SHAMPOO_F32, "bf16": SHAMPOO_BF16}[dtype]
        cfg.param_dtype = cfg.grad_dtype = dt
        self.cfg = cfg
        self.descs = make_tensor_descs(self.shapes, strides)
        self.n = len(self.shapes)
        nbytes = shampoo_tensor_workspace_size(cfg, self.block_dims, self.descs, self.n)
        self.workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        base = self.workspace.data_ptr()
        self._ws_ptr = (base + 255) // 256 * 256
        self._ws_off = self._ws_ptr - base
        self.handle = shampoo_tensor_init(cfg, self.block_dims, self.descs, self.n, self._ws_ptr,
                                          nbytes, self._stream())
        self.layout = shampoo_state_layout(self.handle)
        self.info = shampoo_tensor_info(self.handle)

    @property
    def order(self):
        return len(self.block_dims)

    def grad_packed(self):
        B = self.n_blocks
        E = int(self.info.block_elems)
        return self._view(self.layout.grad_packed, B * E, self.torch.float32).view(B, *self.block_dims)

    def momentum_buffer(self):
        if self.layout.momentum < 0:
            return None
        B, E = self.n_blocks, int(self.info.block_elems)
        return self._view(self.layout.momentum, B * E, self.torch.float32).view(B, *self.block_dims)

    def _per_dim(self, offs):
        B = self.n_blocks
        return [self._view(offs[i], B * n * n, self.torch.float32).view(B, n, n)
                for i, n in enumerate(self.block_dims)]

    def stats(self):
        """[B, n_i, n_i] statistic of every dimension i."""
        return self._per_dim(self.info.stats)

    def roots(self):
        return self._per_dim(self.info.roots)

    def _per_factor(self, off, dtype):
        B, k = self.n_blocks, self.order
        flat = self._view(off, k * B, dtype)
        return [flat[self.info.factor_group[i] * B:(self.info.factor_group[i] + 1) * B]
                for i in range(k)]

    def newton_info(self):
        """Per dimension: (status, iterations, scale) of every block's factor."""
        st = self._per_factor(self.layout.newton_status, self.torch.int32)
        it = self._per_factor(self.layout.newton_iters, self.torch.int32)
        sc = self._per_factor(self.layout.newton_scale, self.torch.float32)
        return list(zip(st, it, sc))

    def newton_residual(self):
        return self._per_factor(self.layout.newton_residual, self.torch.float32)

    def root_maxima(self):
        """Versioned exponent words of the large dimensions' roots (fp16 split
        products only), nb * B of them, the dimensions in order."""
        if self.layout.root_maxima < 0:
            return None
        nb = sum(1 for n in self.block_dims if n % 32 == 0 and 32 <= n <= 4096)
        return self._view(self.layout.root_maxima, nb * self.n_blocks, self.torch.int64)

    def state_regions(self):
        """Flat views of the checkpointed state: statistics, roots, momentum,
        the four Newton records and the root maxima (when present)."""
        t = self.torch
        kB = self.order * self.n_blocks
        out = self.stats() + self.roots()
        if self.momentum_buffer() is not None:
            out.append(self.momentum_buffer())
        out += [self._view(self.layout.newton_status, kB, t.int32),
                self._view(self.layout.newton_iters, kB, t.int32),
                self._view(self.layout.newton_scale, kB, t.float32),
                self._view(self.layout.newton_residual, kB, t.float32)]
        if self.root_maxima() is not None:
            out.append(self.root_maxima())
        return out
