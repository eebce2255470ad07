"""Host-side checks of the C ABI: the library loads, exports every function
include/shampoo.h declares, and rejects bad arguments before touching the GPU.
No compute call is made here (no GPU in this environment)."""
import ctypes
import os

import pytest

from blocked_shampoo_preconditioning_amd import shampoo as S


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(S.LIB_PATH):
        from blocked_shampoo_preconditioning_amd import build
        build.build()
    return S.load_library()


def test_exports_every_declared_function(lib):
    names = S.header_functions()
    assert len(names) >= 17
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(S._SIGNATURES), "binding and header disagree"


def test_config_default(lib):
    c = S.shampoo_config_default()
    assert (c.block_rows, c.block_cols) == (1024, 1024)
    assert c.beta2 == pytest.approx(0.999) and c.eps == pytest.approx(1e-6)
    assert c.lr == pytest.approx(1e-3) and c.root_every == 10 and c.stat_scale < 0
    assert c.newton_max_iters == 25 and c.newton_scale_mode == 3 and c.momentum == 0.0
    assert c.root_method == 0 and c.cheb_degree == 128
    assert c.fp32_gemm == 2  # fp32 products as two scaled fp16 terms on the fp16 MFMA
    assert lib.shampoo_config_default(None) == S.SHAMPOO_ERR_INVALID_ARG


def _ws(cfg, shapes, lds=None):
    d = S.make_descs(shapes, lds)
    out = ctypes.c_size_t(0)
    code = S.load_library().shampoo_workspace_size(ctypes.byref(cfg), d, len(shapes), ctypes.byref(out))
    return code, out.value


def test_workspace_size_grows_with_blocks(lib):
    c = S.shampoo_config_default()
    c.block_rows = c.block_cols = 256
    code1, b1 = _ws(c, [(256, 256)])
    code2, b2 = _ws(c, [(256, 512)])
    code3, b3 = _ws(c, [(300, 257)])  # 2 x 2 blocks with tails
    assert code1 == code2 == code3 == S.SHAMPOO_OK
    one = 256 * 256 * 4
    # packed gradient + statistics, roots, alternate roots and three scratch sets
    assert b1 >= one + 6 * 2 * one
    assert b2 >= 2 * b1 - 4096 * 4 and b3 >= 4 * b1 - 4096 * 16
    code0, b0 = _ws(c, [])
    assert code0 == S.SHAMPOO_OK and 0 < b0 < 1 << 16
    code_e, be = _ws(c, [(0, 5), (7, 0)], [8, 4])
    assert code_e == S.SHAMPOO_OK and be < 1 << 16


@pytest.mark.parametrize("field,value,code", [
    ("block_rows", 48, S.SHAMPOO_ERR_UNSUPPORTED),
    ("block_cols", 0, S.SHAMPOO_ERR_INVALID_ARG),
    ("block_rows", 8192, S.SHAMPOO_ERR_INVALID_ARG),
    ("eps", 0.0, S.SHAMPOO_ERR_INVALID_ARG),
    ("eps", float("nan"), S.SHAMPOO_ERR_INVALID_ARG),
    ("beta2", 1.5, S.SHAMPOO_ERR_INVALID_ARG),
    ("lr", float("inf"), S.SHAMPOO_ERR_INVALID_ARG),
    ("root_every", -1, S.SHAMPOO_ERR_INVALID_ARG),
    ("newton_max_iters", 0, S.SHAMPOO_ERR_INVALID_ARG),
    ("newton_max_iters", 65, S.SHAMPOO_ERR_INVALID_ARG),
    ("newton_scale_mode", 4, S.SHAMPOO_ERR_UNSUPPORTED),
    ("param_dtype", 7, S.SHAMPOO_ERR_UNSUPPORTED),
    ("momentum", 1.0, S.SHAMPOO_ERR_INVALID_ARG),
    ("root_method", 3, S.SHAMPOO_ERR_UNSUPPORTED),
    ("momentum", -0.1, S.SHAMPOO_ERR_INVALID_ARG),
    ("fp32_gemm", 3, S.SHAMPOO_ERR_INVALID_ARG),
    ("fp32_gemm", -1, S.SHAMPOO_ERR_INVALID_ARG),
])
def test_config_validation(lib, field, value, code):
    c = S.shampoo_config_default()
    setattr(c, field, value)
    got, _ = _ws(c, [(64, 64)])
    assert got == code
    assert lib.shampoo_last_error().decode()


@pytest.mark.parametrize("shape,ld,code", [
    ((64, 64), 60, S.SHAMPOO_ERR_INVALID_ARG),
    ((64, 62), 62, S.SHAMPOO_OK),
    ((-1, 4), 4, S.SHAMPOO_ERR_INVALID_ARG),
    ((64, 64), 1 << 26, S.SHAMPOO_OK),              # the largest leading dimension
    ((64, 64), (1 << 26) + 1, S.SHAMPOO_ERR_INVALID_ARG),
])
def test_matrix_validation(lib, shape, ld, code):
    c = S.shampoo_config_default()
    got, _ = _ws(c, [shape], [ld])
    assert got == code


def test_init_rejects_bad_workspace_without_gpu_work(lib):
    c = S.shampoo_config_default()
    c.block_rows = c.block_cols = 64
    d = S.make_descs([(64, 64)])
    code, need = _ws(c, [(64, 64)])
    h = ctypes.c_void_p()
    init = lib.shampoo_init
    assert init(ctypes.byref(c), d, 1, None, need, None, ctypes.byref(h)) == S.SHAMPOO_ERR_INVALID_ARG
    assert init(ctypes.byref(c), d, 1, ctypes.c_void_p(0x1000010), need, None,
                ctypes.byref(h)) == S.SHAMPOO_ERR_MISALIGNED
    assert init(ctypes.byref(c), d, 1, ctypes.c_void_p(0x1000000), need - 1, None,
                ctypes.byref(h)) == S.SHAMPOO_ERR_WORKSPACE_TOO_SMALL
    assert "needs" in lib.shampoo_last_error().decode()
    assert init(ctypes.byref(c), d, 1, ctypes.c_void_p(0x1000000), need, None, None) == \
        S.SHAMPOO_ERR_INVALID_ARG


def test_null_handle_everywhere(lib):
    E = S.SHAMPOO_ERR_INVALID_ARG
    assert lib.shampoo_step(None, None, None, 0, None) == E
    assert lib.shampoo_refresh_roots(None, None) == E
    assert lib.shampoo_destroy(None) == E
    assert lib.shampoo_state_layout(None, None) == E
    assert lib.shampoo_get_step(None, None) == E
    assert lib.shampoo_set_step(None, 3) == E
    assert lib.shampoo_restore(None, 3, None) == E
    assert lib.shampoo_pack(None, None, None) == E
    assert lib.shampoo_unpack(None, None, None) == E
    assert lib.shampoo_precondition(None, None, None) == E
    assert lib.shampoo_get_status(None, None, None) == E
    assert lib.shampoo_set_timing(None, 1, None) == E
    assert lib.shampoo_get_timing(None, None) == E


def test_status_strings(lib):
    for code in range(7):
        assert lib.shampoo_status_string(code).decode()
    assert lib.shampoo_status_string(99).decode() == "unknown status"


def test_product_path_has_no_oracle_or_fallback():
    """The binding and the library sources never reach the oracle."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    pkg = os.path.join(root, "blocked_shampoo_preconditioning_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f


# ---------------------------------------------------------------------------
# Order-k tensor handles: sizes and validation (host only)
# ---------------------------------------------------------------------------
def _tws(cfg, block_dims, shapes, strides=None):
    d = S.make_tensor_descs(shapes, strides)
    out = ctypes.c_size_t(0)
    bd = (ctypes.c_int32 * 4)(*block_dims)
    code = S.load_library().shampoo_tensor_workspace_size(ctypes.byref(cfg), len(block_dims), bd, d,
                                                          len(shapes), ctypes.byref(out))
    return code, out.value


def test_tensor_workspace_size(lib):
    c = S.shampoo_config_default()
    code, b = _tws(c, (64, 32, 3, 3), [(64, 32, 3, 3)])
    E = 64 * 32 * 9
    assert code == S.SHAMPOO_OK
    # packed gradient, two apply buffers, statistics and roots of every dimension
    assert b >= 3 * E * 4 + 2 * 4 * (64 * 64 + 32 * 32 + 9 + 9)
    code2, b2 = _tws(c, (64, 32, 3, 3), [(64, 32, 3, 3), (130, 40, 3, 3)])  # 3 x 2 more blocks
    assert code2 == S.SHAMPOO_OK and b2 >= b + 6 * 3 * E * 4 - 8192
    code3, b3 = _tws(c, (64, 32, 3, 3), [(0, 32, 3, 3)])
    assert code3 == S.SHAMPOO_OK and b3 < 1 << 16
    code4, _ = _tws(c, (3, 3), [(5, 7)])  # two small dimensions: no MFMA factor at all
    assert code4 == S.SHAMPOO_OK


@pytest.mark.parametrize("block_dims,shapes,field,value,code", [
    ((64, 16, 3), [(64, 16, 3)], None, None, S.SHAMPOO_ERR_UNSUPPORTED),   # 16: neither small nor x32
    ((64, 32, 3, 3, 1), [(64, 32, 3, 3, 1)], None, None, S.SHAMPOO_ERR_UNSUPPORTED),  # order 5
    ((64,), [(64,)], None, None, S.SHAMPOO_ERR_UNSUPPORTED),               # order 1
    ((64, 32, 3), [(64, 32)], None, None, S.SHAMPOO_ERR_INVALID_ARG),      # order mismatch
    ((64, 32, 3), [(64, 32, 3)], "root_method", 1, S.SHAMPOO_ERR_UNSUPPORTED),  # DB needs k = 2
    ((64, 32, 3), [(64, 32, 3)], "eps", 0.0, S.SHAMPOO_ERR_INVALID_ARG),
    ((4096, 4096, 128), [(4096, 4096, 128)], None, None, S.SHAMPOO_ERR_UNSUPPORTED),  # 2^31 per block
])
def test_tensor_validation(lib, block_dims, shapes, field, value, code):
    c = S.shampoo_config_default()
    if field:
        setattr(c, field, value)
    k = len(block_dims)
    if k > 4 or len(shapes[0]) > 4:
        # more than SHAMPOO_MAX_ORDER dimensions cannot be described; the order
        # argument alone is rejected
        d = S.make_tensor_descs([s[:4] for s in shapes])
        out = ctypes.c_size_t(0)
        bd = (ctypes.c_int32 * 5)(*block_dims)
        got = lib.shampoo_tensor_workspace_size(ctypes.byref(c), k, ctypes.cast(bd, ctypes.POINTER(ctypes.c_int32)),
                                                d, 1, ctypes.byref(out))
    else:
        got, _ = _tws(c, block_dims, shapes)
    assert got == code


def test_tensor_bad_strides(lib):
    c = S.shampoo_config_default()
    code, _ = _tws(c, (32, 3), [(40, 3)], strides=[(3, 0)])
    assert code == S.SHAMPOO_ERR_INVALID_ARG


def test_tensor_matrix_handle_info_rejected(lib):
    out = S.TensorInfo()
    assert lib.shampoo_tensor_info(None, ctypes.byref(out)) == S.SHAMPOO_ERR_INVALID_ARG
