"""CPU checks of the C ABI library: it loads without a GPU, exports every
function include/bsa.h declares, fails cleanly without a device, and its host
tile-list builders agree with a brute-force reading of the mask."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")


@pytest.fixture(scope="module")
def m():
    import content_dependent_block_amd as mod
    return mod


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:bsa_status|const char\*)\s+(bsa_\w+)\(", text, re.M)))


def test_every_declared_symbol_is_exported(m):
    names = declared_functions()
    assert len(names) >= 15
    lib = ctypes.CDLL(str(m._binding._LIB_PATH))
    for name in names:
        assert hasattr(lib, name), f"{name} declared in bsa.h but not exported"
    assert set(names) == set(m.EXPORTED)


def test_status_strings_and_no_device(m):
    for s in range(6):
        assert m.bsa_status_string(s)
    assert m.bsa_status_string(99) == "unknown status"
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:
        has_gpu = False
    if has_gpu:
        pytest.skip("a GPU is visible")
    with pytest.raises(m.BsaError) as e:
        m.bsa_create(0)
    assert e.value.status == m.BSA_ERR_NO_DEVICE
    assert "no HIP device" in m.bsa_last_error(None)


def test_null_handle_is_rejected(m):
    L = m._binding._lib
    assert L.bsa_forward(None, None, None, None, None, None, 1, 1, 64, 64, 1, 64, 1, 0.1, 0,
                         None) == m.BSA_ERR_INVALID_ARG
    assert L.bsa_forward_varlen(None, None, None, None, None, None, None, None, 1, 1, 64, 1, 64, None, 1, 0.1,
                                0, None) == m.BSA_ERR_INVALID_ARG
    assert L.bsa_backward_varlen(None, None, None, None, None, None, None, None, None, None, None, None, 1, 1,
                                 64, 1, 64, 1, 0.1, 0, None) == m.BSA_ERR_INVALID_ARG
    assert L.bsa_set_option(None, 0, 1) == m.BSA_ERR_INVALID_ARG
    assert L.bsa_profile_enable(None, 1) == m.BSA_ERR_INVALID_ARG
    assert L.bsa_select_fallbacks(None, None, 0) == m.BSA_ERR_INVALID_ARG
    assert L.bsa_destroy(None) == m.BSA_OK


def _brute_tiles(mask, t=64):
    n = mask.shape[0]
    nt = -(-n // t)
    row_ptr, col, rm = [0], [], []
    for qt in range(nt):
        for kt in range(nt):
            blk = np.zeros((t, t), np.uint8)
            part = mask[qt * t:(qt + 1) * t, kt * t:(kt + 1) * t]
            blk[:part.shape[0], :part.shape[1]] = part
            if blk.any():
                col.append(kt)
                rm.append([int(sum(int(b) << c for c, b in enumerate(row))) for row in blk])
        row_ptr.append(len(col))
    return (np.array(row_ptr, np.int32), np.array(col, np.int32),
            np.array(rm, np.uint64).reshape(-1, t))


@pytest.mark.parametrize("n,density,seed", [(256, 0.0, 0), (256, 0.002, 1), (256, 0.05, 2), (256, 1.0, 3),
                                             (200, 0.05, 4), (65, 1.0, 5), (1, 1.0, 6)])
def test_tiles_from_mask_matches_brute_force(m, n, density, seed):
    """n not a multiple of 64 too: the last tile holds n mod 64 rows / keys."""
    rng = np.random.default_rng(seed)
    mask = (rng.random((n, n)) < density).astype(np.uint8)
    rp, col, rm = m.bsa_tiles_from_mask(mask)
    brp, bcol, brm = _brute_tiles(mask)
    np.testing.assert_array_equal(rp, brp)
    np.testing.assert_array_equal(col, bcol)
    np.testing.assert_array_equal(rm, brm)
    assert m.bsa_tiles_validate(rp, col, n)


def test_window_stride_builder_matches_mask(m):
    for n, w, s in [(8192, 32, 512), (1024, 8, 300), (512, 0, 64), (640, 100, 7), (1000, 32, 512),
                    (65, 3, 20), (8200, 32, 512)]:
        a = m.bsa_tiles_window_stride(n, w, s)
        b = m.bsa_tiles_from_mask(oracle.window_stride_mask(n, w, s))
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)


def test_tiles_validate_rejects_bad_lists(m):
    n = 256
    rp = np.array([0, 1, 2, 3, 4], np.int32)
    col = np.array([0, 1, 2, 3], np.int32)
    assert m.bsa_tiles_validate(rp, col, n)
    assert not m.bsa_tiles_validate(np.array([0, 2, 1, 3, 4], np.int32), col, n)   # not monotone
    assert not m.bsa_tiles_validate(rp, np.array([0, 1, 2, 4], np.int32), n)       # col out of range
    assert not m.bsa_tiles_validate(np.array([0, 1, 2, 3, 3], np.int32), col, n)   # last != nnz
    assert not m.bsa_tiles_validate(np.array([1, 1, 2, 3, 4], np.int32), col, n)   # first != 0
    # strictly increasing inside a query tile: no repeat, no descent
    assert m.bsa_tiles_validate(np.array([0, 2, 2, 2, 4], np.int32), np.array([0, 3, 1, 2], np.int32), n)
    assert not m.bsa_tiles_validate(np.array([0, 2, 2, 2, 4], np.int32), np.array([3, 0, 1, 2], np.int32), n)
    assert not m.bsa_tiles_validate(np.array([0, 2, 2, 2, 4], np.int32), np.array([1, 1, 1, 2], np.int32), n)
    # n = 200: four query tiles, key tiles 0 .. 3
    assert m.bsa_tiles_validate(rp, np.array([0, 1, 2, 3], np.int32), 200)
    assert not m.bsa_tiles_validate(np.array([0, 1, 2, 3], np.int32), col[:3], 200)  # row_ptr too short for n
    L = m._binding._lib
    assert L.bsa_tiles_validate(rp.ctypes.data, col.ctypes.data, 4, n, 32) == m.BSA_ERR_UNSUPPORTED
    assert L.bsa_tiles_validate(None, col.ctypes.data, 4, n, 64) == m.BSA_ERR_INVALID_ARG
    assert L.bsa_tiles_create(None, n, 64, rp.ctypes.data, col.ctypes.data, None, 4,
                              ctypes.byref(ctypes.c_void_p())) == m.BSA_ERR_INVALID_ARG


def test_tiles_buffer_too_small_is_an_error(m):
    L = m._binding._lib
    mask = np.ones((128, 128), np.uint8)
    rp = np.zeros(3, np.int32)
    col = np.zeros(1, np.int32)
    nnz = ctypes.c_int64(1)
    st = L.bsa_tiles_from_mask(mask.ctypes.data, 128, 64, rp.ctypes.data, col.ctypes.data, None,
                               ctypes.byref(nnz))
    assert st == m.BSA_ERR_INVALID_ARG
    nnz = ctypes.c_int64(0)
    assert L.bsa_tiles_from_mask(mask.ctypes.data, 128, 64, rp.ctypes.data, None, None,
                                 ctypes.byref(nnz)) == m.BSA_OK
    assert nnz.value == 4
    assert L.bsa_tiles_from_mask(mask.ctypes.data, 100, 64, rp.ctypes.data, None, None,
                                 ctypes.byref(nnz)) == m.BSA_OK   # n = 100: 2 x 2 tiles
    assert nnz.value == 4
    assert L.bsa_tiles_from_mask(mask.ctypes.data, 128, 32, rp.ctypes.data, None, None,
                                 ctypes.byref(nnz)) == m.BSA_ERR_UNSUPPORTED
