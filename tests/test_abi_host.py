"""The C ABI on the host, without a GPU: the library loads, exports every
function include/sffn.h declares, and rejects bad arguments before any HIP call."""
import os
import re

import pytest

from activation_sparse_gated_amd import sffn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "sffn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sffn_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("sffn_create", "sffn_destroy", "sffn_forward_dense", "sffn_forward_sparse",
              "sffn_forward_lopa", "sffn_last_error"):
        assert n in names


def test_library_exports_every_declared_function():
    lib = sffn.load()
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) == set(sffn.EXPORTED)
    assert sffn.sffn_abi_version() == 1


@pytest.mark.parametrize("args,status,needle", [
    ((7, 64, 0, 1, 0, 0), sffn.SFFN_INVALID_ARGUMENT, "multiple of 8"),
    ((0, 64, 0, 1, 0, 0), sffn.SFFN_INVALID_ARGUMENT, "multiple of 8"),
    ((8200, 64, 0, 1, 0, 0), sffn.SFFN_INVALID_ARGUMENT, "at most"),
    ((4104, 64, 0, 1, 0, 1), sffn.SFFN_INVALID_ARGUMENT, "at most 4096"),
    ((64, 0, 0, 1, 0, 0), sffn.SFFN_INVALID_ARGUMENT, "H must"),
    ((64, 64, 12, 1, 0, 0), sffn.SFFN_INVALID_ARGUMENT, "r must"),
    ((64, 64, 4096, 1, 0, 0), sffn.SFFN_INVALID_ARGUMENT, "r must"),
    ((64, 64, 0, 0, 0, 0), sffn.SFFN_INVALID_ARGUMENT, "max_tokens"),
    ((64, 64, 0, 65, 0, 1), sffn.SFFN_INVALID_ARGUMENT, "max_tokens"),
    ((64, 64, 8, 65, 0, 0), sffn.SFFN_INVALID_ARGUMENT, "max_tokens"),
    ((64, 64, 0, 8193, 0, 0), sffn.SFFN_INVALID_ARGUMENT, "max_tokens"),
    ((64, 64, 0, 1, 2, 0), sffn.SFFN_UNSUPPORTED, "activation"),
    ((64, 64, 0, 1, 0, 4), sffn.SFFN_UNSUPPORTED, "dtype"),
])
def test_create_rejects_bad_arguments(args, status, needle):
    st, h = sffn.sffn_create_status(*args)
    assert st == status and h is None
    assert needle in sffn.sffn_last_error(None)


def test_create_int8_checks():
    # int8 weights: D and (LoPA) r multiples of 16
    st, h = sffn.sffn_create_status(264, 64, 0, 1, 0, sffn.SFFN_I8, 0)
    assert st == sffn.SFFN_INVALID_ARGUMENT and h is None and "16" in sffn.sffn_last_error(None)
    st, h = sffn.sffn_create_status(256, 64, 24, 1, 0, sffn.SFFN_I8, 0)
    assert st == sffn.SFFN_INVALID_ARGUMENT and h is None and "r must" in sffn.sffn_last_error(None)


def test_create_int4_checks():
    # int4 weights: D a multiple of 128; LoPA ranks a multiple of 16 (int8 U rows)
    st, h = sffn.sffn_create_status(192, 64, 0, 1, 0, sffn.SFFN_I4, 0)
    assert st == sffn.SFFN_INVALID_ARGUMENT and h is None and "128" in sffn.sffn_last_error(None)
    st, h = sffn.sffn_create_status(256, 64, 24, 1, 0, sffn.SFFN_I4, 0)
    assert st == sffn.SFFN_INVALID_ARGUMENT and h is None and "r must" in sffn.sffn_last_error(None)


def test_create_rejects_flags():
    # gate flags on a standard handle
    st, h = sffn.sffn_create_status(64, 64, 0, 1, 0, 0, sffn.SFFN_FLAG_G_TILED)
    assert st == sffn.SFFN_UNSUPPORTED and h is None and "flags" in sffn.sffn_last_error(None)
    # bits outside the three gate options, on a LoPA handle
    st, h = sffn.sffn_create_status(64, 64, 8, 1, 0, 0, 8)
    assert st == sffn.SFFN_UNSUPPORTED and h is None and "flag" in sffn.sffn_last_error(None)


def test_forward_with_null_handle():
    lib = sffn.load()
    assert lib.sffn_forward_sparse(None, None, None, None, None, None, 1, 0, None, None, None) \
        == sffn.SFFN_INVALID_ARGUMENT
    assert lib.sffn_forward_dense(None, None, None, None, None, None, 1, None) \
        == sffn.SFFN_INVALID_ARGUMENT
    assert lib.sffn_forward_lopa(None, None, None, None, None, None, None, 1, 0, None, None,
                                 None) == sffn.SFFN_INVALID_ARGUMENT
    assert "null handle" in sffn.sffn_last_error(None)


def test_status_strings_and_kernel_names():
    assert sffn.status_string(sffn.SFFN_OK) == "SFFN_OK"
    assert sffn.status_string(-99) == "unknown status"
    names = [sffn.sffn_kernel_name(k) for k in range(sffn.sffn_kernel_kinds())]
    assert "k_gate_up_sparse" in names and "k_down" in names
    assert sffn.sffn_kernel_name(99) == "unknown"
