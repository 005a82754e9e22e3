"""CPU checks of the C ABI: the library loads, exports every function the
header declares, sizes its buffers as documented, and rejects bad arguments
before touching the GPU."""
import ctypes
import os

import pytest

LIB = os.path.join(os.path.dirname(os.path.dirname(__file__)), "sparse_kv_retrieval_dual_amd", "libdd.so")



@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):  # hipcc cross-compiles for gfx950 without a GPU
        from sparse_kv_retrieval_dual_amd import build
        build.build_library(verbose=False)
    import sparse_kv_retrieval_dual_amd as dd
    return dd.load()


def test_exports_every_declared_symbol(lib):
    from sparse_kv_retrieval_dual_amd import _lib
    names = _lib.header_symbols()
    assert len(names) >= 15
    raw = ctypes.CDLL(LIB)
    for name in names:
        assert hasattr(raw, name), name
        assert name in _lib._SIGNATURES, f"binding lacks a signature for {name}"
    assert set(_lib._SIGNATURES) == set(names)


def test_version_and_empty_error(lib):
    assert lib.dd_version() == 100
    assert isinstance(lib.dd_last_error(), bytes)


def test_buffer_sizes(lib):
    # ring: R slots x (K and V) x B*H x 2k rows x D x element size
    assert lib.dd_ring_bytes(2, 1, 32, 128, 128, 1) == 2 * 2 * 32 * 256 * 128 * 2
    assert lib.dd_ring_bytes(1, 1, 8, 64, 64, 0) == 2 * 8 * 128 * 64 * 4
    assert lib.dd_ring_bytes(0, 1, 8, 64, 64, 0) == 0
    # attention partials: one (D + 2)-float record per (b, h, 128-entry chunk), none for one chunk
    assert lib.dd_attn_workspace(1, 32, 128, 128) == 0
    assert lib.dd_attn_workspace(16, 32, 1024, 128) == 16 * 32 * 8 * 130 * 4
    # rows kept across steps, per layer: 2 slots of V rows (B*H x 2k x D x elem), 2 key lists
    # (B*H x 2k int32), the key -> row map (B*H x n_max int32), a 256-byte counter
    per_layer = 2 * 32 * 256 * 128 * 2 + 2 * 32 * 256 * 4 + 32 * 32768 * 4 + 256
    assert lib.dd_resident_bytes(2, 1, 32, 128, 32768, 128, 1) == 2 * per_layer
    assert lib.dd_resident_bytes(0, 1, 32, 128, 32768, 128, 1) == 0
    # layer-step workspace holds the two score planes of a layer
    ws = lib.dd_layer_step_workspace(1, 32, 128, 32768, 128)
    assert ws >= 32 * 2 * 32768 * 4
    assert ws % 256 == 0


@pytest.mark.parametrize("call,code", [
    ("score_bad_D", 2), ("score_bad_Q", 2), ("score_bad_dtype", 2), ("topk_k0", 2),
    ("topk_k_too_big", 2), ("gather_null_idx", 1), ("attn_stride", 1), ("gather_neg_m", 1),
    ("landmarks_chunk3", 1), ("landmarks_chunk128", 1), ("gather_chunks_chunk0", 1),
    ("gather_chunks_null_idx", 1),
])
def test_argument_errors_are_reported(lib, call, code):
    z = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    if call == "score_bad_D":
        rc = lib.dd_score(z, z, z, 1, 1, 2, 96, 10, 1, 0.0, 0, z, None)
    elif call == "score_bad_Q":
        rc = lib.dd_score(z, z, z, 1, 1, 3, 128, 10, 1, 0.0, 0, z, None)
    elif call == "score_bad_dtype":
        rc = lib.dd_score(z, z, z, 1, 1, 2, 128, 10, 7, 0.0, 0, z, None)
    elif call == "topk_k0":
        rc = lib.dd_topk(z, z, 1, 1, 1, 10, 0, z, None)
    elif call == "topk_k_too_big":
        rc = lib.dd_topk(z, z, 1, 1, 1, 10, 4097, z, None)
    elif call == "gather_null_idx":
        rc = lib.dd_gather(z, z, None, None, 1, 1, 4, 128, 10, 1, z, z, None)
    elif call == "gather_neg_m":
        rc = lib.dd_gather(z, z, z, None, 1, 1, -1, 128, 10, 1, z, z, None)
    elif call == "landmarks_chunk3":
        rc = lib.dd_landmarks(z, z, 1, 1, 128, 64, 3, 1, z, None)
    elif call == "landmarks_chunk128":
        rc = lib.dd_landmarks(z, z, 1, 1, 128, 64, 128, 1, z, None)
    elif call == "gather_chunks_chunk0":
        rc = lib.dd_gather_chunks(z, z, z, None, 1, 1, 4, 0, 128, 64, 1, z, z, None)
    elif call == "gather_chunks_null_idx":
        rc = lib.dd_gather_chunks(z, z, None, None, 1, 1, 4, 8, 128, 64, 1, z, z, None)
    else:
        rc = lib.dd_sparse_attn(z, 8, z, z, None, None, 1, 1, 4, 4, 128, 1, 0.0, z, None, None, 0, None)
    assert rc == code
    assert len(lib.dd_last_error()) > 0


def test_empty_shapes_are_no_ops(lib):
    z = ctypes.c_void_p(16)
    assert lib.dd_score(z, z, z, 0, 8, 2, 128, 10, 1, 0.0, 0, z, None) == 0
    assert lib.dd_topk(z, z, 1, 0, 2, 10, 4, z, None) == 0
    assert lib.dd_gather(z, z, z, None, 1, 1, 0, 128, 10, 1, z, z, None) == 0
    assert lib.dd_gather_chunks(z, z, z, None, 1, 1, 0, 8, 128, 10, 1, z, z, None) == 0
    assert lib.dd_landmarks(z, z, 0, 4, 128, 10, 8, 1, z, None) == 0
