"""The C ABI (CPU only): libsqa.so loads, exports every function include/sqa.h
declares, and rejects invalid arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

from sparse_query_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sqa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libsqa.so not built (run __graft_entry__.build())")

FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sqa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_function():
    lib = _lib.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    lib = _lib.load()
    for s in range(5):
        assert lib.sqa_status_string(s)
    assert b"unknown" in lib.sqa_status_string(99)
    assert lib.sqa_padded_length(1) == 256 and lib.sqa_padded_length(256) == 256
    assert lib.sqa_padded_length(257) == 512 and lib.sqa_padded_length(200000) == 200192
    assert lib.sqa_padded_length(0) == 0 and lib.sqa_padded_length(-1) == -1


def _fwd(**kw):
    a = dict(x=FAKE, Wq=FAKE + 0x1000000, Wk=FAKE + 0x2000000, Wv=FAKE + 0x3000000,
             Wo=FAKE + 0x4000000, out=FAKE + 0x5000000, B=1, N=256, d_model=256, H=8, H_q=4,
             H_kv=2, d_head=32, causal=0, dtype=_lib.SQA_DTYPE_BF16)
    a.update(kw)
    lib = _lib.load()
    st = lib.sqa_forward(a["x"], a["Wq"], a["Wk"], a["Wv"], a["Wo"], a["out"], a["B"], a["N"],
                         a["d_model"], a["H"], a["H_q"], a["H_kv"], a["d_head"], a["causal"],
                         a["dtype"], None)
    return st, lib.sqa_last_error_message().decode()


@pytest.mark.parametrize("kw,status,words", [
    (dict(x=0), _lib.SQA_ERR_INVALID_ARG, "x is null"),
    (dict(Wo=0), _lib.SQA_ERR_INVALID_ARG, "Wo is null"),
    (dict(Wq=FAKE + 0x1000008), _lib.SQA_ERR_INVALID_ARG, "aligned"),
    (dict(out=FAKE + 8), _lib.SQA_ERR_INVALID_ARG, "aligned"),
    (dict(out=FAKE), _lib.SQA_ERR_INVALID_ARG, "overlaps"),
    (dict(H_kv=3), _lib.SQA_ERR_INVALID_ARG, "multiple of H_kv"),
    (dict(H_kv=0), _lib.SQA_ERR_INVALID_ARG, "H_kv"),
    (dict(H_q=2, H_kv=4), _lib.SQA_ERR_INVALID_ARG, "H_kv <= H_q"),
    (dict(H_q=16, H_kv=2), _lib.SQA_ERR_INVALID_ARG, "H_q <= H"),
    (dict(d_model=512), _lib.SQA_ERR_INVALID_ARG, "H * d_head"),
    (dict(B=-1), _lib.SQA_ERR_INVALID_ARG, ">= 0"),
    (dict(causal=2), _lib.SQA_ERR_INVALID_ARG, "causal"),
    (dict(d_model=128, H=8, d_head=16), _lib.SQA_ERR_UNSUPPORTED, "d_head"),
    (dict(dtype=7), _lib.SQA_ERR_UNSUPPORTED, "dtype"),
    (dict(N=(1 << 24) + 1), _lib.SQA_ERR_UNSUPPORTED, "SQA_MAX_N"),
])
def test_forward_rejects_invalid_arguments(kw, status, words):
    st, msg = _fwd(**kw)
    assert st == status, msg
    assert words in msg


def test_empty_problem_is_a_no_op():
    # B*N == 0: nothing to compute, no device call, pointers unused
    assert _fwd(B=0, x=0, out=0)[0] == _lib.SQA_OK
    assert _fwd(N=0)[0] == _lib.SQA_OK


def _fwd_noalloc(**kw):
    a = dict(x=FAKE, Wq=FAKE + (1 << 40), Wk=FAKE + (2 << 40), Wv=FAKE + (3 << 40),
             Wo=FAKE + (4 << 40), out=FAKE + (5 << 40), B=1, N=256, d_model=1024, H=16, H_q=8,
             H_kv=4, d_head=64, causal=1, dtype=_lib.SQA_DTYPE_BF16)
    a.update(kw)
    lib = _lib.load()
    st = lib.sqa_forward_noalloc(a["x"], a["Wq"], a["Wk"], a["Wv"], a["Wo"], a["out"], a["B"],
                                 a["N"], a["d_model"], a["H"], a["H_q"], a["H_kv"], a["d_head"],
                                 a["causal"], a["dtype"], None)
    return st, lib.sqa_last_error_message().decode()


@pytest.mark.parametrize("kw,status,words", [
    # the 16/8/4-head bf16 shape needs about 3 KB of workspace per token: 65536
    # tokens exceed the 128 MiB array, rejected on the host before any HIP call
    (dict(N=65536), _lib.SQA_ERR_UNSUPPORTED, "SQA_NOALLOC_SCRATCH_BYTES"),
    (dict(B=4, N=16384), _lib.SQA_ERR_UNSUPPORTED, "SQA_NOALLOC_SCRATCH_BYTES"),
    (dict(x=0), _lib.SQA_ERR_INVALID_ARG, "x is null"),
    (dict(out=FAKE), _lib.SQA_ERR_INVALID_ARG, "overlaps"),
    (dict(H_kv=3), _lib.SQA_ERR_INVALID_ARG, "multiple of H_kv"),
])
def test_forward_noalloc_rejects_on_the_host(kw, status, words):
    st, msg = _fwd_noalloc(**kw)
    assert st == status, msg
    assert words in msg


def test_forward_noalloc_empty_problem_is_a_no_op():
    assert _fwd_noalloc(B=0, x=0, out=0)[0] == _lib.SQA_OK


def test_stage_entry_points_validate():
    lib = _lib.load()
    st = lib.sqa_attention(FAKE, FAKE + 0x100000, FAKE + 0x200000, 0, 1, 10, 4, 2, 64, 0,
                           _lib.SQA_DTYPE_BF16, None)
    assert st == _lib.SQA_ERR_INVALID_ARG and b"a is null" in lib.sqa_last_error_message()
    st = lib.sqa_attention(FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE, 1, 10, 4, 2, 64, 0,
                           _lib.SQA_DTYPE_BF16, None)
    assert st == _lib.SQA_ERR_INVALID_ARG and b"overlaps" in lib.sqa_last_error_message()
    st = lib.sqa_output_projection(FAKE, FAKE + 0x100000, FAKE + 0x200000, 10, 48, 64,
                                   _lib.SQA_DTYPE_BF16, None)
    assert st == _lib.SQA_ERR_UNSUPPORTED
    st = lib.sqa_qkv_projection(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 256, 8, 4, 2, 32,
                                _lib.SQA_DTYPE_FP32, None)
    assert st == _lib.SQA_ERR_INVALID_ARG and b"overlaps" in lib.sqa_last_error_message()


def test_python_binding_maps_statuses_to_exceptions():
    with pytest.raises(ValueError):
        _lib.check(_lib.SQA_ERR_INVALID_ARG)
    with pytest.raises(NotImplementedError):
        _lib.check(_lib.SQA_ERR_UNSUPPORTED)
    with pytest.raises(_lib.SQAError):
        _lib.check(_lib.SQA_ERR_HIP)
    with pytest.raises(_lib.SQAError):
        _lib.check(_lib.SQA_ERR_OUT_OF_MEMORY)
    _lib.check(_lib.SQA_OK)


def _fwd_varlen(lens, **kw):
    a = dict(x=FAKE, Wq=FAKE + 0x1000000, Wk=FAKE + 0x2000000, Wv=FAKE + 0x3000000,
             Wo=FAKE + 0x4000000, out=FAKE + 0x5000000, B=2, N=256, d_model=256, H=8, H_q=4,
             H_kv=2, d_head=32, causal=1, dtype=_lib.SQA_DTYPE_BF16)
    a.update(kw)
    lib = _lib.load()
    st = lib.sqa_forward_varlen(a["x"], a["Wq"], a["Wk"], a["Wv"], a["Wo"], a["out"], lens, a["B"],
                                a["N"], a["d_model"], a["H"], a["H_q"], a["H_kv"], a["d_head"],
                                a["causal"], a["dtype"], None)
    return st, lib.sqa_last_error_message().decode()


@pytest.mark.parametrize("lens,kw,status,words", [
    (0, {}, _lib.SQA_ERR_INVALID_ARG, "lens is null"),
    (FAKE + 0x6000002, {}, _lib.SQA_ERR_INVALID_ARG, "4-byte aligned"),
    (FAKE + 0x5000040, {}, _lib.SQA_ERR_INVALID_ARG, "overlaps lens"),
    (FAKE + 0x6000000, dict(x=0), _lib.SQA_ERR_INVALID_ARG, "x is null"),
    (FAKE + 0x6000000, dict(H_kv=3), _lib.SQA_ERR_INVALID_ARG, "multiple of H_kv"),
    (FAKE + 0x6000000, dict(d_model=128, H=8, d_head=16), _lib.SQA_ERR_UNSUPPORTED, "d_head"),
])
def test_forward_varlen_rejects_invalid_arguments(lens, kw, status, words):
    st, msg = _fwd_varlen(lens, **kw)
    assert st == status, msg
    assert words in msg


def test_forward_varlen_empty_batch_is_a_no_op():
    assert _fwd_varlen(0, B=0)[0] == _lib.SQA_OK


def _decode(**kw):
    a = dict(x=FAKE, Wq=FAKE + 0x1000000, Wk=FAKE + 0x2000000, Wv=FAKE + 0x3000000,
             Wo=FAKE + 0x4000000, out=FAKE + 0x5000000, kc=FAKE + 0x6000000, vc=FAKE + 0x7000000,
             pos=FAKE + 0x8000000, B=2, N_max=1024, d_model=256, H=8, H_q=4, H_kv=2, d_head=32,
             dtype=_lib.SQA_DTYPE_BF16)
    a.update(kw)
    lib = _lib.load()
    st = lib.sqa_decode_step(a["x"], a["Wq"], a["Wk"], a["Wv"], a["Wo"], a["out"], a["kc"], a["vc"],
                             a["pos"], a["B"], a["N_max"], a["d_model"], a["H"], a["H_q"], a["H_kv"],
                             a["d_head"], a["dtype"], None)
    return st, lib.sqa_last_error_message().decode()


@pytest.mark.parametrize("kw,status,words", [
    (dict(pos=0), _lib.SQA_ERR_INVALID_ARG, "pos is null"),
    (dict(pos=FAKE + 0x8000002), _lib.SQA_ERR_INVALID_ARG, "4-byte aligned"),
    (dict(kc=0), _lib.SQA_ERR_INVALID_ARG, "k_cache is null"),
    (dict(vc=FAKE + 0x6000100), _lib.SQA_ERR_INVALID_ARG, "k_cache overlaps v_cache"),
    (dict(out=FAKE + 0x6000000), _lib.SQA_ERR_INVALID_ARG, "overlaps"),
    (dict(pos=FAKE + 0x6000040), _lib.SQA_ERR_INVALID_ARG, "cache overlaps an input"),
    (dict(N_max=0), _lib.SQA_ERR_UNSUPPORTED, "N_max"),
    (dict(B=70000), _lib.SQA_ERR_UNSUPPORTED, "65535"),
    (dict(H_kv=3), _lib.SQA_ERR_INVALID_ARG, "multiple of H_kv"),
    (dict(d_model=128, H=8, d_head=16), _lib.SQA_ERR_UNSUPPORTED, "d_head"),
])
def test_decode_step_rejects_invalid_arguments(kw, status, words):
    st, msg = _decode(**kw)
    assert st == status, msg
    assert words in msg


def test_decode_step_with_no_tokens_is_a_no_op():
    assert _decode(B=0, x=0, pos=0)[0] == _lib.SQA_OK


def test_prefill_validates_the_caches():
    lib = _lib.load()
    args = lambda kc, vc, N, N_max: (FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000,
                                     FAKE + 0x4000000, FAKE + 0x5000000, kc, vc, 2, N, N_max, 256,
                                     8, 4, 2, 32, _lib.SQA_DTYPE_BF16, None)
    assert lib.sqa_prefill(*args(0, FAKE + 0x7000000, 64, 128)) == _lib.SQA_ERR_INVALID_ARG
    assert b"k_cache is null" in lib.sqa_last_error_message()
    assert lib.sqa_prefill(*args(FAKE + 0x6000000, FAKE + 0x7000000, 200, 128)) == _lib.SQA_ERR_INVALID_ARG
    assert b"N exceeds N_max" in lib.sqa_last_error_message()
    assert lib.sqa_prefill(*args(FAKE + 0x6000000, FAKE + 0x7000000, 64, 0)) == _lib.SQA_ERR_UNSUPPORTED
    assert lib.sqa_prefill(*args(FAKE + 0x6000000, FAKE + 0x6000040, 64, 128)) == _lib.SQA_ERR_INVALID_ARG
    assert b"overlaps" in lib.sqa_last_error_message()


def _bwd(**kw):
    a = dict(x=FAKE, Wq=FAKE + 0x1000000, Wk=FAKE + 0x2000000, Wv=FAKE + 0x3000000,
             Wo=FAKE + 0x4000000, dy=FAKE + 0x5000000, dx=FAKE + 0x6000000, dWq=FAKE + 0x7000000,
             dWk=FAKE + 0x8000000, dWv=FAKE + 0x9000000, dWo=FAKE + 0xA000000, saved=None,
             saved_bytes=0, B=2, N=100,
             d_model=256, H=8, H_q=4, H_kv=2, d_head=32, causal=1, dtype=_lib.SQA_DTYPE_BF16)
    a.update(kw)
    lib = _lib.load()
    st = lib.sqa_backward(*(a[k] for k in ("x", "Wq", "Wk", "Wv", "Wo", "dy", "saved", "saved_bytes",
                                           "dx", "dWq", "dWk", "dWv", "dWo", "B", "N", "d_model",
                                           "H", "H_q", "H_kv", "d_head", "causal", "dtype")), None)
    return st, lib.sqa_last_error_message().decode()


@pytest.mark.parametrize("kw,status,words", [
    (dict(dy=0), _lib.SQA_ERR_INVALID_ARG, "dy is null"),
    (dict(dWk=FAKE + 0x8000008), _lib.SQA_ERR_INVALID_ARG, "dWk is null or not 16-byte aligned"),
    (dict(dx=FAKE + 0x5000000), _lib.SQA_ERR_INVALID_ARG, "output overlaps an input"),
    (dict(dWo=FAKE + 0x7000040), _lib.SQA_ERR_INVALID_ARG, "two outputs overlap"),
    (dict(dWq=FAKE + 0x40), _lib.SQA_ERR_INVALID_ARG, "output overlaps an input"),
    (dict(causal=2), _lib.SQA_ERR_INVALID_ARG, "causal"),
    (dict(H_kv=3), _lib.SQA_ERR_INVALID_ARG, "multiple of H_kv"),
    (dict(d_model=128, H=8, d_head=16), _lib.SQA_ERR_UNSUPPORTED, "d_head"),
    (dict(dtype=7), _lib.SQA_ERR_UNSUPPORTED, "dtype"),
    (dict(N=(1 << 24) + 1), _lib.SQA_ERR_UNSUPPORTED, "SQA_MAX_N"),
    (dict(saved=FAKE + 0xB000008, saved_bytes=1 << 24), _lib.SQA_ERR_INVALID_ARG, "saved is not 16"),
    (dict(saved=FAKE + 0xB000000, saved_bytes=1000), _lib.SQA_ERR_INVALID_ARG, "too small"),
    (dict(saved=FAKE + 0x9000100, saved_bytes=1 << 24), _lib.SQA_ERR_INVALID_ARG, "saved overlaps"),
])
def test_backward_rejects_invalid_arguments(kw, status, words):
    st, msg = _bwd(**kw)
    assert st == status, msg
    assert words in msg


def test_backward_of_an_empty_batch_is_a_no_op():
    assert _bwd(B=0, x=0, dy=0)[0] == _lib.SQA_OK


def test_training_saved_bytes_and_forward_train_validate():
    lib = _lib.load()
    n = lib.sqa_training_saved_bytes(2, 100, 4, 2, 32, _lib.SQA_DTYPE_BF16)
    # q + k + vt (Np = 256) + a (N = 100) in bf16, the fp32 row statistics and fp32 a
    want = sum((x + 255) // 256 * 256 for x in (2 * 2 * 256 * 4 * 32, 2 * 2 * 256 * 2 * 32,
                                               2 * 2 * 256 * 2 * 32, 2 * 2 * 100 * 4 * 32,
                                               4 * 2 * 4 * 256, 4 * 2 * 100 * 4 * 32))
    assert n == want
    assert lib.sqa_training_saved_bytes(2, 100, 4, 3, 32, _lib.SQA_DTYPE_BF16) == 0
    args = lambda saved, nb: (FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000,
                              FAKE + 0x4000000, FAKE + 0x5000000, saved, nb, 2, 100, 256, 8, 4, 2,
                              32, 1, _lib.SQA_DTYPE_BF16, None)
    assert lib.sqa_forward_train(*args(None, n)) == _lib.SQA_ERR_INVALID_ARG
    assert b"saved is null" in lib.sqa_last_error_message()
    assert lib.sqa_forward_train(*args(FAKE + 0x6000000, n - 1)) == _lib.SQA_ERR_INVALID_ARG
    assert b"too small" in lib.sqa_last_error_message()
    assert lib.sqa_forward_train(*args(FAKE + 0x5000000, n)) == _lib.SQA_ERR_INVALID_ARG
    assert b"overlaps" in lib.sqa_last_error_message()
