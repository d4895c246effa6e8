"""Host-side checks of the C ABI (no GPU needed): every declared entry point is
exported, the packer round-trips and lays codes out as documented, and
argument validation returns the documented status before anything reaches
the device."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
from tests.blocks import enc_q4_0

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def q():
    import quantized_decode_step_amd as qd
    return qd


def declared_functions():
    src = open(os.path.join(ROOT, "include", "ocrdec.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ocrdec_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_function_is_exported(q):
    names = declared_functions()
    assert len(names) >= 14
    lib = ctypes.CDLL(q.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), "%s declared in include/ocrdec.h but not exported" % n
    # and the binding exposes the same names
    for n in names:
        assert hasattr(q, n), "binding lacks %s" % n


def test_binding_struct_sizes_match_the_header(q):
    # pointer = 8, int32 = 4: the ABI structs are plain C layouts
    assert ctypes.sizeof(q.QMatDesc) == 24
    assert ctypes.sizeof(q.StateDesc) == 32
    assert ctypes.sizeof(q.StepCapture) == 24
    assert ctypes.sizeof(q.MoeCapture) == 40


@pytest.mark.parametrize("fmt", [synth.F16, synth.Q8_0, synth.Q4_0, synth.U8A_G32])
@pytest.mark.parametrize("n,k", [(1, 32), (17, 96), (40, 160), (3, 1280), (129, 64)])
def test_pack_unpack_roundtrip(q, fmt, n, k):
    m = synth.random_qmat(fmt, synth.stream_id(9, "pack", fmt, n, k), n, k, 0.02)
    packed = q.ocrdec_pack(fmt, n, k, m.data)
    assert packed.size == q.ocrdec_packed_bytes(fmt, n, k)
    back = q.ocrdec_unpack(fmt, n, k, packed, m.data.size)
    assert np.array_equal(back, m.data)


def test_packed_bytes_formula(q):
    # tiles of 16 rows x chunks of 128 (Q4_0) / 64 (Q8_0, U8A) / 32 (F16) columns
    assert q.ocrdec_packed_bytes(synth.Q4_0, 1792, 1280) == 112 * 10 * 1152
    assert q.ocrdec_packed_bytes(synth.Q8_0, 3840, 1280) == 240 * 20 * 1088
    assert q.ocrdec_packed_bytes(synth.F16, 129280, 1280) == 8080 * 40 * 1024
    assert q.ocrdec_packed_bytes(synth.U8A_G32, 1536, 512) == 96 * 8 * 1152
    # ragged: 17 rows -> 2 tiles, 96 columns -> 1 Q4_0 chunk; rounded to 256 bytes
    assert q.ocrdec_packed_bytes(synth.Q4_0, 17, 96) == 2 * 1152


def test_q4_packed_lane_layout(q):
    """Lane l of a chunk holds row l % 16 and columns 8*(l//16) .. +7 of each
    of the chunk's four blocks, element 2p at bits 4p and element 2p+1 at bits
    16 + 4p of the block's dword; the scales follow at byte 1024."""
    n, k = 16, 128
    codes = (np.arange(n * k).reshape(n, k) * 7) % 16
    d = np.array([[0.5, 1.0, 2.0, 4.0]] * n)
    d[3] = [0.25, 0.125, 8.0, 16.0]
    m = enc_q4_0(d, codes)
    packed = q.ocrdec_pack(synth.Q4_0, n, k, m.data)
    for lane in (0, 5, 16, 37, 63):
        row, c8 = lane % 16, 8 * (lane // 16)
        words = packed[lane * 16:(lane + 1) * 16].view(np.uint32)
        for j in range(4):
            for i in range(8):
                p, hi = i // 2, i % 2
                bit = (16 if hi else 0) + 4 * p
                assert (int(words[j]) >> bit) & 15 == codes[row, 32 * j + c8 + i]
    scales = packed[1024:1152].view(np.float16).reshape(16, 4)
    assert np.array_equal(scales.astype(np.float64), d)


def _err(q, fn, *a, **kw):
    with pytest.raises(q.OcrdecError) as e:
        fn(*a, **kw)
    return e.value.status


def test_validation_errors_without_a_device(q):
    fake = 1 << 20  # never dereferenced: validation fails first
    W = q.QMatDesc(synth.Q8_0, 64, 1280, fake)
    assert _err(q, q.ocrdec_gemv_q, W, 0, fake, 1280, fake, 0, 64, 0) == q.OCRDEC_ERR_INVALID_ARG
    assert _err(q, q.ocrdec_gemv_q, W, 1, fake, 1000, fake, 0, 64, 0) == q.OCRDEC_ERR_INVALID_ARG
    assert _err(q, q.ocrdec_gemv_q, q.QMatDesc(synth.Q8_0, 64, 1270, fake), 1, fake, 1280, fake, 0, 64, 0) \
        == q.OCRDEC_ERR_INVALID_ARG
    assert _err(q, q.ocrdec_gemv_q, q.QMatDesc(7, 64, 1280, fake), 1, fake, 1280, fake, 0, 64, 0) \
        == q.OCRDEC_ERR_UNSUPPORTED
    assert _err(q, q.ocrdec_gemv_q, q.QMatDesc(synth.Q8_0, 64, 1280, fake + 8), 1, fake, 1280, fake, 0, 64, 0) \
        == q.OCRDEC_ERR_INVALID_ARG
    a = q.AttnArgs(1, 10, 96, fake, 3 * 960, fake, fake, 100, 128, fake, fake, None, 1e4, 0.1, fake, 960)
    assert _err(q, q.ocrdec_attn_workspace_bytes, a) == q.OCRDEC_ERR_UNSUPPORTED
    a.head_dim = 128
    a.ld_qkv = 100
    assert _err(q, q.ocrdec_attn_decode, a, None, 0, 0) == q.OCRDEC_ERR_INVALID_ARG
    a.ld_qkv = 3 * 1280
    a.ld_out = 1280
    assert _err(q, q.ocrdec_attn_decode, a, None, 0, 0) == q.OCRDEC_ERR_WORKSPACE
    assert "need" in q.ocrdec_last_error()
    # the cache capacity and the row count have hard limits (one merge weight
    # per 64-key split in LDS; rows are a grid dimension)
    a.prefix_cap, a.ring_cap = 65536 - 127, 128
    assert _err(q, q.ocrdec_attn_workspace_bytes, a) == q.OCRDEC_ERR_INVALID_ARG
    assert "65536" in q.ocrdec_last_error()
    a.prefix_cap = 65536 - 128
    assert q.ocrdec_attn_workspace_bytes(a) > 0
    a.rows = 65536
    assert _err(q, q.ocrdec_attn_workspace_bytes, a) == q.OCRDEC_ERR_INVALID_ARG
    a.rows, a.prefix_cap = 1, 100
    r = q.QMatDesc(synth.Q8_0, 64, 1280, fake)
    gu = q.QMatDesc(synth.Q4_0, 64 * 2 * 896, 1280, fake)
    dn = q.QMatDesc(synth.Q4_0, 64 * 1280, 896, fake)
    w = q.MoeWeights(1280, 64, 9, 0, 896, r, None, gu, dn, q.QMatDesc(), q.QMatDesc())
    assert _err(q, q.ocrdec_moe_workspace_bytes, w, 1) == q.OCRDEC_ERR_UNSUPPORTED
    w.top_k = 6
    assert q.ocrdec_moe_workspace_bytes(w, 1) > 0
    assert _err(q, q.ocrdec_moe_layer, w, 1, fake, fake, True, None, None, None, 0, 0) == q.OCRDEC_ERR_WORKSPACE
    w.gate_up = q.QMatDesc(synth.Q4_0, 100, 1280, fake)
    assert _err(q, q.ocrdec_moe_workspace_bytes, w, 1) == q.OCRDEC_ERR_INVALID_ARG


def test_device_status_validation_without_a_device(q):
    """The status query checks its arguments before touching the device."""
    assert _err(q, q.ocrdec_device_status, None, 4096, 0) == q.OCRDEC_ERR_INVALID_ARG
    assert _err(q, q.ocrdec_device_status, 1 << 20, 16, 0) == q.OCRDEC_ERR_WORKSPACE
    assert "status" in q.ocrdec_last_error()


def test_prefill_and_round_validation_without_a_device(q):
    """Prompt lengths, rows and requests are checked on the host before any
    device work."""
    fake = 1 << 20
    m = q.ModelDesc()
    m.n_layers, m.hidden, m.n_heads, m.head_dim, m.vocab = 1, 256, 2, 128, 1000
    m.lm_head = q.QMatDesc(synth.F16, 1000, 256, fake)
    st = q.StateDesc(2, 16, 8, fake, fake)
    assert _err(q, q.ocrdec_prefill, m, st, 0, 0, stream=0) == q.OCRDEC_ERR_INVALID_ARG
    assert _err(q, q.ocrdec_prefill_workspace_bytes, m, st, 0) == q.OCRDEC_ERR_INVALID_ARG
    reqs = (q.Request * 2)()
    out = (ctypes.c_int32 * 4)()
    for r in reqs:
        r.tokens, r.P, r.max_new, r.out = fake, 5, 4, ctypes.cast(out, ctypes.c_void_p)
    reqs[1].P = 17  # beyond prefix_cap
    assert _err(q, q.ocrdec_run_round, m, st, reqs, stream=0) == q.OCRDEC_ERR_INVALID_ARG
    assert "prefix_cap" in q.ocrdec_last_error()
    reqs[1].P = 5
    reqs[1].max_new = 0
    assert _err(q, q.ocrdec_run_round, m, st, reqs, stream=0) == q.OCRDEC_ERR_INVALID_ARG
    reqs[1].max_new = 4
    reqs[1].tokens = None
    assert _err(q, q.ocrdec_run_round, m, st, reqs, stream=0) == q.OCRDEC_ERR_INVALID_ARG
