"""CPU tests of the library boundary: it loads, exports what the header
declares, agrees with the oracle's codebook, and rejects bad arguments on the
host before touching the GPU. No compute call runs here."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

from qlora_fine_tuning_blockwise_amd import _lib
import qlora_fine_tuning_blockwise_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from qlora_fine_tuning_blockwise_amd import build
        build.build()
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = _lib.header_functions()
    assert {"qlora_quantize_nf4_dq", "qlora_dequant_bf16", "qlora_linear_fwd",
            "qlora_linear_bwd"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_codebook_matches_oracle_bit_exact(lib, olib):
    lv, th = q.qlora_codebook()
    olv, oth = olib.nf4_codebook()
    assert np.array_equal(lv.view(np.uint32), olv.view(np.uint32))
    assert np.array_equal(th.view(np.uint32), oth.view(np.uint32))
    cid = q.qlora_codebook_id()
    assert cid != 0 and cid == q.qlora_codebook_id()


def test_sizes_accounting(lib):
    cb, qb, sb = q.qlora_nf4_sizes(4096, 4096)
    assert (cb, qb, sb) == (4096 * 4096 // 2, 4096 * 4096 // 64, 4 * 4096 * 4096 // 16384)
    assert 8 * (cb + qb + sb) / (4096 * 4096) == 4.126953125
    cb, qb, sb = q.qlora_nf4_sizes(11008, 4096)  # 172 blocks per row: groups straddle rows
    assert sb == 4 * ((11008 * 4096 // 64 + 255) // 256)
    for N, K in ((0, 64), (4, 0), (4, 96), (4, 32)):
        with pytest.raises(RuntimeError):
            q.qlora_nf4_sizes(N, K)


def test_strerror_covers_codes(lib):
    texts = {q.qlora_strerror(s) for s in range(11)}
    assert len(texts) == 11 and q.qlora_strerror(99) == "unknown status"


FAKE = 1 << 20  # an aligned address never dereferenced: validation fails first


def _p(v):
    return ctypes.c_void_p(v)


def _desc(**kw):
    """A descriptor with aligned fake buffers and this library's metadata."""
    a = dict(N=64, K=128, codes=FAKE, absmax_q=FAKE, absmax_scale=FAKE, dq_format=0,
             format_version=_lib.FORMAT_VERSION, setup_id=None, reserved=0)
    a.update(kw)
    if a["setup_id"] is None:
        a["setup_id"] = q.qlora_setup_id(a["dq_format"]) if a["dq_format"] in (0, 1, 2) else 0
    return ctypes.pointer(_lib.NF4Desc(a["N"], a["K"], a["codes"], a["absmax_q"],
                                       a["absmax_scale"], a["dq_format"], a["format_version"],
                                       a["setup_id"], a["reserved"]))


def test_descriptor_check(lib):
    """[P4] "Operational coupling": a weight is only read with the setup it
    was quantized with. Each mismatch is rejected on the host."""
    c = lib.qlora_nf4_check
    assert c(_desc()) == 0
    for f in (0, 1, 2):
        assert c(_desc(dq_format=f)) == 0
    assert c(None) == 1
    assert c(_desc(codes=None)) == 1
    assert c(_desc(absmax_q=None)) == 1
    assert c(_desc(absmax_scale=None)) == 1
    assert c(_desc(dq_format=3, setup_id=q.qlora_setup_id(0))) == 1   # unknown format
    assert c(_desc(reserved=1)) == 1
    assert c(_desc(K=96)) == 2
    assert c(_desc(N=0)) == 2
    assert c(_desc(codes=FAKE + 4)) == 3
    assert c(_desc(absmax_scale=FAKE + 8)) == 3
    assert c(_desc(format_version=0)) == 9                            # never quantized
    assert c(_desc(format_version=2)) == 9                            # another layout version
    assert c(_desc(setup_id=0)) == 9
    assert c(_desc(setup_id=q.qlora_setup_id(0) ^ 1)) == 9            # another codebook
    # the format travels with its setup id: relabelling the format alone fails
    assert c(_desc(dq_format=1, setup_id=q.qlora_setup_id(0))) == 9
    assert c(_desc(dq_format=0, setup_id=q.qlora_setup_id(2))) == 9
    # every reading entry point runs the same check first
    bad = _desc(setup_id=q.qlora_setup_id(1))
    assert lib.qlora_dequant_bf16(bad, _p(FAKE), 0, None) == 9
    assert _fwd(lib, w=bad) == 9
    assert lib.qlora_merge_lora(bad, None, 64, 128, _p(FAKE), _p(FAKE), 16, 32.0, _p(FAKE),
                                _p(FAKE), 1 << 30, None) == 9
    args = _bwd_base()
    args[0] = bad
    assert lib.qlora_linear_bwd(*args) == 9


def test_quantize_validation(lib):
    f = lib.qlora_quantize_nf4_dq
    d = _desc(N=0, K=0, format_version=0, setup_id=0)
    assert f(None, 1, 4, 64, 0, d, None) == 1
    assert f(_p(FAKE), 1, 4, 64, 0, None, None) == 1
    assert f(_p(FAKE), 1, 4, 64, 0, _desc(codes=None), None) == 1
    assert f(_p(FAKE), 1, 4, 96, 0, d, None) == 2
    assert f(_p(FAKE), 1, 0, 64, 0, d, None) == 2
    assert f(_p(FAKE), 7, 4, 64, 0, d, None) == 4
    assert f(_p(FAKE + 2), 1, 4, 64, 0, d, None) == 3
    assert f(_p(FAKE), 1, 4, 64, 3, d, None) == 1   # dq format
    assert f(_p(FAKE), 1, 4, 64, -1, d, None) == 1
    # rejected calls leave the descriptor untouched
    assert (d.contents.N, d.contents.format_version, d.contents.setup_id) == (0, 0, 0)
    dq = lib.qlora_dequant_bf16
    assert dq(_desc(), None, 0, None) == 1
    assert dq(_desc(absmax_q=None), _p(FAKE), 0, None) == 1
    assert dq(_desc(K=65), _p(FAKE), 0, None) == 2
    assert dq(_desc(absmax_scale=FAKE + 4), _p(FAKE), 0, None) == 3
    assert dq(_desc(), _p(FAKE + 2), 0, None) == 3
    assert dq(_desc(dq_format=9, setup_id=1), _p(FAKE), 0, None) == 1     # dq format
    assert dq(_desc(), _p(FAKE), 2, None) == 1     # layout
    assert dq(_desc(N=1 << 22, K=1 << 16), _p(FAKE), 1, None) == 2


def test_setup_ids(lib):
    """One identifier per second-level format; the default one is the
    codebook id; unknown formats give 0."""
    ids = [lib.qlora_setup_id(f) for f in (0, 1, 2)]
    assert ids[0] == lib.qlora_codebook_id() and len(set(ids)) == 3 and 0 not in ids
    assert lib.qlora_setup_id(3) == 0 and lib.qlora_setup_id(-1) == 0


def _fwd(lib, **kw):
    a = dict(w=None, x=FAKE, M=32, A=FAKE, B=FAKE, r=16, alpha=32.0, y=FAKE, ydt=0, u=None, ws=FAKE,
             wsb=1 << 30)
    wkw = {k: kw.pop(k) for k in list(kw) if k in ("N", "K", "dq_format", "codes")}
    a.update(kw)
    w = a["w"] if a["w"] is not None else _desc(**wkw)
    P = lambda v: None if v is None else _p(v)
    return lib.qlora_linear_fwd(w, P(a["x"]), a["M"], P(a["A"]), P(a["B"]), a["r"], a["alpha"],
                                P(a["y"]), a["ydt"], P(a["u"]), P(a["ws"]), a["wsb"], None)


def test_fwd_validation(lib):
    assert _fwd(lib, x=None) == 1
    assert _fwd(lib, M=-1) == 1
    assert _fwd(lib, K=100) == 2
    assert _fwd(lib, ydt=5) == 4
    assert _fwd(lib, r=8) == 5
    assert _fwd(lib, r=24) == 5
    assert _fwd(lib, r=512) == 5
    assert _fwd(lib, B=FAKE + 8) == 3
    assert _fwd(lib, wsb=16) == 6
    assert _fwd(lib, ws=None) == 6
    assert _fwd(lib, codes=None) == 1
    assert lib.qlora_linear_fwd(None, _p(FAKE), 32, _p(FAKE), _p(FAKE), 16, 32.0, _p(FAKE), 0,
                                None, _p(FAKE), 1 << 30, None) == 1
    assert _fwd(lib, M=0) == 0  # empty batch: a no-op that enqueues nothing


def _bwd_base():
    return [_desc(), _p(FAKE), _p(FAKE), 32, _p(FAKE), _p(FAKE), 16, 32.0, None, _p(FAKE), 0,
            _p(FAKE), _p(FAKE), 0, _p(FAKE), 1 << 30, None]


def test_bwd_validation(lib):
    f = lib.qlora_linear_bwd

    def call(i, v):
        a = _bwd_base()
        a[i] = v
        return f(*a)
    assert call(2, None) == 1          # dY missing
    assert call(1, None) == 1          # x missing while dA/dB wanted
    assert call(0, _desc(K=96)) == 2   # K % 64
    assert call(10, 3) == 4            # dx dtype
    assert call(13, 9) == 4            # grad dtype
    assert call(6, 0) == 5             # r
    assert call(4, _p(FAKE + 1)) == 3  # A misaligned
    assert call(15, 64) == 6           # workspace too small
    assert call(0, None) == 1          # no weight


def test_gemm_nt_validation(lib):
    f = lib.qlora_gemm_bf16_nt
    base = [_p(FAKE), 64, _p(FAKE), 64, 0, _p(FAKE), _p(FAKE), 8, 128, 64, 16, _p(FAKE), 0, None]

    def call(i, v, **kw):
        a = list(base)
        a[i] = v
        for j, w in kw.items():
            a[int(j[1:])] = w
        return f(*a)
    assert call(7, -1) == 1            # M < 0
    assert call(8, 0) == 2             # N < 1
    assert call(9, 48) == 2            # K % 32
    assert call(1, 32) == 2            # lda < K
    assert call(3, 68) == 2            # ldb % 8
    assert call(1, 1 << 22) == 2       # tile row offsets past 2^31 bytes
    assert call(12, 3) == 4            # y dtype
    assert call(10, 8) == 5            # r
    assert call(0, None) == 1          # a missing
    assert call(5, _p(FAKE + 8)) == 3  # e misaligned
    assert call(4, 2) == 1             # b layout
    assert call(4, 1, a1=2048, a8=1 << 20, a9=2048) == 2  # K-slab: 2 N K past 2^31 bytes
    assert call(4, 1, a3=3, a7=-1) == 1  # K-slab ignores ldb (M < 0 still rejected first)
    assert call(7, 0) == 0             # empty: a no-op


def test_merge_validation(lib):
    f = lib.qlora_merge_lora

    def call(i, v):
        a = [_desc(), None, 64, 128, _p(FAKE), _p(FAKE), 16, 32.0, _p(FAKE), _p(FAKE), 1 << 30,
             None]
        a[i] = v
        return f(*a)
    assert call(3, 100) == 2            # K % 64
    assert call(6, 8) == 5              # r
    assert call(8, None) == 1           # merged missing
    assert call(0, None) == 1           # neither NF4 base nor bf16 base
    assert call(4, _p(FAKE + 4)) == 3   # A misaligned
    assert call(10, 64) == 6            # workspace too small
    assert call(0, _desc(dq_format=4, setup_id=1)) == 1  # dq format
    assert call(2, 32) == 2             # descriptor is [64, 128], not [32, 128]
    assert lib.qlora_workspace_bytes(2, 0, 64, 128, 16) >= 2 * 16 * (64 + 128)


def test_workspace_query(lib):
    assert q.qlora_workspace_bytes(0, 16, 4096, 4096, 16) > 0
    assert q.qlora_workspace_bytes(0, 4096, 4096, 4096, 16) > q.qlora_workspace_bytes(0, 1024, 4096, 4096, 16)
    assert q.qlora_workspace_bytes(1, 4096, 11008, 4096, 16) > 0
    assert q.qlora_workspace_bytes(0, 16, 4096, 4000, 16) == 0
    assert q.qlora_workspace_bytes(5, 16, 4096, 4096, 16) == 0  # no such op
    # from 512 rows on the fast routes hold one bf16 copy of the weight; the
    # lean routes (in-register dequantization) hold none
    for fast, lean_op in ((0, 3), (1, 4)):
        assert q.qlora_workspace_bytes(fast, 512, 4096, 1024, 16) \
            - q.qlora_workspace_bytes(lean_op, 512, 4096, 1024, 16) >= 4096 * 1024 * 2
    assert q.qlora_workspace_bytes(1, 512, 4096, 1024, 16) \
        - q.qlora_workspace_bytes(1, 511, 4096, 1024, 16) >= 4096 * 1024 * 2
    # below 512 rows, with few output tiles, the forward's tile kernel splits
    # its reduction over K and the workspace holds the fp32 partial sums: two
    # ranges for 511 x 4096 (8.4 MB each), none with plenty of tiles
    assert q.qlora_workspace_bytes(0, 511, 4096, 1024, 16) >= 2 * 511 * 4096 * 4
    assert q.qlora_workspace_bytes(0, 511, 32768, 1024, 16) < 511 * 32768 * 4
    lean = q.qlora_workspace_bytes(3, 512, 4096, 1024, 16)
    assert 0 < lean < 4096 * 1024 * 2 // 8
    assert q.qlora_workspace_bytes(3, 16, 4096, 1024, 16) == q.qlora_workspace_bytes(0, 16, 4096, 1024, 16)
    # the backward's lean route holds no transposed copy (nor the dense
    # stage's split partials) either
    assert q.qlora_workspace_bytes(1, 512, 4096, 1024, 16) - q.qlora_workspace_bytes(4, 512, 4096, 1024, 16) \
        >= 4096 * 1024 * 2
    assert q.qlora_workspace_bytes(4, 511, 4096, 1024, 16) == q.qlora_workspace_bytes(1, 511, 4096, 1024, 16)


@pytest.fixture(scope="module")
def arith(tmp_path_factory):
    d = tmp_path_factory.mktemp("arith")
    so = str(d / "arith.so")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                    os.path.join(ROOT, "tests", "csrc", "kernel_arith_check.c"), "-o", so, "-lm"],
                   check=True)
    L = ctypes.CDLL(so)
    L.check_division.restype = ctypes.c_int64
    L.check_division.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
                                 ctypes.POINTER(ctypes.c_int64)]
    L.check_buckets.restype = ctypes.c_int64
    L.check_buckets.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64)]
    L.check_quotient_codes.restype = ctypes.c_int64
    L.check_quotient_codes.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.POINTER(ctypes.c_int64)]
    return L


def test_fast_division_exact_for_all_bf16_pairs(arith, lib):
    _, th = q.qlora_codebook()
    th = np.ascontiguousarray(th)
    n, vbad = ctypes.c_int64(), ctypes.c_int64()
    bad = arith.check_division(th.ctypes.data_as(ctypes.c_void_p), ctypes.byref(n), ctypes.byref(vbad))
    assert n.value > 4.9e8
    assert bad == 0 and vbad.value == 0


def test_bucket_code_search_exhaustive(arith, lib):
    _, th = q.qlora_codebook()
    th = np.ascontiguousarray(th)
    n = ctypes.c_int64()
    bad = arith.check_buckets(th.ctypes.data_as(ctypes.c_void_p), ctypes.byref(n))
    assert n.value == 2 * (0x3F800000 + 1) and bad == 0


def test_quotient_thresholds_are_threshold_or_successor(lib):
    _, th = q.qlora_codebook()
    tq = q.qlora_codebook_quotient_thresholds()
    succ = np.nextafter(th, np.float32(np.inf))
    assert np.all((tq == th) | (tq == succ))
    assert lib.qlora_codebook_quotient_thresholds(None) == 1


def test_quotient_code_path_exact_for_all_bf16_pairs(arith, lib):
    _, th = q.qlora_codebook()
    th = np.ascontiguousarray(th)
    tq = np.ascontiguousarray(q.qlora_codebook_quotient_thresholds())
    n = ctypes.c_int64()
    bad = arith.check_quotient_codes(th.ctypes.data_as(ctypes.c_void_p),
                                     tq.ctypes.data_as(ctypes.c_void_p), ctypes.byref(n))
    assert n.value > 4.9e8
    assert bad == 0


def test_adamw_validation(lib):
    f = lib.qlora_adamw_step
    base = [_p(FAKE), _p(FAKE), 1, _p(FAKE), _p(FAKE), None, 1000, 1e-4, 0.9, 0.999, 1e-8, 0.0,
            1, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)
    assert call(6, -1) == 1             # n < 0
    assert call(12, 0) == 1             # step < 1
    assert call(2, 7) == 4              # grad dtype
    assert call(8, 1.0) == 1            # beta1 outside [0, 1)
    assert call(9, -0.1) == 1           # beta2 outside [0, 1)
    assert call(7, float("nan")) == 1   # lr not finite
    assert call(10, float("inf")) == 1  # eps not finite
    assert call(3, None) == 1           # exp_avg missing
    assert call(1, None) == 1           # grad missing
    assert call(0, _p(FAKE + 4)) == 3   # param misaligned
    assert call(5, _p(FAKE + 8)) == 3   # bf16 copy misaligned
    assert call(6, 0) == 0              # empty: nothing to do
