"""The C ABI on the CPU: the library loads, exports every declared symbol, and rejects bad
arguments with the documented status codes before any HIP call (no GPU is touched)."""
import ctypes
import math

import pytest

from tests import _lib

import exact_attention_27_amd as fa


@pytest.fixture(scope="module")
def lib():
    return _lib.ensure_built()


def test_exports_every_declared_symbol(lib):
    declared = _lib.header_functions()
    assert set(declared) == set(fa.EXPORTED_SYMBOLS), declared
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in include/fa.h but not exported"


def test_status_strings(lib):
    for code in (fa.FA_OK, fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED, fa.FA_ERR_HIP):
        s = fa.fa_status_string(code)
        assert s and "unknown" not in s
    assert "unknown" in fa.fa_status_string(99)


# Fake device addresses: never dereferenced, because every call below fails validation
# before anything is enqueued.
A = [0x10000 * (i + 1) * 0x1000 for i in range(10)]


def fwd(lib, q=A[0], k=A[1], v=A[2], o=A[3], lse=A[4], B=1, H=1, N=16, d=64, causal=0, scale=0.125, dtype=0,
        entry="fa_forward"):
    vp = ctypes.c_void_p
    return getattr(lib, entry)(vp(q), vp(k), vp(v), vp(o), vp(lse), B, H, N, d, causal, scale, dtype, vp(0))


def bwd(lib, ptrs=None, B=1, H=1, N=16, d=64, causal=0, scale=0.125, dtype=0):
    vp = ctypes.c_void_p
    p = list(A) if ptrs is None else ptrs
    return lib.fa_backward(*(vp(x) for x in p), B, H, N, d, causal, scale, dtype, vp(0))


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(o=0), fa.FA_ERR_INVALID_ARG),
    (dict(k=A[1] + 8), fa.FA_ERR_INVALID_ARG),          # misaligned
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(H=-1), fa.FA_ERR_INVALID_ARG),
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
    (dict(d=0), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=2), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=math.inf), fa.FA_ERR_INVALID_ARG),
    (dict(scale=math.nan), fa.FA_ERR_INVALID_ARG),
    (dict(o=A[0]), fa.FA_ERR_INVALID_ARG),               # output aliases an input
    (dict(lse=A[0] + 16), fa.FA_ERR_INVALID_ARG),        # lse inside q
    (dict(B=1 << 20, H=1 << 20, N=1 << 20, d=64), fa.FA_ERR_INVALID_ARG),  # size overflow
    (dict(d=100), fa.FA_ERR_UNSUPPORTED),   # not a multiple of 8
    (dict(d=132), fa.FA_ERR_UNSUPPORTED),   # not a multiple of 8
    (dict(d=264), fa.FA_ERR_UNSUPPORTED),   # above 256
    (dict(d=512), fa.FA_ERR_UNSUPPORTED),
])
def test_forward_validation(lib, kw, code):
    assert fwd(lib, **kw) == code
    # the ping-pong forward takes the same arguments and validates them the same way
    assert fwd(lib, entry="fa_forward_pingpong", **{**kw, "d": kw.get("d", 128)}) == code


def test_backward_validation(lib):
    assert bwd(lib, N=0) == fa.FA_ERR_INVALID_ARG
    assert bwd(lib, d=84) == fa.FA_ERR_UNSUPPORTED
    assert bwd(lib, d=320) == fa.FA_ERR_UNSUPPORTED
    assert bwd(lib, scale=math.nan) == fa.FA_ERR_INVALID_ARG
    assert bwd(lib, causal=-1) == fa.FA_ERR_INVALID_ARG
    assert bwd(lib, dtype=7) == fa.FA_ERR_INVALID_ARG
    for i in range(10):  # every pointer is required (delta included)
        p = list(A)
        p[i] = 0
        assert bwd(lib, ptrs=p) == fa.FA_ERR_INVALID_ARG
    p = list(A)
    p[6] = A[0]  # dq aliases q
    assert bwd(lib, ptrs=p) == fa.FA_ERR_INVALID_ARG
    p = list(A)
    p[8] = A[7]  # dv aliases dk
    assert bwd(lib, ptrs=p) == fa.FA_ERR_INVALID_ARG
    p = list(A)
    p[9] = A[2] + 32  # delta misaligned? no: 32 is aligned, but inside v
    assert bwd(lib, ptrs=p) == fa.FA_ERR_INVALID_ARG


def test_stage_validation(lib):
    vp = ctypes.c_void_p
    # preprocess: o, dO, delta
    assert lib.fa_backward_preprocess(vp(0), vp(A[1]), vp(A[2]), 1, 1, 16, 64, 0, vp(0)) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_backward_preprocess(vp(A[0]), vp(A[1]), vp(A[0]), 1, 1, 16, 64, 0, vp(0)) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_backward_preprocess(vp(A[0]), vp(A[1]), vp(A[2]), 1, 1, 16, 52, 0, vp(0)) == fa.FA_ERR_UNSUPPORTED
    # dkv: q k v dO lse delta dk dv
    args = [vp(x) for x in A[:8]]
    assert lib.fa_backward_dkv(*args[:6], vp(0), args[7], 1, 1, 16, 64, 0, 0.1, 0, vp(0)) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_backward_dkv(*args[:6], args[6], args[0], 1, 1, 16, 64, 0, 0.1, 0, vp(0)) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_backward_dkv(*args, 1, 1, 16, 64, 3, 0.1, 0, vp(0)) == fa.FA_ERR_INVALID_ARG
    # dq: q k v dO lse delta dq
    assert lib.fa_backward_dq(*args[:6], args[5], 1, 1, 16, 64, 0, 0.1, 0, vp(0)) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_backward_dq(*args[:6], vp(0), 1, 1, 16, 64, 0, 0.1, 0, vp(0)) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_backward_dq(*args[:7], 1, 1, 16, 64, 0, -0.1, 0, vp(0)) == fa.FA_ERR_INVALID_ARG
    # dq with delta: q k v o dO lse dq delta (o is read, delta written)
    dd = [vp(x) for x in A[:8]]
    assert lib.fa_backward_dq_delta(*dd[:3], vp(0), *dd[4:], 1, 1, 16, 64, 0, 0.1, 0, vp(0)) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_backward_dq_delta(*dd[:7], vp(0), 1, 1, 16, 64, 0, 0.1, 0, vp(0)) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_backward_dq_delta(*dd[:7], dd[3], 1, 1, 16, 64, 0, 0.1, 0, vp(0)) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_backward_dq_delta(*dd, 1, 1, 16, 64, 2, 0.1, 0, vp(0)) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_backward_dq_delta(*dd, 1, 1, 16, 60, 0, 0.1, 0, vp(0)) == fa.FA_ERR_UNSUPPORTED


def test_binding_refuses_cpu_tensors(lib):
    import torch
    q = torch.zeros(1, 1, 16, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa.fa_forward(q, q, q, q.clone(), None, False, 0.125)


def splitkv(lib, q=A[0], k=A[1], v=A[2], o=A[3], lse=A[4], ws=A[5], ws_bytes=1 << 30, splits=2, B=1, H=1, N=16,
            d=64, causal=0, scale=0.125, dtype=0):
    vp = ctypes.c_void_p
    return lib.fa_forward_splitkv(vp(q), vp(k), vp(v), vp(o), vp(lse), B, H, N, d, causal, scale, dtype, splits, vp(ws),
                                  ctypes.c_size_t(ws_bytes), vp(0))


def test_splitkv_workspace_bytes(lib):
    size = fa.fa_forward_splitkv_workspace_bytes
    assert size(2, 3, 100, 64, 4) == 4 * 2 * 3 * 100 * (64 + 2) * 4
    assert size(1, 1, 1, 128, 1) == (128 + 2) * 4
    assert size(1, 1, 16, 64, 0) == 0           # num_splits outside 1..256
    assert size(1, 1, 16, 64, 257) == 0
    assert size(1, 1, 16, 96, 2) == 2 * 16 * (128 + 2) * 4   # d = 96 runs 128 wide
    assert size(1, 1, 16, 32, 2) == 2 * 16 * (64 + 2) * 4    # d = 32 runs 64 wide
    assert size(1, 1, 16, 200, 2) == 2 * 16 * (256 + 2) * 4  # d = 200 runs 256 wide
    assert size(1, 1, 16, 100, 2) == 0          # unsupported head dim
    assert size(1, 1, 16, 264, 2) == 0
    assert size(0, 1, 16, 64, 2) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(splits=0), fa.FA_ERR_INVALID_ARG),
    (dict(splits=257), fa.FA_ERR_INVALID_ARG),
    (dict(ws=0), fa.FA_ERR_INVALID_ARG),
    (dict(ws=A[5] + 4), fa.FA_ERR_INVALID_ARG),                   # misaligned workspace
    (dict(ws_bytes=2 * 16 * (64 + 2) * 4 - 4), fa.FA_ERR_INVALID_ARG),  # one float short
    (dict(ws=A[0] + 64), fa.FA_ERR_INVALID_ARG),                  # workspace inside q
    (dict(ws=A[4]), fa.FA_ERR_INVALID_ARG),                       # workspace aliases lse
    (dict(o=A[1]), fa.FA_ERR_INVALID_ARG),                        # output aliases an input
    (dict(d=260), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=math.nan), fa.FA_ERR_INVALID_ARG),
])
def test_splitkv_validation(lib, kw, code):
    assert splitkv(lib, **kw) == code


# --------------------------------------------------------------- strided / variable-length

def ex_problem(B=2, H=2, N=16, d=64, cu=None, total=0, causal=0, scale=0.125, dtype=0):
    return fa.FAProblem(B, H, N, d, cu, total, causal, scale, dtype)


def bnhd(H=2, N=16, d=64):
    return fa.FAStrides(N * H * d, d, H * d)


def fwd_ex(lib, p=None, ptrs=None, strides=None, lse=A[4]):
    vp = ctypes.c_void_p
    p = ex_problem() if p is None else p
    q, k, v, o = (A[:4] if ptrs is None else ptrs)
    sq, sk, sv, so = ([bnhd()] * 4 if strides is None else strides)
    return lib.fa_forward_ex(ctypes.byref(p), vp(q), sq, vp(k), sk, vp(v), sv, vp(o), so, vp(lse), vp(0))


def bwd_ex(lib, p=None, ptrs=None, strides=None):
    vp = ctypes.c_void_p
    p = ex_problem() if p is None else p
    q, k, v, o, do, lse, dq, dk, dv, delta = (A if ptrs is None else ptrs)
    s = [bnhd()] * 8 if strides is None else strides
    return lib.fa_backward_ex(ctypes.byref(p), vp(q), s[0], vp(k), s[1], vp(v), s[2], vp(o), s[3], vp(do), s[4],
                              vp(lse), vp(dq), s[5], vp(dk), s[6], vp(dv), s[7], vp(delta), vp(0))


@pytest.mark.parametrize("stride,code", [
    (fa.FAStrides(2048, 64, 32), fa.FA_ERR_INVALID_ARG),     # row stride below d
    (fa.FAStrides(2048, 64, 132), fa.FA_ERR_INVALID_ARG),    # not a multiple of 8 elements
    (fa.FAStrides(2048, -64, 128), fa.FA_ERR_INVALID_ARG),   # negative head stride
    (fa.FAStrides(-8, 64, 128), fa.FA_ERR_INVALID_ARG),      # negative batch stride
    (fa.FAStrides(2048, 64, (1 << 23) + 8), fa.FA_ERR_INVALID_ARG),  # row stride above 2^23
    (fa.FAStrides(1 << 61, 64, 128), fa.FA_ERR_INVALID_ARG),  # extent beyond 2^60 elements
])
def test_ex_stride_validation(lib, stride, code):
    for i in range(4):  # every operand's strides are checked
        s = [bnhd()] * 4
        s[i] = stride
        assert fwd_ex(lib, strides=s) == code, i


def test_ex_output_rules(lib):
    # o aliases q with equal strides: refused (exact element test)
    assert fwd_ex(lib, ptrs=[A[0], A[1], A[2], A[0]]) == fa.FA_ERR_INVALID_ARG
    # o interleaved with q inside one (B, N, 2, H, d) buffer shares no element with it, but
    # with strides differing from q's only the address ranges can be compared: refused
    s2 = fa.FAStrides(16 * 2 * 2 * 64, 64, 2 * 2 * 64)
    assert fwd_ex(lib, ptrs=[A[0], A[1], A[2], A[0] + 2 * 64 * 2], strides=[bnhd(), bnhd(), bnhd(), s2]) == \
        fa.FA_ERR_INVALID_ARG
    # an output whose heads coincide (head stride 0 with H = 2) is not injective
    assert fwd_ex(lib, strides=[bnhd()] * 3 + [fa.FAStrides(2048, 0, 128)]) == fa.FA_ERR_INVALID_ARG
    # lse inside an input
    assert fwd_ex(lib, lse=A[1] + 64) == fa.FA_ERR_INVALID_ARG
    # backward: dq and dk the same buffer; delta inside dv
    p = list(A)
    p[7] = p[6]
    assert bwd_ex(lib, ptrs=p) == fa.FA_ERR_INVALID_ARG
    p = list(A)
    p[9] = p[8] + 256
    assert bwd_ex(lib, ptrs=p) == fa.FA_ERR_INVALID_ARG
    # outputs may not overlap inputs even when inputs overlap each other
    p = list(A)
    p[1] = p[2] = p[0]  # q = k = v: allowed for inputs ...
    p[8] = p[0]         # ... but dv on q is not
    assert bwd_ex(lib, ptrs=p) == fa.FA_ERR_INVALID_ARG


def test_ex_problem_validation(lib):
    vp = ctypes.c_void_p
    q, k, v, o = A[:4]
    s = bnhd()
    assert lib.fa_forward_ex(None, vp(q), s, vp(k), s, vp(v), s, vp(o), s, vp(A[4]), vp(0)) == fa.FA_ERR_INVALID_ARG
    assert fwd_ex(lib, p=ex_problem(d=272)) == fa.FA_ERR_UNSUPPORTED  # above 256
    assert fwd_ex(lib, p=ex_problem(d=60)) == fa.FA_ERR_UNSUPPORTED   # not a multiple of 8
    assert fwd_ex(lib, p=ex_problem(N=0)) == fa.FA_ERR_INVALID_ARG
    assert fwd_ex(lib, p=ex_problem(causal=3)) == fa.FA_ERR_INVALID_ARG
    # variable lengths: cu_seqlens misaligned, negative total
    assert fwd_ex(lib, p=ex_problem(cu=A[5] + 4, total=10)) == fa.FA_ERR_INVALID_ARG
    assert fwd_ex(lib, p=ex_problem(cu=A[5], total=-1)) == fa.FA_ERR_INVALID_ARG
    # an empty packed batch validates and enqueues nothing
    assert fwd_ex(lib, p=ex_problem(cu=A[5], total=0)) == fa.FA_OK
    assert bwd_ex(lib, p=ex_problem(cu=A[5], total=0)) == fa.FA_OK


def ex_problem_k(N_k=0, cu_k=None, total_k=0, **kw):
    p = ex_problem(**kw)
    p.N_k, p.cu_seqlens_k, p.total_k = N_k, cu_k, total_k
    return p


def test_ex_key_side_validation(lib):
    assert fwd_ex(lib, p=ex_problem_k(N_k=-1)) == fa.FA_ERR_INVALID_ARG
    assert bwd_ex(lib, p=ex_problem_k(N_k=-1)) == fa.FA_ERR_INVALID_ARG
    assert fwd_ex(lib, p=ex_problem_k(N_k=(1 << 30) + 1)) == fa.FA_ERR_UNSUPPORTED
    # key offsets need query offsets, 16-byte alignment and a non-negative row count
    assert fwd_ex(lib, p=ex_problem_k(cu_k=A[6], total_k=16)) == fa.FA_ERR_INVALID_ARG
    assert fwd_ex(lib, p=ex_problem_k(cu=A[5], total=16, cu_k=A[6] + 4, total_k=16)) == fa.FA_ERR_INVALID_ARG
    assert fwd_ex(lib, p=ex_problem_k(cu=A[5], total=16, cu_k=A[6], total_k=-1)) == fa.FA_ERR_INVALID_ARG
    assert bwd_ex(lib, p=ex_problem_k(cu=A[5], total=16, cu_k=A[6], total_k=-1)) == fa.FA_ERR_INVALID_ARG


def test_ex_key_side_extent(lib):
    # k, v (and dk, dv) span N_k rows: an output placed just past 16 rows of k overlaps a
    # 1000-row k, and a dk placed there overlaps a 1000-row dv
    # (one batch, so only the row count decides whether the byte ranges meet)
    H, N, Nk, d = 2, 16, 1000, 64
    sq, sk = bnhd(H, N, d), bnhd(H, Nk, d)
    past_16_rows = A[1] + N * H * d * 2
    p = ex_problem_k(N_k=Nk, B=1, H=H, N=N, d=d)
    assert fwd_ex(lib, p=p, ptrs=[A[0], A[1], A[2], past_16_rows], strides=[sq, sk, sk, sq]) == fa.FA_ERR_INVALID_ARG
    ptrs = list(A)
    ptrs[7] = A[8] + N * H * d * 2  # dk inside dv
    assert bwd_ex(lib, p=p, ptrs=ptrs, strides=[sq, sk, sk, sq, sq, sq, sk, sk]) == fa.FA_ERR_INVALID_ARG
    # a key-side row stride below d is refused like a query-side one
    assert fwd_ex(lib, p=p, strides=[sq, fa.FAStrides(2048, 64, 32), sk, sq]) == fa.FA_ERR_INVALID_ARG


def splitkv_ex(lib, p, splits=2, ws=A[5], ws_bytes=1 << 30):
    vp = ctypes.c_void_p
    s = bnhd()
    return lib.fa_forward_splitkv_ex(ctypes.byref(p), vp(A[0]), s, vp(A[1]), s, vp(A[2]), s, vp(A[3]), s, vp(A[4]),
                                     splits, vp(ws), ws_bytes, vp(0))


def test_splitkv_ex_workspace_and_validation(lib):
    # bytes: splits * query rows * (kernel width + 2) * 4; query rows are B*H*N, or H*total
    p = ex_problem_k(N_k=4096, B=2, H=2, N=1, d=64)
    assert lib.fa_forward_splitkv_ex_workspace_bytes(ctypes.byref(p), 16) == 16 * 2 * 2 * 1 * (64 + 2) * 4
    p = ex_problem_k(cu=A[5], total=37, cu_k=A[6], total_k=900, N_k=500, B=3, H=2, N=20, d=96)
    assert lib.fa_forward_splitkv_ex_workspace_bytes(ctypes.byref(p), 3) == 3 * 2 * 37 * (128 + 2) * 4
    assert lib.fa_forward_splitkv_ex_workspace_bytes(ctypes.byref(p), 0) == 0
    assert lib.fa_forward_splitkv_ex_workspace_bytes(ctypes.byref(ex_problem_k(N_k=-1)), 2) == 0
    assert lib.fa_forward_splitkv_ex_workspace_bytes(None, 2) == 0
    for splits in (0, 257):
        assert splitkv_ex(lib, ex_problem(), splits=splits) == fa.FA_ERR_INVALID_ARG
    need = lib.fa_forward_splitkv_ex_workspace_bytes(ctypes.byref(ex_problem()), 2)
    assert splitkv_ex(lib, ex_problem(), ws_bytes=need - 4) == fa.FA_ERR_INVALID_ARG
    assert splitkv_ex(lib, ex_problem(), ws=0) == fa.FA_ERR_INVALID_ARG
    assert splitkv_ex(lib, ex_problem(), ws=A[0]) == fa.FA_ERR_INVALID_ARG  # workspace over q
    assert splitkv_ex(lib, ex_problem_k(N_k=-1)) == fa.FA_ERR_INVALID_ARG


def test_binding_requires_one_device():
    """Host logic of the binding: every operand and an explicit stream must sit on q's device
    (a kernel reads all its operands from one GPU). Checked with CPU tensors and a stand-in
    stream object; nothing is launched."""
    import types
    import torch
    cuda0 = torch.device("cuda", 0)
    with pytest.raises(ValueError, match="k is on cpu"):
        fa._one_device(cuda0, k=torch.zeros(1), v=None)
    fa._one_device(torch.device("cpu"), k=torch.zeros(1), v=None, lse=None)  # all on one device: accepted
    with pytest.raises(ValueError, match="the stream is on cuda:1"):
        fa._stream_handle(types.SimpleNamespace(device=torch.device("cuda", 1), cuda_stream=0), cuda0)
    assert fa._stream_handle(types.SimpleNamespace(device=cuda0, cuda_stream=1234), cuda0).value == 1234


def test_noalloc_validation(lib):
    """fa_backward_noalloc refuses bad arguments before any HIP call: a null pointer, a
    non-positive size, and B*H*N beyond its device array (FA_ERR_UNSUPPORTED)."""
    vp = ctypes.c_void_p
    p = [vp(x) for x in A[:9]]
    limit = lib.fa_backward_noalloc_max_rows()
    assert limit == 1 << 22
    for i in range(9):
        q = list(p)
        q[i] = vp(0)
        assert lib.fa_backward_noalloc(*q, 1, 1, 16, 64, 0, 0.125, 0, vp(0)) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_backward_noalloc(*p, 1, 1, 0, 64, 0, 0.125, 0, vp(0)) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_backward_noalloc(*p, 1, 1, limit + 1, 64, 0, 0.125, 0, vp(0)) == fa.FA_ERR_UNSUPPORTED
    assert lib.fa_backward_noalloc(*p, 1 << 16, 1 << 16, 1 << 16, 64, 0, 0.125, 0, vp(0)) == fa.FA_ERR_UNSUPPORTED
