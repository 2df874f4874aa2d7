"""The C-ABI library loads, exports every function include/attn.h declares, and
rejects bad arguments on the host before touching the GPU (CPU only).

No compute call is made here: every call below fails validation, which the
library performs before its first HIP call.
"""

import ctypes
import os
import re

import pytest

import exact_tiled_attention_flashattention_amd as eta

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(eta.LIB_PATH),
                                reason="libattn.so not built (run __graft_entry__.build())")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s+\**([a-z_][a-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("attn_prefill", "attn_prefill_paged", "attn_decode_paged", "kv_append",
              "attn_decode_workspace_bytes",
              "attn_decode_num_splits", "attn_gather_paged", "attn_strerror"):
        assert n in names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(eta.LIB_PATH)
    for n in _declared_functions():
        assert hasattr(lib, n), f"{n} declared in attn.h but not exported"


def test_strerror():
    lib = eta.library()
    assert lib.attn_strerror(0) == b"ok"
    assert b"invalid" in lib.attn_strerror(-1)
    assert b"workspace" in lib.attn_strerror(-3)
    assert lib.attn_strerror(12345) == b"unknown status"


P = ctypes.c_void_p
FAKE = P(0x10000)  # never dereferenced: every call below fails validation first


def _prefill(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, dtype=1, B=1, Hq=4, Hkv=2, Nq=8, Nk=8,
             d=128, scale=0.1, causal=1, q_offset=0)
    a.update(kw)
    return eta.library().attn_prefill(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dtype"], a["B"],
                                      a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"],
                                      a["causal"], a["q_offset"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=6, Hkv=4), eta.ATTN_EINVAL),
    (dict(Hkv=0), eta.ATTN_EINVAL),
    (dict(B=-1), eta.ATTN_EINVAL),
    (dict(Nk=-3), eta.ATTN_EINVAL),
    (dict(scale=0.0), eta.ATTN_EINVAL),
    (dict(scale=float("nan")), eta.ATTN_EINVAL),
    (dict(scale=-1.0), eta.ATTN_EINVAL),
    (dict(q_offset=(1 << 30) + 1), eta.ATTN_EINVAL),
    (dict(q_offset=-(1 << 30) - 1), eta.ATTN_EINVAL),
    (dict(d=96), eta.ATTN_EUNSUPPORTED),
    (dict(dtype=7), eta.ATTN_EUNSUPPORTED),
    (dict(q=None), eta.ATTN_EINVAL),
    (dict(k=None), eta.ATTN_EINVAL),
    (dict(q=P(0x10004)), eta.ATTN_EINVAL),  # not 16-byte aligned
])
def test_prefill_rejects(kw, code):
    assert code != eta.ATTN_OK  # a passing call would launch on fake pointers
    assert _prefill(**kw) == code


def test_prefill_empty_is_ok_without_gpu_work():
    assert _prefill(B=0) == eta.ATTN_OK
    assert _prefill(Nq=0) == eta.ATTN_OK


def _decode(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=None, mb=0, nb=0, sl=FAKE, o=FAKE, lse=None, dtype=1, B=2,
             Hq=32, Hkv=8, Nq=4, d=128, scale=0.1, causal=1, L=4096, S=0, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return eta.library().attn_decode_paged(a["q"], a["k"], a["v"], a["bt"], a["mb"], a["nb"],
                                           a["sl"], a["o"], a["lse"], a["dtype"], a["B"], a["Hq"],
                                           a["Hkv"], a["Nq"], a["d"], a["scale"], a["causal"],
                                           a["L"], a["S"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=0), eta.ATTN_EUNSUPPORTED),       # fp32 decode not built
    (dict(Nq=17), eta.ATTN_EUNSUPPORTED),         # 4 heads x 17 rows > 64
    (dict(d=80), eta.ATTN_EUNSUPPORTED),
    (dict(Hq=30), eta.ATTN_EINVAL),
    (dict(L=-1), eta.ATTN_EINVAL),
    (dict(S=-2), eta.ATTN_EINVAL),
    (dict(sl=None), eta.ATTN_EINVAL),
    (dict(bt=FAKE, mb=0), eta.ATTN_EINVAL),
    (dict(ws=None), eta.ATTN_EWORKSPACE),
    (dict(wsb=16), eta.ATTN_EWORKSPACE),
    (dict(scale=float("inf")), eta.ATTN_EINVAL),
])
def test_decode_rejects(kw, code):
    assert code != eta.ATTN_OK
    assert _decode(**kw) == code


def test_worker_plan_and_workspace_size():
    lib = eta.library()
    # default: a few workers per CU (256 CUs when no device can be queried,
    # as here); an explicit count is rounded down to a multiple of Hkv
    w = lib.attn_decode_num_splits(16, 32, 8, 1, 128, 32768, 0)
    assert w > 0 and w % 8 == 0
    assert lib.attn_decode_num_splits(1, 32, 8, 1, 128, 100, 3) == 8
    assert lib.attn_decode_num_splits(1, 32, 8, 1, 128, 100, 20) == 16
    assert lib.attn_decode_num_splits(1, 32, 2, 1, 128, 100, 7) == 6
    # more than 16 rows per K/V head: groups of 16 rows, workers a multiple of Hkv * groups
    assert lib.attn_decode_num_splits(1, 32, 4, 4, 128, 100, 20) == 16   # G*Nq = 32: 2 groups
    assert lib.attn_decode_num_splits(1, 16, 1, 4, 128, 100, 7) == 4     # G*Nq = 64: 4 groups
    assert lib.attn_decode_num_splits(1, 32, 8, 16, 128, 1000, 0) > 0     # G*Nq = 64
    assert lib.attn_decode_num_splits(1, 32, 8, 17, 128, 1000, 0) == eta.ATTN_EUNSUPPORTED
    # pieces = workers + B*Hkv; [pieces*M*d f32][pieces*M f32][(B+1) int64], 256-byte aligned
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    pieces = 96 + 16 * 8  # 100 requested -> 12 per K/V head
    M = 4
    want = up(pieces * M * 128 * 4) + up(pieces * M * 4) + 17 * 8
    assert lib.attn_decode_workspace_bytes(16, 32, 8, 1, 128, 32768, 100) == want
    assert lib.attn_decode_workspace_bytes(16, 32, 8, 17, 128, 32768, 0) == 0
    # G*Nq = 32 rows: pieces of 16 rows, virtual heads = Hkv * 2
    pieces = 96 + 16 * 16
    want = up(pieces * 16 * 128 * 4) + up(pieces * 16 * 4) + 17 * 8
    assert lib.attn_decode_workspace_bytes(16, 32, 8, 8, 128, 32768, 100) == want


def test_kv_append_and_gather_reject():
    lib = eta.library()
    # Hkv = 0
    assert lib.kv_append(FAKE, FAKE, FAKE, FAKE, None, 0, 0, FAKE, 1, 1, 0, 1, 128, 16, None) == -1
    # unsupported d
    assert lib.kv_append(FAKE, FAKE, FAKE, FAKE, None, 0, 0, FAKE, 1, 1, 2, 1, 48, 16, None) == -2
    # missing cache_lens
    assert lib.kv_append(FAKE, FAKE, FAKE, FAKE, None, 0, 0, None, 1, 1, 2, 1, 128, 16, None) == -1
    # paged without a table width
    assert lib.attn_gather_paged(FAKE, FAKE, 0, 4, FAKE, FAKE, 1, 1, 2, 128, 16, None) == -1
    # nothing to do
    assert lib.kv_append(FAKE, FAKE, FAKE, FAKE, None, 0, 0, FAKE, 1, 0, 2, 1, 128, 16, None) == 0


def _prefill_paged(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=None, mb=0, nb=0, sl=FAKE, o=FAKE, lse=None, dtype=1, B=2,
             Hq=32, Hkv=8, Nq=512, d=128, scale=0.1, causal=1, L=4096)
    a.update(kw)
    return eta.library().attn_prefill_paged(a["q"], a["k"], a["v"], a["bt"], a["mb"], a["nb"],
                                            a["sl"], a["o"], a["lse"], a["dtype"], a["B"], a["Hq"],
                                            a["Hkv"], a["Nq"], a["d"], a["scale"], a["causal"],
                                            a["L"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=0), eta.ATTN_EUNSUPPORTED),       # fp32 cache prefill not built
    (dict(d=80), eta.ATTN_EUNSUPPORTED),
    (dict(Hkv=1 << 20), eta.ATTN_EINVAL),         # Hq % Hkv != 0
    (dict(Hq=30), eta.ATTN_EINVAL),
    (dict(L=-1), eta.ATTN_EINVAL),
    (dict(Nq=-1), eta.ATTN_EINVAL),
    (dict(sl=None), eta.ATTN_EINVAL),
    (dict(q=None), eta.ATTN_EINVAL),
    (dict(bt=FAKE, mb=0), eta.ATTN_EINVAL),
    (dict(bt=FAKE, mb=4, nb=-1), eta.ATTN_EINVAL),
    (dict(scale=float("nan")), eta.ATTN_EINVAL),
    (dict(scale=-1.0), eta.ATTN_EINVAL),
    (dict(q=P(0x10002)), eta.ATTN_EINVAL),        # misaligned
    (dict(Hq=(1 << 19), Hkv=(1 << 19)), eta.ATTN_EUNSUPPORTED),  # 16*Hkv*d*2 >= 2^31
])
def test_prefill_paged_rejects(kw, code):
    assert _prefill_paged(**kw) == code


def test_prefill_paged_empty_is_a_no_op():
    # nothing to compute: returns before touching any (fake) pointer
    assert _prefill_paged(B=0) == eta.ATTN_OK
    assert _prefill_paged(Nq=0) == eta.ATTN_OK


def test_prefill_rejects_key_counts_past_32_bit_offsets():
    lib = eta.library()
    st = lib.attn_prefill(FAKE, FAKE, FAKE, FAKE, None, 1, 1, 8, 8, 16, (1 << 22) + 1, 128, 0.1, 1,
                          0, None)
    assert st == eta.ATTN_EUNSUPPORTED


def _decode_fp8(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, bt=None, mb=0, nb=0, sl=FAKE, o=FAKE,
             lse=None, B=2, Hq=32, Hkv=8, Nq=4, d=128, scale=0.1, causal=1, L=4096, S=0, ws=FAKE,
             wsb=1 << 30)
    a.update(kw)
    return eta.library().attn_decode_paged_fp8(
        a["q"], a["k"], a["v"], a["ks"], a["vs"], a["bt"], a["mb"], a["nb"], a["sl"], a["o"],
        a["lse"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["d"], a["scale"], a["causal"], a["L"],
        a["S"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(ks=None), eta.ATTN_EINVAL),
    (dict(vs=None), eta.ATTN_EINVAL),
    (dict(ks=P(0x10002)), eta.ATTN_EINVAL),   # misaligned scale array
    (dict(d=80), eta.ATTN_EUNSUPPORTED),
    (dict(Nq=17), eta.ATTN_EUNSUPPORTED),     # 4 heads x 17 rows > 64
    (dict(ws=None), eta.ATTN_EWORKSPACE),
    (dict(scale=0.0), eta.ATTN_EINVAL),
])
def test_decode_fp8_rejects(kw, code):
    assert _decode_fp8(**kw) == code


def _append_fp8(**kw):
    a = dict(kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, ks=FAKE, vs=FAKE, bt=None, mb=0, nb=0, cl=FAKE,
             B=2, Hkv=8, Nnew=4, d=128, L=4096)
    a.update(kw)
    return eta.library().kv_append_fp8(a["kn"], a["vn"], a["kc"], a["vc"], a["ks"], a["vs"],
                                       a["bt"], a["mb"], a["nb"], a["cl"], a["B"], a["Hkv"],
                                       a["Nnew"], a["d"], a["L"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(ks=None), eta.ATTN_EINVAL),
    (dict(vs=P(0x10001)), eta.ATTN_EINVAL),
    (dict(kc=None), eta.ATTN_EINVAL),
    (dict(d=96), eta.ATTN_EUNSUPPORTED),
    (dict(cl=None), eta.ATTN_EINVAL),
    (dict(bt=FAKE, mb=0), eta.ATTN_EINVAL),
])
def test_append_fp8_rejects(kw, code):
    assert _append_fp8(**kw) == code


def test_fp8_entries_with_nothing_to_do():
    assert _append_fp8(B=0) == eta.ATTN_OK
    assert _decode_fp8(Nq=0) == eta.ATTN_OK


def _bwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, dout=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
             dtype=1, B=1, Hq=4, Hkv=2, Nq=8, Nk=8, d=128, scale=0.1, causal=1, q_offset=0,
             ws=FAKE, ws_bytes=1 << 20)
    a.update(kw)
    lib = eta.library()
    return lib.attn_prefill_backward(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"],
                                     a["dk"], a["dv"], a["dtype"], a["B"], a["Hq"], a["Hkv"],
                                     a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"],
                                     a["q_offset"], a["ws"], a["ws_bytes"], None)


def test_backward_rejects_bad_arguments():
    assert _bwd(Hq=3, Hkv=2) == eta.ATTN_EINVAL
    assert _bwd(scale=0.0) == eta.ATTN_EINVAL
    assert _bwd(scale=float("nan")) == eta.ATTN_EINVAL
    assert _bwd(dtype=0) == eta.ATTN_EUNSUPPORTED      # fp32 backward is not built
    assert _bwd(d=96) == eta.ATTN_EUNSUPPORTED
    assert _bwd(q=None) == eta.ATTN_EINVAL
    assert _bwd(dk=None) == eta.ATTN_EINVAL
    assert _bwd(lse=None) == eta.ATTN_EINVAL
    assert _bwd(q=P(0x10008)) == eta.ATTN_EINVAL          # not 16-byte aligned
    assert _bwd(ws=None) == eta.ATTN_EWORKSPACE
    assert _bwd(ws_bytes=16) == eta.ATTN_EWORKSPACE
    assert _bwd(B=-1) == eta.ATTN_EINVAL
    assert _bwd(B=0) == eta.ATTN_OK                       # nothing to do, nothing enqueued


def test_backward_workspace_size():
    lib = eta.library()
    f = lib.attn_prefill_backward_workspace_bytes
    # D and the base-2 LSE of every row alone when every K/V head's group fits
    # one workgroup (MHA, or enough work)
    assert f(1, 8, 8, 4096, 4096, 128, 1, 0) == 2 * 8 * 4096 * 4
    assert f(1, 32, 8, 32768, 32768, 128, 1, 0) == 2 * 32 * 32768 * 4
    # the 4k causal GQA workload shares each group between workgroups: D plus
    # the fp32 partial sums of dK and dV for every share
    n = f(1, 32, 8, 4096, 4096, 128, 1, 0)
    extra = n - 2 * 32 * 4096 * 4
    plane = 8 * 4096 * 128 * 4
    assert extra > 0 and extra % (2 * plane) == 0 and extra // (2 * plane) in (2, 4)
    assert f(1, 1, 1, 1, 1, 64, 0, 0) == 512
    assert f(-1, 1, 1, 1, 1, 64, 0, 0) == 0
    assert f(1, 4, 3, 1, 1, 64, 0, 0) == 0          # Hq % Hkv != 0
    assert f(1, 4, 2, 1, 1, 96, 0, 0) == 0          # head dim not built


def test_prefill_width_override_rejects():
    lib = eta.library()
    args = [FAKE, FAKE, FAKE, FAKE, None, 1, 1, 4, 2, 8, 8, 128, ctypes.c_float(0.1), 1, 0]
    assert lib.attn_prefill_waves(*args, 5, None) == eta.ATTN_EINVAL
    args_f32 = list(args)
    args_f32[5] = 0
    assert lib.attn_prefill_waves(*args_f32, 8, None) == eta.ATTN_EINVAL
    assert lib.attn_prefill_paged_waves(FAKE, FAKE, FAKE, FAKE, 4, 10, FAKE, FAKE, None, 1, 1, 4,
                                        2, 8, 128, ctypes.c_float(0.1), 1, 64, 6,
                                        None) == eta.ATTN_EINVAL


def test_prefill_width_choice_on_the_host():
    # with no device to query the library assumes 256 compute units
    lib = eta.library()
    assert lib.attn_prefill_workgroup_waves(1, 1, 32, 8, 4096, 1) == 8
    assert lib.attn_prefill_workgroup_waves(1, 1, 32, 8, 2048, 1) == 4
    assert lib.attn_prefill_workgroup_waves(1, 1, 32, 8, 2048, 0) == 8
    assert lib.attn_prefill_workgroup_waves(1, 1, 8, 2, 300, 1) == 4
    assert lib.attn_prefill_workgroup_waves(0, 1, 32, 8, 4096, 1) == eta.ATTN_EUNSUPPORTED
    assert lib.attn_prefill_workgroup_waves(1, 1, 6, 4, 4096, 1) == eta.ATTN_EINVAL


def test_noalloc_decode_rejects_before_any_device_call():
    lib = eta.library()
    f = ctypes.c_float(0.1)
    # a call that would need more than the library's static array
    big = lib.attn_decode_paged_noalloc(FAKE, FAKE, FAKE, FAKE, 8, 100000, FAKE, FAKE, None, 1,
                                        400, 32, 8, 4, 128, f, 1, 4096, 0, None)
    assert big == eta.ATTN_EWORKSPACE
    assert eta.attn_decode_workspace_bytes(400, 32, 8, 4, 128, 4096) > eta.NOALLOC_SCRATCH_BYTES
    # the usual argument checks come first
    assert lib.attn_decode_paged_noalloc(FAKE, FAKE, FAKE, FAKE, 8, 100, FAKE, FAKE, None, 1, 4,
                                         6, 4, 1, 128, f, 1, 128, 0, None) == eta.ATTN_EINVAL
    assert lib.attn_decode_paged_noalloc(FAKE, FAKE, FAKE, FAKE, 8, 100, FAKE, FAKE, None, 0, 4,
                                         8, 2, 1, 128, f, 1, 128, 0, None) == eta.ATTN_EUNSUPPORTED
    # nothing to do: no device is touched
    assert lib.attn_decode_paged_noalloc(None, None, None, None, 0, 0, None, None, None, 1, 0, 8,
                                         2, 1, 128, f, 1, 128, 0, None) == eta.ATTN_OK
