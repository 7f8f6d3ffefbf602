"""The C-ABI library: it loads, exports every entry point the header declares,
and rejects bad arguments with status codes before launching anything (so
these run without a GPU: no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import atomics_bwd_preprocess_amd as ab

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_bwd.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ab.LIB_PATH),
                                reason="libattn_bwd.so not built (run __graft_entry__.build())")

FAKE = 0x10000  # a 16-byte-aligned, never dereferenced address


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:attn_status_t|const char\*|int)\s+(attn_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_boundary():
    assert _declared() == sorted(["attn_fwd", "attn_bwd_preprocess", "attn_bwd",
                                  "attn_bwd_postprocess", "attn_bwd_dkdv", "attn_bwd_dq",
                                  "attn_bwd_split", "attn_bwd_dkv_reduce", "attn_bwd_dsink",
                                  "attn_bwd_dq_delta", "attn_bwd_static",
                                  "attn_bwd_fused_cast",
                                  "attn_status_string", "attn_last_error",
                                  "attn_abi_version"])


def test_library_exports_every_declared_symbol():
    L = ab.lib()
    for name in _declared():
        assert hasattr(L, name), name
    assert ab.attn_abi_version() == 7
    assert ab.MAX_SPLIT == int(re.search(r"#define ATTN_MAX_SPLIT (\d+)", open(HEADER).read()).group(1))
    assert L.attn_status_string(0) == b"ok"
    assert L.attn_status_string(1) == b"invalid argument"


def _shape(**kw):
    base = dict(num_seqs=2, max_seqlen=64, total_tokens=128, hq=4, hkv=2, head_dim=64, causal=1,
                window=0, scale=0.125, dtype=0)
    base.update(kw)
    return ab.Shape(**{k: v for k, v in base.items()})


def _fwd(shape, q=FAKE, k=FAKE, v=FAKE, cu=None, sink=None, o=FAKE, lse=FAKE):
    return ab.lib().attn_fwd(ctypes.byref(shape), q, k, v, cu, sink, o, lse, None)


@pytest.mark.parametrize("kw,status", [
    (dict(hq=3, hkv=2), 1),
    (dict(hkv=0), 1),
    (dict(num_seqs=0), 1),
    (dict(max_seqlen=0), 1),
    (dict(total_tokens=-1), 1),
    (dict(head_dim=96), 2),
    (dict(head_dim=256), 2),
    (dict(dtype=7), 2),
    (dict(causal=0, window=16), 1),
    (dict(window=-1), 1),
    (dict(causal=2), 1),
    (dict(scale=0.0), 1),
    (dict(scale=float("nan")), 1),
    (dict(total_tokens=100), 1),  # dense batch without cu_seqlens needs T = B * N
    (dict(layout=2), 1),
    (dict(layout=1, total_tokens=100), 1),  # [B, H, S, D] needs T = B * S
    (dict(layout=1, max_seqlen=1 << 26, total_tokens=1 << 27, hq=1, hkv=1), 1),  # S * D >= 2^32
])
def test_shape_validation(kw, status):
    assert _fwd(_shape(**kw)) == status
    assert ab.lib().attn_last_error().decode() != ""


def test_pointer_validation():
    s = _shape()
    assert _fwd(s, q=None) == 1
    assert b"q is NULL" in ab.lib().attn_last_error()
    assert _fwd(s, k=FAKE + 8) == 1
    assert b"aligned" in ab.lib().attn_last_error()
    assert _fwd(s, lse=None) == 1
    L = ab.lib()
    # preprocess: sink without dsink
    assert L.attn_bwd_preprocess(ctypes.byref(s), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None,
                                 None) == 1
    assert b"sink and dsink" in L.attn_last_error()
    # backward: missing dv
    assert L.attn_bwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None,
                      None) == 1
    # postprocess: misaligned dq
    assert L.attn_bwd_postprocess(ctypes.byref(s), FAKE, FAKE + 2, None) == 1
    # preprocess: a NULL dq_accum is allowed (no zeroing), a misaligned one is not
    assert L.attn_bwd_preprocess(ctypes.byref(s), FAKE, FAKE, FAKE, None, None, FAKE, FAKE + 4,
                                 None, None) == 1
    assert b"dq_accum" in L.attn_last_error()
    # deterministic passes: missing dv / misaligned dq / missing delta
    assert L.attn_bwd_dkdv(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None,
                           None) == 1
    assert b"dv is NULL" in L.attn_last_error()
    assert L.attn_bwd_dq(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE + 8,
                         None) == 1
    assert b"dq is not 16-byte aligned" in L.attn_last_error()
    assert L.attn_bwd_dq(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE,
                         None) == 1
    assert b"delta is NULL" in L.attn_last_error()
    assert L.attn_bwd_dq(ctypes.byref(_shape(head_dim=96)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                         None, FAKE, None) == 2
    assert L.attn_bwd_postprocess(None, FAKE, FAKE, None) == 1


def test_split_validation():
    s = _shape()
    L = ab.lib()

    def split(nsplit, part=FAKE, dq=FAKE):
        return L.attn_bwd_split(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, dq,
                                part, nsplit, None)

    assert split(0) == 1 and b"nsplit" in L.attn_last_error()
    assert split(17) == 1
    assert split(2, part=None) == 1 and b"dkv_partial is NULL" in L.attn_last_error()
    assert split(2, dq=FAKE + 4) == 1 and b"dq_accum" in L.attn_last_error()
    assert L.attn_bwd_dkv_reduce(ctypes.byref(s), FAKE, 0, FAKE, FAKE, None) == 1
    assert L.attn_bwd_dkv_reduce(ctypes.byref(s), FAKE, 2, FAKE, None, None) == 1
    # a valid empty problem launches nothing
    e = _shape(total_tokens=0)
    assert L.attn_bwd_split(ctypes.byref(e), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                            FAKE, 2, None) == 0
    assert L.attn_bwd_dkv_reduce(ctypes.byref(e), FAKE, 2, FAKE, FAKE, None) == 0


def test_bhsd_layout_rejects_cu_seqlens():
    s = _shape(layout=1)
    assert _fwd(s, cu=FAKE) == 1
    assert b"cu_seqlens must be NULL" in ab.lib().attn_last_error()
    assert _fwd(_shape(layout=1, total_tokens=0, num_seqs=1, max_seqlen=1)) == 1  # T != B * S


def test_shape_struct_matches_the_header():
    # attn_shape_t: eleven 4-byte fields, layout last
    text = open(HEADER).read()
    body = text[text.index("typedef struct {"):text.index("} attn_shape_t;")]
    fields = re.findall(r"^\s*(?:int32_t|float)\s+(\w+);", body, flags=re.M)
    assert fields == [f for f, _ in ab.Shape._fields_]
    assert ctypes.sizeof(ab.Shape) == 4 * len(fields)


def test_empty_problem_launches_nothing():
    # total_tokens = 0 with explicit cu_seqlens: valid, returns OK without a launch.
    s = _shape(total_tokens=0)
    assert _fwd(s, cu=FAKE) == 0
    L = ab.lib()
    assert L.attn_bwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                      None) == 0
    assert L.attn_bwd_postprocess(ctypes.byref(s), FAKE, FAKE, None) == 0
    assert L.attn_bwd_preprocess(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None,
                                 None) == 0
    assert L.attn_bwd_dkdv(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                           None) == 0
    assert L.attn_bwd_dq(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                         None) == 0
    assert L.attn_last_error() == b""


def test_python_binding_rejects_host_tensors():
    import torch

    s = _shape()
    q = torch.zeros(128, 4, 64, dtype=torch.float16)
    with pytest.raises(ab.AttnError):
        ab.attn_bwd_postprocess(s, torch.zeros(128, 4, 64), q)


def test_dsink_rejects_bad_pointers_before_any_launch():
    L, s = ab.lib(), _shape()
    assert L.attn_bwd_dsink(ctypes.byref(s), None, FAKE, FAKE, FAKE, None) == 1
    assert b"lse" in L.attn_last_error()
    assert L.attn_bwd_dsink(ctypes.byref(s), FAKE, FAKE, None, FAKE, None) == 1
    assert L.attn_bwd_dsink(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE + 2, None) == 1
    assert L.attn_bwd_dsink(ctypes.byref(_shape(hq=3, hkv=2)), FAKE, FAKE, FAKE, FAKE, None) == 1


def test_dq_delta_rejects_bad_pointers_before_any_launch():
    L, s = ab.lib(), _shape()
    args = [FAKE] * 9
    for i, name in [(3, b"o"), (7, b"delta"), (8, b"dq")]:
        bad = list(args)
        bad[i] = None
        assert L.attn_bwd_dq_delta(ctypes.byref(s), *bad, None) == 1
        assert name in L.attn_last_error()
    bad = list(args)
    bad[3] = FAKE + 8  # o misaligned
    assert L.attn_bwd_dq_delta(ctypes.byref(s), *bad, None) == 1
    assert L.attn_bwd_dq_delta(ctypes.byref(_shape(head_dim=96)), *args, None) == 2


def test_static_scratch_entry_rejects_before_any_launch():
    L = ab.lib()
    m = re.search(r"#define ATTN_STATIC_SCRATCH_BYTES \((\d+)u \* (\d+)u \* (\d+)u\)",
                  open(HEADER).read())
    assert ab.STATIC_SCRATCH_BYTES == int(m.group(1)) * int(m.group(2)) * int(m.group(3))
    # 4096 tokens x 64 heads x 128 dims x 4 bytes = 128 MiB > the 64 MiB array
    big = _shape(num_seqs=1, max_seqlen=4096, total_tokens=4096, hq=64, hkv=8, head_dim=128)
    args = [FAKE] * 6 + [None] + [FAKE] * 3
    assert L.attn_bwd_static(ctypes.byref(big), *args, None) == 1
    assert b"scratch array" in L.attn_last_error()
    # a missing output is rejected; an empty problem launches nothing
    s = _shape()
    bad = list(args)
    bad[7] = None  # dq
    assert L.attn_bwd_static(ctypes.byref(s), *bad, None) == 1
    assert b"dq is NULL" in L.attn_last_error()
    e = _shape(total_tokens=0)
    assert L.attn_bwd_static(ctypes.byref(e), *args[:6], FAKE, *args[7:], None) == 0


def test_fused_cast_validation():
    L, s = ab.lib(), _shape()
    args = [FAKE] * 6 + [None] + [FAKE] * 5
    bad = list(args)
    bad[8] = None  # counters
    assert L.attn_bwd_fused_cast(ctypes.byref(s), *bad, None) == 1
    assert b"counters is NULL" in L.attn_last_error()
    bad = list(args)
    bad[7] = FAKE + 4  # dq_accum misaligned
    assert L.attn_bwd_fused_cast(ctypes.byref(s), *bad, None) == 1
    e = _shape(total_tokens=0)
    assert L.attn_bwd_fused_cast(ctypes.byref(e), *args[:6], FAKE, *args[7:], None) == 0
    # the counter count follows the header's macro (blocks of 32 query rows, multiple of 4)
    sh = ab.Shape.make(num_seqs=3, max_seqlen=100, total_tokens=300, hq=5, hkv=1, head_dim=64,
                       causal=True, window=0, scale=0.125, dtype="f16")
    assert ab.fused_cast_counters(sh) == 60
