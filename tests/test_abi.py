"""C ABI of libkda.so on the host (no GPU needed, no kernel is ever launched).

* the library loads and exports every function include/kda.h declares;
* every validation branch returns its documented status before anything is
  enqueued (fake, never-dereferenced pointer values are used, so these cases
  are skipped where a GPU is present);
* the planner and workspace sizing follow their stated rules;
* the Python binding refuses host tensors and a missing library (no fallback).
"""
import ctypes
import os
import re
import subprocess

import pytest

import chunked_gated_delta_13_amd as kda
from chunked_gated_delta_13_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, DEVICE = 0, 1, 2, 3, 4
BF16, F32 = 0, 1


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


@pytest.fixture
def host_only():
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake pointers are only passed where no GPU exists")


def test_header_and_binding_agree():
    assert _declared_functions() == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(kda_\w+)", out))
    for name in _declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_library_has_no_undefined_own_symbols():
    """Every kernel launch stub and internal symbol of libkda is defined in the library
    itself (a missing one would only surface when the library is loaded on a machine with a GPU)."""
    out = subprocess.run(["nm", "-D", "--undefined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    own = [line for line in out.splitlines() if "kda" in line]
    assert not own, own


def test_version_and_status_strings(lib):
    assert lib.kda_abi_version() == 1
    for code in range(5):
        s = lib.kda_status_string(code).decode()
        assert s.startswith("KDA_")
    assert "unknown" in lib.kda_status_string(99).decode()


def _prefill(lib, B=1, T=128, H=2, dk=128, dv=128, chunk=64, dt=BF16, seg=0, nvs=0,
             q=0x10000, k=0x20000, v=0x30000, la=0x40000, beta=0x50000, S0=None, o=0x60000,
             S_T=None, ws=None, ws_bytes=0):
    vp = ctypes.c_void_p
    return lib.kda_chunk_prefill_ex(vp(q), vp(k), vp(v), vp(la), vp(beta), vp(S0), vp(o),
                                    vp(S_T), B, T, H, dk, dv, chunk, dt, seg, nvs, vp(ws),
                                    ws_bytes, None)


BIG = 1 << 40  # fake, well-separated, 16-byte-aligned addresses


def _ptrs(i):
    return BIG * (i + 1)


def _ok_ptrs():
    return dict(q=_ptrs(0), k=_ptrs(1), v=_ptrs(2), la=_ptrs(3), beta=_ptrs(4), o=_ptrs(5))


@pytest.mark.parametrize("kw,expect", [
    (dict(dk=96, dv=96), UNSUPPORTED),
    (dict(dk=128, dv=64), UNSUPPORTED),
    (dict(chunk=48), UNSUPPORTED),
    (dict(B=-1), INVALID),
    (dict(T=-5), INVALID),
    (dict(H=-2), INVALID),
    (dict(dt=7), INVALID),
    (dict(chunk=0), INVALID),
    (dict(seg=100), INVALID),        # not a multiple of the chunk
    (dict(seg=-64), INVALID),
    (dict(nvs=3), INVALID),
    (dict(dk=64, dv=64, nvs=2), INVALID),
])
def test_prefill_shape_validation(lib, kw, expect):
    args = _ok_ptrs()
    args.update(kw)
    assert _prefill(lib, **args) == expect


@pytest.mark.parametrize("field", ["q", "k", "v", "la", "beta", "o"])
def test_prefill_null_pointer(lib, host_only, field):
    args = _ok_ptrs()
    args[field] = None
    assert _prefill(lib, **args) == INVALID


@pytest.mark.parametrize("field", ["q", "k", "v", "la", "o"])
def test_prefill_misaligned_pointer(lib, host_only, field):
    args = _ok_ptrs()
    args[field] += 8
    assert _prefill(lib, **args) == INVALID


def test_prefill_overlaps(lib, host_only):
    args = _ok_ptrs()
    args["o"] = args["q"] + 64          # o overlaps q
    assert _prefill(lib, **args) == INVALID
    args = _ok_ptrs()
    state = 2 * 128 * 128 * 4
    assert _prefill(lib, S0=_ptrs(6), S_T=_ptrs(6) + state // 2, **args) == INVALID
    assert _prefill(lib, S0=_ptrs(6), S_T=args["v"], **args) == INVALID   # S_T over an input


def _split_workspace(bh, n, dk, dv):
    """Bytes of a split's workspace over n segments: transitions and increments of segments
    1 .. n-1 (n - 1 slots each), entry states (n slots), then the transition pass's chunk counts
    (two int32 per (b, h) and segment after the first), padded to 16 bytes."""
    mats = (n - 1) * (dk * dk + dk * dv) + n * dk * dv
    counts = (bh * (n - 1) * 2 * 4 + 15) // 16 * 16
    return bh * mats * 4 + counts


def test_prefill_workspace_required(lib, host_only):
    args = _ok_ptrs()
    need = lib.kda_chunk_prefill_workspace_bytes_ex(1, 8192, 2, 128, 128, 64, BF16, 2048)
    assert need == _split_workspace(2, 4, 128, 128)
    assert _prefill(lib, T=8192, seg=2048, **args) == WORKSPACE
    assert _prefill(lib, T=8192, seg=2048, ws=_ptrs(7), ws_bytes=need - 4, **args) == WORKSPACE


def test_split_unit_count_limit(lib, host_only):
    """A split whose launches would count more than 2^30 units (b, h, segment, slice) is refused
    before anything is enqueued: 2^11 sequences x 2^16 heads (the most B * H allows) in 16
    segments of 64 tokens.  The same shape unsplit is a valid plan."""
    seg = ctypes.c_int(0)
    nvs = ctypes.c_int(0)
    B, H = 1 << 11, 1 << 16
    assert lib.kda_chunk_prefill_workspace_bytes_ex(B, 1024, H, 64, 64, 64, BF16, 64) == 0
    assert _prefill(lib, B=B, T=1024, H=H, dk=64, dv=64, seg=64) == UNSUPPORTED
    assert lib.kda_chunk_prefill_plan(B, 1024, H, 64, 64, 64, BF16, ctypes.byref(seg),
                                      ctypes.byref(nvs)) == OK
    assert seg.value == 1024


def test_prefill_empty_batch_is_noop(lib):
    assert _prefill(lib, B=0, q=None, k=None, v=None, la=None, beta=None, o=None) == OK
    assert _prefill(lib, H=0, q=None, k=None, v=None, la=None, beta=None, o=None) == OK


def _decode(lib, N=2, H=3, dk=128, dv=128, dt=BF16, q=_ptrs(0), k=_ptrs(1), v=_ptrs(2),
            la=_ptrs(3), beta=_ptrs(4), S=_ptrs(5), o=_ptrs(6)):
    vp = ctypes.c_void_p
    return lib.kda_decode_step(vp(q), vp(k), vp(v), vp(la), vp(beta), vp(S), vp(o), N, H, dk, dv,
                               dt, None)


def test_decode_validation(lib, host_only):
    assert _decode(lib, dk=96, dv=96) == UNSUPPORTED
    assert _decode(lib, N=-1) == INVALID
    assert _decode(lib, dt=5) == INVALID
    assert _decode(lib, q=None) == INVALID
    assert _decode(lib, S=_ptrs(5) + 4) == INVALID
    assert _decode(lib, o=_ptrs(5) + 256) == INVALID     # o inside S
    assert _decode(lib, o=_ptrs(2)) == INVALID           # o over v
    assert _decode(lib, N=0, q=None, k=None, v=None, la=None, beta=None, S=None, o=None) == OK


def test_plan_rules(lib):
    seg = ctypes.c_int(0)
    nvs = ctypes.c_int(0)
    # many heads: no split, one column slice per head
    assert lib.kda_chunk_prefill_plan(4, 32768, 56, 128, 128, 64, BF16, ctypes.byref(seg),
                                      ctypes.byref(nvs)) == OK
    assert (seg.value, nvs.value) == (32768, 1)
    # few heads, long sequence (bf16, 8-wave workgroups): segments, one column slice
    assert lib.kda_chunk_prefill_plan(1, 1 << 20, 16, 128, 128, 64, BF16, ctypes.byref(seg),
                                      ctypes.byref(nvs)) == OK
    assert nvs.value == 1 and seg.value % 64 == 0 and seg.value < (1 << 20)
    # the same in fp32 (4-wave workgroups): column slices and segments
    assert lib.kda_chunk_prefill_plan(1, 1 << 20, 16, 128, 128, 32, F32, ctypes.byref(seg),
                                      ctypes.byref(nvs)) == OK
    assert nvs.value == 2 and seg.value % 32 == 0 and seg.value < (1 << 20)
    # short sequence: no split below three minimum segments (max(512, 8 sqrt(T)) tokens each)
    assert lib.kda_chunk_prefill_plan(1, 1500, 1, 128, 128, 64, BF16, ctypes.byref(seg),
                                      ctypes.byref(nvs)) == OK
    assert seg.value == 1500
    assert lib.kda_chunk_prefill_workspace_bytes(1, 1500, 1, 128, 128, 64, BF16) == 0
    # a few thousand tokens on one head: segments of at least the minimum length
    assert lib.kda_chunk_prefill_plan(1, 6000, 1, 128, 128, 64, BF16, ctypes.byref(seg),
                                      ctypes.byref(nvs)) == OK
    assert 8 * 6000 ** 0.5 - 64 <= seg.value < 6000 / 3 and seg.value % 64 == 0


def test_automatic_plan_properties(lib):
    """Over a sweep of shapes the automatic plan keeps its rules: segments are whole chunks of
    equal length (the last one possibly shorter) that cover the sequence; a split has at least 3
    segments, its widest step (every segment at once) fits in fewer workgroups than the 256
    compute units (units * n <= 255), and its segments are not shorter than max(512, 8 sqrt(T));
    shapes that already fill the chip, or are too short, are not split.  The workspace matches
    the plan."""
    import itertools
    import math
    seg = ctypes.c_int(0)
    nvs = ctypes.c_int(0)
    checked = 0
    for B, H, T, d, (dt, chunk) in itertools.product(
            (1, 2, 4), (1, 2, 8, 16, 56), (1, 100, 1000, 1536, 4096, 6000, 12288, 65536, 1 << 20),
            (64, 128), ((BF16, 64), (BF16, 32), (F32, 16), (F32, 32), (F32, 64))):
        assert lib.kda_chunk_prefill_plan(B, T, H, d, d, chunk, dt, ctypes.byref(seg),
                                          ctypes.byref(nvs)) == OK
        L, vs = seg.value, nvs.value
        units = B * H * vs
        ws = lib.kda_chunk_prefill_workspace_bytes(B, T, H, d, d, chunk, dt)
        assert ws == lib.kda_chunk_prefill_workspace_bytes_ex(B, T, H, d, d, chunk, dt, 0)
        lmin = max(512, 8 * math.sqrt(T))
        if L >= T:   # no split
            assert ws == 0
            assert 2 * units > 256 or T < 3 * lmin or min(255 // units, int(T // lmin)) < 3, \
                (B, H, T, d, dt, chunk)
            continue
        n = -(-T // L)
        assert ws == _split_workspace(B * H, n, d, d), (B, H, T, d, dt, chunk, ws)
        assert L % chunk == 0 and L >= lmin - chunk, (B, H, T, d, dt, chunk, L)
        assert n >= 3 and units * n <= 255, (B, H, T, d, dt, chunk, n)
        assert 0 < T - (n - 1) * L <= L, (B, H, T, d, dt, chunk, n, L)
        checked += 1
    assert checked > 20   # the sweep does reach the split branch


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(1, 4, 1, 64, dtype=torch.bfloat16)
    la = torch.zeros(1, 4, 1, 64)
    with pytest.raises(ValueError):
        kda.chunk_prefill(q, q, q, la, torch.zeros(1, 4, 1))
    with pytest.raises(ValueError):
        kda.decode_step(q[:, 0], q[:, 0], q[:, 0], la[:, 0], torch.zeros(1, 1),
                        torch.zeros(1, 1, 64, 64))


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load(str(tmp_path / "libkda.so"))


def _spec(lib, fn, N=2, m=4, H=3, dk=128, dv=128, dt=BF16, q=_ptrs(0), k=_ptrs(1), v=_ptrs(2),
          la=_ptrs(3), beta=_ptrs(4), S=_ptrs(5), last=_ptrs(6)):
    vp = ctypes.c_void_p
    f = getattr(lib, fn)
    return f(vp(q), vp(k), vp(v), vp(la), vp(beta), vp(S), vp(last), N, m, H, dk, dv, dt, None)


@pytest.mark.parametrize("fn", ["kda_spec_verify", "kda_spec_commit"])
def test_spec_validation(lib, host_only, fn):
    assert _spec(lib, fn, m=0) == INVALID
    assert _spec(lib, fn, N=-1) == INVALID
    assert _spec(lib, fn, dk=96, dv=96) == UNSUPPORTED
    assert _spec(lib, fn, dt=4) == INVALID
    assert _spec(lib, fn, S=None) == INVALID
    assert _spec(lib, fn, last=None) == INVALID          # o for verify, accepted for commit
    assert _spec(lib, fn, q=_ptrs(0) + 8) == INVALID     # misaligned
    assert _spec(lib, fn, N=0, q=None, k=None, v=None, la=None, beta=None, S=None, last=None) == OK


def test_spec_commit_state_must_not_overlap_inputs(lib, host_only):
    assert _spec(lib, "kda_spec_commit", S=_ptrs(2) + 64) == INVALID
    assert _spec(lib, "kda_spec_commit", last=_ptrs(5) + 16) == INVALID   # accepted inside S


def _ckpt(lib, every=128, S_ckpt=_ptrs(8), T=1000, chunk=64, **kw):
    args = _ok_ptrs()
    args.update(kw)
    vp = ctypes.c_void_p
    return lib.kda_chunk_prefill_ckpt(vp(args["q"]), vp(args["k"]), vp(args["v"]), vp(args["la"]),
                                      vp(args["beta"]), None, vp(args["o"]), None, 2, T, 3, 128, 128,
                                      chunk, BF16, every, vp(S_ckpt), 0, 0, None, 0, None)


def test_ckpt_validation(lib, host_only):
    assert _ckpt(lib, every=100) == INVALID          # not a multiple of the chunk
    assert _ckpt(lib, every=-64) == INVALID
    assert _ckpt(lib, S_ckpt=None) == INVALID         # T >= every needs the buffer
    assert _ckpt(lib, S_ckpt=_ptrs(8) + 4) == INVALID  # misaligned
    assert _ckpt(lib, S_ckpt=_ptrs(2) + 256) == INVALID   # over v


def _gate(lib, dt=BF16, dk=128, gate=_ptrs(3), nvs=0, **kw):
    args = _ok_ptrs()
    args.update(kw)
    vp = ctypes.c_void_p
    return lib.kda_chunk_prefill_gate(vp(args["q"]), vp(args["k"]), vp(args["v"]), vp(gate), vp(args["beta"]),
                                      None, vp(args["o"]), None, 2, 1000, 3, dk, dk, 64 if dt == BF16 else 32,
                                      dt, 0, nvs, None, 0, None)


def test_gate_validation(lib, host_only):
    assert _gate(lib, dt=F32) == UNSUPPORTED
    assert _gate(lib, dk=64) == UNSUPPORTED
    assert _gate(lib, nvs=2) == UNSUPPORTED
    assert _gate(lib, gate=None) == INVALID
    assert _gate(lib, gate=_ptrs(3) + 2) == INVALID


def test_fp32_chunk64_is_supported(lib):
    """fp32 inputs take every chunk length, 64 included (run as 32-token chunks inside the
    library): the plan and the workspace query accept it, segment lengths are whole 64-token
    chunks, and an explicit segment length must be a multiple of 64."""
    seg = ctypes.c_int(0)
    nvs = ctypes.c_int(0)
    for d in (64, 128):
        assert lib.kda_chunk_prefill_plan(1, 1 << 16, 2, d, d, 64, F32, ctypes.byref(seg),
                                          ctypes.byref(nvs)) == OK
        assert seg.value % 64 == 0 and seg.value < (1 << 16)
        assert lib.kda_chunk_prefill_workspace_bytes(1, 1 << 16, 2, d, d, 64, F32) > 0
        assert lib.kda_chunk_prefill_workspace_bytes_ex(1, 4096, 2, d, d, 64, F32, 1024) == \
            _split_workspace(2, 4, d, d)
    args = _ok_ptrs()
    assert _prefill(lib, dt=F32, chunk=64, seg=96, **args) == INVALID   # not a multiple of 64


def test_spec_long_block_never_needs_workspace(lib, host_only):
    """A drafted block longer than 16 tokens runs as one unsplit chunked prefill, so no length
    asks for a workspace, even where the automatic plan would split a prefill of that many
    tokens (1 sequence, 1 head, 2048 tokens).  Without a GPU the valid call gets as far as the
    launch (KDA_ERR_DEVICE); it never reports a missing workspace or an unsupported length."""
    seg = ctypes.c_int(0)
    nvs = ctypes.c_int(0)
    assert lib.kda_chunk_prefill_plan(1, 2048, 1, 128, 128, 64, BF16, ctypes.byref(seg),
                                      ctypes.byref(nvs)) == OK
    assert seg.value < 2048   # the same shape as a prefill would be split
    for fn in ("kda_spec_verify", "kda_spec_commit"):
        for m, dt in ((2048, BF16), (2048, F32), (40, BF16), (100000, BF16)):
            st = _spec(lib, fn, N=1, m=m, H=1, dt=dt)
            assert st in (OK, DEVICE), (fn, m, dt, st)


def _noalloc(lib, B=1, T=128, H=2, d=128, chunk=64, dt=BF16, seg=0, nvs=0, q=_ptrs(0), k=_ptrs(1),
             v=_ptrs(2), la=_ptrs(3), beta=_ptrs(4), S0=None, o=_ptrs(5), S_T=None):
    vp = ctypes.c_void_p
    return lib.kda_chunk_prefill_noalloc(vp(q), vp(k), vp(v), vp(la), vp(beta), vp(S0), vp(o),
                                         vp(S_T), B, T, H, d, d, chunk, dt, seg, nvs, None)


def test_noalloc_validation(lib, host_only):
    """The allocation-free prefill validates like kda_chunk_prefill_ex and refuses, before
    anything is enqueued, a split whose scratch would exceed its fixed device array."""
    assert _noalloc(lib, d=96) == UNSUPPORTED
    assert _noalloc(lib, B=-1) == INVALID
    assert _noalloc(lib, q=None) == INVALID
    assert _noalloc(lib, o=_ptrs(0) + 64) == INVALID          # o over q
    assert _noalloc(lib, seg=100) == INVALID                  # not a multiple of the chunk
    assert _noalloc(lib, B=0, q=None, k=None, v=None, la=None, beta=None, o=None) == OK
    # 56 heads x 1M tokens in 4096-token segments: about 11 GiB of scratch, over the limit
    need = lib.kda_chunk_prefill_workspace_bytes_ex(1, 1 << 20, 56, 128, 128, 64, BF16, 4096)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    assert _noalloc(lib, T=1 << 20, H=56, seg=4096) == WORKSPACE
    # the 1M-token, 16-head workload fits, on its own 64K segments and on the automatic plan
    assert lib.kda_chunk_prefill_workspace_bytes_ex(1, 1 << 20, 16, 128, 128, 64, BF16,
                                                    1 << 16) <= _lib.NOALLOC_SCRATCH_BYTES
    assert lib.kda_chunk_prefill_workspace_bytes(1, 1 << 20, 16, 128, 128, 64,
                                                 BF16) <= _lib.NOALLOC_SCRATCH_BYTES
