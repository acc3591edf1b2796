"""The C ABI without a GPU: libspla.so loads, exports every function that
include/spla.h declares under its C name, and the host-side validation returns
the documented status codes before anything is launched.  Device pointers
here are never dereferenced: every call below is rejected (or completes) on
the host, ahead of any HIP call."""
import ctypes
import os
import re

import pytest

import block_sparse_linear_amd as bsl
from block_sparse_linear_amd import SplaBuffers, SplaConfig, SplaDecodeAux, load_library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spla.h")

OK, INVALID, UNSUPPORTED, CAPACITY, ALIGN, HIPERR, STATE, SCRATCH = range(8)
FAKE = 0x7F0000000000  # 256-byte aligned stand-in for a device address


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(spla_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return load_library()


def cfg(**kw):
    base = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=64, top_k=16,
                max_blocks_per_seq=40, num_pages=80, kv_dtype=1)
    base.update(kw)
    return SplaConfig(*[base[n] for n, _ in SplaConfig._fields_])


def create(lib, c):
    h = ctypes.c_void_p()
    st = lib.spla_create(ctypes.byref(c), ctypes.byref(h))
    return st, h


def buffers(ws_bytes, **override):
    b = SplaBuffers()
    for i, (n, _) in enumerate(SplaBuffers._fields_[:-1]):
        setattr(b, n, FAKE + i * (1 << 30))
    b.workspace_bytes = ws_bytes
    for k, v in override.items():
        setattr(b, k, v)
    return b


def i32(vals):
    return (ctypes.c_int32 * max(1, len(vals)))(*vals)


def bound(lib, lens=(100, 2000), **kw):
    c = cfg(**kw)
    st, h = create(lib, c)
    assert st == OK
    ws = lib.spla_workspace_bytes(h)
    assert lib.spla_bind(h, ctypes.byref(buffers(ws)), i32(list(lens))) == OK
    return h, c


def lens_of(lib, h, n):
    out = i32([0] * n)
    assert lib.spla_get_lens(h, out) == OK
    return list(out)[:n]


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("spla_create", "spla_bind", "spla_append_kv", "spla_decode", "spla_decode_step", "spla_destroy"):
        assert n in names
    assert sorted(bsl.EXPORTED) == names


def test_library_exports_every_declared_function(lib):
    # a C++-mangled name would not be found under its plain C name
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_abi_version_matches_header(lib):
    m = re.search(r"#define\s+SPLA_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert lib.spla_abi_version() == int(m.group(1))


def test_status_strings(lib):
    strs = [lib.spla_status_str(i).decode() for i in range(8)]
    assert all(strs) and len(set(strs)) == 8
    assert lib.spla_status_str(99).decode() == "unknown status"


@pytest.mark.parametrize("kw,expect", [
    ({}, OK),
    (dict(kv_dtype=0, head_dim=64, block_size=128), OK),
    (dict(n_q_heads=64, n_kv_heads=8), OK),                      # r = 8
    (dict(batch=256), OK),
    (dict(top_k=256), OK),
    (dict(top_k=2), OK),
    (dict(max_blocks_per_seq=16386), OK),
    (dict(batch=0), INVALID),
    (dict(num_pages=0), INVALID),
    (dict(top_k=0), INVALID),
    (dict(batch=257), UNSUPPORTED),
    (dict(head_dim=96), UNSUPPORTED),
    (dict(block_size=32), UNSUPPORTED),
    (dict(n_q_heads=6, n_kv_heads=4), UNSUPPORTED),              # not a multiple
    (dict(n_q_heads=48, n_kv_heads=2), UNSUPPORTED),             # r = 24
    (dict(top_k=1), UNSUPPORTED),
    (dict(top_k=257), UNSUPPORTED),
    (dict(max_blocks_per_seq=16387), UNSUPPORTED),
    (dict(kv_dtype=2), UNSUPPORTED),
])
def test_create_validation(lib, kw, expect):
    st, h = create(lib, cfg(**kw))
    assert st == expect
    assert (h.value is not None) == (expect == OK)
    if h.value:
        lib.spla_destroy(h)


def test_create_null_arguments(lib):
    h = ctypes.c_void_p()
    assert lib.spla_create(None, ctypes.byref(h)) == INVALID
    assert lib.spla_create(ctypes.byref(cfg()), None) == INVALID
    lib.spla_destroy(None)  # no-op


def test_sizes(lib):
    c = cfg(batch=3, n_kv_heads=2, n_q_heads=8, head_dim=64, max_blocks_per_seq=130, top_k=20)
    st, h = create(lib, c)
    assert st == OK
    n_tiles = -(-130 // 64)
    assert lib.spla_stats_floats(h) == 3 * 2 * n_tiles * 64 * 64
    # error word + the one-kernel step's counters (256 lines of 128 bytes) +
    # scores + two index lists + per-head partial records (acc and o_tilde,
    # then their m, l, sum_w, pad headers in an array of their own) + the
    # phi(q)^T S_all and phi(q).z partials of the d * d / 1024 row chunks +
    # phi(q) as bf16 hi / lo, each part rounded up to 256 bytes
    chunks = 64 * 64 // 1024
    need = (256 + 256 * 128 + 3 * 2 * n_tiles * 64 * 4 + 2 * 3 * 2 * 20 * 4 + 3 * 8 * 20 * 2 * 64 * 4
            + 3 * 8 * 20 * 4 * 4 + 3 * 8 * chunks * 64 * 4 + 3 * 8 * chunks * 4 + 3 * 8 * 2 * 64 * 2)
    ws = lib.spla_workspace_bytes(h)
    assert need <= ws <= need + 8 * 256 and ws % 256 == 0
    assert lib.spla_workspace_bytes(None) == 0 and lib.spla_stats_floats(None) == 0
    lib.spla_destroy(h)


def test_bind_validation(lib):
    st, h = create(lib, cfg())
    ws = lib.spla_workspace_bytes(h)
    assert lib.spla_bind(h, None, None) == INVALID
    assert lib.spla_bind(h, ctypes.byref(buffers(ws, s_all=None)), None) == INVALID
    assert lib.spla_bind(h, ctypes.byref(buffers(ws, z_all=FAKE + 8)), None) == ALIGN
    assert lib.spla_bind(h, ctypes.byref(buffers(ws - 1)), None) == INVALID
    cap = 40 * 64
    assert lib.spla_bind(h, ctypes.byref(buffers(ws)), i32([cap + 1, 0])) == INVALID
    assert lib.spla_bind(h, ctypes.byref(buffers(ws)), i32([-1, 0])) == INVALID
    assert lib.spla_bind(h, ctypes.byref(buffers(ws)), i32([cap, 7])) == OK
    assert lens_of(lib, h, 2) == [cap, 7]
    assert lib.spla_bind(h, ctypes.byref(buffers(ws)), None) == OK
    assert lens_of(lib, h, 2) == [0, 0]
    lib.spla_destroy(h)


def test_unbound_handle_is_rejected(lib):
    st, h = create(lib, cfg())
    gate = q = out = ctypes.c_void_p(FAKE)
    assert lib.spla_append_kv(h, 1, i32([0]), i32([1]), FAKE, FAKE, None) == STATE
    assert lib.spla_decode(h, q, gate, out, None, None) == STATE
    assert lib.spla_decode_step(h, FAKE, FAKE, q, gate, out, None, None) == STATE
    lib.spla_destroy(h)


def test_append_validation_leaves_mirror_unchanged(lib):
    h, c = bound(lib)
    cap = c.max_blocks_per_seq * c.block_size
    cases = [
        ((2, [0, 0], [1, 1]), INVALID),          # duplicate sequence
        ((1, [2], [1]), INVALID),                # sequence out of range
        ((1, [-1], [1]), INVALID),
        ((1, [0], [-3]), INVALID),               # negative count
        ((3, [0, 1, 0], [1, 1, 1]), INVALID),    # more entries than the batch
        ((-1, [0], [1]), INVALID),
        ((1, [1], [cap - 2000 + 1]), CAPACITY),
        ((2, [0, 1], [1, cap]), CAPACITY),
    ]
    for (n, ids, cnt), expect in cases:
        assert lib.spla_append_kv(h, n, i32(ids), i32(cnt), FAKE, FAKE, None) == expect, (n, ids, cnt)
        assert lens_of(lib, h, 2) == [100, 2000]
    # nothing to do: accepted without a launch
    assert lib.spla_append_kv(h, 0, None, None, None, None, None) == OK
    assert lib.spla_append_kv(h, 2, i32([0, 1]), i32([0, 0]), None, None, None) == OK
    assert lens_of(lib, h, 2) == [100, 2000]
    # rows present but no K/V pointer, or misaligned ones
    assert lib.spla_append_kv(h, 1, i32([0]), i32([4]), None, FAKE, None) == INVALID
    assert lib.spla_append_kv(h, 1, i32([0]), i32([4]), FAKE + 2, FAKE, None) == ALIGN
    assert lens_of(lib, h, 2) == [100, 2000]
    lib.spla_destroy(h)


def test_decode_validation(lib):
    h, c = bound(lib, lens=(0, 500))
    P = ctypes.c_void_p
    # an empty sequence cannot be decoded
    assert lib.spla_decode(h, P(FAKE), P(FAKE), P(FAKE), None, None) == INVALID
    lib.spla_destroy(h)

    h, c = bound(lib, lens=(64, 500))
    assert lib.spla_decode(h, None, P(FAKE), P(FAKE), None, None) == INVALID
    assert lib.spla_decode(h, P(FAKE + 4), P(FAKE), P(FAKE), None, None) == ALIGN
    aux = SplaDecodeAux()
    aux.o_rla = FAKE + 8
    assert lib.spla_decode(h, P(FAKE), P(FAKE), P(FAKE), ctypes.byref(aux), None) == ALIGN
    aux = SplaDecodeAux()
    aux.kernel_events = FAKE
    aux.n_kernel_events = -1
    assert lib.spla_decode(h, P(FAKE), P(FAKE), P(FAKE), ctypes.byref(aux), None) == INVALID
    # the fused step takes no selection override, needs k / v, and checks capacity
    aux = SplaDecodeAux()
    aux.sel_in = FAKE
    assert lib.spla_decode_step(h, FAKE, FAKE, P(FAKE), P(FAKE), P(FAKE), ctypes.byref(aux), None) == INVALID
    assert lib.spla_decode_step(h, None, FAKE, P(FAKE), P(FAKE), P(FAKE), None, None) == INVALID
    assert lib.spla_decode_step(h, FAKE, FAKE + 6, P(FAKE), P(FAKE), P(FAKE), None, None) == ALIGN
    assert lens_of(lib, h, 2) == [64, 500]
    lib.spla_destroy(h)

    cap = 40 * 64
    h, c = bound(lib, lens=(cap, 1))
    assert lib.spla_decode_step(h, FAKE, FAKE, P(FAKE), P(FAKE), P(FAKE), None, None) == CAPACITY
    assert lens_of(lib, h, 2) == [cap, 1]
    lib.spla_destroy(h)


def test_decode_step_noalloc_validation(lib):
    # the no-alloc step validates like spla_decode_step, on the host, before
    # it looks up its static scratch (no HIP call in any of these)
    P = ctypes.c_void_p
    h, c = bound(lib, lens=(64, 500))
    aux = SplaDecodeAux()
    aux.sel_in = FAKE
    f = lib.spla_decode_step_noalloc
    assert f(None, FAKE, FAKE, P(FAKE), P(FAKE), P(FAKE), None, None) == INVALID
    assert f(h, FAKE, FAKE, P(FAKE), P(FAKE), P(FAKE), ctypes.byref(aux), None) == INVALID
    assert f(h, None, FAKE, P(FAKE), P(FAKE), P(FAKE), None, None) == INVALID
    assert f(h, FAKE, FAKE, None, P(FAKE), P(FAKE), None, None) == INVALID
    assert f(h, FAKE, FAKE + 6, P(FAKE), P(FAKE), P(FAKE), None, None) == ALIGN
    assert lens_of(lib, h, 2) == [64, 500]
    lib.spla_destroy(h)
    st, h = create(lib, cfg())
    assert f(h, FAKE, FAKE, P(FAKE), P(FAKE), P(FAKE), None, None) == STATE
    lib.spla_destroy(h)
    h, c = bound(lib, lens=(40 * 64, 1))
    assert f(h, FAKE, FAKE, P(FAKE), P(FAKE), P(FAKE), None, None) == CAPACITY
    lib.spla_destroy(h)
    # a configuration whose per-call scratch exceeds the static array
    big = dict(batch=256, n_q_heads=32, n_kv_heads=8, top_k=64, max_blocks_per_seq=100, num_pages=100)
    h, c = bound(lib, lens=[300] * 256, **big)
    assert lib.spla_workspace_bytes(h) > bsl.NOALLOC_SCRATCH_BYTES
    assert f(h, FAKE, FAKE, P(FAKE), P(FAKE), P(FAKE), None, None) == SCRATCH
    assert lens_of(lib, h, 256) == [300] * 256
    lib.spla_destroy(h)
    m = re.search(r"#define\s+SPLA_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", open(HEADER).read())
    assert int(m.group(1)) << int(m.group(2)) == bsl.NOALLOC_SCRATCH_BYTES


def test_binding_raises_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        load_library(str(tmp_path / "libspla.so"))


def test_last_hip_error_starts_clear(lib):
    st, h = create(lib, cfg())
    name = ctypes.c_char_p()
    assert lib.spla_last_hip_error(h, ctypes.byref(name)) == 0
    assert name.value == b"hipSuccess"
    assert lib.spla_last_hip_error(None, None) == 0
    lib.spla_destroy(h)


def test_tuning_validation(lib):
    st, h = create(lib, cfg())
    assert lib.spla_set_tuning(h, 0, -1) == OK
    assert lib.spla_set_tuning(h, 0, 0) == OK
    assert lib.spla_set_tuning(h, 0, 1) == OK
    assert lib.spla_set_tuning(h, 0, 2) == INVALID
    for v in (-1, 0, 1):
        assert lib.spla_set_tuning(h, 1, v) == OK
    assert lib.spla_set_tuning(h, 1, 2) == INVALID and lib.spla_set_tuning(h, 1, -2) == INVALID
    for v in (-1, 0, 1):
        assert lib.spla_set_tuning(h, 2, v) == OK
    assert lib.spla_set_tuning(h, 2, 2) == INVALID
    assert lib.spla_set_tuning(h, 7, 0) == INVALID
    assert lib.spla_set_tuning(None, 0, 0) == INVALID
    lib.spla_destroy(h)


SCORE, STEP_SCORE, SELECT, ATTEND, SELECT_ATTEND, COMBINE, STEP_FUSED = range(1, 8)


def plan(lib, h, call):
    out = i32([0] * 8)
    n = lib.spla_launch_plan(h, call, out, 8)
    return list(out)[:n] if n >= 0 else n


def test_launch_plan(lib):
    # bf16, Bk=64, top_k=16; lengths 100 (2 blocks) and 2000 (32 blocks > top_k)
    h, c = bound(lib)
    # automatic: 4 (b, g) pairs -> fused select + attend, then the combine
    assert plan(lib, h, 2) == [STEP_SCORE, SELECT_ATTEND, COMBINE]
    assert plan(lib, h, 0) == [SCORE, SELECT_ATTEND, COMBINE]
    assert plan(lib, h, 1) == [SCORE, ATTEND, COMBINE]              # selection override
    assert lib.spla_set_tuning(h, 2, 1) == OK                       # the fused kernel merges the records itself
    assert plan(lib, h, 2) == [STEP_SCORE, SELECT_ATTEND]
    assert plan(lib, h, 0) == [SCORE, SELECT_ATTEND]
    assert plan(lib, h, 1) == [SCORE, ATTEND, COMBINE]
    assert lib.spla_set_tuning(h, 2, 0) == OK
    assert plan(lib, h, 2) == [STEP_SCORE, SELECT_ATTEND, COMBINE]
    assert lib.spla_set_tuning(h, 1, 1) == OK                       # the step in one kernel
    assert plan(lib, h, 2) == [STEP_FUSED, COMBINE]
    assert plan(lib, h, 0) == [SCORE, SELECT_ATTEND, COMBINE]       # spla_decode: unchanged
    assert lib.spla_set_tuning(h, 1, 0) == OK
    assert plan(lib, h, 2) == [STEP_SCORE, SELECT_ATTEND, COMBINE]
    assert lib.spla_set_tuning(h, 1, 1) == OK
    assert lib.spla_set_tuning(h, 0, 0) == OK                       # the one-kernel step needs the fused selector
    assert plan(lib, h, 2) == [STEP_SCORE, SELECT, ATTEND, COMBINE]
    assert lib.spla_set_tuning(h, 0, 1) == OK
    assert plan(lib, h, 0) == [SCORE, SELECT_ATTEND, COMBINE]
    assert plan(lib, h, 3) == -1 and lib.spla_launch_plan(None, 0, None, 0) == -1
    assert lib.spla_launch_plan(h, 2, None, 0) == 2                 # count only
    # the one-kernel step takes the Taylor score only
    assert lib.spla_set_score_form(h, 1) == OK
    assert plan(lib, h, 2) == [STEP_SCORE, SELECT_ATTEND, COMBINE]
    assert lib.spla_set_score_form(h, 0) == OK
    assert lib.spla_set_tuning(h, 1, -1) == OK
    assert lib.spla_set_tuning(h, 2, -1) == OK
    assert plan(lib, h, 2) == [STEP_SCORE, SELECT_ATTEND, COMBINE]
    assert lens_of(lib, h, 2) == [100, 2000]                       # the query changes nothing
    lib.spla_destroy(h)
    # every sequence short: the first kernel still runs (it forms the
    # phi(q)^T S_all partials of the merge)
    h, c = bound(lib, lens=(5, 64 * 16))
    assert plan(lib, h, 0) == [SCORE, SELECT_ATTEND, COMBINE]
    assert plan(lib, h, 2) == [STEP_SCORE, SELECT_ATTEND, COMBINE]
    assert lib.spla_set_tuning(h, 2, 1) == OK
    assert plan(lib, h, 2) == [STEP_SCORE, SELECT_ATTEND]
    assert lib.spla_set_tuning(h, 1, 1) == OK
    assert plan(lib, h, 2) == [STEP_FUSED, COMBINE]
    lib.spla_destroy(h)
    # 256 (b, h) pairs or more: the combine kernel takes whole heads, and the
    # fused kernel does not merge
    h, c = bound(lib, lens=[100] * 64, batch=64, n_q_heads=4, n_kv_heads=2, max_blocks_per_seq=40, num_pages=64 * 40)
    assert plan(lib, h, 2) == [STEP_SCORE, SELECT, ATTEND, COMBINE]  # 128 (b, g) pairs: split selector
    assert lib.spla_set_tuning(h, 0, 1) == OK and lib.spla_set_tuning(h, 2, 1) == OK
    assert plan(lib, h, 2) == [STEP_SCORE, SELECT_ATTEND, COMBINE]
    lib.spla_destroy(h)
    # the fused kernel needs bf16 and Bk = 64
    for kw in (dict(kv_dtype=0), dict(block_size=128)):
        h, c = bound(lib, lens=(100, 2000), **kw)
        assert lib.spla_set_tuning(h, 0, 1) == OK
        assert plan(lib, h, 2) == [STEP_SCORE, SELECT, ATTEND, COMBINE], kw
        lib.spla_destroy(h)
    # more than 4096 candidates: stand-alone selector
    h, c = bound(lib, lens=(100, 64 * 4200), max_blocks_per_seq=4300)
    assert lib.spla_set_tuning(h, 0, 1) == OK
    assert plan(lib, h, 0) == [SCORE, SELECT, ATTEND, COMBINE]
    lib.spla_destroy(h)


def test_rla_output_validation(lib):
    h, c = bound(lib)
    nan, inf = float("nan"), float("inf")
    assert lib.spla_set_rla_output(h, 0, None, 0.0) == OK
    assert lib.spla_set_rla_output(h, 1, None, 0.0) == OK
    assert lib.spla_set_rla_output(h, 2, FAKE, 1e-6) == OK
    for gamma, eps, want in ((None, 1e-6, INVALID), (FAKE, 0.0, INVALID), (FAKE, -1e-6, INVALID),
                             (FAKE, nan, INVALID), (FAKE, inf, INVALID), (FAKE + 4, 1e-6, ALIGN)):
        assert lib.spla_set_rla_output(h, 2, gamma, eps) == want, (gamma, eps)
    assert lib.spla_set_rla_output(h, 3, None, 0.0) == INVALID
    assert lib.spla_set_rla_output(h, -1, None, 0.0) == INVALID
    assert lib.spla_set_rla_output(None, 0, None, 0.0) == INVALID
    # with the merge asked for, the RMS form keeps the combine kernel; the
    # plain and normalised forms merge inside the fused kernel
    assert lib.spla_set_tuning(h, 2, 1) == OK
    assert plan(lib, h, 2) == [STEP_SCORE, SELECT_ATTEND, COMBINE]
    assert lib.spla_set_rla_output(h, 1, None, 0.0) == OK
    assert plan(lib, h, 2) == [STEP_SCORE, SELECT_ATTEND]
    lib.spla_destroy(h)


def test_score_form_and_block_mass_validation(lib):
    st, h = create(lib, cfg())
    assert lib.spla_block_mass(h, FAKE, FAKE, None) == STATE      # before spla_bind
    assert lib.spla_set_score_form(h, 0) == OK and lib.spla_set_score_form(h, 1) == OK
    assert lib.spla_set_score_form(h, 2) == INVALID and lib.spla_set_score_form(h, -1) == INVALID
    assert lib.spla_set_score_form(None, 0) == INVALID
    lib.spla_destroy(h)
    h, c = bound(lib)
    assert lib.spla_block_mass(h, None, FAKE, None) == INVALID
    assert lib.spla_block_mass(h, FAKE, None, None) == INVALID
    assert lib.spla_block_mass(h, FAKE + 2, FAKE, None) == ALIGN
    assert lib.spla_block_mass(h, FAKE, FAKE + 8, None) == ALIGN
    assert lib.spla_block_mass(None, FAKE, FAKE, None) == INVALID
    lib.spla_destroy(h)
    h, c = bound(lib, lens=(0, 2000))                              # an empty sequence
    assert lib.spla_block_mass(h, FAKE, FAKE, None) == INVALID
    # every sequence has at most two blocks: nothing to launch, nothing touched
    lib.spla_destroy(h)
    h, c = bound(lib, lens=(64, 128))
    assert lib.spla_block_mass(h, FAKE, FAKE, None) == OK
    # the score form changes which score the selection ranks; the one-kernel
    # step takes the Taylor score only
    assert plan(lib, h, 2) == [STEP_SCORE, SELECT_ATTEND, COMBINE]
    assert lib.spla_set_tuning(h, 1, 1) == OK
    assert plan(lib, h, 2) == [STEP_FUSED, COMBINE]
    assert lib.spla_set_score_form(h, 1) == OK
    assert plan(lib, h, 2) == [STEP_SCORE, SELECT_ATTEND, COMBINE]
    lib.spla_destroy(h)


def test_prefill_workspace_and_validation(lib):
    st, h = create(lib, cfg())
    one = lib.spla_prefill_workspace_bytes(h, 1)
    assert 0 < one < lib.spla_prefill_workspace_bytes(h, 2) < lib.spla_prefill_workspace_bytes(h, 256)
    assert lib.spla_prefill_workspace_bytes(h, 0) == 0 and lib.spla_prefill_workspace_bytes(h, 257) == 0
    assert lib.spla_prefill_workspace_bytes(None, 1) == 0
    big = lib.spla_prefill_workspace_bytes(h, 256)
    args = (FAKE, FAKE + 4096, FAKE + 8192, FAKE + 12288, FAKE + 16384, None, None, FAKE + (1 << 31))
    assert lib.spla_prefill(h, 0, 4, *args, big, None) == STATE    # before spla_bind
    lib.spla_destroy(h)
    h, c = bound(lib, lens=(100, 2000))
    for seq, n, want in ((-1, 4, INVALID), (2, 4, INVALID), (0, -1, INVALID), (0, 0, OK)):
        assert lib.spla_prefill(h, seq, n, *args, big, None) == want, (seq, n)
    assert lib.spla_prefill(h, 0, 4, *args, one - 1, None) == INVALID   # workspace below one token
    for i in (0, 1, 2, 3, 4, 7):
        bad = list(args)
        bad[i] = None
        assert lib.spla_prefill(h, 0, 4, *bad, big, None) == INVALID, i
        bad[i] = args[i] + 4
        assert lib.spla_prefill(h, 0, 4, *bad, big, None) == ALIGN, i
    bad = list(args)
    bad[5] = FAKE + 20484                                          # misaligned sel_idx
    assert lib.spla_prefill(h, 0, 4, *bad, big, None) == ALIGN
    bad = list(args)
    bad[6] = FAKE + 24580                                          # misaligned lg
    assert lib.spla_prefill(h, 0, 4, *bad, big, None) == ALIGN
    cap = c.max_blocks_per_seq * c.block_size
    assert lib.spla_prefill(h, 1, cap - 2000 + 1, *args, big, None) == CAPACITY
    assert lens_of(lib, h, 2) == [100, 2000]                       # nothing enqueued, mirror unchanged
    lib.spla_destroy(h)
