"""The benchmark's algorithmic byte counts (what the roofline fractions divide
by), checked on the CPU against counts written out from the workload's shape:
the 128K GQA step is 16.77 MB of candidate statistics + 8.26 MB of selected
K/V + 1.06 MB of S_all / z_all, about 26.1 MB in all (the byte model of the
decode step: statistics of the candidate blocks, the selected blocks' K and V,
the state read and written)."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_step_bytes_128k(bench):
    from workloads import WORKLOADS
    w = WORKLOADS["llama_gqa_128k"]
    T = 131073  # the first decode step after the 131072-token prefill
    b = bench.step_bytes(w, [T], 2)
    nb = 2049
    assert b["stats"] == 8 * (nb - 2) * 2 * 128 * 4                     # 2047 candidates x 8 KV heads x 1 KB
    assert b["kv"] == 8 * (31 * 64 + 1) * 2 * 128 * 2                   # 31 full blocks + the 1-token current one
    assert b["state"] == 8 * 2 * (128 * 128 * 4 + 128 * 4)
    assert abs(b["total"] / 26.1e6 - 1) < 0.01


def test_kernel_bytes_partition(bench):
    from workloads import WORKLOADS
    w = WORKLOADS["llama_gqa_128k"]
    lens = [131072 + 37]
    s = bench.step_bytes(w, lens, 2)
    fused = bench.kernel_bytes("select_attend", w, lens, 2)
    split = bench.kernel_bytes("select", w, lens, 2) + bench.kernel_bytes("attend", w, lens, 2)
    # the fused kernel reads the LG row and the selected K/V, reads q and writes
    # the records; the split plan moves the same plus the selection hand-off
    rec = 8 * 4 * 32 * (2 * 128 + 4) * 4
    lg = 8 * ((131072 + 37 + 63) // 64 - 2) * 4
    assert fused == lg + s["kv"] + rec + 32 * 128 * 2
    assert split == fused + 8 * 32 * 4 * 2
    assert bench.kernel_bytes("step_score", w, lens, 2) == bench.step_score_bytes(w, lens, 2)
    # a fused kernel that also merges the records moves the combine's
    # o_bar / phi(q).z partials and outputs as well
    merged = bench.kernel_bytes("select_attend", w, lens, 2, merged=True)
    assert merged == fused + bench.kernel_bytes("combine", w, lens, 2) - rec
    # the combine reads every record once
    assert bench.kernel_bytes("combine", w, lens, 2) > rec
    with pytest.raises(ValueError):
        bench.kernel_bytes("nope", w, lens, 2)


def test_step_bytes_chunk_and_completion_terms(bench):
    from workloads import WORKLOADS
    w = WORKLOADS["ragged_chunked"]  # G = 8, d = 128, bf16, Bk = 64, 256-token chunks
    lens = [5000 + 7]
    base = bench.step_bytes(w, lens, 2)
    assert base["chunk"] == 0
    # a chunk appended to a sequence of 1000 tokens: K and V of 256 tokens read
    # and written to the pages, S_all / z_all read and written, blocks 15..18
    # completed (block 15 = tokens 960..1023 had 40 tokens before the chunk,
    # which are read back), four mean / variance rows written per KV head
    with_chunk = bench.step_bytes(w, lens, 2, {3: 1000})
    expect = (4 * 256 * 8 * 128 * 2 + 8 * 2 * (128 * 128 * 4 + 128 * 4)
              + 8 * (40 * 128 * 2 + 2 * 128 * 4) + 3 * 8 * (2 * 128 * 4))
    assert with_chunk["chunk"] == expect == 3268608
    assert with_chunk["total"] == base["total"] + expect
    # a block-aligned chunk completes blocks 1..4 and reads no earlier key
    assert bench.step_bytes(w, lens, 2, {0: 64})["chunk"] == (4 * 256 * 8 * 128 * 2 + 8 * 2 * (128 * 128 * 4 + 128 * 4)
                                                            + 4 * 8 * (2 * 128 * 4))
    # the step's own token completing a block: its other 63 keys read, mean and variance written
    done = bench.step_bytes(w, [64 * 100], 2)
    part = bench.step_bytes(w, [64 * 100 + 1], 2)
    assert done["state"] - part["state"] == 8 * (63 * 128 * 2 + 2 * 128 * 4)
    # q in, o out, gate, and the token's k / v read and written to the pages
    assert part["io"] == 64 * 32 * 128 * (2 + 4) + 32 * 4 + 64 * 8 * 128 * (2 * 2) * 2
