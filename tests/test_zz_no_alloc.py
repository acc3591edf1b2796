"""spla_decode_step_noalloc (the per-call scratch in the library's static
device array) against spla_decode_step (the scratch in the bound workspace):
two layers hold the same state, one steps through each entry point, and
every output, aux output and the state after the steps must agree to the
parity bar (selections exact, o / o_sparse / o_rla within 2e-3 of their
largest value, D within 1e-4); they run the same kernels on the same inputs,
so they are also expected to agree bitwise.  The no-alloc calls must leave
the bound workspace untouched past its error word.

Two calls in a row share the static array: a larger configuration first,
then a smaller one (fewer sequences, heads, channels, blocks and slots), so
the second reads an array still holding the first one's contents; then the
larger one again.
"""
import numpy as np
import pytest

from tests.test_gpu_parity import _needs_gpu
from workloads import Workload

pytestmark = pytest.mark.gpu

OUT_REL, D_REL = 2e-3, 1e-4
SENTINEL = 0x5A5A5A5A


def _pair(w, fused):
    import torch
    from block_sparse_linear_amd import SplaLayer

    mb = w.max_blocks_per_seq(4)
    layers = []
    for _ in range(2):
        L = SplaLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k, mb,
                      kv_dtype=w.kv_dtype, device="cuda", page_order="shuffled", seed=w.seed)
        L.set_fused_select(fused)
        layers.append(L)
    a, b = layers
    for s in range(w.batch):
        for _, k, v in w.prefill_chunks(s, 4096):
            kk = torch.from_numpy(k).to("cuda").to(a.dtype)
            vv = torch.from_numpy(v).to("cuda").to(a.dtype)
            a.append([s], [k.shape[0]], kk, vv)
    for dst, src in zip(b.state_tensors(), a.state_tensors()):
        dst.copy_(src)
    b._bind(a.lens)
    torch.cuda.synchronize()
    return a, b


def _aux(L, w):
    import torch
    B, H, G, d = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    return {"sel_idx": torch.full((B, G, w.top_k), -7, dtype=torch.int32, device="cuda"),
            "lg": torch.zeros((B, G, L.mb), dtype=torch.float32, device="cuda"),
            "o_sparse": torch.zeros((B, H, d), dtype=torch.float32, device="cuda"),
            "o_rla": torch.zeros((B, H, d), dtype=torch.float32, device="cuda"),
            "d_rla": torch.zeros((B, H), dtype=torch.float32, device="cuda")}


def _rel(x, ref):
    x, ref = x.double().cpu().numpy(), ref.double().cpu().numpy()
    scale = np.abs(ref).max()
    return float(np.abs(x - ref).max() / (scale if scale > 0 else 1.0))


def _step_and_compare(a, b, w, s):
    import torch
    st = w.step(s)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(a.dtype)  # noqa: E731
    k, v, q = dev(st["k"]), dev(st["v"]), dev(st["q"])
    gate = torch.from_numpy(w.gate()).to("cuda")
    out_a = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    out_b = torch.full_like(out_a, float("nan"))
    aux_a, aux_b = _aux(a, w), _aux(b, w)
    b.workspace[1:] = SENTINEL
    a.decode_step(k, v, q, gate, out=out_a, aux=aux_a)
    b.decode_step_noalloc(k, v, q, gate, out=out_b, aux=aux_b)
    torch.cuda.synchronize()
    assert a.lens == b.lens
    assert torch.equal(aux_a["sel_idx"], aux_b["sel_idx"]), "selections differ"
    for name, x, y, tol in (("o", out_b, out_a, OUT_REL), ("o_sparse", aux_b["o_sparse"], aux_a["o_sparse"], OUT_REL),
                            ("o_rla", aux_b["o_rla"], aux_a["o_rla"], OUT_REL),
                            ("d_rla", aux_b["d_rla"], aux_a["d_rla"], D_REL)):
        e = _rel(x, y)
        assert e <= tol, f"step {s}: {name} rel err {e:.3g}"
        assert torch.equal(x, y), f"step {s}: {name} not bitwise equal (rel err {e:.3g})"
    assert torch.equal(aux_a["lg"], aux_b["lg"]), "group log scores differ"
    assert bool((b.workspace[1:] == SENTINEL).all()), "the no-alloc call wrote into the bound workspace"
    assert a.error_word() == 0 and b.error_word() == 0


def _run_case(w, fused, steps):
    import torch
    print(f"[no-alloc] {w.name}: B={w.batch} H={w.n_q_heads} G={w.n_kv_heads} d={w.head_dim} Bk={w.block_size} "
          f"k={w.top_k} t0={w.t0} fused={fused} steps={steps}", flush=True)
    a, b = _pair(w, fused)
    print(f"[no-alloc]   workspace {a.handle.workspace_bytes} bytes, kernels {a.launch_plan()}", flush=True)
    for s in range(steps):
        _step_and_compare(a, b, w, s)
    for x, y in zip(a.state_tensors(), b.state_tensors()):
        assert torch.equal(x, y), "states differ after the steps"


LARGE = Workload(name="noalloc_large", batch=4, n_q_heads=32, n_kv_heads=8, head_dim=128, block_size=64,
                 top_k=32, kv_dtype="bf16", t0=(20000, 9000, 64 * 40, 15555), steps=3, kind="outlier", seed=91,
                 n_outlier=8)
SMALL = Workload(name="noalloc_small", batch=1, n_q_heads=4, n_kv_heads=2, head_dim=64, block_size=128,
                 top_k=8, kv_dtype="bf16", t0=(128 * 20 + 3,), steps=2, kind="normal", seed=92)


def test_noalloc_matches_decode_step_large_then_small():
    _needs_gpu()
    _run_case(LARGE, -1, 3)
    # the second call in a row: a smaller input, through the stand-alone selector
    _run_case(SMALL, 0, 2)
    # and the larger one again, over what the smaller one left
    _run_case(LARGE.scaled(seed=93), 0, 2)
