"""HIP graph capture of the decode calls through the C ABI: every replay of a
captured spla_decode agrees bitwise with the eager call on the same inputs,
replay after replay, with eager decodes of other queries (which overwrite the
workspace) and synchronisations in between; captured spla_decode_step
graphs, replayed in step order from a restored state, agree bitwise with the
eager steps, twice over; a captured spla_prefill (several launch groups),
replayed from the restored state three times with eager work in between,
agrees bitwise with the eager call in its outputs, selections and state."""
import numpy as np
import pytest

from tests.test_gpu_parity import _needs_gpu, small

pytestmark = pytest.mark.gpu

AUX_KEYS = ("sel_idx", "lg", "o_sparse", "o_rla", "d_rla")


def _aux(layer):
    import torch
    B, H, G, d = layer.B, layer.H, layer.G, layer.d
    dev = layer.device
    return {"sel_idx": torch.zeros((B, G, layer.top_k), dtype=torch.int32, device=dev),
            "lg": torch.zeros((B, G, layer.mb), dtype=torch.float32, device=dev),
            "o_sparse": torch.zeros((B, H, d), dtype=torch.float32, device=dev),
            "o_rla": torch.zeros((B, H, d), dtype=torch.float32, device=dev),
            "d_rla": torch.zeros((B, H), dtype=torch.float32, device=dev)}


def _poison(out, aux):
    # outputs the library writes in full get values it never produces; lg
    # (written only for candidate blocks) goes back to its initial zeros
    out.fill_(float("nan"))
    aux["sel_idx"].fill_(-7)
    for k in ("o_sparse", "o_rla", "d_rla"):
        aux[k].fill_(float("nan"))
    aux["lg"].zero_()


def _snap(out, aux):
    r = {k: aux[k].cpu().numpy().copy() for k in AUX_KEYS}
    r["o"] = out.cpu().numpy().copy()
    return r


def _same(a, b, what):
    for k in a:
        assert np.array_equal(a[k], b[k]), f"{what}: {k} differs"


@pytest.mark.parametrize("fused", [0, 1])
def test_decode_graph_replays_match_eager(fused):
    _needs_gpu()
    import torch
    from tests.spla_parity import ParityRun
    w = small(name="graph_decode", batch=2, t0=(64 * 150 + 37, 64 * 40 + 5), steps=3)
    print(f"[case] graph decode fused={fused}", flush=True)
    run = ParityRun(w, steps=3, page_order="shuffled", fused_select=fused)
    run.prefill()
    st = run.append_step(0)
    L = run.layer
    q = run.dev(st["q"])
    q_other = run.dev(w.step(1)["q"])
    out_ref, aux_ref = torch.zeros((L.B, L.H, L.d), dtype=torch.float32, device=L.device), _aux(L)
    L.decode(q, run.gate, out=out_ref, aux=aux_ref)
    torch.cuda.synchronize()
    ref = _snap(out_ref, aux_ref)
    out, aux = torch.zeros_like(out_ref), _aux(L)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.decode(q, run.gate, out=out, aux=aux)
    for rep in range(4):
        _poison(out, aux)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(ref, _snap(out, aux), f"replay {rep}")
        # eager work between replays: a decode of another query rewrites the
        # workspace (scores, selection, partials)
        L.decode(q_other, run.gate)
        torch.cuda.synchronize()
    assert L.error_word() == 0


def test_step_graphs_match_eager():
    _needs_gpu()
    import torch
    from tests.spla_parity import ParityRun
    n = 4
    w = small(name="graph_step", batch=2, t0=(64 * 90 + 62, 64 * 20 + 1), steps=n)
    print("[case] graph step", flush=True)
    run = ParityRun(w, steps=n, page_order="shuffled")
    run.prefill()
    L = run.layer
    snap = L.snapshot()
    ins = []
    for s in range(n):
        st = w.step(s)
        ins.append((run.dev(st["k"]), run.dev(st["v"]), run.dev(st["q"])))
    # eager steps
    ref = []
    for k, v, q in ins:
        out, aux = torch.zeros((L.B, L.H, L.d), dtype=torch.float32, device=L.device), _aux(L)
        L.decode_step(k, v, q, run.gate, out=out, aux=aux)
        torch.cuda.synchronize()
        ref.append(_snap(out, aux))
    end_state = [x.clone() for x in L.state_tensors()]
    # capture the same steps from the restored state (capture runs nothing;
    # the host mirror advances as the calls are recorded)
    L.restore(snap)
    outs = [(torch.zeros((L.B, L.H, L.d), dtype=torch.float32, device=L.device), _aux(L)) for _ in range(n)]
    graphs = []
    for (k, v, q), (out, aux) in zip(ins, outs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            L.decode_step(k, v, q, run.gate, out=out, aux=aux)
        graphs.append(g)
    torch.cuda.synchronize()
    for rnd in range(2):
        if rnd:
            # back to the prefilled state by plain copies (eager work); the
            # graphs carry their own lengths
            for dst, src in zip(L.state_tensors(), snap[0]):
                dst.copy_(src)
            torch.cuda.synchronize()
        for s, (g, (out, aux)) in enumerate(zip(graphs, outs)):
            _poison(out, aux)
            g.replay()
            torch.cuda.synchronize()
            _same(ref[s], _snap(out, aux), f"round {rnd} step {s}")
        for a, b in zip(L.state_tensors(), end_state):
            assert torch.equal(a, b), f"round {rnd}: state after the replayed steps differs"
    assert L.lens == [t + n for t in snap[1]]
    assert L.error_word() == 0


def test_prefill_graph_replays_match_eager():
    _needs_gpu()
    import torch
    from tests.spla_parity import ParityRun
    w = small(name="graph_prefill", batch=2, t0=(64 * 60 + 17, 64 * 20 + 3), steps=1, extra_capacity_tokens=400)
    seq, n, chunk = 0, 300, 128
    print(f"[case] graph prefill seq={seq} n={n} chunk={chunk}", flush=True)
    run = ParityRun(w, steps=1, page_order="shuffled")
    run.prefill()
    L = run.layer
    snap = L.snapshot()
    rng = np.random.default_rng(11)
    G, H, d = w.n_kv_heads, w.n_q_heads, w.head_dim
    k = run.dev(w.round(rng.standard_normal((n, G, d)).astype(np.float32)))
    v = run.dev(w.round(rng.standard_normal((n, G, d)).astype(np.float32)))
    q = run.dev(w.round(rng.standard_normal((n, H, d)).astype(np.float32)))
    ws = torch.empty(L.handle.prefill_workspace_bytes(chunk) // 4 + 64, dtype=torch.int32, device=L.device)
    # eager call
    out_e = torch.zeros((n, H, d), dtype=torch.float32, device=L.device)
    sel_e = torch.zeros((n, G, w.top_k), dtype=torch.int32, device=L.device)
    L.prefill(seq, k, v, q, run.gate, out=out_e, chunk=chunk, workspace=ws, sel_idx=sel_e)
    torch.cuda.synchronize()
    ref_out, ref_sel = out_e.cpu().numpy(), sel_e.cpu().numpy()
    end_state = [x.clone() for x in L.state_tensors()]
    # capture the same call from the restored state
    L.restore(snap)
    out_g = torch.zeros_like(out_e)
    sel_g = torch.zeros_like(sel_e)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.prefill(seq, k, v, q, run.gate, out=out_g, chunk=chunk, workspace=ws, sel_idx=sel_g)
    torch.cuda.synchronize()
    for rnd in range(3):
        # back to the state before the call by plain copies, and eager work
        # on the workspace and outputs in between (the graph carries its own
        # lengths)
        for dst, src in zip(L.state_tensors(), snap[0]):
            dst.copy_(src)
        ws.fill_(-1)
        out_g.fill_(float("nan"))
        sel_g.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out_g.cpu().numpy(), ref_out), f"replay {rnd}: outputs differ"
        assert np.array_equal(sel_g.cpu().numpy(), ref_sel), f"replay {rnd}: selections differ"
        for a, b in zip(L.state_tensors(), end_state):
            assert torch.equal(a, b), f"replay {rnd}: state after the call differs"
    assert L.lens[seq] == snap[1][seq] + n
    assert L.error_word() == 0
