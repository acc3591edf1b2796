"""Parity machinery shared by the GPU tests, smoke() and bench.py: drive the
HIP library (through its C ABI binding) and the fp64 oracle with the same
seeded inputs and compare them with the acceptance rules of the decode
specification:

  sets     every (b, g) selection holds the sink, the current block and
           |P| = top_k - 2 scored candidates (or every block when nb <= top_k),
           and no excluded candidate beats an included one by more than 1e-5
           relative in the oracle's fp64 score: min_in LG >= max_out LG +
           log(1 - 1e-5).  Outputs are then compared with the oracle re-run on
           the GPU's selection, because a legal near-tie swap moves o_sparse
           far more than the output tolerance.
  scores   the exported group log score LG of every candidate: |gpu - ref|
           <= 1e-6 * max(1, |ref|) (absolute in the log domain; past
           |LG| = 1 the bar follows the fp32 spacing of LG itself).
  outputs  o, o_sparse and o_rla each: max|gpu - ref| <= 2e-3 * max|ref|
           (o_rla ~ 1e5 dwarfs o_sparse ~ 1 at long context, so each is
           checked on its own); D: <= 1e-4 relative.
  state    S_all, z_all per (b, g): max|gpu - ref| <= 1e-4 * max|ref|;
           block mean / variance: <= 1e-5 relative (+1e-6 absolute).

Sampled checks: the method treats every (sequence, KV head) pair on its own,
so at full sizes the oracle is run on a subset of sequences and KV heads (their
slices of the same inputs, with their query heads and gates) and compared with
the matching slices of the GPU's results; the GPU still runs the whole batch.
"""
from __future__ import annotations

import math
import time
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

from oracle import SplaOracle
from workloads import Workload

OUT_REL = 2e-3
D_REL = 1e-4
S_REL = 1e-4
STAT_REL = 1e-5
TIE_REL = 1e-5
LG_ABS = 1e-6


def check_selection(sel_row, lg: Dict[int, float], nb: int, top_k: int) -> Optional[str]:
    """None if the GPU selection of one (b, g) is acceptable, else a message."""
    sel = [int(x) for x in sel_row]
    valid = [x for x in sel if x >= 0]
    if valid != sorted(valid) or len(set(valid)) != len(valid):
        return f"not ascending/distinct: {sel}"
    if sel[:len(valid)] != valid or any(x != -1 for x in sel[len(valid):]):
        return f"-1 padding not at the end: {sel}"
    if nb <= top_k:
        return None if valid == list(range(nb)) else f"expected all {nb} blocks, got {valid}"
    if 0 not in valid or (nb - 1) not in valid:
        return f"sink/current missing: {valid}"
    if len(valid) != top_k:
        return f"expected {top_k} blocks, got {len(valid)}"
    P = [j for j in valid if 0 < j < nb - 1]
    out = [j for j in range(1, nb - 1) if j not in set(P)]
    if not out or not P:  # nothing left out, or top_k = 2 (sink and current only)
        return None
    lo = min(lg[j] for j in P)
    hi = max(lg[j] for j in out)
    if lo < hi + math.log1p(-TIE_REL):
        return f"selection beaten beyond the tie tolerance: min in {lo}, max out {hi}"
    return None


def rel_err(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.abs(ref).max()
    diff = np.abs(x - ref).max() if x.size else 0.0
    if scale == 0:
        return float(diff)
    return float(diff / scale)


@dataclass
class StepReport:
    step: int
    errors: Dict[str, float] = field(default_factory=dict)
    sel_equal: bool = True
    near_ties: int = 0
    failures: List[str] = field(default_factory=list)


class ParityRun:
    """A SplaLayer and a SplaOracle fed from one Workload."""

    def __init__(self, w: Workload, page_order: str = "identity", steps: Optional[int] = None,
                 device: str = "cuda", prefill_chunk: int = 4096, use_step: bool = False,
                 seqs: Optional[List[int]] = None, kv_heads: Optional[List[int]] = None,
                 fused_select: int = -1, rla_form: int = 0, rla_eps: float = 1e-6, score_form: int = 0,
                 step_kernel: int = -1, fused_merge: int = -1):
        import torch
        from block_sparse_linear_amd import SplaLayer

        self.torch = torch
        self.w = w
        self.steps = w.steps if steps is None else steps
        self.device = device
        self.prefill_chunk = prefill_chunk
        self.use_step = use_step  # spla_decode_step instead of spla_append_kv + spla_decode
        mb = w.max_blocks_per_seq(self.steps)
        self.layer = SplaLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k, mb,
                               kv_dtype=w.kv_dtype, device=device, page_order=page_order, seed=w.seed)
        self.layer.set_fused_select(fused_select)
        self.layer.set_step_kernel(step_kernel)
        self.layer.set_fused_merge(fused_merge)
        # sequences / KV heads the oracle checks (all by default)
        self.bs = list(range(w.batch)) if seqs is None else [int(b) for b in seqs]
        self.gs = list(range(w.n_kv_heads)) if kv_heads is None else [int(g) for g in kv_heads]
        r = w.group
        self.hs = [g * r + i for g in self.gs for i in range(r)]
        self.oracle = SplaOracle(len(self.bs), r * len(self.gs), len(self.gs), w.head_dim, w.block_size,
                                 w.top_k, w.max_tokens(self.steps))
        self.gate_np = w.gate()
        self.gate = torch.from_numpy(self.gate_np).to(device)
        # output form of the RLA branch (0 plain, 1 normalised, 2 RMS-normalised)
        self.rla_form, self.rla_eps = rla_form, rla_eps
        self.gamma_np = w.rla_gamma() if rla_form == 2 else None
        self.layer.set_rla_output(rla_form, None if self.gamma_np is None else torch.from_numpy(self.gamma_np),
                                  rla_eps)
        # block score the selection ranks (0 Taylor, 1 mean pooling)
        self.score_form = score_form
        self.layer.set_score_form(score_form)
        self.mix = w.mixture_state()

    def dev(self, x: np.ndarray):
        return self.torch.from_numpy(np.ascontiguousarray(x)).to(self.device).to(self.layer.dtype)

    def _ob(self, b: int) -> int:
        """oracle index of sequence b (-1 if not checked)"""
        return self.bs.index(b) if b in self.bs else -1

    def prefill(self) -> None:
        gs = self.gs
        for b in range(self.w.batch):
            ob = self._ob(b)
            for _, k, v in self.w.prefill_chunks(b, self.prefill_chunk):
                self.layer.append([b], [k.shape[0]], self.dev(k), self.dev(v))
                if ob >= 0:
                    self.oracle.append([ob], [k.shape[0]], k[:, gs], v[:, gs])

    def append_step(self, s: int, token: bool = True) -> Dict[str, np.ndarray]:
        """The step's chunk appends and (token=True) its one-token append, on
        both sides."""
        st = self.w.step(s, self.mix)
        cs = [int(x) for x in st["chunk_seqs"]]
        gs, L = self.gs, self.w.chunk_len
        if cs:
            n = [L] * len(cs)
            self.layer.append(cs, n, self.dev(st["chunk_k"]), self.dev(st["chunk_v"]))
            picks = [i for i, b in enumerate(cs) if self._ob(b) >= 0]
            if picks:
                rows = np.concatenate([np.arange(i * L, (i + 1) * L) for i in picks])
                self.oracle.append([self._ob(cs[i]) for i in picks], [L] * len(picks),
                                   st["chunk_k"][rows][:, gs], st["chunk_v"][rows][:, gs])
        allb = list(range(self.w.batch))
        if token:
            self.layer.append(allb, [1] * self.w.batch, self.dev(st["k"]), self.dev(st["v"]))
        bs = self.bs
        self.oracle.append(list(range(len(bs))), [1] * len(bs), st["k"][bs][:, gs], st["v"][bs][:, gs])
        return st

    def gpu_decode(self, q_np: np.ndarray, sel_in=None, kv=None):
        t = self.torch
        w = self.w
        B, H, G, d = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
        aux = {
            "sel_idx": t.empty((B, G, w.top_k), dtype=t.int32, device=self.device),
            "lg": t.zeros((B, G, self.layer.mb), dtype=t.float32, device=self.device),
            "o_sparse": t.empty((B, H, d), dtype=t.float32, device=self.device),
            "o_rla": t.empty((B, H, d), dtype=t.float32, device=self.device),
            "d_rla": t.empty((B, H), dtype=t.float32, device=self.device),
        }
        if sel_in is not None:
            aux["sel_in"] = t.from_numpy(np.ascontiguousarray(sel_in, np.int32)).to(self.device)
        if kv is not None:
            out = self.layer.decode_step(self.dev(kv[0]), self.dev(kv[1]), self.dev(q_np), self.gate, aux=aux)
        else:
            out = self.layer.decode(self.dev(q_np), self.gate, aux=aux)
        t.cuda.synchronize()
        res = {k: v.cpu().numpy() for k, v in aux.items() if k != "sel_in"}
        res["o"] = out.cpu().numpy()
        return res

    def check_decode(self, s: int, q_np: np.ndarray, sel_in=None, kv=None) -> StepReport:
        w = self.w
        rep = StepReport(step=s)
        bs, gs, hs = self.bs, self.gs, self.hs
        g = self.gpu_decode(q_np, sel_in, kv)
        # the checked slices of the GPU's results
        g = {"o": g["o"][bs][:, hs], "o_sparse": g["o_sparse"][bs][:, hs], "o_rla": g["o_rla"][bs][:, hs],
             "d_rla": g["d_rla"][bs][:, hs], "sel_idx": g["sel_idx"][bs][:, gs], "lg": g["lg"][bs][:, gs]}
        q_o = q_np[bs][:, hs]
        gate_o = self.gate_np[hs]
        form = dict(rla_mode=self.rla_form, eps=self.rla_eps, score_form=self.score_form,
                    gamma=None if self.gamma_np is None else self.gamma_np[hs])
        sel_o = None if sel_in is None else np.asarray(sel_in)[bs][:, gs]
        ref = self.oracle.decode(q_o, gate_o, sel_override=sel_o, **form)
        sel_gpu = g["sel_idx"]
        if sel_in is None:
            for b in range(len(bs)):
                nb = -(-int(self.oracle.lens[b]) // w.block_size)
                for gg in range(len(gs)):
                    msg = check_selection(sel_gpu[b, gg], ref["lg"][b][gg], nb, w.top_k)
                    if msg:
                        rep.failures.append(f"step {s} b {bs[b]} g {gs[gg]}: {msg}")
                    if not np.array_equal(sel_gpu[b, gg], ref["sel"][b, gg]):
                        rep.sel_equal = False
                        rep.near_ties += 1
                    # group log scores: absolute in the log domain, relative past |LG| = 1
                    if nb > w.top_k:
                        js = np.arange(1, nb - 1)
                        lg_ref = np.array([ref["lg"][b][gg][int(j)] for j in js])
                        dlg = np.abs(g["lg"][b, gg, js].astype(np.float64) - lg_ref)
                        rep.errors["lg_abs"] = max(rep.errors.get("lg_abs", 0.0), float(dlg.max()))
                        bad = dlg > LG_ABS * np.maximum(1.0, np.abs(lg_ref))
                        if bad.any():
                            i = int(np.argmax(dlg / np.maximum(1.0, np.abs(lg_ref))))
                            rep.failures.append(f"step {s} b {bs[b]} g {gs[gg]}: group log score of block "
                                                f"{int(js[i])} off by {dlg[i]:.3g} (oracle {lg_ref[i]:.6g})")
            if not rep.sel_equal:
                ref = self.oracle.decode(q_o, gate_o, sel_override=sel_gpu, **form)
        else:
            if not np.array_equal(sel_gpu, sel_o):
                rep.failures.append("sel_idx output != sel_in")
        for k, tol in (("o", OUT_REL), ("o_sparse", OUT_REL), ("o_rla", OUT_REL), ("d_rla", D_REL)):
            e = rel_err(g[k], ref[k])
            rep.errors[k] = e
            if e > tol:
                rep.failures.append(f"step {s}: {k} rel err {e:.3g} > {tol}")
        if self.rla_form != 0:
            # the branch itself, (o - o_sparse) / g, on heads whose gate is not small
            big = np.abs(gate_o) > 0.25
            if big.any():
                br = (g["o"].astype(np.float64) - g["o_sparse"]) / gate_o[None, :, None]
                e = rel_err(br[:, big], ref["rla_out"][:, big])
                rep.errors["rla_out"] = e
                if e > OUT_REL:
                    rep.failures.append(f"step {s}: RLA branch rel err {e:.3g} > {OUT_REL}")
        return rep

    def check_state(self) -> Dict[str, float]:
        w = self.w
        bs, gs = self.bs, self.gs
        S = self.layer.s_all.cpu().numpy()[bs][:, gs]
        z = self.layer.z_all.cpu().numpy()[bs][:, gs]
        mean, var = (x.cpu().numpy()[bs][:, gs] for x in self.layer.stats())
        errs = {"S": 0.0, "z": 0.0, "mean": 0.0, "var": 0.0}
        for b in range(len(bs)):
            nfull = int(self.oracle.lens[b]) // w.block_size
            for g in range(len(gs)):
                errs["S"] = max(errs["S"], rel_err(S[b, g], self.oracle.S[b, g]))
                errs["z"] = max(errs["z"], rel_err(z[b, g], self.oracle.z[b, g]))
                if nfull:
                    for name, gv, ov in (("mean", mean, self.oracle.mean), ("var", var, self.oracle.var)):
                        d = np.abs(gv[b, g, :nfull].astype(np.float64) - ov[b, g, :nfull])
                        scale = np.abs(ov[b, g, :nfull])
                        errs[name] = max(errs[name], float((d / (scale + 1e-6 / STAT_REL)).max()))
        return errs

    def state_failures(self, errs: Dict[str, float]) -> List[str]:
        f = []
        if errs["S"] > S_REL:
            f.append(f"S_all rel err {errs['S']:.3g}")
        if errs["z"] > S_REL:
            f.append(f"z_all rel err {errs['z']:.3g}")
        if errs["mean"] > STAT_REL:
            f.append(f"block mean rel err {errs['mean']:.3g}")
        if errs["var"] > STAT_REL:
            f.append(f"block var rel err {errs['var']:.3g}")
        return f

    def run(self, steps: Optional[int] = None, verbose: bool = False) -> List[str]:
        steps = self.steps if steps is None else steps
        t0 = time.time()
        self.prefill()
        failures = self.state_failures(self.check_state())
        worst: Dict[str, float] = {}
        ties = 0
        for s in range(steps):
            st = self.append_step(s, token=not self.use_step)
            rep = self.check_decode(s, st["q"], kv=(st["k"], st["v"]) if self.use_step else None)
            failures += rep.failures
            ties += rep.near_ties
            for k, v in rep.errors.items():
                worst[k] = max(worst.get(k, 0.0), v)
        errs = self.check_state()
        failures += self.state_failures(errs)
        failures += ([f"error word {self.layer.error_word():#x}"] if self.layer.error_word() else [])
        if verbose:
            print(f"[parity] {self.w.name} steps={steps} worst={worst} state={errs} near_tie_sets={ties} "
                  f"({time.time() - t0:.1f}s)", flush=True)
        return failures
