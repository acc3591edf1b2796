"""Selection fidelity of the SPLA block score on the GPU (synthetic workloads).

For every decode step and every (sequence, KV head) it compares three block
selections of the same size:
  taylor   the second-order Taylor score (the method; SPLA Technical Summary 2.1),
  mean     the first-order mean-pooling score (the heuristic the summary's
           contributions section contrasts it with),
  exact    the top blocks by their exact attention mass (spla_block_mass),
           the best any block score can do,
with three measures:
  recall    fraction of the exact top-k' candidates a selection holds,
  coverage  share of the candidates' exact attention mass (summed over the
            group's query heads) its picks hold, over the share the exact
            top-k' holds,
  attn_mass share of each query head's dense softmax attention (over every
            token, computed by torch from the same pages) that falls on the
            selected tokens: what the sparse branch sees.  One minus it is
            the mass the residual linear-attention branch stands in for, and
            bounds the error of the sparse branch alone (gate 0).
Every measure is an average over steps, sequences and KV (or query) heads.
It also times the exact-mass kernel (HIP events) and reports its bytes per
launch (every key of every candidate block) against the 8 TB/s HBM peak.

    python fidelity.py [--workloads llama_gqa_128k,batched_32k,million_1m] [--steps 8]

Prints one JSON line.
"""
import argparse
import json
import math
import sys
import time

HBM_PEAK_GBS = 8000.0


def log(msg):
    print(f"[fidelity] {msg}", file=sys.stderr, flush=True)


def top_exact(lgx_row, nb, kp):
    """top-kp candidates 1..nb-2 by exact mass, ties to the smaller id"""
    import numpy as np
    js = np.arange(1, nb - 1)
    order = np.lexsort((js, -lgx_row[js]))
    return js[order[:kp]]


def run_workload(name, steps, timing_reps):
    import numpy as np
    import torch
    from block_sparse_linear_amd import SCORE_MEAN, SCORE_TAYLOR, SplaLayer
    from workloads import WORKLOADS

    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    mb = w.max_blocks_per_seq(steps)
    L = SplaLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k, mb,
                  kv_dtype=w.kv_dtype, device="cuda:0")
    t0 = time.time()
    for b in range(w.batch):
        for _, k, v in w.prefill_chunks(b):
            L.append([b], [k.shape[0]], torch.from_numpy(k).to(dev).to(tdt), torch.from_numpy(v).to(dev).to(tdt))
    torch.cuda.synchronize()
    log(f"{name}: prefill {time.time() - t0:.1f}s")
    B, H, G, d, bk, k = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k
    r = H // G
    kp = k - 2
    gate = torch.from_numpy(w.gate()).to(dev)
    mix = w.mixture_state()
    acc = {m: {"recall": [], "coverage": [], "attn_mass": []} for m in ("taylor", "mean", "exact")}
    mass_us, mass_bytes = [], []
    for s in range(steps):
        st = w.step(s, mix)
        cs = [int(x) for x in st["chunk_seqs"]]
        if cs:
            L.append(cs, [w.chunk_len] * len(cs), torch.from_numpy(st["chunk_k"]).to(dev).to(tdt),
                     torch.from_numpy(st["chunk_v"]).to(dev).to(tdt))
        L.append(list(range(B)), [1] * B, torch.from_numpy(st["k"]).to(dev).to(tdt),
                 torch.from_numpy(st["v"]).to(dev).to(tdt))
        q = torch.from_numpy(st["q"]).to(dev).to(tdt)
        lens = L.lens
        # exact mass (timed)
        lgx = torch.full((B, G, mb), float("-inf"), dtype=torch.float32, device=dev)
        L.block_mass(q, lgx)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(timing_reps):
            L.block_mass(q, lgx)
        e1.record()
        torch.cuda.synchronize()
        mass_us.append(e0.elapsed_time(e1) * 1e3 / timing_reps)
        nc_tot = sum(max(-(-t // bk) - 2, 0) for t in lens)
        mass_bytes.append(nc_tot * G * bk * d * (2 if w.kv_dtype == "bf16" else 4) + B * H * d * 2)
        lgx_np = lgx.cpu().numpy()
        # the three selections
        sels = {}
        for m, form in (("taylor", SCORE_TAYLOR), ("mean", SCORE_MEAN)):
            L.set_score_form(form)
            aux = {"sel_idx": torch.empty((B, G, k), dtype=torch.int32, device=dev)}
            L.decode(q, gate, aux=aux)
            torch.cuda.synchronize()
            sels[m] = aux["sel_idx"].cpu().numpy()
        L.set_score_form(SCORE_TAYLOR)
        sel_ex = np.full((B, G, k), -1, np.int32)
        for b in range(B):
            nb = -(-lens[b] // bk)
            for g in range(G):
                if nb <= k:
                    sel_ex[b, g, :nb] = np.arange(nb)
                else:
                    sel_ex[b, g] = np.sort(np.concatenate([[0, nb - 1], top_exact(lgx_np[b, g], nb, kp)]))
        sels["exact"] = sel_ex
        # dense softmax attention over every token (torch, fp32; the pages are
        # in identity order): the share of each head's mass on the selected tokens
        qf = q.float()
        for b in range(B):
            T = lens[b]
            nb = -(-T // bk)
            if nb <= k:
                continue
            pages = L.block_table[b, :nb].long()
            Kb = L.k_pages[pages].float().permute(1, 0, 2, 3).reshape(G, nb * bk, d)[:, :T]
            blk_of = torch.arange(T, device=dev) // bk
            for g in range(G):
                p = torch.softmax((qf[b, g * r:(g + 1) * r] @ Kb[g].T) / math.sqrt(d), dim=-1)  # [r][T]
                for m, sel in sels.items():
                    ids = torch.from_numpy(sel[b, g][sel[b, g] >= 0].astype(np.int64)).to(dev)
                    on = torch.isin(blk_of, ids)
                    acc[m]["attn_mass"].extend(p[:, on].sum(dim=-1).cpu().tolist())
        for m, sel in sels.items():
            for b in range(B):
                nb = -(-lens[b] // bk)
                if nb <= k:
                    continue
                for g in range(G):
                    cand = np.arange(1, nb - 1)
                    ex = set(top_exact(lgx_np[b, g], nb, kp).tolist())
                    pick = [int(j) for j in sel[b, g] if 0 < j < nb - 1]
                    x = lgx_np[b, g, cand].astype(np.float64)
                    mx = x.max()
                    tot = np.exp(x - mx).sum()
                    cov = np.exp(lgx_np[b, g, pick].astype(np.float64) - mx).sum() / tot
                    cov_opt = np.exp(lgx_np[b, g, sorted(ex)].astype(np.float64) - mx).sum() / tot
                    acc[m]["recall"].append(len(ex & set(pick)) / kp)
                    acc[m]["coverage"].append(cov / cov_opt)
        log(f"{name} step {s}: recall taylor {np.mean(acc['taylor']['recall']):.4f} "
            f"mean {np.mean(acc['mean']['recall']):.4f}; mass kernel {mass_us[-1]:.1f} us")
    res = {m: {key: float(np.mean(v)) for key, v in acc[m].items()} for m in acc}
    t_us = float(np.median(mass_us))
    by = float(np.mean(mass_bytes))
    res["block_mass_kernel"] = {"us": t_us, "bytes_per_launch": by, "GBps": by / t_us / 1e3,
                                "frac_of_hbm_peak": by / t_us / 1e3 / HBM_PEAK_GBS}
    res["config"] = {"batch": B, "context": max(w.t0), "n_q_heads": H, "n_kv_heads": G, "head_dim": d,
                     "block_size": bk, "top_k": k, "steps": steps, "pairs_per_step": B * G}
    del L
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", default="llama_gqa_128k,batched_32k,million_1m")
    ap.add_argument("--steps", type=int, default=8)
    ap.add_argument("--timing-reps", type=int, default=10)
    args = ap.parse_args()
    out = {"study": "SPLA block-selection fidelity", "data": "synthetic (seeded; see workloads/)", "results": {}}
    for name in args.workloads.split(","):
        out["results"][name] = run_workload(name, args.steps, args.timing_reps)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
