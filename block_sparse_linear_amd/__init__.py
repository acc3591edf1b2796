"""Python binding of libspla.so, the SPLA decode step for MI355X (gfx950).

Argument marshalling only: every step of the decode path (append, score,
top-k, attend + correct, combine) runs in the HIP kernels of libspla.so.
PyTorch provides device memory and the stream.  The library must be built
(``python -m block_sparse_linear_amd.build``); importing this package
without it raises, there is no fallback.

    layer = SplaLayer(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
                      block_size=64, top_k=32, max_blocks_per_seq=2100,
                      kv_dtype="bf16")
    layer.append([0], [n], k, v)         # k, v: cuda [n][G][d]
    out = layer.decode(q, gate)          # q: cuda [B][H][d], gate: cuda [H] f32
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

__all__ = ["load_library", "SplaError", "SplaHandle", "SplaLayer", "STATUS", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspla.so")

STATUS = {
    0: "SPLA_OK", 1: "SPLA_ERR_INVALID_ARG", 2: "SPLA_ERR_UNSUPPORTED", 3: "SPLA_ERR_CAPACITY",
    4: "SPLA_ERR_ALIGNMENT", 5: "SPLA_ERR_HIP", 6: "SPLA_ERR_STATE", 7: "SPLA_ERR_SCRATCH",
}
SPLA_F32, SPLA_BF16 = 0, 1

EXPORTED = [
    "spla_create", "spla_destroy", "spla_workspace_bytes", "spla_stats_floats", "spla_bind",
    "spla_append_kv", "spla_decode", "spla_decode_step", "spla_get_lens", "spla_status_str", "spla_abi_version",
    "spla_last_hip_error", "spla_set_tuning", "spla_launch_plan", "spla_set_rla_output",
    "spla_set_score_form", "spla_block_mass", "spla_prefill_workspace_bytes", "spla_prefill",
    "spla_decode_step_noalloc",
]
# bytes of the library's static scratch (spla_decode_step_noalloc)
NOALLOC_SCRATCH_BYTES = 64 << 20

# spla_kernel ids (include/spla.h) -> kernel names
KERNELS = {1: "score", 2: "step_score", 3: "select", 4: "attend", 5: "select_attend", 6: "combine",
           7: "step_fused"}
CALL_DECODE, CALL_DECODE_SEL_IN, CALL_DECODE_STEP = 0, 1, 2
TUNE_FUSED_SELECT = 0
TUNE_STEP_KERNEL = 1
TUNE_FUSED_MERGE = 2
# output forms of the RLA branch (spla_rla_form)
RLA_PLAIN, RLA_NORMALIZED, RLA_RMSNORM = 0, 1, 2
# block scores the selection can rank (spla_score_form)
SCORE_TAYLOR, SCORE_MEAN = 0, 1


class SplaConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_q_heads", "n_kv_heads", "head_dim", "block_size", "top_k",
        "max_blocks_per_seq", "num_pages", "kv_dtype")]


class SplaBuffers(ctypes.Structure):
    _fields_ = [
        ("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
        ("blk_mean", ctypes.c_void_p), ("blk_var", ctypes.c_void_p), ("s_all", ctypes.c_void_p),
        ("z_all", ctypes.c_void_p), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


class SplaDecodeAux(ctypes.Structure):
    _fields_ = [
        ("sel_idx", ctypes.c_void_p), ("lg", ctypes.c_void_p), ("o_sparse", ctypes.c_void_p),
        ("o_rla", ctypes.c_void_p), ("d_rla", ctypes.c_void_p), ("sel_in", ctypes.c_void_p),
        ("kernel_events", ctypes.c_void_p), ("n_kernel_events", ctypes.c_int32),
    ]


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libspla.so and declare its signatures.  Raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    # torch ships its own HIP runtime (same soname); load it first so that
    # libspla.so binds to that runtime and shares torch's streams and memory
    import torch  # noqa: F401
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built: run `python -m block_sparse_linear_amd.build`")
    lib = ctypes.CDLL(p)
    I32P = ctypes.POINTER(ctypes.c_int32)
    lib.spla_create.argtypes = [ctypes.POINTER(SplaConfig), ctypes.POINTER(ctypes.c_void_p)]
    lib.spla_create.restype = ctypes.c_int
    lib.spla_destroy.argtypes = [ctypes.c_void_p]
    lib.spla_destroy.restype = None
    lib.spla_workspace_bytes.argtypes = [ctypes.c_void_p]
    lib.spla_workspace_bytes.restype = ctypes.c_size_t
    lib.spla_stats_floats.argtypes = [ctypes.c_void_p]
    lib.spla_stats_floats.restype = ctypes.c_size_t
    lib.spla_bind.argtypes = [ctypes.c_void_p, ctypes.POINTER(SplaBuffers), I32P]
    lib.spla_bind.restype = ctypes.c_int
    lib.spla_append_kv.argtypes = [ctypes.c_void_p, ctypes.c_int32, I32P, I32P, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p]
    lib.spla_append_kv.restype = ctypes.c_int
    lib.spla_decode.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.POINTER(SplaDecodeAux), ctypes.c_void_p]
    lib.spla_decode.restype = ctypes.c_int
    lib.spla_decode_step.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(SplaDecodeAux),
                                     ctypes.c_void_p]
    lib.spla_decode_step.restype = ctypes.c_int
    lib.spla_decode_step_noalloc.argtypes = lib.spla_decode_step.argtypes
    lib.spla_decode_step_noalloc.restype = ctypes.c_int
    lib.spla_get_lens.argtypes = [ctypes.c_void_p, I32P]
    lib.spla_get_lens.restype = ctypes.c_int
    lib.spla_status_str.argtypes = [ctypes.c_int]
    lib.spla_status_str.restype = ctypes.c_char_p
    lib.spla_abi_version.argtypes = []
    lib.spla_abi_version.restype = ctypes.c_int32
    lib.spla_last_hip_error.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_char_p)]
    lib.spla_last_hip_error.restype = ctypes.c_int32
    lib.spla_set_tuning.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32]
    lib.spla_set_tuning.restype = ctypes.c_int
    lib.spla_launch_plan.argtypes = [ctypes.c_void_p, ctypes.c_int32, I32P, ctypes.c_int32]
    lib.spla_launch_plan.restype = ctypes.c_int32
    lib.spla_set_rla_output.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float]
    lib.spla_set_rla_output.restype = ctypes.c_int
    lib.spla_set_score_form.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    lib.spla_set_score_form.restype = ctypes.c_int
    lib.spla_block_mass.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.spla_block_mass.restype = ctypes.c_int
    lib.spla_prefill_workspace_bytes.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    lib.spla_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.spla_prefill.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.spla_prefill.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


class SplaError(RuntimeError):
    def __init__(self, status: int, where: str, hip_error: Optional[str] = None):
        self.status = status
        self.name = STATUS.get(status, str(status))
        self.hip_error = hip_error
        super().__init__(f"{where}: {self.name}" + (f" ({hip_error})" if hip_error else ""))


def _check(st: int, where: str, lib=None, h=None) -> None:
    if st != 0:
        hip = None
        if st == 5 and lib is not None and h is not None:
            name = ctypes.c_char_p()
            code = lib.spla_last_hip_error(h, ctypes.byref(name))
            hip = f"hip error {code}: {name.value.decode() if name.value else '?'}"
        raise SplaError(st, where, hip)


def _i32_array(vals: Sequence[int]):
    arr = (ctypes.c_int32 * max(1, len(vals)))(*[int(v) for v in vals])
    return arr


class SplaHandle:
    """The library handle: configuration checks and the host length mirror.
    Creating one makes no HIP call."""

    def __init__(self, batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, block_size: int,
                 top_k: int, max_blocks_per_seq: int, num_pages: int, kv_dtype: str):
        self.lib = load_library()
        self.cfg = SplaConfig(batch, n_q_heads, n_kv_heads, head_dim, block_size, top_k,
                              max_blocks_per_seq, num_pages, SPLA_BF16 if kv_dtype == "bf16" else SPLA_F32)
        h = ctypes.c_void_p()
        _check(self.lib.spla_create(ctypes.byref(self.cfg), ctypes.byref(h)), "spla_create")
        self.h = h

    def __del__(self):
        h = getattr(self, "h", None)
        if h is not None and h.value:
            self.lib.spla_destroy(h)
            self.h = None

    @property
    def workspace_bytes(self) -> int:
        return int(self.lib.spla_workspace_bytes(self.h))

    @property
    def stats_floats(self) -> int:
        return int(self.lib.spla_stats_floats(self.h))

    def bind(self, bufs: SplaBuffers, lens: Optional[Sequence[int]] = None) -> None:
        arr = _i32_array(lens) if lens is not None else None
        _check(self.lib.spla_bind(self.h, ctypes.byref(bufs), arr), "spla_bind")

    def lens(self):
        arr = (ctypes.c_int32 * self.cfg.batch)()
        _check(self.lib.spla_get_lens(self.h, arr), "spla_get_lens")
        return list(arr)

    def set_tuning(self, key: int, value: int) -> None:
        _check(self.lib.spla_set_tuning(self.h, key, value), "spla_set_tuning")

    def set_rla_output(self, form: int, gamma_ptr: int = 0, eps: float = 0.0) -> None:
        _check(self.lib.spla_set_rla_output(self.h, form, ctypes.c_void_p(gamma_ptr), eps), "spla_set_rla_output")

    def set_score_form(self, form: int) -> None:
        _check(self.lib.spla_set_score_form(self.h, form), "spla_set_score_form")

    def prefill_workspace_bytes(self, chunk: int) -> int:
        return int(self.lib.spla_prefill_workspace_bytes(self.h, chunk))

    def prefill_raw(self, seq: int, n: int, k_ptr: int, v_ptr: int, q_ptr: int, gate_ptr: int, out_ptr: int,
                    sel_ptr: int, lg_ptr: int, ws_ptr: int, ws_bytes: int, stream: int) -> int:
        return self.lib.spla_prefill(self.h, seq, n, ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr),
                                     ctypes.c_void_p(q_ptr), ctypes.c_void_p(gate_ptr), ctypes.c_void_p(out_ptr),
                                     ctypes.c_void_p(sel_ptr or None), ctypes.c_void_p(lg_ptr or None),
                                     ctypes.c_void_p(ws_ptr), ws_bytes, ctypes.c_void_p(stream))

    def block_mass_raw(self, q_ptr: int, lgx_ptr: int, stream: int) -> int:
        return self.lib.spla_block_mass(self.h, ctypes.c_void_p(q_ptr), ctypes.c_void_p(lgx_ptr),
                                        ctypes.c_void_p(stream))

    def launch_plan(self, call: int):
        """Names of the kernels the next call of kind `call` launches, in order."""
        arr = (ctypes.c_int32 * 8)()
        n = self.lib.spla_launch_plan(self.h, call, arr, 8)
        if n < 0:
            raise ValueError(f"spla_launch_plan: bad call {call}")
        return [KERNELS[int(arr[i])] for i in range(n)]

    def append_raw(self, seq_ids, n_new, k_ptr: int, v_ptr: int, stream: int) -> int:
        return self.lib.spla_append_kv(self.h, len(seq_ids), _i32_array(seq_ids), _i32_array(n_new),
                                       ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr), ctypes.c_void_p(stream))

    def decode_raw(self, q_ptr: int, gate_ptr: int, out_ptr: int, aux: Optional[SplaDecodeAux],
                   stream: int) -> int:
        return self.lib.spla_decode(self.h, ctypes.c_void_p(q_ptr), ctypes.c_void_p(gate_ptr),
                                    ctypes.c_void_p(out_ptr), ctypes.byref(aux) if aux is not None else None,
                                    ctypes.c_void_p(stream))

    def decode_step_raw(self, k_ptr: int, v_ptr: int, q_ptr: int, gate_ptr: int, out_ptr: int,
                        aux: Optional[SplaDecodeAux], stream: int) -> int:
        return self.lib.spla_decode_step(self.h, ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr),
                                         ctypes.c_void_p(q_ptr), ctypes.c_void_p(gate_ptr),
                                         ctypes.c_void_p(out_ptr), ctypes.byref(aux) if aux is not None else None,
                                         ctypes.c_void_p(stream))


    def decode_step_noalloc_raw(self, k_ptr: int, v_ptr: int, q_ptr: int, gate_ptr: int, out_ptr: int,
                                aux: Optional[SplaDecodeAux], stream: int) -> int:
        return self.lib.spla_decode_step_noalloc(self.h, ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr),
                                                 ctypes.c_void_p(q_ptr), ctypes.c_void_p(gate_ptr),
                                                 ctypes.c_void_p(out_ptr),
                                                 ctypes.byref(aux) if aux is not None else None,
                                                 ctypes.c_void_p(stream))


class SplaLayer:
    """One SPLA attention layer's decode state in torch-allocated device memory.

    Buffers (see include/spla.h for layouts): k_pages, v_pages, block_table,
    blk_mean, blk_var, s_all, z_all, workspace.  ``page_order="shuffled"``
    maps block j of sequence b to a seeded random page (the library reads
    every page id through block_table)."""

    def __init__(self, batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, block_size: int,
                 top_k: int, max_blocks_per_seq: int, kv_dtype: str = "bf16", device: str = "cuda",
                 num_pages: Optional[int] = None, page_order: str = "identity", seed: int = 0):
        import torch

        self.torch = torch
        self.B, self.H, self.G, self.d = batch, n_q_heads, n_kv_heads, head_dim
        self.bk, self.top_k, self.mb = block_size, top_k, max_blocks_per_seq
        self.kv_dtype = kv_dtype
        self.dtype = torch.bfloat16 if kv_dtype == "bf16" else torch.float32
        dv = torch.device(device)
        if dv.type == "cuda" and dv.index is None:
            dv = torch.device("cuda", torch.cuda.current_device())
        self.device = dv
        npages = num_pages or batch * max_blocks_per_seq
        self.num_pages = npages
        self.handle = SplaHandle(batch, n_q_heads, n_kv_heads, head_dim, block_size, top_k,
                                 max_blocks_per_seq, npages, kv_dtype)
        dev = self.device
        self.k_pages = torch.zeros((npages, n_kv_heads, block_size, head_dim), dtype=self.dtype, device=dev)
        self.v_pages = torch.zeros_like(self.k_pages)
        if page_order == "shuffled":
            g = torch.Generator().manual_seed(seed)
            perm = torch.randperm(npages, generator=g)[: batch * max_blocks_per_seq]
            bt = perm.reshape(batch, max_blocks_per_seq).to(torch.int32)
        else:
            bt = torch.arange(batch * max_blocks_per_seq, dtype=torch.int32).reshape(batch, max_blocks_per_seq)
        self.block_table = bt.to(dev)
        nf = self.handle.stats_floats
        self.blk_mean = torch.zeros(nf, dtype=torch.float32, device=dev)
        self.blk_var = torch.zeros(nf, dtype=torch.float32, device=dev)
        self.s_all = torch.zeros((batch, n_kv_heads, head_dim, head_dim), dtype=torch.float32, device=dev)
        self.z_all = torch.zeros((batch, n_kv_heads, head_dim), dtype=torch.float32, device=dev)
        self.workspace = torch.zeros(self.handle.workspace_bytes // 4 + 64, dtype=torch.int32, device=dev)
        self._bind(None)

    def _buffers(self) -> SplaBuffers:
        return SplaBuffers(self.k_pages.data_ptr(), self.v_pages.data_ptr(), self.block_table.data_ptr(),
                           self.blk_mean.data_ptr(), self.blk_var.data_ptr(), self.s_all.data_ptr(),
                           self.z_all.data_ptr(), self.workspace.data_ptr(), self.workspace.numel() * 4)

    def _bind(self, lens) -> None:
        self.handle.bind(self._buffers(), lens)

    @property
    def lens(self):
        return self.handle.lens()

    def set_fused_select(self, mode: int) -> None:
        """-1 automatic, 0 stand-alone selector, 1 fused select + attend where supported."""
        self.handle.set_tuning(TUNE_FUSED_SELECT, mode)

    def set_fused_merge(self, mode: int) -> None:
        """1: the fused select + attend merges the records itself where it
        supports the call (no combine kernel); -1 automatic and 0: the combine
        kernel."""
        self.handle.set_tuning(TUNE_FUSED_MERGE, mode)

    def set_step_kernel(self, mode: int) -> None:
        """1: decode_step in one kernel (plus the combine) wherever the fused
        select + attend runs; -1 automatic and 0: the separate kernels."""
        self.handle.set_tuning(TUNE_STEP_KERNEL, mode)

    def set_rla_output(self, form: int = RLA_PLAIN, gamma=None, eps: float = 1e-6) -> None:
        """Output form of the RLA branch: RLA_PLAIN (o_rla), RLA_NORMALIZED
        (o_rla / D) or RLA_RMSNORM (gamma * o_rla / rms(o_rla), gamma a float32
        device tensor [H][d] that the layer keeps a reference to)."""
        if form == RLA_RMSNORM:
            t = self.torch
            if gamma is None:
                raise ValueError("the RMS-normalised form needs gamma")
            g = gamma.to(device=self.device, dtype=t.float32).contiguous()
            if tuple(g.shape) != (self.H, self.d):
                raise ValueError(f"gamma must be [{self.H}][{self.d}], got {tuple(g.shape)}")
            self.handle.set_rla_output(form, g.data_ptr(), float(eps))
            self._rla_gamma = g
        else:
            self.handle.set_rla_output(form, 0, 0.0)
            self._rla_gamma = None

    def set_score_form(self, form: int = SCORE_TAYLOR) -> None:
        """Block score the selection ranks: SCORE_TAYLOR or SCORE_MEAN."""
        self.handle.set_score_form(form)

    def prefill(self, seq: int, k_new, v_new, q, gate, out=None, chunk: int = 256, workspace=None, sel_idx=None,
                lg=None):
        """Chunked prefill of sequence seq: append k_new / v_new ([n][G][d]) and
        return out [n][H][d] float32, the decode output of every new token's
        query q ([n][H][d]) at its own position.  chunk: tokens per group of
        launches (the prefill workspace is sized for it unless given).
        sel_idx: optional int32 [n][G][top_k] receiving the selections; lg:
        optional float32 [n][G][MB] receiving the group log scores of every
        token's candidate blocks (other entries untouched)."""
        t = self.torch
        n = int(k_new.shape[0])
        self._check_kv(k_new, v_new, n)
        if q.dtype != self.dtype or tuple(q.shape) != (n, self.H, self.d) or not q.is_contiguous():
            raise ValueError(f"q must be a contiguous [{n}][{self.H}][{self.d}] tensor of the layer dtype")
        if gate.dtype != t.float32 or gate.numel() != self.H:
            raise ValueError("gate must be float32 [H]")
        if out is None:
            out = t.empty((n, self.H, self.d), dtype=t.float32, device=self.device)
        if workspace is None:
            nbytes = self.handle.prefill_workspace_bytes(max(1, min(chunk, 256)))
            workspace = t.empty(nbytes // 4 + 64, dtype=t.int32, device=self.device)
        if sel_idx is not None and (sel_idx.dtype != t.int32 or tuple(sel_idx.shape) != (n, self.G, self.top_k)
                                    or not sel_idx.is_contiguous()):
            raise ValueError(f"sel_idx must be a contiguous int32 [{n}][{self.G}][{self.top_k}] tensor")
        if lg is not None and (lg.dtype != t.float32 or tuple(lg.shape) != (n, self.G, self.mb)
                               or not lg.is_contiguous()):
            raise ValueError(f"lg must be a contiguous float32 [{n}][{self.G}][{self.mb}] tensor")
        st = self.handle.prefill_raw(seq, n, k_new.data_ptr(), v_new.data_ptr(), q.data_ptr(), gate.data_ptr(),
                                     out.data_ptr(), 0 if sel_idx is None else sel_idx.data_ptr(),
                                     0 if lg is None else lg.data_ptr(),
                                     workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                     self._stream())
        _check(st, "spla_prefill", self.handle.lib, self.handle.h)
        return out

    def block_mass(self, q, lgx=None):
        """Exact group log mass of every candidate block ([B][G][MB] float32;
        entries outside 1..nb-2 keep what lgx held, -inf for a new tensor)."""
        t = self.torch
        if q.dtype != self.dtype or tuple(q.shape) != (self.B, self.H, self.d) or not q.is_contiguous():
            raise ValueError("q must be a contiguous [B][H][d] tensor of the layer dtype")
        if lgx is None:
            lgx = t.full((self.B, self.G, self.mb), float("-inf"), dtype=t.float32, device=self.device)
        if lgx.dtype != t.float32 or tuple(lgx.shape) != (self.B, self.G, self.mb) or not lgx.is_contiguous():
            raise ValueError("lgx must be a contiguous float32 [B][G][MB] tensor")
        st = self.handle.block_mass_raw(q.data_ptr(), lgx.data_ptr(), self._stream())
        _check(st, "spla_block_mass", self.handle.lib, self.handle.h)
        return lgx

    def launch_plan(self, step: bool = True, sel_in: bool = False):
        call = CALL_DECODE_STEP if step else (CALL_DECODE_SEL_IN if sel_in else CALL_DECODE)
        return self.handle.launch_plan(call)

    def _stream(self) -> int:
        return self.torch.cuda.current_stream(self.device).cuda_stream

    def append(self, seq_ids: Sequence[int], n_new: Sequence[int], k_new, v_new) -> None:
        """k_new, v_new: device tensors [sum n_new][G][d] of the layer's dtype."""
        self._check_kv(k_new, v_new, sum(int(n) for n in n_new))
        st = self.handle.append_raw(list(seq_ids), list(n_new), k_new.data_ptr(), v_new.data_ptr(), self._stream())
        _check(st, "spla_append_kv", self.handle.lib, self.handle.h)

    def _check_kv(self, k_new, v_new, rows: int) -> None:
        for x in (k_new, v_new):
            if x.dtype != self.dtype or x.device != self.device or not x.is_contiguous():
                raise ValueError("k_new / v_new must be contiguous device tensors of the layer dtype")
            if x.dim() != 3 or x.shape[1:] != (self.G, self.d) or x.shape[0] < rows:
                raise ValueError(f"k_new / v_new must be [rows][{self.G}][{self.d}]")

    def _decode_inputs(self, q, gate, out, aux, kernel_events):
        t = self.torch
        if q.dtype != self.dtype or tuple(q.shape) != (self.B, self.H, self.d) or not q.is_contiguous():
            raise ValueError("q must be a contiguous [B][H][d] tensor of the layer dtype")
        if gate.dtype != t.float32 or gate.numel() != self.H:
            raise ValueError("gate must be float32 [H]")
        if out is None:
            out = t.empty((self.B, self.H, self.d), dtype=t.float32, device=self.device)
        ax = None
        if aux or kernel_events is not None:
            aux = aux or {}
            shapes = {"sel_idx": (self.B, self.G, self.top_k), "lg": (self.B, self.G, self.mb),
                      "o_sparse": (self.B, self.H, self.d), "o_rla": (self.B, self.H, self.d),
                      "d_rla": (self.B, self.H), "sel_in": (self.B, self.G, self.top_k)}
            ptrs = {}
            for k, v in aux.items():
                if k not in shapes:
                    raise KeyError(k)
                want = t.int32 if k in ("sel_idx", "sel_in") else t.float32
                if v.dtype != want or tuple(v.shape) != shapes[k] or not v.is_contiguous():
                    raise ValueError(f"aux[{k}] must be contiguous {want} {shapes[k]}")
                ptrs[k] = v.data_ptr()
            ev_ptr, n_ev = None, 0
            if kernel_events is not None:
                ev_ptr = ctypes.cast(kernel_events, ctypes.c_void_p).value
                n_ev = len(kernel_events) // 2
            ax = SplaDecodeAux(ptrs.get("sel_idx"), ptrs.get("lg"), ptrs.get("o_sparse"), ptrs.get("o_rla"),
                               ptrs.get("d_rla"), ptrs.get("sel_in"), ev_ptr, n_ev)
        return out, ax

    def decode_step(self, k_new, v_new, q, gate, out=None, aux: Optional[Dict[str, object]] = None,
                    kernel_events=None):
        """append one token to every sequence (k_new, v_new: device [B][G][d])
        and decode (spla_decode_step).  Same results as append + decode."""
        self._check_kv(k_new, v_new, self.B)
        out, ax = self._decode_inputs(q, gate, out, aux, kernel_events)
        st = self.handle.decode_step_raw(k_new.data_ptr(), v_new.data_ptr(), q.data_ptr(), gate.data_ptr(),
                                         out.data_ptr(), ax, self._stream())
        _check(st, "spla_decode_step", self.handle.lib, self.handle.h)
        return out

    def decode_step_noalloc(self, k_new, v_new, q, gate, out, aux: Optional[Dict[str, object]] = None):
        """decode_step through spla_decode_step_noalloc: the per-call scratch
        comes from the library's static device array, not the workspace.  out
        must be given (device [B][H][d] float32): nothing is allocated."""
        self._check_kv(k_new, v_new, self.B)
        if out is None:
            raise ValueError("decode_step_noalloc needs an output tensor")
        out, ax = self._decode_inputs(q, gate, out, aux, None)
        st = self.handle.decode_step_noalloc_raw(k_new.data_ptr(), v_new.data_ptr(), q.data_ptr(), gate.data_ptr(),
                                                 out.data_ptr(), ax, self._stream())
        _check(st, "spla_decode_step_noalloc", self.handle.lib, self.handle.h)
        return out

    def decode(self, q, gate, out=None, aux: Optional[Dict[str, object]] = None, kernel_events=None):
        """q: device [B][H][d] layer dtype; gate: device [H] float32.  aux may
        hold tensors under 'sel_idx', 'lg', 'o_sparse', 'o_rla', 'd_rla'
        (outputs) and 'sel_in' (input).  kernel_events: optional ctypes array
        of hipEvent_t handles (2 per launched kernel, see include/spla.h).
        Returns out [B][H][d] float32."""
        out, ax = self._decode_inputs(q, gate, out, aux, kernel_events)
        st = self.handle.decode_raw(q.data_ptr(), gate.data_ptr(), out.data_ptr(), ax, self._stream())
        _check(st, "spla_decode", self.handle.lib, self.handle.h)
        return out

    # ----------------------------------------------------------- helpers
    def stats(self):
        """(mean, var) as [B][G][NT*64][d] views of the tiled statistics."""
        nt = -(-self.mb // 64)
        def unpack(x):
            return (x.view(self.B, self.G, nt, self.d // 4, 64, 4).permute(0, 1, 2, 4, 3, 5)
                    .reshape(self.B, self.G, nt * 64, self.d))
        return unpack(self.blk_mean), unpack(self.blk_var)

    def error_word(self) -> int:
        return int(self.workspace[0].item())

    def clear_error(self) -> None:
        self.workspace[0] = 0

    def state_tensors(self):
        return [self.k_pages, self.v_pages, self.blk_mean, self.blk_var, self.s_all, self.z_all]

    def snapshot(self):
        return [x.clone() for x in self.state_tensors()], self.lens

    def restore(self, snap) -> None:
        tensors, lens = snap
        for dst, src in zip(self.state_tensors(), tensors):
            dst.copy_(src)
        self._bind(lens)
