"""Device-side driver of one workload: allocation with torch, compute in
``libcpattn.so``.

``CPProblem`` holds one workload's Q, K, V on the GPU, their zigzag
partitions and the buffers of one rank's forward share, and issues the
C-ABI calls in the method's order (split, cp steps, merge).  Torch only
allocates memory and provides the stream; every step of the path runs in
the library's kernels.
"""
import numpy as np
import torch

from . import cpattn as C
from .inputs import Workload


def to_device(x: np.ndarray, device="cuda") -> torch.Tensor:
    """Host input array (float32, or uint16 bf16 bits) -> device tensor."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(
            torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Device bf16 tensor -> host uint16 bit pattern."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


class CPProblem:
    """cu_seqlens: optional packing offsets (host, nseq + 1 entries): the
    batch elements then pack independent samples, each split on its own
    (cpattn_partition_varlen, cpattn_forward_fused_varlen)."""

    def __init__(self, w: Workload, q, k, v, s=None, device="cuda", cu_seqlens=None):
        self.w = w
        self.cu = None if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
        self.s = w.s if s is None else s
        self.b = q.shape[0]
        self.cp = w.cp
        self.c = self.s // (2 * self.cp)
        self.dims = C.make_dims(self.b, self.s, w.hq, w.hkv, w.d, w.cp)
        self.dtype = C.CPATTN_BF16 if w.dtype == "bf16" else C.CPATTN_F32
        self.tdtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.device = device
        self.q = to_device(q, device) if isinstance(q, np.ndarray) else q
        self.k = to_device(k, device) if isinstance(k, np.ndarray) else k
        self.v = to_device(v, device) if isinstance(v, np.ndarray) else v
        two_c = 2 * self.c
        self.qz = torch.empty((self.cp, self.b, two_c, w.hq, w.d), dtype=self.tdtype,
                              device=device)
        self.kz = torch.empty((self.cp, self.b, two_c, w.hkv, w.d), dtype=self.tdtype,
                              device=device)
        self.vz = torch.empty_like(self.kz)
        self.pos = torch.empty((self.cp, two_c), dtype=torch.int32, device=device)

    # --- step 1: split -----------------------------------------------------
    def partition(self, stream=None):
        theta = self.w.rope_theta
        if self.cu is not None:
            for h, x, xz, pos, th in ((self.w.hq, self.q, self.qz, self.pos, theta),
                                      (self.w.hkv, self.k, self.kz, None, theta),
                                      (self.w.hkv, self.v, self.vz, None, None)):
                C.cpattn_partition_varlen(self.dims, self.dtype, h, self.cu, x, xz, pos, th,
                                          stream)
            return
        C.cpattn_partition(self.dims, self.dtype, self.w.hq, self.q, self.qz, self.pos,
                           theta, stream)
        C.cpattn_partition(self.dims, self.dtype, self.w.hkv, self.k, self.kz, None,
                           theta, stream)
        C.cpattn_partition(self.dims, self.dtype, self.w.hkv, self.v, self.vz, None,
                           None, stream)

    def partition_one(self, which, stream=None):
        """The split of one tensor ("q", "k" or "v"; unpacked batches)."""
        h, x, xz, pos, theta = {"q": (self.w.hq, self.q, self.qz, self.pos, self.w.rope_theta),
                                "k": (self.w.hkv, self.k, self.kz, None, self.w.rope_theta),
                                "v": (self.w.hkv, self.v, self.vz, None, None)}[which]
        C.cpattn_partition(self.dims, self.dtype, h, x, xz, pos, theta, stream)

    # --- one rank's share ----------------------------------------------------
    def alloc_rank(self, rank, out_dtype=None):
        """Workspace, step partial views and outputs for ``rank``."""
        out_dtype = self.dtype if out_dtype is None else out_dtype
        ws_bytes = C.cpattn_forward_workspace(self.dims, rank)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=self.device)
        two_c = 2 * self.c
        o = torch.empty((self.b, two_c, self.w.hq, self.w.d),
                        dtype=torch.bfloat16 if out_dtype == C.CPATTN_BF16 else torch.float32,
                        device=self.device)
        lse = torch.empty((self.b, self.w.hq, two_c), dtype=torch.float32, device=self.device)
        # each step's partial where cpattn_forward_steps writes it
        steps = []
        base = ws.data_ptr()
        parts = C.cpattn_forward_partials(self.dims, rank, ws, ws_bytes)
        for i, (o_addr, l_addr, row0, rows) in enumerate(parts):
            mode, src = C.cpattn_step_mode(i, rank, self.cp)
            n_o = self.b * rows * self.w.hq * self.w.d
            n_l = self.b * self.w.hq * rows
            po = ws[o_addr - base:o_addr - base + 4 * n_o].view(torch.float32)
            pl = ws[l_addr - base:l_addr - base + 4 * n_l].view(torch.float32)
            steps.append(dict(mode=mode, src=src, rows=rows, row0=row0,
                              o=po.view(self.b, rows, self.w.hq, self.w.d),
                              lse=pl.view(self.b, self.w.hq, rows)))
        return dict(ws=ws, ws_bytes=ws_bytes, o=o, lse=lse, steps=steps, out_dtype=out_dtype,
                    rank=rank)

    def step(self, buf, i, stream=None, scale=0.0):
        st = buf["steps"][i]
        C.cpattn_step_fwd(self.dims, self.dtype, scale, st["mode"], self.qz[buf["rank"]],
                          self.kz[st["src"]], self.vz[st["src"]], st["o"], st["lse"], stream)

    def steps(self, buf, stream=None, scale=0.0):
        """All cp steps of the rank's share through cpattn_forward_steps (one
        grid for bf16), the partials landing in buf's step views."""
        C.cpattn_forward_steps(self.dims, self.dtype, scale, buf["rank"], self.qz, self.kz,
                               self.vz, buf["ws"], buf["ws_bytes"], stream)

    def merge(self, buf, stream=None):
        parts = [(st["o"], st["lse"], st["row0"], st["rows"]) for st in buf["steps"]]
        C.cpattn_merge(self.dims, parts, buf["out_dtype"], buf["o"], buf["lse"], stream)

    def forward(self, buf, stream=None, scale=0.0):
        """The whole share through the single entry point cpattn_forward."""
        C.cpattn_forward(self.dims, self.dtype, scale, buf["rank"], self.qz, self.kz, self.vz,
                         buf["ws"], buf["ws_bytes"], buf["out_dtype"], buf["o"], buf["lse"],
                         stream)

    # --- the same share in one launch ----------------------------------------
    def alloc_out(self, rank, out_dtype=None):
        """Output buffers of ``rank``'s share (the fused form needs no workspace)."""
        out_dtype = self.dtype if out_dtype is None else out_dtype
        two_c = 2 * self.c
        o = torch.empty((self.b, two_c, self.w.hq, self.w.d),
                        dtype=torch.bfloat16 if out_dtype == C.CPATTN_BF16 else torch.float32,
                        device=self.device)
        lse = torch.empty((self.b, self.w.hq, two_c), dtype=torch.float32, device=self.device)
        return dict(o=o, lse=lse, out_dtype=out_dtype, rank=rank)

    def forward_fused(self, out, stream=None, scale=0.0, with_lse=True):
        """The whole share through cpattn_forward_fused (one launch)."""
        if self.cu is not None:
            C.cpattn_forward_fused_varlen(self.dims, self.dtype, scale, out["rank"], self.cu,
                                          self.qz, self.kz, self.vz, out["out_dtype"],
                                          out["o"], out["lse"] if with_lse else None, stream)
            return
        C.cpattn_forward_fused(self.dims, self.dtype, scale, out["rank"], self.qz, self.kz,
                               self.vz, out["out_dtype"], out["o"],
                               out["lse"] if with_lse else None, stream)

    # --- backward of one rank's share ------------------------------------------
    def alloc_grads(self, rank):
        """Gradient buffers of ``rank``'s backward share (fp32)."""
        two_c = 2 * self.c
        f = dict(dtype=torch.float32, device=self.device)
        return dict(rank=rank,
                    delta=torch.empty((2, self.b, self.w.hq, two_c), **f),
                    dq=torch.empty((self.b, two_c, self.w.hq, self.w.d), **f),
                    dkz=torch.empty((self.cp, self.b, two_c, self.w.hkv, self.w.d), **f),
                    dvz=torch.empty((self.cp, self.b, two_c, self.w.hkv, self.w.d), **f))

    def backward(self, grads, o_r, lse_r, do_r, stream=None, scale=0.0):
        """The rank's backward share through cpattn_backward."""
        if self.cu is not None:
            C.cpattn_backward_varlen(self.dims, self.dtype, scale, grads["rank"], self.cu,
                                     self.qz, self.kz, self.vz, o_r, do_r, lse_r,
                                     grads["delta"], grads["dq"], grads["dkz"], grads["dvz"],
                                     stream)
            return
        C.cpattn_backward(self.dims, self.dtype, scale, grads["rank"], self.qz, self.kz,
                          self.vz, o_r, do_r, lse_r, grads["delta"], grads["dq"], grads["dkz"],
                          grads["dvz"], stream)

