"""Periodic Row-wise Muon optimizer step for MI355X (gfx950).

The computation runs in ``libmuon_hip.so`` (hand-written HIP kernels behind
the C ABI of include/muon.h).  ``binding`` mirrors that ABI name for name;
``MuonSession`` is a small convenience that lets PyTorch provide the device
memory (the state buffer) and the stream.  There is no CPU fallback: without
the built library, importing ``binding.lib()`` raises.
"""

from __future__ import annotations

from .binding import (  # noqa: F401
    EXPORTED, KERNEL_CLASSES, MUON_BF16, MUON_BRANCH_BLOCK_NS5, MUON_BRANCH_NS5, MUON_BRANCH_ROWNORM, MUON_F32,
    MUON_KIND_ADAMW, MUON_KIND_MATRIX, MUON_NS_BF16, MUON_NS_BF16_COMP, MUON_NS_F32, MuonConfig, MuonError,
    MuonTensor, lib, muon_branch, muon_config_default, muon_free, muon_init, muon_last_error,
    muon_state, muon_state_bytes, muon_status_str, muon_step, muon_step_noalloc, muon_sync,
    muon_tall_giveups,
    muon_tall_poll_limit, muon_timing_enable, muon_timing_read, tensor_desc)


class MuonSession:
    """One muon_ctx plus the torch-allocated state buffer it lives in.

    params: list of contiguous fp32 CUDA tensors (2-D -> Muon, else AdamW unless
    ``kinds`` says otherwise); grads: matching fp32 or bf16 tensors.
    """

    def __init__(self, params, grads, kinds=None, cfg: MuonConfig | None = None, stream=None,
                 **overrides):
        import torch
        self.cfg = cfg if cfg is not None else muon_config_default(**overrides)
        self.params = list(params)
        self.grads = list(grads)
        if kinds is None:
            kinds = [MUON_KIND_MATRIX if p.dim() == 2 else MUON_KIND_ADAMW for p in self.params]
        self.kinds = list(kinds)
        self.pdesc = [tensor_desc(p) for p in self.params]
        self.gdesc = [tensor_desc(g, d.rows, d.cols) for g, d in zip(self.grads, self.pdesc)]
        self.state_bytes = muon_state_bytes(self.cfg, self.pdesc, self.kinds)
        dev = self.params[0].device if self.params else torch.device("cuda")
        self.state = torch.empty(max(self.state_bytes, 256) + 256, dtype=torch.uint8, device=dev)
        off = (-self.state.data_ptr()) % 256
        self._base = self.state.data_ptr() + off
        self._off = off
        self.stream = stream if stream is not None else torch.cuda.current_stream(dev)
        self.ctx = muon_init(self.cfg, self.pdesc, self.gdesc, self.kinds, self._base,
                             self.state_bytes, self.stream.cuda_stream)

    def step(self, t: int, params=None, grads=None) -> None:
        pd = self.pdesc if params is None else [tensor_desc(p, d.rows, d.cols)
                                                for p, d in zip(params, self.pdesc)]
        gd = self.gdesc if grads is None else [tensor_desc(g, d.rows, d.cols)
                                               for g, d in zip(grads, self.pdesc)]
        muon_step(self.ctx, pd, gd, t)

    def state_view(self, i: int, which: int = 0):
        """fp32 torch view of momentum (which=0) or AdamW v (which=1) of param i."""
        import torch
        v = muon_state(self.ctx, i, which)
        start = v.ptr - self.state.data_ptr()
        n = v.rows * v.cols
        t = self.state[start:start + 4 * n].view(torch.float32)
        return t.view(v.rows, v.cols) if self.params[i].dim() == 2 else t.view(self.params[i].shape)

    def sync(self) -> None:
        """Wait for the stream; raises if a kernel failed."""
        muon_sync(self.ctx)

    def tall_giveups(self) -> int:
        """Waits of the single-pass tall RowNorm that gave up (and were repaired)."""
        return muon_tall_giveups(self.ctx)

    def branch(self, t: int) -> int:
        return muon_branch(self.cfg, t)

    def close(self) -> None:
        if getattr(self, "ctx", None) is not None:
            muon_free(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
