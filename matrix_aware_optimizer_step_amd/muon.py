"""Torch-facing marshalling for libmuon355.

PyTorch supplies device memory and the current HIP stream; this module turns
tensors into ``MuonBatch`` descriptors, sizes workspaces from the library's
own queries, and calls the C entry points in the order one Muon step needs
them ("Matrix optimizers: K-FAC, Shampoo and Muon", subsection "Muon",
steps 1-4).  It does no arithmetic on the tensors.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import _lib as L

QUINTIC = (3.4445, -4.7750, 2.0315)
EPS = 1e-7


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return L.MUON_BF16
    if t.dtype == torch.float32:
        return L.MUON_F32
    raise TypeError(f"libmuon355 takes bfloat16 or float32 matrices, not {t.dtype}")


@dataclass
class Batch:
    """A MuonBatch plus the tensors that must stay alive while it is in use."""
    desc: L.MuonBatch
    count: int
    rows: int
    cols: int
    keep: list = field(default_factory=list)
    owned: list = field(default_factory=list)  # device tensors batch() allocated (the pointer array)


def batch(x) -> Batch:
    """Descriptor for a 2-D tensor (one matrix), a 3-D tensor (strided batch,
    e.g. ``W.view(32, 128, 4096)`` for per-head row blocks), or a list of
    same-shape 2-D tensors (passed as a device pointer array)."""
    if isinstance(x, Batch):
        return x
    if isinstance(x, (list, tuple)):
        if not x:
            raise ValueError("empty list of matrices")
        t0 = x[0]
        for t in x:
            if t.shape != t0.shape or t.dtype != t0.dtype or t.device != t0.device or t.dim() != 2:
                raise ValueError("a pointer-array batch needs same-shape, same-dtype 2-D tensors")
            if t.stride(1) != 1 or t.stride(0) != t0.stride(0):
                raise ValueError("matrices must be row-major with one leading dimension")
            if t.is_sparse:
                raise RuntimeError("dense gradients required")
        ptrs = torch.tensor([t.data_ptr() for t in x], dtype=torch.int64, device=t0.device)
        d = L.MuonBatch(ptrs.data_ptr(), None, 0, len(x), t0.shape[0], t0.shape[1], t0.stride(0),
                        dtype_code(t0), 0)
        return Batch(d, len(x), t0.shape[0], t0.shape[1], [ptrs, *x], [ptrs])
    t = x
    if t.is_sparse:
        raise RuntimeError("dense gradients required")
    if t.dim() == 2:
        if t.stride(1) != 1:
            raise ValueError("matrices must be row-major (last stride 1)")
        d = L.MuonBatch(None, t.data_ptr(), 0, 1, t.shape[0], t.shape[1], t.stride(0), dtype_code(t), 0)
        return Batch(d, 1, t.shape[0], t.shape[1], [t])
    if t.dim() == 3:
        if t.stride(2) != 1:
            raise ValueError("matrices must be row-major (last stride 1)")
        d = L.MuonBatch(None, t.data_ptr(), t.stride(0), t.shape[0], t.shape[1], t.shape[2], t.stride(1),
                        dtype_code(t), 0)
        return Batch(d, t.shape[0], t.shape[1], t.shape[2], [t])
    raise ValueError("expected a 2-D or 3-D tensor or a list of 2-D tensors")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _stream_object(stream):
    """The torch stream object of a ``stream=`` argument (None: the current
    stream, which needs no bookkeeping)."""
    if stream is None or hasattr(stream, "cuda_stream"):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _record_on(stream, tensors) -> None:
    """Tensors this module allocated for one call and drops on return (a
    workspace, the device pointer array of a list input) are still read by
    the kernels enqueued on ``stream``.  The caching allocator ties a block
    to the stream it was allocated on (the current one); recording the
    launch stream keeps the block from going to new work before the kernels
    on that stream are done."""
    if stream is None:
        return
    for t in tensors:
        if t is not None and getattr(t, "is_cuda", False):
            t.record_stream(stream)


def _owned(batches) -> list:
    return [t for b in batches if b is not None for t in b.owned]


def momentum(grad, mom, nout, sumsq: torch.Tensor, beta: float = 0.95, nesterov: bool = True,
             ws: torch.Tensor | None = None, stream=None) -> None:
    g, m = batch(grad), batch(mom)
    n = batch(nout) if nout is not None else None
    need = L.muon_momentum_workspace(g.count, g.rows, g.cols)
    own_ws = ws is None
    if ws is None:
        ws = workspace(need, sumsq.device)
    L.muon_momentum(g.desc, m.desc, n.desc if n else None, sumsq.data_ptr(), beta, nesterov,
                    ws.data_ptr(), ws.numel(), _stream(stream))
    _record_on(_stream_object(stream), ([ws] if own_ws else []) + _owned([g, m, n]))


def momentum_grouped(grads, moms, nouts, sumsqs, beta: float = 0.95, nesterov: bool = True,
                     ws: torch.Tensor | None = None, stream=None) -> None:
    """muon_momentum over several shape classes in one launch; ``nouts`` may
    be None without Nesterov."""
    bg = [batch(x) for x in grads]
    bm = [batch(x) for x in moms]
    bn = None if nouts is None else [batch(x) for x in nouts]
    own_ws = ws is None
    if ws is None:
        need = L.muon_momentum_grouped_workspace([b.count for b in bg], [b.rows for b in bg], [b.cols for b in bg])
        ws = workspace(need, sumsqs[0].device)
    L.muon_momentum_grouped([b.desc for b in bg], [b.desc for b in bm], None if bn is None else [b.desc for b in bn],
                            [s.data_ptr() for s in sumsqs], beta, nesterov, ws.data_ptr(), ws.numel(), _stream(stream))
    _record_on(_stream_object(stream), ([ws] if own_ws else []) + _owned(bg + bm + (bn or [])))


def orthogonalize(inp, out, sumsq: torch.Tensor | None = None, steps: int = 5, coeffs=QUINTIC,
                  eps: float = EPS, compute: int = L.MUON_BF16, ws: torch.Tensor | None = None,
                  stream=None, device=None) -> None:
    i, o = batch(inp), batch(out)
    own_ws = ws is None
    if ws is None:
        need = L.muon_orthogonalize_workspace(i.count, i.rows, i.cols, compute)
        ws = workspace(need, device or (sumsq.device if sumsq is not None else i.keep[-1].device))
    a, b, c = coeffs
    L.muon_orthogonalize(i.desc, sumsq.data_ptr() if sumsq is not None else None, o.desc, steps, a, b, c,
                         eps, compute, ws.data_ptr(), ws.numel(), _stream(stream))
    _record_on(_stream_object(stream), ([ws] if own_ws else []) + _owned([i, o]))


def orthogonalize_grouped(ins, outs, sumsqs=None, steps: int = 5, coeffs=QUINTIC, eps: float = EPS,
                          compute: int = L.MUON_BF16, ws: torch.Tensor | None = None, stream=None,
                          device=None) -> None:
    bi = [batch(x) for x in ins]
    bo = [batch(x) for x in outs]
    own_ws = ws is None
    if ws is None:
        need = L.muon_orthogonalize_grouped_workspace([b.count for b in bi], [b.rows for b in bi],
                                                      [b.cols for b in bi], compute)
        ws = workspace(need, device)
    a, b, c = coeffs
    sp = None if sumsqs is None else [s.data_ptr() if s is not None else 0 for s in sumsqs]
    L.muon_orthogonalize_grouped([x.desc for x in bi], sp, [x.desc for x in bo], steps, a, b, c, eps, compute,
                                 ws.data_ptr(), ws.numel(), _stream(stream))
    _record_on(_stream_object(stream), ([ws] if own_ws else []) + _owned(bi + bo))


def apply(weight, ortho, lr: float, weight_decay: float, mode: int = L.MUON_SCALE_MATCH_RMS,
          coeff: float = 0.2, stream=None) -> None:
    w, o = batch(weight), batch(ortho)
    L.muon_apply(w.desc, o.desc, lr, weight_decay, mode, coeff, _stream(stream))
    _record_on(_stream_object(stream), _owned([w, o]))


def apply_grouped(weights, orthos, lr: float, weight_decay: float, mode: int = L.MUON_SCALE_MATCH_RMS,
                  coeff: float = 0.2, stream=None) -> None:
    """muon_apply over several shape classes in one launch."""
    # the Batch objects own the device pointer arrays of list inputs: keep
    # them alive across the call
    bw = [batch(x) for x in weights]
    bo = [batch(x) for x in orthos]
    L.muon_apply_grouped([b.desc for b in bw], [b.desc for b in bo], lr, weight_decay, mode, coeff, _stream(stream))
    _record_on(_stream_object(stream), _owned(bw + bo))


class MuonStep:
    """One Muon optimizer step over several same-shape groups of weights.

    ``groups`` is a list of ``(weights, grads)`` pairs, each element anything
    ``batch()`` accepts (a 2-D or 3-D tensor or a list of 2-D tensors).  The
    fp32 momentum, the Newton-Schulz output buffers, the sums of squares and
    the workspaces are allocated once here; ``step()`` only enqueues the
    library's kernels on the current stream.

    With ``packed`` (the default, for K >= 1 Newton-Schulz steps) the momentum
    kernel writes the Newton-Schulz input straight into the iteration's
    workspace (muon_momentum_packed_grouped, then
    muon_orthogonalize_packed_grouped), so N is never stored; otherwise N is
    an fp32 buffer between muon_momentum_grouped and
    muon_orthogonalize_grouped.  With ``fused_apply`` as well, the update is
    applied by the last Newton-Schulz step
    (muon_orthogonalize_apply_packed_grouped): O is never stored, and
    ``ortho_buffers`` raises.
    """

    def __init__(self, groups, *, compute: int = L.MUON_BF16, beta: float = 0.95, nesterov: bool = True,
                 steps: int = 5, coeffs=QUINTIC, eps: float = EPS, lr: float = 3e-4,
                 weight_decay: float = 0.1, mode: int = L.MUON_SCALE_MATCH_RMS, coeff: float = 0.2,
                 packed: bool = True, fused_apply: bool = False):
        if not groups:
            raise ValueError("no parameter groups")
        self.compute, self.beta, self.nesterov = compute, beta, nesterov
        self.steps, self.coeffs, self.eps = steps, coeffs, eps
        self.lr, self.weight_decay, self.mode, self.coeff = lr, weight_decay, mode, coeff
        self.w, self.g, self.m, self.n, self.o, self.ss = [], [], [], [], [], []
        dev = None
        for weights, grads in groups:
            w, g = batch(weights), batch(grads)
            if (w.count, w.rows, w.cols) != (g.count, g.rows, g.cols):
                raise ValueError("weights and gradients differ in shape")
            dev = w.keep[-1].device
            shape = (w.count, w.rows, w.cols)
            self.w.append(w)
            self.g.append(g)
            self.m.append(batch(torch.zeros(shape, dtype=torch.float32, device=dev)))
            self.ss.append(torch.empty(w.count, dtype=torch.float32, device=dev))
        self.device = dev
        # each stage runs the groups together, at most 8 per grouped launch
        self.chunks = [list(range(i, min(i + 8, len(self.w)))) for i in range(0, len(self.w), 8)]
        self.packed = bool(packed)
        self.fused_apply = bool(fused_apply) and self.packed
        if not self.fused_apply:
            self._ortho()
        self.pws, self.mws, self.ows = [], [], []
        if self.packed:
            for ch in self.chunks:
                need = L.muon_packed_grouped_workspace([self.g[i].count for i in ch], [self.g[i].rows for i in ch],
                                                       [self.g[i].cols for i in ch], compute)
                self.pws.append(workspace(need, dev))
        else:
            self._unpacked_buffers()

    def _ortho(self) -> None:
        """The Newton-Schulz outputs O (the weights' dtype); made on first use
        when the update is folded into the last step, which needs none."""
        if self.o:
            return
        for w in self.w:
            self.o.append(batch(torch.empty((w.count, w.rows, w.cols), dtype=w.keep[-1].dtype, device=self.device)))

    def _unpacked_buffers(self) -> None:
        """N (fp32 on both paths: the bf16 path's high/low copy of X starts
        from it, and a bf16-rounded start is the error that the iteration
        amplifies most on ill-conditioned inputs) and the workspaces of the
        separate calls; made on first use."""
        if self.mws:
            return
        for g in self.g:
            self.n.append(batch(torch.empty((g.count, g.rows, g.cols), dtype=torch.float32, device=self.device)))
        for ch in self.chunks:
            need = L.muon_momentum_grouped_workspace([self.g[i].count for i in ch], [self.g[i].rows for i in ch],
                                                     [self.g[i].cols for i in ch])
            self.mws.append(workspace(need, self.device))
            need = L.muon_orthogonalize_grouped_workspace([self.g[i].count for i in ch], [self.g[i].rows for i in ch],
                                                          [self.g[i].cols for i in ch], self.compute)
            self.ows.append(workspace(need, self.device))

    @property
    def momentum_buffers(self):
        return [m.keep[0] for m in self.m]

    @property
    def ortho_buffers(self):
        if self.fused_apply and self.steps >= 1:
            raise RuntimeError("with fused_apply the last Newton-Schulz step applies the update and O is never "
                               "stored; use a MuonStep without fused_apply to read O")
        self._ortho()
        return [o.keep[0] for o in self.o]

    @property
    def sumsq_buffers(self):
        return self.ss

    def state_dict(self) -> dict:
        """The state a resumed run needs: the fp32 momentum of every group
        (host copies) and the step's hyperparameters.  Plain tensors and
        Python values, so torch.save / torch.load(weights_only=True) round-trip
        it; the weights themselves are the caller's."""
        return {"momentum": [m.keep[0].detach().to("cpu", copy=True) for m in self.m],
                "hyper": {"beta": self.beta, "nesterov": bool(self.nesterov), "steps": self.steps,
                          "coeffs": [float(x) for x in self.coeffs], "eps": self.eps, "lr": self.lr,
                          "weight_decay": self.weight_decay, "mode": self.mode, "coeff": self.coeff}}

    def load_state_dict(self, state: dict) -> None:
        mom = state["momentum"]
        if len(mom) != len(self.m) or any(tuple(t.shape) != tuple(m.keep[0].shape) for m, t in zip(self.m, mom)):
            raise ValueError("the state was saved for differently shaped groups")
        for m, t in zip(self.m, mom):
            m.keep[0].copy_(t)
        h = state["hyper"]
        self.beta, self.nesterov, self.steps = h["beta"], h["nesterov"], h["steps"]
        self.coeffs, self.eps = tuple(h["coeffs"]), h["eps"]
        self.lr, self.weight_decay, self.mode, self.coeff = h["lr"], h["weight_decay"], h["mode"], h["coeff"]

    def step(self, stream=None, events=None) -> None:
        """Enqueue one step.  ``events``, if given, is four torch.cuda.Event
        objects recorded before momentum, before orthogonalization, before
        apply and after apply (phase timing on the same stream)."""
        st = stream if stream is not None else torch.cuda.current_stream()
        s = _stream(st)
        packed = self.packed and self.steps >= 1
        if not packed:
            self._unpacked_buffers()
        if not (packed and self.fused_apply):
            self._ortho()
        a, b, c = self.coeffs
        if events is not None:
            events[0].record(st)
        for k, ch in enumerate(self.chunks):
            sums = [self.ss[i].data_ptr() for i in ch]
            if packed:
                ws = self.pws[k]
                L.muon_momentum_packed_grouped([self.g[i].desc for i in ch], [self.m[i].desc for i in ch], sums,
                                               self.beta, self.nesterov, self.compute, ws.data_ptr(), ws.numel(), s)
            else:
                ws = self.mws[k]
                L.muon_momentum_grouped([self.g[i].desc for i in ch], [self.m[i].desc for i in ch],
                                        [self.n[i].desc for i in ch], sums, self.beta, self.nesterov, ws.data_ptr(),
                                        ws.numel(), s)
        if events is not None:
            events[1].record(st)
        for k, ch in enumerate(self.chunks):
            sums = [self.ss[i].data_ptr() for i in ch]
            if packed and self.fused_apply:
                ws = self.pws[k]
                L.muon_orthogonalize_apply_packed_grouped(sums, [self.w[i].desc for i in ch], self.steps, a, b, c,
                                                          self.eps, self.lr, self.weight_decay, self.mode,
                                                          self.coeff, self.compute, ws.data_ptr(), ws.numel(), s)
            elif packed:
                ws = self.pws[k]
                L.muon_orthogonalize_packed_grouped(sums, [self.o[i].desc for i in ch], self.steps, a, b, c, self.eps,
                                                    self.compute, ws.data_ptr(), ws.numel(), s)
            else:
                ws = self.ows[k]
                L.muon_orthogonalize_grouped([self.n[i].desc for i in ch], sums, [self.o[i].desc for i in ch],
                                             self.steps, a, b, c, self.eps, self.compute, ws.data_ptr(), ws.numel(),
                                             s)
        if events is not None:
            events[2].record(st)
        for ch in (self.chunks if not (packed and self.fused_apply) else []):
            L.muon_apply_grouped([self.w[i].desc for i in ch], [self.o[i].desc for i in ch], self.lr,
                                 self.weight_decay, self.mode, self.coeff, s)
        if events is not None:
            events[3].record(st)


# ---------------------------------------------------------------- AdamW

class AdamW:
    """AdamW over one parameter group, every tensor in one launch.

    The parameters Muon does not take (embeddings, output head, norms,
    biases) follow AdamW ("LLM Optimizers: From SGD and AdamW to SOAP, Muon,
    and Scalable Training", sections 5 and 6).  ``params`` and ``grads`` are
    lists of contiguous tensors of matching shapes, one dtype per list
    (bfloat16 or float32); the fp32 moments, the device tables of pointers,
    sizes and chunk offsets are built here once, so ``step()`` only enqueues
    ``muon_adamw``.  The gradients are read from the given tensors' storage
    at every step: copy new gradients into them.
    """

    def __init__(self, params, grads, *, lr: float = 1e-3, betas=(0.9, 0.999), eps: float = 1e-8,
                 weight_decay: float = 0.0):
        params, grads = list(params), list(grads)
        if not params or len(params) != len(grads):
            raise ValueError("need matching, non-empty lists of parameters and gradients")
        dev = params[0].device
        for p, g in zip(params, grads):
            if p.shape != g.shape:
                raise ValueError("parameter and gradient shapes differ")
            if p.is_sparse or g.is_sparse:
                raise RuntimeError("AdamW here takes dense gradients only")
            if not (p.is_contiguous() and g.is_contiguous()):
                raise ValueError("parameters and gradients must be contiguous")
            if p.device != dev or g.device != dev:
                raise ValueError("all tensors must be on one device")
            if p.dtype != params[0].dtype or g.dtype != grads[0].dtype:
                raise ValueError("one dtype per list")
        self.params, self.grads = params, grads
        self.exp_avg = [torch.zeros(p.shape, dtype=torch.float32, device=dev) for p in params]
        self.exp_avg_sq = [torch.zeros(p.shape, dtype=torch.float32, device=dev) for p in params]
        self.lr, self.betas, self.eps, self.weight_decay = lr, tuple(betas), eps, weight_decay
        self.t = 0

        def table(ts):
            return torch.tensor([t.data_ptr() for t in ts], dtype=torch.int64, device=dev)

        numels = [p.numel() for p in params]
        chunks = [0]
        for n in numels:
            chunks.append(chunks[-1] + (n + L.ADAMW_CHUNK - 1) // L.ADAMW_CHUNK)
        self._tables = [table(params), table(grads), table(self.exp_avg), table(self.exp_avg_sq),
                        torch.tensor(numels, dtype=torch.int64, device=dev),
                        torch.tensor(chunks, dtype=torch.int64, device=dev)]
        self.desc = L.MuonTensorList(len(params), chunks[-1], *[t.data_ptr() for t in self._tables],
                                     dtype_code(params[0]), dtype_code(grads[0]))
        self.elements = sum(numels)

    def step(self, stream=None) -> None:
        self.t += 1
        b1, b2 = self.betas
        L.muon_adamw(self.desc, self.t, self.lr, b1, b2, self.eps, self.weight_decay, _stream(stream))

    def state_dict(self) -> dict:
        """The step count, both moments of every tensor (host copies) and the
        hyperparameters."""
        return {"step": self.t, "exp_avg": [m.detach().to("cpu", copy=True) for m in self.exp_avg],
                "exp_avg_sq": [v.detach().to("cpu", copy=True) for v in self.exp_avg_sq],
                "hyper": {"lr": self.lr, "betas": list(self.betas), "eps": self.eps, "weight_decay": self.weight_decay}}

    def load_state_dict(self, state: dict) -> None:
        for key, own in (("exp_avg", self.exp_avg), ("exp_avg_sq", self.exp_avg_sq)):
            if len(state[key]) != len(own) or any(t.shape != o.shape for t, o in zip(state[key], own)):
                raise ValueError("the state was saved for differently shaped tensors")
        # copied into the existing buffers: the device pointer tables stay valid
        for key, own in (("exp_avg", self.exp_avg), ("exp_avg_sq", self.exp_avg_sq)):
            for o, t in zip(own, state[key]):
                o.copy_(t)
        self.t = int(state["step"])
        h = state["hyper"]
        self.lr, self.betas, self.eps, self.weight_decay = h["lr"], tuple(h["betas"]), h["eps"], h["weight_decay"]


# ------------------------------------------------------ routing helper

# Module names that mark an embedding or the output head wherever they sit
# in a parameter's dotted name (Hugging Face, GPT-2 and Meta Llama naming).
EMBEDDING_OR_HEAD_MODULES = frozenset({
    "embed", "embeds", "embedding", "embeddings", "embed_tokens", "tok_embeddings", "word_embeddings",
    "position_embeddings", "token_type_embeddings", "embed_positions", "wte", "wpe", "lm_head"})
# Names that are the output head only as a top-level module ("output.weight",
# "head.weight"); deeper in a model they name hidden projections (BERT's
# "attention.output.dense", an MLP's "output" layer) that belong to Muon.
TOP_LEVEL_HEAD_MODULES = frozenset({"output", "head", "classifier", "score"})


def is_muon_param(name: str, p: torch.Tensor, embedding_or_head_modules=EMBEDDING_OR_HEAD_MODULES,
                  top_level_head_modules=TOP_LEVEL_HEAD_MODULES) -> bool:
    """Muon takes the 2-D hidden weight matrices; embeddings, the output head
    and every tensor that is not 2-D (norms, biases) stay with AdamW ("LLM
    Optimizers: From SGD and AdamW to SOAP, Muon, and Scalable Training",
    sections 5-6 and 11.5).

    ``name`` is the parameter's dotted name.  Whole components are matched,
    never substrings: a module listed in ``embedding_or_head_modules``
    anywhere on the path marks an embedding or head; a module listed in
    ``top_level_head_modules`` does so only when it is the top-level module
    that owns the parameter (the path is ``<module>.<parameter>``).
    """
    if p.dim() != 2:
        return False
    parts = [c.lower() for c in name.split(".")]
    modules = parts[:-1]  # the last component names the parameter itself
    if any(c in embedding_or_head_modules for c in modules):
        return False
    if len(modules) == 1 and modules[0] in top_level_head_modules:
        return False
    return True


class OptimizerStep:
    """One optimizer step for a whole model in one call.

    ``named_params`` is a list of ``(name, parameter, gradient)`` triples.
    2-D hidden matrices go to Muon (one ``MuonStep``, same-shape matrices
    batched through pointer arrays); the rest go to AdamW, in a decayed group
    for tensors of two or more dimensions (embeddings, head) and an undecayed
    one for norms and biases, each split by dtype.  ``routing`` records the
    name of every parameter and where it went.
    """

    def __init__(self, named_params, *, compute: int = L.MUON_BF16, muon_lr: float = 3e-4,
                 muon_weight_decay: float = 0.1, adam_lr: float = 3e-4, adam_betas=(0.9, 0.999),
                 adam_eps: float = 1e-8, adam_weight_decay: float = 0.1, is_muon=is_muon_param):
        shapes = {}
        adam = {}
        self.routing = {}
        for name, p, g in named_params:
            if g is None:
                continue  # no gradient: the parameter takes no part in this step
            if is_muon(name, p):
                shapes.setdefault((tuple(p.shape), p.dtype, g.dtype), []).append((p, g))
                self.routing[name] = "muon"
            else:
                decay = p.dim() >= 2
                adam.setdefault((decay, p.dtype, g.dtype), []).append((p, g))
                self.routing[name] = "adamw" if decay else "adamw_no_decay"
        self.muon = None
        if shapes:
            groups = [([p for p, _ in v], [g for _, g in v]) for v in shapes.values()]
            self.muon = MuonStep(groups, compute=compute, lr=muon_lr, weight_decay=muon_weight_decay)
        self.adamw = [AdamW([p for p, _ in v], [g for _, g in v], lr=adam_lr, betas=adam_betas, eps=adam_eps,
                            weight_decay=adam_weight_decay if decay else 0.0)
                      for (decay, _, _), v in adam.items()]

    def step(self, stream=None) -> None:
        if self.muon is not None:
            self.muon.step(stream=stream)
        for group in self.adamw:
            group.step(stream=stream)

    def state_dict(self) -> dict:
        """Everything a resumed run needs besides the weights: the Muon
        momentum, every AdamW group's moments and step count, the
        hyperparameters and the routing they belong to."""
        return {"routing": dict(self.routing), "muon": None if self.muon is None else self.muon.state_dict(),
                "adamw": [g.state_dict() for g in self.adamw]}

    def load_state_dict(self, state: dict) -> None:
        if state["routing"] != self.routing or len(state["adamw"]) != len(self.adamw) or \
                (state["muon"] is None) != (self.muon is None):
            raise ValueError("the state was saved for a different set of parameters")
        if self.muon is not None:
            self.muon.load_state_dict(state["muon"])
        for g, s in zip(self.adamw, state["adamw"]):
            g.load_state_dict(s)
