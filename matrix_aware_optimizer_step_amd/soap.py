"""SOAP on libmuon355: Adam run in the eigenbasis of Shampoo's row and column
statistics ("LLM Optimizers: From SGD and AdamW to SOAP, Muon, and Scalable
Training", sections 11.1-11.2; "初探优化器（一）：从SGD到SOAP-Muon", section
6.2).

Torch tensors supply device memory and the stream only; every step runs in
the library's kernels through the ``soap_*`` entry points of
include/muon355.h, and the weight update through ``muon_apply`` with no
shape factor.
"""

from __future__ import annotations

import torch

from . import _lib as L
from .muon import _owned, _record_on, _stream, _stream_object, batch, workspace

# Adam's defaults ("LLM Optimizers", section 6); 0.9 for the statistics as
# reported for the SOAP-Muon records ("初探优化器（一）", 7.2); refresh
# every 10 steps, the guide's staleness example; axes above 8192 keep the
# identity basis (the guide's identity basis on very large axes).
BETA1 = 0.9
BETA2 = 0.999
EPS = 1e-8
BETA_S = 0.9
FREQ = 10
MAX_DIM = 8192


def _batches(*xs):
    """Batches for optional operands.  The caller keeps the returned list
    alive across the library call: a list of tensors is passed as a device
    pointer array that its Batch owns."""
    return [None if x is None else batch(x) for x in xs]


def _desc(b):
    return None if b is None else b.desc


def statistics(grad, Lstat=None, Rstat=None, beta_s: float = BETA_S, stream=None) -> None:
    """L <- b L + (1-b) G G^T and R <- b R + (1-b) G^T G (either may be None)."""
    bs = _batches(grad, Lstat, Rstat)
    L.soap_statistics(*map(_desc, bs), beta_s, _stream(stream))
    _record_on(_stream_object(stream), _owned(bs))


def statistics_grouped(grads, Lstats, Rstats, beta_s: float = BETA_S, stream=None) -> None:
    """statistics() for up to 8 groups in one call: the products of all
    groups share launches."""
    bg = [batch(x) for x in grads]
    bl, br = ([None if x is None else batch(x) for x in xs] for xs in (Lstats, Rstats))
    L.soap_statistics_grouped([b.desc for b in bg], [_desc(b) for b in bl], [_desc(b) for b in br], beta_s,
                              _stream(stream))
    _record_on(_stream_object(stream), _owned(bg + bl + br))


def qr(a, q, ws: torch.Tensor | None = None, stream=None) -> None:
    """q = the Q factor of a (square, f32), R's diagonal non-negative."""
    ba, bq = batch(a), batch(q)
    need = L.soap_qr_workspace(ba.count, ba.rows)
    own_ws = ws is None
    if ws is None:
        ws = workspace(need, bq.keep[-1].device)
    L.soap_qr(ba.desc, bq.desc, ws.data_ptr(), ws.numel(), _stream(stream))
    _record_on(_stream_object(stream), ([ws] if own_ws else []) + _owned([ba, bq]))


def refresh(mbar, Lstat=None, Rstat=None, QL=None, QR=None, ws: torch.Tensor | None = None, stream=None) -> None:
    """QL <- qr(L QL), QR <- qr(R QR), mbar carried into the new bases."""
    bs = _batches(Lstat, Rstat, QL, QR, mbar)
    bm = bs[-1]
    need = L.soap_refresh_workspace(bm.count, bm.rows, bm.cols, Lstat is not None, Rstat is not None)
    own_ws = ws is None
    if ws is None:
        ws = workspace(need, bm.keep[-1].device)
    L.soap_refresh(*map(_desc, bs), ws.data_ptr(), ws.numel(), _stream(stream))
    _record_on(_stream_object(stream), ([ws] if own_ws else []) + _owned(bs))


def refresh_grouped(mbars, Lstats, Rstats, QLs, QRs, ws: torch.Tensor | None = None, stream=None) -> None:
    """refresh() for up to 8 groups in one call: every QR of one order over
    all groups and sides runs as one batched factorization."""
    bm = [batch(x) for x in mbars]
    bl, br, bql, bqr = ([None if x is None else batch(x) for x in xs] for xs in (Lstats, Rstats, QLs, QRs))
    own_ws = ws is None
    if ws is None:
        need = L.soap_refresh_grouped_workspace([b.count for b in bm], [b.rows for b in bm], [b.cols for b in bm],
                                                [x is not None for x in Lstats], [x is not None for x in Rstats])
        ws = workspace(need, bm[0].keep[-1].device)
    L.soap_refresh_grouped([_desc(b) for b in bl], [_desc(b) for b in br], [_desc(b) for b in bql],
                           [_desc(b) for b in bqr], [b.desc for b in bm], ws.data_ptr(), ws.numel(), _stream(stream))
    _record_on(_stream_object(stream), ([ws] if own_ws else []) + _owned(bm + bl + br + bql + bqr))


def precondition(grad, mbar, vbar, out, step: int, QL=None, QR=None, beta1: float = BETA1, beta2: float = BETA2,
                 eps: float = EPS, ws: torch.Tensor | None = None, stream=None) -> None:
    """out = QL [Adam's direction of QL^T G QR in the rotated basis] QR^T."""
    bs = _batches(grad, QL, QR, mbar, vbar, out)
    bg = bs[0]
    need = L.soap_precondition_workspace(bg.count, bg.rows, bg.cols)
    own_ws = ws is None
    if ws is None:
        ws = workspace(need, bg.keep[-1].device)
    L.soap_precondition(*map(_desc, bs), step, beta1, beta2, eps, ws.data_ptr(), ws.numel(), _stream(stream))
    _record_on(_stream_object(stream), ([ws] if own_ws else []) + _owned(bs))


def precondition_grouped(grads, mbars, vbars, outs, step: int, QLs, QRs, beta1: float = BETA1, beta2: float = BETA2,
                         eps: float = EPS, ws: torch.Tensor | None = None, stream=None) -> None:
    """precondition() for up to 8 groups in one call: every rotation stage
    launches the products of all groups together."""
    bg, bm, bv, bo = ([batch(x) for x in xs] for xs in (grads, mbars, vbars, outs))
    bl, br = ([None if x is None else batch(x) for x in xs] for xs in (QLs, QRs))
    own_ws = ws is None
    if ws is None:
        need = L.soap_precondition_grouped_workspace([b.count for b in bg], [b.rows for b in bg],
                                                     [b.cols for b in bg])
        ws = workspace(need, bg[0].keep[-1].device)
    L.soap_precondition_grouped([b.desc for b in bg], [_desc(b) for b in bl], [_desc(b) for b in br],
                                [b.desc for b in bm], [b.desc for b in bv], [b.desc for b in bo], step, beta1, beta2,
                                eps, ws.data_ptr(), ws.numel(), _stream(stream))
    _record_on(_stream_object(stream), ([ws] if own_ws else []) + _owned(bg + bm + bv + bo + bl + br))


class SoapStep:
    """SOAP state and buffers for groups of same-shape weights.

    ``groups`` is a list of (W, G) pairs: 2-D tensors or 3-D strided batches
    (count x m x n), bf16 or fp32, on one device.  Each group keeps fp32
    statistics (L, R), bases (QL, QR), rotated moments (mbar, vbar) and the
    direction D; an axis longer than ``max_dim`` keeps the identity basis.
    ``step()`` runs, per group and in this order: the statistics, the basis
    refresh on steps 1, 1 + freq, ..., the rotated Adam direction, and
    W <- (1 - lr*wd) W - lr D.  The statistics, the refreshes and the
    rotated Adam directions of up to 8 groups share each call.
    """

    def __init__(self, groups, *, lr: float = 3e-4, weight_decay: float = 0.0, betas=(BETA1, BETA2),
                 eps: float = EPS, beta_s: float = BETA_S, freq: int = FREQ, max_dim: int = MAX_DIM):
        if freq < 1:
            raise ValueError("freq must be >= 1")
        self.lr, self.weight_decay, self.eps, self.beta_s, self.freq = lr, weight_decay, eps, beta_s, freq
        self.beta1, self.beta2 = betas
        self.t = 0
        self.groups = []
        need = 0
        dev = None
        for W, G in groups:
            W3 = W if W.dim() == 3 else W.unsqueeze(0)
            G3 = G if G.dim() == 3 else G.unsqueeze(0)
            if W3.shape != G3.shape:
                raise ValueError("weight and gradient shapes differ")
            c, m, n = W3.shape
            dev = W3.device
            f = dict(device=dev, dtype=torch.float32)
            eye = lambda k: torch.eye(k, **f).expand(c, k, k).contiguous()
            st = {"W": W3, "G": G3,
                  "L": torch.zeros(c, m, m, **f) if m <= max_dim else None,
                  "R": torch.zeros(c, n, n, **f) if n <= max_dim else None,
                  "QL": eye(m) if m <= max_dim else None,
                  "QR": eye(n) if n <= max_dim else None,
                  "mbar": torch.zeros(c, m, n, **f), "vbar": torch.zeros(c, m, n, **f),
                  "D": torch.empty(c, m, n, **f)}
            self.groups.append(st)
        self.chunks = [[i for i in range(k, min(k + 8, len(self.groups))) if self._preconditioned(i)]
                       for k in range(0, len(self.groups), 8)]
        self.chunks = [ch for ch in self.chunks if ch]
        # the rotated Adam direction of every group, 8 groups to a call
        self.all_chunks = [list(range(k, min(k + 8, len(self.groups)))) for k in range(0, len(self.groups), 8)]
        for ch in self.all_chunks:
            ds = [self.groups[i]["D"].shape for i in ch]
            need = max(need, L.soap_precondition_grouped_workspace([d[0] for d in ds], [d[1] for d in ds],
                                                                   [d[2] for d in ds]))
        for ch in self.chunks:
            gs = [self.groups[i] for i in ch]
            need = max(need, L.soap_refresh_grouped_workspace(
                [g["D"].shape[0] for g in gs], [g["D"].shape[1] for g in gs], [g["D"].shape[2] for g in gs],
                [g["L"] is not None for g in gs], [g["R"] is not None for g in gs]))
        self.ws = workspace(need, dev)

    def _preconditioned(self, i) -> bool:
        return self.groups[i]["L"] is not None or self.groups[i]["R"] is not None

    STATE = ("L", "R", "QL", "QR", "mbar", "vbar")

    def state_dict(self) -> dict:
        return {"t": self.t, "groups": [{k: (None if g[k] is None else g[k].clone()) for k in self.STATE}
                                        for g in self.groups]}

    def load_state_dict(self, state: dict) -> None:
        if len(state["groups"]) != len(self.groups):
            raise ValueError("state has a different number of groups")
        for g, s in zip(self.groups, state["groups"]):
            for k in self.STATE:
                if (g[k] is None) != (s[k] is None):
                    raise ValueError(f"state {k}: preconditioned sides differ")
                if g[k] is not None:
                    g[k].copy_(s[k])
        self.t = int(state["t"])

    def step(self, stream=None, events=None) -> None:
        """One SOAP update of every group.  ``events``: five torch.cuda
        Events recorded on the stream before the statistics, after them,
        after the refreshes, after the rotated Adam directions and after the
        weight updates (the phases run group after group)."""
        self.t += 1
        st = stream if stream is not None else torch.cuda.current_stream()
        s = _stream(st)

        def rec(i):
            if events is not None:
                events[i].record(st)

        rec(0)
        for ch in self.chunks:
            gs = [self.groups[i] for i in ch]
            statistics_grouped([g["G"] for g in gs], [g["L"] for g in gs], [g["R"] for g in gs], self.beta_s, stream=s)
        rec(1)
        if (self.t - 1) % self.freq == 0:
            for ch in self.chunks:
                gs = [self.groups[i] for i in ch]
                refresh_grouped([g["mbar"] for g in gs], [g["L"] for g in gs], [g["R"] for g in gs],
                                [g["QL"] for g in gs], [g["QR"] for g in gs], ws=self.ws, stream=s)
        rec(2)
        for ch in self.all_chunks:
            gs = [self.groups[i] for i in ch]
            precondition_grouped([g["G"] for g in gs], [g["mbar"] for g in gs], [g["vbar"] for g in gs],
                                 [g["D"] for g in gs], self.t, [g["QL"] for g in gs], [g["QR"] for g in gs],
                                 self.beta1, self.beta2, self.eps, ws=self.ws, stream=s)
        rec(3)
        for g in self.groups:
            bw, bd = batch(g["W"]), batch(g["D"])
            L.muon_apply(bw.desc, bd.desc, self.lr, self.weight_decay, L.MUON_SCALE_NONE, 1.0, s)
        rec(4)
