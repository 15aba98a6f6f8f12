"""ctypes binding of libmuon355 (include/muon355.h).

Argument marshalling only: every step of the Muon path runs in the library's
HIP kernels.  Each function has the name of the C entry point it wraps,
takes ``MuonBatch`` descriptors and raw device addresses, and raises
``MuonError`` on a non-OK status.  Loading fails loudly when the library has
not been built; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmuon355.so")

MUON_F32 = 0
MUON_BF16 = 1
MUON_SCALE_MATCH_RMS = 0
MUON_SCALE_ORIGINAL = 1
MUON_SCALE_NONE = 2

STATUS = {0: "MUON_OK", 1: "MUON_ERR_INVALID_VALUE", 2: "MUON_ERR_UNSUPPORTED",
          3: "MUON_ERR_WORKSPACE", 4: "MUON_ERR_LAUNCH"}

EXPORTED = ("muon_abi_version", "muon_last_error", "muon_status_string", "muon_momentum_workspace",
            "muon_momentum", "muon_momentum_grouped_workspace", "muon_momentum_grouped", "muon_momentum_grouped_noalloc",
            "muon_orthogonalize_workspace", "muon_orthogonalize", "muon_orthogonalize_grouped_workspace",
            "muon_orthogonalize_grouped", "muon_packed_grouped_workspace", "muon_momentum_packed_grouped",
            "muon_orthogonalize_packed_grouped", "muon_orthogonalize_apply_packed_grouped", "muon_apply", "muon_apply_grouped", "muon_adamw", "soap_statistics",
            "soap_statistics_grouped", "soap_qr_workspace", "soap_qr", "soap_refresh_workspace", "soap_refresh",
            "soap_refresh_grouped_workspace", "soap_refresh_grouped",
            "soap_precondition_workspace", "soap_precondition", "soap_precondition_grouped_workspace",
            "soap_precondition_grouped")

ADAMW_CHUNK = 4096  # MUON_ADAMW_CHUNK


class MuonError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}: {detail}")


class MuonBatch(ctypes.Structure):
    _fields_ = [("ptrs", ctypes.c_void_p), ("base", ctypes.c_void_p), ("stride", ctypes.c_int64),
                ("count", ctypes.c_int64), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ld", ctypes.c_int64), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class MuonTensorList(ctypes.Structure):
    _fields_ = [("count", ctypes.c_int64), ("total_chunks", ctypes.c_int64), ("params", ctypes.c_void_p),
                ("grads", ctypes.c_void_p), ("exp_avg", ctypes.c_void_p), ("exp_avg_sq", ctypes.c_void_p),
                ("numels", ctypes.c_void_p), ("chunk_offsets", ctypes.c_void_p), ("param_dtype", ctypes.c_int32),
                ("grad_dtype", ctypes.c_int32)]


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(the Muon path has no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(MuonBatch)
    vp, f32, i32, i64, sz = ctypes.c_void_p, ctypes.c_float, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "muon_abi_version": (ctypes.c_int, []),
        "muon_last_error": (ctypes.c_char_p, []),
        "muon_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "muon_momentum_workspace": (sz, [i64, i64, i64]),
        "muon_momentum": (ctypes.c_int, [P, P, P, vp, f32, ctypes.c_int, vp, sz, vp]),
        "muon_momentum_grouped_workspace": (sz, [ctypes.c_int, ctypes.POINTER(i64), ctypes.POINTER(i64),
                                                 ctypes.POINTER(i64)]),
        "muon_momentum_grouped": (ctypes.c_int, [ctypes.c_int, P, P, P, ctypes.POINTER(vp), f32, ctypes.c_int, vp,
                                                 sz, vp]),
        "muon_momentum_grouped_noalloc": (ctypes.c_int, [ctypes.c_int, P, P, P, ctypes.POINTER(vp), f32, ctypes.c_int,
                                                         vp]),
        "muon_orthogonalize_workspace": (sz, [i64, i64, i64, i32]),
        "muon_orthogonalize": (ctypes.c_int, [P, vp, P, ctypes.c_int, f32, f32, f32, f32, i32, vp, sz, vp]),
        "muon_orthogonalize_grouped_workspace": (sz, [ctypes.c_int, ctypes.POINTER(i64), ctypes.POINTER(i64),
                                                      ctypes.POINTER(i64), i32]),
        "muon_orthogonalize_grouped": (ctypes.c_int, [ctypes.c_int, P, ctypes.POINTER(vp), P, ctypes.c_int,
                                                      f32, f32, f32, f32, i32, vp, sz, vp]),
        "muon_packed_grouped_workspace": (sz, [ctypes.c_int, ctypes.POINTER(i64), ctypes.POINTER(i64),
                                               ctypes.POINTER(i64), i32]),
        "muon_momentum_packed_grouped": (ctypes.c_int, [ctypes.c_int, P, P, ctypes.POINTER(vp), f32, ctypes.c_int,
                                                        i32, vp, sz, vp]),
        "muon_orthogonalize_packed_grouped": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(vp), P, ctypes.c_int, f32,
                                                             f32, f32, f32, i32, vp, sz, vp]),
        "muon_orthogonalize_apply_packed_grouped": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(vp), P, ctypes.c_int,
                                                                   f32, f32, f32, f32, f32, f32, i32, f32, i32, vp,
                                                                   sz, vp]),
        "muon_apply": (ctypes.c_int, [P, P, f32, f32, i32, f32, vp]),
        "muon_apply_grouped": (ctypes.c_int, [ctypes.c_int, P, P, f32, f32, i32, f32, vp]),
        "muon_adamw": (ctypes.c_int, [ctypes.POINTER(MuonTensorList), i64, f32, f32, f32, f32, f32, vp]),
        "soap_statistics": (ctypes.c_int, [P, P, P, f32, vp]),
        "soap_statistics_grouped": (ctypes.c_int, [ctypes.c_int, P, ctypes.POINTER(P), ctypes.POINTER(P), f32, vp]),
        "soap_qr_workspace": (sz, [i64, i64]),
        "soap_qr": (ctypes.c_int, [P, P, vp, sz, vp]),
        "soap_refresh_workspace": (sz, [i64, i64, i64, ctypes.c_int, ctypes.c_int]),
        "soap_refresh": (ctypes.c_int, [P, P, P, P, P, vp, sz, vp]),
        "soap_refresh_grouped_workspace": (sz, [ctypes.c_int, ctypes.POINTER(i64), ctypes.POINTER(i64),
                                                ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_int),
                                                ctypes.POINTER(ctypes.c_int)]),
        "soap_refresh_grouped": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(P), ctypes.POINTER(P),
                                                ctypes.POINTER(P), ctypes.POINTER(P), P, vp, sz, vp]),
        "soap_precondition_workspace": (sz, [i64, i64, i64]),
        "soap_precondition": (ctypes.c_int, [P, P, P, P, P, P, i64, f32, f32, f32, vp, sz, vp]),
        "soap_precondition_grouped_workspace": (sz, [ctypes.c_int, ctypes.POINTER(i64), ctypes.POINTER(i64),
                                                     ctypes.POINTER(i64)]),
        "soap_precondition_grouped": (ctypes.c_int, [ctypes.c_int, P, ctypes.POINTER(P), ctypes.POINTER(P), P, P, P,
                                                     i64, f32, f32, f32, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, where: str) -> None:
    if status != 0:
        detail = load().muon_last_error().decode(errors="replace")
        raise MuonError(status, where, detail)


def _ref(b):
    return None if b is None else ctypes.byref(b)


def muon_abi_version() -> int:
    return load().muon_abi_version()


def muon_momentum_workspace(count: int, rows: int, cols: int) -> int:
    return load().muon_momentum_workspace(count, rows, cols)


def muon_momentum(grad: MuonBatch, mom: MuonBatch, nout: MuonBatch | None, sumsq_ptr: int, beta: float,
                  nesterov: bool, workspace_ptr: int, ws_bytes: int, stream: int) -> None:
    st = load().muon_momentum(_ref(grad), _ref(mom), _ref(nout), sumsq_ptr, beta, int(bool(nesterov)),
                              workspace_ptr, ws_bytes, stream)
    _check(st, "muon_momentum")


def muon_momentum_grouped_workspace(counts, rows, cols) -> int:
    n = len(counts)
    arr = ctypes.c_int64 * n
    return load().muon_momentum_grouped_workspace(n, arr(*counts), arr(*rows), arr(*cols))


def muon_momentum_grouped(grads, moms, nouts, sumsq_ptrs, beta: float, nesterov: bool, workspace_ptr: int,
                          ws_bytes: int, stream: int) -> None:
    n = len(grads)
    if len(moms) != n or len(sumsq_ptrs) != n or (nouts is not None and len(nouts) != n):
        raise ValueError("per-group lists differ in length")
    no = None if nouts is None else (MuonBatch * n)(*nouts)
    st = load().muon_momentum_grouped(n, (MuonBatch * n)(*grads), (MuonBatch * n)(*moms), no,
                                      (ctypes.c_void_p * n)(*sumsq_ptrs), beta, int(bool(nesterov)),
                                      workspace_ptr, ws_bytes, stream)
    _check(st, "muon_momentum_grouped")


NOALLOC_SCRATCH_BYTES = 8 << 20  # MUON_NOALLOC_SCRATCH_BYTES


def muon_momentum_grouped_noalloc(grads, moms, nouts, sumsq_ptrs, beta: float, nesterov: bool,
                                  stream: int) -> None:
    n = len(grads)
    if len(moms) != n or len(sumsq_ptrs) != n or (nouts is not None and len(nouts) != n):
        raise ValueError("per-group lists differ in length")
    no = None if nouts is None else (MuonBatch * n)(*nouts)
    st = load().muon_momentum_grouped_noalloc(n, (MuonBatch * n)(*grads), (MuonBatch * n)(*moms), no,
                                              (ctypes.c_void_p * n)(*sumsq_ptrs), beta, int(bool(nesterov)),
                                              stream)
    _check(st, "muon_momentum_grouped_noalloc")


def muon_orthogonalize_workspace(count: int, rows: int, cols: int, compute: int) -> int:
    return load().muon_orthogonalize_workspace(count, rows, cols, compute)


def muon_orthogonalize(inp: MuonBatch, sumsq_ptr: int | None, out: MuonBatch, steps: int, a: float, b: float,
                       c: float, eps: float, compute: int, workspace_ptr: int, ws_bytes: int,
                       stream: int) -> None:
    st = load().muon_orthogonalize(_ref(inp), sumsq_ptr, _ref(out), steps, a, b, c, eps, compute,
                                   workspace_ptr, ws_bytes, stream)
    _check(st, "muon_orthogonalize")


def muon_orthogonalize_grouped_workspace(counts, rows, cols, compute: int) -> int:
    n = len(counts)
    arr = ctypes.c_int64 * n
    return load().muon_orthogonalize_grouped_workspace(n, arr(*counts), arr(*rows), arr(*cols), compute)


def muon_orthogonalize_grouped(ins, sumsq_ptrs, outs, steps: int, a: float, b: float, c: float, eps: float,
                               compute: int, workspace_ptr: int, ws_bytes: int, stream: int) -> None:
    n = len(ins)
    if len(outs) != n:
        raise ValueError("ins and outs differ in length")
    ins_arr = (MuonBatch * n)(*ins)
    outs_arr = (MuonBatch * n)(*outs)
    ss = None
    if sumsq_ptrs is not None:
        ss = (ctypes.c_void_p * n)(*[p if p else None for p in sumsq_ptrs])
    st = load().muon_orthogonalize_grouped(n, ins_arr, ss, outs_arr, steps, a, b, c, eps, compute,
                                           workspace_ptr, ws_bytes, stream)
    _check(st, "muon_orthogonalize_grouped")


def muon_packed_grouped_workspace(counts, rows, cols, compute: int) -> int:
    n = len(counts)
    arr = ctypes.c_int64 * n
    return load().muon_packed_grouped_workspace(n, arr(*counts), arr(*rows), arr(*cols), compute)


def muon_momentum_packed_grouped(grads, moms, sumsq_ptrs, beta: float, nesterov: bool, compute: int,
                                 workspace_ptr: int, ws_bytes: int, stream: int) -> None:
    n = len(grads)
    if len(moms) != n or len(sumsq_ptrs) != n:
        raise ValueError("per-group lists differ in length")
    st = load().muon_momentum_packed_grouped(n, (MuonBatch * n)(*grads), (MuonBatch * n)(*moms),
                                             (ctypes.c_void_p * n)(*sumsq_ptrs), beta, int(bool(nesterov)), compute,
                                             workspace_ptr, ws_bytes, stream)
    _check(st, "muon_momentum_packed_grouped")


def muon_orthogonalize_packed_grouped(sumsq_ptrs, outs, steps: int, a: float, b: float, c: float, eps: float,
                                      compute: int, workspace_ptr: int, ws_bytes: int, stream: int) -> None:
    n = len(outs)
    if len(sumsq_ptrs) != n:
        raise ValueError("per-group lists differ in length")
    st = load().muon_orthogonalize_packed_grouped(n, (ctypes.c_void_p * n)(*sumsq_ptrs), (MuonBatch * n)(*outs),
                                                  steps, a, b, c, eps, compute, workspace_ptr, ws_bytes, stream)
    _check(st, "muon_orthogonalize_packed_grouped")


def muon_orthogonalize_apply_packed_grouped(sumsq_ptrs, weights, steps: int, a: float, b: float, c: float,
                                            eps: float, lr: float, weight_decay: float, mode: int, coeff: float,
                                            compute: int, workspace_ptr: int, ws_bytes: int, stream: int) -> None:
    n = len(weights)
    if len(sumsq_ptrs) != n:
        raise ValueError("per-group lists differ in length")
    st = load().muon_orthogonalize_apply_packed_grouped(n, (ctypes.c_void_p * n)(*sumsq_ptrs),
                                                        (MuonBatch * n)(*weights), steps, a, b, c, eps, lr,
                                                        weight_decay, mode, coeff, compute, workspace_ptr, ws_bytes,
                                                        stream)
    _check(st, "muon_orthogonalize_apply_packed_grouped")


def muon_apply(weight: MuonBatch, ortho: MuonBatch, lr: float, weight_decay: float, mode: int, coeff: float,
               stream: int) -> None:
    st = load().muon_apply(_ref(weight), _ref(ortho), lr, weight_decay, mode, coeff, stream)
    _check(st, "muon_apply")


def muon_apply_grouped(weights, orthos, lr: float, weight_decay: float, mode: int, coeff: float,
                       stream: int) -> None:
    n = len(weights)
    if len(orthos) != n:
        raise ValueError("weights and orthos differ in length")
    st = load().muon_apply_grouped(n, (MuonBatch * n)(*weights), (MuonBatch * n)(*orthos), lr, weight_decay,
                                   mode, coeff, stream)
    _check(st, "muon_apply_grouped")


def muon_adamw(tensors: MuonTensorList, step: int, lr: float, beta1: float, beta2: float, eps: float,
               weight_decay: float, stream: int) -> None:
    st = load().muon_adamw(ctypes.byref(tensors), step, lr, beta1, beta2, eps, weight_decay, stream)
    _check(st, "muon_adamw")


def soap_statistics(grad: MuonBatch, L: MuonBatch | None, R: MuonBatch | None, beta_s: float, stream: int) -> None:
    _check(load().soap_statistics(_ref(grad), _ref(L), _ref(R), beta_s, stream), "soap_statistics")


def soap_qr_workspace(count: int, n: int) -> int:
    return load().soap_qr_workspace(count, n)


def soap_qr(a: MuonBatch, q: MuonBatch, workspace_ptr: int, ws_bytes: int, stream: int) -> None:
    _check(load().soap_qr(_ref(a), _ref(q), workspace_ptr, ws_bytes, stream), "soap_qr")


def soap_refresh_workspace(count: int, rows: int, cols: int, with_l: bool, with_r: bool) -> int:
    return load().soap_refresh_workspace(count, rows, cols, int(bool(with_l)), int(bool(with_r)))


def soap_refresh(L: MuonBatch | None, R: MuonBatch | None, QL: MuonBatch | None, QR: MuonBatch | None,
                 mbar: MuonBatch, workspace_ptr: int, ws_bytes: int, stream: int) -> None:
    st = load().soap_refresh(_ref(L), _ref(R), _ref(QL), _ref(QR), _ref(mbar), workspace_ptr, ws_bytes, stream)
    _check(st, "soap_refresh")


def soap_statistics_grouped(grads, Ls, Rs, beta_s: float, stream: int) -> None:
    """grads: per-group MuonBatch; Ls, Rs: per-group MuonBatch or None."""
    n = len(grads)
    if not (len(Ls) == len(Rs) == n):
        raise ValueError("per-group lists differ in length")
    PB = ctypes.POINTER(MuonBatch)
    arr = lambda xs: (PB * n)(*[PB() if x is None else ctypes.pointer(x) for x in xs])
    st = load().soap_statistics_grouped(n, (MuonBatch * n)(*grads), arr(Ls), arr(Rs), beta_s, stream)
    _check(st, "soap_statistics_grouped")


def soap_refresh_grouped_workspace(counts, rows, cols, with_l, with_r) -> int:
    n = len(counts)
    i64, ci = ctypes.c_int64 * n, ctypes.c_int * n
    return load().soap_refresh_grouped_workspace(n, i64(*counts), i64(*rows), i64(*cols),
                                                 ci(*[int(bool(x)) for x in with_l]),
                                                 ci(*[int(bool(x)) for x in with_r]))


def soap_refresh_grouped(Ls, Rs, QLs, QRs, mbars, workspace_ptr: int, ws_bytes: int, stream: int) -> None:
    """Ls, Rs, QLs, QRs: per-group MuonBatch or None; mbars: per-group MuonBatch."""
    n = len(mbars)
    if not (len(Ls) == len(Rs) == len(QLs) == len(QRs) == n):
        raise ValueError("per-group lists differ in length")
    PB = ctypes.POINTER(MuonBatch)
    arr = lambda xs: (PB * n)(*[PB() if x is None else ctypes.pointer(x) for x in xs])
    st = load().soap_refresh_grouped(n, arr(Ls), arr(Rs), arr(QLs), arr(QRs), (MuonBatch * n)(*mbars), workspace_ptr,
                                     ws_bytes, stream)
    _check(st, "soap_refresh_grouped")


def soap_precondition_workspace(count: int, rows: int, cols: int) -> int:
    return load().soap_precondition_workspace(count, rows, cols)


def soap_precondition(grad: MuonBatch, QL: MuonBatch | None, QR: MuonBatch | None, mbar: MuonBatch,
                      vbar: MuonBatch, direction: MuonBatch, step: int, beta1: float, beta2: float, eps: float,
                      workspace_ptr: int, ws_bytes: int, stream: int) -> None:
    st = load().soap_precondition(_ref(grad), _ref(QL), _ref(QR), _ref(mbar), _ref(vbar), _ref(direction), step,
                                  beta1, beta2, eps, workspace_ptr, ws_bytes, stream)
    _check(st, "soap_precondition")


def soap_precondition_grouped_workspace(counts, rows, cols) -> int:
    n = len(counts)
    i64 = ctypes.c_int64 * n
    return load().soap_precondition_grouped_workspace(n, i64(*counts), i64(*rows), i64(*cols))


def soap_precondition_grouped(grads, QLs, QRs, mbars, vbars, dirs, step: int, beta1: float, beta2: float,
                              eps: float, workspace_ptr: int, ws_bytes: int, stream: int) -> None:
    """grads, mbars, vbars, dirs: per-group MuonBatch; QLs, QRs: per-group MuonBatch or None."""
    n = len(grads)
    if not (len(QLs) == len(QRs) == len(mbars) == len(vbars) == len(dirs) == n):
        raise ValueError("per-group lists differ in length")
    PB = ctypes.POINTER(MuonBatch)
    arr = lambda xs: (PB * n)(*[PB() if x is None else ctypes.pointer(x) for x in xs])
    vec = lambda xs: (MuonBatch * n)(*xs)
    st = load().soap_precondition_grouped(n, vec(grads), arr(QLs), arr(QRs), vec(mbars), vec(vbars), vec(dirs), step,
                                          beta1, beta2, eps, workspace_ptr, ws_bytes, stream)
    _check(st, "soap_precondition_grouped")
