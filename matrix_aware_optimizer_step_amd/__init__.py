"""libmuon355: the Muon optimizer step on AMD Instinct MI355X (gfx950).

Momentum, Newton-Schulz orthogonalization and the shape-scaled update run in
hand-written HIP kernels behind the C ABI of include/muon355.h, and so does
the AdamW step for the parameters Muon does not take.  ``_lib`` is
the ctypes binding (same names as the C entry points); ``muon`` turns torch
tensors into descriptors and holds the buffers of a whole step.
"""

from . import _lib
from ._lib import (MUON_BF16, MUON_F32, MUON_SCALE_MATCH_RMS, MUON_SCALE_NONE, MUON_SCALE_ORIGINAL, MuonBatch,
                   MuonError)
from .muon import (EPS, QUINTIC, AdamW, Batch, MuonStep, OptimizerStep, apply, apply_grouped, batch, is_muon_param,
                   momentum, momentum_grouped, orthogonalize, orthogonalize_grouped, workspace)

__all__ = ["_lib", "MUON_BF16", "MUON_F32", "MUON_SCALE_MATCH_RMS", "MUON_SCALE_NONE", "MUON_SCALE_ORIGINAL",
           "MuonBatch", "MuonError", "EPS", "QUINTIC", "Batch", "MuonStep", "apply", "apply_grouped", "batch",
           "momentum", "momentum_grouped", "orthogonalize", "orthogonalize_grouped", "workspace", "AdamW",
           "OptimizerStep", "is_muon_param"]
