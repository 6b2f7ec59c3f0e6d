"""Helpers shared by the GPU parity tests (comparison and conversion only)."""
import numpy as np
import torch

import oracle as O

REL_L2 = 2e-3          # relative L2 error bound for Y, dX, dL1, dL2
MAX_ABS_FRAC = 1e-2    # max abs error bound, as a fraction of max |ref|


def bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16 tensor (any device)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def value(x) -> np.ndarray:
    x = np.asarray(x)
    return O.bf16_value(x) if x.dtype == np.uint16 else x.astype(np.float64)


def assert_close(got, ref, name, log=None):
    g, r = value(got), value(ref)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite output"
    err = g - r
    nref = np.linalg.norm(r)
    rel = np.linalg.norm(err) / nref if nref > 0 else np.linalg.norm(err)
    mx = np.max(np.abs(err)) if err.size else 0.0
    lim = MAX_ABS_FRAC * (np.max(np.abs(r)) if r.size else 0.0)
    msg = f"{name}: rel_l2={rel:.3e} max_abs={mx:.3e} (limit {lim:.3e})"
    print(msg, flush=True)
    if log is not None:
        log.append(msg)
    assert rel <= REL_L2, msg
    assert mx <= lim or mx == 0.0, msg


def assert_bitexact(got, ref, name):
    got, ref = np.asarray(got), np.asarray(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    bad = np.nonzero(got.reshape(-1) != ref.reshape(-1))[0]
    assert bad.size == 0, f"{name}: {bad.size} mismatches, first at {bad[:5]}: got {got.reshape(-1)[bad[:5]]} ref {ref.reshape(-1)[bad[:5]]}"
