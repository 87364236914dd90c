"""Shared helpers of the parity tests (no verify arithmetic here)."""
import sys

import numpy as np
import torch

# tolerances: max |gpu - ref| / RMS(ref) over one call's output
TOL_BF16 = 2e-2
TOL_F32 = 1e-4


def tol_for(dtype):
    return TOL_BF16 if dtype == torch.bfloat16 else TOL_F32


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(got - ref).max() / np.sqrt((ref ** 2).mean()))


def np64(t):
    return t.detach().cpu().double().numpy()


def anc_u64(t):
    return t.detach().cpu().numpy().view(np.uint64)


def say(*a):
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print(*a, flush=True)
    sys.stdout.flush()
