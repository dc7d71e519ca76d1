"""Helpers shared by the GPU tests (not a test module)."""
import numpy as np
import pytest

import long_context_decode_pkv_amd as pkv


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    pkv.lib()  # raises loudly if libpkv.so is missing


def to_dev(a, dtype):
    """Stored numpy array (uint16 bf16 bits or float32) -> device tensor."""
    import torch
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(a.astype(np.float32)).to("cuda:0")


def to_f64(t):
    """Device tensor -> float64 numpy."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    """max |got - ref| / max |ref| over the whole tensor (NaN refs ignored)."""
    m = ~np.isnan(ref)
    return float(np.abs(got[m] - ref[m]).max() / np.abs(ref[m]).max())


def make_cache(d, r_k=None, r_v=None, max_tokens=None, s=None, w=None, store=None):
    """Cache for decode_inputs d; store "int4" keeps INT4 factor pages (the
    inputs' dtype must then be bf16)."""
    cfg = d["cfg"]
    return pkv.Cache(batch=d["B"], n_q_heads=d["Hq"], n_kv_heads=d["Hkv"],
                     rank_k=cfg["r_k"] if r_k is None else r_k,
                     rank_v=cfg["r_v"] if r_v is None else r_v,
                     sink=cfg["s"] if s is None else s, window=cfg["w"] if w is None else w,
                     max_tokens=max_tokens or d["T"], dtype=store or cfg["dtype"])


# Tolerances (relative to max |o_ref| over the tensor): bf16 storage 1e-2,
# fp32 storage 1e-4; INT4 factor pages against the oracle's own INT4 factors,
# the bf16 gate (the two sides may round a code differently where the exact
# factor sits on a rounding boundary).
TOL = {"bf16": 1e-2, "f32": 1e-4, "int4": 1e-2}
