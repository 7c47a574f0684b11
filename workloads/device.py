"""Copy a generated Workload to device tensors (torch), keeping the exact bits."""
from __future__ import annotations

import numpy as np


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def to_tensor(a: np.ndarray, dtype: str, device):
    """numpy storage array -> torch tensor of the storage dtype on `device` (bit-exact)."""
    import torch
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device)


def to_numpy_bits(t, dtype: str) -> np.ndarray:
    """torch tensor -> numpy storage array (bit-exact), on the host."""
    import torch
    t = t.detach().to("cpu").contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def upload(w, device="cuda"):
    """All buffers of a Workload as device tensors, in a dict."""
    import torch
    d = w.cfg.dtype
    if w.cfg.fp8 or getattr(w.cfg, "mxfp4", False):
        pools = {"k_pool": torch.from_numpy(np.ascontiguousarray(w.k_pool)).to(device),
                 "v_pool": torch.from_numpy(np.ascontiguousarray(w.v_pool)).to(device),
                 "k_scale": torch.from_numpy(np.ascontiguousarray(w.k_scale)).to(device),
                 "v_scale": torch.from_numpy(np.ascontiguousarray(w.v_scale)).to(device)}
    else:
        pools = {"k_pool": to_tensor(w.k_pool, d, device), "v_pool": to_tensor(w.v_pool, d, device)}
    out = {
        "q": to_tensor(w.q, d, device),
        **pools,
        "block_tables": torch.from_numpy(np.ascontiguousarray(w.block_tables)).to(device),
        "context_lens": torch.from_numpy(np.ascontiguousarray(w.context_lens)).to(device),
    }
    if w.positions is not None:
        out["positions"] = torch.from_numpy(np.ascontiguousarray(w.positions)).to(device)
        out["k_new"] = to_tensor(w.k_new, d, device)
        out["v_new"] = to_tensor(w.v_new, d, device)
    return out
