"""Upload a ``Workload``'s host arrays to the GPU as torch tensors (memory only, no compute)."""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

__all__ = ["DeviceWorkload", "upload", "torch_dtype", "to_numpy_f64"]


def torch_dtype(dt: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.uint8}[dt]


def _tensor(arr: np.ndarray, dt: str, device):
    import torch
    a = np.ascontiguousarray(arr)
    if dt == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device)


def to_numpy_f64(t) -> np.ndarray:
    """A GPU tensor of f32 / f16 / bf16 values -> float64 numpy (exact)."""
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()


@dataclass
class DeviceWorkload:
    q: object
    k_cache: object
    v_cache: object
    k_scale: Optional[object]
    v_scale: Optional[object]
    tables: object
    lens: object
    k_new: object
    v_new: object
    slots: object
    cow: object


def upload(w, device="cuda") -> DeviceWorkload:
    import torch
    return DeviceWorkload(
        q=_tensor(w.q, w.q_dtype, device),
        k_cache=_tensor(w.k_pool, w.dtype, device),
        v_cache=_tensor(w.v_pool, w.dtype, device),
        k_scale=None if w.k_scale is None else torch.from_numpy(w.k_scale.copy()).to(device),
        v_scale=None if w.v_scale is None else torch.from_numpy(w.v_scale.copy()).to(device),
        tables=torch.from_numpy(np.ascontiguousarray(w.tables, dtype=np.int32)).to(device),
        lens=torch.from_numpy(np.ascontiguousarray(w.lens, dtype=np.int32)).to(device),
        k_new=_tensor(w.k_new, w.new_dtype, device),
        v_new=_tensor(w.v_new, w.new_dtype, device),
        slots=torch.from_numpy(np.ascontiguousarray(w.slots, dtype=np.int32)).to(device),
        cow=torch.from_numpy(np.ascontiguousarray(w.cow, dtype=np.int32).reshape(-1, 2)).to(device),
    )
