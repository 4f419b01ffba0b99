"""Host <-> device helpers for the GPU parity tests (marshalling only)."""
import numpy as np
import torch

DEV = "cuda:0"


def dev(a: np.ndarray, misalign: bool = False) -> torch.Tensor:
    """Copy a numpy array to the device. uint32 travels as int32 bit patterns.
    misalign=True returns a view that starts 4 bytes into its allocation (so
    it is 4-byte but not 16-byte aligned)."""
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    t = torch.from_numpy(np.ascontiguousarray(a))
    if not misalign:
        return t.to(DEV)
    pad = 4 // t.element_size()
    buf = torch.empty(t.numel() + pad, dtype=t.dtype, device=DEV)
    view = buf[pad:]
    view.copy_(t.to(DEV))
    assert view.numel() == 0 or view.data_ptr() % 16 != 0
    return view


def empty(n: int, dtype, misalign: bool = False, fill=None) -> torch.Tensor:
    pad = (4 // torch.empty(0, dtype=dtype).element_size()) if misalign else 0
    buf = torch.empty(n + pad, dtype=dtype, device=DEV)
    if fill is not None:
        buf.fill_(fill)
    return buf[pad:]


def host(t: torch.Tensor, dtype=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def sync():
    torch.cuda.synchronize()
