"""Helpers for GPU tests: move seeded numpy inputs to the device and back."""
import numpy as np
import torch


def dev_bf16(bits: np.ndarray, where: str = "hbm") -> torch.Tensor:
    """bf16 bit patterns -> torch.bfloat16 on the GPU ("hbm") or in pinned host memory ("host")."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.pin_memory() if where == "host" else t.cuda()


def dev_f32(x: np.ndarray, where: str = "hbm") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.pin_memory() if where == "host" else t.cuda()


def empty_bf16(shape, where: str = "hbm", fill_nan: bool = True) -> torch.Tensor:
    """Output buffer, poisoned with NaN so an unwritten element is caught."""
    if where == "host":
        t = torch.empty(shape, dtype=torch.bfloat16, pin_memory=True)
    else:
        t = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    if fill_nan:
        t.fill_(float("nan"))
    return t


def bits(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def np_i32(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()
