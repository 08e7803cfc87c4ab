"""Host <-> device helpers for the GPU tests (uint16 bf16 bit patterns <-> torch)."""
import numpy as np
import torch

DEV = "cuda:0"


def bf16(bits) -> torch.Tensor:
    a = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)


def f32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32))).to(DEV)


def i32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.int32))).to(DEV)


def bits(t: torch.Tensor) -> np.ndarray:
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    if a.shape != b.shape or a.dtype != b.dtype:
        return False
    ia = a.contiguous().view(torch.uint8)
    ib = b.contiguous().view(torch.uint8)
    return bool(torch.equal(ia, ib))


def say(*a):
    print(*a, flush=True)
