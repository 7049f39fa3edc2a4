"""Shared helpers of the GPU parity tests (no oracle arithmetic here)."""
import numpy as np
import torch

DEV = "cuda:0"


def bits16(t: torch.Tensor) -> np.ndarray:
    """uint16 patterns of a bf16 tensor (any device)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy().view(np.uint8)


def npy(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy()


def status_word(dev=DEV) -> torch.Tensor:
    return torch.zeros(1, dtype=torch.int32, device=dev)


def bf16_filled(rows: int, H: int, pattern: int, dev=DEV) -> torch.Tensor:
    """A bf16 tensor whose every element holds the given bit pattern (a canary)."""
    v = pattern - 0x10000 if pattern >= 0x8000 else pattern
    return torch.full((rows, H), v, dtype=torch.int16, device=dev).view(torch.bfloat16)


def announce(msg: str) -> None:
    print("[gpu-case] " + msg, flush=True)
