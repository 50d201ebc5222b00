"""Helpers of the GPU parity tests: host <-> device copies and guard canaries."""

import numpy as np
import torch

DEV = "cuda:0"


def bf16_dev(a):
    """numpy uint16 (bf16 bits) -> device bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


def u8_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host(t):
    """Device tensor -> numpy (bf16 comes back as uint16 bits)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class Guarded:
    """An output tensor embedded between two 4 KiB guard zones filled with 0xA5."""

    GUARD = 4096

    def __init__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        g = self.GUARD
        self.raw = torch.full((g + n + g,), 0xA5, dtype=torch.uint8, device=DEV)
        self.t = self.raw[g:g + n].view(dtype).view(shape)
        self.n = n

    def intact(self):
        r = self.raw.cpu().numpy()
        return bool(np.all(r[:self.GUARD] == 0xA5) and np.all(r[self.GUARD + self.n:] == 0xA5))
