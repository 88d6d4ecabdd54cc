"""Helpers for the GPU parity tests (marked ``gpu``)."""
import sys

import numpy as np
import pytest

CANARY = 0xA5
PAD = 256                       # guard bytes on each side of an output


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def dev_bf16(bits):
    """numpy uint16 bf16 bits -> contiguous torch bf16 tensor on cuda:0."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to("cuda:0").view(torch.bfloat16)


def host_bits(t):
    """torch bf16 / fp16 device tensor -> numpy uint16 bit patterns."""
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host_u8(t):
    return t.cpu().numpy()


class Guarded:
    """An output tensor with canary bytes before and after it."""

    def __init__(self, shape, dtype):
        import torch
        elem = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) * elem
        self.buf = torch.full((n + 2 * PAD,), CANARY, dtype=torch.uint8, device="cuda:0")
        self.n = n
        self.t = self.buf[PAD:PAD + n].view(dtype).view(shape) if n else torch.empty(shape, dtype=dtype, device="cuda:0")

    def intact(self):
        b = self.buf.cpu().numpy()
        return bool(np.all(b[:PAD] == CANARY) and np.all(b[PAD + self.n:] == CANARY))
