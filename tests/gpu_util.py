"""Helpers shared by the GPU tests: device transfers and step announcements."""
import sys

import numpy as np
import torch

DEV = torch.device("cuda", 0)


def say(*args):
    """Name the case before each GPU step (flushed, so a failing box still shows it)."""
    print("[gpu-case]", *args, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32)).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy().astype(np.uint32)
