"""Helpers of the GPU parity tests: device placement and a progress print."""
import sys

import numpy as np


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def say(*args):
    print("[gpu-case]", *args, flush=True)
    sys.stdout.flush()
