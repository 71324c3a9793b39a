"""Host <-> device transfer of raw storage arrays for the GPU tests (no arithmetic)."""
import sys

import numpy as np


def say(*args):
    """Print and flush, so a GPU step names its case before it runs."""
    print(*args, flush=True)
    sys.stdout.flush()


def dev(arr, dtype=None):
    """numpy storage array -> CUDA tensor with the same bytes (optionally re-viewed)."""
    import torch

    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).cuda()
    elif a.dtype == np.uint32:
        t = torch.from_numpy(a.view(np.int32)).cuda()
    else:
        t = torch.from_numpy(a).cuda()
    return t.view(dtype) if dtype is not None else t


def host_u16(t):
    import torch

    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_u32(t):
    import torch

    return t.detach().contiguous().view(torch.int32).cpu().numpy().view(np.uint32)


def upload_int4(d):
    import torch

    return {
        "x": dev(d["x"], torch.bfloat16),
        "qweight": dev(d["qweight"]),
        "scales": dev(d["scales"], torch.float16),
        "qzeros": dev(d["qzeros"]),
    }


def sample_indices(total, count, seed):
    """Sorted sample of indices that always includes both ends."""
    rng = np.random.default_rng(seed)
    if total <= count:
        return np.arange(total)
    pick = rng.choice(total, size=count, replace=False)
    return np.unique(np.concatenate([pick, [0, 1, total - 2, total - 1]]))
