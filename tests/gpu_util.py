"""Helpers for the GPU tests: device buffers from numpy, stream handle,
cosine metrics.  Device tensors are kept referenced for as long as a kernel
may use them."""
import numpy as np

DEV = "cuda:0"


def torch():
    import torch as t
    return t


def dev(a):
    t = torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return t.from_numpy(a).to(DEV)


def empty(shape, dtype):
    t = torch()
    return t.empty(shape, dtype=dtype, device=DEV)


def stream():
    return torch().cuda.current_stream().cuda_stream


def sync():
    torch().cuda.synchronize()


def host(x):
    sync()
    a = x.cpu().numpy()
    return a


def row_cosines(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.sum(a * b, axis=1) / (np.linalg.norm(a, axis=1) * np.linalg.norm(b, axis=1))


def say(msg):
    print(msg, flush=True)
