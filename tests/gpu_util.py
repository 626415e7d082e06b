"""Helpers for GPU tests: move seeded input sets to the device."""
import numpy as np
import torch


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def upload(ts):
    """TensorSet -> dict of device tensors with the library's layouts."""
    if ts.dtype == "bf16":
        q = dev(ts.q_bits.view(np.int16)).view(torch.bfloat16)
        k = dev(ts.k_bits.view(np.int16)).view(torch.bfloat16)
        v = dev(ts.v_bits.view(np.int16)).view(torch.bfloat16)
    else:
        q, k, v = dev(ts.q), dev(ts.k), dev(ts.v)
    return dict(q=q, k=k, v=v, alpha=dev(ts.alpha), beta=dev(ts.beta),
                parent=dev(ts.parent.astype(np.int32)), S0=dev(ts.S0))


def host(t):
    return t.detach().cpu().numpy()
