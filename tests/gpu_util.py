"""Helpers for the GPU parity tests: upload seeded host arrays, run the
library through its binding, and compare with the fp64 oracle using the
normalised error |y_gpu - y_ref| / sum|w x| per output."""
import numpy as np
import torch

from oracle import ref

TOL = 2e-4  # max normalised error for every fp path (fp32 accumulation)


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:  # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def host(t):
    return t.detach().cpu().numpy()


def norm_err(y_gpu, y_ref, nrm):
    return ref.max_norm_err(np.asarray(y_gpu, np.float64), y_ref, nrm)


def upload_experts(ex, only=None):
    """Device copies of an expert set; with `only`, the device stack is zero
    except for those expert ids (saves PCIe time on big stacks)."""
    out = {}
    for key in ("gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s"):
        a = ex[key]
        if only is None:
            out[key] = dev(a)
        else:
            t = torch.zeros(a.shape, dtype=dev(a[:1]).dtype, device="cuda")
            for e in sorted(set(int(i) for i in np.asarray(only).ravel() if 0 <= i < a.shape[0])):
                t[e].copy_(dev(a[e]))
            out[key] = t
    return out
