"""Helpers for the GPU parity tests: host <-> device copies of numpy arrays."""

import numpy as np
import torch

DEV = "cuda:0"


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).to(DEV)
    return torch.from_numpy(a).to(DEV)


def host(t):
    return t.detach().cpu().numpy()


def host_u32(t):
    return host(t).view(np.uint32)


def bits16(a):
    return np.ascontiguousarray(a).view(np.uint16)


def report_mismatch(name, got, want):
    bad = np.argwhere(got != want)
    return f"{name}: {len(bad)} mismatches, first at {bad[:3].tolist()}: got {got[tuple(bad[0])]!r} want {want[tuple(bad[0])]!r}"
