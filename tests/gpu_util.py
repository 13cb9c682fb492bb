"""Helpers for the GPU parity tests (host <-> device marshalling only)."""
import numpy as np


def torch():
    import torch as t
    return t


def dev_bf16(bits: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(t.bfloat16).cuda()


def dev(a: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    tt = torch()
    if t.dtype == tt.bfloat16:
        return t.view(tt.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rel_fro(got, want):
    want = np.asarray(want, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    den = np.linalg.norm(want)
    return np.linalg.norm(got - want) / den if den > 0 else np.linalg.norm(got)


def first_mismatch(a, b):
    idx = np.argwhere(a != b)
    return None if len(idx) == 0 else (tuple(idx[0]), a[tuple(idx[0])], b[tuple(idx[0])], len(idx))
