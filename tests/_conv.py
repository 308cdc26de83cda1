"""Tensor <-> numpy helpers shared by the tests (no arithmetic of the method)."""
import numpy as np
import torch


def u16(t):
    """bf16 tensor (any device) -> numpy uint16 bit patterns."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def np_(t):
    return t.detach().cpu().contiguous().numpy()


def bf16_from_f32(a, device):
    return torch.tensor(np.asarray(a, np.float32), device=device).to(torch.bfloat16)


def bf16_bits_to_f64(a):
    return torch.tensor(np.asarray(a, np.uint16).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def dev_i32(a, device):
    return torch.tensor(np.asarray(a, np.int32), device=device)


def rel_close(got, ref, rtol=1e-3, floor=1e-5):
    """|got - ref| <= rtol * |ref| + floor * max|ref| elementwise (both finite),
    and identical non-finite positions."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    if not np.array_equal(fin, np.isfinite(got)):
        return False, "non-finite positions differ"
    if not np.array_equal(got[~fin], ref[~fin]):
        return False, "non-finite values differ"
    if not fin.any():
        return True, ""
    scale = np.abs(ref[fin]).max()
    err = np.abs(got[fin] - ref[fin])
    lim = rtol * np.abs(ref[fin]) + floor * scale
    bad = err > lim
    if bad.any():
        i = np.argmax(err - lim)
        return False, "max excess at %d: got %r ref %r (%d bad of %d)" % (i, got[fin][i], ref[fin][i], bad.sum(),
                                                                         bad.size)
    return True, ""
