"""Helpers for the GPU parity tests (host <-> device copies and the tiled layout on the host)."""
import numpy as np

# implementations of the decode step that the step tests run (vv_state.path)
STEP_PATHS = ["layered", "chained"]


def dev(a, device="cuda"):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.float16)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device)
    return torch.from_numpy(a).to(device)


def host(t):
    import torch
    t = t.detach()
    if t.dtype == torch.float16:
        return t.view(torch.int16).cpu().numpy().view(np.float16)
    return t.cpu().numpy()


def host_u16(t):
    return host(t).view(np.uint16)


def codes_to_tiled(codes, sbits):
    """Tiled layout of include/vv.h built on the host from [N,K] codes and [N,K/32] scale bits."""
    codes = np.asarray(codes, np.uint32)
    N, K = codes.shape
    nb, T = K // 32, -(-N // 64)
    ng = -(-nb // 8)
    c = np.full((T * 64, K), 8, np.uint32)
    c[:N] = codes
    c = c.reshape(T * 64, nb, 4, 8)
    d = np.zeros((T * 64, nb, 4), np.uint32)
    for i in range(4):
        d |= c[..., 2 * i] << (4 * i)
        d |= c[..., 2 * i + 1] << (16 + 4 * i)
    q = d.reshape(T, 64, nb, 4).transpose(0, 2, 1, 3).astype("<u4").tobytes()
    s = np.zeros((T * 64, ng * 8), np.uint16)
    s[:N, :nb] = sbits
    s = s.reshape(T, 64, ng, 8).transpose(0, 2, 1, 3)
    return np.frombuffer(q, np.uint8).copy(), np.ascontiguousarray(s).reshape(-1)


def rel_err(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(y - ref)) / max(np.max(np.abs(ref)), 1e-300))
