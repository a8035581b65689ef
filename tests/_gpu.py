"""Helpers shared by the GPU tests: device tensors from numpy and back."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")


def have_gpu() -> bool:
    return torch.cuda.is_available()


def q():
    import gemm_q4nx_chunk_amd as mod
    return mod


def dev_u8(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a).reshape(-1).view(np.uint8)).cuda()


def dev_bf16(bits: np.ndarray):
    """bf16 bit patterns (uint16) -> device int16 tensor with the same bytes."""
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda()


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def weight(chunks_dev, N, K, kind, layout=None):
    return q().weight(chunks_dev, N, K, kind, layout)


def gemv(chunks_dev, N, K, kind, x_bits, layout=None):
    """Run q4nx_gemv; returns y [M, N] float32 on the host."""
    M = x_bits.shape[0]
    x = dev_bf16(x_bits)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    q().gemv(weight(chunks_dev, N, K, kind, layout), x, y, M)
    return host(y)


_SHIFT = {}


def shift_xcd_start(n_wg: int = 1):
    """Launch n_wg one-workgroup GEMVs (q4nx_gemv of a 32 x 256 weight).

    Workgroups are dealt to the XCDs round-robin from a starting XCD that
    carries over between launches, so launches of odd workgroup counts move
    where the next launch's workgroup 0 lands.  Tests of the XCD-local
    exchanges put these between calls.
    """
    if "w" not in _SHIFT:
        import numpy as np
        _SHIFT["w"] = torch.zeros(5120, dtype=torch.uint8, device="cuda")
        _SHIFT["x"] = torch.zeros(256, dtype=torch.int16, device="cuda")
        _SHIFT["y"] = torch.empty(32, dtype=torch.float32, device="cuda")
    w = q().weight(_SHIFT["w"], 32, 256, "q4_1")
    for _ in range(n_wg):
        q().gemv(w, _SHIFT["x"], _SHIFT["y"], 1)
