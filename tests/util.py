"""Test helpers: host <-> device transfers of the synthetic inputs (no arithmetic of the method)."""
import numpy as np
import torch


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch.bfloat16 CUDA tensor (bitwise copy)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bf16(t: torch.Tensor) -> np.ndarray:
    """torch.bfloat16 tensor -> uint16 bit patterns on the host (bitwise copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def row_rel_l2(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """rel-L2 of every row (last axis flattened per leading index) of got against ref."""
    got = np.asarray(got, np.float64).reshape(len(got), -1)
    ref = np.asarray(ref, np.float64).reshape(len(ref), -1)
    den = np.linalg.norm(ref, axis=1)
    return np.linalg.norm(got - ref, axis=1) / np.where(den > 0, den, 1.0)


def assert_rel(got, ref, rtol=1e-5):
    """|got - ref| <= rtol * |ref| elementwise; exact zero where ref == 0."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    bad = np.abs(got - ref) > rtol * np.abs(ref)
    if bad.any():
        i = np.flatnonzero(bad)[:5]
        raise AssertionError(f"{bad.sum()} of {bad.size} elements off: idx {i.tolist()} "
                             f"got {got.reshape(-1)[i].tolist()} ref {ref.reshape(-1)[i].tolist()}")
