"""Helpers for the GPU tests: move synth bit patterns to and from torch."""
import os
import sys

import numpy as np
import pytest
import torch

import synth


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def announce(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failure can be traced."""
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a.copy()).view(torch.bfloat16).cuda()


def dev_f16(bits: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a.copy()).view(torch.float16).cuda()


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8).copy()).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host_f64_of_bf16(t: torch.Tensor) -> np.ndarray:
    return synth.bf16_bits_to_f32(host_bits(t)).astype(np.float64)


def rel_l2_rows(got: np.ndarray, want: np.ndarray) -> np.ndarray:
    got = got.reshape(got.shape[0], -1).astype(np.float64)
    want = want.reshape(want.shape[0], -1).astype(np.float64)
    return np.linalg.norm(got - want, axis=1) / np.maximum(np.linalg.norm(want, axis=1), 1e-30)


class env:
    """Temporarily set environment variables read by the library per call."""

    def __init__(self, **kw):
        self.kw = {k: str(v) for k, v in kw.items()}
        self.old = {}

    def __enter__(self):
        for k, v in self.kw.items():
            self.old[k] = os.environ.get(k)
            os.environ[k] = v
        return self

    def __exit__(self, *a):
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
