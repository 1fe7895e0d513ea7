"""Helpers for the GPU parity tests: host <-> device moves of bf16 bit
patterns and byte buffers, and a progress print that names the case before
each GPU step."""
import sys

import numpy as np
import torch

DEV = "cuda:0"
CANARY = 0xA5


def say(*args):
    print("[gpu-case]", *args, flush=True)
    sys.stdout.flush()


def bf16_to_dev(bits: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(bits, np.uint16).view(np.int16)
    return torch.from_numpy(a).view(torch.bfloat16).to(DEV)


def bf16_to_host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def i32_to_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)


def f32_to_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


def u8_to_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def mismatch_report(a: np.ndarray, b: np.ndarray, what: str) -> str:
    bad = np.argwhere(a != b)
    head = bad[:5].tolist()
    return "%s: %d mismatches, first at %s: got %s want %s" % (
        what, len(bad), head, [a[tuple(i)] for i in head],
        [b[tuple(i)] for i in head])


def assert_equal(got: np.ndarray, want: np.ndarray, what: str):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if not np.array_equal(got, want):
        raise AssertionError(mismatch_report(got, want, what))
