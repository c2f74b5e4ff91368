"""Helpers for the GPU parity tests: move bf16 bit patterns to the device and
compare device outputs with the CPU oracle byte for byte."""
import numpy as np
import torch


def to_dev(x_u16: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x_u16).view(np.int16)).view(torch.bfloat16)
    return t.to("cuda:0")


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def assert_bytes_equal(got, exp, name):
    got = np.asarray(got)
    exp = np.asarray(exp)
    assert got.shape == exp.shape, f"{name}: shape {got.shape} != {exp.shape}"
    if got.dtype == np.float32:
        got = got.view(np.uint32)
        exp = exp.view(np.uint32)
    bad = np.nonzero(got.reshape(-1) != exp.reshape(-1))[0]
    if bad.size:
        i = bad[0]
        raise AssertionError(f"{name}: {bad.size} of {got.size} differ; first at flat index {i}: "
                             f"got {got.reshape(-1)[i]:#x} expected {exp.reshape(-1)[i]:#x}")


def compare_cast(dev_out: dict, ref: dict, keys=None):
    keys = keys or [k for k in ("row_q", "row_sf", "row_amax", "col_q", "col_sf", "col_amax") if k in ref]
    for k in keys:
        assert_bytes_equal(host(dev_out[k]).reshape(ref[k].shape), ref[k], k)
