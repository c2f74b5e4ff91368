"""Helpers for the GPU parity tests: move bf16 bit patterns to the device,
give every cast output canary-filled guard regions, and compare device
outputs with the CPU oracle byte for byte."""
import numpy as np
import torch

import nvfp4_block_scaled_bf16_amd as nv

# Every output buffer a parity test hands to the library sits inside a larger
# allocation: GUARD_BYTES on each side, and the buffer itself, are filled with
# CANARY before the call.  After the call the guards must be untouched (no
# write past either end), and the buffer is compared in full with the oracle:
# a byte the kernel never wrote keeps the canary, which is never a valid scale
# byte (sign bit set) nor a valid amax (negative), and matches an expected
# data byte only where that byte happens to be 0xA5.
GUARD_BYTES = 64
CANARY = 0xA5


def to_dev(x_u16: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x_u16).view(np.int16)).view(torch.bfloat16)
    return t.to("cuda:0")


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


class Guarded:
    """Caller buffers with canary-filled guard regions.  spec: name ->
    (element count, torch dtype).  `views` are the buffers to pass."""

    def __init__(self, spec):
        self.views, self._back = {}, {}
        for name, (numel, dtype) in spec.items():
            nbytes = int(numel) * torch.empty((), dtype=dtype).element_size()
            b = torch.full((2 * GUARD_BYTES + nbytes,), CANARY, dtype=torch.uint8, device="cuda:0")
            self._back[name] = (b, nbytes)
            self.views[name] = b[GUARD_BYTES:GUARD_BYTES + nbytes].view(dtype)

    def __getitem__(self, k):
        return self.views[k]

    def __contains__(self, k):
        return k in self.views

    def keys(self):
        return self.views.keys()

    def check_guards(self):
        for name, (b, nbytes) in self._back.items():
            head = host(b[:GUARD_BYTES])
            tail = host(b[GUARD_BYTES + nbytes:])
            if not (head == CANARY).all() or not (tail == CANARY).all():
                raise AssertionError(f"{name}: bytes written outside the buffer "
                                     f"(before: {int((head != CANARY).sum())}, after: {int((tail != CANARY).sum())})")


U8, F32 = torch.uint8, torch.float32


def cast_spec(M, K, mode, rowwise=True, columnwise=True):
    """Output layout of nvfp4_quantize (the header's)."""
    a = (lambda n: 1) if mode == nv.PER_TENSOR else (lambda n: n)
    spec = {}
    if rowwise:
        spec.update(row_q=(M * (K // 2), U8), row_sf=(M * (K // 16), U8), row_amax=(a(M), F32))
    if columnwise:
        spec.update(col_q=(K * (M // 2), U8), col_sf=(K * (M // 16), U8), col_amax=(a(K), F32))
    return spec


def grouped_spec(T, K, G, rowwise=True, columnwise=True):
    spec = {}
    if rowwise:
        spec.update(row_q=(T * (K // 2), U8), row_sf=(T * (K // 16), U8), row_amax=(T, F32))
    if columnwise:
        spec.update(col_q=(T * (K // 2), U8), col_sf=(T * (K // 16), U8), col_amax=(G * K, F32))
    return spec


def quantize_guarded(d, mode, rowwise=True, columnwise=True):
    M, K = d.shape
    g = Guarded(cast_spec(M, K, mode, rowwise, columnwise))
    nv.quantize_into(d, mode, **g.views)
    return g


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


def compare_cast(dev_out, ref, keys=None):
    """Byte-for-byte comparison; for Guarded outputs, the guards first (the
    caller has synchronized the device)."""
    if isinstance(dev_out, Guarded):
        dev_out.check_guards()
    keys = keys or [k for k in ("row_q", "row_sf", "row_amax", "col_q", "col_sf", "col_amax") if k in ref]
    for k in keys:
        assert_bytes_equal(host(dev_out[k]).reshape(ref[k].shape), ref[k], k)
