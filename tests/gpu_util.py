"""Helpers shared by the GPU parity tests: host <-> device marshalling and the
comparison rules (bit-exact for codes/scales/scalars, the stated tolerance for
the RHT paths and the GEMM)."""
import sys

import numpy as np

import oracle


def say(*args):
    print("[gpu-case]", *args, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def gpu_q_as_dict(q) -> dict:
    return dict(codes=host(q.codes), scales=host(q.scales), S=np.float32(host(q.global_scale)[0]),
                amax=np.float32(host(q.amax)[0]), rows=q.rows, cols=q.cols, scale_kind=q.scale_kind)


def assert_bit_exact(g: dict, o: dict, what=""):
    assert g["codes"].shape == o["codes"].shape, what
    assert g["scales"].shape == o["scales"].shape, what
    assert np.float32(g["amax"]).view(np.uint32) == np.float32(o["amax"]).view(np.uint32), (what, g["amax"], o["amax"])
    assert np.float32(g["S"]).view(np.uint32) == np.float32(o["S"]).view(np.uint32), (what, g["S"], o["S"])
    bad_s = np.count_nonzero(g["scales"] != o["scales"])
    bad_c = np.count_nonzero(g["codes"] != o["codes"])
    assert bad_s == 0 and bad_c == 0, "%s: %d scale bytes and %d code bytes differ" % (what, bad_s, bad_c)


def _ordinal(codes_u8):
    lo = (codes_u8 & 15).astype(np.int16)
    hi = (codes_u8 >> 4).astype(np.int16)
    out = []
    for c in (lo, hi):
        mag = c & 7
        out.append(np.where(c & 8, -mag, mag))
    return np.stack(out, axis=-1)


def assert_rht_tolerance(g: dict, o: dict, what=""):
    """RHT paths: codes differ by at most one E2M1 step on at most 1e-5 of the
    elements, scales on at most 1e-5 of the blocks (by at most one E4M3 step),
    S within 2^-20 relative."""
    assert abs(float(g["S"]) - float(o["S"])) <= 2.0 ** -20 * abs(float(o["S"])), what
    d = np.abs(_ordinal(g["codes"]) - _ordinal(o["codes"]))
    n = d.size
    assert d.max(initial=0) <= 1, what
    assert np.count_nonzero(d) <= 1e-5 * n, (what, np.count_nonzero(d))
    ds = np.abs(g["scales"].astype(np.int16) - o["scales"].astype(np.int16))
    assert ds.max(initial=0) <= 1 and np.count_nonzero(ds) <= max(1e-5 * ds.size, 0), (what, np.count_nonzero(ds))


def rel_frobenius(c: np.ndarray, ref: np.ndarray) -> float:
    c = c.astype(np.float64)
    ref = ref.astype(np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(c - ref) / den) if den > 0 else float(np.linalg.norm(c))
