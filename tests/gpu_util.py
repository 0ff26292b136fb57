"""Helpers for the GPU tests: moving seeded inputs to the device and the
oracle's expectations next to the library's outputs.  Expected values always
come from ``oracle`` or from the inputs themselves, never from the library."""

import sys

import numpy as np

import oracle as O

CODE_OF_KIND = {
    "CU_START": -10,
    "CU_MONOTONE": -11,
    "CU_TOTAL": -12,
    "CU_DIVISIBLE": -13,
    "REAL_GT_PADDED": -14,
}


def say(*msg):
    print("[gpu-test]", *msg, flush=True)
    sys.stdout.flush()


def dev_i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).cuda()


def dev_i64(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int64))).cuda()


def expected_route(cu, cp, total):
    r = O.build_route(np.asarray(cu).tolist(), cp, total)
    runs = O.canonical_runs(r)
    return r, runs


def check_route_matches_oracle(route, cu, cp, total):
    """Device route (runs in both orders, split matrix) equals the oracle's
    canonical route exactly."""
    r, runs = expected_route(cu, cp, total)
    assert route.status() == 0
    by_src, by_dst, split = route.copy_out()
    assert by_src.shape == runs.shape, (by_src.shape, runs.shape)
    assert np.array_equal(by_src.astype(np.int64), runs)
    order = np.argsort(runs[:, 1], kind="stable")
    assert np.array_equal(by_dst.astype(np.int64), runs[order])
    assert np.array_equal(split.astype(np.int64), r["split"])
    return r


def oracle_source_rows(r, direction):
    """For each output row, the input row the oracle copies it from."""
    if direction == "z2c":
        return r["src_row"][r["contiguous"]]
    return r["dst_row"][r["zigzag"]]
