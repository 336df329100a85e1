"""Runs PyTorch's header-only Philox4x32-10 engine (compiled from
tests/philox_torch_ref.cpp with g++ on first use) on a batch of
(seed, subsequence, offset) triples."""
import functools
import os
import subprocess
import tempfile

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


@functools.lru_cache(maxsize=1)
def _binary():
    import torch

    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    out = os.path.join(tempfile.mkdtemp(prefix="philox_ref_"), "philox_ref")
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", inc, os.path.join(HERE, "philox_torch_ref.cpp"), "-o", out],
                   check=True, capture_output=True)
    return out


def torch_philox_first_block(triples):
    """[len(triples), 4] uint64: the engine's first four outputs per (seed, subsequence, offset)."""
    text = "".join(f"{int(s)} {int(u)} {int(o)}\n" for s, u, o in triples)
    res = subprocess.run([_binary()], input=text, capture_output=True, text=True, check=True)
    return np.array([[int(v) for v in line.split()] for line in res.stdout.splitlines()], dtype=np.uint64)
