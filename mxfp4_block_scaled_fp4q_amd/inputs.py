"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no step of the quantisation method: it only draws numbers
(numpy PCG64, float32) and rounds them to bf16 with torch's round-to-nearest-
even cast.  bf16 tensors are returned as numpy uint16 bit patterns, fp32 as
float32.  Shapes and distributions mirror the layer workloads of the FP4
training pages (LLaMA-1B FFN up-projection, LLaMA-2 13B-shaped layer with
persistent hot channels, Student-t activations); no dataset is involved.
"""
import hashlib

import numpy as np
import torch


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even, torch's cast) as uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def normal(shape, seed, std=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def student_t(shape, seed, nu=3.0, mult=0.5):
    rng = np.random.default_rng(seed)
    return (rng.standard_t(nu, size=shape) * mult).astype(np.float32)


def with_outliers(a, seed, count, mult):
    """Multiply `count` distinct positions (drawn with `seed`) by `mult`."""
    rng = np.random.default_rng(seed)
    flat = a.reshape(-1).copy()
    pos = rng.choice(flat.size, size=count, replace=False)
    flat[pos] *= np.float32(mult)
    return flat.reshape(a.shape)


def hot_channels(k, seed, ratio=0.09):
    """round(ratio*k) distinct channel indices, sorted ascending (int32)."""
    rng = np.random.default_rng(seed)
    n = int(round(ratio * k))
    return np.sort(rng.choice(k, size=n, replace=False)).astype(np.int32)


# --- the five workloads ----------------------------------------------------

def tiny_ref():
    """256x256 fp32 N(0,1) with 1% (655) entries x50, twice; grad N(0,1)."""
    n = 256 * 256
    cnt = int(round(0.01 * n))
    a = with_outliers(normal((256, 256), 101), 102, cnt, 50.0)
    b = with_outliers(normal((256, 256), 103), 104, cnt, 50.0)
    g = normal((256, 256), 105)
    return {"A": a, "B": b, "G": g}


def activation_sweep(rows=4096, cols=2048):
    """bf16 Student-t(3) x 0.5 activation and an N(0,1) bf16 grad."""
    x = to_bf16_bits(student_t((rows, cols), 201))
    g = to_bf16_bits(normal((rows, cols), 202))
    return {"X": x, "G": g, "sr_seed": 1234}


def ffn_forward(m=8192, k=2048, n=5632):
    """LLaMA-1B FFN up-projection: X bf16 [m,k] N(0,1), W bf16 [k,n] N(0,0.02)."""
    x = to_bf16_bits(normal((m, k), 301))
    w = to_bf16_bits(normal((k, n), 302, 0.02))
    return {"X": x, "W": w}


def ffn_backward_grad(m=8192, n=5632):
    """dY bf16 [m,n] N(0,1e-3); SR seeds 1234 (row) and 1235 (column)."""
    dy = to_bf16_bits(normal((m, n), 401, 1e-3))
    return {"dY": dy, "seed_row": 1234, "seed_col": 1235}


def outlier_layer(m=16384, k=5120, n=13824):
    """13B-shaped layer: X fp32 N(0,1) with 9% hot columns x100 -> bf16;
    W bf16 [k,n] N(0,0.02)."""
    hot = hot_channels(k, 502)
    xf = normal((m, k), 501)
    xf[:, hot] *= np.float32(100.0)
    x = to_bf16_bits(xf)
    del xf
    w = to_bf16_bits(normal((k, n), 503, 0.02))
    return {"X": x, "W": w, "hot": hot}
