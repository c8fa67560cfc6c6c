"""Seeded synthetic inputs for the HFQ4 MoE decode path and its oracle.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no quantization, routing, softmax or GEMV).  Both the
oracle-side tests and the GPU path take their inputs from here.

Recipes (the shapes and distributions of the workloads; all f32):

* tiny layer   -- d=256, F=128, E=8, k=2, 1 token.  Drawn on the host with
  numpy ``default_rng(seed)`` in a fixed order: x ~ N(0,1) [1, d];
  Wr ~ N(0, 0.05) [E, d]; then per expert gate [F, d], up [F, d],
  down [d, F] ~ N(0, 0.02).
* large layers -- d=2048, F=512, E in {256, 512}.  Every expert matrix has
  its own seed derived from (seed, layer, expert, matrix), so any subset of
  experts can be regenerated independently and bit-identically on the
  device that drew it (torch Philox on the GPU, torch CPU generator on the
  host).  Router Wr ~ N(0, 0.02) [E, d], expert weights ~ N(0, 0.02),
  x ~ N(0, 1).
* stack          -- per layer the same expert/router recipe plus a dense
  d x d matrix ~ N(0, 0.1/sqrt(d)) (dense_f32).
* skew           -- a per-expert Zipf(s) log-offset added to the router
  logits: bias[e] = -s * ln(rank[e]) with rank a seeded permutation of
  1..E (the hot set is the experts of low rank).
"""

import numpy as np

GATE, UP, DOWN, ROUTER, DENSE, X = 0, 1, 2, 3, 4, 5


def tiny_layer(seed=0, d=256, F=128, E=8, xstd=1.0, rstd=0.05, wstd=0.02):
    """Host-side tiny layer; returns dict of float32 numpy arrays."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((1, d)).astype(np.float32) * np.float32(xstd)
    Wr = (rng.standard_normal((E, d)) * rstd).astype(np.float32)
    gate = np.empty((E, F, d), np.float32)
    up = np.empty((E, F, d), np.float32)
    down = np.empty((E, d, F), np.float32)
    for e in range(E):
        gate[e] = (rng.standard_normal((F, d)) * wstd).astype(np.float32)
        up[e] = (rng.standard_normal((F, d)) * wstd).astype(np.float32)
        down[e] = (rng.standard_normal((d, F)) * wstd).astype(np.float32)
    return {"x": x, "Wr": Wr, "gate": gate, "up": up, "down": down,
            "d": d, "F": F, "E": E}


def host_matrix(seed, rows, cols, std, *salt):
    """Host (numpy PCG64) normal matrix with a salted seed; float32."""
    ss = np.random.SeedSequence([int(seed)] + [int(s) for s in salt])
    rng = np.random.default_rng(ss)
    return (rng.standard_normal((rows, cols)) * std).astype(np.float32)


def _seed(seed, layer, expert, which):
    # distinct 63-bit seed per (seed, layer, expert, matrix)
    ss = np.random.SeedSequence([int(seed), int(layer), int(expert), int(which)])
    return int(ss.generate_state(2, np.uint64)[0] & np.uint64((1 << 63) - 1))


def device_matrix(torch, device, seed, layer, expert, which, rows, cols, std):
    """Normal(0, std) float32 [rows, cols] drawn by torch on `device` with a
    per-(seed, layer, expert, which) generator."""
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, layer, expert, which))
    t = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def expert_f32(torch, device, seed, layer, expert, d, F, std=0.02):
    """(gate [F, d], up [F, d], down [d, F]) float32 on `device`."""
    return (device_matrix(torch, device, seed, layer, expert, GATE, F, d, std),
            device_matrix(torch, device, seed, layer, expert, UP, F, d, std),
            device_matrix(torch, device, seed, layer, expert, DOWN, d, F, std))


def router_f32(torch, device, seed, layer, E, d, std=0.02):
    return device_matrix(torch, device, seed, layer, 0, ROUTER, E, d, std)


def dense_f32(torch, device, seed, layer, d, std=None):
    """Dense d x d matrix of a stack layer, N(0, std) with std = 0.1/sqrt(d)
    by default: its update D x then has a tenth of the residual's norm, so a
    40-layer residual stack stays near unit scale (N(0, 0.02) at d = 2048
    would grow the residual 1.35x per layer and, through the experts'
    quadratic SiLU(gate)*up term, overflow f32 within about 20 layers)."""
    if std is None:
        std = 0.1 / float(np.sqrt(d))
    return device_matrix(torch, device, seed, layer, 0, DENSE, d, d, std)


def activations(torch, device, seed, n, d, std=1.0):
    """x pool [n, d] ~ N(0, std) float32."""
    return device_matrix(torch, device, seed, 0, 0, X, n, d, std)


def zipf_bias(seed, E, s=1.1):
    """bias[e] = -s * ln(rank[e]), rank a seeded permutation of 1..E (float32)."""
    rng = np.random.default_rng(np.random.SeedSequence([int(seed), 0x5A1F]))
    rank = rng.permutation(E) + 1
    return (-s * np.log(rank.astype(np.float64))).astype(np.float32)
