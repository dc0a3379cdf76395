"""Seeded synthetic inputs for the KLA scan: the five named workloads and
arbitrary shapes.

This module only draws random numbers and shapes them into gate tensors; it
holds none of the filter's arithmetic.  Both the CPU oracle and the HIP
library are fed from here, so both sides always see the same tensors.

Recipe (every workload):
  * draw four float64 tensors of shape [B, H, T, D] from one seeded
    ``torch.Generator`` in the order z_a, z_p, z_phi, y (standard normals, or
    fair coin flips for the "hard" gates);
  * map them to gates in float64;
  * round each gate once to the input dtype (fp32 round-to-nearest-even; bf16
    via fp32, then round-to-nearest-even).
The initial posterior is lam0 = 1, eta0 = 0 (fp32, [B, H, D]) unless a test
asks for a random one.

Gate families:
  std  : a = sigmoid(z_a + 2), p = softplus(z_p), phi = softplus(z_phi),
         b = phi * y
  slow : a = 1 - 1e-3 * sigmoid(z_a), p = 1e-4 * softplus(z_p),
         phi = softplus(z_phi), b = phi * y
  hard : a in {1e-3, 1}, p in {0, 1}, phi in {0, 1e4}, y in {-1, +1}, each
         equiprobable, b = phi * y
softplus(x) = log(1 + e^x) computed as logaddexp(0, x); sigmoid(x) =
1 / (1 + e^-x).

The gate scales follow the KLA parameterisation reviewed on the Pith page for
arXiv 2602.10743 (a decay in (0, 1], learned process noise, non-negative
evidence precision) and the layer shapes of its MAD and MQAR hyper-parameter
tables (H * D = 1024 and 4096 channels, sequence length 2048 and longer).
The data sets themselves are not used: these tensors stand in for them.
"""

from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    key: int
    name: str
    B: int
    H: int
    T: int
    D: int
    dtype: str  # "f32" or "bf16": dtype of a, p, phi, b
    gates: str  # "std", "slow" or "hard"
    seed: int

    @property
    def shape(self):
        return (self.B, self.H, self.T, self.D)

    @property
    def elements(self) -> int:
        return self.B * self.H * self.T * self.D

    @property
    def channels(self) -> int:
        return self.B * self.H * self.D

    def describe(self) -> str:
        return "%s B=%d H=%d T=%d D=%d %s gates=%s seed=%d" % (
            self.name, self.B, self.H, self.T, self.D, self.dtype, self.gates, self.seed)


WORKLOADS = {
    0: Workload(0, "tiny-ref", 1, 1, 256, 16, "f32", "std", 0),
    1: Workload(1, "small-lm-layer", 8, 16, 2048, 64, "f32", "std", 1),
    2: Workload(2, "1b-scale-layer", 4, 32, 8192, 128, "bf16", "std", 2),
    3: Workload(3, "long-context", 1, 32, 131072, 128, "f32", "slow", 3),
    4: Workload(4, "state-tracking-stress", 256, 8, 512, 32, "f32", "hard", 4),
}

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def _round(x64: torch.Tensor, dtype: str) -> torch.Tensor:
    x32 = x64.to(torch.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return x32.to(torch.bfloat16)
    raise ValueError("unknown dtype %r" % dtype)


def _softplus(x: torch.Tensor) -> torch.Tensor:
    return torch.logaddexp(torch.zeros_like(x), x)


def _draw(shape, gen, device, gates):
    if gates == "hard":
        return torch.randint(0, 2, shape, generator=gen, device=device).to(torch.float64)
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float64)


def make_gates(shape, gates: str = "std", dtype: str = "f32", seed: int = 0,
               device="cpu"):
    """Returns dict(a, p, phi, b) of tensors of `shape` ([B, H, T, D])."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    shape = tuple(int(s) for s in shape)

    z = _draw(shape, gen, device, gates)
    if gates == "std":
        a64 = torch.sigmoid(z + 2.0)
    elif gates == "slow":
        a64 = 1.0 - 1e-3 * torch.sigmoid(z)
    elif gates == "hard":
        a64 = torch.where(z > 0.5, 1.0, 1e-3)
    else:
        raise ValueError("unknown gate family %r" % gates)
    a = _round(a64, dtype)
    del z, a64

    z = _draw(shape, gen, device, gates)
    if gates == "std":
        p64 = _softplus(z)
    elif gates == "slow":
        p64 = 1e-4 * _softplus(z)
    else:
        p64 = torch.where(z > 0.5, 1.0, 0.0)
    p = _round(p64, dtype)
    del z, p64

    z = _draw(shape, gen, device, gates)
    if gates in ("std", "slow"):
        phi64 = _softplus(z)
    else:
        phi64 = torch.where(z > 0.5, 1e4, 0.0)
    phi = _round(phi64, dtype)
    del z

    z = _draw(shape, gen, device, gates)
    y = z if gates in ("std", "slow") else torch.where(z > 0.5, 1.0, -1.0)
    b = _round(phi64 * y, dtype)
    del z, y, phi64
    return {"a": a, "p": p, "phi": phi, "b": b}


def make_initial_state(B, H, D, random: bool = False, seed: int = 0, device="cpu"):
    """lam0, eta0 as fp32 [B, H, D]: (1, 0), or lam0 = softplus(N) + 0.1 and
    eta0 = lam0 * N when random."""
    device = torch.device(device)
    if not random:
        return (torch.ones((B, H, D), dtype=torch.float32, device=device),
                torch.zeros((B, H, D), dtype=torch.float32, device=device))
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) + 7919)
    z1 = torch.randn((B, H, D), generator=gen, device=device, dtype=torch.float64)
    z2 = torch.randn((B, H, D), generator=gen, device=device, dtype=torch.float64)
    lam0 = _softplus(z1) + 0.1
    return lam0.to(torch.float32), (lam0 * z2).to(torch.float32)


def make_workload(key: int, device="cpu", seed: int | None = None):
    """Gates and initial state of a named workload (0..4)."""
    w = WORKLOADS[key]
    g = make_gates(w.shape, w.gates, w.dtype, w.seed if seed is None else seed, device)
    g["lam0"], g["eta0"] = make_initial_state(w.B, w.H, w.D, device=device)
    return g


# ---------------------------------------------------------------------------
# Fused-mixer inputs.
#
# Recipe: one seeded torch.Generator draws, in order, four float64 standard
# normal tensors [B, H, T, D] (z_k, z_v, z_lv, z_q) and then, per (h, d)
# channel, u_A, u_dt (uniform [0, 1)) and z_p (standard normal):
#   k = z_k, v = z_v, lam_v = softplus(z_lv), q = z_q         (token inputs)
#   A = 1 + 15 u_A, delta = exp(ln 1e-3 + u_dt (ln 0.1 - ln 1e-3)),
#   a = exp(-A delta)                                          (OU decay)
#   p = 0.01 exp(0.5 z_p)                                      (process noise)
# Token inputs are rounded once to the input dtype (as the gates above); a
# and p are float32.  The ranges follow the free-parameter ledger of the Pith
# review of arXiv 2602.10743 (delta learned in [0.001, 0.1], process-noise
# scale initialised at 0.01, value precision from the input); the decay rates
# A in [1, 16] span one state expansion of 16.

MIXER_WORKLOADS = {
    0: Workload(0, "mixer-tiny", 1, 1, 256, 16, "f32", "mixer", 10),
    1: Workload(1, "mixer-small-lm-layer", 8, 16, 2048, 64, "f32", "mixer", 11),
    2: Workload(2, "mixer-1b-scale-layer", 4, 32, 8192, 128, "bf16", "mixer", 12),
    3: Workload(3, "mixer-long-context", 1, 32, 131072, 128, "f32", "mixer", 13),
}


def make_mixer_inputs(shape, dtype: str = "f32", seed: int = 0, device="cpu"):
    """Returns dict(k, v, lam_v, q, a, p): token tensors of `shape`
    ([B, H, T, D]) and float32 [H, D] channel gates."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    shape = tuple(int(s) for s in shape)
    out = {}
    for name in ("k", "v", "lam_v", "q"):
        z = torch.randn(shape, generator=gen, device=device, dtype=torch.float64)
        out[name] = _round(_softplus(z) if name == "lam_v" else z, dtype)
        del z
    H, D = shape[1], shape[3]
    u_A = torch.rand((H, D), generator=gen, device=device, dtype=torch.float64)
    u_dt = torch.rand((H, D), generator=gen, device=device, dtype=torch.float64)
    z_p = torch.randn((H, D), generator=gen, device=device, dtype=torch.float64)
    A = 1.0 + 15.0 * u_A
    lo, hi = torch.log(torch.tensor(1e-3, dtype=torch.float64)), torch.log(
        torch.tensor(0.1, dtype=torch.float64))
    delta = torch.exp(lo.to(device) + u_dt * (hi - lo).to(device))
    out["a"] = torch.exp(-A * delta).to(torch.float32)
    out["p"] = (0.01 * torch.exp(0.5 * z_p)).to(torch.float32)
    return out


def make_mixer_workload(key: int, device="cpu", seed: int | None = None):
    """Inputs and initial state of a named mixer workload (0..3)."""
    w = MIXER_WORKLOADS[key]
    g = make_mixer_inputs(w.shape, w.dtype, w.seed if seed is None else seed, device)
    g["lam0"], g["eta0"] = make_initial_state(w.B, w.H, w.D, device=device)
    return g


# ---------------------------------------------------------------------------
# Time-invariant-gate (LTI) inputs.
#
# Recipe: one seeded torch.Generator draws z_a, z_p, z_phi per (h, d) channel
# ([H, D]; standard normals, or coin flips for "hard"), maps them with the
# gate family of make_gates to a, p, phi (float32), then draws y per token
# ([B, H, T, D]) and sets b = phi[h, d] * y, rounded once to the input dtype.

LTI_WORKLOADS = {
    0: Workload(0, "lti-tiny", 1, 1, 256, 16, "f32", "std", 20),
    1: Workload(1, "lti-small-lm-layer", 8, 16, 2048, 64, "f32", "std", 21),
    2: Workload(2, "lti-1b-scale-layer", 4, 32, 8192, 128, "bf16", "std", 22),
    3: Workload(3, "lti-long-context", 1, 32, 131072, 128, "f32", "slow", 23),
}


def make_lti_inputs(shape, gates: str = "std", dtype: str = "f32", seed: int = 0,
                    device="cpu"):
    """Returns dict(a, p, phi, b): float32 [H, D] channel gates and the
    token information b of `shape` ([B, H, T, D]) in the input dtype."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    shape = tuple(int(s) for s in shape)
    ch = (shape[1], shape[3])
    z = _draw(ch, gen, device, gates)
    if gates == "std":
        a64 = torch.sigmoid(z + 2.0)
    elif gates == "slow":
        a64 = 1.0 - 1e-3 * torch.sigmoid(z)
    elif gates == "hard":
        a64 = torch.where(z > 0.5, 1.0, 1e-3)
    else:
        raise ValueError("unknown gate family %r" % gates)
    z = _draw(ch, gen, device, gates)
    if gates == "std":
        p64 = _softplus(z)
    elif gates == "slow":
        p64 = 1e-4 * _softplus(z)
    else:
        p64 = torch.where(z > 0.5, 1.0, 0.0)
    z = _draw(ch, gen, device, gates)
    phi64 = _softplus(z) if gates in ("std", "slow") else torch.where(z > 0.5, 1e4, 0.0)
    out = {"a": a64.to(torch.float32), "p": p64.to(torch.float32),
           "phi": phi64.to(torch.float32)}
    z = _draw(shape, gen, device, gates)
    y = z if gates in ("std", "slow") else torch.where(z > 0.5, 1.0, -1.0)
    phi_b = out["phi"].to(torch.float64)[None, :, None, :]
    out["b"] = _round(phi_b * y, dtype)
    return out


def make_lti_workload(key: int, device="cpu", seed: int | None = None):
    """Inputs and initial state of a named LTI workload (0..3)."""
    w = LTI_WORKLOADS[key]
    g = make_lti_inputs(w.shape, w.gates, w.dtype, w.seed if seed is None else seed, device)
    g["lam0"], g["eta0"] = make_initial_state(w.B, w.H, w.D, device=device)
    return g


def broadcast_lti(g):
    """The LTI inputs as full [B, H, T, D] gates (a, p, phi, b) on the CPU in
    float64, for the oracle."""
    b = g["b"].detach().to("cpu").double()
    B, H, T, D = b.shape
    full = {n: g[n].detach().to("cpu").double()[None, :, None, :].expand(B, H, T, D)
            for n in ("a", "p", "phi")}
    full["b"] = b
    return full
