"""Seeded synthetic inputs shaped like the decode workloads the pages discuss.

Shared by the HIP path's tests/bench and by the oracle's tests.  This module
draws random numbers and arranges them into the workload's structure (GQA
group sizes, planted high-scoring positions, a biased recent window); it holds
none of the decode method's arithmetic.

Five workloads (sizes named by what they are):

* ``tiny``          B1, Hq4, Hkv1, d64, N1024, r16, M64; 8 key rows replaced
                    by 3 * (group-mean query) + N(0, 0.1).
* ``gqa7_16k``      B8, Hq28, Hkv4 (G=7), d128, N16384, r32, M2048; 1% of rows
                    per KV head get k += 2 * (group-mean query).
* ``longctx_128k``  B32, Hq32, Hkv8, d128, N131072, r32, M2048; 0.5% of rows
                    get k += 2 * (group-mean query); the last 128 rows get
                    k += 1 * (group-mean query).
* ``reuse8_64k``    8 layers of B16, Hq32, Hkv8, d128, N65536, r32, M2048;
                    independent seeds per layer, no plants; indices computed on
                    layers 0 and 4 only.
* ``lisa_32k``      B16, Hq32, Hkv8, d128, N32768, r32, M1024; gate weights
                    w ~ N(0, 0.02) of shape [Hq, d].

All "N(0, s)" are normal with standard deviation s.  Keys, values and queries
are bf16 (rounded from fp32 draws); the basis P of each KV head is the Q factor
of a seeded d x r Gaussian (orthonormal columns), stored as fp32.
"""

from dataclasses import dataclass, field
import math

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    N: int
    r: int
    M: int
    layers: int = 1
    full_layers: tuple = (0,)
    # planted rows: (fraction of rows or absolute count, alpha, mode)
    plant_count: int = 0
    plant_alpha: float = 0.0
    plant_mode: str = "none"          # "replace" | "add" | "none"
    recent_rows: int = 0
    recent_beta: float = 0.0
    gate_std: float = 0.0

    @property
    def G(self):
        return self.Hq // self.Hkv

    @property
    def units(self):
        return self.B * self.Hkv


def _plants(n, frac):
    return max(1, int(round(n * frac)))


WORKLOADS = {
    "tiny": Workload("tiny", B=1, Hq=4, Hkv=1, d=64, N=1024, r=16, M=64,
                     plant_count=8, plant_alpha=3.0, plant_mode="replace"),
    "gqa7_16k": Workload("gqa7_16k", B=8, Hq=28, Hkv=4, d=128, N=16384, r=32, M=2048,
                         plant_count=_plants(16384, 0.01), plant_alpha=2.0,
                         plant_mode="add"),
    "longctx_128k": Workload("longctx_128k", B=32, Hq=32, Hkv=8, d=128, N=131072, r=32,
                             M=2048, plant_count=_plants(131072, 0.005),
                             plant_alpha=2.0, plant_mode="add",
                             recent_rows=128, recent_beta=1.0),
    "reuse8_64k": Workload("reuse8_64k", B=16, Hq=32, Hkv=8, d=128, N=65536, r=32,
                           M=2048, layers=8, full_layers=(0, 4)),
    "lisa_32k": Workload("lisa_32k", B=16, Hq=32, Hkv=8, d=128, N=32768, r=32, M=1024,
                         gate_std=0.02),
}


def scaled(wl: Workload, **kw) -> Workload:
    """Same recipe at other sizes (for tests that need a smaller instance)."""
    d = dict(wl.__dict__)
    d.update(kw)
    if "N" in kw and "plant_count" not in kw and wl.plant_count and wl.plant_mode == "add":
        frac = wl.plant_count / wl.N
        d["plant_count"] = _plants(kw["N"], frac)
    return Workload(**d)


def _seed(*parts):
    h = 1469598103934665603
    for p in parts:
        for ch in str(p).encode():
            h = ((h ^ ch) * 1099511628211) & ((1 << 63) - 1)
    return h


def orthonormal_basis(d, r, seed):
    """Q factor of a seeded d x r standard-normal matrix (float64)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((d, r))
    q, rr = np.linalg.qr(a)
    q = q * np.sign(np.diag(rr))[None, :]
    return q


@dataclass
class DecodeInputs:
    """Device (or CPU) tensors for one layer of one decode step."""
    wl: Workload
    q: torch.Tensor          # [B, Hq, d] bf16
    k_cache: torch.Tensor    # [B, Hkv, Ncap, d] bf16 (rows < N-1 filled)
    v_cache: torch.Tensor    # [B, Hkv, Ncap, d] bf16
    k_new: torch.Tensor      # [B, Hkv, 1, d] bf16 (token written at row N-1)
    v_new: torch.Tensor      # [B, Hkv, 1, d] bf16
    P: torch.Tensor          # [Hkv, d, r] fp32
    seq_lens: torch.Tensor   # [B] int32 (= N after the append)
    pos: torch.Tensor        # [B] int32 (= N-1)
    w_gate: torch.Tensor = None     # [Hq, d] fp32 (lisa only)
    plants: dict = field(default_factory=dict)   # (b, h) -> np.ndarray of rows


def make_decode_inputs(wl: Workload, seed=0, layer=0, device="cpu", capacity=None,
                       seq_lens=None):
    """Build one layer's inputs.  ``device`` may be "cpu" or "cuda".

    Draws are made with a torch generator on ``device`` so that the large
    workloads never pass through host memory; the same seed on the same kind
    of device gives the same bytes.  The per-KV-head bases come from numpy.
    """
    B, Hq, Hkv, d, N, r = wl.B, wl.Hq, wl.Hkv, wl.d, wl.N, wl.r
    G = wl.G
    Ncap = capacity or N
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(_seed(wl.name, seed, layer) % (1 << 62))

    def randn(*shape, std=1.0):
        x = torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        return x

    q = randn(B, Hq, d).to(torch.bfloat16)
    k_cache = torch.empty(B, Hkv, Ncap, d, dtype=torch.bfloat16, device=dev)
    v_cache = torch.empty(B, Hkv, Ncap, d, dtype=torch.bfloat16, device=dev)
    # fill row blocks so that no fp32 copy of a whole cache is ever held
    step = max(1, (1 << 26) // max(1, B * Hkv * d))
    for n0 in range(0, Ncap, step):
        n1 = min(Ncap, n0 + step)
        k_cache[:, :, n0:n1] = randn(B, Hkv, n1 - n0, d).to(torch.bfloat16)
        v_cache[:, :, n0:n1] = randn(B, Hkv, n1 - n0, d).to(torch.bfloat16)
    k_new = randn(B, Hkv, 1, d).to(torch.bfloat16)
    v_new = randn(B, Hkv, 1, d).to(torch.bfloat16)

    P = torch.from_numpy(np.stack([
        orthonormal_basis(d, r, _seed(wl.name, seed, layer, "P", h) % (1 << 62))
        for h in range(Hkv)]).astype(np.float32)).to(dev)

    # group-mean query: direction of the planted rows (input recipe only)
    qbar = q.float().view(B, Hkv, G, d).mean(dim=2)      # [B, Hkv, d]

    plants = {}
    if wl.plant_mode != "none" and wl.plant_count > 0:
        rng = np.random.default_rng(_seed(wl.name, seed, layer, "plants") % (1 << 62))
        hi = max(1, N - 1 - wl.recent_rows)
        cnt = min(wl.plant_count, hi)
        for b in range(B):
            for h in range(Hkv):
                rows = np.sort(rng.choice(hi, size=cnt, replace=False))
                plants[(b, h)] = rows
                ridx = torch.from_numpy(rows).to(dev)
                if wl.plant_mode == "replace":
                    noise = randn(cnt, d, std=0.1)
                    k_cache[b, h, ridx] = (wl.plant_alpha * qbar[b, h][None, :]
                                           + noise).to(torch.bfloat16)
                else:
                    k_cache[b, h, ridx] = (k_cache[b, h, ridx].float()
                                           + wl.plant_alpha * qbar[b, h][None, :]
                                           ).to(torch.bfloat16)
    if wl.recent_rows > 0:
        lo = max(0, N - wl.recent_rows)
        k_cache[:, :, lo:N - 1] = (k_cache[:, :, lo:N - 1].float()
                                   + wl.recent_beta * qbar[:, :, None, :]
                                   ).to(torch.bfloat16)
        k_new = (k_new.float() + wl.recent_beta * qbar[:, :, None, :]).to(torch.bfloat16)

    if seq_lens is None:
        seq_lens = torch.full((B,), N, dtype=torch.int32, device=dev)
    else:
        seq_lens = torch.as_tensor(seq_lens, dtype=torch.int32).to(dev)
    pos = (seq_lens - 1).clamp(min=0).to(torch.int32)

    w_gate = None
    if wl.gate_std > 0:
        w_gate = randn(Hq, d, std=wl.gate_std)

    return DecodeInputs(wl, q, k_cache, v_cache, k_new, v_new, P, seq_lens, pos,
                        w_gate, plants)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a bf16 tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def default_scale(d):
    return 1.0 / math.sqrt(d)


# ---------------------------------------------------------------- calibration

@dataclass
class AnisoInputs:
    """Keys and queries with per-KV-head anisotropic second moments, for basis
    calibration and selection recall.  Per KV head h a seeded orthonormal
    d x d basis U_h; a key is U_h (sqrt(lk) * z), a query head U_h (sqrt(lq) *
    z'), z, z' ~ N(0, I), lk and lq the spectra below.  Separate draws of the
    same distributions serve as calibration data (cal_q: group-mean queries,
    cal_k: keys) and as the decode step's cache and queries."""
    q: torch.Tensor        # [B, Hq, d] bf16
    K: torch.Tensor        # [B, Hkv, N, d] bf16
    V: torch.Tensor        # [B, Hkv, N, d] bf16
    cal_q: np.ndarray      # [Hkv, n_cal_q, d] float64 group means of calibration queries
    cal_k: np.ndarray      # [Hkv, n_cal_k, d] float64 calibration keys (bf16 values)
    P_random: torch.Tensor # [Hkv, d, r] fp32 seeded orthonormal basis (no calibration)


def aniso_spectra(d):
    """Key energy decays from direction 0; query energy peaks at direction
    40: the directions that carry most key energy are not those the queries
    weigh most, so key-only statistics are not enough."""
    i = np.arange(d, dtype=np.float64)
    return 1.0 / (1.0 + i / 4.0), 1.0 / (1.0 + np.abs(i - 40.0) / 4.0)


def make_aniso_inputs(B=4, Hq=16, Hkv=4, d=128, N=32768, r=32, n_cal_q=512, n_cal_k=16384,
                      seed=0, device="cpu"):
    rng = np.random.default_rng(_seed("aniso", seed))
    lk, lq = aniso_spectra(d)
    G = Hq // Hkv
    U = np.stack([orthonormal_basis(d, d, _seed("aniso-basis", seed, h)) for h in range(Hkv)])

    def draw(shape, lam, h):
        z = rng.standard_normal(shape + (d,)) * np.sqrt(lam)
        return z @ U[h].T

    q = np.zeros((B, Hq, d))
    K = np.zeros((B, Hkv, N, d), dtype=np.float32)
    for h in range(Hkv):
        q[:, h * G:(h + 1) * G] = draw((B, G), lq, h)
        for b in range(B):
            K[b, h] = draw((N,), lk, h)
    V = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    cal_q = np.stack([draw((n_cal_q, G), lq, h).mean(axis=1) for h in range(Hkv)])
    cal_k = np.stack([bf(draw((n_cal_k,), lk, h)).to(torch.float64).numpy()
                      for h in range(Hkv)])
    P = np.stack([orthonormal_basis(d, r, _seed("aniso-P", seed, h)) for h in range(Hkv)])
    return AnisoInputs(q=bf(q).to(device), K=bf(K).to(device), V=bf(V).to(device),
                       cal_q=cal_q, cal_k=cal_k,
                       P_random=torch.from_numpy(np.ascontiguousarray(P, dtype=np.float32))
                       .to(device))
