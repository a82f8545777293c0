"""Seeded synthetic inputs for the codec's tests and benchmark.

This module only makes data: it holds none of the codec's arithmetic, and both the GPU
tests and the CPU oracle tests draw their inputs from it.  Every generator is
deterministic for a given seed and size.  Random numbers come from
``numpy.random.default_rng(seed)`` in the draw order written below; the smooth fields are
computed in float64 (numpy or torch, on the requested device) and cast to float32 at the
end.  The five workloads stand in for the wavefield snapshots a Devito-style solver would
compress ("DevitoComp provider interface": TimeFunction compression); no public dataset is
involved.
"""
from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------------------
# Workload table: name -> dims, options string builder, description.
# ---------------------------------------------------------------------------------------


def _fmt(v: float) -> str:
    return "%.17g" % v


def c1_sines(n: int = 1 << 20, seed: int = 0):
    """1-D sum of four sines (periods 97/1013/4099/65537, amplitudes 1/0.5/0.25/0.1) plus
    N(0, 1e-3) noise.  Absolute bound 1e-3 * (max - min); block 32; outlier_log2 15."""
    i = np.arange(n, dtype=np.float64)
    rng = np.random.default_rng(seed)
    x = (np.sin(2 * np.pi * i / 97) + 0.5 * np.sin(2 * np.pi * i / 1013)
         + 0.25 * np.sin(2 * np.pi * i / 4099) + 0.1 * np.sin(2 * np.pi * i / 65537)
         + rng.normal(0.0, 1e-3, n))
    x = x.astype(np.float32)
    eb = 1e-3 * (float(x.max()) - float(x.min()))
    return x, [n], f"abs={_fmt(eb)};block=32;outlier_log2=15"


def grf(shape, alpha: float, seed: int, device: str = "cpu"):
    """Gaussian random field: white noise filtered by |k|^(-alpha/2) in amplitude (power
    spectrum k^-alpha), integer wavenumbers, k = 0 removed, normalised to zero mean and unit
    std.  Noise drawn with numpy; the FFTs run in torch float64 on `device`."""
    import torch

    rng = np.random.default_rng(seed)
    w = rng.standard_normal(shape)
    wt = torch.from_numpy(w).to(device)
    del w
    W = torch.fft.rfftn(wt)
    del wt
    k2 = None
    for ax, nax in enumerate(shape):
        if ax == len(shape) - 1:
            k = torch.fft.rfftfreq(nax, d=1.0 / nax, dtype=torch.float64, device=device)
        else:
            k = torch.fft.fftfreq(nax, d=1.0 / nax, dtype=torch.float64, device=device)
        view = [1] * len(shape)
        view[ax] = k.numel()
        kk = (k * k).reshape(view)
        k2 = kk if k2 is None else k2 + kk
    amp = torch.where(k2 > 0, k2.clamp_min(1e-300) ** (-alpha / 4.0), torch.zeros_like(k2))
    W = W * amp
    del amp, k2
    f = torch.fft.irfftn(W, s=list(shape))
    del W
    f = (f - f.mean()) / f.std(unbiased=False)
    return f.to(torch.float32).reshape(-1)


def c2_grf2d(N: int = 4096, seed: int = 1, device: str = "cpu"):
    """2-D N x N Gaussian random field with a k^-3 spectrum.  Relative bound 1e-2; block 128;
    outlier_log2 15."""
    x = grf((N, N), 3.0, seed, device)
    return x, [N, N], "rel=1e-2;block=128;outlier_log2=15"


def c3_ricker(N: int = 512, seed: int = 2, device: str = "cpu"):
    """3-D N^3 wavefield snapshot: eight spherical Ricker wavelets of peak wavelength 15 cells
    with random centres, radii and signed amplitudes, and the slowest-axis planes at or past
    ceil(0.6 N) set to zero (a quiescent region).  Relative bound 1e-3; block 256;
    outlier_log2 15.  Draw order: centres along the slowest axis U(0, 0.6N), then the two
    other axes U(0, N), amplitudes U(0.5, 1.5) times random signs, radii U(0.1N, 0.5N)."""
    import torch

    rng = np.random.default_rng(seed)
    p0 = rng.uniform(0, 0.6 * N, 8)
    p1 = rng.uniform(0, N, 8)
    p2 = rng.uniform(0, N, 8)
    amp = rng.uniform(0.5, 1.5, 8) * rng.choice([-1.0, 1.0], 8)
    rad = rng.uniform(0.1 * N, 0.5 * N, 8)
    lam = 15.0
    g = torch.arange(N, dtype=torch.float64, device=device)
    u = torch.zeros((N, N, N), dtype=torch.float64, device=device)
    for s in range(8):
        d0 = (g - p0[s]) ** 2
        d1 = (g - p1[s]) ** 2
        d2 = (g - p2[s]) ** 2
        r = torch.sqrt(d0[:, None, None] + d1[None, :, None] + d2[None, None, :])
        a = (math.pi * (r - rad[s]) / lam) ** 2
        del r
        u += amp[s] * (1 - 2 * a) * torch.exp(-a)
        del a
    z0 = int(math.ceil(0.6 * N))
    u[z0:] = 0
    return u.to(torch.float32).reshape(-1), [N, N, N], "rel=1e-3;block=256;outlier_log2=15"


def c4_ar1_spikes(n: int = 1 << 28, seed: int = 3, side_max: int = 1 << 23):
    """1-D smooth AR(1) signal (phi 0.999, innovations N(0, 1e-2)) with 1 % of the indices
    replaced by spikes uniform in +-1e4 * R, R the signal's range before the spikes.
    Absolute bound 1e-4 * R; block 128; outlier_log2 15; side list capacity side_max."""
    from scipy.signal import lfilter

    rng = np.random.default_rng(seed)
    e = rng.normal(0.0, 1e-2, n)
    x = lfilter([1.0], [1.0, -0.999], e).astype(np.float32)
    del e
    R = float(x.max()) - float(x.min())
    idx = rng.choice(n, n // 100, replace=False)
    x[idx] = rng.uniform(-1e4 * R, 1e4 * R, idx.size).astype(np.float32)
    eb = 1e-4 * R
    return x, [n], f"abs={_fmt(eb)};block=128;outlier_log2=15;side_max={side_max}"


def c5_snapshot(i: int, N: int = 256, rel: float = 1e-6, device: str = "cpu"):
    """Snapshot i of the 64-snapshot batch: an N^3 Gaussian random field with a k^-2
    spectrum, seed 100 + i.  Relative bound 1e-6 or 1e-2; block 256; outlier_log2 30."""
    x = grf((N, N, N), 2.0, 100 + i, device)
    return x, [N, N, N], f"rel={_fmt(rel)};block=256;outlier_log2=30"


def largest_field(n: int, device: str = "cpu", piece: int = 1 << 27):
    """A 1-D field of n values, up to the largest a plan takes (just under 2^32), for the
    maximum-size test: sines of periods 8191 and 65521 (amplitudes 1 and 0.5) and 0.01 sin(0.7 i),
    computed in float64 from each value's index and cast to float32, with +-1e30 (values that
    escape) at indices 3, 2^31 - 1, 2^31, 2^31 + 7, n - 2 and n - 1 (those below n).  Built on
    `device` (a torch device) in pieces of `piece` values; no random draws."""
    import torch

    x = torch.empty(n, dtype=torch.float32, device=device)
    for a in range(0, n, piece):
        b = min(n, a + piece)
        i = torch.arange(a, b, dtype=torch.int64, device=device)
        v = torch.sin((i % 8191).to(torch.float64) * (2 * math.pi / 8191))
        v += 0.5 * torch.sin((i % 65521).to(torch.float64) * (2 * math.pi / 65521))
        v += 0.01 * torch.sin(i.to(torch.float64) * 0.7)
        x[a:b] = v.to(torch.float32)
        del i, v
    for k, idx in enumerate([3, (1 << 31) - 1, 1 << 31, (1 << 31) + 7, n - 2, n - 1]):
        if 0 <= idx < n:
            x[idx] = 1e30 if k % 2 == 0 else -1e30
    return x


# ---------------------------------------------------------------------------------------
# Small adversarial inputs for fuzzing (tiny n, every special value).
# ---------------------------------------------------------------------------------------

SPECIALS = np.array([np.nan, np.inf, -np.inf, -0.0, 0.0, 1e-45, -1e-45, 1.17549435e-38,
                     3.4028235e38, -3.4028235e38, 1e30, -1e30], dtype=np.float32)


def tiny_array(rng: np.random.Generator, n: int, kind: str) -> np.ndarray:
    """kind: 'smooth' (random walk), 'normal', 'specials' (normal with special values mixed
    in), 'bits' (random bit patterns), 'const', 'ramp', 'subnormal'."""
    if kind == "smooth":
        x = np.cumsum(rng.normal(0, 1, n))
    elif kind == "normal":
        x = rng.normal(0, 10, n)
    elif kind == "specials":
        x = rng.normal(0, 1, n)
        k = max(1, n // 10)
        pos = rng.integers(0, n, k)
        x = x.astype(np.float32)
        x[pos] = rng.choice(SPECIALS, k)
        return x
    elif kind == "bits":
        return rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    elif kind == "const":
        x = np.full(n, rng.normal())
    elif kind == "ramp":
        x = np.arange(n) * rng.uniform(0.1, 3)
    elif kind == "subnormal":
        return (rng.normal(0, 1, n) * 1e-40).astype(np.float32)
    else:
        raise ValueError(kind)
    return x.astype(np.float32)


def adversarial(rng: np.random.Generator, n: int, eb: float, s: float, T: int) -> np.ndarray:
    """n float32 values placed where a quantizer with bound eb and step s = 2 eb must decide
    carefully: on cell boundaries (k + 1/2) s, on grid points k s, at +-eb itself and within a
    millionth of it (codes +-1 next to the bound), around the code limit 2^T (k = 2^T - 1, 2^T
    and the boundary between them), small normal values, and special values (NaN, +-Inf, -0,
    subnormals, values whose rounded code passes 2^30); each then nudged by 0, 1 or 2 ulps up
    or down.  Codes stay mostly below min(2^T, 2^14) so that the field is coded rather than copied raw.
    eb and s are taken as given (the caller resolves them); nothing here quantizes."""
    f32 = np.float32
    kmax = float(1 << min(T, 14))
    # |k| log-uniform in [1, kmax), random sign
    k = np.floor(np.exp(rng.uniform(0.0, np.log(kmax), n))) * rng.choice([-1.0, 1.0], n)
    kind = rng.choice(8, n, p=[0.22, 0.18, 0.16, 0.16, 0.12, 0.06, 0.05, 0.05])
    sgn = rng.choice([-1.0, 1.0], n)
    v = np.zeros(n, np.float64)
    v[kind == 0] = ((k + 0.5) * s)[kind == 0]
    v[kind == 1] = (sgn * eb * (1.0 + rng.uniform(-1e-6, 1e-6, n)))[kind == 1]
    v[kind == 2] = (k * s)[kind == 2]
    v[kind == 3] = (rng.normal(0.0, 10.0, n) * s)[kind == 3]
    v[kind == 4] = (sgn * eb)[kind == 4]
    lim = float(1 << T)
    edge = rng.choice([lim - 1.0, lim - 0.5, lim, lim + 0.5], n)
    v[kind == 5] = (sgn * edge * s)[kind == 5]
    v[kind == 6] = (k * s + rng.uniform(-1.0, 1.0, n) * eb)[kind == 6]
    x = v.astype(f32)
    sp = kind == 7
    x[sp] = rng.choice(SPECIALS, int(sp.sum()))
    # ulp nudges (FLT_MAX may step to infinity)
    steps = rng.integers(-2, 3, n)
    with np.errstate(over="ignore"):
        for _ in range(2):
            up = steps > 0
            dn = steps < 0
            x[up] = np.nextafter(x[up], f32(np.inf))
            x[dn] = np.nextafter(x[dn], f32(-np.inf))
            steps = steps - np.sign(steps)
    return x.astype(f32)
