"""Seeded synthetic post-ReLU activation maps.

The workloads stand in for the activation maps of the six ImageNet CNNs that
"Compressing DMA Engine: Leveraging Activation Sparsity for Training Deep
Neural Networks" (Rhu et al., arXiv:1705.01626) studies.  Those maps are not
available here, so the recipes below reproduce what the page says about them:

* §II.B (Training versus Inference): a map is a 4-D array ordered batch,
  channels, height, width (NCHW), stored contiguously.
* §IV (Sparsity of DNN Activations) and §V.A (Compression Algorithm): about
  half to nine tenths of the values are exactly zero; the first conv layer sits
  near 50 %, deeper layers are sparser.
* §V.A: zeros and nonzeros come in clusters (that is what run-length coding
  exploits), which a thresholded, Gaussian-smoothed noise field reproduces.

Three families of generators:

``iid_relu``        zero with probability s, else |N(0,1)|.
``clustered_relu``  per (n, c) plane: Gaussian-smoothed N(0,1) noise, shifted
                    down by the plane's s-quantile and clipped at 0 (a ReLU),
                    so a fraction s of the plane is exactly zero and zeros are
                    spatially clustered.
``sweep_bits_*``    a counter-based integer hash, identical on the host
                    (numpy) and on the GPU (torch), for the 4 GiB sparsity
                    sweep: any window of it can be regenerated on the host
                    without generating the rest.

Everything here is input generation only.
"""

from __future__ import annotations

import math

import numpy as np

_M32 = 0xFFFFFFFF

# Bit patterns that a lossless codec must carry verbatim: negative zero,
# denormals of both signs, NaNs with payloads and infinities.
_SPECIALS32 = np.array(
    [0x80000000, 0x00000001, 0x007FFFFF, 0x80000001,
     0x7FC00000, 0x7F800001, 0xFF800000, 0x7F800000], dtype=np.uint32)
_SPECIALS16 = np.array(
    [0x8000, 0x0001, 0x03FF, 0x8001, 0x7E00, 0x7C01, 0xFC00, 0x7C00],
    dtype=np.uint16)

_CHUNK = 1 << 24


def iid_relu(n: int, zero_frac: float, seed: int, dtype=np.float32) -> np.ndarray:
    """n values: exactly zero with probability ``zero_frac``, else |N(0,1)|.

    A nonzero draw that happens to be exactly 0.0 is replaced by 1.0 so the
    zero fraction is governed by ``zero_frac`` alone.
    """
    out = np.empty(n, dtype=dtype)
    nchunks = max(1, -(-n // _CHUNK))
    children = np.random.SeedSequence(seed).spawn(nchunks)
    for k in range(nchunks):
        lo, hi = k * _CHUNK, min(n, (k + 1) * _CHUNK)
        rng = np.random.default_rng(children[k])
        u = rng.random(hi - lo)
        v = np.abs(rng.standard_normal(hi - lo, dtype=np.float32))
        v[v == 0] = 1.0
        v[u < zero_frac] = 0.0
        out[lo:hi] = v.astype(dtype)
    return out


def _plane_thresholds(g2d: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Per-row linear-interpolated q-quantile of a (rows, m) array."""
    srt = np.sort(g2d, axis=1)
    m = srt.shape[1]
    pos = q * (m - 1)
    lo = np.floor(pos).astype(np.int64)
    hi = np.minimum(lo + 1, m - 1)
    frac = (pos - lo).astype(np.float32)
    a = np.take_along_axis(srt, lo[:, None], axis=1)[:, 0]
    b = np.take_along_axis(srt, hi[:, None], axis=1)[:, 0]
    return a + (b - a) * frac


def clustered_relu(shape, zero_frac, sigma: float, seed: int,
                   dtype=np.float32, channel_frac_range=None) -> np.ndarray:
    """NCHW post-ReLU map whose zeros are spatially clustered.

    ``zero_frac`` is a scalar, or ``None`` with ``channel_frac_range=(lo, hi)``
    to draw one zero fraction per channel from U(lo, hi) (shared across the
    batch).  Per (n, c) plane: g = gaussian_filter(N(0,1) noise, sigma) with
    scipy's defaults (reflect, truncate 4), t = s-quantile of g,
    x = max(g - t, 0) / std(g), computed in float32 then cast to ``dtype``.
    """
    from scipy.ndimage import gaussian_filter

    N, C, H, W = shape
    children = np.random.SeedSequence(seed).spawn(N + 1)
    if zero_frac is None:
        lo, hi = channel_frac_range
        s_c = np.random.default_rng(children[0]).uniform(lo, hi, size=C)
    else:
        s_c = np.full(C, float(zero_frac))
    out = np.empty(shape, dtype=dtype)
    for i in range(N):
        rng = np.random.default_rng(children[i + 1])
        noise = rng.standard_normal((C, H, W), dtype=np.float32)
        g = gaussian_filter(noise, sigma=(0, sigma, sigma), mode="reflect", truncate=4.0)
        g2 = g.reshape(C, H * W)
        t = _plane_thresholds(g2, s_c)
        sd = g2.std(axis=1)
        sd[sd == 0] = 1.0
        x = np.maximum(g2 - t[:, None], 0.0) / sd[:, None]
        out[i] = x.reshape(C, H, W).astype(dtype)
    return out


def inject_specials(x: np.ndarray, frac: float, seed: int) -> np.ndarray:
    """Overwrite about ``frac`` of the positions (in place) with -0.0,
    denormals of both signs, NaN payloads and infinities.  Returns ``x``."""
    flat = x.reshape(-1)
    if flat.dtype.itemsize == 4:
        bits, pool = flat.view(np.uint32), _SPECIALS32
    elif flat.dtype.itemsize == 2:
        bits, pool = flat.view(np.uint16), _SPECIALS16
    else:
        raise ValueError("specials need 16- or 32-bit elements")
    k = int(round(frac * flat.size))
    if k == 0:
        return x
    rng = np.random.default_rng(seed)
    pos = rng.integers(0, flat.size, size=k)
    bits[pos] = pool[rng.integers(0, pool.size, size=k)]
    return x


# ---------------------------------------------------------------------------
# Counter-based sweep generator (host and device produce identical bits)
# ---------------------------------------------------------------------------

SWEEP_ZERO_FRACTIONS = (0.0, 0.25, 0.5, 0.75, 0.9, 0.99, 1.0)
SWEEP_SEEDS = (50, 51, 52, 53, 54, 55, 56)


def _sweep_params(zero_frac: float, seed: int):
    thr = int(round(zero_frac * 2.0 ** 32))
    key = (seed * 0x632BE5AB) & _M32
    forced = 0.0 < zero_frac < 1.0
    return thr, key, forced


def _mix_np(x):
    x = x ^ (x >> np.uint64(16))
    x = (x * np.uint64(0x7FEB352D)) & np.uint64(_M32)
    x = x ^ (x >> np.uint64(15))
    x = (x * np.uint64(0x346CA68B)) & np.uint64(_M32)
    x = x ^ (x >> np.uint64(16))
    return x


def sweep_bits_host(start: int, count: int, zero_frac: float, seed: int) -> np.ndarray:
    """fp32 bit patterns of sweep elements [start, start + count) as uint32.

    Element i: a = mix((i + key) mod 2^32); zero iff mix(a ^ 0x5BD1E995) < thr
    with thr = round(s * 2^32).  For 0 < s < 1 every 32-element group g with
    g % 97 == 0 is forced all-zero and every g % 89 == 1 (not already forced)
    all-nonzero, so fully empty and fully dense groups always occur.  Nonzero
    magnitude: S = sum of the four bytes of mix(a ^ 0x1B873593) (an
    Irwin-Hall approximation of a normal), value = (2|S - 510| + 1) / 256,
    which is exact in fp32 on every platform.
    """
    thr, key, forced = _sweep_params(zero_frac, seed)
    idx = np.arange(start, start + count, dtype=np.uint64)
    a = _mix_np((idx + np.uint64(key)) & np.uint64(_M32))
    zdraw = _mix_np(a ^ np.uint64(0x5BD1E995))
    mdraw = _mix_np(a ^ np.uint64(0x1B873593))
    zero = zdraw < np.uint64(thr) if thr < 2 ** 32 else np.ones(count, dtype=bool)
    if forced:
        g = idx >> np.uint64(5)
        zero = np.where(g % np.uint64(97) == 0, True,
                        np.where(g % np.uint64(89) == 1, False, zero))
    s = ((mdraw & np.uint64(255)) + ((mdraw >> np.uint64(8)) & np.uint64(255))
         + ((mdraw >> np.uint64(16)) & np.uint64(255)) + (mdraw >> np.uint64(24)))
    m = 2 * np.abs(s.astype(np.int64) - 510) + 1
    val = (m.astype(np.float32) * np.float32(1.0 / 256.0)).view(np.uint32)
    return np.where(zero, np.uint32(0), val).astype(np.uint32)


def _mix_t(x):
    x = x ^ (x >> 16)
    x = (x * 0x7FEB352D) & _M32
    x = x ^ (x >> 15)
    x = (x * 0x346CA68B) & _M32
    x = x ^ (x >> 16)
    return x


def sweep_bits_device(n: int, zero_frac: float, seed: int, device="cuda",
                      out=None, chunk: int = 1 << 26):
    """Same bits as :func:`sweep_bits_host` for [0, n), generated with torch
    int64 arithmetic on ``device`` into an int32 tensor (the fp32 bit view).
    All products stay below 2^63, so no platform-dependent overflow occurs."""
    import torch

    thr, key, forced = _sweep_params(zero_frac, seed)
    if out is None:
        out = torch.empty(n, dtype=torch.int32, device=device)
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        idx = torch.arange(lo, hi, dtype=torch.int64, device=device)
        a = _mix_t((idx + key) & _M32)
        zdraw = _mix_t(a ^ 0x5BD1E995)
        mdraw = _mix_t(a ^ 0x1B873593)
        zero = zdraw < thr
        if forced:
            g = idx >> 5
            zero = torch.where(g % 97 == 0, torch.ones_like(zero),
                               torch.where(g % 89 == 1, torch.zeros_like(zero), zero))
        s = (mdraw & 255) + ((mdraw >> 8) & 255) + ((mdraw >> 16) & 255) + (mdraw >> 24)
        m = 2 * (s - 510).abs() + 1
        val = (m.to(torch.float32) * (1.0 / 256.0)).view(torch.int32)
        out[lo:hi] = torch.where(zero, torch.zeros_like(val), val)
        del idx, a, zdraw, mdraw, zero, s, m, val
    return out


# ---------------------------------------------------------------------------
# The named workloads (activation maps shaped like the pages' CNN layers)
# ---------------------------------------------------------------------------

VGG_SHAPES = ((32, 64, 224, 224), (32, 128, 112, 112), (32, 256, 56, 56),
              (32, 512, 28, 28), (32, 512, 14, 14))
VGG_ZERO = (0.35, 0.5, 0.65, 0.8, 0.9)

WORKLOADS = {
    "single_map_fp32_1x64x56x56_s0.5": dict(
        kind="iid", shape=(1, 64, 56, 56), dtype="float32", zero_frac=0.5, seed=1),
    "alexnet_conv1_fp32_128x96x55x55": dict(
        kind="clustered", shape=(128, 96, 55, 55), dtype="float32",
        zero_frac=None, channel_frac_range=(0.3, 0.7), sigma=2.0, seed=2),
    **{
        f"vgg16_layer{k + 1}_fp32_{'x'.join(map(str, VGG_SHAPES[k]))}": dict(
            kind="clustered", shape=VGG_SHAPES[k], dtype="float32",
            zero_frac=VGG_ZERO[k], sigma=2.0, seed=31 + k)
        for k in range(5)
    },
    "fp16_256x256x56x56_s0.6_specials": dict(
        kind="clustered", shape=(256, 256, 56, 56), dtype="float16",
        zero_frac=0.6, sigma=2.0, seed=4, specials=5e-4),
    **{
        f"sweep_fp32_4GiB_s{s}": dict(
            kind="sweep", shape=(1 << 30,), dtype="float32", zero_frac=s, seed=sd)
        for s, sd in zip(SWEEP_ZERO_FRACTIONS, SWEEP_SEEDS)
    },
}


def workload(name: str, scale_n: int | None = None) -> np.ndarray:
    """Generate a named workload on the host (numpy, native dtype).

    ``scale_n`` (clustered/iid only) keeps the recipe but cuts the batch so
    that at most about ``scale_n`` elements are produced, for quick tests.
    """
    spec = WORKLOADS[name]
    dtype = np.dtype(spec["dtype"])
    shape = tuple(spec["shape"])
    if scale_n is not None and spec["kind"] != "sweep":
        per = math.prod(shape[1:])
        shape = (max(1, min(shape[0], scale_n // per)),) + shape[1:]
    if spec["kind"] == "iid":
        x = iid_relu(math.prod(shape), spec["zero_frac"], spec["seed"], dtype).reshape(shape)
    elif spec["kind"] == "clustered":
        x = clustered_relu(shape, spec.get("zero_frac"), spec["sigma"], spec["seed"], dtype,
                           spec.get("channel_frac_range"))
        if spec.get("specials"):
            inject_specials(x, spec["specials"], spec["seed"] + 1000)
    else:
        n = shape[0] if scale_n is None else min(shape[0], scale_n)
        x = sweep_bits_host(0, n, spec["zero_frac"], spec["seed"]).view(np.float32)
    return x


# ---------------------------------------------------------------------------
# Activation layouts (for the layout study)
# ---------------------------------------------------------------------------
#
# The page compares the codecs over three activation layouts without naming
# them (§VII.A); the three common ones for CNN activations are taken: NCHW
# (the maps' own order, §II.B), NHWC and CHWN.  Each entry is the axis order,
# as indices into NCHW.
LAYOUTS = {"NCHW": (0, 1, 2, 3), "NHWC": (0, 2, 3, 1), "CHWN": (1, 2, 3, 0)}


def to_layout(x_nchw: np.ndarray, layout: str) -> np.ndarray:
    """The same values laid out contiguously in ``layout`` (host, numpy)."""
    return np.ascontiguousarray(np.transpose(x_nchw, LAYOUTS[layout]))
