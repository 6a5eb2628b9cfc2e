"""Seeded synthetic KV workloads (stand-ins for model-produced caches).

The pages measure on caches of SmolLM2-1.7B, Llama-3-8B and Llama-3.1-8B run
over GSM8K / WikiText-2-like text (QKVShare results; PolyKV section 4). Neither
models nor datasets are used here: these generators copy only the cache
shapes and a value structure (heavy tails, outlier channels, an attention
sink, width runs) and are the single source of inputs for both the CPU
oracle and the GPU library. No codec arithmetic lives here.

Randomness: numpy PCG64 seeded from SeedSequence([seed, cfg, tensor, layer]),
tensor 0 = K, 1 = V, 2 = structure / widths; values are drawn per layer in
float32 and rounded to bf16 (nearest, ties to even). bf16 tensors are numpy
uint16 arrays of raw bit patterns, shape [L, H, T, d].
"""

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

K_TENSOR, V_TENSOR, STRUCT_TENSOR, ANCHOR_TENSOR = 0, 1, 2, 3


@dataclass(frozen=True)
class Workload:
    cfg: int            # workload number, part of every seed
    name: str
    L: int
    H: int
    T: int
    d: int
    recipe: str         # value distribution, see layer_values()
    mode: str           # "pool" or "card"
    agents: int = 1     # decode fan-out

    @property
    def shape(self):
        return (self.L, self.H, self.T, self.d)


WORKLOADS = {
    1: Workload(1, "tiny-1x4x256x64", 1, 4, 256, 64, "normal_two_channels_x8", "pool"),
    2: Workload(2, "smollm2-1.7b-2k", 24, 32, 2048, 64, "normal_outliers_x20_sink_x50", "pool"),
    3: Workload(3, "llama3-8b-gqa-4k", 32, 8, 4096, 128, "student_t5_lognormal_channels", "pool",
                agents=15),
    4: Workload(4, "llama3.1-8b-cachecard-8k", 32, 8, 8192, 128, "normal", "card"),
    5: Workload(5, "llama3-8b-long-32k", 32, 8, 32768, 128, "normal_outliers_x20", "pool"),
}


def rng(seed, cfg, tensor, layer):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg, tensor, layer])))


def f32_to_bf16_bits(x, out=None, chunk=1 << 20):
    """float32 array -> bf16 bit patterns, round to nearest, ties to even.

    Works in chunks with one reused scratch buffer (large fresh temporaries
    are slow to fault in on some hosts)."""
    x = np.ascontiguousarray(x, np.float32)
    u = x.reshape(-1).view(np.uint32)
    res = np.empty(x.shape, np.uint16) if out is None else out
    r = res.reshape(-1)
    tmp = np.empty(min(chunk, u.size), np.uint32)
    acc = np.empty(min(chunk, u.size), np.uint32)
    for i in range(0, u.size, chunk):
        n = min(chunk, u.size - i)
        a, t = acc[:n], tmp[:n]
        np.right_shift(u[i:i + n], 16, out=t)
        np.bitwise_and(t, 1, out=t)
        np.add(u[i:i + n], 0x7FFF, out=a)
        np.add(a, t, out=a)
        np.right_shift(a, 16, out=a)
        r[i:i + n] = a
    return res


def bf16_bits_to_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def layer_values(recipe, seed, cfg, tensor, layer, H, T, d):
    """float32 [H, T, d] values of one layer of one tensor."""
    g = rng(seed, cfg, tensor, layer)
    if recipe == "normal":
        return g.standard_normal((H, T, d), dtype=np.float32)
    if recipe == "normal_two_channels_x8":
        x = g.standard_normal((H, T, d), dtype=np.float32)
        s = rng(seed, cfg, STRUCT_TENSOR, 1000 + tensor)
        ch = s.choice(d, size=2, replace=False)
        x[:, :, ch] *= np.float32(8.0)
        return x
    if recipe in ("normal_outliers_x20", "normal_outliers_x20_sink_x50"):
        x = g.standard_normal((H, T, d), dtype=np.float32)
        s = rng(seed, cfg, STRUCT_TENSOR, 1000 * (tensor + 1) + layer)
        n_out = int(round(0.02 * H * d))
        flat = s.choice(H * d, size=n_out, replace=False)
        x[flat // d, :, flat % d] *= np.float32(20.0)
        if recipe.endswith("sink_x50"):
            x[:, 0, :] *= np.float32(50.0)
        return x
    if recipe == "student_t5_lognormal_channels":
        x = g.standard_t(5.0, size=(H, T, d)).astype(np.float32)
        s = rng(seed, cfg, STRUCT_TENSOR, 1000 * (tensor + 1) + layer)
        scale = np.exp(0.5 * s.standard_normal((H, 1, d))).astype(np.float32)
        return x * scale
    raise ValueError(f"unknown recipe {recipe}")


def tensor_bits(w, seed, tensor, shape=None, layers=None, threads=8):
    """bf16 bits [L', H, T, d] of one tensor (K or V) of a workload.

    shape overrides the workload's (L, H, T, d) (same recipe, smaller size);
    layers selects a subset of layer indices (default: all)."""
    L, H, T, d = shape if shape is not None else w.shape
    layers = list(range(L)) if layers is None else list(layers)
    out = np.empty((len(layers), H, T, d), np.uint16)

    def one(i):
        f32_to_bf16_bits(layer_values(w.recipe, seed, w.cfg, tensor, layers[i], H, T, d), out=out[i])

    if len(layers) > 1 and threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(len(layers))))
    else:
        for i in range(len(layers)):
            one(i)
    return out


def kv_bits(w, seed=0, shape=None, layers=None, threads=8):
    """(K, V) bf16 bits of a workload."""
    return (tensor_bits(w, seed, K_TENSOR, shape, layers, threads),
            tensor_bits(w, seed, V_TENSOR, shape, layers, threads))


WIDTHS = np.array([2, 4, 8, 16], np.uint8)
WIDTH_PROBS = np.array([0.4, 0.3, 0.2, 0.1])


def card_widths(w, seed=0, T=None, mean_run=16.0):
    """Per-token widths in {2, 4, 8, 16}: runs of geometric length (mean
    `mean_run`), each run's width drawn with probabilities .4/.3/.2/.1."""
    T = w.T if T is None else T
    g = rng(seed, w.cfg, STRUCT_TENSOR, 0)
    out = np.empty(T, np.uint8)
    t = 0
    while t < T:
        n = int(g.geometric(1.0 / mean_run))
        out[t:t + n] = g.choice(WIDTHS, p=WIDTH_PROBS)
        t += n
    return out


# Low-rank anchors (KVCMAS stores corrections as truncated-SVD factors, rank
# r = 32 and V = 10 anchors by default). Synthetic factors with the shape of
# an SVD: R has near-orthonormal columns (entries N(0, 1/D)), A's column k
# has scale delta * s_k * sqrt(D) with s_k = decay**k normalised so that
# sum s_k^2 = 1, making every element of A R^T about N(0, delta^2). Weights
# are similarity weights: positive, summing to one (flat Dirichlet).

def anchor_column_scales(r, delta=0.25, decay=0.85):
    s = decay ** np.arange(r, dtype=np.float64)
    return delta * s / np.sqrt(np.sum(s * s))


def anchor_factors(seed, cfg, L, V, T, D, r, delta=0.25, decay=0.85):
    """(A bits [L][V][T][r], R bits [L][V][D][r], weights float32 [L][V])."""
    A = np.empty((L, V, T, r), np.uint16)
    R = np.empty((L, V, D, r), np.uint16)
    w = np.empty((L, V), np.float32)
    col = (anchor_column_scales(r, delta, decay) * np.sqrt(D)).astype(np.float32)
    for l in range(L):
        g = rng(seed, cfg, ANCHOR_TENSOR, l)
        f32_to_bf16_bits(g.standard_normal((V, T, r), dtype=np.float32) * col, out=A[l])
        f32_to_bf16_bits(g.standard_normal((V, D, r), dtype=np.float32) / np.float32(np.sqrt(D)), out=R[l])
        w[l] = g.dirichlet(np.ones(V)).astype(np.float32)
    return A, R, w


def lowrank_caches(seed, cfg, L, H, T, d, rank=32, noise=0.02, decay=0.9):
    """bf16 bits [L, H, T, d] whose per-layer T x (H*d) view is a rank-`rank`
    signal (singular profile 3 * decay**k on near-orthonormal directions)
    plus N(0, noise^2) elements: the low effective rank the pages report for
    base caches and delta corrections."""
    D = H * d
    out = np.empty((L, H, T, d), np.uint16)
    for l in range(L):
        g = rng(seed, cfg, ANCHOR_TENSOR, 10000 + l)
        a = g.standard_normal((T, rank)) * (3.0 * decay ** np.arange(rank))
        r = np.linalg.qr(g.standard_normal((D, rank)))[0]
        z = a @ r.T + noise * g.standard_normal((T, D))
        f32_to_bf16_bits(z.reshape(T, H, d).transpose(1, 0, 2).astype(np.float32), out=out[l])
    return out


def sketch(seed, cfg, D, k=48):
    """The Gaussian test matrix of the randomized SVD: float32 [D, k], N(0, 1)."""
    return rng(seed, cfg, ANCHOR_TENSOR, 20000).standard_normal((D, k), dtype=np.float32)


# ------------------------------------------------------------------ on-device
# The same recipes drawn on the GPU with torch's generator (Philox), for the
# large workloads of the benchmark. Values differ from the numpy streams of
# the same seed; whoever checks a result copies the inputs it needs back.

def _torch_seed(seed, cfg, tensor, layer):
    return int(np.random.SeedSequence([seed, cfg, tensor, layer]).generate_state(1, np.uint64)[0] >> np.uint64(1))


def layer_values_torch(recipe, seed, cfg, tensor, layer, H, T, d, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(seed, cfg, tensor, layer))
    gs = torch.Generator(device=device)
    gs.manual_seed(_torch_seed(seed, cfg, STRUCT_TENSOR, 1000 * (tensor + 1) + layer))
    if recipe == "normal":
        return torch.randn((H, T, d), generator=g, device=device)
    if recipe == "normal_two_channels_x8":
        x = torch.randn((H, T, d), generator=g, device=device)
        ch = torch.randperm(d, generator=gs, device=device)[:2]
        x[:, :, ch] *= 8.0
        return x
    if recipe in ("normal_outliers_x20", "normal_outliers_x20_sink_x50"):
        x = torch.randn((H, T, d), generator=g, device=device)
        n_out = int(round(0.02 * H * d))
        flat = torch.randperm(H * d, generator=gs, device=device)[:n_out]
        x[flat // d, :, flat % d] *= 20.0
        if recipe.endswith("sink_x50"):
            x[:, 0, :] *= 50.0
        return x
    if recipe == "student_t5_lognormal_channels":
        z = torch.randn((H, T, d), generator=g, device=device)
        chi2 = torch.zeros((H, T, d), device=device)
        for _ in range(5):
            chi2 += torch.randn((H, T, d), generator=g, device=device) ** 2
        x = z / torch.sqrt(chi2 / 5.0)
        scale = torch.exp(0.5 * torch.randn((H, 1, d), generator=gs, device=device))
        return x * scale
    raise ValueError(f"unknown recipe {recipe}")


def kv_tensors_torch(w, seed=0, device="cuda", shape=None):
    """(K, V) as bf16 torch tensors [L, H, T, d] on `device`."""
    import torch
    L, H, T, d = shape if shape is not None else w.shape
    out = []
    for tensor in (K_TENSOR, V_TENSOR):
        t = torch.empty((L, H, T, d), dtype=torch.bfloat16, device=device)
        for l in range(L):
            t[l] = layer_values_torch(w.recipe, seed, w.cfg, tensor, l, H, T, d, device).to(torch.bfloat16)
        out.append(t)
    return out[0], out[1]


def anchor_factors_torch(seed, cfg, L, V, T, D, r, device="cuda", delta=0.25, decay=0.85):
    """The anchor recipe drawn on `device` with torch's generator: A, R as
    bf16 tensors [L, V, T, r] and [L, V, D, r], weights float32 [L, V]."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(seed, cfg, ANCHOR_TENSOR, 0))
    col = torch.tensor(anchor_column_scales(r, delta, decay) * np.sqrt(D), dtype=torch.float32, device=device)
    A = torch.empty((L, V, T, r), dtype=torch.bfloat16, device=device)
    R = torch.empty((L, V, D, r), dtype=torch.bfloat16, device=device)
    for l in range(L):
        A[l] = (torch.randn((V, T, r), generator=g, device=device) * col).to(torch.bfloat16)
        R[l] = (torch.randn((V, D, r), generator=g, device=device) / float(np.sqrt(D))).to(torch.bfloat16)
    e = -torch.log(torch.rand((L, V), generator=g, device=device).clamp_min(1e-12))
    w = (e / e.sum(dim=1, keepdim=True)).to(torch.float32)
    return A, R, w
