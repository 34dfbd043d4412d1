"""Seeded synthetic inputs for the query-free KV-cache eviction step.

This module only draws random K/V rows and filter directions.  It holds none of
the eviction method's arithmetic (no scoring, ranking or compaction), so that the
CPU oracle and the HIP path can both consume the very same bytes.

Workloads (head_dim D = 128 unless a variant sets ``Config.D``; groups
g = (l*B + b)*H + h):

* ``c1`` -- one layer, one KV head, fp32 K/V ~ N(0, 1); one 1024-token block,
  budget 512, 4 sinks, no recent window, L2 norm keep-low.
* ``c2`` -- 28 layers x 8 KV heads, batch 1, bf16; one 4096-token block,
  budget 512, 4 sinks; anisotropic keys ``drift * mu_{l,h} + N(0, 0.5^2)`` with a
  planted unit direction ``mu_{l,h}`` and ``drift ~ U(0.5, 2)`` per token; the
  filter is ``mu_{l,h}``, sign +1.
* ``c3`` -- decode stream: 32 sequences x 28 layers x 8 KV heads, bf16; a
  2048-token prefill fills the cache to its budget of 2048, then 256 steps of one
  token; L2 norm keep-low, 4 sinks, recent window 512; keys ``r * u`` with ``u``
  uniform on the sphere and ``ln r ~ N(0, 0.5^2)``.
* ``c4`` -- chunked long prefill: c2's keys, 32768 tokens in 4096-token chunks,
  budget 4096, 4 sinks; two scorer runs: L2 keep-low, and projection on ``mu``
  with sign -1.
* ``c5`` -- 32 layers x 8 KV heads, bf16, c2's keys; 131072 tokens in 8192-token
  chunks, budget 8192, 4 sinks, sign +1; the filter of each group is estimated
  from the group's first 128 keys (key-SVD fallback) and then frozen.

Every array is drawn from numpy's PCG64 seeded with
``SeedSequence([config_id, layer, batch, head, chunk, tag])`` (tag 0 = K noise /
direction, 1 = V, 2 = mu, 3 = drift, 4 = log-norm), so any (group, chunk) can be
regenerated on its own.  bf16 values are rounded to nearest-even from float32
and carried as raw ``uint16`` bits.

``fill_device`` produces the same recipe at full size directly on the GPU with
torch's seeded generator (different draws, same distributions), then overwrites
a chosen sample of groups with the exact host bytes, so that the sampled groups
can be checked against the oracle while the rest keep the launch at full size.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

D = 128
TAG_K, TAG_V, TAG_MU, TAG_DRIFT, TAG_LOGNORM = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Scorer:
    mode: str          # "l2" or "proj"
    keep: str = "high"  # "low" / "high" (projection is always keep-high)
    sign: int = 1
    filt: str = ""     # "mu" (planted direction) or "keysvd" (fallback estimate)


@dataclasses.dataclass(frozen=True)
class Config:
    cid: int
    name: str
    L: int
    B: int
    H: int
    dtype: str                  # "f32", "bf16" or "f16"
    keys: str                   # "gauss", "aniso", "lognorm"
    chunks: Tuple[int, ...]     # incoming rows per call, in order
    budget: int
    n_sink: int
    recent: int
    scorers: Tuple[Scorer, ...]
    calib_tokens: int = 0
    calib_keys: str = "crossing"   # fallback estimate from the whole crossing block, or the "first" calib_tokens
    D: int = 128                   # head dim (64, 128 or 256)

    @property
    def G(self) -> int:
        return self.L * self.B * self.H

    @property
    def tokens(self) -> int:
        return int(sum(self.chunks))

    def group_lbh(self, g: int) -> Tuple[int, int, int]:
        h = g % self.H
        b = (g // self.H) % self.B
        l = g // (self.H * self.B)
        return l, b, h


CONFIGS = {
    1: Config(1, "c1_single_head_fp32", 1, 1, 1, "f32", "gauss", (1024,), 512, 4, 0,
              (Scorer("l2", "low"),)),
    2: Config(2, "c2_qfilters_calibrated", 28, 1, 8, "bf16", "aniso", (4096,), 512, 4, 0,
              (Scorer("proj", "high", +1, "mu"),)),
    3: Config(3, "c3_decode_stream", 28, 32, 8, "bf16", "lognorm", (2048,) + (1,) * 256,
              2048, 4, 512, (Scorer("l2", "low"),)),
    4: Config(4, "c4_chunked_prefill_32k", 28, 1, 8, "bf16", "aniso", (4096,) * 8, 4096, 4, 0,
              (Scorer("l2", "low"), Scorer("proj", "high", -1, "mu"))),
    5: Config(5, "c5_keysvd_fallback_128k", 32, 1, 8, "bf16", "aniso", (8192,) * 16, 8192, 4, 0,
              (Scorer("proj", "high", +1, "keysvd"),), calib_tokens=128, calib_keys="first"),
}


def _rng(cid: int, l: int, b: int, h: int, chunk: int, tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cid, l, b, h, chunk, tag])))


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns raw uint16 bits.

    Uses torch's CPU conversion (vectorised); ``bf16_bits_from_f32_np`` is the
    plain numpy definition the tests hold it to."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_from_f32_np(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16 bits, written out in numpy (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE binary16 (nearest, ties to even); raw uint16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def bits_to_f32(b: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 values of stored rows (float32, bf16 bits or f16 bits)."""
    if dtype == "f32":
        return np.asarray(b, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)
    return bf16_bits_to_f32(b)


def planted_mu(cfg: Config, l: int, h: int) -> np.ndarray:
    """Unit direction mu_{l,h} (float64) planted in the anisotropic key recipe."""
    m = _rng(cfg.cid, l, 0, h, 0, TAG_MU).standard_normal(cfg.D)
    return m / np.linalg.norm(m)


def filters_mu(cfg: Config) -> np.ndarray:
    """[L, H, D] float32 filters equal to the planted directions."""
    out = np.empty((cfg.L, cfg.H, cfg.D), dtype=np.float32)
    for l in range(cfg.L):
        for h in range(cfg.H):
            out[l, h] = planted_mu(cfg, l, h).astype(np.float32)
    return out


def _keys_f32(cfg: Config, g: int, chunk: int, S: int) -> np.ndarray:
    l, b, h = cfg.group_lbh(g)
    if cfg.keys == "gauss":
        return _rng(cfg.cid, l, b, h, chunk, TAG_K).standard_normal((S, cfg.D), dtype=np.float32)
    if cfg.keys == "aniso":
        mu = planted_mu(cfg, l, h)
        drift = _rng(cfg.cid, l, b, h, chunk, TAG_DRIFT).uniform(0.5, 2.0, S)
        noise = _rng(cfg.cid, l, b, h, chunk, TAG_K).standard_normal((S, cfg.D), dtype=np.float32)
        return (drift[:, None] * mu[None, :] + 0.5 * noise.astype(np.float64)).astype(np.float32)
    if cfg.keys == "lognorm":
        u = _rng(cfg.cid, l, b, h, chunk, TAG_K).standard_normal((S, cfg.D))
        u /= np.linalg.norm(u, axis=1, keepdims=True)
        r = np.exp(0.5 * _rng(cfg.cid, l, b, h, chunk, TAG_LOGNORM).standard_normal(S))
        return (r[:, None] * u).astype(np.float32)
    raise ValueError(cfg.keys)


def _values_f32(cfg: Config, g: int, chunk: int, S: int) -> np.ndarray:
    l, b, h = cfg.group_lbh(g)
    return _rng(cfg.cid, l, b, h, chunk, TAG_V).standard_normal((S, cfg.D), dtype=np.float32)


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> stored row bytes of `dtype` (float32, bf16 or f16 bits)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return f16_bits_from_f32(x)
    return bf16_bits_from_f32(x)


def _encode(cfg: Config, x: np.ndarray) -> np.ndarray:
    return encode(x, cfg.dtype)


def group_chunk(cfg: Config, g: int, chunk: int) -> Tuple[np.ndarray, np.ndarray]:
    """Exact host bytes of (K, V) for one group and one chunk: [S, D] uint16 (bf16) or float32."""
    S = cfg.chunks[chunk]
    return _encode(cfg, _keys_f32(cfg, g, chunk, S)), _encode(cfg, _values_f32(cfg, g, chunk, S))


def group_stream(cfg: Config, g: int, n_chunks: Optional[int] = None) -> List[Tuple[np.ndarray, np.ndarray]]:
    n = len(cfg.chunks) if n_chunks is None else n_chunks
    if cfg.cid == 3 and n > 1:
        # The 256 single-token decode steps of a group are drawn as one block
        # (chunk index 1) and handed out row by row.
        K0, V0 = group_chunk(cfg, g, 0)
        Kd = _encode(cfg, _keys_f32(cfg, g, 1, 256))
        Vd = _encode(cfg, _values_f32(cfg, g, 1, 256))
        out = [(K0, V0)] + [(Kd[i:i + 1], Vd[i:i + 1]) for i in range(256)]
        return out[:n]
    return [group_chunk(cfg, g, c) for c in range(n)]


def decode_block(cfg: Config, g: int) -> Tuple[np.ndarray, np.ndarray]:
    """The decode workload's 256 single-token steps of group g as one [256, D] block."""
    return _encode(cfg, _keys_f32(cfg, g, 1, 256)), _encode(cfg, _values_f32(cfg, g, 1, 256))


def batch_chunk(cfg: Config, groups: Sequence[int], chunk: int, workers: int = 16) -> Tuple[np.ndarray, np.ndarray]:
    """Stacked exact host bytes [len(groups), S, D] for one chunk (groups drawn on
    a thread pool; every group has its own generator, so the bytes do not depend
    on the pool)."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max(1, min(workers, len(groups)))) as ex:
        ks, vs = zip(*ex.map(lambda g: group_chunk(cfg, g, chunk), groups))
    return np.stack(ks), np.stack(vs)


def custom_keys(shape: Tuple[int, ...], seed: int, dtype: str = "bf16", scale: float = 1.0,
                kind: str = "gauss") -> np.ndarray:
    """Seeded keys for edge-case tests.  ``kind``: "gauss", "int" (small integers,
    exact in bf16/fp32 so sums are exact), "dup" (heavy exact duplicates)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([9999, seed])))
    if kind == "gauss":
        x = (scale * rng.standard_normal(shape)).astype(np.float32)
    elif kind == "int":
        x = rng.integers(-8, 9, size=shape).astype(np.float32)
    elif kind == "dup":
        base = rng.integers(-2, 3, size=(4,) + tuple(shape[-1:])).astype(np.float32)
        pick = rng.integers(0, 4, size=shape[:-1])
        x = base[pick]
    else:
        raise ValueError(kind)
    return encode(x, dtype)


# ----------------------------------------------------------------------------
# Query activations for calibration (synthetic stand-in for the pages' 20 x
# 2048-token calibration text, about 3000 samples per head)
# ----------------------------------------------------------------------------

def _query_head_dir(l: int, h: int, r: int, D: int, seed: int):
    """(mu_h, generator for head h's rows) of query_acts."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([5150, seed, l, h // r])))
    mu = g.standard_normal(D)
    mu /= np.linalg.norm(mu)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([5151, seed, l, h])))
    m = mu + 0.25 * rng.standard_normal(D) / np.sqrt(D)
    return m / np.linalg.norm(m), rng


def query_acts(L: int, H_q: int, H_kv: int, N: int, D: int = 128, seed: int = 0, dtype: str = "bf16",
               workers: int = 16) -> np.ndarray:
    """[L, H_q, N, D] activations: query head h of layer l (KV head j = h // (H_q/H_kv))
    has rows drift * mu_h + N(0, 0.5^2), drift ~ U(0.5, 2), with mu_h the unit
    normalisation of mu_{l,j} + 0.25 xi_h (mu_{l,j} unit, xi_h ~ N(0, I/D)): heads
    sharing a KV head lean the same way."""
    from concurrent.futures import ThreadPoolExecutor
    r = H_q // H_kv

    def one(lh):
        m, rng = _query_head_dir(lh[0], lh[1], r, D, seed)
        drift = rng.uniform(0.5, 2.0, (N, 1))
        return encode((drift * m + 0.5 * rng.standard_normal((N, D))).astype(np.float32), dtype)

    heads = [(l, h) for l in range(L) for h in range(H_q)]
    with ThreadPoolExecutor(max(1, min(workers, len(heads)))) as ex:
        rows = list(ex.map(one, heads))
    return np.stack(rows).reshape(L, H_q, N, D)


def query_head_mu(L: int, H_q: int, H_kv: int, D: int = 128, seed: int = 0) -> np.ndarray:
    """[L, H_q, D] the planted per-head directions mu_h of query_acts."""
    return np.stack([np.stack([_query_head_dir(l, h, H_q // H_kv, D, seed)[0] for h in range(H_q)])
                     for l in range(L)])


def query_acts_device(L: int, H_q: int, H_kv: int, N: int, D: int = 128, seed: int = 0, device="cuda"):
    """query_acts' recipe drawn on the device with torch's seeded generator
    (bf16 [L, H_q, N, D]; not the same bytes as query_acts)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    r = H_q // H_kv
    mu = torch.randn((L, H_kv, 1, D), generator=gen, device=device)
    mu = mu / mu.norm(dim=-1, keepdim=True)
    m = mu.repeat_interleave(r, dim=1) + 0.25 * torch.randn((L, H_q, 1, D), generator=gen, device=device) / D ** 0.5
    m = m / m.norm(dim=-1, keepdim=True)
    drift = torch.rand((L, H_q, N, 1), generator=gen, device=device) * 1.5 + 0.5
    q = torch.randn((L, H_q, N, D), generator=gen, device=device).mul_(0.5).add_(drift * m)
    return q.to(torch.bfloat16)


# ----------------------------------------------------------------------------
# Full-size device inputs (torch is only plumbing here)
# ----------------------------------------------------------------------------

def fill_device(cfg: Config, rows: int, seed: int, device="cuda", exact=None, mus=None):
    """Return device tensors (K, V) of shape [G, rows, cfg.D] following ``cfg``'s
    recipe with torch's seeded generator.  ``exact`` maps group -> host (K, V)
    [rows, D] arrays (from ``group_chunk`` / ``group_stream``) that overwrite
    those groups, so that they carry the exact bytes the oracle sees.

    bf16 tensors are returned as torch.bfloat16, f16 as torch.float16, fp32 as
    torch.float32."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    G, D_ = cfg.G, cfg.D
    if cfg.keys == "gauss":
        k = torch.randn((G, rows, D_), generator=gen, device=device, dtype=torch.float32)
    elif cfg.keys == "aniso":
        if mus is None:
            mus = device_mus(cfg, device)
        drift = torch.rand((G, rows, 1), generator=gen, device=device) * 1.5 + 0.5
        k = torch.randn((G, rows, D_), generator=gen, device=device, dtype=torch.float32)
        k.mul_(0.5).add_(drift * mus[:, None, :])
    elif cfg.keys == "lognorm":
        k = torch.randn((G, rows, D_), generator=gen, device=device, dtype=torch.float32)
        k.div_(k.norm(dim=2, keepdim=True))
        r = torch.exp(0.5 * torch.randn((G, rows, 1), generator=gen, device=device))
        k.mul_(r)
    else:
        raise ValueError(cfg.keys)
    v = torch.randn((G, rows, D_), generator=gen, device=device, dtype=torch.float32)
    if cfg.dtype in ("bf16", "f16"):
        td = torch.bfloat16 if cfg.dtype == "bf16" else torch.float16
        k = k.to(td)
        v = v.to(td)
    for g, (Kh, Vh) in (exact or {}).items():
        k[g].copy_(host_to_torch(Kh, cfg.dtype))
        v[g].copy_(host_to_torch(Vh, cfg.dtype))
    return k, v


def device_mus(cfg: Config, device="cuda"):
    """[G, D] float32 planted direction of each group (device tensor)."""
    import torch
    return torch.from_numpy(np.stack([planted_mu(cfg, *cfg.group_lbh(g)[::2])
                                      for g in range(cfg.G)]).astype(np.float32)).to(device)


def host_to_torch(x: np.ndarray, dtype: str):
    """Wrap host bytes as a CPU torch tensor of the matching element type (no value change)."""
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t16 = torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint16).view(np.int16))
    return t16.view(torch.float16 if dtype == "f16" else torch.bfloat16)


def torch_to_host(t, dtype: str) -> np.ndarray:
    import torch
    t = t.detach().cpu().contiguous()
    if dtype == "f32":
        return t.numpy().astype(np.float32, copy=False)
    return t.view(torch.int16).numpy().view(np.uint16)


def sample_groups(cfg: Config, n: int, seed: int = 0) -> List[int]:
    """A fixed, spread-out sample of group indices (always includes the first and last)."""
    if n >= cfg.G:
        return list(range(cfg.G))
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([7777, cfg.cid, seed])))
    mid = rng.choice(np.arange(1, cfg.G - 1), size=max(0, n - 2), replace=False)
    return sorted({0, cfg.G - 1, *map(int, mid)})
