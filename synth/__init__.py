"""Seeded synthetic inputs for block-sparse prefill attention.

This module only draws and lays out input tensors. It holds none of the
method's arithmetic (no block pooling of realised data, no block scores, no
thresholds, no attention): both the CPU oracle and the GPU path consume what it
produces, and neither is imported here.

Workloads follow the five configurations of the FlashPrefill V2 pages' 128K
setting ("The Numbers That Matter", aimodeling.com page; "Why It Matters",
lode.cx page): a Llama-3-8B-shaped layer (32 query heads, 8 KV heads, head
dim 128), post-RoPE Q/K, long causal prefill, optionally a paged varlen batch
with cached prefixes ("Framework integration" bullet of the aimodeling.com
page). The pages give no distributions; the ones below are this library's
stated recipe (see the generator functions).

Recipe (all draws in float64, then one rounding to the storage type):
  * iid kind: q, k, v ~ N(0, 1) per element.
  * walk kind: k and v per KV head are a Gaussian random walk (step sigma 0.1)
    plus N(0, 1) noise; q per query head is mu_h + N(0, 1) with a per-head mean
    mu_h ~ N(0, QMEAN_SCALE^2 I).
  * RoPE (rotate-half pairing, inverse frequency theta^(-2k/d), absolute
    positions) on q and k.
  * walk kind only: a sink (key of token 0 replaced by 8x its own norm along
    the group's latent mean-query direction) and planted key blocks (a key
    block shifted along the latent mean-query direction of a later query block)
    -- both directions come from the generator's own latent means mu_h rotated
    by RoPE, never from the realised noisy data.
  * walk kind only: v divided by max|v| per (sequence, KV head), so output
    tolerances read in units of the largest value magnitude.
  * bf16 storage: round-to-nearest-even of the float64 values.
  * fp8 storage: OCP E4M3FN codes with one float32 scale per (sequence, head,
    128-token block): scale = fp32(amax / 448) (1 for an all-zero block);
    code = e4m3(fp32(clamp(x / scale, -448, 448))).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import List, Optional, Tuple

import numpy as np
import torch

FP8_MAX = 448.0
SCALE_BLOCK = 128          # tokens per fp8 scale
WALK_STEP = 0.1            # sigma of one random-walk step
SINK_GAIN = 8.0            # sink key = SINK_GAIN * |k_0| along the mean-query direction
N_PLANTS = 16              # planted key blocks per KV head
# Scale of the per-head latent query mean.  Chosen once on the S=131072
# construction so the kept-block fraction spans roughly 2 % .. 20 % for
# tau in {2, 4, 6, 8} (measured with the oracle at seed 3: 3.1, 6.9, 12.8,
# 21.0 %); the measured fractions are recorded with every run.
QMEAN_SCALE = 0.35
# Planted shift, as a multiple of the head's RMS key norm.
PLANT_GAIN = 0.5


@dataclass(frozen=True)
class Config:
    id: int
    name: str
    S: int
    Hq: int
    Hkv: int
    d: int
    block: int
    tau: float
    kind: str                  # "iid" | "walk"
    rope_theta: float
    seed: int
    dtype: str = "bf16"        # "bf16" | "fp8"
    batch: int = 1
    taus: Tuple[float, ...] = ()
    paged: bool = False
    n_seqs: int = 0
    len_range: Tuple[int, int] = (0, 0)
    prefix_frac: float = 0.0
    page_size: int = 64


CONFIGS = {
    1: Config(1, "S=2048 GQA 4:1 iid bf16, 64x64 blocks", 2048, 4, 1, 128, 64, 4.0,
              "iid", 1.0e4, 1),
    2: Config(2, "S=32768 32/8 heads walk bf16, 128x128 blocks", 32768, 32, 8, 128, 128,
              4.0, "walk", 5.0e5, 2),
    3: Config(3, "S=131072 32/8 heads walk bf16, 128x128 blocks", 131072, 32, 8, 128,
              128, 4.0, "walk", 5.0e5, 3, taus=(2.0, 4.0, 6.0, 8.0)),
    4: Config(4, "S=131072 32/8 heads walk fp8-e4m3, 128x128 blocks", 131072, 32, 8,
              128, 128, 4.0, "walk", 5.0e5, 3, dtype="fp8"),
    5: Config(5, "paged varlen: 8 seqs 4K-64K, 0-50% cached prefix, 64-token pages",
              0, 32, 8, 128, 128, 4.0, "walk", 5.0e5, 5, paged=True, n_seqs=8,
              len_range=(4096, 65536), prefix_frac=0.5),
}


def config(cid: int, **overrides) -> Config:
    """A registered configuration, optionally with fields overridden (smaller S
    for parity runs, another tau, another seed)."""
    return replace(CONFIGS[cid], **overrides)


# --------------------------------------------------------------------------
# small helpers
# --------------------------------------------------------------------------

def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half RoPE of x [T, d] at absolute positions pos [T] (float64)."""
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.outer(pos.astype(np.float64), inv)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[:, :half], x[:, half:]
    out = np.empty_like(x)
    out[:, :half] = x1 * c - x2 * s
    out[:, half:] = x2 * c + x1 * s
    return out


def _rope_vec_sum(mu: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """sum_t RoPE(mu, t) over positions pos, in closed form per frequency pair."""
    d = mu.shape[-1]
    half = d // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.outer(pos.astype(np.float64), inv)
    cs, sn = np.cos(ang).sum(0), np.sin(ang).sum(0)
    m1, m2 = mu[:half], mu[half:]
    return np.concatenate([m1 * cs - m2 * sn, m2 * cs + m1 * sn])


def _to_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


def quantize_fp8(x: np.ndarray) -> Tuple[torch.Tensor, np.ndarray]:
    """Per-128-token-block E4M3FN quantisation of x [T, d] (float64).

    Returns (codes uint8 [T, d], scales float32 [ceil(T/128)])."""
    T, d = x.shape
    nsb = (T + SCALE_BLOCK - 1) // SCALE_BLOCK
    pad = nsb * SCALE_BLOCK - T
    xp = np.pad(x, ((0, pad), (0, 0))) if pad else x
    amax = np.abs(xp.reshape(nsb, SCALE_BLOCK * d)).max(axis=1)
    scale = (amax / FP8_MAX).astype(np.float32)
    scale[amax == 0] = 1.0
    y = x / np.repeat(scale.astype(np.float64), SCALE_BLOCK)[:T, None]
    y = np.clip(y, -FP8_MAX, FP8_MAX).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


# --------------------------------------------------------------------------
# one sequence, all heads
# --------------------------------------------------------------------------

@dataclass
class SeqMeta:
    plants: List[Tuple[int, int, int, float]] = field(default_factory=list)  # (g, i_p, j_p, beta)


def _gen_sequence(cfg: Config, L: int, ss: np.random.SeedSequence, store, fp8: bool):
    """Draw one sequence of L tokens and hand each head's float64 rows to store().

    store(kind, head, x64) with kind in {"q", "k", "v"} and x64 [L, d]."""
    Hq, Hkv, d, B = cfg.Hq, cfg.Hkv, cfg.d, cfg.block
    G = Hq // Hkv
    kids = ss.spawn(Hq + 2 * Hkv + 1)
    meta_rng = np.random.Generator(np.random.PCG64(kids[-1]))
    pos = np.arange(L)
    meta = SeqMeta()

    if cfg.kind == "walk":
        mu = meta_rng.standard_normal((Hq, d)) * QMEAN_SCALE
    else:
        mu = np.zeros((Hq, d))

    def q_head(h):
        rng = np.random.Generator(np.random.PCG64(kids[h]))
        x = rng.standard_normal((L, d))
        if cfg.kind == "walk":
            x += mu[h]
        x = _rope(x, pos, cfg.rope_theta)
        store("q", h, x)

    def walk(rng):
        steps = rng.standard_normal((L, d))
        steps *= WALK_STEP
        x = np.cumsum(steps, axis=0)
        x += rng.standard_normal((L, d))
        return x

    nb = (L + B - 1) // B
    plants_per_g = []
    if cfg.kind == "walk" and nb >= 4:
        for g in range(Hkv):
            lst = []
            for _ in range(N_PLANTS):
                jp = int(meta_rng.integers(1, nb - 2))          # U{1 .. nb-3}
                ip = int(meta_rng.integers(jp + 2, nb))         # U{jp+2 .. nb-1}
                hp = g * G + int(meta_rng.integers(0, G))       # which head it is aimed at
                lst.append((ip, jp, hp))
            plants_per_g.append(lst)

    def k_head(g):
        rng = np.random.Generator(np.random.PCG64(kids[Hq + g]))
        if cfg.kind == "walk":
            x = walk(rng)
        else:
            x = rng.standard_normal((L, d))
        x = _rope(x, pos, cfg.rope_theta)
        out_plants = []
        if cfg.kind == "walk":
            # sink: token 0's key along the group's latent mean-query direction
            u = sum(_rope_vec_sum(mu[h], pos, cfg.rope_theta) for h in range(g * G, (g + 1) * G))
            u = u / np.linalg.norm(u)
            x[0] = SINK_GAIN * np.linalg.norm(x[0]) * u
            rms = float(np.sqrt(np.mean(np.sum(x * x, axis=1))))
            for (ip, jp, hp) in (plants_per_g[g] if plants_per_g else []):
                qpos = np.arange(ip * B, min((ip + 1) * B, L))
                up = _rope_vec_sum(mu[hp], qpos, cfg.rope_theta)
                up = up / np.linalg.norm(up)
                beta = PLANT_GAIN * rms
                x[jp * B:(jp + 1) * B] += beta * up
                out_plants.append((g, ip, jp, beta))
        store("k", g, x)
        return out_plants

    def v_head(g):
        rng = np.random.Generator(np.random.PCG64(kids[Hq + Hkv + g]))
        if cfg.kind == "walk":
            x = walk(rng)
            x /= np.abs(x).max()
        else:
            x = rng.standard_normal((L, d))
        store("v", g, x)

    with ThreadPoolExecutor(_workers()) as ex:
        futs = [ex.submit(q_head, h) for h in range(Hq)]
        kf = [ex.submit(k_head, g) for g in range(Hkv)]
        futs += [ex.submit(v_head, g) for g in range(Hkv)]
        for f in futs:
            f.result()
        for f in kf:
            meta.plants += f.result()
    return meta


# --------------------------------------------------------------------------
# fixed-shape batch  [batch, S, H, d]
# --------------------------------------------------------------------------

@dataclass
class FixedInputs:
    cfg: Config
    q: torch.Tensor          # [batch, S, Hq, d] bf16, or uint8 E4M3FN codes
    k: torch.Tensor          # [batch, S, Hkv, d]
    v: torch.Tensor
    q_scale: Optional[torch.Tensor] = None   # fp32 [batch, Hq, ceil(S/128)] (fp8 only)
    k_scale: Optional[torch.Tensor] = None
    v_scale: Optional[torch.Tensor] = None
    meta: List[SeqMeta] = field(default_factory=list)


def gen_fixed(cfg: Config) -> FixedInputs:
    """Inputs for a fixed-shape configuration (every sequence has S tokens)."""
    return gen_fixed_multi(cfg, (cfg.dtype,))[cfg.dtype]


def gen_fixed_multi(cfg: Config, dtypes=("bf16", "fp8")):
    """One draw of a fixed-shape configuration stored in several formats
    ({"bf16": FixedInputs, "fp8": FixedInputs}); the fp8 codes come from the
    same float64 values as the bf16 tensors."""
    outs = {}
    for dt in dtypes:
        outs[dt] = _alloc_fixed(replace(cfg, dtype=dt))
    metas = []
    for b, ss in enumerate(np.random.SeedSequence(cfg.seed).spawn(cfg.batch)):
        def store(kind, h, x, b=b):
            for o in outs.values():
                o.store(kind, b, h, x)
        metas.append(_gen_sequence(cfg, cfg.S, ss, store, False))
    res = {}
    for dt, o in outs.items():
        fi = o.finish()
        fi.meta = metas
        res[dt] = fi
    return res


class _alloc_fixed:
    def __init__(self, cfg: Config):
        S, d = cfg.S, cfg.d
        self.cfg = cfg
        self.fp8 = cfg.dtype == "fp8"
        tdt = torch.uint8 if self.fp8 else torch.bfloat16
        self.t = {"q": torch.empty((cfg.batch, S, cfg.Hq, d), dtype=tdt),
                  "k": torch.empty((cfg.batch, S, cfg.Hkv, d), dtype=tdt),
                  "v": torch.empty((cfg.batch, S, cfg.Hkv, d), dtype=tdt)}
        nsb = (S + SCALE_BLOCK - 1) // SCALE_BLOCK
        self.sc = {}
        if self.fp8:
            self.sc = {n: torch.empty((cfg.batch, H, nsb), dtype=torch.float32)
                       for n, H in (("q", cfg.Hq), ("k", cfg.Hkv), ("v", cfg.Hkv))}

    def store(self, kind, b, h, x):
        if self.fp8:
            codes, sc = quantize_fp8(x)
            self.t[kind][b, :, h, :] = codes
            self.sc[kind][b, h, :] = torch.from_numpy(sc)
        else:
            self.t[kind][b, :, h, :] = _to_bf16(x)

    def finish(self) -> "FixedInputs":
        return FixedInputs(self.cfg, self.t["q"], self.t["k"], self.t["v"], self.sc.get("q"),
                           self.sc.get("k"), self.sc.get("v"), [])


# --------------------------------------------------------------------------
# paged varlen batch with cached prefixes
# --------------------------------------------------------------------------

@dataclass
class PagedInputs:
    cfg: Config
    q: torch.Tensor              # [sum_q, Hq, d] bf16 (fp8: uint8 codes), rows [P_b, L_b) of each sequence
    k_cache: torch.Tensor        # [n_pages, page, Hkv, d] bf16 (fp8: uint8 codes)
    v_cache: torch.Tensor
    block_table: torch.Tensor    # int32 [n_seqs, max_pages]; unused entries 0
    cu_seqlens_q: np.ndarray     # int32 [n_seqs + 1]
    seqlens_k: np.ndarray        # int32 [n_seqs]  (L_b)
    prefix: np.ndarray           # int32 [n_seqs]  (P_b = L_b - q_len_b)
    meta: List[SeqMeta] = field(default_factory=list)
    # fp8 only: float32 [n_seqs, H, ceil(max_pages * page / 128)], one scale per
    # 128 positions of each sequence (the queries' from their present rows only)
    q_scale: Optional[torch.Tensor] = None
    k_scale: Optional[torch.Tensor] = None
    v_scale: Optional[torch.Tensor] = None


def paged_lengths(cfg: Config) -> Tuple[np.ndarray, np.ndarray]:
    """(L_b, P_b): lengths log-uniform in len_range, prefixes U(0, prefix_frac) * L_b."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, 1 << 20])))
    lo, hi = cfg.len_range
    L = np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), cfg.n_seqs))).astype(np.int64)
    P = np.floor(rng.uniform(0.0, cfg.prefix_frac, cfg.n_seqs) * L).astype(np.int64)
    return L, P


def gen_paged(cfg: Config, lengths: Optional[Tuple[np.ndarray, np.ndarray]] = None) -> PagedInputs:
    """Inputs for a paged varlen configuration, bf16 or fp8 (cfg.dtype).

    Each sequence b is drawn by the fixed-shape generator at length L_b with
    its own child seed; its keys/values go to pages whose physical ids are one
    random permutation; the queries of rows [P_b, L_b) are packed. fp8 codes
    use one scale per 128 positions of the sequence (quantize_fp8 over the
    sequence's rows; for the queries, over the present rows with the cached
    prefix rows zeroed)."""
    L, P = lengths if lengths is not None else paged_lengths(cfg)
    L = np.asarray(L, dtype=np.int64)
    P = np.asarray(P, dtype=np.int64)
    n = len(L)
    ps = cfg.page_size
    pages_per = (L + ps - 1) // ps
    n_pages = int(pages_per.sum())
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, 1 << 21])))
    perm = rng.permutation(n_pages)
    max_pages = int(pages_per.max())
    table = np.zeros((n, max_pages), dtype=np.int32)
    off = 0
    for b in range(n):
        table[b, :pages_per[b]] = perm[off:off + pages_per[b]]
        off += pages_per[b]
    qlen = L - P
    cu = np.zeros(n + 1, dtype=np.int32)
    cu[1:] = np.cumsum(qlen)
    d = cfg.d
    fp8 = cfg.dtype == "fp8"
    tdt = torch.uint8 if fp8 else torch.bfloat16
    q = torch.empty((int(cu[-1]), cfg.Hq, d), dtype=tdt)
    kc = torch.zeros((n_pages, ps, cfg.Hkv, d), dtype=tdt)
    vc = torch.zeros((n_pages, ps, cfg.Hkv, d), dtype=tdt)
    nsb = (max_pages * ps + SCALE_BLOCK - 1) // SCALE_BLOCK
    scales = {}
    if fp8:
        scales = {n_: torch.ones((n, H, nsb), dtype=torch.float32)
                  for n_, H in (("q", cfg.Hq), ("k", cfg.Hkv), ("v", cfg.Hkv))}
    metas = []
    for b, ss in enumerate(np.random.SeedSequence(cfg.seed).spawn(n)):
        Lb, Pb = int(L[b]), int(P[b])
        pages = torch.from_numpy(table[b, :pages_per[b]].astype(np.int64))

        def store(kind, h, x, Lb=Lb, Pb=Pb, b=b, pages=pages):
            if fp8:
                if kind == "q":
                    x = x.copy()
                    x[:Pb] = 0.0                # scales from the present rows only
                xt, sc = quantize_fp8(x)
                scales[kind][b, h, :len(sc)] = torch.from_numpy(sc)
            else:
                xt = _to_bf16(x)
            if kind == "q":
                q[cu[b]:cu[b + 1], h, :] = xt[Pb:]
            else:
                cache = kc if kind == "k" else vc
                full = torch.zeros((len(pages) * ps, d), dtype=tdt)
                full[:Lb] = xt
                cache[pages, :, h, :] = full.view(len(pages), ps, d)
        metas.append(_gen_sequence(cfg, Lb, ss, store, False))
    return PagedInputs(cfg, q, kc, vc, torch.from_numpy(table), cu,
                       L.astype(np.int32), P.astype(np.int32), metas,
                       scales.get("q"), scales.get("k"), scales.get("v"))


def unpage(inp: PagedInputs, b: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """Contiguous [L_b, Hkv, d] keys and values of sequence b (gathered from pages)."""
    Lb = int(inp.seqlens_k[b])
    ps = inp.cfg.page_size
    npg = (Lb + ps - 1) // ps
    pages = inp.block_table[b, :npg].long()
    k = inp.k_cache[pages].reshape(npg * ps, inp.cfg.Hkv, inp.cfg.d)[:Lb]
    v = inp.v_cache[pages].reshape(npg * ps, inp.cfg.Hkv, inp.cfg.d)[:Lb]
    return k, v
