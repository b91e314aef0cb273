"""Seeded input drawing for the tree-verification workloads.

Recipe (one independent numpy PCG64 stream per component, spawned from
SeedSequence(1000 + config index), so that changing one component never shifts another):

  stream 0  prefix lengths        C4: L_b ~ U{512..8192}; others fixed
  stream 1  trees                 parent[] arrays, topological (0 <= parent[i] < i, parent[0] = -1)
  stream 2  block table           paged layouts: a random permutation of all block ids
  stream 3  Q                     N(0, 1)
  stream 4  K                     N(0, 1) for every used slot (prefix and the tree's own slots)
  stream 5  V                     N(0, 1)
  stream 6  logits                N(0, sigma = 2), float32
  stream 7  draft tokens          uniform ids, distinct among siblings
  stream 8  planting              per internal node: keep-coin (p = 0.85) and target prob pi ~ U[0.8, 0.97]
  stream 9  uniforms              float64 U[0, 1), one per node

bf16 workloads round Q/K/V to bf16 (round to nearest even) and keep them as float32
arrays that hold bf16-exact values, so that both sides consume identical numbers.
Unused cache slots (contiguous: slots at or beyond L_b + T; paged: the unused tail of a
sequence's last block and every unused block) are poisoned with NaN: any stray read
shows up in the output.

Planted mode raises, in each selected internal node's logit row, the logit of the
token drafted for its lowest-index child, so that the target puts most of its mass on
the draft and walks go deep (the serving statistics on the pages report roughly 0.8
acceptance and 3.4 tokens per step).  The raised value uses the expected size of the
row's partition function under N(0, 2^2) logits at temperature 0.7, never the row's
actual softmax, and is floored at (row max + 0.5) so the planted token is the argmax.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import Config

N_STREAMS = 10
_PLANT_ALPHA = 0.85
_PLANT_PI = (0.8, 0.97)
_LOGIT_SIGMA = 2.0
_PLANT_TAU = 0.7


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bias = ((bits >> 16) & 1) + 0x7FFF
    out = ((bits + bias) & 0xFFFF0000).astype(np.uint32)
    return out.view(np.float32).reshape(x.shape)


def static_tree_26() -> np.ndarray:
    """The fixed 26-node tree of the Llama-2-7B-shaped workload (EAGLE-1 style static tree).

    Depth 5, at most 4 children per node, depth histogram 1/4/10/6/3/2.
    """
    return np.array([-1, 0, 0, 0, 0, 1, 1, 1, 1, 2, 2, 2, 3, 3, 4, 5, 5, 5, 6, 9, 12, 15, 15,
                     16, 21, 21], dtype=np.int32)


def _grow_tree(rng: np.random.Generator, T: int, max_depth: int, max_children: int,
               spine: int) -> np.ndarray:
    parent = np.full(T, -1, dtype=np.int32)
    depth = np.zeros(T, dtype=np.int64)
    nchild = np.zeros(T, dtype=np.int64)
    spine = min(spine, T - 1, max_depth)
    for i in range(1, spine + 1):
        parent[i] = i - 1
        depth[i] = i
        nchild[i - 1] += 1
    for i in range(spine + 1, T):
        eligible = [u for u in range(i) if depth[u] < max_depth and nchild[u] < max_children]
        if not eligible:
            raise ValueError("tree shape limits leave no eligible parent")
        u = eligible[int(rng.integers(len(eligible)))]
        parent[i] = u
        depth[i] = depth[u] + 1
        nchild[u] += 1
    return parent


def _make_tree(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    if cfg.tree == "static26":
        p = static_tree_26()
        if cfg.T != len(p):
            raise ValueError("static26 tree needs T = 26")
        return p
    if cfg.tree == "spine3":
        return _grow_tree(rng, cfg.T, cfg.max_depth, cfg.max_children, spine=cfg.max_depth)
    if cfg.tree == "grow":
        return _grow_tree(rng, cfg.T, cfg.max_depth, cfg.max_children, spine=0)
    if cfg.tree == "grow_spine6":
        return _grow_tree(rng, cfg.T, cfg.max_depth, cfg.max_children, spine=6)
    if cfg.tree == "chain":
        return np.arange(-1, cfg.T - 1, dtype=np.int32)
    if cfg.tree == "star":
        p = np.zeros(cfg.T, dtype=np.int32)
        p[0] = -1
        return p
    raise ValueError(f"unknown tree kind {cfg.tree}")


@dataclass
class Inputs:
    cfg: Config
    layout: str                 # "contiguous" or "paged"
    parent: np.ndarray          # int32 [B][T]
    tokens: np.ndarray          # int32 [B][T]; tokens[b][0] is the last committed token
    prefix_len: np.ndarray      # int32 [B]
    q: Optional[np.ndarray]     # float32 [B][T][Hq][d]
    k: Optional[np.ndarray]     # contiguous [B][Hkv][cap][d] | paged [n_blocks][Hkv][bs][d]
    v: Optional[np.ndarray]
    block_table: Optional[np.ndarray]  # int32 [B][max_blocks] (-1 = unused), paged only
    cap: int                    # contiguous slots per sequence (0 when paged)
    logits: Optional[np.ndarray]  # float32 [B][T][V]
    uniforms: np.ndarray        # float64 [B][T]
    tau: np.float32
    planted: np.ndarray         # bool [B][T]: logit row of node u was planted

    @property
    def n_blocks(self) -> int:
        return 0 if self.block_table is None else int(self.k.shape[0])


def generate(cfg: Config, tokens: str = "planted", layout: Optional[str] = None,
             with_kv: bool = True, with_logits: bool = True, seed: Optional[int] = None,
             poison: bool = True) -> Inputs:
    """Draw one batch of inputs for `cfg`.

    tokens: "planted" (deep accepted walks) or "raw" (uniform draft tokens).
    layout: defaults to the config's ("paged" if cfg.paged else "contiguous"); the same
            seed gives the same logical K/V values in either layout.
    """
    if tokens not in ("planted", "raw"):
        raise ValueError(tokens)
    layout = layout or ("paged" if cfg.paged else "contiguous")
    ss = np.random.SeedSequence(1000 + cfg.index if seed is None else seed)
    st = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(N_STREAMS)]
    B, T, V = cfg.B, cfg.T, cfg.V

    lo, hi = cfg.prefix_range()
    if lo == hi:
        prefix_len = np.full(B, lo, dtype=np.int32)
    else:
        prefix_len = st[0].integers(lo, hi + 1, size=B).astype(np.int32)

    parent = np.stack([_make_tree(cfg, st[1]) for _ in range(B)]).astype(np.int32)

    q = k = v = block_table = None
    cap = 0
    if with_kv:
        bf16 = cfg.dtype == "bf16"
        q = st[3].standard_normal((B, T, cfg.Hq, cfg.d), dtype=np.float32)
        if bf16:
            q = round_to_bf16(q)
        nslots = [int(prefix_len[b]) + T for b in range(B)]
        kvals, vvals = [], []
        for b in range(B):
            kb = st[4].standard_normal((cfg.Hkv, nslots[b], cfg.d), dtype=np.float32)
            kvals.append(round_to_bf16(kb) if bf16 else kb)
        for b in range(B):
            vb = st[5].standard_normal((cfg.Hkv, nslots[b], cfg.d), dtype=np.float32)
            vvals.append(round_to_bf16(vb) if bf16 else vb)
        fill = np.nan if poison else 0.0
        if layout == "contiguous":
            cap = max(nslots) + 16
            k = np.full((B, cfg.Hkv, cap, cfg.d), fill, dtype=np.float32)
            v = np.full((B, cfg.Hkv, cap, cfg.d), fill, dtype=np.float32)
            for b in range(B):
                k[b, :, :nslots[b]] = kvals[b]
                v[b, :, :nslots[b]] = vvals[b]
        elif layout == "paged":
            bs = cfg.block_size
            nb = [(n + bs - 1) // bs for n in nslots]
            total = sum(nb)
            n_blocks = total + max(2, total // 32)
            perm = st[2].permutation(n_blocks).astype(np.int32)
            block_table = np.full((B, max(nb)), -1, dtype=np.int32)
            k = np.full((n_blocks, cfg.Hkv, bs, cfg.d), fill, dtype=np.float32)
            v = np.full((n_blocks, cfg.Hkv, bs, cfg.d), fill, dtype=np.float32)
            off = 0
            for b in range(B):
                ids = perm[off:off + nb[b]]
                off += nb[b]
                block_table[b, :nb[b]] = ids
                for j, blk in enumerate(ids):
                    s0 = j * bs
                    cnt = min(bs, nslots[b] - s0)
                    k[blk, :, :cnt] = kvals[b][:, s0:s0 + cnt]
                    v[blk, :, :cnt] = vvals[b][:, s0:s0 + cnt]
        else:
            raise ValueError(layout)

    # Draft tokens: uniform ids, distinct among siblings.
    tok = np.zeros((B, T), dtype=np.int32)
    for b in range(B):
        used = {}
        tok[b, 0] = int(st[7].integers(V))
        for i in range(1, T):
            p = int(parent[b, i])
            sib = used.setdefault(p, set())
            if len(sib) >= V:
                raise ValueError("more siblings than vocabulary entries")
            while True:
                x = int(st[7].integers(V))
                if x not in sib:
                    break
            sib.add(x)
            tok[b, i] = x

    logits = None
    planted = np.zeros((B, T), dtype=bool)
    if with_logits:
        logits = _LOGIT_SIGMA * st[6].standard_normal((B, T, V), dtype=np.float32)
    # Planting draws happen whether or not logits are materialised, so `planted` and the
    # uniforms never depend on with_logits.
    for b in range(B):
        for u in range(T):
            children = np.nonzero(parent[b] == u)[0]
            coin = st[8].random()
            pi = st[8].uniform(*_PLANT_PI)
            if tokens != "planted" or len(children) == 0 or coin >= _PLANT_ALPHA:
                continue
            planted[b, u] = True
            if logits is None:
                continue
            x = int(tok[b, children.min()])
            row = logits[b, u]
            target = _PLANT_TAU * (math.log(pi / (1.0 - pi)) + math.log(V - 1)
                                   + _LOGIT_SIGMA ** 2 / (2.0 * _PLANT_TAU ** 2))
            others = np.delete(row, x)
            floor = float(others.max()) + 0.5 if others.size else 0.0
            row[x] = np.float32(max(target, floor))

    uniforms = st[9].random((B, T))
    return Inputs(cfg=cfg, layout=layout, parent=parent, tokens=tok, prefix_len=prefix_len,
                  q=q, k=k, v=v, block_table=block_table, cap=cap, logits=logits,
                  uniforms=uniforms, tau=np.float32(cfg.tau), planted=planted)


def sampled_drafts(inp: Inputs, draft_tau: float = 0.8, noise: float = 1.0):
    """Draft logits and draft tokens for acceptance with a sampling drafter.

    The drafter's logits are the target's plus N(0, noise^2) noise (a drafter that mostly
    agrees with the target).  Each node's children draw their tokens independently from
    softmax(draft_logits[parent] / draft_tau) by the Gumbel-max trick (the argmax of the
    scaled logits plus Gumbel noise), so no distribution is formed here.  The generator
    is seeded from the configuration index, apart from generate()'s streams.
    Returns (draft_logits float32 [B][T][V], tokens int32 [B][T], root token 0).
    """
    cfg = inp.cfg
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([2000 + cfg.index])))
    B, T, V = inp.logits.shape
    draft = (inp.logits + noise * rng.standard_normal((B, T, V), dtype=np.float32)).astype(np.float32)
    inv = 1.0 / float(np.float32(draft_tau))
    tokens = np.zeros((B, T), np.int32)
    for b in range(B):
        for c in range(1, T):
            a = int(inp.parent[b, c])
            with np.errstate(divide="ignore"):
                gumbel = -np.log(-np.log(rng.random(V)))
            tokens[b, c] = int(np.argmax(draft[b, a].astype(np.float64) * inv + gumbel))
    return draft, tokens


def draft_tree_logits(B: int, V: int, depths: int = 6, beam: int = 8,
                      sharpness: Optional[tuple] = None, seed: int = 3000):
    """Stand-in for the drafter's outputs while a draft tree grows (no trained head exists).

    Returns a list of `depths` float32 arrays [B][beam][V]; row w of sequence b at depth d
    is the drafter's next-token logits after frontier slot w (depth 0: slot 0 is the root).
    Each row is s * N(0, 1) with its own sharpness s, drawn uniformly from `sharpness`.
    A sharp row has a low-entropy distribution and a blunt one a flat distribution, so
    the tree grows deep in some places and wide in others.  The default range spreads
    the perplexity over about 1 to 60 at the vocabulary size given.
    """
    if sharpness is None:
        sharpness = (4.0, 9.0) if V >= 65536 else (6.0, 16.0)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, B, V, depths, beam])))
    out = []
    for _ in range(depths):
        s = rng.uniform(sharpness[0], sharpness[1], size=(B, beam, 1)).astype(np.float32)
        z = rng.standard_normal((B, beam, V), dtype=np.float32)
        out.append((s * z).astype(np.float32))
    return out


def quantize_int4(x: np.ndarray):
    """Symmetric 4-bit quantisation of the last axis of a K or V cache, as a cache writer
    would store it: per row a float32 scale max|x| / 7 and values rint(x / scale) clipped
    to [-8, 7], packed two per byte (element 2j in the low nibble).  Rows holding NaN (the
    poisoned unused slots) get a NaN scale, so a stray read still shows.  Returns (packed
    uint8 [..., d/2], scales float32 [...])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(np.nan_to_num(x)), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(7.0), np.float32(1.0)).astype(np.float32)
    scale = np.where(np.isnan(x).any(axis=-1), np.float32(np.nan), scale)   # keep poisoned rows
    finite = np.where(np.isnan(scale), np.float32(1.0), scale)
    q = np.clip(np.rint(np.nan_to_num(x) / finite[..., None]), -8, 7).astype(np.int16)
    u = (q & 0xF).astype(np.uint8)
    packed = (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)
    return packed, scale
