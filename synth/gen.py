"""Seeded random tensors for one decode step, plus the paged KV pool layout.

Every array comes from its own PCG64 stream, seeded by
``SeedSequence([1000 + config index, stream id])``, so any subset of arrays
can be drawn without changing the others.  Values are drawn in float32 and,
for bf16 workloads, rounded to bfloat16 by round-to-nearest-even; bf16 data is
carried as uint16 bit patterns (numpy has no bf16 type) and the float32 view
of those bits is exact.

Pool layout (the one ``include/clm.h`` documents):
  k_pool[num_blocks, H_kv, block_size, D]   keys, one row per token slot
  v_pool[num_blocks, H_kv, D, block_size]   values, transposed inside a page
  block_table[B, max_blocks]                 logical page -> pool block
A stream's logical page p holds token positions [p*bs, (p+1)*bs).  Pages are a
seeded random permutation of the pool; unused table entries point at a valid
spare block.  Slots that hold no token yet are filled with NaN so that a
kernel which reads past a stream's length, or before the append wrote a row,
shows up as NaN rather than as a plausible number.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

from .configs import DecodeConfig, get_config

_STREAMS = {
    "kv_len": 1, "stage": 2, "blocks": 3, "k_hist": 4, "v_hist": 5, "k_new": 6,
    "v_new": 7, "q": 8, "w": 9, "h_iso": 10, "uniforms": 11, "draft_logits": 12,
    "draft_tokens": 13, "u_accept": 14, "u_resample": 15, "logits_iso": 16,
    "target_logits_iso": 17, "target_logits_bonus_row": 18,
}

BF16_NAN = np.uint16(0x7FC0)


def _rng(seed: int, name: str, step: int = 0) -> np.random.Generator:
    """The stream for array `name`; steps after the first of a multi-step run
    draw from streams keyed by the step as well."""
    key = [seed, _STREAMS[name]] + ([step] if step else [])
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def draw_kv_len(cfg: DecodeConfig, B: Optional[int] = None) -> np.ndarray:
    B = cfg.B if B is None else B
    rng = _rng(cfg.seed, "kv_len")
    kind, *a = cfg.kv_len_dist
    if kind == "fixed":
        n = np.full(B, a[0], dtype=np.int64)
    elif kind == "uniform":
        n = rng.integers(a[0], a[1], size=B, endpoint=True)
    elif kind == "loguniform":
        n = np.floor(np.exp(rng.uniform(math.log(a[0]), math.log(a[1]), size=B))).astype(np.int64)
        n = np.clip(n, a[0], a[1])
    else:
        raise ValueError(kind)
    return np.maximum(n, cfg.Kq).astype(np.int32)


@dataclasses.dataclass
class StepInputs:
    cfg: DecodeConfig
    kv_len: np.ndarray          # [B] int32, keys visible to a stream's last query after the append
    len_before: np.ndarray      # [B] int32, = kv_len - Kq
    hist_off: np.ndarray        # [B+1] int64 offsets into k_hist / v_hist
    k_hist: np.ndarray          # [sum(len_before), H_kv, D]  (uint16 bf16 bits or float32)
    v_hist: np.ndarray
    k_new: np.ndarray           # [B, Kq, H_kv, D]
    v_new: np.ndarray
    q: np.ndarray               # [B, Kq, H_q, D]
    W: np.ndarray               # [G, V, d]
    head_id: np.ndarray         # [M] int32 (all zero when G == 1)
    block_table: np.ndarray     # [B, max_blocks] int32
    num_blocks: int
    max_blocks: int

    # ---- element-type helpers -------------------------------------------------
    def f32(self, a: np.ndarray) -> np.ndarray:
        """Exact float32 values of a stored array."""
        return bf16_bits_to_f32(a) if self.cfg.dtype == "bf16" else np.asarray(a, np.float32)

    @property
    def storage_dtype(self):
        return np.uint16 if self.cfg.dtype == "bf16" else np.float32

    # ---- logical (unpaged) views ----------------------------------------------
    def logical_k(self, b: int) -> np.ndarray:
        """Keys of stream b after the append, [kv_len[b], H_kv, D] float32."""
        h = self.k_hist[self.hist_off[b]:self.hist_off[b + 1]]
        return np.concatenate([self.f32(h), self.f32(self.k_new[b])], axis=0)

    def logical_v(self, b: int) -> np.ndarray:
        h = self.v_hist[self.hist_off[b]:self.hist_off[b + 1]]
        return np.concatenate([self.f32(h), self.f32(self.v_new[b])], axis=0)

    # ---- paged pool -------------------------------------------------------------
    def build_pool(self, include_new: bool):
        """Pool arrays (k_pool, v_pool) with the history written in; when
        ``include_new`` the step's new rows are written too (the state after
        the append).  Empty slots hold NaN."""
        cfg = self.cfg
        bs, Hk, D = cfg.block_size, cfg.H_kv, cfg.D
        if cfg.dtype == "bf16":
            k_pool = np.full((self.num_blocks, Hk, bs, D), BF16_NAN, dtype=np.uint16)
        else:
            k_pool = np.full((self.num_blocks, Hk, bs, D), np.nan, dtype=np.float32)
        v_pool = np.full((self.num_blocks, Hk, D, bs), k_pool.flat[0], dtype=k_pool.dtype)

        def scatter(lens, starts, k_rows, v_rows):
            b_idx = np.repeat(np.arange(cfg.B), lens)
            pos = np.concatenate([np.arange(s, s + n) for s, n in zip(starts, lens)]) if len(lens) else np.zeros(0, np.int64)
            blk = self.block_table[b_idx, pos // bs]
            off = pos % bs
            k_pool[blk, :, off, :] = k_rows
            v_pool[blk, :, :, off] = v_rows

        scatter(self.len_before, np.zeros(cfg.B, np.int64), self.k_hist, self.v_hist)
        if include_new:
            Kq = cfg.Kq
            scatter(np.full(cfg.B, Kq), self.len_before,
                    self.k_new.reshape(cfg.B * Kq, Hk, D), self.v_new.reshape(cfg.B * Kq, Hk, D))
        return k_pool, v_pool

    def pool_with_room(self, extra_tokens: int, idle_streams: int = 0):
        """The pool before this step's append (as build_pool) and a block table
        with room for `extra_tokens` more tokens per stream beyond this step's
        rows: each stream keeps its pages and gets fresh pool blocks after the
        existing ones.  `idle_streams` padding streams follow the live ones,
        each with pages of its own for extra_tokens + Kq tokens from position
        0.  One more fresh block fills the unused table entries (never read).
        Returns (k_pool, v_pool, block_table, num_blocks)."""
        cfg = self.cfg
        bs, Kq = cfg.block_size, cfg.Kq
        kp, vp = self.build_pool(include_new=False)
        have = (self.kv_len.astype(np.int64) + bs - 1) // bs
        need = (self.kv_len.astype(np.int64) + extra_tokens + bs - 1) // bs
        idle_need = (Kq + extra_tokens + bs - 1) // bs
        n_new = int(np.maximum(need - have, 0).sum()) + idle_streams * idle_need + 1
        spare = self.num_blocks + n_new - 1
        width = int(max(need.max(), idle_need if idle_streams else 1))
        bt = np.full((cfg.B + idle_streams, width), spare, np.int32)
        nxt = self.num_blocks
        for b in range(cfg.B):
            bt[b, :have[b]] = self.block_table[b, :have[b]]
            for p in range(int(have[b]), int(need[b])):
                bt[b, p] = nxt
                nxt += 1
        for i in range(idle_streams):
            bt[cfg.B + i, :idle_need] = np.arange(nxt, nxt + idle_need)
            nxt += idle_need
        fill = kp.flat[0]
        kp = np.concatenate([kp, np.full((n_new,) + kp.shape[1:], fill, kp.dtype)])
        vp = np.concatenate([vp, np.full((n_new,) + vp.shape[1:], fill, vp.dtype)])
        return kp, vp, bt, self.num_blocks + n_new

    # ---- further draws (each from its own stream) -------------------------------
    def h_iso(self) -> np.ndarray:
        """Head input for isolated head checks, [M, d] ~ N(0, 1)."""
        cfg = self.cfg
        return _normal(_rng(cfg.seed, "h_iso"), (cfg.M, cfg.d_model), 1.0, cfg.dtype)

    def uniforms(self) -> np.ndarray:
        """One U[0,1) float32 per head row, for temperature sampling."""
        return _rng(self.cfg.seed, "uniforms").random(self.cfg.M, dtype=np.float32)

    def logits_iso(self, scale: float = 1.0) -> np.ndarray:
        """Isolated sampler input [M, V] float32 ~ N(0, 0.9*scale); 0.9 is the
        spread of a 2048-wide projection with N(0,0.02) weights on N(0,1) input."""
        cfg = self.cfg
        x = _rng(cfg.seed, "logits_iso").standard_normal((cfg.M, cfg.V), dtype=np.float32)
        return x * np.float32(0.9 * scale)

    def step_arrays(self, step: int):
        """(k_new, v_new, q) of decode step `step` of a multi-step run: this
        step's arrays for step 0, fresh draws of the same shapes and
        distributions for later steps."""
        if step == 0:
            return self.k_new, self.v_new, self.q
        cfg = self.cfg
        Kq, Hk, Hq, D = cfg.Kq, cfg.H_kv, cfg.H_q, cfg.D
        k = _normal(_rng(cfg.seed, "k_new", step), (cfg.B, Kq, Hk, D), cfg.qkv_std, cfg.dtype)
        v = _normal(_rng(cfg.seed, "v_new", step), (cfg.B, Kq, Hk, D), cfg.qkv_std, cfg.dtype)
        q = _normal(_rng(cfg.seed, "q", step), (cfg.B, Kq, Hq, D), cfg.qkv_std, cfg.dtype)
        return k, v, q

    def uniforms_step(self, step: int) -> np.ndarray:
        """One U[0,1) float32 per head row for step `step` of a multi-step run."""
        return _rng(self.cfg.seed, "uniforms", step).random(self.cfg.M, dtype=np.float32)

    def spec_inputs(self, step: int = 0):
        """Draft side of speculative verification: draft_probs [B,K,V] f32 (softmax
        of N(0, draft_logit_std) logits), draft_tokens [B,K] drawn from them,
        u_accept [B,K], u_resample [B], isolated target logits [B,K,V], and the
        same with one more row [B,K+1,V] for the bonus-token variant.  Later
        steps of a multi-step run (step > 0) draw from their own streams."""
        cfg = self.cfg
        B, K, V = cfg.B, cfg.Kq, cfg.V
        z = _rng(cfg.seed, "draft_logits", step).standard_normal((B, K, V)) * cfg.draft_logit_std
        z -= z.max(axis=-1, keepdims=True)
        p = np.exp(z)
        p /= p.sum(axis=-1, keepdims=True)
        draft_probs = p.astype(np.float32)
        u = _rng(cfg.seed, "draft_tokens", step).random((B, K))
        cdf = np.cumsum(draft_probs.astype(np.float64), axis=-1)
        cdf /= cdf[..., -1:]
        draft_tokens = np.empty((B, K), np.int32)
        for b in range(B):
            for i in range(K):
                draft_tokens[b, i] = min(int(np.searchsorted(cdf[b, i], u[b, i], side="right")), V - 1)
        u_accept = _rng(cfg.seed, "u_accept", step).random((B, K), dtype=np.float32)
        u_resample = _rng(cfg.seed, "u_resample", step).random(B, dtype=np.float32)
        tl = _rng(cfg.seed, "target_logits_iso", step).standard_normal((B, K, V), dtype=np.float32) * np.float32(0.9)
        extra = _rng(cfg.seed, "target_logits_bonus_row", step).standard_normal((B, 1, V), dtype=np.float32) * np.float32(0.9)
        return dict(draft_probs=draft_probs, draft_tokens=draft_tokens, u_accept=u_accept,
                    u_resample=u_resample, target_logits_iso=tl,
                    target_logits_bonus_iso=np.concatenate([tl, extra], axis=1))


def make_inputs(cfg, B: Optional[int] = None, spare_blocks: int = 4) -> StepInputs:
    """Draw the step's core tensors.  ``B`` overrides the stream count (a
    prefix of the config's streams: lengths are drawn for the full batch first
    so a prefix keeps the same per-stream lengths)."""
    cfg = get_config(cfg)
    kv_full = draw_kv_len(cfg)
    if B is not None and B != cfg.B:
        if B > cfg.B:
            kv_full = draw_kv_len(cfg, B)
        cfg = dataclasses.replace(cfg, B=B)
    kv_len = kv_full[:cfg.B].astype(np.int32)
    Kq, Hk, Hq, D, bs = cfg.Kq, cfg.H_kv, cfg.H_q, cfg.D, cfg.block_size
    len_before = (kv_len - Kq).astype(np.int32)
    hist_off = np.concatenate([[0], np.cumsum(len_before.astype(np.int64))])

    if cfg.G > 1:
        stage = _rng(cfg.seed, "stage").integers(1, cfg.G, size=cfg.B, endpoint=True)
        head_id = np.repeat(stage - 1, Kq).astype(np.int32)
    else:
        head_id = np.zeros(cfg.M, np.int32)

    pages = (kv_len.astype(np.int64) + bs - 1) // bs
    max_blocks = int(pages.max()) if cfg.B else 1
    num_blocks = int(pages.sum()) + spare_blocks
    perm = _rng(cfg.seed, "blocks").permutation(num_blocks).astype(np.int32)
    block_table = np.full((cfg.B, max_blocks), perm[-1], dtype=np.int32)  # spare, never read
    cur = 0
    for b in range(cfg.B):
        block_table[b, :pages[b]] = perm[cur:cur + pages[b]]
        cur += int(pages[b])

    n_hist = int(hist_off[-1])
    k_hist = _normal(_rng(cfg.seed, "k_hist"), (n_hist, Hk, D), cfg.qkv_std, cfg.dtype)
    v_hist = _normal(_rng(cfg.seed, "v_hist"), (n_hist, Hk, D), cfg.qkv_std, cfg.dtype)
    k_new = _normal(_rng(cfg.seed, "k_new"), (cfg.B, Kq, Hk, D), cfg.qkv_std, cfg.dtype)
    v_new = _normal(_rng(cfg.seed, "v_new"), (cfg.B, Kq, Hk, D), cfg.qkv_std, cfg.dtype)
    q = _normal(_rng(cfg.seed, "q"), (cfg.B, Kq, Hq, D), cfg.qkv_std, cfg.dtype)
    W = _normal(_rng(cfg.seed, "w"), (cfg.G, cfg.V, cfg.d_model), cfg.w_std, cfg.dtype)
    return StepInputs(cfg=cfg, kv_len=kv_len, len_before=len_before, hist_off=hist_off,
                      k_hist=k_hist, v_hist=v_hist, k_new=k_new, v_new=v_new, q=q, W=W,
                      head_id=head_id, block_table=block_table, num_blocks=num_blocks,
                      max_blocks=max_blocks)
