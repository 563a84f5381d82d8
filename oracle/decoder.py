"""Textbook decoder in fp64 (oracle; test infrastructure only).

The pages fix the method, not the network: the model is a Qwen2.5-shaped
decoder (the model family the pages run), written out from its standard
definition:

  x   = E[token]
  per layer:
    h   = rmsnorm(x) = x / sqrt(mean(x^2) + eps) * w
    q,k,v = h Wq^T, h Wk^T, h Wv^T            (no biases)
    q,k = rotate-half RoPE at absolute positions, inv_freq_j = theta^(-2j/hd)
    o   = softmax(q k^T / sqrt(hd) + mask) v   (query head i uses KV head i // (Hq/Hkv))
    x  += o Wo^T
    h   = rmsnorm(x)
    x  += (silu(h Wg^T) * (h Wu^T)) Wd^T
  logits = rmsnorm(x, w_final) E^T            (tied head; untied uses W_lm)

The property PCD rests on ([Scratch], section "The piece of plumbing you need:
the KV cache"): a token's keys and values depend only on earlier tokens, so a
prefix's cached K/V are exact for any continuation.  ``forward`` therefore takes
an explicit context (cached K/V of earlier tokens, all visible) plus a mask over
the new tokens, and returns the new tokens' K/V.
"""
from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np


class Decoder:
    def __init__(self, weights, dtype=np.float64, cache_weights: bool = True):
        self.w = weights
        self.sh = weights.shape
        self.dt = dtype
        self.cache_weights = cache_weights
        self._cache = {}
        self.zero_head = False  # test hook: replace the LM head by zeros

    # -- parameters ---------------------------------------------------------
    def mat(self, name: str) -> np.ndarray:
        if name in self._cache:
            return self._cache[name]
        a = self.w.values(name).astype(self.dt)
        if self.cache_weights:
            self._cache[name] = a
        return a

    def norm_weight(self) -> np.ndarray:
        # RMSNorm weights of these synthetic models are all ones.
        return np.ones(self.sh.d_model, dtype=self.dt)

    def head(self) -> np.ndarray:
        if self.zero_head:
            return np.zeros((self.sh.vocab_size, self.sh.d_model), dtype=self.dt)
        return self.mat(self.w.lm_head_name())

    # -- building blocks ------------------------------------------------------
    def rmsnorm(self, x: np.ndarray) -> np.ndarray:
        ms = np.mean(x * x, axis=-1, keepdims=True)
        return x / np.sqrt(ms + self.sh.rms_eps) * self.norm_weight()

    def rope(self, x: np.ndarray, positions: np.ndarray) -> np.ndarray:
        """Rotate-half RoPE on x[..., T, hd] at absolute 0-based positions."""
        hd = self.sh.head_dim
        half = hd // 2
        inv_freq = self.sh.rope_theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / hd)
        ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
        cos, sin = np.cos(ang).astype(self.dt), np.sin(ang).astype(self.dt)
        x1, x2 = x[..., :half], x[..., half:]
        return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)

    @staticmethod
    def silu(x: np.ndarray) -> np.ndarray:
        return x / (1.0 + np.exp(-x))

    def attention(self, q, k_ctx, v_ctx, k_new, v_new, mask) -> np.ndarray:
        """q [Hq, T, hd]; k_ctx/v_ctx [Hkv, Pc, hd] (all visible); k_new/v_new
        [Hkv, T, hd]; mask [T, T] (True = query row may see that new token)."""
        Hq, T, hd = q.shape
        Hkv = k_new.shape[0]
        grp = Hq // Hkv
        out = np.empty_like(q)
        scale = 1.0 / np.sqrt(hd)
        chunk = 1024
        for h in range(Hq):
            g = h // grp
            k_all = np.concatenate([k_ctx[g], k_new[g]], axis=0)
            v_all = np.concatenate([v_ctx[g], v_new[g]], axis=0)
            Pc = k_ctx.shape[1]
            for s in range(0, T, chunk):
                qs = q[h, s:s + chunk]
                sc = (qs @ k_all.T) * scale
                vis = np.concatenate([np.ones((qs.shape[0], Pc), bool), mask[s:s + chunk]], axis=1)
                sc = np.where(vis, sc, -np.inf)
                sc = sc - sc.max(axis=1, keepdims=True)
                p = np.exp(sc)
                p /= p.sum(axis=1, keepdims=True)
                out[h, s:s + chunk] = p @ v_all
        return out

    # -- the stack ------------------------------------------------------------
    def forward(self, tokens, positions, mask, ctx: Optional[List[Tuple[np.ndarray, np.ndarray]]] = None,
                n_layers: Optional[int] = None):
        """Run new tokens through the decoder.

        tokens, positions: [T]; mask: [T, T] visibility among the new tokens;
        ctx: per layer (K, V) of earlier tokens, each [Hkv, Pc, hd] after RoPE.
        Returns (x [T, d] residual after the last layer, per-layer (K, V) of the
        new tokens)."""
        sh = self.sh
        L = sh.n_layers if n_layers is None else n_layers
        T = len(tokens)
        hd, Hq, Hkv = sh.head_dim, sh.n_heads, sh.n_kv_heads
        pos = np.asarray(positions)
        x = self.mat("embed")[np.asarray(tokens)].astype(self.dt)
        kv_new = []
        for l in range(L):
            p = f"l{l}."
            h = self.rmsnorm(x)
            q = (h @ self.mat(p + "wq").T).reshape(T, Hq, hd).transpose(1, 0, 2)
            k = (h @ self.mat(p + "wk").T).reshape(T, Hkv, hd).transpose(1, 0, 2)
            v = (h @ self.mat(p + "wv").T).reshape(T, Hkv, hd).transpose(1, 0, 2)
            q = self.rope(q, pos)
            k = self.rope(k, pos)
            kv_new.append((k, v))
            if ctx is None:
                kc = np.zeros((Hkv, 0, hd), self.dt)
                vc = kc
            else:
                kc, vc = ctx[l]
            o = self.attention(q, kc, vc, k, v, mask)
            x = x + o.transpose(1, 0, 2).reshape(T, Hq * hd) @ self.mat(p + "wo").T
            h = self.rmsnorm(x)
            a = self.silu(h @ self.mat(p + "w_gate").T) * (h @ self.mat(p + "w_up").T)
            x = x + a @ self.mat(p + "w_down").T
        return x, kv_new

    def logits(self, x: np.ndarray) -> np.ndarray:
        """Full-vocabulary logits of residual rows x [R, d]."""
        return self.rmsnorm(x) @ self.head().T

    @staticmethod
    def logsumexp(z: np.ndarray) -> np.ndarray:
        m = z.max(axis=-1, keepdims=True)
        return (m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True)))[..., 0]


def causal_mask(T: int) -> np.ndarray:
    return np.tril(np.ones((T, T), dtype=bool))


def kv_bytes(shape, n_tokens: int) -> int:
    """Bytes of a prefix KV cache: tokens x layers x {K,V} x KV heads x head dim
    x element size ([Scratch], section "The piece of plumbing you need: the KV
    cache", gives this product for its triage prompt)."""
    esz = 4 if shape.dtype == "f32" else 2
    return n_tokens * shape.n_layers * 2 * shape.n_kv_heads * shape.head_dim * esz
