"""An fp32 model of the device path's bf16 arithmetic (test infrastructure).

This is not the oracle: it models where the HIP kernels round, so that the
tolerances of the bf16 parity tests can be derived instead of fitted.  The
kernels keep the residual stream, every accumulation, the softmax
statistics and the log-sum-exp in fp32, and round to bf16 (nearest, ties to
even) at these points of each layer:

  1. the RMSNorm output that feeds the QKV GEMM (and the readout rows);
  2. q, k and v after RoPE (k and v are what the KV caches hold);
  3. the attention probabilities exp(s - m) that multiply V (their sum l
     stays fp32);
  4. the attention output o = (P V) / l;
  5. the RMSNorm output that feeds the gate/up GEMM;
  6. the SwiGLU output silu(h Wg) * (h Wu) that feeds the down GEMM;
  7. the final RMSNorm output of the readout rows.

The decoder structure (and the plan, readout and combine steps, which have
no bf16 rounding) come from the oracle; only these rounding points are
added.
"""
import numpy as np

import pcd_inputs as pi
from oracle import decoder as odec


def bf16_round(a) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 (ties to even), back in fp32."""
    return pi.bf16_bits_to_f32(pi.f32_to_bf16_bits(np.asarray(a, np.float32)))


class Bf16Emulation(odec.Decoder):
    """The oracle's decoder in fp32 with the device's bf16 rounding points."""

    def __init__(self, weights):
        super().__init__(weights, np.float32)

    def rmsnorm(self, x):  # points 1, 5 and 7
        return bf16_round(super().rmsnorm(x))

    def attention(self, q, k_ctx, v_ctx, k_new, v_new, mask):  # points 3 and 4 (q, k, v come rounded)
        Hq, T, hd = q.shape
        grp = Hq // k_new.shape[0]
        out = np.empty_like(q)
        scale = np.float32(1.0 / np.sqrt(hd))
        for h in range(Hq):
            g = h // grp
            k_all = np.concatenate([k_ctx[g], k_new[g]], 0)
            v_all = np.concatenate([v_ctx[g], v_new[g]], 0)
            sc = (q[h] @ k_all.T) * scale
            vis = np.concatenate([np.ones((T, k_ctx.shape[1]), bool), mask], 1)
            sc = np.where(vis, sc, -np.inf)
            p = np.exp(sc - sc.max(1, keepdims=True))
            out[h] = (bf16_round(p) @ v_all) / p.sum(1, keepdims=True)
        return bf16_round(out)

    def forward(self, tokens, positions, mask, ctx=None, n_layers=None):
        sh = self.sh
        L = sh.n_layers if n_layers is None else n_layers
        T = len(tokens)
        hd, Hq, Hkv = sh.head_dim, sh.n_heads, sh.n_kv_heads
        pos = np.asarray(positions)
        x = self.mat("embed")[np.asarray(tokens)].astype(np.float32)
        kv_new = []
        for l in range(L):
            p = f"l{l}."
            h = self.rmsnorm(x)
            q = (h @ self.mat(p + "wq").T).reshape(T, Hq, hd).transpose(1, 0, 2)
            k = (h @ self.mat(p + "wk").T).reshape(T, Hkv, hd).transpose(1, 0, 2)
            v = (h @ self.mat(p + "wv").T).reshape(T, Hkv, hd).transpose(1, 0, 2)
            q = bf16_round(self.rope(q, pos))  # point 2
            k = bf16_round(self.rope(k, pos))
            v = bf16_round(v)
            kv_new.append((k, v))
            kc, vc = (np.zeros((Hkv, 0, hd), np.float32),) * 2 if ctx is None else ctx[l]
            o = self.attention(q, kc, vc, k, v, mask)
            x = x + o.transpose(1, 0, 2).reshape(T, Hq * hd) @ self.mat(p + "wo").T
            h = self.rmsnorm(x)
            a = bf16_round(self.silu(h @ self.mat(p + "w_gate").T) * (h @ self.mat(p + "w_up").T))  # point 6
            x = x + a @ self.mat(p + "w_down").T
        return x, kv_new
