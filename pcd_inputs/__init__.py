"""Seeded synthetic inputs shared by the oracle and the HIP path.

This module holds data only: model shapes, seeded random weights and seeded
request workloads.  It contains none of the decoding method's arithmetic, so the
oracle and the device path can both draw from it without sharing any of the
computation they are compared on.

Weights: every matrix has shape ``[out, in]`` (the layout of a linear layer's
weight) and holds ``standard_normal(float32) * 0.02`` draws.  Each block of
``ROW_BLOCK`` rows of a matrix has its own PCG64 stream seeded by
``SeedSequence(seed, spawn_key=(matrix_key, block))``, where matrix_key is 0 for
the embedding, ``1000 * (layer + 1) + j`` for the j-th matrix of a layer in the
order wq, wk, wv, wo, w_gate, w_up, w_down, and 999_999 for an untied LM head.
Blocks are independent, so they are drawn on several threads, and a model cut
to its first layers is bit-identical to the full model in what it keeps.
RMSNorm weights are all ones.  bf16 models round each float32 draw to the
nearest bf16 (ties to even); the bf16 bit patterns are what the device loads
and their exact values are what the oracle reads.

Workloads: prefix token ids are uniform over the vocabulary; each field has a
uniform random scaffold (the row text that ends where the labels part ways) and
candidate token sequences drawn as the recipe of each workload states.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab_size: int
    rope_theta: float
    rms_eps: float
    tied: bool
    dtype: str  # "f32" or "bf16"
    max_seq: int

    @property
    def kv_bytes_per_token(self) -> int:
        esz = 4 if self.dtype == "f32" else 2
        return self.n_layers * 2 * self.n_kv_heads * self.head_dim * esz

    def layer_params(self) -> int:
        d, hd = self.d_model, self.head_dim
        return d * (self.n_heads + 2 * self.n_kv_heads) * hd + self.n_heads * hd * d + 3 * d * self.ffn_dim

    def with_layers(self, n_layers: int) -> "ModelShape":
        return dataclasses.replace(self, name=f"{self.name}-L{n_layers}", n_layers=n_layers)


SHAPES: Dict[str, ModelShape] = {
    "tiny": ModelShape("tiny", 2, 128, 4, 2, 32, 384, 2048, 10000.0, 1e-6, True, "f32", 512),
    "qwen2.5-1.5b": ModelShape("qwen2.5-1.5b", 28, 1536, 12, 2, 128, 8960, 151936, 1e6, 1e-6, True, "bf16", 4096),
    "qwen2.5-7b": ModelShape("qwen2.5-7b", 28, 3584, 28, 4, 128, 18944, 152064, 1e6, 1e-6, False, "bf16", 16640),
}


# ----------------------------------------------------------------------------
# bf16 bit handling (storage format only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bf16, ties to even; returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).reshape(-1)
    out = np.empty(u.shape, np.uint16)
    chunk = 1 << 22
    t = np.empty(min(chunk, max(u.size, 1)), np.uint32)
    t2 = np.empty_like(t)
    for s in range(0, u.size, chunk):
        x = u[s:s + chunk]
        n = x.size
        a1, a2 = t[:n], t2[:n]
        np.right_shift(x, 16, out=a1)
        np.bitwise_and(a1, 1, out=a1)
        np.add(a1, 0x7FFF, out=a1)
        np.add(x, a1, out=a2)
        np.right_shift(a2, 16, out=a2)
        out[s:s + n] = a2
    return out.reshape(np.shape(a))


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# weights
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class Weights:
    """Seeded weights.  ``mats`` holds float32 arrays for f32 models and uint16
    bf16 bit patterns for bf16 models; ``values(name)`` gives float32 values."""
    shape: ModelShape
    seed: int
    mats: Dict[str, np.ndarray]

    def values(self, name: str) -> np.ndarray:
        m = self.mats[name]
        return bf16_bits_to_f32(m) if m.dtype == np.uint16 else m

    def names(self) -> List[str]:
        return list(self.mats.keys())

    def lm_head_name(self) -> str:
        return "embed" if self.shape.tied else "lm_head"


def weight_names(shape: ModelShape) -> List[str]:
    names = ["embed"]
    for l in range(shape.n_layers):
        names += [f"l{l}.{n}" for n in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")]
    if not shape.tied:
        names.append("lm_head")
    return names


def weight_shape(shape: ModelShape, name: str):
    d, hd, F, V = shape.d_model, shape.head_dim, shape.ffn_dim, shape.vocab_size
    base = name.split(".")[-1]
    return {
        "embed": (V, d), "lm_head": (V, d),
        "wq": (shape.n_heads * hd, d), "wk": (shape.n_kv_heads * hd, d), "wv": (shape.n_kv_heads * hd, d),
        "wo": (d, shape.n_heads * hd), "w_gate": (F, d), "w_up": (F, d), "w_down": (d, F),
    }[base]


ROW_BLOCK = 4096


def _matrix_key(name: str) -> int:
    if name == "embed":
        return 0
    if name == "lm_head":
        return 999_999
    l, base = name.split(".")
    j = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down").index(base)
    return 1000 * (int(l[1:]) + 1) + j


def _draw_matrix(seed: int, name: str, shp, bf16: bool, pool) -> np.ndarray:
    rows, cols = shp
    key = _matrix_key(name)
    out = np.empty(shp, np.uint16 if bf16 else np.float32)

    def block(b):
        r0, r1 = b * ROW_BLOCK, min(rows, (b + 1) * ROW_BLOCK)
        ss = np.random.SeedSequence(seed, spawn_key=(key, b))
        a = np.random.Generator(np.random.PCG64(ss)).standard_normal((r1 - r0, cols), dtype=np.float32)
        a *= np.float32(0.02)
        out[r0:r1] = f32_to_bf16_bits(a) if bf16 else a

    nb = (rows + ROW_BLOCK - 1) // ROW_BLOCK
    list(pool.map(block, range(nb)))
    return out


def make_weights(shape: ModelShape, seed: int, n_layers: Optional[int] = None) -> Weights:
    """Draw the seeded weights; ``n_layers`` (if given) keeps only the first
    layers, bit-identical to the same layers of the full model."""
    from concurrent.futures import ThreadPoolExecutor
    import os
    sh = shape if n_layers is None else shape.with_layers(n_layers)
    mats: Dict[str, np.ndarray] = {}
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as pool:
        for name in weight_names(sh):
            mats[name] = _draw_matrix(seed, name, weight_shape(sh, name), sh.dtype == "bf16", pool)
    return Weights(sh, seed, mats)


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class Field:
    """One field of a request.  ``candidates`` holds one token list per label;
    ``spellings``, when given, holds per label every way of writing it (its
    first spelling is the candidate itself); ``mode`` names the scoring rule:
    "path", "exact", "level" or "mean"."""
    scaffold: List[int]
    candidates: List[List[int]]
    kind: str = "enum"
    spellings: Optional[List[List[List[int]]]] = None
    mode: str = "path"


@dataclasses.dataclass
class Request:
    prefix: List[int]
    fields: List[Field]


@dataclasses.dataclass
class Workload:
    name: str
    shape: ModelShape
    weight_seed: int
    input_seed: int
    requests: List[Request]
    description: str = ""

    @property
    def n_fields(self) -> int:
        return sum(len(r.fields) for r in self.requests)


def _distinct(rng: np.random.Generator, V: int, k: int) -> List[int]:
    return [int(t) for t in rng.choice(V, size=k, replace=False)]


def _scaffold(rng, V, lo, hi) -> List[int]:
    n = int(rng.integers(lo, hi + 1))
    return [int(t) for t in rng.integers(0, V, size=n)]


def _id_field(rng, V, n_options: int, width: int, scaffold_len=(8, 12)) -> Field:
    """Fixed-width ID options sharing one lead token: option i is
    (t0, A[i // width], B[i % width]) with A and B lists of distinct ids."""
    sc = _scaffold(rng, V, *scaffold_len)
    t0 = int(rng.integers(0, V))
    n_a = (n_options + width - 1) // width
    A = _distinct(rng, V, n_a)
    B = _distinct(rng, V, width)
    cands = [[t0, A[i // width], B[i % width]] for i in range(n_options)]
    return Field(sc, cands, kind="id")


def _schema_28(rng, V) -> List[Field]:
    """10 booleans (one shared true/false token pair) + 18 four-way enums, in a
    seeded order; scaffolds of 8..12 tokens."""
    pair = _distinct(rng, V, 2)
    kinds = ["bool"] * 10 + ["enum"] * 18
    order = rng.permutation(len(kinds))
    fields = []
    for i in order:
        sc = _scaffold(rng, V, 8, 12)
        if kinds[i] == "bool":
            fields.append(Field(sc, [[pair[0]], [pair[1]]], kind="bool"))
        else:
            fields.append(Field(sc, [[t] for t in _distinct(rng, V, 4)], kind="enum"))
    return fields


def _uniform_prefix(rng, V, P) -> List[int]:
    return [int(t) for t in rng.integers(0, V, size=P)]


def make_workload(name: str) -> Workload:
    """Workloads:
    cfg0   tiny f32 model; 96-token prefix; 4 fields, scaffold 6, 2..4 single-token candidates.
    cfg0t  cfg0's prefix and fields plus one field of 6 three-token IDs sharing the lead token.
    cfg1   1.5B-shaped bf16; 512-token prefix; 28 fields (10 boolean, 18 four-way enums).
    cfg2   1.5B-shaped; 2048-token prefix; 3 booleans + one 255-option 3-token ID field.
    cfg3   1.5B-shaped; 64 requests, each with its own 1024-token prefix and a 28-field schema.
    cfg4   7B-shaped; 16384-token prefix; one 200-option ID field + 63 enums with 2..8 options.
    """
    if name in ("cfg0", "cfg0t"):
        sh = SHAPES["tiny"]
        rng = np.random.Generator(np.random.PCG64(2000))
        V = sh.vocab_size
        prefix = _uniform_prefix(rng, V, 96)
        fields = []
        for _ in range(4):
            sc = [int(t) for t in rng.integers(0, V, size=6)]
            k = int(rng.integers(2, 5))
            fields.append(Field(sc, [[t] for t in _distinct(rng, V, k)]))
        if name == "cfg0t":
            rng2 = np.random.Generator(np.random.PCG64(2010))
            f = _id_field(rng2, V, 6, 3, scaffold_len=(6, 6))
            fields.append(f)
        return Workload(name, sh, 1000, 2000 if name == "cfg0" else 2010, [Request(prefix, fields)])
    if name == "cfg1":
        sh = SHAPES["qwen2.5-1.5b"]
        rng = np.random.Generator(np.random.PCG64(2001))
        prefix = _uniform_prefix(rng, sh.vocab_size, 512)
        return Workload(name, sh, 1001, 2001, [Request(prefix, _schema_28(rng, sh.vocab_size))])
    if name == "cfg2":
        sh = SHAPES["qwen2.5-1.5b"]
        V = sh.vocab_size
        rng = np.random.Generator(np.random.PCG64(2002))
        prefix = _uniform_prefix(rng, V, 2048)
        pair = _distinct(rng, V, 2)
        fields = [Field(_scaffold(rng, V, 8, 12), [[pair[0]], [pair[1]]], kind="bool") for _ in range(3)]
        fields.insert(int(rng.integers(0, 4)), _id_field(rng, V, 255, 16))
        return Workload(name, sh, 1001, 2002, [Request(prefix, fields)])
    if name == "cfg3":
        sh = SHAPES["qwen2.5-1.5b"]
        reqs = []
        for r in range(64):
            rng = np.random.Generator(np.random.PCG64(2003 + r))
            prefix = _uniform_prefix(rng, sh.vocab_size, 1024)
            reqs.append(Request(prefix, _schema_28(rng, sh.vocab_size)))
        return Workload(name, sh, 1001, 2003, reqs)
    if name == "cfg4":
        sh = SHAPES["qwen2.5-7b"]
        V = sh.vocab_size
        rng = np.random.Generator(np.random.PCG64(2004))
        prefix = _uniform_prefix(rng, V, 16384)
        fields = []
        for _ in range(63):
            k = int(rng.integers(2, 9))
            fields.append(Field(_scaffold(rng, V, 8, 12), [[t] for t in _distinct(rng, V, k)]))
        fields.insert(int(rng.integers(0, 64)), _id_field(rng, V, 200, 16))
        return Workload(name, sh, 1002, 2004, [Request(prefix, fields)])
    raise KeyError(name)


def random_trie_fields(seed: int, V: int, n_fields: int, max_cands: int = 12, max_len: int = 4,
                       scaffold_len=(1, 6), small_alphabet: int = 6) -> List[Field]:
    """Random fields whose candidates are token sequences over a small alphabet,
    so that shared prefixes (tries several levels deep) are common.  Candidate
    lists never contain duplicates or one candidate that is a proper prefix of
    another (such fields are outside the accepted input)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    alphabet = _distinct(rng, V, small_alphabet)
    out = []
    for _ in range(n_fields):
        sc = _scaffold(rng, V, *scaffold_len)
        k = int(rng.integers(2, max_cands + 1))
        cands: List[List[int]] = []
        tries = 0
        while len(cands) < k and tries < 1000:
            tries += 1
            L = int(rng.integers(1, max_len + 1))
            c = [alphabet[int(i)] for i in rng.integers(0, small_alphabet, size=L)]
            bad = any(c == o or c[:len(o)] == o or o[:len(c)] == c for o in cands)
            if not bad:
                cands.append(c)
        if len(cands) < 2:
            cands = [[alphabet[0]], [alphabet[1]]]
        out.append(Field(sc, cands, kind="trie"))
    return out


def random_spelling_fields(seed: int, V: int, n_fields: int, max_labels: int = 5, max_spellings: int = 3,
                           max_len: int = 3, scaffold_len=(1, 6), small_alphabet: int = 5,
                           mode: str = "path") -> List[Field]:
    """Random fields whose labels each have 1..max_spellings spellings over a
    small alphabet (so spellings of different labels share prefixes, as a
    quoted and a bare boolean share the quote).  No two spellings of a field
    are equal, and none is a proper prefix of another."""
    rng = np.random.Generator(np.random.PCG64(seed))
    alphabet = _distinct(rng, V, small_alphabet)
    out = []
    for _ in range(n_fields):
        sc = _scaffold(rng, V, *scaffold_len)
        k = int(rng.integers(2, max_labels + 1))
        used: List[List[int]] = []
        labels: List[List[List[int]]] = []
        tries = 0
        while len(labels) < k and tries < 2000:
            tries += 1
            want = int(rng.integers(1, max_spellings + 1))
            lab: List[List[int]] = []
            for _ in range(50):
                if len(lab) == want:
                    break
                L = int(rng.integers(1, max_len + 1))
                c = [alphabet[int(i)] for i in rng.integers(0, small_alphabet, size=L)]
                if not any(c == o or c[:len(o)] == o or o[:len(c)] == c for o in used + lab):
                    lab.append(c)
            if lab:
                labels.append(lab)
                used += lab
        if len(labels) < 2:
            labels = [[[alphabet[0]]], [[alphabet[1]]]]
        out.append(Field(sc, [lab[0] for lab in labels], kind="spellings", spellings=labels, mode=mode))
    return out

