"""ctypes binding of libpcd.so (argument marshalling only).

Every step of the decoding path runs in the library's HIP kernels; this module
only converts Python/NumPy arguments to the C structs of include/pcd.h and
hands torch-allocated device memory and torch's current HIP stream to the
library.  It fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
from itertools import chain
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_void_p
from typing import Dict, List, Optional, Sequence
import weakref

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpcd.so")

PCD_OK = 0
ERROR_NAMES = {-1: "ARG", -2: "TOKEN", -3: "NCAND", -4: "EMPTY", -5: "DUP", -6: "PREFIX", -7: "CAP",
               -8: "STATE", -9: "DEVICE", -10: "NOMEM"}
DTYPE_F32, DTYPE_BF16 = 0, 1
MAX_PENDING = 4  # started, unfinished calls one model holds at most

EXPORTS = ("pcd_workspace_bytes", "pcd_load_weights", "pcd_load_weights_noalloc", "pcd_state_bytes", "pcd_prefill", "pcd_prefill_many",
           "pcd_extend",
           "pcd_fork", "pcd_state_tokens", "pcd_new_state", "pcd_decide", "pcd_extend_decide",
           "pcd_extend_decide_start", "pcd_finish",
           "pcd_decide_sequenced", "pcd_decide_many",
           "pcd_debug_plan", "pcd_get_stats",
           "pcd_free_state", "pcd_free_model", "pcd_last_error", "pcd_set_kernel_timing", "pcd_get_kernel_times")

KERNEL_CLASSES = ("prefill_qkv", "prefill_attn", "prefill_o", "prefill_gateup", "prefill_down", "branch_qkv",
                  "branch_attn", "branch_tail", "branch_o", "branch_gateup", "branch_down", "readout_lmhead",
                  "other", "fused_qkv", "fused_attn", "fused_o", "fused_gateup", "fused_down")


class PcdError(RuntimeError):
    def __init__(self, code: int, msg: str):
        self.code = code
        self.name = ERROR_NAMES.get(code, str(code))
        super().__init__(f"PCD_E_{self.name}: {msg}")


class pcd_config(ctypes.Structure):
    _fields_ = [("n_layers", c_int32), ("d_model", c_int32), ("n_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("ffn_dim", c_int32), ("vocab_size", c_int32), ("max_seq", c_int32),
                ("rope_theta", c_float), ("rms_eps", c_float), ("tied_lm_head", c_int32), ("dtype", c_int32)]


class pcd_weights(ctypes.Structure):
    _fields_ = [("embed", c_void_p), ("lm_head", c_void_p), ("final_norm", c_void_p),
                ("attn_norm", POINTER(c_void_p)), ("mlp_norm", POINTER(c_void_p)),
                ("wq", POINTER(c_void_p)), ("wk", POINTER(c_void_p)), ("wv", POINTER(c_void_p)),
                ("wo", POINTER(c_void_p)), ("w_gate", POINTER(c_void_p)), ("w_up", POINTER(c_void_p)),
                ("w_down", POINTER(c_void_p))]


class pcd_limits(ctypes.Structure):
    _fields_ = [("max_prefill_tokens", c_int32), ("max_branch_tokens", c_int32), ("max_readouts", c_int32),
                ("max_gathers", c_int32), ("max_fields", c_int32), ("max_candidates", c_int32),
                ("max_requests", c_int32), ("max_spellings", c_int32)]


class pcd_candidate(ctypes.Structure):
    _fields_ = [("tokens", POINTER(c_int32)), ("n_tokens", c_int32), ("spell_len", POINTER(c_int32)),
                ("n_spellings", c_int32)]


class pcd_field(ctypes.Structure):
    _fields_ = [("scaffold", POINTER(c_int32)), ("n_scaffold", c_int32), ("cand_offset", c_int32),
                ("n_cands", c_int32), ("score_mode", c_int32)]


# PCD_SCORE_* by name
SCORE_MODES = {"path": 0, "exact": 1, "level": 2, "mean": 3}


class pcd_request(ctypes.Structure):
    _fields_ = [("fields", POINTER(pcd_field)), ("n_fields", c_int32), ("candidates", POINTER(pcd_candidate)),
                ("n_candidates", c_int32)]


class pcd_outputs(ctypes.Structure):
    # pointer-sized address fields (the C struct's float* / int32_t*), set from
    # NumPy arrays' addresses
    _fields_ = [("cand_prob", c_void_p), ("cand_logscore", c_void_p), ("field_mass", c_void_p),
                ("field_margin", c_void_p), ("field_argmax", c_void_p), ("readout_lse", c_void_p),
                ("gather_logit", c_void_p)]


def _result_arrays(n_cands: int, n_fields: int, o: Optional[pcd_outputs] = None):
    """One request's result arrays (the library writes every element when
    the call succeeds) and the pcd_outputs that points at them (o, if given,
    is filled in place)."""
    d = {"prob": np.empty(n_cands, np.float32), "logscore": np.empty(n_cands, np.float32),
         "mass": np.empty(n_fields, np.float32), "margin": np.empty(n_fields, np.float32),
         "argmax": np.empty(n_fields, np.int32)}
    if o is None:
        o = pcd_outputs()
    o.cand_prob, o.cand_logscore = d["prob"].ctypes.data, d["logscore"].ctypes.data
    o.field_mass, o.field_margin = d["mass"].ctypes.data, d["margin"].ctypes.data
    o.field_argmax = d["argmax"].ctypes.data
    return d, o


def _debug_arrays(d: dict, o: pcd_outputs, n_readouts: int, n_gathers: int):
    d["lse"] = np.zeros(max(1, n_readouts), np.float32)
    d["z"] = np.zeros(max(1, n_gathers), np.float32)
    o.readout_lse, o.gather_logit = d["lse"].ctypes.data, d["z"].ctypes.data


class pcd_stats(ctypes.Structure):
    _fields_ = [("prefill_passes", c_int64), ("branch_passes", c_int64), ("last_branch_tokens", c_int32),
                ("last_readouts", c_int32), ("last_gathers", c_int32), ("last_requests", c_int32),
                ("last_prefill_ms", c_float), ("last_branch_ms", c_float), ("last_readout_ms", c_float),
                ("workspace_bytes", c_int64)]


_PLAN_ARRAYS = ("tok", "pos", "req", "field", "anc_off", "anc", "ro_tok", "ro_field", "g_off", "g_tok",
                "f_ro_root", "f_cand_off", "f_mode", "c_spell_off", "s_path_off", "s_path")


class pcd_plan_info(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in ("n_branch", "n_readouts", "n_gathers", "n_fields", "n_candidates",
                                        "n_paths", "n_anc", "n_spellings")] + \
               [(n, POINTER(c_int32)) for n in _PLAN_ARRAYS]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads the in-tree libpcd.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    # torch ships its own HIP runtime under the same soname as the system's;
    # whichever is loaded first serves the whole process.  Loading torch
    # first makes the library share the runtime that owns torch's device
    # memory and streams (loaded the other way round, pinned host allocations
    # were seen to fail).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P = POINTER
    sig = {
        "pcd_workspace_bytes": (c_size_t, [P(pcd_config), P(pcd_limits)]),
        "pcd_load_weights": (c_int32, [P(pcd_config), P(pcd_limits), P(pcd_weights), c_void_p, c_size_t, c_void_p,
                                       P(c_void_p)]),
        "pcd_load_weights_noalloc": (c_int32, [P(pcd_config), P(pcd_limits), P(pcd_weights), c_void_p,
                                               P(c_void_p)]),
        "pcd_state_bytes": (c_size_t, [c_void_p, c_int32]),
        "pcd_prefill": (c_int32, [c_void_p, P(c_int32), c_int32, c_void_p, c_size_t, c_void_p, P(c_void_p)]),
        "pcd_prefill_many": (c_int32, [c_void_p, c_int32, P(c_int32), P(c_int32), P(c_void_p), P(c_size_t),
                                       c_void_p, P(c_void_p)]),
        "pcd_extend": (c_int32, [c_void_p, P(c_int32), c_int32, c_void_p]),
        "pcd_fork": (c_int32, [c_void_p, c_void_p, c_size_t, c_void_p, P(c_void_p)]),
        "pcd_state_tokens": (c_int32, [c_void_p]),
        "pcd_new_state": (c_int32, [c_void_p, c_void_p, c_size_t, P(c_void_p)]),
        "pcd_extend_decide": (c_int32, [c_void_p, P(c_int32), c_int32, P(pcd_field), c_int32, P(pcd_candidate),
                                        c_int32, c_float, P(pcd_outputs), c_void_p]),
        "pcd_extend_decide_start": (c_int32, [c_void_p, P(c_int32), c_int32, P(pcd_field), c_int32,
                                              P(pcd_candidate), c_int32, c_float, P(pcd_outputs), c_void_p,
                                              P(c_void_p)]),
        "pcd_finish": (c_int32, [c_void_p]),
        "pcd_decide_sequenced": (c_int32, [c_void_p, P(pcd_field), c_int32, P(pcd_candidate), c_int32, c_int32,
                                           c_float, P(pcd_outputs), c_void_p]),
        "pcd_decide": (c_int32, [c_void_p, P(pcd_field), c_int32, P(pcd_candidate), c_int32, c_float,
                                 P(pcd_outputs), c_void_p]),
        "pcd_decide_many": (c_int32, [P(c_void_p), P(pcd_request), c_int32, c_float, P(pcd_outputs), c_void_p]),
        "pcd_debug_plan": (c_int32, [c_int32, c_int32, c_int32, P(c_int32), P(pcd_request), P(pcd_plan_info)]),
        "pcd_get_stats": (c_int32, [c_void_p, P(pcd_stats)]),
        "pcd_free_state": (None, [c_void_p]),
        "pcd_free_model": (None, [c_void_p]),
        "pcd_last_error": (ctypes.c_char_p, []),
        "pcd_set_kernel_timing": (c_int32, [c_void_p, c_int32]),
        "pcd_get_kernel_times": (c_int32, [c_void_p, P(c_float), P(c_int64)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(rc: int):
    if rc != PCD_OK:
        raise PcdError(rc, load_library().pcd_last_error().decode(errors="replace"))


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(POINTER(c_int32))




# the 64-bit word layouts _Marshalled writes (x86-64 / little-endian ABI)
assert ctypes.sizeof(pcd_candidate) == 32 and pcd_candidate.spell_len.offset == 16
assert ctypes.sizeof(pcd_field) == 24 and pcd_field.cand_offset.offset == 12 and pcd_field.score_mode.offset == 20


class _Marshalled:
    """C view of requests: lists of fields, each with .scaffold and
    .candidates (token-id sequences), optionally .spellings and .mode.  Per
    request, every token id goes into one int32 buffer, and the pcd_field /
    pcd_candidate arrays are NumPy structured arrays that ctypes views
    without a copy.  Keeps the buffers alive."""

    def __init__(self, requests: Sequence[Sequence]):
        self.keep = []
        self.reqs = (pcd_request * len(requests))()
        self.n_cands, self.n_fields = [], []
        for r, fields in enumerate(requests):
            if isinstance(fields, CompiledFields):
                # already marshalled: share its arrays
                src = fields.m
                self.keep.append(src)
                self.reqs[r] = src.reqs[0]
                self.n_cands.append(src.n_cands[0])
                self.n_fields.append(src.n_fields[0])
                continue
            nf = len(fields)
            spelled = [getattr(f, "spellings", None) for f in fields]
            # token lists: every scaffold, then every candidate (its spellings back to back)
            cand_lists, spl, s_off, s_n = [], [], [], []
            for f, sp in zip(fields, spelled):
                if sp is None:
                    cand_lists += f.candidates
                    s_off += [-1] * len(f.candidates)
                    s_n += [0] * len(f.candidates)
                else:
                    for lab in sp:
                        cand_lists.append(list(chain.from_iterable(lab)))
                        s_off.append(len(spl))
                        s_n.append(len(lab))
                        spl += map(len, lab)
            scaf = [f.scaffold for f in fields]
            nc = len(cand_lists)
            lens = np.fromiter(map(len, chain(scaf, cand_lists)), dtype=np.int64, count=nf + nc)
            offs = np.zeros(nf + nc, dtype=np.int64)
            np.cumsum(lens[:-1], out=offs[1:])
            tok = np.fromiter(chain.from_iterable(chain(scaf, cand_lists)), dtype=np.int32, count=int(lens.sum()))
            sl = np.asarray(spl, dtype=np.int32)
            tb, sb = tok.ctypes.data, sl.ctypes.data
            # pcd_candidate is 4 little-endian 64-bit words: tokens, n_tokens, spell_len, n_spellings;
            # pcd_field is 3: scaffold, n_scaffold | cand_offset << 32, n_cands | score_mode << 32
            cv = np.zeros((max(1, nc), 4), dtype=np.int64)
            cv[:nc, 0] = tb + 4 * offs[nf:]
            cv[:nc, 1] = lens[nf:]
            so = np.asarray(s_off, dtype=np.int64)
            cv[:nc, 2] = np.where(so >= 0, sb + 4 * so, 0)
            cv[:nc, 3] = s_n
            fv = np.zeros((max(1, nf), 3), dtype=np.int64)
            fv[:nf, 0] = tb + 4 * offs[:nf]
            ncf = np.fromiter((len(f.candidates) for f in fields), dtype=np.int64, count=nf)
            c_first = np.zeros(nf, dtype=np.int64)
            np.cumsum(ncf[:-1], out=c_first[1:])
            fv[:nf, 1] = lens[:nf] | (c_first << 32)
            modes = np.asarray([SCORE_MODES.get(getattr(f, "mode", None) or "path", -1) for f in fields],
                               dtype=np.int64)
            fv[:nf, 2] = ncf | ((modes & 0xFFFFFFFF) << 32)
            ca = (pcd_candidate * len(cv)).from_buffer(cv)
            fa = (pcd_field * len(fv)).from_buffer(fv)
            self.keep += [tok, sl, cv, fv, ca, fa]
            self.reqs[r].fields = fa
            self.reqs[r].n_fields = nf
            self.reqs[r].candidates = ca
            self.reqs[r].n_candidates = nc
            self.n_cands.append(nc)
            self.n_fields.append(nf)


class CompiledFields:
    """A schema (list of fields) marshalled once into the C arrays the
    library reads, for reuse across requests: every decide call accepts it in
    place of the field list.  The library still validates the fields and
    builds the plan on every call; only the Python-to-C conversion is saved.
    The fields must not change while it is in use."""

    def __init__(self, fields: Sequence):
        self.fields = list(fields)
        self.m = _Marshalled([self.fields])

    def __len__(self):
        return len(self.fields)

    def __iter__(self):
        return iter(self.fields)

    def __getitem__(self, i):
        return self.fields[i]


def debug_plan(vocab_size: int, max_seq: int, prefix_lens: Sequence[int], requests) -> Dict[str, np.ndarray]:
    """The library's plan for these requests (host only, no device work)."""
    lib = load_library()
    mr = _Marshalled(requests)
    lens = np.ascontiguousarray(prefix_lens, dtype=np.int32)
    info = pcd_plan_info()
    _check(lib.pcd_debug_plan(vocab_size, max_seq, len(requests), _i32p(lens), mr.reqs, ctypes.byref(info)))
    sizes = {"tok": info.n_branch, "pos": info.n_branch, "req": info.n_branch, "field": info.n_branch,
             "anc_off": info.n_branch + 1, "anc": info.n_anc, "ro_tok": info.n_readouts,
             "ro_field": info.n_readouts, "g_off": info.n_readouts + 1, "g_tok": info.n_gathers,
             "f_ro_root": info.n_fields, "f_cand_off": info.n_fields + 1, "f_mode": info.n_fields,
             "c_spell_off": info.n_candidates + 1, "s_path_off": info.n_spellings + 1, "s_path": info.n_paths}
    out = {k: np.zeros(max(1, n), np.int32) for k, n in sizes.items()}
    for k in _PLAN_ARRAYS:
        setattr(info, k, _i32p(out[k]))
    _check(lib.pcd_debug_plan(vocab_size, max_seq, len(requests), _i32p(lens), mr.reqs, ctypes.byref(info)))
    return {k: out[k][:sizes[k]] for k in _PLAN_ARRAYS}


def config_of(shape, max_seq: Optional[int] = None) -> dict:
    """pcd_config fields of a model-shape record (attributes named as in
    pcd_config; `tied` and `dtype` in "f32"/"bf16" form)."""
    return dict(n_layers=shape.n_layers, d_model=shape.d_model, n_heads=shape.n_heads, n_kv_heads=shape.n_kv_heads,
                head_dim=shape.head_dim, ffn_dim=shape.ffn_dim, vocab_size=shape.vocab_size,
                max_seq=max_seq or shape.max_seq, rope_theta=shape.rope_theta, rms_eps=shape.rms_eps,
                tied_lm_head=int(shape.tied), dtype=DTYPE_F32 if shape.dtype == "f32" else DTYPE_BF16)


def limits_for(vocab_size: int, max_seq: int, prefix_lens: Sequence[int], requests, max_prefill: int = 0) -> dict:
    """pcd_limits that fit exactly these requests (counts from the plan)."""
    p = debug_plan(vocab_size, max_seq, prefix_lens, requests)
    return dict(max_prefill_tokens=max(max_prefill, max(prefix_lens)), max_branch_tokens=len(p["tok"]),
                max_readouts=len(p["ro_tok"]), max_gathers=len(p["g_tok"]), max_fields=len(p["f_ro_root"]),
                max_candidates=len(p["c_spell_off"]) - 1, max_requests=len(prefix_lens),
                max_spellings=len(p["s_path_off"]) - 1)


def _stream_handle(torch):
    return c_void_p(torch.cuda.current_stream().cuda_stream)


def upload_weights(mats: Dict[str, np.ndarray], n_layers: int, d_model: int, device="cuda:0"):
    """Copies host weight arrays (float32, or uint16 bf16 patterns) to the
    device and adds all-ones fp32 norm weights.  Returns name -> tensor."""
    import torch
    out = {}
    for k, a in mats.items():
        t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
        out[k] = t.to(device)
    ones = torch.ones(d_model, dtype=torch.float32, device=device)
    out["final_norm"] = ones
    for l in range(n_layers):
        out[f"l{l}.attn_norm"] = ones
        out[f"l{l}.mlp_norm"] = ones
    return out


class PcdState:
    """A prefilled prefix over a torch-allocated KV buffer (`kv`)."""

    def __init__(self, model: "PcdModel", handle: c_void_p, kv, n_tokens: int):
        self.model, self.handle, self.kv, self.n_tokens = model, handle, kv, n_tokens
        model._states.add(self)

    def extend(self, tokens: Sequence[int]) -> "PcdState":
        """pcd_extend: append tokens (the buffer must have the capacity)."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        _check(self.model.lib.pcd_extend(self.handle, _i32p(t), t.size, _stream_handle(self.model.torch)))
        self.n_tokens = int(self.model.lib.pcd_state_tokens(self.handle))
        return self

    def fork(self, capacity: Optional[int] = None, kv=None) -> "PcdState":
        """pcd_fork: a copy of this state's tokens in a new buffer of `capacity` tokens."""
        m = self.model
        if kv is None:
            kv = m.torch.empty(max(m.state_bytes(capacity or self.n_tokens), 1), dtype=m.torch.uint8,
                               device=m.device)
        h = c_void_p()
        _check(m.lib.pcd_fork(self.handle, c_void_p(kv.data_ptr()), kv.numel(), _stream_handle(m.torch),
                              ctypes.byref(h)))
        return PcdState(m, h, kv, self.n_tokens)

    def close(self):
        if self.handle:
            load_library().pcd_free_state(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class PendingDecide:
    """A started extend_decide call: finish() waits for it and returns its
    results (the arrays the library fills)."""

    def __init__(self, model: "PcdModel", handle: c_void_p, result: dict):
        self.model, self.handle, self.result = model, handle, result
        model._pending.add(self)

    def finish(self) -> dict:
        if self.handle is None:
            raise RuntimeError("already finished")
        h, self.handle = self.handle, None
        self.model._pending.discard(self)
        _check(self.model.lib.pcd_finish(h))
        return self.result

    def __del__(self):
        if getattr(self, "handle", None) is not None:
            try:
                self.model.lib.pcd_finish(self.handle)
            except Exception:
                pass


NOALLOC_WORKSPACE_MAX = 128 << 20  # PCD_NOALLOC_WORKSPACE_MAX


class PcdModel:
    """A model over device weights (torch tensors) and a torch-allocated
    workspace (or, with noalloc=True, the library's static workspace:
    pcd_load_weights_noalloc).  `config` holds the pcd_config fields,
    `limits` the pcd_limits fields."""

    def __init__(self, config: dict, weights: Dict[str, "object"], limits: dict, noalloc: bool = False):
        import torch
        self.torch = torch
        self.lib = load_library()
        self._pending = weakref.WeakSet()  # started, unfinished calls (PendingDecide)
        self._states = weakref.WeakSet()   # open states (PcdState)
        self.cfg = pcd_config(**config)
        self.lim = pcd_limits(**limits)
        L = self.cfg.n_layers
        self.weights = weights
        arr = lambda name: (c_void_p * L)(*[weights[f"l{l}.{name}"].data_ptr() for l in range(L)])
        self._arrays = {n: arr(n) for n in ("attn_norm", "mlp_norm", "wq", "wk", "wv", "wo", "w_gate", "w_up",
                                             "w_down")}
        w = pcd_weights()
        w.embed = weights["embed"].data_ptr()
        w.lm_head = weights["lm_head"].data_ptr() if "lm_head" in weights else None
        w.final_norm = weights["final_norm"].data_ptr()
        for n, a in self._arrays.items():
            setattr(w, n, a)
        self.device = weights["embed"].device
        h = c_void_p()
        if noalloc:
            self.workspace = None
            _check(self.lib.pcd_load_weights_noalloc(ctypes.byref(self.cfg), ctypes.byref(self.lim), ctypes.byref(w),
                                                     _stream_handle(torch), ctypes.byref(h)))
        else:
            nbytes = self.lib.pcd_workspace_bytes(ctypes.byref(self.cfg), ctypes.byref(self.lim))
            if nbytes == 0:
                raise PcdError(-1, self.lib.pcd_last_error().decode())
            self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            _check(self.lib.pcd_load_weights(ctypes.byref(self.cfg), ctypes.byref(self.lim), ctypes.byref(w),
                                             c_void_p(self.workspace.data_ptr()), nbytes, _stream_handle(torch),
                                             ctypes.byref(h)))
        self.handle = h

    def state_bytes(self, n_tokens: int) -> int:
        return self.lib.pcd_state_bytes(self.handle, n_tokens)

    def prefill(self, tokens: Sequence[int], kv=None, capacity: Optional[int] = None) -> PcdState:
        """pcd_prefill into `kv` (or a new buffer of `capacity` tokens, default the prefix length)."""
        torch = self.torch
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        nb = self.state_bytes(max(t.size, capacity or 0))
        if kv is None:
            kv = torch.empty(max(nb, 1), dtype=torch.uint8, device=self.device)
        h = c_void_p()
        _check(self.lib.pcd_prefill(self.handle, _i32p(t), t.size, c_void_p(kv.data_ptr()), kv.numel(),
                                    _stream_handle(torch), ctypes.byref(h)))
        return PcdState(self, h, kv, t.size)

    def prefill_many(self, seqs: Sequence[Sequence[int]], kvs=None) -> List[PcdState]:
        """pcd_prefill_many: every sequence prefilled in one pass, each into its
        own buffer (`kvs`, or new buffers of exactly its length)."""
        torch = self.torch
        arrs = [np.ascontiguousarray(q, dtype=np.int32) for q in seqs]
        toks = np.ascontiguousarray(np.concatenate(arrs) if arrs else np.zeros(0, np.int32), dtype=np.int32)
        lens = np.ascontiguousarray([a.size for a in arrs], dtype=np.int32)
        if kvs is None:
            kvs = [torch.empty(max(self.state_bytes(a.size), 1), dtype=torch.uint8, device=self.device)
                   for a in arrs]
        n = len(arrs)
        bufs = (c_void_p * max(1, n))(*[kv.data_ptr() for kv in kvs])
        sizes = (c_size_t * max(1, n))(*[kv.numel() for kv in kvs])
        hs = (c_void_p * max(1, n))()
        _check(self.lib.pcd_prefill_many(self.handle, n, _i32p(toks), _i32p(lens), bufs, sizes,
                                         _stream_handle(torch), hs))
        return [PcdState(self, c_void_p(hs[i]), kvs[i], int(lens[i])) for i in range(n)]

    @staticmethod
    def compile_fields(fields) -> CompiledFields:
        """Marshal a schema once for repeated decide calls."""
        return CompiledFields(fields)

    def decide(self, state: PcdState, fields, temperature: float = 1.0, debug: bool = False) -> dict:
        return self.decide_many([state], [fields], temperature, debug)[0]

    def new_state(self, capacity: int, kv=None) -> PcdState:
        """pcd_new_state: an empty state whose buffer holds `capacity` tokens."""
        torch = self.torch
        if kv is None:
            kv = torch.empty(max(self.state_bytes(capacity), 1), dtype=torch.uint8, device=self.device)
        h = c_void_p()
        _check(self.lib.pcd_new_state(self.handle, c_void_p(kv.data_ptr()), kv.numel(), ctypes.byref(h)))
        return PcdState(self, h, kv, 0)

    def extend_decide(self, state: PcdState, tokens: Sequence[int], fields, temperature: float = 1.0,
                      debug: bool = False) -> dict:
        """pcd_extend_decide: append tokens and decide the fields in one pass."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        mr = _Marshalled([fields])
        d, o = self._outputs(mr, 0, [fields], state.n_tokens + t.size if debug else None)
        rq = mr.reqs[0]
        _check(self.lib.pcd_extend_decide(state.handle, _i32p(t), t.size, rq.fields, rq.n_fields, rq.candidates,
                                          rq.n_candidates, temperature, ctypes.byref(o),
                                          _stream_handle(self.torch)))
        state.n_tokens = int(self.lib.pcd_state_tokens(state.handle))
        return d

    def extend_decide_start(self, state: PcdState, tokens: Sequence[int], fields,
                            temperature: float = 1.0) -> "PendingDecide":
        """pcd_extend_decide_start: enqueue the same work as extend_decide and
        return at once; PendingDecide.finish() waits and returns the results."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        mr = _Marshalled([fields])
        d, o = _result_arrays(mr.n_cands[0], mr.n_fields[0])
        rq = mr.reqs[0]
        h = c_void_p()
        _check(self.lib.pcd_extend_decide_start(state.handle, _i32p(t), t.size, rq.fields, rq.n_fields,
                                                rq.candidates, rq.n_candidates, temperature, ctypes.byref(o),
                                                _stream_handle(self.torch), ctypes.byref(h)))
        state.n_tokens = int(self.lib.pcd_state_tokens(state.handle))
        return PendingDecide(self, h, d)

    def _outputs(self, mr, r, requests, debug_prefix):
        """Result arrays of request r and their pcd_outputs view (debug: sized
        from the plan at a prefix of debug_prefix tokens)."""
        d, o = _result_arrays(mr.n_cands[r], mr.n_fields[r])
        if debug_prefix is not None:
            plan = debug_plan(self.cfg.vocab_size, self.cfg.max_seq, [debug_prefix], [requests[r]])
            _debug_arrays(d, o, len(plan["ro_tok"]), len(plan["g_tok"]))
        return d, o

    def decide_sequenced(self, state: PcdState, fields, n_first: int, temperature: float = 1.0) -> dict:
        """pcd_decide_sequenced: the first n_first fields, their answers appended
        to the state, then the rest; results indexed as for decide()."""
        mr = _Marshalled([fields])
        d, o = _result_arrays(mr.n_cands[0], mr.n_fields[0])
        rq = mr.reqs[0]
        _check(self.lib.pcd_decide_sequenced(state.handle, rq.fields, rq.n_fields, rq.candidates, rq.n_candidates,
                                             n_first, temperature, ctypes.byref(o), _stream_handle(self.torch)))
        state.n_tokens = int(self.lib.pcd_state_tokens(state.handle))
        return d

    def decide_many(self, states: Sequence[PcdState], requests, temperature: float = 1.0,
                    debug: bool = False) -> List[dict]:
        mr = _Marshalled(requests)
        counts = None
        if debug:
            plan = debug_plan(self.cfg.vocab_size, self.cfg.max_seq, [s.n_tokens for s in states], requests)
            counts = []
            ro_req = plan["req"][plan["ro_tok"]]
            g_req = np.repeat(ro_req, np.diff(plan["g_off"]))
            for r in range(len(states)):
                counts.append((int((ro_req == r).sum()), int((g_req == r).sum())))
        outs = (pcd_outputs * len(states))()
        res = []
        for r in range(len(states)):
            d, o = _result_arrays(mr.n_cands[r], mr.n_fields[r], outs[r])
            if debug:
                _debug_arrays(d, o, counts[r][0], counts[r][1])
            res.append(d)
        hs = (c_void_p * len(states))(*[s.handle for s in states])
        _check(self.lib.pcd_decide_many(hs, mr.reqs, len(states), temperature, outs, _stream_handle(self.torch)))
        for r, d in enumerate(res):
            if debug:
                d["lse"] = d["lse"][:counts[r][0]]
                d["z"] = d["z"][:counts[r][1]]
        return res

    def stats(self) -> dict:
        s = pcd_stats()
        _check(self.lib.pcd_get_stats(self.handle, ctypes.byref(s)))
        return {k: getattr(s, k) for k, _ in pcd_stats._fields_}

    def set_kernel_timing(self, enable: bool):
        _check(self.lib.pcd_set_kernel_timing(self.handle, int(bool(enable))))

    def kernel_times(self) -> Dict[str, tuple]:
        """class -> (total ms, launches) since timing was enabled."""
        n = len(KERNEL_CLASSES)
        ms = (c_float * n)()
        cnt = (c_int64 * n)()
        _check(self.lib.pcd_get_kernel_times(self.handle, ms, cnt))
        return {k: (float(ms[i]), int(cnt[i])) for i, k in enumerate(KERNEL_CLASSES)}

    def close(self):
        if getattr(self, "handle", None):
            # the library's handles of started calls point into the model
            for p in list(self._pending):
                if p.handle is not None:
                    h, p.handle = p.handle, None
                    self.lib.pcd_finish(h)
            self._pending.clear()
            # the library frees states before their model
            for st in list(self._states):
                st.close()
            self.lib.pcd_free_model(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
