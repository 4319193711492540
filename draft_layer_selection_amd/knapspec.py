"""ctypes binding of libknapspec.so (the C ABI in include/knapspec.h).

Argument marshalling only: every step of the DP runs in the library's HIP kernels.  The
functions keep the C names; ``Model`` is a convenience wrapper that fills the C structs from
torch tensors (device memory and streams come from PyTorch, nothing else does).
If the shared library is missing this module raises on import: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import math
import os
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("KNAPSPEC_LIB", os.path.join(_HERE, "libknapspec.so"))

KNAPSPEC_OK = 0
KNAPSPEC_EINVAL = -1
KNAPSPEC_ENOMEM = -2
KNAPSPEC_EHIP = -3
KNAPSPEC_EUNSUPPORTED = -4
KNAPSPEC_F32 = 0
KNAPSPEC_BF16 = 1
KNAPSPEC_RETURN_DECISIONS = 1
KNAPSPEC_RETURN_MARGINS = 2
KNAPSPEC_ALPHA_LM_HEAD = 4
KNAPSPEC_KEEP_PRUNED_ROWS = 8
KNAPSPEC_WINDOW_MAX = 16
KNAPSPEC_BEAM_MAX = 8
KERNEL_CLASSES = ["init", "gemm_qkv", "qkv_rope", "attention", "combine", "gemm_o",
                  "gemm_gate_up", "gemm_down", "select", "lm_head"]


class knapspec_model_desc(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("d_ff", C.c_int32),
                ("dtype", C.c_int32), ("rms_eps", C.c_float), ("rope_theta", C.c_float),
                ("max_budgets", C.c_int32), ("max_seqs", C.c_int32), ("max_ctx", C.c_int32),
                ("max_window", C.c_int32), ("max_beam", C.c_int32)]


class knapspec_layer_weights(C.Structure):
    _fields_ = [("w_qkv", C.c_void_p), ("w_o", C.c_void_p), ("w_gate_up", C.c_void_p),
                ("w_down", C.c_void_p)]


class knapspec_latency_model(C.Structure):
    _fields_ = [("attn_base", C.c_double), ("attn_per_token", C.c_double), ("mlp", C.c_double),
                ("fixed", C.c_double), ("per_item", C.POINTER(C.c_double))]


class knapspec_seq(C.Structure):
    _fields_ = [("ctx_len", C.c_int32), ("ctx_capacity", C.c_int32),
                ("k_cache", C.POINTER(C.c_void_p)), ("v_cache", C.POINTER(C.c_void_p)),
                ("x0", C.c_void_p), ("window", C.c_int32)]


class knapspec_solve_args(C.Structure):
    _fields_ = [("n_seqs", C.c_int32), ("seqs", C.POINTER(knapspec_seq)),
                ("n_budgets", C.c_int32), ("gamma_min", C.c_int32), ("gamma_max", C.c_int32),
                ("tau", C.c_float), ("max_skip_weight", C.c_int32), ("flags", C.c_int32),
                ("hip_stream", C.c_void_p), ("beam", C.c_int32)]


class knapspec_result(C.Structure):
    _fields_ = [("masks", C.POINTER(C.c_uint64)), ("cos", C.POINTER(C.c_float)),
                ("valid", C.POINTER(C.c_uint8)), ("t_draft", C.POINTER(C.c_double)),
                ("item_weight", C.POINTER(C.c_int32)), ("best_budget", C.POINTER(C.c_int32)),
                ("best_gamma", C.POINTER(C.c_int32)), ("best_tpt", C.POINTER(C.c_double)),
                ("decisions", C.POINTER(C.c_uint8)), ("margins", C.POINTER(C.c_float)),
                ("alpha", C.POINTER(C.c_float)), ("tokens", C.POINTER(C.c_int32))]


# symbol -> (restype, argtypes); every entry point of include/knapspec.h
SIGNATURES = {
    "knapspec_load_model": (C.c_int, [C.POINTER(knapspec_model_desc),
                                      C.POINTER(knapspec_layer_weights), C.c_void_p,
                                      C.POINTER(C.c_void_p)]),
    "knapspec_set_latency_model": (C.c_int, [C.c_void_p, C.POINTER(knapspec_latency_model)]),
    "knapspec_solve": (C.c_int, [C.c_void_p, C.POINTER(knapspec_solve_args),
                                 C.POINTER(knapspec_result)]),
    "knapspec_solve_static": (C.c_int, [C.c_void_p, C.POINTER(knapspec_solve_args),
                                        C.POINTER(knapspec_result)]),
    "knapspec_tpt_select": (C.c_int, [C.POINTER(C.c_float), C.POINTER(C.c_double),
                                      C.POINTER(C.c_uint8), C.c_int32, C.c_double, C.c_int32,
                                      C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_int32),
                                      C.POINTER(C.c_double)]),
    "knapspec_item_weights": (C.c_int, [C.POINTER(knapspec_latency_model), C.c_int32, C.c_int32,
                                        C.c_int32, C.POINTER(C.c_double),
                                        C.POINTER(C.c_int32)]),
    "knapspec_gemm_plan": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                     C.c_int32, C.c_int64, C.POINTER(C.c_int32)]),
    "knapspec_set_profiling": (C.c_int, [C.c_void_p, C.c_int32]),
    "knapspec_get_kernel_times": (C.c_int, [C.c_void_p, C.POINTER(C.c_double),
                                            C.POINTER(C.c_int64), C.c_int32]),
    "knapspec_mask_words": (C.c_int32, [C.c_int32]),
    "knapspec_free_model": (None, [C.c_void_p]),
    "knapspec_last_error": (C.c_char_p, []),
    "knapspec_abi_version": (C.c_int32, []),
    "knapspec_profile_items": (C.c_int, [C.c_void_p, C.POINTER(knapspec_seq),
                                         C.POINTER(C.c_int32), C.c_int32, C.c_int32, C.c_void_p,
                                         C.POINTER(C.c_double), C.POINTER(C.c_double)]),
    "knapspec_fit_latency": (C.c_int, [C.POINTER(C.c_int32), C.POINTER(C.c_double), C.c_int32,
                                       C.POINTER(C.c_double), C.POINTER(C.c_double),
                                       C.POINTER(C.c_double)]),
    "knapspec_set_lm_head": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32]),
    "knapspec_draft_verify": (C.c_int, [C.c_void_p, C.POINTER(knapspec_seq),
                                        C.POINTER(C.c_uint64), C.c_int32, C.c_void_p,
                                        C.POINTER(C.c_int32), C.POINTER(C.c_int32),
                                        C.POINTER(C.c_int32), C.POINTER(C.c_double),
                                        C.POINTER(C.c_double)]),
}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first "
                      "(there is no CPU fallback)")
lib = C.CDLL(LIB_PATH)
for _name, (_res, _args) in SIGNATURES.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

knapspec_load_model = lib.knapspec_load_model
knapspec_set_latency_model = lib.knapspec_set_latency_model
knapspec_solve = lib.knapspec_solve
knapspec_solve_static = lib.knapspec_solve_static
knapspec_tpt_select = lib.knapspec_tpt_select
knapspec_item_weights = lib.knapspec_item_weights
knapspec_gemm_plan = lib.knapspec_gemm_plan
knapspec_set_profiling = lib.knapspec_set_profiling
knapspec_get_kernel_times = lib.knapspec_get_kernel_times
knapspec_mask_words = lib.knapspec_mask_words
knapspec_free_model = lib.knapspec_free_model
knapspec_last_error = lib.knapspec_last_error
knapspec_abi_version = lib.knapspec_abi_version
knapspec_profile_items = lib.knapspec_profile_items
knapspec_fit_latency = lib.knapspec_fit_latency
knapspec_set_lm_head = lib.knapspec_set_lm_head
knapspec_draft_verify = lib.knapspec_draft_verify


class KnapSpecError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = knapspec_last_error().decode(errors="replace")
        super().__init__(f"{where} failed with {code}: {msg}")
        self.code = code


def _check(rc: int, where: str):
    if rc != KNAPSPEC_OK:
        raise KnapSpecError(rc, where)


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(C.POINTER(ctype))


def latency_struct(attn_base, attn_per_token, mlp, fixed=0.0, per_item=None):
    lat = knapspec_latency_model(attn_base, attn_per_token, mlp, fixed, None)
    keep = None
    if per_item is not None:
        keep = np.ascontiguousarray(per_item, dtype=np.float64)
        lat.per_item = _ptr(keep, C.c_double)
    return lat, keep


def tpt_select(alpha, t_draft, valid, t_target, gamma_min, gamma_max):
    """knapspec_tpt_select on numpy arrays -> (best_budget, best_gamma, best_tpt)."""
    a = np.ascontiguousarray(alpha, dtype=np.float32)
    t = np.ascontiguousarray(t_draft, dtype=np.float64)
    v = np.ascontiguousarray(valid, dtype=np.uint8)
    bb, bg, bt = C.c_int32(), C.c_int32(), C.c_double()
    _check(knapspec_tpt_select(_ptr(a, C.c_float), _ptr(t, C.c_double), _ptr(v, C.c_uint8),
                               len(a), float(t_target), int(gamma_min), int(gamma_max),
                               C.byref(bb), C.byref(bg), C.byref(bt)), "knapspec_tpt_select")
    return bb.value, bg.value, bt.value


def item_weights(n_layers, ctx, n_budgets, attn_base, attn_per_token, mlp, fixed=0.0,
                 per_item=None):
    lat, keep = latency_struct(attn_base, attn_per_token, mlp, fixed, per_item)
    t = np.zeros(2 * n_layers, dtype=np.float64)
    w = np.zeros(2 * n_layers, dtype=np.int32)
    _check(knapspec_item_weights(C.byref(lat), n_layers, ctx, n_budgets, _ptr(t, C.c_double),
                                 _ptr(w, C.c_int32)), "knapspec_item_weights")
    return t, w


def gemm_plan(rows, n_cols, k, swiglu=False, d_ff=0, bf16=True, cap_floats=1 << 40):
    """knapspec_gemm_plan -> dict(ng, mb, m_tiles, n_tiles, splits, k_chunk, areg)."""
    out = (C.c_int32 * 8)()
    _check(knapspec_gemm_plan(int(bool(bf16)), rows, n_cols, k, int(bool(swiglu)), d_ff,
                              int(cap_floats), out), "knapspec_gemm_plan")
    return dict(zip(("ng", "mb", "m_tiles", "n_tiles", "splits", "k_chunk", "areg"), out[:7]))


def fit_latency(n, t):
    """knapspec_fit_latency: least-squares t = a + b*n -> (a, b, r2)."""
    nn = np.ascontiguousarray(n, dtype=np.int32)
    tt = np.ascontiguousarray(t, dtype=np.float64)
    a, b, r2 = C.c_double(), C.c_double(), C.c_double()
    _check(knapspec_fit_latency(_ptr(nn, C.c_int32), _ptr(tt, C.c_double), len(nn), C.byref(a),
                                C.byref(b), C.byref(r2)), "knapspec_fit_latency")
    return a.value, b.value, r2.value


class Result:
    """Host arrays of one solve (numpy views of what the library filled)."""

    def __init__(self, n_seqs, n_budgets, n_items, mw, flags, windows=None):
        self.masks = np.zeros((n_seqs, n_budgets, mw), dtype=np.uint64)
        self.cos = np.zeros((n_seqs, n_budgets), dtype=np.float32)
        self.valid = np.zeros((n_seqs, n_budgets), dtype=np.uint8)
        self.t_draft = np.zeros((n_seqs, n_budgets), dtype=np.float64)
        self.item_weight = np.zeros((n_seqs, n_items), dtype=np.int32)
        self.best_budget = np.zeros(n_seqs, dtype=np.int32)
        self.best_gamma = np.zeros(n_seqs, dtype=np.int32)
        self.best_tpt = np.zeros(n_seqs, dtype=np.float64)
        self.decisions = (np.zeros((n_seqs, n_items, n_budgets), dtype=np.uint8)
                          if flags & KNAPSPEC_RETURN_DECISIONS else None)
        self.margins = (np.zeros((n_seqs, n_items, n_budgets), dtype=np.float32)
                        if flags & KNAPSPEC_RETURN_MARGINS else None)
        self.alpha = np.zeros((n_seqs, n_budgets), dtype=np.float32)
        self.windows = [1] * n_seqs if windows is None else [max(1, int(w)) for w in windows]
        # per sequence (n_budgets + 1) x window token ids, flat in sequence order
        self.tokens_flat = np.full(sum((n_budgets + 1) * w for w in self.windows), -1,
                                   dtype=np.int32)
        self.struct = knapspec_result(
            _ptr(self.masks, C.c_uint64), _ptr(self.cos, C.c_float), _ptr(self.valid, C.c_uint8),
            _ptr(self.t_draft, C.c_double), _ptr(self.item_weight, C.c_int32),
            _ptr(self.best_budget, C.c_int32), _ptr(self.best_gamma, C.c_int32),
            _ptr(self.best_tpt, C.c_double),
            _ptr(self.decisions, C.c_uint8) if self.decisions is not None else None,
            _ptr(self.margins, C.c_float) if self.margins is not None else None,
            _ptr(self.alpha, C.c_float), _ptr(self.tokens_flat, C.c_int32))

    def tokens(self, q: int) -> np.ndarray:
        """[n_budgets + 1][window] greedy tokens of sequence q (row n_budgets: full model)."""
        B = self.alpha.shape[1]
        off = sum((B + 1) * w for w in self.windows[:q])
        w = self.windows[q]
        return self.tokens_flat[off:off + (B + 1) * w].reshape(B + 1, w)


class PreparedSeqs:
    """A knapspec_seq array (device pointers, context lengths, windows) built from a list of
    sequence dicts; keeps the ctypes arrays alive."""

    def __init__(self, model: "Model", seqs: List[dict]):
        self.carr, self._keep = model._seq_array(seqs)
        self.n = len(seqs)
        self.windows = [int(sq.get("window", 1)) for sq in seqs]
        self._tensors = seqs  # the tensors whose pointers the array holds


class Model:
    """Owns a knapspec_model handle built from torch device tensors (kept alive here)."""

    def __init__(self, desc: dict, layers: Sequence[dict], stream=None):
        import torch

        self._torch = torch
        self.desc = knapspec_model_desc(**desc)
        self.n_layers = self.desc.n_layers
        self.mw = int(knapspec_mask_words(self.n_layers))
        self._layers = list(layers)  # keep tensors alive
        arr = (knapspec_layer_weights * self.n_layers)()
        for i, lw in enumerate(layers):
            arr[i] = knapspec_layer_weights(lw["w_qkv"].data_ptr(), lw["w_o"].data_ptr(),
                                            lw["w_gate_up"].data_ptr(), lw["w_down"].data_ptr())
        h = C.c_void_p()
        s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
        _check(knapspec_load_model(C.byref(self.desc), arr, C.c_void_p(s), C.byref(h)),
               "knapspec_load_model")
        self.handle = h

    def set_latency(self, attn_base, attn_per_token, mlp, fixed=0.0, per_item=None):
        lat, keep = latency_struct(attn_base, attn_per_token, mlp, fixed, per_item)
        _check(knapspec_set_latency_model(self.handle, C.byref(lat)),
               "knapspec_set_latency_model")

    def _seq_array(self, seqs: List[dict]):
        carr = (knapspec_seq * len(seqs))()
        keep = []
        for i, sq in enumerate(seqs):
            kp = (C.c_void_p * self.n_layers)(*[t.data_ptr() for t in sq["k_cache"]])
            vp = (C.c_void_p * self.n_layers)(*[t.data_ptr() for t in sq["v_cache"]])
            keep += [kp, vp]
            cap = int(sq["k_cache"][0].shape[1]) if self.n_layers else 0
            carr[i] = knapspec_seq(int(sq["ctx"]), cap, C.cast(kp, C.POINTER(C.c_void_p)),
                                   C.cast(vp, C.POINTER(C.c_void_p)), sq["x0"].data_ptr(),
                                   int(sq.get("window", 1)))
        return carr, keep

    def prepare(self, seqs: List[dict]) -> "PreparedSeqs":
        """The knapspec_seq array of ``seqs`` built once, for repeated solves over the same
        tensors (the pointers are read now; the tensors' contents may change between solves)."""
        return PreparedSeqs(self, seqs)

    def solve(self, seqs, n_budgets: int, gamma, tau: float = -math.inf,
              max_skip_weight: int = -1, flags: int = 0, stream=None,
              result: Optional[Result] = None, beam: int = 1,
              static_scratch: bool = False) -> Result:
        """seqs: dicts with ctx (int), k_cache / v_cache (lists of device tensors per layer,
        [hkv][capacity][dh]), x0 (device float32 [window][d] or [d]) and optionally window
        (int, default 1); or a PreparedSeqs of such a list.  static_scratch: call
        knapspec_solve_static (per-solve device buffers in the library's static scratch;
        allocates nothing)."""
        torch = self._torch
        prep = seqs if isinstance(seqs, PreparedSeqs) else PreparedSeqs(self, seqs)
        S = prep.n
        s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
        args = knapspec_solve_args(S, prep.carr, int(n_budgets), int(gamma[0]), int(gamma[1]),
                                   float(tau), int(max_skip_weight), int(flags), C.c_void_p(s),
                                   int(beam))
        res = result if result is not None else Result(
            S, n_budgets, 2 * self.n_layers, self.mw, flags, windows=prep.windows)
        fn, name = ((knapspec_solve_static, "knapspec_solve_static") if static_scratch
                    else (knapspec_solve, "knapspec_solve"))
        _check(fn(self.handle, C.byref(args), C.byref(res.struct)), name)
        return res

    def profile_items(self, seq: dict, ctx_lens, reps: int = 8, stream=None):
        """knapspec_profile_items: median microseconds of one token through an Attention item
        at each context length in ctx_lens, and through an MLP item -> (attn_us, mlp_us)."""
        torch = self._torch
        carr, keep = self._seq_array([seq])
        n = np.ascontiguousarray(ctx_lens, dtype=np.int32)
        attn = np.zeros(len(n), dtype=np.float64)
        mlp = C.c_double()
        s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
        _check(knapspec_profile_items(self.handle, carr, _ptr(n, C.c_int32), len(n), int(reps),
                                      C.c_void_p(s), _ptr(attn, C.c_double), C.byref(mlp)),
               "knapspec_profile_items")
        return attn, mlp.value

    def set_lm_head(self, w, vocab: int):
        """knapspec_set_lm_head: w is a device tensor [vocab][d] in the model dtype (kept alive
        here)."""
        self._lm_head = w
        _check(knapspec_set_lm_head(self.handle, C.c_void_p(w.data_ptr()), int(vocab)),
               "knapspec_set_lm_head")

    def draft_verify(self, seq: dict, mask: np.ndarray, gamma: int, stream=None):
        """knapspec_draft_verify: mask uint64 [ceil(2L/64)] -> dict(draft [gamma], verify
        [gamma+1], accepted, draft_us, verify_us).  Writes seq's caches at ctx .. ctx+gamma."""
        torch = self._torch
        carr, keep = self._seq_array([seq])
        mk = np.ascontiguousarray(mask, dtype=np.uint64)
        dt = np.zeros(gamma, dtype=np.int32)
        vt = np.zeros(gamma + 1, dtype=np.int32)
        acc = C.c_int32()
        dus, vus = C.c_double(), C.c_double()
        s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
        _check(knapspec_draft_verify(self.handle, carr, _ptr(mk, C.c_uint64), int(gamma),
                                     C.c_void_p(s), _ptr(dt, C.c_int32), _ptr(vt, C.c_int32),
                                     C.byref(acc), C.byref(dus), C.byref(vus)),
               "knapspec_draft_verify")
        return {"draft": dt, "verify": vt, "accepted": acc.value, "draft_us": dus.value,
                "verify_us": vus.value}

    def set_profiling(self, enable: bool):
        _check(knapspec_set_profiling(self.handle, 1 if enable else 0), "knapspec_set_profiling")

    def kernel_times(self) -> dict:
        n = len(KERNEL_CLASSES)
        ms = (C.c_double * n)()
        cnt = (C.c_int64 * n)()
        _check(knapspec_get_kernel_times(self.handle, ms, cnt, n), "knapspec_get_kernel_times")
        return {k: (ms[i], cnt[i]) for i, k in enumerate(KERNEL_CLASSES)}

    def close(self):
        if getattr(self, "handle", None):
            knapspec_free_model(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
