"""ctypes front end of the scalar-C oracle (``mtp_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the HIP library; both sides are fed the same arrays built by
``mtp_speculative_draft_amd.synth``.

Every function takes and returns numpy arrays; the C side accumulates in
double and stores f32 between steps.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mtp_oracle.c")
_HDR = os.path.join(_HERE, "mtp_oracle.h")
LIB_PATH = os.path.join(_HERE, "liboracle.so")
# the same source built with OpenMP: the independent output elements of the
# GEMVs and attention heads are shared out over threads, every element keeping
# its own ascending double sum, so its results equal the plain build's bit for
# bit (used only to time the oracle on all host cores)
LIB_OMP_PATH = os.path.join(_HERE, "liboracle_omp.so")
_libs = {}
_threaded = False


def _build_one(path: str, extra, force: bool) -> str:
    stale = (not os.path.exists(path) or
             os.path.getmtime(path) < max(os.path.getmtime(_SRC), os.path.getmtime(_HDR)))
    if force or stale:
        tmp = path + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-Wall", "-Wno-unknown-pragmas", *extra, "-fPIC", "-shared",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, path)
    return path


def build(force: bool = False) -> str:
    """Compile liboracle.so (gcc -O2 -std=c99, no fast-math) and its OpenMP twin."""
    _build_one(LIB_OMP_PATH, ["-fopenmp"], force)
    return _build_one(LIB_PATH, [], force)


def set_threaded(flag: bool) -> None:
    """Route every following call to the OpenMP build (True) or the plain one."""
    global _threaded
    _threaded = bool(flag)


class _Q4(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("biases", C.c_void_p),
                ("n", C.c_int32), ("k", C.c_int32)]


class _Q8(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("n", C.c_int32), ("k", C.c_int32)]


class _Q4E(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("biases", C.c_void_p),
                ("n", C.c_int32), ("k", C.c_int32)]


class _Layer(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("vocab", C.c_int32), ("ffn_inter", C.c_int32),
                ("rope_theta", C.c_double), ("eps", C.c_float),
                ("gamma_e", C.c_void_p), ("gamma_h", C.c_void_p), ("gamma_attn", C.c_void_p),
                ("gamma_post", C.c_void_p), ("gamma_final", C.c_void_p),
                ("eh_proj", _Q4), ("wq", _Q4), ("wk", _Q4), ("wv", _Q4), ("wo", _Q4),
                ("gate", _Q4), ("up", _Q4), ("down", _Q4), ("lm_head", _Q4),
                ("gamma_q_head", C.c_void_p), ("gamma_k_head", C.c_void_p),
                ("q_gated", C.c_int32), ("rotary_dim", C.c_int32),
                ("sinks", C.c_void_p), ("window", C.c_int32), ("v_head_dim", C.c_int32),
                ("mrope_section", C.c_int32 * 4), ("positions", C.c_void_p)]


class _MoeFfn(C.Structure):
    _fields_ = [("router", C.c_void_p), ("n_experts", C.c_int32), ("top_k", C.c_int32),
                ("gate_exps", C.c_void_p), ("up_exps", C.c_void_p), ("down_exps", C.c_void_p),
                ("sh_gate", C.c_void_p), ("sh_up", C.c_void_p), ("sh_down", C.c_void_p),
                ("q4", C.c_int32),
                ("gate_exps4", C.c_void_p), ("up_exps4", C.c_void_p), ("down_exps4", C.c_void_p),
                ("sh_gate4", C.c_void_p), ("sh_up4", C.c_void_p), ("sh_down4", C.c_void_p)]


def lib():
    key = "omp" if _threaded else "plain"
    _lib = _libs.get(key)
    if _lib is None:
        build()
        _lib = C.CDLL(LIB_OMP_PATH if _threaded else LIB_PATH)
        _libs[key] = _lib
        P, I = C.c_void_p, C.c_int32
        sig = {
            "orc_unpack4": (None, [P, I, I, P]),
            "orc_deq4": (None, [P, P]),
            "orc_deq8": (None, [P, P]),
            "orc_bf16": (C.c_float, [C.c_uint16]),
            "orc_deq4e": (None, [P, P]),
            "orc_gemv4e": (None, [P, P, I, P]),
            "orc_moe4": (I, [P, P, I, I, P, P, P, P, P, P, P, I, P, P, P, P]),
            "orc_gemv4": (None, [P, P, I, P]),
            "orc_gemv8": (None, [P, P, I, P]),
            "orc_gemv_f32": (None, [P, I, I, P, I, P]),
            "orc_rmsnorm": (None, [P, P, I, I, C.c_float, P]),
            "orc_rope": (None, [P, I, I, I, I, C.c_double]),
            "orc_rope_partial": (None, [P, I, I, I, I, I, C.c_double]),
            "orc_imrope_section": (I, [I, P]),
            "orc_rope_sections": (None, [P, I, I, I, I, P, P, C.c_double]),
            "orc_sdpa": (None, [P, P, P, I, I, I, I, I, I, P]),
            "orc_sdpa_window": (None, [P, P, P, I, I, I, I, I, I, I, P, P]),
            "orc_sdpa_kv": (None, [P, P, P, I, I, I, I, I, I, I, I, P, P]),
            "orc_argmax": (I, [P, I]),
            "orc_norm_concat_proj": (None, [P, P, P, P, C.c_float, P, I, P]),
            "orc_attention": (None, [P, P, P, P, I, I, I, P]),
            "orc_ffn_dense": (None, [P, P, P, P, P, I, P]),
            "orc_moe": (I, [P, P, I, I, P, P, P, P, P, P, P, I, P, P, P, P]),
            "orc_head": (None, [P, P, C.c_float, P, I, P, P, P]),
            "orc_head8": (None, [P, P, C.c_float, P, I, P, P, P]),
            "orc_draft_step": (I, [P, P, P, P, P, P, P, I, I, I, P, P, P]),
            "orc_draft_step_moe": (I, [P, P, P, P, P, P, P, P, I, I, I, P, P, P]),
            "orc_append_kv": (None, [P, P, P, P, P, P, P, P, I, I, I]),
        }
        for name, (res, args) in sig.items():
            f = getattr(_lib, name)
            f.restype = res
            f.argtypes = args
    return _lib


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------
def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


class _Keep:
    """Holds the contiguous copies alive while a C call runs."""

    def __init__(self):
        self.refs = []

    def arr(self, a, dtype):
        a = _c(a, dtype)
        self.refs.append(a)
        return a


def _q4(w, keep: _Keep) -> _Q4:
    c = keep.arr(w.codes, np.uint32)
    s = keep.arr(w.scales, np.float32)
    b = keep.arr(w.biases, np.float32)
    return _Q4(c.ctypes.data, s.ctypes.data, b.ctypes.data, w.n, w.k)


def _q8_list(w, keep: _Keep):
    """Array of per-expert _Q8 descriptors over an [E, n, k] stack."""
    c = keep.arr(w.codes, np.int8)
    s = keep.arr(w.scales, np.float32)
    E, n, k = c.shape
    arr = (_Q8 * E)()
    for e in range(E):
        arr[e] = _Q8(c.ctypes.data + e * n * k, s.ctypes.data + e * n * (k // 32) * 4, n, k)
    keep.refs.append(arr)
    return arr


def _q4e_list(w, keep: _Keep):
    """Array of per-expert _Q4E descriptors over an [E, n, k/8] stack."""
    c = keep.arr(w.codes, np.uint32)
    s = keep.arr(w.scales, np.uint16)
    b = keep.arr(w.biases, np.uint16)
    E, n, kw = c.shape
    g = kw * 8 // 32
    arr = (_Q4E * E)()
    for e in range(E):
        arr[e] = _Q4E(c.ctypes.data + e * n * kw * 4, s.ctypes.data + e * n * g * 2, b.ctypes.data + e * n * g * 2,
                      n, kw * 8)
    keep.refs.append(arr)
    return arr


def _experts(w, keep: _Keep):
    return _q4e_list(w, keep) if hasattr(w, "biases") and w.codes.ndim == 3 else _q8_list(w, keep)


def _layer(L, keep: _Keep, positions=None) -> _Layer:
    """The layer descriptor; positions (int32 [m, 4]) are the call's rotary
    position ids when given."""
    f = lambda a: keep.arr(a, np.float32).ctypes.data  # noqa: E731
    opt = lambda a: None if a is None else f(a)  # noqa: E731
    sec = (C.c_int32 * 4)(*[int(v) for v in (getattr(L, "mrope_section", None) or (0, 0, 0, 0))])
    pos = None if positions is None else keep.arr(np.asarray(positions).reshape(-1, 4), np.int32).ctypes.data
    return _Layer(L.hidden, L.n_heads, L.n_kv_heads, L.head_dim, L.vocab, L.ffn_inter,
                  float(L.rope_theta), float(L.eps),
                  f(L.gamma_e), f(L.gamma_h), f(L.gamma_attn), f(L.gamma_post), f(L.gamma_final),
                  _q4(L.eh_proj, keep), _q4(L.wq, keep), _q4(L.wk, keep), _q4(L.wv, keep), _q4(L.wo, keep),
                  _q4(L.gate, keep), _q4(L.up, keep), _q4(L.down, keep), _q4(L.lm_head, keep),
                  opt(getattr(L, "gamma_q_head", None)), opt(getattr(L, "gamma_k_head", None)),
                  int(bool(getattr(L, "q_gated", False))), int(getattr(L, "rotary_dim", 0) or 0),
                  opt(getattr(L, "sinks", None)), int(getattr(L, "window", 0) or 0),
                  int(getattr(L, "v_head_dim", 0) or 0), sec, pos)


# --------------------------------------------------------------------------
# public functions
# --------------------------------------------------------------------------
def unpack4(codes: np.ndarray, k: int) -> np.ndarray:
    codes = _c(codes, np.uint32)
    n = codes.shape[0]
    out = np.empty((n, k), dtype=np.uint8)
    lib().orc_unpack4(_p(codes), n, k, _p(out))
    return out


def deq4(w) -> np.ndarray:
    keep = _Keep()
    d = _q4(w, keep)
    out = np.empty((w.n, w.k), dtype=np.float32)
    lib().orc_deq4(C.byref(d), _p(out))
    return out


def deq8(w, expert: int = 0) -> np.ndarray:
    keep = _Keep()
    arr = _q8_list(w, keep)
    out = np.empty((w.n, w.k), dtype=np.float32)
    lib().orc_deq8(C.byref(arr[expert]), _p(out))
    return out


def bf16(bits) -> np.ndarray:
    """The f32 values of bf16 bit patterns (one C call each)."""
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib().orc_bf16(int(v)) for v in b], dtype=np.float32).reshape(np.shape(bits))


def deq4e(w, expert: int = 0) -> np.ndarray:
    keep = _Keep()
    arr = _q4e_list(w, keep)
    out = np.empty((w.n, w.k), dtype=np.float32)
    lib().orc_deq4e(C.byref(arr[expert]), _p(out))
    return out


def gemv4e(w, x: np.ndarray, expert: int = 0) -> np.ndarray:
    keep = _Keep()
    arr = _q4e_list(w, keep)
    x = keep.arr(np.atleast_2d(x), np.float32)
    y = np.empty((x.shape[0], w.n), dtype=np.float32)
    lib().orc_gemv4e(C.byref(arr[expert]), _p(x), x.shape[0], _p(y))
    return y


def gemv4(w, x: np.ndarray) -> np.ndarray:
    keep = _Keep()
    d = _q4(w, keep)
    x = keep.arr(np.atleast_2d(x), np.float32)
    y = np.empty((x.shape[0], w.n), dtype=np.float32)
    lib().orc_gemv4(C.byref(d), _p(x), x.shape[0], _p(y))
    return y


def gemv8(w, x: np.ndarray, expert: int = 0) -> np.ndarray:
    keep = _Keep()
    arr = _q8_list(w, keep)
    x = keep.arr(np.atleast_2d(x), np.float32)
    y = np.empty((x.shape[0], w.n), dtype=np.float32)
    lib().orc_gemv8(C.byref(arr[expert]), _p(x), x.shape[0], _p(y))
    return y


def gemv_f32(w: np.ndarray, x: np.ndarray) -> np.ndarray:
    w = _c(w, np.float32)
    x = _c(np.atleast_2d(x), np.float32)
    y = np.empty((x.shape[0], w.shape[0]), dtype=np.float32)
    lib().orc_gemv_f32(_p(w), w.shape[0], w.shape[1], _p(x), x.shape[0], _p(y))
    return y


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    x = _c(np.atleast_2d(x), np.float32)
    g = _c(gamma, np.float32)
    y = np.empty_like(x)
    lib().orc_rmsnorm(_p(x), _p(g), x.shape[0], x.shape[1], float(eps), _p(y))
    return y


def rope(x: np.ndarray, n_heads: int, head_dim: int, pos0: int, theta: float, rotary_dim: int = 0) -> np.ndarray:
    y = np.array(np.atleast_2d(x), dtype=np.float32, copy=True, order="C")
    if rotary_dim and rotary_dim != head_dim:
        lib().orc_rope_partial(_p(y), y.shape[0], n_heads, head_dim, int(rotary_dim), pos0, float(theta))
    else:
        lib().orc_rope(_p(y), y.shape[0], n_heads, head_dim, pos0, float(theta))
    return y


def imrope_section(pair: int, sections) -> int:
    sec = (C.c_int32 * 4)(*[int(v) for v in sections])
    return int(lib().orc_imrope_section(int(pair), sec))


def rope_sections(x: np.ndarray, n_heads: int, head_dim: int, rotary_dim: int, positions, sections,
                  theta: float) -> np.ndarray:
    """Rotary with four position ids per row (positions int32 [m, 4])."""
    y = np.array(np.atleast_2d(x), dtype=np.float32, copy=True, order="C")
    pos = _c(np.asarray(positions).reshape(-1, 4), np.int32)
    sec = _c(np.asarray(sections).reshape(4), np.int32)
    lib().orc_rope_sections(_p(y), y.shape[0], n_heads, head_dim, int(rotary_dim), _p(pos), _p(sec), float(theta))
    return y


def sdpa(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, n_heads: int, cache_len: int,
         window: int = 0, sinks: Optional[np.ndarray] = None) -> np.ndarray:
    """Causal GQA attention of q [m, n_heads*d] over the caches; window > 0
    keeps the last `window` positions per row, sinks [n_heads] join the softmax.
    The V cache may have its own row width dv (outputs [m, n_heads*dv])."""
    q = _c(np.atleast_2d(q), np.float32)
    kc = _c(k_cache, np.float32)
    vc = _c(v_cache, np.float32)
    nkv, cap, d = kc.shape
    dv = vc.shape[2]
    assert vc.shape[:2] == (nkv, cap)
    out = np.empty((q.shape[0], n_heads * dv), dtype=np.float32)
    sk = None if sinks is None else _c(sinks, np.float32)
    lib().orc_sdpa_kv(_p(q), _p(kc), _p(vc), q.shape[0], n_heads, nkv, d, dv, cache_len, cap, int(window), _p(sk),
                      _p(out))
    return out


def argmax(v: np.ndarray) -> int:
    v = _c(v, np.float32)
    return int(lib().orc_argmax(_p(v), v.size))


def norm_concat_proj(e, h, gamma_e, gamma_h, eps, w) -> np.ndarray:
    keep = _Keep()
    d = _q4(w, keep)
    e = keep.arr(np.atleast_2d(e), np.float32)
    h = keep.arr(np.atleast_2d(h), np.float32)
    ge, gh = keep.arr(gamma_e, np.float32), keep.arr(gamma_h, np.float32)
    u = np.empty((e.shape[0], w.n), dtype=np.float32)
    lib().orc_norm_concat_proj(_p(e), _p(h), _p(ge), _p(gh), float(eps), C.byref(d), e.shape[0], _p(u))
    return u


def attention(L, u, k_cache: np.ndarray, v_cache: np.ndarray, cache_len: int, positions=None) -> np.ndarray:
    """Attention block with residual; appends K/V rows into the given caches in
    place.  positions: the rows' four rotary position ids (int32 [m, 4])."""
    assert k_cache.flags.c_contiguous and k_cache.dtype == np.float32
    assert v_cache.flags.c_contiguous and v_cache.dtype == np.float32
    keep = _Keep()
    d = _layer(L, keep, positions)
    u = keep.arr(np.atleast_2d(u), np.float32)
    r1 = np.empty_like(u)
    lib().orc_attention(C.byref(d), _p(u), _p(k_cache), _p(v_cache), cache_len, k_cache.shape[1],
                        u.shape[0], _p(r1))
    return r1


def ffn_dense(x, gate, up, down, residual=None) -> np.ndarray:
    keep = _Keep()
    g, u, dn = _q4(gate, keep), _q4(up, keep), _q4(down, keep)
    x = keep.arr(np.atleast_2d(x), np.float32)
    res = None if residual is None else keep.arr(np.atleast_2d(residual), np.float32)
    y = np.empty((x.shape[0], down.n), dtype=np.float32)
    lib().orc_ffn_dense(_p(x), C.byref(g), C.byref(u), C.byref(dn), _p(res), x.shape[0], _p(y))
    return y


def moe(inp, x=None, residual=None):
    """Returns (y, expert_ids [m, top_k], gates [m, top_k], router_logits [m, E])."""
    keep = _Keep()
    x = keep.arr(np.atleast_2d(inp.x if x is None else x), np.float32)
    router = keep.arr(inp.router, np.float32)
    m, E, K = x.shape[0], inp.n_experts, inp.top_k
    ge, ue, de = _experts(inp.gate_exps, keep), _experts(inp.up_exps, keep), _experts(inp.down_exps, keep)
    if inp.sh_gate is not None:
        sg, su, sd = (C.byref(_experts(inp.sh_gate, keep)[0]), C.byref(_experts(inp.sh_up, keep)[0]),
                      C.byref(_experts(inp.sh_down, keep)[0]))
    else:
        sg = su = sd = None
    res = None if residual is None else keep.arr(np.atleast_2d(residual), np.float32)
    y = np.empty((m, inp.gate_exps.k), dtype=np.float32)
    ids = np.empty((m, K), dtype=np.int32)
    gates = np.empty((m, K), dtype=np.float32)
    logits = np.empty((m, E), dtype=np.float32)
    fn = lib().orc_moe4 if inp.q4 else lib().orc_moe
    rc = fn(_p(x), _p(router), E, K, ge, ue, de, sg, su, sd, _p(res), m, _p(y), _p(ids), _p(gates), _p(logits))
    if rc != 0:
        raise ValueError("orc_moe rejected its arguments")
    return y, ids, gates, logits


def head(hidden, gamma, eps, lm):
    """Returns (normed [m, H], logits [m, V], ids [m])."""
    keep = _Keep()
    d = _q4(lm, keep)
    x = keep.arr(np.atleast_2d(hidden), np.float32)
    g = keep.arr(gamma, np.float32)
    m = x.shape[0]
    normed = np.empty((m, lm.k), dtype=np.float32)
    logits = np.empty((m, lm.n), dtype=np.float32)
    ids = np.empty(m, dtype=np.int32)
    lib().orc_head(_p(x), _p(g), float(eps), C.byref(d), m, _p(normed), _p(logits), _p(ids))
    return normed, logits, ids


def head8(hidden, gamma, eps, lm):
    """8-bit lm_head (a Q8 of one matrix): returns (normed [m, H], logits [m, V], ids [m])."""
    keep = _Keep()
    arr = _q8_list(lm, keep)
    x = keep.arr(np.atleast_2d(hidden), np.float32)
    g = keep.arr(gamma, np.float32)
    m = x.shape[0]
    normed = np.empty((m, lm.k), dtype=np.float32)
    logits = np.empty((m, lm.n), dtype=np.float32)
    ids = np.empty(m, dtype=np.int32)
    lib().orc_head8(_p(x), _p(g), float(eps), C.byref(arr[0]), m, _p(normed), _p(logits), _p(ids))
    return normed, logits, ids


def _moe_ffn(inp, keep: _Keep) -> _MoeFfn:
    router = keep.arr(inp.router, np.float32)
    ws = [addr for addr in (C.addressof(_experts(w, keep)) for w in (inp.gate_exps, inp.up_exps, inp.down_exps))]
    sh = [None, None, None]
    if inp.sh_gate is not None:
        sh = [C.addressof(_experts(w, keep)) for w in (inp.sh_gate, inp.sh_up, inp.sh_down)]
    if inp.q4:
        return _MoeFfn(router.ctypes.data, int(inp.n_experts), int(inp.top_k), None, None, None, None, None, None,
                       1, *ws, *sh)
    return _MoeFfn(router.ctypes.data, int(inp.n_experts), int(inp.top_k), *ws, *sh, 0,
                   None, None, None, None, None, None)


def draft_step(L, e, tokens, table, h, k_cache, v_cache, cache_len: int, want_logits: bool = True, moe=None,
               positions=None):
    """One draft-layer forward over m rows; appends K/V rows in place.  With
    moe (a MoE input set of ``synth.moe_inputs``, 8-bit or 4-bit experts) the
    FFN is the routed mixture of those weights instead of the layer's dense
    SwiGLU.  positions: the rows' four rotary position ids (int32 [m, 4]).

    Returns (ids [m], hidden_out [m, H] (post-final-norm), logits [m, V] or None)."""
    assert k_cache.flags.c_contiguous and k_cache.dtype == np.float32
    assert v_cache.flags.c_contiguous and v_cache.dtype == np.float32
    keep = _Keep()
    d = _layer(L, keep, positions)
    h = keep.arr(np.atleast_2d(h), np.float32)
    m = h.shape[0]
    e = None if e is None else keep.arr(np.atleast_2d(e), np.float32)
    tok = None if tokens is None else keep.arr(np.asarray(tokens).reshape(-1), np.int32)
    tab = None if table is None else (table if (table.flags.c_contiguous and table.dtype == np.float32)
                                      else keep.arr(table, np.float32))
    ids = np.empty(m, dtype=np.int32)
    hid = np.empty((m, L.hidden), dtype=np.float32)
    logits = np.empty((m, L.vocab), dtype=np.float32) if want_logits else None
    if moe is None:
        rc = lib().orc_draft_step(C.byref(d), _p(e), _p(tok), _p(tab), _p(h), _p(k_cache), _p(v_cache),
                                  cache_len, k_cache.shape[1], m, _p(ids), _p(hid), _p(logits))
    else:
        mf = _moe_ffn(moe, keep)
        rc = lib().orc_draft_step_moe(C.byref(d), C.byref(mf), _p(e), _p(tok), _p(tab), _p(h), _p(k_cache),
                                      _p(v_cache), cache_len, k_cache.shape[1], m, _p(ids), _p(hid), _p(logits))
    if rc != 0:
        raise ValueError("orc_draft_step rejected its arguments")
    return ids, hid, logits


def append_kv(L, e, tokens, table, pending_h, target_h, k_cache, v_cache, cache_len: int, positions=None) -> None:
    """Cache catch-up after a target batch: writes K/V rows cache_len .. cache_len+m-1
    in place (row r's hidden is target_h row r-1, row 0's pending_h or zero)."""
    assert k_cache.flags.c_contiguous and k_cache.dtype == np.float32
    assert v_cache.flags.c_contiguous and v_cache.dtype == np.float32
    keep = _Keep()
    d = _layer(L, keep, positions)
    tgt = keep.arr(np.atleast_2d(target_h), np.float32)
    m = tgt.shape[0]
    e = None if e is None else keep.arr(np.atleast_2d(e), np.float32)
    tok = None if tokens is None else keep.arr(np.asarray(tokens).reshape(-1), np.int32)
    tab = None if table is None else (table if (table.flags.c_contiguous and table.dtype == np.float32)
                                      else keep.arr(table, np.float32))
    pend = None if pending_h is None else keep.arr(np.asarray(pending_h).reshape(-1), np.float32)
    lib().orc_append_kv(C.byref(d), _p(e), _p(tok), _p(tab), _p(pend), _p(tgt), _p(k_cache), _p(v_cache),
                        cache_len, k_cache.shape[1], m)


def stack_draft(layers, caches, starts, tokens, table, target_h, t: int):
    """Multi-layer draft ([mimo.rs] module doc "How the three layers chain",
    `mimo_mtp_draft`): layer k's rows j = start_k .. t pair the token x_{j+k+1}
    with the target hidden h_j at position j of its own cache; its draft is the
    greedy pick of row t and becomes x_{t+k+2} for the next layer.  Rows before
    t take the cache catch-up (K/V only), row t the full forward.  caches are
    updated in place; returns the drafts."""
    x = [int(v) for v in np.asarray(tokens).reshape(-1)[:t + 2]]
    hs = np.atleast_2d(np.asarray(target_h, np.float32))
    drafts = []
    for k, (L, (kc, vc), st) in enumerate(zip(layers, caches, starts)):
        if st < t:
            append_kv(L, None, np.array(x[st + k + 1:t + k + 1], np.int32), table, hs[st], hs[st + 1:t + 1], kc, vc, st)
        ids, _, _ = draft_step(L, None, np.array([x[t + k + 1]], np.int32), table, hs[t][None], kc, vc, t,
                               want_logits=False)
        x.append(int(ids[0]))
        drafts.append(int(ids[0]))
    return drafts


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    """Cosine similarity with double accumulation; NaN when a norm is zero
    (hf2q 0.1.1 forward_mlx_shared.rs, `cosine_pairwise_f32`)."""
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    na, nb = np.sqrt((a * a).sum()), np.sqrt((b * b).sum())
    if na == 0.0 or nb == 0.0:
        return float("nan")
    return float((a * b).sum() / (na * nb))


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    """||got - ref||_2 / ||ref||_2 in double."""
    g = np.asarray(got, dtype=np.float64).ravel()
    r = np.asarray(ref, dtype=np.float64).ravel()
    den = np.sqrt((r * r).sum())
    num = np.sqrt(((g - r) ** 2).sum())
    return float(num / den) if den > 0 else float(num)
