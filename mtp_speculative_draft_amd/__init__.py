"""MI355X-native quantized MTP (NextN) draft-layer forward.

A thin binding over ``libmtp.so`` (C ABI in ``include/mtp.h``): every function
here marshals torch tensors into pointers and calls the library function of
the same name; all arithmetic runs in the library's HIP kernels.  PyTorch only
provides device memory and the current stream.  The library must be built
(``python -m mtp_speculative_draft_amd.build``); without it every call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmtp.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "mtp.h")

MTP_OK, MTP_ERR_INVALID_ARG, MTP_ERR_UNSUPPORTED, MTP_ERR_WORKSPACE, MTP_ERR_HIP = range(5)
MTP_MAX_ROWS = 8
MTP_NOALLOC_SCRATCH_BYTES = 32 << 20
MTP_FFN_DENSE_Q4, MTP_FFN_MOE_Q8, MTP_FFN_MOE_Q4 = 0, 1, 2


class MtpError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


class MtpQ4(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("biases", C.c_void_p),
                ("n", C.c_int32), ("k", C.c_int32)]


class MtpQ8(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("n", C.c_int32), ("k", C.c_int32),
                ("n_experts", C.c_int32)]


class MtpQ4E(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("biases", C.c_void_p),
                ("n", C.c_int32), ("k", C.c_int32), ("n_experts", C.c_int32)]


MTP_MAX_DRAFT = 16


class MtpStackLayer(C.Structure):
    _fields_ = [("layer", C.c_void_p), ("k_cache", C.c_void_p), ("v_cache", C.c_void_p), ("capacity", C.c_int32),
                ("start", C.c_int32)]


class MtpStats(C.Structure):
    """Speculative round statistics (mtp_stats)."""
    _fields_ = [("rounds", C.c_uint64), ("drafted", C.c_uint64), ("accepted", C.c_uint64),
                ("accept_hist", C.c_uint64 * (MTP_MAX_DRAFT + 1)), ("depth_drafted", C.c_uint64 * MTP_MAX_DRAFT),
                ("depth_accepted", C.c_uint64 * MTP_MAX_DRAFT)]


class MtpLayer(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("vocab", C.c_int32), ("ffn_kind", C.c_int32),
                ("ffn_inter", C.c_int32), ("top_k", C.c_int32), ("rope_theta", C.c_double), ("eps", C.c_float),
                ("gamma_e", C.c_void_p), ("gamma_h", C.c_void_p), ("gamma_attn", C.c_void_p),
                ("gamma_post", C.c_void_p), ("gamma_final", C.c_void_p),
                ("eh_proj", MtpQ4), ("wq", MtpQ4), ("wk", MtpQ4), ("wv", MtpQ4), ("wo", MtpQ4),
                ("gate", MtpQ4), ("up", MtpQ4), ("down", MtpQ4), ("lm_head", MtpQ4),
                ("router", C.c_void_p),
                ("gate_exps", MtpQ8), ("up_exps", MtpQ8), ("down_exps", MtpQ8),
                ("sh_gate", MtpQ8), ("sh_up", MtpQ8), ("sh_down", MtpQ8),
                ("gamma_q_head", C.c_void_p), ("gamma_k_head", C.c_void_p),
                ("q_gated", C.c_int32), ("rotary_dim", C.c_int32),
                ("sinks", C.c_void_p), ("window", C.c_int32), ("v_head_dim", C.c_int32),
                ("gate_exps4", MtpQ4E), ("up_exps4", MtpQ4E), ("down_exps4", MtpQ4E),
                ("sh_gate4", MtpQ4E), ("sh_up4", MtpQ4E), ("sh_down4", MtpQ4E),
                ("mrope_section", C.c_int32 * 4), ("positions", C.c_void_p)]


_lib = None

_P, _I, _Z, _F = C.c_void_p, C.c_int32, C.c_size_t, C.c_float
_SIGS = {
    "mtp_status_string": (C.c_char_p, [_I]),
    "mtp_last_error": (C.c_char_p, []),
    "mtp_version": (C.c_char_p, []),
    "mtp_attn_decode_workspace_size": (_Z, [_P, _I, _I]),
    "mtp_ffn_dense_workspace_size": (_Z, [_I, _I]),
    "mtp_ffn_moe_workspace_size": (_Z, [_I, _I, _I, _I, _I, _I]),
    "mtp_lmhead_workspace_size": (_Z, [_I, _I]),
    "mtp_draft_step_workspace_size": (_Z, [_P, _I, _I]),
    "mtp_dequant_q4": (_I, [_P, _P, _P]),
    "mtp_dequant_q8": (_I, [_P, _I, _P, _P]),
    "mtp_dequant_q4e": (_I, [_P, _I, _P, _P]),
    "mtp_qgemv": (_I, [_P, _P, _P, _P, _I, _P]),
    "mtp_q8gemv": (_I, [_P, _I, _P, _P, _P, _I, _P]),
    "mtp_norm_concat_proj": (_I, [_P, _P, _P, _P, _F, _P, _P, _I, _P]),
    "mtp_attn_decode": (_I, [_P, _P, _P, _P, _I, _I, _I, _P, _P, _Z, _P]),
    "mtp_ffn_dense_q": (_I, [_P, _P, _F, _P, _P, _P, _P, _P, _I, _P, _Z, _P]),
    "mtp_ffn_moe_q": (_I, [_P, _P, _F, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _Z, _P]),
    "mtp_ffn_moe_q4": (_I, [_P, _P, _F, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _Z, _P]),
    "mtp_lmhead_argmax": (_I, [_P, _P, _F, _P, _P, _P, _P, _I, _P, _Z, _P]),
    "mtp_draft_step": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _Z, _P]),
    "mtp_draft_step_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P]),
    "mtp_append_kv_workspace_size": (_Z, [_P]),
    "mtp_append_kv": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _Z, _P]),
    "mtp_accept": (_I, [_P, _P, _I, _P]),
    "mtp_lmhead_argmax_q8": (_I, [_P, _P, _F, _P, _P, _P, _P, _I, _P, _Z, _P]),
    "mtp_stack_draft_workspace_size": (_Z, [_P, _I, _I]),
    "mtp_stack_draft": (_I, [_P, _I, _P, _P, _P, _I, _P, _Z, _P]),
}


def lib() -> C.CDLL:
    """Load libmtp.so (raises when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m mtp_speculative_draft_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int, where: str) -> None:
    if status != MTP_OK:
        raise MtpError(status, where, lib().mtp_last_error().decode())


# --------------------------------------------------------------------------
# device-side weight handles
# --------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dev_tensor(a: np.ndarray, device):
    torch = _torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.uint16:  # bf16 bits
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class DeviceQ4:
    """4-bit affine weight resident on the device (tensors + descriptor)."""

    def __init__(self, w, device="cuda"):
        self.codes = _dev_tensor(w.codes, device)
        self.scales = _dev_tensor(w.scales, device)
        self.biases = _dev_tensor(w.biases, device)
        self.n, self.k = int(w.n), int(w.k)
        self.desc = MtpQ4(self.codes.data_ptr(), self.scales.data_ptr(), self.biases.data_ptr(), self.n, self.k)

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.codes, self.scales, self.biases))


class DeviceQ8:
    """8-bit block weight stack [E, n, k] resident on the device."""

    def __init__(self, w, device="cuda"):
        self.codes = _dev_tensor(w.codes, device)
        self.scales = _dev_tensor(w.scales, device)
        self.n_experts, self.n, self.k = (int(s) for s in w.codes.shape)
        self.desc = MtpQ8(self.codes.data_ptr(), self.scales.data_ptr(), self.n, self.k, self.n_experts)


class DeviceQ4E:
    """4-bit expert stack with bf16 group constants [E, n, k/8] resident on the device."""

    def __init__(self, w, device="cuda"):
        self.codes = _dev_tensor(w.codes, device)
        self.scales = _dev_tensor(w.scales, device)
        self.biases = _dev_tensor(w.biases, device)
        self.n_experts, self.n = (int(s) for s in w.codes.shape[:2])
        self.k = int(w.codes.shape[2]) * 8
        self.desc = MtpQ4E(self.codes.data_ptr(), self.scales.data_ptr(), self.biases.data_ptr(), self.n, self.k,
                           self.n_experts)


def _empty_q8() -> MtpQ8:
    return MtpQ8(None, None, 0, 0, 0)


def _empty_q4e() -> MtpQ4E:
    return MtpQ4E(None, None, None, 0, 0, 0)


def device_experts(w, device="cuda"):
    """DeviceQ4E for a 4-bit stack with bf16 constants, DeviceQ8 for an 8-bit one."""
    return DeviceQ4E(w, device) if w.codes.dtype == np.uint32 else DeviceQ8(w, device)


class DeviceLayer:
    """A draft layer resident on the device; ``desc`` is the mtp_layer struct.

    ``dense`` is a ``synth.DenseLayer``; an optional ``moe`` (``synth.MoeInputs``
    weights, 8-bit or 4-bit experts) turns the FFN into the routed mixture."""

    def __init__(self, dense, device="cuda", moe=None):
        torch = _torch()
        f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)  # noqa: E731
        self.hidden, self.vocab = dense.hidden, dense.vocab
        self.gammas = [f(g) for g in (dense.gamma_e, dense.gamma_h, dense.gamma_attn, dense.gamma_post,
                                      dense.gamma_final)]
        self.q4 = {name: DeviceQ4(getattr(dense, name), device)
                   for name in ("eh_proj", "wq", "wk", "wv", "wo", "gate", "up", "down", "lm_head")}
        self.moe = None
        names = ("gate_exps", "up_exps", "down_exps", "sh_gate", "sh_up", "sh_down")
        q8 = {k: _empty_q8() for k in names}
        q4e = {k: _empty_q4e() for k in names}
        router, top_k, kind = None, 0, MTP_FFN_DENSE_Q4
        if moe is not None:
            self.router = f(moe.router)
            self.moe = {k: device_experts(getattr(moe, k), device) for k in names[:3]}
            if moe.sh_gate is not None:
                self.moe.update({k: device_experts(getattr(moe, k), device) for k in names[3:]})
            is4 = isinstance(self.moe["gate_exps"], DeviceQ4E)
            for k, v in self.moe.items():
                (q4e if is4 else q8)[k] = v.desc
            router, top_k, kind = self.router.data_ptr(), moe.top_k, (MTP_FFN_MOE_Q4 if is4 else MTP_FFN_MOE_Q8)
        g = [t.data_ptr() for t in self.gammas]
        # attention variant: per-head q/k norm weights, gated q, partial rotary
        gq, gk = getattr(dense, "gamma_q_head", None), getattr(dense, "gamma_k_head", None)
        self.head_gammas = None if gq is None else (f(gq), f(gk))
        hq = self.head_gammas[0].data_ptr() if self.head_gammas else None
        hk = self.head_gammas[1].data_ptr() if self.head_gammas else None
        # sliding window and per-head sinks
        sk = getattr(dense, "sinks", None)
        self.sinks = None if sk is None else f(sk)
        q = self.q4
        self.desc = MtpLayer(dense.hidden, dense.n_heads, dense.n_kv_heads, dense.head_dim, dense.vocab, kind,
                             dense.ffn_inter, top_k, float(dense.rope_theta), float(dense.eps), *g,
                             q["eh_proj"].desc, q["wq"].desc, q["wk"].desc, q["wv"].desc, q["wo"].desc,
                             q["gate"].desc, q["up"].desc, q["down"].desc, q["lm_head"].desc, router,
                             q8["gate_exps"], q8["up_exps"], q8["down_exps"], q8["sh_gate"], q8["sh_up"],
                             q8["sh_down"], hq, hk, int(bool(getattr(dense, "q_gated", False))),
                             int(getattr(dense, "rotary_dim", 0) or 0),
                             None if self.sinks is None else self.sinks.data_ptr(),
                             int(getattr(dense, "window", 0) or 0), int(getattr(dense, "v_head_dim", 0) or 0),
                             *(q4e[k] for k in names),
                             (C.c_int32 * 4)(*[int(v) for v in (getattr(dense, "mrope_section", None)
                                                                 or (0, 0, 0, 0))]), None)
        self.positions = None

    def set_positions(self, positions) -> None:
        """The rotary position ids (int32 device tensor [rows, 4]) that the
        following calls read for their rows; None: the rows' cache positions."""
        if positions is not None:
            torch = _torch()
            if positions.dtype != torch.int32 or not positions.is_cuda or positions.dim() != 2 or \
                    positions.shape[1] != 4 or not positions.is_contiguous():
                raise ValueError("positions must be a contiguous int32 device tensor [rows, 4]")
        self.positions = positions
        self.desc.positions = None if positions is None else positions.data_ptr()

    @property
    def weight_nbytes(self) -> int:
        return sum(w.nbytes for w in self.q4.values()) + sum(t.numel() * 4 for t in self.gammas)


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------
def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmtp must be contiguous")
    return t.data_ptr()


def _stream(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _f32(t, name):
    torch = _torch()
    if t is None or t.dtype != torch.float32 or not t.is_cuda:
        raise ValueError(f"{name} must be a float32 device tensor")
    return t


def _rows(t) -> int:
    return int(t.shape[0]) if t.dim() > 1 else 1


def _ws(nbytes: int, like, ws):
    torch = _torch()
    if ws is not None:
        return ws
    # zero-filled: the reserved head-state bytes at its start must read zero
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=like.device)


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


# --------------------------------------------------------------------------
# workspace sizes
# --------------------------------------------------------------------------
def mtp_attn_decode_workspace_size(layer: DeviceLayer, cache_len: int, m: int) -> int:
    return int(lib().mtp_attn_decode_workspace_size(C.byref(layer.desc), cache_len, m))


def mtp_ffn_dense_workspace_size(ffn_inter: int, m: int) -> int:
    return int(lib().mtp_ffn_dense_workspace_size(ffn_inter, m))


def mtp_ffn_moe_workspace_size(hidden: int, n_experts: int, top_k: int, inter: int, shared_inter: int, m: int) -> int:
    return int(lib().mtp_ffn_moe_workspace_size(hidden, n_experts, top_k, inter, shared_inter, m))


def mtp_lmhead_workspace_size(vocab: int, m: int) -> int:
    return int(lib().mtp_lmhead_workspace_size(vocab, m))


def mtp_draft_step_workspace_size(layer: DeviceLayer, cache_len: int, m: int) -> int:
    return int(lib().mtp_draft_step_workspace_size(C.byref(layer.desc), cache_len, m))


def mtp_append_kv_workspace_size(layer: DeviceLayer) -> int:
    return int(lib().mtp_append_kv_workspace_size(C.byref(layer.desc)))


def _stack_array(layers, caches, starts):
    n = len(layers)
    arr = (MtpStackLayer * n)()
    for i, (dl, (kc, vc), st) in enumerate(zip(layers, caches, starts)):
        arr[i] = MtpStackLayer(C.addressof(dl.desc), _ptr(kc), _ptr(vc), int(kc.shape[1]), int(st))
    return arr


def mtp_stack_draft_workspace_size(layers, caches, starts, t: int) -> int:
    return int(lib().mtp_stack_draft_workspace_size(_stack_array(layers, caches, starts), len(layers), int(t)))


# --------------------------------------------------------------------------
# calls
# --------------------------------------------------------------------------
def mtp_dequant_q4(w: DeviceQ4, out=None):
    torch = _torch()
    out = torch.empty((w.n, w.k), dtype=torch.float32, device=w.codes.device) if out is None else out
    _check(lib().mtp_dequant_q4(C.byref(w.desc), _ptr(out), _stream(out)), "mtp_dequant_q4")
    return out


def mtp_dequant_q8(w: DeviceQ8, expert: int = 0, out=None):
    torch = _torch()
    out = torch.empty((w.n, w.k), dtype=torch.float32, device=w.codes.device) if out is None else out
    _check(lib().mtp_dequant_q8(C.byref(w.desc), int(expert), _ptr(out), _stream(out)), "mtp_dequant_q8")
    return out


def mtp_dequant_q4e(w: DeviceQ4E, expert: int = 0, out=None):
    torch = _torch()
    out = torch.empty((w.n, w.k), dtype=torch.float32, device=w.codes.device) if out is None else out
    _check(lib().mtp_dequant_q4e(C.byref(w.desc), int(expert), _ptr(out), _stream(out)), "mtp_dequant_q4e")
    return out


def mtp_qgemv(w: DeviceQ4, x, residual=None, y=None):
    torch = _torch()
    _f32(x, "x")
    m = _rows(x)
    y = torch.empty((m, w.n), dtype=torch.float32, device=x.device) if y is None else y
    _check(lib().mtp_qgemv(C.byref(w.desc), _ptr(x), _ptr(residual), _ptr(y), m, _stream(x)), "mtp_qgemv")
    return y


def mtp_q8gemv(w: DeviceQ8, expert: int, x, residual=None, y=None):
    torch = _torch()
    _f32(x, "x")
    m = _rows(x)
    y = torch.empty((m, w.n), dtype=torch.float32, device=x.device) if y is None else y
    _check(lib().mtp_q8gemv(C.byref(w.desc), int(expert), _ptr(x), _ptr(residual), _ptr(y), m, _stream(x)),
           "mtp_q8gemv")
    return y


def mtp_norm_concat_proj(e, h, gamma_e, gamma_h, eps: float, eh_proj: DeviceQ4, u=None):
    torch = _torch()
    _f32(e, "e")
    _f32(h, "h")
    m = _rows(e)
    u = torch.empty((m, eh_proj.n), dtype=torch.float32, device=e.device) if u is None else u
    _check(lib().mtp_norm_concat_proj(_ptr(e), _ptr(h), _ptr(gamma_e), _ptr(gamma_h), float(eps),
                                      C.byref(eh_proj.desc), _ptr(u), m, _stream(e)), "mtp_norm_concat_proj")
    return u


def mtp_attn_decode(layer: DeviceLayer, u, k_cache, v_cache, cache_len: int, out=None, ws=None):
    torch = _torch()
    _f32(u, "u")
    m = _rows(u)
    out = torch.empty_like(u) if out is None else out
    need = mtp_attn_decode_workspace_size(layer, cache_len, m)
    ws = _ws(need, u, ws)
    _check(lib().mtp_attn_decode(C.byref(layer.desc), _ptr(u), _ptr(k_cache), _ptr(v_cache), int(cache_len),
                                 int(k_cache.shape[1]), m, _ptr(out), _ptr(ws), _nbytes(ws), _stream(u)),
           "mtp_attn_decode")
    return out


def mtp_ffn_dense_q(x, gamma, eps: float, gate: DeviceQ4, up: DeviceQ4, down: DeviceQ4, residual=None, y=None,
                    ws=None):
    torch = _torch()
    _f32(x, "x")
    m = _rows(x)
    y = torch.empty((m, down.n), dtype=torch.float32, device=x.device) if y is None else y
    ws = _ws(mtp_ffn_dense_workspace_size(gate.n, m), x, ws)
    _check(lib().mtp_ffn_dense_q(_ptr(x), _ptr(gamma), float(eps), C.byref(gate.desc), C.byref(up.desc),
                                 C.byref(down.desc), _ptr(residual), _ptr(y), m, _ptr(ws), _nbytes(ws), _stream(x)),
           "mtp_ffn_dense_q")
    return y


def mtp_ffn_moe_q(x, gamma, eps: float, router, top_k: int, gate_exps: DeviceQ8, up_exps: DeviceQ8,
                  down_exps: DeviceQ8, sh_gate: Optional[DeviceQ8] = None, sh_up: Optional[DeviceQ8] = None,
                  sh_down: Optional[DeviceQ8] = None, residual=None, y=None, expert_ids=None, gates=None, ws=None):
    """Returns (y, expert_ids [m, top_k] int32, gates [m, top_k])."""
    torch = _torch()
    _f32(x, "x")
    m = _rows(x)
    y = torch.empty((m, gate_exps.k), dtype=torch.float32, device=x.device) if y is None else y
    expert_ids = torch.empty((m, top_k), dtype=torch.int32, device=x.device) if expert_ids is None else expert_ids
    gates = torch.empty((m, top_k), dtype=torch.float32, device=x.device) if gates is None else gates
    sh_n = sh_gate.n if sh_gate is not None else 0
    ws = _ws(mtp_ffn_moe_workspace_size(gate_exps.k, gate_exps.n_experts, top_k, gate_exps.n, sh_n, m), x, ws)
    ref = lambda w: None if w is None else C.byref(w.desc)  # noqa: E731
    _check(lib().mtp_ffn_moe_q(_ptr(x), _ptr(gamma), float(eps), _ptr(router), int(top_k), ref(gate_exps),
                               ref(up_exps), ref(down_exps), ref(sh_gate), ref(sh_up), ref(sh_down), _ptr(residual),
                               _ptr(y), _ptr(expert_ids), _ptr(gates), m, _ptr(ws), _nbytes(ws), _stream(x)),
           "mtp_ffn_moe_q")
    return y, expert_ids, gates


def mtp_ffn_moe_q4(x, gamma, eps: float, router, top_k: int, gate_exps: DeviceQ4E, up_exps: DeviceQ4E,
                   down_exps: DeviceQ4E, sh_gate: Optional[DeviceQ4E] = None, sh_up: Optional[DeviceQ4E] = None,
                   sh_down: Optional[DeviceQ4E] = None, residual=None, y=None, expert_ids=None, gates=None, ws=None):
    """The routed mixture over 4-bit experts with bf16 constants; returns
    (y, expert_ids [m, top_k] int32, gates [m, top_k])."""
    torch = _torch()
    _f32(x, "x")
    m = _rows(x)
    y = torch.empty((m, gate_exps.k), dtype=torch.float32, device=x.device) if y is None else y
    expert_ids = torch.empty((m, top_k), dtype=torch.int32, device=x.device) if expert_ids is None else expert_ids
    gates = torch.empty((m, top_k), dtype=torch.float32, device=x.device) if gates is None else gates
    sh_n = sh_gate.n if sh_gate is not None else 0
    ws = _ws(mtp_ffn_moe_workspace_size(gate_exps.k, gate_exps.n_experts, top_k, gate_exps.n, sh_n, m), x, ws)
    ref = lambda w: None if w is None else C.byref(w.desc)  # noqa: E731
    _check(lib().mtp_ffn_moe_q4(_ptr(x), _ptr(gamma), float(eps), _ptr(router), int(top_k), ref(gate_exps),
                                ref(up_exps), ref(down_exps), ref(sh_gate), ref(sh_up), ref(sh_down), _ptr(residual),
                                _ptr(y), _ptr(expert_ids), _ptr(gates), m, _ptr(ws), _nbytes(ws), _stream(x)),
           "mtp_ffn_moe_q4")
    return y, expert_ids, gates


def mtp_lmhead_argmax(hidden, gamma, eps: float, lm_head: DeviceQ4, normed_out=None, logits_out=None, ids_out=None,
                      ws=None):
    torch = _torch()
    _f32(hidden, "hidden")
    m = _rows(hidden)
    ids_out = torch.empty(m, dtype=torch.int32, device=hidden.device) if ids_out is None else ids_out
    if ws is None:  # its leading argmax state must start at zero
        ws = torch.zeros(max(mtp_lmhead_workspace_size(lm_head.n, m), 256), dtype=torch.uint8, device=hidden.device)
    _check(lib().mtp_lmhead_argmax(_ptr(hidden), _ptr(gamma), float(eps), C.byref(lm_head.desc), _ptr(normed_out),
                                   _ptr(logits_out), _ptr(ids_out), m, _ptr(ws), _nbytes(ws), _stream(hidden)),
           "mtp_lmhead_argmax")
    return ids_out


def mtp_draft_step(layer: DeviceLayer, e, tokens, embed_table, h, k_cache, v_cache, cache_len: int, ids_out=None,
                   hidden_out=None, logits_out=None, ws=None):
    """One draft-layer forward over m rows; returns (ids_out, hidden_out)."""
    torch = _torch()
    _f32(h, "h")
    m = _rows(h)
    ids_out = torch.empty(m, dtype=torch.int32, device=h.device) if ids_out is None else ids_out
    hidden_out = torch.empty((m, layer.hidden), dtype=torch.float32, device=h.device) if hidden_out is None else hidden_out
    ws = _ws(mtp_draft_step_workspace_size(layer, cache_len, m), h, ws)
    _check(lib().mtp_draft_step(C.byref(layer.desc), _ptr(e), _ptr(tokens), _ptr(embed_table), _ptr(h),
                                _ptr(k_cache), _ptr(v_cache), int(cache_len), int(k_cache.shape[1]), m,
                                _ptr(ids_out), _ptr(hidden_out), _ptr(logits_out), _ptr(ws), _nbytes(ws),
                                _stream(h)), "mtp_draft_step")
    return ids_out, hidden_out


def mtp_draft_step_noalloc(layer: DeviceLayer, e, tokens, embed_table, h, k_cache, v_cache, cache_len: int, ids_out,
                           hidden_out, logits_out=None):
    """mtp_draft_step with the library's static scratch instead of a workspace
    (the outputs are the caller's: nothing is allocated here either)."""
    _f32(h, "h")
    m = _rows(h)
    _check(lib().mtp_draft_step_noalloc(C.byref(layer.desc), _ptr(e), _ptr(tokens), _ptr(embed_table), _ptr(h),
                                        _ptr(k_cache), _ptr(v_cache), int(cache_len), int(k_cache.shape[1]), m,
                                        _ptr(ids_out), _ptr(hidden_out), _ptr(logits_out), _stream(h)),
           "mtp_draft_step_noalloc")
    return ids_out, hidden_out


def mtp_append_kv(layer: DeviceLayer, e, tokens, embed_table, pending_h, target_h, k_cache, v_cache, cache_len: int,
                  ws=None):
    """Cache catch-up after a target batch: writes K/V rows cache_len .. cache_len+m-1."""
    _f32(target_h, "target_h")
    m = _rows(target_h)
    ws = _ws(mtp_append_kv_workspace_size(layer), target_h, ws)
    _check(lib().mtp_append_kv(C.byref(layer.desc), _ptr(e), _ptr(tokens), _ptr(embed_table), _ptr(pending_h),
                               _ptr(target_h), _ptr(k_cache), _ptr(v_cache), int(cache_len), int(k_cache.shape[1]),
                               m, _ptr(ws), _nbytes(ws), _stream(target_h)), "mtp_append_kv")


def mtp_accept(drafts, target_ids, stats: Optional[MtpStats] = None) -> int:
    """Greedy acceptance of one round (host int32 sequences); returns a."""
    d = np.ascontiguousarray(np.asarray(drafts, dtype=np.int32).reshape(-1))
    t = np.ascontiguousarray(np.asarray(target_ids, dtype=np.int32).reshape(-1))
    k = d.size
    if t.size != k + 1:
        raise ValueError("target_ids needs k + 1 entries")
    a = lib().mtp_accept(d.ctypes.data, t.ctypes.data, k, None if stats is None else C.byref(stats))
    if a < 0:
        raise MtpError(MTP_ERR_INVALID_ARG, "mtp_accept", lib().mtp_last_error().decode())
    return int(a)


def mtp_lmhead_argmax_q8(hidden, gamma, eps: float, lm_head: DeviceQ8, normed_out=None, logits_out=None,
                         ids_out=None, ws=None):
    """Fused final norm + 8-bit lm_head + greedy pick; returns ids_out."""
    torch = _torch()
    _f32(hidden, "hidden")
    m = _rows(hidden)
    ids_out = torch.empty(m, dtype=torch.int32, device=hidden.device) if ids_out is None else ids_out
    if ws is None:  # its leading argmax state must start at zero
        ws = torch.zeros(max(mtp_lmhead_workspace_size(lm_head.n, m), 256), dtype=torch.uint8, device=hidden.device)
    _check(lib().mtp_lmhead_argmax_q8(_ptr(hidden), _ptr(gamma), float(eps), C.byref(lm_head.desc),
                                      _ptr(normed_out), _ptr(logits_out), _ptr(ids_out), m, _ptr(ws), _nbytes(ws),
                                      _stream(hidden)), "mtp_lmhead_argmax_q8")
    return ids_out


def mtp_stack_draft(layers, caches, starts, tokens, embed_table, target_h, t: int, ws=None):
    """Multi-layer draft: layers (DeviceLayer list), caches [(k, v)], starts
    (first recomputed row per layer); tokens device int32 [t + 2 + len(layers)]
    gets draft k at t + 2 + k.  Returns tokens."""
    n = len(layers)
    arr = _stack_array(layers, caches, starts)
    need = int(lib().mtp_stack_draft_workspace_size(arr, n, int(t)))
    ws = _ws(need, target_h, ws)
    _check(lib().mtp_stack_draft(arr, n, _ptr(tokens), _ptr(embed_table), _ptr(target_h), int(t), _ptr(ws),
                                 _nbytes(ws), _stream(target_h)), "mtp_stack_draft")
    return tokens
