"""Python binding of libdflash_fuse.so, the MI355X (gfx950) DFlash draft step.

Argument marshalling only: every step of the draft runs in the HIP kernels of
the shared library.  PyTorch provides device memory and the stream.  The names
mirror the C ABI in include/dflash_fuse.h.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# DFLASH_FUSE_LIB may name another build of the same library (tuning sweeps).
LIB_PATH = os.environ.get("DFLASH_FUSE_LIB") or os.path.join(HERE, "libdflash_fuse.so")

DFLASH_F32, DFLASH_BF16 = 0, 1
STATUS = {0: "DFLASH_OK", -1: "DFLASH_EINVAL", -2: "DFLASH_EUNSUPPORTED",
          -3: "DFLASH_ECAPACITY", -4: "DFLASH_EHIP"}

EXPORTED = ("dflash_query_sizes", "dflash_create", "dflash_destroy", "dflash_fuse_ctx",
            "dflash_draft_block", "dflash_accept", "dflash_slot_reset", "dflash_slot_len",
            "dflash_read_cache", "dflow_relay", "dflow_read_relay", "dflash2_select", "dflash2_conv_attach",
            "dflash_spec_draft", "dflash_spec_draft_static", "dflash_spec_verify", "dflash_profile_enable",
            "dflash_profile_read", "dflash_strerror", "dflash_last_error")

KERNEL_KINDS = ("fuse_gemm", "fuse_norm", "ctx_kv_gemm", "embed", "norm", "qkv_gemm", "attention",
                "attn_combine", "o_gemm", "gateup_gemm", "down_gemm", "lm_head", "topk_merge", "relay", "select", "conv",
                "spec_draft", "spec_stats", "spec_resample", "accept")


class DflashError(RuntimeError):
    def __init__(self, code: int, where: str, detail: str):
        super().__init__(f"{where}: {STATUS.get(code, code)} ({detail})")
        self.code = code


class dflash_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("dtype", "D", "L", "Dt", "N", "Hq", "Hkv", "hd", "I", "V", "B",
                 "max_ctx", "max_slots", "max_batch")] + [
        ("rope_base", ctypes.c_float), ("rms_eps", ctypes.c_float), ("use_rope", ctypes.c_int32)]


LAYER_FIELDS = ("g_attn", "w_q", "w_kb", "w_vb", "w_kc", "w_vc", "w_o", "g_ffn", "w_gate",
                "w_up", "w_down")


class dflash_layer_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_FIELDS]


class dflash_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_c", "g_c", "embed", "e_mask", "g_final", "w_lm")] + [
        ("layers", ctypes.POINTER(dflash_layer_weights))]


class dflow_relay_weights(ctypes.Structure):
    _fields_ = [("w1", ctypes.c_void_p), ("w2", ctypes.c_void_p)]


class dflash2_selector_weights(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("w_h", ctypes.c_void_p), ("rank", ctypes.c_int32)]


class dflash2_conv_site(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("kbase", ctypes.c_void_p)]


CONV_SITES = ("attn_in", "attn_out", "ffn_in", "ffn_out")


class dflash2_conv_layer(ctypes.Structure):
    _fields_ = [(n, dflash2_conv_site) for n in CONV_SITES]


_LIB = None


def lib() -> ctypes.CDLL:
    """Load the HIP library; fails loudly when it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "or `python block_diffusion_drafter_fuse_amd/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    P = ctypes.POINTER
    L.dflash_query_sizes.argtypes = [P(dflash_dims), P(sz), P(sz)]
    L.dflash_create.argtypes = [P(dflash_dims), P(dflash_weights), vp, sz, vp, sz, P(vp)]
    L.dflash_destroy.argtypes = [vp]
    L.dflash_destroy.restype = None
    L.dflash_fuse_ctx.argtypes = [vp, vp, i32, P(i32), P(i32), P(vp)]
    L.dflash_draft_block.argtypes = [vp, vp, i32, P(i32), vp, i32, vp, vp, vp]
    L.dflash_accept.argtypes = [vp, i32, i32, vp, i32, vp, vp, vp]
    L.dflash_slot_reset.argtypes = [vp, i32, i32]
    L.dflash_slot_len.argtypes = [vp, i32, P(i32)]
    L.dflash_read_cache.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp]
    L.dflow_relay.argtypes = [vp, vp, i32, P(i32), P(i32), vp, i32, vp, P(vp), P(dflow_relay_weights)]
    L.dflow_read_relay.argtypes = [vp, vp, i32, vp, P(i32)]
    L.dflash2_select.argtypes = [vp, vp, i32, vp, vp, vp, i32, P(dflash2_selector_weights), vp, vp]
    L.dflash2_conv_attach.argtypes = [vp, P(dflash2_conv_layer)]
    u64, f32 = ctypes.c_uint64, ctypes.c_float
    L.dflash_spec_draft.argtypes = [vp, vp, i32, vp, f32, u64, vp, vp, vp]
    L.dflash_spec_verify.argtypes = [vp, vp, i32, vp, vp, vp, vp, f32, u64, vp, vp, vp]
    L.dflash_spec_draft_static.argtypes = [vp, i32, i32, i32, vp, f32, u64, vp, vp, vp]
    L.dflash_profile_enable.argtypes = [vp, ctypes.c_uint32, i32]
    L.dflash_profile_read.argtypes = [vp, P(ctypes.c_double), P(i32)]
    L.dflash_strerror.argtypes = [ctypes.c_int]
    L.dflash_strerror.restype = ctypes.c_char_p
    L.dflash_last_error.argtypes = []
    L.dflash_last_error.restype = ctypes.c_char_p
    for n in EXPORTED:
        if n not in ("dflash_destroy", "dflash_strerror", "dflash_last_error"):
            getattr(L, n).restype = ctypes.c_int
    _LIB = L
    return L


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise DflashError(rc, where, lib().dflash_last_error().decode())


def make_dims(d, max_ctx: int, max_slots: int, max_batch: int) -> dflash_dims:
    """C dims from any object with the model fields (D, L, Dt, N, Hq, Hkv, hd, I,
    V, B, rope_base, rms_eps, use_rope, dtype in {"f32", "bf16"})."""
    return dflash_dims(DFLASH_BF16 if d.dtype == "bf16" else DFLASH_F32, d.D, d.L, d.Dt, d.N,
                       d.Hq, d.Hkv, d.hd, d.I, d.V, d.B, max_ctx, max_slots, max_batch,
                       float(d.rope_base), float(d.rms_eps), int(bool(d.use_rope)))


def query_sizes(dims: dflash_dims):
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().dflash_query_sizes(ctypes.byref(dims), ctypes.byref(a), ctypes.byref(b)),
           "dflash_query_sizes")
    return a.value, b.value


def to_device(a: np.ndarray, device="cuda"):
    """Upload a storage-dtype array (float32, or uint16 bf16 bits)."""
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _i32(xs: Sequence[int]):
    arr = (ctypes.c_int32 * max(1, len(xs)))(*[int(x) for x in xs])
    return arr


class Drafter:
    """One dflash_ctx over caller-owned (torch) device buffers."""

    def __init__(self, d, weights: dict, max_ctx: int, max_slots: int, max_batch: int,
                 device="cuda"):
        import torch
        self.d = d
        self.device = device
        self.dims = make_dims(d, max_ctx, max_slots, max_batch)
        pool_b, ws_b = query_sizes(self.dims)
        self.pool = torch.empty(pool_b, dtype=torch.uint8, device=device)
        self.ws = torch.empty(ws_b, dtype=torch.uint8, device=device)
        self.w = weights  # keep tensors alive
        layers = (dflash_layer_weights * d.N)()
        for l in range(d.N):
            for n in LAYER_FIELDS:
                setattr(layers[l], n, _ptr(weights["layers"][l][n]))
        self._layers = layers
        cw = dflash_weights(_ptr(weights["w_c"]), _ptr(weights["g_c"]), _ptr(weights["embed"]),
                            _ptr(weights["e_mask"]), _ptr(weights["g_final"]), _ptr(weights["w_lm"]),
                            layers)
        h = ctypes.c_void_p()
        _check(lib().dflash_create(ctypes.byref(self.dims), ctypes.byref(cw), _ptr(self.pool), pool_b,
                                   _ptr(self.ws), ws_b, ctypes.byref(h)), "dflash_create")
        self.h = h

    @staticmethod
    def upload_weights(w_np: dict, device="cuda") -> dict:
        out = {k: to_device(v, device) for k, v in w_np.items() if k not in ("layers", "w_lm")}
        out["w_lm"] = out["embed"] if w_np["w_lm"] is w_np["embed"] else to_device(w_np["w_lm"], device)
        out["layers"] = [{k: to_device(v, device) for k, v in lw.items()} for lw in w_np["layers"]]
        return out

    def close(self):
        if getattr(self, "h", None) and self.h.value:
            lib().dflash_destroy(self.h)
            self.h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def fuse_ctx(self, slots: Sequence[int], n_new: Sequence[int], hidden: Sequence, stream=None):
        ptrs = (ctypes.c_void_p * max(1, len(hidden)))(*[_ptr(t) for t in hidden])
        _check(lib().dflash_fuse_ctx(self.h, _stream(stream), len(slots), _i32(slots), _i32(n_new), ptrs),
               "dflash_fuse_ctx")

    def draft_block(self, slots: Sequence[int], anchor, top_k: int, out_ids, out_vals=None,
                    out_logits=None, stream=None):
        _check(lib().dflash_draft_block(self.h, _stream(stream), len(slots), _i32(slots), _ptr(anchor),
                                        int(top_k), _ptr(out_ids), _ptr(out_vals), _ptr(out_logits)),
               "dflash_draft_block")

    def slot_reset(self, slot: int, keep_len: int):
        _check(lib().dflash_slot_reset(self.h, int(slot), int(keep_len)), "dflash_slot_reset")

    def slot_len(self, slot: int) -> int:
        v = ctypes.c_int32()
        _check(lib().dflash_slot_len(self.h, int(slot), ctypes.byref(v)), "dflash_slot_len")
        return v.value

    def profile_enable(self, kinds: Sequence[str], max_launches: int = 4096):
        mask = 0
        for k in kinds:
            mask |= 1 << KERNEL_KINDS.index(k)
        _check(lib().dflash_profile_enable(self.h, mask, int(max_launches)), "dflash_profile_enable")

    def profile_read(self) -> dict:
        n = len(KERNEL_KINDS)
        ms = (ctypes.c_double * n)()
        cnt = (ctypes.c_int32 * n)()
        _check(lib().dflash_profile_read(self.h, ms, cnt), "dflash_profile_read")
        return {KERNEL_KINDS[i]: (ms[i], cnt[i]) for i in range(n) if cnt[i]}

    def relay(self, slots: Sequence[int], n_acc: Sequence[int], cand, cand_stride: int, bonus,
              hidden: Sequence, w1, w2, stream=None):
        """dflow_relay: hidden holds L device tensors [sum(max(0, B-2-n)), Dt]
        (the reusable rejected-suffix features, grouped by request)."""
        ptrs = (ctypes.c_void_p * max(1, len(hidden)))(*[_ptr(t) for t in hidden])
        rw = dflow_relay_weights(_ptr(w1), _ptr(w2))
        _check(lib().dflow_relay(self.h, _stream(stream), len(slots), _i32(slots), _i32(n_acc), _ptr(cand),
                                 int(cand_stride), _ptr(bonus), ptrs, ctypes.byref(rw)), "dflow_relay")

    def select(self, n_req: int, anchor, cand, cand_logits, k: int, tables: dict, out_path, out_scores=None,
               stream=None):
        """dflash2_select over the most recent draft_block call's final hidden
        states; tables holds device tensors a, b [V, rank] and w_h [rank, D]."""
        sw = dflash2_selector_weights(_ptr(tables["a"]), _ptr(tables["b"]), _ptr(tables["w_h"]),
                                      int(tables["a"].shape[1]))
        _check(lib().dflash2_select(self.h, _stream(stream), int(n_req), _ptr(anchor), _ptr(cand),
                                    _ptr(cand_logits), int(k), ctypes.byref(sw), _ptr(out_path), _ptr(out_scores)),
               "dflash2_select")

    def conv_attach(self, layers=None):
        """dflash2_conv_attach: layers is a list of N dicts site -> {"w", "kbase"}
        (device tensors, kept alive here), or None to detach."""
        if layers is None:
            self._conv = None
            _check(lib().dflash2_conv_attach(self.h, None), "dflash2_conv_attach")
            return
        arr = (dflash2_conv_layer * self.d.N)()
        for l in range(self.d.N):
            for s in CONV_SITES:
                setattr(arr[l], s, dflash2_conv_site(_ptr(layers[l][s]["w"]), _ptr(layers[l][s]["kbase"])))
        _check(lib().dflash2_conv_attach(self.h, arr), "dflash2_conv_attach")
        self._conv = (layers, arr)

    def spec_draft(self, n_req: int, draft_logits, temperature: float, seed: int, req_id, cand, draft_lse=None,
                   stream=None):
        """dflash_spec_draft: Gumbel-max drafting from draft_logits [n_req, B-1, V]
        float (device) into cand [n_req, B-1] int32; optionally the rows'
        base-2 log-sum-exps into draft_lse [n_req, B-1] float."""
        _check(lib().dflash_spec_draft(self.h, _stream(stream), int(n_req), _ptr(draft_logits), float(temperature),
                                       int(seed), _ptr(req_id), _ptr(cand), _ptr(draft_lse)), "dflash_spec_draft")

    def spec_verify(self, n_req: int, draft_logits, target_logits, cand, temperature: float, seed: int, req_id,
                    tokens, tau, draft_lse=None, stream=None):
        """dflash_spec_verify: rejection-rule verification of one block per
        request; tokens [n_req, B] and tau [n_req] int32 (device) out."""
        _check(lib().dflash_spec_verify(self.h, _stream(stream), int(n_req), _ptr(draft_logits), _ptr(target_logits),
                                        _ptr(cand), _ptr(draft_lse), float(temperature), int(seed), _ptr(req_id),
                                        _ptr(tokens), _ptr(tau)), "dflash_spec_verify")

    def read_relay(self, slot: int, out, stream=None) -> int:
        n = ctypes.c_int32()
        _check(lib().dflow_read_relay(self.h, _stream(stream), int(slot), _ptr(out), ctypes.byref(n)),
               "dflow_read_relay")
        return n.value

    def read_cache(self, slot: int, layer: int, pos0: int, n: int, k_out, v_out, stream=None):
        _check(lib().dflash_read_cache(self.h, _stream(stream), int(slot), int(layer), int(pos0), int(n),
                                       _ptr(k_out), _ptr(v_out)), "dflash_read_cache")


def spec_draft_static(n_req: int, V: int, B: int, draft_logits, temperature: float, seed: int, req_id, cand,
                      draft_lse=None, stream=None):
    """dflash_spec_draft_static: dflash_spec_draft without a ctx or workspace
    (a fixed per-GPU scratch; allocates nothing)."""
    _check(lib().dflash_spec_draft_static(_stream(stream), int(n_req), int(V), int(B), _ptr(draft_logits),
                                          float(temperature), int(seed), _ptr(req_id), _ptr(cand), _ptr(draft_lse)),
           "dflash_spec_draft_static")


def accept(n_req: int, B: int, cand, cand_stride: int, target, tau, bonus, stream=None):
    _check(lib().dflash_accept(_stream(stream), int(n_req), int(B), _ptr(cand), int(cand_stride),
                               _ptr(target), _ptr(tau), _ptr(bonus)), "dflash_accept")
