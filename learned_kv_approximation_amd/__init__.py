"""Python binding of libkva.so, the MI355X (gfx950) KVA projector library.

Thin ctypes marshalling over the C ABI declared in include/kva.h: the
functions below carry the C names and take plain integers for device
pointers and the HIP stream.  Every step of the projection runs in the HIP
kernels of libkva.so; there is no Python or CPU fallback.  If the library has
not been built, loading it raises KvaError.

`Projector` is a convenience wrapper that fills the C structs from a config
dict and NumPy weights (see the `synth` package for their layout) and takes
torch tensors for device memory and the current stream.
"""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkva.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "kva.h")

c_i32, c_i64, c_f32, c_f64, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_void_p

KVA_OK, KVA_ERR_ARG, KVA_ERR_SHAPE, KVA_ERR_DTYPE = 0, 1, 2, 3
KVA_ERR_OOM, KVA_ERR_RANGE, KVA_ERR_UNSUPPORTED, KVA_ERR_HIP = 4, 5, 6, 7
DTYPES = {"f32": 0, "bf16": 1, "q8_0": 2, "q4_0": 3}
KINDS = {"deltanet": 0, "attn": 1, "draft": 2}


class kva_head_desc(ctypes.Structure):
    _fields_ = [("kind", c_i32), ("layer", c_i32), ("out_dim", c_i32)]


class kva_config(ctypes.Structure):
    _fields_ = [("n_in", c_i32), ("d_model", c_i32), ("n_blocks", c_i32), ("n_heads", c_i32),
                ("head_dim", c_i32), ("d_ffn", c_i32), ("attn_block", c_i32), ("max_tokens", c_i32),
                ("eps", c_f32), ("weight_dtype", c_i32), ("has_head_bias", c_i32),
                ("n_out_heads", c_i32), ("out_heads", ctypes.POINTER(kva_head_desc))]


class kva_block_weights(ctypes.Structure):
    _fields_ = [("attn_norm", c_vp), ("wq", c_vp), ("wk", c_vp), ("wv", c_vp), ("wo", c_vp),
                ("ffn_norm", c_vp), ("w_gate", c_vp), ("w_up", c_vp), ("w_down", c_vp)]


class kva_weights(ctypes.Structure):
    _fields_ = [("in_norm", c_vp), ("in_proj", c_vp), ("blocks", ctypes.POINTER(kva_block_weights)),
                ("out_norm", c_vp), ("head_w", ctypes.POINTER(c_vp)), ("head_b", ctypes.POINTER(c_vp))]


class kva_stats(ctypes.Structure):
    _fields_ = [("calls", ctypes.c_uint64), ("tokens", ctypes.c_uint64), ("blocks", ctypes.c_uint64),
                ("weight_bytes", ctypes.c_uint64), ("scratch_bytes", ctypes.c_uint64)]


class kva_stage_time(ctypes.Structure):
    _fields_ = [("launches", c_i32), ("total_ms", c_f64)]


STAGES = ["norm", "gemm_in", "gemm_qkv", "attn", "gemm_o", "gemm_gateup", "gemm_down", "gemm_heads"]


class kva_paged_kv(ctypes.Structure):
    _fields_ = [("k_pool", c_vp), ("v_pool", c_vp), ("page_table", c_vp), ("page_size", c_i32),
                ("n_pages", c_i32), ("n_logical", c_i32), ("n_kv_heads", c_i32), ("head_dim", c_i32),
                ("n_rot", c_i32), ("rope_base", c_f64), ("eps", c_f32), ("kv_type", c_i32)]


KVA_KV_BF16, KVA_KV_Q8_0_HADAMARD = 0, 1


class kva_attn_dest(ctypes.Structure):
    _fields_ = [("k_gain", c_vp), ("cache", kva_paged_kv)]


class kva_deltanet_layer(ctypes.Structure):
    _fields_ = [("mixer_in", c_vp), ("ld_in", c_i64), ("conv_w", c_vp), ("a_log", c_vp), ("dt_bias", c_vp),
                ("conv_state", c_vp), ("state", c_vp)]


class KvaError(RuntimeError):
    def __init__(self, status: int, where: str = ""):
        self.status = status
        name = _lib.kva_status_str(status).decode() if _lib is not None else str(status)
        detail = _lib.kva_last_error().decode() if _lib is not None else ""
        super().__init__(f"{where}: {name}: {detail}" if where else f"{name}: {detail}")


_lib = None

_SIGS = {
    "kva_validate_config": (c_i32, [ctypes.POINTER(kva_config)]),
    "kva_create": (c_i32, [ctypes.POINTER(kva_config), ctypes.POINTER(kva_weights), c_i32, ctypes.POINTER(c_vp)]),
    "kva_project_ubatch": (c_i32, [c_vp, c_vp, c_i32, ctypes.POINTER(c_vp), c_vp]),
    "kva_project_ubatch_kv": (c_i32, [c_vp, c_vp, c_i32, ctypes.POINTER(c_vp), c_i64,
                                      ctypes.POINTER(kva_attn_dest), c_i32, c_vp]),
    "kva_destroy": (c_i32, [c_vp]),
    "kva_map_create": (c_i32, [c_i32, c_i32, c_i32, ctypes.POINTER(c_vp), ctypes.POINTER(c_vp), c_i32, c_i32,
                               ctypes.POINTER(c_vp)]),
    "kva_map_project": (c_i32, [c_vp, c_vp, c_i32, ctypes.POINTER(c_vp), c_vp]),
    "kva_map_project_noalloc": (c_i32, [c_vp, c_vp, c_i32, ctypes.POINTER(c_vp), c_vp]),
    "kva_deltanet_update": (c_i32, [ctypes.POINTER(kva_deltanet_layer), c_i32, c_i32, c_i32, c_i32, c_i32, c_vp]),
    "kva_attn_kv_write": (c_i32, [c_vp, c_i64, c_i32, c_i64, c_vp, ctypes.POINTER(kva_paged_kv), c_vp]),
    "kva_debug_dequant_q8_0": (c_i32, [c_vp, c_i64, c_vp, c_vp]),
    "kva_debug_dequant_q8_0_f16": (c_i32, [c_vp, c_i64, c_vp, c_vp]),
    "kva_debug_dequant_q4_0_f16": (c_i32, [c_vp, c_i64, c_vp, c_vp]),
    "kva_debug_mfma_loop": (c_i32, [c_i32, c_i32, c_vp, c_vp]),
    "kva_debug_check_q8_scale": (c_i32, [c_vp, c_vp]),
    "kva_debug_copy_z": (c_i32, [c_vp, c_vp, c_i32, c_vp]),
    "kva_debug_poison_scratch": (c_i32, [c_vp, c_vp]),
    "kva_debug_head_plan": (c_i32, [ctypes.POINTER(kva_config), ctypes.POINTER(c_i32), c_vp, c_vp, c_i64]),
    "kva_debug_host_to_f16": (c_i32, [c_vp, c_i32, c_i64, c_vp]),
    "kva_debug_pack_weight": (c_i32, [c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_i64, c_vp, c_i64]),
    "kva_get_stats": (c_i32, [c_vp, ctypes.POINTER(kva_stats)]),
    "kva_profile_enable": (c_i32, [c_vp, ctypes.c_uint32]),
    "kva_profile_read": (c_i32, [c_vp, ctypes.POINTER(kva_stage_time)]),
    "kva_status_str": (ctypes.c_char_p, [c_i32]),
    "kva_last_error": (ctypes.c_char_p, []),
}


def lib():
    """Load libkva.so once (raises KvaError-like RuntimeError if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        # PyTorch ships its own HIP runtime under the same soname as the one
        # libkva.so links: load torch first so that the process has one HIP
        # runtime (the library loaded first would otherwise be torch's too).
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def header_exports() -> list:
    """Names of the functions include/kva.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kva_\w+)\s*\(", text, re.M)))


def _check(status: int, where: str):
    if status != KVA_OK:
        raise KvaError(status, where)


# ------------------------------------------------------------------ C-named entry points

def kva_validate_config(cfg: kva_config) -> int:
    return lib().kva_validate_config(ctypes.byref(cfg))


def kva_create(cfg: kva_config, weights: kva_weights, device: int = 0) -> int:
    out = c_vp()
    _check(lib().kva_create(ctypes.byref(cfg), ctypes.byref(weights), device, ctypes.byref(out)), "kva_create")
    return out.value


def kva_project_ubatch(ctx: int, x_ptr: int, n_tokens: int, head_out_ptrs, stream: int = 0) -> None:
    arr = (c_vp * len(head_out_ptrs))(*head_out_ptrs)
    _check(lib().kva_project_ubatch(ctx, x_ptr, n_tokens, arr, stream), "kva_project_ubatch")


def kva_project_ubatch_kv(ctx: int, x_ptr: int, n_tokens: int, head_out_ptrs, pos0: int, dests,
                          stream: int = 0) -> None:
    """dests: sequence of kva_attn_dest, one per fused attention head (head order)."""
    arr = (c_vp * len(head_out_ptrs))(*head_out_ptrs)
    d = (kva_attn_dest * max(1, len(dests)))(*dests)
    _check(lib().kva_project_ubatch_kv(ctx, x_ptr, n_tokens, arr, pos0, d, len(dests), stream),
           "kva_project_ubatch_kv")


def kva_deltanet_update(layers, n_tokens: int, n_k_heads: int = 16, n_v_heads: int = 48, head_dim: int = 128,
                        stream: int = 0) -> None:
    """layers: sequence of kva_deltanet_layer."""
    arr = (kva_deltanet_layer * max(1, len(layers)))(*layers)
    _check(lib().kva_deltanet_update(arr, len(layers), n_tokens, n_k_heads, n_v_heads, head_dim, stream),
           "kva_deltanet_update")


def kva_map_create(n_in: int, n_maps: int, weight_dtype: int, w_ptrs, b_ptrs, max_tokens: int,
                   device: int = 0) -> int:
    """w_ptrs / b_ptrs: host pointers (ints) per map; b_ptrs may be None."""
    wa = (c_vp * n_maps)(*w_ptrs)
    ba = (c_vp * n_maps)(*b_ptrs) if b_ptrs is not None else None
    out = c_vp()
    _check(lib().kva_map_create(n_in, n_maps, weight_dtype, wa, ba, max_tokens, device, ctypes.byref(out)),
           "kva_map_create")
    return out.value


def kva_map_project(ctx: int, x_ptr: int, n_tokens: int, out_ptrs, stream: int = 0) -> None:
    arr = (c_vp * len(out_ptrs))(*out_ptrs)
    _check(lib().kva_map_project(ctx, x_ptr, n_tokens, arr, stream), "kva_map_project")


def kva_map_project_noalloc(ctx: int, x_ptr: int, n_tokens: int, out_ptrs, stream: int = 0) -> None:
    arr = (c_vp * len(out_ptrs))(*out_ptrs)
    _check(lib().kva_map_project_noalloc(ctx, x_ptr, n_tokens, arr, stream), "kva_map_project_noalloc")


class MapProjector:
    """Owns a single-map context built from NumPy maps ([n_in][n_in] each, in
    the storage format of `dtype`) and optional fp32 biases."""

    def __init__(self, maps, biases=None, dtype: str = "bf16", n_in: int | None = None,
                 max_tokens: int = 1024, device: int = 0):
        import numpy as np
        self.n_in = int(n_in if n_in is not None else maps[0].shape[-1])
        self.n_maps = len(maps)
        self._keep = [np.ascontiguousarray(m) for m in maps]
        self._keep_b = [np.ascontiguousarray(b, dtype=np.float32) for b in biases] if biases is not None else None
        self.ctx = kva_map_create(self.n_in, self.n_maps, DTYPES[dtype], [m.ctypes.data for m in self._keep],
                                  [b.ctypes.data for b in self._keep_b] if self._keep_b is not None else None,
                                  max_tokens, device)
        del self._keep, self._keep_b

    def project(self, x, outs=None, stream: int | None = None):
        import torch
        n = x.shape[0]
        if outs is None:
            outs = [torch.empty((n, self.n_in), dtype=torch.float32, device=x.device) for _ in range(self.n_maps)]
        kva_map_project(self.ctx, x.data_ptr(), n, [o.data_ptr() for o in outs],
                        current_stream() if stream is None else stream)
        return outs

    def close(self):
        if getattr(self, "ctx", None):
            kva_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def kva_destroy(ctx: int) -> None:
    _check(lib().kva_destroy(ctx), "kva_destroy")


def kva_attn_kv_write(kv_ptr: int, ld_kv: int, n_tokens: int, pos0: int, k_gain_ptr: int,
                      cache: kva_paged_kv, stream: int = 0) -> None:
    _check(lib().kva_attn_kv_write(kv_ptr, ld_kv, n_tokens, pos0, k_gain_ptr, ctypes.byref(cache), stream),
           "kva_attn_kv_write")


def kva_debug_dequant_q8_0(blocks_ptr: int, n_blocks: int, out_ptr: int, stream: int = 0) -> None:
    _check(lib().kva_debug_dequant_q8_0(blocks_ptr, n_blocks, out_ptr, stream), "kva_debug_dequant_q8_0")


def kva_debug_mfma_loop(n_iter: int, n_workgroups: int, sink_ptr: int, stream: int = 0) -> None:
    _check(lib().kva_debug_mfma_loop(n_iter, n_workgroups, sink_ptr, stream), "kva_debug_mfma_loop")


def kva_debug_dequant_q4_0_f16(blocks_ptr: int, n_blocks: int, out_ptr: int, stream: int = 0) -> None:
    _check(lib().kva_debug_dequant_q4_0_f16(blocks_ptr, n_blocks, out_ptr, stream), "kva_debug_dequant_q4_0_f16")


def kva_debug_check_q8_scale(counts_ptr: int, stream: int = 0) -> None:
    _check(lib().kva_debug_check_q8_scale(counts_ptr, stream), "kva_debug_check_q8_scale")


def kva_debug_dequant_q8_0_f16(blocks_ptr: int, n_blocks: int, out_ptr: int, stream: int = 0) -> None:
    _check(lib().kva_debug_dequant_q8_0_f16(blocks_ptr, n_blocks, out_ptr, stream), "kva_debug_dequant_q8_0_f16")


def kva_debug_copy_z(ctx: int, dst_ptr: int, n_tokens: int, stream: int = 0) -> None:
    _check(lib().kva_debug_copy_z(ctx, dst_ptr, n_tokens, stream), "kva_debug_copy_z")


def kva_debug_poison_scratch(ctx: int, stream: int = 0) -> None:
    _check(lib().kva_debug_poison_scratch(ctx, stream), "kva_debug_poison_scratch")


def kva_debug_head_plan(cfg: kva_config):
    import numpy as np
    n = c_i32()
    _check(lib().kva_debug_head_plan(ctypes.byref(cfg), ctypes.byref(n), None, None, 0), "kva_debug_head_plan")
    head = np.empty(n.value, dtype=np.int32)
    idx = np.empty(n.value, dtype=np.int32)
    _check(lib().kva_debug_head_plan(ctypes.byref(cfg), ctypes.byref(n), head.ctypes.data, idx.ctypes.data,
                                     n.value), "kva_debug_head_plan")
    return head, idx


def kva_debug_host_to_f16(src, src_dtype: str):
    """Host conversion used for trunk weights; returns (status, fp16 bits)."""
    import numpy as np
    src = np.ascontiguousarray(src)
    dst = np.empty(src.size, dtype=np.uint16)
    st = lib().kva_debug_host_to_f16(src.ctypes.data, DTYPES[src_dtype], src.size, dst.ctypes.data)
    return st, dst.reshape(src.shape)


PACK_TARGETS = {"f16": 0, "bf16": 1, "q8_0": 2, "q4_0": 3}


def kva_debug_pack_weight(src, src_dtype: str, rows: int, K: int, target: str):
    """Host packing of one weight as kva_create lays it out; returns
    (status, values or codes as bytes, scales or None)."""
    import numpy as np
    src = np.ascontiguousarray(src)
    rpad = (rows + 255) // 256 * 256
    quant = target in ("q8_0", "q4_0")
    nbytes = rpad * K * 2 if not quant else (rpad * K if target == "q8_0" else rpad * K // 2)
    out = np.zeros(nbytes, dtype=np.uint8)
    sc = np.zeros(rpad * (K // 32), dtype=np.uint16) if quant else None
    st = lib().kva_debug_pack_weight(src.ctypes.data, DTYPES[src_dtype], rows, K, PACK_TARGETS[target],
                                     out.ctypes.data, out.size, sc.ctypes.data if quant else None,
                                     sc.size if quant else 0)
    return st, out, sc


def kva_get_stats(ctx: int) -> dict:
    s = kva_stats()
    _check(lib().kva_get_stats(ctx, ctypes.byref(s)), "kva_get_stats")
    return {k: getattr(s, k) for k, _ in kva_stats._fields_}


def kva_profile_enable(ctx: int, stage_mask: int) -> None:
    _check(lib().kva_profile_enable(ctx, stage_mask), "kva_profile_enable")


def kva_profile_read(ctx: int) -> dict:
    """{stage name: (launches, total_ms)} since the last read (waits for the events)."""
    arr = (kva_stage_time * len(STAGES))()
    _check(lib().kva_profile_read(ctx, arr), "kva_profile_read")
    return {STAGES[i]: (arr[i].launches, arr[i].total_ms) for i in range(len(STAGES))}


# ------------------------------------------------------------------ struct builders

def make_config(cfg: dict, max_tokens: int | None = None):
    """kva_config for a config dict (synth.config layout).  Returns (struct, keepalive)."""
    heads = (kva_head_desc * len(cfg["heads"]))(
        *[kva_head_desc(KINDS[h["kind"]], h["layer"], h["out_dim"]) for h in cfg["heads"]])
    c = kva_config(cfg["n_in"], cfg["d_model"], cfg["n_blocks"], cfg["n_heads"], cfg["head_dim"],
                   cfg["d_ffn"], cfg["attn_block"], int(max_tokens or cfg["n_tokens"]), cfg["eps"],
                   DTYPES[cfg["weight_dtype"]], 1 if cfg["has_head_bias"] else 0, len(cfg["heads"]),
                   ctypes.cast(heads, ctypes.POINTER(kva_head_desc)))
    return c, heads


def make_weights(cfg: dict, w: dict):
    """kva_weights pointing at host NumPy arrays.  Returns (struct, keepalive)."""
    import numpy as np
    keep = []

    def p(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        keep.append(a)
        return a.ctypes.data

    blocks = (kva_block_weights * len(w["blocks"]))(*[
        kva_block_weights(p(b["attn_norm"]), p(b["wq"]), p(b["wk"]), p(b["wv"]), p(b["wo"]),
                          p(b["ffn_norm"]), p(b["w_gate"]), p(b["w_up"]), p(b["w_down"]))
        for b in w["blocks"]])
    hw = (c_vp * len(w["heads"]))(*[p(h["w"]) for h in w["heads"]])
    hb = (c_vp * len(w["heads"]))(*[p(h["b"]) for h in w["heads"]]) if cfg["has_head_bias"] else None
    keep += [blocks, hw, hb]
    s = kva_weights(p(w["in_norm"]), p(w["in_proj"]), ctypes.cast(blocks, ctypes.POINTER(kva_block_weights)),
                    p(w["out_norm"]), ctypes.cast(hw, ctypes.POINTER(c_vp)),
                    ctypes.cast(hb, ctypes.POINTER(c_vp)) if hb is not None else None)
    return s, keep


def current_stream() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


class Projector:
    """Owns a kva_ctx built from a config dict and NumPy weights."""

    def __init__(self, cfg: dict, weights: dict, max_tokens: int | None = None, device: int = 0):
        self.cfg = cfg
        self.max_tokens = int(max_tokens or cfg["n_tokens"])
        c, self._keep_c = make_config(cfg, self.max_tokens)
        w, keep_w = make_weights(cfg, weights)
        self._c = c
        self.ctx = kva_create(c, w, device)
        del keep_w

    def alloc_outputs(self, n_tokens: int, device="cuda"):
        import torch
        return [torch.empty((n_tokens, h["out_dim"]), dtype=torch.float32, device=device)
                for h in self.cfg["heads"]]

    def project(self, x, outs=None, stream: int | None = None):
        """x: [n, n_in] fp32 cuda tensor.  Returns the per-head fp32 outputs."""
        assert x.is_cuda and x.dtype.is_floating_point and x.dtype.itemsize == 4 and x.is_contiguous()
        n = x.shape[0]
        assert x.shape[1] == self.cfg["n_in"]
        if outs is None:
            outs = self.alloc_outputs(n, x.device)
        for o, h in zip(outs, self.cfg["heads"]):
            assert o.is_contiguous() and o.shape[0] >= n and o.shape[1] == h["out_dim"]
        kva_project_ubatch(self.ctx, x.data_ptr(), n, [o.data_ptr() for o in outs],
                           current_stream() if stream is None else stream)
        return outs

    def copy_z(self, n_tokens: int):
        import torch
        z = torch.empty((n_tokens, self.cfg["d_model"]), dtype=torch.int16, device="cuda")
        kva_debug_copy_z(self.ctx, z.data_ptr(), n_tokens, current_stream())
        return z

    def stats(self) -> dict:
        return kva_get_stats(self.ctx)

    def close(self):
        if getattr(self, "ctx", None):
            kva_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
