"""Python binding of libclha, the CLHA calibration library for MI355X (gfx950).

Argument marshalling only: every step of the calibration path runs in the HIP
kernels behind the C ABI declared in ``include/clha.h``.  PyTorch supplies
device memory (tensors) and streams; this module checks dtypes, shapes and
devices, passes raw pointers through ctypes and turns non-zero status codes
into ``ClhaError``.  The library must be built (``python
gptq_calibration_moe_amd/build.py``); without it, importing the binding raises.

Names follow the C entry points: ``Context.collect_hessians`` calls
``clha_collect_hessians`` and so on.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libclha.so")

OK, ERR_INVALID_ARG, ERR_SHAPE, ERR_ALIGN, ERR_HIP, ERR_NOT_PD, ERR_NONFINITE, ERR_WORKSPACE = range(8)
STATUS_NAMES = {0: "OK", 1: "INVALID_ARG", 2: "SHAPE", 3: "ALIGN", 4: "HIP", 5: "NOT_PD",
                6: "NONFINITE", 7: "WORKSPACE"}
ALPHA_MODES = {"rt": 0, "eq": 1, "explicit": 2, "explicit_slot": 3}
F32, BF16 = 0, 1
GPTQ_ACT_ORDER, GPTQ_STATIC_GROUPS = 1, 2   # clha_gptq_flag

EXPORTS = (
    "clha_create", "clha_destroy", "clha_last_error", "clha_num_slots", "clha_register_layer",
    "clha_reset_layer",
    "clha_collect_workspace_bytes", "clha_collect_hessians", "clha_aggregate",
    "clha_gptq_workspace_bytes", "clha_gptq_quantize", "clha_gptq_workspace_bytes_ex",
    "clha_gptq_quantize_ex", "clha_inverse_cholesky_workspace_bytes",
    "clha_inverse_cholesky", "clha_loss_workspace_bytes", "clha_loss", "clha_set_timing",
    "clha_read_timing", "clha_sync", "clha_pack_codes", "clha_unpack_codes",
    "clha_down_workspace_bytes", "clha_collect_down_hessians", "clha_loss_static",
)
STAGES = ("route", "bucket", "gather", "syrk", "aggregate", "factor", "gptq", "loss", "syrk_reduce")


class ClhaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"CLHA_ERR_{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class MoeDesc(C.Structure):
    _fields_ = [("d", C.c_int32), ("n_routed", C.c_int32), ("top_k", C.c_int32),
                ("n_shared", C.c_int32), ("max_tokens", C.c_int64)]


class GptqJob(C.Structure):
    _fields_ = [("H", C.c_void_p), ("W", C.c_void_p), ("w_dtype", C.c_int32), ("rows", C.c_int32),
                ("bits", C.c_int32), ("pad_", C.c_int32), ("codes", C.c_void_p),
                ("scales", C.c_void_p), ("zeros", C.c_void_p), ("loss", C.c_void_p),
                ("H_eval", C.c_void_p), ("loss_eval", C.c_void_p), ("dead", C.c_void_p),
                ("status", C.c_void_p)]


def _load() -> C.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with "
                          "`python gptq_calibration_moe_amd/build.py`")
    lib = C.CDLL(LIB_PATH)
    vp, i32, i64, sz, f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t, C.c_float
    sig = {
        "clha_create": ([C.POINTER(MoeDesc), C.POINTER(vp)], i32),
        "clha_destroy": ([vp], i32),
        "clha_last_error": ([vp], C.c_char_p),
        "clha_num_slots": ([vp], i32),
        "clha_register_layer": ([vp, i32, vp, vp], i32),
        "clha_reset_layer": ([vp, i32, vp], i32),
        "clha_pack_codes": ([vp, i64, i32, vp, vp, vp], i32),
        "clha_down_workspace_bytes": ([vp, i32], sz),
        "clha_collect_down_hessians": ([vp, i32, i64, i32, i32, vp, vp, vp, vp, vp, sz, vp], i32),
        "clha_unpack_codes": ([vp, i64, i32, vp, vp, vp], i32),
        "clha_collect_workspace_bytes": ([vp], sz),
        "clha_collect_hessians": ([vp, i32, i64, vp, vp, vp, vp, vp, vp, sz, vp], i32),
        "clha_aggregate": ([vp, i32, C.POINTER(i32), i32, C.POINTER(f32), vp, vp, vp], i32),
        "clha_gptq_workspace_bytes": ([vp, i32, C.POINTER(GptqJob), i32], sz),
        "clha_gptq_quantize": ([vp, i32, C.POINTER(GptqJob), i32, i32, i32, f32, vp, sz, vp], i32),
        "clha_gptq_workspace_bytes_ex": ([vp, i32, C.POINTER(GptqJob), i32, C.c_uint32], sz),
        "clha_gptq_quantize_ex": ([vp, i32, C.POINTER(GptqJob), i32, i32, i32, f32, C.c_uint32,
                                   C.POINTER(vp), vp, sz, vp], i32),
        "clha_inverse_cholesky_workspace_bytes": ([vp, i32, i32], sz),
        "clha_inverse_cholesky": ([vp, i32, C.POINTER(vp), i32, f32, vp, vp, vp, vp, sz, vp], i32),
        "clha_loss_workspace_bytes": ([vp, i32, i32], sz),
        "clha_loss": ([vp, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp], i32),
        "clha_loss_static": ([vp, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp], i32),
        "clha_set_timing": ([vp, i32], i32),
        "clha_read_timing": ([vp, C.POINTER(C.c_double), C.POINTER(i64), i32], i32),
        "clha_sync": ([vp, vp], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


lib = _load()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _check_dev(name, t, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _bits16(t: torch.Tensor) -> torch.Tensor:
    """bf16 (or int16/uint16 bit patterns) viewed as 16-bit words; no copy."""
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return t
    raise TypeError(f"expected bf16 activations, got {t.dtype}")


class Context:
    """One clha_ctx: the shape of an MoE block whose routed experts a group of
    layers shares, with the layer registry and a cached device workspace."""

    def __init__(self, d: int, n_routed: int, top_k: int, n_shared: int, max_tokens: int,
                 device: Optional[torch.device] = None):
        dev = torch.device("cuda") if device is None else torch.device(device)
        if dev.type != "cuda":
            raise ValueError("the CLHA library runs on a HIP device")
        self.device = torch.device("cuda", dev.index if dev.index is not None else torch.cuda.current_device())
        self.desc = MoeDesc(d, n_routed, top_k, n_shared, max_tokens)
        h = C.c_void_p()
        with torch.cuda.device(self.device):
            st = lib.clha_create(C.byref(self.desc), C.byref(h))
        if st != OK:
            raise ClhaError(st, "clha_create rejected the block shape")
        self._h = h
        self.d, self.n_routed, self.top_k, self.n_shared = d, n_routed, top_k, n_shared
        self.max_tokens = max_tokens
        self.slots = lib.clha_num_slots(h)
        self._ws = {}
        self._layers = {}

    # ------------------------------------------------------------------ plumbing
    def close(self):
        if getattr(self, "_h", None):
            lib.clha_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _raise(self, st):
        if st != OK:
            raise ClhaError(st, lib.clha_last_error(self._h).decode())

    def workspace(self, key: str, nbytes: int) -> torch.Tensor:
        ws = self._ws.get(key)
        if ws is None or ws.numel() < nbytes:
            ws = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=self.device)
            self._ws[key] = ws
        return ws

    def new_layer_buffers(self):
        """Zeroed (S, counts) accumulators for one layer."""
        S = torch.zeros(self.slots, self.d, self.d, dtype=torch.float32, device=self.device)
        n = torch.zeros(self.slots, dtype=torch.int64, device=self.device)
        return S, n

    # ------------------------------------------------------------------ C entry points
    def register_layer(self, layer: int, S: torch.Tensor, counts: torch.Tensor):
        _check_dev("S", S, torch.float32, (self.slots, self.d, self.d), self.device)
        _check_dev("counts", counts, torch.int64, (self.slots,), self.device)
        self._raise(lib.clha_register_layer(self._h, layer, _ptr(S), _ptr(counts)))
        self._layers[layer] = (S, counts)

    def reset_layer(self, layer: int, stream=None):
        """New accumulation for a registered layer: counts zeroed now, and the next
        collection with tokens overwrites S instead of adding (no clearing of S)."""
        self._raise(lib.clha_reset_layer(self._h, layer, _stream(stream)))

    def collect_down_hessians(self, layer: int, x: torch.Tensor, token_ids: torch.Tensor,
                              offsets: torch.Tensor, wgu: Sequence[torch.Tensor], n_routed: int,
                              workspace: Optional[torch.Tensor] = None, stream=None):
        """down_proj inputs of one layer on a down_proj context (d = f, one slot per
        routed and per shared expert, no shared slot): h = bf16(silu(x Wg^T) * (x Wu^T))
        per slot, over the routing (token_ids, offsets) of the same batch on the block's
        main context for routed slots and all tokens for the shared ones; S[slot] += h^T h."""
        n, dm = x.shape
        _check_dev("x", x, (torch.bfloat16, torch.int16, torch.uint16), (n, dm), self.device)
        if len(wgu) != self.slots:
            raise ValueError(f"wgu needs one [2f, d_model] weight per slot ({self.slots})")
        for w in wgu:
            _check_dev("wgu", w, (torch.bfloat16, torch.int16, torch.uint16), (2 * self.d, dm), self.device)
        _check_dev("token_ids", token_ids, torch.int32, (token_ids.numel(),), self.device)
        _check_dev("offsets", offsets, torch.int64, (n_routed + 1,), self.device)
        need = lib.clha_down_workspace_bytes(self._h, n_routed)
        ws = workspace if workspace is not None else self.workspace("down", need)
        table = (C.c_void_p * len(wgu))(*[w.data_ptr() for w in wgu])
        self._raise(lib.clha_collect_down_hessians(
            self._h, layer, n, dm, n_routed, _ptr(x), _ptr(token_ids), _ptr(offsets), table,
            _ptr(ws), ws.numel(), _stream(stream)))

    def pack_codes(self, codes: torch.Tensor, bits: int, out: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
        """b-bit packing of a uint8 code tensor (last dimension a multiple of 8):
        returns uint8 [..., cols * bits / 8]."""
        if codes.dtype != torch.uint8 or codes.device != self.device or not codes.is_contiguous():
            raise ValueError("codes must be a contiguous uint8 tensor on the context's device")
        if codes.shape[-1] % 8:
            raise ValueError("the last dimension of codes must be a multiple of 8")
        shape = (*codes.shape[:-1], codes.shape[-1] * bits // 8)
        if out is None:
            out = torch.empty(shape, dtype=torch.uint8, device=self.device)
        _check_dev("packed", out, torch.uint8, shape, self.device)
        self._raise(lib.clha_pack_codes(self._h, codes.numel(), bits, _ptr(codes), _ptr(out), _stream(stream)))
        return out

    def unpack_codes(self, packed: torch.Tensor, bits: int, cols: int, stream=None) -> torch.Tensor:
        """Inverse of pack_codes: uint8 [..., cols] codes from [..., cols * bits / 8] bytes."""
        if packed.dtype != torch.uint8 or packed.device != self.device or not packed.is_contiguous():
            raise ValueError("packed must be a contiguous uint8 tensor on the context's device")
        if cols % 8 or packed.shape[-1] != cols * bits // 8:
            raise ValueError("cols must be a multiple of 8 and match the packed width")
        out = torch.empty((*packed.shape[:-1], cols), dtype=torch.uint8, device=self.device)
        self._raise(lib.clha_unpack_codes(self._h, out.numel(), bits, _ptr(packed), _ptr(out), _stream(stream)))
        return out

    def collect_workspace_bytes(self) -> int:
        return lib.clha_collect_workspace_bytes(self._h)

    def collect_hessians(self, layer: int, x: torch.Tensor, logits: torch.Tensor,
                         topk_out: Optional[torch.Tensor] = None,
                         offsets_out: Optional[torch.Tensor] = None,
                         token_ids_out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None):
        n = x.shape[0]
        _check_dev("x", x, (torch.bfloat16, torch.int16, torch.uint16), (n, self.d), self.device)
        _check_dev("logits", logits, torch.float32, (n, self.n_routed), self.device)
        if topk_out is not None:
            _check_dev("topk_out", topk_out, torch.int32, (n, self.top_k), self.device)
        if offsets_out is not None:
            _check_dev("offsets_out", offsets_out, torch.int64, (self.n_routed + 1,), self.device)
        if token_ids_out is not None:
            _check_dev("token_ids_out", token_ids_out, torch.int32, (n * self.top_k,), self.device)
        need = self.collect_workspace_bytes()
        ws = workspace if workspace is not None else self.workspace("collect", need)
        self._raise(lib.clha_collect_hessians(
            self._h, layer, n, _ptr(_bits16(x)), _ptr(logits), _ptr(topk_out), _ptr(offsets_out),
            _ptr(token_ids_out), _ptr(ws), ws.numel(), _stream(stream)))

    def aggregate(self, layers: Sequence[int], mode: str, H_out: torch.Tensor,
                  alpha=None, alpha_out: Optional[torch.Tensor] = None, stream=None):
        """alpha: host sequence of n_layers weights ('explicit'), or a device
        float32 tensor [slots, n_layers] of per-slot weights ('explicit_slot')."""
        _check_dev("H_out", H_out, torch.float32, (self.slots, self.d, self.d), self.device)
        if alpha_out is not None:
            _check_dev("alpha_out", alpha_out, torch.float32, (self.slots, len(layers)), self.device)
        arr = (C.c_int32 * len(layers))(*layers)
        if mode == "explicit_slot":
            _check_dev("alpha", alpha, torch.float32, (self.slots, len(layers)), self.device)
            al = C.cast(C.c_void_p(alpha.data_ptr()), C.POINTER(C.c_float))
        else:
            al = None if alpha is None else (C.c_float * len(alpha))(*alpha)
        self._raise(lib.clha_aggregate(self._h, len(layers), arr, ALPHA_MODES[mode], al,
                                       _ptr(H_out), _ptr(alpha_out), _stream(stream)))

    def _jobs(self, jobs, cols):
        arr = (GptqJob * len(jobs))()
        for i, j in enumerate(jobs):
            W = j["W"]
            rows = W.shape[0]
            _check_dev("H", j["H"], torch.float32, (cols, cols), self.device)
            _check_dev("W", W, (torch.float32, torch.bfloat16), (rows, cols), self.device)
            _check_dev("codes", j["codes"], torch.uint8, (rows, cols), self.device)
            _check_dev("scales", j["scales"], torch.float32, (rows, j["scales"].shape[1]), self.device)
            _check_dev("zeros", j["zeros"], torch.uint8, (rows, j["scales"].shape[1]), self.device)
            if j.get("loss") is not None:
                _check_dev("loss", j["loss"], torch.float32, None, self.device)
            if j.get("H_eval") is not None:
                _check_dev("H_eval", j["H_eval"], torch.float32, (cols, cols), self.device)
            if j.get("loss_eval") is not None:
                _check_dev("loss_eval", j["loss_eval"], torch.float32, None, self.device)
            if j.get("dead") is not None:
                _check_dev("dead", j["dead"], torch.uint8, (cols,), self.device)
            if j.get("status") is not None:
                _check_dev("status", j["status"], torch.int32, None, self.device)

            def opt(k):
                return j[k].data_ptr() if j.get(k) is not None else None
            arr[i] = GptqJob(j["H"].data_ptr(), W.data_ptr(), BF16 if W.dtype == torch.bfloat16 else F32,
                             rows, int(j["bits"]), 0, j["codes"].data_ptr(), j["scales"].data_ptr(),
                             j["zeros"].data_ptr(), opt("loss"), opt("H_eval"), opt("loss_eval"),
                             opt("dead"), opt("status"))
        return arr

    class PreparedGptq:
        """A checked, marshalled job batch for repeated clha_gptq_quantize calls."""

        def __init__(self, arr, n, cols, ws, flags=0):
            self.arr, self.n, self.cols, self.ws, self.flags = arr, n, cols, ws, flags

    def prepare_gptq(self, jobs, cols: int, act_order: bool = False,
                     static_groups: bool = False,
                     workspace: Optional[torch.Tensor] = None) -> "Context.PreparedGptq":
        """Checks and marshals a job batch.  `workspace` (uint8 device tensor) may be
        shared by batches that run one after another on one stream and must hold
        clha_gptq_workspace_bytes_ex bytes."""
        arr = self._jobs(jobs, cols)
        flags = (GPTQ_ACT_ORDER if act_order else 0) | (GPTQ_STATIC_GROUPS if static_groups else 0)
        need = lib.clha_gptq_workspace_bytes_ex(self._h, len(jobs), arr, cols, flags)
        if workspace is not None:
            _check_dev("workspace", workspace, torch.uint8, None, self.device)
            if workspace.numel() < need:
                raise ValueError(f"GPTQ workspace of {workspace.numel()} bytes < {need} needed")
            ws = workspace
        else:
            ws = torch.empty(max(int(need), 256), dtype=torch.uint8, device=self.device)
        prep = Context.PreparedGptq(arr, len(jobs), cols, ws, flags)
        prep.tensors = jobs          # keep the job tensors alive with the pointers
        return prep

    def run_gptq(self, prep: "Context.PreparedGptq", group: int, block: int = 128,
                 damp: float = 0.01, stream=None):
        if prep.flags:
            self._raise(lib.clha_gptq_quantize_ex(self._h, prep.n, prep.arr, prep.cols, group, block,
                                                  damp, prep.flags, None, _ptr(prep.ws), prep.ws.numel(),
                                                  _stream(stream)))
            return
        self._raise(lib.clha_gptq_quantize(self._h, prep.n, prep.arr, prep.cols, group, block,
                                           damp, _ptr(prep.ws), prep.ws.numel(), _stream(stream)))

    def gptq_workspace_bytes(self, jobs, cols: int, act_order: bool = False,
                             static_groups: bool = False) -> int:
        arr = self._jobs(jobs, cols)
        flags = (GPTQ_ACT_ORDER if act_order else 0) | (GPTQ_STATIC_GROUPS if static_groups else 0)
        return lib.clha_gptq_workspace_bytes_ex(self._h, len(jobs), arr, cols, flags)

    def gptq_quantize(self, jobs, cols: int, group: int, block: int = 128, damp: float = 0.01,
                      workspace: Optional[torch.Tensor] = None, stream=None,
                      act_order: bool = False, static_groups: bool = False):
        """jobs: list of dicts with H, W, bits, codes, scales, zeros and optional loss,
        H_eval with loss_eval (the result's loss under a second Hessian), dead (uint8
        [cols]), status (int32 [1]: the job's clha_status code) and g_idx (device int32
        [cols], receives each column's grid index).  act_order and static_groups select
        clha_gptq_quantize_ex's options."""
        arr = self._jobs(jobs, cols)
        flags = (GPTQ_ACT_ORDER if act_order else 0) | (GPTQ_STATIC_GROUPS if static_groups else 0)
        gi = [j.get("g_idx") for j in jobs]
        if not flags and all(g is None for g in gi):
            need = lib.clha_gptq_workspace_bytes(self._h, len(jobs), arr, cols)
            ws = workspace if workspace is not None else self.workspace("gptq", need)
            self._raise(lib.clha_gptq_quantize(self._h, len(jobs), arr, cols, group, block, damp,
                                               _ptr(ws), ws.numel(), _stream(stream)))
            return
        for g in gi:
            if g is not None:
                _check_dev("g_idx", g, torch.int32, (cols,), self.device)
        garr = (C.c_void_p * len(jobs))(*[g.data_ptr() if g is not None else None for g in gi])
        need = lib.clha_gptq_workspace_bytes_ex(self._h, len(jobs), arr, cols, flags)
        ws = workspace if workspace is not None else self.workspace("gptq", need)
        self._raise(lib.clha_gptq_quantize_ex(self._h, len(jobs), arr, cols, group, block, damp, flags,
                                              garr, _ptr(ws), ws.numel(), _stream(stream)))

    def inverse_cholesky(self, H: Sequence[torch.Tensor], U_out: torch.Tensor, damp: float = 0.01,
                         lambda_out: Optional[torch.Tensor] = None,
                         dead_out: Optional[torch.Tensor] = None, stream=None):
        n = len(H)
        cols = U_out.shape[-1]
        for h in H:
            _check_dev("H", h, torch.float32, (cols, cols), self.device)
        _check_dev("U_out", U_out, torch.float32, (n, cols, cols), self.device)
        if lambda_out is not None:
            _check_dev("lambda_out", lambda_out, torch.float32, (n,), self.device)
        if dead_out is not None:
            _check_dev("dead_out", dead_out, torch.uint8, (n, cols), self.device)
        ptrs = (C.c_void_p * n)(*[h.data_ptr() for h in H])
        need = lib.clha_inverse_cholesky_workspace_bytes(self._h, n, cols)
        ws = self.workspace("chol", need)
        self._raise(lib.clha_inverse_cholesky(self._h, n, ptrs, cols, damp, _ptr(U_out),
                                              _ptr(lambda_out), _ptr(dead_out), _ptr(ws),
                                              ws.numel(), _stream(stream)))

    def loss(self, W: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
             H: torch.Tensor, group: int, loss_out: torch.Tensor, stream=None):
        rows, cols = W.shape
        _check_dev("W", W, (torch.float32, torch.bfloat16), (rows, cols), self.device)
        _check_dev("codes", codes, torch.uint8, (rows, cols), self.device)
        _check_dev("scales", scales, torch.float32, (rows, cols // group), self.device)
        _check_dev("zeros", zeros, torch.uint8, (rows, cols // group), self.device)
        _check_dev("H", H, torch.float32, (cols, cols), self.device)
        _check_dev("loss_out", loss_out, torch.float32, None, self.device)
        need = lib.clha_loss_workspace_bytes(self._h, rows, cols)
        ws = self.workspace("loss", need)
        self._raise(lib.clha_loss(self._h, rows, cols, group, _ptr(W),
                                  BF16 if W.dtype == torch.bfloat16 else F32, _ptr(codes),
                                  _ptr(scales), _ptr(zeros), _ptr(H), _ptr(loss_out), _ptr(ws),
                                  ws.numel(), _stream(stream)))

    def loss_static(self, W: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                    H: torch.Tensor, group: int, loss_out: torch.Tensor, stream=None):
        """clha_loss_static: the loss of `loss` with the library's static scratch (no workspace,
        no allocation)."""
        rows, cols = W.shape
        _check_dev("W", W, (torch.float32, torch.bfloat16), (rows, cols), self.device)
        _check_dev("codes", codes, torch.uint8, (rows, cols), self.device)
        _check_dev("scales", scales, torch.float32, (rows, cols // group), self.device)
        _check_dev("zeros", zeros, torch.uint8, (rows, cols // group), self.device)
        _check_dev("H", H, torch.float32, (cols, cols), self.device)
        _check_dev("loss_out", loss_out, torch.float32, None, self.device)
        self._raise(lib.clha_loss_static(self._h, rows, cols, group, _ptr(W),
                                         BF16 if W.dtype == torch.bfloat16 else F32, _ptr(codes),
                                         _ptr(scales), _ptr(zeros), _ptr(H), _ptr(loss_out),
                                         _stream(stream)))

    def set_timing(self, enable: bool):
        self._raise(lib.clha_set_timing(self._h, 1 if enable else 0))

    def read_timing(self) -> dict:
        """{stage: (total ms, calls)} of the stages recorded since the last read."""
        n = len(STAGES)
        ms = (C.c_double * n)()
        calls = (C.c_int64 * n)()
        self._raise(lib.clha_read_timing(self._h, ms, calls, n))
        return {name: (ms[i], calls[i]) for i, name in enumerate(STAGES)}

    def sync(self, stream=None):
        self._raise(lib.clha_sync(self._h, _stream(stream)))
