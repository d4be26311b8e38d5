"""Python binding of libspb (ctypes; argument marshalling only).

Every step of the path runs in libspb: the host packer and metadata builder
(C++) and the gfx950 kernels.  torch tensors are used only as device memory
and for the current HIP stream.  The functions mirror the C ABI in
include/spb.h; errors raise ``SpbError(code, message)``.  If the library is
not built, every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "SpbError", "lib", "library_path", "fingerprint", "Plan", "pack_pass", "branch_attention",
    "score_options_noalloc", "attention_workspace_bytes", "mfma_calibration",
    "PreparedAttention", "PreparedScore", "PreparedScoreBatch", "score_batch_workspace_bytes",
    "score_options_batch",
    "score_workspace_bytes", "score_options", "score_finalize", "F32", "BF16", "FP8_E4M3",
    "HEAD_F32OUT", "HEAD_BF16", "HEAD_FP32",
    "LINEAR_BF16", "LINEAR_RESIDUAL", "LINEAR_SILU_GATE", "LINEAR_QKV_ROPE", "LINEAR_F32", "rope_table",
    "PreparedNorm", "gather_rows", "topk_lse", "topk_workspace_bytes", "decode_attention", "beam_step",
    "quantize_e4m3",
    "PreparedLinear", "rmsnorm", "linear",
    "EXPORTED_SYMBOLS",
]

F32, BF16, FP8_E4M3 = 0, 1, 2
HEAD_F32OUT, HEAD_BF16, HEAD_FP32 = 0, 1, 2  # lm-head output kinds
LINEAR_BF16, LINEAR_RESIDUAL, LINEAR_SILU_GATE, LINEAR_QKV_ROPE, LINEAR_F32 = 0, 1, 2, 3, 4  # linear epilogues
MAX_SLOT_RANGES, MAX_TOPK, MAX_BEAMS = 16, 16, 16
_HERE = os.path.dirname(os.path.abspath(__file__))
# SPB_LIBRARY names another build of the same C ABI (the host-only sanitizer
# build used by the host tests); by default the gfx950 library built in-tree.
library_path = os.environ.get("SPB_LIBRARY") or os.path.join(_HERE, "libspb.so")

EXPORTED_SYMBOLS = [
    "spb_last_error", "spb_fingerprint", "spb_pack_opts_default", "spb_pack_pass", "spb_plan_free",
    "spb_plan_num_passes", "spb_plan_info", "spb_plan_rows", "spb_plan_branches", "spb_plan_inputs",
    "spb_plan_visible",
    "spb_plan_upload", "spb_plan_meta_copy", "spb_branch_attention", "spb_score_workspace_bytes", "spb_score_options",
    "spb_score_options_noalloc", "spb_attention_workspace_bytes", "spb_mfma_calibration",
    "spb_score_batch_workspace_bytes", "spb_score_options_batch",
    "spb_score_finalize", "spb_plan_positions", "spb_rope_table", "spb_rmsnorm", "spb_linear",
    "spb_plan_slot", "spb_gather_rows", "spb_topk_workspace_bytes", "spb_topk_lse", "spb_decode_attention",
    "spb_beam_step", "spb_quantize_e4m3",
]


class SpbError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"spb error {code}: {message}")
        self.code = code


_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.POINTER(ctypes.c_float)


class _Problem(ctypes.Structure):
    _fields_ = [("n_inputs", ctypes.c_int32), ("content_len", _i32p), ("branch_off", _i32p),
                ("branch_q", _i32p), ("n_questions", ctypes.c_int32), ("q_len", _i32p),
                ("opt_off", _i32p), ("tok_off", _i32p), ("tok", _i32p), ("vocab", ctypes.c_int32),
                ("tmpl_tok", _i32p)]


class _PackOpts(ctypes.Structure):
    _fields_ = [("token_budget", ctypes.c_int32), ("floors", ctypes.c_int32),
                ("max_content_tokens", ctypes.c_int32), ("max_query_tokens", ctypes.c_int32),
                ("max_options", ctypes.c_int32), ("max_option_tokens", ctypes.c_int32),
                ("max_prompts_per_input", ctypes.c_int32), ("max_processed_tokens", ctypes.c_int64)]


class _PassInfo(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int32), ("n_segments", ctypes.c_int32), ("n_branches", ctypes.c_int32),
                ("n_options", ctypes.c_int32), ("n_scored_rows", ctypes.c_int32), ("n_targets", ctypes.c_int32),
                ("n_tiles", ctypes.c_int32), ("n_passes", ctypes.c_int32), ("unmasked_pairs", ctypes.c_int64),
                ("meta_bytes", ctypes.c_size_t), ("n_content_branches", ctypes.c_int32),
                ("n_content_options", ctypes.c_int32), ("n_logical_inputs", ctypes.c_int32)]


class _AttnArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("o", ctypes.c_void_p),
                ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32), ("hq", ctypes.c_int32),
                ("hkv", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("s_q", ctypes.c_float), ("s_k", ctypes.c_float), ("s_v", ctypes.c_float),
                ("rows", ctypes.c_int64), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class _ScoreArgs(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_void_p), ("h_dtype", ctypes.c_int32), ("hidden_dim", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("lm_head", ctypes.c_void_p), ("vocab", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("lp", _f32p), ("p", _f32p), ("residual", _f32p),
                ("gemm_event_begin", ctypes.c_void_p), ("gemm_event_end", ctypes.c_void_p),
                ("lm_head_kind", ctypes.c_int32)]


class _NormArgs(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("gain", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("dim", ctypes.c_int32), ("eps", ctypes.c_float)]


class _LinearArgs(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("w", ctypes.c_void_p), ("m", ctypes.c_int64), ("n", ctypes.c_int32),
                ("k", ctypes.c_int32), ("mode", ctypes.c_int32), ("y", ctypes.c_void_p), ("resid", ctypes.c_void_p),
                ("yf", ctypes.c_void_p),
                ("q", ctypes.c_void_p), ("k_out", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("pos", ctypes.c_void_p), ("rope_table", ctypes.c_void_p), ("n_pos", ctypes.c_int32),
                ("gemm_event_begin", ctypes.c_void_p), ("gemm_event_end", ctypes.c_void_p),
                ("fp8", ctypes.c_int32), ("scale_x", ctypes.c_float), ("scale_w", ctypes.c_float)]


class _QuantArgs(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("src_dtype", ctypes.c_int32), ("dst", ctypes.c_void_p),
                ("n", ctypes.c_int64), ("scale", ctypes.c_float)]


class _SlotInfo(ctypes.Structure):
    _fields_ = [("pass_", ctypes.c_int32), ("row", ctypes.c_int32), ("position", ctypes.c_int32),
                ("n_ranges", ctypes.c_int32), ("ranges", (ctypes.c_int32 * 2) * 16)]


class _GatherArgs(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("n_src", ctypes.c_int32), ("idx", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("dim", ctypes.c_int32), ("dst_f32", ctypes.c_void_p),
                ("dst_bf16", ctypes.c_void_p), ("pos", ctypes.c_void_p), ("pos_base", ctypes.c_void_p),
                ("per", ctypes.c_int32), ("pos_add", ctypes.c_int32)]


class _TopkArgs(ctypes.Structure):
    _fields_ = [("logits", ctypes.c_void_p), ("rows", ctypes.c_int64), ("vocab", ctypes.c_int32),
                ("k", ctypes.c_int32), ("masks", ctypes.c_void_p), ("n_masks", ctypes.c_int32),
                ("mask_of_row", ctypes.c_void_p), ("stop_of_row", ctypes.c_void_p), ("ids", ctypes.c_void_p),
                ("lp", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


class _DecodeAttnArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k_pass", ctypes.c_void_p), ("v_pass", ctypes.c_void_p),
                ("n_pass_rows", ctypes.c_int32), ("k_dec", ctypes.c_void_p), ("v_dec", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("rows", ctypes.c_int32), ("beams", ctypes.c_int32), ("hq", ctypes.c_int32),
                ("hkv", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ranges", ctypes.c_void_p),
                ("n_ranges", ctypes.c_void_p), ("path", ctypes.c_void_p), ("t_cap", ctypes.c_int32),
                ("n_path", ctypes.c_int32), ("softmax_scale", ctypes.c_float)]


class _BeamArgs(ctypes.Structure):
    _fields_ = [("n_slots", ctypes.c_int32), ("beams", ctypes.c_int32), ("k", ctypes.c_int32),
                ("t_cap", ctypes.c_int32), ("step", ctypes.c_int32), ("stop", ctypes.c_void_p),
                ("ids", ctypes.c_void_p), ("lp", ctypes.c_void_p)] + \
               [(n, ctypes.c_void_p) for n in ("tok_in", "len_in", "fin_in", "path_in", "nb_in", "score_in",
                                               "tok_out", "len_out", "fin_out", "path_out", "nb_out",
                                               "score_out", "feed")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libspb (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise SpbError(-5, f"{library_path} is not built: run `python -m shared_prefix_branch_amd.build`")
        L = ctypes.CDLL(library_path)
        L.spb_last_error.restype = ctypes.c_char_p
        L.spb_fingerprint.restype = ctypes.c_char_p
        L.spb_pack_opts_default.argtypes = [ctypes.POINTER(_PackOpts)]
        L.spb_pack_opts_default.restype = None
        L.spb_pack_pass.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(_PackOpts), ctypes.POINTER(ctypes.c_void_p)]
        L.spb_plan_free.argtypes = [ctypes.c_void_p]
        L.spb_plan_free.restype = None
        L.spb_plan_num_passes.argtypes = [ctypes.c_void_p, _i32p]
        L.spb_plan_info.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(_PassInfo)]
        L.spb_plan_rows.argtypes = [ctypes.c_void_p, ctypes.c_int32, _i64p, _i32p]
        L.spb_plan_branches.argtypes = [ctypes.c_void_p, ctypes.c_int32, _i32p, _i32p]
        L.spb_plan_inputs.argtypes = [ctypes.c_void_p, _i64p, _i32p]
        L.spb_plan_visible.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, _i32p, ctypes.c_int32, _i32p]
        L.spb_plan_upload.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.spb_plan_meta_copy.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t]
        L.spb_branch_attention.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.POINTER(_AttnArgs), ctypes.c_void_p]
        L.spb_mfma_calibration.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_void_p]
        L.spb_attention_workspace_bytes.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                    ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
        L.spb_score_workspace_bytes.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
        L.spb_score_options.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.POINTER(_ScoreArgs), ctypes.c_void_p]
        L.spb_score_options_noalloc.argtypes = L.spb_score_options.argtypes
        L.spb_score_batch_workspace_bytes.argtypes = [ctypes.c_void_p, ctypes.c_int32, _i32p, ctypes.c_int32,
                                                      ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
        L.spb_score_options_batch.argtypes = [ctypes.c_void_p, ctypes.c_int32, _i32p, ctypes.POINTER(ctypes.c_void_p),
                                              ctypes.POINTER(_ScoreArgs), ctypes.c_void_p, ctypes.c_size_t,
                                              ctypes.c_void_p]
        fpp = ctypes.POINTER(_f32p)
        L.spb_score_finalize.argtypes = [ctypes.c_void_p, fpp, fpp, fpp, _f32p, _f32p, _f32p, _f32p, _f32p]
        L.spb_plan_positions.argtypes = [ctypes.c_void_p, ctypes.c_int32, _i32p]
        L.spb_rope_table.argtypes = [_f32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_double]
        L.spb_rmsnorm.argtypes = [ctypes.POINTER(_NormArgs), ctypes.c_void_p]
        L.spb_linear.argtypes = [ctypes.POINTER(_LinearArgs), ctypes.c_void_p]
        L.spb_plan_slot.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(_SlotInfo)]
        L.spb_quantize_e4m3.argtypes = [ctypes.POINTER(_QuantArgs), ctypes.c_void_p]
        L.spb_gather_rows.argtypes = [ctypes.POINTER(_GatherArgs), ctypes.c_void_p]
        L.spb_topk_lse.argtypes = [ctypes.POINTER(_TopkArgs), ctypes.c_void_p]
        L.spb_topk_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
        L.spb_decode_attention.argtypes = [ctypes.POINTER(_DecodeAttnArgs), ctypes.c_void_p]
        L.spb_beam_step.argtypes = [ctypes.POINTER(_BeamArgs), ctypes.c_void_p]
        for name in EXPORTED_SYMBOLS:
            if name not in ("spb_last_error", "spb_fingerprint", "spb_pack_opts_default", "spb_plan_free"):
                getattr(L, name).restype = ctypes.c_int32
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise SpbError(int(status), lib().spb_last_error().decode())


def fingerprint() -> str:
    return lib().spb_fingerprint().decode()


def _ptr(a: np.ndarray, typ):
    return a.ctypes.data_as(typ)


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Plan:
    """An opaque packing plan (owned here, freed with the object)."""

    def __init__(self, handle: int, keep):
        self._h = ctypes.c_void_p(handle)
        self._keep = keep
        n = ctypes.c_int32()
        _check(lib().spb_plan_num_passes(self._h, ctypes.byref(n)))
        self.n_passes = int(n.value)

    def __del__(self):
        if getattr(self, "_h", None) is not None and self._h.value and _lib is not None:
            _lib.spb_plan_free(self._h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def info(self, pass_: int = -1) -> dict:
        s = _PassInfo()
        _check(lib().spb_plan_info(self._h, pass_, ctypes.byref(s)))
        return {f: getattr(s, f) for f, _ in _PassInfo._fields_}

    def rows(self, pass_: int):
        inf = self.info(pass_)
        lr = np.empty(inf["n_tokens"], np.int64)
        sr = np.empty(inf["n_scored_rows"], np.int32)
        _check(lib().spb_plan_rows(self._h, pass_, _ptr(lr, _i64p), _ptr(sr, _i32p)))
        return lr, sr

    def positions(self, pass_: int) -> np.ndarray:
        """Each pass row's position on its own root path (int32 [n_tokens])."""
        out = np.empty(self.info(pass_)["n_tokens"], np.int32)
        _check(lib().spb_plan_positions(self._h, pass_, _ptr(out, _i32p)))
        return out

    def slot(self, logical_branch: int) -> dict:
        """A slot question's template row and its prefix key runs in the pass."""
        s = _SlotInfo()
        _check(lib().spb_plan_slot(self._h, int(logical_branch), ctypes.byref(s)))
        return {"pass": s.pass_, "row": s.row, "position": s.position,
                "ranges": [(s.ranges[i][0], s.ranges[i][1]) for i in range(s.n_ranges)]}

    def branches(self, pass_: int):
        inf = self.info(pass_)
        lb = np.empty(inf["n_branches"], np.int32)
        of = np.empty(inf["n_branches"], np.int32)
        _check(lib().spb_plan_branches(self._h, pass_, _ptr(lb, _i32p), _ptr(of, _i32p)))
        return lb, of

    def inputs(self):
        """(row_off [n_logical_inputs + 1] int64, floor_question [n_logical_inputs] int32)."""
        n = self.info()["n_logical_inputs"]
        off = np.empty(n + 1, np.int64)
        fq = np.empty(n, np.int32)
        _check(lib().spb_plan_inputs(self._h, _ptr(off, _i64p), _ptr(fq, _i32p)))
        return off, fq

    def visible(self, pass_: int, row: int, cap: int = 1 << 16) -> List[int]:
        keys = np.empty(cap, np.int32)
        n = ctypes.c_int32()
        _check(lib().spb_plan_visible(self._h, pass_, row, _ptr(keys, _i32p), cap, ctypes.byref(n)))
        return keys[:n.value].tolist()

    def upload(self, pass_: int, d_meta, stream=None):
        _check(lib().spb_plan_upload(self._h, pass_, ctypes.c_void_p(d_meta.data_ptr()),
                                     d_meta.numel() * d_meta.element_size(), ctypes.c_void_p(_stream_handle(stream))))

    def meta_copy(self, pass_: int, host_dst):
        """Copies pass metadata into a host buffer (a CPU tensor, e.g. pinned, or a numpy array)."""
        if hasattr(host_dst, "data_ptr"):
            ptr, n = host_dst.data_ptr(), host_dst.numel() * host_dst.element_size()
        else:
            ptr, n = host_dst.ctypes.data, host_dst.nbytes
        _check(lib().spb_plan_meta_copy(self._h, pass_, ctypes.c_void_p(ptr), n))


def pack_pass(problem, token_budget: int = 16384, floors: bool = True, **limits) -> Plan:
    """Packs a logical problem (any object with the CSR fields of spb_problem)."""
    arrs = {f: np.ascontiguousarray(getattr(problem, f), dtype=np.int32)
            for f in ("content_len", "branch_off", "branch_q", "q_len", "opt_off", "tok_off", "tok")}
    P = _Problem()
    P.n_inputs = int(arrs["content_len"].shape[0])
    P.n_questions = int(arrs["q_len"].shape[0])
    for f, a in arrs.items():
        setattr(P, f, _ptr(a, _i32p))
    P.vocab = int(problem.vocab)
    tmpl = getattr(problem, "tmpl_tok", None)
    if tmpl is not None:
        arrs["tmpl_tok"] = np.ascontiguousarray(tmpl, dtype=np.int32)
        if arrs["tmpl_tok"].shape[0] != int(arrs["q_len"].sum()):
            raise SpbError(-1, "tmpl_tok must hold sum(q_len) token ids")
        P.tmpl_tok = _ptr(arrs["tmpl_tok"], _i32p)
    O = _PackOpts()
    lib().spb_pack_opts_default(ctypes.byref(O))
    O.token_budget = int(token_budget)
    O.floors = 1 if floors else 0
    for k, v in limits.items():
        setattr(O, k, int(v))
    h = ctypes.c_void_p()
    _check(lib().spb_pack_pass(ctypes.byref(P), ctypes.byref(O), ctypes.byref(h)))
    return Plan(h.value, None)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    raise SpbError(-3, f"unsupported tensor dtype {t.dtype}")


class PreparedAttention:
    """spb_branch_attention with its arguments marshalled once: calling it
    with a plan (same pass shapes) and a stream only enqueues the kernel."""

    def __init__(self, pass_: int, d_meta, q, k, v, o, softmax_scale: float = 0.0,
                 scales: Sequence[float] = (1.0, 1.0, 1.0), workspace=None):
        for t in (q, k, v, o):
            if not t.is_contiguous():
                raise SpbError(-1, "tensors must be contiguous")
        A = _AttnArgs()
        A.q, A.k, A.v, A.o = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr()
        A.in_dtype = _dtype_code(q)
        if _dtype_code(k) != A.in_dtype or _dtype_code(v) != A.in_dtype:
            raise SpbError(-3, "q, k and v must share one dtype")
        A.out_dtype = _dtype_code(o)
        A.hq, A.hkv, A.head_dim = int(q.shape[1]), int(k.shape[1]), int(q.shape[2])
        if k.shape[2] != A.head_dim or o.shape[1] != A.hq or o.shape[2] != A.head_dim or v.shape != k.shape:
            raise SpbError(-1, "q/k/v/o shapes disagree")
        A.softmax_scale = float(softmax_scale)
        A.s_q, A.s_k, A.s_v = (float(s) for s in scales)
        A.rows = int(min(q.shape[0], k.shape[0], v.shape[0], o.shape[0]))
        if workspace is not None:  # e4m3 inputs: V widened there, K/V copied asynchronously
            A.workspace = workspace.data_ptr()
            A.workspace_bytes = workspace.numel() * workspace.element_size()
        self.args = A
        self.pass_ = pass_
        self.meta = ctypes.c_void_p(d_meta.data_ptr())
        self.fn = lib().spb_branch_attention

    def __call__(self, plan: Plan, stream=None):
        _check(self.fn(plan.handle, self.pass_, self.meta, ctypes.byref(self.args),
                       ctypes.c_void_p(_stream_handle(stream))))


def branch_attention(plan: Plan, pass_: int, d_meta, q, k, v, o, softmax_scale: float = 0.0,
                     scales: Sequence[float] = (1.0, 1.0, 1.0), stream=None, workspace=None):
    """q [rows, hq, d], k/v [rows, hkv, d], o [rows, hq, d]: contiguous device tensors.
    workspace: for e4m3 inputs, a uint8 device buffer of attention_workspace_bytes (or None)."""
    PreparedAttention(pass_, d_meta, q, k, v, o, softmax_scale, scales, workspace)(plan, stream)


def mfma_calibration(out, work_groups: int, iters: int, random_operands: bool, stream=None):
    """Enqueues the MFMA calibration loop (spb_mfma_calibration); out: a float32
    device tensor of at least work_groups * 256 elements."""
    if out.numel() < work_groups * 256:
        raise SpbError(-4, "out holds fewer than work_groups * 256 floats")
    _check(lib().spb_mfma_calibration(ctypes.c_void_p(out.data_ptr()), int(work_groups), int(iters),
                                      1 if random_operands else 0, ctypes.c_void_p(_stream_handle(stream))))


def attention_workspace_bytes(plan: Plan, pass_: int, in_dtype: int, hkv: int, head_dim: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().spb_attention_workspace_bytes(plan.handle, pass_, int(in_dtype), int(hkv), int(head_dim),
                                               ctypes.byref(n)))
    return int(n.value)


def score_workspace_bytes(plan: Plan, pass_: int, vocab: int, hidden_dim: int, lm_head_kind: int = 0) -> int:
    n = ctypes.c_size_t()
    _check(lib().spb_score_workspace_bytes(plan.handle, pass_, int(vocab), int(hidden_dim), int(lm_head_kind),
                                           ctypes.byref(n)))
    return int(n.value)


class PreparedScore:
    """spb_score_options with its arguments marshalled once.  workspace=None:
    spb_score_options_noalloc, whose workspace is the library's own per-GPU
    scratch (calls on one GPU must not overlap)."""

    def __init__(self, pass_: int, d_meta, hidden, lm_head, workspace, lp, p, residual, lm_head_kind: int = 0):
        import torch
        if lm_head.dtype != torch.bfloat16:
            raise SpbError(-3, "lm_head must be bfloat16")
        for t in (lp, p, residual):
            if t.dtype != torch.float32:
                raise SpbError(-3, "outputs must be float32")
        S = _ScoreArgs()
        S.hidden = hidden.data_ptr()
        S.h_dtype = _dtype_code(hidden)
        S.hidden_dim = int(hidden.shape[1])
        S.rows = int(hidden.shape[0])
        if int(lm_head.shape[1]) != S.hidden_dim:
            raise SpbError(-1, "lm_head and hidden disagree on the hidden size")
        S.lm_head = lm_head.data_ptr()
        S.vocab = int(lm_head.shape[0])
        if workspace is not None:
            S.workspace = workspace.data_ptr()
            S.workspace_bytes = workspace.numel() * workspace.element_size()
        S.lp = ctypes.cast(ctypes.c_void_p(lp.data_ptr()), _f32p)
        S.p = ctypes.cast(ctypes.c_void_p(p.data_ptr()), _f32p)
        S.residual = ctypes.cast(ctypes.c_void_p(residual.data_ptr()), _f32p)
        S.lm_head_kind = int(lm_head_kind)
        self.args = S
        self.pass_ = pass_
        self.meta = ctypes.c_void_p(d_meta.data_ptr())
        self.fn = lib().spb_score_options if workspace is not None else lib().spb_score_options_noalloc
        self.out_sizes = (lp.numel(), p.numel(), residual.numel())
        self.meta_bytes = d_meta.numel() * d_meta.element_size()
        self._checked = None  # the plan whose pass shapes were last checked

    def check_plan(self, plan: Plan):
        """The outputs and the metadata buffer must hold the plan's pass:
        the library takes raw pointers and cannot see their sizes."""
        if self._checked is plan:
            return
        inf = plan.info(self.pass_)
        need = (inf["n_options"], inf["n_options"], inf["n_branches"])
        if any(have < n for have, n in zip(self.out_sizes, need)) or self.meta_bytes < inf["meta_bytes"]:
            raise SpbError(-4, f"pass {self.pass_}: outputs hold {self.out_sizes} and metadata "
                               f"{self.meta_bytes} bytes; the plan needs {need} and {inf['meta_bytes']}")
        self._checked = plan

    def __call__(self, plan: Plan, stream=None, gemm_events=None):
        S = self.args
        if gemm_events is not None:
            for ev in gemm_events:
                if not ev.cuda_event:
                    raise SpbError(-1, "timing events must be created (recorded once) before use")
            S.gemm_event_begin, S.gemm_event_end = gemm_events[0].cuda_event, gemm_events[1].cuda_event
        else:
            S.gemm_event_begin = S.gemm_event_end = None
        self.check_plan(plan)
        _check(self.fn(plan.handle, self.pass_, self.meta, ctypes.byref(S), ctypes.c_void_p(_stream_handle(stream))))


def score_options(plan: Plan, pass_: int, d_meta, hidden, lm_head, workspace, lp, p, residual, stream=None,
                  gemm_events=None, lm_head_kind: int = 0):
    """hidden [rows, H] (bf16/f32), lm_head [V, H] bf16, workspace uint8 device buffer,
    lp/p [n_options] and residual [n_branches] float32 device tensors.
    gemm_events: optional pair of created ``torch.cuda.Event`` recorded on the
    stream around the lm-head GEMM kernel.  lm_head_kind: HEAD_F32OUT,
    HEAD_BF16 or HEAD_FP32."""
    PreparedScore(pass_, d_meta, hidden, lm_head, workspace, lp, p, residual, lm_head_kind)(plan, stream,
                                                                                               gemm_events)


def score_options_noalloc(plan: Plan, pass_: int, d_meta, hidden, lm_head, lp, p, residual, stream=None,
                          gemm_events=None, lm_head_kind: int = 0):
    """score_options without a workspace argument: spb_score_options_noalloc
    (no device allocation; the library's per-GPU scratch; calls on one GPU
    must not overlap)."""
    PreparedScore(pass_, d_meta, hidden, lm_head, None, lp, p, residual, lm_head_kind)(plan, stream, gemm_events)


def score_batch_workspace_bytes(plan: Plan, passes: Sequence[int], vocab: int, hidden_dim: int,
                                lm_head_kind: int = 0) -> int:
    ps = np.ascontiguousarray(passes, dtype=np.int32)
    n = ctypes.c_size_t()
    _check(lib().spb_score_batch_workspace_bytes(plan.handle, len(ps), _ptr(ps, _i32p), int(vocab), int(hidden_dim),
                                                 int(lm_head_kind), ctypes.byref(n)))
    return int(n.value)


class PreparedScoreBatch:
    """spb_score_options_batch with its arguments marshalled once: passes[i]
    reads hiddens[i] and writes outs[i] = (lp, p, residual); one lm-head
    stream serves them all."""

    def __init__(self, passes: Sequence[int], d_metas, hiddens, lm_head, workspace, outs, lm_head_kind: int = 0):
        n = len(passes)
        if not (len(d_metas) == len(hiddens) == len(outs) == n):
            raise SpbError(-1, "passes, d_metas, hiddens and outs must have one entry per pass")
        self.passes = np.ascontiguousarray(passes, dtype=np.int32)
        self.metas = (ctypes.c_void_p * n)(*[m.data_ptr() for m in d_metas])
        self.args = (_ScoreArgs * n)()
        self.each = []
        for i in range(n):
            one = PreparedScore(int(passes[i]), d_metas[i], hiddens[i], lm_head, workspace, *outs[i],
                                lm_head_kind=lm_head_kind)
            self.args[i] = one.args
            self.each.append(one)
        self.workspace = ctypes.c_void_p(workspace.data_ptr())
        self.workspace_bytes = workspace.numel() * workspace.element_size()
        self.fn = lib().spb_score_options_batch

    def __call__(self, plan: Plan, stream=None, gemm_events=None):
        A = self.args[0]
        if gemm_events is not None:
            for ev in gemm_events:
                if not ev.cuda_event:
                    raise SpbError(-1, "timing events must be created (recorded once) before use")
            A.gemm_event_begin, A.gemm_event_end = gemm_events[0].cuda_event, gemm_events[1].cuda_event
        else:
            A.gemm_event_begin = A.gemm_event_end = None
        for one in self.each:
            one.check_plan(plan)
        _check(self.fn(plan.handle, len(self.passes), _ptr(self.passes, _i32p), self.metas, self.args,
                       self.workspace, self.workspace_bytes, ctypes.c_void_p(_stream_handle(stream))))


def score_options_batch(plan: Plan, passes: Sequence[int], d_metas, hiddens, lm_head, workspace, outs, stream=None,
                        gemm_events=None, lm_head_kind: int = 0):
    """One lm-head stream for several passes' scored rows (see spb_score_options_batch)."""
    PreparedScoreBatch(passes, d_metas, hiddens, lm_head, workspace, outs, lm_head_kind)(plan, stream, gemm_events)


def score_finalize(plan: Plan, lp_per_pass, p_per_pass, res_per_pass) -> dict:
    """Host floor join.  Inputs: per-pass float32 numpy arrays.  Returns numpy
    arrays lp, p, floor_p, lift [n_content_options], residual [n_content_branches]."""
    inf = plan.info(-1)
    n = plan.n_passes
    keep = []

    def table(arrs):
        t = (_f32p * n)()
        for i, a in enumerate(arrs):
            a = np.ascontiguousarray(a, dtype=np.float32)
            keep.append(a)
            t[i] = _ptr(a, _f32p)
        return t

    tl, tp, tr = table(lp_per_pass), table(p_per_pass), table(res_per_pass)
    no, nb = inf["n_content_options"], inf["n_content_branches"]
    out = {k: np.empty(no, np.float32) for k in ("lp", "p", "floor_p", "lift")}
    out["residual"] = np.empty(nb, np.float32)
    _check(lib().spb_score_finalize(plan.handle, tl, tp, tr, _ptr(out["lp"], _f32p), _ptr(out["p"], _f32p),
                                    _ptr(out["residual"], _f32p), _ptr(out["floor_p"], _f32p),
                                    _ptr(out["lift"], _f32p)))
    return out


# ---------------------------------------------------------------- decoder stack

def rope_table(n_pos: int, head_dim: int, base: float = 10000.0) -> np.ndarray:
    """(cos, sin) of p * base^(-2i/d): float32 [n_pos, head_dim // 2, 2]."""
    out = np.empty((int(n_pos), int(head_dim) // 2, 2), np.float32)
    _check(lib().spb_rope_table(_ptr(out, _f32p), int(n_pos), int(head_dim), float(base)))
    return out


def _dev(t, what: str, dtype=None):
    import torch
    if not t.is_contiguous():
        raise SpbError(-1, f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise SpbError(-3, f"{what} must be {dtype}")
    return t.data_ptr()


class PreparedNorm:
    """spb_rmsnorm with its arguments marshalled once: out = bf16(rmsnorm(x) * gain)."""

    def __init__(self, x, gain, out, eps: float = 1e-6):
        import torch
        A = _NormArgs()
        A.x = _dev(x, "x", torch.float32)
        A.gain = _dev(gain, "gain", torch.bfloat16)
        A.out = _dev(out, "out", torch.bfloat16)
        A.rows = int(x.shape[0])
        A.dim = int(x.shape[1])
        if tuple(out.shape) != tuple(x.shape) or int(gain.numel()) != A.dim:
            raise SpbError(-1, "x, gain and out disagree in shape")
        A.eps = float(eps)
        self.args = A
        self._keep = (x, gain, out)

    def __call__(self, stream=None):
        _check(lib().spb_rmsnorm(ctypes.byref(self.args), ctypes.c_void_p(_stream_handle(stream))))


class PreparedLinear:
    """spb_linear with its arguments marshalled once.  x [m, k] and w [n, k]
    bf16; mode LINEAR_BF16 / LINEAR_SILU_GATE: y; LINEAR_RESIDUAL: resid (f32
    [m, n]); LINEAR_QKV_ROPE: q, k_out, v, heads, pos (int32 [m] device),
    rope (float32 [n_pos, d/2, 2] device)."""

    def __init__(self, x, w, mode: int, y=None, resid=None, yf=None, q=None, k_out=None, v=None, hq: int = 0, hkv: int = 0,
                 head_dim: int = 0, pos=None, rope=None, fp8_scales=None):
        """fp8_scales: (s_x, s_w) with x and w e4m3 bytes (uint8), else bf16 operands."""
        import torch
        A = _LinearArgs()
        op_dt = torch.uint8 if fp8_scales is not None else torch.bfloat16
        A.x = _dev(x, "x", op_dt)
        A.w = _dev(w, "w", op_dt)
        if fp8_scales is not None:
            A.fp8, A.scale_x, A.scale_w = 1, float(fp8_scales[0]), float(fp8_scales[1])
        A.m = int(x.shape[0])
        A.n = int(w.shape[0])
        A.k = int(x.shape[1])
        if int(w.shape[1]) != A.k:
            raise SpbError(-1, "x and w disagree on k")
        A.mode = int(mode)
        keep = [x, w]
        if y is not None:
            A.y = _dev(y, "y", torch.bfloat16)
            keep.append(y)
        if resid is not None:
            A.resid = _dev(resid, "resid", torch.float32)
            keep.append(resid)
        if yf is not None:
            A.yf = _dev(yf, "yf", torch.float32)
            keep.append(yf)
        if q is not None:
            A.q, A.k_out, A.v = (_dev(t, n, torch.bfloat16) for t, n in ((q, "q"), (k_out, "k"), (v, "v")))
            A.hq, A.hkv, A.head_dim = int(hq), int(hkv), int(head_dim)
            A.pos = _dev(pos, "pos", torch.int32)
            A.rope_table = _dev(rope, "rope", torch.float32)
            A.n_pos = int(rope.shape[0])
            keep += [q, k_out, v, pos, rope]
        self.args = A
        self._keep = keep

    def __call__(self, stream=None, events=None):
        """events: optional (begin, end) torch.cuda.Event pair, already recorded
        once, recorded around the kernel."""
        A = self.args
        if events is not None:
            for ev in events:
                if not ev.cuda_event:
                    raise SpbError(-1, "timing events must be created (recorded once) before use")
            A.gemm_event_begin, A.gemm_event_end = events[0].cuda_event, events[1].cuda_event
        else:
            A.gemm_event_begin = A.gemm_event_end = None
        _check(lib().spb_linear(ctypes.byref(A), ctypes.c_void_p(_stream_handle(stream))))


def rmsnorm(x, gain, out, eps: float = 1e-6, stream=None):
    PreparedNorm(x, gain, out, eps)(stream)


def linear(x, w, mode: int, stream=None, **kw):
    PreparedLinear(x, w, mode, **kw)(stream)


# ---------------------------------------------------------------- slot decoding

def _p(t):
    return None if t is None else t.data_ptr()


class PreparedCall:
    """A decode-step call with its argument struct marshalled once."""

    def __init__(self, fn_name: str, args, keep):
        self.fn = getattr(lib(), fn_name)
        self.args = args
        self._keep = keep

    def __call__(self, stream=None):
        _check(self.fn(ctypes.byref(self.args), ctypes.c_void_p(_stream_handle(stream))))


def gather_rows(src, idx, rows: int, dst_f32=None, dst_bf16=None, pos=None, pos_base=None, per: int = 1,
                pos_add: int = 0) -> PreparedCall:
    import torch
    A = _GatherArgs()
    A.src = _dev(src, "src", torch.bfloat16)
    A.n_src = int(src.shape[0])
    A.idx = _dev(idx, "idx", torch.int32)
    A.rows = int(rows)
    A.dim = int(src.shape[1])
    A.dst_f32, A.dst_bf16, A.pos, A.pos_base = _p(dst_f32), _p(dst_bf16), _p(pos), _p(pos_base)
    A.per, A.pos_add = int(per), int(pos_add)
    return PreparedCall("spb_gather_rows", A, (src, idx, dst_f32, dst_bf16, pos, pos_base))


def topk_workspace_bytes(rows: int, vocab: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().spb_topk_workspace_bytes(int(rows), int(vocab), ctypes.byref(n)))
    return int(n.value)


def topk_lse(logits, k: int, ids, lp, lse, masks=None, mask_of_row=None, stop_of_row=None,
             workspace=None) -> PreparedCall:
    """workspace: a device uint8 tensor of topk_workspace_bytes (allocated here if None)."""
    import torch
    if workspace is None:
        workspace = torch.empty(max(16, topk_workspace_bytes(logits.shape[0], logits.shape[1])), dtype=torch.uint8,
                                device=logits.device)
    A = _TopkArgs()
    A.logits = _dev(logits, "logits", torch.float32)
    A.rows, A.vocab, A.k = int(logits.shape[0]), int(logits.shape[1]), int(k)
    A.masks = _p(masks)
    A.n_masks = 0 if masks is None else int(masks.shape[0])
    A.mask_of_row, A.stop_of_row = _p(mask_of_row), _p(stop_of_row)
    A.ids, A.lp, A.lse = _dev(ids, "ids", torch.int32), _dev(lp, "lp", torch.float32), _dev(lse, "lse", torch.float32)
    A.workspace = workspace.data_ptr()
    A.workspace_bytes = workspace.numel() * workspace.element_size()
    return PreparedCall("spb_topk_lse", A, (logits, ids, lp, lse, masks, mask_of_row, stop_of_row, workspace))


def decode_attention(q, k_pass, v_pass, k_dec, v_dec, o, beams: int, ranges, n_ranges, path, n_path: int,
                     softmax_scale: float = 0.0) -> PreparedCall:
    """q / o [rows, hq, d]; k_pass / v_pass [n_pass_rows, hkv, d]; k_dec / v_dec
    [t_cap * rows, hkv, d]; ranges [n_slots, 16, 2], n_ranges [n_slots], path
    [rows, t_cap] int32 device tensors."""
    import torch
    A = _DecodeAttnArgs()
    A.q = _dev(q, "q", torch.bfloat16)
    A.k_pass, A.v_pass = _dev(k_pass, "k_pass", torch.bfloat16), _dev(v_pass, "v_pass", torch.bfloat16)
    A.n_pass_rows = int(k_pass.shape[0])
    A.k_dec, A.v_dec = _dev(k_dec, "k_dec", torch.bfloat16), _dev(v_dec, "v_dec", torch.bfloat16)
    A.o = _dev(o, "o", torch.bfloat16)
    A.rows, A.beams = int(q.shape[0]), int(beams)
    A.hq, A.hkv, A.head_dim = int(q.shape[1]), int(k_pass.shape[1]), int(q.shape[2])
    A.ranges, A.n_ranges, A.path = (_dev(ranges, "ranges", torch.int32), _dev(n_ranges, "n_ranges", torch.int32),
                                    _dev(path, "path", torch.int32))
    A.t_cap, A.n_path = int(path.shape[1]), int(n_path)
    A.softmax_scale = float(softmax_scale)
    return PreparedCall("spb_decode_attention", A, (q, k_pass, v_pass, k_dec, v_dec, o, ranges, n_ranges, path))


def beam_step(n_slots: int, beams: int, k: int, t_cap: int, step: int, stop, ids, lp, state_in, state_out,
              feed) -> PreparedCall:
    """state_*: dict of device tensors tok [n_slots*beams, t_cap], len, fin,
    path [n_slots*beams, t_cap], nb [n_slots] (int32) and score (float32)."""
    A = _BeamArgs()
    A.n_slots, A.beams, A.k, A.t_cap, A.step = int(n_slots), int(beams), int(k), int(t_cap), int(step)
    A.stop, A.ids, A.lp, A.feed = _p(stop), _p(ids), _p(lp), _p(feed)
    for n in ("tok", "len", "fin", "path", "nb", "score"):
        setattr(A, n + "_in", _p(state_in[n]) if state_in is not None else None)
        setattr(A, n + "_out", _p(state_out[n]))
    return PreparedCall("spb_beam_step", A, (stop, ids, lp, state_in, state_out, feed))


def quantize_e4m3(src, dst, scale: float) -> PreparedCall:
    """dst (uint8, same number of elements) = e4m3(src / scale); src f32 or bf16."""
    import torch
    A = _QuantArgs()
    A.src = src.data_ptr()
    A.src_dtype = F32 if src.dtype == torch.float32 else BF16
    A.dst = _dev(dst, "dst", torch.uint8)
    A.n = int(src.numel())
    if int(dst.numel()) != A.n:
        raise SpbError(-1, "src and dst sizes differ")
    A.scale = float(scale)
    return PreparedCall("spb_quantize_e4m3", A, (src, dst))
