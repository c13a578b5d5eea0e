"""Python binding of libcad (the copy-span splice forward on MI355X).

Argument marshalling only: every entry point here forwards to the C function
of the same name in ``libcad.so`` (declared in ``include/cad.h``), passing
device pointers of caller-owned torch tensors and the current HIP stream.
No step of the computation runs in Python or PyTorch, and nothing falls back
to a CPU path: if the library is missing, importing the entry points raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcad.so")

CAD_F32, CAD_BF16 = 0, 1
CAD_COMMIT, CAD_VERIFY = 0, 1
CAD_OK, CAD_E_ARG, CAD_E_CAPACITY, CAD_E_UNSUPPORTED, CAD_E_HIP = 0, 1, 2, 3, 4
CAD_DEV_BAD_TOKEN, CAD_DEV_EMPTY_MASK, CAD_DEV_BAD_BLOCK, CAD_DEV_F16_RANGE = 1, 2, 4, 8
CAD_KV_BLOCK = 16
CAD_MAX_SEQS = 64

EXPORTS = ("cad_model_create", "cad_model_destroy", "cad_last_error", "cad_splice_forward",
           "cad_decode_step", "cad_decode_step_noalloc", "cad_propose_suffix_match",
           "cad_splice_forward_batched", "cad_splice_forward_looped", "cad_loop_step", "cad_loop_create",
           "cad_loop_destroy", "cad_loop_decode", "cad_program_create", "cad_program_destroy",
           "cad_program_decode", "cad_profile_enable", "cad_profile_read")
CAD_NOALLOC_SCRATCH_BYTES = 4 << 20

PROFILE_FAMILIES = ("embed", "rmsnorm", "gemm_qkv", "rope_append", "attention", "attn_merge", "gemm_o",
                    "gemm_gate_up", "gemm_down", "gemm_lm_head", "decide", "loop_state")
CAD_PROFILE_ALL = -1


class CadError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"cad status {status}: {msg}")
        self.status = status


class cad_config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn_dim", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("loop_depth", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("max_tokens", ctypes.c_int32)]


_VP = ctypes.c_void_p
_VPP = ctypes.POINTER(ctypes.c_void_p)


class cad_weights(ctypes.Structure):
    _fields_ = [("tok_embed", _VP), ("final_norm", _VP), ("lm_head", _VP),
                ("attn_norm", _VPP), ("w_qkv", _VPP), ("w_o", _VPP), ("ffn_norm", _VPP),
                ("w_gate_up", _VPP), ("w_down", _VPP)]


class cad_kv(ctypes.Structure):
    _fields_ = [("k", _VP), ("v", _VP), ("num_blocks", ctypes.c_int64),
                ("block_table", _VP), ("max_blocks_per_seq", ctypes.c_int32)]


class cad_loop_group(ctypes.Structure):
    _fields_ = [("pos", ctypes.c_int64), ("rows", ctypes.c_int32), ("depth", ctypes.c_int32),
                ("state", ctypes.c_int32), ("readout", ctypes.c_int32), ("table_row", ctypes.c_int32)]


class cad_loop_params(ctypes.Structure):
    _fields_ = [("screen_depth", ctypes.c_int32), ("max_copy", ctypes.c_int32), ("max_ngram", ctypes.c_int32),
                ("min_ngram", ctypes.c_int32), ("max_rows", ctypes.c_int32), ("branch_depth", ctypes.c_int32)]


class cad_loop_stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("ticks", "rows_run", "blocks", "proposed", "screened_out", "rejected",
                                              "discarded", "committed", "host_syncs", "forks", "forks_kept",
                                              "forks_lost", "fork_rows_dropped")] + \
               [("dev_status", ctypes.c_int32)]


class cad_program_table(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("lt", "lt_slash", "gt", "copy", "gen", "program", "kw", "eq_quote",
                                              "quote", "slash_gt", "hyphen")] + [("digits", ctypes.c_int32 * 10)]


class cad_program_params(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("max_doc", "max_stream", "max_ops", "max_gen", "draft_k", "chain")]


class cad_program_stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("forwards", "idle_steps", "host_syncs")] + \
               [(n, ctypes.c_int32) for n in ("decisions", "masked_steps", "forced_prefills", "copies", "copied_tokens",
                                              "drafts", "draft_tokens", "draft_accepted", "stream_n", "n_ops",
                                              "out_n", "fsm_error", "dev_status")]


PROGRAM_OP_INTS = 5  # op record: kind (0 copy, 1 gen), a, b, body start, body length

_lib = None


def lib() -> ctypes.CDLL:
    """Load libcad.so (built in-tree by ``verify_forward_amd/build.py``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python verify_forward_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        L.cad_model_create.argtypes = [ctypes.POINTER(cad_config), ctypes.POINTER(cad_weights), ctypes.POINTER(_VP)]
        L.cad_model_destroy.argtypes = [_VP]
        L.cad_model_destroy.restype = None
        L.cad_last_error.restype = ctypes.c_char_p
        L.cad_splice_forward.argtypes = [_VP, ctypes.POINTER(cad_kv), i64, _VP, i32, _VP, i32, _VP, _VP,
                                         _VP, _VP, _VP]
        L.cad_decode_step.argtypes = [_VP, ctypes.POINTER(cad_kv), i64, _VP, _VP, _VP, _VP, _VP, _VP]
        L.cad_decode_step_noalloc.argtypes = [_VP, ctypes.POINTER(cad_kv), i64, _VP, _VP, _VP, _VP, _VP, _VP]
        L.cad_propose_suffix_match.argtypes = [_VP, i64, i32, i32, i32, _VP, _VP, _VP, _VP]
        L.cad_splice_forward_batched.argtypes = [_VP, ctypes.POINTER(cad_kv), i32, _VP, _VP, _VP, _VP, i32,
                                                 _VP, _VP, _VP, _VP, _VP]
        L.cad_splice_forward_looped.argtypes = [_VP, ctypes.POINTER(cad_kv), i64, _VP, i32, i32, _VP, _VP,
                                                _VP, _VP, _VP, _VP, _VP, _VP]
        L.cad_loop_step.argtypes = [_VP, ctypes.POINTER(cad_kv), i32, ctypes.POINTER(cad_loop_group), _VP, _VP, i32,
                                    _VP, _VP, _VP, _VP, _VP, _VP]
        L.cad_loop_create.argtypes = [_VP, i64, ctypes.POINTER(cad_loop_params), ctypes.POINTER(_VP)]
        L.cad_loop_destroy.argtypes = [_VP]
        L.cad_loop_destroy.restype = None
        L.cad_loop_decode.argtypes = [_VP, ctypes.POINTER(cad_kv), _VP, i64, i32, _VP, ctypes.POINTER(cad_loop_stats),
                                      _VP]
        L.cad_program_create.argtypes = [_VP, i64, ctypes.POINTER(cad_program_table),
                                         ctypes.POINTER(cad_program_params), ctypes.POINTER(_VP)]
        L.cad_program_destroy.argtypes = [_VP]
        L.cad_program_destroy.restype = None
        L.cad_program_decode.argtypes = [_VP, ctypes.POINTER(cad_kv), _VP, i64, _VP, i32, _VP, i32, i32, _VP, i32,
                                         _VP, _VP, i32, ctypes.POINTER(cad_program_stats), _VP]
        L.cad_profile_enable.argtypes = [_VP, i32]
        L.cad_profile_read.argtypes = [_VP, ctypes.c_char_p, ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_double)]
        for name in ("cad_model_create", "cad_splice_forward", "cad_decode_step", "cad_decode_step_noalloc",
                     "cad_propose_suffix_match", "cad_splice_forward_batched", "cad_splice_forward_looped",
                     "cad_loop_step", "cad_loop_create", "cad_loop_decode", "cad_program_create",
                     "cad_program_decode", "cad_profile_enable", "cad_profile_read"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def cad_last_error() -> str:
    return lib().cad_last_error().decode()


def _check(status: int):
    if status != CAD_OK:
        raise CadError(status, cad_last_error())


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ----------------------------------------------------------------------------
# model
# ----------------------------------------------------------------------------

class Model:
    """Owns a ``cad_model*`` and keeps the weight tensors alive."""

    def __init__(self, handle, cfg: cad_config, weights, keep):
        self.handle, self.cfg, self.weights, self._keep = handle, cfg, weights, keep

    def __del__(self):
        try:
            if self.handle:
                cad_model_destroy(self)
        except Exception:
            pass


def make_config(shape, max_tokens: int) -> cad_config:
    return cad_config(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                      shape.ffn_dim, shape.vocab, getattr(shape, "loop_depth", 1), float(shape.rope_theta),
                      float(shape.rms_eps), CAD_BF16 if shape.dtype == "bf16" else CAD_F32, int(max_tokens))


def cad_model_create(shape, weights, max_tokens: int) -> Model:
    """``shape``: any object with the decoder fields; ``weights``: dict of device
    tensors as produced by ``synth.make_weights`` (nn.Linear layout)."""
    cfg = make_config(shape, max_tokens)
    layers = weights["layers"]
    arr = lambda key: (_VP * len(layers))(*[t.data_ptr() for t in (lw[key] for lw in layers)])
    arrays = {k: arr(k) for k in ("attn_norm", "w_qkv", "w_o", "ffn_norm", "w_gate_up", "w_down")}
    w = cad_weights(weights["tok_embed"].data_ptr(), weights["final_norm"].data_ptr(),
                    weights["lm_head"].data_ptr(),
                    *[ctypes.cast(arrays[k], _VPP) for k in ("attn_norm", "w_qkv", "w_o", "ffn_norm",
                                                             "w_gate_up", "w_down")])
    h = _VP()
    _check(lib().cad_model_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h)))
    return Model(h, cfg, weights, (arrays, w))


def cad_model_destroy(model: Model):
    if model.handle:
        lib().cad_model_destroy(model.handle)
        model.handle = None


# ----------------------------------------------------------------------------
# KV cache
# ----------------------------------------------------------------------------

class KVCache:
    """Caller-owned paged cache: ``k [cache_layers][num_blocks][Hkv][16][hd]``,
    ``v [cache_layers][num_blocks][Hkv][hd][16]`` and an int32 block table
    ``[n_seq][max_blocks_per_seq]``."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor, block_table: torch.Tensor):
        assert k.is_contiguous() and v.is_contiguous() and block_table.is_contiguous()
        assert block_table.dtype == torch.int32
        self.k, self.v, self.block_table = k, v, block_table
        self.num_blocks = k.shape[1]
        self.max_blocks_per_seq = block_table.shape[-1]

    @staticmethod
    def alloc(shape, num_blocks: int, block_table: torch.Tensor, device="cuda") -> "KVCache":
        cl = shape.n_layers * getattr(shape, "loop_depth", 1)
        dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
        k = torch.zeros((cl, num_blocks, shape.n_kv_heads, CAD_KV_BLOCK, shape.head_dim), dtype=dt, device=device)
        v = torch.zeros((cl, num_blocks, shape.n_kv_heads, shape.head_dim, CAD_KV_BLOCK), dtype=dt, device=device)
        return KVCache(k, v, block_table.to(device=device, dtype=torch.int32).contiguous())

    def struct(self) -> cad_kv:
        return cad_kv(self.k.data_ptr(), self.v.data_ptr(), self.num_blocks, self.block_table.data_ptr(),
                      self.max_blocks_per_seq)


# ----------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------

def cad_splice_forward(model: Model, kv: KVCache, L: int, span: torch.Tensor, mask: Optional[torch.Tensor],
                       mode: int, argmax: torch.Tensor, accepted: torch.Tensor,
                       logits: Optional[torch.Tensor] = None, dev_status: Optional[torch.Tensor] = None,
                       stream=None):
    s = kv.struct()
    _check(lib().cad_splice_forward(model.handle, ctypes.byref(s), int(L), _p(span), int(span.numel()),
                                    _p(mask), int(mode), _p(argmax), _p(accepted), _p(logits),
                                    _p(dev_status), _stream(stream)))


def cad_decode_step(model: Model, kv: KVCache, L: int, token: torch.Tensor, mask_row: Optional[torch.Tensor],
                    argmax: torch.Tensor, logits: Optional[torch.Tensor] = None,
                    dev_status: Optional[torch.Tensor] = None, stream=None):
    s = kv.struct()
    _check(lib().cad_decode_step(model.handle, ctypes.byref(s), int(L), _p(token), _p(mask_row), _p(argmax),
                                 _p(logits), _p(dev_status), _stream(stream)))


def cad_decode_step_noalloc(model: Model, kv: KVCache, L: int, token: torch.Tensor,
                            mask_row: Optional[torch.Tensor], argmax: torch.Tensor,
                            logits: Optional[torch.Tensor] = None, dev_status: Optional[torch.Tensor] = None,
                            stream=None):
    s = kv.struct()
    _check(lib().cad_decode_step_noalloc(model.handle, ctypes.byref(s), int(L), _p(token), _p(mask_row),
                                         _p(argmax), _p(logits), _p(dev_status), _stream(stream)))


def cad_propose_suffix_match(tokens: torch.Tensor, max_ngram: int, min_ngram: int, K: int,
                             out_tokens: torch.Tensor, out_len: torch.Tensor, out_pos: torch.Tensor,
                             stream=None, T: Optional[int] = None):
    n = tokens.numel() if T is None else int(T)
    _check(lib().cad_propose_suffix_match(_p(tokens) if n > 0 else None, n, int(max_ngram), int(min_ngram),
                                          int(K), _p(out_tokens), _p(out_len), _p(out_pos), _stream(stream)))


def cad_splice_forward_batched(model: Model, kv: KVCache, seq_L: Sequence[int], offsets: Sequence[int],
                               spans: torch.Tensor, mask: Optional[torch.Tensor], mode: int,
                               argmax: torch.Tensor, accepted: torch.Tensor,
                               logits: Optional[torch.Tensor] = None,
                               dev_status: Optional[torch.Tensor] = None, stream=None):
    n = len(seq_L)
    Ls = (ctypes.c_int64 * n)(*[int(x) for x in seq_L])
    offs = (ctypes.c_int32 * (n + 1))(*[int(x) for x in offsets])
    s = kv.struct()
    _check(lib().cad_splice_forward_batched(model.handle, ctypes.byref(s), n, ctypes.cast(Ls, _VP),
                                            ctypes.cast(offs, _VP), _p(spans), _p(mask), int(mode), _p(argmax),
                                            _p(accepted), _p(logits), _p(dev_status), _stream(stream)))


def cad_splice_forward_looped(model: Model, kv: KVCache, L: int, span: torch.Tensor, screen_depth: int,
                              mask: Optional[torch.Tensor], screen_argmax: torch.Tensor,
                              survivors: torch.Tensor, argmax: torch.Tensor, accepted: torch.Tensor,
                              logits: Optional[torch.Tensor] = None,
                              dev_status: Optional[torch.Tensor] = None, stream=None):
    s = kv.struct()
    _check(lib().cad_splice_forward_looped(model.handle, ctypes.byref(s), int(L), _p(span), int(span.numel()),
                                           int(screen_depth), _p(mask), _p(screen_argmax), _p(survivors),
                                           _p(argmax), _p(accepted), _p(logits), _p(dev_status),
                                           _stream(stream)))


def cad_loop_step(model: Model, kv: KVCache, groups: Sequence, tokens: torch.Tensor, state: torch.Tensor,
                  mask: Optional[torch.Tensor], argmax: Optional[torch.Tensor], accepted: Optional[torch.Tensor],
                  logits: Optional[torch.Tensor] = None, dev_status: Optional[torch.Tensor] = None, stream=None):
    """``groups``: sequence of (pos, rows, depth, state_row, readout[,
    table_row]) tuples (table_row 0 when left out); ``state``: float32
    device tensor [state_rows][d_model]."""
    arr = (cad_loop_group * len(groups))(*[cad_loop_group(int(g[0]), int(g[1]), int(g[2]), int(g[3]), int(g[4]),
                                                          int(g[5]) if len(g) > 5 else 0) for g in groups])
    s = kv.struct()
    _check(lib().cad_loop_step(model.handle, ctypes.byref(s), len(groups), arr, _p(tokens), _p(state),
                               int(state.shape[0]), _p(mask), _p(argmax), _p(accepted), _p(logits),
                               _p(dev_status), _stream(stream)))


class Loop:
    """Owns a ``cad_loop*`` (the pipeline's buffers) and keeps its model alive."""

    def __init__(self, handle, model: Model, params: cad_loop_params):
        self.handle, self.model, self.params = handle, model, params

    def __del__(self):
        try:
            if self.handle:
                cad_loop_destroy(self)
        except Exception:
            pass


def cad_loop_create(model: Model, max_len: int, screen_depth: int, max_copy: int, max_rows: int,
                    max_ngram: int = 4, min_ngram: int = 1, branch_depth: int = 0) -> Loop:
    p = cad_loop_params(int(screen_depth), int(max_copy), int(max_ngram), int(min_ngram), int(max_rows),
                        int(branch_depth))
    h = _VP()
    _check(lib().cad_loop_create(model.handle, int(max_len), ctypes.byref(p), ctypes.byref(h)))
    return Loop(h, model, p)


def cad_loop_destroy(loop: Loop):
    if loop.handle:
        lib().cad_loop_destroy(loop.handle)
        loop.handle = None


def cad_loop_decode(loop: Loop, kv: KVCache, prompt: Sequence[int], n_new: int, stream=None):
    """Returns ``(tokens, stats)``: the ``n_new`` committed tokens and the
    pipeline counters as a dict.  With branching the block table needs two
    rows (row 1 leads with the spare blocks of the second line)."""
    if loop.params.branch_depth > 0 and kv.block_table.numel() < 2 * kv.max_blocks_per_seq:
        raise CadError(CAD_E_ARG, "branching needs a block table of two rows")
    pr = (ctypes.c_int32 * len(prompt))(*[int(t) for t in prompt])
    out = (ctypes.c_int32 * int(n_new))()
    st = cad_loop_stats()
    s = kv.struct()
    _check(lib().cad_loop_decode(loop.handle, ctypes.byref(s), ctypes.cast(pr, _VP), len(prompt), int(n_new),
                                 ctypes.cast(out, _VP), ctypes.byref(st), _stream(stream)))
    return list(out), {n: int(getattr(st, n)) for n, _ in cad_loop_stats._fields_}


class Program:
    """Owns a ``cad_program*`` (the decoder's device buffers) and keeps its
    model alive."""

    def __init__(self, handle, model: Model, params: cad_program_params):
        self.handle, self.model, self.params = handle, model, params

    def __del__(self):
        try:
            if self.handle:
                cad_program_destroy(self)
        except Exception:
            pass


def cad_program_create(model: Model, max_len: int, table, max_doc: int, max_stream: int, max_ops: int,
                       max_gen: int, draft_k: int = 0, chain: int = 4) -> Program:
    """``table``: an object with the structural ids as attributes (lt,
    lt_slash, gt, copy, gen, program, kw, eq_quote, quote, slash_gt, hyphen,
    digits)."""
    t = cad_program_table(*[int(getattr(table, n)) for n, _ in cad_program_table._fields_[:-1]],
                          (ctypes.c_int32 * 10)(*[int(d) for d in table.digits]))
    p = cad_program_params(int(max_doc), int(max_stream), int(max_ops), int(max_gen), int(draft_k), int(chain))
    h = _VP()
    _check(lib().cad_program_create(model.handle, int(max_len), ctypes.byref(t), ctypes.byref(p), ctypes.byref(h)))
    return Program(h, model, p)


def cad_program_destroy(prog: Program):
    if prog.handle:
        lib().cad_program_destroy(prog.handle)
        prog.handle = None


def cad_program_decode(prog: Program, kv: KVCache, prompt: Sequence[int], doc_lines: Sequence[Sequence[int]],
                       unit: str = "lines", stream=None):
    """Decode a program after ``prompt`` over the document ``doc_lines``
    (its lines, each a list of ids).  Returns ``(stream, ops, output,
    stats)``: the program ids fed after the prompt, the ops (``{"op":
    "copy", "a", "b"}`` or ``{"op": "gen", "body"}``, the body read from the
    stream), the resolved output and the counters as a dict."""
    if unit not in ("lines", "tokens"):
        raise ValueError("unit must be 'lines' or 'tokens'")
    flat = [int(x) for line in doc_lines for x in line]
    starts = [0]
    for line in doc_lines:
        starts.append(starts[-1] + len(line))
    p = prog.params
    pr = (ctypes.c_int32 * len(prompt))(*[int(t) for t in prompt])
    doc = (ctypes.c_int32 * len(flat))(*flat)
    ls = (ctypes.c_int32 * len(starts))(*starts)
    stream_cap = int(p.max_stream) + len(flat) + 2 * int(p.draft_k) + 16
    out_cap = int(p.max_ops) * len(flat) + stream_cap
    s_out = (ctypes.c_int32 * stream_cap)()
    o_out = (ctypes.c_int32 * (int(p.max_ops) * PROGRAM_OP_INTS))()
    out = (ctypes.c_int32 * out_cap)()
    st = cad_program_stats()
    s = kv.struct()
    _check(lib().cad_program_decode(prog.handle, ctypes.byref(s), ctypes.cast(pr, _VP), len(prompt),
                                    ctypes.cast(doc, _VP), len(flat), ctypes.cast(ls, _VP), len(doc_lines),
                                    int(unit == "tokens"), ctypes.cast(s_out, _VP), stream_cap,
                                    ctypes.cast(o_out, _VP), ctypes.cast(out, _VP), out_cap, ctypes.byref(st),
                                    _stream(stream)))
    stats = {n: int(getattr(st, n)) for n, _ in cad_program_stats._fields_}
    toks = list(s_out[:stats["stream_n"]])
    ops = []
    for i in range(stats["n_ops"]):
        kind, a, b, start, n = o_out[i * PROGRAM_OP_INTS:(i + 1) * PROGRAM_OP_INTS]
        ops.append({"op": "copy", "a": a, "b": b} if kind == 0 else {"op": "gen", "body": toks[start:start + n]})
    return toks, ops, list(out[:stats["out_n"]]), stats


def cad_profile_enable(model: Model, families=CAD_PROFILE_ALL):
    """Record launch events for ``families``: an iterable of family names,
    ``CAD_PROFILE_ALL`` (every family) or a false value (stop recording)."""
    if families is True or families == CAD_PROFILE_ALL:
        mask = CAD_PROFILE_ALL
    elif not families:
        mask = 0
    else:
        mask = 0
        for f in families:
            mask |= 1 << PROFILE_FAMILIES.index(f)
    _check(lib().cad_profile_enable(model.handle, mask))


def cad_profile_read(model: Model, family: str):
    """Return ``(launches, total_ms)`` recorded for a kernel family."""
    n = ctypes.c_int64()
    ms = ctypes.c_double()
    _check(lib().cad_profile_read(model.handle, family.encode(), ctypes.byref(n), ctypes.byref(ms)))
    return int(n.value), float(ms.value)
