"""ctypes binding of ``libllama_block.so`` (the C ABI of include/llama_block.h).

Argument marshalling only: torch tensors supply device pointers and shapes,
``torch.cuda.current_stream()`` supplies the stream, and workspaces are torch
allocations.  Every computation runs in the library's HIP kernels; if the
library is missing this module raises instead of computing anything itself.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# LLAMA_BLOCK_LIB selects another build of the same library (the tests use a
# host-AddressSanitizer build of it); by default the in-tree build is loaded
LIB_PATH = os.environ.get("LLAMA_BLOCK_LIB") or os.path.join(_PKG, "lib", "libllama_block.so")

F32, BF16 = 0, 1
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported", -3: "workspace too small", -4: "hip error"}

FUNCTIONS = [
    "llama_rmsnorm", "llama_rope", "llama_gqa_attention", "llama_gqa_attention_workspace_bytes",
    "llama_swiglu_ffn", "llama_swiglu_ffn_workspace_bytes", "llama_block_forward",
    "llama_block_forward_workspace_bytes", "llama_last_error", "llama_status_string",
    "llama_version", "llama_profile_enable", "llama_profile_reset", "llama_profile_collect",
    "llama_profile_query", "llama_profile_names", "llama_kv_append_fp8", "llama_gqa_attention_fp8kv",
    "llama_gqa_attention_fp8kv_workspace_bytes", "llama_block_forward_fp8kv",
    "llama_block_forward_fp8kv_workspace_bytes", "llama_kv_append_paged", "llama_gqa_attention_paged",
    "llama_gqa_attention_paged_workspace_bytes", "llama_lm_head_argmax", "llama_lm_head_argmax_workspace_bytes",
    "llama_block_forward_noalloc",
]

NOALLOC_SCRATCH_BYTES = 64 << 20  # LLAMA_NOALLOC_SCRATCH_BYTES


class LlamaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)} ({status}): {message}")
        self.status = status


class BlockWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")]


_lib = None

_vp, _i32, _i64, _f64, _sz, _int = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                    ctypes.c_double, ctypes.c_size_t, ctypes.c_int)


def lib():
    """Load the library once; raise loudly if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                           "(run python -m llama_decoder_block_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "llama_rmsnorm": ([_vp, _vp, _vp, _vp, _vp, _i64, _i32, _f64, _int, _int, _vp], _int),
        "llama_rope": ([_vp, _vp, _vp, _i64, _i32, _i32, _i32, _f64, _int, _vp], _int),
        "llama_gqa_attention": ([_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _int,
                                 _vp, _sz, _vp], _int),
        "llama_gqa_attention_workspace_bytes": ([_i32, _i32, _i32, _i32, _i32, _i32, _int], _sz),
        "llama_swiglu_ffn": ([_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _int, _int, _vp, _sz, _vp],
                             _int),
        "llama_swiglu_ffn_workspace_bytes": ([_i64, _i32, _i32, _int, _int], _sz),
        "llama_block_forward": ([_vp, _vp, ctypes.POINTER(BlockWeights), _vp, _vp, _vp, _i32, _i32, _i32,
                                 _i32, _i32, _i32, _i32, _i32, _f64, _f64, _int, _int, _vp, _sz, _vp],
                                _int),
        "llama_block_forward_workspace_bytes": ([_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _int,
                                                 _int], _sz),
        "llama_last_error": ([], ctypes.c_char_p),
        "llama_status_string": ([_int], ctypes.c_char_p),
        "llama_version": ([], _int),
        "llama_profile_enable": ([_int], _int),
        "llama_profile_reset": ([], _int),
        "llama_profile_collect": ([], _int),
        "llama_profile_query": ([ctypes.c_char_p, ctypes.POINTER(_i64), ctypes.POINTER(_f64)], _int),
        "llama_profile_names": ([ctypes.c_char_p, _sz], _int),
        "llama_kv_append_fp8": ([_vp, _vp, _vp, _i32, _i32, _i32, _i32, _int, _vp, _vp, _vp, _vp, _i32, _vp],
                                _int),
        "llama_gqa_attention_fp8kv": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp,
                                       _sz, _vp], _int),
        "llama_gqa_attention_fp8kv_workspace_bytes": ([_i32, _i32, _i32, _i32, _i32], _sz),
        "llama_block_forward_fp8kv": ([_vp, _vp, ctypes.POINTER(BlockWeights), _vp, _vp, _vp, _vp, _vp, _i32,
                                       _i32, _i32, _i32, _i32, _i32, _i32, _f64, _f64, _int, _vp, _sz, _vp],
                                      _int),
        "llama_block_forward_fp8kv_workspace_bytes": ([_i32, _i32, _i32, _i32, _i32, _i32, _i32, _int], _sz),
        "llama_kv_append_paged": ([_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _i64, _vp],
                                  _int),
        "llama_gqa_attention_paged": ([_vp, _vp, _vp, _vp, _i32, _i32, _i64, _vp, _vp, _i32, _i32, _i32, _i32, _vp,
                                       _sz, _vp], _int),
        "llama_gqa_attention_paged_workspace_bytes": ([_i32, _i32, _i32, _i32, _i32, _i32], _sz),
        "llama_lm_head_argmax": ([_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _f64, _int, _int, _vp, _sz, _vp],
                                 _int),
        "llama_lm_head_argmax_workspace_bytes": ([_i64, _i32, _i32, _int, _int], _sz),
        "llama_block_forward_noalloc": ([_vp, _vp, ctypes.POINTER(BlockWeights), _vp, _vp, _vp, _i32, _i32, _i32,
                                         _i32, _i32, _i32, _i32, _i32, _f64, _f64, _int, _int, _vp], _int),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def _check(status):
    if status != 0:
        raise LlamaError(status, lib().llama_last_error().decode())


def _dt(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t):
    """Device pointer of a dense row-major tensor (the layouts the library reads)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError(f"tensor of shape {tuple(t.shape)} is not contiguous")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        return workspace, workspace.numel() * workspace.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def rmsnorm(x, gamma, eps, residual=None, out=None, sum_out=None):
    """out = (x [+ residual]) * rsqrt(mean(.^2) + eps) * gamma, rows of width x.shape[-1]."""
    d = x.shape[-1]
    if out is None:
        out = torch.empty(x.shape, dtype=gamma.dtype, device=x.device)
    _check(lib().llama_rmsnorm(_p(x), _p(residual), _p(gamma), _p(out), _p(sum_out),
                               x.numel() // d, d, eps, _dt(gamma), _dt(x), _stream()))
    return out


def rope(q, k, positions, theta):
    """In-place RoPE; q [..., n_q, hd], k [..., n_kv, hd] (either may be None)."""
    ref = q if q is not None else k
    hd = ref.shape[-1]
    n_tok = ref.numel() // (ref.shape[-2] * hd)
    nq = q.shape[-2] if q is not None else 0
    nkv = k.shape[-2] if k is not None else 0
    _check(lib().llama_rope(_p(q), _p(k), _p(positions), n_tok, nq, nkv, hd, theta, _dt(ref), _stream()))


def gqa_attention(q, k, v, positions=None, out=None, workspace=None):
    """q [B, Tq, n_q, hd]; k, v [B, S, n_kv, hd]; positions [B, Tq] int32 or None."""
    B, Tq, nq, hd = q.shape
    S, nkv = k.shape[1], k.shape[2]
    if out is None:
        out = torch.empty_like(q)
    L = lib()
    need = L.llama_gqa_attention_workspace_bytes(B, Tq, S, nq, nkv, hd, _dt(q))
    ws, nbytes = _workspace(need, q.device, workspace)
    _check(L.llama_gqa_attention(_p(q), _p(k), _p(v), _p(out), _p(positions), B, Tq, S, nq, nkv, hd,
                                 _dt(q), _p(ws), nbytes, _stream()))
    return out


def swiglu_ffn(x, w_gate, w_up, w_down, residual=None, out=None, out_dtype=torch.float32,
               workspace=None):
    """(residual +) W_down(SiLU(W_gate x) * W_up x); x [N, d] in the weight dtype."""
    d = x.shape[-1]
    n = x.numel() // d
    dff = w_gate.shape[0]
    if out is None:
        out = torch.empty(x.shape, dtype=residual.dtype if residual is not None else out_dtype,
                          device=x.device)
    L = lib()
    need = L.llama_swiglu_ffn_workspace_bytes(n, d, dff, _dt(w_gate), _dt(out))
    ws, nbytes = _workspace(need, x.device, workspace)
    _check(L.llama_swiglu_ffn(_p(x), _p(w_gate), _p(w_up), _p(w_down), _p(residual), _p(out), n, d, dff,
                              _dt(w_gate), _dt(out), _p(ws), nbytes, _stream()))
    return out


def make_weights(w):
    """BlockWeights struct from a dict of device tensors (keeps no reference)."""
    return BlockWeights(*[_p(w[n]) for n, _ in BlockWeights._fields_])


def block_workspace_bytes(batch, seq, d, nq, nkv, hd, dff, kv_cap, wdtype, rdtype):
    return lib().llama_block_forward_workspace_bytes(batch, seq, d, nq, nkv, hd, dff, kv_cap, wdtype, rdtype)


def block_forward(x, w, positions, n_q_heads, n_kv_heads, rope_theta, eps, k_cache=None, v_cache=None,
                  y=None, workspace=None):
    """One decoder block.  x [B, T, d] (residual dtype); w dict of device tensors
    (attn_norm, wq, wk, wv, wo, ffn_norm, w_gate, w_up, w_down); positions
    [B, T] int32; optional caches [B, kv_cap, n_kv, hd] (updated in place)."""
    B, T, d = x.shape
    hd = w["wq"].shape[0] // n_q_heads
    dff = w["w_gate"].shape[0]
    kv_cap = k_cache.shape[1] if k_cache is not None else 0
    wdt, rdt = _dt(w["wq"]), _dt(x)
    if y is None:
        y = torch.empty_like(x)
    L = lib()
    need = L.llama_block_forward_workspace_bytes(B, T, d, n_q_heads, n_kv_heads, hd, dff, kv_cap, wdt, rdt)
    ws, nbytes = _workspace(need, x.device, workspace)
    wt = make_weights(w)
    _check(L.llama_block_forward(_p(x), _p(y), ctypes.byref(wt), _p(positions), _p(k_cache), _p(v_cache),
                                 kv_cap, B, T, d, n_q_heads, n_kv_heads, hd, dff, rope_theta, eps, wdt, rdt,
                                 _p(ws), nbytes, _stream()))
    return y


def block_forward_noalloc(x, w, positions, n_q_heads, n_kv_heads, rope_theta, eps, k_cache=None, v_cache=None,
                          y=None):
    """block_forward on the library's fixed device scratch (no workspace)."""
    B, T, d = x.shape
    hd = w["wq"].shape[0] // n_q_heads
    dff = w["w_gate"].shape[0]
    kv_cap = k_cache.shape[1] if k_cache is not None else 0
    if y is None:
        y = torch.empty_like(x)
    wt = make_weights(w)
    _check(lib().llama_block_forward_noalloc(_p(x), _p(y), ctypes.byref(wt), _p(positions), _p(k_cache),
                                             _p(v_cache), kv_cap, B, T, d, n_q_heads, n_kv_heads, hd, dff,
                                             rope_theta, eps, _dt(w["wq"]), _dt(x), _stream()))
    return y


# --- 8-bit KV cache -----------------------------------------------------------
def fp8_cache(batch, kv_cap, n_kv, hd, device):
    """Empty 8-bit cache: (k codes, v codes) uint8 [B, n_kv, kv_cap, hd] and
    (k scales, v scales) fp32 [B, n_kv, kv_cap]."""
    k8 = torch.zeros(batch, n_kv, kv_cap, hd, dtype=torch.uint8, device=device)
    v8 = torch.zeros_like(k8)
    ks = torch.zeros(batch, n_kv, kv_cap, dtype=torch.float32, device=device)
    vs = torch.zeros_like(ks)
    return k8, v8, ks, vs


def kv_append_fp8(k, v, positions, k8, v8, ks, vs):
    """Quantize k, v [B, T, n_kv, hd] into the 8-bit cache at slots positions [B, T]."""
    B, T, nkv, hd = k.shape
    _check(lib().llama_kv_append_fp8(_p(k), _p(v), _p(positions), B, T, nkv, hd, _dt(k), _p(k8), _p(v8),
                                     _p(ks), _p(vs), k8.shape[2], _stream()))


def gqa_attention_fp8kv(q, k8, v8, ks, vs, positions, out=None, workspace=None):
    """Decode attention: q [B, 1, n_q, hd] bf16 (or [B, n_q, hd]); 8-bit cache;
    positions [B] int32."""
    B, nq, hd = q.shape[0], q.shape[-2], q.shape[-1]
    nkv, kv_cap = k8.shape[1], k8.shape[2]
    if out is None:
        out = torch.empty_like(q)
    L = lib()
    need = L.llama_gqa_attention_fp8kv_workspace_bytes(B, kv_cap, nq, nkv, hd)
    ws, nbytes = _workspace(need, q.device, workspace)
    _check(L.llama_gqa_attention_fp8kv(_p(q), _p(k8), _p(v8), _p(ks), _p(vs), _p(out), _p(positions), B, kv_cap,
                                       nq, nkv, hd, _p(ws), nbytes, _stream()))
    return out


def block_forward_fp8kv(x, w, positions, n_q_heads, n_kv_heads, rope_theta, eps, k8, v8, ks, vs, y=None,
                        workspace=None):
    """Decode step x [B, 1, d] against the 8-bit cache (updated in place)."""
    B, T, d = x.shape
    hd = w["wq"].shape[0] // n_q_heads
    dff = w["w_gate"].shape[0]
    kv_cap = k8.shape[2]
    if y is None:
        y = torch.empty_like(x)
    L = lib()
    need = L.llama_block_forward_fp8kv_workspace_bytes(B, d, n_q_heads, n_kv_heads, hd, dff, kv_cap, _dt(x))
    ws, nbytes = _workspace(need, x.device, workspace)
    wt = make_weights(w)
    _check(L.llama_block_forward_fp8kv(_p(x), _p(y), ctypes.byref(wt), _p(positions), _p(k8), _p(v8), _p(ks),
                                       _p(vs), kv_cap, B, d, n_q_heads, n_kv_heads, hd, dff, rope_theta, eps,
                                       _dt(x), _p(ws), nbytes, _stream()))
    return y


def block_fp8kv_workspace_bytes(batch, d, nq, nkv, hd, dff, kv_cap, rdtype):
    return lib().llama_block_forward_fp8kv_workspace_bytes(batch, d, nq, nkv, hd, dff, kv_cap, rdtype)


# --- paged KV cache ------------------------------------------------------------
def kv_append_paged(k, v, positions, block_table, k_pages, v_pages):
    """Copy k, v [B, T, n_kv, hd] bf16 into the page pools [n_pages, P, n_kv, hd]
    at slots positions [B, T] through block_table [B, max_pages]."""
    B, T, nkv, hd = k.shape
    _check(lib().llama_kv_append_paged(_p(k), _p(v), _p(positions), _p(block_table), block_table.shape[1],
                                       k_pages.shape[1], B, T, nkv, hd, _p(k_pages), _p(v_pages), k_pages.shape[0],
                                       _stream()))


def gqa_attention_paged(q, k_pages, v_pages, block_table, positions, out=None, workspace=None):
    """Decode attention: q [B, 1, n_q, hd] bf16 (or [B, n_q, hd]) over the page pools."""
    B, nq, hd = q.shape[0], q.shape[-2], q.shape[-1]
    n_pages, P, nkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    max_pages = block_table.shape[1]
    if out is None:
        out = torch.empty_like(q)
    L = lib()
    need = L.llama_gqa_attention_paged_workspace_bytes(B, max_pages, P, nq, nkv, hd)
    ws, nbytes = _workspace(need, q.device, workspace)
    _check(L.llama_gqa_attention_paged(_p(q), _p(k_pages), _p(v_pages), _p(block_table), max_pages, P, n_pages,
                                       _p(out), _p(positions), B, nq, nkv, hd, _p(ws), nbytes, _stream()))
    return out


# --- output layer ---------------------------------------------------------------
def lm_head_argmax(h, gamma, w_head, eps, logits=None, best=None, workspace=None):
    """Greedy tokens of rows h [N, d] (residual dtype): RMSNorm(h; gamma), head
    w_head [vocab, d], argmax.  Returns int32 [N]; fills `logits` [N, vocab]
    fp32 and `best` [N] fp32 when given."""
    n, d = h.shape[0], h.shape[-1]
    vocab = w_head.shape[0]
    token = torch.empty(n, dtype=torch.int32, device=h.device)
    L = lib()
    need = L.llama_lm_head_argmax_workspace_bytes(n, d, vocab, _dt(w_head), _dt(h))
    ws, nbytes = _workspace(need, h.device, workspace)
    _check(L.llama_lm_head_argmax(_p(h), _p(gamma), _p(w_head), _p(token), _p(logits), _p(best), n, d, vocab, eps,
                                  _dt(w_head), _dt(h), _p(ws), nbytes, _stream()))
    return token


# --- kernel timing -----------------------------------------------------------
def profile_enable(on=True):
    _check(lib().llama_profile_enable(1 if on else 0))


def profile_reset():
    _check(lib().llama_profile_reset())


def profile_collect():
    """Wait for the recorded events; returns {kernel: (launches, total_ms)}."""
    L = lib()
    _check(L.llama_profile_collect())
    buf = ctypes.create_string_buffer(4096)
    _check(L.llama_profile_names(buf, 4096))
    out = {}
    for name in buf.value.decode().split("\n"):
        if not name:
            continue
        n = _i64()
        ms = _f64()
        _check(L.llama_profile_query(name.encode(), ctypes.byref(n), ctypes.byref(ms)))
        out[name] = (n.value, ms.value)
    return out
