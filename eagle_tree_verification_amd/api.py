"""Thin Python binding of libspecverify.so (include/spec_verify.h).

Argument marshalling only: tensors are handed to the C ABI as device
pointers together with torch's current HIP stream, and every step of the
verify path runs in the library's kernels.  Output tensors are allocated with
torch (device memory is torch's job here).  There is no fallback: if the
shared library is missing, `load()` raises.
"""
import ctypes
import os
import re

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspecverify.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "spec_verify.h")

SPEC_F32, SPEC_BF16 = 0, 1
LAUNCH = {"ordinary": 0, "cooperative": 1}  # SPEC_LAUNCH_ORDINARY, SPEC_LAUNCH_COOPERATIVE
DEVERR_TREE, DEVERR_TOKEN, DEVERR_NONFINITE, DEVERR_CAPACITY, DEVERR_SYNC = 1, 2, 4, 8, 16
DEVERR_ALIGN = 32
TIE_DTYPE = np.dtype([("b", "<i4"), ("node", "<i4"), ("kind", "<i4"), ("u", "<f4"),
                      ("margin", "<f8")])

_lib = None


class SpecError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = _lib.spec_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{fn} failed with status {status}: {msg}")


def declared_functions():
    """Names of the functions include/spec_verify.h declares."""
    with open(HEADER) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z_]+)\s*\(", text)))


def load():
    """Load the HIP library (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                           "`python -m eagle_tree_verification_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    lib.spec_verify_tree_attn.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, F, I, P, P, Z, P, P]
    lib.spec_verify_tree_attn.restype = I
    lib.spec_verify_tree_attn_workspace_size.argtypes = [I, I, I, I, I, I, I]
    lib.spec_verify_tree_attn_workspace_size.restype = Z
    lib.spec_accept_tree.argtypes = [P, P, P, P, P, I, I, I, I, F, P, P, P, P, P, P, P, P, I, P,
                                     P, Z, P, P]
    lib.spec_accept_tree.restype = I
    lib.spec_accept_tree_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, F, P, P, P, P, P, P, P,
                                             P, I, P, P, P]
    lib.spec_accept_tree_noalloc.restype = I
    lib.spec_accept_tree_workspace_size.argtypes = [I, I, I]
    lib.spec_accept_tree_workspace_size.restype = Z
    lib.spec_accept_tree_ex.argtypes = [P, P, P, P, P, I, I, I, I, F, P, P, P, P, I, P, P, P, P,
                                        P, P, P, P, I, P, P, Z, I, P, P]
    lib.spec_accept_tree_ex.restype = I
    lib.spec_accept_tree_ex_workspace_size.argtypes = [I, I, I, I, I]
    lib.spec_accept_tree_ex_workspace_size.restype = Z
    lib.spec_kv_commit.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P, P]
    lib.spec_kv_commit.restype = I
    lib.spec_kv_commit_layers.argtypes = [P, P, P, P, I, P, P, P, I, I, I, I, I, I, I, P, P]
    lib.spec_kv_commit_layers.restype = I
    lib.spec_verify_tree_attn_rope.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, F, I, P, I, P,
                                               P, Z, P, P]
    lib.spec_verify_tree_attn_rope.restype = I
    lib.spec_tree_kv_write.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, P, I, P, P]
    lib.spec_tree_kv_write.restype = I
    lib.spec_tree_state_size.argtypes = [I, I, I]
    lib.spec_tree_state_size.restype = Z
    lib.spec_tree_expand.argtypes = [P, I, P, I, I, I, I, I, P, Z, P, P, P, P]
    lib.spec_tree_expand.restype = I
    lib.spec_tree_finalize.argtypes = [P, Z, I, I, I, I, P, P, I, P, P, P, P, P, P, P, P, P, P]
    lib.spec_tree_finalize.restype = I
    lib.spec_verify_tree_attn_paged.argtypes = [P, P, P, P, I, I, I, P, P, P, I, I, I, I, I, F, I,
                                                P, I, P, P, Z, P, P]
    lib.spec_verify_tree_attn_paged.restype = I
    lib.spec_tree_kv_write_paged.argtypes = [P, P, P, P, P, I, I, I, P, P, P, I, I, I, I, I, P, I,
                                             P, P]
    lib.spec_tree_kv_write_paged.restype = I
    lib.spec_kv_commit_layers_paged.argtypes = [P, P, P, P, I, P, I, I, I, P, P, P, I, I, I, I, I,
                                                I, P, P]
    lib.spec_kv_commit_layers_paged.restype = I
    lib.spec_status_string.argtypes = [I]
    lib.spec_status_string.restype = ctypes.c_char_p
    lib.spec_abi_version.argtypes = []
    lib.spec_abi_version.restype = I
    _lib = lib
    return lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, status):
    if status != 0:
        raise SpecError(fn, status)


def _dev(t, name, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _kv_dtype(t):
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    if t.dtype == torch.float32:
        return SPEC_F32
    raise TypeError(f"unsupported KV dtype {t.dtype}")


def verify_tree_attn_workspace_size(B, n_max, Hq, Hkv, head_dim, L_cap, dtype):
    return int(load().spec_verify_tree_attn_workspace_size(B, n_max, Hq, Hkv, head_dim, L_cap, dtype))


def accept_tree_workspace_size(B, n_max, V):
    return int(load().spec_accept_tree_workspace_size(B, n_max, V))


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


ROPE_STYLES = {"half": 1, "interleaved": 2}


def verify_tree_attn(q, k_cache, v_cache, prefix_len, n_nodes, parents, *, scale=None, out=None,
                     workspace=None, dev_error=None, stream=None, inv_freq=None,
                     rope_style="half"):
    """Tree-masked attention; returns out [B][n_max][Hq][d] float32.

    With inv_freq ([d/2] float32 device tensor) the queries are rotated in
    the kernel (spec_verify_tree_attn_rope)."""
    lib = load()
    B, n_max, Hq, d = q.shape
    _, Hkv, L_cap, _ = k_cache.shape
    dt = _kv_dtype(k_cache)
    for t, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, nm, k_cache.dtype)
    for t, nm in ((prefix_len, "prefix_len"), (n_nodes, "n_nodes"), (parents, "parents")):
        _dev(t, nm, torch.int32)
    if out is None:
        out = torch.empty((B, n_max, Hq, d), dtype=torch.float32, device=q.device)
    _dev(out, "out", torch.float32)
    if scale is None:
        scale = 1.0 / float(np.sqrt(d))
    ws, wsb = _workspace(verify_tree_attn_workspace_size(B, n_max, Hq, Hkv, d, L_cap, dt),
                         q.device, workspace)
    if inv_freq is None:
        st = lib.spec_verify_tree_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(prefix_len),
                                       _ptr(n_nodes), _ptr(parents), B, n_max, Hq, Hkv, d, L_cap,
                                       float(scale), dt, _ptr(out), _ptr(ws), wsb,
                                       _ptr(dev_error), _stream(stream))
        _check("spec_verify_tree_attn", st)
        return out
    _dev(inv_freq, "inv_freq", torch.float32)
    st = lib.spec_verify_tree_attn_rope(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(prefix_len),
                                        _ptr(n_nodes), _ptr(parents), B, n_max, Hq, Hkv, d,
                                        L_cap, float(scale), dt, _ptr(inv_freq),
                                        ROPE_STYLES[rope_style], _ptr(out), _ptr(ws), wsb,
                                        _ptr(dev_error), _stream(stream))
    _check("spec_verify_tree_attn_rope", st)
    return out


def tree_kv_write(k_new, v_new, k_cache, v_cache, prefix_len, n_nodes, parents, *, inv_freq=None,
                  rope_style="half", dev_error=None, stream=None):
    """Write the tree's K (rotated when inv_freq is given) and V into the cache
    rows prefix_len + j.  k_new, v_new: [B][n_max][Hkv][d]."""
    lib = load()
    B, Hkv, L_cap, d = k_cache.shape
    n_max = k_new.shape[1]
    dt = _kv_dtype(k_cache)
    for t, nm in ((k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, nm, k_cache.dtype)
    if tuple(k_new.shape) != (B, n_max, Hkv, d) or tuple(v_new.shape) != (B, n_max, Hkv, d):
        raise ValueError("k_new, v_new must be [B][n_max][Hkv][head_dim]")
    for t, nm in ((prefix_len, "prefix_len"), (n_nodes, "n_nodes"), (parents, "parents")):
        _dev(t, nm, torch.int32)
    if inv_freq is not None:
        _dev(inv_freq, "inv_freq", torch.float32)
    st = lib.spec_tree_kv_write(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                _ptr(prefix_len), _ptr(n_nodes), _ptr(parents), B, n_max, Hkv, d,
                                L_cap, dt, _ptr(inv_freq), ROPE_STYLES[rope_style],
                                _ptr(dev_error), _stream(stream))
    _check("spec_tree_kv_write", st)


def accept_tree(tokens, parents, n_nodes, draft_p, logits, temperature, u_accept, u_sample,
                max_depth, *, final_dist=False, tie_cap=0, workspace=None, dev_error=None,
                outputs=None, stream=None, temperatures=None, d2t=None, top_k=None,
                top_p=None, noalloc=False, launch="ordinary"):
    """Acceptance walk; returns a dict of device tensors.

    Keys: accept_len [B], path [B][max_depth+1], out_tokens [B][max_depth+1],
    n_out [B], final_dist [B][V] or None, tie_log (uint8 bytes of tie_cap
    spec_tie_t records) or None, tie_count [1] or None.

    temperatures ([B] float32 device tensor) gives each sequence its own
    temperature; d2t ([Vd] int32 device tensor) means draft_p rows hold the
    draft vocabulary's Vd entries; top_k ([B] int32) and top_p ([B] float32)
    are per-sequence sampling filters on q (spec_accept_tree_ex).  noalloc
    calls spec_accept_tree_noalloc, whose exchange words live in the
    library's fixed device array instead of a workspace.  launch is
    "ordinary" or "cooperative" (spec_accept_tree_ex's launch argument; the
    cooperative launch has the runtime guarantee that a sequence's
    workgroups are resident together).
    """
    lib = load()
    B, n_max, V = logits.shape
    Vd = 0 if d2t is None else int(d2t.numel())
    if launch not in LAUNCH:
        raise ValueError(f"launch must be one of {sorted(LAUNCH)}")
    if (temperatures is not None or d2t is not None or top_k is not None or top_p is not None
            or launch != "ordinary"):
        if noalloc:
            raise ValueError("noalloc takes none of temperatures, d2t, top_k, top_p, launch")
        return _accept_tree_ex(lib, tokens, parents, n_nodes, draft_p, logits, temperature,
                               u_accept, u_sample, max_depth, final_dist, tie_cap, workspace,
                               dev_error, outputs, stream, temperatures, d2t, top_k, top_p, B,
                               n_max, V, Vd, LAUNCH[launch])
    dev = logits.device
    for t, nm in ((tokens, "tokens"), (parents, "parents"), (n_nodes, "n_nodes")):
        _dev(t, nm, torch.int32)
    for t, nm in ((draft_p, "draft_p"), (logits, "logits"), (u_accept, "u_accept"),
                  (u_sample, "u_sample")):
        _dev(t, nm, torch.float32)
    o = outputs or {}

    def _out(key, shape):
        t = o.get(key)
        return torch.empty(shape, dtype=torch.int32, device=dev) if t is None else _dev(t, key, torch.int32)

    acc = _out("accept_len", (B,))
    path = _out("path", (B, max_depth + 1))
    toks = _out("out_tokens", (B, max_depth + 1))
    nout = _out("n_out", (B,))
    fd = torch.empty((B, V), dtype=torch.float32, device=dev) if final_dist else None
    tlog = torch.zeros(max(tie_cap, 1) * TIE_DTYPE.itemsize, dtype=torch.uint8, device=dev) if tie_cap else None
    tcount = torch.zeros(1, dtype=torch.int32, device=dev) if tie_cap else None
    if noalloc:
        st = lib.spec_accept_tree_noalloc(_ptr(tokens), _ptr(parents), _ptr(n_nodes),
                                          _ptr(draft_p), _ptr(logits), B, n_max, V, int(max_depth),
                                          float(temperature), _ptr(u_accept), _ptr(u_sample),
                                          _ptr(acc), _ptr(path), _ptr(toks), _ptr(nout), _ptr(fd),
                                          _ptr(tlog), int(tie_cap), _ptr(tcount), _ptr(dev_error),
                                          _stream(stream))
        _check("spec_accept_tree_noalloc", st)
        return {"accept_len": acc, "path": path, "out_tokens": toks, "n_out": nout,
                "final_dist": fd, "tie_log": tlog, "tie_count": tcount}
    ws, wsb = _workspace(accept_tree_workspace_size(B, n_max, V), dev, workspace)
    st = lib.spec_accept_tree(_ptr(tokens), _ptr(parents), _ptr(n_nodes), _ptr(draft_p),
                              _ptr(logits), B, n_max, V, int(max_depth), float(temperature),
                              _ptr(u_accept), _ptr(u_sample), _ptr(acc), _ptr(path), _ptr(toks),
                              _ptr(nout), _ptr(fd), _ptr(tlog), int(tie_cap), _ptr(tcount),
                              _ptr(ws), wsb, _ptr(dev_error), _stream(stream))
    _check("spec_accept_tree", st)
    return {"accept_len": acc, "path": path, "out_tokens": toks, "n_out": nout,
            "final_dist": fd, "tie_log": tlog, "tie_count": tcount}


def accept_tree_ex_workspace_size(B, n_max, V, Vd, filters=False):
    return int(load().spec_accept_tree_ex_workspace_size(B, n_max, V, Vd, int(bool(filters))))


def _accept_tree_ex(lib, tokens, parents, n_nodes, draft_p, logits, temperature, u_accept,
                    u_sample, max_depth, final_dist, tie_cap, workspace, dev_error, outputs,
                    stream, temperatures, d2t, top_k, top_p, B, n_max, V, Vd, launch):
    dev = logits.device
    for t, nm in ((tokens, "tokens"), (parents, "parents"), (n_nodes, "n_nodes")):
        _dev(t, nm, torch.int32)
    for t, nm in ((draft_p, "draft_p"), (logits, "logits"), (u_accept, "u_accept"),
                  (u_sample, "u_sample")):
        _dev(t, nm, torch.float32)
    if temperatures is not None:
        _dev(temperatures, "temperatures", torch.float32)
    if d2t is not None:
        _dev(d2t, "d2t", torch.int32)
    if top_k is not None:
        _dev(top_k, "top_k", torch.int32)
    if top_p is not None:
        _dev(top_p, "top_p", torch.float32)
    if tuple(draft_p.shape) != (B, n_max, Vd if d2t is not None else V):
        raise ValueError("draft_p must be [B][n_max][Vd] with d2t, [B][n_max][V] without")
    o = outputs or {}

    def _out(key, shape):
        t = o.get(key)
        return torch.empty(shape, dtype=torch.int32, device=dev) if t is None else _dev(t, key, torch.int32)

    acc = _out("accept_len", (B,))
    path = _out("path", (B, max_depth + 1))
    toks = _out("out_tokens", (B, max_depth + 1))
    nout = _out("n_out", (B,))
    fd = torch.empty((B, V), dtype=torch.float32, device=dev) if final_dist else None
    tlog = torch.zeros(max(tie_cap, 1) * TIE_DTYPE.itemsize, dtype=torch.uint8, device=dev) if tie_cap else None
    tcount = torch.zeros(1, dtype=torch.int32, device=dev) if tie_cap else None
    filters = top_k is not None or top_p is not None
    ws, wsb = _workspace(accept_tree_ex_workspace_size(B, n_max, V, Vd, filters), dev, workspace)
    st = lib.spec_accept_tree_ex(_ptr(tokens), _ptr(parents), _ptr(n_nodes), _ptr(draft_p),
                                 _ptr(logits), B, n_max, V, int(max_depth), float(temperature),
                                 _ptr(temperatures), _ptr(top_k), _ptr(top_p), _ptr(d2t), Vd,
                                 _ptr(u_accept),
                                 _ptr(u_sample), _ptr(acc), _ptr(path), _ptr(toks), _ptr(nout),
                                 _ptr(fd), _ptr(tlog), int(tie_cap), _ptr(tcount), _ptr(ws), wsb,
                                 int(launch), _ptr(dev_error), _stream(stream))
    _check("spec_accept_tree_ex", st)
    return {"accept_len": acc, "path": path, "out_tokens": toks, "n_out": nout,
            "final_dist": fd, "tie_log": tlog, "tie_count": tcount}


def decode_ties(tie_log, tie_count):
    """Host copy of the logged near-tie records."""
    if tie_log is None:
        return np.zeros(0, dtype=TIE_DTYPE)
    cnt = int(tie_count.item())
    cap = tie_log.numel() // TIE_DTYPE.itemsize
    raw = tie_log.cpu().numpy().view(TIE_DTYPE)
    return raw[: min(cnt, cap)].copy()


def kv_commit(k_cache, v_cache, prefix_len, path, accept_len, max_depth, *, dev_error=None,
              stream=None):
    """Commit the accepted paths in place (k_cache, v_cache, prefix_len)."""
    lib = load()
    B, Hkv, L_cap, d = k_cache.shape
    dt = _kv_dtype(k_cache)
    _dev(k_cache, "k_cache")
    _dev(v_cache, "v_cache", k_cache.dtype)
    for t, nm in ((prefix_len, "prefix_len"), (path, "path"), (accept_len, "accept_len")):
        _dev(t, nm, torch.int32)
    st = lib.spec_kv_commit(_ptr(k_cache), _ptr(v_cache), _ptr(prefix_len), _ptr(path),
                            _ptr(accept_len), B, Hkv, d, L_cap, int(max_depth), dt,
                            _ptr(dev_error), _stream(stream))
    _check("spec_kv_commit", st)


def _pointer_table(tensors, name, like=None):
    """Device array of the tensors' data pointers (one small host-to-device
    copy; the tensors must outlive the stream work that reads it)."""
    tensors = list(tensors)
    if not tensors:
        raise ValueError(f"{name}: no layers")
    ref = like if like is not None else tensors[0]
    for t in tensors:
        _dev(t, name, ref.dtype)
        if t.shape != ref.shape:
            raise ValueError(f"{name}: every layer must have shape {tuple(ref.shape)}")
    ptrs = torch.tensor([t.data_ptr() for t in tensors], dtype=torch.int64)
    return ptrs.to(ref.device, non_blocking=False)


def kv_commit_layers(k_layers, v_layers, prefix_len, path, accept_len, max_depth, *,
                     k_tree=None, v_tree=None, dev_error=None, stream=None):
    """Commit the accepted paths of every layer in one call.

    k_layers, v_layers: sequences of per-layer caches [B][Hkv][L_cap][d].
    k_tree, v_tree: None (tree K/V already in the caches, committed in place)
    or sequences of per-layer scratch rows [B][Hkv][n_max][d].
    prefix_len advances once.  Returns the pointer tables, which must stay
    alive until the stream work completes.
    """
    lib = load()
    k_layers, v_layers = list(k_layers), list(v_layers)
    if len(v_layers) != len(k_layers):
        raise ValueError("k_layers and v_layers differ in length")
    B, Hkv, L_cap, d = k_layers[0].shape
    dt = _kv_dtype(k_layers[0])
    kt = _pointer_table(k_layers, "k_layers")
    vt = _pointer_table(v_layers, "v_layers", like=k_layers[0])
    n_max = 0
    tk = tv = None
    if (k_tree is None) != (v_tree is None):
        raise ValueError("give both k_tree and v_tree, or neither")
    if k_tree is not None:
        k_tree, v_tree = list(k_tree), list(v_tree)
        if len(k_tree) != len(k_layers) or len(v_tree) != len(k_layers):
            raise ValueError("one scratch buffer per layer")
        Bt, Ht, n_max, dt_ = k_tree[0].shape
        if (Bt, Ht, dt_) != (B, Hkv, d):
            raise ValueError("scratch rows must be [B][Hkv][n_max][head_dim]")
        tk = _pointer_table(k_tree, "k_tree", like=k_tree[0])
        tv = _pointer_table(v_tree, "v_tree", like=k_tree[0])
        if k_tree[0].dtype != k_layers[0].dtype:
            raise ValueError("scratch rows and caches must share a dtype")
    for t, nm in ((prefix_len, "prefix_len"), (path, "path"), (accept_len, "accept_len")):
        _dev(t, nm, torch.int32)
    st = lib.spec_kv_commit_layers(_ptr(kt), _ptr(vt), _ptr(tk), _ptr(tv), len(k_layers),
                                   _ptr(prefix_len), _ptr(path), _ptr(accept_len), B, n_max, Hkv,
                                   d, L_cap, int(max_depth), dt, _ptr(dev_error), _stream(stream))
    _check("spec_kv_commit_layers", st)
    return (kt, vt, tk, tv)


def tree_state_size(B, top_k, depth):
    return int(load().spec_tree_state_size(B, top_k, depth))


def tree_state(B, top_k, depth, device):
    """A state buffer for one tree per sequence (uninitialised device bytes)."""
    n = tree_state_size(B, top_k, depth)
    if n == 0:
        raise ValueError("tree sizes out of range")
    return torch.empty(n, dtype=torch.uint8, device=device)


def tree_expand(draft_logits, state, level, top_k, depth, *, d2t=None, expanded_tokens=None,
                expanded_ids=None, dev_error=None, stream=None):
    """Grow level `level` (1-based) of every sequence's tree.

    draft_logits: [B][R][Vd] float32 or bfloat16 (R = 1 at level 1, top_k
    after).  Returns (expanded_tokens, expanded_ids), each [B][top_k] int32.
    """
    lib = load()
    B, R, Vd = draft_logits.shape
    dt = _kv_dtype(_dev(draft_logits, "draft_logits"))
    if R != (1 if level == 1 else top_k):
        raise ValueError(f"level {level} takes {1 if level == 1 else top_k} draft rows, got {R}")
    _dev(state, "state", torch.uint8)
    if d2t is not None:
        _dev(d2t, "d2t", torch.int32)
    dev = draft_logits.device
    if expanded_tokens is None:
        expanded_tokens = torch.empty((B, top_k), dtype=torch.int32, device=dev)
    if expanded_ids is None:
        expanded_ids = torch.empty((B, top_k), dtype=torch.int32, device=dev)
    st = lib.spec_tree_expand(_ptr(draft_logits), dt, _ptr(d2t), B, Vd, int(top_k), int(depth),
                              int(level), _ptr(state), state.numel(), _ptr(expanded_tokens),
                              _ptr(expanded_ids), _ptr(dev_error), _stream(stream))
    _check("spec_tree_expand", st)
    return expanded_tokens, expanded_ids


def tree_finalize(state, B, top_k, depth, total_tokens, n_max, *, root_token=None,
                  prefix_len=None, dev_error=None, outputs=None, stream=None):
    """Rerank and emit the trees; returns a dict of device tensors (tokens,
    parents, n_nodes, depth, positions, anc_mask (int64 bit patterns),
    draft_row, value)."""
    lib = load()
    _dev(state, "state", torch.uint8)
    for t, nm in ((root_token, "root_token"), (prefix_len, "prefix_len")):
        if t is not None:
            _dev(t, nm, torch.int32)
    dev = state.device
    o = dict(outputs or {})
    shapes = {"tokens": torch.int32, "parents": torch.int32, "depth": torch.int32,
              "positions": torch.int32, "anc_mask": torch.int64, "draft_row": torch.int32,
              "value": torch.float32}
    for key, dtype in shapes.items():
        if o.get(key) is None:
            o[key] = torch.empty((B, n_max), dtype=dtype, device=dev)
        _dev(o[key], key, dtype)
    if o.get("n_nodes") is None:
        o["n_nodes"] = torch.empty((B,), dtype=torch.int32, device=dev)
    st = lib.spec_tree_finalize(_ptr(state), state.numel(), B, int(top_k), int(depth),
                                int(total_tokens), _ptr(root_token), _ptr(prefix_len), int(n_max),
                                _ptr(o["tokens"]), _ptr(o["parents"]), _ptr(o["n_nodes"]),
                                _ptr(o["depth"]), _ptr(o["positions"]), _ptr(o["anc_mask"]),
                                _ptr(o["draft_row"]), _ptr(o["value"]), _ptr(dev_error),
                                _stream(stream))
    _check("spec_tree_finalize", st)
    return o


# ----------------------------------------------------------------------------
# Paged caches: per layer a pool [num_blocks][Hkv][block_size][d] and a
# [B][max_blocks] int32 block table (logical row r of sequence b is row
# r % block_size of block block_table[b][r // block_size]).
# ----------------------------------------------------------------------------
def _paged_geometry(k_pool, block_table):
    num_blocks, Hkv, block_size, d = k_pool.shape
    _dev(block_table, "block_table", torch.int32)
    B, max_blocks = block_table.shape
    return B, num_blocks, Hkv, block_size, d, max_blocks


def verify_tree_attn_paged(q, k_pool, v_pool, block_table, prefix_len, n_nodes, parents, *,
                           scale=None, out=None, workspace=None, dev_error=None, stream=None,
                           inv_freq=None, rope_style="half"):
    """verify_tree_attn on a paged cache; returns out [B][n_max][Hq][d] float32."""
    lib = load()
    B, n_max, Hq, d = q.shape
    Bt, num_blocks, Hkv, bs, d_, max_blocks = _paged_geometry(k_pool, block_table)
    if Bt != B or d_ != d or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("pools must be [num_blocks][Hkv][block_size][d], table [B][max_blocks]")
    dt = _kv_dtype(k_pool)
    for t, nm in ((q, "q"), (k_pool, "k_pool"), (v_pool, "v_pool")):
        _dev(t, nm, k_pool.dtype)
    for t, nm in ((prefix_len, "prefix_len"), (n_nodes, "n_nodes"), (parents, "parents")):
        _dev(t, nm, torch.int32)
    if inv_freq is not None:
        _dev(inv_freq, "inv_freq", torch.float32)
    if out is None:
        out = torch.empty((B, n_max, Hq, d), dtype=torch.float32, device=q.device)
    _dev(out, "out", torch.float32)
    if scale is None:
        scale = 1.0 / float(np.sqrt(d))
    ws, wsb = _workspace(verify_tree_attn_workspace_size(B, n_max, Hq, Hkv, d, max_blocks * bs, dt),
                         q.device, workspace)
    st = lib.spec_verify_tree_attn_paged(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                         max_blocks, bs, num_blocks, _ptr(prefix_len),
                                         _ptr(n_nodes), _ptr(parents), B, n_max, Hq, Hkv, d,
                                         float(scale), dt, _ptr(inv_freq),
                                         ROPE_STYLES[rope_style], _ptr(out), _ptr(ws), wsb,
                                         _ptr(dev_error), _stream(stream))
    _check("spec_verify_tree_attn_paged", st)
    return out


def tree_kv_write_paged(k_new, v_new, k_pool, v_pool, block_table, prefix_len, n_nodes, parents,
                        *, inv_freq=None, rope_style="half", dev_error=None, stream=None):
    """tree_kv_write into a paged cache."""
    lib = load()
    B, n_max, Hkv, d = k_new.shape
    Bt, num_blocks, Hp, bs, d_, max_blocks = _paged_geometry(k_pool, block_table)
    if (Bt, Hp, d_) != (B, Hkv, d) or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("k_new [B][n_max][Hkv][d] must match the pools and table")
    dt = _kv_dtype(k_pool)
    for t, nm in ((k_new, "k_new"), (v_new, "v_new"), (k_pool, "k_pool"), (v_pool, "v_pool")):
        _dev(t, nm, k_pool.dtype)
    for t, nm in ((prefix_len, "prefix_len"), (n_nodes, "n_nodes"), (parents, "parents")):
        _dev(t, nm, torch.int32)
    if inv_freq is not None:
        _dev(inv_freq, "inv_freq", torch.float32)
    st = lib.spec_tree_kv_write_paged(_ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool),
                                      _ptr(block_table), max_blocks, bs, num_blocks,
                                      _ptr(prefix_len), _ptr(n_nodes), _ptr(parents), B, n_max,
                                      Hkv, d, dt, _ptr(inv_freq), ROPE_STYLES[rope_style],
                                      _ptr(dev_error), _stream(stream))
    _check("spec_tree_kv_write_paged", st)


def kv_commit_layers_paged(k_pools, v_pools, block_table, prefix_len, path, accept_len, max_depth,
                           *, k_tree=None, v_tree=None, dev_error=None, stream=None):
    """kv_commit_layers on per-layer pools sharing one block table.  Returns
    the pointer tables, which must stay alive until the stream work
    completes."""
    lib = load()
    k_pools, v_pools = list(k_pools), list(v_pools)
    if len(v_pools) != len(k_pools):
        raise ValueError("k_pools and v_pools differ in length")
    B, num_blocks, Hkv, bs, d, max_blocks = _paged_geometry(k_pools[0], block_table)
    dt = _kv_dtype(k_pools[0])
    kt = _pointer_table(k_pools, "k_pools")
    vt = _pointer_table(v_pools, "v_pools", like=k_pools[0])
    n_max = 0
    tk = tv = None
    if (k_tree is None) != (v_tree is None):
        raise ValueError("give both k_tree and v_tree, or neither")
    if k_tree is not None:
        k_tree, v_tree = list(k_tree), list(v_tree)
        if len(k_tree) != len(k_pools) or len(v_tree) != len(k_pools):
            raise ValueError("one scratch buffer per layer")
        Bt, Ht, n_max, dt_ = k_tree[0].shape
        if (Bt, Ht, dt_) != (B, Hkv, d):
            raise ValueError("scratch rows must be [B][Hkv][n_max][head_dim]")
        if k_tree[0].dtype != k_pools[0].dtype:
            raise ValueError("scratch rows and pools must share a dtype")
        tk = _pointer_table(k_tree, "k_tree", like=k_tree[0])
        tv = _pointer_table(v_tree, "v_tree", like=k_tree[0])
    for t, nm in ((prefix_len, "prefix_len"), (path, "path"), (accept_len, "accept_len")):
        _dev(t, nm, torch.int32)
    st = lib.spec_kv_commit_layers_paged(_ptr(kt), _ptr(vt), _ptr(tk), _ptr(tv), len(k_pools),
                                         _ptr(block_table), max_blocks, bs, num_blocks,
                                         _ptr(prefix_len), _ptr(path), _ptr(accept_len), B, n_max,
                                         Hkv, d, int(max_depth), dt, _ptr(dev_error),
                                         _stream(stream))
    _check("spec_kv_commit_layers_paged", st)
    return (kt, vt, tk, tv)
