"""Thin torch binding of libmoe: one function per C entry point, same names.

Argument marshalling only: tensors are checked for device, dtype and shape,
made contiguous, outputs are allocated with torch (device memory), and the
current torch stream is passed down.  Every step of the computation runs in
the HIP kernels of libmoe.so.

Index arrays that the C ABI types as uint32 are int32 tensors here (same
bits; every value stays below 2**31 at the sizes torch can allocate).
"""

import torch

from . import _lib
from ._lib import MOE_BF16, MOE_F16, MOE_F32, check, lib

_DT = {torch.float32: MOE_F32, torch.float16: MOE_F16,
       torch.bfloat16: MOE_BF16}
_U32 = torch.int32


def _dt(t, what):
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError("%s: dtype %s is not F32, F16 or BF16" % (what, t.dtype))


def _dev(*ts):
    dev = ts[0].device
    if dev.type != "cuda":
        raise ValueError("libmoe tensors must be on a HIP device, got %s" % dev)
    for t in ts[1:]:
        if t.device != dev:
            raise ValueError("all tensors must be on one device")
    return dev


def _c(t):
    return t if t.is_contiguous() else t.contiguous()


def _p(t):
    return t.data_ptr() if t is not None else None


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def _out(t, shape, dtype, dev, what):
    """A caller's output tensor must be exactly what the kernels write:
    the library only sees a pointer, so a short or strided one would be
    written out of bounds.  None allocates one."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    if (tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != dev
            or not t.is_contiguous()):
        raise ValueError("%s must be a contiguous %s tensor of shape %s on %s"
                         % (what, dtype, tuple(shape), dev))
    return t


def _index(t, shape, what):
    """Index arrays are uint32 in the C ABI: int32 tensors here."""
    if t.dtype != _U32 or tuple(t.shape) != tuple(shape):
        raise ValueError("%s must be an int32 tensor of shape %s"
                         % (what, tuple(shape)))
    return t


def _workspace(ws, need, dev):
    """(tensor, bytes) of a scratch buffer of at least `need` bytes."""
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if ws.device != dev or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on %s" % dev)
    return ws, ws.numel() * ws.element_size()


def _experts_weights(w_gate, w_up, w_down, H, dtype):
    E, I, H2 = w_gate.shape
    if H2 != H or tuple(w_up.shape) != (E, I, H) or tuple(
            w_down.shape) != (E, H, I):
        raise ValueError("expert weight shapes must be gate/up [E,I,H], "
                         "down [E,H,I] with H matching the rows")
    for w in (w_gate, w_up, w_down):
        if w.dtype != dtype:
            raise TypeError("expert weights and rows must share one dtype")
    return E, I


def moe_route(logits, top_k, renormalize=True, idx=None, weights=None):
    """Softmax/top-k routing.  logits [T,E] -> (idx int32 [T,k],
    weights [T,k] in the logits dtype)."""
    logits = _c(logits)
    dev = _dev(logits)
    T, E = logits.shape
    idx = _out(idx, (T, top_k), _U32, dev, "idx")
    weights = _out(weights, (T, top_k), logits.dtype, dev, "weights")
    check(lib().moe_route(_p(logits), _dt(logits, "logits"), T, E, top_k,
                          int(bool(renormalize)), _p(idx), _p(weights),
                          _stream(dev)))
    return idx, weights


def moe_dispatch_workspace_size(T, E, top_k):
    return lib().moe_dispatch_workspace_size(T, E, top_k)


def moe_dispatch(x, idx, num_experts, workspace=None):
    """Compact dispatch.  x [T,H], idx [T,k] -> dict of xd [N,H],
    offsets [E+1], row_expert [N], row_token [N], token_row [T,k]."""
    x = _c(x)
    idx = _c(idx)
    dev = _dev(x, idx)
    T, H = x.shape
    k = idx.shape[1]
    _index(idx, (T, k), "idx")
    N = T * k
    workspace, ws_bytes = _workspace(
        workspace, moe_dispatch_workspace_size(T, num_experts, k), dev)
    out = dict(
        xd=torch.empty((N, H), dtype=x.dtype, device=dev),
        offsets=torch.empty(num_experts + 1, dtype=_U32, device=dev),
        row_expert=torch.empty(N, dtype=_U32, device=dev),
        row_token=torch.empty(N, dtype=_U32, device=dev),
        token_row=torch.empty((T, k), dtype=_U32, device=dev),
    )
    check(lib().moe_dispatch(
        _p(x), _dt(x, "x"), T, H, num_experts, k, _p(idx), _p(out["xd"]),
        _p(out["offsets"]), _p(out["row_expert"]), _p(out["row_token"]),
        _p(out["token_row"]), _p(workspace), ws_bytes, _stream(dev)))
    return out


def moe_dispatch_noalloc(x, idx, num_experts, out=None):
    """moe_dispatch without a workspace (the library's static count table).
    ``out``: optional dict of caller-allocated outputs with the keys of
    moe_dispatch's result (then this call allocates nothing); missing ones
    are allocated here."""
    x = _c(x)
    idx = _c(idx)
    dev = _dev(x, idx)
    T, H = x.shape
    k = idx.shape[1]
    _index(idx, (T, k), "idx")
    N = T * k
    out = dict(out or {})
    shapes = dict(xd=((N, H), x.dtype), offsets=((num_experts + 1,), _U32),
                  row_expert=((N,), _U32), row_token=((N,), _U32),
                  token_row=((T, k), _U32))
    for key, (shape, dtype) in shapes.items():
        out[key] = _out(out.get(key), shape, dtype, dev, key)
    check(lib().moe_dispatch_noalloc(
        _p(x), _dt(x, "x"), T, H, num_experts, k, _p(idx), _p(out["xd"]),
        _p(out["offsets"]), _p(out["row_expert"]), _p(out["row_token"]),
        _p(out["token_row"]), _stream(dev)))
    return out


def moe_experts_forward(xd, offsets, w_gate, w_up, w_down, act=None, y=None):
    """SwiGLU experts over segments.  Returns y [N,H] (act [N,I] is the
    intermediate buffer; pass one in to keep it)."""
    xd, offsets = _c(xd), _c(offsets)
    w_gate, w_up, w_down = _c(w_gate), _c(w_up), _c(w_down)
    dev = _dev(xd, offsets, w_gate, w_up, w_down)
    N, H = xd.shape
    E, I = _experts_weights(w_gate, w_up, w_down, H, xd.dtype)
    _index(offsets, (E + 1,), "offsets")
    act = _out(act, (N, I), xd.dtype, dev, "act")
    y = _out(y, (N, H), xd.dtype, dev, "y")
    check(lib().moe_experts_forward(
        _p(xd), _dt(xd, "xd"), N, H, I, E, _p(w_gate), _p(w_up), _p(w_down),
        _p(offsets), _p(act), _p(y), _stream(dev)))
    return y


def moe_experts_forward_clipped(xd, offsets, w_gate, w_up, w_down,
                                alpha=1.702, limit=7.0, act=None, y=None):
    """moe_experts_forward with the clipped SwiGLU activation (gate clamped
    from above at ``limit``, up to [-limit, limit], swish with parameter
    ``alpha``).  Returns y [N,H]."""
    xd, offsets = _c(xd), _c(offsets)
    w_gate, w_up, w_down = _c(w_gate), _c(w_up), _c(w_down)
    dev = _dev(xd, offsets, w_gate, w_up, w_down)
    N, H = xd.shape
    E, I = _experts_weights(w_gate, w_up, w_down, H, xd.dtype)
    _index(offsets, (E + 1,), "offsets")
    act = _out(act, (N, I), xd.dtype, dev, "act")
    y = _out(y, (N, H), xd.dtype, dev, "y")
    check(lib().moe_experts_forward_clipped(
        _p(xd), _dt(xd, "xd"), N, H, I, E, _p(w_gate), _p(w_up), _p(w_down),
        _p(offsets), float(alpha), float(limit), _p(act), _p(y),
        _stream(dev)))
    return y


def moe_combine(y, weights, token_row, out=None):
    """Weighted merge.  y [N,H], weights [T,k], token_row [T,k] ->
    out [T,H]."""
    y, weights, token_row = _c(y), _c(weights), _c(token_row)
    dev = _dev(y, weights, token_row)
    N, H = y.shape
    T, k = weights.shape
    _index(token_row, (T, k), "token_row")
    out = _out(out, (T, H), y.dtype, dev, "out")
    check(lib().moe_combine(_p(y), _dt(y, "y"), N, T, H, k, _p(weights),
                            _dt(weights, "weights"), _p(token_row), _p(out),
                            _stream(dev)))
    return out


def moe_forward_workspace_size(T, H, I, E, top_k, dtype, logits_dtype=None):
    ldt = _DT[logits_dtype if logits_dtype is not None else dtype]
    return lib().moe_forward_workspace_size(T, H, I, E, top_k, _DT[dtype], ldt)


def moe_forward(x, logits, w_gate, w_up, w_down, top_k, renormalize=True,
                out=None, workspace=None):
    """Whole forward: route -> dispatch -> experts -> combine, one call."""
    x, logits = _c(x), _c(logits)
    w_gate, w_up, w_down = _c(w_gate), _c(w_up), _c(w_down)
    dev = _dev(x, logits, w_gate, w_up, w_down)
    T, H = x.shape
    E, I = _experts_weights(w_gate, w_up, w_down, H, x.dtype)
    if logits.shape != (T, E):
        raise ValueError("logits must be [T, E]")
    workspace, ws_bytes = _workspace(
        workspace,
        moe_forward_workspace_size(T, H, I, E, top_k, x.dtype, logits.dtype),
        dev)
    out = _out(out, (T, H), x.dtype, dev, "out")
    check(lib().moe_forward(
        _p(x), _dt(x, "x"), _p(logits), _dt(logits, "logits"), T, H, I, E,
        top_k, int(bool(renormalize)), _p(w_gate), _p(w_up), _p(w_down),
        _p(out), _p(workspace), ws_bytes, _stream(dev)))
    return out


def moe_forward_clipped(x, logits, w_gate, w_up, w_down, top_k,
                        renormalize=True, alpha=1.702, limit=7.0, out=None,
                        workspace=None):
    """moe_forward with the clipped SwiGLU activation, one call."""
    x, logits = _c(x), _c(logits)
    w_gate, w_up, w_down = _c(w_gate), _c(w_up), _c(w_down)
    dev = _dev(x, logits, w_gate, w_up, w_down)
    T, H = x.shape
    E, I = _experts_weights(w_gate, w_up, w_down, H, x.dtype)
    if logits.shape != (T, E):
        raise ValueError("logits must be [T, E]")
    workspace, ws_bytes = _workspace(
        workspace,
        moe_forward_workspace_size(T, H, I, E, top_k, x.dtype, logits.dtype),
        dev)
    out = _out(out, (T, H), x.dtype, dev, "out")
    check(lib().moe_forward_clipped(
        _p(x), _dt(x, "x"), _p(logits), _dt(logits, "logits"), T, H, I, E,
        top_k, int(bool(renormalize)), float(alpha), float(limit),
        _p(w_gate), _p(w_up), _p(w_down), _p(out), _p(workspace), ws_bytes,
        _stream(dev)))
    return out


def _bias(bias, E, dev):
    """The optional FP32 correction bias [E] (None: no correction)."""
    if bias is None:
        return None
    bias = _c(bias)
    if (bias.dtype != torch.float32 or tuple(bias.shape) != (E,)
            or bias.device != dev):
        raise ValueError("bias must be a float32 tensor of shape (%d,) on %s"
                         % (E, dev))
    return bias


def moe_route_sigmoid_grouped(logits, top_k, groups, selected_groups,
                              bias=None, group_top_two=False,
                              renormalize=True, scale=1.0, idx=None,
                              weights=None):
    """Group-limited sigmoid routing.  logits [T,E], bias None or float32
    [E] -> (idx int32 [T,k], weights [T,k] in the logits dtype)."""
    logits = _c(logits)
    dev = _dev(logits)
    T, E = logits.shape
    bias = _bias(bias, E, dev)
    idx = _out(idx, (T, top_k), _U32, dev, "idx")
    weights = _out(weights, (T, top_k), logits.dtype, dev, "weights")
    check(lib().moe_route_sigmoid_grouped(
        _p(logits), _dt(logits, "logits"), T, E, _p(bias), top_k, groups,
        selected_groups, int(bool(group_top_two)), int(bool(renormalize)),
        float(scale), _p(idx), _p(weights), _stream(dev)))
    return idx, weights


def moe_forward_sigmoid_grouped(x, logits, w_gate, w_up, w_down, top_k,
                                groups, selected_groups, bias=None,
                                group_top_two=False, renormalize=True,
                                scale=1.0, out=None, workspace=None):
    """Whole forward with group-limited sigmoid routing, one call."""
    x, logits = _c(x), _c(logits)
    w_gate, w_up, w_down = _c(w_gate), _c(w_up), _c(w_down)
    dev = _dev(x, logits, w_gate, w_up, w_down)
    T, H = x.shape
    E, I = _experts_weights(w_gate, w_up, w_down, H, x.dtype)
    if logits.shape != (T, E):
        raise ValueError("logits must be [T, E]")
    bias = _bias(bias, E, dev)
    workspace, ws_bytes = _workspace(
        workspace,
        moe_forward_workspace_size(T, H, I, E, top_k, x.dtype, logits.dtype),
        dev)
    out = _out(out, (T, H), x.dtype, dev, "out")
    check(lib().moe_forward_sigmoid_grouped(
        _p(x), _dt(x, "x"), _p(logits), _dt(logits, "logits"), _p(bias), T,
        H, I, E, top_k, groups, selected_groups, int(bool(group_top_two)),
        int(bool(renormalize)), float(scale), _p(w_gate), _p(w_up),
        _p(w_down), _p(out), _p(workspace), ws_bytes, _stream(dev)))
    return out


_INDEX_TYPES = {"u32": (_lib.MOE_IDX_U32, 4), "i32": (_lib.MOE_IDX_I32, 4),
                "i64": (_lib.MOE_IDX_I64, 8)}
_SCORING = {"softmax": _lib.MOE_SCORE_SOFTMAX,
            "sigmoid": _lib.MOE_SCORE_SIGMOID}


def _router_indices(indices, T, index_type):
    """indices [T,k] of int32 (read as "i32", or "u32" for the uint32 bits
    moe_route writes), int64 ("i64") or uint32 ("u32")."""
    if index_type is None:
        index_type = {torch.int32: "i32", torch.int64: "i64",
                      torch.uint32: "u32"}.get(indices.dtype)
        if index_type is None:
            raise TypeError("indices must be int32, int64 or uint32")
    code, size = _INDEX_TYPES[index_type]
    if indices.dim() != 2 or indices.shape[0] != T:
        raise ValueError("indices must be [T, top_k]")
    if indices.element_size() != size or indices.is_floating_point():
        raise TypeError("indices of type %s need %d-byte integer elements"
                        % (index_type, size))
    return code


def moe_selected_router_weights(logits, indices, scoring="softmax",
                                renormalize=False, scale=1.0,
                                index_type=None, out=None):
    """FP32 router weights [T,k] of the experts ``indices`` [T,k] selects
    (softmax or sigmoid scores, optional renormalisation, scale)."""
    logits, indices = _c(logits), _c(indices)
    dev = _dev(logits, indices)
    T, E = logits.shape
    it = _router_indices(indices, T, index_type)
    k = indices.shape[1]
    out = _out(out, (T, k), torch.float32, dev, "weights")
    check(lib().moe_selected_router_weights(
        _p(logits), _dt(logits, "logits"), T, E, _p(indices), it, k,
        _SCORING[scoring], int(bool(renormalize)), float(scale), _p(out),
        _stream(dev)))
    return out


def moe_selected_router_backward(logits, indices, grad_weights,
                                 scoring="softmax", renormalize=False,
                                 scale=1.0, index_type=None, out=None):
    """The logits gradient [T,E] (logits dtype) of
    moe_selected_router_weights for FP32 ``grad_weights`` [T,k]."""
    logits, indices = _c(logits), _c(indices)
    grad_weights = _c(grad_weights)
    dev = _dev(logits, indices, grad_weights)
    T, E = logits.shape
    it = _router_indices(indices, T, index_type)
    k = indices.shape[1]
    if grad_weights.dtype != torch.float32 or grad_weights.shape != (T, k):
        raise ValueError("grad_weights must be a float32 [T, top_k] tensor")
    out = _out(out, (T, E), logits.dtype, dev, "grad_logits")
    check(lib().moe_selected_router_backward(
        _p(logits), _dt(logits, "logits"), T, E, _p(indices), it, k,
        _p(grad_weights), _SCORING[scoring], int(bool(renormalize)),
        float(scale), _p(out), _stream(dev)))
    return out


def moe_experts_forward_training(xd, offsets, w_gate, w_up, w_down):
    """Training forward over segments: returns dict gate, up, act [N,I]
    (the cache the expert backward needs) and y [N,H]."""
    xd, offsets = _c(xd), _c(offsets)
    w_gate, w_up, w_down = _c(w_gate), _c(w_up), _c(w_down)
    dev = _dev(xd, offsets, w_gate, w_up, w_down)
    N, H = xd.shape
    E, I = _experts_weights(w_gate, w_up, w_down, H, xd.dtype)
    _index(offsets, (E + 1,), "offsets")
    out = {name: torch.empty((N, I), dtype=xd.dtype, device=dev)
           for name in ("gate", "up", "act")}
    out["y"] = torch.empty((N, H), dtype=xd.dtype, device=dev)
    check(lib().moe_experts_forward_training(
        _p(xd), _dt(xd, "xd"), N, H, I, E, _p(w_gate), _p(w_up), _p(w_down),
        _p(offsets), _p(out["gate"]), _p(out["up"]), _p(out["act"]),
        _p(out["y"]), _stream(dev)))
    return out


def moe_combine_backward(y, weights, token_row, grad_out):
    """Gradients of moe_combine: (grad_expert [N,H] in y's dtype,
    grad_weights [T,k] float32).  Rows no slot maps stay zero."""
    y, weights = _c(y), _c(weights)
    token_row, grad_out = _c(token_row), _c(grad_out)
    dev = _dev(y, weights, token_row, grad_out)
    N, H = y.shape
    T, k = weights.shape
    _index(token_row, (T, k), "token_row")
    if grad_out.shape != (T, H) or grad_out.dtype != y.dtype:
        raise ValueError("grad_out must be [T, H] in y's dtype")
    grad_expert = torch.zeros((N, H), dtype=y.dtype, device=dev)
    grad_weights = torch.empty((T, k), dtype=torch.float32, device=dev)
    check(lib().moe_combine_backward(
        _p(y), _dt(y, "y"), N, T, H, k, _p(weights), _dt(weights, "weights"),
        _p(token_row), _p(grad_out), _p(grad_expert), _p(grad_weights),
        _stream(dev)))
    return grad_expert, grad_weights


def moe_experts_backward_workspace_size(N, H, I, E, dtype):
    return lib().moe_experts_backward_workspace_size(N, H, I, E, _DT[dtype])


def moe_experts_backward(xd, offsets, w_gate, w_up, w_down, cache, grad_y,
                         workspace=None):
    """Expert backward from the training cache (a dict with gate, up, act as
    moe_experts_forward_training returns).  Returns dict grad_xd [N,H] and
    float32 grad_w_gate, grad_w_up [E,I,H], grad_w_down [E,H,I]."""
    xd, offsets, grad_y = _c(xd), _c(offsets), _c(grad_y)
    w_gate, w_up, w_down = _c(w_gate), _c(w_up), _c(w_down)
    gate, up, act = _c(cache["gate"]), _c(cache["up"]), _c(cache["act"])
    dev = _dev(xd, offsets, w_gate, w_up, w_down, gate, up, act, grad_y)
    N, H = xd.shape
    E, I = _experts_weights(w_gate, w_up, w_down, H, xd.dtype)
    _index(offsets, (E + 1,), "offsets")
    for name, t in (("gate", gate), ("up", up), ("act", act)):
        if t.shape != (N, I) or t.dtype != xd.dtype:
            raise ValueError("cache %s must be [N, I] in xd's dtype" % name)
    if grad_y.shape != (N, H) or grad_y.dtype != xd.dtype:
        raise ValueError("grad_y must be [N, H] in xd's dtype")
    workspace, ws_bytes = _workspace(
        workspace, moe_experts_backward_workspace_size(N, H, I, E, xd.dtype),
        dev)
    out = dict(grad_xd=torch.empty((N, H), dtype=xd.dtype, device=dev),
               grad_w_gate=torch.empty((E, I, H), dtype=torch.float32,
                                       device=dev),
               grad_w_up=torch.empty((E, I, H), dtype=torch.float32,
                                     device=dev),
               grad_w_down=torch.empty((E, H, I), dtype=torch.float32,
                                       device=dev))
    check(lib().moe_experts_backward(
        _p(xd), _dt(xd, "xd"), N, H, I, E, _p(w_gate), _p(w_up), _p(w_down),
        _p(offsets), _p(gate), _p(up), _p(act), _p(grad_y),
        _p(out["grad_xd"]), _p(out["grad_w_gate"]), _p(out["grad_w_up"]),
        _p(out["grad_w_down"]), _p(workspace), ws_bytes, _stream(dev)))
    return out


def moe_dispatch_backward(grad_xd, token_row, out=None):
    """grad_x [T,H]: each token's selected rows of grad_xd [N,H] summed."""
    grad_xd, token_row = _c(grad_xd), _c(token_row)
    dev = _dev(grad_xd, token_row)
    N, H = grad_xd.shape
    T, k = token_row.shape
    _index(token_row, (T, k), "token_row")
    out = _out(out, (T, H), grad_xd.dtype, dev, "grad_x")
    check(lib().moe_dispatch_backward(
        _p(grad_xd), _dt(grad_xd, "grad_xd"), N, T, H, k, _p(token_row),
        _p(out), _stream(dev)))
    return out


__all__ = ["moe_route", "moe_dispatch", "moe_dispatch_workspace_size",
           "moe_experts_forward", "moe_combine", "moe_forward",
           "moe_forward_workspace_size", "moe_route_sigmoid_grouped",
           "moe_forward_sigmoid_grouped", "moe_selected_router_weights",
           "moe_selected_router_backward", "moe_experts_forward_training",
           "moe_combine_backward", "moe_experts_backward_workspace_size",
           "moe_experts_backward", "moe_dispatch_backward",
           "moe_experts_forward_clipped", "moe_forward_clipped", "_lib"]
